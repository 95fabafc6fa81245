"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle.c) is rebuilt with -fsanitize=address,undefined and its
  pin tests run against that build in a child process (the ASan runtime is
  preloaded there, since the Python interpreter itself is not instrumented).
  Two canary libraries loaded the same way, one with a heap overflow under
  ASan and one with a signed overflow under UBSan, must each be caught
  first, so a silent sanitizer cannot pass this test.
* The host side of the C ABI (api.hip: argument validation, the split
  selector, workspace sizes, the provenance gate) is compiled host-only with
  g++ and the same sanitizers, against stand-in kernel launchers that only
  record the launch they were asked for; a C client built with gcc and the
  sanitizers drives every entry point through its validation and planning
  paths.  No GPU is touched.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mla_attention_block_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's libasan is not installed")
    return p


def _preload_env(extra=None):
    env = dict(os.environ)
    pre = [_libasan()] + [x for x in env.get("LD_PRELOAD", "").split(":") if x]
    env["LD_PRELOAD"] = ":".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra or {})
    return env


CANARY = r"""
#include <stdlib.h>
int heap_canary(int i) {
    volatile int* a = (volatile int*)malloc(4 * sizeof(int));
    int v;
    a[0] = 1;
    v = a[i];
    free((void*)a);
    return v;
}
int overflow_canary(int x) { return x + 1; }
"""


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(lib), "-lm", "-lpthread"],
                   check=True)
    can_src = tmp_path / "canary.c"
    can_src.write_text(CANARY)
    env = _preload_env({"DSV4_ORACLE_LIB": str(lib)})

    # Canaries, one per sanitizer: an out-of-bounds heap read (ASan alone)
    # and a signed overflow (UBSan alone) must each stop the process.
    for flag, call, sign in (("-fsanitize=address", "heap_canary(4)", "heap-buffer-overflow"),
                             ("-fsanitize=undefined", "overflow_canary(2147483647)",
                              "signed integer overflow")):
        can = tmp_path / f"libcanary{flag[-3:]}.so"
        subprocess.run(["gcc", "-O1", "-fPIC", "-shared", flag, "-fno-sanitize-recover=all",
                        str(can_src), "-o", str(can)], check=True)
        r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(can)!r}).{call}"],
                           env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode != 0 and sign in r.stderr, r.stderr[-2000:]

    # The oracle package loads the sanitized build.
    r = subprocess.run([sys.executable, "-c",
                        "import oracle; print(oracle.lib()._name)"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == str(lib), r.stdout + r.stderr

    tests = ["tests/test_oracle_decoders.py", "tests/test_oracle_convert.py",
             "tests/test_oracle_writer.py", "tests/test_golden.py",
             "tests/test_oracle_attention.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1200)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr


STUBS = r"""
// Stand-in kernel launchers for a host-only build: each records the launch
// it was asked for and checks the parameters it is given for consistency.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include "internal.hpp"

namespace dsv4 {
static int g_launches = 0;
static void need(bool c, const char* what) {
    if (!c) { fprintf(stderr, "stub: inconsistent %s\n", what); abort(); }
}
static void decode_ok(const DecodeParams& p, int hg, int64_t grid) {
    need(p.B >= 1 && p.H % 16 == 0 && hg % 16 == 0 && p.H % hg == 0, "heads");
    need(p.G == p.H / hg, "head groups");
    need(p.units == (int64_t)p.B * (p.bal ? p.bal : p.S), "units");
    need(p.bal == 0 || (p.B <= 64 && p.bal >= 2 && p.S > p.bal), "balanced splits");
    need(grid >= p.units * p.G && grid % p.G == 0, "grid");
    need(p.S == 1 || (p.part_o && p.part_lse), "split workspace");
}
hipError_t launch_decode_partial(const DecodeParams& p, int hg, int64_t grid, bool, hipStream_t) {
    decode_ok(p, hg, grid);
    need(p.slots == nullptr || (p.bt != nullptr && p.bal == 0 &&
                                (p.topk + p.swa + p.S - 1) / p.S <= 1024),
         "slots need the block table, uniform splits and at most 1024 columns per split");
    ++g_launches; return hipSuccess;
}
hipError_t launch_decode_short(const DecodeParams& p, int hg, int64_t grid, bool, hipStream_t) {
    decode_ok(p, hg, grid);
    need(hg == 16 || hg == 32 || hg == 64, "short-kernel head group");
    need(p.slots == nullptr || p.bt != nullptr, "slots need the block table");
    need(p.bal == 0, "balanced splits run on the pipelined kernel only");
    ++g_launches; return hipSuccess;
}
size_t short_lds_bytes(int) { return 0; }
hipError_t launch_dense_partial(const DecodeParams& p, int hg, int64_t grid, hipStream_t) {
    decode_ok(p, hg, grid); ++g_launches; return hipSuccess;
}
hipError_t launch_gather_dequant(const DecodeParams& p, uint16_t* o, uint8_t* m, bool, hipStream_t) {
    need(o && m && p.idx, "gather pointers"); ++g_launches; return hipSuccess;
}
hipError_t launch_combine(const CombineParams& p, hipStream_t) {
    need(p.S >= 1 && p.B >= 1 && p.part_o && p.out, "combine"); ++g_launches; return hipSuccess;
}
hipError_t launch_convert(const ConvertParams& p, hipStream_t) {
    need(p.num_tokens > 0 && p.width > 0 && p.out, "convert"); ++g_launches; return hipSuccess;
}
hipError_t launch_quantize_store(const StoreParams& p, hipStream_t) {
    need(p.n > 0 && p.rows && p.slots && p.kv, "store"); ++g_launches; return hipSuccess;
}
hipError_t launch_gather_floor(const DecodeParams&, int64_t, uint32_t* w, hipStream_t) {
    need(w != nullptr, "floor"); ++g_launches; return hipSuccess;
}
}  // namespace dsv4

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
extern "C" int stub_launches(void) { return dsv4::g_launches; }
"""

CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "dsv4.h"
#include "dsv4_diag.h"

int stub_launches(void);
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, \
                                         dsv4_last_error()); return 1; } } while (0)
#define DEV(a) ((void*)(uintptr_t)(a))

static void base(dsv4_decode_desc* d, int B, int H, int topk, int swa) {
    memset(d, 0, sizeof *d);
    d->batch = B; d->num_heads = H; d->topk = topk; d->swa = swa;
    d->block_size = 64; d->num_blocks = 4096; d->page_stride = 64 * 584;
    d->max_blocks_per_seq = 2048; d->block_table_stride = 2048; d->sm_scale = 0.044194173f;
}

int main(void) {
    dsv4_decode_desc d;
    dsv4_plan plan;
    int shapes[5][4] = {{1, 16, 128, 0}, {4, 64, 512, 128}, {1, 64, 2048, 0},
                        {256, 64, 512, 128}, {32, 128, 2048, 128}};
    int i, S, n = 0;
    for (i = 0; i < 5; ++i) {
        base(&d, shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3]);
        for (S = 0; S <= 64; S += (S < 4 ? 1 : 15)) {
            size_t ws;
            CHECK(dsv4_sparse_decode_plan(&d, S, &plan) == DSV4_OK);
            ws = dsv4_sparse_decode_workspace_bytes(&d, S);
            CHECK(ws == plan.workspace_bytes);
            CHECK(plan.num_splits >= 1 && plan.num_splits <= DSV4_MAX_SPLITS);
            d.workspace = ws ? DEV(0x10000) : NULL;
            d.workspace_bytes = ws;
            /* A valid call reaches the launcher(s) with consistent parameters. */
            CHECK(dsv4_sparse_decode(&d, DEV(0x1000), DEV(0x2000), (const int32_t*)DEV(0x3000),
                                     (const int32_t*)DEV(0x4000), NULL, (const float*)DEV(0x5000),
                                     DEV(0x6000), (float*)DEV(0x7000), S, NULL) == DSV4_OK);
            n += plan.num_splits > 1 ? 2 : 1;
            CHECK(stub_launches() == n);
            /* The slot-writing decode: one launch more (the conversion) only when
               the pipelined kernel would have more than 1024 index columns a split. */
            CHECK(dsv4_sparse_decode_with_slots(&d, DEV(0x1000), DEV(0x2000),
                                                (const int32_t*)DEV(0x3000),
                                                (const int32_t*)DEV(0x4000), NULL, NULL,
                                                DEV(0x6000), NULL, S, (int32_t*)DEV(0x8000),
                                                NULL) == DSV4_OK);
            {
                const int kt = shapes[i][2] + shapes[i][3];
                const int conv = plan.partial_kernel != DSV4_KERNEL_SHORT &&
                                 (kt + plan.num_splits - 1) / plan.num_splits > 1024;
                n += (plan.num_splits > 1 ? 2 : 1) + conv;
                CHECK(stub_launches() == n);
            }
            CHECK(dsv4_sparse_decode_partial_with_slots(&d, DEV(0x1000), DEV(0x2000),
                                                        (const int32_t*)DEV(0x3000),
                                                        (const int32_t*)DEV(0x4000), NULL, NULL,
                                                        DEV(0x6000), NULL, S,
                                                        (int32_t*)DEV(0x8000), NULL) == DSV4_OK);
            n += (plan.partial_kernel != DSV4_KERNEL_SHORT &&
                  (shapes[i][2] + shapes[i][3] + plan.num_splits - 1) / plan.num_splits > 1024)
                     ? 2 : 1;
            CHECK(stub_launches() == n);
            CHECK(dsv4_sparse_decode_with_slots(&d, DEV(0x1000), DEV(0x2000), NULL,
                                                (const int32_t*)DEV(0x4000), NULL, NULL,
                                                DEV(0x6000), NULL, S, (int32_t*)DEV(0x8000),
                                                NULL) == DSV4_ERR_INVALID_ARGUMENT);
            if (ws) {
                d.workspace_bytes = ws - 1;
                CHECK(dsv4_sparse_decode(&d, DEV(0x1000), DEV(0x2000), NULL,
                                         (const int32_t*)DEV(0x4000), NULL, NULL, DEV(0x6000),
                                         NULL, S, NULL) == DSV4_ERR_WORKSPACE_TOO_SMALL);
            }
        }
    }
    /* Balanced splits: the same grid, S + ceil(S/4) split slots per row, only
       on pipelined plans with S >= 2 and batch <= 64; the slot-writing decode
       then converts in a launch of its own. */
    for (i = 0; i < 5; ++i) {
        dsv4_plan u;
        base(&d, shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3]);
        for (S = 0; S <= 64; S += (S < 4 ? 1 : 15)) {
            int on, want;
            d.flags = 0;
            CHECK(dsv4_sparse_decode_plan(&d, S, &u) == DSV4_OK);
            d.flags = DSV4_DECODE_BALANCE;
            CHECK(dsv4_sparse_decode_plan(&d, S, &plan) == DSV4_OK);
            on = u.partial_kernel == DSV4_KERNEL_PIPELINED && u.num_splits >= 2 && d.batch <= 64;
            want = u.num_splits + (u.num_splits + 3) / 4;
            if (want > DSV4_MAX_SPLITS) want = DSV4_MAX_SPLITS;
            CHECK(plan.balanced_splits == (on ? u.num_splits : 0));
            CHECK(plan.num_splits == (on ? want : u.num_splits));
            CHECK(plan.grid_partial == u.grid_partial);
            CHECK(plan.workspace_bytes ==
                  (plan.num_splits > 1 ? (size_t)d.batch * d.num_heads * plan.num_splits * 1028 : 0));
            d.workspace = plan.workspace_bytes ? DEV(0x10000) : NULL;
            d.workspace_bytes = plan.workspace_bytes;
            CHECK(dsv4_sparse_decode(&d, DEV(0x1000), DEV(0x2000), (const int32_t*)DEV(0x3000),
                                     (const int32_t*)DEV(0x4000), (const int32_t*)DEV(0x9000),
                                     (const float*)DEV(0x5000), DEV(0x6000), (float*)DEV(0x7000),
                                     S, NULL) == DSV4_OK);
            n += plan.num_splits > 1 ? 2 : 1;
            CHECK(stub_launches() == n);
            CHECK(dsv4_sparse_decode_with_slots(&d, DEV(0x1000), DEV(0x2000),
                                                (const int32_t*)DEV(0x3000),
                                                (const int32_t*)DEV(0x4000), NULL, NULL,
                                                DEV(0x6000), NULL, S, (int32_t*)DEV(0x8000),
                                                NULL) == DSV4_OK);
            {
                const int kt = shapes[i][2] + shapes[i][3];
                const int conv = plan.partial_kernel != DSV4_KERNEL_SHORT &&
                                 (on || (kt + plan.num_splits - 1) / plan.num_splits > 1024);
                n += (plan.num_splits > 1 ? 2 : 1) + conv;
                CHECK(stub_launches() == n);
            }
            if (on)
                CHECK(dsv4_gather_floor(&d, DEV(0x2000), (const int32_t*)DEV(0x3000),
                                        (const int32_t*)DEV(0x4000), NULL, S,
                                        (uint32_t*)DEV(0xA000), NULL) == DSV4_ERR_INVALID_ARGUMENT);
            CHECK(stub_launches() == n);
        }
    }
    d.flags = 0;

    /* Validation errors never launch. */
    base(&d, 1, 64, 2048, 0);
    d.num_heads = 24;   CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.num_heads = 144;  CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.num_heads = 64; d.topk = 0;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.topk = 2048; d.page_stride = 64 * 584 - 8;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.page_stride = 64 * 584; d.num_blocks = (int64_t)1 << 62;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.num_blocks = 4096;
    CHECK(dsv4_sparse_decode_plan(&d, 65, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_sparse_decode_plan(&d, -1, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_sparse_decode_plan(NULL, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_sparse_decode_plan(&d, 0, NULL) == DSV4_ERR_INVALID_ARGUMENT);
    d.flags = 0x10;     CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.flags = 0; d.tokens_per_seq = 3;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    d.tokens_per_seq = 0;
    CHECK(dsv4_sparse_decode(&d, DEV(0x1008), DEV(0x2000), NULL, (const int32_t*)DEV(0x4000),
                             NULL, NULL, DEV(0x6000), NULL, 1, NULL) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_sparse_decode(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL)
          == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_combine_splits(0, 64, 4, DEV(0x1000), (const float*)DEV(0x2000), NULL,
                              DEV(0x3000), NULL, NULL) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_convert_req_index_to_global(NULL, 1, (const int32_t*)DEV(0x1000), 4, 8,
                                           (const int32_t*)DEV(0x2000), 4, 1, 4, 64, NULL, -1,
                                           (int32_t*)DEV(0x3000), NULL) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_quantize_store(DEV(0x1000), 500, (const int64_t*)DEV(0x2000), 4, DEV(0x3000), 64,
                              16, 64 * 584, 0, NULL) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(stub_launches() == n);
    /* Valid calls of the other entry points launch once each. */
    CHECK(dsv4_combine_splits(2, 64, 4, DEV(0x1000), (const float*)DEV(0x2000), NULL,
                              DEV(0x3000), NULL, NULL) == DSV4_OK);
    CHECK(dsv4_convert_req_index_to_global(NULL, 1, (const int32_t*)DEV(0x1000), 8, 8,
                                           (const int32_t*)DEV(0x2000), 4, 1, 4, 64, NULL, -1,
                                           (int32_t*)DEV(0x3000), NULL) == DSV4_OK);
    CHECK(dsv4_quantize_store(DEV(0x1000), 512, (const int64_t*)DEV(0x2000), 4, DEV(0x3000), 64,
                              16, 64 * 584, DSV4_STORE_SANITIZE, NULL) == DSV4_OK);
    CHECK(dsv4_gather_dequant(&d, DEV(0x2000), NULL, (const int32_t*)DEV(0x4000), NULL,
                              DEV(0x8000), (uint8_t*)DEV(0x9000), NULL) == DSV4_OK);
    CHECK(stub_launches() == n + 4);
    CHECK(dsv4_decode_flags_for_cache(1, 0, 1, 1) == 0);
    CHECK(dsv4_decode_flags_for_cache(0, 0, 1, 1) == DSV4_DECODE_SCRUB);
    for (i = -1; i < 6; ++i) CHECK(dsv4_status_string(i) != NULL);
    printf("SANITIZED CLIENT OK\n");
    return 0;
}
"""


def test_host_api_under_asan_and_ubsan(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC]
    objs = []
    for name, src in (("api", os.path.join(CSRC, "api.hip")), ("stubs", None)):
        if src is None:
            src = str(tmp_path / "stubs.cpp")
            with open(src, "w") as f:
                f.write(STUBS)
        obj = str(tmp_path / f"{name}.o")
        subprocess.run(["g++", "-x", "c++", "-std=c++17", "-O1", "-fPIC", "-Wall", *SAN, *inc,
                        "-c", src, "-o", obj], check=True)
        objs.append(obj)
    lib = str(tmp_path / "libdsv4_host_san.so")
    subprocess.run(["g++", "-shared", *SAN, *objs, "-o", lib], check=True)
    csrc = tmp_path / "client.c"
    csrc.write_text(CLIENT)
    exe = str(tmp_path / "client")
    subprocess.run(["gcc", "-std=c99", "-O1", *SAN, *inc, str(csrc), "-o", exe, lib,
                    f"-Wl,-rpath,{tmp_path}"], check=True)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "SANITIZED CLIENT OK" in r.stdout, r.stdout + r.stderr
