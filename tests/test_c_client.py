"""The C ABI used from C: a small client compiled with gcc against
include/dsv4.h and linked to libdsv4.so calls the entry points that need no
GPU (plan, workspace size, provenance gate, status strings, validation
errors) and checks their documented results.  No GPU call is made."""

import os
import subprocess

import sparse_mla_attention_block_amd as dsv4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "dsv4.h"

#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); return 1; } } while (0)

int main(void) {
    dsv4_decode_desc d;
    dsv4_plan plan;
    memset(&d, 0, sizeof d);
    d.batch = 1; d.num_heads = 64; d.topk = 2048; d.swa = 0;
    d.block_size = 64; d.num_blocks = 2048; d.page_stride = 64 * 584;
    d.max_blocks_per_seq = 2048; d.block_table_stride = 2048; d.sm_scale = 0.044194173f;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_OK);
    CHECK(plan.num_splits == 32 && plan.heads_per_group == 16 && plan.head_groups == 4);
    CHECK(plan.grid_partial == 128 && plan.block_partial == 512);
    CHECK(plan.workspace_bytes == (size_t)64 * 32 * 1028);
    CHECK(dsv4_sparse_decode_workspace_bytes(&d, 0) == plan.workspace_bytes);
    CHECK(dsv4_sparse_decode_workspace_bytes(&d, 1) == 0);

    d.batch = 256; d.topk = 512; d.swa = 128;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_OK);
    CHECK(plan.num_splits == 1 && plan.heads_per_group == 64 && plan.workspace_bytes == 0);

    d.num_heads = 24;
    CHECK(dsv4_sparse_decode_plan(&d, 0, &plan) == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(strstr(dsv4_last_error(), "num_heads") != NULL);
    CHECK(strcmp(dsv4_status_string(DSV4_ERR_INVALID_ARGUMENT), "DSV4_ERR_INVALID_ARGUMENT") == 0);

    d.num_heads = 64;
    CHECK(dsv4_sparse_decode(&d, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL)
          == DSV4_ERR_INVALID_ARGUMENT);
    CHECK(dsv4_decode_flags_for_cache(1, 0, 1, 1) == 0);
    CHECK(dsv4_decode_flags_for_cache(1, 1, 1, 1) == DSV4_DECODE_SCRUB);
    CHECK(dsv4_quantize_store(NULL, 512, NULL, 0, NULL, 64, 1, 64 * 584, DSV4_STORE_SANITIZE, NULL)
          == DSV4_OK);                                        /* nothing to store */
    printf("C CLIENT OK\n");
    return 0;
}
"""


def test_c_client_links_and_gets_documented_results(tmp_path):
    src = tmp_path / "client.c"
    src.write_text(CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(dsv4.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe), f"-L{libdir}", "-ldsv4",
                    f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "C CLIENT OK" in r.stdout, r.stdout + r.stderr
