"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of oracle.c (a textual edit of a
snippet that must occur exactly once), builds it with gcc into a temporary
directory, swaps it in for the real library and runs the pins.  A mutant that
passes every pin would mean the pins cannot tell it from the oracle.
"""

import ctypes
import inspect
import os
import subprocess
import sys

import pytest

import oracle
from tests import test_oracle_attention as A
from tests import test_oracle_convert as C
from tests import test_oracle_decoders as DEC
from tests import test_oracle_writer as W
from tests import test_golden as G

MUTANTS = {
    "sink_dropped": ("if (has_sink) D += exp(sink - M);", ""),
    "sink_scaled": ("const double sink = has_sink ? (double)J->sink[h] : -INFINITY;",
                    "const double sink = has_sink ? d->sm_scale * (double)J->sink[h] : -INFINITY;"),
    "e4m3_bias_8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                    "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_no_nan": ("if (e == 0xF && m == 0x7) return NAN;", ""),
    "ue8m0_bias": ("return ldexp(1.0, (int)code - 127);", "return ldexp(1.0, (int)code - 128);"),
    "scale_group_63": ("orc_ue8m0(scales[j / 64])", "orc_ue8m0(scales[j / 63 < 7 ? j / 63 : 6])"),
    "rope_big_endian": ("(uint16_t)(data[ORC_DNOPE + 2 * r] | (data[ORC_DNOPE + 2 * r + 1] << 8))",
                        "(uint16_t)(data[ORC_DNOPE + 2 * r + 1] | (data[ORC_DNOPE + 2 * r] << 8))"),
    "scale_stride_7": ("(int64_t)off * ORC_ROW_SCALE;", "(int64_t)off * 7;"),
    "scales_after_row": ("(int64_t)d->block_size * ORC_ROW_DATA +", "ORC_ROW_DATA +"),
    "valid_len_masks_swa": ("return p < vl ? p : d->topk + (p - vl);", "return p;"),
    "lse_without_log": ("*lse = M + log(D);\n        return;", "*lse = M + D;\n        return;"),
    "bt_row_stride_ignored": ("p = block_table[(int64_t)b * d->block_table_stride + blk];",
                              "p = block_table[blk];"),
    "page_upper_bound_unchecked": ("if (p < 0 || p >= d->num_blocks) return 0;",
                                   "if (p < 0) return 0;"),
    "q_head_major": ("qd[j] = orc_bf16(J->q[((int64_t)b * d->H + h) * ORC_D + j]);",
                     "qd[j] = orc_bf16(J->q[((int64_t)h * d->B + b) * ORC_D + j]);"),
    "split_skips_last_chunk": ("if (hi > eff_len) hi = eff_len;",
                               "if (hi >= eff_len) hi = lo;"),
    "convert_fill_ignored": ("int64_t v = invalid_fill;", "int64_t v = 0;"),
    "convert_offset_dropped": ("int64_t g = page * block_size + off;",
                               "int64_t g = page * block_size;"),
    "convert_no_block_check": ("if (blk < max_blocks_per_req) {", "if (1) {"),
    "convert_ragged_dense_base": ("base = cu_seqlens[t];", "base = (int64_t)t * width;"),
    "scrub_nope_only": ("for (j = 0; j < ORC_D; ++j)\n            if (!isfinite(out[j])) out[j] = 0.0;",
                        "for (j = 0; j < ORC_DNOPE; ++j)\n            if (!isfinite(out[j])) out[j] = 0.0;"),
    "scrub_ignored": ("if (d->scrub)\n", "if (0)\n"),
    "writer_cap_ignores_sanitize": ("const int cap = sanitize ? 254 : 255;", "const int cap = 255;"),
    "writer_rope_nan_only": ("if (sanitize && !isfinite(orc_bf16(bits))) bits = 0;",
                             "if (sanitize && isnan(orc_bf16(bits))) bits = 0;"),
    "writer_code_strict": ("if (a <= 448.0 * ldexp(1.0, c - 127)) break;",
                           "if (a < 448.0 * ldexp(1.0, c - 127)) break;"),
    "writer_code_one_low": ("if (a <= 448.0 * ldexp(1.0, c - 127)) break;",
                            "if (a <= 448.0 * ldexp(1.0, c - 126)) break;"),
    "writer_ties_away": ("(d == best_d && (c & 1) == 0 && (best & 1) == 1)", "(d == best_d)"),
    "writer_nan_sets_scale": ("if (!isnan(v) && fabs(v) > a) a = fabs(v);",
                              "if (isnan(v) || fabs(v) > a) a = isnan(v) ? INFINITY : fabs(v);"),
    "writer_sign_of_zero": ("return (uint8_t)(best | (signbit(v) ? 0x80 : 0));",
                            "return (uint8_t)(best | (v < 0 ? 0x80 : 0));"),
    "writer_pad_byte": ("scales[7] = 0;", "scales[7] = scales[0];"),
    "writer_rope_swapped": ("data[ORC_DNOPE + 2 * r] = (uint8_t)(bits & 0xFF);",
                            "data[ORC_DNOPE + 2 * r] = (uint8_t)(bits >> 8);"),
    "s_q_ignored": ("const int32_t seq = d->s_q > 1 ? b / d->s_q : b;",
                    "const int32_t seq = b;"),
    "s_q_table_only": ("valid[p] = (unsigned char)orc_resolve(dp, btp, seq, idx, &page, &off);",
                       "valid[p] = (unsigned char)orc_resolve(dp, btp, b, idx, &page, &off);"),
    "swa_pool_ignored": ("const int use_swa = J->d_swa != NULL && col >= d->topk;",
                         "const int use_swa = 0;"),
    "swa_pool_for_all": ("const int use_swa = J->d_swa != NULL && col >= d->topk;",
                         "const int use_swa = J->d_swa != NULL;"),
    "dot_skips_rope": ("for (j = 0; j < ORC_D; ++j) dot += qd[j] * rows[(int64_t)p * ORC_D + j];",
                       "for (j = 0; j < 448; ++j) dot += qd[j] * rows[(int64_t)p * ORC_D + j];"),
}


def _pins(only_golden=False):
    """Every test function of the pin modules (or of the hand-worked golden
    fixtures alone), expanded over its parameters."""
    out = []
    for mod in ((G,) if only_golden else (DEC, A, C, W, G)):
        for name, fn in inspect.getmembers(mod, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != mod.__name__:
                continue
            marks = getattr(fn, "pytestmark", [])
            grids = [m.args for m in marks if m.name == "parametrize"]
            calls = [dict()]
            for names, values in grids:
                keys = [k.strip() for k in names.split(",")]
                new = []
                for c in calls:
                    for v in values:
                        vv = v if len(keys) > 1 else (v,)
                        d = dict(c)
                        d.update(zip(keys, vv))
                        new.append(d)
                calls = new
            for c in calls:
                out.append((f"{mod.__name__}.{name}{c or ''}", fn, c))
    return out


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"snippet for {name} must occur exactly once"
    d = tmp_path / name
    d.mkdir()
    (d / "oracle.h").write_text(open(os.path.join(oracle.HERE, "oracle.h")).read())
    (d / "oracle.c").write_text(src.replace(old, new))
    so = d / "liboracle.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(d / "oracle.c"), "-o",
                    str(so), "-lm", "-lpthread"], check=True, capture_output=True)
    return str(so)


_CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[2])
import oracle
from tests.test_oracle_mutants import _pins
real = oracle.lib()
mut = ctypes.CDLL(sys.argv[1])
for n in ("orc_e4m3fn", "orc_ue8m0", "orc_bf16", "orc_resolve", "orc_dequant_row",
          "orc_sparse_decode", "orc_convert_req_index_to_global", "orc_quantize_row",
          "orc_store_rows", "orc_sparse_decode_dual"):
    f, g = getattr(mut, n), getattr(real, n)
    f.argtypes, f.restype = g.argtypes, g.restype
oracle._lib = mut
for label, fn, kwargs in _pins(sys.argv[3] == "golden"):
    try:
        fn(**kwargs)
    except Exception:
        print("CAUGHT", label)
        sys.exit(0)
print("PASSED_ALL")
"""


def _run_pins(tmp_path, name, which):
    so = _build_mutant(tmp_path, name, *MUTANTS[name])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CHILD, so, root, which], capture_output=True,
                       text=True, timeout=600)
    assert "PASSED_ALL" not in r.stdout, f"mutant {name} passed every {which} pin"
    assert r.returncode != 0 or "CAUGHT" in r.stdout, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_mutant_fails_some_pin(name, tmp_path):
    """The pins run in a child process: a mutant that reads out of bounds
    may crash, which also counts as caught (the pin run fails)."""
    _run_pins(tmp_path, name, "all")


# Mistakes the hand-worked fixtures of tests/golden/ catch on their own: the
# row format and scale decoding, the sink and the softmax scale, the lse, the
# RoPE part of the dot, the conversion, the sanitising writer's code cap.
GOLDEN_CATCHES = ["sink_dropped", "sink_scaled", "e4m3_bias_8", "ue8m0_bias", "scale_group_63",
                  "rope_big_endian", "scale_stride_7", "scales_after_row", "lse_without_log",
                  "dot_skips_rope", "convert_fill_ignored", "convert_offset_dropped",
                  "convert_no_block_check", "writer_cap_ignores_sanitize"]


@pytest.mark.parametrize("name", GOLDEN_CATCHES)
def test_golden_fixtures_alone_catch(name, tmp_path):
    _run_pins(tmp_path, name, "golden")
