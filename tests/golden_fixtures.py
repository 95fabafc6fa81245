"""Loader for the hand-worked fixtures under tests/golden/: builds the
decode fixture's pool, q and index arrays from its description, and returns
its expected values as arrays.  No arithmetic of the method lives here: the
expected numbers are the fixture's own closed forms."""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def decode_inputs(fx: dict) -> dict:
    g = fx["geometry"]
    bs, nb, stride = g["block_size"], g["num_blocks"], g["page_stride"]
    kv = np.full((nb, stride), 0xFF, dtype=np.uint8)           # NaN everywhere else
    for r in fx["rows"]:
        page, off = r["page"], r["offset"]
        data = kv[page, off * 576:(off + 1) * 576]
        data[:448] = r["nope_byte"]
        rope = np.full(64, r["rope_bf16_bits"], dtype=np.uint16)
        data[448:] = rope.view(np.uint8)                       # little endian
        sc = kv[page, bs * 576 + off * 8: bs * 576 + off * 8 + 8]
        sc[:7] = r["scale_codes"]
        sc[7] = 0
    q = np.zeros((g["B"], g["H"], 512), dtype=np.uint16)
    for h, d in fx["q_ones"]["entries"]:
        q[0, h, d] = 0x3F80
    return dict(kv=kv, q=q, block_table=np.array(fx["block_table"], dtype=np.int32),
                topk_idx=np.array(fx["topk_idx"], dtype=np.int32), geometry=g,
                max_blocks_per_seq=fx["max_blocks_per_seq"])


def decode_expected(fx: dict, case: str):
    """(out [B, H, 512], lse [B, H]) of the named case ("no_sink" or "sink_one")."""
    c = fx[case]
    g = fx["geometry"]
    out = np.zeros((g["B"], g["H"], 512))
    lse = np.zeros((g["B"], g["H"]))
    heads = list(c["out"]) + [c["rest"]] * (g["H"] - len(c["out"]))
    lses = list(c["lse"]) + [c["rest"]["lse"]] * (g["H"] - len(c["out"]))
    for h, hv in enumerate(heads):
        for k, v in enumerate(hv["nope_group_values"]):
            out[0, h, 64 * k:64 * (k + 1)] = v
        out[0, h, 448:] = hv["rope_value"]
        lse[0, h] = lses[h]
    return out, lse
