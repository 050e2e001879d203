"""Writes tests/golden/oracle_tiny.json: the oracle's outputs on two tiny
seeded cases (the tiny fp32 workload with absorbing noise, and a small bf16
case with uniform noise, shifted logits and a softcap).  It calls only the
oracle and the seeded input generators; the library never writes it.

    python tests/golden/make_golden.py
"""

import base64
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as WL  # noqa: E402

CASES = {
    "tiny-absorb-f32": dict(workload=1, seed=0, eps=None, align=None, softcap=None),
    "small-uniform-shifted-softcap-bf16": dict(
        small=dict(seed=77, n_docs=3, max_len=90, H=64, V=300, noise=WL.NOISE_UNIFORM,
                   softcap=5.0),
        seed=12345, eps=0.2, align=oracle.SHIFTED, softcap=5.0),
}


def inputs(spec):
    if "workload" in spec:
        return WL.generate(WL.make_workload(spec["workload"]))
    return WL.small_case(**spec["small"])


def run(name):
    spec = CASES[name]
    inp = inputs(spec)
    wl = inp.wl
    eps = wl.eps if spec["eps"] is None else spec["eps"]
    align = wl.align if spec["align"] is None else spec["align"]
    softcap = wl.softcap if spec["softcap"] is None else spec["softcap"]
    xt, corrupted, p, counts = oracle.corrupt(inp.x0, inp.cu_seqlens, spec["seed"], eps,
                                              wl.noise, wl.mask_id, wl.rand_vocab)
    rows, tgt, w = oracle.compact(corrupted, inp.x0, inp.cu_seqlens, p, align)
    loss, ce, dh = oracle.head_ce(inp.hidden, inp.W, rows, tgt, w, softcap)
    return dict(
        seed=spec["seed"], eps=eps, align=int(align), softcap=softcap, noise=int(wl.noise),
        xt=[int(v) for v in xt], corrupted=[int(v) for v in np.flatnonzero(corrupted)],
        p_doc_bits=[f"{v:016x}" for v in p.view(np.uint64)],
        doc_counts=[int(v) for v in counts], row_idx=[int(v) for v in rows],
        tgt=[int(v) for v in tgt],
        w_bits=[f"{v:08x}" for v in w.astype(np.float32).view(np.uint32)],
        loss=float(loss), row_ce=[float(v) for v in ce],
        d_hidden_row_norms=[float(v) for v in np.linalg.norm(dh[rows], axis=1)],
        d_hidden_norm=float(np.linalg.norm(dh)),
        d_hidden_rows_f32_b64=encode_rows(dh[rows]))


def encode_rows(a):
    """The scored rows of the gradient, [M, H] in row-list order, rounded to
    fp32, little-endian, base64."""
    return base64.b64encode(np.ascontiguousarray(a, dtype="<f4").tobytes()).decode()


def decode_rows(text, H):
    return np.frombuffer(base64.b64decode(text), dtype="<f4").reshape(-1, H)


def main():
    out = {"about": "oracle outputs on two tiny seeded cases, written by make_golden.py "
                    "(oracle only); fp64 p and fp32 w as bit patterns; the gradient's "
                    "scored rows (row-list order) as fp32 little-endian, base64",
           "cases": {name: run(name) for name in CASES}}
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
