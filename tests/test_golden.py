"""Stored fixtures under tests/golden/.

page_constants.json holds values the pages print (each with its page and
row); the workloads and the oracle must use them.  oracle_tiny.json holds the
oracle's outputs on two tiny seeded cases, written by
tests/golden/make_golden.py from the oracle alone: the oracle must reproduce
them (integers and bit patterns exactly, reals to rounding), which guards it
against unintended changes.  The GPU check of the library against the same
file is in test_gpu_golden.py.
"""

import inspect
import json
import os
import sys

import numpy as np

import oracle
import workloads as WL

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
sys.path.insert(0, GOLDEN)

import make_golden  # noqa: E402


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_page_constants_in_workloads_and_oracle():
    c = _load("page_constants.json")
    eps = c["mask_probability_floor"]["value"]
    for k in (1, 2, 3, 4):
        assert WL.make_workload(k).eps == eps
    # p = (1 - eps) t + eps: every p lies in [eps, 1), t = 0 maps to eps
    t, p, _ = oracle.noise_levels(7, eps, 5000)
    assert p.min() >= eps and p.max() < 1.0
    assert np.all(p == eps + (1.0 - eps) * t)
    # the LLaDA-shaped workload is one sequence of the longest chunk
    assert WL.make_workload(2).lengths == [c["max_sequence_tokens"]["value"]]
    # document lengths: clipped to [16, 4096] with arithmetic mean 296
    sig = inspect.signature(WL.lognormal_lengths)
    assert sig.parameters["lo"].default == c["min_chunk_tokens"]["value"]
    assert sig.parameters["hi"].default == c["max_sequence_tokens"]["value"]
    wl3 = WL.make_workload(3)
    assert all(16 <= n <= 4096 for n in wl3.lengths)
    cu = WL.lognormal_stream_offsets(5, c["mean_document_tokens"]["value"], 1 << 22)
    mean = float(np.diff(cu).mean())
    assert abs(mean - 296) < 0.05 * 296  # (the clip moves the mean a little)
    assert WL.make_workload(4).mask_id == c["nemotron_mask_token"]["value"]


def test_oracle_reproduces_its_stored_outputs():
    stored = _load("oracle_tiny.json")["cases"]
    for name, want in stored.items():
        got = make_golden.run(name)
        for key in ("xt", "corrupted", "p_doc_bits", "doc_counts", "row_idx", "tgt", "w_bits"):
            assert got[key] == want[key], (name, key)
        assert abs(got["loss"] - want["loss"]) <= 1e-12 * abs(want["loss"])
        np.testing.assert_allclose(got["row_ce"], want["row_ce"], rtol=1e-12)
        np.testing.assert_allclose(got["d_hidden_row_norms"], want["d_hidden_row_norms"],
                                   rtol=1e-10)
        H = make_golden.inputs(make_golden.CASES[name]).wl.H
        g = make_golden.decode_rows(got["d_hidden_rows_f32_b64"], H)
        w = make_golden.decode_rows(want["d_hidden_rows_f32_b64"], H)
        # (fp32 storage: the oracle's reruns may differ in the last fp32 bit)
        np.testing.assert_allclose(g, w, rtol=1e-6, atol=1e-6 * float(np.abs(w).max()))
