"""Pins the oracle's Philox4x32-10 against an independent implementation.

The second implementation is rocRAND's host-callable Philox engine, compiled
here from its public header and driven through its public API.  Agreement on
random keys and counters (including high counter words and every stream tag
the method uses) pins the round function, multipliers, key schedule and the
counter-to-word mapping.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.philox import philox4x32_10

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_rocrand_ref.cpp")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir(os.path.join(ROCM_INC, "rocrand")):
        pytest.skip("g++ or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([cxx, "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC, SRC,
                    "-o", exe], check=True, capture_output=True)

    def run(seeds, subseqs, offsets):
        text = "".join(f"{int(s)} {int(q)} {int(o)}\n"
                       for s, q, o in zip(seeds, subseqs, offsets))
        out = subprocess.run([exe], input=text, capture_output=True, text=True,
                             check=True).stdout.split()
        return np.array([int(x, 16) for x in out], dtype=np.uint64)
    return run


def _oracle_word(seed, c0, c1, c2, c3, j):
    words = philox4x32_10(c0, c1, c2, c3, seed & 0xFFFFFFFF, seed >> 32)
    return np.stack(words, axis=1)[np.arange(len(j)), j].astype(np.uint64)


def test_philox_matches_rocrand_random_counters(rocrand_ref):
    rng = np.random.default_rng(7)
    n = 2000
    seeds = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) \
        + rng.integers(0, 2, size=n, dtype=np.uint64)
    c0 = rng.integers(0, 2**32, size=n, dtype=np.uint64)
    c1 = rng.integers(0, 2**29, size=n, dtype=np.uint64)
    c2 = rng.integers(0, 2**32, size=n, dtype=np.uint64)
    c3 = rng.integers(0, 2**32, size=n, dtype=np.uint64)
    j = rng.integers(0, 4, size=n)
    subseq = c2 + (c3 << np.uint64(32))
    offset = np.uint64(4) * (c0 + (c1 << np.uint64(32))) + j.astype(np.uint64)
    ref = rocrand_ref(seeds, subseq, offset)
    words = np.stack(philox4x32_10(c0, c1, c2, c3, seeds & np.uint64(0xFFFFFFFF),
                                   seeds >> np.uint64(32)), axis=1)
    ours = words[np.arange(n), j].astype(np.uint64)
    assert np.array_equal(ref, ours)


@pytest.mark.parametrize("tag", [0, 1, 2])
def test_philox_token_layout_matches_rocrand(rocrand_ref, tag):
    """The method's token draws use counter (g >> 2, 0, 0, tag), word g & 3;
    in rocRAND's terms that is subsequence tag * 2^32 at offset g."""
    seed = 0x0123456789ABCDEF
    g = np.concatenate([np.arange(0, 64), np.arange(2**32 - 8, 2**32 + 8),
                        np.array([2**34 + 5, 2**40 + 3])]).astype(np.uint64)
    q = g >> np.uint64(2)
    ours = _oracle_word(seed, q & np.uint64(0xFFFFFFFF), q >> np.uint64(32), 0, tag,
                        (g & np.uint64(3)).astype(np.int64))
    ref = rocrand_ref([seed] * len(g), [tag << 32] * len(g), g)
    assert np.array_equal(ref, ours)


@pytest.mark.parametrize("tag", [1, 2])
def test_token_words_match_rocrand(rocrand_ref, tag):
    """oracle.mdlm.token_words itself (the function the corruption uses),
    across a window that crosses 2^32 tokens."""
    from oracle.mdlm import token_words
    seed = 0xFEDCBA9876543210
    start = 2**32 - 37
    n = 101
    ours = token_words(seed, n, tag, start=start).astype(np.uint64)
    g = np.arange(start, start + n, dtype=np.uint64)
    ref = rocrand_ref([seed] * n, [tag << 32] * n, g)
    assert np.array_equal(ref, ours)


def test_philox_counter_zero_key_zero_against_rocrand(rocrand_ref):
    ours = np.array(philox4x32_10(0, 0, 0, 0, 0, 0), dtype=np.uint64)
    ref = rocrand_ref([0] * 4, [0] * 4, [0, 1, 2, 3])
    assert np.array_equal(ref, ours)
