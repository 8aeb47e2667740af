"""Pins of the oracle's Philox4x32-10: the generator's published known-answer
vectors, rocRAND's independent implementation (its host-callable engine header,
compiled here for the host only), and statistical checks of the element streams
(the default 32-bit words and the opt-in 16-bit halves)."""
import json
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox_kat.json")


def kat():
    return json.load(open(GOLDEN))


def test_known_answer_vectors():
    for v in kat()["vectors"]:
        ctr = np.array([[int(c, 16) for c in v["counter"]]], dtype=np.uint32)
        k0, k1 = (int(k, 16) for k in v["key"])
        out = philox.philox4x32_10(ctr, k0 | (k1 << 32))[0]
        assert [int(o) for o in out] == [int(o, 16) for o in v["out"]]


def test_element_streams_hand_worked():
    g = kat()
    words = philox.element_words(np.arange(4, dtype=np.uint64), 0)
    assert [int(w) for w in words] == [int(w, 16) for w in g["words_seed0_n0_to_3"]]
    halves = philox.element_r16_halves(np.arange(8, dtype=np.uint64), 0)
    assert [int(h) for h in halves] == [int(h, 16) for h in g["halves_seed0_n0_to_7"]]
    # element 8 starts the next counter: it must differ from a reuse of counter 0
    nxt = philox.element_r16_halves(np.arange(8, 16, dtype=np.uint64), 0)
    assert not np.array_equal(nxt, halves)

ROCRAND_PROGRAM = r"""
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
// usage: prog seed n0 count  -> prints the 32-bit word of elements n0 .. n0+count-1
int main(int argc, char** argv) {
  unsigned long long seed = strtoull(argv[1], 0, 0);
  unsigned long long n0 = strtoull(argv[2], 0, 0);
  int count = atoi(argv[3]);
  rocrand_device::philox4x32_10_engine e(seed, 0ull, n0);
  for (int i = 0; i < count; ++i) printf("%u\n", e.next());
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_prog():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not present")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(ROCRAND_PROGRAM)
    subprocess.run([hipcc, "-x", "hip", "--offload-host-only", "-O1", src, "-o", exe], check=True,
                   capture_output=True)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("seed,n0,count", [(0, 0, 16), (7, 0, 64), (7, 3, 9), (0xDEADBEEF12345678, 2 ** 33 + 1, 40),
                                           (4, 0, 4), (2 ** 64 - 1, 2 ** 40 - 5, 12)])
def test_element_words_match_rocrand(rocrand_prog, seed, n0, count):
    out = subprocess.run([rocrand_prog, str(seed), str(n0), str(count)], check=True, capture_output=True,
                         text=True).stdout.split()
    ref = np.array([int(v) for v in out], dtype=np.uint64)
    n = np.uint64(n0) + np.arange(count, dtype=np.uint64)
    ours = philox.element_words(n, seed).astype(np.uint64)
    np.testing.assert_array_equal(ours, ref)


def test_r16_is_uniform_and_seed_dependent():
    r = philox.tensor_r16(256, 1024, seed=7).astype(np.float64)
    hist = np.bincount((r / 4096).astype(np.int64).ravel(), minlength=16)
    expect = r.size / 16
    chi2 = ((hist - expect) ** 2 / expect).sum()
    assert chi2 < 50  # 15 dof: p ~ 1e-5
    r2 = philox.tensor_r16(256, 1024, seed=8)
    assert (r2 != r).mean() > 0.99
    # offsets address the same stream
    a = philox.tensor_r16(4, 64, seed=7, offset=100)
    b = philox.tensor_r16(5, 64, seed=7, offset=36)
    np.testing.assert_array_equal(a.reshape(-1), b.reshape(-1)[64:])


@pytest.mark.parametrize("seed,n0,count", [(0, 0, 32), (7, 0, 64), (7, 6, 20), (0xDEADBEEF12345678, 2 ** 33 + 8, 40),
                                           (2 ** 64 - 1, 2 ** 41 - 16, 24)])
def test_halves_stream_matches_rocrand(rocrand_prog, seed, n0, count):
    # element n of the halves stream is half (n mod 2) of word n div 2 of the element
    # word stream, which rocRAND produces independently
    w0 = n0 // 2
    nw = (n0 + count - 1) // 2 - w0 + 1
    out = subprocess.run([rocrand_prog, str(seed), str(w0), str(nw)], check=True, capture_output=True,
                         text=True).stdout.split()
    words = [int(v) for v in out]
    ref = np.array([(words[n // 2 - w0] >> (16 * (n % 2))) & 0xFFFF for n in range(n0, n0 + count)], dtype=np.uint64)
    n = np.uint64(n0) + np.arange(count, dtype=np.uint64)
    np.testing.assert_array_equal(philox.element_r16_halves(n, seed).astype(np.uint64), ref)


def test_halves_are_uniform_and_independent_of_the_word_stream():
    r = philox.tensor_r16_halves(256, 1024, seed=7).astype(np.float64)
    hist = np.bincount((r / 4096).astype(np.int64).ravel(), minlength=16)
    expect = r.size / 16
    assert ((hist - expect) ** 2 / expect).sum() < 50  # 15 dof: p ~ 1e-5
    # adjacent elements (the two halves of one word) are uncorrelated
    a, b = r.reshape(-1)[0::2] - 32767.5, r.reshape(-1)[1::2] - 32767.5
    corr = (a * b).mean() / np.sqrt((a * a).mean() * (b * b).mean())
    assert abs(corr) < 5 / np.sqrt(a.size)
    w = philox.tensor_r16(256, 1024, seed=7)
    assert (w != r).mean() > 0.99
    # offsets address the same stream
    x = philox.tensor_r16_halves(4, 64, seed=7, offset=96)
    y = philox.tensor_r16_halves(5, 64, seed=7, offset=32)
    np.testing.assert_array_equal(x.reshape(-1), y.reshape(-1)[64:])


def test_sign_mask_from_seed_pins(rocrand_prog):
    # the transform's sign mask of a seed is, by this library's definition, bits 0..15
    # of word 0 of Philox4x32-10(counter 0, key = seed). Seed 0: the first published
    # vector (word 0 = 0x6627e8d5) fixes it; other seeds: element 0 of rocRAND's
    # engine for that seed is the same word
    from oracle import rht
    w0 = int(kat()["vectors"][0]["out"][0], 16)
    assert rht.sign_mask_from_seed(0) == w0 & 0xFFFF == 0xE8D5
    for seed in (1, 4, 9, 13, 14, 0xA5C3, 0xDEADBEEF12345678, 2 ** 64 - 1):
        out = subprocess.run([rocrand_prog, str(seed), "0", "1"], check=True, capture_output=True,
                             text=True).stdout.split()
        assert rht.sign_mask_from_seed(seed) == int(out[0]) & 0xFFFF, seed
