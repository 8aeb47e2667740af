"""Pin of the oracle's Philox4x32-10 against rocRAND's independent implementation
(its host-callable engine header, compiled here for the host only), and
statistical checks of the element stream."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

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
