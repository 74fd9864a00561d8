"""Pins of the oracle's Philox4x32-10 generator and element mapping (CPU only).

* Known-answer vectors distributed with the Random123 reference
  implementation of Salmon et al. (SC'11) for Philox4x32 with 10 rounds.
* An independent implementation: rocRAND's Philox4x32-10 engine, compiled for
  the host from its source header (rocrand_philox4x32_10.h) and called with
  seed = key, subsequence = tag, offset = 4*q, which puts the counter at
  (q lo, q hi, tag, 0).
* Uniformity of the 16-bit draws (chi-square over 256 bins, bit balance).
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import philox

KAT = [  # (ctr0..3, key0..1) -> out0..3
    ((0, 0, 0, 0, 0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 6, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344, 0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("inp,out", KAT)
def test_known_answer_vectors(inp, out):
    got = philox.philox4x32_10(*inp)
    assert tuple(int(w) for w in got) == out


_ROCRAND_SRC = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  unsigned long long seed, tag, q;
  while (std::scanf("%llx %llx %llx", &seed, &tag, &q) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, tag, 4ull * q);
    uint4 r = e.next4();
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
"""


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    return None


def test_against_rocrand_host_engine():
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND source header / hipcc not available")
    r = np.random.default_rng(7)
    cases = [(0x5EED0004, 0, 0), (0x5EED0004, 1, 12345), (2 ** 64 - 1, 2, 2 ** 40 + 3)]
    cases += [(int(r.integers(0, 2 ** 63)), int(r.integers(0, 3)), int(r.integers(0, 2 ** 36)))
              for _ in range(60)]
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "p.cpp")
        exe = os.path.join(d, "p")
        open(src, "w").write(_ROCRAND_SRC)
        subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-I/opt/rocm/include",
                        "-O1", src, "-o", exe], check=True, capture_output=True)
        inp = "".join("%x %x %x\n" % c for c in cases)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = [tuple(int(w, 16) for w in line.split()) for line in out.strip().splitlines()]
    assert len(ref) == len(cases)
    for (seed, tag, q), want in zip(cases, ref):
        got = philox.philox4x32_10(q & 0xFFFFFFFF, q >> 32, tag, 0, seed & 0xFFFFFFFF, seed >> 32)
        assert tuple(int(w) for w in got) == want
        # element mapping: 8 16-bit draws per call, low half of word 0 first
        u = philox.uniform16(seed, tag, np.arange(8 * q, 8 * q + 8))
        halves = []
        for w in want:
            halves += [w & 0xFFFF, w >> 16]
        assert list(u) == halves


def test_range_helper_matches_per_index():
    idx = np.arange(1000, 1000 + 777)
    a = philox.uniform16(99, 1, idx)
    b = philox.uniform16_range(99, 1, 1000, 777)
    assert np.array_equal(a, b)
    assert np.array_equal(philox.uniform16_range(5, 0, 3, 5), philox.uniform16(5, 0, np.arange(3, 8)))


def test_uniformity():
    n = 1 << 20
    u = philox.uniform16_range(0x5EED0002, 2, 0, n).astype(np.int64)
    counts = np.bincount(u >> 8, minlength=256)
    exp = n / 256
    chi2 = np.sum((counts - exp) ** 2 / exp)
    # 255 degrees of freedom: mean 255, sd ~22.6; allow 5 sd
    assert chi2 < 255 + 5 * 22.6
    bits = ((u[:, None] >> np.arange(16)) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 5 * 0.5 / np.sqrt(n))
    # different tags give different streams
    assert not np.array_equal(philox.uniform16_range(1, 0, 0, 64), philox.uniform16_range(1, 1, 0, 64))
