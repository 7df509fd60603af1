"""The selection's binning helpers on the host (CPU only, no GPU).

lin_bin, order_key, key_score and bin_scale of csrc/select_core.h are
__host__ __device__; a host-only build of a small program checks, for scores
spanning every float class (+-0, subnormals, +-3e38, +-FLT_MAX, +-inf, NaN of
either sign, random values over all exponents) and for binning ranges near,
far from and much wider or narrower than the data:
  * every bin lies in [0, 2047];
  * bins never decrease as the order key grows (the exact selection relies on
    every score of a higher bin ranking above every score of a lower one);
  * order_key / key_score round-trip every value (-0 comes back as +0);
  * order_key_nz of a value plus +0 is its order_key (NaN aside).
"""
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_decode_attention_rotate_amd", "csrc")

PROGRAM = r"""
#include <float.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "select_core.h"

using namespace loki;

static float from_bits(unsigned u) { float f; memcpy(&f, &u, 4); return f; }
static unsigned bits(float f) { unsigned u; memcpy(&u, &f, 4); return u; }

int main() {
  std::vector<float> s = {0.f, -0.f, 1e-45f, -1e-45f, FLT_MIN, -FLT_MIN, 1.f, -1.f,
                          3e38f, -3e38f, FLT_MAX, -FLT_MAX, INFINITY, -INFINITY,
                          from_bits(0x7fc00000u), from_bits(0xffc00000u),
                          from_bits(0x7f800001u), from_bits(0xff800001u)};
  std::mt19937 g(7);
  for (int i = 0; i < 20000; i++) s.push_back(from_bits(g()));  // every exponent, NaNs too
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int i = 0; i < 20000; i++) s.push_back(nd(g));
  std::sort(s.begin(), s.end(), [](float a, float b) { return order_key(a) < order_key(b); });

  // order_key / key_score round trip (-0 as +0)
  for (float v : s) {
    const float back = key_score(order_key(v));
    const unsigned want = bits(v) == 0x80000000u ? 0u : bits(v);
    if (bits(back) != want) { printf("FAIL roundtrip %08x -> %08x\n", bits(v), bits(back)); return 1; }
  }

  // order_key_nz after adding +0 (-0 becomes +0) equals order_key for every
  // value but NaN (whose payload the addition may change)
  volatile float zero = 0.f;
  for (float v : s) {
    if (v != v) continue;
    const unsigned a = order_key_nz(v + zero), b = order_key(v);
    if (a != b) { printf("FAIL order_key_nz %08x: %08x != %08x\n", bits(v), a, b); return 1; }
  }

  struct R { float lo, scale; };
  std::vector<R> ranges;
  const float los[] = {0.f, -1.f, 1e30f, -1e30f, 3e38f, -3e38f, FLT_MAX, -FLT_MAX, 1e-40f};
  const float his_rel[] = {1e-7f, 1e-3f, 1.f, 1e10f};
  for (float lo : los)
    for (float r : his_rel) {
      const float hi = lo + (fabsf(lo) > 1.f ? fabsf(lo) * r : r);
      ranges.push_back({lo, bin_scale(lo, hi)});
    }
  const float raw_scales[] = {0.f, 1e-38f, 1e-10f, 1.f, 2047.f, 1e10f, 3e38f, FLT_MAX};
  for (float lo : los)
    for (float sc : raw_scales) ranges.push_back({lo, sc});
  // bin_scale of degenerate ranges: one bin
  if (bin_scale(1.f, 1.f) != 0.f || bin_scale(-INFINITY, 1.f) != 0.f ||
      bin_scale(1.f, INFINITY) != 0.f || bin_scale(-3e38f, 3e38f) != 0.f ||
      bin_scale(from_bits(0x7fc00000u), 1.f) != 0.f) {
    printf("FAIL bin_scale of a degenerate range\n");
    return 1;
  }

  long checked = 0;
  for (const R& r : ranges) {
    int prev = -1;
    unsigned prev_key = 0;
    for (float v : s) {
      const int b = lin_bin(v, r.lo, r.scale);
      if (b < 0 || b > kBins - 1) { printf("FAIL range %d for %08x lo %g scale %g\n", b, bits(v), r.lo, r.scale); return 1; }
      const unsigned key = order_key(v);
      if (b < prev || (key == prev_key && b != prev && prev >= 0)) {
        printf("FAIL order: %08x bin %d after key %08x bin %d (lo %g scale %g)\n", bits(v), b,
               prev_key, prev, r.lo, r.scale);
        return 1;
      }
      prev = b;
      prev_key = key;
      checked++;
    }
  }
  // a positive NaN ranks above +inf, a negative NaN below -inf
  if (lin_bin(from_bits(0x7fc00000u), 0.f, 1.f) != kBins - 1 ||
      lin_bin(from_bits(0xffc00000u), 0.f, 1.f) != 0) { printf("FAIL NaN bins\n"); return 1; }
  printf("ok %ld\n", checked);
  return 0;
}
"""


@pytest.fixture(scope="module")
def program():
    d = tempfile.mkdtemp(prefix="lin_bin_")
    src = os.path.join(d, "lin_bin_check.hip")
    exe = os.path.join(d, "lin_bin_check")
    open(src, "w").write(PROGRAM)
    r = subprocess.run(["hipcc", "--cuda-host-only", "-O2", "-std=c++17", "-I", CSRC,
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        pytest.fail(f"host build failed:\n{r.stdout}\n{r.stderr}")
    return exe


def test_lin_bin_monotone_and_in_range_for_every_input(program):
    r = subprocess.run([program], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok ")
    assert int(r.stdout.split()[1]) > 1_000_000
