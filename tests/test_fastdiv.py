"""The kernels' invariant-divisor quotient (csrc/fastdiv.h) against plain `/`.

The kernels split flat step and workgroup indices into (row, segment) with
mxq_quot; a wrong quotient would send a workgroup to the wrong row, so the
header is compiled here with the host compiler and checked:
* every divisor 1..4096 against dividends at and around every multiple edge
  that matters (0, 1, d-1, d, d+1, k*d-1, k*d, k*d+1, 2^31 +- 1, 2^32 - 1, ...)
  plus random ones;
* every power of two and its neighbours, the largest divisors, random 32-bit
  divisors;
* two divisors (3 and 641) over all 2^32 dividends.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "microscaling_weight_quantization_amd", "csrc")

CHECK_PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include "fastdiv.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {            // splitmix64, upper half
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static long bad = 0, checked = 0;
static void check(uint32_t n, uint32_t d) {
  const MxqDivisor v = mxq_divisor(d);
  const uint32_t q = mxq_quot(n, v);
  checked++;
  if (q != n / d || v.d != d) {
    if (bad < 10) printf("mismatch n=%u d=%u got=%u want=%u\n", n, d, q, n / d);
    bad++;
  }
}
static void edges(uint32_t d) {
  const uint32_t fixed[] = {0u, 1u, 2u, 0x7FFFFFFFu, 0x80000000u, 0x80000001u, 0xFFFFFFFEu, 0xFFFFFFFFu};
  for (uint32_t n : fixed) check(n, d);
  const uint64_t ks[] = {1, 2, 3, 7, 255, 256, 65535, 65536, 1000003};
  for (uint64_t k : ks) {
    for (int dn = -1; dn <= 1; dn++) {
      const uint64_t n = k * d + dn;
      if (n <= 0xFFFFFFFFull) check((uint32_t)n, d);
    }
  }
  const uint64_t top = 0xFFFFFFFFull / d;          // the largest multiple and its neighbours
  for (int dn = -1; dn <= 1; dn++) {
    const uint64_t n = top * d + dn;
    if (n <= 0xFFFFFFFFull) check((uint32_t)n, d);
  }
  for (int i = 0; i < 64; i++) check(rnd(), d);
}
int main(int argc, char** argv) {
  for (uint32_t d = 1; d <= 4096; d++) edges(d);
  for (int k = 0; k < 32; k++) {
    const uint64_t p = 1ull << k;
    for (int dd = -1; dd <= 1; dd++) {
      const uint64_t d = p + dd;
      if (d >= 1 && d <= 0xFFFFFFFFull) edges((uint32_t)d);
    }
  }
  const uint32_t big[] = {0xFFFFFFFFu, 0xFFFFFFFEu, 0x80000000u, 0x80000001u, 0x7FFFFFFFu, 0xC0000000u};
  for (uint32_t d : big) edges(d);
  for (int i = 0; i < 20000; i++) { uint32_t d = rnd(); if (d) edges(d); }
  for (int i = 0; i < 20000; i++) { uint32_t d = rnd() >> (rnd() % 32); if (d) edges(d); }
  if (argc > 1) {                                // exhaustive over every dividend
    const uint32_t ds[] = {3u, 641u};
    for (uint32_t d : ds) {
      const MxqDivisor v = mxq_divisor(d);
      uint32_t n = 0;
      do {
        if (mxq_quot(n, v) != n / d) { if (bad < 10) printf("mismatch n=%u d=%u\n", n, d); bad++; }
        checked++;
      } while (n++ != 0xFFFFFFFFu);
    }
  }
  printf("checked=%ld bad=%ld\n", checked, bad);
  return bad != 0;
}
"""


def _build(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(CHECK_PROGRAM)
    exe = tmp_path / "fastdiv_check"
    subprocess.check_call([cxx, "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)])
    return str(exe)


def test_quotient_matches_division(tmp_path):
    exe = _build(tmp_path)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout
    assert "bad=0" in out.stdout


def test_quotient_exhaustive_for_two_divisors(tmp_path):
    exe = _build(tmp_path)
    out = subprocess.run([exe, "all"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "bad=0" in out.stdout


def test_mutated_multiplier_is_caught(tmp_path):
    """The check itself: an off-by-one multiplier must produce mismatches."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    hdr = open(os.path.join(CSRC, "fastdiv.h")).read()
    mutated = hdr.replace("/ d + 1), l};", "/ d), l};")
    assert mutated != hdr
    (tmp_path / "fastdiv.h").write_text(mutated)
    src = tmp_path / "fastdiv_check.cpp"
    src.write_text(CHECK_PROGRAM)
    exe = tmp_path / "fastdiv_check"
    subprocess.check_call([cxx, "-O2", "-std=c++17", "-I", str(tmp_path), str(src), "-o", str(exe)])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode != 0 and "bad=0" not in out.stdout
