"""Launch sizes of the grid-stride kernels (masking_sparse_gemm_amd/csrc/nm_grid.h), checked
on the CPU: a small C++ program compiled with g++ includes the header the kernels use.

The per-group and per-word kernels of the compress, decompress and transposed passes take
any accepted shape (R*K below 2^36 elements, so up to 2^35 groups), while one launch may
have fewer than 2^32 work-items.  For such shapes the grid must be capped and the kernel's
stride loop must still visit every item exactly once; the sizes are checked up to 2^40
items, past what the checks accept."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masking_sparse_gemm_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "nm_grid.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL line %d: %s\n", __LINE__, #c); ++fails; } } while (0)

// every item of [0, work) visited exactly once by the kernels' loop
//   for (i = block * per + thread; i < work; i += grid * per)
static bool covers_once(int64_t work, int64_t per) {
  const int64_t grid = nm::stride_grid(work, per);
  std::vector<unsigned char> seen((size_t)work, 0);
  for (int64_t b = 0; b < grid; ++b)
    for (int64_t t = 0; t < per; ++t)
      for (int64_t i = b * per + t; i < work; i += grid * per) {
        if (seen[(size_t)i]) return false;
        seen[(size_t)i] = 1;
      }
  for (unsigned char v : seen) if (!v) return false;
  return true;
}

int main() {
  const int64_t per = 256;
  // 2^35 groups is the most an accepted shape has (2^36 elements, groups of 2); the helper
  // is checked well past it
  for (int64_t work : {(int64_t)1 << 32, (int64_t)1 << 38, (int64_t)1 << 39, ((int64_t)1 << 40) - 1}) {
    const int64_t g = nm::stride_grid(work, per);
    CHECK(g >= 1 && g <= nm::kMaxStrideBlocks);
    CHECK(g * per < ((int64_t)1 << 32));            // a legal launch
    // items per work-item: the loop's trip count stays bounded and covers `work`
    const int64_t trips = (work + g * per - 1) / (g * per);
    CHECK(trips * g * per >= work && (trips - 1) * g * per < work);
  }
  // small shapes: exactly one pass, no extra workgroups
  CHECK(nm::stride_grid(0, per) == 1);
  CHECK(nm::stride_grid(1, per) == 1);
  CHECK(nm::stride_grid(256, per) == 1);
  CHECK(nm::stride_grid(257, per) == 2);
  CHECK(nm::stride_grid(nm::kMaxStrideBlocks * per, per) == nm::kMaxStrideBlocks);
  CHECK(nm::stride_grid(nm::kMaxStrideBlocks * per + 1, per) == nm::kMaxStrideBlocks);
  // coverage, including past the cap (3 passes and a ragged tail)
  for (int64_t work : {(int64_t)0, (int64_t)1, (int64_t)255, (int64_t)256, (int64_t)257,
                       (int64_t)1000003, nm::kMaxStrideBlocks * per * 3 + 17})
    CHECK(covers_once(work, per));
  std::printf("%s\n", fails ? "FAILED" : "OK");
  return fails ? 1 : 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_stride_grid_sizes_and_coverage(tmp_path):
    src = tmp_path / "grid_check.cpp"
    exe = tmp_path / "grid_check"
    src.write_text(PROGRAM)
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, str(src), "-o", str(exe)])
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout
