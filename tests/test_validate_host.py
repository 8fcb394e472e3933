"""The host-side checks of the KDA_VALIDATE=1 mode (CPU only): the library's
own header ``csrc/kda_validate.h``, compiled alone with g++ into a small
driver, run on well-formed and malformed cu_seqlens, gates and outputs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_67_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include <cmath>
#include <limits>
#include "kda_validate.h"
using namespace kda::validate;
#define CHECK(c) do { if (!(c)) { std::printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)
int main() {
  int64_t w = 0;
  const int32_t good[] = {0, 3, 3, 10};
  CHECK(cu_seqlens(good, 3, 10, &w) == nullptr);
  const int32_t empty[] = {0};
  CHECK(cu_seqlens(empty, 0, 0, &w) == nullptr);
  const int32_t start[] = {1, 3, 10};
  CHECK(cu_seqlens(start, 2, 10, &w) != nullptr && w == 0);
  const int32_t down[] = {0, 5, 4, 10};
  CHECK(cu_seqlens(down, 3, 10, &w) != nullptr && w == 2);
  CHECK(cu_seqlens(good, 3, 11, &w) != nullptr && w == 3);
  const float inf = std::numeric_limits<float>::infinity(), nan = std::nanf("");
  const float g_ok[] = {0.0f, -1.0f, -inf, -1e-30f};
  CHECK(log_gates(g_ok, 4, &w) == nullptr && w == -1);
  const float g_pos[] = {-1.0f, 1e-7f, -2.0f};
  CHECK(log_gates(g_pos, 3, &w) != nullptr && w == 1);
  const float g_nan[] = {-1.0f, -2.0f, nan};
  CHECK(log_gates(g_nan, 3, &w) != nullptr && w == 2);
  const float g_pinf[] = {inf};
  CHECK(log_gates(g_pinf, 1, &w) != nullptr && w == 0);
  const float o_ok[] = {1.0f, -3e38f, 0.0f};
  CHECK(finite_f32(o_ok, 3, &w) == nullptr);
  const float o_bad[] = {1.0f, 2.0f, -inf, nan};
  CHECK(finite_f32(o_bad, 4, &w) != nullptr && w == 2);
  const uint16_t b_ok[] = {0x3f80, 0xbf80, 0x7f7f, 0x0000};   // 1, -1, bf16 max, 0
  CHECK(finite_bf16(b_ok, 4, &w) == nullptr);
  const uint16_t b_fill[] = {0x3f80, 0xffff};                  // the all-ones NaN fill
  CHECK(finite_bf16(b_fill, 2, &w) != nullptr && w == 1);
  const uint16_t b_inf[] = {0x7f80};
  CHECK(finite_bf16(b_inf, 1, &w) != nullptr && w == 0);
  std::printf("ok\n");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validation_checks(tmp_path):
    src = tmp_path / "driver.cpp"
    src.write_text(DRIVER)
    exe = tmp_path / "driver"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
