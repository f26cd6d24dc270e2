"""Host logic of the GEMM tile order (flow_matching_diffusion_amd/csrc/k2_tiles.h), compiled with the
host C++ compiler: every workgroup index maps to a distinct output tile, for every grid shape and
super-column width, and the super-column widths cover the N tiles in near-equal parts; the attention
grid's XCD-contiguous work map is a bijection too."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "flow_matching_diffusion_amd", "csrc", "k2_tiles.h")

PROGRAM = r"""
#define __host__
#define __device__
#include <cstdio>
#include <vector>
#include "k2_tiles.h"
int main() {
  long bad = 0, cases = 0;
  // bijection: tiles_m x tiles_n grids, every super-column width
  for (int tm_ = 1; tm_ <= 40; ++tm_)
    for (int tn_ = 1; tn_ <= 140; tn_ += (tn_ < 40 ? 1 : 7))
      for (int scn = 1; scn <= tn_ + 1; scn += (scn < 12 ? 1 : 5)) {
        ++cases;
        std::vector<int> seen(tm_ * tn_, 0);
        for (int bid = 0; bid < tm_ * tn_; ++bid) {
          int a = -1, b = -1;
          k2::tile_coords(bid, tm_, tn_, scn, a, b);
          if (a < 0 || a >= tm_ || b < 0 || b >= tn_) { ++bad; continue; }
          seen[a * tn_ + b]++;
        }
        for (int v : seen) bad += v != 1;
      }
  // xcd_item: a bijection, each XCD's items contiguous and in slot order
  for (int total = 1; total <= 5000; total += (total < 100 ? 1 : 37)) {
    ++cases;
    std::vector<int> seen(total, 0), last(8, -1);
    for (int bid = 0; bid < total; ++bid) {
      const int it = k2::xcd_item(bid, total);
      if (it < 0 || it >= total) { ++bad; continue; }
      seen[it]++;
      const int x = bid & 7;
      if (last[x] >= 0 && it != last[x] + 1) ++bad;
      last[x] = it;
    }
    for (int v : seen) bad += v != 1;
  }
  // xcd_item_rows: a bijection; with per_b a multiple of 8 every XCD takes per_b / 8 items of each
  // group, contiguous within the group and in slot order
  for (int B = 1; B <= 5; ++B)
    for (int per_b = 1; per_b <= 700; per_b += (per_b < 64 ? 1 : 29)) {
      ++cases;
      const int total = B * per_b;
      std::vector<int> seen(total, 0), last(8, -1);
      std::vector<std::vector<int>> share(8, std::vector<int>(B, 0));
      for (int bid = 0; bid < total; ++bid) {
        const int it = k2::xcd_item_rows(bid, per_b, B);
        if (it < 0 || it >= total) { ++bad; continue; }
        seen[it]++;
        const int x = bid & 7;
        share[x][it / per_b]++;
        if (per_b % 8 == 0 && last[x] >= 0 && it / per_b == last[x] / per_b && it != last[x] + 1) ++bad;
        last[x] = it;
      }
      for (int v : seen) bad += v != 1;
      if (per_b % 8 == 0)
        for (int x = 0; x < 8; ++x)
          for (int b = 0; b < B; ++b) bad += share[x][b] != per_b / 8;
    }
  // the block's GEMM shapes at 1024^2: 36 M tiles; N tiles 60 (qkvg), 24 (out, down), 128 (swiglu)
  const int shapes[][3] = {{60, 6144, 0}, {24, 6144, 0}, {128, 6144, 0}, {24, 16384, 0}};
  for (auto& sh : shapes) {
    const int w = k2::super_cols(sh[0], 256, sh[1], 2);
    printf("tiles_n %d K %d -> super-column width %d\n", sh[0], sh[1], w);
    if (w < 1 || w > sh[0]) ++bad;
    if ((size_t)w * 256 * sh[1] * 2 > k2::kSuperColumnBytes && w > 1) ++bad;
  }
  printf("cases %ld bad %ld\n", cases, bad);
  return bad != 0;
}
"""


def test_tile_order_is_a_bijection(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "tiles.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "tiles"
    subprocess.run([cxx, "-O2", "-std=c++17", "-I", os.path.dirname(HDR), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert "bad 0" in out.stdout
