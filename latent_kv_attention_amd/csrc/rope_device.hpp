// Table lookup for one rotary pair of the 3D-RoPE block [t | y | x]
// (hyper.ai summary of VideoMLA, Method section: 3D-RoPE on the positional
// key and query). Pair `pr` of the d_rope dims belongs to the t block when
// 2*pr < d_t, to the y block when 2*pr < d_t + d_y, else to the x block.
#pragma once

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

// t is an absolute frame index; it is clamped into the table's range so that a
// frame outside it reads a valid (if wrong) row instead of leaving the buffer.
__device__ __forceinline__ void rope_cos_sin(const RopeLayout& rl, const float* __restrict__ tab, int pr, int t,
                                             int y, int x, float& c, float& s) {
  int off;
  if (2 * pr < rl.d_t) {
    int tt = t - rl.t_first;
    tt = tt < 0 ? 0 : (tt >= rl.n_t ? rl.n_t - 1 : tt);
    off = tt * (rl.d_t / 2) + pr;
    c = tab[rl.off_ct + off];
    s = tab[rl.off_st + off];
  } else if (2 * pr < rl.d_t + rl.d_y) {
    off = y * (rl.d_y / 2) + pr - rl.d_t / 2;
    c = tab[rl.off_cy + off];
    s = tab[rl.off_sy + off];
  } else {
    off = x * (rl.d_x / 2) + pr - (rl.d_t + rl.d_y) / 2;
    c = tab[rl.off_cx + off];
    s = tab[rl.off_sx + off];
  }
}

}  // namespace mla
