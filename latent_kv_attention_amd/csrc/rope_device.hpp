// 3D-RoPE on the device (hyper.ai summary of VideoMLA, Method section: the
// positional key and query are rotated by 3D-RoPE over (t, y, x)). Pair `pr`
// of the d_rope dims belongs to the t block when 2*pr < d_t, to the y block
// when 2*pr < d_t + d_y, else to the x block.
#pragma once

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

// cos and sin of pos * base^(-2i/d) for pair i of an axis of d dims: the
// angle in double precision, each value rounded to float once. The table
// kernel and the per-call rotation of the window's keys both use this
// function (kept out of line, so both get the same instruction sequence),
// which lets the keys' temporal angles be formed for any frame without a
// table while agreeing with the table entries the queries use.
static __device__ __noinline__ void rope_axis_cos_sin(double base, int pos, int i, int d, float* c, float* s) {
  const double inv_freq = pow(base, -2.0 * (double)i / (double)d);
  const double ang = (double)pos * inv_freq;
  *c = (float)cos(ang);
  *s = (float)sin(ang);
}

// Table lookup for the query side. The callers check that every query frame
// lies in the table's t range; t is still clamped so that no index can leave
// the buffer.
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
