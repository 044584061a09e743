// 3D-RoPE cos/sin tables (hyper.ai summary of VideoMLA, Method section: the
// cached positional key is rotated by 3D-RoPE over (t, h, w) at attention
// time). One thread per (position, pair) entry of the three axis tables; the
// angle pos * base^(-2i/d_axis) is formed in double precision and rounded to
// float once.
#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

__global__ __launch_bounds__(256) void rope_tables_kernel(RopeTableParams p) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= p.total) return;
  const RopeLayout& rl = p.rl;
  const int nt = rl.n_t * (rl.d_t / 2);
  const int ny = p.grid_y * (rl.d_y / 2);
  int pos, i, d, off_c, off_s, idx;
  if (e < nt) {
    const int h = rl.d_t / 2;
    pos = rl.t_first + e / h;
    i = e % h;
    d = rl.d_t;
    off_c = rl.off_ct;
    off_s = rl.off_st;
    idx = e;
  } else if (e < nt + ny) {
    const int h = rl.d_y / 2, q = e - nt;
    pos = q / h;
    i = q % h;
    d = rl.d_y;
    off_c = rl.off_cy;
    off_s = rl.off_sy;
    idx = q;
  } else {
    const int h = rl.d_x / 2, q = e - nt - ny;
    pos = q / h;
    i = q % h;
    d = rl.d_x;
    off_c = rl.off_cx;
    off_s = rl.off_sx;
    idx = q;
  }
  float c, sn;
  rope_axis_cos_sin(p.base, pos, i, d, &c, &sn);
  p.tables[off_c + idx] = c;
  p.tables[off_s + idx] = sn;
}

hipError_t launch_rope_tables(const RopeTableParams& p, hipStream_t s) {
  if (p.total <= 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (p.total + threads - 1) / threads;
  hipLaunchKernelGGL(rope_tables_kernel, dim3(blocks), dim3(threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
