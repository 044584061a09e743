// Cache write (hyper.ai summary of VideoMLA, Method section): each token is
// projected once to its content latent c = W_dkv x and its unrotated
// positional key kR = W_kR x, and the row [c | kR] is stored into the
// sliding-window ring (chatpaper.ai abstract: fixed-size window), frame f in
// slot f mod W.
//
// GEMM view: out[r][n] = sum_k x[r][k] * Wcat[n][k], Wcat = [W_dkv ; W_kR]
// (N = d_c + d_rope). Both operands are contiguous along k, so every lane
// loads 8 consecutive elements straight into its matrix-core operand.
// Work-group tile: 64 token rows x 32 outputs, four waves of 16 rows each.
// The 1-D grid is walked XCD-major so that the output tiles sharing a block
// of token rows run on one XCD and its L2 serves the repeated x reads.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {
constexpr int kRowsPerBlock = 64;
constexpr int kColsPerBlock = 32;
constexpr int kXcds = 8;
}  // namespace

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p, int n_tiles_n, int n_logical,
                                                          int per_xcd) {
  typedef typename V8<T>::type v8;
  const int id = blockIdx.x;
  const int logical = (id % kXcds) * per_xcd + id / kXcds;
  if (logical >= n_logical) return;
  const int row_tile = logical / n_tiles_n;
  const int col_tile = logical % n_tiles_n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n_out = p.d_c + p.d_rope;

  if (logical == 0) {
    for (int e = tid; e < p.batch * p.n_frames; e += blockDim.x) {
      const int b = e / p.n_frames, f = p.frame_first + e % p.n_frames;
      p.slot_frame[b * p.W + f % p.W] = f;
    }
  }

  const int row = row_tile * kRowsPerBlock + wave * 16 + li;  // A-operand row of this lane
  const bool row_ok = row < p.rows;
  const T* xrow = (const T*)p.x + (size_t)(row_ok ? row : 0) * p.hidden;
  const T* wrow[2];
  bool col_ok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = col_tile * kColsPerBlock + nb * 16 + li;
    col_ok[nb] = n < n_out;
    const int nn = col_ok[nb] ? n : 0;
    wrow[nb] = nn < p.d_c ? (const T*)p.w_dkv + (size_t)nn * p.hidden
                          : (const T*)p.w_kr + (size_t)(nn - p.d_c) * p.hidden;
  }

  f32x4 acc[2] = {};
  for (int k0 = 0; k0 < p.hidden; k0 += 32) {
    const int k = k0 + lg * 8;
    const bool k_ok = k < p.hidden;
    const v8 a = (row_ok && k_ok) ? load8<T>(xrow + k) : zero8<T>();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const v8 b = (col_ok[nb] && k_ok) ? load8<T>(wrow[nb] + k) : zero8<T>();
      acc[nb] = mma16(a, b, acc[nb]);
    }
  }

  // lane holds out[4*lg + i][16*nb + li] of this wave's 16 x 32 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_tile * kRowsPerBlock + wave * 16 + lg * 4 + i;
    if (r >= p.rows) continue;
    const int b = r / p.rows_per_b, local = r % p.rows_per_b;
    const int f = p.frame_first + local / p.T, tok = local % p.T;
    T* dst = (T*)p.cache + (((size_t)b * p.W + f % p.W) * p.T + tok) * n_out;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = col_tile * kColsPerBlock + nb * 16 + li;
      if (n < n_out) dst[n] = to_t<T>(acc[nb][i]);
    }
  }
}

hipError_t launch_cache_write(int dtype, int d_c, int d_rope, const CacheWriteParams& p, hipStream_t s) {
  (void)d_c;
  (void)d_rope;
  const int n_out = p.d_c + p.d_rope;
  const int n_tiles_n = (n_out + kColsPerBlock - 1) / kColsPerBlock;
  const int n_tiles_m = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int n_logical = n_tiles_m * n_tiles_n;
  const int per_xcd = (n_logical + kXcds - 1) / kXcds;
  const int grid = per_xcd * kXcds;
  if (dtype == 0)
    hipLaunchKernelGGL(cache_write_kernel<bf16>, dim3(grid), dim3(256), 0, s, p, n_tiles_n, n_logical, per_xcd);
  else
    hipLaunchKernelGGL(cache_write_kernel<float>, dim3(grid), dim3(256), 0, s, p, n_tiles_n, n_logical, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
