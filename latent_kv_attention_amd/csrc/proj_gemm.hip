// Dense projections on either side of the chunk attention (hyper.ai summary
// of VideoMLA, Method section): the query latent cQ = W_dq x of each chunk
// token, the per-head content and positional queries W_uq[h] cQ and
// W_qr[h] cQ, and the output projection W_o [o_1; ...; o_H] of the
// concatenated heads (the standard multi-head attention output; the pages do
// not spell it out).
//
// All of them are one GEMM shape: C[M][N] = A[M][K] B[N][K]^T, with the
// weight B stored as [out features][in features], so both operands are
// contiguous along the contraction and each lane's 8-element matrix-core
// operand is one 16-byte row piece, read from LDS without a transpose.
//
// Work-group tile 128 x 128 outputs, or 64 x 64 when the problem has too
// few 128-tiles to fill the chip; 64-wide K steps through two LDS stage
// buffers: the next step's operands are loaded into registers while the
// matrix cores work on the current one, then stored into the other buffer
// (one barrier per step). Rows of the staged tiles are padded by 32 bytes
// (a row stride of 10 sixteen-byte chunks): measured with the bank-conflict
// counter, 128-bit reads of rows at a stride of 2 mod 4 chunks are
// conflict-free and odd strides conflict 2-way (the 16-byte pad, a stride of
// 9, made the projections 5-6% slower). The output tile
// leaves through LDS in 16-byte row pieces. Tiles are numbered row-major and
// dealt to the 8 XCDs in contiguous ranges, so tiles that share A rows share
// an L2.
//
// The output features may come in two parts with their own weight and
// output arrays (features n >= n_split: weight B2 row n - n_split, output
// C2 column n - n_split), so that the per-head content and positional
// queries, which read the same query latent, are one launch. The second
// part's weight may itself be two arrays (B2, then B3 from n_split2 on).
//
// Ring variant (RING): the second part is the cache write of the same
// tokens (hyper.ai summary, Method: the query latent and the compressed
// latent both come from the token): x [W_dq ; W_dkv ; W_kR]^T gives the
// query latent and each token's cached row [c | kR] in one pass over x, and
// the epilogue stores the cached rows into their ring slots.
//
// Absorbed-query variant (QABS): the weight is the per-head stack
// [W_uk[h]^T W_uq[h] ; W_qr[h] ; 0] (qabs_weights_kernel), so one product
// of the query latent gives every head's absorbed content query and
// unrotated positional query, and the epilogue finishes them the way the
// attention reads them: the output tile is staged in float, positional
// pairs are rotated by 3D-RoPE at the row's (t, y, x), everything is scaled
// by the softmax factor in log2 units, then rounded once.
#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

namespace {
constexpr int kGemmBK = 64;
constexpr int kGemmXcds = 8;
}  // namespace

template <typename T, int BM, int BN, bool QABS, bool RING>
__global__ __launch_bounds__(256) void gemm_nt_kernel(GemmParams p) {
  typedef typename V8<T>::type v8;
  constexpr int BK = kGemmBK;
  constexpr int PAD = 32 / sizeof(T);          // 32-byte row pad: a stride of 2 mod 4 16-byte chunks
  constexpr int LDK = BK + PAD;                 // staged row stride (elements)
  constexpr int LDC = BN + PAD;                 // output staging row stride
  constexpr int CHUNKS = BK / 8;                // 8-element pieces per staged row
  constexpr int NLD = (BM + BN) * CHUNKS / 256; // pieces per thread per K step
  constexpr int STAGE = (BM + BN) * LDK;        // elements of one stage buffer
  constexpr int WM = BM / 2, WN = BN / 2;       // wave tile (2 x 2 waves)
  constexpr int NMB = WM / 16, NNB = WN / 16;
  static_assert((BM + BN) * CHUNKS % 256 == 0, "whole pieces per thread");
  static_assert(BM * LDC <= 2 * STAGE, "output tile fits in the stage buffers");
  constexpr int LDF = BN + 4;  // float output staging row stride (QABS)
  static_assert(!QABS || BM * LDF * 4 <= 2 * STAGE * (int)sizeof(T), "float output tile fits in the stage buffers");
  __shared__ __attribute__((aligned(16))) T lds[2 * STAGE];

  const int logical = (blockIdx.x % kGemmXcds) * p.per_xcd + blockIdx.x / kGemmXcds;
  if (logical >= p.n_logical) return;
  if constexpr (RING) {
    if (logical == 0) {
      for (int e = threadIdx.x; e < p.ring.batch * p.ring.n_frames; e += blockDim.x) {
        const int b = e / p.ring.n_frames, f = p.ring.frame_first + e % p.ring.n_frames;
        p.ring.slot_frame[b * p.ring.W + f % p.ring.W] = f;
      }
    }
  }
  const int row0 = (logical / p.tiles_n) * BM;
  const int col0 = (logical % p.tiles_n) * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // staged row r < BM is A row row0 + r, else output feature n = col0 + r - BM
  // (B row n, or B2 row n - n_split past the split); rows past the end
  // repeat the last row (their products are never stored)
  const T* src[NLD];
  int dst[NLD], kof[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int e = tid + 256 * j;
    const int r = e / CHUNKS, c = e % CHUNKS;
    if (r < BM) {
      src[j] = (const T*)p.a + (size_t)min(row0 + r, p.M - 1) * p.lda + c * 8;
    } else {
      const int n = min(col0 + r - BM, p.N - 1);
      src[j] = n < p.n_split ? (const T*)p.b + (size_t)n * p.ldb + c * 8
               : n < p.n_split2 ? (const T*)p.b2 + (size_t)(n - p.n_split) * p.ldb + c * 8
                                : (const T*)p.b3 + (size_t)(n - p.n_split2) * p.ldb + c * 8;
    }
    dst[j] = r * LDK + c * 8;
    kof[j] = c * 8;
  }
  v8 stage[NLD];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) stage[j] = k0 + kof[j] < p.K ? load8<T>(src[j] + k0) : zero8<T>();
  };
  auto stash = [&](T* buf) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) store8<T>(buf + dst[j], stage[j]);
  };

  f32x4 acc[NMB][NNB] = {};
  auto compute = [&](const T* buf) {
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      v8 af[NMB], bf[NNB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) af[mb] = lds_load8<T>(buf + (wm * WM + mb * 16 + li) * LDK + kk * 32 + lg * 8);
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
        bf[nb] = lds_load8<T>(buf + (BM + wn * WN + nb * 16 + li) * LDK + kk * 32 + lg * 8);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) acc[mb][nb] = mma16(af[mb], bf[nb], acc[mb][nb]);
    }
  };

  // two stage buffers: step k computes from buffer k % 2 while the operands
  // of step k + 1 travel to registers and then into the other buffer, which
  // every wave finished reading before the barrier that ended step k - 1
  const int nk = (p.K + BK - 1) / BK;
  fetch(0);
  stash(lds);
  __syncthreads();
  for (int k = 0; k < nk; ++k) {
    if (k + 1 < nk) fetch((k + 1) * BK);
    compute(lds + (k & 1) * STAGE);
    if (k + 1 < nk) stash(lds + ((k + 1) & 1) * STAGE);
    __syncthreads();
  }

  if constexpr (QABS) {
    float* ft = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ft[(wm * WM + mb * 16 + lg * 4 + i) * LDF + wn * WN + nb * 16 + li] = acc[mb][nb][i];
    __syncthreads();
    const GemmQabs& q = p.qa;
    // 8-column pieces lie inside one region of a head's row (dc, dr, kp are multiples of 8)
    for (int e = tid; e < BM * (BN / 8); e += 256) {
      const int r = e / (BN / 8), c8 = (e % (BN / 8)) * 8;
      const int row = row0 + r, n = col0 + c8;
      if (row >= p.M || n >= p.N) continue;
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = ft[r * LDF + c8 + j];
      const int jj = n % q.kp;
      if (jj >= q.dc && jj < q.dc + q.dr) {
        const int i = row % q.n_q;
        const int t = q.q_frame_first + i / q.T, tok = i % q.T;
        const int y = tok / q.grid_x, x = tok % q.grid_x;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float c, sn;
          rope_cos_sin(q.rl, q.tables, (jj - q.dc) / 2 + k, t, y, x, c, sn);
          rotate_pair(f[2 * k], f[2 * k + 1], c, sn);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] *= q.qscale;
      store8<T>((T*)p.c + (size_t)row * p.ldc + n, pack8<T>(f));
    }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lds[(wm * WM + mb * 16 + lg * 4 + i) * LDC + wn * WN + nb * 16 + li] = to_t<T>(acc[mb][nb][i]);
  __syncthreads();
  // 8-column pieces never straddle n_split (both multiples of 8)
  for (int e = tid; e < BM * (BN / 8); e += 256) {
    const int r = e / (BN / 8), c8 = (e % (BN / 8)) * 8;
    const int n = col0 + c8;
    if (row0 + r < p.M && n < p.N) {
      size_t row2 = (size_t)(row0 + r);
      if constexpr (RING) {
        const GemmRing& g = p.ring;
        const int b = (row0 + r) / g.rows_per_b, t = (row0 + r) - b * g.rows_per_b;
        row2 = ((size_t)b * g.W + (g.frame_first + t / g.T) % g.W) * g.T + t % g.T;
      }
      T* dstp = n < p.n_split ? (T*)p.c + (size_t)(row0 + r) * p.ldc + n : (T*)p.c2 + row2 * p.ldc2 + (n - p.n_split);
      store8<T>(dstp, lds_load8<T>(lds + r * LDC + c8));
    }
  }
}

int gemm_tile_rows(int M, int N, int n_cu) {
  const long long big = (long long)((M + 127) / 128) * ((N + 127) / 128);
  return big >= n_cu ? 128 : 64;
}

template <typename T, int BM, int BN, bool QABS, bool RING>
static hipError_t launch_gemm_t(GemmParams p, hipStream_t s) {
  p.tiles_n = (p.N + BN - 1) / BN;
  p.n_logical = ((p.M + BM - 1) / BM) * p.tiles_n;
  p.per_xcd = (p.n_logical + kGemmXcds - 1) / kGemmXcds;
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, QABS, RING>), dim3(p.per_xcd * kGemmXcds), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool QABS, bool RING>
static hipError_t launch_gemm_any(int dtype, const GemmParams& p, int tile_rows, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (tile_rows == 128)
    return dtype == 0 ? launch_gemm_t<bf16, 128, 128, QABS, RING>(p, s)
                      : launch_gemm_t<float, 128, 128, QABS, RING>(p, s);
  if (tile_rows == 64)
    return dtype == 0 ? launch_gemm_t<bf16, 64, 64, QABS, RING>(p, s) : launch_gemm_t<float, 64, 64, QABS, RING>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_nt(int dtype, const GemmParams& p, int tile_rows, hipStream_t s) {
  return launch_gemm_any<false, false>(dtype, p, tile_rows, s);
}

hipError_t launch_gemm_qabs(int dtype, const GemmParams& p, int tile_rows, hipStream_t s) {
  return launch_gemm_any<true, false>(dtype, p, tile_rows, s);
}

hipError_t launch_gemm_ring(int dtype, const GemmParams& p, int tile_rows, hipStream_t s) {
  return launch_gemm_any<false, true>(dtype, p, tile_rows, s);
}

// Absorbed query weights, once per layer: one thread per output element,
// fp32 sums over d_head, rounded once to the element type.
template <typename T>
__global__ __launch_bounds__(256) void qabs_weights_kernel(QabsWeightParams p) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int j = blockIdx.y, h = blockIdx.z;
  if (c >= p.d_cq) return;
  float v = 0.f;
  if (j < p.dc) {
    const T* uk = (const T*)p.w_uk + (size_t)h * p.d_head * p.dc + j;
    const T* uq = (const T*)p.w_uq + (size_t)h * p.d_head * p.d_cq + c;
    for (int i = 0; i < p.d_head; ++i) v += to_f<T>(uk[(size_t)i * p.dc]) * to_f<T>(uq[(size_t)i * p.d_cq]);
  } else if (j < p.dc + p.dr) {
    v = to_f<T>(((const T*)p.w_qr)[((size_t)h * p.dr + (j - p.dc)) * p.d_cq + c]);
  }
  ((T*)p.w_qabs)[((size_t)h * p.kp + j) * p.d_cq + c] = to_t<T>(v);
}

hipError_t launch_qabs_weights(int dtype, const QabsWeightParams& p, hipStream_t s) {
  dim3 grid((p.d_cq + 255) / 256, p.kp, p.H);
  if (dtype == 0)
    hipLaunchKernelGGL(qabs_weights_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(qabs_weights_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
