// Query absorb and rotate (hyper.ai summary of VideoMLA, Method section: the
// score of head h is q_nope . k_nope + q_rope . k_rope with k_nope = W_uk[h] c
// and k_rope the rotated shared key). Since q . (W_uk[h] c) = (W_uk[h]^T q) . c,
// the query is mapped once into latent space, multiplied by the softmax
// temperature in log2 units (qscale = scale * log2 e) so that scores come out
// of the matrix product ready for exp2:
//   q_abs[b,i,h] = qscale [ W_uk[h]^T q_nope[b,i,h] | R(t,y,x) q_r[b,i,h] | 0 ... ]
// Work-group: 128 query tokens x one head (8 waves of 16 tokens, so W_uk[h]
// is read once per 128 tokens). The 32-row slabs of W_uk[h] are staged in
// LDS and read with the transposing LDS load, because the contraction runs
// over W_uk's row index. (The wide variant below serves d_c and d_head
// multiples of 32; this one the other shapes.)
#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

constexpr int kAbsorbRows = 128;               // query tokens per work-group
constexpr int kAbsorbThreads = kAbsorbRows * 4;  // one wave per 16 tokens

template <typename T, int DC, int DR>
__global__ __launch_bounds__(kAbsorbThreads) void absorb_q_kernel(AbsorbParams p) {
  typedef typename V8<T>::type v8;
  constexpr int KP = (DC + DR + 31) / 32 * 32;
  constexpr int PADE = 16 / sizeof(T);
  constexpr int LS = DC + PADE;
  constexpr int NNB = DC / 16;
  __shared__ __attribute__((aligned(16))) T wl[32 * LS];

  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kAbsorbRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int H = p.H, dh = p.d_head;

  const int arow = row0 + wave * 16 + li;
  const bool arow_ok = arow < p.rows;
  const T* qrow = (const T*)p.q_nope + ((size_t)(arow_ok ? arow : 0) * H + h) * dh;
  const T* wbase = (const T*)p.w_uk + (size_t)h * dh * DC;

  f32x4 acc[NNB] = {};
  for (int k0 = 0; k0 < dh; k0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * (DC / 8); e += kAbsorbThreads) {
      const int r = e / (DC / 8), c8 = (e % (DC / 8)) * 8;
      const v8 v = (k0 + r < dh) ? load8<T>(wbase + (size_t)(k0 + r) * DC + c8) : zero8<T>();
      store8<T>(wl + r * LS + c8, v);
    }
    __syncthreads();
    const v8 a = (arow_ok && k0 + lg * 8 < dh) ? load8<T>(qrow + k0 + lg * 8) : zero8<T>();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      const typename V8<T>::type bop = lds_tr8(wl, LS, lg * 8, lg * 8 + 4, nb * 16);
      acc[nb] = mma16(a, bop, acc[nb]);
    }
  }

  T* qa = (T*)p.q_abs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + wave * 16 + lg * 4 + i;
    if (r >= p.rows) continue;
    T* dst = qa + ((size_t)r * H + h) * KP;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) dst[nb * 16 + li] = to_t<T>(acc[nb][i] * p.qscale);
  }

  // rotated positional part and zero padding
  constexpr int NPR = DR / 2;
  for (int e = tid; e < kAbsorbRows * NPR; e += kAbsorbThreads) {
    const int r = row0 + e / NPR, pr = e % NPR;
    if (r >= p.rows) continue;
    const int i = r % p.n_q;
    const int t = p.q_frame_first + i / p.T, tok = i % p.T;
    const int y = tok / p.grid_x, x = tok % p.grid_x;
    const T* src = (const T*)p.q_r + ((size_t)r * H + h) * DR + 2 * pr;
    float a0 = to_f<T>(src[0]), a1 = to_f<T>(src[1]);
    float c, s;
    rope_cos_sin(p.rl, p.tables, pr, t, y, x, c, s);
    rotate_pair(a0, a1, c, s);
    T* dst = qa + ((size_t)r * H + h) * KP + DC + 2 * pr;
    dst[0] = to_t<T>(a0 * p.qscale);
    dst[1] = to_t<T>(a1 * p.qscale);
  }
  if constexpr (KP > DC + DR) {
    constexpr int NPAD = KP - DC - DR;
    for (int e = tid; e < kAbsorbRows * NPAD; e += kAbsorbThreads) {
      const int r = row0 + e / NPAD;
      if (r >= p.rows) continue;
      qa[((size_t)r * H + h) * KP + DC + DR + e % NPAD] = to_t<T>(0.f);
    }
  }
}

// Wide variant (d_c and d_head multiples of 32, d_head <= 128, every Wan
// width): the product runs transposed, q_abs^T = W_uk[h]^T q_nope^T, with
// W_uk[h] staged whole in LDS (every weight load issued before the first LDS
// write) and its columns in expand_pos order, so that a lane ends up with 8
// consecutive latent values of one token and writes them as one piece; the
// positional part is rotated 8 values (4 pairs) per thread.
constexpr int kAbsorbWideMaxHead = 128;

template <typename T, int DC, int DR>
__global__ __launch_bounds__(kAbsorbThreads) void absorb_q_wide_kernel(AbsorbParams p) {
  typedef typename V8<T>::type v8;
  constexpr int KP = (DC + DR + 31) / 32 * 32;
  constexpr int PADE = 32 / sizeof(T);  // 32-byte row pad: a stride of 2 mod 4 16-byte chunks
  constexpr int LS = DC + PADE;
  constexpr int CPR = DC / 8;  // 8-element pieces per weight row
  constexpr int NKM = kAbsorbWideMaxHead / 32;
  constexpr int WPT = (kAbsorbWideMaxHead * CPR + kAbsorbThreads - 1) / kAbsorbThreads;
  static_assert(DC % 32 == 0 && DR % 8 == 0, "wide variant shapes");
  __shared__ __attribute__((aligned(16))) T wl[kAbsorbWideMaxHead * LS];

  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kAbsorbRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int H = p.H, dh = p.d_head, nkc = dh / 32;

  const T* wbase = (const T*)p.w_uk + (size_t)h * dh * DC;
  v8 wst[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + kAbsorbThreads * i;
    if (e < dh * CPR) wst[i] = load8<T>(wbase + (size_t)(e / CPR) * DC + (e % CPR) * 8);
  }
  // this lane's token (column li of the B operand) and its query fragments
  const int tok = row0 + wave * 16 + li;
  const bool tok_ok = tok < p.rows;
  const T* qrow = (const T*)p.q_nope + ((size_t)(tok_ok ? tok : 0) * H + h) * dh;
  v8 qb[NKM];
#pragma unroll
  for (int kc = 0; kc < NKM; ++kc) qb[kc] = (tok_ok && kc < nkc) ? load8<T>(qrow + kc * 32 + lg * 8) : zero8<T>();
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + kAbsorbThreads * i;
    if (e < dh * CPR) {
      const int r = e / CPR, d0 = (e % CPR) * 8;
      store_half8<T>(wl + r * LS + expand_pos(d0), wst[i], 0);
      store_half8<T>(wl + r * LS + expand_pos(d0 + 4), wst[i], 1);
    }
  }
  __syncthreads();

  // lane: latent values 32 m + 8 lg .. + 7 of token tok
  T* qa = (T*)p.q_abs + ((size_t)(tok_ok ? tok : 0) * H + h) * KP;
#pragma unroll 1
  for (int m = 0; m < DC / 32; ++m) {
    f32x4 acc[2] = {};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int kc = 0; kc < NKM; ++kc)
        if (kc < nkc)
          acc[half] = mma16(lds_tr8(wl, LS, kc * 32 + lg * 8, kc * 32 + lg * 8 + 4, (2 * m + half) * 16), qb[kc],
                            acc[half]);
    }
    float f[8] = {acc[0][0] * p.qscale, acc[0][1] * p.qscale, acc[0][2] * p.qscale, acc[0][3] * p.qscale,
                  acc[1][0] * p.qscale, acc[1][1] * p.qscale, acc[1][2] * p.qscale, acc[1][3] * p.qscale};
    if (tok_ok) store8<T>(qa + m * 32 + lg * 8, pack8<T>(f));
  }

  // rotated positional part (4 pairs per thread) and zero padding
  constexpr int NPC = DR / 8;
  for (int e = tid; e < kAbsorbRows * NPC; e += kAbsorbThreads) {
    const int r = row0 + e / NPC, c = e % NPC;
    if (r >= p.rows) continue;
    const int i = r % p.n_q;
    const int t = p.q_frame_first + i / p.T, tk = i % p.T;
    const int y = tk / p.grid_x, x = tk % p.grid_x;
    float f[8];
    unpack8<T>(load8<T>((const T*)p.q_r + ((size_t)r * H + h) * DR + c * 8), f);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float cs, sn;
      rope_cos_sin(p.rl, p.tables, c * 4 + k, t, y, x, cs, sn);
      rotate_pair(f[2 * k], f[2 * k + 1], cs, sn);
      f[2 * k] *= p.qscale;
      f[2 * k + 1] *= p.qscale;
    }
    store8<T>((T*)p.q_abs + ((size_t)r * H + h) * KP + DC + c * 8, pack8<T>(f));
  }
  if constexpr (KP > DC + DR) {
    constexpr int NPAD = (KP - DC - DR) / 8;
    for (int e = tid; e < kAbsorbRows * NPAD; e += kAbsorbThreads) {
      const int r = row0 + e / NPAD;
      if (r >= p.rows) continue;
      store8<T>((T*)p.q_abs + ((size_t)r * H + h) * KP + DC + DR + (e % NPAD) * 8, zero8<T>());
    }
  }
}

template <typename T, int DC, int DR>
static hipError_t launch_absorb_t(const AbsorbParams& p, hipStream_t s) {
  dim3 grid((p.rows + kAbsorbRows - 1) / kAbsorbRows, p.H);
  if constexpr (DC % 32 == 0 && DR % 8 == 0) {
    if (p.d_head % 32 == 0 && p.d_head <= kAbsorbWideMaxHead) {
      hipLaunchKernelGGL((absorb_q_wide_kernel<T, DC, DR>), grid, dim3(kAbsorbThreads), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((absorb_q_kernel<T, DC, DR>), grid, dim3(kAbsorbThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_absorb_q(int dtype, int d_c, int d_rope, const AbsorbParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
#define MLA_ABSORB_CASE(DCV, DRV) \
  if (d_c == DCV && d_rope == DRV) return dtype == 0 ? launch_absorb_t<bf16, DCV, DRV>(p, s) : launch_absorb_t<float, DCV, DRV>(p, s);
  MLA_ABSORB_CASE(192, 32)
  MLA_ABSORB_CASE(128, 32)
  MLA_ABSORB_CASE(160, 64)
  MLA_ABSORB_CASE(192, 64)
  MLA_ABSORB_CASE(16, 8)
#undef MLA_ABSORB_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
