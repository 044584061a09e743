// Value up-projection (hyper.ai summary of VideoMLA, Method section: the
// value of head h is v = W_uv[h] c). The softmax-weighted sum of the values is
// W_uv[h] applied once to the softmax-weighted latent:
//   out[b,i,h,:] = W_uv[h] o_lat[b,i,h,:]
// GEMM per head with both operands contiguous along the contraction (d_c):
// A = o_lat rows, B[k][n] = W_uv[h][n][k]. Work-group: 64 tokens x one head,
// each wave 16 tokens x all d_head outputs; W_uv[h] is staged in LDS in
// slabs of 64 output rows shared by the four waves. (The wide variant below
// serves d_c and d_head multiples of 32; this one the other shapes.)
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

template <typename T, int DC>
__global__ __launch_bounds__(256) void up_v_kernel(UpVParams p) {
  typedef typename V8<T>::type v8;
  constexpr int NKC = (DC + 31) / 32;
  constexpr int PADE = 16 / sizeof(T);
  constexpr int LS = NKC * 32 + PADE;  // LDS row stride, contraction zero-padded to 32
  constexpr int SLAB = 64;             // output rows (d) per LDS slab
  __shared__ __attribute__((aligned(16))) T wl[SLAB * LS];

  const int h = blockIdx.y;
  const int row0 = blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int H = p.H, dh = p.d_head;

  const int arow = row0 + wave * 16 + li;
  const bool arow_ok = arow < p.rows;
  const T* orow = (const T*)p.o_lat + ((size_t)(arow_ok ? arow : 0) * H + h) * DC;
  v8 a[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc)
    a[kc] = (arow_ok && kc * 32 + lg * 8 < DC) ? load8<T>(orow + kc * 32 + lg * 8) : zero8<T>();

  const T* wbase = (const T*)p.w_uv + (size_t)h * dh * DC;
  T* out = (T*)p.out;
  for (int n0 = 0; n0 < dh; n0 += SLAB) {
    __syncthreads();
    for (int e = tid; e < SLAB * (NKC * 4); e += 256) {
      const int r = e / (NKC * 4), c8 = (e % (NKC * 4)) * 8;
      const v8 v = (n0 + r < dh && c8 < DC) ? load8<T>(wbase + (size_t)(n0 + r) * DC + c8) : zero8<T>();
      store8<T>(wl + r * LS + c8, v);
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < SLAB / 16; ++nb) {
      if (n0 + nb * 16 >= dh) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const v8 bop = lds_load8<T>(wl + (nb * 16 + li) * LS + kc * 32 + lg * 8);
        acc = mma16(a[kc], bop, acc);
      }
      const int n = n0 + nb * 16 + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + wave * 16 + lg * 4 + i;
        if (r < p.rows && n < dh) out[((size_t)r * H + h) * dh + n] = to_t<T>(acc[i]);
      }
    }
  }
}

// Wide variant (d_c and d_head multiples of 32, d_head <= 128, every Wan
// width): out^T = W_uv[h] o_lat^T, W_uv[h] staged whole in LDS (every weight
// load issued before the first LDS write) with its rows in expand_pos order,
// so that a lane ends up with 8 consecutive outputs of one token and writes
// them as one piece.
constexpr int kUpVWideMaxHead = 128;

template <typename T, int DC>
__global__ __launch_bounds__(256) void up_v_wide_kernel(UpVParams p) {
  typedef typename V8<T>::type v8;
  constexpr int NKC = DC / 32;
  constexpr int PADE = 32 / sizeof(T);  // 32-byte row pad: a stride of 2 mod 4 16-byte chunks
  constexpr int LS = DC + PADE;
  constexpr int CPR = DC / 8;  // 8-element pieces per weight row
  constexpr int WPT = (kUpVWideMaxHead * CPR + 255) / 256;
  static_assert(DC % 32 == 0, "wide variant shapes");
  __shared__ __attribute__((aligned(16))) T wl[kUpVWideMaxHead * LS];

  const int h = blockIdx.y;
  const int row0 = blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int H = p.H, dh = p.d_head;

  const T* wbase = (const T*)p.w_uv + (size_t)h * dh * DC;
  v8 wst[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + 256 * i;
    if (e < dh * CPR) wst[i] = load8<T>(wbase + (size_t)(e / CPR) * DC + (e % CPR) * 8);
  }
  // this lane's token (column li of the B operand) and its latent fragments
  const int tok = row0 + wave * 16 + li;
  const bool tok_ok = tok < p.rows;
  const T* orow = (const T*)p.o_lat + ((size_t)(tok_ok ? tok : 0) * H + h) * DC;
  v8 ob[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) ob[kc] = tok_ok ? load8<T>(orow + kc * 32 + lg * 8) : zero8<T>();
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + 256 * i;
    if (e < dh * CPR) store8<T>(wl + expand_pos(e / CPR) * LS + (e % CPR) * 8, wst[i]);
  }
  __syncthreads();

  // lane: outputs 32 m + 8 lg .. + 7 of token tok
  T* dst = (T*)p.out + ((size_t)(tok_ok ? tok : 0) * H + h) * dh;
#pragma unroll 1
  for (int m = 0; m < dh / 32; ++m) {
    f32x4 acc[2] = {};
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        acc[half] = mma16(lds_load8<T>(wl + ((2 * m + half) * 16 + li) * LS + kc * 32 + lg * 8), ob[kc], acc[half]);
    float f[8] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3], acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
    if (tok_ok) store8<T>(dst + m * 32 + lg * 8, pack8<T>(f));
  }
}

template <typename T, int DC>
static hipError_t launch_up_v_t(const UpVParams& p, hipStream_t s) {
  dim3 grid((p.rows + 63) / 64, p.H);
  if constexpr (DC % 32 == 0) {
    if (p.d_head % 32 == 0 && p.d_head <= kUpVWideMaxHead) {
      hipLaunchKernelGGL((up_v_wide_kernel<T, DC>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((up_v_kernel<T, DC>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_up_v(int dtype, int d_c, int d_rope, const UpVParams& p, hipStream_t s) {
  (void)d_rope;
  if (p.rows <= 0) return hipSuccess;
  if (d_c == 192) return dtype == 0 ? launch_up_v_t<bf16, 192>(p, s) : launch_up_v_t<float, 192>(p, s);
  if (d_c == 160) return dtype == 0 ? launch_up_v_t<bf16, 160>(p, s) : launch_up_v_t<float, 160>(p, s);
  if (d_c == 128) return dtype == 0 ? launch_up_v_t<bf16, 128>(p, s) : launch_up_v_t<float, 128>(p, s);
  if (d_c == 16) return dtype == 0 ? launch_up_v_t<bf16, 16>(p, s) : launch_up_v_t<float, 16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
