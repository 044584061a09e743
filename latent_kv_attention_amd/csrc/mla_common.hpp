// Device helpers shared by the gfx950 kernels: element types, 8-element
// vectors, the 16x16x32 matrix-core product and the LDS transpose read.
//
// Lane layouts (checked on gfx950 with an in-bounds probe):
//   v_mfma_f32_16x16x32_bf16  A: lane l holds A[l%16][8*(l/16) + j], j = 0..7
//                             B: lane l holds B[8*(l/16) + j][l%16]
//                             C: lane l holds C[4*(l/16) + i][l%16], i = 0..3
//   ds_read_b64_tr_b16        in each 16-lane group, lane L = 4r + c supplies the
//                             address of 4 consecutive 16-bit elements; output
//                             lane i, element r = element (i%4) of lane 4r + i/4,
//                             i.e. column i of the 4 x 16 block the group loaded.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

#define MLA_LDS __attribute__((address_space(3)))

template <typename T>
struct V8;
template <>
struct V8<bf16> {
  typedef bf16x8 type;
  typedef u32x4 bits;
};
template <>
struct V8<float> {
  typedef f32x8 type;
  typedef u32x8 bits;
};

template <typename T>
__device__ __forceinline__ typename V8<T>::type zero8() {
  typename V8<T>::bits z = {};
  return __builtin_bit_cast(typename V8<T>::type, z);
}

// 8 consecutive elements (16 B for bf16, 32 B for float); p 16-byte aligned.
template <typename T>
__device__ __forceinline__ typename V8<T>::type load8(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  } else {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    u32x8 v = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return __builtin_bit_cast(f32x8, v);
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, typename V8<T>::type v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
  } else {
    u32x8 u = __builtin_bit_cast(u32x8, v);
    u32x4 a = {u[0], u[1], u[2], u[3]};
    u32x4 b = {u[4], u[5], u[6], u[7]};
    *reinterpret_cast<u32x4*>(p) = a;
    *reinterpret_cast<u32x4*>(p + 4) = b;
  }
}

template <typename T>
__device__ __forceinline__ T to_t(float f) {
  if constexpr (sizeof(T) == 2) {
    return (bf16)f;  // round to nearest even
  } else {
    return f;
  }
}

template <typename T>
__device__ __forceinline__ float to_f(T v) {
  return (float)v;
}

// 8 floats -> the 8-element operand vector of T.
template <typename T>
__device__ __forceinline__ typename V8<T>::type pack8(const float* f) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)f[j];
    return v;
  } else {
    f32x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = f[j];
    return v;
  }
}

// The 8 elements as floats (exact). bf16 is widened with bit operations.
// Note: __builtin_bit_cast applied directly to a vector element (v[k]) reads
// the vector's first element with this compiler; bit-cast only rvalues
// (expressions, or scalars passed through __uint_as_float).
template <typename T>
__device__ __forceinline__ void unpack8(typename V8<T>::type v, float* f) {
  if constexpr (sizeof(T) == 2) {
    u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __builtin_bit_cast(float, u[k] << 16);
      f[2 * k + 1] = __builtin_bit_cast(float, u[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = v[j];
  }
}

// C += A * B for one 16x16 output block with a contraction of 32, in the
// bf16 lane layout above. The float version issues eight 16x16x4 products,
// product j contracting element j of every lane's 8: the contraction index is
// permuted the same way for A and B, so the sum is the same.
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// Operand for a contraction over the ROW index of an LDS matrix M (row stride
// `stride` elements): lane (i = l%16, g = l/16) receives
//   [M[rowA + 0..3][col0 + i], M[rowB + 0..3][col0 + i]]
// where rowA, rowB may depend on g. Rows and columns must lie inside M;
// (row * stride + col0) must be a multiple of 4 elements.
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* m, int stride, int rowA, int rowB, int col0) {
  typedef __attribute__((__vector_size__(4 * sizeof(bf16)))) bf16 v4bf;
  const int L = threadIdx.x & 15;
  const int r = L >> 2, c4 = (L & 3) * 4;
  const bf16* pa = m + (rowA + r) * stride + col0 + c4;
  const bf16* pb = m + (rowB + r) * stride + col0 + c4;
  v4bf a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS v4bf*)(MLA_LDS bf16*)pa);
  v4bf b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS v4bf*)(MLA_LDS bf16*)pb);
  u32x2 ua = __builtin_bit_cast(u32x2, a);
  u32x2 ub = __builtin_bit_cast(u32x2, b);
  u32x4 u = {ua.x, ua.y, ub.x, ub.y};
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 lds_tr8(const float* m, int stride, int rowA, int rowB, int col0) {
  const int i = threadIdx.x & 15;
  f32x8 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = m[(rowA + r) * stride + col0 + i];
    v[4 + r] = m[(rowB + r) * stride + col0 + i];
  }
  return v;
}

// Output-feature order of the projection kernels that store 8-element
// pieces: a weight whose output features are staged at position
// expand_pos(d) (as rows, or as columns read through lds_tr8) makes the
// 16 x 16 output blocks 2m and 2m + 1 of a product leave lane l (g = l / 16)
// with features 32 m + 8 g .. 32 m + 8 g + 7 of one column (the C layout
// holds rows 4 g .. 4 g + 3 of each block), stored as one piece. Features
// 4 j .. 4 j + 3 stay consecutive.
__host__ __device__ constexpr int expand_pos(int d) {
  return (2 * (d / 32) + ((d % 8) >= 4 ? 1 : 0)) * 16 + 4 * ((d % 32) / 8) + d % 4;
}

// Elements 4 h .. 4 h + 3 of an 8-element vector to p (8-byte aligned for
// bf16, 16-byte for float).
template <typename T>
__device__ __forceinline__ void store_half8(T* p, typename V8<T>::type v, int h) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    *reinterpret_cast<u32x2*>(p) = h == 0 ? u32x2{u.x, u.y} : u32x2{u.z, u.w};
  } else {
    const u32x8 u = __builtin_bit_cast(u32x8, v);
    *reinterpret_cast<u32x4*>(p) = h == 0 ? u32x4{u[0], u[1], u[2], u[3]} : u32x4{u[4], u[5], u[6], u[7]};
  }
}

// 8 consecutive elements from LDS (16-byte aligned).
template <typename T>
__device__ __forceinline__ typename V8<T>::type lds_load8(const T* p) {
  return load8<T>(p);
}

__device__ __forceinline__ float wave_max_across_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_across_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order of a stream's window keys: by the frame their slot holds, oldest
// first (ties, which the ring never produces, by slot), token order inside a
// frame. Rank of the slot whose frame is `f` (this lane's slot `lane`, -1 =
// empty) among the valid slots; every lane of the wave passes its own slot.
// With keys in frame order, the keys a query of frame q may see under the
// frame-causal mask are a prefix of the window.
__device__ __forceinline__ int window_rank(int f, int lane) {
  int r = 0;
#pragma unroll 8
  for (int j = 0; j < 64; ++j) {
    const int fj = __shfl(f, j, 64);
    r += (fj >= 0 && (fj < f || (fj == f && j < lane))) ? 1 : 0;
  }
  return r;
}

// The same rank from the slot table directly (one thread, W reads).
__device__ __forceinline__ int window_rank_of_slot(const int32_t* sf, int W, int slot) {
  const int f = sf[slot];
  int r = 0;
  for (int j = 0; j < W; ++j) {
    const int fj = sf[j];
    r += (fj >= 0 && (fj < f || (fj == f && j < slot))) ? 1 : 0;
  }
  return r;
}

// Work-groups are dealt to the 8 XCDs round-robin (work-group i runs on XCD
// i mod 8). Work-group i gets logical index (XCD-major) so that each XCD's
// work-groups take consecutive work: with several streams (or heads) an XCD
// then walks few key sets and its L2 serves them, instead of every XCD
// touching every one. A bijection of [0, G) for any G.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_major(int id, int G) {
  const int q = G / kXcds, r = G % kXcds;
  const int x = id % kXcds, k = id / kXcds;
  return x * q + min(x, r) + k;
}

// Rotation of one interleaved pair by the angle whose cos/sin are given.
__device__ __forceinline__ void rotate_pair(float& a, float& b, float c, float s) {
  const float a0 = a, b0 = b;
  a = a0 * c - b0 * s;
  b = a0 * s + b0 * c;
}

}  // namespace mla
