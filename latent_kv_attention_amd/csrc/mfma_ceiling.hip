// Measurement aid, not part of the attention path: the dense bf16 matrix-core
// rate this GPU sustains in the attention kernel's occupancy (one work-group
// of 512 threads per compute unit, two waves per SIMD), with no memory or
// LDS traffic at all. Each wave chains v_mfma_f32_16x16x32_bf16 products
// into 8 independent accumulators, so the matrix core never waits for a
// result. The rate it reaches is the ceiling against which the attention
// kernel's own rate is read, beside the nominal peak.
//
// Built into its own library (libmla355_ceiling.so), so the attention
// library exports only its documented interface.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAcc = 8;  // independent accumulators per wave

// LDS held per work-group (unused but for one word): more than half of the
// 160 KB, so a compute unit holds one work-group, as it does in attention
constexpr int kPinFloats = 96 * 1024 / 4;

__global__ __launch_bounds__(512) void mfma_ceiling_kernel(float* sink, int iters) {
  __shared__ float pin[kPinFloats];
  const int t = threadIdx.x;
  const int pin_at = iters % kPinFloats;  // a run-time index keeps the whole array allocated
  if (t == 0) pin[pin_at] = (float)iters;
  __syncthreads();
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(t + j));
    b[j] = (__bf16)(0.002f * (float)(t - j));
  }
  f32x4 c[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) s += c[i].x + c[i].y + c[i].z + c[i].w;
  // the sum never takes this value for these operands; the store keeps the
  // products live without writing memory in a normal run
  if (s == 1234.5f + pin[pin_at]) sink[blockIdx.x * 512 + t] = s;
}

}  // namespace

extern "C" {

// FLOPs one launch performs: blocks x 8 waves x iters x 8 products x
// (2 x 16 x 16 x 32).
__attribute__((visibility("default"))) double mla_ceiling_flops(int32_t blocks, int32_t iters) {
  return (double)blocks * 8.0 * (double)iters * (double)kAcc * (2.0 * 16 * 16 * 32);
}

// Launch the kernel on `stream` (a hipStream_t; NULL = the default stream).
// sink: device buffer of at least blocks x 512 floats (written only in the
// impossible case above). Returns 0, or the HIP error code of the launch;
// 1 for blocks or iters outside [1, 65536] or [1, 1e7], or a NULL sink.
__attribute__((visibility("default"))) int32_t mla_ceiling_run(int32_t blocks, int32_t iters, float* sink,
                                                             void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 10000000 || sink == nullptr) return 1;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, sink, iters);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
