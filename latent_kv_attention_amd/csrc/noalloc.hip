// mla_flash_attend_noalloc: the latent flash attention for callers that
// cannot allocate device memory (code under graph capture, serving loops,
// harnesses that forbid hipMalloc). Its workspace is a fixed array that the
// library holds on each GPU; the call itself allocates nothing.
#include <atomic>

#include "../../include/mla.h"
#include "abi_internal.hpp"
#include "mla_internal.hpp"

#define MLA_API extern "C" __attribute__((visibility("default")))

// One fixed array per GPU, part of this file's code object (each device that
// loads it holds its own copy until the process ends). In host code the name
// only stands for the symbol; the array's device address on the current
// device comes from hipGetSymbolAddress and is the only form ever passed to a
// kernel.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;

// Device address of `scratch` on each device, looked up once, by the first
// call made with that device current: state 0 = not looked up, 1 = lookup in
// progress (other threads wait for it), 2 = address ready.
std::atomic<int> g_scratch_state[kMaxDevices];
void* g_scratch_addr[kMaxDevices];

mla_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  for (;;) {
    int st = g_scratch_state[dev].load(std::memory_order_acquire);
    if (st == 2) {
      *out = g_scratch_addr[dev];
      return MLA_OK;
    }
    if (st == 0 && g_scratch_state[dev].compare_exchange_strong(st, 1, std::memory_order_acq_rel)) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        g_scratch_state[dev].store(0, std::memory_order_release);
        return MLA_ERR_HIP;
      }
      g_scratch_addr[dev] = p;
      g_scratch_state[dev].store(2, std::memory_order_release);
      *out = p;
      return MLA_OK;
    }
  }
}

}  // namespace

MLA_API mla_status mla_flash_attend_noalloc(const mla_shape* shape, const void* q_abs, int32_t q_n_frames,
                                            const void* cache, const int32_t* slot_frame, const float* rope_tables,
                                            int32_t rope_t_first, int32_t rope_n_t, void* o_lat, int32_t kv_splits,
                                            void* stream) {
  size_t need = 0;
  mla_status st = mla_abi::flash_check(shape, q_abs, q_n_frames, cache, slot_frame, rope_tables, rope_t_first,
                                       rope_n_t, o_lat, kv_splits, &need);
  if (st != MLA_OK) return st;
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MLA_OK) return st;
  // The kernels clear the one scratch field that must start at zero (the
  // count of rows for the exact pass) at the start of every call; every other
  // byte is written before it is read within the call, so what an earlier
  // call left there does not matter.
  return mla_abi::flash_run(shape, q_abs, q_n_frames, cache, slot_frame, rope_tables, rope_t_first, rope_n_t, o_lat,
                            kv_splits, ws, stream);
}
