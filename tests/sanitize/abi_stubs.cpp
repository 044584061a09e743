// Launch stubs for the host-sanitizer build of the C ABI layer: the same
// signatures as the kernel launchers, with no device code. Every launch
// reports failure, so a call whose arguments pass validation returns
// MLA_ERR_HIP; what the sanitizers watch is the host-side validation,
// workspace arithmetic and work-split planning on the way there.
#include "../../latent_kv_attention_amd/csrc/mla_internal.hpp"

namespace mla {
hipError_t launch_rope_tables(const RopeTableParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_cache_write(int, int, int, const CacheWriteParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_absorb_q(int, int, int, const AbsorbParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_flash(int, int, int, const FlashParams&, bool, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_up_v(int, int, int, const UpVParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_rope_window(int, int, int, const FlashParams&, hipStream_t) { return hipErrorInvalidValue; }
bool heads_supported(int dtype, int, int, int d_head) { return dtype == 0 && d_head == 128; }
int heads_tile_keys(int, int d_rope) { return d_rope > 32 ? 64 : 128; }
hipError_t launch_heads(int, int, int, const HeadsParams&, bool, bool, hipStream_t) { return hipErrorInvalidValue; }
int gemm_tile_rows(int, int, int) { return 64; }
hipError_t launch_gemm_nt(int, const GemmParams&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_qabs(int, const GemmParams&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_ring(int, const GemmParams&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_qabs_weights(int, const QabsWeightParams&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace mla
