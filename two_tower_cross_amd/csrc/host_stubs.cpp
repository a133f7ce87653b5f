// Device-side entry points replaced by stubs that report that there is no device, for the
// host-only build of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
// (two_tower_cross_amd/build.py, build_host_sanitized). That build exercises argument checking,
// partition planning and workspace sizing, which return before anything would be launched; a call
// that got as far as a launch would fail with TT_EHIP.
#include "kernels.hpp"

namespace tt {

hipError_t launch_block_attn_bf16(const AttnParams &, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNoDevice;
}
hipError_t launch_block_attn_f32(const AttnParams &, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNoDevice;
}
hipError_t launch_attn_reduce(const AttnParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_scratch_address(void **) { return hipErrorNoDevice; }
hipError_t launch_unmask(const UnmaskParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_masked_nll(const UnmaskParams &, const NllParams &, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_mask_corrupt(const CorruptParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_unmask_tiles_finalize(const UnmaskParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_append(const AppendParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_linear(const LinearParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pack_weight(const void *, int, int, void *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream_read(const void *, size_t, int, uint32_t *, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_mfma_rate(int, int, int, float *, hipStream_t) { return hipErrorNoDevice; }

}  // namespace tt
