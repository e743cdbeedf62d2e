// Stand-ins for the device entry points in a host-only build of the library
// (layout.cpp and offload.cpp) made to run the host tests under
// AddressSanitizer and UndefinedBehaviorSanitizer; the host tests that run
// there never call them.
#include "zero_internal.h"
extern "C" {
int zero_pack_grads(zero_layout_t, const uint16_t* const*, uint16_t*, int64_t, int64_t, hipStream_t) { return -1; }
size_t zero_pack_sqnorm_workspace_bytes(zero_layout_t, int64_t, int64_t) { return 0; }
int zero_pack_grads_sqnorm(zero_layout_t, const uint16_t* const*, uint16_t*, int64_t, int64_t, double*, int32_t, void*, size_t, hipStream_t) { return -1; }
int zero_pack_grads_sqnorm_noalloc(zero_layout_t, const uint16_t* const*, uint16_t*, int64_t, int64_t, double*, int32_t, hipStream_t) { return -1; }
size_t zero_sqnorm_workspace_bytes(int64_t) { return 0; }
int zero_shard_sqnorm(const uint16_t*, int64_t, double*, int32_t, void*, size_t, hipStream_t) { return -1; }
int zero_sum_partials(const double*, int64_t, double*, int32_t, hipStream_t) { return -1; }
int zero_pack_grads_sqnorm_partials(zero_layout_t, const uint16_t* const*, uint16_t*, int64_t, int64_t, double*, size_t, int64_t*, hipStream_t) { return -1; }
int zero_sum_partials_rows(const double*, const int64_t*, const int64_t*, int64_t, double*, int32_t, hipStream_t) { return -1; }
int zero_adamw_step(const uint16_t*, float*, uint16_t*, int64_t, int64_t, int64_t, const zero_adamw_hparams*, const double*, int32_t, hipStream_t) { return -1; }
int zero_state_import(const float*, const float*, const float*, float*, int64_t, hipStream_t) { return -1; }
int zero_state_export(const float*, float*, float*, float*, int64_t, hipStream_t) { return -1; }
int zero_accumulate_grads(const uint16_t*, float*, int64_t, int32_t, hipStream_t) { return -1; }
int zero_shard_sqnorm_f32(const float*, int64_t, double*, int32_t, void*, size_t, hipStream_t) { return -1; }
int zero_adamw_step_f32grad(const float*, float*, uint16_t*, int64_t, int64_t, int64_t, const zero_adamw_hparams*, const double*, int32_t, hipStream_t) { return -1; }
int zero_adamw_step_unpack(const uint16_t*, float*, uint16_t*, int64_t, int64_t, int64_t, const zero_adamw_hparams*, const double*, int32_t, zero_layout_t, uint16_t* const*, hipStream_t) { return -1; }
int zero_adamw_step_f32grad_unpack(const float*, float*, uint16_t*, int64_t, int64_t, int64_t, const zero_adamw_hparams*, const double*, int32_t, zero_layout_t, uint16_t* const*, hipStream_t) { return -1; }
int zero_adamw_step_arrays(const uint16_t*, float*, float*, float*, uint16_t*, int64_t, const zero_adamw_hparams*, const double*, int32_t, hipStream_t) { return -1; }
int zero_unpack_params(zero_layout_t, const uint16_t*, uint16_t* const*, int64_t, int64_t, hipStream_t) { return -1; }
}
