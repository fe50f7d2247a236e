// Host-only stand-ins for the kernel launchers of libgdnreplay.so, linked with
// csrc/api.cpp into a CPU build of the C-ABI layer (sanitizer run of the host
// validation, no GPU and no HIP runtime). The C caller that drives it only
// makes calls that the host layer must refuse or that launch nothing, so any
// call reaching a launcher is a validation gap: it aborts.
#include <cstdio>
#include <cstdlib>

#include "../../gated_deltanet_state_replayssm_amd/csrc/internal.h"

namespace {
[[noreturn]] void reached(const char *what) {
  std::fprintf(stderr, "launcher %s reached: the host layer let a call through\n", what);
  std::abort();
}
}  // namespace

namespace gdnr {
hipError_t launch_verify_chunked(const VerifyArgs &, hipStream_t) { reached("verify_chunked"); }
hipError_t launch_flush_chunked(const FlushArgs &, hipStream_t) { reached("flush_chunked"); }
hipError_t launch_verify_flush_long(const VerifyArgs &, int, hipStream_t) {
  reached("verify_flush_long");
}
hipError_t launch_verify_flush_fused(const VerifyArgs &, int, hipStream_t) {
  reached("verify_flush_fused");
}
hipError_t launch_verify_recurrent(const VerifyArgs &, bool, hipStream_t) {
  reached("verify_recurrent");
}
hipError_t launch_flush_recurrent(const FlushArgs &, bool, hipStream_t) {
  reached("flush_recurrent");
}
hipError_t launch_rollback(const RollbackArgs &, hipStream_t) { reached("rollback"); }
hipError_t launch_gated_rmsnorm_fp8(const NormArgs &, int, hipStream_t) {
  reached("gated_rmsnorm_fp8");
}
hipError_t launch_causal_conv_update(const ConvArgs &, int, hipStream_t) {
  reached("causal_conv_update");
}
}  // namespace gdnr
