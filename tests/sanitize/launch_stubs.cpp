// Host-only stand-ins for the kernel launchers of libsparse_attn, linked in
// place of the GPU kernels for a sanitizer build of the C ABI's host code
// (argument validation, workspace sizing, chunking and launch order).  Every
// launcher reports that no device is present, as a GPU-less host does.
#include "kernels.hpp"

namespace sa {

hipError_t launch_gate_alpha(const void *, float *, int, int, int, int, int, const FusedOpts &, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_normalize_rows(const void *, void *, long long, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd(const BwdArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_skip(const SkipArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNoDevice; }

}  // namespace sa
