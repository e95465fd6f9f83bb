// Host-only stand-ins for the kernel launchers of libsparge, for the sanitizer
// build of the C ABI (api.cpp and hilbert.cpp compiled by g++ with AddressSanitizer
// and UndefinedBehaviorSanitizer, no device code).  The ABI tests that run against
// that build exercise argument validation, workspace sizing, default options and the
// host Hilbert order, none of which reaches a launch; every launcher here therefore
// reports hipErrorNotSupported, which the ABI maps to SPARGE_E_HIP.
#include "../../block_sparse_quantized_amd/csrc/sparge_internal.hpp"

namespace sparge {

hipError_t launch_convert16(const View&, int, const Dims&, uint16_t*, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_block_stats(const View&, const View&, int, const Dims&, double*, double*, double*,
                              double*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_pooled_scores(const double*, const double*, const Dims&, int, double, double*,
                                hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_select(const double*, const double*, const double*, const Dims&, int,
                         const SelectParams&, uint8_t*, uint16_t*, int*, unsigned long long*,
                         hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_compact(const uint8_t*, const Dims&, uint16_t*, int*, unsigned long long*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quant_k(const View&, int, const Dims&, int8_t*, int64_t, int64_t, float*, float*,
                          hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_kbar_codes(const float*, const Dims&, int8_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_prep(const View&, const View&, const View&, int, const Dims&, double*, double*, double*,
                       double*, int8_t*, int64_t, int64_t, float*, float*, uint16_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_vt8(const View&, int, const Dims&, const float*, float*, float*, unsigned char*,
                      hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_sparse_attn(const AttnParams&, const Dims&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_reorder(const View&, void*, int64_t, int64_t, int64_t, int, const Dims&, const int32_t*,
                          int64_t, int64_t, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sparge
