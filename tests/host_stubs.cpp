// Stand-ins for the library's device launchers, for a host-only build of the C
// ABI (lightning_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py). The argument checks of the entry points run as in
// the real library; every launcher here reports that no device is present, so a
// call that passes validation returns LT_ERR_HIP, which the ABI tests never
// expect from the calls they make.
#include "internal.h"

namespace lt {

hipError_t noalloc_scratch(hipStream_t, void **ptr, size_t *bytes) {
    *ptr = nullptr;
    *bytes = 0;
    return hipErrorNoDevice;
}
hipError_t launch_backward_kv(const BackwardArgs &, const PrefillPlan &, void *, lt_dtype, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_softmax_prefill(const SoftmaxArgs &, void *, lt_dtype, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_softmax_decode(const SoftmaxDecodeArgs &, const SoftmaxDecodePlan &, float *, lt_dtype,
                                 hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_prefill_slices(const PrefillArgs &, lt_dtype, lt_dtype, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_heads(const PrefillArgs &, const PrefillPlan &, void *, lt_dtype, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t launch_decode(const DecodeArgs &, lt_dtype, lt_dtype, hipStream_t) { return hipErrorNoDevice; }
hipError_t load_prefill_heads_code() { return hipErrorNoDevice; }
hipError_t load_prefill_slices_code() { return hipErrorNoDevice; }
hipError_t load_decode_code() { return hipErrorNoDevice; }
hipError_t load_backward_code() { return hipErrorNoDevice; }
hipError_t load_softmax_code() { return hipErrorNoDevice; }

}  // namespace lt

// the one HIP runtime call of lightning_api.cpp (status strings)
const char *hipGetErrorName(hipError_t) { return "hipErrorNoDevice"; }
