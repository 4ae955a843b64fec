// launch_stubs.cpp -- host-only stand-ins for the kernel launchers of libosm,
// for the sanitizer build of the C ABI layer (abi.cpp) and the host sizes
// (layout.cpp).  Each stand-in records its arguments for the driver to check
// and launches nothing; no pointer it receives is ever dereferenced.
#include "osm_internal.h"

namespace osm {

int g_launches = 0;
SoftmaxArgs g_softmax{};
SoftmaxPlan g_softmax_plan{};
AttnFwdArgs g_fwd{};
AttnFwdFp8Args g_fwd8{};
AttnBwdArgs g_bwd{};
DecodeArgs g_decode{};
DecodeLayout g_decode_layout{};
MergeArgs g_merge{};
MergeLseArgs g_merge_lse{};

hipError_t launch_softmax_rows(const SoftmaxArgs &a, const SoftmaxPlan &p, hipStream_t) {
    ++g_launches;
    g_softmax = a;
    g_softmax_plan = p;
    return hipSuccess;
}
hipError_t launch_attn_fwd(const AttnFwdArgs &a, hipStream_t) {
    ++g_launches;
    g_fwd = a;
    return hipSuccess;
}
hipError_t launch_attn_fwd_fp8(const AttnFwdFp8Args &a, hipStream_t) {
    ++g_launches;
    g_fwd8 = a;
    return hipSuccess;
}
hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t) {
    ++g_launches;
    g_bwd = a;
    return hipSuccess;
}
hipError_t launch_decode_split(const DecodeArgs &a, const DecodeLayout &lay, hipStream_t) {
    ++g_launches;
    g_decode = a;
    g_decode_layout = lay;
    return hipSuccess;
}
hipError_t launch_merge_partials(const MergeArgs &a, hipStream_t) {
    ++g_launches;
    g_merge = a;
    return hipSuccess;
}
hipError_t decode_scratch(void **ptr) {
    *ptr = reinterpret_cast<void *>(static_cast<uintptr_t>(0x7000000));
    return hipSuccess;
}
hipError_t launch_merge_lse(const MergeLseArgs &a, hipStream_t) {
    ++g_launches;
    g_merge_lse = a;
    return hipSuccess;
}

}  // namespace osm
