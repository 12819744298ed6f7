// Stand-ins for the kernel launchers of libfsa, for a host-only build of the
// C ABI (fsa_plan.cpp, fsa_api.cpp) with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU. Each launcher reads every field of
// the validated launch record, touches none of the device pointers, and
// reports success; hip_error_text names no HIP error.
#include <cstdint>

#include "../../frame_windowed_block_amd/csrc/fsa_internal.h"

namespace fsa {

static volatile int64_t g_sink = 0;

int launch_bounds(const BoundsLaunch &a) {
    g_sink = g_sink + a.plan->nnz + a.batch + a.heads + a.head_dim + a.head_offset + a.head_count +
             int64_t(a.scale > 0.0f) + int64_t(a.bound_limit > 0.0f) + int64_t(a.kmean != nullptr);
    return 0;
}

int launch_attention(const AttentionLaunch &a) {
    g_sink = g_sink + a.plan->nnz + a.batch + a.heads + a.head_dim + a.head_offset + a.head_count +
             int64_t(a.scale > 0.0f) + int64_t(a.kmean != nullptr);
    return 0;
}

int launch_pre_attention(const PreAttentionLaunch &a) {
    g_sink = g_sink + a.batch + a.seq_len + a.channels + a.heads + a.head_dim + int64_t(a.eps >= 0.0f);
    return 0;
}

const char *hip_error_text(int) { return "no HIP in the host-only build"; }

}  // namespace fsa
