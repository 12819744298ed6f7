// Internal interface between the host-side C ABI (fsa_plan.cpp, fsa_api.cpp)
// and the HIP kernels (fsa_kernels.hip). Plain C++: no HIP or torch types, so
// the host logic also builds with g++ alone; tests/test_host_sanitizers.py
// builds it that way under AddressSanitizer and UndefinedBehaviorSanitizer.
#pragma once

#include <cstdint>

#include "../../include/fsa.h"

namespace fsa {

// Per-thread error text behind fsa_last_error().
void clear_error();
fsa_status fail(fsa_status status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Recomputes every derived field of a plan from its inputs; FSA_OK iff `p`
// is exactly what fsa_plan would return for (frames, T, window, ref, bq, bk).
fsa_status check_plan_info(const fsa_plan_info *p);

// Count of active blocks of one query block: |V(f)| * (T / bk).
int64_t frames_visible(int32_t f, int32_t frames, int32_t window, int32_t ref_frame);

struct BoundsLaunch {
    const fsa_plan_info *plan;
    const int32_t *row_ptr, *col_idx;
    const void *q, *k;
    int32_t batch, heads, head_dim, head_offset, head_count;
    float scale, bound_limit;
    float *qnorm, *kmax;
    int32_t *eligible;
    float *bmax;
    float *kmean;            // NULL: no key centring
    void *stream;
};

struct AttentionLaunch {
    const fsa_plan_info *plan;
    const int32_t *row_ptr, *col_idx;
    const void *q, *k, *v;
    void *o;
    const float *qnorm, *kmax;
    const int32_t *eligible;
    const float *kmean;      // NULL: no key centring
    int32_t batch, heads, head_dim, head_offset, head_count;
    float scale;
    void *stream;
};

struct PreAttentionLaunch {
    const void *x;
    const void *w_qkv;
    int32_t batch, seq_len, channels, heads, head_dim;
    float eps, rope_base;
    void *q, *k, *v;
    void *stream;
};

// Kernel launchers (fsa_kernels.hip, fsa_preattn.hip). They assume validated arguments and
// return 0 or the HIP runtime's error code; hip_error_text names a code.
int launch_bounds(const BoundsLaunch &a);
int launch_attention(const AttentionLaunch &a);
int launch_pre_attention(const PreAttentionLaunch &a);
const char *hip_error_text(int code);

// Largest number of workgroups one launch may use (grid x times 256 threads
// must stay below 2^32).
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 32) / 1024 - 1;
// fsa_pre_attention's largest channel count: 256 rows of x at 32-bit byte offsets.
constexpr int32_t kMaxPreChannels = 1 << 20;

}  // namespace fsa
