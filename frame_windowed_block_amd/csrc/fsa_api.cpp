// Host side of libfsa: argument checks of the device entry points and the
// hand-off to the kernel launchers. Plain C++ (no device code, no HIP headers):
// every check runs before anything is enqueued, so a rejected call launches
// nothing and leaves every output untouched.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "fsa_internal.h"

namespace fsa {
namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared checks of batch / heads / head range / head_dim / scale. On FSA_OK,
// *count holds the resolved head count and *empty says whether there is no work.
fsa_status check_common(const fsa_plan_info *plan, int32_t batch, int32_t heads, int32_t head_dim,
                        int32_t head_offset, int32_t head_count, float scale, int32_t *count,
                        bool *empty) {
    fsa_status s = check_plan_info(plan);
    if (s != FSA_OK) return s;
    if (batch < 0) return fail(FSA_ERR_INVALID_ARG, "batch = %d, must be >= 0", batch);
    if (heads < 0) return fail(FSA_ERR_INVALID_ARG, "heads = %d, must be >= 0", heads);
    if (head_offset < 0 || head_offset > heads)
        return fail(FSA_ERR_INVALID_ARG, "head_offset = %d outside [0, %d]", head_offset, heads);
    if (head_count < 0)
        return fail(FSA_ERR_INVALID_ARG, "head_count = %d, must be >= 0", head_count);
    const int32_t hc = head_count == 0 ? heads - head_offset : head_count;
    if (int64_t(head_offset) + hc > heads)
        return fail(FSA_ERR_INVALID_ARG, "head range [%d, %lld) exceeds heads = %d", head_offset,
                    (long long)(int64_t(head_offset) + hc), heads);
    if (head_dim <= 0) return fail(FSA_ERR_INVALID_ARG, "head_dim = %d, must be > 0", head_dim);
    if (head_dim != 64 && head_dim != 128)
        return fail(FSA_ERR_UNSUPPORTED, "head_dim = %d; built for 64 and 128", head_dim);
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(FSA_ERR_INVALID_ARG, "scale must be finite and > 0");
    // element counts in 64-bit; keep every offset well inside int64
    const int64_t elems = int64_t(batch) * heads * plan->seq_len * head_dim;
    if (batch > 0 && heads > 0 && elems / batch / heads / plan->seq_len != head_dim)
        return fail(FSA_ERR_INVALID_ARG, "tensor size overflows");
    if (elems > (int64_t(1) << 60)) return fail(FSA_ERR_INVALID_ARG, "tensor size overflows");
    // the kernels address one head's K / V slab with 32-bit byte offsets
    if (int64_t(plan->seq_len) * head_dim * 2 >= (int64_t(1) << 31))
        return fail(FSA_ERR_UNSUPPORTED, "seq_len * head_dim * 2 = %lld bytes per head; must be below 2 GiB",
                    (long long)(int64_t(plan->seq_len) * head_dim * 2));
    *count = hc;
    *empty = batch == 0 || hc == 0;
    return FSA_OK;
}

fsa_status check_csr(const int32_t *row_ptr, const int32_t *col_idx) {
    if (!row_ptr || !col_idx) return fail(FSA_ERR_INVALID_ARG, "device plan arrays must be non-NULL");
    if (!aligned(row_ptr, 4) || !aligned(col_idx, 4))
        return fail(FSA_ERR_INVALID_ARG, "device plan arrays must be 4-byte aligned");
    return FSA_OK;
}

// bf16 tensors and the fp32 key mean are read 16 bytes at a time
fsa_status check_vec16(const void *p, const char *name) {
    if (!p) return fail(FSA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(FSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
    return FSA_OK;
}

fsa_status check_word(const void *p, const char *name) {
    if (!p) return fail(FSA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 4)) return fail(FSA_ERR_INVALID_ARG, "%s must be 4-byte aligned", name);
    return FSA_OK;
}

#define FSA_TRY(expr)                       \
    do {                                    \
        fsa_status _s = (expr);             \
        if (_s != FSA_OK) return _s;        \
    } while (0)

}  // namespace
}  // namespace fsa

extern "C" {

fsa_status fsa_bounds(const fsa_plan_info *plan, const int32_t *d_row_ptr, const int32_t *d_col_idx,
                      const void *q, const void *k, int32_t batch, int32_t heads, int32_t head_dim,
                      int32_t head_offset, int32_t head_count, float scale, float bound_limit,
                      float *qnorm, float *kmax, int32_t *eligible, float *bmax, float *kmean,
                      void *stream) {
    using namespace fsa;
    clear_error();
    int32_t hc = 0;
    bool empty = false;
    FSA_TRY(check_common(plan, batch, heads, head_dim, head_offset, head_count, scale, &hc, &empty));
    if (empty) return FSA_OK;
    FSA_TRY(check_csr(d_row_ptr, d_col_idx));
    FSA_TRY(check_vec16(q, "q"));
    FSA_TRY(check_vec16(k, "k"));
    FSA_TRY(check_word(qnorm, "qnorm"));
    FSA_TRY(check_word(kmax, "kmax"));
    FSA_TRY(check_word(eligible, "eligible"));
    FSA_TRY(check_word(bmax, "bmax"));
    if (kmean) FSA_TRY(check_vec16(kmean, "kmean"));
    const int64_t units = int64_t(batch) * hc * (plan->seq_len / 16 + plan->n_kblocks);
    if (units / 4 + 1 > kMaxWorkgroups || int64_t(batch) * hc * plan->n_qblocks > kMaxWorkgroups)
        return fail(FSA_ERR_UNSUPPORTED, "problem needs more workgroups than one launch holds");
    if (!(bound_limit > 0.0f)) bound_limit = 32.0f;               // <= 0 or NaN: default
    // Any window of at least F frames gives the same (dense) mask; the
    // kernels get it clamped to F so that their window-edge arithmetic
    // (frame + window, in 32 bits) cannot overflow.
    fsa_plan_info pl = *plan;
    if (pl.window > pl.frames) pl.window = pl.frames;
    BoundsLaunch a{&pl, d_row_ptr, d_col_idx, q, k, batch, heads, head_dim, head_offset, hc,
                   scale, bound_limit, qnorm, kmax, eligible, bmax, kmean, stream};
    const int err = launch_bounds(a);
    if (err) return fail(FSA_ERR_HIP, "fsa_bounds launch failed: %s", hip_error_text(err));
    return FSA_OK;
}

fsa_status fsa_attention(const fsa_plan_info *plan, const int32_t *d_row_ptr, const int32_t *d_col_idx,
                         const void *q, const void *k, const void *v, void *o,
                         const float *qnorm, const float *kmax, const int32_t *eligible,
                         const float *kmean, int32_t batch, int32_t heads, int32_t head_dim, float scale,
                         int32_t head_offset, int32_t head_count, void *stream) {
    using namespace fsa;
    clear_error();
    int32_t hc = 0;
    bool empty = false;
    FSA_TRY(check_common(plan, batch, heads, head_dim, head_offset, head_count, scale, &hc, &empty));
    if (empty) return FSA_OK;
    FSA_TRY(check_csr(d_row_ptr, d_col_idx));
    FSA_TRY(check_vec16(q, "q"));
    FSA_TRY(check_vec16(k, "k"));
    FSA_TRY(check_vec16(v, "v"));
    FSA_TRY(check_vec16(o, "o"));
    FSA_TRY(check_word(qnorm, "qnorm"));
    FSA_TRY(check_word(kmax, "kmax"));
    FSA_TRY(check_word(eligible, "eligible"));
    if (kmean) FSA_TRY(check_vec16(kmean, "kmean"));
    // o must not overlap an input: the kernel reads q, k, v while writing o
    const int64_t bytes = int64_t(batch) * heads * plan->seq_len * head_dim * 2;
    const uintptr_t ob = reinterpret_cast<uintptr_t>(o);
    for (const void *in : {q, k, v}) {
        const uintptr_t ib = reinterpret_cast<uintptr_t>(in);
        if (ob < ib + uintptr_t(bytes) && ib < ob + uintptr_t(bytes))
            return fail(FSA_ERR_INVALID_ARG, "o overlaps an input");
    }
    if (int64_t(batch) * hc * plan->n_qblocks + 8 > kMaxWorkgroups)
        return fail(FSA_ERR_UNSUPPORTED, "problem needs more workgroups than one launch holds");
    // the kernel reads the block list with 32-bit byte offsets from its start
    if (int64_t(plan->nnz) * 4 >= (int64_t(1) << 31))
        return fail(FSA_ERR_UNSUPPORTED, "plan has %d active blocks; the block list must stay below 2 GiB "
                    "(at most 2^29 - 1 blocks)", plan->nnz);
    AttentionLaunch a{plan, d_row_ptr, d_col_idx, q, k, v, o, qnorm, kmax, eligible, kmean,
                      batch, heads, head_dim, head_offset, hc, scale, stream};
    const int err = launch_attention(a);
    if (err) return fail(FSA_ERR_HIP, "fsa_attention launch failed: %s", hip_error_text(err));
    return FSA_OK;
}

fsa_status fsa_pre_attention(const void *x, const void *w_qkv, int32_t batch,
                             int32_t seq_len, int32_t channels, int32_t heads, int32_t head_dim, float eps,
                             float rope_base, void *q, void *k, void *v, void *stream) {
    using namespace fsa;
    clear_error();
    if (batch < 0) return fail(FSA_ERR_INVALID_ARG, "batch = %d, must be >= 0", batch);
    if (seq_len < 0) return fail(FSA_ERR_INVALID_ARG, "seq_len = %d, must be >= 0", seq_len);
    if (heads < 0) return fail(FSA_ERR_INVALID_ARG, "heads = %d, must be >= 0", heads);
    if (channels <= 0 || channels % 32)
        return fail(FSA_ERR_UNSUPPORTED, "channels = %d; must be a positive multiple of 32", channels);
    // a workgroup's 256 x rows are addressed with 32-bit byte offsets
    if (channels > kMaxPreChannels)
        return fail(FSA_ERR_UNSUPPORTED, "channels = %d; at most %d", channels, kMaxPreChannels);
    if (head_dim <= 0) return fail(FSA_ERR_INVALID_ARG, "head_dim = %d, must be > 0", head_dim);
    if (head_dim != 64 && head_dim != 128)
        return fail(FSA_ERR_UNSUPPORTED, "head_dim = %d; built for 64 and 128", head_dim);
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(FSA_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!(rope_base > 0.0f) || !std::isfinite(rope_base))
        return fail(FSA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
    if (int64_t(3) * heads * head_dim > (int64_t(1) << 30))
        return fail(FSA_ERR_INVALID_ARG, "3 * heads * head_dim overflows");
    const int64_t tokens = int64_t(batch) * seq_len;
    if (batch > 0 && tokens / batch != seq_len) return fail(FSA_ERR_INVALID_ARG, "tensor size overflows");
    if (tokens > (int64_t(1) << 40) || tokens * channels > (int64_t(1) << 60) ||
        tokens * heads * head_dim > (int64_t(1) << 60))
        return fail(FSA_ERR_INVALID_ARG, "tensor size overflows");
    if (tokens == 0 || heads == 0) return FSA_OK;
    FSA_TRY(check_vec16(x, "x"));
    FSA_TRY(check_vec16(w_qkv, "w_qkv"));
    FSA_TRY(check_vec16(q, "q"));
    FSA_TRY(check_vec16(k, "k"));
    FSA_TRY(check_vec16(v, "v"));
    if (((tokens + 255) / 256) * ((int64_t(3) * heads * head_dim + 255) / 256) + 8 > kMaxWorkgroups)
        return fail(FSA_ERR_UNSUPPORTED, "problem needs more workgroups than one launch holds");
    // the outputs must not overlap each other or an input
    struct Span { uintptr_t lo, hi; };
    const int64_t out_bytes = tokens * heads * head_dim * 2;
    const Span outs[3] = {{reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + uintptr_t(out_bytes)},
                          {reinterpret_cast<uintptr_t>(k), reinterpret_cast<uintptr_t>(k) + uintptr_t(out_bytes)},
                          {reinterpret_cast<uintptr_t>(v), reinterpret_cast<uintptr_t>(v) + uintptr_t(out_bytes)}};
    const Span ins[2] = {
        {reinterpret_cast<uintptr_t>(x), reinterpret_cast<uintptr_t>(x) + uintptr_t(tokens * channels * 2)},
        {reinterpret_cast<uintptr_t>(w_qkv),
         reinterpret_cast<uintptr_t>(w_qkv) + uintptr_t(int64_t(3) * heads * head_dim * channels * 2)}};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 2; ++j)
            if (outs[i].lo < ins[j].hi && ins[j].lo < outs[i].hi)
                return fail(FSA_ERR_INVALID_ARG, "an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (outs[i].lo < outs[j].hi && outs[j].lo < outs[i].hi)
                return fail(FSA_ERR_INVALID_ARG, "q, k and v must not overlap");
    }
    PreAttentionLaunch a{x, w_qkv, batch, seq_len, channels, heads, head_dim, eps, rope_base,
                         q, k, v, stream};
    const int err = launch_pre_attention(a);
    if (err) return fail(FSA_ERR_HIP, "fsa_pre_attention launch failed: %s", hip_error_text(err));
    return FSA_OK;
}

}  // extern "C"
