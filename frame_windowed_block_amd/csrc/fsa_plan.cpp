// Host side of libfsa: the frame-aligned block plan, error reporting and
// version. Plain C++ (no device code).
//
// The plan follows the pages' mask (aihot.vn, "HeyGen tối ưu hóa mô hình
// Avatar IV trên Google Cloud Trillium TPU", section "Xóa bỏ mặt nạ (Mask)"
// and Fig. 3): each query frame attends a window of neighbouring frames plus
// one global reference frame; block sizes are multiples of 16 that divide a
// frame's token range, so every block lies fully inside or fully outside the
// mask, and the reference frame's blocks are simply more full blocks of the
// same row. It is built here at frame granularity: a query block inherits its
// frame's visible set and lists the key blocks of every visible frame.
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fsa_internal.h"

namespace fsa {

namespace {
thread_local char g_error[512];

constexpr int32_t kTile = 16;          // finest bf16 tile along the sequence
constexpr int32_t kAutoBqCap = 256;    // automatic query block: largest aligned size <= 256
constexpr int32_t kAutoBkCap = 128;    // automatic key block:   largest aligned size <= 128

int32_t auto_block(int32_t t, int32_t cap) {
    int32_t best = kTile;
    for (int32_t b = kTile; b <= cap && b <= t; b += kTile)
        if (t % b == 0) best = b;
    return best;
}

// Visible key frames of query frame f, ascending, written to out (capacity >=
// 2w+2 or F); returns the count. Window clipped to [0, F), reference frame added once.
int32_t visible_list(int32_t f, int32_t frames, int32_t window, int32_t ref_frame, int32_t *out) {
    const int64_t lo = f - int64_t(window) < 0 ? 0 : f - int64_t(window);
    const int64_t hi = f + int64_t(window) > frames - 1 ? frames - 1 : f + int64_t(window);
    int32_t n = 0;
    if (ref_frame < lo) out[n++] = ref_frame;
    for (int64_t g = lo; g <= hi; ++g) out[n++] = int32_t(g);
    if (ref_frame > hi) out[n++] = ref_frame;
    return n;
}

fsa_status check_shape(int32_t frames, int32_t t, int32_t window, int32_t ref_frame,
                       int32_t bq, int32_t bk) {
    if (frames < 1) return fail(FSA_ERR_INVALID_ARG, "frames = %d, must be >= 1", frames);
    if (t < kTile || t % kTile != 0)
        return fail(t < 1 ? FSA_ERR_INVALID_ARG : FSA_ERR_UNALIGNED,
                    "tokens_per_frame = %d, must be a positive multiple of 16", t);
    if (window < 0) return fail(FSA_ERR_INVALID_ARG, "window = %d, must be >= 0", window);
    if (ref_frame < 0 || ref_frame >= frames)
        return fail(FSA_ERR_INVALID_ARG, "ref_frame = %d, must lie in [0, %d)", ref_frame, frames);
    if (int64_t(frames) * t > INT32_MAX)
        return fail(FSA_ERR_INVALID_ARG, "sequence length %lld exceeds int32",
                    (long long)(int64_t(frames) * t));
    if (bq <= 0 || bk <= 0) return fail(FSA_ERR_INVALID_ARG, "block sizes must be > 0");
    if (bq % kTile || t % bq)
        return fail(FSA_ERR_UNALIGNED, "block_q = %d must be a multiple of 16 dividing T = %d", bq, t);
    if (bk % kTile || t % bk)
        return fail(FSA_ERR_UNALIGNED, "block_k = %d must be a multiple of 16 dividing T = %d", bk, t);
    return FSA_OK;
}

// nnz = sum_f |V(f)| * (T/bq) * (T/bk), in 64 bits.
int64_t count_nnz(int32_t frames, int32_t t, int32_t window, int32_t ref_frame, int32_t bq, int32_t bk) {
    int64_t pairs = 0;
    for (int32_t f = 0; f < frames; ++f) pairs += frames_visible(f, frames, window, ref_frame);
    return pairs * (t / bq) * (t / bk);
}

fsa_status fill_info(int32_t frames, int32_t t, int32_t window, int32_t ref_frame, int32_t bq,
                     int32_t bk, fsa_plan_info *info) {
    const int64_t n = int64_t(frames) * t;
    const int64_t nnz = count_nnz(frames, t, window, ref_frame, bq, bk);
    if (nnz > INT32_MAX)
        return fail(FSA_ERR_INVALID_ARG, "plan has %lld active blocks, more than int32 holds",
                    (long long)nnz);
    info->frames = frames;
    info->tokens_per_frame = t;
    info->window = window;
    info->ref_frame = ref_frame;
    info->seq_len = int32_t(n);
    info->block_q = bq;
    info->block_k = bk;
    info->n_qblocks = int32_t(n / bq);
    info->n_kblocks = int32_t(n / bk);
    info->nnz = int32_t(nnz);
    return FSA_OK;
}
}  // namespace

void clear_error() { g_error[0] = '\0'; }

fsa_status fail(fsa_status status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return status;
}

int64_t frames_visible(int32_t f, int32_t frames, int32_t window, int32_t ref_frame) {
    const int64_t lo = f - int64_t(window) < 0 ? 0 : f - int64_t(window);
    const int64_t hi = f + int64_t(window) > frames - 1 ? frames - 1 : f + int64_t(window);
    return (hi - lo + 1) + ((ref_frame < lo || ref_frame > hi) ? 1 : 0);
}

fsa_status check_plan_info(const fsa_plan_info *p) {
    if (!p) return fail(FSA_ERR_INVALID_ARG, "plan is NULL");
    fsa_status s = check_shape(p->frames, p->tokens_per_frame, p->window, p->ref_frame,
                               p->block_q, p->block_k);
    if (s != FSA_OK) return s;
    fsa_plan_info want;
    s = fill_info(p->frames, p->tokens_per_frame, p->window, p->ref_frame, p->block_q, p->block_k, &want);
    if (s != FSA_OK) return s;
    if (std::memcmp(&want, p, sizeof want) != 0)
        return fail(FSA_ERR_INVALID_ARG, "plan info is inconsistent with its own shape fields");
    return FSA_OK;
}

}  // namespace fsa

extern "C" {

int32_t fsa_version(void) { return 1 * 10000 + 1 * 100 + 0; }

const char *fsa_status_string(fsa_status status) {
    switch (status) {
        case FSA_OK: return "success";
        case FSA_ERR_INVALID_ARG: return "invalid argument";
        case FSA_ERR_UNALIGNED: return "size not aligned to 16-token frame tiles";
        case FSA_ERR_UNSUPPORTED: return "unsupported configuration";
        case FSA_ERR_BUFFER_TOO_SMALL: return "output buffer too small";
        case FSA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *fsa_last_error(void) { return fsa::g_error; }

fsa_status fsa_plan(int32_t frames, int32_t tokens_per_frame, int32_t window, int32_t ref_frame,
                    int32_t block_q, int32_t block_k, fsa_plan_info *info,
                    int32_t *row_ptr, int64_t row_ptr_cap, int32_t *col_idx, int64_t col_idx_cap) {
    using namespace fsa;
    clear_error();
    if (!info) return fail(FSA_ERR_INVALID_ARG, "info is NULL");
    const int32_t t = tokens_per_frame;
    if (t >= kTile && t % kTile == 0) {
        if (block_q == 0) block_q = auto_block(t, kAutoBqCap);
        if (block_k == 0) block_k = auto_block(t, kAutoBkCap);
    }
    fsa_status s = check_shape(frames, t, window, ref_frame, block_q, block_k);
    if (s != FSA_OK) return s;
    fsa_plan_info p;
    s = fill_info(frames, t, window, ref_frame, block_q, block_k, &p);
    if (s != FSA_OK) return s;
    *info = p;
    if (!row_ptr && !col_idx) return FSA_OK;                       // sizing query
    if (!row_ptr || !col_idx)
        return fail(FSA_ERR_INVALID_ARG, "row_ptr and col_idx must both be NULL or both be set");
    if (row_ptr_cap < int64_t(p.n_qblocks) + 1 || col_idx_cap < p.nnz)
        return fail(FSA_ERR_BUFFER_TOO_SMALL, "need row_ptr[%d] and col_idx[%d], got %lld and %lld",
                    p.n_qblocks + 1, p.nnz, (long long)row_ptr_cap, (long long)col_idx_cap);

    const int32_t qb_per_frame = t / block_q;
    const int32_t kb_per_frame = t / block_k;
    int32_t vis_buf[64];
    int32_t *vis = vis_buf;
    const int64_t cap = int64_t(window) * 2 + 2 < frames ? int64_t(window) * 2 + 2 : frames;
    int32_t *heap = nullptr;
    if (cap > 64) vis = heap = new int32_t[size_t(cap)];
    int32_t nnz = 0;
    row_ptr[0] = 0;
    for (int32_t f = 0; f < frames; ++f) {
        const int32_t nv = visible_list(f, frames, window, ref_frame, vis);
        for (int32_t qi = 0; qi < qb_per_frame; ++qi) {
            const int32_t qb = f * qb_per_frame + qi;
            for (int32_t x = 0; x < nv; ++x)
                for (int32_t kj = 0; kj < kb_per_frame; ++kj) col_idx[nnz++] = vis[x] * kb_per_frame + kj;
            row_ptr[qb + 1] = nnz;
        }
    }
    delete[] heap;
    return FSA_OK;
}

}  // extern "C"
