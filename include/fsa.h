/*
 * fsa.h - frame-windowed sparse attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libfsa.so. Three calls make up the hot path of the super-resolution
 * transformer's self-attention described in the pages on the HeyGen / Google
 * Cloud Avatar IV port (aihot.vn, "HeyGen tối ưu hóa mô hình Avatar IV trên
 * Google Cloud Trillium TPU"; corroborated by bib.com.ua, "HeyGen прискорила
 * Avatar IV на TPU у 1,86 раза"):
 *
 *   fsa_plan       frame-aligned active-block list (section "Xóa bỏ mặt nạ
 *                  (Mask)", Fig. 3): every query frame attends a window of
 *                  neighbouring frames plus one global reference frame; block
 *                  sizes are multiples of 16 that divide a frame, so every
 *                  block is fully inside or fully outside the mask.
 *   fsa_bounds     the norms, computed ahead of attention, that the softmax bound is built from
 *                  (section "Giải phóng Softmax"): per-row query norms,
 *                  per-key-block largest key norms, and the per-head check of
 *                  whether the bound is tight enough to use; optionally with
 *                  the keys mean-centred first (same section), which tightens
 *                  the bound when the keys share a large common component.
 *   fsa_attention  one pass of q, k, v -> o over the whole mask (window and
 *                  reference frame together, no second pass, no merge),
 *                  with each row's softmax shifted by its Cauchy-Schwarz bound
 *                  instead of a running max; heads whose bound is too loose
 *                  take the standard online softmax inside the same kernel
 *                  (section "Giải phóng Softmax", Fig. 4). A head range lets a
 *                  caller run independent head groups that each see exactly the
 *                  ungrouped mask (section "Ẩn đi các tập lệnh tập thể (Collective)").
 *   fsa_pre_attention  the chain that produces q, k, v (normalisation,
 *                  projection, rotary embedding, head packing) as one kernel
 *                  writing the [B, H, N, D] layout the two calls above read
 *                  (section "Bố cục là ABI", Fig. 5).
 *
 * Notation: B batch, H heads, F frames, T tokens per frame, N = F*T tokens,
 * D head dim, w window half-width (frames), r reference frame, bq / bk query /
 * key block sizes, n_qb = N/bq, n_kb = N/bk. frame(i) = i / T. Query frame f
 * sees key frames V(f) = {g : |g - f| <= w, 0 <= g < F} U {r}: the window is
 * clipped at the sequence ends, and r is global as a key only.
 *
 * Layout: q, k, v, o are bf16 [B, H, N, D] row-major (D fastest), tokens in
 * frame-major order; a head group is a contiguous slab of each batch item.
 *
 * Ownership: the caller owns every buffer, host and device. The library
 * allocates no memory, keeps no state between calls, and may be called from
 * several host threads and on several streams at once.
 *
 * Errors: every argument is checked on the host before anything is enqueued.
 * On error nothing is launched, no output is touched, a non-zero status is
 * returned and fsa_last_error() describes it (per host thread). A failed
 * kernel launch returns FSA_ERR_HIP. Faults during kernel execution surface at
 * the caller's next synchronisation of the stream. Nothing is printed and no
 * call aborts.
 */
#ifndef FSA_H
#define FSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fsa_status {
    FSA_OK = 0,
    FSA_ERR_INVALID_ARG = 1,      /* a size, range or pointer is invalid            */
    FSA_ERR_UNALIGNED = 2,        /* T or a block size is not a multiple of 16, or a
                                     block size does not divide T                   */
    FSA_ERR_UNSUPPORTED = 3,      /* valid, but not built (e.g. head_dim not 64/128) */
    FSA_ERR_BUFFER_TOO_SMALL = 4, /* fsa_plan: row_ptr / col_idx capacity too small  */
    FSA_ERR_HIP = 5               /* the HIP runtime refused a launch                */
} fsa_status;

/* Shape of a plan. Filled by fsa_plan; passed back unchanged to the device calls. */
typedef struct fsa_plan_info {
    int32_t frames;           /* F >= 1                                     */
    int32_t tokens_per_frame; /* T >= 16, T % 16 == 0                       */
    int32_t window;           /* w >= 0 (any w >= F-1 gives the dense mask) */
    int32_t ref_frame;        /* 0 <= r < F                                 */
    int32_t seq_len;          /* N = F * T                                  */
    int32_t block_q;          /* bq: multiple of 16 dividing T              */
    int32_t block_k;          /* bk: multiple of 16 dividing T              */
    int32_t n_qblocks;        /* N / bq                                     */
    int32_t n_kblocks;        /* N / bk                                     */
    int32_t nnz;              /* number of active (query block, key block) pairs */
} fsa_plan_info;

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t fsa_version(void);

/*
 * fsa_plan - the frame-aligned active-block list (section "Xóa bỏ mặt nạ
 * (Mask)", Fig. 3). Host only; touches no device; thread-safe.
 *
 * block_q / block_k: 0 selects the automatic size: the largest multiple of 16
 * dividing T that is <= 256 (queries) or <= 128 (keys). Otherwise each must be
 * a multiple of 16 dividing T (FSA_ERR_UNALIGNED).
 * Block (qb, kb) is active iff frame(kb*bk) is in V(frame(qb*bq)). Output is
 * CSR: row_ptr int32 [n_qb + 1], col_idx int32 [nnz], key blocks ascending
 * within each query block; every query block of a frame lists the same keys.
 *
 * info (required) is always filled when the arguments are valid. Pass
 * row_ptr = col_idx = NULL to size the arrays; otherwise both must be non-null
 * with row_ptr_cap >= n_qb + 1 and col_idx_cap >= nnz, else
 * FSA_ERR_BUFFER_TOO_SMALL (info still filled, arrays untouched).
 * Sizes whose counts overflow int32 give FSA_ERR_INVALID_ARG.
 */
fsa_status fsa_plan(int32_t frames, int32_t tokens_per_frame, int32_t window, int32_t ref_frame,
                    int32_t block_q, int32_t block_k, fsa_plan_info *info,
                    int32_t *row_ptr, int64_t row_ptr_cap, int32_t *col_idx, int64_t col_idx_cap);

/*
 * fsa_bounds - the norm array of the softmax bound (section "Giải phóng
 * Softmax"). Device, asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream).
 *
 * plan:       from fsa_plan. d_row_ptr / d_col_idx: device copies of its CSR.
 * q, k:       device bf16 [B, H, N, D], 16-byte aligned.
 * head_offset, head_count: heads [offset, offset + count) are processed, the
 *             others are neither read nor written; count 0 means H - offset.
 * scale:      softmax scale (> 0, finite), the same value later given to
 *             fsa_attention.
 * bound_limit: a head is eligible for the bound path iff its largest row bound
 *             is <= bound_limit; <= 0 or NaN selects the default 32.
 * Outputs (device, 4-byte aligned, full-size arrays; only the head range is
 * written):
 *   qnorm    fp32 [B, H, N]     ||q_i||_2
 *   kmax     fp32 [B, H, n_kb]  largest ||k_j||_2 over key block kb
 *   eligible int32 [B, H]       1 = bound path, 0 = online fallback
 *   bmax     fp32 [B, H]        largest row bound B_i = scale * ||q_i|| *
 *                               (largest kmax over the key blocks active for
 *                               the query block holding i)
 *   kmean    NULL, or fp32 [B, H, D], 16-byte aligned: key mean-centring (section "Giải phóng
 *            Softmax": the keys share a large common component; removing the
 *            mean key tightens the bound and leaves the softmax unchanged).
 *            When given, the call writes the mean of the head's N keys,
 *            mu = (1/N) sum_j k_j, and kmax becomes the largest ||k_j - mu||
 *            over key block kb, so B_i, bmax and eligible use the centred
 *            norms. NULL: no centring (kmax as above).
 * eligible and bmax also serve as the call's own accumulators while it runs,
 * and with kmean the head range of qnorm holds partial key sums until the call
 * overwrites it with the norms: their values are defined only once the stream
 * has completed the call.
 * B == 0 or an empty head range is a no-op returning FSA_OK.
 */
fsa_status fsa_bounds(const fsa_plan_info *plan, const int32_t *d_row_ptr, const int32_t *d_col_idx,
                      const void *q, const void *k, int32_t batch, int32_t heads, int32_t head_dim,
                      int32_t head_offset, int32_t head_count, float scale, float bound_limit,
                      float *qnorm, float *kmax, int32_t *eligible, float *bmax, float *kmean,
                      void *stream);

/*
 * fsa_attention - one pass of frame-windowed sparse attention (sections
 * "Xóa bỏ mặt nạ (Mask)" and "Giải phóng Softmax"). Device, asynchronous on
 * `stream`.
 *
 * o[b,h,i] = sum_j p_ij v_j / sum_j p_ij over the keys j of the active blocks
 * of i's query block, with p_ij = exp(s_ij - B_i), s_ij = scale * q_i . k_j
 * and B_i = scale * qnorm_i * max kmax over those blocks, for heads with
 * eligible = 1; heads with eligible = 0 use the running row max instead.
 * With key centring the bound-path shift is B_i + scale * q_i . mu instead
 * (the centred scores scale * q_i . (k_j - mu) shifted by their bound B_i).
 * All are masked softmax attention in exact arithmetic. Accumulation is fp32;
 * p is rounded to bf16 for the p.v product; o is rounded to bf16 (RNE).
 *
 * plan, d_row_ptr, d_col_idx: as for fsa_bounds (the CSR must be the one
 *             fsa_plan produced for `plan`). The block list (nnz * 4 bytes)
 *             must be below 2 GiB, i.e. nnz < 2^29 (else FSA_ERR_UNSUPPORTED).
 * q, k, v:    device bf16 [B, H, N, D] inputs; o: device bf16 [B, H, N, D]
 *             output; all 16-byte aligned; o must not overlap the inputs.
 * qnorm, kmax, eligible, kmean: the outputs of fsa_bounds for the same q, k,
 *             scale and head range (only the range is read). kmean must be
 *             NULL exactly when that fsa_bounds call had NULL: centred norms
 *             with an uncentred shift (or the reverse) are not a bound.
 * head_dim:   64 or 128 (else FSA_ERR_UNSUPPORTED). One head's q / k / v slab
 *             (N * D * 2 bytes) must be below 2 GiB (else FSA_ERR_UNSUPPORTED),
 *             for fsa_bounds as well.
 * head_offset, head_count: as for fsa_bounds; rows of other heads in o are
 *             not written, so several calls on disjoint head ranges may run
 *             concurrently on different streams.
 * Results are bitwise deterministic and independent of how the heads are
 * grouped into calls. B == 0 or an empty head range is a no-op (FSA_OK).
 */
fsa_status fsa_attention(const fsa_plan_info *plan, const int32_t *d_row_ptr, const int32_t *d_col_idx,
                         const void *q, const void *k, const void *v, void *o,
                         const float *qnorm, const float *kmax, const int32_t *eligible,
                         const float *kmean, int32_t batch, int32_t heads, int32_t head_dim, float scale,
                         int32_t head_offset, int32_t head_count, void *stream);

/*
 * fsa_pre_attention - the chain that makes the attention inputs, fused into
 * one kernel whose outputs are already in the layout fsa_bounds and
 * fsa_attention read (section "Bố cục là ABI", Fig. 5: normalisation, rotary
 * embedding, projection and head packing in one kernel, no repacking copies).
 * Device, asynchronous on `stream`.
 *
 * For token (b, n) with activations x_t = x[b, n, :]:
 *   r_t = 1 / sqrt(mean_c x_t[c]^2 + eps)               (RMS normalisation)
 *   y_t = r_t * (x_t . w_qkv^T)                         (projection, no bias)
 *   q[b,h,n,:] = rot(y_t[h D .. h D + D - 1], n)
 *   k[b,h,n,:] = rot(y_t[H D + h D .. ], n)
 *   v[b,h,n,:] = y_t[2 H D + h D .. ]                   (not rotated)
 * rot(u, n) turns each feature pair (j, j + D/2), j < D/2, by the angle
 * n * rope_base^(-2 j / D): out_j = u_j cos - u_{j+D/2} sin,
 * out_{j+D/2} = u_{j+D/2} cos + u_j sin (n = the token's index in its sequence).
 * A normalisation gain g is folded into the weight beforehand,
 * w_qkv[o, c] = W[o, c] * g[c] rounded to bf16: in exact arithmetic
 * (r x * g) . W^T = r (x . (W diag g)^T).
 * Accumulation is fp32 (bf16 MFMA); r_t and the rotation are applied in fp32;
 * outputs are rounded to bf16 (RNE).
 *
 * x:       device bf16 [B, N, C] (row-major, channels fastest).
 * w_qkv:   device bf16 [3 H D, C], a linear layer's weight (output features
 *          by input channels): q rows of head h at h D, then k, then v.
 * q, k, v: device bf16 [B, H, N, D] outputs; they must not overlap each other
 *          or an input. All five pointers 16-byte aligned.
 * channels C: a positive multiple of 32, at most 1,048,576 (else
 *          FSA_ERR_UNSUPPORTED).
 * head_dim D: 64 or 128 (else FSA_ERR_UNSUPPORTED).
 * eps >= 0 and rope_base > 0, both finite (typical: 1e-6 and 10000).
 * B == 0, N == 0 or H == 0 is a no-op returning FSA_OK. Errors as above.
 */
fsa_status fsa_pre_attention(const void *x, const void *w_qkv, int32_t batch, int32_t seq_len,
                             int32_t channels, int32_t heads, int32_t head_dim, float eps,
                             float rope_base, void *q, void *k, void *v, void *stream);

/* Static English text for a status code (never NULL). */
const char *fsa_status_string(fsa_status status);

/* Detail of the last error on the calling host thread ("" if none). The
 * pointer stays valid until the next fsa_* call on that thread. */
const char *fsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H */
