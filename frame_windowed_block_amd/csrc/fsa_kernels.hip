// HIP kernels of libfsa for AMD Instinct MI355X (gfx950, CDNA4).
//
// Sources: the pages on the HeyGen / Google Cloud Avatar IV port
//   [vi:Mask]    aihot.vn, "HeyGen tối ưu hóa mô hình Avatar IV trên Google Cloud
//                Trillium TPU", section "Xóa bỏ mặt nạ (Mask)" and Fig. 3;
//   [vi:Softmax] same page, section "Giải phóng Softmax" and Fig. 4;
//   [uk:Softmax] bib.com.ua, "HeyGen прискорила Avatar IV на TPU у 1,86 раза",
//                section on breaking the softmax serial chain.
//
// fsa_bounds runs two kernels (four with key centring, which first reduces the
// keys of each head to their mean in two fixed-order kernels). norms_kernel
// streams q and k once (the HBM-bound part): it writes ||q_i|| per row and,
// per key block, the largest ||k_j|| (of k_j - mean when centred): the norms,
// computed ahead of the attention pass, that its bound is built from
// ([vi:Softmax]). bound_reduce_kernel
// then derives, per query block, scale * max ||q_i|| * max kmax over the
// block's active key blocks, folds it into the head's largest row bound, and
// the last block of each head writes the head's eligibility ([vi:Softmax]:
// eligibility is checked per attention head).
//
// fsa_attention is one kernel: one workgroup per (batch, head, query block),
// eight wavefronts of 32 query rows each. It walks the query block's active
// key-block list once, window and reference frame alike ([vi:Mask]: one pass
// covers the whole mask), in 32-key sub-steps that may join the 16-key tail
// of one block to the head of the next; no sub-step needs a mask predicate,
// and an odd count of 16-key tiles leaves one half sub-step at the very end.
// Per sub-step and wavefront:
//   S^T = K Q^T       bf16 MFMA 32x32x16 (K rows permuted so that each lane
//                     ends up holding 16 keys of one query row, in the order
//                     the p.v operand wants them)
//   P   = exp2(S * scale * log2e - B_i * log2e)
//                     B_i = scale * ||q_i|| * max kmax over the row's active
//                     key blocks, fixed before the loop ([vi:Softmax]); no
//                     running max, no rescale (centred keys add scale q_i.mean)
//   O^T += V^T P^T    bf16 MFMA 32x32x16, V^T read from row-major V in LDS
//                     with the transposing LDS reads
// The scores of sub-step j + 1 are computed in the same step as the weights
// and p.v of sub-step j. K and V stages go from global memory straight into
// LDS (buffer loads with the LDS flag), three stages ahead. Heads whose
// bound is too loose run the same walk with the standard running max and
// rescale instead ([vi:Softmax], Fig. 4), chosen by a branch that is uniform
// over the workgroup; it rescales only when a row's max has grown by more
// than 2^8.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "fsa_internal.h"

namespace fsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Device data in the global address space: loads through it are vector
// (global_load) loads, never generic (flat) ones, which also count on the
// LDS counter and so coarsen the LDS waits.
typedef __attribute__((address_space(1))) const int32_t gint32;
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef short v8s __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
// Online fallback: how far (log2 units) a row's running max may lag behind the
// true one before the accumulators are rescaled; weights stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float sumsq8(u32x4 x) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(x[i]), b = bf16_hi(x[i]);
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}

// Sum of squares of (x - m) over 8 bf16 values and their 8 fp32 offsets.
__device__ __forceinline__ float sumsq8_centred(u32x4 x, const float (&m)[8]) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(x[i]) - m[2 * i], b = bf16_hi(x[i]) - m[2 * i + 1];
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}

// Max that lets a NaN through (a NaN norm must make the head ineligible).
__device__ __forceinline__ float nan_max(float a, float b) { return (b > a || b != b) ? b : a; }

// --------------------------------------------------------------------------
// fsa_bounds with key centring ([vi:Softmax]: the keys share a large common
// component; removing the mean key tightens the bound), kernels 0a and 0b:
// the mean of each head's N keys, summed in a fixed order so that the result
// is deterministic. 0a sums chunks of 2D consecutive keys into D fp32
// partials; with more than one chunk per head the partials are parked in the
// head's own qnorm rows (chunks * D <= N, and the norms kernel overwrites them
// later in stream order) and 0b adds them up.
// --------------------------------------------------------------------------
struct KeySumParams {
    const uint16_t *k;
    float *partial;      // qnorm of the head range, used as scratch
    float *kmean;
    int32_t heads, seq_len, h0, hc, chunks;
};

template <int D>
constexpr int key_chunk() { return 2 * D; }

template <int D>
__global__ __launch_bounds__(256) void key_sum_kernel(KeySumParams p) {
    constexpr int LPR = D / 8;              // lanes per key row, 16 bytes each
    constexpr int RPP = 256 / LPR;          // key rows per pass of the workgroup
    constexpr int PASSES = key_chunk<D>() / RPP;
    __shared__ float part[RPP * D];
    const int tid = threadIdx.x, sub = tid / LPR, seg = tid % LPR;
    const int64_t bh = blockIdx.x / p.chunks;
    const int32_t chunk = int32_t(blockIdx.x % p.chunks);
    const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
    const int32_t r0 = chunk * key_chunk<D>();
    const int32_t rows = min(key_chunk<D>(), p.seq_len - r0);
    const uint16_t *base = p.k + (hb * p.seq_len + r0) * D + seg * 8;
    u32x4 x[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int r = ps * RPP + sub;
        x[ps] = *reinterpret_cast<const u32x4 *>(base + int64_t(r < rows ? r : rows - 1) * D);
    }
    float acc[8] = {};
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        if (ps * RPP + sub < rows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += bf16_lo(x[ps][i]);
                acc[2 * i + 1] += bf16_hi(x[ps][i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[sub * D + seg * 8 + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < RPP; ++r) sum += part[r * D + tid];
        if (p.chunks == 1)
            p.kmean[hb * D + tid] = sum / float(p.seq_len);
        else
            p.partial[hb * p.seq_len + int64_t(chunk) * D + tid] = sum;
    }
}

template <int D>
__global__ __launch_bounds__(1024) void key_mean_kernel(KeySumParams p) {
    constexpr int S = 1024 / D;             // interleaved subsets of the chunks
    __shared__ float part[1024];
    const int tid = threadIdx.x, d = tid % D, sub = tid / D;
    const int64_t bh = blockIdx.x;
    const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
    const float *src = p.partial + hb * p.seq_len + d;
    float sum = 0.0f;
    for (int32_t c = sub; c < p.chunks; c += S) sum += src[int64_t(c) * D];
    part[tid] = sum;
    __syncthreads();
    if (tid < D) {
        float total = 0.0f;
#pragma unroll
        for (int j = 0; j < S; ++j) total += part[j * D + tid];
        p.kmean[hb * D + tid] = total / float(p.seq_len);
    }
}

// --------------------------------------------------------------------------
// fsa_bounds, kernel 1: row norms of q, largest key norm per key block (of
// the centred keys k_j - mean when CENTRED).
// Work unit = one wavefront: either QG 16-row groups of q, or one key block.
// --------------------------------------------------------------------------
struct NormsParams {
    const uint16_t *q, *k;
    float *qnorm, *kmax;
    int32_t *eligible;
    float *bmax;
    const float *kmean;
    int64_t q_units, total_units;
    int32_t batch, heads, seq_len, h0, hc, block_k, n_kb;
};

template <int D, int QG, bool CENTRED>
__global__ __launch_bounds__(256) void norms_kernel(NormsParams p) {
    constexpr int LPR = D / 8;          // lanes per row: 16 bytes each
    constexpr int RPL = 64 / LPR;       // rows covered by one wave-wide load
    constexpr int LOADS = 16 / RPL;     // loads per 16-row group
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR;
    const int seg = lane % LPR;

    if (blockIdx.x == 0) {              // outputs that bound_reduce_kernel folds into
        const int64_t nbh = int64_t(p.batch) * p.hc;
        for (int64_t x = threadIdx.x; x < nbh; x += blockDim.x) {
            const int64_t hb = (x / p.hc) * p.heads + p.h0 + x % p.hc;
            p.eligible[hb] = 1;
            p.bmax[hb] = 0.0f;
        }
    }
    // the key-block units (the longer ones) are dispatched first, so that the
    // short query units fill in behind them
    int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (unit >= p.total_units) return;
    const int64_t k_units = p.total_units - p.q_units;
    unit = unit < k_units ? p.q_units + unit : unit - k_units;

    if (unit < p.q_units) {
        const int64_t units_per_head = (p.seq_len / 16 + QG - 1) / QG;
        const int64_t bh = unit / units_per_head;
        const int64_t g0 = (unit % units_per_head) * QG;
        const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
        const uint16_t *base = p.q + hb * p.seq_len * D;
        float ss[QG][LOADS];
        u32x4 x[QG][LOADS];
#pragma unroll
        for (int gi = 0; gi < QG; ++gi)
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                int64_t row = (g0 + gi) * 16 + l * RPL + sub;
                if (row >= p.seq_len) row = p.seq_len - 1;     // past the head: recompute, not stored
                x[gi][l] = *reinterpret_cast<const u32x4 *>(base + row * D + seg * 8);
            }
#pragma unroll
        for (int gi = 0; gi < QG; ++gi)
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                float s = sumsq8(x[gi][l]);
#pragma unroll
                for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
                ss[gi][l] = s;
            }
#pragma unroll
        for (int gi = 0; gi < QG; ++gi)
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                const int64_t row = (g0 + gi) * 16 + l * RPL + sub;
                if (seg == 0 && row < p.seq_len) p.qnorm[hb * p.seq_len + row] = sqrtf(ss[gi][l]);
            }
    } else {
        const int64_t u = unit - p.q_units;
        const int64_t bh = u / p.n_kb;
        const int64_t kb = u % p.n_kb;
        const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
        const uint16_t *base = p.k + (hb * p.seq_len + kb * p.block_k) * D;
        const int groups = p.block_k / 16;
        float mu[8] = {};
        if constexpr (CENTRED) {
            const float4 m0 = *reinterpret_cast<const float4 *>(p.kmean + hb * D + seg * 8);
            const float4 m1 = *reinterpret_cast<const float4 *>(p.kmean + hb * D + seg * 8 + 4);
            mu[0] = m0.x; mu[1] = m0.y; mu[2] = m0.z; mu[3] = m0.w;
            mu[4] = m1.x; mu[5] = m1.y; mu[6] = m1.z; mu[7] = m1.w;
        }
        auto ksq = [&](u32x4 v) { return CENTRED ? sumsq8_centred(v, mu) : sumsq8(v); };
        float best = 0.0f;     // largest squared row norm seen by this lane's rows
        int gi = 0;
        for (; gi + 2 <= groups; gi += 2) {
            u32x4 x[2][LOADS];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int l = 0; l < LOADS; ++l)
                    x[j][l] = *reinterpret_cast<const u32x4 *>(
                        base + int64_t((gi + j) * 16 + l * RPL + sub) * D + seg * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int l = 0; l < LOADS; ++l) {
                    float s = ksq(x[j][l]);
#pragma unroll
                    for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
                    best = nan_max(best, s);
                }
        }
        if (gi < groups) {
            u32x4 x[LOADS];
#pragma unroll
            for (int l = 0; l < LOADS; ++l)
                x[l] = *reinterpret_cast<const u32x4 *>(base + int64_t(gi * 16 + l * RPL + sub) * D + seg * 8);
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                float s = ksq(x[l]);
#pragma unroll
                for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
                best = nan_max(best, s);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) best = nan_max(best, __shfl_xor(best, off));
        if (lane == 0) p.kmax[hb * p.n_kb + kb] = sqrtf(best);
    }
}

// --------------------------------------------------------------------------
// fsa_bounds, kernel 2: per query block, scale * max ||q_i|| * max kmax over
// its active key blocks. A workgroup covers 16 query blocks (16 lanes each)
// and folds its maximum into the head's with one order-independent atomic
// max. The head's eligibility starts at 1 (set by the norms kernel) and a
// workgroup whose maximum exceeds the limit (or is NaN) clears it: the head
// is eligible exactly when no query block's bound exceeds the limit, in any
// arrival order, with no counter and no fence.
// --------------------------------------------------------------------------
struct ReduceParams {
    const float *qnorm, *kmax;
    int32_t *eligible;
    float *bmax;
    int32_t heads, seq_len, h0, hc, block_q, n_qb, n_kb, chunks;
    int32_t frames, tokens_per_frame, window, ref_frame, block_k;
    float scale, limit;
};

constexpr int kReduceQB = 16;   // query blocks per workgroup (16 lanes each)

__global__ __launch_bounds__(256) void bound_reduce_kernel(ReduceParams p) {
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int qi = tid / 16, sl = tid % 16;
    const int64_t bh = blockIdx.x / p.chunks;
    const int32_t chunk = int32_t(blockIdx.x % p.chunks);
    const int32_t qb = chunk * kReduceQB + qi;
    const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
    float bound = 0.0f;
    if (qb < p.n_qb) {
        const float *qn = p.qnorm + hb * p.seq_len + int64_t(qb) * p.block_q;
        // loops unrolled so that each lane's loads are in flight together
        // (the list entries first, then the key-block maxima they index)
        float qm = 0.0f;
#pragma unroll 8
        for (int i = sl; i < p.block_q; i += 16) qm = nan_max(qm, qn[i]);
        // the block's active key blocks, from the plan's frame rule: every
        // block of the frames in the window, clipped at the ends, and of the
        // reference frame (the same list the plan's CSR holds; computed
        // here so that the kmax loads do not wait for list loads)
        const int32_t kbpf = p.tokens_per_frame / p.block_k;
        const int32_t f = qb / (p.tokens_per_frame / p.block_q);
        const int32_t g0 = f - p.window > 0 ? f - p.window : 0;
        const int32_t g1 = f + p.window < p.frames - 1 ? f + p.window : p.frames - 1;
        const float *km_head = p.kmax + hb * p.n_kb;
        float km = 0.0f;
#pragma unroll 4
        for (int32_t kb = g0 * kbpf + sl; kb < (g1 + 1) * kbpf; kb += 16) km = nan_max(km, km_head[kb]);
        if (p.ref_frame < g0 || p.ref_frame > g1) {
#pragma unroll 2
            for (int32_t kb = p.ref_frame * kbpf + sl; kb < (p.ref_frame + 1) * kbpf; kb += 16)
                km = nan_max(km, km_head[kb]);
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) {
            qm = nan_max(qm, __shfl_xor(qm, off));
            km = nan_max(km, __shfl_xor(km, off));
        }
        bound = p.scale * qm * km;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bound = nan_max(bound, __shfl_xor(bound, off));
    if (lane == 0) red[tid >> 6] = bound;
    __syncthreads();
    if (tid == 0) {
        bound = nan_max(nan_max(red[0], red[1]), nan_max(red[2], red[3]));
        if (bound != bound) bound = __uint_as_float(0x7fc00000u);   // canonical NaN sorts above +inf
        atomicMax(reinterpret_cast<unsigned int *>(p.bmax + hb), __float_as_uint(bound));
        if (!(bound <= p.limit)) p.eligible[hb] = 0;
    }
}

// --------------------------------------------------------------------------
// fsa_attention
// --------------------------------------------------------------------------
struct AttnParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    const float *qnorm, *kmax;
    const int32_t *eligible, *row_ptr, *col_idx;
    const float *kmean;     // key mean per head when the bounds were centred, else null
    int64_t total_wg, per_xcd;
    int32_t heads, seq_len, h0, hc;
    int32_t frames, tokens_per_frame, block_q, block_k, n_qb, n_kb;
    float c;            // scale * log2(e)
};

// Geometry of one LDS stage: 64 keys = two 32-key sub-steps, each holding K
// as two 16-key tiles, segment-major inside a tile ([D/8 segments][16 keys]
// [16 bytes]), then V row-major without padding, its 16-byte segments
// permuted per row (segment s of row r sits in slot s ^ vswz(r)). Both are
// what direct global -> LDS loads write: each load instruction fills 1 KB of
// LDS in lane order.
template <int D>
struct Geo {
    static constexpr int SEGS = D / 8;             // 16-byte segments per K / V row
    static constexpr int KS = D / 16;              // q.k MFMA steps over d (16 each)
    static constexpr int DT = D / 32;              // 32-wide output column tiles
    static constexpr int ROWB = 2 * D;             // bytes per K / V row
    static constexpr int TILE_K = 16 * ROWB;       // one 16-key K tile
    static constexpr int SUB_K = 2 * TILE_K;
    static constexpr int SUB_V = 32 * ROWB;
    static constexpr int SUB_BYTES = SUB_K + SUB_V;
    static constexpr int STAGE = 2 * SUB_BYTES;
    static constexpr int RPL = 256 / ROWB;         // V rows per 256-byte line of the 64 LDS banks
};

// V segment permutation. The transposing V reads of a half wave touch rows
// r0 .. r0 + 3 (r0 a multiple of 4) at the four segments of one 32-wide
// column tile; XOR-ing bits 2 and 3 of the segment index with the row's
// position (in 256-byte lines) spreads those 16 segments over all 64 banks.
template <int D>
__device__ __forceinline__ constexpr int vswz(int row) {
    return 4 * ((row / Geo<D>::RPL) % (Geo<D>::SEGS / 4));
}

// Key order of the q.k product. Row n of the 32x32 MFMA's K operand holds key
// sigma(n) of the sub-step (bits 2 and 3 of n swapped). The result registers
// of lane (n, h = lane / 32) then hold, for query n, keys 8h..8h+7 in
// registers 0..7 and keys 16+8h..16+8h+7 in registers 8..15: after exp and
// rounding, exactly the two p.v B operands (k-steps of 16 keys) of that lane.
__device__ __forceinline__ int sigma(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }

// Workgroup barrier for LDS hand-offs. __syncthreads() also waits for every
// outstanding global load (vmcnt(0)), which would drain the next stage's
// prefetch at each stage boundary. Here: a compiler-only fence (no reordering
// of memory accesses across the barrier), this wave's LDS accesses complete
// (lgkmcnt(0)), then s_barrier.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Query-block order inside a head: the plan's own order (frame by frame). The
// workgroups an XCD runs at one time then cover a contiguous run of frames,
// whose key windows overlap in that XCD's L2. (Ordering the frames from the
// middle outwards balanced no better and shared less.)
__device__ __forceinline__ int32_t rank_to_qblock(int32_t rank) { return rank; }

// Buffer descriptor over `bytes` bytes at `base` (raw, unswizzled, 32-bit
// data), in scalar registers.
__device__ __forceinline__ u32x4 head_rsrc(const void *base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(uint32_t(b));
    r[1] = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32) & 0xffffu);
    r[2] = uint32_t(bytes);
    r[3] = 0x00020000u;
    return r;
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E - 1.
template <int B, int E>
struct Unroll {
    template <typename F>
    static __device__ __forceinline__ void run(F &&f) {
        if constexpr (B < E) {
            f(std::integral_constant<int, B>{});
            Unroll<B + 1, E>::run(f);
        }
    }
};

// One direct global -> LDS load of 16 bytes per lane (buffer_load_dwordx4
// ... lds): lane l's bytes land at lds + 16 l. Written as an instruction of
// its own: the compiler cannot tell that these LDS writes never alias the
// LDS reads between them and would otherwise wait for every load in flight
// before each such read, turning the prefetch synchronous. The load has no
// register result; the walk waits for it explicitly (vmcnt) before the
// barrier that publishes its stage. The asm sets M0 (the LDS base of the
// copy); nothing else in these kernels keeps a value in M0.
__device__ __forceinline__ void load_lds16(u32x4 rs, char *lds, int32_t voff, int32_t soff) {
    const uint32_t m0 = uint32_t(reinterpret_cast<uintptr_t>((lds_void *)lds));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
                 : "memory", "m0");
}

// The same for 4 bytes per lane (lane l's bytes land at lds + 4 l).
__device__ __forceinline__ void load_lds4(u32x4 rs, char *lds, int32_t voff) {
    const uint32_t m0 = uint32_t(reinterpret_cast<uintptr_t>((lds_void *)lds));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

// One workgroup per (batch, head, query block): 8 wavefronts, two per SIMD,
// each owning a tile of 32 query rows (Q fragments and the fp32 output
// accumulators in registers). Stages of 64 keys go straight from global
// memory into four rotating LDS buffers, three stages ahead.
template <int D>
struct AttnKernel {
    using G = Geo<D>;
    static constexpr int NW = 8;
    static constexpr int THREADS = 64 * NW;
    static constexpr int KL = 64 * G::SEGS / THREADS;   // half the 1 KB K (and V) load instructions of a 16-key tile
    static constexpr int LPS = 4 * KL;                  // load instructions per loading wave and stage
    static constexpr int RPI = 64 / G::SEGS;            // V rows per load instruction
    static constexpr int NBUF = 4;
    static constexpr int TAB_BYTES = 512;               // per wavefront: two 64-entry tile tables
    static constexpr int LDS_BYTES = NBUF * G::STAGE + NW * TAB_BYTES;
    static_assert(KL >= 1 && NW * KL * 64 == 64 * G::SEGS, "loads cover the stage");
    static_assert(2 * KL * RPI == 16, "2 KL instructions cover one 16-key tile");

    // The row's 16-key tiles as a table in one vector register: lane l of
    // `cur` holds the byte offset of tile 64 m + l of the row's key list, so
    // a wavefront takes its stage tile's offset with one v_readlane (stage
    // s, tile j of the stage: lane 4 (s % 16) + j). The block columns of the
    // next 64 tiles (lane l: list entry e0 + t / hpb) are fetched when a
    // table is taken into use, 16 stages before they are needed, straight
    // into one of two per-wavefront LDS slots (loaded like the stages, so
    // the stage barriers' waits cover them); the tile-in-block positions are
    // computed then. Tiles past the row end repeat the row's last tile: they
    // are loaded but never weighted.
    struct TileTab {
        int32_t cur, j;
        char *slots;
    };
    static __device__ __forceinline__ int32_t tab_tile(int32_t nquart, int32_t m) {
        const int32_t t = 64 * m + int32_t(threadIdx.x & 63);
        return t < nquart ? t : nquart - 1;
    }
    static __device__ __forceinline__ void tab_issue(u32x4 crs, int32_t e0, int32_t nquart, int hpb, int32_t m,
                                                     TileTab &tt) {
        const int32_t t = tab_tile(nquart, m);
        const int32_t blk = int32_t(uint32_t(t) / uint32_t(hpb));
        tt.j = t - blk * hpb;
        load_lds4(crs, tt.slots + (m & 1) * 256, (e0 + blk) * 4);
    }
    // Table 0 from a plain load (nothing else is in flight yet), table 1
    // requested.
    static __device__ __forceinline__ void tab_init(const gint32 *col, u32x4 crs, int32_t e0, int32_t nquart,
                                                    int hpb, int bk, char *slots, TileTab &tt) {
        tt.slots = slots;
        const int32_t t = tab_tile(nquart, 0);
        const int32_t blk = int32_t(uint32_t(t) / uint32_t(hpb));
        tt.cur = (col[e0 + blk] * bk + 16 * (t - blk * hpb)) * (D * 2);
        tab_issue(crs, e0, nquart, hpb, 1, tt);
    }
    static __device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

    // Byte offset of this wavefront's tile (tile `wave` of the stage; waves
    // 0-3 only) in stage `sig` (wave-uniform, counted from 0); advances sig.
    static __device__ __forceinline__ int32_t next_src(u32x4 crs, TileTab &tt, int32_t &sig, int32_t e0,
                                                       int32_t nquart, int hpb, int bk) {
        if ((sig & 15) == 0 && sig > 0) {
            const int32_t m = sig / 16;
            const int32_t c = *reinterpret_cast<const int32_t *>(tt.slots + (m & 1) * 256 + 4 * (threadIdx.x & 63));
            tt.cur = (c * bk + 16 * tt.j) * (D * 2);
            tab_issue(crs, e0, nquart, hpb, m + 1, tt);
        }
        const int i = 4 * (sig & 15) + wave_id();
        ++sig;
        return __builtin_amdgcn_readlane(tt.cur, i);
    }

    // Direct global -> LDS loads of one stage: wavefront t (0-3, one per
    // SIMD) loads 16-key tile t (K and V; the tile's offset `src` is the
    // scalar offset of the buffer loads), instructions X = 0 .. 2 KL - 1 of
    // each. Waves 4-7 issue no loads, so the second wavefront of every SIMD
    // never stops behind the texture unit and keeps the matrix core fed.
    // K instruction X: lane l loads key l % 16, segment 4 X + l / 16, which
    // is slot 64 X + l of the tile's segment-major layout. V instruction X:
    // lane l loads row RPI X + l / SEGS of the tile into slot l % SEGS, i.e.
    // segment (l % SEGS) ^ vswz(row). Each instruction reads 64-byte (K) or
    // whole-row (V) runs of global memory.
    struct LoadOffsets {
        int32_t k, v;              // per-lane bytes of instruction 0 inside a 16-key global tile
    };
    static __device__ __forceinline__ LoadOffsets load_offsets() {
        const int l = threadIdx.x & 63;
        LoadOffsets lo;
        lo.k = (l % 16) * G::ROWB + (l / 16) * 16;
        const int rt = l / G::SEGS;                            // row inside the instruction's rows
        lo.v = rt * G::ROWB + ((l % G::SEGS) ^ vswz<D>(rt)) * 16;   // vswz(RPI X + rt) = vswz(rt)
        return lo;
    }
    static __device__ __forceinline__ void issue_stage(u32x4 krs, u32x4 vrs, const LoadOffsets &lo, int32_t src,
                                                       char *stage) {
        const int t = wave_id();
        char *kt = stage + (t / 2) * G::SUB_BYTES + (t % 2) * G::TILE_K;
        char *vt = stage + (t / 2) * G::SUB_BYTES + G::SUB_K + 16 * (t % 2) * G::ROWB;
#pragma unroll
        for (int x = 0; x < 2 * KL; ++x) {
            load_lds16(krs, kt + 1024 * x, lo.k, src + 64 * x);
            load_lds16(vrs, vt + 1024 * x, lo.v, src + RPI * x * G::ROWB);
        }
    }

    // LDS byte offsets of this lane's fragment reads relative to a sub-step.
    //   K: lane (n, h) reads key sigma(n) (tile n / 16), segment 2 ks + h;
    //      the k-step adds an immediate.
    //   V: transposing reads, per 16-lane group four rows of 16 d: lane a of
    //      the group addresses row a / 4 and d 4 (a % 4) of the group's block
    //      and receives d = its own column, four consecutive keys. The column
    //      tile dt changes the permuted segment per lane (one offset per dt);
    //      the k-step and the second read (rows + 4) add immediates.
    struct ReadOffsets {
        int32_t k, v[G::DT];
    };
    static __device__ __forceinline__ ReadOffsets read_offsets() {
        const int lane = threadIdx.x & 63;
        const int n = lane & 31, h = lane >> 5;
        const int a = lane & 15, g16 = (lane >> 4) & 1;
        ReadOffsets ro;
        ro.k = (n / 16) * G::TILE_K + h * 256 + (sigma(n) % 16) * 16;
        const int row = 8 * h + a / 4;
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) {
            const int seg = 4 * dt + 2 * g16 + (a % 4) / 2;
            ro.v[dt] = G::SUB_K + row * G::ROWB + (seg ^ vswz<D>(row)) * 16 + 8 * (a % 2);
        }
        return ro;
    }

    // K fragments of one 32-key sub-step: lane (n, h) holds key sigma(n),
    // d = 16 ks + 8 h .. + 8 for each k-step ks.
    static __device__ __forceinline__ void read_k(const char *sub, const ReadOffsets &ro, bf16x8 (&ka)[G::KS]) {
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) ka[ks] = *reinterpret_cast<const bf16x8 *>(sub + ro.k + ks * 512);
    }

    // V^T fragments (A operand of p.v): lane (n, h) holds d = 32 dt + n and
    // keys 16 ks + 8 h .. + 8, from two transposing reads of four keys each.
    template <int PVK>
    static __device__ __forceinline__ void read_v(const char *sub, const ReadOffsets &ro, bf16x8 (&va)[G::DT][2]) {
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
            for (int ks = 0; ks < PVK; ++ks) {
                const char *vp = sub + ro.v[dt] + 16 * ks * G::ROWB;
                const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vp));
                const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(vp + 4 * G::ROWB));
                va[dt][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            }
    }

    // S^T of one 32-key sub-step for this wavefront's 32 query rows.
    static __device__ __forceinline__ f32x16 qk(const bf16x8 (&ka)[G::KS], const bf16x8 (&qf)[G::KS]) {
        f32x16 s = {};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], s, 0, 0, 0);
        return s;
    }

    // Row state of this wavefront's tile. Lane (n, h): query n, keys of half h.
    struct Rows {
        bf16x8 qf[G::KS];          // Q fragments (B operand of q.k)
        f32x16 acc[G::DT];         // O^T accumulators, d = 32 dt + 8 (i / 4) + 4 h + i % 4
        f32x16 s;                  // scores of the current sub-step
        float lsum, mrow, brow;    // this lane's part of the row sum; running max; bound shift
    };

    // Softmax weights of a sub-step (bf16, the p.v B operands) and their
    // contribution to this lane's row sum. PVK = 1: only keys 0..15 of the
    // sub-step are valid.
    template <bool ONLINE, int PVK>
    static __device__ __forceinline__ void weights(Rows &rw, float c, bf16x8 (&pk)[2]) {
        constexpr int NV = 8 * PVK;
        float pr[16];
        if constexpr (!ONLINE) {
            // bound path: p = exp2(s c - B_i log2 e), no max, no rescale
#pragma unroll
            for (int i = 0; i < NV; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(rw.s[i], c, -rw.brow));
        } else {
            // online fallback: running max over the row (both halves), rescale.
            // The max is taken on the raw scores and scaled once: c > 0 and
            // rounding is monotonic, so it equals the max of the scaled scores.
            float cm = rw.s[0];
#pragma unroll
            for (int i = 1; i < NV; ++i) cm = fmaxf(cm, rw.s[i]);
            const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm), false, false);
            cm = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * c;
            // rescale only when some row's max has grown by more than
            // kRescaleSlack: until then the stale max keeps every weight below
            // 2^kRescaleSlack, and the common shift cancels in o = O / l (the
            // branch is uniform over the wavefront)
            if (__any(cm > rw.mrow + kRescaleSlack)) {
                const float mn = fmaxf(rw.mrow, cm);
                const float alpha = __builtin_amdgcn_exp2f(rw.mrow - mn);
                rw.mrow = mn;
                rw.lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) rw.acc[dt] *= alpha;
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(rw.s[i], c, -rw.mrow));
        }
#pragma unroll
        for (int ks = 0; ks < PVK; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) pk[ks][i] = static_cast<__bf16>(pr[8 * ks + i]);
        // row sums of the bf16 weights actually used in p.v
        const bf16x2 ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int ks = 0; ks < PVK; ++ks) {
            rw.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[ks], pk[ks], 0, 1), ones2, rw.lsum, false);
            rw.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[ks], pk[ks], 2, 3), ones2, rw.lsum, false);
            rw.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[ks], pk[ks], 4, 5), ones2, rw.lsum, false);
            rw.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pk[ks], pk[ks], 6, 7), ones2, rw.lsum, false);
        }
    }

    // One software-pipelined sub-step: weights of the current sub-step (its
    // scores were computed one step earlier), the next sub-step's scores
    // (NEXT) and the current sub-step's p.v. HALF: only keys 0..15 of the
    // current sub-step are valid (the row's last, odd 16-key tile).
    template <int NG, bool ONLINE, bool HALF, bool NEXT>
    static __device__ __forceinline__ void step(const char *cur, const char *nxt, const ReadOffsets &ro, Rows &rw,
                                                float c) {
        if constexpr (NG > 0) {
            constexpr int PVK = HALF ? 1 : 2;
            bf16x8 va[G::DT][2];
            bf16x8 ka[G::KS];
            if constexpr (NEXT) read_k(nxt, ro, ka);
            read_v<PVK>(cur, ro, va);
            bf16x8 pk[2];
            if constexpr (ONLINE && NEXT) {
                // the fallback's rescale branch splits the step in two blocks:
                // the next scores' MFMAs go first, so they run under the max
                // and the branch instead of waiting behind them
                const f32x16 sn = qk(ka, rw.qf);
                weights<ONLINE, PVK>(rw, c, pk);
                rw.s = sn;
            } else {
                weights<ONLINE, PVK>(rw, c, pk);
                if constexpr (NEXT) rw.s = qk(ka, rw.qf);
            }
#pragma unroll
            for (int ks = 0; ks < PVK; ++ks)
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt)
                    rw.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][ks], pk[ks], rw.acc[dt], 0, 0, 0);
        }
    }

    // Wait until at most `vm` of this wavefront's global loads are
    // outstanding (loads complete in order) and its LDS accesses are done,
    // then meet the workgroup at the barrier.
    template <int vm>
    static __device__ __forceinline__ void stage_barrier() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (0 << 8));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }

    // The block-list walk in stages of 64 keys (two sub-steps), loaded
    // straight into LDS three stages ahead. Stage s sits in buffer s % 4.
    // Its sub-steps 2s and 2s + 1 read K of 2s + 1 and 2s + 2 (the latter in
    // stage s + 1) and V of their own. The barrier after sub-step 2s first
    // waits for this wavefront's loads of stage s + 1 (waves 0-3 load; only
    // their loads of stage s + 2 may still be in flight), so it publishes
    // stage s + 1; every wavefront has then also finished stage s - 1, whose
    // buffer receives stage s + 3. NG = 0: a wavefront without rows still
    // loads its tile of every stage (if it is one of waves 0-3) and meets
    // every barrier.
    template <int NG, bool ONLINE>
    static __device__ __forceinline__ void walk(const AttnParams &p, char *smem, const uint16_t *kh,
                                                const uint16_t *vh, int32_t e0, int32_t nquart, Rows &rw) {
        const int nst = (nquart + 3) / 4;
        if (nst == 0) return;                       // (a plan row always lists its own frame)
        const int hpb = p.block_k / 16;
        const gint32 *col = (const gint32 *)(p.col_idx);
        const int64_t slab = int64_t(p.seq_len) * D * 2;
        const u32x4 krs = head_rsrc(kh, slab), vrs = head_rsrc(vh, slab);
        const u32x4 crs = head_rsrc(p.col_idx, int64_t(e0 + (nquart - 1) / hpb + 1) * 4);
        const LoadOffsets lo = load_offsets();
        const ReadOffsets ro = read_offsets();
        TileTab tt;
        const bool loader = wave_id() < 4;
        if (loader) tab_init(col, crs, e0, nquart, hpb, p.block_k, smem + NBUF * G::STAGE + wave_id() * TAB_BYTES, tt);
        int32_t sig = 0;
        char *const b0 = smem, *const b1 = smem + G::STAGE, *const b2 = smem + 2 * G::STAGE,
                    *const b3 = smem + 3 * G::STAGE;

        // stages 0 .. 2 (those that exist) in flight, 0 and 1 complete
        if (loader) issue_stage(krs, vrs, lo, next_src(crs, tt, sig, e0, nquart, hpb, p.block_k), b0);
        if (loader && nst > 1) issue_stage(krs, vrs, lo, next_src(crs, tt, sig, e0, nquart, hpb, p.block_k), b1);
        if (nst > 2) {
            if (loader) issue_stage(krs, vrs, lo, next_src(crs, tt, sig, e0, nquart, hpb, p.block_k), b2);
            stage_barrier<LPS>();
        } else {
            stage_barrier<0>();
        }
        if constexpr (NG > 0) {
            bf16x8 ka[G::KS];
            read_k(b0, ro, ka);
            rw.s = qk(ka, rw.qf);
        }

        // stage s but the last: two full sub-steps, each with a next one,
        // the barrier between them, then the loads of stage s + 3 (if it
        // exists). The barrier's wait leaves stage s + 2's loads in flight
        // when that stage exists; when it does not (the last such stage),
        // stage s + 1's are the newest and the wait must drain them.
        int s = 0;
        auto body = [&](char *bc, char *bn, char *bl) {
            step<NG, ONLINE, false, true>(bc, bc + G::SUB_BYTES, ro, rw, p.c);
            if (s + 2 < nst)
                stage_barrier<LPS>();
            else
                stage_barrier<0>();
            if (loader && s + 3 < nst) issue_stage(krs, vrs, lo, next_src(crs, tt, sig, e0, nquart, hpb, p.block_k), bl);
            step<NG, ONLINE, false, true>(bc + G::SUB_BYTES, bn, ro, rw, p.c);
            ++s;
        };
        // stage s uses buffer s % 4; the loop is unrolled by four so that
        // every LDS address is a fixed per-lane offset plus an immediate
        while (s + 4 <= nst - 1) {
            body(b0, b1, b3);
            body(b1, b2, b0);
            body(b2, b3, b1);
            body(b3, b0, b2);
        }
        if (s < nst - 1) body(b0, b1, b3);
        if (s < nst - 1) body(b1, b2, b0);
        if (s < nst - 1) body(b2, b3, b1);
        // the last stage: 1 to 4 valid 16-key tiles
        const int r4 = s % 4;
        char *const b = r4 == 0 ? b0 : (r4 == 1 ? b1 : (r4 == 2 ? b2 : b3));
        switch (nquart - 4 * (nst - 1)) {
            case 1: step<NG, ONLINE, true, false>(b, b, ro, rw, p.c); break;
            case 2: step<NG, ONLINE, false, false>(b, b, ro, rw, p.c); break;
            case 3:
                step<NG, ONLINE, false, true>(b, b + G::SUB_BYTES, ro, rw, p.c);
                step<NG, ONLINE, true, false>(b + G::SUB_BYTES, b, ro, rw, p.c);
                break;
            default:
                step<NG, ONLINE, false, true>(b, b + G::SUB_BYTES, ro, rw, p.c);
                step<NG, ONLINE, false, false>(b + G::SUB_BYTES, b, ro, rw, p.c);
                break;
        }
        // no load into LDS may still be in flight when the buffers are reused
        __builtin_amdgcn_s_waitcnt((0) | (0 << 14) | (7 << 4) | (15 << 8));   // vmcnt(0)
    }

    // This wavefront's tile: rows row0 .. row0 + nvalid - 1 (nvalid 16 or 32)
    // for NG = 1; NG = 0 meets every barrier (and loads, if one of waves 0-3).
    // CENTRED: the bounds were taken over centred keys; mu is the head's key mean.
    template <int NG, bool CENTRED>
    static __device__ __forceinline__ void tile(const AttnParams &p, char *smem, int64_t head_row0, int32_t row0,
                                                int nvalid, const uint16_t *kh, const uint16_t *vh, int32_t e0,
                                                int32_t nquart, bool online, float mk, const float *mu) {
        const int lane = threadIdx.x & 63;
        const int n = lane & 31, h = lane >> 5;
        const int32_t row = row0 + (n < nvalid ? n : nvalid - 1);   // rows past the tile recompute a valid one
        Rows rw;
        rw.lsum = 0.0f;
        rw.mrow = -__builtin_huge_valf();
        rw.brow = 0.0f;
        if constexpr (NG > 0) {
            const uint16_t *qr = p.q + (head_row0 + row) * D;
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) rw.qf[ks] = *reinterpret_cast<const bf16x8 *>(qr + 16 * ks + 8 * h);
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt) rw.acc[dt] = f32x16{};
            if (!online) {
                float shift = p.qnorm[head_row0 + row] * mk;
                if constexpr (CENTRED) {
                    // centred keys: s_ij = scale q_i.mu + scale q_i.(k_j - mu), and the
                    // bound covers the second term; add this row's q_i.mu. Each half of
                    // the wavefront holds half of the row's columns.
                    float part = 0.0f;
#pragma unroll
                    for (int ks = 0; ks < G::KS; ++ks) {
                        const float4 m0 = *reinterpret_cast<const float4 *>(mu + 16 * ks + 8 * h);
                        const float4 m1 = *reinterpret_cast<const float4 *>(mu + 16 * ks + 8 * h + 4);
                        const bf16x8 x = rw.qf[ks];
                        part = fmaf(float(x[0]), m0.x, part);
                        part = fmaf(float(x[1]), m0.y, part);
                        part = fmaf(float(x[2]), m0.z, part);
                        part = fmaf(float(x[3]), m0.w, part);
                        part = fmaf(float(x[4]), m1.x, part);
                        part = fmaf(float(x[5]), m1.y, part);
                        part = fmaf(float(x[6]), m1.z, part);
                        part = fmaf(float(x[7]), m1.w, part);
                    }
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                                     __float_as_uint(part), false, false);
                    shift += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // same value in both halves
                }
                rw.brow = p.c * shift;
            }
        }
        if (online)
            walk<NG, true>(p, smem, kh, vh, e0, nquart, rw);
        else
            walk<NG, false>(p, smem, kh, vh, e0, nquart, rw);
        if constexpr (NG > 0) {
            // both halves of a row hold partial sums over disjoint keys
            const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rw.lsum), __float_as_uint(rw.lsum),
                                                              false, false);
            const float inv = 1.0f / (__uint_as_float(sw2[0]) + __uint_as_float(sw2[1]));
            if (n < nvalid) {
                uint16_t *orow = p.o + (head_row0 + row) * D;
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        __bf16 h4[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) h4[i] = static_cast<__bf16>(rw.acc[dt][4 * a + i] * inv);
                        uint2 w;
                        w.x = uint32_t(__builtin_bit_cast(uint16_t, h4[0])) |
                              (uint32_t(__builtin_bit_cast(uint16_t, h4[1])) << 16);
                        w.y = uint32_t(__builtin_bit_cast(uint16_t, h4[2])) |
                              (uint32_t(__builtin_bit_cast(uint16_t, h4[3])) << 16);
                        *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * a + 4 * h) = w;
                    }
            }
        }
    }

    template <bool CENTRED>
    static __device__ void run(const AttnParams &p) {
        extern __shared__ __attribute__((aligned(16))) char smem[];
        // stage buffer 3 receives its first load only after every wavefront has
        // passed the walk's first barrier, so it can hold this reduction
        float *red = reinterpret_cast<float *>(smem + 3 * G::STAGE);
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

        // XCD-aware order: consecutive workgroup ids go to different XCDs, so
        // give each XCD a contiguous range of (head, query block) work.
        const int64_t bid = blockIdx.x;
        const int64_t L = (bid & 7) * p.per_xcd + (bid >> 3);
        if (L >= p.total_wg) return;
        const int64_t bh = L / p.n_qb;
        const int32_t qb = rank_to_qblock(int32_t(L % p.n_qb));
        const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
        const int64_t head_row0 = hb * p.seq_len;
        const uint16_t *kh = p.k + head_row0 * D;
        const uint16_t *vh = p.v + head_row0 * D;
        const int32_t e0 = __builtin_amdgcn_readfirstlane(p.row_ptr[qb]);
        const int32_t e1 = __builtin_amdgcn_readfirstlane(p.row_ptr[qb + 1]);
        const int32_t nquart = (e1 - e0) * (p.block_k / 16);
        const bool online = __builtin_amdgcn_readfirstlane(p.eligible[hb]) == 0;
        const float *mu = CENTRED ? p.kmean + hb * D : nullptr;

        // bound path: largest key norm over the row's active key blocks
        float mk = 0.0f;
        if (!online) {
            for (int32_t e = e0 + tid; e < e1; e += THREADS) mk = fmaxf(mk, p.kmax[hb * p.n_kb + p.col_idx[e]]);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mk = fmaxf(mk, __shfl_xor(mk, off));
            if (lane == 0) red[wave] = mk;
            lds_barrier();
#pragma unroll
            for (int w = 0; w < NW; ++w) mk = fmaxf(mk, red[w]);
        }

        // 32-row tiles of the query block (the last may hold 16 rows), one per
        // wavefront, NW per pass over the keys
        const int ntiles = (p.block_q + 31) / 32;
        for (int t0 = 0; t0 < ntiles; t0 += NW) {
            const int my = t0 + wave;
            const int32_t row0 = qb * p.block_q + 32 * my;
            const int nvalid = p.block_q - 32 * my < 32 ? p.block_q - 32 * my : 32;
            if (online) {
                if (my < ntiles)
                    tile<1, false>(p, smem, head_row0, row0, nvalid, kh, vh, e0, nquart, true, 0.0f, nullptr);
                else
                    tile<0, false>(p, smem, head_row0, row0, nvalid, kh, vh, e0, nquart, true, 0.0f, nullptr);
            } else if (my < ntiles) {
                tile<1, CENTRED>(p, smem, head_row0, row0, nvalid, kh, vh, e0, nquart, false, mk, mu);
            } else {
                tile<0, CENTRED>(p, smem, head_row0, row0, nvalid, kh, vh, e0, nquart, false, mk, mu);
            }
            if (t0 + NW < ntiles) lds_barrier();     // LDS reused by the next pass
        }
    }
};

// One instantiation per head dim, and per centring: the row shift of the
// centred one also adds q_i.mean, the plain one keeps the prologue lean.
template <int D, bool CENTRED>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
attention_kernel(AttnParams p) {
    AttnKernel<D>::template run<CENTRED>(p);
}

}  // namespace

const char *hip_error_text(int code) { return hipGetErrorString(static_cast<hipError_t>(code)); }

int launch_bounds(const BoundsLaunch &a) {
    const fsa_plan_info &pl = *a.plan;
    hipStream_t stream = static_cast<hipStream_t>(a.stream);
    // one 16-row group of q per wavefront: the finest split is the fastest
    // (sr720 -3.5 %, sr1080 -2.5 % against two groups; four are slower)
    constexpr int QG = 1;
    const int64_t nbh = int64_t(a.batch) * a.head_count;
    hipError_t err = hipSuccess;
    if (a.kmean) {
        KeySumParams kp;
        kp.k = static_cast<const uint16_t *>(a.k);
        kp.partial = a.qnorm;
        kp.kmean = a.kmean;
        kp.heads = a.heads;
        kp.seq_len = pl.seq_len;
        kp.h0 = a.head_offset;
        kp.hc = a.head_count;
        const int chunk = a.head_dim == 128 ? key_chunk<128>() : key_chunk<64>();
        kp.chunks = (pl.seq_len + chunk - 1) / chunk;      // > 1 only when N > 2D, so chunks * D <= N
        const unsigned grid0 = unsigned(nbh * kp.chunks);
        if (a.head_dim == 128)
            hipLaunchKernelGGL(key_sum_kernel<128>, dim3(grid0), dim3(256), 0, stream, kp);
        else
            hipLaunchKernelGGL(key_sum_kernel<64>, dim3(grid0), dim3(256), 0, stream, kp);
        err = hipGetLastError();
        if (err != hipSuccess) return int(err);
        if (kp.chunks > 1) {
            if (a.head_dim == 128)
                hipLaunchKernelGGL(key_mean_kernel<128>, dim3(unsigned(nbh)), dim3(1024), 0, stream, kp);
            else
                hipLaunchKernelGGL(key_mean_kernel<64>, dim3(unsigned(nbh)), dim3(1024), 0, stream, kp);
            err = hipGetLastError();
            if (err != hipSuccess) return int(err);
        }
    }
    NormsParams np;
    np.q = static_cast<const uint16_t *>(a.q);
    np.k = static_cast<const uint16_t *>(a.k);
    np.qnorm = a.qnorm;
    np.kmax = a.kmax;
    np.eligible = a.eligible;
    np.bmax = a.bmax;
    np.kmean = a.kmean;
    np.q_units = nbh * ((pl.seq_len / 16 + QG - 1) / QG);
    np.total_units = np.q_units + nbh * pl.n_kblocks;
    np.batch = a.batch;
    np.heads = a.heads;
    np.seq_len = pl.seq_len;
    np.h0 = a.head_offset;
    np.hc = a.head_count;
    np.block_k = pl.block_k;
    np.n_kb = pl.n_kblocks;
    const unsigned grid1 = unsigned((np.total_units + 3) / 4);
    if (a.head_dim == 128) {
        if (a.kmean)
            hipLaunchKernelGGL((norms_kernel<128, QG, true>), dim3(grid1), dim3(256), 0, stream, np);
        else
            hipLaunchKernelGGL((norms_kernel<128, QG, false>), dim3(grid1), dim3(256), 0, stream, np);
    } else {
        if (a.kmean)
            hipLaunchKernelGGL((norms_kernel<64, QG, true>), dim3(grid1), dim3(256), 0, stream, np);
        else
            hipLaunchKernelGGL((norms_kernel<64, QG, false>), dim3(grid1), dim3(256), 0, stream, np);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return int(err);

    ReduceParams rp;
    rp.qnorm = a.qnorm;
    rp.kmax = a.kmax;
    rp.eligible = a.eligible;
    rp.bmax = a.bmax;
    rp.heads = a.heads;
    rp.seq_len = pl.seq_len;
    rp.h0 = a.head_offset;
    rp.hc = a.head_count;
    rp.block_q = pl.block_q;
    rp.n_qb = pl.n_qblocks;
    rp.n_kb = pl.n_kblocks;
    rp.frames = pl.frames;
    rp.tokens_per_frame = pl.tokens_per_frame;
    rp.window = pl.window;
    rp.ref_frame = pl.ref_frame;
    rp.block_k = pl.block_k;
    rp.scale = a.scale;
    rp.limit = a.bound_limit;
    rp.chunks = (pl.n_qblocks + kReduceQB - 1) / kReduceQB;
    const unsigned grid2 = unsigned(nbh * rp.chunks);
    hipLaunchKernelGGL(bound_reduce_kernel, dim3(grid2), dim3(256), 0, stream, rp);
    err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

// One launch: 8 * ceil(work / 8) workgroups of 512 threads (the kernel remaps
// ids XCD-first and returns for ids past the work), dynamic LDS for the three
// stage buffers. The LDS size needs the function attribute, set once per
// device.
template <int D, bool CENTRED>
int launch_cfg(const AttnParams &p, hipStream_t stream) {
    using K = AttnKernel<D>;
    auto fn = attention_kernel<D, CENTRED>;
    static std::atomic<uint64_t> attr_done{0};     // one bit per device
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return int(err);
    const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
    if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  K::LDS_BYTES);
        if (err != hipSuccess) return int(err);
        attr_done.fetch_or(bit, std::memory_order_acq_rel);
    }
    const unsigned grid = unsigned(p.per_xcd * 8);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(K::THREADS), K::LDS_BYTES, stream, p);
    err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

int launch_attention(const AttentionLaunch &a) {
    const fsa_plan_info &pl = *a.plan;
    AttnParams p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.o = static_cast<uint16_t *>(a.o);
    p.qnorm = a.qnorm;
    p.kmax = a.kmax;
    p.eligible = a.eligible;
    p.kmean = a.kmean;
    p.row_ptr = a.row_ptr;
    p.col_idx = a.col_idx;
    p.total_wg = int64_t(a.batch) * a.head_count * pl.n_qblocks;
    p.per_xcd = (p.total_wg + 7) / 8;
    p.heads = a.heads;
    p.seq_len = pl.seq_len;
    p.h0 = a.head_offset;
    p.hc = a.head_count;
    p.frames = pl.frames;
    p.tokens_per_frame = pl.tokens_per_frame;
    p.block_q = pl.block_q;
    p.block_k = pl.block_k;
    p.n_qb = pl.n_qblocks;
    p.n_kb = pl.n_kblocks;
    p.c = a.scale * kLog2e;
    hipStream_t stream = static_cast<hipStream_t>(a.stream);
    if (a.head_dim == 128) return a.kmean ? launch_cfg<128, true>(p, stream) : launch_cfg<128, false>(p, stream);
    return a.kmean ? launch_cfg<64, true>(p, stream) : launch_cfg<64, false>(p, stream);
}

}  // namespace fsa
