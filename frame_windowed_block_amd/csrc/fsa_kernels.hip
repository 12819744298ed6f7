// HIP kernels of libfsa for AMD Instinct MI355X (gfx950, CDNA4).
//
// Sources: the pages on the HeyGen / Google Cloud Avatar IV port
//   [vi:Mask]    aihot.vn, "HeyGen tối ưu hóa mô hình Avatar IV trên Google Cloud
//                Trillium TPU", section "Xóa bỏ mặt nạ (Mask)" and Fig. 3;
//   [vi:Softmax] same page, section "Giải phóng Softmax" and Fig. 4;
//   [uk:Softmax] bib.com.ua, "HeyGen прискорила Avatar IV на TPU у 1,86 раза",
//                section on breaking the softmax serial chain.
//
// fsa_bounds runs two kernels. norms_kernel streams q and k once (the HBM-bound
// part): it writes ||q_i|| per row and, per key block, the largest ||k_j||
// ("a small array of precomputed norms", [vi:Softmax]). bound_reduce_kernel
// then derives, per query block, scale * max ||q_i|| * max kmax over the
// block's active key blocks, folds it into the head's largest row bound, and
// the last block of each head writes the head's eligibility ([vi:Softmax]:
// eligibility is checked per attention head).
//
// fsa_attention is one kernel: one workgroup per (batch, head, query block).
// It walks the query block's active key-block list once, window and reference
// frame alike ([vi:Mask]: one pass covers the whole mask), in 32-key chunks
// that may join the 16-key tail of one block to the head of the next; no chunk
// needs a mask predicate, and an odd count of 16-key tiles leaves one half
// chunk at the very end. Per chunk:
//   S^T = K Q^T       bf16 MFMA 16x16x32 (K rows permuted so that each lane
//                     ends up holding 8 consecutive keys of one query row)
//   P   = exp2(S * scale * log2e - B_i * log2e)
//                     B_i = scale * ||q_i|| * max kmax over the row's active
//                     key blocks, fixed before the loop ([vi:Softmax]); no
//                     running max, no rescale
//   O^T += V^T P^T    bf16 MFMA 16x16x32 with V staged transposed in LDS
// Heads whose bound is too loose run the same walk with the standard running
// max and rescale instead ([vi:Softmax], Fig. 4), chosen by a branch that is
// uniform over the workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fsa_internal.h"

// Attention kernel configuration (overridable at build time for tuning sweeps).
#ifndef FSA_RG
#define FSA_RG 2      // 16-row query groups per wavefront
#endif
#ifndef FSA_NW
#define FSA_NW 8      // wavefronts per workgroup
#endif
#ifndef FSA_KCH
#define FSA_KCH 64    // keys per LDS stage
#endif
#ifndef FSA_WPE
#define FSA_WPE 2     // wavefronts per SIMD the registers are budgeted for
#endif

namespace fsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Read-only device data addressed uniformly: loads through the constant address
// space are selected as scalar (SMEM) loads.
typedef __attribute__((address_space(4))) const int32_t cint32;

constexpr float kLog2e = 1.4426950408889634f;

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

// Max that lets a NaN through (a NaN norm must make the head ineligible).
__device__ __forceinline__ float nan_max(float a, float b) { return (b > a || b != b) ? b : a; }

// --------------------------------------------------------------------------
// fsa_bounds, kernel 1: row norms of q, largest key norm per key block.
// Work unit = one wavefront: either QG 16-row groups of q, or one key block.
// --------------------------------------------------------------------------
struct NormsParams {
    const uint16_t *q, *k;
    float *qnorm, *kmax;
    int32_t *eligible;
    float *bmax;
    int64_t q_units, total_units;
    int32_t batch, heads, seq_len, h0, hc, block_k, n_kb;
};

template <int D, int QG>
__global__ __launch_bounds__(256) void norms_kernel(NormsParams p) {
    constexpr int LPR = D / 8;          // lanes per row: 16 bytes each
    constexpr int RPL = 64 / LPR;       // rows covered by one wave-wide load
    constexpr int LOADS = 16 / RPL;     // loads per 16-row group
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR;
    const int seg = lane % LPR;

    if (blockIdx.x == 0) {              // accumulators of bound_reduce_kernel
        const int64_t nbh = int64_t(p.batch) * p.hc;
        for (int64_t x = threadIdx.x; x < nbh; x += blockDim.x) {
            const int64_t hb = (x / p.hc) * p.heads + p.h0 + x % p.hc;
            p.eligible[hb] = 0;
            p.bmax[hb] = 0.0f;
        }
    }
    const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (unit >= p.total_units) return;

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
                    float s = sumsq8(x[j][l]);
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
                float s = sumsq8(x[l]);
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
// max; the last workgroup of a head to arrive writes the head's eligibility.
// --------------------------------------------------------------------------
struct ReduceParams {
    const float *qnorm, *kmax;
    const int32_t *row_ptr, *col_idx;
    int32_t *eligible;
    float *bmax;
    int32_t heads, seq_len, h0, hc, block_q, n_qb, n_kb, chunks;
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
        float qm = 0.0f;
        for (int i = sl; i < p.block_q; i += 16) qm = nan_max(qm, qn[i]);
        const int32_t e0 = p.row_ptr[qb], e1 = p.row_ptr[qb + 1];
        float km = 0.0f;
        for (int32_t e = e0 + sl; e < e1; e += 16) km = nan_max(km, p.kmax[hb * p.n_kb + p.col_idx[e]]);
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
        __threadfence();
        const int old = atomicAdd(p.eligible + hb, 1);
        if (old == p.chunks - 1) {
            __threadfence();
            const float m = __uint_as_float(atomicOr(reinterpret_cast<unsigned int *>(p.bmax + hb), 0u));
            p.eligible[hb] = (m <= p.limit) ? 1 : 0;
        }
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
    int64_t total_wg, per_xcd;
    int32_t heads, seq_len, h0, hc;
    int32_t frames, tokens_per_frame, block_q, block_k, n_qb, n_kb;
    float c;            // scale * log2(e)
};

// Geometry of one LDS stage: KCH keys = KCH/32 "sub-steps" of 32 keys, each
// holding K [32][D] (16-byte segments swizzled) and V^T [4 key octets][D][8].
template <int D, int KCH>
struct Geo {
    static constexpr int SEGS = D / 8;             // 16-byte segments per K row
    static constexpr int DS = D / 32;              // q.k MFMA steps over d
    static constexpr int DT = D / 16;              // 16-wide output column tiles
    static constexpr int SUB = KCH / 32;           // 32-key p.v MFMA steps per stage
    static constexpr int QUARTERS = KCH / 16;      // 16-key tiles per stage
    static constexpr int SUB_K = 32 * D * 2;
    static constexpr int SUB_BYTES = 2 * SUB_K;    // K then V^T
    static constexpr int STAGE = SUB * SUB_BYTES;
};

// Swizzle of K's 16-byte segments: row r stores segment s at s ^ kswz(r). With
// the permuted row order used by the q.k fragments, the 16 lanes of a quarter
// wave read 16 different segments of their rows: no LDS bank conflicts.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    if constexpr (D == 128) return (r & 3) | (((r >> 3) & 3) << 2);
    else return (r & 3) | (((r >> 3) & 1) << 2);
}

constexpr int ar(int n) { return n > 0 ? n : 1; }   // array extent for n row groups

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

// Query-block order inside a head: frames from the middle outwards, so the
// first workgroups of a head share their key window in L2 and the cheaper edge
// frames (fewer visible frames) run last.
__device__ __forceinline__ int32_t rank_to_qblock(int32_t rank, int32_t frames, int32_t qpf) {
    const int32_t fr = rank / qpf, qi = rank % qpf;
    const int32_t mid = (frames - 1) / 2;
    const int32_t f = (fr & 1) ? mid + (fr + 1) / 2 : mid - fr / 2;
    return f * qpf + qi;
}

// D: head dim. RG: 16-row groups per wavefront. NW: wavefronts per workgroup.
// KCH: keys per LDS stage (32 or 64).
template <int D, int RG, int NW, int KCH>
struct AttnKernel {
    using G = Geo<D, KCH>;
    static constexpr int THREADS = 64 * NW;
    static constexpr int KL = (KCH * G::SEGS + THREADS - 1) / THREADS;            // K segments / thread
    static constexpr int VTASKS = (KCH / 8) * (D / 2);
    static constexpr int VL = (VTASKS + THREADS - 1) / THREADS;                   // V tasks / thread
    static constexpr int LDS_BYTES = 2 * G::STAGE + 64;

    // Global -> register staging of one stage.
    struct Stage {
        u32x4 k[KL];
        uint32_t v[VL][8];
    };

    // Where the 16-key tiles of one stage come from: the raw list entries
    // (col_idx) and tile offsets; the key index col * bk + 16 * j is formed
    // only when the stage is loaded, so the scalar loads of the entries are
    // in flight for a whole stage before they are needed. Named fields, not
    // arrays: a lane-varying pick must stay a select chain.
    static_assert(G::QUARTERS == 2 || G::QUARTERS == 4, "stages of 32 or 64 keys");
    struct Src {
        int c0, c1, c2, c3;     // list entries (block indices), -1 past the row end
        int j0, j1, j2, j3;     // 16-key tile inside the block
    };
    // Cursor over the row's 16-key tiles: list position e and tile j in its block.
    struct Cursor {
        int32_t e, j;
    };

    static __device__ __forceinline__ Src next_src(const cint32 *col, Cursor &cur, int32_t e1, int hpb) {
        Src s;
        auto one = [&](int &c, int &j) {
            if (cur.e < e1) {
                c = col[cur.e];
                j = cur.j;
                if (++cur.j == hpb) {
                    cur.j = 0;
                    ++cur.e;
                }
            } else {
                c = -1;
                j = 0;
            }
        };
        one(s.c0, s.j0);
        one(s.c1, s.j1);
        if constexpr (G::QUARTERS > 2) {
            one(s.c2, s.j2);
            one(s.c3, s.j3);
        } else {
            s.c2 = s.c3 = -1;
            s.j2 = s.j3 = 0;
        }
        return s;
    }

    // src[j] for a lane-varying j, computed on values (a select on field
    // addresses would turn the struct into a dynamically indexed stack array)
    static __device__ __forceinline__ int pick(int j, int q0, int q1, int q2, int q3) {
        const int lo = j == 0 ? q0 : q1;
        const int hi = j == 2 ? q2 : q3;
        return (G::QUARTERS == 2 || j < 2) ? lo : hi;
    }

    // Each wave's loads of a stage fall in one 16-key quarter per (x) slot: a
    // wave-wide K load covers 64 / SEGS consecutive keys and a V load one key
    // octet, both inside one quarter. The quarter index is therefore uniform
    // over the wave and is made scalar, so the source pick is a scalar select.
    static_assert(64 % G::SEGS == 0 && 16 % (64 / G::SEGS) == 0, "wave-wide K load inside one quarter");
    static_assert((D / 2) % 64 == 0 || 64 % (D / 2) == 0, "wave-wide V load inside one quarter");

    // FULL: every quarter of the stage lies inside the row (all but possibly
    // the last stage), so no load needs a validity check.
    template <bool FULL>
    static __device__ __forceinline__ void load_stage(const uint16_t *kh, const uint16_t *vh,
                                                      const Src src, int bk, Stage &st) {
        const int t = threadIdx.x;
        const int s0 = src.c0 < 0 ? -1 : src.c0 * bk + 16 * src.j0;
        const int s1 = src.c1 < 0 ? -1 : src.c1 * bk + 16 * src.j1;
        const int s2 = src.c2 < 0 ? -1 : src.c2 * bk + 16 * src.j2;
        const int s3 = src.c3 < 0 ? -1 : src.c3 * bk + 16 * src.j3;
#pragma unroll
        for (int x = 0; x < KL; ++x) {
            const int idx = t + x * THREADS;
            const int key = idx / G::SEGS, seg = idx % G::SEGS;
            const int quarter = __builtin_amdgcn_readfirstlane(key / 16);
            const int qs = key < KCH ? pick(quarter, s0, s1, s2, s3) : -1;
            if (FULL || qs >= 0)
                st.k[x] = *reinterpret_cast<const u32x4 *>(kh + int64_t(qs + key % 16) * D + seg * 8);
            else
                st.k[x] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int x = 0; x < VL; ++x) {
            const int task = t + x * THREADS;
            const int oct = task / (D / 2), dp = task % (D / 2);
            const int quarter = __builtin_amdgcn_readfirstlane(oct / 2);
            const int qs = oct < KCH / 8 ? pick(quarter, s0, s1, s2, s3) : -1;
            if (FULL || qs >= 0) {
                const uint16_t *vp = vh + int64_t(qs + 8 * (oct & 1)) * D + 2 * dp;
#pragma unroll
                for (int i = 0; i < 8; ++i) st.v[x][i] = *reinterpret_cast<const uint32_t *>(vp + int64_t(i) * D);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) st.v[x][i] = 0u;
            }
        }
    }

    static __device__ __forceinline__ void store_stage(char *stage, const Stage &st) {
        const int t = threadIdx.x;
#pragma unroll
        for (int x = 0; x < KL; ++x) {
            const int idx = t + x * THREADS;
            const int key = idx / G::SEGS, seg = idx % G::SEGS;
            if (key < KCH) {
                const int kk = key % 32;
                char *kb = stage + (key / 32) * G::SUB_BYTES;
                *reinterpret_cast<u32x4 *>(kb + (kk * G::SEGS + (seg ^ kswz<D>(kk))) * 16) = st.k[x];
            }
        }
#pragma unroll
        for (int x = 0; x < VL; ++x) {
            const int task = t + x * THREADS;
            const int oct = task / (D / 2), dp = task % (D / 2);
            if (oct < KCH / 8) {
                u32x4 lo, hi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    lo[j] = __builtin_amdgcn_perm(st.v[x][2 * j + 1], st.v[x][2 * j], 0x05040100u);
                    hi[j] = __builtin_amdgcn_perm(st.v[x][2 * j + 1], st.v[x][2 * j], 0x07060302u);
                }
                char *vt = stage + (oct / 4) * G::SUB_BYTES + G::SUB_K;
                const int kg = oct % 4;
                *reinterpret_cast<u32x4 *>(vt + (kg * D + 2 * dp) * 16) = lo;
                *reinterpret_cast<u32x4 *>(vt + (kg * D + 2 * dp + 1) * 16) = hi;
            }
        }
    }

    // One 32-key sub-step for NG row groups. TAIL: only keys 0..15 are valid.
    template <int NG, bool ONLINE, bool TAIL>
    static __device__ __forceinline__ void compute_sub(const char *sub, const bf16x8 (&qf)[ar(NG)][G::DS],
                                                       f32x4 (&acc)[ar(NG)][G::DT], f32x4 (&lsum)[ar(NG)],
                                                       float (&mrow)[ar(NG)], const float (&brow)[ar(NG)], float c) {
        if constexpr (NG > 0) {
            const int lane = threadIdx.x & 63;
            const int m = lane & 15, g = lane >> 4;
            bf16x8 ka[2][G::DS];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = 8 * (m >> 2) + 4 * j + (m & 3);
#pragma unroll
                for (int ds = 0; ds < G::DS; ++ds) {
                    const int seg = 4 * ds + g;
                    ka[j][ds] = *reinterpret_cast<const bf16x8 *>(sub + (r * G::SEGS + (seg ^ kswz<D>(r))) * 16);
                }
            }
            bf16x8 va[G::DT];
            const char *vt = sub + G::SUB_K;
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt)
                va[dt] = *reinterpret_cast<const bf16x8 *>(vt + (g * D + 16 * dt + m) * 16);
            bf16x8 ones8;
#pragma unroll
            for (int i = 0; i < 8; ++i) ones8[i] = static_cast<__bf16>(1.0f);

#pragma unroll
            for (int rg = 0; rg < NG; ++rg) {
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ds = 0; ds < G::DS; ++ds) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][ds], qf[rg][ds], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][ds], qf[rg][ds], s1, 0, 0, 0);
                }
                // this lane: query row m of the group, keys 8g .. 8g+7 of the sub-step
                const float x[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
                float pr[8];
                if constexpr (!ONLINE) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(x[i], c, -brow[rg]));
                    if constexpr (TAIL) {
                        if (g >= 2) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) pr[i] = 0.0f;
                        }
                    }
                } else {
                    float t[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) t[i] = x[i] * c;
                    if constexpr (TAIL) {
                        if (g >= 2) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) t[i] = -__builtin_huge_valf();
                        }
                    }
                    float cm = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                                     fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
                    cm = fmaxf(cm, __shfl_xor(cm, 16));
                    cm = fmaxf(cm, __shfl_xor(cm, 32));
                    const float mn = fmaxf(mrow[rg], cm);
                    const float alpha = __builtin_amdgcn_exp2f(mrow[rg] - mn);
                    mrow[rg] = mn;
                    lsum[rg] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < G::DT; ++dt) acc[rg][dt] *= alpha;
#pragma unroll
                    for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(t[i] - mn);
                }
                bf16x8 pk;
#pragma unroll
                for (int i = 0; i < 8; ++i) pk[i] = static_cast<__bf16>(pr[i]);
                // row sums of the bf16 weights actually used in p.v, on the matrix
                // unit: a ones "V^T" tile gives every output row the sum over keys
                lsum[rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pk, lsum[rg], 0, 0, 0);
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt)
                    acc[rg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pk, acc[rg][dt], 0, 0, 0);
            }
        }
    }

    template <int NG, bool ONLINE>
    static __device__ __forceinline__ void compute_stage(const char *stage, int valid_quarters,
                                                         const bf16x8 (&qf)[ar(NG)][G::DS], f32x4 (&acc)[ar(NG)][G::DT],
                                                         f32x4 (&lsum)[ar(NG)], float (&mrow)[ar(NG)],
                                                         const float (&brow)[ar(NG)], float c) {
        if (valid_quarters >= G::QUARTERS) {
#pragma unroll
            for (int sb = 0; sb < G::SUB; ++sb)
                compute_sub<NG, ONLINE, false>(stage + sb * G::SUB_BYTES, qf, acc, lsum, mrow, brow, c);
        } else {
#pragma unroll
            for (int sb = 0; sb < G::SUB; ++sb) {
                const int vq = valid_quarters - 2 * sb;
                if (vq >= 2)
                    compute_sub<NG, ONLINE, false>(stage + sb * G::SUB_BYTES, qf, acc, lsum, mrow, brow, c);
                else if (vq == 1)
                    compute_sub<NG, ONLINE, true>(stage + sb * G::SUB_BYTES, qf, acc, lsum, mrow, brow, c);
            }
        }
    }

    // The block-list walk: stages of KCH keys, double-buffered in LDS, the next
    // stage's global loads in flight while the current one is computed.
    template <int NG, bool ONLINE>
    static __device__ __forceinline__ void walk(const AttnParams &p, char *smem, const uint16_t *kh,
                                                const uint16_t *vh, int32_t e0, int32_t e1, int32_t nquart,
                                                const bf16x8 (&qf)[ar(NG)][G::DS], f32x4 (&acc)[ar(NG)][G::DT],
                                                f32x4 (&lsum)[ar(NG)], float (&mrow)[ar(NG)], const float (&brow)[ar(NG)]) {
        const int nst = (nquart + G::QUARTERS - 1) / G::QUARTERS;
        const int hpb = p.block_k / 16;
        const cint32 *col = (const cint32 *)(p.col_idx);
        Cursor cur{e0, 0};
        Stage st;
        const bool last_full = nquart % G::QUARTERS == 0;
        auto load = [&](int stage_idx, const Src &src) {
            if (stage_idx < nst - 1 || last_full)
                load_stage<true>(kh, vh, src, p.block_k, st);
            else
                load_stage<false>(kh, vh, src, p.block_k, st);
        };
        if (nst > 0) {
            load(0, next_src(col, cur, e1, hpb));
            store_stage(smem, st);
        }
        if (nst > 1) load(1, next_src(col, cur, e1, hpb));
        Src nxt = next_src(col, cur, e1, hpb);           // stage 2, fetched a stage early
        lds_barrier();
        for (int s = 0; s < nst - 1; ++s) {
            store_stage(smem + ((s + 1) & 1) * G::STAGE, st);
            if (s + 2 < nst) {
                load(s + 2, nxt);
                nxt = next_src(col, cur, e1, hpb);
            }
            compute_stage<NG, ONLINE>(smem + (s & 1) * G::STAGE, G::QUARTERS, qf, acc, lsum, mrow, brow, p.c);
            lds_barrier();
        }
        if (nst > 0)
            compute_stage<NG, ONLINE>(smem + ((nst - 1) & 1) * G::STAGE, nquart - (nst - 1) * G::QUARTERS,
                                      qf, acc, lsum, mrow, brow, p.c);
    }

    // NG valid row groups for this wavefront, starting at group my_g0 of the query block.
    template <int NG>
    static __device__ __forceinline__ void tile(const AttnParams &p, char *smem, int64_t head_row0,
                                                int32_t qb, int my_g0, const uint16_t *kh,
                                                const uint16_t *vh, int32_t e0, int32_t e1, int32_t nquart,
                                                bool online, float mk) {
        const int lane = threadIdx.x & 63;
        const int m = lane & 15, g = lane >> 4;
        // a wavefront without rows (NG == 0) still stages K/V and meets every barrier
        int rows[ar(NG)];
        bf16x8 qf[ar(NG)][G::DS];
        f32x4 acc[ar(NG)][G::DT];
        f32x4 lsum[ar(NG)];            // row sums (all four entries equal; see compute_sub)
        float mrow[ar(NG)], brow[ar(NG)];
#pragma unroll
        for (int rg = 0; rg < NG; ++rg) {
            rows[rg] = qb * p.block_q + (my_g0 + rg) * 16 + m;
            const uint16_t *qr = p.q + (head_row0 + rows[rg]) * D;
#pragma unroll
            for (int ds = 0; ds < G::DS; ++ds)
                qf[rg][ds] = *reinterpret_cast<const bf16x8 *>(qr + 32 * ds + 8 * g);
#pragma unroll
            for (int dt = 0; dt < G::DT; ++dt) acc[rg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            lsum[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
            mrow[rg] = -__builtin_huge_valf();
            brow[rg] = online ? 0.0f : p.c * p.qnorm[head_row0 + rows[rg]] * mk;
        }
        if (online)
            walk<NG, true>(p, smem, kh, vh, e0, e1, nquart, qf, acc, lsum, mrow, brow);
        else
            walk<NG, false>(p, smem, kh, vh, e0, e1, nquart, qf, acc, lsum, mrow, brow);
        if constexpr (NG > 0) {
            // epilogue: normalise by the row sum, bf16, store
#pragma unroll
            for (int rg = 0; rg < NG; ++rg) {
                const float inv = 1.0f / lsum[rg][0];
                uint16_t *orow = p.o + (head_row0 + rows[rg]) * D;
#pragma unroll
                for (int dt = 0; dt < G::DT; ++dt) {
                    __bf16 h4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) h4[i] = static_cast<__bf16>(acc[rg][dt][i] * inv);
                    uint2 w;
                    w.x = uint32_t(__builtin_bit_cast(uint16_t, h4[0])) |
                          (uint32_t(__builtin_bit_cast(uint16_t, h4[1])) << 16);
                    w.y = uint32_t(__builtin_bit_cast(uint16_t, h4[2])) |
                          (uint32_t(__builtin_bit_cast(uint16_t, h4[3])) << 16);
                    *reinterpret_cast<uint2 *>(orow + 16 * dt + 4 * g) = w;
                }
            }
        }
    }

    template <int NG>
    static __device__ __forceinline__ void dispatch(int ng, const AttnParams &p, char *smem, int64_t head_row0,
                                                    int32_t qb, int my_g0, const uint16_t *kh,
                                                    const uint16_t *vh, int32_t e0, int32_t e1, int32_t nquart,
                                                    bool online, float mk) {
        if constexpr (NG >= 0) {
            if (ng == NG)
                tile<NG>(p, smem, head_row0, qb, my_g0, kh, vh, e0, e1, nquart, online, mk);
            else
                dispatch<NG - 1>(ng, p, smem, head_row0, qb, my_g0, kh, vh, e0, e1, nquart, online, mk);
        }
    }

    static __device__ void run(const AttnParams &p) {
        extern __shared__ __attribute__((aligned(16))) char smem[];
        float *red = reinterpret_cast<float *>(smem + 2 * G::STAGE);
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

        // XCD-aware order: consecutive workgroup ids go to different XCDs, so
        // give each XCD a contiguous range of (head, query block) work.
        const int64_t bid = blockIdx.x;
        const int64_t L = (bid & 7) * p.per_xcd + (bid >> 3);
        if (L >= p.total_wg) return;
        const int64_t bh = L / p.n_qb;
        const int32_t qpf = p.tokens_per_frame / p.block_q;
        const int32_t qb = rank_to_qblock(int32_t(L % p.n_qb), p.frames, qpf);
        const int64_t hb = (bh / p.hc) * p.heads + p.h0 + bh % p.hc;
        const int64_t head_row0 = hb * p.seq_len;
        const uint16_t *kh = p.k + head_row0 * D;
        const uint16_t *vh = p.v + head_row0 * D;
        const int32_t e0 = p.row_ptr[qb], e1 = p.row_ptr[qb + 1];
        const int32_t nquart = (e1 - e0) * (p.block_k / 16);
        const bool online = p.eligible[hb] == 0;

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

        const int groups = p.block_q / 16;
        for (int sub = 0; sub < groups; sub += NW * RG) {
            // spread the sub-tile's groups over the wavefronts, RG at most each
            const int gsub = groups - sub < NW * RG ? groups - sub : NW * RG;
            const int base = gsub / NW, extra = gsub % NW;
            const int ng = base + (wave < extra ? 1 : 0);
            const int my_g0 = sub + wave * base + (wave < extra ? wave : extra);
            dispatch<RG>(ng, p, smem, head_row0, qb, my_g0, kh, vh, e0, e1, nquart, online, mk);
            if (sub + NW * RG < groups) lds_barrier();     // LDS reused by the next sub-tile
        }
    }
};

template <int D, int RG, int NW, int KCH, int WPE>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(WPE, WPE)))
attention_kernel(AttnParams p) {
    AttnKernel<D, RG, NW, KCH>::run(p);
}

}  // namespace

const char *hip_error_text(int code) { return hipGetErrorString(static_cast<hipError_t>(code)); }

int launch_bounds(const BoundsLaunch &a) {
    const fsa_plan_info &pl = *a.plan;
    hipStream_t stream = static_cast<hipStream_t>(a.stream);
    constexpr int QG = 2;
    NormsParams np;
    np.q = static_cast<const uint16_t *>(a.q);
    np.k = static_cast<const uint16_t *>(a.k);
    np.qnorm = a.qnorm;
    np.kmax = a.kmax;
    np.eligible = a.eligible;
    np.bmax = a.bmax;
    const int64_t nbh = int64_t(a.batch) * a.head_count;
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
    if (a.head_dim == 128)
        hipLaunchKernelGGL((norms_kernel<128, QG>), dim3(grid1), dim3(256), 0, stream, np);
    else
        hipLaunchKernelGGL((norms_kernel<64, QG>), dim3(grid1), dim3(256), 0, stream, np);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return int(err);

    ReduceParams rp;
    rp.qnorm = a.qnorm;
    rp.kmax = a.kmax;
    rp.row_ptr = a.row_ptr;
    rp.col_idx = a.col_idx;
    rp.eligible = a.eligible;
    rp.bmax = a.bmax;
    rp.heads = a.heads;
    rp.seq_len = pl.seq_len;
    rp.h0 = a.head_offset;
    rp.hc = a.head_count;
    rp.block_q = pl.block_q;
    rp.n_qb = pl.n_qblocks;
    rp.n_kb = pl.n_kblocks;
    rp.scale = a.scale;
    rp.limit = a.bound_limit;
    rp.chunks = (pl.n_qblocks + kReduceQB - 1) / kReduceQB;
    const unsigned grid2 = unsigned(nbh * rp.chunks);
    hipLaunchKernelGGL(bound_reduce_kernel, dim3(grid2), dim3(256), 0, stream, rp);
    err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

// Kernel configuration: 16-row groups per wavefront, wavefronts per workgroup,
// keys per LDS stage, wavefronts per SIMD.
template <int D, int RG, int NW, int KCH, int WPE>
int launch_cfg(const AttnParams &p, hipStream_t stream) {
    using K = AttnKernel<D, RG, NW, KCH>;
    auto fn = attention_kernel<D, RG, NW, KCH, WPE>;
    static bool attr_done = false;
    if (!attr_done) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS_BYTES);
        attr_done = true;
    }
    const unsigned grid = unsigned(p.per_xcd * 8);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * NW), K::LDS_BYTES, stream, p);
    const hipError_t err = hipGetLastError();
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
    if (a.head_dim == 128) return launch_cfg<128, FSA_RG, FSA_NW, FSA_KCH, FSA_WPE>(p, stream);
    return launch_cfg<64, FSA_RG, FSA_NW, FSA_KCH, FSA_WPE>(p, stream);
}

}  // namespace fsa
