// HIP kernel of fsa_pre_attention for AMD Instinct MI355X (gfx950, CDNA4).
//
// Source: aihot.vn, "HeyGen tối ưu hóa mô hình Avatar IV trên Google Cloud
// Trillium TPU", section "Bố cục là ABI" and Fig. 5: the chain that makes the
// attention inputs (normalisation, rotary embedding, projection, head packing)
// runs as one kernel whose output buffer is exactly the layout the next
// operation reads, so no repacking copies remain in between.
//
// One workgroup computes 256 tokens x 256 projected features (two head parts of
// q, k or v at D = 128, four at D = 64): Y^T = W' . x^T with bf16 MFMA 32x32x16
// over the channels (W' = the projection weight with the norm gain folded in).
// Eight wavefronts in a 4 x 2 grid, each owning 64 tokens x 128 features (128
// fp32 accumulators), two per SIMD.
// * staging: 64 channels (one 128-byte line per row) per stage, two stages in
//   LDS, filled by direct global-to-LDS buffer loads issued one stage ahead;
//   rows are stored with their 16-byte segments XOR-swizzled so that operand
//   reads are free of bank conflicts. Only waves 0-3 issue loads (all of the
//   next stage's at the start of a stage), so the other wavefront of each
//   SIMD never waits behind the texture unit and keeps the matrix core busy;
// * normalisation: each token's sum of squares is accumulated from the x
//   operand fragments with v_dot2 (bf16 pairs) by waves 4-7 (the waves that
//   issue no loads), and 1 / rms scales the fp32 result in the epilogue:
//   diag(r) (x W'^T) = (r x) W'^T;
// * rotary embedding (q and k): with the features as MFMA rows, features j and
//   j + D/2 of a token sit in the same lane and register (output tiles ot and
//   ot + D/64), so the rotation is lane-local. Angles are taken in revolutions
//   (the hardware sine and cosine take revolutions): position * f_j directly
//   for positions below 256, otherwise from an fp64 table entry for the tile's
//   first position plus the row offset;
// * head packing: the finished tile is parked in LDS and stored as whole
//   token rows of each head part (16 bytes per lane, coalesced) into q, k or v
//   [B, H, N, D].
// Workgroups are ordered so that the feature tiles of one token tile run on the
// same XCD (consecutive workgroup ids go to different XCDs), where they share
// the x tile in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fsa_internal.h"

namespace fsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct PreParams {
    const uint16_t *x, *w;
    uint16_t *q, *k, *v;
    int64_t tokens, total_wg, per_xcd;
    int32_t seq_len, channels, heads, ftiles;
    float eps, rope_base;
};

typedef __attribute__((address_space(3))) void lds_void;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to bf16 (round to nearest even) in one register, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Buffer descriptor over `bytes` bytes at `base` (raw, 32-bit data; accesses at
// or past `bytes` read zeros), in scalar registers.
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(uint32_t(b));
    r[1] = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32) & 0xffffu);
    r[2] = uint32_t(bytes > int64_t(0xffffffff) ? int64_t(0xffffffff) : bytes);
    r[3] = 0x00020000u;
    return r;
}

// 16 bytes per lane from the buffer at byte offset voff straight into LDS at
// lds_addr + 16 * lane. Written as an instruction of its own (the asm owns M0)
// so that the compiler does not wait for it before unrelated LDS reads; the
// stage barrier waits for it explicitly.
__device__ __forceinline__ void load_lds16(u32x4 rs, uint32_t lds_addr, int32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

// Barrier for a stage hand-off: this wave's direct-to-LDS loads (counted as
// vector memory operations) and LDS accesses are complete, then s_barrier.
__device__ __forceinline__ void stage_sync() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((0) | (0 << 14) | (7 << 4) | (0 << 8));     // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate: at most `vm` vector memory operations outstanding, no
// LDS operation outstanding (vmcnt in bits 3:0 and 15:14, lgkmcnt in 11:8).
constexpr int wait_vm_lgkm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (0 << 8); }

template <int D>
struct PreAttn {
    static constexpr int TM = 256;                // tokens per workgroup
    static constexpr int TN = 256;                // projected features per workgroup (256 / D head parts)
    static constexpr int THREADS = 512;           // 4 x 2 wavefronts of 64 tokens x 128 features
    static constexpr int KC = 64;                 // channels per stage: one 128-byte line per row
    // A stage holds x rows [256][128 B] then weight rows [256][128 B]. Within a
    // row the eight 16-byte segments are stored at slot seg ^ ((row / 2) % 8),
    // so an operand read of 16 consecutive rows covers all 64 banks once.
    static constexpr int ROWB = KC * 2;
    static constexpr int STAGE = (TM + TN) * ROWB;
    // write-out: per wave 64 token rows of 128 bf16 features, 16-byte pad per row
    static constexpr int OUT_ROW = 128 * 2 + 16;
    static constexpr int OUT_WAVE = 64 * OUT_ROW;
    static constexpr int MAIN_BYTES = 2 * STAGE > 8 * OUT_WAVE ? 2 * STAGE : 8 * OUT_WAVE;
    static constexpr int LDS_BYTES = MAIN_BYTES + TM * 4 + (D / 2) * 8 + TM * 8;

    static __device__ __forceinline__ int slot(int row, int seg) { return seg ^ ((row >> 1) & 7); }

    // Direct-to-LDS loads of a stage: each 1 KB load instruction fills 8 rows;
    // lane l loads segment slot(row, l % 8) of row l / 8 into slot l % 8, so
    // every 8 lanes read one whole 128-byte line. Waves 0-3 load everything:
    // wave w the x and weight rows of row groups w and w + 4 (rows 32 g .. 32 g
    // + 31 of group g), quarter q of a group being its rows 8 q .. 8 q + 7.
    // Rows past the last token or projected feature lie past the end of their
    // buffer and read zeros; a last stage that is half empty (C an odd multiple
    // of 32) reads the next row's channels there, zeroed in LDS before use.
    struct Loads {
        u32x4 xr, wr;               // x rows m0.., weight rows f0..
        uint32_t lds;               // LDS address of the stage buffers
        int32_t off[2][4];          // per-lane byte offsets of (group, quarter) in x and w
    };
    static __device__ __forceinline__ Loads make_loads(const PreParams &p, const char *smem, int64_t m0, int32_t f0) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        Loads l;
        l.xr = buffer_rsrc(p.x + m0 * p.channels, (p.tokens - m0) * p.channels * 2);
        l.wr = buffer_rsrc(p.w + int64_t(f0) * p.channels, int64_t(3 * p.heads * D - f0) * p.channels * 2);
        l.lds = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((const lds_void *)smem)));
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = 32 * ((wave & 3) + 4 * g) + 8 * q + lane / 8;
                l.off[g][q] = row * p.channels * 2 + slot(row, lane % 8) * 16;
            }
        return l;
    }
    // Quarter q of both row groups of this wave, channels k0.. of the stage in
    // LDS buffer `b`.
    static __device__ __forceinline__ void load_quarter(const Loads &l, int b, int32_t k0, int q) {
        const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint32_t dst = l.lds + uint32_t(b * STAGE) + (32 * ((wave & 3) + 4 * g) + 8 * q) * ROWB;
            load_lds16(l.xr, dst, l.off[g][q] + 2 * k0);
            load_lds16(l.wr, dst + TM * ROWB, l.off[g][q] + 2 * k0);
        }
    }

    struct Frags { bf16x8 w[4], x[2]; };

    // Operand fragments of one 16-channel step: weight rows 128 pp + 32 ot + n
    // and x rows 64 th + 32 tt + n, channels 16 ks + 8 h .. + 7.
    static __device__ __forceinline__ void read_frags(const char *buf, int ks, Frags &f) {
        const int lane = threadIdx.x & 63, n = lane & 31, h = lane >> 5, wave = threadIdx.x >> 6;
        const int th = wave & 3, pp = wave >> 2;
        const int so = slot(n, 2 * ks + h) * 16;            // rows start at multiples of 32
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
            f.w[ot] = *reinterpret_cast<const bf16x8 *>(buf + (TM + 128 * pp + 32 * ot + n) * ROWB + so);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            f.x[tt] = *reinterpret_cast<const bf16x8 *>(buf + (64 * th + 32 * tt + n) * ROWB + so);
    }

    // One 16-channel step: 4 x 2 MFMA tiles of 32 x 32 and, with SQ (waves
    // 4-7, which issue no loads), the squares of the tokens' channels.
    template <bool SQ>
    static __device__ __forceinline__ void step(const Frags &f, f32x16 (&acc)[4][2], float (&ss)[2]) {
#pragma unroll
        for (int tt = 0; tt < 2 && SQ; ++tt) {
            const bf16x2 p0 = __builtin_shufflevector(f.x[tt], f.x[tt], 0, 1);
            const bf16x2 p1 = __builtin_shufflevector(f.x[tt], f.x[tt], 2, 3);
            const bf16x2 p2 = __builtin_shufflevector(f.x[tt], f.x[tt], 4, 5);
            const bf16x2 p3 = __builtin_shufflevector(f.x[tt], f.x[tt], 6, 7);
            ss[tt] = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, ss[tt], false);
            ss[tt] = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, ss[tt], false);
            ss[tt] = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, ss[tt], false);
            ss[tt] = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, ss[tt], false);
        }
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                acc[ot][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[ot], f.x[tt], acc[ot][tt], 0, 0, 0);
    }

    // The four steps of a stage, each step's fragments read while the step
    // before it is multiplied. With LOAD (waves 0-3 of a stage that has a
    // successor), all of the next stage's loads go out first, so they have
    // the whole stage to land.
    template <bool LOAD, bool SQ>
    static __device__ __forceinline__ void compute(const char *buf, f32x16 (&acc)[4][2], float (&ss)[2],
                                                   const Loads &l, int nb, int32_t k0) {
        Frags fa, fb;
        read_frags(buf, 0, fa);
        read_frags(buf, 1, fb);
        if (LOAD) {
#pragma unroll
            for (int q = 0; q < 4; ++q) load_quarter(l, nb, k0, q);
        }
        step<SQ>(fa, acc, ss);
        read_frags(buf, 2, fa);
        step<SQ>(fb, acc, ss);
        read_frags(buf, 3, fb);
        step<SQ>(fa, acc, ss);
        step<SQ>(fb, acc, ss);
    }

    // Every stage; LOADER (waves 0-3): this wave issues the loads, the others
    // (waves 4-7) take the squares. One instantiation per role, the last
    // stage included, so that the register allocation of each is one piece.
    template <bool LOADER>
    static __device__ __forceinline__ void main_loop(char *smem, f32x16 (&acc)[4][2], float (&ss)[2], const Loads &l,
                                                     int stages, int channels) {
        for (int st = 0; st + 1 < stages; ++st) {
            compute<LOADER, !LOADER>(smem + (st & 1) * STAGE, acc, ss, l, (st + 1) & 1, KC * (st + 1));
            stage_sync();
        }
        const int st = stages - 1;
        char *buf = smem + (st & 1) * STAGE;
        if (channels % KC != 0) {
            // channels past C in the last stage: zero them in the x rows so
            // they add nothing to the products or the squares
            const int t = threadIdx.x;
            if (t < TM) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4 *>(buf + t * ROWB + slot(t, 4 + i) * 16) = u32x4{};
            }
            stage_sync();
        }
        compute<false, !LOADER>(buf, acc, ss, l, 0, 0);
        stage_sync();
    }

    static __device__ void run(const PreParams &p) {
        __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
        float *rs = reinterpret_cast<float *>(smem + MAIN_BYTES);
        float2 *rot = reinterpret_cast<float2 *>(smem + MAIN_BYTES + TM * 4);
        int64_t *rowoff = reinterpret_cast<int64_t *>(smem + MAIN_BYTES + TM * 4 + (D / 2) * 8);

        const int64_t bid = blockIdx.x;
        const int64_t L = (bid & 7) * p.per_xcd + (bid >> 3);
        if (L >= p.total_wg) return;
        const int64_t m0 = (L / p.ftiles) * TM;
        const int32_t f0 = int32_t(L % p.ftiles) * TN;
        const int64_t b0 = m0 / p.seq_len;
        const int32_t pos0 = int32_t(m0 - b0 * p.seq_len);
        const int t = threadIdx.x;
        const int lane = t & 63, n = lane & 31, h = lane >> 5, wave = t >> 6;
        const int th = wave & 3, pp = wave >> 2;

        // Rotation pair j turns by pos * f_j revolutions, f_j = base^(-2j/D) / (2 pi).
        // Table: (f_j, frac(pos0 * f_j)) for the tile's first position pos0, the
        // latter in fp64 so that large positions keep their precision.
        if (t < D / 2) {
            const double f = exp2(-(2.0 * t / D) * log2(double(p.rope_base))) * (0.5 / M_PI);
            const double u = double(pos0) * f;
            rot[t] = make_float2(float(f), float(u - floor(u)));
        }
        // Output token of each tile row, b N H + n for sequence b and position n
        // (the tile may cross sequence ends), -1 past the last token: one
        // division per row here instead of one per row and store later.
        if (t < TM) {
            const uint32_t pf = uint32_t(pos0) + uint32_t(t);
            const uint32_t wraps = pf / uint32_t(p.seq_len);
            rowoff[t] = m0 + t < p.tokens
                            ? (b0 + wraps) * p.heads * int64_t(p.seq_len) + (pf - wraps * uint32_t(p.seq_len))
                            : int64_t(-1);
        }

        f32x16 acc[4][2];
#pragma unroll
        for (int ot = 0; ot < 4; ++ot) acc[ot][0] = acc[ot][1] = f32x16{};
        float ss[2] = {0.0f, 0.0f};
        // Stage k (64 channels) goes through LDS buffer k % 2; its loads are
        // issued while stage k - 1 is multiplied.
        const int stages = (p.channels + KC - 1) / KC;
        const Loads l = make_loads(p, smem, m0, f0);
        const bool loader = __builtin_amdgcn_readfirstlane(wave) < 4;
        if (loader) {
#pragma unroll
            for (int q = 0; q < 4; ++q) load_quarter(l, 0, 0, q);
        }
        stage_sync();
        if (loader) main_loop<true>(smem, acc, ss, l, stages, p.channels);
        else main_loop<false>(smem, acc, ss, l, stages, p.channels);

        // 1 / rms per token, from the pp = 1 waves (waves 4-7, which took the
        // squares; the two halves of a wave hold disjoint channel halves of
        // each token)
        if (pp == 1) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const float sq = ss[tt] + __shfl_xor(ss[tt], 32);
                if (h == 0) rs[64 * th + 32 * tt + n] = 1.0f / sqrtf(sq / float(p.channels) + p.eps);
            }
        }
        stage_sync();

        // Token of lane row 128 th + 32 tt + n: sequence b0 + wraps, position
        // pos0 + row - wraps N (the tile may cross sequence ends).
        int32_t pos[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int row = 64 * th + 32 * tt + n;
            const uint32_t pf = uint32_t(pos0) + uint32_t(row);
            const uint32_t wraps = pf / uint32_t(p.seq_len);
            pos[tt] = int32_t(pf - wraps * uint32_t(p.seq_len));
            const float r = rs[row];
#pragma unroll
            for (int ot = 0; ot < 4; ++ot) acc[ot][tt] *= r;
        }

        // Feature tile ot covers features f0 + 128 pp + 32 ot + (0..31), all of
        // head part (f0 + 128 pp + 32 ot) / D (the wave's 128 features start on
        // a part boundary). The tiles holding first halves of a part are ot = q
        // (D = 128) or ot = 2 q (D = 64); the partner is tile ot + D / 64.
        // A position below 256 is turned directly (pos * f_j < 41 revolutions
        // keeps fp32 precise); a larger one lies in the tile's first sequence at
        // pos0 + row and starts from the fp64 table entry.
        constexpr int PAIR = D / 64;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int ot = D == 128 ? qq : 2 * qq;
            const int32_t fbase = f0 + 128 * pp + 32 * ot;
            if (fbase / D >= 2 * p.heads) continue;         // v (or past the last part): not rotated
            const int jt = fbase % D;                        // 0 or 32
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float2 fr = rot[jt + 8 * (i / 4) + 4 * h + (i % 4)];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    const bool near = pos[tt] < 256;
                    const float u = near ? float(pos[tt]) * fr.x
                                         : fmaf(float(64 * th + 32 * tt + n), fr.x, fr.y);
                    const float uf = u - floorf(u);
                    const float sn = __builtin_amdgcn_sinf(uf), cs = __builtin_amdgcn_cosf(uf);
                    const float lo = acc[ot][tt][i], hi = acc[ot + PAIR][tt][i];
                    acc[ot][tt][i] = lo * cs - hi * sn;
                    acc[ot + PAIR][tt][i] = hi * cs + lo * sn;
                }
            }
        }

        // Write-out through LDS: each wave parks its 64 tokens x 128 features as
        // bf16 rows of 256 B (plus a 16-byte pad) in the free stage buffers,
        // then stores whole token rows of each head part with 16-byte lanes.
        stage_sync();                                       // every wave is done with the stage buffers
        char *park = smem + wave * OUT_WAVE;
#pragma unroll
        for (int ot = 0; ot < 4; ++ot)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    uint2 w;
                    w.x = pack_bf16(acc[ot][tt][4 * a], acc[ot][tt][4 * a + 1]);
                    w.y = pack_bf16(acc[ot][tt][4 * a + 2], acc[ot][tt][4 * a + 3]);
                    *reinterpret_cast<uint2 *>(park + (32 * tt + n) * OUT_ROW + (32 * ot + 8 * a + 4 * h) * 2) = w;
                }
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm(63));      // this wave's parked rows are in LDS
        __builtin_amdgcn_wave_barrier();
        const int32_t nparts = 3 * p.heads;
        constexpr int LPR = D / 8;                          // lanes per token row of one head part
        constexpr int RPI = 64 / LPR;                       // token rows per store instruction
        constexpr int NJ = 64 / RPI;                        // store instructions per head part
#pragma unroll
        for (int part_i = 0; part_i < 128 / D; ++part_i) {
            const int32_t fbase = f0 + 128 * pp + D * part_i;
            const int32_t part = fbase / D;
            if (part >= nparts) continue;
            const int qkv = part / p.heads, head = part % p.heads;
            uint16_t *out = (qkv == 0 ? p.q : (qkv == 1 ? p.k : p.v)) + int64_t(head) * p.seq_len * D;
            // all of the part's LDS reads first, then the stores (one wait)
            u32x4 v[NJ];
            int64_t tok[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rw = RPI * j + lane / LPR;         // the wave's token row
                tok[j] = rowoff[64 * th + rw];
                v[j] = *reinterpret_cast<const u32x4 *>(park + rw * OUT_ROW + (D * part_i + 8 * (lane % LPR)) * 2);
            }
            // streaming stores: the outputs are not read again by this kernel;
            // only the last token tile has rows past the end
            if (m0 + TM <= p.tokens) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4 *>(out + tok[j] * D + 8 * (lane % LPR)));
            } else {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    if (tok[j] >= 0)
                        __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4 *>(out + tok[j] * D + 8 * (lane % LPR)));
            }
        }
    }
};

template <int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
pre_attention_kernel(PreParams p) {
    PreAttn<D>::run(p);
}

}  // namespace

// One launch: 8 * ceil(work / 8) workgroups (ids remapped XCD-first inside the
// kernel; ids past the work return at once), 512 threads, about 141 KB of
// static LDS (one workgroup per CU).
int launch_pre_attention(const PreAttentionLaunch &a) {
    PreParams p;
    p.x = static_cast<const uint16_t *>(a.x);
    p.w = static_cast<const uint16_t *>(a.w_qkv);
    p.q = static_cast<uint16_t *>(a.q);
    p.k = static_cast<uint16_t *>(a.k);
    p.v = static_cast<uint16_t *>(a.v);
    p.tokens = int64_t(a.batch) * a.seq_len;
    p.seq_len = a.seq_len;
    p.channels = a.channels;
    p.heads = a.heads;
    p.ftiles = (3 * a.heads * a.head_dim + 255) / 256;   // feature tiles of 256
    p.eps = a.eps;
    p.rope_base = a.rope_base;
    p.total_wg = ((p.tokens + 255) / 256) * p.ftiles;
    p.per_xcd = (p.total_wg + 7) / 8;
    hipStream_t stream = static_cast<hipStream_t>(a.stream);
    const unsigned grid = unsigned(p.per_xcd * 8);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(pre_attention_kernel<128>, dim3(grid), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL(pre_attention_kernel<64>, dim3(grid), dim3(512), 0, stream, p);
    const hipError_t err = hipGetLastError();
    return err == hipSuccess ? 0 : int(err);
}

}  // namespace fsa
