// Chunked gated delta rule for gfx950: one fused kernel over 64-token chunks (WY/UT form).
//
// Two kernels: chunk_flow_kernel (below, near the end) for bf16 I/O with the scalar gate at K = V = 128,
// which solves v_new from the state and overlaps the state-dependent step of one chunk with the
// state-independent steps of the next, and chunk_fused_kernel for every other configuration,
// described here.
//
// One workgroup owns the whole state S[V][K] of one (sequence, value head) -- or a 64-wide
// V tile of it -- and walks the sequence's chunks in order.  Wave w keeps the 16 state
// columns v = 16*w + lane%16 of its tile in MFMA accumulators for the whole sequence.
// Per chunk (rows r = 0..63 from the chunk start, the last chunk of a sequence may be
// short; rows past its end are zero):
//
//   A  raw q, k (and v) rows into LDS; gamma = chunk-local prefix sum of the log-decay
//   B  L = strictly lower  beta_r (k_r . k_j) e^{gamma_r - gamma_j}      (K K^T on MFMA)
//      P = lower incl. diag  (q_r . k_j) e^{gamma_r - gamma_j}           (Q K^T on MFMA)
//   C  D_I = (I + L_II)^-1 for the four 16x16 diagonal blocks (fp32 substitution)
//   D  [W | U] = (I + L)^-1 [diag(beta e^gamma) K | diag(beta) V] by blocked forward
//      substitution X_I = D_I (B_I - sum_{J<I} L_IJ X_J) on MFMA;
//      -W -> LDS, U -> the registers of the wave owning those value columns
//   E  v_new = U - W S^T;  O = scale (diag(e^gamma) Q S^T + P v_new);
//      S <- e^{gamma_last} S + sum_r v_new_r (k_r * e^{gamma_last - gamma_r})^T
//
// This is the chunked algorithm whose parts (cumulative gate, kkt/solve/A, w, u, the
// inter-chunk recurrence with per-chunk h and v_new, the chunk output) the cuLA PR #113
// "[GDN2] Add Hopper SM90 CuTe DSL prefill" and attention-gym PR #344 "Replace the KDA
// inter-chunk recurrence with a warp-specialized kernel" pages build on, derived here from the
// token recurrence.  Stages B-D are the intra-chunk WY/UT transform, the S-dependent part of E
// is the inter-chunk state pass and the rest of E is the chunk output; fusing them keeps W, U,
// v_new and the per-chunk states out of HBM, which then only sees q, k, v, g, beta, o and
// the initial/final states.  The next chunk's inputs are loaded into registers while the
// current chunk computes.
//
// Overflow: every exponential evaluated has a non-positive argument -- a prefix gamma or a
// (later - earlier) prefix difference -- so no exp(-prefix) factor is ever formed (cuLA PR
// #113 review, finding P1).  With the scalar gate the decays are applied as row factors of
// MFMA inputs/outputs.  With the per-key-channel gate they cannot be factored out of K K^T
// and Q K^T: off-diagonal 16x16 blocks use a reference point rho (the prefix at the last
// row before the block row), exp(g_r - g_j) = exp(g_r - rho) exp(rho - g_j) with both
// factors <= 1, and the four diagonal blocks are evaluated element-wise.
//
// MFMA: bf16 I/O uses v_mfma_f32_16x16x32_bf16 for the products over K and the chunk, and
// v_mfma_f32_16x16x16_bf16 for the blocked substitution (bf16 operands, fp32 accumulation);
// fp32 I/O uses v_mfma_f32_16x16x4f32 throughout.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int CH = 64;  // chunk length

#ifdef GDR_FLOW_STAMPS
// Measurement build only (libgdr_stamps.so, never libgdr.so): shader-clock counters of the flow kernel.
//   g_flow_stamps[role][iteration][slot]: lane 0 of wave 0 (role 0, state) and of wave 4 (role 1, prep)
//     of the workgroup (sequence g_flow_target[0], head g_flow_target[1]), at the phase boundaries
//     and inside the phases (slots listed where they are taken);
//   g_flow_wg[sequence][head]: thread 0 of every workgroup, shader clock and 100 MHz real-time clock
//     at entry and after the state waves' last iteration.
constexpr int kStampIters = 128, kStampSeqs = 8, kStampHeads = 32;
__device__ unsigned long long g_flow_stamps[2][kStampIters][8];
__device__ unsigned long long g_flow_wg[kStampSeqs][kStampHeads][4];
__device__ int g_flow_target[2];
#define FLOW_STAMP(rec, role, it, slot)                                                                   \
    do {                                                                                                  \
        if ((rec) && (it) < kStampIters) g_flow_stamps[role][it][slot] = __builtin_amdgcn_s_memtime();    \
    } while (0)
#define FLOW_WG_CLOCK(first)                                                                              \
    do {                                                                                                  \
        if (threadIdx.x == 0 && blockIdx.z < kStampSeqs && blockIdx.y < kStampHeads) {                    \
            g_flow_wg[blockIdx.z][blockIdx.y][(first) ? 0 : 2] = __builtin_amdgcn_s_memtime();            \
            g_flow_wg[blockIdx.z][blockIdx.y][(first) ? 1 : 3] = __builtin_amdgcn_s_memrealtime();        \
        }                                                                                                 \
    } while (0)
#else
#define FLOW_STAMP(rec, role, it, slot) \
    do {                                \
    } while (0)
#define FLOW_WG_CLOCK(first) \
    do {                     \
    } while (0)
#endif

// ---------------------------------------------------------------------------
// MFMA tile products on LDS operands, "NT" form: C[i][j] += sum_k A[i][k] * Bt[j][k]
// with A and Bt both row-major over the reduction index.  sA / sB point at the first
// row of the 16-row tile.  C layout: lane l holds C[4*(l/16) + e][l%16], e = 0..3.
template <typename MT> struct MM;

template <> struct MM<bf16_t> {
    typedef uint16_t S;  // LDS element
    // rows padded to a stride of 8 dwords modulo 32 banks: the 16-row MFMA operand reads (16-byte
    // lanes, rows l % 16, column granules l / 16) are then free of bank conflicts
    static constexpr int PAD = 16;
    __device__ __forceinline__ static S cvt(float x) { return f32_to_bf16(x); }
    __device__ __forceinline__ static float back(S x) { return bf16_to_f32(x); }
    __device__ __forceinline__ static void nt(f32x4_t& acc, const S* sA, int lda, const S* sB, int ldb, int kdim) {
        const int l = threadIdx.x & 63;
        const S* pa = sA + (l & 15) * lda + 8 * (l >> 4);
        const S* pb = sB + (l & 15) * ldb + 8 * (l >> 4);
        for (int k0 = 0; k0 < kdim; k0 += 32) {
            bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(pa + k0);
            bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(pb + k0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
        }
    }
    // two independent tiles: every operand read is issued before the first product
    template <int KD>
    __device__ __forceinline__ static void nt2(f32x4_t& c0, const S* a0, const S* b0, f32x4_t& c1, const S* a1,
                                               const S* b1, int ld) {
        const int l = threadIdx.x & 63, o = (l & 15) * ld + 8 * (l >> 4);
        bf16x8_t va0[KD / 32], vb0[KD / 32], va1[KD / 32], vb1[KD / 32];
#pragma unroll
        for (int s = 0; s < KD / 32; ++s) {
            va0[s] = *reinterpret_cast<const bf16x8_t*>(a0 + o + 32 * s);
            vb0[s] = *reinterpret_cast<const bf16x8_t*>(b0 + o + 32 * s);
            va1[s] = *reinterpret_cast<const bf16x8_t*>(a1 + o + 32 * s);
            vb1[s] = *reinterpret_cast<const bf16x8_t*>(b1 + o + 32 * s);
        }
#pragma unroll
        for (int s = 0; s < KD / 32; ++s) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va0[s], vb0[s], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va1[s], vb1[s], c1, 0, 0, 0);
        }
    }
    // store 8 floats (row-contiguous) into LDS
    __device__ __forceinline__ static void st8(S* p, const float* x) {
        uint4 w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        w.z = pack_bf16x2(x[4], x[5]);
        w.w = pack_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(p) = w;
    }
};

template <> struct MM<float> {
    typedef float S;
    static constexpr int PAD = 4;
    __device__ __forceinline__ static S cvt(float x) { return x; }
    __device__ __forceinline__ static float back(S x) { return x; }
    __device__ __forceinline__ static void nt(f32x4_t& acc, const S* sA, int lda, const S* sB, int ldb, int kdim) {
        const int l = threadIdx.x & 63;
        const S* pa = sA + (l & 15) * lda + (l >> 4);
        const S* pb = sB + (l & 15) * ldb + (l >> 4);
        for (int k0 = 0; k0 < kdim; k0 += 4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0], pb[k0], acc, 0, 0, 0);
    }
    template <int KD>
    __device__ __forceinline__ static void nt2(f32x4_t& c0, const S* a0, const S* b0, f32x4_t& c1, const S* a1,
                                               const S* b1, int ld) {
        const int l = threadIdx.x & 63, o = (l & 15) * ld + (l >> 4);
        float va0[KD / 4], vb0[KD / 4], va1[KD / 4], vb1[KD / 4];
#pragma unroll
        for (int s = 0; s < KD / 4; ++s) {
            va0[s] = a0[o + 4 * s];
            vb0[s] = b0[o + 4 * s];
            va1[s] = a1[o + 4 * s];
            vb1[s] = b1[o + 4 * s];
        }
#pragma unroll
        for (int s = 0; s < KD / 4; ++s) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(va0[s], vb0[s], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(va1[s], vb1[s], c1, 0, 0, 0);
        }
    }
    __device__ __forceinline__ static void st8(S* p, const float* x) {
        f32x4_t* q = reinterpret_cast<f32x4_t*>(p);
        q[0] = f32x4_t{x[0], x[1], x[2], x[3]};
        q[1] = f32x4_t{x[4], x[5], x[6], x[7]};
    }
};

// Column order inside every 32-wide block of a bf16 LDS operand row: logical column
// c = 32m + 16h + 4g + e is stored at 32m + 8g + 4h + e.  An MFMA lane group then finds the
// two 4-element runs it needs (below) in one 16-byte read.  fp32 layouts keep natural order.
template <typename MT>
__device__ __forceinline__ int perm(int c) {
    if constexpr (sizeof(typename MM<MT>::S) == 2)
        return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
    else
        return c;
}

// Logical column of physical column p (the inverse of perm).
template <typename MT>
__device__ __forceinline__ int iperm(int p) {
    if constexpr (sizeof(typename MM<MT>::S) == 2)
        return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
    else
        return p;
}

// c0 += A0 B'^T and c1 += A1 B'^T over KD columns (16-row tiles from LDS, as MM::nt), where B'
// is B with every column multiplied by f[column] (fp32, physical column order; NULL: none).  The
// two products share the scaled B operand, and every operand read is issued before the first
// product.  With TWO = false only c0 is formed (a1 is not read).  With TR the products are formed
// transposed (B' A^T): lane (g, i) then holds row i of A's tile, columns 4g .. 4g+3 of B's.
template <typename MT, int KD, bool TWO = true, bool TR = false>
__device__ __forceinline__ void nt2_bscaled(f32x4_t& c0, const typename MM<MT>::S* a0, f32x4_t& c1,
                                            const typename MM<MT>::S* a1, int lda, const typename MM<MT>::S* b,
                                            int ldb, const float* f) {
    const int l = threadIdx.x & 63;
    if constexpr (sizeof(typename MM<MT>::S) == 2) {
        // in halves of at most 64 columns: the operands of one half are in flight at a time, which
        // bounds the registers this needs inside a kernel that holds its state in registers
        constexpr int NS = KD > 64 ? 2 : KD / 32;
        const int oa = (l & 15) * lda + 8 * (l >> 4), ob = (l & 15) * ldb + 8 * (l >> 4), of = 8 * (l >> 4);
#pragma unroll
        for (int h0 = 0; h0 < KD; h0 += 32 * NS) {
        bf16x8_t va0[NS], va1[NS];
        uint4 vb[NS];
        f32x4_t f0[NS], f1[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            va0[s] = *reinterpret_cast<const bf16x8_t*>(a0 + oa + h0 + 32 * s);
            if constexpr (TWO) va1[s] = *reinterpret_cast<const bf16x8_t*>(a1 + oa + h0 + 32 * s);
            vb[s] = *reinterpret_cast<const uint4*>(b + ob + h0 + 32 * s);
            if (f) {
                f0[s] = *reinterpret_cast<const f32x4_t*>(f + of + h0 + 32 * s);
                f1[s] = *reinterpret_cast<const f32x4_t*>(f + of + h0 + 32 * s + 4);
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 w = vb[s];
            if (f) {
                w.x = pack_bf16x2(__uint_as_float(w.x << 16) * f0[s][0], __uint_as_float(w.x & 0xFFFF0000u) * f0[s][1]);
                w.y = pack_bf16x2(__uint_as_float(w.y << 16) * f0[s][2], __uint_as_float(w.y & 0xFFFF0000u) * f0[s][3]);
                w.z = pack_bf16x2(__uint_as_float(w.z << 16) * f1[s][0], __uint_as_float(w.z & 0xFFFF0000u) * f1[s][1]);
                w.w = pack_bf16x2(__uint_as_float(w.w << 16) * f1[s][2], __uint_as_float(w.w & 0xFFFF0000u) * f1[s][3]);
            }
            const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, w);
            if constexpr (TR) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, va0[s], c0, 0, 0, 0);
                if constexpr (TWO) c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, va1[s], c1, 0, 0, 0);
            } else {
                c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va0[s], bv, c0, 0, 0, 0);
                if constexpr (TWO) c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va1[s], bv, c1, 0, 0, 0);
            }
        }
        }
    } else {
        constexpr int NS = KD / 4;
        const int oa = (l & 15) * lda + (l >> 4), ob = (l & 15) * ldb + (l >> 4);
        float va0[NS], va1[NS], vb[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            va0[s] = a0[oa + 4 * s];
            if constexpr (TWO) va1[s] = a1[oa + 4 * s];
            vb[s] = f ? b[ob + 4 * s] * f[4 * s + (l >> 4)] : b[ob + 4 * s];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if constexpr (TR) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(vb[s], va0[s], c0, 0, 0, 0);
                if constexpr (TWO) c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(vb[s], va1[s], c1, 0, 0, 0);
            } else {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(va0[s], vb[s], c0, 0, 0, 0);
                if constexpr (TWO) c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(va1[s], vb[s], c1, 0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ uint32_t pack_tile_lo(const f32x4_t& t) { return pack_bf16x2(t[0], t[1]); }
__device__ __forceinline__ uint32_t pack_tile_hi(const f32x4_t& t) { return pack_bf16x2(t[2], t[3]); }

// acc[i] += A[16*i + .., :] B, where B (NP x 16, one column per lane%16) is given as NP/16
// accumulator tiles Bt[p/16] (lane l holds B[16*t + 4*(l/16) + e][l%16] in Bt[t][e]), i.e.
// the state or v_new straight from registers.  The reduction index is visited in the order
// the tiles provide it: for a 32-wide bf16 step m, MFMA position 8*(l/16) + e is index
// 32m + 4*(l/16) + e (e < 4) or 32m + 16 + 4*(l/16) + e - 4 (e >= 4) -- one 16-byte read of a
// perm()-ordered A row; for an fp32 step (t, e) position l/16 is index 16t + 4*(l/16) + e.
// With LOWER, A is lower triangular (A[r][j] = 0 for j > r): reduction steps entirely above the
// diagonal of a 16-row tile are skipped.  The A reads of two k-steps are issued together, before
// their products.  With TR the tiles are formed transposed (lane (g, i) holds row 16*tile + i,
// columns 4g .. 4g+3 of B's 16).
template <typename MT, int NP, int NI, bool LOWER = false, bool TR = false>
__device__ __forceinline__ void gemm_regs(f32x4_t* acc, const typename MM<MT>::S* sA, int lda, const f32x4_t* Bt) {
    const int l = threadIdx.x & 63, g4 = l >> 4, lr = l & 15;
    if constexpr (sizeof(typename MM<MT>::S) == 2) {
        constexpr int MS = NP / 32, G = MS < 2 ? MS : 2;
#pragma unroll
        for (int m0 = 0; m0 < MS; m0 += G) {
            bf16x8_t av[G][NI];
#pragma unroll
            for (int m = 0; m < G; ++m)
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    if (!(LOWER && 32 * (m0 + m) > 16 * i + 15))
                        av[m][i] = *reinterpret_cast<const bf16x8_t*>(sA + (16 * i + lr) * lda + 32 * (m0 + m) + 8 * g4);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < G; ++m) {
                const uint4 bw = {pack_tile_lo(Bt[2 * (m0 + m)]), pack_tile_hi(Bt[2 * (m0 + m)]),
                                  pack_tile_lo(Bt[2 * (m0 + m) + 1]), pack_tile_hi(Bt[2 * (m0 + m) + 1])};
                const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    if (LOWER && 32 * (m0 + m) > 16 * i + 15) continue;
                    if constexpr (TR) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, av[m][i], acc[i], 0, 0, 0);
                    else acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m][i], bv, acc[i], 0, 0, 0);
                }
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < NP / 16; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    if (LOWER && t > i) continue;
                    const float av = sA[(16 * i + lr) * lda + 16 * t + 4 * g4 + e];
                    if constexpr (TR) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(Bt[t][e], av, acc[i], 0, 0, 0);
                    else acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, Bt[t][e], acc[i], 0, 0, 0);
                }
            }
        }
    }
}

// acc0[i] += A[16*i + .., :] B0 and acc1[i] += A[16*i + .., :] B1 (gemm_regs for two right operands
// from registers with one left operand from LDS, bf16): each A read feeds both products.
template <typename MT, int NP, int NI>
__device__ __forceinline__ void gemm_regs_2b(f32x4_t* acc0, const f32x4_t* Bt0, f32x4_t* acc1, const f32x4_t* Bt1,
                                             const typename MM<MT>::S* sA, int lda) {
    static_assert(sizeof(typename MM<MT>::S) == 2, "bf16 operands");
    const int l = threadIdx.x & 63, g4 = l >> 4, lr = l & 15;
#pragma unroll
    for (int m = 0; m < NP / 32; ++m) {
        bf16x8_t av[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            av[i] = *reinterpret_cast<const bf16x8_t*>(sA + (16 * i + lr) * lda + 32 * m + 8 * g4);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 b0 = {pack_tile_lo(Bt0[2 * m]), pack_tile_hi(Bt0[2 * m]), pack_tile_lo(Bt0[2 * m + 1]),
                          pack_tile_hi(Bt0[2 * m + 1])};
        const uint4 b1 = {pack_tile_lo(Bt1[2 * m]), pack_tile_hi(Bt1[2 * m]), pack_tile_lo(Bt1[2 * m + 1]),
                          pack_tile_hi(Bt1[2 * m + 1])};
        const bf16x8_t bv0 = __builtin_bit_cast(bf16x8_t, b0), bv1 = __builtin_bit_cast(bf16x8_t, b1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            acc0[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv0, acc0[i], 0, 0, 0);
            acc1[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv1, acc1[i], 0, 0, 0);
        }
    }
}

// acc0[i] += A0[16*i + .., :] B and acc1[i] += A1[16*i + .., :] B (gemm_regs for two left operands with
// one right operand): each packing of B feeds both, and the two accumulator chains interleave.  With
// TR1 the acc1 tiles are formed transposed (as gemm_regs with TR).
template <typename MT, int NP, int NI, bool TR1 = false>
__device__ __forceinline__ void gemm_regs2(f32x4_t* acc0, const typename MM<MT>::S* sA0, f32x4_t* acc1,
                                           const typename MM<MT>::S* sA1, int lda, const f32x4_t* Bt) {
    if constexpr (sizeof(typename MM<MT>::S) == 2) {
        const int l = threadIdx.x & 63, g4 = l >> 4, lr = l & 15;
#pragma unroll
        for (int m = 0; m < NP / 32; ++m) {
            bf16x8_t a0[NI], a1[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                a0[i] = *reinterpret_cast<const bf16x8_t*>(sA0 + (16 * i + lr) * lda + 32 * m + 8 * g4);
                a1[i] = *reinterpret_cast<const bf16x8_t*>(sA1 + (16 * i + lr) * lda + 32 * m + 8 * g4);
            }
            __builtin_amdgcn_sched_barrier(0);
            const uint4 bw = {pack_tile_lo(Bt[2 * m]), pack_tile_hi(Bt[2 * m]), pack_tile_lo(Bt[2 * m + 1]),
                              pack_tile_hi(Bt[2 * m + 1])};
            const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                acc0[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], bv, acc0[i], 0, 0, 0);
                if constexpr (TR1) acc1[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, a1[i], acc1[i], 0, 0, 0);
                else acc1[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], bv, acc1[i], 0, 0, 0);
            }
        }
    } else {
        gemm_regs<MT, NP, NI>(acc0, sA0, lda, Bt);
        gemm_regs<MT, NP, NI, false, TR1>(acc1, sA1, lda, Bt);
    }
}

// Buffer resource over the rows of one chunk: `rows` rows of `row_bytes` starting at `base`.
// Loads at byte offsets past rows * row_bytes return zeros, so rows past the end of a short
// chunk read as zero without a clamp, a select or a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int rows, int row_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, rows * row_bytes, 0x00020000);
}

// Eight consecutive elements held raw in registers, so that a whole tile's worth of
// global loads can be issued before any of them is used.
template <typename IO> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 w;
    template <int AUX = 0>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff) {
        w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
    }
    __device__ __forceinline__ void get(float* x) const {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(ws[j] << 16);
            x[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
        }
    }
    // elements 4hh .. 4hh+3
    __device__ __forceinline__ void get4(float* x, int hh) const {
        const uint32_t w0 = hh ? w.z : w.x, w1 = hh ? w.w : w.y;
        x[0] = __uint_as_float(w0 << 16);
        x[1] = __uint_as_float(w0 & 0xFFFF0000u);
        x[2] = __uint_as_float(w1 << 16);
        x[3] = __uint_as_float(w1 & 0xFFFF0000u);
    }
};
template <> struct Raw8<float> {
    f32x4_t a, b;
    template <int AUX = 0>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff) {
        a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, AUX));
        b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, AUX));
    }
    __device__ __forceinline__ void get(float* x) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
    __device__ __forceinline__ void get4(float* x, int hh) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = hh ? b[e] : a[e];
    }
};

// Ownership of a [ROWS][D] row-major tile by NTHR threads in vectors of 8 elements:
// thread t holds NV vectors, all in the same 8-column slot.
template <int ROWS, int D, int NTHR> struct Tile {
    static constexpr int VPR = D / 8;
    static_assert(NTHR % VPR == 0 && (ROWS * VPR) % NTHR == 0, "tile mapping");
    static constexpr int NV = ROWS * VPR / NTHR;
    static constexpr int RSTEP = NTHR / VPR;
    __device__ __forceinline__ static int row(int tid, int i) { return tid / VPR + RSTEP * i; }
    __device__ __forceinline__ static int col(int tid) { return (tid % VPR) * 8; }
};

// Ownership of a [64][D] row-major tile by NTHR threads for transposed LDS builds, in units
// of (row pair, 8-column group): a thread holds rows 2p and 2p+1 of 8 consecutive columns, so
// the transpose is written one 32-bit word (two rows) per column without unpacking bf16 data.
// The 64 units of one wave-wide pass are 8 row pairs x 8 column groups: each load instruction
// then reads 8 rows of 128 contiguous bytes (one cache line each), and the transposed stores
// of a pass fall into 16 distinct bank groups (4-way at most).  Units past the end (only when
// the tile has fewer units than threads) duplicate unit 0's loads and store nothing.
template <int D, int NTHR> struct PairTile {
    static constexpr int CG = D / 8;          // 8-column groups
    static constexpr int CB = CG / 8;         // blocks of 8 column groups
    static_assert(CG % 8 == 0, "whole blocks of 8 column groups");
    static constexpr int UNITS = 32 * CG;
    static constexpr int NPASS = (UNITS + NTHR - 1) / NTHR;
    __device__ __forceinline__ static bool valid(int tid, int i) { return tid + NTHR * i < UNITS; }
    __device__ __forceinline__ static int pair(int tid, int i) {
        const int u = (tid + NTHR * i) % UNITS;
        return 8 * ((u >> 6) / CB) + ((u >> 3) & 7);
    }
    __device__ __forceinline__ static int col(int tid, int i) {
        const int u = (tid + NTHR * i) % UNITS;
        return 8 * (8 * ((u >> 6) % CB) + (u & 7));
    }
};

// Transposed store of a row pair: dst[(c8 + e) * ldt + perm(r0)] = {row r0, row r0 + 1}[e].
// bf16 rows are interleaved in 32-bit words (v_perm_b32) without unpacking.
template <typename MT, typename IO>
__device__ __forceinline__ void st_pair_t(typename MM<MT>::S* dst, int ldt, int c8, int r0, const Raw8<IO>& x0,
                                          const Raw8<IO>& x1) {
    if constexpr (sizeof(typename MM<MT>::S) == 2 && std::is_same<IO, bf16_t>::value) {
        const int pr = perm<MT>(r0);
        const uint32_t a[4] = {x0.w.x, x0.w.y, x0.w.z, x0.w.w}, b[4] = {x1.w.x, x1.w.y, x1.w.z, x1.w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint32_t*>(dst + (c8 + 2 * j) * ldt + pr) = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
            *reinterpret_cast<uint32_t*>(dst + (c8 + 2 * j + 1) * ldt + pr) =
                __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
        }
    } else {
        float a[8], b[8];
        x0.get(a);
        x1.get(b);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dst[(c8 + e) * ldt + perm<MT>(r0)] = MM<MT>::cvt(a[e]);
            dst[(c8 + e) * ldt + perm<MT>(r0 + 1)] = MM<MT>::cvt(b[e]);
        }
    }
}

// Row stride (floats) of the fp32 16x16 diagonal blocks of L in LDS: rows stay 16-byte aligned.
constexpr int LDN = 20;

// Value of register x held by the lanes of row group S (lanes 16S .. 16S+15), broadcast to the
// same lane position of every row group.  v_permlane16_swap with both operands x yields
// [x.r0, x.r0, x.r2, x.r2] and [x.r1, x.r1, x.r3, x.r3]; v_permlane32_swap of such a value
// with itself yields its lower half [a.r0, a.r1, a.r0, a.r1] and upper half [a.r2, a.r3, a.r2, a.r3].
template <int S>
__device__ __forceinline__ float row_group_bcast(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t a = (S & 1) ? p[1] : p[0];
    const auto q = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return __uint_as_float((S & 2) ? q[1] : q[0]);
}

// D = (I + N)^-1 for a strictly lower 16x16 N (fp32 in LDS, row stride LDN, zero on and above
// the diagonal), with all 64 lanes of the calling wave: lane (g, j) = (l / 16, l % 16) holds
// rows 4g .. 4g+3 of column j (the MFMA accumulator layout).  Blockwise forward substitution
// over the four 4-row groups: at step s the lanes of group s finish their rows by a local 4x4
// substitution, the four finished values of each column are broadcast across row groups, and
// the groups below subtract their N(4g.., 4s..) block times them.  D is written row-major
// (stride ldd) in the MFMA operand dtype.
template <typename MT>
__device__ __forceinline__ void invert_unit_lower_16(const float* sN, typename MM<MT>::S* sD, int ldd) {
    const int l = threadIdx.x & 63, g = l >> 4, j = l & 15;
    f32x4_t nb[4][4];  // nb[s][a] = N[4g + a][4s .. 4s+3]
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int a = 0; a < 4; ++a) nb[s][a] = *reinterpret_cast<const f32x4_t*>(sN + (4 * g + a) * LDN + 4 * s);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (4 * g + e == j) ? 1.0f : 0.0f;
    auto step = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        // rows of group s: local substitution with the diagonal 4x4 block of N
        float y[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
        for (int e = 1; e < 4; ++e)
#pragma unroll
            for (int f = 0; f < e; ++f) y[e] = fmaf(-nb[s][e][f], y[f], y[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (g == s) ? y[e] : x[e];
        if constexpr (s < 3) {
            float b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = row_group_bcast<s>(x[e]);
            float z[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int f = 0; f < 4; ++f) z[a] = fmaf(-nb[s][a][f], b[f], z[a]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (g > s) ? z[e] : x[e];
        }
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
#pragma unroll
    for (int e = 0; e < 4; ++e) sD[(4 * g + e) * ldd + j] = MM<MT>::cvt(x[e]);
}

// Transposing LDS read (ds_read_b64_tr_b16): for the 16 lanes of each row group g, lane i receives
// [M[r0][c0+i], M[r0+1][c0+i], M[r0+2][c0+i], M[r0+3][c0+i]] of a row-major bf16 matrix M
// (row stride ld elements), where r0 and c0 may differ between row groups.  Lanes 4r .. 4r+3 of
// the group hand the hardware row r0+r, columns c0 .. c0+15 in four 8-byte pieces.  With PERM
// the columns are stored in perm() order (4-element runs stay contiguous).
template <bool PERM>
__device__ __forceinline__ uint2 ld_tr4(const uint16_t* m, int ld, int r0, int c0) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int l = threadIdx.x & 63, r = (l >> 2) & 3, q = l & 3;
    const int c = c0 + 4 * q;
    const uint16_t* p = m + (r0 + r) * ld + (PERM ? perm<bf16_t>(c) : c);
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    return __builtin_bit_cast(uint2, v);
}

// RHS block loaders for block_solve: rows 16I + 4*(l/16) + e (e = 0..3) of column l%16 of a
// 16-column tile, scaled per row by sc[t].
// A loader's raw() issues the block's LDS reads; value() forms the scaled block from them.
template <typename MT> struct RhsFromTransposed {   // the tile's transposed row (this lane's column)
    const typename MM<MT>::S* bt;
    const float* sc;
    struct Raw {
        f32x4_t f;
        typename std::conditional<sizeof(typename MM<MT>::S) == 2, uint2, f32x4_t>::type x;
    };
    __device__ __forceinline__ Raw raw(int I) const {
        const int t0 = 16 * I + 4 * ((threadIdx.x & 63) >> 4);
        Raw r;
        r.f = *reinterpret_cast<const f32x4_t*>(sc + t0);
        if constexpr (sizeof(typename MM<MT>::S) == 2)
            r.x = *reinterpret_cast<const uint2*>(bt + perm<MT>(t0));
        else
            r.x = *reinterpret_cast<const f32x4_t*>(bt + t0);
        return r;
    }
    __device__ __forceinline__ static f32x4_t value(const Raw& r) {
        if constexpr (sizeof(typename MM<MT>::S) == 2)
            return f32x4_t{__uint_as_float(r.x.x << 16) * r.f[0], __uint_as_float(r.x.x & 0xFFFF0000u) * r.f[1],
                           __uint_as_float(r.x.y << 16) * r.f[2], __uint_as_float(r.x.y & 0xFFFF0000u) * r.f[3]};
        else
            return r.x * r.f;
    }
};
struct RhsFromRows {                               // row-major bf16 rows (perm() columns), columns c0 .. c0+15
    const uint16_t* m;
    int ld, c0;
    const float* sc;
    struct Raw {
        f32x4_t f;
        uint2 x;
    };
    __device__ __forceinline__ Raw raw(int I) const {
        const int t0 = 16 * I + 4 * ((threadIdx.x & 63) >> 4);
        return Raw{*reinterpret_cast<const f32x4_t*>(sc + t0), ld_tr4<true>(m, ld, t0, c0)};
    }
    __device__ __forceinline__ static f32x4_t value(const Raw& r) {
        return f32x4_t{__uint_as_float(r.x.x << 16) * r.f[0], __uint_as_float(r.x.x & 0xFFFF0000u) * r.f[1],
                       __uint_as_float(r.x.y << 16) * r.f[2], __uint_as_float(r.x.y & 0xFFFF0000u) * r.f[3]};
    }
};

struct RhsFromRowsF32 {                            // row-major fp32 rows (natural columns), columns c0 .. c0+15
    const float* m;
    int ld, c0;
    const float* sc;
    struct Raw {
        f32x4_t f, x;
    };
    __device__ __forceinline__ Raw raw(int I) const {
        const int t0 = 16 * I + 4 * ((threadIdx.x & 63) >> 4), c = c0 + (threadIdx.x & 15);
        return Raw{*reinterpret_cast<const f32x4_t*>(sc + t0),
                   f32x4_t{m[t0 * ld + c], m[(t0 + 1) * ld + c], m[(t0 + 2) * ld + c], m[(t0 + 3) * ld + c]}};
    }
    __device__ __forceinline__ static f32x4_t value(const Raw& r) { return r.x * r.f; }
};

// X = (I + L)^-1 B for NR 16-column tiles of B (64 rows each), by blocked forward substitution:
// X_I = D_I (B_I - sum_{J<I} L_IJ X_J), D_I = (I + L_II)^-1.  L's off-diagonal blocks are read
// negated from sLo (row-major, stride ldo), the D_I from sD (block I at sD + 16*I*ldd); rhs[n].raw(I)
// returns block I of tile n.  X stays in registers in C layout; with v_mfma_f32_16x16x16_bf16 the
// C layout of one block is the B operand layout of the next product, so each wave solves its own
// columns without synchronising with the others.  The NR tiles share every read of L and D, and
// their dependency chains interleave.  A scheduling barrier keeps the chain behind the reads.
template <typename MT, int NR, typename Rhs>
__device__ __forceinline__ void block_solve(f32x4_t (*X)[4], const typename MM<MT>::S* sLo, int ldo,
                                            const typename MM<MT>::S* sD, int ldd, const Rhs* rhs) {
    const int l = threadIdx.x & 63, g4 = l >> 4, lr = l & 15;
    typedef typename MM<MT>::S S;
    // every LDS read of the solve (the right-hand sides and, for bf16, the blocks of L and D) is
    // issued before the first is used, so the dependency chain below waits on no LDS access
    typename Rhs::Raw raw[NR][4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int n = 0; n < NR; ++n) raw[n][I] = rhs[n].raw(I);
    if constexpr (sizeof(S) == 2) {
        s16x4_t lv[6], dv[4];  // L_IJ at I (I - 1) / 2 + J, J < I
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            dv[I] = *reinterpret_cast<const s16x4_t*>(sD + (16 * I + lr) * ldd + 4 * g4);
#pragma unroll
            for (int J = 0; J < I; ++J)
                lv[I * (I - 1) / 2 + J] = *reinterpret_cast<const s16x4_t*>(sLo + (16 * I + lr) * ldo + 16 * J + 4 * g4);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t R[NR][4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int n = 0; n < NR; ++n) R[n][I] = Rhs::value(raw[n][I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int J = 0; J < I; ++J) {
#pragma unroll
                for (int n = 0; n < NR; ++n) {
                    const s16x4_t bv = __builtin_bit_cast(s16x4_t, uint2{pack_tile_lo(X[n][J]), pack_tile_hi(X[n][J])});
                    R[n][I] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lv[I * (I - 1) / 2 + J], bv, R[n][I], 0, 0, 0);
                }
            }
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const s16x4_t rv = __builtin_bit_cast(s16x4_t, uint2{pack_tile_lo(R[n][I]), pack_tile_hi(R[n][I])});
                X[n][I] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dv[I], rv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
        }
    } else {
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t R[NR][4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int n = 0; n < NR; ++n) R[n][I] = Rhs::value(raw[n][I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int J = 0; J < I; ++J) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float av = sLo[(16 * I + lr) * ldo + 16 * J + 4 * g4 + e];
#pragma unroll
                    for (int n = 0; n < NR; ++n)
                        R[n][I] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, X[n][J][e], R[n][I], 0, 0, 0);
                }
            }
#pragma unroll
            for (int n = 0; n < NR; ++n) X[n][I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dv = sD[(16 * I + lr) * ldd + 4 * g4 + e];
#pragma unroll
                for (int n = 0; n < NR; ++n)
                    X[n][I] = __builtin_amdgcn_mfma_f32_16x16x4f32(dv, R[n][I][e], X[n][I], 0, 0, 0);
            }
        }
    }
}

// The 6 strictly lower (I, J) tiles of a 64x64 matrix: (1,0),(2,0),(2,1),(3,0),(3,1),(3,2).
__device__ __forceinline__ void strict_tile(int t, int& I, int& J) {
    I = t >= 3 ? 3 : t >= 1 ? 2 : 1;
    J = t - I * (I - 1) / 2;
}

// Store the 8 consecutive logical columns c8 .. c8+7 of a row into a perm()-ordered LDS row.
template <typename MT, typename IO>
__device__ __forceinline__ void st8_perm(typename MM<MT>::S* row, int c8, const Raw8<IO>& x) {
    if constexpr (sizeof(typename MM<MT>::S) == 2 && std::is_same<IO, bf16_t>::value) {
        *reinterpret_cast<uint2*>(row + perm<MT>(c8)) = uint2{x.w.x, x.w.y};
        *reinterpret_cast<uint2*>(row + perm<MT>(c8 + 4)) = uint2{x.w.z, x.w.w};
    } else {
        float f[8];
        x.get(f);
        MM<MT>::st8(row + c8, f);
    }
}

// Four fp32 values into four adjacent elements (natural column order) of the operand type.
template <typename MT>
__device__ __forceinline__ void st4f(typename MM<MT>::S* p, const float* f) {
    if constexpr (sizeof(typename MM<MT>::S) == 2)
        *reinterpret_cast<uint2*>(p) = uint2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
    else
        *reinterpret_cast<f32x4_t*>(p) = f32x4_t{f[0], f[1], f[2], f[3]};
}

// Four fp32 values of logical columns c4 .. c4+3 (c4 a multiple of 4) into an operand row, in the
// operand's type and column order (the four stay adjacent under perm()).
template <typename MT>
__device__ __forceinline__ void st4f_perm(typename MM<MT>::S* row, int c4, const float* f) {
    if constexpr (sizeof(typename MM<MT>::S) == 2)
        *reinterpret_cast<uint2*>(row + perm<MT>(c4)) = uint2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
    else
        *reinterpret_cast<f32x4_t*>(row + c4) = f32x4_t{f[0], f[1], f[2], f[3]};
}

// Eight fp32 values of logical columns c8 .. c8+7 into an operand row, in the operand's type and
// column order.
template <typename MT>
__device__ __forceinline__ void st8f_perm(typename MM<MT>::S* row, int c8, const float* f) {
    if constexpr (sizeof(typename MM<MT>::S) == 2) {
        *reinterpret_cast<uint2*>(row + perm<MT>(c8)) = uint2{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        *reinterpret_cast<uint2*>(row + perm<MT>(c8 + 4)) = uint2{pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
    } else {
        MM<MT>::st8(row + c8, f);
    }
}

// ---------------------------------------------------------------------------
// LDS layout (bytes).  A-operand rows of the MFMA products are perm()-ordered.
template <int K, int BV, typename MT, bool PER_K>
struct Layout {
    typedef typename MM<MT>::S S;
    static constexpr bool BF = sizeof(S) == 2;
    static constexpr int LDK = K + MM<MT>::PAD;   // rows over the K channels
    static constexpr int LDT = CH + MM<MT>::PAD;  // rows over the 64 chunk positions
    static constexpr int LDO = CH + MM<MT>::PAD;  // -L off-diagonal blocks, natural order
    static constexpr int LDD = 16 + MM<MT>::PAD;  // diagonal-block inverses
    static constexpr size_t ROWK = sizeof(S) * CH * LDK;   // [64][LDK]
    static constexpr size_t ROWT = sizeof(S) * CH * LDT;   // [64][LDT]
    static constexpr size_t KT_ = sizeof(S) * K * LDT;     // [K][LDT]
    static constexpr size_t VT_ = sizeof(S) * BV * LDT;    // [BV][LDT]
    static constexpr size_t LO_ = sizeof(S) * CH * LDO;    // [64][LDO]
    static constexpr size_t LD_ = sizeof(float) * 4 * 16 * LDN;  // diagonal L blocks, fp32
    static constexpr size_t D_ = sizeof(S) * CH * LDD;     // [4*16][LDD]
    // bf16 scalar gate with one K tile per wave: V is kept row-major ([64][LDV], perm() columns)
    // in the V^T area and read through transposing LDS reads, and K^T is not built
    static constexpr int LDV = BV + MM<MT>::PAD;
    static constexpr bool TRK = !PER_K && BF && K / 16 == BV / 16;
    static_assert(!TRK || sizeof(S) * CH * LDV <= VT_, "row-major V fits the V^T area");
    // fp32 operands at K = 128 (scalar gate): an fp32 MFMA operand is one element per lane, so K^T is
    // read from the row-major K rows with transposed indexing and no K^T copy is built; the fp32
    // diagonal blocks of L live in the -W area (W is dead from E until D rewrites it)
    static constexpr bool KROW = !PER_K && !BF && K == 128;

    // ---- scalar gate ----
    static constexpr size_t g_q = 0;              // Q rows
    static constexpr size_t g_k = g_q + ROWK;     // K rows
    static constexpr size_t g_w = g_k + ROWK;     // -W rows
    static constexpr size_t g_kt = g_w + ROWK;    // K^T
    static constexpr size_t g_vt = g_kt + (KROW ? 0 : KT_);  // V^T
    static constexpr size_t g_lo = g_vt + VT_;
    static constexpr size_t g_ld = KROW ? g_w : g_lo + LO_;
    static constexpr size_t g_d = g_lo + LO_ + (KROW ? 0 : LD_);
    static constexpr size_t g_p = g_d + D_;       // P rows
    static constexpr size_t g_g = g_p + ROWT;     // gamma [64]
    static constexpr size_t g_b = g_g + sizeof(float) * CH;    // beta [64]
    static constexpr size_t g_be = g_b + sizeof(float) * CH;   // beta e^gamma [64]
    static constexpr size_t g_eg = g_be + sizeof(float) * CH;  // e^gamma [64]
    static constexpr size_t g_ed = g_eg + sizeof(float) * CH;  // e^(gamma_last - gamma) [64]
    // off-diagonal decay factors with reference point rho_J = gamma[16J + 15]:
    // e^(gamma_r - gamma_j) = e^(gamma_r - rho_J) e^(rho_J - gamma_j), both <= 1 for r in a
    // later 16-row block than j (block J)
    static constexpr size_t g_fa = g_ed + sizeof(float) * CH;  // [3][64] e^(gamma_r - rho_J)
    static constexpr size_t g_fb = g_fa + sizeof(float) * 3 * CH;  // [64] e^(rho_(j/16) - gamma_j)
    static constexpr size_t g_total = g_fb + sizeof(float) * CH;

    // ---- per-K gate: fixed part, then X (phases A-B, then C-E) and Y (B-D), W (D-E) ----
    static constexpr size_t k_g = 0;                                  // gamma [64][K]
    static constexpr size_t k_gl = k_g + sizeof(float) * CH * K;      // e^{gamma_last} [K]
    static constexpr size_t k_b = k_gl + sizeof(float) * K;           // beta [64]
    static constexpr size_t k_p = k_b + sizeof(float) * CH;           // P rows
    static constexpr size_t X = k_p + ROWT;
    static constexpr size_t AB = 2 * ROWK + sizeof(S) * 96 * LDK;     // Q, K rows; 16 + 16 + 64 operand rows
    static constexpr size_t CE = KT_ + VT_ + ROWK + KT_;              // (K e^g)^T, V^T, Q e^g, (K e^{gl-g})^T
    static constexpr size_t SX = AB > CE ? AB : CE;
    static constexpr size_t k_q = X;
    static constexpr size_t k_k = k_q + ROWK;
    static constexpr size_t k_lk = k_k + ROWK;                        // K_I e^{gamma - rho}   [16][LDK]
    static constexpr size_t k_lq = k_lk + sizeof(S) * 16 * LDK;       // Q_I e^{gamma - rho}   [16][LDK]
    static constexpr size_t k_rg = k_lq + sizeof(S) * 16 * LDK;       // K_<=I e^{rho - gamma} [64][LDK]
    static constexpr size_t k_kgt = X;
    static constexpr size_t k_vt = k_kgt + KT_;
    static constexpr size_t k_qt = k_vt + VT_;
    static constexpr size_t k_kdt = k_qt + ROWK;
    static constexpr size_t Y = X + SX;
    static constexpr size_t k_lo = Y;
    static constexpr size_t k_ld = k_lo + LO_;
    static constexpr size_t k_d = k_ld + LD_;
    static constexpr size_t k_w = k_d + D_;
    static constexpr size_t k_part = k_w;                             // gamma partial sums (phase A)
    static constexpr size_t k_fp = k_lk;                              // [7][K] pair factors (A to B/C, MFMA form)
    static constexpr size_t k_total = k_w + ROWK;

    // output tile staging [64][BV] in the IO type, 16-byte granules XOR-swizzled by row.  It is
    // written at the end of E and flushed at the start of the next iteration; the -L and
    // diagonal-inverse area it overlays is rewritten only in B/C, after the next phase-A barrier.
    static constexpr size_t o_stage = PER_K ? k_lo : g_lo;
    static constexpr size_t o_room = PER_K ? LO_ + LD_ + D_ : g_d + D_ - g_lo;  // bytes the staging may overlay
    static constexpr size_t total = PER_K ? k_total : g_total;
};

template <int BV, typename IO>
struct OStage {
    static constexpr int SZ = sizeof(IO) == 4 ? 4 : 2;
    static constexpr int ROWB = BV * SZ;        // bytes per staged row
    static constexpr int NG = ROWB / 16;        // 16-byte granules per row
    static constexpr int EPG = 16 / SZ;         // elements per granule
    static constexpr size_t bytes = (size_t)CH * ROWB;
    __device__ __forceinline__ static int off(int r, int c) {
        const int gr = (c / EPG) ^ (r % NG);
        return r * ROWB + gr * 16 + (c % EPG) * SZ;
    }
};

// Per-channel gate: largest decay range (in natural-log units) across one 16-row diagonal block
// that the MFMA form of that block accepts; e^64 ~ 6e27 keeps both scaled operands and their
// products well inside the fp32 / bf16 exponent range.
constexpr float kKdaDiagRange = 64.0f;

// With MAP (bf16, K = V, either gate; the segmented route), one run forms both end-of-segment
// quantities of a (segment, head): the state reached from h0 with the inputs (ht) and the linear part
// of the segment's map, the state reached from the identity with v = 0 (map [N, HV, K, K]).  Wave w
// holds value columns 16w .. 16w+15 of the first and rows 16w .. 16w+15 of the second; the two share
// every chunk's k, gate and beta reads and the whole intra-chunk transform, and each product of E
// reads its LDS operand once for both.  No q is read and no output is formed.
template <int K, int BV, typename IO, typename MT, bool PER_K, bool MAP = false>
__global__ __launch_bounds__(4 * BV) void chunk_fused_kernel(const ChunkArgs a) {
    constexpr int NW = BV / 16;       // waves; wave w owns value columns 16w .. 16w+15 of the tile
    constexpr int NTHR = 64 * NW;
    static_assert(!MAP || (K == BV && sizeof(typename MM<MT>::S) == 2), "paired run: K = V, bf16");
    constexpr int KT = K / 16;
    typedef MM<MT> M;
    typedef typename M::S S;
    typedef Layout<K, BV, MT, PER_K> Lay;
    constexpr int LDK = Lay::LDK, LDT = Lay::LDT, LDO = Lay::LDO, LDD = Lay::LDD;
    static_assert(NW >= 4, "four waves invert the diagonal blocks");
    // without outputs (the segment-offset and segment-map runs) q, P and the output are skipped
    const bool want_o = !MAP && a.o != nullptr;
    typedef OStage<BV, IO> OS;
    constexpr bool TRK = Lay::TRK;
    static_assert(Lay::total <= 160 * 1024, "LDS budget");
    static_assert(OS::bytes <= Lay::o_room, "output staging overlays -L and the inverses");
    constexpr bool KROW = Lay::KROW;
    __shared__ __align__(16) char smem[Lay::total];
    auto SP = [&](size_t off) { return reinterpret_cast<S*>(smem + off); };
    auto FP = [&](size_t off) { return reinterpret_cast<float*>(smem + off); };

    const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    const int hk = h / (a.HV / a.HK);
    int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, lr = l & 15;  // laundered each chunk (below)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    const int v0 = vt * BV;
    const int vcol = v0 + 16 * w + lr;
    const int64_t s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
    const int64_t s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : a.T;
    const int nc = (int)((s1 - s0 + CH - 1) / CH);

    // state tiles: hs[kt][e] = S[vcol][16*kt + 4*(l/16) + e]
    f32x4_t hs[KT];
    const int64_t sidx = (((int64_t)n * a.HV + h) * a.V + vcol) * K;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        hs[kt] = a.h0 ? *reinterpret_cast<const f32x4_t*>(a.h0 + sidx + 16 * kt + 4 * g4)
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // MAP: rows 16w .. 16w+15 of the segment map, from the identity (row 16w + l%16 of the K x K map)
    f32x4_t hm[MAP ? KT : 1];
    if constexpr (MAP) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hm[kt][e] = (16 * kt + 4 * g4 + e == 16 * w + lr) ? 1.0f : 0.0f;
    }

    // strictly upper tiles of P are never written: zero them once
    {
        S* sP = SP(PER_K ? Lay::k_p : Lay::g_p);
        for (int idx = tid; idx < CH * CH; idx += NTHR) {
            const int r = idx / CH, j = idx % CH;
            if ((j >> 4) > (r >> 4)) sP[r * LDT + perm<MT>(j)] = M::cvt(0.0f);
        }
    }

    // ---- per-chunk inputs, double-buffered in registers ----
    typedef Tile<CH, K, NTHR> TQ;           // q rows
    typedef PairTile<K, NTHR> PK;            // k row pairs
    typedef PairTile<BV, NTHR> PV;           // v row pairs
    constexpr int GQ = NTHR / K;                   // per-K gate: row groups per channel
    constexpr int RPQ = PER_K ? CH / GQ : 1;       // gate values per thread
    // per-K gate: q in the row-pair mapping of k, so that both share the decay factors of a unit
    constexpr int NQ = PER_K ? 2 * PK::NPASS : TQ::NV;
    Raw8<IO> qn[NQ], kn[2 * PK::NPASS], vn[2 * PV::NPASS];
    float gn[RPQ] = {};
    uint32_t bn = 0;  // beta kept as loaded (bf16 bits or fp32 bits): converting here would wait on the load
    // byte strides of one token row and this thread's byte offsets inside a chunk (fixed)
    constexpr int ESZ = sizeof(IO) == 4 ? 4 : 2;
    const int qk_row = a.HK * K * ESZ, v_row = a.HV * a.V * ESZ;
    const int g_row = (PER_K ? a.HV * K : a.HV) * 4, b_row = a.HV * ESZ;
    const int gq_c = PER_K ? tid % K : 0, gq_r = PER_K ? (tid / K) * RPQ : (tid & 63);
    // the next chunk's rows are loaded in three parts at three points of the current chunk, so
    // that the cache-line misses a workgroup has in flight stay bounded and no wave stalls long
    // on issue: q (end of B/C), k (start of D), v with g and beta (in E, after v_new)
    auto chunk_len = [&](int ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        return (s1 - bos) < CH ? (int)(s1 - bos) : CH;
    };
    auto load_q = [&](int ci) {
        if (!want_o) return;  // q only feeds P and the output
        const int64_t bos = s0 + (int64_t)CH * ci;
        const __amdgpu_buffer_rsrc_t rq =
            chunk_rsrc(static_cast<const char*>(a.q) + ((bos * a.HK + hk) * K) * ESZ, chunk_len(ci), qk_row);
        if constexpr (PER_K) {
#pragma unroll
            for (int i = 0; i < PK::NPASS; ++i)
#pragma unroll
                for (int u = 0; u < 2; ++u) qn[2 * i + u].load(rq, (2 * PK::pair(tid, i) + u) * qk_row + PK::col(tid, i) * ESZ);
        } else {
#pragma unroll
            for (int i = 0; i < TQ::NV; ++i) qn[i].load(rq, TQ::row(tid, i) * qk_row + TQ::col(tid) * ESZ);
        }
    };
    auto load_k = [&](int ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        const __amdgpu_buffer_rsrc_t rk =
            chunk_rsrc(static_cast<const char*>(a.k) + ((bos * a.HK + hk) * K) * ESZ, chunk_len(ci), qk_row);
#pragma unroll
        for (int i = 0; i < PK::NPASS; ++i)
#pragma unroll
            for (int u = 0; u < 2; ++u) kn[2 * i + u].load(rk, (2 * PK::pair(tid, i) + u) * qk_row + PK::col(tid, i) * ESZ);
    };
    auto load_vgb = [&](int ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        const int len = chunk_len(ci);
        // v == NULL reads as zeros (a zero-byte range): the run that forms a segment's linear map
        const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(
            a.v ? static_cast<const char*>(a.v) + ((bos * a.HV + h) * a.V + v0) * ESZ : nullptr, a.v ? len : 0, v_row);
#pragma unroll
        for (int i = 0; i < PV::NPASS; ++i)
#pragma unroll
            for (int u = 0; u < 2; ++u) vn[2 * i + u].load(rv, (2 * PV::pair(tid, i) + u) * v_row + PV::col(tid, i) * ESZ);
        // the scalar gate and beta are read by wave 0 only (one value per row, one cache line each)
        if (PER_K || w == 0) {
            const float* g0 = a.g + (PER_K ? (bos * a.HV + h) * K : bos * a.HV + h);
            const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(g0, len, g_row);
#pragma unroll
            for (int i = 0; i < RPQ; ++i)
                gn[i] = __builtin_bit_cast(float,
                                           __builtin_amdgcn_raw_buffer_load_b32(rg, (gq_r + i) * g_row + gq_c * 4, 0, 0));
        }
        if (w == 0) {
            const __amdgpu_buffer_rsrc_t rb =
                chunk_rsrc(static_cast<const char*>(a.beta) + (bos * a.HV + h) * ESZ, len, b_row);
            if constexpr (std::is_same<IO, float>::value)
                bn = __builtin_amdgcn_raw_buffer_load_b32(rb, (tid & 63) * b_row, 0, 0);
            else
                bn = __builtin_amdgcn_raw_buffer_load_b16(rb, (tid & 63) * b_row, 0, 0);
        }
    };
    auto load_chunk = [&](int ci) {
        load_q(ci);
        load_k(ci);
        load_vgb(ci);
    };
    if (nc > 0) load_chunk(0);

    // staged output rows of a chunk -> o, one 16-byte granule per thread and pass
    char* const so = smem + Lay::o_stage;
    auto flush_o = [&](int64_t bos, int len) {
        if (!want_o) return;  // outputs not wanted (the segment-offset and segment-map runs)
        for (int idx = tid; idx < CH * OS::NG; idx += NTHR) {
            const int r = idx / OS::NG, gi = idx % OS::NG;
            if (r < len) {
                const uint4 x = *reinterpret_cast<const uint4*>(so + OS::off(r, gi * OS::EPG));
                char* dst = static_cast<char*>(a.o) + (((bos + r) * a.HV + h) * a.V + v0 + gi * OS::EPG) * OS::SZ;
                *reinterpret_cast<uint4*>(dst) = x;
            }
        }
    };

    for (int ci = 0; ci < nc; ++ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        if constexpr (PER_K) {
            // the lane indices look new to the compiler in every chunk: the many per-lane addresses
            // derived from them are then recomputed where used instead of being hoisted out of the
            // loop and held in registers (the per-K form has too few to spare)
            asm volatile("" : "+v"(tid));
            l = tid & 63;
            g4 = l >> 4;
            lr = l & 15;
        }

        // current chunk <- prefetched registers (the next chunk's loads are issued in B/C, D and E)
        Raw8<IO> qr[NQ], kr[2 * PK::NPASS], vr[2 * PV::NPASS];
        float gr[RPQ];
        const float br = std::is_same<IO, float>::value ? __uint_as_float(bn) : __uint_as_float(bn << 16);
#pragma unroll
        for (int i = 0; i < NQ; ++i) qr[i] = qn[i];
#pragma unroll
        for (int i = 0; i < 2 * PK::NPASS; ++i) kr[i] = kn[i];
#pragma unroll
        for (int i = 0; i < 2 * PV::NPASS; ++i) vr[i] = vn[i];
#pragma unroll
        for (int i = 0; i < RPQ; ++i) gr[i] = gn[i];
        if (ci > 0) flush_o(bos - CH, CH);

        S* sQ = SP(PER_K ? Lay::k_q : Lay::g_q);
        S* sK = SP(PER_K ? Lay::k_k : Lay::g_k);
        S* sP = SP(PER_K ? Lay::k_p : Lay::g_p);
        S* sLo = SP(PER_K ? Lay::k_lo : Lay::g_lo);
        float* sLd = FP(PER_K ? Lay::k_ld : Lay::g_ld);
        S* sD = SP(PER_K ? Lay::k_d : Lay::g_d);
        S* sW = SP(PER_K ? Lay::k_w : Lay::g_w);
        float* sg = FP(PER_K ? Lay::k_g : Lay::g_g);
        float* sb = FP(PER_K ? Lay::k_b : Lay::g_b);

        // ===== A: raw rows into LDS (scalar gate; the per-K gate scales them from registers in B),
        //       gate prefix =====
        bool wide = false;  // per-K gate: some 16-row block spans more decay than its MFMA form accepts
#pragma unroll
        for (int i = 0; i < TQ::NV; ++i) {
            if (PER_K || !want_o) break;
            st8_perm<MT, IO>(sQ + TQ::row(tid, i) * LDK, TQ::col(tid), qr[i]);
        }
#pragma unroll
        for (int i = 0; i < PK::NPASS; ++i) {
            if (PER_K) break;
            if (PK::valid(tid, i)) {
                const int c8 = PK::col(tid, i), pr0 = 2 * PK::pair(tid, i);
                st8_perm<MT, IO>(sK + pr0 * LDK, c8, kr[2 * i]);
                st8_perm<MT, IO>(sK + (pr0 + 1) * LDK, c8, kr[2 * i + 1]);
                if constexpr (!PER_K && !TRK && !KROW) st_pair_t<MT, IO>(SP(Lay::g_kt), LDT, c8, pr0, kr[2 * i], kr[2 * i + 1]);
            }
        }
        if constexpr (!PER_K) {
#pragma unroll
            for (int i = 0; i < PV::NPASS; ++i) {
                if (PV::valid(tid, i)) {
                    const int c8 = PV::col(tid, i), pr0 = 2 * PV::pair(tid, i);
                    if constexpr (TRK) {
                        st8_perm<MT, IO>(SP(Lay::g_vt) + pr0 * Lay::LDV, c8, vr[2 * i]);
                        st8_perm<MT, IO>(SP(Lay::g_vt) + (pr0 + 1) * Lay::LDV, c8, vr[2 * i + 1]);
                    } else {
                        st_pair_t<MT, IO>(SP(Lay::g_vt), LDT, c8, pr0, vr[2 * i], vr[2 * i + 1]);
                    }
                }
            }
            if (tid < 64) {  // wave 0: inclusive prefix sum of the 64 gates (rows past the end are 0)
                const int r = tid;
                const float x = wave_inclusive_sum(gr[0]);
                const float xl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), CH - 1));
                const float ex = exp_f32(x);
                sg[r] = x;
                sb[r] = br;
                FP(Lay::g_be)[r] = br * ex;
                FP(Lay::g_eg)[r] = ex;                   // row factors of E, both <= 1
                FP(Lay::g_ed)[r] = exp_f32(xl - x);
                float rho[4];
#pragma unroll
                for (int J = 0; J < 4; ++J) rho[J] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16 * J + 15));
#pragma unroll
                for (int J = 0; J < 3; ++J) FP(Lay::g_fa)[J * CH + r] = exp_f32(fminf(x - rho[J], 0.0f));
                const int jb = r >> 4;
                const float rj = jb == 0 ? rho[0] : jb == 1 ? rho[1] : jb == 2 ? rho[2] : rho[3];
                FP(Lay::g_fb)[r] = exp_f32(rj - x);
            }
        } else {
            // thread (c, qd): prefix over its RPQ rows of channel c, then group offsets
            const int c = tid % K, qd = tid / K;
            float* part = FP(Lay::k_part);
            float x = 0.0f;
#pragma unroll
            for (int i = 0; i < RPQ; ++i) {
                x += gr[i];
                gr[i] = x;
            }
            part[qd * K + c] = x;
            if (tid < 64) sb[tid] = br;
            __syncthreads();
            float off = 0.0f;
            for (int j = 0; j < qd; ++j) off += part[j * K + c];
#pragma unroll
            for (int i = 0; i < RPQ; ++i) sg[(qd * RPQ + i) * K + c] = gr[i] + off;
            // decay across the 16-row blocks this thread's rows close: with reference point
            // rho = gamma[16I - 1] the right factor of block I's own rows reaches e^(-(block sum))
            if constexpr (RPQ >= 16) {
#pragma unroll
                for (int b = 0; b < RPQ / 16; ++b)
                    wide = wide || (-(gr[16 * b + 15] - (b ? gr[16 * b - 1] : 0.0f)) > kKdaDiagRange);
            } else {
                static_assert(RPQ == 8, "row groups of 8, 16 or 32");
                if (qd & 1) wide = -(part[(qd - 1) * K + c] + part[qd * K + c]) > kKdaDiagRange;
            }
        }
        // the per-K form learns here whether any block of the chunk needs the element-wise form
        int wide_any = 0;
        if constexpr (PER_K) wide_any = __syncthreads_or(wide);
        else __syncthreads();

        // ===== B/C: L = beta (K K^T) decay (strictly lower), P = (Q K^T) decay (lower incl. diag);
        //       waves 0-3 also invert the diagonal block of L they computed =====
        if constexpr (!PER_K) {
            // L(I, J) and P(I, J) share their right operand K_J: they are computed as pairs, with every
            // operand read issued before the first product, and transposed (K_J as the left operand):
            // lane (g, i) then holds row 16I + i, columns 16J + 4g .. +3, and writes them with one store
            auto pair = [&](int I, int J, f32x4_t& cl, f32x4_t& cp) {
                cl = f32x4_t{0.f, 0.f, 0.f, 0.f};
                cp = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (want_o)
                    M::template nt2<K>(cl, sK + 16 * J * LDK, sK + 16 * I * LDK, cp, sK + 16 * J * LDK,
                                       sQ + 16 * I * LDK, LDK);
                else  // P only feeds the output
                    M::nt(cl, sK + 16 * J * LDK, LDK, sK + 16 * I * LDK, LDK, K);
            };
            auto store_p_diag = [&](int I, const f32x4_t& acc) {  // element-wise decay, masked (transposed tile)
                const int r = 16 * I + lr;
                const float gr = sg[r];
                const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(sg + 16 * I + 4 * g4);
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = exp_f32(gr - gj[e]) * acc[e];  // inf above the diagonal is discarded
                    x[e] = (lr >= 4 * g4 + e) ? v : 0.0f;
                }
                st4f_perm<MT>(sP + r * LDT, 16 * I + 4 * g4, x);
            };
            // off-diagonal blocks (I > J): decay from the per-row factor tables (transposed tiles)
            auto store_off = [&](int I, int J, const f32x4_t& cl, const f32x4_t& cp) {
                const int r = 16 * I + lr;
                const float fa = FP(Lay::g_fa)[J * CH + r];
                const float br = sb[r];
                const f32x4_t fb = *reinterpret_cast<const f32x4_t*>(FP(Lay::g_fb) + 16 * J + 4 * g4);
                float lx[4], px[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = fa * fb[e];
                    lx[e] = -br * d * cl[e];
                    px[e] = d * cp[e];
                }
                st4f<MT>(sLo + r * LDO + 16 * J + 4 * g4, lx);
                if (want_o) st4f_perm<MT>(sP + r * LDT, 16 * J + 4 * g4, px);
            };
            auto off_pair = [&](int q) {  // q-th of the pairs (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
                int I, J;
                strict_tile(q, I, J);
                f32x4_t cl, cp;
                pair(I, J, cl, cp);
                store_off(I, J, cl, cp);
            };
            // diagonal blocks: with eight waves, waves 0-3 compute L(w, w) and invert it while waves
            // 6 and 7 (which have one off-diagonal pair each) compute the diagonal P tiles
            if (w < 4) {  // diagonal L(w, w) (and P(w, w) with four waves), then D_w = (I + L_ww)^-1
                f32x4_t cl, cp;
                if constexpr (NW > 4) {
                    cl = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    M::nt(cl, sK + 16 * w * LDK, LDK, sK + 16 * w * LDK, LDK, K);
                } else {
                    pair(w, w, cl, cp);
                }
                // (K_w K_w^T is symmetric: the tile reads as transposed like the pairs)
                float* sN = sLd + w * 16 * LDN;
                const float gr = sg[16 * w + lr];
                const float br = sb[16 * w + lr];
                const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(sg + 16 * w + 4 * g4);
                f32x4_t xn;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = br * exp_f32(gr - gj[e]) * cl[e];
                    xn[e] = (lr > 4 * g4 + e) ? x : 0.0f;
                }
                *reinterpret_cast<f32x4_t*>(sN + lr * LDN + 4 * g4) = xn;
                if constexpr (NW == 4) {
                    if (want_o) store_p_diag(w, cp);
                }
                // the tile's LDS writes complete before this wave's lanes read other lanes' entries
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                invert_unit_lower_16<MT>(sN, sD + 16 * w * LDD, LDD);
            }
            if constexpr (NW > 4) {
                // waves 4-7: the six off-diagonal pairs (two each for waves 4 and 5)
                if (w >= 4) {
                    off_pair(w - 4);
                    if (w < 6) {
                        off_pair(w - 4 + 4);
                    } else if (want_o) {  // waves 6 and 7: diagonal P tiles (I, I), I = 2 (w - 6), 2 (w - 6) + 1
                        const int I0 = 2 * (w - 6);
                        f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
                        M::template nt2<K>(c0, sK + 16 * I0 * LDK, sQ + 16 * I0 * LDK, c1, sK + 16 * (I0 + 1) * LDK,
                                           sQ + 16 * (I0 + 1) * LDK, LDK);
                        store_p_diag(I0, c0);
                        store_p_diag(I0 + 1, c1);
                    }
                }
            } else {
                off_pair(w);
                if (w < 2) off_pair(w + 4);
            }
            if (ci + 1 < nc) load_q(ci + 1);
        } else {
            S* sLK = SP(Lay::k_lk);
            S* sLQ = SP(Lay::k_lq);
            S* sRG = SP(Lay::k_rg);
            // 8 consecutive channels of gamma in two 16-byte reads
            auto g8 = [&](int r, int c8, float* x) {
                const f32x4_t a = *reinterpret_cast<const f32x4_t*>(sg + r * K + c8);
                const f32x4_t b = *reinterpret_cast<const f32x4_t*>(sg + r * K + c8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = a[e];
                    x[4 + e] = b[e];
                }
            };
            if (!wide_any) {
                // Row block I against blocks J <= I on MFMA with reference points: e^(gamma_r - gamma_j) =
                // e^(gamma_r - rho_I) f_IJ e^(G_J - gamma_j), rho_I = gamma[16I - 1] (0 for I = 0),
                // G_J = gamma[16J + 15], f_IJ = e^(rho_I - G_J): 1 for J = I - 1, <= 1 for J < I - 1, and
                // below e^kKdaDiagRange for J = I (the test of phase A).  The two outer factors are <= 1
                // and scale the operands: each thread scales its own row pair of k (and q) from the
                // registers, so the two operands of a unit share one set of exponentials.
                static_assert(7 * K * sizeof(float) <= 2 * 16 * LDK * sizeof(S), "pair factors fit the left-operand rows");
                if (tid < K) {  // f_IJ of the pairs (0,0) (1,1) (2,2) (3,3) (2,0) (3,0) (3,1), physical column order
                    const int c = tid, pc = perm<MT>(c);
                    const float G0 = sg[15 * K + c], G1 = sg[31 * K + c], G2 = sg[47 * K + c], G3 = sg[63 * K + c];
                    float* fp = FP(Lay::k_fp);
                    fp[0 * K + pc] = exp_f32(-G0);
                    fp[1 * K + pc] = exp_f32(G0 - G1);
                    fp[2 * K + pc] = exp_f32(G1 - G2);
                    fp[3 * K + pc] = exp_f32(G2 - G3);
                    fp[4 * K + pc] = exp_f32(G1 - G0);
                    fp[5 * K + pc] = exp_f32(G2 - G0);
                    fp[6 * K + pc] = exp_f32(G2 - G1);
                }
                // The diagonal of P is q_r . k_r: its decay factor is exactly 1, but the scaled bf16
                // operands would round each factor on its own, which under cancellation (a small q_r . k_r)
                // leaves a large relative error in a one-token output.  It is summed here from the unscaled
                // rows in fp32 (partial sums of the 8 lanes of a row pair, one per 64-channel block, in the
                // W area, free until D) and replaces the MFMA value below.
                float* const sdg = FP(Lay::k_w);
                static_assert(K / 64 * CH * sizeof(float) <= Lay::ROWK, "diagonal partial sums fit the W area");
#pragma unroll
                for (int i = 0; i < PK::NPASS; ++i) {
                    if (!PK::valid(tid, i)) continue;
                    const int c8 = PK::col(tid, i), r0 = 2 * PK::pair(tid, i), I = r0 >> 4;
                    float dqa = 0.0f, dqb = 0.0f;  // this lane's part of q_r0 . k_r0 and q_r0+1 . k_r0+1
                    // two halves of four channels keep the temporaries few
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int c4 = c8 + 4 * hh;
                        const f32x4_t ga = *reinterpret_cast<const f32x4_t*>(sg + r0 * K + c4);
                        const f32x4_t gb = *reinterpret_cast<const f32x4_t*>(sg + (r0 + 1) * K + c4);
                        const f32x4_t g0 = I ? *reinterpret_cast<const f32x4_t*>(sg + (16 * I - 1) * K + c4)
                                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
                        const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(sg + (16 * I + 15) * K + c4);
                        float ka[4], kb[4], la[4], lb[4], y[4];
                        kr[2 * i].get4(ka, hh);
                        kr[2 * i + 1].get4(kb, hh);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            la[e] = exp_f32(ga[e] - g0[e]);
                            lb[e] = exp_f32(gb[e] - g0[e]);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = ka[e] * la[e];
                        st4f_perm<MT>(sK + r0 * LDK, c4, y);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = kb[e] * lb[e];
                        st4f_perm<MT>(sK + (r0 + 1) * LDK, c4, y);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = ka[e] * exp_f32(g1[e] - ga[e]);
                        st4f_perm<MT>(sRG + r0 * LDK, c4, y);
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[e] = kb[e] * exp_f32(g1[e] - gb[e]);
                        st4f_perm<MT>(sRG + (r0 + 1) * LDK, c4, y);
                        if (want_o) {  // P only feeds the output
                            qr[2 * i].get4(y, hh);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                dqa = fmaf(y[e], ka[e], dqa);
                                y[e] *= la[e];
                            }
                            st4f_perm<MT>(sQ + r0 * LDK, c4, y);
                            qr[2 * i + 1].get4(y, hh);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                dqb = fmaf(y[e], kb[e], dqb);
                                y[e] *= lb[e];
                            }
                            st4f_perm<MT>(sQ + (r0 + 1) * LDK, c4, y);
                        }
                    }
                    if (want_o) {  // the 8 lanes of the row pair (consecutive lanes, whole waves valid or not)
                        dqa += dpp_mov<0xB1>(dqa);   // quad_perm [1,0,3,2]
                        dqb += dpp_mov<0xB1>(dqb);
                        dqa += dpp_mov<0x4E>(dqa);   // quad_perm [2,3,0,1]
                        dqb += dpp_mov<0x4E>(dqb);
                        dqa += dpp_mov<0x141>(dqa);  // row_half_mirror: the other quad of the 8 lanes
                        dqb += dpp_mov<0x141>(dqb);
                        if ((tid & 7) == 0) {
                            const int blk = (c8 / 64) * CH;
                            sdg[blk + r0] = dqa;
                            sdg[blk + r0 + 1] = dqb;
                        }
                    }
                }
                __syncthreads();
                // the pairs (I, J): L and P tiles share the scaled right operand.  Waves 0-3 take the
                // diagonal pair (w, w) and invert their diagonal block of L right away; the six
                // off-diagonal pairs go to waves 4.. (or, with four waves, to the same waves afterwards).
                const float* fperm = FP(Lay::k_fp);
                auto do_pair = [&](int I, int J) {
                    const int fi = J == I ? I : J == I - 1 ? -1 : (I == 2 ? 4 : (J == 0 ? 5 : 6));
                    f32x4_t cl = {0.f, 0.f, 0.f, 0.f}, cp = {0.f, 0.f, 0.f, 0.f};
                    // transposed products: lane (g, i) holds row 16I + i, columns 16J + 4g .. +3, so each
                    // lane writes its four entries of L and of P with one store each
                    if (want_o)
                        nt2_bscaled<MT, K, true, true>(cl, sK + 16 * I * LDK, cp, sQ + 16 * I * LDK, LDK,
                                                       sRG + 16 * J * LDK, LDK, fi >= 0 ? fperm + fi * K : nullptr);
                    else  // no outputs: P is not needed
                        nt2_bscaled<MT, K, false, true>(cl, sK + 16 * I * LDK, cp, sQ + 16 * I * LDK, LDK,
                                                        sRG + 16 * J * LDK, LDK, fi >= 0 ? fperm + fi * K : nullptr);
                    const int r = 16 * I + lr, c4 = 4 * g4;
                    const float br = sb[r];
                    float lv[4], pv[4];
                    if (J < I) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) lv[e] = -br * cl[e];
                        st4f<MT>(sLo + r * LDO + 16 * J + c4, lv);
                        if (want_o) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) pv[e] = cp[e];
                            st4f_perm<MT>(sP + r * LDT, 16 * J + c4, pv);
                        }
                    } else {  // diagonal blocks: L in fp32, strictly lower, for the inversion; P lower
                        *reinterpret_cast<f32x4_t*>(sLd + I * 16 * LDN + lr * LDN + c4) =
                            f32x4_t{c4 < lr ? br * cl[0] : 0.0f, c4 + 1 < lr ? br * cl[1] : 0.0f,
                                    c4 + 2 < lr ? br * cl[2] : 0.0f, c4 + 3 < lr ? br * cl[3] : 0.0f};
                        if (want_o) {
                            float dg = sdg[r];  // q_r . k_r from the unscaled rows
#pragma unroll
                            for (int b = 1; b < K / 64; ++b) dg += sdg[b * CH + r];
#pragma unroll
                            for (int e = 0; e < 4; ++e) pv[e] = c4 + e == lr ? dg : c4 + e < lr ? cp[e] : 0.0f;
                            st4f_perm<MT>(sP + r * LDT, 16 * I + c4, pv);
                        }
                    }
                };
                if (w < 4) {
                    do_pair(w, w);
                    // the block's LDS writes complete before this wave's lanes read other lanes' entries
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    invert_unit_lower_16<MT>(sLd + w * 16 * LDN, sD + 16 * w * LDD, LDD);
                }
                constexpr int OW = NW > 4 ? NW - 4 : NW;  // waves that take off-diagonal pairs
                for (int q = NW > 4 ? w - 4 : w; q < 6; q += OW) {
                    if (q < 0) break;
                    int I, J;
                    strict_tile(q, I, J);
                    do_pair(I, J);
                }
                __syncthreads();
            } else {
                // raw rows for the element-wise form
#pragma unroll
                for (int i = 0; i < PK::NPASS; ++i) {
                    if (!PK::valid(tid, i)) continue;
                    const int c8 = PK::col(tid, i), pr0 = 2 * PK::pair(tid, i);
                    st8_perm<MT, IO>(sK + pr0 * LDK, c8, kr[2 * i]);
                    st8_perm<MT, IO>(sK + (pr0 + 1) * LDK, c8, kr[2 * i + 1]);
                    if (want_o) {
                        st8_perm<MT, IO>(sQ + pr0 * LDK, c8, qr[2 * i]);
                        st8_perm<MT, IO>(sQ + (pr0 + 1) * LDK, c8, qr[2 * i + 1]);
                    }
                }
                __syncthreads();
                // diagonal 16x16 blocks, element-wise: (r, j) in the same block, j <= r
                for (int p = tid; p < 4 * 256; p += NTHR) {
                    const int b = p >> 8, rr = (p >> 4) & 15, jj = p & 15;
                    const int r = 16 * b + rr, j = 16 * b + jj;
                    float accp = 0.0f, accl = 0.0f;
                    if (jj <= rr) {
                        for (int c = 0; c < K; ++c) {
                            const int pc = perm<MT>(c);
                            const float d = exp_f32(sg[r * K + c] - sg[j * K + c]);
                            const float kj = M::back(sK[j * LDK + pc]) * d;
                            if (want_o) accp = fmaf(M::back(sQ[r * LDK + pc]), kj, accp);
                            accl = fmaf(M::back(sK[r * LDK + pc]), kj, accl);
                        }
                    }
                    sP[r * LDT + perm<MT>(j)] = M::cvt(accp);  // zero above the diagonal
                    sLd[b * 16 * LDN + rr * LDN + jj] = (jj < rr) ? sb[r] * accl : 0.0f;
                }
                // off-diagonal blocks (I > J) through MFMA, reference point rho = gamma[16I - 1]
                for (int I = 1; I < 4; ++I) {
                    const int rho_row = 16 * I - 1;
                    for (int idx = tid; idx < 16 * K; idx += NTHR) {
                        const int r = idx / K, c = idx % K, rr = 16 * I + r, pc = perm<MT>(c);
                        const float f = exp_f32(sg[rr * K + c] - sg[rho_row * K + c]);
                        sLK[r * LDK + pc] = M::cvt(M::back(sK[rr * LDK + pc]) * f);
                        if (want_o) sLQ[r * LDK + pc] = M::cvt(M::back(sQ[rr * LDK + pc]) * f);
                    }
                    for (int idx = tid; idx < 16 * I * K; idx += NTHR) {
                        const int j = idx / K, c = idx % K, pc = perm<MT>(c);
                        sRG[j * LDK + pc] =
                            M::cvt(M::back(sK[j * LDK + pc]) * exp_f32(sg[rho_row * K + c] - sg[j * K + c]));
                    }
                    __syncthreads();
                    for (int t = w; t < 2 * I; t += NW) {
                        const int J = t >> 1;
                        const bool isL = (t & 1) == 0;
                        if (!want_o && !isL) continue;
                        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                        M::nt(acc, isL ? sLK : sLQ, LDK, sRG + 16 * J * LDK, LDK, K);
    #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * I + 4 * g4 + e, j = 16 * J + lr;
                            if (isL) sLo[r * LDO + j] = M::cvt(-sb[r] * acc[e]);
                            else sP[r * LDT + perm<MT>(j)] = M::cvt(acc[e]);
                        }
                    }
                    __syncthreads();
                }
                if (w < 4) invert_unit_lower_16<MT>(sLd + w * 16 * LDN, sD + 16 * w * LDD, LDD);
            }
            // the transposed / scaled operands of D and E, from this chunk's registers (the scaled rows
            // of B are dead): (K e^gamma)^T, (K e^(gamma_last - gamma))^T and Q e^gamma from one row pair
            // and 8 channels per unit, V^T
            S* sKgT = SP(Lay::k_kgt);
            S* sVT = SP(Lay::k_vt);
            S* sQt = SP(Lay::k_qt);
            S* sKdT = SP(Lay::k_kdt);
#pragma unroll
            for (int i = 0; i < PK::NPASS; ++i) {
                if (PK::valid(tid, i)) {
                    const int c8 = PK::col(tid, i), pr0 = 2 * PK::pair(tid, i);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int c4 = c8 + 4 * hh;
                        const f32x4_t ga = *reinterpret_cast<const f32x4_t*>(sg + pr0 * K + c4);
                        const f32x4_t gb = *reinterpret_cast<const f32x4_t*>(sg + (pr0 + 1) * K + c4);
                        const f32x4_t gl = *reinterpret_cast<const f32x4_t*>(sg + (CH - 1) * K + c4);
                        float ka[4], kb[4], ea[4], eb[4];
                        kr[2 * i].get4(ka, hh);
                        kr[2 * i + 1].get4(kb, hh);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            ea[e] = exp_f32(ga[e]);
                            eb[e] = exp_f32(gb[e]);
                            const float ya = ka[e] * ea[e], yb = kb[e] * eb[e];
                            const float da = ka[e] * exp_f32(gl[e] - ga[e]), db = kb[e] * exp_f32(gl[e] - gb[e]);
                            if constexpr (Lay::BF) {
                                *reinterpret_cast<uint32_t*>(sKgT + (c4 + e) * LDT + perm<MT>(pr0)) = pack_bf16x2(ya, yb);
                                *reinterpret_cast<uint32_t*>(sKdT + (c4 + e) * LDT + perm<MT>(pr0)) = pack_bf16x2(da, db);
                            } else {
                                sKgT[(c4 + e) * LDT + pr0] = ya;
                                sKgT[(c4 + e) * LDT + pr0 + 1] = yb;
                                sKdT[(c4 + e) * LDT + pr0] = da;
                                sKdT[(c4 + e) * LDT + pr0 + 1] = db;
                            }
                        }
                        if (want_o) {  // Q e^gamma only feeds the output
                            float y[4];
                            qr[2 * i].get4(y, hh);
#pragma unroll
                            for (int e = 0; e < 4; ++e) y[e] *= ea[e];
                            st4f_perm<MT>(sQt + pr0 * LDK, c4, y);
                            qr[2 * i + 1].get4(y, hh);
#pragma unroll
                            for (int e = 0; e < 4; ++e) y[e] *= eb[e];
                            st4f_perm<MT>(sQt + (pr0 + 1) * LDK, c4, y);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < PV::NPASS; ++i) {
                if (PV::valid(tid, i))
                    st_pair_t<MT, IO>(sVT, LDT, PV::col(tid, i), 2 * PV::pair(tid, i), vr[2 * i], vr[2 * i + 1]);
            }
            for (int c = tid; c < K; c += NTHR) FP(Lay::k_gl)[c] = exp_f32(sg[(CH - 1) * K + c]);
        }
        __syncthreads();

        // ===== D: [W | U] = (I + L)^-1 [beta e^gamma K | beta V] by blocked substitution =====
        if constexpr (PER_K) {
            if (ci + 1 < nc) load_q(ci + 1);
        }
        if (ci + 1 < nc) load_k(ci + 1);
        f32x4_t nu[4];
        {
            const S* sKb = SP(PER_K ? Lay::k_kgt : Lay::g_kt);
            const S* sVb = SP(PER_K ? Lay::k_vt : Lay::g_vt);
            const float* wsc = PER_K ? sb : FP(Lay::g_be);
            auto store_w = [&](int jt, const f32x4_t* X) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sW[(16 * i + 4 * g4 + e) * LDK + perm<MT>(16 * jt + lr)] = M::cvt(-X[i][e]);
            };
            if constexpr (TRK) {
                // one W tile and the U tile per wave, solved together, both read straight from the
                // row-major K and V copies through transposing LDS reads
                static_assert(KT == NW, "one W tile per wave");
                const uint16_t* sVr = SP(Lay::g_vt);
                f32x4_t X[2][4];
                const RhsFromRows rhs[2] = {{sK, LDK, 16 * w, wsc}, {sVr, Lay::LDV, 16 * w, sb}};
                block_solve<MT, 2>(X, sLo, LDO, sD, LDD, rhs);
                store_w(w, X[0]);
#pragma unroll
                for (int i = 0; i < 4; ++i) nu[i] = X[1][i];
            } else if constexpr (KT == NW) {
                // one W tile and the U tile per wave, solved together
                f32x4_t X[2][4];
                const RhsFromTransposed<MT> rhs[2] = {{sKb + (16 * w + lr) * LDT, wsc}, {sVb + (16 * w + lr) * LDT, sb}};
                block_solve<MT, 2>(X, sLo, LDO, sD, LDD, rhs);
                store_w(w, X[0]);
#pragma unroll
                for (int i = 0; i < 4; ++i) nu[i] = X[1][i];
            } else {
                for (int jt = w; jt < KT; jt += NW) {
                    f32x4_t X[1][4];
                    if constexpr (KROW) {
                        const RhsFromRowsF32 rhs[1] = {{FP(Lay::g_k), LDK, 16 * jt, wsc}};
                        block_solve<MT, 1>(X, sLo, LDO, sD, LDD, rhs);
                    } else {
                        const RhsFromTransposed<MT> rhs[1] = {{sKb + (16 * jt + lr) * LDT, wsc}};
                        block_solve<MT, 1>(X, sLo, LDO, sD, LDD, rhs);
                    }
                    store_w(jt, X[0]);
                }
                f32x4_t X[1][4];
                const RhsFromTransposed<MT> rhs[1] = {{sVb + (16 * w + lr) * LDT, sb}};
                block_solve<MT, 1>(X, sLo, LDO, sD, LDD, rhs);
#pragma unroll
                for (int i = 0; i < 4; ++i) nu[i] = X[0][i];
            }
        }
        __syncthreads();

        // ===== E: v_new, output, state update (wave w: columns 16w .. 16w+15) =====
        // v_new = U - W S^T (LDS holds -W) and, when outputs are wanted, the Q S^T part of
        // O = scale (diag(e^gamma) Q S^T + P v_new): one packing of the state feeds both
        if constexpr (MAP) {
            // both states: v_new = U - W S^T and, for the map rows (U = 0), -W M^T; then the decays and
            // the rank-64 updates with (K e^(gamma_last - gamma))^T, each LDS operand read once
            f32x4_t nm[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) nm[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            gemm_regs_2b<MT, K, 4>(nu, hs, nm, hm, sW, LDK);
            if (ci + 1 < nc) load_vgb(ci + 1);
            if constexpr (PER_K) {
                const float* sgl = FP(Lay::k_gl);
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float d = sgl[16 * kt + 4 * g4 + e];
                        hs[kt][e] *= d;
                        hm[kt][e] *= d;
                    }
                gemm_regs_2b<MT, CH, KT>(hs, nu, hm, nm, SP(Lay::k_kdt), LDT);
            } else {
                // scalar gate: S <- e^{gamma_last} S + K^T (v_new * e^{gamma_last - gamma}), the K^T operand read
                // from the row-major K rows with transposing reads, once for both states
                static_assert(!MAP || TRK, "the paired scalar-gate run reads K^T from the row-major K rows");
                const float dec = FP(Lay::g_eg)[CH - 1];
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hs[kt][e] *= dec;
                        hm[kt][e] *= dec;
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4_t f = *reinterpret_cast<const f32x4_t*>(FP(Lay::g_ed) + 16 * i + 4 * g4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        nu[i][e] *= f[e];
                        nm[i][e] *= f[e];
                    }
                }
#pragma unroll
                for (int m = 0; m < CH / 32; ++m) {
                    const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, uint4{pack_tile_lo(nu[2 * m]), pack_tile_hi(nu[2 * m]),
                                                                          pack_tile_lo(nu[2 * m + 1]),
                                                                          pack_tile_hi(nu[2 * m + 1])});
                    const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, uint4{pack_tile_lo(nm[2 * m]), pack_tile_hi(nm[2 * m]),
                                                                          pack_tile_lo(nm[2 * m + 1]),
                                                                          pack_tile_hi(nm[2 * m + 1])});
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const uint2 lo = ld_tr4<true>(sK, LDK, 32 * m + 4 * g4, 16 * kt);
                        const uint2 hi = ld_tr4<true>(sK, LDK, 32 * m + 16 + 4 * g4, 16 * kt);
                        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, uint4{lo.x, lo.y, hi.x, hi.y});
                        hs[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0, hs[kt], 0, 0, 0);
                        hm[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, hm[kt], 0, 0, 0);
                    }
                }
            }
            __syncthreads();
            continue;
        }
        // the output tiles are formed transposed: lane (g, i) holds token 16t + i, value columns
        // 16w + 4g .. +3, written to the staging area with one store per tile
        f32x4_t oa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) oa[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (want_o) gemm_regs2<MT, K, 4, true>(nu, sW, oa, SP(PER_K ? Lay::k_qt : Lay::g_q), LDK, hs);
        else gemm_regs<MT, K, 4>(nu, sW, LDK, hs);
        if (ci + 1 < nc) load_vgb(ci + 1);
        if (want_o) {
        if constexpr (!PER_K) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = FP(Lay::g_eg)[16 * i + lr];
#pragma unroll
                for (int e = 0; e < 4; ++e) oa[i][e] *= f;
            }
        }
        gemm_regs<MT, CH, 4, true, true>(oa, sP, LDT, nu);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            {
                const int r = 16 * i + lr, c = 16 * w + 4 * g4;  // four adjacent columns, inside one granule
                if constexpr (std::is_same<IO, float>::value)
                    *reinterpret_cast<f32x4_t*>(so + OS::off(r, c)) =
                        f32x4_t{a.scale * oa[i][0], a.scale * oa[i][1], a.scale * oa[i][2], a.scale * oa[i][3]};
                else
                    *reinterpret_cast<uint2*>(so + OS::off(r, c)) =
                        uint2{pack_bf16x2(a.scale * oa[i][0], a.scale * oa[i][1]),
                              pack_bf16x2(a.scale * oa[i][2], a.scale * oa[i][3])};
            }
        }
        }
        // S <- e^{gamma_last} S + sum_r v_new_r (k_r e^{gamma_last - gamma_r})^T
        if constexpr (!PER_K) {
            const float dec = FP(Lay::g_eg)[CH - 1];
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hs[kt][e] *= dec;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t f = *reinterpret_cast<const f32x4_t*>(FP(Lay::g_ed) + 16 * i + 4 * g4);
#pragma unroll
                for (int e = 0; e < 4; ++e) nu[i][e] *= f[e];
            }
            if constexpr (TRK) {
                // hs[kt] += K[:, 16 kt ..]^T v_new~ with the A operand read from the row-major K rows:
                // MFMA position 8 (l/16) + e is chunk row 32m + 4 (l/16) + e or 32m + 16 + 4 (l/16) + e - 4
#pragma unroll
                for (int m = 0; m < CH / 32; ++m) {
                    const uint4 bw = {pack_tile_lo(nu[2 * m]), pack_tile_hi(nu[2 * m]), pack_tile_lo(nu[2 * m + 1]),
                                      pack_tile_hi(nu[2 * m + 1])};
                    const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const uint2 lo = ld_tr4<true>(sK, LDK, 32 * m + 4 * g4, 16 * kt);
                        const uint2 hi = ld_tr4<true>(sK, LDK, 32 * m + 16 + 4 * g4, 16 * kt);
                        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, uint4{lo.x, lo.y, hi.x, hi.y});
                        hs[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, hs[kt], 0, 0, 0);
                    }
                }
            } else if constexpr (KROW) {
                // hs[kt] += K[:, 16 kt ..]^T v_new~: A[c][t] = K[t][c] read with transposed indexing
                const float* sKf = FP(Lay::g_k);
#pragma unroll
                for (int t = 0; t < CH / 16; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt)
                            hs[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sKf[(16 * t + 4 * g4 + e) * LDK + 16 * kt + lr],
                                                                          nu[t][e], hs[kt], 0, 0, 0);
            } else {
                gemm_regs<MT, CH, KT>(hs, SP(Lay::g_kt), LDT, nu);
            }
        } else {
            const float* sgl = FP(Lay::k_gl);
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int e = 0; e < 4; ++e) hs[kt][e] *= sgl[16 * kt + 4 * g4 + e];
            gemm_regs<MT, CH, KT>(hs, SP(Lay::k_kdt), LDT, nu);
        }
        __syncthreads();
    }
    if (nc > 0) {
        const int64_t bos = s0 + (int64_t)CH * (nc - 1);
        flush_o(bos, (int)(s1 - bos));
    }

    if (a.ht) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) *reinterpret_cast<f32x4_t*>(a.ht + sidx + 16 * kt + 4 * g4) = hs[kt];
    }
    if constexpr (MAP) {
        float* const dm = a.map + (((int64_t)n * a.HV + h) * K + 16 * w + lr) * K;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) *reinterpret_cast<f32x4_t*>(dm + 16 * kt + 4 * g4) = hm[kt];
    }
}

// ---------------------------------------------------------------------------
// Flow form for the common case (scalar gate, bf16 operands, K = V = 128): v_new is solved from the
// state directly, so no W is formed.  With R = diag(beta) V - diag(beta e^gamma) K S^T,
//
//     v_new = (I + L)^-1 R,
//
// which equals U - W S^T of the WY form: one triangular solve per chunk instead of two (one for U,
// one for W).  The solve sits on the state-dependent path, but it is short: 20 products of
// 16x16x16 per wave over four block rows.  Every iteration has two workgroup barriers:
//
//            waves 0-3 (state, 32 columns each)              waves 4-7 (prep)
//   phase X  E1(c-1): Y = K S^T and S Q^T from one packing   loads of chunk c + 2 into registers;
//            of the state, R, v_new, the state update        L(c), the four diagonal inverses and
//                                                            the four diagonal P tiles of chunk c
//   phase Y  E2(c-1): the P v_new part of the output and     chunk c + 1 from registers into LDS,
//            its stores; the six off-diagonal P tiles of c   its gate tables
//
// Q, K, V, -L, the inverses, P and the gate tables are double-buffered, and the prep waves keep two
// register sets of raw rows, so a chunk's loads are in flight for about three phases (issued during
// phase X two iterations ahead, written to LDS in the phase Y of the iteration before its use).  L
// and P tiles are formed transposed (K_J K_I^T, K_J Q_I^T), so that each lane holds four consecutive
// columns of one row and writes them with one 8-byte store.  The output scale is folded into the e^gamma table
// and into P.
//
// Lazy decay: the state waves hold S / sigma.  The prep waves, which form the gate tables in chunk
// order, track sigma (the product of the chunk decays e^{gamma_last}) and fold it into the factors
// that touch the state: beta e^gamma sigma_c for R, scale e^gamma sigma_c for the output, and
// e^{gamma_last - gamma} / sigma_{c+1} for the update.  When sigma would fall below 2^-40 (or
// underflow, with the strongest decays), the chunk's table asks the state waves to multiply the
// registers by sigma_c e^{gamma_last} and sigma restarts at 1; the final state is written as
// sigma * registers.  This replaces a multiply of the whole state by e^{gamma_last} in every chunk.
struct FlowLayout {
    static constexpr int K = 128, V = 128;
    static constexpr int LDK = K + 16, LDT = CH + 16, LDO = CH + 16, LDD = 16 + 8;
    static constexpr size_t ROWK = 2 * CH * LDK;          // [64][LDK] bf16
    static constexpr size_t ROWT = 2 * CH * LDT;          // [64][LDT] bf16
    static constexpr size_t ROWO = 2 * (CH - 16) * LDO;   // rows 16..63 of -L (row 0..15 has no off-diagonal block)
    static constexpr size_t ROWD = 2 * CH * LDD;          // the four 16x16 diagonal inverses, bf16
    static constexpr int TABF = 9 * CH + 4;               // floats per gate-table set
    static constexpr int t_g = 0, t_b = CH, t_be = 2 * CH, t_egs = 3 * CH, t_ed = 4 * CH, t_fa = 5 * CH, t_fb = 8 * CH,
                         t_x = 9 * CH;                    // [0] explicit state rescale of the chunk, [1] sigma after it
    static constexpr size_t q0 = 0;                       // Q rows, two buffers
    static constexpr size_t k0 = q0 + 2 * ROWK;           // K rows, two buffers
    static constexpr size_t v0 = k0 + 2 * ROWK;           // V rows, two buffers
    static constexpr size_t lo = v0 + 2 * ROWK;           // -L off-diagonal blocks, two buffers
    static constexpr size_t dd = lo + 2 * ROWO;           // diagonal inverses, two buffers
    static constexpr size_t ld = dd + 2 * ROWD;           // diagonal blocks of L, fp32 (prep scratch)
    static constexpr size_t p0 = ld + sizeof(float) * 4 * 16 * LDN;  // P rows, two buffers
    static constexpr size_t tab = p0 + 2 * ROWT;          // gate tables, two sets
    static constexpr size_t total = tab + 2 * sizeof(float) * TABF;
};

template <typename IO>
__global__ __launch_bounds__(512) void chunk_flow_kernel(const ChunkArgs a) {
    typedef FlowLayout L;
    typedef MM<bf16_t> M;
    typedef uint16_t S;
    constexpr int K = L::K, KT = K / 16;
    constexpr int LDK = L::LDK, LDT = L::LDT, LDO = L::LDO, LDD = L::LDD;
    static_assert(L::total <= 160 * 1024, "LDS budget");
    static_assert(std::is_same<IO, bf16_t>::value, "bf16 I/O");
    __shared__ __align__(16) char smem[L::total];
    auto SP = [&](size_t off) { return reinterpret_cast<S*>(smem + off); };
    auto FP = [&](size_t off) { return reinterpret_cast<float*>(smem + off); };

    const int h = blockIdx.y, n = blockIdx.z;
    const int tid = threadIdx.x, l = tid & 63, g4 = l >> 4, lr = l & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
    const int64_t s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : a.T;
    const int nc = (int)((s1 - s0 + CH - 1) / CH);
    // without outputs (the segment runs of context parallelism) the S Q^T products, P and the output
    // stage are left out.  A run-time flag on purpose: as a template parameter the branch-free product
    // loop measured about 4% slower end to end
    const bool want_o = a.o != nullptr;
    auto chunk_len = [&](int ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        return (s1 - bos) < CH ? (int)(s1 - bos) : CH;
    };
    float* const sLd = FP(L::ld);
#ifdef GDR_FLOW_STAMPS
    const bool rec = (int)n == g_flow_target[0] && (int)h == g_flow_target[1] && l == 0;
#else
    constexpr bool rec = false;
#endif
    FLOW_WG_CLOCK(true);

    if (w < 4) {
        // ================= state waves =================
        // hs[j][kt][e] = S[32w + 16j + lane%16][16kt + 4(l/16) + e]
        f32x4_t hs[2][KT];
        const int64_t sbase = ((int64_t)n * a.HV + h) * a.V * K;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                hs[j][kt] = a.h0 ? *reinterpret_cast<const f32x4_t*>(a.h0 + sbase + (int64_t)(32 * w + 16 * j + lr) * K +
                                                                    16 * kt + 4 * g4)
                                 : f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t ot[2][4];   // O^T tiles of chunk c - 1 between E1 and E2: lane (g, i) holds value columns
                            // 32w + 16j + 4g .. +3 of token 16i + lane%16
        uint4 na[2][2];     // v_new of chunk c - 1 packed as the A operand of the P v_new product
        // zero the strictly upper tiles of both P buffers once (the P v_new product reads (0,1) and (2,3))
        for (int idx = tid; idx < 2 * CH * CH; idx += 256) {
            const int b = idx / (CH * CH), r = (idx / CH) % CH, j = idx % CH;
            if ((j >> 4) > (r >> 4)) SP(L::p0 + b * L::ROWT)[r * LDT + perm<bf16_t>(j)] = M::cvt(0.0f);
        }
        __syncthreads();  // prologue: chunk 0 staged, tables of chunk 0 formed
        for (int it = 0; it <= nc; ++it) {
            const int b1 = it & 1, b0 = b1 ^ 1;  // buffers of chunk it and of chunk it - 1
            // ===== phase X: E1(it - 1) =====
            if (it >= 1) {
                const S* sQ0 = SP(L::q0 + b0 * L::ROWK);
                const S* sK0 = SP(L::k0 + b0 * L::ROWK);
                const S* sV0 = SP(L::v0 + b0 * L::ROWK);
                const S* sLo0 = SP(L::lo + b0 * L::ROWO);
                const S* sD0 = SP(L::dd + b0 * L::ROWD);
                const float* tb0 = FP(L::tab) + b0 * L::TABF;
                // Y[r][v] = sum_k K[r][k] S[v][k] and O^T[v][r] = sum_k S[v][k] Q[r][k], sharing each packing of S
                f32x4_t y[2][4];
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        ot[j][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                for (int m = 0; m < K / 32; ++m) {
                    bf16x8_t av[4], bq[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        av[i] = *reinterpret_cast<const bf16x8_t*>(sK0 + (16 * i + lr) * LDK + 32 * m + 8 * g4);
                        if (want_o) bq[i] = *reinterpret_cast<const bf16x8_t*>(sQ0 + (16 * i + lr) * LDK + 32 * m + 8 * g4);
                    }
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const bf16x8_t sv = __builtin_bit_cast(
                            bf16x8_t, uint4{pack_tile_lo(hs[j][2 * m]), pack_tile_hi(hs[j][2 * m]),
                                            pack_tile_lo(hs[j][2 * m + 1]), pack_tile_hi(hs[j][2 * m + 1])});
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            y[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], sv, y[j][i], 0, 0, 0);
                            if (want_o) ot[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sv, bq[i], ot[j][i], 0, 0, 0);
                        }
                    }
                }
                FLOW_STAMP(rec && w == 0, 0, it, 5);  // products done
                // R = beta V - beta e^gamma Y (rows 16I + 4(l/16) + e, column 32w + 16j + lane%16), then
                // v_new = (I + L)^-1 R by blocked forward substitution (-L and the inverses from LDS)
                s16x4_t lv[6], dv[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    dv[I] = *reinterpret_cast<const s16x4_t*>(sD0 + (16 * I + lr) * LDD + 4 * g4);
#pragma unroll
                    for (int J = 0; J < I; ++J)
                        lv[I * (I - 1) / 2 + J] =
                            *reinterpret_cast<const s16x4_t*>(sLo0 + (16 * I - 16 + lr) * LDO + 16 * J + 4 * g4);
                }
                f32x4_t x[2][4];
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    const int t0 = 16 * I + 4 * g4;
                    const f32x4_t bb = *reinterpret_cast<const f32x4_t*>(tb0 + L::t_b + t0);
                    const f32x4_t be = *reinterpret_cast<const f32x4_t*>(tb0 + L::t_be + t0);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint2 vr = ld_tr4<true>(sV0, LDK, t0, 32 * w + 16 * j);
                        const float vv[4] = {__uint_as_float(vr.x << 16), __uint_as_float(vr.x & 0xFFFF0000u),
                                             __uint_as_float(vr.y << 16), __uint_as_float(vr.y & 0xFFFF0000u)};
#pragma unroll
                        for (int e = 0; e < 4; ++e) y[j][I][e] = fmaf(-be[e], y[j][I][e], bb[e] * vv[e]);
                    }
                }
#pragma unroll
                for (int I = 0; I < 4; ++I) {
#pragma unroll
                    for (int J = 0; J < I; ++J)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const s16x4_t bv = __builtin_bit_cast(s16x4_t, uint2{pack_tile_lo(x[j][J]), pack_tile_hi(x[j][J])});
                            y[j][I] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lv[I * (I - 1) / 2 + J], bv, y[j][I], 0, 0, 0);
                        }
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const s16x4_t rv = __builtin_bit_cast(s16x4_t, uint2{pack_tile_lo(y[j][I]), pack_tile_hi(y[j][I])});
                        x[j][I] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dv[I], rv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    }
                }
                FLOW_STAMP(rec && w == 0, 0, it, 6);  // R and the solve done
                if (want_o) {
                    // the S Q^T part scaled by scale e^gamma_r; v_new packed for E2
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float f = tb0[L::t_egs + 16 * i + lr];
#pragma unroll
                        for (int j = 0; j < 2; ++j) ot[j][i] *= f;
                    }
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int m = 0; m < 2; ++m)
                            na[j][m] = uint4{pack_tile_lo(x[j][2 * m]), pack_tile_hi(x[j][2 * m]),
                                             pack_tile_lo(x[j][2 * m + 1]), pack_tile_hi(x[j][2 * m + 1])};
                }
                // S <- e^{gamma_last} S + sum_r v_new_r (k_r e^{gamma_last - gamma_r})^T, the K^T operand read
                // from the row-major K rows with transposing reads
                // the registers hold S / sigma; the decay of the chunk only moves sigma, except when sigma would
                // leave the safe range: then the table holds the factor that folds it into the registers
                const float resc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tb0[L::t_x])));
                if (resc != 1.0f) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int kt = 0; kt < KT; ++kt) hs[j][kt] *= resc;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4_t f = *reinterpret_cast<const f32x4_t*>(tb0 + L::t_ed + 16 * i + 4 * g4);
#pragma unroll
                    for (int j = 0; j < 2; ++j) x[j][i] *= f;
                }
#pragma unroll
                for (int m = 0; m < CH / 32; ++m) {
                    bf16x8_t bw[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        bw[j] = __builtin_bit_cast(bf16x8_t, uint4{pack_tile_lo(x[j][2 * m]), pack_tile_hi(x[j][2 * m]),
                                                                   pack_tile_lo(x[j][2 * m + 1]),
                                                                   pack_tile_hi(x[j][2 * m + 1])});
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const uint2 lo = ld_tr4<true>(sK0, LDK, 32 * m + 4 * g4, 16 * kt);
                        const uint2 hi = ld_tr4<true>(sK0, LDK, 32 * m + 16 + 4 * g4, 16 * kt);
                        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, uint4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                        for (int j = 0; j < 2; ++j) hs[j][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw[j], hs[j][kt], 0, 0, 0);
                    }
                }
            }
            FLOW_STAMP(rec && w == 0, 0, it, 0);
            __syncthreads();  // end of phase X
            FLOW_STAMP(rec && w == 0, 0, it, 1);
            // ===== phase Y: E2(it - 1), then the off-diagonal P tiles of chunk it =====
            if (it >= 1 && want_o) {
                const int ce = it - 1;
                const int64_t bos = s0 + (int64_t)CH * ce;
                const int len = chunk_len(ce);
                const S* sP0 = SP(L::p0 + b0 * L::ROWT);
                // O^T_j += v_new^T P^T (P holds scale e^{gamma_r - gamma_t} q_r . k_t); P is lower triangular:
                // token tile i needs the steps m with 32m <= 16i + 15
                bf16x8_t bp[2][4];
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (32 * m <= 16 * i + 15)
                            bp[m][i] = *reinterpret_cast<const bf16x8_t*>(sP0 + (16 * i + lr) * LDT + 32 * m + 8 * g4);
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const bf16x8_t nv = __builtin_bit_cast(bf16x8_t, na[j][m]);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (32 * m <= 16 * i + 15)
                                ot[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nv, bp[m][i], ot[j][i], 0, 0, 0);
                    }
                // rows g and g + 1 of a lane pair exchange halves (v_permlane16_swap), so that each lane holds
                // eight consecutive value columns of its token: columns 32w + {0, 16, 8, 24}[g] .. +7, one 16-byte
                // store per token tile, 64 contiguous bytes per token and store instruction
                // written through (device scope, not read again in the call) by a buffer store over the chunk's
                // len token rows: rows past a short chunk's end fall outside the range and are dropped
                const int ostride = a.HV * a.V;
                const int ocol = 32 * w + ((g4 & 1) ? 16 + 4 * (g4 - 1) : 4 * g4);
                const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint16_t*>(a.o) + (bos * a.HV + h) * a.V, 0, len * ostride * 2, 0x00020000);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x0 = pack_bf16x2(ot[0][i][0], ot[0][i][1]), x1 = pack_bf16x2(ot[0][i][2], ot[0][i][3]);
                    const uint32_t y0 = pack_bf16x2(ot[1][i][0], ot[1][i][1]), y1 = pack_bf16x2(ot[1][i][2], ot[1][i][3]);
                    const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
                    const int r = 16 * i + lr;
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{s0[0], s1[0], s0[1], s1[1]}, ors,
                                                           (uint32_t)(r * ostride * 2 + ocol * 2), 0, kWriteThrough);
                }
            }
            FLOW_STAMP(rec && w == 0, 0, it, 4);  // the output part done
            if (it < nc && want_o) {
                // the six off-diagonal P tiles of chunk it (the prep waves form the diagonal ones), transposed
                // products K_J Q_I^T: lane (g, i) holds P[16I + lane%16][16J + 4g + e]
                const S* sQ1 = SP(L::q0 + b1 * L::ROWK);
                const S* sK1 = SP(L::k0 + b1 * L::ROWK);
                S* const sP1 = SP(L::p0 + b1 * L::ROWT);
                const float* tb1 = FP(L::tab) + b1 * L::TABF;
                auto store_off = [&](int q, const f32x4_t& cp) {
                    int I, J;
                    strict_tile(q, I, J);
                    const int r = 16 * I + lr;
                    const float fa = tb1[L::t_fa + J * CH + r] * a.scale;
                    const f32x4_t fb = *reinterpret_cast<const f32x4_t*>(tb1 + L::t_fb + 16 * J + 4 * g4);
                    *reinterpret_cast<uint2*>(sP1 + r * LDT + perm<bf16_t>(16 * J + 4 * g4)) =
                        uint2{pack_bf16x2(fa * fb[0] * cp[0], fa * fb[1] * cp[1]),
                              pack_bf16x2(fa * fb[2] * cp[2], fa * fb[3] * cp[3])};
                };
                int I0, J0;
                strict_tile(w, I0, J0);
                f32x4_t c0 = {0.f, 0.f, 0.f, 0.f};
                M::nt(c0, sK1 + 16 * J0 * LDK, LDK, sQ1 + 16 * I0 * LDK, LDK, K);
                store_off(w, c0);
                if (w < 2) {
                    int I1, J1;
                    strict_tile(w + 4, I1, J1);
                    f32x4_t c1 = {0.f, 0.f, 0.f, 0.f};
                    M::nt(c1, sK1 + 16 * J1 * LDK, LDK, sQ1 + 16 * I1 * LDK, LDK, K);
                    store_off(w + 4, c1);
                }
            }
            FLOW_STAMP(rec && w == 0, 0, it, 2);
            __syncthreads();  // end of phase Y
            FLOW_STAMP(rec && w == 0, 0, it, 3);
        }
        FLOW_WG_CLOCK(false);
        if (a.ht) {
            // S = sigma * registers, sigma after the last chunk (1 for an empty sequence)
            const float sig = nc > 0 ? FP(L::tab)[((nc - 1) & 1) * L::TABF + L::t_x + 1] : 1.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int kt = 0; kt < KT; ++kt)
                    *reinterpret_cast<f32x4_t*>(a.ht + sbase + (int64_t)(32 * w + 16 * j + lr) * K + 16 * kt + 4 * g4) =
                        hs[j][kt] * sig;
        }
    } else {
        // ================= prep waves =================
        constexpr int NLD = 256;
        const int lt = tid - 256;  // thread index among waves 4-7
        const int u = w - 4;
        const int hk = h / (a.HV / a.HK);
        typedef Tile<CH, K, NLD> TQ;
        typedef PairTile<K, NLD> PK;
        typedef PairTile<128, NLD> PV;
        // one chunk's q, k, v rows (and, on wave 4, g and beta) held raw in registers; two sets, so that
        // the loads of chunk c + 2 are in flight while chunk c + 1 is written to LDS
        struct Regs {
            Raw8<IO> qn[TQ::NV], kn[2 * PK::NPASS], vn[2 * PV::NPASS];
            float gn;
            uint32_t bn;
        };
        Regs ra, rb;
        // sigma: the state waves hold S / sigma.  The tables of chunk c carry sigma_c (the value at the start of
        // the chunk) in beta e^gamma and scale e^gamma, and 1 / sigma_{c+1} in e^{gamma_last - gamma}; sigma
        // follows the chunk decays and is folded back into the registers (reset to 1) whenever it would fall
        // below 2^-40, so that every factor stays far from overflow and underflow
        float sig = 1.0f;
        constexpr int ESZ = 2;
        const int qk_row = a.HK * K * ESZ, v_row = a.HV * a.V * ESZ;
        // global -> registers: the parts of chunk ci named in `part` (q: 1, k: 2, v with g and beta: 4)
        auto load = [&](int ci, Regs& r, int part) {
            const int64_t bos = s0 + (int64_t)CH * ci;
            const int len = chunk_len(ci);
            if (part & 1) {
                // without outputs q reads as zeros (a zero-byte range): it only feeds P and the output
                const __amdgpu_buffer_rsrc_t rq =
                    chunk_rsrc(want_o ? static_cast<const char*>(a.q) + ((bos * a.HK + hk) * K) * ESZ : nullptr,
                               want_o ? len : 0, qk_row);
#pragma unroll
                for (int i = 0; i < TQ::NV; ++i) r.qn[i].template load<kNonTemporal>(rq, TQ::row(lt, i) * qk_row + TQ::col(lt) * ESZ);
            }
            if (part & 2) {
                const __amdgpu_buffer_rsrc_t rk =
                    chunk_rsrc(static_cast<const char*>(a.k) + ((bos * a.HK + hk) * K) * ESZ, len, qk_row);
#pragma unroll
                for (int i = 0; i < PK::NPASS; ++i)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        r.kn[2 * i + q].template load<kNonTemporal>(rk, (2 * PK::pair(lt, i) + q) * qk_row + PK::col(lt, i) * ESZ);
            }
            if (part & 4) {
                // v == NULL reads as zeros (a zero-byte range): the run that forms a segment's linear map
                const __amdgpu_buffer_rsrc_t rv =
                    chunk_rsrc(a.v ? static_cast<const char*>(a.v) + ((bos * a.HV + h) * a.V) * ESZ : nullptr,
                               a.v ? len : 0, v_row);
#pragma unroll
                for (int i = 0; i < PV::NPASS; ++i)
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        r.vn[2 * i + q].template load<kNonTemporal>(rv, (2 * PV::pair(lt, i) + q) * v_row + PV::col(lt, i) * ESZ);
                if (u == 0) {
                    const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(a.g + bos * a.HV + h, len, a.HV * 4);
                    r.gn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, l * a.HV * 4, 0, 0));
                    const __amdgpu_buffer_rsrc_t rbt =
                        chunk_rsrc(static_cast<const char*>(a.beta) + (bos * a.HV + h) * 2, len, a.HV * 2);
                    r.bn = __builtin_amdgcn_raw_buffer_load_b16(rbt, l * a.HV * 2, 0, 0);
                }
            }
        };
        auto stage = [&](int b, const Regs& r) {  // registers -> LDS buffers b; wave 4 forms the gate tables
            S* const sQ = SP(L::q0 + b * L::ROWK);
            S* const sK = SP(L::k0 + b * L::ROWK);
            S* const sV = SP(L::v0 + b * L::ROWK);
#pragma unroll
            for (int i = 0; i < TQ::NV; ++i) st8_perm<bf16_t, IO>(sQ + TQ::row(lt, i) * LDK, TQ::col(lt), r.qn[i]);
#pragma unroll
            for (int i = 0; i < PK::NPASS; ++i) {
                if (PK::valid(lt, i)) {
                    const int c8 = PK::col(lt, i), pr0 = 2 * PK::pair(lt, i);
                    st8_perm<bf16_t, IO>(sK + pr0 * LDK, c8, r.kn[2 * i]);
                    st8_perm<bf16_t, IO>(sK + (pr0 + 1) * LDK, c8, r.kn[2 * i + 1]);
                }
            }
#pragma unroll
            for (int i = 0; i < PV::NPASS; ++i) {
                if (PV::valid(lt, i)) {
                    const int c8 = PV::col(lt, i), pr0 = 2 * PV::pair(lt, i);
                    st8_perm<bf16_t, IO>(sV + pr0 * LDK, c8, r.vn[2 * i]);
                    st8_perm<bf16_t, IO>(sV + (pr0 + 1) * LDK, c8, r.vn[2 * i + 1]);
                }
            }
            if (u == 0) {  // inclusive prefix of the 64 gates (rows past the end are 0) and the factor tables
                float* const tb = FP(L::tab) + b * L::TABF;
                const float br = __uint_as_float(r.bn << 16);
                const float x = wave_inclusive_sum(r.gn);
                const float xl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), CH - 1));
                const float ex = exp_f32(x);
                const float prod = sig * exp_f32(xl);          // sigma_c times the chunk's decay
                const bool fold = !(prod >= 0x1p-40f);
                const float sig_next = fold ? 1.0f : prod;
                tb[L::t_g + l] = x;
                tb[L::t_b + l] = br;
                tb[L::t_be + l] = br * ex * sig;
                tb[L::t_egs + l] = a.scale * ex * sig;
                tb[L::t_ed + l] = exp_f32(xl - x) * __builtin_amdgcn_rcpf(sig_next);
                if (l == 0) {
                    tb[L::t_x] = fold ? prod : 1.0f;
                    tb[L::t_x + 1] = sig_next;
                }
                sig = sig_next;
                float rho[4];
#pragma unroll
                for (int J = 0; J < 4; ++J) rho[J] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16 * J + 15));
#pragma unroll
                for (int J = 0; J < 3; ++J) tb[L::t_fa + J * CH + l] = exp_f32(fminf(x - rho[J], 0.0f));
                const int jb = l >> 4;
                const float rj = jb == 0 ? rho[0] : jb == 1 ? rho[1] : jb == 2 ? rho[2] : rho[3];
                tb[L::t_fb + l] = exp_f32(rj - x);
            }
        };
        // phase X of iteration it: L of chunk it (transposed products K_J K_I^T), the diagonal inverses and
        // the diagonal P tiles (taken off the state waves, whose phase Y bounded the iteration), with the
        // loads of chunk it + 2 into the register set written to LDS in the previous phase: q and k before
        // the tile work, v, g and beta after the inverses.  Issued at the end of the phase, the loads left
        // too little time on the heads whose rows sit where memory answers slowest, and those heads set
        // the kernel's end; issued all at once at the start, they stalled the wave behind the memory
        // queue.  Split, no head lags.
        auto phase_x = [&](int it, Regs& nxt) {
            const int b1 = it & 1;
            FLOW_STAMP(rec && w == 4, 1, it, 5);
            if (it + 2 < nc) load(it + 2, nxt, 1 | 2);
            FLOW_STAMP(rec && w == 4, 1, it, 6);
            if (it < nc) {
                const S* sK1 = SP(L::k0 + b1 * L::ROWK);
                S* const sLo1 = SP(L::lo + b1 * L::ROWO);
                S* const sD1 = SP(L::dd + b1 * L::ROWD);
                const float* tb1 = FP(L::tab) + b1 * L::TABF;
                auto store_off = [&](int q, const f32x4_t& cl) {
                    int I, J;
                    strict_tile(q, I, J);
                    const int r = 16 * I + lr;
                    const float fr = -tb1[L::t_b + r] * tb1[L::t_fa + J * CH + r];
                    const f32x4_t fb = *reinterpret_cast<const f32x4_t*>(tb1 + L::t_fb + 16 * J + 4 * g4);
                    *reinterpret_cast<uint2*>(sLo1 + (r - 16) * LDO + 16 * J + 4 * g4) =
                        uint2{pack_bf16x2(fr * fb[0] * cl[0], fr * fb[1] * cl[1]),
                              pack_bf16x2(fr * fb[2] * cl[2], fr * fb[3] * cl[3])};
                };
                int I0, J0;
                strict_tile(u, I0, J0);
                f32x4_t cd = {0.f, 0.f, 0.f, 0.f}, c0 = {0.f, 0.f, 0.f, 0.f};
                M::template nt2<K>(cd, sK1 + 16 * u * LDK, sK1 + 16 * u * LDK, c0, sK1 + 16 * J0 * LDK, sK1 + 16 * I0 * LDK,
                                   LDK);
                const S* sQ1 = SP(L::q0 + b1 * L::ROWK);
                S* const sP1 = SP(L::p0 + b1 * L::ROWT);
                f32x4_t cq = {0.f, 0.f, 0.f, 0.f};  // the diagonal P tile, K_u Q_u^T
                M::nt(cq, sK1 + 16 * u * LDK, LDK, sQ1 + 16 * u * LDK, LDK, K);
                float* sN = sLd + u * 16 * LDN;
                {
                    const int r = 16 * u + lr;
                    const float gr = tb1[L::t_g + r], br = tb1[L::t_b + r];
                    const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(tb1 + L::t_g + 16 * u + 4 * g4);
                    f32x4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = br * exp_f32(gr - gj[e]) * cd[e];  // inf above the diagonal is discarded
                        x[e] = (lr > 4 * g4 + e) ? v : 0.0f;
                    }
                    *reinterpret_cast<f32x4_t*>(sN + lr * LDN + 4 * g4) = x;
                }
                // the tile's LDS writes complete before this wave's lanes read other lanes' entries
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                invert_unit_lower_16<bf16_t>(sN, sD1 + 16 * u * LDD, LDD);
                FLOW_STAMP(rec && w == 4, 1, it, 4);
                if (it + 2 < nc) load(it + 2, nxt, 4);
                FLOW_STAMP(rec && w == 4, 1, it, 7);
                store_off(u, c0);
                if (u < 2) {
                    int I1, J1;
                    strict_tile(u + 4, I1, J1);
                    f32x4_t c1 = {0.f, 0.f, 0.f, 0.f};
                    M::nt(c1, sK1 + 16 * J1 * LDK, LDK, sK1 + 16 * I1 * LDK, LDK, K);
                    store_off(u + 4, c1);
                }
                {   // the diagonal P tile of chunk it: scale e^{gamma_r - gamma_t} k_t . q_r, r >= t
                    const int r = 16 * u + lr;
                    const float gr = tb1[L::t_g + r];
                    const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(tb1 + L::t_g + 16 * u + 4 * g4);
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = exp_f32(gr - gj[e]) * cq[e] * a.scale;  // inf above the diagonal is discarded
                        x[e] = (lr >= 4 * g4 + e) ? v : 0.0f;
                    }
                    *reinterpret_cast<uint2*>(sP1 + r * LDT + perm<bf16_t>(16 * u + 4 * g4)) =
                        uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                }
            }
            FLOW_STAMP(rec && w == 4, 1, it, 0);
            __syncthreads();  // end of phase X
            FLOW_STAMP(rec && w == 4, 1, it, 1);
        };
        // phase Y of iteration it: chunk it + 1 from registers into LDS
        auto phase_y = [&](int it, const Regs& cur) {
            if (it + 1 < nc) stage((it & 1) ^ 1, cur);
            FLOW_STAMP(rec && w == 4, 1, it, 2);
            __syncthreads();  // end of phase Y
            FLOW_STAMP(rec && w == 4, 1, it, 3);
        };
        if (nc > 0) {
            load(0, ra, 7);
            stage(0, ra);
        }
        if (nc > 1) load(1, rb, 7);
        __syncthreads();  // prologue
        // chunk c lives in register set ra for even c, rb for odd c
        for (int it = 0; it <= nc; it += 2) {
            phase_x(it, ra);
            phase_y(it, rb);
            if (it + 1 <= nc) {
                phase_x(it + 1, rb);
                phase_y(it + 1, ra);
            }
        }
    }
}

template <int K, int V, typename IO, bool PER_K>
hipError_t launch_fused(const ChunkArgs& a, hipStream_t stream) {
    // bf16: the workgroup owns all V columns; fp32 operands (K = 64 only) use 64-column tiles
    constexpr int BV = std::is_same<IO, float>::value ? 64 : V;
    if constexpr (K == 128 && V == 128 && std::is_same<IO, bf16_t>::value && !PER_K) {
        hipLaunchKernelGGL(chunk_flow_kernel<IO>, dim3(1, a.HV, a.N), dim3(512), 0, stream, a);
    } else {
        hipLaunchKernelGGL((chunk_fused_kernel<K, BV, IO, IO, PER_K>), dim3(V / BV, a.HV, a.N), dim3(4 * BV), 0,
                           stream, a);
    }
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_kv(const ChunkArgs& a, int io, bool per_k, hipStream_t s) {
    if (a.map) {  // the paired offset/map run of the segmented route
        if constexpr (K == V) {
            if (io == 1) {
                if (per_k)
                    hipLaunchKernelGGL((chunk_fused_kernel<K, V, bf16_t, bf16_t, true, true>), dim3(1, a.HV, a.N),
                                       dim3(4 * V), 0, s, a);
                else
                    hipLaunchKernelGGL((chunk_fused_kernel<K, V, bf16_t, bf16_t, false, true>), dim3(1, a.HV, a.N),
                                       dim3(4 * V), 0, s, a);
                return hipGetLastError();
            }
        }
        return hipErrorNotSupported;
    }
    if (io == 0) {
        // fp32 operands: every shape with the scalar gate; the per-channel gate at K = 128 does not
        // fit the 160 KiB of LDS in this design
        if constexpr (K == 64) return per_k ? launch_fused<K, V, float, true>(a, s) : launch_fused<K, V, float, false>(a, s);
        else return per_k ? hipErrorNotSupported : launch_fused<K, V, float, false>(a, s);
    }
    return per_k ? launch_fused<K, V, bf16_t, true>(a, s) : launch_fused<K, V, bf16_t, false>(a, s);
}

}  // namespace

#ifdef GDR_FLOW_STAMPS
extern "C" __attribute__((visibility("default"))) int gdr_dbg_flow_target(int seq, int head) {
    const int t[2] = {seq, head};
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_flow_target), t, sizeof(t), 0, hipMemcpyHostToDevice);
}
extern "C" __attribute__((visibility("default"))) int gdr_dbg_flow_stamps(void* stamps, void* wg) {
    hipError_t e = hipMemcpyFromSymbol(stamps, HIP_SYMBOL(g_flow_stamps), sizeof(g_flow_stamps), 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpyFromSymbol(wg, HIP_SYMBOL(g_flow_wg), sizeof(g_flow_wg), 0, hipMemcpyDeviceToHost);
    return (int)e;
}
#endif

hipError_t launch_chunk(const ChunkArgs& a, int io_dtype, bool per_k, hipStream_t stream) {
    if (a.K == 64) {
        return a.V == 64 ? launch_kv<64, 64>(a, io_dtype, per_k, stream) : launch_kv<64, 128>(a, io_dtype, per_k, stream);
    }
    return a.V == 64 ? launch_kv<128, 64>(a, io_dtype, per_k, stream) : launch_kv<128, 128>(a, io_dtype, per_k, stream);
}

}  // namespace gdr
