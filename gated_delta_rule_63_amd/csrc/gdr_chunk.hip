// Chunked gated delta rule for gfx950: 64-token chunks, WY/UT form.
//
// Stages (each a kernel, launched back to back on the caller's stream):
//   index    chunk -> sequence map for a packed varlen batch (one small workgroup)
//   H2       per (chunk, head): chunk-local cumulative gate gamma, the strictly lower
//            L = beta * (K K^T) * decay, A = (I + L)^-1, W = A diag(beta) (K * e^gamma),
//            U = A diag(beta) V                                  -> gamma, W, U to workspace
//   H3       per (sequence, head, 64-wide V tile), sequential over the sequence's chunks:
//            v_new = U - W S^T,  S <- S * e^{gamma_last} + v_new^T (K * e^{gamma_last - gamma})
//            with the state S held in MFMA accumulators    -> chunk-start states, v_new
//   H4       per (chunk, head): O = scale * ((Q * e^gamma) S0^T + P v_new),
//            P[r][j] = q_r . k_j * decay(r, j) for j <= r
//
// Method: the chunked algorithm that the cuLA PR #113 ("[GDN2] Add Hopper SM90 CuTe DSL
// prefill") and attention-gym PR #344 ("Replace the KDA inter-chunk recurrence with a
// warp-specialized kernel") pages build on (kkt/solve/A, w, u, per-chunk h, v_new), written
// out from the token recurrence.  Overflow: every exponential evaluated here has a
// non-positive argument -- (later - earlier) prefix differences or a prefix itself --
// so no exp(-prefix) factor exists (cuLA PR #113 review, finding P1).  For the per-key-channel
// gate the decay cannot be pulled out of K K^T / Q K^T as a matrix factor; off-diagonal
// 16x16 blocks use a reference point rho (the prefix at the last row before the block row):
// exp(g_r - g_j) = exp(g_r - rho) * exp(rho - g_j), both factors <= 1, so they become MFMA
// operands; the four diagonal 16x16 blocks are evaluated element-wise.
//
// MFMA: bf16 I/O uses v_mfma_f32_16x16x32_bf16, fp32 I/O uses v_mfma_f32_16x16x4f32
// (fp32-accurate products).  Accumulation is fp32 throughout.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int CH = 64;  // chunk length

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// MFMA tile products on LDS operands, "NT" form: C[i][j] += sum_k A[i][k] * Bt[j][k]
// with A and Bt both row-major over the reduction index.  sA / sB point at the first
// row of the 16-row tile.  C layout: lane l holds C[4*(l/16) + e][l%16], e = 0..3.
template <typename MT> struct MM;

template <> struct MM<bf16_t> {
    typedef uint16_t S;  // LDS element
    static constexpr int PAD = 8;
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
    __device__ __forceinline__ static void st8(S* p, const float* x) {
        f32x4_t* q = reinterpret_cast<f32x4_t*>(p);
        q[0] = f32x4_t{x[0], x[1], x[2], x[3]};
        q[1] = f32x4_t{x[4], x[5], x[6], x[7]};
    }
};

struct ChunkInfo {
    int64_t bos;
    int len;
    int n;
};

__device__ __forceinline__ bool chunk_info(const ChunkArgs& a, int c, ChunkInfo& ci) {
    const int n = a.chunk_seq[c];
    if (n < 0) return false;
    const int64_t s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
    const int64_t s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : a.T;
    ci.n = n;
    ci.bos = s0 + (int64_t)CH * (c - a.chunk_first[n]);
    const int64_t rem = s1 - ci.bos;
    ci.len = rem < CH ? (int)rem : CH;
    return true;
}

// Eight consecutive elements held raw in registers, so that a whole tile's worth of
// global loads can be issued before any of them is used.  Rows past the end of a chunk
// are loaded from a clamped (valid) row and zeroed on conversion: a conditional load
// would be compiled as a branch with an immediate wait on every load.
template <typename IO> struct Raw8;
template <> struct Raw8<bf16_t> {
    uint4 w;
    __device__ __forceinline__ void load(const void* p, int64_t off) {
        w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + off);
    }
    __device__ __forceinline__ void get(float* x, bool valid) const {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = valid ? __uint_as_float(ws[j] << 16) : 0.0f;
            x[2 * j + 1] = valid ? __uint_as_float(ws[j] & 0xFFFF0000u) : 0.0f;
        }
    }
};
template <> struct Raw8<float> {
    f32x4_t a, b;
    __device__ __forceinline__ void load(const void* p, int64_t off) {
        const f32x4_t* q = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + off);
        a = q[0];
        b = q[1];
    }
    __device__ __forceinline__ void get(float* x, bool valid) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = valid ? a[e] : 0.0f;
            x[4 + e] = valid ? b[e] : 0.0f;
        }
    }
};

// Ownership of a [64][D] row-major tile by 256 threads in vectors of 8 elements:
// thread t holds NV = D/32 vectors, all in the same 8-column slot.
template <int D> struct Tile64 {
    static constexpr int VPR = D / 8;          // vectors per row
    static constexpr int NV = D / 32;          // vectors per thread
    static constexpr int RSTEP = 256 / VPR;    // row step between a thread's vectors
    __device__ __forceinline__ static int row(int tid, int i) { return tid / VPR + RSTEP * i; }
    __device__ __forceinline__ static int col(int tid) { return (tid % VPR) * 8; }
};

// Chunk-local cumulative gate into LDS (and optionally to the workspace).
// Scalar gate: sg[64]; per-K gate: sg[64][K].  Rows >= len repeat the last prefix.
template <int K, bool PER_K>
__device__ __forceinline__ void load_gamma(const ChunkArgs& a, const ChunkInfo& ci, int h, float* sg, bool from_ws,
                                           bool write_ws) {
    const int tid = threadIdx.x;
    if constexpr (!PER_K) {
        if (tid < 64) {
            const int r = tid;
            const int rc = r < ci.len ? r : ci.len - 1;
            const int64_t idx = (ci.bos + rc) * a.HV + h;
            float x;
            if (from_ws) {
                x = a.gcum[idx];
            } else {
                x = a.g[idx];
                x = r < ci.len ? x : 0.0f;
                // inclusive prefix sum across the 64 lanes of wave 0
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const float y = __shfl_up(x, d, 64);
                    if (r >= d) x += y;
                }
                if (write_ws && r < ci.len) a.gcum[idx] = x;
            }
            sg[r] = x;
        }
    } else {
        // thread (c, quarter): 16 rows of one channel, loads issued as a batch
        static_assert(K * 4 >= 256 || K * 4 == 256 || K == 64, "per-K gamma mapping");
        constexpr int Q = 256 / K;            // row groups per channel (2 for K=128, 4 for K=64)
        constexpr int RPQ = CH / Q;           // rows per group
        __shared__ float part[Q][K];
        const int c = tid % K, qd = tid / K;
        float vals[RPQ];
#pragma unroll
        for (int i = 0; i < RPQ; ++i) {
            const int r = qd * RPQ + i;
            const int rc = r < ci.len ? r : ci.len - 1;
            vals[i] = from_ws ? a.gcum[((ci.bos + rc) * a.HV + h) * K + c] : a.g[((ci.bos + rc) * a.HV + h) * K + c];
        }
        if (from_ws) {
#pragma unroll
            for (int i = 0; i < RPQ; ++i) sg[(qd * RPQ + i) * K + c] = vals[i];
        } else {
            float x = 0.0f;
#pragma unroll
            for (int i = 0; i < RPQ; ++i) {
                const int r = qd * RPQ + i;
                x += r < ci.len ? vals[i] : 0.0f;
                vals[i] = x;
            }
            part[qd][c] = x;
            __syncthreads();
            float off = 0.0f;
            for (int j = 0; j < qd; ++j) off += part[j][c];
#pragma unroll
            for (int i = 0; i < RPQ; ++i) {
                const int r = qd * RPQ + i;
                const float y = vals[i] + off;
                sg[r * K + c] = y;
                if (write_ws && r < ci.len) a.gcum[((ci.bos + r) * a.HV + h) * K + c] = y;
            }
        }
    }
}

template <int K, bool PER_K>
__device__ __forceinline__ float gam(const float* sg, int r, int c) {
    if constexpr (PER_K) return sg[r * K + c];
    else return sg[r];
}

// Decayed dot products for the per-K gate, the 16x16 diagonal blocks of a 64x64 matrix:
// out[r][j] = sum_c x_r[c] y_j[c] exp(g_r[c] - g_j[c]) for j < r (j <= r when INCL), same block.
template <int K, typename MT, bool INCL>
__device__ void diag_blocks_per_k(const typename MM<MT>::S* sX, int ldx, const typename MM<MT>::S* sY, int ldy,
                                  const float* sg, float* out, int ldo, const float* rowscale) {
    // 4 blocks x 16 x 16 (r, j) pairs; one thread per pair, masked pairs skipped
    for (int p = threadIdx.x; p < 4 * 256; p += blockDim.x) {
        const int b = p >> 8, rr = (p >> 4) & 15, jj = p & 15;
        const int r = 16 * b + rr, j = 16 * b + jj;
        if (INCL ? (jj > rr) : (jj >= rr)) continue;
        float acc = 0.0f;
        for (int c = 0; c < K; ++c) {
            const float d = exp_f32(sg[r * K + c] - sg[j * K + c]);
            acc = fmaf(MM<MT>::back(sX[r * ldx + c]) * MM<MT>::back(sY[j * ldy + c]), d, acc);
        }
        out[r * ldo + j] = rowscale ? rowscale[r] * acc : acc;
    }
}

// Off-diagonal blocks (I > J) for the per-K gate through MFMA with reference point
// rho_I = gamma[16*I - 1]:  left = X_I * exp(gamma_I - rho_I), right = Y_{<16I} * exp(rho_I - gamma).
template <int K, typename MT>
__device__ void offdiag_blocks_per_k(const typename MM<MT>::S* sX, int ldx, const typename MM<MT>::S* sY, int ldy,
                                     const float* sg, typename MM<MT>::S* sLft, typename MM<MT>::S* sRgt,
                                     float* out, int ldo, const float* rowscale) {
    typedef typename MM<MT>::S S;
    constexpr int LD = K + MM<MT>::PAD;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    for (int I = 1; I < 4; ++I) {
        const int rho_row = 16 * I - 1;
        for (int idx = tid; idx < 16 * K; idx += blockDim.x) {
            const int r = idx / K, c = idx % K;
            const float rho = sg[rho_row * K + c];
            const int rr = 16 * I + r;
            sLft[r * LD + c] = MM<MT>::cvt(MM<MT>::back(sX[rr * ldx + c]) * exp_f32(sg[rr * K + c] - rho));
        }
        for (int idx = tid; idx < 16 * I * K; idx += blockDim.x) {
            const int j = idx / K, c = idx % K;
            const float rho = sg[rho_row * K + c];
            sRgt[j * LD + c] = MM<MT>::cvt(MM<MT>::back(sY[j * ldy + c]) * exp_f32(rho - sg[j * K + c]));
        }
        __syncthreads();
        for (int J = w; J < I; J += 4) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            MM<MT>::nt(acc, sLft, LD, sRgt + 16 * J * LD, LD, K);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * I + 4 * (l >> 4) + e, j = 16 * J + (l & 15);
                out[r * ldo + j] = rowscale ? rowscale[r] * acc[e] : acc[e];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// index: chunk_first[n] = first chunk of sequence n; chunk_seq[c] = sequence of chunk c.
__global__ __launch_bounds__(1024) void chunk_index_kernel(const ChunkArgs a) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int N = a.N;
    const int per = (N + 1023) / 1024;
    const int n0 = tid * per, n1 = min(N, n0 + per);
    int32_t sum = 0;
    for (int n = n0; n < n1; ++n) {
        const int64_t len = a.cu_seqlens ? (int64_t)a.cu_seqlens[n + 1] - a.cu_seqlens[n] : a.T;
        sum += (int32_t)((len + CH - 1) / CH);
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
        const int32_t y = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += y;
        __syncthreads();
    }
    int32_t first = part[tid] - sum;
    for (int n = n0; n < n1; ++n) {
        const int64_t len = a.cu_seqlens ? (int64_t)a.cu_seqlens[n + 1] - a.cu_seqlens[n] : a.T;
        const int32_t nc = (int32_t)((len + CH - 1) / CH);
        a.chunk_first[n] = first;
        for (int j = 0; j < nc; ++j) a.chunk_seq[first + j] = n;
        first += nc;
    }
    const int32_t total = part[1023];
    if (tid == 0) a.chunk_first[N] = total;
    for (int c = total + tid; c < a.max_chunks; c += 1024) a.chunk_seq[c] = -1;
}

// ---------------------------------------------------------------------------
// H2: intra-chunk WY/UT transform.
// LDS phases: (1) K rows -> L; (2) A = (I + L)^-1 in fp32; (3) W and U on MFMA.  The
// K rows (phase 1) and the transposed operands of phase 3 share one region.
template <int K, int V, typename IO, typename MT, bool PER_K>
struct PrepSmem {
    typedef typename MM<MT>::S S;
    static constexpr int LDK = K + MM<MT>::PAD;     // rows over K
    static constexpr int LDT = CH + MM<MT>::PAD;    // rows over the 64 chunk positions
    static constexpr int LDL = CH + 1;              // fp32 L and A
    static constexpr size_t g_off = 0;                                                // f32 [64] or [64][K]
    static constexpr size_t b_off = g_off + sizeof(float) * CH * (PER_K ? K : 1);     // f32 [64]
    static constexpr size_t l_off = b_off + sizeof(float) * CH;                       // f32 [64][LDL]
    static constexpr size_t a_off = l_off + sizeof(float) * CH * LDL;                 // f32 [64][LDL]
    static constexpr size_t u_off = a_off + sizeof(float) * CH * LDL;                 // union
    // phase 1
    static constexpr size_t k_off = u_off;                                            // S [64][LDK]
    static constexpr size_t lft_off = k_off + sizeof(S) * CH * LDK;
    static constexpr size_t rgt_off = lft_off + (PER_K ? sizeof(S) * 16 * LDK : 0);
    static constexpr size_t ph1_end = rgt_off + (PER_K ? sizeof(S) * 48 * LDK : 0);
    // phase 3
    static constexpr size_t am_off = u_off;                                           // S [64][LDT]
    static constexpr size_t kst_off = am_off + sizeof(S) * CH * LDT;                  // S [K][LDT]
    static constexpr size_t vst_off = kst_off + sizeof(S) * K * LDT;                  // S [V][LDT]
    static constexpr size_t ph3_end = vst_off + sizeof(S) * V * LDT;
    static constexpr size_t total = ph1_end > ph3_end ? ph1_end : ph3_end;
};

// A = (I + L)^-1 for a strictly lower 64x64 L (fp32, row stride LDL) into sA.
// The four unit-lower 16x16 diagonal blocks are inverted by forward substitution; then
// row block by row block, A_IJ = -D_I sum_{M=J}^{I-1} L_IM A_MJ on fp32 MFMA, the two
// products chained in registers (the C layout of the first is the B operand of the
// second once the reduction index runs over rows 4*(l/16) + e, step e).
template <int LDL>
__device__ __forceinline__ void invert_unit_lower_64(const float* sL, float* sA) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4;
    for (int idx = tid; idx < CH * CH; idx += 256) {      // zero the strictly upper blocks
        const int r = idx / CH, j = idx % CH;
        if ((j >> 4) > (r >> 4)) sA[r * LDL + j] = 0.0f;
    }
    if (l < 16) {
        const int b0 = 16 * w, j = l;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.0f : 0.0f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc = fmaf(-sL[(b0 + i) * LDL + b0 + m], x[m], acc);
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[(b0 + i) * LDL + b0 + j] = x[i];
    }
    __syncthreads();
    for (int I = 1; I < 4; ++I) {
        if (w < I) {
            const int J = w;
            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
            for (int M = J; M < I; ++M) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const float av = sL[(16 * I + (l & 15)) * LDL + 16 * M + 4 * st + g4];
                    const float bv = sA[(16 * M + 4 * st + g4) * LDL + 16 * J + (l & 15)];
                    t = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, t, 0, 0, 0);
                }
            }
            f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float av = sA[(16 * I + (l & 15)) * LDL + 16 * I + 4 * g4 + e];
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(av, t[e], x, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sA[(16 * I + 4 * g4 + e) * LDL + 16 * J + (l & 15)] = -x[e];
        }
        __syncthreads();
    }
}

template <int K, int V, typename IO, typename MT, bool PER_K>
__global__ __launch_bounds__(256) void chunk_prepare_kernel(const ChunkArgs a) {
    typedef PrepSmem<K, V, IO, MT, PER_K> L;
    typedef typename MM<MT>::S S;
    __shared__ __align__(16) char smem[L::total];
    float* sg = reinterpret_cast<float*>(smem + L::g_off);
    float* sb = reinterpret_cast<float*>(smem + L::b_off);
    float* sL = reinterpret_cast<float*>(smem + L::l_off);
    float* sA = reinterpret_cast<float*>(smem + L::a_off);
    S* sK = reinterpret_cast<S*>(smem + L::k_off);
    S* sAm = reinterpret_cast<S*>(smem + L::am_off);
    S* sKsT = reinterpret_cast<S*>(smem + L::kst_off);
    S* sVsT = reinterpret_cast<S*>(smem + L::vst_off);

    ChunkInfo ci;
    if (!chunk_info(a, blockIdx.x, ci)) return;
    const int h = blockIdx.y;
    const int hk = h / (a.HV / a.HK);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;

    // all global loads of the chunk first: K and V rows, beta
    typedef Tile64<K> TK;
    typedef Tile64<V> TV;
    Raw8<IO> kr[TK::NV], vr[TV::NV];
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        const int r = TK::row(tid, i), rc = r < ci.len ? r : ci.len - 1;
        kr[i].load(a.k, ((ci.bos + rc) * a.HK + hk) * K + TK::col(tid));
    }
#pragma unroll
    for (int i = 0; i < TV::NV; ++i) {
        const int r = TV::row(tid, i), rc = r < ci.len ? r : ci.len - 1;
        vr[i].load(a.v, ((ci.bos + rc) * a.HV + h) * V + TV::col(tid));
    }
    float bt = 0.0f;
    if (tid < CH) {
        const int rc = tid < ci.len ? tid : ci.len - 1;
        bt = Elem<IO>::load(a.beta, (ci.bos + rc) * a.HV + h);
    }
    load_gamma<K, PER_K>(a, ci, h, sg, false, true);
    if (tid < CH) sb[tid] = tid < ci.len ? bt : 0.0f;
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        float x[8];
        kr[i].get(x, TK::row(tid, i) < ci.len);
        MM<MT>::st8(sK + TK::row(tid, i) * L::LDK + TK::col(tid), x);
    }
    __syncthreads();

    // L = strictly lower beta_r * (k_r . k_j) * decay(r, j)
    if constexpr (!PER_K) {
        for (int t = w; t < 16; t += 4) {
            const int I = t >> 2, J = t & 3;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if (I >= J) MM<MT>::nt(acc, sK + 16 * I * L::LDK, L::LDK, sK + 16 * J * L::LDK, L::LDK, K);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * I + 4 * (l >> 4) + e, j = 16 * J + (l & 15);
                sL[r * L::LDL + j] = (r > j) ? sb[r] * exp_f32(sg[r] - sg[j]) * acc[e] : 0.0f;
            }
        }
    } else {
        S* sLft = reinterpret_cast<S*>(smem + L::lft_off);
        S* sRgt = reinterpret_cast<S*>(smem + L::rgt_off);
        for (int idx = tid; idx < CH * CH; idx += 256) {
            const int r = idx / CH, j = idx % CH;
            if (j >= r) sL[r * L::LDL + j] = 0.0f;
        }
        diag_blocks_per_k<K, MT, false>(sK, L::LDK, sK, L::LDK, sg, sL, L::LDL, sb);
        offdiag_blocks_per_k<K, MT>(sK, L::LDK, sK, L::LDK, sg, sLft, sRgt, sL, L::LDL, sb);
    }
    __syncthreads();

    invert_unit_lower_64<L::LDL>(sL, sA);

    // phase 3 operands: A (MFMA dtype), (beta e^gamma K)^T and (beta V)^T from registers
    for (int idx = tid; idx < CH * CH; idx += 256) {
        const int r = idx / CH, j = idx % CH;
        sAm[r * L::LDT + j] = MM<MT>::cvt(sA[r * L::LDL + j]);
    }
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        const int r = TK::row(tid, i), c8 = TK::col(tid);
        float x[8];
        kr[i].get(x, r < ci.len);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sKsT[(c8 + e) * L::LDT + r] = MM<MT>::cvt(x[e] * sb[r] * exp_f32(gam<K, PER_K>(sg, r, c8 + e)));
    }
#pragma unroll
    for (int i = 0; i < TV::NV; ++i) {
        const int r = TV::row(tid, i), c8 = TV::col(tid);
        float x[8];
        vr[i].get(x, r < ci.len);
#pragma unroll
        for (int e = 0; e < 8; ++e) sVsT[(c8 + e) * L::LDT + r] = MM<MT>::cvt(x[e] * sb[r]);
    }
    __syncthreads();

    // W = A (beta e^gamma K), U = A (beta V)
    constexpr int TW = 4 * (K / 16), TU = 4 * (V / 16);
    for (int t = w; t < TW + TU; t += 4) {
        const bool isw = t < TW;
        const int tt = isw ? t : t - TW;
        const int D = isw ? K : V;
        const int I = tt / (D / 16), J = tt % (D / 16);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        // A is lower triangular: row block I only needs columns below 16*(I+1)
        const int kdim = MM<MT>::PAD == 8 ? ((16 * (I + 1) + 31) / 32) * 32 : 16 * (I + 1);
        MM<MT>::nt(acc, sAm + 16 * I * L::LDT, L::LDT, (isw ? sKsT : sVsT) + 16 * J * L::LDT, L::LDT, kdim);
        void* dst = isw ? a.w : a.u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * I + 4 * (l >> 4) + e, c = 16 * J + (l & 15);
            if (r < ci.len) Elem<IO>::store(dst, ((ci.bos + r) * a.HV + h) * D + c, acc[e]);
        }
    }
}

// ---------------------------------------------------------------------------
// H3: inter-chunk state pass.  A workgroup owns BV = 64*NT value columns of one
// (sequence, head); wave w owns 16*NT of them: v = BV*blockIdx.x + 16*(NT*w + nt) + lane%16.
// The state S[v][k] of a 16-column slice lives in K/16 accumulator tiles: tile kt,
// element e of lane l holds S[v][16*kt + 4*(l/16) + e].  That layout is the MFMA B
// operand of the next product once the reduction index is permuted consistently on the
// A side, so S and v_new never leave registers.  The next chunk's inputs are loaded into
// registers while the current chunk computes.
template <int K, typename MT> struct StateSmem {
    typedef typename MM<MT>::S S;
    static constexpr int LDW = K + MM<MT>::PAD;                  // -W rows [64][LDW]
    static constexpr bool TRANS = sizeof(S) == 2;                // bf16: K_d^T [K][LDT]; fp32: K_d [64][LDW]
    static constexpr int LDT = CH + MM<MT>::PAD;
    static constexpr size_t w_off = 0;
    static constexpr size_t kd_off = w_off + sizeof(S) * CH * LDW;
    static constexpr size_t dec_off = kd_off + (TRANS ? sizeof(S) * K * LDT : sizeof(S) * CH * LDW);
    static constexpr size_t u_off = dec_off + sizeof(float) * K;              // U tile f32 [64][BVMAX+1]
    static constexpr int LDU = 128 + 1;
    static constexpr size_t total = u_off + sizeof(float) * CH * LDU;
};

template <int K, int V, typename IO, typename MT, bool PER_K, int NT>
__global__ __launch_bounds__(256) void chunk_state_kernel(const ChunkArgs a) {
    typedef StateSmem<K, MT> L;
    typedef typename MM<MT>::S S;
    typedef Tile64<K> TK;
    constexpr int BV = 64 * NT;
    __shared__ __align__(16) char smem[L::total];
    S* sW = reinterpret_cast<S*>(smem + L::w_off);
    S* sKd = reinterpret_cast<S*>(smem + L::kd_off);
    float* sDec = reinterpret_cast<float*>(smem + L::dec_off);
    float* sU = reinterpret_cast<float*>(smem + L::u_off);
    typedef Tile64<BV> TU;

    const int h = blockIdx.y, n = blockIdx.z;
    const int hk = h / (a.HV / a.HK);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g4 = l >> 4;
    int vcol[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vcol[nt] = BV * blockIdx.x + 16 * (NT * w + nt) + (l & 15);
    const int64_t s0 = a.cu_seqlens ? a.cu_seqlens[n] : 0;
    const int64_t s1 = a.cu_seqlens ? a.cu_seqlens[n + 1] : a.T;
    const int nc = (int)((s1 - s0 + CH - 1) / CH);
    const int c0 = a.chunk_first[n];
    const int c8 = TK::col(tid);
    constexpr int GE = PER_K ? 8 : 1;

    constexpr int KT = K / 16;
    f32x4_t hs[NT][KT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int64_t sidx = (((int64_t)n * a.HV + h) * V + vcol[nt]) * K;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            if (a.h0) {
                hs[nt][kt] = *reinterpret_cast<const f32x4_t*>(a.h0 + sidx + 16 * kt + 4 * g4);
            } else {
                hs[nt][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    // registers holding the next chunk's inputs (loaded one chunk ahead)
    Raw8<IO> wr[TK::NV], kr[TK::NV], ur[TU::NV];
    float gr[TK::NV][GE], gl[GE], gdec = 0.0f;
    auto prefetch = [&](int ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        const int len = (s1 - bos) < CH ? (int)(s1 - bos) : CH;
        const int64_t last = bos + len - 1;
#pragma unroll
        for (int i = 0; i < TK::NV; ++i) {
            const int r = TK::row(tid, i), rc = r < len ? r : len - 1;
            wr[i].load(a.w, ((bos + rc) * a.HV + h) * K + c8);
            kr[i].load(a.k, ((bos + rc) * a.HK + hk) * K + c8);
#pragma unroll
            for (int e = 0; e < GE; ++e)
                gr[i][e] = PER_K ? a.gcum[((bos + rc) * a.HV + h) * K + c8 + e] : a.gcum[(bos + rc) * a.HV + h];
        }
#pragma unroll
        for (int e = 0; e < GE; ++e) gl[e] = PER_K ? a.gcum[(last * a.HV + h) * K + c8 + e] : a.gcum[last * a.HV + h];
        if (tid < K) gdec = PER_K ? a.gcum[(last * a.HV + h) * K + tid] : a.gcum[last * a.HV + h];
#pragma unroll
        for (int i = 0; i < TU::NV; ++i) {
            const int r = TU::row(tid, i), rc = r < len ? r : len - 1;
            ur[i].load(a.u, ((bos + rc) * a.HV + h) * V + BV * blockIdx.x + TU::col(tid));
        }
    };
    if (nc > 0) prefetch(0);

    for (int ci = 0; ci < nc; ++ci) {
        const int64_t bos = s0 + (int64_t)CH * ci;
        const int len = (s1 - bos) < CH ? (int)(s1 - bos) : CH;
        const int c = c0 + ci;

        // stage -W and the decayed keys K_d = K * e^{gamma_last - gamma} from registers
#pragma unroll
        for (int i = 0; i < TK::NV; ++i) {
            const int r = TK::row(tid, i);
            const bool ok = r < len;
            float x[8], kx[8];
            wr[i].get(x, ok);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = -x[e];
            MM<MT>::st8(sW + r * L::LDW + c8, x);
            kr[i].get(kx, ok);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ge = PER_K ? e : 0;
                const float kd = kx[e] * exp_f32(gl[ge] - gr[i][ge]);
                if constexpr (L::TRANS) sKd[(c8 + e) * L::LDT + r] = MM<MT>::cvt(kd);
                else sKd[r * L::LDW + c8 + e] = MM<MT>::cvt(kd);
            }
        }
        if (tid < K) sDec[tid] = exp_f32(gdec);
#pragma unroll
        for (int i = 0; i < TU::NV; ++i) {
            const int r = TU::row(tid, i), cc = TU::col(tid);
            float x[8];
            ur[i].get(x, r < len);
#pragma unroll
            for (int e = 0; e < 8; ++e) sU[r * L::LDU + cc + e] = x[e];
        }
        if (ci + 1 < nc) prefetch(ci + 1);
        __syncthreads();
        f32x4_t nu[NT][4];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    nu[nt][mt][e] = sU[(16 * mt + 4 * g4 + e) * L::LDU + 16 * (NT * w + nt) + (l & 15)];

        // chunk-start state -> workspace (io dtype), V-major
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t hb = (((int64_t)c * a.HV + h) * V + vcol[nt]) * K;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                float x[4] = {hs[nt][kt][0], hs[nt][kt][1], hs[nt][kt][2], hs[nt][kt][3]};
                Vec<IO, 4>::store(a.hc, hb + 16 * kt + 4 * g4, x);
            }
        }

        // v_new = U - W S^T
        if constexpr (sizeof(S) == 2) {
#pragma unroll
            for (int m = 0; m < K / 32; ++m) {
                bf16x8_t bv[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bv[nt][e] = __builtin_bit_cast(__bf16, f32_to_bf16(hs[nt][2 * m][e]));
                        bv[nt][4 + e] = __builtin_bit_cast(__bf16, f32_to_bf16(hs[nt][2 * m + 1][e]));
                    }
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const S* pa = sW + (16 * mt + (l & 15)) * L::LDW + 32 * m + 4 * g4;
                    const uint2 lo = *reinterpret_cast<const uint2*>(pa);
                    const uint2 hi = *reinterpret_cast<const uint2*>(pa + 16);
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, uint4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        nu[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[nt], nu[nt][mt], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const float av = sW[(16 * mt + (l & 15)) * L::LDW + 16 * kt + 4 * g4 + e];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            nu[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, hs[nt][kt][e], nu[nt][mt], 0, 0, 0);
                    }
                }
            }
        }

        // v_new -> workspace (io dtype)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mt + 4 * g4 + e;
                    if (r < len) Elem<IO>::store(a.vnew, ((bos + r) * a.HV + h) * V + vcol[nt], nu[nt][mt][e]);
                }
            }
        }

        // S <- S * e^{gamma_last} + v_new^T K_d
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = sDec[16 * kt + 4 * g4 + e];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) hs[nt][kt][e] *= d;
            }
        }
        if constexpr (sizeof(S) == 2) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                bf16x8_t bv[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bv[nt][e] = __builtin_bit_cast(__bf16, f32_to_bf16(nu[nt][2 * m][e]));
                        bv[nt][4 + e] = __builtin_bit_cast(__bf16, f32_to_bf16(nu[nt][2 * m + 1][e]));
                    }
                }
#pragma unroll
                for (int kt = 0; kt < KT; ++kt) {
                    const S* pa = sKd + (16 * kt + (l & 15)) * L::LDT + 32 * m + 4 * g4;
                    const uint2 lo = *reinterpret_cast<const uint2*>(pa);
                    const uint2 hi = *reinterpret_cast<const uint2*>(pa + 16);
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, uint4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        hs[nt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[nt], hs[nt][kt], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
#pragma unroll
                    for (int kt = 0; kt < KT; ++kt) {
                        const float av = sKd[(16 * mt + 4 * g4 + e) * L::LDW + 16 * kt + (l & 15)];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            hs[nt][kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, nu[nt][mt][e], hs[nt][kt], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
    }

    if (a.ht) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t sidx = (((int64_t)n * a.HV + h) * V + vcol[nt]) * K;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                *reinterpret_cast<f32x4_t*>(a.ht + sidx + 16 * kt + 4 * g4) = hs[nt][kt];
        }
    }
}

// ---------------------------------------------------------------------------
// H4: chunk output.
template <int K, int V, typename IO, typename MT, bool PER_K>
struct OutSmem {
    typedef typename MM<MT>::S S;
    static constexpr int LDK = K + MM<MT>::PAD;
    static constexpr int LDT = CH + MM<MT>::PAD;
    static constexpr int LDP = CH + 1;
    static constexpr size_t q_off = 0;                                          // S [64][LDK]
    static constexpr size_t p_off = q_off + sizeof(S) * CH * LDK;               // S [64][LDT]
    static constexpr size_t g_off = p_off + sizeof(S) * CH * LDT;               // f32 [64] or [64][K]
    static constexpr size_t pf_off = g_off + sizeof(float) * CH * (PER_K ? K : 1);  // f32 [64][LDP] (per-K only)
    static constexpr size_t u_off = pf_off + (PER_K ? sizeof(float) * CH * LDP : 0);
    // union: phase 1 {K rows, left, right}; phase 2 {S0 [V][LDK], v_new^T [V][LDT]}
    static constexpr size_t k_off = u_off;
    static constexpr size_t lft_off = k_off + sizeof(S) * CH * LDK;
    static constexpr size_t rgt_off = lft_off + (PER_K ? sizeof(S) * 16 * LDK : 0);
    static constexpr size_t ph1_end = rgt_off + (PER_K ? sizeof(S) * 48 * LDK : 0);
    static constexpr size_t s_off = u_off;
    static constexpr size_t nt_off = s_off + sizeof(S) * V * LDK;
    static constexpr size_t ph2_end = nt_off + sizeof(S) * V * LDT;
    static constexpr size_t total = ph1_end > ph2_end ? ph1_end : ph2_end;
};

template <int K, int V, typename IO, typename MT, bool PER_K>
__global__ __launch_bounds__(256) void chunk_output_kernel(const ChunkArgs a) {
    typedef OutSmem<K, V, IO, MT, PER_K> L;
    typedef typename MM<MT>::S S;
    __shared__ __align__(16) char smem[L::total];
    S* sQ = reinterpret_cast<S*>(smem + L::q_off);
    S* sP = reinterpret_cast<S*>(smem + L::p_off);
    float* sg = reinterpret_cast<float*>(smem + L::g_off);
    S* sK = reinterpret_cast<S*>(smem + L::k_off);
    S* sS = reinterpret_cast<S*>(smem + L::s_off);
    S* sNT = reinterpret_cast<S*>(smem + L::nt_off);

    ChunkInfo ci;
    const int c = blockIdx.x;
    if (!chunk_info(a, c, ci)) return;
    const int h = blockIdx.y;
    const int hk = h / (a.HV / a.HK);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;

    // every global load of the chunk is issued first: q, k rows, the chunk-start state, v_new
    typedef Tile64<K> TK;
    typedef Tile64<V> TV;
    constexpr int SNV = (V / 64) * TK::NV;
    Raw8<IO> qr[TK::NV], kr[TK::NV], sr[SNV], nr[TV::NV];
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        const int r = TK::row(tid, i), rc = r < ci.len ? r : ci.len - 1;
        const int64_t off = ((ci.bos + rc) * a.HK + hk) * K + TK::col(tid);
        qr[i].load(a.q, off);
        kr[i].load(a.k, off);
    }
#pragma unroll
    for (int i = 0; i < SNV; ++i) {
        const int vv = 64 * (i / TK::NV) + TK::row(tid, i % TK::NV);
        sr[i].load(a.hc, (((int64_t)c * a.HV + h) * V + vv) * K + TK::col(tid));
    }
#pragma unroll
    for (int i = 0; i < TV::NV; ++i) {
        const int r = TV::row(tid, i), rc = r < ci.len ? r : ci.len - 1;
        nr[i].load(a.vnew, ((ci.bos + rc) * a.HV + h) * V + TV::col(tid));
    }
    load_gamma<K, PER_K>(a, ci, h, sg, true, false);
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        const int r = TK::row(tid, i), c8 = TK::col(tid);
        float x[8];
        qr[i].get(x, r < ci.len);
        MM<MT>::st8(sQ + r * L::LDK + c8, x);
        kr[i].get(x, r < ci.len);
        MM<MT>::st8(sK + r * L::LDK + c8, x);
    }
    __syncthreads();

    // P[r][j] = q_r . k_j * decay(r, j), j <= r
    if constexpr (!PER_K) {
        for (int t = w; t < 16; t += 4) {
            const int I = t >> 2, J = t & 3;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if (I >= J) MM<MT>::nt(acc, sQ + 16 * I * L::LDK, L::LDK, sK + 16 * J * L::LDK, L::LDK, K);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * I + 4 * (l >> 4) + e, j = 16 * J + (l & 15);
                sP[r * L::LDT + j] = MM<MT>::cvt((r >= j) ? exp_f32(sg[r] - sg[j]) * acc[e] : 0.0f);
            }
        }
    } else {
        float* sPf = reinterpret_cast<float*>(smem + L::pf_off);
        S* sLft = reinterpret_cast<S*>(smem + L::lft_off);
        S* sRgt = reinterpret_cast<S*>(smem + L::rgt_off);
        for (int idx = tid; idx < CH * CH; idx += 256) {
            const int r = idx / CH, j = idx % CH;
            if (j > r) sPf[r * L::LDP + j] = 0.0f;
        }
        diag_blocks_per_k<K, MT, true>(sQ, L::LDK, sK, L::LDK, sg, sPf, L::LDP, nullptr);
        offdiag_blocks_per_k<K, MT>(sQ, L::LDK, sK, L::LDK, sg, sLft, sRgt, sPf, L::LDP, nullptr);
        __syncthreads();
        for (int idx = tid; idx < CH * CH; idx += 256) {
            const int r = idx / CH, j = idx % CH;
            sP[r * L::LDT + j] = MM<MT>::cvt(sPf[r * L::LDP + j]);
        }
    }
    __syncthreads();

    // Q~ = Q * e^gamma from registers; S0 and v_new^T into the phase-2 area
#pragma unroll
    for (int i = 0; i < TK::NV; ++i) {
        const int r = TK::row(tid, i), c8 = TK::col(tid);
        float x[8];
        qr[i].get(x, r < ci.len);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= exp_f32(gam<K, PER_K>(sg, r, c8 + e));
        MM<MT>::st8(sQ + r * L::LDK + c8, x);
    }
#pragma unroll
    for (int i = 0; i < SNV; ++i) {
        const int vv = 64 * (i / TK::NV) + TK::row(tid, i % TK::NV);
        float x[8];
        sr[i].get(x, true);
        MM<MT>::st8(sS + vv * L::LDK + TK::col(tid), x);
    }
#pragma unroll
    for (int i = 0; i < TV::NV; ++i) {
        const int r = TV::row(tid, i), c8 = TV::col(tid);
        float x[8];
        nr[i].get(x, r < ci.len);
#pragma unroll
        for (int e = 0; e < 8; ++e) sNT[(c8 + e) * L::LDT + r] = MM<MT>::cvt(x[e]);
    }
    __syncthreads();

    // O = scale * (Q~ S0^T + P v_new)
    for (int t = w; t < 4 * (V / 16); t += 4) {
        const int I = t / (V / 16), J = t % (V / 16);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        MM<MT>::nt(acc, sQ + 16 * I * L::LDK, L::LDK, sS + 16 * J * L::LDK, L::LDK, K);
        const int kdim = MM<MT>::PAD == 8 ? ((16 * (I + 1) + 31) / 32) * 32 : 16 * (I + 1);
        MM<MT>::nt(acc, sP + 16 * I * L::LDT, L::LDT, sNT + 16 * J * L::LDT, L::LDT, kdim);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * I + 4 * (l >> 4) + e, vv = 16 * J + (l & 15);
            if (r < ci.len) Elem<IO>::store(a.o, ((ci.bos + r) * a.HV + h) * V + vv, a.scale * acc[e]);
        }
    }
}

template <int K, int V, typename IO, bool PER_K>
hipError_t launch_all(const ChunkArgs& a, hipStream_t stream) {
    typedef IO MT;
    hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL((chunk_prepare_kernel<K, V, IO, MT, PER_K>), dim3(a.max_chunks, a.HV), dim3(256), 0, stream, a);
    // the state pass is sequential over chunks: one workgroup per (sequence, head) when that
    // already gives a wave per SIMD, otherwise 64-column V tiles for more workgroups
    if (V == 128 && (int64_t)a.N * a.HV >= 128) {
        hipLaunchKernelGGL((chunk_state_kernel<K, V, IO, MT, PER_K, 2>), dim3(1, a.HV, a.N), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL((chunk_state_kernel<K, V, IO, MT, PER_K, 1>), dim3(V / 64, a.HV, a.N), dim3(256), 0, stream,
                           a);
    }
    hipLaunchKernelGGL((chunk_output_kernel<K, V, IO, MT, PER_K>), dim3(a.max_chunks, a.HV), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_kv(const ChunkArgs& a, int io, bool per_k, hipStream_t s) {
    if (io == 0) {
        // fp32 operands at K = 128 do not fit the 160 KiB of LDS in this design
        if constexpr (K == 64) return per_k ? launch_all<K, V, float, true>(a, s) : launch_all<K, V, float, false>(a, s);
        else return hipErrorNotSupported;
    }
    return per_k ? launch_all<K, V, bf16_t, true>(a, s) : launch_all<K, V, bf16_t, false>(a, s);
}

}  // namespace

ChunkWorkspaceLayout chunk_workspace_layout(int64_t T, int32_t N, int32_t HV, int32_t K, int32_t V, int io_bytes,
                                            bool per_k) {
    ChunkWorkspaceLayout L{};
    const int64_t max_chunks = T / CH + N;
    size_t off = 0;
    L.chunk_seq = off; off = align256(off + sizeof(int32_t) * (size_t)max_chunks);
    L.chunk_first = off; off = align256(off + sizeof(int32_t) * (size_t)(N + 1));
    L.gcum = off; off = align256(off + sizeof(float) * (size_t)T * HV * (per_k ? K : 1));
    L.w = off; off = align256(off + (size_t)io_bytes * T * HV * K);
    L.u = off; off = align256(off + (size_t)io_bytes * T * HV * V);
    L.vnew = off; off = align256(off + (size_t)io_bytes * T * HV * V);
    L.hc = off; off = align256(off + (size_t)io_bytes * max_chunks * HV * V * K);
    L.total = off;
    return L;
}

hipError_t launch_chunk(const ChunkArgs& a, int io_dtype, bool per_k, hipStream_t stream) {
    if (a.K == 64) {
        return a.V == 64 ? launch_kv<64, 64>(a, io_dtype, per_k, stream) : launch_kv<64, 128>(a, io_dtype, per_k, stream);
    }
    return a.V == 64 ? launch_kv<128, 64>(a, io_dtype, per_k, stream) : launch_kv<128, 128>(a, io_dtype, per_k, stream);
}

}  // namespace gdr
