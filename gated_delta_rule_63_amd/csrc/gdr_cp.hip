// Context parallelism inside one GPU for a few long sequences (the "auto-CP" named in the
// FlashQLA PR #1 design commit; the exchange design follows from the affine form of the
// recurrence).  Per key channel row of the state, one token maps the state affinely:
//
//     s <- s D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
//
// so a run of tokens (a segment) maps its start state as S_end = S_start M_seg + B_seg, where
// B_seg is the segment's end state from a zero start and M_seg (K x K) is the end state of the
// same segment run with v = 0 from the identity (row i of M_seg is e_i pushed through the
// segment).  The chunk kernel computes both as ordinary runs over the segments in parallel; the
// scan below chains the segments' maps into each segment's true start state, and a last chunk
// run over all segments from those states produces the outputs and the final state.
//
// Every sequence is cut into segments of seg_tokens tokens (a multiple of 64; the last segment of a
// sequence may be shorter, an empty sequence gets one empty segment).  The host only knows T and N,
// so the workspace is sized for an upper bound P_max on the segment count; the segment table is
// built on the device from cu_seqlens, and the segments past the real count are empty.
//
// Kernels here: the segment table and identity fill, the scan and the copy of each sequence's
// final state.  The host sequencing is in gdr_api.hip (gdr_chunk_fwd).
#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// Segment table from cu_seqlens (cu = NULL: one sequence of T tokens).  Sequence n gets
// nseg_n = max(1, ceil(len_n / seg_tokens)) segments; seg_first[n] = sum of nseg over the earlier
// sequences, seg_first[N] = the real segment count.  cu_seg[seg_first[n] + j] = start of segment j of
// sequence n, cu_seg[s] = T for every s from the real count up to P_max (empty trailing segments).
// M[s][h] = I (K x K) for every segment and head when the maps are formed by a run of their own.  One
// thread forms seg_first (N is small on this route); every thread fills cu_seg and M.
__global__ __launch_bounds__(256) void cp_setup_kernel(const int32_t* __restrict__ cu, int32_t N,
                                                       int32_t* __restrict__ cu_seg, int32_t* __restrict__ seg_first,
                                                       int P_max, int64_t seg_tokens, int64_t T,
                                                       float* __restrict__ M, int64_t n_maps_heads, int K) {
    const int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x;
    const int64_t kk = (int64_t)K * K;
    const int64_t total = n_maps_heads * kk;
    for (int64_t e = i; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t r = (e % kk) / K, c = e % K;
        M[e] = r == c ? 1.0f : 0.0f;
    }
    if (blockIdx.x != 0) return;
    if (threadIdx.x == 0) {
        int32_t acc = 0;
        for (int n = 0; n < N; ++n) {
            seg_first[n] = acc;
            const int64_t len = cu ? (int64_t)cu[n + 1] - cu[n] : T;
            const int64_t ns = len > 0 ? (len + seg_tokens - 1) / seg_tokens : 1;
            acc += (int32_t)ns;
        }
        seg_first[N] = acc;
    }
    __syncthreads();
    const int32_t real = seg_first[N];
    for (int n = 0; n < N; ++n) {
        const int64_t bos = cu ? cu[n] : 0, eos = cu ? cu[n + 1] : T;
        const int32_t f = seg_first[n], ns = seg_first[n + 1] - f;
        for (int j = threadIdx.x; j < ns; j += 256) {
            const int64_t st = bos + (int64_t)j * seg_tokens;
            cu_seg[f + j] = (int32_t)(st < eos ? st : eos);
        }
    }
    for (int s2 = real + (int)threadIdx.x; s2 <= P_max; s2 += 256) cu_seg[s2] = (int32_t)T;
}

// Per sequence n: S[f] = h0[n] (or zeros) and S[s+1] = S[s] M_s + B_s for the segments s = f .. l - 2 of
// the sequence (f = seg_first[n], l = seg_first[n + 1]), per value head.  One workgroup owns 16 state rows
// of one head of one sequence (V/16 x HV x N workgroups) and keeps them in LDS between steps; wave w forms
// output columns 32w .. 32w + 31 (two 16-column tiles; one tile when K = 64) with fp32 MFMA (16x16x4):
// A = the 16 rows from LDS, B = M_s, C starting from B_s.  M_s and B_s do not depend on the chain, so
// each lane holds its share of them for the next segment in registers, loaded while the current step's
// products run: a step then waits on no global load.  With the XCD-aware grid below, the 65573-token
// KDA call went from 1.2313 to 1.2024 ms (results bitwise unchanged), the 4 x 16384 GDN scan from 32 to
// 20 us.
template <int K>
__global__ __launch_bounds__(256) void cp_scan_kernel(const float* __restrict__ h0, const float* __restrict__ B,
                                                      const float* __restrict__ M, float* __restrict__ S,
                                                      const int32_t* __restrict__ seg_first, int HV, int V,
                                                      int nseq) {
    constexpr int LDR = K + 4;                  // padded LDS row: the A reads of a k-step hit 16 banks
    constexpr int TPW = K / 64;                 // 16-column tiles per wave (K / 16 tiles over 4 waves)
    constexpr int NK = K / 4;                   // k-steps of one product
    __shared__ __align__(16) float rows[16][LDR];
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    // one-dimensional grid, XCD-aware: workgroups are handed to the 8 XCDs in turn by linear index, so
    // the V/16 row blocks of one (sequence, head) take indices congruent modulo 8 and share an XCD, and
    // its M_s is fetched from memory once per step into that XCD's L2 instead of once per row block
    constexpr int kXcds = 8;
    const int nvt = V / 16;
    const int i = blockIdx.x;
    const int hs = (i / (kXcds * nvt)) * kXcds + i % kXcds;  // (sequence, head) pair
    if (hs >= HV * nseq) return;                              // padding of the last group of 8 pairs
    const int h = hs % HV, n = hs / HV, r0 = ((i / kXcds) % nvt) * 16;
    const int64_t vk = (int64_t)V * K;
    const int f = seg_first[n], last = seg_first[n + 1] - 1;
    // this lane's operands of one step: M_s[4k + l/16][col_t] for every k-step k and tile t, and
    // B_s[4(l/16) + e][col_t]; two sets, for the current and the next segment
    float mb[2][TPW][NK];
    f32x4_t bb[2][TPW];
    // through buffer resources: the lane's part of an address is one register, the k-step's part a
    // uniform offset, so the loads of a whole step need no per-load address registers
    auto fetch = [&](auto SET, int s) {
        constexpr int b = decltype(SET)::value;
        const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(M + ((int64_t)s * HV + h) * K * K), 0, K * K * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(B + ((int64_t)s * HV + h) * vk + (int64_t)r0 * K), 0, 16 * K * 4, 0x00020000);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int col = (w * TPW + t) * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bb[b][t][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                            rb, ((4 * (l >> 4) + e) * K + col) * 4, 0, 0));
#pragma unroll
            for (int k = 0; k < NK; ++k)
                mb[b][t][k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                            rm, ((l >> 4) * K + col) * 4, 16 * K * k, 0));
        }
    };
    auto step = [&](auto SET, int s) {
        constexpr int b = decltype(SET)::value;
        if (s + 1 < last) fetch(std::integral_constant<int, b ^ 1>{}, s + 1);
        f32x4_t acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] = bb[b][t];
        // the A operands of every k-step read from LDS together, then the products
        float av[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) av[k] = rows[l & 15][4 * k + (l >> 4)];
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
        for (int k = 0; k < NK; ++k) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], mb[b][t][k], acc[t], 0, 0, 0);
        }
        __syncthreads();  // every wave has read the previous rows
        float* Sn = S + ((int64_t)(s + 1) * HV + h) * vk + (int64_t)r0 * K;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int col = (w * TPW + t) * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                rows[4 * (l >> 4) + e][col] = acc[t][e];
                Sn[(int64_t)(4 * (l >> 4) + e) * K + col] = acc[t][e];
            }
        }
        __syncthreads();
    };
    // the first step's operands, then the start rows (every load of the prologue in flight together)
    if (f < last) fetch(std::integral_constant<int, 0>{}, f);
    constexpr int IPT = 16 * K / 256;  // start-state elements per thread
    float x0[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int e = tid + 256 * i, rr = e / K, cc = e % K;
        x0[i] = h0 ? h0[((int64_t)n * HV * V + (int64_t)h * V + r0 + rr) * K + cc] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int e = tid + 256 * i, rr = e / K, cc = e % K;
        rows[rr][cc] = x0[i];
        S[((int64_t)f * HV * V + (int64_t)h * V + r0 + rr) * K + cc] = x0[i];  // the first segment's start state
    }
    __syncthreads();
    for (int s = f; s < last; s += 2) {
        step(std::integral_constant<int, 0>{}, s);
        if (s + 1 < last) step(std::integral_constant<int, 1>{}, s + 1);
    }
}

// final_state[n] = S[seg_first[n + 1] - 1] (the end state of the sequence's last segment), every head.
__global__ __launch_bounds__(256) void cp_final_kernel(const float* __restrict__ S, const int32_t* __restrict__ seg_first,
                                                       float* __restrict__ out, int64_t hvk) {
    const int n = blockIdx.y;
    const float* src = S + (int64_t)(seg_first[n + 1] - 1) * hvk;
    float* dst = out + (int64_t)n * hvk;
    for (int64_t e = (blockIdx.x * (int64_t)256 + threadIdx.x) * 4; e < hvk; e += (int64_t)gridDim.x * 256 * 4)
        *reinterpret_cast<f32x4_t*>(dst + e) = *reinterpret_cast<const f32x4_t*>(src + e);
}

CpPlan cp_plan(int64_t T, int32_t N, int32_t HV, int32_t K, int32_t V, int io_bytes) {
    CpPlan pl{};
    pl.P = 1;
    if (N < 1 || T <= 0) return pl;
    const int vtiles = io_bytes == 4 ? V / 64 : 1;           // workgroups per head of the chunk kernel
    const int64_t wg_seq = (int64_t)N * HV * vtiles;          // workgroups of the direct route
    const int64_t per_seq = kCpWorkgroups / wg_seq;           // segments per sequence in one round
    if (per_seq < kCpMinSegments) return pl;
    const int64_t nchunks = (T + 63) / 64;
    // segment length: one round of the chunk kernel if the sequences were equal, at least 8 chunks
    int64_t seg_chunks = (nchunks + per_seq * N - 1) / (per_seq * N);
    if (seg_chunks < kCpMinChunks) seg_chunks = kCpMinChunks;
    const int64_t seg = seg_chunks * 64;
    if (T / seg / N < kCpMinSegments) return pl;             // too few segments per sequence on average
    // max(1, ceil(len / seg)) <= floor((len + seg) / seg), so for any lengths summing to T the segment
    // count is at most floor(T / seg) + N (exact for one sequence)
    const int64_t P_max = T / seg + N;
    pl.P = (int)P_max;
    pl.N = N;
    pl.seg_tokens = seg;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = 0;
    pl.cu_seg = off;    off += up(sizeof(int32_t) * (size_t)(P_max + 1));
    pl.seg_first = off; off += up(sizeof(int32_t) * (size_t)(N + 1));
    pl.B = off;         off += up(sizeof(float) * (size_t)P_max * HV * V * K);
    pl.M = off;         off += up(sizeof(float) * (size_t)P_max * HV * K * K);
    pl.S = off;         off += up(sizeof(float) * (size_t)P_max * HV * V * K);
    pl.total = off;
    return pl;
}

hipError_t launch_cp_setup(const CpPlan& pl, char* ws, const int32_t* cu, int64_t T, int32_t HV, int32_t K,
                           bool identity, hipStream_t stream) {
    const int64_t maps = identity ? (int64_t)pl.P * HV : 0;
    int64_t blocks = (maps * K * K + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(cp_setup_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cu, pl.N,
                       reinterpret_cast<int32_t*>(ws + pl.cu_seg), reinterpret_cast<int32_t*>(ws + pl.seg_first), pl.P,
                       pl.seg_tokens, T, reinterpret_cast<float*>(ws + pl.M), maps, K);
    return hipGetLastError();
}

hipError_t launch_cp_scan(const CpPlan& pl, char* ws, const float* h0, int32_t HV, int32_t K, int32_t V,
                          hipStream_t stream) {
    const int64_t pairs = (int64_t)HV * pl.N;
    const dim3 grid((unsigned)(((pairs + 7) / 8) * 8 * (V / 16)));
    const float* B = reinterpret_cast<const float*>(ws + pl.B);
    const float* M = reinterpret_cast<const float*>(ws + pl.M);
    float* S = reinterpret_cast<float*>(ws + pl.S);
    const int32_t* sf = reinterpret_cast<const int32_t*>(ws + pl.seg_first);
    if (K == 64)
        hipLaunchKernelGGL(cp_scan_kernel<64>, grid, dim3(256), 0, stream, h0, B, M, S, sf, HV, V, pl.N);
    else
        hipLaunchKernelGGL(cp_scan_kernel<128>, grid, dim3(256), 0, stream, h0, B, M, S, sf, HV, V, pl.N);
    return hipGetLastError();
}

hipError_t launch_cp_final(const CpPlan& pl, const char* ws, float* out, int32_t HV, int32_t K, int32_t V,
                           hipStream_t stream) {
    const int64_t hvk = (int64_t)HV * V * K;
    int64_t bx = (hvk / 4 + 255) / 256;
    if (bx > 1024) bx = 1024;
    hipLaunchKernelGGL(cp_final_kernel, dim3((unsigned)bx, pl.N), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(ws + pl.S), reinterpret_cast<const int32_t*>(ws + pl.seg_first),
                       out, hvk);
    return hipGetLastError();
}

}  // namespace gdr
