// Context parallelism inside one GPU for a single long sequence (the "auto-CP" named in the
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
// Kernels here: the segment table and identity fill, and the scan.  The host sequencing is in
// gdr_api.hip (gdr_chunk_fwd).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// cu_seg[i] = min(i * seg_tokens, T) for i = 0..P; M[s][h] = I (K x K) for s < nmaps, every head.
__global__ __launch_bounds__(256) void cp_setup_kernel(int32_t* __restrict__ cu_seg, int P, int64_t seg_tokens,
                                                       int64_t T, float* __restrict__ M, int64_t n_maps_heads, int K) {
    const int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x;
    if (i <= P) cu_seg[i] = (int32_t)(i * seg_tokens < T ? i * seg_tokens : T);
    const int64_t kk = (int64_t)K * K;
    const int64_t total = n_maps_heads * kk;
    for (int64_t e = i; e < total; e += (int64_t)gridDim.x * 256) {
        const int64_t r = (e % kk) / K, c = e % K;
        M[e] = r == c ? 1.0f : 0.0f;
    }
}

// S[0] = h0 (or zeros); S[s+1] = S[s] M_s + B_s for s = 0..P-2, per value head.  One workgroup
// owns 16 state rows of one head (grid: V/16 x HV) and keeps them in LDS between steps; wave w
// forms output columns 32w .. 32w + 31 (two 16-column tiles; one tile when K = 64) with fp32
// MFMA (16x16x4): A = the 16 rows from LDS, B = M_s from L2, C starting from B_s.
template <int K>
__global__ __launch_bounds__(256) void cp_scan_kernel(const float* __restrict__ h0, const float* __restrict__ B,
                                                      const float* __restrict__ M, float* __restrict__ S, int P,
                                                      int HV, int V) {
    constexpr int LDR = K + 4;                  // padded LDS row: the A reads of a k-step hit 16 banks
    constexpr int TPW = K / 64;                 // 16-column tiles per wave (K / 16 tiles over 4 waves)
    __shared__ __align__(16) float rows[16][LDR];
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    const int h = blockIdx.y, r0 = blockIdx.x * 16;
    const int64_t vk = (int64_t)V * K;
    for (int e = tid; e < 16 * K; e += 256) {
        const int rr = e / K, cc = e % K;
        const int64_t idx = ((int64_t)h * V + r0 + rr) * K + cc;  // segment 0 of S / h0
        const float x = h0 ? h0[idx] : 0.0f;
        rows[rr][cc] = x;
        S[idx] = x;
    }
    __syncthreads();
    for (int s = 0; s + 1 < P; ++s) {
        const float* Ms = M + ((int64_t)s * HV + h) * K * K;
        const float* Bs = B + ((int64_t)s * HV + h) * vk + (int64_t)r0 * K;
        f32x4_t acc[TPW];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int col = (w * TPW + t) * 16 + (l & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t][e] = Bs[(int64_t)(4 * (l >> 4) + e) * K + col];
        }
#pragma unroll 8
        for (int k0 = 0; k0 < K; k0 += 4) {
            const float av = rows[l & 15][k0 + (l >> 4)];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const float bv = Ms[(int64_t)(k0 + (l >> 4)) * K + (w * TPW + t) * 16 + (l & 15)];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[t], 0, 0, 0);
            }
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
    }
}

CpPlan cp_plan(int64_t T, int32_t N, int32_t HV, int32_t K, int32_t V, int io_bytes) {
    CpPlan pl{};
    pl.P = 1;
    if (N != 1 || T <= 0) return pl;
    const int vtiles = io_bytes == 4 ? V / 64 : 1;           // workgroups per head of the chunk kernel
    const int64_t nchunks = (T + 63) / 64;
    int64_t P = kCpWorkgroups / ((int64_t)HV * vtiles);       // one round of the chunk kernel
    if (P > nchunks / kCpMinChunks) P = nchunks / kCpMinChunks;
    if (P < kCpMinSegments) return pl;
    const int64_t seg_chunks = (nchunks + P - 1) / P;
    P = (nchunks + seg_chunks - 1) / seg_chunks;              // no empty segment
    if (P < kCpMinSegments) return pl;
    pl.P = (int)P;
    pl.seg_tokens = seg_chunks * 64;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t off = 0;
    pl.cu_seg = off;  off += up(sizeof(int32_t) * (size_t)(P + 1));
    pl.B = off;       off += up(sizeof(float) * (size_t)(P - 1) * HV * V * K);
    pl.M = off;       off += up(sizeof(float) * (size_t)(P - 1) * HV * K * K);
    pl.S = off;       off += up(sizeof(float) * (size_t)P * HV * V * K);
    pl.total = off;
    return pl;
}

hipError_t launch_cp_setup(const CpPlan& pl, char* ws, int64_t T, int32_t HV, int32_t K, hipStream_t stream) {
    const int64_t maps = (int64_t)(pl.P - 1) * HV;
    int64_t blocks = (maps * K * K + 255) / 256;
    if (blocks < (pl.P + 1 + 255) / 256) blocks = (pl.P + 1 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(cp_setup_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<int32_t*>(ws + pl.cu_seg), pl.P, pl.seg_tokens, T,
                       reinterpret_cast<float*>(ws + pl.M), maps, K);
    return hipGetLastError();
}

hipError_t launch_cp_scan(const CpPlan& pl, char* ws, const float* h0, int32_t HV, int32_t K, int32_t V,
                          hipStream_t stream) {
    const dim3 grid(V / 16, HV);
    const float* B = reinterpret_cast<const float*>(ws + pl.B);
    const float* M = reinterpret_cast<const float*>(ws + pl.M);
    float* S = reinterpret_cast<float*>(ws + pl.S);
    if (K == 64)
        hipLaunchKernelGGL(cp_scan_kernel<64>, grid, dim3(256), 0, stream, h0, B, M, S, pl.P, HV, V);
    else
        hipLaunchKernelGGL(cp_scan_kernel<128>, grid, dim3(256), 0, stream, h0, B, M, S, pl.P, HV, V);
    return hipGetLastError();
}

}  // namespace gdr
