// Gating front as a pass of its own (FlashQLA PR #1, verify pre-pass commit: the in-loop
// gating is repeated for every value head of a key-head group and every V-tile, so a
// separate pass computes it once per token and feeds the plain kernels).
//
//   g[t,h]    = -exp(A_log[h]) softplus(a[t,h] + dt_bias[h])   (softplus: beta 1, threshold 20)
//   beta[t,h] = sigmoid(b[t,h]), times 2 when negative eigenvalues are allowed
//   q, k      <- x / sqrt(sum_c x_c^2 + eps) per (token, key head)
//
// Design (MI355X, wave64): one launch, 256-thread workgroups of two kinds.  The first
// ceil(2 T HK / 16) workgroups normalise rows: each 16-lane DPP row owns one q or k row
// (K / 16 channels per lane, loaded as whole 8- or 16-byte vectors), sums the squares with
// the 4-step DPP reduction and writes the scaled row.  The remaining workgroups form one
// (token, value head) gate pair per thread.  Everything is streamed once: the pass is
// HBM-bound and tiny next to the state traffic of the kernels it feeds.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

template <int K, typename IO>
__global__ __launch_bounds__(256) void gating_prepass_kernel(const GatingArgs a) {
    constexpr int EPL = K / 16;
    constexpr int VW = (16 / Elem<IO>::bytes) < EPL ? (16 / Elem<IO>::bytes) : EPL;
    constexpr int UNITS = EPL / VW;
    const int tid = threadIdx.x;
    const int64_t qrows = a.qk_l2norm ? a.T * a.HK : 0;
    const int64_t row_blocks = (2 * qrows + 15) / 16;
    const int64_t blk = blockIdx.x;

    if (blk < row_blocks) {
        const int64_t r = blk * 16 + (tid >> 4);                 // one row per 16-lane DPP row
        const int j = tid & 15;
        if (r >= 2 * qrows) return;                              // all 16 lanes of the row leave together
        const bool is_k = r >= qrows;
        const int64_t base = (is_k ? r - qrows : r) * K;
        const void* src = is_k ? a.k : a.q;
        void* dst = is_k ? a.k_out : a.q_out;
        float x[EPL];
#pragma unroll
        for (int u = 0; u < UNITS; ++u) Vec<IO, VW>::load(src, base + (u * 16 + j) * VW, &x[u * VW]);
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
        const float rn = rsqrtf(row16_sum(ss) + a.l2_eps);
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] *= rn;
#pragma unroll
        for (int u = 0; u < UNITS; ++u) Vec<IO, VW>::store(dst, base + (u * 16 + j) * VW, &x[u * VW]);
        return;
    }

    const int64_t i = (blk - row_blocks) * 256 + tid;
    if (i >= a.T * a.HV) return;
    const int h = (int)(i % a.HV);
    a.g_out[i] = gate_decay(Elem<IO>::load(a.a, i), -exp_f32(a.A_log[h]), a.dt_bias[h]);
    Elem<IO>::store(a.beta_out, i, a.beta_mul * sigmoid_f32(Elem<IO>::load(a.b, i)));
}

namespace {

template <int K, typename IO>
hipError_t launch_kio(const GatingArgs& a, hipStream_t stream) {
    const int64_t qrows = a.qk_l2norm ? a.T * a.HK : 0;
    const int64_t blocks = (2 * qrows + 15) / 16 + (a.T * a.HV + 255) / 256;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gating_prepass_kernel<K, IO>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gating(const GatingArgs& a, int K, int io_dtype, hipStream_t stream) {
    if (K == 64) return io_dtype == 0 ? launch_kio<64, float>(a, stream) : launch_kio<64, bf16_t>(a, stream);
    return io_dtype == 0 ? launch_kio<128, float>(a, stream) : launch_kio<128, bf16_t>(a, stream);
}

}  // namespace gdr
