// Fused KDA decode front for gfx950: causal convolution with SiLU over q, k and v, the low-rank gate
// projection to one decay per key channel, q/k l2 normalisation, beta = sigmoid(b), the delta-rule
// recurrence with the per-key-channel gate against the paged state, and an optional gated RMSNorm
// epilogue -- one launch per call.
//
// Method: tokenspeed PR #834 "[WIP] perf(k3): optimize decode" (the commit that rewrites the
// single-launch KDA decode: conv + SiLU, gate projection, QK l2 norm, recurrence against the paged
// fp32 state; the commit that folds rmsnorm(o) * w * sigmoid(gate) into the epilogue).  The
// recurrence is the one of FlashQLA PR #1 "Fused recurrent GDN decode + SGLang DFlash verify
// kernel (TileLang, SM90)" with the decay applied per key channel.
//
// Design (MI355X, wave64):
//  * one workgroup = 512 threads = 8 waves owns one (sequence, head) with all V state rows, so it
//    also owns every convolution channel of that head (q, k and v): the window is read at the start
//    and written back at the end by the same workgroup, and no other workgroup touches it (the page
//    reports a race where column-split programs shared an in-place window shift);
//  * per token, threads 0 .. 2K+V-1 each run one convolution channel (taps, bias and window in
//    registers); every thread also takes a 1/TPC share of one key channel's gate projection (a dot
//    product of length R; TPC = 512/K threads per channel, their partial sums reduced across the
//    consecutive lanes); thread 0 also forms beta.  All of a token's front loads are independent, so
//    they are in flight together.  Results go through LDS (double-buffered by token parity);
//  * the recurrence runs on 16-lane row groups as in the token-loop kernel: lane j holds K/16 key
//    channels of SLOTS = V/32 rows, the two row GEMVs reduce with DPP, q and k are normalised with
//    one more 16-lane reduction each;
//  * the epilogue's mean square over the V outputs of a token is reduced through LDS by every wave.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int kKdaThreads = 512;

// Eight consecutive elements held as loaded (bf16 pairs stay packed), so that a slice of the gate
// projection costs 4 registers in bf16.
template <typename IO> struct Slice8;
template <> struct Slice8<bf16_t> {
    uint4 w;
    __device__ __forceinline__ void load(const void* p, int64_t i) {
        w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    }
    __device__ __forceinline__ void zero() { w = uint4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float dot(const Slice8& o, float acc) const {
        const uint32_t a[4] = {w.x, w.y, w.z, w.w}, b[4] = {o.w.x, o.w.y, o.w.z, o.w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc = fmaf(__uint_as_float(a[j] << 16), __uint_as_float(b[j] << 16), acc);
            acc = fmaf(__uint_as_float(a[j] & 0xFFFF0000u), __uint_as_float(b[j] & 0xFFFF0000u), acc);
        }
        return acc;
    }
};
template <> struct Slice8<float> {
    f32x4_t x, y;
    __device__ __forceinline__ void load(const void* p, int64_t i) {
        const f32x4_t* s = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
        x = s[0];
        y = s[1];
    }
    __device__ __forceinline__ void zero() { x = y = f32x4_t{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float dot(const Slice8& o, float acc) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = fmaf(x[j], o.x[j], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = fmaf(y[j], o.y[j], acc);
        return acc;
    }
};

template <int K, int V, typename IO, typename ST, bool EPI>
__global__ __launch_bounds__(kKdaThreads) void kda_decode_kernel(const KdaArgs a) {
    constexpr int EPL = K / 16;                                  // key channels per lane
    constexpr int VW = (16 / Elem<ST>::bytes) < EPL ? (16 / Elem<ST>::bytes) : EPL;
    constexpr int UNITS = EPL / VW;
    constexpr int SLOTS = V / 32;                                // rows per row group (32 row groups)
    constexpr int C = 2 * K + V;                                 // convolution channels of one head
    static_assert(C <= kKdaThreads, "one thread per convolution channel");
    constexpr int TPC = kKdaThreads / K;                         // threads per key channel of the gate
    constexpr int GSLOTS = 4;                                    // 8-input slices per thread kept in registers

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane & 15;
    const int rg = (tid >> 6) * 4 + (lane >> 4);                 // row group 0..31
    const int h = blockIdx.x, n = blockIdx.y;
    const int row0 = rg * SLOTS;

    const int slot = a.slots[n];
    if (slot < 0) return;                                        // padded sequence: skip all
    const int64_t bos = a.cu_seqlens ? a.cu_seqlens[n] : n;
    const int64_t eos = a.cu_seqlens ? a.cu_seqlens[n + 1] : n + 1;

    __shared__ __align__(16) float sx[2][C];                     // conv + SiLU outputs: q | k | v
    __shared__ __align__(16) float sd[2][K];                     // decay factors e^{gk}
    __shared__ float sb[2];                                      // beta
    __shared__ __align__(16) float so[EPI ? 2 : 1][EPI ? V : 1]; // outputs before the epilogue

    // ---- this thread's front roles ----
    const bool conv_thread = tid < C;
    int64_t gchan = 0;                                           // global convolution channel
    const void* src = nullptr;                                   // raw input tensor of the channel
    int64_t src_row = 0, src_col = 0;                            // element (t * src_row + src_col)
    if (conv_thread) {
        if (tid < K) {
            gchan = (int64_t)h * K + tid;
            src = a.q; src_row = (int64_t)a.HV * K; src_col = (int64_t)h * K + tid;
        } else if (tid < 2 * K) {
            gchan = (int64_t)a.HV * K + (int64_t)h * K + (tid - K);
            src = a.k; src_row = (int64_t)a.HV * K; src_col = (int64_t)h * K + (tid - K);
        } else {
            gchan = 2 * (int64_t)a.HV * K + (int64_t)h * V + (tid - 2 * K);
            src = a.v; src_row = (int64_t)a.HV * V; src_col = (int64_t)h * V + (tid - 2 * K);
        }
    }
    const int W = a.conv_width;
    const int64_t nchan = 2 * (int64_t)a.HV * K + (int64_t)a.HV * V;
    float taps[4] = {0.f, 0.f, 0.f, 0.f}, win[3] = {0.f, 0.f, 0.f}, bias = 0.f;
    const int64_t win_base = ((int64_t)slot * nchan + gchan) * (W - 1);
    if (conv_thread) {
        for (int i = 0; i < W; ++i) taps[4 - W + i] = Elem<IO>::load(a.conv_weight, gchan * W + i);  // right-aligned
        for (int i = 0; i < W - 1; ++i) win[3 - (W - 1) + i] = Elem<IO>::load(a.conv_state, win_base + i);
        if (a.conv_bias) bias = Elem<IO>::load(a.conv_bias, gchan);
    }
    const int gc = tid / TPC, gq = tid % TPC;                    // gate: key channel and share of it
    const float neg_exp_a_log = -exp_f32(a.A_log[h]);
    const float dtb = a.dt_bias[(int64_t)h * K + gc];
    const int R = a.gate_rank;
    const int64_t wrow = ((int64_t)h * K + gc) * R;
    // this thread's slices of the projection row are (gq + i TPC) * 8 .. +7; up to GSLOTS of them are read
    // per token with every load in flight together
    const bool gate_short = R <= 8 * TPC * GSLOTS;

    // ---- state tile (all V rows of the head) through a buffer resource ----
    int cols[UNITS];
#pragma unroll
    for (int u = 0; u < UNITS; ++u) cols[u] = (u * 16 + j) * VW;
    float S[SLOTS][EPL];
    {
        const int64_t tile = ((int64_t)slot * a.HV + h) * V * K;
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(static_cast<const char*>(a.pool) + tile * Elem<ST>::bytes), 0, V * K * Elem<ST>::bytes,
            0x00020000);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
            for (int u = 0; u < UNITS; ++u)
                BufVec<ST, VW>::template load<kNonTemporal>(
                    srs, (uint32_t)(((row0 + s) * K + cols[u]) * Elem<ST>::bytes), &S[s][u * VW]);
    }

    for (int64_t t = bos; t < eos; ++t) {
        const int pb = (int)((t - bos) & 1);
        // ===== front =====
        float x = 0.f;
        if (conv_thread) x = Elem<IO>::load(src, t * src_row + src_col);
        // raw = gate_weight[h K + c, :] . gate_in[t, :]: this thread's slices, then the channel's TPC lanes
        float acc = 0.f;
        if (gate_short) {
            Slice8<IO> wv[GSLOTS], av[GSLOTS];
#pragma unroll
            for (int i = 0; i < GSLOTS; ++i) {
                const int r = (gq + i * TPC) * 8;
                if (r < R) {
                    wv[i].load(a.gate_weight, wrow + r);
                    av[i].load(a.gate_in, t * R + r);
                } else {
                    wv[i].zero();
                    av[i].zero();
                }
            }
#pragma unroll
            for (int i = 0; i < GSLOTS; ++i) acc = wv[i].dot(av[i], acc);
        } else {
            for (int r = gq * 8; r < R; r += 8 * TPC) {
                Slice8<IO> wv, av;
                wv.load(a.gate_weight, wrow + r);
                av.load(a.gate_in, t * R + r);
                acc = wv.dot(av, acc);
            }
        }
#pragma unroll
        for (int m = 1; m < TPC; m <<= 1) acc += __shfl_xor(acc, m);
        if (gq == 0) sd[pb][gc] = exp_f32(gate_decay(acc, neg_exp_a_log, dtb));
        if (conv_thread) {
            const float z = bias + taps[0] * win[0] + taps[1] * win[1] + taps[2] * win[2] + taps[3] * x;
            sx[pb][tid] = z * sigmoid_f32(z);
            win[0] = win[1];
            win[1] = win[2];
            win[2] = x;
        }
        if (tid == 0) sb[pb] = sigmoid_f32(Elem<IO>::load(a.b, t * a.HV + h));
        __syncthreads();  // the token's front is in LDS
        // ===== recurrence on this thread's rows =====
        float kk[EPL], qq[EPL], al[EPL];
#pragma unroll
        for (int u = 0; u < UNITS; ++u)
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                qq[u * VW + e] = sx[pb][cols[u] + e];
                kk[u * VW + e] = sx[pb][K + cols[u] + e];
                al[u * VW + e] = sd[pb][cols[u] + e];
            }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            sq = fmaf(qq[e], qq[e], sq);
            sk = fmaf(kk[e], kk[e], sk);
        }
        const float rq = rsqrtf(row16_sum(sq) + a.l2_eps), rk = rsqrtf(row16_sum(sk) + a.l2_eps);
        float ka[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qq[e] *= rq;
            kk[e] *= rk;
            ka[e] = al[e] * kk[e];
        }
        const float bt = sb[pb];
        float ov[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) p = fmaf(S[s][e], ka[e], p);
            p = row16_sum(p);
            const float nu = bt * (sx[pb][2 * K + row0 + s] - p);
            float po = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                S[s][e] = fmaf(nu, kk[e], al[e] * S[s][e]);        // decay + rank-1
                po = fmaf(S[s][e], qq[e], po);
            }
            ov[s] = a.scale * row16_sum(po);                         // post-update read
        }
        float mine = ov[0];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s) mine = ((j % SLOTS) == s) ? ov[s] : mine;
        const int myrow = row0 + (j % SLOTS);
        const int64_t orow = (t * a.HV + h) * V;
        if constexpr (EPI) {
            // o <- o / sqrt(mean_v o^2 + eps) * w * sigmoid(z): every wave reduces the token's V outputs
            if (j < SLOTS) so[pb][myrow] = mine;
            __syncthreads();
            float ss = 0.f;
#pragma unroll
            for (int i = lane; i < V; i += 64) ss = fmaf(so[pb][i], so[pb][i], ss);
            ss = row16_sum(ss);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            const float inv = rsqrtf(ss * (1.0f / V) + a.norm_eps);
            const float wv = Elem<IO>::load(a.norm_weight, myrow);
            const float zv = Elem<IO>::load(a.norm_gate, orow + myrow);
            mine = mine * inv * wv * sigmoid_f32(zv);
        }
        Elem<IO>::store(a.o, orow + myrow, mine);
    }

    if (a.commit) {
        // written through (device scope): the state is not read again in this call (64 x 32 heads:
        // unchanged at 0.063 ms; 16 x 32 heads: 0.021 -> 0.0205 ms)
        const int64_t tile = ((int64_t)slot * a.HV + h) * V * K;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char*>(a.pool) + tile * Elem<ST>::bytes, 0, V * K * Elem<ST>::bytes, 0x00020000);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
            for (int u = 0; u < UNITS; ++u)
                BufStore<ST, VW>::template store<kWriteThrough>(
                    crs, (uint32_t)(((row0 + s) * K + cols[u]) * Elem<ST>::bytes), &S[s][u * VW]);
        if (conv_thread)
            for (int i = 0; i < W - 1; ++i) Elem<IO>::store(a.conv_state, win_base + i, win[3 - (W - 1) + i]);
    }
}

template <int K, int V, typename IO, typename ST>
hipError_t launch_kv(const KdaArgs& a, hipStream_t stream) {
    const dim3 grid(a.HV, a.N);
    if (a.norm_weight)
        hipLaunchKernelGGL((kda_decode_kernel<K, V, IO, ST, true>), grid, dim3(kKdaThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((kda_decode_kernel<K, V, IO, ST, false>), grid, dim3(kKdaThreads), 0, stream, a);
    return hipGetLastError();
}

template <int K, int V>
hipError_t launch_dt(const KdaArgs& a, int io_dtype, int st_dtype, hipStream_t stream) {
    if (io_dtype == 0) return st_dtype == 0 ? launch_kv<K, V, float, float>(a, stream) : launch_kv<K, V, float, bf16_t>(a, stream);
    return st_dtype == 0 ? launch_kv<K, V, bf16_t, float>(a, stream) : launch_kv<K, V, bf16_t, bf16_t>(a, stream);
}

}  // namespace

hipError_t launch_kda(const KdaArgs& a, int K, int V, int io_dtype, int st_dtype, hipStream_t stream) {
    if (K == 64) return V == 64 ? launch_dt<64, 64>(a, io_dtype, st_dtype, stream) : launch_dt<64, 128>(a, io_dtype, st_dtype, stream);
    return V == 64 ? launch_dt<128, 64>(a, io_dtype, st_dtype, stream) : launch_dt<128, 128>(a, io_dtype, st_dtype, stream);
}

}  // namespace gdr
