// H1: token-by-token gated delta rule for gfx950 -- dense recurrent forward, paged
// decode (commit) and speculative verify (per-token intermediate states, no commit).
//
// Method: FlashQLA PR #1 "Fused recurrent GDN decode + SGLang DFlash verify kernel"
// (core decode-kernel commit: decay -> kS -> v_new -> rank-1 -> o, post-update read;
// verify-kernel commit: paged gather/scatter through state_indices, -1 skips the
// sequence, V-major pool, per-token intermediate states, no-commit mode).
//
// Design (MI355X, wave64):
//  * one workgroup = 256 threads = 4 waves owns BV = 16*SLOTS consecutive state rows
//    of one (sequence, value head); V-rows are independent, so V-tiles never talk;
//  * 16 lanes share a row: lane j holds K/16 key channels of it in fp32 registers
//    (whole 16-byte vectors; in fp32 the two halves of a 128-wide row go to lanes
//    j and j+16-units so every load instruction reads 256 contiguous bytes per row);
//  * a thread owns SLOTS consecutive rows; the two row GEMVs (S.k and S.q) are
//    in-register FMAs followed by a 4-step DPP reduction over the 16 lanes;
//  * the state is read once, kept in registers for all tokens of the sequence and
//    written once (commit / final state), V-major, no transpose; the verify mode
//    streams each post-update state out as it is produced;
//  * with several tokens per sequence, token t+1's inputs are loaded while token t
//    computes (PF); single-token decode skips that to keep the register count low;
//  * GATED instantiations take the raw gating inputs instead of g and beta (FlashQLA
//    PR #1, in-kernel gated verify commit): per token g = -exp(A_log) softplus(a + dt_bias),
//    beta = sigmoid(b) (doubled when negative eigenvalues are allowed), and q, k are
//    l2-normalised with one more 16-lane reduction each.  Every row group repeats this
//    small per-token work; it hides under the state traffic.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// GATE: 0 = g and beta given; 1 = gating front (g, beta from a, b); 2 = gating front and q/k
// l2 normalisation.  The normalisation is a template choice, not a runtime branch, so the
// token loop stays one basic block and its loads issue together.
template <int K, typename IO, typename ST, typename DT, typename IB, bool PER_K, int SLOTS, bool PF, int GATE>
__global__ __launch_bounds__(256) void recurrent_kernel(const RecurrentArgs a) {
    constexpr bool GATED = GATE > 0;
    static_assert(!(GATED && PER_K), "the gating front defines a scalar decay only");
    constexpr int EPL = K / 16;                                  // key channels per lane
    constexpr int VW = (16 / Elem<ST>::bytes) < EPL ? (16 / Elem<ST>::bytes) : EPL;
    constexpr int UNITS = EPL / VW;                              // vectors per lane per row
    constexpr int BV = 16 * SLOTS;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane & 15;                                     // lane within the row group
    const int rg = (tid >> 6) * 4 + (lane >> 4);                 // row group 0..15
    const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
    const int hk = h / (a.HV / a.HK);
    const int row0 = vt * BV + rg * SLOTS;                       // first of this thread's rows

    const int slot = a.slots ? a.slots[n] : n;
    if (slot < 0) return;                                        // padded sequence: skip all

    int64_t bos, eos;
    if (a.cu_seqlens) {
        bos = a.cu_seqlens[n];
        eos = a.cu_seqlens[n + 1];
    } else if (a.one_token_per_seq) {
        bos = n;
        eos = n + 1;
    } else {
        bos = 0;
        eos = a.T;
    }

    int cols[UNITS];
#pragma unroll
    for (int u = 0; u < UNITS; ++u) cols[u] = (u * 16 + j) * VW;

    // per-head gate constants
    const float neg_exp_a_log = GATED ? -exp_f32(a.A_log[h]) : 0.0f;
    const float dt_bias = GATED ? a.dt_bias[h] : 0.0f;
    const int64_t ib_row = a.ibuf ? (int64_t)a.ibuf_idx[n] * a.cache_steps : 0;

    float S[SLOTS][EPL];
    // The workgroup's state tile (BV rows of K) is read through a buffer resource that spans the
    // tile, or nothing when there is no source state: reads then return zeros, so the start state
    // needs no branch and its loads schedule together with the first token's.  The reads are
    // non-temporal: each state byte is read once per call (decode 0.153 -> 0.146 ms).
    auto load_state = [&]() {
        const int64_t tile = (((int64_t)slot * a.HV + h) * a.V + vt * BV) * K;
        const char* tile_ptr = a.src ? static_cast<const char*>(a.src) + tile * Elem<ST>::bytes : nullptr;
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(tile_ptr), 0, a.src ? BV * K * Elem<ST>::bytes : 0, 0x00020000);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
            for (int u = 0; u < UNITS; ++u)
                BufVec<ST, VW>::template load<kNonTemporal>(
                    srs, (uint32_t)(((rg * SLOTS + s) * K + cols[u]) * Elem<ST>::bytes), &S[s][u * VW]);
    };

    // One token on this thread's SLOTS rows, from its unpacked inputs: k and q (this lane's
    // channels), the decay factors, beta and v (this thread's rows).
    auto step = [&](int64_t t, float* kk, float* qq, const float* al, float bt, const float* vv) {
        const int64_t th = t * a.HV + h;
        if constexpr (GATE == 2) {
            float sk = 0.0f, sq = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                sk = fmaf(kk[e], kk[e], sk);
                sq = fmaf(qq[e], qq[e], sq);
            }
            const float rk = rsqrtf(row16_sum(sk) + a.l2_eps);
            const float rq = rsqrtf(row16_sum(sq) + a.l2_eps);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kk[e] *= rk;
                qq[e] *= rq;
            }
        }
        // (decayed S) . k: with the per-channel gate the decay multiplies k element-wise; a scalar
        // gate multiplies the reduced dot product once (fewer registers and instructions)
        float ka[PER_K ? EPL : 1];
        if constexpr (PER_K) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) ka[e] = al[e] * kk[e];
        }
        float ov[SLOTS];
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) {
            float p = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) p = fmaf(S[s][e], PER_K ? ka[e] : kk[e], p);
            p = row16_sum(p);
            if constexpr (!PER_K) p *= al[0];
            const float nu = bt * (vv[s] - p);
            float po = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                S[s][e] = fmaf(nu, kk[e], al[PER_K ? e : 0] * S[s][e]);  // decay + rank-1
                po = fmaf(S[s][e], qq[e], po);
            }
            ov[s] = a.scale * row16_sum(po);                              // post-update read
        }
        // Lane j of each row group writes row (row0 + j % SLOTS): lanes past SLOTS repeat the same
        // value to the same address, so no store in the token loop is conditional.
        float mine = ov[0];
#pragma unroll
        for (int s = 1; s < SLOTS; ++s) mine = ((j % SLOTS) == s) ? ov[s] : mine;
        Elem<IO>::store(a.o, th * a.V + row0 + (j % SLOTS), mine);

        if constexpr (!std::is_same<IB, void>::value) {  // instantiated only with an intermediate buffer
            // written through (device scope): the per-token states are not read again in this call
            // (verify 0.147 -> 0.145 ms)
            const int64_t ibt = (((ib_row + (t - bos)) * a.HV + h) * a.V + vt * BV) * K;
            const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<char*>(a.ibuf) + ibt * Elem<IB>::bytes, 0, BV * K * Elem<IB>::bytes, 0x00020000);
#pragma unroll
            for (int s = 0; s < SLOTS; ++s)
#pragma unroll
                for (int u = 0; u < UNITS; ++u)
                    BufStore<IB, VW>::template store<kWriteThrough>(
                        irs, (uint32_t)(((rg * SLOTS + s) * K + cols[u]) * Elem<IB>::bytes), &S[s][u * VW]);
        }
    };
    // scalar decay factor and beta from the raw per-token values (gating front when GATED)
    auto gate_scalar = [&](float graw) { return exp_f32(GATED ? gate_decay(graw, neg_exp_a_log, dt_bias) : graw); };
    auto beta_of = [&](float braw) { return GATED ? a.beta_mul * sigmoid_f32(braw) : braw; };

    if constexpr (PF) {
        // Several tokens per sequence: the workgroup stages TB tokens' inputs in LDS at a time, so
        // the token loop itself waits on no global load, and every row group reads the shared k,
        // q, gate and beta from LDS (one copy per workgroup instead of one per row group).
        typedef typename RawT<IO>::T R;
        constexpr int ESZ = Elem<IO>::bytes;
        constexpr int TB = ESZ == 2 ? 16 : 8;                      // tokens per block
        constexpr int KROW = K * ESZ / 16, VROW = BV * ESZ / 16, GROW = K * 4 / 16;  // 16-byte chunks per row
        constexpr int NK = (TB * KROW + 255) / 256, NV = (TB * VROW + 255) / 256;
        constexpr int NG = PER_K ? (TB * GROW + 255) / 256 : 0;
        __shared__ __align__(16) R sk[TB][K], sq[TB][K], sv[TB][BV];
        __shared__ __align__(16) float sgk[PER_K ? TB : 1][PER_K ? K : 4];
        __shared__ float sg[TB], sb[TB];
        uint4 rk[NK], rq[NK], rv[NV], rgk[NG > 0 ? NG : 1];
        uint32_t rgs = 0, rbs = 0;                                 // raw bits, widened in put()
        auto raw_bits = [](const void* p, int64_t i) -> uint32_t {
            if constexpr (ESZ == 2) return static_cast<const uint16_t*>(p)[i];
            else return __float_as_uint(static_cast<const float*>(p)[i]);
        };
        auto widen = [](uint32_t u) { return ESZ == 2 ? __uint_as_float(u << 16) : __uint_as_float(u); };
        auto fetch = [&](int64_t tb, int nt) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int c = tid + 256 * i, r = c / KROW, c16 = c % KROW;
                if (c < TB * KROW && r < nt) {
                    const int64_t off = ((tb + r) * a.HK + hk) * K * ESZ + c16 * 16;
                    rk[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k) + off);
                    rq[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + off);
                }
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int c = tid + 256 * i, r = c / VROW, c16 = c % VROW;
                if (c < TB * VROW && r < nt)
                    rv[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v) +
                                                             (((tb + r) * a.HV + h) * a.V + vt * BV) * ESZ + c16 * 16);
            }
            if constexpr (PER_K) {
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int c = tid + 256 * i, r = c / GROW, c16 = c % GROW;
                    if (c < TB * GROW && r < nt)
                        rgk[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.g) +
                                                                  ((tb + r) * a.HV + h) * K * 4 + c16 * 16);
                }
            }
            if (tid < nt) {
                const int64_t th = (tb + tid) * a.HV + h;
                if constexpr (!PER_K) rgs = GATED ? raw_bits(a.ga, th) : __float_as_uint(a.g[th]);
                rbs = raw_bits(GATED ? a.gb : a.beta, th);
            }
        };
        auto put = [&](int nt) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int c = tid + 256 * i, r = c / KROW, c16 = c % KROW;
                if (c < TB * KROW && r < nt) {
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sk[r][0]) + c16 * 16) = rk[i];
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sq[r][0]) + c16 * 16) = rq[i];
                }
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int c = tid + 256 * i, r = c / VROW, c16 = c % VROW;
                if (c < TB * VROW && r < nt) *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sv[r][0]) + c16 * 16) = rv[i];
            }
            if constexpr (PER_K) {
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int c = tid + 256 * i, r = c / GROW, c16 = c % GROW;
                    if (c < TB * GROW && r < nt)
                        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(&sgk[r][0]) + c16 * 16) = rgk[i];
                }
            }
            if (tid < nt) {
                sg[tid] = GATED ? widen(rgs) : __uint_as_float(rgs);
                sb[tid] = widen(rbs);
            }
        };

        fetch(bos, (int)(eos - bos < TB ? eos - bos : TB));   // the first block's loads, then the state's
        load_state();
        for (int64_t tb = bos; tb < eos; tb += TB) {
            const int nt = (int)(eos - tb < TB ? eos - tb : TB);
            if (tb > bos) __syncthreads();                      // the previous block has been read
            put(nt);
            __syncthreads();
            // the next block's loads are in flight while this block's tokens run
            if (tb + TB < eos) fetch(tb + TB, (int)(eos - tb - TB < TB ? eos - tb - TB : TB));
            for (int i = 0; i < nt; ++i) {
                float kk[EPL], qq[EPL], al[PER_K ? EPL : 1], vv[SLOTS];
#pragma unroll
                for (int u = 0; u < UNITS; ++u) {
                    LdsVec<IO, VW>::get(&sk[i][cols[u]], &kk[u * VW]);
                    LdsVec<IO, VW>::get(&sq[i][cols[u]], &qq[u * VW]);
                }
                if constexpr (PER_K) {
#pragma unroll
                    for (int u = 0; u < UNITS; ++u) LdsVec<float, VW>::get(&sgk[i][cols[u]], &al[u * VW]);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) al[e] = exp_f32(al[e]);
                } else {
                    al[0] = gate_scalar(sg[i]);
                }
                LdsVec<IO, SLOTS>::get(&sv[i][rg * SLOTS], vv);
                step(tb + i, kk, qq, al, beta_of(sb[i]), vv);
            }
        }
    } else {
        // One token per sequence in practice (decode): the token's inputs come straight into
        // registers, requested before the state so the first token waits one round trip; a longer
        // sequence loads each further token after the previous one.
        struct TokIn {
            RawVec<IO, VW> k[UNITS], q[UNITS];
            RawVec<float, VW> gk[PER_K ? UNITS : 1];
            float g;
            RawElem<IO> ga;                                      // GATED: raw decay input a
            RawElem<IO> b;                                       // beta, or GATED: raw input b
            RawVec<IO, SLOTS> v;
        };
        auto load_tok = [&](int64_t t, TokIn& x) {
            const int64_t qk_off = (t * a.HK + hk) * K;
            const int64_t th = t * a.HV + h;
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                x.k[u].load(a.k, qk_off + cols[u]);
                x.q[u].load(a.q, qk_off + cols[u]);
            }
            if constexpr (PER_K) {
#pragma unroll
                for (int u = 0; u < UNITS; ++u) x.gk[u].load(a.g, th * K + cols[u]);
            } else if constexpr (GATED) {
                x.ga.load(a.ga, th);
            } else {
                x.g = a.g[th];
            }
            x.b.load(GATED ? a.gb : a.beta, th);
            x.v.load(a.v, th * a.V + row0);
        };
        TokIn nxt;
        load_tok(bos < eos ? bos : a.T - 1, nxt);  // an empty sequence reads a valid token it never uses
        load_state();
        for (int64_t t = bos; t < eos; ++t) {
            TokIn cur = nxt;
            float kk[EPL], qq[EPL], al[PER_K ? EPL : 1], vv[SLOTS];
#pragma unroll
            for (int u = 0; u < UNITS; ++u) {
                cur.k[u].get(&kk[u * VW]);
                cur.q[u].get(&qq[u * VW]);
            }
            if constexpr (PER_K) {
#pragma unroll
                for (int u = 0; u < UNITS; ++u) cur.gk[u].get(&al[u * VW]);
#pragma unroll
                for (int e = 0; e < EPL; ++e) al[e] = exp_f32(al[e]);
            } else {
                al[0] = gate_scalar(GATED ? cur.ga.get() : cur.g);
            }
            cur.v.get(vv);
            step(t, kk, qq, al, beta_of(cur.b.get()), vv);
            if (t + 1 < eos) load_tok(t + 1, nxt);
        }
    }

    if (a.dst) {
        // the committed / final state, written through (device scope): not read again in this call
        // (decode 0.146 -> 0.142 ms; non-temporal stores measured slower than either)
        const int64_t tile = (((int64_t)slot * a.HV + h) * a.V + vt * BV) * K;
        const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<char*>(a.dst) + tile * Elem<DT>::bytes, 0, BV * K * Elem<DT>::bytes, 0x00020000);
#pragma unroll
        for (int s = 0; s < SLOTS; ++s)
#pragma unroll
            for (int u = 0; u < UNITS; ++u)
                BufStore<DT, VW>::template store<kWriteThrough>(
                    drs, (uint32_t)(((rg * SLOTS + s) * K + cols[u]) * Elem<DT>::bytes), &S[s][u * VW]);
    }
}

// Empty batch with a final state requested: final = initial (or zeros), fp32.
__global__ __launch_bounds__(256) void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         int64_t n) {
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src ? src[i] : 0.0f;
}

hipError_t launch_state_copy(const float* src, float* dst, int64_t n, hipStream_t stream) {
    if (n <= 0 || src == dst) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, n);
    return hipGetLastError();
}

namespace {

constexpr int kSlots = 4;  // BV = 64 rows per workgroup

template <int K, typename IO, typename ST, typename DT, typename IB, bool PER_K, int GATE>
hipError_t launch_t(const RecurrentArgs& a, hipStream_t stream) {
    dim3 grid(a.V / (16 * kSlots), a.HV, a.N);
    if (a.prefetch)
        hipLaunchKernelGGL((recurrent_kernel<K, IO, ST, DT, IB, PER_K, kSlots, true, GATE>), grid, dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((recurrent_kernel<K, IO, ST, DT, IB, PER_K, kSlots, false, GATE>), grid, dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

template <int K, typename IO, typename ST, typename DT, bool PER_K, int GATE>
hipError_t launch_ib(const RecurrentArgs& a, int ib_dtype, hipStream_t stream) {
    if (ib_dtype < 0) return launch_t<K, IO, ST, DT, void, PER_K, GATE>(a, stream);
    if (ib_dtype == 0) return launch_t<K, IO, ST, DT, float, PER_K, GATE>(a, stream);
    return launch_t<K, IO, ST, DT, bf16_t, PER_K, GATE>(a, stream);
}

template <int K, typename IO, bool PER_K, int GATE>
hipError_t launch_st(const RecurrentArgs& a, int st_dtype, int ib_dtype, hipStream_t stream) {
    // state source and destination share a dtype (pool) except in the dense mode,
    // where both are fp32
    if (st_dtype == 0) return launch_ib<K, IO, float, float, PER_K, GATE>(a, ib_dtype, stream);
    return launch_ib<K, IO, bf16_t, bf16_t, PER_K, GATE>(a, ib_dtype, stream);
}

template <int K, bool PER_K, int GATE>
hipError_t launch_io(const RecurrentArgs& a, int io_dtype, int st_dtype, int ib_dtype, hipStream_t stream) {
    if (io_dtype == 0) return launch_st<K, float, PER_K, GATE>(a, st_dtype, ib_dtype, stream);
    return launch_st<K, bf16_t, PER_K, GATE>(a, st_dtype, ib_dtype, stream);
}

template <int K>
hipError_t launch_k(const RecurrentArgs& a, int io_dtype, int st_dtype, int ib_dtype, bool per_k, bool gated,
                    hipStream_t stream) {
    if (per_k) return launch_io<K, true, 0>(a, io_dtype, st_dtype, ib_dtype, stream);
    if (gated && a.qk_l2norm) return launch_io<K, false, 2>(a, io_dtype, st_dtype, ib_dtype, stream);
    if (gated) return launch_io<K, false, 1>(a, io_dtype, st_dtype, ib_dtype, stream);
    return launch_io<K, false, 0>(a, io_dtype, st_dtype, ib_dtype, stream);
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a, int K, int io_dtype, int st_dtype, int ib_dtype,
                            bool per_k, bool gated, hipStream_t stream) {
    if (per_k && gated) return hipErrorInvalidValue;
    if (a.T < 1) return hipErrorInvalidValue;  // the kernel reads one token per sequence up front
    if (K == 64) return launch_k<64>(a, io_dtype, st_dtype, ib_dtype, per_k, gated, stream);
    return launch_k<128>(a, io_dtype, st_dtype, ib_dtype, per_k, gated, stream);
}

}  // namespace gdr
