// Device-side helpers shared by the gfx950 kernels of libgdr: element types,
// vector loads/stores with fp32 <-> bf16 conversion, and 16-lane DPP reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Storage tags: fp32 is `float`, bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Two floats -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32), packed lo|hi<<16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t x = {lo, hi};
    bf16x2_t y = __builtin_convertvector(x, bf16x2_t);
    return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// ---- scalar element access -------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float load(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
    __device__ __forceinline__ static void store(void* p, int64_t i, float x) { static_cast<float*>(p)[i] = x; }
};
template <> struct Elem<bf16_t> {
    static constexpr int bytes = 2;
    __device__ __forceinline__ static float load(const void* p, int64_t i) {
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    __device__ __forceinline__ static void store(void* p, int64_t i, float x) {
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
    }
};

// ---- vector access: N consecutive elements (N*bytes in {8, 16, 32}) ----------
template <typename T, int N> struct Vec;

template <int N> struct Vec<float, N> {
    static_assert(N % 4 == 0, "fp32 vectors are whole float4s");
    __device__ __forceinline__ static void load(const void* p, int64_t i, float* out) {
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            f32x4_t x = src[j];
            out[4 * j + 0] = x[0];
            out[4 * j + 1] = x[1];
            out[4 * j + 2] = x[2];
            out[4 * j + 3] = x[3];
        }
    }
    __device__ __forceinline__ static void store(void* p, int64_t i, const float* in) {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i);
#pragma unroll
        for (int j = 0; j < N / 4; ++j) dst[j] = f32x4_t{in[4 * j], in[4 * j + 1], in[4 * j + 2], in[4 * j + 3]};
    }
};

template <int N> struct Vec<bf16_t, N> {
    static_assert(N == 4 || N == 8, "bf16 vectors are 8 or 16 bytes");
    __device__ __forceinline__ static void load(const void* p, int64_t i, float* out) {
        const uint16_t* base = static_cast<const uint16_t*>(p) + i;
        if constexpr (N == 8) {
            uint4 w = *reinterpret_cast<const uint4*>(base);
            uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[2 * j] = __uint_as_float(ws[j] << 16);
                out[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
            }
        } else {
            uint2 w = *reinterpret_cast<const uint2*>(base);
            out[0] = __uint_as_float(w.x << 16);
            out[1] = __uint_as_float(w.x & 0xFFFF0000u);
            out[2] = __uint_as_float(w.y << 16);
            out[3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
    }
    __device__ __forceinline__ static void store(void* p, int64_t i, const float* in) {
        uint16_t* base = static_cast<uint16_t*>(p) + i;
        if constexpr (N == 8) {
            uint4 w;
            w.x = pack_bf16x2(in[0], in[1]);
            w.y = pack_bf16x2(in[2], in[3]);
            w.z = pack_bf16x2(in[4], in[5]);
            w.w = pack_bf16x2(in[6], in[7]);
            *reinterpret_cast<uint4*>(base) = w;
        } else {
            uint2 w;
            w.x = pack_bf16x2(in[0], in[1]);
            w.y = pack_bf16x2(in[2], in[3]);
            *reinterpret_cast<uint2*>(base) = w;
        }
    }
};

// ---- LDS staging: raw element type, and N consecutive elements read back as fp32 ----
template <typename T> struct RawT;
template <> struct RawT<float> { typedef float T; };
template <> struct RawT<bf16_t> { typedef uint16_t T; };

template <typename T, int N> struct LdsVec;

template <int N> struct LdsVec<float, N> {
    static_assert(N % 4 == 0, "fp32 vectors are whole float4s");
    __device__ __forceinline__ static void get(const float* p, float* out) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            const f32x4_t x = reinterpret_cast<const f32x4_t*>(p)[j];
            out[4 * j + 0] = x[0];
            out[4 * j + 1] = x[1];
            out[4 * j + 2] = x[2];
            out[4 * j + 3] = x[3];
        }
    }
};

template <int N> struct LdsVec<bf16_t, N> {
    static_assert(N == 4 || N == 8, "bf16 vectors are 8 or 16 bytes");
    __device__ __forceinline__ static void get(const uint16_t* p, float* out) {
        if constexpr (N == 8) {
            const uint4 w = *reinterpret_cast<const uint4*>(p);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[2 * j] = __uint_as_float(ws[j] << 16);
                out[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
            }
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(p);
            out[0] = __uint_as_float(w.x << 16);
            out[1] = __uint_as_float(w.x & 0xFFFF0000u);
            out[2] = __uint_as_float(w.y << 16);
            out[3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
    }
};

// ---- loads through a buffer resource: bytes past the resource's range read as zero ----
template <typename T, int N> struct BufVec;

// cache-policy operand of the buffer loads: 0 = default, kNonTemporal = streaming data read once
// (the nt bit: the lines are the first to be replaced)
constexpr int kNonTemporal = 2;

template <int N> struct BufVec<float, N> {
    static_assert(N % 4 == 0, "fp32 vectors are whole float4s");
    template <int AUX = 0>
    __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float* out) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * j, 0, AUX));
            out[4 * j + 0] = x[0];
            out[4 * j + 1] = x[1];
            out[4 * j + 2] = x[2];
            out[4 * j + 3] = x[3];
        }
    }
};

template <int N> struct BufVec<bf16_t, N> {
    static_assert(N == 4 || N == 8, "bf16 vectors are 8 or 16 bytes");
    template <int AUX = 0>
    __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, uint32_t off, float* out) {
        if constexpr (N == 8) {
            const uint4 w = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[2 * j] = __uint_as_float(ws[j] << 16);
                out[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
            }
        } else {
            const uint2 w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
            out[0] = __uint_as_float(w.x << 16);
            out[1] = __uint_as_float(w.x & 0xFFFF0000u);
            out[2] = __uint_as_float(w.y << 16);
            out[3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
    }
};

// Cache-policy operand of buffer stores: kWriteThrough = device scope (sc1), the store is written
// through the caches toward memory.  For state written once and not read again in the call.
constexpr int kWriteThrough = 16;

// N converted elements of a row stored as one or two 16-byte (or one 8-byte) vectors through a
// buffer resource, byte offset `off`, cache policy AUX
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <typename T, int N> struct BufStore;
template <int N> struct BufStore<float, N> {
    static_assert(N % 4 == 0, "fp32 vectors are whole float4s");
    template <int AUX>
    __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* in) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, f32x4_t{in[4 * j], in[4 * j + 1], in[4 * j + 2], in[4 * j + 3]}), r,
                off + 16 * j, 0, AUX);
    }
};
template <int N> struct BufStore<bf16_t, N> {
    static_assert(N == 4 || N == 8, "bf16 vectors are 8 or 16 bytes");
    template <int AUX>
    __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* in) {
        if constexpr (N == 8) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                                                           pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7])},
                                                   r, off, 0, AUX);
        } else {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3])}, r,
                                                  off, 0, AUX);
        }
    }
};

// ---- raw (unconverted) vectors, so loads can be issued well before their use ----
template <typename T, int N> struct RawVec;
template <int N> struct RawVec<float, N> {
    static_assert(N % 4 == 0, "fp32 raw vectors are whole float4s");
    f32x4_t v[N / 4];
    __device__ __forceinline__ void load(const void* p, int64_t i) {
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
#pragma unroll
        for (int j = 0; j < N / 4; ++j) v[j] = src[j];
    }
    __device__ __forceinline__ void get(float* out) const {
#pragma unroll
        for (int j = 0; j < N; ++j) out[j] = v[j / 4][j % 4];
    }
};
template <int N> struct RawVec<bf16_t, N> {
    static_assert(N == 4 || N == 8, "bf16 raw vectors are 8 or 16 bytes");
    uint32_t w[N / 2];
    __device__ __forceinline__ void load(const void* p, int64_t i) {
        const uint16_t* base = static_cast<const uint16_t*>(p) + i;
        if constexpr (N == 8) {
            const uint4 x = *reinterpret_cast<const uint4*>(base);
            w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        } else {
            const uint2 x = *reinterpret_cast<const uint2*>(base);
            w[0] = x.x; w[1] = x.y;
        }
    }
    __device__ __forceinline__ void get(float* out) const {
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            out[2 * j] = __uint_as_float(w[j] << 16);
            out[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
};

// One element held as its bits.
template <typename T> struct RawElem;
template <> struct RawElem<float> {
    float x;
    __device__ __forceinline__ void load(const void* p, int64_t i) { x = static_cast<const float*>(p)[i]; }
    __device__ __forceinline__ float get() const { return x; }
};
template <> struct RawElem<bf16_t> {
    uint32_t x;
    __device__ __forceinline__ void load(const void* p, int64_t i) { x = static_cast<const uint16_t*>(p)[i]; }
    __device__ __forceinline__ float get() const { return __uint_as_float(x << 16); }
};

// ---- 16-lane reductions through DPP ----------------------------------------
// Lanes are grouped in DPP rows of 16.  After the four steps every lane of the row
// holds the same, bitwise-identical sum (each step adds the same two operands in
// both partner lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^1
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^2
    x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <-> 7-i within each half row
    x += dpp_mov<0x140>(x);  // row_mirror: lane i <-> 15-i within the row
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.  row_shr steps (lanes shifted in from
// outside the 16-lane row read 0) scan each DPP row; row_bcast:15 then adds row 0's total to
// row 1 and row 2's to row 3, and row_bcast:31 adds the total of rows 0-1 to rows 2-3 (rows
// outside the row mask keep the 0 passed as the old value).
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, BOUND_ZERO));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_or_zero<0x111, 0xF, true>(x);   // row_shr:1
    x += dpp_or_zero<0x112, 0xF, true>(x);   // row_shr:2
    x += dpp_or_zero<0x114, 0xF, true>(x);   // row_shr:4
    x += dpp_or_zero<0x118, 0xF, true>(x);   // row_shr:8
    x += dpp_or_zero<0x142, 0xA, false>(x);  // row_bcast:15
    x += dpp_or_zero<0x143, 0xC, false>(x);  // row_bcast:31
    return x;
}

__device__ __forceinline__ float exp_f32(float x) {
    // e^x = 2^(x * log2(e)); v_exp_f32 evaluates 2^y.
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---- gating front (FlashQLA PR #1: host-gating and in-kernel gated verify commits) ----
// log(1 + e) for e >= 0 from the hardware log2: log(u) e / (u - 1) with u = fl(1 + e) cancels
// the rounding of 1 + e, and u == 1 means log(1 + e) = e to fp32 precision.  This is the method of
// D. Goldberg, "What Every Computer Scientist Should Know About Floating-Point Arithmetic" (ACM
// Computing Surveys 23(1), 1991), Theorem 4.  A few ulps; no table constants, so it costs few
// registers.
__device__ __forceinline__ float log1p_nonneg_f32(float e) {
    const float u = 1.0f + e;
    const float d = u - 1.0f;
    const float r = __builtin_amdgcn_logf(u) * 0.69314718055994531f * (e * __builtin_amdgcn_rcpf(d));
    return d == 0.0f ? e : r;
}

// softplus with beta 1 and threshold 20: inputs above 20 pass through unchanged.  Both sides
// are evaluated and selected (no branch), so the token loop stays one basic block.
__device__ __forceinline__ float softplus_f32(float x) {
    const float smooth = log1p_nonneg_f32(exp_f32(fminf(x, 20.0f)));
    return x > 20.0f ? x : smooth;
}

// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp); 0 once e^-x overflows
__device__ __forceinline__ float sigmoid_f32(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_f32(-x)); }

// decay g = -exp(A_log) softplus(a + dt_bias), with neg_exp_a_log = -exp(A_log) of the head
__device__ __forceinline__ float gate_decay(float a, float neg_exp_a_log, float dt_bias) {
    return neg_exp_a_log * softplus_f32(a + dt_bias);
}

}  // namespace gdr
