// Measurement probe, not part of the gated-delta-rule path: a kernel that keeps every SIMD's
// matrix core busy with back-to-back dense bf16 products (v_mfma_f32_16x16x32_bf16), so that the
// benchmark can price the chunked prefill against a measured MFMA rate as well as the nominal one.
// Built into its own library (libgdr_probe.so); libgdr.so does not contain it.
//
// Two operand modes: 0 = a few bit patterns per lane (the rate the matrix cores reach when little
// toggles), 1 = hashed, random-looking finite bf16 operands (closer to real data, which draws more
// power and can run at a lower clock).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int kChains = 8;  // independent accumulators per wave: enough to cover the product latency

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// No launch bound: with one the compiler placed the accumulators in AGPRs and shuffled them
// through VGPRs every iteration, which halved the rate.
__global__ void mfma_peak_bf16_kernel(int iters, int mode, float* out) {
    const uint32_t t = threadIdx.x + 977u * blockIdx.x;
    uint4 ra, rb;
    if (mode == 0) {
        ra.x = 0x3F803F80u ^ (t & 0x007F007Fu);
        ra.y = 0x3F003F00u ^ ((t >> 3) & 0x007F007Fu);
        ra.z = 0xBF403F40u ^ ((t >> 5) & 0x007F007Fu);
        ra.w = 0x3E803E80u ^ ((t >> 7) & 0x007F007Fu);
        rb.x = ra.w ^ 0x00010001u;
        rb.y = ra.z ^ 0x00020002u;
        rb.z = ra.y ^ 0x00040004u;
        rb.w = ra.x ^ 0x00080008u;
    } else {
        // sign and mantissa bits random, exponents in [2^-31, 2^0): finite, no overflow over the loop
        const uint32_t m = 0x80FF80FFu, e = 0x30003000u;
        ra.x = (mix32(4 * t) & (m | 0x0F000F00u)) | e;
        ra.y = (mix32(4 * t + 1) & (m | 0x0F000F00u)) | e;
        ra.z = (mix32(4 * t + 2) & (m | 0x0F000F00u)) | e;
        ra.w = (mix32(4 * t + 3) & (m | 0x0F000F00u)) | e;
        rb.x = (mix32(~(4 * t)) & (m | 0x0F000F00u)) | e;
        rb.y = (mix32(~(4 * t + 1)) & (m | 0x0F000F00u)) | e;
        rb.z = (mix32(~(4 * t + 2)) & (m | 0x0F000F00u)) | e;
        rb.w = (mix32(~(4 * t + 3)) & (m | 0x0F000F00u)) | e;
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ra);
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, rb);
    f32x4_t acc[kChains];
    for (int j = 0; j < kChains; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
    for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Dense flops one launch performs: blocks x 4 waves x iters x kChains products of 16x16x32.
__attribute__((visibility("default"))) double gdr_probe_mfma_bf16_flops(int32_t blocks, int32_t iters) {
    return (double)blocks * 4.0 * (double)iters * kChains * (2.0 * 16 * 16 * 32);
}

// Launch on `stream` (blocks of 256 threads): `out` must hold blocks * 256 floats.  mode 0 or 1
// (see above).  Returns the hipError_t of the launch.
__attribute__((visibility("default"))) int gdr_probe_mfma_bf16(int32_t blocks, int32_t iters, int32_t mode,
                                                               float* out, void* stream) {
    if (blocks <= 0 || iters <= 0 || !out || (mode != 0 && mode != 1)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_bf16_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                       mode, out);
    return (int)hipGetLastError();
}

}  // extern "C"
