// Achievable-peak probes for the roofline figures (gfx950): a streaming copy
// (the HBM bandwidth a plain kernel reaches) and a loop of independent bf16
// MFMA products (the matrix-core rate a plain kernel reaches).  They are
// measurement kernels, built as their own library (libssd_probe.so) beside
// libssd.so; the SSD path does not use them.
//
// C entry points (host pointers to device memory, asynchronous on `stream`,
// 0 on success, -1 on bad arguments, -2 on a HIP launch error):
//   ssd_probe_copy(src, dst, bytes, stream)
//     dst[0, bytes) = src[0, bytes); bytes a multiple of 4096, both pointers
//     16-byte aligned.  One workgroup of 64 threads moves 4 KiB (256 16-byte
//     elements), every lane issuing its four 16-byte loads before its four
//     stores; the grid is bytes / 4096 workgroups.
//   ssd_probe_mfma(out, blocks, iters, shape, stream)
//     `blocks` workgroups of 256 threads; every wave runs `iters` rounds of
//     8 independent v_mfma_f32_16x16x32_bf16 (shape 16, 16*16*32*2 flops
//     each) or 4 independent v_mfma_f32_32x32x16_bf16 (shape 32, 32*32*16*2
//     flops each) on constant operands a = b = 1/64.  Chain c starts from c
//     (distinct chains, which the compiler cannot merge), so after the loop its
//     accumulator elements equal c + iters * K / 4096 (K = 32 or 16).
//     out[blocks * 256] receives, per thread, the sum of its 8 * 4 or 4 * 16
//     accumulator elements, so the products are not dead code and the run is
//     checkable.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int MFMA_CHAINS = 8;    // independent products per wave, 16x16x32
constexpr int MFMA32_CHAINS = 4;  // the same for 32x32x16 (16 accumulators each)

// workgroup w copies 16-byte elements 256 w .. 256 w + 255: lane t takes t, t + 64,
// t + 128 and t + 192 of them
__global__ void __launch_bounds__(64) k_probe_copy(const f32x4* __restrict__ src,
                                                   f32x4* __restrict__ dst) {
    const int64_t base = (int64_t)blockIdx.x * 256 + threadIdx.x;
    f32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = src[base + q * 64];
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[base + q * 64] = v[q];
}

__global__ void __launch_bounds__(256) k_probe_mfma16(float* __restrict__ out, int iters) {
    bf16x8 a;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = (__bf16)(1.f / 64.f);
    f32x4 acc[MFMA_CHAINS];
#pragma unroll
    for (int c = 0; c < MFMA_CHAINS; ++c) acc[c] = f32x4{(float)c, (float)c, (float)c, (float)c};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < MFMA_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < MFMA_CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) k_probe_mfma32(float* __restrict__ out, int iters) {
    typedef __attribute__((ext_vector_type(16))) float f32x16;
    bf16x8 a;
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = (__bf16)(1.f / 64.f);
    f32x16 acc[MFMA32_CHAINS];
#pragma unroll
    for (int c = 0; c < MFMA32_CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = (float)c;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < MFMA32_CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < MFMA32_CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int ssd_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || bytes % 4096 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16)
        return -1;
    // workgroup w covers 16-byte elements [256 w, 256 w + 256)
    const size_t blocks = bytes / 4096;
    if (blocks > 0x7fffffffu) return -1;
    hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)blocks), dim3(64), 0, (hipStream_t)stream,
                       (const f32x4*)src, (f32x4*)dst);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ssd_probe_mfma(float* out, int32_t blocks, int32_t iters, int32_t shape, void* stream) {
    if (!out || blocks <= 0 || iters <= 0 || (shape != 16 && shape != 32)) return -1;
    hipLaunchKernelGGL(shape == 16 ? k_probe_mfma16 : k_probe_mfma32, dim3((unsigned)blocks),
                       dim3(256), 0, (hipStream_t)stream, out, (int)iters);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// flops of one ssd_probe_mfma call, for the caller's rate (16384 flops per
// 16x16x32 instruction, 32768 per 32x32x16 instruction)
double ssd_probe_mfma_flops(int32_t blocks, int32_t iters, int32_t shape) {
    const double per = shape == 16 ? MFMA_CHAINS * (16.0 * 16.0 * 32.0 * 2.0)
                                   : MFMA32_CHAINS * (32.0 * 32.0 * 16.0 * 2.0);
    return (double)blocks * 4.0 * iters * per;
}

}  // extern "C"
