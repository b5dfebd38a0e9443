// Achievable-peak microbenchmarks for the roofline denominators: the rate the
// MI355X's fp16 matrix cores and its HBM deliver to a kernel that does nothing
// else.  The attention kernels are reported against both these measured peaks
// and the published ones.  Used only by the benchmark; not part of the C ABI of
// the attention library.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Four independent accumulator chains of v_mfma_f32_32x32x16_f16 per wave, so
// that the matrix pipe never waits for a result.  Operands come from the lane
// index so the compiler cannot fold them.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
        b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
    }
    f16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming read of n16 16-byte words: each workgroup reads one contiguous
// chunk of the buffer, U independent non-temporal 16-byte loads per lane in
// flight per step (consecutive lanes read consecutive words), folded by xor
// so every byte is used.
template <int U>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u4* __restrict__ src, int64_t n16,
                                                       uint32_t* out) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < n16 ? beg + per : n16;
    int64_t i = beg + threadIdx.x;
    u4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * 256 < end; i += U * 256) {
        u4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= x[u];
    }
    for (; i < end; i += 256) acc ^= __builtin_nontemporal_load(src + i);
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// Enqueue the matrix-core probe: `blocks` workgroups of 4 waves, each wave
// issuing 4 * iters products (32768 flops each).  out: device, blocks * 256
// floats.  Returns 0 or a HIP error code.
int peak_mfma_f16(float* out, int blocks, int iters, hipStream_t stream) {
    if (!out || blocks < 1 || iters < 1) return -1;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}

// Enqueue the HBM read probe over src (device, n16 16-byte words), with
// `unroll` (4, 8 or 16) loads per lane in flight.  out: device, blocks * 256
// uint32.  Returns 0 or a HIP error code.
int peak_hbm_read(const void* src, long long n16, uint32_t* out, int blocks, int unroll,
                  hipStream_t stream) {
    if (!src || !out || n16 < 1 || blocks < 1) return -1;
    auto k = unroll >= 16 ? hbm_read_kernel<16> : unroll >= 8 ? hbm_read_kernel<8>
                                                              : hbm_read_kernel<4>;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(256), 0, stream, (const u4*)src, (int64_t)n16, out);
    return (int)hipGetLastError();
}

}  // extern "C"
