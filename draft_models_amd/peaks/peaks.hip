// Measured roofline denominators of an MI355X: HBM bandwidth of a plain
// 16-byte-per-lane copy and of a plain read (sum) over buffers far larger
// than the 256 MB Infinity Cache, and the issue rate of the bf16 matrix
// cores in a loop of independent MFMA chains with no memory traffic.
// Measurement tooling beside the MLA library (its own shared object); every
// kernel has a fixed trip count.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PEAKS_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// every lane sums the words it reads; one word per workgroup is written so
// that the loads cannot be removed
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const uint4 v = src[i];
    acc += v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int j = 0; j < 256; ++j) t += red[j];
    out[blockIdx.x] = t;
  }
}

// Each wave runs 4 independent accumulation chains of one MFMA shape for
// `iters` rounds (operands held in registers).
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float seed, float* out) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(threadIdx.x - e));
  }
  float sum = 0.f;
  if constexpr (SHAPE == 32) {
    floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int e = 0; e < 16; ++e) sum += c0[e] + c1[e] + c2[e] + c3[e];
  } else {
    floatx4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
    }
    for (int e = 0; e < 4; ++e) sum += c0[e] + c1[e] + c2[e] + c3[e];
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = sum;
}

}  // namespace

// dst[i] = src[i] for `bytes` bytes (a multiple of 16); grid of `blocks` x 256 lanes
PEAKS_API int peaks_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// reads `bytes` bytes of src; out: `blocks` uint32 words
PEAKS_API int peaks_read(const void* src, int64_t bytes, int blocks, void* out, void* stream) {
  if (!src || !out || bytes <= 0 || bytes % 16 || blocks <= 0) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// `blocks` workgroups of 4 waves, each wave 4 x iters MFMAs of the given shape
// (32: 32x32x16 bf16, 32768 flops each; 16: 16x16x32 bf16, 16384 flops);
// out: blocks * 256 floats
PEAKS_API int peaks_mfma(int shape, int iters, int blocks, void* out, void* stream) {
  if (!out || iters <= 0 || blocks <= 0 || (shape != 16 && shape != 32)) return 1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (shape == 32) hipLaunchKernelGGL(mfma_kernel<32>, dim3(blocks), dim3(256), 0, s, iters, 1e-3f, static_cast<float*>(out));
  else hipLaunchKernelGGL(mfma_kernel<16>, dim3(blocks), dim3(256), 0, s, iters, 1e-3f, static_cast<float*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
