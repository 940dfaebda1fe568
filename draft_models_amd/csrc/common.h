// Shared device-side definitions for the gfx950 MLA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// 8-element MFMA operand fragment of one lane: 8 consecutive elements of the
// contraction axis. bf16: one 16-byte register quad; fp32: two.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { floatx8 v; };

__device__ __forceinline__ void load_frag(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_frag(Frag<float>& f, const float* p) {
  f.v = *reinterpret_cast<const floatx8*>(p);
}

// acc[16x16] += A(16 rows x 32) * B(32 x 16 cols). Lane l supplies row/col
// (l % 16) and contraction elements 8 * (l / 16) .. + 7 of both operands; the
// result holds rows 4 * (l / 16) + i, column l % 16 in acc[i]. The hardware's
// own order of the contraction elements does not matter as long as A and B
// use the same lane/element -> k assignment, which they do.
__device__ __forceinline__ floatx4 mfma16(const Frag<bf16>& a, const Frag<bf16>& b, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(const Frag<float>& a, const Frag<float>& b, floatx4 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  return acc;
}

// 16-byte vector of T.
template <typename T> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef floatx4 type; static constexpr int n = 4; };

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Reductions over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the rows of one
// MFMA output column) with the gfx950 VALU lane swaps: permlane16_swap(x, x)
// returns {x[l], x[l ^ 16]} in every lane, permlane32_swap(x, x) returns
// {x[l], x[l ^ 32]} (in some order), so no LDS round trip is needed.
__device__ __forceinline__ float red4_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
__device__ __forceinline__ float red4_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  const uint32_t v = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// Reductions over the lane pair l, l ^ 32 (the two halves of a 32x32 MFMA
// output column) with one permlane32_swap.
__device__ __forceinline__ float red2_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
__device__ __forceinline__ float red2_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds_base + 16 l. Issued through inline
// asm so that the compiler does not treat later LDS reads as aliasing the
// in-flight copy; completion is tracked by the caller with an explicit
// vmcnt wait followed by a workgroup barrier.
__device__ __forceinline__ void dma16(const void* gptr, const void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}

// Same copy with a scalar base address and a 32-bit per-lane byte offset
// (the saddr form: no 64-bit vector address per lane); lds_addr is the
// wave-uniform LDS byte address of the destination.
__device__ __forceinline__ void dma16_sbase(uint32_t voff_bytes, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff_bytes), "s"(sbase),
               "s"(lds_addr)
               : "memory", "m0");
}

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Workgroup barrier that the compiler may not move memory accesses across,
// without the vmcnt(0) that __syncthreads implies (prefetches stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// vmcnt(n) with expcnt / lgkmcnt unconstrained (gfx9 s_waitcnt encoding)
#define MLA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

// 2^x with the hardware instruction (v_exp_f32; results below 2^-126 flush to
// zero, which is harmless for softmax weights)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// logistic sigmoid with the hardware reciprocal (v_rcp_f32, ~1 ulp)
__device__ __forceinline__ float sigmoidf(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace mla
