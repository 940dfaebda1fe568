// Absorbed-form MLA decode attention (MLA blog, the decode branch and the
// forward_mqa listing). Every head's query lives in latent space:
// q_lat[h] = [q_nope[h] W_UK[h] (c dims) | rope(q_pe[h]) (r dims)], and all
// heads attend to the same E = c + r wide cache entries (one shared latent
// head, MQA-style). The value is the first c dims of the same entries, so the
// output stays in latent space (c wide); W_UV maps it to v_head_dim later.
//
// The key axis of each sequence is cut into `splits` chunks (split-KV, as
// the listing sizes its KV splits from the longest sequence); each
// workgroup handles one (sequence, chunk, group of 64 heads) and writes a
// partial output normalised by its own softmax sum plus its log-sum-exp. A
// second kernel merges the partials by log-sum-exp weights, the same merge
// the forward_mha listing uses for its prefix/suffix attentions; chunks with
// no visible key get weight zero.
//
// Inside a workgroup the 4 wavefronts own 16 heads each. Scores are computed
// transposed (S^T = C q_lat^T over 32-key tiles) so that each lane holds the
// probabilities of one head for 8 keys -- the B-operand layout of the
// latent P C product. The cache tile is staged once in LDS per workgroup,
// row-major for the score product and transposed ([dim][key]) for the
// value product. This kernel serves fp32 and latent widths other than
// 512 + 64; the bf16 512 + 64 latent takes the stream-K kernel
// (attn_decode_sk.hip).
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void lds4(Frag<bf16>& f, int o, const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  f.v[o] = v[0]; f.v[o + 1] = v[1]; f.v[o + 2] = v[2]; f.v[o + 3] = v[3];
}
__device__ __forceinline__ void lds4(Frag<float>& f, int o, const float* p) {
  floatx4 v = *reinterpret_cast<const floatx4*>(p);
  f.v[o] = v[0]; f.v[o + 1] = v[1]; f.v[o + 2] = v[2]; f.v[o + 3] = v[3];
}
__device__ __forceinline__ void lds_frag(Frag<bf16>& f, const bf16* p) { f.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void lds_frag(Frag<float>& f, const float* p) {
  floatx4 lo = *reinterpret_cast<const floatx4*>(p), hi = *reinterpret_cast<const floatx4*>(p + 4);
  f.v = floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void glb_frag(Frag<bf16>& f, const bf16* p) { f.v = *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void glb_frag(Frag<float>& f, const float* p) { lds_frag(f, p); }

__device__ __forceinline__ void decode_interval(const DecodeAttnArgs& a, int b, int& L, int& lo, int& hi) {
  L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int p = L - 1;
  if (a.mask.kind == 2) lo = max(0, p - a.mask.window + 1);
  else lo = 0;
  hi = L;
}

template <typename T, int EP, int CP>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  using V16 = typename Vec16<T>::type;
  constexpr int BKEY = 32;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CROW = EP + VEC;      // row-major tile row (elements)
  constexpr int TROW = BKEY + VEC;    // transposed tile row
  constexpr int KS = EP / 32;
  constexpr int DB = CP / 16;
  __shared__ __attribute__((aligned(16))) T Cs[BKEY * CROW];
  __shared__ __attribute__((aligned(16))) T Ct[CP * TROW];

  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int h = hg * 64 + wave * 16 + lr;
  const bool hok = h < a.H;

  int L, lo, hi;
  decode_interval(a, b, L, lo, hi);
  const int k_begin = lo + split * a.chunk;
  const int k_end = min(hi, k_begin + a.chunk);

  const int64_t pidx = ((int64_t)b * a.splits + split) * a.H;
  if (k_begin >= k_end) {
    // empty chunk: log-sum-exp -inf (weight zero in the merge)
    if (tid < 64 && hg * 64 + tid < a.H) a.part_lse[pidx + hg * 64 + tid] = -INFINITY;
    return;
  }

  // latent query of this lane's head (B operand: column = head)
  Frag<T> qf[KS];
  {
    const T* ql = reinterpret_cast<const T*>(a.ql) + (int64_t)b * a.ldql + (int64_t)(hok ? h : 0) * a.c;
    const T* qp = reinterpret_cast<const T*>(a.q) + (int64_t)b * a.ldq + (int64_t)(hok ? h : 0) * a.qk_head + a.n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int e = ks * 32 + g * 8;
      if (hok && e < a.c) glb_frag(qf[ks], ql + e);
      else if (hok && e < a.c + a.r) glb_frag(qf[ks], qp + (e - a.c));
      else qf[ks].v = {};
    }
  }

  floatx4 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * kLog2e;
  const T* cache = reinterpret_cast<const T*>(a.cache);
  const int E = a.c + a.r;
  constexpr int VPR = EP / VEC;

  for (int k0 = k_begin; k0 < k_end; k0 += BKEY) {
    for (int v = tid; v < BKEY * VPR; v += 256) {
      const int jj = v / VPR, col = (v % VPR) * VEC;
      const int key = k0 + jj;
      V16 val = {};
      if (key < k_end && col < E) {
        const int blk = a.block_table[(int64_t)b * a.max_blocks + key / a.page];
        if (blk >= 0 && blk < a.num_blocks)
          val = *reinterpret_cast<const V16*>(cache + ((int64_t)blk * a.page + key % a.page) * E + col);
      }
      *reinterpret_cast<V16*>(&Cs[jj * CROW + col]) = val;
      if (col < CP) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) Ct[(col + e) * TROW + jj] = (col + e < a.c) ? val[e] : T(0.f);
      }
    }
    __syncthreads();

    floatx4 s[2];
    s[0] = floatx4{0.f, 0.f, 0.f, 0.f};
    s[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<T> cf;
        lds_frag(cf, &Cs[(kb * 16 + lr) * CROW + ks * 32 + g * 8]);
        s[kb] = mfma16(cf, qf[ks], s[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + g * 4 + i;
        const float x = key < k_end ? s[kb][i] * sl2 : -INFINITY;
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);  // finite: every tile has a visible key
    const float alpha = fast_exp2(m - mnew);
    float sum = 0.f;
    Frag<T> pf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(s[kb][i] - mnew);
        sum += p;
        pf.v[kb * 4 + i] = from_f32<T>(p);
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    l = l * alpha + sum;
    m = mnew;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      Frag<T> vf;
      const T* row = &Ct[(d * 16 + lr) * TROW + g * 4];
      lds4(vf, 0, row);
      lds4(vf, 4, row + 16);
      o[d] = mfma16(vf, pf, o[d] * alpha);
    }
    __syncthreads();
  }

  if (!hok) return;
  const float inv = 1.f / l;
  float* po = a.part_o + (pidx + h) * a.c;
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    const int d0 = d * 16 + g * 4;
    if (d0 + 3 < a.c) {
      *reinterpret_cast<floatx4*>(po + d0) = o[d] * inv;
    } else {
      for (int i = 0; i < 4; ++i)
        if (d0 + i < a.c) po[d0 + i] = o[d][i] * inv;
    }
  }
  if (g == 0) a.part_lse[pidx + h] = m + log2f(l);  // log2 domain
}

// o_lat[b, h, :] = sum_s w_s part_o[b, s, h, :] / sum_s w_s, w_s = 2^(lse_s - max lse)
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeAttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t base = (int64_t)b * a.splits * a.H + h;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.part_lse[base + (int64_t)s * a.H]);
  T* dst = reinterpret_cast<T*>(a.o_lat) + ((int64_t)b * a.H + h) * a.c;
  if (mx == -INFINITY) {
    for (int d = threadIdx.x; d < a.c; d += 256) dst[d] = from_f32<T>(0.f);
    return;
  }
  float den = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float ls = a.part_lse[base + (int64_t)s * a.H];
    if (ls != -INFINITY) den += fast_exp2(ls - mx);
  }
  const float inv = 1.f / den;
  for (int d = threadIdx.x; d < a.c; d += 256) {
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float ls = a.part_lse[base + (int64_t)s * a.H];
      if (ls == -INFINITY) continue;
      acc += fast_exp2(ls - mx) * a.part_o[(base + (int64_t)s * a.H) * a.c + d];
    }
    dst[d] = from_f32<T>(acc * inv);
  }
}

template <typename T, int EP, int CP>
hipError_t launch_dims(const DecodeAttnArgs& a, hipStream_t s) {
  dim3 grid(a.splits, (a.H + 63) / 64, a.batch);
  hipLaunchKernelGGL((decode_attn_kernel<T, EP, CP>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeAttnArgs& a, hipStream_t s) {
  const int E = a.c + a.r;
  if (E <= 64 && a.c <= 48) return launch_dims<T, 64, 48>(a, s);
  if (E <= 576 && a.c <= 512) return launch_dims<T, 576, 512>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

const char* decode_attn_check(const DecodeAttnArgs& a, bool is_bf16) {
  const int vec = is_bf16 ? 8 : 4;
  if (a.c + a.r > 576 || a.c > 512) return "decode attention: kv_lora_rank + rope above 512 + 64 is not supported";
  if (a.c % 8 || a.r % vec) return "decode attention: kv_lora_rank must be a multiple of 8 and rope a 16-byte multiple";
  if (a.ldql % vec || a.ldq % vec || a.qk_head % vec || a.n % vec) return "decode attention: strides must be 16-byte multiples";
  if (a.chunk <= 0 || a.splits <= 0) return "decode attention: bad split";
  return nullptr;
}

hipError_t decode_attn_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  return is_bf16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

hipError_t decode_merge_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  if (is_bf16) hipLaunchKernelGGL(decode_combine_kernel<bf16>, dim3(a.H, a.batch), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(a.H, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
