// Latent RMSNorm, partial RoPE and the cache write of the new tokens.
//
// For each new token (MLA blog, MultiHeadLatentAttentionWrapper.forward and
// do_kv_cache_update listings): the latent kv_c is RMS-normalised with the
// kv_a_layernorm gain, k_pe and the rope part q[..., n:] of every head are
// rotated at the token's logical position, and the entry
// [RMSNorm(kv_c) | RoPE(k_pe)] is stored into its paged-cache slot. The write
// happens before any attention kernel of the same call runs (stream order),
// so each query sees its own entry.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_cache_kernel(RopeCacheArgs a) {
  const int b = blockIdx.y, i = blockIdx.x;
  int t, pos;
  if (a.decode) {
    if (i != 0) return;
    const int L = a.seq_lens[b];
    if (L < 1) return;
    t = b;
    pos = min(L, a.max_seq_len) - 1;
  } else {
    const int cb = a.cu_seqlens ? a.cu_seqlens[b] : b * a.max_q_len;
    int ql = a.cu_seqlens ? a.cu_seqlens[b + 1] - cb : a.max_q_len;
    ql = min(max(ql, 0), a.max_q_len);
    if (i >= ql) return;
    t = cb + i;
    if (t < 0 || t >= a.total_tokens) return;
    const int pl = min(max(a.prefix_lens[b], 0), a.max_kv_len - ql);
    pos = pl + i;
  }
  const int half = a.r / 2;
  const float* cs = a.rope_cos + (int64_t)pos * half;
  const float* sn = a.rope_sin + (int64_t)pos * half;
  auto pair = [&](int j, int& ia, int& ib) {
    if (a.interleaved) { ia = 2 * j; ib = 2 * j + 1; }
    else { ia = j; ib = j + half; }
  };

  // rotate q[t, h, n:] for every head, in place
  T* q = reinterpret_cast<T*>(a.q) + (int64_t)t * a.ldq;
  bool done = false;
  if constexpr (sizeof(T) == 2) {
    if (a.r == 64 && a.ldq % 8 == 0 && a.qk_head % 8 == 0 && a.n % 8 == 0) {
      // thread (h, v) holds dims 8 v .. 8 v + 7 and 32 + 8 v .. of head h's
      // 64 rope dims as two 16-byte vectors: NeoX pairs (j, j + 32) are the
      // same element of both, interleaved pairs (2 j, 2 j + 1) neighbours in one
      for (int p = threadIdx.x; p < a.H * 4; p += 256) {
        const int h = p >> 2, v = p & 3;
        bf16x8* qh = reinterpret_cast<bf16x8*>(q + (int64_t)h * a.qk_head + a.n);
        bf16x8 x0 = qh[v], x1 = qh[v + 4];
        if (a.interleaved) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j0 = 4 * v + e, j1 = 16 + 4 * v + e;
            const float a0 = (float)x0[2 * e], b0 = (float)x0[2 * e + 1];
            const float a1 = (float)x1[2 * e], b1 = (float)x1[2 * e + 1];
            x0[2 * e] = (bf16)(a0 * cs[j0] - b0 * sn[j0]);
            x0[2 * e + 1] = (bf16)(a0 * sn[j0] + b0 * cs[j0]);
            x1[2 * e] = (bf16)(a1 * cs[j1] - b1 * sn[j1]);
            x1[2 * e + 1] = (bf16)(a1 * sn[j1] + b1 * cs[j1]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 8 * v + e;
            const float xa = (float)x0[e], xb = (float)x1[e];
            x0[e] = (bf16)(xa * cs[j] - xb * sn[j]);
            x1[e] = (bf16)(xa * sn[j] + xb * cs[j]);
          }
        }
        qh[v] = x0;
        qh[v + 4] = x1;
      }
      done = true;
    }
  }
  if (!done) {
    for (int p = threadIdx.x; p < a.H * half; p += 256) {
      const int h = p / half, j = p % half;
      int ia, ib;
      pair(j, ia, ib);
      T* qh = q + (int64_t)h * a.qk_head + a.n;
      const float xa = to_f32(qh[ia]), xb = to_f32(qh[ib]);
      qh[ia] = from_f32<T>(xa * cs[j] - xb * sn[j]);
      qh[ib] = from_f32<T>(xa * sn[j] + xb * cs[j]);
    }
  }

  // RMSNorm of the latent
  const T* kv = reinterpret_cast<const T*>(a.kv) + (int64_t)t * a.ldkv;
  __shared__ float red[4];
  float ss = 0.f;
  for (int e = threadIdx.x; e < a.c; e += 256) {
    const float f = to_f32(kv[e]);
    ss += f * f;
  }
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float scale = rsqrtf(tot / (float)a.c + a.eps);

  // slot of logical position pos
  if (pos / a.page >= a.max_blocks) return;
  const int blk = a.block_table[(int64_t)b * a.max_blocks + pos / a.page];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int64_t ent = ((int64_t)blk * a.page + pos % a.page) * (a.c + a.r);
  const T* gamma = reinterpret_cast<const T*>(a.gamma_kv);
  const T* kpe = kv + a.c;
  if (a.kv_fp8) {
    // 8-bit entry. The wrapper forward hands the cache update bf16 tensors
    // (kv_c_normed and the roped k_pe of a bf16 model), so each value is
    // rounded to bf16 first; its code is the E4M3 code of value / scale
    // (a correctly rounded fp32 division), rounded to nearest with ties to
    // the even code by the hardware conversion, saturated to +-448.
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.cache) + ent;
    auto code = [&](float v) {
      const float x = fminf(fmaxf((float)(bf16)v / a.kv_scale, -448.f), 448.f);
      return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xff);
    };
    for (int e = threadIdx.x; e < a.c; e += 256) dst[e] = code(to_f32(kv[e]) * scale * to_f32(gamma[e]));
    for (int j = threadIdx.x; j < half; j += 256) {
      int ia, ib;
      pair(j, ia, ib);
      const float xa = to_f32(kpe[ia]), xb = to_f32(kpe[ib]);
      dst[a.c + ia] = code(xa * cs[j] - xb * sn[j]);
      dst[a.c + ib] = code(xa * sn[j] + xb * cs[j]);
    }
    return;
  }
  T* dst = reinterpret_cast<T*>(a.cache) + ent;
  for (int e = threadIdx.x; e < a.c; e += 256) dst[e] = from_f32<T>(to_f32(kv[e]) * scale * to_f32(gamma[e]));
  for (int j = threadIdx.x; j < half; j += 256) {
    int ia, ib;
    pair(j, ia, ib);
    const float xa = to_f32(kpe[ia]), xb = to_f32(kpe[ib]);
    dst[a.c + ia] = from_f32<T>(xa * cs[j] - xb * sn[j]);
    dst[a.c + ib] = from_f32<T>(xa * sn[j] + xb * cs[j]);
  }
}

// bf16 form for a 512 + 64 latent with 16-byte aligned rows: NT tokens per
// workgroup, the three parts of each side by side and every access 16 bytes
// wide, each wavefront's loads for all NT tokens issued before the first is
// used. Wavefronts 0-1 rotate the rope dims of the query heads (a lane holds
// two 16-byte vectors of one head: NeoX pairs (j, j + 32) are the same
// element of both, interleaved pairs neighbours in one), wavefront 2
// normalises the latents (8 dims per lane, one wavefront reduction per token)
// and writes them, wavefront 3 rotates the k_pe (4 lanes per token) and writes
// them. Same arithmetic per value as the general kernel. NT = 4 when there
// are enough tokens for the grid to fill the CUs several times (the pass is
// then bound by HBM read-modify-write), else 1.

// token k of the workgroup: prefill (b = blockIdx.y, i = NT blockIdx.x + k),
// decode (b = NT blockIdx.y + k); false if it does not exist
template <int NT>
__device__ __forceinline__ bool rope_token(const RopeCacheArgs& a, int k, int& b, int& t, int& pos) {
  if (a.decode) {
    b = NT * blockIdx.y + k;
    if (blockIdx.x != 0 || b >= a.batch) return false;
    const int L = a.seq_lens[b];
    if (L < 1) return false;
    t = b;
    pos = min(L, a.max_seq_len) - 1;
    return true;
  }
  b = blockIdx.y;
  const int i = NT * blockIdx.x + k;
  const int cb = a.cu_seqlens ? a.cu_seqlens[b] : b * a.max_q_len;
  int ql = a.cu_seqlens ? a.cu_seqlens[b + 1] - cb : a.max_q_len;
  ql = min(max(ql, 0), a.max_q_len);
  if (i >= ql) return false;
  t = cb + i;
  if (t < 0 || t >= a.total_tokens) return false;
  pos = min(max(a.prefix_lens[b], 0), a.max_kv_len - ql) + i;
  return true;
}

template <int NT>
__global__ __launch_bounds__(256) void rope_cache_bf16_kernel(RopeCacheArgs a) {
  constexpr int C = 512, HALF = 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int tb[NT], tt[NT], tp[NT];
  bool ok[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) ok[k] = rope_token<NT>(a, k, tb[k], tt[k], tp[k]);
  // rotation of the two 16-byte vectors x0 (dims 8 v ..) and x1 (dims 32 + 8 v ..) at position pos
  auto rotate = [&](bf16x8& x0, bf16x8& x1, int v, int pos) {
    const float* cs = a.rope_cos + (int64_t)pos * HALF;
    const float* sn = a.rope_sin + (int64_t)pos * HALF;
    if (a.interleaved) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j0 = 4 * v + e, j1 = 16 + 4 * v + e;
        const float a0 = (float)x0[2 * e], b0 = (float)x0[2 * e + 1];
        const float a1 = (float)x1[2 * e], b1 = (float)x1[2 * e + 1];
        x0[2 * e] = (bf16)(a0 * cs[j0] - b0 * sn[j0]);
        x0[2 * e + 1] = (bf16)(a0 * sn[j0] + b0 * cs[j0]);
        x1[2 * e] = (bf16)(a1 * cs[j1] - b1 * sn[j1]);
        x1[2 * e + 1] = (bf16)(a1 * sn[j1] + b1 * cs[j1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 8 * v + e;
        const float xa = (float)x0[e], xb = (float)x1[e];
        x0[e] = (bf16)(xa * cs[j] - xb * sn[j]);
        x1[e] = (bf16)(xa * sn[j] + xb * cs[j]);
      }
    }
  };
  if (wave < 2) {
    for (int p = threadIdx.x; p < a.H * 4; p += 128) {
      const int h = p >> 2, v = p & 3;
      bf16x8 x0[NT], x1[NT];
      bf16x8* qh[NT];
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        qh[k] = reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.q) + (int64_t)(ok[k] ? tt[k] : 0) * a.ldq +
                                          (int64_t)h * a.qk_head + a.n);
        if (ok[k]) {
          x0[k] = qh[k][v];
          x1[k] = qh[k][v + 4];
        }
      }
#pragma unroll
      for (int k = 0; k < NT; ++k) {
        if (!ok[k]) continue;
        rotate(x0[k], x1[k], v, tp[k]);
        qh[k][v] = x0[k];
        qh[k][v + 4] = x1[k];
      }
    }
    return;
  }
  // cache entry of token k (-1: no slot)
  int64_t ent[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    ent[k] = -1;
    if (!ok[k] || tp[k] / a.page >= a.max_blocks) continue;
    const int blk = a.block_table[(int64_t)tb[k] * a.max_blocks + tp[k] / a.page];
    if (blk >= 0 && blk < a.num_blocks) ent[k] = ((int64_t)blk * a.page + tp[k] % a.page) * (C + 2 * HALF);
  }
  // 8-bit entry: as in the general kernel, each value rounded to bf16 first,
  // then the E4M3 code of value / scale
  auto codes = [&](const float (&v)[8]) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = fminf(fmaxf((float)(bf16)v[e] / a.kv_scale, -448.f), 448.f);
      const uint32_t cd = (uint32_t)(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xff);
      if (e < 4) w0 |= cd << (8 * e);
      else w1 |= cd << (8 * (e - 4));
    }
    return uint2{w0, w1};
  };
  if (wave == 2) {
    bf16x8 x[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k)
      if (ent[k] >= 0)
        x[k] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.kv) + (int64_t)tt[k] * a.ldkv + 8 * lane);
    const bf16x8 gm = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.gamma_kv) + 8 * lane);
#pragma unroll
    for (int k = 0; k < NT; ++k) {
      if (ent[k] < 0) continue;  // uniform over the wavefront
      float f[8], ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = (float)x[k][e];
        ss += f[e] * f[e];
      }
      ss = warp_sum(ss);
      const float scale = rsqrtf(ss / (float)C + a.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * scale * (float)gm[e];
      if (a.kv_fp8) {
        *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(a.cache) + ent[k] + 8 * lane) = codes(f);
      } else {
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)f[e];
        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.cache) + ent[k] + 8 * lane) = y;
      }
    }
    return;
  }
  // wavefront 3: lane 4 k + v rotates chunks v and v + 4 of token k's k_pe
  const int k = lane >> 2, v = lane & 3;
  if (k >= NT) return;
  int64_t e_k = -1;
  int t_k = 0, p_k = 0;
#pragma unroll
  for (int kk = 0; kk < NT; ++kk)
    if (kk == k) { e_k = ent[kk]; t_k = tt[kk]; p_k = tp[kk]; }
  if (e_k < 0) return;
  const bf16x8* kp = reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.kv) + (int64_t)t_k * a.ldkv + C);
  bf16x8 x0 = kp[v], x1 = kp[v + 4];
  rotate(x0, x1, v, p_k);
  if (a.kv_fp8) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(a.cache) + e_k + C;
    float f0[8], f1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f0[e] = (float)x0[e];
      f1[e] = (float)x1[e];
    }
    *reinterpret_cast<uint2*>(dst + 8 * v) = codes(f0);
    *reinterpret_cast<uint2*>(dst + 8 * (v + 4)) = codes(f1);
  } else {
    bf16x8* dst = reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.cache) + e_k + C);
    dst[v] = x0;
    dst[v + 4] = x1;
  }
}

}  // namespace

hipError_t rope_cache_launch(const RopeCacheArgs& a, bool is_bf16, int grid_x, int batch, hipStream_t s) {
  if (grid_x <= 0 || batch <= 0) return hipSuccess;
  dim3 grid(grid_x, batch);
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool fast = is_bf16 && a.c == 512 && a.r == 64 && a.ldq % 8 == 0 && a.qk_head % 8 == 0 && a.n % 8 == 0 &&
                    a.ldkv % 8 == 0 && al16(a.q) && al16(a.kv) && al16(a.gamma_kv) && al16(a.cache);
  if (fast) {
    RopeCacheArgs a4 = a;
    a4.batch = batch;
    const int64_t tokens = a.decode ? batch : (int64_t)grid_x * batch;
    if (tokens >= 8192) {
      const dim3 g4 = a.decode ? dim3(1, (batch + 3) / 4) : dim3((grid_x + 3) / 4, batch);
      hipLaunchKernelGGL(rope_cache_bf16_kernel<4>, g4, dim3(256), 0, s, a4);
    } else {
      hipLaunchKernelGGL(rope_cache_bf16_kernel<1>, grid, dim3(256), 0, s, a4);
    }
  }
  else if (is_bf16) hipLaunchKernelGGL(rope_cache_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(rope_cache_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
