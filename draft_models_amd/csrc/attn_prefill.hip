// Expanded-form MLA attention for prefill (MLA blog, forward_mha listing):
// per head, K = [k_nope (from the kv_b expansion) | k_pe (the one shared rope
// key, read from the latent cache)], V = the expanded v. Flash-style: the key
// axis is streamed through LDS in 64-key tiles with an online softmax, so the
// score matrix never reaches HBM. Queries of a sequence see the cached prefix
// and the new tokens in one pass over [lo, hi), which equals attending to the
// prefix and to the new tokens separately and merging the two results by
// their log-sum-exp (the listing's merge_attn_states step).
//
// Work split (generic kernel): one workgroup = 4 wavefronts x (16 * QB) queries of one head of
// one sequence. Scores are computed transposed (S^T = K Q^T) so that each
// lane ends up holding the probabilities of one query for 8 keys -- exactly
// the B-operand layout of the P V product -- and no LDS round trip of P is
// needed. V is stored transposed in LDS ([d][key]) for the A operand of P V.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void visible(const MaskArgs& m, int t, int p, int L, int& lo, int& hi) {
  if (m.row_lo != nullptr && m.row_hi != nullptr) {
    lo = min(max(m.row_lo[t], 0), L);
    hi = min(max(m.row_hi[t], 0), L);
    return;
  }
  if (m.kind == 0) { lo = 0; hi = L; }
  else if (m.kind == 1) { lo = 0; hi = min(p + 1, L); }
  else { lo = max(0, p - m.window + 1); hi = min(p + 1, L); }
}

template <typename T>
__device__ __forceinline__ void load_frag_g(Frag<T>& f, const T* p, bool ok);
template <>
__device__ __forceinline__ void load_frag_g(Frag<bf16>& f, const bf16* p, bool ok) {
  f.v = ok ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{};
}
template <>
__device__ __forceinline__ void load_frag_g(Frag<float>& f, const float* p, bool ok) {
  floatx4 lo = ok ? *reinterpret_cast<const floatx4*>(p) : floatx4{};
  floatx4 hi = ok ? *reinterpret_cast<const floatx4*>(p + 4) : floatx4{};
  f.v = floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 4 consecutive elements from LDS into fragment slots [o, o+4)
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

template <typename T, int DQK, int DV, int QB>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillAttnArgs a) {
  using V16 = typename Vec16<T>::type;
  constexpr int BKEY = 64;
  constexpr int BQ = 64 * QB;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KROW = DQK + VEC;
  constexpr int VROW = BKEY + VEC;
  constexpr int KS = DQK / 32;   // contraction steps of Q K^T
  constexpr int DB = DV / 16;    // 16-row blocks of O^T
  static_assert(DQK % 32 == 0 && DV % 16 == 0, "padded head dims");
  __shared__ __attribute__((aligned(16))) T Ks[BKEY * KROW];
  __shared__ __attribute__((aligned(16))) T Vt[DV * VROW];
  __shared__ int kmin_s, kmax_s;

  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ql = a.cu_seqlens[b + 1] - a.cu_seqlens[b];
  ql = min(max(ql, 0), a.max_q_len);
  if (qt * BQ >= ql) return;
  const int pl = min(max(a.prefix_lens[b], 0), a.max_kv_len - ql);
  const int L = pl + ql;
  const int t0 = a.cu_seqlens[b];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, g = lane >> 4;
  const float sl2 = a.scale * kLog2e;

  if (tid == 0) { kmin_s = 0x7fffffff; kmax_s = 0; }
  __syncthreads();
  int lo[QB], hi[QB], qi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qi[qb] = qt * BQ + wave * 16 * QB + qb * 16 + lr;
    lo[qb] = 0; hi[qb] = 0;
    if (qi[qb] < ql && t0 + qi[qb] < a.total_tokens) visible(a.mask, t0 + qi[qb], pl + qi[qb], L, lo[qb], hi[qb]);
    if (g == 0 && lo[qb] < hi[qb]) {
      atomicMin(&kmin_s, lo[qb]);
      atomicMax(&kmax_s, hi[qb]);
    }
  }
  __syncthreads();
  const int kbeg = (kmin_s / BKEY) * BKEY, kend = kmax_s;

  // queries in registers (B operand: column = query, 8 contraction elements)
  Frag<T> qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool qok = qi[qb] < ql && t0 + qi[qb] < a.total_tokens;
    const T* qrow = reinterpret_cast<const T*>(a.q) + (int64_t)(t0 + (qok ? qi[qb] : 0)) * a.ldq + (int64_t)h * a.qk_head;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int e = ks * 32 + g * 8;
      load_frag_g(qf[qb][ks], qrow + e, qok && e < a.n + a.r);
    }
  }

  floatx4 o[DB][QB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY; l[qb] = 0.f;
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const T* kvb = reinterpret_cast<const T*>(a.kv) + (int64_t)b * a.max_kv_len * a.ldkv + (int64_t)h * (a.n + a.dv);
  const T* cache = reinterpret_cast<const T*>(a.cache);
  const int E = a.c + a.r;
  constexpr int KVPR = DQK / VEC;   // vectors per K row
  constexpr int VVPR = DV / VEC;    // vectors per V row

  for (int k0 = kbeg; k0 < kend; k0 += BKEY) {
    // ---- stage K (rows = keys) and V^T (rows = value dims) in LDS
    for (int v = tid; v < BKEY * KVPR; v += 256) {
      const int jj = v / KVPR, col = (v % KVPR) * VEC;
      const int key = k0 + jj;
      V16 val = {};
      if (key < kend) {
        if (col < a.n) {
          val = *reinterpret_cast<const V16*>(kvb + (int64_t)key * a.ldkv + col);
        } else if (col < a.n + a.r) {
          const int blk = a.block_table[(int64_t)b * a.max_blocks + key / a.page];
          if (blk >= 0 && blk < a.num_blocks)
            val = *reinterpret_cast<const V16*>(cache + ((int64_t)blk * a.page + key % a.page) * E + a.c + (col - a.n));
        }
      }
      *reinterpret_cast<V16*>(&Ks[jj * KROW + col]) = val;
    }
    for (int v = tid; v < BKEY * VVPR; v += 256) {
      const int jj = v / VVPR, d0 = (v % VVPR) * VEC;
      const int key = k0 + jj;
      V16 val = {};
      if (key < kend && d0 < a.dv) val = *reinterpret_cast<const V16*>(kvb + (int64_t)key * a.ldkv + a.n + d0);
#pragma unroll
      for (int e = 0; e < VEC; ++e) Vt[(d0 + e) * VROW + jj] = val[e];
    }
    __syncthreads();

    // ---- S^T = K Q^T : s[kb][qb][i] is key k0 + 16 kb + 4 g + i, query lr of block qb
    floatx4 s[4][QB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag<T> kf;
        lds_frag(kf, &Ks[(kb * 16 + lr) * KROW + ks * 32 + g * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma16(kf, qf[qb][ks], s[kb][qb]);
      }
    }

    // ---- online softmax (log2 domain), per query
    Frag<T> pf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + kb * 16 + g * 4 + i;
          const bool vis = key >= lo[qb] && key < hi[qb];
          const float x = vis ? s[kb][qb][i] * sl2 : -INFINITY;
          s[kb][qb][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = red4_max(mx);
      const float mnew = fmaxf(m[qb], mx);
      float alpha = 1.f, sum = 0.f;
      if (mnew != -INFINITY) {
        alpha = fast_exp2(m[qb] - mnew);  // m = -inf -> 0
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(s[kb][qb][i] - mnew);  // masked -> 0
            s[kb][qb][i] = p;
            sum += p;
          }
        m[qb] = mnew;
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      sum = red4_sum(sum);
      l[qb] = l[qb] * alpha + sum;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d][qb] *= alpha;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[qb][k2].v[e] = from_f32<T>(s[2 * k2][qb][e]);
          pf[qb][k2].v[4 + e] = from_f32<T>(s[2 * k2 + 1][qb][e]);
        }
    }

    // ---- O^T += V^T P^T  (keys of step k2 for lane group g: 32k2 + 4g + {0..3}, 32k2 + 16 + 4g + {0..3})
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        Frag<T> vf;
        const T* row = &Vt[(d * 16 + lr) * VROW + k2 * 32 + g * 4];
        lds4(vf, 0, row);
        lds4(vf, 4, row + 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[d][qb] = mfma16(vf, pf[qb][k2], o[d][qb]);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds O[query lr][d .. d+3], d = 16 db + 4 g
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qi[qb] >= ql) continue;
    const int t = t0 + qi[qb];
    if (t >= a.total_tokens) continue;
    const float inv = l[qb] > 0.f ? 1.f / l[qb] : 0.f;
    if (a.lse && g == 0) a.lse[(int64_t)t * a.H + h] = l[qb] > 0.f ? m[qb] + __log2f(l[qb]) : -INFINITY;
    T* orow = reinterpret_cast<T*>(a.out) + (int64_t)t * a.ldo + (int64_t)h * a.dv;
    const T* grow = a.gate ? reinterpret_cast<const T*>(a.gate) + (int64_t)t * a.ldg + (int64_t)h * a.dv : nullptr;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const int d0 = d * 16 + g * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (d0 + i >= a.dv) break;
        float v = o[d][qb][i] * inv;
        if (grow) v *= sigmoidf(to_f32(grow[d0 + i]));
        orow[d0 + i] = from_f32<T>(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for the DeepSeek head shape (n = 128, r = 64, dv = 128). One
// workgroup = 8 wavefronts (two per SIMD) x 32 queries of one head, on the
// 32x32x16 MFMA. 64-key tiles stream from HBM straight into LDS
// (global_load_lds_dwordx4) through a 3-tile ring: k_nope and v rows of the
// expanded buffer through the scalar-base form, the shared rope key from the
// paged cache. Rows are unpadded with XOR-swizzled 16-byte chunks: by the
// row's low bits for the key tiles (row & 15 for the 16-chunk k_nope rows,
// row & 7 for the 8-chunk rope rows: the rows of a 16-byte score operand read
// hit distinct banks) and by 4 (row & 3) for the value tile (the 4 rows x 64
// bytes that 32 lanes of transposing reads take in one pass hit distinct
// banks). Tiles inside every query's visible interval skip the masking.
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 tr_pair(const bf16* p0, const bf16* p1) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

namespace big {
constexpr int KT = 64;                  // keys per tile
constexpr int NW = 8;                   // wavefronts per workgroup (two per SIMD)
constexpr int BQ = NW * 32;             // queries per workgroup
constexpr int NOPE_CH = 16, PE_CH = 8, V_CH = 16;   // 16-byte chunks per key row
constexpr int NBUF = 3;                 // tile ring: t (values), t + 1 (scores), t + 2 (in flight)
__device__ __forceinline__ int kslot(int row, int c, int ch) { return row * ch + (c ^ (row & (ch - 1))); }
__device__ __forceinline__ int vslot(int row, int c) { return row * V_CH + (c ^ ((row & 3) << 2)); }
}  // namespace big

// S^T = K Q^T per 32-key block: element e of lane l is key
// 32 kb + 8 (e / 4) + 4 (l / 32) + e % 4 of query l % 32 (lanes l and l ^ 32
// hold the same query), so a row reduction is one in-lane pass plus one
// permlane32_swap, and the accumulator's 8 consecutive elements of a 16-key
// step are exactly the B operand of O^T = V^T P^T in the same key order. The
// V^T operand comes from two transposing reads per fragment (keys
// 16 s + 4 (l / 32) + 0..3 and + 8). Software pipeline: step t computes the
// scores of tile t + 1, the softmax of tile t, then P V of tile t, as fenced
// blocks; the wavefront runs at priority 3 over its MFMA blocks and 0 over
// the softmax, so that the two wavefronts of a SIMD drift half a phase apart
// and one's softmax VALU runs beside the other's MFMAs. K and V fragments are
// read two ahead of their MFMAs.
//
// LOG2Q: the queries were multiplied by scale * log2(e), so the products are
// the scaled scores in log2 units; each tile's score accumulators then start
// at minus the row's reference max and the probabilities are exp2 of the
// products as they come out of the MFMAs (a rare reference move shifts the
// current and the next tile's scores)

template <bool LOG2Q>
__global__ __launch_bounds__(512, 1) void prefill_attn_bf16_kernel(PrefillAttnArgs a) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) bf16x8 knope[NBUF][KT * NOPE_CH];
  __shared__ __attribute__((aligned(16))) bf16x8 kpe[NBUF][KT * PE_CH];
  __shared__ __attribute__((aligned(16))) bf16x8 vt[NBUF][KT * V_CH];
  __shared__ int iv[4];  // union lo, union hi, intersection lo, intersection hi

  // workgroup id -> (query tile, head, sequence). Workgroups go to the 8 XCDs
  // round-robin by id: XCD x takes the (sequence, head) pairs p = x mod 8, so
  // every query tile of a pair reads its keys through one L2, and within the
  // XCD the heaviest (latest, for causal masks) query tiles come first
  const int np = a.H * a.batch, npx = (np + 7) / 8;
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int nqt = (a.max_q_len + BQ - 1) / BQ;
  const int pr = (slot % npx) * 8 + xcd;
  const int qt = nqt - 1 - slot / npx;
  if (pr >= np || qt < 0) return;
  const int h = pr % a.H, b = pr / a.H;
  int ql = a.cu_seqlens[b + 1] - a.cu_seqlens[b];
  ql = min(max(ql, 0), a.max_q_len);
  if (qt * BQ >= ql) return;
  const int pl = min(max(a.prefix_lens[b], 0), a.max_kv_len - ql);
  const int L = pl + ql;
  const int t0 = a.cu_seqlens[b];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;  // query of the lane, half of the key group
  const int lr = lane & 15, g = lane >> 4;
  const float sl2 = LOG2Q ? 1.f : a.scale * kLog2e;

  if (tid == 0) { iv[0] = 0x7fffffff; iv[1] = 0; iv[2] = 0; iv[3] = 0x7fffffff; }
  __syncthreads();
  const int qi = qt * BQ + wave * 32 + lq;
  int lo = 0, hi = 0;
  if (qi < ql && t0 + qi < a.total_tokens) visible(a.mask, t0 + qi, pl + qi, L, lo, hi);
  if (hf == 0 && lo < hi) {
    atomicMin(&iv[0], lo);
    atomicMax(&iv[1], hi);
    atomicMax(&iv[2], lo);
    atomicMin(&iv[3], hi);
  }
  if (hf == 0 && qi < ql && lo >= hi) atomicMax(&iv[2], 0x7fffffff);  // an empty row: no tile is unmasked for it
  __syncthreads();
  const int kbeg = (iv[0] / KT) * KT, kend = iv[1];
  const int in_lo = iv[2], in_hi = iv[3];  // tiles inside [in_lo, in_hi) need no mask
  // the union of this wavefront's visible intervals (tiles outside it are skipped)
  int wlo = lo < hi ? lo : 0x7fffffff, whi = lo < hi ? hi : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    wlo = min(wlo, __shfl_xor(wlo, o));
    whi = max(whi, __shfl_xor(whi, o));
  }
  wlo = __builtin_amdgcn_readfirstlane(wlo);
  whi = __builtin_amdgcn_readfirstlane(whi);
  auto live = [&](int k0) { return k0 < whi && k0 + KT > wlo; };

  // queries in registers (B operand of step ks: dims 16 ks + 8 hf .. + 7 of query lq)
  bf16x8 qf[12];
  {
    const bool qok = qi < ql && t0 + qi < a.total_tokens;
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + (int64_t)(t0 + (qok ? qi : 0)) * a.ldq + (int64_t)h * a.qk_head;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hf * 8);
      qf[ks] = qok ? v : bf16x8{};
    }
  }

  // DMA geometry. k_nope / v: 16 chunks per key row, 2 instructions per wave
  // each; byte offsets relative to the tile's first key row of this head in
  // the expanded buffer. k_pe: 8 chunks per row, 1 instruction per wave, byte
  // offsets relative to the tile's first entry in its cache page (tiles never
  // cross a page: they start at multiples of 64 keys and the page size is a
  // multiple of 64)
  const bf16* kvb = reinterpret_cast<const bf16*>(a.kv) + (int64_t)b * a.max_kv_len * a.ldkv + (int64_t)h * (a.n + a.dv);
  const int64_t row_bytes = a.ldkv * 2;
  uint32_t noff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sl = (j * NW + wave) * 64 + lane;
    const int row = sl / NOPE_CH, cs = sl % NOPE_CH;
    noff[j] = (uint32_t)(row * row_bytes) + (uint32_t)((cs ^ (row & (NOPE_CH - 1))) * 16);
    const int cv = cs ^ ((row & 3) << 2);
    voff[j] = (uint32_t)(row * row_bytes) + 256u + (uint32_t)(cv * 16);
  }
  const bf16* cache = reinterpret_cast<const bf16*>(a.cache);
  const int E = a.c + a.r;
  const int32_t* __restrict__ btab = a.block_table + (int64_t)b * a.max_blocks;
  const uint32_t knope_lds = lds_addr(&knope[0][0]), vt_lds = lds_addr(&vt[0][0]), kpe_lds = lds_addr(&kpe[0][0]);
  uint32_t poff;
  {
    const int sl = wave * 64 + lane;
    const int row = sl / PE_CH, cs = sl % PE_CH;
    poff = (uint32_t)(row * E * 2) + (uint32_t)(a.c * 2) + (uint32_t)((cs ^ (row & 7)) * 16);
  }
  int pbase = kbeg / a.page;
  int btreg = (pbase + lane < a.max_blocks) ? btab[pbase + lane] : -1;

  auto issue = [&](int k0, int buf) {
    // rows past the last key re-read the last key (their scores are masked)
    const int last = min(kend, L) - 1;
    const int rows_valid = last - k0 + 1;
    const bf16* base = kvb + (int64_t)k0 * a.ldkv;
    const int pg = k0 / a.page;
    if (pg - pbase >= 64) {
      pbase = pg;
      btreg = (pbase + lane < a.max_blocks) ? btab[pbase + lane] : -1;
    }
    int blk = __builtin_amdgcn_readlane(btreg, pg - pbase);
    if (blk < 0 || blk >= a.num_blocks) blk = 0;  // unmapped page: any valid memory (output is garbage-in)
    const bf16* pbase_ptr = cache + ((int64_t)blk * a.page + (k0 - pg * a.page)) * E;
    const uint32_t nb = knope_lds + (uint32_t)(buf * KT * NOPE_CH * 16);
    const uint32_t vb = vt_lds + (uint32_t)(buf * KT * V_CH * 16);
    const uint32_t pb = kpe_lds + (uint32_t)(buf * KT * PE_CH * 16);
    if (rows_valid >= KT) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dma16_sbase(noff[j], base, nb + (uint32_t)(j * NW + wave) * 1024u);
        dma16_sbase(voff[j], base, vb + (uint32_t)(j * NW + wave) * 1024u);
      }
      dma16_sbase(poff, pbase_ptr, pb + (uint32_t)wave * 1024u);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sl = (j * NW + wave) * 64 + lane;
        const int row = sl / NOPE_CH;
        const uint32_t back = row >= rows_valid ? (uint32_t)((row - rows_valid + 1) * row_bytes) : 0u;
        dma16_sbase(noff[j] - back, base, nb + (uint32_t)(j * NW + wave) * 1024u);
        dma16_sbase(voff[j] - back, base, vb + (uint32_t)(j * NW + wave) * 1024u);
      }
      {
        const int row = (wave * 64 + lane) / PE_CH;
        const uint32_t back = row >= rows_valid ? (uint32_t)((row - rows_valid + 1) * E * 2) : 0u;
        dma16_sbase(poff - back, pbase_ptr, pb + (uint32_t)wave * 1024u);
      }
    }
  };

  // O^T block db: element e of lane l is dim 32 db + 8 (e / 4) + 4 hf + e % 4 of query lq
  floatx16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m = -INFINITY, l = 0.f, alpha = 1.f;
  const bool active = qt * BQ + wave * 32 < ql;

  // ---- S^T = K Q^T of the tile in buffer bf: sc[kb] = keys 32 kb .. + 31
  auto scores = [&](int bf, floatx16 (&sc)[2]) {
    const bf16x8* KN = knope[bf];
    const bf16x8* KP = kpe[bf];
    // LOG2Q: start at minus the reference max (0 while the row has none)
    const float z = LOG2Q && m != -INFINITY ? -m : 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[kb][e] = z;
    // fragment j = 2 ks + kb: key 32 kb + lq, dims 16 ks + 8 hf .. + 7; read
    // two fragments ahead of its MFMA behind fences
    auto kfr = [&](int j) -> bf16x8 {
      const int ks = j >> 1, kb = j & 1, row = kb * 32 + lq;
      return ks < 8 ? KN[kslot(row, ks * 2 + hf, NOPE_CH)] : KP[kslot(row, (ks - 8) * 2 + hf, PE_CH)];
    };
    bf16x8 fr[3];
    fr[0] = kfr(0);
    fr[1] = kfr(1);
#pragma unroll
    for (int j = 0; j < 24; ++j) {
      if (j + 2 < 24) fr[(j + 2) % 3] = kfr(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      sc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j % 3], qf[j >> 1], sc[j & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mask = [&](floatx16 (&sc)[2], int k0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (key < lo || key >= hi) sc[kb][e] = -INFINITY;
      }
  };
  // online softmax (log2 domain) with lazy rescaling; probabilities replace the scores
  auto softmax = [&](floatx16 (&sc)[2], floatx16 (&nx)[2]) -> bool {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[kb][e]);
    mx = red2_max(mx);
    if constexpr (LOG2Q) {
      // sc = score - ref (ref = m, 0 while m = -inf); a reference move d
      // shifts this tile and the next one (computed against the old ref)
      const bool none = m == -INFINITY;
      const float mnew = none ? mx : (mx > 8.f ? m + mx : m);
      const float d = mnew == -INFINITY ? 0.f : mnew - (none ? 0.f : m);
      alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
      const bool rescale = mnew != m;
      m = mnew;
      if (__any(d != 0.f)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sc[kb] -= d;
          nx[kb] -= d;
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(sc[kb][e]);  // masked -> 0
          sc[kb][e] = p;
          sum += p;
        }
      l = l * alpha + red2_sum(sum);
      return rescale;
    } else {
      mx *= sl2;  // the scale is positive: the max of the scaled scores
      const float mnew = (mx > m + 8.f) ? mx : m;
      alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
      const bool rescale = mnew != m;
      const float nm = (mnew == -INFINITY) ? 0.f : -mnew;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(sc[kb][e], sl2, nm));
          sc[kb][e] = p;
          sum += p;
        }
      l = l * alpha + red2_sum(sum);
      m = mnew;
      return rescale;
    }
  };
  // ---- O^T += V^T P^T: k step s = keys 16 s .. + 15 of the tile; the B
  // operand is accumulator elements 8 (s & 1) .. + 7 of block s / 2 (keys
  // 16 s + 4 hf + (0..3), 16 s + 8 + 4 hf + (0..3)); the A operand of dim
  // block db is read in the same key order: group G = lane / 16 of 16 lanes
  // covers dims 32 db + 16 (G & 1) .., lane 4 a + b' points at key row
  // 16 s + 4 hf + a (+ 8), dims + 4 b' .. + 3
  auto pv = [&](int bf, const floatx16 (&sc)[2]) {
    const bf16x8* VT = vt[bf];
    bf16x8 pf[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[st][e] = (bf16)sc[st >> 1][8 * (st & 1) + e];
    const int ra = lr >> 2, rb = lr & 3;
    // fragment j = 4 s + db, read two ahead of its MFMA behind fences
    auto vfr = [&](int j) -> bf16x8 {
      const int st = j >> 2, db = j & 3;
      const int el = db * 32 + (g & 1) * 16 + rb * 4;
      const int c = el >> 3, half = (el >> 2) & 1;
      const int r0 = st * 16 + hf * 4 + ra;
      return tr_pair(reinterpret_cast<const bf16*>(&VT[vslot(r0, c)]) + half * 4,
                     reinterpret_cast<const bf16*>(&VT[vslot(r0 + 8, c)]) + half * 4);
    };
    bf16x8 vr[3];
    vr[0] = vfr(0);
    vr[1] = vfr(1);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j + 2 < 16) vr[(j + 2) % 3] = vfr(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      o[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[j % 3], pf[j >> 2], o[j & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- software pipeline over the key tiles; tile t + 2 streams in meanwhile.
  // Two score arrays alternate (the loop is unrolled by two).
  const int ntl = kbeg < kend ? (kend - kbeg + KT - 1) / KT : 0;
  MLA_WAIT_VMCNT(0);  // query fragments landed: in the loop only tile copies are outstanding
  if (ntl > 0) issue(kbeg, 0);
  if (ntl > 1) issue(kbeg + KT, 1);
  if (ntl > 1) MLA_WAIT_VMCNT(5);  // the copies of tile 1 may stay in flight
  else MLA_WAIT_VMCNT(0);
  lds_barrier();
  floatx16 s0[2], s1[2];
  if (active && ntl > 0 && live(kbeg)) scores(0, s0);
  auto step = [&](int t, floatx16 (&cur)[2], floatx16 (&nxt)[2]) {
    const int k0 = kbeg + t * KT;
    MLA_WAIT_VMCNT(0);  // tile t + 1 landed (the only copies in flight)
    lds_barrier();      // ... for every wavefront; P V of tile t - 1 is done everywhere
    if (t + 2 < ntl) issue(k0 + 2 * KT, (t + 2) % NBUF);
    if (!active) return;  // no query of this wavefront exists: it only helps stream tiles
    const bool cur_live = live(k0), nxt_live = live(k0 + KT);
    if (cur_live && !(k0 >= in_lo && k0 + KT <= in_hi)) mask(cur, k0);
    // priority 3 over the MFMA blocks, 0 over the softmax (the fences keep each block whole)
    __builtin_amdgcn_s_setprio(3);
    if (nxt_live) scores((t + 1) % NBUF, nxt);  // after the last tile: a stale buffer, unused
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if (!cur_live) return;
    const bool rescale = softmax(cur, nxt);
    __builtin_amdgcn_sched_barrier(0);
    if (__any(rescale)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    __builtin_amdgcn_s_setprio(3);
    pv(t % NBUF, cur);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  int t = 0;
  for (; t + 1 < ntl; t += 2) {
    step(t, s0, s1);
    step(t + 1, s1, s0);
  }
  if (t < ntl) step(t, s0, s1);

  // ---- epilogue: lane holds O[query lq][32 db + 8 i + 4 hf + (0..3)]
  if (qi >= ql) return;
  const int tt = t0 + qi;
  if (tt >= a.total_tokens) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.lse && hf == 0) a.lse[(int64_t)tt * a.H + h] = l > 0.f ? m + __log2f(l) : -INFINITY;
  bf16* orow = reinterpret_cast<bf16*>(a.out) + (int64_t)tt * a.ldo + (int64_t)h * a.dv;
  const bf16* grow = a.gate ? reinterpret_cast<const bf16*>(a.gate) + (int64_t)tt * a.ldg + (int64_t)h * a.dv : nullptr;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + i * 8 + hf * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = o[db][4 * i + j] * inv;
      if (grow) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= sigmoidf((float)grow[d0 + j]);
      }
      *reinterpret_cast<bf16x4*>(orow + d0) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    }
}

template <typename T, int DQK, int DV>
hipError_t launch_dims(const PrefillAttnArgs& a, hipStream_t s) {
  // one 16-query block per wave for short query runs (draft blocks), two otherwise
  const int QB = a.max_q_len <= 64 ? 1 : 2;
  const int BQ = 64 * QB;
  dim3 grid((a.max_q_len + BQ - 1) / BQ, a.H, a.batch);
  if (QB == 1) hipLaunchKernelGGL((prefill_attn_kernel<T, DQK, DV, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((prefill_attn_kernel<T, DQK, DV, 2>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const PrefillAttnArgs& a, hipStream_t s) {
  const int dqk = a.n + a.r, dv = a.dv;
  if (dqk <= 32 && dv <= 16) return launch_dims<T, 32, 16>(a, s);
  if (dqk <= 64 && dv <= 32) return launch_dims<T, 64, 32>(a, s);
  if (dqk <= 192 && dv <= 128) return launch_dims<T, 192, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

const char* prefill_attn_check(const PrefillAttnArgs& a, bool is_bf16) {
  const int vec = is_bf16 ? 8 : 4;
  if (a.n + a.r > 192 || a.dv > 128) return "prefill attention: head dims above 192 (q/k) or 128 (v) are not supported";
  if (a.n % vec || a.r % vec || a.dv % vec || a.c % vec) return "prefill attention: n, r, dv and c must be 16-byte multiples";
  if ((a.n + a.r) % 8) return "prefill attention: n + r must be a multiple of 8";
  if (a.ldq % vec || a.qk_head % vec || a.ldkv % vec) return "prefill attention: row strides must be 16-byte multiples";
  return nullptr;
}

hipError_t prefill_attn_launch(const PrefillAttnArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0 || a.max_q_len <= 0) return hipSuccess;
  if (is_bf16 && a.n == 128 && a.r == 64 && a.dv == 128 && a.c % 8 == 0 && a.page % big::KT == 0) {
    const int64_t nqt = (a.max_q_len + big::BQ - 1) / big::BQ, npx = ((int64_t)a.H * a.batch + 7) / 8;
    if (8 * npx * nqt > 0x7fffffff) return hipErrorInvalidValue;
    if (a.q_log2) hipLaunchKernelGGL(prefill_attn_bf16_kernel<true>, dim3((unsigned)(8 * npx * nqt)), dim3(64 * big::NW), 0, s, a);
    else hipLaunchKernelGGL(prefill_attn_bf16_kernel<false>, dim3((unsigned)(8 * npx * nqt)), dim3(64 * big::NW), 0, s, a);
    return hipGetLastError();
  }
  if (a.q_log2) return hipErrorInvalidValue;  // only the kernel above takes log2-scaled queries
  return is_bf16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace mla
