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
// value product.
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

// ---------------------------------------------------------------------------
// bf16 kernel. One workgroup = 4 wavefronts = 64 heads of one (sequence,
// chunk). Each 32-key tile of the cache is streamed from HBM straight into LDS
// (global_load_lds_dwordx4, double-buffered: tile t+1 is in flight while t is
// used), and every element of the tile is read from LDS by one wavefront
// only, because the work is split by DIMENSION rather than by head:
//   * scores: wavefront w computes partial S^T = C q_lat^T for all 64 heads
//     over its quarter of the 576 entry dims; the four partials are summed
//     through LDS, each wavefront then owns the softmax of 16 heads;
//   * values: wavefront w owns 128 of the 512 latent value dims of O^T for all
//     64 heads; the probabilities (and rescale factors) of all heads are
//     shared through LDS.
// The tile stays row-major (key rows of 16-byte chunks) with the chunk index
// XOR-swizzled by (row & 7) inside groups of 8 chunks, which makes the
// 16-byte score operand reads (8 rows, one chunk) and the transposing value
// operand reads (ds_read_b64_tr_b16: 4 rows x 32 bytes per 16 lanes)
// bank-conflict free. The 64-head groups of one (sequence, chunk) are
// placed on the same XCD so that the second reads the tiles from L2.
// ---------------------------------------------------------------------------

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Two transposing LDS reads (4 keys each) concatenated into one 8-element
// MFMA operand: elements 0-3 from p0, 4-7 from p1.
__device__ __forceinline__ bf16x8 tr_pair(const bf16* p0, const bf16* p1) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

template <int ECH>
__device__ __forceinline__ int dslot(int row, int c) {
  return row * ECH + (c & ~7) + ((c & 7) ^ (row & 7));
}

// vmcnt(n) with expcnt / lgkmcnt left unconstrained (gfx9 s_waitcnt encoding)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)
// LDS-only workgroup barrier: this wavefront's LDS traffic is complete, then
// s_barrier (global prefetches stay in flight)
#define LDS_BARRIER() do { WAIT_LGKM0(); __builtin_amdgcn_s_barrier(); } while (0)

// ECH: 16-byte chunks per cache entry (padded to a multiple of 8; chunks past
// the entry are read from a zero page). CB: 16-wide blocks of the latent c.
template <int ECH, int CB, int NBUF>
__global__ __launch_bounds__(256, 1) void decode_attn_bf16_kernel(DecodeAttnArgs a, int groups) {
  constexpr int KT = 32;                    // keys per tile
  constexpr int SLOTS = KT * ECH;           // 16-byte chunks per tile
  constexpr int PER_WAVE = SLOTS / 256;     // DMA instructions per wave per tile
  constexpr int KS = ECH / 4;               // 32-dim steps of the score product
  constexpr int KSW = (KS + 3) / 4;         // most score steps of one wavefront
  constexpr int CBW = (CB + 3) / 4;         // most value blocks of one wavefront
  constexpr int HB = 4;                     // 16-head blocks per workgroup
  static_assert(SLOTS % 256 == 0, "tile slots");
  static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
  __shared__ __attribute__((aligned(16))) bf16x8 tile[NBUF][SLOTS];
  __shared__ __attribute__((aligned(16))) floatx4 spart[4][2 * HB][64];  // partial scores
  __shared__ __attribute__((aligned(16))) bf16x8 pshare[HB][64];         // probabilities
  __shared__ float ashare[HB * 16];                                      // rescale factors
  __shared__ float lshare[HB * 16];                                      // softmax sums

  // workgroup id -> (item = sequence x chunk, head group): ids 8k + x of the
  // same k / groups and x share an item and an XCD (x = id % 8)
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int hg = slot % groups;
  const int item = (slot / groups) * 8 + xcd;
  if (item >= a.batch * a.splits) return;
  const int b = item / a.splits, split = item % a.splits;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, g = lane >> 4;
  const int hbase = hg * 64;

  int L, lo, hi;
  decode_interval(a, b, L, lo, hi);
  const int k_begin = lo + split * a.chunk;
  const int k_end = min(hi, k_begin + a.chunk);
  const int64_t pidx = ((int64_t)b * a.splits + split) * a.H;
  if (k_begin >= k_end) {
    if (tid < 64 && hbase + tid < a.H) a.part_lse[pidx + hbase + tid] = -INFINITY;
    return;
  }

  // this wavefront's share of the dims: score steps [ks0, ks1), value blocks [cb0, cb1)
  const int ks0 = wave * KS / 4, ks1 = (wave + 1) * KS / 4;
  const int cb0 = wave * CB / 4, cb1 = (wave + 1) * CB / 4;

  // latent queries of all 64 heads over this wavefront's dims (B operand:
  // column = head, 8 consecutive dims per lane)
  Frag<bf16> qf[HB][KSW];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hbase + hb * 16 + lr;
    const bool hok = h < a.H;
    const bf16* ql = reinterpret_cast<const bf16*>(a.ql) + (int64_t)b * a.ldql + (int64_t)(hok ? h : 0) * a.c;
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + (int64_t)b * a.ldq + (int64_t)(hok ? h : 0) * a.qk_head + a.n;
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      // branch-free: every fragment is one 16-byte load (padding reads the zero page)
      const int e = (ks0 + i) * 32 + g * 8;
      const bool ok = hok && ks0 + i < ks1 && e < a.c + a.r;
      const bf16* src = !ok ? a.zeros : (e < a.c ? ql + e : qp + (e - a.c));
      qf[hb][i].v = *reinterpret_cast<const bf16x8*>(src);
    }
  }

  const bf16* cache = reinterpret_cast<const bf16*>(a.cache);
  const int E = a.c + a.r;
  const int ech_real = E / 8;
  const int32_t* __restrict__ bt = a.block_table + (int64_t)b * a.max_blocks;

  // tile-independent geometry of this lane's DMA slots: slot s of the tile
  // holds chunk (row, c) of the swizzled layout; c8 < 0 marks padding chunks
  int drow[PER_WAVE], dc8[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int sl = (j * 4 + wave) * 64 + lane;
    const int row = sl / ECH, cs = sl % ECH;
    const int c = (cs & ~7) | ((cs & 7) ^ (row & 7));
    drow[j] = row;
    dc8[j] = c < ech_real ? c * 8 : -1;
  }

  // Block-table entries of the chunk live in a register, one page per lane
  // (refreshed every 64 pages), so forming a tile's addresses never waits
  // on a memory load. The page position advances incrementally (page >= 32).
  const int npages_total = a.max_blocks;
  int pbase = k_begin / a.page;  // first page held in `btreg`
  int btreg = (pbase + lane < npages_total) ? bt[pbase + lane] : -1;
  int p0 = pbase, off0 = k_begin - pbase * a.page;  // page / offset of the next tile to issue

  // stream the next tile (start k0 = page p0, offset off0) into buffer `buf`:
  // rows [0, b0) lie in page p0 at offsets off0 + row, rows [b0, 32) in page
  // p0 + 1 (a tile spans at most two pages). Rows past the visible range and
  // padding chunks read the zero page.
  auto issue = [&](int k0, int buf) {
    if (p0 + 1 - pbase >= 64) {  // the tile reaches past the cached entries
      pbase = p0;
      btreg = (pbase + lane < npages_total) ? bt[pbase + lane] : -1;
    }
    const int b0 = a.page - off0;
    const int rows = min(k_end - k0, KT);
    const int blk0 = __builtin_amdgcn_readlane(btreg, p0 - pbase);
    const int blk1 = __builtin_amdgcn_readlane(btreg, p0 + 1 - pbase);
    const bool ok0 = blk0 >= 0 && blk0 < a.num_blocks;
    const bool ok1 = rows > b0 && blk1 >= 0 && blk1 < a.num_blocks;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int row = drow[j];
      const bool first = row < b0;
      const int pos = first ? off0 + row : row - b0;
      const int blk = first ? blk0 : blk1;
      const bool ok = (first ? ok0 : ok1) && row < rows && dc8[j] >= 0;
      const bf16* src = ok ? cache + ((int64_t)(blk * a.page + pos) * E + dc8[j]) : a.zeros;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)(&tile[buf][(j * 4 + wave) * 64]),
                                       16, 0, 0);
    }
    off0 += KT;
    if (off0 >= a.page) { off0 -= a.page; ++p0; }
  };

  floatx4 o[CBW][HB];  // O^T blocks: dims 16 (cb0 + i) + 4 g + {0..3}, head lr of block hb
#pragma unroll
  for (int i = 0; i < CBW; ++i)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) o[i][hb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // softmax state of head wave * 16 + lr (owned)
  const float sl2 = a.scale * kLog2e;
  const int ra = (lr >> 2), rb = (lr & 3);

  WAIT_VMCNT(0);  // query fragments are in registers: in the loop only tile prefetches are outstanding
  // NBUF-deep ring: tiles t+1 .. t+NBUF-1 are in flight while tile t is used
  const int ntiles = (k_end - k_begin + KT - 1) / KT;
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t)
    if (t < ntiles) issue(k_begin + t * KT, t);
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = k_begin + t * KT;
    const int buf = t % NBUF;
    if (t + NBUF - 1 < ntiles) issue(k0 + (NBUF - 1) * KT, (t + NBUF - 1) % NBUF);
    // wait until this tile's loads landed: later tiles may stay in flight
    const int later = min(NBUF - 1, ntiles - 1 - t);
    if (later >= 2) WAIT_VMCNT(2 * PER_WAVE);
    else if (later == 1) WAIT_VMCNT(PER_WAVE);
    else WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    const bf16x8* T = tile[buf];

    // ---- partial scores over this wavefront's dims, all 64 heads
    floatx4 sp[2][HB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sp[kb][hb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KSW; ++i) {
      if (ks0 + i < ks1) {
        Frag<bf16> cf0, cf1;
        cf0.v = T[dslot<ECH>(lr, (ks0 + i) * 4 + g)];
        cf1.v = T[dslot<ECH>(16 + lr, (ks0 + i) * 4 + g)];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          sp[0][hb] = mfma16(cf0, qf[hb][i], sp[0][hb]);
          sp[1][hb] = mfma16(cf1, qf[hb][i], sp[1][hb]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) spart[wave][kb * HB + hb][lane] = sp[kb][hb];
    LDS_BARRIER();

    // ---- full scores of the owned 16 heads; online softmax (log2 domain)
    floatx4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = spart[0][kb * HB + wave][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) s[kb] += spart[w][kb * HB + wave][lane];
    }
    const bool partial = k0 + KT > k_end;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[kb][i] * sl2;
        if (partial && k0 + kb * 16 + g * 4 + i >= k_end) x = -INFINITY;
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // lazy rescaling: the reference max moves only when the tile's max exceeds
    // it by more than 2^8 (probabilities stay <= 256, exact after the final
    // division by l); rescaling the accumulators is then rare
    const float mnew = (mx > m + 8.f) ? mx : m;
    const float alpha = fast_exp2(m - mnew);
    float sum = 0.f;
    Frag<bf16> pf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(s[kb][i] - mnew);
        sum += p;
        pf.v[kb * 4 + i] = (bf16)p;
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    l = l * alpha + sum;
    m = mnew;
    pshare[wave][lane] = pf.v;
    if (g == 0) ashare[wave * 16 + lr] = alpha;
    LDS_BARRIER();

    // ---- O^T (this wavefront's value dims, all heads) += C^T P^T
    Frag<bf16> pa[HB];
    float al[HB];
    bool rescale = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      pa[hb].v = pshare[hb][lane];
      al[hb] = ashare[hb * 16 + lr];
      rescale |= al[hb] != 1.f;
    }
    if (__any(rescale)) {
#pragma unroll
      for (int i = 0; i < CBW; ++i)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[i][hb] *= al[hb];
    }
    // the transposed operand comes from the row-major tile: lane k = 4a + b'
    // of a 16-lane group points at key row (4g + a) [+16], dims 16 d + 4 b' ..
    // +3, and receives keys 4g + {0..3} [+16] of dim 16 d + lr
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      if (cb0 + i < cb1) {
        const int el = (cb0 + i) * 16 + rb * 4;
        const int c = el >> 3, half = (el >> 2) & 1;
        Frag<bf16> vf;
        vf.v = tr_pair(reinterpret_cast<const bf16*>(&T[dslot<ECH>(g * 4 + ra, c)]) + half * 4,
                       reinterpret_cast<const bf16*>(&T[dslot<ECH>(16 + g * 4 + ra, c)]) + half * 4);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[i][hb] = mfma16(vf, pa[hb], o[i][hb]);
      }
    }
    LDS_BARRIER();
  }

  // ---- partial outputs normalised by their own softmax sums, and log-sum-exp
  if (g == 0) lshare[wave * 16 + lr] = l;
  LDS_BARRIER();
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = hbase + hb * 16 + lr;
    if (h >= a.H) continue;
    const float inv = 1.f / lshare[hb * 16 + lr];
    float* po = a.part_o + (pidx + h) * a.c;
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
      const int d0 = (cb0 + i) * 16 + g * 4;
      if (cb0 + i < cb1) *reinterpret_cast<floatx4*>(po + d0) = o[i][hb] * inv;
    }
  }
  if (g == 0 && hbase + wave * 16 + lr < a.H) a.part_lse[pidx + hbase + wave * 16 + lr] = m + log2f(l);
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

template <int ECH, int CB>
hipError_t launch_bf16(const DecodeAttnArgs& a, hipStream_t s) {
  const int groups = (a.H + 63) / 64;
  const int items = a.batch * a.splits;
  dim3 grid(((items + 7) / 8) * 8 * groups);
  hipLaunchKernelGGL((decode_attn_bf16_kernel<ECH, CB, 3>), grid, dim3(256), 0, s, a, groups);
  return hipGetLastError();
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

// bf16 with one of the instantiated latent shapes takes the LDS-streaming
// kernel; fp32 (and other shapes) the generic one
static bool bf16_fast_shape(const DecodeAttnArgs& a, int* ech, int* cb) {
  const int E = a.c + a.r;
  if (a.c % 16 || a.page < 32) return false;
  if (E <= 64 && a.c <= 32) { *ech = 8; *cb = 2; return true; }
  if (E <= 576 && a.c == 512) { *ech = 72; *cb = 32; return true; }
  return false;
}

hipError_t decode_attn_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  int ech, cb;
  if (is_bf16 && bf16_fast_shape(a, &ech, &cb)) {
    if (ech == 8) return launch_bf16<8, 2>(a, s);
    return launch_bf16<72, 32>(a, s);
  }
  return is_bf16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

int decode_heads_per_group(const DecodeAttnArgs& a, bool is_bf16) {
  int ech, cb;
  (void)is_bf16; (void)ech; (void)cb;
  return 64;
}

hipError_t decode_merge_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  if (is_bf16) hipLaunchKernelGGL(decode_combine_kernel<bf16>, dim3(a.H, a.batch), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(decode_combine_kernel<float>, dim3(a.H, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
