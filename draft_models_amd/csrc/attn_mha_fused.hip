// Expanded-form MLA attention with the kv_b expansion fused in, for sequences
// with few new tokens (MLA blog, forward_mha listing: per head,
// K = [kv_c_normed W_UK^T | k_pe] and V = kv_c_normed W_UV^T, both taken
// from kv_b_proj). Draft blocks verify 16 tokens against a long latent
// prefix: expanding every prefix entry into per-head keys and values costs
// 256 output values per head and entry, and writing them to HBM only to read
// them back for 16 queries is the whole cost of the unfused form. Here the
// expanded keys and values of a 256-entry chunk of one head never leave the
// registers: the workgroup computes them with the MFMA (the same bf16
// rounding as a stored expansion), then attends to them from every query of
// the sequence and writes a normalised partial output with its log-sum-exp;
// mha_fused_merge_kernel combines the chunks of a sequence (the merge of
// partial attention states the listing uses for prefix and suffix).
//
// Work item = (sequence, 256-entry chunk, head); 8 wavefronts, two per SIMD.
// Wavefront w owns entries 64 (w & 3) .. + 63 of the chunk; w < 4 computes
// their 128 k_nope columns, w >= 4 their 128 v columns. The k axis (512
// latent dims) moves in 32-wide steps through a 4-buffer LDS ring, two steps
// per barrier: while steps kt and kt + 1 are multiplied, the head's kv_b_proj
// rows and the chunk's latent rows (read from the paged cache through the
// block table) for steps kt + 2 and kt + 3 are copied HBM -> LDS with
// global_load_lds_dwordx4, each wavefront's copies spread between the MFMAs
// of the first step so that the other wavefront of the SIMD keeps the matrix
// core busy while one waits for the copy path. The 16-byte chunks of a 64-byte tile row are XOR-ed with
// (row >> 1) & 3, so every 8 consecutive rows of a fragment read (the lanes
// the LDS serves together, 128 bytes) hit distinct banks.
//
// The k_nope part is computed as K^T (kv_b rows as the MFMA A operand) and
// the v part as V (latent rows as A): every lane then holds, for one entry,
// 4 consecutive k_nope dims per block, and for one v dim, 4 consecutive
// entries per block. Pairs of blocks are exactly the operands of the score
// product S = K q^T (contraction over dims, in a fixed permuted order that
// the q operand follows) and of the value product O^T = V^T P^T (contraction
// over entries, in the order the score output already has): the k_nope
// wavefront of an entry block hands its probabilities to the v wavefront of
// the same block through LDS in register order, and no transpose is needed.
// The 4 entry blocks' softmax states are merged through LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kC = 512, kE = 576, kNope = 128, kDv = 128, kQk = 192;
constexpr int KC = 256;                  // cache entries per chunk
constexpr int BK = 32;                   // k step
constexpr int ROWCH = BK / 8;            // 16-byte chunks per 64-byte tile row
constexpr int SLOTS = 256 * ROWCH;       // 16-byte slots per operand tile (16 KB)
constexpr int NBUF = 4;                  // ring buffers (two steps multiplied, two copied)
constexpr int NWAVE = 8;
constexpr int DPW = SLOTS / (NWAVE * 64);  // copies per wavefront per operand per step
constexpr int NK = kC / BK;               // expansion steps
constexpr int NKR = NK + 2;               // + the rope keys (latent columns 512..575, no kv_b rows)
constexpr int OPAD = kDv + 4;            // LDS row of one query's partial output (floats)
constexpr int QCH = kQk / 8;             // 16-byte chunks of one query row (24)
constexpr int QSLOTS = (kMhaFusedMaxQ / 16) * 16 * QCH;  // LDS copy of the item's queries
constexpr float kLog2e = 1.4426950408889634f;
static_assert(DPW == 2 && NK % 2 == 0 && (kE - kC) == 2 * BK, "copy schedule assumes these sizes");

__device__ __forceinline__ int swz(int row, int c) { return row * ROWCH + (c ^ ((row >> 1) & 3)); }

__device__ __forceinline__ void visible_rows(const MaskArgs& m, int t, int p, int L, int& lo, int& hi) {
  if (m.row_lo != nullptr && m.row_hi != nullptr) {
    lo = min(max(m.row_lo[t], 0), L);
    hi = min(max(m.row_hi[t], 0), L);
    return;
  }
  if (m.kind == 0) { lo = 0; hi = L; }
  else if (m.kind == 1) { lo = 0; hi = min(p + 1, L); }
  else { lo = max(0, p - m.window + 1); hi = min(p + 1, L); }
}

__device__ __forceinline__ bf16x8 pack8(const floatx4& x, const floatx4& y) {
  return bf16x8{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3], (bf16)y[0], (bf16)y[1], (bf16)y[2], (bf16)y[3]};
}

// sequence geometry shared by the two kernels
struct SeqGeom {
  int q0, ql, pl, L;
};
__device__ __forceinline__ SeqGeom seq_geom(const MhaFusedArgs& a, int b) {
  SeqGeom g;
  g.q0 = a.cu_seqlens[b];
  int ql = a.cu_seqlens[b + 1] - g.q0;
  g.ql = min(max(ql, 0), a.max_q_len);
  g.pl = min(max(a.prefix_lens[b], 0), a.max_kv_len - g.ql);
  g.L = g.pl + g.ql;
  return g;
}

__global__ __launch_bounds__(NWAVE * 64, 1) void mha_fused_kernel(MhaFusedArgs a) {
  // operand ring: buffer i = kv_b rows, then latent rows (16 KB each); after
  // the k loop buffers 0 and 1 hold the rope keys, buffers 2 and 3 the
  // epilogue's exchange areas
  __shared__ __attribute__((aligned(16))) bf16x8 lds[NBUF * 2 * SLOTS + QSLOTS];
  // the sequence's roped queries of this head, row r = query r, chunk c at
  // position c ^ (r & 7) (copied before the k loop, read by the epilogue)
  const bf16x8* qlds = &lds[NBUF * 2 * SLOTS];
  bf16x8* pex = &lds[4 * SLOTS];                               // [4 blocks][2][64 lanes] probabilities
  float* om = reinterpret_cast<float*>(&lds[4 * SLOTS + 4 * 64 * 2]);  // [4 blocks][16 queries][OPAD]
  float* mm = om + 4 * 16 * OPAD;                              // [4][16] max (log2 units)
  float* ll = mm + 64;                                         // [4][16] probability sums

  // work item: the heads of a sequence-chunk pair are spread over the XCD's
  // band of H / 8 heads; consecutive items of an XCD share the chunk's latent
  const int id = blockIdx.x;
  const int xcd = id & 7, u = id >> 3;
  const int hx = a.H >> 3;
  const int h = xcd * hx + u % hx;
  const int bc = u / hx;
  const int b = bc / a.nchunks, ch = bc % a.nchunks;
  const SeqGeom sg = seq_geom(a, b);
  const int k0 = ch * KC;
  if (sg.ql <= 0 || k0 >= sg.L) return;  // whole workgroup: no barrier reached yet

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int eb = wave & 3;          // entry block: entries 64 eb .. 64 eb + 63
  const bool vpart = wave >= 4;     // v columns (else k_nope columns)
  const int lr = lane & 15, g4 = lane >> 4;
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(a.wkvb);
  const bf16* __restrict__ cache = reinterpret_cast<const bf16*>(a.cache);
  const int32_t* __restrict__ bt = a.block_table + (int64_t)b * a.max_blocks;

  // element offset of cache entry `key` of this sequence; entries past the
  // end re-read the last one (their scores are masked), unmapped pages read
  // entry 0 (bad block tables stay inside the cache)
  auto entry_off = [&](int key) -> int64_t {
    key = min(key, sg.L - 1);
    const int blk = bt[key / a.page];
    return (blk >= 0 && blk < a.num_blocks) ? ((int64_t)blk * a.page + key % a.page) * kE : 0;
  };

  // copy geometry: slot (j * 8 + wave) * 64 + lane of an operand tile holds
  // row s / 4, chunk s % 4 (swizzled) of the step's 32-wide k slice
  uint32_t woff[DPW], aoff[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int s = (j * NWAVE + wave) * 64 + lane;
    const int row = s / ROWCH, cs = s % ROWCH;
    const uint32_t colb = (uint32_t)(cs ^ ((row >> 1) & 3)) * 16u;
    woff[j] = (uint32_t)(((int64_t)h * 256 + row) * kC * 2) + colb;
    aoff[j] = (uint32_t)(entry_off(k0 + row) * 2) + colb;
  }
  const uint32_t lds0 = lds_addr(&lds[0]);
  // copy g (0, 1: kv_b rows; 2, 3: latent rows) of step kt into its buffer;
  // steps NK and NK + 1 copy only the latent rows' rope keys
  auto copy = [&](int kt, int g) {
    const uint32_t dst = lds0 + (uint32_t)((kt % NBUF) * 2 * SLOTS + (g >> 1) * SLOTS) * 16u +
                         (uint32_t)(((g & 1) * NWAVE + wave) * 1024);
    if (g < 2) dma16_sbase(woff[g & 1], W + kt * BK, dst);
    else dma16_sbase(aoff[g & 1], cache + kt * BK, dst);
  };

  // k_nope wavefront: acc[x][y][i] = K^T[dim 16 x + 4 g4 + i][entry 16 y + lr]
  // v wavefront:      acc[x][y][i] = V[entry 16 y + 4 g4 + i][v dim 16 x + lr]
  floatx4 acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};

  // one k step: fragments from buffer kt % NBUF; with `copies`, the copies of
  // steps kt + 2 and kt + 3 spread over its 32 MFMAs (one per 4)
  auto step = [&](int kt, auto vtag, bool copies) {
    constexpr bool V = decltype(vtag)::value;
    const bf16x8* TW = &lds[(kt % NBUF) * 2 * SLOTS];
    const bf16x8* TA = TW + SLOTS;
    Frag<bf16> af[4], wf[8];
#pragma unroll
    for (int y = 0; y < 4; ++y) af[y].v = TA[swz(eb * 64 + y * 16 + lr, g4)];
#pragma unroll
    for (int x = 0; x < 8; ++x) wf[x].v = TW[swz((V ? 128 : 0) + x * 16 + lr, g4)];
    // rope steps: the 2 latent copies only
    const int n0 = copies ? (kt + 2 < NK ? 4 : (kt + 2 < NKR ? 2 : 0)) : 0;
    const int n1 = copies ? (kt + 3 < NK ? 4 : (kt + 3 < NKR ? 2 : 0)) : 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      __builtin_amdgcn_sched_barrier(0);
      if (x < 4) {
        if (x < n0) copy(kt + 2, n0 == 4 ? x : x + 2);
      } else {
        if (x - 4 < n1) copy(kt + 3, n1 == 4 ? x - 4 : x - 2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = V ? mfma16(af[y], wf[x], acc[x][y]) : mfma16(wf[x], af[y], acc[x][y]);
    }
  };

  // the queries (1 KB per copy, 6 per 16-query block) go first: the first
  // wait of the k loop covers them
  {
    const int nq = ((sg.ql + 15) >> 4) * 16 * QCH / 64;
    const bf16* Qh = reinterpret_cast<const bf16*>(a.q) + (int64_t)sg.q0 * a.ldq + (int64_t)h * kQk;
    for (int i = wave; i < nq; i += NWAVE) {
      const int c = i * 64 + lane;
      const int r = c / QCH, p = c % QCH;
      const int rr = min(r, sg.ql - 1);  // rows past the sequence re-read its last query (masked)
      const uint32_t off = (uint32_t)(((int64_t)rr * a.ldq + (p ^ (r & 7)) * 8) * 2);
      dma16_sbase(off, Qh, lds0 + (uint32_t)(NBUF * 2 * SLOTS + i * 64) * 16u);
    }
  }
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int g = 0; g < 4; ++g) copy(kt, g);
  auto kloop = [&](auto vtag) {
    for (int kt = 0; kt < NK; kt += 2) {
      // this wavefront's copies of steps kt, kt + 1 (issued during step
      // kt - 2) are done; no newer ones exist yet
      MLA_WAIT_VMCNT(0);
      lds_barrier();  // every wavefront's copies of kt, kt + 1 landed; kt - 2, kt - 1 read by all
      step(kt, vtag, true);
      step(kt + 1, vtag, false);
    }
  };
  if (vpart) kloop(std::true_type{});
  else kloop(std::false_type{});
  MLA_WAIT_VMCNT(0);
  lds_barrier();  // rope keys landed; the last buffers read by all before reuse

  // the shared rope key of every entry a k_nope lane scores: entry 16 y + lr
  // of the block, rope dims 32 jr + 8 g4 .. + 7 (score A operand), from the
  // rope steps' latent tiles
  bf16x8 kpe[4][2];
  if (!vpart) {
#pragma unroll
    for (int jr = 0; jr < 2; ++jr) {
      const bf16x8* TA = &lds[((NK + jr) % NBUF) * 2 * SLOTS + SLOTS];
#pragma unroll
      for (int y = 0; y < 4; ++y) kpe[y][jr] = TA[swz(eb * 64 + y * 16 + lr, g4)];
    }
  }

  const float sl2 = a.q_log2 ? 1.f : a.scale * kLog2e;  // q_log2: the products are the scaled scores
  const int key_b = k0 + eb * 64;  // first entry of this block
  const int qblocks = (sg.ql + 15) >> 4;
  // expanded keys (k_nope wavefronts) or values (v wavefronts) in bf16, the
  // rounding a stored expansion has:
  //   op[y][j] = K[entry 16 y + lr][dims 32 j + 4 g4 + (0..3), 32 j + 16 + 4 g4 + (0..3)]   (y, j < 4)
  //   op[x][j] = V^T[v dim 16 x + lr][entries 32 j + 4 g4 + (0..3), 32 j + 16 + 4 g4 + (0..3)]  (x < 8, j < 2)
  bf16x8 op[8][2];
  bf16x8 kop[4][4];
  if (vpart) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int j = 0; j < 2; ++j) op[x][j] = pack8(acc[x][2 * j], acc[x][2 * j + 1]);
  } else {
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int j = 0; j < 4; ++j) kop[y][j] = pack8(acc[2 * j][y], acc[2 * j + 1][y]);
  }

  for (int qb = 0; qb < qblocks; ++qb) {
    if (!vpart) {
      // query lr of the block: q operands in the dims order of kop
      const int qi = qb * 16 + lr;
      const int t = sg.q0 + qi;
      const bool qok = qi < sg.ql && t < a.total_tokens;
      int lo = 0, hi = 0;
      if (qok) visible_rows(a.mask, t, sg.pl + qi, sg.L, lo, hi);
      bf16x8 qn[4], qp[2];
      {
        const int r = qb * 16 + lr;
        auto qc = [&](int c) { return reinterpret_cast<const char*>(qlds + r * QCH + (c ^ (r & 7))); };
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x4 x = *reinterpret_cast<const bf16x4*>(qc(4 * j + (g4 >> 1)) + (g4 & 1) * 8);
          const bf16x4 y = *reinterpret_cast<const bf16x4*>(qc(4 * j + 2 + (g4 >> 1)) + (g4 & 1) * 8);
          qn[j] = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        }
#pragma unroll
        for (int jr = 0; jr < 2; ++jr) qp[jr] = *reinterpret_cast<const bf16x8*>(qc(16 + 4 * jr + g4));
      }
      // scores s[y][i] = S[entry 16 y + 4 g4 + i][query lr]
      floatx4 s[4];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        floatx4 z = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[y][j], qn[j], z, 0, 0, 0);
#pragma unroll
        for (int jr = 0; jr < 2; ++jr) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kpe[y][jr], qp[jr], z, 0, 0, 0);
        s[y] = z;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key_b + y * 16 + 4 * g4 + i;
          const float x = (key >= lo && key < hi) ? s[y][i] * sl2 : -INFINITY;
          s[y][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = red4_max(mx);
      const float mref = mx == -INFINITY ? 0.f : mx;
      float lsum = 0.f;
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(s[y][i] - mref);  // masked -> 0
          s[y][i] = p;
          lsum += p;
        }
      lsum = red4_sum(lsum);
      // the v wavefront's B operands, in register order
      pex[eb * 128 + lane] = pack8(s[0], s[1]);
      pex[eb * 128 + 64 + lane] = pack8(s[2], s[3]);
      if (g4 == 0) {
        mm[eb * 16 + lr] = mx;
        ll[eb * 16 + lr] = lsum;
      }
    }
    __syncthreads();
    if (vpart) {
      // o[x][i] = O^T[v dim 16 x + 4 g4 + i][query lr] over the block's entries
      const bf16x8 p0 = pex[eb * 128 + lane], p1 = pex[eb * 128 + 64 + lane];
      float* orow = om + (eb * 16 + lr) * OPAD;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        floatx4 z = floatx4{0.f, 0.f, 0.f, 0.f};
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[x][0], p0, z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[x][1], p1, z, 0, 0, 0);
        *reinterpret_cast<floatx4*>(orow + 16 * x + 4 * g4) = z;
      }
    }
    __syncthreads();
    {
      // merge the 4 entry blocks: query tid / 32, v dims 4 (tid % 32) .. + 3
      const int q = tid >> 5, d4 = (tid & 31) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * 16 + q]);
      float den = 0.f;
      floatx4 o4 = floatx4{0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mw = mm[w * 16 + q];
          if (mw == -INFINITY) continue;
          const float e = fast_exp2(mw - M);
          den += e * ll[w * 16 + q];
          const floatx4 v = *reinterpret_cast<const floatx4*>(om + (w * 16 + q) * OPAD + d4);
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] += e * v[i];
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int64_t pi = (((int64_t)b * a.nchunks + ch) * a.qblocks + qb) * a.H + h;
      *reinterpret_cast<bf16x4*>(a.part_o + (pi * 16 + q) * kDv + d4) =
          bf16x4{(bf16)(o4[0] * inv), (bf16)(o4[1] * inv), (bf16)(o4[2] * inv), (bf16)(o4[3] * inv)};
      if (d4 == 0) a.part_lse[pi * 16 + q] = den > 0.f ? M + __log2f(den) : -INFINITY;
    }
    __syncthreads();
  }
}

// One workgroup per (head, query block, sequence): 16 queries x 128 v dims,
// 8 dims per thread; chunks combined by their log-sum-exp, then the optional
// output gate, then the attention output row [T, H * 128].
__global__ __launch_bounds__(256) void mha_fused_merge_kernel(MhaFusedArgs a) {
  const int h = blockIdx.x, qb = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(a, b);
  const int q = threadIdx.x >> 4, d8 = (threadIdx.x & 15) * 8;
  const int qi = qb * 16 + q;
  const int t = sg.q0 + qi;
  if (qi >= sg.ql || t >= a.total_tokens) return;
  const int nc = (sg.L + KC - 1) / KC;
  const int64_t base = (((int64_t)b * a.nchunks) * a.qblocks + qb) * a.H + h;  // chunk 0
  const int64_t cstride = (int64_t)a.qblocks * a.H;
  // groups of 8 chunks: their loads issued together, a running max across groups
  constexpr int G = 8;
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += G) {
    float l[G];
    bf16x8 v[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int c = c0 + k;
      const int64_t pi = base + (int64_t)min(c, nc - 1) * cstride;  // every chunk below nc was written
      l[k] = c < nc ? a.part_lse[pi * 16 + q] : -INFINITY;
      v[k] = *reinterpret_cast<const bf16x8*>(a.part_o + (pi * 16 + q) * kDv + d8);
    }
    float mg = M;
#pragma unroll
    for (int k = 0; k < G; ++k) mg = fmaxf(mg, l[k]);
    if (mg == -INFINITY) continue;
    const float r = fast_exp2(M - mg);  // 0 while M is still -inf
    den *= r;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= r;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (l[k] == -INFINITY) continue;
      const float e = fast_exp2(l[k] - mg);
      den += e;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += e * (float)v[k][i];
    }
    M = mg;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  bf16x8 ov;
  const bf16* g = a.gate ? reinterpret_cast<const bf16*>(a.gate) + (int64_t)t * a.ldg + (int64_t)h * kDv + d8 : nullptr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = acc[i] * inv;
    if (g) x *= sigmoidf((float)g[i]);
    ov[i] = (bf16)x;
  }
  *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.out) + (int64_t)t * a.ldo + (int64_t)h * kDv + d8) = ov;
}

}  // namespace

const char* mha_fused_check(const MhaFusedArgs& a) {
  if (a.H <= 0 || a.H % 8) return "fused expansion needs a head count that is a multiple of 8";
  if (a.qk_head != kQk) return "fused expansion needs q heads of 128 + 64";
  if (a.max_q_len <= 0 || a.max_q_len > kMhaFusedMaxQ) return "fused expansion takes at most 64 new tokens per sequence";
  if (a.max_kv_len < a.max_q_len || a.batch <= 0) return "bad sequence limits";
  if ((int64_t)a.max_blocks * a.page < a.max_kv_len) return "block table does not cover max_kv_len";
  if (a.nchunks != (a.max_kv_len + KC - 1) / KC || a.qblocks != (a.max_q_len + 15) / 16) return "bad chunk counts";
  // per-slot copy offsets are 32-bit byte offsets
  if ((int64_t)a.num_blocks * a.page * kE * 2 >= ((int64_t)1 << 32)) return "cache too large for 32-bit offsets";
  if ((int64_t)a.H * 256 * kC * 2 >= ((int64_t)1 << 32)) return "kv_b_proj too large for 32-bit offsets";
  // 8- and 16-byte vector accesses
  if (a.ldq % 8 || (reinterpret_cast<uintptr_t>(a.q) & 15) || (reinterpret_cast<uintptr_t>(a.cache) & 15) ||
      (reinterpret_cast<uintptr_t>(a.wkvb) & 15))
    return "q, cache and kv_b_proj must be 16-byte aligned with row strides of 8 elements";
  if (a.ldo % 8 || (reinterpret_cast<uintptr_t>(a.out) & 15)) return "output must be 16-byte aligned";
  if (a.gate && (a.ldg % 8 || (reinterpret_cast<uintptr_t>(a.gate) & 15))) return "gate must be 16-byte aligned";
  if (!a.part_o || !a.part_lse || (reinterpret_cast<uintptr_t>(a.part_o) & 15)) return "partial buffers missing";
  return nullptr;
}

size_t mha_fused_partial_bytes(int batch, int nchunks, int qblocks, int H) {
  const size_t n = (size_t)batch * nchunks * qblocks * H * 16;
  return ((n * kDv * 2 + 255) & ~(size_t)255) + n * sizeof(float);
}

hipError_t mha_fused_launch(const MhaFusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mha_fused_kernel, dim3((unsigned)(a.batch * a.nchunks * a.H)), dim3(NWAVE * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t mha_fused_merge_launch(const MhaFusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mha_fused_merge_kernel, dim3((unsigned)a.H, (unsigned)a.qblocks, (unsigned)a.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace mla
