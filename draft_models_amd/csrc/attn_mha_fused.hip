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
// Work item = (sequence, 256-entry chunk, head); 4 wavefronts, wavefront w
// owns entries 64 w .. 64 w + 63 of the chunk and all 256 expansion columns
// of the head (128 k_nope, 128 v). The k axis (512 latent dims) moves in
// 64-wide steps: the head's kv_b_proj rows and the chunk's latent rows (read
// from the paged cache through the block table) are copied HBM -> LDS with
// global_load_lds_dwordx4, double-buffered, 16-byte chunks of a row XOR-ed
// with (row & 7). The k_nope part is computed as K^T (kv_b rows as the MFMA A
// operand) and the v part as V (latent rows as A), which leaves every lane
// holding, for one entry, 4 consecutive k_nope dims per block, and for one v
// dim, 4 consecutive entries per block. Pairs of blocks are then exactly the
// operands of the score product S = K q^T (contraction over dims, in a fixed
// permuted order that the q operand follows) and of the value product
// O^T = V^T P^T (contraction over entries, in the order the score output
// already has), so no LDS transposes are needed. The 4 wavefronts' partial
// softmax states are merged through LDS.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kC = 512, kE = 576, kNope = 128, kDv = 128, kQk = 192;
constexpr int KC = 256;                 // cache entries per chunk
constexpr int BK = 64;                  // k step
constexpr int ROWCH = BK / 8;           // 16-byte chunks per 128-byte tile row
constexpr int SLOTS = 256 * ROWCH;      // 16-byte slots per operand tile
constexpr int DMA_PER_WAVE = SLOTS / 256;
constexpr int OPAD = kDv + 4;           // LDS row of one query's partial output (floats)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row, int c) { return row * ROWCH + (c ^ (row & 7)); }

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

__global__ __launch_bounds__(256, 1) void mha_fused_kernel(MhaFusedArgs a) {
  // operand rings (kv_b rows, then latent rows); after the k loop the same
  // memory holds the wavefronts' partial outputs
  __shared__ __attribute__((aligned(16))) bf16x8 lds[4 * SLOTS];
  bf16x8 (*tw)[SLOTS] = reinterpret_cast<bf16x8(*)[SLOTS]>(&lds[0]);
  bf16x8 (*ta)[SLOTS] = reinterpret_cast<bf16x8(*)[SLOTS]>(&lds[2 * SLOTS]);
  float* om = reinterpret_cast<float*>(&lds[0]);  // [4 waves][16 queries][OPAD]
  float* mm = om + 4 * 16 * OPAD;                  // [4][16] running max (log2 units)
  float* ll = mm + 64;                             // [4][16] probability sums

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

  uint32_t woff[DMA_PER_WAVE], aoff[DMA_PER_WAVE];
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int s = (j * 4 + wave) * 64 + lane;
    const int row = s / ROWCH, cs = s % ROWCH;
    const uint32_t colb = (uint32_t)(cs ^ (row & 7)) * 16u;
    woff[j] = (uint32_t)(((int64_t)h * 256 + row) * kC * 2) + colb;
    aoff[j] = (uint32_t)(entry_off(k0 + row) * 2) + colb;
  }
  // the shared rope key of every entry this lane scores: entry 16 bb + lr of
  // the wavefront's 64, rope dims 32 jr + 8 g4 .. + 7 (score A operand)
  bf16x8 kpe[4][2];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const bf16* er = cache + entry_off(k0 + wave * 64 + bb * 16 + lr) + kC + 8 * g4;
#pragma unroll
    for (int jr = 0; jr < 2; ++jr) kpe[bb][jr] = *reinterpret_cast<const bf16x8*>(er + 32 * jr);
  }

  const uint32_t tw_lds = lds_addr(&tw[0][0]), ta_lds = lds_addr(&ta[0][0]);
  auto issue = [&](int kt, int buf) {
    const bf16* wb = W + kt * BK;
    const bf16* ab = cache + kt * BK;
    const uint32_t bo = (uint32_t)buf * SLOTS * 16u;
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; ++j) dma16_sbase(woff[j], wb, tw_lds + bo + (uint32_t)(j * 4 + wave) * 1024u);
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; ++j) dma16_sbase(aoff[j], ab, ta_lds + bo + (uint32_t)(j * 4 + wave) * 1024u);
  };

  // accK[a][bb][i] = K^T[dim 16 a + 4 g4 + i][entry 16 bb + lr]
  // accV[a][bb][i] = V[entry 16 bb + 4 g4 + i][v dim 16 a + lr]
  floatx4 accK[8][4], accV[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      accK[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};
      accV[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  auto compute = [&](const bf16x8* TW, const bf16x8* TA) {
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      Frag<bf16> wf[16], af[4];
#pragma unroll
      for (int x = 0; x < 16; ++x) wf[x].v = TW[swz(x * 16 + lr, ks * 4 + g4)];
#pragma unroll
      for (int y = 0; y < 4; ++y) af[y].v = TA[swz(wave * 64 + y * 16 + lr, ks * 4 + g4)];
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) accK[x][y] = mfma16(wf[x], af[y], accK[x][y]);
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) accV[x][y] = mfma16(af[y], wf[8 + x], accV[x][y]);
    }
  };

  constexpr int nk = kC / BK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, buf ^ 1);
      MLA_WAIT_VMCNT(2 * DMA_PER_WAVE);
    } else {
      MLA_WAIT_VMCNT(0);
    }
    lds_barrier();
    compute(tw[buf], ta[buf]);
    lds_barrier();
  }

  // expanded keys and values in bf16 (the rounding a stored expansion has):
  // kop[bb][j] = K[entry 16 bb + lr][dims 32 j + 4 g4 + (0..3), 32 j + 16 + 4 g4 + (0..3)]
  // vop[x][j]  = V^T[v dim 16 x + lr][entries 32 j + 4 g4 + (0..3), 32 j + 16 + 4 g4 + (0..3)]
  bf16x8 kop[4][4], vop[8][2];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int j = 0; j < 4; ++j) kop[bb][j] = pack8(accK[2 * j][bb], accK[2 * j + 1][bb]);
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int j = 0; j < 2; ++j) vop[x][j] = pack8(accV[x][2 * j], accV[x][2 * j + 1]);

  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q);
  const float sl2 = a.scale * kLog2e;
  const int key_w = k0 + wave * 64;  // first entry of this wavefront
  const int qblocks = (sg.ql + 15) >> 4;
  for (int qb = 0; qb < qblocks; ++qb) {
    // query lr of the block: q operands in the dims order of kop
    const int qi = qb * 16 + lr;
    const int t = sg.q0 + qi;
    const bool qok = qi < sg.ql && t < a.total_tokens;
    int lo = 0, hi = 0;
    if (qok) visible_rows(a.mask, t, sg.pl + qi, sg.L, lo, hi);
    bf16x8 qn[4], qp[2];
    if (qok) {
      const bf16* qr = Q + (int64_t)t * a.ldq + (int64_t)h * kQk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 x = *reinterpret_cast<const bf16x4*>(qr + 32 * j + 4 * g4);
        const bf16x4 y = *reinterpret_cast<const bf16x4*>(qr + 32 * j + 16 + 4 * g4);
        qn[j] = bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
      }
#pragma unroll
      for (int jr = 0; jr < 2; ++jr) qp[jr] = *reinterpret_cast<const bf16x8*>(qr + kNope + 32 * jr + 8 * g4);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qn[j] = bf16x8{};
      qp[0] = qp[1] = bf16x8{};
    }

    // scores s[bb][i] = S[entry 16 bb + 4 g4 + i][query lr]
    floatx4 s[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      floatx4 z = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[bb][j], qn[j], z, 0, 0, 0);
#pragma unroll
      for (int jr = 0; jr < 2; ++jr) z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kpe[bb][jr], qp[jr], z, 0, 0, 0);
      s[bb] = z;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key_w + bb * 16 + 4 * g4 + i;
        const float x = (key >= lo && key < hi) ? s[bb][i] * sl2 : -INFINITY;
        s[bb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = red4_max(mx);
    const float mref = mx == -INFINITY ? 0.f : mx;
    float lsum = 0.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(s[bb][i] - mref);  // masked -> 0
        s[bb][i] = p;
        lsum += p;
      }
    lsum = red4_sum(lsum);
    const bf16x8 pop0 = pack8(s[0], s[1]), pop1 = pack8(s[2], s[3]);
    // o[x][i] = O^T[v dim 16 x + 4 g4 + i][query lr] over this wavefront's entries
    floatx4 o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      floatx4 z = floatx4{0.f, 0.f, 0.f, 0.f};
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[x][0], pop0, z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[x][1], pop1, z, 0, 0, 0);
      o[x] = z;
    }

    // merge the 4 wavefronts' states: max, sum and unnormalised output per query
    float* orow = om + (wave * 16 + lr) * OPAD;
#pragma unroll
    for (int x = 0; x < 8; ++x) *reinterpret_cast<floatx4*>(orow + 16 * x + 4 * g4) = o[x];
    if (g4 == 0) {
      mm[wave * 16 + lr] = mx;
      ll[wave * 16 + lr] = lsum;
    }
    __syncthreads();
    {
      const int q = tid >> 4, d8 = (tid & 15) * 8;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mm[w * 16 + q]);
      float den = 0.f;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float mw = mm[w * 16 + q];
          if (mw == -INFINITY) continue;
          const float e = fast_exp2(mw - M);
          den += e * ll[w * 16 + q];
          const float* src = om + (w * 16 + q) * OPAD + d8;
          const floatx4 v0 = *reinterpret_cast<const floatx4*>(src);
          const floatx4 v1 = *reinterpret_cast<const floatx4*>(src + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i] += e * v0[i];
            acc[4 + i] += e * v1[i];
          }
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const int64_t pi = (((int64_t)b * a.nchunks + ch) * a.qblocks + qb) * a.H + h;
      bf16x8 ov;
#pragma unroll
      for (int i = 0; i < 8; ++i) ov[i] = (bf16)(acc[i] * inv);
      *reinterpret_cast<bf16x8*>(a.part_o + (pi * 16 + q) * kDv + d8) = ov;
      if (d8 == 0) a.part_lse[pi * 16 + q] = den > 0.f ? M + __log2f(den) : -INFINITY;
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
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_lse[(base + c * cstride) * 16 + q]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < nc; ++c) {
      const int64_t pi = base + c * cstride;
      const float l = a.part_lse[pi * 16 + q];
      if (l == -INFINITY) continue;
      const float e = fast_exp2(l - M);
      den += e;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(a.part_o + (pi * 16 + q) * kDv + d8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += e * (float)v[i];
    }
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
  hipLaunchKernelGGL(mha_fused_kernel, dim3((unsigned)(a.batch * a.nchunks * a.H)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t mha_fused_merge_launch(const MhaFusedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mha_fused_merge_kernel, dim3((unsigned)a.H, (unsigned)a.qblocks, (unsigned)a.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace mla
