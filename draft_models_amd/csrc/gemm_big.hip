// Large-tile bf16 MFMA GEMM for gfx950: C[M, N] = A[M, K] . W[N, K]^T.
//
// A 256 x 256 output tile per workgroup of 4 wavefronts (2 x 2, 128 x 128
// each, 64 accumulator blocks of 16 x 16 held in AGPRs). The k axis moves in
// 64-wide steps; both operand tiles (256 rows x 128 bytes) stream from HBM
// straight into LDS with global_load_lds_dwordx4 (no register staging),
// double-buffered so that step t+1 is in flight while step t feeds the
// MFMAs. LDS rows are unpadded; the 16-byte chunk index of a row is XOR-ed
// with (row & 7), so the fragment reads (8 consecutive rows, one chunk) hit
// distinct banks. Rows that do not exist (past M or N, or absent gathered
// rows) read a zero page. Tiles are ordered so that each XCD (workgroup id
// mod 8) walks a contiguous range of M-tiles with all of their N-tiles,
// keeping the activation rows in that XCD's L2.
#include "common.h"
#include "gemm.h"

namespace mla {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROWCH = BK / 8;                    // 16-byte chunks per tile row
constexpr int TILE_SLOTS = 256 * ROWCH;          // per operand
constexpr int DMA_PER_WAVE = TILE_SLOTS / 256;   // per operand per wave per k step


__device__ __forceinline__ int swz(int row, int c) { return row * ROWCH + (c ^ (row & 7)); }

__global__ __launch_bounds__(256, 1) void gemm_big_kernel(GemmArgs g, int mtiles, int ntiles) {
  __shared__ __attribute__((aligned(16))) bf16x8 tw[2][TILE_SLOTS];  // weight rows (n)
  __shared__ __attribute__((aligned(16))) bf16x8 ta[2][TILE_SLOTS];  // activation rows (m)
  __shared__ float rowscale[BM];

  // XCD-aware tile order: ids with the same (id % 8) share an XCD and take a
  // contiguous range of the M-major tile sequence
  const int total = mtiles * ntiles;
  const int id = blockIdx.x;
  const int per_xcd = (total + 7) / 8;
  const int t = (id & 7) * per_xcd + (id >> 3);
  if (t >= total) return;
  const int mt = t / ntiles, nt = t % ntiles;
  const int m0 = mt * BM, n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, g4 = lane >> 4;
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A);
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W);

  // per-lane DMA geometry (k-independent): slot s of a tile holds chunk
  // (row, c); its source is byte offset row_base + 16 c of the operand, the
  // base (advanced by k) sitting in scalar registers. Rows that do not exist
  // are clamped to an existing row: their products are never stored. Offsets
  // fit 32 bits (host check).
  uint32_t woff[DMA_PER_WAVE], aoff[DMA_PER_WAVE];
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int s = (j * 4 + wave) * 64 + lane;
    const int row = s / ROWCH, cs = s % ROWCH;
    const uint32_t colb = (uint32_t)(cs ^ (row & 7)) * 16u;
    const int n = min(n0 + row, g.N - 1);
    woff[j] = (uint32_t)((int64_t)n * g.ldw * 2) + colb;
    const int m = min(m0 + row, g.M - 1);
    int64_t off = 0;
    if (!g.gather) {
      off = (int64_t)m * g.lda;
    } else {
      const GatherA& ga = g.ga;
      const int b = m / ga.max_kv_len, jj = m % ga.max_kv_len;
      int ql = ga.cu_seqlens[b + 1] - ga.cu_seqlens[b];
      ql = min(max(ql, 0), ga.max_q_len);
      const int pl = min(max(ga.prefix_lens[b], 0), ga.max_kv_len - ql);
      if (jj < pl + ql) {
        const int blk = ga.block_table[(int64_t)b * ga.max_blocks + jj / ga.page];
        if (blk >= 0 && blk < ga.num_blocks) off = ((int64_t)blk * ga.page + jj % ga.page) * ga.entry;
      }
    }
    aoff[j] = (uint32_t)(off * 2) + colb;
  }

  const uint32_t tw_lds = lds_addr(&tw[0][0]), ta_lds = lds_addr(&ta[0][0]);
  auto issue = [&](int kt, int buf) {
    const bf16* wb = W + kt * BK;
    const bf16* ab = A + kt * BK;
    const uint32_t bo = (uint32_t)buf * TILE_SLOTS * 16u;
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; ++j) dma16_sbase(woff[j], wb, tw_lds + bo + (uint32_t)(j * 4 + wave) * 1024u);
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; ++j) dma16_sbase(aoff[j], ab, ta_lds + bo + (uint32_t)(j * 4 + wave) * 1024u);
  };

  floatx4 acc[8][8];  // [n block][m block]
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sq[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) sq[b] = 0.f;
  // the RMSNorm row statistic: only the wavefronts that publish it (wn == 0)
  const bool rownorm = g.epi == EPI_ROWNORM;
  const bool rowstat = rownorm && wn == 0;

  auto compute = [&](const bf16x8* TW, const bf16x8* TA) {
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      Frag<bf16> wf[8], af[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) wf[a].v = TW[swz(wn * 128 + a * 16 + lr, ks * 4 + g4)];
#pragma unroll
      for (int b = 0; b < 8; ++b) af[b].v = TA[swz(wm * 128 + b * 16 + lr, ks * 4 + g4)];
      if (rowstat) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)af[b].v[e];
            sq[b] += f * f;
          }
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = mfma16(wf[a], af[b], acc[a][b]);
    }
  };

  // double buffer: step t+1 streams in while step t is multiplied
  const int nk = g.K / BK;
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

  if (rownorm) {
    // lanes lr, lr+16, lr+32, lr+48 hold disjoint k chunks of the same rows;
    // waves wn = 0 and 1 both saw every row of their wm half: wave wn = 0 writes
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      float s = sq[b];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (wn == 0 && g4 == 0) rowscale[wm * 128 + b * 16 + lr] = rsqrtf(s / (float)g.K + g.eps);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n + 3], m = m0 + 128 wm + 16 b + lr, n = n0 + 128 wn + 16 a + 4 g4
  bf16* C = reinterpret_cast<bf16*>(g.C);
  const bf16* G = reinterpret_cast<const bf16*>(g.G);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int ml = wm * 128 + b * 16 + lr;
    const int m = m0 + ml;
    if (m >= g.M) continue;
    if (g.gather) {
      // absent gathered rows are not stored
      const GatherA& ga = g.ga;
      const int bb = m / ga.max_kv_len, jj = m % ga.max_kv_len;
      int ql = ga.cu_seqlens[bb + 1] - ga.cu_seqlens[bb];
      ql = min(max(ql, 0), ga.max_q_len);
      const int pl = min(max(ga.prefix_lens[bb], 0), ga.max_kv_len - ql);
      if (jj >= pl + ql) continue;
    }
    const float rs = rownorm ? rowscale[ml] : 1.f;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int n = n0 + wn * 128 + a * 16 + g4 * 4;
      if (n >= g.N) continue;
      floatx4 v = acc[a][b];
      if (rownorm) v = v * rs;
      if (g.epi == EPI_GATE) {
        const bf16* gp = G + (int64_t)m * g.ldg + n;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) v[e] *= sigmoidf((float)gp[e]);
      }
      bf16* dst = C + (int64_t)m * g.ldc + n;
      if (n + 3 < g.N) {
        *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      } else {
        for (int e = 0; e < 4 && n + e < g.N; ++e) dst[e] = (bf16)v[e];
      }
    }
  }
}

}  // namespace

bool gemm_big_eligible(const GemmArgs& g, bool is_bf16) {
  if (!is_bf16 || g.batch != 1 || g.K % BK != 0 || g.M < 512 || g.N < 256) return false;
  // per-slot source offsets are 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 31;  // elements (2 bytes each)
  if ((int64_t)g.N * g.ldw >= lim) return false;
  if (!g.gather && (int64_t)g.M * g.lda >= lim) return false;
  if (g.gather && (int64_t)g.ga.num_blocks * g.ga.page * g.ga.entry >= lim) return false;
  return (int64_t)((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) >= 256;
}

hipError_t gemm_big_launch(const GemmArgs& g, const void* zeros, hipStream_t s) {
  const int mtiles = (g.M + BM - 1) / BM, ntiles = (g.N + BN - 1) / BN;
  const int total = mtiles * ntiles;
  const int grid = ((total + 7) / 8) * 8;
  (void)zeros;
  hipLaunchKernelGGL(gemm_big_kernel, dim3(grid), dim3(256), 0, s, g, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace mla
