// Large-tile bf16 MFMA GEMM for gfx950: C[M, N] = A[M, K] . W[N, K]^T.
//
// A 256 x 256 output tile per workgroup of 8 wavefronts, two per SIMD:
// wavefront w computes rows 64 (w & 3) .. + 63 and columns 128 (w >> 2) ..
// + 127 (32 accumulator blocks of 16 x 16). The k axis moves in 32-wide steps,
// two per barrier interval, through two LDS buffers that each hold the 64 k
// of one interval as 128-byte rows: while steps kt and kt + 1 are multiplied,
// both operand tiles of steps kt + 2 and kt + 3 (256 rows x 128 bytes each)
// stream from HBM straight into LDS with global_load_lds_dwordx4, issued right
// after the barrier (the copy-issue stall of one wavefront is covered by the
// other wavefront of its SIMD, and the copies get the whole interval to land).
// One copy instruction moves 8 whole 128-byte rows: each source cache line is
// requested once, not once per 32-wide step. The 16-byte chunks of a row are
// XOR-ed with (row >> 1) & 7: the LDS serves a 16-byte read 16 lanes (16 rows
// of one fragment) at a time, and those rows then hit distinct banks (rows
// r and r + 8 shared banks with (row >> 1) & 3: half the LDS cycles were
// conflicts). Rows that do not exist
// (past M or N, or absent gathered rows) re-read an existing row and are not
// stored. Tiles are placed on XCDs in 2-D blocks (see TileMap) so that each
// XCD's L2 keeps its band of weight rows. Products with too few output tiles
// to fill the CUs (weight gradients: K = tokens) split K: split z
// (blockIdx.y) runs its k range and writes an fp32 partial tile, summed by a
// reduce kernel.
#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace mla {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int ROWCH = 2 * BK / 8;                // 16-byte chunks per 128-byte tile row (two k steps)
constexpr int SLOTS = 256 * ROWCH;               // 16-byte slots per operand tile (32 KB)
constexpr int NBUF = 2;                          // buffers (one interval multiplied, one copied)
constexpr int NWAVE = 8;
constexpr int DPW = SLOTS / (NWAVE * 64);        // copies per wavefront per operand per interval
static_assert(DPW == 4, "copy schedule assumes 4 copies per operand and wavefront");

__device__ __forceinline__ int swz(int row, int c) { return row * ROWCH + (c ^ ((row >> 1) & 7)); }

// Tile placement: the 8 XCDs (workgroup id mod 8) form an xm x xn grid; XCD
// (xi, xj) owns the block of M-tile band xi and N-tile band xj and walks it
// M-major (all N-tiles of its band for one M-tile, then the next M-tile), so
// the weight rows of its N band stay in that XCD's L2 while the activation
// rows stream through once per N band.
struct TileMap {
  int mtiles, ntiles, xm, xn;
};

__global__ __launch_bounds__(NWAVE * 64, 1) void gemm_big_kernel(GemmArgs g, TileMap tm, float* part, int kper) {
  // operand ring (buffer i: weight rows, then activation rows); after the k
  // loop the same 128 KB stage the output tile for coalesced stores
  __shared__ __attribute__((aligned(16))) bf16x8 lds[NBUF * 2 * SLOTS];
  __shared__ float rowscale[BM];
  __shared__ int rowok[BM];  // output row exists (inside M, gathered row present)

  const int id = blockIdx.x;
  const int xcd = id & 7, u = id >> 3;
  const int xi = xcd / tm.xn, xj = xcd % tm.xn;
  const int mb0 = xi * tm.mtiles / tm.xm, mb1 = (xi + 1) * tm.mtiles / tm.xm;
  const int nb0 = xj * tm.ntiles / tm.xn, nb1 = (xj + 1) * tm.ntiles / tm.xn;
  const int bw = nb1 - nb0;
  if (bw <= 0 || u >= (mb1 - mb0) * bw) return;
  const int mt = mb0 + u / bw, nt = nb0 + u % bw;
  const int m0 = mt * BM, n0 = nt * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
  const int wm = wave & 3, wn = wave >> 2;
  const int lr = lane & 15, g4 = lane >> 4;
  // split-K: steps [kt0, kt0 + NK) of this split (kper steps per split, even)
  const int kt0 = part ? (int)blockIdx.y * kper : 0;
  const bf16* __restrict__ A = reinterpret_cast<const bf16*>(g.A) + (int64_t)kt0 * BK;
  const bf16* __restrict__ W = reinterpret_cast<const bf16*>(g.W) + (int64_t)kt0 * BK;

  // per-lane copy geometry (k-independent): slot s = (j * 8 + wave) * 64 +
  // lane of a tile holds chunk (row s / 8, c), its source at byte offset
  // row_base + 16 (c ^ ((row >> 1) & 7)), the base (advanced by k) in scalar
  // registers. Offsets fit 32 bits (host check).
  uint32_t woff[DPW], aoff[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int s = (j * NWAVE + wave) * 64 + lane;
    const int row = s / ROWCH, cs = s % ROWCH;
    const uint32_t colb = (uint32_t)(cs ^ ((row >> 1) & 7)) * 16u;
    const int n = min(n0 + row, g.N - 1);
    woff[j] = (uint32_t)((int64_t)n * g.ldw * 2) + colb;
    const int m = min(m0 + row, g.M - 1);
    int64_t off = 0;
    if (!g.gather) {
      off = (int64_t)m * g.lda;
    } else {
      const GatherA& ga = g.ga;
      const int b = m / ga.max_kv_len, jj = m % ga.max_kv_len;
      // the block-table read does not wait for the lengths: its index is in
      // bounds for every row (max_blocks * page covers max_kv_len, host check)
      const int blk = ga.block_table[(int64_t)b * ga.max_blocks + jj / ga.page];
      int ql = ga.cu_seqlens[b + 1] - ga.cu_seqlens[b];
      ql = min(max(ql, 0), ga.max_q_len);
      const int pl = min(max(ga.prefix_lens[b], 0), ga.max_kv_len - ql);
      if (jj < pl + ql && blk >= 0 && blk < ga.num_blocks) off = ((int64_t)blk * ga.page + jj % ga.page) * ga.entry;
    }
    aoff[j] = (uint32_t)(off * 2) + colb;
  }

  if (tid < BM) {
    const int m = m0 + tid;  // one output row per thread
    bool ok = m < g.M;
    if (ok && g.gather) {
      const GatherA& ga = g.ga;
      const int bb = m / ga.max_kv_len, jj = m % ga.max_kv_len;
      int ql = ga.cu_seqlens[bb + 1] - ga.cu_seqlens[bb];
      ql = min(max(ql, 0), ga.max_q_len);
      const int pl = min(max(ga.prefix_lens[bb], 0), ga.max_kv_len - ql);
      ok = jj < pl + ql;  // absent gathered rows are not stored
    }
    rowok[tid] = ok;
  }
  const uint32_t lds0 = lds_addr(&lds[0]);
  // copy q (0..3: weight rows; 4..7: activation rows) of the interval of
  // steps kt, kt + 1 (kt even) into its buffer
  auto copy = [&](int kt, int q) {
    const uint32_t dst = lds0 + (uint32_t)(((kt >> 1) % NBUF) * 2 * SLOTS + (q >> 2) * SLOTS) * 16u +
                         (uint32_t)(((q & 3) * NWAVE + wave) * 1024);
    if (q < 4) dma16_sbase(woff[q & 3], W + kt * BK, dst);
    else dma16_sbase(aoff[q & 3], A + kt * BK, dst);
  };

  floatx4 acc[8][4];  // [n block][m block]: C[m 64 wm + 16 y + lr][n 128 wn + 16 x + 4 g4 + i]
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sq[4] = {0.f, 0.f, 0.f, 0.f};
  // the RMSNorm row statistic: only the wavefronts that publish it (wn == 0)
  const bool rownorm = g.epi == EPI_ROWNORM;
  const bool rowstat = rownorm && wn == 0;
  const int NK = part ? min(kper, g.K / BK - kt0) : g.K / BK;

  // two k steps (one barrier interval): fragments of step kt from buffer
  // kt % NBUF are read before its MFMAs, those of step kt + 1 in between them
  // (both steps' tiles are in LDS), so that only the first step's reads wait
  // on the LDS latency; the copies of steps kt + 2 and kt + 3 are issued first
  auto frags = [&](int kt, Frag<bf16>* af, Frag<bf16>* wf, int x) __attribute__((always_inline)) {
    const bf16x8* TW = &lds[((kt >> 1) % NBUF) * 2 * SLOTS];
    const bf16x8* TA = TW + SLOTS;
    const int c = (kt & 1) * 4 + g4;  // chunk of step kt in the interval's 128-byte rows
    // x < 0: all twelve fragments; else the ones read during MFMA group x
    if (x < 0) {
#pragma unroll
      for (int y = 0; y < 4; ++y) af[y].v = TA[swz(wm * 64 + y * 16 + lr, c)];
#pragma unroll
      for (int xx = 0; xx < 8; ++xx) wf[xx].v = TW[swz(wn * 128 + xx * 16 + lr, c)];
    } else if (x < 4) {
      af[x].v = TA[swz(wm * 64 + x * 16 + lr, c)];
      wf[2 * x].v = TW[swz(wn * 128 + 2 * x * 16 + lr, c)];
      wf[2 * x + 1].v = TW[swz(wn * 128 + (2 * x + 1) * 16 + lr, c)];
    }
  };
  auto rstat = [&](const Frag<bf16>* af) __attribute__((always_inline)) {
    if (rowstat) {
#pragma unroll
      for (int y = 0; y < 4; ++y)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = (float)af[y].v[e];
          sq[y] += f * f;
        }
    }
  };
  auto pair = [&](int kt) __attribute__((always_inline)) {
    Frag<bf16> af0[4], wf0[8], af1[4], wf1[8];
    frags(kt, af0, wf0, -1);
    // the copies of steps kt + 2 and kt + 3 all go out first: the earlier they
    // are issued, the less the next barrier interval waits for them
    if (kt + 2 < NK)
#pragma unroll
      for (int q = 0; q < 8; ++q) copy(kt + 2, q);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      __builtin_amdgcn_sched_barrier(0);
      frags(kt + 1, af1, wf1, x);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = mfma16(wf0[x], af0[y], acc[x][y]);
    }
    rstat(af0);
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = mfma16(wf1[x], af1[y], acc[x][y]);
    rstat(af1);
  };

#pragma unroll
  for (int q = 0; q < 8; ++q) copy(0, q);
  for (int kt = 0; kt < NK; kt += 2) {
    // this wavefront's copies of steps kt, kt + 1 (issued during step kt - 2)
    // are done; no newer ones exist yet
    MLA_WAIT_VMCNT(0);
    lds_barrier();  // every wavefront's copies of kt, kt + 1 landed; kt - 2, kt - 1 read by all
    pair(kt);
  }
  if (part) {
    // fp32 partial tile of split blockIdx.y: lane holds C[m][n .. n + 3]
    float* P = part + (int64_t)blockIdx.y * g.M * g.N;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int m = m0 + wm * 64 + y * 16 + lr;
      if (m >= g.M) continue;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int n = n0 + wn * 128 + x * 16 + 4 * g4;
        if (n + 3 < g.N) {
          *reinterpret_cast<floatx4*>(P + (int64_t)m * g.N + n) = acc[x][y];
        } else {
          for (int e = 0; e < 4 && n + e < g.N; ++e) P[(int64_t)m * g.N + n + e] = acc[x][y][e];
        }
      }
    }
    return;
  }
  lds_barrier();  // the ring is read by all before it stages the output

  if (rownorm) {
    // lanes lr, lr+16, lr+32, lr+48 hold disjoint k chunks of the same rows;
    // wavefronts wn = 0 and 1 both saw every row of their wm band: wn = 0 writes
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      float t = sq[y];
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      if (wn == 0 && g4 == 0) rowscale[wm * 64 + y * 16 + lr] = rsqrtf(t / (float)g.K + g.eps);
    }
    __syncthreads();
  }

  // epilogue, staged through LDS: lane holds C[m][n .. n + 3] for
  // m = 64 wm + 16 y + lr, n = 128 wn + 16 x + 4 g4 (tile-local). The bf16
  // tile is written as 256 rows of 32 16-byte chunks, chunk c of row r at
  // position c ^ (r & 31) (the 16 rows of one write land on distinct chunks),
  // then stored to C with 16 contiguous bytes per lane, 512 bytes per row.
  char* cst = reinterpret_cast<char*>(&lds[0]);
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int ml = wm * 64 + y * 16 + lr;
    const float rs = rownorm ? rowscale[ml] : 1.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const floatx4 v = acc[x][y] * rs;
      const int c = wn * 16 + x * 2 + (g4 >> 1);
      *reinterpret_cast<bf16x4*>(cst + (ml * 32 + (c ^ (ml & 31))) * 16 + (g4 & 1) * 8) =
          bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    }
  }
  __syncthreads();
  bf16* C = reinterpret_cast<bf16*>(g.C);
  const bf16* G = reinterpret_cast<const bf16*>(g.G);
  const int c = tid & 31;
  const int n = n0 + c * 8;
#pragma unroll 4
  for (int it = 0; it < BM / 16; ++it) {
    const int ml = it * 16 + (tid >> 5);
    const int m = m0 + ml;
    if (!rowok[ml] || n >= g.N) continue;
    bf16x8 v = *reinterpret_cast<const bf16x8*>(cst + (ml * 32 + (c ^ (ml & 31))) * 16);
    if (g.epi == EPI_GATE) {
      const bf16* gp = G + (int64_t)m * g.ldg + n;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < g.N) v[e] = (bf16)((float)v[e] * sigmoidf((float)gp[e]));
    }
    bf16* dst = C + (int64_t)m * g.ldc + n;
    if (n + 7 < g.N) {
      *reinterpret_cast<bf16x8*>(dst) = v;
    } else {
      for (int e = 0; e < 8 && n + e < g.N; ++e) dst[e] = v[e];
    }
  }
}

}  // namespace

namespace {
// every condition of the kernel except the number of output tiles (min_n:
// the narrowest product worth 256-wide tiles)
bool big_shape_ok(const GemmArgs& g, bool is_bf16, int min_n = 256) {
  if (!is_bf16 || g.batch != 1 || g.K % (2 * BK) != 0 || g.M < 512 || g.N < min_n) return false;  // two steps per barrier
  // 16-byte output stores (and gate loads)
  if (g.ldc % 8 || (reinterpret_cast<uintptr_t>(g.C) & 15)) return false;
  if (g.epi == EPI_GATE && (g.ldg % 8 || (reinterpret_cast<uintptr_t>(g.G) & 15))) return false;
  // per-slot source offsets are 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 31;  // elements (2 bytes each)
  if ((int64_t)g.N * g.ldw >= lim) return false;
  if (!g.gather && (int64_t)g.M * g.lda >= lim) return false;
  if (g.gather && (int64_t)g.ga.num_blocks * g.ga.page * g.ga.entry >= lim) return false;
  return true;
}
int64_t big_tiles(const GemmArgs& g) { return (int64_t)((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN); }
}  // namespace

bool gemm_big_eligible(const GemmArgs& g, bool is_bf16) { return big_shape_ok(g, is_bf16) && big_tiles(g) >= 256; }

int gemm_big_splits(const GemmArgs& g, bool is_bf16, int64_t ws_elems, bool narrow) {
  if (!big_shape_ok(g, is_bf16, narrow ? 8 : 256) || g.gather || g.epi != EPI_STORE) return 0;
  const int64_t tiles = big_tiles(g);
  if (tiles >= 256) return 0;
  // 2..8 splits of at least 512 of K, even step counts per split: the count
  // with the least estimated time = rounds of the 256 CUs x steps per split x
  // ~0.95 us per 32-wide step of a 256 x 256 tile, plus the fp32 partials the
  // reduce reads and the output it writes at ~4 TB/s
  const int nk = g.K / BK;
  int best = 0;
  double best_us = 1e300;
  for (int sp = 2; sp <= std::min(8, g.K / 512); ++sp) {
    if ((int64_t)sp * g.M * g.N > ws_elems) break;
    const int kper = ((nk + sp - 1) / sp + 1) / 2 * 2;
    const int used = (nk + kper - 1) / kper;  // splits left non-empty by the rounding
    const double rounds = (double)((tiles * used + 255) / 256);
    const double us = rounds * kper * 0.95 + (double)g.M * g.N * (4.0 * used + 2.0) / 4.0e6;
    if (us < best_us - 1e-9) { best_us = us; best = used; }
  }
  return best >= 2 ? best : 0;
}

hipError_t gemm_big_launch(const GemmArgs& g, float* part, int splits, hipStream_t s) {
  TileMap tm;
  tm.mtiles = (g.M + BM - 1) / BM;
  tm.ntiles = (g.N + BN - 1) / BN;
  // XCD grid: estimated Infinity-Cache traffic xn |A| + xm |W| (each XCD reads
  // its A band once per N band and its W band once); with a short k loop the W
  // band must also stay resident in the 4 MB L2 of the XCD
  const double a_bytes = (double)g.M * g.K * 2, w_bytes = (double)g.N * g.K * 2;
  const int opts[4][2] = {{1, 8}, {2, 4}, {4, 2}, {8, 1}};
  double best = 1e300;
  tm.xm = 2; tm.xn = 4;
  for (const auto& o : opts) {
    if (o[0] > tm.mtiles || o[1] > tm.ntiles) continue;
    if (g.K <= 1024 && w_bytes / o[1] > 3.0 * 1024 * 1024 && o[1] < 8) continue;
    const double cost = o[1] * a_bytes + o[0] * w_bytes;
    if (cost < best) { best = cost; tm.xm = o[0]; tm.xn = o[1]; }
  }
  // workgroups per XCD: the largest block
  int per = 0;
  for (int x = 0; x < 8; ++x) {
    const int xi = x / tm.xn, xj = x % tm.xn;
    const int mb = (xi + 1) * tm.mtiles / tm.xm - xi * tm.mtiles / tm.xm;
    const int nb = (xj + 1) * tm.ntiles / tm.xn - xj * tm.ntiles / tm.xn;
    per = std::max(per, mb * nb);
  }
  if (splits > 1) {
    const int nk = g.K / BK, kper = ((nk + splits - 1) / splits + 1) / 2 * 2;
    hipLaunchKernelGGL(gemm_big_kernel, dim3(per * 8, splits), dim3(NWAVE * 64), 0, s, g, tm, part, kper);
  } else {
    hipLaunchKernelGGL(gemm_big_kernel, dim3(per * 8), dim3(NWAVE * 64), 0, s, g, tm, (float*)nullptr, 0);
  }
  return hipGetLastError();
}

}  // namespace mla
