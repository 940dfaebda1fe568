// MFMA GEMM for gfx950: C[M, N] = A[M, K] . W[N, K]^T (nn.Linear weights).
//
// One workgroup of 4 wavefronts computes a BM x BN tile; the k axis is staged
// through LDS in 128-byte rows (64 bf16 or 32 fp32 per row, padded by 16 bytes
// so that the 16-byte fragment reads of 8 consecutive rows hit distinct banks),
// double-buffered with a register prefetch of the next k tile. The weight tile
// is the MFMA "A" operand and the activation tile the "B" operand, so each
// lane ends up holding 4 consecutive output columns of one output row and the
// epilogue stores 4 contiguous elements per lane.
//
// Few activation rows (M <= 128, bf16): gemm_stream_kernel. Such products
// stream their weights from HBM once, so what a CU loads should be mostly
// weight bytes and as much of it in flight as possible: a BM x BN tile with
// BN >= BM (64 activation rows against 64-128 weight rows), 256-byte k rows
// copied straight into LDS (global_load_lds_dwordx4, no staging registers)
// through a ring of 3-4 stages, so that two or three stages are in flight
// while one feeds the MFMAs; the tile width and split-K are chosen so that
// the workgroups fill the CUs in one round.
#include "common.h"
#include "gemm.h"

namespace mla {

namespace {

// RB bytes of k per tile row: 128, or 256 for few activation rows (the
// weight-streaming shapes), where a deeper k tile doubles the bytes each
// register prefetch has in flight
template <typename T, int RB>
struct Tile {
  static constexpr int BK = RB / sizeof(T);          // k elements per LDS row
  static constexpr int VEC = 16 / sizeof(T);         // elements per 16-byte vector
  static constexpr int VPR = RB / 16;                // 16-byte vectors per row
  static constexpr int ROW = BK + VEC;                // padded LDS row (elements)
  static constexpr int KSTEPS = BK / 32;             // 32-element MFMA steps per k tile
};

template <typename T, int BM, int BN, int WM, int WN, int RB>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g, float* ws, int splits) {
  using TT = Tile<T, RB>;
  using V = typename Vec16<T>::type;
  constexpr int BK = TT::BK, VEC = TT::VEC, ROW = TT::ROW, VPR = TT::VPR;
  constexpr int TM = BM / WM, TN = BN / WN, MB = TM / 16, NB = TN / 16;
  static_assert(WM * WN == 4, "4 wavefronts");
  static_assert(MB >= 1 && NB >= 1, "wave tile");
  constexpr int NV = (BM + BN) * VPR;       // 16-byte vectors per k tile
  constexpr int VPT = (NV + 255) / 256;
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * ROW];
  __shared__ int64_t rowoff[BM];
  __shared__ float rowscale[BM];
  __shared__ int any_row;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int split = blockIdx.z % splits, bz = blockIdx.z / splits;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const T* __restrict__ A = reinterpret_cast<const T*>(g.A) + (g.gather ? 0 : bz * g.sA);
  const T* __restrict__ W = reinterpret_cast<const T*>(g.W) + bz * g.sW;

  // k range of this split (whole k tiles)
  const int ktiles_total = (g.K + BK - 1) / BK;
  const int kt_per = (ktiles_total + splits - 1) / splits;
  const int kt0 = split * kt_per;
  const int kt1 = min(ktiles_total, kt0 + kt_per);

  if (tid == 0) any_row = 0;
  __syncthreads();
  // source offset (elements) of every activation row of the tile, -1 = absent
  for (int r = tid; r < BM; r += 256) {
    const int m = m0 + r;
    int64_t off = -1;
    if (m < g.M) {
      if (!g.gather) {
        off = (int64_t)m * g.lda;
      } else {
        const GatherA& ga = g.ga;
        const int b = m / ga.max_kv_len, j = m % ga.max_kv_len;
        int ql = ga.cu_seqlens[b + 1] - ga.cu_seqlens[b];
        ql = min(max(ql, 0), ga.max_q_len);
        const int pl = min(max(ga.prefix_lens[b], 0), ga.max_kv_len - ql);
        if (j < pl + ql) {
          const int blk = ga.block_table[(int64_t)b * ga.max_blocks + j / ga.page];
          if (blk >= 0 && blk < ga.num_blocks)
            off = ((int64_t)blk * ga.page + j % ga.page) * ga.entry;
        }
      }
    }
    rowoff[r] = off;
    if (off >= 0) any_row = 1;
  }
  __syncthreads();
  // no row of this tile exists (rows past M or past a sequence's length):
  // nothing is stored for it, and split-K partials of such rows are never read
  if (!any_row) return;

  V regs[VPT];
  float sq[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) sq[i] = 0.f;

  auto load_tile = [&](int kt) {
    const int kbase = kt * BK;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * 256;
      V val = {};
      if (v < NV) {
        const int row = v / VPR, k = kbase + (v % VPR) * VEC;
        if (k < g.K) {
          if (row < BN) {
            const int n = n0 + row;
            if (n < g.N) val = *reinterpret_cast<const V*>(W + (int64_t)n * g.ldw + k);
          } else {
            const int64_t off = rowoff[row - BN];
            if (off >= 0) val = *reinterpret_cast<const V*>(A + off + k);
          }
        }
      }
      regs[i] = val;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = tid + i * 256;
      if (v < NV) {
        const int row = v / VPR;
        *reinterpret_cast<V*>(&lds[buf][row * ROW + (v % VPR) * VEC]) = regs[i];
        if (g.epi == EPI_ROWNORM && row >= BN) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float f = to_f32(regs[i][e]);
            sq[i] += f * f;
          }
        }
      }
    }
  };

  floatx4 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
  }
  __syncthreads();
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) load_tile(kt + 1);
    const T* base = lds[buf];
#pragma unroll
    for (int ks = 0; ks < TT::KSTEPS; ++ks) {
      Frag<T> wf[NB], af[MB];
#pragma unroll
      for (int a = 0; a < NB; ++a) load_frag(wf[a], base + (wn * TN + a * 16 + lr) * ROW + ks * 32 + lk);
#pragma unroll
      for (int b = 0; b < MB; ++b) load_frag(af[b], base + (BN + wm * TM + b * 16 + lr) * ROW + ks * 32 + lk);
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = mfma16(wf[a], af[b], acc[a][b]);
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (g.epi == EPI_ROWNORM) {
    // rows of A loaded by this thread: sum over the VPR lanes sharing a row
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      float s = sq[i];
#pragma unroll
      for (int o = 1; o < VPR; o <<= 1) s += __shfl_xor(s, o);
      const int v = tid + i * 256;
      if (v < NV && (v % VPR) == 0 && (v / VPR) >= BN)
        rowscale[(v / VPR) - BN] = rsqrtf(s / (float)g.K + g.eps);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n+3]
  const int nl = 4 * (lane >> 4);
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int ml = wm * TM + b * 16 + lr;
    const int m = m0 + ml;
    if (m >= g.M || rowoff[ml] < 0) continue;
    const float rs = (g.epi == EPI_ROWNORM) ? rowscale[ml] : 1.f;
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int n = n0 + wn * TN + a * 16 + nl;
      if (n >= g.N) continue;
      floatx4 v = acc[a][b];
      if (splits > 1) {
        float* dst = ws + ((int64_t)split * g.M + m) * g.N + n;
        if (n + 3 < g.N) {
          *reinterpret_cast<floatx4*>(dst) = v;
        } else {
          for (int e = 0; e < 4 && n + e < g.N; ++e) dst[e] = v[e];
        }
        continue;
      }
      if (g.epi == EPI_ROWNORM) v = v * rs;
      if (g.epi == EPI_GATE) {
        const T* G = reinterpret_cast<const T*>(g.G) + bz * g.sG + (int64_t)m * g.ldg + n;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) v[e] *= sigmoidf(to_f32(G[e]));
      }
      T* dst = reinterpret_cast<T*>(g.C) + bz * g.sC + (int64_t)m * g.ldc + n;
      if (n + 3 < g.N) {
        if constexpr (sizeof(T) == 2) {
          bf16x4 o = {from_f32<T>(v[0]), from_f32<T>(v[1]), from_f32<T>(v[2]), from_f32<T>(v[3])};
          *reinterpret_cast<bf16x4*>(dst) = o;
        } else {
          *reinterpret_cast<floatx4*>(dst) = v;
        }
      } else {
        for (int e = 0; e < 4 && n + e < g.N; ++e) dst[e] = from_f32<T>(v[e]);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// weight-streaming kernel (bf16, M <= 128)
// ---------------------------------------------------------------------------
// SBK k elements per stage: 128 (256-byte rows) or 64 (128-byte rows, for the
// widest tiles). Split-K writes fp32 partial sums to ws[split][M][N] and, for
// the RMSNorm epilogue, each split's partial row sums of squares (from the
// workgroups of the first N tile) to ws[splits * M * N + split * M + m]; the
// reduce kernel applies the row scale.
template <int BM, int BN, int WM, int WN, int NST, int SBK>
__global__ __launch_bounds__(256, 1) void gemm_stream_kernel(GemmArgs g, float* ws, int splits) {
  constexpr int SCH = SBK / 8;  // 16-byte chunks per row
  constexpr int TM = BM / WM, TN = BN / WN, MB = TM / 16, NB = TN / 16;
  static_assert(WM * WN == 4 && MB >= 1 && NB >= 1 && TM % 16 == 0 && TN % 16 == 0, "wave tile");
  constexpr int SLOTS = (BN + BM) * SCH;  // 16-byte slots per stage: weight rows, then activation rows
  static_assert(SLOTS % 256 == 0 && (BN * SCH) % 64 == 0, "whole 64-lane copy instructions per operand");
  constexpr int DPW = SLOTS / 256;        // copy instructions per wavefront per stage
  constexpr int WSL = BN * SCH;           // weight slots
  static_assert(NST >= 2 && NST <= 4, "ring of 2-4 stages");
  // stage s, row r (weight rows 0..BN-1, activation rows BN..): chunk c at slot r * SCH + (c ^ (r % SCH)),
  // so the 16 rows of one fragment read land on distinct chunks of the row
  __shared__ __attribute__((aligned(16))) bf16x8 lds[NST][SLOTS];
  __shared__ float rowscale[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const int lr = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.z % splits, bz = blockIdx.z / splits;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const char* Wb = reinterpret_cast<const char*>(g.W) + (int64_t)bz * g.sW * 2;
  const char* Ab = reinterpret_cast<const char*>(g.A) + (int64_t)bz * g.sA * 2;
  const int ktiles = g.K / SBK;
  const int kt_per = (ktiles + splits - 1) / splits;
  const int kt0 = split * kt_per, kt1 = min(ktiles, kt0 + kt_per);

  // per-lane source byte offsets of this wavefront's slots (k-independent;
  // rows past N or M read the last row: their products are never stored;
  // 32-bit offsets, host check)
  uint32_t off[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int sl = (4 * j + wave) * 64 + lane;
    const int row = sl / SCH, c = (sl % SCH) ^ (row & (SCH - 1));
    if (row < BN) off[j] = (uint32_t)((int64_t)min(n0 + row, g.N - 1) * g.ldw * 2) + (uint32_t)(c * 16);
    else off[j] = (uint32_t)((int64_t)min(m0 + row - BN, g.M - 1) * g.lda * 2) + (uint32_t)(c * 16);
  }
  const uint32_t lds0 = lds_addr(&lds[0][0]);
  auto issue = [&](int kt, int buf) {
    const uint32_t dst = lds0 + (uint32_t)buf * (SLOTS * 16);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const bool w = (4 * j + wave) * 64 < WSL;  // uniform: the instruction's 64 slots are weight rows
      dma16_sbase(off[j], (w ? Wb : Ab) + (int64_t)kt * (SBK * 2), dst + (uint32_t)(4 * j + wave) * 1024u);
    }
  };

  floatx4 acc[NB][MB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  float sq[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) sq[b] = 0.f;
  const bool rownorm = g.epi == EPI_ROWNORM;
  // these wavefronts see every activation row (split-K: only the first N
  // tile's workgroups publish the statistic)
  const bool rowstat = rownorm && wn == 0 && (splits == 1 || blockIdx.x == 0);

  auto compute = [&](int buf) {
    const bf16x8* T = &lds[buf][0];
#pragma unroll
    for (int ks = 0; ks < SBK / 32; ++ks) {
      Frag<bf16> wf[NB], af[MB];
#pragma unroll
      for (int a = 0; a < NB; ++a) {
        const int row = wn * TN + a * 16 + lr;
        wf[a].v = T[row * SCH + ((ks * 4 + g4) ^ (row & (SCH - 1)))];
      }
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int row = BN + wm * TM + b * 16 + lr;
        af[b].v = T[row * SCH + ((ks * 4 + g4) ^ (row & (SCH - 1)))];
      }
      if (rowstat) {
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)af[b].v[e];
            sq[b] += f * f;
          }
      }
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = mfma16(wf[a], af[b], acc[a][b]);
    }
  };

  // ring: stages kt + 1 .. kt + NST - 1 are in flight while stage kt is used
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (kt0 + p < kt1) issue(kt0 + p, p);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int i = kt - kt0;
    const int later = min(NST - 2, kt1 - 1 - kt);  // stages after kt already issued
    if (later <= 0) MLA_WAIT_VMCNT(0);
    else if (later == 1) MLA_WAIT_VMCNT(DPW);
    else MLA_WAIT_VMCNT(2 * DPW);
    lds_barrier();  // stage kt is in LDS for every wavefront; stage kt - 1 is no longer read
    if (kt + NST - 1 < kt1) issue(kt + NST - 1, (i + NST - 1) % NST);
    compute(i % NST);
  }

  if (rownorm) {
    // lanes lr, lr + 16, lr + 32, lr + 48 hold disjoint k chunks of one row
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      float s = sq[b];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int ml = wm * TM + b * 16 + lr;
      if (rowstat && g4 == 0) {
        if (splits == 1) rowscale[ml] = rsqrtf(s / (float)g.K + g.eps);
        else if (m0 + ml < g.M) ws[(int64_t)splits * g.M * g.N + (int64_t)split * g.M + m0 + ml] = s;
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n + 3]
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int ml = wm * TM + b * 16 + lr;
    const int m = m0 + ml;
    if (m >= g.M) continue;
    const float rs = rownorm && splits == 1 ? rowscale[ml] : 1.f;
#pragma unroll
    for (int a = 0; a < NB; ++a) {
      const int n = n0 + wn * TN + a * 16 + 4 * g4;
      if (n >= g.N) continue;
      floatx4 v = acc[a][b];
      if (splits > 1) {
        float* dst = ws + ((int64_t)split * g.M + m) * g.N + n;
        if (n + 3 < g.N) {
          *reinterpret_cast<floatx4*>(dst) = v;
        } else {
          for (int e = 0; e < 4 && n + e < g.N; ++e) dst[e] = v[e];
        }
        continue;
      }
      if (rownorm) v = v * rs;
      if (g.epi == EPI_GATE) {
        const bf16* G = reinterpret_cast<const bf16*>(g.G) + bz * g.sG + (int64_t)m * g.ldg + n;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) v[e] *= sigmoidf((float)G[e]);
      }
      bf16* dst = reinterpret_cast<bf16*>(g.C) + bz * g.sC + (int64_t)m * g.ldc + n;
      if (n + 3 < g.N) {
        *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      } else {
        for (int e = 0; e < 4 && n + e < g.N; ++e) dst[e] = (bf16)v[e];
      }
    }
  }
}

// C[m, n] = sum_s ws[s][m][n]; rownorm: times rsqrt(mean of row m's squares
// + eps), the squares summed over the splits' partials after the partial sums
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ ws, int splits, int M, int N,
                                                      T* __restrict__ C, int64_t ldc, bool rownorm = false,
                                                      int K = 1, float eps = 0.f) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  auto row_scale = [&](int m) {
    if (!rownorm) return 1.f;
    float q = 0.f;
    for (int k = 0; k < splits; ++k) q += ws[(int64_t)splits * total + (int64_t)k * M + m];
    return rsqrtf(q / (float)K + eps);
  };
  const int m = (int)(i / N), n = (int)(i % N);
  if (n + 3 < N) {
    floatx4 s = *reinterpret_cast<const floatx4*>(ws + i);
    for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const floatx4*>(ws + (int64_t)k * total + i);
    s = s * row_scale(m);
    T* dst = C + (int64_t)m * ldc + n;
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(s[e]);
  } else {
    for (int e = 0; e < 4; ++e) {
      const int64_t j = i + e;
      if (j >= total) break;
      const int mm = (int)(j / N), nn = (int)(j % N);
      float s = 0.f;
      for (int k = 0; k < splits; ++k) s += ws[(int64_t)k * total + j];
      C[(int64_t)mm * ldc + nn] = from_f32<T>(s * row_scale(mm));
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN, int RB>
hipError_t launch_cfg(const GemmArgs& g, float* ws, int splits, hipStream_t s) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch * splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, RB>), grid, dim3(256), 0, s, g, ws, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  const int blocks = (int)((total / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(splitk_reduce<T>, dim3(blocks), dim3(256), 0, s, ws, splits, g.M, g.N,
                     reinterpret_cast<T*>(g.C), g.ldc);
  return hipGetLastError();
}


template <int BM, int BN, int WM, int WN, int NST, int SBK>
hipError_t launch_stream(const GemmArgs& g, float* ws, int splits, hipStream_t s) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch * splits);
  hipLaunchKernelGGL((gemm_stream_kernel<BM, BN, WM, WN, NST, SBK>), grid, dim3(256), 0, s, g, ws, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = (int64_t)g.M * g.N;
  const int blocks = (int)((total / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(splitk_reduce<bf16>, dim3(blocks), dim3(256), 0, s, ws, splits, g.M, g.N,
                     reinterpret_cast<bf16*>(g.C), g.ldc, g.epi == EPI_ROWNORM, g.K, g.eps);
  return hipGetLastError();
}

// (activation rows, weight rows, k per stage) of the weight-streaming configurations
struct StreamCfg {
  int bm, bn, sbk;
};
constexpr StreamCfg kStreamCfgs[] = {
    {64, 128, 128}, {64, 96, 128}, {64, 64, 128},
    {32, 128, 128}, {32, 96, 128}, {32, 64, 128},
    {16, 128, 128}, {16, 64, 128},
};

// The weight-streaming configuration and split-K for g, or false when it
// does not apply. Score of a choice: the fraction of the CU slots its
// workgroups fill per round (one workgroup per CU) x the fraction of the
// loaded bytes that are weights x the fraction of the weight rows that exist.
bool stream_pick(const GemmArgs& g, float* ws, int64_t ws_elems, int cus, int* cfg_out, int* splits_out) {
  if (g.gather || g.M > 128 || g.K % 128 != 0 || g.K < 256) return false;
  const int64_t lim = (int64_t)1 << 32;  // 32-bit per-lane byte offsets
  if ((int64_t)(g.N - 1) * g.ldw * 2 + 2 * (int64_t)g.K >= lim) return false;
  if ((int64_t)(g.M - 1) * g.lda * 2 + 2 * (int64_t)g.K >= lim) return false;
  const int bm = g.M <= 16 ? 16 : (g.M <= 32 ? 32 : 64);
  double best = -1.0;
  for (int ci = 0; ci < (int)(sizeof(kStreamCfgs) / sizeof(kStreamCfgs[0])); ++ci) {
    const StreamCfg& c = kStreamCfgs[ci];
    if (c.bm != bm) continue;
    const int ktiles = g.K / c.sbk;
    const int64_t nt = (g.N + c.bn - 1) / c.bn;
    const int64_t tiles = nt * ((g.M + bm - 1) / bm) * g.batch;
    int sp = 1;
    if ((g.epi == EPI_STORE || g.epi == EPI_ROWNORM) && g.batch == 1 && ws != nullptr && tiles < cus) {
      sp = (int)std::min<int64_t>(cus / tiles, 16);
      sp = std::min(sp, std::max(1, ktiles / 2));  // at least two stages per split
      while (sp > 1 && (int64_t)sp * g.M * (g.N + 1) > ws_elems) --sp;
      if (sp > 1) {
        const int per = (ktiles + sp - 1) / sp;
        sp = (ktiles + per - 1) / per;
      }
    }
    const int64_t wgs = tiles * sp;
    const int64_t rounds = (wgs + cus - 1) / cus;
    const double score = (double)wgs / (double)(rounds * cus) * c.bn / (double)(c.bn + bm) *
                         (double)g.N / (double)(nt * c.bn);
    if (score > best + 1e-9) { best = score; *cfg_out = ci; *splits_out = sp; }
  }
  return best > 0.0;
}

hipError_t launch_stream_cfg(const GemmArgs& g, float* ws, int ci, int splits, hipStream_t s) {
  switch (ci) {
    case 0: return launch_stream<64, 128, 1, 4, 3, 128>(g, ws, splits, s);
    case 1: return launch_stream<64, 96, 2, 2, 3, 128>(g, ws, splits, s);
    case 2: return launch_stream<64, 64, 1, 4, 4, 128>(g, ws, splits, s);
    case 3: return launch_stream<32, 128, 1, 4, 3, 128>(g, ws, splits, s);
    case 4: return launch_stream<32, 96, 2, 2, 3, 128>(g, ws, splits, s);
    case 5: return launch_stream<32, 64, 1, 4, 4, 128>(g, ws, splits, s);
    case 6: return launch_stream<16, 128, 1, 4, 4, 128>(g, ws, splits, s);
    default: return launch_stream<16, 64, 1, 4, 4, 128>(g, ws, splits, s);
  }
}

template <typename T>
hipError_t launch_t(const GemmArgs& g, float* ws, int64_t ws_elems, hipStream_t s) {
  // k elements per tile: 256 bytes per row for few activation rows, else 128
  const bool deep = g.M <= 64 && sizeof(T) == 2 && g.K >= 1024;
  const int BK = (deep ? 256 : 128) / (int)sizeof(T);
  // tile shape by M; split-K when the grid is too small to fill 256 CUs
  int bm, bn;
  if (g.M <= 16) { bm = 16; bn = 64; }
  else if (g.M <= 64) { bm = 64; bn = 64; }
  else if ((int64_t)((g.M + 127) / 128) * ((g.N + 127) / 128) * g.batch >= 512) { bm = 128; bn = 128; }
  else { bm = 64; bn = 64; }
  const int64_t tiles = (int64_t)((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn) * g.batch;
  int splits = 1;
  const int ktiles = (g.K + BK - 1) / BK;
  if (tiles < 512 && g.batch == 1 && g.epi == EPI_STORE && !g.gather && ws != nullptr) {
    // deep tiles (70 KB of LDS) fit two workgroups per CU: fill those 512
    // slots in one round rather than spill a few workgroups into a second
    splits = deep ? (int)std::max<int64_t>(1, 512 / tiles) : (int)((512 + tiles - 1) / tiles);
    splits = std::min(splits, std::max(1, ktiles / 4));
    splits = std::min(splits, 16);
    while (splits > 1 && (int64_t)splits * g.M * g.N > ws_elems) --splits;
    // every split must own at least one k tile
    if (splits > 1) {
      const int per = (ktiles + splits - 1) / splits;
      splits = (ktiles + per - 1) / per;
    }
  }
  if (bm == 16) return deep ? launch_cfg<T, 16, 64, 1, 4, 256>(g, ws, splits, s) : launch_cfg<T, 16, 64, 1, 4, 128>(g, ws, splits, s);
  if (bm == 64) return deep ? launch_cfg<T, 64, 64, 1, 4, 256>(g, ws, splits, s) : launch_cfg<T, 64, 64, 1, 4, 128>(g, ws, splits, s);
  return launch_cfg<T, 128, 128, 2, 2, 128>(g, ws, splits, s);
}

}  // namespace

const char* gemm_check(const GemmArgs& g, bool is_bf16) {
  const int vec = is_bf16 ? 8 : 4;
  if (g.M < 0 || g.N <= 0 || g.K <= 0 || g.batch <= 0) return "gemm: bad sizes";
  if (g.K % vec) return "gemm: K must be a multiple of 16 bytes";
  if ((g.lda % vec) || (g.ldw % vec) || (g.sA % vec) || (g.sW % vec)) return "gemm: A/W strides must be 16-byte multiples";
  if ((g.ldc % 4) || (g.sC % 4)) return "gemm: C strides must be multiples of 4 elements";
  if ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.W)) & 15) return "gemm: A/W must be 16-byte aligned";
  if (reinterpret_cast<uintptr_t>(g.C) & (is_bf16 ? 7 : 15)) return "gemm: C misaligned";
  if (g.gather && (g.ga.entry % vec)) return "gemm: gathered rows must be 16-byte multiples";
  return nullptr;
}

constexpr int kMaxReduceSplitsBig = 8;  // gemm_big_splits never returns more

hipError_t gemm_launch(const GemmArgs& g, bool is_bf16, float* ws, int64_t ws_elems, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  if (g.zeros != nullptr && gemm_big_eligible(g, is_bf16)) {
    // a narrow last column of 256-wide tiles (N mod 256 <= 128, e.g. the
    // 2112-wide first projection) still costs full tiles; when it adds a
    // round of workgroups, the 256-multiple part runs alone and the narrow
    // columns run as a product of their own
    const int tail = g.N % 256;
    if (tail > 0 && tail <= 128 && g.epi == EPI_STORE && !g.gather && g.batch == 1) {
      GemmArgs head = g;
      head.N = g.N - tail;
      const int64_t mt = (g.M + 255) / 256;
      const int64_t rounds_all = (mt * ((g.N + 255) / 256) + 255) / 256, rounds_head = (mt * (head.N / 256) + 255) / 256;
      if (rounds_head < rounds_all && gemm_big_eligible(head, is_bf16)) {
        if (hipError_t e = gemm_big_launch(head, nullptr, 1, s); e != hipSuccess) return e;
        GemmArgs t = g;
        t.N = tail;
        t.W = reinterpret_cast<const char*>(g.W) + (size_t)head.N * g.ldw * 2;
        t.C = reinterpret_cast<char*>(g.C) + (size_t)head.N * 2;
        // the narrow columns on the same kernel, k split over the CUs
        if (const int sp = ws != nullptr ? gemm_big_splits(t, is_bf16, ws_elems, true) : 0;
            sp > 1 && sp <= kMaxReduceSplitsBig) {
          if (hipError_t e = gemm_big_launch(t, ws, sp, s); e != hipSuccess) return e;
          const int64_t total = (int64_t)t.M * t.N;
          const int blocks = (int)((total / 4 + 255) / 256 + 1);
          hipLaunchKernelGGL(splitk_reduce<bf16>, dim3(blocks), dim3(256), 0, s, ws, sp, t.M, t.N,
                             reinterpret_cast<bf16*>(t.C), t.ldc, false, t.K, 0.f);
          return hipGetLastError();
        }
        return gemm_launch(t, is_bf16, ws, ws_elems, s);
      }
    }
    return gemm_big_launch(g, nullptr, 1, s);
  }
  if (g.zeros != nullptr && ws != nullptr) {
    if (const int sp = gemm_big_splits(g, is_bf16, ws_elems); sp > 1) {
      if (hipError_t e = gemm_big_launch(g, ws, sp, s); e != hipSuccess) return e;
      const int64_t total = (int64_t)g.M * g.N;
      const int blocks = (int)((total / 4 + 255) / 256 + 1);
      hipLaunchKernelGGL(splitk_reduce<bf16>, dim3(blocks), dim3(256), 0, s, ws, sp, g.M, g.N,
                         reinterpret_cast<bf16*>(g.C), g.ldc, false, g.K, 0.f);
      return hipGetLastError();
    }
  }
  int ci = 0, splits = 1;
  if (is_bf16 && stream_pick(g, ws, ws_elems, 256, &ci, &splits)) return launch_stream_cfg(g, ws, ci, splits, s);
  return is_bf16 ? launch_t<bf16>(g, ws, ws_elems, s) : launch_t<float>(g, ws, ws_elems, s);
}

}  // namespace mla
