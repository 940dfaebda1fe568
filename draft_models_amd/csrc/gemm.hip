// MFMA GEMM for gfx950: C[M, N] = A[M, K] . W[N, K]^T (nn.Linear weights).
//
// One workgroup of 4 wavefronts computes a BM x BN tile; the k axis is staged
// through LDS in 128-byte rows (64 bf16 or 32 fp32 per row, padded by 16 bytes
// so that the 16-byte fragment reads of 8 consecutive rows hit distinct banks),
// double-buffered with a register prefetch of the next k tile. The weight tile
// is the MFMA "A" operand and the activation tile the "B" operand, so each
// lane ends up holding 4 consecutive output columns of one output row and the
// epilogue stores 4 contiguous elements per lane.
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

// C[m, n] = sum_s ws[s][m][n]
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ ws, int splits, int M, int N,
                                                      T* __restrict__ C, int64_t ldc) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const int64_t total = (int64_t)M * N;
  if (i >= total) return;
  const int m = (int)(i / N), n = (int)(i % N);
  if (n + 3 < N) {
    floatx4 s = *reinterpret_cast<const floatx4*>(ws + i);
    for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const floatx4*>(ws + (int64_t)k * total + i);
    T* dst = C + (int64_t)m * ldc + n;
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(s[e]);
  } else {
    for (int e = 0; e < 4; ++e) {
      const int64_t j = i + e;
      if (j >= total) break;
      const int mm = (int)(j / N), nn = (int)(j % N);
      float s = 0.f;
      for (int k = 0; k < splits; ++k) s += ws[(int64_t)k * total + j];
      C[(int64_t)mm * ldc + nn] = from_f32<T>(s);
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

hipError_t gemm_launch(const GemmArgs& g, bool is_bf16, float* ws, int64_t ws_elems, hipStream_t s) {
  if (g.M == 0) return hipSuccess;
  if (g.zeros != nullptr && gemm_big_eligible(g, is_bf16)) return gemm_big_launch(g, g.zeros, s);
  return is_bf16 ? launch_t<bf16>(g, ws, ws_elems, s) : launch_t<float>(g, ws, ws_elems, s);
}

}  // namespace mla
