// Backward pass of the expanded MLA layer on whole training sequences (no
// cached prefix; token j of a sequence at position j). SpecForge PR "Add
// config-selectable MLA draft attention" trains MLA as a draft attention and
// validates it with gradients (Validation); the forward is the expanded form
// of the MLA blog's wrapper forward and forward_mha listings, and every
// kernel here is the derivative of one of its steps:
//   * attention: dV = P^T dO, dP = dO V^T, dS = P (dP - D) with
//     D = rowsum(dO * O), dQ = scale dS K, dK = scale dS^T Q, recomputing
//     P = 2^(s log2e scale - lse2) from the forward's log-sum-exp;
//   * the shared rope key collects the rope part of dK of every head;
//   * RoPE: the opposite turn; RMSNorm: dx = rho (g - x rho^2 mean(g x)),
//     g = dy * gamma, and dgamma = sum over tokens of dy * x * rho;
//   * output gate: dO = dA sigma, d(gate input) = dA O sigma (1 - sigma).
// The dense products (x W^T, dY W, dY^T X) are the library's GEMMs; the
// token-axis contractions of the weight gradients run on transposed copies
// made here (transpose_kernel).
//
// Layouts: token-packed rows t = cu_seqlens[b] + j for every per-token buffer
// except the two the forward kernels address per sequence: the latent cache
// (identity pages, row b Lp + j) and the expanded keys/values (row b Lp + j),
// Lp = max_q_len rounded up to the cache page.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

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

// tokens of sequence b, clamped so that every row cu[b] + j stays below total_tokens
__device__ __forceinline__ int seq_len(const TrainArgs& a, int b) {
  const int t0 = a.cu_seqlens[b];
  return min(min(max(a.cu_seqlens[b + 1] - t0, 0), a.max_q_len), max(a.total_tokens - t0, 0));
}

// sequence of token t (cu_seqlens is nondecreasing; binary search)
__device__ __forceinline__ int seq_of(const TrainArgs& a, int t) {
  int lo = 0, hi = a.batch;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu_seqlens[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <typename T>
__device__ __forceinline__ void ld_frag(Frag<T>& f, const T* p, bool ok);
template <>
__device__ __forceinline__ void ld_frag(Frag<bf16>& f, const bf16* p, bool ok) {
  f.v = ok ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{};
}
template <>
__device__ __forceinline__ void ld_frag(Frag<float>& f, const float* p, bool ok) {
  if (ok) {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(p), hi = *reinterpret_cast<const floatx4*>(p + 4);
    f.v = floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    f.v = floatx8{};
  }
}

// element d of head h's key of token (b, j): k_nope from the expansion,
// k_pe (shared by the heads) from the latent cache
template <typename T>
__device__ __forceinline__ T key_elem(const TrainArgs& a, int b, int j, int h, int d) {
  const int64_t row = (int64_t)b * a.Lp + j;
  if (d < a.n) return reinterpret_cast<const T*>(a.kvexp)[row * a.ldkv + (int64_t)h * (a.n + a.dv) + d];
  if (d < a.n + a.r) return reinterpret_cast<const T*>(a.cache)[row * (a.c + a.r) + a.c + (d - a.n)];
  return T(0.f);
}
template <typename T>
__device__ __forceinline__ T val_elem(const TrainArgs& a, int b, int j, int h, int d) {
  if (d >= a.dv) return T(0.f);
  const int64_t row = (int64_t)b * a.Lp + j;
  return reinterpret_cast<const T*>(a.kvexp)[row * a.ldkv + (int64_t)h * (a.n + a.dv) + a.n + d];
}

// ---------------------------------------------------------------------------
// attention backward, keys side: dK and dV of one 64-key tile of one head.
// Wave w owns keys 16 w .. 16 w + 15 of the tile (MFMA A rows). Per 64-query
// tile: S^T = K Q^T and dP^T = V dO^T (lane: keys 4 g + i, query lr of each
// 16-query block), P^T and dS^T go through LDS to become A operands of
// dV += P^T dO and dK += dS^T Q, whose B operands read transposed copies of
// the query tile (Qt, dOt).
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(TrainArgs a) {
  constexpr int BT = 64, KS = DQK / 32, VS = DV / 32;
  constexpr int DKB = DQK / 16, DVB = DV / 16;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int QROW = DQK + PAD, DOROW = DV + PAD, TROW = BT + PAD;
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "padded head dims");
  __shared__ __attribute__((aligned(16))) T Qs[BT * QROW];
  __shared__ __attribute__((aligned(16))) T Qt[DQK * TROW];
  __shared__ __attribute__((aligned(16))) T dOs[BT * DOROW];
  __shared__ __attribute__((aligned(16))) T dOt[DV * TROW];
  __shared__ __attribute__((aligned(16))) T Pw[4][16 * TROW];
  __shared__ __attribute__((aligned(16))) T dSw[4][16 * TROW];
  __shared__ float lse_s[BT], D_s[BT];
  __shared__ int lo_s[BT], hi_s[BT];

  const int kt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = seq_len(a, b);
  const int k0 = kt * BT;
  if (k0 >= S) return;
  const int t0 = a.cu_seqlens[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const float sl2 = a.scale * kLog2e;
  const int qk = a.n + a.r;

  // this wave's keys as A operands
  const int kr = k0 + wave * 16 + lr;
  const bool krok = kr < S;
  Frag<T> kf[KS], vf[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[ks].v[e] = krok ? key_elem<T>(a, b, kr, h, ks * 32 + g * 8 + e) : T(0.f);
#pragma unroll
  for (int vs = 0; vs < VS; ++vs)
#pragma unroll
    for (int e = 0; e < 8; ++e) vf[vs].v[e] = krok ? val_elem<T>(a, b, kr, h, vs * 32 + g * 8 + e) : T(0.f);

  floatx4 dk[DKB], dv[DVB];
#pragma unroll
  for (int i = 0; i < DKB; ++i) dk[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < DVB; ++i) dv[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  // queries that can see a key of this tile
  int qbeg = 0, qend = S;
  if (a.mask.row_lo == nullptr) {
    if (a.mask.kind == 1) qbeg = k0;
    else if (a.mask.kind == 2) { qbeg = k0; qend = min(S, k0 + BT - 1 + max(a.mask.window, 0)); }
  }
  qbeg = (qbeg / BT) * BT;
  const T* Qg = reinterpret_cast<const T*>(a.q);
  const T* dOg = reinterpret_cast<const T*>(a.dO);

  for (int q0 = qbeg; q0 < qend; q0 += BT) {
    // ---- stage the query tile: Q, Q^T, dO, dO^T and the per-query statistics
    for (int v = tid; v < BT * DQK; v += 256) {
      const int qq = v / DQK, d = v % DQK;
      const int qi = q0 + qq;
      T val = T(0.f);
      if (qi < S && d < qk) val = Qg[(int64_t)(t0 + qi) * a.ldq + (int64_t)h * qk + d];
      Qs[qq * QROW + d] = val;
      Qt[d * TROW + qq] = val;
    }
    for (int v = tid; v < BT * DV; v += 256) {
      const int qq = v / DV, d = v % DV;
      const int qi = q0 + qq;
      T val = T(0.f);
      if (qi < S && d < a.dv) val = dOg[(int64_t)(t0 + qi) * a.ldo + (int64_t)h * a.dv + d];
      dOs[qq * DOROW + d] = val;
      dOt[d * TROW + qq] = val;
    }
    if (tid < BT) {
      const int qi = q0 + tid;
      float l2 = -INFINITY, dd = 0.f;
      int lo = 0, hi = 0;
      if (qi < S) {
        const int t = t0 + qi;
        l2 = a.lse[(int64_t)t * a.H + h];
        dd = a.D[(int64_t)t * a.H + h];
        visible_rows(a.mask, t, qi, S, lo, hi);
      }
      lse_s[tid] = l2; D_s[tid] = dd; lo_s[tid] = lo; hi_s[tid] = hi;
    }
    __syncthreads();

    // ---- S^T, dP^T -> P^T, dS^T (bf16/fp32 in LDS, this wave's 16 keys)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> qf;
        ld_frag(qf, &Qs[(qb * 16 + lr) * QROW + ks * 32 + g * 8], true);
        s = mfma16(kf[ks], qf, s);
      }
#pragma unroll
      for (int vs = 0; vs < VS; ++vs) {
        Frag<T> of;
        ld_frag(of, &dOs[(qb * 16 + lr) * DOROW + vs * 32 + g * 8], true);
        dp = mfma16(vf[vs], of, dp);
      }
      const int qq = qb * 16 + lr;
      const float l2 = lse_s[qq], dd = D_s[qq];
      const int lo = lo_s[qq], hi = hi_s[qq];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + wave * 16 + g * 4 + i;
        const bool vis = key < S && key >= lo && key < hi;
        const float p = vis ? fast_exp2(s[i] * sl2 - l2) : 0.f;
        Pw[wave][(g * 4 + i) * TROW + qq] = from_f32<T>(p);
        dSw[wave][(g * 4 + i) * TROW + qq] = from_f32<T>(p * (dp[i] - dd));
      }
    }
    __syncthreads();

    // ---- dV += P^T dO, dK += dS^T Q (contraction over the 64 queries)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      Frag<T> pf, sf;
      ld_frag(pf, &Pw[wave][lr * TROW + qs * 32 + g * 8], true);
      ld_frag(sf, &dSw[wave][lr * TROW + qs * 32 + g * 8], true);
#pragma unroll
      for (int db = 0; db < DVB; ++db) {
        Frag<T> bfr;
        ld_frag(bfr, &dOt[(db * 16 + lr) * TROW + qs * 32 + g * 8], true);
        dv[db] = mfma16(pf, bfr, dv[db]);
      }
#pragma unroll
      for (int db = 0; db < DKB; ++db) {
        Frag<T> bfr;
        ld_frag(bfr, &Qt[(db * 16 + lr) * TROW + qs * 32 + g * 8], true);
        dk[db] = mfma16(sf, bfr, dk[db]);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds dK / dV of keys 4 g + i, dim 16 db + lr
  T* dkvb = reinterpret_cast<T*>(a.dkvb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = k0 + wave * 16 + g * 4 + i;
    if (key >= S) continue;
    const int64_t t = t0 + key;
    T* row = dkvb + t * a.lddkvb + (int64_t)h * (a.n + a.dv);
#pragma unroll
    for (int db = 0; db < DKB; ++db) {
      const int d = db * 16 + lr;
      const float v = dk[db][i] * a.scale;
      if (d < a.n) row[d] = from_f32<T>(v);
      else if (d < qk) a.dkr[(t * a.H + h) * a.r + (d - a.n)] = v;
    }
#pragma unroll
    for (int db = 0; db < DVB; ++db) {
      const int d = db * 16 + lr;
      if (d < a.dv) row[a.n + d] = from_f32<T>(dv[db][i]);
    }
  }
}

// ---------------------------------------------------------------------------
// attention backward, queries side: dQ of one 64-query tile of one head.
// Wave w owns queries 16 w .. + 15 (A rows of S = Q K^T and dP = dO V^T; lane
// holds queries 4 g + i, key lr of each 16-key block); dS goes through LDS
// to become the A operand of dQ += dS K, whose B operand reads K^T.
// ---------------------------------------------------------------------------
template <typename T, int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(TrainArgs a) {
  constexpr int BT = 64, KS = DQK / 32, VS = DV / 32, DKB = DQK / 16;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int KROW = DQK + PAD, VROW = DV + PAD, TROW = BT + PAD;
  __shared__ __attribute__((aligned(16))) T Ks[BT * KROW];
  __shared__ __attribute__((aligned(16))) T Kt[DQK * TROW];
  __shared__ __attribute__((aligned(16))) T Vs[BT * VROW];
  __shared__ __attribute__((aligned(16))) T dSw[4][16 * TROW];

  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = seq_len(a, b);
  const int q0 = qt * BT;
  if (q0 >= S) return;
  const int t0 = a.cu_seqlens[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const float sl2 = a.scale * kLog2e;
  const int qk = a.n + a.r;
  const T* Qg = reinterpret_cast<const T*>(a.q);
  const T* dOg = reinterpret_cast<const T*>(a.dO);

  // this wave's queries as A operands (rows lr)
  const int qa = q0 + wave * 16 + lr;
  const bool qaok = qa < S;
  Frag<T> qf[KS], of[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d = ks * 32 + g * 8;
    ld_frag(qf[ks], Qg + (int64_t)(t0 + (qaok ? qa : 0)) * a.ldq + (int64_t)h * qk + d, qaok && d < qk);
  }
#pragma unroll
  for (int vs = 0; vs < VS; ++vs) {
    const int d = vs * 32 + g * 8;
    ld_frag(of[vs], dOg + (int64_t)(t0 + (qaok ? qa : 0)) * a.ldo + (int64_t)h * a.dv + d, qaok && d < a.dv);
  }
  // statistics of the 4 output rows of this lane (queries 4 g + i)
  float l2[4], dd[4];
  int lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = q0 + wave * 16 + g * 4 + i;
    l2[i] = -INFINITY; dd[i] = 0.f; lo[i] = 0; hi[i] = 0;
    if (qi < S) {
      const int t = t0 + qi;
      l2[i] = a.lse[(int64_t)t * a.H + h];
      dd[i] = a.D[(int64_t)t * a.H + h];
      visible_rows(a.mask, t, qi, S, lo[i], hi[i]);
    }
  }
  floatx4 dq[DKB];
#pragma unroll
  for (int i = 0; i < DKB; ++i) dq[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  // keys some query of this tile can see
  int kbeg = 0, kend = S;
  if (a.mask.row_lo == nullptr) {
    if (a.mask.kind == 1) kend = min(S, q0 + BT);
    else if (a.mask.kind == 2) { kend = min(S, q0 + BT); kbeg = max(0, q0 - max(a.mask.window, 0) + 1); }
  }
  kbeg = (kbeg / BT) * BT;

  for (int k0 = kbeg; k0 < kend; k0 += BT) {
    for (int v = tid; v < BT * DQK; v += 256) {
      const int kk = v / DQK, d = v % DQK;
      const int j = k0 + kk;
      const T val = (j < S) ? key_elem<T>(a, b, j, h, d) : T(0.f);
      Ks[kk * KROW + d] = val;
      Kt[d * TROW + kk] = val;
    }
    for (int v = tid; v < BT * DV; v += 256) {
      const int kk = v / DV, d = v % DV;
      const int j = k0 + kk;
      Vs[kk * VROW + d] = (j < S) ? val_elem<T>(a, b, j, h, d) : T(0.f);
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag<T> kfr;
        ld_frag(kfr, &Ks[(kb * 16 + lr) * KROW + ks * 32 + g * 8], true);
        s = mfma16(qf[ks], kfr, s);
      }
#pragma unroll
      for (int vs = 0; vs < VS; ++vs) {
        Frag<T> vfr;
        ld_frag(vfr, &Vs[(kb * 16 + lr) * VROW + vs * 32 + g * 8], true);
        dp = mfma16(of[vs], vfr, dp);
      }
      const int key = k0 + kb * 16 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = key < S && key >= lo[i] && key < hi[i];
        const float p = vis ? fast_exp2(s[i] * sl2 - l2[i]) : 0.f;
        dSw[wave][(g * 4 + i) * TROW + kb * 16 + lr] = from_f32<T>(p * (dp[i] - dd[i]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      Frag<T> sf;
      ld_frag(sf, &dSw[wave][lr * TROW + ks2 * 32 + g * 8], true);
#pragma unroll
      for (int db = 0; db < DKB; ++db) {
        Frag<T> bfr;
        ld_frag(bfr, &Kt[(db * 16 + lr) * TROW + ks2 * 32 + g * 8], true);
        dq[db] = mfma16(sf, bfr, dq[db]);
      }
    }
    __syncthreads();
  }

  T* dQg = reinterpret_cast<T*>(a.dQ);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = q0 + wave * 16 + g * 4 + i;
    if (qi >= S) continue;
    T* row = dQg + (int64_t)(t0 + qi) * a.lddq + (int64_t)h * qk;
#pragma unroll
    for (int db = 0; db < DKB; ++db) {
      const int d = db * 16 + lr;
      if (d < qk) row[d] = from_f32<T>(dq[db][i] * a.scale);
    }
  }
}

// ---------------------------------------------------------------------------
// elementwise and per-token kernels (one workgroup per token)
// ---------------------------------------------------------------------------

// rows of the q_a projection -> RMSNorm(q_a) * gamma (qn) and rho
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const T* x, int64_t ldx, const T* gamma, int N, float eps,
                                                           T* y, int64_t ldy, float* rho, int rows) {
  const int t = blockIdx.x;
  if (t >= rows) return;
  __shared__ float red[4];
  const T* xr = x + (int64_t)t * ldx;
  float ss = 0.f;
  for (int e = threadIdx.x; e < N; e += 256) {
    const float f = to_f32(xr[e]);
    ss += f * f;
  }
  ss = warp_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
  for (int e = threadIdx.x; e < N; e += 256) y[(int64_t)t * ldy + e] = from_f32<T>(to_f32(xr[e]) * r * to_f32(gamma[e]));
  if (threadIdx.x == 0) rho[t] = r;
}

// A = O * sigmoid(gate input)  (or a copy of O without a gate)
template <typename T>
__global__ __launch_bounds__(256) void gate_fwd_kernel(TrainArgs a) {
  const int t = blockIdx.x;
  const int HD = a.H * a.dv;
  const T* O = reinterpret_cast<const T*>(a.O) + (int64_t)t * HD;
  T* A = reinterpret_cast<T*>(a.A) + (int64_t)t * HD;
  const T* gp = a.gate ? reinterpret_cast<const T*>(a.gate) + (int64_t)t * a.ldg : nullptr;
  for (int e = threadIdx.x; e < HD; e += 256) {
    float v = to_f32(O[e]);
    if (gp) v *= sigmoidf(to_f32(gp[e]));
    A[e] = from_f32<T>(v);
  }
}

// dO = dA * sigma (in place), d(gate input) = dA O sigma (1 - sigma) into
// dbuf1, D[t, h] = sum_d dO O
template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(TrainArgs a) {
  const int t = blockIdx.x;
  const int HD = a.H * a.dv;
  T* dA = reinterpret_cast<T*>(a.dO) + (int64_t)t * HD;
  const T* O = reinterpret_cast<const T*>(a.O) + (int64_t)t * HD;
  const T* gp = a.gate ? reinterpret_cast<const T*>(a.gate) + (int64_t)t * a.ldg : nullptr;
  T* dgp = a.gate ? reinterpret_cast<T*>(a.dbuf1) + (int64_t)t * a.lddb1 + a.off_g : nullptr;
  // thread -> (head, 1/64 of its dims): 64 lanes of a wave per head
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < a.H; h += 4) {
    float acc = 0.f;
    for (int d = lane; d < a.dv; d += 64) {
      const int e = h * a.dv + d;
      const float da = to_f32(dA[e]), o = to_f32(O[e]);
      float dov = da;
      if (gp) {
        const float s = sigmoidf(to_f32(gp[e]));
        dov = da * s;
        dgp[e] = from_f32<T>(da * o * s * (1.f - s));
      }
      const T dq = from_f32<T>(dov);
      dA[e] = dq;
      acc += to_f32(dq) * o;
    }
    acc = warp_sum(acc);
    if (lane == 0) a.D[(int64_t)t * a.H + h] = acc;
  }
}

// rotation of pair j at position p by -angle (the adjoint of RoPE)
__device__ __forceinline__ void rope_back(const TrainArgs& a, int p, int j, float xa, float xb, float& ya, float& yb) {
  const float cs = a.rope_cos[(int64_t)p * (a.r / 2) + j], sn = a.rope_sin[(int64_t)p * (a.r / 2) + j];
  ya = xa * cs + xb * sn;
  yb = -xa * sn + xb * cs;
}
__device__ __forceinline__ void rope_idx(const TrainArgs& a, int j, int& ia, int& ib) {
  if (a.interleaved) { ia = 2 * j; ib = 2 * j + 1; }
  else { ia = j; ib = j + a.r / 2; }
}

// latent side, per token: dkv_c = RMSNorm backward of dcn, dk_pe = the rope
// gradient summed over heads and turned back; both into dbuf1 (kv block);
// rho of the latent row into rho_kv
template <typename T>
__global__ __launch_bounds__(256) void kv_bwd_kernel(TrainArgs a) {
  const int t = blockIdx.x;
  if (t >= a.total_tokens) return;
  const int b = seq_of(a, t), p = t - a.cu_seqlens[b];
  __shared__ float red[4], red2[4];
  const T* x = reinterpret_cast<const T*>(a.buf1) + (int64_t)t * a.ldb1 + a.off_kv;
  const T* dy = reinterpret_cast<const T*>(a.dcn) + (int64_t)t * a.c;
  const T* gamma = reinterpret_cast<const T*>(a.gamma_kv);
  T* out = reinterpret_cast<T*>(a.dbuf1) + (int64_t)t * a.lddb1 + a.off_kv;
  float ss = 0.f, gx = 0.f;
  for (int e = threadIdx.x; e < a.c; e += 256) {
    const float f = to_f32(x[e]);
    ss += f * f;
    gx += to_f32(dy[e]) * to_f32(gamma[e]) * f;
  }
  ss = warp_sum(ss);
  gx = warp_sum(gx);
  if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6] = ss; red2[threadIdx.x >> 6] = gx; }
  __syncthreads();
  const float rho = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)a.c + a.eps);
  const float mg = (red2[0] + red2[1] + red2[2] + red2[3]) / (float)a.c;
  for (int e = threadIdx.x; e < a.c; e += 256) {
    const float f = to_f32(x[e]);
    out[e] = from_f32<T>(rho * (to_f32(dy[e]) * to_f32(gamma[e]) - f * rho * rho * mg));
  }
  if (threadIdx.x == 0) a.rho_kv[t] = rho;
  // rope key: sum over heads, then the opposite turn
  for (int j = threadIdx.x; j < a.r / 2; j += 256) {
    int ia, ib;
    rope_idx(a, j, ia, ib);
    float sa = 0.f, sb = 0.f;
    for (int h = 0; h < a.H; ++h) {
      sa += a.dkr[((int64_t)t * a.H + h) * a.r + ia];
      sb += a.dkr[((int64_t)t * a.H + h) * a.r + ib];
    }
    float ya, yb;
    rope_back(a, p, j, sa, sb, ya, yb);
    out[a.c + ia] = from_f32<T>(ya);
    out[a.c + ib] = from_f32<T>(yb);
  }
}

// query side, per token: dq = dQ with its rope part turned back (in place in
// dQ, then also into dbuf1's q block when the query has no low-rank path)
template <typename T>
__global__ __launch_bounds__(256) void q_rope_bwd_kernel(TrainArgs a) {
  const int t = blockIdx.x;
  if (t >= a.total_tokens) return;
  const int b = seq_of(a, t), p = t - a.cu_seqlens[b];
  const int qk = a.n + a.r;
  T* dq = reinterpret_cast<T*>(a.dQ) + (int64_t)t * a.lddq;
  for (int v = threadIdx.x; v < a.H * (a.r / 2); v += 256) {
    const int h = v / (a.r / 2), j = v % (a.r / 2);
    int ia, ib;
    rope_idx(a, j, ia, ib);
    T* row = dq + (int64_t)h * qk + a.n;
    float ya, yb;
    rope_back(a, p, j, to_f32(row[ia]), to_f32(row[ib]), ya, yb);
    row[ia] = from_f32<T>(ya);
    row[ib] = from_f32<T>(yb);
  }
  if (a.q_lora == 0) {
    __syncthreads();
    T* out = reinterpret_cast<T*>(a.dbuf1) + (int64_t)t * a.lddb1 + a.off_q;
    for (int e = threadIdx.x; e < a.H * qk; e += 256) out[e] = dq[e];
  }
}

// low-rank query, per token: dq_a = RMSNorm backward of dqn into dbuf1's q block
template <typename T>
__global__ __launch_bounds__(256) void q_norm_bwd_kernel(TrainArgs a) {
  const int t = blockIdx.x;
  if (t >= a.total_tokens) return;
  __shared__ float red[4];
  const int N = a.q_lora;
  const T* x = reinterpret_cast<const T*>(a.buf1) + (int64_t)t * a.ldb1 + a.off_q;
  const T* dy = reinterpret_cast<const T*>(a.dqn) + (int64_t)t * N;
  const T* gamma = reinterpret_cast<const T*>(a.gamma_q);
  T* out = reinterpret_cast<T*>(a.dbuf1) + (int64_t)t * a.lddb1 + a.off_q;
  const float rho = a.rho_q[t];
  float gx = 0.f;
  for (int e = threadIdx.x; e < N; e += 256) gx += to_f32(dy[e]) * to_f32(gamma[e]) * to_f32(x[e]);
  gx = warp_sum(gx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = gx;
  __syncthreads();
  const float mg = (red[0] + red[1] + red[2] + red[3]) / (float)N;
  for (int e = threadIdx.x; e < N; e += 256) {
    const float f = to_f32(x[e]);
    out[e] = from_f32<T>(rho * (to_f32(dy[e]) * to_f32(gamma[e]) - f * rho * rho * mg));
  }
}

// dgamma partial sums: part[blk][j] = sum over rows of block blk of
// dy[t, j] * x[t, j] * rho[t] (64 columns x 256 rows per workgroup)
template <typename T>
__global__ __launch_bounds__(256) void gamma_partial_kernel(const T* dy, int64_t lddy, const T* x, int64_t ldx,
                                                            const float* rho, int rows, int cols, float* part) {
  const int cb = blockIdx.x, rb = blockIdx.y;
  const int col = cb * 64 + (threadIdx.x & 63), r0 = rb * 256 + (threadIdx.x >> 6) * 64;
  __shared__ float red[4][64];
  float acc = 0.f;
  if (col < cols)
    for (int r = r0; r < min(r0 + 64, rows); ++r)
      acc += to_f32(dy[(int64_t)r * lddy + col]) * to_f32(x[(int64_t)r * ldx + col]) * rho[r];
  red[threadIdx.x >> 6][threadIdx.x & 63] = acc;
  __syncthreads();
  if (threadIdx.x < 64 && col < cols)
    part[(int64_t)rb * cols + col] = red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x] + red[3][threadIdx.x];
}

template <typename T>
__global__ __launch_bounds__(256) void gamma_final_kernel(const float* part, int nparts, int cols, T* out) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= cols) return;
  float acc = 0.f;
  for (int i = 0; i < nparts; ++i) acc += part[(int64_t)i * cols + col];
  out[col] = from_f32<T>(acc);
}

// dst[c][t] = src[row(t)][c] for t < rows, 0 for rows <= t < rows_pad. With
// a row map (cache rows of training tokens), row(t) = b Lp + (t - cu[b]).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, int64_t lds, int rows, int cols, T* dst,
                                                        int64_t ldd, TrainArgs a, int map_rows) {
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int v = threadIdx.x; v < 64 * 64; v += 256) {
    const int rr = v / 64, cc = v % 64;
    const int r = r0 + rr, c = c0 + cc;
    T val = T(0.f);
    if (r < rows && c < cols) {
      int64_t sr = r;
      if (map_rows) {
        const int b = seq_of(a, r);
        sr = (int64_t)b * a.Lp + (r - a.cu_seqlens[b]);
      }
      val = src[sr * lds + c];
    }
    tile[rr][cc] = val;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 64 * 64; v += 256) {
    const int cc = v / 64, rr = v % 64;
    const int r = r0 + rr, c = c0 + cc;
    if (c < cols && r < ldd) dst[(int64_t)c * ldd + r] = tile[rr][cc];
  }
}

// The same for bf16 with 16-byte accesses (rows of src and dst, and both
// pointers, 16-byte aligned): a 64 x 64 tile is loaded as 8-element row
// chunks, and every output chunk gathers 8 tokens of one column from LDS.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* src, int64_t lds, int rows, int cols,
                                                             bf16* dst, int64_t ldd, TrainArgs a, int map_rows) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64][64 + 8];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  for (int v = threadIdx.x; v < 64 * 8; v += 256) {
    const int rr = v >> 3, ch = v & 7;
    const int r = r0 + rr, c = c0 + ch * 8;
    bf16x8 val = {};
    if (r < rows && c < cols) {
      int64_t sr = r;
      if (map_rows) {
        const int b = seq_of(a, r);
        sr = (int64_t)b * a.Lp + (r - a.cu_seqlens[b]);
      }
      const bf16* p = src + sr * lds + c;
      if (c + 8 <= cols) {
        val = *reinterpret_cast<const bf16x8*>(p);
      } else {
        for (int e = 0; e < 8 && c + e < cols; ++e) val[e] = p[e];
      }
    }
    *reinterpret_cast<bf16x8*>(&tile[rr][ch * 8]) = val;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < 64 * 8; v += 256) {
    const int cc = v >> 3, ch = v & 7;
    const int c = c0 + cc, r = r0 + ch * 8;
    if (c >= cols || r >= ldd) continue;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = tile[ch * 8 + e][cc];
    bf16* q = dst + (int64_t)c * ldd + r;
    if (r + 8 <= ldd) {
      *reinterpret_cast<bf16x8*>(q) = o;
    } else {
      for (int e = 0; e < 8 && r + e < ldd; ++e) q[e] = o[e];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 attention backward with register-resident probabilities. In the
// keys-side kernel S = Q K^T is computed with the queries as rows, so the
// accumulator of two 16-query blocks holds, in each lane, the 8 probabilities
// of one key for queries 16 (e / 4) + 4 g + e % 4 -- the B-operand layout of
// dV^T = dO^T P and dK^T = Q^T dS over those 32 queries, whose A operands
// (dO^T, Q^T) come from the row-major query tile through the transposing LDS
// read (ds_read_b64_tr_b16). The queries-side kernel computes S^T = K Q^T
// (keys as rows) and dQ^T = K^T dS^T the same way. Tiles are staged with
// 16-byte loads; no probability or transposed copy goes through LDS.
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

// rows r0 .. r0 + 3 (first read) and r0 + 16 .. r0 + 19 (second) of a
// row-major LDS tile, columns c .. c + 3 of each lane's 16-lane group
// distributed one column per lane: element e of lane (g, lr) is row
// 16 (e / 4) + 4 g + e % 4, column 16 D + lr when the lane points at row
// 4 g + lr / 4, column 16 D + 4 (lr % 4)
__device__ __forceinline__ bf16x8 tr_pair16(const bf16* p0, const bf16* p1) {
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  const v8i16 z = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, z);
}

// Element index of element e of row r in a bf16 tile with NCH 16-byte
// chunks of data per row, padded by 16 elements, chunk bit 0 XOR-ed with row
// bit 3. The LDS serves a 16-byte read 16 lanes at a time and an 8-byte
// (transposing) read 32 lanes at a time; with this layout the 16 rows of a
// fragment read and the 8 rows x 4 column groups of a transposing read both
// land on distinct banks (rows padded by 8 left the transposing reads 2-way
// conflicted), and each read pattern needs one per-lane base address.
template <int NCH>
__device__ __forceinline__ int swz_el(int r, int e) {
  return r * (NCH * 8 + 16) + (((e >> 3) ^ ((r >> 3) & 1)) << 3) + (e & 7);
}

// 8 elements d .. d + 7 (d a multiple of 8) of head h's key of token (b, j)
__device__ __forceinline__ bf16x8 key_vec(const TrainArgs& a, int b, int j, int h, int d) {
  const int64_t row = (int64_t)b * a.Lp + j;
  if (d < a.n) return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.kvexp) + row * a.ldkv +
                                                       (int64_t)h * (a.n + a.dv) + d);
  if (d < a.n + a.r)
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.cache) + row * (a.c + a.r) + a.c + (d - a.n));
  return bf16x8{};
}
__device__ __forceinline__ bf16x8 val_vec(const TrainArgs& a, int b, int j, int h, int d) {
  if (d >= a.dv) return bf16x8{};
  const int64_t row = (int64_t)b * a.Lp + j;
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(a.kvexp) + row * a.ldkv +
                                          (int64_t)h * (a.n + a.dv) + a.n + d);
}

// Workgroup id -> (64-row tile, head, sequence) of the bf16 backward kernels.
// The (sequence, head) pairs go to the 8 XCDs round-robin (a workgroup runs
// on XCD id mod 8): pair p on XCD p mod 8, whose workgroups take all tiles of
// one pair before the next, so that the pair's rows are fetched into one L2
// and re-read from there by every tile. desc: tiles in descending order
// (causal query tiles: the last sees the most keys), else ascending (key
// tiles: the first sees the most queries), heaviest first.
__device__ __forceinline__ bool bwd_tile(const TrainArgs& a, int tiles, bool desc, int& t, int& h, int& b) {
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int p = (slot / tiles) * 8 + xcd, ti = slot % tiles;
  if (p >= a.H * a.batch) return false;
  h = p % a.H;
  b = p / a.H;
  t = desc ? tiles - 1 - ti : ti;
  return true;
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16_kernel(TrainArgs a) {
  constexpr int BT = 64, KS = DQK / 32, VS = DV / 32, DKB = DQK / 16, DVB = DV / 16;
  constexpr int QCH = DQK / 8, OCH = DV / 8;  // 16-byte chunks per row
  static_assert(QCH % 2 == 0 && OCH % 2 == 0, "even chunk counts (chunk bit 0 is swizzled)");
  __shared__ __attribute__((aligned(16))) bf16 Qs[BT * (DQK + 16)];
  __shared__ __attribute__((aligned(16))) bf16 dOs[BT * (DV + 16)];
  __shared__ __attribute__((aligned(16))) float lse_s[BT], D_s[BT];
  __shared__ __attribute__((aligned(16))) int lo_s[BT], hi_s[BT];

  int kt, h, b;
  if (!bwd_tile(a, (a.max_q_len + BT - 1) / BT, false, kt, h, b)) return;
  const int S = seq_len(a, b);
  const int k0 = kt * BT;
  if (k0 >= S) return;
  const int t0 = a.cu_seqlens[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int qa = lr >> 2, qb4 = (lr & 3) * 4;
  const float sl2 = a.scale * kLog2e;
  const int qk = a.n + a.r;

  // this lane's key (column lr of the wave's 16) as B operands
  const int key = k0 + wave * 16 + lr;
  const bool kok = key < S;
  Frag<bf16> kf[KS], vf[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks].v = kok ? key_vec(a, b, key, h, ks * 32 + g * 8) : bf16x8{};
#pragma unroll
  for (int vs = 0; vs < VS; ++vs) vf[vs].v = kok ? val_vec(a, b, key, h, vs * 32 + g * 8) : bf16x8{};
  floatx4 dkt[DKB], dvt[DVB];
#pragma unroll
  for (int i = 0; i < DKB; ++i) dkt[i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < DVB; ++i) dvt[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  int qbeg = 0, qend = S;
  if (a.mask.row_lo == nullptr) {
    if (a.mask.kind == 1) qbeg = k0;
    else if (a.mask.kind == 2) { qbeg = k0; qend = min(S, k0 + BT - 1 + max(a.mask.window, 0)); }
  }
  qbeg = (qbeg / BT) * BT;
  const bf16* Qg = reinterpret_cast<const bf16*>(a.q);
  const bf16* dOg = reinterpret_cast<const bf16*>(a.dO);

  // staging: every load of the tile is issued before the first store (one
  // memory latency per tile, not one per vector)
  constexpr int NQV = BT * (DQK / 8) / 256, NOV = BT * (DV / 8) / 256;
  static_assert(BT * (DQK / 8) % 256 == 0 && BT * (DV / 8) % 256 == 0, "whole staging rounds");
  for (int q0 = qbeg; q0 < qend; q0 += BT) {
    bf16x8 qv[NQV], ov[NOV];
#pragma unroll
    for (int u = 0; u < NQV; ++u) {
      const int v = tid + 256 * u;
      const int qq = v / (DQK / 8), d = (v % (DQK / 8)) * 8;
      const int qi = q0 + qq;
      qv[u] = (qi < S && d < qk) ? *reinterpret_cast<const bf16x8*>(Qg + (int64_t)(t0 + qi) * a.ldq + (int64_t)h * qk + d)
                                 : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NOV; ++u) {
      const int v = tid + 256 * u;
      const int qq = v / (DV / 8), d = (v % (DV / 8)) * 8;
      const int qi = q0 + qq;
      ov[u] = (qi < S && d < a.dv)
                  ? *reinterpret_cast<const bf16x8*>(dOg + (int64_t)(t0 + qi) * a.ldo + (int64_t)h * a.dv + d)
                  : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NQV; ++u) {
      const int v = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&Qs[swz_el<QCH>(v / QCH, (v % QCH) * 8)]) = qv[u];
    }
#pragma unroll
    for (int u = 0; u < NOV; ++u) {
      const int v = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&dOs[swz_el<OCH>(v / OCH, (v % OCH) * 8)]) = ov[u];
    }
    if (tid < BT) {
      const int qi = q0 + tid;
      float l2 = -INFINITY, dd = 0.f;
      int lo = 0, hi = 0;
      if (qi < S) {
        const int t = t0 + qi;
        l2 = a.lse[(int64_t)t * a.H + h];
        dd = a.D[(int64_t)t * a.H + h];
        visible_rows(a.mask, t, qi, S, lo, hi);
      }
      lse_s[tid] = l2; D_s[tid] = dd; lo_s[tid] = lo; hi_s[tid] = hi;
    }
    __syncthreads();

    // S and dP of the four 16-query blocks: sv[qb][i] is query 16 qb + 4 g + i,
    // key lr of the wave. The four blocks' chains are interleaved (k step
    // outer), and every A fragment is read two MFMAs ahead of its use; the
    // fences keep the compiler from moving a read back next to its MFMA.
    constexpr int NSF = 4 * (KS + VS);  // fragment j: Q (ks = j / 4) or dO (vs = j / 4 - KS) of block j % 4
    auto sfrag = [&](int j) -> bf16x8 {
      const int qb = j & 3, st = j >> 2;
      return st < KS ? *reinterpret_cast<const bf16x8*>(&Qs[swz_el<QCH>(qb * 16 + lr, st * 32 + g * 8)])
                     : *reinterpret_cast<const bf16x8*>(&dOs[swz_el<OCH>(qb * 16 + lr, (st - KS) * 32 + g * 8)]);
    };
    floatx4 sv[4], dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) sv[qb] = dp[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      Frag<bf16> fr[3];
      fr[0].v = sfrag(0);
      fr[1].v = sfrag(1);
#pragma unroll
      for (int j = 0; j < NSF; ++j) {
        if (j + 2 < NSF) fr[(j + 2) % 3].v = sfrag(j + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int qb = j & 3, st = j >> 2;
        if (st < KS) sv[qb] = mfma16(fr[j % 3], kf[st], sv[qb]);
        else dp[qb] = mfma16(fr[j % 3], vf[st - KS], dp[qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // probabilities and dS; a lane's four rows 16 qb + 4 g .. + 3 of every
    // row value come in one 16-byte read (branch-free visibility test)
    Frag<bf16> pf[2], sf[2];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const int q4 = qb * 16 + g * 4;
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[q4]);
      const floatx4 d4 = *reinterpret_cast<const floatx4*>(&D_s[q4]);
      const intx4 lo4 = *reinterpret_cast<const intx4*>(&lo_s[q4]);
      const intx4 hi4 = *reinterpret_cast<const intx4*>(&hi_s[q4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = kok & (key >= lo4[i]) & (key < hi4[i]);
        const float p = vis ? fast_exp2(sv[qb][i] * sl2 - l4[i]) : 0.f;
        // B operands of the 32-query halves: element e of lane (g, lr) is
        // query 16 (e / 4) + 4 g + e % 4 of half qb / 2
        pf[qb >> 1].v[(qb & 1) * 4 + i] = (bf16)p;
        sf[qb >> 1].v[(qb & 1) * 4 + i] = (bf16)(p * (dp[qb][i] - d4[i]));
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS over the two 32-query halves: 40
    // transposed A fragments, each read two MFMAs ahead
    constexpr int NTF = 2 * (DVB + DKB);  // fragment x: half x / (DVB + DKB), dO^T block or Q^T block
    auto tfrag = [&](int x) -> bf16x8 {
      const int j = x / (DVB + DKB), d = x % (DVB + DKB);
      const int r0 = 32 * j + 4 * g + qa;
      return d < DVB ? tr_pair16(&dOs[swz_el<OCH>(r0, 16 * d + qb4)], &dOs[swz_el<OCH>(r0 + 16, 16 * d + qb4)])
                     : tr_pair16(&Qs[swz_el<QCH>(r0, 16 * (d - DVB) + qb4)],
                                 &Qs[swz_el<QCH>(r0 + 16, 16 * (d - DVB) + qb4)]);
    };
    {
      Frag<bf16> fr[3];
      fr[0].v = tfrag(0);
      fr[1].v = tfrag(1);
#pragma unroll
      for (int x = 0; x < NTF; ++x) {
        if (x + 2 < NTF) fr[(x + 2) % 3].v = tfrag(x + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int j = x / (DVB + DKB), d = x % (DVB + DKB);
        if (d < DVB) dvt[d] = mfma16(fr[x % 3], pf[j], dvt[d]);
        else dkt[d - DVB] = mfma16(fr[x % 3], sf[j], dkt[d - DVB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }

  // dkt[D][i]: dK of key lr, dim 16 D + 4 g + i (dvt likewise)
  if (!kok) return;
  const int64_t t = t0 + key;
  bf16* row = reinterpret_cast<bf16*>(a.dkvb) + t * a.lddkvb + (int64_t)h * (a.n + a.dv);
#pragma unroll
  for (int D = 0; D < DKB; ++D)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * D + 4 * g + i;
      const float v = dkt[D][i] * a.scale;
      if (d < a.n) row[d] = (bf16)v;
      else if (d < qk) a.dkr[(t * a.H + h) * a.r + (d - a.n)] = v;
    }
#pragma unroll
  for (int D = 0; D < DVB; ++D)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * D + 4 * g + i;
      if (d < a.dv) row[a.n + d] = (bf16)dvt[D][i];
    }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(TrainArgs a) {
  constexpr int BT = 64, KS = DQK / 32, VS = DV / 32, DKB = DQK / 16;
  constexpr int KCH = DQK / 8, VCH = DV / 8;  // 16-byte chunks per row
  static_assert(KCH % 2 == 0 && VCH % 2 == 0, "even chunk counts (chunk bit 0 is swizzled)");
  __shared__ __attribute__((aligned(16))) bf16 Ks[BT * (DQK + 16)];
  __shared__ __attribute__((aligned(16))) bf16 Vs[BT * (DV + 16)];

  int qt, h, b;
  if (!bwd_tile(a, (a.max_q_len + BT - 1) / BT, true, qt, h, b)) return;
  const int S = seq_len(a, b);
  const int q0 = qt * BT;
  if (q0 >= S) return;
  const int t0 = a.cu_seqlens[b];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
  const int qa = lr >> 2, qb4 = (lr & 3) * 4;
  const float sl2 = a.scale * kLog2e;
  const int qk = a.n + a.r;
  const bf16* Qg = reinterpret_cast<const bf16*>(a.q);
  const bf16* dOg = reinterpret_cast<const bf16*>(a.dO);

  // this lane's query (column lr of the wave's 16) as B operands
  const int qi = q0 + wave * 16 + lr;
  const bool qok = qi < S;
  const int t = t0 + (qok ? qi : 0);
  Frag<bf16> qf[KS], of[VS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d = ks * 32 + g * 8;
    qf[ks].v = (qok && d < qk) ? *reinterpret_cast<const bf16x8*>(Qg + (int64_t)t * a.ldq + (int64_t)h * qk + d)
                               : bf16x8{};
  }
#pragma unroll
  for (int vs = 0; vs < VS; ++vs) {
    const int d = vs * 32 + g * 8;
    of[vs].v = (qok && d < a.dv) ? *reinterpret_cast<const bf16x8*>(dOg + (int64_t)t * a.ldo + (int64_t)h * a.dv + d)
                                 : bf16x8{};
  }
  float l2 = -INFINITY, dd = 0.f;
  int lo = 0, hi = 0;
  if (qok) {
    l2 = a.lse[(int64_t)t * a.H + h];
    dd = a.D[(int64_t)t * a.H + h];
    visible_rows(a.mask, t, qi, S, lo, hi);
  }
  floatx4 dqt[DKB];
#pragma unroll
  for (int i = 0; i < DKB; ++i) dqt[i] = floatx4{0.f, 0.f, 0.f, 0.f};

  int kbeg = 0, kend = S;
  if (a.mask.row_lo == nullptr) {
    if (a.mask.kind == 1) kend = min(S, q0 + BT);
    else if (a.mask.kind == 2) { kend = min(S, q0 + BT); kbeg = max(0, q0 - max(a.mask.window, 0) + 1); }
  }
  kbeg = (kbeg / BT) * BT;

  // staging: every load of the tile is issued before the first store
  constexpr int NKV = BT * (DQK / 8) / 256, NVV = BT * (DV / 8) / 256;
  static_assert(BT * (DQK / 8) % 256 == 0 && BT * (DV / 8) % 256 == 0, "whole staging rounds");
  for (int k0 = kbeg; k0 < kend; k0 += BT) {
    bf16x8 kv[NKV], vv[NVV];
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int v = tid + 256 * u;
      const int j = k0 + v / (DQK / 8);
      kv[u] = j < S ? key_vec(a, b, j, h, (v % (DQK / 8)) * 8) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NVV; ++u) {
      const int v = tid + 256 * u;
      const int j = k0 + v / (DV / 8);
      vv[u] = j < S ? val_vec(a, b, j, h, (v % (DV / 8)) * 8) : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int v = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&Ks[swz_el<KCH>(v / KCH, (v % KCH) * 8)]) = kv[u];
    }
#pragma unroll
    for (int u = 0; u < NVV; ++u) {
      const int v = tid + 256 * u;
      *reinterpret_cast<bf16x8*>(&Vs[swz_el<VCH>(v / VCH, (v % VCH) * 8)]) = vv[u];
    }
    __syncthreads();
    // S^T and dP^T of the four 16-key blocks: sv[kb][i] is key 16 kb + 4 g +
    // i, query lr of the wave. The four blocks' chains are interleaved (k step
    // outer), and every A fragment is read two MFMAs ahead of its use; the
    // fences keep the compiler from moving a read back next to its MFMA.
    constexpr int NSF = 4 * (KS + VS);  // fragment j: K (ks = j / 4) or V (vs = j / 4 - KS) of block j % 4
    auto sfrag = [&](int j) -> bf16x8 {
      const int kb = j & 3, st = j >> 2;
      return st < KS ? *reinterpret_cast<const bf16x8*>(&Ks[swz_el<KCH>(kb * 16 + lr, st * 32 + g * 8)])
                     : *reinterpret_cast<const bf16x8*>(&Vs[swz_el<VCH>(kb * 16 + lr, (st - KS) * 32 + g * 8)]);
    };
    floatx4 sv[4], dp[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sv[kb] = dp[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
      Frag<bf16> fr[3];
      fr[0].v = sfrag(0);
      fr[1].v = sfrag(1);
#pragma unroll
      for (int j = 0; j < NSF; ++j) {
        if (j + 2 < NSF) fr[(j + 2) % 3].v = sfrag(j + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = j & 3, st = j >> 2;
        if (st < KS) sv[kb] = mfma16(fr[j % 3], qf[st], sv[kb]);
        else dp[kb] = mfma16(fr[j % 3], of[st - KS], dp[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // dS^T as the B operands of the two 32-key halves: element e of lane
    // (g, lr) is key 16 (e / 4) + 4 g + e % 4 of half kb / 2 (branch-free
    // visibility test)
    Frag<bf16> sf[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + g * 4 + i;
        const bool vis = qok & (key < S) & (key >= lo) & (key < hi);
        const float p = vis ? fast_exp2(sv[kb][i] * sl2 - l2) : 0.f;
        sf[kb >> 1].v[(kb & 1) * 4 + i] = (bf16)(p * (dp[kb][i] - dd));
      }
    // dQ^T += K^T dS^T over the two 32-key halves: 2 DKB transposed A
    // fragments, each read two MFMAs ahead
    constexpr int NTF = 2 * DKB;
    auto tfrag = [&](int x) -> bf16x8 {
      const int j = x / DKB, d = x % DKB;
      const int r0 = 32 * j + 4 * g + qa;
      return tr_pair16(&Ks[swz_el<KCH>(r0, 16 * d + qb4)], &Ks[swz_el<KCH>(r0 + 16, 16 * d + qb4)]);
    };
    {
      Frag<bf16> fr[3];
      fr[0].v = tfrag(0);
      fr[1].v = tfrag(1);
#pragma unroll
      for (int x = 0; x < NTF; ++x) {
        if (x + 2 < NTF) fr[(x + 2) % 3].v = tfrag(x + 2);
        __builtin_amdgcn_sched_barrier(0);
        dqt[x % DKB] = mfma16(fr[x % 3], sf[x / DKB], dqt[x % DKB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }

  if (!qok) return;
  bf16* row = reinterpret_cast<bf16*>(a.dQ) + (int64_t)t * a.lddq + (int64_t)h * qk;
#pragma unroll
  for (int D = 0; D < DKB; ++D)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * D + 4 * g + i;
      if (d < qk) row[d] = (bf16)(dqt[D][i] * a.scale);
    }
}

// dQ of the bf16 backward at n 128, r 64, dv 128 on the 32x32x16 MFMA: a
// workgroup is 8 wavefronts x 32 queries of one (sequence, head) pair (two
// wavefronts per SIMD); 64-key tiles (k_nope and v rows of the expanded
// buffer, the rope key from the cache) stream HBM -> LDS by
// global_load_lds_dwordx4 through a 3-tile ring. Per 32-key block: S^T = K Q^T
// (12 MFMAs, the wavefront's queries as B operands in registers), dP^T = V dO^T
// (8, dO in registers), dS^T = P^T (dP^T - D) in registers, whose accumulator
// elements are, lane for lane, the B operand of dQ^T += K^T dS^T (12, K^T from
// transposing reads). Rows are unpadded with XOR-swizzled 16-byte chunks: the
// 16 rows of a row read and the 4 rows x 32 bytes of a transposing-read pass
// hit distinct banks (k_nope: chunk ^ ((row & 3) << 2 | (row >> 2) & 3), rope
// rows of 8 chunks: chunk ^ (((row >> 1) & 1) << 2 | (row >> 2) & 3), value
// rows, read by rows only: chunk ^ (row & 15)).
namespace bwdq {
constexpr int KT = 64, NW = 8, BQ = NW * 32, NOPE_CH = 16, PE_CH = 8, V_CH = 16, NBUF = 3;
__device__ __forceinline__ int nsw(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int psw(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int nslot(int row, int c) { return row * NOPE_CH + (c ^ nsw(row)); }
__device__ __forceinline__ int pslot(int row, int c) { return row * PE_CH + (c ^ psw(row)); }
__device__ __forceinline__ int vslot(int row, int c) { return row * V_CH + (c ^ (row & 15)); }
}  // namespace bwdq

__global__ __launch_bounds__(512, 1) void attn_bwd_dq_big_kernel(TrainArgs a) {
  using namespace bwdq;
  __shared__ __attribute__((aligned(16))) bf16x8 kn[NBUF][KT * NOPE_CH];
  __shared__ __attribute__((aligned(16))) bf16x8 kp[NBUF][KT * PE_CH];
  __shared__ __attribute__((aligned(16))) bf16x8 vr[NBUF][KT * V_CH];
  __shared__ int iv[4];  // union lo, union hi, intersection lo, intersection hi

  // workgroup id -> (query tile, head, sequence): the pairs go to the XCDs
  // round-robin, heaviest (latest) query tiles first
  const int np = a.H * a.batch, npx = (np + 7) / 8;
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int nqt = (a.max_q_len + BQ - 1) / BQ;
  const int pr = (slot % npx) * 8 + xcd;
  const int qt = nqt - 1 - slot / npx;
  if (pr >= np || qt < 0) return;
  const int h = pr % a.H, b = pr / a.H;
  const int S = seq_len(a, b);
  if (qt * BQ >= S) return;
  const int t0 = a.cu_seqlens[b];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hf = lane >> 5;  // query of the lane, half of the key group
  const int lr = lane & 15, g = lane >> 4, ra = lr >> 2, rb = lr & 3;
  const float sl2 = a.scale * kLog2e;
  const int qk = a.n + a.r;

  if (tid == 0) { iv[0] = 0x7fffffff; iv[1] = 0; iv[2] = 0; iv[3] = 0x7fffffff; }
  __syncthreads();
  const int qi = qt * BQ + wave * 32 + lq;
  const bool qok = qi < S;
  const int tq = t0 + (qok ? qi : 0);
  int lo = 0, hi = 0;
  if (qok) visible_rows(a.mask, tq, qi, S, lo, hi);
  if (hf == 0 && lo < hi) {
    atomicMin(&iv[0], lo);
    atomicMax(&iv[1], hi);
    atomicMax(&iv[2], lo);
    atomicMin(&iv[3], hi);
  }
  if (hf == 0 && qok && lo >= hi) atomicMax(&iv[2], 0x7fffffff);  // an empty row: every tile is masked for it
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

  // B operands: q of step ks = dims 16 ks + 8 hf .. + 7, dO of step s likewise
  bf16x8 qf[12], of[8];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(a.q) + (int64_t)tq * a.ldq + (int64_t)h * qk;
    const bf16* orow = reinterpret_cast<const bf16*>(a.dO) + (int64_t)tq * a.ldo + (int64_t)h * a.dv;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + hf * 8);
      qf[ks] = qok ? v : bf16x8{};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(orow + s * 16 + hf * 8);
      of[s] = qok ? v : bf16x8{};
    }
  }
  const float l2 = qok ? a.lse[(int64_t)tq * a.H + h] : 0.f;
  const float dd = qok ? a.D[(int64_t)tq * a.H + h] : 0.f;

  // copy geometry (as in the forward prefill kernel): 2 k_nope and 2 v
  // instructions of 1 KB per wavefront, 1 rope instruction
  const bf16* kvb = reinterpret_cast<const bf16*>(a.kvexp) + (int64_t)b * a.Lp * a.ldkv + (int64_t)h * (a.n + a.dv);
  const int64_t row_bytes = a.ldkv * 2;
  const int E = a.c + a.r;
  const bf16* crow = reinterpret_cast<const bf16*>(a.cache) + (int64_t)b * a.Lp * E;
  uint32_t noff[2], voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sl = (j * NW + wave) * 64 + lane;
    const int row = sl / NOPE_CH, cs = sl % NOPE_CH;
    noff[j] = (uint32_t)(row * row_bytes) + (uint32_t)((cs ^ nsw(row)) * 16);
    voff[j] = (uint32_t)(row * row_bytes) + (uint32_t)(a.n * 2) + (uint32_t)((cs ^ (row & 15)) * 16);
  }
  uint32_t poff;
  {
    const int sl = wave * 64 + lane;
    const int row = sl / PE_CH, cs = sl % PE_CH;
    poff = (uint32_t)(row * E * 2) + (uint32_t)(a.c * 2) + (uint32_t)((cs ^ psw(row)) * 16);
  }
  const uint32_t kn_lds = lds_addr(&kn[0][0]), vr_lds = lds_addr(&vr[0][0]), kp_lds = lds_addr(&kp[0][0]);
  auto issue = [&](int k0, int buf) {
    // rows past the last key re-read the last key (their probabilities are masked)
    const int rows_valid = min(kend, S) - k0;
    const bf16* base = kvb + (int64_t)k0 * a.ldkv;
    const bf16* pbase = crow + (int64_t)k0 * E;
    const uint32_t nb = kn_lds + (uint32_t)(buf * KT * NOPE_CH * 16);
    const uint32_t vb = vr_lds + (uint32_t)(buf * KT * V_CH * 16);
    const uint32_t pb = kp_lds + (uint32_t)(buf * KT * PE_CH * 16);
    if (rows_valid >= KT) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dma16_sbase(noff[j], base, nb + (uint32_t)(j * NW + wave) * 1024u);
        dma16_sbase(voff[j], base, vb + (uint32_t)(j * NW + wave) * 1024u);
      }
      dma16_sbase(poff, pbase, pb + (uint32_t)wave * 1024u);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = ((j * NW + wave) * 64 + lane) / NOPE_CH;
        const uint32_t back = row >= rows_valid ? (uint32_t)((row - rows_valid + 1) * row_bytes) : 0u;
        dma16_sbase(noff[j] - back, base, nb + (uint32_t)(j * NW + wave) * 1024u);
        dma16_sbase(voff[j] - back, base, vb + (uint32_t)(j * NW + wave) * 1024u);
      }
      const int row = (wave * 64 + lane) / PE_CH;
      const uint32_t back = row >= rows_valid ? (uint32_t)((row - rows_valid + 1) * E * 2) : 0u;
      dma16_sbase(poff - back, pbase, pb + (uint32_t)wave * 1024u);
    }
  };

  // dQ^T block db: element e of lane l is dim 32 db + 8 (e / 4) + 4 hf + e % 4 of query lq
  floatx16 dq[6];
#pragma unroll
  for (int db = 0; db < 6; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
  const bool active = qt * BQ + wave * 32 < S;

  // keys 32 kb .. + 31 of the tile in buffer bf (first key k0)
  auto block = [&](int bf, int kb, int k0, bool edge) {
    const bf16x8* KN = kn[bf];
    const bf16x8* KP = kp[bf];
    const bf16x8* VR = vr[bf];
    // the lane coordinates made opaque here, so that the fragment addresses
    // are computed next to their reads instead of held across the tile loop
    int lq = lane & 31, hf = lane >> 5, g = lane >> 4, ra = (lane & 15) >> 2, rb = lane & 3;
    asm volatile("" : "+v"(lq), "+v"(hf), "+v"(g), "+v"(ra), "+v"(rb));
    floatx16 sc, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = dp[e] = 0.f;
    // S^T (fragments 0..11: key 32 kb + lq, dims 16 j + 8 hf) and dP^T
    // (12..19: value dims 16 (j - 12) + 8 hf), each read two MFMAs ahead
    const int row = kb * 32 + lq;
    auto sfr = [&](int j) -> bf16x8 {
      return j < 8 ? KN[nslot(row, 2 * j + hf)] : (j < 12 ? KP[pslot(row, 2 * (j - 8) + hf)] : VR[vslot(row, 2 * (j - 12) + hf)]);
    };
    bf16x8 fr[3];
    fr[0] = sfr(0);
    fr[1] = sfr(1);
#pragma unroll
    for (int j = 0; j < 20; ++j) {
      if (j + 2 < 20) fr[(j + 2) % 3] = sfr(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (j < 12) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j % 3], qf[j], sc, 0, 0, 0);
      else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[j % 3], of[j - 12], dp, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dS^T = P^T (dP^T - D); element e is key k0 + 32 kb + 8 (e / 4) + 4 hf + e % 4
    bf16x8 dsf[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
      const bool vis = !edge || (qok & (key >= lo) & (key < hi));
      const float p = vis ? fast_exp2(__builtin_fmaf(sc[e], sl2, -l2)) : 0.f;
      dsf[e >> 3][e & 7] = (bf16)(p * (dp[e] - dd));
    }
    // dQ^T += K^T dS^T: fragment x = (half sp = x / 6, dim block db = x % 6);
    // the A operand is read in the key order of the B operand (keys 16 st +
    // 4 hf + (0..3) and + 8): group G of 16 lanes covers dims 32 db + 16 (G &
    // 1) .., lane 4 ra + rb points at key row 16 st + 4 hf + ra (+ 8), dims
    // + 4 rb .. + 3
    auto tfr = [&](int x) -> bf16x8 {
      const int sp = x / 6, db = x % 6, st = 2 * kb + sp;
      const int r0 = st * 16 + hf * 4 + ra;
      int el = db * 32 + (g & 1) * 16 + rb * 4;
      if (db < 4) {
        const int c = el >> 3, half = (el >> 2) & 1;
        return tr_pair16(reinterpret_cast<const bf16*>(&KN[nslot(r0, c)]) + half * 4,
                         reinterpret_cast<const bf16*>(&KN[nslot(r0 + 8, c)]) + half * 4);
      }
      el -= 128;
      const int c = el >> 3, half = (el >> 2) & 1;
      return tr_pair16(reinterpret_cast<const bf16*>(&KP[pslot(r0, c)]) + half * 4,
                       reinterpret_cast<const bf16*>(&KP[pslot(r0 + 8, c)]) + half * 4);
    };
    fr[0] = tfr(0);
    fr[1] = tfr(1);
#pragma unroll
    for (int x = 0; x < 12; ++x) {
      if (x + 2 < 12) fr[(x + 2) % 3] = tfr(x + 2);
      __builtin_amdgcn_sched_barrier(0);
      dq[x % 6] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[x % 3], dsf[x / 6], dq[x % 6], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int ntl = kbeg < kend ? (kend - kbeg + KT - 1) / KT : 0;
  MLA_WAIT_VMCNT(0);  // queries and dO landed: in the loop only tile copies are outstanding
  if (ntl > 0) issue(kbeg, 0);
  if (ntl > 1) issue(kbeg + KT, 1);
  for (int t = 0; t < ntl; ++t) {
    const int k0 = kbeg + t * KT;
    if (t + 1 < ntl) MLA_WAIT_VMCNT(5);  // tile t landed; the copies of tile t + 1 may stay in flight
    else MLA_WAIT_VMCNT(0);
    lds_barrier();  // ... for every wavefront; tile t - 1 is no longer read
    if (t + 2 < ntl) issue(k0 + 2 * KT, (t + 2) % NBUF);
    if (!active || !live(k0)) continue;
    const bool edge = !(k0 >= in_lo && k0 + KT <= in_hi);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) block(t % NBUF, kb, k0, edge);
  }

  // epilogue: lane holds dQ[query lq][32 db + 8 i + 4 hf + (0..3)], times the scale
  if (!qok) return;
  bf16* out = reinterpret_cast<bf16*>(a.dQ) + (int64_t)tq * a.lddq + (int64_t)h * qk;
#pragma unroll
  for (int db = 0; db < 6; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = db * 32 + i * 8 + hf * 4;
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = dq[db][4 * i + j] * a.scale;
      *reinterpret_cast<bf16x4*>(out + d0) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    }
}

template <typename T, int DQK, int DV>
hipError_t launch_attn_bwd(const TrainArgs& a, hipStream_t s) {
  const int tiles = (a.max_q_len + 63) / 64;
  dim3 grid(tiles, a.H, a.batch);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DQK, DV>), grid, dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DQK, DV>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_attn_bwd_bf16(const TrainArgs& a, hipStream_t s) {
  const int tiles = (a.max_q_len + 63) / 64;
  const int npx = (a.H * a.batch + 7) / 8;  // (sequence, head) pairs per XCD
  dim3 grid((unsigned)(8 * npx * tiles));
  hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<DQK, DV>), grid, dim3(256), 0, s, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (DQK == 192 && a.n == 128 && a.r == 64 && a.dv == 128 && a.c % 8 == 0) {
    const int64_t nqt = (a.max_q_len + bwdq::BQ - 1) / bwdq::BQ;
    if (8 * (int64_t)npx * nqt > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_bwd_dq_big_kernel, dim3((unsigned)(8 * npx * nqt)), dim3(64 * bwdq::NW), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<DQK, DV>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_bwd_t(const TrainArgs& a, hipStream_t s) {
  const int qk = a.n + a.r;
  if constexpr (sizeof(T) == 2) {
    // 16-byte staging: every 8-element vector of a key lies in one source
    if (a.n % 8 == 0 && a.r % 8 == 0 && a.dv % 8 == 0) {
      if (qk <= 64 && a.dv <= 64) return launch_attn_bwd_bf16<64, 64>(a, s);
      if (qk <= 192 && a.dv <= 128) return launch_attn_bwd_bf16<192, 128>(a, s);
    }
  }
  if (qk <= 32 && a.dv <= 32) return launch_attn_bwd<T, 32, 32>(a, s);
  if (qk <= 64 && a.dv <= 64) return launch_attn_bwd<T, 64, 64>(a, s);
  if constexpr (sizeof(T) == 2) {
    if (qk <= 192 && a.dv <= 128) return launch_attn_bwd<T, 192, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_all(void (*k)(TrainArgs), int grid, const TrainArgs& a, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

const char* train_check(const TrainArgs& a, bool is_bf16) {
  const int qk = a.n + a.r;
  if (qk > 192 || a.dv > 128) return "backward: head dims above 192 (q/k) or 128 (v) are not supported";
  if (!is_bf16 && (qk > 64 || a.dv > 64)) return "backward: fp32 supports q/k head dims up to 64 and v up to 64";
  if (a.r % 2) return "backward: odd rope dim";
  return nullptr;
}

hipError_t train_rmsnorm_rows(const void* x, int64_t ldx, const void* gamma, int N, float eps, void* y, int64_t ldy,
                              float* rho, int rows, bool is_bf16, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<bf16>, dim3(rows), dim3(256), 0, s, static_cast<const bf16*>(x), ldx,
                       static_cast<const bf16*>(gamma), N, eps, static_cast<bf16*>(y), ldy, rho, rows);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<float>, dim3(rows), dim3(256), 0, s, static_cast<const float*>(x), ldx,
                       static_cast<const float*>(gamma), N, eps, static_cast<float*>(y), ldy, rho, rows);
  return hipGetLastError();
}

hipError_t train_gate_fwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_all<bf16>(gate_fwd_kernel<bf16>, a.total_tokens, a, s)
                 : launch_all<float>(gate_fwd_kernel<float>, a.total_tokens, a, s);
}
hipError_t train_gate_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_all<bf16>(gate_bwd_kernel<bf16>, a.total_tokens, a, s)
                 : launch_all<float>(gate_bwd_kernel<float>, a.total_tokens, a, s);
}
hipError_t train_attn_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  if (a.batch <= 0 || a.max_q_len <= 0) return hipSuccess;
  return is_bf16 ? attn_bwd_t<bf16>(a, s) : attn_bwd_t<float>(a, s);
}
hipError_t train_kv_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_all<bf16>(kv_bwd_kernel<bf16>, a.total_tokens, a, s)
                 : launch_all<float>(kv_bwd_kernel<float>, a.total_tokens, a, s);
}
hipError_t train_q_rope_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_all<bf16>(q_rope_bwd_kernel<bf16>, a.total_tokens, a, s)
                 : launch_all<float>(q_rope_bwd_kernel<float>, a.total_tokens, a, s);
}
hipError_t train_q_norm_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_all<bf16>(q_norm_bwd_kernel<bf16>, a.total_tokens, a, s)
                 : launch_all<float>(q_norm_bwd_kernel<float>, a.total_tokens, a, s);
}

hipError_t train_gamma_grad(const void* dy, int64_t lddy, const void* x, int64_t ldx, const float* rho, int rows,
                            int cols, float* part, void* out, bool is_bf16, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int nparts = (rows + 255) / 256;
  dim3 g1((cols + 63) / 64, nparts);
  if (is_bf16) {
    hipLaunchKernelGGL(gamma_partial_kernel<bf16>, g1, dim3(256), 0, s, static_cast<const bf16*>(dy), lddy,
                       static_cast<const bf16*>(x), ldx, rho, rows, cols, part);
    hipLaunchKernelGGL(gamma_final_kernel<bf16>, dim3((cols + 255) / 256), dim3(256), 0, s, part, nparts, cols,
                       static_cast<bf16*>(out));
  } else {
    hipLaunchKernelGGL(gamma_partial_kernel<float>, g1, dim3(256), 0, s, static_cast<const float*>(dy), lddy,
                       static_cast<const float*>(x), ldx, rho, rows, cols, part);
    hipLaunchKernelGGL(gamma_final_kernel<float>, dim3((cols + 255) / 256), dim3(256), 0, s, part, nparts, cols,
                       static_cast<float*>(out));
  }
  return hipGetLastError();
}

hipError_t train_transpose(const void* src, int64_t lds, int rows, int cols, void* dst, int64_t ldd,
                           const TrainArgs& a, bool map_rows, bool is_bf16, hipStream_t s) {
  if (cols <= 0 || ldd <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (int)((ldd + 63) / 64));
  const bool vec = lds % 8 == 0 && ldd % 8 == 0 && ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
  if (is_bf16 && vec)
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, static_cast<const bf16*>(src), lds, rows, cols,
                       static_cast<bf16*>(dst), ldd, a, (int)map_rows);
  else if (is_bf16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, static_cast<const bf16*>(src), lds, rows, cols,
                       static_cast<bf16*>(dst), ldd, a, (int)map_rows);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(src), lds, rows,
                       cols, static_cast<float*>(dst), ldd, a, (int)map_rows);
  return hipGetLastError();
}

}  // namespace mla
