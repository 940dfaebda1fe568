// Absorbed-form MLA decode attention over the 512 + 64 latent cache, bf16
// (MLA blog: the decode branch, forward_mqa and its split-KV merge).
//
// Work partition (stream-K). The visible key interval [lo, hi) of every
// sequence is cut into 32-key tiles aligned to multiples of 32 (a tile never
// straddles a page, since pages hold a multiple of 32 entries); the tiles of
// all sequences, in sequence order, form one list of T tiles. Workgroup range
// r of R takes tiles [r T / R, (r + 1) T / R), so every workgroup streams the
// same number of cache bytes whatever the length mix. A range cuts at most
// two sequences: a sequence that lies wholly inside one range is finished
// there (normalised latent output written directly); the pieces of a cut
// sequence are written as partial outputs with their log-sum-exp and merged
// by a second kernel with log-sum-exp weights.
//
// Inside a workgroup: 8 wavefronts and all (at most 128) heads, so each
// workgroup reads every tile once from HBM. The score product is split by
// head: wavefront w computes the scores and the online softmax of heads
// 16 w .. 16 w + 15 over all 576 dims, its latent queries held in registers.
// The value product is split by latent dim: wavefront w accumulates
// O^T = C^T P^T for latent dims 64 w .. 64 w + 63 and all heads, reading the
// probabilities of every head block (bf16, 1 KB per block) and the rare
// rescale factors that the other wavefronts shared through LDS. So the
// transposing reads of the values touch each tile byte once per workgroup,
// and the queries (72 VGPRs) plus outputs (128 VGPRs) of a wavefront fit two
// wavefronts per SIMD. Tiles stream from HBM straight into LDS
// (global_load_lds_dwordx4) through a ring of NBUF buffers; the scores read
// 16-byte key-row fragments and the value product reads the same rows through
// the transposing LDS read (ds_read_b64_tr_b16), so the tile is stored once,
// row-major, with a swizzle that keeps both access patterns free of bank
// conflicts.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int KT = 32;              // keys per tile
constexpr int ECH = 72;             // 16-byte chunks per 576-wide bf16 entry
constexpr int SLOTS = KT * ECH;     // 16-byte chunks per tile
constexpr int NW = 8;               // wavefronts per workgroup
constexpr int NT = NW * 64;         // threads per workgroup
constexpr int DMA_N = (SLOTS + NT - 1) / NT;  // DMA instructions per lane per tile (the last one partial)
constexpr int KS = 18;              // 32-dim steps of the score product
constexpr int DB = 32;              // 16-dim blocks of the 512 value dims
constexpr int DBW = DB / NW;        // value blocks of one wavefront (64 latent dims)
constexpr int HBW = NW;             // 16-head blocks of a workgroup (128 heads)
static_assert(HBW == 8, "the rescale flags of the head blocks are read as one 8-byte word");
constexpr int ROWB = ECH * 16;      // bytes per tile row
constexpr float kLog2e = 1.4426950408889634f;
static_assert(SLOTS % 256 == 0 && (SLOTS % NT) % 256 == 0, "tile slots: whole 64-lane DMA instructions");

// Chunk c (16 bytes) of tile row `row` sits at chunk (c & ~7) + ((c & 7) ^ (row & 7))
// of the row (rows are 72 chunks = 1152 bytes). Measured on gfx950 with the
// LDS bank-conflict counter, this XOR keeps both access patterns of the tile
// conflict free: 16-byte score reads (16 rows, one chunk) and transposing
// value reads (4 rows x 2 adjacent chunks per 16 lanes).
__device__ __forceinline__ int swz(int row) { return row & 7; }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// Two transposing LDS reads (4 keys each) concatenated into one 8-element
// MFMA operand: elements 0-3 from byte address p0, 4-7 from p1.
__device__ __forceinline__ bf16x8 tr_pair(const char* p0, const char* p1) {
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p0);
  const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p1);
  const v8i16 z = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, z);
}

// Global -> LDS copy of 16 bytes per lane with a per-lane 64-bit address;
// lane l's bytes land at LDS byte address lds + 16 l.
__device__ __forceinline__ void dma16_v(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}

// Visible keys [lo, hi) of the query of sequence b (its own position L - 1;
// a query block sees every entry of its physical sequence)
__device__ __forceinline__ void visible(const DecodeAttnArgs& a, int b, int& lo, int& hi) {
  const int L = min(max(a.seq_lens[b / a.seq_div], 0), a.max_seq_len);
  lo = a.mask.kind == 2 ? max(0, L - a.mask.window) : 0;
  hi = L;
}
__device__ __forceinline__ int tile_count(int lo, int hi) { return hi > lo ? (hi - 1) / KT - lo / KT + 1 : 0; }

// first tile of range r of R over T tiles
__device__ __forceinline__ int range_start(int r, int R, int T) { return (int)(((int64_t)r * T) / R); }

template <int NBUF>
__global__ __launch_bounds__(NT, 1) void decode_sk_kernel(DecodeAttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16x8 tile[NBUF][SLOTS];
  __shared__ int t_ent[kDecodeMaxTiles];  // first cache entry of the tile, -1: unmapped page
  __shared__ int t_k0[kDecodeMaxTiles];   // key of the tile's row 0
  __shared__ int t_seq[kDecodeMaxTiles];
  __shared__ int t_lo[kDecodeMaxTiles], t_hi[kDecodeMaxTiles];
  __shared__ int t_end[kDecodeMaxTiles];  // end (local index) of the tile's piece
  __shared__ int wsum[NW];
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[HBW][64];  // probabilities of every head block
  __shared__ float abuf[HBW][16];                                // rescale factors of every head
  __shared__ __attribute__((aligned(8))) unsigned char aflag[HBW];  // head block needs a rescale
  __shared__ float mbuf[HBW][16], lbuf[HBW][16];                 // softmax state at a piece's end

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int R = a.ranges;
  // ranges r .. r + R/8 - 1 run on one XCD (workgroup id mod 8): neighbouring
  // ranges share sequences, so their latent queries are read from that L2
  const int id = blockIdx.x;
  const int r = (id & 7) * (R >> 3) + (id >> 3);
  const int B = a.batch;

  // ---- tile list: prefix sum of the per-sequence tile counts (in tile 0's
  // memory, before any copy into it), then this range's tiles
  constexpr int SPT = kDecodeMaxBatch / NT;  // sequences per thread in the scan
  int* tstart = reinterpret_cast<int*>(&tile[0][0]);
  {
    int cnt[SPT], loc = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int b = SPT * tid + i;
      cnt[i] = 0;
      if (b < B) {
        int lo, hi;
        visible(a, b, lo, hi);
        cnt[i] = tile_count(lo, hi);
      }
      loc += cnt[i];
    }
    int incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int ex = incl - loc;
    for (int w = 0; w < wave; ++w) ex += wsum[w];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int b = SPT * tid + i;
      if (b < B) tstart[b] = ex;
      ex += cnt[i];
    }
    if (tid == NT - 1) tstart[B] = ex;
    __syncthreads();
  }
  const int T = tstart[B];
  const int s0 = range_start(r, R, T);
  const int n = min(range_start(r + 1, R, T) - s0, kDecodeMaxTiles);
  if (r == 0)
    for (int b = tid; b <= B; b += NT) a.tstart[b] = tstart[b];
  for (int i = tid; i < n; i += NT) {
    const int gi = s0 + i;
    int lb = 0, ub = B;  // tstart[lb] <= gi < tstart[ub]
    while (ub - lb > 1) {
      const int mid = (lb + ub) >> 1;
      if (tstart[mid] <= gi) lb = mid;
      else ub = mid;
    }
    int lo, hi;
    visible(a, lb, lo, hi);
    const int k0 = (lo / KT + gi - tstart[lb]) * KT;
    const int pg = k0 / a.page;
    const int blk = pg < a.max_blocks ? a.block_table[(int64_t)(lb / a.seq_div) * a.max_blocks + pg] : -1;
    t_ent[i] = (blk >= 0 && blk < a.num_blocks) ? blk * a.page + (k0 - pg * a.page) : -1;
    t_k0[i] = k0;
    t_seq[i] = lb;
    t_lo[i] = lo;
    t_hi[i] = hi;
    t_end[i] = min(n, tstart[lb + 1] - s0);
  }
  __syncthreads();
  if (n <= 0) return;

  // ---- DMA geometry: instruction j of this wavefront fills tile slots
  // [(NW j + wave) 64, +64) (the last instruction only on the first waves);
  // the lane's slot holds chunk c of row `row`. The byte offsets are derived
  // at every issue from an opaque zero, so that they are not hoisted into
  // registers that would stay live across the whole loop.
  const bool last_dma = (DMA_N - 1) * NW * 64 + wave * 64 < SLOTS;  // this wave issues instruction DMA_N - 1
  const char* cache = reinterpret_cast<const char*>(a.cache);
  const uint32_t tile_lds = lds_addr(&tile[0][0]);
  auto slot_offset = [&](int j, uint32_t z) {
    const uint32_t p = min((uint32_t)((j * NW + wave) * 64 + lane) + z, (uint32_t)(SLOTS - 1));
    const uint32_t row = p / ECH, pc = p % ECH;
    const uint32_t c = (pc & ~7u) | ((pc & 7u) ^ (uint32_t)swz((int)row));
    return row * ROWB + c * 16u;
  };

  auto issue = [&](int i, int buf) {
    const int ent = __builtin_amdgcn_readfirstlane(t_ent[i]);
    const int k0 = __builtin_amdgcn_readfirstlane(t_k0[i]);
    const int lo = __builtin_amdgcn_readfirstlane(t_lo[i]);
    const int hi = __builtin_amdgcn_readfirstlane(t_hi[i]);
    const uint32_t dst = tile_lds + (uint32_t)buf * (SLOTS * 16) + (uint32_t)wave * 1024u;
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    if (ent >= 0 && k0 >= lo && k0 + KT <= hi) {
      const char* base = cache + (int64_t)ent * ROWB;
#pragma unroll
      for (int j = 0; j < DMA_N; ++j)
        if (j < DMA_N - 1 || last_dma) dma16_sbase(slot_offset(j, z), base, dst + (uint32_t)j * (NW * 1024u));
    } else {
      // edge tile: rows outside [lo, hi) and unmapped pages read the zero page
      const char* base = cache + (int64_t)(ent < 0 ? 0 : ent) * ROWB;
#pragma unroll
      for (int j = 0; j < DMA_N; ++j) {
        if (j == DMA_N - 1 && !last_dma) continue;
        const uint32_t off = slot_offset(j, z);
        const int key = k0 + (int)(off / ROWB);
        const bool ok = ent >= 0 && key >= lo && key < hi;
        const void* src = ok ? (const void*)(base + off) : (const void*)a.zeros;
        dma16_v(src, dst + (uint32_t)j * (NW * 1024u));
      }
    }
  };

  // ---- per-lane LDS read bases (bytes). Scores: rows lr and 16 + lr, chunk
  // 4 s + g. Values (transposing reads) of this wavefront's 64 latent dims:
  // lane k = 4 qa + qb of its 16-lane group points at rows 4 g + qa (and
  // 16 + 4 g + qa), dims 64 wave + 16 d + 4 qb .. + 3.
  int kbase[2], vrow, vx;
#pragma unroll
  for (int x = 0; x < 2; ++x) kbase[x] = (lr * ECH + ((4 * x + g) ^ swz(lr))) * 16;
  {
    // chunk 8 wave + (2 d + (qb >> 1)) of the row, the low 3 bits XOR-ed with swz(row)
    const int qa = lr >> 2, qb = lr & 3;
    const int row = 4 * g + qa;
    vrow = (row * ECH + 8 * wave) * 16 + (qb & 1) * 8;
    vx = (qb >> 1) ^ swz(row);
  }

  const int h = wave * 16 + lr;  // head of this lane's scores and softmax
  const bool hok = h < a.H;
  const float sl2 = a.scale * kLog2e;

  // ---- ring: tiles i + 1 .. i + NBUF - 1 are in flight while tile i is used
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < n) issue(i, i);
  int i = 0;
  while (i < n) {
    // ---- one piece: the consecutive tiles [i, iend) of sequence b
    const int b = __builtin_amdgcn_readfirstlane(t_seq[i]);
    const int iend = __builtin_amdgcn_readfirstlane(t_end[i]);
    const int lo = __builtin_amdgcn_readfirstlane(t_lo[i]);
    const int hi = __builtin_amdgcn_readfirstlane(t_hi[i]);
    const bool piece_start = __builtin_amdgcn_readfirstlane(t_k0[i]) == (lo / KT) * KT;

    // latent query of head h: B operand of S^T, dims 32 s + 8 g .. + 7
    Frag<bf16> q[KS];
    {
      const bf16* ql = reinterpret_cast<const bf16*>(a.ql) + (int64_t)b * a.ldql + (int64_t)(hok ? h : 0) * a.c;
      // roped query: token and head of the (query, head) pair in query blocks
      int64_t qt = b, qh = hok ? h : 0;
      if (a.Hr > 0) {
        const int64_t pair = (int64_t)b * a.H + qh;
        qt = pair / a.Hr;
        qh = pair % a.Hr;
      }
      const bf16* qp = reinterpret_cast<const bf16*>(a.q) + qt * a.ldq + qh * a.qk_head + a.n;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int e = s * 32 + g * 8;
        const bf16* src = !hok ? a.zeros : (s < 16 ? ql + e : qp + (e - 512));
        q[s].v = *reinterpret_cast<const bf16x8*>(src);
      }
    }
    // the queries, and the outputs stored by the previous piece (stores may
    // complete out of order with loads): wait for everything
    MLA_WAIT_VMCNT(0);
    // O^T blocks: latent dims 64 wave + 16 d + 4 g + {0..3}, head 16 hb + lr
    floatx4 o[DBW][HBW];
#pragma unroll
    for (int d = 0; d < DBW; ++d)
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) o[d][hb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (; i < iend; ++i) {
      const int buf = i % NBUF;
      const int later = min(NBUF - 2, n - 1 - i);  // tiles after i already issued
      if (later <= 0) MLA_WAIT_VMCNT(0);
      else if (later == 1) { if (last_dma) MLA_WAIT_VMCNT(DMA_N); else MLA_WAIT_VMCNT(DMA_N - 1); }
      else { if (last_dma) MLA_WAIT_VMCNT(2 * DMA_N); else MLA_WAIT_VMCNT(2 * DMA_N - 2); }
      lds_barrier();  // tile i is in LDS for every wavefront; tile i - 1 and the shared probabilities are no longer read
      if (i + NBUF - 1 < n) issue(i + NBUF - 1, (i + NBUF - 1) % NBUF);
      const int k0 = __builtin_amdgcn_readfirstlane(t_k0[i]);
      const char* Tb = reinterpret_cast<const char*>(&tile[buf][0]);

      // ---- S^T (32 keys x the 16 heads of this wavefront) = C q^T over the 576 dims
      floatx4 sc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        Frag<bf16> k0f, k1f;
        const char* p = Tb + kbase[s & 1] + (s >> 1) * 128;
        k0f.v = *reinterpret_cast<const bf16x8*>(p);
        k1f.v = *reinterpret_cast<const bf16x8*>(p + 16 * ROWB);
        sc[0] = mfma16(k0f, q[s], sc[0]);
        sc[1] = mfma16(k1f, q[s], sc[1]);
      }

      // ---- online softmax of head h (log2 domain); lane holds keys 16 kb + 4 g + e
      const bool edge = k0 < lo || k0 + KT > hi;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = sc[kb][e] * sl2;
          if (edge) {
            const int key = k0 + kb * 16 + g * 4 + e;
            if (key < lo || key >= hi) x = -INFINITY;
          }
          sc[kb][e] = x;
          mx = fmaxf(mx, x);
        }
      mx = red4_max(mx);
      // lazy rescaling: the reference max moves only when exceeded by more
      // than 2^8 (probabilities stay <= 256; exact after the division by l)
      const float mnew = (mx > m + 8.f) ? mx : m;
      const float alpha = m == -INFINITY ? 1.f : fast_exp2(m - mnew);
      Frag<bf16> pf;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = fast_exp2(sc[kb][e] - mnew);
          sum += pv;
          pf.v[kb * 4 + e] = (bf16)pv;
        }
      l = l * alpha + sum;
      m = mnew;
      // share the probabilities (the B operand of head block `wave`) and the
      // rescale factors with the wavefronts that own the other latent dims
      pbuf[wave][lane] = pf.v;
      const bool resc = __any(alpha != 1.f);
      if (resc && g == 0) abuf[wave][lr] = alpha;
      if (lane == 0) aflag[wave] = resc ? 1 : 0;
      lds_barrier();

      // ---- O^T (this wavefront's 64 latent dims x 128 heads) += C^T P^T;
      // operand element e of lane (g, lr) is key 16 (e / 4) + 4 g + e % 4,
      // the order the scores came in
      // one 8-byte read of all the rescale flags (rare: lazy rescaling)
      const uint64_t flags = *reinterpret_cast<const uint64_t*>(aflag);
      if (__builtin_amdgcn_readfirstlane((uint32_t)flags) | __builtin_amdgcn_readfirstlane((uint32_t)(flags >> 32))) {
#pragma unroll
        for (int hb = 0; hb < HBW; ++hb) {
          if ((flags >> (8 * hb)) & 0xff) {
            const float al = abuf[hb][lr];
#pragma unroll
            for (int d = 0; d < DBW; ++d) o[d][hb] *= al;
          }
        }
      }
      Frag<bf16> vf[DBW];
#pragma unroll
      for (int d = 0; d < DBW; ++d) {
        const char* p = Tb + vrow + ((2 * d) ^ vx) * 16;
        vf[d].v = tr_pair(p, p + 16 * ROWB);
      }
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) {
        Frag<bf16> ph;
        ph.v = pbuf[hb][lane];
#pragma unroll
        for (int d = 0; d < DBW; ++d) o[d][hb] = mfma16(vf[d], ph, o[d][hb]);
      }
    }

    // ---- finish this piece of sequence b: whole sequence -> normalised latent
    // output; a cut piece -> partial output + log-sum-exp in slot 1 (piece
    // starts the sequence, range ends inside it) or slot 0 (the range starts
    // inside the sequence). Each head's softmax state comes from the
    // wavefront that owns its scores.
    {
      const float lsum = red4_sum(l);
      if (g == 0) {
        mbuf[wave][lr] = m;
        lbuf[wave][lr] = lsum;
      }
      lds_barrier();
      const int klast = __builtin_amdgcn_readfirstlane(t_k0[iend - 1]);
      const bool whole = piece_start && klast + KT >= hi;
      const int64_t slot = 2 * (int64_t)r + (piece_start ? 1 : 0);
#pragma unroll
      for (int hb = 0; hb < HBW; ++hb) {
        const int hh = hb * 16 + lr;
        if (hh >= a.H) continue;
        const float inv = 1.f / lbuf[hb][lr];
        if (whole) {
          bf16* dst = reinterpret_cast<bf16*>(a.o_lat) + ((int64_t)b * a.H + hh) * a.c + wave * 64 + g * 4;
#pragma unroll
          for (int d = 0; d < DBW; ++d) {
            const floatx4 v = o[d][hb] * inv;
            *reinterpret_cast<bf16x4*>(dst + d * 16) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
          }
        } else {
          // partial output, normalised by its own sum, stored as bf16 (the
          // merged latent output is rounded to bf16 in any case)
          bf16* dst = reinterpret_cast<bf16*>(a.part_o) + (slot * a.H + hh) * a.c + wave * 64 + g * 4;
#pragma unroll
          for (int d = 0; d < DBW; ++d) {
            const floatx4 v = o[d][hb] * inv;
            *reinterpret_cast<bf16x4*>(dst + d * 16) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
          }
        }
      }
      if (!whole && g == 0 && hok) a.part_lse[slot * a.H + h] = m + __log2f(lsum);
    }
  }
}

// o_lat of the sequences that were cut between ranges: log-sum-exp weighted
// sum of the pieces' normalised outputs; sequences with no visible key get 0.
// Tile-to-range arithmetic in double: exact for the integer sizes involved.
__device__ __forceinline__ int range_start_d(int r, int R, int T) { return (int)floor((double)r * T / R); }

__global__ __launch_bounds__(256) void decode_sk_merge_kernel(DecodeAttnArgs a) {
  const int b = blockIdx.y;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t = threadIdx.x & 63;  // dims 8 t .. 8 t + 7
  if (h >= a.H) return;
  const int R = a.ranges;
  const int T = a.tstart[a.batch], ts = a.tstart[b], te = a.tstart[b + 1];
  bf16* dst = reinterpret_cast<bf16*>(a.o_lat) + ((int64_t)b * a.H + h) * a.c + t * 8;
  if (ts >= te) {
    *reinterpret_cast<bf16x8*>(dst) = bf16x8{};
    return;
  }
  // range holding tile x: the largest g with range_start(g) <= x
  auto range_of = [&](int x) { return (int)ceil((double)(x + 1) * R / T) - 1; };
  const int gs = range_of(ts), ge = range_of(te - 1);
  if (gs == ge) return;  // finished inside one range
  const bf16* po = reinterpret_cast<const bf16*>(a.part_o);
  float mx = -INFINITY;
  for (int gg = gs; gg <= ge; ++gg) {
    if (gg > gs && range_start_d(gg + 1, R, T) == range_start_d(gg, R, T)) continue;  // empty range
    const int64_t slot = 2 * (int64_t)gg + (gg == gs ? 1 : 0);
    mx = fmaxf(mx, a.part_lse[slot * a.H + h]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int gg = gs; gg <= ge; ++gg) {
    if (gg > gs && range_start_d(gg + 1, R, T) == range_start_d(gg, R, T)) continue;
    const int64_t slot = 2 * (int64_t)gg + (gg == gs ? 1 : 0);
    const float w = fast_exp2(a.part_lse[slot * a.H + h] - mx);
    den += w;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(po + (slot * a.H + h) * a.c + t * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[e];
  }
  const float inv = 1.f / den;
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x8*>(dst) = v;
}

}  // namespace

const char* decode_sk_check(const DecodeAttnArgs& a) {
  if (a.c != 512 || a.r != 64) return "stream-K decode: the latent must be 512 + 64 wide";
  if (a.H <= 0 || a.H > 128) return "stream-K decode: at most 128 heads";
  if (a.page % KT) return "stream-K decode: page size must be a multiple of 32";
  if (a.batch > kDecodeMaxBatch) return "stream-K decode: batch above 1024";
  if ((int64_t)a.num_blocks * a.page >= ((int64_t)1 << 31)) return "stream-K decode: cache above 2^31 entries";
  if (a.ldql % 8 || a.ldq % 8 || a.qk_head % 8 || a.n % 8) return "stream-K decode: query strides must be 16-byte multiples";
  if (a.seq_div < 1 || a.Hr < 0) return "stream-K decode: bad query-block mapping";
  if (a.ranges <= 0 || a.ranges % 8 || !a.tstart || !a.part_o || !a.part_lse || !a.zeros)
    return "stream-K decode: ranges (a multiple of 8) and workspaces are required";
  return nullptr;
}

int decode_sk_ranges(int batch, int max_visible, int cus) {
  // one workgroup per range: cus ranges fill the device once
  const int64_t tiles_upper = (int64_t)batch * ((max_visible + KT - 1) / KT + 1);
  int64_t r = std::max<int64_t>(std::max(cus, 8), (tiles_upper + kDecodeMaxTiles - 1) / kDecodeMaxTiles);
  r = (r + 7) / 8 * 8;
  return (int)r;
}

hipError_t decode_sk_launch(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_sk_kernel<3>, dim3(a.ranges), dim3(NT), 0, s, a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t decode_sk_merge_launch(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_sk_merge_kernel, dim3((a.H + 3) / 4, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
