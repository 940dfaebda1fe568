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
// workgroup reads every tile once from HBM. Tiles stream from HBM straight
// into LDS (global_load_lds_dwordx4) through a ring of NBUF buffers, stored
// once, row-major, with a swizzle that keeps both access patterns below free
// of bank conflicts. The wavefronts have two roles:
//  * score wavefront s (0..3) computes S^T (32 keys x 32 heads, heads
//    32 s .. 32 s + 31) with the 32x32x16 MFMA: its latent queries (144
//    VGPRs) are the B operand, and each 16-byte key fragment read from LDS
//    serves 32 heads, half the LDS traffic of 16-head wavefronts. It runs the
//    online softmax (one lane swap per row reduction) and publishes the bf16
//    probabilities and the rare rescale factors in LDS;
//  * every wavefront accumulates O^T = C^T P^T for its share of the 512
//    latent dims over all heads, the value operand read through the
//    transposing LDS read (ds_read_b64_tr_b16): a value wavefront holds 52
//    16x16 blocks, a score wavefront 12 next to its queries.
// Step t: the score wavefronts score tile t while all wavefronts multiply
// tile t - 1 by its probabilities (double-buffered by tile parity), so the
// MFMA pipe of each SIMD (score wavefront s and value wavefront s + 4) is fed
// by both, and a step ends on one barrier. The two roles are compiled as two
// copies of the piece loop, so each has its own register allocation.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int KT = 32;              // keys per tile
constexpr int ECH = 72;             // 16-byte chunks per 576-wide bf16 entry
constexpr int SLOTS = KT * ECH;     // 16-byte chunks per tile
constexpr int NW = 8;               // wavefronts per workgroup
constexpr int NT = NW * 64;         // threads per workgroup
constexpr int DMA_N = (SLOTS + NT - 1) / NT;  // copy instructions per lane per tile (the last one partial)
static_assert(SLOTS % 256 == 0 && (SLOTS % NT) % 256 == 0, "tile slots: whole 64-lane copy instructions");
constexpr int KS2 = 36;             // 16-dim steps of the score product (32x32x16 MFMA)
constexpr int HB = 8;               // 16-head blocks of a workgroup (128 heads)
static_assert(HB == 8, "the rescale flags of the head blocks are read as one 8-byte word");
constexpr int ROWB = ECH * 16;      // bytes per tile row
constexpr float kLog2e = 1.4426950408889634f;
static_assert(SLOTS % 256 == 0 && (SLOTS % NT) % 256 == 0, "tile slots: whole 64-lane DMA instructions");
// 8-bit cache: a tile is copied as 36 chunks of 16 codes per row into a ring
// of staging buffers, where both products read the codes and widen them to
// bf16 in registers
constexpr int ECH8 = 36;
constexpr int SLOTS8 = KT * ECH8;
constexpr int DMA_N8 = (SLOTS8 + NT - 1) / NT;
static_assert(SLOTS8 % 64 == 0 && ECH8 * 16 == ROWB / 2, "8-bit tile: whole 64-lane copy instructions");

// Staged 8-bit tile: chunk c (16 codes) of row `row` sits in slot
// 36 row + (c ^ swz8(row)) (the XOR stays inside an aligned group of 4 chunks).
// Rows are 576 bytes (16 row mod 64 banks), so the 16 rows that one 16-byte
// read serves at a time land on distinct banks, as do the 8 rows x 2 halves
// of a chunk that 16 lanes of an 8-byte transposing read take.
__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 3; }

// Chunk c (16 bytes) of tile row `row` sits at chunk (c & ~7) + ((c & 7) ^ swz(row))
// of the row (rows are 72 chunks = 1152 bytes, so rows r and r + 2 start on
// the same banks). The low bit of the XOR also takes bit 3 of the row: the
// 32-row score reads then put rows r and r + 8 on different banks.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
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
// a query block sees every entry of its physical sequence; a sparse list is
// its gather_k listed keys)
template <bool GATHER>
__device__ __forceinline__ void visible(const DecodeAttnArgs& a, int b, int& lo, int& hi) {
  if constexpr (GATHER) {
    lo = 0;
    hi = a.gather_k;
    return;
  }
  const int64_t len = (int64_t)a.seq_lens[b / a.seq_div] + a.len_add;
  const int L = (int)min(max(len, (int64_t)0), (int64_t)a.max_seq_len);
  lo = a.mask.kind == 2 ? max(0, L - a.mask.window) : 0;
  hi = L;
}
__device__ __forceinline__ int tile_count(int lo, int hi) { return hi > lo ? (hi - 1) / KT - lo / KT + 1 : 0; }

// first tile of range r of R over T tiles
__device__ __forceinline__ int range_start(int r, int R, int T) { return (int)(((int64_t)r * T) / R); }

// O^T blocks (16 latent dims x 16 heads) held by one wavefront, as slots j
// of 16 dims D(j) over a range of head blocks; reg(j, hb) is the index of the
// block in the wavefront's register array (-1: not held). Score wavefront s
// holds dims 16 (28 + s) .. for all heads and 16 (24 + s) .. for heads 0-63
// (12 blocks after its 36 query registers); value wavefront v holds dims
// 96 v .. 96 v + 95 for all heads and 16 (24 + v) .. for heads 64-127 (52
// blocks). Value wavefronts multiply in two passes (4 + 3 slots) so that at
// most 4 value operands are live.
template <bool S> struct Blocks;
template <> struct Blocks<true> {
  static constexpr int NREG = 48, NSLOT = 2, NPASS = 1;
  static constexpr int first(int) { return 0; }
  static constexpr int last(int) { return 2; }
  __device__ static int D(int j, int w) { return j == 0 ? 28 + w : 24 + w; }
  static constexpr int reg(int j, int hb) { return j == 0 ? 36 + hb : (hb < 4 ? 44 + hb : -1); }
};
template <> struct Blocks<false> {
  static constexpr int NREG = 52, NSLOT = 7, NPASS = 2;
  static constexpr int first(int p) { return p == 0 ? 0 : 4; }
  static constexpr int last(int p) { return p == 0 ? 4 : 7; }
  __device__ static int D(int j, int v) { return j < 6 ? 6 * v + j : 24 + v; }
  static constexpr int reg(int j, int hb) { return j < 6 ? 8 * j + hb : (hb >= 4 ? 44 + hb : -1); }
};

// GATHER: sparse lists (a.gather_ent), compiled separately so that the
// contiguous-range kernel carries none of its registers
// FP8: 8-bit cache. The codes of tile t stay in staging buffer t % 3, where
// both products read them (16-byte reads for the scores, 8-bit transposing
// reads for the values) and widen them to bf16 in registers; no bf16 ring.
template <int NBUF, bool GATHER, bool FP8>
__global__ __launch_bounds__(NT, 1) void decode_sk_kernel(DecodeAttnArgs a) {
  constexpr int NSTAGE = FP8 ? 3 : 1;
  __shared__ __attribute__((aligned(16))) bf16x8 tile[FP8 ? 1 : NBUF][FP8 ? 1 : SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 stage8[NSTAGE][FP8 ? SLOTS8 : 1];
  __shared__ int t_ent[kDecodeMaxTiles];  // first cache entry of the tile, -1: unmapped page
  __shared__ int t_k0[kDecodeMaxTiles];   // key of the tile's row 0
  __shared__ int t_seq[kDecodeMaxTiles];
  __shared__ int t_lo[kDecodeMaxTiles], t_hi[kDecodeMaxTiles];
  __shared__ int t_end[kDecodeMaxTiles];  // end (local index) of the tile's piece
  __shared__ int wsum[NW];
  // probabilities of tile t in buffer t & 1, as the B operands of the value
  // product: head block hb, lane (g, lr) -> 8 bf16 of head 16 hb + lr, keys
  // 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3
  __shared__ __attribute__((aligned(16))) bf16x8 pbuf[2][HB][64];
  __shared__ float abuf[2][HB * 16];                                // rescale factor of every head
  __shared__ __attribute__((aligned(8))) unsigned char aflag[2][HB];  // head block needs a rescale
  __shared__ float lbuf[HB * 16];                                   // softmax normaliser at a piece's end

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = a.ranges;
  // ranges r .. r + R/8 - 1 run on one XCD (workgroup id mod 8): neighbouring
  // ranges share sequences, so their latent queries are read from that L2
  const int id = blockIdx.x;
  const int r = (id & 7) * (R >> 3) + (id >> 3);
  const int B = a.batch;

  // ---- tile list: prefix sum of the per-sequence tile counts (in tile 0's
  // memory, before any copy into it), then this range's tiles
  constexpr int SPT = kDecodeMaxBatch / NT;  // sequences per thread in the scan
  int* tstart = FP8 ? reinterpret_cast<int*>(&stage8[0][0]) : reinterpret_cast<int*>(&tile[0][0]);
  {
    int cnt[SPT], loc = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int b = SPT * tid + i;
      cnt[i] = 0;
      if (b < B) {
        int lo, hi;
        visible<GATHER>(a, b, lo, hi);
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
    visible<GATHER>(a, lb, lo, hi);
    const int k0 = (lo / KT + gi - tstart[lb]) * KT;
    if constexpr (GATHER) {
      t_ent[i] = lb * a.gather_k + k0;  // the tile's row 0 in the sparse lists
    } else {
      const int pg = k0 / a.page;
      const int blk = pg < a.max_blocks ? a.block_table[(int64_t)(lb / a.seq_div) * a.max_blocks + pg] : -1;
      t_ent[i] = (blk >= 0 && blk < a.num_blocks) ? blk * a.page + (k0 - pg * a.page) : -1;
    }
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

  // ---- sparse lists: lane l holds the cache entry of row l % 32 of a tile
  // (-1: no key), loaded one step before the tile's copies are issued, so
  // that the issue never waits for it; its ballot is the tile's row mask
  constexpr bool gather = GATHER;
  const int gather_rows = a.num_blocks * a.page;
  auto gather_load = [&](int t) {
    int e = -1;
    if (gather && t < n) {
      const int row = lane & 31;
      if (t_k0[t] + row < t_hi[t]) e = a.gather_ent[t_ent[t] + row];
      if (e >= gather_rows) e = -1;
    }
    return e;
  };

  // 8-bit cache: instruction j of this wavefront fills staging slots
  // [(NW j + wave) 64, +64) of buffer `buf`; slot p holds chunk
  // (p % 36) ^ swz8(p / 36) of row p / 36
  const bool last_dma8 = (DMA_N8 - 1) * NW * 64 + wave * 64 < SLOTS8;
  const uint32_t stage_lds = lds_addr(&stage8[0][0]);
  auto issue8 = [&](int buf, int ent, int k0, int lo, int hi, int ev) {
    const uint8_t* cache8 = reinterpret_cast<const uint8_t*>(a.cache);
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    const bool inner = !gather && ent >= 0 && k0 >= lo && k0 + KT <= hi;
#pragma unroll
    for (int j = 0; j < DMA_N8; ++j) {
      if (j == DMA_N8 - 1 && !last_dma8) continue;
      const int pidx = (j * NW + wave) * 64 + lane + (int)z;
      const int row = pidx / ECH8;
      const int c = (pidx - row * ECH8) ^ swz8(row);  // source chunk of the slot
      const void* src;
      if (gather) {
        const int e = __shfl(ev, row);
        src = e >= 0 ? (const void*)(cache8 + (int64_t)e * (ECH8 * 16) + c * 16) : (const void*)a.zeros;
      } else {
        const int key = k0 + row;
        const bool ok = inner || (ent >= 0 && key >= lo && key < hi);
        src = ok ? (const void*)(cache8 + ((int64_t)ent + row) * (ECH8 * 16) + c * 16) : (const void*)a.zeros;
      }
      dma16_v(src, stage_lds + (uint32_t)buf * (SLOTS8 * 16) + (uint32_t)(j * NW + wave) * 1024u);
    }
  };
  // 8 codes (two dwords) -> one bf16 operand (exact: every E4M3 value is a
  // bf16 value)
  auto widen8x8 = [](uint32_t x, uint32_t y) __attribute__((always_inline)) {
    const auto d0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
    const auto d1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
    const auto d2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, false);
    const auto d3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, true);
    return bf16x8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
  };
  // ev: the gathered entries of tile i (sparse lists only)
  auto issue = [&](int i, int ev) {
    const int ent = __builtin_amdgcn_readfirstlane(t_ent[i]);
    const int k0 = __builtin_amdgcn_readfirstlane(t_k0[i]);
    const int lo = __builtin_amdgcn_readfirstlane(t_lo[i]);
    const int hi = __builtin_amdgcn_readfirstlane(t_hi[i]);
    if constexpr (FP8) {
      issue8(i % NSTAGE, ent, k0, lo, hi, ev);
      return;
    }
    const int buf = i % NBUF;
    const uint32_t dst = tile_lds + (uint32_t)buf * (SLOTS * 16) + (uint32_t)wave * 1024u;
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    if (gather) {
      // every row its own entry; rows without a key read the zero page
#pragma unroll
      for (int j = 0; j < DMA_N; ++j) {
        if (j == DMA_N - 1 && !last_dma) continue;
        const uint32_t off = slot_offset(j, z);
        const int row = (int)(off / ROWB);
        const int e = __shfl(ev, row);
        const void* src = e >= 0 ? (const void*)(cache + (int64_t)e * ROWB + (off - (uint32_t)row * ROWB))
                                 : (const void*)a.zeros;
        dma16_v(src, dst + (uint32_t)j * (NW * 1024u));
      }
    } else if (ent >= 0 && k0 >= lo && k0 + KT <= hi) {
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

  // ---- roles: wavefronts 0-3 score (heads 32 wave .. + 31), wavefronts
  // 4-7 only multiply; wavefronts w and w + 4 share a SIMD. The O^T blocks of
  // each role are listed in Blocks<>; a score wavefront keeps its queries in
  // RG[0..35] of its register array.
  const bool sw = wave < 4;
  const int hs = wave * 32 + (lane & 31);  // score waves: head of this lane's scores
  const bool hok = sw && hs < a.H;
  const bool sact = sw && wave * 32 < a.H;  // the score wave owns at least one head
  const int nhb = (a.H + 15) >> 4;           // head blocks with at least one head
  // (an 8-bit cache: the scale of the codes multiplies every score and output)
  const float kvs = FP8 ? a.kv_scale : 1.f;
  const float sl2 = a.scale * kLog2e * kvs;
  const int lr = lane & 15, g = (lane >> 4) & 3;

  // score operand A (32 keys x 16 dims, step t): lane l reads key l % 32,
  // dims 16 t + 8 (l / 32) .. + 7, i.e. chunk 2 t + l / 32 of the row, stored at
  // 8 (t / 4) + ((2 (t % 4) + l / 32) ^ swz(row)); kb[u] is the byte offset for
  // t % 4 == u without the 128 (t / 4)
  int kb[4];
  {
    const int row = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int u = 0; u < 4; ++u) kb[u] = row * ROWB + (((2 * u) | hl) ^ swz(row)) * 16;
  }
  // 8-bit cache: steps 2 u and 2 u + 1 take the codes of chunk 2 u + l / 32
  // (codes 0-7, then 8-15) from one 16-byte read of the staged tile: lane l
  // reads row l % 32, slot 36 row + 4 (u / 2) + ((2 (u % 2) + l / 32) ^ swz8(row));
  // kb8[u % 2] is the byte offset without the 64 (u / 2). The queries follow
  // the same order of the 576 dims (step t, half h: dims 16 (2 (t / 2) + h) +
  // 8 (t % 2) .. + 7).
  int kb8[2];
  {
    const int row = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int u = 0; u < 2; ++u) kb8[u] = row * (ECH8 * 16) + (((2 * u) | hl) ^ swz8(row)) * 16;
  }
  // value operand A (16 dims x 32 keys, transposing reads): lane k = 4 qa + qb
  // of 16-lane group g points at rows 4 g + qa (and 16 + 4 g + qa), dims
  // 16 D + 4 qb .. + 3 = chunk 2 D + qb / 2, byte (qb & 1) * 8 of the chunk.
  // 8-bit cache (ds_read_b64_tr_b8: element r of lane t of a 16-lane group
  // is byte t % 8 of the 8 read by lane 2 r + t / 8): lane s of group g points
  // at key row 8 g + s / 2, codes 16 D + 8 (s % 2) .. + 7, so that lane t
  // receives dim 16 D + t of keys 8 g .. 8 g + 7
  int vrow, vx;
  {
    const int qa = lr >> 2, qb = lr & 3;
    const int row = FP8 ? 8 * g + (lr >> 1) : 4 * g + qa;
    vrow = FP8 ? row * (ECH8 * 16) + (lr & 1) * 8 : row * ROWB + (qb & 1) * 8;
    vx = FP8 ? swz8(row) : (qb >> 1) ^ swz(row);
  }

  // O^T (this wavefront's blocks) += C^T P^T for tile t; operand element e of
  // lane (g, lr) is key 16 (e / 4) + 4 g + e % 4 (8-bit cache: key 8 g + e)
  auto value = [&](floatx4* RG, auto rolec, int t) __attribute__((always_inline)) {
    using BK = Blocks<decltype(rolec)::value>;
    const int wl = wave & 3;
    const char* Tb = FP8 ? reinterpret_cast<const char*>(&stage8[t % NSTAGE][0])
                         : reinterpret_cast<const char*>(&tile[t % NBUF][0]);
    const int pb = t & 1;
    // one 8-byte read of all the rescale flags (rare: lazy rescaling)
    const uint64_t flags = *reinterpret_cast<const uint64_t*>(&aflag[pb][0]);
    if (__builtin_amdgcn_readfirstlane((uint32_t)flags) | __builtin_amdgcn_readfirstlane((uint32_t)(flags >> 32))) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if ((flags >> (8 * hb)) & 0xff) {
          const float al = abuf[pb][hb * 16 + lr];
#pragma unroll
          for (int j = 0; j < BK::NSLOT; ++j)
            if (BK::reg(j, hb) >= 0) RG[BK::reg(j, hb)] *= al;
        }
      }
    }
#pragma unroll
    for (int ps = 0; ps < BK::NPASS; ++ps) {
      Frag<bf16> vf[4];
#pragma unroll
      for (int j = BK::first(ps); j < BK::last(ps); ++j) {
        const int D = BK::D(j, wl);
        if constexpr (FP8) {
          const v2i32 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) v2i32*)(Tb + vrow + (D ^ vx) * 16));
          vf[j - BK::first(ps)].v = widen8x8((uint32_t)w[0], (uint32_t)w[1]);
        } else {
          const char* p = Tb + vrow + (D >> 2) * 128 + ((2 * (D & 3)) ^ vx) * 16;
          vf[j - BK::first(ps)].v = tr_pair(p, p + 16 * ROWB);
        }
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if (hb < nhb) {
          Frag<bf16> ph;
          ph.v = pbuf[pb][hb][lane];
#pragma unroll
          for (int j = BK::first(ps); j < BK::last(ps); ++j)
            if (BK::reg(j, hb) >= 0)
              RG[BK::reg(j, hb)] = mfma16(vf[j - BK::first(ps)], ph, RG[BK::reg(j, hb)]);
        }
      }
    }
  };

  // ---- ring of NBUF tiles: tile t is read in steps t (scores) and t + 1
  // (values), so step t refills the buffer of tile t - 2 with tile t + NBUF - 2.
  // 8-bit cache: likewise, step t copies tile t + 1 into the staging buffer of
  // tile t - 2.
  static_assert(NBUF >= 3 && NBUF <= 4, "ring of 3 or 4 tiles");
  auto wait_tiles = [&](int later) {  // all but the copies of the `later` tiles issued last have landed
    if (later <= 0) MLA_WAIT_VMCNT(0);
    else if (last_dma) MLA_WAIT_VMCNT(DMA_N);
    else MLA_WAIT_VMCNT(DMA_N - 1);
  };
  static_assert(NBUF == 3, "the sparse-list entries run one tile ahead of the copies");
  int ev = gather_load(0);                              // entries of the next tile to copy
  uint32_t gm = gather ? (uint32_t)__ballot(ev >= 0) : 0u;  // row mask of the next tile to score
  issue(0, ev);
  ev = gather_load(1);

  // the piece loop, compiled once per role: each copy has its own register
  // allocation, and both run the same sequence of barriers
  auto run = [&](auto rolec) __attribute__((always_inline)) {
  constexpr bool sw = decltype(rolec)::value;
  floatx4 RG[Blocks<sw>::NREG];
  float m = -INFINITY, l = 0.f;
  int i = 0;
  while (i < n) {
    // ---- one piece: the consecutive tiles [i, iend) of sequence b
    const int b = __builtin_amdgcn_readfirstlane(t_seq[i]);
    const int iend = __builtin_amdgcn_readfirstlane(t_end[i]);
    const int lo = __builtin_amdgcn_readfirstlane(t_lo[i]);
    const int hi = __builtin_amdgcn_readfirstlane(t_hi[i]);
    const bool seq_start = __builtin_amdgcn_readfirstlane(t_k0[i]) == (lo / KT) * KT;
    const bool whole = seq_start && __builtin_amdgcn_readfirstlane(t_k0[iend - 1]) + KT >= hi;
    const int64_t slot = 2 * (int64_t)r + (seq_start ? 1 : 0);

    if constexpr (sw) {
      // latent query of head hs: B operand of S^T, step t = dims 16 t + 8 (l / 32) .. + 7
      const int hq = hok ? hs : 0;
      const bf16* ql = reinterpret_cast<const bf16*>(a.ql) + (int64_t)b * a.ldql + (int64_t)hq * a.c;
      // roped query: token and head of the (query, head) pair in query blocks
      int64_t qt = b, qh = hq;
      if (a.Hr > 0) {
        const int64_t pair = (int64_t)b * a.H + qh;
        qt = pair / a.Hr;
        qh = pair % a.Hr;
      }
      const bf16* qp = reinterpret_cast<const bf16*>(a.q) + qt * a.ldq + qh * a.qk_head + a.n;
#pragma unroll
      for (int t = 0; t < KS2; ++t) {
        const int e = FP8 ? (2 * (t >> 1) + (lane >> 5)) * 16 + (t & 1) * 8 : t * 16 + (lane >> 5) * 8;
        const bf16* src = !hok ? a.zeros : (e < 512 ? ql + e : qp + (e - 512));
        RG[t] = __builtin_bit_cast(floatx4, *reinterpret_cast<const bf16x8*>(src));
      }
#pragma unroll
      for (int k = KS2; k < Blocks<sw>::NREG; ++k) RG[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
      for (int k = 0; k < Blocks<sw>::NREG; ++k) RG[k] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    // the queries, the tiles in flight and the outputs stored by the previous
    // piece (stores may complete out of order with loads): wait for everything
    MLA_WAIT_VMCNT(0);
    // ... for every wavefront; the previous piece's normalisers are no longer read
    lds_barrier();
    m = -INFINITY;
    l = 0.f;

    // step it: the score wavefronts score tile it and publish its
    // probabilities (buffer it & 1); every wavefront multiplies tile it - 1 by
    // its probabilities (buffer (it - 1) & 1)
    for (int it = i; it <= iend; ++it) {
      // the copies of tile it + 1 go into the buffer of tile it - 2 (read
      // last in step it - 1)
      const uint32_t gm_cur = gm;  // row mask of tile it (sparse lists)
      if (it < iend && it + 1 < n) {
        issue(it + 1, ev);
        if (gather) {
          gm = (uint32_t)__ballot(ev >= 0);
          ev = gather_load(it + 2);
        }
      }
      if constexpr (sw) {
        const bool scoring = it < iend && sact;
        bf16x4 pq[4];
        float alpha = 1.f;
        if (scoring) {
          // ---- S^T (32 keys x 32 heads) = C q^T over the 576 dims
          const int k0 = __builtin_amdgcn_readfirstlane(t_k0[it]);
          floatx16 sc = {};
          if constexpr (FP8) {
            // 16-byte code reads PLA step pairs ahead, widened just before
            // their two MFMAs
            const char* Sb = reinterpret_cast<const char*>(&stage8[it % NSTAGE][0]);
            constexpr int NP = KS2 / 2, PLA = 2;
            uint4 kw[PLA];
#pragma unroll
            for (int u = 0; u < PLA; ++u) kw[u] = *reinterpret_cast<const uint4*>(Sb + kb8[u & 1] + (u >> 1) * 64);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < NP; ++u) {
              const uint4 w = kw[u % PLA];
              if (u + PLA < NP) kw[u % PLA] = *reinterpret_cast<const uint4*>(Sb + kb8[(u + PLA) & 1] + ((u + PLA) >> 1) * 64);
              sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8x8(w.x, w.y), __builtin_bit_cast(bf16x8, RG[2 * u]), sc, 0, 0, 0);
              sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(widen8x8(w.z, w.w), __builtin_bit_cast(bf16x8, RG[2 * u + 1]), sc, 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            const char* Tb = reinterpret_cast<const char*>(&tile[it % NBUF][0]);
            // key fragments are read KLA steps ahead of their MFMA (one wavefront
            // per SIMD scores, so its own reads must cover the LDS latency)
            constexpr int KLA = GATHER ? 3 : 4;  // (the sparse lists hold more registers)
            bf16x8 kf[KLA];
#pragma unroll
            for (int t = 0; t < KLA; ++t) kf[t] = *reinterpret_cast<const bf16x8*>(Tb + kb[t & 3] + (t >> 2) * 128);
            // hard scheduling fences keep each read KLA steps ahead (the
            // scheduler would otherwise sink it to its MFMA)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < KS2; ++t) {
              sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % KLA], __builtin_bit_cast(bf16x8, RG[t]), sc, 0, 0, 0);
              if (t + KLA < KS2) kf[t % KLA] = *reinterpret_cast<const bf16x8*>(Tb + kb[(t + KLA) & 3] + ((t + KLA) >> 2) * 128);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // ---- online softmax of head hs (log2 domain); element e of lane l
          // is key 8 (e / 4) + 4 (l / 32) + e % 4; lanes l and l ^ 32 hold the
          // same head
          const bool edge = gather || k0 < lo || k0 + KT > hi;
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float x = sc[e] * sl2;
            if (edge) {
              const int kk = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
              const int key = k0 + kk;
              if (key < lo || key >= hi || (gather && !((gm_cur >> kk) & 1u))) x = -INFINITY;
            }
            sc[e] = x;
            mx = fmaxf(mx, x);
          }
          mx = red2_max(mx);
          // lazy rescaling: the reference max moves only when exceeded by
          // more than 2^8 (probabilities stay <= 256; exact after the
          // division by l)
          const float mnew = (mx > m + 8.f) ? mx : m;
          alpha = m == -INFINITY ? 1.f : fast_exp2(m - mnew);
          // (a sparse list can leave a whole tile without keys: weights 0)
          const float mref = mnew == -INFINITY ? 0.f : mnew;
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float pv = fast_exp2(sc[e] - mref);
            sum += pv;
            pq[e >> 2][e & 3] = (bf16)pv;
          }
          l = l * alpha + red2_sum(sum);
          m = mnew;
        }
        if (scoring) {
          // probabilities: key group kg = 2 q + l / 32 (keys 4 kg .. 4 kg + 3)
          // goes to lane 16 (kg % 4) + lr of head block hb, half kg / 4
          // (8-bit cache: lane 16 (kg / 2) + lr, half kg % 2)
          const int hb = 2 * wave + ((lane >> 4) & 1);
          char* pbase = reinterpret_cast<char*>(&pbuf[it & 1][hb][0]);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int kg = 2 * q4 + (lane >> 5);
            const int off = FP8 ? (16 * (kg >> 1) + lr) * 16 + (kg & 1) * 8 : (16 * (kg & 3) + lr) * 16 + (kg >> 2) * 8;
            *reinterpret_cast<bf16x4*>(pbase + off) = pq[q4];
          }
          const uint64_t rm = __ballot(alpha != 1.f);
          if (lane < 32) abuf[it & 1][hs] = alpha;
          if (lane == 0) {
            aflag[it & 1][2 * wave] = (rm & 0xffffull) ? 1 : 0;
            aflag[it & 1][2 * wave + 1] = (rm & 0xffff0000ull) ? 1 : 0;
          }
          if (it == iend - 1) {
            // the piece ends here: share the normaliser; a cut piece also
            // writes its log-sum-exp (slot 1: the piece starts the sequence
            // and the range ends inside it; slot 0: the range starts inside
            // the sequence)
            if (lane < 32) lbuf[hs] = l;
            if (!whole && lane < 32 && hok) a.part_lse[slot * a.H + hs] = m + __log2f(l);
          }
        } else if (it < iend && lane == 0) {
          // no head of this wave: no rescale flags for its head blocks
          aflag[it & 1][2 * wave] = 0;
          aflag[it & 1][2 * wave + 1] = 0;
        }
        if (it > i) value(RG, rolec, it - 1);
      } else if (it > i) {
        value(RG, rolec, it - 1);
      }
      if (it < iend) wait_tiles(min(NBUF - 3, n - 2 - it));  // tile it + 1 landed
      // tile it + 1 is in LDS for every wavefront; the probabilities of tile
      // it are shared; tile it - 1 and the probabilities of tile it - 1 are no
      // longer read
      lds_barrier();
    }

    // ---- finish the piece: a whole sequence -> normalised latent output; a
    // cut piece -> partial output (normalised by its own sum, stored as bf16:
    // the merged latent output is rounded to bf16 in any case)
    {
      using BK = Blocks<sw>;
      const int wl = wave & 3;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int hh = 16 * hb + lr;
        if (hh >= a.H) continue;
        const float lv = lbuf[hh];
        const float inv = lv > 0.f ? kvs / lv : 0.f;  // no key at all: a zero row
        bf16* dst = whole ? reinterpret_cast<bf16*>(a.o_lat) + ((int64_t)b * a.H + hh) * a.c
                          : reinterpret_cast<bf16*>(a.part_o) + (slot * a.H + hh) * a.c;
        dst += 4 * g;
#pragma unroll
        for (int j = 0; j < BK::NSLOT; ++j) {
          if (BK::reg(j, hb) < 0) continue;
          const floatx4 v = RG[BK::reg(j, hb)] * inv;
          *reinterpret_cast<bf16x4*>(dst + 16 * BK::D(j, wl)) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        }
      }
    }
    i = iend;
  }
  };
  if (sw) run(std::true_type{});
  else run(std::false_type{});
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
  // the pieces in groups of 8, each group's loads issued together, combined
  // with a running maximum of the log-sum-exps
  float mx = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int g0 = gs; g0 <= ge; g0 += 8) {
    float lse[8];
    bf16x8 x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int gg = g0 + e;
      // (an empty range past the first holds no piece)
      const bool ok = gg <= ge && (gg == gs || range_start_d(gg + 1, R, T) != range_start_d(gg, R, T));
      const int64_t slot = 2 * (int64_t)gg + (gg == gs ? 1 : 0);
      lse[e] = ok ? a.part_lse[slot * a.H + h] : -INFINITY;
      x[e] = ok ? *reinterpret_cast<const bf16x8*>(po + (slot * a.H + h) * a.c + t * 8) : bf16x8{};
    }
    float cm = mx;
#pragma unroll
    for (int e = 0; e < 8; ++e) cm = fmaxf(cm, lse[e]);
    const float sc = mx == -INFINITY ? 0.f : fast_exp2(mx - cm);
    den *= sc;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = lse[e] == -INFINITY ? 0.f : fast_exp2(lse[e] - cm);
      den += w;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] += w * (float)x[e][d];
    }
    mx = cm;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;  // no key in any piece: a zero row
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
  if (a.gather_ent && (a.gather_k <= 0 || (int64_t)a.batch * a.gather_k >= ((int64_t)1 << 31)))
    return "stream-K decode: sparse lists need 0 < batch * gather_k < 2^31";
  if (a.kv_fp8 && !(a.kv_scale > 0.f)) return "stream-K decode: the 8-bit cache needs a positive scale";
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
  if (a.kv_fp8) {
    if (a.gather_ent) hipLaunchKernelGGL((decode_sk_kernel<3, true, true>), dim3(a.ranges), dim3(NT), 0, s, a);
    else hipLaunchKernelGGL((decode_sk_kernel<3, false, true>), dim3(a.ranges), dim3(NT), 0, s, a);
  } else if (a.gather_ent) {
    hipLaunchKernelGGL((decode_sk_kernel<3, true, false>), dim3(a.ranges), dim3(NT), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_sk_kernel<3, false, false>), dim3(a.ranges), dim3(NT), 0, s, a);
  }
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return hipSuccess;
}

hipError_t decode_sk_merge_launch(const DecodeAttnArgs& a, hipStream_t s) {
  if (a.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_sk_merge_kernel, dim3((a.H + 3) / 4, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
