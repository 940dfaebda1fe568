// Host-side interface of the MFMA GEMM used by every dense contraction of the
// MLA forward (projections, kv_b expansion, W_UK / W_UV per-head products).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

enum GemmEpilogue : int {
  EPI_STORE = 0,    // C = acc
  EPI_ROWNORM = 1,  // C = acc * rsqrt(mean_k A[m,k]^2 + eps)   (RMSNorm of A folded in)
  EPI_GATE = 2,     // C = acc * sigmoid(G[m, n])
};

// Rows of A read from the paged latent cache instead of a dense matrix
// (expansion of every visible latent through kv_b_proj). Output row
// m = b * max_kv_len + j holds position j of sequence b.
struct GatherA {
  const void* cache = nullptr;     // [num_blocks, page, E]
  const int32_t* block_table = nullptr;
  const int32_t* cu_seqlens = nullptr;  // [batch + 1]
  const int32_t* prefix_lens = nullptr; // [batch]
  int batch = 0, max_kv_len = 0, page = 0, max_blocks = 0, num_blocks = 0, entry = 0;
  int max_q_len = 0;
};

// C[z][M, N] = A[z][M, K] . W[z][N, K]^T  for z < batch (strides in elements).
struct GemmArgs {
  const void* A = nullptr; int64_t lda = 0, sA = 0;
  const void* W = nullptr; int64_t ldw = 0, sW = 0;
  void* C = nullptr; int64_t ldc = 0, sC = 0;
  int M = 0, N = 0, K = 0, batch = 1;
  int epi = EPI_STORE;
  const void* G = nullptr; int64_t ldg = 0, sG = 0;
  float eps = 0.f;
  bool gather = false;
  GatherA ga;
  const void* zeros = nullptr;  // >= 16 zero bytes (source of absent rows for streamed tiles)
};

// Launch (choosing tile shape and split-K). `ws` is an fp32 workspace of
// `ws_elems` floats used for split-K partial sums (may be null: no split-K).
// Returns hipSuccess or the launch error. bf16 == true selects bf16 operands.
hipError_t gemm_launch(const GemmArgs& g, bool is_bf16, float* ws, int64_t ws_elems, hipStream_t s);

// The 256 x 256 LDS-streaming kernel (gemm_big.hip) and when it applies.
bool gemm_big_eligible(const GemmArgs& g, bool is_bf16);
// Split-K count (>= 2) for a product the kernel fits except for having too
// few output tiles, with splits * M * N fp32 partials within ws_elems; else 0.
// narrow: also products narrower than one 256-wide tile (the narrow last
// columns of a wider product, whose tiles are mostly idle columns but whose
// k range is split over the CUs).
int gemm_big_splits(const GemmArgs& g, bool is_bf16, int64_t ws_elems, bool narrow = false);
// splits == 1: C directly; else fp32 partials part[split][M][N] (summed by
// the caller)
hipError_t gemm_big_launch(const GemmArgs& g, float* part, int splits, hipStream_t s);

// Validation of the alignment and size assumptions of gemm_launch; returns
// nullptr when fine, else a static message.
const char* gemm_check(const GemmArgs& g, bool is_bf16);

}  // namespace mla
