// Host-side interface of the non-GEMM kernels of the MLA forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

using bf16_t = __bf16;

struct RopeCacheArgs {
  void* q = nullptr; int64_t ldq = 0; int qk_head = 0;  // q [T, H, n + r] rows of stride ldq
  const void* kv = nullptr; int64_t ldkv = 0;            // [T, c + r] rows of stride ldkv
  const void* gamma_kv = nullptr;                         // [c]
  void* cache = nullptr;
  const int32_t* block_table = nullptr;
  int num_blocks = 0, max_blocks = 0, page = 0;
  const float* rope_cos = nullptr; const float* rope_sin = nullptr;  // [max_seq_len, r/2]
  int H = 0, n = 0, r = 0, c = 0;
  int interleaved = 0;
  float eps = 0.f;
  // token -> (sequence, position)
  int decode = 0;
  const int32_t* seq_lens = nullptr;     // decode
  const int32_t* cu_seqlens = nullptr;   // prefill; null: blocks of max_q_len tokens, block b at b max_q_len
  const int32_t* prefix_lens = nullptr;  // prefill
  int max_q_len = 0, max_kv_len = 0, max_seq_len = 0, total_tokens = 0;
  int batch = 0;  // sequences (rope_cache_launch sets it from its argument)
  // 8-bit cache (OCP E4M3 codes of value / scale), else the compute dtype
  int kv_fp8 = 0;
  float kv_scale = 1.f;
};
hipError_t rope_cache_launch(const RopeCacheArgs& a, bool is_bf16, int grid_x, int batch, hipStream_t s);

// Visible-key rule shared by the attention kernels.
struct MaskArgs {
  int kind = 0, window = 0;
  const int32_t* row_lo = nullptr; const int32_t* row_hi = nullptr;  // prefill, optional
};

struct PrefillAttnArgs {
  const void* q = nullptr; int64_t ldq = 0; int qk_head = 0;  // roped q [T, H, n + r]
  const void* kv = nullptr; int64_t ldkv = 0;                  // expanded [B * max_kv_len, H, n + dv]
  const void* cache = nullptr;                                  // k_pe from the paged cache
  const int32_t* block_table = nullptr;
  int num_blocks = 0, max_blocks = 0, page = 0;
  const int32_t* cu_seqlens = nullptr; const int32_t* prefix_lens = nullptr;
  int batch = 0, max_q_len = 0, max_kv_len = 0, total_tokens = 0;
  int H = 0, n = 0, r = 0, c = 0, dv = 0;
  float scale = 0.f;
  int q_log2 = 0;  // q was multiplied by scale * log2(e) (bf16 DeepSeek-head kernel only)
  MaskArgs mask;
  void* out = nullptr; int64_t ldo = 0;             // [T, H * dv]
  const void* gate = nullptr; int64_t ldg = 0;      // raw gate pre-activation [T, H * dv] or null
  float* lse = nullptr;                             // optional [T, H]: log2-domain log-sum-exp of the
                                                    // scaled scores (-inf for a row with no visible key)
};
hipError_t prefill_attn_launch(const PrefillAttnArgs& a, bool is_bf16, hipStream_t s);
const char* prefill_attn_check(const PrefillAttnArgs& a, bool is_bf16);

// Expanded-form attention with the kv_b expansion fused in, for few new
// tokens per sequence (attn_mha_fused.hip): bf16, c 512, n 128, r 64, dv 128.
constexpr int kMhaFusedMaxQ = 64;  // new tokens per sequence
struct MhaFusedArgs {
  const void* q = nullptr; int64_t ldq = 0; int qk_head = 0;  // roped q [T, H, n + r]
  const void* cache = nullptr;                                  // latent cache [blocks, page, 576]
  const int32_t* block_table = nullptr;
  int num_blocks = 0, max_blocks = 0, page = 0;
  const void* wkvb = nullptr;                                   // kv_b_proj [H (n + dv), c]
  const int32_t* cu_seqlens = nullptr; const int32_t* prefix_lens = nullptr;
  int batch = 0, max_q_len = 0, max_kv_len = 0, total_tokens = 0;
  int H = 0;
  float scale = 0.f;
  int q_log2 = 0;  // q was multiplied by scale * log2(e)
  MaskArgs mask;
  int nchunks = 0;                                  // ceil(max_kv_len / 256)
  int qblocks = 0;                                  // ceil(max_q_len / 16)
  bf16_t* part_o = nullptr;                         // [batch, nchunks, qblocks, H, 16, dv]
  float* part_lse = nullptr;                        // [batch, nchunks, qblocks, H, 16]
  void* out = nullptr; int64_t ldo = 0;             // [T, H * dv]
  const void* gate = nullptr; int64_t ldg = 0;      // raw gate pre-activation [T, H * dv] or null
};
const char* mha_fused_check(const MhaFusedArgs& a);
// bytes of part_o (rounded up to 256) followed by part_lse
size_t mha_fused_partial_bytes(int batch, int nchunks, int qblocks, int H);
hipError_t mha_fused_launch(const MhaFusedArgs& a, hipStream_t s);
hipError_t mha_fused_merge_launch(const MhaFusedArgs& a, hipStream_t s);

struct DecodeAttnArgs {
  const void* ql = nullptr; int64_t ldql = 0;       // latent query q_nope W_UK [B, H, c], row stride ldql
  const void* q = nullptr; int64_t ldq = 0; int qk_head = 0;  // roped q (rope part at offset n)
  const void* cache = nullptr;
  const int32_t* block_table = nullptr;
  int num_blocks = 0, max_blocks = 0, page = 0;
  const int32_t* seq_lens = nullptr;
  int len_add = 0;                                  // added to every seq_lens entry (stream-K only)
  int max_seq_len = 0, batch = 0;
  int H = 0, n = 0, r = 0, c = 0;
  float scale = 0.f;
  MaskArgs mask;
  int chunk = 0, splits = 0;                        // keys per split, splits per sequence
  float* part_o = nullptr;                          // [B, splits, H, c]
  float* part_lse = nullptr;                        // [B, splits, H]
  void* o_lat = nullptr;                            // [B, H, c] combined latent output
  const bf16_t* zeros = nullptr;                    // >= 16 zero bytes (tile padding source)
  // stream-K partition (512 + 64 bf16 latent): `ranges` workgroup ranges,
  // pieces in part_o [2 ranges, H, c] / part_lse [2 ranges, H]
  int ranges = 0;
  int32_t* tstart = nullptr;                        // [batch + 1] first tile of every sequence
  // query blocks (stream-K only): sequence index b of this struct is a virtual
  // sequence of H (query, head) pairs of physical sequence b / seq_div, which
  // owns the block-table row and the length. With Hr > 0 the pair j of b is
  // token (b H + j) / Hr, head (b H + j) % Hr of a model with Hr heads (the
  // latent queries and outputs are then [tokens, Hr, c] in the same order).
  int seq_div = 1;
  int Hr = 0;
  // sparse lists (stream-K only): sequence b sees the gather_k keys
  // gather_ent[b * gather_k + j], cache entry indices (-1 = no key), instead
  // of the visible range of its block table
  const int32_t* gather_ent = nullptr;
  int gather_k = 0;
  // 8-bit cache (stream-K only): entries are 576 OCP E4M3 codes, value = code * kv_scale
  int kv_fp8 = 0;
  float kv_scale = 1.f;
};
hipError_t decode_attn_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s);
hipError_t decode_merge_launch(const DecodeAttnArgs& a, bool is_bf16, hipStream_t s);
const char* decode_attn_check(const DecodeAttnArgs& a, bool is_bf16);

// Backward pass of the expanded layer on training sequences (train.hip).
// Token-packed rows t = cu_seqlens[b] + j unless noted; element type = the
// compute dtype unless noted.
struct TrainArgs {
  const int32_t* cu_seqlens = nullptr;
  int batch = 0, max_q_len = 0, total_tokens = 0;
  int Lp = 0;                                   // per-sequence row stride of cache / kvexp
  int H = 0, n = 0, r = 0, c = 0, dv = 0, q_lora = 0;
  float scale = 0.f, eps = 0.f;
  MaskArgs mask;
  const float* rope_cos = nullptr; const float* rope_sin = nullptr;  // [positions, r/2]
  int interleaved = 0;
  const void* q = nullptr; int64_t ldq = 0;     // roped q [T, H (n + r)]
  const void* cache = nullptr;                  // entries [b Lp + j, c + r]
  const void* kvexp = nullptr; int64_t ldkv = 0;  // [b Lp + j, H (n + dv)]
  const void* O = nullptr;                      // attention output (ungated) [T, H dv]
  void* A = nullptr;                            // gated output [T, H dv]
  const float* lse = nullptr;                   // [T, H] log2-domain log-sum-exp of the scaled scores
  const void* buf1 = nullptr; int64_t ldb1 = 0; // fused first projection [T, N1]
  int off_q = 0, off_kv = 0, off_g = -1;
  const void* gate = nullptr; int64_t ldg = 0;  // gate input (inside buf1) or null
  const void* gamma_kv = nullptr; const void* gamma_q = nullptr;
  float* rho_q = nullptr; float* rho_kv = nullptr;  // [T] RMSNorm scales
  // backward buffers
  void* dO = nullptr; int64_t ldo = 0;          // dA in, dO out (in place) [T, H dv]
  float* D = nullptr;                           // [T, H]
  void* dkvb = nullptr; int64_t lddkvb = 0;     // [T, H (n + dv)] per head [dk_nope | dv]
  float* dkr = nullptr;                         // [T, H, r] per-head gradient of the rope key (fp32)
  void* dQ = nullptr; int64_t lddq = 0;         // [T, H (n + r)]
  const void* dcn = nullptr;                    // [T, c] gradient of RMSNorm(kv_c)
  const void* dqn = nullptr;                    // [T, q_lora] gradient of RMSNorm(q_c)
  void* dbuf1 = nullptr; int64_t lddb1 = 0;     // [T, N1] gradient of the fused first projection output
};
const char* train_check(const TrainArgs& a, bool is_bf16);
hipError_t train_rmsnorm_rows(const void* x, int64_t ldx, const void* gamma, int N, float eps, void* y, int64_t ldy,
                              float* rho, int rows, bool is_bf16, hipStream_t s);
hipError_t train_gate_fwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
hipError_t train_gate_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
hipError_t train_attn_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
hipError_t train_kv_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
hipError_t train_q_rope_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
hipError_t train_q_norm_bwd(const TrainArgs& a, bool is_bf16, hipStream_t s);
// out[j] = sum_t dy[t, j] x[t, j] rho[t]; part: fp32 [ceil(rows / 256), cols]
hipError_t train_gamma_grad(const void* dy, int64_t lddy, const void* x, int64_t ldx, const float* rho, int rows,
                            int cols, float* part, void* out, bool is_bf16, hipStream_t s);
// dst [cols, ldd] = src^T with zero columns from rows to ldd; map_rows: source
// row of token t is b Lp + (t - cu[b])
hipError_t train_transpose(const void* src, int64_t lds, int rows, int cols, void* dst, int64_t ldd,
                           const TrainArgs& a, bool map_rows, bool is_bf16, hipStream_t s);

// Stream-K decode of the 512 + 64 bf16 latent (attn_decode_sk.hip).
constexpr int kDecodeMaxTiles = 256;   // 32-key tiles per workgroup range
constexpr int kDecodeMaxBatch = 1024;  // sequences per call
// nullptr when `a` (with ranges / workspaces filled in) can take this path
const char* decode_sk_check(const DecodeAttnArgs& a);
// ranges for `batch` sequences of at most `max_visible` visible keys on `cus` compute units
int decode_sk_ranges(int batch, int max_visible, int cus);
hipError_t decode_sk_launch(const DecodeAttnArgs& a, hipStream_t s);
hipError_t decode_sk_merge_launch(const DecodeAttnArgs& a, hipStream_t s);

}  // namespace mla
