/*
 * mla.h — C ABI of the MI355X (gfx950) Multi-head Latent Attention forward.
 *
 * The operation is the MLA layer described by the "MLA(Multi-Head Latent
 * Attention)" blog walk-through of vLLM's MLA code (the DeepseekV2MLAAttention,
 * MultiHeadLatentAttentionWrapper.forward, MLAAttention.forward,
 * do_kv_cache_update, forward_mha and forward_mqa listings) with the options of
 * SpecForge PR "Add config-selectable MLA draft attention" (Summary: optional
 * low-rank Q, shared compressed KV latent, partial interleaved or NeoX RoPE,
 * optional output gate, full/sliding masks; Structure: fully-masked-query
 * zeroing and o_proj):
 *
 *   q     = (q_lora ? RMSNorm(x W_qa^T) W_qb^T : x W_q^T)      viewed [T, H, n + r]
 *   kv    = x W_kva^T = [kv_c (c) | k_pe (r)]
 *   entry = [RMSNorm(kv_c) | RoPE(k_pe)]                        written to the cache first
 *   q[..., n:] = RoPE(q[..., n:])
 *   attention per head over the visible cache entries, then optional gate
 *   sigma(x W_g^T), then o_proj.
 *
 * Notation: H heads, n = qk_nope_head_dim, r = qk_rope_head_dim,
 * c = kv_lora_rank, dv = v_head_dim, E = c + r (one cache entry, 576 for the
 * DeepSeek dims 512 + 64).
 *
 * Conventions shared by every entry point
 *  - "device" pointers are HIP device memory on the current device; "host"
 *    arguments are plain values. Element type of every floating-point array is
 *    the context's dtype (fp32 or bf16, row-major, contiguous).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = default
 *    stream) and never synchronises, except mla_init_weights (once, at the end).
 *  - Host-side validation of every host argument happens before any HIP call;
 *    on failure the function returns a nonzero mla_status, launches nothing and
 *    mla_last_error() describes the problem. Contents of device arrays are not
 *    validated on the host (that would need a synchronisation): kernels clamp
 *    lengths, positions and intervals into range and ignore block-table entries
 *    outside [0, num_blocks), so bad indices cannot address outside the buffers.
 *  - A context may be used by one stream at a time (its workspaces are shared
 *    between calls). Errors inside kernels surface at the caller's next
 *    synchronisation, as HIP reports them.
 *  - The paged latent cache is [num_blocks, page_size, E] (one KV head, no
 *    separate K and V planes; get_kv_cache_shape and MLAAttentionSpec listings).
 *    Entry j of sequence b (its logical position j) lives at
 *    cache[block_table[b * max_blocks + j / page_size]][j % page_size].
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_API __attribute__((visibility("default")))

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer, negative or zero size, bad enum */
  MLA_ERR_DIMS = 2,        /* inconsistent model dimensions */
  MLA_ERR_UNSUPPORTED = 3, /* valid but not supported by these kernels (alignment, sizes) */
  MLA_ERR_CAPACITY = 4,    /* call exceeds the limits given at init */
  MLA_ERR_HIP = 5,         /* a HIP runtime call failed */
  MLA_ERR_OOM = 6          /* device allocation failed */
} mla_status;

typedef enum mla_dtype { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

/* NeoX rotates pairs (j, j + r/2); interleaved rotates pairs (2j, 2j + 1);
 * both by angle pos * theta^(-2j/r). Rotated pairs stay in place. */
typedef enum mla_rope_style { MLA_ROPE_NEOX = 0, MLA_ROPE_INTERLEAVED = 1 } mla_rope_style;

/* Visible keys of a query at logical position p in a sequence of L entries:
 * FULL [0, L); CAUSAL [0, p + 1); SLIDING [max(0, p - window + 1), p + 1)
 * (exactly `window` keys including itself). A query with no visible key gets
 * an attention output of exactly zero. */
typedef enum mla_mask_kind { MLA_MASK_FULL = 0, MLA_MASK_CAUSAL = 1, MLA_MASK_SLIDING = 2 } mla_mask_kind;

/* Cache entry storage. COMPUTE: the entries in the compute dtype (c + r
 * values of `dtype`). FP8_E4M3: c + r bytes per entry, each the OCP E4M3
 * ("fn" variant: no infinities, 0x7F/0xFF NaN) code of value / kv_cache_scale,
 * rounded to nearest with ties to the even code and saturated to +-448; one
 * scale for the whole cache. The MLA blog's MLAAttention.forward listing
 * computes dynamic q/k/v scales for an FP8 KV cache and its cache-shape
 * listings name a packed 656-byte fp8 entry without its packing; this plain
 * 576-byte entry with a per-tensor scale is the reading taken (the scale is
 * an input, not computed). The encoded values are the bf16 tensors the MLA
 * blog's wrapper forward hands to the cache update (kv_c_normed and the roped
 * k_pe of a bf16 model): each entry value is rounded to bf16 before its code
 * is taken. With FP8_E4M3, mla_init_weights returns
 * MLA_ERR_UNSUPPORTED unless dtype is BF16, c = 512, r = 64, num_heads <= 128,
 * page_size % 32 == 0 and max_batch <= 1024, and MLA_ERR_INVALID_ARG for a
 * scale that is not finite and > 0; the prefill reads a library-owned bf16
 * copy of the visible entries (max_prefill_kv + max_batch * page_size rows,
 * allocated at init). The caller's cache is c + r bytes per entry. */
typedef enum mla_kv_cache_dtype { MLA_KV_CACHE_COMPUTE = 0, MLA_KV_CACHE_FP8_E4M3 = 1 } mla_kv_cache_dtype;

typedef struct mla_config {
  int32_t hidden_size;
  int32_t num_heads;
  int32_t q_lora_rank;      /* 0 = no low-rank Q path (q_proj is used) */
  int32_t kv_lora_rank;     /* c */
  int32_t qk_nope_head_dim; /* n */
  int32_t qk_rope_head_dim; /* r (even) */
  int32_t v_head_dim;       /* dv */
  int32_t rope_style;       /* mla_rope_style */
  double rope_theta;        /* > 1 */
  double rms_norm_eps;      /* >= 0, both RMSNorms */
  double softmax_scale;     /* <= 0 selects 1 / sqrt(n + r) */
  int32_t use_output_gate;  /* 0 or 1: out = o_proj(attn * sigmoid(x W_g^T)) */
  int32_t dtype;            /* mla_dtype of weights, activations and cache */
  int32_t page_size;        /* tokens per cache block */
  /* capacity limits; workspaces are allocated once at init from these */
  int32_t max_batch;        /* sequences per call */
  int32_t max_tokens;       /* new tokens per call (decode: = batch) */
  int32_t max_seq_len;      /* cache entries per sequence (positions < max_seq_len) */
  int32_t max_prefill_kv;   /* prefill: batch * max_kv_len rows of expanded K/V; 0 = no prefill */
  int32_t max_block_tokens; /* mla_decode_absorbed_block: batch * q_len new tokens per call; 0 = not used */
  int32_t max_topk;         /* mla_decode_absorbed_sparse: listed keys per query; 0 = not used */
  int32_t kv_cache_dtype;   /* mla_kv_cache_dtype; FP8_E4M3 needs dtype BF16, c = 512, r = 64 */
  float kv_cache_scale;     /* FP8_E4M3: value = code * scale (> 0, finite); a power of two keeps the
                               prefill's bf16 copy of the entries exact */
  int32_t max_train_tokens; /* mla_backward_expanded: tokens per call; 0 = not used */
} mla_config;

/* Layer weights, device pointers in nn.Linear [out, in] row-major layout with
 * the names used on the pages. Unused entries may be NULL. */
typedef struct mla_weights {
  const void* q_a_proj;           /* [q_lora_rank, hidden]        (q_lora_rank > 0) */
  const void* q_a_layernorm;      /* [q_lora_rank]                (q_lora_rank > 0) */
  const void* q_b_proj;           /* [H * (n + r), q_lora_rank]   (q_lora_rank > 0) */
  const void* q_proj;             /* [H * (n + r), hidden]        (q_lora_rank == 0) */
  const void* kv_a_proj_with_mqa; /* [c + r, hidden] */
  const void* kv_a_layernorm;     /* [c] */
  const void* kv_b_proj;          /* [H * (n + dv), c], per head [k_nope rows | v rows] */
  const void* o_proj;             /* [hidden, H * dv] */
  const void* g_proj;             /* [H * dv, hidden]             (use_output_gate) */
} mla_weights;

/* Gradients of the layer weights (mla_backward_expanded): device pointers
 * with the shapes and element type of the mla_weights entries of the same
 * name. A NULL entry is not computed. */
typedef struct mla_grads {
  void* q_a_proj;
  void* q_a_layernorm;
  void* q_b_proj;
  void* q_proj;
  void* kv_a_proj_with_mqa;
  void* kv_a_layernorm;
  void* kv_b_proj;
  void* o_proj;
  void* g_proj;
} mla_grads;

typedef struct mla_ctx mla_ctx;

/*
 * mla_init_weights — validate the configuration and create a context.
 * Dimension identities checked here (MLA blog, dimension summary and
 * MLAAttention.__init__): q head dim = n + r, cache entry = c + r, one KV
 * head; r even; every size > 0. The library copies and repacks the weights
 * into device memory it owns (fused first projection, the q_a RMSNorm gain
 * folded into q_b_proj, the per-head W_UK^T blocks of kv_b_proj for the
 * absorbed decode); the caller may free its weight tensors after return.
 * Workspaces are sized from the capacity fields. Synchronises `stream` once.
 * On success *out receives the context; on failure *out is NULL.
 */
MLA_API int mla_init_weights(const mla_config* cfg, const mla_weights* w, void* stream, mla_ctx** out);

/*
 * mla_prefill_expanded — MLA forward of `total_tokens` new tokens in expanded
 * form (MLA blog, forward_mha listing: the latent is expanded through kv_b_proj
 * into per-head k_nope and v, K = [k_nope, k_pe]).
 *   x            device [total_tokens, hidden]; sequence b owns rows
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   cu_seqlens_q device int32 [batch + 1], nondecreasing, cu[0] = 0, cu[batch] = total_tokens
 *   prefix_lens  device int32 [batch]: entries already cached for sequence b
 *                (its latent prefix); new token i is at logical position prefix_len + i
 *   max_q_len    host: >= every q_len; max_kv_len host: >= every prefix_len + q_len
 *   kv_cache     device [num_blocks, page_size, E]; the new entries
 *                [RMSNorm(kv_c) | RoPE(k_pe)] are written at their positions
 *                before attention, so each query sees its own entry
 *   block_table  device int32 [batch, max_blocks]
 *   mask_kind, window  mla_mask_kind and its window (SLIDING only)
 *   row_lo, row_hi     optional device int32 [total_tokens]: when both are
 *                non-NULL they replace the mask with the visible interval
 *                [row_lo, row_hi) of positions (clamped to [0, L)); lo >= hi
 *                drops the row (its output is zero)
 *   out          device [total_tokens, hidden]
 * Limits: batch <= max_batch, total_tokens <= max_tokens, max_kv_len <=
 * max_seq_len, batch * max_kv_len <= max_prefill_kv (else MLA_ERR_CAPACITY).
 * With at most 64 new tokens per sequence (bf16, 512 + 64 latent, 128 + 64 /
 * 128 heads, heads a multiple of 8) the expanded keys and values are never
 * stored: each 256-entry chunk is expanded and attended in one kernel and the
 * chunks are merged by their log-sum-exp (same arithmetic, one fewer round
 * trip through HBM).
 */
MLA_API int mla_prefill_expanded(mla_ctx* ctx, const void* x, int32_t batch, int32_t total_tokens,
                         const int32_t* cu_seqlens_q, const int32_t* prefix_lens,
                         int32_t max_q_len, int32_t max_kv_len,
                         void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks, int32_t mask_kind, int32_t window,
                         const int32_t* row_lo, const int32_t* row_hi,
                         void* out, void* stream);

/*
 * mla_backward_expanded — gradient of the expanded MLA layer on whole training
 * sequences (no cached prefix; token j of a sequence is at position j). The
 * SpecForge PR "Add config-selectable MLA draft attention" trains MLA as a
 * draft attention and validates it with gradients (Validation); the PR
 * "extract GQA/MLA attention into reusable layers" checks outputs and
 * gradients (Accuracy Test). The forward is mla_prefill_expanded's (MLA blog,
 * wrapper forward and forward_mha listings) with prefix_lens = 0; given
 * dout = dL/dout, the call writes dx = dL/dx and dL/dW of every weight named
 * in grads, each by the chain rule through that forward: o_proj, the output
 * gate, softmax attention (recomputed from the saved log-sum-exp), the
 * kv_b_proj expansion, the rope key shared by the heads, RoPE, both RMSNorms
 * and the first projections. The forward is recomputed inside the call.
 *   x            device [total_tokens, hidden]; sequence b owns rows
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   cu_seqlens_q device int32 [batch + 1] (as mla_prefill_expanded)
 *   max_q_len    host: >= every sequence length
 *   mask_kind, window, row_lo, row_hi: as mla_prefill_expanded
 *   dout         device [total_tokens, hidden]
 *   dx           device [total_tokens, hidden] (written)
 *   grads        host struct of device outputs (overwritten, not accumulated)
 * Every array is in the context's dtype. Limits: total_tokens <=
 * max_train_tokens and <= max_tokens, batch <= max_batch, max_q_len <=
 * max_seq_len, and batch * (max_q_len rounded up to page_size) <=
 * max_prefill_kv (else MLA_ERR_CAPACITY). Supports q/k head dims n + r <= 192
 * and v_head_dim <= 128 in bf16, <= 64 and <= 64 in fp32 (else
 * MLA_ERR_UNSUPPORTED). Asynchronous; the context's workspaces are used.
 */
MLA_API int mla_backward_expanded(mla_ctx* ctx, const void* x, int32_t batch, int32_t total_tokens,
                         const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t mask_kind, int32_t window,
                         const int32_t* row_lo, const int32_t* row_hi, const void* dout, void* dx,
                         const mla_grads* grads, void* stream);

/*
 * mla_decode_absorbed — one new token per sequence in absorbed form (MLA blog,
 * the decode branch and forward_mqa listing: q_nope is projected into latent
 * space through W_UK, attention runs over the whole E-wide cache entries as
 * MQA with one shared latent head, the latent output is projected back through
 * W_UV).
 *   x            device [batch, hidden]
 *   seq_lens     device int32 [batch]: cache length INCLUDING the new token,
 *                which is written at position seq_len - 1 before attention
 *   max_seq_len  host: >= every seq_len (sizes the split-KV grid)
 *   out          device [batch, hidden]
 * kv_cache must not be NULL (the listing asserts a non-empty cache).
 * Limits: batch <= max_batch and <= max_tokens, max_seq_len <= the init max_seq_len.
 */
MLA_API int mla_decode_absorbed(mla_ctx* ctx, const void* x, int32_t batch,
                        void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                        int32_t mask_kind, int32_t window, void* out, void* stream);

/*
 * mla_decode_absorbed_block — a block of q_len new tokens per sequence (a
 * draft block being verified) in absorbed form: every token of the block
 * sees every cache entry of its sequence, the prefix and the whole block
 * (block-visible, the FULL mask). The MLA blog's forward listing sends the
 * tokens that the metadata counts as decode through this MQA branch, and the
 * SpecForge PR "Add config-selectable MLA draft attention" (Validation) runs
 * its draft blocks through spec_generate decode; this is the same arithmetic
 * as mla_prefill_expanded with the FULL mask, without expanding any latent.
 *   x            device [batch * q_len, hidden]: token i of sequence b is row
 *                b * q_len + i, at logical position prefix_lens[b] + i, and is
 *                written to the cache before attention
 *   prefix_lens  device int32 [batch]: cache entries before the block
 *   max_kv_len   host: >= prefix_lens[b] + q_len for every b
 *   out          device [batch * q_len, hidden]
 * Requires the bf16 512 + 64 latent and q_len * num_heads a multiple of 128
 * (MLA_ERR_UNSUPPORTED otherwise). Limits: batch <= max_batch,
 * batch * q_len <= max_block_tokens and <= max_tokens, max_kv_len <= max_seq_len.
 * Profiled under the decode stage names (wuk_absorb, decode_attn, ...).
 */
MLA_API int mla_decode_absorbed_block(mla_ctx* ctx, const void* x, int32_t batch, int32_t q_len,
                        void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* prefix_lens, int32_t max_kv_len,
                        void* out, void* stream);

/*
 * mla_decode_absorbed_sparse — mla_decode_absorbed where each sequence's query
 * sees only the cache positions listed for it (sparse, top-k MLA). The MLA
 * blog's wrapper forward computes top-k indices with an indexer when the layer
 * is sparse, and its MLAAttention.forward sends every token of a sparse
 * backend through the MQA (absorbed) branch; the indexer is not specified on
 * the pages, so the lists are an input here.
 *   topk_indices device int32 [batch, topk]: logical positions of sequence b's
 *                keys, in any order; entries < 0 or >= seq_lens[b] (and
 *                positions on unmapped pages) are ignored; a position listed
 *                twice is attended twice. A query with no listed key gets an
 *                attention output of exactly zero. The new token is written
 *                to the cache (position seq_len - 1) before attention and is
 *                attended only if listed.
 *   topk         host: list length, 0 < topk <= max_topk
 * Other arguments as mla_decode_absorbed (no mask: the lists replace it).
 * Requires the bf16 512 + 64 latent with at most 128 heads (MLA_ERR_UNSUPPORTED
 * otherwise). Profiled under the decode stage names; the entry lookup of the
 * lists runs inside decode_attn.
 */
MLA_API int mla_decode_absorbed_sparse(mla_ctx* ctx, const void* x, int32_t batch,
                        void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                        const int32_t* topk_indices, int32_t topk, void* out, void* stream);

/*
 * mla_decode_absorbed_noalloc — mla_decode_absorbed for callers that cannot
 * allocate device memory during the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, errors
 * and result as mla_decode_absorbed (the same kernels; outputs are bitwise
 * equal), but every per-call workspace (projection outputs, latent queries
 * and outputs, stream-K partials, split-K GEMM sums) is carved from one
 * static device array of 128 MiB that the library holds on each device it
 * runs on until the process ends; the call allocates nothing. The context
 * (weights, RoPE table) still comes from mla_init_weights.
 * Requires the stream-K shape (bf16, 512 + 64 latent, <= 128 heads, page
 * size a multiple of 32) and batch <= 1024, else MLA_ERR_UNSUPPORTED; a call
 * whose workspaces exceed the array returns MLA_ERR_CAPACITY before any
 * launch (the DeepSeek-V3 decode of 64 sequences x 128 heads needs about
 * 95 MiB). Every call on a device shares that device's array, which keeps
 * the last call's contents: calls that overlap on one device (on different
 * streams, or different contexts) race and must be serialised by the caller.
 */
MLA_API int mla_decode_absorbed_noalloc(mla_ctx* ctx, const void* x, int32_t batch,
                        void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                        int32_t mask_kind, int32_t window, void* out, void* stream);

/*
 * Stage timing, for measurement. When enabled, every launch sequence of the
 * context records a pair of HIP events around each stage on the call's own
 * stream (the stream the stage's kernels run on); mla_profile_read waits for
 * them, returns per-stage totals and clears the record. Stages (index: name):
 *   0 qkv_a_gemm   fused first projection (x -> [q_c | q], kv_c, k_pe, gate)
 *   1 q_b_gemm     q_b projection with the q_a RMSNorm folded in
 *   2 rope_cache   latent RMSNorm, RoPE of q_pe and k_pe, cache write
 *   3 kv_b_expand  prefill: expansion of every visible latent through kv_b_proj
 *   4 prefill_attn prefill: flash attention over the expanded keys/values
 *   5 wuk_absorb   decode: q_nope -> latent space through W_UK
 *   6 decode_attn  decode: split-KV latent attention over the paged cache
 *   7 decode_merge decode: log-sum-exp merge of the splits
 *   8 wuv_gemm     decode: latent output -> v_head_dim through W_UV (+ gate)
 *   9 o_proj_gemm  output projection
 *  10 expand_attn  prefill with at most 64 new tokens per sequence (bf16,
 *                  512 + 64 latent, 128 + 64 / 128 heads): the kv_b expansion
 *                  and the attention over each 256-entry chunk of the cache in
 *                  one kernel (stages 3 and 4 do not run then)
 *  11 expand_merge log-sum-exp merge of those chunks (+ output gate)
 *  12 kv_dequant   8-bit cache, prefill: bf16 copy of the visible entries
 *  13 attn_bwd     backward: attention gradient kernels (dK/dV and dQ)
 *  14 bwd_gemm     backward: dA, dcn, dqn and dx products
 *  15 wgrad_gemm   backward: weight gradients (with their transposed copies)
 *  16 bwd_pointwise backward: gate, RMSNorm, RoPE and RMSNorm-gain kernels
 * The backward's forward recomputation is timed under stages 0-4.
 * A stage may be more than one kernel (a split-K GEMM adds its reduction).
 */
#define MLA_NUM_STAGES 17
MLA_API int mla_profile_enable(mla_ctx* ctx, int32_t enable);
/* ms[i]: total elapsed milliseconds of stage i; count[i]: times it ran. Both
 * host arrays of MLA_NUM_STAGES entries (count may be NULL). Synchronises. */
MLA_API int mla_profile_read(mla_ctx* ctx, double* ms, int32_t* count);
MLA_API const char* mla_profile_stage_name(int32_t stage);

/* mla_free — release everything the context owns. It first waits for the
 * context's last call to finish (an event recorded on that call's stream when
 * it returned; stream order covers the calls before it), not for other work
 * on the device. NULL is a no-op. */
MLA_API void mla_free(mla_ctx* ctx);

/* mla_last_error — message of the last failure on the calling thread
 * (thread-local, valid until the next call on that thread). */
MLA_API const char* mla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
