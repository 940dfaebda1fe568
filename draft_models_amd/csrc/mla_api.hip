// C ABI of the MLA forward: context creation (validation, weight repacking,
// workspaces) and the stream-ordered launch sequences of the expanded prefill
// and the absorbed decode.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mla.h"
#include "common.h"
#include "gemm.h"
#include "kernels.h"

using namespace mla;

// Per-call device workspaces of the projections, the decode attention and
// the split-K GEMMs (a context's own, or carved from the static scratch array
// by mla_decode_absorbed_noalloc).
struct Workspace {
  void* buf1 = nullptr;     // [tokens, N1] fused first projection output
  void* qbuf = nullptr;     // [tokens, H (n + r)]  (low-rank Q path)
  void* qlat = nullptr;     // [rows, H, c] latent queries
  void* olat = nullptr;     // [rows, H, c] latent outputs
  void* attn = nullptr;     // [tokens, H dv]
  float* part_o = nullptr;  // decode partial outputs
  float* part_lse = nullptr;
  int32_t* sk_tstart = nullptr;  // [batch + 1] stream-K tile offsets
  float* gemm_ws = nullptr;      // split-K partial sums
  int64_t gemm_ws_elems = 0;
  int32_t* sp_ent = nullptr;     // [batch, topk] cache entries of the sparse lists
};

struct mla_ctx {
  mla_config cfg;
  bool bf16 = true;
  int esz = 2;
  int H = 0, n = 0, r = 0, c = 0, dv = 0, ql = 0, hid = 0, E = 0, qkh = 0;
  float scale = 0.f;
  int device = 0;
  // owned, repacked weights
  void* W1 = nullptr;  // fused first projection [N1, hid] = [q_a | q ; kv_a ; g]
  int N1 = 0, off_q = 0, off_kv = 0, off_g = -1;
  void* Wqb = nullptr;     // q_b_proj with the q_a_layernorm gain folded into its columns
  void* Wqb_l2 = nullptr;  // the same times scale * log2(e): queries for the bf16 prefill attention
  void* Wkvb = nullptr;    // kv_b_proj [H (n + dv), c]
  void* Wuk_t = nullptr;   // per head W_UK^T [H][c][n]
  void* Wo = nullptr;      // o_proj [hid, H dv]
  void* gamma_kv = nullptr;
  float* rope_cos = nullptr;
  float* rope_sin = nullptr;
  // workspaces of the calls (allocated at init from the capacity fields)
  Workspace ws;
  void* kvexp = nullptr;   // [max_prefill_kv, H (n + dv)]
  int max_splits = 32;
  int cus = 256;            // compute units of the device
  bool sk_shape = false;    // bf16 512 + 64 latent: stream-K decode
  int sk_max_ranges = 0;
  void* zeros = nullptr;   // 256 zero bytes: source of padding chunks in streamed tiles
  // 8-bit cache (codes of value / kv_scale): the prefill reads a bf16 copy of
  // the visible entries, sequence b's page p at block b mbs + p of kv_shadow
  bool kv_fp8 = false;
  float kv_scale = 1.f;
  void* kv_shadow = nullptr;        // [max_prefill_kv + max_batch page, c + r] bf16
  int32_t* kv_shadow_bt = nullptr;  // [max_batch, ceil(max_seq_len / page)] identity block table
  // training (mla_backward_expanded): weights in the forms the backward
  // products read, and its workspaces (max_train_tokens rows)
  struct Train {
    int Tm = 0;
    void* Wqb = nullptr;      // q_b_proj as given [H (n + r), ql]
    void* gamma_q = nullptr;  // q_a_layernorm [ql]
    void* WqbT = nullptr;     // [ql, H (n + r)]
    void* W1T = nullptr;      // fused first projection transposed [hid, N1]
    void* WkvbT = nullptr;    // [c, H (n + dv)]
    void* WoT = nullptr;      // [H dv, hid]
    void* buf1 = nullptr;     // [Tm, N1]
    void* qn = nullptr;       // [Tm, ql]
    void* q = nullptr;        // [Tm, H (n + r)]
    float* rho_q = nullptr;
    float* rho_kv = nullptr;
    void* cache = nullptr;    // [max_prefill_kv, E] entries, identity pages
    int32_t* bt = nullptr;    // identity block table
    int32_t* zero_prefix = nullptr;  // [max_batch] zeros
    void* O = nullptr;
    void* A = nullptr;
    float* lse = nullptr;
    void* dA = nullptr;
    float* D = nullptr;
    void* dkvb = nullptr;
    float* dkr = nullptr;
    void* dQ = nullptr;
    void* dcn = nullptr;
    void* dqn = nullptr;
    void* dbuf1 = nullptr;
    void* TX = nullptr;       // [hid, Tp] x^T
    void* TA = nullptr;       // [maxA, Tp] left operands of the weight-gradient products
    void* TB = nullptr;       // [maxB, Tp] right operands
    float* part = nullptr;    // column-sum partials
  } tr;
  std::vector<void*> allocs;
  hipEvent_t done = nullptr;  // recorded on the call's stream when an entry point returns
  // stage timing (mla_profile_*)
  bool profiling = false;
  struct Mark { int stage; hipEvent_t start, stop; };
  std::vector<Mark> marks;
  std::vector<hipEvent_t> event_pool;
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t _e = (expr);                                                        \
    if (_e != hipSuccess)                                                          \
      return fail(MLA_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

// Static device scratch of mla_decode_absorbed_noalloc. Each device the
// library runs on holds its own copy until the process ends. Host code never
// uses the array's name as an address: its device address is looked up once
// per device (scratch_setup, at context creation with that device current)
// and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)128 << 20;
constexpr size_t kScratchGemmBytes = (size_t)8 << 20;  // split-K partial sums of its GEMMs
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return MLA_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p)
    return fail(MLA_ERR_HIP, std::string("hipGetSymbolAddress of the scratch array failed: ") + hipGetErrorString(e));
  g_scratch_ptr[device] = p;
  return MLA_OK;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

__global__ void scale_cols_kernel(const void* src, const void* gamma, void* dst, int64_t rows, int cols, int bf,
                                  float mul) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * cols) return;
  const int col = (int)(i % cols);
  if (bf) {
    const bf16* s = reinterpret_cast<const bf16*>(src);
    const bf16* g = reinterpret_cast<const bf16*>(gamma);
    reinterpret_cast<bf16*>(dst)[i] = (bf16)((float)s[i] * (float)g[col] * mul);
  } else {
    const float* s = reinterpret_cast<const float*>(src);
    const float* g = reinterpret_cast<const float*>(gamma);
    reinterpret_cast<float*>(dst)[i] = s[i] * g[col] * mul;
  }
}

// Wuk_t[h][cc][nn] = kv_b_proj[h (n + dv) + nn][cc]
// training cache: sequence b's page p is block b mbs + p
__global__ void identity_table_kernel(int32_t* bt, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) bt[i] = i;
}

// sparse lists: ent[b][j] = the cache entry of listed position idx[b][j] of
// sequence b, -1 when the position is outside [0, L_b) or its page unmapped
__global__ void sparse_entries_kernel(const int32_t* idx, int topk, const int32_t* seq_lens, int max_seq_len,
                                      const int32_t* block_table, int max_blocks, int num_blocks, int page,
                                      int32_t* ent) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x, b = blockIdx.y;
  if (j >= topk) return;
  const int64_t o = (int64_t)b * topk + j;
  const int p = idx[o];
  const int L = min(max(seq_lens[b], 0), max_seq_len);
  int e = -1;
  if (p >= 0 && p < L && p / page < max_blocks) {
    const int blk = block_table[(int64_t)b * max_blocks + p / page];
    if (blk >= 0 && blk < num_blocks) e = blk * page + p % page;
  }
  ent[o] = e;
}

// bf16 copy of the visible entries of an 8-bit cache (576 codes per entry):
// grid (mbs pages, batch); page p of sequence b goes to block b mbs + p of the
// copy, each code decoded (exact in bf16) and multiplied by the cache scale in
// fp32; entries at or past the sequence's length prefix + q_len, and unmapped
// pages, are zero. Also writes the copy's identity block table.
__global__ __launch_bounds__(256) void kv_shadow_kernel(const uint8_t* cache, const int32_t* block_table,
                                                        int max_blocks, int num_blocks, int page,
                                                        const int32_t* cu_seqlens, const int32_t* prefix_lens,
                                                        int mbs, float scale, bf16* shadow, int32_t* shadow_bt) {
  constexpr int CH = 36;  // 16-code chunks per entry
  const int p = blockIdx.x, b = blockIdx.y;
  const int L = prefix_lens[b] + cu_seqlens[b + 1] - cu_seqlens[b];
  const int blk = block_table[(int64_t)b * max_blocks + p];
  const bool mapped = blk >= 0 && blk < num_blocks;
  const int64_t dblk = (int64_t)b * mbs + p;
  if (threadIdx.x == 0) shadow_bt[dblk] = (int32_t)dblk;
  for (int i = threadIdx.x; i < page * CH; i += 256) {
    const int e = i / CH, ch = i % CH;
    uint4 w = {0u, 0u, 0u, 0u};
    if (mapped && p * page + e < L) w = *reinterpret_cast<const uint4*>(cache + ((int64_t)blk * page + e) * (CH * 16) + ch * 16);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    bf16x8 o[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[q] >> (16 * h), 1.0f, false);
        o[q >> 1][4 * (q & 1) + 2 * h] = (bf16)((float)d[0] * scale);
        o[q >> 1][4 * (q & 1) + 2 * h + 1] = (bf16)((float)d[1] * scale);
      }
    }
    bf16x8* dst = reinterpret_cast<bf16x8*>(shadow + ((dblk * page + e) * CH + ch) * 16);
    dst[0] = o[0];
    dst[1] = o[1];
  }
}

__global__ void wuk_transpose_kernel(const void* wkvb, void* out, int H, int n, int dv, int c, int bf) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)H * c * n;
  if (i >= total) return;
  const int nn = (int)(i % n);
  const int cc = (int)((i / n) % c);
  const int h = (int)(i / ((int64_t)n * c));
  const int64_t src = ((int64_t)h * (n + dv) + nn) * c + cc;
  if (bf) reinterpret_cast<bf16*>(out)[i] = reinterpret_cast<const bf16*>(wkvb)[src];
  else reinterpret_cast<float*>(out)[i] = reinterpret_cast<const float*>(wkvb)[src];
}

int dev_alloc(mla_ctx* ctx, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return MLA_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    return fail(MLA_ERR_OOM, "hipMalloc of " + std::to_string(bytes) + " bytes failed: " + hipGetErrorString(e));
  }
  ctx->allocs.push_back(*p);
  return MLA_OK;
}

void free_all(mla_ctx* ctx) {
  for (void* p : ctx->allocs) (void)hipFree(p);
  ctx->allocs.clear();
}

int validate_config(const mla_config* c, const mla_weights* w) {
  if (!c || !w) return fail(MLA_ERR_INVALID_ARG, "config and weights must not be NULL");
  if (c->hidden_size <= 0 || c->num_heads <= 0 || c->kv_lora_rank <= 0 || c->qk_nope_head_dim <= 0 ||
      c->qk_rope_head_dim <= 0 || c->v_head_dim <= 0 || c->q_lora_rank < 0)
    return fail(MLA_ERR_DIMS, "every model dimension must be positive (q_lora_rank >= 0)");
  if (c->qk_rope_head_dim % 2) return fail(MLA_ERR_DIMS, "qk_rope_head_dim must be even (RoPE rotates pairs)");
  if (c->dtype != MLA_DTYPE_F32 && c->dtype != MLA_DTYPE_BF16) return fail(MLA_ERR_INVALID_ARG, "unknown dtype");
  if (c->rope_style != MLA_ROPE_NEOX && c->rope_style != MLA_ROPE_INTERLEAVED)
    return fail(MLA_ERR_INVALID_ARG, "unknown rope_style");
  if (!(c->rope_theta > 1.0) || !std::isfinite(c->rope_theta)) return fail(MLA_ERR_INVALID_ARG, "rope_theta must be > 1");
  if (!(c->rms_norm_eps >= 0.0) || !std::isfinite(c->rms_norm_eps)) return fail(MLA_ERR_INVALID_ARG, "rms_norm_eps must be >= 0");
  if (!std::isfinite(c->softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (c->use_output_gate != 0 && c->use_output_gate != 1) return fail(MLA_ERR_INVALID_ARG, "use_output_gate must be 0 or 1");
  if (c->page_size <= 0 || c->max_batch <= 0 || c->max_tokens <= 0 || c->max_seq_len <= 0 || c->max_prefill_kv < 0 ||
      c->max_block_tokens < 0 || c->max_topk < 0)
    return fail(MLA_ERR_INVALID_ARG, "page_size, max_batch, max_tokens, max_seq_len must be positive, "
                                     "max_prefill_kv, max_block_tokens and max_topk >= 0");
  const int vec = c->dtype == MLA_DTYPE_BF16 ? 8 : 4;
  const int n = c->qk_nope_head_dim, r = c->qk_rope_head_dim, kc = c->kv_lora_rank, dv = c->v_head_dim;
  if (n % vec || r % vec || kc % vec || dv % vec || c->hidden_size % vec || (c->q_lora_rank % vec))
    return fail(MLA_ERR_UNSUPPORTED, "every dimension must be a multiple of 16 bytes of the dtype");
  if ((n + r) % 8 || (kc + r) % 8 || kc % 8)
    return fail(MLA_ERR_UNSUPPORTED, "n + r, c + r and c must be multiples of 8");
  if (n + r > 192 || dv > 128 || kc > 512 || kc + r > 576)
    return fail(MLA_ERR_UNSUPPORTED, "head dims above n + r = 192, dv = 128, c = 512, c + r = 576 are not supported");
  if (c->kv_cache_dtype != MLA_KV_CACHE_COMPUTE && c->kv_cache_dtype != MLA_KV_CACHE_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARG, "unknown kv_cache_dtype");
  if (c->kv_cache_dtype == MLA_KV_CACHE_FP8_E4M3) {
    if (!(c->kv_cache_scale > 0.f) || !std::isfinite(c->kv_cache_scale))
      return fail(MLA_ERR_INVALID_ARG, "kv_cache_scale must be > 0 and finite");
    if (c->dtype != MLA_DTYPE_BF16 || kc != 512 || r != 64 || c->num_heads > 128 || c->page_size % 32)
      return fail(MLA_ERR_UNSUPPORTED, "the 8-bit cache needs bf16, c = 512, r = 64, <= 128 heads and a page "
                                       "size that is a multiple of 32");
    if (c->max_batch > 1024)
      return fail(MLA_ERR_UNSUPPORTED, "the 8-bit cache decodes at most 1024 sequences per call (max_batch)");
  }
  if (!w->kv_a_proj_with_mqa || !w->kv_a_layernorm || !w->kv_b_proj || !w->o_proj)
    return fail(MLA_ERR_INVALID_ARG, "kv_a_proj_with_mqa, kv_a_layernorm, kv_b_proj and o_proj are required");
  if (c->q_lora_rank > 0 && (!w->q_a_proj || !w->q_a_layernorm || !w->q_b_proj))
    return fail(MLA_ERR_INVALID_ARG, "q_lora_rank > 0 needs q_a_proj, q_a_layernorm and q_b_proj");
  if (c->q_lora_rank == 0 && !w->q_proj) return fail(MLA_ERR_INVALID_ARG, "q_lora_rank == 0 needs q_proj");
  if (c->use_output_gate && !w->g_proj) return fail(MLA_ERR_INVALID_ARG, "use_output_gate needs g_proj");
  return MLA_OK;
}

int check_mask(int kind, int window) {
  if (kind != MLA_MASK_FULL && kind != MLA_MASK_CAUSAL && kind != MLA_MASK_SLIDING)
    return fail(MLA_ERR_INVALID_ARG, "unknown mask kind");
  if (kind == MLA_MASK_SLIDING && window < 0) return fail(MLA_ERR_INVALID_ARG, "window must be >= 0");
  return MLA_OK;
}

enum Stage { ST_QKV_A = 0, ST_Q_B, ST_ROPE_CACHE, ST_KV_B, ST_PREFILL_ATTN, ST_WUK, ST_DECODE_ATTN,
             ST_DECODE_MERGE, ST_WUV, ST_O_PROJ, ST_EXPAND_ATTN, ST_EXPAND_MERGE, ST_KV_DEQUANT, ST_BWD_ATTN,
             ST_BWD_GEMM, ST_BWD_WGRAD, ST_BWD_POINTWISE, ST_COUNT };
const char* kStageNames[ST_COUNT] = {"qkv_a_gemm", "q_b_gemm", "rope_cache", "kv_b_expand", "prefill_attn",
                                     "wuk_absorb", "decode_attn", "decode_merge", "wuv_gemm", "o_proj_gemm",
                                     "expand_attn", "expand_merge", "kv_dequant", "attn_bwd", "bwd_gemm",
                                     "wgrad_gemm", "bwd_pointwise"};

hipEvent_t pool_event(mla_ctx* ctx) {
  if (!ctx->event_pool.empty()) {
    hipEvent_t e = ctx->event_pool.back();
    ctx->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records a start event now and the stop event when it goes out of scope
// (only while profiling is on).
struct StageTimer {
  mla_ctx* ctx;
  hipStream_t s;
  int stage;
  hipEvent_t start = nullptr;
  StageTimer(mla_ctx* c, hipStream_t st, int sg) : ctx(c), s(st), stage(sg) {
    if (ctx->profiling && (start = pool_event(ctx)) != nullptr) (void)hipEventRecord(start, s);
  }
  ~StageTimer() {
    if (!start) return;
    hipEvent_t stop = pool_event(ctx);
    if (!stop) return;
    (void)hipEventRecord(stop, s);
    ctx->marks.push_back({stage, start, stop});
  }
};

// Records the context's completion event on the call's stream when the
// entry point returns (mla_free waits for it).
struct CallDone {
  mla_ctx* ctx;
  hipStream_t s;
  CallDone(mla_ctx* c, hipStream_t st) : ctx(c), s(st) {}
  ~CallDone() { (void)hipEventRecord(ctx->done, s); }
};

int run_gemm(mla_ctx* ctx, const Workspace& ws, const GemmArgs& g0, hipStream_t s) {
  GemmArgs g = g0;
  g.zeros = ctx->zeros;
  if (const char* m = gemm_check(g, ctx->bf16)) return fail(MLA_ERR_UNSUPPORTED, m);
  HIP_TRY(gemm_launch(g, ctx->bf16, ws.gemm_ws, ws.gemm_ws_elems, s));
  return MLA_OK;
}

// where project() leaves the roped-to-be query [T, H, n + r] and its row stride
void query_buffer(mla_ctx* ctx, const Workspace& ws, void** q, int64_t* ldq) {
  if (ctx->ql > 0) {
    *q = ws.qbuf;
    *ldq = (int64_t)ctx->H * ctx->qkh;
  } else {
    *q = static_cast<char*>(ws.buf1) + (size_t)ctx->off_q * ctx->esz;
    *ldq = ctx->N1;
  }
}

// fused first projection and (low-rank path) the q_b projection with the
// q_a RMSNorm folded into its epilogue; fills q / ldq
int project(mla_ctx* ctx, const Workspace& ws, const void* x, int T, hipStream_t s, void** q, int64_t* ldq,
            bool log2_q = false) {
  GemmArgs g1;
  g1.A = x; g1.lda = ctx->hid;
  g1.W = ctx->W1; g1.ldw = ctx->hid;
  g1.C = ws.buf1; g1.ldc = ctx->N1;
  g1.M = T; g1.N = ctx->N1; g1.K = ctx->hid;
  {
    StageTimer st(ctx, s, ST_QKV_A);
    if (int e = run_gemm(ctx, ws, g1, s)) return e;
  }
  if (ctx->ql > 0) {
    GemmArgs g2;
    g2.A = ws.buf1; g2.lda = ctx->N1;
    g2.W = log2_q ? ctx->Wqb_l2 : ctx->Wqb; g2.ldw = ctx->ql;
    g2.C = ws.qbuf; g2.ldc = (int64_t)ctx->H * ctx->qkh;
    g2.M = T; g2.N = ctx->H * ctx->qkh; g2.K = ctx->ql;
    g2.epi = EPI_ROWNORM; g2.eps = (float)ctx->cfg.rms_norm_eps;
    StageTimer st(ctx, s, ST_Q_B);
    if (int e = run_gemm(ctx, ws, g2, s)) return e;
  }
  query_buffer(ctx, ws, q, ldq);
  return MLA_OK;
}

// copies and transposed weights and the workspaces of mla_backward_expanded
int init_training(mla_ctx* ctx, const mla_weights* w, hipStream_t s) {
  const mla_config& cfg = ctx->cfg;
  auto& t = ctx->tr;
  const int H = ctx->H, esz = ctx->esz;
  const int64_t hid = ctx->hid, qkh = ctx->qkh, hdv = (int64_t)H * ctx->dv, kvbn = (int64_t)H * (ctx->n + ctx->dv);
  const int64_t Tm = cfg.max_train_tokens, Tp = (Tm + 63) / 64 * 64;
  if (cfg.max_prefill_kv <= 0) return fail(MLA_ERR_INVALID_ARG, "max_train_tokens > 0 needs max_prefill_kv > 0");
  t.Tm = (int)Tm;
  TrainArgs none;
  int e;
  auto alloc = [&](void** p, size_t bytes) { return dev_alloc(ctx, p, bytes); };
  auto transpose = [&](const void* src, int64_t rows, int64_t cols, void** dst) -> int {
    if (int e1 = alloc(dst, (size_t)rows * cols * esz)) return e1;
    if (train_transpose(src, cols, (int)rows, (int)cols, *dst, rows, none, false, ctx->bf16, s) != hipSuccess)
      return fail(MLA_ERR_HIP, "weight transpose failed");
    return MLA_OK;
  };
  if (ctx->ql > 0) {
    if ((e = alloc(&t.Wqb, (size_t)H * qkh * ctx->ql * esz))) return e;
    if ((e = alloc(&t.gamma_q, (size_t)ctx->ql * esz))) return e;
    if (hipMemcpyAsync(t.Wqb, w->q_b_proj, (size_t)H * qkh * ctx->ql * esz, hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipMemcpyAsync(t.gamma_q, w->q_a_layernorm, (size_t)ctx->ql * esz, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return fail(MLA_ERR_HIP, "q_b weight copy failed");
    if ((e = transpose(t.Wqb, H * qkh, ctx->ql, &t.WqbT))) return e;
  }
  if ((e = transpose(ctx->W1, ctx->N1, hid, &t.W1T))) return e;
  if ((e = transpose(ctx->Wkvb, kvbn, ctx->c, &t.WkvbT))) return e;
  if ((e = transpose(ctx->Wo, hid, hdv, &t.WoT))) return e;
  void* p;
  if ((e = alloc(&t.buf1, (size_t)Tm * ctx->N1 * esz))) return e;
  if (ctx->ql > 0) {
    if ((e = alloc(&t.qn, (size_t)Tm * ctx->ql * esz))) return e;
    if ((e = alloc(&t.q, (size_t)Tm * H * qkh * esz))) return e;
    if ((e = alloc(&p, (size_t)Tm * sizeof(float)))) return e;
    t.rho_q = static_cast<float*>(p);
  }
  if ((e = alloc(&p, (size_t)Tm * sizeof(float)))) return e;
  t.rho_kv = static_cast<float*>(p);
  if ((e = alloc(&t.cache, (size_t)cfg.max_prefill_kv * ctx->E * esz))) return e;
  const int64_t nbt = (int64_t)cfg.max_batch * ((cfg.max_seq_len + cfg.page_size - 1) / cfg.page_size + 1);
  if ((e = alloc(&p, (size_t)nbt * sizeof(int32_t)))) return e;
  t.bt = static_cast<int32_t*>(p);
  hipLaunchKernelGGL(identity_table_kernel, dim3((unsigned)((nbt + 255) / 256)), dim3(256), 0, s, t.bt, (int)nbt);
  if ((e = alloc(&p, (size_t)cfg.max_batch * sizeof(int32_t)))) return e;
  t.zero_prefix = static_cast<int32_t*>(p);
  if (hipMemsetAsync(t.zero_prefix, 0, (size_t)cfg.max_batch * sizeof(int32_t), s) != hipSuccess)
    return fail(MLA_ERR_HIP, "zero prefix init failed");
  if ((e = alloc(&t.O, (size_t)Tm * hdv * esz))) return e;
  if (ctx->off_g >= 0 && (e = alloc(&t.A, (size_t)Tm * hdv * esz))) return e;
  if ((e = alloc(&p, (size_t)Tm * H * sizeof(float)))) return e;
  t.lse = static_cast<float*>(p);
  if ((e = alloc(&t.dA, (size_t)Tm * hdv * esz))) return e;
  if ((e = alloc(&p, (size_t)Tm * H * sizeof(float)))) return e;
  t.D = static_cast<float*>(p);
  if ((e = alloc(&t.dkvb, (size_t)Tm * kvbn * esz))) return e;
  if ((e = alloc(&p, (size_t)Tm * H * ctx->r * sizeof(float)))) return e;
  t.dkr = static_cast<float*>(p);
  if ((e = alloc(&t.dQ, (size_t)Tm * H * qkh * esz))) return e;
  if ((e = alloc(&t.dcn, (size_t)Tm * ctx->c * esz))) return e;
  if (ctx->ql > 0 && (e = alloc(&t.dqn, (size_t)Tm * ctx->ql * esz))) return e;
  if ((e = alloc(&t.dbuf1, (size_t)Tm * ctx->N1 * esz))) return e;
  const int64_t maxA = std::max<int64_t>(std::max<int64_t>(hid, ctx->N1), std::max<int64_t>(kvbn, H * qkh));
  const int64_t maxB = std::max<int64_t>(std::max<int64_t>(hdv, ctx->c), ctx->ql);
  if ((e = alloc(&t.TX, (size_t)hid * Tp * esz))) return e;
  if ((e = alloc(&t.TA, (size_t)maxA * Tp * esz))) return e;
  if ((e = alloc(&t.TB, (size_t)maxB * Tp * esz))) return e;
  const int64_t cols = std::max<int64_t>(ctx->c, ctx->ql);
  if ((e = alloc(&p, (size_t)((Tm + 255) / 256) * cols * sizeof(float)))) return e;
  t.part = static_cast<float*>(p);
  if (hipGetLastError() != hipSuccess) return fail(MLA_ERR_HIP, "training set-up launch failed");
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_err.c_str(); }

int mla_init_weights(const mla_config* cfg, const mla_weights* w, void* stream, mla_ctx** out) {
  if (!out) return fail(MLA_ERR_INVALID_ARG, "out must not be NULL");
  *out = nullptr;
  if (int e = validate_config(cfg, w)) return e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  mla_ctx* ctx = new mla_ctx();
  ctx->cfg = *cfg;
  ctx->bf16 = cfg->dtype == MLA_DTYPE_BF16;
  ctx->esz = ctx->bf16 ? 2 : 4;
  ctx->H = cfg->num_heads; ctx->n = cfg->qk_nope_head_dim; ctx->r = cfg->qk_rope_head_dim;
  ctx->c = cfg->kv_lora_rank; ctx->dv = cfg->v_head_dim; ctx->ql = cfg->q_lora_rank;
  ctx->hid = cfg->hidden_size; ctx->E = ctx->c + ctx->r; ctx->qkh = ctx->n + ctx->r;
  ctx->scale = cfg->softmax_scale > 0 ? (float)cfg->softmax_scale : (float)(1.0 / std::sqrt((double)ctx->qkh));
  const int H = ctx->H, esz = ctx->esz;
  const int64_t hid = ctx->hid;

  auto bail = [&](int e) {
    free_all(ctx);
    if (ctx->done) (void)hipEventDestroy(ctx->done);
    delete ctx;
    return e;
  };
  if (hipGetDevice(&ctx->device) != hipSuccess) return bail(fail(MLA_ERR_HIP, "hipGetDevice failed"));
  if (hipEventCreateWithFlags(&ctx->done, hipEventDisableTiming) != hipSuccess) {
    ctx->done = nullptr;
    return bail(fail(MLA_ERR_HIP, "hipEventCreateWithFlags failed"));
  }
  if (int e = scratch_setup(ctx->device)) return bail(e);

  // fused first projection rows: [q_a_proj | q_proj] ; kv_a_proj_with_mqa ; g_proj
  const int nq = ctx->ql > 0 ? ctx->ql : H * ctx->qkh;
  ctx->off_q = 0;
  ctx->off_kv = nq;
  ctx->N1 = nq + ctx->E;
  if (cfg->use_output_gate) {
    ctx->off_g = ctx->N1;
    ctx->N1 += H * ctx->dv;
  }
  int e;
  if ((e = dev_alloc(ctx, &ctx->W1, (size_t)ctx->N1 * hid * esz))) return bail(e);
  {
    char* dst = static_cast<char*>(ctx->W1);
    const void* qsrc = ctx->ql > 0 ? w->q_a_proj : w->q_proj;
    if (hipMemcpyAsync(dst, qsrc, (size_t)nq * hid * esz, hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipMemcpyAsync(dst + (size_t)ctx->off_kv * hid * esz, w->kv_a_proj_with_mqa, (size_t)ctx->E * hid * esz,
                       hipMemcpyDeviceToDevice, s) != hipSuccess ||
        (cfg->use_output_gate &&
         hipMemcpyAsync(dst + (size_t)ctx->off_g * hid * esz, w->g_proj, (size_t)H * ctx->dv * hid * esz,
                        hipMemcpyDeviceToDevice, s) != hipSuccess))
      return bail(fail(MLA_ERR_HIP, "copy of the first projection weights failed"));
  }
  if (ctx->ql > 0) {
    const int64_t rows = (int64_t)H * ctx->qkh;
    if ((e = dev_alloc(ctx, &ctx->Wqb, (size_t)rows * ctx->ql * esz))) return bail(e);
    const int64_t tot = rows * ctx->ql;
    hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, w->q_b_proj,
                       w->q_a_layernorm, ctx->Wqb, rows, ctx->ql, (int)ctx->bf16, 1.f);
    if (hipGetLastError() != hipSuccess) return bail(fail(MLA_ERR_HIP, "q_b_proj repack failed"));
    // the bf16 prefill attention kernels (the conditions under which
    // prefill_attn_launch and the fused kernel take them) get queries already
    // multiplied by scale * log2(e) (one rounding, as for the folded gain):
    // the q_b projection of the prefill uses this copy
    if (ctx->bf16 && ctx->n == 128 && ctx->r == 64 && ctx->dv == 128 && ctx->c % 8 == 0 && cfg->page_size % 64 == 0) {
      if ((e = dev_alloc(ctx, &ctx->Wqb_l2, (size_t)rows * ctx->ql * esz))) return bail(e);
      hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, w->q_b_proj,
                         w->q_a_layernorm, ctx->Wqb_l2, rows, ctx->ql, (int)ctx->bf16, ctx->scale * 1.4426950408889634f);
      if (hipGetLastError() != hipSuccess) return bail(fail(MLA_ERR_HIP, "q_b_proj repack failed"));
    }
  }
  const int64_t kvb_rows = (int64_t)H * (ctx->n + ctx->dv);
  if ((e = dev_alloc(ctx, &ctx->Wkvb, (size_t)kvb_rows * ctx->c * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->Wuk_t, (size_t)H * ctx->c * ctx->n * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->Wo, (size_t)hid * H * ctx->dv * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->gamma_kv, (size_t)ctx->c * esz))) return bail(e);
  if (hipMemcpyAsync(ctx->Wkvb, w->kv_b_proj, (size_t)kvb_rows * ctx->c * esz, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(ctx->Wo, w->o_proj, (size_t)hid * H * ctx->dv * esz, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      hipMemcpyAsync(ctx->gamma_kv, w->kv_a_layernorm, (size_t)ctx->c * esz, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return bail(fail(MLA_ERR_HIP, "weight copy failed"));
  {
    const int64_t tot = (int64_t)H * ctx->c * ctx->n;
    hipLaunchKernelGGL(wuk_transpose_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, w->kv_b_proj,
                       ctx->Wuk_t, H, ctx->n, ctx->dv, ctx->c, (int)ctx->bf16);
    if (hipGetLastError() != hipSuccess) return bail(fail(MLA_ERR_HIP, "W_UK repack failed"));
  }

  // RoPE table: fp64 angles rounded once to fp32 cos/sin
  {
    const int half = ctx->r / 2;
    const size_t cnt = (size_t)cfg->max_seq_len * half;
    std::vector<float> hc(cnt), hs(cnt);
    for (int p = 0; p < cfg->max_seq_len; ++p)
      for (int j = 0; j < half; ++j) {
        const double ang = (double)p * std::pow(cfg->rope_theta, -2.0 * j / (double)ctx->r);
        hc[(size_t)p * half + j] = (float)std::cos(ang);
        hs[(size_t)p * half + j] = (float)std::sin(ang);
      }
    void *pc, *ps;
    if ((e = dev_alloc(ctx, &pc, cnt * sizeof(float)))) return bail(e);
    if ((e = dev_alloc(ctx, &ps, cnt * sizeof(float)))) return bail(e);
    ctx->rope_cos = static_cast<float*>(pc);
    ctx->rope_sin = static_cast<float*>(ps);
    if (hipMemcpyAsync(pc, hc.data(), cnt * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipMemcpyAsync(ps, hs.data(), cnt * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess)
      return bail(fail(MLA_ERR_HIP, "RoPE table upload failed"));
    // the host vectors must outlive the asynchronous copies
    if (hipStreamSynchronize(s) != hipSuccess) return bail(fail(MLA_ERR_HIP, "stream synchronize failed"));
  }

  // workspaces
  const int64_t T = cfg->max_tokens, B = cfg->max_batch;
  if ((e = dev_alloc(ctx, &ctx->ws.buf1, (size_t)T * ctx->N1 * esz))) return bail(e);
  if (ctx->ql > 0 && (e = dev_alloc(ctx, &ctx->ws.qbuf, (size_t)T * H * ctx->qkh * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->kvexp, (size_t)cfg->max_prefill_kv * kvb_rows * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->ws.attn, (size_t)T * H * ctx->dv * esz))) return bail(e);
  const int64_t QR = std::max<int64_t>(B, cfg->max_block_tokens);  // latent query / output rows
  if ((e = dev_alloc(ctx, &ctx->ws.qlat, (size_t)QR * H * ctx->c * esz))) return bail(e);
  if ((e = dev_alloc(ctx, &ctx->ws.olat, (size_t)QR * H * ctx->c * esz))) return bail(e);
  void* p;
  if (cfg->max_topk > 0) {
    if ((e = dev_alloc(ctx, &p, (size_t)B * cfg->max_topk * sizeof(int32_t)))) return bail(e);
    ctx->ws.sp_ent = static_cast<int32_t*>(p);
  }
  if (hipDeviceGetAttribute(&ctx->cus, hipDeviceAttributeMultiprocessorCount, ctx->device) != hipSuccess ||
      ctx->cus <= 0)
    return bail(fail(MLA_ERR_HIP, "querying the compute-unit count failed"));
  ctx->sk_shape = ctx->bf16 && ctx->c == 512 && ctx->r == 64 && H <= 128 && cfg->page_size % 32 == 0;
  // decode partials: stream-K pieces [2 ranges, H, c] for batches it covers,
  // per-split partials [B, splits, H, c] otherwise
  int64_t part_rows = 0;
  if (ctx->sk_shape) {
    // decode sequences, and the virtual sequences of query blocks (128
    // (query, head) pairs each)
    const int64_t vb = (int64_t)cfg->max_block_tokens * H / 128;
    const int skb = (int)std::min<int64_t>(std::max<int64_t>(B, vb), kDecodeMaxBatch);
    ctx->sk_max_ranges = decode_sk_ranges(skb, std::max(cfg->max_seq_len, cfg->max_topk), ctx->cus);
    part_rows = 2 * (int64_t)ctx->sk_max_ranges;
    if ((e = dev_alloc(ctx, &p, (size_t)(skb + 1) * sizeof(int32_t)))) return bail(e);
    ctx->ws.sk_tstart = static_cast<int32_t*>(p);
  }
  if (!ctx->sk_shape || B > kDecodeMaxBatch) part_rows = std::max<int64_t>(part_rows, B * ctx->max_splits);
  // partial rows hold every head of a (virtual) sequence: query blocks run
  // with 128 (query, head) pairs per virtual sequence
  const int64_t part_heads = cfg->max_block_tokens > 0 ? std::max(H, 128) : H;
  if ((e = dev_alloc(ctx, &p, (size_t)part_rows * part_heads * ctx->c * sizeof(float)))) return bail(e);
  ctx->ws.part_o = static_cast<float*>(p);
  if ((e = dev_alloc(ctx, &p, (size_t)part_rows * part_heads * sizeof(float)))) return bail(e);
  ctx->ws.part_lse = static_cast<float*>(p);
  // (training: the split-K partials of the weight and data gradients, e.g.
  // 3 x 6144 x 1536 or 4 x 8192 x 1536 floats at the draft-block dims)
  ctx->ws.gemm_ws_elems = cfg->max_train_tokens > 0 ? (int64_t)56 << 20 : (int64_t)16 << 20;
  if ((e = dev_alloc(ctx, &p, (size_t)ctx->ws.gemm_ws_elems * sizeof(float)))) return bail(e);
  ctx->ws.gemm_ws = static_cast<float*>(p);
  if ((e = dev_alloc(ctx, &ctx->zeros, 256))) return bail(e);
  if (hipMemsetAsync(ctx->zeros, 0, 256, s) != hipSuccess) return bail(fail(MLA_ERR_HIP, "zero page init failed"));
  ctx->kv_fp8 = cfg->kv_cache_dtype == MLA_KV_CACHE_FP8_E4M3;
  ctx->kv_scale = ctx->kv_fp8 ? cfg->kv_cache_scale : 1.f;
  if (ctx->kv_fp8 && cfg->max_prefill_kv > 0) {
    // per sequence, max_kv_len rounded up to whole pages
    const int64_t rows = (int64_t)cfg->max_prefill_kv + B * cfg->page_size;
    const int64_t mbs = (cfg->max_seq_len + cfg->page_size - 1) / cfg->page_size;
    if ((e = dev_alloc(ctx, &ctx->kv_shadow, (size_t)rows * ctx->E * 2))) return bail(e);
    if ((e = dev_alloc(ctx, &p, (size_t)B * mbs * sizeof(int32_t)))) return bail(e);
    ctx->kv_shadow_bt = static_cast<int32_t*>(p);
  }

  if (cfg->max_train_tokens > 0) {
    if (int e2 = init_training(ctx, w, s)) return bail(e2);
  }

  if (hipStreamSynchronize(s) != hipSuccess) return bail(fail(MLA_ERR_HIP, "stream synchronize failed"));
  *out = ctx;
  return MLA_OK;
}

int mla_prefill_expanded(mla_ctx* ctx, const void* x, int32_t batch, int32_t total_tokens,
                         const int32_t* cu_seqlens_q, const int32_t* prefix_lens, int32_t max_q_len,
                         int32_t max_kv_len, void* kv_cache, int32_t num_blocks, const int32_t* block_table,
                         int32_t max_blocks, int32_t mask_kind, int32_t window, const int32_t* row_lo,
                         const int32_t* row_hi, void* out, void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (!x || !cu_seqlens_q || !prefix_lens || !kv_cache || !block_table || !out)
    return fail(MLA_ERR_INVALID_ARG, "x, cu_seqlens_q, prefix_lens, kv_cache, block_table and out must not be NULL");
  if (batch <= 0 || total_tokens <= 0 || max_q_len <= 0 || max_kv_len <= 0 || num_blocks <= 0 || max_blocks <= 0)
    return fail(MLA_ERR_INVALID_ARG, "batch, total_tokens, max_q_len, max_kv_len, num_blocks, max_blocks must be positive");
  if ((row_lo == nullptr) != (row_hi == nullptr)) return fail(MLA_ERR_INVALID_ARG, "row_lo and row_hi go together");
  if (int e = check_mask(mask_kind, window)) return e;
  const mla_config& c = ctx->cfg;
  if (max_q_len > total_tokens || max_kv_len < max_q_len)
    return fail(MLA_ERR_INVALID_ARG, "need max_q_len <= total_tokens and max_kv_len >= max_q_len");
  if (batch > c.max_batch || total_tokens > c.max_tokens || max_kv_len > c.max_seq_len)
    return fail(MLA_ERR_CAPACITY, "batch, total_tokens or max_kv_len above the init limits");
  if ((int64_t)batch * max_kv_len > c.max_prefill_kv)
    return fail(MLA_ERR_CAPACITY, "batch * max_kv_len exceeds max_prefill_kv");
  if ((int64_t)max_blocks * c.page_size < max_kv_len)
    return fail(MLA_ERR_INVALID_ARG, "max_blocks * page_size must cover max_kv_len");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  CallDone call_done(ctx, s);
  const Workspace& ws = ctx->ws;

  void* q;
  int64_t ldq;
  // queries multiplied by scale * log2(e) when the bf16 attention kernels run
  const bool log2_q = ctx->Wqb_l2 != nullptr;
  if (int e = project(ctx, ws, x, total_tokens, s, &q, &ldq, log2_q)) return e;

  RopeCacheArgs rc;
  rc.q = q; rc.ldq = ldq; rc.qk_head = ctx->qkh;
  rc.kv = static_cast<char*>(ws.buf1) + (size_t)ctx->off_kv * ctx->esz; rc.ldkv = ctx->N1;
  rc.gamma_kv = ctx->gamma_kv;
  rc.cache = kv_cache; rc.block_table = block_table;
  rc.num_blocks = num_blocks; rc.max_blocks = max_blocks; rc.page = c.page_size;
  rc.rope_cos = ctx->rope_cos; rc.rope_sin = ctx->rope_sin;
  rc.H = ctx->H; rc.n = ctx->n; rc.r = ctx->r; rc.c = ctx->c;
  rc.interleaved = c.rope_style == MLA_ROPE_INTERLEAVED;
  rc.eps = (float)c.rms_norm_eps;
  rc.kv_fp8 = ctx->kv_fp8; rc.kv_scale = ctx->kv_scale;
  rc.decode = 0; rc.cu_seqlens = cu_seqlens_q; rc.prefix_lens = prefix_lens;
  rc.max_q_len = max_q_len; rc.max_kv_len = max_kv_len; rc.max_seq_len = c.max_seq_len;
  rc.total_tokens = total_tokens;
  {
    StageTimer st(ctx, s, ST_ROPE_CACHE);
    HIP_TRY(rope_cache_launch(rc, ctx->bf16, max_q_len, batch, s));
  }

  // an 8-bit cache: the attention reads a bf16 copy of the visible entries
  const void* acache = kv_cache;
  const int32_t* abt = block_table;
  int anb = num_blocks, amb = max_blocks;
  if (ctx->kv_fp8) {
    const int mbs = (max_kv_len + c.page_size - 1) / c.page_size;
    StageTimer st(ctx, s, ST_KV_DEQUANT);
    hipLaunchKernelGGL(kv_shadow_kernel, dim3(mbs, batch), dim3(256), 0, s, static_cast<const uint8_t*>(kv_cache),
                       block_table, max_blocks, num_blocks, c.page_size, cu_seqlens_q, prefix_lens, mbs,
                       ctx->kv_scale, static_cast<bf16*>(ctx->kv_shadow), ctx->kv_shadow_bt);
    HIP_TRY(hipGetLastError());
    acache = ctx->kv_shadow; abt = ctx->kv_shadow_bt;
    anb = batch * mbs; amb = mbs;
  }

  // few new tokens per sequence: the expansion is fused into the attention
  // (the expanded keys and values stay in registers; partial outputs per
  // 256-entry chunk live in the expansion buffer, which this form does not use)
  MhaFusedArgs fa;
  fa.q = q; fa.ldq = ldq; fa.qk_head = ctx->qkh;
  fa.cache = acache; fa.block_table = abt;
  fa.num_blocks = anb; fa.max_blocks = amb; fa.page = c.page_size;
  fa.wkvb = ctx->Wkvb;
  fa.cu_seqlens = cu_seqlens_q; fa.prefix_lens = prefix_lens;
  fa.batch = batch; fa.max_q_len = max_q_len; fa.max_kv_len = max_kv_len; fa.total_tokens = total_tokens;
  fa.H = ctx->H; fa.scale = ctx->scale; fa.q_log2 = log2_q;
  fa.mask.kind = mask_kind; fa.mask.window = window; fa.mask.row_lo = row_lo; fa.mask.row_hi = row_hi;
  fa.nchunks = (max_kv_len + 255) / 256;
  fa.qblocks = (max_q_len + 15) / 16;
  fa.out = ws.attn; fa.ldo = (int64_t)ctx->H * ctx->dv;
  if (ctx->off_g >= 0) {
    fa.gate = static_cast<char*>(ws.buf1) + (size_t)ctx->off_g * ctx->esz;
    fa.ldg = ctx->N1;
  }
  const size_t part_bytes = mha_fused_partial_bytes(batch, fa.nchunks, fa.qblocks, ctx->H);
  const size_t exp_bytes = (size_t)c.max_prefill_kv * ctx->H * (ctx->n + ctx->dv) * ctx->esz;
  const bool fused_shape = ctx->bf16 && ctx->c == 512 && ctx->n == 128 && ctx->r == 64 && ctx->dv == 128 &&
                           max_q_len <= kMhaFusedMaxQ && part_bytes <= exp_bytes;
  if (fused_shape) {
    fa.part_o = static_cast<bf16_t*>(ctx->kvexp);
    fa.part_lse = reinterpret_cast<float*>(static_cast<char*>(ctx->kvexp) +
                                           (((size_t)batch * fa.nchunks * fa.qblocks * ctx->H * 16 * 128 * 2 + 255) &
                                            ~(size_t)255));
  }
  if (fused_shape && mha_fused_check(fa) == nullptr) {
    {
      StageTimer st(ctx, s, ST_EXPAND_ATTN);
      HIP_TRY(mha_fused_launch(fa, s));
    }
    {
      StageTimer st(ctx, s, ST_EXPAND_MERGE);
      HIP_TRY(mha_fused_merge_launch(fa, s));
    }
    GemmArgs go;
    go.A = ws.attn; go.lda = (int64_t)ctx->H * ctx->dv;
    go.W = ctx->Wo; go.ldw = (int64_t)ctx->H * ctx->dv;
    go.C = out; go.ldc = ctx->hid;
    go.M = total_tokens; go.N = ctx->hid; go.K = ctx->H * ctx->dv;
    StageTimer st(ctx, s, ST_O_PROJ);
    return run_gemm(ctx, ws, go, s);
  }

  // expand every visible latent (prefix and new) through kv_b_proj
  GemmArgs gk;
  gk.gather = true;
  gk.ga.cache = acache; gk.ga.block_table = abt; gk.ga.cu_seqlens = cu_seqlens_q;
  gk.ga.prefix_lens = prefix_lens; gk.ga.batch = batch; gk.ga.max_kv_len = max_kv_len;
  gk.ga.page = c.page_size; gk.ga.max_blocks = amb; gk.ga.num_blocks = anb;
  gk.ga.entry = ctx->E; gk.ga.max_q_len = max_q_len;
  gk.A = acache; gk.lda = ctx->E;
  gk.W = ctx->Wkvb; gk.ldw = ctx->c;
  gk.C = ctx->kvexp; gk.ldc = (int64_t)ctx->H * (ctx->n + ctx->dv);
  gk.M = batch * max_kv_len; gk.N = ctx->H * (ctx->n + ctx->dv); gk.K = ctx->c;
  {
    StageTimer st(ctx, s, ST_KV_B);
    if (int e = run_gemm(ctx, ws, gk, s)) return e;
  }

  PrefillAttnArgs pa;
  pa.q = q; pa.ldq = ldq; pa.qk_head = ctx->qkh;
  pa.kv = ctx->kvexp; pa.ldkv = (int64_t)ctx->H * (ctx->n + ctx->dv);
  pa.cache = acache; pa.block_table = abt;
  pa.num_blocks = anb; pa.max_blocks = amb; pa.page = c.page_size;
  pa.cu_seqlens = cu_seqlens_q; pa.prefix_lens = prefix_lens;
  pa.batch = batch; pa.max_q_len = max_q_len; pa.max_kv_len = max_kv_len; pa.total_tokens = total_tokens;
  pa.H = ctx->H; pa.n = ctx->n; pa.r = ctx->r; pa.c = ctx->c; pa.dv = ctx->dv;
  pa.scale = ctx->scale; pa.q_log2 = log2_q;
  pa.mask.kind = mask_kind; pa.mask.window = window; pa.mask.row_lo = row_lo; pa.mask.row_hi = row_hi;
  pa.out = ws.attn; pa.ldo = (int64_t)ctx->H * ctx->dv;
  if (ctx->off_g >= 0) {
    pa.gate = static_cast<char*>(ws.buf1) + (size_t)ctx->off_g * ctx->esz;
    pa.ldg = ctx->N1;
  }
  if (const char* m = prefill_attn_check(pa, ctx->bf16)) return fail(MLA_ERR_UNSUPPORTED, m);
  {
    StageTimer st(ctx, s, ST_PREFILL_ATTN);
    HIP_TRY(prefill_attn_launch(pa, ctx->bf16, s));
  }

  GemmArgs go;
  go.A = ws.attn; go.lda = (int64_t)ctx->H * ctx->dv;
  go.W = ctx->Wo; go.ldw = (int64_t)ctx->H * ctx->dv;
  go.C = out; go.ldc = ctx->hid;
  go.M = total_tokens; go.N = ctx->hid; go.K = ctx->H * ctx->dv;
  StageTimer st(ctx, s, ST_O_PROJ);
  return run_gemm(ctx, ws, go, s);
}

int mla_backward_expanded(mla_ctx* ctx, const void* x, int32_t batch, int32_t total_tokens,
                          const int32_t* cu_seqlens_q, int32_t max_q_len, int32_t mask_kind, int32_t window,
                          const int32_t* row_lo, const int32_t* row_hi, const void* dout, void* dx,
                          const mla_grads* grads, void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (!x || !cu_seqlens_q || !dout || !dx || !grads)
    return fail(MLA_ERR_INVALID_ARG, "x, cu_seqlens_q, dout, dx and grads must not be NULL");
  if (batch <= 0 || total_tokens <= 0 || max_q_len <= 0)
    return fail(MLA_ERR_INVALID_ARG, "batch, total_tokens and max_q_len must be positive");
  if ((row_lo == nullptr) != (row_hi == nullptr)) return fail(MLA_ERR_INVALID_ARG, "row_lo and row_hi go together");
  if (int e = check_mask(mask_kind, window)) return e;
  const mla_config& c = ctx->cfg;
  auto& tr = ctx->tr;
  if (tr.Tm == 0) return fail(MLA_ERR_CAPACITY, "the context was created with max_train_tokens = 0");
  if (max_q_len > total_tokens) return fail(MLA_ERR_INVALID_ARG, "need max_q_len <= total_tokens");
  const int Lp = (max_q_len + c.page_size - 1) / c.page_size * c.page_size;
  if (batch > c.max_batch || total_tokens > tr.Tm || max_q_len > c.max_seq_len ||
      (int64_t)batch * Lp > c.max_prefill_kv)
    return fail(MLA_ERR_CAPACITY, "batch, total_tokens, max_q_len or batch * padded max_q_len above the init limits");
  const int H = ctx->H, esz = ctx->esz;
  const int64_t hid = ctx->hid, qkh = ctx->qkh, hdv = (int64_t)H * ctx->dv, kvbn = (int64_t)H * (ctx->n + ctx->dv);
  const int T = total_tokens;
  const int64_t Tp = ((int64_t)T + 63) / 64 * 64;
  const int mbs = Lp / c.page_size;
  const bool bf = ctx->bf16;

  TrainArgs ta;
  ta.cu_seqlens = cu_seqlens_q; ta.batch = batch; ta.max_q_len = max_q_len; ta.total_tokens = T; ta.Lp = Lp;
  ta.H = H; ta.n = ctx->n; ta.r = ctx->r; ta.c = ctx->c; ta.dv = ctx->dv; ta.q_lora = ctx->ql;
  ta.scale = ctx->scale; ta.eps = (float)c.rms_norm_eps;
  ta.mask.kind = mask_kind; ta.mask.window = window; ta.mask.row_lo = row_lo; ta.mask.row_hi = row_hi;
  ta.rope_cos = ctx->rope_cos; ta.rope_sin = ctx->rope_sin; ta.interleaved = c.rope_style == MLA_ROPE_INTERLEAVED;
  if (ctx->ql > 0) { ta.q = tr.q; ta.ldq = H * qkh; }
  else { ta.q = static_cast<char*>(tr.buf1) + (size_t)ctx->off_q * esz; ta.ldq = ctx->N1; }
  ta.cache = tr.cache; ta.kvexp = ctx->kvexp; ta.ldkv = kvbn;
  ta.O = tr.O; ta.A = tr.A ? tr.A : tr.O; ta.lse = tr.lse;
  ta.buf1 = tr.buf1; ta.ldb1 = ctx->N1; ta.off_q = ctx->off_q; ta.off_kv = ctx->off_kv; ta.off_g = ctx->off_g;
  if (ctx->off_g >= 0) { ta.gate = static_cast<char*>(tr.buf1) + (size_t)ctx->off_g * esz; ta.ldg = ctx->N1; }
  ta.gamma_kv = ctx->gamma_kv; ta.gamma_q = tr.gamma_q; ta.rho_q = tr.rho_q; ta.rho_kv = tr.rho_kv;
  ta.dO = tr.dA; ta.ldo = hdv; ta.D = tr.D;
  ta.dkvb = tr.dkvb; ta.lddkvb = kvbn; ta.dkr = tr.dkr; ta.dQ = tr.dQ; ta.lddq = H * qkh;
  ta.dcn = tr.dcn; ta.dqn = tr.dqn; ta.dbuf1 = tr.dbuf1; ta.lddb1 = ctx->N1;
  if (const char* m = train_check(ta, bf)) return fail(MLA_ERR_UNSUPPORTED, m);

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  CallDone call_done(ctx, s);
  const Workspace& ws = ctx->ws;
  auto gemm = [&](const void* A, int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc, int M, int N,
                  int K) -> int {
    GemmArgs g;
    g.A = A; g.lda = lda; g.W = W; g.ldw = ldw; g.C = C; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
    return run_gemm(ctx, ws, g, s);
  };
  auto at = [&](void* base, int64_t off_elems) { return static_cast<void*>(static_cast<char*>(base) + off_elems * esz); };

  // ---- forward, keeping what the backward reads
  {
    StageTimer st(ctx, s, ST_QKV_A);
    if (int e = gemm(x, hid, ctx->W1, hid, tr.buf1, ctx->N1, T, ctx->N1, (int)hid)) return e;
  }
  if (ctx->ql > 0) {
    StageTimer st(ctx, s, ST_Q_B);
    HIP_TRY(train_rmsnorm_rows(tr.buf1, ctx->N1, tr.gamma_q, ctx->ql, (float)c.rms_norm_eps, tr.qn, ctx->ql,
                               tr.rho_q, T, bf, s));
    if (int e = gemm(tr.qn, ctx->ql, tr.Wqb, ctx->ql, tr.q, H * qkh, T, (int)(H * qkh), ctx->ql)) return e;
  }
  RopeCacheArgs rc;
  rc.q = const_cast<void*>(ta.q); rc.ldq = ta.ldq; rc.qk_head = ctx->qkh;
  rc.kv = at(tr.buf1, ctx->off_kv); rc.ldkv = ctx->N1;
  rc.gamma_kv = ctx->gamma_kv;
  rc.cache = tr.cache; rc.block_table = tr.bt;
  rc.num_blocks = batch * mbs; rc.max_blocks = mbs; rc.page = c.page_size;
  rc.rope_cos = ctx->rope_cos; rc.rope_sin = ctx->rope_sin;
  rc.H = H; rc.n = ctx->n; rc.r = ctx->r; rc.c = ctx->c;
  rc.interleaved = c.rope_style == MLA_ROPE_INTERLEAVED;
  rc.eps = (float)c.rms_norm_eps;
  rc.decode = 0; rc.cu_seqlens = cu_seqlens_q; rc.prefix_lens = tr.zero_prefix;
  rc.max_q_len = max_q_len; rc.max_kv_len = Lp; rc.max_seq_len = c.max_seq_len; rc.total_tokens = T;
  {
    StageTimer st(ctx, s, ST_ROPE_CACHE);
    HIP_TRY(rope_cache_launch(rc, bf, max_q_len, batch, s));
  }
  {
    StageTimer st(ctx, s, ST_KV_B);
    GemmArgs gk;
    gk.gather = true;
    gk.ga.cache = tr.cache; gk.ga.block_table = tr.bt; gk.ga.cu_seqlens = cu_seqlens_q;
    gk.ga.prefix_lens = tr.zero_prefix; gk.ga.batch = batch; gk.ga.max_kv_len = Lp;
    gk.ga.page = c.page_size; gk.ga.max_blocks = mbs; gk.ga.num_blocks = batch * mbs;
    gk.ga.entry = ctx->E; gk.ga.max_q_len = max_q_len;
    gk.A = tr.cache; gk.lda = ctx->E;
    gk.W = ctx->Wkvb; gk.ldw = ctx->c;
    gk.C = ctx->kvexp; gk.ldc = kvbn;
    gk.M = batch * Lp; gk.N = (int)kvbn; gk.K = ctx->c;
    if (int e = run_gemm(ctx, ws, gk, s)) return e;
  }
  {
    PrefillAttnArgs pa;
    pa.q = ta.q; pa.ldq = ta.ldq; pa.qk_head = ctx->qkh;
    pa.kv = ctx->kvexp; pa.ldkv = kvbn;
    pa.cache = tr.cache; pa.block_table = tr.bt;
    pa.num_blocks = batch * mbs; pa.max_blocks = mbs; pa.page = c.page_size;
    pa.cu_seqlens = cu_seqlens_q; pa.prefix_lens = tr.zero_prefix;
    pa.batch = batch; pa.max_q_len = max_q_len; pa.max_kv_len = Lp; pa.total_tokens = T;
    pa.H = H; pa.n = ctx->n; pa.r = ctx->r; pa.c = ctx->c; pa.dv = ctx->dv;
    pa.scale = ctx->scale;
    pa.mask.kind = mask_kind; pa.mask.window = window; pa.mask.row_lo = row_lo; pa.mask.row_hi = row_hi;
    pa.out = tr.O; pa.ldo = hdv;
    pa.lse = tr.lse;
    if (const char* m = prefill_attn_check(pa, bf)) return fail(MLA_ERR_UNSUPPORTED, m);
    StageTimer st(ctx, s, ST_PREFILL_ATTN);
    HIP_TRY(prefill_attn_launch(pa, bf, s));
  }
  if (tr.A) {
    StageTimer st(ctx, s, ST_BWD_POINTWISE);
    HIP_TRY(train_gate_fwd(ta, bf, s));
  }

  // ---- backward
  {
    StageTimer st(ctx, s, ST_BWD_GEMM);
    if (int e = gemm(dout, hid, tr.WoT, hid, tr.dA, hdv, T, (int)hdv, (int)hid)) return e;
  }
  {
    StageTimer st(ctx, s, ST_BWD_POINTWISE);
    HIP_TRY(train_gate_bwd(ta, bf, s));
  }
  {
    StageTimer st(ctx, s, ST_BWD_ATTN);
    HIP_TRY(train_attn_bwd(ta, bf, s));
  }
  {
    StageTimer st(ctx, s, ST_BWD_GEMM);
    if (int e = gemm(tr.dkvb, kvbn, tr.WkvbT, kvbn, tr.dcn, ctx->c, T, ctx->c, (int)kvbn)) return e;
  }
  {
    StageTimer st(ctx, s, ST_BWD_POINTWISE);
    HIP_TRY(train_kv_bwd(ta, bf, s));
    if (grads->kv_a_layernorm)
      HIP_TRY(train_gamma_grad(tr.dcn, ctx->c, at(tr.buf1, ctx->off_kv), ctx->N1, tr.rho_kv, T, ctx->c, tr.part,
                               grads->kv_a_layernorm, bf, s));
    HIP_TRY(train_q_rope_bwd(ta, bf, s));
  }
  if (ctx->ql > 0) {
    {
      StageTimer st(ctx, s, ST_BWD_GEMM);
      if (int e = gemm(tr.dQ, H * qkh, tr.WqbT, H * qkh, tr.dqn, ctx->ql, T, ctx->ql, (int)(H * qkh))) return e;
    }
    StageTimer st(ctx, s, ST_BWD_POINTWISE);
    HIP_TRY(train_q_norm_bwd(ta, bf, s));
    if (grads->q_a_layernorm)
      HIP_TRY(train_gamma_grad(tr.dqn, ctx->ql, tr.buf1, ctx->N1, tr.rho_q, T, ctx->ql, tr.part, grads->q_a_layernorm,
                               bf, s));
  }
  {
    StageTimer st(ctx, s, ST_BWD_GEMM);
    if (int e = gemm(tr.dbuf1, ctx->N1, tr.W1T, ctx->N1, dx, hid, T, (int)hid, ctx->N1)) return e;
  }
  StageTimer st_w(ctx, s, ST_BWD_WGRAD);

  // ---- weight gradients: dW = dY^T X over the token axis, on transposed copies
  auto tpose = [&](const void* src, int64_t lds, int cols, void* dst, bool map) {
    return train_transpose(src, lds, T, cols, dst, Tp, ta, map, bf, s);
  };
  if (grads->o_proj) {
    HIP_TRY(tpose(dout, hid, (int)hid, tr.TA, false));
    HIP_TRY(tpose(ta.A, hdv, (int)hdv, tr.TB, false));
    if (int e = gemm(tr.TA, Tp, tr.TB, Tp, grads->o_proj, hdv, (int)hid, (int)hdv, (int)Tp)) return e;
  }
  if (grads->q_a_proj || grads->q_proj || grads->kv_a_proj_with_mqa || grads->g_proj) {
    HIP_TRY(tpose(x, hid, (int)hid, tr.TX, false));
    HIP_TRY(tpose(tr.dbuf1, ctx->N1, ctx->N1, tr.TA, false));
    void* gq = ctx->ql > 0 ? grads->q_a_proj : grads->q_proj;
    const int nq = ctx->ql > 0 ? ctx->ql : H * (int)qkh;
    if (gq)
      if (int e = gemm(at(tr.TA, (int64_t)ctx->off_q * Tp), Tp, tr.TX, Tp, gq, hid, nq, (int)hid, (int)Tp)) return e;
    if (grads->kv_a_proj_with_mqa)
      if (int e = gemm(at(tr.TA, (int64_t)ctx->off_kv * Tp), Tp, tr.TX, Tp, grads->kv_a_proj_with_mqa, hid, ctx->E,
                       (int)hid, (int)Tp))
        return e;
    if (grads->g_proj && ctx->off_g >= 0)
      if (int e = gemm(at(tr.TA, (int64_t)ctx->off_g * Tp), Tp, tr.TX, Tp, grads->g_proj, hid, (int)hdv, (int)hid,
                       (int)Tp))
        return e;
  }
  if (grads->kv_b_proj) {
    HIP_TRY(tpose(tr.dkvb, kvbn, (int)kvbn, tr.TA, false));
    HIP_TRY(tpose(tr.cache, ctx->E, ctx->c, tr.TB, true));
    if (int e = gemm(tr.TA, Tp, tr.TB, Tp, grads->kv_b_proj, ctx->c, (int)kvbn, ctx->c, (int)Tp)) return e;
  }
  if (ctx->ql > 0 && grads->q_b_proj) {
    HIP_TRY(tpose(tr.dQ, H * qkh, (int)(H * qkh), tr.TA, false));
    HIP_TRY(tpose(tr.qn, ctx->ql, ctx->ql, tr.TB, false));
    if (int e = gemm(tr.TA, Tp, tr.TB, Tp, grads->q_b_proj, ctx->ql, (int)(H * qkh), ctx->ql, (int)Tp)) return e;
  }
  return MLA_OK;
}

}  // extern "C"

namespace {

// longest visible key range of a decode query (sizes the split-KV partition)
int decode_max_visible(int mask_kind, int window, int max_seq_len) {
  return mask_kind == MLA_MASK_SLIDING ? std::min(window, max_seq_len) : max_seq_len;
}

// one new token per sequence in absorbed form; with topk_idx, each query sees
// only its listed positions (sparse lists, stream-K only)
int decode_impl(mla_ctx* ctx, const Workspace& ws, const void* x, int32_t batch, void* kv_cache, int32_t num_blocks,
                const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                int32_t mask_kind, int32_t window, const int32_t* topk_idx, int32_t topk, void* out,
                void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (!kv_cache) return fail(MLA_ERR_INVALID_ARG, "kv_cache must not be NULL (decode reads the latent cache)");
  if (!x || !block_table || !seq_lens || !out)
    return fail(MLA_ERR_INVALID_ARG, "x, block_table, seq_lens and out must not be NULL");
  if (batch <= 0 || num_blocks <= 0 || max_blocks <= 0 || max_seq_len <= 0)
    return fail(MLA_ERR_INVALID_ARG, "batch, num_blocks, max_blocks and max_seq_len must be positive");
  if (int e = check_mask(mask_kind, window)) return e;
  const mla_config& c = ctx->cfg;
  if (batch > c.max_batch || batch > c.max_tokens || max_seq_len > c.max_seq_len)
    return fail(MLA_ERR_CAPACITY, "batch or max_seq_len above the init limits");
  if ((int64_t)max_blocks * c.page_size < max_seq_len)
    return fail(MLA_ERR_INVALID_ARG, "max_blocks * page_size must cover max_seq_len");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  CallDone call_done(ctx, s);
  const int H = ctx->H;

  // the attention path and its arguments are settled before the first
  // launch, so a call that cannot run leaves the caller's cache untouched
  void* q;
  int64_t ldq;
  query_buffer(ctx, ws, &q, &ldq);
  DecodeAttnArgs da;
  da.ql = ws.qlat; da.ldql = (int64_t)H * ctx->c;
  da.q = q; da.ldq = ldq; da.qk_head = ctx->qkh;
  da.cache = kv_cache; da.block_table = block_table;
  da.num_blocks = num_blocks; da.max_blocks = max_blocks; da.page = c.page_size;
  da.seq_lens = seq_lens; da.max_seq_len = max_seq_len; da.batch = batch;
  da.H = H; da.n = ctx->n; da.r = ctx->r; da.c = ctx->c;
  da.scale = ctx->scale;
  da.kv_fp8 = ctx->kv_fp8; da.kv_scale = ctx->kv_scale;
  da.mask.kind = mask_kind; da.mask.window = window;
  da.part_o = ws.part_o; da.part_lse = ws.part_lse;
  da.o_lat = ws.olat;
  da.zeros = static_cast<const bf16_t*>(ctx->zeros);
  int max_vis = decode_max_visible(mask_kind, window, max_seq_len);
  if (topk_idx) {
    da.gather_ent = ws.sp_ent;
    da.gather_k = topk;
    max_vis = topk;
  }
  const bool stream_k = ctx->sk_shape && batch <= kDecodeMaxBatch;
  if (stream_k) {
    // stream-K: equal tile ranges over all sequences, pieces merged afterwards
    da.ranges = decode_sk_ranges(batch, max_vis, ctx->cus);
    da.tstart = ws.sk_tstart;
    if (da.ranges > ctx->sk_max_ranges) return fail(MLA_ERR_CAPACITY, "decode ranges above the init sizing");
    if (const char* m = decode_sk_check(da)) return fail(MLA_ERR_UNSUPPORTED, m);
  } else if (topk_idx) {
    return fail(MLA_ERR_UNSUPPORTED, "sparse lists need the bf16 512 + 64 latent with at most 128 heads");
  } else if (ctx->kv_fp8) {
    return fail(MLA_ERR_UNSUPPORTED, "the 8-bit cache decodes at most 1024 sequences per call");
  } else {
    // split-KV sizing from the longest visible range (keys per split a multiple of 32)
    const int groups = (H + 63) / 64;
    int want = (512 + batch * groups - 1) / (batch * groups);
    want = std::max(1, std::min(want, ctx->max_splits));
    int chunk = std::max(1, (max_vis + want - 1) / want);
    chunk = std::max(64, ((chunk + 31) / 32) * 32);
    const int splits = std::max(1, std::min(ctx->max_splits, (max_vis + chunk - 1) / chunk));
    if ((int64_t)splits * chunk < max_vis) chunk = ((max_vis + splits - 1) / splits + 31) / 32 * 32;
    da.chunk = chunk; da.splits = splits;
    if (const char* m = decode_attn_check(da, ctx->bf16)) return fail(MLA_ERR_UNSUPPORTED, m);
  }

  if (int e = project(ctx, ws, x, batch, s, &q, &ldq)) return e;

  RopeCacheArgs rc;
  rc.q = q; rc.ldq = ldq; rc.qk_head = ctx->qkh;
  rc.kv = static_cast<char*>(ws.buf1) + (size_t)ctx->off_kv * ctx->esz; rc.ldkv = ctx->N1;
  rc.gamma_kv = ctx->gamma_kv;
  rc.cache = kv_cache; rc.block_table = block_table;
  rc.num_blocks = num_blocks; rc.max_blocks = max_blocks; rc.page = c.page_size;
  rc.rope_cos = ctx->rope_cos; rc.rope_sin = ctx->rope_sin;
  rc.H = H; rc.n = ctx->n; rc.r = ctx->r; rc.c = ctx->c;
  rc.interleaved = c.rope_style == MLA_ROPE_INTERLEAVED;
  rc.eps = (float)c.rms_norm_eps;
  rc.kv_fp8 = ctx->kv_fp8; rc.kv_scale = ctx->kv_scale;
  rc.decode = 1; rc.seq_lens = seq_lens; rc.max_seq_len = max_seq_len; rc.total_tokens = batch;
  {
    StageTimer st(ctx, s, ST_ROPE_CACHE);
    HIP_TRY(rope_cache_launch(rc, ctx->bf16, 1, batch, s));
  }

  // W_UK absorption: ql_nope[b, h] = q_nope[b, h] . W_UK^T[h]   (per head: [B, n] x [n, c])
  GemmArgs ga;
  ga.A = q; ga.lda = ldq; ga.sA = ctx->qkh;
  ga.W = ctx->Wuk_t; ga.ldw = ctx->n; ga.sW = (int64_t)ctx->c * ctx->n;
  ga.C = ws.qlat; ga.ldc = (int64_t)H * ctx->c; ga.sC = ctx->c;
  ga.M = batch; ga.N = ctx->c; ga.K = ctx->n; ga.batch = H;
  {
    StageTimer st(ctx, s, ST_WUK);
    if (int e = run_gemm(ctx, ws, ga, s)) return e;
  }

  if (stream_k) {
    {
      StageTimer st(ctx, s, ST_DECODE_ATTN);
      if (topk_idx) {
        hipLaunchKernelGGL(sparse_entries_kernel, dim3((topk + 255) / 256, batch), dim3(256), 0, s, topk_idx, topk,
                           seq_lens, max_seq_len, block_table, max_blocks, num_blocks, c.page_size, ws.sp_ent);
        HIP_TRY(hipGetLastError());
      }
      HIP_TRY(decode_sk_launch(da, s));
    }
    {
      StageTimer st(ctx, s, ST_DECODE_MERGE);
      HIP_TRY(decode_sk_merge_launch(da, s));
    }
  } else {
    {
      StageTimer st(ctx, s, ST_DECODE_ATTN);
      HIP_TRY(decode_attn_launch(da, ctx->bf16, s));
    }
    {
      StageTimer st(ctx, s, ST_DECODE_MERGE);
      HIP_TRY(decode_merge_launch(da, ctx->bf16, s));
    }
  }

  // W_UV: out_v[b, h] = o_lat[b, h] . W_UV[h]^T (per head: [B, c] x [c, dv]), gated
  GemmArgs gv;
  gv.A = ws.olat; gv.lda = (int64_t)H * ctx->c; gv.sA = ctx->c;
  gv.W = static_cast<char*>(ctx->Wkvb) + (size_t)ctx->n * ctx->c * ctx->esz;
  gv.ldw = ctx->c; gv.sW = (int64_t)(ctx->n + ctx->dv) * ctx->c;
  gv.C = ws.attn; gv.ldc = (int64_t)H * ctx->dv; gv.sC = ctx->dv;
  gv.M = batch; gv.N = ctx->dv; gv.K = ctx->c; gv.batch = H;
  if (ctx->off_g >= 0) {
    gv.epi = EPI_GATE;
    gv.G = static_cast<char*>(ws.buf1) + (size_t)ctx->off_g * ctx->esz;
    gv.ldg = ctx->N1; gv.sG = ctx->dv;
  }
  {
    StageTimer st(ctx, s, ST_WUV);
    if (int e = run_gemm(ctx, ws, gv, s)) return e;
  }

  GemmArgs go;
  go.A = ws.attn; go.lda = (int64_t)H * ctx->dv;
  go.W = ctx->Wo; go.ldw = (int64_t)H * ctx->dv;
  go.C = out; go.ldc = ctx->hid;
  go.M = batch; go.N = ctx->hid; go.K = H * ctx->dv;
  StageTimer st(ctx, s, ST_O_PROJ);
  return run_gemm(ctx, ws, go, s);
}

}  // namespace

extern "C" {

int mla_decode_absorbed(mla_ctx* ctx, const void* x, int32_t batch, void* kv_cache, int32_t num_blocks,
                        const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                        int32_t max_seq_len, int32_t mask_kind, int32_t window, void* out, void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  return decode_impl(ctx, ctx->ws, x, batch, kv_cache, num_blocks, block_table, max_blocks, seq_lens, max_seq_len,
                     mask_kind, window, nullptr, 0, out, stream);
}

int mla_decode_absorbed_sparse(mla_ctx* ctx, const void* x, int32_t batch, void* kv_cache, int32_t num_blocks,
                               const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                               int32_t max_seq_len, const int32_t* topk_indices, int32_t topk, void* out,
                               void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (!topk_indices) return fail(MLA_ERR_INVALID_ARG, "topk_indices must not be NULL");
  if (topk <= 0) return fail(MLA_ERR_INVALID_ARG, "topk must be positive");
  if (topk > ctx->cfg.max_topk) return fail(MLA_ERR_CAPACITY, "topk above the init max_topk");
  return decode_impl(ctx, ctx->ws, x, batch, kv_cache, num_blocks, block_table, max_blocks, seq_lens, max_seq_len,
                     MLA_MASK_FULL, 0, topk_indices, topk, out, stream);
}

int mla_decode_absorbed_noalloc(mla_ctx* ctx, const void* x, int32_t batch, void* kv_cache, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                int32_t max_seq_len, int32_t mask_kind, int32_t window, void* out, void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (batch <= 0 || max_seq_len <= 0) return fail(MLA_ERR_INVALID_ARG, "batch and max_seq_len must be positive");
  if (int e = check_mask(mask_kind, window)) return e;
  if (!ctx->sk_shape || batch > kDecodeMaxBatch)
    return fail(MLA_ERR_UNSUPPORTED, "the allocation-free decode needs the bf16 512 + 64 latent, <= 128 heads, "
                                     "a page size that is a multiple of 32 and <= 1024 sequences");
  char* base = static_cast<char*>(scratch_ptr(ctx->device));
  if (!base) return fail(MLA_ERR_HIP, "no scratch address for the context's device");
  // carve the call's workspaces out of the scratch array (256-byte aligned)
  const int H = ctx->H;
  const int ranges = decode_sk_ranges(batch, decode_max_visible(mask_kind, window, max_seq_len), ctx->cus);
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    char* p = base + off;
    off += (bytes + 255) & ~(size_t)255;
    return static_cast<void*>(p);
  };
  Workspace ws;
  ws.buf1 = carve((size_t)batch * ctx->N1 * ctx->esz);
  if (ctx->ql > 0) ws.qbuf = carve((size_t)batch * H * ctx->qkh * ctx->esz);
  ws.qlat = carve((size_t)batch * H * ctx->c * ctx->esz);
  ws.olat = carve((size_t)batch * H * ctx->c * ctx->esz);
  ws.attn = carve((size_t)batch * H * ctx->dv * ctx->esz);
  ws.sk_tstart = static_cast<int32_t*>(carve((size_t)(batch + 1) * sizeof(int32_t)));
  // stream-K pieces: two per range, bf16 partial outputs and fp32 LSEs
  ws.part_o = static_cast<float*>(carve((size_t)2 * ranges * H * ctx->c * sizeof(bf16_t)));
  ws.part_lse = static_cast<float*>(carve((size_t)2 * ranges * H * sizeof(float)));
  ws.gemm_ws = static_cast<float*>(carve(kScratchGemmBytes));
  ws.gemm_ws_elems = (int64_t)(kScratchGemmBytes / sizeof(float));
  if (off > kScratchBytes)
    return fail(MLA_ERR_CAPACITY, "the call's workspaces (" + std::to_string(off) + " bytes) exceed the " +
                                      std::to_string(kScratchBytes) + "-byte scratch array");
  // nothing in these workspaces needs to start at zero: every kernel writes
  // what a later kernel reads
  return decode_impl(ctx, ws, x, batch, kv_cache, num_blocks, block_table, max_blocks, seq_lens, max_seq_len,
                     mask_kind, window, nullptr, 0, out, stream);
}

int mla_decode_absorbed_block(mla_ctx* ctx, const void* x, int32_t batch, int32_t q_len, void* kv_cache,
                              int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                              const int32_t* prefix_lens, int32_t max_kv_len, void* out, void* stream) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  if (!x || !kv_cache || !block_table || !prefix_lens || !out)
    return fail(MLA_ERR_INVALID_ARG, "x, kv_cache, block_table, prefix_lens and out must not be NULL");
  if (batch <= 0 || q_len <= 0 || num_blocks <= 0 || max_blocks <= 0 || max_kv_len <= 0)
    return fail(MLA_ERR_INVALID_ARG, "batch, q_len, num_blocks, max_blocks and max_kv_len must be positive");
  if (max_kv_len < q_len) return fail(MLA_ERR_INVALID_ARG, "max_kv_len must cover the block (>= q_len)");
  const mla_config& c = ctx->cfg;
  const int H = ctx->H;
  const int64_t T = (int64_t)batch * q_len;
  if (batch > c.max_batch || T > c.max_block_tokens || T > c.max_tokens || max_kv_len > c.max_seq_len)
    return fail(MLA_ERR_CAPACITY, "batch, batch * q_len or max_kv_len above the init limits");
  if ((int64_t)max_blocks * c.page_size < max_kv_len)
    return fail(MLA_ERR_INVALID_ARG, "max_blocks * page_size must cover max_kv_len");
  if (!ctx->sk_shape) return fail(MLA_ERR_UNSUPPORTED, "query blocks need the bf16 512 + 64 latent and <= 128 heads");
  if (((int64_t)q_len * H) % 128) return fail(MLA_ERR_UNSUPPORTED, "q_len * num_heads must be a multiple of 128");
  const int64_t V = T * H / 128;  // virtual sequences of 128 (query, head) pairs
  if (V > kDecodeMaxBatch) return fail(MLA_ERR_CAPACITY, "batch * q_len * num_heads above 128 K pairs");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  CallDone call_done(ctx, s);
  const Workspace& ws = ctx->ws;

  // latent attention (its arguments are settled and checked before the first
  // launch): virtual sequence v holds the (token, head) pairs
  // v * 128 .. v * 128 + 127 of [T, H] (q_len * H / 128 per sequence), all of
  // whose tokens see the same cache entries
  DecodeAttnArgs da;
  da.ql = ws.qlat; da.ldql = (int64_t)128 * ctx->c;
  void* q;
  int64_t ldq;
  query_buffer(ctx, ws, &q, &ldq);
  da.q = q; da.ldq = ldq; da.qk_head = ctx->qkh;
  da.cache = kv_cache; da.block_table = block_table;
  da.num_blocks = num_blocks; da.max_blocks = max_blocks; da.page = c.page_size;
  da.seq_lens = prefix_lens; da.len_add = q_len; da.max_seq_len = max_kv_len; da.batch = (int)V;
  da.H = 128; da.Hr = H; da.seq_div = (int)(V / batch);
  da.n = ctx->n; da.r = ctx->r; da.c = ctx->c;
  da.scale = ctx->scale;
  da.kv_fp8 = ctx->kv_fp8; da.kv_scale = ctx->kv_scale;
  da.mask.kind = MLA_MASK_FULL; da.mask.window = 0;
  da.part_o = ws.part_o; da.part_lse = ws.part_lse;
  da.o_lat = ws.olat;
  da.zeros = static_cast<const bf16_t*>(ctx->zeros);
  da.ranges = decode_sk_ranges((int)V, max_kv_len, ctx->cus);
  da.tstart = ws.sk_tstart;
  if (da.ranges > ctx->sk_max_ranges) return fail(MLA_ERR_CAPACITY, "decode ranges above the init sizing");
  if (const char* m = decode_sk_check(da)) return fail(MLA_ERR_UNSUPPORTED, m);

  if (int e = project(ctx, ws, x, (int)T, s, &q, &ldq)) return e;

  RopeCacheArgs rc;
  rc.q = q; rc.ldq = ldq; rc.qk_head = ctx->qkh;
  rc.kv = static_cast<char*>(ws.buf1) + (size_t)ctx->off_kv * ctx->esz; rc.ldkv = ctx->N1;
  rc.gamma_kv = ctx->gamma_kv;
  rc.cache = kv_cache; rc.block_table = block_table;
  rc.num_blocks = num_blocks; rc.max_blocks = max_blocks; rc.page = c.page_size;
  rc.rope_cos = ctx->rope_cos; rc.rope_sin = ctx->rope_sin;
  rc.H = H; rc.n = ctx->n; rc.r = ctx->r; rc.c = ctx->c;
  rc.interleaved = c.rope_style == MLA_ROPE_INTERLEAVED;
  rc.eps = (float)c.rms_norm_eps;
  rc.kv_fp8 = ctx->kv_fp8; rc.kv_scale = ctx->kv_scale;
  rc.decode = 0; rc.cu_seqlens = nullptr; rc.prefix_lens = prefix_lens;  // blocks of q_len tokens
  rc.max_q_len = q_len; rc.max_kv_len = max_kv_len; rc.max_seq_len = c.max_seq_len;
  rc.total_tokens = (int)T;
  {
    StageTimer st(ctx, s, ST_ROPE_CACHE);
    HIP_TRY(rope_cache_launch(rc, ctx->bf16, q_len, batch, s));
  }

  // W_UK absorption of every token: ql_nope[t, h] = q_nope[t, h] . W_UK^T[h]
  GemmArgs ga;
  ga.A = q; ga.lda = ldq; ga.sA = ctx->qkh;
  ga.W = ctx->Wuk_t; ga.ldw = ctx->n; ga.sW = (int64_t)ctx->c * ctx->n;
  ga.C = ws.qlat; ga.ldc = (int64_t)H * ctx->c; ga.sC = ctx->c;
  ga.M = (int)T; ga.N = ctx->c; ga.K = ctx->n; ga.batch = H;
  {
    StageTimer st(ctx, s, ST_WUK);
    if (int e = run_gemm(ctx, ws, ga, s)) return e;
  }

  {
    StageTimer st(ctx, s, ST_DECODE_ATTN);
    HIP_TRY(decode_sk_launch(da, s));
  }
  {
    StageTimer st(ctx, s, ST_DECODE_MERGE);
    HIP_TRY(decode_sk_merge_launch(da, s));
  }

  // W_UV of every token, gated
  GemmArgs gv;
  gv.A = ws.olat; gv.lda = (int64_t)H * ctx->c; gv.sA = ctx->c;
  gv.W = static_cast<char*>(ctx->Wkvb) + (size_t)ctx->n * ctx->c * ctx->esz;
  gv.ldw = ctx->c; gv.sW = (int64_t)(ctx->n + ctx->dv) * ctx->c;
  gv.C = ws.attn; gv.ldc = (int64_t)H * ctx->dv; gv.sC = ctx->dv;
  gv.M = (int)T; gv.N = ctx->dv; gv.K = ctx->c; gv.batch = H;
  if (ctx->off_g >= 0) {
    gv.epi = EPI_GATE;
    gv.G = static_cast<char*>(ws.buf1) + (size_t)ctx->off_g * ctx->esz;
    gv.ldg = ctx->N1; gv.sG = ctx->dv;
  }
  {
    StageTimer st(ctx, s, ST_WUV);
    if (int e = run_gemm(ctx, ws, gv, s)) return e;
  }

  GemmArgs go;
  go.A = ws.attn; go.lda = (int64_t)H * ctx->dv;
  go.W = ctx->Wo; go.ldw = (int64_t)H * ctx->dv;
  go.C = out; go.ldc = ctx->hid;
  go.M = (int)T; go.N = ctx->hid; go.K = H * ctx->dv;
  StageTimer st(ctx, s, ST_O_PROJ);
  return run_gemm(ctx, ws, go, s);
}

int mla_profile_enable(mla_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(MLA_ERR_INVALID_ARG, "ctx must not be NULL");
  ctx->profiling = enable != 0;
  return MLA_OK;
}

int mla_profile_read(mla_ctx* ctx, double* ms, int32_t* count) {
  if (!ctx || !ms) return fail(MLA_ERR_INVALID_ARG, "ctx and ms must not be NULL");
  for (int i = 0; i < ST_COUNT; ++i) {
    ms[i] = 0.0;
    if (count) count[i] = 0;
  }
  int rc = MLA_OK;
  for (auto& mk : ctx->marks) {
    float t = 0.f;
    if (hipEventSynchronize(mk.stop) != hipSuccess || hipEventElapsedTime(&t, mk.start, mk.stop) != hipSuccess)
      rc = fail(MLA_ERR_HIP, "reading a stage event failed");
    ms[mk.stage] += t;
    if (count) count[mk.stage] += 1;
    ctx->event_pool.push_back(mk.start);
    ctx->event_pool.push_back(mk.stop);
  }
  ctx->marks.clear();
  return rc;
}

const char* mla_profile_stage_name(int32_t stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : nullptr;
}

void mla_free(mla_ctx* ctx) {
  if (!ctx) return;
  int cur = 0;
  (void)hipGetDevice(&cur);
  (void)hipSetDevice(ctx->device);
  // the last call's work (stream order covers the calls before it)
  (void)hipEventSynchronize(ctx->done);
  (void)hipEventDestroy(ctx->done);
  for (auto& mk : ctx->marks) {
    (void)hipEventDestroy(mk.start);
    (void)hipEventDestroy(mk.stop);
  }
  for (hipEvent_t e : ctx->event_pool) (void)hipEventDestroy(e);
  free_all(ctx);
  (void)hipSetDevice(cur);
  delete ctx;
}

}  // extern "C"
