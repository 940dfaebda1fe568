"""Seeded synthetic inputs for the MLA forward (shared by the oracle tests, the
GPU parity tests and the benchmark).

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage dtype and lays them out (weights in nn.Linear
[out, in] layout, a paged latent cache addressed through a block table).

Recipe (every draw comes from ``numpy.random.default_rng(seed)`` in float32 and
is then rounded to the storage dtype, round-to-nearest-even for bf16):

  1. weights, in this order: q_a_proj, q_a_layernorm (only drawn when
     ``gamma_noise``; otherwise ones), q_b_proj | q_proj, kv_a_proj_with_mqa,
     kv_a_layernorm (same rule), kv_b_proj, g_proj (gate only), o_proj.
     Projection weights ~ N(0, 0.02); noisy RMSNorm gains ~ 1 + N(0, 0.1).
  2. x ~ N(0, 1), shape [total_tokens, hidden].
  3. cache lengths (decode workloads: integer uniform, inclusive bounds; the
     length includes the token being decoded).
  4. latent-prefix rows, sequence by sequence: all kv_lora_rank + rope dims
     ~ N(0, 1) (the stored latent of a real cache is RMS-normalised, so unit
     variance matches it with gain 1; the rope half's scale is a free choice).
  5. the physical-block permutation of the paged cache.

The five named workloads are the shapes of the MLA configurations this library
is measured on (a tiny fp32 model, a draft block over a latent prefix, a
DeepSeek-V3-shaped absorbed decode, a long causal prefill and a long-context
sliding-window decode with an output gate); train_bf16 is four causal
training sequences of 2048 tokens at the draft-block model dims, for the
backward pass (with dL/dout from draw_dout).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

MASK_FULL = 0
MASK_CAUSAL = 1
MASK_SLIDING = 2

ROPE_NEOX = 0
ROPE_INTERLEAVED = 1


@dataclass(frozen=True)
class ModelDims:
    hidden_size: int
    num_heads: int
    q_lora_rank: int  # 0 = no low-rank Q path (q_proj instead)
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    rope_style: int = ROPE_NEOX
    rope_theta: float = 10000.0
    rms_norm_eps: float = 1e-6
    use_output_gate: bool = False
    dtype: str = "bf16"  # "bf16" or "f32"
    page_size: int = 64

    @property
    def entry_dim(self) -> int:
        return self.kv_lora_rank + self.qk_rope_head_dim

    @property
    def qk_head_dim(self) -> int:
        return self.qk_nope_head_dim + self.qk_rope_head_dim


@dataclass
class Workload:
    """One batch of synthetic input plus the weights of one layer."""

    name: str
    dims: ModelDims
    mode: str  # "prefill" or "decode"
    seed: int
    weights: Dict[str, np.ndarray]  # float32 values, already rounded to dtype
    x: np.ndarray  # [T, hidden] float32 (rounded)
    q_lens: np.ndarray  # [B] int64: new tokens per sequence
    prefix_lens: np.ndarray  # [B] int64: cached entries before the new tokens
    prefix_rows: List[np.ndarray]  # B arrays [prefix_len_b, entry_dim] float32 (rounded)
    block_table: np.ndarray  # [B, max_blocks] int32, padding = -1
    num_blocks: int
    mask_kind: int
    window: int = 0
    row_lo: Optional[np.ndarray] = None  # [T] int32 explicit visible interval (prefill)
    row_hi: Optional[np.ndarray] = None
    # 8-bit cache: scale > 0; prefix_codes are the stored E4M3 codes (uint8)
    # and prefix_rows the values they hold
    kv_scale: float = 0.0
    prefix_codes: Optional[List[np.ndarray]] = None

    @property
    def batch(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def kv_lens(self) -> np.ndarray:
        return self.q_lens + self.prefix_lens

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


# --------------------------------------------------------------------------
# storage rounding (data preparation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return the raw bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    raise ValueError(f"unknown dtype {dtype}")


# --------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------

_DEEPSEEK_HEAD = dict(kv_lora_rank=512, qk_nope_head_dim=128, qk_rope_head_dim=64, v_head_dim=128)

DIMS: Dict[str, ModelDims] = {
    "tiny_f32": ModelDims(hidden_size=256, num_heads=4, q_lora_rank=0, kv_lora_rank=32,
                          qk_nope_head_dim=16, qk_rope_head_dim=8, v_head_dim=16,
                          rope_style=ROPE_NEOX, dtype="f32"),
    "draft_block_bf16": ModelDims(hidden_size=4096, num_heads=32, q_lora_rank=1536,
                                  rope_style=ROPE_INTERLEAVED, **_DEEPSEEK_HEAD),
    "decode_bf16": ModelDims(hidden_size=7168, num_heads=128, q_lora_rank=1536,
                             rope_style=ROPE_INTERLEAVED, **_DEEPSEEK_HEAD),
    "prefill_bf16": ModelDims(hidden_size=4096, num_heads=32, q_lora_rank=1536,
                              rope_style=ROPE_NEOX, **_DEEPSEEK_HEAD),
    "long_decode_bf16": ModelDims(hidden_size=7168, num_heads=128, q_lora_rank=0,
                                  rope_style=ROPE_INTERLEAVED, use_output_gate=True,
                                  **_DEEPSEEK_HEAD),
}
# training sequences at the draft-block model dims (the backward pass)
DIMS["train_bf16"] = DIMS["draft_block_bf16"]

# Full-size batch shapes of each workload.
SHAPES = {
    "tiny_f32": dict(mode="prefill", seed=0, q_lens=[16], prefix_lens=[0], mask_kind=MASK_CAUSAL),
    "draft_block_bf16": dict(mode="prefill", seed=1, q_lens=[16] * 8, prefix_lens=[2048] * 8,
                             mask_kind=MASK_FULL),
    "decode_bf16": dict(mode="decode", seed=2, batch=64, len_range=(1024, 8192),
                        mask_kind=MASK_CAUSAL),
    "prefill_bf16": dict(mode="prefill", seed=3, q_lens=[4096] * 4, prefix_lens=[0] * 4,
                         mask_kind=MASK_CAUSAL),
    "long_decode_bf16": dict(mode="decode", seed=4, batch=16, len_range=(16384, 32768),
                             mask_kind=MASK_SLIDING, window=1024),
    "train_bf16": dict(mode="prefill", seed=5, q_lens=[2048] * 4, prefix_lens=[0] * 4, mask_kind=MASK_CAUSAL),
}


def weight_shapes(d: ModelDims) -> Dict[str, tuple]:
    """nn.Linear [out, in] shapes of one MLA layer, in draw order."""
    H = d.num_heads
    s: Dict[str, tuple] = {}
    if d.q_lora_rank > 0:
        s["q_a_proj"] = (d.q_lora_rank, d.hidden_size)
        s["q_a_layernorm"] = (d.q_lora_rank,)
        s["q_b_proj"] = (H * d.qk_head_dim, d.q_lora_rank)
    else:
        s["q_proj"] = (H * d.qk_head_dim, d.hidden_size)
    s["kv_a_proj_with_mqa"] = (d.entry_dim, d.hidden_size)
    s["kv_a_layernorm"] = (d.kv_lora_rank,)
    s["kv_b_proj"] = (H * (d.qk_nope_head_dim + d.v_head_dim), d.kv_lora_rank)
    if d.use_output_gate:
        s["g_proj"] = (H * d.v_head_dim, d.hidden_size)
    s["o_proj"] = (d.hidden_size, H * d.v_head_dim)
    return s


def _draw_normal(rng, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_dtype(a, dtype)


def make_workload(name: str, *, seed: Optional[int] = None, batch: Optional[int] = None,
                  q_lens: Optional[Sequence[int]] = None,
                  prefix_lens: Optional[Sequence[int]] = None,
                  len_range: Optional[tuple] = None, seq_lens: Optional[Sequence[int]] = None,
                  mask_kind: Optional[int] = None, window: Optional[int] = None,
                  gamma_noise: bool = False, dims: Optional[ModelDims] = None,
                  dims_override: Optional[dict] = None, mode: Optional[str] = None,
                  row_interval: Optional[tuple] = None, kv_scale: float = 0.0) -> Workload:
    """Draw one workload. Keyword arguments override the named full-size shape
    (smaller batches and ragged lengths for the parity tests)."""
    d = dims if dims is not None else DIMS[name]
    if dims_override:
        d = dataclasses.replace(d, **dims_override)
    sh = dict(SHAPES[name]) if name in SHAPES else {}
    mode = mode or sh.get("mode", "prefill")
    seed = sh.get("seed", 0) if seed is None else seed
    mask_kind = sh.get("mask_kind", MASK_CAUSAL) if mask_kind is None else mask_kind
    window = sh.get("window", 0) if window is None else window
    rng = np.random.default_rng(seed)

    # 1. weights
    weights: Dict[str, np.ndarray] = {}
    for wname, shape in weight_shapes(d).items():
        if wname.endswith("layernorm"):
            if gamma_noise:
                weights[wname] = round_to_dtype(
                    1.0 + 0.1 * rng.standard_normal(shape, dtype=np.float32), d.dtype)
            else:
                weights[wname] = np.ones(shape, dtype=np.float32)
        else:
            weights[wname] = _draw_normal(rng, shape, 0.02, d.dtype)

    # lengths are fixed by the shape for prefill; drawn for decode (step 3,
    # after x, whose size only depends on the batch for decode)
    if mode == "prefill":
        ql = np.asarray(q_lens if q_lens is not None else sh["q_lens"], dtype=np.int64)
        pl = np.asarray(prefix_lens if prefix_lens is not None else sh.get("prefix_lens", [0] * len(ql)),
                        dtype=np.int64)
        assert ql.shape == pl.shape
        T = int(ql.sum())
        x = _draw_normal(rng, (T, d.hidden_size), 1.0, d.dtype)  # 2.
    else:
        B = batch if batch is not None else (len(seq_lens) if seq_lens is not None else sh["batch"])
        x = _draw_normal(rng, (B, d.hidden_size), 1.0, d.dtype)  # 2.
        if seq_lens is not None:
            L = np.asarray(seq_lens, dtype=np.int64)
        else:
            lo, hi = len_range if len_range is not None else sh["len_range"]
            L = rng.integers(lo, hi + 1, size=B).astype(np.int64)  # 3.
        assert L.shape == (B,) and (L >= 1).all()
        ql = np.ones(B, dtype=np.int64)
        pl = L - 1

    # 4. latent-prefix rows
    E = d.entry_dim
    prefix_rows = [_draw_normal(rng, (int(p), E), 1.0, d.dtype) for p in pl]
    prefix_codes = None
    if kv_scale > 0:
        # 8-bit cache: the rows stored as E4M3 codes of row / kv_scale by
        # torch's float8_e4m3fn cast, and the values those codes hold
        import torch
        prefix_codes, vals = [], []
        for rows in prefix_rows:
            f8 = torch.from_numpy(np.ascontiguousarray(rows / np.float32(kv_scale))).to(torch.float8_e4m3fn)
            prefix_codes.append(f8.view(torch.uint8).numpy().copy())
            vals.append((f8.to(torch.float32) * kv_scale).numpy())
        prefix_rows = vals

    # 5. paged cache: a random permutation of physical blocks
    page = d.page_size
    kv = ql + pl
    nblk = [max(1, -(-int(n) // page)) for n in kv]
    total = int(sum(nblk))
    perm = rng.permutation(total).astype(np.int32)
    max_blocks = max(nblk)
    bt = np.full((len(kv), max_blocks), -1, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[o:o + n]
        o += n

    row_lo = row_hi = None
    if row_interval is not None:
        row_lo, row_hi = (np.asarray(a, dtype=np.int32) for a in row_interval)

    return Workload(name=name, dims=d, mode=mode, seed=seed, weights=weights, x=x,
                    q_lens=ql, prefix_lens=pl, prefix_rows=prefix_rows, block_table=bt,
                    num_blocks=total, mask_kind=mask_kind, window=window,
                    row_lo=row_lo, row_hi=row_hi, kv_scale=float(kv_scale), prefix_codes=prefix_codes)


def draw_dout(w: Workload, seed: int) -> np.ndarray:
    """dL/dout of a training workload [total_tokens, hidden]: N(0, 1) from a
    generator of its own, rounded to the workload's dtype (an input of the
    backward pass, like x)."""
    rng = np.random.default_rng(seed)
    return round_to_dtype(rng.standard_normal((w.total_tokens, w.dims.hidden_size), dtype=np.float32),
                          w.dims.dtype)


# seed of dL/dout of the training workload
TRAIN_DOUT_SEED = 8

# seed of the sparse decode workload's lists (decode_bf16 shapes, 2048 per sequence)
SPARSE_TOPK_SEED = 7


def draw_topk(w: Workload, topk: int, seed: int) -> np.ndarray:
    """Top-k key lists [B, topk] int32 for a decode workload: for sequence b,
    min(topk, L_b) distinct positions drawn uniformly from [0, L_b) (its
    query's own position L_b - 1 included with the rest), sorted, padded with
    -1. Drawn from a generator of its own, after the workload."""
    rng = np.random.default_rng(seed)
    L = w.kv_lens
    out = np.full((w.batch, topk), -1, dtype=np.int32)
    for b in range(w.batch):
        k = min(topk, int(L[b]))
        out[b, :k] = np.sort(rng.choice(int(L[b]), size=k, replace=False))
    return out


def paged_cache(w: Workload) -> np.ndarray:
    """The paged latent cache [num_blocks, page, entry_dim] holding the prefix
    rows at their logical positions (other slots zero). float32 values; uint8
    codes for an 8-bit cache."""
    d = w.dims
    fp8 = w.kv_scale > 0
    cache = np.zeros((w.num_blocks, d.page_size, d.entry_dim), dtype=np.uint8 if fp8 else np.float32)
    for b, rows in enumerate(w.prefix_codes if fp8 else w.prefix_rows):
        for j0 in range(0, rows.shape[0], d.page_size):
            blk = w.block_table[b, j0 // d.page_size]
            n = min(d.page_size, rows.shape[0] - j0)
            cache[blk, :n] = rows[j0:j0 + n]
    return cache


def gather_entries(w: Workload, cache: np.ndarray, b: int, lo: int, hi: int) -> np.ndarray:
    """Rows [lo, hi) of sequence b read back from a paged cache array."""
    page = w.dims.page_size
    out = np.empty((hi - lo, cache.shape[-1]), dtype=cache.dtype)
    for j in range(lo, hi):
        out[j - lo] = cache[w.block_table[b, j // page], j % page]
    return out
