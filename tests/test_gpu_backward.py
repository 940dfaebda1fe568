"""GPU parity of mla_backward_expanded (the gradient of the expanded MLA layer
on training sequences) against the fp64 oracle's analytic gradient
(oracle.backward, pinned by finite differences and torch.autograd on the
CPU): dx and every weight gradient, same seeded inputs."""
import numpy as np
import pytest
import torch

import mla_synth as ms
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only with -m gpu
    pytest.skip("needs a GPU", allow_module_level=True)


def _check(w, seed, **kw):
    dout = U.draw_dout(w, seed)
    dx, g = U.run_backward(w, dout)
    U.check_backward(w, dout, dx, g, **kw)


def test_backward_tiny_f32():
    """The tiny fp32 model: two causal sequences (16 and 9 tokens)."""
    w = ms.make_workload("tiny_f32", q_lens=[16, 9], prefix_lens=[0, 0], seed=70)
    _check(w, 170)


@pytest.mark.parametrize("variant", [
    dict(q_lora_rank=64, rope_style=ms.ROPE_INTERLEAVED, use_output_gate=True),
    dict(use_output_gate=True),
])
@pytest.mark.parametrize("mask,window", [(ms.MASK_FULL, 0), (ms.MASK_SLIDING, 7), (ms.MASK_CAUSAL, 0)])
def test_backward_tiny_f32_variants(variant, mask, window):
    """Low-rank query, gate, both RoPE styles, every mask; lengths across
    the 64-token tiles (70, 1, 130)."""
    w = ms.make_workload("tiny_f32", dims_override=variant, q_lens=[70, 1, 130], prefix_lens=[0, 0, 0],
                         mask_kind=mask, window=window, seed=71, gamma_noise=True)
    _check(w, 171)


def test_backward_tiny_f32_dropped_rows():
    """Explicit visible intervals: dropped rows (no visible key) pass no
    gradient; an interval that ends before the row's own position."""
    q_lens = [20, 12]
    T = sum(q_lens)
    lo = np.zeros(T, np.int32)
    hi = np.array([i + 1 for q in q_lens for i in range(q)], np.int32)
    hi[3:6] = 0
    lo[25:27], hi[25:27] = 2, 4
    w = ms.make_workload("tiny_f32", q_lens=q_lens, prefix_lens=[0, 0], row_interval=(lo, hi), seed=72,
                         dims_override=dict(q_lora_rank=64))
    _check(w, 172)


def test_backward_draft_block_dims_bf16():
    """bf16 at the draft-block model dims (hidden 4096, 32 heads, q_lora
    1536, kv_lora 512, nope 128, rope 64, v 128, interleaved RoPE): two
    causal training sequences of 200 and 77 tokens."""
    w = ms.make_workload("draft_block_bf16", q_lens=[200, 77], prefix_lens=[0, 0], mask_kind=ms.MASK_CAUSAL,
                         seed=73)
    _check(w, 173)


def test_backward_split_k_bf16():
    """bf16 at the draft-block model dims with 2 x 512 causal tokens: enough
    rows for the 256 x 256 GEMM kernel, too few output tiles to fill the
    GPU, so the weight gradients (K = 1024 tokens), the data gradients and
    the recomputed first projection run split-K with fp32 partials."""
    w = ms.make_workload("draft_block_bf16", q_lens=[512, 512], prefix_lens=[0, 0], mask_kind=ms.MASK_CAUSAL,
                         seed=75)
    _check(w, 175)


def test_backward_split_k3_bf16():
    """bf16 at the draft-block model dims with 2 x 1024 causal tokens: the
    q_b and first-projection weight gradients (144 output tiles, K = 2048
    tokens) split K three ways (22, 22 and 20 of the 64 32-wide steps), the
    split count chosen by estimated time."""
    w = ms.make_workload("draft_block_bf16", q_lens=[1024, 1024], prefix_lens=[0, 0], mask_kind=ms.MASK_CAUSAL,
                         seed=76)
    _check(w, 176)


def test_backward_gate_neox_bf16():
    """bf16, 16 heads, output gate, NeoX RoPE, sliding window 50, lengths 130,
    64 and 1."""
    w = ms.make_workload("draft_block_bf16", q_lens=[130, 64, 1], prefix_lens=[0, 0, 0], mask_kind=ms.MASK_SLIDING,
                         window=50, seed=74,
                         dims_override={"num_heads": 16, "use_output_gate": True, "rope_style": ms.ROPE_NEOX})
    _check(w, 174)


def test_backward_full_mask_bf16():
    """bf16 at the draft-block model dims under the FULL mask (every query
    sees its whole sequence, keys after it included): 300 and 40 tokens,
    over a 256-query tile boundary and ragged 64-key tiles."""
    w = ms.make_workload("draft_block_bf16", q_lens=[300, 40], prefix_lens=[0, 0], mask_kind=ms.MASK_FULL, seed=77)
    _check(w, 177)


def test_backward_intervals_bf16():
    """bf16 at the draft-block model dims with explicit visible intervals:
    a wavefront's 32 rows dropped, empty intervals away from key 0, rows
    that see keys after their own position, a one-key row and random
    intervals whose ends are not tile multiples."""
    q_lens = [290, 50]
    T = sum(q_lens)
    rng = np.random.default_rng(78)
    pos = np.concatenate([np.arange(q) for q in q_lens])
    kv = np.concatenate([[q] * q for q in q_lens])
    lo = np.zeros(T, np.int64)
    hi = pos + 1
    r = np.arange(100, 250)
    lo[r] = rng.integers(0, pos[r] + 1)
    hi[r] = rng.integers(lo[r], kv[r] + 1)
    hi[32:64] = 0
    lo[70:80], hi[70:80] = 40, 40
    lo[80:90], hi[80:90] = 13, kv[80]
    lo[260:264], hi[260:264] = 5, 6
    w = ms.make_workload("draft_block_bf16", q_lens=q_lens, prefix_lens=[0, 0],
                         row_interval=(lo.astype(np.int32), hi.astype(np.int32)), seed=78)
    _check(w, 178)


def test_backward_sliding_multi_tile_bf16():
    """bf16 at the draft-block model dims under a sliding window of 300 over
    sequences of 600 and 257 tokens: several 256-query tiles whose first
    visible key is past key 0 and not a tile multiple."""
    w = ms.make_workload("draft_block_bf16", q_lens=[600, 257], prefix_lens=[0, 0], mask_kind=ms.MASK_SLIDING,
                         window=300, seed=79)
    _check(w, 179)


def test_backward_small_heads_bf16():
    """bf16 with 8 heads of nope 64, rope 32, v 64 (q/k head 96): the
    general bf16 attention-gradient kernels (16 keys or queries per
    wavefront, staged tiles) that shapes other than nope 128 / rope 64 /
    v 128 take."""
    w = ms.make_workload("draft_block_bf16", q_lens=[150, 70], prefix_lens=[0, 0], mask_kind=ms.MASK_CAUSAL, seed=80,
                         dims_override={"num_heads": 8, "qk_nope_head_dim": 64, "qk_rope_head_dim": 32,
                                        "v_head_dim": 64})
    _check(w, 180)
