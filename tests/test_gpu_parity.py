"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. bf16: max |err| <= 2e-2 and relative L2 <= 5e-3; fp32:
max |err| <= 1e-4. Small cases compare every output row and every written
cache entry; full-size workloads compare sampled sequences / rows that the
oracle computes one by one."""
import numpy as np
import pytest
import torch

import mla_synth as ms
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only with -m gpu
    pytest.skip("needs a GPU", allow_module_level=True)


def _run_and_check(w, **kw):
    out, cache = U.run_gpu(w, **kw)
    res = U.oracle(w)
    U.check(w, out, cache, res)
    return out


# ---------------------------------------------------------------- tiny fp32

def test_tiny_f32_prefill():
    """The tiny fp32 model: 16 causal tokens, hidden 256, 4 heads, no low-rank Q."""
    _run_and_check(ms.make_workload("tiny_f32"))


def test_tiny_f32_decode():
    w = ms.make_workload("tiny_f32", mode="decode", seq_lens=[1, 17, 40, 64, 65, 200], mask_kind=ms.MASK_CAUSAL)
    _run_and_check(w)


@pytest.mark.parametrize("variant", [
    dict(q_lora_rank=64, rope_style=ms.ROPE_INTERLEAVED),
    dict(use_output_gate=True),
])
@pytest.mark.parametrize("mask,window", [(ms.MASK_FULL, 0), (ms.MASK_SLIDING, 5)])
def test_tiny_f32_variants_prefill(variant, mask, window):
    w = ms.make_workload("tiny_f32", dims_override=variant, q_lens=[7, 70, 1], prefix_lens=[3, 60, 130],
                         mask_kind=mask, window=window, seed=10)
    _run_and_check(w)


@pytest.mark.parametrize("variant", [
    dict(q_lora_rank=64, rope_style=ms.ROPE_INTERLEAVED, use_output_gate=True),
])
def test_tiny_f32_variants_decode(variant):
    w = ms.make_workload("tiny_f32", dims_override=variant, mode="decode", seq_lens=[3, 90, 129],
                         mask_kind=ms.MASK_SLIDING, window=33, seed=11)
    _run_and_check(w)


def test_tiny_gamma_noise_bf16():
    """Nonunit RMSNorm gains (the q_a gain is folded into q_b_proj) in bf16."""
    w = ms.make_workload("tiny_f32", dims_override=dict(q_lora_rank=64, dtype="bf16"), q_lens=[20, 9],
                         prefix_lens=[5, 40], gamma_noise=True, seed=12)
    _run_and_check(w)


# ---------------------------------------------------- model dims, short runs

def test_draft_block_small():
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 16, 16], prefix_lens=[100, 37, 300])
    _run_and_check(w)


def test_draft_block_absorbed_small():
    """The draft-block shape through the absorbed block entry point: each
    16-token block sees its whole prefix and itself; same oracle (expanded,
    FULL mask) as the expanded entry point."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 16, 16], prefix_lens=[100, 37, 300])
    _run_and_check(w, block=True)


def test_draft_block_absorbed_gate_neox():
    """Absorbed blocks with an output gate, NeoX RoPE, 8-token blocks of a
    16-head model (two blocks per 128 (query, head) pairs) and a prefix of 0."""
    w = ms.make_workload("draft_block_bf16", q_lens=[8, 8, 8, 8], prefix_lens=[0, 63, 64, 1000], seed=23,
                         dims_override={"num_heads": 16, "use_output_gate": True, "rope_style": ms.ROPE_NEOX})
    _run_and_check(w, block=True)


def test_expand_fused_query_blocks():
    """The fused expansion + attention (at most 64 new tokens per sequence):
    causal chunks of 1-64 tokens (up to four 16-query blocks) after prefixes
    that end inside, at and across 256-entry chunk edges."""
    w = ms.make_workload("prefill_bf16", q_lens=[40, 64, 17, 1], prefix_lens=[300, 0, 1000, 255],
                         mask_kind=ms.MASK_CAUSAL, seed=41)
    _run_and_check(w)


def test_expand_fused_sliding_gate():
    """Fused path with a sliding window (chunks wholly outside some windows),
    the output gate and 16 heads (two heads per XCD band)."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 33, 5], prefix_lens=[500, 7, 256],
                         mask_kind=ms.MASK_SLIDING, window=100, seed=42,
                         dims_override={"num_heads": 16, "use_output_gate": True})
    _run_and_check(w)


def test_expand_fused_many_sequences():
    """Fused expansion + attention over 8 sequences x 32 heads: 1-16 new
    tokens, prefixes ending inside, at and across 256-entry chunk and
    64-entry page edges."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 5, 1, 16, 9, 16, 16, 3],
                         prefix_lens=[100, 37, 300, 0, 255, 240, 511, 700], seed=43)
    _run_and_check(w)


def test_expand_fused_causal_gate():
    """Fused path with a causal mask, the output gate, NeoX RoPE and 16 heads
    over 16 sequences."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16] * 8 + [7] * 8,
                         prefix_lens=[40 * i + 3 for i in range(16)], mask_kind=ms.MASK_CAUSAL, seed=44,
                         dims_override={"num_heads": 16, "use_output_gate": True, "rope_style": ms.ROPE_NEOX})
    _run_and_check(w)


def test_expand_fused_dropped_rows():
    """Explicit visible intervals through the fused path: dropped rows are
    exactly zero; an interval inside the prefix only."""
    q_lens, prefix = [16] * 8, [300, 20, 64, 1000, 5, 256, 128, 77]
    T = sum(q_lens)
    lo = np.zeros(T, np.int32)
    hi = np.array([p + q for p, q in zip(prefix, q_lens) for _ in range(q)], np.int32)
    hi[3:9] = 0
    lo[20:24] = 30
    hi[20:24] = 30
    lo[50:52], hi[50:52] = 600, 900
    w = ms.make_workload("draft_block_bf16", q_lens=q_lens, prefix_lens=prefix, row_interval=(lo, hi), seed=45)
    out = _run_and_check(w)
    assert np.all(out[3:9] == 0) and np.all(out[20:24] == 0)


def test_decode_small():
    w = ms.make_workload("decode_bf16", seq_lens=[1, 65, 700, 333, 64])
    _run_and_check(w)


def test_decode_window_edges():
    """Sliding windows whose first visible key is not a multiple of the
    32-key tile, lengths around tile and page edges."""
    w = ms.make_workload("decode_bf16", seq_lens=[1, 31, 32, 33, 95, 130, 700], mask_kind=ms.MASK_SLIDING,
                         window=33, seed=18)
    _run_and_check(w)


def test_decode_window_zero_bf16():
    """No visible key (window 0): the attention output, hence the layer
    output, is exactly zero for every sequence."""
    w = ms.make_workload("decode_bf16", seq_lens=[5, 64, 300], mask_kind=ms.MASK_SLIDING, window=0, seed=19)
    out, _ = U.run_gpu(w)
    assert np.all(out == 0)


def test_decode_projection_k_tails():
    """Few activation rows (M = 5) with projection k axes that are not a
    multiple of the 128-element weight-streaming k tile (hidden and q_lora
    1056), plus an output gate: the zero-filled k tail of every projection."""
    w = ms.make_workload("decode_bf16", seq_lens=[40, 300, 64, 1, 129], seed=21,
                         dims_override={"hidden_size": 1056, "num_heads": 16, "q_lora_rank": 1056,
                                        "use_output_gate": True})
    _run_and_check(w)


def test_sparse_decode_small():
    """Sparse (top-k) lists through mla_decode_absorbed_sparse: 96 entries =
    three 32-key tiles, lists longer than some sequences (padded with -1),
    and on one sequence an unsorted list with a negative entry, entries at
    and past its length (ignored) and a repeated position (attended twice)."""
    w = ms.make_workload("decode_bf16", seq_lens=[1, 40, 300, 64, 129, 700], seed=31)
    topk = ms.draw_topk(w, 96, seed=32)
    L2 = int(w.kv_lens[2])
    row = topk[2].copy()
    row[5], row[6], row[7], row[8] = -7, L2, L2 + 100, row[9]
    topk[2] = np.random.default_rng(33).permutation(row)
    out, cache = U.run_gpu(w, topk=topk)
    U.check(w, out, cache, U.oracle(w, topk=topk))


def test_sparse_decode_empty_and_tails():
    """A list with no usable entry gives exactly zero; 33-entry lists (one
    key in the second tile); a query whose own position is not listed."""
    w = ms.make_workload("decode_bf16", seq_lens=[5, 64, 300, 33], seed=34)
    topk = ms.draw_topk(w, 33, seed=35)
    topk[0] = -1
    topk[1][topk[1] == 63] = -1
    out, cache = U.run_gpu(w, topk=topk, extra_capacity=True)
    assert np.all(out[0] == 0)
    U.check(w, out, cache, U.oracle(w, topk=topk))


def test_sparse_decode_gate_heads16():
    """Sparse lists with 16 heads (one score wavefront), an output gate and NeoX RoPE."""
    w = ms.make_workload("decode_bf16", seq_lens=[70, 1000, 3, 257], seed=36,
                         dims_override={"num_heads": 16, "use_output_gate": True, "rope_style": ms.ROPE_NEOX})
    topk = ms.draw_topk(w, 200, seed=37)
    out, cache = U.run_gpu(w, topk=topk)
    U.check(w, out, cache, U.oracle(w, topk=topk))


def test_prefill_small():
    w = ms.make_workload("prefill_bf16", q_lens=[300, 129], prefix_lens=[0, 0])
    _run_and_check(w)


def test_long_decode_small():
    w = ms.make_workload("long_decode_bf16", seq_lens=[1500, 2999, 1024, 1025, 7])
    _run_and_check(w)


def test_prefill_big_tiles():
    """Prefill with enough rows for the 256 x 256 GEMM tiles (900 tokens):
    partial last N tile of the first projection (2112 columns), the q_a
    RMSNorm row scale of the q_b GEMM, gathered expansion rows with a ragged
    last M tile, causal attention."""
    w = ms.make_workload("prefill_bf16", q_lens=[600, 300], prefix_lens=[0, 37], seed=46)
    _run_and_check(w)


def test_prefill_big_tiles_interleaved():
    """Interleaved RoPE through the 256 x 256 tiles: the query rotation in the
    q_b projection's epilogue (token positions found from the sequence
    offsets, a one-token sequence between two long ones, cached prefixes)."""
    w = ms.make_workload("draft_block_bf16", q_lens=[520, 1, 390], prefix_lens=[0, 11, 3], seed=81)
    _run_and_check(w)


def test_prefill_chunked_sliding():
    """Causal prefill of a chunk after a cached prefix under a sliding window."""
    w = ms.make_workload("prefill_bf16", q_lens=[77, 200], prefix_lens=[300, 5], mask_kind=ms.MASK_SLIDING,
                         window=128, seed=13)
    _run_and_check(w)


def test_dropped_rows_are_exact_zero():
    """Explicit visible intervals with lo >= hi (a dropped draft block) give
    output rows that are exactly zero; the other rows match the oracle."""
    q_lens, prefix = [16, 16], [50, 20]
    T = sum(q_lens)
    lo = np.zeros(T, np.int32)
    hi = np.array([p + q for p, q in zip(prefix, q_lens) for _ in range(q)], np.int32)
    hi[3:9] = 0
    lo[20:24] = 30
    hi[20:24] = 30
    w = ms.make_workload("draft_block_bf16", q_lens=q_lens, prefix_lens=prefix, row_interval=(lo, hi), seed=14)
    out = _run_and_check(w)
    assert np.all(out[3:9] == 0) and np.all(out[20:24] == 0)


def test_prefill_full_mask_bf16():
    """FULL mask through the bf16 flash kernel (more than 64 new tokens, so
    not the fused path): every query sees its whole sequence, keys after its
    own position included, over ragged last tiles and a cached prefix."""
    w = ms.make_workload("prefill_bf16", q_lens=[150, 90], prefix_lens=[20, 0], mask_kind=ms.MASK_FULL, seed=83)
    _run_and_check(w)


def test_prefill_explicit_intervals_bf16():
    """Explicit visible intervals through the bf16 flash kernel: a wave's
    32 rows all dropped, empty intervals away from key 0, single-key rows,
    rows that see keys after their own position, and random intervals whose
    ends are not tile multiples; dropped rows are exactly zero."""
    q_lens, prefix = [300, 170], [37, 0]
    kv = [p + q for p, q in zip(prefix, q_lens)]
    T = sum(q_lens)
    seq = np.repeat(np.arange(2), q_lens)
    pos = np.concatenate([p + np.arange(q) for p, q in zip(prefix, q_lens)])
    kvr = np.asarray(kv)[seq]
    lo = np.zeros(T, np.int64)
    hi = pos + 1
    rng = np.random.default_rng(84)
    r = np.arange(150, 300)
    lo[r] = rng.integers(0, pos[r] + 1)
    hi[r] = rng.integers(lo[r], kvr[r] + 1)
    r = np.arange(380, 470)
    lo[r] = rng.integers(0, kvr[r])
    hi[r] = rng.integers(lo[r], kvr[r] + 1)
    hi[0:32] = 0
    lo[40:48], hi[40:48] = 100, 100
    lo[60:91] = 65 + np.arange(31) % 7
    hi[60:91] = kv[0]
    lo[100:104], hi[100:104] = 200, 201
    lo[300:364], hi[300:364] = 0, 0
    lo[364:380], hi[364:380] = 0, kv[1]
    dropped = lo >= hi
    w = ms.make_workload("prefill_bf16", q_lens=q_lens, prefix_lens=prefix,
                         row_interval=(lo.astype(np.int32), hi.astype(np.int32)), seed=85)
    out = _run_and_check(w)
    assert dropped.sum() >= 100
    assert np.all(out[dropped] == 0)


def test_window_zero_gives_zero_output():
    w = ms.make_workload("tiny_f32", mask_kind=ms.MASK_SLIDING, window=0, q_lens=[9], prefix_lens=[4], seed=15)
    out, _ = U.run_gpu(w)
    assert np.all(out == 0)


def test_softmax_scale_override():
    w = ms.make_workload("tiny_f32", q_lens=[12], prefix_lens=[30], seed=16)
    out, cache = U.run_gpu(w, softmax_scale=0.05)
    U.check(w, out, cache, U.oracle(w, softmax_scale=0.05))


def test_prefill_large_scale_bf16():
    """bf16 prefill with a softmax scale 3x the default: peaked rows whose
    running maximum moves by more than the lazy-rescale margin after the
    first tile, so the reference moves of the attention kernels (both tiles
    in registers shifted) are exercised, with cached prefixes and a ragged
    last tile."""
    w = ms.make_workload("prefill_bf16", q_lens=[300, 700], prefix_lens=[0, 100], seed=82)
    scale = 0.22
    out, cache = U.run_gpu(w, softmax_scale=scale)
    # the bf16 storage errors of q and of the keys enter the logits times the
    # scale: the output bar grows with it (default 1 / sqrt(192))
    grow = scale * np.sqrt(192.0)
    tol = dict(max_abs=U.TOL_BF16["max_abs"] * grow, rel_l2=U.TOL_BF16["rel_l2"] * grow)
    U.check(w, out, cache, U.oracle(w, softmax_scale=scale), out_tol=tol)


def test_capacity_above_call():
    """Context limits larger than the call (workspace rows beyond the batch)."""
    w = ms.make_workload("decode_bf16", seq_lens=[100, 3000], seed=17)
    out, cache = U.run_gpu(w, extra_capacity=True)
    U.check(w, out, cache, U.oracle(w))


# ------------------------------------------------ full sizes, sampled checks

# ---------------------------------------------------------------- 8-bit cache
# E4M3 codes of value / kv_scale; a power-of-two scale keeps every value the
# cache holds exact in bf16, the decode cases also take one that is not.

def test_fp8_decode_small():
    w = ms.make_workload("decode_bf16", seq_lens=[1, 65, 700, 333, 64, 31], seed=41, kv_scale=0.0421875)
    _run_and_check(w)


def test_fp8_decode_sliding():
    """Window edges that are not tile multiples, lengths around tile and page edges."""
    w = ms.make_workload("decode_bf16", seq_lens=[1, 31, 32, 33, 95, 130, 700], mask_kind=ms.MASK_SLIDING,
                         window=33, seed=42, kv_scale=2.0 ** -5)
    _run_and_check(w)


def test_fp8_sparse_decode():
    """Sparse lists over an 8-bit cache: 96 listed keys (three tiles), lists
    longer than some sequences."""
    w = ms.make_workload("decode_bf16", seq_lens=[1, 40, 300, 64, 129, 700], seed=43, kv_scale=2.0 ** -5)
    topk = ms.draw_topk(w, 96, seed=47)
    out, cache = U.run_gpu(w, topk=topk)
    U.check(w, out, cache, U.oracle(w, topk=topk))


def test_fp8_query_blocks():
    """Query blocks (mla_decode_absorbed_block) over an 8-bit cache."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 16, 16], prefix_lens=[100, 300, 0], seed=44,
                         mask_kind=ms.MASK_FULL, kv_scale=2.0 ** -5)
    out, cache = U.run_gpu(w, block=True)
    U.check(w, out, cache, U.oracle(w))


def test_fp8_prefill_fused():
    """Draft blocks (fused expansion) reading the bf16 copy of an 8-bit cache,
    ragged blocks and prefixes, one prefix that is not a page multiple."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 7, 16], prefix_lens=[100, 300, 0], seed=45,
                         kv_scale=2.0 ** -5)
    _run_and_check(w)


def test_fp8_prefill_expanded():
    """Long prefills (the kv_b expansion GEMM gathers from the bf16 copy),
    causal, one with a cached prefix."""
    w = ms.make_workload("prefill_bf16", q_lens=[300, 129], prefix_lens=[0, 70], seed=46, kv_scale=2.0 ** -4)
    _run_and_check(w)


def test_fp8_prefill_fused_scale_not_pow2():
    """Draft blocks (fused expansion) over an 8-bit cache whose scale is not a
    power of two: the prefill's bf16 copy of the entries (code * scale) is
    then rounded, not exact."""
    w = ms.make_workload("draft_block_bf16", q_lens=[16, 9, 16], prefix_lens=[200, 41, 0], seed=48,
                         kv_scale=0.0421875)
    _run_and_check(w)


def test_fp8_prefill_expanded_scale_not_pow2():
    """Long causal prefills (the expansion GEMM gathers from the bf16 copy)
    over an 8-bit cache with a scale that is not a power of two."""
    w = ms.make_workload("prefill_bf16", q_lens=[257, 100], prefix_lens=[30, 0], seed=49, kv_scale=0.0371)
    _run_and_check(w)


# ------------------------------------- generic split-KV decode (bf16 shapes)

def test_decode_generic_160_heads_bf16():
    """bf16 decode with 160 heads (above the stream-K kernel's 128): the
    generic split-KV kernel and its merge, in bf16, with an output gate."""
    w = ms.make_workload("decode_bf16", seq_lens=[1, 40, 700, 129, 2000], seed=50,
                         dims_override={"num_heads": 160, "hidden_size": 1024, "q_lora_rank": 256,
                                        "use_output_gate": True})
    _run_and_check(w)


def test_decode_generic_small_latent_bf16():
    """bf16 decode with a 256 + 32 latent and a page of 16 tokens (not the
    stream-K shape), sliding window."""
    w = ms.make_workload("decode_bf16", seq_lens=[3, 64, 500, 17], seed=51, mask_kind=ms.MASK_SLIDING, window=70,
                         dims_override={"kv_lora_rank": 256, "qk_rope_head_dim": 32, "num_heads": 16,
                                        "hidden_size": 512, "q_lora_rank": 128, "page_size": 16})
    _run_and_check(w)


def test_decode_generic_batch_above_1024_bf16():
    """1100 bf16 decode sequences (above the stream-K kernel's 1024 per
    call): the generic split-KV kernel; sampled sequences checked."""
    rng = np.random.default_rng(52)
    w = ms.make_workload("decode_bf16", seq_lens=list(rng.integers(1, 90, 1100)), seed=52,
                         dims_override={"num_heads": 16, "hidden_size": 512, "q_lora_rank": 128})
    out, cache = U.run_gpu(w)
    seqs = [0, 1, 517, 1023, 1024, 1099]
    U.check(w, out, cache, U.oracle(w, seqs=seqs))


def test_full_draft_block():
    """8 sequences x 16 fully visible tokens over a 2048-entry latent prefix."""
    w = ms.make_workload("draft_block_bf16")
    out, cache = U.run_gpu(w)
    U.check(w, out, cache, U.oracle(w, seqs=[0, 5]))


def test_full_decode():
    """64 sequences, cache lengths uniform in [1024, 8192]; sampled sequences
    checked against the oracle's absorbed form (pinned equal to the expanded
    form in fp64 by the CPU tests)."""
    w = ms.make_workload("decode_bf16")
    out, cache = U.run_gpu(w)
    L = w.kv_lens
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 17, 40})
    U.check(w, out, cache, U.oracle(w, seqs=seqs, form="absorbed"))


def test_full_sparse_decode():
    """The sparse decode workload: 64 sequences of 1024-8192 entries, 2048
    listed positions each (shorter sequences padded); sampled sequences
    against the oracle's absorbed form."""
    w = ms.make_workload("decode_bf16")
    topk = ms.draw_topk(w, 2048, seed=ms.SPARSE_TOPK_SEED)
    out, cache = U.run_gpu(w, topk=topk)
    L = w.kv_lens
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 17, 40})
    U.check(w, out, cache, U.oracle(w, seqs=seqs, form="absorbed", topk=topk))


def test_full_fp8_decode():
    """The decode workload (64 sequences of 1024-8192 entries) over an 8-bit
    cache (scale 2^-5); sampled sequences against the oracle's absorbed form."""
    w = ms.make_workload("decode_bf16", kv_scale=2.0 ** -5)
    out, cache = U.run_gpu(w)
    L = w.kv_lens
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), 17, 40})
    U.check(w, out, cache, U.oracle(w, seqs=seqs, form="absorbed"))


def test_full_prefill():
    """4 x 4096 causal tokens; sampled rows (tile edges, the first and last)."""
    w = ms.make_workload("prefill_bf16")
    out, cache = U.run_gpu(w)
    rows = [0, 1, 15, 16, 63, 64, 127, 128, 1000, 2047, 4095]
    rps = {0: rows, 3: rows}
    U.check(w, out, cache, U.oracle(w, seqs=[0, 3], rows_per_seq=rps), rows_per_seq=rps)


def test_full_long_decode():
    """16 sequences with 16k-32k cached entries under a 1024-token sliding
    window and the output gate; the oracle sees only the visible window."""
    w = ms.make_workload("long_decode_bf16")
    out, cache = U.run_gpu(w)
    seqs = [0, int(np.argmax(w.kv_lens)), 9]
    first = {b: int(w.kv_lens[b]) - w.window for b in seqs}
    trimmed = ms.Workload(**{**w.__dict__})
    trimmed.prefix_rows = [r[first.get(b, 0):] if b in first else r for b, r in enumerate(w.prefix_rows)]
    res = U.oracle(trimmed, seqs=seqs, form="absorbed", first_positions=first)
    U.check(w, out, cache, res)
