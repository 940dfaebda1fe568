"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` raises AssertionError when the oracle disagrees. They are
called by tests/test_oracle.py directly and again under planted mistakes
(mutations of the oracle, on the CPU) to show that each pin can fail.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import mla as om
import mla_synth as ms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# page values
# --------------------------------------------------------------------------

def pin_page_dims():
    g = json.load(open(os.path.join(GOLDEN, "page_values.json")))
    d = g["deepseek_dims"]
    dims = ms.DIMS["decode_bf16"]
    assert d["kv_lora_rank"] + d["qk_rope_head_dim"] == d["cache_entry_dim"]
    assert dims.kv_lora_rank == d["kv_lora_rank"] and dims.qk_rope_head_dim == d["qk_rope_head_dim"]
    # the oracle's cache entries have the printed width, q heads are nope+rope
    w = ms.make_workload("tiny_f32", dims=ms.ModelDims(
        hidden_size=64, num_heads=2, q_lora_rank=0, kv_lora_rank=d["kv_lora_rank"],
        qk_nope_head_dim=8, qk_rope_head_dim=d["qk_rope_head_dim"], v_head_dim=8, dtype="f32"),
        q_lens=[3], prefix_lens=[0])
    q, ent, _ = om.project_tokens(w.dims, w.weights, w.x, np.arange(3))
    assert ent.shape == (3, d["cache_entry_dim"])
    assert q.shape == (3, 2, 8 + d["qk_rope_head_dim"])
    # paged cache layout: [num_blocks, block_size, 576], page bytes have no x2
    pb = g["page_bytes"]
    cache_shape = (w.num_blocks, w.dims.page_size, w.dims.entry_dim)
    assert len(cache_shape) == g["cache_shape"]["rank"] and cache_shape[-1] == g["cache_shape"]["last_dim"]
    bf16_page = pb["mla_factor"] * 64 * g["identities"]["num_kv_heads"] * 576 * 2
    assert bf16_page == 73728
    assert pb["full_attention_factor"] * 64 * 1 * 576 * 2 == 2 * bf16_page
    assert pb["fp8_ds_mla_bytes_per_token"] > 576  # packed fp8 entry carries more than one byte per dim


# --------------------------------------------------------------------------
# RMSNorm: library routine and closed forms
# --------------------------------------------------------------------------

def pin_rms_norm():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 33))
    g = 1 + 0.1 * rng.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.max(np.abs(om.rms_norm(x, g, 1e-6) - ref)) < 1e-13
    # constant row c -> gamma * c / sqrt(c^2 + eps)
    c = 3.0
    y = om.rms_norm(np.full((1, 5), c), np.ones(5), 1e-6)
    assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=0, atol=1e-15)
    # with eps = 0 it is scale invariant and has unit RMS
    y1, y2 = om.rms_norm(x, np.ones(33), 0.0), om.rms_norm(5.0 * x, np.ones(33), 0.0)
    assert np.max(np.abs(y1 - y2)) < 1e-13
    assert np.allclose(np.sqrt(np.mean(y1 ** 2, axis=-1)), 1.0, atol=1e-13)


# --------------------------------------------------------------------------
# RoPE: complex-rotation form, identities
# --------------------------------------------------------------------------

def _rope_complex(x, pos, theta, style):
    """RoPE as multiplication of the complex pairs by exp(i * p * w_j)."""
    r = x.shape[-1]
    w = theta ** (-2.0 * np.arange(r // 2) / r)
    if style == om.ROPE_NEOX:
        z = x[..., : r // 2] + 1j * x[..., r // 2:]
    else:
        z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * np.asarray(pos, np.float64)[:, None] * w[None, :])
    out = np.empty_like(x)
    if style == om.ROPE_NEOX:
        out[..., : r // 2], out[..., r // 2:] = z.real, z.imag
    else:
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def pin_rope():
    rng = np.random.default_rng(12)
    for style in (om.ROPE_NEOX, om.ROPE_INTERLEAVED):
        x = rng.standard_normal((9, 16))
        pos = rng.integers(0, 40000, size=9)
        y = om.apply_rope(x, pos, 10000.0, style)
        assert np.max(np.abs(y - _rope_complex(x, pos, 10000.0, style))) < 1e-9
        assert np.max(np.abs(om.apply_rope(x, np.zeros(9), 1e4, style) - x)) == 0.0  # p=0: identity
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
        # relative position: <R(p)q, R(t)k> depends on p - t only
        q, k = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
        a = om.apply_rope(q, [1000], 1e4, style) @ om.apply_rope(k, [990], 1e4, style).T
        b = om.apply_rope(q, [10], 1e4, style) @ om.apply_rope(k, [0], 1e4, style).T
        assert abs(float((a - b).item())) < 1e-10
        # first pair rotates by exactly p radians (theta^0 = 1)
        e0 = np.zeros((1, 16))
        a_idx, b_idx = om.rope_pairs(16, style)
        e0[0, a_idx[0]] = 1.0
        z = om.apply_rope(e0, [3], 1e4, style)
        assert abs(z[0, a_idx[0]] - math.cos(3)) < 1e-15 and abs(z[0, b_idx[0]] - math.sin(3)) < 1e-15
    # interleaved == NeoX under the fixed permutation that de-interleaves pairs
    x = rng.standard_normal((5, 16))
    pos = np.arange(5) * 77
    perm = np.concatenate([np.arange(0, 16, 2), np.arange(1, 16, 2)])
    yi = om.apply_rope(x, pos, 1e4, om.ROPE_INTERLEAVED)
    yn = om.apply_rope(x[:, perm], pos, 1e4, om.ROPE_NEOX)
    assert np.max(np.abs(yi[:, perm] - yn)) < 1e-13


# --------------------------------------------------------------------------
# attention core: library routine, softmax properties, empty rows
# --------------------------------------------------------------------------

def pin_attention_core():
    rng = np.random.default_rng(13)
    S, L, H, d, dv = 11, 29, 3, 12, 7
    q = rng.standard_normal((S, H, d))
    k = rng.standard_normal((L, H, d))
    v = rng.standard_normal((L, H, dv))
    lo = rng.integers(0, 20, size=S)
    hi = lo + rng.integers(1, 10, size=S)
    hi = np.minimum(hi, L)
    lo[3], hi[3] = 5, 5  # one empty row
    o, lse, P = om.attention_core(q, k, v, lo, hi, 0.3, return_probs=True)
    j = np.arange(L)
    mask = torch.from_numpy((j[None, :] >= lo[:, None]) & (j[None, :] < hi[:, None]))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2), attn_mask=mask, scale=0.3).permute(1, 0, 2).numpy()
    rows = np.array([i for i in range(S) if hi[i] > lo[i]])
    assert np.max(np.abs(o[rows] - ref[rows])) < 1e-13
    assert np.all(P >= 0)
    assert np.max(np.abs(P[rows].sum(-1) - 1.0)) < 1e-14
    assert np.all(P[~mask.numpy()[:, None, :].repeat(H, 1)] == 0)
    # empty row: exact zeros, lse = -inf
    assert np.all(o[3] == 0.0) and np.all(np.isneginf(lse[3]))
    # a single visible key gets probability 1 and returns its value
    o1, _ = om.attention_core(q, k, v, [4] * S, [5] * S, 0.3)
    assert np.max(np.abs(o1 - v[4][None])) < 1e-15
    # lse is the log of the partition function
    i = 0
    s = 0.3 * (k[lo[i]:hi[i], 0, :] @ q[i, 0])
    assert abs(lse[i, 0] - math.log(np.exp(s).sum())) < 1e-12


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def tiny_dims(**kw):
    base = dict(hidden_size=48, num_heads=3, q_lora_rank=0, kv_lora_rank=16, qk_nope_head_dim=8,
                qk_rope_head_dim=6, v_head_dim=5, rope_style=om.ROPE_NEOX, dtype="f32", page_size=4)
    base.update(kw)
    return ms.ModelDims(**base)


def pin_brute_force(w):
    """Vectorised oracle == scalar-loop brute force (one sequence)."""
    assert w.batch == 1
    ref_out, ref_ent = om.brute_force_forward(w.dims, w.weights, w.x, w.prefix_rows[0],
                                              w.mask_kind, w.window)
    out, ent, _ = om.forward_sequence(w.dims, w.weights, w.x, w.prefix_rows[0], w.mask_kind, w.window)
    assert np.max(np.abs(ent - ref_ent)) <= 1e-12 * max(1.0, np.max(np.abs(ref_ent)))
    assert np.max(np.abs(out - ref_out)) <= 1e-12 * max(1.0, np.max(np.abs(ref_out))), \
        np.max(np.abs(out - ref_out))


def pin_absorbed_equals_expanded(w, seqs=None):
    """The absorbed (decode) form equals the expanded (prefill) form in fp64
    up to reassociation: the two are one computation regrouped."""
    e = om.mla_forward(w.dims, w.weights, w.x, w.q_lens, w.prefix_rows, w.mask_kind, w.window,
                       w.row_lo, w.row_hi, form="expanded", seqs=seqs)
    a = om.mla_forward(w.dims, w.weights, w.x, w.q_lens, w.prefix_rows, w.mask_kind, w.window,
                       w.row_lo, w.row_hi, form="absorbed", seqs=seqs)
    for b in e:
        ref = e[b][0]
        assert _rel(a[b][0], ref) < 1e-12, (b, _rel(a[b][0], ref))
        assert np.max(np.abs(a[b][0] - ref)) < 1e-12 * max(1.0, np.max(np.abs(ref)))


def pin_masks(w):
    """Special cases of the masks on one sequence of w (prefill)."""
    x, pre = w.x, w.prefix_rows[0]
    S, P = x.shape[0], pre.shape[0]
    # window >= L is the causal mask
    c = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_CAUSAL)
    s = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_SLIDING, window=P + S + 3)
    assert np.max(np.abs(c[0] - s[0])) == 0.0
    # window 1: each query sees only its own entry -> attention output = own v
    _, ent, attn = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_SLIDING, window=1)
    _, v = om.expand_kv(w.dims, w.weights, ent)
    gate = om.project_tokens(w.dims, w.weights, x, P + np.arange(S))[2]
    own = v.reshape(S, -1) * (gate if gate is not None else 1.0)
    assert np.max(np.abs(attn - own)) < 1e-12
    # window 0 or an empty explicit interval: the whole output row is exactly 0
    out0, _, _ = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_SLIDING, window=0)
    assert np.all(out0 == 0.0)
    lo = np.arange(S) + P
    hi = lo.copy()
    hi[::2] += 1  # odd rows dropped
    o, _, _ = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_CAUSAL, row_lo=lo, row_hi=hi)
    assert np.all(o[1::2] == 0.0) and np.all(np.abs(o[0::2]).max(axis=1) > 0)


def pin_cache_consistency(w, split: int):
    """prefill(S) == prefill(k) then prefill(S-k) over the cached prefix ==
    successive one-token decodes (causal mask)."""
    x, pre = w.x, w.prefix_rows[0]
    S = x.shape[0]
    full, ent, _ = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_CAUSAL)
    a, ent_a, _ = om.forward_sequence(w.dims, w.weights, x[:split], pre, om.MASK_CAUSAL)
    b, ent_b, _ = om.forward_sequence(w.dims, w.weights, x[split:], np.concatenate([pre, ent_a]),
                                      om.MASK_CAUSAL)
    assert np.max(np.abs(np.concatenate([a, b]) - full)) < 1e-12 * max(1, np.abs(full).max())
    assert np.max(np.abs(np.concatenate([ent_a, ent_b]) - ent)) < 1e-12
    cache = pre
    for i in range(S):
        o, e, _ = om.forward_sequence(w.dims, w.weights, x[i:i + 1], cache, om.MASK_CAUSAL)
        assert np.max(np.abs(o[0] - full[i])) < 1e-12 * max(1, np.abs(full).max())
        cache = np.concatenate([cache, e])


def pin_window_trim(w, window: int):
    """Under a sliding window, dropping the prefix rows no query can see (and
    giving the position of the first kept row) leaves every output unchanged."""
    x, pre = w.x, w.prefix_rows[0]
    P, S = pre.shape[0], x.shape[0]
    full = om.forward_sequence(w.dims, w.weights, x, pre, om.MASK_SLIDING, window)
    f0 = max(0, P + 1 - window)  # first key the earliest new query can see
    trim = om.forward_sequence(w.dims, w.weights, x, pre[f0:], om.MASK_SLIDING, window, first_position=f0)
    assert np.max(np.abs(full[0] - trim[0])) == 0.0
    assert np.max(np.abs(full[1] - trim[1])) == 0.0


def pin_sparse(w):
    """Sparse (top-k) attention over listed keys, on one sequence of w:
    special cases that reduce to the masks, invariances of a softmax over a
    list, and the log-sum-exp merge of two lists (which fixes how a position
    listed twice counts)."""
    x, pre = w.x, w.prefix_rows[0]
    S, P = x.shape[0], pre.shape[0]
    L = P + S
    pos = P + np.arange(S)
    dims, W = w.dims, w.weights
    full = om.forward_sequence(dims, W, x, pre, om.MASK_FULL)
    tol = 1e-12 * max(1.0, np.abs(full[0]).max())  # per-query vs batched products: rounding order only
    # every position listed, in order: the full mask
    lists = [np.arange(L) for _ in range(S)]
    sp = om.forward_sequence(dims, W, x, pre, om.MASK_CAUSAL, key_lists=lists)
    assert np.max(np.abs(sp[0] - full[0])) <= tol
    assert np.max(np.abs(sp[1] - full[1])) == 0.0  # the cache entries do not depend on the lists
    # the last 3 positions up to the query's own: the sliding window of 3
    win = om.forward_sequence(dims, W, x, pre, om.MASK_SLIDING, window=3)
    lists = [np.arange(max(0, p - 2), p + 1) for p in pos]
    sp = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=lists)
    assert np.max(np.abs(sp[0] - win[0])) <= tol
    # order of a list is irrelevant; padding and positions outside [0, L) are ignored
    rng = np.random.default_rng(11)
    lists = [rng.choice(L, size=5, replace=False) for _ in range(S)]
    base = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=lists)
    perm = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=[rng.permutation(a) for a in lists])
    assert np.max(np.abs(perm[0] - base[0])) <= 1e-12 * max(1.0, np.abs(base[0]).max())
    padded = [np.concatenate([[-1], a, [L, L + 7, -5, -1]]) for a in lists]
    pad = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=padded)
    assert np.max(np.abs(pad[0] - base[0])) == 0.0
    # one listed key: the attention output is that key's value (P = 1)
    j = np.array([int(rng.integers(0, L)) for _ in range(S)])
    _, ent, attn = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=[[t] for t in j])
    _, v = om.expand_kv(dims, W, np.concatenate([pre, ent]))
    gate = om.project_tokens(dims, W, x, pos)[2]
    own = v[j].reshape(S, -1) * (gate if gate is not None else 1.0)
    assert np.max(np.abs(attn - own)) < 1e-12
    # nothing listed (or only padding): the output row is exactly 0
    out0, _, _ = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=[[-1, L] for _ in range(S)])
    assert np.all(out0 == 0.0)
    # a list split in two: the attention over the whole list is the
    # log-sum-exp-weighted merge of the two halves' attentions (the merge of
    # the MLA blog's prefix/suffix outputs); B repeats a position of A
    q = om.project_tokens(dims, W, x, pos)[0]
    k, v = om.expand_kv(dims, W, np.concatenate([pre, ent]))
    scale = 1.0 / np.sqrt(dims.qk_nope_head_dim + dims.qk_rope_head_dim)
    i = S - 1
    A = np.array([0, 2, L - 1])
    B = np.array([2, 1])
    oa, la = om.attention_core(q[i:i + 1], k[A], v[A], [0], [len(A)], scale)
    ob, lb = om.attention_core(q[i:i + 1], k[B], v[B], [0], [len(B)], scale)
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (wa[..., None] * oa + wb[..., None] * ob) / (wa + wb)[..., None]
    _, _, at = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, rows=[i], key_lists=[np.concatenate([A, B])])
    g = gate[i] if gate is not None else 1.0
    assert np.max(np.abs(at[0] - merged.reshape(-1) * g)) < 1e-12
    # the absorbed form over the same lists
    ab = om.forward_sequence(dims, W, x, pre, om.MASK_FULL, key_lists=lists, form="absorbed")
    assert np.max(np.abs(ab[0] - base[0])) <= 1e-12 * max(1.0, np.abs(base[0]).max())


def pin_fp8_e4m3():
    """The 8-bit cache format against its definition (OCP E4M3 "fn") and an
    independent implementation of it (torch's float8_e4m3fn cast): closed
    forms of named codes, every finite code decodes and re-encodes to itself,
    ties between neighbouring codes go to the even mantissa, values beyond
    the largest finite value saturate."""
    dec, enc = om.fp8_e4m3_decode, om.fp8_e4m3_encode
    named = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, value in named.items():
        assert dec(code) == value, (hex(code), dec(code), value)
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    codes = np.arange(256)
    vals = dec(codes)
    fin = ~np.isnan(vals)
    assert np.all(enc(vals[fin]) == codes[fin])
    pos = np.sort(vals[fin & (vals > 0)])
    assert pos[0] == 2.0 ** -9 and pos[-1] == 448.0 and np.all(np.diff(pos) > 0) and len(pos) == 126
    # the same codes as torch's cast: random values and every midpoint (a tie)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(2000) * 0.01,
                        (pos[1:] + pos[:-1]) / 2, -(pos[1:] + pos[:-1]) / 2]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(enc(x.astype(np.float64)), ref)
    mids = (pos[1:] + pos[:-1]) / 2
    got = enc(mids)
    assert np.all(dec(got) % 1 == dec(got) % 1)  # finite
    assert np.all((got & 1) == 0), "a tie goes to the even mantissa"
    assert enc(1e4) == 0x7E and enc(-1e4) == 0xFE and enc(448.0 + 15.9) == 0x7E
    # quantize: idempotent, scale-covariant for power-of-two scales
    y = rng.standard_normal(1000) * 3
    q = om.fp8_quantize(y, 0.0625)
    assert np.array_equal(om.fp8_quantize(q, 0.0625), q)
    assert np.array_equal(om.fp8_quantize(y * 2, 0.125), q * 2)
    assert np.max(np.abs(q - y) / np.maximum(np.abs(y), 2.0 ** -6 * 0.0625)) <= 2.0 ** -4 + 1e-12


def pin_round_bf16():
    """round_bf16 against torch's float32 -> bfloat16 cast (round to nearest,
    ties to even), on values over many binades and on exact ties."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4096) * 10.0 ** rng.integers(-30, 30, 4096)
    bits = (rng.integers(0, 0x7F000000, 2048, dtype=np.uint64) & ~np.uint64(0xFFFF)) | np.uint64(0x8000)
    ties = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    x = np.concatenate([x, ties, -ties, [0.0, 1.0, -2.5]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(om.round_bf16(x), want)


def pin_model_bf16(w):
    """The cache entries of a bf16 model (project_tokens with model_bf16)
    against a construction from other primitives: a float64 torch matmul,
    torch's float32 -> bfloat16 cast at each bf16 tensor of the wrapper
    forward listing (kv_lora, kv_c_normed, the roped k_pe), torch's rms_norm
    and RoPE as a complex rotation. With one-hot tokens kv_lora is a weight
    column (already bf16), and the entries are then the fp64 entries rounded
    once."""
    d, W = w.dims, w.weights
    c = d.kv_lora_rank
    S = w.x.shape[0]
    pos = int(w.prefix_lens[0]) + np.arange(S)

    def bf(t):
        return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)

    def build(x):
        kv = bf(torch.from_numpy(np.asarray(x, np.float64)) @
                torch.from_numpy(np.asarray(W["kv_a_proj_with_mqa"], np.float64)).T)
        lat = bf(torch.nn.functional.rms_norm(kv[:, :c], (c,), torch.from_numpy(
            np.asarray(W["kv_a_layernorm"], np.float64)), eps=d.rms_norm_eps))
        pe = bf(torch.from_numpy(_rope_complex(kv[:, c:].numpy(), pos, d.rope_theta, d.rope_style)))
        return torch.cat([lat, pe], 1).numpy()

    _, got, _ = om.project_tokens(d, W, w.x, pos, model_bf16=True)
    assert np.array_equal(got, build(w.x)), "bf16 entries differ from the torch construction"
    x1 = np.zeros_like(w.x)
    x1[np.arange(S), (7 * np.arange(S)) % d.hidden_size] = 1.0
    _, plain, _ = om.project_tokens(d, W, x1, pos)
    _, rounded, _ = om.project_tokens(d, W, x1, pos, model_bf16=True)
    want = torch.from_numpy(plain).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rounded, want)


def pin_fp8_cache(w, kv_scale: float):
    """Forward with an 8-bit cache: the new entries are stored as the codes an
    independent E4M3 implementation (torch's float8_e4m3fn cast) gives for
    entry / scale, and attention reads the stored values: the last query's
    output equals a one-token run whose prefix holds all stored entries
    before it."""
    d, W = w.dims, w.weights
    x = w.x
    pre = torch.from_numpy((np.asarray(w.prefix_rows[0], np.float32) / kv_scale).clip(-448, 448)).to(
        torch.float8_e4m3fn).to(torch.float64).numpy() * kv_scale
    out, ent, attn = om.forward_sequence(d, W, x, pre, w.mask_kind, w.window, kv_scale=kv_scale)
    _, ent_plain, _ = om.forward_sequence(d, W, x, pre, w.mask_kind, w.window)
    # torch's cast rounds the fp32 value: compare where the fp64 value is not
    # within fp32 rounding of a tie between two codes
    v = ent_plain / kv_scale
    expect = torch.from_numpy(v.clip(-448, 448)).to(torch.float8_e4m3fn).to(torch.float64).numpy() * kv_scale
    pos = np.sort(om.fp8_e4m3_decode(np.arange(1, 0x7F)))
    mids = np.concatenate([[2.0 ** -10], (pos[1:] + pos[:-1]) / 2])
    near_tie = np.min(np.abs(np.abs(v)[..., None] - mids), axis=-1) <= 1e-6 * np.maximum(np.abs(v), 1.0)
    assert np.array_equal(ent[~near_tie], expect[~near_tie]), "new entries are not stored as 8-bit values"
    S = x.shape[0]
    if w.mask_kind != om.MASK_SLIDING and S > 1:
        pre2 = np.concatenate([pre, ent[:-1]], axis=0)
        out2, ent2, _ = om.forward_sequence(d, W, x[-1:], pre2, w.mask_kind, w.window, kv_scale=kv_scale)
        assert np.array_equal(ent2[0], ent[-1])
        assert np.max(np.abs(out2[0] - out[-1])) <= 1e-12 * max(1.0, np.abs(out[-1]).max())


# --------------------------------------------------------------------------
# gradient of the expanded layer (training form)
# --------------------------------------------------------------------------

def _loss(dims, W, x, mask, window, dout, lo, hi):
    """<dout, out> of the oracle's forward on one training sequence (no prefix)."""
    pre = np.zeros((0, dims.kv_lora_rank + dims.qk_rope_head_dim))
    out, _, _ = om.forward_sequence(dims, W, x, pre, mask, window, row_lo=lo, row_hi=hi)
    return float(np.sum(out * dout))


def pin_backward_fd(w, rows=None, seed: int = 21):
    """Every gradient of oracle.backward against central finite differences
    of the oracle's forward (an independent code path: the forward is pinned
    on its own), along a random direction per tensor and at a few single
    elements. Five-point central stencil (truncation O(h^4)), h = 1e-4;
    agreement 1e-6 relative, plus the rounding of the loss differences
    (1e-14 sum|dout * out| / h)."""
    from oracle import backward as ob
    d, W = w.dims, {k: np.asarray(v, np.float64) for k, v in w.weights.items()}
    x = np.asarray(w.x, np.float64)
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((x.shape[0], d.hidden_size))
    lo, hi = (None, None) if rows is None else rows
    dx, dW, out = ob.backward_sequence(d, W, x, w.mask_kind, dout, w.window, lo, hi)
    pre = np.zeros((0, d.entry_dim))
    ref_out, _, _ = om.forward_sequence(d, W, x, pre, w.mask_kind, w.window, row_lo=lo, row_hi=hi)
    assert np.max(np.abs(out - ref_out)) <= 1e-12 * max(1.0, np.abs(ref_out).max())
    eps = 1e-4
    L0 = float(np.sum(np.abs(dout * ref_out)))
    tensors = {"x": (x, dx)}
    tensors.update({k: (W[k], dW[k]) for k in W})
    assert set(dW) == set(W), (set(dW), set(W))
    for name, (val, grad) in tensors.items():
        dirs = [rng.standard_normal(val.shape)]
        for _ in range(2):
            e = np.zeros(val.size)
            e[rng.integers(val.size)] = 1.0
            dirs.append(e.reshape(val.shape))
        for u in dirs:
            def at(t):
                if name == "x":
                    return _loss(d, W, val + t * u, w.mask_kind, w.window, dout, lo, hi)
                W2 = dict(W)
                W2[name] = val + t * u
                return _loss(d, W2, x, w.mask_kind, w.window, dout, lo, hi)
            fd = (8 * (at(eps) - at(-eps)) - (at(2 * eps) - at(-2 * eps))) / (12 * eps)
            an = float(np.sum(grad * u))
            scale = max(1e-3, abs(fd), np.sqrt(np.sum(grad * grad)) * np.sqrt(np.sum(u * u)) * 1e-3)
            assert abs(fd - an) <= 1e-6 * scale + 1e-14 * L0 / eps, (name, fd, an)


def pin_backward_autograd(w, seed: int = 22):
    """oracle.backward against torch.autograd of a float64 torch forward built
    from torch's own primitives (linear layers as matmuls, rms_norm, RoPE as a
    complex rotation, scaled_dot_product_attention with a boolean mask).
    Masks with at least one visible key per row. Agreement 1e-10 relative."""
    from oracle import backward as ob
    d = w.dims
    W = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in w.weights.items()}
    x = torch.tensor(np.asarray(w.x, np.float64), requires_grad=True)
    S, H, n, r, c, dv = x.shape[0], d.num_heads, d.qk_nope_head_dim, d.qk_rope_head_dim, d.kv_lora_rank, d.v_head_dim
    pos = torch.arange(S, dtype=torch.float64)
    inv = d.rope_theta ** (-2.0 * torch.arange(r // 2, dtype=torch.float64) / r)
    rot = torch.polar(torch.ones(S, r // 2, dtype=torch.float64), pos[:, None] * inv[None, :])

    def rope(t):  # t [S, ..., r]
        if d.rope_style == om.ROPE_NEOX:
            z = torch.complex(t[..., : r // 2], t[..., r // 2:])
        else:
            z = torch.complex(t[..., 0::2], t[..., 1::2])
        z = z * rot.reshape((S,) + (1,) * (t.dim() - 2) + (r // 2,))
        if d.rope_style == om.ROPE_NEOX:
            return torch.cat([z.real, z.imag], dim=-1)
        return torch.stack([z.real, z.imag], dim=-1).reshape(t.shape)

    rms = lambda t, g: torch.nn.functional.rms_norm(t, (t.shape[-1],), g, eps=d.rms_norm_eps)
    if d.q_lora_rank > 0:
        q = rms(x @ W["q_a_proj"].T, W["q_a_layernorm"]) @ W["q_b_proj"].T
    else:
        q = x @ W["q_proj"].T
    q = q.reshape(S, H, n + r)
    kv = x @ W["kv_a_proj_with_mqa"].T
    cn = rms(kv[:, :c], W["kv_a_layernorm"])
    Q = torch.cat([q[..., :n], rope(q[..., n:])], dim=-1)
    kvb = (cn @ W["kv_b_proj"].T).reshape(S, H, n + dv)
    K = torch.cat([kvb[..., :n], rope(kv[:, c:])[:, None, :].expand(S, H, r)], dim=-1)
    vis = np.zeros((S, S), dtype=bool)
    for i in range(S):
        a, b = om.visible_interval(i, S, w.mask_kind, w.window)
        vis[i, a:b] = True
    assert vis.any(axis=1).all()
    o = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1), K.transpose(0, 1), kvb[..., n:].transpose(0, 1), attn_mask=torch.from_numpy(vis),
        scale=1.0 / math.sqrt(n + r)).transpose(0, 1).reshape(S, H * dv)
    if d.use_output_gate:
        o = o * torch.sigmoid(x @ W["g_proj"].T)
    out = o @ W["o_proj"].T
    dout = np.random.default_rng(seed).standard_normal((S, d.hidden_size))
    out.backward(torch.from_numpy(dout))
    dx, dW, _ = ob.backward_sequence(d, w.weights, w.x, w.mask_kind, dout, w.window)
    assert _rel(dx, x.grad.numpy()) <= 1e-10
    for k in W:
        assert _rel(dW[k], W[k].grad.numpy()) <= 1e-10, k
