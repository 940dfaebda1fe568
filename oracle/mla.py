"""Plain fp64 oracle of the MLA forward (test infrastructure only).

Everything is float64 numpy; inputs are the same dtype-rounded values the GPU
receives, upcast. Nothing here is blocked, fused or reordered beyond the
definitions below; a matmul is the only library primitive used. One option
leaves fp64: model_bf16 keeps the three tensors that the MLA blog's wrapper
forward hands to the cache update as bf16 values (kv_lora, kv_c_normed and
the roped k_pe of a bf16 model), the precision in which an 8-bit cache's
codes are decided (a code is an integer decision). Every function is pinned
by the CPU tests (tests/oracle_pins.py), including the E4M3 encode/decode
against torch's float8_e4m3fn cast, round_bf16 against torch's bfloat16 cast
and the model_bf16 entries against a torch construction of them.

Notation (as on the pages): n = qk_nope_head_dim, r = qk_rope_head_dim,
c = kv_lora_rank, dv = v_head_dim, H = heads, E = c + r (one cache entry).
Weights are nn.Linear [out, in] matrices named as on the pages.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

MASK_FULL = 0
MASK_CAUSAL = 1
MASK_SLIDING = 2
ROPE_NEOX = 0
ROPE_INTERLEAVED = 1


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# building blocks
# ---------------------------------------------------------------------------

# 8-bit cache entries. The MLA blog's MLAAttention.forward listing computes
# dynamic q/k/v scales for an FP8 KV cache, and its cache-shape listings name
# a packed 656-byte fp8 format without specifying its packing; the plain
# reading taken here: each of the 576 values of an entry is one OCP E4M3
# ("fn": no infinities, one NaN per sign) code of value / scale, with one
# scale per cache tensor.
FP8_E4M3_MAX = 448.0


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 encodes m/8 * 2^-6, others
    (1 + m/8) * 2^(e-7); codes 0x7F / 0xFF are NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, s * mag)


_FP8_POS = fp8_e4m3_decode(np.arange(0x7F))  # the 127 finite non-negative values, increasing


def fp8_e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of v (a tie goes to the code with an even mantissa),
    saturating to +-448; the sign of zero is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), FP8_E4M3_MAX)
    hi = np.clip(np.searchsorted(_FP8_POS, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _FP8_POS[lo], _FP8_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def round_bf16(x) -> np.ndarray:
    """x rounded to fp32 and then to the nearest bfloat16 (ties to even), as
    fp64 values: the storage of a result accumulated in fp32 and kept in a
    bf16 buffer."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def fp8_quantize(x, scale: float) -> np.ndarray:
    """The value an 8-bit cache holds for x: decode(encode(x / scale)) * scale."""
    return fp8_e4m3_decode(fp8_e4m3_encode(_f64(x) / scale)) * scale


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    The MLA blog applies it to the low-rank query (q_a_layernorm) and to the
    compressed KV latent before it is cached (kv_a_layernorm), in the
    DeepseekV2MLAAttention.__init__ and MultiHeadLatentAttentionWrapper.forward
    listings; the pages name the layer without its formula, so this is the
    textbook definition."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gamma)


def rope_pairs(rot_dim: int, style: int) -> Tuple[np.ndarray, np.ndarray]:
    """Index pairs (a_j, b_j), j < rot_dim/2, rotated together by angle_j.

    SpecForge PR "Add config-selectable MLA draft attention" (Summary) names
    interleaved and NeoX partial RoPE without defining them; the textbook
    conventions are: NeoX pairs (j, j + r/2), interleaved pairs (2j, 2j + 1)."""
    j = np.arange(rot_dim // 2)
    if style == ROPE_NEOX:
        return j, j + rot_dim // 2
    if style == ROPE_INTERLEAVED:
        return 2 * j, 2 * j + 1
    raise ValueError(style)


def rope_angles(positions, rot_dim: int, theta: float) -> np.ndarray:
    """angle[p, j] = p * theta^(-2j / rot_dim)  (the rotary dim is r only)."""
    j = np.arange(rot_dim // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * j / rot_dim)
    return _f64(positions)[:, None] * inv_freq[None, :]


def apply_rope(x, positions, theta: float, style: int) -> np.ndarray:
    """Rotate each pair (x_a, x_b) -> (x_a cos - x_b sin, x_a sin + x_b cos).

    x has the token axis first ([S, r] or [S, H, r]); positions is [S]. The MLA
    blog rotates only q[..., n:] and k_pe (MultiHeadLatentAttentionWrapper.forward
    listing); the nope part of q is not rotated."""
    x = _f64(x)
    r = x.shape[-1]
    a, b = rope_pairs(r, style)
    ang = rope_angles(positions, r, theta)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (r // 2,)
    cos = np.cos(ang).reshape(shape)
    sin = np.sin(ang).reshape(shape)
    out = x.copy()
    xa, xb = x[..., a], x[..., b]
    out[..., a] = xa * cos - xb * sin
    out[..., b] = xa * sin + xb * cos
    return out


def visible_interval(p: int, kv_len: int, mask_kind: int, window: int) -> Tuple[int, int]:
    """Visible keys [lo, hi) of a query at logical position p (key position =
    cache index). Full: all kv_len keys. Causal: keys <= p. Sliding window W:
    p - W < j <= p (exactly W keys including itself). SpecForge PR "extract
    GQA/MLA attention into reusable layers" (Modifications) applies causal and
    window masks by logical position; the window boundary is not written out
    on the pages, this is the plainest reading."""
    if mask_kind == MASK_FULL:
        return 0, kv_len
    if mask_kind == MASK_CAUSAL:
        return 0, min(p + 1, kv_len)
    if mask_kind == MASK_SLIDING:
        return max(0, p - window + 1), min(p + 1, kv_len)
    raise ValueError(mask_kind)


def attention_core(q, k, v, lo, hi, scale: float, return_probs: bool = False):
    """Softmax attention per head over visible keys [lo_i, hi_i).

    q [S, H, d], k [L, Hk, d], v [L, Hk, dv] with Hk = H or 1 (one shared
    key/value head, MQA-style, as the latent cache is in the MLA blog's
    MLAAttention.__init__ listing). s_j = scale * q.k_j; p = softmax over the
    visible j (max subtracted); o = sum_j p_j v_j. A query with no visible key
    gets o = 0 and lse = -inf (fully-masked-query zeroing, SpecForge PR "Add
    config-selectable MLA draft attention", Structure)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, H, _ = q.shape
    L = k.shape[0]
    dv = v.shape[-1]
    lo = np.asarray(lo, dtype=np.int64)
    hi = np.asarray(hi, dtype=np.int64)
    o = np.zeros((S, H, dv))
    lse = np.full((S, H), -np.inf)
    probs = np.zeros((S, H, L)) if return_probs else None
    j = np.arange(L)
    vis = (j[None, :] >= lo[:, None]) & (j[None, :] < hi[:, None])  # [S, L]
    has_key = vis.any(axis=1)
    for h in range(H):
        kh = k[:, h if k.shape[1] > 1 else 0, :]
        vh = v[:, h if v.shape[1] > 1 else 0, :]
        s = scale * (q[:, h, :] @ kh.T)  # [S, L]
        s = np.where(vis, s, -np.inf)
        m = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(s - m[:, None]), 0.0)
        z = e.sum(axis=1)
        p = np.where(has_key[:, None], e / np.where(has_key, z, 1.0)[:, None], 0.0)
        o[:, h, :] = p @ vh
        lse[:, h] = np.where(has_key, m + np.log(np.where(has_key, z, 1.0)), -np.inf)
        if return_probs:
            probs[:, h, :] = p
    if return_probs:
        return o, lse, probs
    return o, lse


# ---------------------------------------------------------------------------
# the MLA layer
# ---------------------------------------------------------------------------

def project_tokens(dims, W: Dict[str, np.ndarray], x, positions, model_bf16: bool = False):
    """Projections of the new tokens (MLA blog, MultiHeadLatentAttentionWrapper.forward
    and DeepseekV2MLAAttention.__init__ listings).

    With a low-rank Q: q_c = x W_qa^T, q_c <- RMSNorm(q_c), q = q_c W_qb^T; else
    q = x W_q^T. kv = x W_kva^T split [c | r] into kv_c and k_pe; the cached
    latent is RMSNorm(kv_c) (not the raw kv_c). q is viewed [S, H, n + r], nope
    first; RoPE rotates q[..., n:] and k_pe (one rope key shared by all heads).

    Returns q [S, H, n+r], the cache entries [S, E] = [RMSNorm(kv_c) | rope(k_pe)]
    (the layout concat_and_cache_mla writes, do_kv_cache_update listing), and
    the output-gate value sigma(x W_g^T) [S, H*dv] or None.
    model_bf16: the layer's activations are bf16 tensors. In the wrapper
    forward listing the cache entry is built from three of them: kv_lora
    (the kv projection's output), kv_c_normed (kv_a_layernorm's output) and
    k_pe after the rotary embedding; each is rounded to bf16 where the
    listing produces it (round_bf16), the arithmetic in between stays fp64.
    The query path is not rounded."""
    x = _f64(x)
    S = x.shape[0]
    H, n, r, c = dims.num_heads, dims.qk_nope_head_dim, dims.qk_rope_head_dim, dims.kv_lora_rank
    eps = dims.rms_norm_eps
    if dims.q_lora_rank > 0:
        q_c = x @ _f64(W["q_a_proj"]).T
        q_c = rms_norm(q_c, W["q_a_layernorm"], eps)
        q = q_c @ _f64(W["q_b_proj"]).T
    else:
        q = x @ _f64(W["q_proj"]).T
    q = q.reshape(S, H, n + r).copy()
    kv = x @ _f64(W["kv_a_proj_with_mqa"]).T
    if model_bf16:
        kv = round_bf16(kv)
    kv_c, k_pe = kv[:, :c], kv[:, c:]
    kv_c_normed = rms_norm(kv_c, W["kv_a_layernorm"], eps)
    q[:, :, n:] = apply_rope(q[:, :, n:], positions, dims.rope_theta, dims.rope_style)
    k_pe = apply_rope(k_pe, positions, dims.rope_theta, dims.rope_style)
    if model_bf16:
        kv_c_normed, k_pe = round_bf16(kv_c_normed), round_bf16(k_pe)
    entries = np.concatenate([kv_c_normed, k_pe], axis=1)
    gate = None
    if dims.use_output_gate:
        gate = 1.0 / (1.0 + np.exp(-(x @ _f64(W["g_proj"]).T)))
    return q, entries, gate


def expand_kv(dims, W, entries):
    """Expanded K and V from cache entries (MLA blog, forward_mha listing):
    [k_nope | v] = c_n W_kvb^T viewed [L, H, n + dv]; K = [k_nope, k_pe] with the
    one shared k_pe broadcast to every head."""
    entries = _f64(entries)
    L = entries.shape[0]
    H, n, dv, c = dims.num_heads, dims.qk_nope_head_dim, dims.v_head_dim, dims.kv_lora_rank
    kvb = (entries[:, :c] @ _f64(W["kv_b_proj"]).T).reshape(L, H, n + dv)
    k_nope, v = kvb[:, :, :n], kvb[:, :, n:]
    k_pe = np.broadcast_to(entries[:, None, c:], (L, H, entries.shape[1] - c))
    k = np.concatenate([k_nope, k_pe], axis=2)
    return k, v


def _absorbed_attention(dims, W, q, entries, lo, hi, scale):
    """Absorbed form (MLA blog, the decode branch and forward_mqa listing):
    ql_nope[h] = q_nope[h] W_UK[h] with W_UK[h] the k_nope rows of head h of
    kv_b_proj; scores over the whole E-wide cache entry with the query
    [ql_nope, q_pe]; latent output o_lat = sum p_j c_j over the first c dims;
    out_v[h] = W_UV[h] o_lat[h] with W_UV[h] the v rows of head h."""
    H, n, dv, c = dims.num_heads, dims.qk_nope_head_dim, dims.v_head_dim, dims.kv_lora_rank
    Wkvb = _f64(W["kv_b_proj"]).reshape(H, n + dv, c)
    W_UK, W_UV = Wkvb[:, :n, :], Wkvb[:, n:, :]
    ql_nope = np.einsum("shn,hnc->shc", q[:, :, :n], W_UK)
    q_lat = np.concatenate([ql_nope, q[:, :, n:]], axis=2)
    entries = _f64(entries)
    o_lat, _ = attention_core(q_lat, entries[:, None, :], entries[:, None, :c], lo, hi, scale)
    return np.einsum("shc,hvc->shv", o_lat, W_UV)


def listed_keys(key_list, L: int) -> np.ndarray:
    """The keys a query of a sparse (top-k) attention sees: its listed logical
    positions, in list order, without the entries outside [0, L) (padding
    -1 and positions past the sequence). Each list slot is one key: a
    position listed twice is attended twice. The pages leave the indexer
    that produces the lists unspecified (MLA blog, the indexer branch of
    MultiHeadLatentAttentionWrapper.forward), so the lists are inputs."""
    idx = np.asarray(key_list, dtype=np.int64).reshape(-1)
    return idx[(idx >= 0) & (idx < L)]


def forward_sequence(dims, W, x, prefix_rows, mask_kind: int, window: int = 0,
                     rows: Optional[Sequence[int]] = None, row_lo=None, row_hi=None,
                     form: str = "expanded", softmax_scale: Optional[float] = None,
                     first_position: int = 0, key_lists=None, kv_scale: Optional[float] = None,
                     model_bf16: bool = False):
    """One sequence: S new tokens at logical positions P..P+S-1 after P cached
    prefix entries. The new entries are appended to the cache before attention,
    so each query sees its own entry (MLAAttention.forward listing: cache update
    first, then attention).

    rows: indices (within the sequence) of the queries to compute outputs for
    (default all). row_lo/row_hi: explicit visible intervals [lo, hi) of
    positions per new token, replacing the mask (clamped to [0, L)).
    first_position: the given prefix rows are the cache entries at positions
    first_position .. first_position + P - 1 (a window of a longer cache); every
    selected query must then see no key before first_position.
    key_lists: sparse (top-k) attention, one list of logical key positions
    per selected query (listed_keys), replacing the mask: a sparse backend
    runs every token in the MQA form over its selected entries (MLA blog,
    MLAAttention.forward listing, the sparse branch); the result is the same
    attention restricted to those keys, evaluated here in the given form.
    kv_scale: an 8-bit cache with this scale (fp8_quantize): the given prefix
    rows are the values it holds, the new entries are stored (and returned)
    quantized, and attention reads the stored values.
    model_bf16: the new entries are built from the bf16 tensors of a bf16
    model (project_tokens). Quantizing decides an integer code, and the cache
    update listing encodes those bf16 values; every other step stays fp64.
    Returns (out [len(rows), hidden], new entries [S, E], attn [len(rows), H*dv])."""
    x = _f64(x)
    prefix_rows = _f64(prefix_rows).reshape(-1, dims.kv_lora_rank + dims.qk_rope_head_dim)
    S, P = x.shape[0], prefix_rows.shape[0]
    f0 = int(first_position)
    L = f0 + P + S  # absolute length of the sequence
    H, dv = dims.num_heads, dims.v_head_dim
    scale = softmax_scale if softmax_scale else 1.0 / math.sqrt(dims.qk_nope_head_dim + dims.qk_rope_head_dim)
    positions = f0 + P + np.arange(S)
    q, new_entries, gate = project_tokens(dims, W, x, positions, model_bf16=model_bf16)
    if kv_scale is not None:
        new_entries = fp8_quantize(new_entries, kv_scale)
    entries = np.concatenate([prefix_rows, new_entries], axis=0)
    sel = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    if row_lo is not None:
        lo = np.clip(np.asarray(row_lo, dtype=np.int64)[sel], 0, L)
        hi = np.clip(np.asarray(row_hi, dtype=np.int64)[sel], 0, L)
    else:
        iv = [visible_interval(int(positions[i]), L, mask_kind, window) for i in sel]
        lo = np.array([a for a, _ in iv], dtype=np.int64)
        hi = np.array([b for _, b in iv], dtype=np.int64)
    if f0:
        if np.any((lo < f0) & (hi > lo)):
            raise ValueError("a query sees keys before first_position")
        lo, hi = np.maximum(lo - f0, 0), np.maximum(hi - f0, 0)
    if key_lists is not None:
        if f0 or len(key_lists) != len(sel):
            raise ValueError("key_lists: one list per selected query, whole cache given")
        o = np.zeros((len(sel), H, dv))
        if form == "expanded":
            k, v = expand_kv(dims, W, entries)
        for r, i in enumerate(sel):
            idx = listed_keys(key_lists[r], L)
            if form == "expanded":
                o[r] = attention_core(q[i:i + 1], k[idx], v[idx], [0], [len(idx)], scale)[0][0]
            elif form == "absorbed":
                o[r] = _absorbed_attention(dims, W, q[i:i + 1], entries[idx], [0], [len(idx)], scale)[0]
            else:
                raise ValueError(form)
    elif form == "expanded":
        k, v = expand_kv(dims, W, entries)
        o, _ = attention_core(q[sel], k, v, lo, hi, scale)
    elif form == "absorbed":
        o = _absorbed_attention(dims, W, q[sel], entries, lo, hi, scale)
    else:
        raise ValueError(form)
    attn = o.reshape(len(sel), H * dv)
    if gate is not None:
        attn = attn * gate[sel]
    out = attn @ _f64(W["o_proj"]).T
    return out, new_entries, attn


def mla_forward(dims, W, x, q_lens, prefix_rows: List[np.ndarray], mask_kind: int,
                window: int = 0, row_lo=None, row_hi=None, form: str = "expanded",
                seqs: Optional[Sequence[int]] = None, rows_per_seq: Optional[dict] = None,
                softmax_scale: Optional[float] = None, first_positions: Optional[dict] = None,
                key_lists: Optional[dict] = None, kv_scale: Optional[float] = None,
                model_bf16: bool = False):
    """A batch of sequences packed along the token axis (x is [sum q_lens, hidden]).

    seqs: the sequences to evaluate (default all); rows_per_seq: optional
    {seq: [row indices]} subset of queries; first_positions: optional
    {seq: position of its first given prefix row}; key_lists: optional
    {seq: one key list per evaluated query} (sparse attention, see
    forward_sequence). Returns dict seq -> (out, entries, attn)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    res = {}
    for b in (range(len(q_lens)) if seqs is None else seqs):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        lo = hi = None
        if row_lo is not None:
            lo, hi = np.asarray(row_lo)[s0:s1], np.asarray(row_hi)[s0:s1]
        rows = None if rows_per_seq is None else rows_per_seq.get(b)
        res[b] = forward_sequence(dims, W, np.asarray(x)[s0:s1], prefix_rows[b], mask_kind, window,
                                  rows=rows, row_lo=lo, row_hi=hi, form=form,
                                  softmax_scale=softmax_scale,
                                  first_position=0 if first_positions is None else first_positions.get(b, 0),
                                  key_lists=None if key_lists is None else key_lists.get(b), kv_scale=kv_scale,
                                  model_bf16=model_bf16)
    return res


# ---------------------------------------------------------------------------
# brute force: scalar Python loops, for tiny shapes only
# ---------------------------------------------------------------------------

def brute_force_forward(dims, W, x, prefix_rows, mask_kind: int, window: int = 0):
    """The same layer written as scalar loops over Python floats (no numpy
    arithmetic), used to pin the vectorised oracle on tiny shapes. Follows the
    same page definitions step by step, independently of the helpers above."""
    H, n, r, c, dv = (dims.num_heads, dims.qk_nope_head_dim, dims.qk_rope_head_dim,
                      dims.kv_lora_rank, dims.v_head_dim)
    eps, theta = float(dims.rms_norm_eps), float(dims.rope_theta)
    Wl = {k: np.asarray(v, dtype=np.float64).tolist() for k, v in W.items()}
    xs = np.asarray(x, dtype=np.float64).tolist()
    pre = np.asarray(prefix_rows, dtype=np.float64).reshape(-1, c + r).tolist()
    S, P = len(xs), len(pre)
    scale = 1.0 / math.sqrt(n + r)

    def linear(vec, mat):  # mat is [out][in]
        return [sum(wi * vi for wi, vi in zip(row, vec)) for row in mat]

    def rmsn(vec, g):
        ms = sum(t * t for t in vec) / len(vec)
        d = math.sqrt(ms + eps)
        return [t / d * gi for t, gi in zip(vec, g)]

    def rot(vec, pos):
        out = list(vec)
        half = r // 2
        for j in range(half):
            ang = pos * theta ** (-2.0 * j / r)
            if dims.rope_style == ROPE_NEOX:
                a, b = j, j + half
            else:
                a, b = 2 * j, 2 * j + 1
            out[a] = vec[a] * math.cos(ang) - vec[b] * math.sin(ang)
            out[b] = vec[a] * math.sin(ang) + vec[b] * math.cos(ang)
        return out

    qs, ents, gates = [], [], []
    for i in range(S):
        pos = P + i
        if dims.q_lora_rank > 0:
            qv = linear(rmsn(linear(xs[i], Wl["q_a_proj"]), Wl["q_a_layernorm"]), Wl["q_b_proj"])
        else:
            qv = linear(xs[i], Wl["q_proj"])
        heads = []
        for h in range(H):
            hv = qv[h * (n + r):(h + 1) * (n + r)]
            heads.append(hv[:n] + rot(hv[n:], pos))
        qs.append(heads)
        kv = linear(xs[i], Wl["kv_a_proj_with_mqa"])
        ents.append(rmsn(kv[:c], Wl["kv_a_layernorm"]) + rot(kv[c:], pos))
        if dims.use_output_gate:
            gates.append([1.0 / (1.0 + math.exp(-t)) for t in linear(xs[i], Wl["g_proj"])])
    allents = pre + ents
    L = len(allents)
    # expanded keys/values
    kvb = [linear(e[:c], Wl["kv_b_proj"]) for e in allents]
    outs = []
    for i in range(S):
        pos = P + i
        if mask_kind == MASK_FULL:
            lo, hi = 0, L
        elif mask_kind == MASK_CAUSAL:
            lo, hi = 0, pos + 1
        else:
            lo, hi = max(0, pos - window + 1), pos + 1
        attn = []
        for h in range(H):
            if hi <= lo:
                attn.extend([0.0] * dv)
                continue
            sc = []
            for j in range(lo, hi):
                kn = kvb[j][h * (n + dv):h * (n + dv) + n]
                kk = kn + allents[j][c:]
                sc.append(scale * sum(a * b for a, b in zip(qs[i][h], kk)))
            m = max(sc)
            ex = [math.exp(t - m) for t in sc]
            z = sum(ex)
            acc = [0.0] * dv
            for jj, j in enumerate(range(lo, hi)):
                vv = kvb[j][h * (n + dv) + n:(h + 1) * (n + dv)]
                for d in range(dv):
                    acc[d] += ex[jj] / z * vv[d]
            attn.extend(acc)
        if dims.use_output_gate:
            attn = [a * g for a, g in zip(attn, gates[i])]
        outs.append(linear(attn, Wl["o_proj"]))
    return np.array(outs), np.array(ents)
