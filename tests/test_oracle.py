"""CPU pins of the fp64 oracle (no GPU), plus planted mistakes that each pin
must catch (mutation check, as in the SpecForge refactor-parity test that
scales Q by 1+1e-6 and drops empty-row zeroing)."""
import numpy as np
import pytest

import mla_synth as ms
from oracle import mla as om
from tests import oracle_pins as P


def _tiny(mask=ms.MASK_CAUSAL, window=0, **dims_kw):
    dims = P.tiny_dims(**dims_kw)
    return ms.make_workload("tiny", dims=dims, seed=5, q_lens=[9], prefix_lens=[6],
                            mask_kind=mask, window=window)


def test_page_dims():
    P.pin_page_dims()


def test_rms_norm():
    P.pin_rms_norm()


def test_rope():
    P.pin_rope()


def test_attention_core():
    P.pin_attention_core()


@pytest.mark.parametrize("variant", [
    dict(),
    dict(q_lora_rank=12, rope_style=om.ROPE_INTERLEAVED),
    dict(use_output_gate=True, rope_style=om.ROPE_INTERLEAVED),
])
@pytest.mark.parametrize("mask,window", [(ms.MASK_CAUSAL, 0), (ms.MASK_FULL, 0), (ms.MASK_SLIDING, 4)])
def test_brute_force(variant, mask, window):
    P.pin_brute_force(_tiny(mask, window, **variant))


def test_brute_force_tiny_config():
    """The tiny fp32 workload itself (hidden 256, 4 heads, 16 causal tokens)."""
    P.pin_brute_force(ms.make_workload("tiny_f32"))


def test_brute_force_gamma():
    dims = P.tiny_dims(q_lora_rank=10)
    w = ms.make_workload("tiny", dims=dims, seed=6, q_lens=[5], prefix_lens=[3], gamma_noise=True)
    P.pin_brute_force(w)


@pytest.mark.parametrize("variant", [dict(), dict(q_lora_rank=12, use_output_gate=True)])
def test_masks(variant):
    P.pin_masks(_tiny(**variant))


def test_window_trim():
    w = ms.make_workload("tiny", dims=P.tiny_dims(q_lora_rank=12, use_output_gate=True), seed=7,
                         q_lens=[3], prefix_lens=[40])
    P.pin_window_trim(w, window=5)
    with pytest.raises(ValueError):  # a query that would see a trimmed key
        om.forward_sequence(w.dims, w.weights, w.x, w.prefix_rows[0][10:], om.MASK_SLIDING, 40,
                            first_position=10)


def test_cache_consistency():
    P.pin_cache_consistency(_tiny(q_lora_rank=12), split=4)


def _small(name, **kw):
    """A named workload's model dims with a handful of short sequences."""
    return ms.make_workload(name, **kw)


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", dict()),
    ("draft_block_bf16", dict(q_lens=[16, 16], prefix_lens=[40, 3])),
    ("decode_bf16", dict(batch=3, len_range=(1, 70))),
    ("prefill_bf16", dict(q_lens=[37], prefix_lens=[0])),
    ("long_decode_bf16", dict(batch=2, len_range=(30, 90), window=16)),
])
def test_absorbed_equals_expanded(name, kw, workload_cache):
    key = ("abs", name)
    if key not in workload_cache:
        workload_cache[key] = _small(name, **kw)
    P.pin_absorbed_equals_expanded(workload_cache[key])


def test_dropped_block_rows():
    """Explicit empty intervals (a dropped draft block) give exact-zero rows
    through the batched entry too."""
    w = _tiny()
    S = w.total_tokens
    lo = np.zeros(S, np.int32)
    hi = np.full(S, 6 + S, np.int32)
    hi[2:5] = 0
    res = om.mla_forward(w.dims, w.weights, w.x, w.q_lens, w.prefix_rows, w.mask_kind,
                         row_lo=lo, row_hi=hi)
    out = res[0][0]
    assert np.all(out[2:5] == 0) and np.all(np.abs(out[5:]).max(1) > 0)


# --------------------------------------------------------------------------
# mutations: each planted mistake must make some pin fail
# --------------------------------------------------------------------------

def _expect_fail(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_mutation_scale_q(monkeypatch):
    orig = om.project_tokens

    def bad(*a, **k):
        q, e, g = orig(*a, **k)
        return q * (1 + 1e-6), e, g
    monkeypatch.setattr(om, "project_tokens", bad)
    _expect_fail(P.pin_brute_force, _tiny())


def test_mutation_drop_zeroing(monkeypatch):
    orig = om.attention_core

    def bad(q, k, v, lo, hi, scale, return_probs=False):
        lo = np.asarray(lo).copy()
        hi = np.asarray(hi).copy()
        empty = hi <= lo
        lo[empty], hi[empty] = 0, k.shape[0]  # an empty row silently attends to everything
        return orig(q, k, v, lo, hi, scale, return_probs)
    monkeypatch.setattr(om, "attention_core", bad)
    _expect_fail(P.pin_attention_core)
    _expect_fail(P.pin_masks, _tiny())


def test_mutation_rope_style(monkeypatch):
    orig = om.rope_pairs
    monkeypatch.setattr(om, "rope_pairs", lambda r, s: orig(r, 1 - s))
    _expect_fail(P.pin_rope)
    _expect_fail(P.pin_brute_force, _tiny())


def test_mutation_rope_sign(monkeypatch):
    orig = om.rope_angles
    monkeypatch.setattr(om, "rope_angles", lambda p, r, t: -orig(p, r, t))
    _expect_fail(P.pin_rope)


def test_mutation_window_off_by_one(monkeypatch):
    def bad(p, kv_len, kind, window):
        if kind == om.MASK_SLIDING:
            return max(0, p - window), min(p + 1, kv_len)
        return orig(p, kv_len, kind, window)
    orig = om.visible_interval
    monkeypatch.setattr(om, "visible_interval", bad)
    _expect_fail(P.pin_masks, _tiny())
    _expect_fail(P.pin_brute_force, _tiny(ms.MASK_SLIDING, 4))


def test_mutation_transposed_absorption(monkeypatch):
    """W_UV taken from the k_nope rows instead of the v rows (a swapped split)."""
    orig = om._absorbed_attention

    def bad(dims, W, q, entries, lo, hi, scale):
        W2 = dict(W)
        H, n, dv, c = dims.num_heads, dims.qk_nope_head_dim, dims.v_head_dim, dims.kv_lora_rank
        wk = np.asarray(W["kv_b_proj"]).reshape(H, n + dv, c)
        W2["kv_b_proj"] = np.concatenate([wk[:, :n], wk[:, n:][:, ::-1]], axis=1).reshape(-1, c)
        return orig(dims, W2, q, entries, lo, hi, scale)
    monkeypatch.setattr(om, "_absorbed_attention", bad)
    _expect_fail(P.pin_absorbed_equals_expanded, _tiny())


def test_mutation_cache_raw_latent(monkeypatch):
    """Caching the raw kv_c instead of the RMSNorm'd latent."""
    orig = om.rms_norm
    calls = {"n": 0}

    def bad(x, g, eps):
        calls["n"] += 1
        y = orig(x, g, eps)
        return np.asarray(x, np.float64) if x.shape[-1] == 16 else y
    monkeypatch.setattr(om, "rms_norm", bad)
    _expect_fail(P.pin_brute_force, _tiny())


def test_mutation_gate_dropped(monkeypatch):
    orig = om.project_tokens

    def bad(*a, **k):
        q, e, g = orig(*a, **k)
        return q, e, None
    monkeypatch.setattr(om, "project_tokens", bad)
    _expect_fail(P.pin_brute_force, _tiny(use_output_gate=True))


@pytest.mark.parametrize("variant", [dict(), dict(q_lora_rank=12, use_output_gate=True,
                                                  rope_style=om.ROPE_INTERLEAVED)])
def test_sparse_lists(variant):
    P.pin_sparse(_tiny(**variant))


def test_mutation_sparse_duplicates_once(monkeypatch):
    # set semantics (a position listed twice counted once) breaks the merge pin
    orig = om.listed_keys
    monkeypatch.setattr(om, "listed_keys", lambda key_list, L: np.unique(orig(key_list, L)))
    _expect_fail(P.pin_sparse, _tiny())


def test_mutation_sparse_range_filter(monkeypatch):
    # keeping position L (one past the sequence) wraps to another key
    monkeypatch.setattr(om, "listed_keys",
                        lambda key_list, L: (lambda i: i[(i >= 0) & (i <= L)] % L)(np.asarray(key_list).reshape(-1)))
    _expect_fail(P.pin_sparse, _tiny())


def test_fp8_e4m3():
    P.pin_fp8_e4m3()


def test_round_bf16():
    P.pin_round_bf16()


@pytest.mark.parametrize("variant", [dict(dtype="bf16"), dict(dtype="bf16", rope_style=om.ROPE_INTERLEAVED,
                                                              q_lora_rank=12)])
def test_model_bf16(variant):
    w = ms.make_workload("tiny", dims=P.tiny_dims(**variant), seed=5, q_lens=[9], prefix_lens=[6],
                         mask_kind=ms.MASK_CAUSAL, gamma_noise=True)
    P.pin_model_bf16(w)


@pytest.mark.parametrize("skip", [0, 1, 2])
def test_mutation_model_bf16_rounding_point(monkeypatch, skip):
    # leaving out any one of the three roundings (kv_lora, kv_c_normed, the
    # roped k_pe) fails the pin
    orig, calls = om.round_bf16, []

    def rnd(x):
        calls.append(1)
        return np.asarray(x, np.float64) if (len(calls) - 1) % 3 == skip else orig(x)
    monkeypatch.setattr(om, "round_bf16", rnd)
    w = ms.make_workload("tiny", dims=P.tiny_dims(dtype="bf16"), seed=5, q_lens=[9], prefix_lens=[6],
                         mask_kind=ms.MASK_CAUSAL)
    _expect_fail(P.pin_model_bf16, w)


@pytest.mark.parametrize("variant", [dict(), dict(q_lora_rank=12, use_output_gate=True)])
def test_fp8_cache(variant):
    P.pin_fp8_cache(_tiny(**variant), 0.0625)


def test_mutation_fp8_round_half_up(monkeypatch):
    # rounding ties away from zero instead of to the even code
    def enc(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.minimum(np.abs(v), om.FP8_E4M3_MAX)
        hi = np.clip(np.searchsorted(om._FP8_POS, a, side="left"), 0, 0x7E)
        lo = np.maximum(hi - 1, 0)
        code = np.where(om._FP8_POS[hi] - a <= a - om._FP8_POS[lo], hi, lo)
        return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(om, "fp8_e4m3_encode", enc)
    _expect_fail(P.pin_fp8_e4m3)


def test_mutation_fp8_new_entries_unquantized(monkeypatch):
    # attending to (and storing) the new entries at full precision
    monkeypatch.setattr(om, "fp8_quantize", lambda x, s: np.asarray(x, np.float64))
    _expect_fail(P.pin_fp8_cache, _tiny(), 0.0625)


def test_mutation_fp8_scale_inverted(monkeypatch):
    # multiplying by the scale where the definition divides
    monkeypatch.setattr(om, "fp8_quantize",
                        lambda x, s: om.fp8_e4m3_decode(om.fp8_e4m3_encode(np.asarray(x, np.float64) * s)) / s)
    _expect_fail(P.pin_fp8_cache, _tiny(), 0.0625)


# ------------------------------------------------------------ backward pass

def _train(mask=ms.MASK_CAUSAL, window=0, S=9, **dims_kw):
    return ms.make_workload("tiny", dims=P.tiny_dims(**dims_kw), seed=6, q_lens=[S], prefix_lens=[0],
                            mask_kind=mask, window=window, gamma_noise=True)


_BW_VARIANTS = [
    dict(),
    dict(q_lora_rank=12, use_output_gate=True, rope_style=om.ROPE_INTERLEAVED),
]


@pytest.mark.parametrize("variant", _BW_VARIANTS)
@pytest.mark.parametrize("mask,window", [(ms.MASK_CAUSAL, 0), (ms.MASK_FULL, 0), (ms.MASK_SLIDING, 3)])
def test_backward_finite_differences(variant, mask, window):
    P.pin_backward_fd(_train(mask, window, **variant))


def test_backward_finite_differences_dropped_rows():
    # explicit intervals: an empty row (its output is the constant 0) and a
    # row that sees only earlier keys
    lo = np.array([0, 0, 0, 5, 0, 0, 1, 0, 0])
    hi = np.array([1, 2, 3, 5, 5, 6, 4, 8, 9])
    P.pin_backward_fd(_train(q_lora_rank=12, use_output_gate=True), rows=(lo, hi))


@pytest.mark.parametrize("variant", _BW_VARIANTS)
@pytest.mark.parametrize("mask,window", [(ms.MASK_CAUSAL, 0), (ms.MASK_SLIDING, 4)])
def test_backward_autograd(variant, mask, window):
    P.pin_backward_autograd(_train(mask, window, **variant))


def test_mutation_backward_softmax_no_row_term(monkeypatch):
    # dS = P * dP (the row term sum_j P_j dP_j left out)
    from oracle import backward as ob

    def bad(q, k, v, lo, hi, scale, do):
        _, _, Pr = om.attention_core(q, k, v, lo, hi, scale, return_probs=True)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for h in range(q.shape[1]):
            Ph = Pr[:, h, :]
            dv[:, h] = Ph.T @ do[:, h]
            dS = Ph * (do[:, h] @ v[:, h].T)
            dq[:, h], dk[:, h] = scale * dS @ k[:, h], scale * dS.T @ q[:, h]
        return dq, dk, dv
    monkeypatch.setattr(ob, "attention_backward", bad)
    _expect_fail(P.pin_backward_fd, _train())


def test_mutation_backward_rope_forward_turn(monkeypatch):
    # the gradient turned by +angle instead of -angle
    from oracle import backward as ob
    monkeypatch.setattr(ob, "rope_backward", lambda dy, pos, theta, style: om.apply_rope(dy, pos, theta, style))
    _expect_fail(P.pin_backward_fd, _train())


def test_mutation_backward_rope_key_one_head(monkeypatch):
    # the shared rope key's gradient taken from head 0 only
    from oracle import backward as ob
    orig = ob.attention_backward

    def bad(q, k, v, lo, hi, scale, do):
        dq, dk, dv = orig(q, k, v, lo, hi, scale, do)
        dk = dk.copy()
        dk[:, 1:, -k.shape[2] + q.shape[2] - 6:] = 0.0  # rope part (r = 6) of heads >= 1
        return dq, dk, dv
    monkeypatch.setattr(ob, "attention_backward", bad)
    _expect_fail(P.pin_backward_fd, _train())


def test_mutation_backward_rmsnorm_no_mean_term(monkeypatch):
    # dx = rho * dy * gamma only (the statistic's own dependence left out)
    from oracle import backward as ob

    def bad(x, gamma, eps, dy):
        rho = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
        return rho * dy * gamma, np.sum(dy * x * rho, axis=0)
    monkeypatch.setattr(ob, "rms_norm_backward", bad)
    _expect_fail(P.pin_backward_fd, _train())
