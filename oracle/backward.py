"""Plain fp64 gradient of the expanded MLA layer (test infrastructure only).

The training side of the pages: SpecForge PR "Add config-selectable MLA draft
attention" makes MLA a draft-model attention that is trained, and validates it
with gradients (Validation), as does PR "extract GQA/MLA attention into
reusable layers" (Accuracy Test: outputs, gradients and optimizer steps). The
forward is the expanded form of the MLA blog (MultiHeadLatentAttentionWrapper
.forward and forward_mha listings) on whole training sequences: no cached
prefix, token i at position i. Its gradient with respect to the layer input
and every weight follows by the chain rule through the same steps, taken in
reverse; each rule below is the derivative of the forward step it names.
Everything is float64 numpy; a matmul is the only library primitive used.
Pinned by tests/oracle_pins.py (central finite differences of the oracle's
own forward, torch.autograd in float64, planted mistakes).

Notation as in oracle.mla: n = qk_nope_head_dim, r = qk_rope_head_dim,
c = kv_lora_rank, dv = v_head_dim, H heads. Loss convention: the caller gives
dout = dL/dout [S, hidden]; the function returns dL/dx [S, hidden] and
dL/dW for each weight, in the weight's own [out, in] (or [n]) layout.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import mla as om


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rms_norm_backward(x, gamma, eps: float, dy):
    """Gradient of y = x * rho * gamma, rho = (mean(x^2) + eps)^(-1/2) over
    the last axis (N values), for rows of x. With g = dy * gamma:
    dx = rho * g - x * rho^3 * sum(g * x) / N, and dgamma = sum over rows of
    dy * x * rho."""
    x, dy, gamma = _f64(x), _f64(dy), _f64(gamma)
    N = x.shape[-1]
    rho = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = dy * gamma
    dx = rho * g - x * rho ** 3 * np.sum(g * x, axis=-1, keepdims=True) / N
    dgamma = np.sum(dy * x * rho, axis=0)
    return dx, dgamma


def rope_backward(dy, positions, theta: float, style: int):
    """RoPE turns each pair by the angle p * theta^(-2j/r); its Jacobian is
    that rotation matrix, whose transpose is the turn by the opposite angle,
    i.e. the same rotation at position -p."""
    return om.apply_rope(dy, -np.asarray(positions, dtype=np.float64), theta, style)


def attention_backward(q, k, v, lo, hi, scale: float, do):
    """Gradient of the softmax attention of oracle.mla.attention_core (one
    key/value set per head, k [L, H, d], v [L, H, dv]) given do [S, H, dv].
    With P the probabilities over the visible keys and o = P v:
    dv = P^T do; dP = do v^T; dS = P * (dP - sum_j P_j dP_j) (the softmax
    Jacobian); ds/dq = scale * k, ds/dk = scale * q, so dq = scale * dS k and
    dk = scale * dS^T q. Rows with no visible key have P = 0 and pass no
    gradient (their output is the constant 0)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, P = om.attention_core(q, k, v, lo, hi, scale, return_probs=True)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(q.shape[1]):
        Ph = P[:, h, :]
        dv[:, h, :] = Ph.T @ do[:, h, :]
        dP = do[:, h, :] @ v[:, h, :].T
        dS = Ph * (dP - np.sum(Ph * dP, axis=1, keepdims=True))
        dq[:, h, :] = scale * dS @ k[:, h, :]
        dk[:, h, :] = scale * dS.T @ q[:, h, :]
    return dq, dk, dv


def backward_sequence(dims, W: Dict[str, np.ndarray], x, mask_kind: int, dout, window: int = 0,
                      row_lo=None, row_hi=None, softmax_scale: Optional[float] = None):
    """Gradient of one training sequence (S tokens at positions 0..S-1, no
    prefix) of the expanded MLA layer. row_lo / row_hi: explicit visible
    intervals [lo, hi) replacing the mask. Returns (dx [S, hidden],
    {weight name: dW}, out [S, hidden])."""
    x, dout = _f64(x), _f64(dout)
    S = x.shape[0]
    H, n, r, c, dv = (dims.num_heads, dims.qk_nope_head_dim, dims.qk_rope_head_dim, dims.kv_lora_rank,
                      dims.v_head_dim)
    eps = dims.rms_norm_eps
    theta, style = dims.rope_theta, dims.rope_style
    scale = softmax_scale if softmax_scale else 1.0 / math.sqrt(n + r)
    pos = np.arange(S)
    Wf = {k: _f64(v) for k, v in W.items()}

    # forward, keeping what the backward needs
    if dims.q_lora_rank > 0:
        qa = x @ Wf["q_a_proj"].T
        qn = om.rms_norm(qa, Wf["q_a_layernorm"], eps)
        q = qn @ Wf["q_b_proj"].T
    else:
        q = x @ Wf["q_proj"].T
    q = q.reshape(S, H, n + r)
    kv = x @ Wf["kv_a_proj_with_mqa"].T
    kvc, kpe = kv[:, :c], kv[:, c:]
    cn = om.rms_norm(kvc, Wf["kv_a_layernorm"], eps)
    qr = om.apply_rope(q[:, :, n:], pos, theta, style)
    kr = om.apply_rope(kpe, pos, theta, style)
    Q = np.concatenate([q[:, :, :n], qr], axis=2)
    kvb = (cn @ Wf["kv_b_proj"].T).reshape(S, H, n + dv)
    kn, V = kvb[:, :, :n], kvb[:, :, n:]
    K = np.concatenate([kn, np.broadcast_to(kr[:, None, :], (S, H, r))], axis=2)
    if row_lo is not None:
        lo = np.clip(np.asarray(row_lo, dtype=np.int64), 0, S)
        hi = np.clip(np.asarray(row_hi, dtype=np.int64), 0, S)
    else:
        iv = [om.visible_interval(i, S, mask_kind, window) for i in range(S)]
        lo = np.array([a for a, _ in iv], dtype=np.int64)
        hi = np.array([b for _, b in iv], dtype=np.int64)
    O, _ = om.attention_core(Q, K, V, lo, hi, scale)
    Of = O.reshape(S, H * dv)
    gate = None
    if dims.use_output_gate:
        gate = 1.0 / (1.0 + np.exp(-(x @ Wf["g_proj"].T)))
        A = Of * gate
    else:
        A = Of
    out = A @ Wf["o_proj"].T

    # backward, step by step in reverse
    dW: Dict[str, np.ndarray] = {}
    dW["o_proj"] = dout.T @ A                       # out = A Wo^T
    dA = dout @ Wf["o_proj"]
    dx = np.zeros_like(x)
    if gate is not None:                              # A = Of * sigma(x Wg^T)
        dOf = dA * gate
        dgp = dA * Of * gate * (1.0 - gate)
        dW["g_proj"] = dgp.T @ x
        dx += dgp @ Wf["g_proj"]
    else:
        dOf = dA
    dQ, dK, dV = attention_backward(Q, K, V, lo, hi, scale, dOf.reshape(S, H, dv))
    dkn = dK[:, :, :n]
    dkr = dK[:, :, n:].sum(axis=1)                    # k_pe is shared by every head
    dkvb = np.concatenate([dkn, dV], axis=2).reshape(S, H * (n + dv))
    dW["kv_b_proj"] = dkvb.T @ cn                     # [k_nope | v] = cn Wkvb^T
    dcn = dkvb @ Wf["kv_b_proj"]
    dkvc, dW["kv_a_layernorm"] = rms_norm_backward(kvc, Wf["kv_a_layernorm"], eps, dcn)
    dkpe = rope_backward(dkr, pos, theta, style)
    dkv = np.concatenate([dkvc, dkpe], axis=1)
    dW["kv_a_proj_with_mqa"] = dkv.T @ x              # kv = x Wkva^T
    dx += dkv @ Wf["kv_a_proj_with_mqa"]
    dq = np.concatenate([dQ[:, :, :n], rope_backward(dQ[:, :, n:], pos, theta, style)], axis=2)
    dq = dq.reshape(S, H * (n + r))
    if dims.q_lora_rank > 0:
        dW["q_b_proj"] = dq.T @ qn                    # q = qn Wqb^T
        dqn = dq @ Wf["q_b_proj"]
        dqa, dW["q_a_layernorm"] = rms_norm_backward(qa, Wf["q_a_layernorm"], eps, dqn)
        dW["q_a_proj"] = dqa.T @ x                    # qa = x Wqa^T
        dx += dqa @ Wf["q_a_proj"]
    else:
        dW["q_proj"] = dq.T @ x
        dx += dq @ Wf["q_proj"]
    return dx, dW, out


def backward(dims, W, x, q_lens, mask_kind: int, dout, window: int = 0, row_lo=None, row_hi=None,
             softmax_scale: Optional[float] = None, seqs=None):
    """A batch of training sequences packed along the token axis: dx for the
    evaluated sequences' rows and the weight gradients summed over them
    (weights are shared by every token). seqs: the sequences to evaluate
    (default all). Returns (dx rows {seq: [S_b, hidden]}, dW, out rows)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(q_lens)])
    dxs, outs, dW = {}, {}, {}
    for b in (range(len(q_lens)) if seqs is None else seqs):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        lo = hi = None
        if row_lo is not None:
            lo, hi = np.asarray(row_lo)[s0:s1], np.asarray(row_hi)[s0:s1]
        dx, dWb, out = backward_sequence(dims, W, np.asarray(x)[s0:s1], mask_kind, np.asarray(dout)[s0:s1],
                                         window, lo, hi, softmax_scale)
        dxs[b], outs[b] = dx, out
        for k, v in dWb.items():
            dW[k] = dW[k] + v if k in dW else v
    return dxs, dW, outs
