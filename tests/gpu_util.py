"""Helpers of the GPU parity tests: run a workload through the C ABI and
compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mla_synth as ms
from mla_synth.device import from_torch, upload
from draft_models_amd import binding as B
from oracle import mla as om

TOL_BF16 = dict(max_abs=2e-2, rel_l2=5e-3)
TOL_F32 = dict(max_abs=1e-4, rel_l2=None)
# Gradients (mla_backward_expanded). The forward's bf16 bar covers one chain
# of bf16 storage points (q_c, q, cache entries, expanded K/V, probabilities,
# attention output), observed 3-4.5e-3 rel-L2. A gradient recomputes that
# forward and adds its own chain (dA, dO, P and dS of the attention backward,
# dQ / dK / dV, dcn or dqn, the first projection's gradient, the output),
# about 8 more roundings of 2^-9 / sqrt(3) relative each: sqrt(8) * 1.1e-3 =
# 3.2e-3 in quadrature with the forward's 4e-3 gives 5.1e-3; the bar is twice
# the forward's. Max error relative to the tensor's scale (max(1, max |ref|)):
# a weight gradient sums over every token, so an element that cancels to a
# small value keeps the absolute error of its large terms.
TOL_BF16_GRAD = dict(max_abs=2e-2, rel_l2=1e-2)
TOL_F32_GRAD = dict(max_abs=1e-4, rel_l2=None)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w: ms.Workload, *, softmax_scale: float = 0.0, extra_capacity: bool = False, block: bool = False,
            topk=None):
    """One call of the workload's entry point (block: a prefill workload of
    equal block lengths under the FULL mask through mla_decode_absorbed_block;
    topk: [batch, k] int32 key lists of a decode workload through
    mla_decode_absorbed_sparse). Returns (out [T, hidden], cache
    [num_blocks, page, E]) as float32 numpy."""
    say(f"[gpu] {w.name} mode={w.mode} B={w.batch} T={w.total_tokens} "
        f"max_kv={int(w.kv_lens.max())} mask={w.mask_kind} window={w.window} seed={w.seed} "
        f"kv_scale={w.kv_scale}")
    t = upload(w)
    d = w.dims
    max_kv = int(w.kv_lens.max())
    prefill = w.mode == "prefill"
    if block:
        assert prefill and w.mask_kind == ms.MASK_FULL and len(set(int(q) for q in w.q_lens)) == 1
    cfg = B.make_config(d, max_batch=w.batch + (3 if extra_capacity else 0),
                        max_tokens=w.total_tokens + (5 if extra_capacity else 0),
                        max_seq_len=max_kv + (7 if extra_capacity else 0),
                        max_prefill_kv=w.batch * max_kv if prefill and not block else 0,
                        softmax_scale=softmax_scale, max_block_tokens=w.total_tokens if block else 0,
                        max_topk=0 if topk is None else topk.shape[1] + (9 if extra_capacity else 0),
                        kv_scale=w.kv_scale)
    m = B.MLA(cfg, t["weights"])
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    out = torch.full((w.total_tokens, d.hidden_size), float("nan"), dtype=dt, device="cuda")
    if topk is not None:
        assert not prefill
        say(f"  sparse lists: {topk.shape[1]} per sequence")
        lists = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda()
        m.decode_sparse(t["x"], t["cache"], t["block_table"], t["seq_lens"], max_kv, lists, out)
    elif block:
        m.decode_block(t["x"], int(w.q_lens[0]), t["cache"], t["block_table"], t["prefix_lens"], max_kv, out)
    elif prefill:
        m.prefill(t["x"], t["cu_seqlens"], t["prefix_lens"], int(w.q_lens.max()), max_kv, t["cache"],
                  t["block_table"], w.mask_kind, w.window, out, row_lo=t.get("row_lo"), row_hi=t.get("row_hi"))
    else:
        m.decode(t["x"], t["cache"], t["block_table"], t["seq_lens"], max_kv, w.mask_kind, w.window, out)
    torch.cuda.synchronize()
    m.close()
    cache = t["cache"].cpu().numpy() if w.kv_scale > 0 else from_torch(t["cache"])
    return from_torch(out), cache


def oracle(w: ms.Workload, seqs=None, rows_per_seq=None, form="expanded", first_positions=None,
           softmax_scale=None, topk=None):
    """topk: [batch, k] key lists of a decode workload (one query per sequence)."""
    key_lists = None
    if topk is not None:
        key_lists = {b: [topk[b]] for b in (range(w.batch) if seqs is None else seqs)}
    return om.mla_forward(w.dims, w.weights, w.x, w.q_lens, w.prefix_rows, w.mask_kind, w.window,
                          w.row_lo, w.row_hi, form=form, seqs=seqs, rows_per_seq=rows_per_seq,
                          softmax_scale=softmax_scale, first_positions=first_positions, key_lists=key_lists,
                          kv_scale=w.kv_scale if w.kv_scale > 0 else None,
                          model_bf16=w.kv_scale > 0 and w.dims.dtype == "bf16")


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str, magnitude_scaled: bool = False, tol=None,
                 tensor_scaled: bool = False):
    """max |got - ref| <= max_abs and ||got - ref|| / ||ref|| <= rel_l2.

    magnitude_scaled: the max-abs bar is applied to |got - ref| / max(1, |ref|).
    Used for stored cache entries: a bf16 value is only representable to within
    2^-9 |v| (0.0156 at |v| = 8, above 2e-2 beyond), and the unnormalised rope
    key reaches |v| of about 8, so an absolute bar cannot hold for any bf16
    storage of it; the relative L2 bar is unchanged."""
    tol = tol or (TOL_BF16 if dtype == "bf16" else TOL_F32)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    max_abs, rel = errors(got, ref)
    worst = max_abs
    if tensor_scaled and got.size:
        worst = max_abs / max(1.0, float(np.max(np.abs(np.asarray(ref, np.float64)))))
    elif magnitude_scaled and got.size:
        d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        worst = float(np.max(d / np.maximum(1.0, np.abs(np.asarray(ref, np.float64)))))
    say(f"  {what}: max_abs={max_abs:.3e} scaled_max={worst:.3e} rel_l2={rel:.3e}")
    assert worst <= tol["max_abs"], f"{what}: max error {worst} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: relative L2 error {rel} > {tol['rel_l2']}"


# 8-bit cache codes: differing codes allowed per 10 000 (at least three)
CODE_DIFF_PER = 10000
CODE_DIFF_MIN = 3
# a differing code must be the neighbour across an E4M3 midpoint that lies
# within this relative distance of the oracle's value (two bf16 steps)
CODE_TIE_RADIUS = 2.0 ** -6


def tie_radius(entries, dims):
    """Per value of the oracle's bf16 entries [S, E], the size that a bf16
    rounding of its inputs can move it by, up to CODE_TIE_RADIUS: |value|
    for the latent, and for a rope value the norm of its rotated pair (a
    rotation mixes the two inputs, so a change of either moves the result by
    a step of the pair's size)."""
    e = np.asarray(entries, np.float64)
    c, r = dims.kv_lora_rank, dims.qk_rope_head_dim
    rho = np.abs(e).copy()
    a, b = om.rope_pairs(r, dims.rope_style)
    nrm = np.sqrt(e[:, c + a] ** 2 + e[:, c + b] ** 2)
    rho[:, c + a] = nrm
    rho[:, c + b] = nrm
    return rho


def check_codes(got, ref_unq, rho, scale: float):
    """8-bit cache entries against the oracle. ref_unq: the oracle's entries
    before encoding (the bf16 values of a bf16 model, model_bf16); rho: their
    tie_radius. The codes the oracle stores are encode(ref_unq / scale). The
    library computes the same bf16 values in fp32 from a bf16 projection
    that may sit one bf16 step off the oracle's rounding where the fp64
    projection is near a bf16 tie, so a code can legitimately differ only
    where the oracle's value lies near an E4M3 midpoint (a simulation of the
    fp32 arithmetic on the decode shapes gives about 4 per 100 000). The bar:
    at most one code per CODE_DIFF_PER differs (CODE_DIFF_MIN at least, for
    small calls), and each differing
    code is the neighbour of the oracle's across a midpoint m with
    |ref_unq - m scale| <= CODE_TIE_RADIUS rho."""
    got = np.asarray(got, np.uint8).reshape(-1)
    ref_unq = np.asarray(ref_unq, np.float64).reshape(-1)
    rho = np.asarray(rho, np.float64).reshape(-1)
    ref = np.asarray(om.fp8_e4m3_encode(ref_unq / scale), np.uint8)
    diff = got != ref
    n = int(diff.sum())
    say(f"  cache codes: {n} of {got.size} differ")
    assert n <= max(CODE_DIFF_MIN, got.size // CODE_DIFF_PER), f"{n} of {got.size} codes differ"

    def ordinal(cd):
        cd = cd.astype(np.int64)
        mag = cd & 0x7F
        return np.where(cd & 0x80, -mag, mag)
    idx = np.flatnonzero(diff)
    for i in idx:
        og, orf = int(ordinal(got[i:i + 1])[0]), int(ordinal(ref[i:i + 1])[0])
        gv = float(om.fp8_e4m3_decode(int(got[i])))
        rv = float(om.fp8_e4m3_decode(int(ref[i])))
        say(f"    code {i}: got {got[i]:#04x} ({gv * scale:.6g}) oracle {ref[i]:#04x} ({rv * scale:.6g}), "
            f"oracle value {ref_unq[i]:.8g}, radius {rho[i]:.4g}")
        assert not np.isnan(gv), f"code {i} is NaN"
        if gv == rv:  # +0 / -0
            continue
        assert abs(og - orf) == 1, f"code {i} is not the neighbour of the oracle's"
        mid = (gv + rv) / 2 * scale
        assert abs(ref_unq[i] - mid) <= CODE_TIE_RADIUS * rho[i], \
            f"code {i} differs away from a tie: |{ref_unq[i]} - {mid}| > {CODE_TIE_RADIUS} * {rho[i]}"


def check(w: ms.Workload, out, cache, res, rows_per_seq=None, out_tol=None):
    """Compare the GPU output rows and written cache entries of the sequences
    in `res` (oracle results) and check the prefix entries are untouched
    (out_tol: the output bar, default TOL_BF16 / TOL_F32)."""
    cu = w.cu_seqlens
    got_o, ref_o, got_e, ref_e = [], [], [], []
    for b, (o_ref, e_ref, _) in res.items():
        rows = np.arange(w.q_lens[b]) if rows_per_seq is None else np.asarray(rows_per_seq[b])
        got_o.append(out[cu[b] + rows])
        ref_o.append(o_ref)
        P = int(w.prefix_lens[b])
        got_e.append(ms.gather_entries(w, cache, b, P, P + int(w.q_lens[b])))
        ref_e.append(e_ref)
        if P:
            kept = ms.gather_entries(w, cache, b, 0, P)
            want = w.prefix_codes[b] if w.kv_scale > 0 else w.prefix_rows[b]
            assert np.array_equal(kept, want), f"prefix entries of sequence {b} changed"
    if w.kv_scale > 0:
        # the oracle's entries before encoding: the bf16 tensors the cache
        # update receives (new tokens depend only on x and the weights)
        unq = []
        for b in res:
            P, S = int(w.prefix_lens[b]), int(w.q_lens[b])
            unq.append(om.project_tokens(w.dims, w.weights, w.x[cu[b]:cu[b] + S], P + np.arange(S),
                                         model_bf16=True)[1])
        unq = np.concatenate(unq)
        assert np.array_equal(om.fp8_quantize(unq, w.kv_scale), np.concatenate(ref_e))
        check_codes(np.concatenate(got_e), unq, tie_radius(unq, w.dims), w.kv_scale)
    else:
        assert_close(np.concatenate(got_e), np.concatenate(ref_e), w.dims.dtype, "cache entries",
                     magnitude_scaled=True)
    assert_close(np.concatenate(got_o), np.concatenate(ref_o), w.dims.dtype, "out", tol=out_tol)


# ------------------------------------------------------------ backward pass

draw_dout = ms.draw_dout


def run_backward(w: ms.Workload, dout: np.ndarray):
    """One mla_backward_expanded call on a training workload (no prefix).
    Returns (dx [T, hidden], {weight name: dW}) as float32 numpy."""
    from mla_synth.device import to_torch
    say(f"[gpu-bwd] {w.name} B={w.batch} T={w.total_tokens} max_q={int(w.q_lens.max())} mask={w.mask_kind} "
        f"window={w.window} seed={w.seed} heads={w.dims.num_heads} dtype={w.dims.dtype}")
    assert int(w.prefix_lens.max()) == 0
    t = upload(w)
    d = w.dims
    max_q = int(w.q_lens.max())
    lp = -(-max_q // d.page_size) * d.page_size
    cfg = B.make_config(d, max_batch=w.batch, max_tokens=w.total_tokens, max_seq_len=max_q,
                        max_prefill_kv=w.batch * lp, max_train_tokens=w.total_tokens)
    m = B.MLA(cfg, t["weights"])
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    g = {k: torch.full_like(v, float("nan")) for k, v in t["weights"].items()}
    dx = torch.full((w.total_tokens, d.hidden_size), float("nan"), dtype=dt, device="cuda")
    m.backward(t["x"], t["cu_seqlens"], max_q, w.mask_kind, w.window, to_torch(dout, d.dtype, "cuda"), dx, g,
               row_lo=t.get("row_lo"), row_hi=t.get("row_hi"))
    torch.cuda.synchronize()
    m.close()
    return from_torch(dx), {k: from_torch(v) for k, v in g.items()}


def check_backward(w: ms.Workload, dout, dx, grads, seqs=None, tol=None):
    """dx rows and every weight gradient against oracle.backward (the weight
    gradients are compared only when every sequence is evaluated), to the
    gradient bars TOL_BF16_GRAD / TOL_F32_GRAD with the max error taken
    relative to each tensor's scale."""
    from oracle import backward as ob
    dxs, dW, _ = ob.backward(w.dims, w.weights, w.x, w.q_lens, w.mask_kind, dout, w.window, w.row_lo, w.row_hi,
                             seqs=seqs)
    cu = w.cu_seqlens
    got = np.concatenate([dx[cu[b]:cu[b + 1]] for b in dxs])
    ref = np.concatenate([dxs[b] for b in dxs])
    pairs = [("dx", got, ref)]
    if seqs is None:
        pairs += [(f"d{k}", grads[k], dW[k]) for k in sorted(dW)]
    failures = []
    tol = tol or (TOL_BF16_GRAD if w.dims.dtype == "bf16" else TOL_F32_GRAD)
    for what, gv, rv in pairs:  # every comparison is printed before the first failure is raised
        try:
            assert_close(gv, rv, w.dims.dtype, what, tol=tol, tensor_scaled=True)
        except AssertionError as e:
            failures.append(str(e))
    assert not failures, "; ".join(failures)
