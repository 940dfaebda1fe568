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
                          kv_round_bf16=w.kv_scale > 0 and w.dims.dtype == "bf16")


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    return max_abs, rel


def assert_close(got, ref, dtype: str, what: str, magnitude_scaled: bool = False):
    """max |got - ref| <= max_abs and ||got - ref|| / ||ref|| <= rel_l2.

    magnitude_scaled: the max-abs bar is applied to |got - ref| / max(1, |ref|).
    Used for stored cache entries: a bf16 value is only representable to within
    2^-9 |v| (0.0156 at |v| = 8, above 2e-2 beyond), and the unnormalised rope
    key reaches |v| of about 8, so an absolute bar cannot hold for any bf16
    storage of it; the relative L2 bar is unchanged."""
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    max_abs, rel = errors(got, ref)
    worst = max_abs
    if magnitude_scaled and got.size:
        d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        worst = float(np.max(d / np.maximum(1.0, np.abs(np.asarray(ref, np.float64)))))
    say(f"  {what}: max_abs={max_abs:.3e} scaled_max={worst:.3e} rel_l2={rel:.3e}")
    assert worst <= tol["max_abs"], f"{what}: max error {worst} > {tol['max_abs']}"
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], f"{what}: relative L2 error {rel} > {tol['rel_l2']}"


def check_codes(got, ref_vals, scale: float):
    """8-bit cache entries against the oracle's quantized entries (ref_vals,
    values code * scale). The GPU rounds the kv_a projection output to the
    compute dtype (bf16) before the RMSNorm and RoPE, a relative change of up
    to 2^-9 per input: a value then lands on the other side of a code boundary
    (code steps are 2^-4 to 2^-3 relative) for about 2 % of the entries, and
    the RoPE rotation, a difference of two products, can move a value near
    zero by more than one step of its own size. The bar: at most 5 % of the
    codes differ, and every stored value is within one E4M3 step of the
    oracle's, |got - ref| <= 2^-3 max(scale, |ref|) (the magnitude-scaled bar
    of the bf16 cache check with a one-code width)."""
    got = np.asarray(got, np.uint8)
    ref_vals = np.asarray(ref_vals, np.float64)
    ref = np.asarray(om.fp8_e4m3_encode(ref_vals / scale), np.uint8)
    diff = got != ref
    n = int(diff.sum())
    gv = om.fp8_e4m3_decode(got.astype(np.int64)) * scale
    err = np.abs(gv - ref_vals) / np.maximum(scale, np.abs(ref_vals))
    worst = float(err.max()) if err.size else 0.0
    say(f"  cache codes: {n} of {got.size} differ, worst scaled error {worst:.3e}")
    if n:
        idx = np.flatnonzero(diff)[:6]
        say("  first differing codes (index, got, oracle, oracle value / scale): " + ", ".join(
            f"({i}, {got.flat[i]:#04x}, {ref.flat[i]:#04x}, {ref_vals.flat[i] / scale:.5g})" for i in idx))
    assert n <= max(2, got.size // 20), f"{n} of {got.size} codes differ"
    assert worst <= 0.125, f"a stored value is more than one code step from the oracle's ({worst})"


def check(w: ms.Workload, out, cache, res, rows_per_seq=None):
    """Compare the GPU output rows and written cache entries of the sequences
    in `res` (oracle results) and check the prefix entries are untouched."""
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
        check_codes(np.concatenate(got_e), np.concatenate(ref_e), w.kv_scale)
    else:
        assert_close(np.concatenate(got_e), np.concatenate(ref_e), w.dims.dtype, "cache entries",
                     magnitude_scaled=True)
    assert_close(np.concatenate(got_o), np.concatenate(ref_o), w.dims.dtype, "out")
