#!/usr/bin/env python3
"""MLA forward benchmark on one MI355X.

Default (the headline line): the two configurations the metric is quoted on,
each through the library's C ABI on synthetic seeded inputs already resident
in HBM when the timed region starts:
  * value: expanded prefill bf16 -- 4 x 4096 causal tokens, hidden 4096, 32
    heads, q_lora_rank 1536, kv_lora_rank 512, qk_nope 128, qk_rope 64, v_head
    128, NeoX RoPE (mla_prefill_expanded), in TFLOP/s of algorithmic work;
  * "decode": DeepSeek-V3-shaped absorbed decode bf16 -- 64 sequences x 1
    query, cache length uniform in [1024, 8192], hidden 7168, 128 heads
    (mla_decode_absorbed), in latent-cache GB/s.
One step = one call of the entry point = the whole hot path of that form.
Each carries the roofline of its dominant kernel (HIP events on the library's
stream, with the profiled launches queued behind a GPU spin so that no host
gap enters a stage), the measured roofline denominators (copy / read / MFMA
loop kernels of libmla_peaks.so) and the fp64 oracle timed on the host cores
on a bounded sample of the same workload. --workload NAME measures one other
workload on its own line (parity-test configurations, profiling runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "MLA decode latent-cache GB/s + prefill TFLOP/s (% of MI355X roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}

DESCR = {
    "tiny_f32": "tiny MLA fp32: 1 x 16 causal tokens, hidden 256, 4 heads, no q_lora, kv_lora 32, "
                "nope 16, rope 8, v 16, NeoX RoPE",
    "draft_block_bf16": "draft-block MLA bf16: 8 x 16-token fully visible block over a 2048-entry latent "
                        "prefix, hidden 4096, 32 heads, q_lora 1536, kv_lora 512, nope 128, rope 64, v 128, "
                        "interleaved RoPE",
    "decode_bf16": "DeepSeek-V3-shaped absorbed decode bf16: 64 sequences x 1 query, cache length "
                   "uniform in [1024, 8192], hidden 7168, 128 heads, q_lora 1536, kv_lora 512, nope 128, "
                   "rope 64, v 128",
    "prefill_bf16": "expanded prefill bf16: 4 x 4096 causal tokens, hidden 4096, 32 heads, q_lora 1536, "
                    "kv_lora 512, nope 128, rope 64, v 128, NeoX RoPE",
    "long_decode_bf16": "long-context decode bf16: 16 sequences, cache length uniform in [16384, 32768], "
                        "1024-token sliding window, sigmoid output gate, 128 heads, kv_lora 512, nope 128, "
                        "rope 64, v 128, hidden 7168, no q_lora",
    "draft_block_absorbed_bf16": "the draft-block workload (8 x 16-token fully visible block over a 2048-entry "
                                 "latent prefix, hidden 4096, 32 heads, q_lora 1536) through the absorbed "
                                 "query-block entry point (no latent expansion)",
}
DESCR["sparse_decode_bf16"] = ("the decode workload (64 sequences, cache length uniform in [1024, 8192], 128 heads, "
                               "q_lora 1536) through mla_decode_absorbed_sparse: each query attends 2048 listed "
                               "positions (distinct, uniform over its sequence; all of a shorter sequence)")
DESCR["decode_fp8"] = ("the decode workload (64 sequences, cache length uniform in [1024, 8192], 128 heads, "
                       "q_lora 1536) over an 8-bit latent cache: OCP E4M3 codes with one per-tensor scale "
                       "(2^-5), 576 bytes per entry")
DESCR["train_bf16"] = ("backward pass bf16 (mla_backward_expanded): 4 x 2048 causal training tokens at the "
                       "draft-block model dims (hidden 4096, 32 heads, q_lora 1536, kv_lora 512, nope 128, rope 64, "
                       "v 128, interleaved RoPE); dx and every weight gradient, forward recomputed in the call")
# training workloads (the backward entry point)
TRAIN = {"train_bf16"}
# workloads that run another workload's data through mla_decode_absorbed_block
BLOCK_OF = {"draft_block_absorbed_bf16": "draft_block_bf16"}
# workloads that run a decode workload through mla_decode_absorbed_sparse: (base, list length)
SPARSE_OF = {"sparse_decode_bf16": ("decode_bf16", 2048)}
# workloads that store another workload's cache as 8-bit codes: (base, scale)
FP8_OF = {"decode_fp8": ("decode_bf16", 2.0 ** -5)}


def listed_keys(w, topk):
    """Keys each sequence's query attends under its list (entries in [0, L))."""
    L = np.asarray(w.kv_lens, dtype=np.int64)[:, None]
    t = np.asarray(topk, dtype=np.int64)
    return ((t >= 0) & (t < L)).sum(axis=1)


# ----------------------------------------------------------------------------
# algorithmic work (from shapes only)
# ----------------------------------------------------------------------------

def visible_counts(w):
    """Visible keys of every query (same rule as the library's masks)."""
    counts = []
    for b in range(w.batch):
        P, S = int(w.prefix_lens[b]), int(w.q_lens[b])
        L = P + S
        for i in range(S):
            p = P + i
            if w.row_lo is not None:
                t = int(w.cu_seqlens[b]) + i
                lo, hi = max(0, min(int(w.row_lo[t]), L)), max(0, min(int(w.row_hi[t]), L))
            elif w.mask_kind == 0:
                lo, hi = 0, L
            elif w.mask_kind == 1:
                lo, hi = 0, min(p + 1, L)
            else:
                lo, hi = max(0, p - w.window + 1), min(p + 1, L)
            counts.append(max(0, hi - lo))
    return np.asarray(counts, dtype=np.int64)


def train_work(w, seqs=None):
    """Algorithmic flops of one backward call (forward recomputation up to
    the attention output, then the gradient): GEMMs 2 M N K each; the
    attention forward 2 H (n + r + dv) per visible (query, key) pair and its
    gradient 2 H (2 (n + r) + 2 dv) (dV, dP, dQ, dK; the recomputed scores are
    not counted)."""
    d = w.dims
    H, n, r, c, dv, hid, ql = (d.num_heads, d.qk_nope_head_dim, d.qk_rope_head_dim, d.kv_lora_rank,
                              d.v_head_dim, d.hidden_size, d.q_lora_rank)
    sel = np.arange(w.batch) if seqs is None else np.asarray(seqs)
    T = int(w.q_lens[sel].sum())
    vis = visible_counts(w)
    cu = w.cu_seqlens
    pairs = int(sum(vis[cu[b]:cu[b + 1]].sum() for b in sel))
    E = c + r
    n1 = (ql if ql else H * (n + r)) + E + (H * dv if d.use_output_gate else 0)
    f_qkv, f_qb = 2 * T * hid * n1, (2 * T * ql * H * (n + r) if ql else 0)
    f_kvb, f_o = 2 * T * c * H * (n + dv), 2 * T * H * dv * hid
    work = {"qkv_a_gemm": dict(flops=f_qkv, bytes=None), "kv_b_expand": dict(flops=f_kvb, bytes=None),
            "prefill_attn": dict(flops=2 * pairs * H * (n + r + dv), bytes=None),
            "attn_bwd": dict(flops=2 * pairs * H * (2 * (n + r) + 2 * dv), bytes=None),
            "bwd_gemm": dict(flops=f_o + f_kvb + f_qb + f_qkv, bytes=None),
            "wgrad_gemm": dict(flops=f_o + f_kvb + f_qb + f_qkv, bytes=None)}
    if ql:
        work["q_b_gemm"] = dict(flops=f_qb, bytes=None)
    work["_step"] = dict(flops=sum(v["flops"] for v in work.values()), cache_bytes=0, bytes=0)
    return work


def stage_work(w, seqs=None, absorbed=False, topk=None):
    """Algorithmic flops and bytes of each stage of one step (optionally for a
    subset of the sequences); absorbed: a prefill workload run through the
    absorbed query-block path (no expansion; latent attention); topk: the
    key lists of a sparse decode (the attention reads the listed entries)."""
    d = w.dims
    esz = 2 if d.dtype == "bf16" else 4
    H, n, r, c, dv, hid, ql = (d.num_heads, d.qk_nope_head_dim, d.qk_rope_head_dim, d.kv_lora_rank,
                              d.v_head_dim, d.hidden_size, d.q_lora_rank)
    E = c + r
    cesz = 1 if getattr(w, "kv_scale", 0.0) > 0 else esz  # bytes per cached value (8-bit cache: one)
    sel = np.arange(w.batch) if seqs is None else np.asarray(seqs)
    T = int(w.q_lens[sel].sum())
    kv = int(w.kv_lens[sel].sum())
    vis_all = visible_counts(w)
    cu = w.cu_seqlens
    pairs = int(sum(vis_all[cu[b]:cu[b + 1]].sum() for b in sel))
    if topk is not None:
        pairs = int(listed_keys(w, topk)[sel].sum())
    n1 = (ql if ql else H * (n + r)) + E + (H * dv if d.use_output_gate else 0)
    work = {}
    work["qkv_a_gemm"] = dict(flops=2 * T * hid * n1, bytes=(n1 * hid + T * (hid + n1)) * esz)
    if ql:
        work["q_b_gemm"] = dict(flops=2 * T * ql * H * (n + r), bytes=(H * (n + r) * ql + T * (ql + H * (n + r))) * esz)
    work["o_proj_gemm"] = dict(flops=2 * T * H * dv * hid, bytes=(hid * H * dv + T * (H * dv + hid)) * esz)
    if w.mode == "prefill" and not absorbed:
        work["kv_b_expand"] = dict(flops=2 * kv * c * H * (n + dv),
                                   bytes=(H * (n + dv) * c + kv * (c + H * (n + dv))) * esz)
        work["prefill_attn"] = dict(flops=2 * pairs * H * (n + r + dv), bytes=None)
        # few new tokens per sequence: the library runs both in one kernel
        # (expand_attn, the same algorithmic work) and merges its chunks
        work["expand_attn"] = dict(flops=work["kv_b_expand"]["flops"] + work["prefill_attn"]["flops"],
                                   bytes=None, fused_of=("kv_b_expand", "prefill_attn"))
    else:
        work["wuk_absorb"] = dict(flops=2 * T * H * n * c, bytes=(H * n * c + T * H * (n + c)) * esz)
        # bytes: the cache entries each sequence's queries read (once per
        # sequence: every query of a block sees the same entries)
        attn_bytes = pairs * E * cesz if not absorbed else int(w.kv_lens[sel].sum()) * E * cesz
        work["decode_attn"] = dict(flops=2 * pairs * H * (E + c), bytes=attn_bytes)
        work["wuv_gemm"] = dict(flops=2 * T * H * c * dv, bytes=(H * dv * c + T * H * (c + dv)) * esz)
    parts = [v for k, v in work.items() if k != "expand_attn"]
    work["_step"] = dict(flops=sum(v["flops"] for v in parts),
                         cache_bytes=pairs * E * cesz,
                         bytes=sum((v["bytes"] or 0) for v in parts))
    return work


def step_value(w, work):
    """(value per step, unit): TFLOP for prefill, latent-cache GB for decode."""
    if w.mode == "prefill":
        return work["_step"]["flops"] / 1e12, "TFLOP/s"
    return work["_step"]["cache_bytes"] / 1e9, "GB/s"


# ----------------------------------------------------------------------------
# measured HBM traffic (committed rocprofv3 counter summaries)
# ----------------------------------------------------------------------------

def kernel_source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "draft_models_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_GEMM_SRC = ["gemm.hip", "gemm_big.hip", "gemm.h", "kernels.h", "common.h"]
STAGE_SOURCES = {
    "kv_b_expand": _GEMM_SRC, "qkv_a_gemm": _GEMM_SRC, "q_b_gemm": _GEMM_SRC, "o_proj_gemm": _GEMM_SRC,
    "wuk_absorb": _GEMM_SRC, "wuv_gemm": _GEMM_SRC,
    "prefill_attn": ["attn_prefill.hip", "kernels.h", "common.h"],
    "decode_attn": ["attn_decode_sk.hip", "attn_decode.hip", "kernels.h", "common.h"],
    "decode_merge": ["attn_decode_sk.hip", "attn_decode.hip", "kernels.h", "common.h"],
    "rope_cache": ["rope_cache.hip", "kernels.h", "common.h"],
    "expand_attn": ["attn_mha_fused.hip", "kernels.h", "common.h"],
    "expand_merge": ["attn_mha_fused.hip", "kernels.h", "common.h"],
    "kv_dequant": ["mla_api.hip", "kernels.h", "common.h"],
    "attn_bwd": ["train.hip", "kernels.h", "common.h"],
}
# kernel that carries a stage (the one whose counters are summarised); a
# stage whose kernel name also runs other stages of the workload (a GEMM
# shared with other projections) is only summarised when all its dispatches
# have one grid size
STAGE_KERNEL = {
    "decode_attn": "decode_sk_kernel", "decode_merge": "decode_sk_merge_kernel",
    "prefill_attn": "prefill_attn_bf16_kernel", "kv_b_expand": "gemm_big_kernel",
    "rope_cache": "rope_cache", "expand_attn": "mha_fused_kernel", "expand_merge": "mha_fused_merge_kernel",
    "kv_dequant": "kv_shadow_kernel",
    # a stage of two kernels (the dQ pattern names both dQ kernels): its traffic is
    # the sum of both per-dispatch averages
    "attn_bwd": ("attn_bwd_dkdv_bf16_kernel", "attn_bwd_dq_"),
}
COPY_KERNEL = "neg_kernel"  # torch's elementwise negation kernel of the copy calibration (not the flush fill)


def _pmc_rows(d):
    rows = []
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                import csv
                rows += list(csv.DictReader(open(os.path.join(root, f))))
    return rows


def _per_dispatch(rows, counter, pat):
    """{dispatch id: (grid size, counter value summed over its rows)} of kernels matching pat"""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter or pat not in r["Kernel_Name"]:
            continue
        k = r["Dispatch_Id"]
        g, v = out.get(k, (int(r["Grid_Size"]), 0.0))
        out[k] = (g, v + float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_dir, write_dir, workload, copy_mib, commands, out_dir=None):
    """profiles/traffic_<stage>_<workload>.json from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE: KiB per dispatch), each counter scaled by what
    it reads for the copy calibration (copy_mib MiB read and written by each
    of several negation dispatches, each after a 512 MiB eviction write): the
    factor is the mean over those dispatches, its spread is recorded."""
    known_kib = copy_mib * 1024.0
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d)
        cp = _per_dispatch(rows, counter, COPY_KERNEL)
        if not cp:
            raise SystemExit(f"no copy-calibration dispatches in {d}")
        gmax = max(g for g, _ in cp.values())
        fac = [known_kib / v for g, v in cp.values() if g == gmax and v > 0]
        res[counter] = (rows, sum(fac) / len(fac), (min(fac), max(fac)), len(fac))
    written = []
    for stage, pats in STAGE_KERNEL.items():
        pats = (pats,) if isinstance(pats, str) else pats
        per = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            rows, factor, spread, ncal = res[counter]
            tot, nd = 0.0, None
            for pat in pats:
                disp = _per_dispatch(rows, counter, pat)
                if not disp or len({g for g, _ in disp.values()}) != 1:
                    nd = None
                    break
                tot += sum(v for _, v in disp.values()) / len(disp)
                nd = len(disp)
            if nd is None:
                per = None
                break
            per[counter] = (tot, factor, nd, spread, ncal)
        if not per:
            continue
        fk, ff, n, fs, fn = per["FETCH_SIZE"]
        wk, wf, _, ws, wn = per["WRITE_SIZE"]
        rec = {"stage": stage, "workload": workload, "kernel": " + ".join(pats), "dispatches": n,
               "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
               "copy_calibration_mib": copy_mib, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
               "fetch_factor_spread": [round(fs[0], 4), round(fs[1], 4)],
               "write_factor_spread": [round(ws[0], 4), round(ws[1], 4)],
               "calibration_dispatches": [fn, wn],
               "bytes_per_launch": int((fk * ff + wk * wf) * 1024),
               "source_sha": kernel_source_sha(STAGE_SOURCES[stage]), "commands": commands}
        path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"traffic_{stage}_{workload}.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        written.append(path)
    return written


def trace_summary(stats_csv, workload, command, bench_line, out_dir=None):
    """profiles/<stage>_<workload>.md: the rocprofv3 --kernel-trace --stats
    table of a bench.py run, with the bench line of the same run and the
    hash of the kernel sources it was taken on."""
    import csv
    # torch's spin kernel is the measuring harness's own (it holds the GPU while
    # the profiled pass's launches are queued), not part of the workload
    rows = [r for r in csv.DictReader(open(stats_csv)) if "spin_kernel" not in r["Name"]]
    line = json.loads(bench_line)
    rf = line.get("roofline") or {}
    stage = rf.get("kernel", "step")
    srcs = sorted({f for v in STAGE_SOURCES.values() for f in v})
    out = [f"# {stage} on the {workload} workload", "",
           f"Kernel sources (sha256 of {', '.join(srcs)}, first 16 hex): `{kernel_source_sha(srcs)}`;"
           f" dominant-stage sources: `{kernel_source_sha(STAGE_SOURCES.get(stage, srcs))}`.", "",
           "Command (`<repo>` is the repository root, `<out>` any output directory):", "",
           f"    {command}", "", f"Workload: {DESCR.get(workload, workload)}.", "",
           "## rocprofv3 kernel statistics (all calls, including warmup and context setup; the",
           "harness's GPU spin before the profiled pass left out)", "",
           "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows[:12]:
        name = r["Name"][:90]
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    out += ["", "## bench.py line of the same run (stage times from HIP events on the library's stream)", "",
            f"- value: {line['value']} {line['unit']}, ms_per_step {line['ms_per_step']}"]
    if rf:
        out.append(f"- dominant stage `{stage}`: {rf['kernel_ms']} ms per launch, {rf['achieved']} {rf['unit']} = "
                   f"{100 * rf['frac']:.1f}% of {rf['peak']} ({rf['bound']} bound)")
    out.append("- stage ms per launch: " + ", ".join(f"{k} {v}" for k, v in line.get("stages_ms", {}).items()))
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"{stage}_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    return path


MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16"]
SIMD_NUM = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCD_NUM = 8         # the per-dispatch GRBM_GUI_ACTIVE value is the sum over the 8 XCDs


def _kernel_short(name):
    """mla::gemm_big_kernel from a demangled name (mangled names stay as they are)"""
    return name.replace("(anonymous namespace)::", "").split("(")[0].strip()


def mfma_summary(pmc_dir, workload, command, out_dir=None):
    """profiles/mfma_<workload>.json from one rocprofv3 --pmc run of MFMA_COUNTERS:
    per (kernel, grid size): MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES /
    (GRBM_GUI_ACTIVE / XCD_NUM * SIMD_NUM) (rocprofv3's MfmaUtil, which takes
    the largest per-XCD GUI-active count), and the bf16 MFMA flops the
    counters saw (SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512) per dispatch."""
    rows = _pmc_rows(pmc_dir)
    disp = {}
    for r in rows:
        if r["Counter_Name"] not in MFMA_COUNTERS:
            continue
        k = r["Dispatch_Id"]
        rec = disp.setdefault(k, {"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size"]), "ns": None})
        rec[r["Counter_Name"]] = rec.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("End_Timestamp") and r.get("Start_Timestamp"):
            rec["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    groups = {}
    for rec in disp.values():
        if not all(c in rec for c in MFMA_COUNTERS) or rec["GRBM_GUI_ACTIVE"] <= 0:
            continue
        name = _kernel_short(rec["kernel"])
        groups.setdefault((name, rec["grid"]), []).append(rec)
    out = []
    for (name, grid), recs in sorted(groups.items(), key=lambda kv: -sum(x["GRBM_GUI_ACTIVE"] for x in kv[1])):
        busy = sum(x["SQ_VALU_MFMA_BUSY_CYCLES"] / (x["GRBM_GUI_ACTIVE"] / XCD_NUM * SIMD_NUM) for x in recs) / len(recs)
        flops = sum(x["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for x in recs) / len(recs)
        if flops <= 0:
            continue
        ent = {"kernel": name, "grid": grid, "dispatches": len(recs), "mfma_busy_pct": round(100 * busy, 2),
               "bf16_mfma_gflop_per_dispatch": round(flops / 1e9, 3)}
        ns = [x["ns"] for x in recs if x["ns"]]
        if ns:
            ent["avg_dispatch_us_under_counters"] = round(sum(ns) / len(ns) / 1e3, 2)
            ent["mfma_tflops_under_counters"] = round(flops / (sum(ns) / len(ns)) / 1e3, 1)
        out.append(ent)
    srcs = sorted({f for v in STAGE_SOURCES.values() for f in v})
    rec = {"workload": workload, "counters": MFMA_COUNTERS, "simd_num": SIMD_NUM, "xcd_num": XCD_NUM, "kernels": out,
           "source_sha": kernel_source_sha(srcs), "command": command}
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"mfma_{workload}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return path


def measured_traffic(stage, workload):
    """HBM bytes per launch from profiles/traffic_<stage>_<workload>.json, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != kernel_source_sha(STAGE_SOURCES[stage]):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ----------------------------------------------------------------------------

def cpu_baseline(w, budget_s: float, absorbed: bool = False, topk=None):
    from threadpoolctl import threadpool_info
    from oracle import mla as om
    order = list(np.argsort(w.kv_lens))  # shortest first keeps the sample bounded
    done, t0 = [], time.perf_counter()
    first = {}
    for b in order:
        b = int(b)
        if w.mode == "decode" and w.mask_kind == 2:
            # only the visible window of a sliding-window decode enters the computation
            first[b] = max(0, int(w.kv_lens[b]) - w.window)
        pre = w.prefix_rows[b][first.get(b, 0):]
        cu = w.cu_seqlens
        if getattr(w, "_train_dout", None) is not None:
            # the oracle's analytic gradient of the sequence
            from oracle import backward as ob
            ob.backward_sequence(w.dims, w.weights, w.x[cu[b]:cu[b + 1]], w.mask_kind, w._train_dout[cu[b]:cu[b + 1]],
                                 w.window)
        elif topk is not None:
            # the oracle's absorbed form over the listed entries (pinned equal
            # to its expanded form, which expands every entry of the sequence)
            om.forward_sequence(w.dims, w.weights, w.x[cu[b]:cu[b + 1]], pre, w.mask_kind, w.window,
                                form="absorbed", key_lists=[topk[b]])
        else:
            om.forward_sequence(w.dims, w.weights, w.x[cu[b]:cu[b + 1]], pre, w.mask_kind, w.window,
                                first_position=first.get(b, 0), kv_scale=w.kv_scale if w.kv_scale > 0 else None)
        done.append(b)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    train = getattr(w, "_train_dout", None) is not None
    work = train_work(w, seqs=done) if train else stage_work(w, seqs=done, absorbed=absorbed, topk=topk)
    per, unit = step_value(w, work)
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas"})
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": per / el, "unit": unit, "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "blas": ", ".join(blas),
            "sample": f"{len(done)} of {w.batch} sequences (ids {sorted(done)}), "
                      f"{'gradient' if train else ('absorbed' if topk is not None else 'expanded')} fp64 oracle, "
                      f"{el:.1f} s wall", "wall_s": round(el, 3)}


# ----------------------------------------------------------------------------

# ----------------------------------------------------------------------------
# measured roofline denominators (libmla_peaks.so)
# ----------------------------------------------------------------------------

def measured_peaks(torch):
    """HBM copy and read bandwidth over 2 GiB buffers (8x the Infinity Cache)
    and the bf16 MFMA issue rate of a register-only MFMA loop, each the best
    of three timed launches (HIP events on the current stream)."""
    import ctypes as C
    path = os.path.join(ROOT, "draft_models_amd", "libmla_peaks.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with __graft_entry__.build()")
    lib = C.CDLL(path)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    lib.peaks_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.peaks_read.argtypes = [vp, i64, i32, vp, vp]
    lib.peaks_mfma.argtypes = [i32, i32, i32, vp, vp]
    st = torch.cuda.current_stream().cuda_stream
    nbytes = 2 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    blocks = 256 * 16
    red = torch.empty(blocks, dtype=torch.int32, device="cuda")

    def best(fn, n=3):
        t = []
        for _ in range(n + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if fn() != 0:
                raise RuntimeError("peaks kernel launch failed")
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t[1:])  # the first launch loads the code object
    copy_ms = best(lambda: lib.peaks_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, st))
    read_ms = best(lambda: lib.peaks_read(src.data_ptr(), nbytes, blocks, red.data_ptr(), st))
    del src, dst, red
    res = {"hbm_copy_gbs": round(2 * nbytes / (copy_ms / 1e3) / 1e9, 1),
           "hbm_read_gbs": round(nbytes / (read_ms / 1e3) / 1e9, 1), "buffer_gib": nbytes >> 30}
    mblocks, iters = 256 * 8, 4000
    out = torch.empty(mblocks * 256, dtype=torch.float32, device="cuda")
    for shape, flops in ((32, 32768), (16, 16384)):
        ms = best(lambda: lib.peaks_mfma(shape, iters, mblocks, out.data_ptr(), st))
        res[f"mfma_bf16_{shape}x{shape}x{512 // shape}_tflops"] = round(
            mblocks * 4 * 4 * iters * flops / (ms / 1e3) / 1e12, 1)
    del out
    res["mfma_bf16_tflops"] = max(v for k, v in res.items() if k.startswith("mfma_bf16_") and k.endswith("tflops"))
    return res


# ----------------------------------------------------------------------------
# one workload
# ----------------------------------------------------------------------------

def measure(name, args, torch, peaks=None):
    """Time one workload through its entry point; returns its JSON object."""
    import mla_synth as ms
    from mla_synth.device import upload
    from draft_models_amd import binding as B

    block = name in BLOCK_OF
    sparse = name in SPARSE_OF
    train = name in TRAIN
    base = BLOCK_OF.get(name, SPARSE_OF.get(name, FP8_OF.get(name, (name,)))[0])
    w = ms.make_workload(base, kv_scale=FP8_OF[name][1] if name in FP8_OF else 0.0)
    t = upload(w)
    w._train_dout = ms.draw_dout(w, ms.TRAIN_DOUT_SEED) if train else None
    topk = lists = None
    if sparse:
        topk = ms.draw_topk(w, SPARSE_OF[name][1], ms.SPARSE_TOPK_SEED)
        lists = torch.from_numpy(topk).cuda()
    d = w.dims
    max_kv = int(w.kv_lens.max())
    prefill = w.mode == "prefill"
    max_q = int(w.q_lens.max())
    lp = -(-max_q // d.page_size) * d.page_size
    cfg = B.make_config(d, max_batch=w.batch, max_tokens=w.total_tokens, max_seq_len=max_kv,
                        max_prefill_kv=(w.batch * (lp if train else max_kv)) if prefill and not block else 0,
                        max_block_tokens=w.total_tokens if block else 0,
                        max_topk=0 if topk is None else topk.shape[1], kv_scale=w.kv_scale,
                        max_train_tokens=w.total_tokens if train else 0)
    m = B.MLA(cfg, t["weights"])
    dt = torch.bfloat16 if d.dtype == "bf16" else torch.float32
    out = torch.empty((w.total_tokens, d.hidden_size), dtype=dt, device="cuda")
    if train:
        from mla_synth.device import to_torch
        dout_t = to_torch(w._train_dout, d.dtype, "cuda")
        grads = {k: torch.empty_like(v) for k, v in t["weights"].items()}

    def step():
        if train:
            m.backward(t["x"], t["cu_seqlens"], max_q, w.mask_kind, w.window, dout_t, out, grads)
        elif block:
            m.decode_block(t["x"], max_q, t["cache"], t["block_table"], t["prefix_lens"], max_kv, out)
        elif prefill:
            m.prefill(t["x"], t["cu_seqlens"], t["prefix_lens"], max_q, max_kv, t["cache"], t["block_table"],
                      w.mask_kind, w.window, out)
        elif sparse:
            m.decode_sparse(t["x"], t["cache"], t["block_table"], t["seq_lens"], max_kv, lists, out)
        else:
            m.decode(t["x"], t["cache"], t["block_table"], t["seq_lens"], max_kv, w.mask_kind, w.window, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K steps back to back, no per-stage events
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # decode: calls timed one by one, each after a 512 MiB write that evicts
    # the Infinity Cache (the back-to-back figure above is the headline)
    flushed = None
    if w.mode == "decode" and args.flushed_steps > 0:
        scratch = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(args.flushed_steps):
            scratch.fill_(1.0)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        flushed = {"ms_per_step_median": round(float(np.median(times)), 5), "steps": len(times), "flush_mib": 512}
    # per-stage times: a separate pass of the same steps with the library's
    # stage events (HIP events recorded on the call's stream around each
    # stage's launches). The steps are queued behind a GPU spin of about
    # 0.1 s so that every launch is in the queue before the GPU reaches it:
    # a stage's events then bracket its kernels with no host gap.
    stages = {}
    if not args.no_profile:
        m.profile(True)
        m.profile_read()  # clear
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(200_000_000)
        for _ in range(max(3, min(args.steps, 10))):
            step()
        stages = m.profile_read()
        m.profile(False)

    work = train_work(w) if train else stage_work(w, absorbed=block, topk=topk)
    per_step, unit = step_value(w, work)
    value = per_step / (ms_step / 1e3)

    # dominant kernel: the stage with the largest total time
    timed = {k: v for k, v in stages.items() if v[1] > 0}
    roofline = None
    if timed:
        dom = max(timed, key=lambda k: timed[k][0])
        dom_ms = timed[dom][0] / timed[dom][1]
        wk = work.get(dom, {})
        # latent attention of query blocks reads each entry once for 16 queries
        # (about 970 flop per byte): matrix-core bound
        hbm = dom in ("rope_cache", "decode_merge") or (dom == "decode_attn" and not block) or \
            (w.mode == "decode" and wk.get("bytes"))
        if hbm:
            bound, peak, unit_r = "hbm", HBM_PEAK_GBS, "GB/s"
            achieved = (wk.get("bytes") or 0) / (dom_ms / 1e3) / 1e9
            mpeak = (peaks or {}).get("hbm_read_gbs")
        else:
            bound, peak, unit_r = "mfma", MFMA_PEAK_TFLOPS[d.dtype], "TFLOP/s"
            achieved = wk.get("flops", 0) / (dom_ms / 1e3) / 1e12
            mpeak = (peaks or {}).get("mfma_bf16_tflops") if d.dtype == "bf16" else None
        roofline = {"bound": bound, "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                    "unit": unit_r, "frac": round(achieved / peak, 4),
                    "traffic": measured_traffic(dom, name), "kernel_ms": round(dom_ms, 5),
                    "algorithmic": (wk.get("bytes") if hbm else wk.get("flops"))}
        if mpeak:
            roofline["measured_peak"] = mpeak
            roofline["frac_of_measured"] = round(achieved / mpeak, 4)

    res = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": d.dtype, "data": "synthetic (seeded, random-init weights)",
        "config": {"workload": name, "description": DESCR[name], "batch": w.batch,
                   "new_tokens": w.total_tokens, "max_kv_len": max_kv, "entry_point":
                       "mla_backward_expanded" if train else
                       ("mla_decode_absorbed_block" if block else ("mla_decode_absorbed_sparse" if sparse else
                        ("mla_prefill_expanded" if prefill else "mla_decode_absorbed"))),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages_ms": {k: round(v[0] / max(v[1], 1), 5) for k, v in timed.items()},
        "step_work": {"tflop": round(work["_step"]["flops"] / 1e12, 4),
                      "latent_cache_gb": round(work["_step"]["cache_bytes"] / 1e9, 4)},
    }
    if not prefill:
        res["whole_call_gbps"] = round(work["_step"]["bytes"] / (ms_step / 1e3) / 1e9, 2)
    if flushed is not None:
        flushed["value"] = round(per_step / (flushed["ms_per_step_median"] / 1e3), 3)
        flushed["unit"] = unit
        res["mall_flushed"] = flushed
    m.close()
    if train:
        del grads, dout_t
    del t, out, lists
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res["_w"] = (w, block, topk)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(DESCR),
                    help="measure this one workload (default: the prefill and decode headline pair)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget per workload (0 = skip)")
    ap.add_argument("--no-profile", action="store_true", help="skip the profiled pass (no roofline)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak kernels")
    ap.add_argument("--flushed-steps", type=int, default=10,
                    help="decode workloads: calls timed one by one after writing 512 MiB (evicts the 256 MB "
                         "Infinity Cache); reported as mall_flushed, 0 = skip")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="first run a plain elementwise copy of MIB MiB five times, each after a 512 MiB "
                         "eviction write (HBM counter calibration)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_*.json from two rocprofv3 --pmc runs of --workload "
                         "(FETCH_SIZE, WRITE_SIZE) made with --copy-calibrate; no GPU work")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write profiles/mfma_<workload>.json from one rocprofv3 --pmc run of --workload "
                         "with the MFMA counters; no GPU work")
    ap.add_argument("--out-dir", default=None, help="directory of the summary files (default: profiles/)")
    ap.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write profiles/<stage>_<workload>.md from the kernel_stats.csv of a rocprofv3 "
                         "--kernel-trace --stats run of --workload and that run's bench line; no GPU work")
    args = ap.parse_args()
    if args.mfma_summary or args.traffic_summary or args.trace_summary:
        if not args.workload:
            raise SystemExit("the summary modes need --workload")
    if args.mfma_summary:
        cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) +
               f" --output-format csv -d <out> -o run -- python3 <repo>/bench.py --workload {args.workload} "
               f"--steps {args.steps} --warmup {args.warmup} --cpu-seconds 0 --no-peaks")
        print("wrote", mfma_summary(args.mfma_summary, args.workload, cmd, args.out_dir))
        return
    if args.traffic_summary:
        cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- "
               f"python3 <repo>/bench.py --workload {args.workload} --steps {args.steps} --warmup {args.warmup} "
               f"--cpu-seconds 0 --no-peaks --copy-calibrate {args.copy_calibrate}")
        for p in traffic_summary(*args.traffic_summary, args.workload, args.copy_calibrate,
                                 [cmd.format(c="FETCH_SIZE"), cmd.format(c="WRITE_SIZE")], args.out_dir):
            print("wrote", p)
        return
    if args.trace_summary:
        cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <out> "
               f"-o run -- python3 <repo>/bench.py --workload {args.workload} --steps {args.steps} "
               f"--warmup {args.warmup} --cpu-seconds 0 --no-peaks")
        line = next(ln for ln in open(args.trace_summary[1]) if ln.startswith("{"))
        print("wrote", trace_summary(args.trace_summary[0], args.workload, cmd, line, args.out_dir))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(each GPU would run its own sequences with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibrate > 0:
        # a plain elementwise kernel of known traffic (reads and writes
        # copy_calibrate MiB), each launch after a 512 MiB write that evicts
        # the Infinity Cache
        n = args.copy_calibrate * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        evict = torch.empty((512 << 20) // 4, dtype=torch.float32, device="cuda")
        for _ in range(5):
            evict.fill_(2.0)
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst, evict

    peaks = None if args.no_peaks else measured_peaks(torch)
    names = [args.workload] if args.workload else ["prefill_bf16", "decode_bf16"]
    results = [measure(nm, args, torch, peaks) for nm in names]
    for r in results:
        w, block, topk = r.pop("_w")
        if args.cpu_seconds > 0:
            r["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, absorbed=block, topk=topk)
        else:
            r["cpu_baseline"] = None
    line = results[0]
    if len(results) > 1:
        dec = results[1]
        for k in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "data"):
            dec.pop(k, None)
        line["decode"] = dec
        line["config"]["headline"] = ("value: prefill TFLOP/s (mla_prefill_expanded); decode: latent-cache GB/s "
                                      "(mla_decode_absorbed)")
    if peaks is not None:
        line["measured_peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
