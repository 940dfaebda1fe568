"""Host-side logic of bench.py (no GPU): the algorithmic work it counts, the
counter summaries it builds from rocprofv3 CSV files, and its one-GPU guard."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench
import mla_synth as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shape_only(name, q_lens, prefix_lens, mask_kind, window=0, mode="prefill"):
    """The fields stage_work reads, without drawing any tensor."""
    q = np.asarray(q_lens, dtype=np.int64)
    p = np.asarray(prefix_lens, dtype=np.int64)
    return SimpleNamespace(dims=ms.DIMS[name], batch=len(q), q_lens=q, prefix_lens=p, kv_lens=p + q,
                           cu_seqlens=np.concatenate([[0], np.cumsum(q)]), mask_kind=mask_kind,
                           window=window, row_lo=None, row_hi=None, mode=mode)


def test_draft_block_work_matches_the_closed_form():
    # 8 sequences x 16 fully visible tokens over a 2048-entry prefix
    w = _shape_only("draft_block_bf16", [16] * 8, [2048] * 8, ms.MASK_FULL)
    work = bench.stage_work(w)
    T, kv, H = 128, 8 * 2064, 32
    assert work["kv_b_expand"]["flops"] == 2 * kv * 512 * H * 256
    assert work["prefill_attn"]["flops"] == 2 * (T * 2064) * H * (128 + 64 + 128)
    proj = 2 * T * 4096 * (1536 + 576) + 2 * T * 1536 * H * 192 + 2 * T * H * 128 * 4096
    assert work["_step"]["flops"] == proj + 2 * kv * 512 * H * 256 + 2 * (T * 2064) * H * 320
    assert abs(work["_step"]["flops"] / 1e9 - 152.8) < 0.1
    # the fused kernel carries the expansion and the attention, counted once in the step
    assert work["expand_attn"]["flops"] == work["kv_b_expand"]["flops"] + work["prefill_attn"]["flops"]


def test_causal_prefill_work_counts_the_triangle():
    # 4 x 4096 causal tokens: S (S + 1) / 2 visible pairs per sequence
    w = _shape_only("prefill_bf16", [4096] * 4, [0] * 4, ms.MASK_CAUSAL)
    work = bench.stage_work(w)
    pairs = 4 * 4096 * 4097 // 2
    assert work["prefill_attn"]["flops"] == 2 * pairs * 32 * 320
    assert abs(work["_step"]["flops"] / 1e9 - 1967.2) < 0.2


def test_sliding_window_decode_reads_window_entries():
    # one query per sequence at position L - 1 with a 1024-key window
    w = _shape_only("long_decode_bf16", [1, 1], [20000, 500], ms.MASK_SLIDING, window=1024, mode="decode")
    work = bench.stage_work(w)
    keys = 1024 + 501
    assert work["decode_attn"]["bytes"] == keys * 576 * 2
    assert work["decode_attn"]["flops"] == 2 * keys * 128 * (576 + 512)


def _write_pmc(d, rows):
    os.makedirs(d, exist_ok=True)
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=cols)
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(cols, r)))


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    # the copy of 256 MiB reads 96 MiB of FETCH_SIZE and 256 MiB of WRITE_SIZE
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # (the 512 MiB fill that evicts the Infinity Cache before flushed decode
    # calls is another elementwise kernel of the same grid: not a copy)
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>(int)"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int)"
    k = "void mla::(anonymous namespace)::decode_sk_kernel<3>(mla::DecodeAttnArgs)"
    _write_pmc(fetch, [(1, 67108864, copy, "FETCH_SIZE", 96 * 1024, 0, 1),
                       (4, 67108864, fill, "FETCH_SIZE", 16.0, 0, 1),
                       (2, 131072, k, "FETCH_SIZE", 1000.0, 0, 1),
                       (3, 131072, k, "FETCH_SIZE", 3000.0, 0, 1)])
    _write_pmc(write, [(1, 67108864, copy, "WRITE_SIZE", 256 * 1024, 0, 1),
                       (4, 67108864, fill, "WRITE_SIZE", 512 * 1024, 0, 1),
                       (2, 131072, k, "WRITE_SIZE", 10.0, 0, 1),
                       (3, 131072, k, "WRITE_SIZE", 30.0, 0, 1)])
    paths = bench.traffic_summary(fetch, write, "unit", 256, ["a", "b"], out_dir=str(tmp_path))
    rec = json.load(open([p for p in paths if "decode_attn" in p][0]))
    assert rec["dispatches"] == 2
    assert rec["fetch_factor"] == pytest.approx(256 / 96, rel=1e-4)
    assert rec["bytes_per_launch"] == int((2000.0 * 256 / 96 + 20.0) * 1024)


def test_mfma_summary_uses_the_per_xcd_active_cycles(tmp_path):
    # GRBM_GUI_ACTIVE of a dispatch is summed over the 8 XCDs: 8 x 1000 cycles;
    # half of the 1024 SIMDs' cycles MFMA-busy -> 50 %
    d = str(tmp_path / "m")
    k = "mla::(anonymous namespace)::prefill_attn_bf16_kernel(mla::PrefillAttnArgs)"
    rows = []
    for disp in (1, 2):
        rows += [(disp, 1048576, k, "GRBM_GUI_ACTIVE", 8 * 1000.0, 0, 2000),
                 (disp, 1048576, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 500.0, 0, 2000),
                 (disp, 1048576, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6, 0, 2000)]
    _write_pmc(d, rows)
    rec = json.load(open(bench.mfma_summary(d, "unit", "cmd", out_dir=str(tmp_path))))
    (ent,) = rec["kernels"]
    assert ent["kernel"] == "mla::prefill_attn_bf16_kernel"
    assert ent["dispatches"] == 2
    assert ent["mfma_busy_pct"] == pytest.approx(50.0)
    assert ent["bf16_mfma_gflop_per_dispatch"] == pytest.approx(0.512)
    assert ent["mfma_tflops_under_counters"] == pytest.approx(256.0)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_sparse_decode_counts_listed_entries():
    # a list counts its entries inside [0, L): padding and positions past L read nothing
    w = _shape_only("decode_bf16", [1, 1], [9, 4999], ms.MASK_CAUSAL, mode="decode")
    topk = np.full((2, 16), -1, dtype=np.int32)
    topk[0, :10] = np.arange(10)
    topk[0, 10] = 10  # = L, ignored
    topk[1, :16] = np.arange(0, 4800, 300)
    work = bench.stage_work(w, topk=topk)
    keys = 10 + 16
    assert work["decode_attn"]["bytes"] == keys * 576 * 2
    assert work["_step"]["cache_bytes"] == keys * 576 * 2
    assert work["decode_attn"]["flops"] == 2 * keys * 128 * (576 + 512)
