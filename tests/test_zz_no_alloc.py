"""mla_decode_absorbed_noalloc (workspaces in the library's static scratch
array) against mla_decode_absorbed on the same inputs: two calls in a row,
the second with fewer and shorter sequences, so that it runs over scratch
contents the first call left behind. Same kernels, so the outputs and the
written cache entries must be bitwise equal; the first call is also checked
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import mla_synth as ms
from mla_synth.device import from_torch, upload
from draft_models_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts only with -m gpu
    pytest.skip("needs a GPU", allow_module_level=True)


def _calls(big, small, mask_kind=ms.MASK_CAUSAL, window=0):
    tb, ts = upload(big), upload(small)
    d = big.dims
    max_kv = int(big.kv_lens.max())
    cfg = B.make_config(d, max_batch=big.batch, max_tokens=big.batch, max_seq_len=max_kv, max_prefill_kv=0,
                        kv_scale=big.kv_scale)
    m = B.MLA(cfg, tb["weights"])
    res = {}
    caches = {k: (tb["cache"].clone(), ts["cache"].clone()) for k in ("noalloc", "regular")}
    for kind in ("noalloc", "regular"):
        call = m.decode_noalloc if kind == "noalloc" else m.decode
        outs = []
        for w, t, cache in ((big, tb, caches[kind][0]), (small, ts, caches[kind][1])):
            U.say(f"  {kind}: batch {w.batch}, max_kv {int(w.kv_lens.max())}")
            out = torch.full((w.batch, d.hidden_size), float("nan"), dtype=torch.bfloat16, device="cuda")
            call(t["x"], cache, t["block_table"], t["seq_lens"], int(w.kv_lens.max()), mask_kind, window, out)
            outs.append(out)
        torch.cuda.synchronize()
        res[kind] = outs
    m.close()
    for i in range(2):
        a, b = res["noalloc"][i], res["regular"][i]
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i}: outputs differ"
        ca, cb = caches["noalloc"][i], caches["regular"][i]
        assert torch.equal(ca.view(torch.uint8), cb.view(torch.uint8)), f"call {i}: caches differ"
    cache0 = caches["noalloc"][0]
    cache0 = cache0.cpu().numpy() if big.kv_scale > 0 else from_torch(cache0)
    U.check(big, from_torch(res["noalloc"][0]), cache0, U.oracle(big))


def test_noalloc_matches_decode():
    big = ms.make_workload("decode_bf16", seq_lens=[1, 65, 700, 333, 64, 2000, 31, 129], seed=61)
    small = ms.make_workload("decode_bf16", seq_lens=[5, 300, 40], seed=61)
    U.say("[noalloc] decode_bf16 seed 61, batches 8 then 3")
    _calls(big, small)


def test_noalloc_matches_decode_window_fp8():
    """Sliding window and an 8-bit cache, 16 heads with an output gate."""
    over = {"num_heads": 16, "use_output_gate": True}
    big = ms.make_workload("decode_bf16", seq_lens=[90, 1000, 3, 257, 64], seed=62, dims_override=over,
                           kv_scale=2.0 ** -5, mask_kind=ms.MASK_SLIDING, window=100)
    small = ms.make_workload("decode_bf16", seq_lens=[17, 33], seed=62, dims_override=over, kv_scale=2.0 ** -5,
                             mask_kind=ms.MASK_SLIDING, window=100)
    U.say("[noalloc] decode_bf16 16 heads, gate, fp8, window 100, batches 5 then 2")
    _calls(big, small, ms.MASK_SLIDING, 100)


def test_noalloc_rejects_oversized_call():
    """A call whose workspaces do not fit the scratch array fails before any
    launch with MLA_ERR_CAPACITY: 1024 sequences x 128 heads."""
    w = ms.make_workload("decode_bf16", seq_lens=[8] * 1024, seed=63)
    t = upload(w)
    d = w.dims
    cfg = B.make_config(d, max_batch=w.batch, max_tokens=w.batch, max_seq_len=8, max_prefill_kv=0)
    m = B.MLA(cfg, t["weights"])
    before = t["cache"].clone()
    out = torch.zeros((w.batch, d.hidden_size), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MLAError) as e:
        m.decode_noalloc(t["x"], t["cache"], t["block_table"], t["seq_lens"], 8, ms.MASK_CAUSAL, 0, out)
    torch.cuda.synchronize()
    m.close()
    assert e.value.code == 4
    assert torch.equal(before.view(torch.int16), t["cache"].view(torch.int16))
