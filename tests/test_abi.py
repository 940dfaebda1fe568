"""CPU checks of the C ABI: the library loads without a GPU, exports every
function include/mla.h declares, the ctypes structures match the C layout,
and host-side validation rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re
import subprocess

import pytest

from draft_models_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"MLA_API\s+[\w\s\*]+?\b(mla_\w+)\s*\(", src)


def test_exports_every_declared_symbol():
    lib = B.load_library()
    names = _declared()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    assert exported == set(names), exported


def test_struct_layout_matches_header(tmp_path):
    prog = tmp_path / "layout.c"
    fields_c = [f for f, _ in B.mla_config._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "mla.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(mla_config), sizeof(mla_weights));']
    lines += [f'printf("%zu\\n", offsetof(mla_config, {f}));' for f in fields_c]
    lines += [f'printf("%zu\\n", offsetof(mla_weights, {f}));' for f, _ in B.mla_weights._fields_]
    lines += ["return 0;}"]
    prog.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == C.sizeof(B.mla_config) and vals[1] == C.sizeof(B.mla_weights)
    got = vals[2:]
    want = [getattr(B.mla_config, f).offset for f in fields_c] + \
           [getattr(B.mla_weights, f).offset for f, _ in B.mla_weights._fields_]
    assert got == want


def _good_cfg(**kw):
    base = dict(hidden_size=256, num_heads=4, q_lora_rank=0, kv_lora_rank=32, qk_nope_head_dim=16,
                qk_rope_head_dim=8, v_head_dim=16, rope_style=0, rope_theta=1e4, rms_norm_eps=1e-6,
                softmax_scale=0.0, use_output_gate=0, dtype=B.DTYPE_F32, page_size=64, max_batch=1,
                max_tokens=16, max_seq_len=64, max_prefill_kv=64)
    base.update(kw)
    return B.mla_config(**base)


def _good_weights(**kw):
    fake = 0x1000  # never dereferenced: validation fails before any device access
    base = dict(q_proj=fake, kv_a_proj_with_mqa=fake, kv_a_layernorm=fake, kv_b_proj=fake, o_proj=fake)
    base.update(kw)
    return B.mla_weights(**base)


def _init(cfg, w):
    lib = B.load_library()
    ctx = C.c_void_p(123)
    code = lib.mla_init_weights(C.byref(cfg), C.byref(w), None, C.byref(ctx))
    return code, ctx.value


@pytest.mark.parametrize("kw,code", [
    (dict(hidden_size=0), 2),
    (dict(num_heads=-1), 2),
    (dict(qk_rope_head_dim=7), 2),
    (dict(dtype=9), 1),
    (dict(rope_style=5), 1),
    (dict(rope_theta=0.5), 1),
    (dict(rms_norm_eps=-1.0), 1),
    (dict(use_output_gate=2), 1),
    (dict(page_size=0), 1),
    (dict(max_batch=0), 1),
    (dict(max_prefill_kv=-1), 1),
    (dict(qk_nope_head_dim=256), 3),       # n + r above 192
    (dict(kv_lora_rank=1024), 3),
    (dict(qk_nope_head_dim=18), 3),        # not a 16-byte multiple of fp32
    (dict(use_output_gate=1), 1),          # g_proj missing
    (dict(q_lora_rank=64), 1),             # q_a_proj / q_b_proj missing
    (dict(kv_cache_dtype=1, kv_cache_scale=0.0), 1),  # 8-bit cache needs a positive scale
    (dict(kv_cache_dtype=1, kv_cache_scale=0.5), 3),  # 8-bit cache needs bf16, c 512, r 64
    (dict(kv_cache_dtype=1, kv_cache_scale=0.5, dtype=B.DTYPE_BF16, kv_lora_rank=512, qk_rope_head_dim=64,
          qk_nope_head_dim=128, v_head_dim=128, max_batch=1025), 3),  # 8-bit cache: at most 1024 sequences
])
def test_init_validation(kw, code):
    got, ctx = _init(_good_cfg(**kw), _good_weights())
    assert got == code, B.last_error()
    assert ctx is None
    assert B.last_error()


def test_init_null_args():
    lib = B.load_library()
    ctx = C.c_void_p()
    assert lib.mla_init_weights(None, None, None, C.byref(ctx)) == 1
    assert lib.mla_init_weights(C.byref(_good_cfg()), C.byref(_good_weights()), None, None) == 1
    w = _good_weights(kv_b_proj=None)
    assert _init(_good_cfg(), w)[0] == 1


def test_calls_reject_null_context():
    lib = B.load_library()
    assert lib.mla_prefill_expanded(None, None, 1, 1, None, None, 1, 1, None, 1, None, 1, 0, 0,
                                    None, None, None, None) == 1
    assert "ctx" in B.last_error()
    assert lib.mla_decode_absorbed(None, None, 1, None, 1, None, 1, None, 1, 0, 0, None, None) == 1
    assert lib.mla_backward_expanded(None, None, 1, 1, None, 1, 0, 0, None, None, None, None, None, None) == 1
    assert "ctx" in B.last_error()
    assert lib.mla_decode_absorbed_noalloc(None, None, 1, None, 1, None, 1, None, 1, 0, 0, None, None) == 1
    lib.mla_free(None)  # no-op
