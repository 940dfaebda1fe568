"""ctypes binding of libmla.so (include/mla.h): argument marshalling only.

Every step of the MLA forward runs in the library's HIP kernels; this module
turns torch tensors into device pointers and the current HIP stream into a
hipStream_t, and raises MLAError on a nonzero status. There is no fallback:
if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

MLA_OK = 0
STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_DIMS", 3: "MLA_ERR_UNSUPPORTED",
          4: "MLA_ERR_CAPACITY", 5: "MLA_ERR_HIP", 6: "MLA_ERR_OOM"}
DTYPE_F32, DTYPE_BF16 = 0, 1
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1
MASK_FULL, MASK_CAUSAL, MASK_SLIDING = 0, 1, 2

EXPORTS = ("mla_init_weights", "mla_prefill_expanded", "mla_backward_expanded", "mla_decode_absorbed",
           "mla_decode_absorbed_block",
           "mla_decode_absorbed_sparse", "mla_decode_absorbed_noalloc", "mla_free", "mla_last_error",
           "mla_profile_enable", "mla_profile_read", "mla_profile_stage_name")
NUM_STAGES = 17


class MLAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class mla_config(C.Structure):
    _fields_ = [("hidden_size", C.c_int32), ("num_heads", C.c_int32), ("q_lora_rank", C.c_int32),
                ("kv_lora_rank", C.c_int32), ("qk_nope_head_dim", C.c_int32),
                ("qk_rope_head_dim", C.c_int32), ("v_head_dim", C.c_int32), ("rope_style", C.c_int32),
                ("rope_theta", C.c_double), ("rms_norm_eps", C.c_double), ("softmax_scale", C.c_double),
                ("use_output_gate", C.c_int32), ("dtype", C.c_int32), ("page_size", C.c_int32),
                ("max_batch", C.c_int32), ("max_tokens", C.c_int32), ("max_seq_len", C.c_int32),
                ("max_prefill_kv", C.c_int32), ("max_block_tokens", C.c_int32), ("max_topk", C.c_int32),
                ("kv_cache_dtype", C.c_int32), ("kv_cache_scale", C.c_float), ("max_train_tokens", C.c_int32)]

KV_CACHE_COMPUTE, KV_CACHE_FP8_E4M3 = 0, 1


WEIGHT_NAMES = ("q_a_proj", "q_a_layernorm", "q_b_proj", "q_proj", "kv_a_proj_with_mqa",
                "kv_a_layernorm", "kv_b_proj", "o_proj", "g_proj")


class mla_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_NAMES]


class mla_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_NAMES]


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load libmla.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m draft_models_amd.build`")
    lib = C.CDLL(path)
    vp, i32 = C.c_void_p, C.c_int32
    lib.mla_init_weights.argtypes = [C.POINTER(mla_config), C.POINTER(mla_weights), vp, C.POINTER(vp)]
    lib.mla_init_weights.restype = C.c_int
    lib.mla_prefill_expanded.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                         vp, vp, vp, vp]
    lib.mla_prefill_expanded.restype = C.c_int
    lib.mla_backward_expanded.argtypes = [vp, vp, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp, C.POINTER(mla_grads),
                                          vp]
    lib.mla_backward_expanded.restype = C.c_int
    lib.mla_decode_absorbed.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, vp, vp]
    lib.mla_decode_absorbed.restype = C.c_int
    lib.mla_decode_absorbed_block.argtypes = [vp, vp, i32, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_decode_absorbed_block.restype = C.c_int
    lib.mla_decode_absorbed_sparse.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, i32, vp, i32, vp, vp]
    lib.mla_decode_absorbed_sparse.restype = C.c_int
    lib.mla_decode_absorbed_noalloc.argtypes = [vp, vp, i32, vp, i32, vp, i32, vp, i32, i32, i32, vp, vp]
    lib.mla_decode_absorbed_noalloc.restype = C.c_int
    lib.mla_free.argtypes = [vp]
    lib.mla_free.restype = None
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = C.c_char_p
    lib.mla_profile_enable.argtypes = [vp, i32]
    lib.mla_profile_enable.restype = C.c_int
    lib.mla_profile_read.argtypes = [vp, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
    lib.mla_profile_read.restype = C.c_int
    lib.mla_profile_stage_name.argtypes = [i32]
    lib.mla_profile_stage_name.restype = C.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().mla_last_error().decode()


def _check(code: int):
    if code != MLA_OK:
        raise MLAError(code, last_error())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_config(dims, *, max_batch: int, max_tokens: int, max_seq_len: int, max_prefill_kv: int,
                softmax_scale: float = 0.0, max_block_tokens: int = 0, max_topk: int = 0,
                kv_scale: float = 0.0, max_train_tokens: int = 0) -> mla_config:
    """mla_config from an object with the model-dimension attributes; kv_scale
    > 0 selects the 8-bit (E4M3) cache with that per-tensor scale."""
    return mla_config(
        hidden_size=dims.hidden_size, num_heads=dims.num_heads, q_lora_rank=dims.q_lora_rank,
        kv_lora_rank=dims.kv_lora_rank, qk_nope_head_dim=dims.qk_nope_head_dim,
        qk_rope_head_dim=dims.qk_rope_head_dim, v_head_dim=dims.v_head_dim,
        rope_style=dims.rope_style, rope_theta=dims.rope_theta, rms_norm_eps=dims.rms_norm_eps,
        softmax_scale=softmax_scale, use_output_gate=int(dims.use_output_gate),
        dtype=DTYPE_BF16 if dims.dtype == "bf16" else DTYPE_F32, page_size=dims.page_size,
        max_batch=max_batch, max_tokens=max_tokens, max_seq_len=max_seq_len,
        max_prefill_kv=max_prefill_kv, max_block_tokens=max_block_tokens, max_topk=max_topk,
        kv_cache_dtype=KV_CACHE_FP8_E4M3 if kv_scale > 0 else KV_CACHE_COMPUTE, kv_cache_scale=float(kv_scale),
        max_train_tokens=max_train_tokens)


class MLA:
    """One MLA layer on the GPU: owns an mla_ctx."""

    def __init__(self, cfg: mla_config, weights: Dict[str, "object"], stream=None):
        lib = load_library()
        w = mla_weights(**{n: _ptr(weights.get(n)) for n in WEIGHT_NAMES})
        ctx = C.c_void_p()
        _check(lib.mla_init_weights(C.byref(cfg), C.byref(w), _stream(stream), C.byref(ctx)))
        self._lib, self.ctx, self.cfg = lib, ctx, cfg

    def prefill(self, x, cu_seqlens, prefix_lens, max_q_len: int, max_kv_len: int, kv_cache, block_table,
                mask_kind: int, window: int, out, row_lo=None, row_hi=None, stream=None):
        _check(self._lib.mla_prefill_expanded(
            self.ctx, _ptr(x), cu_seqlens.numel() - 1, x.shape[0], _ptr(cu_seqlens), _ptr(prefix_lens),
            max_q_len, max_kv_len, _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
            block_table.shape[1], mask_kind, window, _ptr(row_lo), _ptr(row_hi), _ptr(out), _stream(stream)))

    def backward(self, x, cu_seqlens, max_q_len: int, mask_kind: int, window: int, dout, dx,
                 grads: Dict[str, "object"], row_lo=None, row_hi=None, stream=None):
        """Gradient of the expanded layer on training sequences: dx and the
        weight gradients named in grads (tensors shaped like the weights)."""
        g = mla_grads(**{n: _ptr(grads.get(n)) for n in WEIGHT_NAMES})
        _check(self._lib.mla_backward_expanded(
            self.ctx, _ptr(x), cu_seqlens.numel() - 1, x.shape[0], _ptr(cu_seqlens), max_q_len, mask_kind, window,
            _ptr(row_lo), _ptr(row_hi), _ptr(dout), _ptr(dx), C.byref(g), _stream(stream)))

    def decode(self, x, kv_cache, block_table, seq_lens, max_seq_len: int, mask_kind: int, window: int, out,
               stream=None):
        _check(self._lib.mla_decode_absorbed(
            self.ctx, _ptr(x), x.shape[0], _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), max_seq_len, mask_kind, window, _ptr(out), _stream(stream)))

    def decode_noalloc(self, x, kv_cache, block_table, seq_lens, max_seq_len: int, mask_kind: int, window: int,
                       out, stream=None):
        """decode() with the per-call workspaces in the library's static scratch array."""
        _check(self._lib.mla_decode_absorbed_noalloc(
            self.ctx, _ptr(x), x.shape[0], _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), max_seq_len, mask_kind, window, _ptr(out), _stream(stream)))

    def decode_block(self, x, q_len: int, kv_cache, block_table, prefix_lens, max_kv_len: int, out, stream=None):
        """Blocks of q_len tokens per sequence, block-visible, absorbed form."""
        _check(self._lib.mla_decode_absorbed_block(
            self.ctx, _ptr(x), prefix_lens.numel(), q_len, _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(prefix_lens), max_kv_len, _ptr(out), _stream(stream)))

    def decode_sparse(self, x, kv_cache, block_table, seq_lens, max_seq_len: int, topk_indices, out, stream=None):
        """One token per sequence attending to its listed positions (topk_indices [batch, topk] int32)."""
        _check(self._lib.mla_decode_absorbed_sparse(
            self.ctx, _ptr(x), x.shape[0], _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), max_seq_len, _ptr(topk_indices), topk_indices.shape[1],
            _ptr(out), _stream(stream)))

    def profile(self, enable: bool):
        _check(self._lib.mla_profile_enable(self.ctx, int(enable)))

    def profile_read(self) -> Dict[str, tuple]:
        """{stage name: (total ms, launches)} since the last read (synchronises)."""
        ms = (C.c_double * NUM_STAGES)()
        cnt = (C.c_int32 * NUM_STAGES)()
        _check(self._lib.mla_profile_read(self.ctx, ms, cnt))
        return {self._lib.mla_profile_stage_name(i).decode(): (ms[i], cnt[i]) for i in range(NUM_STAGES)}

    def close(self):
        if self.ctx:
            self._lib.mla_free(self.ctx)
            self.ctx = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
