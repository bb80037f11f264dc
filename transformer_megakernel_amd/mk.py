"""Python binding of libmk.so (argument marshalling only; every step runs in HIP kernels).

Mirrors include/mk.h: ``Megakernel`` wraps an ``mk_ctx``; torch supplies device memory
and the stream handle.  If the library is missing the binding raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

from .synth import ModelShape, Weights

_PKG = os.path.dirname(os.path.abspath(__file__))
# MK_LIBRARY may name another build of the library (e.g. one compiled with other options).
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(_PKG, "libmk.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mk.h")

MK_OK, MK_EINVAL, MK_ERANGE, MK_ESTATE, MK_EHIP, MK_ETIMEOUT, MK_ENOMEM = 0, -1, -2, -3, -4, -5, -6


class MkError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with {code}: {msg}")
        self.code = code


class MkConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class MkWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP),
                ("mlp_norm", _PP), ("w_gate", _PP), ("w_up", _PP), ("w_down", _PP)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmk.so (built in-tree by transformer_megakernel_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.mk_create.argtypes = [ctypes.POINTER(MkConfig), ctypes.c_int, ctypes.POINTER(vp)]
        L.mk_plan_only.argtypes = [ctypes.POINTER(MkConfig), ctypes.c_int, ctypes.POINTER(vp)]
        L.mk_load_weights.argtypes = [vp, ctypes.POINTER(MkWeights)]
        L.mk_decode_step.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.mk_decode_step_dev.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.mk_decode_step_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, vp]
        L.mk_sync.argtypes = [vp, vp]
        L.mk_set_watchdog_us.argtypes = [vp, i64]
        L.mk_plan_info.argtypes = [vp, ctypes.POINTER(i32)]
        L.mk_plan_copy.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), i64]
        L.mk_debug_dump.argtypes = [vp, ctypes.POINTER(ctypes.c_uint64), i64, ctypes.POINTER(i64)]
        L.mk_set_trace.argtypes = [vp, vp, i64, ctypes.POINTER(i64)]
        L.mk_stream_read.argtypes = [vp, i64, vp, i32, i32, vp]
        L.mk_bench_gemv_page.argtypes = [i32, i32, i32, vp, vp, vp]
        L.mk_bench_poll_latency.argtypes = [vp, i64, vp, i32, i32, i32, i32, vp, vp]
        L.mk_bench_bcast_read.argtypes = [vp, i32, i32, i32, vp, vp]
        L.mk_destroy.argtypes = [vp]
        L.mk_destroy.restype = None
        L.mk_strerror.argtypes = [ctypes.c_int]
        L.mk_strerror.restype = ctypes.c_char_p
        L.mk_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_symbols() -> list:
    """Function names include/mk.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", txt)))


def _check(code: int, where: str):
    if code != MK_OK:
        raise MkError(code, where, lib().mk_strerror(code).decode())


check = _check


def make_config(shape: ModelShape, max_ctx: int) -> MkConfig:
    return MkConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                    shape.ffn, shape.vocab, max_ctx, shape.rms_eps, shape.rope_theta)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


ptr = _ptr


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


class Megakernel:
    """One decode context: static schedule + device buffers for a model shape."""

    def __init__(self, shape: ModelShape, max_ctx: int, device: int = 0):
        self.shape, self.max_ctx, self.device = shape, max_ctx, device
        self._cfg = make_config(shape, max_ctx)
        h = ctypes.c_void_p()
        _check(lib().mk_create(ctypes.byref(self._cfg), device, ctypes.byref(h)), "mk_create")
        self._h = h
        self._keep = None

    @classmethod
    def plan_only(cls, shape: ModelShape, max_ctx: int, n_cus: int) -> "Megakernel":
        self = cls.__new__(cls)
        self.shape, self.max_ctx, self.device = shape, max_ctx, -1
        self._cfg = make_config(shape, max_ctx)
        h = ctypes.c_void_p()
        _check(lib().mk_plan_only(ctypes.byref(self._cfg), n_cus, ctypes.byref(h)), "mk_plan_only")
        self._h = h
        self._keep = None
        return self

    def load_weights(self, W: Weights):
        L = self.shape.n_layers

        def arr(ts):
            a = (ctypes.c_void_p * L)(*[_ptr(t) for t in ts])
            return a

        arrays = {k: arr(getattr(W, k)) for k in
                  ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")}
        mw = MkWeights(_ptr(W.embed), _ptr(W.lm_head), _ptr(W.final_norm),
                       *[ctypes.cast(arrays[k], _PP) for k in
                         ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")])
        _check(lib().mk_load_weights(self._h, ctypes.byref(mw)), "mk_load_weights")
        self._keep = W   # the library borrows the pointers

    def decode_step(self, token: int, pos: int, kv, logits, next_token=None, stream=None):
        _check(lib().mk_decode_step(self._h, int(token), int(pos), _ptr(kv), _ptr(logits), _ptr(next_token),
                                    _stream(stream)), "mk_decode_step")

    def decode_step_dev(self, token_dev, pos: int, kv, logits, next_token=None, stream=None):
        _check(lib().mk_decode_step_dev(self._h, _ptr(token_dev), int(pos), _ptr(kv), _ptr(logits),
                                        _ptr(next_token), _stream(stream)), "mk_decode_step_dev")

    def decode_step_noalloc(self, token: int, pos: int, kv, logits, next_token=None, stream=None):
        """mk_decode_step_noalloc: the step on the device's static scratch (allocates nothing)."""
        _check(lib().mk_decode_step_noalloc(self._h, int(token), int(pos), _ptr(kv), _ptr(logits),
                                            _ptr(next_token), _stream(stream)), "mk_decode_step_noalloc")

    def sync(self, stream=None) -> int:
        """Wait for the stream; raise on a device-side error."""
        code = lib().mk_sync(self._h, _stream(stream))
        _check(code, "mk_sync")
        return code

    def sync_code(self, stream=None) -> int:
        return lib().mk_sync(self._h, _stream(stream))

    def set_watchdog_us(self, us: int):
        _check(lib().mk_set_watchdog_us(self._h, int(us)), "mk_set_watchdog_us")

    def plan(self) -> dict:
        info = (ctypes.c_int32 * 8)()
        _check(lib().mk_plan_info(self._h, info), "mk_plan_info")
        n_cus, words, n_rec = info[0], info[1], info[2]
        off = np.zeros(n_cus + 1, np.int32)
        rec = np.zeros(n_rec * words, np.int32)
        _check(lib().mk_plan_copy(self._h, off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  rec.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), rec.size), "mk_plan_copy")
        return dict(n_cus=n_cus, offsets=off, records=rec.reshape(n_rec, words), page_bytes=info[3],
                    ring_pages=info[4], compute_waves=info[5], s_max=info[6], lds_bytes=info[7])

    def enable_trace(self, device="cuda:0"):
        """Allocate a trace buffer (torch, on the device) and start recording; returns it."""
        import torch
        need = ctypes.c_int64()
        _check(lib().mk_set_trace(self._h, None, 0, ctypes.byref(need)), "mk_set_trace")
        buf = torch.zeros(need.value, dtype=torch.int64, device=device)
        _check(lib().mk_set_trace(self._h, _ptr(buf), need.value, ctypes.byref(need)), "mk_set_trace")
        self._trace = buf
        return buf

    def disable_trace(self):
        need = ctypes.c_int64()
        _check(lib().mk_set_trace(self._h, None, 0, ctypes.byref(need)), "mk_set_trace")
        self._trace = None

    def debug_dump(self) -> dict:
        """Intermediates of the last step as (values fp32, epochs) per buffer."""
        offs = (ctypes.c_int64 * 6)()
        _check(lib().mk_debug_dump(self._h, None, 0, offs), "mk_debug_dump")
        buf = np.zeros(offs[5], np.uint64)
        _check(lib().mk_debug_dump(self._h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), buf.size, offs),
               "mk_debug_dump")
        vals = (buf & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
        ep = (buf >> np.uint64(32)).astype(np.uint32)
        names = ["x", "qkv", "part", "o", "a"]
        out = {}
        for i, n in enumerate(names):
            out[n] = (vals[offs[i]:offs[i + 1]], ep[offs[i]:offs[i + 1]])
        return out

    def close(self):
        if getattr(self, "_h", None):
            lib().mk_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# opcode numbers of the instruction records
OP_QKV, OP_ATTN, OP_O, OP_GATEUP, OP_DOWN, OP_LMHEAD = 1, 2, 3, 4, 5, 6


def stream_read(buf, sink, blocks: int, unroll: int, stream=None):
    """Launch the library's plain streaming-read kernel over the whole of ``buf`` (a
    device tensor); ``sink``: device int32 tensor of at least ``blocks`` elements."""
    _check(lib().mk_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(blocks), int(unroll),
                                _stream(stream)), "mk_stream_read")
