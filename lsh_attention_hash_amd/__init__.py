"""MI355X-native Reformer shared-QK LSH self-attention (forward).

Thin Python binding of the C ABI in include/lsh_attn.h. This module only
marshals arguments: it checks devices, dtypes, shapes and contiguity, allocates
outputs with torch on the current device, and passes raw pointers and torch's
current HIP stream to liblsh_attn.so. Every step of the computation runs in the
library's HIP kernels. There is no CPU fallback: if the library is not built or
cannot be loaded, use of this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["LSHAttention", "ChunkedFeedForward", "forward_static", "load_library",
           "library_path", "LSHAttnError", "EXPORTED_SYMBOLS", "FLAG_SEPARATE_GATHER"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "_lib", "liblsh_attn.so")

FP32, BF16 = 0, 1
FLAG_SEPARATE_GATHER = 1
FLAG_FP32_ROUND_OUTPUTS = 2
FLAG_BACKWARD = 4
FLAG_LOOK_AHEAD = 8
FLAG_SAME_BUCKET = 16
FLAG_NORM_QUERIES = 32
FLAG_DEDUP = 64
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "OUT_OF_MEMORY", 4: "HIP",
          5: "WORKSPACE_TOO_LARGE"}
STATIC_SCRATCH_BYTES = 64 << 20

# Every function declared in include/lsh_attn.h.
EXPORTED_SYMBOLS = ("lsh_attn_create", "lsh_attn_forward", "lsh_attn_forward_x",
                    "lsh_attn_backward", "lsh_attn_backward_buckets", "lsh_attn_forward_static",
                    "lsh_attn_get_stats",
                    "lsh_attn_set_timing", "lsh_attn_get_timing", "lsh_attn_get_backward_timing",
                    "lsh_attn_workspace_bytes", "lsh_attn_destroy", "lsh_attn_strerror",
                    "lsh_ffn_create", "lsh_ffn_forward", "lsh_ffn_set_timing",
                    "lsh_ffn_get_timing", "lsh_ffn_workspace_bytes", "lsh_ffn_destroy")
N_STAGES = 8
STAGES = ("hash_prep", "hash", "hash_rescore", "sort", "gather", "attend", "combine", "project")
N_BWD_STAGES = 4
BWD_STAGES = ("recompute", "rows", "products", "reduce")
N_FFN_STAGES = 2
FFN_STAGES = ("ffn_up", "ffn_down")


class LSHAttnError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        msg = lib.lsh_attn_strerror(status).decode() if lib is not None else ""
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "seq_len", "head_dim", "n_buckets", "n_rounds", "chunk_len", "causal",
        "dtype", "out_dtype", "flags")]


class FFNConfig(ctypes.Structure):
    _fields_ = [("max_rows", ctypes.c_int64), ("chunk_rows", ctypes.c_int64),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("n_exact_rescored", ctypes.c_int64), ("n_full_fallback", ctypes.c_int64),
                ("n_round_rows_at_fp16_limit", ctypes.c_int64),
                ("n_grad_rows_at_fp16_limit", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load liblsh_attn.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m lsh_attention_hash_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.lsh_attn_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
    lib.lsh_attn_forward.argtypes = [P, P, P, P, P, P, P, P, P]
    lib.lsh_attn_forward_x.argtypes = [P, P, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P]
    lib.lsh_attn_backward.argtypes = [P, P, P, P, P, P, P, P]
    lib.lsh_attn_backward_buckets.argtypes = [P, P, P, P, P, P, P, P, P]
    lib.lsh_attn_forward_static.argtypes = [ctypes.POINTER(Config), P, P, P, P, P, P, P, P]
    lib.lsh_attn_get_stats.argtypes = [P, ctypes.POINTER(Stats)]
    lib.lsh_attn_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.lsh_attn_set_timing.argtypes = [P, I]
    lib.lsh_attn_get_timing.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
    lib.lsh_attn_get_backward_timing.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                                 ctypes.POINTER(ctypes.c_int64)]
    lib.lsh_attn_destroy.argtypes = [P]
    lib.lsh_attn_strerror.argtypes = [I]
    lib.lsh_attn_strerror.restype = ctypes.c_char_p
    lib.lsh_ffn_create.argtypes = [ctypes.POINTER(FFNConfig), ctypes.POINTER(P)]
    lib.lsh_ffn_forward.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P, P, P]
    lib.lsh_ffn_set_timing.argtypes = [P, I]
    lib.lsh_ffn_get_timing.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64)]
    lib.lsh_ffn_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.lsh_ffn_destroy.argtypes = [P]
    for n in ("lsh_attn_create", "lsh_attn_forward", "lsh_attn_forward_x", "lsh_attn_backward",
              "lsh_attn_backward_buckets", "lsh_attn_forward_static",
              "lsh_attn_get_stats",
              "lsh_attn_set_timing", "lsh_attn_get_timing", "lsh_attn_get_backward_timing",
              "lsh_attn_workspace_bytes", "lsh_attn_destroy", "lsh_ffn_create",
              "lsh_ffn_forward", "lsh_ffn_set_timing", "lsh_ffn_get_timing",
              "lsh_ffn_workspace_bytes", "lsh_ffn_destroy"):
        getattr(lib, n).restype = I
    _lib = lib
    return lib


def _dtype_code(dt) -> int:
    if dt in (torch.bfloat16, "bf16", BF16):
        return BF16
    if dt in (torch.float32, "fp32", FP32):
        return FP32
    raise ValueError(f"unsupported dtype {dt!r}")


_TORCH = {BF16: torch.bfloat16, FP32: torch.float32}


def make_config(batch, heads, seq_len, head_dim, n_buckets, n_rounds, chunk_len=64,
                causal=False, dtype=torch.bfloat16, out_dtype=None, flags=0) -> Config:
    dc = _dtype_code(dtype)
    oc = dc if out_dtype is None else _dtype_code(out_dtype)
    return Config(int(batch), int(heads), int(seq_len), int(head_dim), int(n_buckets),
                  int(n_rounds), int(chunk_len), int(causal), dc, oc, int(flags))


def forward_static(qk, v, rotations, n_buckets, n_rounds, chunk_len=64, causal=False,
                   out=None, lse=None, buckets=None, perm=None, out_dtype=None,
                   separate_gather=False, fp32_round_outputs=False, look_ahead=False,
                   same_bucket=False, norm_queries=False, dedup=False, stream=None):
    """The forward through lsh_attn_forward_static: no handle, and no device
    allocation in the library (its workspace is a static device array of
    STATIC_SCRATCH_BYTES per GPU; calls that overlap on one GPU race). qk, v
    [B, H, L, d] and rotations as for LSHAttention; out [B, H, L, d] and the
    optional lse, buckets, perm [B, H, R, L] are written when given (out is
    allocated with torch if None, on the caller's side of the boundary).
    Returns out."""
    lib = load_library()
    B, H, L, d = qk.shape
    flags = (FLAG_SEPARATE_GATHER if separate_gather else 0) | (
        FLAG_FP32_ROUND_OUTPUTS if fp32_round_outputs else 0) | (
        FLAG_LOOK_AHEAD if look_ahead else 0) | (FLAG_SAME_BUCKET if same_bucket else 0) | (
        FLAG_NORM_QUERIES if norm_queries else 0) | (FLAG_DEDUP if dedup else 0)
    cfg = make_config(B, H, L, d, n_buckets, n_rounds, chunk_len, causal, qk.dtype,
                      out_dtype, flags)
    dev = qk.device
    for name, t in (("qk", qk), ("v", v)):
        if t.device != dev or t.dtype != qk.dtype or tuple(t.shape) != (B, H, L, d) or \
                not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {qk.dtype} tensor {(B, H, L, d)} "
                             f"on {dev}")
    if out is None:
        out = torch.empty((B, H, L, d), dtype=_TORCH[cfg.out_dtype], device=dev)
    per_round = (B, H, n_rounds, L)
    for name, t, dt, shp in (("out", out, _TORCH[cfg.out_dtype], (B, H, L, d)),
                             ("rotations", rotations, torch.float32,
                              (n_rounds, d, n_buckets // 2)),
                             ("lse", lse, torch.float32, per_round),
                             ("buckets", buckets, torch.int32, per_round),
                             ("perm", perm, torch.int32, per_round)):
        if t is None:
            continue
        if t.device != dev or t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {dt} tensor {shp} on {dev}")
    s = (stream if stream is not None else torch.cuda.current_stream(dev)).cuda_stream
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    with torch.cuda.device(dev):
        rc = lib.lsh_attn_forward_static(ctypes.byref(cfg), ptr(qk), ptr(v), ptr(rotations),
                                         ptr(out), ptr(lse), ptr(buckets), ptr(perm),
                                         ctypes.c_void_p(s))
    if rc != 0:
        raise LSHAttnError(rc, "lsh_attn_forward_static", lib)
    return out


class LSHAttention:
    """One problem shape bound to a library handle (and its device workspace).

    Call with qk, v [B, H, L, d] (dtype) and rotations [n_rounds, d, n_buckets/2]
    float32, all contiguous on the handle's device. Returns out [B, H, L, d]
    (out_dtype), or (out, extras) when any return_* flag is set, with extras
    holding lse [B, H, R, L] float32, buckets and perm [B, H, R, L] int32.
    """

    def __init__(self, batch, heads, seq_len, head_dim, n_buckets, n_rounds, chunk_len=64,
                 causal=False, dtype=torch.bfloat16, out_dtype=None, separate_gather=False,
                 fp32_round_outputs=False, backward=False, device=None, look_ahead=False,
                 same_bucket=False, norm_queries=False, dedup=False):
        self.lib = load_library()
        flags = (FLAG_SEPARATE_GATHER if separate_gather else 0) | (
            FLAG_FP32_ROUND_OUTPUTS if fp32_round_outputs else 0) | (
            FLAG_BACKWARD if backward else 0) | (FLAG_LOOK_AHEAD if look_ahead else 0) | (
            FLAG_SAME_BUCKET if same_bucket else 0) | (
            FLAG_NORM_QUERIES if norm_queries else 0) | (FLAG_DEDUP if dedup else 0)
        self.cfg = make_config(batch, heads, seq_len, head_dim, n_buckets, n_rounds, chunk_len,
                               causal, dtype, out_dtype, flags)
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None
                                   else torch.device(device).index or 0)
        self.handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = self.lib.lsh_attn_create(ctypes.byref(self.cfg), ctypes.byref(self.handle))
        if rc != 0:
            self.handle = ctypes.c_void_p()
            raise LSHAttnError(rc, "lsh_attn_create", self.lib)

    @property
    def dtype(self):
        return _TORCH[self.cfg.dtype]

    @property
    def out_dtype(self):
        return _TORCH[self.cfg.out_dtype]

    def _check(self, name, t, shape, dtype):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, expected {self.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def __call__(self, qk, v, rotations, out=None, return_lse=False, return_buckets=False,
                 return_perm=False, stream=None):
        c = self.cfg
        shp = (c.batch, c.heads, c.seq_len, c.head_dim)
        self._check("qk", qk, shp, self.dtype)
        self._check("v", v, shp, self.dtype)
        if c.n_buckets > 1:
            self._check("rotations", rotations, (c.n_rounds, c.head_dim, c.n_buckets // 2),
                        torch.float32)
        elif rotations is not None:
            raise ValueError("rotations must be None when n_buckets == 1")
        if out is None:
            out = torch.empty(shp, dtype=self.out_dtype, device=self.device)
        else:
            self._check("out", out, shp, self.out_dtype)
        per_round = (c.batch, c.heads, c.n_rounds, c.seq_len)
        lse = torch.empty(per_round, dtype=torch.float32, device=self.device) if return_lse else None
        bk = torch.empty(per_round, dtype=torch.int32, device=self.device) if return_buckets else None
        pm = torch.empty(per_round, dtype=torch.int32, device=self.device) if return_perm else None
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        with torch.cuda.device(self.device):
            rc = self.lib.lsh_attn_forward(self.handle, ptr(qk), ptr(v), ptr(rotations), ptr(out),
                                           ptr(lse), ptr(bk), ptr(pm), ctypes.c_void_p(s))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_forward", self.lib)
        if return_lse or return_buckets or return_perm:
            return out, {"lse": lse, "buckets": bk, "perm": pm}
        return out

    def forward_x(self, x, w_qk, w_v, rotations, qk=None, v=None, out=None, return_lse=False,
                  return_buckets=False, return_perm=False, stream=None):
        """The forward from a layer input: x [B, L, model_dim] (dtype) and the
        weights w_qk, w_v [H * d, model_dim] (dtype) give qk and v [B, H, L, d],
        then the forward runs on them. Returns (out, qk, v), with the extras
        dict appended when any return_* flag is set."""
        c = self.cfg
        if x.dim() != 3 or x.shape[0] != c.batch or x.shape[1] != c.seq_len:
            raise ValueError(f"x: expected [B={c.batch}, L={c.seq_len}, model_dim], got {tuple(x.shape)}")
        model_dim = x.shape[2]
        self._check("x", x, (c.batch, c.seq_len, model_dim), self.dtype)
        self._check("w_qk", w_qk, (c.heads * c.head_dim, model_dim), self.dtype)
        self._check("w_v", w_v, (c.heads * c.head_dim, model_dim), self.dtype)
        shp = (c.batch, c.heads, c.seq_len, c.head_dim)
        if c.n_buckets > 1:
            self._check("rotations", rotations, (c.n_rounds, c.head_dim, c.n_buckets // 2),
                        torch.float32)
        elif rotations is not None:
            raise ValueError("rotations must be None when n_buckets == 1")
        qk = torch.empty(shp, dtype=self.dtype, device=self.device) if qk is None else qk
        v = torch.empty(shp, dtype=self.dtype, device=self.device) if v is None else v
        self._check("qk", qk, shp, self.dtype)
        self._check("v", v, shp, self.dtype)
        if out is None:
            out = torch.empty(shp, dtype=self.out_dtype, device=self.device)
        else:
            self._check("out", out, shp, self.out_dtype)
        per_round = (c.batch, c.heads, c.n_rounds, c.seq_len)
        lse = torch.empty(per_round, dtype=torch.float32, device=self.device) if return_lse else None
        bk = torch.empty(per_round, dtype=torch.int32, device=self.device) if return_buckets else None
        pm = torch.empty(per_round, dtype=torch.int32, device=self.device) if return_perm else None
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        with torch.cuda.device(self.device):
            rc = self.lib.lsh_attn_forward_x(self.handle, ptr(x), ctypes.c_int32(model_dim),
                                             ptr(w_qk), ptr(w_v), ptr(rotations), ptr(qk), ptr(v),
                                             ptr(out), ptr(lse), ptr(bk), ptr(pm),
                                             ctypes.c_void_p(s))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_forward_x", self.lib)
        if return_lse or return_buckets or return_perm:
            return out, qk, v, {"lse": lse, "buckets": bk, "perm": pm}
        return out, qk, v

    def backward(self, qk, v, perm, dout, dqk=None, dv=None, stream=None, buckets=None):
        """Gradients (dqk, dv) [B, H, L, d] (dtype) given dout = dL/dout, at the
        permutations perm [B, H, R, L] int32 returned by the forward (call it
        with return_perm=True; with the same-bucket reading also pass its
        buckets [B, H, R, L] int32, return_buckets=True). Needs backward=True
        at construction."""
        c = self.cfg
        shp = (c.batch, c.heads, c.seq_len, c.head_dim)
        self._check("qk", qk, shp, self.dtype)
        self._check("v", v, shp, self.dtype)
        self._check("perm", perm, (c.batch, c.heads, c.n_rounds, c.seq_len), torch.int32)
        if buckets is not None:
            self._check("buckets", buckets, (c.batch, c.heads, c.n_rounds, c.seq_len),
                        torch.int32)
        self._check("dout", dout, shp, self.dtype)
        if dqk is None:
            dqk = torch.empty(shp, dtype=self.dtype, device=self.device)
        else:
            self._check("dqk", dqk, shp, self.dtype)
        if dv is None:
            dv = torch.empty(shp, dtype=self.dtype, device=self.device)
        else:
            self._check("dv", dv, shp, self.dtype)
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        with torch.cuda.device(self.device):
            if buckets is None:
                rc = self.lib.lsh_attn_backward(self.handle, ptr(qk), ptr(v), ptr(perm),
                                                ptr(dout), ptr(dqk), ptr(dv), ctypes.c_void_p(s))
                name = "lsh_attn_backward"
            else:
                rc = self.lib.lsh_attn_backward_buckets(self.handle, ptr(qk), ptr(v), ptr(perm),
                                                        ptr(buckets), ptr(dout), ptr(dqk),
                                                        ptr(dv), ctypes.c_void_p(s))
                name = "lsh_attn_backward_buckets"
        if rc != 0:
            raise LSHAttnError(rc, name, self.lib)
        return dqk, dv

    def stats(self) -> dict:
        st = Stats()
        rc = self.lib.lsh_attn_get_stats(self.handle, ctypes.byref(st))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_get_stats", self.lib)
        return {k: getattr(st, k) for k, _ in Stats._fields_}

    def set_timing(self, capacity: int) -> None:
        """Record per-stage HIP events for the next `capacity` forwards (0 disables)."""
        rc = self.lib.lsh_attn_set_timing(self.handle, int(capacity))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_set_timing", self.lib)

    def get_timing(self):
        """(dict stage -> summed ms, number of timed forwards); resets the sums."""
        ms = (ctypes.c_double * N_STAGES)()
        n = ctypes.c_int64()
        rc = self.lib.lsh_attn_get_timing(self.handle, ms, ctypes.byref(n))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_get_timing", self.lib)
        return {k: float(ms[j]) for j, k in enumerate(STAGES)}, int(n.value)

    def get_backward_timing(self):
        """(dict backward stage -> summed ms, number of timed backwards); resets
        the sums. Timing is enabled by set_timing (handles made with backward=True)."""
        ms = (ctypes.c_double * N_BWD_STAGES)()
        n = ctypes.c_int64()
        rc = self.lib.lsh_attn_get_backward_timing(self.handle, ms, ctypes.byref(n))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_get_backward_timing", self.lib)
        return {k: float(ms[j]) for j, k in enumerate(BWD_STAGES)}, int(n.value)

    def workspace_bytes(self) -> int:
        b = ctypes.c_int64()
        rc = self.lib.lsh_attn_workspace_bytes(self.handle, ctypes.byref(b))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_attn_workspace_bytes", self.lib)
        return int(b.value)

    def close(self):
        if self.handle:
            rc = self.lib.lsh_attn_destroy(self.handle)
            self.handle = ctypes.c_void_p()
            if rc != 0:
                raise LSHAttnError(rc, "lsh_attn_destroy", self.lib)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                self.lib.lsh_attn_destroy(self.handle)
                self.handle = ctypes.c_void_p()
        except Exception:
            pass


class ChunkedFeedForward:
    """The chunked feed-forward half of the reversible block, bound to a
    library handle (which holds one chunk's hidden rows on the device).

    Call with y1 [rows, d_model], w1 [d_ff, d_model], b1 [d_ff], w2
    [d_model, d_ff], b2 [d_model] and optionally the residual x2
    [rows, d_model], all contiguous in dtype on the handle's device, rows at
    most max_rows. Returns y2 = x2 + relu(y1 w1^T + b1) w2^T + b2 [rows, d_model],
    computed chunk_rows rows at a time (0: all rows at once).
    """

    def __init__(self, max_rows, d_model, d_ff, chunk_rows=0, dtype=torch.bfloat16, device=None):
        self.lib = load_library()
        self.cfg = FFNConfig(int(max_rows), int(chunk_rows), int(d_model), int(d_ff),
                             _dtype_code(dtype))
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None
                                   else torch.device(device).index or 0)
        self.handle = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = self.lib.lsh_ffn_create(ctypes.byref(self.cfg), ctypes.byref(self.handle))
        if rc != 0:
            self.handle = ctypes.c_void_p()
            raise LSHAttnError(rc, "lsh_ffn_create", self.lib)

    @property
    def dtype(self):
        return _TORCH[self.cfg.dtype]

    _check = LSHAttention._check

    def __call__(self, y1, w1, b1, w2, b2, x2=None, out=None, stream=None):
        c, dt = self.cfg, self.dtype
        if not isinstance(y1, torch.Tensor) or y1.dim() != 2:
            raise ValueError("y1 must be a 2-D tensor [rows, d_model]")
        rows = y1.shape[0]
        self._check("y1", y1, (rows, c.d_model), dt)
        self._check("w1", w1, (c.d_ff, c.d_model), dt)
        self._check("b1", b1, (c.d_ff,), dt)
        self._check("w2", w2, (c.d_model, c.d_ff), dt)
        self._check("b2", b2, (c.d_model,), dt)
        if x2 is not None:
            self._check("x2", x2, (rows, c.d_model), dt)
        if out is None:
            out = torch.empty((rows, c.d_model), dtype=dt, device=self.device)
        else:
            self._check("out", out, (rows, c.d_model), dt)
        s = (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream
        rc = self.lib.lsh_ffn_forward(self.handle, ctypes.c_int64(rows), y1.data_ptr(),
                                      w1.data_ptr(), b1.data_ptr(), w2.data_ptr(), b2.data_ptr(),
                                      None if x2 is None else x2.data_ptr(), out.data_ptr(), s)
        if rc != 0:
            raise LSHAttnError(rc, "lsh_ffn_forward", self.lib)
        return out

    def set_timing(self, capacity: int) -> None:
        """Record HIP events around every launch of the next `capacity` forwards."""
        rc = self.lib.lsh_ffn_set_timing(self.handle, int(capacity))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_ffn_set_timing", self.lib)

    def get_timing(self):
        """(dict stage -> summed ms, timed forwards, chunks in them); resets the sums."""
        ms = (ctypes.c_double * N_FFN_STAGES)()
        n, nc = ctypes.c_int64(), ctypes.c_int64()
        rc = self.lib.lsh_ffn_get_timing(self.handle, ms, ctypes.byref(n), ctypes.byref(nc))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_ffn_get_timing", self.lib)
        return {k: float(ms[j]) for j, k in enumerate(FFN_STAGES)}, int(n.value), int(nc.value)

    def workspace_bytes(self) -> int:
        b = ctypes.c_int64()
        rc = self.lib.lsh_ffn_workspace_bytes(self.handle, ctypes.byref(b))
        if rc != 0:
            raise LSHAttnError(rc, "lsh_ffn_workspace_bytes", self.lib)
        return int(b.value)

    def close(self):
        if self.handle:
            rc = self.lib.lsh_ffn_destroy(self.handle)
            self.handle = ctypes.c_void_p()
            if rc != 0:
                raise LSHAttnError(rc, "lsh_ffn_destroy", self.lib)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                self.lib.lsh_ffn_destroy(self.handle)
                self.handle = ctypes.c_void_p()
        except Exception:
            pass
