"""ctypes wrapper around the fp64 CPU oracle (lsh_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline may import this package. The product path never does.

Every array argument is converted to a contiguous float64 / int32 numpy array;
the library computes in float64 throughout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsh_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "liblsh_oracle.so")

SELF_LOGIT = -1.0e5


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "lsh_oracle.h"))):
        return _LIB
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "seq_len", "head_dim", "n_buckets", "n_rounds", "chunk_len",
        "causal", "variant")]


# variant bits (lsh_oracle.h): readings the pages also allow; 0 is the default
LOOK_AHEAD = 1
SAME_BUCKET = 2
NORM_QUERIES = 4
DEDUP = 8


_lib = None
_lib_path = None


def use_library(path: Optional[str] = None) -> None:
    """Switch to another build of lsh_oracle.c (the tests use this to check that
    the pins catch mistakes planted in a copy of the source). None restores the
    default build."""
    global _lib, _lib_path
    _lib = None
    _lib_path = path


def compile_source(src_text: str, out_path: str) -> str:
    """Compile C source text of the oracle (same flags as build()) to out_path."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fPIC", "-shared", "-I", _HERE, "-o", out_path, src,
                    "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _load():
    global _lib
    if _lib is None:
        if _lib_path is None:
            build(force=False)
        lib = ctypes.CDLL(_lib_path or _LIB)
        P = ctypes.c_void_p
        C = ctypes.POINTER(Config)
        for name, argt in {
            "lsh_oracle_check": [C],
            "lsh_oracle_hash": [C, P, P, P, P],
            "lsh_oracle_sort": [C, P, P, P],
            "lsh_oracle_attend": [C, P, P, P, P, P, P],
            "lsh_oracle_combine": [C, P, P, P],
            "lsh_oracle_forward": [C, P, P, P, P, P, P, P, P, P],
            "lsh_oracle_attend_rows": [C, P, P, P, P, ctypes.c_int64, P, P, P],
            "lsh_oracle_backward": [C, P, P, P, P, P, P, P],
            "lsh_oracle_backward_magnitudes": [C, P, P, P, P, P, P, P],
            "lsh_oracle_project": [C, ctypes.c_int64, P, P, P, P, P],
            "lsh_oracle_ffn": [ctypes.c_int64] * 4 + [P] * 8,
        }.items():
            f = getattr(lib, name)
            f.argtypes = argt
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def config(w=None, **kw) -> Config:
    """Config from a workloads.Workload (or any object with the same fields) and/or keywords."""
    names = ("batch", "heads", "seq_len", "head_dim", "n_buckets", "n_rounds", "chunk_len",
             "causal", "variant")
    vals = {"variant": 0}
    if w is not None:
        for n in names:
            if hasattr(w, n):
                vals[n] = int(getattr(w, n))
    vals.update({k: int(v) for k, v in kw.items()})
    return Config(**{n: vals[n] for n in names})


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _chk(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc}")


def _shapes(c: Config):
    return (c.batch, c.heads, c.n_rounds, c.seq_len)


def hash(c: Config, qk, rotations):
    """Bucket ids and margins [B, H, R, L]."""
    qk, rot = _f64(qk), _f64(rotations)
    bk = np.empty(_shapes(c), np.int32)
    mg = np.empty(_shapes(c), np.float64)
    _chk(_load().lsh_oracle_hash(ctypes.byref(c), _p(qk), _p(rot), _p(bk), _p(mg)), "hash")
    return bk, mg


def sort(c: Config, buckets):
    """perm (sorted slot -> position) and inv, [B, H, R, L]."""
    bk = _i32(buckets)
    pm = np.empty(_shapes(c), np.int32)
    iv = np.empty(_shapes(c), np.int32)
    _chk(_load().lsh_oracle_sort(ctypes.byref(c), _p(bk), _p(pm), _p(iv)), "sort")
    return pm, iv


def attend(c: Config, qk, v, perm, buckets=None):
    """Per-round outputs o [B, H, R, L, d] and logsumexp [B, H, R, L], original order.
    buckets [B, H, R, L] is needed with the SAME_BUCKET variant."""
    qk, v, pm, bk = _f64(qk), _f64(v), _i32(perm), _i32(buckets)
    o = np.empty(_shapes(c) + (c.head_dim,), np.float64)
    lse = np.empty(_shapes(c), np.float64)
    _chk(_load().lsh_oracle_attend(ctypes.byref(c), _p(qk), _p(v), _p(pm), _p(bk), _p(o),
                                   _p(lse)), "attend")
    return o, lse


def combine(c: Config, o, lse):
    o, lse = _f64(o), _f64(lse)
    out = np.empty((c.batch, c.heads, c.seq_len, c.head_dim), np.float64)
    _chk(_load().lsh_oracle_combine(ctypes.byref(c), _p(o), _p(lse), _p(out)), "combine")
    return out


def forward(c: Config, qk, v, rotations, buckets_override: Optional[np.ndarray] = None):
    """Whole forward; returns dict(out, lse, buckets, perm, margin)."""
    qk, v, rot, bo = _f64(qk), _f64(v), _f64(rotations), _i32(buckets_override)
    out = np.empty((c.batch, c.heads, c.seq_len, c.head_dim), np.float64)
    lse = np.empty(_shapes(c), np.float64)
    bk = np.empty(_shapes(c), np.int32)
    pm = np.empty(_shapes(c), np.int32)
    mg = np.full(_shapes(c), np.nan, np.float64)
    _chk(_load().lsh_oracle_forward(ctypes.byref(c), _p(qk), _p(v), _p(rot), _p(bo), _p(out),
                                    _p(lse), _p(bk), _p(pm), _p(mg)), "forward")
    return {"out": out, "lse": lse, "buckets": bk, "perm": pm, "margin": mg}


def attend_rows(c: Config, qk, v, perm, rows, buckets=None):
    """Combined output rows [n, d] and per-round lse [n, R] for rows = (b*H+h)*L+i
    (buckets as for attend)."""
    qk, v, pm, bk = _f64(qk), _f64(v), _i32(perm), _i32(buckets)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, c.head_dim), np.float64)
    lse = np.empty((rows.size, c.n_rounds), np.float64)
    _chk(_load().lsh_oracle_attend_rows(ctypes.byref(c), _p(qk), _p(v), _p(pm), _p(bk),
                                        ctypes.c_int64(rows.size), _p(rows), _p(out), _p(lse)),
         "attend_rows")
    return out, lse


def backward(c: Config, qk, v, perm, dout, buckets=None):
    """Gradients (dqk, dv) [B, H, L, d] of a loss given dout = dL/dout, at the
    permutations perm [B, H, R, L] of the forward (buckets held fixed; the
    forward's buckets [B, H, R, L] are needed with SAME_BUCKET)."""
    qk, v, pm, do, bk = _f64(qk), _f64(v), _i32(perm), _f64(dout), _i32(buckets)
    dqk = np.empty((c.batch, c.heads, c.seq_len, c.head_dim), np.float64)
    dv = np.empty_like(dqk)
    _chk(_load().lsh_oracle_backward(ctypes.byref(c), _p(qk), _p(v), _p(pm), _p(bk), _p(do),
                                     _p(dqk), _p(dv)), "backward")
    return dqk, dv


def backward_magnitudes(c: Config, qk, v, perm, dout, buckets=None):
    """(mdqk, mdv) [B, H, L, d]: sums of upper bounds of the absolute values of
    the terms of dqk and dv (|dqk| <= mdqk, |dv| <= mdv), for error bounds of
    a finite-precision backward (buckets as for backward)."""
    qk, v, pm, do, bk = _f64(qk), _f64(v), _i32(perm), _f64(dout), _i32(buckets)
    mq = np.empty((c.batch, c.heads, c.seq_len, c.head_dim), np.float64)
    mv = np.empty_like(mq)
    _chk(_load().lsh_oracle_backward_magnitudes(ctypes.byref(c), _p(qk), _p(v), _p(pm), _p(bk),
                                                _p(do), _p(mq), _p(mv)), "backward_magnitudes")
    return mq, mv


def ffn(y1, w1, b1, w2, b2, x2=None, chunk_rows=None, return_hidden=False):
    """Chunked feed-forward: y2 [rows, d_model] from y1 [rows, d_model], w1
    [d_ff, d_model], b1 [d_ff], w2 [d_model, d_ff], b2 [d_model] and the
    optional residual x2 [rows, d_model]; chunk_rows defaults to all rows.
    With return_hidden, also the ReLU activations [rows, d_ff]."""
    y1, w1, b1, w2, b2 = (_f64(a) for a in (y1, w1, b1, w2, b2))
    rows, d_model = y1.shape
    d_ff = w1.shape[0]
    if w1.shape != (d_ff, d_model) or w2.shape != (d_model, d_ff) or b1.shape != (d_ff,) \
            or b2.shape != (d_model,):
        raise ValueError("ffn: inconsistent shapes")
    x2p = None
    if x2 is not None:
        x2 = _f64(x2)
        if x2.shape != y1.shape:
            raise ValueError("ffn: x2 must match y1")
        x2p = _p(x2)
    y2 = np.empty((rows, d_model), np.float64)
    hid = np.empty((rows, d_ff), np.float64) if return_hidden else None
    _chk(_load().lsh_oracle_ffn(ctypes.c_int64(rows), ctypes.c_int64(d_model),
                                ctypes.c_int64(d_ff), ctypes.c_int64(chunk_rows or max(rows, 1)),
                                _p(y1), _p(w1), _p(b1), _p(w2), _p(b2), x2p, _p(y2),
                                None if hid is None else _p(hid)), "ffn")
    return (y2, hid) if return_hidden else y2


def project(c: Config, x, w_qk, w_v):
    """qk, v [B, H, L, d] from x [B, L, model_dim] and the weights [H*d, model_dim]."""
    x, wq, wv = _f64(x), _f64(w_qk), _f64(w_v)
    model_dim = x.shape[-1]
    qk = np.empty((c.batch, c.heads, c.seq_len, c.head_dim), np.float64)
    v = np.empty_like(qk)
    _chk(_load().lsh_oracle_project(ctypes.byref(c), ctypes.c_int64(model_dim), _p(x), _p(wq),
                                    _p(wv), _p(qk), _p(v)), "project")
    return qk, v
