"""Seeded synthetic inputs for shared-QK LSH attention.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic (no hashing, sorting or attention),
so that both the HIP path and the fp64 oracle can take their inputs from it
without sharing any computation.

Shapes follow the workloads the pages describe: 64K-token text and 12K-token
images (64x64x3 pixels flattened) from the experiments section of the Reformer
summary at p2.ttnews.xyz, plus a clustered-key case that skews bucket sizes.
The datasets themselves (enwik8-64K, imagenet64) are not used; i.i.d. or
clustered Gaussian vectors of the same shapes stand in for trained activations.

Recipe (all streams are numpy ``Generator(PCG64(seed))``):
  * qk  ~ N(0, 1) float32, seed ``seed_base + 1000``; for the clustered kind
    qk_i = c_{z_i} + sigma * eps_i with 8 unit-norm centres c (seed
    ``seed_base + 4000``; centres ~ N(0, I) then normalised, z_i uniform).
  * v   ~ N(0, 1) float32, seed ``seed_base + 2000``.
  * rotations R ~ N(0, 1) float32 of shape [n_rounds, head_dim, n_buckets/2],
    seed ``seed_base + 3000``.
  * layer inputs (the projections' case): x ~ N(0, 1) [B, L, model_dim], seed
    ``seed_base + 5000``; the weights w_qk, w_v ~ N(0, 1/model_dim)
    [H * head_dim, model_dim], seeds ``seed_base + 6000`` and ``+ 7000`` (so
    qk and v come out with unit variance, as the direct inputs above).
  * bf16 storage: float32 rounded to bfloat16 with round-to-nearest-even.
The oracle receives exactly the stored values, widened to float64.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "make_inputs", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "Inputs", "LayerInputs", "make_layer_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    dtype: str          # "fp32" or "bf16": storage type of qk, v and out
    n_buckets: int
    n_rounds: int
    chunk_len: int
    causal: bool
    kind: str = "normal"  # "normal" or "clustered"
    seed_base: int = 0

    @property
    def n_token_heads(self) -> int:
        return self.batch * self.heads * self.seq_len

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads. seed_base k gives seeds 1000+k (qk), 2000+k (v),
# 3000+k (rotations), 4000+k (cluster centres and labels).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1024, 64, "fp32", 16, 1, 64, False, "normal", 0),
    "c4k": Workload("c4k", 4, 8, 4096, 64, "bf16", 64, 2, 64, True, "normal", 1),
    "text64k": Workload("text64k", 1, 8, 65536, 128, "bf16", 1024, 4, 64, True, "normal", 2),
    "image12k": Workload("image12k", 8, 8, 12288, 64, "bf16", 192, 8, 64, True, "normal", 3),
    "skewed": Workload("skewed", 2, 8, 32768, 64, "bf16", 512, 8, 64, False, "clustered", 4),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Finite inputs only (the generators never produce NaN or Inf).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Stored inputs. ``qk``/``v`` are float32 arrays holding exactly the stored
    values (bf16-representable when dtype is bf16); ``qk_bits``/``v_bits`` are
    the uint16 bf16 bit patterns (None for fp32). ``rotations`` is float32."""
    workload: Workload
    qk: np.ndarray
    v: np.ndarray
    rotations: Optional[np.ndarray]
    qk_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None


def _store(x: np.ndarray, dtype: str):
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32), None
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, sigma: float = 0.1, n_centres: int = 8) -> Inputs:
    """Draw the seeded inputs of workload ``w``."""
    B, H, L, d = w.batch, w.heads, w.seq_len, w.head_dim
    k = w.seed_base
    rng_qk = np.random.Generator(np.random.PCG64(1000 + k))
    rng_v = np.random.Generator(np.random.PCG64(2000 + k))
    rng_r = np.random.Generator(np.random.PCG64(3000 + k))
    if w.kind == "normal":
        qk = rng_qk.standard_normal((B, H, L, d), dtype=np.float32)
    elif w.kind == "clustered":
        rng_c = np.random.Generator(np.random.PCG64(4000 + k))
        centres = rng_c.standard_normal((n_centres, d), dtype=np.float32)
        centres /= np.linalg.norm(centres, axis=1, keepdims=True)
        labels = rng_c.integers(0, n_centres, size=(B, H, L))
        eps = rng_qk.standard_normal((B, H, L, d), dtype=np.float32)
        qk = centres[labels] + np.float32(sigma) * eps
        del eps
    else:
        raise ValueError(f"unknown kind {w.kind!r}")
    v = rng_v.standard_normal((B, H, L, d), dtype=np.float32)
    rot = None
    if w.n_buckets >= 2:
        rot = rng_r.standard_normal((w.n_rounds, d, w.n_buckets // 2), dtype=np.float32)
    qk_s, qk_bits = _store(qk, w.dtype)
    del qk
    v_s, v_bits = _store(v, w.dtype)
    del v
    return Inputs(w, qk_s, v_s, rot, qk_bits, v_bits)


@dataclasses.dataclass
class LayerInputs:
    """A layer input and the two projection weights, stored as for Inputs."""
    workload: Workload
    model_dim: int
    x: np.ndarray
    w_qk: np.ndarray
    w_v: np.ndarray
    rotations: Optional[np.ndarray]
    x_bits: Optional[np.ndarray] = None
    w_qk_bits: Optional[np.ndarray] = None
    w_v_bits: Optional[np.ndarray] = None


def make_layer_inputs(w: Workload, model_dim: int) -> LayerInputs:
    """Draw x [B, L, model_dim] and the weights [H * d, model_dim] of workload ``w``
    (the rotations are those of make_inputs)."""
    k = w.seed_base
    B, L, F = w.batch, w.seq_len, w.heads * w.head_dim
    x = np.random.Generator(np.random.PCG64(5000 + k)).standard_normal(
        (B, L, model_dim), dtype=np.float32)
    scale = np.float32(1.0 / np.sqrt(model_dim))
    wq = np.random.Generator(np.random.PCG64(6000 + k)).standard_normal(
        (F, model_dim), dtype=np.float32) * scale
    wv = np.random.Generator(np.random.PCG64(7000 + k)).standard_normal(
        (F, model_dim), dtype=np.float32) * scale
    rot = None
    if w.n_buckets >= 2:
        rot = np.random.Generator(np.random.PCG64(3000 + k)).standard_normal(
            (w.n_rounds, w.head_dim, w.n_buckets // 2), dtype=np.float32)
    x_s, x_bits = _store(x, w.dtype)
    wq_s, wq_bits = _store(wq, w.dtype)
    wv_s, wv_bits = _store(wv, w.dtype)
    return LayerInputs(w, model_dim, x_s, wq_s, wv_s, rot, x_bits, wq_bits, wv_bits)


@dataclasses.dataclass
class FFNInputs:
    """Stored inputs of the chunked feed-forward: float32 arrays holding the
    stored values (bf16-representable for bf16) and, for bf16, the uint16 bit
    patterns in ``bits`` (name -> array)."""
    rows: int
    d_model: int
    d_ff: int
    dtype: str
    y1: np.ndarray
    w1: np.ndarray
    b1: np.ndarray
    w2: np.ndarray
    b2: np.ndarray
    x2: np.ndarray
    bits: dict


def make_ffn_inputs(rows: int, d_model: int, d_ff: int, dtype: str = "bf16",
                    seed: int = 0) -> FFNInputs:
    """Draw y1 and x2 [rows, d_model] standard normal (the two halves of the
    reversible block's input), w1 [d_ff, d_model] and w2 [d_model, d_ff]
    normal with variance 1 / fan_in, and biases b1 [d_ff], b2 [d_model]
    normal with standard deviation 0.1; seeds 8000 + 100 j + seed."""
    def draw(j, shape, scale=1.0):
        a = np.random.Generator(np.random.PCG64(8000 + 100 * j + seed)).standard_normal(
            shape, dtype=np.float32)
        return a * np.float32(scale) if scale != 1.0 else a
    arrays = {"y1": draw(0, (rows, d_model)),
              "w1": draw(1, (d_ff, d_model), 1.0 / np.sqrt(d_model)),
              "b1": draw(2, (d_ff,), 0.1),
              "w2": draw(3, (d_model, d_ff), 1.0 / np.sqrt(d_ff)),
              "b2": draw(4, (d_model,), 0.1),
              "x2": draw(5, (rows, d_model))}
    stored, bits = {}, {}
    for k, a in arrays.items():
        stored[k], bits[k] = _store(a, dtype)
    return FFNInputs(rows, d_model, d_ff, dtype, bits=bits, **stored)
