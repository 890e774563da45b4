"""A seeded sweep over small random configurations, the forward and the
backward of each against the oracle, through the C ABI: sequence lengths of
1 to 40 chunks, even bucket counts up to 128, 1 to 5 rounds, d = 64 and 128,
causal or not, batch and heads of 1 or 2, bf16 and fp32, and the variant
readings in random combination. The list comes from a fixed seed, so every
run (and every test id) is the same.

Forward: bucket ids equal to the oracle's hash everywhere (near-ties
included), the permutation equal to the oracle's stable sort, outputs within
the bf16 (2e-2) or fp32 (1e-5) tolerance and the logsumexps within
parity.lse_tol, against the oracle's forward of the reading. Backward: dqk
and dv against the oracle's backward at the GPU forward's permutation, within
the bound of the path that runs (test_gpu_backward derives each).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import _cmp_lse, check_buckets, lse_tol, run_gpu
from test_gpu_backward import _VFLAGS, _variant_backward_check

pytestmark = pytest.mark.gpu

_READINGS = ("look_ahead", "same_bucket", "norm_queries", "dedup")
_OUT_TOL = {"bf16": 2e-2, "fp32": 1e-5}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _configs(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        w = workloads.get("text64k" if d == 128 else "c4k").with_(
            batch=int(rng.integers(1, 3)), heads=int(rng.integers(1, 3)),
            seq_len=64 * int(rng.integers(1, 41)), n_buckets=2 * int(rng.integers(1, 65)),
            n_rounds=int(rng.integers(1, 6)), causal=bool(rng.integers(0, 2)),
            dtype="fp32" if rng.random() < 0.15 else "bf16")
        kw = {}
        if rng.random() < 0.6:
            kw = {k: True for k in _READINGS if rng.integers(0, 2)}
        out.append((w, kw))
    return out


CASES = _configs()
IDS = [f"{i}-{w.dtype}-B{w.batch}H{w.heads}L{w.seq_len}d{w.head_dim}nb{w.n_buckets}"
       f"R{w.n_rounds}{'c' if w.causal else 'n'}-" + ("+".join(kw) or "default")
       for i, (w, kw) in enumerate(CASES)]


@pytest.mark.parametrize("w,kw", CASES, ids=IDS)
def test_sweep_forward(w, kw):
    _say(f"[sweep forward] {w} {sorted(kw)}")
    inp = workloads.make_inputs(w)
    gpu = run_gpu(w, inp, **kw)
    check_buckets(w, inp, gpu["buckets"])
    variant = sum(_VFLAGS[k] for k in kw)
    ref = oracle.forward(oracle.config(w, variant=variant), inp.qk, inp.v, inp.rotations,
                         buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(gpu["perm"], ref["perm"])
    err = float(np.abs(gpu["out"] - ref["out"]).max())
    _say(f"  out max err {err:.3g}")
    assert err <= _OUT_TOL[w.dtype], f"out max err {err}"
    _cmp_lse(w, gpu["lse"], ref["lse"], lse_tol(w, inp.qk))


@pytest.mark.parametrize("w,kw", CASES, ids=IDS)
def test_sweep_backward(w, kw):
    _say(f"[sweep backward] {w} {sorted(kw)}")
    _variant_backward_check(w, kw, workloads.make_inputs(w))
