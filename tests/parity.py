"""Parity helpers: run the HIP path through the C ABI and compare it with the
fp64 oracle on the same seeded inputs.

Comparison protocol
  * bucket ids: equal to the oracle's everywhere except where the oracle's
    top-two margin is below TIE_MARGIN (such near-ties are counted);
  * perm: the oracle's stable sort of the GPU's bucket ids, bit-exact;
  * outputs and logsumexps: the oracle run on the GPU's bucket ids (one
    flipped near-tie re-chunks whole buckets, so outputs are only comparable
    under identical buckets), max-abs error within OUT_TOL; lse compared on
    rounds that saw more than the query itself, and the self-only flag
    (lse == -1e5) must agree exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
import lsh_attention_hash_amd as lat

TIE_MARGIN = 1e-5
OUT_TOL = {"bf16": 2e-2, "fp32": 1e-5}
LSE_TOL = {"bf16": 1e-4, "fp32": 1e-5}


def to_device(inp: workloads.Inputs, device="cuda"):
    w = inp.workload
    if w.dtype == "bf16":
        qk = torch.from_numpy(inp.qk_bits.view(np.int16)).to(device).view(torch.bfloat16)
        v = torch.from_numpy(inp.v_bits.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        qk = torch.from_numpy(inp.qk).to(device)
        v = torch.from_numpy(inp.v).to(device)
    rot = None if inp.rotations is None else torch.from_numpy(inp.rotations).to(device)
    return qk, v, rot


def make_op(w: workloads.Workload, out_dtype=None, separate_gather=False,
            fp32_round_outputs=False):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                            w.chunk_len, w.causal, dtype=dt, out_dtype=out_dtype,
                            separate_gather=separate_gather,
                            fp32_round_outputs=fp32_round_outputs)


def run_gpu(w, inp, out_dtype=None, separate_gather=False, fp32_round_outputs=False):
    op = make_op(w, out_dtype, separate_gather, fp32_round_outputs)
    qk, v, rot = to_device(inp)
    out, ex = op(qk, v, rot, return_lse=True, return_buckets=True, return_perm=True)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy().astype(np.float64),
           "lse": ex["lse"].cpu().numpy(), "buckets": ex["buckets"].cpu().numpy(),
           "perm": ex["perm"].cpu().numpy(), "stats": op.stats()}
    op.close()
    return res


def check_buckets(w, inp, gpu_buckets, bh_sel=None):
    """Compare bucket ids on the (b, h) pairs in bh_sel (all if None).
    Returns (n_checked, n_ties, n_tie_mismatch); asserts no mismatch outside ties."""
    if w.n_buckets == 1:
        assert np.all(gpu_buckets == 0)
        return gpu_buckets.size, 0, 0
    B, H = w.batch, w.heads
    sel = [(b, h) for b in range(B) for h in range(H)] if bh_sel is None else bh_sel
    n_chk = n_ties = n_tie_mis = 0
    for b, h in sel:
        c = oracle.config(w, batch=1, heads=1)
        bk, mg = oracle.hash(c, inp.qk[b:b + 1, h:h + 1], inp.rotations)
        g = gpu_buckets[b:b + 1, h:h + 1]
        tie = mg < TIE_MARGIN
        mis = bk != g
        assert not np.any(mis & ~tie), (
            f"bucket mismatch outside the tie band at (b={b}, h={h}): "
            f"{int(np.sum(mis & ~tie))} rows, margins {mg[mis & ~tie][:5]}")
        n_chk += bk.size
        n_ties += int(tie.sum())
        n_tie_mis += int((mis & tie).sum())
    return n_chk, n_ties, n_tie_mis


def check_perm(w, gpu_buckets, gpu_perm):
    c = oracle.config(w)
    pm, _ = oracle.sort(c, gpu_buckets)
    np.testing.assert_array_equal(gpu_perm, pm)


def _cmp_lse(w, got, want):
    self_g = got == np.float32(oracle.SELF_LOGIT)
    self_w = want == oracle.SELF_LOGIT
    np.testing.assert_array_equal(self_g, self_w)
    if np.any(~self_w):
        err = np.abs(got[~self_w].astype(np.float64) - want[~self_w])
        assert err.max() <= LSE_TOL[w.dtype], f"lse max err {err.max()}"
        return float(err.max())
    return 0.0


def check_outputs_full(w, inp, gpu):
    c = oracle.config(w)
    ref = oracle.forward(c, inp.qk, inp.v, inp.rotations, buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(ref["perm"], gpu["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    assert err.max() <= OUT_TOL[w.dtype], f"out max err {err.max()}"
    lse_err = _cmp_lse(w, gpu["lse"], ref["lse"])
    return float(err.max()), lse_err


def check_outputs_rows(w, inp, gpu, n_rows=2048, seed=0):
    rng = np.random.default_rng(seed)
    N = w.batch * w.heads * w.seq_len
    rows = np.unique(np.concatenate([
        rng.choice(N, size=min(n_rows, N), replace=False),
        np.array([0, w.seq_len - 1, N - 1, N - w.seq_len])]))
    c = oracle.config(w)
    out_r, lse_r = oracle.attend_rows(c, inp.qk, inp.v, gpu["perm"], rows)
    got = gpu["out"].reshape(N, w.head_dim)[rows]
    err = np.abs(got - out_r)
    assert err.max() <= OUT_TOL[w.dtype], f"out max err {err.max()}"
    bh, i = rows // w.seq_len, rows % w.seq_len
    lse_g = gpu["lse"].reshape(w.batch * w.heads, w.n_rounds, w.seq_len)[bh, :, i]
    lse_err = _cmp_lse(w, lse_g, lse_r)
    return float(err.max()), lse_err
