"""Parity helpers: run the HIP path through the C ABI and compare it with the
fp64 oracle on the same seeded inputs.

Comparison protocol
  * bucket ids: equal to the oracle's everywhere. The GPU certifies each
    decision of its fp16 projection with an error bound and re-scores every
    row it cannot certify in fp64 with the oracle's own summation order (the
    products of a bf16 or fp32 input and an fp32 rotation are exact in fp64),
    so even the near-ties (oracle top-two margin below TIE_MARGIN, the band
    within which the benchmark spec's tolerance would let them differ) must agree;
    the near-ties are counted and reported;
  * perm: bit-exact, the oracle's own stable sort of its own buckets;
  * outputs: max-abs error within OUT_TOL times the scale of v (the outputs
    are convex combinations of v rows, so errors scale with v);
  * logsumexps: compared on rounds that saw more than the query itself,
    within lse_tol (below); the self-only flag (lse == -1e5) must agree
    exactly.

lse tolerance, derived from the kernels' arithmetic: the logit of key j for
query i is (q_i . k_j) times log2(e) / (sqrt(d) |k_j|), the dot product of
bf16 values summed in fp32 (error at most d 2^-24 sum_t |q_t k_t| <=
d 2^-24 |q| |k|), the key scale from an fp32 norm (a few ulp), so every
logit, hence the logsumexp, is off by at most (d + 8) 2^-24 |q_i| / sqrt(d);
the exp2/log2 and the fp32 sum of at most 3 m terms add far less than the
1e-4 (bf16 inputs) or 1e-5 (fp32) floor kept from the proposed diagnostic
bound. For N(0, 1) rows the derived term is ~1e-5 at d = 128; it matters for
rows scaled far beyond that (large-magnitude cases).
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
            fp32_round_outputs=False, **kw):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return lat.LSHAttention(w.batch, w.heads, w.seq_len, w.head_dim, w.n_buckets, w.n_rounds,
                            w.chunk_len, w.causal, dtype=dt, out_dtype=out_dtype,
                            separate_gather=separate_gather,
                            fp32_round_outputs=fp32_round_outputs, **kw)


def run_gpu(w, inp, out_dtype=None, separate_gather=False, fp32_round_outputs=False, **kw):
    op = make_op(w, out_dtype, separate_gather, fp32_round_outputs, **kw)
    qk, v, rot = to_device(inp)
    out, ex = op(qk, v, rot, return_lse=True, return_buckets=True, return_perm=True)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy().astype(np.float64),
           "lse": ex["lse"].cpu().numpy(), "buckets": ex["buckets"].cpu().numpy(),
           "perm": ex["perm"].cpu().numpy(), "stats": op.stats()}
    op.close()
    return res


def compare_buckets(ref_buckets, ref_margin, gpu_buckets, where=""):
    """Bucket ids equal everywhere; returns (n_compared, n_ties). The ties
    (oracle margin < TIE_MARGIN) are reported and must agree too."""
    tie = ref_margin < TIE_MARGIN
    mis = ref_buckets != gpu_buckets
    if np.any(mis):
        idx = np.argwhere(mis)[:5]
        raise AssertionError(
            f"bucket ids differ from the oracle{where}: {int(mis.sum())} rows "
            f"({int((mis & tie).sum())} of them near-ties), first at [b, h, r, i] = "
            f"{idx.tolist()}, margins {ref_margin[mis][:5]}")
    return int(ref_buckets.size), int(tie.sum())


def check_buckets(w, inp, gpu_buckets, bh_sel=None):
    """Compare bucket ids on the (b, h) pairs in bh_sel (all if None) with the
    oracle's hash. Returns (n_checked, n_ties, 0); asserts equality everywhere."""
    if w.n_buckets == 1:
        assert np.all(gpu_buckets == 0)
        return gpu_buckets.size, 0, 0
    B, H = w.batch, w.heads
    if bh_sel is None:
        c = oracle.config(w)
        bk, mg = oracle.hash(c, inp.qk, inp.rotations)
        n, ties = compare_buckets(bk, mg, gpu_buckets)
        return n, ties, 0
    n_chk = n_ties = 0
    for b, h in bh_sel:
        c = oracle.config(w, batch=1, heads=1)
        bk, mg = oracle.hash(c, inp.qk[b:b + 1, h:h + 1], inp.rotations)
        n, ties = compare_buckets(bk, mg, gpu_buckets[b:b + 1, h:h + 1], f" at (b={b}, h={h})")
        n_chk += n
        n_ties += ties
    return n_chk, n_ties, 0


def check_perm(w, gpu_buckets, gpu_perm):
    c = oracle.config(w)
    pm, _ = oracle.sort(c, gpu_buckets)
    np.testing.assert_array_equal(gpu_perm, pm)


def lse_tol(w, qk):
    """Per token-head logsumexp tolerance [B, H, 1, L] (module docstring)."""
    d = w.head_dim
    qn = np.sqrt(np.sum(np.asarray(qk, dtype=np.float64) ** 2, axis=-1))
    return (LSE_TOL[w.dtype] + (d + 8) * 2.0 ** -24 * qn / np.sqrt(d))[:, :, None, :]


def _cmp_lse(w, got, want, tol=None):
    self_g = got == np.float32(oracle.SELF_LOGIT)
    self_w = want == oracle.SELF_LOGIT
    np.testing.assert_array_equal(self_g, self_w)
    if tol is None:
        tol = LSE_TOL[w.dtype]
    tol = np.broadcast_to(tol, want.shape)
    if np.any(~self_w):
        err = np.abs(got.astype(np.float64) - want)
        bad = (err > tol) & ~self_w
        assert not np.any(bad), (f"lse error {err[bad].max()} over its bound "
                                 f"{tol[bad][np.argmax(err[bad])]} at {int(bad.sum())} entries")
        return float(err[~self_w].max())
    return 0.0


def out_tol(w, inp, v_scale=1.0, scaled_qk=False):
    """Output tolerance: OUT_TOL times the scale of v. For qk rows scaled far
    beyond the workloads' unit-variance rows (scaled_qk), the logit error
    bound of lse_tol, dl = (d + 8) 2^-24 max|q| / sqrt(d), moves every softmax
    weight by a factor within exp(+-2 dl), so the output by at most
    ~2 dl max|v| more; that term is added (it is what limits fp32 there)."""
    tol = OUT_TOL[w.dtype] * v_scale
    if scaled_qk:
        d = w.head_dim
        qn = float(np.sqrt(np.max(np.sum(np.asarray(inp.qk, np.float64) ** 2, axis=-1))))
        dl = (d + 8) * 2.0 ** -24 * qn / np.sqrt(d)
        tol += 2.0 * dl * float(np.max(np.abs(inp.v))) * 1.01
    return tol


def check_forward(w, inp, gpu, v_scale=1.0, variant=0, ref=None, scaled_qk=False):
    """The whole forward against the oracle's own (its hash, sort, attention
    and combination): buckets and perm bit-exact everywhere, every output
    element within out_tol, every lse within lse_tol. Returns a dict of the
    figures (ties, errors)."""
    c = oracle.config(w, variant=variant)
    if ref is None:
        ref = oracle.forward(c, inp.qk, inp.v, inp.rotations)
    n, ties = compare_buckets(ref["buckets"], ref["margin"], gpu["buckets"])
    np.testing.assert_array_equal(gpu["perm"], ref["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    emax = float(err.max()) if err.size else 0.0
    tol = out_tol(w, inp, v_scale, scaled_qk)
    assert emax <= tol, f"out max err {emax} > {tol}"
    lerr = _cmp_lse(w, gpu["lse"], ref["lse"], lse_tol(w, inp.qk))
    return {"buckets": n, "ties": ties, "out_err": emax, "lse_err": lerr}


def check_outputs_full(w, inp, gpu, v_scale=1.0):
    """Outputs and lse over every element against the oracle run on the GPU's
    buckets (used where the buckets were compared separately)."""
    c = oracle.config(w)
    ref = oracle.forward(c, inp.qk, inp.v, inp.rotations, buckets_override=gpu["buckets"])
    np.testing.assert_array_equal(ref["perm"], gpu["perm"])
    err = np.abs(gpu["out"] - ref["out"])
    assert err.max() <= OUT_TOL[w.dtype] * v_scale, f"out max err {err.max()}"
    lse_err = _cmp_lse(w, gpu["lse"], ref["lse"], lse_tol(w, inp.qk))
    return float(err.max()), lse_err


def sample_rows(w, per_head=64, seed=0):
    """Row indices (b*H + h)*L + i: per_head positions of every (b, h), the
    first and last position and the ends of the first and last chunk among
    them, the rest drawn uniformly."""
    rng = np.random.default_rng(seed)
    L, m = w.seq_len, w.chunk_len
    fixed = np.unique(np.array([0, m - 1, m, L - m, L - 1]).clip(0, L - 1))
    rows = []
    for bh in range(w.batch * w.heads):
        k = max(per_head - fixed.size, 0)
        pos = np.unique(np.concatenate([fixed, rng.choice(L, size=min(k, L), replace=False)]))
        rows.append(bh * L + pos)
    return np.concatenate(rows)


def check_outputs_rows(w, inp, gpu, per_head=64, seed=0, variant=0):
    """Sampled output rows of every (b, h) (sample_rows) against the oracle's
    single-row attention at the GPU's permutation."""
    rows = sample_rows(w, per_head, seed)
    N = w.batch * w.heads * w.seq_len
    c = oracle.config(w, variant=variant)
    out_r, lse_r = oracle.attend_rows(c, inp.qk, inp.v, gpu["perm"], rows,
                                      gpu["buckets"] if variant else None)
    got = gpu["out"].reshape(N, w.head_dim)[rows]
    err = np.abs(got - out_r)
    assert err.max() <= OUT_TOL[w.dtype], f"out max err {err.max()}"
    bh, i = rows // w.seq_len, rows % w.seq_len
    lse_g = gpu["lse"].reshape(w.batch * w.heads, w.n_rounds, w.seq_len)[bh, :, i]
    tol = lse_tol(w, inp.qk).reshape(w.batch * w.heads, w.seq_len)[bh, i][:, None]
    lse_err = _cmp_lse(w, lse_g, lse_r, tol)
    return float(err.max()), lse_err


def scaled_inputs(inp: workloads.Inputs, qk_exp: int = 0, v_exp: int = 0) -> workloads.Inputs:
    """The same inputs with qk multiplied by 2^qk_exp and v by 2^v_exp: exact
    in bf16 and fp32 (an exponent shift) while the values stay in range."""
    w = inp.workload

    def sc(x, bits, e):
        y = (x * np.float32(2.0 ** e)).astype(np.float32)
        assert np.all(np.isfinite(y))
        if w.dtype == "bf16":
            b = workloads.f32_to_bf16_bits(y)
            assert np.array_equal(workloads.bf16_bits_to_f32(b), y)
            return y, b
        return y, None

    qk, qb = sc(inp.qk, inp.qk_bits, qk_exp)
    v, vb = sc(inp.v, inp.v_bits, v_exp)
    return workloads.Inputs(w, qk, v, inp.rotations, qb, vb)
