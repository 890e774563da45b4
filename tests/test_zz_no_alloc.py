"""lsh_attn_forward_static (no handle, no allocation: its workspace is the
library's static device scratch) against lsh_attn_forward through a handle,
through the C ABI, on two calls in a row, the second with a smaller input:
the same kernels run on the same inputs, so every output must be bitwise
equal (bucket ids, permutations, logsumexps, outputs). Each case prints what
it is before it runs."""
import sys

import numpy as np
import pytest
import torch

import workloads
import lsh_attention_hash_amd as lat
from parity import make_op, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lat.load_library()


def _outputs(w, dev):
    per_round = (w.batch, w.heads, w.n_rounds, w.seq_len)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return {"out": torch.empty((w.batch, w.heads, w.seq_len, w.head_dim), dtype=dt, device=dev),
            "lse": torch.empty(per_round, dtype=torch.float32, device=dev),
            "buckets": torch.empty(per_round, dtype=torch.int32, device=dev),
            "perm": torch.empty(per_round, dtype=torch.int32, device=dev)}


def _static(w, inp, dev):
    qk, v, rot = to_device(inp, dev)
    o = _outputs(w, dev)
    lat.forward_static(qk, v, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal,
                       out=o["out"], lse=o["lse"], buckets=o["buckets"], perm=o["perm"])
    torch.cuda.synchronize()
    return {k: t.cpu() for k, t in o.items()}


def _handle(w, inp, dev):
    qk, v, rot = to_device(inp, dev)
    op = make_op(w)
    try:
        out, ex = op(qk, v, rot, return_lse=True, return_buckets=True, return_perm=True)
        torch.cuda.synchronize()
        res = {"out": out.cpu(), **{k: ex[k].cpu() for k in ("lse", "buckets", "perm")}}
    finally:
        op.close()
    return res


def _same(a, b, what):
    for k in ("buckets", "perm", "lse", "out"):
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"{what}: {k} differs"


BIG = workloads.get("c4k").with_(batch=2, heads=4, seq_len=2048, n_buckets=32, n_rounds=3,
                                 causal=True)
SMALL = workloads.get("text64k").with_(batch=1, heads=2, seq_len=1024, n_buckets=16,
                                       n_rounds=2, causal=False)


def test_static_forward_equals_the_handle_forward_on_two_calls():
    dev = torch.device("cuda", 0)
    results = []
    for w in (BIG, SMALL):  # the second call's input is smaller
        _say(f"[static forward] {w}")
        inp = workloads.make_inputs(w)
        s = _static(w, inp, dev)
        results.append((w, inp, s))
    for w, inp, s in results:
        _same(s, _handle(w, inp, dev), f"{w.name} L={w.seq_len}")


def test_static_forward_fp32_and_full_c4k():
    """fp32 inputs (the plain kernels), then the largest workload that fits the
    scratch (batch 4, 8 heads, L 4096), then the small one again."""
    dev = torch.device("cuda", 0)
    for w in (workloads.get("tiny"), workloads.get("c4k"), SMALL):
        _say(f"[static forward] {w}")
        inp = workloads.make_inputs(w)
        _same(_static(w, inp, dev), _handle(w, inp, dev), f"{w.name} L={w.seq_len}")


def test_static_forward_rejects_a_workspace_beyond_the_scratch():
    w = workloads.get("image12k")
    dev = torch.device("cuda", 0)
    inp = workloads.make_inputs(w.with_(batch=1, heads=1))
    qk = torch.zeros((w.batch, w.heads, w.seq_len, w.head_dim), dtype=torch.bfloat16,
                     device=dev)
    rot = torch.from_numpy(inp.rotations).to(dev)
    with pytest.raises(lat.LSHAttnError) as e:
        lat.forward_static(qk, qk, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal)
    assert e.value.status == 5
