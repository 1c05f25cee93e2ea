"""decode_step_noalloc — decode_step with its workspace in the library's own
device array, for callers that cannot allocate — against decode_step with a
caller workspace: two calls in a row on one GPU (the second with a smaller
batch, on the array the first one left behind) give the output and lse of
decode_step bit for bit, and stay within the attention tolerance of the
oracle. The refusal of steps larger than the array is a CPU test in
test_abi.py."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import step as OS
from tests import parity as PT

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_decode_mxfp4_amd as m
    m.lib()
    return m


def _make(mx, wl):
    import workloads.gpu as WG
    inp = W.make_inputs(wl)
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    cache = WG.make_cache(inp, pools)
    t = WG.step_tensors(inp)
    kw = dict(k_new=t.get("k_new"), v_new=t.get("v_new"), idx_new=t.get("idx_new"))
    ref = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, **kw)
    na = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, noalloc=True, **kw)
    assert na.ws is None
    return inp, ref, na


@pytest.mark.parametrize("name", ["mxfp4_65k", "fp8"])
def test_noalloc_two_calls_match_decode_step(mx, name):
    big = W.WORKLOADS[name]
    small = big.with_(B=2, ctx_rule=("list", (9000, 3001)) if name == "mxfp4_65k" else ("fixed", 4096))
    inp_a, ref_a, na_a = _make(mx, big)
    inp_b, ref_b, na_b = _make(mx, small)
    need = mx.workspace_bytes(big.B, big.q, big.H, big.H_I, big.topk, inp_a.max_pages)
    assert need <= mx.NOALLOC_SCRATCH_BYTES
    # two calls in a row on the library's array: the big step, then the small one
    na_a.run()
    na_b.run()
    torch.cuda.synchronize()
    got = [(na_a.out.clone(), na_a.lse.clone()), (na_b.out.clone(), na_b.lse.clone())]
    # the same steps through decode_step with caller workspaces
    ref_a.run()
    ref_b.run()
    torch.cuda.synchronize()
    for (o, l), r, what in zip(got, (ref_a, ref_b), ("first", "second")):
        assert torch.equal(o, r.out), f"{what} call: output differs from decode_step"
        assert torch.equal(l, r.lse), f"{what} call: lse differs from decode_step"
    # and within the attention tolerance of the oracle (one sequence of each)
    for inp, (o, _) in ((inp_a, got[0]), (inp_b, got[1])):
        r = OS.decode_step_ref(inp, seqs=[1])
        PT.check_attention(o.float().cpu().numpy()[1], r["O"][1], f"{inp.wl.name} noalloc b=1")
    # a third call on the big step again, after the small one: still identical
    na_a.run()
    torch.cuda.synchronize()
    assert torch.equal(na_a.out, ref_a.out) and torch.equal(na_a.lse, ref_a.lse)
