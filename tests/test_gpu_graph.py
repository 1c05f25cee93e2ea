"""The decode steps under HIP graph capture (ATOM PR #2812: the Mono decode
path runs in eager mode and under CUDA/HIP graphs, with the addresses a graph
captured kept stable).

A captured step is replayed several times, with eager work of the program's
own (other steps on other buffers) and synchronizations between replays;
every replay must equal the eager run of the same step bit for bit, and the
eager result is checked against the oracle once.
"""
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


def _setup(name):
    import workloads.gpu as WG
    if name == "one_launch":       # 4 x 2048-entry page tables, through decode_step_one_launch
        wl = W.WORKLOADS["mxfp4_65k"].with_(name="one_launch", table_stride=2048)
    else:
        wl = W.WORKLOADS[name].with_(B=4)
    inp = W.make_inputs(wl)
    pools = WG.fill_prefix(inp, WG.empty_pools(inp))
    return inp, WG.make_cache(inp, pools), WG.step_tensors(inp)


@pytest.mark.parametrize("name", ["mxfp4_65k", "fp8", "nvfp4", "one_launch"])
def test_decode_step_graph_replays_equal_eager(mx, name):
    inp, cache, t = _setup(name)
    wl = inp.wl
    kw = dict(k_new=t.get("k_new"), v_new=t.get("v_new"), idx_new=t.get("idx_new"))
    kw["one_launch"] = name == "one_launch"
    step = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, **kw)
    other_q = (t["query"].float() * 0.5 - 0.25).to(t["query"].dtype).contiguous()
    other = mx.DecodeStep(cache, other_q, t["q_idx"], t["w"], wl.topk, wl.sm_scale, **kw)
    step.run()
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    other.run()
    torch.cuda.synchronize()
    other0 = other.out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for i in range(5):
        step.out.zero_()
        step.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, out0) and torch.equal(step.lse, lse0), f"replay {i}"
        other.run()                                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other.out, other0), f"eager run after replay {i}"
    r = OS.decode_step_ref(inp, seqs=[0])
    PT.check_attention(out0.float().cpu().numpy()[0], r["O"][0], f"{name} graph b=0")


@pytest.mark.parametrize("one_launch", [False, True])
def test_reuse_step_graph_replays_equal_eager(mx, one_launch):
    inp, cache, t = _setup("mxfp4_65k")
    wl = inp.wl
    full = mx.DecodeStep(cache, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                         v_new=t.get("v_new"), idx_new=t.get("idx_new"),
                         block_table_out=torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda"))
    full.run()
    torch.cuda.synchronize()
    table = full.block_table_out.clone()
    step = mx.DecodeStepReuse(cache, t["query"], table, wl.sm_scale, k_new=t.get("k_new"), v_new=t.get("v_new"),
                              one_launch=one_launch)
    step.run()
    torch.cuda.synchronize()
    out0, lse0 = step.out.clone(), step.lse.clone()
    assert torch.equal(out0, full.out)               # the reuse step over the step's own selection

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for i in range(5):
        step.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, out0) and torch.equal(step.lse, lse0), f"replay {i}"
        full.run()                                   # eager work between replays
        torch.cuda.synchronize()
    assert np.isfinite(out0.float().cpu().numpy()).all()
