"""A decode step captured as a HIP graph (torch.cuda.CUDAGraph on the current
stream) replays to the eager result bit for bit.

The library issues only kernel launches on the caller's stream during a step
(no allocation, memset or synchronisation), so the step can be captured; the
selection states, split counters and error word are reset by its own kernels.
Each replay follows eager work of the program (fills of the outputs, a
synchronisation) and is checked on its own.
"""

import pytest
import torch

from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup

pytestmark = pytest.mark.gpu

AUTO, MULTI, SINGLE = hws.HWS_LAUNCH_AUTO, hws.HWS_LAUNCH_MULTI, hws.HWS_LAUNCH_SINGLE


@pytest.mark.parametrize("cfg,kw,launch", [
    (1, dict(n=5000), AUTO), (1, dict(n=5000), SINGLE), (2, dict(n=6000, batch=3), AUTO),
    (3, dict(n=40000, batch=2), AUTO), (5, dict(n=20000, batch=4), MULTI),
    (4, dict(n=20000), AUTO), (5, dict(n=20000, batch=4), AUTO),
    (5, dict(n=20000, batch=4), hws.HWS_LAUNCH_SCAN_SELECT), (2, dict(n=6000, batch=3), hws.HWS_LAUNCH_SCAN_SINGLE),
], ids=["tiny-auto", "tiny-single", "layer-auto", "oracle-topk-fused", "ragged-fp8-multi", "long-auto",
        "ragged-fp8-auto", "ragged-fp8-scan-select", "layer-scan-single"])
def test_graph_replays_match_eager(cfg, kw, launch):
    wl = W.make_workload(cfg, **kw)
    print(f"\n[case] graph {wl.name} B={wl.B} N={wl.seq_lens[:4]} launch={launch}", flush=True)
    st = DecodeSetup(wl)
    st.ctx.set_launch_mode(launch)
    st.decode()
    torch.cuda.synchronize()
    ref = (st.out.clone(), st.lse.clone(), st.sel_counts.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.decode()
    for r in range(3):
        st.out.fill_(7.0)
        st.lse.fill_(7.0)
        st.sel_counts.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref[0]), f"replay {r}: out"
        assert torch.equal(st.lse, ref[1]), f"replay {r}: lse"
        assert torch.equal(st.sel_counts, ref[2]), f"replay {r}: sel_counts"
    # an eager step after the replays still gives the same result
    st.decode()
    torch.cuda.synchronize()
    assert torch.equal(st.out, ref[0]) and torch.equal(st.sel_counts, ref[2])
