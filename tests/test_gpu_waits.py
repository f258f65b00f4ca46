"""GPU: the time-out path of the single launch's hand-off waits.

The host raises every wait's target past what can arrive (hws_set_wait_limit
with unreachable = 1) and shortens the bound to 256 polls, so each wait of the
step gives up after a few hundred microseconds: every kernel still exits,
the step's retrieval heads come out NaN, and the next step with the normal
limit is correct again.  The step's status word says which step gave up
(HWS_STEP_WAIT_TIMEOUT) and which did not.  Nothing here faults or hangs: each wait is bounded
by the poll limit whatever the counters hold.
"""

import numpy as np
import pytest
import torch

from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup
from gpu_check import check_decode

pytestmark = pytest.mark.gpu

CASES = {
    # (workload, AUTO's single launch, whether the per-stage attention follows)
    "fused_128k_shape": (lambda: W.make_workload(3, n=32768, batch=1), "fused", False),
    "fused_cooperative": (lambda: W.make_workload(3, n=32768, batch=1), "fused", False),
    "fused_index_8k": (lambda: W.make_workload(2, n=8192, batch=2), "fused_index", False),
    "fused_index_cooperative": (lambda: W.make_workload(1), "fused_index", False),
    "tail_4k": (lambda: W.make_workload(1, Hq=4, Hkv=2, score_mode="full"), "tail", False),
    "select_then_attend_8k": (lambda: W.make_workload(1, n=8192, Hq=4, Hkv=2, score_mode="full", batch=2),
                              "select", True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_waits_that_cannot_finish_end_with_nan_and_recover(case):
    make, stage, per_stage_after = CASES[case]
    wl = make()
    print(f"\n[case] {case}: {wl.name} B={wl.B} N={wl.seq_lens[0]}", flush=True)
    st = DecodeSetup(wl, keep_host=True)
    if case.endswith("cooperative"):
        st.ctx.set_launch_mode(hws.HWS_LAUNCH_COOPERATIVE)

    st.ctx.set_wait_limit(256, unreachable=True)
    st.ctx.profile_enable(True)
    bad = st.decode(debug=True)                       # returns after a device sync
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof[stage][1] == 1, prof                  # the launch that waits ran
    assert bad["status"] == hws.HWS_STEP_WAIT_TIMEOUT, bad["status"]   # visible to the caller
    G = wl.G
    for h in wl.retrieval_heads:
        assert np.isnan(bad["out"][:, h * G:(h + 1) * G]).all(), f"head {h} not NaN"
        assert np.isnan(bad["lse"][:, h * G:(h + 1) * G]).all(), f"head {h} lse not NaN"
    if per_stage_after:
        assert np.isnan(bad["out"]).all() and np.isnan(bad["lse"]).all()

    st.ctx.set_wait_limit(0, unreachable=False)
    good = st.decode(debug=True)
    assert good["status"] == hws.HWS_STEP_OK
    check_decode(st, good, verbose=False)
    torch.cuda.synchronize()
