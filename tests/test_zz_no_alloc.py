"""GPU: hws_decode_noalloc, the decode step whose workspace is the library's
static device array, against hws_decode with a caller workspace.

Four calls in a row through the C ABI share the array: each leaves its
selection state, partials and counters there, and the next, smaller one
(fewer sequences, shorter contexts, another launch shape) must still match
hws_decode bit for bit, because the step's own kernels reset what they read.
(The refusal of a step beyond the array is a host check, tested without a GPU
in test_abi_host.)
"""

import numpy as np
import pytest
import torch

from head_wise_sparse_02_amd import hws
from head_wise_sparse_02_amd import workloads as W
from head_wise_sparse_02_amd.runner import DecodeSetup
from gpu_check import check_decode

pytestmark = pytest.mark.gpu

KEYS = ("out", "lse", "sel_counts", "sel_idx", "scores", "rows_read", "sel_mass", "status")


def _both(wl, stage, mode=hws.HWS_LAUNCH_AUTO):
    print(f"\n[case] noalloc {wl.name} B={wl.B} N={wl.seq_lens[:3]} expects {stage}", flush=True)
    st = DecodeSetup(wl, keep_host=True)
    st.ctx.set_launch_mode(mode)
    need = st.ctx.workspace_size(wl.B, st.Nmax, st.score_mode, st.scope)
    assert need <= hws.HWS_NOALLOC_SCRATCH_BYTES, need
    ref = st.decode(debug=True)
    st.ctx.profile_enable(True)
    got = st.decode(debug=True, noalloc=True)
    prof = st.ctx.profile_read()
    st.ctx.profile_enable(False)
    assert prof[stage][1] == 1, prof
    for key in KEYS:
        if key in ref:
            np.testing.assert_array_equal(np.asarray(got[key]), np.asarray(ref[key]), err_msg=key)
    check_decode(st, got, verbose=False)
    # the timed form (no debug outputs) gives the same bits as well
    st.decode(noalloc=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.out.cpu().numpy(), ref["out"])
    return st


def test_noalloc_matches_decode_then_smaller_call():
    # 1: the single launch with the scan inside (full-dim scores, G = 4), 2 x 40000
    _both(W.make_workload(3, n=40000, batch=2), "fused")
    # 2: smaller, the one-launch selection, then the attention balanced by kept
    #    rows (index scores, local heads)
    _both(W.make_workload(2, n=9000, batch=2), "select", hws.HWS_LAUNCH_SCAN_SELECT)
    # 3: smaller, the single launch with the index scan inside
    _both(W.make_workload(2, n=6000, batch=2), "fused_index")
    # 4: smaller still, the single launch after the scan (short context)
    _both(W.make_workload(1, n=3000), "tail", hws.HWS_LAUNCH_SCAN_SINGLE)

