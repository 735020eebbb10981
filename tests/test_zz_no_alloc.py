"""moe_layer_decode_static (the entry point that allocates nothing: a library-owned scratch array
per GPU instead of a caller workspace) against moe_layer_decode, through the C ABI, bit for bit.
Two calls in a row, the second with a smaller input; shapes beyond the scratch are refused."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from moe_synth import workloads as W

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import mid_workloads  # noqa: E402

pytestmark = pytest.mark.gpu


def _call(moe, G, wl, x, M, static):
    S = wl.slots
    ids = torch.full((M, S), -9, dtype=torch.int32, device="cuda")
    w = torch.zeros((M, S), dtype=torch.float32, device="cuda")
    lg = torch.zeros((M, wl.n_routed), dtype=torch.float64, device="cuda")
    y = torch.zeros((M, wl.hidden), dtype=torch.int16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    if static:
        moe.layer_decode_static(G.desc, x, M, ids, w, y, logits=lg, dev_status=st)
    else:
        ws = moe.new_workspace(G.desc, M)
        moe.layer_decode(G.desc, x, M, ids, w, y, ws, logits=lg, dev_status=st)
    torch.cuda.synchronize()
    return [t.cpu().numpy().copy() for t in (ids, w, lg, y, st)]


@pytest.mark.parametrize("name", ["glm_fp8_m1", "mid_mx_bias"])
def test_static_scratch_matches_workspace_call(name):
    import bit_moe_expert_route_amd as moe
    from bit_moe_expert_route_amd.synthetic import GpuLayer, tokens
    base = W.WORKLOADS.get(name) or [w for w in mid_workloads() if w.name == name][0]
    print(f"[no-alloc] {name}", flush=True)
    G = GpuLayer(base.with_m(16))
    # two calls in a row on the shared scratch, the second with fewer tokens (first M = 16 or
    # 4: the several-token launches; then M = 1: the one-token launches)
    for M, first in ((16 if base.hidden < 4096 else 4, 3), (1, 40)):
        wl = base.with_m(M)
        x = tokens(wl, first, M)
        got = _call(moe, G, wl, x, M, static=True)
        ref = _call(moe, G, wl, x, M, static=False)
        for a, b in zip(got, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (name, M)
        assert got[4][0] == 0
        assert np.any(got[3] != 0)


def test_static_scratch_refuses_shapes_beyond_it():
    """A layer whose workspace would exceed the scratch is refused before anything runs."""
    import bit_moe_expert_route_amd as moe
    L = moe.Layer(W.WFMT_MXFP4, 8192, 8192, 64, 15, 1, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000,
                  None, None)
    assert moe.workspace_bytes(L, 16) > moe.STATIC_SCRATCH_BYTES
    st = moe.lib().moe_layer_decode_static(ctypes.byref(L), 0x10000, 16, 0x20000, 0x30000, None,
                                           0x40000, None, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
