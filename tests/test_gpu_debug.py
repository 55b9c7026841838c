"""The debug library (libmoe_debug.so, built with MOE_DEBUG_CHECKS): its dispatch checks the
caller's expert ids (in [0, E), distinct within a token) into the status word read by
moe_debug_status, and lays out valid ids exactly as the release library does.  Invalid ids
are passed only to the debug build, whose layout kernels drop a slot whose id lies outside
[0, E) instead of indexing with it (a repeated id stays in bounds: its slots share a row)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def moe():
    import expert_ffn_moe_amd

    return expert_ffn_moe_amd


def debug_dispatch(m, p, x, ids):
    """moe_dispatch of the debug library (layout only); returns the layout tensors."""
    dl = m.debug_lib()
    T, k, E = p.T, p.k, p.E
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               row_token=torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
               slot_to_row=torch.empty(T, k, dtype=torch.int32, device=DEV))
    ws = m.workspace(p, m.OP_DISPATCH, DEV)
    c = p.c()
    m._call_on(dl, "moe_dispatch", ctypes.byref(c), ctypes.c_void_p(x.data_ptr()),
               ctypes.c_void_p(ids.data_ptr()), None,
               *(ctypes.c_void_p(out[n].data_ptr()) for n in ("counts", "offsets", "row_token",
                                                              "slot_to_row")),
               None, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return out


def test_release_library_has_no_status_word():
    m = moe()
    v = ctypes.c_uint32(123)
    assert m.lib.moe_debug_status(ctypes.byref(v)) == m.MOE_ERR_UNSUPPORTED and v.value == 0


@pytest.mark.parametrize("wl", [
    Workload("dbg_prefill", T=700, H=128, E=16, k=3, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=81),
    Workload("dbg_many_experts", T=300, H=64, E=1000, k=8, I=64, capacity=0, dtype="bf16",
             logits="normal", seed=82),
], ids=lambda w: w.name)
def test_debug_dispatch_valid_ids_match_release_and_report_nothing(wl):
    print(f"case {wl.name}", flush=True)
    m = moe()
    p = m.Problem.of(wl)
    assert m.debug_status() == 0  # (clears anything left from before)
    logits = synth.make_logits(wl, DEV)
    x = synth.make_x(wl, DEV)
    ids, w, keep = m.route(p, logits)
    rel = m.dispatch(p, x, ids, None, rows=False)
    dbg = debug_dispatch(m, p, x, ids)
    assert m.debug_status() == 0
    N = int(rel["offsets"][-1])
    for n in ("counts", "offsets", "slot_to_row"):
        assert torch.equal(dbg[n], rel[n]), n
    assert torch.equal(dbg["row_token"][:N], rel["row_token"][:N])
    lay = oracle.layout(ids.cpu().numpy(), None, wl.E)
    assert np.array_equal(dbg["offsets"].cpu().numpy(), lay["offsets"])


def test_debug_dispatch_reports_invalid_ids():
    m = moe()
    T, E, k = 200, 16, 4
    p = m.Problem(T=T, H=64, E=E, k=k, I=64)
    rng = np.random.default_rng(83)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = torch.zeros(T, 64, dtype=torch.bfloat16, device=DEV)
    assert m.debug_status() == 0
    # an id past E and a negative one: bit 0; the slots are dropped
    bad = ids.copy()
    bad[5, 1], bad[77, 3] = E, -3
    out = debug_dispatch(m, p, x, torch.as_tensor(bad, device=DEV))
    assert m.debug_status() == 1
    s2r = out["slot_to_row"].cpu().numpy()
    assert s2r[5, 1] == -1 and s2r[77, 3] == -1
    keep = np.ones_like(bad, np.uint8)
    keep[5, 1] = keep[77, 3] = 0
    lay = oracle.layout(np.where(keep == 1, bad, 0).astype(np.int32), keep, E)
    assert np.array_equal(out["offsets"].cpu().numpy(), lay["offsets"])
    assert np.array_equal(s2r, lay["slot_to_row"])
    # the same expert twice in a token: bit 1
    dup = ids.copy()
    dup[9, 2] = dup[9, 0]
    debug_dispatch(m, p, x, torch.as_tensor(dup, device=DEV))
    assert m.debug_status() == 2
    # the word is sticky until read, and reading clears it
    debug_dispatch(m, p, x, torch.as_tensor(bad, device=DEV))
    debug_dispatch(m, p, x, torch.as_tensor(dup, device=DEV))
    assert m.debug_status() == 3
    assert m.debug_status() == 0
