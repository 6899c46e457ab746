"""The allocation-free entry point (ssd_scan_fwd_noalloc) against ssd_scan_fwd.

Two calls in a row on each path the scratch serves, the second smaller than
the first (the scratch keeps the first call's contents), each compared element
by element with ssd_scan_fwd on the same inputs at the parity bar.  The fp32
case needs more workspace than the scratch holds, so it runs in slices of
batch rows.
"""
import math

import numpy as np
import pytest
import torch

import selective_state_space_ssd_amd as ssd
from parity import TOL, compare, log, np64, upload
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _w(seed, b, L, H, N, G, Q, dtype):
    return Workload(f"noalloc{seed}", b, L, H, 64, N, G, Q, dtype, seed, init=True, final=True)


# (description, first call, second call: smaller)
PAIRS = [
    ("fp32 staged, rows in slices", _w(901, 4, 2048, 32, 128, 1, 128, "f32"),
     _w(902, 1, 700, 32, 128, 1, 128, "f32")),
    ("bf16 fused per head", _w(903, 2, 1000, 8, 128, 2, 256, "bf16"),
     _w(904, 1, 300, 8, 128, 2, 256, "bf16")),
    ("fp32 dstate 16, chunk 64", _w(905, 2, 777, 4, 16, 1, 64, "f32"),
     _w(906, 1, 65, 4, 16, 1, 64, "f32")),
]


def _noalloc(t, w):
    out = torch.empty_like(t["x"])
    fin = torch.full((w.batch, w.nheads, w.headdim, w.dstate), math.nan, device=t["x"].device)
    ptr = lambda v: None if v is None else v.data_ptr()
    code = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    st = ssd.scan_fwd_noalloc_raw(
        ptr(t["x"]), ptr(t["dt"]), ptr(t["A"]), ptr(t["B"]), ptr(t["C"]), ptr(t["D"]),
        ptr(t["z"]), ptr(t["dt_bias"]), 0.0, math.inf, w.chunk_size, w.ngroups,
        ptr(t["initial_states"]), out.data_ptr(), fin.data_ptr(), w.batch, w.seqlen, w.nheads,
        w.headdim, w.dstate, code, torch.cuda.current_stream().cuda_stream)
    assert st == 0, ssd.status_string(st)
    torch.cuda.synchronize()
    return out, fin


@pytest.mark.parametrize("desc,first,second", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_scan_fwd(desc, first, second):
    for w in (first, second):
        code = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
        need = ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                                  w.chunk_size, code)
        log(f"test_noalloc {desc}: b={w.batch} L={w.seqlen} H={w.nheads} N={w.dstate} "
            f"G={w.ngroups} Q={w.chunk_size} {w.dtype}, workspace {need} bytes "
            f"(scratch {ssd.NOALLOC_SCRATCH_BYTES})")
        inp = make_inputs(w)
        t = upload(inp, w.dtype)
        got, gfin = _noalloc(t, w)
        ref, rfin = ssd.scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                 dt_bias=t["dt_bias"], chunk_size=w.chunk_size,
                                 initial_states=t["initial_states"], return_final_states=True)
        torch.cuda.synchronize()
        compare("out noalloc vs scan_fwd", np64(got), np64(ref), TOL[w.dtype])
        compare("final noalloc vs scan_fwd", np64(gfin), np64(rfin), TOL[w.dtype])
        log(f"  bitwise equal: out {torch.equal(got, ref)}, final {torch.equal(gfin, rfin)}")


def test_noalloc_first_case_is_sliced():
    """The fp32 case above needs more workspace than the scratch: it is the
    one that exercises the slicing by batch rows."""
    w = PAIRS[0][1]
    need = ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                              w.chunk_size, ssd.SSD_F32)
    one = ssd.workspace_size(1, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                             w.chunk_size, ssd.SSD_F32)
    assert need > ssd.NOALLOC_SCRATCH_BYTES >= one
