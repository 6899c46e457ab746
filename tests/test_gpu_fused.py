"""GPU checks specific to the fused bf16 kernels (per-head and group forms):
their hand-off of states between workgroups (error word, reuse of a
workspace, determinism, in-place continuation) and their agreement with the
staged bf16 kernels."""
import math

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import (TOL, bf16_path, compare, current_path, log, np64, poisoned_workspace,
                    run_gpu, upload)
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

KINDS = ("fused_head", "fused_group")


def _wait_status(ws, b, L, H, N, G):
    """The fused path's bounded-wait status of the last call on `ws`, read
    through the C ABI (ssd_scan_fwd_wait_status)."""
    return ssd.wait_status(ws.data_ptr(), ws.numel(), b, L, H, 64, N, G, 256, ssd.SSD_BF16,
                           kernel_path=current_path())


def _inputs(seed, b=2, L=700, H=8, N=128, G=4, init=True):
    w = Workload(f"fused{seed}", b, L, H, 64, N, G, 256, "bf16", seed, init=init)
    inp = make_inputs(w)
    return w, inp, upload(inp, "bf16")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("b,L,H,N,G", [(2, 700, 8, 128, 4), (1, 1000, 6, 64, 3),
                                       (4, 129, 16, 128, 2), (1, 400, 24, 128, 2)])
def test_fused_reuse_and_error_word(kind, b, L, H, N, G):
    """Two calls on one workspace: bitwise-equal outputs, error word 0
    (the set-up kernel re-arms the flags and tickets each call)."""
    w, inp, t = _inputs(600 + L, b, L, H, N, G)
    log(f"test_fused_reuse {kind} b={b} L={L} H={H} N={N} G={G}")
    with bf16_path(kind):
        ws = poisoned_workspace(ssd.workspace_size(b, L, H, 64, N, G, 256, 1, current_path()),
                                t["x"].device)
        o1, f1 = run_gpu(t, 256, init=t["initial_states"], workspace=ws)
        assert _wait_status(ws, b, L, H, N, G) == 0
        o2, f2 = run_gpu(t, 256, init=t["initial_states"], workspace=ws)
        assert _wait_status(ws, b, L, H, N, G) == 0
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    ref, rfin = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                               z=inp["z"], dt_bias=inp["dt_bias"],
                               initial_states=inp["initial_states"], return_final_states=True)
    compare("out", np64(o1), ref, TOL["bf16"])
    compare("final", np64(f1), rfin, TOL["bf16"])


@pytest.mark.parametrize("kind", KINDS)
def test_fused_inplace_continuation(kind):
    """final_states may be the initial_states buffer on the fused path too."""
    w, inp, t = _inputs(610, b=2, L=2 * 300, H=8, N=128, G=8)
    with bf16_path(kind):
        full, ffin = run_gpu(t, 256, init=t["initial_states"])
        state = t["initial_states"].clone()
        outs = []
        for lo, hi in ((0, 300), (300, 600)):
            seg = {k: (v[:, lo:hi].contiguous() if k in ("x", "z", "B", "C", "dt") else v)
                   for k, v in t.items()}
            out, fin = run_gpu(seg, 256, init=state, final_states=state)
            assert fin.data_ptr() == state.data_ptr()
            outs.append(out)
    compare("segments vs full", np64(torch.cat(outs, dim=1)), np64(full), TOL["bf16"])
    compare("final in place", np64(state), np64(ffin), 1e-4)


@pytest.mark.parametrize("kind", KINDS)
def test_fused_matches_staged(kind):
    """The bf16 paths differ only in rounding order: outputs within two bf16
    ulps of each other, final states within 1e-4 (1 + |ref|)."""
    w, inp, t = _inputs(620, b=2, L=1500, H=16, N=128, G=2)
    res = {}
    for path in (kind, "staged"):
        with bf16_path(path):
            res[path] = [np64(v) for v in run_gpu(t, 256, init=t["initial_states"])]
    o_f, f_f = res[kind]
    o_s, f_s = res["staged"]
    compare(f"{kind} vs staged out", o_f, o_s, 2 * 2.0 ** -8)
    compare(f"{kind} vs staged final", f_f, f_s, 1e-4)


@pytest.mark.parametrize("kind", KINDS)
def test_fused_repeat_bitwise(kind):
    """Many back-to-back calls of a problem with hundreds of chains in flight
    (2048 workgroups) on one workspace: every call bitwise identical to the
    first and error word 0.  A state read before its producer's stores were
    visible would make a call differ."""
    w, inp, t = _inputs(630, b=4, L=2048, H=32, N=128, G=8)
    with bf16_path(kind):
        ws = poisoned_workspace(
            ssd.workspace_size(4, 2048, 32, 64, 128, 8, 256, 1, current_path()), t["x"].device)
        o0, f0 = run_gpu(t, 256, init=t["initial_states"], workspace=ws)
        for k in range(12):
            o, f = run_gpu(t, 256, init=t["initial_states"], workspace=ws)
            assert _wait_status(ws, 4, 2048, 32, 128, 8) == 0
            assert torch.equal(o, o0) and torch.equal(f, f0), k
    mask = np.zeros((4, 32), bool)
    mask[[0, 1, 3], [5, 17, 31]] = True
    ref, rfin = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                               z=inp["z"], dt_bias=inp["dt_bias"],
                               initial_states=inp["initial_states"], return_final_states=True,
                               head_mask=mask)
    compare("out (sampled heads)", np64(o0), ref, TOL["bf16"],
            mask=np.broadcast_to(mask[:, None, :, None], ref.shape))
    compare("final (sampled heads)", np64(f0), rfin, TOL["bf16"],
            mask=np.broadcast_to(mask[:, :, None, None], rfin.shape))
