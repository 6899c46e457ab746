"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every comparison is element by element at the bar of tests/parity.py
(fp32 inputs 1e-3 * (1 + |ref|), bf16 inputs 2e-2 * (1 + |ref|)).  Small
cases span several chunks and a ragged tail and are checked everywhere;
the full-size workloads are checked everywhere where the oracle is quick and
on sampled (batch, head) pairs -- every timestep and channel of them -- where
it is not.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import (TOL, bf16_path, compare, current_path, log, np64, paths_for,
                    poisoned_workspace, run_gpu, upload, ws_regions)
from ssd_workloads import WORKLOADS, Workload, make_inputs, small

pytestmark = pytest.mark.gpu


def _oracle(inp, dt_limit=(0.0, math.inf), init=None, head_mask=None):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], dt_bias=inp["dt_bias"], dt_limit=dt_limit,
                          initial_states=init, return_final_states=True, head_mask=head_mask)


def _case(seed, b, L, H, P, N, G, Q, dtype, **kw):
    return Workload(f"case{seed}", b, L, H, P, N, G, Q, dtype, seed, **kw)


# --------------------------------------------------------------------------
# small problems, full comparison (several chunks + a ragged tail)
# --------------------------------------------------------------------------

# (dtype, Q, N, nheads, ngroups).  nheads / ngroups = 2 takes the general
# chunk-scan kernel; a multiple of 4 takes the four-heads-per-workgroup one
# (Q 64/128, N 64/128); nheads = 6 leaves idle waves in the chunk-state kernel.
SMALL = [(dt, Q, N, 4, 2) for dt in ("f32", "bf16") for Q in (64, 128, 256) for N in (16, 128)]
SMALL += [("f32", 128, 32, 4, 2), ("f32", 128, 64, 4, 2), ("bf16", 64, 32, 4, 2),
          ("bf16", 256, 64, 4, 2)]
SMALL += [(dt, Q, N, 8, G) for dt in ("f32", "bf16") for Q in (64, 128) for N in (64, 128)
          for G in (1, 2)]
SMALL += [("f32", 128, 128, 6, 3), ("f32", 64, 64, 12, 3), ("bf16", 128, 128, 16, 1)]
# an odd number of heads leaves the last chunk-state workgroup (two heads) with
# one idle head
SMALL += [("f32", 128, 128, 5, 1), ("bf16", 64, 64, 3, 1)]
# batch * ngroups a multiple of 8: the fused bf16 kernel deals its chains to
# eight ticket classes (one group per class here)
SMALL += [("bf16", 256, 128, 8, 4), ("bf16", 128, 64, 8, 8)]


@pytest.mark.parametrize("dtype,Q,N,H,G", SMALL,
                         ids=[f"{d}-Q{q}-N{n}-H{h}-G{g}" for d, q, n, h, g in SMALL])
def test_small_ragged(dtype, Q, N, H, G):
    L = 2 * Q + Q // 2 + 7
    w = _case(1000 + Q + N + H, 2, L, H, 64, N, G, Q, dtype, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    ref, rfin = _oracle(inp, init=inp["initial_states"])
    for path in paths_for(dtype):
        log(f"test_small_ragged {dtype} Q={Q} N={N} H={H} G={G} L={L} path={path}")
        with bf16_path(path):
            out, fin = run_gpu(t, Q, init=t["initial_states"])
        compare(f"out {path}", np64(out), ref, TOL[dtype])
        compare(f"final {path}", np64(fin), rfin, TOL[dtype])


INTER = [("f32", 128, 128), ("bf16", 128, 128), ("f32", 64, 16), ("bf16", 256, 32),
         ("f32", 256, 64)]


@pytest.mark.parametrize("dtype,Q,N", INTER, ids=[f"{d}-Q{q}-N{n}" for d, q, n in INTER])
def test_stage_intermediates(dtype, Q, N):
    """Each stage's output in the workspace against the oracle's per-chunk
    intermediates: dt and dA_cumsum (stage 1), chunk-local states (stage 2),
    states entering each chunk (stage 3)."""
    b, L, H, P, G = 2, 2 * Q + 44, 4, 64, 2
    w = _case(77, b, L, H, P, N, G, Q, dtype, init=True)
    log(f"test_stage_intermediates {dtype}")
    inp = make_inputs(w)
    t = upload(inp, dtype)
    with bf16_path("staged"):  # the intermediates live in the staged path's workspace
        ws = poisoned_workspace(ssd.workspace_size(b, L, H, P, N, G, Q, 1 if dtype == "bf16"
                                                   else 0, current_path()), t["x"].device)
        run_gpu(t, Q, init=t["initial_states"], workspace=ws)
    got = {k: np64(v) for k, v in ws_regions(ws, b, L, H, P, N, Q).items()}
    ref = oracle.chunk_intermediates(inp["x"], inp["dt"], inp["A"], inp["B"], Q,
                                     dt_bias=inp["dt_bias"], initial_states=inp["initial_states"])
    valid = np.zeros((b, H, 3, Q), bool)
    assert -(-L // Q) == 3
    valid.reshape(b, H, -1)[:, :, :L] = True
    compare("dt", got["dt"], ref["dt"], 1e-5, mask=valid)
    compare("dA_cumsum", got["cum"], ref["cum"], 1e-4, mask=valid)
    compare("chunk_states", got["chunk_states"], ref["chunk_states"], TOL[dtype])
    compare("states_in", got["states_in"], ref["states_in"], TOL[dtype])


# Shapes whose first three stages run as one pass (fp32, batch x heads x
# dstate/32 between half and all of the 256 compute units): dt and the
# running sums (written by the slice-0 workgroups), the states entering each
# chunk (no chunk states go through memory there), out and the final states.
# (the last two: enough heads that 32-column slices would need two rounds,
# so the pass takes 64-column ones)
SCAN23 = [(128, 128, 2, 300, True, 32), (64, 64, 4, 5 * 64 + 7, False, 32),
          (128, 128, 1, 128, True, 32), (64, 128, 2, 32 * 64 - 5, True, 32),
          (128, 128, 4, 300, True, 64), (64, 64, 8, 3 * 64 + 1, False, 128)]


@pytest.mark.parametrize("Q,N,G,L,init,H", SCAN23,
                         ids=[f"Q{q}-N{n}-G{g}-L{l}-{'init' if i else 'zero'}-H{h}"
                              for q, n, g, l, i, h in SCAN23])
def test_state_scan_pass(Q, N, G, L, init, H):
    b, P = 2, 64
    w = _case(880 + Q + N + L, b, L, H, P, N, G, Q, "f32", init=init)
    log(f"test_state_scan_pass Q={Q} N={N} G={G} L={L} init={init} H={H}")
    assert ssd.taken_path(b, L, H, P, N, G, Q, 0) == "staged_scan"
    inp = make_inputs(w)
    t = upload(inp, "f32")
    i0 = inp["initial_states"] if init else None
    ws = poisoned_workspace(ssd.workspace_size(b, L, H, P, N, G, Q, 0), t["x"].device)
    out, fin = run_gpu(t, Q, init=t["initial_states"] if init else None, workspace=ws)
    got = {k: np64(v) for k, v in ws_regions(ws, b, L, H, P, N, Q).items()}
    ref = oracle.chunk_intermediates(inp["x"], inp["dt"], inp["A"], inp["B"], Q,
                                     dt_bias=inp["dt_bias"], initial_states=i0)
    nc = -(-L // Q)
    valid = np.zeros((b, H, nc, Q), bool)
    valid.reshape(b, H, -1)[:, :, :L] = True
    compare("dt", got["dt"], ref["dt"], 1e-5, mask=valid)
    compare("dA_cumsum", got["cum"], ref["cum"], 1e-4, mask=valid)
    compare("states_in", got["states_in"], ref["states_in"], TOL["f32"])
    ro, rf = _oracle(inp, init=i0)
    compare("out", np64(out), ro, TOL["f32"])
    compare("final", np64(fin), rf, TOL["f32"])


def test_state_scan_pass_limits_and_groups():
    """The one-pass stages with dt_limit clamping softplus(dt + dt_bias) on
    both sides, and with two heads per group (the general chunk scan after
    it, no C·Bᵀ tiles in the workspace), D and the gate off."""
    b, H, P, N, Q, L = 2, 32, 64, 128, 128, 3 * 128 - 9
    for G, lim, gate in ((2, (0.01, 0.05), True), (16, (0.0, math.inf), False)):
        w = _case(900 + G, b, L, H, P, N, G, Q, "f32", init=True, gate=gate, skip=gate)
        assert ssd.taken_path(b, L, H, P, N, G, Q, 0) == "staged_scan"
        log(f"test_state_scan_pass_limits_and_groups G={G} dt_limit={lim} gate={gate}")
        inp = make_inputs(w)
        t = upload(inp, "f32")
        out, fin = run_gpu(t, Q, dt_limit=lim, init=t["initial_states"])
        ref, rfin = _oracle(inp, dt_limit=lim, init=inp["initial_states"])
        compare(f"out G={G}", np64(out), ref, TOL["f32"])
        compare(f"final G={G}", np64(fin), rfin, TOL["f32"])


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

EDGE = [
    ("L=1", dict(seqlen=1)),
    ("L<Q", dict(seqlen=45)),
    ("L=Q", dict(seqlen="Q")),
    ("L=Q+1", dict(seqlen="Q+1")),
    ("G=H", dict(ngroups=8, nheads=8)),
    ("no gate, no skip", dict(gate=False, skip=False)),
    ("dt_limit", dict(), ),
]
# fp32 at chunk 128 and bf16 at chunk 256 (the bf16 matrix-core kernels)
EDGE_PATHS = [("f32", 128), ("bf16", 256)]
EDGE_CASES = [(d, q, desc, ch) for d, q in EDGE_PATHS for desc, ch in EDGE]


@pytest.mark.parametrize("dtype,Q,desc,changes", EDGE_CASES,
                         ids=[f"{d}-Q{q}-{e}" for d, q, e, _ in EDGE_CASES])
def test_edge_cases(dtype, Q, desc, changes):
    base = dict(seqlen=200, nheads=4, ngroups=2, gate=True, skip=True)
    base.update(changes)
    L = {"Q": Q, "Q+1": Q + 1}.get(base["seqlen"], base["seqlen"])
    w = _case(300, 2, L, base["nheads"], 64, 128, base["ngroups"], Q, dtype,
              gate=base["gate"], skip=base["skip"], init=True)
    lim = (0.01, 0.05) if desc == "dt_limit" else (0.0, math.inf)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    ref, rfin = _oracle(inp, dt_limit=lim, init=inp["initial_states"])
    for path in paths_for(dtype):
        log(f"test_edge_cases {dtype} Q={Q} {desc} path={path}")
        with bf16_path(path):
            out, fin = run_gpu(t, Q, dt_limit=lim, init=t["initial_states"])
        compare(f"out {path}", np64(out), ref, TOL[dtype])
        compare(f"final {path}", np64(fin), rfin, TOL[dtype])


def test_no_bias_no_init():
    w = _case(301, 1, 333, 4, 64, 64, 1, 64, "f32")
    inp = make_inputs(w)
    inp["dt_bias"] = None
    t = upload(inp, "f32")
    out, fin = run_gpu(t, 64)
    ref, rfin = _oracle(inp)
    compare("out", np64(out), ref, TOL["f32"])
    compare("final", np64(fin), rfin, TOL["f32"])
    out2 = run_gpu(t, 64, final=False)
    assert torch.equal(out, out2)


def test_empty_sequence_and_batch():
    dev = torch.device("cuda:0")
    H, P, N = 4, 64, 16
    x = torch.zeros(2, 0, H, P, device=dev)
    dt = torch.zeros(2, 0, H, device=dev)
    A = -torch.ones(H, device=dev)
    Bc = torch.zeros(2, 0, 1, N, device=dev)
    init = torch.randn(2, H, P, N, device=dev)
    out, fin = ssd.scan_fwd(x, dt, A, Bc, Bc.clone(), chunk_size=64, initial_states=init,
                            return_final_states=True)
    torch.cuda.synchronize()
    assert out.shape == x.shape and torch.equal(fin, init)
    out, fin = ssd.scan_fwd(x, dt, A, Bc, Bc.clone(), chunk_size=64, return_final_states=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin) == 0
    x0 = torch.zeros(0, 10, H, P, device=dev)
    out = ssd.scan_fwd(x0, torch.zeros(0, 10, H, device=dev), A,
                       torch.zeros(0, 10, 1, N, device=dev), torch.zeros(0, 10, 1, N, device=dev),
                       chunk_size=64)
    assert out.shape == x0.shape


def test_unsupported_raises():
    dev = torch.device("cuda:0")
    x = torch.zeros(1, 8, 2, 32, device=dev)
    with pytest.raises(ssd.SsdError) as e:
        ssd.scan_fwd(x, torch.zeros(1, 8, 2, device=dev), -torch.ones(2, device=dev),
                     torch.zeros(1, 8, 1, 16, device=dev), torch.zeros(1, 8, 1, 16, device=dev),
                     chunk_size=64)
    assert e.value.status == -2


# --------------------------------------------------------------------------
# properties of the GPU path
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,Q", [("f32", 128), ("bf16", 256)])
def test_ngroups_invariance(dtype, Q):
    """B, C replicated over G groups give bit-identical outputs to G = 1."""
    w = small("f32_b2_L2048_H32_P64_N128_G1_Q128", seqlen=700, seed=21, init=True,
              dtype=dtype, chunk_size=Q)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    for path in paths_for(dtype):
        with bf16_path(path):
            ref_out, ref_fin = run_gpu(t, Q, init=t["initial_states"])
            for G in (2, 4, 8):
                t2 = dict(t)
                t2["B"] = t["B"].repeat_interleave(G, dim=2).contiguous()
                t2["C"] = t["C"].repeat_interleave(G, dim=2).contiguous()
                out, fin = run_gpu(t2, Q, init=t["initial_states"])
                assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin), (path, G)


def test_chunk_size_invariance():
    w = _case(400, 2, 1000, 4, 64, 128, 2, 128, "f32", init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    ref, rfin = _oracle(inp, init=inp["initial_states"])
    outs = {}
    for Q in (64, 128, 256):
        out, fin = run_gpu(t, Q, init=t["initial_states"])
        compare(f"out Q={Q}", np64(out), ref, TOL["f32"])
        compare(f"final Q={Q}", np64(fin), rfin, TOL["f32"])
        outs[Q] = np64(out)
    compare("Q=64 vs Q=256", outs[64], outs[256], TOL["f32"])


def test_deterministic():
    w = small("f32_b2_L2048_H32_P64_N128_G2_Q128", seqlen=1000, seed=31)
    t = upload(make_inputs(w), "f32")
    a, fa = run_gpu(t, 128)
    b, fb = run_gpu(t, 128)
    assert torch.equal(a, b) and torch.equal(fa, fb)


def test_inplace_continuation():
    """final_states may be the initial_states buffer (chunked prefill in place)."""
    w = _case(500, 2, 2 * 257, 4, 64, 64, 2, 128, "f32", init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    full, ffin = run_gpu(t, 128, init=t["initial_states"])
    state = t["initial_states"].clone()
    outs = []
    for lo, hi in ((0, 257), (257, 514)):
        seg = {k: (v[:, lo:hi].contiguous() if k in ("x", "z", "B", "C", "dt") else v)
               for k, v in t.items()}
        out, fin = run_gpu(seg, 128, init=state, final_states=state)
        assert fin.data_ptr() == state.data_ptr()
        outs.append(out)
    compare("segments vs full", np64(torch.cat(outs, dim=1)), np64(full), TOL["f32"])
    compare("final in place", np64(state), np64(ffin), TOL["f32"])


@pytest.mark.parametrize("H", [32, 64], ids=["slices32", "slices64"])
def test_inplace_continuation_state_scan(H):
    """The same on shapes whose stages 1-3 run as one pass (32- and 64-column
    state slices): each lane reads its init elements before it writes the
    same final ones."""
    w = _case(510 + H, 2, 2 * 300, H, 64, 128, 4, 128, "f32", init=True)
    assert ssd.taken_path(2, 300, H, 64, 128, 4, 128, 0) == "staged_scan"
    inp = make_inputs(w)
    t = upload(inp, "f32")
    full, ffin = run_gpu(t, 128, init=t["initial_states"])
    state = t["initial_states"].clone()
    outs = []
    for lo, hi in ((0, 300), (300, 600)):
        seg = {k: (v[:, lo:hi].contiguous() if k in ("x", "z", "B", "C", "dt") else v)
               for k, v in t.items()}
        out, fin = run_gpu(seg, 128, init=state, final_states=state)
        assert fin.data_ptr() == state.data_ptr()
        outs.append(out)
    compare("segments vs full", np64(torch.cat(outs, dim=1)), np64(full), TOL["f32"])
    compare("final in place", np64(state), np64(ffin), TOL["f32"])
    ref, rfin = _oracle(inp, init=inp["initial_states"])
    compare("out vs oracle", np64(torch.cat(outs, dim=1)), ref, TOL["f32"])
    compare("final vs oracle", np64(state), rfin, TOL["f32"])


# --------------------------------------------------------------------------
# the full-size workloads
# --------------------------------------------------------------------------

def _sample_mask(b, H, G, k, seed):
    """(batch, head) pairs the oracle checks on a full-size workload: in every
    (batch, group) both heads of one randomly chosen pair (2j, 2j + 1) of the
    group -- so every group, every ticket class of the fused kernels (they are
    dealt by (batch, group)) and both heads of a chain-kernel pair are covered
    --, plus `k` random pairs and the last pair."""
    rng = np.random.default_rng(seed)
    mask = np.zeros((b, H), bool)
    hpg = H // G
    for bb in range(b):
        for g in range(G):
            j = int(rng.integers(0, max(1, hpg // 2)))
            lo = g * hpg + min(2 * j, hpg - 1)
            mask[bb, lo] = True
            if hpg > 1:
                mask[bb, min(lo + 1, (g + 1) * hpg - 1)] = True
    idx = rng.choice(b * H, size=min(k, b * H), replace=False)
    mask.reshape(-1)[idx] = True
    mask[b - 1, H - 1] = True  # always the last pair
    return mask


FULL = list(WORKLOADS)


def _run_workload(w, t, name):
    if w.segments == 1:
        log(f"test_workload {name}: GPU run")
        return run_gpu(t, w.chunk_size)
    seg = w.seqlen // w.segments
    state = None
    outs = []
    for i in range(w.segments):
        log(f"test_workload {name}: GPU segment {i}")
        sl = {k: (v[:, i * seg:(i + 1) * seg].contiguous()
                  if k in ("x", "z", "B", "C", "dt") and v is not None else v)
              for k, v in t.items()}
        o, state = run_gpu(sl, w.chunk_size, init=state)
        outs.append(o)
    out, fin = torch.cat(outs, dim=1), state
    full_out, full_fin = run_gpu(t, w.chunk_size)
    tol = TOL[w.dtype]
    compare("segments vs one GPU scan", np64(out), np64(full_out), tol)
    compare("segment final vs one GPU scan", np64(fin), np64(full_fin), tol)
    return out, fin


@pytest.mark.parametrize("name", FULL)
def test_workload(name):
    w = WORKLOADS[name]
    log(f"test_workload {name}: generating inputs")
    inp = make_inputs(w)
    t = upload(inp, w.dtype)
    tol = TOL[w.dtype]
    big = w.batch * w.seqlen * w.nheads > 2 * 2048 * 32
    mask = _sample_mask(w.batch, w.nheads, w.ngroups, 6, w.seed) if big else None
    if mask is not None:
        log(f"test_workload {name}: oracle on {int(mask.sum())} of {mask.size} (batch, head) "
            "pairs (both heads of a pair in every (batch, group))")
    results = {}
    for path in paths_for(w.dtype):
        with bf16_path(path):
            out, fin = _run_workload(w, t, f"{name} [{path}]")
        results[path] = (np64(out), np64(fin))
        del out, fin
    log(f"test_workload {name}: oracle")
    ref, rfin = _oracle(inp, head_mask=mask)
    for path, (got, gfin) in results.items():
        if mask is not None:
            sel = np.broadcast_to(mask[:, None, :, None], ref.shape)
            compare(f"out (sampled heads) {path}", got, ref, tol, mask=sel)
            compare(f"final (sampled heads) {path}", gfin, rfin,
                    tol, mask=np.broadcast_to(mask[:, :, None, None], rfin.shape))
        else:
            compare(f"out {path}", got, ref, tol)
            compare(f"final {path}", gfin, rfin, tol)
