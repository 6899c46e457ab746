"""GPU parity of the backward (ssd_scan_bwd, fp32): every gradient against
the oracle's adjoint recurrence (itself pinned by torch autograd and finite
differences), element by element, on ragged small problems over every dstate
and option, at the edges (one step, no steps, a single block), and at the
full fp32 2 x 2048 size."""
import math

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import TOL, compare, log, np64, upload
from ssd_workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dinitial_states")


def _run(inp, t, dout, dfin, lim=(0.0, math.inf), Q=128, init=True):
    g = ssd.scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"],
                     torch.from_numpy(dout.astype(np.float32)).to(DEV), D=t["D"], z=t["z"],
                     dt_bias=t["dt_bias"], dt_limit=lim, chunk_size=Q,
                     initial_states=t["initial_states"] if init else None,
                     dfinal_states=None if dfin is None else
                     torch.from_numpy(dfin.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         dout.astype(np.float32).astype(np.float64), D=inp["D"], z=inp["z"],
                         dt_bias=inp["dt_bias"], dt_limit=lim,
                         initial_states=inp["initial_states"] if init else None,
                         dfinal=None if dfin is None else dfin.astype(np.float32).astype(np.float64))
    return g, ref


def _compare_all(g, ref, tol=TOL["f32"]):
    for k in NAMES:
        if k in g and ref.get(k) is not None:
            compare(k, np64(g[k]), ref[k], tol)


# (dstate, nheads, ngroups, gate, skip, bias)
# heads per group a multiple of four (N 64/128) with a gate: dY and dz come from
# the re-run chunk scan's epilogue; the other gated cases from the gate kernel
CASES = [(128, 4, 2, True, True, True), (64, 8, 4, True, True, True), (32, 4, 1, False, True, True),
         (16, 6, 3, True, False, False), (128, 8, 1, False, False, True),
         (128, 8, 2, True, True, True), (64, 8, 1, True, False, True)]


@pytest.mark.parametrize("N,H,G,gate,skip,bias", CASES,
                         ids=[f"N{c[0]}-H{c[1]}-G{c[2]}{'' if c[3] else '-nogate'}"
                              f"{'' if c[4] else '-noD'}{'' if c[5] else '-nobias'}" for c in CASES])
def test_bwd_parity(N, H, G, gate, skip, bias):
    rng = np.random.default_rng(N + H + G)
    for L in (2 * 64 + 37, 5):
        w = Workload("bwd", 2, L, H, 64, N, G, 128, "f32", 7000 + N + L, gate=gate, skip=skip,
                     init=True)
        inp = make_inputs(w)
        if not bias:
            inp["dt_bias"] = None
        t = upload(inp, "f32")
        dout = rng.standard_normal(inp["x"].shape)
        dfin = rng.standard_normal((2, H, 64, N))
        log(f"test_bwd_parity N={N} H={H} G={G} gate={gate} skip={skip} bias={bias} L={L}")
        g, ref = _run(inp, t, dout, dfin)
        _compare_all(g, ref)


def test_bwd_dt_limit_and_no_initial_state():
    """An active dt_limit clamp (zero gradient where it clamps), no initial
    state and no final-state gradient."""
    rng = np.random.default_rng(3)
    w = Workload("bwdlim", 2, 200, 4, 64, 64, 2, 64, "f32", 7100)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    dout = rng.standard_normal(inp["x"].shape)
    log("test_bwd_dt_limit_and_no_initial_state")
    g, ref = _run(inp, t, dout, None, lim=(0.05, 0.5), Q=64, init=False)
    _compare_all(g, ref)


@pytest.mark.parametrize("L", [1, 64, 65])
def test_bwd_edges(L):
    rng = np.random.default_rng(L)
    w = Workload("bwdedge", 1, L, 4, 64, 128, 1, 128, "f32", 7200 + L, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    log(f"test_bwd_edges L={L}")
    g, ref = _run(inp, t, rng.standard_normal(inp["x"].shape), rng.standard_normal((1, 4, 64, 128)))
    _compare_all(g, ref)


def test_bwd_no_steps():
    """seqlen 0: the initial state's gradient is dfinal; the per-head sums are 0."""
    H, N = 4, 64
    x = torch.zeros((2, 0, H, 64), device=DEV)
    dt = torch.zeros((2, 0, H), device=DEV)
    Bm = torch.zeros((2, 0, 1, N), device=DEV)
    A = -torch.ones(H, device=DEV)
    init = torch.randn(2, H, 64, N, device=DEV)
    dfin = torch.randn(2, H, 64, N, device=DEV)
    log("test_bwd_no_steps")
    g = ssd.scan_bwd(x, dt, A, Bm, Bm.clone(), torch.zeros_like(x), D=torch.ones(H, device=DEV),
                     dt_bias=torch.zeros(H, device=DEV), initial_states=init, dfinal_states=dfin)
    torch.cuda.synchronize()
    assert torch.equal(g["dinitial_states"], dfin)
    for k in ("dA", "dD", "ddt_bias"):
        assert torch.count_nonzero(g[k]).item() == 0


def test_bwd_deterministic():
    rng = np.random.default_rng(5)
    w = Workload("bwddet", 2, 300, 8, 64, 128, 2, 128, "f32", 7300, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    dout = torch.from_numpy(rng.standard_normal(inp["x"].shape).astype(np.float32)).to(DEV)
    log("test_bwd_deterministic")
    runs = [ssd.scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], dout, D=t["D"], z=t["z"],
                         dt_bias=t["dt_bias"], initial_states=t["initial_states"])
            for _ in range(3)]
    torch.cuda.synchronize()
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]) and torch.equal(runs[0][k], runs[2][k]), k


def test_bwd_full_size():
    """The fp32 batch 2 x seqlen 2048 workload (32 heads, dstate 128, ngroups 1):
    every gradient everywhere."""
    w = WORKLOADS["f32_b2_L2048_H32_P64_N128_G1_Q128"]
    rng = np.random.default_rng(9)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    dout = rng.standard_normal(inp["x"].shape)
    log("test_bwd_full_size: GPU and oracle")
    g, ref = _run(inp, t, dout, None, init=False)
    _compare_all(g, ref)


# --------------------------------------------------------------------------
# bf16 inputs: widened to fp32 in the workspace, the fp32 backward, gradients
# of the bf16 tensors rounded to bf16.  With heads per group a multiple of
# four the gate gradient is formed in the re-run's chunk scan, which reads z
# and dout and writes dz in bf16 itself (the last two cases); otherwise z and
# dout are widened and dz rounded like the rest.
# --------------------------------------------------------------------------

BF16_OUT = ("dx", "ddt", "dB", "dC", "dz")
F32_OUT = ("dA", "dD", "ddt_bias", "dinitial_states")


def _bf16_bits(a):
    """float32 -> (bf16 bit patterns as int16, the rounded values), nearest even."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bits.view(np.int16), (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("N,H,G,L", [(128, 4, 2, 2 * 64 + 37), (64, 8, 8, 300), (16, 6, 3, 1),
                                     (128, 8, 2, 300), (64, 16, 1, 5 * 64 + 1)])
def test_bwd_bf16(N, H, G, L):
    """Every gradient against the oracle on the bf16-rounded inputs (bf16
    gradients to the bf16 bar, fp32 ones to the fp32 bar), and the call equal
    bit for bit to the fp32 backward of the same values with the bf16
    gradients rounded."""
    rng = np.random.default_rng(7300 + N + L)
    w = Workload("bwd16", 2, L, H, 64, N, G, 128, "bf16", 7300 + N + L, init=True)
    inp = make_inputs(w)
    t = upload(inp, "bf16")
    dout_bits, dout = _bf16_bits(rng.standard_normal(inp["x"].shape).astype(np.float32))
    dout16 = torch.from_numpy(dout_bits).to(DEV).view(torch.bfloat16)
    dfin = torch.from_numpy(rng.standard_normal((2, H, 64, N)).astype(np.float32)).to(DEV)
    log(f"test_bwd_bf16 N={N} H={H} G={G} L={L}")
    kw = dict(D=t["D"], dt_bias=t["dt_bias"], chunk_size=128,
              initial_states=t["initial_states"], dfinal_states=dfin)
    g = ssd.scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], dout16, z=t["z"], **kw)
    g32 = ssd.scan_bwd(t["x"].float(), t["dt"].float(), t["A"], t["B"].float(), t["C"].float(),
                       dout16.float(), z=t["z"].float(), **kw)
    torch.cuda.synchronize()
    for k in BF16_OUT:
        assert g[k].dtype == torch.bfloat16, k
        assert torch.equal(g[k], g32[k].to(torch.bfloat16)), k
    for k in F32_OUT:
        assert g[k].dtype == torch.float32 and torch.equal(g[k], g32[k]), k
    ref = oracle.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         dout.astype(np.float64), D=inp["D"], z=inp["z"],
                         dt_bias=inp["dt_bias"], initial_states=inp["initial_states"],
                         dfinal=dfin.cpu().numpy().astype(np.float64))
    for k in BF16_OUT:
        compare(k, np64(g[k]), ref[k], TOL["bf16"])
    for k in F32_OUT:
        compare(k, np64(g[k]), ref[k], TOL["f32"])


@pytest.mark.parametrize("gate", [True, False], ids=["gate", "nogate"])
def test_bwd_leaves_inputs_unchanged(gate):
    """Without a gate dY is dout itself, read in place by the reverse pass;
    with one it is formed in the workspace.  Either way every input, dout
    included, must be bitwise what the caller passed."""
    w = Workload("bwd_inputs", 2, 3 * 64 + 11, 8, 64, 128, 2, 128, "f32", 7300 + gate, gate=gate,
                 skip=True, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    log(f"test_bwd_leaves_inputs_unchanged gate={gate}")
    rng = np.random.default_rng(7301)
    dout = torch.from_numpy(rng.standard_normal(t["x"].shape).astype(np.float32)).to(DEV)
    dfin = torch.from_numpy(
        rng.standard_normal(t["initial_states"].shape).astype(np.float32)).to(DEV)
    args = {k: v for k, v in t.items() if isinstance(v, torch.Tensor)}
    before = {k: v.clone() for k, v in args.items()}
    dout0, dfin0 = dout.clone(), dfin.clone()
    g = ssd.scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], dout, D=t["D"], z=t["z"],
                     dt_bias=t["dt_bias"], initial_states=t["initial_states"], dfinal_states=dfin)
    torch.cuda.synchronize()
    for k, v in args.items():
        assert torch.equal(v, before[k]), k
    assert torch.equal(dout, dout0)
    assert torch.equal(dfin, dfin0)
    assert torch.isfinite(g["dx"]).all()
