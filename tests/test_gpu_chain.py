"""GPU checks specific to the chain bf16 kernel (one workgroup carries a pair
of heads of one group through the whole sequence, or one segment of it, the
state in registers): block and segment edges, agreement with the staged bf16
kernels, in-place continuation, run-to-run determinism, and the fallback for
groups with an odd number of heads.  Every bf16 parity test elsewhere also
runs on both the unsegmented and the segmented chain."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import TOL, bf16_path, compare, current_path, log, np64, run_gpu, upload
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _inputs(seed, b, L, H, N, G, init=True, gate=True, skip=True):
    w = Workload(f"chain{seed}", b, L, H, 64, N, G, 256, "bf16", seed, init=init, gate=gate,
                 skip=skip)
    inp = make_inputs(w)
    return w, inp, upload(inp, "bf16")


def _oracle(inp, init=True):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], dt_bias=inp["dt_bias"],
                          initial_states=inp["initial_states"] if init else None,
                          return_final_states=True)


# sequence lengths around the 128-step block of the kernel (L <= 16 takes the
# step kernel), both state sizes, one to four head pairs per group
EDGES = [(L, N, H, G) for L in (17, 127, 128, 129, 255, 257) for (N, H, G) in
         ((128, 4, 2), (64, 8, 1))]


@pytest.mark.parametrize("L,N,H,G", EDGES, ids=[f"L{e[0]}-N{e[1]}-H{e[2]}-G{e[3]}" for e in EDGES])
def test_chain_block_edges(L, N, H, G):
    w, inp, t = _inputs(700 + L + N, 2, L, H, N, G)
    ref, rfin = _oracle(inp)
    for path in ("chain", "chain_segmented"):
        log(f"test_chain_block_edges L={L} N={N} H={H} G={G} path={path}")
        with bf16_path(path):
            ws = ssd.workspace_size(2, L, H, 64, N, G, 256, ssd.SSD_BF16, current_path())
            taken = ssd.taken_path(2, L, H, 64, N, G, 256, ssd.SSD_BF16, kernel_path=path)
            # a one-block sequence is one segment; longer ones are cut into
            # segments of one block here (few pairs), so every block edge is
            # a segment edge
            assert taken == ("chain" if path == "chain" or L <= 128 else "chain_segmented")
            assert (ws == 0) == (taken == "chain")
            out, fin = run_gpu(t, 256, init=t["initial_states"])
        compare(f"out {path}", np64(out), ref, TOL["bf16"])
        compare(f"final {path}", np64(fin), rfin, TOL["bf16"])


# segments of several blocks, each cut into units for the unit-state pass:
# (b, L, H, G, N); the workgroups (pairs x segments) fill the 256 compute
# units, the segment length is not a multiple of the block, L is ragged
SEGMENTS = [(1, 40 * 128 - 37, 128, 8, 128), (2, 33 * 128 + 5, 64, 8, 64),
            (1, 24 * 128, 96, 4, 128)]


@pytest.mark.parametrize("b,L,H,G,N", SEGMENTS, ids=[f"b{s[0]}-L{s[1]}-H{s[2]}" for s in SEGMENTS])
def test_chain_segments_with_units(b, L, H, G, N):
    """Segments of several blocks whose entering states fold several units:
    against the oracle on both heads of a pair in every (batch, group), and
    against the unsegmented chain everywhere."""
    w, inp, t = _inputs(760 + L, b, L, H, N, G)
    with bf16_path("chain_segmented"):
        assert ssd.taken_path(b, L, H, 64, N, G, 256, ssd.SSD_BF16,
                              kernel_path="chain_segmented") == "chain_segmented"
        log(f"test_chain_segments b={b} L={L} H={H} G={G} N={N}: segmented")
        out, fin = run_gpu(t, 256, init=t["initial_states"])
    with bf16_path("chain"):
        log(f"test_chain_segments b={b} L={L} H={H} G={G} N={N}: unsegmented")
        out1, fin1 = run_gpu(t, 256, init=t["initial_states"])
    compare("segmented vs unsegmented out", np64(out), np64(out1), TOL["bf16"])
    compare("segmented vs unsegmented final", np64(fin), np64(fin1), 1e-4)
    mask = np.zeros((b, H), bool)
    hpg = H // G
    for bb in range(b):
        for g in range(G):
            lo = g * hpg + 2 * ((bb + g) % (hpg // 2))
            mask[bb, lo:lo + 2] = True
    ref, rfin = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                               z=inp["z"], dt_bias=inp["dt_bias"],
                               initial_states=inp["initial_states"], return_final_states=True,
                               head_mask=mask)
    compare("out (sampled heads)", np64(out), ref, TOL["bf16"],
            mask=np.broadcast_to(mask[:, None, :, None], ref.shape))
    compare("final (sampled heads)", np64(fin), rfin, TOL["bf16"],
            mask=np.broadcast_to(mask[:, :, None, None], rfin.shape))


# shapes whose default path is the segmented chain with segments of one or two
# blocks: (b, L, H, G); 8 blocks in one-block segments, the same with a ragged
# last block, 4 blocks in two segments of two filling the round
SHORT = [(2, 1024, 32, 4), (2, 1024 - 37, 32, 4), (8, 512, 32, 4)]


@pytest.mark.parametrize("b,L,H,G", SHORT, ids=[f"b{s[0]}-L{s[1]}-H{s[2]}" for s in SHORT])
def test_chain_short_segments_default(b, L, H, G):
    """The default path of these shapes is the segmented chain with segments
    of a block or two (each folding up to seven one-block units): every head
    against the oracle, final states included, and against the unsegmented
    chain."""
    w, inp, t = _inputs(790 + L + b, b, L, H, 128, G)
    assert ssd.taken_path(b, L, H, 64, 128, G, 256, ssd.SSD_BF16) == "chain_segmented"
    log(f"test_chain_short_segments_default b={b} L={L} H={H} G={G}")
    out, fin = run_gpu(t, 256, init=t["initial_states"])
    with bf16_path("chain"):
        out1, fin1 = run_gpu(t, 256, init=t["initial_states"])
    compare("segmented vs unsegmented out", np64(out), np64(out1), TOL["bf16"])
    compare("segmented vs unsegmented final", np64(fin), np64(fin1), 1e-4)
    ref, rfin = _oracle(inp)
    compare("out", np64(out), ref, TOL["bf16"])
    compare("final", np64(fin), rfin, TOL["bf16"])


def test_chain_segmented_is_the_default_for_the_long_sequence():
    """batch 1 x 65536 at 128 heads: 64 pairs, four segments of 128 blocks,
    units of 16 blocks for the unit-state pass."""
    assert ssd.taken_path(1, 65536, 128, 64, 128, 8, 256, ssd.SSD_BF16) == "chain_segmented"
    assert ssd.workspace_size(1, 65536, 128, 64, 128, 8, 256, ssd.SSD_BF16) >= \
        128 * 24 * 64 * 128 * 4


@pytest.mark.parametrize("gate,skip,init", [(False, False, False), (True, False, True),
                                            (False, True, False)])
def test_chain_options(gate, skip, init):
    """Without the z gate, the D skip or an initial state."""
    w, inp, t = _inputs(710, 2, 600, 8, 128, 4, init=init, gate=gate, skip=skip)
    log(f"test_chain_options gate={gate} skip={skip} init={init}")
    ref, rfin = _oracle(inp, init=init)
    for path in ("chain", "chain_segmented"):
        with bf16_path(path):
            out, fin = run_gpu(t, 256, init=t["initial_states"] if init else None)
        compare(f"out {path}", np64(out), ref, TOL["bf16"])
        compare(f"final {path}", np64(fin), rfin, TOL["bf16"])


def test_chain_matches_staged():
    """The two bf16 paths differ only in rounding order: outputs within two
    bf16 ulps of each other, final states within 1e-4 (1 + |ref|)."""
    w, inp, t = _inputs(720, 2, 1500, 16, 128, 2)
    res = {}
    for path in ("chain", "staged"):
        with bf16_path(path):
            res[path] = [np64(v) for v in run_gpu(t, 256, init=t["initial_states"])]
    compare("chain vs staged out", res["chain"][0], res["staged"][0], 2 * 2.0 ** -8)
    compare("chain vs staged final", res["chain"][1], res["staged"][1], 1e-4)


def test_chain_inplace_continuation():
    """final_states may be the initial_states buffer: the state is read at the
    start and written at the end of each workgroup's own heads."""
    w, inp, t = _inputs(730, 2, 2 * 300, 8, 128, 2)
    with bf16_path("chain"):
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


def test_chain_repeat_bitwise():
    """Back-to-back calls of a problem with 256 workgroups give bitwise equal
    outputs and final states (no atomics, fixed reduction orders)."""
    w, inp, t = _inputs(740, 4, 1024, 64, 128, 8)
    with bf16_path("chain"):
        o0, f0 = run_gpu(t, 256, init=t["initial_states"])
        for k in range(6):
            o, f = run_gpu(t, 256, init=t["initial_states"])
            assert torch.equal(o, o0) and torch.equal(f, f0), k
    mask = np.zeros((4, 64), bool)
    mask[[0, 1, 3], [0, 33, 63]] = True
    ref, rfin = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                               z=inp["z"], dt_bias=inp["dt_bias"],
                               initial_states=inp["initial_states"], return_final_states=True,
                               head_mask=mask)
    compare("out (sampled heads)", np64(o0), ref, TOL["bf16"],
            mask=np.broadcast_to(mask[:, None, :, None], ref.shape))


def test_chain_odd_heads_per_group_falls_back():
    """Groups of 3 heads do not pair up: asking for the chain kernel takes the
    fused path (with its workspace) and still matches the oracle."""
    w, inp, t = _inputs(750, 2, 400, 6, 128, 2)
    with bf16_path("chain"):
        assert ssd.workspace_size(2, 400, 6, 64, 128, 2, 256, ssd.SSD_BF16, current_path()) > 0
        out, fin = run_gpu(t, 256, init=t["initial_states"])
    ref, rfin = _oracle(inp)
    compare("out", np64(out), ref, TOL["bf16"])
    compare("final", np64(fin), rfin, TOL["bf16"])
