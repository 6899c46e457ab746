"""GPU checks of the chunk scan's tiles of C.B^T formed once per (chunk, group)
by the state-passing launch (four-heads chunk-scan kernel, nheads/ngroups >=
8): sequence ends inside and on the edges of the 32-step tiles and of the
chunk, both the fp32 path and bf16 inputs at chunk 64, and bitwise agreement
with the kernel that forms the same tiles itself."""
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import TOL, compare, log, np64, run_gpu, upload
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _problem(seed, b, L, H, N, G, Q, dtype):
    w = Workload(f"gram{seed}", b, L, H, 64, N, G, Q, dtype, seed, init=True)
    inp = make_inputs(w)
    return inp, upload(inp, dtype)


def _oracle(inp):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], dt_bias=inp["dt_bias"],
                          initial_states=inp["initial_states"], return_final_states=True)


# (dtype, Q, N, H, G, L): sequence ends at, just before and just after tile and
# chunk edges (L <= 16 would take the step kernel)
EDGES = [("f32", 128, 128, 8, 1, L) for L in (17, 31, 32, 33, 127, 128, 129, 300)]
EDGES += [("f32", 64, 64, 16, 2, L) for L in (40, 64, 65, 150)]
EDGES += [("bf16", 64, 128, 16, 2, L) for L in (17, 63, 64, 65, 200)]


@pytest.mark.parametrize("dtype,Q,N,H,G,L", EDGES,
                         ids=[f"{d}-Q{q}-N{n}-H{h}-G{g}-L{l}" for d, q, n, h, g, l in EDGES])
def test_gram_edges(dtype, Q, N, H, G, L):
    log(f"test_gram_edges {dtype} Q={Q} N={N} H={H} G={G} L={L}")
    ws = ssd.workspace_size(2, L, H, 64, N, G, Q, ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32)
    assert ws > 0
    inp, t = _problem(900 + L + Q, 2, L, H, N, G, Q, dtype)
    out, fin = run_gpu(t, Q, init=t["initial_states"])
    ref, rfin = _oracle(inp)
    compare("out", np64(out), ref, TOL[dtype])
    compare("final", np64(fin), rfin, TOL[dtype])


@pytest.mark.parametrize("L", [300, 2048])
def test_gram_matches_in_kernel_tiles(L):
    """8 heads in one group (tiles formed once per group by the state-passing
    launch) against the same problem with B and C copied into two groups of 4
    heads (one chunk-scan workgroup per group, which forms the tiles itself):
    the same products in the same order, so bitwise equal outputs."""
    inp, t = _problem(950, 2, L, 8, 128, 1, 128, "f32")
    log(f"test_gram_matches_in_kernel_tiles L={L}")
    out1, fin1 = run_gpu(t, 128, init=t["initial_states"])
    t2 = dict(t)
    t2["B"] = t["B"].repeat(1, 1, 2, 1).contiguous()
    t2["C"] = t["C"].repeat(1, 1, 2, 1).contiguous()
    out2, fin2 = run_gpu(t2, 128, init=t["initial_states"])
    assert torch.equal(out1, out2)
    assert torch.equal(fin1, fin2)
