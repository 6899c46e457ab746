"""The scan captured in a HIP graph (through torch's graph capture) and
replayed: every replay, with eager work and synchronizations in between,
must reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import selective_state_space_ssd_amd as ssd
from parity import log, upload
from ssd_workloads import make_inputs, small

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,seqlen", [("f32_b2_L2048_H32_P64_N128_G2_Q128", 700),
                                         ("f32_b1_L256_H4_P64_N16_G1_Q64", 200)])
def test_graph_replay_matches_eager(name, seqlen):
    w = small(name, seqlen=seqlen, init=True)
    log(f"test_graph_replay_matches_eager {name} L={seqlen}")
    inp = make_inputs(w)
    t = upload(inp, "f32")
    dev = t["x"].device
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    ws = torch.empty(ssd.workspace_size(b, L, H, P, N, G, Q, 0), dtype=torch.uint8, device=dev)

    def call(out, fin):
        return ssd.scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                            dt_bias=t["dt_bias"], chunk_size=Q, initial_states=t["initial_states"],
                            return_final_states=True, out=out, final_states=fin, workspace=ws)

    out_e = torch.empty_like(t["x"])
    fin_e = torch.empty(b, H, P, N, device=dev)
    call(out_e, fin_e)
    torch.cuda.synchronize()

    out_g = torch.empty_like(out_e)
    fin_g = torch.empty_like(fin_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_g, fin_g)  # warm-up on the side stream, as torch asks before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out_g, fin_g)
    other = torch.empty_like(out_e)
    for rep in range(4):
        out_g.zero_()
        fin_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: out differs from eager"
        assert torch.equal(fin_g, fin_e), f"replay {rep}: final state differs from eager"
        # unrelated eager work between replays, reusing the same workspace
        call(other, torch.empty_like(fin_e))
        torch.cuda.synchronize()
        assert torch.equal(other, out_e)
