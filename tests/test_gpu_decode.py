"""GPU parity of the short-sequence (decode) kernel: seqlen <= 16 takes the
step-by-step kernel whatever the chunk size.  Checked against the oracle,
against the chunked path on the same tokens, and as a chain of one-token
calls continuing in place (serving one token at a time)."""
import math

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import TOL, compare, log, np64, run_gpu, upload
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _oracle(inp, init=None):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], dt_bias=inp["dt_bias"], initial_states=init,
                          return_final_states=True)


CASES = [(dt, L, N, H, G, init) for dt in ("f32", "bf16") for L in (1, 2, 5, 16)
         for (N, H, G) in ((128, 8, 2), (16, 4, 1)) for init in (True, False)]
CASES += [("f32", 3, 32, 6, 3, True), ("bf16", 7, 64, 16, 8, True)]


@pytest.mark.parametrize("dtype,L,N,H,G,init", CASES,
                         ids=[f"{d}-L{l}-N{n}-H{h}-G{g}-{'init' if i else 'zero'}"
                              for d, l, n, h, g, i in CASES])
def test_decode_parity(dtype, L, N, H, G, init):
    w = Workload(f"dec{L}", 3, L, H, 64, N, G, 128, dtype, 900 + L + N + H, init=init)
    log(f"test_decode_parity {dtype} L={L} N={N} H={H} G={G} init={init}")
    inp = make_inputs(w)
    t = upload(inp, dtype)
    out, fin = run_gpu(t, 128, init=t["initial_states"])
    ref, rfin = _oracle(inp, inp["initial_states"])
    compare("out", np64(out), ref, TOL[dtype])
    compare("final", np64(fin), rfin, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_options_off(dtype):
    """No gate, no skip, no bias, finite dt_limit, no final state requested."""
    w = Workload("decopt", 2, 4, 8, 64, 128, 4, 64, dtype, 950, gate=False, skip=False, init=True)
    inp = make_inputs(w)
    inp["dt_bias"] = None
    t = upload(inp, dtype)
    lim = (0.01, 0.05)
    out = run_gpu(t, 64, dt_limit=lim, init=t["initial_states"], final=False)
    ref, _ = oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], dt_limit=lim,
                            initial_states=inp["initial_states"], return_final_states=True)
    compare("out", np64(out), ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_chain_in_place(dtype):
    """A prefix through the chunked path, then one-token calls updating the
    state in place, equals one chunked scan of the whole sequence."""
    prefix, steps = 300, 6
    w = Workload("decchain", 2, prefix + steps, 8, 64, 128, 2, 128, dtype, 960, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    full, ffin = run_gpu(t, 128, init=t["initial_states"])
    state = t["initial_states"].clone()

    def seg(lo, hi):
        return {k: (v[:, lo:hi].contiguous() if k in ("x", "z", "B", "C", "dt") else v)
                for k, v in t.items()}
    outs = [run_gpu(seg(0, prefix), 128, init=state, final_states=state)[0]]
    for k in range(steps):
        o, f = run_gpu(seg(prefix + k, prefix + k + 1), 128, init=state, final_states=state)
        assert f.data_ptr() == state.data_ptr()
        outs.append(o)
    got = np64(torch.cat(outs, dim=1))
    compare("decode chain vs one scan", got, np64(full), TOL[dtype])
    compare("state after the chain", np64(state), np64(ffin), 1e-4)
    ref, rfin = _oracle(inp, inp["initial_states"])
    compare("decode chain vs oracle", got, ref, TOL[dtype])


def test_decode_matches_chunked_at_the_threshold():
    """seqlen 16 (step kernel) and 17 (chunked kernels) agree on their common
    16 tokens to fp32 rounding."""
    w = Workload("dec17", 2, 17, 8, 64, 128, 2, 64, "f32", 970, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    o17, _ = run_gpu(t, 64, init=t["initial_states"])
    t16 = {k: (v[:, :16].contiguous() if k in ("x", "z", "B", "C", "dt") else v) for k, v in t.items()}
    o16, _ = run_gpu(t16, 64, init=t["initial_states"])
    compare("L=16 vs first 16 of L=17", np64(o16), np64(o17[:, :16]), 1e-5)
