"""GPU parity of packed sequences (seq_idx, ssd_scan_fwd_varlen): several
sequences one after another in a batch row, the state reset where the label
changes.  Checked element by element against the oracle's recurrence with
resets, on every kernel variant the call can take (fp32 four-heads and
general kernels, staged bf16 matrix-core and general kernels, the step
kernel for seqlen <= 16), on the per-chunk intermediates, and at the full
size of the fp32 2 x 2048 and bf16 8 x 4096 workloads."""
import math

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_ssd_amd as ssd
from parity import (TOL, bf16_path, compare, current_path, log, np64, paths_for,
                    poisoned_workspace, run_gpu, upload, ws_regions)
from ssd_workloads import WORKLOADS, Workload, make_inputs, make_seq_idx

pytestmark = pytest.mark.gpu


def _oracle(inp, seq, init=None, head_mask=None):
    return oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                          z=inp["z"], dt_bias=inp["dt_bias"], initial_states=init,
                          return_final_states=True, head_mask=head_mask, seq_idx=seq)


def _seq(seq_np):
    return torch.from_numpy(np.ascontiguousarray(seq_np, np.int32)).to("cuda:0")


def _from_lengths(b, L, lengths):
    """Labels for sequences of the given lengths (cycled until the row is full)."""
    out = np.empty((b, L), np.int32)
    for r in range(b):
        t, lab, k = 0, 0, r
        while t < L:
            n = lengths[k % len(lengths)]
            out[r, t:t + n] = lab
            t, lab, k = t + n, lab + 1, k + 1
    return out


# (dtype, Q, N, nheads, ngroups): the kernel variants.  fp32 Q 64/128 with N
# 64/128 and four heads per group: chunk state with dt fused, four-heads chunk
# scan; fp32 N 16/32 or Q 256: general kernels; bf16 Q 128/256 with N 64/128:
# the staged matrix-core kernels; bf16 N 16/32: general kernels.
VAR = [("f32", 128, 128, 8, 2), ("f32", 64, 64, 4, 1), ("f32", 64, 16, 4, 2),
       ("f32", 256, 128, 4, 2), ("f32", 128, 32, 6, 3), ("bf16", 256, 128, 8, 4),
       ("bf16", 128, 64, 8, 8), ("bf16", 64, 16, 4, 2)]
MEANS = (4, "Q/2", "3Q")


@pytest.mark.parametrize("dtype,Q,N,H,G", VAR, ids=[f"{d}-Q{q}-N{n}-H{h}-G{g}"
                                                    for d, q, n, h, g in VAR])
def test_varlen_parity(dtype, Q, N, H, G):
    b, L = 2, 2 * Q + Q // 2 + 7
    w = Workload(f"var{Q}{N}", b, L, H, 64, N, G, Q, dtype, 3000 + Q + N + H, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    for i, m in enumerate(MEANS):
        mean = {"Q/2": Q / 2, "3Q": 3 * Q}.get(m, m)
        seq = make_seq_idx(b, L, mean, 40 + i)
        ref, rfin = _oracle(inp, seq, inp["initial_states"])
        for path in paths_for(dtype):
            log(f"test_varlen_parity {dtype} Q={Q} N={N} H={H} G={G} L={L} mean length {m} "
                f"path={path}")
            with bf16_path(path):
                out, fin = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq))
            compare(f"out mean {m} {path}", np64(out), ref, TOL[dtype])
            compare(f"final mean {m} {path}", np64(fin), rfin, TOL[dtype])


EDGES = [
    ("starts on chunk edges", lambda Q: [Q, Q, 1, Q - 1, 2 * Q]),
    ("length-1 sequences", lambda Q: [1]),
    ("starts next to chunk edges", lambda Q: [Q - 1, 2, Q - 2, Q + 1]),
    ("one sequence", lambda Q: [10 ** 6]),
]


@pytest.mark.parametrize("dtype,Q", [("f32", 128), ("f32", 64), ("bf16", 256)])
@pytest.mark.parametrize("desc,lengths", EDGES, ids=[e[0] for e in EDGES])
def test_varlen_edges(dtype, Q, desc, lengths):
    N, H, G = (128, 8, 2) if Q != 64 else (16, 4, 2)
    b, L = 2, 3 * Q + 5
    w = Workload("varedge", b, L, H, 64, N, G, Q, dtype, 3100 + Q, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    seq = _from_lengths(b, L, lengths(Q))
    ref, rfin = _oracle(inp, seq, inp["initial_states"])
    for path in paths_for(dtype):
        log(f"test_varlen_edges {dtype} Q={Q}: {desc} path={path}")
        with bf16_path(path):
            out, fin = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq))
        compare(f"out {path}", np64(out), ref, TOL[dtype])
        compare(f"final {path}", np64(fin), rfin, TOL[dtype])


def test_varlen_one_label_is_the_plain_scan():
    """A single label per row gives the plain call's result bit for bit (the
    masks are all ones; the same kernels run)."""
    Q, b, L = 128, 2, 300
    w = Workload("varone", b, L, 8, 64, 128, 2, Q, "f32", 3200, init=True)
    t = upload(make_inputs(w), "f32")
    log("test_varlen_one_label_is_the_plain_scan")
    o1, f1 = run_gpu(t, Q, init=t["initial_states"])
    o2, f2 = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(np.full((b, L), 5, np.int32)))
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_labels_only_changes_matter(dtype):
    """Labels that return to earlier values start new sequences all the same:
    two labellings with the same change points give identical results."""
    Q, b, L = 128, 2, 400
    N = 128
    w = Workload("varlab", b, L, 8, 64, N, 2, Q, dtype, 3300, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    seq = make_seq_idx(b, L, 30, 9)
    log(f"test_varlen_labels_only_changes_matter {dtype}")
    ref, rfin = _oracle(inp, seq % 2, inp["initial_states"])
    for path in paths_for(dtype):
        with bf16_path(path):
            o1, f1 = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq))
            o2, f2 = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq % 2))
        assert torch.equal(o1, o2) and torch.equal(f1, f2), path
        compare(f"out {path}", np64(o2), ref, TOL[dtype])
        compare(f"final {path}", np64(f2), rfin, TOL[dtype])


@pytest.mark.parametrize("dtype,Q,N", [("f32", 128, 128), ("bf16", 256, 128), ("f32", 64, 16)])
def test_varlen_intermediates(dtype, Q, N):
    """Workspace after a packed call: the sequence-start counts, the chunk-local
    states (only each chunk's last sequence) and the states entering each chunk,
    against their definitions and the oracle's intermediates."""
    b, L, H, P, G = 2, 2 * Q + 44, 4, 64, 2
    w = Workload("varint", b, L, H, P, N, G, Q, dtype, 3400 + Q, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    seq = make_seq_idx(b, L, Q / 3, 11)
    code = 1 if dtype == "bf16" else 0
    log(f"test_varlen_intermediates {dtype} Q={Q} N={N}")
    with bf16_path("staged"):  # the intermediates live in the staged path's workspace
        total = ssd.varlen_workspace_size(b, L, H, P, N, G, Q, code, current_path())
        ws = poisoned_workspace(total, t["x"].device)
        run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq), workspace=ws)
    nc = -(-L // Q)
    seg_bytes = (b * nc * Q * 4 + 255) // 256 * 256
    seg = ws[total - seg_bytes:total - seg_bytes + b * nc * Q * 4].view(torch.int32)
    starts = np.zeros((b, nc * Q), np.int64)
    starts[:, 1:L] = seq[:, 1:] != seq[:, :-1]
    want = np.cumsum(starts.reshape(b, nc, Q), axis=2)
    assert np.array_equal(seg.view(b, nc, Q).cpu().numpy(), want)
    got = {k: np64(v) for k, v in ws_regions(ws, b, L, H, P, N, Q).items()}
    ref = oracle.chunk_intermediates(inp["x"], inp["dt"], inp["A"], inp["B"], Q,
                                     dt_bias=inp["dt_bias"], initial_states=inp["initial_states"],
                                     seq_idx=seq)
    compare("chunk_states", got["chunk_states"], ref["chunk_states"], TOL[dtype])
    compare("states_in", got["states_in"], ref["states_in"], TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [2, 7, 16])
def test_varlen_step_kernel(dtype, L):
    """seqlen <= 16 (the step kernel): resets inside a few-token call, e.g.
    speculative tokens that straddle the end of one request."""
    w = Workload("vardec", 3, L, 8, 64, 128, 2, 128, dtype, 3500 + L, init=True)
    inp = make_inputs(w)
    t = upload(inp, dtype)
    seq = make_seq_idx(3, L, 2.5, 12 + L)
    log(f"test_varlen_step_kernel {dtype} L={L}")
    assert ssd.varlen_workspace_size(3, L, 8, 64, 128, 2, 128, 1 if dtype == "bf16" else 0) == 0
    out, fin = run_gpu(t, 128, init=t["initial_states"], seq_idx=_seq(seq))
    ref, rfin = _oracle(inp, seq, inp["initial_states"])
    compare("out", np64(out), ref, TOL[dtype])
    compare("final", np64(fin), rfin, TOL[dtype])


# shapes whose stages 1-3 run as one pass (32- and 64-column state slices):
# (Q, N, H, G)
SCAN23 = [(128, 128, 32, 2), (64, 64, 32, 4), (128, 128, 64, 4)]


@pytest.mark.parametrize("Q,N,H,G", SCAN23, ids=[f"Q{q}-N{n}-H{h}-G{g}" for q, n, h, g in SCAN23])
def test_varlen_state_scan_pass(Q, N, H, G):
    """Packed sequences on the one-pass stages 1-3 (the mask of a chunk's
    earlier sequences, the dropped carry where one starts): mean lengths 4,
    Q/2 and 3Q, sequences starting on and next to chunk edges, and every
    step its own sequence."""
    b, L = 2, 2 * Q + Q // 2 + 7
    assert ssd.taken_path(b, L, H, 64, N, G, Q, 0, varlen=True) == "staged_scan"
    w = Workload(f"var23{Q}{N}{H}", b, L, H, 64, N, G, Q, "f32", 3700 + Q + N + H, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    seqs = [(f"mean {m}", make_seq_idx(b, L, {"Q/2": Q / 2, "3Q": 3 * Q}.get(m, m), 50 + i))
            for i, m in enumerate(MEANS)]
    seqs.append(("chunk edges", _from_lengths(b, L, [Q, Q - 1, 2, Q + 1])))
    seqs.append(("every step", np.tile(np.arange(L, dtype=np.int32), (b, 1))))
    for desc, seq in seqs:
        log(f"test_varlen_state_scan_pass Q={Q} N={N} H={H} G={G} {desc}")
        out, fin = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq))
        ref, rfin = _oracle(inp, seq, inp["initial_states"])
        compare(f"out {desc}", np64(out), ref, TOL["f32"])
        compare(f"final {desc}", np64(fin), rfin, TOL["f32"])


def test_varlen_every_step_new():
    """Every step its own sequence: only each token's own term remains."""
    Q, b, L = 128, 2, 260
    w = Workload("varevery", b, L, 8, 64, 128, 2, Q, "f32", 3600, init=True)
    inp = make_inputs(w)
    t = upload(inp, "f32")
    seq = np.tile(np.arange(L, dtype=np.int32), (b, 1))
    log("test_varlen_every_step_new")
    out, fin = run_gpu(t, Q, init=t["initial_states"], seq_idx=_seq(seq))
    ref, rfin = _oracle(inp, seq, inp["initial_states"])
    compare("out", np64(out), ref, TOL["f32"])
    compare("final", np64(fin), rfin, TOL["f32"])


def _sample_mask(b, H, k, seed):
    rng = np.random.default_rng(seed)
    mask = np.zeros((b, H), bool)
    mask.reshape(-1)[rng.choice(b * H, size=min(k, b * H), replace=False)] = True
    mask[b - 1, H - 1] = True
    return mask


FULL = [("f32_b2_L2048_H32_P64_N128_G1_Q128", 256), ("f32_b2_L2048_H32_P64_N128_G4_Q128", 64),
        ("bf16_b8_L4096_H64_P64_N128_G8_Q256", 512)]


@pytest.mark.parametrize("name,mean", FULL, ids=[f"{n}-mean{m}" for n, m in FULL])
def test_varlen_workload(name, mean):
    """The full-size workloads with packed sequences of the given mean length:
    every output for fp32 2 x 2048, sampled (batch, head) pairs for bf16."""
    w = WORKLOADS[name]
    log(f"test_varlen_workload {name} mean {mean}: inputs")
    inp = make_inputs(w)
    t = upload(inp, w.dtype)
    seq = make_seq_idx(w.batch, w.seqlen, mean, 77)
    results = {}
    for path in paths_for(w.dtype):
        with bf16_path(path):
            out, fin = run_gpu(t, w.chunk_size, seq_idx=_seq(seq))
        results[path] = (np64(out), np64(fin))
        del out, fin
    big = w.batch * w.seqlen * w.nheads > 2 * 2048 * 32
    mask = _sample_mask(w.batch, w.nheads, 8, w.seed) if big else None
    log(f"test_varlen_workload {name}: oracle")
    ref, rfin = _oracle(inp, seq, head_mask=mask)
    tol = TOL[w.dtype]
    for path, (got, gfin) in results.items():
        if mask is None:
            compare(f"out {path}", got, ref, tol)
            compare(f"final {path}", gfin, rfin, tol)
        else:
            compare(f"out (sampled heads) {path}", got, ref, tol,
                    mask=np.broadcast_to(mask[:, None, :, None], ref.shape))
            compare(f"final (sampled heads) {path}", gfin, rfin, tol,
                    mask=np.broadcast_to(mask[:, :, None, None], rfin.shape))
