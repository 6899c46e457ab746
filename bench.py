"""Throughput of the SSD scan forward on one MI355X.

One step = one pass of the whole scan (dt/cumsum, chunk state, state passing,
chunk scan with the D/z epilogue) over the fp32 workload batch 2 x seqlen
2048, 32 heads of 64, dstate 128, chunk 128, at ngroups 1, 2 and 4: three
ssd_scan_fwd calls, 3 x 4096 tokens.  Inputs are seeded, synthetic and
resident in HBM before timing starts; two copies of every input rotate across
steps so that consecutive steps touch more memory than the 256 MB Infinity
Cache holds.

Prints one JSON line: tokens/s over the timed steps, the roofline of the
dominant kernel (its algorithmic flops per launch over its mean launch time,
measured with HIP events recorded by the library on the launch stream), the
CPU oracle's throughput on the same workload, and (unless --no-bf16) three
more workloads: bf16 batch 8 x seqlen 4096 and a one-token bf16 decode step
(batch 128, state in place), against the HBM roofline, and the fp32 batch 2 x
seqlen 2048 shape holding packed sequences (seq_idx), against the fp32
matrix roofline, and the block around the scan (conv1d prologue, gated RMSNorm
epilogue) at the fp32 2 x 2048 size, its prologue and epilogue against the HBM
roofline, and the backward (every gradient) of the fp32 2 x 2048 workload
against the fp32 matrix roofline.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ssd_workloads import BENCH_WORKLOADS, WORKLOADS, make_inputs, make_seq_idx  # noqa: E402

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


# Kernel sources whose counters the committed traffic summary describes.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_scan_group_f32_b2_L2048_traffic.json")


def measured_traffic(kernel_stage):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    import json
    if kernel_stage != "chunk_scan" or not os.path.exists(TRAFFIC_FILE):
        return None
    from rocprof_summary import sources_hash
    t = json.load(open(TRAFFIC_FILE))
    csrc = os.path.join(ROOT, "selective_state_space_ssd_amd", "csrc")
    if sources_hash([os.path.join(csrc, n) for n in t["sources"]]) != t["sources_sha256_16"]:
        return None
    return t["bytes_per_dispatch"]


def alg_flops(w):
    """Algorithmic flops of one call, by stage (chunked SSD, causal, C.B^T once
    per group): chunk state 2QPN per (chunk, head); state passing 2PN per
    (chunk, head); chunk scan 2QPN + PQ(Q+1) per (chunk, head); C.B^T NQ(Q+1)
    per (chunk, group), in the stage that forms it: the state-passing launch
    when the four-heads chunk scan runs with two or more of its workgroups per
    group (it reads the tiles from there), else the chunk scan."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    nc = math.ceil(L / Q)
    gram = b * nc * G * N * Q * (Q + 1)
    group_scan = (Q in (64, 128) and N in (64, 128) and (H // G) % 4 == 0 and H // G >= 8
                  and not (w.dtype == "bf16" and Q == 128))
    return {
        "prep": b * L * H * 2.0,
        "chunk_state": b * nc * H * 2.0 * Q * P * N,
        "state_passing": b * nc * H * 2.0 * P * N + (gram if group_scan else 0),
        "chunk_scan": b * nc * H * (2.0 * Q * P * N + P * Q * (Q + 1)) + (0 if group_scan else gram),
    }


def alg_bytes(w):
    """Bytes the method must move: read x, dt, B, C, (z), (init), A, D, dt_bias;
    write out, (final).  Intermediates are not counted."""
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    es = 2 if w.dtype == "bf16" else 4
    n = b * L * H * P * es * (2 + (1 if w.gate else 0))     # x, out, z
    n += b * L * H * es + 2 * b * L * G * N * es              # dt, B, C
    n += 3 * H * 4
    st = b * H * P * N * 4
    n += st * ((1 if w.init else 0) + (1 if w.final else 0))
    return n


def cpu_baseline(workloads, min_seconds=10.0):
    """The oracle (untuned fp64 recurrence, OpenMP over batch x heads) on the
    whole step, repeated until at least `min_seconds` have passed."""
    import oracle
    inputs = [make_inputs(w) for w in workloads]
    threads = oracle.max_threads()
    tokens, elapsed, passes = 0, 0.0, 0
    while elapsed < min_seconds:
        for w, inp in zip(workloads, inputs):
            t0 = time.perf_counter()
            oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                           z=inp["z"], dt_bias=inp["dt_bias"])
            elapsed += time.perf_counter() - t0
            tokens += w.tokens
        passes += 1
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} full step(s): ngroups 1, 2, 4 at batch 2 x seqlen 2048 "
                      f"({tokens} tokens, {elapsed:.1f} s, fp64 recurrence)",
            "cpu": _cpu_model()}


def bf16_kernel(ssd, workspace_bytes):
    """The kernel a bf16 call takes: the chain kernel needs no workspace."""
    opt = ssd.get_bf16_path()
    if workspace_bytes == 0:
        return "chain"
    return opt if opt != "auto" else "fused"


def bf16_workload(steps, warmup, name="bf16_b8_L4096_H64_P64_N128_G8_Q256"):
    """The bf16 workload (batch 8 x seqlen 4096, 64 heads, 8 groups, chunk 256,
    z and D on, final states returned) on the default bf16 path: calls per
    second over `steps` calls after `warmup`, with the algorithmic bytes of a
    call over its mean duration against the HBM peak."""
    import torch
    import selective_state_space_ssd_amd as ssd
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    t = {"z": None, "D": None}
    for k in ("x", "z", "B", "C", "dt"):
        if k in inp["bits"]:
            t[k] = torch.from_numpy(inp["bits"][k].view(np.int16)).to(dev).view(torch.bfloat16)
    for k in ("A", "D", "dt_bias"):
        if inp.get(k) is not None:
            t[k] = torch.from_numpy(inp[k]).to(dev)
    del inp
    out = torch.empty_like(t["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    wsz = ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                             w.chunk_size, ssd.SSD_BF16)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    ptr = lambda v: None if v is None else v.data_ptr()
    a = (t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(),
         t["C"].data_ptr(), ptr(t["D"]), ptr(t["z"]), t["dt_bias"].data_ptr(), 0.0,
         math.inf, w.chunk_size, w.ngroups, None, out.data_ptr(), fin.data_ptr(), w.batch,
         w.seqlen, w.nheads, w.headdim, w.dstate, ssd.SSD_BF16, ws.data_ptr(), wsz)
    s = torch.cuda.current_stream(dev).cuda_stream

    def call():
        st = ssd.scan_fwd_raw(*a, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    nbytes = alg_bytes(w)
    return {
        "workload": "ssd_scan_fwd bf16 batch 8 x seqlen 4096, 64 heads x headdim 64, dstate "
                    "128, ngroups 8, chunk 256, z gate and D on, final states returned",
        "path": bf16_kernel(ssd, wsz),
        "tokens_per_s": w.tokens / el,
        "ms_per_call": el * 1e3,
        "calls": steps,
        "roofline": {"bound": "hbm", "achieved": nbytes / el / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / el / 1e9 / PEAK_HBM_GBS,
                     "alg_bytes": nbytes},
    }


def decode_workload(steps, warmup, batch=128, nheads=64, dstate=128, ngroups=8):
    """One-token decode steps (bf16 inputs, fp32 state updated in place, z and D
    on): the short-sequence kernel.  Bound by reading and writing the state, so
    the roofline is HBM on the state bytes plus the token's inputs."""
    import torch
    import selective_state_space_ssd_amd as ssd
    dev = torch.device("cuda:0")
    P = 64
    g = torch.Generator(device="cpu").manual_seed(11)

    def bf(*shape):
        return torch.randn(*shape, generator=g).to(torch.bfloat16).to(dev)

    x, z = bf(batch, 1, nheads, P), bf(batch, 1, nheads, P)
    dt = bf(batch, 1, nheads)
    B, C = bf(batch, 1, ngroups, dstate), bf(batch, 1, ngroups, dstate)
    A = (-torch.exp(torch.rand(nheads, generator=g) * math.log(16.0))).to(dev)
    D = torch.randn(nheads, generator=g).to(dev)
    dt_bias = torch.full((nheads,), -2.0).to(dev)
    state = torch.randn(batch, nheads, P, dstate, generator=g).to(dev)
    out = torch.empty_like(x)
    a = (x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(),
         z.data_ptr(), dt_bias.data_ptr(), 0.0, math.inf, 128, ngroups, state.data_ptr(),
         out.data_ptr(), state.data_ptr(), batch, 1, nheads, P, dstate, ssd.SSD_BF16, None, 0)
    s = torch.cuda.current_stream(dev).cuda_stream

    def call():
        st = ssd.scan_fwd_raw(*a, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    nbytes = 2 * batch * nheads * P * dstate * 4 + batch * (
        3 * nheads * P * 2 + nheads * 2 + 2 * ngroups * dstate * 2)
    return {
        "workload": f"one-token decode, bf16 inputs, batch {batch}, {nheads} heads x headdim 64, "
                    f"dstate {dstate}, ngroups {ngroups}, z and D on, fp32 state in place",
        "tokens_per_s": batch / el,
        "us_per_call": el * 1e6,
        "calls": steps,
        "roofline": {"bound": "hbm", "achieved": nbytes / el / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": nbytes / el / 1e9 / PEAK_HBM_GBS,
                     "alg_bytes": nbytes},
    }


def varlen_workload(steps, warmup, name="f32_b2_L2048_H32_P64_N128_G1_Q128", mean_len=256):
    """Packed sequences (seq_idx) on the fp32 batch 2 x seqlen 2048 shape: each row
    holds sequences of mean length `mean_len` (uniform lengths 1 .. 2*mean-1).
    Calls alternate between two input copies, like the main measurement; the
    same calls without seq_idx are timed alongside.  The chunked form does the
    same work with or without sequence starts, so the roofline is the whole
    call's algorithmic flops over its time against the fp32 matrix peak."""
    import torch
    import selective_state_space_ssd_amd as ssd
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    code = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
    ws_bytes = max(ssd.varlen_workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                             w.ngroups, w.chunk_size, code),
                   ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                      w.ngroups, w.chunk_size, code))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    seq = torch.from_numpy(make_seq_idx(w.batch, w.seqlen, mean_len, 77)).to(dev)
    keep, calls = [], []
    for _ in range(2 if w.dtype == "f32" else 1):
        inp = make_inputs(w)
        t = {k: torch.from_numpy(v).to(dev) for k, v in inp.items()
             if isinstance(v, np.ndarray)}
        if w.dtype == "bf16":
            for k in ("x", "z", "B", "C", "dt"):
                t[k] = torch.from_numpy(inp["bits"][k].view(np.int16)).to(dev).view(torch.bfloat16)
        out = torch.empty_like(t["x"])
        fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), device=dev)
        keep.append((t, out, fin))
        calls.append((t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(),
                      t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(),
                      t["z"].data_ptr(), t["dt_bias"].data_ptr(), 0.0, math.inf, w.chunk_size,
                      w.ngroups, None, out.data_ptr(), fin.data_ptr() if w.final else None))
    tail = (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, code, ws.data_ptr(),
            ws_bytes, torch.cuda.current_stream(dev).cuda_stream)

    def run(k, packed):
        a = calls[k % len(calls)]
        st = (ssd.scan_fwd_varlen_raw(*a, seq.data_ptr(), *tail) if packed
              else ssd.scan_fwd_raw(*a, *tail))
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    res = {}
    for packed in (True, False):
        for k in range(warmup):
            run(k, packed)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            run(k, packed)
        torch.cuda.synchronize()
        res[packed] = (time.perf_counter() - t0) / steps
    el = res[True]
    nseq = int((seq[:, 1:] != seq[:, :-1]).sum().item()) + w.batch
    line = {
        "workload": f"ssd_scan_fwd_varlen {w.dtype} batch {w.batch} x seqlen {w.seqlen} holding "
                    f"{nseq} packed sequences (mean length {mean_len}), {w.nheads} heads x "
                    f"headdim 64, dstate {w.dstate}, chunk {w.chunk_size}, ngroups {w.ngroups}, "
                    "z gate and D on",
        "path": "staged" if w.dtype == "f32" else bf16_kernel(ssd, ws_bytes),
        "tokens_per_s": w.tokens / el,
        "us_per_call": el * 1e6,
        "plain_us_per_call": res[False] * 1e6,
        "calls": steps,
    }
    if w.dtype == "f32":  # matrix-bound, like the plain fp32 workload
        fl = sum(alg_flops(w).values())
        line["roofline"] = {"bound": "mfma", "achieved": fl / el / 1e12,
                            "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                            "frac": fl / el / 1e12 / PEAK_FP32_MFMA_TFLOPS, "alg_flops": fl}
    else:  # HBM-bound, like the plain bf16 workload
        nbytes = alg_bytes(w) + w.batch * w.seqlen * 4
        line["roofline"] = {"bound": "hbm", "achieved": nbytes / el / 1e9, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": nbytes / el / 1e9 / PEAK_HBM_GBS,
                            "alg_bytes": nbytes}
    return line


def block_workload(steps, warmup, ngroups=1, norm_groups=1):
    """The block around the scan (split + conv1d + SiLU prologue, scan, gated
    RMSNorm epilogue) at mamba issue #647's repro size: fp32, batch 2 x seqlen
    2048, dim 2048 (32 heads of 64), dstate 128, conv width 4, chunk 128, with
    seeded random inputs.  Calls alternate two input copies.  The scan alone on
    same-shaped inputs (no gate) is timed alongside; the difference is the
    prologue and epilogue, whose algorithmic bytes over that time give the
    HBM roofline line."""
    import torch
    import selective_state_space_ssd_amd as ssd
    b, L, H, P, N, W, Q = 2, 2048, 32, 64, 128, 4, 128
    G = ngroups
    dim, gn = H * P, G * N
    width = 2 * dim + 2 * gn + H
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(21)
    f = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev)
    zx = [f(b, L, width) for _ in range(2)]
    cw, cb = 0.5 * f(dim + 2 * gn, W), 0.1 * f(dim + 2 * gn)
    dt_bias = torch.full((H,), -2.0, device=dev)
    A = -torch.exp(torch.from_numpy(rng.uniform(0, math.log(16.0), H).astype(np.float32)).to(dev))
    D, nw = f(H), 1.0 + 0.1 * f(dim)
    out = torch.empty((b, L, dim), device=dev)
    wsz = ssd.block_workspace_size(b, L, H, P, N, G, Q, ssd.SSD_F32, W, norm_groups)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    # the scan alone on same-shaped inputs, no gate (the scan inside the block)
    xs = [f(b, L, H, P) for _ in range(2)]
    Bs, Cs, dts = f(b, L, G, N), f(b, L, G, N), f(b, L, H)
    y = torch.empty_like(xs[0])
    swsz = ssd.workspace_size(b, L, H, P, N, G, Q, ssd.SSD_F32)
    sws = torch.empty(swsz, dtype=torch.uint8, device=dev)

    def block_call(k):
        st = ssd.split_conv1d_scan_fwd_raw(
            zx[k % 2].data_ptr(), cw.data_ptr(), cb.data_ptr(), dt_bias.data_ptr(), A.data_ptr(),
            D.data_ptr(), Q, None, 0.0, math.inf, nw.data_ptr(), 1e-5, P, G, norm_groups,
            out.data_ptr(), None, b, L, H, N, W, ssd.SSD_F32, ws.data_ptr(), wsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    def scan_call(k):
        st = ssd.scan_fwd_raw(xs[k % 2].data_ptr(), dts.data_ptr(), A.data_ptr(), Bs.data_ptr(),
                              Cs.data_ptr(), D.data_ptr(), None, dt_bias.data_ptr(), 0.0,
                              math.inf, Q, G, None, y.data_ptr(), None, b, L, H, P, N,
                              ssd.SSD_F32, sws.data_ptr(), swsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    res = {}
    for name, fn in (("block", block_call), ("scan", scan_call)):
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            fn(k)
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) / steps
    extra = res["block"] - res["scan"]
    # prologue: read the xBC and dt columns (plus a 3-step halo per 32-step
    # tile) and write x, B, C, dt; epilogue: read y and z, write out
    halo = 1.0 + (W - 1) / 32.0
    nbytes = b * L * 4 * ((dim + 2 * gn + H) * (1.0 + halo) + 3 * dim)
    return {
        "workload": f"ssd_split_conv1d_scan_fwd f32 batch 2 x seqlen 2048, dim 2048 (32 heads x "
                    f"headdim 64), dstate 128, ngroups {G}, conv width 4, chunk 128, gated "
                    f"RMSNorm over {'the whole width' if norm_groups == 1 else 'each group'}",
        "tokens_per_s": b * L / res["block"],
        "us_per_call": res["block"] * 1e6,
        "scan_alone_us_per_call": res["scan"] * 1e6,
        "calls": steps,
        "roofline": {"kernels": "prologue + epilogue (block time minus scan time)",
                     "bound": "hbm", "achieved": nbytes / extra / 1e9 if extra > 0 else None,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / extra / 1e9 / PEAK_HBM_GBS if extra > 0 else None,
                     "alg_bytes": nbytes},
    }


def bwd_alg_flops(w, T=64):
    """Algorithmic flops of one backward call: the forward re-run in T-step
    blocks plus, per (block, head), the causal in-block products (C.B^T once
    per group, dY.x^T, the masked products with dY, C and B: T(T+1)/2 pairs
    each) and the five T x P x N products with the block's states (P_c, G.B,
    X.G, dY.H_in and the state part of dC)."""
    from dataclasses import replace
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    nb = math.ceil(L / T)
    fwd = sum(alg_flops(replace(w, chunk_size=T)).values())
    pairs = T * (T + 1) / 2
    per = 2.0 * (pairs * (P + P + 2 * N) + 5 * T * P * N)
    return fwd + b * nb * (H * per + G * 2.0 * pairs * N)


def bwd_workload(steps, warmup, name="f32_b2_L2048_H32_P64_N128_G1_Q128", dtype="f32"):
    """The backward (every gradient, dfinal zero, z, D and dt_bias on) of the
    batch 2 x seqlen 2048 workload at ngroups 1, alternating two input copies;
    the forward on the same inputs is timed alongside.  dtype "bf16": x, dt,
    B, C, z, dout and their gradients in bf16 (the inputs rounded)."""
    import torch
    import selective_state_space_ssd_amd as ssd
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    io = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32
    rng = np.random.default_rng(31)
    copies = []
    for _ in range(2):
        t = {k: torch.from_numpy(v).to(dev) for k, v in make_inputs(w).items()
             if isinstance(v, np.ndarray)}
        t["dout"] = torch.from_numpy(rng.standard_normal((b, L, H, P)).astype(np.float32)).to(dev)
        for k in ("x", "dt", "B", "C", "z", "dout"):
            t[k] = t[k].to(io)
        copies.append(t)
    e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    eio = lambda *shape: torch.empty(shape, dtype=io, device=dev)
    gr = dict(dx=eio(b, L, H, P), ddt=eio(b, L, H), dA=e(H), dB=eio(b, L, G, N),
              dC=eio(b, L, G, N), dD=e(H), dz=eio(b, L, H, P), ddt_bias=e(H))
    wsz = ssd.bwd_workspace_size(b, L, H, P, N, G, w.chunk_size, code)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    fsz = ssd.workspace_size(b, L, H, P, N, G, w.chunk_size, code)
    fws = torch.empty(max(fsz, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((b, L, H, P), dtype=io, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream

    def bwd_call(k):
        t = copies[k % 2]
        st = ssd.scan_bwd_raw(
            t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(),
            t["C"].data_ptr(), t["D"].data_ptr(), t["z"].data_ptr(), t["dt_bias"].data_ptr(),
            0.0, math.inf, w.chunk_size, G, None, t["dout"].data_ptr(), None,
            gr["dx"].data_ptr(), gr["ddt"].data_ptr(), gr["dA"].data_ptr(), gr["dB"].data_ptr(),
            gr["dC"].data_ptr(), gr["dD"].data_ptr(), gr["dz"].data_ptr(),
            gr["ddt_bias"].data_ptr(), None, b, L, H, P, N, code, ws.data_ptr(), wsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    def fwd_call(k):
        t = copies[k % 2]
        st = ssd.scan_fwd_raw(t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(),
                              t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(),
                              t["z"].data_ptr(), t["dt_bias"].data_ptr(), 0.0, math.inf,
                              w.chunk_size, G, None, out.data_ptr(), None, b, L, H, P, N,
                              code, fws.data_ptr(), fsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    res = {}
    for nm, fn in (("bwd", bwd_call), ("fwd", fwd_call)):
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            fn(k)
        torch.cuda.synchronize()
        res[nm] = (time.perf_counter() - t0) / steps
    fl = bwd_alg_flops(w)
    el = res["bwd"]
    return {
        "workload": f"ssd_scan_bwd {dtype} batch 2 x seqlen 2048, 32 heads x headdim 64, "
                    "dstate 128, ngroups 1, z gate, D and dt_bias on: every gradient (forward "
                    "re-run inside" + (", inputs widened to fp32 and bf16 gradients rounded)"
                                       if dtype == "bf16" else ")"),
        "tokens_per_s": w.tokens / el,
        "us_per_call": el * 1e6,
        "forward_us_per_call": res["fwd"] * 1e6,
        "calls": steps,
        "roofline": {"bound": "mfma", "achieved": fl / el / 1e12, "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": fl / el / 1e12 / PEAK_FP32_MFMA_TFLOPS,
                     "alg_flops": fl},
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the second measured workload (bf16, batch 8 x seqlen 4096)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the step once as a HIP graph per input copy, replay "
                         "it, and report the replay rate as the value")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the steps, run 3 plain device copies of this many MiB "
                         "(reference kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the scan is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_ssd_amd as ssd

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    workloads = [WORKLOADS[n] for n in BENCH_WORKLOADS]
    stream = torch.cuda.current_stream(dev)

    # inputs, two copies of each, plus outputs and one shared workspace
    calls = []   # per rotation copy: list of argument tuples for ssd_scan_fwd
    keep = []
    ws_bytes = max(ssd.workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                      w.ngroups, w.chunk_size, 0) for w in workloads)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for copy in range(2):
        args_copy = []
        for w in workloads:
            inp = make_inputs(w)
            t = {k: torch.from_numpy(v).to(dev) for k, v in inp.items()
                 if isinstance(v, np.ndarray)}
            out = torch.empty_like(t["x"])
            keep.append((t, out))
            args_copy.append((
                t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(),
                t["C"].data_ptr(), t["D"].data_ptr(), t["z"].data_ptr(),
                t["dt_bias"].data_ptr(), 0.0, math.inf, w.chunk_size, w.ngroups, None,
                out.data_ptr(), None, w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                ssd.SSD_F32, ws.data_ptr(), ws_bytes))
        calls.append(args_copy)

    def step(k, timings=None):
        s = torch.cuda.current_stream(dev).cuda_stream
        for i, a in enumerate(calls[k % 2]):
            st = ssd.scan_fwd_raw(*a, s, timing=None if timings is None else timings[i])
            if st != 0:
                raise ssd.SsdError(st, ssd.status_string(st))

    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    # eager launches: exactly `steps` steps
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t0

    # the same step captured as one HIP graph per input copy (three calls,
    # nine kernels, no allocation or memset inside), replayed
    elapsed_graph = None
    if args.graph:
        graphs = []
        for k in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        for k in range(args.warmup):
            graphs[k % 2].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[k % 2].replay()
        torch.cuda.synchronize()
        elapsed_graph = time.perf_counter() - t0
    elapsed = elapsed_graph if elapsed_graph is not None else elapsed_eager

    # per-stage durations: the same steps again, with the library recording a
    # HIP event around each stage on the launch stream
    timings = [[ssd.Timing() for _ in workloads] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(k, timings[k])
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    stage_ms = np.array([[tm.read() for tm in row] for row in timings])  # [steps, calls, stages]
    mean_ms = stage_ms.mean(axis=0)                                        # [calls, stages]

    tokens = sum(w.tokens for w in workloads)
    value = tokens * args.steps / elapsed
    flops = [alg_flops(w) for w in workloads]
    per_stage_total = mean_ms.sum(axis=0)
    dom = int(np.argmax(per_stage_total))
    dom_name = ssd.STAGES[dom]
    dom_flops = sum(f[dom_name] for f in flops)
    dom_s = per_stage_total[dom] / 1e3
    achieved = dom_flops / dom_s / 1e12
    path_flops = sum(sum(f.values()) for f in flops)
    step_s = elapsed / args.steps
    path_bytes = sum(alg_bytes(w) for w in workloads)

    line = {
        "metric": "SSD scan fwd tokens/sec at 1 MI355X; % of MFMA/HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "ssd_scan_fwd f32 batch 2 x seqlen 2048, 32 heads x headdim 64, "
                        "dstate 128, chunk 128, ngroups 1/2/4 (3 calls per step), "
                        "z gate and D skip on, dt_limit (0, inf)",
            "batch": 2, "seqlen": 2048, "nheads": 32, "headdim": 64, "dstate": 128,
            "chunk_size": 128, "ngroups": [1, 2, 4], "tokens_per_step": tokens,
            "launch": "hip graph replay" if elapsed_graph is not None else "eager",
        },
        "roofline": {
            "kernel": dom_name,
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
            "traffic": measured_traffic(dom_name),
            "launches_timed": args.steps * len(workloads),
            "mean_launch_us": dom_s / len(workloads) * 1e6,
        },
        "path": {
            "alg_tflops_per_s": path_flops / step_s / 1e12,
            "mfma_frac": path_flops / step_s / 1e12 / PEAK_FP32_MFMA_TFLOPS,
            "alg_gbytes_per_s": path_bytes / step_s / 1e9,
            "hbm_frac": path_bytes / step_s / 1e9 / PEAK_HBM_GBS,
            "stage_us_per_call": {s: float(per_stage_total[i] / len(workloads) * 1e3)
                                  for i, s in enumerate(ssd.STAGES)},
            "event_pass_ms_per_step": elapsed_ev / args.steps * 1e3,
            "eager_ms_per_step": elapsed_eager / args.steps * 1e3,
            "eager_tokens_per_s": tokens * args.steps / elapsed_eager,
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(workloads),
    }
    if not args.no_bf16:
        del keep, calls, ws
        torch.cuda.empty_cache()
        line["other_workloads"] = [bf16_workload(max(5, args.steps // 5), 3),
                                   decode_workload(max(20, args.steps), 5),
                                   varlen_workload(max(20, args.steps), 5),
                                   varlen_workload(max(5, args.steps // 5), 3,
                                                   "bf16_b8_L4096_H64_P64_N128_G8_Q256", 512),
                                   block_workload(max(20, args.steps), 5),
                                   bwd_workload(max(10, args.steps // 2), 3),
                                   bwd_workload(max(10, args.steps // 2), 3, dtype="bf16")]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
