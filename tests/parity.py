"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the oracle element by element."""
from contextlib import contextmanager

import numpy as np
import torch

import selective_state_space_ssd_amd as ssd

# Elementwise bars: |gpu - ref| <= tol * (1 + |ref|).  fp32 inputs: 1e-3; bf16
# inputs (fp32 state and accumulation, bf16 output): 2e-2.  The (1 + |ref|)
# form keeps near-zero outputs from inflating relative errors.
TOL = {"f32": 1e-3, "bf16": 2e-2}


# The kernel path the enclosed test calls ask for: a setting of these test
# helpers, passed to every call as its kernel_path argument (the library keeps
# no state).
_PATH = ["auto"]


@contextmanager
def bf16_path(name):
    """Run the enclosed run_gpu calls on kernel path `name` ("chain",
    "chain_segmented", "fused", "fused_head", "fused_group", "staged" or
    "auto")."""
    ssd.path_code(name)  # reject unknown names here
    prev = _PATH[0]
    _PATH[0] = name
    try:
        yield
    finally:
        _PATH[0] = prev


def current_path():
    """The kernel path bf16_path set for the enclosing block."""
    return _PATH[0]


def paths_for(dtype):
    """The kernel paths a problem of this dtype can take."""
    return (("chain", "chain_segmented", "fused_head", "fused_group", "staged") if dtype == "bf16"
            else ("auto",))


def log(msg):
    print(msg, flush=True)


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def upload(inp, dtype):
    """numpy inputs -> dict of device tensors (bf16 from the exact bit patterns)."""
    dev = device()
    t = {}
    for k in ("x", "z", "B", "C", "dt"):
        v = inp.get(k)
        if v is None:
            t[k] = None
        elif dtype == "bf16":
            t[k] = torch.from_numpy(inp["bits"][k].view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)
    for k in ("A", "D", "dt_bias", "initial_states"):
        v = inp.get(k)
        t[k] = None if v is None else torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(dev)
    return t


# Every parity call runs with its workspace filled with 0xFF bytes (a NaN in
# every fp32 and bf16 slot, -1 in every int32 one), its output filled with
# NaN, and canary bytes on both sides of out and final_states that must come
# back untouched: a read of an intermediate nobody wrote, an output element
# nobody wrote, or a store past either end shows up.
GUARD_BYTES = 4096
CANARY = 0x5A


def poisoned_workspace(nbytes, dev):
    return torch.full((max(int(nbytes), 1),), 0xFF, dtype=torch.uint8, device=dev)


def guarded(shape, dtype, dev):
    """(buffer, view): `view` has `shape`, lies GUARD_BYTES into `buffer` and
    is NaN-filled; the GUARD_BYTES before and after it hold CANARY."""
    es = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape))
    g = GUARD_BYTES // es
    buf = torch.empty(n + 2 * g, dtype=dtype, device=dev)
    buf.view(torch.uint8).fill_(CANARY)
    view = buf[g:g + n].view(shape)
    view.fill_(float("nan"))
    return buf, view


def check_guards(buf, name):
    raw = buf.view(torch.uint8)
    head, tail = raw[:GUARD_BYTES], raw[raw.numel() - GUARD_BYTES:]
    assert bool((head == CANARY).all()) and bool((tail == CANARY).all()), \
        f"{name}: bytes outside the tensor were written"


def run_gpu(t, chunk_size, dt_limit=(0.0, float("inf")), init=None, final=True, **kw):
    """One call through the C ABI on the kernel path bf16_path set, with a
    poisoned workspace and guarded outputs unless the caller passes its own."""
    kw.setdefault("kernel_path", current_path())
    kw.setdefault("check_wait", True)  # a fused-path workgroup that gave up waiting fails the call
    x = t["x"]
    dev = x.device
    b, L, H, P = x.shape
    G, N = t["B"].shape[2], t["B"].shape[3]
    guards = []
    if "workspace" not in kw:
        code = 1 if x.dtype == torch.bfloat16 else 0
        size_fn = ssd.varlen_workspace_size if kw.get("seq_idx") is not None else \
            ssd.workspace_size
        kw["workspace"] = poisoned_workspace(
            size_fn(b, L, H, P, N, G, chunk_size, code, kw["kernel_path"]), dev)
    if "out" not in kw:
        buf, kw["out"] = guarded(tuple(x.shape), x.dtype, dev)
        guards.append((buf, "out"))
    if final and "final_states" not in kw:
        buf, kw["final_states"] = guarded((b, H, P, N), torch.float32, dev)
        guards.append((buf, "final_states"))
    res = ssd.scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                       dt_bias=t["dt_bias"], dt_limit=dt_limit, chunk_size=chunk_size,
                       initial_states=init, return_final_states=final, **kw)
    torch.cuda.synchronize()
    for buf, name in guards:
        check_guards(buf, name)
    return res


def np64(t):
    return t.detach().double().cpu().numpy()


def compare(name, got, ref, tol, mask=None):
    """Assert |got - ref| <= tol (1 + |ref|) everywhere (where mask is true);
    report max|diff|, mean(diff), mean|diff| and the worst index."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    diff = got - ref
    scaled = np.abs(diff) / (1.0 + np.abs(ref))
    worst = np.unravel_index(int(np.argmax(scaled)), scaled.shape) if scaled.size else ()
    stats = (f"{name}: n={diff.size} max|d|={np.max(np.abs(diff)) if diff.size else 0:.3e} "
             f"mean(d)={diff.mean() if diff.size else 0:.3e} "
             f"mean|d|={np.abs(diff).mean() if diff.size else 0:.3e} "
             f"max scaled={scaled.max() if scaled.size else 0:.3e} at {worst} (tol {tol})")
    log(stats)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert np.all(scaled <= tol), stats
    return stats


def state_tile_offsets(N):
    """offs[p, n] = float offset of state element (p, n) in a tiled block
    (the workspace layout documented in include/ssd.h; headdim 64)."""
    p = np.arange(64)[:, None]
    n = np.arange(N)[None, :]
    half = N // 2
    k, q, e = n // half, (n % half) // 4, n % 4
    return (((q * 2 + p % 2) * 64) + 32 * k + p // 2) * 4 + e


def ws_regions(ws, b, L, H, P, N, Q):
    """The staged path's intermediates in a workspace (layout of include/ssd.h),
    states untiled to [b, nc, H, P, N]."""
    nc = -(-L // Q)
    r = lambda v: (v + 255) // 256 * 256
    dtn, stn = b * H * nc * Q, b * nc * H * P * N
    f = ws.view(torch.float32)
    o_cum = r(dtn * 4) // 4
    o_st = o_cum + r(dtn * 4) // 4
    o_in = o_st + r(stn * 4) // 4
    offs = torch.from_numpy(state_tile_offsets(N).reshape(-1)).to(ws.device)

    def dense(block):
        return block.view(b, nc, H, P * N)[..., offs].view(b, nc, H, P, N)

    return {"dt": f[:dtn].view(b, H, nc, Q), "cum": f[o_cum:o_cum + dtn].view(b, H, nc, Q),
            "chunk_states": dense(f[o_st:o_st + stn]),
            "states_in": dense(f[o_in:o_in + stn])}
