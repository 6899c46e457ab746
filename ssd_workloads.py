"""Seeded synthetic inputs for the SSD scan forward.

This module is the only thing the oracle side and the HIP side share.  It
draws random numbers and rounds them to the input dtype; it holds none of the
method's arithmetic.

Distributions (the same for every workload unless stated):
  x, z, B, C ~ N(0, 1);  dt_raw ~ N(0, 1);
  dt_bias = softplus^{-1}(U(1e-3, 1e-1)) = log(expm1(u)), so softplus(dt_bias)
            lies in [1e-3, 1e-1];
  A = -exp(U(0, log 16)) (so A in [-16, -1]);  D ~ N(0, 1);
  initial states (when asked for) ~ N(0, 1).
The long bf16 sequence draws dt_raw = softplus^{-1}(U(1e-3, 1e-1)) per
(b, t, h) with dt_bias = 0, so dt lies in [1e-3, 1e-1] up to bf16 rounding.

Draw order from one numpy PCG64 generator: x, z, B, C, dt_raw, dt_bias, A, D,
initial states.  Everything is drawn in float32; bf16 workloads round x, z,
B, C and dt_raw to bf16 (round to nearest even) and keep the rounded values,
so both sides consume identical numbers.  A, D, dt_bias and states stay fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    dtype: str                 # "f32" or "bf16": dtype of x, dt, B, C, z, out
    seed: int
    gate: bool = True          # z given
    skip: bool = True          # D given
    dt_uniform: bool = False   # dt_raw = softplus^-1(U(1e-3,1e-1)), dt_bias = 0
    init: bool = False         # draw initial states
    final: bool = False        # return final states
    segments: int = 1          # continuation: the sequence is scanned in this many calls
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five workloads the scan is measured and checked on.
WORKLOADS = {
    "f32_b1_L256_H4_P64_N16_G1_Q64": Workload(
        "f32_b1_L256_H4_P64_N16_G1_Q64", 1, 256, 4, 64, 16, 1, 64, "f32", seed=1),
    "f32_b2_L2048_H32_P64_N128_G1_Q128": Workload(
        "f32_b2_L2048_H32_P64_N128_G1_Q128", 2, 2048, 32, 64, 128, 1, 128, "f32", seed=2),
    "f32_b2_L2048_H32_P64_N128_G2_Q128": Workload(
        "f32_b2_L2048_H32_P64_N128_G2_Q128", 2, 2048, 32, 64, 128, 2, 128, "f32", seed=2),
    "f32_b2_L2048_H32_P64_N128_G4_Q128": Workload(
        "f32_b2_L2048_H32_P64_N128_G4_Q128", 2, 2048, 32, 64, 128, 4, 128, "f32", seed=2),
    "bf16_b8_L4096_H64_P64_N128_G8_Q256": Workload(
        "bf16_b8_L4096_H64_P64_N128_G8_Q256", 8, 4096, 64, 64, 128, 8, 256, "bf16", seed=3,
        final=True),
    "f32_b4_L8192x4seg_H32_P64_N128_G1_Q128": Workload(
        "f32_b4_L8192x4seg_H32_P64_N128_G1_Q128", 4, 8192, 32, 64, 128, 1, 128, "f32", seed=4,
        final=True, segments=4),
    "bf16_b1_L65536_H128_P64_N128_G8_Q256": Workload(
        "bf16_b1_L65536_H128_P64_N128_G8_Q256", 1, 65536, 128, 64, 128, 8, 256, "bf16", seed=5,
        gate=False, dt_uniform=True),
}

# The measured workload: fp32, batch 2, seqlen 2048, 32 heads of 64, dstate 128,
# chunk 128, run at ngroups 1, 2 and 4.
BENCH_WORKLOADS = (
    "f32_b2_L2048_H32_P64_N128_G1_Q128",
    "f32_b2_L2048_H32_P64_N128_G2_Q128",
    "f32_b2_L2048_H32_P64_N128_G4_Q128",
)


def small(name: str, **changes) -> Workload:
    """A workload with some fields replaced (used for reduced-size cases)."""
    return replace(WORKLOADS[name], **changes)


def round_bf16(a: np.ndarray):
    """Round float32 to bf16, nearest-even.  Returns (bits uint16, values float32)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    bits = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits, vals


def _inv_softplus(u: np.ndarray) -> np.ndarray:
    return np.log(np.expm1(u.astype(np.float64))).astype(np.float32)


def make_inputs(w: Workload) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict of float32 arrays ``x, z, B, C, dt, dt_bias, A, D,
    initial_states`` (absent ones are None) holding the exact input values, and
    for bf16 workloads ``bits``: a dict of the uint16 bf16 patterns of x, z, B,
    C, dt, for upload."""
    rng = np.random.default_rng(w.seed)
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    f32 = np.float32
    x = rng.standard_normal((b, L, H, P), dtype=f32)
    z = rng.standard_normal((b, L, H, P), dtype=f32) if w.gate else None
    B = rng.standard_normal((b, L, G, N), dtype=f32)
    C = rng.standard_normal((b, L, G, N), dtype=f32)
    if w.dt_uniform:
        dt = _inv_softplus(rng.uniform(1e-3, 1e-1, size=(b, L, H)))
        dt_bias = np.zeros((H,), dtype=f32)
    else:
        dt = rng.standard_normal((b, L, H), dtype=f32)
        dt_bias = _inv_softplus(rng.uniform(1e-3, 1e-1, size=(H,)))
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=(H,)))).astype(f32)
    D = rng.standard_normal((H,), dtype=f32) if w.skip else None
    init = rng.standard_normal((b, H, P, N), dtype=f32) if w.init else None
    out = {"x": x, "z": z, "B": B, "C": C, "dt": dt, "dt_bias": dt_bias, "A": A, "D": D,
           "initial_states": init}
    if w.dtype == "bf16":
        bits = {}
        for k in ("x", "z", "B", "C", "dt"):
            if out[k] is not None:
                bits[k], out[k] = round_bf16(out[k])
        out["bits"] = bits
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype}")
    return out


def make_seq_idx(batch: int, seqlen: int, mean_len: float, seed: int) -> np.ndarray:
    """Labels of packed sequences, int32 [batch, seqlen].

    Each row is filled with sequences whose lengths are drawn uniformly from
    [1, 2*mean_len - 1] (the last one cut at the row end), labelled 0, 1, 2,
    ... in order.  A generator of its own (seeded by ``seed``), so drawing
    labels leaves every other input unchanged."""
    rng = np.random.default_rng(seed)
    hi = max(1, int(round(2 * mean_len - 1)))
    out = np.empty((batch, seqlen), dtype=np.int32)
    for b in range(batch):
        t, label = 0, 0
        while t < seqlen:
            n = int(rng.integers(1, hi + 1))
            out[b, t:t + n] = label
            t += n
            label += 1
    return out


def random_small(seed: int, batch=2, seqlen=37, nheads=4, headdim=8, dstate=4, ngroups=2,
                 gate=True, skip=True, init=False, dtype="f32") -> dict:
    """Small inputs with the same distributions, for oracle self-tests."""
    w = Workload("small", batch, seqlen, nheads, headdim, dstate, ngroups, 16, dtype, seed,
                 gate=gate, skip=skip, init=init)
    return make_inputs(w)
