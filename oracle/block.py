"""Block-level forward around the scan (split, conv1d prologue, gated RMSNorm
epilogue), NumPy fp64 plus the C recurrence for the scan itself.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written from mamba
issue #647's repro script, which calls the fused block
``mamba_split_conv1d_scan_combined`` with a packed in-projection ``zxbcdt``,
a depthwise conv (weight [dim + 2*ngroups*dstate, conv_dim], bias), SiLU
activation, the scan (dt_bias, A, D, dt_limit, chunk_size, ngroups), a gated
RMSNorm (``rmsnorm_weight``, ``rmsnorm_eps``, ``norm_before_gate=False``) and
an out_proj linear.  out_proj is a dense GEMM and not part of this block.

Readings taken where the page is silent:
  * zxbcdt holds, per token, [z (dim) | xBC (dim + 2 G N) | dt (H)], and
    xBC holds [x (dim) | B (G N) | C (G N)] -- the order the argument's name
    spells; dim = nheads * headdim;
  * the conv is causal and depthwise with zeros before the first step, in the
    cross-correlation orientation of a framework Conv1d:
        conv[t, c] = bias[c] + sum_{k=0}^{W-1} w[c, k] * xBC[t - (W-1) + k, c]
    so w[c, W-1] weighs the current step; then SiLU;
  * x, B and C after the conv are tensors of the input dtype (fp32, or bf16
    rounded to nearest even) when the scan reads them;
  * the gate comes before the norm (norm_before_gate=False):
        g = y * silu(z),  out = g / sqrt(mean(g^2) + eps) * weight,
    the mean taken over the whole width (norm_groups = 1) or separately over
    each of norm_groups equal slices of it.  The page's printed outputs fix
    both forms: 17.6951 for the whole width at every ngroups, 18.8725 and
    19.5926 per group at ngroups 2 and 4 (tests/golden).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def _round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _as_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return _round_bf16(a.astype(np.float32))
    if dtype == "f32":
        return a.astype(np.float32)
    raise ValueError(dtype)


def split_conv1d(zxbcdt, conv_weight, conv_bias, nheads, headdim, ngroups, dstate,
                 dtype="f32"):
    """zxbcdt [b, L, 2 dim + 2 G N + H] -> dict of z [b,L,H,P], x [b,L,H,P],
    B, C [b,L,G,N] (the conv + SiLU outputs, held in `dtype`), dt [b,L,H], and
    the fp64 activations ``xbc`` [b, L, dim + 2 G N] before that rounding."""
    zxbcdt = np.asarray(zxbcdt, dtype=np.float64)
    b, L, width = zxbcdt.shape
    dim, gn = nheads * headdim, ngroups * dstate
    assert width == 2 * dim + 2 * gn + nheads
    w = np.asarray(conv_weight, dtype=np.float64)
    nch, W = w.shape
    assert nch == dim + 2 * gn
    z = zxbcdt[..., :dim]
    xbc_in = zxbcdt[..., dim:2 * dim + 2 * gn]
    dt = zxbcdt[..., 2 * dim + 2 * gn:]
    padded = np.concatenate([np.zeros((b, W - 1, nch)), xbc_in], axis=1)
    conv = np.zeros((b, L, nch))
    for k in range(W):
        conv += w[:, k] * padded[:, k:k + L, :]
    if conv_bias is not None:
        conv += np.asarray(conv_bias, dtype=np.float64)
    act = conv * expit(conv)
    held = _as_dtype(act, dtype)
    return {
        "z": z.reshape(b, L, nheads, headdim),
        "x": held[..., :dim].reshape(b, L, nheads, headdim),
        "B": held[..., dim:dim + gn].reshape(b, L, ngroups, dstate),
        "C": held[..., dim + gn:].reshape(b, L, ngroups, dstate),
        "dt": dt,
        "xbc": act,
    }


def gated_rmsnorm(y, z, weight, eps, norm_groups):
    """out = g / sqrt(mean(g^2) + eps) * weight with g = y * silu(z), the mean
    over each of `norm_groups` equal slices of the last axis.  weight None:
    out = g (gate only)."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    g = y * z * expit(z)
    if weight is None:
        return g
    shape = g.shape
    dim = shape[-1]
    assert dim % norm_groups == 0
    parts = g.reshape(shape[:-1] + (norm_groups, dim // norm_groups))
    normed = parts / np.sqrt((parts * parts).mean(axis=-1, keepdims=True) + eps)
    return normed.reshape(shape) * np.asarray(weight, dtype=np.float64)


def split_conv1d_scan(scan_fwd, zxbcdt, conv_weight, conv_bias, dt_bias, A, D, nheads, headdim,
                      ngroups, dstate, rmsnorm_weight=None, eps=1e-5, norm_groups=1,
                      dt_limit=(0.0, float("inf")), initial_states=None, dtype="f32"):
    """The block without out_proj: out [b, L, dim] fp64 and the final state.

    ``scan_fwd`` is the recurrence (``oracle.ssd_fwd`` or a compiled copy of
    it): it runs on x, B, C held in `dtype`, dt straight from zxbcdt, no gate;
    the gate and the norm follow in fp64."""
    parts = split_conv1d(zxbcdt, conv_weight, conv_bias, nheads, headdim, ngroups, dstate, dtype)
    b, L = parts["x"].shape[:2]
    y, fin = scan_fwd(parts["x"], parts["dt"].astype(np.float32), A, parts["B"], parts["C"],
                      D=D, z=None, dt_bias=dt_bias, dt_limit=dt_limit,
                      initial_states=initial_states, return_final_states=True)
    dim = nheads * headdim
    out = gated_rmsnorm(y.reshape(b, L, dim), parts["z"].reshape(b, L, dim), rmsnorm_weight, eps,
                        norm_groups)
    return out, fin
