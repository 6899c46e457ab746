"""C ABI checks that need no GPU.

The library must load and export every function ``include/ssd.h`` declares,
and every rejected argument must come back with its status code before any
HIP call is made.  Fake pointer values are passed; none is ever dereferenced
because every case below fails validation.  No case supplies a workspace of
the needed size unless another argument is invalid, and the workspace is the
last thing validated, so no case can reach a kernel launch.
"""
import ctypes
import glob
import math
import os
import re

import pytest

import selective_state_space_ssd_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP, WAIT = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(ssd_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("ssd_scan_fwd", "ssd_scan_fwd_workspace_size", "ssd_status_string",
                 "ssd_abi_version", "ssd_scan_fwd_timed", "ssd_timing_create",
                 "ssd_timing_read", "ssd_timing_destroy", "ssd_scan_fwd_path",
                 "ssd_scan_fwd_path_workspace_size", "ssd_scan_fwd_wait_status",
                 "ssd_scan_fwd_taken_path", "ssd_scan_fwd_noalloc",
                 "ssd_scan_fwd_varlen", "ssd_scan_fwd_varlen_workspace_size",
                 "ssd_split_conv1d_scan_fwd", "ssd_split_conv1d_scan_fwd_workspace_size",
                 "ssd_scan_bwd", "ssd_scan_bwd_workspace_size"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ssd.binding.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_abi_version_and_status_strings():
    assert ssd.abi_version() == 2
    assert ssd.status_string(0) == "ok"
    seen = {ssd.status_string(s) for s in (INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP, WAIT)}
    assert len(seen) == 6 and "unknown status" not in seen
    assert ssd.status_string(12345) == "unknown status"


def _ws(b, L, H, P, N, G, Q, dt=0, path="auto"):
    return ssd.workspace_size(b, L, H, P, N, G, Q, dt, path)


DECODE_MAX_L = 16  # sequences this short take the step-by-step kernel


def test_short_sequences_need_no_workspace():
    for L in (1, 2, 16):
        assert _ws(2, L, 4, 64, 128, 1, 128) == 0 and _ws(2, L, 4, 64, 128, 1, 256, 1) == 0
    assert _ws(2, 17, 4, 64, 128, 1, 128) > 0


def _r(v):
    return (v + 255) // 256 * 256


def _gram(b, L, H, N, G, Q, bf16):
    """Tiles of B C^T per (chunk, group) for the four-heads chunk scan (chunk
    64/128, dstate 64/128, nheads/ngroups a multiple of 4; bf16 inputs at chunk
    128 take the bf16 kernels instead), formed once per group when at least
    two of its workgroups share them (nheads/ngroups >= 8): Q/32 (Q/32 + 1)/2
    tiles of 32 x 32 fp32."""
    if Q not in (64, 128) or N not in (64, 128) or (H // G) % 4 or (bf16 and Q == 128):
        return 0
    if H // G < 8:
        return 0
    nt = Q // 32
    return _r(b * math.ceil(L / Q) * G * nt * (nt + 1) // 2 * 1024 * 4)


SIZES = [(2, 2048, 32, 64, 128, 1, 128), (1, 300, 4, 64, 16, 1, 64),
         (8, 4096, 64, 64, 128, 8, 256), (3, 1, 2, 64, 32, 2, 128), (1, 200, 4, 64, 64, 2, 64),
         (2, 17, 4, 64, 128, 2, 128), (1, 200, 16, 64, 64, 2, 64),
         (1, 300, 8, 64, 128, 2, 128)]


def test_workspace_size_formula():
    for (b, L, H, P, N, G, Q) in SIZES:
        nc = math.ceil(L / Q)
        want = 2 * _r(b * H * nc * Q * 4) + 2 * _r(b * nc * H * P * N * 4)
        if L <= DECODE_MAX_L:
            assert _ws(b, L, H, P, N, G, Q, 0, "staged") == 0
            assert _ws(b, L, H, P, N, G, Q, 1, "staged") == 0
            continue
        assert _ws(b, L, H, P, N, G, Q, 0, "staged") == want + _gram(b, L, H, N, G, Q, False)
        # intermediates are fp32 for bf16 too; the staged bf16 matrix-core
        # kernels (chunk 128/256, dstate 64/128) add B^T per (chunk, group)
        bt = _r(b * nc * G * N * Q * 2) if (Q in (128, 256) and N in (64, 128)) else 0
        assert _ws(b, L, H, P, N, G, Q, 1, "staged") == want + bt + _gram(b, L, H, N, G, Q, True)


def _fused_ws(b, L, H, P, N):
    """Fused bf16 layout: ring of two states per (batch, head), one flag per
    128-step block, one 256-byte control region."""
    return _r(b * H * 2 * P * N * 4) + _r(b * H * math.ceil(L / 128) * 4) + 256


def _chain_fills(b, H):
    """The chain kernel is the default when its workgroups (head pairs) fill
    each round of 256 compute units at least 3/4."""
    n = b * H // 2
    rounds = -(-n // 256)
    return n > 0 and 4 * n >= 3 * 256 * rounds


def test_workspace_size_fused_bf16():
    """Fused bf16 path (dstate 64/128), asked for explicitly."""
    for path in ("fused", "fused_head", "fused_group"):
        for (b, L, H, P, N, G, Q) in SIZES:
            nc = math.ceil(L / Q)
            staged = 2 * _r(b * H * nc * Q * 4) + 2 * _r(b * nc * H * P * N * 4)
            if L <= DECODE_MAX_L:  # short sequences: the step-by-step kernel, no workspace
                assert _ws(b, L, H, P, N, G, Q, 0, path) == 0
                assert _ws(b, L, H, P, N, G, Q, 1, path) == 0
                continue
            # fp32 is always staged
            assert _ws(b, L, H, P, N, G, Q, 0, path) == staged + _gram(b, L, H, N, G, Q, False)
            want = _fused_ws(b, L, H, P, N) if N in (64, 128) else staged  # dstate 16/32: staged
            if want == staged:
                bt = _r(b * nc * G * N * Q * 2) if Q in (128, 256) else 0
                want += bt + _gram(b, L, H, N, G, Q, True)
            assert _ws(b, L, H, P, N, G, Q, 1, path) == want


def _chain_plan(b, L, H, force):
    """(segments, blocks per segment, blocks per unit, units per head) of the
    chain bf16 path: one segment unless the pairs alone do not fill the 256
    compute units; then as many segments as fill one round (at most one per
    block), by default when they fill it at least 3/4, or from 8 blocks on at
    least half."""
    npairs, nblk = b * H // 2, -(-L // 128)
    if npairs <= 0 or nblk < 2:
        return 1, nblk, 0, 0
    nseg = 256 // npairs
    if force:
        nseg = max(nseg, 2)
    else:
        nseg = min(nseg, nblk)
        full = 4 * npairs * nseg >= 3 * 256
        half_long = nblk >= 8 and 2 * npairs * nseg >= 256
        if nseg < 2 or not (full or half_long):
            return 1, nblk, 0, 0
    nseg = min(nseg, nblk)
    span = -(-nblk // nseg)
    nseg = -(-nblk // span)
    if nseg < 2:
        return 1, nblk, 0, 0
    unit = span
    while unit % 2 == 0 and unit > 8 and npairs * (nseg - 1) * (span // unit) < 1024:
        unit //= 2
    return nseg, span, unit, (nseg - 1) * (span // unit)


def _seg_ws(b, L, H, P, N, force):
    nseg, _, _, nunits = _chain_plan(b, L, H, force)
    return _r(b * H * nunits * P * N * 4) + _r(b * H * nunits * 4) if nseg > 1 else 0


def test_chain_plan():
    assert _chain_plan(1, 65536, 128, False) == (4, 128, 16, 24)   # the long sequence
    assert _chain_plan(8, 4096, 64, False)[0] == 1                 # 256 pairs: no segments
    assert _chain_plan(1, 1000, 8, True) == (8, 1, 1, 7)
    assert _chain_plan(1, 1000, 8, False)[0] == 1                  # a quarter of the CUs
    assert _chain_plan(2, 2048, 32, False) == (8, 2, 2, 7)         # 32 pairs, 16 blocks
    assert _chain_plan(2, 1024, 32, False) == (8, 1, 1, 7)         # one block per segment
    assert _chain_plan(2, 512, 32, False)[0] == 1                  # 4 blocks, half: fused
    assert _chain_plan(8, 512, 32, False) == (2, 2, 2, 1)          # 128 pairs x 2: full
    assert _chain_plan(2, 768, 32, False) == (6, 1, 1, 5)          # 3/4 of the round
    assert _chain_plan(1, 2048, 16, False) == (16, 1, 1, 15)       # half the CUs


def test_workspace_size_default_bf16():
    """Default bf16 path: the chain kernel (no workspace) when the heads of a
    group pair up and the pairs fill the machine, else the fused layout; the
    chain option takes the chain kernel whenever the heads pair up."""
    cases = SIZES + [(8, 4096, 64, 64, 128, 64, 256), (4, 1000, 64, 64, 64, 2, 128),
                     (2, 1000, 6, 64, 128, 2, 128), (6, 1000, 64, 64, 128, 8, 128),
                     (5, 1000, 64, 64, 128, 8, 128), (1, 65536, 128, 64, 128, 8, 256),
                     (12, 500, 64, 64, 128, 8, 128), (13, 500, 64, 64, 128, 8, 128)]
    for (b, L, H, P, N, G, Q) in cases:
        if L <= DECODE_MAX_L or N not in (64, 128):
            continue
        pairs_up = (H // G) % 2 == 0
        chain = pairs_up and _chain_fills(b, H)
        seg = pairs_up and not chain and _chain_plan(b, L, H, False)[0] > 1
        want = 0 if chain else _seg_ws(b, L, H, P, N, False) if seg else _fused_ws(b, L, H, P, N)
        assert _ws(b, L, H, P, N, G, Q, 1) == want
        assert ssd.taken_path(b, L, H, P, N, G, Q, 1) == (
            "chain" if chain else "chain_segmented" if seg else "fused_head")
        assert _ws(b, L, H, P, N, G, Q, 1, "auto") == _ws(b, L, H, P, N, G, Q, 1)
        assert (_ws(b, L, H, P, N, G, Q, 1, "chain")
                == (0 if pairs_up else _fused_ws(b, L, H, P, N)))
        assert (_ws(b, L, H, P, N, G, Q, 1, "chain_segmented")
                == (_seg_ws(b, L, H, P, N, True) if pairs_up else _fused_ws(b, L, H, P, N)))
        assert _ws(b, L, H, P, N, G, Q, 0, "chain") > 0  # fp32 stays staged
    assert _ws(8, 4096, 64, 64, 128, 8, 256, 1) == 0  # the bf16 8 x 4096 workload: chain
    assert _ws(1, 65536, 128, 64, 128, 8, 256, 1) > 0  # the 1 x 65536 one: segmented chain
    assert _chain_fills(6, 64) and not _chain_fills(5, 64)  # 192 of 256 / 160 of 256
    assert _chain_fills(12, 64) and not _chain_fills(11, 64)  # 384 of 512 (3/4) / 352


def test_workspace_size_varlen():
    """Packed-sequence calls: on the staged path the staged layout plus
    [b, nc, Q] int32 sequence-start counts; on the chain and fused bf16 paths
    (headdim 64, dstate 64/128) the plain call's layout; nothing for seqlen
    <= 16."""
    for (b, L, H, P, N, G, Q) in SIZES:
        nc = math.ceil(L / Q)
        staged = 2 * _r(b * H * nc * Q * 4) + 2 * _r(b * nc * H * P * N * 4)
        for dt in (0, 1):
            got = ssd.varlen_workspace_size(b, L, H, P, N, G, Q, dt)
            if L <= DECODE_MAX_L:
                assert got == 0
                continue
            if dt and N in (64, 128):
                assert got == _ws(b, L, H, P, N, G, Q, 1)  # as the plain call
                got = ssd.varlen_workspace_size(b, L, H, P, N, G, Q, dt, "staged")
            bt = _r(b * nc * G * N * Q * 2) if (dt and Q in (128, 256) and N in (64, 128)) else 0
            assert got == staged + bt + _gram(b, L, H, N, G, Q, dt) + _r(b * nc * Q * 4)
    assert ssd.varlen_workspace_size(2, 100, 4, 64, 16, 3, 64, 0) == 0  # rejected shapes


def test_kernel_path_argument():
    """The path is an argument of each call: out-of-range codes are rejected,
    and asking for one path leaves every later query unchanged."""
    lib = ssd.load_library()
    for bad in (-1, 6, 8, 99):
        assert lib.ssd_scan_fwd_path_workspace_size(2, 300, 8, 64, 128, 2, 128, 1, 0, bad) == 0
    before = _ws(1, 65536, 128, 64, 128, 8, 256, 1)
    assert _ws(1, 65536, 128, 64, 128, 8, 256, 1, "chain") == 0
    assert _ws(1, 65536, 128, 64, 128, 8, 256, 1, "staged") > before
    assert _ws(1, 65536, 128, 64, 128, 8, 256, 1) == before
    with pytest.raises(ValueError):
        ssd.path_code("fastest")
    assert _ws(0, 100, 4, 64, 16, 1, 64) == 0
    assert _ws(2, 0, 4, 64, 16, 1, 64) == 0
    assert _ws(2, 100, 4, 64, 16, 3, 64) == 0       # rejected: 3 does not divide 4
    assert _ws(2, 100, 4, 32, 16, 1, 64) == 0       # rejected: headdim 32 not compiled


def test_no_mutable_globals_in_the_abi(tmp_path):
    """The C ABI keeps no state between calls: compiled on its own,
    ssd_api.hip defines no writable data symbol besides the HIP runtime's
    registration handles and the scratch of the allocation-free entry point
    (the array itself and its per-device address table, filled once per
    device)."""
    import shutil
    import subprocess
    from selective_state_space_ssd_amd import _build
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    obj = tmp_path / "ssd_api.o"
    subprocess.run([_build.hipcc(), *_build.CFLAGS, "-c",
                    os.path.join(_build.CSRC, "ssd_api.hip"), "-o", str(obj)], check=True,
                   capture_output=True)
    out = subprocess.run(["nm", "-C", str(obj)], check=True, capture_output=True,
                         text=True).stdout
    data = []
    for line in out.splitlines():
        parts = line.split(None, 2)
        if len(parts) == 3 and parts[1] in "bBdDcCgGsS":
            data.append(parts[2])
    mutable = [d for d in data if not d.startswith("__hip_") and "scratch" not in d]
    assert mutable == [], mutable


# A base argument set with distinct, 256-byte-aligned fake addresses.
BASE = dict(x=0x10000000, dt=0x20000000, A=0x30000000, B=0x40000000, C=0x50000000,
            D=0x60000000, z=0x70000000, dt_bias=0x80000000, dt_min=0.0, dt_max=math.inf,
            chunk_size=64, ngroups=1, init=0x90000000, out=0xA0000000, final=0xB0000000,
            batch=1, seqlen=100, nheads=4, headdim=64, dstate=16, dtype=0, ws=None, ws_bytes=0,
            stream=None)


def call(**changes):
    a = dict(BASE)
    a.update(changes)
    st = ssd.scan_fwd_raw(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"],
                          a["dt_bias"], a["dt_min"], a["dt_max"], a["chunk_size"],
                          a["ngroups"], a["init"], a["out"], a["final"], a["batch"],
                          a["seqlen"], a["nheads"], a["headdim"], a["dstate"], a["dtype"],
                          a["ws"], a["ws_bytes"], a["stream"])
    return st


CASES = [
    ("null x", dict(x=None), INVALID),
    ("null dt", dict(dt=None), INVALID),
    ("null A", dict(A=None), INVALID),
    ("null B", dict(B=None), INVALID),
    ("null C", dict(C=None), INVALID),
    ("null out", dict(out=None), INVALID),
    ("negative batch", dict(batch=-1), INVALID),
    ("negative seqlen", dict(seqlen=-5), INVALID),
    ("zero heads", dict(nheads=0), INVALID),
    ("zero headdim", dict(headdim=0), INVALID),
    ("zero dstate", dict(dstate=0), INVALID),
    ("zero groups", dict(ngroups=0), INVALID),
    ("zero chunk", dict(chunk_size=0), INVALID),
    ("groups do not divide heads", dict(ngroups=3), INVALID),
    ("unknown dtype", dict(dtype=7), INVALID),
    ("dt_min NaN", dict(dt_min=math.nan), INVALID),
    ("dt_max NaN", dict(dt_max=math.nan), INVALID),
    ("dt_min > dt_max", dict(dt_min=0.5, dt_max=0.1), INVALID),
    ("headdim 32", dict(headdim=32), UNSUPPORTED),
    ("dstate 256", dict(dstate=256), UNSUPPORTED),
    ("dstate 24", dict(dstate=24), UNSUPPORTED),
    ("chunk 32", dict(chunk_size=32), UNSUPPORTED),
    ("chunk 100", dict(chunk_size=100), UNSUPPORTED),
    ("too many chunks", dict(seqlen=64 * 65536), UNSUPPORTED),
    # rows of B/C wider than 2^22 elements (32-bit byte offsets over 256 steps)
    ("B row too wide", dict(nheads=65535, ngroups=65535, dstate=128), UNSUPPORTED),
    ("x misaligned", dict(x=0x10000004), ALIGN),
    ("out misaligned", dict(out=0xA0000008), ALIGN),
    ("B misaligned", dict(B=0x40000002), ALIGN),
    ("C misaligned", dict(C=0x50000004), ALIGN),
    ("z misaligned", dict(z=0x70000004), ALIGN),
    ("dt misaligned fp32", dict(dt=0x20000002), ALIGN),
    ("dt misaligned bf16", dict(dt=0x20000001, dtype=1), ALIGN),
    ("A misaligned", dict(A=0x30000002), ALIGN),
    ("init misaligned", dict(init=0x90000004), ALIGN),
    ("final misaligned", dict(final=0xB0000004), ALIGN),
    ("out overlaps x", dict(out=0x10000000 + 256), INVALID),
    ("out overlaps z", dict(out=0x70000000 - 256), INVALID),
    ("out overlaps B", dict(out=0x40000000), INVALID),
    ("out overlaps final", dict(final=0xA0000000 + 1024), INVALID),
    ("final partially overlaps init", dict(final=0x90000000 + 4096), INVALID),
    ("out overlaps initial_states", dict(out=0x90000000 + 512), INVALID),
    ("out overlaps A", dict(out=0x30000000 - 256), INVALID),
    ("out overlaps D", dict(out=0x60000000 - 64), INVALID),
    ("out overlaps dt_bias", dict(out=0x80000000 - 16), INVALID),
    ("out overlaps workspace", dict(ws=0xA0000000 + 4096, ws_bytes=16), INVALID),
    ("final overlaps x", dict(final=0x10000000 + 1024), INVALID),
    ("final overlaps dt", dict(final=0x20000000 - 256), INVALID),
    ("final overlaps B", dict(final=0x40000000), INVALID),
    ("final overlaps C", dict(final=0x50000000 + 16), INVALID),
    ("final overlaps z", dict(final=0x70000000 + 4096), INVALID),
    ("final overlaps A", dict(final=0x30000000 - 16), INVALID),
    ("final overlaps workspace", dict(ws=0xB0000000 - 256, ws_bytes=512), INVALID),
    ("no workspace", dict(), WORKSPACE),
    ("workspace too small", dict(ws=0xC0000000, ws_bytes=1024), WORKSPACE),
    ("final aliases init exactly (valid, stops at workspace)", dict(final=0x90000000),
     WORKSPACE),
    ("bf16 dt 2-byte aligned (valid, stops at workspace)", dict(dt=0x20000002, dtype=1),
     WORKSPACE),
    ("optional pointers absent (valid, stops at workspace)",
     dict(D=None, z=None, dt_bias=None, init=None, final=None), WORKSPACE),
]


@pytest.mark.parametrize("desc,changes,want", CASES, ids=[c[0] for c in CASES])
def test_rejected_before_launch(desc, changes, want):
    assert want != OK
    assert call(**changes) == want


def call_path(path, seq=None, **changes):
    a = dict(BASE)
    a.update(changes)
    return ssd.scan_fwd_path_raw(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                 a["dt_bias"], a["dt_min"], a["dt_max"], a["chunk_size"],
                                 a["ngroups"], a["init"], a["out"], a["final"], seq, a["batch"],
                                 a["seqlen"], a["nheads"], a["headdim"], a["dstate"], a["dtype"],
                                 path, a["ws"], a["ws_bytes"], a["stream"])


def test_path_entry_point_rejections():
    """ssd_scan_fwd_path validates like ssd_scan_fwd, and the path code too."""
    for bad in (-1, 6, 8, 1000):
        assert call_path(bad) == INVALID
    for name, code in ssd.KERNEL_PATHS.items():
        assert call_path(code) == WORKSPACE, name            # valid, stops at workspace
        assert call_path(code, ngroups=3) == INVALID, name
        assert call_path(code, x=0x10000004) == ALIGN, name
    bf = dict(dtype=1, dstate=128, chunk_size=256, seqlen=1000, nheads=8, ngroups=2)
    need = ssd.workspace_size(1, 1000, 8, 64, 128, 2, 256, 1, "fused_head")
    assert need > 0
    assert call_path(3, ws=0xC0000000, ws_bytes=need - 1, **bf) == WORKSPACE
    # seq_idx on the path entry point: packed-sequence rules apply
    assert call_path(0, seq=0xD0000002) == ALIGN


def test_taken_path():
    """The path each call takes, after the documented fallbacks."""
    tp = ssd.taken_path
    assert tp(8, 4096, 64, 64, 128, 8, 256, 1) == "chain"           # pairs fill the machine
    assert tp(1, 65536, 128, 64, 128, 8, 256, 1) == "chain_segmented"  # 64 pairs x 4 segments
    assert tp(1, 1000, 8, 64, 128, 2, 256, 1) == "fused_head"       # too few pairs to segment
    assert tp(2, 2048, 32, 64, 128, 1, 256, 1) == "chain_segmented"  # 32 pairs x 8 segments
    assert tp(2, 512, 32, 64, 128, 1, 256, 1) == "fused_head"       # 4 blocks, half the CUs
    assert tp(8, 512, 32, 64, 128, 4, 256, 1) == "chain_segmented"  # 128 pairs x 2 segments
    assert tp(2, 2048, 32, 64, 128, 1, 128, 0) == "staged_scan"     # fp32, one round
    assert tp(4, 2048, 32, 64, 128, 1, 128, 0) == "staged_scan"     # 64-column slices
    assert tp(8, 2048, 32, 64, 128, 1, 128, 0) == "staged"          # two rounds even so
    assert tp(2, 2048, 32, 64, 64, 4, 64, 0) == "staged_scan"       # half the units
    assert tp(1, 2048, 32, 64, 64, 4, 64, 0) == "staged"            # a quarter
    assert tp(2, 8192, 32, 64, 128, 1, 128, 0) == "staged"          # 64 chunks
    assert tp(2, 4096, 32, 64, 128, 1, 128, 0) == "staged_scan"     # 32 chunks
    assert tp(2, 2048, 32, 64, 32, 1, 128, 0) == "staged"           # dstate 32
    assert tp(2, 2048, 32, 64, 128, 1, 256, 0) == "staged"          # chunk 256
    assert tp(2, 2048, 32, 64, 128, 1, 128, 0, varlen=True) == "staged_scan"  # packed too
    assert tp(2, 16, 32, 64, 128, 1, 128, 1) == "step"              # seqlen <= 16
    assert tp(2, 400, 6, 64, 128, 2, 256, 1, kernel_path="chain") == "fused_head"  # odd group
    assert tp(2, 400, 8, 64, 16, 2, 256, 1, kernel_path="chain") == "staged"       # dstate 16
    assert tp(2, 400, 8, 64, 128, 2, 256, 1, kernel_path="fused_group") == "fused_group"
    assert tp(2, 400, 8, 64, 128, 2, 256, 1, True, "fused_group") == "fused_head"  # packed
    assert tp(2, 400, 8, 64, 128, 2, 256, 0, kernel_path="chain") == "staged"      # fp32
    with pytest.raises(ssd.SsdError):
        tp(2, 400, 8, 64, 128, 3, 256, 1)


def test_wait_status_rejections_without_gpu():
    """Shape and path checks come before any HIP call."""
    lib = ssd.load_library()
    assert lib.ssd_scan_fwd_wait_status(None, 0, 1, 100, 4, 64, 16, 3, 64, 0, 0, 0, None) == INVALID
    assert lib.ssd_scan_fwd_wait_status(None, 0, 1, 100, 4, 64, 16, 1, 64, 0, 0, 9, None) == INVALID
    assert lib.ssd_scan_fwd_wait_status(None, 0, 1, 100, 4, 32, 16, 1, 64, 0, 0, 0, None) == \
        UNSUPPORTED


def call_noalloc(**changes):
    a = dict(BASE)
    a.update(changes)
    return ssd.scan_fwd_noalloc_raw(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                    a["dt_bias"], a["dt_min"], a["dt_max"], a["chunk_size"],
                                    a["ngroups"], a["init"], a["out"], a["final"], a["batch"],
                                    a["seqlen"], a["nheads"], a["headdim"], a["dstate"],
                                    a["dtype"], a["stream"])


NOALLOC_CASES = [c for c in CASES if c[2] != WORKSPACE and "workspace" not in c[0]]


@pytest.mark.parametrize("desc,changes,want", NOALLOC_CASES, ids=[c[0] for c in NOALLOC_CASES])
def test_noalloc_rejected_before_launch(desc, changes, want):
    """The allocation-free entry point checks every argument as ssd_scan_fwd
    does, before any HIP call (no case here is valid)."""
    assert call_noalloc(**changes) == want


def test_noalloc_empty_and_too_large():
    assert call_noalloc(batch=0) == OK
    # one fp32 row of 65536 steps x 32 heads x 64 x 128 needs ~2.2 GB of
    # intermediates on the staged path: more than the scratch holds
    far = {k: (i + 1) << 34 for i, k in enumerate(("x", "dt", "A", "B", "C", "D", "z", "dt_bias",
                                                   "init", "out", "final"))}
    assert call_noalloc(seqlen=65536, nheads=32, dstate=128, chunk_size=128, **far) == WORKSPACE


def call_varlen(seq=0xD0000000, **changes):
    a = dict(BASE)
    a.update(changes)
    return ssd.scan_fwd_varlen_raw(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                   a["dt_bias"], a["dt_min"], a["dt_max"], a["chunk_size"],
                                   a["ngroups"], a["init"], a["out"], a["final"], seq,
                                   a["batch"], a["seqlen"], a["nheads"], a["headdim"],
                                   a["dstate"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


VARLEN_CASES = [
    ("seq_idx missing", dict(seq=None), INVALID),
    ("seq_idx misaligned", dict(seq=0xD0000002), ALIGN),
    ("out overlaps seq_idx", dict(seq=0xA0000000 + 64), INVALID),
    ("shape checks as ssd_scan_fwd", dict(ngroups=3), INVALID),
    ("valid, stops at workspace", dict(), WORKSPACE),
    ("bf16 fused shape, workspace one byte short", dict(dtype=1, dstate=128, chunk_size=128,
     ws=0xC0000000, ws_bytes=ssd.workspace_size(1, 100, 4, 64, 128, 1, 128, 1) - 1), WORKSPACE),
]


@pytest.mark.parametrize("desc,changes,want", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_varlen_rejected_before_launch(desc, changes, want):
    assert call_varlen(**changes) == want


def test_workspace_size_block():
    """Block calls: x [b,L,H,P], B and C [b,L,G,N], dt [b,L,H] in the input
    dtype, then the scan's workspace for the same problem."""
    for (b, L, H, P, N, G, Q) in SIZES:
        for dt in (0, 1):
            es = 2 if dt else 4
            pre = (_r(b * L * H * P * es) + 2 * _r(b * L * G * N * es) + _r(b * L * H * es))
            want = pre + _ws(b, L, H, P, N, G, Q, dt)
            assert ssd.block_workspace_size(b, L, H, P, N, G, Q, dt, 4, 1) == want
    assert ssd.block_workspace_size(2, 100, 4, 64, 16, 1, 64, 0, 5, 1) == 0   # conv width 5
    assert ssd.block_workspace_size(2, 100, 4, 64, 16, 1, 64, 0, 4, 3) == 0   # 3 does not divide 256
    assert ssd.block_workspace_size(2, 100, 256, 64, 16, 1, 64, 0, 4, 1) == 0  # dim 16384 > 15360
    assert ssd.block_workspace_size(0, 100, 4, 64, 16, 1, 64, 0, 4, 1) == 0


BLOCK = dict(zx=0x10000000, cw=0x20000000, cb=0x30000000, dt_bias=0x40000000, A=0x50000000,
             D=0x60000000, Q=64, init=None, dt_min=0.0, dt_max=math.inf, nw=0x70000000,
             eps=1e-5, P=64, G=1, ng=1, out=0x80000000, final=None, b=1, L=100, H=4, N=16,
             W=4, dtype=0, ws=None, ws_bytes=0, stream=None)


def call_block(**changes):
    a = dict(BLOCK)
    a.update(changes)
    return ssd.split_conv1d_scan_fwd_raw(a["zx"], a["cw"], a["cb"], a["dt_bias"], a["A"], a["D"],
                                         a["Q"], a["init"], a["dt_min"], a["dt_max"], a["nw"],
                                         a["eps"], a["P"], a["G"], a["ng"], a["out"], a["final"],
                                         a["b"], a["L"], a["H"], a["N"], a["W"], a["dtype"],
                                         a["ws"], a["ws_bytes"], a["stream"])


BLOCK_CASES = [
    ("conv width 5", dict(W=5), UNSUPPORTED),
    ("conv width 1", dict(W=1), UNSUPPORTED),
    ("norm groups do not divide dim", dict(ng=3), UNSUPPORTED),
    ("negative eps", dict(eps=-1.0), INVALID),
    ("NaN eps", dict(eps=math.nan), INVALID),
    ("null zxbcdt", dict(zx=None), INVALID),
    ("null conv weight", dict(cw=None), INVALID),
    ("null A", dict(A=None), INVALID),
    ("out misaligned", dict(out=0x80000008), ALIGN),
    ("conv weight misaligned", dict(cw=0x20000002), ALIGN),
    ("norm weight not 16-byte aligned", dict(nw=0x70000004), ALIGN),
    ("out overlaps zxbcdt", dict(out=0x10000000 + 4096), INVALID),
    ("groups do not divide heads", dict(G=3), INVALID),
    ("no workspace", dict(), WORKSPACE),
    ("valid without bias, weight or D (stops at workspace)", dict(cb=None, nw=None, D=None),
     WORKSPACE),
    ("eps ignored without a weight (stops at workspace)", dict(nw=None, eps=-1.0), WORKSPACE),
]


@pytest.mark.parametrize("desc,changes,want", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_rejected_before_launch(desc, changes, want):
    assert call_block(**changes) == want


def test_workspace_size_backward():
    """dt, cum [b, H, nb, 64]; two state arrays and G [b, nb, H, P N]; y/dY
    [b, L, H, P]; dB and dC parts [b, L, H, N]; dA and dD parts [b, nb, H];
    nb = ceil(L / 64) whatever the chunk size.  bf16 adds fp32 copies of x,
    dt, B, C, z, dout and fp32 buffers for dx, ddt, dB, dC, dz."""
    for (b, L, H, P, N, G, Q) in SIZES:
        nb = math.ceil(L / 64)
        st = _r(b * nb * H * P * N * 4)
        want = (2 * _r(b * H * nb * 64 * 4) + 3 * st + _r(b * L * H * P * 4) +
                2 * _r(b * L * H * N * 4) + 2 * _r(b * nb * H * 4))
        assert ssd.bwd_workspace_size(b, L, H, P, N, G, Q, 0) == want
        xn, ndt, gn = b * L * H * P, b * L * H, b * L * G * N
        wide = 5 * _r(xn * 4) + 2 * _r(ndt * 4) + 4 * _r(gn * 4)
        assert ssd.bwd_workspace_size(b, L, H, P, N, G, Q, 1) == want + wide


BWD = dict(x=0x10000000, dt=0x11000000, A=0x12000000, B=0x13000000, C=0x14000000,
           D=0x15000000, z=0x16000000, dt_bias=0x17000000, init=None, dout=0x18000000,
           dfinal=None, dx=0x20000000, ddt=0x21000000, dA=0x22000000, dB=0x23000000,
           dC=0x24000000, dD=0x25000000, dz=0x26000000, ddt_bias=0x27000000, dinit=None,
           b=1, L=100, H=4, P=64, N=16, G=1, Q=64, dtype=0, ws=None, ws_bytes=0)


def call_bwd(**changes):
    a = dict(BWD)
    a.update(changes)
    return ssd.scan_bwd_raw(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["dt_bias"],
                            0.0, math.inf, a["Q"], a["G"], a["init"], a["dout"], a["dfinal"],
                            a["dx"], a["ddt"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
                            a["ddt_bias"], a["dinit"], a["b"], a["L"], a["H"], a["P"], a["N"],
                            a["dtype"], a["ws"], a["ws_bytes"], None)


BWD_CASES = [
    ("bf16 (stops at workspace)", dict(dtype=1), WORKSPACE),
    ("bf16 dt on an odd address", dict(dtype=1, dt=0x11000001), ALIGN),
    ("f32 ddt 2-byte aligned", dict(ddt=0x21000002), ALIGN),
    ("bf16 dx overlaps x", dict(dtype=1, dx=0x10000000 + 100 * 4 * 64 * 2 - 16), INVALID),
    ("D given without dD", dict(dD=None), INVALID),
    ("dz without z", dict(z=None), INVALID),
    ("dt_bias without ddt_bias", dict(ddt_bias=None), INVALID),
    ("null dout", dict(dout=None), INVALID),
    ("null dA", dict(dA=None), INVALID),
    ("dx misaligned", dict(dx=0x20000004), ALIGN),
    ("dB misaligned", dict(dB=0x23000008), ALIGN),
    ("dx overlaps x", dict(dx=0x10000000 + 1024), INVALID),
    ("dB overlaps dC", dict(dB=0x24000000 - 256), INVALID),
    ("ddt overlaps dout", dict(ddt=0x18000000 + 64), INVALID),
    ("headdim 32", dict(P=32), UNSUPPORTED),
    ("no workspace", dict(), WORKSPACE),
    ("options absent (stops at workspace)",
     dict(D=None, dD=None, z=None, dz=None, dt_bias=None, ddt_bias=None), WORKSPACE),
]


@pytest.mark.parametrize("desc,changes,want", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_rejected_before_launch(desc, changes, want):
    assert call_bwd(**changes) == want


def test_empty_batch_is_a_no_op():
    # batch == 0: nothing to compute, nothing launched
    assert call(batch=0) == OK
    assert call(batch=0, x=None, dt=None, B=None, C=None, out=None) == OK


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        ssd.scan_fwd(x, torch.zeros(1, 4, 2), torch.zeros(2), torch.zeros(1, 4, 1, 16),
                     torch.zeros(1, 4, 1, 16))
