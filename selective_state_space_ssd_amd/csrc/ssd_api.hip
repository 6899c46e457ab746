// C ABI of the SSD scan forward: argument checks, workspace layout and the
// launch sequence.  Declarations and the contract are in include/ssd.h.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>

#include "ssd.h"
#include "ssd_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [p, p + n) of a tensor; used for overlap checks.
struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + (uintptr_t)bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// Multiply non-negative sizes, failing on int64 overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Layout {
  int64_t nc = 0;
  bool decode = false;  // seqlen <= kDecodeMaxL: step-by-step kernel, no workspace
  bool fused = false;
  bool chain = false;  // chain bf16 kernel: no workspace unless segmented
  ssd::ChainPlan plan;
  size_t off_cs_states = 0, off_cs_decay = 0;
  // staged path (off_seg: packed-sequence counts, varlen calls only)
  // (off_gram: tiles of B C^T for the four-heads chunk scan, ssd::use_gram)
  size_t off_dt = 0, off_cum = 0, off_states = 0, off_states_in = 0, off_bt = 0, off_seg = 0;
  size_t off_gram = 0;
  bool gram = false;
  // fused bf16 path
  size_t off_ring = 0, off_flags = 0, off_ctl = 0;
  size_t total = 0;
  int path = SSD_PATH_AUTO;  // the kernel path the call asked for (SSD_PATH_*)
};

constexpr int64_t kMaxRowElems = ((int64_t)1 << 32) / (256 * 4);

// The staged bf16 matrix-core kernels (same rule as ssd::use_bf16_kernels).
bool bf16_path(int dtype, int64_t dstate, int chunk_size) {
  return dtype == SSD_BF16 && (chunk_size == 128 || chunk_size == 256) &&
         (dstate == 64 || dstate == 128);
}

// The fused bf16 kernel (same rule as ssd::use_fused_bf16), unless the call
// asks for the staged path.
bool fused_path(int dtype, int64_t headdim, int64_t dstate, int path) {
  return dtype == SSD_BF16 && headdim == 64 && (dstate == 64 || dstate == 128) &&
         path != SSD_PATH_STAGED;
}

// The chain bf16 kernel: asked for, or chosen by SSD_PATH_AUTO when the head
// pairs fill the machine, or (segmented) when pairs times segments do (same
// shape rule as ssd::use_chain_bf16).  Fills *plan.
bool chain_path(int dtype, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                int64_t dstate, int ngroups, int path, ssd::ChainPlan* plan) {
  const bool shape = dtype == SSD_BF16 && headdim == 64 && (dstate == 64 || dstate == 128) &&
                     (nheads / ngroups) % 2 == 0;
  if (!shape) return false;
  *plan = ssd::ChainPlan{};
  plan->span = (seqlen + 127) / 128;
  if (path == SSD_PATH_CHAIN) return true;
  if (path == SSD_PATH_CHAIN_SEGMENTED) {
    *plan = ssd::chain_plan(batch, seqlen, nheads, true);
    return true;
  }
  if (path != SSD_PATH_AUTO) return false;
  if (ssd::chain_fills_machine(batch, nheads)) return true;
  *plan = ssd::chain_plan(batch, seqlen, nheads, false);
  return plan->nseg > 1;
}

bool path_valid(int path) {
  return (path >= SSD_PATH_AUTO && path <= SSD_PATH_CHAIN) || path == SSD_PATH_CHAIN_SEGMENTED;
}

// Shape checks shared by the workspace query and the entry point.
// varlen: the call carries seq_idx (packed sequences).  On the staged path its
// workspace ends with the per-chunk sequence-start counts; the fused bf16
// kernel counts the starts itself.
int check_shapes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int ngroups, int chunk_size, int dtype, bool varlen, int path, Layout* lay) {
  if (!path_valid(path)) return SSD_ERR_INVALID_ARG;
  lay->path = path;
  if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
      chunk_size <= 0)
    return SSD_ERR_INVALID_ARG;
  if (nheads % ngroups != 0) return SSD_ERR_INVALID_ARG;
  if (dtype != SSD_F32 && dtype != SSD_BF16) return SSD_ERR_INVALID_ARG;
  if (!ssd::config_supported(headdim, dstate, chunk_size)) return SSD_ERR_UNSUPPORTED;
  const int64_t nc = (seqlen + chunk_size - 1) / chunk_size;
  // every element count must fit in int64 and every grid in its limits
  int64_t t1, t2, t3, pn, per_chunk;
  if (!mul_ok(batch, seqlen, &t1) || !mul_ok(t1, nheads, &t2) || !mul_ok(t2, headdim, &t3))
    return SSD_ERR_INVALID_ARG;
  if (!mul_ok(t1, ngroups, &t2) || !mul_ok(t2, dstate, &t3)) return SSD_ERR_INVALID_ARG;
  if (!mul_ok(headdim, dstate, &pn) || !mul_ok(pn, nheads, &per_chunk)) return SSD_ERR_INVALID_ARG;
  int64_t units;
  if (!mul_ok(batch, nc, &t1) || !mul_ok(t1, nheads, &units)) return SSD_ERR_INVALID_ARG;
  if (units > INT32_MAX || nc > 65535 || batch > 65535 || nheads > 65535)
    return SSD_ERR_UNSUPPORTED;
  // the kernels address a chunk's (or 256-step block's) rows of x, z, out and
  // of B, C with 32-bit byte offsets: a row may hold at most 2^32 / (256 * 4)
  // elements
  if (nheads * headdim > kMaxRowElems || (int64_t)ngroups * dstate > kMaxRowElems)
    return SSD_ERR_UNSUPPORTED;
  int64_t dtn, stn;
  if (!mul_ok(units, chunk_size, &dtn) || !mul_ok(units, pn, &stn)) return SSD_ERR_INVALID_ARG;
  if (stn > INT64_MAX / 8) return SSD_ERR_INVALID_ARG;
  lay->nc = nc;
  if (ssd::use_decode(seqlen)) {
    lay->decode = true;
    lay->total = 0;
    return SSD_OK;
  }
  if (seqlen > 0 && batch > 0 &&
      chain_path(dtype, batch, seqlen, nheads, headdim, dstate, ngroups, path, &lay->plan)) {
    lay->chain = true;
    lay->total = 0;
    if (lay->plan.nseg > 1) {  // unit end states and decays of the unit-state pass
      int64_t units, stn;
      if (!mul_ok(batch * nheads, lay->plan.nunits, &units) || !mul_ok(units, pn, &stn))
        return SSD_ERR_INVALID_ARG;
      if (units > INT32_MAX) return SSD_ERR_UNSUPPORTED;
      lay->off_cs_states = 0;
      lay->off_cs_decay = round_up((size_t)stn * 4);
      lay->total = lay->off_cs_decay + round_up((size_t)units * 4);
    }
    return SSD_OK;
  }
  if (fused_path(dtype, headdim, dstate, path) && seqlen > 0 && batch > 0) {
    const int64_t nblk = ssd::fused_blocks(seqlen);
    int64_t nchain, grid, ringn, flagn;
    if (!mul_ok(batch, nheads, &nchain) || !mul_ok(nchain, nblk, &grid) ||
        !mul_ok(nchain, 2 * pn, &ringn) || !mul_ok(nchain, nblk, &flagn))
      return SSD_ERR_INVALID_ARG;
    if (grid > INT32_MAX || ringn > INT64_MAX / 8) return SSD_ERR_UNSUPPORTED;
    lay->fused = true;
    lay->off_ring = 0;
    lay->off_flags = round_up((size_t)ringn * 4);
    lay->off_ctl = lay->off_flags + round_up((size_t)flagn * 4);
    lay->total = lay->off_ctl + kAlign;
    return SSD_OK;
  }
  lay->off_dt = 0;
  lay->off_cum = round_up((size_t)dtn * 4);
  lay->off_states = lay->off_cum + round_up((size_t)dtn * 4);
  lay->off_states_in = lay->off_states + round_up((size_t)stn * 4);
  lay->off_bt = lay->off_states_in + round_up((size_t)stn * 4);
  lay->total = lay->off_bt;
  if (bf16_path(dtype, dstate, chunk_size)) {
    int64_t btn;
    if (!mul_ok(batch * nc * ngroups, dstate * chunk_size, &btn)) return SSD_ERR_INVALID_ARG;
    lay->total += round_up((size_t)btn * 2);
  }
  if (ssd::use_gram(nheads, dstate, ngroups, chunk_size, dtype == SSD_BF16)) {
    int64_t gramn;
    if (!mul_ok(batch * nc * ngroups, ssd::gram_tile_floats(chunk_size), &gramn))
      return SSD_ERR_INVALID_ARG;
    // the state-passing launch adds grid planes for the tiles; past the
    // grid's limit the chunk scan forms them itself
    if (ssd::gram_planes(batch, nc, nheads, dstate, ngroups, chunk_size) + batch <= 65535) {
      lay->gram = true;
      lay->off_gram = lay->total;
      lay->total += round_up((size_t)gramn * 4);
    }
  }
  if (varlen) {
    int64_t segn;
    if (!mul_ok(batch * nc, chunk_size, &segn)) return SSD_ERR_INVALID_ARG;
    lay->off_seg = lay->total;
    lay->total += round_up((size_t)segn * 4);
  }
  if (batch == 0 || seqlen == 0) lay->total = 0;
  return SSD_OK;
}

int validate(const void* x, const void* dt, const float* A, const void* B, const void* C,
             const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
             int chunk_size, int ngroups, const float* initial_states, void* out,
             float* final_states, const int32_t* seq_idx, bool varlen, int64_t batch,
             int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype, int path,
             void* workspace, size_t workspace_bytes, Layout* lay, bool check_workspace = true) {
  int st = check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, varlen,
                        path, lay);
  if (st != SSD_OK) return st;
  if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return SSD_ERR_INVALID_ARG;
  if (!A) return SSD_ERR_INVALID_ARG;
  const bool nonempty = batch > 0 && seqlen > 0;
  if (nonempty && (!x || !dt || !B || !C || !out)) return SSD_ERR_INVALID_ARG;
  if (varlen && nonempty && !seq_idx) return SSD_ERR_INVALID_ARG;
  if (!aligned(seq_idx, 4)) return SSD_ERR_ALIGNMENT;

  const size_t es = dtype == SSD_BF16 ? 2 : 4;
  if (!aligned(A, 4) || !aligned(D, 4) || !aligned(dt_bias, 4)) return SSD_ERR_ALIGNMENT;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(B, 16) ||
      !aligned(C, 16) || !aligned(dt, es) || !aligned(initial_states, 16) ||
      !aligned(final_states, 16))
    return SSD_ERR_ALIGNMENT;
  // Overlap rules: out and final_states are written while inputs are still
  // being read (a later workgroup may read a row or an initial state that an
  // earlier one has already overwritten), so neither may overlap any input,
  // the other output or the workspace -- except that final_states may be
  // exactly initial_states (each element is read before it is written).
  const int64_t nx = batch * seqlen * nheads * headdim;
  const int64_t nbc = batch * seqlen * ngroups * dstate;
  const int64_t nst = batch * nheads * headdim * dstate;
  const Span none{0, 0};
  const Span sx = nonempty ? span(x, nx * (int64_t)es) : none;
  const Span sdt = nonempty ? span(dt, batch * seqlen * nheads * (int64_t)es) : none;
  const Span sB = nonempty ? span(B, nbc * (int64_t)es) : none;
  const Span sC = nonempty ? span(C, nbc * (int64_t)es) : none;
  const Span sz = nonempty && z ? span(z, nx * (int64_t)es) : none;
  const Span sseq = nonempty && seq_idx ? span(seq_idx, batch * seqlen * 4) : none;
  const Span sA = span(A, nheads * 4);
  const Span sD = D ? span(D, nheads * 4) : none;
  const Span sbias = dt_bias ? span(dt_bias, nheads * 4) : none;
  const Span sinit = initial_states ? span(initial_states, nst * 4) : none;
  const Span sws = lay->total > 0 && workspace ? span(workspace, (int64_t)lay->total) : none;
  const Span so = nonempty ? span(out, nx * (int64_t)es) : none;
  const Span sfin = final_states ? span(final_states, nst * 4) : none;
  auto hits = [](Span a, Span b) { return a.hi > a.lo && b.hi > b.lo && overlap(a, b); };
  for (const Span& s : {sx, sdt, sB, sC, sz, sseq, sA, sD, sbias, sinit, sws, sfin})
    if (hits(so, s)) return SSD_ERR_INVALID_ARG;
  for (const Span& s : {sx, sdt, sB, sC, sz, sseq, sA, sD, sbias, sws})
    if (hits(sfin, s)) return SSD_ERR_INVALID_ARG;
  if (final_states != initial_states && hits(sfin, sinit)) return SSD_ERR_INVALID_ARG;
  // the workspace is checked last: a call that gets past it launches kernels
  if (check_workspace && lay->total > 0) {
    if (!workspace || workspace_bytes < lay->total) return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return SSD_ERR_ALIGNMENT;
  }
  return SSD_OK;
}

// Block forward (split + conv1d prologue, scan, gated RMSNorm epilogue): its
// workspace holds x, B, C and dt in the input dtype, then the scan's own.
struct BlockLayout {
  Layout scan;
  size_t off_x = 0, off_b = 0, off_c = 0, off_dt = 0, off_scan = 0, total = 0;
};

int block_shapes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                 int ngroups, int chunk_size, int dtype, int conv_width, int norm_groups,
                 BlockLayout* bl) {
  int st = check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, false,
                        SSD_PATH_AUTO, &bl->scan);
  if (st != SSD_OK) return st;
  if (!ssd::block_supported(nheads * headdim, norm_groups, conv_width)) return SSD_ERR_UNSUPPORTED;
  // grids: the prologue tiles time by 32 steps (y dimension <= 65535), the
  // norm takes one workgroup per token
  if (seqlen > 65535LL * 32 || batch * seqlen > INT32_MAX) return SSD_ERR_UNSUPPORTED;
  const size_t es = dtype == SSD_BF16 ? 2 : 4;
  // element counts fit in int64: check_shapes checked b*L*H*P and b*L*G*N
  const size_t nx = (size_t)(batch * seqlen * nheads * headdim);
  const size_t nbc = (size_t)(batch * seqlen * ngroups * dstate);
  const size_t ndt = (size_t)(batch * seqlen * nheads);
  bl->off_x = 0;
  bl->off_b = round_up(nx * es);
  bl->off_c = bl->off_b + round_up(nbc * es);
  bl->off_dt = bl->off_c + round_up(nbc * es);
  bl->off_scan = bl->off_dt + round_up(ndt * es);
  bl->total = bl->off_scan + bl->scan.total;
  if (batch == 0 || seqlen == 0) bl->total = 0;
  return SSD_OK;
}

// Backward workspace (fp32, each region on a 256-byte boundary), blocks of 64:
// dt, cum [b, H, nb, 64]; chunk-local states (then P_c) and entering states
// [b, nb, H, P N]; y / dY [b, L, H, P]; G [b, nb, H, P N]; per-head dB and dC
// parts [b, L, H, N]; dA and dD parts [b, nb, H].
struct BwdLayout {
  int64_t nb = 0;
  size_t off_dt = 0, off_cum = 0, off_s = 0, off_in = 0, off_y = 0, off_g = 0, off_db = 0,
         off_dc = 0, off_da = 0, off_dd = 0, total = 0;
  // bf16 calls: fp32 copies of the inputs x, dt, B, C, z, dout and fp32
  // gradients dx, ddt, dB, dC, dz, in this order (kWide* index below)
  bool bf16 = false;
  size_t off_w[11] = {};
};
enum { kWideX, kWideDt, kWideB, kWideC, kWideZ, kWideDout, kWideDx, kWideDdt, kWideDb, kWideDc,
       kWideDz };

int bwd_shapes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
               int ngroups, int chunk_size, int dtype, BwdLayout* bl) {
  Layout lay;
  int st = check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, false,
                        SSD_PATH_AUTO, &lay);
  if (st != SSD_OK) return st;
  if (!ssd::config_supported(headdim, dstate, 64)) return SSD_ERR_UNSUPPORTED;
  const int64_t nb = ssd::bwd_blocks(seqlen);
  int64_t units, blkn, stn, xn, bcn;
  if (!mul_ok(batch * nb, nheads, &units) || !mul_ok(units, 64, &blkn) ||
      !mul_ok(units, headdim * dstate, &stn) || !mul_ok(batch * seqlen * nheads, headdim, &xn) ||
      !mul_ok(batch * seqlen * nheads, dstate, &bcn))
    return SSD_ERR_INVALID_ARG;
  if (units > INT32_MAX || nb > 65535) return SSD_ERR_UNSUPPORTED;
  bl->nb = nb;
  bl->off_dt = 0;
  bl->off_cum = round_up((size_t)blkn * 4);
  bl->off_s = bl->off_cum + round_up((size_t)blkn * 4);
  bl->off_in = bl->off_s + round_up((size_t)stn * 4);
  bl->off_y = bl->off_in + round_up((size_t)stn * 4);
  bl->off_g = bl->off_y + round_up((size_t)xn * 4);
  bl->off_db = bl->off_g + round_up((size_t)stn * 4);
  bl->off_dc = bl->off_db + round_up((size_t)bcn * 4);
  bl->off_da = bl->off_dc + round_up((size_t)bcn * 4);
  bl->off_dd = bl->off_da + round_up((size_t)units * 4);
  bl->total = bl->off_dd + round_up((size_t)units * 4);
  if (dtype == SSD_BF16) {
    int64_t gn;
    if (!mul_ok(batch * seqlen * ngroups, dstate, &gn)) return SSD_ERR_INVALID_ARG;
    const int64_t ndt = batch * seqlen * nheads;
    const int64_t sizes[11] = {xn, ndt, gn, gn, xn, xn, xn, ndt, gn, gn, xn};
    bl->bf16 = true;
    for (int k = 0; k < 11; ++k) {
      bl->off_w[k] = bl->total;
      bl->total += round_up((size_t)sizes[k] * 4);
    }
  }
  if (batch == 0 || seqlen == 0) bl->total = 0;
  return SSD_OK;
}

}  // namespace

struct ssd_timing {
  hipEvent_t ev[SSD_NUM_STAGES + 1];
  bool recorded;
};

static int run(const void* x, const void* dt, const float* A, const void* B, const void* C,
               const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
               int chunk_size, int ngroups, const float* initial_states, void* out,
               float* final_states, const int32_t* seq_idx, bool varlen, int64_t batch,
               int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype,
               int path, void* workspace, size_t workspace_bytes, hipStream_t stream,
               ssd_timing* timing) {
  Layout lay;
  int st = validate(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups,
                    initial_states, out, final_states, seq_idx, varlen, batch, seqlen, nheads,
                    headdim, dstate, dtype, path, workspace, workspace_bytes, &lay);
  if (st != SSD_OK) return st;
  if (batch == 0) return SSD_OK;

  ssd::Problem p;
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.z = z; p.dt_bias = dt_bias;
  p.dt_min = dt_min; p.dt_max = dt_max; p.init = initial_states; p.out = out;
  p.final_states = final_states;
  p.seq_idx = varlen ? seq_idx : nullptr;
  p.b = batch; p.L = seqlen; p.H = nheads; p.P = headdim; p.N = dstate; p.G = ngroups;
  p.Q = chunk_size; p.nc = lay.nc; p.bf16 = dtype == SSD_BF16;
  char* ws = static_cast<char*>(workspace);
  const bool staged_ws = lay.total && !lay.fused && !lay.chain;
  p.ws_dt = staged_ws ? reinterpret_cast<float*>(ws + lay.off_dt) : nullptr;
  p.ws_cum = staged_ws ? reinterpret_cast<float*>(ws + lay.off_cum) : nullptr;
  p.ws_states = staged_ws ? reinterpret_cast<float*>(ws + lay.off_states) : nullptr;
  p.ws_states_in = staged_ws ? reinterpret_cast<float*>(ws + lay.off_states_in) : nullptr;
  p.ws_bt = staged_ws ? reinterpret_cast<uint16_t*>(ws + lay.off_bt) : nullptr;
  p.ws_seg = staged_ws && varlen ? reinterpret_cast<int32_t*>(ws + lay.off_seg) : nullptr;
  p.ws_gram = staged_ws && lay.gram ? reinterpret_cast<float*>(ws + lay.off_gram) : nullptr;
  p.fs_ring = lay.fused ? reinterpret_cast<float*>(ws + lay.off_ring) : nullptr;
  p.fs_flags = lay.fused ? reinterpret_cast<unsigned*>(ws + lay.off_flags) : nullptr;
  p.fs_ctl = lay.fused ? reinterpret_cast<unsigned*>(ws + lay.off_ctl) : nullptr;
  p.fused_kind = path == SSD_PATH_FUSED_HEAD ? 1 : path == SSD_PATH_FUSED_GROUP ? 2 : 0;
  p.chain = lay.plan;
  p.cs_states = lay.chain && lay.plan.nseg > 1 ? reinterpret_cast<float*>(ws + lay.off_cs_states)
                                               : nullptr;
  p.cs_decay = lay.chain && lay.plan.nseg > 1 ? reinterpret_cast<float*>(ws + lay.off_cs_decay)
                                              : nullptr;

  auto mark = [&](int i) -> bool {
    return !timing || hipEventRecord(timing->ev[i], stream) == hipSuccess;
  };
  if (!mark(0)) return SSD_ERR_HIP;
  if (lay.decode) {
    if (!mark(1) || !mark(2) || !mark(3)) return SSD_ERR_HIP;
    if ((seqlen > 0 || final_states) && ssd::launch_decode(p, stream) != hipSuccess)
      return SSD_ERR_HIP;
    if (!mark(4)) return SSD_ERR_HIP;
    if (timing) timing->recorded = true;
    return SSD_OK;
  }
  if (lay.chain) {
    // segmented: the unit-state pass (reported as the chunk-state stage),
    // then the chain (reported as the chunk scan)
    if (!mark(1)) return SSD_ERR_HIP;
    if (ssd::launch_chain_bf16(p, stream, 0) != hipSuccess || !mark(2) || !mark(3))
      return SSD_ERR_HIP;
    if (ssd::launch_chain_bf16(p, stream, 1) != hipSuccess || !mark(4)) return SSD_ERR_HIP;
    if (timing) timing->recorded = true;
    return SSD_OK;
  }
  if (lay.fused) {
    // set-up (tickets, flags, ring slot 0), then the one scan kernel
    if (ssd::launch_fused_bf16(p, stream, 0) != hipSuccess) return SSD_ERR_HIP;
    if (!mark(1) || !mark(2) || !mark(3)) return SSD_ERR_HIP;
    if (ssd::launch_fused_bf16(p, stream, 1) != hipSuccess || !mark(4)) return SSD_ERR_HIP;
    if (timing) timing->recorded = true;
    return SSD_OK;
  }
  const bool bf16k = ssd::use_bf16_kernels(p);
  // fp32 with few chunks: stages 1-3 in one pass (reported as the chunk-state
  // stage, with an empty state-passing stage)
  const bool scan23 = seqlen > 0 && !bf16k &&
                      ssd::use_state_scan(p.bf16, varlen, batch, seqlen, nheads, dstate,
                                          chunk_size);
  if (p.ws_seg && ssd::launch_seq_count(p, stream) != hipSuccess) return SSD_ERR_HIP;
  if (scan23) {
    if (!mark(1) || ssd::launch_state_scan(p, stream) != hipSuccess || !mark(2))
      return SSD_ERR_HIP;
  } else if (seqlen > 0 && bf16k) {
    // prep (B^T), then the chunk state with dt/cumsum fused in
    if (ssd::launch_bf16_stage(p, stream, 0) != hipSuccess || !mark(1)) return SSD_ERR_HIP;
    if (ssd::launch_bf16_stage(p, stream, 1) != hipSuccess || !mark(2)) return SSD_ERR_HIP;
  } else if (seqlen > 0) {
    if (!ssd::chunk_state_fuses_dt(p) && ssd::launch_dt_cumsum(p, stream) != hipSuccess)
      return SSD_ERR_HIP;
    if (!mark(1)) return SSD_ERR_HIP;
    if (ssd::launch_chunk_state(p, stream) != hipSuccess || !mark(2)) return SSD_ERR_HIP;
  } else if (!mark(1) || !mark(2)) {
    return SSD_ERR_HIP;
  }
  // state passing also covers seqlen == 0: final = initial state (or zeros)
  if (!scan23 && (seqlen > 0 || final_states)) {
    if (ssd::launch_state_passing(p, stream) != hipSuccess) return SSD_ERR_HIP;
  }
  if (!mark(3)) return SSD_ERR_HIP;
  if (seqlen > 0) {
    const hipError_t e = bf16k ? ssd::launch_bf16_stage(p, stream, 2) : ssd::launch_chunk_scan(p, stream);
    if (e != hipSuccess) return SSD_ERR_HIP;
  }
  if (!mark(4)) return SSD_ERR_HIP;
  if (timing) timing->recorded = true;
  return SSD_OK;
}

// ---- allocation-free entry point ------------------------------------------
// Its workspace is this library-owned array (one copy per GPU, alive until the
// process ends).  Host code never uses the array's name as an address: the
// name is a host-side stand-in, and a kernel handed it would fault.  The
// device address is looked up once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];  // written once per device, under its once_flag

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int ssd_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
                 int chunk_size, int ngroups, const float* initial_states, void* out,
                 float* final_states, int64_t batch, int64_t seqlen, int64_t nheads,
                 int64_t headdim, int64_t dstate, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return run(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups, initial_states,
             out, final_states, nullptr, false, batch, seqlen, nheads, headdim, dstate, dtype,
             SSD_PATH_AUTO, workspace, workspace_bytes, stream, nullptr);
}

int ssd_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* dt_bias,
                         float dt_min, float dt_max, int chunk_size, int ngroups,
                         const float* initial_states, void* out, float* final_states,
                         int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                         int64_t dstate, int dtype, hipStream_t stream) {
  // every argument of the whole call first, with no workspace (the scratch is
  // library memory no caller tensor can overlap)
  Layout lay;
  int st = validate(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups,
                    initial_states, out, final_states, nullptr, false, batch, seqlen, nheads,
                    headdim, dstate, dtype, SSD_PATH_AUTO, nullptr, 0, &lay, false);
  if (st != SSD_OK) return st;
  if (batch == 0) return SSD_OK;
  // batch rows are independent: rows whose workspace does not fit the scratch
  // at once run in slices of rows, one after the other on `stream`, all on
  // the kernel path the whole call takes (so the result does not depend on
  // the slicing)
  const int taken = ssd_scan_fwd_taken_path(batch, seqlen, nheads, headdim, dstate, ngroups,
                                            chunk_size, dtype, 0, SSD_PATH_AUTO);
  if (taken < 0) return taken;
  const int path = taken == SSD_PATH_STAGED || taken == SSD_PATH_STAGED_SCAN ? SSD_PATH_STAGED
                   : taken == SSD_PATH_FUSED_HEAD          ? SSD_PATH_FUSED_HEAD
                   : taken == SSD_PATH_CHAIN_SEGMENTED ? SSD_PATH_CHAIN_SEGMENTED
                                                           : SSD_PATH_AUTO;
  int64_t rows = batch;
  if (lay.total > SSD_NOALLOC_SCRATCH_BYTES) {
    Layout one;
    if (check_shapes(1, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, false, path,
                     &one) != SSD_OK || one.total > SSD_NOALLOC_SCRATCH_BYTES)
      return SSD_ERR_WORKSPACE;  // one batch row needs more than the scratch holds
    rows = (int64_t)(SSD_NOALLOC_SCRATCH_BYTES / one.total);
    for (;; --rows) {  // the layout is not exactly linear in the rows (alignment)
      Layout part;
      if (check_shapes(rows, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, false,
                       path, &part) == SSD_OK && part.total <= SSD_NOALLOC_SCRATCH_BYTES)
        break;
    }
  }
  void* ws = scratch_address();
  if (!ws) return SSD_ERR_HIP;
  const int64_t es = dtype == SSD_BF16 ? 2 : 4;
  const int64_t xrow = seqlen * nheads * headdim * es, dtrow = seqlen * nheads * es;
  const int64_t bcrow = seqlen * (int64_t)ngroups * dstate * es, strow = nheads * headdim * dstate;
  for (int64_t b0 = 0; b0 < batch; b0 += rows) {
    const int64_t nb = batch - b0 < rows ? batch - b0 : rows;
    auto at = [b0](const void* p, int64_t row_bytes) -> const char* {
      return p ? static_cast<const char*>(p) + b0 * row_bytes : nullptr;
    };
    st = run(at(x, xrow), at(dt, dtrow), A, at(B, bcrow), at(C, bcrow), D, at(z, xrow), dt_bias,
             dt_min, dt_max, chunk_size, ngroups,
             initial_states ? initial_states + b0 * strow : nullptr,
             const_cast<char*>(at(out, xrow)), final_states ? final_states + b0 * strow : nullptr,
             nullptr, false, nb, seqlen, nheads, headdim, dstate, dtype, path, ws,
             SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr);
    if (st != SSD_OK) return st;
  }
  return SSD_OK;
}

int ssd_scan_fwd_varlen(const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        float dt_min, float dt_max, int chunk_size, int ngroups,
                        const float* initial_states, void* out, float* final_states,
                        const int32_t* seq_idx, int64_t batch, int64_t seqlen, int64_t nheads,
                        int64_t headdim, int64_t dstate, int dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return run(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups, initial_states,
             out, final_states, seq_idx, true, batch, seqlen, nheads, headdim, dstate, dtype,
             SSD_PATH_AUTO, workspace, workspace_bytes, stream, nullptr);
}

int ssd_scan_fwd_path(const void* x, const void* dt, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* dt_bias, float dt_min,
                      float dt_max, int chunk_size, int ngroups, const float* initial_states,
                      void* out, float* final_states, const int32_t* seq_idx, int64_t batch,
                      int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype,
                      int kernel_path, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return run(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups, initial_states,
             out, final_states, seq_idx, seq_idx != nullptr, batch, seqlen, nheads, headdim,
             dstate, dtype, kernel_path, workspace, workspace_bytes, stream, nullptr);
}

size_t ssd_scan_fwd_path_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                        int64_t headdim, int64_t dstate, int ngroups,
                                        int chunk_size, int dtype, int varlen, int kernel_path) {
  Layout lay;
  if (check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                   varlen != 0, kernel_path, &lay) != SSD_OK)
    return 0;
  return lay.total;
}

int ssd_scan_fwd_taken_path(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int ngroups, int chunk_size, int dtype, int varlen,
                            int kernel_path) {
  Layout lay;
  int st = check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                        varlen != 0, kernel_path, &lay);
  if (st != SSD_OK) return st;
  if (lay.decode) return SSD_PATH_STEP;
  if (lay.chain) return lay.plan.nseg > 1 ? SSD_PATH_CHAIN_SEGMENTED : SSD_PATH_CHAIN;
  if (lay.fused)
    return kernel_path == SSD_PATH_FUSED_GROUP && !varlen ? SSD_PATH_FUSED_GROUP
                                                         : SSD_PATH_FUSED_HEAD;
  return ssd::use_state_scan(dtype == SSD_BF16, varlen != 0, batch, seqlen, nheads, dstate,
                             chunk_size)
             ? SSD_PATH_STAGED_SCAN
             : SSD_PATH_STAGED;
}

int ssd_scan_fwd_wait_status(const void* workspace, size_t workspace_bytes, int64_t batch,
                             int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                             int ngroups, int chunk_size, int dtype, int varlen, int kernel_path,
                             hipStream_t stream) {
  Layout lay;
  int st = check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                        varlen != 0, kernel_path, &lay);
  if (st != SSD_OK) return st;
  if (hipStreamSynchronize(stream) != hipSuccess) return SSD_ERR_HIP;
  if (!lay.fused || lay.total == 0) return SSD_OK;  // no bounded wait on this path
  if (!workspace || workspace_bytes < lay.total) return SSD_ERR_WORKSPACE;
  if (!aligned(workspace, kAlign)) return SSD_ERR_ALIGNMENT;
  unsigned word = 0;
  const char* src = static_cast<const char*>(workspace) + lay.off_ctl + ssd::kFusedErrorWordByte;
  if (hipMemcpy(&word, src, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
    return SSD_ERR_HIP;
  return word == 0 ? SSD_OK : SSD_ERR_WAIT;
}

int ssd_scan_fwd_timed(const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       float dt_min, float dt_max, int chunk_size, int ngroups,
                       const float* initial_states, void* out, float* final_states,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, ssd_timing* timing) {
  if (!timing) return SSD_ERR_INVALID_ARG;
  return run(x, dt, A, B, C, D, z, dt_bias, dt_min, dt_max, chunk_size, ngroups, initial_states,
             out, final_states, nullptr, false, batch, seqlen, nheads, headdim, dstate, dtype,
             SSD_PATH_AUTO, workspace, workspace_bytes, stream, timing);
}

int ssd_split_conv1d_scan_fwd(const void* zxbcdt, const float* conv1d_weight,
                              const float* conv1d_bias, const float* dt_bias, const float* A,
                              const float* D, int chunk_size, const float* initial_states,
                              float dt_min, float dt_max, const float* rmsnorm_weight,
                              float rmsnorm_eps, int64_t headdim, int ngroups, int norm_groups,
                              void* out, float* final_states, int64_t batch, int64_t seqlen,
                              int64_t nheads, int64_t dstate, int conv_width, int dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  BlockLayout bl;
  int st = block_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype,
                        conv_width, norm_groups, &bl);
  if (st != SSD_OK) return st;
  if (!A) return SSD_ERR_INVALID_ARG;
  const bool nonempty = batch > 0 && seqlen > 0;
  if (nonempty && (!zxbcdt || !conv1d_weight || !out)) return SSD_ERR_INVALID_ARG;
  if (rmsnorm_weight && !(rmsnorm_eps >= 0.0f && std::isfinite(rmsnorm_eps)))
    return SSD_ERR_INVALID_ARG;
  const size_t es = dtype == SSD_BF16 ? 2 : 4;
  if (!aligned(zxbcdt, es) || !aligned(conv1d_weight, 4) || !aligned(conv1d_bias, 4) ||
      !aligned(rmsnorm_weight, 16) || !aligned(out, 16))
    return SSD_ERR_ALIGNMENT;
  const int64_t dim = nheads * headdim;
  const int64_t width = 2 * dim + 2 * (int64_t)ngroups * dstate + nheads;
  if (nonempty) {
    const Span so = span(out, batch * seqlen * dim * (int64_t)es);
    if (overlap(so, span(zxbcdt, batch * seqlen * width * (int64_t)es))) return SSD_ERR_INVALID_ARG;
    if (bl.total > 0 && overlap(so, span(workspace, (int64_t)bl.total))) return SSD_ERR_INVALID_ARG;
    if (final_states &&
        overlap(so, span(final_states, batch * nheads * headdim * dstate * (int64_t)4)))
      return SSD_ERR_INVALID_ARG;
  }
  if (bl.total > 0) {
    if (!workspace || workspace_bytes < bl.total) return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return SSD_ERR_ALIGNMENT;
  }
  if (batch == 0) return SSD_OK;
  char* ws = static_cast<char*>(workspace);
  ssd::BlockProblem q;
  q.zxbcdt = zxbcdt;
  q.conv_w = conv1d_weight;
  q.conv_b = conv1d_bias;
  q.W = conv_width;
  q.x = nonempty ? ws + bl.off_x : nullptr;
  q.B = nonempty ? ws + bl.off_b : nullptr;
  q.C = nonempty ? ws + bl.off_c : nullptr;
  q.dt = nonempty ? ws + bl.off_dt : nullptr;
  q.y = out;
  q.out = out;
  q.norm_w = rmsnorm_weight;
  q.eps = rmsnorm_eps;
  q.norm_groups = norm_groups;
  q.b = batch; q.L = seqlen; q.H = nheads; q.P = headdim; q.N = dstate; q.G = ngroups;
  q.bf16 = dtype == SSD_BF16;
  if (nonempty && ssd::launch_conv_split(q, stream) != hipSuccess) return SSD_ERR_HIP;
  // the scan without the gate, straight into out; the epilogue gates and
  // normalises it in place
  st = run(q.x, q.dt, A, q.B, q.C, D, nullptr, dt_bias, dt_min, dt_max, chunk_size, ngroups,
           initial_states, out, final_states, nullptr, false, batch, seqlen, nheads, headdim,
           dstate, dtype, SSD_PATH_AUTO, nonempty ? ws + bl.off_scan : nullptr,
           nonempty ? workspace_bytes - bl.off_scan : 0, stream, nullptr);
  if (st != SSD_OK) return st;
  if (nonempty && ssd::launch_gated_rmsnorm(q, stream) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

int ssd_scan_bwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
                 int chunk_size, int ngroups, const float* initial_states, const void* dout,
                 const float* dfinal_states, void* dx, void* ddt, float* dA, void* dB, void* dC,
                 float* dD, void* dz, float* ddt_bias, float* dinitial_states, int64_t batch,
                 int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  BwdLayout bl;
  int st = bwd_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, &bl);
  if (st != SSD_OK) return st;
  if (std::isnan(dt_min) || std::isnan(dt_max) || dt_min > dt_max) return SSD_ERR_INVALID_ARG;
  if (!A || !dA) return SSD_ERR_INVALID_ARG;
  if ((D != nullptr) != (dD != nullptr) || (z != nullptr) != (dz != nullptr) ||
      (dt_bias != nullptr) != (ddt_bias != nullptr))
    return SSD_ERR_INVALID_ARG;
  const bool nonempty = batch > 0 && seqlen > 0;
  if (nonempty && (!x || !dt || !B || !C || !dout || !dx || !ddt || !dB || !dC))
    return SSD_ERR_INVALID_ARG;
  const void* v16[] = {x, B, C, z, dout, dx, dz, dB, dC, initial_states, dfinal_states,
                       dinitial_states};
  for (const void* q : v16)
    if (!aligned(q, 16)) return SSD_ERR_ALIGNMENT;
  const int es = dtype == SSD_BF16 ? 2 : 4;  // bytes per element of the dtype tensors
  const void* v4[] = {A, D, dt_bias, dA, dD, ddt_bias};
  for (const void* q : v4)
    if (!aligned(q, 4)) return SSD_ERR_ALIGNMENT;
  if (!aligned(dt, es) || !aligned(ddt, es)) return SSD_ERR_ALIGNMENT;
  // outputs must not overlap any input, each other or the workspace
  const int64_t nx = batch * seqlen * nheads * headdim, nbc = batch * seqlen * ngroups * dstate;
  const int64_t nst = batch * nheads * headdim * dstate, ndt = batch * seqlen * nheads;
  const Span ins[] = {span(x, nx * es), span(dt, ndt * es), span(A, nheads * 4),
                      span(B, nbc * es), span(C, nbc * es), span(D, D ? nheads * 4 : 0),
                      span(z, z ? nx * es : 0), span(dt_bias, dt_bias ? nheads * 4 : 0),
                      span(initial_states, initial_states ? nst * 4 : 0), span(dout, nx * es),
                      span(dfinal_states, dfinal_states ? nst * 4 : 0),
                      span(workspace, (int64_t)bl.total)};
  const Span outs[] = {span(dx, nx * es), span(ddt, ndt * es), span(dA, nheads * 4),
                       span(dB, nbc * es), span(dC, nbc * es), span(dD, dD ? nheads * 4 : 0),
                       span(dz, dz ? nx * es : 0), span(ddt_bias, ddt_bias ? nheads * 4 : 0),
                       span(dinitial_states, dinitial_states ? nst * 4 : 0)};
  for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
    if (outs[a].hi <= outs[a].lo) continue;
    for (const Span& s2 : ins)
      if (s2.hi > s2.lo && overlap(outs[a], s2)) return SSD_ERR_INVALID_ARG;
    for (size_t c = a + 1; c < sizeof(outs) / sizeof(outs[0]); ++c)
      if (outs[c].hi > outs[c].lo && overlap(outs[a], outs[c])) return SSD_ERR_INVALID_ARG;
  }
  if (bl.total > 0) {
    if (!workspace || workspace_bytes < bl.total) return SSD_ERR_WORKSPACE;
    if (!aligned(workspace, kAlign)) return SSD_ERR_ALIGNMENT;
  }
  if (batch == 0) return SSD_OK;

  char* ws = static_cast<char*>(workspace);
  // With a gate and the four-heads chunk scan, the re-run's chunk scan forms
  // dY and dz from y in its epilogue (no y round trip, no gate kernel); it
  // reads z and dout, and writes dz, in their own dtype.
  const bool fuse_gate = nonempty && z && ssd::use_group_scan(nheads, dstate, ngroups, 64, false);
  // bf16: every other step runs on fp32 copies; the gradients of the bf16
  // tensors land in fp32 buffers and are rounded into the caller's at the end
  // (z, dout and dz stay bf16 when the chunk scan's epilogue is their only
  // user)
  const void* in[6] = {x, dt, B, C, z, dout};
  void* grad[5] = {dx, ddt, dB, dC, dz};
  if (bl.bf16 && nonempty) {
    const int64_t nin[6] = {nx, ndt, nbc, nbc, nx, nx};
    ssd::ConvList wl;
    for (int k = 0; k < 6; ++k) {
      if (!in[k] || (fuse_gate && k >= 4)) continue;
      float* w = reinterpret_cast<float*>(ws + bl.off_w[k]);
      wl.src[wl.count] = in[k];
      wl.dst[wl.count] = w;
      wl.n[wl.count++] = nin[k];
      in[k] = w;
    }
    if (ssd::launch_widen_bf16(wl, stream) != hipSuccess) return SSD_ERR_HIP;
    for (int k = 0; k < 5; ++k)
      if (grad[k] && !(fuse_gate && k == 4)) grad[k] = ws + bl.off_w[kWideDx + k];
  }
  x = in[0]; dt = in[1]; B = in[2]; C = in[3]; z = in[4]; dout = in[5];
  ssd::Problem p;
  p.x = x; p.dt = dt; p.A = A; p.B = B; p.C = C; p.D = D; p.z = nullptr; p.dt_bias = dt_bias;
  p.dt_min = dt_min; p.dt_max = dt_max; p.init = initial_states;
  p.out = nonempty ? ws + bl.off_y : nullptr;
  p.final_states = nullptr;
  p.seq_idx = nullptr;
  p.b = batch; p.L = seqlen; p.H = nheads; p.P = headdim; p.N = dstate; p.G = ngroups;
  p.Q = 64; p.nc = bl.nb; p.bf16 = false;
  p.ws_dt = nonempty ? reinterpret_cast<float*>(ws + bl.off_dt) : nullptr;
  p.ws_cum = nonempty ? reinterpret_cast<float*>(ws + bl.off_cum) : nullptr;
  p.ws_states = nonempty ? reinterpret_cast<float*>(ws + bl.off_s) : nullptr;
  p.ws_states_in = nonempty ? reinterpret_cast<float*>(ws + bl.off_in) : nullptr;
  p.ws_bt = nullptr;
  p.ws_seg = nullptr;
  p.ws_gram = nullptr;  // the chunk scan forms its tiles of B C^T itself
  p.fs_ring = nullptr; p.fs_flags = nullptr; p.fs_ctl = nullptr;
  p.fused_kind = 0;
  if (nonempty) {
    // the forward again (64-step blocks, no gate): dt, cum, states, and the
    // ungated y, which only dz needs (no gate: no y)
    if (ssd::use_state_scan(false, false, batch, seqlen, nheads, dstate, 64)) {
      if (ssd::launch_state_scan(p, stream) != hipSuccess) return SSD_ERR_HIP;
    } else {
      if (!ssd::chunk_state_fuses_dt(p) && ssd::launch_dt_cumsum(p, stream) != hipSuccess)
        return SSD_ERR_HIP;
      if (ssd::launch_chunk_state(p, stream) != hipSuccess) return SSD_ERR_HIP;
      if (ssd::launch_state_passing(p, stream) != hipSuccess) return SSD_ERR_HIP;
    }
    // With a gate and the four-heads chunk scan, its epilogue forms dY and dz
    // from y directly (no y round trip, no gate kernel)
    if (fuse_gate) {
      p.z = z;
      p.gate_dout = dout;
      p.gate_dz = grad[4];
      p.gate_bf16 = bl.bf16;
    }
    if (z && ssd::launch_chunk_scan(p, stream) != hipSuccess) return SSD_ERR_HIP;
    p.z = nullptr;
    p.gate_dout = nullptr;
    p.gate_dz = nullptr;
    p.gate_bf16 = false;
  }
  ssd::BwdProblem q;
  q.fwd = p;
  q.fwd.z = z;
  q.dout = static_cast<const float*>(dout);
  q.dfinal = dfinal_states;
  // dY: formed over y when there is a gate, else dout itself (only read)
  q.dy = !nonempty ? nullptr
         : z       ? reinterpret_cast<float*>(ws + bl.off_y)
                   : const_cast<float*>(static_cast<const float*>(dout));
  q.gst = nonempty ? reinterpret_cast<float*>(ws + bl.off_g) : nullptr;
  q.dBh = nonempty ? reinterpret_cast<float*>(ws + bl.off_db) : nullptr;
  q.dCh = nonempty ? reinterpret_cast<float*>(ws + bl.off_dc) : nullptr;
  q.dA_p = nonempty ? reinterpret_cast<float*>(ws + bl.off_da) : nullptr;
  q.dD_p = nonempty ? reinterpret_cast<float*>(ws + bl.off_dd) : nullptr;
  q.dx = static_cast<float*>(grad[0]);
  q.ddt = static_cast<float*>(grad[1]);
  q.dB = static_cast<float*>(grad[2]);
  q.dC = static_cast<float*>(grad[3]);
  q.dz = static_cast<float*>(grad[4]);
  q.dA = dA; q.dD = dD; q.ddt_bias = ddt_bias; q.dinit = dinitial_states;
  q.dy_formed = fuse_gate;
  if (ssd::launch_bwd(q, stream) != hipSuccess) return SSD_ERR_HIP;
  if (bl.bf16 && nonempty) {
    void* outs_bf16[5] = {dx, ddt, dB, dC, dz};
    const int64_t nout[5] = {nx, ndt, nbc, nbc, nx};
    ssd::ConvList nl;
    for (int k = 0; k < 5; ++k) {
      if (!outs_bf16[k] || (fuse_gate && k == 4)) continue;  // dz: written as bf16
      nl.src[nl.count] = grad[k];
      nl.dst[nl.count] = outs_bf16[k];
      nl.n[nl.count++] = nout[k];
    }
    if (ssd::launch_narrow_bf16(nl, stream) != hipSuccess) return SSD_ERR_HIP;
  }
  return SSD_OK;
}

size_t ssd_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int ngroups, int chunk_size,
                                   int dtype) {
  BwdLayout bl;
  if (bwd_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, &bl) !=
      SSD_OK)
    return 0;
  return bl.total;
}

size_t ssd_split_conv1d_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                                int64_t headdim, int64_t dstate, int ngroups,
                                                int chunk_size, int dtype, int conv_width,
                                                int norm_groups) {
  BlockLayout bl;
  if (block_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, conv_width,
                   norm_groups, &bl) != SSD_OK)
    return 0;
  return bl.total;
}

size_t ssd_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int ngroups, int chunk_size,
                                   int dtype) {
  Layout lay;
  if (check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, false,
                   SSD_PATH_AUTO, &lay) != SSD_OK)
    return 0;
  return lay.total;
}

size_t ssd_scan_fwd_varlen_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int ngroups,
                                          int chunk_size, int dtype) {
  Layout lay;
  if (check_shapes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, dtype, true,
                   SSD_PATH_AUTO, &lay) != SSD_OK)
    return 0;
  return lay.total;
}

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSD_ERR_ALIGNMENT: return "misaligned pointer";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP launch failure";
    case SSD_ERR_WAIT: return "a workgroup gave up waiting for its entering state";
    default: return "unknown status";
  }
}

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

int ssd_timing_create(ssd_timing** out) {
  if (!out) return SSD_ERR_INVALID_ARG;
  ssd_timing* t = new (std::nothrow) ssd_timing();
  if (!t) return SSD_ERR_HIP;
  for (int i = 0; i <= SSD_NUM_STAGES; ++i) {
    if (hipEventCreate(&t->ev[i]) != hipSuccess) {
      for (int k = 0; k < i; ++k) (void)hipEventDestroy(t->ev[k]);
      delete t;
      return SSD_ERR_HIP;
    }
  }
  t->recorded = false;
  *out = t;
  return SSD_OK;
}

int ssd_timing_destroy(ssd_timing* t) {
  if (!t) return SSD_ERR_INVALID_ARG;
  for (int i = 0; i <= SSD_NUM_STAGES; ++i) (void)hipEventDestroy(t->ev[i]);
  delete t;
  return SSD_OK;
}

int ssd_timing_read(ssd_timing* t, float* stage_ms) {
  if (!t || !stage_ms || !t->recorded) return SSD_ERR_INVALID_ARG;
  if (hipEventSynchronize(t->ev[SSD_NUM_STAGES]) != hipSuccess) return SSD_ERR_HIP;
  for (int i = 0; i < SSD_NUM_STAGES; ++i) {
    if (hipEventElapsedTime(&stage_ms[i], t->ev[i], t->ev[i + 1]) != hipSuccess)
      return SSD_ERR_HIP;
  }
  return SSD_OK;
}

}  // extern "C"
