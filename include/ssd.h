/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD chunked selective-scan
 * forward.
 *
 * The operation (per batch row b and head h, t = 0 .. seqlen-1):
 *
 *   dt_t  = min(max(softplus(dt_raw[b,t,h] + dt_bias[h]), dt_min), dt_max)
 *   h_t   = exp(dt_t * A[h]) * h_{t-1} + dt_t * x[b,t,h,:] (outer) B[b,t,g,:]
 *   y_t   = h_t . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *   out[b,t,h,:] = y_t * silu(z[b,t,h,:])            (y_t when z is NULL)
 *
 * with g = h / (nheads / ngroups), h_{-1} = initial_states[b,h] (zeros when
 * NULL) and final_states[b,h] = h_{seqlen-1}.  The state h_t is stored as a
 * headdim x dstate matrix (element [p][n]).
 *
 * Where each piece comes from (the pages are GitHub threads on the mamba
 * kernels):
 *  - the recurrence is the Mamba-2 state-space-duality layer (Dao & Gu 2024),
 *    which the flash-linear-attention PR #49 page ("Replace mamba2
 *    mamba_chunk_scan_combined triton kernel by simple_gla triton kernel")
 *    cites; the same page's list of differences between simple_gla and the
 *    mamba2_ssd kernel fixes the [batch, seq, head, hidden] layout, the
 *    absence of a 1/sqrt(d) scale on C.B, dt as a discretization input folded
 *    into the gate dt*A with A constant in time, and B/C shared by groups of
 *    heads ("group query attention");
 *  - dt_bias, dt_limit, D with one value per head, the SiLU gate applied
 *    before any norm, initial_states and return_final_states are the
 *    arguments of the repro script on mamba issue #647 ("...exhibit large
 *    numerical differences when ngroups > 1");
 *  - starting from a given state for chunked prefill is mamba issue #488
 *    ("feat: Initial state support for Mamba SSM (1)").
 *
 * The work is done in chunks of chunk_size timesteps: a dt/cumsum pass, a
 * per-chunk state pass on the matrix cores, a sequential inter-chunk state
 * pass, and a chunk-scan pass with the D-skip / z-gate epilogue fused in.
 * The result does not depend on chunk_size beyond rounding.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 2

/* Element type of x, dt, B, C, z and out.  A, D, dt_bias, dt_limit and both
 * state tensors are always float32; accumulation is always float32. */
#define SSD_F32 0
#define SSD_BF16 1

/* Status codes. */
#define SSD_OK 0
#define SSD_ERR_INVALID_ARG (-1) /* null required pointer, negative or zero size where a
                                    positive one is needed, nheads % ngroups != 0, dt_min or
                                    dt_max NaN, dt_min > dt_max, unknown dtype, out
                                    overlapping an input, final_states partially overlapping
                                    initial_states */
#define SSD_ERR_UNSUPPORTED (-2) /* a (headdim, dstate, chunk_size) combination not compiled:
                                    headdim must be 64, dstate one of 16/32/64/128, chunk_size
                                    one of 64/128/256; or sizes past the kernels' limits
                                    (nheads*headdim or ngroups*dstate above 2^22, batch, nheads
                                    or chunks above 65535) */
#define SSD_ERR_ALIGNMENT (-3)   /* x, z, out, B, C, states not 16-byte aligned; dt, A, D,
                                    dt_bias not aligned to their element; workspace not
                                    256-byte aligned */
#define SSD_ERR_WORKSPACE (-4)   /* workspace NULL or smaller than ssd_scan_fwd_workspace_size */
#define SSD_ERR_HIP (-5)         /* a kernel launch failed (hipGetLastError), or a HIP call of
                                    ssd_scan_fwd_wait_status failed */
#define SSD_ERR_WAIT (-6)        /* ssd_scan_fwd_wait_status only: on the fused path a
                                    workgroup gave up its bounded wait for the state entering
                                    its block; out and final_states of that call are invalid */

/*
 * ssd_scan_fwd -- enqueue the forward on `stream`.
 *
 * Arguments (all pointers are device memory owned by the caller):
 *   x        [batch, seqlen, nheads, headdim]   dtype       required
 *   dt       [batch, seqlen, nheads]            dtype       required (raw, before softplus)
 *   A        [nheads]                           float32     required
 *   B        [batch, seqlen, ngroups, dstate]   dtype       required
 *   C        [batch, seqlen, ngroups, dstate]   dtype       required
 *   D        [nheads]                           float32     NULL: no skip term
 *   z        [batch, seqlen, nheads, headdim]   dtype       NULL: no gate
 *   dt_bias  [nheads]                           float32     NULL: zero bias
 *   dt_min, dt_max    clamp applied after softplus ((0, +inf) leaves dt unchanged)
 *   chunk_size        timesteps per chunk (64, 128 or 256)
 *   ngroups           number of B/C groups; must divide nheads
 *   initial_states [batch, nheads, headdim, dstate] float32  NULL: zero state
 *   out      [batch, seqlen, nheads, headdim]   dtype       required; written
 *   final_states [batch, nheads, headdim, dstate] float32   NULL: not returned;
 *                     may be the same pointer as initial_states (in-place
 *                     continuation), but must not partially overlap it
 *   batch, seqlen     >= 0 (batch == 0: nothing is done; seqlen == 0:
 *                     final_states = initial_states or zeros)
 *   nheads, headdim, dstate  > 0
 *   dtype    SSD_F32 or SSD_BF16 (bf16 output is rounded to nearest even)
 *   workspace, workspace_bytes  scratch of at least
 *                     ssd_scan_fwd_workspace_size(...) bytes, 256-byte aligned
 *   stream   HIP stream the kernels are enqueued on (0: the null stream)
 *
 * All tensors are contiguous row-major.  `out` must not overlap any input.
 * Every argument is checked before anything is enqueued; on an error nothing
 * is launched and nothing is written.  The call does not synchronize: errors
 * inside a kernel surface at the caller's next synchronization.  The library
 * allocates no memory and keeps no pointer after the call returns; calls are
 * reentrant and deterministic (bitwise identical results run to run).
 *
 * Short sequences (seqlen <= 16, either dtype, any supported shape) take
 * the step kernel: the recurrence run step by step from initial_states, one
 * workgroup per (batch, head) with the state held in registers (serving one
 * token at a time, or a few speculative tokens, continuing a state).  It
 * needs no workspace (ssd_scan_fwd_workspace_size returns 0; workspace may
 * be NULL) and ignores chunk_size beyond checking it.  final_states may be
 * initial_states.
 *
 * Longer sequences take one of three kernel paths.  bf16 inputs with headdim
 * 64 and dstate 64 or 128 take, by default (ssd_scan_fwd_path selects a path
 * explicitly), the chain
 * path when each group holds an even number of heads and the head pairs fill
 * the machine: one kernel in which each workgroup carries a pair of heads of one
 * group through the whole sequence in 128-step blocks with the state held on
 * chip (no workspace: ssd_scan_fwd_workspace_size returns 0).  When the pairs
 * alone do not fill it but pairs times segments (at most one per block) fill
 * a round of the compute units at least 3/4, or half of it when the sequence
 * has at least 8 blocks, the chain runs over segments
 * (SSD_PATH_CHAIN_SEGMENTED below); the workspace then holds the units' end
 * states [batch, nheads, units] (headdim x dstate floats, row-major) and
 * their decays [batch, nheads, units].  Otherwise they
 * take the fused path: one set-up kernel and one scan kernel, in which each
 * workgroup handles 128 timesteps of one (batch, head) and hands the state to
 * the workgroup of the next 128 timesteps through the workspace.  (The
 * chunked form gives the same result for any block length, up to rounding;
 * chunk_size is still checked.)  Every other case takes the staged path:
 * dt/cumsum, chunk state, state passing and chunk scan kernels with their
 * intermediates in the workspace.
 *
 * Staged path: after the enqueued work completes, the workspace holds the
 * intermediates (float32, in this order, each region starting on a 256-byte
 * boundary):
 *   dt        [batch, nheads, nchunks, chunk_size]   0 past the sequence end
 *   dA_cumsum [batch, nheads, nchunks, chunk_size]   in-chunk running sum of dt*A
 *   chunk_states [batch, nchunks, nheads] blocks of headdim*dstate floats:
 *             each chunk's own contribution (the recurrence over the chunk
 *             from a zero state)
 *   states_in [batch, nchunks, nheads] blocks of headdim*dstate floats: the
 *             state entering each chunk
 *   B^T       [batch, nchunks, ngroups] blocks of dstate x chunk_size bf16
 *             (present only when dtype is SSD_BF16, chunk_size 128 or 256 and
 *             dstate 64 or 128: the bf16 matrix-core kernels' transposed B)
 *   C.B^T     [batch, nchunks, ngroups] blocks of T(T+1)/2 x 1024 floats,
 *             T = chunk_size/32: the causal 32 x 32 tiles of B C^T of each
 *             chunk (tile s <= t numbered t(t+1)/2 + s; in each tile the
 *             float4 at R*64 + lane holds the values lane `lane` of a
 *             v_mfma_f32_32x32x2_f32 result keeps in registers 4R..4R+3).
 *             Present only when chunk_size is 64 or 128, dstate 64 or 128,
 *             nheads/ngroups a multiple of 4 and at least 8, and the inputs
 *             are SSD_F32 or SSD_BF16 at chunk_size 64.
 * with nchunks = ceil(seqlen / chunk_size).  Inside a state block (headdim
 * 64) element (p, n) sits at float offset
 *   ((q*2 + p%2)*64 + 32*k + p/2)*4 + n%4,  k = n / (dstate/2),
 *   q = (n % (dstate/2)) / 4,
 * i.e. float4 tiles of four consecutive n, ordered so that the kernels read
 * and write them with one contiguous 1 KB access per wave.
 *
 * Fused path: the workspace holds, each region on a 256-byte boundary,
 *   ring   [batch*nheads][2] state blocks (tiled as above): the states
 *          handed between consecutive 128-step blocks
 *   flags  [batch*nheads][ceil(seqlen/128)] uint32 ready flags
 *   control 9 uint32: eight ticket counters, then an error word that is
 *          non-zero if a workgroup gave up waiting for its entering state
 *          (outputs are then invalid; it cannot happen unless the device
 *          stops making progress).  ssd_scan_fwd_wait_status reads it.
 * The workspace of one call must not be in use by another call at the same
 * time (true of both paths).
 */
int ssd_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
                 int chunk_size, int ngroups, const float* initial_states, void* out,
                 float* final_states, int64_t batch, int64_t seqlen, int64_t nheads,
                 int64_t headdim, int64_t dstate, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * ssd_scan_fwd_noalloc -- ssd_scan_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, checks,
 * status codes and results are those of ssd_scan_fwd (same kernels, same
 * path), except that the workspace is a library-owned device array of
 * SSD_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the library's first
 * use on that GPU until the process ends.  The call allocates nothing (no
 * hipMalloc, no allocating library routine).  A problem whose workspace is
 * larger than the array runs in slices of batch rows, one after another on
 * `stream`, on the path the whole problem takes; SSD_ERR_WORKSPACE when a
 * single batch row needs more than SSD_NOALLOC_SCRATCH_BYTES (e.g. fp32
 * sequences of 65536 steps at 32 heads x 64 x 128).  Every call on a GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (two
 * streams, two threads) race and give wrong results; calls enqueued on one
 * stream are ordered and safe.  What must start at zero (the fused path's
 * tickets, flags and error word) is cleared by a kernel at every call.  The
 * first call on a device looks the array's address up (SSD_ERR_HIP if that
 * fails).
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ssd_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* dt_bias,
                         float dt_min, float dt_max, int chunk_size, int ngroups,
                         const float* initial_states, void* out, float* final_states,
                         int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                         int64_t dstate, int dtype, hipStream_t stream);

/* Bytes of workspace ssd_scan_fwd needs for these sizes (0 for an empty
 * problem, for seqlen <= 16, on the unsegmented chain path, and for arguments ssd_scan_fwd
 * would reject); pure host computation, no HIP call.  The workspace holds
 * the chunked form's intermediates: per-chunk states and the states entering
 * each chunk, as the Mamba-1 CUDA forward on mamba issue #488 keeps its
 * per-chunk scan intermediates in a buffer the caller receives. */
size_t ssd_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int ngroups, int chunk_size,
                                   int dtype);

/*
 * Kernel paths of ssd_scan_fwd_path (the path ssd_scan_fwd takes is
 * SSD_PATH_AUTO).  They compute the same operation and differ only in
 * rounding order; testing and measuring each path needs a way to ask for it
 * by name, per call:
 *   SSD_PATH_AUTO        the choice described at ssd_scan_fwd
 *   SSD_PATH_STAGED      dt/cumsum, chunk state, state passing, chunk scan
 *   SSD_PATH_FUSED       the fused bf16 path, kernel form chosen from the shape
 *   SSD_PATH_FUSED_HEAD  fused, one workgroup per 128-step block and head
 *   SSD_PATH_FUSED_GROUP fused, one workgroup per 128-step block, B/C group
 *                        and set of up to 8 of its heads (packed-sequence
 *                        calls run the per-head form)
 *   SSD_PATH_CHAIN       the chain bf16 kernel (one workgroup per pair of
 *                        heads of a group for the whole sequence)
 *   SSD_PATH_CHAIN_SEGMENTED  the chain kernel over segments of the sequence:
 *                        a unit-state pass computes the local end state of
 *                        every unit of blocks before the last segment, then
 *                        one workgroup per (pair, segment) runs the chain from
 *                        the units before it folded into its entering state;
 *                        as many segments as fill one round of the compute
 *                        units (at least two; a one-block sequence is one)
 * A path the shape cannot take falls back, always the same way: SSD_PATH_CHAIN
 * with an odd number of heads per group takes the fused path; every fused or
 * chain path takes the staged path unless the inputs are bf16 with headdim 64
 * and dstate 64 or 128; seqlen <= 16 always takes the step kernel.  Any other
 * value is SSD_ERR_INVALID_ARG.
 */
#define SSD_PATH_AUTO 0
#define SSD_PATH_STAGED 1
#define SSD_PATH_FUSED 2
#define SSD_PATH_FUSED_HEAD 3
#define SSD_PATH_FUSED_GROUP 4
#define SSD_PATH_CHAIN 5
#define SSD_PATH_STEP 6 /* reported by ssd_scan_fwd_taken_path only (seqlen <= 16) */
#define SSD_PATH_CHAIN_SEGMENTED 7
/* reported by ssd_scan_fwd_taken_path only: the staged path with its first
 * three stages as one pass (fp32, dstate 64 or 128, chunk 64 or 128, at
 * most 32 chunks per sequence row, batch x nheads x dstate/32, or else
 * x dstate/64, between half and all of the 256 compute units) */
#define SSD_PATH_STAGED_SCAN 8

/*
 * ssd_scan_fwd_path -- ssd_scan_fwd on an explicitly chosen kernel path.
 * Arguments as for ssd_scan_fwd_varlen, except that seq_idx may be NULL (one
 * sequence per row, exactly ssd_scan_fwd), plus kernel_path (SSD_PATH_*).  The
 * workspace is ssd_scan_fwd_path_workspace_size(..., varlen = seq_idx != NULL,
 * kernel_path) bytes.  Stateless: the path is an argument, nothing is kept
 * between calls.
 */
int ssd_scan_fwd_path(const void* x, const void* dt, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* dt_bias, float dt_min,
                      float dt_max, int chunk_size, int ngroups, const float* initial_states,
                      void* out, float* final_states, const int32_t* seq_idx, int64_t batch,
                      int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype,
                      int kernel_path, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Workspace bytes of ssd_scan_fwd_path (varlen: non-zero when seq_idx will
 * be given).  0 for arguments the call would reject; pure host computation. */
size_t ssd_scan_fwd_path_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                        int64_t headdim, int64_t dstate, int ngroups,
                                        int chunk_size, int dtype, int varlen, int kernel_path);

/* The kernel path a call with these arguments takes: SSD_PATH_STAGED,
 * SSD_PATH_STAGED_SCAN, SSD_PATH_FUSED_HEAD, SSD_PATH_FUSED_GROUP,
 * SSD_PATH_CHAIN, SSD_PATH_CHAIN_SEGMENTED or SSD_PATH_STEP (the step kernel
 * of seqlen <= 16),
 * after the fallbacks above; kernel_path
 * is what the call asks for (SSD_PATH_AUTO for ssd_scan_fwd).  A negative
 * status for arguments the call would reject.  Pure host computation. */
int ssd_scan_fwd_taken_path(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                            int64_t dstate, int ngroups, int chunk_size, int dtype, int varlen,
                            int kernel_path);

/*
 * ssd_scan_fwd_wait_status -- whether the last call enqueued on `stream` with
 * this workspace and these arguments (the sizes, dtype, varlen and path of
 * that call; ssd_scan_fwd, ssd_scan_fwd_varlen and ssd_scan_fwd_timed are
 * SSD_PATH_AUTO) completed its hand-offs.  It synchronizes `stream`.  On the
 * fused path it reads the error word of the workspace's control region:
 * SSD_OK, or SSD_ERR_WAIT when a workgroup gave up its bounded wait (then
 * out and final_states of that call are invalid).  Other paths have no
 * bounded wait and return SSD_OK after the synchronization.  SSD_ERR_HIP if
 * the synchronization or the read fails; the shape checks of ssd_scan_fwd
 * otherwise.  The word is cleared by the next call's set-up kernel, so
 * query before enqueueing another call on the same workspace.
 */
int ssd_scan_fwd_wait_status(const void* workspace, size_t workspace_bytes, int64_t batch,
                             int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                             int ngroups, int chunk_size, int dtype, int varlen, int kernel_path,
                             hipStream_t stream);

/*
 * Packed sequences: ssd_scan_fwd over batch rows that each hold several
 * sequences one after another (the seq_idx argument of the chunked scan in
 * mamba issue #647's repro script).
 *
 *   seq_idx  [batch, seqlen]  int32, 4-byte aligned, required (non-NULL when
 *            batch and seqlen are > 0): a label per step.  Wherever the label
 *            of step t differs from that of step t-1 a new sequence starts:
 *            the state is reset to zero before step t, so nothing flows from
 *            one sequence into the next.  Labels need not be ordered; only
 *            changes between neighbouring steps count.
 *
 * initial_states is the state entering the row's first sequence and
 * final_states the state after the row's last step (its last sequence).
 * Every other argument, the checks and the execution rules are those of
 * ssd_scan_fwd; `out` must not overlap seq_idx either.  The call takes the
 * same path as ssd_scan_fwd (the chain and fused bf16 kernels count the
 * sequence starts themselves; asked for SSD_PATH_FUSED_GROUP the fused path
 * runs its per-head form) and needs ssd_scan_fwd_varlen_workspace_size(...)
 * bytes of workspace: that of the plain call on the chain and fused paths, on the
 * staged path the staged layout followed, on a 256-byte boundary, by
 *   seg [batch, nchunks, chunk_size] int32: for step q of chunk c the number
 *       of sequence starts at steps c*chunk_size .. c*chunk_size + q (steps
 *       past the sequence end repeat the last count).
 * Returns the ssd_scan_fwd status codes (SSD_ERR_INVALID_ARG for a missing
 * seq_idx).
 */
int ssd_scan_fwd_varlen(const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        float dt_min, float dt_max, int chunk_size, int ngroups,
                        const float* initial_states, void* out, float* final_states,
                        const int32_t* seq_idx, int64_t batch, int64_t seqlen, int64_t nheads,
                        int64_t headdim, int64_t dstate, int dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ssd_scan_fwd_varlen needs (0 for an empty problem, for
 * seqlen <= 16 and for rejected arguments); pure host computation. */
size_t ssd_scan_fwd_varlen_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                          int64_t headdim, int64_t dstate, int ngroups,
                                          int chunk_size, int dtype);

/*
 * Block forward around the scan: the fused Mamba-2 block of mamba issue #647's
 * repro (mamba_split_conv1d_scan_combined) up to, not including, its out_proj
 * linear.  With dim = nheads * headdim:
 *
 *   zxbcdt  [batch, seqlen, 2*dim + 2*ngroups*dstate + nheads]  dtype
 *           per token [z (dim) | x (dim) | B (ngroups*dstate) | C (ngroups*dstate)
 *           | dt (nheads)]
 *   conv1d_weight [dim + 2*ngroups*dstate, conv_width] float32, required
 *   conv1d_bias   [dim + 2*ngroups*dstate] float32, NULL: no bias
 *   conv_width    2, 3 or 4
 *   rmsnorm_weight [dim] float32, 16-byte aligned, NULL: no norm
 *                 (out = y * silu(z))
 *   rmsnorm_eps   >= 0, finite (used only with a weight)
 *   norm_groups   the norm's mean runs over dim / norm_groups channels: 1 for
 *                 the whole width, ngroups for one slice per B/C group (the
 *                 page's python reference and fused kernel respectively);
 *                 must divide dim; dim <= 15360, norm_groups <= 256
 *   out     [batch, seqlen, dim]  dtype; written
 *   every other argument as for ssd_scan_fwd (dt_bias, A, D, dt_min/dt_max,
 *   chunk_size, ngroups, initial_states, final_states, sizes, dtype, stream).
 *
 * Steps, all on `stream`:
 *   1. xBC = SiLU(causal depthwise conv(xBC) + bias): conv[t][c] =
 *      sum_k weight[c][k] * xBC[t - (conv_width-1) + k][c], zeros before step
 *      0; x, B, C land in the workspace in the input dtype, dt is copied;
 *   2. the scan of ssd_scan_fwd on them, without a gate, into out;
 *   3. out = g / sqrt(mean(g^2) + eps) * rmsnorm_weight with g = out * silu(z)
 *      (gate before norm), in place.
 * Workspace: ssd_split_conv1d_scan_fwd_workspace_size(...) bytes, 256-byte
 * aligned: x [b,L,H,P], B and C [b,L,G,N], dt [b,L,H] (input dtype, each on a
 * 256-byte boundary), then the scan's workspace.  out must not overlap
 * zxbcdt, the workspace or final_states.  Status codes as for ssd_scan_fwd
 * (SSD_ERR_UNSUPPORTED also for conv_width, dim or norm_groups out of range).
 */
int ssd_split_conv1d_scan_fwd(const void* zxbcdt, const float* conv1d_weight,
                              const float* conv1d_bias, const float* dt_bias, const float* A,
                              const float* D, int chunk_size, const float* initial_states,
                              float dt_min, float dt_max, const float* rmsnorm_weight,
                              float rmsnorm_eps, int64_t headdim, int ngroups, int norm_groups,
                              void* out, float* final_states, int64_t batch, int64_t seqlen,
                              int64_t nheads, int64_t dstate, int conv_width, int dtype,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ssd_split_conv1d_scan_fwd needs (0 for an empty problem
 * and for rejected arguments); pure host computation. */
size_t ssd_split_conv1d_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                                int64_t headdim, int64_t dstate, int ngroups,
                                                int chunk_size, int dtype, int conv_width,
                                                int norm_groups);

/*
 * Backward of ssd_scan_fwd: the gradients of
 *     l = sum(dout * out) + sum(dfinal_states * final_states)
 * with respect to every input, for training (the pages note the backward as
 * missing or separate).  Arguments x .. initial_states, the sizes and dtype are
 * those of the forward call; chunk_size is checked as there (the gradients do
 * not depend on it: the backward works in 64-step blocks).
 *
 * dtype SSD_F32: every tensor below is float32.  dtype SSD_BF16: x, dt, B, C,
 * z and dout are bfloat16, and so are their gradients dx, ddt, dB, dC and dz
 * (rounded to nearest even from fp32); A, D, dt_bias, the states and dA, dD,
 * ddt_bias, dinitial_states stay float32.  bf16 inputs are widened to fp32
 * (exactly) in the workspace and every step runs in fp32, as for SSD_F32.
 *
 *   dout            [batch, seqlen, nheads, headdim]  required
 *   dfinal_states   [batch, nheads, headdim, dstate]  NULL: zero
 *   dx              [batch, seqlen, nheads, headdim]  required
 *   ddt             [batch, seqlen, nheads]  gradient of dt (the raw input);
 *                   zero where dt_limit clamps softplus(dt + dt_bias)
 *   dA              [nheads]                          required
 *   dB, dC          [batch, seqlen, ngroups, dstate]  required (summed over
 *                   the heads of each group)
 *   dD              [nheads]    exactly when D is given
 *   dz              like x      exactly when z is given
 *   ddt_bias        [nheads]    exactly when dt_bias is given
 *   dinitial_states [batch, nheads, headdim, dstate]  NULL: not returned
 * All contiguous; x, B, C, z, dout, dx, dz, dB, dC and the state tensors
 * 16-byte aligned, dt and ddt aligned to their element, the float32 vectors
 * 4-byte aligned.  No output may overlap an input, another output or the
 * workspace.
 *
 * The forward is re-run inside (dt, running sums, the states entering each
 * block and the ungated output go to the workspace), then the reverse pass.
 * Workspace: ssd_scan_bwd_workspace_size(...) bytes, 256-byte aligned (for
 * bf16 it adds fp32 copies of x, dt, B, C, z, dout and fp32 buffers for their
 * gradients).  Like the forward the call is asynchronous and deterministic.
 * Status codes as for ssd_scan_fwd.
 */
int ssd_scan_bwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                 const float* D, const void* z, const float* dt_bias, float dt_min, float dt_max,
                 int chunk_size, int ngroups, const float* initial_states, const void* dout,
                 const float* dfinal_states, void* dx, void* ddt, float* dA, void* dB, void* dC,
                 float* dD, void* dz, float* ddt_bias, float* dinitial_states, int64_t batch,
                 int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace ssd_scan_bwd needs (0 for an empty problem and for
 * rejected arguments); pure host computation. */
size_t ssd_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads,
                                   int64_t headdim, int64_t dstate, int ngroups, int chunk_size,
                                   int dtype);

/* Static text for a status code ("unknown status" for others).  Every case
 * the kernels do not cover gets a code of its own instead of a different
 * result: mamba issue #647 shows a fused kernel that silently diverged for
 * ngroups > 1 and asks whether that was "a not supported feature". */
const char* ssd_status_string(int status);

/* SSD_ABI_VERSION of the loaded library.  Mamba issue #488 shows a change of
 * the positional signature of the CUDA forward breaking a second caller
 * (MambaInnerFn); a caller checks this number against the header it was
 * built with. */
int ssd_abi_version(void);

/*
 * Per-stage timing, for measurement.  A timing object holds HIP events;
 * ssd_scan_fwd_timed behaves exactly like ssd_scan_fwd and also records an
 * event before the first stage and after each stage on `stream`.
 * ssd_timing_read waits for those events and writes the milliseconds spent in
 * each stage (SSD_NUM_STAGES floats: prep -- the dt/cumsum kernel, or the B^T
 * transpose of the bf16 kernels, empty when dt/cumsum is fused into the chunk
 * state --, chunk state, state passing, chunk scan).  On the fused path prep
 * is the set-up kernel, the scan kernel is reported as chunk scan and the two
 * middle stages are empty; on the chain path its kernel is reported as chunk
 * scan (on the segmented chain the unit-state pass as chunk state) and the
 * other stages are empty.  Returns SSD_OK or SSD_ERR_HIP /
 * SSD_ERR_INVALID_ARG.
 */
#define SSD_NUM_STAGES 4
typedef struct ssd_timing ssd_timing;
int ssd_timing_create(ssd_timing** out);
int ssd_timing_destroy(ssd_timing* t);
int ssd_scan_fwd_timed(const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       float dt_min, float dt_max, int chunk_size, int ngroups,
                       const float* initial_states, void* out, float* final_states,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t dstate, int dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, ssd_timing* timing);
int ssd_timing_read(ssd_timing* t, float* stage_ms);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
