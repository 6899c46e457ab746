// Internal launch interface between the C ABI (ssd_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Segments of the chain bf16 kernel (chain_plan below).
struct ChainPlan {
  int64_t nseg = 1, span = 0, unit = 0, nunits = 0;
};

// One validated problem.  Sizes follow the notation of the scan:
// b = batch, L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups,
// Q = chunk_size, nc = ceil(L / Q).
struct Problem {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // may be null
  const void* z;         // may be null
  const float* dt_bias;  // may be null
  float dt_min, dt_max;
  const float* init;     // may be null
  void* out;
  float* final_states;   // may be null
  const int32_t* seq_idx;  // [b, L] labels of packed sequences; null: one per row
  int64_t b, L, H, P, N, G, Q, nc;
  bool bf16;
  // workspace regions (float32)
  float* ws_dt;          // [b, H, nc, Q]
  float* ws_cum;         // [b, H, nc, Q]
  float* ws_states;      // [b, nc, H] tiled P x N blocks: chunk-local states
  float* ws_states_in;   // [b, nc, H] tiled P x N blocks: state entering each chunk
  uint16_t* ws_bt;       // [b, nc, G] blocks of N x Q bf16: B^T per chunk (bf16 kernels only)
  int32_t* ws_seg;       // [b, nc, Q] sequence starts counted from the chunk start
                         // (seq_idx only; null otherwise)
  float* ws_gram;        // [b, nc, G] causal 32 x 32 tiles of G^T = B C^T per chunk
                         // (gram_tile_floats(Q) floats each, ssd_device.h layout): formed
                         // by the state-passing launch for the four-heads chunk-scan
                         // kernel; null: that kernel forms them itself
  // fused bf16 kernel
  float* fs_ring;        // [b*H chains][2 slots] tiled P x N states
  unsigned* fs_flags;    // [b*H chains][blocks] "state entering this block is ready"
  unsigned* fs_ctl;      // 8 ticket counters, then the error word
  int fused_kind;        // 0: choose, 1: per-head kernel, 2: group kernel
  // chain bf16 kernel: segments, and the unit-state pass's outputs
  ChainPlan chain;
  float* cs_states = nullptr;  // [b, H, nunits] P x N row-major unit end states
  float* cs_decay = nullptr;   // [b, H, nunits] unit decay products
  // Backward re-run only (fp32, four-heads chunk scan): with gate_dout set the
  // chunk scan's epilogue writes dY = dout silu(z) to out and dz = dout y
  // silu'(z) to gate_dz in place of y (z is then the gate input).  z, dout
  // and dz are bf16 when gate_bf16 is set (fp32 otherwise), whatever the
  // other inputs are.
  const void* gate_dout = nullptr;
  void* gate_dz = nullptr;
  bool gate_bf16 = false;
};

// Each launcher enqueues one stage on `stream` and returns hipGetLastError().
hipError_t launch_dt_cumsum(const Problem& p, hipStream_t stream);
// Packed sequences: ws_seg[b][c][q] = number of steps t in [c*Q, c*Q + q]
// (t >= 1, t < L) whose seq_idx differs from step t-1's; constant past L.
hipError_t launch_seq_count(const Problem& p, hipStream_t stream);
hipError_t launch_chunk_state(const Problem& p, hipStream_t stream);
hipError_t launch_state_passing(const Problem& p, hipStream_t stream);
// fp32 stages 2 and 3 as one pass (and stage 1 with them; the chunk scan's
// G^T tiles beside it), for the shapes use_state_scan accepts
bool use_state_scan(bool bf16, bool varlen, int64_t b, int64_t L, int64_t H, int64_t N,
                    int64_t Q);
hipError_t launch_state_scan(const Problem& p, hipStream_t stream);
hipError_t launch_chunk_scan(const Problem& p, hipStream_t stream);

// The four-heads-per-workgroup chunk-scan kernel (fp32 scan of fp32 inputs,
// or of bf16 inputs at chunk 64; Q 64/128, N 64/128, nheads/ngroups a
// multiple of 4).
bool use_group_scan(int64_t H, int64_t N, int64_t G, int64_t Q, bool bf16);
// When that kernel runs with at least two of its workgroups per group and
// chunk (nheads/ngroups >= 8), the state-passing launch forms each chunk's
// tiles of B C^T once per group (ws_gram) and the chunk scan reads them
// instead of forming them in every workgroup of four heads.
bool use_gram(int64_t H, int64_t N, int64_t G, int64_t Q, bool bf16);
// Grid planes (z) of G^T tiles that the state-passing launch adds in front of
// its b planes; the grid's z extent gram_planes + b must stay within 65535.
int64_t gram_planes(int64_t b, int64_t nc, int64_t H, int64_t N, int64_t G, int64_t Q);
// Floats of one (batch, chunk, group) block of ws_gram: the Q/32 (Q/32 + 1) / 2
// causal tiles of 32 x 32.
int64_t gram_tile_floats(int64_t Q);

// True when the chunk-state kernel chosen for this problem also computes dt
// and its in-chunk cumsum (stage 1), so no separate stage-1 launch is needed.
bool chunk_state_fuses_dt(const Problem& p);

// bf16 matrix-core kernels (bf16 inputs, Q 128/256, N 64/128): stage 0 is the
// B^T prep, stage 1 the chunk state (with dt/cumsum fused), stage 2 the chunk
// scan.  The state passing between them is the common stage-3 kernel.
bool use_bf16_kernels(const Problem& p);
hipError_t launch_bf16_stage(const Problem& p, hipStream_t stream, int stage);

// Fused bf16 kernel (bf16 inputs, P 64, N 64/128): stage 0 is the set-up
// kernel, stage 1 the scan.  Blocks of 128 timesteps whatever Q is.
bool use_fused_bf16(const Problem& p);
int64_t fused_blocks(int64_t L);
// Byte offset, inside fs_ctl, of the error word both fused kernels set when a
// workgroup gives up its bounded wait (after the eight ticket counters); the
// set-up kernel clears it on every call.
constexpr size_t kFusedErrorWordByte = 8 * sizeof(unsigned);
hipError_t launch_fused_bf16(const Problem& p, hipStream_t stream, int stage);

// Chain bf16 kernel (bf16 inputs, P 64, N 64/128, an even number of heads
// per group): one workgroup per pair of heads of one group for the whole
// sequence, the state in registers; no workspace.  One workgroup fills one
// of the 256 compute units for the whole call, so it is the default only
// when the pairs fill the machine: each round of 256 workgroups at least 3/4
// full (below that the fused kernel, which spreads the blocks of a chain
// over workgroups, is faster).
constexpr int64_t kChainCUs = 256;
bool use_chain_bf16(const Problem& p);
int64_t chain_workgroups(int64_t b, int64_t H);
bool chain_fills_machine(int64_t b, int64_t H);
// Segmented chain: when the head pairs alone do not fill the machine, the
// sequence is cut into nseg segments of `span` 128-step blocks (one
// workgroup per (pair, segment)); a unit-state launch first computes the
// local end state of every unit of `unit` blocks before the last segment
// (nunits per head), and each segment starts from the units before it folded
// into its entering state.  nseg = 1: the unsegmented chain (no workspace).
// force: segment whenever the sequence has two blocks or more (testing).
ChainPlan chain_plan(int64_t b, int64_t L, int64_t H, bool force);
// pass 0: the unit-state pass (nothing when nseg = 1); pass 1: the chain.
hipError_t launch_chain_bf16(const Problem& p, hipStream_t stream, int pass);
// The unit-state pass of the segmented chain (ssd_fused_bf16.hip): one
// workgroup per (unit, batch, pair of heads) writes cs_states / cs_decay.
hipError_t launch_unit_state_bf16(const Problem& p, hipStream_t stream);

// Group form of the fused kernel: one workgroup per (block, group, head set).
int64_t fused_group_units(const Problem& p);
hipError_t launch_fused_group_bf16(const Problem& p, hipStream_t stream);

// Short sequences: the recurrence step by step, one workgroup per (batch,
// head), no workspace.  Used for seqlen <= kDecodeMaxL whatever the chunk size.
constexpr int kDecodeMaxL = 16;
bool use_decode(int64_t seqlen);
hipError_t launch_decode(const Problem& p, hipStream_t stream);

// Block-level prologue / epilogue around the scan (ssd_block.hip).  The
// prologue turns the packed in-projection zxbcdt [b, L, 2 dim + 2 G N + H]
// into x, B, C (causal depthwise conv of width W + SiLU) and dt; the epilogue
// is the gated RMSNorm out = norm(y * silu(z)) * weight (or the gate alone).
constexpr int kNormMaxDim = 15360;   // channels per token the norm holds in LDS (60 KB)
constexpr int kNormMaxGroups = 256;
struct BlockProblem {
  const void* zxbcdt;
  const float* conv_w;   // [dim + 2 G N, W]
  const float* conv_b;   // [dim + 2 G N], may be null
  int W;
  void* x;               // [b, L, H, P]  prologue outputs (input dtype)
  void* B;               // [b, L, G, N]
  void* C;               // [b, L, G, N]
  void* dt;              // [b, L, H]
  const void* y;         // [b, L, dim] scan output (may be out)
  void* out;             // [b, L, dim]
  const float* norm_w;   // [dim], may be null (gate only)
  float eps;
  int norm_groups;
  int64_t b, L, H, P, N, G;
  bool bf16;
};
bool block_supported(int64_t dim, int norm_groups, int conv_width);
hipError_t launch_conv_split(const BlockProblem& q, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const BlockProblem& q, hipStream_t stream);

// Backward (ssd_backward.hip, fp32).  `fwd` is the forward problem re-run with
// 64-step blocks (Q = 64, nc = bwd_blocks(L)) whose workspace regions hold dt,
// cum, the chunk-local states and the states entering each
// block; fwd.z is the gate input.
struct BwdProblem {
  Problem fwd;
  const float* dout;     // [b, L, H, P]
  const float* dfinal;   // [b, H, P, N], may be null
  float* dy;             // [b, L, H, P]: the ungated y, then dY (without a gate: dout, read only)
  float* gst;            // [b, nb, H] row-major P x N blocks: gradient of each block's end state
  float* dBh;            // [b, L, H, N]: dB parts, one per 1, 2 or 4 heads (H/HPW used)
  float* dCh;            // [b, L, H, N]: parts of dC, the same
  float* dA_p;           // [b, nb, H]
  float* dD_p;           // [b, nb, H]
  float* dx;             // outputs
  float* dz;             // may be null (no gate)
  float* ddt;            // gradient of dt_raw
  float* dA;
  float* dB;
  float* dC;
  float* dD;             // may be null
  float* ddt_bias;       // may be null
  float* dinit;          // may be null
  bool dy_formed = false;  // dY and dz already written by the re-run's chunk scan
};
int64_t bwd_blocks(int64_t L);
hipError_t launch_bwd(const BwdProblem& q, hipStream_t stream);
// bf16 [n] -> fp32 [n] (exact) and fp32 -> bf16 (nearest even), for the
// backward of bf16 inputs.
// Lists of tensors converted by one launch: bf16 -> fp32 (widen) or fp32 ->
// bf16 rounded to nearest even (narrow); count <= kConvMax, n elements each;
// start and vec are filled by the launcher.
constexpr int kConvMax = 6;
struct ConvList {
  const void* src[kConvMax];
  void* dst[kConvMax];
  int64_t n[kConvMax];
  int64_t start[kConvMax + 1];
  bool vec[kConvMax];
  int count = 0;
};
hipError_t launch_widen_bf16(ConvList list, hipStream_t stream);
hipError_t launch_narrow_bf16(ConvList list, hipStream_t stream);

// True when (P, N, Q) is one of the compiled tile configurations.
bool config_supported(int64_t P, int64_t N, int64_t Q);

}  // namespace ssd
