// Device-side helpers shared by the SSD scan kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage of a bfloat16 value

constexpr int kWave = 64;

// ---- element conversion ---------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet bit set).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- loads of 1 / 4 consecutive elements as fp32 --------------------------

__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ float ld1(const bf16_t* p) { return to_f32(*p); }

// p must be aligned to 4 elements.
__device__ __forceinline__ f4 ld4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 ld4(const bf16_t* p) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  f4 r;
  r[0] = bf16_lo(v.x);
  r[1] = bf16_hi(v.x);
  r[2] = bf16_lo(v.y);
  r[3] = bf16_hi(v.y);
  return r;
}

// p must be aligned to 2 elements.
__device__ __forceinline__ f2 ld2(const float* p) { return *reinterpret_cast<const f2*>(p); }
__device__ __forceinline__ f2 ld2(const bf16_t* p) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  f2 r;
  r[0] = bf16_lo(w);
  r[1] = bf16_hi(w);
  return r;
}

__device__ __forceinline__ void st2(float* p, f2 v) { *reinterpret_cast<f2*>(p) = v; }
__device__ __forceinline__ void st2(bf16_t* p, f2 v) {
  *reinterpret_cast<uint32_t*>(p) = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
}

__device__ __forceinline__ void st4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ void st4(bf16_t* p, f4 v) {
  uint2 w;
  w.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
  w.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

// ---- buffer-addressed rows ------------------------------------------------------
// A raw buffer resource over [base, base + bytes): loads at byte offsets past
// the end return 0 and stores there are dropped by the hardware's range check
// (the whole access lies either inside or outside in the uses here).  The
// offset is a 32-bit per-lane value, so a row walk costs one add instead of
// 64-bit address arithmetic, and rows past a sequence's end need no clamp,
// select or branch.  base and bytes must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// one element at byte offset off, as fp32
__device__ __forceinline__ float bld1(__amdgpu_buffer_rsrc_t r, uint32_t off, float) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float bld1(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16_t) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
}
// four consecutive fp32 elements at byte offset off
__device__ __forceinline__ f4 bld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// one fp32 element stored at byte offset off
__device__ __forceinline__ void bst1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}
// four consecutive fp32 elements stored at byte offset off
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t r, uint32_t off, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         r, off, 0, 0);
}
// two consecutive elements at byte offset off, as fp32
__device__ __forceinline__ f2 bld2(__amdgpu_buffer_rsrc_t r, uint32_t off, float) {
  return __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ f2 bld2(__amdgpu_buffer_rsrc_t r, uint32_t off, bf16_t) {
  const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  f2 v;
  v[0] = bf16_lo(w);
  v[1] = bf16_hi(w);
  return v;
}
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, uint32_t off, f2 v, float) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v),
                                        r, off, 0, 0);
}
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, uint32_t off, f2 v, bf16_t) {
  __builtin_amdgcn_raw_buffer_store_b32(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16), r,
                                        off, 0, 0);
}

// ---- matrix core ------------------------------------------------------------
// v_mfma_f32_16x16x4_f32: D[16x16] += A[16x4] * B[4x16].  Lane l supplies
// A[l%16][l/16] and B[l/16][l%16]; D element (row 4*(l/16)+r, col l%16) is
// register r of lane l.
__device__ __forceinline__ f4 mfma16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x2_f32: D[32x32] += A[32x2] * B[2x32].  Lane l supplies
// A[l%32][l/32] and B[l/32][l%32]; register r of lane l holds D element
// (row 8*(r/4) + 4*(l/32) + r%4, col l%32).
__device__ __forceinline__ f16x mfma32x32x2(float a, float b, f16x c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---- bf16 matrix-core operands ------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].  Lane l supplies
// A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; the result has the
// layout of the 32x32x2 fp32 instruction above.
__device__ __forceinline__ f16x mfma32x32x16(s16x8 a, s16x8 b, f16x c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Pack two fp32 into two bf16 (round to nearest even) in one 32-bit word:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight fp32 -> one 8 x bf16 operand.
__device__ __forceinline__ s16x8 to_bf16x8(const float (&v)[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  return __builtin_bit_cast(s16x8, w);
}

// bf16_lo by one v_perm_b32: bytes 1, 0 of w into bytes 3, 2, zeros below.
__device__ __forceinline__ float bf16_lo_perm(uint32_t w) {
  return __uint_as_float(__builtin_amdgcn_perm(0u, w, 0x01000c0cu));
}

// Split eight fp32 into two bf16 operands, hi = bf16(v) and lo = bf16(v - hi)
// (v - hi is exact in fp32).  hi + lo carries 16 significant bits, so the
// pair of products A.hi + A.lo of an exact bf16 operand A is accurate to about
// 2^-16 relative, where a single bf16 operand gives 2^-8.
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], s16x8& hi, s16x8& lo) {
  uint4 h, l;
  h.x = pack_bf16x2(v[0], v[1]);
  h.y = pack_bf16x2(v[2], v[3]);
  h.z = pack_bf16x2(v[4], v[5]);
  h.w = pack_bf16x2(v[6], v[7]);
  // The low half's value is moved up with a byte permute rather than a
  // shift: through a shift the compiler forms it with a conversion of its own
  // and then shifts it, one instruction more per pair.
  l.x = pack_bf16x2(v[0] - bf16_lo_perm(h.x), v[1] - bf16_hi(h.x));
  l.y = pack_bf16x2(v[2] - bf16_lo_perm(h.y), v[3] - bf16_hi(h.y));
  l.z = pack_bf16x2(v[4] - bf16_lo_perm(h.z), v[5] - bf16_hi(h.z));
  l.w = pack_bf16x2(v[6] - bf16_lo_perm(h.w), v[7] - bf16_hi(h.w));
  hi = __builtin_bit_cast(s16x8, h);
  lo = __builtin_bit_cast(s16x8, l);
}

// Transposed read of four bf16 from an LDS tile X (row-major, ld elements per
// row, ld and c0 multiples of 4): lane l receives X[r0 + 0..3][c0 + l%32],
// where r0 may differ between the two halves of the wave (lanes 0-31 and
// 32-63).  ds_read_b64_tr_b16: in every group of 16 lanes, lane 4a + e gets
// element e of the 8-byte words read by lanes a, a+4, a+8, a+12 of the group;
// so lane m of a group reads row r0 + m/4 at column c0 + 16*(group%2) + 4*(m%4).
__device__ __forceinline__ s16x4 lds_tr4(const bf16_t* lds, int ld, int r0, int c0) {
  const int lane = threadIdx.x % 64;
  const int m = lane % 16, half = (lane / 16) % 2;
  const bf16_t* p = lds + (r0 + m / 4) * ld + c0 + 16 * half + 4 * (m % 4);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// B operand of a 32x32x16 MFMA whose contraction index is the row index of an
// LDS tile: lane l supplies rows {r0 + 0..3} and {r1 + 0..3} of column c0 + l%32.
__device__ __forceinline__ s16x8 lds_tr_operand(const bf16_t* lds, int ld, int r0, int r1, int c0) {
  const s16x4 a = lds_tr4(lds, ld, r0, c0), b = lds_tr4(lds, ld, r1, c0);
  s16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

__device__ __forceinline__ f16x zero16() {
  f16x z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// ---- state layout in the workspace ------------------------------------------
// A [P = 64][N] state block is stored in tiles of four consecutive n: the
// float4 at index ((q*2 + pj)*64 + lane) holds row p = 2*(lane%32) + pj,
// columns n = (N/2)*(lane/32) + 4*q + 0..3.  A wave that walks q reads (and
// the chunk-state kernel writes) 1 KB of contiguous memory per instruction.
__device__ __forceinline__ int state_tile_offset(int p, int n, int N) {
  const int half = N / 2;
  const int kk = n / half, q = (n % half) >> 2, e = n & 3;
  return (((q * 2 + (p & 1)) * 64) + 32 * kk + (p >> 1)) * 4 + e;
}
// Row p and first column n of the float4 at tile index k (inverse of above).
__device__ __forceinline__ void state_tile_coords(int k, int N, int* p, int* n) {
  const int lane = k & 63, pj = (k >> 6) & 1, q = k >> 7;
  *p = 2 * (lane & 31) + pj;
  *n = (N / 2) * (lane >> 5) + 4 * q;
}

// ---- tiles of G^T = B C^T (chunk scan) ------------------------------------------
// The causal 32 x 32 tiles (s-tile si <= t-tile ti) of one chunk of one group
// are numbered tau = ti*(ti+1)/2 + si.  A tile is stored in the register order
// of v_mfma_f32_32x32x2_f32: the float4 at ((tau*4 + R)*64 + lane) holds
// registers 4R..4R+3 of that lane, i.e. 1 KB per R, lane-contiguous.
template <int NT>
__device__ __forceinline__ void tile_of(int tau, int* si, int* ti) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (tau >= t * (t + 1) / 2 && tau < (t + 1) * (t + 2) / 2) {
      *ti = t;
      *si = tau - t * (t + 1) / 2;
    }
}

// ---- math -------------------------------------------------------------------

// 2^x on v_exp_f32 (results below the normal range flush to zero) and 1/x on
// v_rcp_f32 (1 ulp): the decays and gates here are all in (0, 1] or feed a
// bf16/fp32 output far coarser than these errors.
// ---- wave-wide scans on the DPP lane moves ---------------------------------

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes within each row of 16, then each row's total broadcast into the rows
// after it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).
// Lanes without a source add 0.  Six register-to-register moves where a
// shuffle-up scan takes six LDS permutes, each waited for.
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}
__device__ __forceinline__ float wave_incl_sum(float v) {
  auto mv = [](float x, int y) { return x + __int_as_float(y); };
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v = mv(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
}
// Sum over the 16 lanes of each row of a wave, every lane of the row left
// with it: the pairings of xor shuffles by 1, 2, 4 and 8 (quad_perm [1,0,3,2]
// and [2,3,0,1], then the half-row and row mirrors) on DPP lane moves.
__device__ __forceinline__ float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
  return v;
}
// Sum over the four rows at each lane position (the pairings of xor shuffles
// by 16 and 32) on the row swaps of gfx950: v_permlane16_swap exchanges the
// odd rows of its first operand with the even rows of its second,
// v_permlane32_swap the upper half of the first with the lower half of the
// second; with both operands v, the two results hold each lane's partner.
__device__ __forceinline__ float rows_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// Sum over the wave, in every lane.
__device__ __forceinline__ float wave_sum(float v) { return rows_sum4(row_sum16(v)); }
// Lane l takes the value of lane 63 - l: the row mirror, then the rows in
// reverse order through the two row swaps.
__device__ __forceinline__ float wave_reverse(float v) {
  const int lane = threadIdx.x % kWave;
  v = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(lane < 32 ? a[1] : a[0]);  // halves exchanged
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((lane & 16) ? c[0] : c[1]);  // rows of each half exchanged
}

// The value of lane `src` (wave-uniform) in every lane: one scalar read.
__device__ __forceinline__ float wave_read(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ int wave_read(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// silu(v) = v * sigmoid(v) = v / (1 + e^-v)
__device__ __forceinline__ float silu(float v) {
  return v * fast_rcp(1.0f + fast_exp2(-v * 1.4426950408889634f));
}

// ---- launch order -------------------------------------------------------------
// Workgroups are handed to the 8 XCDs round-robin (block i -> XCD i % 8).  This
// maps block i to a work index so that consecutive work indices (heads of one
// group, which share B and C) run on the same XCD and share its L2.  It is a
// bijection of [0, nblocks) for any nblocks.
__device__ __forceinline__ int64_t xcd_remap(int64_t i, int64_t nblocks) {
  const int64_t q = nblocks / 8, rem = nblocks % 8;
  const int64_t x = i % 8, k = i / 8;
  return x * q + (x < rem ? x : rem) + k;
}

}  // namespace ssd
