// Tile staging shared by the bf16 matrix-core kernels.
#pragma once

#include "ssd_device.h"

namespace ssd {
namespace bf16t {
constexpr int kP = 64;
constexpr int kXLD = 96;  // LDS row stride (bf16) of a staged x tile: conflict-free transposed reads
constexpr float kLog2e = 1.4426950408889634f;

// The x tile in flight: the 16-byte pieces of one thread (256 threads).
template <int Q>
struct XTile {
  static constexpr int ITER = Q * kP / 8 / 256;
  uint4 v[ITER];
};

template <int Q>
__device__ __forceinline__ void load_x_tile(XTile<Q>& t, const bf16_t* xs, int64_t xstride,
                                            int last) {
#pragma unroll
  for (int k = 0; k < XTile<Q>::ITER; ++k) {
    const int e = (k * 256 + (int)threadIdx.x) * 8;
    const int row = e / kP, col = e % kP;
    const int r = row < last ? row : last;
    t.v[k] = *reinterpret_cast<const uint4*>(xs + r * xstride + col);
  }
}

// Writes a loaded x tile to LDS with the column permutation of stage_x_tile.
template <int Q>
__device__ __forceinline__ void store_x_tile(bf16_t* x_lds, const XTile<Q>& t, int last) {
#pragma unroll
  for (int k = 0; k < XTile<Q>::ITER; ++k) {
    const int e = (k * 256 + (int)threadIdx.x) * 8;
    const int row = e / kP, col = e % kP;
    const uint4 v = t.v[k];
    const uint32_t m = row > last ? 0u : 0xffffffffu;
    uint2 even, odd;
    even.x = ((v.x & 0xffffu) | (v.y << 16)) & m;
    even.y = ((v.z & 0xffffu) | (v.w << 16)) & m;
    odd.x = ((v.x >> 16) | (v.y & 0xffff0000u)) & m;
    odd.y = ((v.z >> 16) | (v.w & 0xffff0000u)) & m;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + col / 2) = even;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + 32 + col / 2) = odd;
  }
}

// A row-major R x W bf16 tile in flight (256 threads).
template <int R, int W>
struct RowTile {
  static constexpr int ITER = R * W / 8 / 256;
  static_assert(ITER * 256 * 8 == R * W, "tile must split evenly over 256 threads");
  uint4 v[ITER];
};

template <int R, int W>
__device__ __forceinline__ void load_rows(RowTile<R, W>& t, const bf16_t* src, int64_t stride,
                                          int last) {
#pragma unroll
  for (int k = 0; k < RowTile<R, W>::ITER; ++k) {
    const int e = k * 256 + (int)threadIdx.x;
    const int row = e / (W / 8), col = (e % (W / 8)) * 8;
    const int r = row < last ? row : last;
    t.v[k] = *reinterpret_cast<const uint4*>(src + r * stride + col);
  }
}

template <int R, int W>
__device__ __forceinline__ void store_rows(bf16_t* lds, int ld, const RowTile<R, W>& t, int last) {
#pragma unroll
  for (int k = 0; k < RowTile<R, W>::ITER; ++k) {
    const int e = k * 256 + (int)threadIdx.x;
    const int row = e / (W / 8), col = (e % (W / 8)) * 8;
    *reinterpret_cast<uint4*>(lds + row * ld + col) = row > last ? uint4{0u, 0u, 0u, 0u} : t.v[k];
  }
}

// Stage the x tile of one (chunk, head) into LDS, bf16 bits unchanged, with
// permuted columns: logical column p goes to LDS column 32*(p%2) + p/2, so
// that a transposed read of columns 32*pt + l%32 yields p = 2*(l%32) + pt.
// Rows past `last` are zero.
template <int Q>
__device__ __forceinline__ void stage_x_tile(bf16_t* x_lds, const bf16_t* xs, int64_t xstride,
                                             int last) {
  constexpr int ITER = Q * kP / 8 / 256;  // 16-byte pieces per thread
  const int tid = threadIdx.x;
  uint4 vv[ITER];
#pragma unroll
  for (int k = 0; k < ITER; ++k) {
    const int e = (k * 256 + tid) * 8;
    const int row = e / kP, col = e % kP;
    const int r = row < last ? row : last;
    vv[k] = *reinterpret_cast<const uint4*>(xs + r * xstride + col);
  }
#pragma unroll
  for (int k = 0; k < ITER; ++k) {
    const int e = (k * 256 + tid) * 8;
    const int row = e / kP, col = e % kP;
    const uint4 v = vv[k];
    // elements 0,2,4,6 -> LDS cols col/2 + 0..3; 1,3,5,7 -> 32 + col/2 + 0..3
    const uint32_t m = row > last ? 0u : 0xffffffffu;
    uint2 even, odd;
    even.x = ((v.x & 0xffffu) | (v.y << 16)) & m;
    even.y = ((v.z & 0xffffu) | (v.w << 16)) & m;
    odd.x = ((v.x >> 16) | (v.y & 0xffff0000u)) & m;
    odd.y = ((v.z >> 16) | (v.w & 0xffff0000u)) & m;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + col / 2) = even;
    *reinterpret_cast<uint2*>(x_lds + row * kXLD + 32 + col / 2) = odd;
  }
}

// Eight consecutive bf16 at p (16-byte aligned) as an operand.
__device__ __forceinline__ s16x8 ld_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(s16x8, *reinterpret_cast<const uint4*>(p));
}

// Stage rows 0..R-1 of a row-major bf16 matrix with W columns (row stride
// `stride` elements, 16-byte aligned rows) into LDS with row stride `ld`;
// rows past `last` are zero.
// Needs a 256-thread workgroup; all loads are issued before the LDS stores.
template <int R, int W>
__device__ __forceinline__ void stage_rows(bf16_t* lds, int ld, const bf16_t* src, int64_t stride,
                                           int last) {
  constexpr int ITER = R * W / 8 / 256;  // 16-byte pieces per thread
  static_assert(ITER * 256 * 8 == R * W, "tile must split evenly over 256 threads");
  uint4 v[ITER];
#pragma unroll
  for (int k = 0; k < ITER; ++k) {
    const int e = k * 256 + (int)threadIdx.x;
    const int row = e / (W / 8), col = (e % (W / 8)) * 8;
    const int r = row < last ? row : last;
    v[k] = *reinterpret_cast<const uint4*>(src + r * stride + col);
  }
#pragma unroll
  for (int k = 0; k < ITER; ++k) {
    const int e = k * 256 + (int)threadIdx.x;
    const int row = e / (W / 8), col = (e % (W / 8)) * 8;
    if (row > last) v[k] = uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(lds + row * ld + col) = v[k];
  }
}

}  // namespace bf16t
}  // namespace ssd
