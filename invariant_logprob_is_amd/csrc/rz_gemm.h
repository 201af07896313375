// bf16 MFMA tile core for gfx950 (CDNA4), 64-wide wavefronts.
//
// One workgroup of 256 threads (4 waves) computes a 256 x 256 fp32 tile
//   C[a][b] = sum_k A[a0 + a][k] * B[b0 + b][k]
// where both operands are row-major with K contiguous ("TN"), which is the
// natural layout of hidden states [T,H], the LM-head weight [V,H], a
// probability block [T,V] and a transposed weight [H,V].  Waves form a 2 x 2
// grid, each owning a 128 x 128 sub-tile held as 4 x 4 blocks of the 32x32
// output of v_mfma_f32_32x32x16_bf16.
//
// Operand staging: K is consumed in stages of kBK = 64.  Each stage of both
// operands (2 x 256 rows x 128 B) is loaded with 16-byte global loads into
// registers while the previous stage is multiplied out of LDS, then written
// to the other half of a double buffer.  LDS rows are padded to 144 B so the
// 16-byte fragment reads of 32 consecutive rows are bank-conflict free.
//
// Reduction order: for every output element, the K sum is taken in the same
// fixed order (stage 0, 1, ...; within a stage four MFMA steps of 16) no
// matter which tile, sub-tile, block or lane the element lands in, and no
// matter how many rows are valid.  Rows beyond the valid range are clamped to
// the last valid row; their results are discarded by the caller.
#pragma once

#include "rz_internal.h"

namespace rz {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsStride = kBK + 8;                 // elements per LDS row
constexpr int kStageElems = 2 * kTile * kLdsStride;  // A rows, then B rows
constexpr int kLdsElems = 2 * kStageElems;          // double buffer
constexpr int kThreads = 256;

// Output coordinates of acc[i][j][r] inside the workgroup tile, for lane l of
// wave (wm, wn):
//   a = wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4      (operand-A row)
//   b = wn*128 + j*32 + l%32                          (operand-B row)
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 128 + j * 32 + (lane & 31);
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// A rows [a0, a0+256) clamped to a_rows-1; B rows likewise; ld = row stride
// (elements) of both operands; K a multiple of kBK.  Ends with a barrier, so
// the caller may reuse `lds` immediately.
__device__ __forceinline__ void gemm_tile_256(
    const uint16_t* __restrict__ A, int64_t a0, int64_t a_rows,
    const uint16_t* __restrict__ B, int64_t b0, int64_t b_rows,
    int64_t ld, int K, uint16_t* lds, f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int lrow = tid >> 3;        // 0..31
  const int lcol = (tid & 7) * 8;   // element offset inside a stage row

  const uint16_t* pa = A + a0 * ld;
  const uint16_t* pb = B + b0 * ld;
  uint32_t offa[8], offb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = lrow + 32 * j;
    const int64_t ra = (a0 + r < a_rows ? r : a_rows - 1 - a0);
    const int64_t rb = (b0 + r < b_rows ? r : b_rows - 1 - b0);
    offa[j] = uint32_t(ra * ld + lcol);
    offb[j] = uint32_t(rb * ld + lcol);
  }

  u32x4 ra_[8], rb_[8];
  auto gload = [&](int kt) {
    const uint16_t* ka = pa + int64_t(kt) * kBK;
    const uint16_t* kb = pb + int64_t(kt) * kBK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ra_[j] = *reinterpret_cast<const u32x4*>(ka + offa[j]);
      rb_[j] = *reinterpret_cast<const u32x4*>(kb + offb[j]);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* s = lds + buf * kStageElems;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      *reinterpret_cast<u32x4*>(s + (lrow + 32 * j) * kLdsStride + lcol) = ra_[j];
      *reinterpret_cast<u32x4*>(s + (kTile + lrow + 32 * j) * kLdsStride + lcol) = rb_[j];
    }
  };

  const int nk = K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* s = lds + buf * kStageElems;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[4], bfr[4];
      const int col = kk * 16 + fk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(s + (wm * 128 + i * 32 + frow) * kLdsStride + col);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(s + (kTile + wn * 128 + j * 32 + frow) * kLdsStride + col);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
}

// XCD-aware tile raster.  Workgroups are dealt to the 8 XCDs round-robin by
// id; we undo that so each XCD walks a contiguous range of the logical order,
// and the logical order visits `kTokenGroup` token tiles for every tile of the
// other operand, so the workgroups resident on one XCD share both operands in
// that XCD's L2.  The grid is padded to a multiple of 8; returns false for the
// padding.
__device__ __forceinline__ bool tile_of(int64_t n_token_tiles, int64_t n_other_tiles,
                                        int64_t& tt, int64_t& ot) {
  const uint64_t nb = gridDim.x;
  const uint64_t b = blockIdx.x;
  const uint64_t w = (b & 7) * (nb >> 3) + (b >> 3);
  const uint64_t n_tiles = uint64_t(n_token_tiles) * uint64_t(n_other_tiles);
  if (w >= n_tiles) return false;
  const uint64_t per_group = uint64_t(kTokenGroup) * uint64_t(n_other_tiles);
  const uint64_t g = w / per_group;
  const uint64_t rem = w - g * per_group;
  const uint64_t left = uint64_t(n_token_tiles) - g * kTokenGroup;
  const uint64_t gsz = left < uint64_t(kTokenGroup) ? left : uint64_t(kTokenGroup);
  tt = int64_t(g * kTokenGroup + rem % gsz);
  ot = int64_t(rem / gsz);
  return true;
}

inline uint32_t raster_grid(int64_t n_tiles) { return uint32_t(round_up(n_tiles, 8)); }

}  // namespace rz
