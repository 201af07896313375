// HIP kernels of the learner head for gfx950.  Built with -ffp-contract=off so
// that every fused multiply-add below is an explicit fmaf and the arithmetic a
// row sees is exactly what is written.
#include <math.h>

#include <atomic>

#include "rz_gemm.h"
#include "rz_gemm_tr.h"
#include "rz_util.h"

namespace rz {

// float64 -> bf16, round to nearest even, with a single rounding: round to
// odd at float32 precision (24 bits, >= 8 + 2) and then to nearest even at
// bf16 precision, which composes to the correctly rounded result.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
  const float f = float(d);
  uint32_t u = __float_as_uint(f);
  const double back = double(f);
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // step the magnitude back toward zero
    u |= 1u;                            // sticky bit: round to odd
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Final RMSNorm (forward), one 64-lane wave per row, float64 internally.
//   ms = (1/H) sum_k x_k^2,  r = (ms + eps)^(-1/2),  hhat_k = bf16(gamma_k x_k r)
// Each lane accumulates its strided 8-element chunks in a fixed order; the
// wave then reduces with wave_sum.
// ---------------------------------------------------------------------------
// Loads are issued kNormGroup 16-byte chunks per lane at a time before any is
// used, so a wave has that many in flight instead of one; the arithmetic and
// its order are those of the plain strided loop.
constexpr int kNormGroup = 4;

__device__ __forceinline__ double row_sumsq(const uint16_t* __restrict__ xr, int H, int lane) {
  double ss = 0.0;
  for (int c0 = lane * 8; c0 < H; c0 += kNormGroup * 512) {
    u32x4 v[kNormGroup];
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      const int c = c0 + k * 512;
      v[k] = c < H ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      if (c0 + k * 512 >= H) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = double(__uint_as_float(v[k][q] << 16));
        const double hi = double(__uint_as_float(v[k][q] & 0xFFFF0000u));
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
    }
  }
  return wave_sum(ss);
}

__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ gamma, float eps,
                                                     int64_t T, int H, uint16_t* __restrict__ hhat,
                                                     float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xr = x + t * H;
  const double ss = row_sumsq(xr, H, lane);
  const double r = 1.0 / sqrt(ss / double(H) + double(eps));
  if (rstd && lane == 0) rstd[t] = float(r);
  uint16_t* hr = hhat + t * H;
  for (int c0 = lane * 8; c0 < H; c0 += kNormGroup * 512) {
    u32x4 v[kNormGroup], g[kNormGroup];
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      const int c = c0 + k * 512;
      const bool in = c < H;
      v[k] = in ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
      g[k] = in ? *reinterpret_cast<const u32x4*>(gamma + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      const int c = c0 + k * 512;
      if (c >= H) break;
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double xl = double(__uint_as_float(v[k][q] << 16));
        const double xh = double(__uint_as_float(v[k][q] & 0xFFFF0000u));
        const double gl = double(__uint_as_float(g[k][q] << 16));
        const double gh = double(__uint_as_float(g[k][q] & 0xFFFF0000u));
        const uint32_t yl = f64_to_bf16_rne((gl * xl) * r);
        const uint32_t yh = f64_to_bf16_rne((gh * xh) * r);
        o[q] = yl | (yh << 16);
      }
      *reinterpret_cast<u32x4*>(hr + c) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// RMSNorm backward, in place on dh (fp32), one wave per row.
//   dx_j = r gamma_j g_j - x_j r^3 (1/H) sum_k gamma_k g_k x_k
// r is recomputed with the forward's exact code (row_sumsq), so it has the
// forward's bits.  Loads are grouped as in the forward.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ gamma, float eps,
                                                     int64_t T, int H, float* __restrict__ dh) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* xr = x + t * H;
  float* gr = dh + t * H;
  const double ss = row_sumsq(xr, H, lane);
  const double r = 1.0 / sqrt(ss / double(H) + double(eps));
  // the 8 values of chunk c: x, gamma (bf16) and dh (fp32, two 16-byte halves)
  auto load = [&](int c, u32x4& v, u32x4& g, f32x4& d0, f32x4& d1) {
    v = *reinterpret_cast<const u32x4*>(xr + c);
    g = *reinterpret_cast<const u32x4*>(gamma + c);
    d0 = *reinterpret_cast<const f32x4*>(gr + c);
    d1 = *reinterpret_cast<const f32x4*>(gr + c + 4);
  };
  double sg = 0.0;
  for (int c0 = lane * 8; c0 < H; c0 += kNormGroup * 512) {
    u32x4 v[kNormGroup], g[kNormGroup];
    f32x4 d0[kNormGroup], d1[kNormGroup];
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k)
      if (c0 + k * 512 < H) load(c0 + k * 512, v[k], g[k], d0[k], d1[k]);
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      if (c0 + k * 512 >= H) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double xl = double(__uint_as_float(v[k][q] << 16));
        const double xh = double(__uint_as_float(v[k][q] & 0xFFFF0000u));
        const double gl = double(__uint_as_float(g[k][q] << 16));
        const double gh = double(__uint_as_float(g[k][q] & 0xFFFF0000u));
        const float dl = q < 2 ? d0[k][2 * q] : d1[k][2 * q - 4];
        const float dhh = q < 2 ? d0[k][2 * q + 1] : d1[k][2 * q - 3];
        sg = fma(gl * double(dl), xl, sg);
        sg = fma(gh * double(dhh), xh, sg);
      }
    }
  }
  sg = wave_sum(sg);
  const double c3 = r * r * r * sg / double(H);
  for (int c0 = lane * 8; c0 < H; c0 += kNormGroup * 512) {
    u32x4 v[kNormGroup], g[kNormGroup];
    f32x4 d0[kNormGroup], d1[kNormGroup];
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k)
      if (c0 + k * 512 < H) load(c0 + k * 512, v[k], g[k], d0[k], d1[k]);
#pragma unroll
    for (int k = 0; k < kNormGroup; ++k) {
      const int c = c0 + k * 512;
      if (c >= H) break;
      float o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double xl = double(__uint_as_float(v[k][q] << 16));
        const double xh = double(__uint_as_float(v[k][q] & 0xFFFF0000u));
        const double gl = double(__uint_as_float(g[k][q] << 16));
        const double gh = double(__uint_as_float(g[k][q] & 0xFFFF0000u));
        const float dl = q < 2 ? d0[k][2 * q] : d1[k][2 * q - 4];
        const float dhh = q < 2 ? d0[k][2 * q + 1] : d1[k][2 * q - 3];
        o[2 * q] = float(r * gl * double(dl) - xl * c3);
        o[2 * q + 1] = float(r * gh * double(dhh) - xh * c3);
      }
      *reinterpret_cast<f32x4*>(gr + c) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(gr + c + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

// ---------------------------------------------------------------------------
// LM head forward with a fused per-tile log-sum-exp and target gather.
//
// Operand A = W (vocabulary rows), operand B = hhat (token rows), so each lane
// holds one token column and 16 vocabulary rows per 32x32 block.  For every
// token of the tile the epilogue takes, in this order:
//   1. the tile max M over its 256 vocabulary rows: in-lane over 64 values,
//      then with lane l^32, then between the two waves sharing the column,
//      and the reference m = ceil(M log2 e), an integer in log2 units;
//   2. e = 2^(z log2 e - m) (so 1/2 < max e <= 1) for each of its values and
//      their sum: in-lane in a fixed order, then with lane l^32, then wave
//      (wm=0) + wave (wm=1).  The tile's partial is (M, S); m is recomputed
//      from M with the same float expression wherever it is needed.
// Every token goes through the same operations whatever its column or tile
// position, so the partial (M, S) of a token depends only on that token's
// row.  Partials are written per vocabulary tile and merged by k_lse_combine
// in its fixed two-level order (tiles within each vocabulary split, then the
// splits).  With Store, the values e (rounded to bf16) are also written
// out, straight from registers, in the fragment order of the contraction that
// consumes them (frag_offset, token tiles x 16-wide vocabulary steps):
// lanes l and l+32 of a 32x32 block hold vocabulary rows 8q..8q+3 and
// 8q+4..8q+7 of token l % 32, so one v_permlane32_swap per register pair
// (q, q+1) leaves lane l < 32 with rows 8q..8q+7 and lane l + 32 with rows
// 8q+8..8q+15: exactly one A fragment, stored as a contiguous 1 KB per wave.
// Rows V <= v < Vp hold 0; token columns past T hold finite values that the
// contraction only carries into rows it does not write.  The stored variant
// computes M and S with the same code.
// ---------------------------------------------------------------------------
constexpr int kFwdPipe = 0;
// The persistent forward (k_lmhead_fwd_p) instead of one workgroup per tile.
constexpr bool kFwdPersistent = true;
// Workgroups of the persistent forward: one per CU of the device (256 on
// an MI355X in its whole-chip mode), rounded down to a multiple of the 8
// per-XCD counters.
constexpr int kFwdPersistentGridMax = 256;
constexpr int kMaxDevices = 64;
// The GEMM ring + the exchange area; a ring that fills the LDS holds the
// exchange area in its last 2 KB, used only after the ring's final barrier.
constexpr int fwd_lds(int pipe) { return pipe == 2 ? 5 * kOpStageBytes : kLdsBytes + 2048; }
constexpr int kFwdLds = fwd_lds(kFwdPipe);
// A batch of at most one token tile (the decode-style call of a few rows)
// runs the relaunched forward with the deep ring on W (3 stages of W, 2 of
// hhat: twice the W bytes in flight per CU) and skips the MFMAs of the
// token blocks that hold no row.  Neither moves an MFMA of a valid row, so
// the bits are the same as in any batch.
constexpr int kFwdSmallPipe = 2;

// Steps 1-2 of the epilogue and the partials, on the tile's accumulators.
// Mask: the last vocabulary tile, whose rows v >= V (read as zeros) count as
// -inf.  The masked values are formed on the fly instead of written into
// the accumulators: in-place writes there make the compiler spill in every
// tile's epilogue.
template <bool Store, bool Mask, int NB, int Lds = kFwdLds>
__device__ __forceinline__ void fwd_tile_lse(const f32x16 (&acc)[4][NB], char* lds, int64_t tt,
                                             int64_t vt, int64_t T, int V, int64_t Vp,
                                             float* __restrict__ pm, float* __restrict__ ps,
                                             uint16_t* __restrict__ E) {
  const int64_t v0 = vt * kTile;
  const int64_t t0 = tt * kTile;
  // The lane-derived values are recomputed here from an opaque copy of the
  // thread index rather than kept live from before the main loop, where a
  // persistent caller cannot afford the registers.
  int tid = int(threadIdx.x);
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int half = lane >> 5;
  const int col = lane & 31;
  float* xch = reinterpret_cast<float*>(lds + Lds - 2048);
  // rows of this lane below V: acc_row(wm, i, r, lane) < V - v0, i.e. the
  // block offset i*32 + 8*(r/4) + r%4 (a constant of the unrolled loops)
  // below lim (the last tile only, so lim < 256)
  const int lim = Mask ? int(int64_t(V) - v0) - (wm * 128 + 4 * (lane >> 5)) : 0;
  auto val = [&](int i, int j, int r) -> float {
    return (!Mask || i * 32 + 8 * (r >> 2) + (r & 3) < lim) ? acc[i][j][r] : -INFINITY;
  };

  // 1. tile max
  float Mj[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, val(i, j, r));
    Mj[j] = fmaxf(m, __shfl_xor(m, 32, 64));
  }
  if (half == 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) xch[(wm * 8 + wn * NB + j) * 32 + col] = Mj[j];
  }
  // The exchanges below order LDS traffic only: a bare barrier, so the
  // e stores already issued keep draining instead of being waited for.
  GemmCore::barrier();
#pragma unroll
  for (int j = 0; j < NB; ++j) Mj[j] = fmaxf(Mj[j], xch[((wm ^ 1) * 8 + wn * NB + j) * 32 + col]);

  // 2. e = 2^(z log2 e - m) and its sum (order: i, then r); with Store, e is
  // packed to bf16 and written out as A fragments (see above), one 32x32
  // block at a time to keep few values live.
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int64_t n_ks = Vp / 16;
  // The e of this (token tile, vocabulary tile) pair is one contiguous block
  // of 16 steps x 8 fragments: the stores address it from a uniform base
  // with 32-bit offsets (a per-lane part and a constant per store).  Steps at
  // or past n_ks exist only in the last vocabulary tile; a wave's steps are
  // wm*8 .. wm*8+7, so the check is uniform per wave.
  char* eb = nullptr;
  uint32_t evo = 0;
  int nvs = 0;   // valid steps of this wave's eight
  if (Store) {
    const int64_t ks_first = v0 / 16;
    eb = reinterpret_cast<char*>(E) + frag_offset(tt, ks_first, 0, n_ks);
    evo = uint32_t(lane * 16 + wn * NB * 1024 + wm * 8 * 8 * 1024);
    const int64_t tile_steps = n_ks - ks_first;    // >= 1
    const int left = int(tile_steps < 16 ? tile_steps : 16) - __builtin_amdgcn_readfirstlane(wm) * 8;
    nvs = __builtin_amdgcn_readfirstlane(left < 0 ? 0 : left);
  }
  float Sj[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float s = 0.0f;
    // A column whose values are all -inf gets reference +inf: its exponents
    // are -inf and its e exactly 0, with no select per value.
    const float mb = Mj[j] != -INFINITY ? tile_ref(Mj[j]) : INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 X[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          e[q] = __builtin_amdgcn_exp2f(fmaf(val(i, j, r4 * 4 + q), kLog2e, -mb));
          s += e[q];
        }
        if (Store) {
          X[r4][0] = pack_bf16x2(e[0], e[1]);
          X[r4][1] = pack_bf16x2(e[2], e[3]);
        }
      }
      if (Store) {
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          const auto d0 = __builtin_amdgcn_permlane32_swap(X[2 * qp][0], X[2 * qp + 1][0], false, false);
          const auto d1 = __builtin_amdgcn_permlane32_swap(X[2 * qp][1], X[2 * qp + 1][1], false, false);
          u32x4 f;
          f[0] = d0[0];
          f[1] = d1[0];
          f[2] = d0[1];
          f[3] = d1[1];
          // step wm*8 + 2i + qp of the block, fragment wn*NB + j
          const uint32_t soff = uint32_t(((i * 2 + qp) * 8 + j) * 1024);
          if (i * 2 + qp < nvs)
            __builtin_nontemporal_store(f, reinterpret_cast<u32x4*>(eb + (evo + soff)));
        }
      }
    }
    Sj[j] = s + __shfl_xor(s, 32, 64);
  }
  GemmCore::barrier();  // everyone has read the maxima
  if (wm == 1 && half == 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) xch[(wn * NB + j) * 32 + col] = Sj[j];
  }
  GemmCore::barrier();
  if (wm == 0 && half == 0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t t = t0 + acc_col(wn, j, lane, NB);
      if (t < T) {
        pm[vt * T + t] = Mj[j];
        ps[vt * T + t] = Sj[j] + xch[(wn * NB + j) * 32 + col];
      }
    }
  }
}

// Eight waves, two per SIMD (128 x 64 of the tile each): one wave's MFMAs
// issue while the other of its SIMD waits on LDS, loads or the barrier, and
// the accumulators live in VGPRs, which the epilogue reads directly.
constexpr int kFwdWaves = 8;

// The targets of the lane's token columns of token tile tt (0 past T), as
// stored.  Loaded before the main loop and used only in the epilogue, so the
// epilogue issues no load that the memory operations in flight would have to
// drain for.
template <int NB>
__device__ __forceinline__ void fwd_targets(const int32_t* __restrict__ target, int64_t tt,
                                            int64_t T, int32_t (&tg)[NB]) {
  const int lane = threadIdx.x & 63;
  const int wn = (threadIdx.x >> 6) >> 1;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t t = tt * kTile + acc_col(wn, j, lane, NB);
    tg[j] = t < T ? target[t] : 0;
  }
}

// The epilogue of one forward tile (vocabulary tile vt, token tile tt) on its
// accumulators: the target gather (tg from fwd_targets), then the tile's
// partials and (Store) the stored e.
template <bool Store, int NB, int Lds = kFwdLds>
__device__ __forceinline__ void fwd_epilogue(const f32x16 (&acc)[4][NB], char* lds, int64_t tt,
                                             int64_t vt, const int32_t (&tgs)[NB],
                                             int64_t tgt_off, int64_t T, int V, int64_t Vp,
                                             float* __restrict__ pm,
                                             float* __restrict__ ps, float* __restrict__ ztgt,
                                             uint16_t* __restrict__ E) {
  const int64_t v0 = vt * kTile;
  const int64_t t0 = tt * kTile;
  int tid = int(threadIdx.x);
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int half = lane >> 5;
  const int64_t vbase = v0 + wm * 128;

  // Target gather: exactly one lane of one workgroup holds z[t, target[t]]
  // (target rows relative to W's first row).
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t t = t0 + acc_col(wn, j, lane, NB);
    if (t < T) {
      const int64_t tg = int64_t(tgs[j]) - tgt_off;
      const int64_t loc = tg - vbase;
      if (tg >= 0 && tg < V && loc >= 0 && loc < 128) {
        const int q = int(loc & 31);
        if (((q >> 2) & 1) == half) {
          const int ib = int(loc >> 5);
          const int rb = ((q >> 3) << 2) | (q & 3);
          float val = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (i == ib && r == rb) val = acc[i][j][r];
          ztgt[t] = val;
        }
      }
    }
  }

  if (v0 + kTile > V)
    fwd_tile_lse<Store, true, NB, Lds>(acc, lds, tt, vt, T, V, Vp, pm, ps, E);
  else
    fwd_tile_lse<Store, false, NB, Lds>(acc, lds, tt, vt, T, V, Vp, pm, ps, E);
}

template <bool Store, int Pipe = kFwdPipe>
__global__ __launch_bounds__(64 * kFwdWaves)
__attribute__((amdgpu_waves_per_eu(kFwdWaves / 4, kFwdWaves / 4)))
void k_lmhead_fwd(const uint16_t* __restrict__ hhat, const uint16_t* __restrict__ W,
                  const int32_t* __restrict__ target, int64_t tgt_off, int64_t T, int H, int V,
                  int64_t n_vt, int64_t n_tt, int64_t Vp, float* __restrict__ pm,
                  float* __restrict__ ps, float* __restrict__ ztgt, uint16_t* __restrict__ E, int raster_group) {
  constexpr int kLds = fwd_lds(Pipe);
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  int64_t tt, vt;
  // Vocabulary tiles are grouped (raster_group of them, chosen on the host
  // from H so that the group's W rows and the chunk's hhat fit the MALL
  // together) and the token tiles stream past them: the chunk's hhat
  // (100 MB at H = 1536) stays cache-resident across the groups, where
  // re-streaming W (467 MB) from HBM for every token group would not.
  if (!tile_of(n_vt, n_tt, vt, tt, raster_group)) return;
  using Core = GemmCoreT<false, false, kFwdWaves, 4, Pipe>;
  static_assert(Core::kLds <= kLds, "LDS");
  Core g;
  int32_t tg[Core::kNB];
  fwd_targets<Core::kNB>(target, tt, T, tg);
  g.init(W, vt * kTile, V, hhat, tt * kTile, T, H, lds);
  if ((tt + 1) * kTile <= T) {
    g.run(H);
  } else {
    // token blocks (32 rows) of this wave below T
    const int wn = Core::wave_n(__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)));
    const int64_t left = T - tt * kTile - int64_t(wn) * Core::kNB * 32;
    g.nbv = left <= 0 ? 0 : (left >= Core::kNB * 32 ? Core::kNB : int((left + 31) / 32));
    g.template run<true>(H);
  }
#pragma unroll
  for (int j = 0; j < Core::kNB; ++j) asm volatile("" : "+v"(tg[j]));
  fwd_epilogue<Store, Core::kNB, kLds>(g.acc, lds, tt, vt, tg, tgt_off, T, V, Vp, pm, ps, ztgt,
                                       E);
}

// The forward of a batch of at most R rows (R = 64 or 128, the decode-style
// call): the token rows of the first R / 64 wave columns of k_lmhead_fwd's
// tile.  Its stages hold R hhat rows (8 or 16 KB) instead of 256, which
// leaves the LDS for a deeper ring on W: 4 stages at R = 64, 3 at R = 128,
// against one W stage in flight in the 256-row tile.  The waves of those
// columns read the same fragments and run the same MFMAs in the same order on
// the same accumulators as in k_lmhead_fwd, skipping the 32-row blocks with
// no row, and all waves take the same epilogue, so every row keeps its bits.
template <int R>
struct FewFwd {
  static_assert(R == 64 || R == 128, "64 or 128 rows");
  static constexpr int kBStage = R * kRowBytes;                          // 8 or 16 KB
  static constexpr int kStages = R == 64 ? 4 : 3;
  static constexpr int kLds = kStages * (kOpStageBytes + kBStage);        // 160 or 144 KB
  static constexpr int kBLoads = R / kRowsPerLoad / kFwdWaves;            // 1 or 2 per wave
  static constexpr int kLoads = 4 + kBLoads;                              // per wave and stage
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert(kFwdWaves == 8 && kBK == 64, "4 W loads per wave and stage");
};

// vmcnt(L n): wait until at most n stages of this wave's loads (L of them
// per stage) are in flight.
template <int L>
__device__ __forceinline__ void few_wait(int n) {
  static_assert(2 * L <= 15, "vmcnt low bits");
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | L); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * L)); break;
  }
}

template <bool Store, int R>
__global__ __launch_bounds__(64 * kFwdWaves)
__attribute__((amdgpu_waves_per_eu(kFwdWaves / 4, kFwdWaves / 4)))
void k_lmhead_fwd_few(const uint16_t* __restrict__ hhat, const uint16_t* __restrict__ W,
                      const int32_t* __restrict__ target, int64_t tgt_off, int64_t T, int H,
                      int V, int64_t n_vt, int64_t Vp, float* __restrict__ pm,
                      float* __restrict__ ps, float* __restrict__ ztgt,
                      uint16_t* __restrict__ E, int raster_group) {
  using F = FewFwd<R>;
  __shared__ __attribute__((aligned(16))) char lds[F::kLds];
  int64_t vt, tt;
  if (!tile_of(n_vt, 1, vt, tt, raster_group)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(W, vt * kTile, V, H);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(hhat, 0, T, H);   // rows >= T read as 0
  const uint32_t ldb = uint32_t(H) * 2u;
  // load instruction q of a stage moves rows 8q .. 8q+7 into LDS bytes
  // [1024 q, 1024 q + 1024), lane l's 16 bytes at slot l % 8 of its row,
  // holding global chunk (l % 8) ^ swz(row): W's q = 4 wave + j, hhat's
  // q = kBLoads wave + j
  uint32_t va[4], vb[F::kBLoads];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t row = uint32_t((wave * 4 + j) * kRowsPerLoad + lane / kChunks);
    va[j] = row * ldb + ((uint32_t(lane % kChunks) ^ swz(row)) << 4);
  }
#pragma unroll
  for (int j = 0; j < F::kBLoads; ++j) {
    const uint32_t row = uint32_t((wave * F::kBLoads + j) * kRowsPerLoad + lane / kChunks);
    vb[j] = row * ldb + ((uint32_t(lane % kChunks) ^ swz(row)) << 4);
  }
  auto issue = [&](int st) {
    char* sa = lds + (st % F::kStages) * kOpStageBytes;
    char* sb = lds + F::kStages * kOpStageBytes + (st % F::kStages) * F::kBStage;
    const int soff = st * kRowBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t vo = va[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sa + (wave * 4 + j) * 1024), 16,
                                               vo, soff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < F::kBLoads; ++j) {
      const uint32_t vo = vb[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (lds_void_t*)(sb + (wave * F::kBLoads + j) * 1024), 16, vo, soff, 0, 0);
    }
  };

  // 32-row blocks of this wave's token rows (wn * 64 ...) below T
  const int64_t left = T - int64_t(wn) * 64;
  const int nbv = (wn >= R / 64 || left <= 0) ? 0 : (left >= 64 ? 2 : int((left + 31) / 32));
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  int32_t tg[2];
  fwd_targets<2>(target, tt, T, tg);

  const int nk = H / kBK;
  const int pre = nk < F::kStages - 1 ? nk : F::kStages - 1;
  for (int st = 0; st < pre; ++st) issue(st);
  few_wait<F::kLoads>(pre - 1);
  GemmCore::barrier();
  const uint32_t r32 = uint32_t(lane & 31);
  const uint32_t slot0 = (uint32_t(lane >> 5) ^ swz(r32)) << 4;
  const uint32_t aoff = uint32_t(wm * 128 + int(r32)) * kRowBytes + slot0;
  const uint32_t boff = uint32_t(wn * 64 + int(r32)) * kRowBytes + slot0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + F::kStages - 1 < nk) issue(kt + F::kStages - 1);
    if (nbv > 0) {
      const char* sa = lds + (kt % F::kStages) * kOpStageBytes;
      const char* sb = lds + F::kStages * kOpStageBytes + (kt % F::kStages) * F::kBStage;
#pragma unroll
      for (int kk = 0; kk < kSteps; ++kk) {
        const uint32_t oa = aoff ^ uint32_t(kk << 5);
        const uint32_t ob = boff ^ uint32_t(kk << 5);
        bf16x8 fa[4], fb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const bf16x8*>(sa + oa + i * 32 * kRowBytes);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[j] = *reinterpret_cast<const bf16x8*>(sb + ob + j * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (j < nbv)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0,
                                                                  0);
      }
    }
    if (kt + 1 < nk) {
      // stage kt+1 complete; the stages after it stay in flight
      const int last = kt + F::kStages - 1 < nk - 1 ? kt + F::kStages - 1 : nk - 1;
      few_wait<F::kLoads>(last - (kt + 1));
      GemmCore::barrier();
    }
  }
  GemmCore::barrier();
#pragma unroll
  for (int j = 0; j < 2; ++j) asm volatile("" : "+v"(tg[j]));
  fwd_epilogue<Store, 2, F::kLds>(acc, lds, tt, vt, tg, tgt_off, T, V, Vp, pm, ps, ztgt, E);
}

// The same forward with one workgroup per CU: each takes the logical tile
// positions of its XCD's range of the raster order (workgroup b runs on XCD
// b % 8) from that XCD's counter, ticket[b % 8], so the XCD's workgroups run
// the range in the order a relaunched grid would, and it issues the next
// tile's first stage as soon as a tile's main loop is done, so those loads
// overlap the tile's epilogue instead of following a relaunch.  The counter
// of the next tile is fetched while the main loop runs.  Which workgroup
// computes a tile changes no bit of it.
template <bool Store>
__global__ __launch_bounds__(64 * kFwdWaves)
__attribute__((amdgpu_waves_per_eu(kFwdWaves / 4, kFwdWaves / 4)))
void k_lmhead_fwd_p(const uint16_t* __restrict__ hhat, const uint16_t* __restrict__ W,
                    const int32_t* __restrict__ target, int64_t tgt_off, int64_t T, int H, int V,
                    int64_t n_vt, int64_t n_tt, int64_t Vp, float* __restrict__ pm,
                    float* __restrict__ ps, float* __restrict__ ztgt, uint16_t* __restrict__ E,
                    int raster_group, int64_t n_logical, int* __restrict__ ticket) {
  // One LDS object: the ticket broadcast lives past the ring and the
  // exchange area.  A second __shared__ variable would give LDS accesses
  // alias scopes, and the compiler then waits for every LDS-direct load in
  // flight before each fragment read of the main loop.
  __shared__ __attribute__((aligned(16))) char lds[kFwdLds + 16];
  int& nextk = *reinterpret_cast<int*>(lds + kFwdLds);
  using Core = GemmCoreT<false, false, kFwdWaves, 4, kFwdPipe>;
  const int x = blockIdx.x & 7;
  const int64_t per = n_logical >> 3;
  if (threadIdx.x == 0) nextk = atomicAdd(ticket + x, 1);
  __syncthreads();
  int64_t vt, tt;
  if (nextk >= per || !tile_at(uint64_t(x * per + nextk), n_vt, n_tt, vt, tt, raster_group)) return;
  Core g;
  int32_t tg[Core::kNB];
  g.init(W, vt * kTile, V, hhat, tt * kTile, T, H, lds);
  g.issue_first();
  while (true) {
    g.begin_tile();
    fwd_targets<Core::kNB>(target, tt, T, tg);
    int k = 0;
    if (threadIdx.x == 0) k = atomicAdd(ticket + x, 1);
    g.mainloop(H);
    // the targets and the counter are first used here: their loads have
    // completed during the main loop, and nothing before it waits for them
#pragma unroll
    for (int j = 0; j < Core::kNB; ++j) asm volatile("" : "+v"(tg[j]));
    if (threadIdx.x == 0) nextk = k;
    Core::barrier();
    k = nextk;
    int64_t nvt = 0, ntt = 0;
    const bool more = k < per && tile_at(uint64_t(x * per + k), n_vt, n_tt, nvt, ntt,
                                         raster_group);
    if (more) {
      g.retile(W, nvt * kTile, V, hhat, ntt * kTile, T, H);
      g.issue_first();
    }
    fwd_epilogue<Store, Core::kNB>(g.acc, lds, tt, vt, tg, tgt_off, T, V, Vp, pm, ps, ztgt, E);
    if (!more) break;
    vt = nvt;
    tt = ntt;
  }
}

// Shift table and row factor that turn the stored e of a token back into its
// probabilities: with m = max_j m_j over the tile references,
//   p_v = e_v 2^(m_j - m) * 2^m exp(-lse) = (e_v >> d_j) * g,
// d_j = m - m_j (a bf16 exponent shift, 255 = flush), g = exp(m ln 2 - lse).
// D[j * ds + t] holds d_j << 7 in both 16-bit halves.  lse is the float value
// handed out, so the step and the stand-alone backward agree bit for bit.
__device__ __forceinline__ void shift_range(const float* __restrict__ pm, int64_t T, int64_t t,
                                            int64_t j0, int64_t j1, float m,
                                            uint32_t* __restrict__ D, int64_t ds) {
#pragma unroll 8
  for (int64_t j = j0; j < j1; ++j) {
    const float dm = m - tile_ref(pm[j * T + t]);
    const uint32_t d = (dm >= 0.0f && dm < 255.0f) ? uint32_t(dm) : 255u;
    D[j * ds + t] = (d << 7) | (d << 23);
  }
}

__device__ __forceinline__ float row_factor(float m, float lse_f) {
  return float(exp(double(m) * kLn2 - double(lse_f)));
}

__device__ __forceinline__ void shift_tables(const float* __restrict__ pm, int64_t T, int64_t n_vt,
                                             int64_t t, float m, float lse_f,
                                             uint32_t* __restrict__ D, int64_t ds,
                                             float* __restrict__ g) {
  shift_range(pm, T, t, 0, n_vt, m, D, ds);
  g[t] = row_factor(m, lse_f);
}

// max_j M_j (natural units) over the tiles of token t.
__device__ __forceinline__ float max_tile_max(const float* __restrict__ pm, int64_t T,
                                              int64_t n_vt, int64_t t) {
  float M = -INFINITY;
#pragma unroll 8
  for (int64_t j = 0; j < n_vt; ++j) M = fmaxf(M, pm[j * T + t]);
  return M;
}

// One vocabulary split's partial of a row, over its tiles j0 .. j1-1 in
// order, in float64: mx = max_j M_j, m = tile_ref(mx) (= max_j m_j, since
// tile_ref is monotone) and s = sum_j S_j 2^(m_j - m).  An empty split (or
// one whose tiles are all -inf) gives s = 0, m = mx = -inf.
struct SplitPart {
  double s;
  float m, mx;
};

__device__ __forceinline__ SplitPart split_part(const float* __restrict__ pm,
                                                const float* __restrict__ ps, int64_t T,
                                                int64_t t, int64_t j0, int64_t j1) {
  // Loads go out kU at a time (the loops are latency bound); the reductions
  // still run j = j0, j0+1, ... one after another.
  constexpr int kU = 8;
  float mx = -INFINITY;
  int64_t j = j0;
  for (; j + kU <= j1; j += kU) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = pm[(j + u) * T + t];
#pragma unroll
    for (int u = 0; u < kU; ++u) mx = fmaxf(mx, v[u]);
  }
  for (; j < j1; ++j) mx = fmaxf(mx, pm[j * T + t]);
  const float m = tile_ref(mx);
  double sum = 0.0;
  j = j0;
  for (; j + kU <= j1; j += kU) {
    float mj[kU], sj[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      mj[u] = pm[(j + u) * T + t];
      sj[u] = ps[(j + u) * T + t];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (mj[u] != -INFINITY)
        sum += ldexp(double(sj[u]), int(fmaxf(tile_ref(mj[u]) - m, -4096.0f)));
  }
  for (; j < j1; ++j) {
    const float mj = pm[j * T + t];
    if (mj != -INFINITY)
      sum += ldexp(double(ps[j * T + t]), int(fmaxf(tile_ref(mj) - m, -4096.0f)));
  }
  return {sum, m, mx};
}

// Merge of a row's kVocabSplits split partials, in split order, in float64:
// with m = max_s m_s, lse = max(m ln 2 + log sum_s s_s 2^(m_s - m), max_s mx_s)
// (the max keeps lse >= every logit against the rounding of the sums).
// part(s) returns split s's partial; m is returned for the shift table.
template <class Part>
__device__ __forceinline__ double merge_splits(Part part, float& m_out) {
  float m = -INFINITY, mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < kVocabSplits; ++q) {
    m = fmaxf(m, part(q).m);
    mx = fmaxf(mx, part(q).mx);
  }
  double sum = 0.0;
#pragma unroll
  for (int q = 0; q < kVocabSplits; ++q)
    if (part(q).m != -INFINITY) sum += ldexp(part(q).s, int(fmaxf(part(q).m - m, -4096.0f)));
  m_out = m;
  return fmax(double(m) * kLn2 + log(sum), double(mx));
}

// The log-sum-exp of each token from its per-tile partials (M_j, S_j): split
// partials over each split's tiles, then their merge (both in order),
// logprob = z_target - lse.  If cs is given (learner step), also
// coef = cs * exp(logprob - mu), the same expression rz_is_loss evaluates,
// and if D is given the shift table and row factor of the stored e.
// A block covers 64 tokens with one wave per split: wave q reduces split q's
// tiles for its lane's token (coalesced along tokens), wave 0 merges the 8
// partials in split order, and each wave then writes its tiles' shifts.
constexpr int kCombineThreads = 64 * kVocabSplits;

__global__ __launch_bounds__(kCombineThreads) void k_lse_combine(
    const float* __restrict__ pm, const float* __restrict__ ps, const float* __restrict__ ztgt,
    int64_t T, int64_t n_vt, float* __restrict__ logprob, float* __restrict__ lse,
    const double* __restrict__ cs, const float* __restrict__ mu, float* __restrict__ coef,
    uint32_t* __restrict__ D, int64_t ds, float* __restrict__ g) {
  __shared__ SplitPart part[kVocabSplits][64];
  __shared__ float mref[64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 64 + lane;
  const bool live = t < T;
  const int64_t j0 = n_vt * q / kVocabSplits, j1 = n_vt * (q + 1) / kVocabSplits;
  if (live) part[q][lane] = split_part(pm, ps, T, t, j0, j1);
  __syncthreads();
  if (q == 0 && live) {
    float m;
    const double l =
        merge_splits([&](int s) -> const SplitPart& { return part[s][lane]; }, m);
    const float lp = float(double(ztgt[t]) - l);
    const float lf = float(l);
    logprob[t] = lp;
    if (lse) lse[t] = lf;
    if (cs) coef[t] = float(cs[t] * exp(double(lp) - double(mu[t])));
    if (D) g[t] = row_factor(m, lf);
    mref[lane] = m;
  }
  if (D) {
    __syncthreads();
    if (live) shift_range(pm, T, t, j0, j1, mref[lane], D, ds);
  }
}

// One row's record of one vocabulary split (struct rz_vocab_split).
struct SplitRec {
  double s;
  float m, mx, z, pad;
};
static_assert(sizeof(SplitRec) == 24, "record layout");

// Records of splits [s0, s1) of a model with n_vt vocabulary tiles and V
// rows, from the tile partials of a forward over those splits' rows (its
// tile 0 is split s0's first tile).  z is the target logit in the split
// that holds the target row and 0 in the others.
__global__ __launch_bounds__(256) void k_split_partials(const float* __restrict__ pm,
                                                        const float* __restrict__ ps,
                                                        const float* __restrict__ ztgt,
                                                        const int32_t* __restrict__ target,
                                                        int64_t T, int V, int64_t n_vt, int s0,
                                                        int s1, SplitRec* __restrict__ out,
                                                        int64_t out_stride) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  const int64_t jb = n_vt * s0 / kVocabSplits;
  const int64_t tg = target[t];
  for (int q = s0; q < s1; ++q) {
    const int64_t j0 = n_vt * q / kVocabSplits, j1 = n_vt * (q + 1) / kVocabSplits;
    const SplitPart p = split_part(pm, ps, T, t, j0 - jb, j1 - jb);
    const bool owner = tg >= j0 * kTile && tg < j1 * kTile && tg < V;
    out[(q - s0) * out_stride + t] = {p.s, p.m, p.mx, owner ? ztgt[t] : 0.0f, 0.0f};
  }
}

// logprob and lse of each row from all of its split records: the merge of
// k_lse_combine, z = the sum of the records' z (one of them is the target
// logit), NaN for a target outside [0, V).
__global__ __launch_bounds__(256) void k_split_merge(const SplitRec* __restrict__ parts,
                                                     int64_t part_stride,
                                                     const int32_t* __restrict__ target,
                                                     int64_t T, int V, float* __restrict__ logprob,
                                                     float* __restrict__ lse) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  SplitPart P[kVocabSplits];
  float z = 0.0f;
#pragma unroll
  for (int q = 0; q < kVocabSplits; ++q) {
    const SplitRec r = parts[q * part_stride + t];
    P[q] = {r.s, r.m, r.mx};
    z += r.z;
  }
  const int32_t tg = target[t];
  if (tg < 0 || tg >= V) z = NAN;
  float m;
  const double l = merge_splits([&](int q) -> const SplitPart& { return P[q]; }, m);
  logprob[t] = float(double(z) - l);
  if (lse) lse[t] = float(l);
}

// The same shift table and row factor from a given lse (stand-alone backward).
__global__ __launch_bounds__(256) void k_shift_prep(const float* __restrict__ pm, int64_t T,
                                                    int64_t n_vt, const float* __restrict__ lse,
                                                    uint32_t* __restrict__ D, int64_t ds,
                                                    float* __restrict__ g) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  shift_tables(pm, T, n_vt, t, tile_ref(max_tile_max(pm, T, n_vt, t)), lse[t], D, ds, g);
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Backward pieces.
// ---------------------------------------------------------------------------

// Wt[h][v] = W[v][h] for v < V, 0 for V <= v < Vp.  64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void k_transpose_w(const uint16_t* __restrict__ W, int H, int V,
                                                     int64_t Vp, uint16_t* __restrict__ Wt) {
  __shared__ uint16_t tile[64][65];
  const int64_t v0 = int64_t(blockIdx.x) * 64;
  const int h0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t v = v0 + r;
    tile[r][tx] = (v < V) ? W[v * H + h0 + tx] : uint16_t(0);
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t v = v0 + tx;
    if (v < Vp) Wt[int64_t(h0 + r) * Vp + v] = tile[tx][r];
  }
}

// dhhat[t][h] = coef_t * (W[target_t][h] - sum_v p_tv W[v][h]) for a chunk,
// with p_tv = (e_tv >> d(t, v / 256)) * g_t rebuilt from the stored e
// (k_lmhead_fwd) and the shift table (shift_tables): the exponent shift is
// applied to the A fragments inside the contraction, g_t to its result.
// Operand A = E (token rows, K = padded vocabulary, in fragment order),
// operand B = Wt (hidden rows).  The one-hot term is gathered from W exactly
// in fp32.
// Eight waves, two per SIMD, as a 4 x 2 grid of 64 x 128 sub-tiles: two A
// fragments (token rows) per step carry the exponent shift, half as many as
// in a 128-row sub-tile.
constexpr int kDhWaves = 8;
// Rows of an accumulator block whose epilogue loads are issued together.
constexpr int kEpiRows = 4;
constexpr int kDhABlocks = 2;
constexpr int kDhPipe = 2;   // the deep A ring: e is streamed from HBM

__global__ __launch_bounds__(64 * kDhWaves)
__attribute__((amdgpu_waves_per_eu(kDhWaves / 4, kDhWaves / 4)))
void k_dhidden(const uint16_t* __restrict__ E, const uint32_t* __restrict__ D, int64_t ds,
               const float* __restrict__ gf, const uint16_t* __restrict__ Wt,
               const uint16_t* __restrict__ W, const int32_t* __restrict__ target,
               const float* __restrict__ coef, int64_t TC, int H, int V, int64_t Vp,
               int64_t n_tt, int64_t n_ht, float* __restrict__ dh) {
  using Core = GemmCoreT<true, true, kDhWaves, kDhABlocks, kDhPipe>;
  __shared__ __attribute__((aligned(16))) char lds[Core::kLds];
  int64_t tt, ht;
  if (!tile_of(n_tt, n_ht, tt, ht)) return;
  const int64_t t0 = tt * kTile;
  const int64_t h0 = ht * kTile;
  Core g;
  g.init(E, t0, TC, Wt, h0, H, Vp, lds);
  g.set_shift(D, ds, t0, (int64_t(V) + kTile - 1) / kTile);
  g.run(int(Vp));
  f32x16 (&acc)[Core::kNA][Core::kNB] = g.acc;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = Core::wave_m(wave);
  const int wn = Core::wave_n(wave);
  // kEpiRows rows at a time: their targets, scales and target-row weights are all
  // loaded before the first is used, so the loads are in flight together
  // instead of one round trip per output.
#pragma unroll
  for (int i = 0; i < Core::kNA; ++i) {
#pragma unroll
    for (int rq = 0; rq < 16 / kEpiRows; ++rq) {
      int64_t t[kEpiRows];
      int32_t tg[kEpiRows];
      float c[kEpiRows], gt[kEpiRows];
#pragma unroll
      // (addresses are clamped to the tile's first row and column, which
      // exist, so the loads need no branch that would hold them apart)
      for (int u = 0; u < kEpiRows; ++u) {
        t[u] = t0 + acc_row(wm, i, rq * kEpiRows + u, lane, Core::kNA);
        const int64_t tl = t[u] < TC ? t[u] : t0;
        tg[u] = target[tl];
        c[u] = coef[tl];
        gt[u] = gf[tl];
      }
      uint16_t w[kEpiRows][Core::kNB];
#pragma unroll
      for (int u = 0; u < kEpiRows; ++u)
#pragma unroll
        for (int j = 0; j < Core::kNB; ++j) {
          const int64_t h = h0 + acc_col(wn, j, lane, Core::kNB);
          const bool ok = tg[u] >= 0 && tg[u] < V && h < H;
          w[u][j] = W[ok ? int64_t(tg[u]) * H + h : int64_t(0)];
        }
#pragma unroll
      for (int u = 0; u < kEpiRows; ++u) {
        if (t[u] >= TC) continue;
        const bool ok = tg[u] >= 0 && tg[u] < V;
#pragma unroll
        for (int j = 0; j < Core::kNB; ++j) {
          const int64_t h = h0 + acc_col(wn, j, lane, Core::kNB);
          if (h < H) {
            const float wt = ok ? bf16_to_f32(w[u][j]) : NAN;
            dh[t[u] * H + h] = c[u] * (wt - gt[u] * acc[i][j][rq * kEpiRows + u]);
          }
        }
      }
    }
  }
}

// Shared by the loss and the per-token scale: the group of response i (the g
// with go[g] <= i < go[g+1]) and its advantage A_i = r_i - mean_group(r),
// with validation of the structure (ok = 0 on anything malformed).
__device__ void response_advantage(const int64_t* __restrict__ ro, int R,
                                   const int64_t* __restrict__ go, int G,
                                   const float* __restrict__ reward, int64_t T, int i,
                                   double& A, int& ok) {
  const int64_t a = ro[i];
  const int64_t b = ro[i + 1];
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (go[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int64_t ga = go[lo];
  const int64_t gb = go[lo + 1];
  ok = (ga <= i && i < gb && ga >= 0 && gb <= R) ? 1 : 0;
  ok = ok && (a >= 0 && a < b && b <= T);
  A = NAN;
  if (ok) {
    double sr = 0.0;
    for (int64_t k = ga; k < gb; ++k) sr += double(reward[k]);
    A = double(reward[i]) - sr / double(gb - ga);
  }
}

// The ragged structure, checked once on the device: *ok = 1 iff resp_offsets
// run from 0 to T and strictly increase, and group_offsets run from 0 to R
// and strictly increase.  The kernels below read *ok; with a malformed
// structure they write NaN to every token (coef, the token scale), every
// advantage and the loss, and read no offset beyond its array.
__global__ __launch_bounds__(256) void k_check_structure(const int64_t* __restrict__ ro, int R,
                                                         const int64_t* __restrict__ go, int G,
                                                         int64_t T, int* __restrict__ ok) {
  int bad = 0;
  if (threadIdx.x == 0) bad = (ro[0] != 0 || ro[R] != T || go[0] != 0 || go[G] != R) ? 1 : 0;
  for (int i = threadIdx.x; i < R; i += 256) bad |= ro[i] >= ro[i + 1] ? 1 : 0;
  for (int i = threadIdx.x; i < G; i += 256) bad |= go[i] >= go[i + 1] ? 1 : 0;
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) *ok = bad ? 0 : 1;
}

// NaN into every one of the T entries of out, spread over the R workgroups
// of a per-response kernel (malformed structure).
template <class F>
__device__ __forceinline__ void fill_nan_tokens(F* __restrict__ out, int64_t T, int R) {
  for (int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x; t < T; t += int64_t(R) * 256)
    out[t] = F(NAN);
}

// cs[t] = -A_i / (R L_i) for every token t of response i (float64): the
// factor that turns w_t into d loss / d logprob_t.  One workgroup per
// response; a malformed structure gives NaN for every token.
__global__ __launch_bounds__(256) void k_token_scale(const int64_t* __restrict__ ro, int R,
                                                     const int64_t* __restrict__ go, int G,
                                                     const float* __restrict__ reward, int64_t T,
                                                     const int* __restrict__ okp,
                                                     double* __restrict__ cs) {
  __shared__ double sA;
  __shared__ int sok;
  if (!*okp) {
    fill_nan_tokens(cs, T, R);
    return;
  }
  const int i = blockIdx.x;
  if (threadIdx.x == 0) {
    double A;
    int ok;
    response_advantage(ro, R, go, G, reward, T, i, A, ok);
    sA = A;
    sok = ok;
  }
  __syncthreads();
  if (!sok) return;
  const int64_t a = ro[i];
  const int64_t b = ro[i + 1];
  const double c = -sA / (double(R) * double(b - a));
  for (int64_t t = a + threadIdx.x; t < b; t += 256) cs[t] = c;
}

// ---------------------------------------------------------------------------
// IS loss, coef, advantages (float64 accumulation, fixed order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum_256(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) sh[tid] = sh[tid] + sh[tid + w];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_max_256(double v, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) sh[tid] = fmax(sh[tid], sh[tid + w]);
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

// One workgroup per response i.
__global__ __launch_bounds__(256) void k_is_resp(const float* __restrict__ logprob,
                                                 const float* __restrict__ mu, int64_t T,
                                                 const int64_t* __restrict__ ro, int R,
                                                 const int64_t* __restrict__ go, int G,
                                                 const float* __restrict__ reward,
                                                 const int* __restrict__ okp,
                                                 float* __restrict__ coef, float* __restrict__ adv,
                                                 double* __restrict__ part) {
  __shared__ double sh[256];
  __shared__ double sA;
  __shared__ int sok;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  if (!*okp) {
    if (coef) fill_nan_tokens(coef, T, R);
    if (tid == 0) {
      part[i] = NAN;
      if (adv) adv[i] = NAN;
    }
    return;
  }
  const int64_t a = ro[i];
  const int64_t b = ro[i + 1];
  if (tid == 0) {
    double A;
    int ok;
    response_advantage(ro, R, go, G, reward, T, i, A, ok);
    sA = A;
    sok = ok;
    if (adv) adv[i] = float(A);
  }
  __syncthreads();
  if (!sok) {
    if (tid == 0) part[i] = NAN;
    return;
  }
  const double A = sA;
  const double L = double(b - a);
  const double cscale = -A / (double(R) * L);
  double sw = 0.0;
  for (int64_t t = a + tid; t < b; t += 256) {
    const double w = exp(double(logprob[t]) - double(mu[t]));
    sw += w;
    if (coef) coef[t] = float(cscale * w);
  }
  sw = block_sum_256(sw, sh);
  if (tid == 0) part[i] = A * (sw / L);
}

__global__ __launch_bounds__(256) void k_is_final(const double* __restrict__ part, int R,
                                                  const int* __restrict__ okp,
                                                  double* __restrict__ loss) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < R; i += 256) s += part[i];
  s = block_sum_256(s, sh);
  if (threadIdx.x == 0) *loss = *okp ? -s / double(R) : NAN;
}

constexpr int64_t kD3Block = 16384;

// The three KL estimators over one update's tokens, delta = logprob - mu:
// per block of kD3Block tokens the partial sums of -delta, delta^2 / 2 and
// expm1(delta) - delta (float64, a fixed in-block tree), then one block sums
// the partials in block order.  D3 is the third of them; rz_d3 runs the same
// kernels, so its bits equal k3's.
__global__ __launch_bounds__(256) void k_kl_part(const float* __restrict__ logprob,
                                                 const float* __restrict__ mu, int64_t T,
                                                 double* __restrict__ part) {
  __shared__ double sh[256];
  const int64_t a = int64_t(blockIdx.x) * kD3Block;
  const int64_t b = a + kD3Block < T ? a + kD3Block : T;
  double s1 = 0.0, s2 = 0.0, s3 = 0.0;
  for (int64_t t = a + threadIdx.x; t < b; t += 256) {
    const double d = double(logprob[t]) - double(mu[t]);
    s1 -= d;
    s2 += 0.5 * d * d;
    s3 += expm1(d) - d;
  }
  s1 = block_sum_256(s1, sh);
  s2 = block_sum_256(s2, sh);
  s3 = block_sum_256(s3, sh);
  if (threadIdx.x == 0) {
    part[3 * blockIdx.x] = s1;
    part[3 * blockIdx.x + 1] = s2;
    part[3 * blockIdx.x + 2] = s3;
  }
}

// out[0..2] = (k1, k2, k3), or with only_k3 out[0] = k3.
__global__ __launch_bounds__(256) void k_kl_final(const double* __restrict__ part, int64_t nb,
                                                  int64_t T, int only_k3,
                                                  double* __restrict__ out) {
  __shared__ double sh[256];
  double k[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < nb; i += 256) s += part[3 * i + q];
    k[q] = block_sum_256(s, sh) / double(T);
  }
  if (threadIdx.x == 0) {
    if (only_k3) {
      out[0] = k[2];
    } else {
      out[0] = k[0];
      out[1] = k[1];
      out[2] = k[2];
    }
  }
}

// The log-ratio decomposition per token: lag = lp_new - lp_old and mismatch =
// lp_old - mu (each difference exact in float64, then rounded once), and per
// block of kD3Block tokens: max |lag|, sum lag, max |mismatch| and the count
// of tokens whose mismatch is not exactly 0 (NaN counts).  lag and mismatch
// may alias lp_new and lp_old.
__global__ __launch_bounds__(256) void k_decompose(const float* lp_new, const float* lp_old,
                                                   const float* __restrict__ mu, int64_t T,
                                                   float* lag, float* mismatch,
                                                   double* __restrict__ part) {
  __shared__ double sh[256];
  const int64_t a = int64_t(blockIdx.x) * kD3Block;
  const int64_t b = a + kD3Block < T ? a + kD3Block : T;
  double mx_lag = 0.0, sum_lag = 0.0, mx_mis = 0.0, n_mis = 0.0;
  for (int64_t t = a + threadIdx.x; t < b; t += 256) {
    const double pn = double(lp_new[t]), po = double(lp_old[t]), m = double(mu[t]);
    const double l = pn - po, d = po - m;
    lag[t] = float(l);
    mismatch[t] = float(d);
    mx_lag = fmax(mx_lag, fabs(l));
    sum_lag += l;
    mx_mis = fmax(mx_mis, fabs(d));
    n_mis += (d == 0.0) ? 0.0 : 1.0;
  }
  mx_lag = block_max_256(mx_lag, sh);
  sum_lag = block_sum_256(sum_lag, sh);
  mx_mis = block_max_256(mx_mis, sh);
  n_mis = block_sum_256(n_mis, sh);
  if (threadIdx.x == 0) {
    part[4 * blockIdx.x] = mx_lag;
    part[4 * blockIdx.x + 1] = sum_lag;
    part[4 * blockIdx.x + 2] = mx_mis;
    part[4 * blockIdx.x + 3] = n_mis;
  }
}

// summary = (max |lag|, mean lag, max |mismatch|, tokens with mismatch != 0).
__global__ __launch_bounds__(256) void k_decompose_final(const double* __restrict__ part,
                                                         int64_t nb, int64_t T,
                                                         double* __restrict__ summary) {
  __shared__ double sh[256];
  double v[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t i = threadIdx.x; i < nb; i += 256) {
    v[0] = fmax(v[0], part[4 * i]);
    v[1] += part[4 * i + 1];
    v[2] = fmax(v[2], part[4 * i + 2]);
    v[3] += part[4 * i + 3];
  }
  v[0] = block_max_256(v[0], sh);
  v[1] = block_sum_256(v[1], sh);
  v[2] = block_max_256(v[2], sh);
  v[3] = block_sum_256(v[3], sh);
  if (threadIdx.x == 0) {
    summary[0] = v[0];
    summary[1] = v[1] / double(T);
    summary[2] = v[2];
    summary[3] = v[3];
  }
}

// ---------------------------------------------------------------------------
// Weight gradients (optional outputs of the learner step).
//   dW[v] = sum_t coef_t (onehot(target_t)_v - p_tv) hhat_t
//   dgamma[k] = sum_t dhhat[t, k] x[t, k] r_t
// The softmax part is a contraction over tokens, sum_t (e_tv 2^-d) hs_t with
// hs_t = bf16(coef_t g_t hhat_t) (one rounding): the 256x256 MFMA tile core
// of rz_gemm_tr.h reads e straight from the forward's fragment order with
// transposing LDS reads and applies the exact exponent shift in registers.
// Chunks add into dW in chunk order.
// The one-hot part, and the exact terms of each token's dominant
// probabilities, are added in fp32 per vocabulary row in token order
// (rz_exact.hip).
// ---------------------------------------------------------------------------

// hsT[h][t] = bf16(coef_t g_t hhat[t][h]) for the chunk's tokens t < TC
// and 0 for TC <= t < TCp (the per-token factor of p moved onto the other
// operand of the token contraction; one rounding), token-contiguous so that
// the contraction reads it as a plain row-major operand.  64 x 64 tiles
// through LDS.
__global__ __launch_bounds__(256) void k_scale_rows_t(const uint16_t* __restrict__ hh,
                                                      const float* __restrict__ coef,
                                                      const float* __restrict__ gf, int64_t TC,
                                                      int64_t TCp, int H,
                                                      uint16_t* __restrict__ hsT) {
  __shared__ uint16_t tile[64][66];
  const int64_t t0 = int64_t(blockIdx.x) * 64;
  const int h0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t t = t0 + r;
    uint16_t v = 0;
    if (t < TC) {
      const float x = __uint_as_float(uint32_t(hh[t * H + h0 + tx]) << 16);
      v = scaled_hidden(x, coef[t], gf[t]);
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) hsT[int64_t(h0 + r) * TCp + t0 + tx] = tile[tx][r];
}

// The softmax part of dW straight from the stored e (GemmCoreTrT): dW[v][h] =
// (first ? 0 : dW[v][h]) - sum_t (e_tv 2^-d(t, vt)) hsT[h][t].
constexpr int kDwWaves = 8;
using DwCore = GemmCoreTrT<kDwWaves>;

__global__ __launch_bounds__(64 * kDwWaves)
__attribute__((amdgpu_waves_per_eu(kDwWaves / 4, kDwWaves / 4)))
void k_dw_tr(const uint16_t* __restrict__ E, const uint32_t* __restrict__ D, int64_t ds,
             const uint16_t* __restrict__ hsT, int64_t TCp, int H, int V, int64_t Vp,
             int64_t n_vt, int64_t n_ht, int first, float* __restrict__ dW) {
  __shared__ __attribute__((aligned(16))) char lds[DwCore::kRing];
  int64_t vt, ht;
  if (!tile_of(n_vt, n_ht, vt, ht)) return;
  const int64_t v0 = vt * kTile;
  const int64_t h0 = ht * kTile;
  DwCore g;
  g.init(E, Vp / 16, vt, hsT, H, ht, D + vt * ds, TCp, lds);
  g.run(int(TCp));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % DwCore::kWM;
  const int wn = wave / DwCore::kWM;
  // kEpiRows rows at a time: the previous chunks' sums of those rows are all
  // loaded before the first store, so the loads are in flight together (the
  // first chunk loads and ignores them; clamped addresses need no branch).
#pragma unroll
  for (int i = 0; i < DwCore::kNA; ++i) {
#pragma unroll
    for (int rq = 0; rq < 16 / kEpiRows; ++rq) {
      float old[kEpiRows][DwCore::kNB];
#pragma unroll
      for (int u = 0; u < kEpiRows; ++u) {
        const int64_t v = v0 + acc_row(wm, i, rq * kEpiRows + u, lane, DwCore::kNA);
#pragma unroll
        for (int j = 0; j < DwCore::kNB; ++j) {
          const int64_t h = h0 + acc_col(wn, j, lane, DwCore::kNB);
          const float o = dW[(v < V && h < H) ? v * H + h : v0 * H + h0];
          old[u][j] = first ? 0.0f : o;
        }
      }
#pragma unroll
      for (int u = 0; u < kEpiRows; ++u) {
        const int64_t v = v0 + acc_row(wm, i, rq * kEpiRows + u, lane, DwCore::kNA);
        if (v >= V) continue;
#pragma unroll
        for (int j = 0; j < DwCore::kNB; ++j) {
          const int64_t h = h0 + acc_col(wn, j, lane, DwCore::kNB);
          if (h < H) dW[v * H + h] = old[u][j] - g.acc[i][j][rq * kEpiRows + u];
        }
      }
    }
  }
}

// r_t = (mean x_t^2 + eps)^(-1/2) of a chunk's rows (float64, as the norm).
__global__ __launch_bounds__(256) void k_row_rstd(const uint16_t* __restrict__ x, float eps,
                                                  int64_t TC, int H, double* __restrict__ r) {
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= TC) return;
  const double ss = row_sumsq(x + t * H, H, threadIdx.x & 63);
  if ((threadIdx.x & 63) == 0) r[t] = 1.0 / sqrt(ss / double(H) + double(eps));
}

// dgamma partials: block (b, c) sums dhhat[t, k] x[t, k] r_t over the 256
// rows of block b in row order (float64) for the 256 columns of block c;
// global row block gb0 + b.  Loads run 8 rows ahead of the sum.
__global__ __launch_bounds__(256) void k_dgamma_part(const float* __restrict__ dhh,
                                                     const uint16_t* __restrict__ x,
                                                     const double* __restrict__ r, int64_t TC,
                                                     int H, int64_t gb0,
                                                     double* __restrict__ part) {
  const int k = blockIdx.y * 256 + threadIdx.x;
  if (k >= H) return;
  const int64_t a = int64_t(blockIdx.x) * 256;
  const int64_t b = a + 256 < TC ? a + 256 : TC;
  double s = 0.0;
  int64_t t = a;
  for (; t + 8 <= b; t += 8) {
    float dv[8], xv[8];
    double rv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      dv[u] = dhh[(t + u) * H + k];
      xv[u] = bf16_to_f32(x[(t + u) * H + k]);
      rv[u] = r[t + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += double(dv[u]) * double(xv[u]) * rv[u];
  }
  for (; t < b; ++t) s += double(dhh[t * H + k]) * double(bf16_to_f32(x[t * H + k])) * r[t];
  part[(gb0 + blockIdx.x) * H + k] = s;
}

// dgamma[k] = the sum of the row-block partials part[b][k] in block order,
// cut into 16 contiguous ranges of blocks (a function of nb alone): each of
// 16 waves sums one range in order for 64 columns, and the 16 range sums are
// added in range order.  Loads run 8 blocks ahead of the sum.
__global__ __launch_bounds__(1024) void k_dgamma_final(const double* __restrict__ part,
                                                       int64_t nb, int H,
                                                       float* __restrict__ dgamma) {
  __shared__ double rs[16][64];
  const int c = threadIdx.x & 63;
  const int r = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + c;
  double s = 0.0;
  if (k < H) {
    const int64_t b0 = nb * r / 16, b1 = nb * (r + 1) / 16;
    int64_t b = b0;
    for (; b + 8 <= b1; b += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(b + u) * H + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += part[b * H + k];
  }
  rs[r][c] = s;
  __syncthreads();
  if (r == 0 && k < H) {
    double t = 0.0;
    for (int q = 0; q < 16; ++q) t += rs[q][c];
    dgamma[k] = float(t);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline uint32_t blocks_for(int64_t n, int64_t per) { return uint32_t(ceil_div(n, per)); }

hipError_t launch_rmsnorm_fwd(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                              int H, uint16_t* hhat, float* rstd, hipStream_t s) {
  ProfScope prof("k_rmsnorm_fwd", s);
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(blocks_for(T, 4)), dim3(256), 0, s, x, gamma, eps, T, H,
                     hhat, rstd);
  return hipGetLastError();
}

// The persistent forward's grid: the current device's CU count, looked up
// once per device, as a multiple of the kFwdTickets counters.  Every
// counter then has workgroups of its own (the workgroups of counter x are
// those with blockIdx % 8 == x), whatever the count.
static int persistent_grid() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return kFwdPersistentGridMax;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g > 0) return g;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = kFwdPersistentGridMax;
  g = cus - cus % kFwdTickets;
  if (g < kFwdTickets) g = kFwdTickets;
  if (g > kFwdPersistentGridMax) g = kFwdPersistentGridMax;
  cache[dev].store(g, std::memory_order_relaxed);
  return g;
}

// Launches the forward over n_vt x n_tt tiles, relaunched per tile or
// persistent (ticket: kFwdTickets ints of device memory).
template <bool Store>
static void launch_fwd_grid(const uint16_t* hhat, const uint16_t* W, const int32_t* target,
                            int64_t tgt_off, int64_t T, int H, int V, int64_t n_vt, int64_t n_tt,
                            float* pm, float* ps, float* ztgt, uint16_t* E, int* ticket,
                            hipStream_t s) {
  const uint32_t nl = raster_grid(n_vt * n_tt);
  if (T <= 64) {
    hipLaunchKernelGGL((k_lmhead_fwd_few<Store, 64>), dim3(nl), dim3(64 * kFwdWaves), 0, s, hhat,
                       W, target, tgt_off, T, H, V, n_vt, vocab_pad(V), pm, ps, ztgt, E,
                       fwd_raster_group(H));
  } else if (T <= 128) {
    hipLaunchKernelGGL((k_lmhead_fwd_few<Store, 128>), dim3(nl), dim3(64 * kFwdWaves), 0, s, hhat,
                       W, target, tgt_off, T, H, V, n_vt, vocab_pad(V), pm, ps, ztgt, E,
                       fwd_raster_group(H));
  } else if (n_tt == 1) {
    hipLaunchKernelGGL((k_lmhead_fwd<Store, kFwdSmallPipe>), dim3(nl), dim3(64 * kFwdWaves), 0, s,
                       hhat, W, target, tgt_off, T, H, V, n_vt, n_tt, vocab_pad(V), pm, ps, ztgt,
                       E, fwd_raster_group(H));
  } else if (kFwdPersistent) {
    hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, s, ticket, int64_t(kFwdTickets), 0);
    const uint32_t cap = uint32_t(persistent_grid());
    const uint32_t grid = nl < cap ? nl : cap;
    hipLaunchKernelGGL(k_lmhead_fwd_p<Store>, dim3(grid), dim3(64 * kFwdWaves), 0, s, hhat, W,
                       target, tgt_off, T, H, V, n_vt, n_tt, vocab_pad(V), pm, ps, ztgt, E,
                       fwd_raster_group(H), int64_t(nl), ticket);
  } else {
    hipLaunchKernelGGL(k_lmhead_fwd<Store>, dim3(nl), dim3(64 * kFwdWaves), 0, s, hhat, W, target,
                       tgt_off, T, H, V, n_vt, n_tt, vocab_pad(V), pm, ps, ztgt, E,
                       fwd_raster_group(H));
  }
}

hipError_t launch_lmhead_fwd(const uint16_t* hhat, const uint16_t* W, const int32_t* target,
                             int64_t T, int H, int V, float* pm, float* ps, float* ztgt,
                             uint16_t* E, int* ticket, hipStream_t s) {
  ProfScope prof("k_lmhead_fwd", s);
  const int64_t n_vt = n_vocab_tiles(V);
  const int64_t n_tt = ceil_div(T, kTile);
  hipLaunchKernelGGL(k_fill_f32, dim3(blocks_for(T, 256)), dim3(256), 0, s, ztgt, T, NAN);
  if (E)
    launch_fwd_grid<true>(hhat, W, target, 0, T, H, V, n_vt, n_tt, pm, ps, ztgt, E, ticket, s);
  else
    launch_fwd_grid<false>(hhat, W, target, 0, T, H, V, n_vt, n_tt, pm, ps, ztgt, E, ticket, s);
  return hipGetLastError();
}

hipError_t launch_lmhead_fwd_range(const uint16_t* hhat, const uint16_t* W, const int32_t* target,
                                   int64_t T, int H, int64_t v0, int Vs, float* pm, float* ps,
                                   float* ztgt, int* ticket, hipStream_t s) {
  ProfScope prof("k_lmhead_fwd", s);
  const int64_t n_vt = n_vocab_tiles(Vs);
  const int64_t n_tt = ceil_div(T, kTile);
  hipLaunchKernelGGL(k_fill_f32, dim3(blocks_for(T, 256)), dim3(256), 0, s, ztgt, T, 0.0f);
  if (n_vt > 0)
    launch_fwd_grid<false>(hhat, W, target, v0, T, H, Vs, n_vt, n_tt, pm, ps, ztgt, nullptr,
                           ticket, s);
  return hipGetLastError();
}

hipError_t launch_split_partials(const float* pm, const float* ps, const float* ztgt,
                                 const int32_t* target, int64_t T, int V, int s0, int s1,
                                 void* out, int64_t out_stride, hipStream_t s) {
  ProfScope prof("k_lse_combine", s);
  hipLaunchKernelGGL(k_split_partials, dim3(blocks_for(T, 256)), dim3(256), 0, s, pm, ps, ztgt,
                     target, T, V, n_vocab_tiles(V), s0, s1, static_cast<SplitRec*>(out),
                     out_stride);
  return hipGetLastError();
}

hipError_t launch_split_merge(const void* parts, int64_t part_stride, const int32_t* target,
                              int64_t T, int V, float* logprob, float* lse, hipStream_t s) {
  ProfScope prof("k_lse_combine", s);
  hipLaunchKernelGGL(k_split_merge, dim3(blocks_for(T, 256)), dim3(256), 0, s,
                     static_cast<const SplitRec*>(parts), part_stride, target, T, V, logprob, lse);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float* pm, const float* ps, const float* ztgt, int64_t T,
                              int V, float* logprob, float* lse, const double* cs,
                              const float* mu, float* coef, uint32_t* D, int64_t ds, float* g,
                              hipStream_t s) {
  ProfScope prof("k_lse_combine", s);
  hipLaunchKernelGGL(k_lse_combine, dim3(blocks_for(T, 64)), dim3(kCombineThreads), 0, s, pm, ps,
                     ztgt, T, n_vocab_tiles(V), logprob, lse, cs, mu, coef, D, ds, g);
  return hipGetLastError();
}

hipError_t launch_shift_prep(const float* pm, const float* lse, int64_t T, int V, uint32_t* D,
                             int64_t ds, float* g, hipStream_t s) {
  ProfScope prof("k_shift_prep", s);
  hipLaunchKernelGGL(k_shift_prep, dim3(blocks_for(T, 256)), dim3(256), 0, s, pm, T,
                     n_vocab_tiles(V), lse, D, ds, g);
  return hipGetLastError();
}

hipError_t launch_token_scale(const int64_t* ro, int R, const int64_t* go, int G,
                              const float* reward, int64_t T, int* ok, double* cs,
                              hipStream_t s) {
  ProfScope prof("k_token_scale", s);
  hipLaunchKernelGGL(k_check_structure, dim3(1), dim3(256), 0, s, ro, R, go, G, T, ok);
  hipLaunchKernelGGL(k_token_scale, dim3(R), dim3(256), 0, s, ro, R, go, G, reward, T, ok, cs);
  return hipGetLastError();
}

hipError_t launch_transpose_w(const uint16_t* W, int H, int V, uint16_t* Wt, hipStream_t s) {
  ProfScope prof("k_transpose_w", s);
  const int64_t Vp = vocab_pad(V);
  hipLaunchKernelGGL(k_transpose_w, dim3(blocks_for(Vp, 64), H / 64), dim3(256), 0, s, W, H, V, Vp,
                     Wt);
  return hipGetLastError();
}

hipError_t launch_dhidden(const uint16_t* E, const uint32_t* D, int64_t ds, const float* g,
                          const uint16_t* Wt, const uint16_t* W, const int32_t* target_chunk,
                          const float* coef_chunk, int64_t TC, int H, int V, float* dh_chunk,
                          hipStream_t s) {
  ProfScope prof("k_dhidden", s);
  const int64_t n_ht = ceil_div(H, kTile);
  const int64_t n_tt = ceil_div(TC, kTile);
  hipLaunchKernelGGL(k_dhidden, dim3(raster_grid(n_ht * n_tt)), dim3(64 * kDhWaves), 0, s, E, D, ds, g,
                     Wt, W, target_chunk, coef_chunk, TC, H, V, vocab_pad(V), n_tt, n_ht,
                     dh_chunk);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                              int H, float* dh, hipStream_t s) {
  ProfScope prof("k_rmsnorm_bwd", s);
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(blocks_for(T, 4)), dim3(256), 0, s, x, gamma, eps, T, H,
                     dh);
  return hipGetLastError();
}

hipError_t launch_is_loss(const float* logprob, const float* mu, int64_t T, const int64_t* ro,
                          int R, const int64_t* go, int G, const float* reward, double* loss,
                          float* coef, float* adv, double* part, int* ok, bool check,
                          hipStream_t s) {
  ProfScope prof("k_is_loss", s);
  if (check)
    hipLaunchKernelGGL(k_check_structure, dim3(1), dim3(256), 0, s, ro, R, go, G, T, ok);
  hipLaunchKernelGGL(k_is_resp, dim3(R), dim3(256), 0, s, logprob, mu, T, ro, R, go, G, reward,
                     ok, coef, adv, part);
  hipLaunchKernelGGL(k_is_final, dim3(1), dim3(256), 0, s, part, R, ok, loss);
  return hipGetLastError();
}

hipError_t launch_d3(const float* logprob, const float* mu, int64_t T, double* d3, double* part,
                     hipStream_t s) {
  ProfScope prof("k_kl", s);
  const int64_t nb = ceil_div(T, kD3Block);
  hipLaunchKernelGGL(k_kl_part, dim3(uint32_t(nb)), dim3(256), 0, s, logprob, mu, T, part);
  hipLaunchKernelGGL(k_kl_final, dim3(1), dim3(256), 0, s, part, nb, T, 1, d3);
  return hipGetLastError();
}

hipError_t launch_weight_grads_chunk(const uint16_t* E, const uint32_t* D, int64_t ds,
                                    const float* g, const float* coef_chunk,
                                    const int32_t* target_chunk, const uint16_t* hh,
                                    const uint16_t* x_chunk, float eps, const float* dhh_chunk,
                                    int64_t TC, int H, int V, int64_t gb0, int first,
                                    uint16_t* hs, const SelRec* rec, const DwExactBufs& wb,
                                    double* rbuf, double* gpart, float* dW, hipStream_t s) {
  const int64_t Vp = vocab_pad(V);
  const int64_t TCp = shift_stride(TC);
  {
    ProfScope prof("k_dgamma_part", s);
    hipLaunchKernelGGL(k_row_rstd, dim3(blocks_for(TC, 4)), dim3(256), 0, s, x_chunk, eps, TC, H,
                       rbuf);
    hipLaunchKernelGGL(k_dgamma_part, dim3(blocks_for(TC, 256), blocks_for(H, 256)), dim3(256), 0,
                       s, dhh_chunk, x_chunk, rbuf, TC, H, gb0, gpart);
  }
  {
    // hsT = coef g hhat (the chunk's rows, token-contiguous), then the token
    // contraction straight from the stored e
    ProfScope prof("k_dw", s);
    hipLaunchKernelGGL(k_scale_rows_t, dim3(uint32_t(TCp / 64), H / 64), dim3(256), 0, s, hh,
                       coef_chunk, g, TC, TCp, H, hs);
    const int64_t n_vt = n_vocab_tiles(V);
    const int64_t n_ht = ceil_div(H, kTile);
    hipLaunchKernelGGL(k_dw_tr, dim3(raster_grid(n_vt * n_ht)), dim3(64 * kDwWaves), 0, s, E, D, ds,
                       hs, TCp, H, V, Vp, n_vt, n_ht, first, dW);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the one-hot terms and the exact records, per row in token order
  return launch_dw_exact(target_chunk, coef_chunk, g, rec, hh, TC, H, V, wb, dW, s);
}

hipError_t launch_dgamma_final(const double* gpart, int64_t nb, int H, float* dgamma,
                               hipStream_t s) {
  ProfScope prof("k_dgamma_part", s);
  hipLaunchKernelGGL(k_dgamma_final, dim3(blocks_for(H, 64)), dim3(1024), 0, s, gpart, nb, H,
                     dgamma);
  return hipGetLastError();
}

hipError_t launch_kl(const float* logprob, const float* mu, int64_t T, double* kl, double* part,
                     hipStream_t s) {
  ProfScope prof("k_kl", s);
  const int64_t nb = ceil_div(T, kD3Block);
  hipLaunchKernelGGL(k_kl_part, dim3(uint32_t(nb)), dim3(256), 0, s, logprob, mu, T, part);
  hipLaunchKernelGGL(k_kl_final, dim3(1), dim3(256), 0, s, part, nb, T, 0, kl);
  return hipGetLastError();
}

hipError_t launch_decompose(const float* lp_new, const float* lp_old, const float* mu, int64_t T,
                            float* lag, float* mismatch, double* summary, double* part,
                            hipStream_t s) {
  ProfScope prof("k_decompose", s);
  const int64_t nb = ceil_div(T, kD3Block);
  hipLaunchKernelGGL(k_decompose, dim3(uint32_t(nb)), dim3(256), 0, s, lp_new, lp_old, mu, T, lag,
                     mismatch, part);
  hipLaunchKernelGGL(k_decompose_final, dim3(1), dim3(256), 0, s, part, nb, T, summary);
  return hipGetLastError();
}

}  // namespace rz
