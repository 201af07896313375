// MFMA tile core for the token contraction of the LM-head weight gradient,
//   C[v][h] = sum_t (e[t][v] 2^-d(t, vt)) hsT[h][t],
// with K = tokens.  Operand B, hsT = (coef g hhat)^T, is token-contiguous and
// staged exactly as in rz_gemm.h.  Operand A is e in the A-fragment order the
// forward wrote for the P*W^T contraction (8 consecutive vocabulary values
// of one token per lane), while this contraction needs 8 consecutive tokens
// per lane: its fragments are read from LDS with gfx950's transposing read
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 64-bit words that lanes 4q + i / 4 (q = 0..3) address.  A
// source lane therefore addresses 4 consecutive vocabulary values of one
// token; 16 lanes cover 4 tokens x 16 values and each lane receives 4 tokens
// of one value.
//
// Tile 256 (vocabulary tile vt) x 256 (hidden tile ht), 4 waves of 128 x 128
// as in rz_gemm.h, K stages of 64 tokens in a 2-stage LDS ring.  Per stage:
//  - A: the 32 e fragments (16 vocabulary steps x 2 token blocks of 32) of
//    the stage, 1 KB each, copied by LDS-direct loads.  Inside a fragment the
//    16-byte lane slots are permuted on the way in (slot L holds the
//    forward's lane (L/8)*4 + L%4 + 32 ((L/4) % 2)), so the 16 lanes of one
//    transposing read touch 128 contiguous bytes; fragments of odd vocabulary
//    steps also swap their 128-byte halves (slot L ^ 8), so the two 16-lane
//    groups that the LDS serves together use different banks;
//  - B: 256 hidden rows x 64 tokens of hsT, 128 bytes per row with the
//    16-byte chunks XOR-swizzled per row (rz_gemm.h's layout, read with
//    plain 16-byte fragment reads);
//  - the 64 per-token shifts d(t, vt) << 7 (256 bytes, wave 0 loads them).
// The exponent shift is applied to the assembled A fragments with a
// saturating packed 16-bit subtract, as in the P*W^T contraction.
#pragma once

#include "rz_gemm.h"

namespace rz {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16 as inline asm.  Through the compiler builtin every such
// read is preceded by a wait for all LDS-direct loads in flight (the compiler
// cannot tell that they fill the other stage buffer), which serialises the
// pipeline; the asm form carries no such wait, and its results are waited
// for explicitly (GemmCoreTr::settle) before anything reads them.
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t lds_addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr) : "memory");
  return r;
}

// NW: 4 waves (one per SIMD), each owning 128 vocabulary rows x 128 hidden
// columns (4 x 4 blocks), or 8 waves (two per SIMD), each owning 64 x 128
// (2 x 4 blocks): waves wm = w % kWM along the vocabulary, wn = w / kWM
// along the hidden dimension.
template <int NW>
struct GemmCoreTrT {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static constexpr int kNA = NW == 4 ? 4 : 2;  // A (vocabulary) blocks per wave
  static constexpr int kNB = 4;                // B (hidden) blocks per wave
  static constexpr int kWM = 8 / kNA;          // waves along the vocabulary
  static constexpr int kNM = kNA * kNB;        // MFMAs per k-step
  static constexpr int kNR = kNA + kNB;        // read units per k-step
  static constexpr int kLPw = 32 / NW;         // load pairs per wave per stage
  static constexpr int kA = 32768;            // A stage bytes (32 fragments)
  static constexpr int kB = 32768;            // B stage bytes
  static constexpr int kD = 256;              // shift bytes per stage
  static constexpr int kStage = kA + kB + kD;
  static constexpr int kRing = 2 * kStage;

  __amdgpu_buffer_rsrc_t ra, rb, rd;
  const char* e_tile0;    // e fragments of (token tile 0, vocabulary step vt*16)
  int64_t e_tile_stride;  // bytes between token tiles in the e block
  uint32_t va[2], vb[kLPw];  // per-lane load offsets (A within a fragment, even/odd step; B rows)
  uint32_t boff;          // per-lane LDS offset of the B fragment reads (k-step 0)
  char* smem;
  int wave, nk, a_range;
  uint32_t a_rd[kNA][2];            // per-lane LDS byte offsets of the tr reads (k-step 0)
  uint32_t d_rd;                    // LDS offset of the lane's 8 token shifts (k-step 0)
  f32x16 acc[kNA][kNB];
  u32x4 fa[2][kNA], fb[2][kNB];  // fragments (8 bf16 each) as read
  uint32_t lds_base;         // LDS address of smem
  u16x8 sh[2];            // per-set exponent shifts (d << 7) of the lane's 8 tokens
  u32x4 shr[2][2];        // the same as read from LDS (one token per 32-bit word)

  // E: e block of the chunk (fragment order, n_ks = Vp/16 steps); hsT: [H][TCp]
  // bf16 rows (zero for tokens past the chunk); D: shift table row of tile vt
  // (d << 7 in the low 16 bits), at least TCp entries.
  __device__ __forceinline__ void init(const uint16_t* E, int64_t n_ks, int64_t vt,
                                       const uint16_t* hsT, int H, int64_t ht,
                                       const uint32_t* Drow, int64_t TCp, char* lds) {
    smem = lds;
    lds_base = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds));
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int wm = wave % kWM;
    const int wn = wave / kWM;
    e_tile0 = reinterpret_cast<const char*>(E) + frag_offset(0, vt * 16, 0, n_ks);
    e_tile_stride = n_ks * 8 * 1024;
    // the last vocabulary tile may hold fewer than 16 steps (the vocabulary is
    // padded to 64): its missing fragments read as 0 instead of running into
    // the next token tile or past the block
    const int64_t left = n_ks - vt * 16;
    a_range = int(left < 16 ? left : 16) * 8 * 1024;
    set_a_tile(0);
    rb = tile_rsrc(hsT, ht * kTile, H, TCp);
    {
      const uint64_t p = reinterpret_cast<uint64_t>(Drow);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
      const int n = __builtin_amdgcn_readfirstlane(int(TCp * 4));
      rd = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0,
                                             n, kBufferFlags);
    }
    // A: LDS slot L <- forward lane (L/8)*4 + L%4 + 32*((L/4)%2), with
    // L = lane (even vocabulary step) or lane ^ 8 (odd)
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int L = lane ^ (8 * o);
      va[o] = uint32_t(((L >> 3) << 2) + (L & 3) + 32 * ((L >> 2) & 1)) * 16u;
    }
    // B load q = wave*kLPw + u: rows 8q .. 8q+7, lane -> row 8q + lane/8, LDS
    // slot lane%8 holding the row's chunk (lane%8) ^ swz(row)
#pragma unroll
    for (int u = 0; u < kLPw; ++u) {
      const uint32_t row = uint32_t((wave * kLPw + u) * 8 + lane / 8);
      vb[u] = row * uint32_t(TCp) * 2u + ((uint32_t(lane % 8) ^ swz(row)) * 16u);
    }
    {
      const uint32_t r32 = uint32_t(lane & 31);
      boff = uint32_t(kA) + uint32_t(wn * 128 + r32) * 128u + ((uint32_t(lane >> 5) ^ swz(r32)) << 4);
    }
    // tr-read addresses for k-step 0 (read_step adds the k-step's offsets)
    const int g = lane >> 4, s = lane & 15, q = s >> 2, j = s & 3;
#pragma unroll
    for (int i = 0; i < kNA; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // A block i of wave wm: vocabulary step wm*2*kNA + 2i + g%2 of the
        // tile, token t = 8*(g/2) + 4h + q of the k-step
        const int ksl = wm * 2 * kNA + 2 * i + (g & 1);
        const int t = 8 * (g >> 1) + 4 * h + q;
        const int slot = ((t >> 2) * 8 + (j >> 1) * 4 + (t & 3)) ^ (8 * (ksl & 1));
        a_rd[i][h] = uint32_t(ksl * 2 * 1024 + slot * 16 + 8 * (j & 1));
      }
    // the lane's 8 token shifts: tokens 8*(lane/32) .. +7 of the k-step
    d_rd = uint32_t(kA + kB + (lane >> 5) * 8 * 4);
#pragma unroll
    for (int i = 0; i < kNA; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  __device__ __forceinline__ void set_a_tile(int64_t tt) {
    const uint64_t p = reinterpret_cast<uint64_t>(e_tile0 + tt * e_tile_stride);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
    ra = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(a_range), kBufferFlags);
  }

  // Loads of stage kt: pair u (0..kLPw-1) = A fragment and B piece
  // q = wave*kLPw + u; wave 0 also loads the stage's shifts with pair 0.
  __device__ __forceinline__ void load_pair(int kt, int u) {
    char* s = smem + (kt & 1) * kStage;
    const int q = wave * kLPw + u;
    // A fragment q: vocabulary step q/2, token block 2*(kt%4) + q%2 of the tile
    const int soffA = ((kt & 3) * 2) * 1024;
    // (the operands go through locals: hipcc's host pass rejects member
    // arrays of a dependent size among the builtin's operands)
    const uint32_t voa = uint32_t((q >> 1) * 8192 + (q & 1) * 1024) + va[(u >> 1) & 1];
    const uint32_t vob = vb[u];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(s + q * 1024), 16, voa, soffA, 0,
                                             0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(s + kA + q * 1024), 16, vob,
                                             kt * 128, 0, 0);
    if (u == 0 && wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void_t*)(s + kA + kB), 4,
                                               uint32_t((threadIdx.x & 63) * 4), kt * 256, 0, 0);
  }
  static __device__ __forceinline__ uint32_t da_of(int kk) {
    // k-step kk = tokens 16kk .. 16kk+15 of the stage: token block kk/2
    // (the next 1 KB fragment), rows (kk%2)*16 of it (4 slot groups of 8)
    return uint32_t((kk >> 1) * 1024 + (kk & 1) * 4 * 8 * 16);
  }

  // Read unit u (0..kNR-1) of k-step kk into set F: A block u (u < kNA, two
  // transposing reads) or B block u - kNA (one 16-byte read).
  template <int F>
  __device__ __forceinline__ void read_unit(const char* s, int kk, int u) {
    if (u < kNA) {
      const uint32_t b = lds_base + uint32_t(s - smem) + da_of(kk);
      const u32x2 lo = ds_read_tr16(b + a_rd[u][0]);
      const u32x2 hi = ds_read_tr16(b + a_rd[u][1]);
      fa[F][u] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    } else {
      fb[F][u - kNA] =
          *reinterpret_cast<const u32x4*>(s + (boff ^ uint32_t(kk << 5)) + (u - kNA) * 32 * 128);
    }
  }

  // Wait for every LDS read in flight, with the set-F fragments as operands
  // of the wait, so that no use of them can be placed before it.
  template <int F>
  __device__ __forceinline__ void settle() {
    if constexpr (kNA == 4)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[F][0]), "+v"(fa[F][1]), "+v"(fa[F][2]), "+v"(fa[F][3]),
                     "+v"(fb[F][0]), "+v"(fb[F][1]), "+v"(fb[F][2]), "+v"(fb[F][3])
                   :
                   : "memory");
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[F][0]), "+v"(fa[F][1]),
                     "+v"(fb[F][0]), "+v"(fb[F][1]), "+v"(fb[F][2]), "+v"(fb[F][3])
                   :
                   : "memory");
    unpack_shift<F>();
  }

  // The lane's 8 token shifts of k-step kk into set F (as read; unpacked by
  // unpack_shift once the reads have settled).
  template <int F>
  __device__ __forceinline__ void read_shift(const char* s, int kk) {
    shr[F][0] = *reinterpret_cast<const u32x4*>(s + d_rd + kk * 64);
    shr[F][1] = *reinterpret_cast<const u32x4*>(s + d_rd + kk * 64 + 16);
  }

  template <int F>
  __device__ __forceinline__ void unpack_shift() {
    u16x8 d;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d[c] = static_cast<unsigned short>(shr[F][0][c]);
      d[4 + c] = static_cast<unsigned short>(shr[F][1][c]);
    }
    sh[F] = d;
  }

  template <int F>
  __device__ __forceinline__ void shift_frag(int i) {
    fa[F][i] = __builtin_bit_cast(
        u32x4, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x8, fa[F][i]), sh[F]));
  }

  template <int F>
  __device__ __forceinline__ void mfma_one(int idx) {
    const int i = idx >> 2, j = idx & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[F][i]),
                                                        __builtin_bit_cast(bf16x8, fb[F][j]),
                                                        acc[i][j], 0, 0, 0);
  }

  // One k-step on set F while reading k-step kk of stage buffer s into set
  // F^1 (one read unit per MFMA) and, if Load, issuing a load pair of stage
  // lkt at every fourth MFMA, from first_pair on.  A block i of set F is
  // shifted just before its first MFMA.
  template <int F, bool Load>
  __device__ __forceinline__ void step(const char* s, int kk, int lkt, int first_pair) {
#pragma unroll
    for (int idx = 0; idx < kNM; ++idx) {
      mfma_one<F>(idx);
      if (idx < kNR) read_unit<F ^ 1>(s, kk, idx);
      if (idx == kNR) read_shift<F ^ 1>(s, kk);
      if (Load && (idx & 3) == 0) load_pair(lkt, first_pair + (idx >> 2));
      if ((idx & 3) == 3 && idx < kNM - 1) shift_frag<F>((idx >> 2) + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    settle<F ^ 1>();
    shift_frag<F ^ 1>(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Stage kt (4 k-steps), whose k-step-0 fragments are in set 0.  If Load,
  // stage kt+1's loads go out over the first two k-steps; if More, stage
  // kt+1 is waited for and published in the middle of the last k-step and
  // its k-step-0 fragments are read during the second half.
  template <bool Load, bool More>
  __device__ __forceinline__ void stage(int kt) {
    const char* s = smem + (kt & 1) * kStage;
    const int lkt = kt + 1;
    if (Load && (lkt & 3) == 0) set_a_tile(lkt >> 2);
    step<0, Load>(s, 1, lkt, 0);
    step<1, Load>(s, 2, lkt, kLPw / 2);
    step<0, false>(s, 3, lkt, 0);
    constexpr int kHalf = kNM / 2;
#pragma unroll
    for (int idx = 0; idx < kHalf; ++idx) {
      mfma_one<1>(idx);
      if ((idx & 3) == 3) shift_frag<1>((idx >> 2) + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (More) {
      GemmCore::wait_loads_except(0);
      GemmCore::barrier();
      const char* sn = smem + ((kt + 1) & 1) * kStage;
#pragma unroll
      for (int idx = kHalf; idx < kNM; ++idx) {
        mfma_one<1>(idx);
        // the next stage's k-step-0 units, spread over the second half
#pragma unroll
        for (int u = (idx - kHalf) * kNR / (kNM - kHalf); u < (idx - kHalf + 1) * kNR / (kNM - kHalf);
             ++u)
          read_unit<0>(sn, 0, u);
        if ((idx & 3) == 3 && idx < kNM - 1) shift_frag<1>((idx >> 2) + 1);
        if (idx == (kHalf > kNM - 4 ? kHalf : kNM - 4)) read_shift<0>(sn, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      settle<0>();
      shift_frag<0>(0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int idx = kHalf; idx < kNM; ++idx) {
        mfma_one<1>(idx);
        if ((idx & 3) == 3 && idx < kNM - 1) shift_frag<1>((idx >> 2) + 1);
      }
    }
  }

  // K = TCp tokens (a multiple of 256).  Ends with no load in flight and no
  // LDS read outstanding.
  __device__ __forceinline__ void run(int K) {
    nk = K / 64;
#pragma unroll
    for (int u = 0; u < kLPw; ++u) load_pair(0, u);
    GemmCore::wait_loads_except(0);
    GemmCore::barrier();
#pragma unroll
    for (int u = 0; u < kNR; ++u) read_unit<0>(smem, 0, u);
    read_shift<0>(smem, 0);
    settle<0>();
    shift_frag<0>(0);
    int kt = 0;
    for (; kt + 1 < nk; ++kt) stage<true, true>(kt);
    stage<false, false>(kt);
    GemmCore::barrier();
  }
};

using GemmCoreTr = GemmCoreTrT<4>;

}  // namespace rz
