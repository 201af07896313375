// bf16 MFMA tile core for gfx950 (CDNA4), 64-wide wavefronts.
//
// One workgroup computes a 256 x 256 fp32 tile
//   C[a][b] = sum_k A[a0 + a][k] * B[b0 + b][k]
// where both operands are row-major with K contiguous ("TN"), the natural
// layout of hidden states [T,H], the LM-head weight [V,H], a probability
// block [T,V] and a transposed weight [H,V].  With 4 waves (256 threads)
// they form a 2 x 2 grid, each owning a 128 x 128 sub-tile held as 4 x 4
// blocks of the 32x32 output of v_mfma_f32_32x32x16_bf16 (accumulators in
// AGPRs); with 8 waves, two per SIMD, each owns 8 blocks (see GemmCoreT).
//
// Operand staging.  K is consumed in stages of kBK bf16 (2*kBK bytes per
// row).  A stage of both operands (2 x 256 rows) is fetched with
// buffer_load_dwordx4 ... lds, which writes straight into LDS without passing
// through VGPRs; the LDS holds a ring of kStages stages and the loads of stage
// s are issued while stage s - (kStages - 1) is multiplied, one load pair
// after every few MFMAs (the Pipe parameter of GemmCoreT varies this, and can
// give A a deeper ring of its own).  Each load instruction moves 1 KB (64 lanes x 16 B,
// lane-major in LDS); a row's 16-byte chunks are stored XOR-swizzled by a
// function of the row so that the 16-byte fragment reads of consecutive rows
// are bank-conflict free whether the LDS serves 8 or 16 lanes x 16 B per
// clock:  f(row) = (row & 7) ^ ((row >> 3) & 1) for 128-byte rows (kBK = 64),
// f(row) = ((row >> 1) ^ (row >> 3)) & 3 for 64-byte rows (kBK = 32).
//
// Range.  Each operand tile is read through a buffer resource whose size
// covers only the tile's valid rows; rows past the end read as zeros, so no
// row index is ever clamped and no access leaves the operand.
//
// Pipeline per stage (kBK/16 MFMA steps of K=16, 16 MFMAs each): the
// fragments of the next step are read from LDS while a step multiplies (two
// fragment register sets, one read after each of the first eight MFMAs); the
// wait for the next stage and the workgroup barrier sit inside the last step
// (halfway, or three quarters of the way: Pipe), so the first fragments of
// the next stage load while MFMAs run.
//
// Reduction order: for every output element the K sum is taken in the same
// fixed order (stage 0, 1, ...; inside a stage steps of 16) no matter which
// tile, sub-tile, block or lane the element lands in, and no matter how many
// rows are valid.
#pragma once

#include "rz_internal.h"

namespace rz {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;
constexpr int kStages = 2;                          // LDS ring depth
constexpr int kRowBytes = kBK * 2;                  // bytes of one operand row per stage
constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row (8 or 4)
constexpr int kRowsPerLoad = 64 / kChunks;          // rows moved by one load instruction
constexpr int kLoadsPerOp = kTile / kRowsPerLoad / 4;   // load instructions per wave per operand
constexpr int kSteps = kBK / 16;                    // MFMA steps per stage
constexpr int kOpStageBytes = kTile * kRowBytes;    // one operand, one stage
constexpr int kStageBytes = 2 * kOpStageBytes;      // A then B
constexpr int kLdsBytes = kStages * kStageBytes;    // the ring
constexpr int kBufferFlags = 0x00020000;            // raw buffer, 32-bit data
static_assert(kChunks == 8 || kChunks == 4, "kBK must be 64 or 32");
static_assert(kLdsBytes <= 160 * 1024, "LDS ring too large");

// Chunk swizzle of an LDS row (see above).
__device__ __forceinline__ uint32_t swz(uint32_t row) {
  return kChunks == 8 ? ((row & 7) ^ ((row >> 3) & 1)) : (((row >> 1) ^ (row >> 3)) & 3);
}

// Output coordinates of acc[i][j][r] inside the workgroup tile, for lane l of
// wave (wm, wn) owning na A blocks and nb B blocks of 32 rows:
//   a = wm*32*na + i*32 + 8*(r/4) + 4*(l/32) + r%4    (operand-A row)
//   b = wn*32*nb + j*32 + l%32                        (operand-B row)
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane, int na = 4) {
  return wm * 32 * na + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane, int nb = 4) {
  return wn * 32 * nb + j * 32 + (lane & 31);
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Buffer resource over rows [row0, min(row0 + 256, rows)) of a row-major
// operand with `ld` elements per row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int64_t row0,
                                                            int64_t rows, int64_t ld) {
  const int64_t left = rows - row0;
  const int64_t valid = left < kTile ? left : kTile;
  // The values are uniform; say so, or the compiler wraps every load that
  // uses the resource in a per-lane loop.
  const uint64_t p = reinterpret_cast<uint64_t>(base + row0 * ld);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane(int(valid * ld * 2));
  void* up = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(up, 0, n, kBufferFlags);
}

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// bf16 x 2^-d for the 8 values of an A fragment, exactly, by a saturating
// subtract of (d << 7) from each bf16 bit pattern (the values are >= 0;
// results below the smallest normal come out as 0 or a value of the same
// tiny order).  The low 16 bits of dd hold d << 7.
__device__ __forceinline__ bf16x8 shift_down(bf16x8 f, uint32_t dd) {
  const u16x8 d8 = static_cast<unsigned short>(dd);
  return __builtin_bit_cast(bf16x8, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x8, f), d8));
}

// ShiftA: operand A holds values stored relative to a reference per row and
// per 256-wide K block; before it is multiplied, fragment row a of K block q
// is scaled by 2^-d(a, q), d read from dtab[q * dstride + a0 + a] (packed as
// for shift_down; the table covers every row of the tile, valid or not).
//
// ANative: operand A is stored in fragment order instead of row-major.  For
// each 256-row tile, K step ks (16 wide) and 32-row block mb, the 1 KB
// fragment [ks][mb] holds lane l's eight K values k = 8 (l / 32) .. + 7 of
// row 32 mb + l % 32 at byte 16 l; fragments follow each other in
// ([tile][ks][mb]) order (frag_offset).  A stage of A is then one contiguous
// 32 KB block, loaded as 1 KB pieces and read back at lane * 16 with no
// swizzle.  Rows past the end of the operand hold whatever the producer left
// there; they only reach the matching output rows.
__host__ __device__ constexpr int64_t frag_offset(int64_t tile, int64_t ks, int64_t mb,
                                                  int64_t n_ks) {
  return ((tile * n_ks + ks) * 8 + mb) * 1024;  // bytes
}

// NW: waves per workgroup, 4 (one per SIMD, each owning 128 x 128 of the
// tile: 4 x 4 blocks of 32 x 32) or 8 (two per SIMD, accumulators small
// enough for two waves' registers, so one wave's MFMAs issue while the other
// waits on LDS, loads or the barrier).  NA: A blocks per wave (4, or 2 with
// eight waves: 64 x 128 per wave, half the A fragments to shift per step).
// Waves form a kWA x kWB grid, wave w at wm = w % kWA (A rows
// [wm*32*NA, +32*NA)), wn = w / kWA (B rows [wn*32*kNB, +32*kNB)).
//
// Pipe: the stage pipeline.
//   0: a ring of kStages stages of both operands.  The loads of stage kt+1
//      are spread over the first two steps of stage kt, and the wait for them
//      sits halfway through the last step.
//   1: the same ring.  All of stage kt+1's loads are issued in step 0 and the
//      wait sits three quarters of the way through the last step, which gives
//      loads that miss in L2 more time.
//   2: (8 waves) A gets a ring of 3 stages and B one of
//      2, 160 KB in all.  In step 0 of stage kt the loads of B's stage kt+1
//      are issued, then those of A's stage kt+2, and the wait at three
//      quarters of the last step leaves A's stage kt+2 in flight (loads
//      return in issue order).  An A operand streamed from HBM thus gets
//      about two stages to arrive instead of one.
template <bool ShiftA, bool ANative = false, int NW = 4, int NA = 4, int Pipe = 0>
struct GemmCoreT {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(Pipe >= 0 && Pipe <= 2, "pipeline 0, 1 or 2");
  static_assert(Pipe != 2 || (NW == 8 && kStages == 2), "the deep A ring is built for 8 waves");
  static_assert(NA == 4 || (NA == 2 && NW == 8), "4 A blocks, or 2 with 8 waves");
  static constexpr int kNA = NA;                             // A blocks per wave
  static constexpr int kWA = 8 / NA;                         // waves along A
  static constexpr int kNB = 8 / (NW / kWA);                 // B blocks per wave
  static constexpr int kLP = kTile / kRowsPerLoad / NW;      // loads per wave per operand
  static constexpr int kNM = kNA * kNB;                      // MFMAs per step
  static constexpr int kNR = kNA + kNB;                      // fragment reads per step
  static constexpr bool kDeep = Pipe == 2;
  static constexpr int kSplit = Pipe == 0 ? kNM / 2 : kNM * 3 / 4;   // MFMAs before the wait
  static constexpr int kLds = kDeep ? 5 * kOpStageBytes : kLdsBytes;  // LDS bytes used
  static_assert(kLds <= 160 * 1024, "LDS");
  static_assert(!kDeep || 2 * kLP <= kNM, "one load per MFMA of step 0");
  __device__ __forceinline__ static int wave_m(int w) { return w % kWA; }
  __device__ __forceinline__ static int wave_n(int w) { return w / kWA; }
  __amdgpu_buffer_rsrc_t ra, rb;
  // Per-lane byte offsets of the load instructions (B, and A if row-major).
  // With the 2-stage ring only those of instructions 0 and 1 are kept, and
  // instruction j adds the uniform (j & ~1) * kRowsPerLoad * ld * 2 bytes
  // (soff_j): fewer registers for a caller that keeps them live across an
  // epilogue.  The deep ring keeps one offset per instruction.
  static constexpr int kVa = kDeep ? kLP : 2;
  uint32_t va[kVa];
  uint32_t ldb;              // bytes per operand row (ld * 2)
  uint32_t aoff, boff;       // per-lane LDS byte offsets of fragment reads (step 0)
  char* smem;
  int wave;
  int nk;                    // number of stages (K / kBK)
  f32x16 acc[kNA][kNB];
  bf16x8 fa[2][kNA], fb[2][kNB];
  // ShiftA only: per-lane table pointer (row of block 0), current and next
  // K block's shifts of the lane's kNA fragment rows.
  const uint32_t* dsrc;
  int64_t dstride;
  int nq;
  uint32_t dsh[kNA], dnxt[kNA];
  // kDeep only: LDS offsets of this stage's A and B buffers.
  uint32_t abase_ = 0, bbase_ = 0;
  // Partial runs only: this wave's B blocks that hold a valid row.
  int nbv = kNB;

  __device__ __forceinline__ void set_shift(const uint32_t* dtab, int64_t stride, int64_t a0,
                                            int64_t n_kblocks) {
    const int lane = threadIdx.x & 63;
    const int wm = wave_m(threadIdx.x >> 6);
    dsrc = dtab + a0 + wm * 32 * kNA + (lane & 31);
    dstride = stride;
    nq = int(n_kblocks);
  }

  __device__ __forceinline__ void init(const uint16_t* A, int64_t a0, int64_t a_rows,
                                       const uint16_t* B, int64_t b0, int64_t b_rows, int64_t ld,
                                       char* lds) {
    smem = lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: M0 needs it
    const int wm = wave_m(wave);
    const int wn = wave_n(wave);
    if (ANative) {
      // the whole fragment block of this 256-row tile (a0 is a multiple of 256)
      const int64_t n_ks = ld / 16;
      const uint64_t p = reinterpret_cast<uint64_t>(
          reinterpret_cast<const char*>(A) + frag_offset(a0 / kTile, 0, 0, n_ks));
      const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
      const int n = __builtin_amdgcn_readfirstlane(int(n_ks * 8 * 1024));
      ra = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0,
                                             n, kBufferFlags);
    } else {
      ra = tile_rsrc(A, a0, a_rows, ld);
    }
    rb = tile_rsrc(B, b0, b_rows, ld);
    // Load instruction q = wave*kLP + j moves rows [q*R, q*R + R)
    // (R = kRowsPerLoad); lane -> row q*R + lane/kChunks and LDS slot
    // lane%kChunks, which holds global chunk slot ^ swz(row).
    // swz(row) depends on the row's low three bits (lane / kChunks for every
    // j) and on bit 3, the parity of wave * kLP + j: instructions j and j & 1
    // differ by a whole number of rows.
    ldb = uint32_t(ld) * 2u;
#pragma unroll
    for (int j = 0; j < kVa; ++j) {
      const uint32_t row = uint32_t((wave * kLP + j) * kRowsPerLoad + lane / kChunks);
      const uint32_t chunk = uint32_t(lane % kChunks) ^ swz(row);
      va[j] = row * ldb + chunk * 16u;
    }
    // Fragment rows are 32-aligned blocks + lane%32; swz depends on row mod 16.
    const uint32_t r32 = uint32_t(lane & 31);
    const uint32_t slot0 = (uint32_t(lane >> 5) ^ swz(r32)) << 4;
    aoff = ANative ? uint32_t(wm * kNA * 1024 + lane * 16)
                   : uint32_t(wm * 32 * kNA + r32) * kRowBytes + slot0;
    boff = uint32_t(kDeep ? 3 * kOpStageBytes : kOpStageBytes) +
           uint32_t(wn * 32 * kNB + r32) * kRowBytes + slot0;
#pragma unroll
    for (int i = 0; i < kNA; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  }

  // The per-lane offset of load instruction j, and its uniform part.  The
  // callers copy them into locals before the load builtin: with a member
  // call among its operands the builtin fails overload resolution in
  // hipcc's host pass.
  __device__ __forceinline__ uint32_t va_j(int j) const { return kDeep ? va[j] : va[j & 1]; }
  __device__ __forceinline__ uint32_t soff_j(int j) const {
    return kDeep ? 0u : uint32_t(j & ~1) * uint32_t(kRowsPerLoad) * ldb;
  }

  // Load pair j (one A and one B instruction) of stage kt.
  __device__ __forceinline__ void load_pair(int kt, int j) {
    const int soff = kt * kRowBytes + int(soff_j(j));
    const uint32_t vo = va_j(j);
    char* s = smem + (kt % kStages) * kStageBytes;
    const int q = wave * kLP + j;
    if (ANative)  // piece q of the stage's contiguous 32 KB block, lane-major as stored
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(s + q * 1024), 16,
                                               uint32_t(q * 1024 + (threadIdx.x & 63) * 16),
                                               kt * kOpStageBytes, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(s + q * 1024), 16, vo, soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(s + kOpStageBytes + q * 1024), 16,
                                             vo, soff, 0, 0);
  }

  // kDeep: A's and B's instructions of stage kt, each into its own ring.
  __device__ __forceinline__ void load_a(int kt, int j) {
    const int q = wave * kLP + j;
    char* s = smem + (kt % 3) * kOpStageBytes;
    const uint32_t vo = va_j(j);
    const int soff = kt * kRowBytes + int(soff_j(j));
    if (ANative)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(s + q * 1024), 16,
                                               uint32_t(q * 1024 + (threadIdx.x & 63) * 16),
                                               kt * kOpStageBytes, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(s + q * 1024), 16, vo, soff, 0, 0);
  }
  __device__ __forceinline__ void load_b(int kt, int j) {
    const int q = wave * kLP + j;
    char* s = smem + (3 + kt % 2) * kOpStageBytes;
    const uint32_t vo = va_j(j);
    const int soff = kt * kRowBytes + int(soff_j(j));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(s + q * 1024), 16, vo, soff, 0, 0);
  }

  // Fragment read number q (0 .. kNR-1) into set F: A blocks first.
  template <int F>
  __device__ __forceinline__ void read_one(const char* s, uint32_t oa, uint32_t ob, int q) {
    constexpr int kBlockBytes = 32 * kRowBytes;
    constexpr int kABlockBytes = ANative ? 1024 : kBlockBytes;
    if (q < kNA)
      fa[F][q] = *reinterpret_cast<const bf16x8*>(s + oa + q * kABlockBytes);
    else
      fb[F][q - kNA] = *reinterpret_cast<const bf16x8*>(s + ob + (q - kNA) * kBlockBytes);
  }

  // Partial: the MFMAs of B blocks j >= nbv (blocks with no valid operand-B
  // row; nbv is uniform per wave) are skipped.  Every other output element
  // takes the same MFMAs in the same order, so it keeps its bits.
  template <int F, bool Partial = false>
  __device__ __forceinline__ void mfma_one(int idx) {
    const int i = idx / kNB, j = idx % kNB;
    if (!Partial || j < nbv)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[F][i], fb[F][j], acc[i][j], 0, 0, 0);
  }

  // K block of 256 (4 stages of kBK = 64) whose shifts stage kt uses.
  static constexpr int kStagesPerQ = kTile / kBK;

  __device__ __forceinline__ void load_shift(int q, uint32_t (&d)[kNA]) {
    const int qq = q < nq ? q : nq - 1;
    const uint32_t* p = dsrc + qq * dstride;
#pragma unroll
    for (int i = 0; i < kNA; ++i) d[i] = p[i * 32];
  }

  template <int F>
  __device__ __forceinline__ void shift_frag(int i) {
    if (ShiftA) fa[F][i] = shift_down(fa[F][i], dsh[i]);
  }

  // Workgroup barrier without a memory fence: the caller has already waited
  // for exactly the loads that must be complete (a fence would also drain
  // later stages still in flight).  The empty asm keeps the compiler from
  // moving memory operations across it.
  __device__ __forceinline__ static void barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt untouched
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Wait until at most `stages_after` stages of this wave's loads are in
  // flight.  s_waitcnt encoding (gfx9): vmcnt[3:0], expcnt[6:4],
  // lgkmcnt[11:8], vmcnt[5:4] at bits 15:14.
  __device__ __forceinline__ static void wait_loads_except(int stages_after) {
    const int n = stages_after * 2 * kLP;
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
      case 8: __builtin_amdgcn_s_waitcnt(0x0F70 | 8); break;
      case 16: __builtin_amdgcn_s_waitcnt(0x0F70 | (1 << 14)); break;
      case 24: __builtin_amdgcn_s_waitcnt(0x0F70 | 8 | (1 << 14)); break;
      case 32: __builtin_amdgcn_s_waitcnt(0x0F70 | (2 << 14)); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  }

  // One full MFMA step on set F, reading step kk of stage buffer s into set
  // F^1 and issuing the loads of stage lkt (if Load; and with kDeep, A's
  // stage lkt+1 if LoadA) as the pipeline places them.
  template <int F, bool Load, bool LoadA = false, bool Partial = false>
  __device__ __forceinline__ void step(const char* s, int kk, int lkt, int first_pair) {
    uint32_t oa = ANative ? aoff + uint32_t(kk * 8 * 1024) : aoff ^ uint32_t(kk << 5);
    uint32_t ob = boff ^ uint32_t(kk << 5);
    if constexpr (kDeep) {
      oa += abase_;
      ob += bbase_;
    }
#pragma unroll
    for (int idx = 0; idx < kNM; ++idx) {
      mfma_one<F, Partial>(idx);
      if (idx < kNR) read_one<F ^ 1>(s, oa, ob, idx);
      if constexpr (Pipe == 0) {
        if (Load && (idx & 3) == 0 && first_pair + (idx >> 2) < kLP)
          load_pair(lkt, first_pair + (idx >> 2));
      } else if constexpr (Pipe == 1) {
        if (Load && first_pair == 0 && idx < kLP) load_pair(lkt, idx);
      } else {
        if (Load && first_pair == 0 && idx < kLP) load_b(lkt, idx);
        if (LoadA && first_pair == 0 && idx >= kLP && idx < 2 * kLP) load_a(lkt + 1, idx - kLP);
      }
      if (idx % kNB == kNB - 1 && idx < kNM - 1) shift_frag<F>(idx / kNB + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    shift_frag<F ^ 1>(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // Multiply out stage kt, whose step-0 fragments are in set 0.  If Load,
  // the loads of stage kt + kStages - 1 are spread over the first steps; if
  // More, stage kt+1 is waited for and published between the halves of the
  // last step and its step-0 fragments are read during the second half.
  template <bool Load, bool More, bool LoadA = false, bool Partial = false>
  __device__ __forceinline__ void stage(int kt) {
    const char* s = kDeep ? smem : smem + (kt % kStages) * kStageBytes;
    if constexpr (kDeep) {
      abase_ = uint32_t((kt % 3) * kOpStageBytes);
      bbase_ = uint32_t((kt % 2) * kOpStageBytes);
    }
    const int lkt = kt + kStages - 1;
    // The next K block's shifts: issued before this stage's loads, so the
    // wait at the end of the stage covers them too.
    if (ShiftA) load_shift(kt / kStagesPerQ + 1, dnxt);
    // steps 0 .. kSteps-2 (sets alternate 0,1,0,...), each reading the next step
    step<0, Load, LoadA, Partial>(s, 1, lkt, 0);
    if (kSteps == 4) {
      step<1, Load, LoadA, Partial>(s, 2, lkt, kNM / 4);
      step<0, false, false, Partial>(s, 3, lkt, 0);
    }
    // last step (set 1): kSplit MFMAs, publish stage kt+1, the rest with the
    // reads of its step 0
#pragma unroll
    for (int idx = 0; idx < kSplit; ++idx) {
      mfma_one<1, Partial>(idx);
      if (idx % kNB == kNB - 1) shift_frag<1>(idx / kNB + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (More) {
      if constexpr (kDeep) {
        if (LoadA)
          __builtin_amdgcn_s_waitcnt(0x0F70 | kLP);   // vmcnt(kLP): A's stage kt+2 stays
        else
          wait_loads_except(0);
      } else {
        wait_loads_except(Load ? kStages - 2 : 0);
      }
      barrier();
      const char* sn = kDeep ? smem : smem + ((kt + 1) % kStages) * kStageBytes;
      const uint32_t na = kDeep ? aoff + uint32_t(((kt + 1) % 3) * kOpStageBytes) : aoff;
      const uint32_t nb = kDeep ? boff + uint32_t(((kt + 1) % 2) * kOpStageBytes) : boff;
#pragma unroll
      for (int idx = kSplit; idx < kNM; ++idx) {
        mfma_one<1, Partial>(idx);
        // read u goes with MFMA kSplit + u (kNM - kSplit) / kNR
#pragma unroll
        for (int u = 0; u < kNR; ++u)
          if (u * (kNM - kSplit) / kNR == idx - kSplit) read_one<0>(sn, na, nb, u);
        if (idx % kNB == kNB - 1 && idx < kNM - 1) shift_frag<1>(idx / kNB + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ShiftA) {
        const bool nq_ = ((kt + 1) % kStagesPerQ) == 0;
#pragma unroll
        for (int i = 0; i < kNA; ++i) dsh[i] = nq_ ? dnxt[i] : dsh[i];
      }
      shift_frag<0>(0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int idx = kSplit; idx < kNM; ++idx) {
        mfma_one<1, Partial>(idx);
        if (idx % kNB == kNB - 1 && idx < kNM - 1) shift_frag<1>(idx / kNB + 1);
      }
    }
  }

  // Persistent use (ring of kStages = 2, Pipe 0 or 1, operands row-major):
  // a workgroup that computes tile after tile issues the next tile's first
  // stage (issue_first, after retile) as soon as a tile's main loop is done,
  // overlapping those loads with the tile's epilogue, then begin_tile()
  // waits for them (and for every other memory operation of the wave),
  // zeroes the accumulators and reads the first fragments, and mainloop()
  // runs the stages.
  __device__ __forceinline__ void retile(const uint16_t* A, int64_t a0, int64_t a_rows,
                                         const uint16_t* B, int64_t b0, int64_t b_rows,
                                         int64_t ld) {
    static_assert(!ANative && !kDeep && kStages == 2, "persistent use: row-major 2-stage ring");
    ra = tile_rsrc(A, a0, a_rows, ld);
    rb = tile_rsrc(B, b0, b_rows, ld);
  }
  __device__ __forceinline__ void issue_first() {
#pragma unroll
    for (int j = 0; j < kLP; ++j) load_pair(0, j);
  }
  __device__ __forceinline__ void begin_tile() {
    wait_loads_except(0);
    barrier();
#pragma unroll
    for (int i = 0; i < kNA; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll
    for (int q = 0; q < kNR; ++q) read_one<0>(smem, aoff, boff, q);
  }
  __device__ __forceinline__ void mainloop(int K) {
    nk = K / kBK;
    int kt = 0;
    for (; kt + 1 < nk; ++kt) stage<true, true>(kt);
    stage<false, false>(kt);
    barrier();
  }

  // K must be a multiple of kBK.  Ends with no load in flight and, after the
  // trailing barrier, no LDS read outstanding, so the caller may reuse the LDS.
  template <bool Partial = false>
  __device__ __forceinline__ void run(int K) {
    nk = K / kBK;
    if constexpr (kDeep) {
      // A's stages 0 and 1 and B's stage 0 in flight; wait for the first two.
      // The shifts go first, so that waiting for them never waits for A's
      // stage 1.
      if (ShiftA) load_shift(0, dsh);
#pragma unroll
      for (int j = 0; j < kLP; ++j) load_a(0, j);
#pragma unroll
      for (int j = 0; j < kLP; ++j) load_b(0, j);
      if (nk > 1) {
#pragma unroll
        for (int j = 0; j < kLP; ++j) load_a(1, j);
        __builtin_amdgcn_s_waitcnt(0x0F70 | kLP);
      } else {
        wait_loads_except(0);
      }
      barrier();
      // dsh has arrived.  Route it through an empty asm so the compiler
      // stops treating its registers as a load in flight: it would otherwise
      // wait at the top of every stage for all older loads, A's next stage
      // among them.
      if (ShiftA)
#pragma unroll
        for (int i = 0; i < kNA; ++i) asm volatile("" : "+v"(dsh[i]));
#pragma unroll
      for (int q = 0; q < kNR; ++q) read_one<0>(smem, aoff, boff, q);
      shift_frag<0>(0);
      int kt = 0;
      for (; kt + 2 < nk; ++kt) stage<true, true, true, Partial>(kt);
      for (; kt + 1 < nk; ++kt) stage<true, true, false, Partial>(kt);
      stage<false, false, false, Partial>(kt);
      barrier();
      return;
    }
    const int pre = nk < kStages - 1 ? nk : kStages - 1;
    for (int st = 0; st < pre; ++st)
#pragma unroll
      for (int j = 0; j < kLP; ++j) load_pair(st, j);
    if (ShiftA) load_shift(0, dsh);
    wait_loads_except(pre - 1);
    barrier();
#pragma unroll
    for (int q = 0; q < kNR; ++q) read_one<0>(smem, aoff, boff, q);
    shift_frag<0>(0);
    int kt = 0;
    for (; kt + kStages - 1 < nk; ++kt) stage<true, true, false, Partial>(kt);
    for (; kt + 1 < nk; ++kt) stage<false, true, false, Partial>(kt);
    stage<false, false, false, Partial>(kt);
    barrier();
  }
};

using GemmCore = GemmCoreT<false>;

// XCD-aware tile raster over an (n_a x n_b) grid of tiles.  Workgroups are
// dealt to the 8 XCDs round-robin by id; we undo that so each XCD walks a
// contiguous range of the logical order.  When the second dimension has few
// tiles (the hidden dimension of the P*W^T product: 6 tiles at H = 1536), the
// logical order runs all of them side by side for each tile of the first
// (32 / n_b first-dimension tiles at a time), so each long operand row block
// of the first streams through one XCD's L2 once.  Otherwise it visits
// `group` tiles of the first dimension for every tile of the second:
// the group's operand blocks stay in that XCD's L2 while the second
// dimension's operand streams past, and the workgroups resident on one XCD
// share both.  The grid is padded to a multiple of 8; returns false for the
// padding.
__device__ __forceinline__ bool tile_at(uint64_t w, int64_t n_a, int64_t n_b, int64_t& ta,
                                        int64_t& tb, int group = kRasterGroup);

__device__ __forceinline__ bool tile_of(int64_t n_a, int64_t n_b, int64_t& ta, int64_t& tb,
                                        int group = kRasterGroup) {
  const uint64_t nb = gridDim.x;
  const uint64_t b = blockIdx.x;
  const uint64_t w = (b & 7) * (nb >> 3) + (b >> 3);
  return tile_at(w, n_a, n_b, ta, tb, group);
}

// The tile at logical position w of the raster order described above (false
// for the padding past the last tile).
__device__ __forceinline__ bool tile_at(uint64_t w, int64_t n_a, int64_t n_b, int64_t& ta,
                                        int64_t& tb, int group) {
  const uint64_t no = uint64_t(n_b);
  const uint64_t n_tiles = uint64_t(n_a) * no;
  if (w >= n_tiles) return false;
  if (no <= 32) {
    ta = int64_t(w / no);
    tb = int64_t(w % no);
    return true;
  }
  const uint64_t gr = uint64_t(group);
  const uint64_t per_group = gr * no;
  const uint64_t g = w / per_group;
  const uint64_t rem = w - g * per_group;
  const uint64_t left = uint64_t(n_a) - g * gr;
  const uint64_t gsz = left < gr ? left : gr;
  ta = int64_t(g * gr + rem % gsz);
  tb = int64_t(rem / gsz);
  return true;
}

inline uint32_t raster_grid(int64_t n_tiles) { return uint32_t(round_up(n_tiles, 8)); }

}  // namespace rz
