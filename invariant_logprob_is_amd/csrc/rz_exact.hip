// Exact terms of the backward: the one-hot term of the weight gradient and
// the exact replacement of each token's dominant probabilities in both
// contractions over the vocabulary.
//
// Why.  The contractions multiply the stored e rounded to bf16 (relative
// error up to 2^-9).  For a row whose softmax is flat, that error averages
// out against the exact one-hot term.  For a row whose softmax is peaked --
// the usual case for a token the rollout sampled from its own policy -- the
// gradient coef (onehot - p) is of the size of 1 - p_t while the rounding of
// the few large p is of the size of 2^-9 p.  Making the target and the kSelK
// largest p of the row exact bounds the relative error of the row by about
// 2^-9 / sqrt(kSelK + 1), whatever the peak.
//
// Per token (k_select): the threshold tau (1 - p_t), p_t = exp(z_t - lse);
// the vocabulary tiles whose max logit reaches it (at most kSelK, the largest
// first); inside them the kSelK largest contraction operands g e 2^-d that
// reach it (ties: lower vocabulary row first), plus the target if it
// reaches it; for each, z recomputed in float64 from hhat and W, p = exp(z -
// lse) and the record (v, p, pp = e 2^-d, beta = p - g pp).
//   dhhat_t -= coef_t sum_records beta W[v]                   (k_dh_fix)
//   dW[v]   += -coef_t p hhat_t + pp hs_t   per record        (k_seg_sum)
// (hs_t = bf16(coef_t g_t hhat_t) is the weight-gradient contraction's B
// operand, which subtracted pp hs_t for every entry.)  The one-hot term
// dW[target_t] += coef_t hhat_t goes through the same sums.
//
// Order.  The weight-gradient entries of a chunk -- per token the one-hot
// entry and its records -- are sorted by vocabulary row with a stable LSD
// radix sort (integer counts, stable ranks within a block from wave ballots),
// so each row's entries are summed in token order.  Buckets are summed in
// aligned blocks of 64 sorted positions, and a bucket that spans blocks is
// finished by adding its blocks' partial sums in block order: a fixed order
// whatever the bucket sizes (a target repeated through a whole chunk costs
// the same as distinct ones).
#include <math.h>

#include "rz_gemm.h"
#include "rz_internal.h"

namespace rz {

// ---------------------------------------------------------------------------
// Selection of the exact entries.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 64 * kVocabSplits;   // 64 tokens, one wave per split

// Insert (m, j) into a list sorted by m, largest first, of which the last
// entry drops out (a carried entry passes equal ones).
__device__ __forceinline__ void top_insert(float (&bm)[kSelK], int32_t (&bj)[kSelK], float m,
                                           int32_t j) {
#pragma unroll
  for (int k = 0; k < kSelK; ++k) {
    const bool s = m > bm[k];
    const float tm = bm[k];
    const int32_t tj = bj[k];
    bm[k] = s ? m : tm;
    bj[k] = s ? j : tj;
    m = s ? tm : m;
    j = s ? tj : j;
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ pm, int64_t TC, int64_t n_vt, const float* __restrict__ lse,
    const float* __restrict__ zt, const int32_t* __restrict__ target,
    const float* __restrict__ coef, const uint32_t* __restrict__ D, int64_t ds,
    const float* __restrict__ gf, const uint16_t* __restrict__ E, int64_t n_ks,
    const uint16_t* __restrict__ hh, const uint16_t* __restrict__ W, int H, int V,
    SelRec* __restrict__ rec) {
  __shared__ float lm[kVocabSplits][kSelK][64];
  __shared__ int32_t lj[kVocabSplits][kSelK][64];
  __shared__ int32_t ft[kSelK][64];
  __shared__ int32_t fn[64];
  __shared__ double thr[64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 64 + lane;
  const bool live = t < TC;

  // Threshold tp on p, tz = lse + log tp on logits (+inf: nothing to make
  // exact -- a NaN row (target out of range), or coef 0).
  double tp = 2.0, tz = INFINITY;
  if (live) {
    const double l = double(lse[t]);
    const double lz = double(zt[t]) - l;
    if (coef[t] != 0.0f && lz == lz && l == l) {
      const double qt = -expm1(lz);
      tp = qt > 0.0 ? kSelTau * qt : 0.0;
      tz = qt > 0.0 ? l + log(tp) : -INFINITY;
    }
  }

  // 1. The qualifying tiles of split q with the largest maxima, per token.
  float bm[kSelK];
  int32_t bj[kSelK];
#pragma unroll
  for (int k = 0; k < kSelK; ++k) {
    bm[k] = -INFINITY;
    bj[k] = -1;
  }
  if (live && tz != INFINITY) {
    const int64_t j0 = n_vt * q / kVocabSplits, j1 = n_vt * (q + 1) / kVocabSplits;
    constexpr int kU = 8;
    int64_t j = j0;
    for (; j + kU <= j1; j += kU) {
      float v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = pm[(j + u) * TC + t];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (double(v[u]) >= tz) top_insert(bm, bj, v[u], int32_t(j + u));
    }
    for (; j < j1; ++j) {
      const float v = pm[j * TC + t];
      if (double(v) >= tz) top_insert(bm, bj, v, int32_t(j));
    }
  }
#pragma unroll
  for (int k = 0; k < kSelK; ++k) {
    lm[q][k][lane] = bm[k];
    lj[q][k][lane] = bj[k];
  }
  __syncthreads();
  if (q == 0) {
    // merge the splits' lists in split order
#pragma unroll
    for (int k = 0; k < kSelK; ++k) {
      bm[k] = -INFINITY;
      bj[k] = -1;
    }
    for (int s = 0; s < kVocabSplits; ++s)
#pragma unroll
      for (int k = 0; k < kSelK; ++k)
        if (lj[s][k][lane] >= 0) top_insert(bm, bj, lm[s][k][lane], lj[s][k][lane]);
    int n = 0;
#pragma unroll
    for (int k = 0; k < kSelK; ++k) {
      ft[k][lane] = bj[k];
      n += bj[k] >= 0 ? 1 : 0;
    }
    fn[lane] = n;
    thr[lane] = tp;
  }
  __syncthreads();

  // 2. Per token with candidate tiles, one wave: the largest operands in
  // those tiles, the target, and their exact probabilities.  Wave q takes
  // tokens 8q .. 8q+7 of the block.
  for (int i = 0; i < 8; ++i) {
    const int tl = q * 8 + i;
    const int64_t tk = int64_t(blockIdx.x) * 64 + tl;
    if (tk >= TC) break;
    SelRec* r = rec + tk * kSelSlots;
    const int nt = fn[tl];
    if (nt == 0) {
      if (lane < kSelSlots) r[lane] = SelRec{-1, 0.0f, 0.0f, 0.0f};
      continue;
    }
    const double tpv = thr[tl];
    const float gt = gf[tk];
    const int64_t ttile = tk / kTile;
    const int mb = int((tk % kTile) / 32);
    const int tl32 = int(tk % 32);
    const char* Eb = reinterpret_cast<const char*>(E);
    // the lane's values: tile 2k + lane/32 of the list, 16-byte chunk c =
    // lane % 32 of the token's 256 values there (16-wide step c/2, half c%2)
    const int c = lane & 31;
    float val[32];
    int32_t vb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ti = 2 * k + (lane >> 5);
      vb[k] = -1;
      u32x4 raw = {0u, 0u, 0u, 0u};
      uint32_t dd = 0;
      if (ti < nt) {
        const int32_t j = ft[ti][tl];
        const int64_t ks = int64_t(j) * 16 + (c >> 1);
        vb[k] = j * kTile + (c >> 1) * 16 + (c & 1) * 8;
        if (ks < n_ks)
          raw = *reinterpret_cast<const u32x4*>(Eb + frag_offset(ttile, ks, mb, n_ks) +
                                                (tl32 + 32 * (c & 1)) * 16);
        dd = D[int64_t(j) * ds + tk];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = uint16_t(raw[e >> 1] >> (16 * (e & 1)));
        const float pp = bf16_to_f32(shift_bits(bits, dd));
        // rows past V hold e = 0 as the forward stores them; the row bound
        // keeps a selection in W's rows whatever the stored values
        val[k * 8 + e] = (vb[k] >= 0 && vb[k] + e < V && pp > 0.0f &&
                          double(gt) * double(pp) >= tpv) ? pp : -1.0f;
      }
    }
    // kSelK rounds: the largest remaining operand of the wave (ties: lower
    // row); lane s keeps selection s
    int nsel = 0;
    int32_t my_v = -1;
    float my_pp = 0.0f;
    for (int rd = 0; rd < kSelK; ++rd) {
      float bv = -1.0f;
      int32_t bvv = 0x7FFFFFFF;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = val[k * 8 + e];
          const int32_t v = vb[k] + e;
          if (x >= 0.0f && (x > bv || (x == bv && v < bvv))) {
            bv = x;
            bvv = v;
          }
        }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int32_t ovv = __shfl_xor(bvv, m, 64);
        if (ov > bv || (ov == bv && ovv < bvv)) {
          bv = ov;
          bvv = ovv;
        }
      }
      if (bv < 0.0f) break;
      if (lane == nsel) {
        my_v = bvv;
        my_pp = bv;
      }
      ++nsel;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (vb[k] >= 0 && vb[k] + e == bvv) val[k * 8 + e] = -1.0f;
    }
    // the target, if it qualifies and is not among them
    const int32_t tg = target[tk];
    bool have = false;
    for (int s = 0; s < nsel; ++s) have |= __shfl(my_v, s, 64) == tg;
    if (!have && tg >= 0 && tg < V && exp(double(zt[tk]) - double(lse[tk])) >= tpv) {
      const int64_t ks = tg / 16;
      const uint16_t bits = *reinterpret_cast<const uint16_t*>(
          Eb + frag_offset(ttile, ks, mb, n_ks) + (tl32 + 32 * ((tg % 16) / 8)) * 16 +
          (tg % 8) * 2);
      const uint32_t dd = D[int64_t(tg / kTile) * ds + tk];
      if (lane == nsel) {
        my_v = tg;
        my_pp = bf16_to_f32(shift_bits(bits, dd));
      }
      ++nsel;
    }
    // exact z in float64 (lanes over H in a fixed order, then the butterfly)
    float my_p = 0.0f, my_beta = 0.0f;
    const uint16_t* hr = hh + tk * H;
    for (int s = 0; s < nsel; ++s) {
      const int32_t v = __shfl(my_v, s, 64);
      const float pps = __shfl(my_pp, s, 64);
      const uint16_t* wr = W + int64_t(v) * H;
      double acc = 0.0;
      for (int h = lane * 8; h < H; h += 512) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(hr + h);
        const u32x4 b = *reinterpret_cast<const u32x4*>(wr + h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fma(double(__uint_as_float(a[e] << 16)), double(__uint_as_float(b[e] << 16)), acc);
          acc = fma(double(__uint_as_float(a[e] & 0xFFFF0000u)),
                    double(__uint_as_float(b[e] & 0xFFFF0000u)), acc);
        }
      }
      const double z = wave_sum(acc);
      const double p = exp(z - double(lse[tk]));
      if (lane == s) {
        my_p = float(p);
        my_beta = float(p - double(gt) * double(pps));
      }
    }
    if (lane < kSelSlots)
      r[lane] = lane < nsel ? SelRec{my_v, my_p, my_pp, my_beta} : SelRec{-1, 0.0f, 0.0f, 0.0f};
  }
}

// dhhat_t -= coef_t sum_records beta W[v], one wave per token with records.
__global__ __launch_bounds__(256) void k_dh_fix(const SelRec* __restrict__ rec,
                                                const float* __restrict__ coef,
                                                const uint16_t* __restrict__ W, int64_t TC, int H,
                                                float* __restrict__ dh) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= TC) return;
  const SelRec* r = rec + t * kSelSlots;
  if (r[0].v < 0) return;
  const float c = coef[t];
  float* dr = dh + t * H;
  for (int h = lane * 8; h < H; h += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < kSelSlots; ++s) {
      const SelRec rs = r[s];
      if (rs.v < 0) break;
      const u32x4 w = *reinterpret_cast<const u32x4*>(W + int64_t(rs.v) * H + h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(rs.beta, __uint_as_float(w[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(rs.beta, __uint_as_float(w[e] & 0xFFFF0000u), acc[2 * e + 1]);
      }
    }
    f32x4 d0 = *reinterpret_cast<const f32x4*>(dr + h);
    f32x4 d1 = *reinterpret_cast<const f32x4*>(dr + h + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d0[e] = d0[e] - c * acc[e];
      d1[e] = d1[e] - c * acc[4 + e];
    }
    *reinterpret_cast<f32x4*>(dr + h) = d0;
    *reinterpret_cast<f32x4*>(dr + h + 4) = d1;
  }
}

// ---------------------------------------------------------------------------
// The weight-gradient entries of a chunk and their stable sort by row.
// Entry e = t (kSelSlots + 1) + s: s = 0 the one-hot entry of token t, s >= 1
// its record s - 1.  A token with coef 0 has none (its terms vanish).  The
// entries are written compacted, in (t, s) order, after a scan of the
// per-token counts; the count of entries, n, stays in device memory.
// ---------------------------------------------------------------------------
constexpr int kEnt = kSelSlots + 1;

__device__ __forceinline__ int32_t entry_row(const int32_t* __restrict__ target,
                                             const SelRec* __restrict__ rec, int64_t t, int s,
                                             int V) {
  if (s == 0) {
    const int32_t tg = target[t];
    return (tg >= 0 && tg < V) ? tg : -1;
  }
  return rec[t * kSelSlots + s - 1].v;
}

__global__ __launch_bounds__(256) void k_dw_count(const int32_t* __restrict__ target,
                                                  const float* __restrict__ coef,
                                                  const SelRec* __restrict__ rec, int64_t TC,
                                                  int V, int32_t* __restrict__ cnt) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t > TC) return;
  int32_t n = 0;
  if (t < TC && coef[t] != 0.0f)
    for (int s = 0; s < kEnt; ++s) n += entry_row(target, rec, t, s, V) >= 0 ? 1 : 0;
  cnt[t] = n;          // cnt[TC] = 0: after the scan it holds the total
}

__global__ __launch_bounds__(256) void k_dw_keys(const int32_t* __restrict__ target,
                                                 const float* __restrict__ coef,
                                                 const SelRec* __restrict__ rec, int64_t TC,
                                                 int V, const int32_t* __restrict__ off,
                                                 int32_t* __restrict__ keys,
                                                 int32_t* __restrict__ vals) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= TC || coef[t] == 0.0f) return;
  int32_t o = off[t];
  for (int s = 0; s < kEnt; ++s) {
    const int32_t v = entry_row(target, rec, t, s, V);
    if (v < 0) continue;
    keys[o] = v;
    vals[o] = int32_t(t * kEnt + s);
    ++o;
  }
}

constexpr int kRsRounds = 16;                   // rounds of 256 keys per block
constexpr int kRsItems = 256 * kRsRounds;
static_assert(kRsItems == kRsItemsPerBlock, "sort block size");
static_assert(kEnt == kEntPerToken, "entries per token");

// Per block: the count of each 8-bit digit of its keys.  hist[d * nblk + b];
// blocks past the n entries write zeros.
__global__ __launch_bounds__(256) void k_rs_hist(const int32_t* __restrict__ keys,
                                                 const int32_t* __restrict__ nptr, int shift,
                                                 int nblk, int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[256];
  const int64_t N = *nptr;
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kRsItems;
  for (int r = 0; r < kRsRounds; ++r) {
    const int64_t i = base + r * 256 + threadIdx.x;
    if (i < N) atomicAdd(&cnt[(uint32_t(keys[i]) >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[int64_t(threadIdx.x) * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive prefix sum of a[0..n) in place, one block, n <= kScanMax: the
// array is copied into LDS with coalesced loads, each thread sums a
// contiguous run there, the run totals are scanned, each run is rewritten,
// and the result is copied back.
constexpr int kScanMax = 33 * 1024;
static_assert(kBwdChunk + 1 <= kScanMax, "per-token offsets fit the scan");
static_assert(256 * ((kBwdChunk * kEnt + kRsItems - 1) / kRsItems) <= kScanMax,
              "digit counts fit the scan");

__global__ __launch_bounds__(1024) void k_rs_scan(int32_t* __restrict__ a, int64_t n) {
  __shared__ int32_t buf[kScanMax];
  __shared__ int32_t sh[1024];
  const int tid = threadIdx.x;
  for (int64_t i = tid; i < n; i += 1024) buf[i] = a[i];
  __syncthreads();
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = tid * per, e = b + per < n ? b + per : n;
  int32_t s = 0;
  for (int64_t i = b; i < e; ++i) s += buf[i];
  sh[tid] = s;
  __syncthreads();
  for (int w = 1; w < 1024; w <<= 1) {
    const int32_t add = tid >= w ? sh[tid - w] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  int32_t run = sh[tid] - s;
  for (int64_t i = b; i < e; ++i) {
    const int32_t v = buf[i];
    buf[i] = run;
    run += v;
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 1024) a[i] = buf[i];
}

// Stable scatter by digit: within a round of 256 keys, a key's rank among
// the equal digits of lower threads comes from eight wave ballots (lanes
// with the same digit) and the per-wave digit counts of lower waves; rounds
// run in key order and advance a per-digit cursor.
__global__ __launch_bounds__(256) void k_rs_scatter(const int32_t* __restrict__ kin,
                                                    const int32_t* __restrict__ vin,
                                                    const int32_t* __restrict__ nptr, int shift,
                                                    int nblk, const int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ kout,
                                                    int32_t* __restrict__ vout) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[4][256];
  const int64_t N = *nptr;
  const int64_t base = int64_t(blockIdx.x) * kRsItems;
  if (base >= N) return;                         // uniform: nothing of this block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  run[tid] = hist[int64_t(tid) * nblk + blockIdx.x];
  const uint64_t lt = (uint64_t(1) << lane) - 1u;
  for (int r = 0; r < kRsRounds; ++r) {
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    const int64_t i = base + r * 256 + tid;
    const bool ok = i < N;
    const int32_t key = ok ? kin[i] : 0;
    const uint32_t d = (uint32_t(key) >> shift) & 255u;
    uint64_t m = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t bb = __ballot((d >> b) & 1u);
      m &= ((d >> b) & 1u) ? bb : ~bb;
    }
    const int rank = __popcll(m & lt);
    if (ok && rank == 0) wcnt[wave][d] = __popcll(m);
    __syncthreads();
    if (ok) {
      int32_t pos = run[d] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][d];
      kout[pos] = key;
      vout[pos] = vin[i];
    }
    __syncthreads();
    run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// The weight-gradient term of sorted entry `ent` for 8 hidden columns at h,
// added into acc (fp32, in the fixed order of the expression).
__device__ __forceinline__ void dw_entry(int32_t ent, const float* __restrict__ coef,
                                         const float* __restrict__ gf,
                                         const SelRec* __restrict__ rec,
                                         const uint16_t* __restrict__ hh, int H, int h,
                                         float (&acc)[8]) {
  const int64_t t = ent / kEnt;
  const int s = int(ent - t * kEnt);
  const u32x4 a = *reinterpret_cast<const u32x4*>(hh + t * H + h);
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(a[e] << 16);
    x[2 * e + 1] = __uint_as_float(a[e] & 0xFFFF0000u);
  }
  const float c = coef[t];
  if (s == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(c, x[e], acc[e]);
  } else {
    const SelRec r = rec[t * kSelSlots + s - 1];
    const float g = gf[t];
    const float am = -(c * r.p);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] = fmaf(am, x[e], acc[e]);
      acc[e] = fmaf(r.pp, bf16_to_f32(scaled_hidden(x[e], c, g)), acc[e]);
    }
  }
}

// The sorted positions are cut into aligned blocks of 64; a piece is a run
// of equal keys inside one block.  One wave per position: a wave whose
// position starts a piece sums the piece in position order.  A piece that is
// a whole bucket is added to dW[v] directly; a piece of a bucket that spans
// blocks goes to its block's partial slot 0 (the piece starts at the block
// start) or 1 (it starts later, so it is the block's last piece).
__global__ __launch_bounds__(256) void k_seg_sum(const int32_t* __restrict__ keys,
                                                 const int32_t* __restrict__ vals,
                                                 const int32_t* __restrict__ nptr,
                                                 const float* __restrict__ coef,
                                                 const float* __restrict__ gf,
                                                 const SelRec* __restrict__ rec,
                                                 const uint16_t* __restrict__ hh, int H,
                                                 float* __restrict__ dW,
                                                 float* __restrict__ part) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t N = *nptr;
  if (i >= N) return;
  const int32_t v = keys[i];
  const int64_t b = i / 64, b0 = b * 64, b1 = b0 + 64 < N ? b0 + 64 : N;
  const bool bucket_start = i == 0 || keys[i - 1] != v;
  if (i != b0 && !bucket_start) return;          // not the start of a piece
  // piece end: the first position after i in the block with another key
  const int64_t pos = i + 1 + lane;
  const uint64_t stop = __ballot(pos >= b1 || keys[pos] != v);
  const int64_t e = i + 1 + __builtin_ctzll(stop);
  const bool tail = e < b1 || e == N || keys[e] != v;
  const bool whole = bucket_start && tail;
  const int32_t my_ent = lane < e - i ? vals[i + lane] : 0;
  for (int h = lane * 8; h < H; h += 512) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < int(e - i); ++q)
      dw_entry(__builtin_amdgcn_readlane(my_ent, q), coef, gf, rec, hh, H, h, acc);
    float* o = whole ? dW + int64_t(v) * H + h
                     : part + ((2 * b + (i == b0 ? 0 : 1)) * int64_t(H) + h);
    f32x4 o0 = {acc[0], acc[1], acc[2], acc[3]}, o1 = {acc[4], acc[5], acc[6], acc[7]};
    if (whole) {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(o);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(o + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o0[k] = p0[k] + o0[k];
        o1[k] = p1[k] + o1[k];
      }
    }
    *reinterpret_cast<f32x4*>(o) = o0;
    *reinterpret_cast<f32x4*>(o + 4) = o1;
  }
}

// The buckets that span blocks: the wave of the bucket's first position adds
// the partials of its blocks in block order, then the sum to dW[v].
__global__ __launch_bounds__(256) void k_seg_merge(const int32_t* __restrict__ keys,
                                                   const int32_t* __restrict__ nptr, int H,
                                                   const float* __restrict__ part,
                                                   float* __restrict__ dW) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t N = *nptr;
  if (i >= N) return;
  const int32_t v = keys[i];
  if (i > 0 && keys[i - 1] == v) return;         // not a bucket start
  const int64_t b = i / 64, b1 = (b + 1) * 64;
  if (b1 >= N || keys[b1] != v) return;          // the bucket ends in its block
  for (int h = lane * 8; h < H; h += 512) {
    const float* p = part + (2 * b + (i == b * 64 ? 0 : 1)) * int64_t(H) + h;
    f32x4 a0 = *reinterpret_cast<const f32x4*>(p);
    f32x4 a1 = *reinterpret_cast<const f32x4*>(p + 4);
    for (int64_t bb = b + 1; bb * 64 < N && keys[bb * 64] == v; ++bb) {
      const float* pb = part + (2 * bb) * int64_t(H) + h;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(pb);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(pb + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        a0[k] = a0[k] + c0[k];
        a1[k] = a1[k] + c1[k];
      }
    }
    float* o = dW + int64_t(v) * H + h;
    f32x4 o0 = *reinterpret_cast<const f32x4*>(o);
    f32x4 o1 = *reinterpret_cast<const f32x4*>(o + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o0[k] = o0[k] + a0[k];
      o1[k] = o1[k] + a1[k];
    }
    *reinterpret_cast<f32x4*>(o) = o0;
    *reinterpret_cast<f32x4*>(o + 4) = o1;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline uint32_t nblocks(int64_t n, int64_t per) { return uint32_t(ceil_div(n, per)); }

hipError_t launch_select(const float* pm, int64_t TC, int V, const float* lse, const float* zt,
                         const int32_t* target, const float* coef, const uint32_t* D, int64_t ds,
                         const float* g, const uint16_t* E, const uint16_t* hh, const uint16_t* W,
                         int H, SelRec* rec, hipStream_t s) {
  ProfScope prof("k_select", s);
  hipLaunchKernelGGL(k_select, dim3(nblocks(TC, 64)), dim3(kSelThreads), 0, s, pm, TC,
                     n_vocab_tiles(V), lse, zt, target, coef, D, ds, g, E, vocab_pad(V) / 16, hh,
                     W, H, V, rec);
  return hipGetLastError();
}

hipError_t launch_dh_fix(const SelRec* rec, const float* coef, const uint16_t* W, int64_t TC,
                         int H, float* dh, hipStream_t s) {
  ProfScope prof("k_dh_fix", s);
  hipLaunchKernelGGL(k_dh_fix, dim3(nblocks(TC, 4)), dim3(256), 0, s, rec, coef, W, TC, H, dh);
  return hipGetLastError();
}

hipError_t launch_dw_exact(const int32_t* target, const float* coef, const float* g,
                           const SelRec* rec, const uint16_t* hh, int64_t TC, int H, int V,
                           const DwExactBufs& wb, float* dW, hipStream_t s) {
  ProfScope prof("k_onehot", s);
  const int64_t nmax = TC * kEnt;
  const int nblk = int(ceil_div(nmax, kRsItems));
  int32_t* k[2] = {wb.keys[0], wb.keys[1]};
  int32_t* v[2] = {wb.vals[0], wb.vals[1]};
  int32_t* n = wb.off + TC;                      // the entry count, after the scan
  hipLaunchKernelGGL(k_dw_count, dim3(nblocks(TC + 1, 256)), dim3(256), 0, s, target, coef, rec,
                     TC, V, wb.off);
  hipLaunchKernelGGL(k_rs_scan, dim3(1), dim3(1024), 0, s, wb.off, TC + 1);
  hipLaunchKernelGGL(k_dw_keys, dim3(nblocks(TC, 256)), dim3(256), 0, s, target, coef, rec, TC, V,
                     wb.off, k[0], v[0]);
  int cur = 0;
  for (int shift = 0; (int64_t(V) >> shift) != 0; shift += 8) {
    hipLaunchKernelGGL(k_rs_hist, dim3(nblk), dim3(256), 0, s, k[cur], n, shift, nblk, wb.hist);
    hipLaunchKernelGGL(k_rs_scan, dim3(1), dim3(1024), 0, s, wb.hist, int64_t(256) * nblk);
    hipLaunchKernelGGL(k_rs_scatter, dim3(nblk), dim3(256), 0, s, k[cur], v[cur], n, shift, nblk,
                       wb.hist, k[cur ^ 1], v[cur ^ 1]);
    cur ^= 1;
  }
  hipLaunchKernelGGL(k_seg_sum, dim3(nblocks(nmax, 4)), dim3(256), 0, s, k[cur], v[cur], n, coef,
                     g, rec, hh, H, dW, wb.seg);
  hipLaunchKernelGGL(k_seg_merge, dim3(nblocks(nmax, 4)), dim3(256), 0, s, k[cur], n, H, wb.seg,
                     dW);
  return hipGetLastError();
}

}  // namespace rz
