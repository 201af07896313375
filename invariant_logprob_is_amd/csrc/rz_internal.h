// Internal declarations shared by the kernel and ABI translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rz_util.h"

namespace rz {

// ---------------------------------------------------------------------------
// Fixed tiling.  Every shape decision below depends on (H, V) only, never on
// the token count T or on where a row sits in the batch.
// ---------------------------------------------------------------------------
constexpr int kTile = 256;          // operand rows per workgroup tile (both operands)
constexpr int kBK = 64;             // K elements per pipeline stage
constexpr int kHAlign = 64;         // H must be a multiple of this
constexpr int kMaxH = 16384;
constexpr int64_t kMaxV = 4000000;  // keeps a 256-row tile of the padded V below 2^31 bytes
constexpr int64_t kBwdChunk = 32768;  // tokens per backward / learner-step chunk (bounds the P workspace)
constexpr int kRasterGroup = 8;     // first-dimension tiles per L2 group in the tile raster
constexpr int kFwdTickets = 8;      // per-XCD tile counters of the persistent forward

// Raster group of the forward (vocabulary tiles visited for every token
// tile).  The forward keeps two things in the MALL (256 MB): the W rows of
// the current group on each of the 8 XCDs, 8 * g * 256 * H * 2 bytes, and
// the chunk's hhat, kBwdChunk * H * 2 bytes.  The largest g in {8, 4, 2}
// whose sum stays within 210 MB is taken.  Measured per step on the forward:
// at H = 1536, g = 8 beat 4 and 2 by 1% and 3%; at H = 2048, 8 and 4 tied
// (151 and 168 MB) and 2 lost 2%; at H = 2560, g = 4 (210 MB) beat 8
// (252 MB) by 8% and 2 by 1.5%.  The grouping only decides which workgroup
// computes which tile, never a result bit.
inline int fwd_raster_group(int64_t H) {
  const int64_t budget = 210LL * 1000 * 1000;
  for (int g = 8; g > 2; g /= 2)
    if (H * (8 * int64_t(g) * kTile * 2 + kBwdChunk * 2) <= budget) return g;
  return 2;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align256(size_t a) { return (a + 255) & ~size_t(255); }

inline int64_t n_vocab_tiles(int64_t V) { return ceil_div(V, kTile); }
inline int64_t vocab_pad(int64_t V) { return round_up(V, kBK); }
// Vocabulary splits: the log-sum-exp of a row is combined in two fixed
// levels, over the 256-row tiles of each split and then over the splits, in
// order.  Split s covers tiles [s n_vt / kVocabSplits, (s+1) n_vt /
// kVocabSplits), a function of V alone, so a device that holds any whole
// number of splits of W produces the same per-split partials and every
// merge gives the same bits.
constexpr int kVocabSplits = 8;
inline int64_t split_first_tile(int64_t V, int s) { return n_vocab_tiles(V) * s / kVocabSplits; }
inline int64_t split_first_row(int64_t V, int s) {
  const int64_t r = split_first_tile(V, s) * kTile;
  return r < V ? r : V;
}
// Row stride of the per-tile shift table of a chunk of tc tokens: whole
// 256-row token tiles, so the contraction reads it without a bounds check.
inline int64_t shift_stride(int64_t tc) { return round_up(tc, kTile); }

// Buffers of the weight gradient's exact entries (rz_exact.hip) for a chunk
// of tc tokens: per token kEntPerToken entries at most (the one-hot entry and
// the kSelSlots records), sorted by vocabulary row with an LSD radix sort of
// kRsItemsPerBlock keys per block; the partial sums of buckets that span
// blocks of 64 sorted positions, two per block.
constexpr int kEntPerToken = kSelSlots + 1;
constexpr int kRsItemsPerBlock = 4096;
struct DwExactBufs {
  int32_t* keys[2];
  int32_t* vals[2];
  int32_t* off;     // per-token entry offsets; off[tc] = the entry count
  int32_t* hist;    // 256 digit counts per sort block
  float* seg;       // 2 partial rows of H per block of 64 sorted positions
};
inline int64_t dw_exact_nmax(int64_t tc) { return tc * kEntPerToken; }
inline size_t dw_exact_bytes(int64_t tc, int64_t H) {
  const int64_t n = dw_exact_nmax(tc);
  const int64_t nblk = (n + kRsItemsPerBlock - 1) / kRsItemsPerBlock;
  const int64_t nseg = (n + 63) / 64;
  size_t o = 0;
  for (int i = 0; i < 4; ++i) o = align256(o + size_t(n) * 4);
  o = align256(o + size_t(tc + 1) * 4);
  o = align256(o + size_t(256) * nblk * 4);
  o = align256(o + size_t(2) * nseg * H * 4);
  return o;
}
inline DwExactBufs dw_exact_bufs(void* base, int64_t tc, int64_t H) {
  (void)H;
  const int64_t n = dw_exact_nmax(tc);
  const int64_t nblk = (n + kRsItemsPerBlock - 1) / kRsItemsPerBlock;
  char* b = static_cast<char*>(base);
  DwExactBufs w;
  size_t o = 0;
  w.keys[0] = reinterpret_cast<int32_t*>(b + o); o = align256(o + size_t(n) * 4);
  w.vals[0] = reinterpret_cast<int32_t*>(b + o); o = align256(o + size_t(n) * 4);
  w.keys[1] = reinterpret_cast<int32_t*>(b + o); o = align256(o + size_t(n) * 4);
  w.vals[1] = reinterpret_cast<int32_t*>(b + o); o = align256(o + size_t(n) * 4);
  w.off = reinterpret_cast<int32_t*>(b + o);     o = align256(o + size_t(tc + 1) * 4);
  w.hist = reinterpret_cast<int32_t*>(b + o);    o = align256(o + size_t(256) * nblk * 4);
  w.seg = reinterpret_cast<float*>(b + o);
  return w;
}

// Workspace layout; every region starts on a 256-byte boundary.  Regions of
// different entry points overlap (calls on one workspace are ordered).
struct WsLayout {
  // rz_logprob (chunks of at most kBwdChunk tokens)
  size_t tick, hhat, pm, ps, ztgt, fwd_end;
  // rz_backward (chunks of at most kBwdChunk tokens)
  size_t b_tick, b_hhat, b_wt, b_e, b_pm, b_ps, b_zt, b_d, b_g, b_rec, bwd_end;
  // rz_is_loss / rz_d3
  size_t part, flag, loss_end;
  // rz_learner_step (chunks of at most kBwdChunk tokens)
  size_t s_tick, s_hhat, s_wt, s_e, s_pm, s_ps, s_zt, s_d, s_g, s_rec, s_cs, s_lse, s_coef,
      s_part, s_flag, step_end;
  // rz_learner_step with weight gradients: the step region, then these
  size_t g_hs, g_dw, g_rbuf, g_part, grads_end;
  size_t total;
};

inline WsLayout ws_layout(int64_t T, int64_t H, int64_t V) {
  WsLayout L{};
  const int64_t nvt = n_vocab_tiles(V);
  const int64_t Vp = vocab_pad(V);
  const int64_t tc = T < kBwdChunk ? T : kBwdChunk;
  const int64_t tcp = shift_stride(tc);
  size_t o = 0;
  L.tick = o;  o = align256(o + kFwdTickets * 4);
  L.hhat = o;  o = align256(o + size_t(tc) * H * 2);
  L.pm = o;    o = align256(o + size_t(nvt) * tc * 4);
  L.ps = o;    o = align256(o + size_t(nvt) * tc * 4);
  L.ztgt = o;  o = align256(o + size_t(tc) * 4);
  L.fwd_end = o;
  o = 0;
  L.b_tick = o; o = align256(o + kFwdTickets * 4);
  L.b_hhat = o; o = align256(o + size_t(tc) * H * 2);
  L.b_wt = o;   o = align256(o + size_t(H) * Vp * 2);
  L.b_e = o;    o = align256(o + size_t(tcp) * Vp * 2);
  L.b_pm = o;   o = align256(o + size_t(nvt) * tc * 4);
  L.b_ps = o;   o = align256(o + size_t(nvt) * tc * 4);
  L.b_zt = o;   o = align256(o + size_t(tc) * 4);
  L.b_d = o;    o = align256(o + size_t(nvt) * tcp * 4);
  L.b_g = o;    o = align256(o + size_t(tc) * 4);
  L.b_rec = o;  o = align256(o + size_t(tc) * kSelSlots * sizeof(SelRec));
  L.bwd_end = o;
  o = 0;
  L.part = o;   o = align256(o + size_t(T + 8) * 8);
  L.flag = o;   o = align256(o + 4);
  L.loss_end = o;
  o = 0;
  L.s_tick = o; o = align256(o + kFwdTickets * 4);
  L.s_hhat = o; o = align256(o + size_t(tc) * H * 2);
  L.s_wt = o;   o = align256(o + size_t(H) * Vp * 2);
  L.s_e = o;    o = align256(o + size_t(tcp) * Vp * 2);
  L.s_pm = o;   o = align256(o + size_t(nvt) * tc * 4);
  L.s_ps = o;   o = align256(o + size_t(nvt) * tc * 4);
  L.s_zt = o;   o = align256(o + size_t(tc) * 4);
  L.s_d = o;    o = align256(o + size_t(nvt) * tcp * 4);
  L.s_g = o;    o = align256(o + size_t(tc) * 4);
  L.s_rec = o;  o = align256(o + size_t(tc) * kSelSlots * sizeof(SelRec));
  L.s_cs = o;   o = align256(o + size_t(T) * 8);
  L.s_lse = o;  o = align256(o + size_t(T) * 4);
  L.s_coef = o; o = align256(o + size_t(T) * 4);
  L.s_part = o; o = align256(o + size_t(T + 8) * 8);
  L.s_flag = o; o = align256(o + 4);
  L.step_end = o;
  // the chunk's hhat rows scaled by coef_t g_t (bf16), token-contiguous
  L.g_hs = o;   o = align256(o + size_t(H) * tcp * 2);
  // the sort and sums of the exact entries; then the chunk's row factors r_t
  L.g_dw = o;   o = align256(o + dw_exact_bytes(tc, H));
  L.g_rbuf = o; o = align256(o + size_t(tc) * 8);
  L.g_part = o; o = align256(o + size_t(ceil_div(T, kTile)) * H * 8);
  L.grads_end = o;
  L.total = L.fwd_end;
  if (L.bwd_end > L.total) L.total = L.bwd_end;
  if (L.loss_end > L.total) L.total = L.loss_end;
  if (L.step_end > L.total) L.total = L.step_end;
  return L;
}

// Stored logits (rz_logprob_store / rz_backward_stored): chunk c of at most
// kBwdChunk tokens at byte c * stride holds its e block (fragment order, as
// the forward writes it), its tile maxima pm [n_vt][tc] and its target
// logits [tc].
struct StoredLayout {
  size_t e, pm, zt, stride, total;
};

inline StoredLayout stored_layout(int64_t T, int64_t V) {
  StoredLayout S{};
  const int64_t tc = T < kBwdChunk ? T : kBwdChunk;
  const int64_t tcp = shift_stride(tc);
  size_t o = 0;
  S.e = o;   o = align256(o + size_t(tcp) * vocab_pad(V) * 2);
  S.pm = o;  o = align256(o + size_t(n_vocab_tiles(V)) * tc * 4);
  S.zt = o;  o = align256(o + size_t(tc) * 4);
  S.stride = o;
  S.total = size_t(ceil_div(T, kBwdChunk)) * S.stride;
  return S;
}

// ---------------------------------------------------------------------------
// Optional per-kernel timing (rz_profile.hip).  While enabled, a ProfScope
// records a hipEvent on the launch stream before and after the launches in
// its scope; disabled, it costs one relaxed load.
// ---------------------------------------------------------------------------
bool profile_enabled();
void profile_record(const char* name, hipStream_t s, bool start);

struct ProfScope {
  const char* name;
  hipStream_t s;
  bool on;
  ProfScope(const char* n, hipStream_t st) : name(n), s(st), on(profile_enabled()) {
    if (on) profile_record(name, s, true);
  }
  ~ProfScope() {
    if (on) profile_record(name, s, false);
  }
};

// ---------------------------------------------------------------------------
// Kernel launchers (rz_kernels.hip).  All enqueue on `s` and return the
// launch status (hipGetLastError after the launches).
// ---------------------------------------------------------------------------
// rstd (fp32 rounding of the float64 r of each row) may be null.
hipError_t launch_rmsnorm_fwd(const uint16_t* x, const uint16_t* gamma, float eps,
                              int64_t T, int H, uint16_t* hhat, float* rstd, hipStream_t s);
// ticket: kFwdTickets ints of device memory for the persistent forward's
// tile counters (reset by the launch).
hipError_t launch_lmhead_fwd(const uint16_t* hhat, const uint16_t* W, const int32_t* target,
                             int64_t T, int H, int V, float* pm, float* ps, float* ztgt,
                             uint16_t* E, int* ticket, hipStream_t s);
// The forward over the vocabulary rows [v0, v0 + Vs) of a model with V rows
// in all (W points at row v0; targets are global row indices).  ztgt starts
// at 0: only rows whose target lies in the range get their logit.
hipError_t launch_lmhead_fwd_range(const uint16_t* hhat, const uint16_t* W, const int32_t* target,
                                   int64_t T, int H, int64_t v0, int Vs, float* pm, float* ps,
                                   float* ztgt, int* ticket, hipStream_t s);
// Per-split records (struct rz_vocab_split of rz.h) for splits [s0, s1) of a
// model with V rows, from the tile partials of the range forward above
// (whose first tile is split s0's); out[(s - s0) * out_stride + t].
hipError_t launch_split_partials(const float* pm, const float* ps, const float* ztgt,
                                 const int32_t* target, int64_t T, int V, int s0, int s1,
                                 void* out, int64_t out_stride, hipStream_t s);
// logprob and lse from all kVocabSplits records of each row (the same
// arithmetic as launch_lse_combine).
hipError_t launch_split_merge(const void* parts, int64_t part_stride, const int32_t* target,
                              int64_t T, int V, float* logprob, float* lse, hipStream_t s);
hipError_t launch_lse_combine(const float* pm, const float* ps, const float* ztgt,
                              int64_t T, int V, float* logprob, float* lse, const double* cs,
                              const float* mu, float* coef, uint32_t* D, int64_t ds, float* g,
                              hipStream_t s);
hipError_t launch_shift_prep(const float* pm, const float* lse, int64_t T, int V, uint32_t* D,
                             int64_t ds, float* g, hipStream_t s);
// Checks the ragged structure into *ok (an int in device memory), then
// writes the token scale (NaN for every token when the structure is
// malformed).
hipError_t launch_token_scale(const int64_t* ro, int R, const int64_t* go, int G,
                              const float* reward, int64_t T, int* ok, double* cs,
                              hipStream_t s);
hipError_t launch_transpose_w(const uint16_t* W, int H, int V, uint16_t* Wt, hipStream_t s);
hipError_t launch_dhidden(const uint16_t* E, const uint32_t* D, int64_t ds, const float* g,
                          const uint16_t* Wt, const uint16_t* W, const int32_t* target_chunk,
                          const float* coef_chunk, int64_t TC, int H, int V, float* dh_chunk,
                          hipStream_t s);
hipError_t launch_rmsnorm_bwd(const uint16_t* x, const uint16_t* gamma, float eps,
                              int64_t T, int H, float* dh, hipStream_t s);
// The loss, coef and advantages; with check, the structure flag *ok is
// computed first, otherwise it is the one launch_token_scale computed.
hipError_t launch_is_loss(const float* logprob, const float* mu, int64_t T,
                          const int64_t* ro, int R, const int64_t* go, int G,
                          const float* reward, double* loss, float* coef, float* adv,
                          double* part, int* ok, bool check, hipStream_t s);
hipError_t launch_d3(const float* logprob, const float* mu, int64_t T, double* d3,
                     double* part, hipStream_t s);
// The exact entries of a chunk (rz_exact.hip): the records of each token's
// dominant probabilities, from the tile partials pm, lse, the target logit
// zt, coef, the shift table and row factor, the stored e, hhat and W.
hipError_t launch_select(const float* pm, int64_t TC, int V, const float* lse, const float* zt,
                         const int32_t* target, const float* coef, const uint32_t* D, int64_t ds,
                         const float* g, const uint16_t* E, const uint16_t* hh, const uint16_t* W,
                         int H, SelRec* rec, hipStream_t s);
// dhhat_t -= coef_t sum_records beta W[v] (before the RMSNorm backward).
hipError_t launch_dh_fix(const SelRec* rec, const float* coef, const uint16_t* W, int64_t TC,
                         int H, float* dh, hipStream_t s);
// dW[v] += the one-hot terms and the records' exact terms, per row in token
// order (after the chunk's weight-gradient contraction).
hipError_t launch_dw_exact(const int32_t* target, const float* coef, const float* g,
                           const SelRec* rec, const uint16_t* hh, int64_t TC, int H, int V,
                           const DwExactBufs& wb, float* dW, hipStream_t s);
hipError_t launch_weight_grads_chunk(const uint16_t* E, const uint32_t* D, int64_t ds,
                                    const float* g, const float* coef_chunk,
                                    const int32_t* target_chunk, const uint16_t* hh,
                                    const uint16_t* x_chunk, float eps, const float* dhh_chunk,
                                    int64_t TC, int H, int V, int64_t gb0, int first,
                                    uint16_t* hs, const SelRec* rec, const DwExactBufs& wb,
                                    double* rbuf, double* gpart, float* dW, hipStream_t s);
hipError_t launch_dgamma_final(const double* gpart, int64_t nb, int H, float* dgamma,
                               hipStream_t s);
hipError_t launch_kl(const float* logprob, const float* mu, int64_t T, double* kl,
                     double* part, hipStream_t s);
hipError_t launch_decompose(const float* lp_new, const float* lp_old, const float* mu, int64_t T,
                            float* lag, float* mismatch, double* summary, double* part,
                            hipStream_t s);

}  // namespace rz
