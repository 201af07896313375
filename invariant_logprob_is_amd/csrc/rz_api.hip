// C ABI of the learner head (declared in include/rz.h).  Every check that
// needs no device data runs before the first HIP call.
#include <atomic>
#include <mutex>

#include "rz.h"
#include "rz_internal.h"

namespace {

using namespace rz;

constexpr int kVersion = (0 << 16) | (1 << 8) | 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return RZ_ENODEV;
  }
  return RZ_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? RZ_OK : RZ_EHIP; }

// Shape checks shared by rz_logprob and rz_backward.
int check_head_shape(int64_t T, int32_t H, int32_t V) {
  if (T < 1 || H < 1 || V < 1) return RZ_EINVAL;
  if (H % kHAlign != 0 || H > kMaxH || int64_t(V) > kMaxV) return RZ_EUNSUPPORTED;
  return RZ_OK;
}

template <class T_>
T_* at(void* ws, size_t off) {
  return reinterpret_cast<T_*>(static_cast<char*>(ws) + off);
}

// a1-a3 for rz_logprob and rz_decompose (arguments already checked), in
// chunks of at most kBwdChunk tokens: a chunk's hhat (100 MB at H = 1536)
// stays cache-resident while the vocabulary tiles stream past it.  Rows are
// independent, so the chunking changes no bit of any row.
hipError_t run_logprob(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                       const int32_t* target, int64_t T, int32_t H, int32_t V, float* logprob,
                       float* lse, void* workspace, const WsLayout& L, hipStream_t s) {
  uint16_t* hhat = at<uint16_t>(workspace, L.hhat);
  float* pm = at<float>(workspace, L.pm);
  float* ps = at<float>(workspace, L.ps);
  float* zt = at<float>(workspace, L.ztgt);
  int* tick = at<int>(workspace, L.tick);
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hhat, nullptr, s);
    if (e == hipSuccess)
      e = launch_lmhead_fwd(hhat, W, target + c0, tc, H, V, pm, ps, zt, nullptr, tick, s);
    if (e == hipSuccess)
      e = launch_lse_combine(pm, ps, zt, tc, V, logprob + c0, lse ? lse + c0 : nullptr, nullptr,
                             nullptr, nullptr, nullptr, 0, nullptr, s);
  }
  return e;
}

// The forward of rz_logprob over the rows of splits [s0, s1) (W points at
// the first of them), reduced to one record per split and row.
hipError_t run_shard(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                     const int32_t* target, int64_t T, int32_t H, int32_t V, int s0, int s1,
                     void* partials, void* workspace, const WsLayout& L, hipStream_t s) {
  uint16_t* hhat = at<uint16_t>(workspace, L.hhat);
  float* pm = at<float>(workspace, L.pm);
  float* ps = at<float>(workspace, L.ps);
  float* zt = at<float>(workspace, L.ztgt);
  const int64_t v0 = split_first_row(V, s0);
  const int Vs = int(split_first_row(V, s1) - v0);
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hhat, nullptr, s);
    if (e == hipSuccess)
      e = launch_lmhead_fwd_range(hhat, W, target + c0, tc, H, v0, Vs, pm, ps, zt,
                                  at<int>(workspace, L.tick), s);
    if (e == hipSuccess)
      e = launch_split_partials(pm, ps, zt, target + c0, tc, V, s0, s1,
                                static_cast<char*>(partials) + c0 * sizeof(rz_vocab_split), T, s);
  }
  return e;
}

// ---------------------------------------------------------------------------
// Scratch of rz_logprob_noalloc: a file-scope device array, which every GPU
// the library runs on holds until the process ends.  In host code its name
// is only a stand-in; the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what
// the kernels get.  Nothing in it has to start at zero: the forward writes
// every partial it later reads, and the target logits are filled by a
// kernel before the forward.
// ---------------------------------------------------------------------------
static_assert(RZ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[RZ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

// Argument checks shared by rz_backward and rz_backward_stored.
int check_backward(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                   const int32_t* target, const float* lse, const float* coef, int64_t T,
                   int32_t H, int32_t V, float* dhidden, void* workspace,
                   size_t workspace_bytes) {
  if (!x || !gamma || !W || !target || !lse || !coef || !dhidden || !workspace) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W) || !aligned4(target) || !aligned4(lse) ||
      !aligned4(coef) || !aligned16(dhidden) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  const int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  if (workspace_bytes < ws_layout(T, H, V).total) return RZ_EWORKSPACE;
  return RZ_OK;
}

// rz_backward, rz_backward_stored (stored != nullptr) and rz_backward_grads
// (dW != nullptr): per chunk, the forward with the e store (its (m, S,
// z_target) partials are recomputed and left unused) or the stored chunk, the
// shift table from the given lse, then the same contractions the learner
// step runs (with the weight gradients, dW and dgamma as well).
hipError_t run_backward(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                        const int32_t* target, const float* lse, const float* coef, int64_t T,
                        int32_t H, int32_t V, const char* stored, float* dhidden, float* dW,
                        float* dgamma, void* workspace, hipStream_t s) {
  const WsLayout L = ws_layout(T, H, V);
  const StoredLayout SL = stored_layout(T, V);
  uint16_t* hh = at<uint16_t>(workspace, L.b_hhat);
  uint16_t* Wt = at<uint16_t>(workspace, L.b_wt);
  uint32_t* D = at<uint32_t>(workspace, L.b_d);
  float* g = at<float>(workspace, L.b_g);
  SelRec* rec = at<SelRec>(workspace, L.b_rec);
  hipError_t e = launch_transpose_w(W, H, V, Wt, s);
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    const int64_t ds = shift_stride(tc);
    const uint16_t* E;
    const float* pm;
    const float* zt;
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hh, nullptr, s);
    if (stored) {
      const char* c = stored + size_t(c0 / kBwdChunk) * SL.stride;
      E = reinterpret_cast<const uint16_t*>(c + SL.e);
      pm = reinterpret_cast<const float*>(c + SL.pm);
      zt = reinterpret_cast<const float*>(c + SL.zt);
    } else {
      uint16_t* Ew = at<uint16_t>(workspace, L.b_e);
      float* pmw = at<float>(workspace, L.b_pm);
      float* ztw = at<float>(workspace, L.b_zt);
      if (e == hipSuccess)
        e = launch_lmhead_fwd(hh, W, target + c0, tc, H, V, pmw, at<float>(workspace, L.b_ps), ztw,
                              Ew, at<int>(workspace, L.b_tick), s);
      E = Ew;
      pm = pmw;
      zt = ztw;
    }
    if (e == hipSuccess) e = launch_shift_prep(pm, lse + c0, tc, V, D, ds, g, s);
    if (e == hipSuccess)
      e = launch_select(pm, tc, V, lse + c0, zt, target + c0, coef + c0, D, ds, g, E, hh, W, H,
                        rec, s);
    if (e == hipSuccess)
      e = launch_dhidden(E, D, ds, g, Wt, W, target + c0, coef + c0, tc, H, V, dhidden + c0 * H, s);
    if (e == hipSuccess) e = launch_dh_fix(rec, coef + c0, W, tc, H, dhidden + c0 * H, s);
    if (e == hipSuccess && dW)
      e = launch_weight_grads_chunk(E, D, ds, g, coef + c0, target + c0, hh, x + c0 * H, eps,
                                    dhidden + c0 * H, tc, H, V, c0 / kTile, c0 == 0,
                                    at<uint16_t>(workspace, L.g_hs), rec,
                                    dw_exact_bufs(at<char>(workspace, L.g_dw), tc, H),
                                    at<double>(workspace, L.g_rbuf),
                                    at<double>(workspace, L.g_part), dW, s);
    if (e == hipSuccess) e = launch_rmsnorm_bwd(x + c0 * H, gamma, eps, tc, H, dhidden + c0 * H, s);
  }
  if (e == hipSuccess && dW)
    e = launch_dgamma_final(at<double>(workspace, L.g_part), ceil_div(T, kTile), H, dgamma, s);
  return e;
}

}  // namespace

extern "C" {

int rz_version(void) { return kVersion; }

const char* rz_status_string(int status) {
  switch (status) {
    case RZ_OK: return "ok";
    case RZ_EINVAL: return "invalid argument";
    case RZ_EUNSUPPORTED: return "unsupported shape";
    case RZ_ENODEV: return "no HIP device";
    case RZ_EHIP: return "HIP runtime error";
    case RZ_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

size_t rz_workspace_bytes(int64_t T, int32_t H, int32_t V) {
  if (T < 1 || H < 1 || V < 1) return 0;
  return ws_layout(T, H, V).total;
}

size_t rz_workspace_bytes_grads(int64_t T, int32_t H, int32_t V) {
  if (T < 1 || H < 1 || V < 1) return 0;
  const WsLayout L = ws_layout(T, H, V);
  return L.grads_end > L.total ? L.grads_end : L.total;
}

int rz_logprob(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
               const int32_t* target, int64_t T, int32_t H, int32_t V, float* logprob,
               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !gamma || !W || !target || !logprob || !workspace) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W) || !aligned4(target) ||
      !aligned4(logprob) || (lse && !aligned4(lse)) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  const WsLayout L = ws_layout(T, H, V);
  if (workspace_bytes < L.total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;

  return status_of(run_logprob(x, gamma, eps, W, target, T, H, V, logprob, lse, workspace, L,
                               static_cast<hipStream_t>(stream)));
}

int rz_logprob_noalloc(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                       const int32_t* target, int64_t T, int32_t H, int32_t V, float* logprob,
                       float* lse, void* stream) {
  if (!x || !gamma || !W || !target || !logprob) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W) || !aligned4(target) ||
      !aligned4(logprob) || (lse && !aligned4(lse)))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  const WsLayout L = ws_layout(T, H, V);
  if (L.fwd_end > size_t(RZ_NOALLOC_SCRATCH_BYTES)) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;
  void* ws = nullptr;
  if (scratch_on_current_device(&ws) != hipSuccess) return RZ_EHIP;
  // the same launches as rz_logprob, on the built-in scratch
  return status_of(run_logprob(x, gamma, eps, W, target, T, H, V, logprob, lse, ws, L,
                               static_cast<hipStream_t>(stream)));
}

int rz_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T, int32_t H,
               uint16_t* hhat, float* rstd, void* stream) {
  if (!x || !gamma || !hhat) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(hhat) || (rstd && !aligned4(rstd)))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  if (T < 1 || H < 1) return RZ_EINVAL;
  if (H % kHAlign != 0 || H > kMaxH) return RZ_EUNSUPPORTED;
  const int st = check_device();
  if (st != RZ_OK) return st;
  // the same kernel and chunking as the first step of rz_logprob
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hhat + c0 * H, rstd ? rstd + c0 : nullptr,
                           s);
  }
  return status_of(e);
}

static_assert(RZ_VOCAB_SPLITS == kVocabSplits, "split count");
static_assert(sizeof(rz_vocab_split) == 24 && alignof(rz_vocab_split) == 8, "record layout");

int64_t rz_vocab_split_begin(int32_t V, int32_t s) {
  if (V < 1 || int64_t(V) > kMaxV || s < 0 || s > RZ_VOCAB_SPLITS) return -1;
  return split_first_row(V, s);
}

int rz_logprob_shard(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W_rows,
                     const int32_t* target, int64_t T, int32_t H, int32_t V, int32_t s0,
                     int32_t s1, rz_vocab_split* partials, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!x || !gamma || !W_rows || !target || !partials || !workspace) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W_rows) || !aligned4(target) ||
      (reinterpret_cast<uintptr_t>(partials) & 7u) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  if (s0 < 0 || s1 <= s0 || s1 > RZ_VOCAB_SPLITS) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  const WsLayout L = ws_layout(T, H, V);
  if (workspace_bytes < L.total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;
  return status_of(run_shard(x, gamma, eps, W_rows, target, T, H, V, s0, s1, partials, workspace,
                             L, static_cast<hipStream_t>(stream)));
}

int rz_logprob_merge(const rz_vocab_split* partials, const int32_t* target, int64_t T, int32_t V,
                     float* logprob, float* lse, void* stream) {
  if (!partials || !target || !logprob) return RZ_EINVAL;
  if ((reinterpret_cast<uintptr_t>(partials) & 7u) || !aligned4(target) || !aligned4(logprob) ||
      (lse && !aligned4(lse)))
    return RZ_EINVAL;
  if (T < 1 || V < 1 || int64_t(V) > kMaxV) return RZ_EINVAL;
  const int st = check_device();
  if (st != RZ_OK) return st;
  return status_of(launch_split_merge(partials, T, target, T, V, logprob, lse,
                                      static_cast<hipStream_t>(stream)));
}

int rz_is_loss(const float* logprob, const float* rollout_logprob, int64_t T,
               const int64_t* resp_offsets, int32_t R, const int64_t* group_offsets, int32_t G,
               const float* reward, double* loss, float* coef, float* advantage, void* workspace,
               size_t workspace_bytes, void* stream) {
  if (!logprob || !rollout_logprob || !resp_offsets || !group_offsets || !reward || !loss ||
      !workspace)
    return RZ_EINVAL;
  if (!aligned4(logprob) || !aligned4(rollout_logprob) || !aligned8(resp_offsets) ||
      !aligned8(group_offsets) || !aligned4(reward) || !aligned8(loss) ||
      (coef && !aligned4(coef)) || (advantage && !aligned4(advantage)) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (T < 1 || R < 1 || G < 1 || int64_t(R) > T || G > R) return RZ_EINVAL;
  const WsLayout L = ws_layout(T, 64, 1);
  if (workspace_bytes < L.loss_end) return RZ_EWORKSPACE;
  const int st = check_device();
  if (st != RZ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(launch_is_loss(logprob, rollout_logprob, T, resp_offsets, R, group_offsets, G,
                                  reward, loss, coef, advantage, at<double>(workspace, L.part),
                                  at<int>(workspace, L.flag), true, s));
}

int rz_d3(const float* logprob, const float* rollout_logprob, int64_t T, double* d3,
          void* workspace, size_t workspace_bytes, void* stream) {
  if (!logprob || !rollout_logprob || !d3 || !workspace) return RZ_EINVAL;
  if (!aligned4(logprob) || !aligned4(rollout_logprob) || !aligned8(d3) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (T < 1) return RZ_EINVAL;
  const WsLayout L = ws_layout(T, 64, 1);
  if (workspace_bytes < L.loss_end) return RZ_EWORKSPACE;
  const int st = check_device();
  if (st != RZ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(launch_d3(logprob, rollout_logprob, T, d3, at<double>(workspace, L.part), s));
}

int rz_kl(const float* logprob, const float* rollout_logprob, int64_t T, double* kl,
          void* workspace, size_t workspace_bytes, void* stream) {
  if (!logprob || !rollout_logprob || !kl || !workspace) return RZ_EINVAL;
  if (!aligned4(logprob) || !aligned4(rollout_logprob) || !aligned8(kl) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (T < 1) return RZ_EINVAL;
  const WsLayout L = ws_layout(T, 64, 1);
  if (workspace_bytes < L.loss_end) return RZ_EWORKSPACE;
  const int st = check_device();
  if (st != RZ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(launch_kl(logprob, rollout_logprob, T, kl, at<double>(workspace, L.part), s));
}

int rz_decompose(const uint16_t* x_new, const uint16_t* gamma_new, const uint16_t* W_new,
                 const uint16_t* x_old, const uint16_t* gamma_old, const uint16_t* W_old,
                 float eps, const int32_t* target, const float* rollout_logprob, int64_t T,
                 int32_t H, int32_t V, float* lag, float* mismatch, double* summary,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!x_new || !gamma_new || !W_new || !x_old || !gamma_old || !W_old || !target ||
      !rollout_logprob || !lag || !mismatch || !summary || !workspace)
    return RZ_EINVAL;
  if (!aligned16(x_new) || !aligned16(gamma_new) || !aligned16(W_new) || !aligned16(x_old) ||
      !aligned16(gamma_old) || !aligned16(W_old) || !aligned4(target) ||
      !aligned4(rollout_logprob) || !aligned4(lag) || !aligned4(mismatch) || !aligned8(summary) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (lag == mismatch || rollout_logprob == lag || rollout_logprob == mismatch) return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  const WsLayout L = ws_layout(T, H, V);
  if (workspace_bytes < L.total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the two log-probabilities go straight into the output arrays; the last
  // kernel turns them into (lag, mismatch) in place
  hipError_t e = run_logprob(x_new, gamma_new, eps, W_new, target, T, H, V, lag, nullptr,
                             workspace, L, s);
  if (e == hipSuccess)
    e = run_logprob(x_old, gamma_old, eps, W_old, target, T, H, V, mismatch, nullptr, workspace,
                    L, s);
  if (e == hipSuccess)
    e = launch_decompose(lag, mismatch, rollout_logprob, T, lag, mismatch, summary,
                         at<double>(workspace, L.part), s);
  return status_of(e);
}

int rz_backward(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                const int32_t* target, const float* lse, const float* coef, int64_t T, int32_t H,
                int32_t V, float* dhidden, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_backward(x, gamma, eps, W, target, lse, coef, T, H, V, dhidden, workspace,
                          workspace_bytes);
  if (st != RZ_OK) return st;
  st = check_device();
  if (st != RZ_OK) return st;
  return status_of(run_backward(x, gamma, eps, W, target, lse, coef, T, H, V, nullptr, dhidden,
                                nullptr, nullptr, workspace, static_cast<hipStream_t>(stream)));
}

size_t rz_logits_bytes(int64_t T, int32_t H, int32_t V) {
  if (T < 1 || H < 1 || V < 1) return 0;
  return stored_layout(T, V).total;
}

int rz_logprob_store(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                     const int32_t* target, int64_t T, int32_t H, int32_t V, float* logprob,
                     float* lse, void* logits, size_t logits_bytes, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!x || !gamma || !W || !target || !logprob || !logits || !workspace) return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W) || !aligned4(target) ||
      !aligned4(logprob) || (lse && !aligned4(lse)) ||
      (reinterpret_cast<uintptr_t>(logits) & 255u) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  const WsLayout L = ws_layout(T, H, V);
  const StoredLayout SL = stored_layout(T, V);
  if (workspace_bytes < L.total || logits_bytes < SL.total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;

  // rz_logprob's chunks, with the e store and the partials in `logits`
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* hhat = at<uint16_t>(workspace, L.hhat);
  float* ps = at<float>(workspace, L.ps);
  int* tick = at<int>(workspace, L.tick);
  hipError_t e = hipSuccess;
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    char* c = static_cast<char*>(logits) + size_t(c0 / kBwdChunk) * SL.stride;
    float* pm = reinterpret_cast<float*>(c + SL.pm);
    float* zt = reinterpret_cast<float*>(c + SL.zt);
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hhat, nullptr, s);
    if (e == hipSuccess)
      e = launch_lmhead_fwd(hhat, W, target + c0, tc, H, V, pm, ps, zt,
                            reinterpret_cast<uint16_t*>(c + SL.e), tick, s);
    if (e == hipSuccess)
      e = launch_lse_combine(pm, ps, zt, tc, V, logprob + c0, lse ? lse + c0 : nullptr, nullptr,
                             nullptr, nullptr, nullptr, 0, nullptr, s);
  }
  return status_of(e);
}

int rz_backward_stored(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                       const int32_t* target, const float* lse, const float* coef, int64_t T,
                       int32_t H, int32_t V, const void* logits, size_t logits_bytes,
                       float* dhidden, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_backward(x, gamma, eps, W, target, lse, coef, T, H, V, dhidden, workspace,
                          workspace_bytes);
  if (st != RZ_OK) return st;
  if (!logits || (reinterpret_cast<uintptr_t>(logits) & 255u)) return RZ_EINVAL;
  if (logits_bytes < stored_layout(T, V).total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;
  return status_of(run_backward(x, gamma, eps, W, target, lse, coef, T, H, V,
                                static_cast<const char*>(logits), dhidden, nullptr, nullptr,
                                workspace, static_cast<hipStream_t>(stream)));
}

int rz_backward_grads(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                      const int32_t* target, const float* lse, const float* coef, int64_t T,
                      int32_t H, int32_t V, const void* logits, size_t logits_bytes,
                      float* dhidden, float* dW, float* dgamma, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_backward(x, gamma, eps, W, target, lse, coef, T, H, V, dhidden, workspace,
                          workspace_bytes);
  if (st != RZ_OK) return st;
  if (!dW || !dgamma || !aligned16(dW) || !aligned4(dgamma)) return RZ_EINVAL;
  if (logits && (reinterpret_cast<uintptr_t>(logits) & 255u)) return RZ_EINVAL;
  if (workspace_bytes < ws_layout(T, H, V).grads_end) return RZ_EWORKSPACE;
  if (logits && logits_bytes < stored_layout(T, V).total) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;
  return status_of(run_backward(x, gamma, eps, W, target, lse, coef, T, H, V,
                                static_cast<const char*>(logits), dhidden, dW, dgamma, workspace,
                                static_cast<hipStream_t>(stream)));
}



int rz_learner_step(const uint16_t* x, const uint16_t* gamma, float eps, const uint16_t* W,
                    const int32_t* target, const float* rollout_logprob, int64_t T, int32_t H,
                    int32_t V, const int64_t* resp_offsets, int32_t R,
                    const int64_t* group_offsets, int32_t G, const float* reward, float* logprob,
                    float* lse, double* loss, double* d3, double* kl, float* coef, float* dhidden,
                    float* dW, float* dgamma, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!x || !gamma || !W || !target || !rollout_logprob || !resp_offsets || !group_offsets ||
      !reward || !logprob || !loss || !d3 || !dhidden || !workspace)
    return RZ_EINVAL;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(W) || !aligned4(target) ||
      !aligned4(rollout_logprob) || !aligned8(resp_offsets) || !aligned8(group_offsets) ||
      !aligned4(reward) || !aligned4(logprob) || (lse && !aligned4(lse)) || !aligned8(loss) ||
      !aligned8(d3) || (kl && !aligned8(kl)) || (coef && !aligned4(coef)) || !aligned16(dhidden) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return RZ_EINVAL;
  if (!(eps >= 0.0f)) return RZ_EINVAL;
  if ((dW == nullptr) != (dgamma == nullptr)) return RZ_EINVAL;
  if ((dW && !aligned16(dW)) || (dgamma && !aligned4(dgamma))) return RZ_EINVAL;
  int st = check_head_shape(T, H, V);
  if (st != RZ_OK) return st;
  if (R < 1 || G < 1 || int64_t(R) > T || G > R) return RZ_EINVAL;
  const WsLayout L = ws_layout(T, H, V);
  const bool grads = dW != nullptr;
  if (workspace_bytes < L.total || (grads && workspace_bytes < L.grads_end)) return RZ_EWORKSPACE;
  st = check_device();
  if (st != RZ_OK) return st;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* hh = at<uint16_t>(workspace, L.s_hhat);
  uint16_t* Wt = at<uint16_t>(workspace, L.s_wt);
  uint16_t* E = at<uint16_t>(workspace, L.s_e);
  float* pm = at<float>(workspace, L.s_pm);
  float* ps = at<float>(workspace, L.s_ps);
  float* zt = at<float>(workspace, L.s_zt);
  uint32_t* D = at<uint32_t>(workspace, L.s_d);
  float* g = at<float>(workspace, L.s_g);
  SelRec* rec = at<SelRec>(workspace, L.s_rec);
  double* cs = at<double>(workspace, L.s_cs);
  float* lse_ = lse ? lse : at<float>(workspace, L.s_lse);
  float* coef_ = coef ? coef : at<float>(workspace, L.s_coef);
  double* part = at<double>(workspace, L.s_part);
  int* ok = at<int>(workspace, L.s_flag);

  hipError_t e = launch_transpose_w(W, H, V, Wt, s);
  if (e == hipSuccess)
    e = launch_token_scale(resp_offsets, R, group_offsets, G, reward, T, ok, cs, s);
  for (int64_t c0 = 0; c0 < T && e == hipSuccess; c0 += kBwdChunk) {
    const int64_t tc = (T - c0 < kBwdChunk) ? T - c0 : kBwdChunk;
    const int64_t ds = shift_stride(tc);
    e = launch_rmsnorm_fwd(x + c0 * H, gamma, eps, tc, H, hh, nullptr, s);
    if (e == hipSuccess)
      e = launch_lmhead_fwd(hh, W, target + c0, tc, H, V, pm, ps, zt, E,
                            at<int>(workspace, L.s_tick), s);
    if (e == hipSuccess)
      e = launch_lse_combine(pm, ps, zt, tc, V, logprob + c0, lse_ + c0, cs + c0,
                             rollout_logprob + c0, coef_ + c0, D, ds, g, s);
    if (e == hipSuccess)
      e = launch_select(pm, tc, V, lse_ + c0, zt, target + c0, coef_ + c0, D, ds, g, E, hh, W, H,
                        rec, s);
    if (e == hipSuccess)
      e = launch_dhidden(E, D, ds, g, Wt, W, target + c0, coef_ + c0, tc, H, V, dhidden + c0 * H,
                         s);
    if (e == hipSuccess) e = launch_dh_fix(rec, coef_ + c0, W, tc, H, dhidden + c0 * H, s);
    if (e == hipSuccess && grads)
      e = launch_weight_grads_chunk(E, D, ds, g, coef_ + c0, target + c0, hh, x + c0 * H, eps,
                                    dhidden + c0 * H, tc, H, V, c0 / kTile, c0 == 0,
                                    at<uint16_t>(workspace, L.g_hs), rec,
                                    dw_exact_bufs(at<char>(workspace, L.g_dw), tc, H),
                                    at<double>(workspace, L.g_rbuf),
                                    at<double>(workspace, L.g_part), dW, s);
    if (e == hipSuccess) e = launch_rmsnorm_bwd(x + c0 * H, gamma, eps, tc, H, dhidden + c0 * H, s);
  }
  if (e == hipSuccess)
    e = launch_is_loss(logprob, rollout_logprob, T, resp_offsets, R, group_offsets, G, reward,
                       loss, nullptr, nullptr, part, ok, false, s);
  if (e == hipSuccess) e = launch_d3(logprob, rollout_logprob, T, d3, part, s);
  if (e == hipSuccess && kl) e = launch_kl(logprob, rollout_logprob, T, kl, part, s);
  if (e == hipSuccess && grads)
    e = launch_dgamma_final(at<double>(workspace, L.g_part), ceil_div(T, kTile), H, dgamma, s);
  return status_of(e);
}

}  // extern "C"
