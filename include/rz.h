/*
 * rz.h -- C ABI of the REINFORCE Zero learner head for AMD MI355X (gfx950).
 *
 * The library computes, for a ragged batch of response tokens:
 *   - per-token log-probabilities of the sampled tokens whose bits do not
 *     depend on how the batch is composed (batch size, a row's offset, a
 *     single-row call versus a large one);
 *   - the unclipped token-level importance-sampled REINFORCE loss and its
 *     gradient with respect to each log-probability;
 *   - the D3 diagnostic;
 *   - the gradient of the loss with respect to the pre-norm hidden states.
 *
 * Sources (web pages describing the method):
 *   [P1] "REINFORCE-Zero: kernel alignment + unclipped IS enables 20K-step
 *        stable async RL", sections "Core insight" and "Results".
 *   [P2] "Zero Mismatch, Simple Async RL: REINFORCE Zero, DeepSeek-V4.1 and
 *        Kimi K3.1", sections "Only one probability gap comes from old
 *        weights" (the log-ratio decomposition equation), "Alignment permits a
 *        simpler learning path", "Large-model validation exposes concrete
 *        failure mechanisms".
 *   [P3] "REINFORCE Zero：为什么内核对齐后，极简 IS 能让异步 RL 稳定训练 20,000 步？",
 *        body text and the captions of Fig. 1 and Fig. 2.
 *
 * Conventions for every entry point:
 *   - Memory: every array pointer is a caller-owned DEVICE pointer on the
 *     current HIP device.  The library never allocates or frees memory; all
 *     scratch comes from the caller's `workspace` (device memory, 256-byte
 *     aligned, at least rz_workspace_bytes(T, H, V) bytes).
 *   - bf16 arrays are passed as uint16_t storage bits.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls
 *     enqueue their kernels and return without synchronising; outputs are
 *     valid once the stream reaches that point.  Calls on one workspace must
 *     be ordered (same stream or explicit events).
 *   - Validation: every check that needs no device data runs on the host
 *     before any HIP call, so argument errors are reported on machines
 *     without a GPU.  Data that lives on the device (targets, offsets) is
 *     not inspected on the host: an out-of-range target yields NaN for that
 *     token's log-probability (and gradient row), and malformed offsets are
 *     detected on the device and yield NaN for the loss and every coef.
 *   - Determinism: outputs are bitwise identical run to run.  Every
 *     floating-point sum runs in a fixed order; the only atomics are integer
 *     counters: the forward's per-XCD tile counters, which decide which
 *     workgroup computes a tile but never how it is computed, and the digit
 *     histograms of the weight gradient's bucketing, whose totals do not
 *     depend on the order (each entry's place in a bucket is fixed by its
 *     token index, not by arrival).
 *   - Layout: row t pairs the final hidden state that predicts target[t] with
 *     that target (the caller applies the next-token shift and drops prompt
 *     tokens).  Tokens of a response are contiguous; the responses of one
 *     prompt group are contiguous.
 *   - Thread safety: no global mutable state apart from the opt-in timing
 *     records of rz_profile_* (process-wide, behind a lock), per-device
 *     values looked up once (the CU count; the address of
 *     rz_logprob_noalloc's scratch) and that scratch itself; concurrent
 *     calls are safe if they use distinct workspaces and outputs (for
 *     rz_logprob_noalloc, see there).
 */
#ifndef RZ_H_
#define RZ_H_

#include <stddef.h>
#include <stdint.h>

/* Only the entry points below are exported from the shared library. */
#if defined(__GNUC__) || defined(__clang__)
#define RZ_API __attribute__((visibility("default")))
#else
#define RZ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RZ_OK 0
#define RZ_EINVAL 1        /* null/misaligned pointer, negative or zero size   */
#define RZ_EUNSUPPORTED 2  /* valid but unsupported shape (see each call)      */
#define RZ_ENODEV 3        /* no HIP device available                          */
#define RZ_EHIP 4          /* a HIP runtime call or kernel launch failed       */
#define RZ_EWORKSPACE 5    /* workspace smaller than rz_workspace_bytes()      */

/* Library version, (major << 16) | (minor << 8) | patch. */
RZ_API int rz_version(void);

/* Static, human-readable text for a status code. */
RZ_API const char* rz_status_string(int status);

/* Workspace size (bytes) that suffices for every entry point below at these
 * sizes.  Returns 0 if the sizes are invalid.  Host only, no HIP call. */
RZ_API size_t rz_workspace_bytes(int64_t T, int32_t H, int32_t V);

/*
 * rz_workspace_bytes_grads -- workspace for rz_learner_step with the weight
 * gradients (dW, dgamma): the above plus one chunk of scaled hidden states
 * (32768 x H bf16), the sort buffers and partial sums of the per-row exact
 * terms, and the dgamma partials (about 200 MB more at H = 1536,
 * V = 151,936 and T = 584,025).
 * 0 for invalid sizes.
 */
RZ_API size_t rz_workspace_bytes_grads(int64_t T, int32_t H, int32_t V);

/*
 * rz_rmsnorm -- the final RMSNorm alone: the first step of rz_logprob.
 *
 * The learner and the rollout must run the same forward computation for a
 * row ([P3] body: batch-invariant kernels and a matching forward pass).  The
 * pages do not print the norm.  This library takes the usual final RMSNorm:
 *   r_t     = (mean_k x_tk^2 + eps)^(-1/2)
 *   hhat_tk = bf16_rne(gamma_k * x_tk * r_t)
 * evaluated in float64 and rounded once to bf16.  hhat has exactly the bits
 * that rz_logprob, rz_backward and rz_learner_step feed to the LM head (the
 * same kernel), and a row's bits depend on that row alone.
 *
 * x [T,H] bf16 row-major; gamma [H] bf16; hhat [T,H] bf16 out; rstd [T] fp32
 * out (r_t rounded to fp32), may be NULL.  x, gamma and hhat 16-byte aligned,
 * rstd 4-byte aligned.  No workspace.
 * Errors: RZ_EINVAL (null pointer, misalignment, T < 1, H < 1, eps negative
 * or NaN), RZ_EUNSUPPORTED (H not a multiple of 64, H > 16384), RZ_ENODEV,
 * RZ_EHIP.
 */
RZ_API int rz_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps,
                      int64_t T, int32_t H, uint16_t* hhat, float* rstd, void* stream);

/*
 * rz_logprob -- batch-invariant learner log-probabilities.
 *
 * Computes, for every row t < T:
 *   hhat_t   = bf16_rne(gamma * x_t * (mean_k x_tk^2 + eps)^(-1/2))
 *   z_tv     = sum_k hhat_tk W_vk          (bf16 MFMA, fp32 accumulation)
 *   lse[t]   = log sum_v exp(z_tv)
 *   logprob[t] = z_{t, target[t]} - lse[t]
 * This is the learner's log pi(y_t | history) of [P2] "Only one probability
 * gap comes from old weights"; its bits must not depend on batch composition
 * so that the kernel-mismatch term of the decomposition is exactly zero
 * ([P2] "Alignment permits a simpler learning path"; [P3] body).
 *
 * Invariance: the bits of logprob[t] and lse[t] depend only on x_t, gamma,
 * eps, W and target[t]: not on T, on t, or on the other rows.  Tile shapes
 * and the vocabulary reduction order depend on (H, V) only.
 *
 * x [T,H] bf16 row-major; gamma [H] bf16; W [V,H] bf16 row-major; target [T]
 * int32 in [0, V) (out of range -> NaN logprob); logprob [T] fp32 out;
 * lse [T] fp32 out, may be NULL.  All pointers 16-byte aligned.
 * Errors: RZ_EINVAL (null pointer, T < 1, H < 1, V < 1, misalignment),
 * RZ_EUNSUPPORTED (H not a multiple of 64, H > 16384, V > 4000000),
 * RZ_EWORKSPACE, RZ_ENODEV, RZ_EHIP.
 */
RZ_API int rz_logprob(const uint16_t* x, const uint16_t* gamma, float eps,
               const uint16_t* W, const int32_t* target,
               int64_t T, int32_t H, int32_t V,
               float* logprob, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_logprob_noalloc -- rz_logprob for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It takes no workspace and allocates nothing: its
 * scratch is a built-in device array of RZ_NOALLOC_SCRATCH_BYTES that each
 * GPU the library runs on holds until the process ends (its address is
 * looked up on the first call on each device).  The results are those of
 * rz_logprob, bit for bit (same kernels, same invariance).
 *
 * Limit: the call's scratch, the rz_logprob part of rz_workspace_bytes (the
 * normalised rows and per-tile partials of one chunk of at most 32,768
 * tokens), must fit: about 8,500 tokens at H = 1536 and V = 151,936; larger
 * calls return RZ_EWORKSPACE before any HIP call.  Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 *
 * Arguments and other errors as rz_logprob.
 */
#define RZ_NOALLOC_SCRATCH_BYTES (64u << 20)
RZ_API int rz_logprob_noalloc(const uint16_t* x, const uint16_t* gamma, float eps,
                              const uint16_t* W, const int32_t* target,
                              int64_t T, int32_t H, int32_t V,
                              float* logprob, float* lse, void* stream);

/*
 * rz_is_loss -- unclipped token-level IS REINFORCE loss and its gradient.
 *
 * ([P2] "Alignment permits a simpler learning path": advantage = reward minus
 *  the group mean, tokens averaged within each response, no value model, no
 *  rejection gate; [P1] lede and [P3] body: unclipped token-level IS with
 *  w = exp(log pi - log mu).)
 *   A_i     = reward[i] - mean_{j in group(i)} reward[j]
 *   w_t     = exp(logprob[t] - rollout_logprob[t])            (no clip)
 *   loss    = -(1/R) sum_i A_i (1/L_i) sum_{t in i} w_t
 *   coef[t] = d loss / d logprob[t] = -A_i w_t / (R L_i)
 * Sums are accumulated in fp64 in a fixed order.
 *
 * logprob, rollout_logprob [T] fp32; resp_offsets [R+1] int64 token offsets
 * (resp_offsets[0] = 0, resp_offsets[R] = T, strictly increasing);
 * group_offsets [G+1] int64 response offsets of the prompt groups
 * (group_offsets[0] = 0, group_offsets[G] = R, strictly increasing);
 * reward [R] fp32.  Outputs: loss [1] fp64; coef [T] fp32 (may be NULL);
 * advantage [R] fp32 (may be NULL).  Offsets are read on the device and
 * checked there first: a malformed structure (offsets that do not start at
 * 0, do not end at T or R, or do not strictly increase) writes NaN to loss,
 * to every coef and to every advantage; no out-of-bounds access happens.
 * Errors: RZ_EINVAL (null pointer, T < 1, R < 1, G < 1, R > T, G > R),
 * RZ_EWORKSPACE, RZ_ENODEV, RZ_EHIP.
 */
/*
 * Vocabulary splits -- rz_logprob's log-sum-exp is combined in two fixed
 * levels: over the 256-row vocabulary tiles of each of RZ_VOCAB_SPLITS
 * splits, then over the splits, each in order.  Split s covers the tiles
 * [s n / RZ_VOCAB_SPLITS, (s+1) n / RZ_VOCAB_SPLITS), n = ceil(V / 256): a
 * function of V alone.  A device that holds the rows of any whole number of
 * consecutive splits of W can therefore produce those splits' partials
 * (rz_logprob_shard), and the merge of all splits (rz_logprob_merge) gives
 * logprob and lse bit for bit equal to rz_logprob's, whatever the number of
 * devices the vocabulary was spread over (1, 2, 4 or 8 equal shares).  This
 * is the fixed-order reduction that keeps a vocabulary-parallel head at zero
 * difference across device counts ([P2] "Large-model validation exposes
 * concrete failure mechanisms": zero difference on a multi-node run, with
 * arrival-ordered reductions named as a source of batch variance).
 */
#define RZ_VOCAB_SPLITS 8

/* One row's partial of one split (24 bytes, 8-byte aligned). */
typedef struct rz_vocab_split {
  double s;          /* sum over the split's tiles j of S_j 2^(m_j - m), in tile order */
  float m;           /* the split's reference exponent max_j m_j (integer-valued; -inf if empty) */
  float max_logit;   /* max over the split's rows of z_tv (-inf if empty) */
  float z_target;    /* z_{t, target[t]} if target[t] lies in the split, else 0 */
  float reserved;    /* 0 */
} rz_vocab_split;
/* (S_j = sum over tile j's rows of 2^(z_tv log2 e - m_j), m_j =
 *  ceil(max_v z_tv log2 e), both computed as in rz_logprob.) */

/*
 * rz_vocab_split_begin -- first vocabulary row of split s (0 <= s <=
 * RZ_VOCAB_SPLITS; s = RZ_VOCAB_SPLITS gives V).  The rows of splits
 * [s0, s1) are [rz_vocab_split_begin(V, s0), rz_vocab_split_begin(V, s1)).
 * Returns -1 for V < 1, V > 4000000 or s out of range.  Host only.
 */
RZ_API int64_t rz_vocab_split_begin(int32_t V, int32_t s);

/*
 * rz_logprob_shard -- the partials of splits [s0, s1) of every row.
 *
 * W_rows points at row rz_vocab_split_begin(V, s0) of the [V,H] weight and
 * holds the rows of splits s0 .. s1-1 (row-major, as in W).  x, gamma, eps,
 * target (global row indices), T, H, V as for rz_logprob.  partials
 * [(s1 - s0), T] out: partials[(s - s0) * T + t] is split s's record of row
 * t.  workspace as rz_logprob (rz_workspace_bytes(T, H, V)).
 * Errors: RZ_EINVAL (null pointer, misalignment, not 0 <= s0 < s1 <=
 * RZ_VOCAB_SPLITS), and those of rz_logprob.
 */
RZ_API int rz_logprob_shard(const uint16_t* x, const uint16_t* gamma, float eps,
                            const uint16_t* W_rows, const int32_t* target,
                            int64_t T, int32_t H, int32_t V, int32_t s0, int32_t s1,
                            rz_vocab_split* partials,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_logprob_merge -- logprob and lse from the records of all splits.
 *
 * partials [RZ_VOCAB_SPLITS, T] (split-major, as rz_logprob_shard writes
 * them: the blocks of consecutive shards simply follow each other); target
 * [T] int32 (a target outside [0, V) gives NaN, as in rz_logprob); logprob
 * [T] fp32 out; lse [T] fp32 out, may be NULL.  With m = max_s m_s:
 *   lse = max(m ln 2 + log sum_s s_s 2^(m_s - m), max_s max_logit_s)
 * in fp64 and split order; logprob = sum_s z_target_s - lse.  Needs no
 * workspace.
 * Errors: RZ_EINVAL (null pointer, misalignment, T < 1, V < 1,
 * V > 4000000), RZ_ENODEV, RZ_EHIP.
 */
RZ_API int rz_logprob_merge(const rz_vocab_split* partials, const int32_t* target,
                            int64_t T, int32_t V, float* logprob, float* lse, void* stream);

RZ_API int rz_is_loss(const float* logprob, const float* rollout_logprob, int64_t T,
               const int64_t* resp_offsets, int32_t R,
               const int64_t* group_offsets, int32_t G,
               const float* reward,
               double* loss, float* coef, float* advantage,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_d3 -- the D3 diagnostic ([P2] "Only one probability gap comes from old
 * weights": the per-update token mean of w - 1 - log w; [P3] Fig. 2 caption:
 * a batch average).  With delta = logprob - rollout_logprob,
 *   d3 = (1/T) sum_t (expm1(delta_t) - delta_t),   fp64, fixed order.
 * Output d3 [1] fp64.
 * Errors: RZ_EINVAL (null pointer, T < 1), RZ_EWORKSPACE, RZ_ENODEV, RZ_EHIP.
 */
RZ_API int rz_d3(const float* logprob, const float* rollout_logprob, int64_t T,
          double* d3, void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_kl -- sample estimates of the rollout-to-learner KL, KL(mu || pi), over
 * the tokens of one update ([P3] Fig. 1 caption: a KL estimated from the
 * rollout's samples; the pages name no estimator).  With delta = logprob -
 * rollout_logprob:
 *   kl[0] = k1 = (1/T) sum_t (-delta_t),
 *   kl[1] = k2 = (1/T) sum_t delta_t^2 / 2,
 *   kl[2] = k3 = (1/T) sum_t (expm1(delta_t) - delta_t)   (= rz_d3's value,
 *                                                           bit for bit),
 * fp64 with a fixed order.  k1 and k3 are unbiased for KL(mu || pi) when the
 * tokens were drawn from mu.  Output kl [3] fp64 (device).
 * Errors: RZ_EINVAL (null pointer, T < 1), RZ_EWORKSPACE, RZ_ENODEV, RZ_EHIP.
 */
RZ_API int rz_kl(const float* logprob, const float* rollout_logprob, int64_t T,
          double* kl, void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_decompose -- the log-ratio decomposition of [P2] "Only one probability
 * gap comes from old weights", token by token:
 *   log pi_new - log mu = (log pi_new - log pi_old) + (log pi_old - log mu),
 * lag[t] = the first term (weight lag), mismatch[t] = the second (kernel
 * mismatch): pi_new and pi_old are this library's log-probabilities at the
 * learner's current head (x_new, gamma_new, W_new) and at the rollout's
 * (x_old, gamma_old, W_old), for the same targets, and mu is what the rollout
 * recorded.  When mu came from this library's rz_logprob at the rollout's
 * weights, in any batching, the mismatch is exactly 0 for every token (the
 * pages' claim, checked token by token).
 * Each difference is exact in fp64 and rounded once to fp32.
 * summary [4] fp64: max |lag|, mean lag, max |mismatch|, and the number of
 * tokens whose mismatch is not exactly 0 (NaN counts).
 * x_*, gamma_*, W_*, eps, target, T, H, V as for rz_logprob (both versions
 * share the shape); rollout_logprob [T] fp32; lag, mismatch [T] fp32 out
 * (distinct, and distinct from rollout_logprob); workspace as rz_logprob.
 * Errors: as rz_logprob.
 */
RZ_API int rz_decompose(const uint16_t* x_new, const uint16_t* gamma_new, const uint16_t* W_new,
                 const uint16_t* x_old, const uint16_t* gamma_old, const uint16_t* W_old,
                 float eps, const int32_t* target, const float* rollout_logprob,
                 int64_t T, int32_t H, int32_t V,
                 float* lag, float* mismatch, double* summary,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_backward -- gradient of the loss with respect to the pre-norm hidden
 * states, given lse (from rz_logprob) and coef (from rz_is_loss).
 *
 * With p_tv = exp(z_tv - lse_t), the logit gradient is coef_t (onehot - p)
 * and
 *   dhhat_t = coef_t * (W[target_t] - sum_v p_tv W_v)
 * (the one-hot term is gathered exactly in fp32; the logits are recomputed
 * and stored as e = 2^(z log2 e - m_j) in bf16 with m_j an integer reference
 * per 256-wide vocabulary tile, then contracted with W on bf16 MFMA with fp32
 * accumulation in a fixed vocabulary order, p = e 2^(m_j - m) exp(m ln 2 -
 * lse) being applied as an exact exponent shift of e inside the contraction
 * and a per-token factor after it).  The row's dominant probabilities are
 * then made exact: with p_t the target's, the target and the 8 largest p_tv
 * that reach 2^-10 (1 - p_t) have z recomputed in fp64 from hhat and W, and
 * their bf16 terms in the contraction are replaced by the exact ones, so a
 * row whose softmax is peaked (a token sampled from the policy itself) keeps
 * the accuracy of a flat one.  The RMSNorm backward follows in fp64/fp32, the
 * bf16 rounding of hhat being treated as the identity:
 *   dx_j = r gamma_j g_j - x_j r^3 (1/H) sum_k gamma_k g_k x_k.
 *
 * x, gamma, eps, W, target as for rz_logprob; lse, coef [T] fp32;
 * dhidden [T,H] fp32 out.  Given the lse and coef that rz_learner_step
 * hands out, dhidden is bit-identical to that call's.
 * Errors: as rz_logprob.
 */
RZ_API int rz_backward(const uint16_t* x, const uint16_t* gamma, float eps,
                const uint16_t* W, const int32_t* target,
                const float* lse, const float* coef,
                int64_t T, int32_t H, int32_t V,
                float* dhidden,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stored logits (the same gradient of the loss, [P2] "Alignment permits a
 * simpler learning path"; the same forward, [P3] body): rz_logprob_store is
 * rz_logprob that also keeps, in a caller-owned buffer `logits`, what
 * rz_backward needs from the forward --
 * the values e of every logit (bf16, relative to their vocabulary tile's
 * integer reference), the tile maxima and the target logits -- and
 * rz_backward_stored is rz_backward that takes them from there instead of
 * recomputing the logits: 2 H V flops per token instead of 4 for the two
 * calls after the forward.  Each e is relative to its tile's own reference,
 * which is known as soon as the tile is computed, so the forward can store
 * it before the row's log-sum-exp exists; the backward turns e into the
 * probabilities with exponent shifts it derives from lse.  The buffer takes
 * about T * V * 2 bytes (181 GB, 168 GiB, at T = 584,025, V = 151,936):
 * the caller decides whether that fits beside everything else.
 *
 * rz_logits_bytes -- size of `logits` for these sizes; 0 if invalid.  Host
 * only, no HIP call.
 */
RZ_API size_t rz_logits_bytes(int64_t T, int32_t H, int32_t V);

/*
 * rz_logprob_store -- rz_logprob (same arguments, same logprob and lse bits)
 * that also fills `logits` (device memory, 256-byte aligned, at least
 * rz_logits_bytes(T, H, V) bytes, owned by the caller; RZ_EWORKSPACE if
 * smaller).  Its contents are only meaningful to rz_backward_stored with the
 * same x, gamma, eps, W, target and sizes.
 */
RZ_API int rz_logprob_store(const uint16_t* x, const uint16_t* gamma, float eps,
                const uint16_t* W, const int32_t* target,
                int64_t T, int32_t H, int32_t V,
                float* logprob, float* lse,
                void* logits, size_t logits_bytes,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_backward_stored -- rz_backward (same arguments) with the logits that
 * rz_logprob_store kept for the same inputs: its dhidden is bit-identical
 * to rz_backward's.  Errors: as rz_backward; RZ_EWORKSPACE if logits_bytes
 * is below rz_logits_bytes(T, H, V).
 */
RZ_API int rz_backward_stored(const uint16_t* x, const uint16_t* gamma, float eps,
                const uint16_t* W, const int32_t* target,
                const float* lse, const float* coef,
                int64_t T, int32_t H, int32_t V,
                const void* logits, size_t logits_bytes,
                float* dhidden,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_backward_grads -- rz_backward (logits NULL: the logits are recomputed)
 * or rz_backward_stored (logits from rz_logprob_store) that also gives the
 * gradients of the same objective with respect to the LM-head weight and
 * the RMSNorm weight ([P2] "Alignment permits a simpler learning path": the
 * update applies the loss gradient to all weights):
 *   dW[v, k]  = sum_t coef_t (onehot_t - p_t)[v] hhat[t, k],
 *   dgamma[k] = sum_t dhhat[t, k] x[t, k] r_t,
 * with the kernels and orders of rz_learner_step's weight gradients (sorted
 * one-hot and exact-probability terms, dW summed over 32768-row chunks in
 * order, dgamma in float64).  coef is any per-token weight: the gradient of
 * sum_t coef_t logprob_t, so a caller's own loss goes through it.  With the
 * lse and coef that rz_learner_step hands out, dhidden, dW and dgamma equal
 * that call's bit for bit.
 *
 * dW [V,H] fp32 (16-byte aligned) and dgamma [H] fp32 out, overwritten;
 * workspace of at least rz_workspace_bytes_grads(T, H, V) bytes.  Errors: as
 * rz_backward and rz_backward_stored; RZ_EINVAL without dW or dgamma.
 */
RZ_API int rz_backward_grads(const uint16_t* x, const uint16_t* gamma, float eps,
                const uint16_t* W, const int32_t* target,
                const float* lse, const float* coef,
                int64_t T, int32_t H, int32_t V,
                const void* logits, size_t logits_bytes,
                float* dhidden, float* dW, float* dgamma,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * rz_learner_step -- the whole learner head for one update in one call:
 * rz_logprob, rz_is_loss, rz_d3 and the gradient to the hidden states, with
 * the log-probabilities bit-identical to rz_logprob's.
 *
 * The batch is processed in chunks of at most 32768 tokens.  Per chunk: the
 * forward stores e (bf16, as in rz_backward) for every logit while it forms
 * the log-sum-exp, coef_t = -A_i w_t / (R L_i) is formed as soon as the
 * chunk's log-probabilities exist (it needs only the token's own w_t and the
 * response metadata), e is contracted with W with the shift to
 * p = exp(z - lse) applied inside the contraction (dhhat = coef (W[target] -
 * p W)), and the RMSNorm backward follows.  The logits are therefore
 * computed once per step, not twice as in rz_logprob + rz_backward.
 *
 * Arguments as for rz_logprob, rz_is_loss, rz_d3 and rz_backward.  Outputs:
 * logprob [T] fp32; lse [T] fp32 (may be NULL); loss [1] fp64; d3 [1] fp64;
 * kl [3] fp64 (may be NULL; as rz_kl); coef [T] fp32 (may be NULL);
 * dhidden [T,H] fp32.
 *
 * Weight gradients (dW and dgamma both given, or both NULL): the rest of the
 * head's backward, the gradient of the same loss with respect to the LM-head
 * weight and the RMSNorm weight ([P2] "Alignment permits a simpler learning
 * path": the update applies the loss gradient to the weights):
 *   dW[v] = sum_t coef_t (onehot(target_t)_v - p_tv) hhat_t      [V,H] fp32
 *   dgamma[k] = sum_t dhhat_tk x_tk r_t                          [H] fp32
 * (the bf16 rounding of hhat is straight-through).  The softmax part is
 * contracted on bf16 MFMA from coef_t p_tv rounded once to bf16, fp32
 * accumulation, chunks added in order; the one-hot part and the exact terms
 * of each token's dominant probabilities (those of rz_backward) are added in
 * fp32, per vocabulary row in token order; dgamma is summed in float64 in a
 * fixed order.  Deterministic run to run.  dW must be 16-byte aligned.  They
 * need the larger workspace of rz_workspace_bytes_grads.
 * A malformed response structure gives NaN for the loss, every coef, every
 * dhidden row and the weight gradients; logprob, lse, d3 and kl do not
 * depend on it.
 * Errors: the union of those of rz_logprob and rz_is_loss; RZ_EINVAL also for
 * exactly one of dW, dgamma NULL.
 */
RZ_API int rz_learner_step(const uint16_t* x, const uint16_t* gamma, float eps,
                    const uint16_t* W, const int32_t* target,
                    const float* rollout_logprob, int64_t T, int32_t H, int32_t V,
                    const int64_t* resp_offsets, int32_t R,
                    const int64_t* group_offsets, int32_t G,
                    const float* reward,
                    float* logprob, float* lse, double* loss, double* d3, double* kl,
                    float* coef, float* dhidden, float* dW, float* dgamma,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing, for benchmarks (not for the caller's hot loop).
 *
 * rz_profile_enable(1) clears earlier records and starts recording: every
 * kernel launch of the library is bracketed by two hipEvents recorded on the
 * stream the kernel is launched on; rz_profile_enable(0) stops recording (and
 * also clears).  rz_profile_count() waits for the recorded events, aggregates
 * them by kernel name and returns the number of names (or -RZ_EHIP);
 * rz_profile_get(i, ...) then returns name i (a library-owned string valid
 * until the next rz_profile_* call), its summed duration in milliseconds and
 * its launch count.  Recording creates host-side event objects; it takes a
 * process-wide lock, so concurrent callers serialise while it is on.
 */
RZ_API int rz_profile_enable(int on);
RZ_API int rz_profile_count(void);
RZ_API int rz_profile_get(int i, const char** name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* RZ_H_ */
