// Small device helpers shared by the kernel translation units.  Where two
// kernels must reproduce each other's values bit for bit (the scaled hidden
// rows of the weight-gradient contraction and its exact correction, the
// exponent shift of the stored e), both call the one definition here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

// The integer log2 reference of a vocabulary tile with max logit M: stored
// values are e = 2^(z log2 e - m), 1/2 < max e <= 1.
__device__ __forceinline__ float tile_ref(float M) { return ceilf(M * kLog2e); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// Sum over a 64-lane wavefront by xor butterfly.  At every level the two
// partners add the same two values (a + b and b + a), so all lanes finish with
// identical bits, and the tree does not depend on where the row sits in the
// batch.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = v + __shfl_xor(v, m, 64);
  return v;
}

// One stored e (bf16 bits) times 2^-d, as the contractions apply it: a
// saturating subtract of d << 7 from the bit pattern (exact for normal
// results; 0 once d reaches the exponent).  dd holds d << 7 in its low 16
// bits (the shift-table format).
__device__ __forceinline__ uint16_t shift_bits(uint16_t e, uint32_t dd) {
  const uint32_t d7 = dd & 0xFFFFu;
  return uint16_t(e > d7 ? e - d7 : 0u);
}

// Element h of the token-contiguous B operand of the weight-gradient
// contraction: bf16(hhat_th * (coef_t * g_t)), the one rounding of the
// per-token factor of p moved onto the hidden row.
__device__ __forceinline__ uint16_t scaled_hidden(float hhat, float coef, float g) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(hhat * (coef * g)));
}

// ---------------------------------------------------------------------------
// Exact correction of the dominant probabilities.  The contractions over the
// vocabulary multiply e rounded to bf16; for a row whose softmax is peaked,
// the rounding of its few large p is not small against the gradient of that
// row (for the sampled token, 1 - p_t).  Per token, the entries with
// p >= kSelTau * (1 - p_t) are candidates; the kSelK largest of them and the
// target (when it qualifies) are recomputed exactly (z in float64 from hhat
// and W) and their contraction terms replaced.
// ---------------------------------------------------------------------------
constexpr int kSelK = 8;                  // dominant entries made exact per token
constexpr int kSelSlots = kSelK + 1;      // + the target
constexpr double kSelTau = 1.0 / 1024.0;  // threshold relative to 1 - p_target

// One exact entry of a token: vocabulary row v (-1: empty slot), its exact
// probability p, pp = the contraction's operand value e 2^-d (exact in
// fp32), and beta = p - g pp, the error of the contraction's p.
struct SelRec {
  int32_t v;
  float p;
  float pp;
  float beta;
};
static_assert(sizeof(SelRec) == 16, "record layout");

}  // namespace rz
