// sampler.h -- in-graph temperature sampling for the gfx950 kernels.
//
// The pages keep the sampler inside the decode graph (qwentts.cpp tests-branch
// log, "fused codec mode removed" entry) and decode greedily; the distribution
// here is our definition: for a head's logits l and temperature T > 0 the
// code is argmax_n (l_n * (1/T) + g_n), the lowest index winning ties, where
// g_n = -log(-log(u_n)) is a standard Gumbel variate, so the code is a draw
// from softmax(l / T) (the Gumbel-max rule).  The argmax structure of every
// decode path is unchanged: each score is computed where its logit is.
//
// u_n comes from Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11): the first output word x at counter
// (n, j, q, slot) and key (seed, 0), mapped to ((x >> 11) + 0.5) * 2^-53.
// j: the code's index in its frame (0 = the talker's code); q: the frame's
// talker position (a talker head at position p decides frame p + 1); slot:
// the stream.  g is computed in double and rounded to float once; the scale
// and the sum are single float operations (no fused multiply-add), so the
// score is one exact function of the logit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtk {

__device__ __forceinline__ uint64_t philox4x64_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                     uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  return c0;
}

// Gumbel variate of logit n of code j of frame q, stream slot.
__device__ __forceinline__ float gumbel_noise(uint64_t seed, int slot, int q, int j, int n) {
  const uint64_t x = philox4x64_word0((uint64_t)n, (uint64_t)j, (uint64_t)q, (uint64_t)slot, seed, 0);
  const double u = ((double)(x >> 11) + 0.5) * 0x1p-53;
  return (float)(-log(-log(u)));
}
// Score of logit n of code j of frame q, stream slot: its argmax over n is the
// sampled code.
__device__ __forceinline__ float sample_score(float logit, float inv_temp, uint64_t seed, int slot, int q, int j,
                                              int n) {
  return __fadd_rn(__fmul_rn(logit, inv_temp), gumbel_noise(seed, slot, q, j, n));
}


}  // namespace qtk
