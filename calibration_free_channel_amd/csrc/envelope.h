// Decode-layer envelope around the routed-expert block (gfx950): the RMSNorm
// that forms the block's input, the router's softmax top-K, and the helpers
// both forward passes use for them, so that the per-pair and the grouped pass
// form the same bits. The pages measure MoE-block and whole-model decoding
// with routing in place (arXiv:2610.37386, abstract); they do not describe
// these steps, so each follows the plainest reading:
//   x = BF16((h s) g), s = 1 / sqrt(mean(h^2) + eps), one rounding;
//   logits W_r[e] . x from the BF16 x; softmax over all E experts;
//   the K most probable experts in descending probability, lower id first on
//   ties, as the K routing slots; their probabilities as the weights,
//   optionally renormalised to sum 1.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "cfm_internal.h"
#include "topk.h"

namespace cfm {

constexpr int kEnvNT = 256;          // workgroup size of the envelope steps
constexpr int kEnvMaxE = 4 * kEnvNT; // experts the router step handles (4 per thread)

typedef __bf16 env_bf16x2 __attribute__((ext_vector_type(2)));

// Sum over the 64 lanes (DPP row shifts and broadcasts), in every lane.
__device__ __forceinline__ float env_wave_sum(float x) {
  float v = x;
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// acc + the dot product of eight BF16 pairs (float32 accumulation).
__device__ __forceinline__ float env_dot8(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(env_bf16x2, a.x), __builtin_bit_cast(env_bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(env_bf16x2, a.y), __builtin_bit_cast(env_bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(env_bf16x2, a.z), __builtin_bit_cast(env_bf16x2, b.z), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(env_bf16x2, a.w), __builtin_bit_cast(env_bf16x2, b.w), acc, false);
}

// Order-preserving map of a finite float to an unsigned key, and back.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// x = RMSNorm(h) of one token into xb (LDS, BF16 [H]); h: the token's row.
// Whole workgroup; red: 4 floats of LDS scratch; ends with a barrier.
__device__ __forceinline__ void env_normalise(const uint16_t* h, const uint16_t* gamma, int H, float eps,
                                              uint16_t* xb, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nch = H / 8;
  const uint4* hrow = reinterpret_cast<const uint4*>(h);
  const uint4* grow = reinterpret_cast<const uint4*>(gamma);
  float ss = 0.f;
  for (int ci = tid; ci < nch; ci += kEnvNT) {
    const uint4 h4 = hrow[ci];
    const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16lo(hw[i]), hi = bf16hi(hw[i]);
      ss += lo * lo + hi * hi;
    }
  }
  ss = env_wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  const float sc = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int ci = tid; ci < nch; ci += kEnvNT) {
    const uint4 h4 = hrow[ci], g4 = grow[ci];
    const uint32_t hw[4] = {h4.x, h4.y, h4.z, h4.w};
    const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)f32_to_bf16(bf16lo(hw[i]) * sc * bf16lo(gw[i])) |
             ((uint32_t)f32_to_bf16(bf16hi(hw[i]) * sc * bf16hi(gw[i])) << 16);
    reinterpret_cast<uint4*>(xb)[ci] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
}

// One router logit W_r[e] . x by one wavefront: chunks lane, lane + 64, ... in
// order; pre[m] (m < NPRE) may hold chunk lane + 64 m already loaded. In every lane.
template <int NPRE>
__device__ __forceinline__ float env_logit(const uint16_t* wrow, const uint16_t* xb, int H, const uint4 (&pre)[NPRE],
                                           bool use_pre) {
  const int lane = threadIdx.x & 63, nch = H / 8;
  const uint4* row = reinterpret_cast<const uint4*>(wrow);
  const uint4* x4 = reinterpret_cast<const uint4*>(xb);
  float d = 0.f;
#pragma unroll
  for (int m = 0; m < NPRE; ++m) {
    const int ci = lane + 64 * m;
    if (ci < nch) d = env_dot8(use_pre ? pre[m] : row[ci], x4[ci], d);
  }
  for (int ci = lane + 64 * NPRE; ci < nch; ci += 64) d = env_dot8(row[ci], x4[ci], d);
  return env_wave_sum(d);
}

// The routing from the token's E logits, all in rl (LDS; E <= kEnvMaxE,
// K <= 64): the softmax denominator (the largest logit, then the sum of
// exp(l - max) over per-thread ranges and the four wavefronts in a fixed
// order), the K largest logits by block_topk (ascending ids into rida), then
// each one's slot by its rank (descending logit, lower id first on ties).
// Writes the experts to rid and their weights to rw (LDS), renormalised to sum
// 1 if asked. Whole workgroup: joins it before (rl complete) and after.
// red: 8 floats of LDS scratch; rida: K ints; tks: top-k scratch.
__device__ __forceinline__ void env_pick(const float* rl, int E, int K, int renorm, int32_t* rida, int32_t* rid,
                                         float* rw, float* red, uint32_t* tks) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __syncthreads();
  int cnt;
  const int i0 = topk_range<kEnvNT>(E, &cnt);
  float lv[4];
  uint32_t keys[4];
  uint32_t km = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lv[j] = j < cnt ? rl[i0 + j] : 0.f;
    keys[j] = j < cnt ? ordered_key(lv[j]) : 0u;
    km = max(km, keys[j]);
  }
  km = wave_max_u32(km);
  if (lane == 0) reinterpret_cast<uint32_t*>(red)[wv] = km;
  __syncthreads();
  const uint32_t* rk = reinterpret_cast<const uint32_t*>(red);
  const float lmax = key_value(max(max(rk[0], rk[1]), max(rk[2], rk[3])));
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) se += j < cnt ? expf(lv[j] - lmax) : 0.f;
  se = env_wave_sum(se);
  if (lane == 0) red[4 + wv] = se;
  // the K largest logits, ascending ids (ends with a barrier)
  block_topk<kEnvNT, 4>(keys, i0, cnt, E, K, rida, tks);
  const float sum = red[4] + red[5] + red[6] + red[7];
  if (tid < K) {
    const int id = rida[tid];
    const float l = rl[id];
    int rank = 0;
    for (int j = 0; j < K; ++j) {
      const int o = rida[j];
      const float lo = rl[o];
      rank += (lo > l) || (lo == l && o < id);
    }
    rid[rank] = id;
    rw[rank] = expf(l - lmax) / sum;
  }
  __syncthreads();
  if (renorm) {
    float ws = 0.f;
    for (int j = 0; j < K; ++j) ws += rw[j];
    __syncthreads();
    if (tid < K) rw[tid] = rw[tid] / ws;
    __syncthreads();
  }
}

}  // namespace cfm
