// Rotation of the hidden state into fixed-point digit planes, and the MFMA
// operands of the sketch screen (gfx950). Shared by the per-pair and the
// expert-grouped forward kernels so that both compute identical sketch
// activations.
//
// The rotation is the random-sign Walsh-Hadamard transform the sketch was built
// with (arXiv:2610.37386, abstract; aimodeling.com article, section "A reader
// that needs no data at all": the screen uses a rotated ternary sketch).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "topk.h"

namespace cfm {
namespace {

constexpr int kRotNT = 256;                   // threads of every workgroup that rotates
constexpr int kPlanes = 6;                    // base-16 digit planes of the 24-bit fixed-point x~
constexpr int kDShift = 7;                    // x~ in units of 2^(7 - F0) before the digit split
constexpr int kZeroExp = 255;                 // fixed-point exponent of an all-zero block (any value works)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Buffers of one rotation: xs [max(H, 256)] int32 exchange, limb [kPlanes][Hp]
// digit bytes with Hp = max(H, 256) (both LDS).
struct RotBuf {
  int H, log2H;
  int32_t* xs;
  uint8_t* limb;
};

// Value of lane (lane ^ M): DPP quad permutes for 1 and 2, bank-masked row
// shifts for 4, a row rotation for 8, and the gfx950 row / half swaps for 16
// and 32; all are VALU operations (no LDS traffic).
template <int M>
__device__ __forceinline__ int lane_xor(int v) {
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  else if constexpr (M == 4) {
    const int a = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0x5, false);
    return __builtin_amdgcn_update_dpp(a, v, 0x114, 0xF, 0xA, false);
  } else if constexpr (M == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
  else if constexpr (M == 16) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? (int)s[0] : (int)s[1];
  } else {
    static_assert(M == 32, "lane masks 1..32");
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? (int)s[0] : (int)s[1];
  }
}

// ------------------------------------------------------------------ phase A: rotation and digits
//
// x~ = Hadamard(d . x) in fixed point: X_i = rint(d_i x_i 2^F0) as int32 with
// F0 = 30 - log2 H - E (max |x| < 2^E), so |X~| <= 2^30 and the transform of
// the integers is exact. The digit planes hold the six base-16 digits of
// Y = floor(X~ / 2^7) + 2^23 (0 <= Y < 2^24); the MFMA column of ones gives the
// row sums of the codes, which remove the offset: t . floor(X~ / 2^7) =
// sum_l 16^l D_l - 2^23 D_ones.

// F0 from the largest |x| bit pattern mx of the token (0 for an all-zero row).
__device__ __forceinline__ int exponent_from_max(uint32_t mx, int log2H) {
  if (mx == 0) return kZeroExp;
  const int E = (int)((mx >> 7) & 0xFF) - 126;          // max |x| < 2^E
  return 30 - log2H - E;
}
// The same from this thread's values, over the workgroup (one barrier).
__device__ __forceinline__ int fixed_exponent(uint32_t mx, int log2H, uint32_t* wred) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  mx = wave_max_u32(mx);
  if (lane == 0) wred[wv] = mx;
  __syncthreads();
  const uint4 m4 = *reinterpret_cast<const uint4*>(wred);
  return exponent_from_max(max(max(m4.x, m4.y), max(m4.z, m4.w)), log2H);
}
__device__ __forceinline__ int32_t fix_value(uint32_t xb, int8_t s, int F0) {
  const float f = ldexpf(__uint_as_float(xb << 16), F0);   // exact scaling; |f| < 2^(30 - log2 H)
  const int32_t q = (int32_t)rintf(f);
  return s < 0 ? -q : q;
}

// Writes the digit bytes of Y for EPT consecutive elements starting at i0.
template <int EPT>
__device__ __forceinline__ void put_digit_planes(uint8_t* limb, int Hp, int i0, const int32_t* v) {
  uint32_t y[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) y[q] = (uint32_t)((v[q] >> kDShift) + (1 << 23));
#pragma unroll
  for (int l = 0; l < kPlanes; ++l) {
    uint32_t w[(EPT + 3) / 4];
#pragma unroll
    for (int g = 0; g < (EPT + 3) / 4; ++g) {
      float f[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) f[h] = 4 * g + h < EPT ? (float)((y[4 * g + h] >> (4 * l)) & 15u) : 0.f;
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pk, true);
      w[g] = (uint32_t)pk;
    }
    uint8_t* dst = limb + (size_t)l * Hp + i0;
    if constexpr (EPT == 4) *reinterpret_cast<uint32_t*>(dst) = w[0];
    else if constexpr (EPT == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    else {
#pragma unroll
      for (int g = 0; g < EPT / 16; ++g)
        reinterpret_cast<uint4*>(dst)[g] = make_uint4(w[4 * g], w[4 * g + 1], w[4 * g + 2], w[4 * g + 3]);
    }
  }
}

// Butterfly of one lane stage: partner p, this lane upper (bit set) or lower.
__device__ __forceinline__ int32_t bfly(int32_t v, int32_t p, bool upper) {
  const int32_t m = upper ? -1 : 0;               // p + v (lower lane) or p - v (upper lane)
  return p + (v ^ m) + (m & 1);
}

// x~ for H = 256 EPT with EPT >= 4 (H >= 1024). Thread t holds i = EPT t + q:
// in-register stages for the low log2 EPT bits, VALU lane exchanges for the
// next six, one LDS exchange among the four wavefronts for the top two. Each
// wavefront scales its quarter by its own F0 (no barrier for the scale); at the
// exchange the quarters are brought to the smallest F0 of the four by an exact
// right shift (floor), so the result is X~ for that F0 with each input rounded
// once to its own grid and once more to the common one. xq: this thread's EPT
// BF16 values as loaded (16-byte words; 8 bytes for EPT 4), sq: its EPT signs
// as loaded. Returns the common F0.
template <int EPT>
__device__ __forceinline__ int rotate_fast(const RotBuf& R, const uint4* xq, const uint32_t* sq,
                           int* wf0) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t xb[EPT];
  int8_t sg[EPT];
#pragma unroll
  for (int g = 0; g < (EPT + 7) / 8; ++g) {
    const uint32_t ww[4] = {xq[g].x, xq[g].y, xq[g].z, xq[g].w};
#pragma unroll
    for (int q = 0; q < 8 && 8 * g + q < EPT; ++q) xb[8 * g + q] = (q & 1) ? ww[q >> 1] >> 16 : ww[q >> 1] & 0xFFFFu;
  }
#pragma unroll
  for (int g = 0; g < EPT / 4; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) sg[4 * g + q] = (int8_t)(sq[g] >> (8 * q));
  uint32_t mx = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) mx = max(mx, xb[q] & 0x7FFFu);
  // |partial sums of a quarter| <= 2^(30 - log2 H) H / 4 = 2^28
  const int F0w = exponent_from_max(wave_max_u32(mx), R.log2H);
  int32_t v[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = fix_value(xb[q], sg[q], F0w);
#pragma unroll
  for (int h = 1; h < EPT; h <<= 1)
#pragma unroll
    for (int q = 0; q < EPT; ++q)
      if (!(q & h)) { const int32_t x0 = v[q], x1 = v[q + h]; v[q] = x0 + x1; v[q + h] = x0 - x1; }
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<1>(v[q]), lane & 1);
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<2>(v[q]), lane & 2);
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<4>(v[q]), lane & 4);
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<8>(v[q]), lane & 8);
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<16>(v[q]), lane & 16);
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = bfly(v[q], lane_xor<32>(v[q]), lane & 32);
  // the two wavefront bits: a 4-point Hadamard across the wavefronts
  int32_t* mine = R.xs + EPT * tid;
#pragma unroll
  for (int g = 0; g < EPT / 4; ++g)
    reinterpret_cast<int4*>(mine)[g] = make_int4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
  if (lane == 0) wf0[wv] = F0w;
  __syncthreads();
  const int4 f4 = *reinterpret_cast<const int4*>(wf0);
  const int F0 = min(min(f4.x, f4.y), min(f4.z, f4.w));
  const int fw[4] = {f4.x, f4.y, f4.z, f4.w};
  int32_t acc[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) acc[q] = 0;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const int32_t* src = R.xs + EPT * (64 * w2 + lane);
    const bool neg = __builtin_popcount(w2 & wv) & 1;
    const int sh = min(fw[w2] - F0, 31);
#pragma unroll
    for (int g = 0; g < EPT / 4; ++g) {
      const int4 u = reinterpret_cast<const int4*>(src)[g];
      const int32_t u4[4] = {u.x >> sh, u.y >> sh, u.z >> sh, u.w >> sh};
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[4 * g + q] += neg ? -u4[q] : u4[q];
    }
  }
  put_digit_planes<EPT>(R.limb, R.H, EPT * tid, acc);
  __syncthreads();
  return F0;
}

// x~ for small H (< 1024): LDS butterflies. Digits for i >= H (up to 256) are
// written too; the sketch codes there are zero, so their value does not matter.
__device__ __forceinline__ int rotate_small(const RotBuf& R, const uint16_t* xt, const int8_t* signs, uint32_t* wred) {
  const int tid = threadIdx.x, H = R.H;
  uint32_t mx = 0;
  for (int i = tid; i < H; i += kRotNT) mx = max(mx, (uint32_t)xt[i] & 0x7FFFu);
  const int F0 = fixed_exponent(mx, R.log2H, wred);
  for (int i = tid; i < H; i += kRotNT) R.xs[i] = fix_value(xt[i], signs[i], F0);
  __syncthreads();
  for (int s = 0; s < R.log2H; ++s) {
    const int h = 1 << s;
    for (int b = tid; b < H / 2; b += kRotNT) {
      const int i = ((b >> s) << (s + 1)) | (b & (h - 1));
      const int32_t u = R.xs[i], w = R.xs[i + h];
      R.xs[i] = u + w;
      R.xs[i + h] = u - w;
    }
    __syncthreads();
  }
  const int Hp = max(H, 256);
  for (int i0 = 4 * tid; i0 < Hp; i0 += 4 * kRotNT) {
    int32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = i0 + q < H ? R.xs[i0 + q] : 0;
    put_digit_planes<4>(R.limb, Hp, i0, v);
  }
  __syncthreads();
  return F0;
}

// A operand: sixteen 2-bit codes per 32-bit word become FP4 E2M1 +1 / -1 / 0 by
// masking (the packing puts the nonzero and sign flags of each value at the
// mantissa and sign bits of its nibble). The products use the unscaled
// FP8/FP6/FP4 MFMA (v_mfma_f32_16x16x128_f8f6f4), which the builtin selects when
// both block-scale operands are 0. (The block-scaled form with an explicit 2^0
// scale gave wrong accumulator rows in this kernel.)
__device__ __forceinline__ v8i trit_operand(uint32_t w0, uint32_t w1) {
  constexpr uint32_t M = 0xAAAAAAAAu;
  v8i a;
  a[0] = (int)(w0 & M); a[1] = (int)((w0 << 1) & M);
  a[2] = (int)(w1 & M); a[3] = (int)((w1 << 1) & M);
  a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  return a;
}

}  // namespace
}  // namespace cfm
