// Rotated ternary sketch of W_gate / W_up rows (offline, once per layer).
//
// Method: the per-expert sketch of the gate and up projections that screens
// candidate channels (arXiv:2610.37386 abstract; aimodeling.com article,
// section "A reader that needs no data at all"). The rotation is a random-sign
// Walsh-Hadamard transform (unnormalised, natural order); the ternary rule is
// Ternary Weight Networks (threshold 0.7 * mean |w~|, least-squares scale).
//
// One workgroup per row. The row is rotated in float64 in LDS: every partial
// sum of a BF16 row is exact in float64 unless the row's magnitudes span more
// than about 2^33, so the rotated values do not depend on summation order.
// FP contraction is off in this file: the threshold and scale follow the
// stated expressions operation by operation.
#pragma clang fp contract(off)

#include "cfm_internal.h"
#include "cfm_launch.h"

namespace cfm {
namespace {

constexpr int kSketchThreads = 256;

__device__ double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kSketchThreads / 64; ++w) s += red[w];
  return s;
}

__device__ int block_sum_i(int v, double* red) {
  return static_cast<int>(block_sum_d(static_cast<double>(v), red));
}

__global__ __launch_bounds__(kSketchThreads) void k_sketch_rows(
    const uint16_t* __restrict__ w_gate, const uint16_t* __restrict__ w_up, int rows_per_mat,
    int H, int log2H, const int8_t* __restrict__ signs, uint8_t* __restrict__ tg,
    uint8_t* __restrict__ tu, float* __restrict__ sg, float* __restrict__ su) {
  extern __shared__ double v[];          // H values
  __shared__ double red[kSketchThreads / 64];
  const int tid = threadIdx.x;
  const long row = blockIdx.x;
  const bool up = row >= rows_per_mat;
  const long r = up ? row - rows_per_mat : row;
  const uint16_t* src = (up ? w_up : w_gate) + r * H;

  for (int i = tid; i < H; i += kSketchThreads)
    v[i] = static_cast<double>(bf16_to_f32(src[i])) * static_cast<double>(signs[i]);
  __syncthreads();

  // in-place fast Walsh-Hadamard transform (natural / Sylvester order)
  for (int s = 0; s < log2H; ++s) {
    const int h = 1 << s;
    for (int b = tid; b < H / 2; b += kSketchThreads) {
      const int i = ((b >> s) << (s + 1)) | (b & (h - 1));
      const double a = v[i], c = v[i + h];
      v[i] = a + c;
      v[i + h] = a - c;
    }
    __syncthreads();
  }

  double s1 = 0.0;
  for (int i = tid; i < H; i += kSketchThreads) s1 += fabs(v[i]);
  s1 = block_sum_d(s1, red);
  const double mean_abs = s1 / static_cast<double>(H);
  const double delta = 0.7 * mean_abs;

  double s2 = 0.0;
  int nnz = 0;
  for (int i = tid; i < H; i += kSketchThreads) {
    const double a = fabs(v[i]);
    if (v[i] > delta || v[i] < -delta) { s2 += a; ++nnz; }
  }
  s2 = block_sum_d(s2, red);
  nnz = block_sum_i(nnz, red);
  const double alpha = nnz > 0 ? s2 / static_cast<double>(nnz) : 0.0;
  if (tid == 0) (up ? su : sg)[r] = static_cast<float>(alpha / static_cast<double>(H));

  // pack: one 32-bit word per 16 values
  uint32_t* dst = reinterpret_cast<uint32_t*>((up ? tu : tg) + r * (H / 4));
  for (int b = tid; b < H / 16; b += kSketchThreads) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const double lo = v[16 * b + q], hi = v[16 * b + 8 + q];
      const uint32_t nz_lo = (lo > delta || lo < -delta), neg_lo = lo < -delta;
      const uint32_t nz_hi = (hi > delta || hi < -delta), neg_hi = hi < -delta;
      word |= (nz_hi << (4 * q)) | (nz_lo << (4 * q + 1)) | (neg_hi << (4 * q + 2)) |
              (neg_lo << (4 * q + 3));
    }
    dst[b] = word;
  }
}

// The layer's rotation signs from a seed: d_i = +1 if bit 63 of the i-th output
// of SplitMix64 started at `seed` is 0, else -1. SplitMix64 (Steele, Lea and
// Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014): the
// state advances by the golden-ratio constant and each output is the state
// after two xor-shift-multiply rounds and a final xor-shift, so output i
// depends only on seed + (i + 1) * gamma (counter-based).
__global__ void k_rotation_signs(uint64_t seed, int H, int8_t* __restrict__ signs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H) return;
  uint64_t z = seed + (uint64_t)(i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  signs[i] = (z >> 63) ? (int8_t)-1 : (int8_t)1;
}

}  // namespace

int launch_rotation_signs(uint64_t seed, int H, int8_t* signs, hipStream_t stream) {
  hipLaunchKernelGGL(k_rotation_signs, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, stream, seed, H, signs);
  CFM_LAUNCH_CHECK("k_rotation_signs");
  return CFM_OK;
}

int launch_sketch_build(const uint16_t* w_gate, const uint16_t* w_up, int E, int I, int H,
                        const int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su,
                        hipStream_t stream) {
  const long rows = static_cast<long>(E) * I;
  int log2H = 0;
  while ((1 << log2H) < H) ++log2H;
  const size_t lds = static_cast<size_t>(H) * sizeof(double);
  if (lds > 65536)
    CFM_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sketch_rows),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL(k_sketch_rows, dim3(static_cast<unsigned>(2 * rows)), dim3(kSketchThreads),
                     lds, stream, w_gate, w_up, static_cast<int>(rows), H, log2H, signs, tg, tu,
                     sg, su);
  CFM_LAUNCH_CHECK("k_sketch_rows");
  return CFM_OK;
}

}  // namespace cfm
