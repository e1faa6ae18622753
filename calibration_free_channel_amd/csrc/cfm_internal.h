// Internal helpers shared by the HIP translation units of libcfm (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <initializer_list>
#include <string>

#include "../../include/cfm.h"

namespace cfm {

// ------------------------------------------------------------------ host side

// Records a message for cfm_last_error() and returns `code`.
int set_error(int code, const std::string& msg);
void clear_error();

// Clears the first `bytes` of a forward workspace on `stream` (a fill kernel)
// when its previous call laid it out differently (signature `sig`); the first
// call on a workspace takes it as zero-filled by the caller.
int prepare_workspace(void* ws, size_t bytes, uint64_t sig, hipStream_t stream);
// FNV-1a hash of a plan's layout-determining values.
inline uint64_t layout_signature(std::initializer_list<long> v) {
  uint64_t h = 1469598103934665603ull;
  for (long x : v) {
    for (int b = 0; b < 8; ++b) {
      h ^= (uint64_t)((unsigned long)x >> (8 * b)) & 0xFF;
      h *= 1099511628211ull;
    }
  }
  return h;
}
// Polls of one exchanged value before a single-launch forward pass gives up
// (cfm_set_wait_limit; 0: every wait gives up at once).
unsigned wait_limit();
// Cap on the workgroups a single-launch forward pass may assume resident at
// once (cfm_set_resident_limit; -1: none, the device's own count).
int resident_limit();
// The process-wide forward-pass setting (cfm_set_forward_path).
int forward_path();

// Optional per-kernel event timing (cfm_timing_enable); no-ops while disabled.
bool timing_on();
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);

#define CFM_HIP_TRY(expr)                                                             \
  do {                                                                                \
    hipError_t e_ = (expr);                                                           \
    if (e_ != hipSuccess)                                                             \
      return ::cfm::set_error(CFM_EHIP, std::string(#expr ": ") + hipGetErrorString(e_)); \
  } while (0)

#define CFM_LAUNCH_CHECK(name)                                                        \
  do {                                                                                \
    hipError_t e_ = hipGetLastError();                                                \
    if (e_ != hipSuccess)                                                             \
      return ::cfm::set_error(CFM_EHIP, std::string("launch of " name ": ") + hipGetErrorString(e_)); \
  } while (0)

inline bool is_pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace carve-out helper: hands out 256-byte aligned slices.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

// Largest supported sizes.
constexpr int kMaxH = 8192;
constexpr int kMaxI = 8192;
constexpr int kMaxRank = 128;
constexpr int kMaxK = 64;

// ------------------------------------------------------------------ device side

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> BF16 bits, nearest, ties to even; NaN kept quiet.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Order-preserving key of a nonnegative score: larger score -> larger key; NaN -> 0.
__device__ __forceinline__ uint32_t score_key(float s) {
  float a = fabsf(s);
  return (a != a) ? 0u : __float_as_uint(a);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
}  // namespace cfm
