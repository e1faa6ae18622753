// Internal helpers shared by the HIP translation units of libcfm (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <string>

#include "../../include/cfm.h"

namespace cfm {

// ------------------------------------------------------------------ host side

// Records a message for cfm_last_error() and returns `code`.
int set_error(int code, const std::string& msg);
void clear_error();

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
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Agent-scope (all XCDs of the device) completion counter: returns the old value.
// Release orders this block's prior global writes before the increment; acquire
// makes the writes of blocks that incremented earlier visible to the caller.
__device__ __forceinline__ unsigned arrive_counter(unsigned* ctr) {
  return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(unsigned* ctr) {
  __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- block top-k
//
// Selects, among n nonnegative keys held in LDS (key[i] for item i), the k
// items with the largest keys, ties going to the lower index. Writes the
// selected item indices in ascending order to out_idx[0..k). Uses a 4-pass,
// 8-bit radix select to find the k-th key, then an ordered compaction.
// All threads of the block must call it; NT = blockDim.x (a multiple of 64,
// at most 1024). scratch must hold 256 + NT/64 + 8 uint32 words.

template <int NT>
__device__ void block_topk_ascending(const uint32_t* key, int n, int k, int* out_idx,
                                    uint32_t* scratch) {
  uint32_t* hist = scratch;              // 256 bins
  uint32_t* wsum = scratch + 256;        // per-wave partial sums
  uint32_t* sh = scratch + 256 + NT / 64;  // [0]=prefix [1]=remaining k [2]=count > thr
  const int tid = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out_idx[i] = i;
    __syncthreads();
    return;
  }
  if (tid == 0) { sh[0] = 0; sh[1] = (uint32_t)k; }
  uint32_t mask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += NT) hist[b] = 0;
    __syncthreads();
    const uint32_t prefix = sh[0];
    for (int i = tid; i < n; i += NT) {
      uint32_t kv = key[i];
      if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // suffix sums from the top bin down: lane l owns bins 255-4l .. 252-4l
      uint32_t c0 = hist[255 - 4 * tid], c1 = hist[254 - 4 * tid], c2 = hist[253 - 4 * tid],
               c3 = hist[252 - 4 * tid];
      uint32_t tot = c0 + c1 + c2 + c3;
      uint32_t incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_up(incl, o, 64);
        if (tid >= o) incl += v;
      }
      uint32_t before = incl - tot;      // keys in higher bins than this lane's group
      uint32_t need = sh[1];
      // the bin where the running count from the top first reaches `need`
      uint32_t run = before;
      int found = -1;
      uint32_t above = 0;
      uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (found < 0 && run < need && run + cs[q] >= need) { found = 255 - 4 * tid - q; above = run; }
        run += cs[q];
      }
      if (found >= 0) {
        sh[0] = prefix | ((uint32_t)found << shift);
        sh[1] = need - above;
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = sh[0];
  const uint32_t take_eq = sh[1];        // how many keys equal to thr are selected
  // ordered compaction: item i is selected if key > thr, or key == thr and it is
  // among the first take_eq such items in index order.
  const int per = (n + NT - 1) / NT;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    uint32_t kv = key[i];
    ngt += kv > thr;
    neq += kv == thr;
  }
  // block exclusive scans of (neq) then (selected)
  const int lane = tid & 63, wv = tid >> 6;
  uint32_t v = neq;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wv; ++w) base += wsum[w];
  uint32_t eq_before = base + v - neq;
  __syncthreads();
  uint32_t sel_eq = 0;
  if (eq_before < take_eq) sel_eq = min(neq, take_eq - eq_before);
  uint32_t mine = ngt + sel_eq;
  v = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  base = 0;
  for (int w = 0; w < wv; ++w) base += wsum[w];
  uint32_t pos = base + v - mine;
  uint32_t eq_seen = eq_before;
  for (int i = i0; i < i1; ++i) {
    uint32_t kv = key[i];
    bool s = kv > thr;
    if (kv == thr) { s = eq_seen < take_eq; ++eq_seen; }
    if (s) out_idx[pos++] = i;
  }
  __syncthreads();
}

}  // namespace cfm
