// Block-wide top-k selection with ties to the lower index (gfx950).
//
// Top-k keeps each token's k highest-scoring channels (arXiv:2610.37386,
// abstract; aimodeling.com article, section "Swapping the threshold for
// top-k"). Keys are the IEEE bit patterns of nonnegative float scores, so
// unsigned order is score order. Every workgroup that selects from the same
// keys returns the same set, in ascending index order.
//
// Method: radix select. Each thread holds its keys in registers (a contiguous
// index range). The first digit is cut from the keys' own range: the smallest
// shift s with (max >> s) - (min >> s) < 256, so the first histogram spreads
// the keys over all 256 bins instead of piling them into the few bins of their
// float exponent (LDS atomics to one address serialise). Each later pass takes
// the next 8 bits below the settled ones and stops as soon as the boundary bin
// is taken whole, or after the last bit; keys equal to the final prefix are
// then taken lowest index first. Three rotating histograms let each pass clear
// the next one, so a pass costs one barrier; every wavefront locates the
// boundary bin itself with one DPP prefix scan, so no second barrier is needed.
// An ordered compaction (one barrier) writes the result.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace cfm {

constexpr int kTopkScratchWords = 4 * 256 + 32;    // three histograms, a dummy row, per-wave words

// Default observer of block_topk's steps (instrumentation builds pass one that
// records a clock stamp): called by every thread after each barrier with the
// step: 0 range known, 1.. histogram passes, 8 ranks known, 9 done.
struct NoStepHook {
  __device__ void operator()(int) const {}
};

// Inclusive prefix sum over the 64 lanes of a wavefront: row shifts by 1..3
// build sums of four, shifts by 4 and 8 (bank-masked) extend them over a row of
// 16, and the row broadcasts of lanes 15 and 31 carry across rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int xi = (int)x;
  int v = xi + __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, xi, 0x113, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xE, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xC, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return (uint32_t)v;
}

// Maximum / minimum over the 64 lanes of a wavefront (the same DPP pattern
// as the scan; lanes outside a shift keep the identity), returned in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));
  v = max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  int v = (int)x;
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x111, 0xF, 0xF, false));
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x112, 0xF, 0xF, false));
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x114, 0xF, 0xF, false));
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x118, 0xF, 0xF, false));
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x142, 0xA, 0xF, false));
  v = min((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(-1, v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// The boundary bin of one pass, found by every lane of a wavefront: h[0..256)
// holds the counts of the keys still in play (a higher bin = larger keys).
// Returns the bin; need becomes the number still to take inside it and *m its
// count.
__device__ __forceinline__ uint32_t boundary_digit(const uint32_t* h, uint32_t& need, uint32_t* m) {
  const int lane = threadIdx.x & 63;
  const uint4 q4 = *reinterpret_cast<const uint4*>(h + 252 - 4 * lane);   // bins 252-4l .. 255-4l
  const uint32_t s = q4.x + q4.y + q4.z + q4.w;
  const uint32_t incl = wave_incl_scan(s);
  const unsigned long long hit = __ballot(incl >= need);
  const int L = __builtin_ffsll((long long)hit) - 1;
  uint32_t run = __builtin_amdgcn_readlane(incl - s, L);      // keys in higher bins
  const uint32_t c0 = __builtin_amdgcn_readlane(q4.w, L);     // bin 255 - 4L
  const uint32_t c1 = __builtin_amdgcn_readlane(q4.z, L);
  const uint32_t c2 = __builtin_amdgcn_readlane(q4.y, L);
  const uint32_t c3 = __builtin_amdgcn_readlane(q4.x, L);
  const uint32_t r1 = run + c0, r2 = r1 + c1, r3 = r2 + c2;
  const uint32_t q = (r1 < need) + (r2 < need) + (r3 < need);   // r1 <= r2 <= r3
  *m = q == 0 ? c0 : q == 1 ? c1 : q == 2 ? c2 : c3;
  run = q == 0 ? run : q == 1 ? r1 : q == 2 ? r2 : r3;
  need -= run;
  return (uint32_t)(255 - 4 * L) - q;
}

// Per-thread key range of an n-key selection: thread t holds indices
// [t per, t per + cnt) with per = ceil(n / NT).
template <int NT>
__device__ __forceinline__ int topk_range(int n, int* cnt) {
  const int per = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * per);
  *cnt = min(n, i0 + per) - i0;
  return i0;
}

// Selects the k largest of n keys by (key desc, index asc) and writes their
// indices in ascending order to out_idx[0..k) (LDS). kr[0..cnt) are this
// thread's keys for indices [i0, i0 + cnt) as given by topk_range (requires
// ceil(n / NT) <= KPT and n < 65536). scratch: kTopkScratchWords words of LDS,
// 16-byte aligned. Called by the whole workgroup; ends with a barrier.
template <int NT, int KPT, typename StepHook = NoStepHook>
__device__ __forceinline__ void block_topk(const uint32_t (&kr)[KPT], int i0, int cnt, int n, int k, int32_t* out_idx,
                           uint32_t* scratch, StepHook step = StepHook());

// The same with the writer of the result given: emit(take, pos, j) is called
// for each of this thread's keys j < KPT (take: key j is selected, at rank pos
// of the ascending result; j >= cnt is never taken), then the workgroup joins.
template <int NT, int KPT, typename Emit, typename StepHook = NoStepHook>
__device__ __forceinline__ void block_topk_emit(const uint32_t (&kr)[KPT], int i0, int cnt, int n, int k, Emit emit,
                                                uint32_t* scratch, StepHook step = StepHook()) {
  static_assert(NT == 256, "four wavefronts");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (k <= 0) return;
  if (k >= n) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) emit(j < cnt, (uint32_t)(i0 + j), j);
    __syncthreads();
    return;
  }
  uint32_t* hist = scratch;
  uint32_t* red = scratch + 4 * 256;       // [0, 8): per-wave min / max; [8, 12): per-wave totals
  // keys beyond this thread's range become a sentinel above every real key
  // (real keys are nonnegative floats, below 2^31), which no pass counts
  uint32_t kk[KPT];
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    kk[j] = j < cnt ? kr[j] : ~0u;
    kmin = min(kmin, kk[j]);
    kmax = max(kmax, j < cnt ? kk[j] : 0u);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) { red[2 * wv] = kmin; red[2 * wv + 1] = kmax; }
  hist[tid] = 0;
  __syncthreads();
  {
    const uint4 a = *reinterpret_cast<const uint4*>(red);
    const uint4 b = *reinterpret_cast<const uint4*>(red + 4);
    kmin = min(min(a.x, a.z), min(b.x, b.z));
    kmax = max(max(a.y, a.w), max(b.y, b.w));
  }
  step(0);
  int s = kmax == kmin ? 0 : max(0, 24 - __builtin_clz(kmax - kmin));
  if ((kmax >> s) - (kmin >> s) > 255u) ++s;
  uint32_t base = kmin >> s;       // digit = (key >> s) - base
  uint32_t lim = (kmax >> s) - base;   // digits in play: 0 .. lim
  int S = 32;                      // settled: (key >> S) == V (nothing settled yet)
  uint32_t V = 0, need = (uint32_t)k, m = 0;
  for (int pass = 0;; ++pass) {
    uint32_t* h = hist + 256 * (pass % 3);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      // a key is in play iff its digit lies in 0..lim (keys with other settled
      // digits, and the sentinel, fall outside); keys out of play add 0 to a
      // bin of their own lane, so they cause no conflicts
      const uint32_t d = (kk[j] >> s) - base;
      const bool in = d <= lim;
      atomicAdd(&h[in ? d : (uint32_t)lane], in ? 1u : 0u);
    }
    hist[256 * ((pass + 1) % 3) + tid] = 0;      // the next pass's histogram
    __syncthreads();
    step(1 + pass);
    V = base + boundary_digit(h, need, &m);
    S = s;
    if (m == need || S == 0) break;
    s = max(S - 8, 0);
    base = V << (S - s);
    lim = (1u << (S - s)) - 1u;
  }
  uint32_t nd = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t v = kk[j] >> S;       // the sentinel is above V: count it, never write it
    nd += v > V;
    ne += v == V;
  }
  nd -= (uint32_t)(KPT - cnt);
  const uint32_t packed = (nd << 16) | ne;
  const uint32_t incl = wave_incl_scan(packed);
  if (lane == 63) red[8 + wv] = incl;
  __syncthreads();
  step(8);
  const uint4 wt = *reinterpret_cast<const uint4*>(red + 8);
  const uint32_t basew = (wv > 0 ? wt.x : 0u) + (wv > 1 ? wt.y : 0u) + (wv > 2 ? wt.z : 0u);
  const uint32_t ex = basew + incl - packed;
  uint32_t d = ex >> 16, e = ex & 0xFFFFu;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t v = kk[j] >> S;
    const bool gt = j < cnt && v > V, eq = v == V;
    const bool take = gt || (eq && e < need);
    const uint32_t pos = gt ? d + min(e, need) : d + e;
    emit(take, pos, j);
    d += gt;
    e += eq;
  }
  __syncthreads();
  step(9);
}

template <int NT, int KPT, typename StepHook>
__device__ __forceinline__ void block_topk(const uint32_t (&kr)[KPT], int i0, int cnt, int n, int k, int32_t* out_idx,
                                           uint32_t* scratch, StepHook step) {
  static_assert(NT == 256, "four wavefronts");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out_idx[i] = i;
    __syncthreads();
    return;
  }
  uint32_t* hist = scratch;
  uint32_t* dummy = scratch + 3 * 256;     // sink for the stores of keys not taken
  uint32_t* red = scratch + 4 * 256;       // [0, 8): per-wave min / max; [8, 12): per-wave totals
  // keys beyond this thread's range become a sentinel above every real key
  // (real keys are nonnegative floats, below 2^31), which no pass counts
  uint32_t kk[KPT];
  uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    kk[j] = j < cnt ? kr[j] : ~0u;
    kmin = min(kmin, kk[j]);
    kmax = max(kmax, j < cnt ? kk[j] : 0u);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) { red[2 * wv] = kmin; red[2 * wv + 1] = kmax; }
  hist[tid] = 0;
  __syncthreads();
  {
    const uint4 a = *reinterpret_cast<const uint4*>(red);
    const uint4 b = *reinterpret_cast<const uint4*>(red + 4);
    kmin = min(min(a.x, a.z), min(b.x, b.z));
    kmax = max(max(a.y, a.w), max(b.y, b.w));
  }
  step(0);
  int s = kmax == kmin ? 0 : max(0, 24 - __builtin_clz(kmax - kmin));
  if ((kmax >> s) - (kmin >> s) > 255u) ++s;
  uint32_t base = kmin >> s;       // digit = (key >> s) - base
  uint32_t lim = (kmax >> s) - base;   // digits in play: 0 .. lim
  int S = 32;                      // settled: (key >> S) == V (nothing settled yet)
  uint32_t V = 0, need = (uint32_t)k, m = 0;
  for (int pass = 0;; ++pass) {
    uint32_t* h = hist + 256 * (pass % 3);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      // a key is in play iff its digit lies in 0..lim (keys with other settled
      // digits, and the sentinel, fall outside); keys out of play add 0 to a
      // bin of their own lane, so they cause no conflicts
      const uint32_t d = (kk[j] >> s) - base;
      const bool in = d <= lim;
      atomicAdd(&h[in ? d : (uint32_t)lane], in ? 1u : 0u);
    }
    hist[256 * ((pass + 1) % 3) + tid] = 0;      // the next pass's histogram
    __syncthreads();
    step(1 + pass);
    V = base + boundary_digit(h, need, &m);
    S = s;
    if (m == need || S == 0) break;
    s = max(S - 8, 0);
    base = V << (S - s);
    lim = (1u << (S - s)) - 1u;
  }
  uint32_t nd = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t v = kk[j] >> S;       // the sentinel is above V: count it, never write it
    nd += v > V;
    ne += v == V;
  }
  nd -= (uint32_t)(KPT - cnt);
  const uint32_t packed = (nd << 16) | ne;
  const uint32_t incl = wave_incl_scan(packed);
  if (lane == 63) red[8 + wv] = incl;
  __syncthreads();
  step(8);
  const uint4 wt = *reinterpret_cast<const uint4*>(red + 8);
  const uint32_t basew = (wv > 0 ? wt.x : 0u) + (wv > 1 ? wt.y : 0u) + (wv > 2 ? wt.z : 0u);
  const uint32_t ex = basew + incl - packed;
  uint32_t d = ex >> 16, e = ex & 0xFFFFu;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t v = kk[j] >> S;
    const bool gt = j < cnt && v > V, eq = v == V;
    const bool take = gt || (eq && e < need);
    const uint32_t pos = gt ? d + min(e, need) : d + e;
    *(take ? reinterpret_cast<uint32_t*>(out_idx) + pos : dummy + tid) = (uint32_t)(i0 + j);
    d += gt;
    e += eq;
  }
  __syncthreads();
  step(9);
}

// The threshold keep rule in place of top-k (abstract: selectors typically
// keep the channels whose score passes a threshold calibrated offline): the
// indices whose key reaches tkey (key >= tkey) are written in ascending order
// to out_idx (LDS); returns how many, in every thread (uniform). key_at(i)
// gives the key of index i; this thread's indices are [i0, i0 + cnt) as given
// by topk_range (read twice: a count, then the writes, so no key is held in
// registers). Scratch as in block_topk (one scan per wavefront, one barrier for
// the per-wave totals). Called by the whole workgroup; ends with a barrier.
template <int NT, typename KeyAt>
__device__ __forceinline__ int block_threshold(KeyAt key_at, int i0, int cnt, uint32_t tkey, int32_t* out_idx,
                                               uint32_t* scratch) {
  static_assert(NT == 256, "four wavefronts");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t* red = scratch + 4 * 256 + 8;
  uint32_t n = 0;
  for (int j = 0; j < cnt; ++j) n += key_at(i0 + j) >= tkey ? 1u : 0u;
  const uint32_t incl = wave_incl_scan(n);
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  const uint4 wt = *reinterpret_cast<const uint4*>(red);
  uint32_t pos = (wv > 0 ? wt.x : 0u) + (wv > 1 ? wt.y : 0u) + (wv > 2 ? wt.z : 0u) + incl - n;
  const int total = __builtin_amdgcn_readfirstlane((int)(wt.x + wt.y + wt.z + wt.w));
  for (int j = 0; j < cnt; ++j)
    if (key_at(i0 + j) >= tkey) out_idx[pos++] = i0 + j;
  __syncthreads();
  return total;
}

}  // namespace cfm
