// Block-wide top-k selection with ties to the lower index (gfx950).
//
// Top-k keeps each token's k highest-scoring channels (arXiv:2610.37386,
// abstract). Keys are the IEEE bit patterns of nonnegative float scores, so
// unsigned order is score order. Every workgroup that selects from the same
// keys returns the same set.
//
// Method: a 2048-bin histogram of the top 12 key bits (sign, exponent and three
// mantissa bits) finds the bin that holds the k-th largest key; keys above it
// are taken, keys below it dropped, and the keys inside it (few, since scores
// spread over many bins) are ranked exactly by (key desc, index asc). If that
// bin holds more than kListMax keys, a 4-pass 8-bit radix select settles it.
// The selected indices are written in ascending order.
#pragma once

#include "cfm_internal.h"

namespace cfm {

constexpr int kHistBins = 2048;
constexpr int kListMax = 256;

struct TopkScratch {
  uint32_t* hist;      // [kHistBins]
  uint8_t* flag;       // [n] selected flags
  uint32_t* lkey;      // [kListMax]
  int32_t* lidx;       // [kListMax]
  uint32_t* misc;      // [16 + NT/64]
};

__host__ __device__ constexpr size_t topk_scratch_bytes(int n, int nt) {
  return 4ull * kHistBins + ((size_t(n) + 15) & ~size_t(15)) + 8ull * kListMax + 4ull * (16 + nt / 64) + 64;
}

// Block exclusive scan of one uint32 per thread; returns the exclusive prefix
// and writes the block total to *total. Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t s = wsum[w];
    if (w < wv) base += s;
    tot += s;
  }
  *total = tot;
  __syncthreads();
  return base + incl - v;
}

template <int NT>
__device__ void block_topk(const uint32_t* key, int n, int k, int32_t* out_idx, const TopkScratch& s,
                           uint32_t* radix_scratch) {
  const int tid = threadIdx.x;
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += NT) out_idx[i] = i;
    __syncthreads();
    return;
  }
  uint32_t* wsum = s.misc + 16;
  // 1. histogram of the top 12 bits
  for (int b = tid; b < kHistBins; b += NT) s.hist[b] = 0;
  if (tid == 0) s.misc[2] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += NT) atomicAdd(&s.hist[key[i] >> 20], 1u);
  __syncthreads();
  // 2. the bin of the k-th largest key: thread t owns bins counted from the top
  constexpr int BPT = kHistBins / NT;
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < BPT; ++u) cnt += s.hist[kHistBins - 1 - (tid * BPT + u)];
  uint32_t total;
  const uint32_t before = block_excl_scan<NT>(cnt, wsum, &total);
  if (before < (uint32_t)k && before + cnt >= (uint32_t)k) {
    uint32_t run = before;
    for (int u = 0; u < BPT; ++u) {
      const int b = kHistBins - 1 - (tid * BPT + u);
      const uint32_t h = s.hist[b];
      if (run + h >= (uint32_t)k) { s.misc[0] = (uint32_t)b; s.misc[1] = run; break; }
      run += h;
    }
  }
  __syncthreads();
  const uint32_t bstar = s.misc[0];
  const uint32_t need = (uint32_t)k - s.misc[1];
  const uint32_t m = s.hist[bstar];
  if (m > (uint32_t)kListMax && need != m) {
    block_topk_ascending<NT>(key, n, k, out_idx, radix_scratch);
    return;
  }
  // 3. flags: above the bin -> taken; inside it -> taken when all of it is needed,
  //    otherwise collected for exact ranking
  for (int i = tid; i < n; i += NT) {
    const uint32_t b = key[i] >> 20;
    uint8_t f = b > bstar ? 1 : 0;
    if (b == bstar) {
      if (need == m) {
        f = 1;
      } else {
        const uint32_t slot = atomicAdd(&s.misc[2], 1u);
        s.lkey[slot] = key[i];
        s.lidx[slot] = i;
      }
    }
    s.flag[i] = f;
  }
  __syncthreads();
  if (need != m) {
    for (int j = tid; j < (int)m; j += NT) {
      const uint32_t kj = s.lkey[j];
      const int ij = s.lidx[j];
      uint32_t rank = 0;
      for (int q = 0; q < (int)m; ++q) {
        const uint32_t kq = s.lkey[q];
        rank += (kq > kj) || (kq == kj && s.lidx[q] < ij);
      }
      if (rank < need) s.flag[ij] = 1;
    }
    __syncthreads();
  }
  // 4. ordered compaction over contiguous index ranges
  const int per = (n + NT - 1) / NT;
  const int i0 = tid * per, i1 = min(n, i0 + per);
  uint32_t c = 0;
  for (int i = i0; i < i1; ++i) c += s.flag[i];
  uint32_t tot;
  uint32_t pos = block_excl_scan<NT>(c, wsum, &tot);
  for (int i = i0; i < i1; ++i)
    if (s.flag[i]) out_idx[pos++] = i;
  __syncthreads();
}

}  // namespace cfm
