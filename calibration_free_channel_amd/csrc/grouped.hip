// Expert-grouped forward pass for decode batches (gfx950).
//
// Same method and same selections as the per-pair kernel (arXiv:2610.37386,
// abstract; aimodeling.com article, section "A reader that needs no data at
// all"): each routed (token, expert) pair still screens with the sketch, takes
// its own top-c candidates, its own exact top-k and its own recovery term. What
// changes is who reads the weights. Once a batch routes several tokens to one
// expert (batch 8 and up: the article's batch-size table), the pairs are
// grouped by expert and every weight row an expert needs is read once for all
// of its tokens:
//   - the sketch rows of an expert, screened for up to 16 of its tokens per
//     read on the FP8/FP4 matrix cores (two tokens per 16-column tile);
//   - the gate / up rows of the union of the expert's candidate sets, dotted
//     with all of its tokens on the BF16 matrix cores (each token then uses the
//     rows of its own candidates only);
//   - the down rows of the union of the kept sets, contracted with a per-token
//     masked BF16 activation matrix (zero outside the token's kept set), plus
//     the low-rank term A z on the same tiles.
// The sketch activations are bit-identical to the per-pair kernel's (same
// rotation code, exact integer dot products), so the candidate sets are the
// same; exact activations and outputs differ from it by float rounding only.
//
// Unlike the per-pair kernel this is a short sequence of ordinary launches
// (no inter-workgroup waits): each stage is a streaming kernel with many
// workgroups per compute unit, which is what hides memory latency once there
// is enough work in flight.
//
//   k_g_prep    rotation and digit planes of every token; grouping of the
//               pairs by expert (one workgroup)
//   k_g_screen  (64-channel tile, expert and token group) work items
//   k_g_topc    top-c candidates per pair, candidate bitmaps
//   k_g_exact   (16 union rows, expert) work items: gate / up / h
//   k_g_topk    top-k per pair, masked BF16 activations, recovery coefficients
//   k_g_down    (64 output columns, expert) work items: down rows and A z
//   k_g_combine router-weighted sum per token, BF16 output
#include <algorithm>

#include "cfm_internal.h"
#include "cfm_launch.h"
#include "rotate.h"
#include "topk.h"

namespace cfm {
namespace {

constexpr int GT = 256;            // threads per workgroup
constexpr int kTile = 64;          // channels per screen work item (128 sketch rows, 8 MFMA row tiles)
constexpr int kTokGroup = 16;      // tokens per screen work item
constexpr int kSbReg = 8;          // super-blocks of sketch rows held in registers (H <= 2048)
constexpr int kRowBlk = 16;        // union rows per exact work item (one MFMA row tile)
constexpr int kKc = 8;             // 32-element steps of one exact load batch
constexpr int kColTile = 64;       // output columns per down work item (16 per wavefront)
constexpr int kDnRows = 128;       // union rows per down step
constexpr int kDnPitch = kDnRows + 8;   // LDS row pitch (BF16) of the down operands
constexpr int kRPad = 128;         // recovery rank padded to whole 32-element steps (r <= 128)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint4 ld16(const void* p) {        // streamed weights
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16c(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// D += A B on the BF16 matrix cores: lane l holds row (l % 16) of A and column
// (l % 16) of B at the same eight k positions (group l / 16); D lane l holds
// rows 4 (l / 16) + v of column l % 16.
__device__ __forceinline__ v4f mfma_bf16(const uint4& a, const uint4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

struct GArgs {
  const uint16_t* x; const int32_t* ids; const float* topk_w;
  const uint16_t *wg, *wu, *wd;
  const int8_t* signs; const uint8_t *tg, *tu; const float *sg, *su;
  const uint16_t *A, *Bt;
  uint16_t* out; int32_t *cand_out, *keep_out;
  uint32_t* meta;     // [0] experts used, [1] screen work items
  int32_t* goff;      // [E + 1] first position of each expert's pairs in gpl
  int32_t* gpl;       // [P] pairs sorted by expert
  int32_t* gue;       // [E] used experts, ascending
  int32_t* gwork;     // [nwork] screen work items: used expert << 16 | token group
  uint8_t* xd;        // [T][kPlanes][Hp] digit planes of x~
  int32_t* xf0;       // [T] fixed-point exponents
  float* hs;          // [P][I] sketch activations
  float* zp;          // [P][ntile][r] sketch-activation recovery sums per channel tile
  uint32_t* cm;       // [P][IW] candidate bitmaps
  int32_t* cl;        // [P][c] candidates, ascending
  float* hx;          // [P][I] exact activations (meaningful at the pair's candidates)
  uint32_t* km;       // [P][IW] kept bitmaps
  uint16_t* hk;       // [P][I] BF16 exact activations at the kept channels, 0 elsewhere
  float* zf;          // [P][r] recovery coefficients
  float* yp;          // [P][H] pair outputs
  uint32_t* ucnt;     // [E] candidate-union rows per used expert
  uint32_t* dcnt;     // [E] kept-union rows per used expert
  int T, K, P, E, I, H, log2H, k, c, r, ntile, IW, dense;
};

// ------------------------------------------------------------------ block helpers

// In-place exclusive prefix sum of v[0..n) (LDS), n <= 16 GT; returns the total.
// wtot: 4 words of LDS. Called by the whole workgroup; ends with a barrier.
__device__ __forceinline__ uint32_t block_exscan(uint32_t* v, int n, uint32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (n + GT - 1) / GT;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  uint32_t s = 0;
  for (int i = i0; i < i1; ++i) s += v[i];
  const uint32_t incl = wave_incl_scan(s);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wv; ++w) base += wtot[w];
  const uint32_t total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  uint32_t run = base + incl - s;
  for (int i = i0; i < i1; ++i) {
    const uint32_t x = v[i];
    v[i] = run;
    run += x;
  }
  __syncthreads();
  return total;
}

// Union of the bitmaps of pairs pl[0..n) (or all channels when dense) into
// U[0..IW) with exclusive prefix popcounts pc[0..IW); returns the union size.
__device__ __forceinline__ uint32_t union_rows(const uint32_t* bm, const int32_t* pl, int n, int IW, int I,
                                               bool dense, uint32_t* U, uint32_t* pc, uint32_t* wtot) {
  for (int w = threadIdx.x; w < IW; w += GT) {
    uint32_t u = 0;
    if (dense) {
      const int left = I - 32 * w;
      u = left >= 32 ? ~0u : ((1u << left) - 1u);
    } else {
      for (int s = 0; s < n; ++s) u |= bm[(size_t)pl[s] * IW + w];
    }
    U[w] = u;
    pc[w] = __builtin_popcount(u);
  }
  __syncthreads();
  return block_exscan(pc, IW, wtot);
}

// rows[q - lo] = the channel of union rank q, for lo <= q < hi.
__device__ __forceinline__ void union_list(const uint32_t* U, const uint32_t* pc, int IW, uint32_t lo, uint32_t hi,
                                           uint16_t* rows) {
  for (int w = threadIdx.x; w < IW; w += GT) {
    uint32_t u = U[w], q = pc[w];
    if (q >= hi || q + __builtin_popcount(u) <= lo) continue;
    while (u) {
      const int b = __builtin_ctz(u);
      u &= u - 1;
      if (q >= lo && q < hi) rows[q - lo] = (uint16_t)(32 * w + b);
      ++q;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ stage 1: rotation and grouping

template <int EPT>
__global__ __launch_bounds__(GT) void k_g_prep(GArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) uint32_t wred[4];
  __shared__ __align__(16) int wf0[4];
  const int tid = threadIdx.x, H = a.H;
  const int Hp = max(H, 256);
  if ((int)blockIdx.x < a.T) {
    if (a.dense) return;
    const int t = blockIdx.x;
    const RotBuf rb{H, a.log2H, reinterpret_cast<int32_t*>(smem), smem + 4 * (size_t)Hp};
    int F0;
    if constexpr (EPT >= 4) {
      uint4 xq[EPT >= 8 ? EPT / 8 : 1];
      uint32_t sq[EPT / 4];
      const uint16_t* xt = a.x + (size_t)t * H + EPT * tid;
      if constexpr (EPT >= 8) {
#pragma unroll
        for (int g = 0; g < EPT / 8; ++g) xq[g] = ld16c(xt + 8 * g);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(xt);
        xq[0] = make_uint4(u.x, u.y, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < EPT / 4; ++g) sq[g] = *reinterpret_cast<const uint32_t*>(a.signs + EPT * tid + 4 * g);
      F0 = rotate_fast<EPT>(rb, xq, sq, wf0);
    } else {
      F0 = rotate_small(rb, a.x + (size_t)t * H, a.signs, wred);
    }
    const uint4* src = reinterpret_cast<const uint4*>(rb.limb);
    uint4* dst = reinterpret_cast<uint4*>(a.xd + (size_t)t * kPlanes * Hp);
    for (int i = tid; i < kPlanes * Hp / 16; i += GT) dst[i] = src[i];
    if (tid == 0) a.xf0[t] = F0;
    return;
  }
  // grouping: counts, offsets, pair lists, used experts, screen work items
  const int E = a.E, P = a.P;
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem);          // [E]
  uint32_t* off = cnt + E;                                     // [E]
  uint32_t* uix = off + E;                                     // [E]
  uint32_t* wof = uix + E;                                     // [E]
  for (int e = tid; e < E; e += GT) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += GT) atomicAdd(&cnt[min(max(a.ids[p], 0), E - 1)], 1u);
  __syncthreads();
  for (int e = tid; e < E; e += GT) {
    const uint32_t n = cnt[e];
    off[e] = n;
    uix[e] = n > 0;
    wof[e] = (n + kTokGroup - 1) / kTokGroup;
  }
  __syncthreads();
  block_exscan(off, E, wred);
  const uint32_t nue = block_exscan(uix, E, wred);
  const uint32_t nwork = block_exscan(wof, E, wred);
  for (int e = tid; e < E; e += GT) {
    a.goff[e] = (int)off[e];
    const uint32_t n = cnt[e];
    if (n > 0) {
      a.gue[uix[e]] = e;
      const uint32_t ng = (n + kTokGroup - 1) / kTokGroup;
      for (uint32_t g = 0; g < ng; ++g) a.gwork[wof[e] + g] = (int)((uix[e] << 16) | g);
    }
  }
  if (tid == 0) {
    a.goff[E] = P;
    a.meta[0] = nue;
    a.meta[1] = nwork;
  }
  __syncthreads();
  // pairs into their expert's segment (the order inside a segment does not
  // change any result: every column of a tile is computed independently)
  for (int p = tid; p < P; p += GT) {
    const int e = min(max(a.ids[p], 0), E - 1);
    a.gpl[atomicAdd(&off[e], 1u)] = p;
  }
}

// ------------------------------------------------------------------ stage 2: screen

// B operand of two tokens for super-block sb and half m: columns 0..5 are the
// digit planes of the first token (LDS rows 0..5), 6..11 those of the second
// (rows 6..11), column 12 all ones, 13..15 zero; the hidden-index order matches
// the FP4 A operand of the sketch rows (as in the per-pair screen).
__device__ __forceinline__ v8i digit_operand2(const uint8_t* limb2, int Hp, int sb, int m) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, gB = lane >> 4;
  const uint8_t* row = limb2 + (size_t)min(col, 2 * kPlanes - 1) * Hp;
  const int i0 = sb * 256 + 64 * (gB >> 1) + 32 * m + 16 * (gB & 1);
  const uint4 lo = *reinterpret_cast<const uint4*>(row + i0);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + i0 + 128);
  const unsigned keep = col < 2 * kPlanes ? 0xFFFFFFFFu : 0u;
  const unsigned one = col == 2 * kPlanes ? 0x38383838u : 0u;       // FP8 E4M3 1.0
  v8i b;
  b[0] = (lo.x & keep) | one; b[1] = (lo.y & keep) | one; b[2] = (lo.z & keep) | one; b[3] = (lo.w & keep) | one;
  b[4] = (hi.x & keep) | one; b[5] = (hi.y & keep) | one; b[6] = (hi.z & keep) | one; b[7] = (hi.w & keep) | one;
  return b;
}

// Sketch item of row tile q (rows 16 (wv + 4 q) .. +16 of the 128 rows of a
// 64-channel tile: rows 0..63 gate, 64..127 up) and super-block s: lane
// (row = lane & 15, g = lane >> 4) takes the 16 bytes at 64 s + 16 g of its row.
__device__ __forceinline__ uint4 sketch_item2(const GArgs& a, int e, int j0, int cw, int q, int s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rho = 16 * (wv + 4 * q) + (lane & 15);
  const int rowb = a.H / 4;
  const int off = 64 * s + 16 * (lane >> 4);
  const int jj = min(rho & 63, cw - 1);              // rows past the tile repeat a valid row (never read)
  const uint8_t* base = rho < 64 ? a.tg : a.tu;
  return ld16(base + ((size_t)e * a.I + j0 + jj) * rowb + (off < rowb ? off : 0));
}

// Work item (tile, screen item): the sketch rows of channels [j0, j0 + 64) of
// expert e against up to 16 of its tokens, two per pass.
template <bool REG>
__global__ __launch_bounds__(GT) void k_g_screen(GArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  if ((uint32_t)blockIdx.y >= a.meta[1]) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, r = a.r;
  const int Hp = max(H, 256);
  const int nsb = (H + 255) / 256;
  const int item = a.gwork[blockIdx.y];
  const int e = a.gue[item >> 16];
  const int g0 = (item & 0xFFFF) * kTokGroup;
  const int p0 = a.goff[e], n = min(a.goff[e + 1] - p0 - g0, kTokGroup);
  const int tile = blockIdx.x, j0 = tile * kTile, cw = min(kTile, I - j0);
  uint8_t* limb2 = smem;                                                   // [12][Hp]
  float* dsum = reinterpret_cast<float*>(smem + 2 * kPlanes * (size_t)Hp);  // [128][16]
  float* gu = dsum + 128 * 16;                                             // [2][128]
  float* hl = gu + 2 * 128;                                                // [2][64]
  float* scl = hl + 2 * 64;                                                // [128]
  uint16_t* bts = reinterpret_cast<uint16_t*>(scl + 128);                  // [64][r]

  uint4 wa[2][kSbReg];
  if constexpr (REG) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int s = 0; s < kSbReg; ++s) wa[q][s] = sketch_item2(a, e, j0, cw, q, min(s, nsb - 1));
  }
  if (tid < 128) {
    const int jj = min(tid & 63, cw - 1);
    scl[tid] = (tid < 64 ? a.sg : a.su)[(size_t)e * I + j0 + jj];
  }
  if (r > 0) {
    const uint16_t* src = a.Bt + ((size_t)e * I + j0) * r;
    for (int i = tid; i < kTile * r; i += GT) bts[i] = i < cw * r ? src[i] : (uint16_t)0;
  }
  for (int q2 = 0; q2 < n; q2 += 2) {
    const int pa = a.gpl[p0 + g0 + q2];
    const int pb = a.gpl[p0 + g0 + min(q2 + 1, n - 1)];
    const int ta = pa / a.K, tb = pb / a.K;
    // digit planes of the two tokens
    {
      const uint4* sa = reinterpret_cast<const uint4*>(a.xd + (size_t)ta * kPlanes * Hp);
      const uint4* sb = reinterpret_cast<const uint4*>(a.xd + (size_t)tb * kPlanes * Hp);
      uint4* d = reinterpret_cast<uint4*>(limb2);
      const int half = kPlanes * Hp / 16;
      for (int i = tid; i < 2 * half; i += GT) d[i] = i < half ? sa[i] : sb[i - half];
    }
    __syncthreads();
    v4f acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsb; s0 += kSbReg) {
      uint4 wl[2][kSbReg];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int u = 0; u < kSbReg; ++u) {
          if constexpr (REG) wl[q][u] = wa[q][u];
          else wl[q][u] = sketch_item2(a, e, j0, cw, q, min(s0 + u, nsb - 1));
        }
#pragma unroll
      for (int u = 0; u < kSbReg; ++u) {
        const int s = s0 + u;
        if (s < nsb) {
          const uint32_t km = 64 * s + 16 * (lane >> 4) < H / 4 ? ~0u : 0u;   // codes past the row end (H < 256)
          const v8i d0 = digit_operand2(limb2, Hp, s, 0);
          const v8i d1 = digit_operand2(limb2, Hp, s, 1);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                trit_operand(wl[q][u].x & km, wl[q][u].y & km), d0, acc[q], 4, 0, 0, 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                trit_operand(wl[q][u].z & km, wl[q][u].w & km), d1, acc[q], 4, 0, 0, 0, 0, 0);
          }
        }
      }
    }
    // lane holds D[4 (lane / 16) + v][lane % 16] of each of its two row tiles
    {
      const int col = lane & 15;
      if (col <= 2 * kPlanes) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) dsum[(16 * (wv + 4 * q) + 4 * (lane >> 4) + v) * 16 + col] = acc[q][v];
      }
    }
    __syncthreads();
    // per-row scale times the exact integer dot (as in the per-pair screen)
    {
      const int tk = tid >> 7, rho = tid & 127;
      const float* d = dsum + rho * 16 + kPlanes * tk;
      const long long S = (long long)(int)d[0] + ((long long)(int)d[1] << 4) + ((long long)(int)d[2] << 8) +
                          ((long long)(int)d[3] << 12) + ((long long)(int)d[4] << 16) +
                          ((long long)(int)d[5] << 20) - ((long long)(int)dsum[rho * 16 + 2 * kPlanes] << 23);
      const int F0 = a.xf0[tk ? tb : ta];
      gu[tk * 128 + rho] = (float)((double)scl[rho] * ldexp((double)S, kDShift - F0));
    }
    __syncthreads();
    if (tid < 128) {
      const int tk = tid >> 6, jj = tid & 63;
      const bool ok = jj < cw && q2 + tk < n;
      const float hv = silu_f32(gu[tk * 128 + jj]) * gu[tk * 128 + 64 + jj];
      hl[tk * 64 + jj] = ok ? hv : 0.f;
      if (ok) a.hs[(size_t)(tk ? pb : pa) * I + j0 + jj] = hv;
    }
    __syncthreads();
    // this tile's share of the recovery sums: sum_j hhat_j Bt[j][:]
    if (r > 0) {
      const int tk = tid >> 7, l = tid & 127;
      if (l < r && q2 + tk < n) {
        float z = 0.f;
        for (int jj = 0; jj < cw; ++jj) z += hl[tk * 64 + jj] * bf16_to_f32(bts[jj * r + l]);
        a.zp[((size_t)(tk ? pb : pa) * a.ntile + tile) * r + l] = z;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ stage 3: top-c

template <int KPT>
__global__ __launch_bounds__(GT) void k_g_topc(GArgs a) {
  __shared__ __align__(16) uint32_t tks[kTopkScratchWords];
  __shared__ __align__(16) int32_t cand[kMaxI];
  __shared__ uint32_t bm[kMaxI / 32];
  const int p = blockIdx.x, tid = threadIdx.x;
  const int I = a.I, c = a.c;
  int cnt;
  const int i0 = topk_range<GT>(I, &cnt);
  uint32_t kr[KPT];
  const float* src = a.hs + (size_t)p * I + i0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) kr[j] = j < cnt ? score_key(src[j]) : 0u;
  block_topk<GT, KPT>(kr, i0, cnt, I, c, cand, tks);
  for (int w = tid; w < a.IW; w += GT) bm[w] = 0;
  __syncthreads();
  for (int i = tid; i < c; i += GT) {
    const int j = cand[i];
    a.cl[(size_t)p * c + i] = j;
    if (a.cand_out) a.cand_out[(size_t)p * c + i] = j;
    atomicOr(&bm[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  for (int w = tid; w < a.IW; w += GT) a.cm[(size_t)p * a.IW + w] = bm[w];
}

// ------------------------------------------------------------------ stage 4: exact gate / up

// Work item (row block, used expert): union rows [16 b, 16 b + 16) of the
// expert's candidate union, against all of its tokens. Wavefront w takes a
// contiguous quarter of the 32-element k steps; the quarters are summed in LDS.
__global__ __launch_bounds__(GT) void k_g_exact(GArgs a) {
  __shared__ __align__(16) uint32_t U[kMaxI / 32];
  __shared__ __align__(16) uint32_t pc[kMaxI / 32];
  __shared__ uint32_t wtot[4];
  __shared__ uint16_t rows[kRowBlk];
  __shared__ __align__(16) float red[4 * 2 * 4 * 256];     // [wave][gate, up][token tile][D]
  const int u = blockIdx.y;
  if ((uint32_t)u >= a.meta[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I;
  const int e = a.gue[u];
  const int p0 = a.goff[e], n = a.goff[e + 1] - p0;
  const int32_t* pl = a.gpl + p0;
  const uint32_t nU = union_rows(a.cm, pl, n, a.IW, I, a.dense != 0, U, pc, wtot);
  if (blockIdx.x == 0 && tid == 0) a.ucnt[u] = nU;
  const uint32_t lo = kRowBlk * blockIdx.x;
  if (lo >= nU) return;
  const int nrow = (int)min((uint32_t)kRowBlk, nU - lo);
  union_list(U, pc, a.IW, lo, lo + nrow, rows);
  const int row = lane & 15, g = lane >> 4;
  const int j = rows[min(row, nrow - 1)];
  const uint16_t* wgr = a.wg + ((size_t)e * I + j) * H + 8 * g;
  const uint16_t* wur = a.wu + ((size_t)e * I + j) * H + 8 * g;
  const int nks = H / 32, per = (nks + 3) / 4;
  const int ks0 = min(nks, wv * per), ks1 = min(nks, ks0 + per);
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int ngrp = min(4, (n - s0 + 15) / 16);
    const uint16_t* xr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = min(s0 + 16 * q + row, n - 1);
      xr[q] = a.x + (size_t)(pl[s] / a.K) * H + 8 * g;
    }
    v4f ag[4], au[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) { ag[q] = (v4f){0.f, 0.f, 0.f, 0.f}; au[q] = ag[q]; }
    for (int kc = ks0; kc < ks1; kc += kKc) {
      uint4 wgv[kKc], wuv[kKc];
#pragma unroll
      for (int i = 0; i < kKc; ++i) {
        const int ks = min(kc + i, ks1 - 1);
        wgv[i] = ld16(wgr + 32 * ks);
        wuv[i] = ld16(wur + 32 * ks);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < ngrp) {
#pragma unroll
          for (int i = 0; i < kKc; ++i) {
            if (kc + i < ks1) {
              const uint4 xb = ld16c(xr[q] + 32 * (kc + i));
              ag[q] = mfma_bf16(wgv[i], xb, ag[q]);
              au[q] = mfma_bf16(wuv[i], xb, au[q]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<float4*>(red + ((wv * 2 + 0) * 4 + q) * 256 + 4 * lane) =
          make_float4(ag[q][0], ag[q][1], ag[q][2], ag[q][3]);
      *reinterpret_cast<float4*>(red + ((wv * 2 + 1) * 4 + q) * 256 + 4 * lane) =
          make_float4(au[q][0], au[q][1], au[q][2], au[q][3]);
    }
    __syncthreads();
    // element tid of a tile: D[4 (l / 16) + v][l % 16] with l = tid / 4, v = tid % 4
    const int rho = 4 * (tid >> 6) + (tid & 3), col = (tid >> 2) & 15;
    for (int q = 0; q < ngrp; ++q) {
      const int s = s0 + 16 * q + col;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        gs += red[((w * 2 + 0) * 4 + q) * 256 + tid];
        us += red[((w * 2 + 1) * 4 + q) * 256 + tid];
      }
      if (rho < nrow && s < n) {
        const int pp = pl[s];
        const int jr = rows[rho];
        const float h = silu_f32(gs) * us;
        if (a.dense) a.hk[(size_t)pp * I + jr] = f32_to_bf16(h);
        else a.hx[(size_t)pp * I + jr] = h;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ stage 5: top-k and recovery coefficients

template <int KPT>
__global__ __launch_bounds__(GT) void k_g_topk(GArgs a) {
  __shared__ __align__(16) uint32_t tks[kTopkScratchWords];
  __shared__ __align__(16) int32_t sel[kMaxI];
  __shared__ __align__(16) uint16_t hrow[kMaxI];
  __shared__ uint32_t bm[kMaxI / 32];
  __shared__ float zred[GT];
  const int p = blockIdx.x, tid = threadIdx.x;
  const int I = a.I, c = a.c, k = a.k, r = a.r;
  const int e = min(max(a.ids[p], 0), a.E - 1);
  const int32_t* cl = a.cl + (size_t)p * c;
  if (k > 0) {
    int cnt;
    const int i0 = topk_range<GT>(c, &cnt);
    uint32_t kr[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = j < cnt ? score_key(a.hx[(size_t)p * I + cl[i0 + j]]) : 0u;
    block_topk<GT, KPT>(kr, i0, cnt, c, k, sel, tks);
  }
  for (int i = tid; i < I; i += GT) hrow[i] = 0;
  for (int w = tid; w < a.IW; w += GT) bm[w] = 0;
  __syncthreads();
  for (int i = tid; i < k; i += GT) {
    const int j = cl[sel[i]];
    sel[i] = j;                                   // kept channel (each thread rewrites its own entries)
    hrow[j] = f32_to_bf16(a.hx[(size_t)p * I + j]);
    atomicOr(&bm[j >> 5], 1u << (j & 31));
    if (a.keep_out) a.keep_out[(size_t)p * k + i] = j;
  }
  __syncthreads();
  {
    uint16_t* hdst = a.hk + (size_t)p * I;
    if ((I & 1) == 0) {                           // rows start 4-byte aligned
      const uint32_t* hsrc = reinterpret_cast<const uint32_t*>(hrow);
      for (int i = tid; i < I / 2; i += GT) reinterpret_cast<uint32_t*>(hdst)[i] = hsrc[i];
    } else {
      for (int i = tid; i < I; i += GT) hdst[i] = hrow[i];
    }
  }
  for (int w = tid; w < a.IW; w += GT) a.km[(size_t)p * a.IW + w] = bm[w];
  // z = sum over all channels of hhat_j Bt[j] (the screen's tile sums) minus the kept ones
  if (r > 0) {
    const int groups = GT / r, l = tid % r, gi = tid / r;
    float z = 0.f;
    if (gi < groups) {
      const float* zs = a.zp + (size_t)p * a.ntile * r;
      for (int t = gi; t < a.ntile; t += groups) z += zs[(size_t)t * r + l];
      const float* hsp = a.hs + (size_t)p * I;
      for (int i = gi; i < k; i += groups) {
        const int j = sel[i];
        z -= hsp[j] * bf16_to_f32(a.Bt[((size_t)e * I + j) * r + l]);
      }
    }
    zred[tid] = z;
    __syncthreads();
    if (tid < r) {
      float s = 0.f;
      for (int q = 0; q < groups; ++q) s += zred[q * r + tid];
      a.zf[(size_t)p * r + tid] = s;
    }
  }
}

// ------------------------------------------------------------------ stage 6: down projection and A z

// Work item (column tile, used expert): output columns [64 b, 64 b + 64) of all
// of the expert's tokens, 16 tokens at a time. Wavefront w owns columns
// 16 w .. 16 w + 15. D = tokens x columns: the A operand is the token's masked
// activations (or its recovery coefficients), the B operand the down rows (or
// the rows of A), staged column-major in LDS so that each lane reads eight
// consecutive contraction indices.
__global__ __launch_bounds__(GT) void k_g_down(GArgs a) {
  __shared__ __align__(16) uint32_t U[kMaxI / 32];
  __shared__ __align__(16) uint32_t pc[kMaxI / 32];
  __shared__ uint32_t wtot[4];
  __shared__ __align__(16) uint16_t rows[kMaxI];
  __shared__ __align__(16) uint16_t hA[16 * kDnPitch];        // [token][row]
  __shared__ __align__(16) uint16_t wT[kColTile * kDnPitch];  // [column][row]
  const int u = blockIdx.y;
  if ((uint32_t)u >= a.meta[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, r = a.r;
  const int e = a.gue[u];
  const int p0 = a.goff[e], n = a.goff[e + 1] - p0;
  const int32_t* pl = a.gpl + p0;
  const int c0 = kColTile * blockIdx.x;
  const uint32_t nU = union_rows(a.km, pl, n, a.IW, I, a.dense != 0, U, pc, wtot);
  if (blockIdx.x == 0 && tid == 0) a.dcnt[u] = nU;
  union_list(U, pc, a.IW, 0, nU, rows);
  const int m16 = lane & 15, g = lane >> 4;
  const int col = c0 + 16 * wv + m16;            // this lane's output column (B operand and D)
  for (int s0 = 0; s0 < n; s0 += 16) {
    const int nt = min(16, n - s0);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    // recovery: D += z (tokens x r) A[e]^T (r x columns); z staged in hA
    if (r > 0 && !a.dense) {
      for (int i = tid; i < 16 * kRPad; i += GT) {
        const int m = i / kRPad, l = i % kRPad;
        const float z = (m < nt && l < r) ? a.zf[(size_t)pl[s0 + m] * r + l] : 0.f;
        hA[m * kDnPitch + l] = f32_to_bf16(z);
      }
      __syncthreads();
      const uint16_t* arow = a.A + ((size_t)e * H + col) * r;
      for (int ks = 0; ks < (r + 31) / 32; ++ks) {
        const int l0 = 32 * ks + 8 * g;
        const uint4 bv = l0 < r ? ld16c(arow + l0) : make_uint4(0, 0, 0, 0);
        const uint4 av = *reinterpret_cast<const uint4*>(hA + m16 * kDnPitch + l0);
        acc = mfma_bf16(av, bv, acc);
      }
      __syncthreads();
    }
    for (uint32_t q0 = 0; q0 < nU; q0 += kDnRows) {
      const int nr = (int)min((uint32_t)kDnRows, nU - q0);
      // down rows: 16-byte pieces (row rho, columns 8 cc .. 8 cc + 7)
      uint4 wv4[kDnRows * 8 / GT];
#pragma unroll
      for (int qq = 0; qq < kDnRows * 8 / GT; ++qq) {
        const int idx = tid + GT * qq, rho = idx >> 3, cc = idx & 7;
        const int jr = rows[q0 + min(rho, nr - 1)];
        wv4[qq] = ld16(a.wd + ((size_t)e * I + jr) * H + c0 + 8 * cc);
      }
      // masked activations of the tokens at these rows
      for (int i = tid; i < 16 * kDnRows; i += GT) {
        const int m = i / kDnRows, rho = i % kDnRows;
        hA[m * kDnPitch + rho] = (m < nt && rho < nr) ? a.hk[(size_t)pl[s0 + m] * I + rows[q0 + rho]] : (uint16_t)0;
      }
#pragma unroll
      for (int qq = 0; qq < kDnRows * 8 / GT; ++qq) {
        const int idx = tid + GT * qq, rho = idx >> 3, cc = idx & 7;
        const bool ok = rho < nr;
        const uint32_t w4[4] = {ok ? wv4[qq].x : 0u, ok ? wv4[qq].y : 0u, ok ? wv4[qq].z : 0u, ok ? wv4[qq].w : 0u};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          wT[(8 * cc + 2 * h) * kDnPitch + rho] = (uint16_t)(w4[h] & 0xFFFFu);
          wT[(8 * cc + 2 * h + 1) * kDnPitch + rho] = (uint16_t)(w4[h] >> 16);
        }
      }
      __syncthreads();
      for (int ks = 0; ks < (nr + 31) / 32; ++ks) {
        const uint4 av = *reinterpret_cast<const uint4*>(hA + m16 * kDnPitch + 32 * ks + 8 * g);
        const uint4 bv = *reinterpret_cast<const uint4*>(wT + (16 * wv + m16) * kDnPitch + 32 * ks + 8 * g);
        acc = mfma_bf16(av, bv, acc);
      }
      __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < nt) a.yp[(size_t)pl[s0 + m] * H + col] = acc[v];
    }
  }
}

// ------------------------------------------------------------------ stage 7: combine

__global__ __launch_bounds__(GT) void k_g_combine(GArgs a) {
  const int t = blockIdx.x, H = a.H, K = a.K;
  for (int h0 = 8 * threadIdx.x; h0 < H; h0 += 8 * GT) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int q = 0; q < K; ++q) {
      const float w = a.topk_w[(size_t)t * K + q];
      const float4* y = reinterpret_cast<const float4*>(a.yp + ((size_t)t * K + q) * H + h0);
      const float4 y0 = y[0], y1 = y[1];
      acc[0] += w * y0.x; acc[1] += w * y0.y; acc[2] += w * y0.z; acc[3] += w * y0.w;
      acc[4] += w * y1.x; acc[5] += w * y1.y; acc[6] += w * y1.z; acc[7] += w * y1.w;
    }
    *reinterpret_cast<uint4*>(a.out + (size_t)t * H + h0) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7]));
  }
}

// ------------------------------------------------------------------ stats

__global__ void k_g_stats(GArgs a, cfm_stats* st) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const uint32_t nue = a.meta[0];
  uint64_t uc = 0, dc = 0;
  for (uint32_t u = 0; u < nue; ++u) {
    if (!a.dense) uc += a.ucnt[u];
    dc += a.dcnt[u];
  }
  if (a.dense) uc = dc;
  else if (a.k == 0) uc = 0;                     // no exact phase ran
  const uint64_t I = a.I, H = a.H, r = a.r;
  cfm_stats s;
  s.bytes_io = 2ull * a.T * H + 8ull * a.T * a.K + 2ull * a.T * H;
  s.bytes_dense_equiv = (uint64_t)nue * 6ull * I * H + s.bytes_io;
  s.experts_used = nue;
  s.bytes_sketch = a.dense ? 0 : (uint64_t)nue * (2ull * I * (H / 4) + 8ull * I);
  s.bytes_candidates = 4ull * H * uc;
  s.bytes_down = 2ull * H * dc;
  s.bytes_recovery = (a.dense || r == 0) ? 0 : (uint64_t)nue * (2ull * H * r + 2ull * I * r);
  s.rows_candidates = (uint32_t)uc;
  s.rows_down = (uint32_t)dc;
  s.pad = 0;
  *st = s;
}

// ------------------------------------------------------------------ host side

size_t prep_lds(int H, int E) {
  const size_t Hp = std::max(H, 256);
  return std::max(10 * Hp, (size_t)16 * E);
}
size_t screen_lds(int H, int r) {
  const size_t Hp = std::max(H, 256);
  return 2 * kPlanes * Hp + 4 * (128 * 16 + 2 * 128 + 2 * 64 + 128) + 2 * (size_t)kTile * std::max(r, 1);
}

int launch_k(const char* name, const void* fn, dim3 grid, size_t lds, const GArgs& ga, hipStream_t stream) {
  if (grid.x == 0 || grid.y == 0) return CFM_OK;
  if (lds > 65536) CFM_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  timing_begin(name, stream);
  void* args[] = {const_cast<GArgs*>(&ga)};
  hipError_t e = hipLaunchKernel(fn, grid, dim3(GT), args, lds, stream);
  timing_end(stream);
  if (e != hipSuccess) return set_error(CFM_EHIP, std::string(name) + ": " + hipGetErrorString(e));
  CFM_LAUNCH_CHECK("grouped stage");
  return CFM_OK;
}

}  // namespace

// ------------------------------------------------------------------ plan

bool grouped_supported(int T, int K, int E, int I, int H, int r, bool dense) {
  const long P = (long)T * K;
  if (P < 1 || P > 65535 || E > 4096 || I > kMaxI || H < 64 || H > kMaxH || H % kColTile) return false;
  return dense || (is_pow2(H) && r >= 0 && r <= kRPad && r % 8 == 0);
}

GroupPlan group_plan(int T, int K, int E, int I, int H, int k, int c, int r, bool dense, size_t base) {
  GroupPlan g{};
  g.T = T; g.K = K; g.P = T * K; g.E = E; g.I = I; g.H = H; g.k = k; g.c = c; g.r = r; g.dense = dense;
  g.ntile = (I + kTile - 1) / kTile;
  g.IW = (I + 31) / 32;
  g.maxu = std::min(E, g.P);
  g.maxwork = g.maxu + (g.P + kTokGroup - 1) / kTokGroup;
  const size_t P = (size_t)g.P, Hp = std::max(H, 256);
  Carve cv;
  cv.off = base;
  g.off_meta = cv.take(16);
  g.off_goff = cv.take(4 * ((size_t)E + 1));
  g.off_gpl = cv.take(4 * P);
  g.off_gue = cv.take(4 * (size_t)E);
  g.off_gwork = cv.take(4 * (size_t)g.maxwork);
  g.off_xf0 = cv.take(4 * (size_t)T);
  g.off_xd = cv.take(dense ? 16 : (size_t)T * kPlanes * Hp);
  g.off_hs = cv.take(dense ? 16 : P * I * 4);
  g.off_zp = cv.take(dense || r == 0 ? 16 : P * g.ntile * r * 4);
  g.off_cm = cv.take(dense ? 16 : P * g.IW * 4);
  g.off_cl = cv.take(dense ? 16 : P * std::max(c, 1) * 4);
  g.off_hx = cv.take(dense ? 16 : P * I * 4);
  g.off_km = cv.take(dense ? 16 : P * g.IW * 4);
  g.off_hk = cv.take(P * I * 2);
  g.off_zf = cv.take(dense || r == 0 ? 16 : P * r * 4);
  g.off_yp = cv.take(P * H * 4);
  g.off_ucnt = cv.take(4 * (size_t)E);
  g.off_dcnt = cv.take(4 * (size_t)E);
  g.bytes = cv.off;
  return g;
}

int launch_grouped_forward(const SelectArgs& s, const GroupPlan& g, hipStream_t stream) {
  GArgs a{};
  a.x = s.x; a.ids = s.ids; a.topk_w = s.topk_w;
  a.wg = s.w_gate; a.wu = s.w_up; a.wd = s.w_down_t;
  a.signs = s.signs; a.tg = s.tg; a.tu = s.tu; a.sg = s.sg; a.su = s.su;
  a.A = s.A; a.Bt = s.Bt;
  a.out = s.out; a.cand_out = s.cand_out; a.keep_out = s.keep_out;
  char* ws = s.ws;
  a.meta = reinterpret_cast<uint32_t*>(ws + g.off_meta);
  a.goff = reinterpret_cast<int32_t*>(ws + g.off_goff);
  a.gpl = reinterpret_cast<int32_t*>(ws + g.off_gpl);
  a.gue = reinterpret_cast<int32_t*>(ws + g.off_gue);
  a.gwork = reinterpret_cast<int32_t*>(ws + g.off_gwork);
  a.xd = reinterpret_cast<uint8_t*>(ws + g.off_xd);
  a.xf0 = reinterpret_cast<int32_t*>(ws + g.off_xf0);
  a.hs = reinterpret_cast<float*>(ws + g.off_hs);
  a.zp = reinterpret_cast<float*>(ws + g.off_zp);
  a.cm = reinterpret_cast<uint32_t*>(ws + g.off_cm);
  a.cl = reinterpret_cast<int32_t*>(ws + g.off_cl);
  a.hx = reinterpret_cast<float*>(ws + g.off_hx);
  a.km = reinterpret_cast<uint32_t*>(ws + g.off_km);
  a.hk = reinterpret_cast<uint16_t*>(ws + g.off_hk);
  a.zf = reinterpret_cast<float*>(ws + g.off_zf);
  a.yp = reinterpret_cast<float*>(ws + g.off_yp);
  a.ucnt = reinterpret_cast<uint32_t*>(ws + g.off_ucnt);
  a.dcnt = reinterpret_cast<uint32_t*>(ws + g.off_dcnt);
  a.T = g.T; a.K = g.K; a.P = g.P; a.E = g.E; a.I = g.I; a.H = g.H;
  int log2H = 0;
  while ((1 << log2H) < g.H) ++log2H;
  a.log2H = log2H;
  a.k = g.dense ? g.I : g.k; a.c = g.dense ? g.I : g.c; a.r = g.dense ? 0 : g.r;
  a.ntile = g.ntile; a.IW = g.IW; a.dense = g.dense ? 1 : 0;
  const int H = g.H;

  // 1. rotation + grouping
  {
    const int ept = H >= 1024 ? H / 256 : 0;
    const void* fn = nullptr;
    switch (ept) {
      case 0: fn = reinterpret_cast<const void*>(&k_g_prep<0>); break;
      case 4: fn = reinterpret_cast<const void*>(&k_g_prep<4>); break;
      case 8: fn = reinterpret_cast<const void*>(&k_g_prep<8>); break;
      case 16: fn = reinterpret_cast<const void*>(&k_g_prep<16>); break;
      case 32: fn = reinterpret_cast<const void*>(&k_g_prep<32>); break;
      default: return set_error(CFM_EUNSUPPORTED, "hidden width not supported");
    }
    if (int rc = launch_k("k_g_prep", fn, dim3(g.T + 1), prep_lds(H, g.E), a, stream)) return rc;
  }
  if (!g.dense) {
    // 2. screen
    {
      const bool reg = (H + 255) / 256 <= kSbReg;
      const void* fn = reg ? reinterpret_cast<const void*>(&k_g_screen<true>)
                           : reinterpret_cast<const void*>(&k_g_screen<false>);
      if (int rc = launch_k("k_g_screen", fn, dim3(g.ntile, g.maxwork), screen_lds(H, g.r), a, stream)) return rc;
    }
    // 3. top-c
    {
      const int per = (g.I + GT - 1) / GT;
      const void* fn = per <= 4 ? reinterpret_cast<const void*>(&k_g_topc<4>)
                                : reinterpret_cast<const void*>(&k_g_topc<32>);
      if (int rc = launch_k("k_g_topc", fn, dim3(g.P), 0, a, stream)) return rc;
    }
  }
  // 4. exact gate / up over the candidate unions (all channels when dense)
  if (g.dense || g.k > 0) {
    if (int rc = launch_k("k_g_exact", reinterpret_cast<const void*>(&k_g_exact),
                          dim3((g.I + kRowBlk - 1) / kRowBlk, g.maxu), 0, a, stream))
      return rc;
  }
  if (!g.dense) {
    // 5. top-k, masked activations, recovery coefficients
    const int per = (std::max(g.c, 1) + GT - 1) / GT;
    const void* fn = per <= 4 ? reinterpret_cast<const void*>(&k_g_topk<4>)
                              : reinterpret_cast<const void*>(&k_g_topk<32>);
    if (int rc = launch_k("k_g_topk", fn, dim3(g.P), 0, a, stream)) return rc;
  }
  // 6. down + recovery, 7. combine
  if (int rc = launch_k("k_g_down", reinterpret_cast<const void*>(&k_g_down), dim3(H / kColTile, g.maxu), 0, a,
                        stream))
    return rc;
  if (int rc = launch_k("k_g_combine", reinterpret_cast<const void*>(&k_g_combine), dim3(g.T), 0, a, stream))
    return rc;
  if (s.stats) {
    hipLaunchKernelGGL(k_g_stats, dim3(1), dim3(64), 0, stream, a, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_g_stats");
  }
  return CFM_OK;
}

}  // namespace cfm
