// Expert-grouped forward pass for decode batches (gfx950).
//
// Same method and same selections as the per-pair kernel (arXiv:2610.37386,
// abstract; aimodeling.com article, section "A reader that needs no data at
// all"): each routed (token, expert) pair still screens with the sketch, takes
// its own top-c candidates, its own exact top-k and its own recovery term. What
// changes is who reads the weights. Once a batch routes several tokens to one
// expert (batch 8 and up, where the article, section "Numbers and limits",
// reports its largest gains, peaking at batch 8 or 16), the pairs are
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
// with no inter-workgroup waits. Each stage is a streaming kernel with many
// workgroups per compute unit; every global load of a stage is issued in one
// batch before its first use, so a workgroup pays about one memory latency per
// step. Where a stage needs a per-expert or per-token result that several
// workgroups contribute to, the last contributor (release fence, counter,
// acquire fence) computes it; the counters are reset by that workgroup.
//
//   k_g_prep    rotation and digit planes of every token; grouping of the
//               pairs by expert (one workgroup)
//   k_g_screen  (64-channel tile, expert and token group) work items
//   k_g_topc    top-c candidates per pair; the last pair of an expert lists
//               the expert's candidate union and queues its exact work items
//   k_g_exact   (16 union rows, expert) work items: gate / up / h
//   k_g_topk    top-k per pair, masked BF16 activations, recovery
//               coefficients; the last pair of an expert lists its kept union
//   k_g_down    (64 output columns, expert) work items: down rows and A z; the
//               last contribution to a (token, column tile) combines the
//               token's K pairs into the BF16 output
#include <algorithm>

#include "cfm_internal.h"
#include "cfm_launch.h"
#include "envelope.h"
#include "rotate.h"
#include "topk.h"

namespace cfm {
namespace {

constexpr int GT = 256;            // threads per workgroup
constexpr int kTile = 64;          // channels per screen work item (128 sketch rows, 8 MFMA row tiles)
constexpr int kTokGroup = 16;      // tokens per screen work item
constexpr int kSbReg = 8;          // super-blocks of sketch rows held in registers (H <= 2048)
constexpr int kRowBlk = 64;        // union rows per exact work item (one MFMA row tile per wavefront)
constexpr int kKc = 8;             // 32-element steps of one exact load batch (two batches in flight; fewer for H < 256)
constexpr int kColTile = 64;       // output columns per down work item (16 per wavefront)
constexpr int kRPad = 128;         // recovery rank padded to whole 32-element steps (r <= 128)
constexpr int kDP = 17;            // LDS pitch (FP32) of a screen wavefront's D tiles: odd, so the per-row reads hit distinct banks
constexpr int kExactGrid = 512;    // workgroups of the exact stage (wavefronts loop over its work list)

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

// Values read by another workgroup of the same launch go through agent-scope
// atomic stores and loads (coherent across the XCDs' L2 caches without a cache
// flush); a drained store queue then orders them before a counter update.
__device__ __forceinline__ void st_f(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Completes this wave's outstanding memory operations, then joins the workgroup.
__device__ __forceinline__ void drain_and_join() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
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
  uint32_t* meta;     // [0] experts used, [1] screen work items, [2] exact work items
  int32_t* goff;      // [E + 1] first position of each expert's pairs in gpl
  int32_t* gpl;       // [P] pairs sorted by expert
  int32_t* gue;       // [E] used experts, ascending
  int32_t* gux;       // [E] used index of each expert (-1: not routed)
  int4* gwork;        // [maxwork] screen work items: {expert, first slot in gpl, pairs, 0}
  int32_t* gexw;      // [maxu nrb] exact work items: used expert << 16 | row block
  uint8_t* xd;        // [T][kPlanes][Hp] digit planes of x~
  int32_t* xf0;       // [T] fixed-point exponents
  float* hs;          // [P][I] sketch activations
  float* zp;          // [P][nz][r] sketch-activation recovery sums per 16 channels
  uint32_t* cm;       // [P][IW] candidate bitmaps
  int32_t* cl;        // [P][c] candidates, ascending
  float* hx;          // [P][I] exact activations (meaningful at the pair's candidates)
  uint32_t* km;       // [P][IW] kept bitmaps
  uint16_t* hk;       // [P][I] BF16 exact activations at the kept channels, 0 elsewhere
  float* zf;          // [P][r] recovery coefficients
  float* yp;          // [P][H] pair outputs
  uint32_t* ucnt;     // [maxu] candidate-union rows per used expert
  uint32_t* dcnt;     // [maxu] kept-union rows per used expert
  uint16_t* urows;    // [maxu][IP] candidate-union rows, ascending
  uint16_t* drows;    // [maxu][IP] kept-union rows, ascending
  uint32_t* uctr;     // [E] top-c arrivals per expert (zero between calls)
  uint32_t* kctr;     // [E] top-k arrivals per expert (zero between calls)
  uint32_t* octr;     // [T][H / 64] pair outputs arrived per (token, column tile) (zero between calls)
  int T, K, P, E, I, H, log2H, k, c, r, ntile, nz, IW, nrb, IP, dense;
  int rec_exact;      // dropped candidates enter the recovery with their exact activation
  // the recovery variant with every channel a candidate: no sketch activation
  // enters the result, so the screen does not run (hs and zp are not written
  // and count as zero) and the sketch is not read
  int nosk;
  const uint16_t* resid;   // decode-layer envelope: the residual stream added to the output, else null
  // threshold keep rule (thr != 0): S = the candidates whose score key reaches
  // tkey, in place of the top k (k is then c, the most that can pass)
  int thr;
  uint32_t tkey;
  int32_t* keep_count;     // [P] |S| (optional output; threshold rule)
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

// Arrival of this workgroup at *ctr once its agent-scope stores are complete;
// true in the workgroup that completes `total` arrivals, which resets the
// counter (its agent-scope loads then see every arrival's stores).
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, uint32_t total, int* s_flag) {
  drain_and_join();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == total - 1;
    if (last) st_u(ctr, 0u);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Union of the channel bitmaps bm[p][IW] of expert e's pairs: its channels in
// ascending order into rows_out (global), count returned. U, pc: IW words of
// LDS each; U holds the calling pair's own bitmap on entry (a subset of the
// union). The (pair, word) items are spread over the whole workgroup with four
// requests in flight per thread, so an expert with many pairs costs a round
// trip or two, not one per eight pairs. Called by the whole workgroup.
__device__ __forceinline__ uint32_t expert_union(const GArgs& a, const uint32_t* bm, int e, uint16_t* rows_out,
                                                 uint32_t* U, uint32_t* pc, uint32_t* wtot) {
  const int p0 = a.goff[e], n = a.goff[e + 1] - p0, IW = a.IW;
  const int items = n * IW;
  for (int i0 = threadIdx.x; i0 < items; i0 += 4 * GT) {
    uint32_t x[4];
    int wd[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int it = min(i0 + v * GT, items - 1);
      const int q = it / IW;
      wd[v] = it - q * IW;
      x[v] = ld_u(bm + (size_t)a.gpl[p0 + q] * IW + wd[v]);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (i0 + v * GT < items) atomicOr(&U[wd[v]], x[v]);
  }
  __syncthreads();
  for (int w = threadIdx.x; w < IW; w += GT) pc[w] = __builtin_popcount(U[w]);
  __syncthreads();
  const uint32_t nU = block_exscan(pc, IW, wtot);
  for (int w = threadIdx.x; w < IW; w += GT) {
    uint32_t u = U[w], q = pc[w];
    while (u) {
      const int b = __builtin_ctz(u);
      u &= u - 1;
      rows_out[q++] = (uint16_t)(32 * w + b);
    }
  }
  return nU;
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
    a.gux[e] = n > 0 ? (int)uix[e] : -1;
    if (n > 0) {
      a.gue[uix[e]] = e;
      const uint32_t ng = (n + kTokGroup - 1) / kTokGroup;
      for (uint32_t g = 0; g < ng; ++g)
        a.gwork[wof[e] + g] = make_int4(e, (int)(off[e] + kTokGroup * g), (int)min(n - kTokGroup * g, (uint32_t)kTokGroup), 0);
    }
  }
  if (tid == 0) {
    a.goff[E] = P;
    a.meta[0] = nue;
    a.meta[1] = nwork;
    a.meta[2] = 0;
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

// B operand of two tokens for super-block sb and half m, read from the digit
// planes in global memory (they are L2-resident: T kPlanes Hp bytes in all):
// columns 0..5 are the planes of token a, 6..11 those of token b, column 12
// all ones, 13..15 zero. The hidden-index order matches the FP4 A operand of
// the sketch rows (as in the per-pair screen). Returns (lo, hi) 16-byte halves.
__device__ __forceinline__ void digit_load2(const uint8_t* xa, const uint8_t* xb, int Hp, int sb, int m, uint4& lo,
                                            uint4& hi) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, gB = lane >> 4;
  const int pl = min(col, 2 * kPlanes - 1);
  const uint8_t* row = (pl < kPlanes ? xa + (size_t)pl * Hp : xb + (size_t)(pl - kPlanes) * Hp);
  const int i0 = sb * 256 + 64 * (gB >> 1) + 32 * m + 16 * (gB & 1);
  lo = ld16c(row + i0);
  hi = ld16c(row + i0 + 128);
}
__device__ __forceinline__ v8i digit_operand2(const uint4& lo, const uint4& hi) {
  const int col = threadIdx.x & 15;
  const unsigned keep = col < 2 * kPlanes ? 0xFFFFFFFFu : 0u;
  const unsigned one = col == 2 * kPlanes ? 0x38383838u : 0u;       // FP8 E4M3 1.0
  v8i b;
  b[0] = (lo.x & keep) | one; b[1] = (lo.y & keep) | one; b[2] = (lo.z & keep) | one; b[3] = (lo.w & keep) | one;
  b[4] = (hi.x & keep) | one; b[5] = (hi.y & keep) | one; b[6] = (hi.z & keep) | one; b[7] = (hi.w & keep) | one;
  return b;
}

// Sketch item of row tile q of wavefront wv (q = 0: gate rows of channels
// jw + 0..15, q = 1: their up rows) and super-block s: lane (row = lane & 15,
// g = lane >> 4) takes the 16 bytes at 64 s + 16 g of its row.
__device__ __forceinline__ uint4 sketch_item2(const GArgs& a, int e, int jw, int cwv, int q, int s) {
  const int lane = threadIdx.x & 63;
  const int rowb = a.H / 4;
  const int off = 64 * s + 16 * (lane >> 4);
  const int jj = min(lane & 15, cwv - 1);            // rows past the channels repeat a valid row (never read)
  return ld16((q ? a.tu : a.tg) + ((size_t)e * a.I + jw + jj) * rowb + (off < rowb ? off : 0));
}

// Work item (tile, screen item): channels [j0, j0 + 64) of expert e against up
// to 16 of its tokens, two per pass. Wavefront w owns channels j0 + 16 w ..
// + 15 (its gate and up sketch rows are two MFMA row tiles), so it computes
// their sketch activations and its share of the recovery sums by itself; the
// wavefronts never wait for each other.
template <bool REG>
__global__ __launch_bounds__(GT, 2) void k_g_screen(GArgs a) {
  __shared__ __align__(16) float dsw[4][32 * kDP];       // per wavefront: D of its two row tiles
  __shared__ __align__(16) float hw[4][2 * 16];          // per wavefront: its activations, two tokens
  __shared__ __align__(16) uint16_t btw[4][16 * kRPad];  // per wavefront: Bt rows of its channels
  const int4 wd = a.gwork[blockIdx.y];                     // (requested with the item count: one round trip)
  if ((uint32_t)blockIdx.y >= a.meta[1]) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I, r = a.r;
  const int Hp = max(H, 256);
  const int nsb = (H + 255) / 256;
  const int e = wd.x, q0 = wd.y, n = wd.z;                // expert, its pairs gpl[q0 .. q0 + n - 1]
  const int jw = blockIdx.x * kTile + 16 * wv;             // this wavefront's first channel
  const int cwv = min(16, I - jw);
  if (cwv <= 0) return;
  const int zslot = jw / 16;                               // its recovery-sum slot
  const int row = lane & 15, qe = (lane >> 4) & 1, tk = lane >> 5;   // epilogue: row, gate / up, token
  float* myD = dsw[wv];
  float* myH = hw[wv];
  uint16_t* myB = btw[wv];

  // requests that do not depend on the tokens
  uint4 wa[2][kSbReg];
  if constexpr (REG) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int s = 0; s < kSbReg; ++s) wa[q][s] = sketch_item2(a, e, jw, cwv, q, min(s, nsb - 1));
  }
  const float sc = (qe ? a.su : a.sg)[(size_t)e * I + jw + min(row, cwv - 1)];
  if (r > 0) {
    // Bt rows jw .. jw + cwv - 1 (contiguous): 2 r pieces of 16 bytes at most
    const uint4* src4 = reinterpret_cast<const uint4*>(a.Bt + ((size_t)e * I + jw) * r);
    const int npc = cwv * r / 8;
    uint4 bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = ld16c(src4 + min(lane + 64 * i, npc - 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane + 64 * i;
      if (idx < 2 * r) reinterpret_cast<uint4*>(myB)[idx] = idx < npc ? bv[i] : make_uint4(0, 0, 0, 0);
    }
  }
  for (int q2 = 0; q2 < n; q2 += 2) {
    const int pa = a.gpl[q0 + q2], pb = a.gpl[q0 + min(q2 + 1, n - 1)];
    const int ta = pa / a.K, tb = pb / a.K;
    const uint8_t* xa = a.xd + (size_t)ta * kPlanes * Hp;
    const uint8_t* xb = a.xd + (size_t)tb * kPlanes * Hp;
    const int F0 = a.xf0[tk ? tb : ta];
    v4f acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) acc[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsb; s0 += kSbReg) {
      uint4 wl[2][kSbReg], dlo[kSbReg][2], dhi[kSbReg][2];
#pragma unroll
      for (int u = 0; u < kSbReg; ++u) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if constexpr (REG) wl[q][u] = wa[q][u];
          else wl[q][u] = sketch_item2(a, e, jw, cwv, q, min(s0 + u, nsb - 1));
        }
        digit_load2(xa, xb, Hp, min(s0 + u, nsb - 1), 0, dlo[u][0], dhi[u][0]);
        digit_load2(xa, xb, Hp, min(s0 + u, nsb - 1), 1, dlo[u][1], dhi[u][1]);
      }
#pragma unroll
      for (int u = 0; u < kSbReg; ++u) {
        const int s = s0 + u;
        if (s < nsb) {
          const uint32_t km = 64 * s + 16 * (lane >> 4) < H / 4 ? ~0u : 0u;   // codes past the row end (H < 256)
          const v8i d0 = digit_operand2(dlo[u][0], dhi[u][0]);
          const v8i d1 = digit_operand2(dlo[u][1], dhi[u][1]);
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
    // lane holds D[4 (lane / 16) + v][lane % 16] of each tile; to this wavefront's LDS
    {
      const int col = lane & 15;
      if (col <= 2 * kPlanes) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v) myD[(16 * q + 4 * (lane >> 4) + v) * kDP + col] = acc[q][v];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane (row, qe, tk): the row's scale times its exact integer dot for token
    // tk (as in the per-pair screen); gate lanes pair with the up lane 16 above
    const float* d = myD + (16 * qe + row) * kDP + kPlanes * tk;
    const long long S = (long long)(int)d[0] + ((long long)(int)d[1] << 4) + ((long long)(int)d[2] << 8) +
                        ((long long)(int)d[3] << 12) + ((long long)(int)d[4] << 16) + ((long long)(int)d[5] << 20) -
                        ((long long)(int)myD[(16 * qe + row) * kDP + 2 * kPlanes] << 23);
    const float val = (float)((double)sc * ldexp((double)S, kDShift - F0));
    const float other = __int_as_float(lane_xor<16>(__float_as_int(val)));
    const bool ok = row < cwv && q2 + tk < n;
    if (qe == 0) {
      const float hv = silu_f32(val) * other;
      myH[tk * 16 + row] = ok ? hv : 0.f;
      if (ok) a.hs[(size_t)(tk ? pb : pa) * I + jw + row] = hv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // this wavefront's share of the recovery sums: sum_j hhat_j Bt[j][:]
    for (int idx = lane; idx < 2 * r; idx += 64) {
      const int t2 = idx / r, l = idx % r;
      if (q2 + t2 < n) {
        float z = 0.f;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) z += myH[t2 * 16 + jj] * bf16_to_f32(myB[jj * r + l]);
        a.zp[((size_t)(t2 ? pb : pa) * a.nz + zslot) * r + l] = z;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// The same screen for H <= 2048 with each token pair's digit planes staged
// in LDS once per workgroup (the four wavefronts share them; reading them from
// L2 in every wavefront made the screen L2-bound): the next pair's planes are
// requested before the current pair is multiplied and stored after a barrier
// that follows the multiply (one plane buffer, two barriers per pair).
constexpr int kStgPS = 2048 + 16;                                  // plane pitch in LDS (bytes)
constexpr int kStgPieces = 2 * kPlanes * 2048 / 16 / GT;           // 16-byte pieces per thread and pair

// (H is a power of two: a plane of Hp bytes is 2^lppl pieces of 16 bytes)
__device__ __forceinline__ void stage_load(const GArgs& a, int ta, int tb, int Hp, int lppl, uint4 (&v)[kStgPieces]) {
  const int tid = threadIdx.x;
  const uint8_t* xa = a.xd + (size_t)ta * kPlanes * Hp;
  const uint8_t* xb = a.xd + (size_t)tb * kPlanes * Hp;
#pragma unroll
  for (int u = 0; u < kStgPieces; ++u) {
    const int i = tid + GT * u, pl = min(i >> lppl, 2 * kPlanes - 1), off = i & ((1 << lppl) - 1);   // (pieces past the planes: not stored)
    const uint8_t* src = (pl < kPlanes ? xa : xb) + (size_t)(pl % kPlanes) * Hp + 16 * off;
    v[u] = ld16c(src);
  }
}
__device__ __forceinline__ void stage_store(uint8_t* buf, int lppl, const uint4 (&v)[kStgPieces]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kStgPieces; ++u) {
    const int i = tid + GT * u, pl = i >> lppl, off = i & ((1 << lppl) - 1);
    if (pl < 2 * kPlanes) *reinterpret_cast<uint4*>(buf + pl * kStgPS + 16 * off) = v[u];
  }
}
// B operand of super-block sb, half m, from the staged planes (the layout of
// digit_load2): plane 2 kPlanes of the buffer holds FP8 ones, set once, and
// columns 13..15 read it too (their sums are not used), so the operand needs
// no masking.
__device__ __forceinline__ v8i digit_lds_op(const uint8_t* buf, int sb, int m) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, gB = lane >> 4;
  const int pl = min(col, 2 * kPlanes);
  const uint8_t* row = buf + pl * kStgPS + sb * 256 + 64 * (gB >> 1) + 32 * m + 16 * (gB & 1);
  const uint4 lo = *reinterpret_cast<const uint4*>(row);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + 128);
  v8i b;
  b[0] = (int)lo.x; b[1] = (int)lo.y; b[2] = (int)lo.z; b[3] = (int)lo.w;
  b[4] = (int)hi.x; b[5] = (int)hi.y; b[6] = (int)hi.z; b[7] = (int)hi.w;
  return b;
}

// The item's pair numbers, tokens and scale exponents are read once, one per
// lane, and kept in LDS for the passes; every request is unconditional (a
// wavefront past the last channel requests channels 0 .. 15 and does not use
// them), so no register is cleared while a request to it may be in flight and
// the planes of the next pass stay in flight while the current pass is
// multiplied. Three workgroups fit a CU (160 registers, 52 KB of LDS).
__global__ __launch_bounds__(GT, 3) void k_g_screen_lds(GArgs a) {
  __shared__ __align__(16) float dsw[4][32 * kDP];
  __shared__ __align__(16) float hw[4][2 * 16];
  __shared__ __align__(16) uint16_t btw[4][16 * kRPad];
  __shared__ __align__(16) uint8_t stg[(2 * kPlanes + 1) * kStgPS];
  __shared__ int s_pl[kTokGroup], s_tk[kTokGroup], s_f0[kTokGroup];   // the item's pairs, their tokens, scale exponents
  const int4 wd = a.gwork[blockIdx.y];                     // (requested with the item count: one round trip)
  if ((uint32_t)blockIdx.y >= a.meta[1]) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, I = a.I, r = a.r;
  const int Hp = max(H, 256);
  const int nsb = (H + 255) / 256;                         // <= kSbReg
  const int lppl = max(a.log2H, 8) - 4;                    // log2 of the 16-byte pieces of a plane
  const int e = wd.x, q0 = wd.y, n = wd.z;                // expert, its pairs gpl[q0 .. q0 + n - 1] (n <= 16)
  const int jw = blockIdx.x * kTile + 16 * wv;
  const int cwv = min(16, I - jw);
  const bool active = cwv > 0;                             // (inactive wavefronts still stage and join)
  const int jv = active ? jw : 0, cv = active ? cwv : min(16, I);
  const int zslot = jw / 16;
  const int row = lane & 15, qe = (lane >> 4) & 1, tk = lane >> 5;
  float* myD = dsw[wv];
  float* myH = hw[wv];
  uint16_t* myB = btw[wv];
  const int pl_l = a.gpl[q0 + min(lane, n - 1)];          // lane i: pair i of the item
  const int tk_l = pl_l / a.K;                             // and its token
  uint4 wa[2][kSbReg];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int s = 0; s < kSbReg; ++s) {
      const uint32_t km = 64 * s + 16 * (lane >> 4) < H / 4 ? ~0u : 0u;   // codes past the row end (H < 256)
      const uint4 w = sketch_item2(a, e, jv, cv, q, min(s, nsb - 1));
      wa[q][s] = make_uint4(w.x & km, w.y & km, w.z & km, w.w & km);
    }
  // the ones plane (FP8 E4M3 1.0)
  for (int i = threadIdx.x; i < Hp / 16; i += GT)
    *reinterpret_cast<uint4*>(stg + 2 * kPlanes * kStgPS + 16 * i) = make_uint4(0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u);
  const float sc = (qe ? a.su : a.sg)[(size_t)e * I + jv + min(row, cv - 1)];
  uint4 bv[4];
  if (r > 0) {
    const uint4* src4 = reinterpret_cast<const uint4*>(a.Bt + ((size_t)e * I + jv) * r);
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[i] = ld16c(src4 + min(lane + 64 * i, cv * r / 8 - 1));
  }
  uint4 nx[kStgPieces];
  stage_load(a, __builtin_amdgcn_readlane(tk_l, 0), __builtin_amdgcn_readlane(tk_l, min(1, n - 1)), Hp, lppl, nx);
  const int f0_l = a.xf0[tk_l];                            // lane i: the scale exponent of pair i's token
  if (active && r > 0) {
    // Bt rows jw .. jw + cwv - 1 (contiguous): 2 r pieces of 16 bytes at most
    const int npc = cwv * r / 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane + 64 * i;
      if (idx < 2 * r) reinterpret_cast<uint4*>(myB)[idx] = idx < npc ? bv[i] : make_uint4(0, 0, 0, 0);
    }
  }
  if (threadIdx.x < kTokGroup) {
    s_pl[threadIdx.x] = pl_l;
    s_tk[threadIdx.x] = tk_l;
    s_f0[threadIdx.x] = f0_l;
  }
  stage_store(stg, lppl, nx);
  __syncthreads();
  for (int q2 = 0; q2 < n; q2 += 2) {
    // (from LDS: reading them waits for no request to memory)
    const int pa = __builtin_amdgcn_readfirstlane(s_pl[q2]), pb = __builtin_amdgcn_readfirstlane(s_pl[min(q2 + 1, n - 1)]);
    const int F0a = __builtin_amdgcn_readfirstlane(s_f0[q2]), F0b = __builtin_amdgcn_readfirstlane(s_f0[min(q2 + 1, n - 1)]);
    const bool more = q2 + 2 < n;
    // the next pass's planes (the last pass: the first pair's again, not stored)
    const int qn = more ? q2 + 2 : 0;
    stage_load(a, __builtin_amdgcn_readfirstlane(s_tk[qn]), __builtin_amdgcn_readfirstlane(s_tk[min(qn + 1, n - 1)]), Hp,
               lppl, nx);
    if (active) {
      // (the sketch words are opaque to the compiler here: it converts them on
      // every pass instead of keeping converted copies live across the loop)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int s = 0; s < kSbReg; ++s)
          asm volatile("" : "+v"(wa[q][s].x), "+v"(wa[q][s].y), "+v"(wa[q][s].z), "+v"(wa[q][s].w));
      const uint8_t* sb8 = stg;
      v4f acc[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSbReg; ++s) {
        if (s < nsb) {
          const v8i d0 = digit_lds_op(sb8, s, 0);
          const v8i d1 = digit_lds_op(sb8, s, 1);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(wa[q][s].x, wa[q][s].y), d0, acc[q],
                                                                      4, 0, 0, 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(wa[q][s].z, wa[q][s].w), d1, acc[q],
                                                                      4, 0, 0, 0, 0, 0);
          }
        }
      }
      {
        const int col = lane & 15;
        if (col <= 2 * kPlanes) {
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) myD[(16 * q + 4 * (lane >> 4) + v) * kDP + col] = acc[q][v];
        }
      }
    }
    // one plane buffer: the next pass's planes go in once every wavefront has
    // multiplied (the activations below do not read the planes)
    if (more) {
      __syncthreads();
      stage_store(stg, lppl, nx);
    }
    if (active) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // lane (row, qe, tk): the row's scale times its exact integer dot for
      // token tk (as in the per-pair screen); gate lanes pair with the up lane 16 above
      const int F0 = tk ? F0b : F0a;
      const float* d = myD + (16 * qe + row) * kDP + kPlanes * tk;
      const long long S = (long long)(int)d[0] + ((long long)(int)d[1] << 4) + ((long long)(int)d[2] << 8) +
                          ((long long)(int)d[3] << 12) + ((long long)(int)d[4] << 16) + ((long long)(int)d[5] << 20) -
                          ((long long)(int)myD[(16 * qe + row) * kDP + 2 * kPlanes] << 23);
      const float val = (float)((double)sc * ldexp((double)S, kDShift - F0));
      const float other = __int_as_float(lane_xor<16>(__float_as_int(val)));
      const bool ok = row < cwv && q2 + tk < n;
      if (qe == 0) {
        const float hv = silu_f32(val) * other;
        myH[tk * 16 + row] = ok ? hv : 0.f;
        if (ok) a.hs[(size_t)(tk ? pb : pa) * I + jw + row] = hv;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // this wavefront's share of the recovery sums: sum_j hhat_j Bt[j][:]
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        if (q2 + t2 < n) {
          for (int l = lane; l < r; l += 64) {
            float z = 0.f;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) z += myH[t2 * 16 + jj] * bf16_to_f32(myB[jj * r + l]);
            a.zp[((size_t)(t2 ? pb : pa) * a.nz + zslot) * r + l] = z;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ stage 3: top-c

template <int KPT>
__global__ __launch_bounds__(GT) void k_g_topc(GArgs a) {
  __shared__ __align__(16) uint32_t tks[kTopkScratchWords];
  __shared__ __align__(16) int32_t cand[kMaxI];
  __shared__ __align__(16) uint32_t bm[kMaxI / 32];
  __shared__ __align__(16) uint32_t pc[kMaxI / 32];
  __shared__ uint32_t wtot[4];
  __shared__ int s_flag;
  __shared__ uint32_t s_base;
  const int p = blockIdx.x, tid = threadIdx.x;
  const int I = a.I, c = a.c;
  const int e = min(max(a.ids[p], 0), a.E - 1);
  int cnt;
  const int i0 = topk_range<GT>(I, &cnt);
  uint32_t kr[KPT];
  const float* src = a.hs + (size_t)p * I + i0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) kr[j] = j < cnt && !a.nosk ? score_key(src[j]) : 0u;
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
  for (int w = tid; w < a.IW; w += GT) st_u(a.cm + (size_t)p * a.IW + w, bm[w]);
  // the last pair of the expert lists the candidate union and queues its exact work
  if (!arrive_last(a.uctr + e, (uint32_t)(a.goff[e + 1] - a.goff[e]), &s_flag)) return;
  const int u = a.gux[e];
  const uint32_t nU = expert_union(a, a.cm, e, a.urows + (size_t)u * a.IP, bm, pc, wtot);
  const uint32_t nb = (nU + kRowBlk - 1) / kRowBlk;
  if (tid == 0) {
    a.ucnt[u] = nU;
    s_base = atomicAdd(a.meta + 2, nb);
  }
  __syncthreads();
  for (uint32_t b = tid; b < nb; b += GT) a.gexw[s_base + b] = (int)(((uint32_t)u << 16) | b);
}

// ------------------------------------------------------------------ stage 4: exact gate / up

// Work items (64-row block, used expert): union rows [64 b, 64 b + 64) of the
// expert's candidate union (every channel when dense) over the whole hidden
// width, against all of its tokens. Wavefront w takes rows 64 b + 16 w .. + 15
// (one MFMA row tile) and up to 64 tokens (four MFMA column tiles) per pass over
// the rows, so a row is read once per 64 tokens. The tokens' x for one batch of
// KC 32-element steps is staged in LDS and shared by the four wavefronts
// (double-buffered, one barrier per batch); the next batch's gate / up rows and
// x are requested before the current batch is multiplied. A persistent loop
// walks the work list.
template <int KC>
struct ExactRows {
  uint4 g[KC], u[KC];
};
template <int KC>
__device__ __forceinline__ void exact_rows_load(ExactRows<KC>& b, const uint16_t* wgr, const uint16_t* wur, int kb,
                                                int nbat) {
  const int k0 = 32 * KC * min(kb, nbat - 1);        // past the end: the last batch again (not multiplied)
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    b.g[i] = ld16(wgr + k0 + 32 * i);
    b.u[i] = ld16(wur + k0 + 32 * i);
  }
}
// x of this pass's tokens for batch kb: piece f = tid + 256 v is token f / (4 KC),
// 16-byte part f % (4 KC); tokens past the pass repeat its last token.
template <int KC>
__device__ __forceinline__ void exact_x_load(uint4 (&xv)[KC], const GArgs& a, const int* tok, int ntk, int kb,
                                             int nbat) {
  const int k0 = 32 * KC * min(kb, nbat - 1);
#pragma unroll
  for (int v = 0; v < KC; ++v) {
    const int f = threadIdx.x + GT * v, m = f / (4 * KC), pc = f % (4 * KC);
    xv[v] = ld16c(a.x + (size_t)tok[min(m, ntk - 1)] * a.H + k0 + 8 * pc);
  }
}
template <int KC>
__device__ __forceinline__ void exact_x_store(const uint4 (&xv)[KC], uint16_t* xb) {
#pragma unroll
  for (int v = 0; v < KC; ++v) {
    const int f = threadIdx.x + GT * v, m = f / (4 * KC), pc = f % (4 * KC);
    *reinterpret_cast<uint4*>(xb + m * (32 * KC + 8) + 8 * pc) = xv[v];
  }
}
template <int KC>
__device__ __forceinline__ void exact_rows_mul(const ExactRows<KC>& b, const uint16_t* xb, int ngrp, v4f (&ag)[4],
                                               v4f (&au)[4]) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < ngrp) {
      const uint16_t* xr = xb + (16 * q + col) * (32 * KC + 8) + 8 * g;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const uint4 xq = *reinterpret_cast<const uint4*>(xr + 32 * i);
        ag[q] = mfma_bf16(b.g[i], xq, ag[q]);
        au[q] = mfma_bf16(b.u[i], xq, au[q]);
      }
    }
  }
}

template <int KC>
__global__ __launch_bounds__(GT, 2) void k_g_exact(GArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* xs0 = reinterpret_cast<uint16_t*>(smem);                     // [64][32 KC + 8]
  uint16_t* xs1 = xs0 + 64 * (32 * KC + 8);
  __shared__ int tok[64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I;
  const uint32_t nwork = a.dense ? a.meta[0] * (uint32_t)a.nrb : a.meta[2];
  const int row = lane & 15, g = lane >> 4;
  const int nbat = H / (32 * KC);
  for (uint32_t wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
    int u, b;
    if (a.dense) { u = (int)(wi / a.nrb); b = (int)(wi % a.nrb); }
    else { const int it = a.gexw[wi]; u = it >> 16; b = it & 0xFFFF; }
    const int e = a.gue[u];
    const int p0 = a.goff[e], n = a.goff[e + 1] - p0;
    const int nU = a.dense ? I : (int)a.ucnt[u];
    const int r0 = kRowBlk * b + 16 * wv;
    const int nrow = min(16, nU - r0);                  // rows of this wavefront (may be <= 0)
    const int q = min(r0 + row, nU - 1);
    const int j = a.dense ? q : a.urows[(size_t)u * a.IP + q];
    const uint16_t* wgr = a.wg + ((size_t)e * I + j) * H + 8 * g;
    const uint16_t* wur = a.wu + ((size_t)e * I + j) * H + 8 * g;
    const int32_t* pl = a.gpl + p0;
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int ntk = min(64, n - s0), ngrp = (ntk + 15) / 16;
      __syncthreads();                                   // the previous pass is done with tok and the x buffers
      if (tid < 64) tok[tid] = pl[s0 + min(tid, ntk - 1)] / a.K;
      __syncthreads();
      v4f ag[4], au[4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) { ag[qq] = (v4f){0.f, 0.f, 0.f, 0.f}; au[qq] = ag[qq]; }
      ExactRows<KC> A, B;
      uint4 xv[KC];
      // x is requested before the rows of the same batch: loads complete in
      // order, so storing x to LDS waits for x only and the rows stay in
      // flight across the barrier (two batches of rows outstanding)
      exact_x_load(xv, a, tok, ntk, 0, nbat);
      exact_rows_load(A, wgr, wur, 0, nbat);
      exact_x_store(xv, xs0);
      __syncthreads();
      for (int kb = 0; kb < nbat; kb += 2) {
        exact_x_load(xv, a, tok, ntk, kb + 1, nbat);
        exact_rows_load(B, wgr, wur, kb + 1, nbat);
        exact_rows_mul(A, xs0, ngrp, ag, au);
        exact_x_store(xv, xs1);
        __syncthreads();
        exact_x_load(xv, a, tok, ntk, kb + 2, nbat);
        exact_rows_load(A, wgr, wur, kb + 2, nbat);
        if (kb + 1 < nbat) exact_rows_mul(B, xs1, ngrp, ag, au);
        exact_x_store(xv, xs0);
        __syncthreads();
      }
      // lane holds D[4 g + v][lane % 16] of token tile qq: rows r0 + 4 g + v, token slot s0 + 16 qq + lane % 16
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (qq < ngrp) {
          const int s = s0 + 16 * qq + row;
          const int pp = pl[min(s, n - 1)];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int rr = 4 * g + v;
            const int jr = __shfl(j, rr, 64);
            if (rr < nrow && s < n) {
              const float h = silu_f32(ag[qq][v]) * au[qq][v];
              if (a.dense) a.hk[(size_t)pp * I + jr] = f32_to_bf16(h);
              else a.hx[(size_t)pp * I + jr] = h;
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ stage 5: top-k and recovery coefficients

template <int KPT>
__global__ __launch_bounds__(GT) void k_g_topk(GArgs a) {
  __shared__ __align__(16) uint32_t tks[kTopkScratchWords];
  __shared__ __align__(16) int32_t sel[kMaxI];
  __shared__ __align__(16) uint16_t hrow[kMaxI];
  __shared__ __align__(16) uint32_t bm[kMaxI / 32];
  __shared__ __align__(16) uint32_t pc[kMaxI / 32];
  __shared__ __align__(16) float zpart[GT * 8];
  __shared__ uint32_t wtot[4];
  __shared__ int s_flag;
  const int p = blockIdx.x, tid = threadIdx.x;
  const int I = a.I, c = a.c, k = a.k, r = a.r;
  const int e = min(max(a.ids[p], 0), a.E - 1);
  const int32_t* cl = a.cl + (size_t)p * c;
  int kk = k;                                     // |S| (the threshold rule's count varies by pair)
  if (k > 0) {
    int cnt;
    const int i0 = topk_range<GT>(c, &cnt);
    int jc[KPT];
    uint32_t kr[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) jc[j] = cl[min(i0 + j, c - 1)];
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = score_key(a.hx[(size_t)p * I + jc[j]]);
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = j < cnt ? kr[j] : 0u;
    if (a.thr)
      kk = block_threshold<GT>([&](int i) { return score_key(a.hx[(size_t)p * I + cl[i]]); }, i0, cnt, a.tkey,
                               sel, tks);
    else block_topk<GT, KPT>(kr, i0, cnt, c, k, sel, tks);
  }
  if (a.thr && a.keep_count && tid == 0) a.keep_count[p] = kk;
  for (int i = tid; i < I; i += GT) hrow[i] = 0;
  for (int w = tid; w < a.IW; w += GT) bm[w] = 0;
  __syncthreads();
  for (int i = tid; i < k; i += GT) {
    if (i >= kk) {
      if (a.keep_out) a.keep_out[(size_t)p * k + i] = -1;
      continue;
    }
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
  for (int w = tid; w < a.IW; w += GT) st_u(a.km + (size_t)p * a.IW + w, bm[w]);
  // z = sum over all channels of hhat_j Bt[j] (the screen's tile sums) minus the
  // kept channels' terms (with dropped candidates recovered exactly: minus
  // (hhat_j - h_j) Bt[j] for each of them too). Thread (cc, gi): 8 columns
  // 8 cc .. 8 cc + 7, rows and tiles gi, gi + groups, ... (loads in batches of four)
  if (r > 0) {
    const int npr = r / 8, groups = GT / npr;
    const int cc = tid % npr, gi = tid / npr;
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.f;
    if (gi < groups) {
      const float* zs = a.zp + (size_t)p * a.nz * r + 8 * cc;
      for (int t0 = gi; t0 < (a.nosk ? 0 : a.nz); t0 += 4 * groups) {
        float4 z4[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = min(t0 + u * groups, a.nz - 1);
          z4[u][0] = *reinterpret_cast<const float4*>(zs + (size_t)t * r);
          z4[u][1] = *reinterpret_cast<const float4*>(zs + (size_t)t * r + 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (t0 + u * groups < a.nz) {
            acc[0] += z4[u][0].x; acc[1] += z4[u][0].y; acc[2] += z4[u][0].z; acc[3] += z4[u][0].w;
            acc[4] += z4[u][1].x; acc[5] += z4[u][1].y; acc[6] += z4[u][1].z; acc[7] += z4[u][1].w;
          }
        }
      }
      const float* hsp = a.hs + (size_t)p * I;
      const float* hxp = a.hx + (size_t)p * I;
      const int nzr = a.rec_exact ? c : kk;         // terms taken out of the screen's sum
      for (int i0 = gi; i0 < nzr; i0 += 4 * groups) {
        uint4 bw[4];
        float hv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = min(i0 + u * groups, nzr - 1);
          const int j = a.rec_exact ? cl[i] : sel[i];
          bw[u] = ld16c(a.Bt + ((size_t)e * I + j) * r + 8 * cc);
          const bool dropped = a.rec_exact && !((bm[j >> 5] >> (j & 31)) & 1u);
          hv[u] = (a.nosk ? 0.f : hsp[j]) - (dropped ? hxp[j] : 0.f);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float h = i0 + u * groups < nzr ? -hv[u] : 0.f;
          acc[0] += h * bf16lo(bw[u].x); acc[1] += h * bf16hi(bw[u].x);
          acc[2] += h * bf16lo(bw[u].y); acc[3] += h * bf16hi(bw[u].y);
          acc[4] += h * bf16lo(bw[u].z); acc[5] += h * bf16hi(bw[u].z);
          acc[6] += h * bf16lo(bw[u].w); acc[7] += h * bf16hi(bw[u].w);
        }
      }
    }
    if (gi < groups) {
#pragma unroll
      for (int v = 0; v < 8; ++v) zpart[gi * r + 8 * cc + v] = acc[v];
    }
    __syncthreads();
    if (tid < r) {
      float s = 0.f;
      for (int q = 0; q < groups; ++q) s += zpart[q * r + tid];
      a.zf[(size_t)p * r + tid] = s;
    }
  }
  // the last pair of the expert lists the kept union
  if (!arrive_last(a.kctr + e, (uint32_t)(a.goff[e + 1] - a.goff[e]), &s_flag)) return;
  const int u = a.gux[e];
  const uint32_t nU = expert_union(a, a.km, e, a.drows + (size_t)u * a.IP, bm, pc, wtot);
  if (tid == 0) a.dcnt[u] = nU;
}

// ------------------------------------------------------------------ stage 6: down projection, A z, combine

// Work item (column tile, used expert): output columns [64 b, 64 b + 64) of all
// of the expert's tokens, 16 tokens at a time. D = tokens x columns, one MFMA
// column tile per 16 output columns. Wavefront w takes the 32-row chunks
// w, w + 4, ... of the expert's kept-union rows (every row when dense): it
// requests the next chunk, stores the current one row-major in its own LDS
// (one 16-byte write per lane) and gathers each lane's eight consecutive
// contraction indices with 16-bit reads, then multiplies, with no barrier; the
// four partial tiles are summed at the end. The 16-byte column blocks of row
// rho sit at block ^ 2 ((rho >> 3) & 3), which keeps both the row writes and
// the column gathers free of bank conflicts. The recovery term z A^T of column
// tile w is computed by wavefront w.
constexpr int kDnP = 40;           // LDS pitch (BF16) of a wavefront's [token][row] activation chunk

__device__ __forceinline__ int dn_swz(int rho, int blk) {      // BF16 offset of block blk of chunk row rho
  return rho * kColTile + 8 * (blk ^ (2 * ((rho >> 3) & 3)));
}

struct DownChunk {
  uint4 w[4];        // down-row pieces: row (lane >> 3) + 8 i, columns 8 (lane & 7) .. + 7
  uint16_t h[8];     // masked activations: token (lane + 64 i) >> 5, row (lane + 64 i) & 31
};

__device__ __forceinline__ void down_load(DownChunk& d, const GArgs& a, int e, int c0, const uint16_t* rows,
                                          const int* pls, int q0, int nr) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = q0 + min((lane >> 3) + 8 * i, nr - 1);
    const int jr = a.dense ? q : rows[q];
    d.w[i] = ld16(a.wd + ((size_t)e * a.I + jr) * a.H + c0 + 8 * (lane & 7));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = lane + 64 * i, m = idx >> 5;
    const int q = q0 + min(idx & 31, nr - 1);
    d.h[i] = a.hk[(size_t)pls[m] * a.I + (a.dense ? q : rows[q])];
  }
}

__global__ __launch_bounds__(GT, 2) void k_g_down(GArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* rows = reinterpret_cast<uint16_t*>(smem);          // [IP] kept-union rows (selected layer)
  __shared__ __align__(16) uint16_t wT[4][32 * kColTile];     // per wavefront: [row][column] (swizzled); then its partial tile
  __shared__ __align__(16) uint16_t hA[4][16 * kDnP];         // per wavefront: [token][row]
  __shared__ int pls[16];
  __shared__ int lastt[16];
  const int u = blockIdx.y;
  if ((uint32_t)u >= a.meta[0]) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, I = a.I, r = a.r, K = a.K;
  const int e = a.gue[u];
  const int p0 = a.goff[e], n = a.goff[e + 1] - p0;
  const int c0 = kColTile * blockIdx.x;
  const int nct = H / kColTile;
  const int nU = a.dense ? I : (int)a.dcnt[u];
  if (!a.dense) {
    // the kept-union rows of the expert, staged once
    const uint4* src = reinterpret_cast<const uint4*>(a.drows + (size_t)u * a.IP);
    const int n8 = (nU + 7) / 8;
    for (int b0 = 0; b0 < n8; b0 += 4 * GT) {
      uint4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = src[min(b0 + tid + GT * q, max(n8 - 1, 0))];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (b0 + tid + GT * q < n8) reinterpret_cast<uint4*>(rows)[b0 + tid + GT * q] = v[q];
    }
  }
  const int m16 = lane & 15, g = lane >> 4;
  const int nch = (nU + 31) / 32;
  uint16_t* myT = wT[wv];
  uint16_t* myA = hA[wv];
  for (int s0 = 0; s0 < n; s0 += 16) {
    const int nt = min(16, n - s0);
    if (tid < 16) pls[tid] = a.gpl[p0 + s0 + min(tid, nt - 1)];
    __syncthreads();
    v4f acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    // recovery, column tile wv: D += z (tokens x r) A[e]^T (r x columns)
    v4f accr = {0.f, 0.f, 0.f, 0.f};
    if (r > 0 && !a.dense) {
      const uint16_t* arow = a.A + ((size_t)e * H + c0 + 16 * wv + m16) * r;
      const float* zrow = a.zf + (size_t)pls[m16] * r;
      for (int ks = 0; ks < (r + 31) / 32; ++ks) {
        const int l0 = 32 * ks + 8 * g;
        const bool ok = l0 < r && m16 < nt;
        const int lc = min(l0, r - 8);
        const uint4 bq = ld16c(arow + lc);
        const float4 z0 = *reinterpret_cast<const float4*>(zrow + lc);
        const float4 z1 = *reinterpret_cast<const float4*>(zrow + lc + 4);
        const uint4 av = ok ? make_uint4(pack_bf16x2(z0.x, z0.y), pack_bf16x2(z0.z, z0.w), pack_bf16x2(z1.x, z1.y),
                                         pack_bf16x2(z1.z, z1.w))
                            : make_uint4(0, 0, 0, 0);
        accr = mfma_bf16(av, l0 < r ? bq : make_uint4(0, 0, 0, 0), accr);
      }
    }
    if (wv < nch) {
      // chunk ch of this wavefront into its LDS (rows past the union: zeros), then multiplied;
      // the next chunk is requested before the current one is multiplied
      auto mul_chunk = [&](const DownChunk& d, int ch) {
        const int nr = min(32, nU - 32 * ch);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rho = (lane >> 3) + 8 * i;
          *reinterpret_cast<uint4*>(myT + dn_swz(rho, lane & 7)) = rho < nr ? d.w[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int idx = lane + 64 * i, m = idx >> 5, rho = idx & 31;
          myA[m * kDnP + rho] = (m < nt && rho < nr) ? d.h[i] : (uint16_t)0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint4 av = *reinterpret_cast<const uint4*>(myA + m16 * kDnP + 8 * g);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          // column 16 ct + m16, rows 8 g .. 8 g + 7
          const uint16_t* col = myT + dn_swz(8 * g, 2 * ct + (m16 >> 3)) + (m16 & 7);
          uint32_t b2[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            b2[s2] = (uint32_t)col[2 * s2 * kColTile] | ((uint32_t)col[(2 * s2 + 1) * kColTile] << 16);
          acc[ct] = mfma_bf16(av, make_uint4(b2[0], b2[1], b2[2], b2[3]), acc[ct]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
      DownChunk cur, nxt;
      down_load(cur, a, e, c0, rows, pls, 32 * wv, min(32, nU - 32 * wv));
      for (int ch = wv; ch < nch; ch += 4) {
        const int cn = ch + 4 < nch ? ch + 4 : ch;          // (past the end: a repeat, not used)
        down_load(nxt, a, e, c0, rows, pls, 32 * cn, min(32, nU - 32 * cn));
        mul_chunk(cur, ch);
        cur = nxt;
      }
    }
    // partial tiles of the four wavefronts (each into its own transpose buffer,
    // which it no longer needs): lane holds D[4 g + v][m16] of column tile ct
    float* myR = reinterpret_cast<float*>(myT);                // [token][column]
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v4f d = ct == wv ? acc[ct] + accr : acc[ct];
#pragma unroll
      for (int v = 0; v < 4; ++v) myR[(4 * g + v) * kColTile + 16 * ct + m16] = d[v];
    }
    __syncthreads();
    {
      const int m = tid >> 4, cq = 4 * (tid & 15);
      if (m < nt) {
        float4 y = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(wT[0]) + m * kColTile + cq);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float4 t4 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(wT[w]) + m * kColTile + cq);
          y.x += t4.x; y.y += t4.y; y.z += t4.z; y.w += t4.w;
        }
        float* dst = a.yp + (size_t)pls[m] * H + c0 + cq;
        st_f(dst, y.x); st_f(dst + 1, y.y); st_f(dst + 2, y.z); st_f(dst + 3, y.w);
      }
    }
    // arrivals per (token, column tile); the last of a token's K pairs combines it
    drain_and_join();
    if (tid < 16) {
      int last = 0;
      if (tid < nt) {
        const int t = pls[tid] / K;
        uint32_t* ctr = a.octr + (size_t)t * nct + blockIdx.x;
        const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (uint32_t)K - 1;
        if (last) st_u(ctr, 0u);
      }
      lastt[tid] = last;
    }
    __syncthreads();
    for (int m = 0; m < nt; ++m) {
      if (!lastt[m]) continue;
      const int t = pls[m] / K;
      if (tid < kColTile) {
        float sum = 0.f;
        for (int q0 = 0; q0 < K; q0 += 8) {
          float yv[8], wq[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int qc = min(q0 + q, K - 1);
            yv[q] = ld_f(a.yp + ((size_t)t * K + qc) * H + c0 + tid);
            wq[q] = a.topk_w[(size_t)t * K + qc];
          }
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (q0 + q < K) sum += wq[q] * yv[q];
        }
        if (a.resid) sum += bf16_to_f32(a.resid[(size_t)t * H + c0 + tid]);
        a.out[(size_t)t * H + c0 + tid] = f32_to_bf16(sum);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ stage 0 (envelope): router

// The decode-layer envelope ahead of the grouped pass. Workgroup (t, b)
// normalises token t (every workgroup of the token forms the same bits; the
// first writes them out), computes the router logits of experts
// [64 b, 64 b + 64) (16 per wavefront, one row each at a time) and stores
// them; the last of the token's workgroups to finish reads its E logits and
// forms the routing (softmax, top-K slot order, weights). The same helpers as
// the per-pair kernel's envelope, so both passes route identically.
struct RouteArgs {
  const uint16_t *h, *gamma, *wr;
  float eps;
  int renorm, T, K, E, H, nb;
  uint16_t* xw;        // [T][H] normalised states (BF16)
  float* lg;           // [T][E] logits
  int32_t* ids;        // [T][K] routing, slot order
  float* w;            // [T][K] weights
  uint32_t* rctr;      // [T] arrivals (zero between calls)
  int32_t* ids_out;
  float* w_out;
  uint16_t* x_out;
};
constexpr int kRouteRows = 64;

__global__ __launch_bounds__(GT) void k_g_route(RouteArgs a) {
  __shared__ __align__(16) uint16_t xb[kMaxH];
  __shared__ __align__(16) float rl[kEnvMaxE];
  __shared__ __align__(16) float red[8];
  __shared__ __align__(16) uint32_t tks[kTopkScratchWords];
  __shared__ int32_t rida[kMaxK], rid[kMaxK];
  __shared__ float rw[kMaxK];
  __shared__ int s_flag;
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, K = a.K, nch = H / 8;
  env_normalise(a.h + (size_t)t * H, a.gamma, H, a.eps, xb, red);
  if (b == 0)
    for (int ci = tid; ci < nch; ci += GT) {
      const uint4 v = reinterpret_cast<const uint4*>(xb)[ci];
      reinterpret_cast<uint4*>(a.xw + (size_t)t * H)[ci] = v;
      if (a.x_out) reinterpret_cast<uint4*>(a.x_out + (size_t)t * H)[ci] = v;
    }
  const uint4 none[1] = {make_uint4(0, 0, 0, 0)};
  for (int j = wv; j < kRouteRows; j += GT / 64) {
    const int e = b * kRouteRows + j;
    if (e < E) {
      const float d = env_logit<1>(a.wr + (size_t)e * H, xb, H, none, false);
      if (lane == 0) st_f(a.lg + (size_t)t * E + e, d);
    }
  }
  if (!arrive_last(a.rctr + t, (uint32_t)a.nb, &s_flag)) return;
  for (int i = tid; i < E; i += GT) rl[i] = ld_f(a.lg + (size_t)t * E + i);
  env_pick(rl, E, K, a.renorm, rida, rid, rw, red, tks);
  if (tid < K) {
    a.ids[(size_t)t * K + tid] = rid[tid];
    a.w[(size_t)t * K + tid] = rw[tid];
    if (a.ids_out) a.ids_out[(size_t)t * K + tid] = rid[tid];
    if (a.w_out) a.w_out[(size_t)t * K + tid] = rw[tid];
  }
}

// ------------------------------------------------------------------ stats

__global__ void k_g_stats(GArgs a, cfm_stats* st) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const uint32_t nue = a.meta[0];
  uint64_t uc = 0, dc = 0;
  if (!a.dense) {
    for (uint32_t u = 0; u < nue; ++u) {
      uc += a.ucnt[u];
      dc += a.dcnt[u];
    }
    if (a.k == 0 && !a.rec_exact) uc = 0;       // no exact phase ran
  } else {
    uc = dc = (uint64_t)nue * a.I;
  }
  const uint64_t I = a.I, H = a.H, r = a.r;
  cfm_stats s;
  s.bytes_io = 2ull * a.T * H + 8ull * a.T * a.K + 2ull * a.T * H;
  s.bytes_dense_equiv = (uint64_t)nue * 6ull * I * H + s.bytes_io;
  s.experts_used = nue;
  s.bytes_sketch = (a.dense || a.nosk) ? 0 : (uint64_t)nue * (2ull * I * (H / 4) + 8ull * I);
  s.bytes_candidates = 4ull * H * uc;
  s.bytes_down = 2ull * H * dc;
  s.bytes_recovery = (a.dense || r == 0) ? 0 : (uint64_t)nue * (2ull * H * r + 2ull * I * r);
  s.rows_candidates = (uint32_t)uc;
  s.rows_down = (uint32_t)dc;
  s.pad = 0;
  s.bytes_requested = s.bytes_sketch + s.bytes_candidates + s.bytes_down + s.bytes_recovery + s.bytes_io;
  *st = s;
}

// ------------------------------------------------------------------ host side

size_t prep_lds(int H, int E) {
  const size_t Hp = std::max(H, 256);
  return std::max(10 * Hp, (size_t)16 * E);
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
  g.nrb = (I + kRowBlk - 1) / kRowBlk;
  g.IP = (I + 7) / 8 * 8;
  g.maxu = std::min(E, g.P);
  g.maxwork = g.maxu + (g.P + kTokGroup - 1) / kTokGroup;
  const size_t P = (size_t)g.P, Hp = std::max(H, 256), U = (size_t)g.maxu;
  Carve cv;
  cv.off = base;
  // counters that must read zero between calls come first
  g.off_uctr = cv.take(4 * (size_t)E);
  g.off_kctr = cv.take(4 * (size_t)E);
  g.off_octr = cv.take(4 * (size_t)T * (H / kColTile));
  g.off_rctr = cv.take(4 * (size_t)std::max(T, 1));
  g.off_meta = cv.take(16);
  g.off_goff = cv.take(4 * ((size_t)E + 1));
  g.off_gpl = cv.take(4 * P);
  g.off_gue = cv.take(4 * (size_t)E);
  g.off_gux = cv.take(4 * (size_t)E);
  g.off_gwork = cv.take(16 * (size_t)g.maxwork);
  g.off_gexw = cv.take(dense ? 16 : 4 * U * g.nrb);
  g.off_xf0 = cv.take(4 * (size_t)T);
  g.off_xd = cv.take(dense ? 16 : (size_t)T * kPlanes * Hp);
  g.off_hs = cv.take(dense ? 16 : P * I * 4);
  g.off_zp = cv.take(dense || r == 0 ? 16 : P * (size_t)((I + 15) / 16) * r * 4);
  g.off_cm = cv.take(dense ? 16 : P * g.IW * 4);
  g.off_cl = cv.take(dense ? 16 : P * std::max(c, 1) * 4);
  g.off_hx = cv.take(dense ? 16 : P * I * 4);
  g.off_km = cv.take(dense ? 16 : P * g.IW * 4);
  g.off_hk = cv.take(P * I * 2);
  g.off_zf = cv.take(dense || r == 0 ? 16 : P * r * 4);
  g.off_yp = cv.take(P * H * 4);
  g.off_ucnt = cv.take(4 * U);
  g.off_dcnt = cv.take(4 * U);
  g.off_urows = cv.take(2 * U * g.IP);
  g.off_drows = cv.take(2 * U * g.IP);
  g.off_xw = cv.take(2 * (size_t)T * H);
  g.off_lg = cv.take(4 * (size_t)T * E);
  g.off_idw = cv.take(4 * (size_t)T * K);
  g.off_ww = cv.take(4 * (size_t)T * K);
  g.bytes = cv.off;
  return g;
}

// The pass's arguments from the call and the plan (routing fields aside).
static void fill_args(GArgs& a, const SelectArgs& s, const GroupPlan& g) {
  a.wg = s.w_gate; a.wu = s.w_up; a.wd = s.w_down_t;
  a.signs = s.signs; a.tg = s.tg; a.tu = s.tu; a.sg = s.sg; a.su = s.su;
  a.A = s.A; a.Bt = s.Bt;
  a.out = s.out; a.cand_out = s.cand_out; a.keep_out = s.keep_out;
  char* ws = s.ws;
  a.meta = reinterpret_cast<uint32_t*>(ws + g.off_meta);
  a.goff = reinterpret_cast<int32_t*>(ws + g.off_goff);
  a.gpl = reinterpret_cast<int32_t*>(ws + g.off_gpl);
  a.gue = reinterpret_cast<int32_t*>(ws + g.off_gue);
  a.gux = reinterpret_cast<int32_t*>(ws + g.off_gux);
  a.gwork = reinterpret_cast<int4*>(ws + g.off_gwork);
  a.gexw = reinterpret_cast<int32_t*>(ws + g.off_gexw);
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
  a.urows = reinterpret_cast<uint16_t*>(ws + g.off_urows);
  a.drows = reinterpret_cast<uint16_t*>(ws + g.off_drows);
  a.uctr = reinterpret_cast<uint32_t*>(ws + g.off_uctr);
  a.kctr = reinterpret_cast<uint32_t*>(ws + g.off_kctr);
  a.octr = reinterpret_cast<uint32_t*>(ws + g.off_octr);
  a.T = g.T; a.K = g.K; a.P = g.P; a.E = g.E; a.I = g.I; a.H = g.H;
  int log2H = 0;
  while ((1 << log2H) < g.H) ++log2H;
  a.log2H = log2H;
  a.k = g.dense ? g.I : g.k; a.c = g.dense ? g.I : g.c; a.r = g.dense ? 0 : g.r;
  a.ntile = g.ntile; a.nz = (g.I + 15) / 16; a.IW = g.IW; a.nrb = g.nrb; a.IP = g.IP; a.dense = g.dense ? 1 : 0;
  a.rec_exact = !g.dense && (s.flags & CFM_RECOVER_CANDIDATES_EXACT) ? 1 : 0;
  a.nosk = a.rec_exact && g.c >= g.I ? 1 : 0;
  a.thr = !g.dense && s.thr ? 1 : 0;
  a.tkey = s.tkey;
  a.keep_count = s.keep_count;
}

// The router stage of the decode-layer envelope: x = RMSNorm(resid) into the
// plan's xw region and the routing into idw / ww (and the optional outputs).
int launch_grouped_route(const SelectArgs& s, const GroupPlan& g, hipStream_t stream) {
  RouteArgs ra{};
  ra.h = s.resid; ra.gamma = s.gamma; ra.wr = s.wr; ra.eps = s.eps; ra.renorm = s.renorm;
  ra.T = g.T; ra.K = g.K; ra.E = g.E; ra.H = g.H; ra.nb = (g.E + kRouteRows - 1) / kRouteRows;
  ra.xw = reinterpret_cast<uint16_t*>(s.ws + g.off_xw);
  ra.lg = reinterpret_cast<float*>(s.ws + g.off_lg);
  ra.ids = reinterpret_cast<int32_t*>(s.ws + g.off_idw);
  ra.w = reinterpret_cast<float*>(s.ws + g.off_ww);
  ra.rctr = reinterpret_cast<uint32_t*>(s.ws + g.off_rctr);
  ra.ids_out = s.ids_out; ra.w_out = s.w_out; ra.x_out = s.x_out;
  timing_begin("k_g_route", stream);
  hipLaunchKernelGGL(k_g_route, dim3(g.T, ra.nb), dim3(GT), 0, stream, ra);
  timing_end(stream);
  CFM_LAUNCH_CHECK("k_g_route");
  return CFM_OK;
}

int launch_grouped_forward(const SelectArgs& s, const GroupPlan& g, hipStream_t stream) {
  if (int rc = prepare_workspace(s.ws, g.bytes,
                                 layout_signature({3, g.T, g.K, g.E, g.I, g.H, g.k, g.c, g.r, g.dense ? 1 : 0,
                                                   s.resid ? 1 : 0, (long)g.bytes}),
                                 stream))
    return rc;
  GArgs a{};
  a.x = s.x; a.ids = s.ids; a.topk_w = s.topk_w;
  if (s.resid) {
    // decode-layer envelope: the router first; the pass then reads the
    // normalised states and the routing it wrote, and adds the residual
    if (int rc = launch_grouped_route(s, g, stream)) return rc;
    a.x = reinterpret_cast<const uint16_t*>(s.ws + g.off_xw);
    a.ids = reinterpret_cast<const int32_t*>(s.ws + g.off_idw);
    a.topk_w = reinterpret_cast<const float*>(s.ws + g.off_ww);
    a.resid = s.resid;
  }
  fill_args(a, s, g);
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
    // 2. screen (not needed when no sketch activation enters the result)
    if (!a.nosk) {
      const bool reg = (H + 255) / 256 <= kSbReg;
      const void* fn = reg ? reinterpret_cast<const void*>(&k_g_screen_lds)
                           : reinterpret_cast<const void*>(&k_g_screen<false>);
      if (int rc = launch_k("k_g_screen", fn, dim3(g.ntile, g.maxwork), 0, a, stream)) return rc;
    }
    // 3. top-c, candidate unions, exact work list
    {
      const int per = (g.I + GT - 1) / GT;
      const void* fn = per <= 4 ? reinterpret_cast<const void*>(&k_g_topc<4>)
                                : reinterpret_cast<const void*>(&k_g_topc<32>);
      if (int rc = launch_k("k_g_topc", fn, dim3(g.P), 0, a, stream)) return rc;
    }
  }
  // 4. exact gate / up over the candidate unions (all channels when dense)
  if (g.dense || g.k > 0 || a.rec_exact) {
    const int grid = std::min(kExactGrid, g.maxu * g.nrb);
    const int kc = std::min(kKc, H / 32);
    const void* fn = kc == 8 ? reinterpret_cast<const void*>(&k_g_exact<8>)
                   : kc == 4 ? reinterpret_cast<const void*>(&k_g_exact<4>)
                             : reinterpret_cast<const void*>(&k_g_exact<2>);
    const size_t lds = 2 * 64 * (size_t)(32 * kc + 8) * 2;
    if (int rc = launch_k("k_g_exact", fn, dim3(grid), lds, a, stream)) return rc;
  }
  if (!g.dense) {
    // 5. top-k, masked activations, recovery coefficients, kept unions
    const int per = (std::max(g.c, 1) + GT - 1) / GT;
    const void* fn = per <= 4 ? reinterpret_cast<const void*>(&k_g_topk<4>)
                              : reinterpret_cast<const void*>(&k_g_topk<32>);
    if (int rc = launch_k("k_g_topk", fn, dim3(g.P), 0, a, stream)) return rc;
  }
  // 6. down + recovery + combine
  if (int rc = launch_k("k_g_down", reinterpret_cast<const void*>(&k_g_down), dim3(H / kColTile, g.maxu),
                        g.dense ? 16 : 2 * (size_t)g.IP, a, stream))
    return rc;
  if (s.stats) {
    hipLaunchKernelGGL(k_g_stats, dim3(1), dim3(64), 0, stream, a, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_g_stats");
  }
  return CFM_OK;
}

// The expert-grouped pass's first two stages only (rotation, grouping and
// the screen), in front of the per-pair kernel for several tokens: every
// routed expert's sketch rows are read once for all of its tokens, and the
// pairs' sketch activations (hs) and partial recovery sums (zp) are left in
// the workspace for the per-pair kernel. The caller prepares the workspace.
bool grouped_screen_supported(int T, int K, int E, int I, int H, int r) {
  return grouped_supported(T, K, E, I, H, r, false) && (H + 255) / 256 <= kSbReg;
}

int launch_grouped_screen(const SelectArgs& s, const GroupPlan& g, hipStream_t stream) {
  GArgs a{};
  a.x = s.x; a.ids = s.ids; a.topk_w = s.topk_w;
  fill_args(a, s, g);
  const int H = g.H;
  const int ept = H >= 1024 ? H / 256 : 0;
  const void* fn = nullptr;
  switch (ept) {
    case 0: fn = reinterpret_cast<const void*>(&k_g_prep<0>); break;
    case 4: fn = reinterpret_cast<const void*>(&k_g_prep<4>); break;
    case 8: fn = reinterpret_cast<const void*>(&k_g_prep<8>); break;
    default: return set_error(CFM_EUNSUPPORTED, "grouped screen: hidden width not supported");
  }
  if (int rc = launch_k("k_g_prep", fn, dim3(g.T + 1), prep_lds(H, g.E), a, stream)) return rc;
  return launch_k("k_g_screen", reinterpret_cast<const void*>(&k_g_screen_lds), dim3(g.ntile, g.maxwork), 0, a,
                  stream);
}

}  // namespace cfm
