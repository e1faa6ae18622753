// Forward passes as single persistent kernels (gfx950): the selected-channel
// routed-expert SwiGLU layer and the dense comparator.
//
// Selected layer, per routed (token, expert) pair (arXiv:2610.37386 abstract;
// aimodeling.com article, section "A reader that needs no data at all"):
//   phase A  screen: x~ = Hadamard (signs . x) exactly in float64, fixed point,
//            FP8 base-16 digits; sketch activations hhat_j of this workgroup's
//            channels from FP4 ternary rows x FP8 digits on MFMA (exact integer
//            dot products); partial recovery sums over its channels;
//   phase B  top-c candidates (every workgroup of the pair, identically), exact
//            BF16 gate / up dot products over its share of the candidates;
//   phase C  top-k kept set, recovery coefficients z, down projection over the
//            kept rows of its 64-column output slice plus A z, and the token's
//            router-weighted combine by the last of its K pairs to arrive.
//
// A pair is served by nw workgroups. They exchange hhat, partial recovery sums
// and h through global memory with agent-coherent loads and stores (these
// bypass the per-XCD L2, so no cache flush or invalidation is needed), and
// meet at two per-pair phase counters (epoch in the high 16 bits, arrivals in
// the low 16; the last arrival advances the epoch, so the counters reset
// themselves). The grid never exceeds one workgroup per compute unit, so all
// workgroups are co-resident; waits are bounded and raise an error flag.
// Workgroup g serves pair g % P: with P a multiple of 8 all workgroups of a pair
// share an XCD (workgroups are dispatched round-robin over the 8 XCDs).
// Everything a workgroup can fetch without knowing the selections (x, its
// sketch rows, its Bt rows, its A slice) is requested at the start.
//
// The dense layer uses the same skeleton without the screen and selections.
#include <algorithm>

#include "cfm_internal.h"
#include "cfm_launch.h"
#include "topk.h"

namespace cfm {
namespace {

constexpr int NT = 256;                       // threads per workgroup
constexpr int kSubChunk = 32;                 // channels per phase-A sub-chunk
constexpr unsigned kSpinLimit = 1u << 22;     // bounded waits (seconds); then an error flag
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ memory helpers

__device__ __forceinline__ uint4 ld16(const void* p) {       // streamed weights
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16c(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Cross-workgroup exchange: agent-coherent (L2-bypassing) scalar loads / stores.
__device__ __forceinline__ void st_x(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_x(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_ctr(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Completes this wave's outstanding memory operations, then joins the workgroup.
__device__ __forceinline__ void drain_and_join() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  return dot2_bf16(a.w, b.w, acc);
}
__device__ __forceinline__ void fma8(float* acc, float h, const uint4& w) {
  acc[0] += h * bf16lo(w.x); acc[1] += h * bf16hi(w.x);
  acc[2] += h * bf16lo(w.y); acc[3] += h * bf16hi(w.y);
  acc[4] += h * bf16lo(w.z); acc[5] += h * bf16hi(w.z);
  acc[6] += h * bf16lo(w.w); acc[7] += h * bf16hi(w.w);
}
__device__ __forceinline__ float dot8_f(const uint4& w, const float* z) {
  return bf16lo(w.x) * z[0] + bf16hi(w.x) * z[1] + bf16lo(w.y) * z[2] + bf16hi(w.y) * z[3] +
         bf16lo(w.z) * z[4] + bf16hi(w.z) * z[5] + bf16lo(w.w) * z[6] + bf16hi(w.w) * z[7];
}

// ------------------------------------------------------------------ phase counters

// Epoch of a phase counter; read by thread 0 before this workgroup arrives.
__device__ __forceinline__ unsigned counter_epoch(unsigned* ctr) { return ld_ctr(ctr) >> 16; }

__device__ __forceinline__ void arrive(unsigned* ctr, unsigned epoch, unsigned n) {
  drain_and_join();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((old & 0xFFFFu) == n - 1)
      __hip_atomic_store(ctr, ((epoch + 1) & 0xFFFFu) << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void wait_all(unsigned* ctr, unsigned epoch, unsigned n, int* err) {
  if (threadIdx.x == 0) {
    unsigned it = 0;
    for (;;) {
      const unsigned v = ld_ctr(ctr);
      if ((v >> 16) != epoch || (v & 0xFFFFu) >= n) break;
      __builtin_amdgcn_s_sleep(1);
      if (++it > kSpinLimit) { atomicOr(err, 1); break; }
    }
  }
  __syncthreads();
}

// True in the workgroup that arrives last of `total` at *ctr (which it resets).
__device__ __forceinline__ bool last_of(unsigned* ctr, unsigned total, int* s_flag) {
  drain_and_join();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old == total - 1);
    if (old == total - 1) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *s_flag != 0;
}

// e4m3 encodings of the integers -8..7 (index d + 8)
__constant__ uint8_t kE4M3Digit[16] = {0xD0, 0xCE, 0xCC, 0xCA, 0xC8, 0xC4, 0xC0, 0xB8,
                                       0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E};

struct FusedArgs {
  const uint16_t* x; const int32_t* ids; const float* topk_w;
  const uint16_t *wg, *wu, *wd;
  const int8_t* signs; const uint8_t *tg, *tu; const float *sg, *su;
  const uint16_t *A, *Bt;
  uint16_t* out; int32_t *cand_out, *keep_out;
  float* hhat;      // [P][I]  sketch activations (selected) / exact activations (dense)
  float* zpart;     // [P][nw][r]
  float* hc;        // [P][c]  exact activations of the candidates
  float* ypart;     // [P][H]
  unsigned* ctr;    // [P][2] phase counters, [T][nhs] combine counters
  int* err;
  int T, K, P, E, I, H, log2H, k, c, r, nw, cw, cpw, nhs, G;
};

// ------------------------------------------------------------------ LDS layout (host and device)

struct Lds {
  double* xs;        // [H] x~ (float64) transpose buffer
  uint8_t* limb;     // [6][Hp] FP8 digits of the fixed-point x~
  float* hloc;       // [sub-chunk] sketch activations of the current channels
  float* dsum;       // [ntile][16][8] digit partial dots
  float* btc;        // [sub-chunk][r] Bt rows of the current channels (float)
  float* hh;         // [I] hhat of the pair
  uint32_t* keys;    // [max(I, c)]
  int32_t* candp;    // [c] candidate channel ids
  int32_t* sel;      // [max(c, k)]
  int32_t* keep;     // [k] kept channel ids
  float* hk;         // [k] kept activations
  float* hcl;        // [c] exact activations of the candidates
  float* zsum;       // [r]
  float* zv;         // [r] recovery coefficients
  float* red;        // [max(32*64+64, 32 r)] reduction scratch
  float* gu;         // [2][cpw]
  uint8_t* tks;      // top-k scratch
};

__host__ __device__ inline size_t lds_layout(int H, int I, int c, int k, int r, int cw, int cpw,
                                             size_t* off) {
  size_t o = 0;
  int n = 0;
  auto take = [&](size_t b) { off[n++] = o; o = (o + b + 15) & ~size_t(15); };
  const int Hp = H > 256 ? H : 256;
  cw = cw < kSubChunk ? cw : kSubChunk;       // phase A works in sub-chunks of channels
  const int ntile = (2 * cw + 15) / 16;
  const int ic = I > c ? I : c;
  const int ck = c > k ? c : k;
  const int r1 = r > 1 ? r : 1;
  take(8 * (size_t)H);
  take(6 * (size_t)Hp);
  take(4 * (size_t)cw);
  take(4 * (size_t)ntile * 128);
  take(4 * (size_t)cw * r1);
  take(4 * (size_t)I);
  take(4 * (size_t)ic);
  take(4 * (size_t)(c > 1 ? c : 1));
  take(4 * (size_t)(ck > 1 ? ck : 1));
  take(4 * (size_t)(k > 1 ? k : 1));
  take(4 * (size_t)(k > 1 ? k : 1));
  take(4 * (size_t)(c > 1 ? c : 1));
  take(4 * (size_t)r1);
  take(4 * (size_t)r1);
  const int nred = 32 * r1 > 32 * 64 + 64 ? 32 * r1 : 32 * 64 + 64;     // >= 8 NT, >= nw r
  take(4 * (size_t)nred);
  take(8 * (size_t)(cpw > 1 ? cpw : 1));
  take(topk_scratch_bytes(ic, NT));
  return o;
}

__device__ Lds carve(unsigned char* smem, const FusedArgs& a, TopkScratch* ts) {
  size_t off[20];
  lds_layout(a.H, a.I, a.c, a.k, a.r, a.cw, a.cpw, off);
  Lds L;
  L.xs = reinterpret_cast<double*>(smem + off[0]);
  L.limb = smem + off[1];
  L.hloc = reinterpret_cast<float*>(smem + off[2]);
  L.dsum = reinterpret_cast<float*>(smem + off[3]);
  L.btc = reinterpret_cast<float*>(smem + off[4]);
  L.hh = reinterpret_cast<float*>(smem + off[5]);
  L.keys = reinterpret_cast<uint32_t*>(smem + off[6]);
  L.candp = reinterpret_cast<int32_t*>(smem + off[7]);
  L.sel = reinterpret_cast<int32_t*>(smem + off[8]);
  L.keep = reinterpret_cast<int32_t*>(smem + off[9]);
  L.hk = reinterpret_cast<float*>(smem + off[10]);
  L.hcl = reinterpret_cast<float*>(smem + off[11]);
  L.zsum = reinterpret_cast<float*>(smem + off[12]);
  L.zv = reinterpret_cast<float*>(smem + off[13]);
  L.red = reinterpret_cast<float*>(smem + off[14]);
  L.gu = reinterpret_cast<float*>(smem + off[15]);
  L.tks = smem + off[16];
  const int ic = a.I > a.c ? a.I : a.c;
  ts->hist = reinterpret_cast<uint32_t*>(L.tks);
  ts->flag = L.tks + 4 * kHistBins;
  ts->lkey = reinterpret_cast<uint32_t*>(ts->flag + ((ic + 15) & ~15));
  ts->lidx = reinterpret_cast<int32_t*>(ts->lkey + kListMax);
  ts->misc = reinterpret_cast<uint32_t*>(ts->lidx + kListMax);
  return L;
}

// ------------------------------------------------------------------ phase A: rotation and digits

// Writes the six FP8 digits of X = rint(x~ 2^F) for element i.
__device__ __forceinline__ void put_digits(const Lds& L, int Hp, int i, double v, int F) {
  int X = (int32_t)rint(ldexp(v, F));
#pragma unroll
  for (int l = 0; l < 6; ++l) {
    const int d = ((X + 8) & 15) - 8;
    L.limb[l * Hp + i] = kE4M3Digit[d + 8];
    X = (X - d) >> 4;
  }
}

__device__ __forceinline__ int scale_exponent(double m, double* dred) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  if (lane == 0) dred[wv] = m;
  __syncthreads();
  m = dred[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) m = fmax(m, dred[w]);
  int F = 0;
  if (m > 0.0) { int ex; frexp(m, &ex); F = 22 - ex; }   // max |x~| 2^F in [2^21, 2^22)
  return F;
}

// x~ for H = 256 EPT with EPT >= 4. Layout A (thread t holds i = EPT t + q):
// in-register stages for the low bits, wavefront shuffles for the next six; one
// LDS transpose to layout B (i = t + 256 q) for the two bits that cross
// wavefronts. xv: the thread's EPT BF16 values of x (prefetched).
template <int EPT>
__device__ int rotate_fast(const FusedArgs& a, const Lds& L, const uint4* xv, double* dred) {
  const int tid = threadIdx.x, lane = tid & 63;
  double v[EPT];
  const int8_t* sg = a.signs + EPT * tid;
  if constexpr (EPT >= 8) {
#pragma unroll
    for (int u = 0; u < EPT / 8; ++u) {
      const uint4 w = xv[u];
      const uint2 s8 = *reinterpret_cast<const uint2*>(sg + 8 * u);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      const uint32_t ss[2] = {s8.x, s8.y};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float f = (q & 1) ? bf16hi(ww[q >> 1]) : bf16lo(ww[q >> 1]);
        const int s = (int8_t)((ss[q >> 2] >> (8 * (q & 3))) & 0xFF);
        v[8 * u + q] = (double)f * (double)s;
      }
    }
  } else {
    const uint4 w = xv[0];                 // EPT == 4: the first 8 bytes
    const uint32_t s4 = *reinterpret_cast<const uint32_t*>(sg);
    const uint32_t ww[2] = {w.x, w.y};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float f = (q & 1) ? bf16hi(ww[q >> 1]) : bf16lo(ww[q >> 1]);
      v[q] = (double)f * (double)(int8_t)((s4 >> (8 * q)) & 0xFF);
    }
  }
#pragma unroll
  for (int h = 1; h < EPT; h <<= 1)
#pragma unroll
    for (int q = 0; q < EPT; ++q)
      if (!(q & h)) { const double x0 = v[q], x1 = v[q + h]; v[q] = x0 + x1; v[q + h] = x0 - x1; }
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int m = 1 << s;
    const bool upper = lane & m;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const double o = __shfl_xor(v[q], m, 64);
      v[q] = upper ? o - v[q] : v[q] + o;
    }
  }
#pragma unroll
  for (int q = 0; q < EPT; ++q) L.xs[EPT * tid + q] = v[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < EPT; ++q) v[q] = L.xs[tid + NT * q];
#pragma unroll
  for (int h = EPT / 4; h < EPT; h <<= 1)
#pragma unroll
    for (int q = 0; q < EPT; ++q)
      if (!(q & h)) { const double x0 = v[q], x1 = v[q + h]; v[q] = x0 + x1; v[q + h] = x0 - x1; }
  double m = 0.0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) m = fmax(m, fabs(v[q]));
  const int F = scale_exponent(m, dred);
#pragma unroll
  for (int q = 0; q < EPT; ++q) put_digits(L, a.H, tid + NT * q, v[q], F);
  __syncthreads();
  return F;
}

// x~ for small H (< 1024): LDS butterflies.
__device__ int rotate_small(const FusedArgs& a, const Lds& L, int t, double* dred) {
  const int tid = threadIdx.x, H = a.H;
  const uint16_t* xt = a.x + (size_t)t * H;
  for (int i = tid; i < H; i += NT) L.xs[i] = (double)bf16_to_f32(xt[i]) * (double)a.signs[i];
  __syncthreads();
  for (int s = 0; s < a.log2H; ++s) {
    const int h = 1 << s;
    for (int b = tid; b < H / 2; b += NT) {
      const int i = ((b >> s) << (s + 1)) | (b & (h - 1));
      const double u = L.xs[i], w = L.xs[i + h];
      L.xs[i] = u + w;
      L.xs[i + h] = u - w;
    }
    __syncthreads();
  }
  double m = 0.0;
  for (int i = tid; i < H; i += NT) m = fmax(m, fabs(L.xs[i]));
  const int F = scale_exponent(m, dred);
  const int Hp = max(H, 256);
  for (int i = tid; i < Hp; i += NT) put_digits(L, Hp, i, i < H ? L.xs[i] : 0.0, F);
  __syncthreads();
  return F;
}

// ------------------------------------------------------------------ phase A: screen

// B operand: FP8 digit l of x~ in column l < 6 (zero in columns 6..15), for
// super-block sb (256 hidden indices) and half m; it matches the FP4 A operand
// layout where lane group g holds hidden indices sb*256 + 64 g + 32 m + (0..31).
__device__ __forceinline__ v8i digit_operand(const Lds& L, int Hp, int sb, int m) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, gB = lane >> 4;
  const uint8_t* row = L.limb + (size_t)min(col, 5) * Hp;
  const int i0 = sb * 256 + 64 * (gB >> 1) + 32 * m + 16 * (gB & 1);
  const uint4 lo = *reinterpret_cast<const uint4*>(row + i0);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + i0 + 128);
  const unsigned keep = col < 6 ? 0xFFFFFFFFu : 0u;
  v8i b;
  b[0] = lo.x & keep; b[1] = lo.y & keep; b[2] = lo.z & keep; b[3] = lo.w & keep;
  b[4] = hi.x & keep; b[5] = hi.y & keep; b[6] = hi.z & keep; b[7] = hi.w & keep;
  return b;
}

// The products are formed with the unscaled FP8/FP6/FP4 MFMA (v_mfma_f32_16x16x128_f8f6f4):
// the builtin selects it when both block-scale operands are 0. (The block-scaled
// encoding with an explicit 2^0 scale gave wrong accumulator rows in this kernel.)
__device__ __forceinline__ v8i trit_operand(uint32_t w0, uint32_t w1) {
  constexpr uint32_t M = 0xAAAAAAAAu;   // flag pairs -> FP4 E2M1 codes of +1 / -1 / 0
  v8i a;
  a[0] = (int)(w0 & M); a[1] = (int)((w0 << 1) & M);
  a[2] = (int)(w1 & M); a[3] = (int)((w1 << 1) & M);
  a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  return a;
}

// Screen items of a wavefront: (tile u, super-block sb = wave + 4 s); item it = u * nsbw + s.
constexpr int kScreenBatch = 8;

struct ScreenGeom {
  int cwk, nrows, ntile, nsb, nsbw, nitems;
};
__device__ __forceinline__ ScreenGeom screen_geom(const FusedArgs& a, int j0, int j1) {
  ScreenGeom g;
  const int wv = threadIdx.x >> 6;
  g.cwk = j1 - j0;
  g.nrows = 2 * g.cwk;
  g.ntile = (g.nrows + 15) / 16;
  g.nsb = (a.H + 255) / 256;
  g.nsbw = g.nsb > wv ? (g.nsb - wv + 3) / 4 : 0;
  g.nitems = g.ntile * g.nsbw;
  return g;
}

__device__ __forceinline__ uint4 screen_load(const FusedArgs& a, const ScreenGeom& g, int e,
                                             int j0, int it) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (it >= g.nitems) return make_uint4(0, 0, 0, 0);
  const int u = it / g.nsbw, s = it % g.nsbw;
  const int sb = wv + 4 * s;
  const int rho = u * 16 + (lane & 15);
  const int rowb = a.H / 4;
  const int off = sb * 64 + (lane >> 4) * 16;
  if (rho < g.nrows && off < rowb) {
    const int j = j0 + (rho < g.cwk ? rho : rho - g.cwk);
    return ld16((rho < g.cwk ? a.tg : a.tu) + ((size_t)e * a.I + j) * rowb + off);
  }
  return make_uint4(0, 0, 0, 0);
}

// Sketch activations of channels [j0, j1) of expert e into L.hloc and hhat[p][.].
// pre[]: the first batch of this wave's screen items, prefetched (if use_pre).
__device__ void screen_chunk(const FusedArgs& a, const Lds& L, int p, int e, int j0, int j1,
                             int F, const uint4* pre, bool use_pre) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int Hp = max(a.H, 256);
  const ScreenGeom g = screen_geom(a, j0, j1);
  const int wv = tid >> 6;
  for (int o = tid; o < g.ntile * 128; o += NT) L.dsum[o] = 0.f;
  __syncthreads();
  for (int b0 = 0; b0 < g.nitems; b0 += kScreenBatch) {
    uint4 w[kScreenBatch];
#pragma unroll
    for (int u = 0; u < kScreenBatch; ++u)
      w[u] = (use_pre && b0 == 0) ? pre[u] : screen_load(a, g, e, j0, b0 + u);
    v4f acc[kScreenBatch];
#pragma unroll
    for (int u = 0; u < kScreenBatch; ++u) {
      acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
      const int it = b0 + u;
      if (it < g.nitems) {
        const int sb = wv + 4 * (it % g.nsbw);
        const v8i d0 = digit_operand(L, Hp, sb, 0);
        const v8i d1 = digit_operand(L, Hp, sb, 1);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(w[u].x, w[u].y), d0, acc[u], 4, 0, 0, 0, 0, 0);
        acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(w[u].z, w[u].w), d1, acc[u], 4, 0, 0, 0, 0, 0);
      }
    }
    // lane holds D[4 (lane / 16) + v][lane % 16]: (row within tile, digit column);
    // partial dots of each item are integers, so the LDS sums are exact in any order
    const int col = lane & 15;
    if (col < 6) {
#pragma unroll
      for (int u = 0; u < kScreenBatch; ++u) {
        const int it = b0 + u;
        if (it < g.nitems) {
          const int tile = it / g.nsbw;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            atomicAdd(&L.dsum[(tile * 16 + 4 * (lane >> 4) + v) * 8 + col], acc[u][v]);
        }
      }
    }
  }
  __syncthreads();
  // exact integer dot per row: sum_l 16^l D_l (each D_l an integer below 8 H)
  for (int jj = tid; jj < g.cwk; jj += NT) {
    long long dg = 0, du = 0;
#pragma unroll
    for (int l = 0; l < 6; ++l) {
      dg += (long long)(int)L.dsum[jj * 8 + l] << (4 * l);
      du += (long long)(int)L.dsum[(g.cwk + jj) * 8 + l] << (4 * l);
    }
    const int j = j0 + jj;
    const float gh = (float)((double)a.sg[(size_t)e * a.I + j] * ldexp((double)dg, -F));
    const float uh = (float)((double)a.su[(size_t)e * a.I + j] * ldexp((double)du, -F));
    const float hv = silu_f32(gh) * uh;
    L.hloc[jj] = hv;
    st_x(a.hhat + (size_t)p * a.I + j, hv);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ phase B: exact gate / up

// h for items [q0, q1) of `chan` (null: channel = position) into out[q0..q1)
// (exchange stores). One wavefront per (row, matrix).
template <int CH>
__device__ void exact_rows(const FusedArgs& a, const Lds& L, int e, const int32_t* chan, int q0,
                           int q1, const uint4* xr, float* out) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, H = a.H;
  const int nchunk = H / 8;
  const int nitems = 2 * (q1 - q0);
  constexpr int RB = CH >= 16 ? 1 : (CH >= 8 ? 2 : 20 / CH);
  for (int it0 = wv * RB; it0 < nitems; it0 += (NT / 64) * RB) {
    uint4 wr[RB][CH];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int it = it0 + u;
      const int pos = q0 + (it >> 1);
      const int j = it < nitems ? (chan ? chan[pos] : pos) : 0;
      const uint16_t* Wm = (it & 1) ? a.wu : a.wg;
      const uint4* row = reinterpret_cast<const uint4*>(Wm + ((size_t)e * a.I + j) * H);
#pragma unroll
      for (int m = 0; m < CH; ++m) {
        const int ci = lane + 64 * m;
        wr[u][m] = (it < nitems && ci < nchunk) ? ld16(row + ci) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int it = it0 + u;
      if (it < nitems) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < CH; ++m) acc = dot8_bf16(wr[u][m], xr[m], acc);
        acc = wave_sum(acc);
        if (lane == 0) L.gu[(it & 1) * a.cpw + (it >> 1)] = acc;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < q1 - q0; i += NT) st_x(out + q0 + i, silu_f32(L.gu[i]) * L.gu[a.cpw + i]);
}

// ------------------------------------------------------------------ phase C: down + combine

// Recovery term of a 64-column slice into L.red[32*64 + 0..64): A[e][c0 + hh][:] . z.
// apre: the slice prefetched as 16-byte chunks f = tid + NT u (valid when r % 8 == 0).
__device__ void recovery_slice(const FusedArgs& a, const Lds& L, int e, int hs, const uint4* apre,
                               bool have_pre) {
  const int tid = threadIdx.x, r = a.r;
  const int c0 = hs * 64;
  if (r % 8 == 0) {
    const int cpr = r / 8;                 // 16-byte chunks per row
    const int nchunk = 64 * cpr;           // <= 1024
    float* part = L.red;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = tid + NT * u;
      if (f < nchunk) {
        const uint4 w = have_pre ? apre[u] : ld16(a.A + ((size_t)e * a.H + c0) * r + 8 * (size_t)f);
        part[f] = dot8_f(w, L.zv + 8 * (f % cpr));
      }
    }
    __syncthreads();
    float s = 0.f;
    if (tid < 64)
      for (int q = 0; q < cpr; ++q) s += part[tid * cpr + q];
    __syncthreads();
    if (tid < 64) L.red[32 * 64 + tid] = s;
  } else {
    float s = 0.f;
    if (tid < 64) {
      const uint16_t* arow = a.A + ((size_t)e * a.H + c0 + tid) * r;
      for (int l = 0; l < r; ++l) s += bf16_to_f32(arow[l]) * L.zv[l];
    }
    __syncthreads();
    if (tid < 64) L.red[32 * 64 + tid] = s;
  }
  __syncthreads();
}

// y[c0 .. c0+64) = sum_i h_i Wd_t[e][row_i][c0..] (+ the recovery term already in
// L.red[32*64 ..]), published for the combine; the last of the token's K pairs
// writes out[t][c0 .. c0+64).
__device__ void down_slice(const FusedArgs& a, const Lds& L, int p, int t, int e, int hs,
                           const int32_t* rows, const float* hv, int n, bool add_rec, int* s_flag) {
  const int tid = threadIdx.x, l8 = tid & 7, g = tid >> 3;
  const int c0 = hs * 64;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const uint16_t* base = a.wd + (size_t)e * a.I * a.H + c0 + 8 * l8;
  constexpr int DB = 8;
  for (int i0 = g; i0 < n; i0 += 32 * DB) {
    uint4 w[DB];
    float h[DB];
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const int i = i0 + 32 * u;
      const bool ok = i < n;
      const int row = ok ? (rows ? rows[i] : i) : 0;
      h[u] = ok ? hv[i] : 0.f;
      w[u] = ok ? ld16(base + (size_t)row * a.H) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < DB; ++u) fma8(acc, h[u], w[u]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) L.red[g * 64 + 8 * l8 + i] = acc[i];
  __syncthreads();
  if (tid < 64) {
    float y = 0.f;
    for (int gg = 0; gg < 32; ++gg) y += L.red[gg * 64 + tid];
    if (add_rec) y += L.red[32 * 64 + tid];
    st_x(a.ypart + (size_t)p * a.H + c0 + tid, y);
  }
  unsigned* cc = a.ctr + 2 * (size_t)a.P + (size_t)t * a.nhs + hs;
  if (last_of(cc, (unsigned)a.K, s_flag)) {
    if (tid < 64) {
      float o = 0.f;
      for (int q = 0; q < a.K; ++q)
        o += a.topk_w[(size_t)t * a.K + q] * ld_x(a.ypart + (size_t)(t * a.K + q) * a.H + c0 + tid);
      const bool bad = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      a.out[(size_t)t * a.H + c0 + tid] = bad ? (uint16_t)0x7FC0 : f32_to_bf16(o);
    }
  }
  __syncthreads();
}

// Loads n exchange values src[0..n) into dst (LDS), batched; optionally keys too.
__device__ void fetch_exchange(const float* src, int n, float* dst, uint32_t* keys) {
  constexpr int HB = 8;
  const int tid = threadIdx.x;
  for (int i0 = tid; i0 < n; i0 += NT * HB) {
    float hv[HB];
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int i = i0 + NT * u;
      hv[u] = i < n ? ld_x(src + i) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < HB; ++u) {
      const int i = i0 + NT * u;
      if (i < n) {
        dst[i] = hv[u];
        if (keys) keys[i] = score_key(hv[u]);
      }
    }
  }
}

// ------------------------------------------------------------------ kernels

template <int EPT>
__global__ __launch_bounds__(NT) void k_select_fused(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ double dred[NT / 64];
  __shared__ int s_flag;
  __shared__ unsigned s_epoch[2];
  __shared__ uint32_t radix_scratch[256 + NT / 64 + 8];
  TopkScratch ts;
  const Lds L = carve(smem, a, &ts);
  const int tid = threadIdx.x, lane = tid & 63;
  const int nw = a.nw, H = a.H, r = a.r;
  constexpr int CH = EPT >= 2 ? EPT / 2 : 1;        // 16-byte chunks of x per lane (H / 512)
  constexpr int XV = EPT >= 8 ? EPT / 8 : 1;

  for (int slot = blockIdx.x; slot < a.P * nw; slot += a.G) {
    const int p = slot % a.P, w = slot / a.P;
    const int t = p / a.K;
    const int e = a.ids[p];
    unsigned* ctrA = a.ctr + 2 * (size_t)p;
    unsigned* ctrB = ctrA + 1;
    const int j0 = min(a.I, w * a.cw), j1 = min(a.I, j0 + a.cw);
    const int hs0 = w;                              // first output slice of this workgroup
    const bool one_slice = hs0 < a.nhs && hs0 + nw >= a.nhs;

    // ---- requests that need no selection: x, sketch rows, Bt rows, A slice
    uint4 xv[XV];
    if constexpr (EPT >= 4) {
      const uint16_t* xt = a.x + (size_t)t * H + EPT * tid;
#pragma unroll
      for (int u = 0; u < XV; ++u) {
        if constexpr (EPT >= 8) xv[u] = ld16c(xt + 8 * u);
        else { const uint2 h2 = *reinterpret_cast<const uint2*>(xt); xv[u] = make_uint4(h2.x, h2.y, 0, 0); }
      }
    }
    const int sj1f = min(j1, j0 + kSubChunk);       // first sub-chunk
    const ScreenGeom sgm = screen_geom(a, j0, sj1f);
    uint4 spre[kScreenBatch];
#pragma unroll
    for (int u = 0; u < kScreenBatch; ++u) spre[u] = screen_load(a, sgm, e, j0, u);
    constexpr int BTP = 8;                          // Bt rows of the first sub-chunk: flat bf16
    uint16_t btp[BTP];
    const uint16_t* btbase = a.Bt + ((size_t)e * a.I + j0) * r;
#pragma unroll
    for (int u = 0; u < BTP; ++u) {
      const int f = tid + NT * u;
      btp[u] = f < (sj1f - j0) * r ? btbase[f] : (uint16_t)0;
    }
    uint4 apre[4];
    const bool have_apre = one_slice && r > 0 && r % 8 == 0 && 8 * r <= 4 * NT;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = tid + NT * u;
      apre[u] = (have_apre && f < 8 * r) ? ld16(a.A + ((size_t)e * H + hs0 * 64) * r + 8 * (size_t)f)
                                         : make_uint4(0, 0, 0, 0);
    }
    if (tid == 0) { s_epoch[0] = counter_epoch(ctrA); s_epoch[1] = counter_epoch(ctrB); }

    // ---- phase A: screen this workgroup's channels, sub-chunk by sub-chunk
    int F;
    if constexpr (EPT >= 4) F = rotate_fast<EPT>(a, L, xv, dred);
    else F = rotate_small(a, L, t, dred);
    float zacc = 0.f;                               // partial recovery sum for l = tid
    for (int sj0 = j0; sj0 < j1; sj0 += kSubChunk) {
      const int sj1 = min(j1, sj0 + kSubChunk);
      const bool first = sj0 == j0;
      screen_chunk(a, L, p, e, sj0, sj1, F, spre, first);
      if (r > 0) {
        const int nbt = (sj1 - sj0) * r;
        const uint16_t* bb = a.Bt + ((size_t)e * a.I + sj0) * r;
        if (first) {
#pragma unroll
          for (int u = 0; u < BTP; ++u) {
            const int f = tid + NT * u;
            if (f < nbt) L.btc[f] = bf16_to_f32(btp[u]);
          }
        }
        for (int f = tid + (first ? NT * BTP : 0); f < nbt; f += NT) L.btc[f] = bf16_to_f32(bb[f]);
        __syncthreads();
        if (tid < r)
          for (int jj = 0; jj < sj1 - sj0; ++jj) zacc += L.hloc[jj] * L.btc[jj * r + tid];
        __syncthreads();
      }
    }
    if (tid < r) st_x(a.zpart + ((size_t)p * nw + w) * r + tid, zacc);
    arrive(ctrA, s_epoch[0], (unsigned)nw);
    wait_all(ctrA, s_epoch[0], (unsigned)nw, a.err);

    // ---- top-c candidates (identical in every workgroup of the pair)
    fetch_exchange(a.hhat + (size_t)p * a.I, a.I, L.hh, L.keys);
    if (r > 0) fetch_exchange(a.zpart + (size_t)p * nw * r, nw * r, L.red, nullptr);
    __syncthreads();
    for (int l = tid; l < r; l += NT) {
      float s = 0.f;
      for (int q = 0; q < nw; ++q) s += L.red[q * r + l];
      L.zsum[l] = s;
    }
    block_topk<NT>(L.keys, a.I, a.c, L.candp, ts, radix_scratch);
    if (w == 0 && a.cand_out)
      for (int i = tid; i < a.c; i += NT) a.cand_out[(size_t)p * a.c + i] = L.candp[i];

    // ---- phase B: exact activations of this workgroup's candidates
    const int q0 = min(a.c, w * a.cpw), q1 = min(a.c, q0 + a.cpw);
    if (a.k > 0 && q0 < q1) {
      uint4 xr[CH];
      const uint4* xg = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
#pragma unroll
      for (int m = 0; m < CH; ++m) {
        const int ci = lane + 64 * m;
        xr[m] = ci < H / 8 ? ld16c(xg + ci) : make_uint4(0, 0, 0, 0);
      }
      exact_rows<CH>(a, L, e, L.candp, q0, q1, xr, a.hc + (size_t)p * a.c);
    }
    arrive(ctrB, s_epoch[1], (unsigned)nw);
    wait_all(ctrB, s_epoch[1], (unsigned)nw, a.err);

    // ---- top-k kept set and recovery coefficients
    if (a.k > 0) {
      fetch_exchange(a.hc + (size_t)p * a.c, a.c, L.hcl, L.keys);
      __syncthreads();
      block_topk<NT>(L.keys, a.c, a.k, L.sel, ts, radix_scratch);
      for (int i = tid; i < a.k; i += NT) {
        L.keep[i] = L.candp[L.sel[i]];
        L.hk[i] = L.hcl[L.sel[i]];
      }
      __syncthreads();
      if (w == 0 && a.keep_out)
        for (int i = tid; i < a.k; i += NT) a.keep_out[(size_t)p * a.k + i] = L.keep[i];
    }
    if (r > 0) {
      // z = zsum - sum_{j in S} hhat_j Bt[e][j]
      if (r % 8 == 0) {
        const int cpr = r / 8, groups = NT / cpr;   // r <= 128: cpr <= 16, groups >= 16
        const int cc = tid % cpr, g = tid / cpr;
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.f;
        constexpr int ZB = 8;
        for (int i0 = g; i0 < a.k; i0 += groups * ZB) {
          uint4 bw[ZB];
          float hv[ZB];
#pragma unroll
          for (int u = 0; u < ZB; ++u) {
            const int i = i0 + groups * u;
            const bool ok = i < a.k;
            const int j = ok ? L.keep[i] : 0;
            hv[u] = ok ? L.hh[j] : 0.f;
            bw[u] = ok ? ld16c(a.Bt + ((size_t)e * a.I + j) * r + 8 * cc) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < ZB; ++u) fma8(acc, hv[u], bw[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) L.red[g * r + 8 * cc + u] = acc[u];    // groups * r = 8 NT
        __syncthreads();
        for (int l = tid; l < r; l += NT) {
          float s = 0.f;
          for (int gg = 0; gg < groups; ++gg) s += L.red[gg * r + l];
          L.zv[l] = L.zsum[l] - s;
        }
      } else {
        for (int l = tid; l < r; l += NT) {
          float s = 0.f;
          for (int i = 0; i < a.k; ++i) {
            const int j = L.keep[i];
            s += L.hh[j] * bf16_to_f32(a.Bt[((size_t)e * a.I + j) * r + l]);
          }
          L.zv[l] = L.zsum[l] - s;
        }
      }
      __syncthreads();
    }

    // ---- phase C: down projection over kept rows for this workgroup's output slices
    for (int hs = hs0; hs < a.nhs; hs += nw) {
      if (r > 0) recovery_slice(a, L, e, hs, apre, have_apre && hs == hs0);
      down_slice(a, L, p, t, e, hs, L.keep, L.hk, a.k, r > 0, &s_flag);
    }
  }
}

template <int EPT>
__global__ __launch_bounds__(NT) void k_dense_fused(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_flag;
  __shared__ unsigned s_epoch;
  TopkScratch ts;
  const Lds L = carve(smem, a, &ts);
  const int tid = threadIdx.x, lane = tid & 63;
  const int nw = a.nw, H = a.H;
  constexpr int CH = EPT >= 2 ? EPT / 2 : 1;
  for (int slot = blockIdx.x; slot < a.P * nw; slot += a.G) {
    const int p = slot % a.P, w = slot / a.P;
    const int t = p / a.K;
    const int e = a.ids[p];
    unsigned* ctrB = a.ctr + 2 * (size_t)p + 1;
    if (tid == 0) s_epoch = counter_epoch(ctrB);
    const int q0 = min(a.I, w * a.cpw), q1 = min(a.I, q0 + a.cpw);
    if (q0 < q1) {
      uint4 xr[CH];
      const uint4* xg = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
#pragma unroll
      for (int m = 0; m < CH; ++m) {
        const int ci = lane + 64 * m;
        xr[m] = ci < H / 8 ? ld16c(xg + ci) : make_uint4(0, 0, 0, 0);
      }
      exact_rows<CH>(a, L, e, nullptr, q0, q1, xr, a.hhat + (size_t)p * a.I);
    }
    arrive(ctrB, s_epoch, (unsigned)nw);
    wait_all(ctrB, s_epoch, (unsigned)nw, a.err);
    fetch_exchange(a.hhat + (size_t)p * a.I, a.I, L.hh, nullptr);
    __syncthreads();
    for (int hs = w; hs < a.nhs; hs += nw)
      down_slice(a, L, p, t, e, hs, nullptr, L.hh, a.I, false, &s_flag);
  }
}

// ------------------------------------------------------------------ stats

__global__ void k_stats(const int32_t* ids, int P, int E, int I, int H, int k, int c, int r, int T,
                        int K, int select, cfm_stats* st) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  unsigned used = 0;
  for (int pp = 0; pp < P; ++pp) {
    bool first = true;
    for (int qq = 0; qq < pp; ++qq) if (ids[qq] == ids[pp]) { first = false; break; }
    used += first;
  }
  cfm_stats s;
  const uint64_t Pu = (uint64_t)P;
  s.bytes_io = 2ull * T * H + 8ull * T * K + 2ull * T * H;
  s.bytes_dense_equiv = (uint64_t)used * 6ull * I * H + s.bytes_io;
  s.experts_used = used;
  if (select) {
    s.bytes_sketch = Pu * (2ull * I * (H / 4) + 8ull * I);
    s.bytes_candidates = k > 0 ? Pu * 4ull * H * c : 0;
    s.bytes_down = Pu * 2ull * H * k;
    s.bytes_recovery = r > 0 ? Pu * (2ull * H * r + 2ull * I * r) : 0;
    s.rows_candidates = k > 0 ? (uint32_t)(P * c) : 0;
    s.rows_down = (uint32_t)(P * k);
  } else {
    s.bytes_sketch = 0;
    s.bytes_candidates = Pu * 4ull * H * I;
    s.bytes_down = Pu * 2ull * H * I;
    s.bytes_recovery = 0;
    s.rows_candidates = (uint32_t)(P * I);
    s.rows_down = (uint32_t)(P * I);
  }
  s.pad = 0;
  *st = s;
}

template <bool SELECT>
int launch_fused(const FusedArgs& fa, size_t lds, hipStream_t stream) {
  const int H = fa.H;
  const int ept = H >= 1024 ? H / 256 : 0;
  const void* fn = nullptr;
#define CFM_PICK(E) fn = SELECT ? reinterpret_cast<const void*>(&k_select_fused<E>) \
                                : reinterpret_cast<const void*>(&k_dense_fused<E>)
  switch (ept) {
    case 0: if (H == 512) CFM_PICK(2); else CFM_PICK(0); break;
    case 4: CFM_PICK(4); break;
    case 8: CFM_PICK(8); break;
    case 16: CFM_PICK(16); break;
    case 32: CFM_PICK(32); break;
    default: return set_error(CFM_EUNSUPPORTED, "hidden width not supported");
  }
#undef CFM_PICK
  if (lds > 163840) return set_error(CFM_EUNSUPPORTED, "shape needs more LDS than a workgroup has");
  if (lds > 65536)
    CFM_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  timing_begin(SELECT ? "k_select_fused" : "k_dense_fused", stream);
  void* args[] = {const_cast<FusedArgs*>(&fa)};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)fa.G), dim3(NT), args, lds, stream);
  timing_end(stream);
  if (e != hipSuccess) return set_error(CFM_EHIP, std::string("fused launch: ") + hipGetErrorString(e));
  CFM_LAUNCH_CHECK("fused");
  return CFM_OK;
}

}  // namespace

// ------------------------------------------------------------------ plans

static void fused_geometry(ForwardPlan& p, int G_max) {
  const int P = std::max(p.P, 1);
  int nw = 1;
  while (nw * 2 * P <= G_max && nw * 2 <= 32) nw *= 2;
  p.nw = nw;
  p.G = std::min(P * nw, G_max);
  p.nhs = p.H / 64;
}

ForwardPlan select_plan(int T, int K, int E, int I, int H, int k, int c, int r) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = k; p.c = c; p.r = r;
  fused_geometry(p, 256);
  p.cw = (I + p.nw - 1) / p.nw;
  p.cpw = std::max(1, (c + p.nw - 1) / p.nw);
  size_t off[20];
  p.lds = lds_layout(H, I, c, k, r, p.cw, p.cpw, off);
  Carve cv;
  const size_t Pz = (size_t)p.P;
  p.off_hhat = cv.take(Pz * I * 4);
  p.off_zpart = cv.take(Pz * p.nw * std::max(r, 1) * 4);
  p.off_hc = cv.take(Pz * std::max(c, 1) * 4);
  p.off_ypart = cv.take(Pz * H * 4);
  p.off_ctr = cv.take((2 * Pz + (size_t)T * p.nhs) * 4);
  p.off_err = cv.take(64);
  p.bytes = cv.off;
  return p;
}

ForwardPlan dense_plan(int T, int K, int E, int I, int H) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = 0; p.c = 0; p.r = 0;
  fused_geometry(p, 256);
  p.cw = 1;
  p.cpw = std::max(1, (I + p.nw - 1) / p.nw);
  size_t off[20];
  p.lds = lds_layout(H, I, 0, 0, 0, p.cw, p.cpw, off);
  Carve cv;
  const size_t Pz = (size_t)p.P;
  p.off_hhat = cv.take(Pz * I * 4);
  p.off_ypart = cv.take(Pz * H * 4);
  p.off_ctr = cv.take((2 * Pz + (size_t)T * p.nhs) * 4);
  p.off_err = cv.take(64);
  p.bytes = cv.off;
  return p;
}

// ------------------------------------------------------------------ launches

static FusedArgs fused_args(const SelectArgs& s, const ForwardPlan& p) {
  FusedArgs a{};
  a.x = s.x; a.ids = s.ids; a.topk_w = s.topk_w;
  a.wg = s.w_gate; a.wu = s.w_up; a.wd = s.w_down_t;
  a.signs = s.signs; a.tg = s.tg; a.tu = s.tu; a.sg = s.sg; a.su = s.su;
  a.A = s.A; a.Bt = s.Bt;
  a.out = s.out; a.cand_out = s.cand_out; a.keep_out = s.keep_out;
  a.hhat = reinterpret_cast<float*>(s.ws + p.off_hhat);
  a.zpart = reinterpret_cast<float*>(s.ws + p.off_zpart);
  a.hc = reinterpret_cast<float*>(s.ws + p.off_hc);
  a.ypart = reinterpret_cast<float*>(s.ws + p.off_ypart);
  a.ctr = reinterpret_cast<unsigned*>(s.ws + p.off_ctr);
  a.err = reinterpret_cast<int*>(s.ws + p.off_err);
  a.T = p.T; a.K = p.K; a.P = p.P; a.E = p.E; a.I = p.I; a.H = p.H;
  int log2H = 0;
  while ((1 << log2H) < p.H) ++log2H;
  a.log2H = log2H;
  a.k = p.k; a.c = p.c; a.r = p.r; a.nw = p.nw; a.cw = p.cw; a.cpw = p.cpw; a.nhs = p.nhs; a.G = p.G;
  return a;
}

int launch_select_forward(const SelectArgs& s, const ForwardPlan& p, hipStream_t stream) {
  const FusedArgs a = fused_args(s, p);
  int rc = launch_fused<true>(a, p.lds, stream);
  if (rc) return rc;
  if (s.stats) {
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, s.ids, p.P, p.E, p.I, p.H, p.k, p.c,
                       p.r, p.T, p.K, 1, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

int launch_dense_forward(const SelectArgs& s, const ForwardPlan& p, hipStream_t stream) {
  const FusedArgs a = fused_args(s, p);
  int rc = launch_fused<false>(a, p.lds, stream);
  if (rc) return rc;
  if (s.stats) {
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, s.ids, p.P, p.E, p.I, p.H, p.I, p.I, 0,
                       p.T, p.K, 0, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

}  // namespace cfm
