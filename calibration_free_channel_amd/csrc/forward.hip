// Forward passes: the selected-channel routed-expert SwiGLU layer and the dense
// comparator (gfx950).
//
// Selected layer, per routed (token, expert) pair (arXiv:2610.37386 abstract;
// aimodeling.com article, section "A reader that needs no data at all"):
//   k_screen  : rotate x, ternary-sketch activations hhat_j for every channel,
//               partial recovery sums, and (last workgroup of the pair) the
//               top-c candidate set;
//   k_gu      : exact BF16 gate/up dot products over the candidates only, and
//               (last workgroup of the pair) the top-k kept set plus the
//               recovery coefficients z = sum over skipped channels;
//   k_down    : down projection over the kept channels' rows, low-rank recovery
//               A z, and (last workgroup of a token's output slice) the
//               router-weighted combine into BF16.
// Every weight row is read as whole, contiguous 16-byte-per-lane wavefront
// loads; nothing outside the selected rows of W_gate / W_up / W_down is read.
// Cross-workgroup hand-offs use agent-scope release/acquire completion
// counters; the last arriving workgroup does the reduction, so no workgroup
// ever waits on another and results are independent of arrival order.
#include "cfm_internal.h"
#include "cfm_launch.h"

namespace cfm {
namespace {

constexpr int NT = 256;                  // threads per workgroup in every kernel here
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (the weights are read once per call: keep them out of the way).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
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

__device__ __forceinline__ void release_fence() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// True in every thread of the workgroup that arrives last at *ctr (of `total`);
// that workgroup also resets the counter for the next call.
__device__ __forceinline__ bool last_arrival(unsigned* ctr, unsigned total, int* s_flag) {
  release_fence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = arrive_counter(ctr);
    *s_flag = (old == total - 1);
    if (old == total - 1) reset_counter(ctr);
  }
  __syncthreads();
  const bool last = *s_flag != 0;
  if (last) acquire_fence();
  return last;
}

// ------------------------------------------------------------------------------------ screen
//
// Workgroup (pair p, chunk ch) computes hhat_j for channels [ch*cw, ...) of the
// pair's expert. x~ = Hadamard (signs . x) is formed exactly in float64 and turned
// into 24-bit fixed point X_i = rint(x~_i 2^F); each ternary row's dot product
// with X is then an exact integer, so the sketch activations do not depend on
// the summation order.

struct ScreenArgs {
  const uint16_t* x; const int32_t* ids; const int8_t* signs;
  const uint8_t *tg, *tu; const float *sg, *su; const uint16_t* Bt;
  float* hhat; float* zpart; float* zsum; int32_t* cand; int32_t* cand_out;
  unsigned* ctr;
  int K, I, H, log2H, c, r, nch, cw;
};

__global__ __launch_bounds__(NT) void k_screen(ScreenArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p = blockIdx.x / a.nch, ch = blockIdx.x % a.nch;
  const int t = p / a.K;
  const int e = a.ids[p];
  const int H = a.H, I = a.I;
  const int j0 = ch * a.cw, j1 = min(I, j0 + a.cw);

  double* xs = reinterpret_cast<double*>(smem);                       // [H]
  int32_t* X = reinterpret_cast<int32_t*>(smem + 8 * (size_t)max(H, (I + 1) / 2));  // [H]
  float* hloc = reinterpret_cast<float*>(X + max(H, a.c));            // [cw]
  __shared__ double dred[NT / 64];
  __shared__ int s_flag;
  __shared__ uint32_t sel_scratch[256 + NT / 64 + 8];

  // 1. x~ in float64 (exact), then fixed point
  const uint16_t* xt = a.x + (size_t)t * H;
  for (int i = tid; i < H; i += NT) xs[i] = (double)bf16_to_f32(xt[i]) * (double)a.signs[i];
  __syncthreads();
  for (int s = 0; s < a.log2H; ++s) {
    const int h = 1 << s;
    for (int b = tid; b < H / 2; b += NT) {
      const int i = ((b >> s) << (s + 1)) | (b & (h - 1));
      const double u = xs[i], w = xs[i + h];
      xs[i] = u + w;
      xs[i + h] = u - w;
    }
    __syncthreads();
  }
  double m = 0.0;
  for (int i = tid; i < H; i += NT) m = fmax(m, fabs(xs[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  if (lane == 0) dred[wv] = m;
  __syncthreads();
  m = dred[0];
  for (int w = 1; w < NT / 64; ++w) m = fmax(m, dred[w]);
  int F = 0;
  if (m > 0.0) { int ex; frexp(m, &ex); F = 23 - ex; }   // max |x~| * 2^F in [2^22, 2^23)
  for (int i = tid; i < H; i += NT) X[i] = (int32_t)rint(ldexp(xs[i], F));
  __syncthreads();

  // 2. sketch activations, one wavefront per channel
  const int words = H / 16;
  for (int j = j0 + wv; j < j1; j += NT / 64) {
    const uint32_t* rg = reinterpret_cast<const uint32_t*>(a.tg + ((size_t)e * I + j) * (H / 4));
    const uint32_t* ru = reinterpret_cast<const uint32_t*>(a.tu + ((size_t)e * I + j) * (H / 4));
    long long dg = 0, du = 0;
    for (int b = lane; b < words; b += 64) {
      const uint32_t wg = rg[b], wu = ru[b];
      int ag = 0, au = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int xl = X[16 * b + q], xh = X[16 * b + 8 + q];
        ag += ((wg >> (4 * q + 1)) & 1u) ? (((wg >> (4 * q + 3)) & 1u) ? -xl : xl) : 0;
        ag += ((wg >> (4 * q)) & 1u) ? (((wg >> (4 * q + 2)) & 1u) ? -xh : xh) : 0;
        au += ((wu >> (4 * q + 1)) & 1u) ? (((wu >> (4 * q + 3)) & 1u) ? -xl : xl) : 0;
        au += ((wu >> (4 * q)) & 1u) ? (((wu >> (4 * q + 2)) & 1u) ? -xh : xh) : 0;
      }
      dg += ag;
      du += au;
    }
    dg = wave_sum_ll(dg);
    du = wave_sum_ll(du);
    if (lane == 0) {
      const float gh = (float)((double)a.sg[(size_t)e * I + j] * ldexp((double)dg, -F));
      const float uh = (float)((double)a.su[(size_t)e * I + j] * ldexp((double)du, -F));
      const float hh = silu_f32(gh) * uh;
      a.hhat[(size_t)p * I + j] = hh;
      hloc[j - j0] = hh;
    }
  }
  __syncthreads();

  // 3. partial recovery sums over this chunk: zpart[l] = sum_j hhat_j Bt[e][j][l]
  if (a.r > 0) {
    for (int l = tid; l < a.r; l += NT) {
      float acc = 0.f;
      for (int j = j0; j < j1; ++j) acc += hloc[j - j0] * bf16_to_f32(a.Bt[((size_t)e * I + j) * a.r + l]);
      a.zpart[((size_t)p * a.nch + ch) * a.r + l] = acc;
    }
  }

  // 4. the pair's last workgroup selects C and totals the recovery sums
  if (!last_arrival(a.ctr + p, (unsigned)a.nch, &s_flag)) return;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);   // [I], reuses xs
  int32_t* sel = X;                                      // [c]
  for (int i = tid; i < I; i += NT) keys[i] = score_key(__builtin_nontemporal_load(a.hhat + (size_t)p * I + i));
  __syncthreads();
  block_topk_ascending<NT>(keys, I, a.c, sel, sel_scratch);
  for (int i = tid; i < a.c; i += NT) {
    a.cand[(size_t)p * a.c + i] = sel[i];
    if (a.cand_out) a.cand_out[(size_t)p * a.c + i] = sel[i];
  }
  for (int l = tid; l < a.r; l += NT) {
    float s = 0.f;
    for (int q = 0; q < a.nch; ++q) s += a.zpart[((size_t)p * a.nch + q) * a.r + l];
    a.zsum[(size_t)p * a.r + l] = s;
  }
}

// ------------------------------------------------------------------------------------ gate / up
//
// Workgroup (pair p, slot s) computes exact h_j = SiLU(Wg_j . x) (Wu_j . x) for its
// share of rows: the candidate set C (selected layer) or every channel (dense).
// One wavefront per row; each lane keeps its slice of x in registers and reads
// 16 contiguous bytes of the row per load.

struct GuArgs {
  const uint16_t* x; const int32_t* ids; const uint16_t *wg, *wu;
  const int32_t* cand;       // [P][c] or null (dense: every channel)
  float* hout;               // [P][n]
  // selected layer only: top-k + recovery coefficients
  const float* hhat; const float* zsum; const uint16_t* Bt;
  int32_t* keep; float* hk; float* z; int32_t* keep_out; unsigned* ctr;
  int K, I, H, n, per, nslot, k, r;
};

template <int CH, bool SELECT>
__global__ __launch_bounds__(NT) void k_gu(GuArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int p = blockIdx.x / a.nslot, s = blockIdx.x % a.nslot;
  const int t = p / a.K;
  const int e = a.ids[p];
  const int H = a.H;
  const int pos0 = s * a.per, pos1 = min(a.n, pos0 + a.per);
  float* gl = reinterpret_cast<float*>(smem);   // [per]
  float* ul = gl + a.per;                        // [per]
  __shared__ int s_flag;
  __shared__ uint32_t sel_scratch[256 + NT / 64 + 8];

  uint4 xr[CH];
  const uint4* xv = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
  const int nchunk = H / 8;
#pragma unroll
  for (int m = 0; m < CH; ++m) {
    const int ci = lane + 64 * m;
    xr[m] = ci < nchunk ? xv[ci] : make_uint4(0, 0, 0, 0);
  }
  const int nitems = 2 * (pos1 - pos0);
  for (int it = wv; it < nitems; it += NT / 64) {
    const int pos = pos0 + (it >> 1);
    const int j = SELECT ? a.cand[(size_t)p * a.n + pos] : pos;
    const uint16_t* W = (it & 1) ? a.wu : a.wg;
    const uint4* row = reinterpret_cast<const uint4*>(W + ((size_t)e * a.I + j) * H);
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < CH; ++m) {
      const int ci = lane + 64 * m;
      if (ci < nchunk) acc = dot8_bf16(ld_stream16(row + ci), xr[m], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) ((it & 1) ? ul : gl)[pos - pos0] = acc;
  }
  __syncthreads();
  for (int i = tid; i < pos1 - pos0; i += NT)
    a.hout[(size_t)p * a.n + pos0 + i] = silu_f32(gl[i]) * ul[i];
  if constexpr (!SELECT) return;

  // the pair's last workgroup: S = top-k of C by |h|, and z = zsum - sum_{j in S} hhat_j Bt[j]
  if (!last_arrival(a.ctr + p, (unsigned)a.nslot, &s_flag)) return;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);          // [n]
  int32_t* sel = reinterpret_cast<int32_t*>(keys + a.n);        // [k]
  for (int i = tid; i < a.n; i += NT) keys[i] = score_key(__builtin_nontemporal_load(a.hout + (size_t)p * a.n + i));
  __syncthreads();
  block_topk_ascending<NT>(keys, a.n, a.k, sel, sel_scratch);
  for (int i = tid; i < a.k; i += NT) {
    const int j = a.cand[(size_t)p * a.n + sel[i]];
    a.keep[(size_t)p * a.k + i] = j;
    a.hk[(size_t)p * a.k + i] = __builtin_nontemporal_load(a.hout + (size_t)p * a.n + sel[i]);
    if (a.keep_out) a.keep_out[(size_t)p * a.k + i] = j;
  }
  __syncthreads();
  for (int l = tid; l < a.r; l += NT) {
    float acc = a.zsum[(size_t)p * a.r + l];
    for (int i = 0; i < a.k; ++i) {
      const int j = a.cand[(size_t)p * a.n + sel[i]];
      acc -= a.hhat[(size_t)p * a.I + j] * bf16_to_f32(a.Bt[((size_t)e * a.I + j) * a.r + l]);
    }
    a.z[(size_t)p * a.r + l] = acc;
  }
}

// ------------------------------------------------------------------------------------ down + combine
//
// Workgroup (token t, 64-column slice hs, slot q) accumulates
//   y[cols] = sum_i h_i Wd_t[e][row_i][cols]  (+ A[e][cols][:] . z)
// over the kept rows (selected) or every row (dense), then the token's last slot
// to arrive writes out[t][cols] = BF16(sum_q w_q y_q[cols]) in slot order.

struct DownArgs {
  const int32_t* ids; const float* w; const uint16_t* wd;
  const int32_t* rows;       // [P][n] row ids, or null = 0..n-1
  const float* h;            // [P][n]
  const uint16_t* A; const float* z;   // recovery (r > 0)
  float* ypart; uint16_t* out; unsigned* ctr;
  int K, I, H, n, r, nhs;
};

template <bool SELECT>
__global__ __launch_bounds__(NT) void k_down(DownArgs a) {
  __shared__ float red[NT / 8][64];
  __shared__ float zs[kMaxRank];
  __shared__ float yrec[64];
  __shared__ int s_flag;
  const int tid = threadIdx.x, l8 = tid & 7, g = tid >> 3;
  const int q = blockIdx.x % a.K;
  const int hs = (blockIdx.x / a.K) % a.nhs;
  const int t = blockIdx.x / (a.K * a.nhs);
  const int p = t * a.K + q;
  const int e = a.ids[p];
  const int c0 = hs * 64;

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const uint16_t* base = a.wd + (size_t)e * a.I * a.H + c0 + 8 * l8;
  for (int i = g; i < a.n; i += NT / 8) {
    const int row = SELECT ? a.rows[(size_t)p * a.n + i] : i;
    const float hv = a.h[(size_t)p * a.n + i];
    const uint4 wv = ld_stream16(base + (size_t)row * a.H);
    acc[0] += hv * bf16lo(wv.x); acc[1] += hv * bf16hi(wv.x);
    acc[2] += hv * bf16lo(wv.y); acc[3] += hv * bf16hi(wv.y);
    acc[4] += hv * bf16lo(wv.z); acc[5] += hv * bf16hi(wv.z);
    acc[6] += hv * bf16lo(wv.w); acc[7] += hv * bf16hi(wv.w);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[g][8 * l8 + i] = acc[i];

  if (SELECT && a.r > 0) {
    for (int l = tid; l < a.r; l += NT) zs[l] = a.z[(size_t)p * a.r + l];
    __syncthreads();
    for (int hh = g; hh < 64; hh += NT / 8) {
      const uint16_t* arow = a.A + ((size_t)e * a.H + c0 + hh) * a.r;
      float s = 0.f;
      for (int l = l8; l < a.r; l += 8) s += bf16_to_f32(arow[l]) * zs[l];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if (l8 == 0) yrec[hh] = s;
    }
  }
  __syncthreads();
  if (tid < 64) {
    float y = 0.f;
    for (int gg = 0; gg < NT / 8; ++gg) y += red[gg][tid];
    if (SELECT && a.r > 0) y += yrec[tid];
    a.ypart[(size_t)p * a.H + c0 + tid] = y;
  }
  if (!last_arrival(a.ctr + (size_t)t * a.nhs + hs, (unsigned)a.K, &s_flag)) return;
  if (tid < 64) {
    float o = 0.f;
    for (int qq = 0; qq < a.K; ++qq)
      o += a.w[(size_t)t * a.K + qq] *
           __builtin_nontemporal_load(a.ypart + (size_t)(t * a.K + qq) * a.H + c0 + tid);
    a.out[(size_t)t * a.H + c0 + tid] = f32_to_bf16(o);
  }
}

// ------------------------------------------------------------------------------------ stats

__global__ void k_stats(const int32_t* ids, int P, int E, int I, int H, int k, int c, int r,
                        int T, int K, int select, cfm_stats* st) {
  // one thread: counts routed experts and the rows each launch streams
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
    s.bytes_candidates = Pu * 4ull * H * c;
    s.bytes_down = Pu * 2ull * H * k;
    s.bytes_recovery = r > 0 ? Pu * (2ull * H * r + 2ull * I * r) : 0;
    s.rows_candidates = (uint32_t)(P * c);
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
int launch_gu(const GuArgs& g, int P, int H, hipStream_t stream) {
  const size_t lds = std::max<size_t>(8 * (size_t)g.per, SELECT ? 4 * (size_t)(g.n + g.k) : 0);
  const dim3 grid((unsigned)(P * g.nslot));
  switch (H <= 512 ? 1 : H / 512) {
    case 1: hipLaunchKernelGGL((k_gu<1, SELECT>), grid, dim3(NT), lds, stream, g); break;
    case 2: hipLaunchKernelGGL((k_gu<2, SELECT>), grid, dim3(NT), lds, stream, g); break;
    case 4: hipLaunchKernelGGL((k_gu<4, SELECT>), grid, dim3(NT), lds, stream, g); break;
    case 8: hipLaunchKernelGGL((k_gu<8, SELECT>), grid, dim3(NT), lds, stream, g); break;
    case 16: hipLaunchKernelGGL((k_gu<16, SELECT>), grid, dim3(NT), lds, stream, g); break;
    default: return set_error(CFM_EUNSUPPORTED, "hidden width not supported");
  }
  CFM_LAUNCH_CHECK("k_gu");
  return CFM_OK;
}

}  // namespace

// ------------------------------------------------------------------------------------ plans

ForwardPlan select_plan(int T, int K, int E, int I, int H, int k, int c, int r) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = k; p.c = c; p.r = r;
  const int P = std::max(p.P, 1);
  p.nch = std::min(std::max(1, (512 + P - 1) / P), std::max(1, (I + 3) / 4));
  p.cw = (I + p.nch - 1) / p.nch;
  p.nch = (I + p.cw - 1) / p.cw;
  if (c > 0) {
    p.nex = std::min(std::max(1, (512 + P - 1) / P), std::max(1, (c + 1) / 2));
    p.per_ex = (c + p.nex - 1) / p.nex;
    p.nex = (c + p.per_ex - 1) / p.per_ex;
  }
  p.nhs = H / 64;
  Carve cv;
  const size_t Pz = (size_t)p.P;
  p.off_hhat = cv.take(Pz * I * 4);
  p.off_zpart = cv.take(Pz * p.nch * r * 4);
  p.off_zsum = cv.take(Pz * r * 4);
  p.off_cand = cv.take(Pz * c * 4);
  p.off_hc = cv.take(Pz * c * 4);
  p.off_keep = cv.take(Pz * k * 4);
  p.off_hk = cv.take(Pz * k * 4);
  p.off_z = cv.take(Pz * r * 4);
  p.off_ypart = cv.take(Pz * H * 4);
  p.off_ctr_screen = cv.take(Pz * 4);
  p.off_ctr_exact = cv.take(Pz * 4);
  p.off_ctr_down = cv.take((size_t)T * p.nhs * 4);
  p.bytes = cv.off;
  return p;
}

ForwardPlan dense_plan(int T, int K, int E, int I, int H) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = I; p.c = I; p.r = 0;
  const int P = std::max(p.P, 1);
  p.nex = std::min(std::max(1, (512 + P - 1) / P), std::max(1, (I + 1) / 2));
  p.per_ex = (I + p.nex - 1) / p.nex;
  p.nex = (I + p.per_ex - 1) / p.per_ex;
  p.nhs = H / 64;
  Carve cv;
  const size_t Pz = (size_t)p.P;
  p.off_hhat = cv.take(Pz * I * 4);
  p.off_ypart = cv.take(Pz * H * 4);
  p.off_ctr_down = cv.take((size_t)T * p.nhs * 4);
  p.bytes = cv.off;
  return p;
}

// ------------------------------------------------------------------------------------ launches

int launch_select_forward(const SelectArgs& s, const ForwardPlan& p, hipStream_t stream) {
  char* ws = s.ws;
  float* hhat = reinterpret_cast<float*>(ws + p.off_hhat);
  float* zpart = reinterpret_cast<float*>(ws + p.off_zpart);
  float* zsum = reinterpret_cast<float*>(ws + p.off_zsum);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + p.off_cand);
  float* hc = reinterpret_cast<float*>(ws + p.off_hc);
  int32_t* keep = reinterpret_cast<int32_t*>(ws + p.off_keep);
  float* hk = reinterpret_cast<float*>(ws + p.off_hk);
  float* z = reinterpret_cast<float*>(ws + p.off_z);
  float* ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  unsigned* ctr_screen = reinterpret_cast<unsigned*>(ws + p.off_ctr_screen);
  unsigned* ctr_exact = reinterpret_cast<unsigned*>(ws + p.off_ctr_exact);
  unsigned* ctr_down = reinterpret_cast<unsigned*>(ws + p.off_ctr_down);
  int log2H = 0;
  while ((1 << log2H) < p.H) ++log2H;

  ScreenArgs sa{s.x, s.ids, s.signs, s.tg, s.tu, s.sg, s.su, s.Bt, hhat, zpart, zsum, cand,
                s.cand_out, ctr_screen, p.K, p.I, p.H, log2H, p.c, p.r, p.nch, p.cw};
  const size_t lds_screen = 8 * (size_t)std::max(p.H, (p.I + 1) / 2) +
                            4 * (size_t)std::max(p.H, p.c) + 4 * (size_t)p.cw;
  if (lds_screen > 65536)
    CFM_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_screen),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_screen));
  hipLaunchKernelGGL(k_screen, dim3((unsigned)(p.P * p.nch)), dim3(NT), lds_screen, stream, sa);
  CFM_LAUNCH_CHECK("k_screen");

  if (p.k > 0) {
    GuArgs g{s.x, s.ids, s.w_gate, s.w_up, cand, hc, hhat, zsum, s.Bt, keep, hk, z, s.keep_out,
             ctr_exact, p.K, p.I, p.H, p.c, p.per_ex, p.nex, p.k, p.r};
    int rc = launch_gu<true>(g, p.P, p.H, stream);
    if (rc) return rc;
  }
  DownArgs d{s.ids, s.topk_w, s.w_down_t, keep, hk, s.A, p.k > 0 ? z : zsum, ypart, s.out,
             ctr_down, p.K, p.I, p.H, p.k, p.r, p.nhs};
  hipLaunchKernelGGL((k_down<true>), dim3((unsigned)(p.T * p.nhs * p.K)), dim3(NT), 0, stream, d);
  CFM_LAUNCH_CHECK("k_down");
  if (s.stats) {
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, s.ids, p.P, p.E, p.I, p.H, p.k, p.c,
                       p.r, p.T, p.K, 1, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

int launch_dense_forward(const SelectArgs& s, const ForwardPlan& p, hipStream_t stream) {
  char* ws = s.ws;
  float* h = reinterpret_cast<float*>(ws + p.off_hhat);
  float* ypart = reinterpret_cast<float*>(ws + p.off_ypart);
  unsigned* ctr_down = reinterpret_cast<unsigned*>(ws + p.off_ctr_down);
  GuArgs g{s.x, s.ids, s.w_gate, s.w_up, nullptr, h, nullptr, nullptr, nullptr, nullptr, nullptr,
           nullptr, nullptr, nullptr, p.K, p.I, p.H, p.I, p.per_ex, p.nex, 0, 0};
  int rc = launch_gu<false>(g, p.P, p.H, stream);
  if (rc) return rc;
  DownArgs d{s.ids, s.topk_w, s.w_down_t, nullptr, h, nullptr, nullptr, ypart, s.out, ctr_down,
             p.K, p.I, p.H, p.I, 0, p.nhs};
  hipLaunchKernelGGL((k_down<false>), dim3((unsigned)(p.T * p.nhs * p.K)), dim3(NT), 0, stream, d);
  CFM_LAUNCH_CHECK("k_down");
  if (s.stats) {
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, s.ids, p.P, p.E, p.I, p.H, p.I, p.I, 0,
                       p.T, p.K, 0, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

}  // namespace cfm
