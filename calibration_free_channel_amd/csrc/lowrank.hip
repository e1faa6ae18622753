// Rank-r map of each expert's down projection (offline, once per layer).
//
// "The skipped channels are recovered through a low-rank map of the down
// projections", built from the weights alone (aimodeling.com article on
// arXiv:2610.37386, section "A reader that needs no data at all"). The map is
// the rank-r truncated SVD W_down ~ A Bt^T (Eckart-Young optimal), found on
// the device in float64:
//   G = W_down^T W_down                      (k_gram, tiled fp64 GEMM)
//   Q <- orth(G Q), repeated                  (k_subspace: block subspace
//                                              iteration, CholQR2)
//   every 4 iterations Rayleigh-Ritz: M = Q^T G Q, Jacobi eigen-decomposition
//   M = W L W^T in LDS, Q <- Q W ordered by Ritz value (k_subspace)
//   V_r = the leading r columns of Q
//   Bt = V_r, A = W_down V_r                   (k_lowrank_a)
// The block is r plus 32 columns of oversampling (at most 96, or r if larger,
// and never more than min(I, H), the rank bound of G);
// the iteration runs until the energy the r leading Ritz vectors capture has
// converged (relative change at most 1e-11 between Rayleigh-Ritz steps).
#include <algorithm>

#include "cfm_internal.h"
#include "cfm_launch.h"

namespace cfm {
namespace {

constexpr int LT = 256;   // threads per workgroup

// ------------------------------------------------------------------ Gram matrix
// G[e][i][j] = sum_h Wd_t[e][i][h] Wd_t[e][j][h], 64x64 tiles, K-chunks of 32.
__global__ __launch_bounds__(LT) void k_gram(const uint16_t* __restrict__ wd, int I, int H,
                                             double* __restrict__ G) {
  __shared__ double As[32][65];
  __shared__ double Bs[32][65];
  const int e = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const uint16_t* W = wd + (size_t)e * I * H;
  double acc[4][4] = {};
  for (int h0 = 0; h0 < H; h0 += 32) {
    for (int idx = tid; idx < 64 * 32; idx += LT) {
      const int rr = idx >> 5, cc = idx & 31;
      const int ia = i0 + rr, ib = j0 + rr;
      As[cc][rr] = ia < I ? (double)bf16_to_f32(W[(size_t)ia * H + h0 + cc]) : 0.0;
      Bs[cc][rr] = ib < I ? (double)bf16_to_f32(W[(size_t)ib * H + h0 + cc]) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < 32; ++kk) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { a[u] = As[kk][ty * 4 + u]; b[u] = Bs[kk][tx * 4 + u]; }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  double* Ge = G + (size_t)e * I * I;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty * 4 + u, j = j0 + tx * 4 + v;
      if (i < I && j < I) Ge[(size_t)i * I + j] = acc[u][v];
    }
}

// ------------------------------------------------------------------ one workgroup per expert

__device__ __forceinline__ double hash_uniform(uint64_t a) {
  // SplitMix64 finaliser of a counter -> uniform in [-1, 1)
  uint64_t z = a + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 4503599627370496.0) - 1.0;
}

// Y[I][p] = G[I][I] * Q[I][p]; row blocks of 64, K-chunks of 32 staged in LDS,
// each thread a 4 x ceil(p/16) register tile.
__device__ void gemm_gq(const double* G, const double* Q, double* Y, int I, int p, double* lds) {
  double* Gs = lds;              // [64][33]
  double* Qs = lds + 64 * 33;    // [32][p]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int cpt = (p + 15) / 16;  // <= 8
  for (int r0 = 0; r0 < I; r0 += 64) {
    double acc[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[u][v] = 0.0;
    for (int k0 = 0; k0 < I; k0 += 32) {
      for (int idx = tid; idx < 64 * 32; idx += LT) {
        const int rr = idx >> 5, cc = idx & 31;
        Gs[rr * 33 + cc] = (r0 + rr < I && k0 + cc < I) ? G[(size_t)(r0 + rr) * I + k0 + cc] : 0.0;
      }
      for (int idx = tid; idx < 32 * p; idx += LT) {
        const int rr = idx / p, cc = idx % p;
        Qs[rr * p + cc] = (k0 + rr < I) ? Q[(size_t)(k0 + rr) * p + cc] : 0.0;
      }
      __syncthreads();
      for (int kk = 0; kk < 32; ++kk) {
        double a[4], b[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = Gs[(ty * 4 + u) * 33 + kk];
#pragma unroll
        for (int v = 0; v < 8; ++v) b[v] = (v < cpt && tx + 16 * v < p) ? Qs[kk * p + tx + 16 * v] : 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 8; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int row = r0 + ty * 4 + u, col = tx + 16 * v;
        if (v < cpt && col < p && row < I) Y[(size_t)row * p + col] = acc[u][v];
      }
  }
}

// out[p][p] (LDS) = A^T B for A, B [I][p] in global memory, staged 16 rows at a
// time through LDS; each thread accumulates up to 64 outputs in registers.
// Uses lds[0 .. max(32 p, p p)).
__device__ void gram_ab(const double* A, const double* B, double* lds, int I, int p) {
  const int tid = threadIdx.x;
  double* As = lds;              // [16][p]
  double* Bs = lds + 16 * p;     // [16][p]
  const int nout = p * p;
  double acc[64];
#pragma unroll
  for (int u = 0; u < 64; ++u) acc[u] = 0.0;
  for (int i0 = 0; i0 < I; i0 += 16) {
    for (int idx = tid; idx < 16 * p; idx += LT) {
      const int ii = idx / p, cc = idx % p;
      As[idx] = (i0 + ii < I) ? A[(size_t)(i0 + ii) * p + cc] : 0.0;
      Bs[idx] = (i0 + ii < I) ? B[(size_t)(i0 + ii) * p + cc] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      const int o = tid + u * LT;
      if (o < nout) {
        const int a = o / p, b = o % p;
        double s = acc[u];
#pragma unroll 4
        for (int ii = 0; ii < 16; ++ii) s = fma(As[ii * p + a], Bs[ii * p + b], s);
        acc[u] = s;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const int o = tid + u * LT;
    if (o < nout) lds[o] = acc[u];
  }
  __syncthreads();
}

// In place: Y [I][p] -> Y R^-1 with R^T R = Y^T Y (Cholesky QR); R lives in LDS.
// A column whose pivot falls to 1e-13 * trace / p or below depends on the
// columns before it (to rounding): it is dropped (set to zero, its row of R
// zero) rather than divided by a tiny pivot, which would amplify rounding
// until it overflows. Dropped columns stay zero in later passes.
__device__ void cholqr(double* Y, int I, int p, double* lds, double* sh) {
  gram_ab(Y, Y, lds, I, p);
  double* S = lds;
  const int tid = threadIdx.x;
  if (tid == 0) {
    double tr = 0.0;
    for (int a = 0; a < p; ++a) tr += S[a * p + a];
    sh[0] = tr > 0.0 ? 1e-13 * tr / p : 1e-300;
  }
  __syncthreads();
  for (int k = 0; k < p; ++k) {
    if (tid == 0) {
      const double d2 = S[k * p + k];
      const double d = d2 > sh[0] ? sqrt(d2) : 0.0;
      S[k * p + k] = d;
      sh[1] = d;
    }
    __syncthreads();
    const double d = sh[1];
    for (int b = k + 1 + tid; b < p; b += LT) S[k * p + b] = d > 0.0 ? S[k * p + b] / d : 0.0;
    __syncthreads();
    const int m = p - k - 1;
    for (int o = tid; o < m * m; o += LT) {
      const int a = k + 1 + o / m, b = k + 1 + o % m;
      if (b >= a) S[a * p + b] -= S[k * p + a] * S[k * p + b];
    }
    __syncthreads();
  }
  for (int i = tid; i < I; i += LT) {
    double* y = Y + (size_t)i * p;
    for (int b = 0; b < p; ++b) {
      double s = y[b];
      for (int a = 0; a < b; ++a) s -= y[a] * S[a * p + b];
      const double d = S[b * p + b];
      y[b] = d > 0.0 ? s / d : 0.0;
    }
  }
  __syncthreads();
}

__device__ double block_sum_lr(double v, double* red) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < LT / 64; ++w) s += red[w];
  return s;
}

// Rayleigh-Ritz on the block Q [I][p]: M = Q^T G Q (p x p, padded to even
// size pp with a zero row and column) is diagonalised in LDS by cyclic Jacobi
// with round-robin ordering (each round rotates pp/2 disjoint pairs); its
// eigenvectors W rotate the block, Q <- Q W, with the columns ordered by Ritz
// value, descending (lower index on ties). Returns the sum of the r largest
// Ritz values (the energy tr(V_r^T G V_r) the leading r Ritz vectors
// capture). Y is scratch [I][p]; Wm holds W [pp][pp].
__device__ double rayleigh_ritz(const double* G, double* Q, double* Y, double* Wm, int I, int p, int pp, int r,
                                double* lds, double* sh, double* red, int* order, double* cs) {
  const int tid = threadIdx.x;
  gemm_gq(G, Q, Y, I, p, lds);
  __syncthreads();
  gram_ab(Q, Y, lds, I, p);          // lds[a*p+b] = (Q^T G Q)[a][b]
  double* M = lds;
  if (pp != p) {                     // re-stride to pp in place, back to front
    if (tid == 0)
      for (int a = p - 1; a >= 0; --a)
        for (int b = p - 1; b >= 0; --b) M[a * pp + b] = M[a * p + b];
    __syncthreads();
    for (int o = tid; o < pp * pp; o += LT)
      if (o / pp >= p || o % pp >= p) M[o] = 0.0;
  }
  for (int o = tid; o < pp * pp; o += LT) Wm[o] = (o / pp == o % pp) ? 1.0 : 0.0;
  __syncthreads();
  for (int o = tid; o < pp * pp; o += LT) {          // symmetrise (round-off)
    const int a = o / pp, b = o % pp;
    if (a < b) { const double v = 0.5 * (M[a * pp + b] + M[b * pp + a]); M[a * pp + b] = v; M[b * pp + a] = v; }
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    double off = 0.0, dia = 0.0;
    for (int o = tid; o < pp * pp; o += LT) {
      const double v = M[o] * M[o];
      if (o / pp == o % pp) dia += v; else off += v;
    }
    off = block_sum_lr(off, red);
    dia = block_sum_lr(dia, red);
    if (!(off > 1e-30 * dia)) break;
    for (int rr = 0; rr < pp - 1; ++rr) {
      for (int i = tid; i < pp / 2; i += LT) {
        const int ka = i, kb = pp - 1 - i;
        const int pa = ka == 0 ? 0 : 1 + (ka - 1 + rr) % (pp - 1);
        const int pb = kb == 0 ? 0 : 1 + (kb - 1 + rr) % (pp - 1);
        const int a = min(pa, pb), b = max(pa, pb);
        const double app = M[a * pp + a], aqq = M[b * pp + b], apq = M[a * pp + b];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 1e-300) {
          const double tau = (aqq - app) / (2.0 * apq);
          const double tt = (tau >= 0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + tt * tt);
          s = tt * c;
        }
        cs[4 * i + 0] = c; cs[4 * i + 1] = s;
        cs[4 * i + 2] = (double)a; cs[4 * i + 3] = (double)b;
      }
      __syncthreads();
      for (int o = tid; o < (pp / 2) * pp; o += LT) {      // rows a, b of M <- J^T M
        const int i = o / pp, x = o % pp;
        const double c = cs[4 * i], s = cs[4 * i + 1];
        const int a = (int)cs[4 * i + 2], b = (int)cs[4 * i + 3];
        const double ma = M[a * pp + x], mb = M[b * pp + x];
        M[a * pp + x] = c * ma - s * mb;
        M[b * pp + x] = s * ma + c * mb;
      }
      __syncthreads();
      for (int o = tid; o < (pp / 2) * pp; o += LT) {      // columns a, b of M and W <- M J, W J
        const int i = o / pp, y = o % pp;
        const double c = cs[4 * i], s = cs[4 * i + 1];
        const int a = (int)cs[4 * i + 2], b = (int)cs[4 * i + 3];
        const double ma = M[y * pp + a], mb = M[y * pp + b];
        M[y * pp + a] = c * ma - s * mb;
        M[y * pp + b] = s * ma + c * mb;
        const double wa = Wm[y * pp + a], wb = Wm[y * pp + b];
        Wm[y * pp + a] = c * wa - s * wb;
        Wm[y * pp + b] = s * wa + c * wb;
      }
      __syncthreads();
    }
  }
  // order the real (non-padding) Ritz values, descending, lower index on ties
  if (tid == 0) {
    for (int a = 0; a < p; ++a) order[a] = a;
    for (int a = 1; a < p; ++a) {          // insertion sort, p <= 128
      const int v = order[a];
      const double lv = M[v * pp + v];
      int b = a - 1;
      while (b >= 0 && (M[order[b] * pp + order[b]] < lv ||
                        (M[order[b] * pp + order[b]] == lv && order[b] > v))) {
        order[b + 1] = order[b];
        --b;
      }
      order[b + 1] = v;
    }
    double e = 0.0;
    for (int l = 0; l < r; ++l) e += M[order[l] * pp + order[l]];
    sh[0] = e;
  }
  __syncthreads();
  const double energy = sh[0];
  // Q <- Q W[:, order], through Y
  for (int o = tid; o < I * p; o += LT) {
    const int i = o / p, l = o % p;
    const int col = order[l];
    double s = 0.0;
    for (int a = 0; a < p; ++a) s = fma(Q[(size_t)i * p + a], Wm[a * pp + col], s);
    Y[o] = s;
  }
  __syncthreads();
  for (int o = tid; o < I * p; o += LT) Q[o] = Y[o];
  __syncthreads();
  return energy;
}

// Block subspace iteration Q <- orth(G Q) with a Rayleigh-Ritz step every
// kRitzEvery iterations, until the energy the r leading Ritz vectors capture
// changes by at most 1e-11 of itself between two Rayleigh-Ritz steps (at most
// `iters` iterations). The leading r columns of the rotated block are then the
// map's V_r, written to Y with stride r and each column signed so that its
// largest-magnitude entry is positive (lowest index on ties).
constexpr int kRitzEvery = 4;

__global__ __launch_bounds__(LT) void k_subspace(const double* Gall, double* Qall, double* Yall,
                                                 double* Wall, int I, int p, int pp, int r,
                                                 int iters) {
  extern __shared__ double lds[];      // GEMM staging / Cholesky factor / Jacobi matrix
  __shared__ double sh[2];
  __shared__ double red[LT / 64];
  __shared__ int order[kMaxRank + 2];
  __shared__ double cs[4 * (kMaxRank / 2 + 1)];   // per-pair (c, s, a, b) of one Jacobi round
  const int e = blockIdx.x, tid = threadIdx.x;
  const double* G = Gall + (size_t)e * I * I;
  double* Q = Qall + (size_t)e * I * p;
  double* Y = Yall + (size_t)e * I * p;
  double* W = Wall + (size_t)e * pp * pp;   // Ritz vectors of M

  for (int o = tid; o < I * p; o += LT) Q[o] = hash_uniform(((uint64_t)e << 40) ^ (uint64_t)o);
  __syncthreads();
  cholqr(Q, I, p, lds, sh);
  cholqr(Q, I, p, lds, sh);
  double prev = -1.0;
  for (int it = 1; it <= iters; ++it) {
    gemm_gq(G, Q, Y, I, p, lds);
    __syncthreads();
    cholqr(Y, I, p, lds, sh);
    cholqr(Y, I, p, lds, sh);
    for (int o = tid; o < I * p; o += LT) Q[o] = Y[o];
    __syncthreads();
    if (it % kRitzEvery == 0 || it == iters) {
      const double energy = rayleigh_ritz(G, Q, Y, W, I, p, pp, r, lds, sh, red, order, cs);
      if (fabs(energy - prev) <= 1e-11 * energy) break;
      prev = energy;
    }
  }
  // V_r = the leading r columns of the rotated block, into Y (I x r, stride r)
  double* Vr = Y;
  for (int o = tid; o < I * r; o += LT) {
    const int i = o / r, l = o % r;
    Vr[o] = Q[(size_t)i * p + l];
  }
  __syncthreads();
  // sign: largest-magnitude entry of each column positive (lowest index on ties)
  for (int l = tid; l < r; l += LT) {
    double best = -1.0;
    int bi = 0;
    for (int i = 0; i < I; ++i) {
      const double v = fabs(Vr[(size_t)i * r + l]);
      if (v > best) { best = v; bi = i; }
    }
    if (Vr[(size_t)bi * r + l] < 0)
      for (int i = 0; i < I; ++i) Vr[(size_t)i * r + l] = -Vr[(size_t)i * r + l];
  }
}

// Bt[e] = bf16(V_r); A[e][h][l] = bf16(sum_i Wd_t[e][i][h] V_r[i][l]).
__global__ __launch_bounds__(LT) void k_lowrank_a(const uint16_t* __restrict__ wd,
                                                  const double* __restrict__ Vall, int I, int H,
                                                  int r, int p, uint16_t* __restrict__ A,
                                                  uint16_t* __restrict__ Bt) {
  __shared__ double Ws[32][65];
  extern __shared__ double Vs[];   // [32][r]
  const int e = blockIdx.y, h0 = blockIdx.x * 64, tid = threadIdx.x;
  const double* V = Vall + (size_t)e * I * p;    // V_r stored with stride r in the Y slot
  const uint16_t* W = wd + (size_t)e * I * H;
  if (blockIdx.x == 0)
    for (int o = tid; o < I * r; o += LT)
      Bt[(size_t)e * I * r + o] = f32_to_bf16((float)V[o]);
  const int nout = 64 * r;
  const int per = (nout + LT - 1) / LT;   // <= 32
  double acc[32];
#pragma unroll
  for (int u = 0; u < 32; ++u) acc[u] = 0.0;
  for (int i0 = 0; i0 < I; i0 += 32) {
    for (int idx = tid; idx < 32 * 64; idx += LT) {
      const int ii = idx >> 6, hh = idx & 63;
      Ws[ii][hh] = (i0 + ii < I) ? (double)bf16_to_f32(W[(size_t)(i0 + ii) * H + h0 + hh]) : 0.0;
    }
    for (int idx = tid; idx < 32 * r; idx += LT) {
      const int ii = idx / r, l = idx % r;
      Vs[idx] = (i0 + ii < I) ? V[(size_t)(i0 + ii) * r + l] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      if (u < per) {
        const int o = tid + u * LT;
        if (o < nout) {
          const int hh = o / r, l = o % r;
          double s = acc[u];
          for (int ii = 0; ii < 32; ++ii) s = fma(Ws[ii][hh], Vs[ii * r + l], s);
          acc[u] = s;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    if (u < per) {
      const int o = tid + u * LT;
      if (o < nout) {
        const int hh = o / r, l = o % r;
        A[((size_t)e * H + h0 + hh) * r + l] = f32_to_bf16((float)acc[u]);
      }
    }
  }
}

}  // namespace

LowrankPlan lowrank_plan(int E, int I, int H, int r) {
  LowrankPlan pl{};
  // the block never exceeds the rank bound of G = W_down^T W_down, min(I, H):
  // columns beyond it would only carry rounding
  int p = std::max(r, std::min(r + 32, 96));
  p = std::min(p, std::min(I, H));
  pl.p = std::max(p, 1);     // p <= 128
  pl.iters = 200;             // at most; the iteration stops once the Ritz energy has converged
  const int pp = (pl.p + 1) & ~1;
  Carve cv;
  pl.off_gram = cv.take((size_t)E * I * I * 8);
  pl.off_q = cv.take((size_t)E * I * pl.p * 8);
  pl.off_y = cv.take((size_t)E * I * pl.p * 8);
  pl.off_v = cv.take((size_t)E * pp * pp * 8);
  pl.bytes = cv.off;
  return pl;
}

int launch_lowrank_build(const uint16_t* w_down_t, int E, int I, int H, int r, uint16_t* A,
                         uint16_t* Bt, void* ws, const LowrankPlan& plan, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  double* G = reinterpret_cast<double*>(w + plan.off_gram);
  double* Q = reinterpret_cast<double*>(w + plan.off_q);
  double* Y = reinterpret_cast<double*>(w + plan.off_y);
  double* Wr = reinterpret_cast<double*>(w + plan.off_v);
  const int p = plan.p, pp = (p + 1) & ~1;
  const int ti = (I + 63) / 64;
  hipLaunchKernelGGL(k_gram, dim3(ti, ti, E), dim3(LT), 0, stream, w_down_t, I, H, G);
  CFM_LAUNCH_CHECK("k_gram");
  const size_t lds_gemm = (size_t)(64 * 33 + 32 * p) * 8;
  const size_t lds = std::max(lds_gemm, (size_t)pp * pp * 8);   // <= 128 KiB
  CFM_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_subspace),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL(k_subspace, dim3(E), dim3(LT), lds, stream, G, Q, Y, Wr, I, p, pp, r,
                     plan.iters);
  CFM_LAUNCH_CHECK("k_subspace");
  hipLaunchKernelGGL(k_lowrank_a, dim3(H / 64, E), dim3(LT), (size_t)32 * r * 8, stream, w_down_t,
                     Y, I, H, r, p, A, Bt);
  CFM_LAUNCH_CHECK("k_lowrank_a");
  CFM_HIP_TRY(hipStreamSynchronize(stream));
  return CFM_OK;
}

}  // namespace cfm
