// CPU oracle for the channel-selected routed-expert SwiGLU FFN, plain C++17
// (standard library only), float64 throughout.
//
// TEST INFRASTRUCTURE ONLY. This library is the slow, plain reference the HIP
// library is checked against; only the tests, the smoke check and the CPU
// baseline leg of the benchmark load it (through oracle/cfm_oracle.py). It
// shares no code, header, table or helper with the HIP path: its transform,
// sketch, packing, selection, low-rank map and combine are written here from
// the method's description.
//
// The method (arXiv:2610.37386, "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data": abstract; aimodeling.com article on
// it, sections "Swapping the threshold for top-k" and "A reader that needs no
// data at all"): each routed (token, expert) pair screens its expert's
// intermediate channels with a rotated ternary sketch of the gate and up
// projections, keeps the top-k channels by exact BF16 activations (no
// calibrated threshold), reads only those channels' down-projection weights,
// and adds back the skipped channels through a low-rank map of the down
// projection built from the weights alone. The pages give no formulas; the
// plain readings taken where they are silent are stated at each step.
//
// Layouts: expert weights [E][I][H] as raw BF16 bits; the down projection is
// channel-major (row j is column j of W_down). All arrays are host memory,
// row-major.
//
// Every function is pinned by the tests in tests/test_oracle_*.py against
// closed forms, independent constructions, library routines or brute force.
// A test can plant a named mistake (cfo_set_mutation) to check that a pin
// catches it; with no mutation set the code below is the method.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

namespace {

// ----------------------------------------------------------------------------- planted mistakes (tests only)

std::string g_mutation;
bool mut(const char* name) { return !g_mutation.empty() && g_mutation == name; }

// ----------------------------------------------------------------------------- numerics

// BF16 bits -> value: the 16 bits are the top half of an IEEE binary32.
double bf16_value(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// value -> BF16 bits, rounded once to nearest with ties to even, written from
// the format: 8 significant bits, smallest normal 2^-126, subnormal spacing
// 2^-133, overflow to infinity, NaN to the quiet pattern 0x7FC0.
uint16_t bf16_bits(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                       // a = m 2^e, 0.5 <= m < 1
  e = std::max(e, -125);                   // below 2^-126 the spacing stays 2^-133
  const double q = std::nearbyint(std::ldexp(a, 8 - e));   // significand in units of the spacing (ties even)
  const double val = std::ldexp(q, e - 8);
  if (val >= std::ldexp(1.0, 128)) return sign | 0x7F80;
  const float f = static_cast<float>(val);  // exact: val has at most 8 significant bits in range
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return sign | static_cast<uint16_t>(u >> 16);
}

double silu(double z) {
  if (mut("silu_sign")) return z / (1.0 + std::exp(z));
  return z / (1.0 + std::exp(-z));
}

// ----------------------------------------------------------------------------- rotation

uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  // output i (from 0): the state after i + 1 golden-ratio increments, then two
  // xor-shift-multiply rounds and a final xor-shift (Steele, Lea and Flood,
  // "Fast splittable pseudorandom number generators", OOPSLA 2014)
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool is_pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }

// In-place fast Walsh-Hadamard transform (unnormalised, natural / Sylvester
// order) of one vector: after it, v'_i = sum_j (-1)^popcount(i & j) v_j.
void fwht(double* v, long H) {
  for (long h = 1; h < H; h <<= 1)
    for (long i = 0; i < H; i += 2 * h)
      for (long j = i; j < i + h; ++j) {
        const double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

// T(v) = Hadamard (d . v): the random-sign Walsh-Hadamard rotation the sketch
// is built with (reading of "rotated", article section "A reader that needs
// no data at all"), one sign vector per layer; the 1/sqrt(H) factors of the
// orthonormal rotation are folded into the sketch scale.
void rotate_row(const double* v, const int8_t* d, long H, double* out) {
  for (long i = 0; i < H; ++i) out[i] = mut("rotate_ignores_signs") ? v[i] : v[i] * d[i];
  fwht(out, H);
}

// ----------------------------------------------------------------------------- ternary sketch

constexpr double kTwnDelta = 0.7;   // Ternary Weight Networks threshold factor (Li & Liu, 2016)

// Ternary Weight Networks on one rotated row: delta = 0.7 mean|w~|; t = +1
// above delta, -1 below -delta, 0 otherwise (exactly at the threshold: 0);
// alpha = mean |w~| over the nonzero codes (0 if none).
void ternarize_row(const double* wt, long H, int8_t* codes, double* alpha) {
  double s1 = 0.0;
  for (long i = 0; i < H; ++i) s1 += std::fabs(wt[i]);
  const double delta = (mut("twn_delta_half") ? 0.5 : kTwnDelta) * (s1 / static_cast<double>(H));
  double s2 = 0.0;
  long n = 0;
  for (long i = 0; i < H; ++i) {
    const bool pos = mut("threshold_inclusive") ? wt[i] >= delta : wt[i] > delta;
    const bool neg = mut("threshold_inclusive") ? wt[i] <= -delta : wt[i] < -delta;
    codes[i] = pos ? 1 : (neg ? -1 : 0);
    if (codes[i] != 0) {
      s2 += std::fabs(wt[i]);
      ++n;
    }
  }
  *alpha = n > 0 ? s2 / static_cast<double>(n) : 0.0;
  if (mut("scale_mean_all")) *alpha = s1 / static_cast<double>(H);
}

// Pack: value 16b+q (q < 8) and value 16b+8+q share nibble q of the
// little-endian 32-bit word b: bit 4q = nz(t[16b+8+q]), 4q+1 = nz(t[16b+q]),
// 4q+2 = neg(t[16b+8+q]), 4q+3 = neg(t[16b+q]). (The pages say only that the
// sketch is ternary; this layout is a reading.)
void pack_row(const int8_t* codes, long H, uint8_t* out) {
  for (long b = 0; b < H / 16; ++b) {
    uint32_t w = 0;
    for (int q = 0; q < 8; ++q) {
      int8_t lo = codes[16 * b + q], hi = codes[16 * b + 8 + q];
      if (mut("pack_sign_swap")) { lo = -lo; hi = -hi; }
      w |= (uint32_t)(hi != 0) << (4 * q) | (uint32_t)(lo != 0) << (4 * q + 1) |
           (uint32_t)(hi < 0) << (4 * q + 2) | (uint32_t)(lo < 0) << (4 * q + 3);
    }
    for (int byte = 0; byte < 4; ++byte) out[4 * b + byte] = static_cast<uint8_t>(w >> (8 * byte));
  }
}

void unpack_row(const uint8_t* packed, long H, int8_t* codes) {
  for (long b = 0; b < H / 16; ++b) {
    uint32_t w = 0;
    for (int byte = 0; byte < 4; ++byte) w |= static_cast<uint32_t>(packed[4 * b + byte]) << (8 * byte);
    for (int q = 0; q < 8; ++q) {
      const uint32_t nz_hi = (w >> (4 * q)) & 1, nz_lo = (w >> (4 * q + 1)) & 1;
      const uint32_t ng_hi = (w >> (4 * q + 2)) & 1, ng_lo = (w >> (4 * q + 3)) & 1;
      codes[16 * b + q] = nz_lo ? (ng_lo ? -1 : 1) : 0;
      codes[16 * b + 8 + q] = nz_hi ? (ng_hi ? -1 : 1) : 0;
    }
  }
}

// One BF16 row -> (codes, scale = float32(alpha / H)).
void sketch_row(const uint16_t* w, const int8_t* signs, long H, int8_t* codes, float* scale,
                std::vector<double>& v, std::vector<double>& wt) {
  for (long i = 0; i < H; ++i) v[i] = bf16_value(w[i]);
  rotate_row(v.data(), signs, H, wt.data());
  double alpha;
  ternarize_row(wt.data(), H, codes, &alpha);
  *scale = static_cast<float>(alpha / static_cast<double>(H));
}

// ----------------------------------------------------------------------------- low-rank map

// A team of threads that run the same function over a range in lock-step
// rounds (fork once, then one barrier per round).
class Team {
 public:
  explicit Team(int n) : n_(std::max(1, n)) {}
  // f(tid, nthreads) for each round; rounds() returns false to stop
  template <typename Round>
  void run(long rounds, Round f) {
    if (n_ == 1) {
      for (long r = 0; r < rounds; ++r) f(r, 0, 1);
      return;
    }
    std::atomic<long> arrived{0};
    auto barrier = [&](long& phase) {
      ++phase;
      arrived.fetch_add(1);
      while (arrived.load() < phase * n_) std::this_thread::yield();
    };
    std::vector<std::thread> th;
    for (int t = 0; t < n_; ++t)
      th.emplace_back([&, t] {
        long phase = 0;
        for (long r = 0; r < rounds; ++r) {
          f(r, t, n_);
          barrier(phase);
        }
      });
    for (auto& x : th) x.join();
  }

 private:
  int n_;
};

// Right singular vectors of an m x n matrix M with m >= n, given as its n
// columns of length m (column j at M[j * m ...], overwritten). When m > n a
// Householder QR first reduces M to its n x n triangular factor R (M = Q R, so
// M and R share singular values and right singular vectors). One-sided Jacobi
// (Hestenes) then rotates pairs of columns of R until all are mutually
// orthogonal: R V = U_R Sigma, with V the accumulated rotations. On return
// sv[j] is the length of rotated column j (a singular value) and V [n][n]
// holds the matching right singular vector j at V[j * n ...].
void right_singular(long m, long n, std::vector<double>& M, int nthreads, std::vector<double>& sv,
                    std::vector<double>& V) {
  Team team(n >= 64 ? nthreads : 1);
  const long L = n;                              // length of the columns Jacobi works on
  std::vector<double> Rm((size_t)n * L, 0.0);    // column j at Rm[j * L ...]
  if (m > n) {
    std::vector<double> v(m);
    double vv = 0;
    // round 2k: one thread forms the reflector of column k (v, vv); round
    // 2k + 1: the threads apply it to columns k + 1 .. n - 1
    team.run(2 * n, [&](long ro, int tid, int nt) {
      const long k = ro / 2;
      if ((ro & 1) == 0) {
        if (tid != 0) return;
        double* ck = &M[(size_t)k * m];
        double norm = 0;
        for (long i = k; i < m; ++i) norm += ck[i] * ck[i];
        norm = std::sqrt(norm);
        const double alpha = ck[k] >= 0 ? -norm : norm;   // reflect onto alpha e_k
        for (long i = 0; i < m; ++i) v[i] = i < k ? 0.0 : ck[i];
        v[k] -= alpha;
        vv = 0;
        for (long i = k; i < m; ++i) vv += v[i] * v[i];
        for (long i = 0; i < k; ++i) Rm[(size_t)k * L + i] = ck[i];
        Rm[(size_t)k * L + k] = vv > 0 ? alpha : ck[k];
        return;
      }
      if (vv <= 0) return;
      for (long j = k + 1 + tid; j < n; j += nt) {
        double* cj = &M[(size_t)j * m];
        double d = 0;
        for (long i = k; i < m; ++i) d += v[i] * cj[i];
        const double f = 2.0 * d / vv;
        for (long i = k; i < m; ++i) cj[i] -= f * v[i];
      }
    });
  } else {
    std::copy(M.begin(), M.begin() + (size_t)n * L, Rm.begin());
  }
  V.assign((size_t)n * n, 0.0);
  for (long j = 0; j < n; ++j) V[(size_t)j * n + j] = 1.0;
  // round-robin ordering: n (padded to even) columns in n - 1 rounds of
  // disjoint pairs, so the pairs of a round are rotated at once
  const long np = n + (n & 1);
  std::vector<long> perm(np);
  std::iota(perm.begin(), perm.end(), 0);
  std::vector<double> offmax(std::max(1, nthreads) + 1, 0.0);
  auto rotate_pair = [&](long p, long q, double* off) {
    double* a = &Rm[(size_t)p * L];
    double* b = &Rm[(size_t)q * L];
    double al[4] = {0, 0, 0, 0}, be[4] = {0, 0, 0, 0}, ga[4] = {0, 0, 0, 0};
    long i = 0;
    for (; i + 4 <= L; i += 4)
      for (int u = 0; u < 4; ++u) {
        al[u] += a[i + u] * a[i + u];
        be[u] += b[i + u] * b[i + u];
        ga[u] += a[i + u] * b[i + u];
      }
    for (; i < L; ++i) {
      al[0] += a[i] * a[i];
      be[0] += b[i] * b[i];
      ga[0] += a[i] * b[i];
    }
    const double alpha = (al[0] + al[1]) + (al[2] + al[3]);
    const double beta = (be[0] + be[1]) + (be[2] + be[3]);
    const double gamma = (ga[0] + ga[1]) + (ga[2] + ga[3]);
    if (gamma == 0.0) return;
    const double rel = std::fabs(gamma) / std::sqrt(alpha * beta);
    if (rel > *off) *off = rel;
    if (rel < 1e-15) return;
    const double zeta = (beta - alpha) / (2.0 * gamma);
    const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
    const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
    for (long i2 = 0; i2 < L; ++i2) {
      const double x = a[i2], y = b[i2];
      a[i2] = cs * x - sn * y;
      b[i2] = sn * x + cs * y;
    }
    double* va = &V[(size_t)p * n];
    double* vb = &V[(size_t)q * n];
    for (long i3 = 0; i3 < n; ++i3) {
      const double x = va[i3], y = vb[i3];
      va[i3] = cs * x - sn * y;
      vb[i3] = sn * x + cs * y;
    }
  };
  for (int sweep = 0; sweep < 60; ++sweep) {
    std::fill(offmax.begin(), offmax.end(), 0.0);
    // round ro: pairs (ring_ro[i], ring_ro[np - 1 - i]) with ring_ro the ring
    // rotated ro times (position 0 fixed)
    team.run(np - 1, [&](long ro, int tid, int nt) {
      auto at = [&](long i) -> long {
        if (i == 0) return perm[0];
        const long mm = np - 1;
        return perm[1 + ((i - 1 - ro) % mm + mm) % mm];
      };
      for (long i = tid; i < np / 2; i += nt) {
        long p = at(i), q = at(np - 1 - i);
        if (p >= n || q >= n) continue;
        if (p > q) std::swap(p, q);
        rotate_pair(p, q, &offmax[tid]);
      }
    });
    double off = 0;
    for (double o : offmax) off = std::max(off, o);
    if (off < 1e-14) break;
  }
  sv.assign(n, 0.0);
  for (long j = 0; j < n; ++j) {
    double s2 = 0;
    for (long i = 0; i < L; ++i) s2 += Rm[(size_t)j * L + i] * Rm[(size_t)j * L + i];
    sv[j] = std::sqrt(s2);
  }
}

// Truncated SVD of W_down (H x I). Reading of "a low-rank map of the down
// projections" (article section "A reader that needs no data at all"): the
// best rank-r approximation (Eckart-Young), W_down ~ A B with A = U_r Sigma_r
// and B = V_r^T. When H >= I the right singular vectors V come from W_down
// itself; when H < I from W_down^T, whose right singular vectors are W_down's
// left ones U, with V_l = W_down^T U_l / sigma_l (a zero column in both
// factors where sigma_l = 0, which happens only when the rank is below r).
// Singular values are taken in decreasing order (lower index first on ties).
// Each column of V_r is signed so that its largest-magnitude entry (lowest
// index on ties) is positive, and A_l = W_down V_l (= sigma_l U_l).
int lowrank_one(long I, long H, const double* wdt, long r, double* A, double* Bt, int nthreads) {
  if (r < 0 || r > std::min(H, I)) return -1;
  if (r == 0) return 0;
  const bool tall = H >= I;
  const long n = tall ? I : H;
  std::vector<double> M((size_t)I * H), sv, V;
  if (tall) {
    std::copy(wdt, wdt + (size_t)I * H, M.begin());       // column j of W_down = row j of wdt
  } else {
    for (long j = 0; j < I; ++j)                          // column i of W_down^T = row i of W_down
      for (long i = 0; i < H; ++i) M[(size_t)i * I + j] = wdt[(size_t)j * H + i];
  }
  right_singular(tall ? H : I, n, M, nthreads, sv, V);
  std::vector<long> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](long x, long y) { return sv[x] > sv[y]; });
  std::vector<double> b(I);
  for (long l = 0; l < r; ++l) {
    const long j = order[l];
    const double* v = &V[(size_t)j * n];
    if (tall) {
      std::copy(v, v + I, b.begin());
    } else {
      const double inv = sv[j] > 0 ? 1.0 / sv[j] : 0.0;
      for (long jj = 0; jj < I; ++jj) {
        double d = 0;
        for (long i = 0; i < H; ++i) d += wdt[(size_t)jj * H + i] * v[i];
        b[jj] = d * inv;
      }
    }
    long jm = 0;
    for (long i = 1; i < I; ++i)
      if (std::fabs(b[i]) > std::fabs(b[jm])) jm = i;
    const double sgn = b[jm] < 0 ? -1.0 : 1.0;
    for (long i = 0; i < I; ++i) Bt[i * r + l] = sgn * b[i];
    // A_l = W_down V_l = sum_j V_l[j] (column j of W_down), the l-th column of U Sigma
    const double scale = mut("map_without_singular_values") ? 1.0 / std::max(sv[j], 1e-300) : 1.0;
    for (long i = 0; i < H; ++i) A[i * r + l] = 0.0;
    for (long jj = 0; jj < I; ++jj) {
      const double c = sgn * scale * b[jj];
      const double* col = wdt + (size_t)jj * H;
      for (long i = 0; i < H; ++i) A[i * r + l] += c * col[i];
    }
  }
  return 0;
}

// ----------------------------------------------------------------------------- selection

// The k largest scores by (score desc, index asc), by a full sort; NaN counts
// as 0; returned in ascending index order. (Top-k keeps each token's k
// highest-scoring channels: abstract; ties to the lower index.)
void topk(const double* s, long n, long k, int64_t* out) {
  std::vector<long> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  auto val = [&](long i) { return std::isnan(s[i]) ? 0.0 : s[i]; };
  std::sort(idx.begin(), idx.end(), [&](long a, long b) {
    const double va = val(a), vb = val(b);
    if (va != vb) return va > vb;
    return mut("topk_tie_high") ? a > b : a < b;
  });
  k = std::min(k, n);
  std::vector<long> sel(idx.begin(), idx.begin() + k);
  std::sort(sel.begin(), sel.end());
  for (long i = 0; i < k; ++i) out[i] = sel[i];
}

// {j : s_j >= tau} in ascending order (NaN counts as 0): the keep rule that
// top-k replaces (abstract; article section "Calibrated thresholds do not pin
// down how much you read"). Returns the count.
long threshold(const double* s, long n, double tau, int64_t* out) {
  long m = 0;
  for (long i = 0; i < n; ++i) {
    const double v = std::isnan(s[i]) ? 0.0 : s[i];
    if (mut("threshold_strict") ? v > tau : v >= tau) out[m++] = i;
  }
  return m;
}

// ----------------------------------------------------------------------------- one routed pair

struct PairIn {
  long I, H, r;
  const uint16_t* x;                       // [H]
  const uint16_t *wg, *wu, *wd;            // [I][H] of the pair's expert
  const uint8_t *tg, *tu;                  // [I][H/4]
  const float *sg, *su;                    // [I]
  const int8_t* signs;                     // [H]
  const double *A, *Bt;                    // [H][r], [I][r] (values of the stored map)
  long k, c;
  int recovery;                            // 0 sketch, 1 candidates_exact
  int use_tau;
  double tau;
};
struct PairOut {
  double* hhat;      // [I]
  int64_t* C;        // [c]
  double* h_all;     // [I]
  int64_t* S;        // [c] (first nS used)
  long nS;
  double* y;         // [H]
};

// Sketch activations of every channel: ghat_j = sg_j (t^g_j . T(x)), uhat_j
// likewise, hhat_j = SiLU(ghat_j) uhat_j (screen; article section "A reader
// that needs no data at all").
void screen(const PairIn& in, double* hhat) {
  const long H = in.H;
  std::vector<double> x(H), xt(H);
  for (long i = 0; i < H; ++i) x[i] = bf16_value(in.x[i]);
  rotate_row(x.data(), in.signs, H, xt.data());
  std::vector<int8_t> cg(H), cu(H);
  for (long j = 0; j < in.I; ++j) {
    unpack_row(in.tg + (size_t)j * (H / 4), H, cg.data());
    unpack_row(in.tu + (size_t)j * (H / 4), H, cu.data());
    double dg = 0, du = 0;
    for (long i = 0; i < H; ++i) {
      dg += cg[i] * xt[i];
      du += cu[i] * xt[i];
    }
    const double g = static_cast<double>(in.sg[j]) * dg, u = static_cast<double>(in.su[j]) * du;
    hhat[j] = silu(g) * u;
  }
}

// Exact activations h_j = SiLU(Wg_j . x) (Wu_j . x) from the native BF16 rows
// ("the top-k is computed exactly from the native BF16 weights").
void exact_rows(const uint16_t* x, const uint16_t* wg, const uint16_t* wu, long I, long H, double* h) {
  std::vector<double> xv(H);
  for (long i = 0; i < H; ++i) xv[i] = bf16_value(x[i]);
  for (long j = 0; j < I; ++j) {
    const uint16_t* g_row = (mut("gate_up_swapped") ? wu : wg) + (size_t)j * H;
    const uint16_t* u_row = (mut("gate_up_swapped") ? wg : wu) + (size_t)j * H;
    double g = 0, u = 0;
    for (long i = 0; i < H; ++i) {
      g += bf16_value(g_row[i]) * xv[i];
      u += bf16_value(u_row[i]) * xv[i];
    }
    h[j] = silu(g) * u;
  }
}

void pair_output(const PairIn& in, const double* hhat, const double* h_all, const int64_t* C, long nC,
                 const int64_t* S, long nS, double* y);

// The method for one pair: C = top-c of |hhat|; S = top-k of C by |h| (or the
// threshold rule on the same score); y = sum_{j in S} h_j Wd_j (ascending j)
// + A z, z = sum_{j not in S} a_j Bt_j with a_j = hhat_j (every skipped
// channel, including candidates screened in but not kept), or, with the
// candidates_exact variant, a_j = h_j for j in C \ S.
void select_pair(const PairIn& in, PairOut& out) {
  const long I = in.I, H = in.H, r = in.r;
  screen(in, out.hhat);
  std::vector<double> ah(I);
  for (long j = 0; j < I; ++j) ah[j] = std::fabs(out.hhat[j]);
  topk(ah.data(), I, in.c, out.C);
  exact_rows(in.x, in.wg, in.wu, I, H, out.h_all);
  std::vector<double> hc(in.c);
  for (long i = 0; i < in.c; ++i) hc[i] = std::fabs(out.h_all[out.C[i]]);
  std::vector<int64_t> pos(in.c);
  long nS;
  if (in.use_tau) {
    nS = threshold(hc.data(), in.c, in.tau, pos.data());
  } else if (in.k > 0) {
    if (mut("keep_by_sketch_score"))
      for (long i = 0; i < in.c; ++i) hc[i] = ah[out.C[i]];
    topk(hc.data(), in.c, in.k, pos.data());
    nS = std::min(in.k, in.c);
  } else {
    nS = 0;
  }
  for (long i = 0; i < nS; ++i) out.S[i] = out.C[pos[i]];
  out.nS = nS;
  pair_output(in, out.hhat, out.h_all, out.C, in.c, out.S, nS, out.y);
}

// y for given candidate and kept sets (the down projection over S and the
// recovery of the rest), from the activations hhat and h_all.
void pair_output(const PairIn& in, const double* hhat, const double* h_all, const int64_t* C, long nC,
                 const int64_t* S, long nS, double* y) {
  const long I = in.I, H = in.H, r = in.r;
  struct Out { double* y; } out{y};
  for (long i = 0; i < H; ++i) out.y[i] = 0.0;
  for (long m = 0; m < nS; ++m) {
    const long j = S[m];
    const double hj = h_all[j];
    const uint16_t* row = in.wd + (size_t)j * H;
    for (long i = 0; i < H; ++i) out.y[i] += hj * bf16_value(row[i]);
  }
  if (r > 0) {
    std::vector<double> coef(hhat, hhat + I);
    if (in.recovery == 1)
      for (long i = 0; i < nC; ++i) coef[C[i]] = h_all[C[i]];
    std::vector<char> skip(I, 1);
    for (long m = 0; m < nS; ++m) skip[S[m]] = 0;
    if (mut("recovery_unscreened_only"))
      for (long i = 0; i < nC; ++i) skip[C[i]] = 0;
    if (mut("candidates_exact_everywhere") && in.recovery == 1)
      for (long j = 0; j < I; ++j) coef[j] = h_all[j];
    std::vector<double> z(r, 0.0);
    for (long j = 0; j < I; ++j)
      if (skip[j])
        for (long l = 0; l < r; ++l) z[l] += coef[j] * in.Bt[(size_t)j * r + l];
    for (long i = 0; i < H; ++i) {
      double s = 0;
      for (long l = 0; l < r; ++l) s += in.A[(size_t)i * r + l] * z[l];
      out.y[i] += s;
    }
  }
}

// out = BF16( resid + sum_q w_q y_q ), one rounding (weights used as given).
void combine(const double* ys, const double* w, long K, long H, const uint16_t* resid, uint16_t* out) {
  for (long i = 0; i < H; ++i) {
    double acc = 0;
    for (long q = 0; q < K; ++q) acc += w[q] * ys[q * H + i];
    if (resid) {
      if (mut("residual_rounded_separately"))
        acc = bf16_value(bf16_bits(acc)) + bf16_value(resid[i]);
      else
        acc += bf16_value(resid[i]);
    }
    out[i] = bf16_bits(acc);
  }
}

template <typename F>
void parallel_for(long n, int nthreads, F f) {
  const int nt = std::max(1, std::min<int>(nthreads, (int)std::max<long>(n, 1)));
  if (nt == 1) {
    for (long i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([&, t] {
      for (long i = t; i < n; i += nt) f(i);
    });
  for (auto& x : th) x.join();
}

}  // namespace

extern "C" {

int cfo_set_mutation(const char* name) {
  g_mutation = name ? name : "";
  return 0;
}

void cfo_bf16_to_f64(long n, const uint16_t* in, double* out) {
  for (long i = 0; i < n; ++i) out[i] = bf16_value(in[i]);
}
void cfo_f64_to_bf16(long n, const double* in, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = bf16_bits(in[i]);
}
void cfo_silu(long n, const double* in, double* out) {
  for (long i = 0; i < n; ++i) out[i] = silu(in[i]);
}

void cfo_splitmix64(uint64_t seed, long n, uint64_t* out) {
  for (long i = 0; i < n; ++i) out[i] = splitmix64_at(seed, (uint64_t)i);
}
// d_i = -1 if bit 63 of output i is set, else +1 (reading: the pages do not
// say how the rotation is drawn).
void cfo_rotation_signs(uint64_t seed, long H, int8_t* out) {
  for (long i = 0; i < H; ++i) out[i] = (splitmix64_at(seed, (uint64_t)i) >> 63) ? -1 : 1;
}

int cfo_hadamard(long H, double* out) {
  if (!is_pow2(H)) return -1;
  for (long i = 0; i < H; ++i)
    for (long j = 0; j < H; ++j) out[i * H + j] = (__builtin_popcountl(i & j) & 1) ? -1.0 : 1.0;
  return 0;
}

int cfo_rotate(long n, long H, const double* v, const int8_t* signs, double* out) {
  if (!is_pow2(H)) return -1;
  for (long r = 0; r < n; ++r) rotate_row(v + r * H, signs, H, out + r * H);
  return 0;
}

void cfo_ternarize(long n, long H, const double* wt, int8_t* codes, double* alpha) {
  for (long r = 0; r < n; ++r) ternarize_row(wt + r * H, H, codes + r * H, alpha + r);
}

int cfo_sketch_rows(long n, long H, const uint16_t* w, const int8_t* signs, int8_t* codes, float* scale) {
  if (!is_pow2(H)) return -1;
  std::vector<double> v(H), wt(H);
  for (long r = 0; r < n; ++r) sketch_row(w + r * H, signs, H, codes + r * H, scale + r, v, wt);
  return 0;
}

int cfo_pack_codes(long n, long H, const int8_t* codes, uint8_t* packed) {
  if (H % 16) return -1;
  if (mut("pack_natural_order")) {
    for (long r = 0; r < n; ++r)
      for (long b = 0; b < H / 4; ++b) {
        uint8_t v = 0;
        for (int q = 0; q < 4; ++q) {
          const int8_t t = codes[r * H + 4 * b + q];
          v |= (uint8_t)((t == 1 ? 1 : t == -1 ? 3 : 0) << (2 * q));
        }
        packed[r * (H / 4) + b] = v;
      }
    return 0;
  }
  for (long r = 0; r < n; ++r) pack_row(codes + r * H, H, packed + r * (H / 4));
  return 0;
}

int cfo_unpack_codes(long n, long H, const uint8_t* packed, int8_t* codes) {
  if (H % 16) return -1;
  for (long r = 0; r < n; ++r) unpack_row(packed + r * (H / 4), H, codes + r * H);
  return 0;
}

// Sketch of every expert's gate and up rows: tg, tu [E][I][H/4], sg, su [E][I].
int cfo_sketch_build(long E, long I, long H, const uint16_t* wg, const uint16_t* wu, const int8_t* signs,
                     uint8_t* tg, uint8_t* tu, float* sg, float* su, int nthreads) {
  if (!is_pow2(H) || H < 16) return -1;
  parallel_for(2 * E, nthreads, [&](long m) {
    const bool up = m >= E;
    const long e = up ? m - E : m;
    const uint16_t* w = (up ? wu : wg) + (size_t)e * I * H;
    std::vector<double> v(H), wt(H);
    std::vector<int8_t> codes(H);
    for (long j = 0; j < I; ++j) {
      float scale;
      sketch_row(w + (size_t)j * H, signs, H, codes.data(), &scale, v, wt);
      pack_row(codes.data(), H, (up ? tu : tg) + ((size_t)e * I + j) * (H / 4));
      (up ? su : sg)[(size_t)e * I + j] = scale;
    }
  });
  return 0;
}

// wdt: one expert's channel-major down projection as values [I][H].
int cfo_lowrank(long I, long H, const double* wdt, long r, double* A, double* Bt, int nthreads) {
  return lowrank_one(I, H, wdt, r, A, Bt, nthreads);
}

void cfo_topk_set(long n, const double* scores, long k, int64_t* out) { topk(scores, n, k, out); }
long cfo_threshold_set(long n, const double* scores, double tau, int64_t* out) {
  return threshold(scores, n, tau, out);
}

// The threshold that keeps k per pair on average over n calibration pairs:
// the (k n)-th largest pooled score (NaN as 0); +inf for k n = 0; NaN if
// k n exceeds the pooled count.
double cfo_calibrate_threshold(long npool, const double* pooled, long nsets, long k) {
  const long m = k * nsets;
  if (m <= 0) return std::numeric_limits<double>::infinity();
  if (m > npool) return std::numeric_limits<double>::quiet_NaN();
  std::vector<double> v(pooled, pooled + npool);
  for (double& x : v)
    if (std::isnan(x)) x = 0.0;
  std::sort(v.begin(), v.end(), [](double a, double b) { return a > b; });
  return v[(size_t)(mut("calibration_off_by_one") ? m : m - 1)];
}

int cfo_screen_scores(long I, long H, const uint16_t* x, const uint8_t* tg, const uint8_t* tu, const float* sg,
                      const float* su, const int8_t* signs, double* hhat) {
  if (!is_pow2(H)) return -1;
  PairIn in{};
  in.I = I; in.H = H; in.x = x; in.tg = tg; in.tu = tu; in.sg = sg; in.su = su; in.signs = signs;
  screen(in, hhat);
  return 0;
}

void cfo_exact_activations(long I, long H, const uint16_t* x, const uint16_t* wg, const uint16_t* wu, double* h) {
  exact_rows(x, wg, wu, I, H, h);
}

int cfo_select_pair(long I, long H, long r, const uint16_t* x, const uint16_t* wg, const uint16_t* wu,
                    const uint16_t* wd, const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                    const int8_t* signs, const double* A, const double* Bt, long k, long c, int recovery, int use_tau,
                    double tau, double* hhat, int64_t* C, double* h_all, int64_t* S, long* nS, double* y) {
  if (!is_pow2(H) || c > I || k > c || k < 0 || c < 0) return -1;
  PairIn in{I, H, r, x, wg, wu, wd, tg, tu, sg, su, signs, A, Bt, k, c, recovery, use_tau, tau};
  PairOut out{hhat, C, h_all, S, 0, y};
  select_pair(in, out);
  *nS = out.nS;
  return 0;
}

void cfo_combine(long K, long H, const double* ys, const double* w, const uint16_t* resid, uint16_t* out) {
  combine(ys, w, K, H, resid, out);
}

// The selected layer over a batch: tokens[0..nt) (indices into x, ids, w),
// pairs spread over nthreads threads. A [E][H][r] and Bt [E][I][r] values.
// Per-pair details (hhat, C, h_all, S, nS, y; pair n = token slot n of the
// list times K plus q) are written when the pointers are given.
int cfo_select_forward(long T, long K, long E, long I, long H, long r, const uint16_t* x, const int32_t* ids,
                       const double* w, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, const uint8_t* tg,
                       const uint8_t* tu, const float* sg, const float* su, const int8_t* signs, const double* A,
                       const double* Bt, long k, long c, int recovery, int use_tau, double tau, const uint16_t* resid,
                       const int64_t* tokens, long ntok, int nthreads, uint16_t* out, double* hhat, int64_t* C,
                       double* h_all, int64_t* S, long* nS, double* y) {
  if (!is_pow2(H) || c > I || k > c || k < 0 || c < 0) return -1;
  const long P = ntok * K;
  std::vector<double> ys((size_t)P * H), hh, ha;
  std::vector<int64_t> cc, ss;
  std::vector<long> ns(P);
  if (!hhat) hh.resize((size_t)P * I);
  if (!h_all) ha.resize((size_t)P * I);
  if (!C) cc.resize((size_t)P * std::max<long>(c, 1));
  if (!S) ss.resize((size_t)P * std::max<long>(c, 1));
  for (long n = 0; n < ntok; ++n)
    if (tokens[n] < 0 || tokens[n] >= T) return -1;
  parallel_for(P, nthreads, [&](long pn) {
    const long t = tokens[pn / K], q = pn % K;
    const long e = ids[t * K + q];
    PairIn in{I, H, r, x + (size_t)t * H, wg + (size_t)e * I * H, wu + (size_t)e * I * H, wd + (size_t)e * I * H,
              tg + (size_t)e * I * (H / 4), tu + (size_t)e * I * (H / 4), sg + (size_t)e * I, su + (size_t)e * I,
              signs, A ? A + (size_t)e * H * r : nullptr, Bt ? Bt + (size_t)e * I * r : nullptr, k, c, recovery,
              use_tau, tau};
    PairOut po{(hhat ? hhat : hh.data()) + (size_t)pn * I, (C ? C : cc.data()) + (size_t)pn * std::max<long>(c, 1),
               (h_all ? h_all : ha.data()) + (size_t)pn * I, (S ? S : ss.data()) + (size_t)pn * std::max<long>(c, 1),
               0, ys.data() + (size_t)pn * H};
    select_pair(in, po);
    ns[pn] = po.nS;
  });
  for (long n = 0; n < ntok; ++n) {
    const long t = tokens[n];
    combine(ys.data() + (size_t)n * K * H, w + t * K, K, H, resid ? resid + (size_t)t * H : nullptr,
            out + (size_t)n * H);
  }
  if (nS)
    for (long pn = 0; pn < P; ++pn) nS[pn] = ns[pn];
  if (y) std::copy(ys.begin(), ys.end(), y);
  return 0;
}

// The selected layer with the candidate and kept sets given per pair (C
// [P][c] ascending; S [P][cmax] ascending, nS [P] of them) instead of
// selected: the oracle's own activations and recovery on someone else's
// selection, to check the arithmetic after a selection that differs from the
// oracle's by near-ties. Pairs and tokens as in cfo_select_forward.
int cfo_staged_forward(long T, long K, long E, long I, long H, long r, const uint16_t* x, const int32_t* ids,
                       const double* w, const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, const uint8_t* tg,
                       const uint8_t* tu, const float* sg, const float* su, const int8_t* signs, const double* A,
                       const double* Bt, const int64_t* C, long c, const int64_t* S, long smax, const int64_t* nS,
                       int recovery, const uint16_t* resid, const int64_t* tokens, long ntok, int nthreads,
                       uint16_t* out) {
  if (!is_pow2(H)) return -1;
  const long P = ntok * K;
  std::vector<double> ys((size_t)P * H);
  for (long n = 0; n < ntok; ++n)
    if (tokens[n] < 0 || tokens[n] >= T) return -1;
  parallel_for(P, nthreads, [&](long pn) {
    const long t = tokens[pn / K], q = pn % K;
    const long e = ids[t * K + q];
    PairIn in{I, H, r, x + (size_t)t * H, wg + (size_t)e * I * H, wu + (size_t)e * I * H, wd + (size_t)e * I * H,
              tg + (size_t)e * I * (H / 4), tu + (size_t)e * I * (H / 4), sg + (size_t)e * I, su + (size_t)e * I,
              signs, A ? A + (size_t)e * H * r : nullptr, Bt ? Bt + (size_t)e * I * r : nullptr, 0, c, recovery, 0,
              0.0};
    std::vector<double> hhat(I), h_all(I);
    screen(in, hhat.data());
    exact_rows(in.x, in.wg, in.wu, I, H, h_all.data());
    pair_output(in, hhat.data(), h_all.data(), C + (size_t)pn * c, c, S + (size_t)pn * smax, nS[pn],
                ys.data() + (size_t)pn * H);
  });
  for (long n = 0; n < ntok; ++n) {
    const long t = tokens[n];
    combine(ys.data() + (size_t)n * K * H, w + t * K, K, H, resid ? resid + (size_t)t * H : nullptr,
            out + (size_t)n * H);
  }
  return 0;
}

// The dense layer (every channel): y = sum_j h_j Wd_j over all j, ascending.
int cfo_dense_forward(long T, long K, long E, long I, long H, const uint16_t* x, const int32_t* ids, const double* w,
                      const uint16_t* wg, const uint16_t* wu, const uint16_t* wd, const uint16_t* resid,
                      const int64_t* tokens, long ntok, int nthreads, uint16_t* out) {
  const long P = ntok * K;
  std::vector<double> ys((size_t)P * H, 0.0);
  for (long n = 0; n < ntok; ++n)
    if (tokens[n] < 0 || tokens[n] >= T) return -1;
  parallel_for(P, nthreads, [&](long pn) {
    const long t = tokens[pn / K], q = pn % K;
    const long e = ids[t * K + q];
    std::vector<double> h(I);
    exact_rows(x + (size_t)t * H, wg + (size_t)e * I * H, wu + (size_t)e * I * H, I, H, h.data());
    double* y = ys.data() + (size_t)pn * H;
    for (long j = 0; j < I; ++j) {
      const uint16_t* row = wd + ((size_t)e * I + j) * H;
      for (long i = 0; i < H; ++i) y[i] += h[j] * bf16_value(row[i]);
    }
  });
  for (long n = 0; n < ntok; ++n) {
    const long t = tokens[n];
    combine(ys.data() + (size_t)n * K * H, w + t * K, K, H, resid ? resid + (size_t)t * H : nullptr,
            out + (size_t)n * H);
  }
  return 0;
}

// ----------------------------------------------------------------------------- decode-layer envelope
// RMSNorm with a learned per-feature weight, rounded once to BF16; router
// logits from the BF16 normalised state; softmax over all experts; the K most
// probable in descending probability, lower id first on ties; weights their
// probabilities, optionally renormalised (readings: the pages measure MoE
// blocks and whole-model decoding with routing in place but do not describe
// these steps).

void cfo_rmsnorm(long T, long H, const uint16_t* h, const uint16_t* gamma, double eps, uint16_t* out) {
  for (long t = 0; t < T; ++t) {
    double ss = 0;
    for (long i = 0; i < H; ++i) {
      const double v = bf16_value(h[t * H + i]);
      ss += v * v;
    }
    const double inv = 1.0 / std::sqrt(ss / static_cast<double>(H) + eps);
    for (long i = 0; i < H; ++i) {
      const double g = mut("rmsnorm_without_weight") ? 1.0 : bf16_value(gamma[i]);
      out[t * H + i] = bf16_bits(bf16_value(h[t * H + i]) * inv * g);
    }
  }
}

// x [T][H] BF16 bits, wr [E][H] router rows (values). ids [T][K], w [T][K], logits [T][E].
void cfo_router(long T, long H, long E, const uint16_t* x, const double* wr, long K, int renorm, int32_t* ids,
                double* w, double* logits) {
  for (long t = 0; t < T; ++t) {
    double* l = logits + t * E;
    for (long e = 0; e < E; ++e) {
      double s = 0;
      for (long i = 0; i < H; ++i) s += bf16_value(x[t * H + i]) * wr[e * H + i];
      l[e] = mut("router_lowest") ? -s : s;
    }
    double mx = -std::numeric_limits<double>::infinity();
    for (long e = 0; e < E; ++e) mx = std::max(mx, l[e]);
    std::vector<double> p(E);
    double sum = 0;
    for (long e = 0; e < E; ++e) sum += (p[e] = std::exp(l[e] - mx));
    for (long e = 0; e < E; ++e) p[e] /= sum;
    std::vector<long> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](long a, long b) { return p[a] > p[b]; });
    double ws = 0;
    for (long q = 0; q < K; ++q) ws += p[order[q]];
    for (long q = 0; q < K; ++q) {
      ids[t * K + q] = static_cast<int32_t>(order[q]);
      w[t * K + q] = renorm ? p[order[q]] / ws : p[order[q]];
    }
    if (mut("router_lowest"))
      for (long e = 0; e < E; ++e) l[e] = -l[e];
  }
}

}  // extern "C"
