// Kernels of the single-launch forward passes (gfx950): the selected-channel
// routed-expert SwiGLU layer and the dense comparator. Included by fused.hip
// (plans and launches) and by the fused_inst_*.hip translation units, each of
// which instantiates the kernels of one hidden-width class so that they
// compile in parallel.
//
// Forward passes as single persistent kernels (gfx950): the selected-channel
// routed-expert SwiGLU layer and the dense comparator.
//
// Selected layer, per routed (token, expert) pair (arXiv:2610.37386, abstract;
// aimodeling.com article, section "A reader that needs no data at all"):
//   phase A  screen: x~ = Hadamard(d . x) exactly in fixed point, split into
//            base-16 digit planes (FP8 operands); sketch activations hhat_j of
//            this workgroup's channels from the FP4 ternary rows on the matrix
//            cores (exact integer dot products); partial recovery sums over
//            this workgroup's channels;
//   phase B  top-c candidates (every workgroup of the pair, identically) and
//            the exact BF16 gate / up dot products of this workgroup's share;
//   phase C  top-k kept set, recovery coefficients z, down projection over the
//            kept rows of this workgroup's 64-column output slices plus A z,
//            and the token's router-weighted combine by the last of its K
//            pairs to finish a slice.
//
// A pair is served by nw workgroups, all resident at once (the grid never
// exceeds one workgroup per compute unit). They exchange values through global
// memory as 64-bit words (float, launch tag): the writer stores each value with
// this launch's tag; a reader polls the word itself until the tag matches. No
// counter, fence or cache flush is involved, and a value is read in one round
// trip once it is there. Every wait is bounded: on expiry the launch records
// its tag in the failure word and its outputs become NaN.
//
// The launch tag is one more than the sequence number in the workspace; each
// workgroup reads its own slot at the start and every slot is rewritten at the
// end, so all workgroups of a launch agree and tags never repeat (2^32 launches).
// Workgroup g serves pair g % P: with P a multiple of 8 the workgroups of a pair
// share an XCD (workgroups are dispatched round-robin over the 8 XCDs).
//
// The dense layer uses the same skeleton without the screen and selections.
#pragma once

#include <algorithm>

#include "cfm_internal.h"
#include "cfm_launch.h"
#include "envelope.h"
#include "rotate.h"
#include "topk.h"

namespace cfm {
namespace {

constexpr int NT = 256;                       // threads per workgroup
constexpr int kSubChunk = 32;                 // channels per screen sub-chunk (4 MFMA tiles of 16 rows)
constexpr int kOnes = kPlanes;                // MFMA column of constant ones (row sums of the codes)
constexpr unsigned kSpinLimit = 1u << 20;     // default polls of one exchanged value before the launch fails
constexpr int kSeqSlots = 256;                // launch sequence slots (one per possible workgroup)
constexpr int kMaxNw = 32;                    // workgroups per pair (power of two)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ memory helpers

__device__ __forceinline__ uint4 ld16(const void* p) {        // streamed weights
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16c(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Agent-coherent float stores / loads (bypass the non-coherent caches).
__device__ __forceinline__ void st_f(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of values that no workgroup changes during the launch, through the
// scalar data cache (which is invalidated at each dispatch): the router ids,
// and this workgroup's sequence slot (read before the workgroup rewrites it at
// its end; no other workgroup touches it).
typedef __attribute__((address_space(4))) const uint32_t* const_u32_p;
__device__ __forceinline__ uint32_t ld_scalar(const void* p) { return *(const_u32_p)p; }

// ------------------------------------------------------------------ tagged exchange

__device__ __forceinline__ void put_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Set once a bounded wait of this workgroup has expired: its later waits give
// up at once, so a failed launch drains quickly. Cleared at the kernel's start
// (wait_state_reset).
__shared__ int g_wait_expired;
__device__ __forceinline__ void wait_state_reset() {
  if (threadIdx.x == 0) g_wait_expired = 0;
  __syncthreads();
}

// The value of *p once it carries `tag` (v: its first load). On expiry of the
// bounded wait (`limit` polls; limit 0: every wait gives up at once, the
// failure path's test setting) the launch is marked failed and 0 is returned.
__device__ __forceinline__ float await_tagged(const uint64_t* p, uint64_t v, uint32_t tag, uint32_t* fail,
                                              unsigned limit) {
  for (unsigned it = 0; limit == 0 || (uint32_t)(v >> 32) != tag; ++it) {
    if (it >= limit || g_wait_expired) {
      st_u(fail, tag);
      g_wait_expired = 1;
      return 0.f;
    }
    __builtin_amdgcn_s_sleep(2);
    v = ld_tagged(p);
  }
  return __uint_as_float((uint32_t)v);
}

// The values at ptr[0..N) once each carries `tag` (v: their first loads, in
// flight). Every round reloads all N words together and the wavefront leaves
// when every lane has all of its values, so a round costs one round trip
// whatever N is. Entries a lane does not need must point at a word that does
// get this launch's tag. On expiry (as await_tagged) the launch is marked
// failed and the values become 0.
template <int N>
__device__ __forceinline__ void await_all(const uint64_t* const (&ptr)[N], uint64_t (&v)[N], uint32_t tag,
                                          uint32_t* fail, unsigned limit) {
  for (unsigned it = 0;; ++it) {
    bool ok = limit != 0;
#pragma unroll
    for (int j = 0; j < N; ++j) ok = ok && (uint32_t)(v[j] >> 32) == tag;
    if (__all(ok)) return;
    if (it >= limit || g_wait_expired) {
      st_u(fail, tag);
      g_wait_expired = 1;
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] = 0;
      return;
    }
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < N; ++j)          // only the entries still stale are read again
      if ((uint32_t)(v[j] >> 32) != tag) v[j] = ld_tagged(ptr[j]);
  }
}
__device__ __forceinline__ float tagged_value(uint64_t v) { return __uint_as_float((uint32_t)v); }

// Completes this wave's outstanding memory operations, then joins the workgroup.
__device__ __forceinline__ void drain_and_join() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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

// ------------------------------------------------------------------ wavefront primitives

// Sum over the 64 lanes (DPP row shifts and broadcasts), in every lane.
__device__ __forceinline__ float wave_sum_f(float x) {
  float v = x;
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

// ------------------------------------------------------------------ arguments and LDS

struct FusedArgs {
  const uint16_t* x; const int32_t* ids; const float* topk_w;
  const uint16_t *wg, *wu, *wd;
  const int8_t* signs; const uint8_t *tg, *tu; const float *sg, *su;
  const uint16_t *A, *Bt;
  uint16_t* out; int32_t *cand_out, *keep_out;
  uint32_t* seq;     // [256] launch sequence numbers
  uint32_t* fail;    // tag of the last launch whose wait expired
  unsigned* ctr;     // [T][32] combine counters (token, workgroup of the pair)
  uint64_t* xh;      // [P][I]  sketch activations (selected) / exact activations (dense)
  uint64_t* xz;      // [P][nw][r] partial recovery sums
  uint64_t* xc;      // [P][c]  exact activations of the candidates
  float* ypart;      // [P][H]
  uint64_t* ypt;     // [P][H] tagged pair outputs (lean instance)
  int T, K, P, E, I, H, log2H, k, c, r, nw, cw, cpw, nhs, G;
  int pre;           // column chunks per workgroup when the candidates' rows are prefetched into LDS, else 0
  int rec_exact;     // dropped candidates enter the recovery with their exact activation
  // threshold keep rule (thr != 0): S = the candidates whose score key reaches
  // tkey, in place of the top k; k is then c (the most that can pass)
  int thr;
  uint32_t tkey;
  int32_t* kcnt;       // [P] |S| of each pair (workspace; threshold rule)
  int32_t* keep_count; // [P] |S| (optional output; threshold rule)
  // decode-layer envelope (env != 0): x = RMSNorm(resid) computed in the
  // launch, routing from the router rows wr, resid added to the output
  int env, renorm;
  int env_pair;      // the router logits are computed by each pair's own workgroups (else shared by the token's)
  float eps;
  const uint16_t *resid, *gamma, *wr;
  uint64_t* xl;      // [T or P][E] router logits (tagged), per token or per pair
  int32_t* ids_out;  // [T][K] (optional)
  float* w_out;      // [T][K] (optional)
  uint16_t* x_out;   // [T][H] (optional)
  uint64_t* trace;   // phase timestamps [G][kTraceSlots] (trace builds only; else unused)
  unsigned spin;     // polls of one exchanged value before the launch fails (0: at once)
  // prescreened instance (I <= 4 NT): the sketch activations and the partial
  // recovery sums, computed before the launch by the expert-grouped screen,
  // which reads each routed expert's sketch once for all of its tokens
  const float* hs;   // [P][I] sketch activations
  const float* zp;   // [P][nzp][r] partial recovery sums over 16-channel groups
  int nzp;
};

// Phase timestamps (instrumentation, compiled in only with CFM_PHASE_TRACE):
// thread 0 of workgroup b stores the 100 MHz device clock at point n of the
// launch into trace[b][n], and the XCD the workgroup runs on into the last slot.
constexpr int kTraceSlots = 32;
__device__ __forceinline__ void phase_stamp(const FusedArgs& a, int n) {
#ifdef CFM_PHASE_TRACE
  if (a.trace && threadIdx.x == 0) {
    uint64_t* t = a.trace + (size_t)blockIdx.x * kTraceSlots;
    t[n] = __builtin_amdgcn_s_memrealtime();
    if (n == 0) t[kTraceSlots - 1] = (uint64_t)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15);
  }
#else
  (void)a; (void)n;
#endif
}
// The same from lane 0 of every wavefront, into slot n + wavefront.
__device__ __forceinline__ void wave_stamp(const FusedArgs& a, int n) {
#ifdef CFM_PHASE_TRACE
  if (a.trace && (threadIdx.x & 63) == 0)
    a.trace[(size_t)blockIdx.x * kTraceSlots + n + (threadIdx.x >> 6)] = __builtin_amdgcn_s_memrealtime();
#else
  (void)a; (void)n;
#endif
}
// A block_topk step observer: the clock after step 0 (range known) into slot
// base, after the first pass into base + 1, after each later pass into
// base + 2 as (clock << 4 | passes so far), after the ranks into base + 3.
struct TopkStamp {
  const FusedArgs* a;
  int base;
  __device__ void operator()(int st) const {
#ifdef CFM_PHASE_TRACE
    if (a->trace && threadIdx.x == 0) {
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      const int slot = st == 0 ? 0 : st == 1 ? 1 : st == 8 ? 3 : st == 9 ? -1 : 2;
      if (slot >= 0)
        a->trace[(size_t)blockIdx.x * kTraceSlots + base + slot] = slot == 2 ? (now << 4) | (uint64_t)st : now;
    }
#else
    (void)st;
#endif
  }
};

struct Lds {
  int32_t* xs;       // [max(H, 256)] rotation exchange
  uint8_t* limb;     // [kPlanes][Hp] FP8 digit planes of x~
  float* dsum;       // [64][8] per-row digit dots of a sub-chunk
  float* hloc;       // [kSubChunk] sketch activations of the current sub-chunk
  float* hh;         // [I] sketch (selected) / exact (dense) activations of the pair
  int32_t* candp;    // [c] candidate channels
  int32_t* sel;      // [k] positions of the kept channels among the candidates
  int32_t* keep;     // [k] kept channels
  float* hk;         // [k] their exact activations
  float* hcl;        // [c] exact activations of the candidates
  float* zsum;       // [r] sum of the partial recovery sums
  float* zv;         // [r] recovery coefficients
  float* red;        // reduction scratch
  float* gu;         // [2][cpw] gate / up dots of the exact phase
  float* part;       // [NT][8] phase C partial sums
  uint32_t* tks;     // top-k scratch
  uint8_t* btc;      // [c][r] Bt rows of the candidates (BF16), when prefetched
  uint8_t* dnc;      // [c][64] down rows of the candidates for this workgroup's slice, when prefetched
  // envelope only
  uint16_t* xb;      // [H] the token's normalised state (BF16)
  float* rl;         // [E] the token's router logits
  int32_t* rida;     // [K] its experts in ascending id order
  int32_t* rid;      // [K] its experts in slot order (descending probability)
  float* rw;         // [K] their weights
};

__host__ __device__ inline size_t lds_layout(int H, int I, int c, int k, int r, int cpw, int pre, size_t* off,
                                             int env = 0, int E = 0, int K = 0) {
  size_t o = 0;
  int n = 0;
  auto take = [&](size_t b) { off[n++] = o; o = (o + b + 15) & ~size_t(15); };
  const int Hp = H > 256 ? H : 256;
  const int c1 = c > 1 ? c : 1, k1 = k > 1 ? k : 1, r1 = r > 1 ? r : 1;
  take(4 * (size_t)Hp);
  take((size_t)kPlanes * Hp);
  take(4 * 64 * 8);
  take(4 * (size_t)kSubChunk);
  take(4 * (size_t)I);
  take(4 * (size_t)c1);
  take(4 * (size_t)k1);
  take(4 * (size_t)k1);
  take(4 * (size_t)k1);
  take(4 * (size_t)c1);
  take(4 * (size_t)r1);
  take(4 * (size_t)r1);
  take(4 * (size_t)(32 * 64 + 64 > 8 * NT ? 32 * 64 + 64 : 8 * NT));   // >= 8 NT, >= groups r
  take(8 * (size_t)(cpw > 1 ? cpw : 1));
  take(4 * (size_t)NT * 8);
  take(4 * (size_t)kTopkScratchWords);
  // prefetch buffers, in whole 1 KB wavefront transfers
  const size_t nbt = pre ? (size_t)c * (r / 8) : 0, ndn = pre ? (size_t)c * pre : 0;   // pre: column chunks
  take(16 * ((nbt + 63) / 64 * 64));
  take(16 * ((ndn + 63) / 64 * 64));
  take(env ? 2 * (size_t)H : 0);
  take(env ? 4 * (size_t)E : 0);
  take(env ? 4 * (size_t)K : 0);
  take(env ? 4 * (size_t)K : 0);
  take(env ? 4 * (size_t)K : 0);
  return o;
}

__device__ __forceinline__ Lds carve(unsigned char* smem, const FusedArgs& a) {
  size_t off[24];
  lds_layout(a.H, a.I, a.c, a.k, a.r, a.cpw, a.pre, off, a.env, a.E, a.K);
  Lds L;
  L.xs = reinterpret_cast<int32_t*>(smem + off[0]);
  L.limb = smem + off[1];
  L.dsum = reinterpret_cast<float*>(smem + off[2]);
  L.hloc = reinterpret_cast<float*>(smem + off[3]);
  L.hh = reinterpret_cast<float*>(smem + off[4]);
  L.candp = reinterpret_cast<int32_t*>(smem + off[5]);
  L.sel = reinterpret_cast<int32_t*>(smem + off[6]);
  L.keep = reinterpret_cast<int32_t*>(smem + off[7]);
  L.hk = reinterpret_cast<float*>(smem + off[8]);
  L.hcl = reinterpret_cast<float*>(smem + off[9]);
  L.zsum = reinterpret_cast<float*>(smem + off[10]);
  L.zv = reinterpret_cast<float*>(smem + off[11]);
  L.red = reinterpret_cast<float*>(smem + off[12]);
  L.gu = reinterpret_cast<float*>(smem + off[13]);
  L.part = reinterpret_cast<float*>(smem + off[14]);
  L.tks = reinterpret_cast<uint32_t*>(smem + off[15]);
  L.btc = smem + off[16];
  L.dnc = smem + off[17];
  L.xb = reinterpret_cast<uint16_t*>(smem + off[18]);
  L.rl = reinterpret_cast<float*>(smem + off[19]);
  L.rida = reinterpret_cast<int32_t*>(smem + off[20]);
  L.rid = reinterpret_cast<int32_t*>(smem + off[21]);
  L.rw = reinterpret_cast<float*>(smem + off[22]);
  return L;
}

// ------------------------------------------------------------------ phase A: screen

// B operand for super-block sb (256 hidden indices) and half m: column col < 6
// is digit plane col, column 6 is all ones, columns 7..15 are zero. It matches
// the FP4 A operand, where lane group g holds hidden indices
// sb*256 + 64 g + 32 m + (0..31).
__device__ __forceinline__ v8i digit_operand(const Lds& L, int Hp, int sb, int m) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, gB = lane >> 4;
  const uint8_t* row = L.limb + (size_t)min(col, kPlanes - 1) * Hp;
  const int i0 = sb * 256 + 64 * (gB >> 1) + 32 * m + 16 * (gB & 1);
  const uint4 lo = *reinterpret_cast<const uint4*>(row + i0);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + i0 + 128);
  const unsigned keep = col < kPlanes ? 0xFFFFFFFFu : 0u;
  const unsigned one = col == kOnes ? 0x38383838u : 0u;       // FP8 E4M3 1.0
  v8i b;
  b[0] = (lo.x & keep) | one; b[1] = (lo.y & keep) | one; b[2] = (lo.z & keep) | one; b[3] = (lo.w & keep) | one;
  b[4] = (hi.x & keep) | one; b[5] = (hi.y & keep) | one; b[6] = (hi.z & keep) | one; b[7] = (hi.w & keep) | one;
  return b;
}

// The sketch rows of a sub-chunk of cwk channels: rows 0..cwk-1 are the gate
// rows, rows cwk..2cwk-1 the up rows; tile u = rows 16u..16u+15. Wavefront w
// computes tile w over all super-blocks. Its loads: item s = super-block s,
// lane (row = lane & 15, g = lane >> 4) takes 16 bytes of its row at byte
// 64 s + 16 g.
__device__ __forceinline__ uint4 sketch_item(const FusedArgs& a, int e, int j0, int cwk, int s) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rho = 16 * wv + (lane & 15);
  const int rowb = a.H / 4;
  const int off = 64 * s + 16 * (lane >> 4);
  // every lane loads from a valid address (no branch around the load, so the
  // request is not held back); rows past the sub-chunk only reach D rows that
  // are never read, and bytes past H / 4 are masked where the operand is built
  const int rr = rho < 2 * cwk ? rho : 0;
  const int j = j0 + (rr < cwk ? rr : rr - cwk);
  return ld16((rr < cwk ? a.tg : a.tu) + ((size_t)e * a.I + j) * rowb + (off < rowb ? off : 0));
}

// This thread's row scales for a sub-chunk: thread c < cwk takes the gate and
// up scales of channel c (other threads: values that are not used).
__device__ __forceinline__ float2 load_scale(const FusedArgs& a, int e, int j0, int cwk) {
  const size_t o = (size_t)e * a.I + j0 + min((int)threadIdx.x, cwk - 1);
  return make_float2(a.sg[o], a.su[o]);
}
// Bt values of a sub-chunk for thread (zl, zg): channels zg, zg + groups, ...
// (entries past the sub-chunk, and threads beyond the groups, load a value the
// consumer skips).
template <int N>
__device__ __forceinline__ void load_bt(const FusedArgs& a, int e, int j0, int cwk, int zl, int zg, int groups,
                                        uint32_t (&btv)[N]) {
  const bool gok = zg < groups;
  const uint16_t* src = a.r > 0 ? a.Bt : a.x;        // rank 0: nothing to read, a valid address
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int jj = zg + groups * u;
    const bool ok = a.r > 0 && gok && jj < cwk;
    btv[u] = src[ok ? ((size_t)e * a.I + j0 + jj) * a.r + zl : 0];
  }
}

constexpr int kSketchPre = 8;   // super-blocks of the first sub-chunk requested up front

// Sketch activations of channels [j0, j0 + cwk) into hloc (LDS) and the
// exchange. pre: the first kSketchPre items of this wavefront (if use_pre);
// sgu: this thread's prefetched scales (thread c < cwk: gate and up scales of
// channel c).
// ALLPRE: every super-block is among the prefetched items (H <= 256 kSketchPre),
// so the loop below issues no loads (and no wait for later requests is forced).
template <bool ALLPRE>
__device__ __forceinline__ void screen_chunk(const FusedArgs& a, const Lds& L, int p, int e, int j0, int cwk, int F0,
                                             const uint4 (&pre)[kSketchPre], bool use_pre, float2 sgu, uint32_t tag) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int Hp = max(a.H, 256);
  const int nsb = (a.H + 255) / 256;
  if (16 * wv < 2 * cwk) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsb; s0 += kSketchPre) {
      uint4 w[kSketchPre];
#pragma unroll
      for (int u = 0; u < kSketchPre; ++u) {
        const int s = s0 + u;
        if constexpr (ALLPRE) w[u] = pre[u];
        else w[u] = (use_pre && s0 == 0) ? pre[u] : (s < nsb ? sketch_item(a, e, j0, cwk, s) : make_uint4(0, 0, 0, 0));
      }
#pragma unroll
      for (int u = 0; u < kSketchPre; ++u) {
        const int s = s0 + u;
        if (s < nsb) {
          // codes past the row end (H < 256 only) were loaded from a clamped address
          const uint32_t km = 64 * s + 16 * (lane >> 4) < a.H / 4 ? ~0u : 0u;
          const v8i d0 = digit_operand(L, Hp, s, 0);
          const v8i d1 = digit_operand(L, Hp, s, 1);
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(w[u].x & km, w[u].y & km), d0, acc, 4, 0, 0, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(trit_operand(w[u].z & km, w[u].w & km), d1, acc, 4, 0, 0, 0, 0, 0);
        }
      }
    }
    // lane holds D[4 (lane / 16) + v][lane % 16]: (row within the tile, column)
    const int col = lane & 15;
    if (col < 8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) L.dsum[(16 * wv + 4 * (lane >> 4) + v) * 8 + col] = acc[v];
    }
  }
  // per-row scale times the exact integer dot: sum_l 16^l D_l - 2^23 D_ones, in
  // units of 2^(7 - F0); thread c < cwk forms the gate row c and the up row cwk + c
  __syncthreads();
  if (tid < cwk) {
    float gu2[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float* d = L.dsum + (m * cwk + tid) * 8;
      const float4 d0 = *reinterpret_cast<const float4*>(d);
      const float4 d1 = *reinterpret_cast<const float4*>(d + 4);
      const long long S = (long long)(int)d0.x + ((long long)(int)d0.y << 4) + ((long long)(int)d0.z << 8) +
                          ((long long)(int)d0.w << 12) + ((long long)(int)d1.x << 16) +
                          ((long long)(int)d1.y << 20) - ((long long)(int)d1.z << 23);
      gu2[m] = (float)((double)(m ? sgu.y : sgu.x) * ldexp((double)S, kDShift - F0));
    }
    const float hv = silu_f32(gu2[0]) * gu2[1];
    L.hloc[tid] = hv;
    put_tagged(a.xh + (size_t)p * a.I + j0 + tid, hv, tag);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ phase B: exact gate / up

// h for items [q0, q1) of `chan` (null: channel = position), published as
// out[q0 .. q1) with the tag. One wavefront per (row, matrix).
template <int CH, typename Hook>
__device__ __forceinline__ void exact_rows(const FusedArgs& a, const Lds& L, int e, const int32_t* chan, int q0, int q1,
                           const uint4* xr, uint64_t* out, uint32_t tag, Hook hook) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, H = a.H;
  const int nchunk = H / 8;
  const int nitems = 2 * (q1 - q0);
  constexpr int RB = CH >= 16 ? 1 : (CH >= 8 ? 2 : 20 / CH);
  bool hooked = false;
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
    // requests issued after these rows do not delay them (loads complete in order)
    if (!hooked) { hook(); hooked = true; }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int it = it0 + u;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < CH; ++m) acc = dot8_bf16(wr[u][m], xr[m], acc);
      acc = wave_sum_f(acc);
      if (lane == 0 && it < nitems) L.gu[(it & 1) * a.cpw + (it >> 1)] = acc;
    }
  }
  if (!hooked) hook();
  __syncthreads();
  for (int i = tid; i < q1 - q0; i += NT) put_tagged(out + q0 + i, silu_f32(L.gu[i]) * L.gu[a.cpw + i], tag);
}

// ------------------------------------------------------------------ prefetch of the candidates' rows

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

// 16 bytes per lane straight into LDS: lane l's bytes land at lds_base + 16 l
// (lds_base uniform over the wavefront); counted like any other load.
__device__ __forceinline__ void lds_dma16(const void* g, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds_base, 16, 0, 0);
}

// Copies rows[0..n) of a row-major BF16 matrix (row pitch `pitch` elements),
// 2^lp 16-byte pieces per row starting at element col0, into LDS as
// [n][2^lp] pieces: wavefront transfer q carries pieces 64 q .. 64 q + 63 to
// dst + 1024 q. Lanes past the end repeat the last row (their bytes land in the
// padding). The row indices of BATCH transfers are read from LDS before any of
// them is issued, so the reads overlap.
template <int BATCH>
__device__ __forceinline__ void dma_rows(const uint16_t* base, size_t pitch, int col0, const int32_t* rows, int n,
                                         int lp, uint8_t* dst) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nq = ((n << lp) + 63) >> 6;
  for (int q0 = wv; q0 < nq; q0 += (NT / 64) * BATCH) {
    int row[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) row[u] = rows[min(((q0 + (NT / 64) * u) * 64 + lane) >> lp, n - 1)];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int q = q0 + (NT / 64) * u;
      if (q < nq) {
        const int f = q * 64 + lane;
        lds_dma16(base + (size_t)row[u] * pitch + col0 + 8 * (f & ((1 << lp) - 1)), dst + (size_t)q * 1024);
      }
    }
  }
}

// Requests the down rows of all candidates for output chunks [ck0, ck0 + nck)
// ([c][nck] 16-byte pieces into L.dnc) and, if with_bt, their Bt rows ([c][r]
// BF16 into L.btc). nck and r / 8 are powers of two.
__device__ __forceinline__ void prefetch_candidate_rows(const FusedArgs& a, const Lds& L, int e, int ck0, int nck,
                                                        bool with_bt) {
  dma_rows<8>(a.wd + (size_t)e * a.I * a.H, a.H, 8 * ck0, L.candp, a.c, __builtin_ctz(nck), L.dnc);
  if (with_bt && a.r > 0) dma_rows<8>(a.Bt + (size_t)e * a.I * a.r, a.r, 0, L.candp, a.c, __builtin_ctz(a.r / 8), L.btc);
}

// Sum over the lanes of a wavefront that share (lane mod span): lane bits
// log2(span) .. 5 (span a power of two, <= 64).
__device__ __forceinline__ float sum_over_high_lanes(float v, int span) {
  if (span < 2) v += __int_as_float(lane_xor<1>(__float_as_int(v)));
  if (span < 4) v += __int_as_float(lane_xor<2>(__float_as_int(v)));
  if (span < 8) v += __int_as_float(lane_xor<4>(__float_as_int(v)));
  if (span < 16) v += __int_as_float(lane_xor<8>(__float_as_int(v)));
  if (span < 32) v += __int_as_float(lane_xor<16>(__float_as_int(v)));
  if (span < 64) v += __int_as_float(lane_xor<32>(__float_as_int(v)));
  return v;
}
// Sum over aligned groups of `span` consecutive lanes (lane bits 0 .. log2(span)-1).
__device__ __forceinline__ float sum_over_low_lanes(float v, int span) {
  if (span > 1) v += __int_as_float(lane_xor<1>(__float_as_int(v)));
  if (span > 2) v += __int_as_float(lane_xor<2>(__float_as_int(v)));
  if (span > 4) v += __int_as_float(lane_xor<4>(__float_as_int(v)));
  if (span > 8) v += __int_as_float(lane_xor<8>(__float_as_int(v)));
  if (span > 16) v += __int_as_float(lane_xor<16>(__float_as_int(v)));
  if (span > 32) v += __int_as_float(lane_xor<32>(__float_as_int(v)));
  return v;
}

// ------------------------------------------------------------------ phase C over a column range
//
// Output columns are split into 16-byte chunks (8 columns); workgroup w of a
// pair owns chunks [w nck, (w + 1) nck), nck = max(1, H / 8 / nw) (a power of
// two). The down projection reads each kept row's segment of those columns as
// contiguous 16-byte pieces; the combine of the K pairs of a token happens once
// per (token, w).

__device__ __forceinline__ int col_chunks(const FusedArgs& a) { return max(1, (a.H / 8) / a.nw); }

// y[8 ck0 .. 8 (ck0 + ncb)) of pair p into the exchange buffer: the down
// projection over rows[0..n) with coefficients hv, plus (use_rec) A z.
// ncb: a power of two <= NT. Ends with a barrier.
__device__ __forceinline__ void cols_block(const FusedArgs& a, const Lds& L, int p, int e, int ck0, int ncb,
                           const int32_t* rows, const float* hv, int n, bool use_rec) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, H = a.H;
  float* rec = L.red;                      // [8 ncb] recovery term
  float* part = L.part;                    // [NT][8] partial sums
  if (use_rec && !(a.r % 8 == 0 && 64 % (a.r / 8) == 0)) {
    // any other rank: one thread per column
    for (int col = tid; col < 8 * ncb; col += NT) {
      const uint16_t* arow = a.A + ((size_t)e * H + 8 * ck0 + col) * a.r;
      float sacc = 0.f;
      for (int l = 0; l < a.r; ++l) sacc += bf16_to_f32(arow[l]) * L.zv[l];
      rec[col] = sacc;
    }
  } else if (use_rec) {
    // item f = col cpr + lc: 16 bytes of A's row for column col, rank chunk lc
    const int cpr = a.r / 8, nitem = 8 * ncb * cpr;
    const uint16_t* abase = a.A + ((size_t)e * H + 8 * ck0) * a.r;
    constexpr int AB = 8;
    for (int f0 = 0; f0 < nitem; f0 += NT * AB) {
      uint4 w[AB];
#pragma unroll
      for (int u = 0; u < AB; ++u) w[u] = ld16(abase + 8 * (size_t)min(f0 + tid + NT * u, nitem - 1));
#pragma unroll
      for (int u = 0; u < AB; ++u) {
        const int f = f0 + tid + NT * u;
        float d = f < nitem ? dot8_f(w[u], L.zv + 8 * (f % cpr)) : 0.f;
        d = sum_over_low_lanes(d, cpr);
        if (f < nitem && f % cpr == 0) rec[f / cpr] = d;
      }
    }
  }
  const int cc = tid % ncb, g = tid / ncb, ng = NT / ncb;
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  const uint16_t* base = a.wd + (size_t)e * a.I * H + 8 * (ck0 + cc);
  constexpr int DB = 8;
  for (int m0 = g; m0 < n; m0 += ng * DB) {
    uint4 w[DB];
    float h[DB];
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const int m = min(m0 + ng * u, n - 1);
      w[u] = ld16(base + (size_t)(rows ? rows[m] : m) * H);
      h[u] = m0 + ng * u < n ? hv[m] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < DB; ++u) fma8(acc, h[u], w[u]);
  }
  // sum over the threads that share a chunk: lane bits above log2 ncb in the
  // wavefront, then the wavefronts (ncb < 64); groups g < ng (ncb >= 64)
  int slot;
  if (ncb < 64) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = sum_over_high_lanes(acc[u], ncb);
    slot = lane < ncb ? wv * ncb + lane : -1;
  } else {
    slot = tid;
  }
  if (slot >= 0) {
    reinterpret_cast<float4*>(part)[2 * slot] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(part)[2 * slot + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  const int nsrc = ncb < 64 ? NT / 64 : ng;   // partial sums per chunk
  for (int col = tid; col < 8 * ncb; col += NT) {
    const int c8 = col / 8, j = col % 8;
    float y = use_rec ? rec[col] : 0.f;
    for (int q = 0; q < nsrc; ++q) y += part[(q * ncb + c8) * 8 + j];
    st_f(a.ypart + (size_t)p * H + 8 * ck0 + col, y);
  }
  __syncthreads();
}

// After this workgroup's y columns of pair p are stored: the last of the
// token's K pairs to arrive writes out[t][8 ck0 .. 8 (ck0 + nck)) in BF16.
// lw: the token's router weights in LDS (envelope), else null (topk_w). With
// the envelope the residual is added before the single rounding.
__device__ __forceinline__ void combine_cols(const FusedArgs& a, int t, int w, int ck0, int nck, int* s_flag, uint32_t tag,
                                             const float* lw = nullptr) {
  const int tid = threadIdx.x;
  unsigned* cc = a.ctr + (size_t)t * kMaxNw + w;
  if (last_of(cc, (unsigned)a.K, s_flag)) {
    const bool bad = ld_u(a.fail) == tag;
    for (int col = 8 * ck0 + tid; col < 8 * (ck0 + nck); col += NT) {
      float o = 0.f;
      for (int q = 0; q < a.K; ++q)
        o += (lw ? lw[q] : a.topk_w[(size_t)t * a.K + q]) * ld_f(a.ypart + (size_t)(t * a.K + q) * a.H + col);
      if (a.resid) o += bf16_to_f32(a.resid[(size_t)t * a.H + col]);   // (envelope: the residual)
      a.out[(size_t)t * a.H + col] = bad ? (uint16_t)0x7FC0 : f32_to_bf16(o);
    }
  }
  __syncthreads();
}

// Phase C of a workgroup: its columns in blocks of at most NT chunks, then the combine.
__device__ __forceinline__ void phase_c(const FusedArgs& a, const Lds& L, int p, int t, int e, int w,
                        const int32_t* rows, const float* hv, int n, bool use_rec, int* s_flag, uint32_t tag,
                        const float* lw = nullptr) {
  const int nck = col_chunks(a), ck0 = w * nck;
  if (ck0 >= a.H / 8) return;
  for (int cb = 0; cb < nck; cb += NT) cols_block(a, L, p, e, ck0 + cb, min(NT, nck - cb), rows, hv, n, use_rec);
  combine_cols(a, t, w, ck0, nck, s_flag, tag, lw);
}

// Phase C of a workgroup without the candidate-row prefetch (several tokens
// per launch), with the requests that wait on nothing else issued early: the
// Bt pieces of the recovery coefficients' rows first, then this workgroup's
// A pieces and the first batch of its kept down-row pieces (EARLY: together
// with the Bt pieces; else once the Bt pieces are used, in flight during the
// reduction of z); later down batches are requested one batch ahead (two
// register buffers). AB, DB: A and down pieces per thread and batch. The
// arithmetic and its order are those of the step-by-step form (z, then
// cols_block): z over the rows in index order per thread, then the groups;
// each column's down sum over the thread's rows in order, then the threads.
// Requires nck <= NT and r = 0 or (r % 8 == 0, 64 % (r / 8) == 0). nz rows
// enter z (the kept rows, or every candidate with the recovery variant).
template <bool RECX, int AB, int DB, bool EARLY>
__device__ __forceinline__ void phase_c_stream(const FusedArgs& a, const Lds& L, int p, int t, int e, int w, int kk,
                                               int* s_flag, uint32_t tag, const float* lw) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, H = a.H, r = a.r;
  const int nck = col_chunks(a), ck0 = w * nck;
  const bool cols = ck0 < H / 8;
  // ---- requests
  const int nz = RECX ? a.c : kk;
  const int cpr = r > 0 ? r / 8 : 1, ngz = NT / cpr;
  const int zc = tid % cpr, zgi = tid / cpr;
  constexpr int ZB = 8;
  uint4 bz[ZB];
  float hz[ZB];
  auto z_issue = [&](int i0) {
#pragma unroll
    for (int u = 0; u < ZB; ++u) {
      const int i = i0 + ngz * u;
      const int ic = max(min(i, nz - 1), 0);
      const int j = nz > 0 ? (RECX ? L.candp[ic] : L.keep[ic]) : 0;
      hz[u] = i < nz ? (RECX ? L.hcl[ic] : L.hh[j]) : 0.f;
      bz[u] = ld16c(a.Bt + ((size_t)e * a.I + j) * r + 8 * zc);
    }
  };
  const int nitem = 8 * nck * cpr;                  // A pieces of this workgroup's columns
  const uint16_t* abase = a.A + ((size_t)e * H + 8 * ck0) * r;
  uint4 av[AB];
  auto a_issue = [&](int f0) {
#pragma unroll
    for (int u = 0; u < AB; ++u) av[u] = ld16(abase + 8 * (size_t)min(f0 + tid + NT * u, nitem - 1));
  };
  const int cc = tid % nck, g = tid / nck, ngd = NT / nck;
  const int n = kk;
  const uint16_t* dbase = a.wd + (size_t)e * a.I * H + 8 * (ck0 + cc);
  uint4 dA[DB], dB[DB];
  float hA[DB], hB[DB];
  auto d_issue = [&](int m0, uint4 (&wq)[DB], float (&hq)[DB]) {
#pragma unroll
    for (int u = 0; u < DB; ++u) {
      const int mm = m0 + ngd * u, m = max(min(mm, n - 1), 0);
      wq[u] = ld16(dbase + (size_t)(n > 0 ? L.keep[m] : 0) * H);
      hq[u] = mm < n ? L.hk[m] : 0.f;
    }
  };
  if (cols && r > 0) z_issue(zgi);
  if constexpr (EARLY) {
    // (registers to spare) the A pieces and the first down batch are in
    // flight while z is formed
    if (cols && r > 0) a_issue(0);
    if (cols && n > 0) d_issue(g, dA, hA);
  }
  // ---- recovery coefficients z = zsum - sum_j coef_j Bt[j] (coef: sketch
  //      activation of a kept row, or the variant's per-candidate term)
  float* rec = L.red;                               // [8 nck] recovery term (after z is formed)
  if (cols && r > 0) {
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
    for (int i0 = zgi;;) {
#pragma unroll
      for (int u = 0; u < ZB; ++u) fma8(acc, hz[u], bz[u]);
      i0 += ngz * ZB;
      if (i0 >= nz) break;
      z_issue(i0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) L.red[zgi * r + 8 * zc + u] = acc[u];    // ngz r = 8 NT
  }
  if constexpr (!EARLY) {
    // the A pieces and the first down batch are in flight during the reduction
    if (cols && r > 0) a_issue(0);
    if (cols && n > 0) d_issue(g, dA, hA);
  }
  __syncthreads();
  if (cols && r > 0) {
    for (int l = tid; l < r; l += NT) {
      float s = 0.f;
      for (int gg = 0; gg < ngz; ++gg) s += L.red[gg * r + l];
      L.zv[l] = L.zsum[l] - s;
    }
  }
  __syncthreads();
  phase_stamp(a, 11);
  if (!cols) return;
  // ---- A z over this workgroup's columns
  if (r > 0) {
    // every piece of this thread is rank chunk tid % cpr (cpr divides NT)
    float zq[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) zq[i] = L.zv[8 * zc + i];
    for (int f0 = 0;;) {
#pragma unroll
      for (int u = 0; u < AB; ++u) {
        const int f = f0 + tid + NT * u;
        float d = f < nitem ? dot8_f(av[u], zq) : 0.f;
        d = sum_over_low_lanes(d, cpr);
        if (f < nitem && f % cpr == 0) rec[f / cpr] = d;
      }
      f0 += NT * AB;
      if (f0 >= nitem) break;
      a_issue(f0);
    }
  }
  phase_stamp(a, 12);
  // ---- down projection over the kept rows: two batches in flight
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  if (n > 0) {
    const int trips = (n + ngd * DB - 1) / (ngd * DB);        // the same for every thread
    for (int it = 0;;) {
      d_issue(g + ngd * DB * (it + 1), dB, hB);                // (past the end: row n - 1, weight 0, not used)
#pragma unroll
      for (int u = 0; u < DB; ++u) fma8(acc, hA[u], dA[u]);
      if (++it >= trips) break;
      d_issue(g + ngd * DB * (it + 1), dA, hA);
#pragma unroll
      for (int u = 0; u < DB; ++u) fma8(acc, hB[u], dB[u]);
      if (++it >= trips) break;
    }
  }
  float* part = L.part;
  int slot;
  if (nck < 64) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = sum_over_high_lanes(acc[u], nck);
    slot = lane < nck ? wv * nck + lane : -1;
  } else {
    slot = tid;
  }
  if (slot >= 0) {
    reinterpret_cast<float4*>(part)[2 * slot] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    reinterpret_cast<float4*>(part)[2 * slot + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  __syncthreads();
  const int nsrc = nck < 64 ? NT / 64 : ngd;
  for (int col = tid; col < 8 * nck; col += NT) {
    const int c8 = col / 8, j = col % 8;
    float y = r > 0 ? rec[col] : 0.f;
    for (int q = 0; q < nsrc; ++q) y += part[(q * nck + c8) * 8 + j];
    st_f(a.ypart + (size_t)p * H + 8 * ck0 + col, y);
  }
  __syncthreads();
  phase_stamp(a, 13);
  combine_cols(a, t, w, ck0, nck, s_flag, tag, lw);
  phase_stamp(a, 14);
}

// ------------------------------------------------------------------ exchange reads

// Partial recovery sums of all nw workgroups of pair p: thread (zl, zg) adds
// those of workgroups zg, zg + groups, ... into L.red[NT + zg r + zl]. All its
// loads are issued before the first wait.
constexpr int kZsumPer = 16;                       // nw <= 32 and groups >= 2 (r <= 128)

// Issues the loads of fetch_zsum (so that they can be in flight with others);
// N >= ceil(nw / groups).
template <int N>
__device__ __forceinline__ void zsum_issue(const FusedArgs& a, int p, int zl, int zg, int groups,
                                           uint64_t (&raw)[N]) {
  const uint64_t* zp = a.xz + (size_t)p * a.nw * a.r + zl;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int q = zg + groups * u;
    raw[u] = (zg < groups && q < a.nw) ? ld_tagged(zp + (size_t)q * a.r) : 0;
  }
}
template <int N>
__device__ __forceinline__ void zsum_finish(const FusedArgs& a, const Lds& L, int p, int zl, int zg, int groups,
                                            const uint64_t (&raw)[N], uint32_t tag) {
  if (zg >= groups) return;
  const uint64_t* zp = a.xz + (size_t)p * a.nw * a.r + zl;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int q = zg + groups * u;
    if (q < a.nw) s += await_tagged(zp + (size_t)q * a.r, raw[u], tag, a.fail, a.spin);
  }
  L.red[NT + zg * a.r + zl] = s;
}
__device__ __forceinline__ void fetch_zsum(const FusedArgs& a, const Lds& L, int p, int zl, int zg,
                                           int groups, uint32_t tag) {
  uint64_t raw[kZsumPer];
  zsum_issue(a, p, zl, zg, groups, raw);
  zsum_finish(a, L, p, zl, zg, groups, raw, tag);
}

// One sub-chunk of phase A: the screen, then this thread's partial recovery sum.
template <int EPT, int NBT>
__device__ __forceinline__ void screen_and_sum(const FusedArgs& a, const Lds& L, int p, int e, int sj0, int cwk,
                                               int F0, const uint4 (&pre)[kSketchPre], float2 sc,
                                               const uint32_t (&bt)[NBT], int zg, int groups, float& zacc,
                                               uint32_t tag) {
  screen_chunk<(EPT <= kSketchPre)>(a, L, p, e, sj0, cwk, F0, pre, true, sc, tag);
  if (a.r > 0 && zg < groups) {
    // branch-free: every entry is read (clamped) and the ones past the sub-chunk add zero
    float hv[NBT];
#pragma unroll
    for (int u = 0; u < NBT; ++u) hv[u] = L.hloc[min(zg + groups * u, kSubChunk - 1)];
#pragma unroll
    for (int u = 0; u < NBT; ++u) zacc += (zg + groups * u < cwk ? hv[u] : 0.f) * bf16_to_f32((uint16_t)bt[u]);
  }
  __syncthreads();
}

// Phase A for a slice of more than one sub-chunk (the multi-sub-chunk
// instance). The sketch rows and scales of the next sub-chunk are requested
// before the current one is screened, into the other of two register sets
// that alternate: a copy from one set to the other would wait for the
// requests still filling it. The slice's sketch activations are kept in L.hh
// (the exchange later writes the same values there) and its partial recovery
// sums are formed once, after the last sub-chunk, from the slice's contiguous
// Bt rows, whose first batch is requested in place of a next sub-chunk.
// Returns thread (zl, zg)'s share of the slice's partial sum of column zl
// (with r % 8 = 0 the whole sum sits in zg = 0 and the other groups hold zero).
template <int EPT>
__device__ __forceinline__ float screen_slice(const FusedArgs& a, const Lds& L, int p, int e, int j0, int j1, int F0,
                                              uint4 (&s1)[kSketchPre], float2 sg1, int zl, int zg, int groups,
                                              uint32_t tag) {
  const int tid = threadIdx.x, H = a.H, r = a.r;
  const int nsb = (H + 255) / 256;
  const int nsub = (j1 - j0 + kSubChunk - 1) / kSubChunk;
  const bool vec = r > 0 && r % 8 == 0;                       // Bt rows as whole 16-byte pieces
  const int cpr = vec ? r / 8 : 1;                            // pieces per row (divides NT)
  const int npc = vec ? (j1 - j0) * cpr : 1;
  const uint16_t* btb = vec ? a.Bt + ((size_t)e * a.I + j0) * r : a.x;   // (otherwise a valid address, unused)
  auto request = [&](int i, uint4 (&sk)[kSketchPre], float2& sg) {
    if (i < nsub) {
      const int nj0 = j0 + i * kSubChunk, ncwk = min(j1 - nj0, kSubChunk);
#pragma unroll
      for (int u = 0; u < kSketchPre; ++u) sk[u] = sketch_item(a, e, nj0, ncwk, min(u, nsb - 1));
      sg = load_scale(a, e, nj0, ncwk);
    } else {
#pragma unroll
      for (int u = 0; u < kSketchPre; ++u) sk[u] = ld16c(btb + 8 * (size_t)min(tid + NT * u, npc - 1));
    }
  };
  auto screen = [&](int i, const uint4 (&sk)[kSketchPre], float2 sg) {
    const int sj0 = j0 + i * kSubChunk, cwk = min(j1 - sj0, kSubChunk);
    screen_chunk<(EPT <= kSketchPre)>(a, L, p, e, sj0, cwk, F0, sk, true, sg, tag);
    if (tid < cwk) L.hh[sj0 + tid] = L.hloc[tid];
  };
  // the partial sums from the slice's Bt rows; bt: the first batch of pieces
  auto bt_sum = [&](uint4 (&bt)[kSketchPre]) -> float {
    __syncthreads();                                          // the slice's activations are in L.hh
    float zs = 0.f;
    if (vec) {
      // thread tid takes pieces tid + NT u: rank chunk tid % cpr of rows (tid + NT u) / cpr
      float acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = 0.f;
      for (int f0 = 0;;) {
#pragma unroll
        for (int u = 0; u < kSketchPre; ++u) {
          const int f = f0 + tid + NT * u;
          const float h = f < npc ? L.hh[j0 + f / cpr] : 0.f;
          fma8(acc, h, bt[u]);
        }
        f0 += NT * kSketchPre;
        if (f0 >= npc) break;
#pragma unroll
        for (int u = 0; u < kSketchPre; ++u) bt[u] = ld16c(btb + 8 * (size_t)min(f0 + tid + NT * u, npc - 1));
      }
      const int ng = NT / cpr, c8 = 8 * (tid % cpr);
#pragma unroll
      for (int u = 0; u < 8; ++u) L.red[(tid / cpr) * r + c8 + u] = acc[u];    // ng r = 8 NT
      __syncthreads();
      if (tid < r)
        for (int g = 0; g < ng; ++g) zs += L.red[g * r + tid];
      __syncthreads();
    } else if (r > 0 && zg < groups) {
      // any other rank: one Bt value at a time (channels zg, zg + groups, ...)
      for (int jj = zg; jj < j1 - j0; jj += groups)
        zs += L.hh[j0 + jj] * bf16_to_f32(a.Bt[((size_t)e * a.I + j0 + jj) * r + zl]);
    }
    return zs;
  };
  uint4 s2[kSketchPre];
  float2 sg2 = sg1;
  for (int i = 0;;) {
    request(i + 1, s2, sg2);
    screen(i, s1, sg1);
    if (++i >= nsub) return bt_sum(s2);
    request(i + 1, s1, sg1);
    screen(i, s2, sg2);
    if (++i >= nsub) return bt_sum(s1);
  }
}

// 16-byte piece i of a row of x (in LDS with the envelope, global memory otherwise).
__device__ __forceinline__ uint4 x16(const uint16_t* row, int i) {
  return ld16c(reinterpret_cast<const uint4*>(row) + i);
}

// ------------------------------------------------------------------ decode-layer envelope

// The envelope's first steps for token t, run by every workgroup that serves
// one of its pairs (slot q, workgroup w of the pair), in two parts so that
// work that needs no routing can run while the logits are exchanged:
// env_begin forms x = RMSNorm(h[t]) into L.xb and publishes this workgroup's
// router logits W_r[e] . x (experts u, u + UT, ...) as tagged words;
// env_finish reads all E back and forms the routing (L.rid, L.rw) and returns
// the expert of slot q. The workgroups that share the logits: the pair's own
// (u = w, UT = nw; they sit on one XCD, so no pair waits for a later-starting
// XCD) when that leaves at most one logit to each wavefront, else all of the
// token's (u = q nw + w, UT = K nw). Every workgroup of the token forms the
// same L.xb, L.rid and L.rw (the same arithmetic on the same values, shared
// with the grouped pass's router step).
__device__ __forceinline__ uint64_t* env_logits(const FusedArgs& a, int t, int q) {
  return a.xl + (size_t)(a.env_pair ? t * a.K + q : t) * a.E;
}
__device__ __forceinline__ void env_begin(const FusedArgs& a, const Lds& L, int t, int q, int w, uint32_t tag) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = a.H, E = a.E, K = a.K;
  const int nch = H / 8;                                  // 16-byte chunks of a row (H >= 64)
  const int UT = a.env_pair ? a.nw : K * a.nw, u = a.env_pair ? w : q * a.nw + w;
  const int nlog = u < E ? (E - u + UT - 1) / UT : 0;     // logits this workgroup computes
  uint64_t* xl = env_logits(a, t, q);
  // requests first: the first router row of each wavefront (chunks lane, lane + 64, ...)
  constexpr int RP = 4;
  uint4 rp[RP];
  {
    const bool has = wv < nlog;
    const uint4* row = reinterpret_cast<const uint4*>(a.wr + (size_t)(has ? u + UT * wv : 0) * H);
#pragma unroll
    for (int m = 0; m < RP; ++m) {
      const int ci = lane + 64 * m;
      rp[m] = (has && ci < nch) ? ld16c(row + ci) : make_uint4(0, 0, 0, 0);
    }
  }
  env_normalise(a.resid + (size_t)t * H, a.gamma, H, a.eps, L.xb, L.red);
  // this workgroup's logits: wavefront v takes experts u + UT (v + 4 i)
  for (int i = wv; i < nlog; i += NT / 64) {
    const float d = env_logit<RP>(a.wr + (size_t)(u + UT * i) * H, L.xb, H, rp, i == wv);
    if (lane == 0) put_tagged(xl + u + UT * i, d, tag);
  }
}
__device__ __forceinline__ int env_finish(const FusedArgs& a, const Lds& L, int t, int q, int w, uint32_t tag) {
  const int tid = threadIdx.x;
  const int H = a.H, E = a.E, K = a.K, nch = H / 8;
  const uint64_t* xl = env_logits(a, t, q);
  {
    uint64_t raw[kEnvMaxE / NT];
#pragma unroll
    for (int j = 0; j < kEnvMaxE / NT; ++j) {
      const int i = tid + NT * j;
      raw[j] = i < E ? ld_tagged(xl + i) : 0;
    }
#pragma unroll
    for (int j = 0; j < kEnvMaxE / NT; ++j) {
      const int i = tid + NT * j;
      if (i < E) L.rl[i] = await_tagged(xl + i, raw[j], tag, a.fail, a.spin);
    }
  }
  env_pick(L.rl, E, K, a.renorm, L.rida, L.rid, L.rw, L.red, L.tks);
  // the token's routing and normalised state, for the caller (first workgroup of its first pair)
  if (q == 0 && w == 0) {
    if (a.ids_out && tid < K) a.ids_out[(size_t)t * K + tid] = L.rid[tid];
    if (a.w_out && tid < K) a.w_out[(size_t)t * K + tid] = L.rw[tid];
    if (a.x_out)
      for (int ci = tid; ci < nch; ci += NT)
        reinterpret_cast<uint4*>(a.x_out + (size_t)t * H)[ci] = reinterpret_cast<const uint4*>(L.xb)[ci];
  }
  return __builtin_amdgcn_readfirstlane(L.rid[q]);
}

// ------------------------------------------------------------------ launch tag

// Every thread reads the tag itself (no barrier); it is first needed when this
// workgroup publishes a value.
__device__ __forceinline__ uint32_t launch_tag(const FusedArgs& a) { return ld_scalar(a.seq + blockIdx.x) + 1u; }
// Every sequence slot is rewritten by exactly one workgroup of the launch.
__device__ __forceinline__ void finish_launch(const FusedArgs& a, uint32_t tag) {
  if (threadIdx.x == 0)
    for (int b = blockIdx.x; b < kSeqSlots; b += a.G) st_u(a.seq + b, tag);
}

// ------------------------------------------------------------------ kernels

// LNCK > 0: the lean instance, compiled for one configuration only (the plain
// method: no variant flag, envelope or threshold; one screen sub-chunk per
// workgroup; at most 4 keys per thread in each selection; 8 16-byte output
// chunks per workgroup (LNCK), rank 64 (8 LCPR), at most 32 LKPT kept
// channels), so that only the code this configuration executes is emitted and
// it stays resident in the instruction cache. Nothing is prefetched
// speculatively: once the kept set is known, each thread loads its LKPT kept
// rows' 16-byte pieces of the down rows (this workgroup's columns) and of Bt in
// one batch, so the layer reads exactly the kept rows.
// PS: the prescreened instance (several tokens per launch, no envelope): the
// sketch activations and partial recovery sums come from the expert-grouped
// screen that ran before the launch (a.hs, a.zp), and phase A is not compiled.
// MS: the multi-sub-chunk instance (several sub-chunks of channels per
// workgroup below the grouped screen's pair count, no envelope, I <= 4 NT, no
// candidate-row prefetch): the screen keeps the next sub-chunk's rows in
// flight (screen_slice), which fits in registers only without the general
// instance's other paths.
template <int EPT, bool RECX, bool ENV, int LNCK = 0, int LCPR = 0, int LKPT = 1, bool PS = false, bool MS = false>
__global__ __launch_bounds__(NT) void k_select_fused(FusedArgs a) {
  constexpr bool LEAN = LNCK > 0;
  static_assert(!LEAN || (!RECX && !ENV && LNCK == 8 && LCPR == 8), "lean instance: plain method, 8 chunks, rank 64");
  static_assert(!PS || (!LEAN && !ENV), "prescreened instance: general, no envelope");
  static_assert(!MS || (!LEAN && !ENV && !PS), "multi-sub-chunk instance: general, no envelope");
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) uint32_t wred[NT / 64];
  __shared__ __align__(16) int wf0[NT / 64];
  __shared__ int s_flag;
  const Lds L = carve(smem, a);
  wait_state_reset();
  const int tid = threadIdx.x, lane = tid & 63;
  const int nw = a.nw, H = EPT >= 4 ? 256 * EPT : a.H, r = LEAN ? 8 * LCPR : a.r;
  constexpr int CH = EPT >= 2 ? EPT / 2 : 1;        // 16-byte chunks of x per lane (H / 512)
  const uint32_t tag = launch_tag(a);
  const int groups = r > 0 ? NT / r : 1;             // recovery partial sums: thread (l, g)
  const int zl = r > 0 ? tid % r : 0, zg = r > 0 ? tid / r : groups;

  for (int slot = blockIdx.x; slot < a.P * nw; slot += a.G) {
    const int p = slot % a.P, w = slot / a.P;
    const int t = p / a.K;
    phase_stamp(a, 0);
    const int j0 = min(a.I, w * a.cw), j1 = min(a.I, j0 + a.cw);
    const int nck = LEAN ? LNCK : col_chunks(a), ck0 = w * nck;   // this workgroup's output columns: 16-byte chunks

    // ---- requests that need no selection, issued before anything waits on
    //      them: x (this thread's elements and the whole row) and signs first,
    //      then the sketch rows, scales and Bt rows of the first sub-chunk, and
    //      the A slice
    // (with the envelope, x is formed here from the hidden state and the
    // routing is computed: the pair's expert comes from it)
    int e = 0;
    if constexpr (ENV) env_begin(a, L, t, p % a.K, w, tag);
    const uint16_t* xrow = ENV ? L.xb : a.x + (size_t)t * H;
    uint4 xq[EPT >= 8 ? EPT / 8 : 1];
    uint32_t sq[EPT >= 4 ? EPT / 4 : 1];
    if constexpr (EPT >= 4) {
      const uint16_t* xt = xrow + EPT * tid;
      if constexpr (EPT >= 8) {
#pragma unroll
        for (int g = 0; g < EPT / 8; ++g) xq[g] = x16(xt, g);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(xt);
        xq[0] = make_uint4(u.x, u.y, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < EPT / 4; ++g) sq[g] = *reinterpret_cast<const uint32_t*>(a.signs + EPT * tid + 4 * g);
    }
    if constexpr (!ENV) e = (int)ld_scalar(a.ids + __builtin_amdgcn_readfirstlane(p));
    // with the recovery variant and every channel a candidate no sketch
    // activation enters the result: the screen is skipped (ĥ = 0, zero recovery
    // sums, every channel a candidate) and the sketch is not read
    const bool nosk = RECX && a.c >= a.I;
    const RotBuf rb{H, a.log2H, L.xs, L.limb};
    int F0 = 0;
    if constexpr (ENV) {
      // x is ready: rotate it while the router logits are exchanged, then route
      if (!nosk) {
        if constexpr (EPT >= 4) F0 = rotate_fast<EPT>(rb, xq, sq, wf0);
        else F0 = rotate_small(rb, xrow, a.signs, wred);
      }
      e = env_finish(a, L, t, p % a.K, w, tag);
    }
    if (!nosk && !PS) {
      const int cwk0 = min(j1 - j0, kSubChunk);
      // (every prefetch below is issued on every path, so no later wait has to
      //  assume that some of them were skipped; unused ones read valid addresses)
      uint4 spre[kSketchPre];
#pragma unroll
      for (int u = 0; u < kSketchPre; ++u) spre[u] = sketch_item(a, e, j0, cwk0, min(u, (H + 255) / 256 - 1));
      // (loads below are unconditional at clamped addresses, masked afterwards)
      float2 sgu = load_scale(a, e, j0, cwk0);
      constexpr int kBtPer = kMaxRank * kSubChunk / NT;   // Bt values per thread and sub-chunk (<= 16)
      uint32_t btv[kBtPer];
      load_bt(a, e, j0, cwk0, zl, zg, groups, btv);
      // ---- phase A: screen this workgroup's channels, sub-chunk by sub-chunk
      phase_stamp(a, 1);
      if constexpr (!ENV) {
        if constexpr (EPT >= 4) F0 = rotate_fast<EPT>(rb, xq, sq, wf0);
        else F0 = rotate_small(rb, xrow, a.signs, wred);
      }
      phase_stamp(a, 2);
      float zacc = 0.f;                               // partial recovery sum for (zl, zg)
      if (LEAN || j1 - j0 <= kSubChunk) {
        if (j1 > j0) screen_and_sum<EPT>(a, L, p, e, j0, j1 - j0, F0, spre, sgu, btv, zg, groups, zacc, tag);
      } else if constexpr (MS) {
        zacc = screen_slice<EPT>(a, L, p, e, j0, j1, F0, spre, sgu, zl, zg, groups, tag);
      } else {
        // several sub-chunks: the next one's rows are requested before this one is
        // screened (unconditionally inside the loop; the last one is peeled)
        const int nsb = (H + 255) / 256;
        int sj0 = j0;
        for (; sj0 + kSubChunk < j1; sj0 += kSubChunk) {
          const int nj0 = sj0 + kSubChunk, ncwk = min(j1 - nj0, kSubChunk);
          uint4 snext[kSketchPre];
#pragma unroll
          for (int u = 0; u < kSketchPre; ++u) snext[u] = sketch_item(a, e, nj0, ncwk, min(u, nsb - 1));
          const float2 nsgu = load_scale(a, e, nj0, ncwk);
          uint32_t nbtv[kBtPer];
          load_bt(a, e, nj0, ncwk, zl, zg, groups, nbtv);
          screen_and_sum<EPT>(a, L, p, e, sj0, kSubChunk, F0, spre, sgu, btv, zg, groups, zacc, tag);
#pragma unroll
          for (int u = 0; u < kSketchPre; ++u) spre[u] = snext[u];
          sgu = nsgu;
#pragma unroll
          for (int u = 0; u < kBtPer; ++u) btv[u] = nbtv[u];
        }
        screen_and_sum<EPT>(a, L, p, e, sj0, j1 - sj0, F0, spre, sgu, btv, zg, groups, zacc, tag);
      }
      phase_stamp(a, 3);
      if (r > 0) {
        if (zg < groups) L.red[zg * r + zl] = zacc;
        __syncthreads();
        for (int l = tid; l < r; l += NT) {
          float s = 0.f;
          for (int g = 0; g < groups; ++g) s += L.red[g * r + l];
          put_tagged(a.xz + ((size_t)p * nw + w) * r + l, s, tag);
        }
      }
    }

    // the A rows of this workgroup's columns (prefetched path): requested now, used at the end
    uint4 apre[4];
    const bool have_apre = !MS && a.pre && r > 0 && ck0 < H / 8;
    {
      const uint16_t* abase = have_apre ? a.A + ((size_t)e * H + 8 * ck0) * r : a.x;
      const int nA = have_apre ? nck * r : 1;          // 16-byte pieces (<= 1024)
#pragma unroll
      for (int u = 0; u < 4; ++u) apre[u] = ld16(abase + 8 * (size_t)min(tid + NT * u, nA - 1));   // past nA: unused
    }

    // ---- top-c candidates (identical in every workgroup of the pair)
    phase_stamp(a, 4);
    const uint64_t* zptr[8];        // (lean instance) the partial recovery sums, awaited after the exact step
#pragma unroll
    for (int u = 0; u < 8; ++u) zptr[u] = a.xh + (size_t)p * a.I;
    if (nosk) {
      for (int i = tid; i < a.I; i += NT) {
        L.hh[i] = 0.f;
        L.candp[i] = i;
      }
      for (int i = tid; i < groups * r; i += NT) L.red[NT + i] = 0.f;
      __syncthreads();
    } else if (PS) {
      if constexpr (PS) {
        // this thread's sketch activations and its share of the pair's partial
        // recovery sums (groups zg, zg + groups, ... of 16 channels), written by
        // an earlier launch: plain loads, all requested before the first use
        int cnt;
        const int i0 = topk_range<NT>(a.I, &cnt);           // (I <= 4 NT)
        const float* hp = a.hs + (size_t)p * a.I;
        float hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[j] = hp[j < cnt ? i0 + j : 0];
        uint32_t k4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < cnt) L.hh[i0 + j] = hv[j];
          k4[j] = score_key(j < cnt ? hv[j] : 0.f);
        }
        phase_stamp(a, 5);
        block_topk<NT, 4>(k4, i0, cnt, a.I, a.c, L.candp, L.tks, TopkStamp{&a, 23});
        if (r > 0) {
          // (all of a batch's loads issued before the first add)
          constexpr int ZQ = 16;
          float zs = 0.f;
          const float* zb = a.zp + (size_t)p * a.nzp * r + zl;
          for (int q0 = zg; q0 < a.nzp; q0 += groups * ZQ) {
            float zq[ZQ];
#pragma unroll
            for (int u = 0; u < ZQ; ++u) zq[u] = zb[(size_t)min(q0 + groups * u, a.nzp - 1) * r];
#pragma unroll
            for (int u = 0; u < ZQ; ++u) zs += q0 + groups * u < a.nzp ? zq[u] : 0.f;
          }
          if (zg < groups) L.red[NT + zg * r + zl] = zs;
        }
        __syncthreads();
      }
    } else {
      int cnt;
      const int i0 = topk_range<NT>(a.I, &cnt);
      const uint64_t* src = a.xh + (size_t)p * a.I + i0;
      uint64_t raw[32];
      uint32_t kr[32];
      const int per = (a.I + NT - 1) / NT;
      if (LEAN || MS || per <= 4) {
        uint32_t k4[4];
        if constexpr (LEAN) {
          // (lean instance) this thread's sketch activations, awaited together;
          // the pair's partial recovery sums are published after them and are
          // needed only after top-k, so they are awaited with the exact
          // activations (unused entries watch the pair's first activation)
          const uint64_t* pb = a.xh + (size_t)p * a.I;
          const uint64_t* zp = a.xz + (size_t)p * a.nw * r + zl;
          const uint64_t* ptr[4];
          uint64_t v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ptr[j] = pb + (j < cnt ? i0 + j : 0);
            v[j] = ld_tagged(ptr[j]);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int q = zg + groups * u;
            zptr[u] = (zg < groups && q < nw) ? zp + (size_t)q * r : pb;
          }
          await_all<4>(ptr, v, tag, a.fail, a.spin);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float hv = j < cnt ? tagged_value(v[j]) : 0.f;
            if (j < cnt) L.hh[i0 + j] = hv;
            k4[j] = score_key(hv);
          }
        } else {
          // this thread's sketch activations and, when each thread reads at most
          // 8 of them, its share of the pair's partial recovery sums, requested
          // together and then waited for one by one (few registers: this
          // instance is at its register limit)
          uint64_t raw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) raw[j] = j < cnt ? ld_tagged(src + j) : 0;
          const bool zpre = EPT <= 16 && r > 0 && a.nw * r <= 8 * NT;
          uint64_t zraw[8];
          if (zpre) zsum_issue(a, p, zl, zg, groups, zraw);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float hv = j < cnt ? await_tagged(src + j, raw[j], tag, a.fail, a.spin) : 0.f;
            if (j < cnt) L.hh[i0 + j] = hv;
            k4[j] = score_key(hv);
          }
          if (zpre) zsum_finish(a, L, p, zl, zg, groups, zraw, tag);
          else if (r > 0) fetch_zsum(a, L, p, zl, zg, groups, tag);
        }
        phase_stamp(a, 5);
        wave_stamp(a, 15);
        block_topk<NT, 4>(k4, i0, cnt, a.I, a.c, L.candp, L.tks, TopkStamp{&a, 23});
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) raw[j] = j < cnt ? ld_tagged(src + j) : 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float hv = j < cnt ? await_tagged(src + j, raw[j], tag, a.fail, a.spin) : 0.f;
          if (j < cnt) L.hh[i0 + j] = hv;
          kr[j] = score_key(hv);
        }
        if (r > 0) fetch_zsum(a, L, p, zl, zg, groups, tag);
        block_topk<NT, 32>(kr, i0, cnt, a.I, a.c, L.candp, L.tks);
      }
      if (a.c >= a.I || a.c <= 0) __syncthreads();   // block_topk's early exits skip its barrier
    }
    if constexpr (!LEAN) {
      for (int l = tid; l < r; l += NT) {
        float s = 0.f;
        for (int g = 0; g < groups; ++g) s += L.red[NT + g * r + l];
        L.zsum[l] = s;
      }
    }
    if (w == 0 && a.cand_out)
      for (int i = tid; i < a.c; i += NT) a.cand_out[(size_t)p * a.c + i] = L.candp[i];

    // ---- phase B: exact activations of this workgroup's candidates
    phase_stamp(a, 6);
    const int q0 = min(a.c, w * a.cpw), q1 = min(a.c, q0 + a.cpw);
    const bool exact_step = LEAN || a.k > 0 || RECX;   // the candidates' exact activations are used
    const bool thr = !LEAN && !ENV && a.thr;          // threshold keep rule (not with the envelope)
    if (exact_step && q0 < q1) {
      uint4 xr[CH];
#pragma unroll
      for (int m = 0; m < CH; ++m) xr[m] = x16(xrow, min(lane + 64 * m, H / 8 - 1));   // past H / 8: times zero rows
      exact_rows<CH>(a, L, e, L.candp, q0, q1, xr, a.xc + (size_t)p * a.c, tag, [] {});
    }
    // (general instance) candidate rows for the down projection: requested
    // once the exact rows are in (so they do not share bandwidth with them),
    // landing in LDS while the exact activations are exchanged and the kept
    // set is selected; z needs the kept channels' Bt rows, read after top-k
    // (with the variant, or at the largest hidden width where registers are
    // short, every candidate's Bt row is prefetched into LDS with them)
    constexpr bool kBtLate = !RECX && EPT <= 16;
    phase_stamp(a, 7);
    if (!LEAN && !MS && a.pre && ck0 < H / 8) prefetch_candidate_rows(a, L, e, ck0, nck, !kBtLate);
    phase_stamp(a, 8);

    // ---- top-k (or threshold) kept set and recovery coefficients
    int kk = a.k;                              // |S| (the threshold rule's count varies by pair)
    if (exact_step) {
      int cnt;
      const int i0 = topk_range<NT>(a.c, &cnt);
      const uint64_t* src = a.xc + (size_t)p * a.c + i0;
      const int per = (a.c + NT - 1) / NT;
      if (LEAN || MS || per <= 4) {
        uint32_t k4[4];
        // (lean instance) this thread's candidates' channels and sketch
        // activations, read before the exchange so that the kept set's
        // writer below needs no further LDS round
        int32_t chn[4];
        float hzc[4], hvv[4];
        if constexpr (LEAN) {
#pragma unroll
          for (int j = 0; j < 4; ++j) chn[j] = L.candp[min(i0 + j, a.c - 1)];
#pragma unroll
          for (int j = 0; j < 4; ++j) hzc[j] = L.hh[chn[j]];
        }
        const uint64_t* pc = a.xc + (size_t)p * a.c;
        uint64_t v[12] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (LEAN) {
          if (a.c > 0) {   // (unused entries watch the pair's first candidate, which exists)
            // with the partial recovery sums (published long before; read
            // again here rather than carried from the screen, when some of
            // them were still stale)
            const uint64_t* ptr[12];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              ptr[j] = pc + (j < cnt ? i0 + j : 0);
              v[j] = ld_tagged(ptr[j]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              ptr[4 + u] = zptr[u];
              v[4 + u] = ld_tagged(zptr[u]);
            }
            await_all<12>(ptr, v, tag, a.fail, a.spin);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = j < cnt ? ld_tagged(pc + i0 + j) : 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j < cnt)
              v[j] = ((uint64_t)tag << 32) | __float_as_uint(await_tagged(pc + i0 + j, v[j], tag, a.fail, a.spin));
        }
        if constexpr (LEAN) {
          // this thread's share of the pair's partial recovery sums (group zg)
          if (zg < groups) {
            float zs = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) zs += zg + groups * u < nw ? tagged_value(v[4 + u]) : 0.f;
            L.red[NT + zg * r + zl] = zs;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float hv = j < cnt ? tagged_value(v[j]) : 0.f;
          if (j < cnt) L.hcl[i0 + j] = hv;
          hvv[j] = hv;
          k4[j] = score_key(hv);
        }
        phase_stamp(a, 9);
        wave_stamp(a, 19);
        if constexpr (LEAN) {
          // the kept set written as (channel, exact activation, sketch
          // activation bits in L.sel) at each rank
          auto emit = [&](bool take, uint32_t pos, int j) {
            if (take) {
              L.keep[pos] = chn[j];
              L.hk[pos] = hvv[j];
              L.sel[pos] = __float_as_int(hzc[j]);
            }
          };
          block_topk_emit<NT, 4>(k4, i0, cnt, a.c, a.k, emit, L.tks, TopkStamp{&a, 27});
        } else if (!thr) {
          block_topk<NT, 4>(k4, i0, cnt, a.c, a.k, L.sel, L.tks, TopkStamp{&a, 27});
        }
      } else {
        uint64_t raw[32];
        uint32_t kr[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) raw[j] = j < cnt ? ld_tagged(src + j) : 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float hv = j < cnt ? await_tagged(src + j, raw[j], tag, a.fail, a.spin) : 0.f;
          if (j < cnt) L.hcl[i0 + j] = hv;
          kr[j] = score_key(hv);
        }
        if (!thr) block_topk<NT, 32>(kr, i0, cnt, a.c, a.k, L.sel, L.tks);
      }
      // threshold rule: this thread's range of the candidates' activations is
      // in LDS (written by this thread above)
      if (thr)   // (the envelope entry points keep the top k)
        kk = block_threshold<NT>([&](int i) { return score_key(L.hcl[i]); }, i0, cnt, a.tkey, L.sel, L.tks);
      if (!LEAN && a.k >= a.c) __syncthreads();
      if constexpr (!LEAN) {
        for (int i = tid; i < kk; i += NT) {
          L.keep[i] = L.candp[L.sel[i]];
          L.hk[i] = L.hcl[L.sel[i]];
        }
        __syncthreads();
      }
      phase_stamp(a, 10);
      if (w == 0 && a.keep_out)
        for (int i = tid; i < a.k; i += NT) a.keep_out[(size_t)p * a.k + i] = i < kk ? L.keep[i] : -1;
      if (w == 0 && thr && tid == 0) {
        a.kcnt[p] = kk;
        if (a.keep_count) a.keep_count[p] = kk;
      }
      if (RECX && r > 0) {
        // each candidate's term to take out of the screen's recovery sum: its
        // sketch activation if kept, (sketch - exact) if dropped, so that a
        // dropped candidate is recovered with its exact activation
        for (int i = tid; i < a.c; i += NT) L.hcl[i] = L.hh[L.candp[i]] - L.hcl[i];
        __syncthreads();
        for (int i = tid; i < kk; i += NT) L.hcl[L.sel[i]] = L.hh[L.keep[i]];
        __syncthreads();
      }
    } else {
      if (w == 0 && thr && tid == 0) {          // c = 0: nothing to keep
        a.kcnt[p] = 0;
        if (a.keep_count) a.keep_count[p] = 0;
      }
      __syncthreads();
    }
    if constexpr (LEAN) {
      // thread (cc, g) = (tid % 8, tid / 8) takes the kept channels g + 32 u:
      // 16-byte chunk cc of their down rows (this workgroup's columns) times
      // their exact activations, and chunk cc of their Bt rows times their
      // sketch activations (taken out of the screen's recovery sum). Every LDS
      // read and every load is issued before the first one is waited for.
      const int cc = tid & 7, g = tid >> 3;
      int jj[LKPT];
      float hd[LKPT], hz[LKPT];
#pragma unroll
      for (int u = 0; u < LKPT; ++u) {
        const int m = min(g + 32 * u, kk - 1);
        const bool ok = g + 32 * u < kk;
        jj[u] = L.keep[m];
        hd[u] = ok ? L.hk[m] : 0.f;
        hz[u] = ok ? __int_as_float(L.sel[m]) : 0.f;
      }
      const uint16_t* db = a.wd + (size_t)e * a.I * H + 8 * (ck0 + cc);
      const uint16_t* bb = a.Bt + (size_t)e * a.I * r + 8 * cc;
      uint4 dw[LKPT], bw[LKPT];
#pragma unroll
      for (int u = 0; u < LKPT; ++u) dw[u] = ld16(db + (size_t)jj[u] * H);
#pragma unroll
      for (int u = 0; u < LKPT; ++u) bw[u] = ld16c(bb + (size_t)jj[u] * r);
      phase_stamp(a, 11);
      float dacc[8], zacc8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) dacc[u] = zacc8[u] = 0.f;
#pragma unroll
      for (int u = 0; u < LKPT; ++u) {
        fma8(dacc, hd[u], dw[u]);
        fma8(zacc8, hz[u], bw[u]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        dacc[u] = sum_over_high_lanes(dacc[u], 8);
        zacc8[u] = sum_over_high_lanes(zacc8[u], 8);
      }
      float* rec = L.red + 4 * 128;                       // [64] recovery term of the 64 columns
      float* part = L.red + 4 * 128 + 64;                 // [4][64] per-wavefront down partials
      if (lane < 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          part[(tid >> 6) * 64 + 8 * lane + u] = dacc[u];
          L.red[(tid >> 6) * 64 + 8 * lane + u] = zacc8[u];
        }
      }
      __syncthreads();
      for (int l = tid; l < 64; l += NT) {
        float zs = 0.f;
        for (int g2 = 0; g2 < groups; ++g2) zs += L.red[NT + g2 * r + l];
        L.zv[l] = zs - (L.red[l] + L.red[64 + l] + L.red[128 + l] + L.red[192 + l]);
      }
      __syncthreads();
      phase_stamp(a, 12);
#pragma unroll
      for (int u = 0; u < 2; ++u) {                       // A z over this workgroup's 64 columns: 512 pieces
        const int f = tid + NT * u;
        const float d = sum_over_low_lanes(dot8_f(apre[u], L.zv + 8 * (f & 7)), 8);
        if ((f & 7) == 0) rec[f >> 3] = d;
      }
      __syncthreads();
      // this pair's 64 output columns as tagged words; workgroup w of the
      // token's pair w mod K combines column block w: it waits for the K
      // pairs' words of its columns and sums them in slot order (the order of
      // the other instances' combine), then writes the BF16 output
      if (tid < 64)
        put_tagged(a.ypt + (size_t)p * H + 8 * ck0 + tid,
                   part[tid] + part[64 + tid] + part[128 + tid] + part[192 + tid] + rec[tid], tag);
      phase_stamp(a, 13);
      if (p % a.K == w % a.K) {
        constexpr int KQ = 2;                            // pair slots per thread (this instance: K <= 8)
        const int col = tid & 63, q0 = tid >> 6;
        const uint64_t* yt = a.ypt + (size_t)t * a.K * H + 8 * ck0 + col;
        const uint64_t* ptr[KQ];
        uint64_t v[KQ];
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          const int q = q0 + (NT / 64) * u;
          ptr[u] = yt + (size_t)(q < a.K ? q : 0) * H;
        }
        const int nq = (a.K - q0 + (NT / 64) - 1) / (NT / 64);   // slots of this thread
#pragma unroll
        for (int u = 0; u < KQ; ++u) if (u < nq) v[u] = ld_tagged(ptr[u]); else v[u] = ((uint64_t)tag << 32);
        await_all<KQ>(ptr, v, tag, a.fail, a.spin);
        float* ys = L.red + 1024;                        // [K][64]
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          const int q = q0 + (NT / 64) * u;
          if (q < a.K) ys[q * 64 + col] = tagged_value(v[u]);
        }
        __syncthreads();
        if (tid < 64) {
          const bool bad = ld_u(a.fail) == tag;
          float o = 0.f;
          for (int q = 0; q < a.K; ++q) o += a.topk_w[(size_t)t * a.K + q] * ys[q * 64 + tid];
          a.out[(size_t)t * H + 8 * ck0 + tid] = bad ? (uint16_t)0x7FC0 : f32_to_bf16(o);
        }
      }
      phase_stamp(a, 14);
      continue;
    } else if (!MS && a.pre) {
      // candidate down rows are in LDS: the down projection of this workgroup's
      // slice needs no further memory reads. z takes the kept channels' Bt rows,
      // requested once the prefetch has landed and in flight while the down
      // projection runs (default), or prefetched into LDS with the down rows
      // (variant)
      constexpr int ZB = 5;
      const int cpr = LEAN ? LCPR : (r > 0 ? r / 8 : 1), ng = NT / cpr;
      const int zc = tid % cpr, zgi = tid / cpr;
      uint4 bz[ZB];
      float hz[ZB];
      auto kept_bt = [&](int i0) {
#pragma unroll
        for (int u = 0; u < ZB; ++u) {
          const int i = i0 + ng * u;
          const bool ok = i < kk;
          const int j = ok ? L.keep[i] : 0;
          hz[u] = ok ? L.hh[j] : 0.f;
          bz[u] = ok ? ld16c(a.Bt + ((size_t)e * a.I + j) * r + 8 * zc) : make_uint4(0, 0, 0, 0);
        }
      };
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      phase_stamp(a, 11);
      if (kBtLate && r > 0) kept_bt(zgi);
      const bool cols = ck0 < H / 8;
      float* rec = L.red + 4 * 128;                       // [8 nck] recovery term (nck <= 8)
      float* part = L.red + 4 * 128 + 64;                 // [4][8 nck] per-wavefront down partials
      if (cols) {
        const int cc = tid % nck, g = tid / nck;
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.f;
        for (int m = g; m < kk; m += NT / nck)
          fma8(acc, L.hk[m], *reinterpret_cast<const uint4*>(L.dnc + ((size_t)L.sel[m] * nck + cc) * 16));
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = sum_over_high_lanes(acc[u], nck);
        if (lane < nck)
#pragma unroll
          for (int u = 0; u < 8; ++u) part[(tid >> 6) * 8 * nck + 8 * lane + u] = acc[u];
      }
      if (r > 0) {
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.f;
        if constexpr (!kBtLate) {
          const int nz = RECX ? a.c : kk;      // terms taken out of the screen's sum
          for (int m = zgi; m < nz; m += ng) {
            const int pos = RECX ? m : L.sel[m];
            const float cf = RECX ? L.hcl[m] : L.hh[L.keep[m]];
            fma8(acc, cf, *reinterpret_cast<const uint4*>(L.btc + (size_t)pos * 2 * r + 16 * zc));
          }
        } else {
          for (int i0 = zgi;;) {
#pragma unroll
            for (int u = 0; u < ZB; ++u) fma8(acc, hz[u], bz[u]);
            i0 += ng * ZB;
            if (i0 >= kk) break;
            kept_bt(i0);
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = sum_over_high_lanes(acc[u], cpr);
        if (lane < cpr)
#pragma unroll
          for (int u = 0; u < 8; ++u) L.red[(tid >> 6) * r + 8 * lane + u] = acc[u];
        __syncthreads();
        for (int l = tid; l < r; l += NT) L.zv[l] = L.zsum[l] - (L.red[l] + L.red[r + l] + L.red[2 * r + l] + L.red[3 * r + l]);
        __syncthreads();
        phase_stamp(a, 12);
        if (cols) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int f = tid + NT * u;
            float d = f < nck * r ? dot8_f(apre[u], L.zv + 8 * (f % cpr)) : 0.f;
            d = sum_over_low_lanes(d, cpr);
            if (f < nck * r && f % cpr == 0) rec[f / cpr] = d;
          }
        }
      }
      if (cols) {
        __syncthreads();
        for (int col = tid; col < 8 * nck; col += NT) {
          const float y = part[col] + part[8 * nck + col] + part[16 * nck + col] + part[24 * nck + col] +
                          (r > 0 ? rec[col] : 0.f);
          st_f(a.ypart + (size_t)p * H + 8 * ck0 + col, y);
        }
        phase_stamp(a, 13);
        combine_cols(a, t, w, ck0, nck, &s_flag, tag, ENV ? L.rw : nullptr);
        phase_stamp(a, 14);
      }
      continue;
    }
    // (hidden widths up to 2048 and not in the envelope instances: its
    // registers would spill in the others)
    constexpr bool kStream = !ENV && EPT <= 8;
    if (kStream && (r == 0 || (r % 8 == 0 && 64 % (r / 8) == 0)) && col_chunks(a) <= NT) {
      // (A pieces and kept-row pieces per request batch: the prescreened
      // instance has the registers for twice as many)
      if constexpr (kStream)
        phase_c_stream<RECX, PS ? 16 : 8, PS ? 16 : 8, PS>(a, L, p, t, e, w, kk, &s_flag, tag, nullptr);
      continue;
    }
    if (r > 0) {
      // z = zsum - sum_{j in S} hhat_j Bt[e][j] (with dropped candidates recovered
      // exactly: minus sum over the candidates of their coefficient in hcl)
      const int nz = RECX ? a.c : kk;
      if (r % 8 == 0) {
        const int cpr = r / 8, ng = NT / cpr;       // r <= 128: cpr <= 16, ng >= 16
        const int cc = tid % cpr, g = tid / cpr;
        float acc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[u] = 0.f;
        constexpr int ZB = 8;
        for (int i0 = g; i0 < nz; i0 += ng * ZB) {
          uint4 bw[ZB];
          float hv[ZB];
#pragma unroll
          for (int u = 0; u < ZB; ++u) {
            const int i = i0 + ng * u;
            const bool ok = i < nz;
            const int j = ok ? (RECX ? L.candp[i] : L.keep[i]) : 0;
            hv[u] = ok ? (RECX ? L.hcl[i] : L.hh[j]) : 0.f;
            bw[u] = ok ? ld16c(a.Bt + ((size_t)e * a.I + j) * r + 8 * cc) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < ZB; ++u) fma8(acc, hv[u], bw[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) L.red[g * r + 8 * cc + u] = acc[u];    // ng * r = 8 NT
        __syncthreads();
        for (int l = tid; l < r; l += NT) {
          float s = 0.f;
          for (int gg = 0; gg < ng; ++gg) s += L.red[gg * r + l];
          L.zv[l] = L.zsum[l] - s;
        }
      } else {
        for (int l = tid; l < r; l += NT) {
          float s = 0.f;
          for (int i = 0; i < nz; ++i) {
            const int j = RECX ? L.candp[i] : L.keep[i];
            s += (RECX ? L.hcl[i] : L.hh[j]) * bf16_to_f32(a.Bt[((size_t)e * a.I + j) * r + l]);
          }
          L.zv[l] = L.zsum[l] - s;
        }
      }
      __syncthreads();
    }

    // ---- phase C: down projection over kept rows for this workgroup's output slices
    phase_c(a, L, p, t, e, w, L.keep, L.hk, kk, r > 0, &s_flag, tag, ENV ? L.rw : nullptr);
  }
  finish_launch(a, tag);
}

template <int EPT, bool ENV>
__global__ __launch_bounds__(NT) void k_dense_fused(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_flag;
  const Lds L = carve(smem, a);
  wait_state_reset();
  const int tid = threadIdx.x, lane = tid & 63;
  const int nw = a.nw, H = a.H;
  constexpr int CH = EPT >= 2 ? EPT / 2 : 1;
  const uint32_t tag = launch_tag(a);
  for (int slot = blockIdx.x; slot < a.P * nw; slot += a.G) {
    const int p = slot % a.P, w = slot / a.P;
    const int t = p / a.K;
    int e;
    if constexpr (ENV) {
      env_begin(a, L, t, p % a.K, w, tag);
      e = env_finish(a, L, t, p % a.K, w, tag);
    } else {
      e = (int)ld_scalar(a.ids + __builtin_amdgcn_readfirstlane(p));
    }
    phase_stamp(a, 0);
    const uint16_t* xrow = ENV ? L.xb : a.x + (size_t)t * H;
    const int q0 = min(a.I, w * a.cpw), q1 = min(a.I, q0 + a.cpw);
    if (q0 < q1) {
      uint4 xr[CH];
#pragma unroll
      for (int m = 0; m < CH; ++m) {
        const int ci = lane + 64 * m;
        xr[m] = ci < H / 8 ? x16(xrow, ci) : make_uint4(0, 0, 0, 0);
      }
      exact_rows<CH>(a, L, e, nullptr, q0, q1, xr, a.xh + (size_t)p * a.I, tag, [] {});
    }
    // all activations of the pair
    phase_stamp(a, 20);
    {
      const uint64_t* src = a.xh + (size_t)p * a.I;
      constexpr int HB = 8;
      for (int i0 = tid; i0 < a.I; i0 += NT * HB) {
        uint64_t raw[HB];
#pragma unroll
        for (int u = 0; u < HB; ++u) raw[u] = i0 + NT * u < a.I ? ld_tagged(src + i0 + NT * u) : 0;
#pragma unroll
        for (int u = 0; u < HB; ++u) {
          const int i = i0 + NT * u;
          if (i < a.I) L.hh[i] = await_tagged(src + i, raw[u], tag, a.fail, a.spin);
        }
      }
    }
    __syncthreads();
    phase_stamp(a, 21);
    phase_c(a, L, p, t, e, w, nullptr, L.hh, a.I, false, &s_flag, tag, ENV ? L.rw : nullptr);
    phase_stamp(a, 22);
  }
  finish_launch(a, tag);
}

}  // namespace
}  // namespace cfm
