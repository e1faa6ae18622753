// Plans and launches of the single-launch forward passes (gfx950). The kernels
// live in fused_kernels.h and are instantiated in fused_inst_*.hip.
#include <map>
#include <mutex>
#include <tuple>

#include "fused_kernels.h"

namespace cfm {

// Kernel entry of one instance (defined in fused_inst_*.hip; null if none).
const void* fused_kernel_e0(bool select, bool recx, bool env);
const void* fused_kernel_e2(bool select, bool recx, bool env);
const void* fused_kernel_e4(bool select, bool recx, bool env);
const void* fused_kernel_e8(bool select, bool recx, bool env);
const void* fused_kernel_e16(bool select, bool recx, bool env);
const void* fused_kernel_e32(bool select, bool recx, bool env);
const void* fused_kernel_e8_lean();
const void* fused_kernel_e0_ps(bool recx);
const void* fused_kernel_e2_ps(bool recx);
const void* fused_kernel_e4_ps(bool recx);
const void* fused_kernel_e8_ps(bool recx);
const void* fused_kernel_e0_ms();
const void* fused_kernel_e2_ms();
const void* fused_kernel_e4_ms();
const void* fused_kernel_e8_ms();

namespace {

// ------------------------------------------------------------------ stats

// Byte counts of a per-pair launch. Every field bills each pair's rows (when
// pairs share an expert this is an upper bound of the per-expert unions the
// method needs); bytes_requested bills every pair's requests as issued, with
// down_req down rows per pair (the c candidates' where they are prefetched,
// -1: the kept rows as in bytes_down).
__global__ void k_stats(const int32_t* ids, int P, int E, int I, int H, int k, int c, int r, int T,
                        int K, int select, int exact_step, int sketch_read, const int32_t* kcnt,
                        int down_req, int screen_per_expert, cfm_stats* st) {
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
    s.bytes_sketch = sketch_read ? Pu * (2ull * I * (H / 4) + 8ull * I) : 0;
    s.bytes_candidates = exact_step ? Pu * 4ull * H * c : 0;
    uint64_t kept = Pu * (uint64_t)k;
    if (kcnt) {                                  // threshold rule: the rows each pair kept
      kept = 0;
      for (int pp = 0; pp < P; ++pp) kept += (uint64_t)kcnt[pp];
    }
    s.bytes_down = 2ull * H * kept;
    s.bytes_recovery = r > 0 ? Pu * (2ull * H * r + 2ull * I * r) : 0;
    s.rows_candidates = exact_step ? (uint32_t)(P * c) : 0;
    s.rows_down = (uint32_t)kept;
  } else {
    s.bytes_sketch = 0;
    s.bytes_candidates = Pu * 4ull * H * I;
    s.bytes_down = Pu * 2ull * H * I;
    s.bytes_recovery = 0;
    s.rows_candidates = (uint32_t)(P * I);
    s.rows_down = (uint32_t)(P * I);
  }
  s.pad = 0;
  if (select) {
    // the screen's reads (sketch rows and scales, every Bt row for the partial
    // recovery sums): once per pair, or once per used expert when the grouped
    // screen ran in front of the per-pair kernel
    const uint64_t screen = (sketch_read ? 2ull * I * (H / 4) + 8ull * I : 0) + (r > 0 ? 2ull * I * r : 0);
    const uint64_t per_pair = (exact_step ? 4ull * H * c : 0) + (r > 0 ? 2ull * H * r : 0);
    s.bytes_requested = (screen_per_expert ? (uint64_t)used : Pu) * screen + Pu * per_pair +
                        (down_req >= 0 ? Pu * 2ull * H * down_req : s.bytes_down) + s.bytes_io;
  } else {
    s.bytes_requested = Pu * 6ull * I * H + s.bytes_io;
  }
  *st = s;
}

// Zero fill, 16 bytes per thread per step.
__global__ void k_zero_fill(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The kernel instance serving a plan (null for an unsupported hidden width).
const void* fused_fn(bool select, int H, bool recx, bool env) {
  switch (H >= 1024 ? H / 256 : 0) {
    case 0: return H == 512 ? fused_kernel_e2(select, recx, env) : fused_kernel_e0(select, recx, env);
    case 4: return fused_kernel_e4(select, recx, env);
    case 8: return fused_kernel_e8(select, recx, env);
    case 16: return fused_kernel_e16(select, recx, env);
    case 32: return fused_kernel_e32(select, recx, env);
    default: return nullptr;
  }
}

// The prescreened instance for hidden width H (H <= 2048), or null.
const void* fused_fn_ps(int H, bool recx) {
  switch (H >= 1024 ? H / 256 : 0) {
    case 0: return H == 512 ? fused_kernel_e2_ps(recx) : fused_kernel_e0_ps(recx);
    case 4: return fused_kernel_e4_ps(recx);
    case 8: return fused_kernel_e8_ps(recx);
    default: return nullptr;
  }
}

// The multi-sub-chunk instance of the plain method for hidden width H (H <= 2048), or null.
const void* fused_fn_ms(int H) {
  switch (H >= 1024 ? H / 256 : 0) {
    case 0: return H == 512 ? fused_kernel_e2_ms() : fused_kernel_e0_ms();
    case 4: return fused_kernel_e4_ms();
    case 8: return fused_kernel_e8_ms();
    default: return nullptr;
  }
}

// How many workgroups of `fn` with `lds` bytes of LDS the current device holds
// at once (compute units times resident workgroups per unit), capped at the
// launch sequence slots (cached per device, kernel and LDS size) and at the
// process-wide resident limit when one is set.
int resident_workgroups(const void* fn, size_t lds, int* out) {
  int dev = 0;
  CFM_HIP_TRY(hipGetDevice(&dev));
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  const auto key = std::make_tuple(dev, fn, lds);
  const int cap = resident_limit();
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) { *out = cap >= 0 ? std::min(cap, it->second) : it->second; return CFM_OK; }
  }
  if (lds > 65536)
    CFM_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  int cus = 0, per_cu = 0;
  CFM_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  CFM_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, lds));
  const int n = std::min(kSeqSlots, cus * per_cu);
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = n;
  *out = cap >= 0 ? std::min(cap, n) : n;
  return CFM_OK;
}

// Whether the lean instance serves a selected launch: the plain method at
// hidden width 2048 with the candidates' rows prefetched over 8 output chunks
// per workgroup, rank 64, one screen sub-chunk per workgroup, at most 4 keys
// per thread in each selection, 1 to 160 kept channels and at most 8 experts
// per token (the configuration it is compiled for).
bool lean_fits(const ForwardPlan& p, const SelectArgs& s) {
  return p.H == 2048 && !(s.flags & CFM_RECOVER_CANDIDATES_EXACT) && !p.env && !s.thr && p.pre == 8 && p.r == 64 &&
         p.k > 0 && p.k <= 160 && p.cw <= kSubChunk && p.I <= 4 * NT && p.c <= 4 * NT && p.K <= 8 && p.off_ypt != 0;
}

template <bool SELECT>
int launch_fused(const FusedArgs& fa, size_t lds, hipStream_t stream, bool lean = false, bool ms = false) {
  const void* fn = lean                     ? fused_kernel_e8_lean()
                   : (SELECT && fa.hs != nullptr) ? fused_fn_ps(fa.H, fa.rec_exact != 0)
                   : (SELECT && ms)               ? fused_fn_ms(fa.H)
                                                  : fused_fn(SELECT, fa.H, fa.rec_exact != 0, fa.env != 0);
  if (!fn) return set_error(CFM_EUNSUPPORTED, "hidden width not supported");
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

static void common_regions(ForwardPlan& p, Carve& cv) {
  p.off_seq = cv.take(4 * (size_t)kSeqSlots);
  p.off_err = cv.take(4);                                      // == kFailWordOffset
  p.off_ctr = cv.take(4 * (size_t)std::max(p.T, 1) * kMaxNw);
  p.off_xl = cv.take(8 * (size_t)std::max(p.P, 1) * p.E);   // router logits (envelope calls)
  p.off_kc = cv.take(4 * (size_t)std::max(p.P, 1));           // kept counts (threshold rule)
}

// With the envelope a workgroup waits for router logits computed by the other
// workgroups of its token: when the grid is smaller than the slot count, it is
// a whole number of tokens' slots (K nw), so that no token straddles two rounds
// of the persistent loop.
static void env_geometry(ForwardPlan& p) {
  if (!p.env || p.P * p.nw <= p.G) return;
  const int ut = p.K * p.nw;
  p.G = std::max(ut, (p.G / ut) * ut);
}

ForwardPlan select_plan(int T, int K, int E, int I, int H, int k, int c, int r, bool env, int G_max) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = k; p.c = c; p.r = r; p.env = env ? 1 : 0;
  fused_geometry(p, G_max);
  env_geometry(p);
  p.cw = (I + p.nw - 1) / p.nw;
  p.cpw = std::max(1, (c + p.nw - 1) / p.nw);
  size_t off[24];
  // prefetch of the candidates' rows when every workgroup has at most one output
  // slice and the buffers fit
  const int nck = std::max(1, (H / 8) / p.nw);
  const bool pre_ok = nck <= 8 && k > 0 && (r == 0 || (r % 8 == 0 && 64 % (r / 8) == 0));
  p.pre = pre_ok && lds_layout(H, I, c, k, r, p.cpw, nck, off, p.env, E, K) <= 160 * 1024 ? nck : 0;
  p.lds = lds_layout(H, I, c, k, r, p.cpw, p.pre, off, p.env, E, K);
  Carve cv;
  common_regions(p, cv);
  const size_t Pz = (size_t)p.P;
  p.off_xh = cv.take(Pz * I * 8);
  p.off_xz = cv.take(Pz * p.nw * std::max(r, 1) * 8);
  p.off_xc = cv.take(Pz * std::max(c, 1) * 8);
  p.off_ypart = cv.take(Pz * H * 4);
  p.off_ypt = p.P <= 8 ? cv.take(Pz * H * 8) : 0;         // (only the lean instance's batch-1 grid uses it)
  p.bytes = cv.off;
  return p;
}

ForwardPlan dense_plan(int T, int K, int E, int I, int H, bool env, int G_max) {
  ForwardPlan p{};
  p.T = T; p.K = K; p.P = T * K; p.E = E; p.I = I; p.H = H; p.k = 0; p.c = 0; p.r = 0; p.env = env ? 1 : 0;
  fused_geometry(p, G_max);
  env_geometry(p);
  p.cw = 1;
  p.cpw = std::max(1, (I + p.nw - 1) / p.nw);
  size_t off[24];
  p.lds = lds_layout(H, I, 0, 0, 0, p.cpw, 0, off, p.env, E, K);
  Carve cv;
  common_regions(p, cv);
  const size_t Pz = (size_t)p.P;
  p.off_xh = cv.take(Pz * I * 8);
  p.off_xz = p.off_xh;
  p.off_xc = p.off_xh;
  p.off_ypart = cv.take(Pz * H * 4);
  p.bytes = cv.off;
  return p;
}

// ------------------------------------------------------------------ launches

// Phase-timestamp buffer of the trace build (cfm_phase_trace); null otherwise.
static uint64_t* g_trace = nullptr;

int set_phase_trace(void* buf) {
#ifdef CFM_PHASE_TRACE
  g_trace = static_cast<uint64_t*>(buf);
  return CFM_OK;
#else
  (void)buf;
  return set_error(CFM_EUNSUPPORTED, "phase timestamps need the trace build of the library");
#endif
}

static FusedArgs fused_args(const SelectArgs& s, const ForwardPlan& p) {
  FusedArgs a{};
  a.trace = g_trace;
  a.spin = wait_limit();
  // (with the envelope x is formed in LDS; a.x still serves as a valid address
  // for requests whose result is unused: Bt at rank 0, the A slice when it is
  // not prefetched, so it points at the hidden states then)
  a.x = s.x ? s.x : s.resid;
  a.ids = s.ids; a.topk_w = s.topk_w;
  a.wg = s.w_gate; a.wu = s.w_up; a.wd = s.w_down_t;
  a.signs = s.signs; a.tg = s.tg; a.tu = s.tu; a.sg = s.sg; a.su = s.su;
  a.A = s.A; a.Bt = s.Bt;
  a.out = s.out; a.cand_out = s.cand_out; a.keep_out = s.keep_out;
  a.seq = reinterpret_cast<uint32_t*>(s.ws + p.off_seq);
  a.fail = reinterpret_cast<uint32_t*>(s.ws + p.off_err);
  a.ctr = reinterpret_cast<unsigned*>(s.ws + p.off_ctr);
  a.xh = reinterpret_cast<uint64_t*>(s.ws + p.off_xh);
  a.xz = reinterpret_cast<uint64_t*>(s.ws + p.off_xz);
  a.xc = reinterpret_cast<uint64_t*>(s.ws + p.off_xc);
  a.ypart = reinterpret_cast<float*>(s.ws + p.off_ypart);
  a.ypt = reinterpret_cast<uint64_t*>(s.ws + (p.off_ypt ? p.off_ypt : p.off_ypart));
  a.T = p.T; a.K = p.K; a.P = p.P; a.E = p.E; a.I = p.I; a.H = p.H;
  int log2H = 0;
  while ((1 << log2H) < p.H) ++log2H;
  a.log2H = log2H;
  a.k = p.k; a.c = p.c; a.r = p.r; a.nw = p.nw; a.cw = p.cw; a.cpw = p.cpw; a.nhs = p.nhs; a.G = p.G;
  a.pre = p.pre;
  a.rec_exact = (s.flags & CFM_RECOVER_CANDIDATES_EXACT) ? 1 : 0;
  a.thr = s.thr;
  a.tkey = s.tkey;
  a.kcnt = reinterpret_cast<int32_t*>(s.ws + p.off_kc);
  a.keep_count = s.keep_count;
  a.env = p.env;
  a.env_pair = p.E <= 4 * p.nw ? 1 : 0;      // one logit per wavefront at most
  a.renorm = s.renorm;
  a.eps = s.eps;
  a.resid = s.resid; a.gamma = s.gamma; a.wr = s.wr;
  a.xl = reinterpret_cast<uint64_t*>(s.ws + p.off_xl);
  a.ids_out = s.ids_out; a.w_out = s.w_out; a.x_out = s.x_out;
  return a;
}

// The plan refitted to the workgroups the current device holds at once (the
// size queries assume the largest grid; a smaller grid only shrinks the
// layout). Every workgroup of a launch is then resident, which the exchanges
// between a pair's workgroups rely on.
template <bool SELECT>
int fit_plan(const ForwardPlan& p0, bool recx, ForwardPlan* out) {
  ForwardPlan p = p0;
  for (int round = 0; round < 3; ++round) {
    const void* fn = fused_fn(SELECT, p.H, recx, p.env != 0);
    if (!fn) return set_error(CFM_EUNSUPPORTED, "hidden width not supported");
    if (p.lds > 163840) return set_error(CFM_EUNSUPPORTED, "shape needs more LDS than a workgroup has");
    int g = 0;
    if (int rc = resident_workgroups(fn, p.lds, &g)) return rc;
    if (g < 1) return set_error(CFM_EUNSUPPORTED, "the device cannot hold one workgroup of the forward kernel");
    if (p.G <= g) { *out = p; return CFM_OK; }
    p = SELECT ? select_plan(p.T, p.K, p.E, p.I, p.H, p.k, p.c, p.r, p.env != 0, g)
               : dense_plan(p.T, p.K, p.E, p.I, p.H, p.env != 0, g);
  }
  return set_error(CFM_EUNSUPPORTED, "no grid of the forward kernel fits the device");
}

// Routed pairs from which the per-pair pass puts the grouped screen in front
// of its kernel (Qwen3-30B-A3B-shaped layer, 18 % budget, µs per token with /
// without it: 4 tokens 14.9 / 13.9, 6 tokens 11.9 / 13.2, 8 tokens 9.7 / 10.3,
// 16 tokens 7.3 / 8.8, 32 tokens 6.1 / 8.0).
constexpr int kGroupedScreenMinPairs = 40;

// Whether the per-pair pass runs the expert-grouped screen before its kernel:
// from kGroupedScreenMinPairs pairs, with several sub-chunks of channels per
// workgroup, when the screen is needed, the shape suits the grouped screen and
// the workspace holds its regions (sized from the unrefitted plan, as
// select_workspace is). A grid refitted to fewer workgroups only widens the
// slices, so the decision holds for the launch.
bool select_prescreen_ok(const SelectArgs& s, const ForwardPlan& p0) {
  if (forward_path() >= 3 || p0.P < kGroupedScreenMinPairs || p0.cw <= kSubChunk || p0.I > 4 * NT || p0.H > 2048)
    return false;
  if ((s.flags & CFM_RECOVER_CANDIDATES_EXACT) && p0.c >= p0.I) return false;   // no sketch activation is used
  if (!grouped_screen_supported(p0.T, p0.K, p0.E, p0.I, p0.H, p0.r)) return false;
  return s.ws_bytes >= group_plan(p0.T, p0.K, p0.E, p0.I, p0.H, p0.k, p0.c, p0.r, false, p0.bytes).bytes;
}

static bool use_grouped_screen(const SelectArgs& s, const ForwardPlan& p0, const ForwardPlan& p, GroupPlan* g) {
  if (p.env || !select_prescreen_ok(s, p0)) return false;
  *g = group_plan(p.T, p.K, p.E, p.I, p.H, p.k, p.c, p.r, false, p0.bytes);
  return true;
}

int launch_select_forward(const SelectArgs& s, const ForwardPlan& p0, hipStream_t stream) {
  ForwardPlan p;
  if (int rc = fit_plan<true>(p0, (s.flags & CFM_RECOVER_CANDIDATES_EXACT) != 0, &p)) return rc;
  GroupPlan g{};
  const bool gscreen = use_grouped_screen(s, p0, p, &g);
  if (int rc = prepare_workspace(s.ws, gscreen ? g.bytes : p.bytes,
                                 layout_signature({gscreen ? (s.route_first ? 5 : 4) : 1, p.T, p.K, p.E, p.I, p.H, p.k,
                                                   p.c, p.r, p.env,
                                                   p.nw, p.G, gscreen ? (long)g.bytes : 0}),
                                 stream))
    return rc;
  // (decode-layer envelope) the grouped pass's router stage first; the pass
  // then reads the normalised states and the routing it wrote, and the
  // combine adds the residual
  SelectArgs sr = s;
  if (s.route_first) {
    if (!gscreen) return set_error(CFM_EUNSUPPORTED, "layer forward: the per-pair pass cannot route first here");
    if (int rc = launch_grouped_route(s, g, stream)) return rc;
    sr.x = reinterpret_cast<const uint16_t*>(s.ws + g.off_xw);
    sr.ids = reinterpret_cast<const int32_t*>(s.ws + g.off_idw);
    sr.topk_w = reinterpret_cast<const float*>(s.ws + g.off_ww);
  }
  FusedArgs a = fused_args(sr, p);
  if (!a.x) return set_error(CFM_EINVAL, "select forward: no hidden states");
  if (gscreen) {
    if (int rc = launch_grouped_screen(sr, g, stream)) return rc;
    a.hs = reinterpret_cast<const float*>(s.ws + g.off_hs);
    a.zp = reinterpret_cast<const float*>(s.ws + g.off_zp);
    a.nzp = (p.I + 15) / 16;
  }
  const bool lean = forward_path() != 3 && forward_path() != 4 && lean_fits(p, s);
  // three or more sub-chunks per workgroup with the screen inside the launch:
  // the instance that keeps the next sub-chunk's rows in flight (plain method;
  // Qwen3-30B-A3B-shaped layer, µs per token against the general instance:
  // 3 tokens 17.7 / 18.0, 4 tokens 13.6 / 14.0; with two sub-chunks, 2 tokens,
  // 22.3 / 22.1)
  const bool ms = !lean && !gscreen && forward_path() != 3 && !p.env && !p.pre && p.cw > 2 * kSubChunk &&
                  p.I <= 4 * NT && p.H <= 2048 && !(s.flags & CFM_RECOVER_CANDIDATES_EXACT);
  int rc = launch_fused<true>(a, p.lds, stream, lean, ms);
  if (rc) return rc;
  if (s.stats) {
    // the general instances prefetch every candidate's down row (for their columns) when p.pre
    const int down_req = (p.pre && !lean) ? p.c : -1;
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, sr.ids, p.P, p.E, p.I, p.H, p.k, p.c,
                       p.r, p.T, p.K, 1, (p.k > 0 || a.rec_exact) ? 1 : 0,
                       (a.rec_exact && p.c >= p.I) ? 0 : 1, a.thr ? a.kcnt : nullptr, down_req, gscreen ? 1 : 0,
                       static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

int launch_dense_forward(const SelectArgs& s, const ForwardPlan& p0, hipStream_t stream) {
  ForwardPlan p;
  if (int rc = fit_plan<false>(p0, false, &p)) return rc;
  if (int rc = prepare_workspace(s.ws, p.bytes,
                                 layout_signature({2, p.T, p.K, p.E, p.I, p.H, p.env, p.nw, p.G}), stream))
    return rc;
  const FusedArgs a = fused_args(s, p);
  if (!a.x) return set_error(CFM_EINVAL, "dense forward: no hidden states");
  int rc = launch_fused<false>(a, p.lds, stream);
  if (rc) return rc;
  if (s.stats) {
    hipLaunchKernelGGL(k_stats, dim3(1), dim3(64), 0, stream, s.ids, p.P, p.E, p.I, p.H, p.I, p.I, 0,
                       p.T, p.K, 0, 1, 0, nullptr, -1, 0, static_cast<cfm_stats*>(s.stats));
    CFM_LAUNCH_CHECK("k_stats");
  }
  return CFM_OK;
}

int launch_zero_fill(void* p, size_t n, hipStream_t stream) {
  const size_t n16 = (n + 15) / 16;         // workspaces are 256-byte multiples
  if (n16 == 0) return CFM_OK;
  const unsigned blocks = (unsigned)std::min<size_t>((n16 + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero_fill, dim3(blocks), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  CFM_LAUNCH_CHECK("k_zero_fill");
  return CFM_OK;
}

}  // namespace cfm
