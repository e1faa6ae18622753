// C ABI entry points: argument validation, workspace sizing, dispatch.
// Validation is plain host code that runs before any HIP call, so argument
// errors are reported the same way on machines without a GPU.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "cfm_internal.h"
#include "cfm_launch.h"

namespace cfm {

static thread_local std::string g_last_error;

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
void clear_error() { g_last_error.clear(); }

// ---------------------------------------------------------------- event timing
namespace {
struct Pending { std::string name; hipEvent_t a, b; };
bool g_timing = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::string g_open;
hipEvent_t g_open_ev = nullptr;

hipEvent_t take_event() {
  if (!g_pool.empty()) { hipEvent_t e = g_pool.back(); g_pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

bool timing_on() { return g_timing; }

// ---------------------------------------------------------------- workspace layouts
namespace {
std::mutex g_ws_mu;
std::unordered_map<uintptr_t, uint64_t> g_ws_sig;    // workspace address -> layout of its last call
std::atomic<unsigned> g_wait_limit{1u << 20};
std::atomic<int> g_resident_limit{-1};
}  // namespace

int prepare_workspace(void* ws, size_t bytes, uint64_t sig, hipStream_t stream) {
  bool clear = false;
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    auto it = g_ws_sig.find(reinterpret_cast<uintptr_t>(ws));
    if (it == g_ws_sig.end()) {
      g_ws_sig.emplace(reinterpret_cast<uintptr_t>(ws), sig);
    } else if (it->second != sig) {
      it->second = sig;
      clear = true;
    }
  }
  return clear ? launch_zero_fill(ws, bytes, stream) : CFM_OK;
}

unsigned wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
int resident_limit() { return g_resident_limit.load(std::memory_order_relaxed); }


void timing_begin(const char* name, hipStream_t s) {
  if (!g_timing) return;
  g_open = name;
  g_open_ev = take_event();
  if (g_open_ev) (void)hipEventRecord(g_open_ev, s);
}

void timing_end(hipStream_t s) {
  if (!g_timing || !g_open_ev) return;
  hipEvent_t b = take_event();
  if (!b) return;
  (void)hipEventRecord(b, s);
  g_pending.push_back({g_open, g_open_ev, b});
  g_open_ev = nullptr;
}

namespace {

int check_shape(int E, int I, int H, bool need_pow2_h) {
  if (E <= 0 || I <= 0 || H <= 0) return set_error(CFM_EINVAL, "E, I and H must be positive");
  if (H < 64 || H > kMaxH) return set_error(CFM_EUNSUPPORTED, "H must lie in [64, 8192]");
  if (need_pow2_h && !is_pow2(H)) return set_error(CFM_EUNSUPPORTED, "H must be a power of two");
  if (!need_pow2_h && H % 64) return set_error(CFM_EUNSUPPORTED, "H must be a multiple of 64");
  if (I > kMaxI) return set_error(CFM_EUNSUPPORTED, "I must be at most 8192");
  return CFM_OK;
}

int check_budget(int I, int H, int k, int c, int r) {
  if (k < 0 || c < 0 || r < 0) return set_error(CFM_EUNSUPPORTED, "k, c and r must be nonnegative");
  if (c > I) return set_error(CFM_EUNSUPPORTED, "c must not exceed I");
  if (k > c) return set_error(CFM_EUNSUPPORTED, "k must not exceed c");
  if (r > std::min(H, I)) return set_error(CFM_EUNSUPPORTED, "r must not exceed min(H, I)");
  if (r > kMaxRank) return set_error(CFM_EUNSUPPORTED, "r must be at most 128");
  return CFM_OK;
}

// Forward-pass variant: 0 automatic, 1 per-pair, 2 expert-grouped, 3 per-pair
// on the general instance only, 4 per-pair with the screen inside the single
// launch (process-wide).
std::atomic<int> g_path{0};
// Automatic choice: the grouped pass from these batch sizes on, and for the
// selected layer also once the routed pairs outnumber the per-pair kernel's
// resident workgroups (it would serve them in rounds). Measured on the
// Qwen3-30B-A3B-shaped layer (18 % budget, µs per token, per-pair / grouped):
// 32 tokens 6.1 / 7.1, 40 tokens 8.0 / 6.0, 64 tokens 5.5 / 4.6; the dense
// layer at 64 tokens 11.3 / 5.2.
constexpr int kGroupedMinTokensSelect = 48;
constexpr int kGroupedMinPairsSelect = 257;
constexpr int kGroupedMinTokensDense = 32;

// Whether a forward call uses the grouped pass (or an error status).
int pick_grouped(int T, int K, int E, int I, int H, int r, bool dense, bool* grouped) {
  const bool ok = grouped_supported(T, K, E, I, H, r, dense);
  const int path = g_path.load(std::memory_order_relaxed);
  if (path == 2 && !ok) return set_error(CFM_EUNSUPPORTED, "expert-grouped pass: shape not supported");
  const bool large = dense ? T >= kGroupedMinTokensDense
                           : T >= kGroupedMinTokensSelect || (long)T * K >= kGroupedMinPairsSelect;
  *grouped = path == 2 || (path == 0 && ok && large);
  return CFM_OK;
}

int check_tokens(int T, int K) {
  if (T < 0) return set_error(CFM_EINVAL, "T must be nonnegative");
  if (K <= 0) return set_error(CFM_EINVAL, "K must be positive");
  if (K > kMaxK) return set_error(CFM_EUNSUPPORTED, "K must be at most 64");
  if ((long)T * K > (1L << 24)) return set_error(CFM_EUNSUPPORTED, "T*K too large");
  return CFM_OK;
}

}  // namespace

int forward_path() { return g_path.load(std::memory_order_relaxed); }

// ---------------------------------------------------------------- scratch of the no-allocation entry point
// Device memory of moe_select_forward_noalloc: one copy per GPU, held until
// the process ends. In host code `scratch` is only a symbol: its device
// address on the current GPU comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;       // device -> its copy of `scratch`

// The current device's scratch address; on a device's first call, looked up
// and zero-filled (a fill kernel on `stream`, ahead of the caller's work).
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  CFM_HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return CFM_OK;
  }
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return set_error(CFM_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  if (int rc = launch_zero_fill(ptr, kScratchBytes, stream)) return rc;
  g_scratch_ptr.emplace(dev, ptr);
  *out = ptr;
  return CFM_OK;
}
}  // namespace
}  // namespace cfm

using namespace cfm;

namespace {
// The selected forward pass behind moe_select_forward_ex and
// moe_select_forward_threshold (thr: S by the threshold tau on |h| in place of
// the top k; k is then c, the most that can pass).
int select_entry(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T, int K,
                 const cfm_bf16* w_gate, const cfm_bf16* w_up, const cfm_bf16* w_down_t, int E, int I, int H,
                 const int8_t* signs, const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                 const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r, unsigned flags, bool thr, float tau,
                 cfm_bf16* out, int32_t* cand_out, int32_t* keep_out, int32_t* keep_count, cfm_stats* stats,
                 void* ws, size_t ws_bytes, void* stream) {
  if (flags & ~CFM_RECOVER_CANDIDATES_EXACT) return set_error(CFM_EINVAL, "moe_select_forward_ex: unknown flag bits");
  if (int rc = check_tokens(T, K)) return rc;
  if (int rc = check_shape(E, I, H, true)) return rc;
  if (int rc = check_budget(I, H, k, c, r)) return rc;
  if (T == 0) return CFM_OK;
  if (!x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down_t || !signs || !tg || !tu ||
      !sg || !su || !out)
    return set_error(CFM_EINVAL, "moe_select_forward: null pointer");
  if (r > 0 && (!A || !Bt)) return set_error(CFM_EINVAL, "moe_select_forward: null A or Bt with r > 0");
  bool grouped = false;
  if (int rc = pick_grouped(T, K, E, I, H, r, false, &grouped)) return rc;
  const ForwardPlan plan = select_plan(T, K, E, I, H, k, c, r);
  const size_t need = grouped ? group_plan(T, K, E, I, H, k, c, r, false, plan.bytes).bytes : plan.bytes;
  if (!ws || ws_bytes < need)
    return set_error(CFM_EWORKSPACE, "moe_select_forward: workspace smaller than select_workspace()");
  SelectArgs a{x, w_gate, w_up, w_down_t, A, Bt, topk_ids, topk_w, signs, tg, tu, sg, su, out,
               cand_out, keep_out, stats, static_cast<char*>(ws), flags};
  a.thr = thr ? 1 : 0;
  const float tpos = tau == 0.f ? 0.f : tau;             // -0 as +0: every score reaches it
  std::memcpy(&a.tkey, &tpos, sizeof a.tkey);             // |h| >= tau iff bits(|h|) >= bits(tau)
  a.keep_count = thr ? keep_count : nullptr;
  a.ws_bytes = ws_bytes;
  if (grouped)
    return launch_grouped_forward(a, group_plan(T, K, E, I, H, k, c, r, false, plan.bytes),
                                  static_cast<hipStream_t>(stream));
  return launch_select_forward(a, plan, static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" {

const char* cfm_last_error(void) { return g_last_error.c_str(); }

const char* cfm_version(void) { return "cfm 0.1.0 gfx950"; }

int cfm_set_forward_path(int path) {
  if (path < 0 || path > 4) return set_error(CFM_EINVAL, "path must be 0, 1, 2, 3 or 4");
  return g_path.exchange(path);
}

int cfm_timing_enable(int on) {
  g_timing = on != 0;
  return CFM_OK;
}

int cfm_set_wait_limit(unsigned polls) { return (int)g_wait_limit.exchange(polls); }

int cfm_set_resident_limit(int workgroups) { return g_resident_limit.exchange(workgroups < 0 ? -1 : workgroups); }

int cfm_workspace_status(void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!ws) return set_error(CFM_EINVAL, "cfm_workspace_status: null workspace");
  if (ws_bytes < kFailWordOffset + 4) return set_error(CFM_EWORKSPACE, "cfm_workspace_status: workspace too small");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  char* fail = static_cast<char*>(ws) + kFailWordOffset;
  CFM_HIP_TRY(hipMemcpyAsync(&word, fail, 4, hipMemcpyDeviceToHost, s));
  CFM_HIP_TRY(hipStreamSynchronize(s));
  if (word == 0) return CFM_OK;
  static const uint32_t zero = 0;
  CFM_HIP_TRY(hipMemcpyAsync(fail, &zero, 4, hipMemcpyHostToDevice, s));
  CFM_HIP_TRY(hipStreamSynchronize(s));
  return set_error(CFM_ETIMEOUT, "a bounded wait expired in a forward call on this workspace (launch tag " +
                                     std::to_string(word) + "): that call's outputs are NaN");
}

int cfm_phase_trace(void* buf) {
  clear_error();
  return set_phase_trace(buf);
}

int cfm_timing_report(char* buf, size_t len) {
  std::map<std::string, std::pair<long, double>> acc;
  for (auto& p : g_pending) {
    if (hipEventSynchronize(p.b) != hipSuccess) return set_error(CFM_EHIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return set_error(CFM_EHIP, "elapsed time failed");
    auto& v = acc[p.name];
    v.first += 1;
    v.second += ms;
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
  std::string out;
  char line[256];
  for (auto& kv : acc) {
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (buf && len) {
    const size_t n = std::min(len - 1, out.size());
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return (int)acc.size();
}

int sketch_build(const cfm_bf16* w_gate, const cfm_bf16* w_up, int E, int I, int H,
                 const int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su,
                 void* stream) {
  clear_error();
  if (int rc = check_shape(E, I, H, true)) return rc;
  if (!w_gate || !w_up || !signs || !tg || !tu || !sg || !su)
    return set_error(CFM_EINVAL, "sketch_build: null pointer");
  if ((long)E * I * 2 > 0x7FFFFFFFL) return set_error(CFM_EUNSUPPORTED, "too many rows");
  return launch_sketch_build(w_gate, w_up, E, I, H, signs, tg, tu, sg, su,
                             static_cast<hipStream_t>(stream));
}

int rotation_signs(uint64_t seed, int H, int8_t* signs, void* stream) {
  clear_error();
  if (H <= 0 || H > (1 << 24)) return set_error(CFM_EINVAL, "rotation_signs: H must lie in [1, 2^24]");
  if (!signs) return set_error(CFM_EINVAL, "rotation_signs: null pointer");
  return launch_rotation_signs(seed, H, signs, static_cast<hipStream_t>(stream));
}

size_t sketch_bytes(int E, int I, int H) {
  if (E <= 0 || I <= 0 || H < 64 || H > kMaxH || !is_pow2(H) || I > kMaxI) return 0;
  const size_t rows = (size_t)E * I;
  return 2 * rows * (size_t)(H / 4) + 2 * rows * sizeof(float) + (size_t)H;
}

int sketch_build_seeded(const cfm_bf16* w_gate, const cfm_bf16* w_up, int E, int I, int H, uint64_t seed,
                        int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su, void* stream) {
  clear_error();
  if (int rc = check_shape(E, I, H, true)) return rc;
  if (!w_gate || !w_up || !signs || !tg || !tu || !sg || !su)
    return set_error(CFM_EINVAL, "sketch_build_seeded: null pointer");
  if ((long)E * I * 2 > 0x7FFFFFFFL) return set_error(CFM_EUNSUPPORTED, "too many rows");
  if (int rc = launch_rotation_signs(seed, H, signs, static_cast<hipStream_t>(stream))) return rc;
  return launch_sketch_build(w_gate, w_up, E, I, H, signs, tg, tu, sg, su, static_cast<hipStream_t>(stream));
}

size_t lowrank_workspace(int E, int I, int H, int r) {
  if (E <= 0 || I <= 0 || H <= 0 || r < 0 || r > kMaxRank || r > std::min(H, I)) return 0;
  return lowrank_plan(E, I, H, r).bytes;
}

int lowrank_build(const cfm_bf16* w_down_t, int E, int I, int H, int r, cfm_bf16* A,
                  cfm_bf16* Bt, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_shape(E, I, H, false)) return rc;
  if (r < 0) return set_error(CFM_EUNSUPPORTED, "r must be nonnegative");
  if (r > std::min(H, I)) return set_error(CFM_EUNSUPPORTED, "r must not exceed min(H, I)");
  if (r > kMaxRank) return set_error(CFM_EUNSUPPORTED, "r must be at most 128");
  if (r == 0) return CFM_OK;
  if (!w_down_t || !A || !Bt) return set_error(CFM_EINVAL, "lowrank_build: null pointer");
  const LowrankPlan plan = lowrank_plan(E, I, H, r);
  if (!ws || ws_bytes < plan.bytes)
    return set_error(CFM_EWORKSPACE, "lowrank_build: workspace smaller than lowrank_workspace()");
  return launch_lowrank_build(w_down_t, E, I, H, r, A, Bt, ws, plan,
                              static_cast<hipStream_t>(stream));
}

size_t select_workspace(int T, int K, int E, int I, int H, int k, int c, int r) {
  if (T < 0 || K <= 0 || K > kMaxK || E <= 0 || I <= 0 || I > kMaxI || H < 64 || H > kMaxH ||
      k < 0 || c < k || c > I || r < 0 || r > kMaxRank || r > std::min(H, I))
    return 0;
  const size_t base = select_plan(T, K, E, I, H, k, c, r).bytes;
  if (!grouped_supported(T, K, E, I, H, r, false)) return base;
  return group_plan(T, K, E, I, H, k, c, r, false, base).bytes;
}

int moe_select_forward_ex(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                          int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                          const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                          const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                          const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r,
                          unsigned flags, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out,
                          cfm_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  return select_entry(x, topk_ids, topk_w, T, K, w_gate, w_up, w_down_t, E, I, H, signs, tg, tu, sg, su, A, Bt,
                      k, c, r, flags, false, 0.f, out, cand_out, keep_out, nullptr, stats, ws, ws_bytes, stream);
}

int moe_select_forward_threshold(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                                 int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                                 const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                                 const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                                 const cfm_bf16* A, const cfm_bf16* Bt, float tau, int c, int r,
                                 unsigned flags, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out,
                                 int32_t* keep_count, cfm_stats* stats, void* ws, size_t ws_bytes,
                                 void* stream) {
  clear_error();
  if (!(tau >= 0.f)) return set_error(CFM_EINVAL, "moe_select_forward_threshold: tau must be >= 0 (not NaN)");
  return select_entry(x, topk_ids, topk_w, T, K, w_gate, w_up, w_down_t, E, I, H, signs, tg, tu, sg, su, A, Bt,
                      c, c, r, flags, true, tau, out, cand_out, keep_out, keep_count, stats, ws, ws_bytes,
                      stream);
}

int moe_select_forward_noalloc(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T, int K,
                               const cfm_bf16* w_gate, const cfm_bf16* w_up, const cfm_bf16* w_down_t, int E,
                               int I, int H, const int8_t* signs, const uint8_t* tg, const uint8_t* tu,
                               const float* sg, const float* su, const cfm_bf16* A, const cfm_bf16* Bt, int k,
                               int c, int r, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out, cfm_stats* stats,
                               void* stream) {
  clear_error();
  if (int rc = check_tokens(T, K)) return rc;
  if (int rc = check_shape(E, I, H, true)) return rc;
  if (int rc = check_budget(I, H, k, c, r)) return rc;
  if (T == 0) return CFM_OK;
  const size_t need = select_workspace(T, K, E, I, H, k, c, r);
  if (need > kScratchBytes)
    return set_error(CFM_EWORKSPACE, "moe_select_forward_noalloc: the call needs " + std::to_string(need) +
                                         " bytes of scratch, more than its 32 MiB (use moe_select_forward with a "
                                         "workspace)");
  void* ws = nullptr;
  if (int rc = scratch_address(static_cast<hipStream_t>(stream), &ws)) return rc;
  return select_entry(x, topk_ids, topk_w, T, K, w_gate, w_up, w_down_t, E, I, H, signs, tg, tu, sg, su, A, Bt,
                      k, c, r, 0u, false, 0.f, out, cand_out, keep_out, nullptr, stats, ws, kScratchBytes, stream);
}

int moe_select_forward(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                       const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                       const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                       const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r, cfm_bf16* out,
                       int32_t* cand_out, int32_t* keep_out, cfm_stats* stats, void* ws,
                       size_t ws_bytes, void* stream) {
  return moe_select_forward_ex(x, topk_ids, topk_w, T, K, w_gate, w_up, w_down_t, E, I, H, signs, tg, tu,
                               sg, su, A, Bt, k, c, r, 0u, out, cand_out, keep_out, stats, ws, ws_bytes,
                               stream);
}

namespace {
int check_envelope(int K, int E, float eps, const void* h, const void* norm_w, const void* w_router,
                   const void* out) {
  if (E > 1024) return set_error(CFM_EUNSUPPORTED, "decode-layer envelope: E must be at most 1024");
  if (K > E) return set_error(CFM_EUNSUPPORTED, "decode-layer envelope: K must not exceed E");
  if (!(eps >= 0.f) || eps > 1.f) return set_error(CFM_EINVAL, "decode-layer envelope: eps must lie in [0, 1]");
  if (!h || !norm_w || !w_router || !out) return set_error(CFM_EINVAL, "decode-layer envelope: null pointer");
  return CFM_OK;
}
}  // namespace

int moe_layer_forward(const cfm_bf16* h, const cfm_bf16* norm_w, float eps, const cfm_bf16* w_router,
                      int renorm, int T, int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                      const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                      const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                      const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r, unsigned flags,
                      cfm_bf16* out, int32_t* ids_out, float* w_out, cfm_bf16* x_out, void* ws,
                      size_t ws_bytes, void* stream) {
  clear_error();
  if (flags & ~CFM_RECOVER_CANDIDATES_EXACT) return set_error(CFM_EINVAL, "moe_layer_forward: unknown flag bits");
  if (int rc = check_tokens(T, K)) return rc;
  if (int rc = check_shape(E, I, H, true)) return rc;
  if (int rc = check_budget(I, H, k, c, r)) return rc;
  if (T == 0) return CFM_OK;
  if (int rc = check_envelope(K, E, eps, h, norm_w, w_router, out)) return rc;
  if (!w_gate || !w_up || !w_down_t || !signs || !tg || !tu || !sg || !su)
    return set_error(CFM_EINVAL, "moe_layer_forward: null pointer");
  if (r > 0 && (!A || !Bt)) return set_error(CFM_EINVAL, "moe_layer_forward: null A or Bt with r > 0");
  bool grouped = false;
  if (int rc = pick_grouped(T, K, E, I, H, r, false, &grouped)) return rc;
  const ForwardPlan plan = select_plan(T, K, E, I, H, k, c, r, true);
  const size_t need = grouped ? group_plan(T, K, E, I, H, k, c, r, false, plan.bytes).bytes : plan.bytes;
  if (!ws || ws_bytes < need)
    return set_error(CFM_EWORKSPACE, "moe_layer_forward: workspace smaller than select_workspace()");
  SelectArgs a{nullptr, w_gate, w_up, w_down_t, A, Bt, nullptr, nullptr, signs, tg, tu, sg, su, out,
               nullptr, nullptr, nullptr, static_cast<char*>(ws), flags,
               h, norm_w, w_router, eps, renorm ? 1 : 0, ids_out, w_out, x_out};
  if (grouped)
    return launch_grouped_forward(a, group_plan(T, K, E, I, H, k, c, r, false, plan.bytes),
                                  static_cast<hipStream_t>(stream));
  // many tokens: the grouped pass's router stage and screen in front of the
  // per-pair kernel (its prescreened instance adds the residual). Fewer pairs
  // keep the envelope in the single launch, which overlaps the routing with
  // the rotation (48-layer chained stack, µs per token per layer, route first /
  // fused: 8 tokens 13.6 / 11.3, 16 tokens 9.5 / 9.6, 32 tokens 7.3 / 8.8).
  constexpr long kLayerRouteFirstMinPairs = 192;
  SelectArgs b = a;
  b.route_first = 1;
  b.ws_bytes = ws_bytes;
  const ForwardPlan plain = select_plan(T, K, E, I, H, k, c, r);
  if ((long)T * K >= kLayerRouteFirstMinPairs && select_prescreen_ok(b, plain))
    return launch_select_forward(b, plain, static_cast<hipStream_t>(stream));
  return launch_select_forward(a, plan, static_cast<hipStream_t>(stream));
}

int moe_layer_dense_forward(const cfm_bf16* h, const cfm_bf16* norm_w, float eps, const cfm_bf16* w_router,
                            int renorm, int T, int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                            const cfm_bf16* w_down_t, int E, int I, int H, cfm_bf16* out, int32_t* ids_out,
                            float* w_out, cfm_bf16* x_out, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_tokens(T, K)) return rc;
  if (int rc = check_shape(E, I, H, false)) return rc;
  if (T == 0) return CFM_OK;
  if (int rc = check_envelope(K, E, eps, h, norm_w, w_router, out)) return rc;
  if (!w_gate || !w_up || !w_down_t) return set_error(CFM_EINVAL, "moe_layer_dense_forward: null pointer");
  bool grouped = false;
  if (int rc = pick_grouped(T, K, E, I, H, 0, true, &grouped)) return rc;
  const ForwardPlan plan = dense_plan(T, K, E, I, H, true);
  const size_t need = grouped ? group_plan(T, K, E, I, H, I, I, 0, true, plan.bytes).bytes : plan.bytes;
  if (!ws || ws_bytes < need)
    return set_error(CFM_EWORKSPACE, "moe_layer_dense_forward: workspace smaller than dense_workspace()");
  SelectArgs a{nullptr, w_gate, w_up, w_down_t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
               nullptr, nullptr, nullptr, out, nullptr, nullptr, nullptr, static_cast<char*>(ws), 0u,
               h, norm_w, w_router, eps, renorm ? 1 : 0, ids_out, w_out, x_out};
  if (grouped)
    return launch_grouped_forward(a, group_plan(T, K, E, I, H, I, I, 0, true, plan.bytes),
                                  static_cast<hipStream_t>(stream));
  return launch_dense_forward(a, plan, static_cast<hipStream_t>(stream));
}

size_t dense_workspace(int T, int K, int E, int I, int H) {
  if (T < 0 || K <= 0 || K > kMaxK || E <= 0 || I <= 0 || I > kMaxI || H < 64 || H > kMaxH ||
      H % 64)
    return 0;
  const size_t base = dense_plan(T, K, E, I, H).bytes;
  if (!grouped_supported(T, K, E, I, H, 0, true)) return base;
  return group_plan(T, K, E, I, H, I, I, 0, true, base).bytes;
}

int moe_dense_forward(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                      int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                      const cfm_bf16* w_down_t, int E, int I, int H, cfm_bf16* out, void* ws,
                      size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = check_tokens(T, K)) return rc;
  if (int rc = check_shape(E, I, H, false)) return rc;
  if (T == 0) return CFM_OK;
  if (!x || !topk_ids || !topk_w || !w_gate || !w_up || !w_down_t || !out)
    return set_error(CFM_EINVAL, "moe_dense_forward: null pointer");
  bool grouped = false;
  if (int rc = pick_grouped(T, K, E, I, H, 0, true, &grouped)) return rc;
  const ForwardPlan plan = dense_plan(T, K, E, I, H);
  const size_t need = grouped ? group_plan(T, K, E, I, H, I, I, 0, true, plan.bytes).bytes : plan.bytes;
  if (!ws || ws_bytes < need)
    return set_error(CFM_EWORKSPACE, "moe_dense_forward: workspace smaller than dense_workspace()");
  SelectArgs a{x, w_gate, w_up, w_down_t, nullptr, nullptr, topk_ids, topk_w, nullptr, nullptr,
               nullptr, nullptr, nullptr, out, nullptr, nullptr, nullptr, static_cast<char*>(ws)};
  if (grouped)
    return launch_grouped_forward(a, group_plan(T, K, E, I, H, I, I, 0, true, plan.bytes),
                                  static_cast<hipStream_t>(stream));
  return launch_dense_forward(a, plan, static_cast<hipStream_t>(stream));
}

}  // extern "C"
