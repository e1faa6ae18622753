// Host-side launchers of the HIP kernels (one translation unit each) and the
// workspace layouts shared between the size queries and the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace cfm {

// Byte offset of the failed-launch word in every forward workspace (after the
// 256 launch sequence slots; the same in every layout).
constexpr size_t kFailWordOffset = 1024;
// Zero-fills bytes [0, n) of device memory on `stream` (a fill kernel: no
// memset node, so it may be captured in a graph).
int launch_zero_fill(void* p, size_t n, hipStream_t stream);

int launch_rotation_signs(uint64_t seed, int H, int8_t* signs, hipStream_t stream);
int launch_sketch_build(const uint16_t* w_gate, const uint16_t* w_up, int E, int I, int H,
                        const int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su,
                        hipStream_t stream);

// ---------------------------------------------------------------- low-rank map
struct LowrankPlan {
  int p;          // subspace block width (rank + oversampling, padded to even)
  int iters;      // subspace iterations
  size_t off_gram, off_q, off_y, off_v, bytes;
};
LowrankPlan lowrank_plan(int E, int I, int H, int r);
int launch_lowrank_build(const uint16_t* w_down_t, int E, int I, int H, int r, uint16_t* A,
                         uint16_t* Bt, void* ws, const LowrankPlan& plan, hipStream_t stream);

// ---------------------------------------------------------------- forward passes
// Workspace of a forward pass. The first three regions sit at the same offsets
// in the selected and the dense layouts, so one zeroed buffer can serve both:
// per-workgroup launch sequence numbers (the tag of exchanged values), the
// failed-launch word and the combine counters. Then the exchange buffers.
struct ForwardPlan {
  int T, K, P, E, I, H, k, c, r;
  int nw;         // workgroups per routed pair
  int G;          // grid size (<= one workgroup per compute unit)
  int cw;         // channels screened per workgroup
  int cpw;        // candidates (selected) or channels (dense) per workgroup in the exact phase
  int nhs;        // 64-column output slices per token
  size_t lds;     // dynamic LDS bytes per workgroup
  int pre;        // candidate rows prefetched into LDS (selected pass)
  int env;        // decode-layer envelope (norm, router, residual) fused into the launch
  size_t off_seq, off_err, off_ctr;      // u32 [256], u32, u32 [T][nhs]
  size_t off_xh, off_xz, off_xc;         // tagged u64 [P][I], [P][nw][r], [P][c]
  size_t off_ypart;                      // f32 [P][H]
  size_t off_ypt;                        // tagged u64 [P][H] pair outputs (lean instance's combine)
  size_t off_xl;                         // tagged u64 [T][E] router logits (envelope)
  size_t off_kc;                         // i32 [P] kept counts (threshold keep rule)
  size_t bytes;
};
// G_max: the most workgroups one launch may use (256 for the size queries;
// the launch refits the plan to what the device holds at once)
ForwardPlan select_plan(int T, int K, int E, int I, int H, int k, int c, int r, bool env = false, int G_max = 256);
ForwardPlan dense_plan(int T, int K, int E, int I, int H, bool env = false, int G_max = 256);

struct SelectArgs {
  const uint16_t *x, *w_gate, *w_up, *w_down_t, *A, *Bt;
  const int32_t* ids;
  const float* topk_w;
  const int8_t* signs;
  const uint8_t *tg, *tu;
  const float *sg, *su;
  uint16_t* out;
  int32_t *cand_out, *keep_out;
  void* stats;
  char* ws;
  unsigned flags;   // CFM_RECOVER_* variant bits (0: the default method)
  // decode-layer envelope (moe_layer_forward): x above is unused; the block's
  // input is RMSNorm(resid) and the routing comes from the router rows wr
  const uint16_t *resid, *gamma, *wr;
  float eps;
  int renorm;
  int32_t* ids_out;
  float* w_out;
  uint16_t* x_out;
  // threshold keep rule (thr != 0): S = the candidates whose score key
  // (the bits of |h|) reaches tkey, in place of the top k; the plan's k is c
  int thr;
  uint32_t tkey;
  int32_t* keep_count;
  // bytes of ws (0: unknown); the per-pair pass puts the expert-grouped screen
  // in front of its kernel only when the workspace holds that pass's regions
  size_t ws_bytes;
  // decode-layer envelope served by the per-pair pass with the grouped screen
  // in front: the grouped pass's router stage runs first (x above unused), and
  // the residual resid is added by the per-pair kernel's combine
  int route_first;
};
// Whether the per-pair pass for plan p0 (from select_plan) runs the expert-
// grouped screen in front of its kernel.
bool select_prescreen_ok(const SelectArgs& a, const ForwardPlan& p0);
int launch_select_forward(const SelectArgs& a, const ForwardPlan& p, hipStream_t stream);
// Phase-timestamp buffer for the single-launch kernels (trace build only).
int set_phase_trace(void* buf);
int launch_dense_forward(const SelectArgs& a, const ForwardPlan& p, hipStream_t stream);

// ---------------------------------------------------------------- expert-grouped forward pass
// Workspace of the grouped pass: its regions start at `base` (the end of the
// per-pair layout, so the per-pair pass's persistent words are never touched).
struct GroupPlan {
  int T, K, P, E, I, H, k, c, r;
  bool dense;
  int ntile, IW, nrb;     // 64-channel screen tiles, words of a channel bitmap, 16-row exact blocks
  int IP;                 // row pitch of the union row lists (I rounded up to 8)
  int maxu, maxwork;      // bounds on used experts and screen work items (grid sizes)
  size_t off_uctr, off_kctr, off_octr;   // arrival counters (zero between calls)
  size_t off_rctr;                       // router arrivals per token (zero between calls)
  size_t off_xw, off_lg, off_idw, off_ww; // envelope: normalised states, logits, routing
  size_t off_meta, off_goff, off_gpl, off_gue, off_gux, off_gwork, off_gexw, off_xf0, off_xd, off_hs, off_zp,
      off_cm, off_cl, off_hx, off_km, off_hk, off_zf, off_yp, off_ucnt, off_dcnt, off_urows, off_drows;
  size_t bytes;           // end of the layout (including base)
};
bool grouped_supported(int T, int K, int E, int I, int H, int r, bool dense);
GroupPlan group_plan(int T, int K, int E, int I, int H, int k, int c, int r, bool dense, size_t base);
int launch_grouped_forward(const SelectArgs& a, const GroupPlan& p, hipStream_t stream);
// The grouped pass's rotation, grouping and screen stages alone (sketch
// activations and partial recovery sums into the plan's hs and zp regions),
// for the per-pair pass with several tokens; the caller prepares the workspace.
bool grouped_screen_supported(int T, int K, int E, int I, int H, int r);
int launch_grouped_screen(const SelectArgs& a, const GroupPlan& p, hipStream_t stream);
// The grouped pass's router stage alone (decode-layer envelope): RMSNorm and
// routing into the plan's xw, idw and ww regions, and the optional outputs.
int launch_grouped_route(const SelectArgs& a, const GroupPlan& p, hipStream_t stream);

}  // namespace cfm
