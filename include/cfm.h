/*
 * cfm.h - C ABI of the channel-selected routed-expert SwiGLU FFN for MI355X (gfx950).
 *
 * The method: arXiv:2610.37386, "Channel Selection for Mixture-of-Experts
 * Decoding Needs No Calibration Data" (abstract), and the aimodeling.com
 * article on it (section "A reader that needs no data at all"). Each routed
 * (token, expert) pair screens its expert's intermediate channels with a
 * resident rotated ternary sketch of W_gate / W_up, keeps the top-k channels by
 * exact BF16 gate/up activations (top-k, no calibrated threshold), runs the down
 * projection over those k channels only, and adds back the skipped channels
 * through a rank-r map of W_down built offline from the weights.
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers, allocated and owned by the
 *     caller; the library keeps no device state and allocates no memory,
 *     except where an entry point says otherwise.
 *   - BF16 values are passed as raw 16-bit patterns (cfm_bf16).
 *   - Layouts are row-major and dense. E experts, I intermediate channels per
 *     expert, H hidden width, T tokens, K experts per token, P = T*K pairs.
 *     Expert weights are [E][I][H]; the down projection is passed
 *     channel-major (w_down_t[e][j][:] is column j of W_down), so every
 *     channel's weights are one contiguous H-row.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call except
 *     lowrank_build only enqueues work and returns without waiting.
 *   - Return value: CFM_OK or a negative status; cfm_last_error() gives a
 *     message (thread-local). Argument errors are detected on the host before
 *     anything is enqueued. Asynchronous device faults surface at the next
 *     synchronisation, as with any HIP call.
 *   - Not checked (preconditions): router ids in [0, E) and distinct within a
 *     token; finite inputs; buffers of the documented sizes.
 */
#ifndef CFM_H_
#define CFM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t cfm_bf16;

enum {
  CFM_OK = 0,
  CFM_EINVAL = -1,        /* null pointer where one is required, negative or zero sizes */
  CFM_EUNSUPPORTED = -2,  /* shape or budget outside the supported range (see each call) */
  CFM_EWORKSPACE = -3,    /* workspace missing or smaller than the size query returns */
  CFM_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  CFM_ETIMEOUT = -5       /* a bounded wait inside a forward call expired (cfm_workspace_status) */
};

/* Message of the last failing call on this thread ("" if none). */
const char* cfm_last_error(void);

/* Library version string. */
const char* cfm_version(void);

/*
 * sketch_build - rotated ternary sketch of every expert's gate and up rows.
 * (article section "A reader that needs no data at all": a rotated ternary
 * sketch of each expert's gate and up projections, resident on the GPU,
 * used to screen candidate channels.)
 *
 * For every row w (one channel of W_gate or W_up):
 *   w~ = Hadamard_H * (signs (.) w)     unnormalised Sylvester-Hadamard, float64
 *   delta = 0.7 * mean_i |w~_i|          Ternary Weight Networks threshold
 *   t_i = +1 if w~_i > delta, -1 if w~_i < -delta, else 0
 *   scale = float32( mean_{t_i != 0} |w~_i| / H )   (0 if no t_i is nonzero)
 *
 *   w_gate, w_up : [E][I][H] BF16.
 *   signs        : [H] int8, each +1 or -1; the layer's rotation; the same
 *                  vector must be passed to moe_select_forward.
 *   tg, tu       : out [E][I][H/4] bytes, 2 bits per value. Per row, value
 *                  16b+q and value 16b+8+q (q < 8) share nibble q of the
 *                  little-endian 32-bit word b: bit 4q+0 = (t[16b+8+q] != 0),
 *                  bit 4q+1 = (t[16b+q] != 0), bit 4q+2 = (t[16b+8+q] < 0),
 *                  bit 4q+3 = (t[16b+q] < 0). (word & 0xAAAAAAAA) is then the
 *                  FP4 E2M1 encoding of values 16b..16b+7, and
 *                  ((word << 1) & 0xAAAAAAAA) that of values 16b+8..16b+15.
 *   sg, su       : out [E][I] float32 scales.
 * Supported: H a power of two, 64 <= H <= 8192; E, I >= 1.
 * Sizes: tg/tu E*I*H/4 bytes each (H/4 bytes per row).
 */
int sketch_build(const cfm_bf16* w_gate, const cfm_bf16* w_up, int E, int I, int H,
                 const int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su,
                 void* stream);

/*
 * rotation_signs - the layer's random rotation signs from a seed (article
 * section "A reader that needs no data at all": the sketch is a rotated
 * ternary one; the rotation is a random-sign Walsh-Hadamard transform, and the
 * same signs rotate the hidden states at run time).
 *   signs[i] = +1 if bit 63 of z_i is 0, else -1, for i < H, where z_i is
 *   output i (counting from 0) of SplitMix64 seeded with `seed`:
 *     s = seed + (i + 1) * 0x9E3779B97F4A7C15 (mod 2^64)
 *     z = (s ^ (s >> 30)) * 0xBF58476D1CE4E5B9
 *     z = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *     z_i = z ^ (z >> 31)
 *   signs : out [H] int8 (device). 1 <= H <= 2^24. Enqueued on `stream`.
 */
int rotation_signs(uint64_t seed, int H, int8_t* signs, void* stream);

/*
 * sketch_bytes - device bytes of one layer's sketch: the packed codes tg and
 * tu (E*I*H/4 bytes each), the scales sg and su (E*I float32 each) and the
 * signs (H int8). 0 for a shape sketch_build does not support.
 */
size_t sketch_bytes(int E, int I, int H);

/*
 * sketch_build_seeded - rotation_signs(seed, H, signs) followed by
 * sketch_build with those signs, in stream order: the sketch of a layer from
 * its weights and a seed alone. signs is an output here ([H] int8); every
 * other argument, the layouts, the supported range and the errors are those
 * of sketch_build.
 */
int sketch_build_seeded(const cfm_bf16* w_gate, const cfm_bf16* w_up, int E, int I, int H, uint64_t seed,
                        int8_t* signs, uint8_t* tg, uint8_t* tu, float* sg, float* su, void* stream);

/*
 * lowrank_build - rank-r map of every expert's down projection.
 * (article section "A reader that needs no data at all": the skipped
 * channels are recovered through a low-rank map of the down projections,
 * built from the weights alone.)
 *
 * Computes the rank-r truncated SVD W_down ~ A * Bt^T per expert, with
 * A = W_down V_r = U_r diag(s_r) and Bt = V_r (orthonormal columns), both
 * rounded to BF16. Computed on the device in float64: Gram matrix
 * W_down^T W_down, block subspace iteration with oversampling and a
 * Rayleigh-Ritz step every 4 iterations (until the energy the r leading Ritz
 * vectors capture changes by at most 1e-11 of itself between two such steps,
 * at most 200 iterations). Each column of
 * V_r is signed so that its largest-magnitude entry is positive. Where an
 * expert's W_down has rank below r, the columns past its rank are zero in
 * both A and Bt (they would carry no energy).
 *
 *   w_down_t : [E][I][H] BF16 (channel-major W_down).
 *   A        : out [E][H][r] BF16.   Bt : out [E][I][r] BF16.
 *   ws       : device workspace of at least lowrank_workspace(E, I, H, r) bytes.
 * Supported: 0 <= r <= min(H, I), r <= 128, H <= 8192, I <= 8192.
 * Synchronises `stream` before returning (offline call).
 */
size_t lowrank_workspace(int E, int I, int H, int r);
int lowrank_build(const cfm_bf16* w_down_t, int E, int I, int H, int r, cfm_bf16* A,
                  cfm_bf16* Bt, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_select_forward - the selected-channel MoE layer for a decode batch.
 * (abstract: top-k keeps each token's k highest-scoring channels and reads
 * only their weights; article section "A reader that needs no data at all":
 * sketch screen, exact top-k from the BF16 weights, low-rank recovery.)
 *
 * For each pair (t, q) with e = topk_ids[t][q]:
 *   x~ = Hadamard_H (signs (.) x[t]); ghat_j = sg[e][j] (t^g_j . x~),
 *   uhat_j = su[e][j] (t^u_j . x~), hhat_j = SiLU(ghat_j) uhat_j  (all j < I)
 *   C = the c channels with largest |hhat_j| (ties: lower j)
 *   h_j = SiLU(Wg[e][j] . x[t]) (Wu[e][j] . x[t]) for j in C (BF16 weights,
 *         float32 accumulation)
 *   S = the k channels of C with largest |h_j| (ties: lower j)
 *   y = sum_{j in S} h_j Wd_t[e][j] + A[e] (sum_{j not in S} hhat_j Bt[e][j])
 * out[t] = BF16( sum_q topk_w[t][q] y_(t,q) )  (weights used as given).
 *
 *   x        : [T][H] BF16 hidden states.
 *   topk_ids : [T][K] int32 router choices. topk_w : [T][K] float32.
 *   w_gate, w_up, w_down_t : [E][I][H] BF16.
 *   signs, tg, tu, sg, su  : the layer's sketch from sketch_build.
 *   A [E][H][r], Bt [E][I][r] : the map from lowrank_build (ignored if r = 0).
 *   out      : out [T][H] BF16.
 *   cand_out : optional out [T*K][c] int32, C of each pair in ascending order.
 *   keep_out : optional out [T*K][k] int32, S of each pair in ascending order.
 *   stats    : optional out, device cfm_stats (bytes the call reads: the
 *              per-expert algorithmic count of the method per field, and
 *              bytes_requested as the kernels issue them).
 *   ws       : device workspace of at least select_workspace(...) bytes. It
 *              must be zero-filled once after allocation; every call leaves it
 *              ready for the next call of the same shape. When a call's layout
 *              differs from the previous call on the same workspace (another
 *              T, K, E, I, H, k, c or r, another pass, the dense layer), the
 *              library clears the workspace first with a fill kernel on
 *              `stream` (the library remembers, per workspace address, the
 *              layout of its last call). Calls sharing a workspace must not
 *              overlap. A wait between the workgroups of the single-launch
 *              pass that expires (see cfm_workspace_status) makes that call's
 *              outputs NaN instead of hanging.
 * Supported: H a power of two, 64 <= H <= 8192; 1 <= I <= 8192;
 *            0 <= k <= c <= I; 0 <= r <= min(H, I), r <= 128; K <= 64.
 *            T = 0 is a no-op.
 */
typedef struct {
  uint64_t bytes_sketch;       /* packed sketch + scales of the routed experts */
  uint64_t bytes_candidates;   /* BF16 gate + up rows of the candidates */
  uint64_t bytes_down;         /* BF16 down rows of the kept channels */
  uint64_t bytes_recovery;     /* A and Bt of the routed experts */
  uint64_t bytes_io;           /* x, router output, out */
  uint64_t bytes_dense_equiv;  /* what the dense layer reads for the same routing */
  uint32_t experts_used, rows_candidates, rows_down, pad;
  /* bytes the kernels request from memory (cache hits included), as issued:
     the per-pair pass requests each pair's rows on its own, also when pairs
     share an expert, and where it prefetches the down rows of all c
     candidates (every per-pair instance except the lean one) it requests
     those; the grouped pass requests the per-expert unions above */
  uint64_t bytes_requested;
} cfm_stats;

size_t select_workspace(int T, int K, int E, int I, int H, int k, int c, int r);
int moe_select_forward(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                       const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                       const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                       const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r, cfm_bf16* out,
                       int32_t* cand_out, int32_t* keep_out, cfm_stats* stats, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moe_select_forward_noalloc - moe_select_forward for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). It takes no workspace:
 * its scratch is a 32 MiB array in the library's own device memory, one copy
 * per GPU, created with the library and held until the process ends; the call
 * allocates nothing (no hipMalloc, no allocating library routine). The first
 * call on a GPU looks the array up and zero-fills it on `stream`.
 *   Every argument, output, layout and supported range is that of
 *   moe_select_forward (flags 0, top-k keep rule). A call whose
 *   select_workspace(T, K, E, I, H, k, c, r) exceeds 32 MiB returns
 *   CFM_EWORKSPACE (the Qwen3-30B-A3B-shaped layer fits up to 64 tokens).
 *   All calls on one GPU share its scratch, which keeps the last call's
 *   contents (a call at another shape clears it first, as with any
 *   workspace): calls that overlap on one GPU (concurrent streams or threads)
 *   race and must not be issued. The scratch has no handle for
 *   cfm_workspace_status; an expired exchange wait shows only as NaN outputs.
 */
int moe_select_forward_noalloc(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T, int K,
                               const cfm_bf16* w_gate, const cfm_bf16* w_up, const cfm_bf16* w_down_t, int E,
                               int I, int H, const int8_t* signs, const uint8_t* tg, const uint8_t* tu,
                               const float* sg, const float* su, const cfm_bf16* A, const cfm_bf16* Bt, int k,
                               int c, int r, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out, cfm_stats* stats,
                               void* stream);

/*
 * moe_select_forward_ex - moe_select_forward with variant flags (flags = 0 is
 * moe_select_forward exactly).
 *
 * CFM_RECOVER_CANDIDATES_EXACT: a variant of the recovery step (article
 * section "A reader that needs no data at all" names only a low-rank map of
 * the down projection for the skipped channels). Candidates screened in but
 * not kept (j in C, j not in S) enter the map with their exact activation h_j,
 * which the top-k step has computed, instead of hhat_j; channels never
 * screened in keep hhat_j:
 *   y = sum_{j in S} h_j Wd_t[e][j] + A[e] (sum_{j in C \ S} h_j Bt[e][j]
 *                                          + sum_{j not in C} hhat_j Bt[e][j])
 * With k = 0 the candidates' exact activations are still computed (the only
 * case where the flag adds reads). Every other argument, the supported range,
 * the workspace and the error codes are those of moe_select_forward; a flag
 * bit that is not defined here returns CFM_EINVAL.
 */
#define CFM_RECOVER_CANDIDATES_EXACT 1u
int moe_select_forward_ex(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                          int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                          const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                          const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                          const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r,
                          unsigned flags, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out,
                          cfm_stats* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_select_forward_threshold - the reader with a threshold keep rule in
 * place of top-k, on the same score (abstract: selectors typically keep the
 * channels whose score passes a threshold calibrated offline, and the number
 * that pass varies with the input; article section "Calibrated thresholds do
 * not pin down how much you read"). For each routed pair:
 *   C = as in moe_select_forward (the top c of |hhat|);
 *   S = { j in C : |h_j| >= tau }, ascending, 0 <= |S| <= c (varies by pair);
 *   y, out as in moe_select_forward (or _ex with flags) with that S.
 *   tau        : >= 0 (+inf keeps nothing, 0 every candidate); NaN or a
 *                negative value returns CFM_EINVAL. The calibration that picks
 *                it is the caller's.
 *   keep_out   : optional out [T*K][c] int32: S in ascending order, then -1.
 *   keep_count : optional out [T*K] int32: |S| of each pair.
 *   stats      : rows_down / bytes_down count the kept rows actually read.
 *   ws         : at least select_workspace(T, K, E, I, H, c, c, r) bytes.
 * Every other argument, the supported range, the pass choice and the error
 * codes are those of moe_select_forward_ex.
 */
int moe_select_forward_threshold(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                                 int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                                 const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                                 const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                                 const cfm_bf16* A, const cfm_bf16* Bt, float tau, int c, int r,
                                 unsigned flags, cfm_bf16* out, int32_t* cand_out, int32_t* keep_out,
                                 int32_t* keep_count, cfm_stats* stats, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * moe_dense_forward - the same routed-expert SwiGLU layer reading every channel
 * (the comparator the method is measured against: abstract, "MoE blocks ...
 * faster than optimized vLLM").
 *   out[t] = BF16( sum_q w[t][q] sum_j SiLU(Wg[e][j].x) (Wu[e][j].x) Wd_t[e][j] )
 * Arguments as in moe_select_forward. Same workspace rules.
 * Supported: 64 <= H <= 8192 (multiple of 64), 1 <= I <= 8192, K <= 64.
 */
size_t dense_workspace(int T, int K, int E, int I, int H);
int moe_dense_forward(const cfm_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                      int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                      const cfm_bf16* w_down_t, int E, int I, int H, cfm_bf16* out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * moe_layer_forward - the routed-expert block of one decode layer with its
 * envelope, in one launch: the RMSNorm before it, the router, and the
 * residual add after it (the pages measure MoE-block and whole-model decoding
 * with routing in place: abstract). For each token t:
 *   x[t]   = BF16( (h[t] s) norm_w ),  s = 1 / sqrt(mean_i h[t][i]^2 + eps)
 *            (float32, one rounding);
 *   l_e    = W_r[e] . x[t] (float32 accumulation), p = softmax(l) over E;
 *   ids[t] = the K experts of largest p in descending order (lower id first
 *            on ties), w[t] = their p, divided by their sum if renorm != 0;
 *   out[t] = BF16( h[t] + sum_q w[t][q] y_(t,q) ), y as in moe_select_forward
 *            (or moe_select_forward_ex with flags) on x, ids, w.
 *
 *   h        : [T][H] BF16 hidden states (the residual stream); out may be h.
 *   norm_w   : [H] BF16 RMSNorm weight. eps: 0 <= eps <= 1.
 *   w_router : [E][H] BF16 router rows.
 *   ids_out, w_out : optional out [T][K] int32 / float32, the routing used.
 *   x_out    : optional out [T][H] BF16, the normalised states.
 *   Every other argument as in moe_select_forward_ex; the workspace is
 *   select_workspace(T, K, E, I, H, k, c, r) bytes, same rules.
 * Supported: as moe_select_forward, and E <= 1024, K <= E. The pass is chosen
 * as for moe_select_forward (cfm_set_forward_path): the per-pair kernel forms
 * the envelope inside its one launch; the expert-grouped pass runs a router
 * step first, and so does the per-pair pass from 192 routed pairs (with a
 * workspace of select_workspace bytes, forward path 0 or 1), followed by the
 * grouped screen and the per-pair kernel, which adds the residual. All of
 * them form the same normalised states and routing.
 */
int moe_layer_forward(const cfm_bf16* h, const cfm_bf16* norm_w, float eps, const cfm_bf16* w_router,
                      int renorm, int T, int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                      const cfm_bf16* w_down_t, int E, int I, int H, const int8_t* signs,
                      const uint8_t* tg, const uint8_t* tu, const float* sg, const float* su,
                      const cfm_bf16* A, const cfm_bf16* Bt, int k, int c, int r, unsigned flags,
                      cfm_bf16* out, int32_t* ids_out, float* w_out, cfm_bf16* x_out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * moe_layer_dense_forward - the same envelope around the dense block
 * (moe_dense_forward), the comparator. Workspace: dense_workspace(T, K, E, I, H).
 * Supported: as moe_dense_forward, and E <= 1024, K <= E.
 */
int moe_layer_dense_forward(const cfm_bf16* h, const cfm_bf16* norm_w, float eps, const cfm_bf16* w_router,
                            int renorm, int T, int K, const cfm_bf16* w_gate, const cfm_bf16* w_up,
                            const cfm_bf16* w_down_t, int E, int I, int H, cfm_bf16* out, int32_t* ids_out,
                            float* w_out, cfm_bf16* x_out, void* ws, size_t ws_bytes, void* stream);

/*
 * cfm_set_forward_path - which kernels serve moe_select_forward and
 * moe_dense_forward (process-wide, shared by every thread of the process; an
 * atomic setting, but a call on one thread changes the pass of concurrent
 * calls on others; returns the previous setting, or CFM_EINVAL).
 *   0 automatic (default): the expert-grouped pass where the shape allows it
 *     and the batch is large (selected layer: 48 tokens or more, or more than
 *     256 routed pairs; dense layer: 32 tokens or more), the per-pair pass
 *     otherwise;
 *   1 the per-pair pass (one persistent launch; lowest latency at batch 1).
 *     With several sub-chunks of channels per workgroup (several tokens per
 *     call, H <= 2048, I <= 1024, r a multiple of 8, a workspace of
 *     select_workspace bytes) the expert-grouped pass's screen runs first, as
 *     two short launches that read each routed expert's sketch once for all
 *     of its tokens, and the persistent launch starts from its sketch
 *     activations (the same values the launch would compute itself);
 *   2 the expert-grouped pass (pairs grouped by expert; each weight row an
 *     expert needs is read once for all of its tokens: the larger batches at
 *     which the article, section "Numbers and limits", reports the largest
 *     gains, peaking at batch 8 or 16). Calls whose
 *     shape it does not cover return CFM_EUNSUPPORTED: it needs T K <= 65535,
 *     E <= 4096, and for the selected layer r a multiple of 8;
 *   3 the per-pair pass on its general instance only: not the batch-1
 *     instance (compiled for the Qwen3-30B-A3B-shaped batch-1 call: H 2048,
 *     r 64, at most 8 pairs), not the instance that keeps the next sub-chunk
 *     of sketch rows in flight (several sub-chunks of channels per workgroup,
 *     plain method, H <= 2048, I <= 1024), and no grouped screen in front;
 *     for comparison and testing;
 *   4 the per-pair pass with the screen always inside the persistent launch
 *     (no grouped screen in front), for comparison and testing.
 * Both passes compute the same selections (identical sketch activations, so
 * identical candidate sets; exact activations and outputs agree to float
 * rounding). The workspace sizes returned by select_workspace and
 * dense_workspace cover both.
 */
int cfm_set_forward_path(int path);

/*
 * Instrumentation (not part of the method). While enabled, every kernel the
 * library launches is bracketed by a pair of HIP events recorded on the
 * launch stream. cfm_timing_report synchronises those events, writes one line
 * per kernel name, "<name> <launches> <total_ms>\n", into buf (NUL-terminated,
 * truncated to len), clears the record and returns the number of kernel names
 * (or a negative status). Host-side state only; not thread-safe.
 */
int cfm_timing_enable(int on);
int cfm_timing_report(char* buf, size_t len);

/*
 * cfm_workspace_status - the failure channel of the forward calls. The
 * single-launch pass (the per-pair kernel behind moe_select_forward, its
 * variants, moe_dense_forward and the moe_layer_* calls at small batch) runs
 * all of its workgroups at once, sized from the device's compute units and the
 * kernel's occupancy, and they exchange values through the workspace with
 * bounded waits. If a wait expires (for instance because other work occupied
 * compute units, so the workgroups were not all resident), the call's outputs
 * are NaN and a failure word in the workspace records it. This call
 * synchronises `stream`, reads and clears that word, and returns CFM_OK if no
 * wait expired since the last check (or since the workspace was zeroed), else
 * CFM_ETIMEOUT. ws_bytes: the workspace size (at least 1028 bytes).
 */
int cfm_workspace_status(void* ws, size_t ws_bytes, void* stream);

/*
 * cfm_set_wait_limit - polls of one exchanged value before a single-launch
 * forward pass gives up (process-wide; default 2^20, about one second). 0
 * makes every wait give up at once, so that the failure path can be exercised
 * without a fault: every workgroup still runs to its end. Returns the
 * previous value. Instrumentation and testing only.
 */
int cfm_set_wait_limit(unsigned polls);

/*
 * cfm_set_resident_limit - caps the number of workgroups a single-launch
 * forward pass assumes resident at once (process-wide; -1, the default: the
 * device's compute units times the kernel's occupancy). A smaller grid runs
 * the routed pairs in rounds of the same launch; 0 stands for a device that
 * holds none, so that the refusal can be exercised: the call then returns
 * CFM_EUNSUPPORTED before launching anything. For callers that share the GPU
 * with other resident work, and for testing. Returns the previous value.
 */
int cfm_set_resident_limit(int workgroups);

/*
 * cfm_phase_trace - instrumentation of the single-launch kernels (not part of
 * the method). In the trace build of the library (compiled with
 * CFM_PHASE_TRACE), every later per-pair launch stores, from thread 0 of each
 * workgroup b, the 100 MHz device clock at fixed points of its phases into
 * buf[b * 32 + n] (uint64, device memory of at least 256 * 32 * 8 bytes) and
 * the XCD it runs on into buf[b * 32 + 31]; buf = NULL stops it. Each launch
 * overwrites the previous one's stamps. Host-side state only; not
 * thread-safe. The default build returns CFM_EUNSUPPORTED.
 */
int cfm_phase_trace(void* buf);

#ifdef __cplusplus
}
#endif

#endif /* CFM_H_ */
