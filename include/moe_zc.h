/*
 * moe_zc.h -- C ABI of the MI355X (gfx950) MoE layer with zero-computation
 * experts.
 *
 * The layer (LongCat-Flash; page 『衝上熱搜！美團大模型，靠「快」火了』,
 * section 零計算專家 -- its defining equation was an image that did not survive,
 * so the formula below is rebuilt from that section's symbol legend):
 *   a pool of E = N + Z experts: N SwiGLU FFN experts (indices 0..N-1) and Z
 *   zero-computation experts (indices N..E-1) that return their input as is;
 *   a softmax router R; a per-expert bias b_i that only steers which K experts
 *   a token goes to.  For each token t:
 *     l[t,i] = x_t . W_router[i]                     (fp32)
 *     p[t,i] = softmax over all E experts of l[t,:]   (evaluated in fp64)
 *     key    = fl32(fl32(p) + b_i); top-K by key descending, ties to the lower
 *              expert index
 *     g      = fl32(p) of each chosen expert (unbiased, not renormalised)
 *     y_t    = r_t + sum over chosen slots, in key order, of
 *              g * (W_down_i (silu(W_gate_i x_t) * (W_up_i x_t)))  for i < N
 *              g * x_t                                             for i >= N
 *   The bias is adjusted between forwards by a PID controller on the expert
 *   loads (same section; page 『美团的 LongCat-Flash：用 27B 激活算力跑起一个
 *   560B 模型』, section 关键要点).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous,
 *     owned by the caller.  The library keeps no pointer after a call returns
 *     and allocates no device memory: scratch comes from the caller's
 *     workspace.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; no call synchronises the device.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is enqueued and outputs are untouched.
 *   - A launch failure returns MOE_ZC_ERR_HIP.  Faults inside kernels surface
 *     at the caller's next synchronisation.
 *   - Non-finite inputs are outside the contract (results are undefined).
 *   - Results are bitwise reproducible run to run: no floating-point atomics,
 *     fixed reduction orders.
 *   - Calls on different streams with disjoint outputs and workspaces may run
 *     concurrently; the library has no mutable global state.
 *   - No entry point allocates, synchronises or issues a memset, so the
 *     work-enqueuing calls can be captured in a HIP graph and replayed.
 */
#ifndef MOE_ZC_H
#define MOE_ZC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ZC_ABI_VERSION 3

typedef enum {
  MOE_ZC_OK = 0,
  MOE_ZC_ERR_INVALID = 1,      /* bad argument: NULL, negative size, K > E ... */
  MOE_ZC_ERR_WORKSPACE = 2,    /* workspace NULL or smaller than required     */
  MOE_ZC_ERR_UNSUPPORTED = 3,  /* valid but outside what the kernels handle   */
  MOE_ZC_ERR_HIP = 4,          /* a HIP launch or runtime call failed         */
  /* not a status: makes every int a valid value of the type, so that an
   * out-of-range value passed in from C is well defined (and rejected) */
  MOE_ZC_STATUS_INT32_ = 0x7fffffff
} moe_zc_status;

typedef enum {
  MOE_ZC_F32 = 0,   /* x, FFN weights, residual, y in fp32 (fp32 FMA path)     */
  MOE_ZC_BF16 = 1,  /* x, FFN weights, residual, y in bf16 (bf16 MFMA path)    */
  MOE_ZC_DTYPE_INT32_ = 0x7fffffff  /* not a dtype (as above): rejected as invalid */
} moe_zc_dtype;

/* Limits of this implementation (else MOE_ZC_ERR_UNSUPPORTED):
 *   E = N + Z in [1, 2048]; K in [1, min(E, 32)];
 *   bf16: d a multiple of 64 and I of 128 (the gate/up GEMM pairs 128 gate
 *   and 128 up rows of the same hidden units in one 256-column panel, so
 *   that SwiGLU needs no second pass);  f32: d and I multiples of 32;
 *   d, I < 2^20, d * I < 2^31, 2 * d * E < 2^31, T * min(K, N) < 2^31 and
 *   T * max(d, I, E) < 2^40. */
#define MOE_ZC_MAX_EXPERTS 2048
#define MOE_ZC_MAX_TOPK 32

/* Timed stages of moe_zc_forward (see moe_zc_aux.stage_events), in order:
 * 0 router GEMM, 1 softmax + bias + top-K, 2 per-chunk expert histogram,
 * 3 scan (loads, offsets, tile schedule), 4 permute (grouping and row
 * gather), 5 grouped GEMM gate/up + SwiGLU, 6 grouped GEMM down, 7 combine.
 * Event i is recorded just before stage i, event 8 after the combine. */
#define MOE_ZC_NUM_STAGES 8
#define MOE_ZC_NUM_EVENTS (MOE_ZC_NUM_STAGES + 1)

/* Optional extra outputs of moe_zc_forward.  Every field may be NULL (not
 * produced).  All arrays are device memory owned by the caller.
 *   logits      [T, E]  fp32 router logits l
 *   topk_idx    [T, K]  chosen experts, key descending, ties to lower index
 *   topk_gate   [T, K]  fl32(p) of the chosen experts
 *   loads       [E]     slots routed to each expert (FFN and zero alike);
 *                       this is what moe_zc_bias_update consumes
 *   offsets     [N + 1] exclusive prefix sum of loads[0..N-1]; offsets[N] = S,
 *                       the number of (token, FFN expert) rows (there is no
 *                       separate row-count output: offsets[N] is it)
 *   perm        [T * min(K, N)]  token held by grouped row s (first S valid);
 *                       rows are grouped by expert, tokens ascending
 *   pos         [T, K]  grouped row of slot (t,k), -1 for a zero expert
 *   stage_events [MOE_ZC_NUM_EVENTS] created HIP events, recorded on
 *                       `stream` at stage boundaries (for timing), or NULL
 *   act         [T * min(K, N), 2I] bf16 (16-byte aligned): the expert
 *                       pre-activations of grouped row s, a = W_gate x in
 *                       columns [0, I) and u = W_up x in [I, 2I), rounded
 *                       once from the fp32 accumulators (first S rows valid).
 *                       What moe_zc_backward reads instead of recomputing
 *                       them.  dt = bf16 only (else MOE_ZC_ERR_UNSUPPORTED).
 * (act was added in ABI version 2.) */
typedef struct moe_zc_aux {
  float* logits;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* loads;
  int32_t* offsets;
  int32_t* perm;
  int32_t* pos;
  hipEvent_t* stage_events;
  void* act;
} moe_zc_aux;

/* Bytes of device workspace moe_zc_forward needs for these sizes (0 if the
 * sizes are invalid).  Host only; enqueues nothing. */
size_t moe_zc_workspace_size(int64_t T, int64_t d, int64_t I, int32_t N,
                             int32_t Z, int32_t K, moe_zc_dtype dt);

/* Forward of the layer for T tokens (definition at the top of this file).
 *   x         [T, d]      dt
 *   w_router  [E, d]      fp32   (E = N + Z; row i scores expert i)
 *   bias      [E]         fp32   selection bias b
 *   w_gate    [N, I, d]   dt     (nn.Linear layout [out, in])
 *   w_up      [N, I, d]   dt
 *   w_down    [N, d, I]   dt
 *   residual  [T, d]      dt or NULL (then y = MoE(x))
 *   y         [T, d]      dt     output; may not alias any input
 *   aux       NULL or extra outputs (see moe_zc_aux)
 *   workspace device buffer of at least moe_zc_workspace_size(...) bytes,
 *             256-byte aligned; contents on entry are ignored.
 * N may be 0 (every expert is a zero expert; the FFN weights may be NULL).
 * T = 0 returns MOE_ZC_OK and enqueues nothing.
 * Precision: router logits fp32 (bf16 path: x times a two-term bf16 split of
 * W_router on MFMA, fp32 accumulation; with few tokens the reduction is cut
 * into equal parts whose fp32 partial sums are added in a fixed order);
 * softmax in fp64; FFN on bf16 MFMA
 * with fp32 accumulation, SiLU in fp32, the hidden activation and expert
 * outputs stored in dt; combine accumulated in fp32 and rounded once. */
moe_zc_status moe_zc_forward(const void* x, const float* w_router,
                             const float* bias, const void* w_gate,
                             const void* w_up, const void* w_down,
                             const void* residual, void* y, int64_t T,
                             int64_t d, int64_t I, int32_t N, int32_t Z,
                             int32_t K, moe_zc_dtype dt, moe_zc_aux* aux,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---- packed expert weights (bf16) ------------------------------------------
 * The bf16 expert GEMMs stream every expert's weights from HBM once per
 * forward; they run fastest when those weights sit in the order the matrix
 * cores consume them.  Pack them once, when the model is loaded, with
 * moe_zc_pack_expert_weights, then call moe_zc_forward_packed: it computes
 * exactly what moe_zc_forward computes on the row-major weights (bitwise
 * equal outputs), only faster.  The packed layout is opaque; its size per
 * expert comes from moe_zc_packed_expert_bytes.  Expert e's packed weights
 * start at byte e * gate_up_bytes (resp. e * down_bytes), so a model can be
 * packed expert by expert into offset pointers. */

/* Bytes of ONE expert's packed weights: *gate_up_bytes for the gate and up
 * projections together (4 d I), *down_bytes for the down projection
 * (2 I * d rounded up to a multiple of 256 rows).  dt must be MOE_ZC_BF16
 * (MOE_ZC_ERR_UNSUPPORTED for MOE_ZC_F32); d and I follow the limits of
 * moe_zc_forward.  Host only. */
moe_zc_status moe_zc_packed_expert_bytes(int64_t d, int64_t I, moe_zc_dtype dt,
                                         size_t* gate_up_bytes,
                                         size_t* down_bytes);

/* Pack n_experts experts (device pointers, bf16, row-major as taken by
 * moe_zc_forward):
 *   w_gate, w_up [n_experts, I, d],  w_down [n_experts, d, I]
 * into gate_up_packed (n_experts * gate_up_bytes) and down_packed
 * (n_experts * down_bytes), all 16-byte aligned and owned by the caller.
 * Enqueued on `stream`; reads the inputs once.  n_experts = 0 does nothing. */
moe_zc_status moe_zc_pack_expert_weights(const void* w_gate, const void* w_up,
                                         const void* w_down, int32_t n_experts,
                                         int64_t d, int64_t I, moe_zc_dtype dt,
                                         void* gate_up_packed, void* down_packed,
                                         hipStream_t stream);

/* moe_zc_forward with the FFN expert weights packed by
 * moe_zc_pack_expert_weights (gate_up_packed, down_packed: N experts each;
 * NULL allowed when N = 0).  bf16 only (MOE_ZC_ERR_UNSUPPORTED otherwise);
 * every other argument, the workspace size and the outputs are those of
 * moe_zc_forward. */
moe_zc_status moe_zc_forward_packed(const void* x, const float* w_router,
                                    const float* bias,
                                    const void* gate_up_packed,
                                    const void* down_packed,
                                    const void* residual, void* y, int64_t T,
                                    int64_t d, int64_t I, int32_t N, int32_t Z,
                                    int32_t K, moe_zc_dtype dt, moe_zc_aux* aux,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ---- the packed forward without allocation ----------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The library holds one fixed scratch array of
 * MOE_ZC_NOALLOC_SCRATCH_BYTES per GPU (a static device array: each GPU the
 * library runs on keeps it until the process ends) and uses it as the
 * workspace of moe_zc_forward_packed.  The call allocates nothing.  Sizes
 * whose workspace (moe_zc_workspace_size) exceeds the scratch are refused
 * with MOE_ZC_ERR_WORKSPACE before anything is enqueued: 64 MiB holds the
 * decode-shaped layer (d = 6144, I = 2048, N = 512, Z = 256, K = 12) up to
 * T = 160 tokens.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap in time on one GPU (for example on two streams) race and
 * must be serialised by the caller.  Nothing in the scratch needs to start
 * at zero.  `stream` must belong to the current device (else
 * MOE_ZC_ERR_INVALID).  Everything else -- arguments, outputs, aux, results
 * (bitwise equal to moe_zc_forward_packed) -- is as moe_zc_forward_packed. */
#define MOE_ZC_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_zc_status moe_zc_forward_packed_noalloc(const void* x, const float* w_router,
                                            const float* bias,
                                            const void* gate_up_packed,
                                            const void* down_packed,
                                            const void* residual, void* y,
                                            int64_t T, int64_t d, int64_t I,
                                            int32_t N, int32_t Z, int32_t K,
                                            moe_zc_dtype dt, moe_zc_aux* aux,
                                            hipStream_t stream);

/* ---- block-FP8 expert projections (mixed precision) -------------------------
 * The LongCat pages report that the model quantizes with DeepSeek-V3's
 * fine-grained block scheme and picks precision layer by layer, because the
 * down projection's input activations reach about 1e6 (『衝上熱搜！美團大模型，
 * 靠「快」火了』, paragraph on quantization in the system-optimisation
 * section).  This path runs the expert gate/up projection in block FP8, and
 * the down projection in bf16 or (per layer, down_fp8 = 1) block FP8 too; the
 * router and the combine stay bf16 / fp32.  The block geometry departs from
 * DeepSeek-V3's (1 x 128 activation tiles and 128 x 128 weight blocks with
 * fp32 scales): it is the MX form the MI355X matrix cores consume.
 *   FP8 block: 32 consecutive values along the reduction axis share one
 *   power-of-two scale 2^s, stored as the byte s + 127; s is the smallest
 *   integer with max|v| <= 448 * 2^s, clamped to [-127, 127] (an all-zero
 *   block takes -127); each value is stored as the E4M3 code (1 sign, 4
 *   exponent bits with bias 7, 3 mantissa bits, largest finite 448) of
 *   v / 2^s, rounded to nearest even, sign bit copied from v.
 * gate/up: x is quantized per token along d, W_gate and W_up per output row;
 * h is rounded to bf16 as on the bf16 path.  down (FP8): h of each grouped
 * row is quantized along I from its fp32 value (the gate/up epilogue writes
 * the codes and scales instead of bf16 h), W_down per output row along I.  The
 * matrix cores apply both scales and accumulate in fp32.  Results differ from
 * moe_zc_forward by the FP8 rounding of the quantized inputs (about 2^-4
 * relative per value); routing is unchanged.
 * Requires dt = bf16, d a multiple of 128, T * d < 2^31 and
 * T * min(K, N) * I < 2^31 (else MOE_ZC_ERR_UNSUPPORTED); other limits as
 * moe_zc_forward. */

/* Bytes of ONE expert's packed FP8 weights (host only): *gate_up_bytes for
 * gate and up (I / 128 panels by d / 128 stages of 33 KB: 2 d I bytes of
 * codes, 2 d I / 32 of scales); *down_bytes, when down_bytes is not NULL, for
 * the FP8 down projection (d rounded up to 256 rows, I / 128 stages of 33 KB).
 * A bf16 down projection keeps moe_zc_packed_expert_bytes' down_bytes.
 * (down_bytes was added in ABI version 3.) */
moe_zc_status moe_zc_packed_fp8_expert_bytes(int64_t d, int64_t I,
                                             size_t* gate_up_bytes,
                                             size_t* down_bytes);

/* Quantize and pack n_experts experts' gate and up weights (device, bf16,
 * row-major [n_experts, I, d] each, 16-byte aligned) into gate_up_fp8
 * (n_experts * gate_up_bytes, 16-byte aligned, caller-owned; expert e at byte
 * e * gate_up_bytes), and, when w_down ([n_experts, d, I] bf16) and down_fp8
 * (n_experts * down_bytes) are given, the down weights too (both NULL or both
 * set, else MOE_ZC_ERR_INVALID).  Enqueued on `stream`.  n_experts = 0 does
 * nothing.  (w_down and down_fp8 were added in ABI version 3.) */
moe_zc_status moe_zc_pack_expert_weights_fp8(const void* w_gate,
                                             const void* w_up,
                                             const void* w_down,
                                             int32_t n_experts, int64_t d,
                                             int64_t I, void* gate_up_fp8,
                                             void* down_fp8, hipStream_t stream);

/* Workspace bytes of moe_zc_forward_packed_fp8 (moe_zc_forward's plus the
 * FP8 codes and scales of x and of h); 0 for unsupported sizes.  Host only. */
size_t moe_zc_workspace_size_fp8(int64_t T, int64_t d, int64_t I, int32_t N,
                                 int32_t Z, int32_t K);

/* moe_zc_forward (dt = bf16) with the gate/up projection in block FP8:
 * gate_up_fp8 from moe_zc_pack_expert_weights_fp8; down_fp8 = 0: `down` is
 * the bf16 down projection packed by moe_zc_pack_expert_weights; down_fp8 = 1:
 * `down` is the FP8 down projection packed by moe_zc_pack_expert_weights_fp8
 * (any other value: MOE_ZC_ERR_INVALID).  N experts each; NULL allowed when
 * N = 0.  The workspace must hold moe_zc_workspace_size_fp8 bytes.  Outputs
 * and the aux contract are those of moe_zc_forward; the FP8 stage of x counts
 * in the gate/up stage event.
 * (down_fp8 was added in ABI version 3.) */
moe_zc_status moe_zc_forward_packed_fp8(const void* x, const float* w_router,
                                        const float* bias,
                                        const void* gate_up_fp8,
                                        const void* down, int32_t down_fp8,
                                        const void* residual, void* y,
                                        int64_t T, int64_t d, int64_t I,
                                        int32_t N, int32_t Z, int32_t K,
                                        moe_zc_aux* aux, void* workspace,
                                        size_t workspace_bytes,
                                        hipStream_t stream);

/* Block-FP8 quantization of bf16 rows (device): x [rows, d] (16-byte
 * aligned) -> codes [rows, d] E4M3 bytes (16-byte aligned) and scales
 * [rows, d / 32] bytes, by the rule above.  d must be a multiple of 32
 * (MOE_ZC_ERR_UNSUPPORTED).  Enqueued on `stream`; rows = 0 does nothing. */
moe_zc_status moe_zc_quantize_mx(const void* x, int64_t rows, int64_t d,
                                 void* codes, void* scales, hipStream_t stream);

/* ---- backward (training) --------------------------------------------------
 * The pages count fully deterministic computation among LongCat-Flash's
 * training techniques: runs reproduce bit for bit, which also exposes silent
 * data corruption (『衝上熱搜！美團大模型，靠「快」火了』, section
 * 模型擴展策略與多階段訓練, its fourth point).  This is the layer's backward
 * with that property: no atomics, every reduction in a fixed order.
 * Given the upstream gradient dy = dL/dy and the routing the forward saved in
 * its moe_zc_aux (routing is piecewise constant and passes no gradient; the
 * selection bias receives none; the gate is the probability itself):
 *   slot (t,k) on FFN expert e, a = W_gate x_t, u = W_up x_t, s = sigmoid(a),
 *   h = silu(a) u, o = W_down h, q = W_down^T dy_t:
 *     gate gradient  <dy_t, o> = <q, h>
 *     da = g q u s (1 + a (1 - s)),  du = g q silu(a)
 *     dx_t += W_gate^T da + W_up^T du
 *     dW_down[e] += (g dy_t) h^T,  dW_gate[e] += da x_t^T,  dW_up[e] += du x_t^T
 *   slot (t,k) on a zero expert: gate gradient <dy_t, x_t>, dx_t += g dy_t
 *   router: dl_t = p_t * (dp_t - <p_t, dp_t>), dp_t = gate gradients at the
 *   chosen experts (0 elsewhere), p = softmax(l_t);
 *     dx_t += W_router^T dl_t,  dW_router += dl_t x_t^T
 *   The residual's gradient is dy itself and is not returned.
 * Precision: q (and a, u when not saved by the forward) come from bf16 MFMA
 * with fp32 accumulation; da, du, h, g dy and dl are rounded to bf16 as
 * operands of the following products (fp32 accumulation), and so is W_router
 * in the router's dx term; dx is accumulated in fp32 and rounded once to
 * bf16.
 * Requires dt = bf16 and T * d < 2^31 (else MOE_ZC_ERR_UNSUPPORTED); other
 * limits as moe_zc_forward. */

/* Bytes of ONE expert's transposed weights for the backward (host only):
 * *gate_up_t_bytes for [W_gate; W_up]^T ([d, 2I]) and *down_t_bytes for
 * W_down^T ([I, d]), each in the packed layout of moe_zc_pack_expert_weights'
 * down projection (rows padded to 256).  Shape rules of
 * moe_zc_pack_expert_weights (bf16). */
moe_zc_status moe_zc_transposed_expert_bytes(int64_t d, int64_t I,
                                             size_t* gate_up_t_bytes,
                                             size_t* down_t_bytes);

/* The transposed expert weights the backward reads, packed (device, bf16):
 *   w_gate, w_up [n, I, d], w_down [n, d, I] (row-major, 16-byte aligned)
 *   -> w_gate_up_t: n blocks of gate_up_t_bytes holding M[e][j][k] =
 *      W_gate[e][k][j] (k < I), W_up[e][k - I][j] (k >= I), j < d;
 *      w_down_t: n blocks of down_t_bytes holding W_down[e]^T [I, d];
 *   both in the opaque packed layout (sizes: moe_zc_transposed_expert_bytes).
 * Outputs are caller-owned and 16-byte aligned.  Built once, like the packed
 * forward weights; enqueued on `stream`; n_experts = 0 does nothing. */
moe_zc_status moe_zc_transpose_expert_weights(const void* w_gate,
                                              const void* w_up,
                                              const void* w_down,
                                              int32_t n_experts, int64_t d,
                                              int64_t I, void* w_gate_up_t,
                                              void* w_down_t,
                                              hipStream_t stream);

/* Workspace bytes of moe_zc_backward (0 for invalid or unsupported sizes).
 * Host only. */
size_t moe_zc_backward_workspace_size(int64_t T, int64_t d, int64_t I,
                                      int32_t N, int32_t Z, int32_t K);

/* Gradients of the layer (definition above), dt = bf16.
 *   x, w_router, w_gate, w_up   the forward's inputs (w_router fp32)
 *   w_gate_up_t, w_down_t       from moe_zc_transpose_expert_weights
 *   fwd       the forward's aux with logits, topk_idx, topk_gate, offsets,
 *             perm and pos filled (same x, w_router, bias, sizes); read only.
 *             With fwd->act filled as well, a and u are taken from it
 *             instead of being recomputed, and w_gate, w_up may be NULL.
 *   dy        [T, d] bf16 upstream gradient
 *   dx        [T, d] bf16 output
 *   dw_router [E, d] fp32 output
 *   dw_gate, dw_up [N, I, d], dw_down [N, d, I] fp32 outputs (every expert
 *             written; experts no token chose get zeros)
 *   Every tensor pointer, outputs included, must be 16-byte aligned (else
 *   MOE_ZC_ERR_INVALID): the kernels use 16-byte vector accesses.
 *   workspace device buffer of moe_zc_backward_workspace_size(...) bytes,
 *             256-byte aligned; contents on entry are ignored.
 * Outputs overwrite (do not accumulate into) their buffers and may not alias
 * inputs.  N = 0: the expert arguments may be NULL.  T = 0 returns MOE_ZC_OK
 * and enqueues nothing (the weight gradients are then not written). */
moe_zc_status moe_zc_backward(const void* x, const float* w_router,
                              const void* w_gate, const void* w_up,
                              const void* w_gate_up_t, const void* w_down_t,
                              const moe_zc_aux* fwd, const void* dy, void* dx,
                              float* dw_router, float* dw_gate, float* dw_up,
                              float* dw_down, int64_t T, int64_t d, int64_t I,
                              int32_t N, int32_t Z, int32_t K, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Routing alone, from given fp32 logits [T, E] and bias [E]: the softmax,
 * bias key and top-K step of the forward, bit for bit.
 *   topk_idx [T, K] int32 and topk_gate [T, K] fp32 outputs (device).
 *   loads    [E] int32 output (device) or NULL: slots routed to each expert,
 *            FFN and zero experts alike (what moe_zc_bias_update consumes);
 *            with T = 0 it is set to zeros.
 * Same validation rules and limits as moe_zc_forward.  (loads was added in
 * ABI version 3.) */
moe_zc_status moe_zc_route(const float* logits, const float* bias, int64_t T,
                           int32_t E, int32_t K, int32_t* topk_idx,
                           float* topk_gate, int32_t* loads,
                           hipStream_t stream);

/* PID controller state for moe_zc_bias_update.  Gains live on the host; the
 * error histories are device arrays of E floats, owned by the caller, zeroed
 * before the first step and carried between steps (save and restore them with
 * the bias to resume: that reproduces the uninterrupted run bit for bit).
 * The velocity form below needs no step counter: the two error histories
 * are the whole state, so the struct carries none. */
typedef struct moe_zc_pid {
  float kp, ki, kd;
  float* e_prev;    /* [E] error of the previous step        */
  float* e_prev2;   /* [E] error of the step before that     */
} moe_zc_pid;

/* One PID step on the expert bias from measured loads (pages: a PID
 * controller tunes the expert bias in real time from recent usage --
 * 『衝上熱搜！美團大模型，靠「快」火了』, section 零計算專家; busy experts get
 * less work, idle ones more -- 『美团 LongCat-Flash 这个5600亿参数的懒AI，
 * 竟然比勤奋的模型跑得更快？』).  With e_i = (target_i - loads_i) / sum(target):
 *   bias_i += kp (e_i - e1_i) + ki e_i + kd (e_i - 2 e1_i + e2_i)
 *   e2 <- e1, e1 <- e        (computed in fp64, stored in fp32)
 *   loads [E] int32 (e.g. moe_zc_aux.loads), target [E] fp32 with a positive
 *   sum, bias [E] fp32 updated in place.  E in [1, MOE_ZC_MAX_EXPERTS]. */
moe_zc_status moe_zc_bias_update(const int32_t* loads, const float* target,
                                 float* bias, const moe_zc_pid* pid, int32_t E,
                                 hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* moe_zc_status_string(moe_zc_status s);

/* MOE_ZC_ABI_VERSION of the built library. */
int32_t moe_zc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ZC_H */
