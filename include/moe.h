/*
 * moe.h -- C ABI of libmoe: one sparse Mixture-of-Experts FFN layer's forward
 * pass on one AMD Instinct MI355X (gfx950), all steps in HIP kernels.
 *
 * The layer (pages cited by address and section):
 *   1. router logits  L = x . Wr (+ b), Wr of shape (hidden, experts)
 *      [zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析"
 *      sec. 3.1; m.nxbn.cn/news/47896 sec. 3.2]
 *   2. per token the top_k largest logits (ties to the lower expert index),
 *      then a softmax over those k logits [www.lmnt.cn/news/246575 sec. 2.2,
 *      route_tokens steps 1-3]
 *   3. dispatch: the (token, slot) pairs grouped into one batch per expert
 *      [zskr.cn page sec. 3.3, stage 3]
 *   4. per-expert SwiGLU FFN without bias: gate_proj and up_proj, SiLU, then
 *      down_proj [zskr.cn page sec. 3.1 and sec. 3.3, stage 4]
 *   5. combine: y[t] = sum_j w[t][j] * FFN_{idx[t][j]}(x[t]), slots in
 *      ascending order, no atomics [zskr.cn page sec. 3.3, stage 5;
 *      www.pnsm.cn/news/1892388.html sec. 2.2]
 *   Optional: y = h + MoE(rmsnorm(h)), the residual taken inside the forward
 *   call [www.pnsm.cn page sec. 2.1], with a parameter-free RMS normalisation
 *   of the branch input (MOE_FLAG_RESIDUAL_PRENORM).
 *
 * Life cycle init / forward / free with caller-owned buffers follows the
 * pages' C API [zskr.cn page sec. 4.2; www.pnsm.cn page sec. 2.1 and 4.4].
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (hipMalloc or equivalent) on
 *     the device that was current when the layer was created, 16-byte aligned.
 *     They are borrowed: the caller owns them and keeps the weights alive
 *     until moe_layer_free.  The layer owns only its workspace, allocated
 *     once by moe_layer_create for max_tokens; no call allocates afterwards.
 *   - Matrices are row-major.  dtype MOE_BF16 means bfloat16 (stored as 16-bit
 *     patterns), MOE_F32 means IEEE float.
 *   - Calls validate their arguments synchronously and return MOE_OK or a
 *     negative MOE_ERR_* code without launching anything on error.  Work is
 *     queued on `stream` (a hipStream_t; NULL = the null stream) and runs
 *     asynchronously; a launch failure returns MOE_ERR_DEVICE.
 *   - One call in flight per layer (calls share the layer's workspace):
 *     create one layer per concurrent stream.  Results are bitwise
 *     reproducible for identical inputs (no floating-point atomics).
 *   - bf16 batches of up to 64 tokens route and dispatch in one launch whose
 *     workgroups count their completion in a counter in the workspace (for
 *     moe_forward_noalloc, in its device array); every launch that runs to
 *     completion leaves it at zero.  A launch that does not complete (a
 *     device fault) leaves it wrong and later small-batch calls on that
 *     workspace would skip their dispatch; as the device context has to be
 *     re-created after a fault anyway, create the layer anew with it.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer moe_layer_t; /* opaque */

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment or descriptor field */
  MOE_ERR_NO_MEMORY = -2,   /* workspace allocation failed */
  MOE_ERR_DEVICE = -3,      /* a HIP call or kernel launch failed */
  MOE_ERR_UNSUPPORTED = -4  /* valid, but outside what the kernels implement */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage of the expert weights (moe_layer_desc.expert_format). */
enum {
  MOE_EXPERT_DTYPE = 0, /* in the layer's dtype */
  /* uint8 codes with one affine map per weight matrix, weight = (q - zero) *
   * scale: post-training quantisation of each expert matrix from its range,
   * 255 levels, integer zero point [www.pnsm.cn/news/1892388.html sec. 3.1
   * and sec. 5.2].  Expert e at expert_base + e*expert_stride holds
   *   Wg [F][H], Wu [F][H], Wd [H][F]   uint8 (same orientation as above)
   *   at byte 3*H*F: moe_u8_params (64 bytes)
   * and expert_stride >= 3*H*F + 64 (a multiple of 256).  bf16 layers only;
   * x and the router stay bf16.  The expert FFN runs on the weight-streaming
   * kernels for every batch size (MOE_FLAG_PATH_GROUPED is unsupported),
   * which read one byte per weight and take their token operands in fp16:
   * the layer input is converted once from bf16 to fp16, and the SwiGLU
   * activation is rounded to bf16 and then stored as fp16, both conversions
   * rounding toward zero.  For magnitudes in fp16's normal range
   * [2^-14, 65504] they are exact (such bf16 values are fp16 values);
   * smaller magnitudes keep an absolute error below 2^-24 (fp16 subnormals)
   * and larger ones saturate to +-65504. */
  MOE_EXPERT_U8 = 1
};

/* Parameters of a uint8 expert, matrix m = 0 (Wg), 1 (Wu), 2 (Wd). */
typedef struct {
  float scale[3];
  int32_t zero[3];      /* 0..255 */
  float min[3], max[3]; /* the range the map was made from; it includes 0 */
  uint32_t pad[4];
} moe_u8_params;

enum {
  /* Stacked-layer mode: x is the fp32 residual stream h [T][H]; the branch
   * input is bf16(h[t] / sqrt(mean_h h[t]^2 + 1e-6)) and y = h + MoE(.).
   * y may alias x.  bf16 layers with H <= 16384 only. */
  MOE_FLAG_RESIDUAL_PRENORM = 1u << 0,
  /* Kernel path for the expert FFN of bf16 layers.  By default a call with
   * T*k <= 32*E (few rows per expert: decode batches, many small experts)
   * streams each non-empty expert's weights once; otherwise the rows go
   * through grouped GEMMs on 256x256 tiles.  A call with T == 1 whose widths
   * suit it (H*w and F*w multiples of 1024 bytes, w the bytes per weight,
   * with H*w/1024 in {2, 4, 6, 8}, F*w/1024 a multiple of 4 or 14, k <= 8 and
   * k*F <= 40832) takes matrix-vector kernels instead, the combine folded
   * into the down projection.  These flags pin one path (results agree
   * within rounding; all are deterministic); MOE_FLAG_PATH_STREAM also keeps
   * single tokens on the streaming kernels. */
  MOE_FLAG_PATH_GROUPED = 1u << 1,
  MOE_FLAG_PATH_STREAM = 1u << 2,
  /* Gate variant: the same top-k selection, and the gate weights are the k
   * selected logits themselves (fp32, no softmax) -- the default router of
   * m.nxbn.cn/news/47896 sec. 3.2 and www.pnsm.cn/news/1892388.html sec. 3.3.
   * Without it the weights are the softmax over the k selected logits.
   * (Soft routing, every expert weighted, is top_k == num_experts with the
   * softmax gate.) */
  MOE_FLAG_GATE_RAW = 1u << 3,
  /* On the streaming path the down projection folds step 5 in when one
   * workgroup can own every expert's rows of a hidden slice (H/16 slices at
   * least as many as compute units, T*k <= 256), and the single-token
   * matrix-vector path always does: it sums the k expert rows of each token
   * in the same fixed slot order with the same fp32 operations as the
   * separate combine, so the results are bit-identical.  This flag keeps the
   * combine a kernel of its own (for profiling and testing). */
  MOE_FLAG_COMBINE_SEPARATE = 1u << 4
};

typedef struct {
  uint32_t struct_size;   /* sizeof(moe_layer_desc) */
  int32_t hidden;         /* H: model width */
  int32_t ffn;            /* F: expert FFN width */
  int32_t num_experts;    /* E: 1..256 */
  int32_t top_k;          /* k: 1..E (k = E: soft routing, every expert
                             weighted by the softmax of all logits) */
  int32_t max_tokens;     /* largest T any call will pass: 1..65536 */
  int32_t dtype;          /* moe_dtype of x, router_w, the experts and the
                             stored SwiGLU activation */
  uint32_t flags;         /* MOE_FLAG_* */
  const void* router_w;   /* [H][E] dtype: element (h, e) at h*E + e */
  const float* router_b;  /* [E] fp32 added to the logits, or NULL */
  const void* expert_base;/* expert e starts at expert_base + e*expert_stride
                             bytes and holds, contiguously,
                               Wg [F][H]  gate_proj (row f = output unit f)
                               Wu [F][H]  up_proj
                               Wd [H][F]  down_proj
                             so g_f = sum_h x_h Wg[f][h] and
                             y_h = sum_f a_f Wd[h][f].  This output-major
                             orientation is that of the pages' weight format
                             (gate/up stored (intermediate, hidden), down
                             (hidden, intermediate) [zskr.cn page sec. 3.1]),
                             chosen deliberately over input-major
                             [Wg H x F][Wu H x F][Wd F x H]: both GEMMs then
                             read K-contiguous rows.  A caller holding
                             input-major matrices transposes them once. */
  uint64_t expert_stride; /* bytes, >= 3*H*F*sizeof(dtype), multiple of 256 */
  int32_t expert_capacity;/* (token, slot) pairs an expert takes per call, 0 = no
                             limit.  Pairs beyond it are dropped: the pairs of
                             each expert are taken in ascending token (then
                             slot) order and the first expert_capacity kept; a
                             dropped pair adds nothing to its token's output and
                             the other gate weights are unchanged (the pages'
                             hard_capacity, www.cf-1.com/news/4750020/ sec. 4.2
                             --expert-capacity; zskr.cn page sec. 2.2).  A soft
                             capacity is a larger value of this limit. */
  int32_t expert_format;  /* MOE_EXPERT_DTYPE or MOE_EXPERT_U8 */
} moe_layer_desc;

/* Validates *d, allocates the workspace for d->max_tokens on the current
 * device and returns the layer, or NULL with *status (if non-NULL) set to the
 * error.  Shape limits of the kernels (else MOE_ERR_UNSUPPORTED): bf16 layers
 * need H % 256 == 0 and F % 128 == 0; fp32 layers H % 4 == 0 and F % 4 == 0;
 * E <= 256; max_tokens*k*max(H, F), max_tokens*H and 3*H*F below 2^31.
 * (k > 8 selects by ranks; bf16 batches of up to 64 tokens then route and
 * dispatch in separate launches.)  Nothing is launched. */
moe_layer_t* moe_layer_create(const moe_layer_desc* d, int* status);

/* Steps 1-3 only, with their results copied out (for inspection and tests).
 *   x          [T][H] dtype (fp32 h in RESIDUAL_PRENORM mode), 1 <= T <= max_tokens
 *   logits_in  [T][E] fp32 or NULL: when given, step 1 is skipped and these
 *              logits are used as they are
 *   topk_idx   [T][k] int32 out: expert of slot j of token t, slots ordered by
 *              descending logit, equal logits by ascending expert index
 *   topk_w     [T][k] fp32 out: softmax of the selected logits (the logits
 *              themselves with MOE_FLAG_GATE_RAW)
 *   counts     [E] int32 out or NULL: pairs each expert takes (routed, capped
 *              at expert_capacity)
 *   offsets    [E+1] int32 out or NULL: exclusive prefix sum of counts
 *   perm       [T*k] int32 out or NULL: perm[p] = t*k + j of the p-th pair in
 *              (expert, token) order, p < offsets[E]; -1 beyond
 *   inv        [T*k] int32 out or NULL: inv[t*k + j] = p, the inverse of perm,
 *              or -1 for a pair dropped by the capacity */
int moe_route(moe_layer_t* L, const void* x, int32_t T, const float* logits_in,
              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* perm, int32_t* inv, void* stream);

/* The whole layer, steps 1-5.
 *   x  [T][H] dtype; fp32 h in RESIDUAL_PRENORM mode
 *   y  [T][H] fp32 out; may alias x only in RESIDUAL_PRENORM mode
 * T in 1..max_tokens. */
int moe_forward(moe_layer_t* L, const void* x, int32_t T, float* y, void* stream);

/* moe_forward with per-stage timing events.  stage_events is NULL (same as
 * moe_forward) or an array of MOE_NUM_STAGES + 1 hipEvent_t created by the
 * caller; event i is recorded on `stream` right before stage i is enqueued
 * and event MOE_NUM_STAGES after the last stage, so hipEventElapsedTime
 * between events i and i+1 is the device time of stage i:
 *   MOE_STAGE_ROUTE    (branch normalisation,) router logits, top-k, softmax
 *   MOE_STAGE_DISPATCH histogram, scan, scatter
 *   MOE_STAGE_GATE_UP  gate/up projections + SiLU (one kernel)
 *   MOE_STAGE_DOWN     down projection (one kernel)
 *   MOE_STAGE_COMBINE  weighted combine (+ residual) (one kernel)
 * For bf16 layers with T <= 64 routing and dispatch run as one kernel inside
 * MOE_STAGE_ROUTE, and MOE_STAGE_DISPATCH is empty (its two events are
 * recorded back to back; their distance is event overhead only). */
enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_DISPATCH = 1,
  MOE_STAGE_GATE_UP = 2,
  MOE_STAGE_DOWN = 3,
  MOE_STAGE_COMBINE = 4,
  MOE_NUM_STAGES = 5
};
int moe_forward_ev(moe_layer_t* L, const void* x, int32_t T, float* y, void* stream,
                   void* const* stage_events);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * forward as moe_forward (steps 1-5, the same kernels) without a layer
 * handle: *d describes the layer (its pointers are borrowed for the call,
 * max_tokens bounds T), and the call's workspace is carved, for this T, from
 * a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends.  Nothing is allocated.
 *   - The first call on a device also queues, on `stream`, a one-time clear
 *     of a completion counter in that array (every later launch leaves it at
 *     zero).
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind: calls that overlap on one GPU (any stream, any thread) race,
 *     so the caller serialises them.
 *   - Results equal moe_forward's bit for bit, except on calls that run the
 *     grouped GEMMs (T*k > 32*E, or MOE_FLAG_PATH_GROUPED): there the down
 *     projection does not split its last round of tiles along K (that needs
 *     64 MB of partial sums), so the sums are added in another order
 *     (deterministic, within rounding of moe_forward).
 * Errors: those of moe_layer_create's validation of *d and of moe_forward's
 * arguments; MOE_ERR_UNSUPPORTED when the workspace of this call does not
 * fit the array (8 experts of H=4096, F=14336, k=2: up to about 540
 * tokens); nothing is launched on an error. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_layer_desc* d, const void* x, int32_t T, float* y,
                        void* stream);

/* Quantises E bf16 experts (src: expert e at src + e*src_stride bytes, laid
 * out as in moe_layer_desc) into uint8 experts for MOE_EXPERT_U8 (dst, e at
 * dst + e*dst_stride).  Per matrix, in fp32 arithmetic with IEEE division
 * and rint (ties to even):
 *   mn = min(0, min w), mx = max(0, max w), scale = (mx - mn) / 255 (1 if 0),
 *   zero = clamp(rint(-mn / scale), 0, 255),
 *   q = clamp(rint(w / scale) + zero, 0, 255).
 * Both buffers are device memory, 16-byte aligned; src_stride >= 6*H*F,
 * dst_stride >= 3*H*F + 64, both multiples of 256; H % 16 == 0 and F % 16
 * == 0; 3*H*F < 2^31.  Queued on `stream`; allocates nothing (the parameter
 * blocks of dst serve as scratch).  Errors: MOE_ERR_INVALID_ARG, or
 * MOE_ERR_DEVICE on a launch failure.  Non-finite weights give unspecified
 * codes. */
int moe_quantize_experts_u8(const void* src, uint64_t src_stride, int32_t E, int32_t H,
                            int32_t F, void* dst, uint64_t dst_stride, void* stream);

/* Releases the workspace (after synchronising the device).  NULL-safe. */
void moe_layer_free(moe_layer_t* L);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
