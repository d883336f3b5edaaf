/*
 * moe_oracle.h -- plain, slow fp64 CPU oracle of one sparse MoE FFN layer's
 * forward pass.  TEST INFRASTRUCTURE: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * What it computes, and where the pages define it (pages named by address):
 *   logits   L[t][e] = sum_h x[t][h] * Wr[h][e] (+ b[e])
 *              router as one linear layer of shape (hidden, experts):
 *              zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析"
 *              sec. 3.1 (router weight matrix) and m.nxbn.cn/news/47896 sec. 3.2
 *              (logits from a matrix-vector product); the bias only for the
 *              skewed 128-expert workload, added before selection.
 *   top-k    the k largest logits per token, ties to the lower expert index,
 *            then a softmax over the k selected logits: www.lmnt.cn/news/246575
 *            sec. 2.2 (route_tokens: logits, top-k, in-place softmax).
 *            Gate variant ORC_GATE_RAW: the same selection, and the weights
 *            are the selected raw logits themselves, no softmax (the default
 *            router of m.nxbn.cn/news/47896 sec. 3.2 and of
 *            www.pnsm.cn/news/1892388.html sec. 3.3).
 *   dispatch the (token, slot) pairs grouped by expert into one batch per
 *            expert: zskr.cn page sec. 3.3, stage 3.  Optional expert
 *            capacity C: an expert takes at most C pairs per call, the rest
 *            are dropped (www.cf-1.com/news/4750020/ sec. 4.2,
 *            --expert-capacity; zskr.cn page sec. 2.2, hard_capacity);
 *            reading: the pairs of lowest token index (then slot) are kept,
 *            a dropped pair adds nothing, the other weights are unchanged.
 *   expert   SwiGLU without bias, gate/up of shape (intermediate, hidden),
 *            down of shape (hidden, intermediate): zskr.cn page sec. 3.1 and
 *            sec. 3.3 stage 4 (gate_proj, up_proj, SiLU, down_proj).
 *   combine  sum over the k slots of the gate weight times the expert output:
 *            zskr.cn page sec. 2.2 and sec. 3.3 stage 5; www.pnsm.cn page
 *            sec. 2.2 (weighted fusion).
 *   stack    residual inside the forward call: www.pnsm.cn/news/1892388.html
 *            sec. 2.1; with a parameter-free RMS normalisation of the branch
 *            input (a reading: the literal residual stack overflows).
 *   uint8    expert weights quantised after training, one affine map per
 *   experts  weight matrix from its minimum and maximum, 255 levels, read as
 *            w = (q - zero) * scale: www.pnsm.cn page sec. 3.1 (per-expert
 *            min/max quantisation) and sec. 5.2 (dequantisation with an
 *            integer zero point); the layer is then the same method on the
 *            dequantised weights.
 *
 * Storage (all row-major):
 *   x        [T][H]   dtype          Wr  [H][E] dtype       b [E] fp32
 *   expert e at byte offset e*stride of `experts`:
 *            Wg [F][H], Wu [F][H], Wd [H][F]   dtype
 *   dtype ORC_F32: float; ORC_BF16: bfloat16 bit patterns (uint16).
 *   expert_format ORC_EXPERT_U8 (bf16 layers): the three matrices as uint8
 *            codes, then at byte 3*H*F an orc_u8_params_t block.
 * Every stored value is widened exactly to double; all sums are in double,
 * in ascending index order.  In bf16 layers the SwiGLU activation is rounded
 * to bf16 (round to nearest even) before the down projection, because the
 * method stores that activation in bf16.
 *
 * Return codes: 0 ok, -1 invalid argument, -2 non-finite logit.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_GATE_SOFTMAX = 0, ORC_GATE_RAW = 1 };
enum { ORC_EXPERT_DTYPE = 0, ORC_EXPERT_U8 = 1 };

/* per-expert quantisation parameters, matrix m = 0 (Wg), 1 (Wu), 2 (Wd) */
typedef struct {
  float scale[3];
  int32_t zero[3];
  float min[3], max[3]; /* the range the map was made from (includes 0) */
  uint32_t pad[4];
} orc_u8_params_t;      /* 64 bytes */

typedef struct {
  int32_t H, F, E, k;
  int32_t dtype;
  const void* router_w;
  const float* router_b;
  const void* experts;
  uint64_t stride;
  int32_t gate;      /* ORC_GATE_SOFTMAX or ORC_GATE_RAW */
  int32_t capacity;  /* pairs an expert takes per call; 0 = no limit */
  int32_t expert_format; /* ORC_EXPERT_DTYPE or ORC_EXPERT_U8 */
} orc_layer_t;

int orc_logits(const orc_layer_t* L, const void* x, int32_t T, double* logits);
int orc_topk_softmax(int32_t T, int32_t E, int32_t k, const double* logits, int32_t* idx,
                     double* w);
/* the same selection with gate ORC_GATE_SOFTMAX or ORC_GATE_RAW */
int orc_topk(int32_t T, int32_t E, int32_t k, int32_t gate, const double* logits,
             int32_t* idx, double* w);
int orc_dispatch(int32_t T, int32_t E, int32_t k, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv);
/* the same with capacity cap (0 = none): dropped pairs get inv = -1 */
int orc_dispatch_cap(int32_t T, int32_t E, int32_t k, int32_t cap, const int32_t* idx,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv);
int orc_expert_ffn(const orc_layer_t* L, int32_t e, const double* xrow, double* yrow);
int orc_expert_rows(const orc_layer_t* L, const void* x, int32_t T, const int32_t* offsets,
                    const int32_t* perm, double* yp);
int orc_combine(int32_t T, int32_t H, int32_t k, const double* w, const int32_t* inv,
                const double* yp, double* y);
int orc_layer_forward(const orc_layer_t* L, const void* x, int32_t T, double* y, int32_t* idx,
                      double* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                      int32_t* inv);
int orc_layer_tokens(const orc_layer_t* L, const void* x, int32_t T, const int32_t* tokens,
                     int32_t ntok, const int32_t* idx_override, const int32_t* keep, double* y,
                     int32_t* idx, double* w, double* logits);
int orc_prenorm_bf16(int32_t T, int32_t H, const float* h, uint16_t* xt);
/* uint8 quantisation of n bf16 weights (one matrix), in fp32 arithmetic:
 * mn = min(0, min w), mx = max(0, max w), scale = (mx - mn) / 255 (1 if 0),
 * zero = clamp(rint(-mn / scale), 0, 255),
 * q = clamp(rint(w / scale) + zero, 0, 255); rint rounds half to even. */
int orc_quantize_u8(const uint16_t* w, size_t n, uint8_t* q, orc_u8_params_t* p, int32_t m);
/* every matrix of E bf16 experts (stride src_stride bytes) into uint8
 * experts with their parameter blocks (stride dst_stride >= 3*H*F + 64) */
int orc_quantize_experts_u8(const void* src, uint64_t src_stride, int32_t E, int32_t H,
                            int32_t F, void* dst, uint64_t dst_stride);
double orc_bf16_round(double v);
int orc_num_threads(void);
/* Threads of later OpenMP regions (timing only; results do not depend on it). */
void orc_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
