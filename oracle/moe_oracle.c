/*
 * moe_oracle.c -- plain fp64 CPU oracle of one sparse MoE FFN layer forward.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline of the bench).
 * The definitions and their sources are listed in moe_oracle.h.
 *
 * Written for a reader to check by eye against the definitions: one loop per
 * sum, ascending index order, double accumulation, no blocking or fusion.
 * OpenMP only splits independent tokens (or rows) across threads; no sum is
 * split or reordered, so results do not depend on the thread count.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp -shared -fPIC
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* exact widening of one stored element to double */
static double widen(const void* base, int32_t dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_size(int32_t dtype) { return dtype == ORC_F32 ? 4u : 2u; }

static int check_layer(const orc_layer_t* L) {
  if (!L || L->H < 1 || L->F < 1 || L->E < 1 || L->k < 1 || L->k > L->E) return -1;
  if (L->dtype != ORC_F32 && L->dtype != ORC_BF16) return -1;
  if (!L->router_w || !L->experts) return -1;
  if (L->gate != ORC_GATE_SOFTMAX && L->gate != ORC_GATE_RAW) return -1;
  if (L->capacity < 0) return -1;
  const uint64_t hf = (uint64_t)L->H * (uint64_t)L->F;
  if (L->expert_format == ORC_EXPERT_U8) {
    if (L->dtype != ORC_BF16 || L->stride < 3ull * hf + sizeof(orc_u8_params_t)) return -1;
  } else if (L->expert_format != ORC_EXPERT_DTYPE || L->stride < 3ull * hf * elem_size(L->dtype)) {
    return -1;
  }
  return 0;
}

/* Weight matrix m (0 Wg, 1 Wu, 2 Wd) of an expert block: element i as a
 * double, exactly (a stored value, or (q - zero) * scale of a uint8 code). */
typedef struct {
  const unsigned char* base;
  int32_t dtype, u8;
  double scale, zero;
} orc_mat_t;

static orc_mat_t expert_matrix(const orc_layer_t* L, const unsigned char* blk, int m) {
  orc_mat_t M;
  const size_t hf = (size_t)L->H * L->F;
  M.dtype = L->dtype;
  M.u8 = L->expert_format == ORC_EXPERT_U8;
  M.scale = 1.0;
  M.zero = 0.0;
  if (M.u8) {
    orc_u8_params_t p;
    memcpy(&p, blk + 3 * hf, sizeof p);
    M.base = blk + (size_t)m * hf;
    M.scale = (double)p.scale[m];
    M.zero = (double)p.zero[m];
  } else {
    M.base = blk + (size_t)m * hf * elem_size(L->dtype);
  }
  return M;
}

/* sum_i x[i] * M[off + i], i ascending (one row of a weight matrix) */
static double row_dot(const orc_mat_t* M, size_t off, const double* x, int32_t n) {
  double s = 0.0;
  if (M->u8) {
    for (int32_t i = 0; i < n; ++i) s += x[i] * (((double)M->base[off + i] - M->zero) * M->scale);
  } else {
    for (int32_t i = 0; i < n; ++i) s += x[i] * widen(M->base, M->dtype, off + i);
  }
  return s;
}

/* Round a double to the nearest bfloat16 value (8 significant bits), ties to
 * even: v = m * 2^ex with 0.5 <= |m| < 1, so m * 2^8 carries exactly the kept
 * bits in its integer part and rint() rounds the rest half-to-even. */
double orc_bf16_round(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int ex;
  double m = frexp(v, &ex);
  return ldexp(rint(ldexp(m, 8)), ex - 8);
}

/* O1: L[t][e] = sum_h x[t][h] * Wr[h][e] (+ b[e]) */
int orc_logits(const orc_layer_t* L, const void* x, int32_t T, double* logits) {
  if (check_layer(L) || !x || T < 0 || !logits) return -1;
  const int32_t H = L->H, E = L->E;
#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int32_t h = 0; h < H; ++h)
        s += widen(x, L->dtype, (size_t)t * H + h) * widen(L->router_w, L->dtype, (size_t)h * E + e);
      if (L->router_b) s += (double)L->router_b[e];
      logits[(size_t)t * E + e] = s;
    }
  }
  return 0;
}

/* O3: the gate weights of the k picks idx[0..k-1] (pick 0 the largest). */
static void gate_weights(int32_t k, int32_t gate, const double* Lt, const int32_t* idx,
                         double* w) {
  if (gate == ORC_GATE_RAW) {
    for (int32_t j = 0; j < k; ++j) w[j] = Lt[idx[j]];
    return;
  }
  double m = Lt[idx[0]];
  double z = 0.0;
  for (int32_t j = 0; j < k; ++j) z += exp(Lt[idx[j]] - m);
  for (int32_t j = 0; j < k; ++j) w[j] = exp(Lt[idx[j]] - m) / z;
}

/* O2 + O3 for one token: k rounds of "largest unpicked logit", scanning e
 * upwards and replacing only on strictly greater, so equal logits go to the
 * lower index; then w_j = exp(L_j - L_0) / sum_i exp(L_i - L_0), or, with
 * the raw gate, w_j = L_j. */
static int topk_one(int32_t E, int32_t k, int32_t gate, const double* Lt, int32_t* idx,
                    double* w) {
  for (int32_t e = 0; e < E; ++e)
    if (!isfinite(Lt[e])) return -2;
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      int taken = 0;
      for (int32_t i = 0; i < j; ++i)
        if (idx[i] == e) taken = 1;
      if (taken) continue;
      if (best < 0 || Lt[e] > Lt[best]) best = e;
    }
    idx[j] = best;
  }
  gate_weights(k, gate, Lt, idx, w);
  return 0;
}

int orc_topk(int32_t T, int32_t E, int32_t k, int32_t gate, const double* logits,
             int32_t* idx, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E || !logits || !idx || !w) return -1;
  if (gate != ORC_GATE_SOFTMAX && gate != ORC_GATE_RAW) return -1;
  int rc = 0;
  for (int32_t t = 0; t < T; ++t) {
    int r = topk_one(E, k, gate, logits + (size_t)t * E, idx + (size_t)t * k,
                     w + (size_t)t * k);
    if (r) rc = r;
  }
  return rc;
}

int orc_topk_softmax(int32_t T, int32_t E, int32_t k, const double* logits, int32_t* idx,
                     double* w) {
  return orc_topk(T, E, k, ORC_GATE_SOFTMAX, logits, idx, w);
}

/* O4: counting sort of the T*k (token, slot) pairs by expert.  The pairs
 * of each expert are taken in order of ascending token, then ascending slot.
 * With a capacity C > 0 an expert keeps only its first C pairs, the rest are
 * dropped (reading: lowest token index kept first).  counts[e] = the pairs
 * kept; offsets = exclusive prefix sum of counts (E+1 entries); the kept
 * pairs sit at the next free position of their expert: perm[p] = t*k + j,
 * inv[t*k + j] = p; a dropped pair has inv = -1 and perm[p] = -1 for
 * offsets[E] <= p < T*k. */
int orc_dispatch_cap(int32_t T, int32_t E, int32_t k, int32_t cap, const int32_t* idx,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv) {
  if (T < 0 || E < 1 || k < 1 || cap < 0 || !idx || !counts || !offsets || !perm || !inv)
    return -1;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int32_t s = 0; s < T * k; ++s) {
    if (idx[s] < 0 || idx[s] >= E) return -1;
    if (cap == 0 || counts[idx[s]] < cap) counts[idx[s]] += 1;
  }
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!next) return -1;
  for (int32_t e = 0; e < E; ++e) next[e] = offsets[e];
  for (int32_t p = offsets[E]; p < T * k; ++p) perm[p] = -1;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      int32_t s = t * k + j;
      if (next[idx[s]] == offsets[idx[s] + 1]) {  /* the expert is full */
        inv[s] = -1;
        continue;
      }
      int32_t p = next[idx[s]]++;
      perm[p] = s;
      inv[s] = p;
    }
  }
  free(next);
  return 0;
}

int orc_dispatch(int32_t T, int32_t E, int32_t k, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv) {
  return orc_dispatch_cap(T, E, k, 0, idx, counts, offsets, perm, inv);
}

/* O5 for one row: g_f = sum_h x_h Wg[f][h], u_f = sum_h x_h Wu[f][h],
 * a_f = g_f / (1 + exp(-g_f)) * u_f (bf16-rounded in bf16 layers),
 * y_h = sum_f a_f Wd[h][f]. */
int orc_expert_ffn(const orc_layer_t* L, int32_t e, const double* xrow, double* yrow) {
  if (check_layer(L) || e < 0 || e >= L->E || !xrow || !yrow) return -1;
  const int32_t H = L->H, F = L->F;
  const unsigned char* blk = (const unsigned char*)L->experts + (size_t)e * L->stride;
  const orc_mat_t Wg = expert_matrix(L, blk, 0), Wu = expert_matrix(L, blk, 1),
                  Wd = expert_matrix(L, blk, 2);
  double* a = (double*)malloc(sizeof(double) * (size_t)F);
  if (!a) return -1;
  for (int32_t f = 0; f < F; ++f) {
    const double g = row_dot(&Wg, (size_t)f * H, xrow, H);
    const double u = row_dot(&Wu, (size_t)f * H, xrow, H);
    double act = g / (1.0 + exp(-g)) * u;
    a[f] = (L->dtype == ORC_BF16) ? orc_bf16_round(act) : act;
  }
  for (int32_t h = 0; h < H; ++h) {
    yrow[h] = row_dot(&Wd, (size_t)h * F, a, F);
  }
  free(a);
  return 0;
}

/* O5 over the dispatched rows: row p of expert e (offsets[e] <= p <
 * offsets[e+1]) is token perm[p] / k through expert e. */
int orc_expert_rows(const orc_layer_t* L, const void* x, int32_t T, const int32_t* offsets,
                    const int32_t* perm, double* yp) {
  if (check_layer(L) || !x || T < 0 || !offsets || !perm || !yp) return -1;
  const int32_t H = L->H, E = L->E, k = L->k;
  int rc = 0;
  for (int32_t e = 0; e < E; ++e) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p) {
      int32_t t = perm[p] / k;
      double* xr = (double*)malloc(sizeof(double) * (size_t)H);
      if (!xr) { rc = -1; continue; }
      for (int32_t h = 0; h < H; ++h) xr[h] = widen(x, L->dtype, (size_t)t * H + h);
      if (orc_expert_ffn(L, e, xr, yp + (size_t)p * H)) rc = -1;
      free(xr);
    }
  }
  return rc;
}

/* O6: y[t][h] = sum_{j=0}^{k-1} w[t][j] * yp[inv[t*k+j]][h], j ascending. */
int orc_combine(int32_t T, int32_t H, int32_t k, const double* w, const int32_t* inv,
                const double* yp, double* y) {
  if (T < 0 || H < 1 || k < 1 || !w || !inv || !yp || !y) return -1;
  for (int32_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h) {
      double s = 0.0;
      for (int32_t j = 0; j < k; ++j)  /* a dropped pair (inv < 0) adds nothing */
        if (inv[t * k + j] >= 0) s += w[(size_t)t * k + j] * yp[(size_t)inv[t * k + j] * H + h];
      y[(size_t)t * H + h] = s;
    }
  return 0;
}

/* O1..O6 for all T tokens.  idx [T*k], w [T*k], counts [E], offsets [E+1],
 * perm [T*k], inv [T*k] are outputs too. */
int orc_layer_forward(const orc_layer_t* L, const void* x, int32_t T, double* y, int32_t* idx,
                      double* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                      int32_t* inv) {
  if (check_layer(L) || !x || T < 0 || !y) return -1;
  const int32_t H = L->H, E = L->E, k = L->k;
  double* logits = (double*)malloc(sizeof(double) * ((size_t)T * E + 1));
  double* yp = (double*)malloc(sizeof(double) * ((size_t)T * k * H + 1));
  int rc = (!logits || !yp) ? -1 : 0;
  if (!rc) rc = orc_logits(L, x, T, logits);
  if (!rc) rc = orc_topk(T, E, k, L->gate, logits, idx, w);
  if (!rc) rc = orc_dispatch_cap(T, E, k, L->capacity, idx, counts, offsets, perm, inv);
  if (!rc) rc = orc_expert_rows(L, x, T, offsets, perm, yp);
  if (!rc) rc = orc_combine(T, H, k, w, inv, yp, y);
  free(logits);
  free(yp);
  return rc;
}

/* The layer output of selected tokens only, straight from the per-token
 * definition y[t] = sum_j w_j * FFN_{idx_j}(x[t]) (the same value that
 * O1..O6 give row t without a capacity).  keep [ntok*k] or NULL: with it,
 * only the slots with keep != 0 count (a capacity's drops, which depend on
 * the other tokens, are given by the caller).  tokens [ntok]; idx_override [ntok*k] or NULL: when
 * given, those experts (in that slot order) replace the top-k choice and the
 * weights are the gate (softmax or raw) of the oracle's logits at them.  Outputs y
 * [ntok*H], idx [ntok*k], w [ntok*k], logits [ntok*E]. */
int orc_layer_tokens(const orc_layer_t* L, const void* x, int32_t T, const int32_t* tokens,
                     int32_t ntok, const int32_t* idx_override, const int32_t* keep, double* y,
                     int32_t* idx, double* w, double* logits) {
  if (check_layer(L) || !x || T < 0 || ntok < 0 || !tokens || !y || !idx || !w || !logits)
    return -1;
  const int32_t H = L->H, E = L->E, k = L->k;
  for (int32_t n = 0; n < ntok; ++n)
    if (tokens[n] < 0 || tokens[n] >= T) return -1;
  double* xs = (double*)malloc(sizeof(double) * ((size_t)ntok * H + 1));
  double* ye = (double*)malloc(sizeof(double) * ((size_t)ntok * k * H + 1));
  if (!xs || !ye) { free(xs); free(ye); return -1; }
  int rc = 0;
  for (int32_t n = 0; n < ntok && !rc; ++n) {
    const int32_t t = tokens[n];
    double* xr = xs + (size_t)n * H;
    for (int32_t h = 0; h < H; ++h) xr[h] = widen(x, L->dtype, (size_t)t * H + h);
    double* Lt = logits + (size_t)n * E;
    for (int32_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int32_t h = 0; h < H; ++h) s += xr[h] * widen(L->router_w, L->dtype, (size_t)h * E + e);
      if (L->router_b) s += (double)L->router_b[e];
      Lt[e] = s;
    }
    int32_t* it = idx + (size_t)n * k;
    double* wt = w + (size_t)n * k;
    rc = topk_one(E, k, L->gate, Lt, it, wt);
    if (!rc && idx_override) {
      for (int32_t j = 0; j < k; ++j) {
        it[j] = idx_override[(size_t)n * k + j];
        if (it[j] < 0 || it[j] >= E) rc = -1;
      }
      if (!rc) gate_weights(k, L->gate, Lt, it, wt);
    }
  }
  if (!rc) {
    /* every (token, slot) pair through its expert; pairs are independent */
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t q = 0; q < ntok * k; ++q) {
      const int32_t n = q / k;
      if (orc_expert_ffn(L, idx[q], xs + (size_t)n * H, ye + (size_t)q * H)) rc = -1;
    }
  }
  if (!rc) {
    for (int32_t n = 0; n < ntok; ++n)
      for (int32_t h = 0; h < H; ++h) {
        double s = 0.0;
        for (int32_t j = 0; j < k; ++j)
          if (!keep || keep[(size_t)n * k + j])
            s += w[(size_t)n * k + j] * ye[((size_t)n * k + j) * H + h];
        y[(size_t)n * H + h] = s;
      }
  }
  free(xs);
  free(ye);
  return rc;
}

/* Branch input of a stacked layer: xt[t] = bf16( h[t] / sqrt(mean_h h^2 + 1e-6) ). */
int orc_prenorm_bf16(int32_t T, int32_t H, const float* h, uint16_t* xt) {
  if (T < 0 || H < 1 || !h || !xt) return -1;
  for (int32_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int32_t i = 0; i < H; ++i) ss += (double)h[(size_t)t * H + i] * (double)h[(size_t)t * H + i];
    double r = sqrt(ss / (double)H + 1e-6);
    for (int32_t i = 0; i < H; ++i) {
      float f = (float)orc_bf16_round((double)h[(size_t)t * H + i] / r);
      uint32_t bits;
      memcpy(&bits, &f, sizeof bits);
      xt[(size_t)t * H + i] = (uint16_t)(bits >> 16);
    }
  }
  return 0;
}

/* Affine uint8 quantisation of one weight matrix from its range, as the
 * pages convert expert weights after training: per-matrix minimum and
 * maximum, 255 levels (www.pnsm.cn/news/1892388.html sec. 3.1), read back as
 * (q - zero) * scale with an integer zero point (same page, sec. 5.2).
 * Readings: the range is widened to include 0 so that the zero point is a
 * code in [0, 255] and 0 is exact; codes are unsigned bytes; every step is
 * fp32 arithmetic (IEEE, round to nearest even), written out in order. */
int orc_quantize_u8(const uint16_t* w, size_t n, uint8_t* q, orc_u8_params_t* p, int32_t m) {
  if (!w || !q || !p || m < 0 || m > 2) return -1;
  float mn = 0.0f, mx = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    const float v = (float)widen(w, ORC_BF16, i);
    if (!isfinite(v)) return -1;
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  float scale = (mx - mn) / 255.0f;
  if (!(scale > 0.0f)) scale = 1.0f;
  int32_t zero = (int32_t)rintf(-mn / scale);
  if (zero < 0) zero = 0;
  if (zero > 255) zero = 255;
  for (size_t i = 0; i < n; ++i) {
    const float v = (float)widen(w, ORC_BF16, i);
    int32_t c = (int32_t)rintf(v / scale) + zero;
    if (c < 0) c = 0;
    if (c > 255) c = 255;
    q[i] = (uint8_t)c;
  }
  p->scale[m] = scale;
  p->zero[m] = zero;
  p->min[m] = mn;
  p->max[m] = mx;
  return 0;
}

int orc_quantize_experts_u8(const void* src, uint64_t src_stride, int32_t E, int32_t H,
                            int32_t F, void* dst, uint64_t dst_stride) {
  if (!src || !dst || E < 1 || H < 1 || F < 1) return -1;
  const size_t hf = (size_t)H * F;
  if (src_stride < 3 * hf * 2 || dst_stride < 3 * hf + sizeof(orc_u8_params_t)) return -1;
  for (int32_t e = 0; e < E; ++e) {
    const unsigned char* sb = (const unsigned char*)src + (size_t)e * src_stride;
    unsigned char* db = (unsigned char*)dst + (size_t)e * dst_stride;
    orc_u8_params_t p;
    memset(&p, 0, sizeof p);
    for (int32_t m = 0; m < 3; ++m)
      if (orc_quantize_u8((const uint16_t*)(sb + (size_t)m * hf * 2), hf, db + (size_t)m * hf, &p, m))
        return -1;
    memcpy(db + 3 * hf, &p, sizeof p);
  }
  return 0;
}
