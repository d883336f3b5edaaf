// router.hip -- steps 1 and 2 of the layer: router logits, top-k, softmax.
//
// Logits L = x . Wr with Wr of shape (hidden, experts) [zskr.cn/news/2275853
// "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1; m.nxbn.cn/news/47896
// sec. 3.2], optional per-expert bias; then per token the k largest logits
// (equal logits: lower expert index first) and a softmax over those k
// [www.lmnt.cn/news/246575 sec. 2.2, route_tokens].
//
// bf16 layers, batches beyond 64 tokens: a first kernel computes partial
// logits of 64-token tiles over slices of the hidden dimension (split so
// that the batch fills hundreds of workgroups) with v_mfma_f32_16x16x32_bf16
// (tokens as the A operand, the router as the B operand, staged in LDS
// chunk by chunk: up to 64 experts transposed on the way from its [H][E]
// layout, beyond that from a copy transposed by a kernel of its own; fp32
// accumulation; the next hidden step's operands loaded during this one's
// MFMAs); a second kernel adds the slices in a fixed order
// (+ bias) and selects with a DPP max-reduction over (value desc, index asc):
// one token per 16-lane row, each lane holding up to 16 experts' sums in
// registers (k beyond 8: one token per wave, ranks).  Batches of up to 64 tokens route and dispatch in one launch (the
// one-workgroup kernels below).  fp32 layers use one plain-FMA kernel.  The
// softmax over the k picks is evaluated in fp64.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int RT_TOK = 64;  // tokens per workgroup
constexpr int RT_HC = 64;   // hidden chunk staged per step
constexpr int RT_PAD = 8;   // bf16 padding of a staged router row
constexpr int RT_MAX_SPLITS = 16;

struct Cand {
  float v;
  int e;  // INT32_MAX = no candidate
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  // a is a candidate and either b is none or a beats it: larger value, or the
  // same value and the lower index (bitwise operators: no branches)
  return (a.e != INT32_MAX) &
         ((b.e == INT32_MAX) | (a.v > b.v) | ((a.v == b.v) & (a.e < b.e)));
}

// The best candidate of the wave, in every lane: row-local steps (DPP
// row_shr 1, 2, 4, 8 leave each row's best in its lane 15), then rows 0-1 and
// 2-3 (row_bcast 15), then all four (row_bcast 31) into lane 63, read back as
// a uniform value.  A lane whose DPP source lies outside its row, or whose row
// is masked off, keeps its own candidate.  "better" is a total order on the
// candidates, so the result does not depend on the reduction's shape.
__device__ __forceinline__ Cand dpp_best_step(Cand c, Cand o) { return better(o, c) ? o : c; }
#define DPP_CAND(c, ctrl, rmask)                                                                  \
  Cand{__int_as_float(__builtin_amdgcn_update_dpp(__float_as_int((c).v), __float_as_int((c).v), \
                                                  ctrl, rmask, 0xF, false)),                    \
       __builtin_amdgcn_update_dpp((c).e, (c).e, ctrl, rmask, 0xF, false)}
__device__ __forceinline__ Cand wave_best(Cand c) {
  c = dpp_best_step(c, DPP_CAND(c, 0x111, 0xF));  // row_shr:1
  c = dpp_best_step(c, DPP_CAND(c, 0x112, 0xF));  // row_shr:2
  c = dpp_best_step(c, DPP_CAND(c, 0x114, 0xF));  // row_shr:4
  c = dpp_best_step(c, DPP_CAND(c, 0x118, 0xF));  // row_shr:8
  c = dpp_best_step(c, DPP_CAND(c, 0x142, 0xA));  // row_bcast:15 into rows 1, 3
  c = dpp_best_step(c, DPP_CAND(c, 0x143, 0xC));  // row_bcast:31 into rows 2, 3
  return Cand{__int_as_float(__builtin_amdgcn_readlane(__float_as_int(c.v), 63)),
              __builtin_amdgcn_readlane(c.e, 63)};
}
#undef DPP_CAND

// DPP move of a 32-bit value; lanes without a source (row_shr past the row's
// start) read 0.  CTRL: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// The best candidate of each 16-lane row, in every lane of the row: rotations
// by 8, 4, 2 and 1 within the row ("better" is a total order, so the shape
// of the reduction does not matter).
__device__ __forceinline__ Cand row_best16(Cand c) {
#define ROW_STEP(ctrl) \
  c = dpp_best_step(c, Cand{__int_as_float(dpp_i<ctrl>(__float_as_int(c.v))), dpp_i<ctrl>(c.e)})
  ROW_STEP(0x128);
  ROW_STEP(0x124);
  ROW_STEP(0x122);
  ROW_STEP(0x121);
#undef ROW_STEP
  return c;
}
// Inclusive prefix sum of an integer over the 64 lanes: row-local steps
// (row_shr 1, 2, 4, 8), then the rows' totals carried by row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Top-k of one token by ranks, for k > MOE_MAX_TOPK (up to every expert:
// soft routing): the rank of expert e is the number of experts that beat it
// ((value desc, index asc), the same total order as the picks below), the k
// best take the slots 0..k-1 by rank, and the softmax adds the exponentials
// in slot order (lane 0, from ex_lds: [k] doubles of this wave).
__device__ __forceinline__ void topk_rank_row(const float* row, int t, int E, int k, int raw, int32_t* idx_out,
                              float* w_out, double* ex_lds) {
  const int lane = threadIdx.x & 63;
  float v[4];
  int rnk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    v[c] = (e < E) ? row[e] : 0.0f;
    rnk[c] = 0;
  }
  for (int e2 = 0; e2 < E; ++e2) {
    const float v2 = row[e2];
#pragma unroll
    for (int c = 0; c < 4; ++c) rnk[c] += (v2 > v[c]) | ((v2 == v[c]) & (e2 < lane + 64 * c));
  }
  // the largest logit (the pick of slot 0), for the softmax
  float m = v[0];
#pragma unroll
  for (int c = 1; c < 4; ++c)
    if (lane + 64 * c < E) m = fmaxf(m, v[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    if (e < E && rnk[c] < k) {
      idx_out[(size_t)t * k + rnk[c]] = e;
      if (!raw) ex_lds[rnk[c]] = exp((double)v[c] - (double)m);
    }
  }
  if (raw) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c < E && rnk[c] < k) w_out[(size_t)t * k + rnk[c]] = v[c];
    return;
  }
  __builtin_amdgcn_wave_barrier();
  double z = 0.0;
  if (lane == 0)
    for (int j = 0; j < k; ++j) z += ex_lds[j];
  z = __shfl(z, 0);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    if (lane + 64 * c < E && rnk[c] < k) w_out[(size_t)t * k + rnk[c]] = (float)(ex_lds[rnk[c]] / z);
  __builtin_amdgcn_wave_barrier();  // ex_lds is free for this wave's next token
}

// Top-k + softmax of tokens tile0 + wave, tile0 + wave + nwaves, ... below
// tile0 + rows (interleaved so that small batches still spread over the
// waves).  lg: LDS logits [rows][ldl].  idx_lds (optional): an LDS copy of the
// picks of the tile, [RT_TOK][k].  k > MOE_MAX_TOPK takes topk_rank_row with
// ex_lds: [nwaves][MOE_MAX_EXPERTS] doubles of LDS (required then).
__device__ __forceinline__ void topk_rows(const float* lg, int ldl, int tile0, int T, int E, int k, int raw,
                          int32_t* idx_out, float* w_out, int nwaves = 4,
                          int32_t* idx_lds = nullptr, int rows = RT_TOK,
                          double* ex_lds = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (k > MOE_MAX_TOPK) {
    for (int r = wave; r < rows; r += nwaves) {
      const int t = tile0 + r;
      if (t >= T) break;
      topk_rank_row(lg + (size_t)r * ldl, t, E, k, raw, idx_out, w_out,
                    ex_lds + wave * MOE_MAX_EXPERTS);
    }
    return;
  }
  for (int r = wave; r < rows; r += nwaves) {
    const int t = tile0 + r;
    if (t >= T) break;
    const float* row = lg + (size_t)r * ldl;
    float v[4];
    uint32_t avail = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int e = lane + 64 * c;
      v[c] = (e < E) ? row[e] : 0.0f;
      if (e < E) avail |= 1u << c;
    }
    float sel_v[8];
    int sel_e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sel_v[j] = 0.0f;
      sel_e[j] = 0;
      if (j >= k) continue;
      Cand best{0.0f, INT32_MAX};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Cand cand{v[c], (avail >> c & 1u) ? lane + 64 * c : INT32_MAX};
        if (better(cand, best)) best = cand;
      }
      best = wave_best(best);
      sel_v[j] = best.v;
      sel_e[j] = best.e;
      if ((best.e & 63) == lane) avail &= ~(1u << (best.e >> 6));
    }
    // softmax over the k selected logits, in double (raw gate: the logits):
    // lane j < k evaluates pick j's exponential, z adds them in pick order
    const double m = (double)sel_v[0];
    float vj = sel_v[0];
    int ej = sel_e[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (j < k && j == lane) {
        vj = sel_v[j];
        ej = sel_e[j];
      }
    const double num = (!raw && lane < k) ? exp((double)vj - m) : 0.0;
    double z = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) z += __shfl(num, j);
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = ej;
      w_out[(size_t)t * k + lane] = raw ? vj : (float)(num / z);
      if (idx_lds) idx_lds[r * k + lane] = ej;
    }
  }
}

// Top-k + softmax (raw gate: the selected logits) for E <= 16: each 16-lane
// group (a DPP row) of a wave takes one token (lane = expert), so a wave
// handles 4 tokens at once: tokens tile0 + 4 (wave + nwaves j) + g,
// g = lane / 16.  Each pick is the row's best by DPP rotations; same ordering
// (value desc, index asc) and fp64 softmax as topk_rows; lane j of the group
// evaluates the exponential of pick j.
__device__ __forceinline__ void topk_rows16(const float* lg, int ldl, int tile0, int T, int E, int k, int raw,
                            int32_t* idx_out, float* w_out, int nwaves, int32_t* idx_lds,
                            int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, el = lane & 15;
  for (int r0 = wave * 4; r0 < rows; r0 += nwaves * 4) {
    const int r = r0 + g;
    const int t = tile0 + r;
    const bool ok = r < rows && t < T;
    const float v = (ok && el < E) ? lg[(size_t)r * ldl + el] : 0.0f;
    bool avail = ok && el < E;
    float my_v = 0.0f, m = 0.0f;
    int my_e = 0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j >= k) break;
      const Cand best = row_best16(Cand{v, avail ? el : INT32_MAX});
      if (best.e == el) avail = false;
      if (el == j) {
        my_v = best.v;
        my_e = best.e;
      }
      if (j == 0) m = best.v;  // the maximum, for the softmax
    }
    // softmax over the picks (lane j < k holds pick j): z adds the
    // exponentials in pick order, as topk_rows does, so that every route
    // kernel gives the same weights bit for bit -- a running sum passed along
    // the row (lane j adds its term to lane j-1's sum), then lane k-1's total
    // sent to the whole row by adding it to zeros (exact)
    const double ex = (el < k && !raw) ? exp((double)my_v - (double)m) : 0.0;
    double s = ex;
#pragma unroll
    for (int j = 1; j < MOE_MAX_TOPK; ++j) {
      if (j >= k) break;
      const double prev = dpp_d<0x111>(s);  // row_shr:1
      if (el == j) s = prev + s;
    }
    double z = (el == k - 1) ? s : 0.0;
    z += dpp_d<0x128>(z);
    z += dpp_d<0x124>(z);
    z += dpp_d<0x122>(z);
    z += dpp_d<0x121>(z);
    if (ok && el < k) {
      idx_out[(size_t)t * k + el] = my_e;
      w_out[(size_t)t * k + el] = raw ? my_v : (float)(ex / z);
      if (idx_lds) idx_lds[r * k + el] = my_e;
    }
  }
}

// The same top-k + softmax (k <= MOE_MAX_TOPK) for one token per 16-lane row
// with C candidates per lane already in registers: lane el of the row holds
// the logits of experts el, el + 16, ..., el + 16 (C - 1) (avail: which of
// them exist).  Each pick is the lane's best candidate, then the row's best
// by DPP rotations (the same total order, so the same picks as topk_rows);
// the softmax as in topk_rows16.  Token t is written when ok.
template <int C>
__device__ __forceinline__ void topk_row16c(const float (&v)[C], uint32_t avail, bool ok, int t,
                                            int k, int raw, int32_t* idx_out, float* w_out) {
  const int el = threadIdx.x & 15;
  float my_v = 0.0f, m = 0.0f;
  int my_e = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j >= k) break;
    Cand best{0.0f, INT32_MAX};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const Cand cand{v[c], (avail >> c & 1u) ? el + 16 * c : INT32_MAX};
      if (better(cand, best)) best = cand;
    }
    best = row_best16(best);
    if (best.e != INT32_MAX && (best.e & 15) == el) avail &= ~(1u << (best.e >> 4));
    if (el == j) {
      my_v = best.v;
      my_e = best.e;
    }
    if (j == 0) m = best.v;
  }
  const double ex = (el < k && !raw) ? exp((double)my_v - (double)m) : 0.0;
  double s = ex;
#pragma unroll
  for (int j = 1; j < MOE_MAX_TOPK; ++j) {
    if (j >= k) break;
    const double prev = dpp_d<0x111>(s);  // row_shr:1
    if (el == j) s = prev + s;
  }
  double z = (el == k - 1) ? s : 0.0;
  z += dpp_d<0x128>(z);
  z += dpp_d<0x124>(z);
  z += dpp_d<0x122>(z);
  z += dpp_d<0x121>(z);
  if (ok && el < k) {
    idx_out[(size_t)t * k + el] = my_e;
    w_out[(size_t)t * k + el] = raw ? my_v : (float)(ex / z);
  }
}

// Dispatch of S = T*k <= RT_TOK*8 slots whose expert ids are in LDS
// (idx_lds[S], published to wave 0), by wave 0 alone: it ranks the slots of
// each expert with ballot matches in slot order, scans the counts (capped at
// cap > 0) over the experts with lane-parallel prefix sums, and scatters (a
// slot ranked at or beyond cap is dropped: inv = -1).  Same stable counting
// sort as the dispatch kernels.  cnt, off_l, rank_l: LDS.  The other waves
// return at once; nothing here waits for the workgroup.
__device__ __forceinline__ void dispatch_small(const int32_t* idx_lds, int S, int E, int tile_rows, int cap,
                               int32_t* cnt, int32_t* off_l, int32_t* rank_l,
                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                               int32_t* __restrict__ tile_off, int32_t* __restrict__ active,
                               int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid >= 64) return;
  // (one wave: its LDS operations complete in order; the compiler fences keep
  // them in program order)
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  asm volatile("" ::: "memory");
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = 0; c * 64 < S; ++c) {
    const int sl = c * 64 + lane;
    const bool valid = sl < S;
    const int e = valid ? idx_lds[sl] : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const uint64_t earlier = match & below;
    const int c0 = valid ? cnt[e] : 0;
    asm volatile("" ::: "memory");
    if (valid) {
      rank_l[sl] = c0 + __popcll(earlier);
      if (earlier == 0) cnt[e] = c0 + __popcll(match);
    }
    asm volatile("" ::: "memory");
  }
  // offsets / tile schedule / non-empty list: lane-parallel over 64 experts
  // at a time, carried across the chunks
  int o = 0, tt = 0, n = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const bool in = e < E;
    int c = in ? cnt[e] : 0;
    if (cap > 0 && c > cap) c = cap;  // pairs kept
    const int tl = (c + tile_rows - 1) / tile_rows;
    const int ic = wave_incl_scan(c), it = wave_incl_scan(tl);
    const uint64_t nz = __ballot(c > 0);
    if (in) {
      const int oe = o + ic - c;
      off_l[e] = oe;
      offsets[e] = oe;
      counts[e] = c;
      tile_off[e] = tt + it - tl;
      if (c > 0) active[n + __popcll(nz & below)] = e;
    }
    o += __builtin_amdgcn_readlane(ic, 63);
    tt += __builtin_amdgcn_readlane(it, 63);
    n += __popcll(nz);
  }
  if (lane == 0) {
    off_l[E] = o;
    offsets[E] = o;
    tile_off[E] = tt;
    active[E] = n;
  }
  asm volatile("" ::: "memory");
  for (int sl = lane; sl < S; sl += 64) {
    if (sl >= o) perm[sl] = -1;  // beyond the kept pairs
    const int rk = rank_l[sl];
    if (cap > 0 && rk >= cap) {
      inv[sl] = -1;  // dropped
      continue;
    }
    const int p = off_l[idx_lds[sl]] + rk;
    perm[p] = sl;
    inv[sl] = p;
  }
}

// Wr [H][E] -> WrT [E][H] (64 x 64 tiles through LDS), so that the router
// operand of the logits GEMM is K-contiguous like the tokens (routers of more
// than 64 experts).  Rows move as 16-byte runs of 8 values (E a multiple of
// 8; else element by element).
__global__ __launch_bounds__(256) void router_transpose_kernel(const uint16_t* __restrict__ wr,
                                                               int H, int E,
                                                               uint16_t* __restrict__ wrt) {
  constexpr int P = 72;  // row pitch (elements): 16-byte aligned rows, spread banks
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];  // [h][e]
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  if (E % 8 == 0) {
#pragma unroll
    for (int i = threadIdx.x; i < 64 * 8; i += 256) {
      const int r = i >> 3, c = (i & 7) * 8;  // hidden unit, first of 8 experts
      u32x4 v{0u, 0u, 0u, 0u};
      if (h0 + r < H && e0 + c < E) v = ldg16(wr + (size_t)(h0 + r) * E + e0 + c);
      *reinterpret_cast<u32x4*>(tile + r * P + c) = v;
    }
  } else {
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int r = i >> 6, c = i & 63;
      tile[r * P + c] = (h0 + r < H && e0 + c < E) ? wr[(size_t)(h0 + r) * E + e0 + c] : (uint16_t)0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int r = i >> 3, c = (i & 7) * 8;  // expert, first of 8 hidden units
    if (e0 + r >= E || h0 + c >= H) continue;  // H is a multiple of 8
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)tile[(c + 2 * q) * P + r] | ((uint32_t)tile[(c + 2 * q + 1) * P + r] << 16);
    *reinterpret_cast<u32x4*>(wrt + (size_t)(e0 + r) * H + h0 + c) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Partial logits of one hidden slice for 64 tokens: part[split][t][e] = sum
// over h in the slice of x[t][h] * Wr[h][e], tokens as the A operand and the
// router as the B operand of v_mfma_f32_16x16x32_bf16, the token operands
// read straight from global memory a chunk ahead.  Each 128-wide hidden
// chunk of the router is staged in LDS once per workgroup and shared by its
// 4 waves (read straight from L2 every wave would fetch it four times), as
// [e][h] rows so that the MFMA B operand is a 16-byte read, double-buffered
// with the next chunk's loads in flight during the MFMAs.  DIRECT (E <= 64):
// the router is read in its [H][E] layout and transposed on the way: a piece
// of the staging is 8 experts of one hidden row (16 bytes; element by
// element when E is not a multiple of 8), the 64 lanes of a wave taking 64
// consecutive hidden rows, so that its 2-byte LDS writes fall on
// consecutive addresses.  Else the router comes transposed ([E][H],
// router_transpose_kernel) and a piece is 8 hidden units of one expert.
// (Direct staging saves the transpose launch: Mixtral-shaped prefill route
// 27 -> 19 us, 64-expert route 16.5 -> 13.3 us; at 128 experts its loads
// touch 64 lines per instruction and the route took 1 us longer.)
template <int NT, bool DIRECT>
__global__ __launch_bounds__(256) void router_partial_lds_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, const uint16_t* __restrict__ wr,
    int hslice, float* __restrict__ part) {
  constexpr int CH = 128;      // hidden units per chunk
  constexpr int LW = CH + 8;   // LDS row pitch (bf16): 16 rows of one read hit 16 bank groups
  constexpr int NE = NT * 16;  // router rows staged (rows >= E are zeros)
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][NE * LW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile0 = blockIdx.x * RT_TOK;
  const int hb = blockIdx.y * hslice;
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int my_tok = tile0 + wave * 16 + (lane & 15);
  const bool tok_ok = my_tok < T;
  const int kq = (lane >> 4) * 8;
  const uint16_t* xrow = x + (size_t)(tok_ok ? my_tok : 0) * H + hb + kq;
  // staging, NT pieces of 16 bytes per thread.  DIRECT: CH hidden rows x
  // NE / 8 groups of 8 experts, piece pc = hidden row pc % CH, experts
  // 8 (pc / CH) .. + 7.  Else NE rows x 16 pieces: piece pc = expert pc / 16,
  // hidden units 8 (pc % 16) .. + 7.
  u32x4 r[NT];
  const bool e8 = (E & 7) == 0;
  auto stage_load = [&](int h) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int pc = tid + i * 256;
      if constexpr (DIRECT) {
        const int hh = pc % CH, e0 = 8 * (pc / CH);
        const bool in = h + hh < hslice && e0 < E;
        const uint16_t* src = wr + (size_t)(hb + h + hh) * E + e0;
        if (e8) {
          r[i] = in ? ldg16(src) : u32x4{0u, 0u, 0u, 0u};
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          if (in)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (e0 + j < E) w[j >> 1] |= (uint32_t)src[j] << (16 * (j & 1));
          r[i] = u32x4{w[0], w[1], w[2], w[3]};
        }
      } else {
        const int row = pc >> 4, c = pc & 15;
        r[i] = (row < E && h + c * 8 < hslice) ? ldg16(wr + (size_t)row * H + hb + h + c * 8)
                                               : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stage_store = [&](int b) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int pc = tid + i * 256;
      if constexpr (DIRECT) {
        const int hh = pc % CH, e0 = 8 * (pc / CH);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t v = r[i][j >> 1];
          wl[b][(e0 + j) * LW + hh] = (uint16_t)(v >> (16 * (j & 1)));
        }
      } else {
        const int row = pc >> 4, c = pc & 15;
        *reinterpret_cast<u32x4*>(&wl[b][row * LW + c * 8]) = r[i];
      }
    }
  };
  // the token operands of a chunk are loaded a chunk ahead
  u32x4 an[4];
  auto tok_load = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      an[s] = (tok_ok && h + s * 32 < hslice) ? ldg16(xrow + h + s * 32) : u32x4{0u, 0u, 0u, 0u};
  };
  stage_load(0);
  tok_load(0);
  stage_store(0);
  __syncthreads();
  int b = 0;
  for (int h = 0; h < hslice; h += CH) {
    const bool more = h + CH < hslice;
    u32x4 av[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) av[s] = an[s];
    if (more) {
      stage_load(h + CH);
      tok_load(h + CH);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (h + s * 32 < hslice)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const u32x4 bv =
              *reinterpret_cast<const u32x4*>(&wl[b][(n * 16 + (lane & 15)) * LW + s * 32 + kq]);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[s]), as_bf16x8(bv), acc[n],
                                                           0, 0, 0);
        }
    if (more) stage_store(b ^ 1);  // its readers finished at the previous barrier
    __syncthreads();
    b ^= 1;
  }
  float* out = part + (size_t)blockIdx.y * T * E;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = n * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tile0 + wave * 16 + (lane >> 4) * 4 + j;
      if (e < E && t < T) out[(size_t)t * E + e] = acc[n][j];
    }
  }
}

// Sum of the partial logits in split order (+ bias), then top-k and softmax,
// for k <= MOE_MAX_TOPK and E <= 16 C: 16 tokens per workgroup, one per
// 16-lane row (lane el sums and ranks experts el + 16 c in registers, no LDS).
// The splits are read four at a time, all loads of a group in flight.
// nsplit == 0: `part` holds caller-given logits [T][E], used as they are.
constexpr int RK16_TOK = 16;
template <int C>
__global__ __launch_bounds__(256) void router_topk16_kernel(const float* __restrict__ part,
                                                            int nsplit, int T, int E, int k,
                                                            int raw, const float* __restrict__ bias,
                                                            int32_t* __restrict__ idx_out,
                                                            float* __restrict__ w_out) {
  const int el = threadIdx.x & 15;
  const int t = blockIdx.x * RK16_TOK + (threadIdx.x >> 4);
  const bool ok = t < T;
  uint32_t avail = 0;
  float v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const bool in = ok && el + 16 * c < E;
    avail |= (uint32_t)in << c;
    v[c] = 0.0f;
  }
  const int np = nsplit > 0 ? nsplit : 1;
  for (int p0 = 0; p0 < np; p0 += 4) {
    float q[4][C];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int c = 0; c < C; ++c)
        q[d][c] = (p0 + d < np && (avail >> c & 1u))
                      ? part[((size_t)(p0 + d) * T + t) * E + el + 16 * c]
                      : 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (p0 + d < np) v[c] = (p0 + d == 0) ? q[d][c] : v[c] + q[d][c];
  }
  if (nsplit > 0 && bias) {
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (avail >> c & 1u) v[c] += bias[el + 16 * c];
  }
  topk_row16c<C>(v, avail, ok, t, k, raw, idx_out, w_out);
}

// The same for k > MOE_MAX_TOPK (top-k by ranks): RK_TOK tokens per
// workgroup, one per wave, the sums staged in LDS.
constexpr int RK_TOK = 4;
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part,
                                                          int nsplit, int T, int E, int k, int raw,
                                                          const float* __restrict__ bias,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out) {
  __shared__ float lg[RK_TOK * (MOE_MAX_EXPERTS + 1)];
  __shared__ double exs[4 * MOE_MAX_EXPERTS];  // (k > MOE_MAX_TOPK only)
  const int ldl = E + 1;
  const int tid = threadIdx.x;
  const int tile0 = blockIdx.x * RK_TOK;
  for (int i = tid; i < RK_TOK * E; i += 256) {
    const int r = i / E, e = i % E, t = tile0 + r;
    if (t >= T) continue;
    float v[RT_MAX_SPLITS];
#pragma unroll
    for (int p = 0; p < RT_MAX_SPLITS; ++p)
      v[p] = (p < nsplit || p == 0) ? part[((size_t)p * T + t) * E + e] : 0.0f;
    float s = v[0];
#pragma unroll
    for (int p = 1; p < RT_MAX_SPLITS; ++p)
      if (p < nsplit) s += v[p];
    if (nsplit > 0 && bias) s += bias[e];
    lg[r * ldl + e] = s;
  }
  __syncthreads();
  topk_rows(lg, ldl, tile0, T, E, k, raw, idx_out, w_out, 4, nullptr, RK_TOK, exs);
}

__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, int T, int H, int E, int k, int raw,
    const float* __restrict__ wr, const float* __restrict__ bias,
    const float* __restrict__ logits_in, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out) {
  __shared__ float lg[RT_TOK * 257];
  __shared__ double exs[4 * MOE_MAX_EXPERTS];  // (k > MOE_MAX_TOPK only)
  const int ldl = E + 1;
  const int tid = threadIdx.x;
  const int tile0 = blockIdx.x * RT_TOK;
  for (int i = tid; i < RT_TOK * E; i += 256) {
    const int r = i / E, e = i % E, t = tile0 + r;
    if (t >= T) continue;
    float s;
    if (logits_in) {
      s = logits_in[(size_t)t * E + e];
    } else {
      s = 0.0f;
      for (int h = 0; h < H; ++h) s = fmaf(x[(size_t)t * H + h], wr[(size_t)h * E + e], s);
      if (bias) s += bias[e];
    }
    lg[r * ldl + e] = s;
  }
  __syncthreads();
  topk_rows(lg, ldl, tile0, T, E, k, raw, idx_out, w_out, 4, nullptr, RT_TOK, exs);
}

// Branch input of a stacked layer: xt[t] = bf16(h[t] / sqrt(mean(h[t]^2) + 1e-6)),
// the division taken as one fp32 reciprocal and a product per element.
// One workgroup per token.  Thread i holds the 4-float groups i, i + 256, ...
// of the row in registers (NV of them, all loads in flight together), sums
// their squares in that order, the waves reduce with a butterfly and the four
// wave sums are added in wave order, so the reduction order is fixed.
template <int NV>
__global__ __launch_bounds__(256) void prenorm_kernel(const float* __restrict__ h, int H,
                                                      uint16_t* __restrict__ xt) {
  __shared__ float wsum[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const f32x4* row = reinterpret_cast<const f32x4*>(h + (size_t)t * H);
  const int n4 = H >> 2;
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * 256;
    v[i] = c < n4 ? row[c] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fmaf(v[i][j], v[i][j], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float ri = 1.0f / sqrtf(tot / (float)H + 1e-6f);
  uint2* out = reinterpret_cast<uint2*>(xt + (size_t)t * H);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = tid + i * 256;
    if (c < n4) {
      const bf16x2 lo = {(__bf16)(v[i][0] * ri), (__bf16)(v[i][1] * ri)};
      const bf16x2 hi = {(__bf16)(v[i][2] * ri), (__bf16)(v[i][3] * ri)};
      out[c] = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
  }
}

// Small batches (T <= 64, one token tile): routing and dispatch in one
// launch.  Every workgroup computes the partial logits of its hidden slice;
// the last one to finish (counted with a device-scope atomic after a
// release fence) adds the slices in split order, selects the top-k of each
// token, and builds counts / offsets / tile schedule / non-empty expert list
// / perm / inv with the same ballot-ranked counting sort as the dispatch
// kernels.  That workgroup resets the counter for the next launch.  The
// result does not depend on which workgroup finishes last.
template <int NT>
__global__ __launch_bounds__(256) void route_small_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, int k, int raw,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int hslice,
    float* __restrict__ part, int32_t* __restrict__ counter, int tile_rows, int cap,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
    int32_t* __restrict__ active, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  constexpr int EP = NT * 16;
  constexpr int LDW = RT_HC + RT_PAD;
  __shared__ __attribute__((aligned(16))) uint16_t wt[EP * LDW];
  __shared__ float lg[RT_TOK * (EP + 1)];
  __shared__ int32_t cnt[MOE_MAX_EXPERTS];
  __shared__ int32_t off_l[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t rank_l[RT_TOK * MOE_MAX_TOPK];
  __shared__ int32_t idx_l[RT_TOK * MOE_MAX_TOPK];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int hb = split * hslice;

  {  // partial logits of all T (<= 64) tokens over this hidden slice
    f32x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int my_tok = wave * 16 + (lane & 15);
    const bool tok_ok = my_tok < T;
    const uint16_t* xrow = x + (size_t)(tok_ok ? my_tok : 0) * H;
    const int kq = (lane >> 4) * 8;
    for (int h0 = hb; h0 < hb + hslice; h0 += RT_HC) {
      u32x4 av[RT_HC / 32];
#pragma unroll
      for (int q = 0; q < RT_HC / 32; ++q)
        av[q] = tok_ok ? ldg16(xrow + h0 + q * 32 + kq) : u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
      for (int i = tid; i < RT_HC * EP; i += 256) {
        const int r = i / EP, e = i % EP;
        wt[e * LDW + r] = (e < E) ? wr[(size_t)(h0 + r) * E + e] : (uint16_t)0;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < RT_HC / 32; ++q) {
        const bf16x8 a = as_bf16x8(av[q]);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint16_t* bp = wt + (n * 16 + (lane & 15)) * LDW + q * 32 + kq;
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, as_bf16x8(*reinterpret_cast<const u32x4*>(bp)), acc[n], 0, 0, 0);
        }
      }
    }
    float* out = part + (size_t)split * T * E;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = n * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = wave * 16 + (lane >> 4) * 4 + j;
        if (e < E && t < T) out[(size_t)t * E + e] = acc[n][j];
      }
    }
  }
  if (!last_workgroup(counter, &s_last)) return;  // then every block's partials are seen

  const int ns = gridDim.x;
  const int ldl = E + 1;
  for (int i = tid; i < T * E; i += 256) {
    const int t = i / E, e = i % E;
    float s = part[(size_t)t * E + e];
    for (int q = 1; q < ns; ++q) s += part[((size_t)q * T + t) * E + e];
    if (bias) s += bias[e];
    lg[t * ldl + e] = s;
  }
  __syncthreads();
  // (no LDS for the top-k-by-ranks path: the small-batch routes are taken
  // only with k <= MOE_MAX_TOPK)
  topk_rows(lg, ldl, 0, T, E, k, raw, idx_out, w_out, 4, idx_l);
  __syncthreads();
  dispatch_small(idx_l, T * k, E, tile_rows, cap, cnt, off_l, rank_l, counts, offsets, tile_off,
                 active, perm, inv);
}

// Small batches with few experts (T <= 64, E <= 16, H <= 4096, H a multiple
// of 512): routing and dispatch in one workgroup of 16 waves, no device-scope
// synchronisation.  The router is staged transposed in LDS ([e][h], padded
// rows), wave w takes the hidden slice [w H/16, (w+1) H/16) for all tokens
// (tokens as the A operand, read from global memory), the 16 partial logit
// tiles are added in wave order (+ bias), then top-k and the dispatch.
// MULTI: one workgroup per 16 tokens (the token rows of a larger batch are
// then read through several CUs); each routes its tokens, and the last to
// finish (a device-scope atomic after a release fence, as in the split-H
// kernel) reads every token's experts back and dispatches them all, then
// resets the counter for the next launch.
constexpr int R1_HMAX = 4096;
constexpr int R1_LDW = R1_HMAX + 8;  // padded router row (bf16)
// PN: the input is the fp32 residual stream h; the workgroup also forms the
// branch input bf16(h / sqrt(mean h^2 + 1e-6)) of its tokens (written to xt
// for the expert kernels) and routes on it.  Each lane loads the fp32 values
// of exactly the bf16 operand fragments it feeds to the MFMA, so the norm
// needs only a reduction: over the 4 lane groups of a wave (butterfly), then
// over the 16 waves in wave order.
template <int MB, int EV, bool MULTI, bool PN>
__global__ __launch_bounds__(1024) void route_one_kernel(
    const uint16_t* __restrict__ x, int T_all, int H, int E, int k, int raw,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int tile_rows, int cap,
    int32_t* __restrict__ counter, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
    int32_t* __restrict__ active, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    const float* __restrict__ hres, uint16_t* __restrict__ xt_out, uint16_t* __restrict__ x16_out) {
  static_assert(!MULTI || MB == 1, "one token block per workgroup");
  static_assert(!PN || MB == 1, "prenorm: one token block per workgroup");
  const int tok0 = MULTI ? (int)blockIdx.x * 16 : 0;  // this workgroup's first token
  const int T = MULTI ? min(16, T_all - tok0) : T_all;
  x += (size_t)tok0 * H;
  if (PN) {
    hres += (size_t)tok0 * H;
    xt_out += (size_t)tok0 * H;
  }
  if (x16_out) x16_out += (size_t)tok0 * H;
  // the staged router, later the 16 partial logit tiles [16][RT_TOK][17]
  __shared__ __attribute__((aligned(16))) uint16_t wt[16 * R1_LDW];
  __shared__ float lg[RT_TOK * 17];
  __shared__ int32_t idx_l[RT_TOK * MOE_MAX_TOPK];
  __shared__ int32_t cnt[16];
  __shared__ int32_t off_l[17];
  __shared__ int32_t rank_l[RT_TOK * MOE_MAX_TOPK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;

  // The loads come first, all in flight together: this wave's token
  // fragments of the first two token blocks, then the router rows.
  const int hw = H / 16, hb = wave * hw, nks = hw / 32;  // nks <= 8
  constexpr int KS = R1_HMAX / 16 / 32;
  u32x4 xa[2][KS];
  f32x4 hv[PN ? KS : 1][2];  // PN: this lane's 8 fp32 values per K step
  auto load_x = [&](int m0) {
    if (PN) {
      const float* hr = hres + (size_t)min(r16, T - 1) * H + hb + kg * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (s < nks) {
          hv[s][0] = *reinterpret_cast<const f32x4*>(hr + s * 32);
          hv[s][1] = *reinterpret_cast<const f32x4*>(hr + s * 32 + 4);
        }
      return;
    }
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const uint16_t* xr = x + (size_t)min((m0 + mm) * 16 + r16, T - 1) * H + hb + kg * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        if (m0 + mm < MB && s < nks) xa[mm][s] = ldg16(xr + s * 32);
    }
  };
  load_x(0);
  __shared__ float pn_ss[PN ? 16 * 16 : 1];  // [wave][token] sums of squares
  // stage Wr^T (EV = 8: E is 8 and a router row is one 16-byte load)
  if (EV > 0) {
    // thread i < H/8 takes router rows 8i .. 8i+7 (8 experts per 16-byte
    // load) in two halves of 4 rows, transposes the 4x8 bf16 blocks in
    // registers and writes each expert's 4 consecutive hidden units as one
    // 8-byte LDS store
    const int g = tid;  // group of 8 rows
    if (g * 8 < H) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 rv[4][EV / 8];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int q = 0; q < EV / 8; ++q)
            rv[r][q] = ldg16(wr + (size_t)(g * 8 + half * 4 + r) * EV + q * 8);
#pragma unroll
        for (int q = 0; q < EV / 8; ++q)
#pragma unroll
          for (int ee = 0; ee < 8; ++ee) {  // expert q*8 + ee
            uint2 o;
            const int sh = 16 * (ee & 1);
            o.x = ((rv[0][q][ee >> 1] >> sh) & 0xffffu) | (((rv[1][q][ee >> 1] >> sh) & 0xffffu) << 16);
            o.y = ((rv[2][q][ee >> 1] >> sh) & 0xffffu) | (((rv[3][q][ee >> 1] >> sh) & 0xffffu) << 16);
            *reinterpret_cast<uint2*>(wt + (q * 8 + ee) * R1_LDW + g * 8 + half * 4) = o;
          }
      }
      if (EV == 8) {
#pragma unroll
        for (int ee = 8; ee < 16; ++ee)
          *reinterpret_cast<u32x4*>(wt + ee * R1_LDW + g * 8) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  } else {
    for (int h = tid; h < H; h += 1024) {
      uint16_t wv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) wv[e] = e < E ? wr[(size_t)h * E + e] : (uint16_t)0;
#pragma unroll
      for (int e = 0; e < 16; ++e) wt[e * R1_LDW + h] = wv[e];
    }
  }
  if (PN) {  // this lane's part of its token's sum of squares, in K order
    float ss = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (s < nks)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int j = 0; j < 4; ++j) ss = fmaf(hv[s][hf][j], hv[s][hf][j], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (kg == 0) pn_ss[wave * 16 + r16] = ss;
  }
  __syncthreads();
  if (PN) {
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) tot += pn_ss[w * 16 + r16];
    const float ri = 1.0f / sqrtf(tot / (float)H + 1e-6f);
    const bool own = r16 < T;  // rows past T repeat the last token: no store
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (s < nks) {
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = hv[s][j >> 1];
          const int o = (j & 1) * 2;
          const bf16x2 b2 = {(__bf16)(v[o] * ri), (__bf16)(v[o + 1] * ri)};
          q[j] = __builtin_bit_cast(uint32_t, b2);
        }
        xa[0][s] = u32x4{q[0], q[1], q[2], q[3]};
        if (own)
          *reinterpret_cast<u32x4*>(xt_out + (size_t)r16 * H + hb + s * 32 + kg * 8) = xa[0][s];
      }
  }
  // uint8 expert layers take the expert input in fp16: this lane's operand
  // values as fp16 (exact in fp16's normal range), one 16-byte store each
  if (x16_out && r16 < T) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      if (s < nks) {
        const u32x4 v = xa[0][s];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                                  __uint_as_float(d[j] << 16),
                                                  __uint_as_float(d[j] & 0xFFFF0000u)));
        *reinterpret_cast<u32x4*>(x16_out + (size_t)r16 * H + hb + s * 32 + kg * 8) =
            u32x4{o[0], o[1], o[2], o[3]};
      }
  }

  f32x4 acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m0 = 0; m0 < MB; m0 += 2) {
    if (m0 > 0) load_x(m0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s >= nks) break;
      const bf16x8 b =
          as_bf16x8(*reinterpret_cast<const u32x4*>(wt + r16 * R1_LDW + hb + s * 32 + kg * 8));
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
        if (m0 + mm < MB)
          acc[m0 + mm] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mm][s]), b, acc[m0 + mm], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the staged router
  // 16x16 layout: lane l holds expert column l%16 and token rows 4(l/16)+j
  float* part = reinterpret_cast<float*>(wt);
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      part[(wave * RT_TOK + m * 16 + 4 * kg + j) * 17 + r16] = acc[m][j];
  __syncthreads();
  for (int i = tid; i < T * E; i += 1024) {
    const int t = i / E, e = i - t * E;
    float s = part[t * 17 + e];
    for (int w = 1; w < 16; ++w) s += part[(w * RT_TOK + t) * 17 + e];
    if (bias) s += bias[e];
    lg[t * 17 + e] = s;
  }
  __syncthreads();
  if (MULTI) {
    topk_rows16(lg, 17, 0, T, E, k, raw, idx_out + (size_t)tok0 * k, w_out + (size_t)tok0 * k,
                16, nullptr, RT_TOK);
    __shared__ int s_last;
    if (!last_workgroup(counter, &s_last)) return;  // then every block's experts are seen
    for (int i = tid; i < T_all * k; i += 1024) idx_l[i] = idx_out[i];
    __syncthreads();
  } else {
    topk_rows16(lg, 17, 0, T, E, k, raw, idx_out, w_out, 16, idx_l, RT_TOK);
    __syncthreads();
  }
  dispatch_small(idx_l, T_all * k, E, tile_rows, cap, cnt, off_l, rank_l, counts, offsets,
                 tile_off, active, perm, inv);
}

// Single-token decode (E = 8 or 16, H a multiple of 1024 up to R1_HMAX; the
// kernel takes up to TT tokens): routing
// and dispatch without matrix instructions or a staged router.  Thread i
// holds hidden units i, i + 1024, ... of every token and of the router rows
// (coalesced loads, all in flight at once), forms its partial logits in that
// order, and each wave adds its lanes' partials with DPP steps (row shifts,
// then row broadcasts: a fixed tree); the 16 wave sums are added in wave
// order.  With hres (residual layers) the workgroup first forms the branch
// input bf16(h / sqrt(mean h^2 + 1e-6)) the same way (squares, then the same
// reductions) and writes it for the expert kernels; with x16_out it writes
// the fp16 copy of the expert input.  Top-k and dispatch as in route_one;
// with nodisp the dispatch is left out (the matrix-vector expert kernels
// that follow take the slots in order).
__device__ __forceinline__ float wave_sum_dpp(float v) {
#define DPP_ADD(ctrl, rmask) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, false))
  DPP_ADD(0x111, 0xF);  // row_shr:1
  DPP_ADD(0x112, 0xF);  // row_shr:2
  DPP_ADD(0x114, 0xF);  // row_shr:4
  DPP_ADD(0x118, 0xF);  // row_shr:8: lane 15 of each row holds the row's sum
  DPP_ADD(0x142, 0xA);  // row_bcast:15: lanes 31, 63 hold rows 0-1, 2-3
  DPP_ADD(0x143, 0xC);  // row_bcast:31: lane 63 holds all four
#undef DPP_ADD
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

template <int TT, int EV>  // tokens (at most), experts per router row (8 or 16)
__global__ __launch_bounds__(1024) void route_tiny_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ hres, int T, int H, int E, int k,
    int raw, const uint16_t* __restrict__ wr, const float* __restrict__ bias, int tile_rows,
    int cap, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
    int32_t* __restrict__ active, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    uint16_t* __restrict__ xt_out, uint16_t* __restrict__ x16_out, int nodisp) {
  constexpr int HPT = R1_HMAX / 1024;  // hidden units per thread, at most
  __shared__ float red[16][TT * 16];  // per-wave partial logits
  __shared__ float ssq[16][TT];
  __shared__ float lg[16 * 17];        // [token][expert], row pitch 17
  __shared__ int32_t idx_l[16 * MOE_MAX_TOPK];
  __shared__ int32_t cnt[16];
  __shared__ int32_t off_l[17];
  __shared__ int32_t rank_l[16 * MOE_MAX_TOPK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hpt = H >> 10;
  float xv[TT][HPT];
  u32x4 wv[HPT][EV / 8];
#pragma unroll
  for (int i = 0; i < HPT; ++i)
    if (i < hpt) {
      const int h = tid + (i << 10);
#pragma unroll
      for (int q = 0; q < EV / 8; ++q)
        wv[i][q] = ldg16(wr + (size_t)h * EV + q * 8);  // E == EV
#pragma unroll
      for (int t = 0; t < TT; ++t)
        if (t < T) xv[t][i] = hres ? hres[(size_t)t * H + h] : bf16_to_f32(x[(size_t)t * H + h]);
    }
  if (hres) {  // branch input: the same reduction order for the squares
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < HPT; ++i)
        if (i < hpt && t < T) ss = fmaf(xv[t][i], xv[t][i], ss);
      ss = wave_sum_dpp(ss);
      if (lane == 0) ssq[wave][t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= T) continue;
      float tot = 0.0f;
      for (int w = 0; w < 16; ++w) tot += ssq[w][t];
      const float ri = 1.0f / sqrtf(tot / (float)H + 1e-6f);
#pragma unroll
      for (int i = 0; i < HPT; ++i)
        if (i < hpt) {
          const __bf16 b = (__bf16)(xv[t][i] * ri);
          xv[t][i] = (float)b;
          xt_out[(size_t)t * H + tid + (i << 10)] = __builtin_bit_cast(uint16_t, b);
        }
    }
  }
  if (x16_out) {  // the expert input in fp16 (exact in fp16's normal range)
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int i = 0; i < HPT; ++i)
        if (i < hpt && t < T) {
          const auto f = __builtin_amdgcn_cvt_pkrtz(xv[t][i], 0.0f);
          x16_out[(size_t)t * H + tid + (i << 10)] =
              (uint16_t)(__builtin_bit_cast(uint32_t, f) & 0xFFFFu);
        }
  }
  // partial logits of this thread's hidden units, in unit order
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t >= T) continue;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      if (e >= E) continue;
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < HPT; ++i)
        if (i < hpt) {
          const uint32_t w2 = wv[i][e >> 3][(e & 7) >> 1];
          const float wf = __uint_as_float((e & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
          acc = fmaf(xv[t][i], wf, acc);
        }
      acc = wave_sum_dpp(acc);
      if (lane == 0) red[wave][t * 16 + e] = acc;
    }
  }
  __syncthreads();
  if (tid < T * 16) {  // waves added in order, then the bias
    const int t = tid >> 4, e = tid & 15;
    if (e < E) {
      float sum = 0.0f;
      for (int w = 0; w < 16; ++w) sum += red[w][t * 16 + e];
      if (bias) sum += bias[e];
      lg[t * 17 + e] = sum;
    }
  }
  __syncthreads();
  topk_rows16(lg, 17, 0, T, E, k, raw, idx_out, w_out, 16, idx_l, 16);
  if (nodisp) return;  // the expert kernels take the slots in order
  __syncthreads();
  dispatch_small(idx_l, T * k, E, tile_rows, cap, cnt, off_l, rank_l, counts, offsets,
                 tile_off, active, perm, inv);
}

}  // namespace

int router_splits(int T, int H, int E) {
  const int ntt = (T + RT_TOK - 1) / RT_TOK;
  // aim at >= 2048 workgroups when a workgroup's router share is small
  // (E <= 16: the tokens dominate its loads), else >= 512
  const int aim = E <= 16 ? 2048 : 512;
  int ns = (aim + ntt - 1) / ntt;
  int max_ns = H / 256;                    // slices of at least 256
  if (max_ns > RT_MAX_SPLITS) max_ns = RT_MAX_SPLITS;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  while (H % (ns * RT_HC)) --ns;           // slices made of whole chunks
  return ns;
}

// Step 2 over the logits (nsplit partial planes, or given logits with 0).
static void launch_topk(const float* part, int nsplit, const RouterArgs& a, const float* bias,
                 hipStream_t st) {
  if (a.k > MOE_MAX_TOPK) {
    const int kgrid = (a.T + RK_TOK - 1) / RK_TOK;
    router_topk_kernel<<<kgrid, 256, 0, st>>>(part, nsplit, a.T, a.E, a.k, a.raw_gate, bias,
                                              a.idx, a.w);
    return;
  }
  const int grid = (a.T + RK16_TOK - 1) / RK16_TOK;
#define RK16_ARGS part, nsplit, a.T, a.E, a.k, a.raw_gate, bias, a.idx, a.w
  if (a.E <= 16) router_topk16_kernel<1><<<grid, 256, 0, st>>>(RK16_ARGS);
  else if (a.E <= 32) router_topk16_kernel<2><<<grid, 256, 0, st>>>(RK16_ARGS);
  else if (a.E <= 64) router_topk16_kernel<4><<<grid, 256, 0, st>>>(RK16_ARGS);
  else if (a.E <= 128) router_topk16_kernel<8><<<grid, 256, 0, st>>>(RK16_ARGS);
  else router_topk16_kernel<16><<<grid, 256, 0, st>>>(RK16_ARGS);
#undef RK16_ARGS
}

int launch_router(const RouterArgs& a, hipStream_t st) {
  const int grid = (a.T + RT_TOK - 1) / RT_TOK;
  if (a.dtype_f32) {
    router_f32_kernel<<<grid, 256, 0, st>>>((const float*)a.x, a.T, a.H, a.E, a.k, a.raw_gate,
                                            (const float*)a.wr, a.bias, a.logits_in, a.idx,
                                            a.w);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (a.logits_in) {
    launch_topk(a.logits_in, 0, a, nullptr, st);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int ns = router_splits(a.T, a.H, a.E);
  const int hs = a.H / ns;
  const dim3 g2(grid, ns);
  const int nt = (a.E + 15) / 16;
  auto* xx = (const uint16_t*)a.x;
  auto* ww = (const uint16_t*)a.wr;
  if (nt <= 4) {  // the router staged from its own layout (no transpose launch)
    if (nt <= 1)
      router_partial_lds_kernel<1, true><<<g2, 256, 0, st>>>(xx, a.T, a.H, a.E, ww, hs, a.part);
    else if (nt <= 2)
      router_partial_lds_kernel<2, true><<<g2, 256, 0, st>>>(xx, a.T, a.H, a.E, ww, hs, a.part);
    else
      router_partial_lds_kernel<4, true><<<g2, 256, 0, st>>>(xx, a.T, a.H, a.E, ww, hs, a.part);
    launch_topk(a.part, ns, a, a.bias, st);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const dim3 gt((a.H + 63) / 64, (a.E + 63) / 64);
  router_transpose_kernel<<<gt, 256, 0, st>>>(ww, a.H, a.E, a.wrt);
  const uint16_t* wt = a.wrt;
  if (nt <= 8)
    router_partial_lds_kernel<8, false><<<g2, 256, 0, st>>>(xx, a.T, a.H, a.E, wt, hs, a.part);
  else
    router_partial_lds_kernel<16, false><<<g2, 256, 0, st>>>(xx, a.T, a.H, a.E, wt, hs, a.part);
  launch_topk(a.part, ns, a, a.bias, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// (one workgroup: with several, the workgroups' fp32 loads of the stream
// lengthen the route more than a separate normalisation launch costs)
bool route_small_folds_prenorm(int T, int H, int E) {
  return E <= 16 && H <= R1_HMAX && H % 512 == 0 && T <= 16;
}

bool route_small_writes_x16(int T, int H, int E) {
  return E <= 16 && H <= R1_HMAX && H % 512 == 0 && T <= RT_TOK;
}

int launch_route_small(const RouterArgs& a, const DispatchArgs& d, int32_t* counter,
                       hipStream_t st) {
  if ((a.hres && !route_small_folds_prenorm(a.T, a.H, a.E)) ||
      (a.x16_out && !route_small_writes_x16(a.T, a.H, a.E)))
    return -1;
  // (at T = 4 the one-token-per-row MFMA route below is the faster one)
  if ((a.E == 8 || a.E == 16) && a.H <= R1_HMAX && a.H % 1024 == 0 && a.T == 1) {
    auto* xx = (const uint16_t*)a.x;
    auto* ww = (const uint16_t*)a.wr;
#define RT_ARGS xx, a.hres, a.T, a.H, a.E, a.k, a.raw_gate, ww, a.bias, d.tile_rows, d.capacity, \
                a.idx, a.w, d.counts, d.offsets, d.tile_off, d.active, d.perm, d.inv, a.xt_out, a.x16_out, \
                d.none ? 1 : 0
    // a router row is one (E = 8) or two (E = 16) 16-byte loads
    if (a.E == 8) route_tiny_kernel<1, 8><<<1, 1024, 0, st>>>(RT_ARGS);
    else route_tiny_kernel<1, 16><<<1, 1024, 0, st>>>(RT_ARGS);
#undef RT_ARGS
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (a.E <= 16 && a.H <= R1_HMAX && a.H % 512 == 0 && a.T <= RT_TOK) {
    auto* xx = (const uint16_t*)a.x;
    auto* ww = (const uint16_t*)a.wr;
#define R1_ARGS xx, a.T, a.H, a.E, a.k, a.raw_gate, ww, a.bias, d.tile_rows, d.capacity, counter, a.idx, \
                a.w, d.counts, d.offsets, d.tile_off, d.active, d.perm, d.inv, a.hres, a.xt_out, a.x16_out
    const int mb = (a.T + 15) / 16;
    // one workgroup up to 16 tokens, one per 16 tokens beyond
#define R1_MB(EV, PN)                                                                \
    if (mb <= 1) route_one_kernel<1, EV, false, PN><<<1, 1024, 0, st>>>(R1_ARGS);    \
    else route_one_kernel<1, EV, true, PN><<<mb, 1024, 0, st>>>(R1_ARGS);
    if (a.hres) {
      if (a.E == 8) { R1_MB(8, true) }
      else { R1_MB(0, true) }
    } else {
      if (a.E == 8) { R1_MB(8, false) }
      else { R1_MB(0, false) }
    }
#undef R1_MB
#undef R1_ARGS
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int ns = router_splits(a.T, a.H, a.E);
  const int hs = a.H / ns;
  const int nt = (a.E + 15) / 16;
  auto* xx = (const uint16_t*)a.x;
  auto* ww = (const uint16_t*)a.wr;
#define RS_ARGS xx, a.T, a.H, a.E, a.k, a.raw_gate, ww, a.bias, hs, a.part, counter, d.tile_rows, d.capacity, a.idx, a.w, \
                d.counts, d.offsets, d.tile_off, d.active, d.perm, d.inv
  if (nt <= 1) route_small_kernel<1><<<ns, 256, 0, st>>>(RS_ARGS);
  else if (nt <= 2) route_small_kernel<2><<<ns, 256, 0, st>>>(RS_ARGS);
  else if (nt <= 4) route_small_kernel<4><<<ns, 256, 0, st>>>(RS_ARGS);
  else if (nt <= 8) route_small_kernel<8><<<ns, 256, 0, st>>>(RS_ARGS);
  else route_small_kernel<16><<<ns, 256, 0, st>>>(RS_ARGS);
#undef RS_ARGS
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prenorm(const float* h, int T, int H, uint16_t* xt, hipStream_t st) {
  // H is a multiple of 4 (a multiple of 256 for bf16 layers, the only ones
  // with a residual stream) and at most 64 K: up to 64 floats per thread
  const int nv = (H / 4 + 255) / 256;
  if (H % 4 || nv > 16) return -1;
  if (nv <= 1) prenorm_kernel<1><<<T, 256, 0, st>>>(h, H, xt);
  else if (nv <= 2) prenorm_kernel<2><<<T, 256, 0, st>>>(h, H, xt);
  else if (nv <= 4) prenorm_kernel<4><<<T, 256, 0, st>>>(h, H, xt);
  else if (nv <= 8) prenorm_kernel<8><<<T, 256, 0, st>>>(h, H, xt);
  else prenorm_kernel<16><<<T, 256, 0, st>>>(h, H, xt);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
