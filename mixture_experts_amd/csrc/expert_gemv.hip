// expert_gemv.hip -- steps 4 and 5 for a single token (decode at batch 1).
//
// Same SwiGLU expert as the other paths [zskr.cn/news/2275853
// "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1, sec. 3.3 stage 4],
// and the same weighted sum of the routed experts' outputs (step 5, sec. 3.3
// stage 5); uint8 experts hold (q - zero) * scale per matrix
// [www.pnsm.cn/news/1892388.html sec. 3.1 and sec. 5.2].
//
// With one token, every routed expert's FFN is two matrix-vector products:
// each weight byte is used once, so the work is a stream of the routed
// experts' weights from HBM and nothing else matters as much as keeping
// enough of that stream in flight.  The weights therefore go straight from
// HBM into registers (non-temporal 16-byte loads, no LDS staging, no
// barriers), each wave keeps the loads of its next task in flight while it
// computes the current one, and enough waves run per SIMD that the chip
// holds well over a hundred KB of loads per CU.  The products run on the
// packed dot instructions (v_dot2_f32_f16 for uint8 codes against fp16
// operands, v_dot2_f32_bf16 for bf16), fp32 accumulation; the matrix cores
// would idle at one column.
//
// A weight row (K contiguous elements) is read in 1 KB pieces, one 16-byte
// load per lane: lane l of piece i holds the V elements i*64*V + l*V ..
// + V - 1 (V = 16 uint8 codes or 8 bf16 weights).  A lane's partial sums
// run over its pieces in order (two chains, even and odd pieces, added at
// the end), then the wave adds its lanes in a fixed DPP order: the result
// is the same on every call.
//
// Both kernels read the routing itself (expert and activation row of each
// slot: one step of dependent loads before the first weight load).
// gate/up: one task = gate row f and up row f of one routed expert; the
// token's operand for the lane's K positions sits in registers for the
// whole kernel; the task ends with SiLU(g) * u rounded to bf16 (stored as
// fp16 for uint8 layers, whose down projection takes fp16 operands).
// down: one task = hidden row h of every routed expert; the activation rows
// of the token's slots are copied to LDS once per workgroup; the task ends
// with y[h] = (residual[h] +) sum_j w_j * out_j[h], slots in ascending order,
// one fp32 fused multiply-add per slot (the separate combine's arithmetic),
// or, when the combine runs separately, with the per-slot rows.
#include "common.h"
#include "kernels.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Sum over the wave, every lane's value added in one fixed order; the
// result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#define WS_DPP(ctrl, rmask) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, false))
  WS_DPP(0x111, 0xF);  // row_shr:1
  WS_DPP(0x112, 0xF);  // row_shr:2
  WS_DPP(0x114, 0xF);  // row_shr:4
  WS_DPP(0x118, 0xF);  // row_shr:8: lane 15 of each row of 16 holds its sum
  WS_DPP(0x142, 0xA);  // row_bcast:15: lanes 31 and 63 hold rows 0-1 and 2-3
  WS_DPP(0x143, 0xC);  // row_bcast:31: lane 63 holds all four
#undef WS_DPP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Element d of a 4-dword vector as a scalar.  (A bit cast applied straight
// to a vector element, v[d], reads element 0 with this compiler; casting a
// scalar copy is exact.)
__device__ __forceinline__ uint32_t dw(u32x4 v, int d) {
  const uint32_t r = v[d];
  return r;
}

// The lane's operand of one 16-byte weight piece: 16 fp16 values in pairs
// (uint8 codes) or 8 bf16 values in pairs.
template <bool Q8> struct Opnd;
template <> struct Opnd<true> { h2_t v[8]; };
template <> struct Opnd<false> { b2_t v[4]; };

__device__ __forceinline__ Opnd<true> opnd_of(u32x4 a, u32x4 b, Opnd<true>*) {
  Opnd<true> o;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    o.v[d] = __builtin_bit_cast(h2_t, dw(a, d));
    o.v[4 + d] = __builtin_bit_cast(h2_t, dw(b, d));
  }
  return o;
}
__device__ __forceinline__ Opnd<false> opnd_of(u32x4 a, u32x4, Opnd<false>*) {
  Opnd<false> o;
#pragma unroll
  for (int d = 0; d < 4; ++d) o.v[d] = __builtin_bit_cast(b2_t, dw(a, d));
  return o;
}

// acc + the dot product of one 16-byte weight piece with the operand.
// uint8: a byte permute of each code under the constant byte 0x64 gives the
// fp16 value 1024 + q, exactly, and one packed add of bias = -(1024 + zero)
// gives q - zero, exactly; the scale multiplies the finished row sum.
__device__ __forceinline__ float dot_piece(u32x4 w, const Opnd<true>& x, h2_t bias, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const h2_t lo =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, dw(w, d), 0x04010400u)) + bias;
    const h2_t hi =
        __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, dw(w, d), 0x04030402u)) + bias;
    acc = __builtin_amdgcn_fdot2(lo, x.v[2 * d], acc, false);
    acc = __builtin_amdgcn_fdot2(hi, x.v[2 * d + 1], acc, false);
  }
  return acc;
}
__device__ __forceinline__ float dot_piece(u32x4 w, const Opnd<false>& x, h2_t, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, dw(w, d)), x.v[d], acc, false);
  return acc;
}

// The uint8 parameter block after an expert's three matrices: scale[3],
// zero[3] (matrix m: 0 gate, 1 up, 2 down).
struct QParams {
  float scale;
  h2_t bias;
};
__device__ __forceinline__ QParams qparams(const uint8_t* eb, int H, int F, int m) {
  const uint8_t* pb = eb + 3 * (size_t)F * H;
  QParams q;
  q.scale = reinterpret_cast<const float*>(pb)[m];
  const _Float16 b = (_Float16)(-(1024 + reinterpret_cast<const int32_t*>(pb)[3 + m]));
  q.bias = h2_t{b, b};
  return q;
}

// ---------------------------------------------------------------- gate/up
// One wave's gate/up tasks.  LR: 1 KB pieces per weight row (K = H).  x: the
// token's expert input (fp16 for uint8 experts, bf16 otherwise); idx, inv:
// its routing (slot s: expert idx[s], activation row inv[s], or row s when
// inv is null); act: [S][F]
// out.  One token: its k slots reach k different experts, none beyond a
// capacity (an expert sees at most one pair), so there are k * F tasks.
template <bool Q8, int LR>
struct GuTasks {
  static constexpr int WE = Q8 ? 1 : 2;  // bytes per weight
  static constexpr int V = 16 / WE;      // weights per 16-byte piece
  struct Task {
    u32x4 w[2][LR];  // gate row, up row
    const uint8_t* eb;
    int p, f;
  };
  const uint8_t* experts;
  uint64_t stride_b;
  const uint16_t* x;
  const int32_t* idx;
  const int32_t* inv;
  uint16_t* act;
  int H, F, ntask, lane;
  size_t row_b;
  Opnd<Q8> xo[LR];  // the token's operand at this lane's K positions

  __device__ __forceinline__ GuTasks(const uint8_t* experts_, uint64_t stride_b_,
                                     const uint16_t* x_, const int32_t* idx_, const int32_t* inv_,
                                     int ktop, int H_, int F_, uint16_t* act_)
      : experts(experts_), stride_b(stride_b_), x(x_), idx(idx_), inv(inv_), act(act_), H(H_),
        F(F_), ntask(ktop * F_), lane((int)threadIdx.x & 63), row_b((size_t)H_ * WE) {}

  __device__ __forceinline__ void load_x() {
#pragma unroll
    for (int i = 0; i < LR; ++i) {
      const uint16_t* xp = x + i * 64 * V + lane * V;
      const u32x4 a = *reinterpret_cast<const u32x4*>(xp);
      const u32x4 b = Q8 ? *reinterpret_cast<const u32x4*>(xp + 8) : a;
      xo[i] = opnd_of(a, b, (Opnd<Q8>*)nullptr);
    }
  }
  // issue the loads of task t (t >= ntask: loads of the token row instead,
  // in bounds and cached, never used)
  __device__ __forceinline__ void issue(int t, Task& k) const {
    const uint8_t* g;
    const uint8_t* u;
    if (t < ntask) {
      const int s = t / F;
      k.f = t - s * F;
      const int e = idx[s];
      k.p = inv ? inv[s] : s;
      k.eb = experts + stride_b * e;
      g = k.eb + (size_t)k.f * row_b;
      u = k.eb + (size_t)(F + k.f) * row_b;
    } else {
      g = u = reinterpret_cast<const uint8_t*>(x);
    }
#pragma unroll
    for (int i = 0; i < LR; ++i) {
      k.w[0][i] = ld_nt(g + i * 1024 + lane * 16);
      k.w[1][i] = ld_nt(u + i * 1024 + lane * 16);
    }
  }
  __device__ __forceinline__ void finish(const Task& k) const {
    QParams qg{1.0f, h2_t{0, 0}}, qu{1.0f, h2_t{0, 0}};
    if (Q8) {
      qg = qparams(k.eb, H, F, 0);
      qu = qparams(k.eb, H, F, 1);
    }
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int i = 0; i < LR; i += 2) {
      g0 = dot_piece(k.w[0][i], xo[i], qg.bias, g0);
      u0 = dot_piece(k.w[1][i], xo[i], qu.bias, u0);
      if (i + 1 < LR) {
        g1 = dot_piece(k.w[0][i + 1], xo[i + 1], qg.bias, g1);
        u1 = dot_piece(k.w[1][i + 1], xo[i + 1], qu.bias, u1);
      }
    }
    float g = wave_sum(g0 + g1), u = wave_sum(u0 + u1);
    if (Q8) {
      g *= qg.scale;
      u *= qu.scale;
    }
    if (lane == 0 && k.p >= 0) {
      const __bf16 a = (__bf16)(silu_f32(g) * u);
      uint16_t bits = __builtin_bit_cast(uint16_t, a);
      if (Q8) {  // the bf16-rounded value in fp16 (exact in fp16's normal range)
        const auto h = __builtin_amdgcn_cvt_pkrtz((float)a, 0.0f);
        bits = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
      }
      act[(size_t)k.p * F + k.f] = bits;
    }
  }
  // tasks gw, gw + NW, ... (gw < ntask), the next one's loads in flight while
  // the current one computes
  __device__ __forceinline__ void run(int gw, int NW) const {
    Task A, B;
    int t = gw;
    issue(t, A);
    for (;;) {
      const int tb = t + NW;
      issue(tb, B);
      finish(A);
      if (tb >= ntask) break;
      t = tb + NW;
      issue(t, A);
      finish(B);
      if (t >= ntask) break;
    }
  }
};

// WPE: waves per SIMD the register budget is cut for.  (Tasks of two or four
// row pairs, and two or five waves per SIMD, measured the same at the Mixtral
// width.)
template <bool Q8, int LR, int WPE>
__global__ __launch_bounds__(256, WPE) void gemv_gate_up_kernel(
    const uint8_t* __restrict__ experts, uint64_t stride_b, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ inv, int ktop, int H, int F,
    uint16_t* __restrict__ act) {
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  GuTasks<Q8, LR> gu(experts, stride_b, x, idx, inv, ktop, H, F, act);
  if (gw >= gu.ntask) return;
  gu.load_x();
  gu.run(gw, gridDim.x * 4);
}

// ------------------------------------------------------------- down + combine
// LDS of the down projection: the activation rows of the token's routed
// slots (F 16-bit values each) and the slot table, 80 KB in all, so that two
// workgroups share a CU.  The slot table holds byte offsets into the expert
// blocks, not pointers: a weight address formed from the kernel's expert
// pointer is a global load (a pointer read back from LDS would make every
// weight load a flat one, which also counts as an LDS access and holds up
// the waits for the activation reads).
constexpr int kDnMaxSlots = 8;
constexpr int kDnActElems = (80 * 1024 - 256) / 2;
struct DnLds {
  uint16_t act[kDnActElems];
  uint64_t sl_off[kDnMaxSlots];  // byte offset of the slot's down matrix in the expert blocks
  float sl_w[kDnMaxSlots];             // its gate weight
  int sl_p[kDnMaxSlots];               // its activation row
  int sl_n;
};
static_assert(sizeof(DnLds) <= 80 * 1024, "two workgroups per CU");
// the block through an LDS pointer, so that every access is a ds_ operation
typedef __attribute__((address_space(3))) DnLds* DnLdsP;
typedef __attribute__((address_space(3))) const uint16_t lds_cu16;
typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// The token's slots that reach an expert, in slot order (thread 0).
template <bool Q8, bool FOLD>
__device__ __forceinline__ void dn_slot_table(DnLdsP L, uint64_t stride_b,
                                              const int32_t* idx, const int32_t* cinv,
                                              const float* cw, int k, int H, int F) {
  constexpr int WE = Q8 ? 1 : 2;
  int v = 0;
  for (int j = 0; j < k; ++j) {
    const int p = cinv ? cinv[j] : j, e = idx[j];
    if (p < 0) continue;  // dropped by the expert capacity
    L->sl_off[v] = stride_b * e + 2 * (size_t)F * H * WE;
    L->sl_w[v] = FOLD ? cw[j] : 0.0f;
    L->sl_p[v] = p;
    ++v;
  }
  L->sl_n = v;
}

// One wave's down tasks: task = hidden row h over every routed slot, in
// chunks of CH pieces (nch chunks per row); FOLD: y[h] written here (step 5),
// else the per-slot rows yp[p][h].
template <bool Q8, int CH, bool FOLD>
struct DnTasks {
  static constexpr int WE = Q8 ? 1 : 2;
  static constexpr int V = 16 / WE;
  struct Chunk {
    u32x4 w[CH];
    int v, c;  // slot (of the nv), chunk of the row
  };
  DnLdsP L;
  const uint8_t* experts;  // (weight addresses from it: global loads)
  const uint16_t* act;
  const float* cres;
  float* cy;
  float* yp;
  int H, F, nch, nv, nseq, NW, lane;
  size_t row_b;
  float a0 = 0.f, a1 = 0.f;  // the current slot's partial sums (even / odd pieces)
  float yacc = 0.f;          // step 5 for the task's row

  __device__ __forceinline__ DnTasks(DnLdsP L_, const uint8_t* experts_, const uint16_t* act_,
                                     const float* cres_, float* cy_, float* yp_, int H_, int F_,
                                     int nch_, int NW_)
      : L(L_), experts(experts_), act(act_), cres(cres_), cy(cy_), yp(yp_), H(H_), F(F_), nch(nch_), nv(L_->sl_n),
        nseq(L_->sl_n * nch_), NW(NW_), lane((int)threadIdx.x & 63), row_b((size_t)F_ * WE) {}

  // issue chunk q of task tk (tk >= H: loads of the first weight bytes
  // instead, in bounds, never used)
  __device__ __forceinline__ void issue(int tk, int q, Chunk& ck) const {
    const uint8_t* src = experts;
    if (tk < H) {
      ck.v = q / nch;
      ck.c = q - ck.v * nch;
      src = experts + L->sl_off[ck.v] + (size_t)tk * row_b + (size_t)ck.c * CH * 1024;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) ck.w[i] = ld_nt(src + i * 1024 + lane * 16);
  }
  // next chunk of the sequence (task t, chunk q of nseq): tasks gw, gw + NW, ...
  __device__ __forceinline__ void next(int t, int q, int& t2, int& q2) const {
    q2 = q + 1;
    t2 = t;
    if (q2 == nseq) {
      q2 = 0;
      t2 = t + NW;
    }
  }
  __device__ __forceinline__ void finish(int tk, const Chunk& ck) {
    QParams qd{1.0f, h2_t{0, 0}};
    if (Q8) qd = qparams(experts + L->sl_off[ck.v] - 2 * (size_t)F * H * WE, H, F, 2);
    lds_cu16* arow = L->act + (size_t)ck.v * F + (size_t)ck.c * CH * 64 * V + lane * V;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const u32x4 xa = *(lds_cu32x4*)(arow + i * 64 * V);
      const u32x4 xb = Q8 ? *(lds_cu32x4*)(arow + i * 64 * V + 8) : xa;
      const Opnd<Q8> xo = opnd_of(xa, xb, (Opnd<Q8>*)nullptr);
      if (i & 1) a1 = dot_piece(ck.w[i], xo, qd.bias, a1);
      else a0 = dot_piece(ck.w[i], xo, qd.bias, a0);
    }
    if (ck.c + 1 < nch) return;
    float o = wave_sum(a0 + a1);
    a0 = a1 = 0.f;
    if (Q8) o *= qd.scale;
    const int h = tk;
    if (FOLD) {
      yacc = fmaf(L->sl_w[ck.v], o, yacc);
      if (ck.v + 1 == nv) {  // the row's last slot
        if (lane == 0) cy[h] = cres ? cres[h] + yacc : yacc;
        yacc = 0.f;
      }
    } else if (lane == 0) {
      yp[(size_t)L->sl_p[ck.v] * H + h] = o;
    }
  }
  // chunks A = (ta, qa) and B = (tb, qb) in flight (ta < H): finish one,
  // issue the one after the other
  __device__ __forceinline__ void run(int ta, int qa, int tb, int qb, Chunk& A, Chunk& B) {
    for (;;) {
      finish(ta, A);
      if (tb >= H) break;
      next(tb, qb, ta, qa);
      issue(ta, qa, A);
      finish(tb, B);
      if (ta >= H) break;
      next(ta, qa, tb, qb);
      issue(tb, qb, B);
    }
  }
  // no slot reached an expert: y = residual (+ nothing)
  __device__ __forceinline__ void empty(int gw) const {
    if (FOLD && lane == 0)
      for (int h = gw; h < H; h += NW) cy[h] = cres ? cres[h] + 0.0f : 0.0f;
  }
};

// The slots' activation rows to LDS, by the workgroup's 64 * WGW threads, in
// two halves: load (into registers) and store, so that loads issued in
// between stay in flight.
template <int WGW>
struct ActStage {
  static constexpr int kN = (kDnActElems / 8 + 64 * WGW - 1) / (64 * WGW);
  u32x4 r[kN];
  __device__ __forceinline__ void load(DnLdsP L, const uint16_t* act, int F) {
    const int per = F / 8, tot = L->sl_n * per;  // 16-byte pieces of one row, of all
#pragma unroll
    for (int m = 0; m < kN; ++m) {
      const int i = threadIdx.x + m * 64 * WGW;
      if (i < tot) {
        const int v = i / per;
        r[m] = reinterpret_cast<const u32x4*>(act + (size_t)L->sl_p[v] * F)[i - v * per];
      }
    }
  }
  __device__ __forceinline__ void store(DnLdsP L, int F) const {
    const int tot = L->sl_n * (F / 8);
#pragma unroll
    for (int m = 0; m < kN; ++m) {
      const int i = threadIdx.x + m * 64 * WGW;
      if (i < tot) ((lds_u32x4*)L->act)[i] = r[m];
    }
  }
};

// CH: 1 KB pieces per chunk of a down row (K = F).  WGW: waves per workgroup
// (two workgroups per CU share its LDS).  (Tasks of two or four hidden rows
// measured the same at the Mixtral width.)
template <bool Q8, int CH, int WGW, bool FOLD>
__global__ __launch_bounds__(64 * WGW, 4) void gemv_down_kernel(
    const uint8_t* __restrict__ experts, uint64_t stride_b, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ idx, int H, int F, int k, int nch,
    const float* __restrict__ cw, const int32_t* __restrict__ cinv, const float* cres, float* cy,
    float* __restrict__ yp) {
  __shared__ __attribute__((aligned(16))) DnLds Ls;
  const DnLdsP L = (DnLdsP)&Ls;
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * WGW + (threadIdx.x >> 6)));
  if (threadIdx.x == 0) dn_slot_table<Q8, FOLD>(L, stride_b, idx, cinv, cw, k, H, F);
  __syncthreads();
  DnTasks<Q8, CH, FOLD> dn(L, experts, act, cres, cy, yp, H, F, nch, gridDim.x * WGW);
  if (dn.nseq == 0) {
    dn.empty(gw);
    return;
  }
  // The activation rows' loads are issued first, then the wave's first two
  // weight chunks: waiting for the activation (the oldest loads) leaves both
  // chunks in flight.
  ActStage<WGW> stage;
  stage.load(L, act, F);
  typename DnTasks<Q8, CH, FOLD>::Chunk A, B;
  int ta = gw, qa = 0, tb, qb;
  dn.next(ta, qa, tb, qb);
  dn.issue(ta, qa, A);
  dn.issue(tb, qb, B);
  stage.store(L, F);
  __syncthreads();
  if (ta >= H) return;
  dn.run(ta, qa, tb, qb, A, B);
}

template <bool Q8, int LR, int WPE>
int launch_gu(const ExpertArgs& a, hipStream_t st) {
  const int slots = a.E < a.S ? a.E : a.S;
  const int tasks = slots * a.F;
  // WPE workgroups of four waves per CU: each wave keeps one task in flight
  // while it computes another
  int grid = cu_count() * WPE;
  if (grid * 4 > tasks) grid = (tasks + 3) / 4;
  gemv_gate_up_kernel<Q8, LR, WPE><<<grid, 256, 0, st>>>(
      (const uint8_t*)a.experts, a.stride_elems * (Q8 ? 1 : 2), (const uint16_t*)a.x, a.cidx,
      a.cinv, a.k, a.H, a.F, (uint16_t*)a.act);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool Q8, int CH, int WGW>
int launch_dn(const ExpertArgs& a, bool fold, hipStream_t st) {
  const int nch = a.F * (Q8 ? 1 : 2) / 1024 / CH;
  // 16 waves per CU (80 KB of LDS per workgroup)
  int grid = cu_count() * (16 / WGW);
  if (grid * WGW > a.H) grid = (a.H + WGW - 1) / WGW;
  auto* ex = (const uint8_t*)a.experts;
  const uint64_t sb = a.stride_elems * (Q8 ? 1 : 2);
  if (fold)
    gemv_down_kernel<Q8, CH, WGW, true><<<grid, 64 * WGW, 0, st>>>(
        ex, sb, (const uint16_t*)a.act, a.cidx, a.H, a.F, a.k, nch, a.cw, a.cinv, a.cres, a.cy,
        a.yp);
  else
    gemv_down_kernel<Q8, CH, WGW, false><<<grid, 64 * WGW, 0, st>>>(
        ex, sb, (const uint16_t*)a.act, a.cidx, a.H, a.F, a.k, nch, nullptr, a.cinv, nullptr,
        nullptr, a.yp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool Q8>
int launch_gu_q(const ExpertArgs& a, hipStream_t st) {
  switch (a.H * (Q8 ? 1 : 2) / 1024) {
    case 2: return launch_gu<Q8, 2, 4>(a, st);
    case 4: return launch_gu<Q8, 4, 4>(a, st);
    case 6: return launch_gu<Q8, 6, 2>(a, st);
    case 8: return launch_gu<Q8, 8, 2>(a, st);
    default: return -1;
  }
}

// Eight waves per workgroup (four per SIMD) and chunks of at most 8 KB:
// 7-piece chunks and 8-wave workgroups measured 2 us faster at the Mixtral
// width (both expert formats) than 14-piece chunks in 4-wave workgroups; one
// 16-wave workgroup per CU (half the activation copies) measured the same.
template <bool Q8>
int launch_dn_q(const ExpertArgs& a, bool fold, hipStream_t st) {
  const int lr = a.F * (Q8 ? 1 : 2) / 1024;
  if (lr % 14 == 0) return launch_dn<Q8, 7, 8>(a, fold, st);
  if (lr % 8 == 0) return launch_dn<Q8, 8, 8>(a, fold, st);
  if (lr % 12 == 0) return launch_dn<Q8, 6, 8>(a, fold, st);
  return launch_dn<Q8, 4, 8>(a, fold, st);
}

}  // namespace

bool gemv_supported(int T, int H, int F, int k, bool u8) {
  if (T != 1) return false;
  const int we = u8 ? 1 : 2;
  const int lr_gu = H * we / 1024, lr_dn = F * we / 1024;
  if ((H * we) % 1024 || (F * we) % 1024) return false;
  if (lr_gu != 2 && lr_gu != 4 && lr_gu != 6 && lr_gu != 8) return false;
  if (lr_dn % 14 && lr_dn % 4) return false;  // rows of 7-, 8-, 6- or 4-piece chunks
  // the activation rows of the token's slots fit the down kernel's LDS
  return k <= kDnMaxSlots && (size_t)k * F <= (size_t)kDnActElems;
}

int launch_gemv_gate_up(const ExpertArgs& a, hipStream_t st) {
  if (!gemv_supported(a.T, a.H, a.F, a.k, a.u8)) return -1;
  if (!a.experts || !a.x || !a.cidx || !a.act) return -1;
  return a.u8 ? launch_gu_q<true>(a, st) : launch_gu_q<false>(a, st);
}

int launch_gemv_down(const ExpertArgs& a, bool* combined, hipStream_t st) {
  if (!gemv_supported(a.T, a.H, a.F, a.k, a.u8)) return -1;
  if (!a.experts || !a.act || !a.cidx) return -1;
  const bool fold = combined && a.cy;
  if (fold ? !a.cw : !a.yp) return -1;
  if (combined) *combined = fold;
  return a.u8 ? launch_dn_q<true>(a, fold, st) : launch_dn_q<false>(a, fold, st);
}
