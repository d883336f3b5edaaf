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
// LR: 1 KB pieces per weight row (K = H); WPE: waves per SIMD the register
// budget is cut for.  x: the token's expert input (fp16 for uint8 experts,
// bf16 otherwise); idx, inv: its routing (slot s: expert idx[s], activation
// row inv[s]); act: [S][F] out.  (Tasks of two or four row pairs, and
// two or five waves per SIMD, measured the same at the Mixtral width.)
template <bool Q8, int LR, int WPE>
__global__ __launch_bounds__(256, WPE) void gemv_gate_up_kernel(
    const uint8_t* __restrict__ experts, uint64_t stride_b, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ inv, int ktop, int H, int F,
    uint16_t* __restrict__ act) {
  constexpr int WE = Q8 ? 1 : 2;  // bytes per weight
  constexpr int V = 16 / WE;      // weights per 16-byte piece
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int NW = gridDim.x * 4;
  // one token: its k slots reach k different experts, none beyond a capacity
  // (an expert sees at most one pair); slot s writes activation row inv[s]
  const int ntask = ktop * F;
  if (gw >= ntask) return;
  const size_t row_b = (size_t)H * WE;

  // the token's operand at this lane's K positions, all pieces
  Opnd<Q8> xo[LR];
#pragma unroll
  for (int i = 0; i < LR; ++i) {
    const uint16_t* xp = x + i * 64 * V + lane * V;
    const u32x4 a = *reinterpret_cast<const u32x4*>(xp);
    const u32x4 b = Q8 ? *reinterpret_cast<const u32x4*>(xp + 8) : a;
    xo[i] = opnd_of(a, b, (Opnd<Q8>*)nullptr);
  }

  struct Task {
    u32x4 w[2][LR];  // gate row, up row
    const uint8_t* eb;
    int p, f;
  };
  // issue the loads of task t (t >= ntask: loads of the token row instead,
  // in bounds and cached, never used)
  auto issue = [&](int t, Task& k) __attribute__((always_inline)) {
    const uint8_t* g;
    const uint8_t* u;
    if (t < ntask) {
      const int s = t / F;
      k.f = t - s * F;
      const int e = idx[s];
      k.p = inv[s];
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
  };
  auto finish = [&](const Task& k) __attribute__((always_inline)) {
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
    if (lane == 0) {
      const __bf16 a = (__bf16)(silu_f32(g) * u);
      uint16_t bits = __builtin_bit_cast(uint16_t, a);
      if (Q8) {  // the bf16-rounded value in fp16 (exact in fp16's normal range)
        const auto h = __builtin_amdgcn_cvt_pkrtz((float)a, 0.0f);
        bits = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
      }
      act[(size_t)k.p * F + k.f] = bits;
    }
  };

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

// ------------------------------------------------------------- down + combine
// LDS of the down kernel: the activation rows of the token's routed slots
// (F 16-bit values each) and the slot table, 80 KB in all, so that two
// workgroups share a CU.
constexpr int kDnMaxSlots = 8;
constexpr int kDnActElems = (80 * 1024 - 256) / 2;

// CH: 1 KB pieces per chunk of a down row (K = F); a row is nch chunks.
// WGW: waves per workgroup (two workgroups per CU share its LDS).  FOLD: y
// written here (step 5); else the per-slot rows yp[p][h].  (Tasks of two
// or four hidden rows measured the same at the Mixtral width.)
template <bool Q8, int CH, int WGW, bool FOLD>
__global__ __launch_bounds__(64 * WGW, 4) void gemv_down_kernel(
    const uint8_t* __restrict__ experts, uint64_t stride_b, const uint16_t* __restrict__ act,
    const int32_t* __restrict__ idx, int H, int F, int k, int nch,
    const float* __restrict__ cw, const int32_t* __restrict__ cinv, const float* cres, float* cy,
    float* __restrict__ yp) {
  constexpr int WE = Q8 ? 1 : 2;
  constexpr int V = 16 / WE;
  __shared__ __attribute__((aligned(16))) uint16_t act_lds[kDnActElems];
  __shared__ const uint8_t* sl_row[kDnMaxSlots];  // down matrix of the slot's expert
  __shared__ float sl_w[kDnMaxSlots];             // its gate weight
  __shared__ int sl_p[kDnMaxSlots];               // its activation row
  __shared__ int sl_n;
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * WGW + (threadIdx.x >> 6)));
  const int NW = gridDim.x * WGW;
  const int ntask = H;  // one hidden row per task
  const size_t row_b = (size_t)F * WE;

  if (threadIdx.x == 0) {  // the token's slots that reach an expert, in slot order
    int v = 0;
    for (int j = 0; j < k; ++j) {
      const int p = cinv[j], e = idx[j];
      if (p < 0) continue;  // dropped by the expert capacity
      sl_row[v] = experts + stride_b * e + 2 * (size_t)F * H * WE;
      sl_w[v] = FOLD ? cw[j] : 0.0f;
      sl_p[v] = p;
      ++v;
    }
    sl_n = v;
  }
  __syncthreads();
  const int nv = sl_n;
  const int nseq = nv * nch;  // chunks per task
  if (nseq == 0) {  // no slot reached an expert: y = residual (+ nothing)
    if (FOLD && lane == 0)
      for (int h = gw; h < H; h += NW) cy[h] = cres ? cres[h] + 0.0f : 0.0f;
    return;
  }

  struct Chunk {
    u32x4 w[CH];
    int v, c;  // slot (of the nv), chunk of the row
  };
  // issue chunk q of task tk (tk >= ntask: loads of the first activation
  // row instead, in bounds and cached, never used)
  auto issue = [&](int tk, int q, Chunk& ck) __attribute__((always_inline)) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(act);
    if (tk < ntask) {
      ck.v = q / nch;
      ck.c = q - ck.v * nch;
      src = sl_row[ck.v] + (size_t)tk * row_b + (size_t)ck.c * CH * 1024;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) ck.w[i] = ld_nt(src + i * 1024 + lane * 16);
  };

  // next chunk of the sequence (task t, chunk q of nseq) of this wave: tasks
  // gw, gw + NW, ...
  auto next = [&](int t, int q, int& t2, int& q2) __attribute__((always_inline)) {
    q2 = q + 1;
    t2 = t;
    if (q2 == nseq) {
      q2 = 0;
      t2 = t + NW;
    }
  };
  // The slots' activation rows go to LDS.  Their loads are issued first, then
  // the wave's first two weight chunks: waiting for the activation (the
  // oldest loads) leaves both chunks in flight.
  constexpr int kStage = (kDnActElems / 8 + 64 * WGW - 1) / (64 * WGW);
  const int per = F / 8, tot = nv * per;  // 16-byte pieces of one row, of all
  u32x4 stage[kStage];
#pragma unroll
  for (int m = 0; m < kStage; ++m) {
    const int i = threadIdx.x + m * 64 * WGW;
    if (i < tot) {
      const int v = i / per;
      stage[m] = reinterpret_cast<const u32x4*>(act + (size_t)sl_p[v] * F)[i - v * per];
    }
  }
  Chunk A, B;
  int ta = gw, qa = 0, tb, qb;
  next(ta, qa, tb, qb);
  issue(ta, qa, A);
  issue(tb, qb, B);
#pragma unroll
  for (int m = 0; m < kStage; ++m) {
    const int i = threadIdx.x + m * 64 * WGW;
    if (i < tot) reinterpret_cast<u32x4*>(act_lds)[i] = stage[m];
  }
  __syncthreads();
  if (ta >= ntask) return;

  float a0 = 0.f, a1 = 0.f;  // the current slot's partial sums (even / odd pieces)
  float yacc = 0.f;          // step 5 for the task's row
  auto finish = [&](int tk, const Chunk& ck) __attribute__((always_inline)) {
    QParams qd{1.0f, h2_t{0, 0}};
    if (Q8) qd = qparams(sl_row[ck.v] - 2 * (size_t)F * H * WE, H, F, 2);
    const uint16_t* arow = act_lds + (size_t)ck.v * F + (size_t)ck.c * CH * 64 * V + lane * V;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(arow + i * 64 * V);
      const u32x4 xb = Q8 ? *reinterpret_cast<const u32x4*>(arow + i * 64 * V + 8) : xa;
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
      yacc = fmaf(sl_w[ck.v], o, yacc);
      if (ck.v + 1 == nv) {  // the row's last slot
        if (lane == 0) cy[h] = cres ? cres[h] + yacc : yacc;
        yacc = 0.f;
      }
    } else if (lane == 0) {
      yp[(size_t)sl_p[ck.v] * H + h] = o;
    }
  };

  // two chunks in flight: finish one, issue the one after the other
  for (;;) {
    finish(ta, A);
    if (tb >= ntask) break;
    next(tb, qb, ta, qa);
    issue(ta, qa, A);
    finish(tb, B);
    if (ta >= ntask) break;
    next(ta, qa, tb, qb);
    issue(tb, qb, B);
  }
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
  if (!a.experts || !a.x || !a.cidx || !a.cinv || !a.act) return -1;
  return a.u8 ? launch_gu_q<true>(a, st) : launch_gu_q<false>(a, st);
}

int launch_gemv_down(const ExpertArgs& a, bool* combined, hipStream_t st) {
  if (!gemv_supported(a.T, a.H, a.F, a.k, a.u8)) return -1;
  if (!a.experts || !a.act || !a.cidx || !a.cinv) return -1;
  const bool fold = combined && a.cy;
  if (fold ? !a.cw : !a.yp) return -1;
  if (combined) *combined = fold;
  return a.u8 ? launch_dn_q<true>(a, fold, st) : launch_dn_q<false>(a, fold, st);
}
