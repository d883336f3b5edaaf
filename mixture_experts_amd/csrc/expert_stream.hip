// expert_stream.hip -- steps 4 and 5 when each expert sees few rows (decode
// batches, many small experts): the weights of every expert that received at
// least one row are streamed from HBM exactly once.
//
// Same SwiGLU expert as the grouped path [zskr.cn/news/2275853
// "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1, sec. 3.3 stage 4];
// experts are addressed as base + id * stride inside one contiguous buffer
// [www.lmnt.cn/news/246575 sec. 2.1].
//
// Work item: one non-empty expert x 16 output rows (gate AND up rows
// f0..f0+15 for the first kernel, 32 weight rows; down rows h0..h0+15 for the
// second, h0..h0+63 when a pass covers 32 token rows), over all of the
// expert's token rows in passes of TR.  The grid is
// persistent: workgroup b takes items b, b + G, b + 2G, ... and treats the
// K chunks of all its items as one sequence.  A chunk is CK (512, 256 or
// 128, as K allows) K elements: the 2 CK-byte run of every
// weight row and of every token row of the pass.  It reaches LDS through
// direct global->LDS loads, weight rows as non-temporal 1 KB loads of
// 1024 / (2 CK) row runs each; a ring of NS chunk stages keeps NS-1
// chunks in flight, across item boundaries, so HBM sees long runs and never
// waits for an item's epilogue.  MFMA v_mfma_f32_16x16x32_bf16 with weight
// rows as A and token rows as B; each of the 4 waves takes a quarter of the
// 32-wide K steps of a chunk, and the four partial sums are added in LDS in
// a fixed order (deterministic) before the gate/up epilogue applies SiLU(g)*u
// and stores bf16, or the down epilogue stores fp32 rows for the combine.
//
// uint8 experts (weights (q - zero) * scale, one map per matrix
// [www.pnsm.cn/news/1892388.html sec. 3.1 and sec. 5.2]): the weight runs
// hold one byte per weight, and an item is 16, 32 or 64 weight rows (QNA
// blocks of 16) as the batch size suits.  In registers each group of 4
// codes becomes two fp16 pairs by a byte permute with 0x64 (fp16 1024 + q)
// and one packed fp16 add of -(1024 + zero), exactly (q - zero).  The token
// rows arrive in fp16: the layer input is copied to fp16 before the gate/up
// kernel (by the small-batch route itself, else by a conversion kernel), and
// that kernel's epilogue stores the bf16-rounded activation as fp16 (bf16
// values in fp16's normal range are fp16 values).  The MFMA is
// v_mfma_f32_16x16x32_f16 and the scale multiplies the reduced sums once
// per output.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace {


// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(h8_t a, h8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 uint8 codes -> 8 fp16 values q - zero (bias = -(1024 + zero) in both
// halves): byte permute of each code under the constant byte 0x64 gives the
// fp16 value 1024 + q, exactly, and one packed add subtracts 1024 + zero.
__device__ __forceinline__ h8_t dequant8(uint2 w, h2_t bias) {
  constexpr uint32_t k64 = 0x64646464u;
  const h2_t p0 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(k64, w.x, 0x04010400u)) + bias;
  const h2_t p1 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(k64, w.x, 0x04030402u)) + bias;
  const h2_t p2 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(k64, w.y, 0x04010400u)) + bias;
  const h2_t p3 = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(k64, w.y, 0x04030402u)) + bias;
  return h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Wait until a wave's loads of its oldest chunk in flight have landed: of
// `ahead` chunks issued (at most A), the PER loads of each of the ahead - 1
// younger ones may stay outstanding (loads complete in order).
template <int PER, int A>
__device__ __forceinline__ void wait_chunk(int ahead) {
  if constexpr (A <= 1) {
    WAIT_VMCNT(0);
  } else {
    if (ahead >= A) WAIT_VMCNT((A - 1) * PER);
    else wait_chunk<PER, A - 1>(ahead);
  }
}

// One LDS row run holds its chunks of 16 bytes with chunk c of run r at slot
// c ^ (r % SPR) (SPR = chunks per run, at most 16), so the 16 lanes of an
// MFMA operand read (16 runs, one chunk) spread over the bank groups.
template <int SPR>
__device__ __forceinline__ int run_slot(int r, int c) { return c ^ (r & ((SPR < 16 ? SPR : 16) - 1)); }

// FC (down projection only): the items of one 16-row hidden slice, every
// non-empty expert's, run back to back in one workgroup, which keeps their
// outputs in LDS and then writes y for that slice (step 5, the combine's
// arithmetic in the combine's order) instead of storing per-row outputs.
template <bool GATED, bool Q8, int QNA, int TR, int NS, int CK, bool FC = false>
__global__ __launch_bounds__(256) void stream_kernel(
    const uint8_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active, int E, int H,
    int F, int T, void* __restrict__ out, const float* __restrict__ cw,
    const int32_t* __restrict__ cinv, const float* cres, float* cy) {
  constexpr int WE = Q8 ? 1 : 2;                // bytes per weight
  constexpr int NA = (Q8 || !GATED) ? QNA : 2;  // weight row blocks of 16 per item
  constexpr int WR = 16 * NA;                   // weight rows per item
  constexpr int OB = GATED ? NA / 2 : NA;       // output row blocks of 16 per item
  constexpr int NB = (TR + 15) / 16;            // token column blocks of the MFMA
  constexpr int RBW = WE * CK, RBT = 2 * CK;    // bytes per weight / token row run
  constexpr int SPRW = RBW / 16, SPRT = RBT / 16;  // 16-byte slots per run
  constexpr int RPIW = 64 / SPRW, RPIT = 64 / SPRT;  // runs per 1 KB load
  constexpr int IW = WR / RPIW / 4;             // weight loads per wave per chunk
  constexpr int IT = TR / RPIT / 4;             // token loads per wave per chunk
  constexpr int KSW = CK / 32 / 4;              // 32-wide K steps per wave per chunk
  constexpr int STAGE = WR * RBW + TR * RBT;
  static_assert((CK == 128 || CK == 256 || CK == 512) && IT >= 1 && TR % (4 * RPIT) == 0 &&
                    IW >= 1 && WR % (4 * RPIW) == 0,
                "chunk width and token rows per pass");
  static_assert(NS >= 2 && NS <= 8 && (NS - 2) * (IW + IT) <= 63, "ring depth");
  // the waves' partial sums at the end of a pass, [4 waves][NA*NB][64 lanes],
  // in the ring stage just computed when it is large enough
  constexpr int RED = 4 * NA * NB * 64;
  constexpr bool RED_IN_RING = RED * 16 <= STAGE;
  static_assert(!FC || (!GATED && WR == 16), "combine folded into 16-row down items");
  // one LDS block: the ring of NS stages, then the partial sums when a stage
  // cannot hold them, then (FC) the down outputs of the slice, [pair t*k + j]
  // [16 rows], pairs < 256; nothing else, so that the launch's occupancy
  // arithmetic is exact
  constexpr int LDS_BYTES = NS * STAGE + (RED_IN_RING ? 0 : RED * 16) + (FC ? 256 * 16 * 4 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  uint8_t (*const ring)[STAGE] = reinterpret_cast<uint8_t (*)[STAGE]>(smem);
  f32x4* const red_own = reinterpret_cast<f32x4*>(smem + NS * STAGE);
  f32x4* const comb =
      reinterpret_cast<f32x4*>(smem + NS * STAGE + (RED_IN_RING ? 0 : RED * 16));

  const int K = GATED ? H : F;
  const int NWT = GATED ? F / (16 * OB) : H / WR;
  const int NC = K / CK;
  const int n_act = active[E];
  const int n_items = n_act * NWT;
  const int G = gridDim.x;
  // item j of this workgroup: (expert slot, weight row block); without FC
  // items are numbered slot-major and dealt round-robin, with FC the
  // workgroup takes hidden slices b, b + G, ... with every slot of each
  auto item_of = [&](int j, int& slot, int& wt) -> bool {
    if (FC) {
      if (n_act <= 0) return false;
      const int q = j / n_act;
      slot = j - q * n_act;
      wt = blockIdx.x + q * G;
      return wt < NWT;
    }
    const int item = blockIdx.x + j * G;
    slot = item / NWT;
    wt = item - slot * NWT;
    return item < n_items;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- the load cursor: (item j of this workgroup, token pass, chunk) ----
  int l_j = 0, l_pass = 0, l_c = 0, l_npass = 0;
  bool l_ok = false;
  const uint8_t* wsrc[IW];
  const uint16_t* tsrc[IT];
  auto l_item = [&]() {  // sets l_ok, l_npass and the weight sources for item l_j
    int slot, wt;
    l_ok = item_of(l_j, slot, wt);
    if (!l_ok) return;
    const int e = active[slot];
    const int n_e = offsets[e + 1] - offsets[e];
    l_npass = (n_e + TR - 1) / TR;
    const uint8_t* eb = experts + (size_t)stride_elems * WE * e;
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const int r = (wave * IW + i) * RPIW + lane / SPRW;  // weight row of the item
      size_t w;  // weight index of the row's first element
      if (GATED)  // rows 0 .. 16 OB - 1 gate, then the same f rows of up
        w = (size_t)(r < 16 * OB ? 0 : F) * H + (size_t)(wt * 16 * OB + r % (16 * OB)) * H;
      else
        w = 2 * (size_t)F * H + (size_t)(wt * WR + r) * F;
      wsrc[i] = eb + w * WE + run_slot<SPRW>(r, lane % SPRW) * 16;
    }
  };
  // token sources of pass l_pass of item l_j.  Each load covers RPIT token
  // rows; their indices are read with scalar loads (uniform addresses), so
  // no vector load the compiler would have to wait for joins the loads in
  // flight.
  auto l_pass_rows = [&]() {
    int slot, wt;
    (void)item_of(l_j, slot, wt);
    const int e = active[slot];
    const int p_beg = offsets[e], n_e = offsets[e + 1] - p_beg;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int r0 = (wave * IT + i) * RPIT;  // token rows r0 .. r0 + RPIT - 1 of the pass
      int xr = 0;
#pragma unroll
      for (int u = 0; u < RPIT; ++u) {
        const int p = p_beg + min(l_pass * TR + r0 + u, n_e - 1);
        const int x = GATED ? min(max(perm[p], 0) / k_top, T - 1) : p;
        if (lane / SPRT == u) xr = x;
      }
      tsrc[i] = tok + (size_t)xr * K + run_slot<SPRT>(r0 + lane / SPRT, lane % SPRT) * 8;
    }
  };
  // issue the chunk under the load cursor into stage st, then advance it
  auto l_issue = [&](int st) {
    const uint32_t base =
        (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)&ring[st][0]);
    const int k0 = l_c * CK;
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const uint32_t dst = base + (uint32_t)((wave * IW + i) * RPIW * RBW);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(wsrc[i] + k0 * WE)
                   : "memory", "m0");
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t dst = base + (uint32_t)(WR * RBW + (wave * IT + i) * RPIT * RBT);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(tsrc[i] + k0)
                   : "memory", "m0");
    }
    if (++l_c == NC) {
      l_c = 0;
      if (++l_pass == l_npass) {
        l_pass = 0;
        ++l_j;
        l_item();
      }
      if (l_ok) l_pass_rows();
    }
  };

  // ---- the compute cursor ----
  int c_j = 0, c_pass = 0, c_c = 0;
  int c_wt = 0, c_pbeg = 0, c_ne = 0, c_npass = 0;
  bool c_ok = false;
  float c_scale[NA];  // uint8 experts: scale of each weight row block
  h2_t c_bias[NA];    // and -(1024 + zero point) for the dequantisation
  auto c_item = [&]() {
    int slot;
    c_ok = item_of(c_j, slot, c_wt);
    if (!c_ok) return;
    const int e = active[slot];
    c_pbeg = offsets[e];
    c_ne = offsets[e + 1] - c_pbeg;
    c_npass = (c_ne + TR - 1) / TR;
    if (Q8) {  // parameter block after the three matrices: scale[3], zero[3]
      const uint8_t* pb = experts + (size_t)stride_elems * e + 3 * (size_t)F * H;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int m = GATED ? (i < OB ? 0 : 1) : 2;
        c_scale[i] = reinterpret_cast<const float*>(pb)[m];
        const _Float16 b = (_Float16)(-(1024 + reinterpret_cast<const int32_t*>(pb)[3 + m]));
        c_bias[i] = h2_t{b, b};
      }
    }
  };

  if (FC && n_act <= 0) {  // no pair reached an expert: y = resid (+ nothing)
    for (int wt = blockIdx.x; wt < NWT; wt += G)
      for (int u = threadIdx.x; u < T * 16; u += 256) {
        const size_t o = (size_t)(u >> 4) * H + wt * 16 + (u & 15);
        cy[o] = cres ? cres[o] + 0.0f : 0.0f;
      }
    return;
  }
  l_item();
  if (l_ok) l_pass_rows();
  c_item();
  // prologue: chunks 0 .. NS-2 of the sequence
  int ahead = 0;  // chunks issued and not yet computed
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (l_ok) {
      l_issue(s);
      ++ahead;
    }

  f32x4 acc[NA][NB];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, kg = lane >> 4;

  int st = 0;  // stage of the chunk being computed
  while (c_ok) {
    // this wave's loads of the current chunk have landed once at most the
    // loads of the (ahead - 1) younger chunks are outstanding
    wait_chunk<IW + IT, NS - 1>(ahead);
    // publishes the chunk, and ends every wave's reads of the previous one
    asm volatile("s_barrier" ::: "memory");
    --ahead;
    if (l_ok) {
      l_issue(st == 0 ? NS - 1 : st - 1);  // the previous chunk's stage
      ++ahead;
    }
    // K steps KSW wave .. KSW wave + KSW - 1 of the chunk
    const uint8_t* sb = &ring[st][0];
#pragma unroll
    for (int s2 = 0; s2 < KSW; ++s2) {
      const int c = (wave * KSW + s2) * 4 + kg;  // group of 8 K elements in the run
      using op_t = typename std::conditional<Q8, h8_t, bf16x8>::type;
      op_t a[NA], b[NB];
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int r = i * 16 + r16;
        if constexpr (Q8) {  // 8 bytes: half of 16-byte chunk c / 2
          const uint2 w8 = *reinterpret_cast<const uint2*>(sb + r * RBW +
                                                           run_slot<SPRW>(r, c >> 1) * 16 + (c & 1) * 8);
          a[i] = dequant8(w8, c_bias[i]);
        } else {
          a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(sb + r * RBW + run_slot<SPRW>(r, c) * 16));
        }
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        // token columns beyond TR read row 0 again; their results are dropped
        const int r = n * 16 + r16 < TR ? n * 16 + r16 : 0;
        const u32x4 v =
            *reinterpret_cast<const u32x4*>(sb + WR * RBW + r * RBT + run_slot<SPRT>(r, c) * 16);
        if constexpr (Q8) b[n] = __builtin_bit_cast(h8_t, v);  // fp16 token rows
        else b[n] = as_bf16x8(v);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int i = 0; i < NA; ++i) acc[i][n] = mfma16(a[i], b[n], acc[i][n]);
    }
    const int cst = st;  // the stage just computed
    st = st == NS - 1 ? 0 : st + 1;

    if (++c_c == NC) {  // end of a token pass: reduce the 4 K partial sums
      c_c = 0;
      f32x4* red = RED_IN_RING ? reinterpret_cast<f32x4*>(&ring[cst][0]) : red_own;
      // every wave's reads of that stage are done (its next loads are issued
      // only after the next chunk barrier, when the sums below have been read)
      if (RED_IN_RING) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          red[(wave * NA * NB + i * NB + n) * 64 + lane] = acc[i][n];
          acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      // LDS writes done, then the barrier; no wait on the loads in flight
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // 16x16 accumulator layout: lane l holds token column l%16 and weight
      // rows 4*(l/16) + j.  Thread (n, l) sums the waves' partials in order.
      if (threadIdx.x < NB * 64) {
        const int n = threadIdx.x >> 6, l = threadIdx.x & 63;
        const int col = n * 16 + (l & 15);
        const int t = c_pass * TR + col;
        if (col < TR && t < c_ne) {
          const int p = c_pbeg + t;
          const int r0 = c_wt * 16 * OB + 4 * (l >> 4);
          auto block = [&](int i) {  // the waves' partials of row block i, in wave order
            constexpr int WS = NA * NB * 64;  // one wave's partials
            const int o = (i * NB + n) * 64 + l;
            f32x4 v = red[o];
            v += red[WS + o];
            v += red[2 * WS + o];
            v += red[3 * WS + o];
            if (Q8) v *= c_scale[i];
            return v;
          };
#pragma unroll
          for (int i = 0; i < OB; ++i) {
            const f32x4 g = block(i);
            if (GATED) {
              const f32x4 u = block(OB + i);
              const bf16x2 lo = {(__bf16)(silu_f32(g[0]) * u[0]), (__bf16)(silu_f32(g[1]) * u[1])};
              const bf16x2 hi = {(__bf16)(silu_f32(g[2]) * u[2]), (__bf16)(silu_f32(g[3]) * u[3])};
              uint2 pk;
              pk.x = __builtin_bit_cast(uint32_t, lo);
              pk.y = __builtin_bit_cast(uint32_t, hi);
              if (Q8) {  // the bf16-rounded activation, stored as fp16 for the down kernel
                pk.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                    __uint_as_float(pk.x << 16), __uint_as_float(pk.x & 0xFFFF0000u)));
                pk.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                    __uint_as_float(pk.y << 16), __uint_as_float(pk.y & 0xFFFF0000u)));
              }
              *reinterpret_cast<uint2*>((uint16_t*)out + (size_t)p * F + r0 + 16 * i) = pk;
            } else if (FC) {  // pair perm[p], rows 4 (l / 16) .. + 3 of the slice
              comb[(perm[p] * 16 + 4 * (l >> 4)) >> 2] = g;
            } else {
              *reinterpret_cast<f32x4*>((float*)out + (size_t)p * H + r0 + 16 * i) = g;
            }
          }
        }
      }
      // red is written again only after at least one more chunk barrier
      if (++c_pass == c_npass) {
        c_pass = 0;
        const int wt_done = c_wt;
        ++c_j;
        c_item();
        if (FC && (!c_ok || c_wt != wt_done)) {
          // every expert's rows of slice wt_done are in comb: y for the slice,
          // y[t] = (resid[t] +) sum_j w[t][j] * out_j in slot order, pairs
          // dropped by the capacity (slot -1) skipped
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          const float* cs = reinterpret_cast<const float*>(comb);
          const int h0 = wt_done * 16;
          for (int u = threadIdx.x; u < T * 16; u += 256) {
            const int t = u >> 4, hh = u & 15;
            float acc = 0.0f;
            for (int j = 0; j < k_top; ++j) {
              if (cinv[t * k_top + j] < 0) continue;
              acc = fmaf(cw[t * k_top + j], cs[(t * k_top + j) * 16 + hh], acc);
            }
            const size_t o = (size_t)t * H + h0 + hh;
            cy[o] = cres ? cres[o] + acc : acc;
          }
          // comb is written again only after at least one more chunk barrier
        }
      }
    }
  }
  WAIT_VMCNT(0);
}

template <bool GATED, bool Q8, int QNA, int TR, int NS, int CK>
int launch_tr(const ExpertArgs& a, hipStream_t st, bool* combined = nullptr) {
  constexpr int NA = (Q8 || !GATED) ? QNA : 2, NB = (TR + 15) / 16;
  constexpr int OB = GATED ? NA / 2 : NA;
  constexpr int stage = (16 * NA * (Q8 ? 1 : 2) + TR * 2) * CK, red = 4 * NA * NB * 64 * 16;
  constexpr int lds = NS * stage + (red <= stage ? 0 : red);
  const int nwt = GATED ? a.F / (16 * OB) : a.H / (16 * NA);
  const int slots = a.E < a.S ? a.E : a.S;
  const uint16_t* tok = GATED ? (const uint16_t*)a.x : (const uint16_t*)a.act;
  const int per_cu = (160 * 1024) / lds;
  int grid = cu_count() * (per_cu < 1 ? 1 : per_cu);
  if (grid > nwt * slots) grid = nwt * slots;
  // the down projection folds the combine in when the slice's outputs of all
  // T*k pairs fit the LDS buffer and one workgroup per 16-row hidden slice is
  // as many workgroups as the plain launch would run (then no CU idles)
  if constexpr (!GATED && NA == 1) {
    constexpr int lds_fc = lds + 256 * 16 * 4;
    const int grid_fc = nwt < cu_count() * ((160 * 1024) / lds_fc) ? nwt
                                                                   : cu_count() * ((160 * 1024) / lds_fc);
    if (combined && a.cy && a.S <= 256 && lds_fc <= 160 * 1024 && grid_fc >= grid) {
      stream_kernel<GATED, Q8, QNA, TR, NS, CK, true><<<grid_fc, 256, 0, st>>>(
          (const uint8_t*)a.experts, a.stride_elems, tok, a.perm, a.k, a.offsets, a.active, a.E,
          a.H, a.F, a.T, nullptr, a.cw, a.cinv, a.cres, a.cy);
      *combined = true;
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  void* out = GATED ? a.act : (void*)a.yp;
  stream_kernel<GATED, Q8, QNA, TR, NS, CK><<<grid, 256, 0, st>>>(
      (const uint8_t*)a.experts, a.stride_elems, tok, a.perm, a.k, a.offsets, a.active, a.E,
      a.H, a.F, a.T, out, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <bool GATED, bool Q8>
int launch_stream_q(const ExpertArgs& a, hipStream_t st, bool* combined) {
  // token rows per pass (experts with more rows take several passes) and the
  // chunk width: 512 for batches of up to 8 rows per expert (16 for the down
  // projection), else 256 when K allows it (bf16 layers have H % 256 == 0
  // and F % 128 == 0), else 128
  const int rows = a.rows_hint;
  const int K = GATED ? a.H : a.F;
  if constexpr (Q8) {
    // uint8 weights: a chunk holds half the bytes of a bf16 one, so batches
    // take items of 64 weight rows (the bytes of a bf16 item); the down
    // projection of single tokens keeps 16-row items so that every
    // workgroup has one, with a deeper ring
    if (K % 512 == 0) {
      if (GATED) {
        if (rows <= 8) return launch_tr<GATED, Q8, 4, 8, 3, 256>(a, st, combined);
        if (rows <= 16) return launch_tr<GATED, Q8, 4, 16, 2, 256>(a, st, combined);
      } else {
        if (rows <= 2) return launch_tr<GATED, Q8, 1, 8, 4, 512>(a, st, combined);
        if (rows > 8 && rows <= 16) return launch_tr<GATED, Q8, 4, 16, 2, 256>(a, st, combined);
      }
      if (rows > 16) return launch_tr<GATED, Q8, 4, 32, 2, 256>(a, st, combined);
    }
  }
  // bf16 down items: one 16-row block (A1) while a pass covers up to 16
  // token rows; at 32 token rows a 16-row item would load twice as many
  // token bytes as weight bytes per chunk, so items take 64 rows (A4).
  // (bf16 gate/up items stay at 16 gate + 16 up rows: two workgroups per
  // CU at 32 token rows were faster than one with 32 + 32-row items.)
  constexpr int A1 = (GATED || Q8) ? 2 : 1, A4 = (GATED || Q8) ? 2 : 4;
  if (GATED && K % 512 == 0 && rows <= 8)  // 1 KB row runs, one deep ring per CU
    return launch_tr<GATED, Q8, 2, 8, 3, 512>(a, st, combined);
  if (!GATED && K % 512 == 0 && rows <= 16) {  // down: 1 KB row runs
    if (rows <= 8) return launch_tr<GATED, Q8, A1, 8, Q8 ? 3 : 4, 512>(a, st, combined);
    return launch_tr<GATED, Q8, A1, 16, 3, 512>(a, st, combined);
  }
  if (K % 256 == 0) {
    if (rows <= 8) return launch_tr<GATED, Q8, A1, 8, GATED ? 3 : 4, 256>(a, st, combined);
    if (rows <= 16) return launch_tr<GATED, Q8, A1, 16, GATED ? 3 : 4, 256>(a, st, combined);
    return launch_tr<GATED, Q8, A4, 32, GATED ? 2 : 3, 256>(a, st, combined);
  }
  if (rows <= 16) return launch_tr<GATED, Q8, A1, 16, 4, 128>(a, st, combined);
  return launch_tr<GATED, Q8, A4, 32, GATED ? 3 : 4, 128>(a, st, combined);
}

template <bool GATED>
int launch_stream(const ExpertArgs& a, hipStream_t st, bool* combined) {
  if (combined) *combined = false;
  return a.u8 ? launch_stream_q<GATED, true>(a, st, combined)
              : launch_stream_q<GATED, false>(a, st, combined);
}

}  // namespace

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int launch_stream_gate_up(const ExpertArgs& a, hipStream_t st) {
  return launch_stream<true>(a, st, nullptr);
}
int launch_stream_down(const ExpertArgs& a, bool* combined, hipStream_t st) {
  return launch_stream<false>(a, st, combined);
}
