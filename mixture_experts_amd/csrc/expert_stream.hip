// expert_stream.hip -- steps 4 and 5 when each expert sees few rows (decode
// batches, many small experts): the weights of every expert that received at
// least one row are streamed from HBM exactly once, straight into registers.
//
// Same SwiGLU expert as the grouped path [zskr.cn/news/2275853
// "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1, sec. 3.3 stage 4];
// experts are addressed as base + id * stride inside one contiguous buffer
// [www.lmnt.cn/news/246575 sec. 2.1].
//
// Work unit: one non-empty expert x 16 weight rows (gate AND up rows f0..f0+15
// for the first kernel; down rows h0..h0+15 for the second), all of the
// expert's token rows in passes of NB*16.  The 4 waves split the K dimension;
// lanes load 16 bytes each, four lanes covering 64 contiguous bytes of a row
// per instruction, with 8 (gate: 16) loads per lane in flight per batch of 8
// MFMA steps; the token rows (L2-resident) use the same lane -> K mapping.  MFMA:
// v_mfma_f32_16x16x32_bf16 with weight rows as A and tokens as B.  The four
// K partial sums are added in LDS in a fixed order (deterministic), then the
// gate/up kernel applies SiLU(g)*u and stores the activation in bf16; the
// down kernel stores fp32 rows for the fixed-order combine.
#include "common.h"
#include "kernels.h"

namespace {

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <bool GATED, int NB>
__global__ __launch_bounds__(256) void stream_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active, int E, int H,
    int F, int T, void* __restrict__ out) {
  constexpr int NA = GATED ? 2 : 1;
  __shared__ f32x4 red[4][NA * NB][64];

  const int K = GATED ? H : F;
  const int NWT = (GATED ? F : H) / 16;
  const int slot = blockIdx.x / NWT;
  const int wt = blockIdx.x - slot * NWT;
  if (slot >= active[E]) return;
  const int e = active[slot];
  const int p_beg = offsets[e];
  const int n_e = offsets[e + 1] - p_beg;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const uint16_t* eb = experts + (size_t)e * stride_elems;
  const uint16_t* wa;
  const uint16_t* wu = nullptr;
  if (GATED) {
    wa = eb + (size_t)(wt * 16 + r16) * H;
    wu = eb + (size_t)F * H + (size_t)(wt * 16 + r16) * H;
  } else {
    wa = eb + 2 * (size_t)F * H + (size_t)(wt * 16 + r16) * F;
  }
  const int nsteps = K / 32;
  const int s_beg = wave * nsteps / 4, s_end = (wave + 1) * nsteps / 4;

  for (int pass0 = 0; pass0 < n_e; pass0 += NB * 16) {
    f32x4 acc[NA][NB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* brow[NB];
    bool bok[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int t = pass0 + n * 16 + r16;
      bok[n] = t < n_e;
      const int p = p_beg + (bok[n] ? t : 0);
      brow[n] = GATED ? tok + (size_t)min(max(perm[p], 0) / k_top, T - 1) * H : tok + (size_t)p * F;
    }
    // MFMA step s covers k in [32 s, 32 s + 32); lane group kg holds
    // k = 32 s + 8 kg .. +7, so one load instruction reads 64 contiguous
    // bytes of each of the 16 rows.  Steps go in batches of 8 so that 8 (or
    // 16) weight loads per lane are in flight before the first MFMA.
    int s = s_beg;
    for (; s + 8 <= s_end; s += 8) {
      u32x4 va[8], vu[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kb = (s + q) * 32 + kg * 8;
        va[q] = ldg16(wa + kb);
        if (GATED) vu[q] = ldg16(wu + kb);
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        u32x4 vb[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          vb[q] = bok[n] ? ldg16(brow[n] + (s + q) * 32 + kg * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          acc[0][n] = mfma16(va[q], vb[q], acc[0][n]);
          if (GATED) acc[NA - 1][n] = mfma16(vu[q], vb[q], acc[NA - 1][n]);
        }
      }
    }
    for (; s < s_end; ++s) {
      const int kb = s * 32 + kg * 8;
      const u32x4 va = ldg16(wa + kb);
      u32x4 vu = u32x4{0u, 0u, 0u, 0u};
      if (GATED) vu = ldg16(wu + kb);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const u32x4 vb = bok[n] ? ldg16(brow[n] + kb) : u32x4{0u, 0u, 0u, 0u};
        acc[0][n] = mfma16(va, vb, acc[0][n]);
        if (GATED) acc[NA - 1][n] = mfma16(vu, vb, acc[NA - 1][n]);
      }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int n = 0; n < NB; ++n) red[wave][i * NB + n][lane] = acc[i][n];
    __syncthreads();
    // 16x16 accumulator layout: lane l holds token column l%16 and weight
    // rows 4*(l/16) + j.  Thread (n, l) sums the four K quarters in order.
    if (tid < NB * 64) {
      const int n = tid >> 6, l = tid & 63;
      const int t = pass0 + n * 16 + (l & 15);
      if (t < n_e) {
        const int p = p_beg + t;
        const int r0 = wt * 16 + 4 * (l >> 4);
        f32x4 g = red[0][n][l];
        g += red[1][n][l];
        g += red[2][n][l];
        g += red[3][n][l];
        if (GATED) {
          f32x4 u = red[0][NB + n][l];
          u += red[1][NB + n][l];
          u += red[2][NB + n][l];
          u += red[3][NB + n][l];
          uint2 pk;
          pk.x = pack_bf16x2(silu_f32(g[0]) * u[0], silu_f32(g[1]) * u[1]);
          pk.y = pack_bf16x2(silu_f32(g[2]) * u[2], silu_f32(g[3]) * u[3]);
          *reinterpret_cast<uint2*>((uint16_t*)out + (size_t)p * F + r0) = pk;
        } else {
          *reinterpret_cast<f32x4*>((float*)out + (size_t)p * H + r0) = g;
        }
      }
    }
    __syncthreads();
  }
}

template <bool GATED>
int launch_stream(const ExpertArgs& a, hipStream_t st) {
  const int nwt = (GATED ? a.F : a.H) / 16;
  const int slots = a.E < a.S ? a.E : a.S;
  const int grid = nwt * slots;
  // token passes of NB*16 rows; experts with more rows take several passes
  const int rows = a.rows_hint;
  const uint16_t* tok = GATED ? (const uint16_t*)a.x : (const uint16_t*)a.act;
  void* out = GATED ? a.act : (void*)a.yp;
  auto* ex = (const uint16_t*)a.experts;
  if (rows <= 16)
    stream_kernel<GATED, 1><<<grid, 256, 0, st>>>(ex, a.stride_elems, tok, a.perm, a.k, a.offsets, a.active, a.E, a.H, a.F, a.T, out);
  else if (rows <= 32)
    stream_kernel<GATED, 2><<<grid, 256, 0, st>>>(ex, a.stride_elems, tok, a.perm, a.k, a.offsets, a.active, a.E, a.H, a.F, a.T, out);
  else
    stream_kernel<GATED, 4><<<grid, 256, 0, st>>>(ex, a.stride_elems, tok, a.perm, a.k, a.offsets, a.active, a.E, a.H, a.F, a.T, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_stream_gate_up(const ExpertArgs& a, hipStream_t st) { return launch_stream<true>(a, st); }
int launch_stream_down(const ExpertArgs& a, hipStream_t st) { return launch_stream<false>(a, st); }
