// expert_grouped.hip -- steps 4 and 5 for many rows per expert: grouped
// bf16 MFMA GEMMs over the dispatched rows.
//
// Expert FFN = SwiGLU without bias: gate_proj, up_proj, SiLU, down_proj
// [zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1,
// sec. 3.3 stage 4].  The pages fuse gate/up/SiLU/down into one kernel; here
// gate and up share one GEMM whose epilogue applies SiLU(g)*u and stores the
// activation in bf16, and the down projection is a second GEMM writing fp32
// per-row outputs for the fixed-order combine.
//
// Both GEMMs compute C^T = W . B^T with the expert's weight rows as the MFMA
// A operand ("weight rows": f for gate/up, h for down) and the expert's
// token rows as the B operand; both are K-contiguous in memory.  Work unit:
// 256 weight rows x 256 token rows, K in steps of 64, 4 waves in a 2x2
// arrangement, each wave 128x128 with 16 v_mfma_f32_32x32x16_bf16
// accumulators (256 fp32 per lane).  For gate/up the 256 weight rows are 128
// gate rows and the same 128 up rows, so SiLU(g)*u pairs accumulators that
// sit in the same lane.  Tiles are staged in LDS (2 buffers x 64 KB) by
// direct global->LDS loads (global_load_lds_dwordx4, no register staging),
// with the 16-byte chunks of each 128-byte row XOR-swizzled by (row & 7) so
// that the MFMA operand reads are free of bank conflicts; the loads of K step
// k+1 are in flight while step k is multiplied, and the operands of MFMA
// sub-step s+1 are read from LDS while sub-step s runs.  Within a K step
// lane group g reads chunks 4g..4g+3 of its row (a fixed permutation of the
// summation index, applied identically to both operands).
//
// Tiles are built on the device from the expert offsets (no host sync): the
// grid is sized for the worst case, and block b maps to (expert, token tile,
// weight tile) through tile_off; blocks are renumbered so that each XCD gets
// a contiguous range, and consecutive blocks on an XCD cover groups of 8
// weight tiles x all token tiles of one expert, which then share L2.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kGroupW = 8;  // weight tiles per L2 group

__device__ __forceinline__ int lds_chunk(int row, int c) { return row * 8 + (c ^ (row & 7)); }

template <bool GATED>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int T, void* __restrict__ out) {
  __shared__ u32x4 lds[2][2 * GG_BW * 8];  // [buffer][(256 A rows + 256 B rows) x 8 chunks]

  const int K = GATED ? H : F;
  const int MW = GATED ? F / 128 : H / 256;
  const int total = tile_off[E] * MW;
  const uint32_t n8 = ((uint32_t)total + 7u) & ~7u;
  if (blockIdx.x >= n8) return;
  const int L = (int)xcd_logical_id(blockIdx.x, n8);
  if (L >= total) return;

  // block -> (expert, token tile, weight tile)
  const int e = upper_segment(tile_off, E, L / MW);
  const int nt_e = tile_off[e + 1] - tile_off[e];
  const int local = L - tile_off[e] * MW;
  const int fg = local / (nt_e * kGroupW);
  const int rem = local - fg * nt_e * kGroupW;
  const int gsz = min(kGroupW, MW - fg * kGroupW);
  const int tt = rem / gsz;
  const int mt = fg * kGroupW + rem % gsz;

  const int p_beg = offsets[e];
  const int rows_left = offsets[e + 1] - p_beg - tt * GG_BT;  // >= 1
  const int p0 = p_beg + tt * GG_BT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Global -> LDS: waves 0-1 bring the 256 weight rows, waves 2-3 the 256
  // token rows of each K step.  One global_load_lds_dwordx4 of a wave fills
  // 1 KB of LDS = 8 rows; lane l lands in row r0 + l/8 at physical chunk l%8,
  // so it fetches logical chunk (l%8) ^ (row & 7) of that row (the swizzle).
  const uint16_t* eb = experts + (size_t)e * stride_elems;
  const uint16_t* gbase = (wave < 2) ? eb : tok;
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;  // rows r0 + lrow with r0 % 8 == 0
  uint32_t roff[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = (wave & 1) * 128 + i * 8 + lrow;  // row within the A or B half
    if (wave < 2) {
      if (GATED) {
        const int f0 = mt * 128;
        roff[i] = (r < 128) ? (uint32_t)(f0 + r) * H
                            : (uint32_t)F * H + (uint32_t)(f0 + r - 128) * H;
      } else {
        roff[i] = 2u * (uint32_t)F * H + (uint32_t)(mt * 256 + r) * F;
      }
    } else {
      const int p = p0 + min(r, rows_left - 1);
      roff[i] = GATED ? (uint32_t)min(max(perm[p], 0) / k_top, T - 1) * H : (uint32_t)p * F;
    }
    roff[i] += lchunk * 8;
  }
  auto issue = [&](int buf, int k0) {
    __attribute__((address_space(3))) u32x4* dst =
        (__attribute__((address_space(3))) u32x4*)&lds[buf][wave * 128 * 8];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(gbase + roff[i] + k0),
                                       (__attribute__((address_space(3))) void*)(dst + i * 64),
                                       16, 0, 0);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  int arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    arow[i] = (GATED ? ((i < 2) ? wm * 64 + 32 * i : 128 + wm * 64 + 32 * (i - 2))
                     : wm * 128 + 32 * i) + (lane & 31);
  const int brow = GG_BW + wn * 128 + (lane & 31);
  const int kg = lane >> 5;

  bf16x8 a[2][4], b[2][4];
  auto fetch = [&](int buf, int s, int slot) {
    const int c = kg * 4 + s;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[slot][i] = as_bf16x8(lds[buf][lds_chunk(arow[i], c)]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[slot][j] = as_bf16x8(lds[buf][lds_chunk(brow + 32 * j, c)]);
  };

  const int nk = K / GG_BK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue(cur ^ 1, (kt + 1) * GG_BK);
    fetch(cur, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 reads of sub-step 0
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) fetch(cur, s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j],
                                                              acc[i][j], 0, 0, 0);
      // interleave the next sub-step's LDS reads with this sub-step's MFMAs
      if (s < 3) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0): this wave's loads have landed
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (token) lane%32,
  // rows (weight) 8q + 4*(lane/32) + jj for element 4q + jj.
  const int tcol = lane & 31;
  const int rsub = 4 * (lane >> 5);
  if (GATED) {
    uint16_t* act = (uint16_t*)out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wn * 128 + 32 * j + tcol;
      if (tl >= rows_left) continue;
      const size_t prow = (size_t)(p0 + tl) * F;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = mt * 128 + wm * 64 + 32 * i + 8 * q + rsub;
          float o[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float g = acc[i][j][4 * q + jj];
            const float u = acc[i + 2][j][4 * q + jj];
            o[jj] = silu_f32(g) * u;
          }
          uint2 pk;
          pk.x = pack_bf16x2(o[0], o[1]);
          pk.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2*>(act + prow + f) = pk;
        }
    }
  } else {
    float* yp = (float*)out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wn * 128 + 32 * j + tcol;
      if (tl >= rows_left) continue;
      const size_t prow = (size_t)(p0 + tl) * H;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int h = mt * 256 + wm * 128 + 32 * i + 8 * q + rsub;
          f32x4 o{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                  acc[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(yp + prow + h) = o;
        }
    }
  }
}

int grid_for(const ExpertArgs& a, int mw) {
  const int max_tiles = (a.S + GG_BT - 1) / GG_BT + (a.E < a.S ? a.E : a.S);
  const int g = max_tiles * mw;
  return (g + 7) & ~7;
}

}  // namespace

int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st) {
  const int grid = grid_for(a, a.F / 128);
  grouped_gemm_kernel<true><<<grid, 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.x, a.perm, a.k, a.offsets,
      a.tile_off, a.E, a.H, a.F, a.T, a.act);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_down(const ExpertArgs& a, hipStream_t st) {
  const int grid = grid_for(a, a.H / 256);
  grouped_gemm_kernel<false><<<grid, 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.act, a.perm, a.k,
      a.offsets, a.tile_off, a.E, a.H, a.F, a.T, a.yp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
