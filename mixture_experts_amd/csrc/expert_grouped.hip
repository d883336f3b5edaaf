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
// A operand ("weight rows": f for gate/up, h for down) and the expert's token
// rows as the B operand; both are K-contiguous in memory.  Work unit: 256
// weight rows x 256 token rows, 8 waves (two per SIMD), each owning 128
// weight rows x 64 token rows = 8 v_mfma_f32_32x32x16_bf16 accumulators.
// For gate/up the 256 weight rows are 128 gate rows and the same 128 up rows,
// so SiLU(g)*u pairs accumulators that sit in the same lane.  Tiles reach LDS
// through direct global->LDS loads (global_load_lds_dwordx4, no register
// staging) into two buffers of one K step (64) each, with the 16-byte chunks
// of every 128-byte row XOR-swizzled so that MFMA operand reads are free of
// bank conflicts.  Within a K step lane group g reads chunks 4g..4g+3 of its
// row (a fixed permutation of the summation index, applied identically to
// both operands).  The schedule is a ping-pong between the two waves of each
// SIMD (see grouped_gemm_kernel).
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

#ifndef GG_PP_BK
#define GG_PP_BK 64  // K step of one phase
#endif

// LDS tile rows hold BK bf16 = CPR chunks of 16 B.  The LDS serves a 16-byte
// read of 16 lanes per cycle from its 64 x 4-byte banks (a 256-byte window),
// and the 16 lanes of an MFMA operand read take 16 consecutive rows at the
// same logical chunk.  Chunk c of row r is stored at physical chunk
// c ^ ((r / RPW) % CPR), RPW = rows per 256-byte window, so those 16 rows
// occupy 16 distinct 16-byte slots of the window.
template <int BK>
__device__ __forceinline__ int lds_chunk(int row, int c) {
  constexpr int CPR = BK / 8, RPW = 16 / CPR;
  return row * CPR + (c ^ ((row / RPW) & (CPR - 1)));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)

// Each SIMD runs two waves, one from group 0
// (waves 0-3) and one from group 1 (waves 4-7).  Time is cut into phases
// separated by workgroup barriers; in every phase one wave of each SIMD runs
// the 32 MFMAs of a whole K step from fragments already in its registers
// ("compute") while the other reads the fragments of its next K step from
// LDS and issues its share of the global->LDS loads ("memory").  Group 0
// computes in odd phases, group 1 in even phases.  Two LDS buffers:
//   weight rows of step k+1 are loaded by group 0 during its memory(k) phase
//     (phase 2k) and waited for at the end of its compute(k) phase;
//   token rows of step k+2 are loaded by group 1 at the start of its
//     compute(k) phase (phase 2k+2) into the buffer of step k, and waited for
//     in its memory(k+1) phase.
// So every read follows a completed load and a barrier, and every buffer is
// refilled only after a barrier that ends both groups' reads of it (the rows
// one wave loads are read by other waves).
template <bool GATED, int BK>
__global__ __launch_bounds__(512, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int T, int ksplit, size_t plane, void* __restrict__ out) {
  constexpr int CPR = BK / 8;      // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPR;    // rows per wave-wide 1 KB load
  constexpr int IPS = 64 / RPI;    // loads per wave per K step (64 rows per wave)
  constexpr int NSUB = BK / 16;    // MFMA sub-steps per K step
  __shared__ u32x4 lds_a[2][GG_BW * CPR];
  __shared__ u32x4 lds_b[2][GG_BT * CPR];

  // ksplit > 1 (down projection only): the K range is cut into ksplit
  // slices, slice ks writes its partial sums to plane ks of the output.
  const int K = (GATED ? H : F) / ksplit;
  const int MW = GATED ? F / 128 : H / 256;
  const int tiles = tile_off[E] * MW;
  const int total = tiles * ksplit;
  const uint32_t n8 = ((uint32_t)total + 7u) & ~7u;
  if (blockIdx.x >= n8) return;
  const int L0 = (int)xcd_logical_id(blockIdx.x, n8);
  if (L0 >= total) return;
  const int ks = L0 / tiles;
  const int L = L0 - ks * tiles;
  const int kbase = ks * K;

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = wave & 3, grp = wave >> 2;
  const int wm = q4 & 1, wn = q4 >> 1;
  const int lrow = q4 * 64;  // this wave's 64 rows of the A (group 0) or B (group 1) tile

  const uint16_t* eb = experts + (size_t)e * stride_elems;
  const uint16_t* gbase = grp == 0 ? eb : tok;
  uint32_t roff[IPS];
#pragma unroll
  for (int i = 0; i < IPS; ++i) {
    const int r = lrow + i * RPI + lane / CPR;
    const int lchunk = (lane % CPR) ^ ((r / (16 / CPR)) & (CPR - 1));
    if (grp == 0) {
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
    roff[i] += lchunk * 8 + kbase;
  }
  auto issue = [&](int k0, u32x4* ring_slot) {
    const uint32_t dst = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) u32x4*)(ring_slot + lrow * CPR));
#pragma unroll
    for (int i = 0; i < IPS; ++i) {
      const uint16_t* src = gbase + roff[i] + k0;
      // one wait state between the M0 write and the LDS-DMA load that reads it
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(dst + i * 1024)), "v"(src)
                   : "memory", "m0");
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  int arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    arow[i] = (GATED ? ((i < 2) ? wm * 64 + 32 * i : 128 + wm * 64 + 32 * (i - 2))
                     : wm * 128 + 32 * i) + (lane & 31);
  const int brow = wn * 128 + grp * 64 + (lane & 31);
  const int kg = lane >> 5;

  bf16x8 fa[NSUB][4], fb[NSUB][2];  // [sub-step][block] fragments of one K step
  auto read_step = [&](int buf) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int c = kg * NSUB + s;
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[s][i] = as_bf16x8(lds_a[buf][lds_chunk<BK>(arow[i], c)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[s][j] = as_bf16x8(lds_b[buf][lds_chunk<BK>(brow + 32 * j, c)]);
    }
  };
  auto compute_step = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j],
                                                              0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
#define PP_BARRIER() asm volatile("s_barrier" ::: "memory")

  const int nk = K / BK;
  if (grp == 0) {
    issue(0, lds_a[0]);
    WAIT_VMCNT(0);
  } else {
    issue(0, lds_b[0]);
    if (nk > 1) {
      issue(BK, lds_b[1]);
      WAIT_VMCNT(IPS);
    } else {
      WAIT_VMCNT(0);
    }
  }
  PP_BARRIER();
  if (grp == 0) {
    for (int k = 0; k < nk; ++k) {
      // phase 2k: memory(k)
      read_step(k & 1);
      if (k + 1 < nk) issue((k + 1) * BK, lds_a[(k & 1) ^ 1]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      PP_BARRIER();
      // phase 2k+1: compute(k)
      compute_step();
      WAIT_VMCNT(0);  // weight rows of step k+1 have landed
      PP_BARRIER();
    }
    PP_BARRIER();  // phase 2nk: group 1 computes its last step
  } else {
    PP_BARRIER();  // phase 0: group 0 reads step 0
    for (int k = 0; k < nk; ++k) {
      // phase 2k+1: memory(k)
      read_step(k & 1);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      WAIT_VMCNT(0);  // token rows of step k+1 have landed
      PP_BARRIER();
      // phase 2k+2: compute(k).  The token rows of step k+2 go into the
      // buffer of step k, which both groups finished reading before this
      // barrier (a wave's loaded rows are read by other waves, so the
      // refill must not start within the phase that reads them).
      if (k + 2 < nk) issue((k + 2) * BK, lds_b[k & 1]);
      compute_step();
      PP_BARRIER();
    }
  }
#undef PP_BARRIER

  const int tcol = lane & 31;
  const int rsub = 4 * (lane >> 5);
  if (GATED) {
    uint16_t* act = (uint16_t*)out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tl = wn * 128 + grp * 64 + 32 * j + tcol;
      if (tl >= rows_left) continue;
      const size_t prow = (size_t)(p0 + tl) * F;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int f = mt * 128 + wm * 64 + 32 * i + 8 * q + rsub;
          float o[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            o[jj] = silu_f32(acc[i][j][4 * q + jj]) * acc[i + 2][j][4 * q + jj];
          uint2 pk;
          pk.x = pack_bf16x2(o[0], o[1]);
          pk.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2*>(act + prow + f) = pk;
        }
    }
  } else {
    float* yp = (float*)out + (size_t)ks * plane;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tl = wn * 128 + grp * 64 + 32 * j + tcol;
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

int grid_for(const ExpertArgs& a, int mw, int ksplit) {
  const int max_tiles = (a.S + GG_BT - 1) / GG_BT + (a.E < a.S ? a.E : a.S);
  const int g = max_tiles * mw * ksplit;
  return (g + 7) & ~7;
}

}  // namespace

int grouped_down_ksplit(const ExpertArgs& a) {
  // split the long K of the down projection in two when there are too few
  // tiles to fill the 256 CUs a few times over (bounded by the worst case)
  const int max_tiles = (a.S + GG_BT - 1) / GG_BT + (a.E < a.S ? a.E : a.S);
  return (max_tiles * (a.H / 256) < 3 * 256 && a.F % (2 * GG_PP_BK) == 0) ? 2 : 1;
}

int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st) {
  const int grid = grid_for(a, a.F / 128, 1);
  grouped_gemm_kernel<true, GG_PP_BK><<<grid, 512, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.x, a.perm, a.k, a.offsets,
      a.tile_off, a.E, a.H, a.F, a.T, 1, 0, a.act);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_down(const ExpertArgs& a, int ksplit, hipStream_t st) {
  const int grid = grid_for(a, a.H / 256, ksplit);
  grouped_gemm_kernel<false, GG_PP_BK><<<grid, 512, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.act, a.perm, a.k,
      a.offsets, a.tile_off, a.E, a.H, a.F, a.T, ksplit, (size_t)a.S * a.H, a.yp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
