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
// weight rows x 256 token rows, 4 waves (one per SIMD), each owning 128
// weight rows x 128 token rows = 16 v_mfma_f32_32x32x16_bf16 accumulators
// (256 accumulator registers).  For gate/up the 256 weight rows are 128 gate
// rows and the same 128 up rows, so SiLU(g)*u pairs accumulators that sit in
// the same lane.
//
// Operands reach LDS through direct global->LDS loads (global_load_lds_dwordx4,
// no register staging) into a ring of NS stages of one K step (32) each; the
// 16-byte chunks of every 64-byte row are XOR-swizzled so that MFMA operand
// reads are free of bank conflicts.  Each wave runs one instruction stream in
// which the MFMAs of a half step (16 k) are interleaved with the LDS reads of
// the next half step and with its share of the loads of a later K step, so
// the matrix cores keep issuing while LDS and the load path work in their
// shadow; one workgroup barrier per K step publishes a landed stage.
//
// Tiles are built on the device from the expert offsets (no host sync): the
// grid is sized for the worst case, and block b maps to (expert, token tile,
// weight tile) through tile_off; blocks are renumbered so that each XCD gets
// a contiguous range, and consecutive blocks on an XCD cover groups of 8
// weight tiles x all token tiles of one expert, which then share L2.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int kGroupW = 8;  // weight tiles per L2 group
constexpr int kBK = 32;     // K step (elements): one 64-byte row slice
constexpr int kCPR = 4;     // 16-byte chunks per LDS row
constexpr int kNS = 4;      // LDS ring depth (4 x 32 KB)

// Chunk c of row r sits at physical chunk c ^ ((r / 4) % 4): the 16 lanes of
// one MFMA operand read take 16 consecutive rows at one logical chunk, and
// those land in 16 distinct 16-byte slots of a 256-byte bank window.
__device__ __forceinline__ int lds_slot(int row, int c) {
  return row * kCPR + (c ^ ((row >> 2) & 3));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)

template <bool GATED, int NS>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int T, int ksplit, size_t plane, void* __restrict__ out) {
  // [stage][0: weight rows, 1: token rows][256 rows x 4 chunks]; after the
  // K loop the ring is reused to stage the output tile
  __shared__ u32x4 lds[NS][2][256 * kCPR];
  static_assert(sizeof(lds) >= 256 * 272 && sizeof(lds) >= 128 * 1024,
                "output staging must fit in the operand ring");

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

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // Loads: per K step each wave moves weight rows and token rows
  // [64 wave, 64 wave + 64), 4 + 4 instructions of 16 rows x 64 bytes; lane l
  // fills row l / 4, physical chunk l % 4, from the logical chunk stored there.
  const uint16_t* eb = experts + (size_t)stride_elems * e;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 64 + i * 16 + (lane >> 2);
    const int lc = (lane & 3) ^ ((r >> 2) & 3);
    if (GATED) {
      const int f0 = mt * 128;
      aoff[i] = (r < 128) ? (uint32_t)(f0 + r) * H : (uint32_t)F * H + (uint32_t)(f0 + r - 128) * H;
    } else {
      aoff[i] = 2u * (uint32_t)F * H + (uint32_t)(mt * 256 + r) * F;
    }
    const int p = p0 + min(r, rows_left - 1);
    boff[i] = GATED ? (uint32_t)min(max(perm[p], 0) / k_top, T - 1) * H : (uint32_t)p * F;
    aoff[i] += lc * 8 + kbase;
    boff[i] += lc * 8 + kbase;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)&lds[0][0][0]);
  // one 16-row load: operand op (0 weights, 1 tokens), row group i, K step s
  auto dma = [&](int s, int op, int i) {
    const uint16_t* src = (op == 0 ? eb + aoff[i] : tok + boff[i]) + s * kBK;
    const uint32_t dst = lds_base + (uint32_t)(((s % NS) * 2 + op) * 256 * kCPR * 16) +
                         (uint32_t)((wave * 64 + i * 16) * kCPR * 16);
    // one wait state between the M0 write and the LDS-DMA load that reads it
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
                 : "memory", "m0");
  };

  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = (GATED ? ((i < 2) ? wm * 64 + 32 * i : 128 + wm * 64 + 32 * (i - 2))
                     : wm * 128 + 32 * i) + (lane & 31);
    brow[i] = wn * 128 + 32 * i + (lane & 31);
  }
  const int kg = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // fragments of one half step (16 k): lane group kg reads chunk 2 kg + h, a
  // fixed permutation of the summation index applied to both operands
  bf16x8 fa[2][4], fb[2][4];
  // the 8 reads of half step (s, h) in the order of first use by the MFMAs
  // (row block i of the weights, then token blocks 0..3, then weights 1..3)
  auto rd = [&](int buf, int s, int h, int n) {
    const int c = kg * 2 + h;
    const int st = s % NS;
    if (n == 0) fa[buf][0] = as_bf16x8(lds[st][0][lds_slot(arow[0], c)]);
    else if (n < 5) fb[buf][n - 1] = as_bf16x8(lds[st][1][lds_slot(brow[n - 1], c)]);
    else fa[buf][n - 4] = as_bf16x8(lds[st][0][lds_slot(arow[n - 4], c)]);
  };
  // 16 MFMAs on fragment buffer buf, with the 8 reads of (rs, rh) into the
  // other buffer and up to four 16-row loads of K step ls (half lh) woven in.
  // RD / LD are std::bool_constant (fixed) or bool (decided at run time).
  auto half_step = [&](int buf, auto RD, int rs, int rh, auto LD, int ls, int lh) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int i = m >> 2, j = m & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
      if ((m & 1) == 0 && RD) rd(buf ^ 1, rs, rh, m >> 1);
      if ((m & 3) == 1 && LD) dma(ls, lh, m >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
#define GG_BARRIER() asm volatile("s_barrier" ::: "memory")

  const int nk = K / kBK;
  // prologue: K steps 0 .. NS-2 in flight, wait for step 0
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma(s, 0, i);
#pragma unroll
      for (int i = 0; i < 4; ++i) dma(s, 1, i);
    }
  if (nk >= NS - 1) WAIT_VMCNT((NS - 2) * 8); else WAIT_VMCNT(0);
  GG_BARRIER();
#pragma unroll
  for (int n = 0; n < 8; ++n) rd(0, 0, 0, n);

  // K step k:  half 0 computes (k, 0) while reading (k, 1) and loading the
  // token rows of step k+NS-2 into the stage of step k-2;  then every wave
  // waits for its loads of step k+1 and a barrier publishes that stage and
  // ends all reads of step k-1;  half 1 computes (k, 1) while reading
  // (k+1, 0) and loading the weight rows of step k+NS-1 into the stage of
  // step k-1.  Loads complete in issue order, so after half 0 of step k the
  // loads still allowed in flight are those of steps k+2 .. k+NS-2.
  // The steps 1 .. nk-NS run with every read and load present and take the
  // branch-free body; the first and the last NS-1 steps decide at run time.
  auto step = [&](int k) {
    half_step(0, std::true_type(), k, 1, k >= 1 && k + NS - 2 < nk, k + NS - 2, 1);
    if (k + NS - 2 < nk) WAIT_VMCNT((NS - 3) * 8); else WAIT_VMCNT(0);
    GG_BARRIER();
    half_step(1, k + 1 < nk, k + 1, 0, k + NS - 1 < nk, k + NS - 1, 0);
  };
  int k = 0;
  if (nk > 0) step(k++);
  for (; k + NS - 1 < nk; ++k) {
    half_step(0, std::true_type(), k, 1, std::true_type(), k + NS - 2, 1);
    WAIT_VMCNT((NS - 3) * 8);
    GG_BARRIER();
    half_step(1, std::true_type(), k + 1, 0, std::true_type(), k + NS - 1, 0);
  }
  for (; k < nk; ++k) step(k);
#undef GG_BARRIER

  const int tcol = lane & 31;
  const int rsub = 4 * (lane >> 5);
  if (GATED) {
    // SiLU(g) * u to bf16, staged through LDS as [token][f] rows (272-byte
    // pitch: 16 bytes of padding spread the 8-byte writes of one MFMA column
    // over the banks), then written out as 256-byte row runs.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    constexpr int OP = 272;
    uint8_t* ob = (uint8_t*)&lds[0][0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = wn * 128 + 32 * j + tcol;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int fl = wm * 64 + 32 * i + 8 * q + rsub;
          float o[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float g = acc[i][j][4 * q + jj];
            o[jj] = silu_f32(g) * acc[i + 2][j][4 * q + jj];
          }
          const bf16x2 lo = {(__bf16)o[0], (__bf16)o[1]}, hi = {(__bf16)o[2], (__bf16)o[3]};
          uint2 pk;
          pk.x = __builtin_bit_cast(uint32_t, lo);
          pk.y = __builtin_bit_cast(uint32_t, hi);
          *reinterpret_cast<uint2*>(ob + tl * OP + fl * 2) = pk;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    uint16_t* act = (uint16_t*)out;
    const int c = threadIdx.x & 15;
#pragma unroll 4
    for (int r0 = 0; r0 < 256; r0 += 16) {
      const int row = r0 + (threadIdx.x >> 4);
      if (row < rows_left)
        *reinterpret_cast<u32x4*>(act + (size_t)(p0 + row) * F + mt * 128 + c * 8) =
            *reinterpret_cast<const u32x4*>(ob + row * OP + c * 16);
    }
  } else {
    // fp32 partial rows, staged through LDS in two rounds (token rows
    // 0-127, then 128-255) as [token][256 h] 1 KB rows whose 16-byte chunks
    // are XOR-swizzled by the row (chunk c of row t at c ^ (t % 16)), then
    // written out as 1 KB row runs.
    float* yp = (float*)out + (size_t)ks * plane;
    uint8_t* ob = (uint8_t*)&lds[0][0][0];  // 128 KB: exactly the ring
    const int c = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wn == r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tl = 32 * j + tcol;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int hc = (wm * 128 + 32 * i + 8 * q + rsub) >> 2;
              f32x4 o{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
              *reinterpret_cast<f32x4*>(ob + tl * 1024 + ((hc ^ (tl & 15)) << 4)) = o;
            }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll 4
      for (int r0 = 0; r0 < 128; r0 += 4) {
        const int row = r0 + (threadIdx.x >> 6);
        const int tl = r * 128 + row;
        if (tl < rows_left)
          *reinterpret_cast<u32x4*>(yp + (size_t)(p0 + tl) * H + mt * 256 + ((c ^ (row & 15)) << 2)) =
              *reinterpret_cast<const u32x4*>(ob + row * 1024 + (c << 4));
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
  return (max_tiles * (a.H / 256) < 3 * 256 && a.F % (2 * kBK) == 0) ? 2 : 1;
}

int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st) {
  const int grid = grid_for(a, a.F / 128, 1);
  grouped_gemm_kernel<true, kNS><<<grid, 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.x, a.perm, a.k, a.offsets,
      a.tile_off, a.E, a.H, a.F, a.T, 1, 0, a.act);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_down(const ExpertArgs& a, int ksplit, hipStream_t st) {
  const int grid = grid_for(a, a.H / 256, ksplit);
  grouped_gemm_kernel<false, kNS><<<grid, 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.act, a.perm, a.k,
      a.offsets, a.tile_off, a.E, a.H, a.F, a.T, ksplit, (size_t)a.S * a.H, a.yp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
