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
// The kernels are persistent (one workgroup per compute unit) and build their
// tile lists on the device from the expert offsets (no host sync).  A
// workgroup starts the first K steps of its next tile before it writes out
// the current one, so tile boundaries cost little.  In a tile whose token
// rows end early, waves skip the MFMAs of 32-row blocks past the end.  In
// the down projection the tiles of an XCD's last, partial round are cut
// along K into pieces run by the workgroups that would otherwise idle; the
// pieces store fp32 partial sums and a second, short launch adds them in
// piece order and writes those tiles (no cross-workgroup waiting, and the
// same result on every call).  Gate/up tiles are shorter (K = H) and gain
// nothing from it.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int kGroupW = 8;  // weight tiles per L2 group
constexpr int kBK = 32;     // K step (elements): one 64-byte row slice
constexpr int kCPR = 4;     // 16-byte chunks per LDS row
constexpr int kNS = 4;      // LDS ring depth (4 x 32 KB)
constexpr int kStage = 2 * 256 * kCPR;   // 16-byte chunks per ring stage (32 KB)
// down projection: its output is staged in the 64 KB from kStageOut, clear of
// ring stages 0-2 where the next tile's first K steps land meanwhile
constexpr int kStageOut = 3 * kStage;
constexpr int kLdsDown = kStageOut + 64 * 1024 / 16;  // 160 KB

// Chunk c of row r sits at physical chunk c ^ ((r / 4) % 4): the 16 lanes of
// one MFMA operand read take 16 consecutive rows at one logical chunk, and
// those land in 16 distinct 16-byte slots of a 256-byte bank window.
__device__ __forceinline__ int lds_slot(int row, int c) {
  return row * kCPR + (c ^ ((row >> 2) & 3));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
#define GG_BARRIER() asm volatile("s_barrier" ::: "memory")

// Tail split (down projection): the tiles that would leave most workgroups
// of an XCD idle in its last round are cut along K into np pieces of at
// least kMinPiece steps.
constexpr int kMaxPieces = 4;
constexpr int kMinPiece = 16;
constexpr int kPartFloats = 256 * 256;  // one piece's fp32 partial sums

// One tile: expert e, K slice ks, weight tile mt, token rows p0 .. p0+rows-1,
// K steps k0 .. k0+nk-1 of the slice.  np > 1: piece `piece` of np; the np
// pieces of leftover tile l are taken by the workgroups l + p * nleft.
struct Tile {
  int e, ks, mt, p0, rows;
  int k0, nk, np, piece, l;
};

// Persistent schedule.  Tiles are numbered (K slice, weight group, expert,
// token tile, weight tile), a weight group being a run of up to 8 weight
// tiles; the tiles of one (K slice, weight group, expert) share weight rows
// and token rows.  Each XCD (workgroup b runs on XCD b % 8) takes one
// contiguous eighth of the numbering and its nw workgroups take those tiles
// in turn, so tiles running together on an XCD share data in its L2, and
// each XCD sees every expert, whatever the routing skew.  With split set,
// the nleft tiles of a last, partial round are cut into np K pieces each
// (np * nleft <= nw); each piece stores its fp32 partial sums and a second
// launch adds the np partials in piece order and writes the tile.
struct Plan {
  int MW, ngpe, ntt, per_ks, nk_slice, q_beg, q_end, nfull, nleft, np;
};

__device__ Plan make_plan(bool gated, const int32_t* tile_off, int E, int H, int F, int ksplit,
                          int xcd, int nw, bool split) {
  Plan p;
  p.MW = gated ? F / 128 : H / 256;  // weight tiles per expert
  p.ngpe = (p.MW + kGroupW - 1) / kGroupW;
  p.ntt = tile_off[E];               // token tiles over all experts
  p.per_ks = p.ntt * p.MW;
  p.nk_slice = (gated ? H : F) / ksplit / kBK;
  const int ntiles = ksplit * p.per_ks;
  p.q_beg = (int)(((int64_t)xcd * ntiles) >> 3);
  p.q_end = (int)(((int64_t)(xcd + 1) * ntiles) >> 3);
  p.nfull = (p.q_end - p.q_beg) / nw;
  p.nleft = p.q_end - p.q_beg - p.nfull * nw;
  p.np = 1;
  if (split && p.nleft > 0)
    p.np = max(1, min(min(nw / p.nleft, kMaxPieces), p.nk_slice / kMinPiece));
  return p;
}

// Tile q of the numbering (whole K slice).
__device__ void tile_at(const Plan& p, int q, const int32_t* tile_off, const int32_t* offsets,
                        int E, Tile& t) {
  const int ks = q / p.per_ks;
  const int r = q - ks * p.per_ks;
  const int fg = min(r / (p.ntt * kGroupW), p.ngpe - 1);
  const int r2 = r - fg * p.ntt * kGroupW;
  const int gsz = min(kGroupW, p.MW - fg * kGroupW);
  const int u = r2 / gsz;  // token tile over all experts
  const int e = upper_segment(tile_off, E, u);
  t.e = e;
  t.ks = ks;
  t.mt = fg * kGroupW + (r2 - u * gsz);
  t.p0 = offsets[e] + (u - tile_off[e]) * GG_BT;
  t.rows = min(offsets[e + 1] - t.p0, GG_BT);
  t.k0 = 0;
  t.nk = p.nk_slice;
  t.np = 1;
  t.piece = 0;
  t.l = 0;
}

// Output of one tile by the 4 waves of a workgroup.  Gate/up: lane (tcol,
// rsub) of wave (wm, wn) holds 4 consecutive f for token tcol of each token
// block and writes SiLU(g) * u as 8 bf16 bytes; the four waves together
// write every 128-byte line of the tile's rows.  Down: the fp32 partial sums
// go through the 64 KB of LDS at ob in four rounds, round j holding token
// blocks 2j and 2j+1 as [64 tokens][256 h] 1 KB rows whose 16-byte chunks are
// XOR-swizzled by the row (chunk c of row r at c ^ (r % 16)), written out as
// 1 KB runs to plane t.ks.  get4(i, j, q) gives the lane's 4 sums of block
// (i, j) at rows 8q + rsub; prep(j) runs before the blocks (., j) are read.
// jsel >= 0: only the token blocks 2 jsel and 2 jsel + 1.
template <bool GATED, class Prep, class Get>
__device__ __forceinline__ void write_tile(const Tile& t, Prep prep, Get get4,
                                           void* __restrict__ out, int F, int H, size_t plane,
                                           uint8_t* ob, int wave, int jsel = -1) {
  const int wm = wave & 1, wn = wave >> 1;
  int tid;  // the thread id, opaque so that the addressing below is not kept live across tiles
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int tcol = tid & 31;
  const int rsub = 4 * ((tid >> 5) & 1);
  if (GATED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tl = (2 * j + wn) * 32 + tcol;
      if (tl >= t.rows || (jsel >= 0 && j != jsel)) continue;
      prep(j);
      uint16_t* row = (uint16_t*)out + (size_t)(t.p0 + tl) * F + t.mt * 128 + wm * 64 + rsub;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 g = get4(i, j, q), u = get4(i + 2, j, q);
          float o[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) o[jj] = silu_f32(g[jj]) * u[jj];
          const bf16x2 lo = {(__bf16)o[0], (__bf16)o[1]}, hi = {(__bf16)o[2], (__bf16)o[3]};
          uint2 pk;
          pk.x = __builtin_bit_cast(uint32_t, lo);
          pk.y = __builtin_bit_cast(uint32_t, hi);
          *reinterpret_cast<uint2*>(row + 32 * i + 8 * q) = pk;
        }
    }
  } else {
    float* yp = (float*)out + (size_t)t.ks * plane;
    const int c = tid & 63;
    const int sr = wn * 32 + tcol;  // staging row of this lane's token
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (jsel >= 0 && j != jsel) continue;
      if (j > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      prep(j);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int hc = (wm * 128 + 32 * i + 8 * q + rsub) >> 2;
          *reinterpret_cast<f32x4*>(ob + sr * 1024 + ((hc ^ (sr & 15)) << 4)) = get4(i, j, q);
        }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll 4
      for (int r0 = 0; r0 < 64; r0 += 4) {
        const int row = r0 + (tid >> 6);
        const int tl = (2 * j + (row >> 5)) * 32 + (row & 31);
        if (tl < t.rows)
          *reinterpret_cast<u32x4*>(yp + (size_t)(t.p0 + tl) * H + t.mt * 256 + ((c ^ (row & 15)) << 2)) =
              *reinterpret_cast<const u32x4*>(ob + row * 1024 + (c << 4));
      }
    }
  }
}

// A piece's partial sums, lane-major: wave, block (i, j), quad q, lane (the
// lane id opaque, so that no address is formed before it is needed).
__device__ __forceinline__ f32x4* part_base(float* ws, int slot, int wave) {
  int ln;
  asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
  return reinterpret_cast<f32x4*>(ws + (size_t)slot * kPartFloats + wave * 16384) + ln;
}

template <bool GATED, int NS>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int T, int ksplit, size_t plane, void* __restrict__ out, float* __restrict__ ws) {
  // ring stage s at lds + s * kStage: [weight rows | token rows] x 256 x 4 chunks
  __shared__ u32x4 lds[GATED ? NS * kStage : kLdsDown];
  static_assert(GATED || (NS - 1) * kStage <= kStageOut, "LDS layout");

  // ksplit > 1 (down projection only): the K range is cut into ksplit
  // slices, slice ks writes its partial sums to plane ks of the output.
  const int K = (GATED ? H : F) / ksplit;
  const int xcd = blockIdx.x & 7;
  const int nw = gridDim.x >> 3;   // workgroups per XCD
  const int jw = blockIdx.x >> 3;  // this workgroup's place on its XCD
  const Plan pl = make_plan(GATED, tile_off, E, H, F, ksplit, xcd, nw, !GATED && ws != nullptr);
  // work item w of this workgroup (rounds 0, 1, ...)
  auto locate = [&](int w, Tile& t) -> bool {
    if (pl.np < 2 || w < pl.nfull) {
      const int q = pl.q_beg + jw + w * nw;
      if (q >= pl.q_end) return false;
      tile_at(pl, q, tile_off, offsets, E, t);
      return true;
    }
    if (w > pl.nfull || jw >= pl.nleft * pl.np) return false;
    const int l = jw % pl.nleft, piece = jw / pl.nleft;
    tile_at(pl, pl.q_beg + pl.nfull * nw + l, tile_off, offsets, E, t);
    t.l = l;
    t.piece = piece;
    t.np = pl.np;
    t.k0 = piece * pl.nk_slice / pl.np;
    t.nk = (piece + 1) * pl.nk_slice / pl.np - t.k0;
    return true;
  };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // Loads: per K step each wave moves weight rows and token rows
  // [64 wave, 64 wave + 64), 4 + 4 instructions of 16 rows x 64 bytes; lane l
  // fills row l / 4, physical chunk l % 4, from the logical chunk stored there.
  const uint16_t* eb = experts;
  uint32_t aoff[4], boff[4];
  // gate/up: the slot ids of this lane's 4 token rows (rows past the tile's
  // end repeat its last row)
  auto load_perm = [&](const Tile& t, int (&pv)[4]) {
    if (!GATED) return;
    int ln;  // the lane id, opaque so that the addressing below is not kept live across tiles
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = perm[t.p0 + min(wave * 64 + i * 16 + (ln >> 2), t.rows - 1)];
  };
  auto set_tile = [&](const Tile& t, const int (&pv)[4]) {
    eb = experts + (size_t)stride_elems * t.e;
    const int kbase = t.ks * K + t.k0 * kBK;
    int ln;  // the lane id, opaque as above
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 64 + i * 16 + (ln >> 2);
      const int lc = (ln & 3) ^ ((r >> 2) & 3);
      uint32_t a;
      if (GATED) {
        const int f0 = t.mt * 128;
        a = (r < 128) ? (uint32_t)(f0 + r) * H : (uint32_t)F * H + (uint32_t)(f0 + r - 128) * H;
      } else {
        a = 2u * (uint32_t)F * H + (uint32_t)(t.mt * 256 + r) * F;
      }
      const int p = t.p0 + min(r, t.rows - 1);
      const uint32_t b = GATED ? (uint32_t)min(max(pv[i], 0) / k_top, T - 1) * H : (uint32_t)p * F;
      aoff[i] = a + lc * 8 + kbase;
      boff[i] = b + lc * 8 + kbase;
    }
  };
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)&lds[0]);
  // one 16-row load: operand op (0 weights, 1 tokens), row group i, K step s
  auto dma = [&](int s, int op, int i) {
    const uint16_t* src = (op == 0 ? eb + aoff[i] : tok + boff[i]) + s * kBK;
    const uint32_t dst = lds_base + (uint32_t)(((s % NS) * kStage + op * 256 * kCPR) * 16) +
                         (uint32_t)((wave * 64 + i * 16) * kCPR * 16);
    // one wait state between the M0 write and the LDS-DMA load that reads it
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
                 : "memory", "m0");
  };
  // the first NS-1 K steps of a tile of nk steps (ring stages 0 .. NS-2)
  auto prologue = [&](int nk) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma(s, 0, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma(s, 1, i);
      }
  };

  // The K loop of one tile for a wave that computes its first NJ token
  // blocks (the others lie beyond the tile's rows).  Loads never depend on
  // NJ, so every wave keeps the same load and barrier sequence.
  auto kloop = [&](auto NJc, f32x16 (&acc)[4][4], int nk) {
    constexpr int NJ = decltype(NJc)::value;
    int ln;  // the lane id, opaque as above
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
    // MFMA operands: row block i of the weights (for gate/up blocks 0-1 are
    // gate rows, 2-3 the matching up rows) and token block j; wave (wm, wn)
    // owns token blocks 2j + wn, j = 0..3, so that a ragged tile's rows
    // split evenly over the two wave columns
    int arow[4], brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      arow[i] = (GATED ? ((i < 2) ? wm * 64 + 32 * i : 128 + wm * 64 + 32 * (i - 2))
                       : wm * 128 + 32 * i) + (ln & 31);
      brow[i] = (2 * i + wn) * 32 + (ln & 31);
    }
    const int kg = ln >> 5;
    // fragments of one half step (16 k): lane group kg reads chunk 2 kg + h,
    // a fixed permutation of the summation index applied to both operands
    bf16x8 fa[2][4], fb[2][4];
    // the 8 reads of half step (s, h) in the order of first use by the MFMAs
    // (row block i of the weights, then token blocks 0..3, then weights 1..3)
    auto rd = [&](int buf, int s, int h, int n) {
      const int c = kg * 2 + h;
      const u32x4* st = lds + (s % NS) * kStage;
      if (n == 0) fa[buf][0] = as_bf16x8(st[lds_slot(arow[0], c)]);
      else if (n < 5) {
        if (n - 1 < NJ) fb[buf][n - 1] = as_bf16x8(st[256 * kCPR + lds_slot(brow[n - 1], c)]);
      } else fa[buf][n - 4] = as_bf16x8(st[lds_slot(arow[n - 4], c)]);
    };
    // the MFMAs of fragment buffer buf, with the 8 reads of (rs, rh) into the
    // other buffer and up to four 16-row loads of K step ls (half lh) woven in.
    // RD / LD are std::bool_constant (fixed) or bool (decided at run time).
    auto half_step = [&](int buf, auto RD, int rs, int rh, auto LD, int ls, int lh) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        if (j < NJ)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
        if ((m & 1) == 0 && RD) rd(buf ^ 1, rs, rh, m >> 1);
        if ((m & 3) == 1 && LD) dma(ls, lh, m >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
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
  };

  int round = 0;
  Tile cur, nxt;
  if (!locate(round, cur)) return;
  {
    int pv[4];
    load_perm(cur, pv);
    set_tile(cur, pv);
  }
  prologue(cur.nk);
  // one tile for waves that compute NJ token blocks; returns whether a next
  // tile exists (then its first stages are in flight)
  auto tile = [&](auto NJc) -> bool {
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    // the next tile, located and its token rows looked up while this one
    // computes (those loads precede the K loop's and only strengthen its waits)
    const bool more = locate(round + 1, nxt);
    int pn[4] = {0, 0, 0, 0};
    if (more) load_perm(nxt, pn);
    kloop(NJc, acc, cur.nk);
    // every load of the tile has landed; end every wave's reads of the ring,
    // then start the next tile's first stages under this tile's epilogue
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (more) {
      set_tile(nxt, pn);
      prologue(nxt.nk);
    }
    // read each accumulator where it is used: left to itself the compiler
    // copies all of them to VGPRs at once and spills
    auto from_acc = [&](int i, int j, int q) -> f32x4 {
      f32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a;
        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a) : "a"(acc[i][j][4 * q + u]));
        v[u] = a;
      }
      return v;
    };
    if (cur.np < 2) {
      write_tile<GATED>(cur, [](int) {}, from_acc, out, F, H, plane, (uint8_t*)&lds[kStageOut],
                        wave);
    } else {  // a piece: its partial sums, for the launch that finishes the tile
      f32x4* dst = part_base(ws, xcd * nw + jw, wave);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[((i * 4 + j) * 4 + q) * 64] = from_acc(i, j, q);
    }
    return more;
  };
  for (;;) {
    // this tile's first NS-1 stages have landed (and the previous tile's
    // output stores have completed, as vmcnt counts both); the barrier also
    // ends every wave's reads of the previous tile's output staging
    WAIT_VMCNT(0);
    GG_BARRIER();
    const int nb = (cur.rows + 31) >> 5;        // 32-row token blocks in the tile
    const int nj = max((nb - wn + 1) >> 1, 1);  // this wave's (at least one)
    bool more;
    switch (nj) {
      case 1: more = tile(std::integral_constant<int, 1>()); break;
      case 2: more = tile(std::integral_constant<int, 2>()); break;
      case 3: more = tile(std::integral_constant<int, 3>()); break;
      default: more = tile(std::integral_constant<int, 4>()); break;
    }
    if (!more) break;
    cur = nxt;
    ++round;
  }
}

// The split tail tiles of a grouped_gemm_kernel launch: workgroup b finishes
// token blocks 2 (b % 4) and 2 (b % 4) + 1 of leftover tile (b / 4) % nw of
// XCD share b / (4 nw) (if there is one), adding the np pieces' partial sums
// in piece order.
template <bool GATED>
__global__ __launch_bounds__(256) void grouped_fixup_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int ksplit, size_t plane, void* __restrict__ out, float* __restrict__ ws, int nw) {
  __shared__ u32x4 ob[GATED ? 1 : 64 * 1024 / 16];
  const int jsel = blockIdx.x & 3, xcd = (blockIdx.x >> 2) / nw, l = (blockIdx.x >> 2) % nw;
  const Plan pl = make_plan(GATED, tile_off, E, H, F, ksplit, xcd, nw, true);
  if (pl.np < 2 || l >= pl.nleft) return;
  Tile t;
  tile_at(pl, pl.q_beg + pl.nfull * nw + l, tile_off, offsets, E, t);
  if (64 * jsel >= t.rows) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const f32x4* src = part_base(ws, xcd * nw + l, wave);
  const size_t pstep = (size_t)pl.nleft * kPartFloats / 4;  // between pieces
  // the sums of token block column j, all loads of a column in flight at once
  f32x4 col[4][4];
  auto prep = [&](int j) {
    f32x4 v[kMaxPieces][4][4];
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p)
      if (p < pl.np)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) v[p][i][q] = src[p * pstep + ((i * 4 + j) * 4 + q) * 64];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 a = v[0][i][q];
#pragma unroll
        for (int p = 1; p < kMaxPieces; ++p)
          if (p < pl.np) a += v[p][i][q];
        col[i][q] = a;
      }
  };
  write_tile<GATED>(t, prep, [&](int i, int, int q) -> f32x4 { return col[i][q]; }, out, F, H,
                    plane, (uint8_t*)ob, wave, jsel);
}

// One workgroup per compute unit, a multiple of 8 (one share per XCD).
int persistent_grid() {
  const int w = cu_count() / 8;
  return 8 * (w < 1 ? 1 : w);
}

}  // namespace

int grouped_grid() { return persistent_grid(); }

int grouped_down_ksplit(const ExpertArgs& a) {
  // split the long K of the down projection in two when there are too few
  // tiles to fill the 256 CUs a few times over (bounded by the worst case)
  const int max_tiles = (a.S + GG_BT - 1) / GG_BT + (a.E < a.S ? a.E : a.S);
  return (max_tiles * (a.H / 256) < 3 * 256 && a.F % (2 * kBK) == 0) ? 2 : 1;
}

int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st) {
  grouped_gemm_kernel<true, kNS><<<persistent_grid(), 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.x, a.perm, a.k, a.offsets,
      a.tile_off, a.E, a.H, a.F, a.T, 1, 0, a.act, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_down(const ExpertArgs& a, int ksplit, hipStream_t st) {
  grouped_gemm_kernel<false, kNS><<<persistent_grid(), 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.act, a.perm, a.k,
      a.offsets, a.tile_off, a.E, a.H, a.F, a.T, ksplit, (size_t)a.S * a.H, a.yp, a.gws);
  if (a.gws)
    grouped_fixup_kernel<false><<<4 * persistent_grid(), 256, 0, st>>>(
        a.offsets, a.tile_off, a.E, a.H, a.F, ksplit, (size_t)a.S * a.H, a.yp, a.gws,
        persistent_grid() / 8);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
