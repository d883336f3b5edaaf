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
// Operands reach LDS through direct global->LDS loads (global_load_lds_dwordx4
// for weight rows, buffer_load_dwordx4 ... lds for token rows; no register
// staging) in K steps of 64: one instruction moves 8 rows x 128 bytes, so
// every request to L2 is a whole 128-byte line.  LDS holds three K steps of
// weight rows and two of token rows (5 x 32 KB): weight rows, which come
// from HBM on first touch, are loaded two steps ahead, token rows one step
// ahead.  The 16-byte chunks of every 128-byte row are XOR-swizzled so that
// MFMA operand reads are free of bank conflicts.  Each wave runs one
// instruction stream in which the MFMAs of a slice (16 k) are interleaved
// with the LDS reads of the next slice and with its share of the loads of
// later K steps, spread over the slices so that the matrix cores keep
// issuing; one workgroup barrier per K step publishes a landed step.
//
// The kernels are persistent (one workgroup per compute unit) and build their
// tile lists on the device from the expert offsets (no host sync).  In
// gate/up a workgroup starts the first K steps of its next tile before it
// writes out the current one, so tile boundaries cost little; the down
// projection stages its fp32 output through LDS first.  In a tile whose
// token rows end early, the loads of rows past the end fall outside the
// token buffer's range, so they move no data (the hardware returns zeros
// for them), and gate/up waves skip the MFMAs of 32-row blocks past the end
// (the down projection computes them: with more than one variant of its K
// loop the compiler no longer keeps the accumulators in place).  In
// the down projection the tiles of an XCD's last, partial round are cut
// along K into pieces run by the workgroups that would otherwise idle; the
// pieces store fp32 partial sums and a second, short launch adds them in
// piece order and writes those tiles (no cross-workgroup waiting, and the
// same result on every call).  Gate/up tiles are shorter (K = H) and gained
// nothing from K pieces; their last round's tiles are cut into pieces of
// token rows instead, which need no second pass.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace {

constexpr int kGroupW = 8;  // weight tiles per L2 group
constexpr int kBK = 64;     // K step (elements): one 128-byte row slice
constexpr int kCPR = 8;     // 16-byte chunks per LDS row
// LDS: three buffers of one K step of the weight rows and two of the token
// rows (256 rows x 128 bytes = 32 KB each), 160 KB in all; K step s takes
// weight buffer s % 3 and token buffer 3 + s % 2
constexpr int kBuf = 256 * kCPR;   // 16-byte chunks per buffer

// Chunk c of row r sits at physical chunk c ^ ((r / 2) % 8): the 16 lanes of
// one MFMA operand read take 16 consecutive rows at one logical chunk, and
// those land in 16 distinct 16-byte slots of a 256-byte bank window (rows of
// one parity share a half of the window; r / 2 spreads them over it).
__device__ __forceinline__ int lds_slot(int row, int c) {
  return row * kCPR + (c ^ ((row >> 1) & 7));
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0f70)
#define GG_BARRIER() asm volatile("s_barrier" ::: "memory")

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource of `bytes` bytes at base (a raw buffer: stride 0; word 3
// as for every gfx9-family raw buffer).  A buffer load whose offset lies at
// or beyond `bytes` reads nothing from memory and yields zeros.
__device__ __forceinline__ i32x4 raw_buffer(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;
  return r;
}

// Tail split (down projection): the tiles that would leave most workgroups
// of an XCD idle in its last round are cut along K into np pieces of at
// least kMinPiece steps.
constexpr int kMaxPieces = 4;
constexpr int kMinPiece = 8;
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
// the nleft tiles of a last, partial round are cut into np pieces each
// (np * nleft <= nw).  Down projection: K pieces; each stores its fp32
// partial sums and a second launch adds the np partials in piece order and
// writes the tile.  Gate/up: pieces of the tile's 32-row token blocks, each
// a tile of its own (disjoint output rows, nothing to add): a piece of at
// most two blocks per wave column keeps the MFMAs and the token loads of
// the blocks it leaves out.
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
    p.np = gated ? min(nw / p.nleft, kMaxPieces)
                 : max(1, min(min(nw / p.nleft, kMaxPieces), p.nk_slice / kMinPiece));
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
          // (plain stores: as non-temporal 8-byte stores, partial lines, the
          // Mixtral prefill gate/up took 1.75 -> 1.85 ms)
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
        if (tl < t.rows)  // whole 1 KB row runs, written once: non-temporal
          __builtin_nontemporal_store(
              *reinterpret_cast<const u32x4*>(ob + row * 1024 + (c << 4)),
              reinterpret_cast<u32x4*>(yp + (size_t)(t.p0 + tl) * H + t.mt * 256 +
                                       ((c ^ (row & 15)) << 2)));
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

// NTW: the weight rows are loaded non-temporal (each weight tile meets one
// token tile: the experts hold one tile of rows on average), so that they
// do not push the token rows, which every weight tile reuses, out of L2.
template <bool GATED, bool NTW>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(
    const uint16_t* __restrict__ experts, uint64_t stride_elems,
    const uint16_t* __restrict__ tok, const int32_t* __restrict__ perm, int k_top,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_off, int E, int H,
    int F, int T, int ksplit, size_t plane, void* __restrict__ out, float* __restrict__ ws) {
  // weight buffers 0-2, token buffers 3-4 (the down projection's output is
  // staged in weight buffers 1-2 after the K loop)
  __shared__ u32x4 lds[5 * kBuf];

  // ksplit > 1 (down projection only): the K range is cut into ksplit
  // slices, slice ks writes its partial sums to plane ks of the output.
  const int K = (GATED ? H : F) / ksplit;
  const int xcd = blockIdx.x & 7;
  const int nw = gridDim.x >> 3;   // workgroups per XCD
  const int jw = blockIdx.x >> 3;  // this workgroup's place on its XCD
  const Plan pl = make_plan(GATED, tile_off, E, H, F, ksplit, xcd, nw, GATED || ws != nullptr);
  // work item w of this workgroup (rounds 0, 1, ...)
  auto locate = [&](int w, Tile& t) __attribute__((always_inline)) -> bool {
    if (pl.np < 2 || w < pl.nfull) {
      const int q = pl.q_beg + jw + w * nw;
      if (q >= pl.q_end) return false;
      tile_at(pl, q, tile_off, offsets, E, t);
      return true;
    }
    if (w > pl.nfull || jw >= pl.nleft * pl.np) return false;
    const int l = jw % pl.nleft, piece = jw / pl.nleft;
    tile_at(pl, pl.q_beg + pl.nfull * nw + l, tile_off, offsets, E, t);
    if (GATED) {  // token blocks [b0, b1) of the tile's nb
      const int nb = (t.rows + 31) >> 5;
      const int b0 = piece * nb / pl.np, b1 = (piece + 1) * nb / pl.np;
      if (b1 <= b0) return false;
      t.p0 += 32 * b0;
      t.rows = min(t.rows - 32 * b0, 32 * (b1 - b0));
      return true;
    }
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
  // [64 wave, 64 wave + 64), 8 + 8 instructions of 8 rows x 128 bytes; lane l
  // fills row l / 8, physical chunk l % 8, from the logical chunk stored there.
  const uint16_t* eb = experts;
  // row group i of a lane is row group i & 1 plus 8 i rows (the swizzle of a
  // row depends on (r / 2) % 8, which repeats every 16 rows): one base offset
  // per parity, the rest uniform; gathered token rows (gate/up) take one each
  uint32_t aoff[2], boff[GATED ? 8 : 2];
  i32x4 brs = raw_buffer(tok, (uint32_t)T * H * 2u);
  const bool tok_oob = (uint64_t)T * H * 2 <= 0x80000000ull;
  // gate/up: the slot ids of this lane's 8 token rows (rows past the tile's
  // end take its last row's)
  auto load_perm = [&](const Tile& t, int (&pv)[8]) {
    if (!GATED) return;
    int ln;  // the lane id, opaque so that the addressing below is not kept live across tiles
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
#pragma unroll
    for (int i = 0; i < 8; ++i) pv[i] = perm[t.p0 + min(wave * 64 + i * 8 + (ln >> 3), t.rows - 1)];
  };
  auto set_tile = [&](const Tile& t, const int (&pv)[8]) {
    eb = experts + (size_t)stride_elems * t.e;
    // the token buffer: all T tokens (gate/up, rows gathered through perm),
    // or exactly this tile's rows of the activation (down projection)
    if (!GATED) brs = raw_buffer(tok + (size_t)t.p0 * F, (uint32_t)t.rows * F * 2u);
    const int kbase = t.ks * K + t.k0 * kBK;
    int ln;  // the lane id, opaque as above
    asm volatile("v_and_b32 %0, 63, %1" : "=v"(ln) : "v"((int)threadIdx.x));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (ln >> 3);
      const int lc = (ln & 7) ^ ((r >> 1) & 7);
      if (i < 2) {
        uint32_t a;
        if (GATED) {  // waves 0-1 load gate rows, waves 2-3 the up rows
          const int f0 = t.mt * 128;
          a = (r < 128) ? (uint32_t)(f0 + r) * H : (uint32_t)F * H + (uint32_t)(f0 + r - 128) * H;
        } else {
          a = 2u * (uint32_t)F * H + (uint32_t)(t.mt * 256 + r) * F;
        }
        aoff[i] = a + lc * 8 + kbase;
      }
      // token rows, byte offsets in the token buffer (see brs); a row past the
      // tile's end lies outside it, so its loads read nothing
      if (GATED) {
        // past the end: offset 2^31 (outside a token buffer of at most 2^31
        // bytes), else the tile's last row again
        const uint32_t o = ((uint32_t)min(max(pv[i], 0) / k_top, T - 1) * H + lc * 8 + kbase) * 2u;
        boff[i] = (r >= t.rows && tok_oob) ? 0x80000000u : o;
      } else if (i < 2) {
        boff[i] = ((uint32_t)r * F + lc * 8 + kbase) * 2u;
      }
    }
  };
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)&lds[0]);
  // one 8-row load: operand op (0 weights, 1 tokens), row group i, K step s,
  // into LDS buffer b
  auto dma = [&](int s, int op, int i, int b) __attribute__((always_inline)) {
    const uint32_t dst = lds_base + (uint32_t)(b * kBuf * 16) +
                         (uint32_t)((wave * 64 + i * 8) * kCPR * 16);
    // one wait state between the M0 write and the LDS-DMA load that reads it
    if (op == 0) {
      const uint16_t* src = eb + aoff[i & 1] + (size_t)(i & 6) * 8 * (GATED ? H : F) + s * kBK;
      if constexpr (NTW)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
                     : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
                     : "memory", "m0");
    } else {
      // the row's offset in VADDR, the K step's in SOFFSET: a row inside the
      // buffer stays inside it at every K step of the row, a row past it stays
      // past it
      i32x4 rs;  // the resource is uniform; keep it in SGPRs
#pragma unroll
      for (int c = 0; c < 4; ++c) rs[c] = __builtin_amdgcn_readfirstlane(brs[c]);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(boff[GATED ? i : (i & 1)]), "s"(rs),
                     "s"(__builtin_amdgcn_readfirstlane(s * (kBK * 2) + (GATED ? 0 : (i & 6) * 8 * F * 2)))
                   : "memory", "m0");
    }
  };
  // the first K steps of a tile of nk steps: tokens and weights of steps 0
  // and 1, then the weights of step 2 (issued last: the first wait lets
  // exactly those 8 loads stay in flight)
  auto prologue = [&](int nk) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < nk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma(s, 1, i, 3 + s);
#pragma unroll
        for (int i = 0; i < 8; ++i) dma(s, 0, i, s);
      }
    if (nk > 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma(2, 0, i, 2);
    }
  };
  // The down projection's prologue in two parts around its epilogue, which
  // stages the output in weight buffers 1-2: the token rows of steps 0 and 1
  // and the weights of step 0 before it, the weights of steps 1 and 2 after
  // it (the same issue order of the step-1 and step-2 weights as above, so
  // the K loop's counted waits still hold).
  auto prologue_a = [&](int nk) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < nk) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dma(s, 1, i, 3 + s);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) dma(0, 0, i, 0);
  };
  auto prologue_b = [&](int nk) __attribute__((always_inline)) -> int {
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma(1, 0, i, 1);
    }
    if (nk > 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dma(2, 0, i, 2);
    }
    return (nk > 1 ? 8 : 0) + (nk > 2 ? 8 : 0);  // loads issued
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
    // fragments of one slice (16 k) of a K step: lane group kg reads chunk
    // 4 kg + n in slice n, a fixed permutation of the summation index applied
    // to both operands
    bf16x8 fa[2][4], fb[2][4];
    // the 8 reads of slice n of the step in weight buffer wb and token buffer
    // tb, in the order of first use by the MFMAs (row block 0 of the
    // weights, then token blocks 0..3, then weights 1..3)
    auto rd = [&](int buf, int wb, int tb, int n, int q) __attribute__((always_inline)) {
      const int c = kg * 4 + n;
      const u32x4* wst = lds + wb * kBuf;
      const u32x4* tst = lds + (3 + tb) * kBuf;
      if (q == 0) fa[buf][0] = as_bf16x8(wst[lds_slot(arow[0], c)]);
      else if (q < 5) {
        if (q - 1 < NJ) fb[buf][q - 1] = as_bf16x8(tst[lds_slot(brow[q - 1], c)]);
      } else fa[buf][q - 4] = as_bf16x8(wst[lds_slot(arow[q - 4], c)]);
    };
    // the 16 MFMAs of fragment buffer buf, with the 8 reads of slice rn of
    // buffers (wb, tb) into the other fragment buffer and some loads woven
    // in: the token loads of K step ts (8, into token buffer ts % 2) when LT,
    // and the weight rows [wr0, wr0 + wn) of K step ws into weight buffer wsb
    // when LW (4 rows: at every other MFMA of the second half; 2 rows: at
    // MFMAs 4 and 12).
    // RD / LT / LW are std::bool_constant (fixed) or bool (decided at run time).
    auto slice = [&](int buf, auto RD, int wb, int tb, int rn, auto LT, int ts, auto LW, int ws,
                     int wsb, auto WR0, auto WN) __attribute__((always_inline)) {
      constexpr int wr0 = decltype(WR0)::value, wnum = decltype(WN)::value;
      constexpr bool LT_SLICE = wr0 == 0;  // slice 3 (token loads at MFMAs 0-7)
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int i = m >> 2, j = m & 3;
        if (j < NJ)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
        if ((m & 1) == 0 && RD) rd(buf ^ 1, wb, tb, rn, m >> 1);
        // (every token load of a step precedes every weight load issued in
        // the same slice: the waits count the weight loads as the last ones)
        if (m < 8 && LT) dma(ts, 1, m, 3 + (ts & 1));
        if (wnum == 4 && m >= 8 && (m & 1) == 0 && LW) dma(ws, 0, wr0 + ((m - 8) >> 1), wsb);
        if (wnum == 2 && m == (LT_SLICE ? 10 : 4) && LW) dma(ws, 0, wr0, wsb);
        if (wnum == 2 && m == (LT_SLICE ? 14 : 12) && LW) dma(ws, 0, wr0 + 1, wsb);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
#pragma unroll
    for (int q = 0; q < 8; ++q) rd(0, 0, 0, 0, q);
    using I0 = std::integral_constant<int, 0>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I6 = std::integral_constant<int, 6>;
    // K step s in weight buffer w = s % 3 and token buffer t = s % 2:
    // slices 0-2 compute while reading slices 1-3, and load part of the
    // weight rows of step s+2 into the buffer freed one step earlier (gate/up:
    // rows 4-7 in slices 0-1; down projection: rows 2-7 in slices 0-2); then
    // every wave waits for its loads of step s+1 (the weights of step s+2,
    // issued after every token load, may stay in flight) and a barrier
    // publishes that step and ends all reads of step s (slice 3's fragments
    // are already in registers); slice 3 computes while reading slice 0 of
    // step s+1 and loading the tokens of step s+2 and the first weight rows
    // of step s+3 (gate/up 0-3, down 0-1) into the buffers just freed.
    // Spreading the loads over the slices keeps the matrix cores issuing
    // (measured: one burst per step was slower).  Step 0 takes no weight rows
    // in slices 0-2 (the prologue loaded all of step 2); the steps 1 .. nk-4
    // take the branch-free body; the last three decide at run time.
    auto step = [&](int s, int w, auto W2, auto NX, auto LT, auto LW, bool wait_all)
        __attribute__((always_inline)) {
      const int w1 = w == 2 ? 0 : w + 1, wp = w == 0 ? 2 : w - 1, t = s & 1;
      if constexpr (GATED) {  // weight rows 0-3 | 4-5, 6-7
        slice(0, std::true_type(), w, t, 1, std::false_type(), 0, W2, s + 2, wp, I4(), I2());
        slice(1, std::true_type(), w, t, 2, std::false_type(), 0, W2, s + 2, wp, I6(), I2());
        slice(0, std::true_type(), w, t, 3, std::false_type(), 0, std::false_type(), 0, 0, I0(), I0());
      } else {  // weight rows 0-1 | 2-3, 4-5, 6-7
        slice(0, std::true_type(), w, t, 1, std::false_type(), 0, W2, s + 2, wp, I2(), I2());
        slice(1, std::true_type(), w, t, 2, std::false_type(), 0, W2, s + 2, wp, I4(), I2());
        slice(0, std::true_type(), w, t, 3, std::false_type(), 0, W2, s + 2, wp, I6(), I2());
      }
      if (wait_all) WAIT_VMCNT(0); else WAIT_VMCNT(8);
      GG_BARRIER();
      slice(1, NX, w1, t ^ 1, 0, LT, s + 2, LW, s + 3, w, I0(),
            std::integral_constant<int, GATED ? 4 : 2>());
      return w1;
    };
    int s = 0, w = 0;
    if (nk > 3) w = step(s++, w, std::false_type(), std::true_type(), std::true_type(), std::true_type(), false);
    for (; s + 3 < nk; ++s)
      w = step(s, w, std::true_type(), std::true_type(), std::true_type(), std::true_type(), false);
    for (; s < nk; ++s)
      w = step(s, w, s >= 1 && s + 2 < nk, s + 1 < nk, s + 2 < nk, false, s + 2 >= nk);
  };

  int round = 0;
  int st_groups = 0;  // gate/up: token-block groups the wave stored after the current tile's first loads
  int tail_loads = 0;  // down: the current tile's first loads issued after the previous epilogue
  Tile cur, nxt;
  if (!locate(round, cur)) return;
  {
    int pv[8];
    load_perm(cur, pv);
    set_tile(cur, pv);
  }
  prologue(cur.nk);
  // one tile for waves that compute NJ token blocks; returns whether a next
  // tile exists (then its first stages are in flight)
  auto tile = [&](auto NJc) __attribute__((always_inline)) -> bool {
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
    int pn[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (more) load_perm(nxt, pn);
    kloop(NJc, acc, cur.nk);
    // every load of the tile has landed; end every wave's reads of the ring,
    // then start the next tile's first K steps under this tile's epilogue
    // (the down projection stages its output in weight buffers 1-2 and
    // loads their weights after it)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (more) {
      set_tile(nxt, pn);
      if (GATED) prologue(nxt.nk);
      else prologue_a(nxt.nk);
    }
    // read each accumulator where it is used: left to itself the compiler
    // copies all of them to VGPRs at once and spills
    auto from_acc = [&](int i, int j, int q) __attribute__((always_inline)) -> f32x4 {
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
      write_tile<GATED>(cur, [](int) {}, from_acc, out, F, H, plane, (uint8_t*)&lds[kBuf], wave);
      if (GATED) {  // groups j with a row of this wave's token block 2 j + wn
        st_groups = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) st_groups += (2 * j + wn) * 32 < cur.rows ? 1 : 0;
      }
    } else {  // a piece: its partial sums, for the launch that finishes the tile
      f32x4* dst = part_base(ws, xcd * nw + jw, wave);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[((i * 4 + j) * 4 + q) * 64] = from_acc(i, j, q);
    }
    if (!GATED && more) {
      // every wave is done with the output staging
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      tail_loads = prologue_b(nxt.nk);
    }
    return more;
  };
  for (;;) {
    // this tile's first stages have landed; the barrier also ends every
    // wave's reads of the previous tile's output staging.  Gate/up issued its
    // previous output stores (8 per token-block group the wave wrote) after
    // this tile's first loads, and vmcnt counts loads and stores in issue
    // order: those stores may stay in flight here (the K loop's first wait
    // takes them in); the down projection waits for everything.
    if (GATED) {
      switch (st_groups) {
        case 1: WAIT_VMCNT(8); break;
        case 2: WAIT_VMCNT(16); break;
        case 3: WAIT_VMCNT(24); break;
        case 4: WAIT_VMCNT(32); break;
        default: WAIT_VMCNT(0); break;
      }
    } else {
      // the down projection: its step-1 and step-2 weights, issued after
      // the epilogue, may stay in flight
      if (tail_loads == 16) WAIT_VMCNT(16);
      else if (tail_loads == 8) WAIT_VMCNT(8);
      else WAIT_VMCNT(0);
    }
    GG_BARRIER();
    const int nb = (cur.rows + 31) >> 5;        // 32-row token blocks in the tile
    const int nj = max((nb - wn + 1) >> 1, 1);  // this wave's (at least one)
    bool more;
    if (GATED) {
      switch (nj) {
        case 1: more = tile(std::integral_constant<int, 1>()); break;
        case 2: more = tile(std::integral_constant<int, 2>()); break;
        case 3: more = tile(std::integral_constant<int, 3>()); break;
        default: more = tile(std::integral_constant<int, 4>()); break;
      }
    } else {
      // the down projection computes every token block: with several K loop
      // variants in one kernel the compiler no longer keeps its accumulators
      // in place (it copies all of them every K step)
      more = tile(std::integral_constant<int, 4>());
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
  // With the tail-split workspace the tiles of the last, partial round are
  // cut along K anyway (the makespan in K steps comes out the same as with
  // two K halves), and one plane halves the combine's reads: Mixtral prefill
  // layer 2.625 -> 2.573 ms.  Without it, split the long K in two when there
  // are too few tiles to fill the 256 CUs a few times over.
  if (a.gws) return 1;
  const int max_tiles = (a.S + GG_BT - 1) / GG_BT + (a.E < a.S ? a.E : a.S);
  return (max_tiles * (a.H / 256) < 3 * 256 && a.F % (2 * kBK) == 0) ? 2 : 1;
}

// the experts hold at most one token tile of rows on average
static bool weights_once(const ExpertArgs& a) { return a.S <= (int64_t)GG_BT * a.E; }

int launch_grouped_gate_up(const ExpertArgs& a, hipStream_t st) {
  auto kern = weights_once(a) ? grouped_gemm_kernel<true, true> : grouped_gemm_kernel<true, false>;
  kern<<<persistent_grid(), 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.x, a.perm, a.k, a.offsets,
      a.tile_off, a.E, a.H, a.F, a.T, 1, 0, a.act, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_down(const ExpertArgs& a, int ksplit, hipStream_t st) {
  auto kern =
      weights_once(a) ? grouped_gemm_kernel<false, true> : grouped_gemm_kernel<false, false>;
  kern<<<persistent_grid(), 256, 0, st>>>(
      (const uint16_t*)a.experts, a.stride_elems, (const uint16_t*)a.act, a.perm, a.k,
      a.offsets, a.tile_off, a.E, a.H, a.F, a.T, ksplit, (size_t)a.S * a.H, a.yp, a.gws);
  if (a.gws)
    grouped_fixup_kernel<false><<<4 * persistent_grid(), 256, 0, st>>>(
        a.offsets, a.tile_off, a.E, a.H, a.F, ksplit, (size_t)a.S * a.H, a.yp, a.gws,
        persistent_grid() / 8);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
