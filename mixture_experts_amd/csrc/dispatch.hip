// dispatch.hip -- step 3: group the T*k (token, slot) pairs by expert.
//
// The pages batch all tokens routed to one expert together before the
// expert GEMMs [zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析"
// sec. 3.3, stage 3].  Here that is a stable counting sort of the slots
// s = t*k + j by expert: counts[e], offsets = exclusive prefix sum,
// perm[p] = s for the p-th pair in (expert, token) order, inv[s] = p.
//
// With a capacity C an expert keeps the first C of its pairs in slot order
// (www.cf-1.com/news/4750020/ sec. 4.2, --expert-capacity): counts, offsets
// and the tile schedule count the kept pairs, a dropped pair gets inv = -1,
// perm is -1 beyond the kept pairs.
//
// Up to 8192 pairs, one workgroup does it all (dispatch_one_kernel: 16 waves
// rank their share of the slots as below, the per-wave counts give each
// wave's base per expert, the experts are scanned in parallel, every thread
// scatters); beyond that three kernels.  All deterministic (no ordering
// depends on atomics):
//   hist    one wave per run of 512 slots; the rank of a slot among the
//           earlier slots of the same expert in its run comes from a
//           bit-sliced ballot match (lanes holding the same expert id) and a
//           popcount; per-run expert counts go to hist[run][e].
//   scan    one workgroup: per-expert prefix over runs, offsets, the tile
//           schedule of the grouped GEMM and the list of non-empty experts.
//   scatter one thread per slot: p = run base of its expert + its rank.
#include "common.h"
#include "kernels.h"

namespace {

// Exclusive prefix over the experts, for a workgroup of at least 256
// threads (E <= 256): offsets[e] = sum of sc[e'] for e' < e, tile_off[e] the
// same over ceil(sc / tile_rows), active[] = the experts with sc > 0 in
// ascending order, and the totals at [E].  Waves 0-3 scan 64 experts each
// (shuffle-up steps), then add the earlier waves' totals.  off_l (LDS, E+1)
// receives the offsets too.  Ends with a workgroup barrier.
__device__ void expert_prefix(const int32_t* sc, int E, int tile_rows,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
                              int32_t* __restrict__ active, int32_t* off_l) {
  __shared__ int32_t wsum[4][3];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c = 0, t = 0, f = 0;
  int ic = 0, it = 0, iff = 0;  // inclusive prefixes within the wave
  if (tid < 256) {
    c = tid < E ? sc[tid] : 0;
    t = (c + tile_rows - 1) / tile_rows;
    f = c > 0 ? 1 : 0;
    ic = c;
    it = t;
    iff = f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int uc = __shfl_up(ic, d), ut = __shfl_up(it, d), uf = __shfl_up(iff, d);
      if (lane >= d) {
        ic += uc;
        it += ut;
        iff += uf;
      }
    }
    if (lane == 63) {
      wsum[wave][0] = ic;
      wsum[wave][1] = it;
      wsum[wave][2] = iff;
    }
  }
  __syncthreads();
  if (tid < 256) {
    int bc = 0, bt = 0, bf = 0;
    for (int w = 0; w < wave; ++w) {
      bc += wsum[w][0];
      bt += wsum[w][1];
      bf += wsum[w][2];
    }
    const int ec = bc + ic - c, et = bt + it - t, ef = bf + iff - f;  // exclusive
    if (tid < E) {
      offsets[tid] = ec;
      tile_off[tid] = et;
      off_l[tid] = ec;
      if (f) active[ef] = tid;
    }
    if (tid == E - 1) {
      offsets[E] = ec + c;
      tile_off[E] = et + t;
      off_l[E] = ec + c;
      active[E] = ef + f;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(64) void dispatch_hist_kernel(const int32_t* __restrict__ idx,
                                                           int S, int E, int nbits,
                                                           int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ rank) {
  __shared__ int32_t cnt[MOE_MAX_EXPERTS];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * DISPATCH_RUN;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the run's expert ids, all loads in flight together
  int ev[DISPATCH_RUN / 64];
#pragma unroll
  for (int c = 0; c < DISPATCH_RUN / 64; ++c) {
    const int s = base + c * 64 + lane;
    ev[c] = s < S ? idx[s] : 0;
  }
#pragma unroll
  for (int c = 0; c < DISPATCH_RUN / 64; ++c) {
    const int s = base + c * 64 + lane;
    const bool valid = s < S;
    const int e = ev[c];
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const uint64_t earlier = match & below;
    const int c0 = valid ? cnt[e] : 0;
    __syncthreads();
    if (valid) {
      rank[s] = c0 + __popcll(earlier);
      if (earlier == 0) cnt[e] = c0 + __popcll(match);
    }
    __syncthreads();
  }
  for (int e = lane; e < E; e += 64) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads, thread (c, e) = (tid / 256, tid % 256):
// base[r][e] = sum of hist[r'][e] for r' < r (the expert's pairs in earlier
// runs), each thread summing one quarter of the runs (its loads in flight
// together) and starting from the quarters before it.  counts[e] = the pairs
// kept (capped at cap when cap > 0).  tile_off[e] = sum over e' < e of
// ceil(counts[e'] / tile_rows).  active[0..n) = the experts with counts > 0,
// ascending; active[E] = n.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int nrun, int E, int tile_rows, int cap,
    int32_t* __restrict__ base, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_off, int32_t* __restrict__ active) {
  __shared__ int32_t qs[4][MOE_MAX_EXPERTS];  // per-quarter sums
  __shared__ int32_t sc[MOE_MAX_EXPERTS];
  __shared__ int32_t off_l[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x, q = tid >> 8, e = tid & 255;
  const int rq = (nrun + 3) / 4;  // runs per quarter
  const int r_beg = q * rq, r_end = min(nrun, r_beg + rq);
  int sum = 0;
  int h0[16] = {};  // a quarter of at most 16 runs: its counts, kept for the second pass
  if (e < E) {
    for (int r0 = r_beg; r0 < r_end; r0 += 16) {
      int h[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) h[j] = r0 + j < r_end ? hist[(size_t)(r0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sum += h[j];
        h0[j] = h[j];
      }
    }
  }
  qs[q][e] = sum;
  __syncthreads();
  if (e < E && rq <= 16) {
    int run = 0;
    for (int p = 0; p < q; ++p) run += qs[p][e];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (r_beg + j < r_end) base[(size_t)(r_beg + j) * E + e] = run;
      run += h0[j];
    }
  } else if (e < E) {
    int run = 0;
    for (int p = 0; p < q; ++p) run += qs[p][e];
    for (int r0 = r_beg; r0 < r_end; r0 += 16) {
      int h[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) h[j] = r0 + j < r_end ? hist[(size_t)(r0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (r0 + j < r_end) base[(size_t)(r0 + j) * E + e] = run;
        run += h[j];
      }
    }
  }
  if (e < E && q == 0) {
    int tot = qs[0][e] + qs[1][e] + qs[2][e] + qs[3][e];
    if (cap > 0 && tot > cap) tot = cap;
    counts[e] = tot;
    sc[e] = tot;
  }
  __syncthreads();
  expert_prefix(sc, E, tile_rows, offsets, tile_off, active, off_l);
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ rank,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets, int S, int E,
    int cap, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const int e = idx[s];
  const int g = base[(size_t)(s / DISPATCH_RUN) * E + e] + rank[s];  // rank in the expert
  if (s >= offsets[E]) perm[s] = -1;  // beyond the kept pairs (never a kept p below)
  if (cap > 0 && g >= cap) {
    inv[s] = -1;  // dropped
    return;
  }
  const int p = offsets[e] + g;
  // p is in [0, offsets[E]) by construction; the guard keeps a logic error
  // from turning into an out-of-bounds store
  if (p >= 0 && p < S) {
    perm[p] = s;
    inv[s] = p;
  } else {
    inv[s] = -1;
  }
}

// The whole dispatch of S <= D1_MAX pairs in one workgroup of 16 waves.
// Wave w ranks slots [w SW, (w+1) SW) (SW a multiple of 64) within the wave
// by the same ballot match; wh[w][e] then turns from that wave's count into
// the pairs of expert e in waves before w.
constexpr int D1_MAX = 8192;
__global__ __launch_bounds__(1024) void dispatch_one_kernel(
    const int32_t* __restrict__ idx, int S, int E, int nbits, int tile_rows, int cap,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
    int32_t* __restrict__ active, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t idx_l[D1_MAX];
  __shared__ int32_t rank_l[D1_MAX];
  __shared__ int32_t wh[16][MOE_MAX_EXPERTS];
  __shared__ int32_t tot[MOE_MAX_EXPERTS];
  __shared__ int32_t off_l[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {  // the expert ids, all loads in flight together
    int v[D1_MAX / 1024];
#pragma unroll
    for (int j = 0; j < D1_MAX / 1024; ++j) v[j] = tid + 1024 * j < S ? idx[tid + 1024 * j] : 0;
#pragma unroll
    for (int j = 0; j < D1_MAX / 1024; ++j)
      if (tid + 1024 * j < S) idx_l[tid + 1024 * j] = v[j];
  }
  for (int i = tid; i < 16 * MOE_MAX_EXPERTS; i += 1024) wh[i / MOE_MAX_EXPERTS][i % MOE_MAX_EXPERTS] = 0;
  __syncthreads();
  const int SW = ((S + 1023) / 1024) * 64;  // slots per wave
  int32_t* cnt = wh[wave];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = 0; c * 64 < SW; ++c) {
    const int sl = wave * SW + c * 64 + lane;
    const bool valid = sl < S;
    const int e = valid ? idx_l[sl] : 0;
    uint64_t match = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const uint64_t earlier = match & below;
    const int c0 = valid ? cnt[e] : 0;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      rank_l[sl] = c0 + __popcll(earlier);
      if (earlier == 0) cnt[e] = c0 + __popcll(match);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (tid < E) {  // per-wave bases of expert tid, its total kept
    int run = 0;
    for (int w = 0; w < 16; ++w) {
      const int h = wh[w][tid];
      wh[w][tid] = run;
      run += h;
    }
    tot[tid] = (cap > 0 && run > cap) ? cap : run;
    counts[tid] = tot[tid];
  }
  __syncthreads();
  expert_prefix(tot, E, tile_rows, offsets, tile_off, active, off_l);
  for (int sl = tid; sl < S; sl += 1024) {
    const int e = idx_l[sl];
    const int g = wh[sl / SW][e] + rank_l[sl];  // rank of the pair in its expert
    if (sl >= off_l[E]) perm[sl] = -1;          // beyond the kept pairs
    if (cap > 0 && g >= cap) {
      inv[sl] = -1;  // dropped
      continue;
    }
    const int p = off_l[e] + g;
    if (p >= 0 && p < S) {  // by construction; kept as in the scatter kernel
      perm[p] = sl;
      inv[sl] = p;
    } else {
      inv[sl] = -1;
    }
  }
}

}  // namespace

int launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int S = a.S;
  if (S <= D1_MAX) {
    int nb = 0;
    while ((1 << nb) < a.E) ++nb;
    dispatch_one_kernel<<<1, 1024, 0, st>>>(a.idx, S, a.E, nb, a.tile_rows, a.capacity,
                                            a.counts, a.offsets, a.tile_off, a.active, a.perm,
                                            a.inv);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int nrun = (S + DISPATCH_RUN - 1) / DISPATCH_RUN;
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  dispatch_hist_kernel<<<nrun, 64, 0, st>>>(a.idx, S, a.E, nbits, a.hist, a.rank);
  dispatch_scan_kernel<<<1, 1024, 0, st>>>(a.hist, nrun, a.E, a.tile_rows,
                                                      a.capacity, a.base, a.counts, a.offsets,
                                                      a.tile_off, a.active);
  dispatch_scatter_kernel<<<(S + 255) / 256, 256, 0, st>>>(a.idx, a.rank, a.base, a.offsets, S,
                                                           a.E, a.capacity, a.perm, a.inv);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
