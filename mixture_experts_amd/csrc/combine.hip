// combine.hip -- step 5: y[t] = sum_{j<k} w[t][j] * yp[inv[t*k+j]], slots in
// ascending order, one fp32 fused multiply-add per slot, no atomics, slots
// dropped by an expert capacity (inv < 0) skipped; plus the residual h[t]
// when the layer runs inside a residual stack.
//
// The pages accumulate the K expert outputs weighted by their gate scores
// [zskr.cn/news/2275853 "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.3
// stage 5, there with atomicAdd; www.pnsm.cn/news/1892388.html sec. 2.2]; here
// each output element is owned by one thread, which fixes the order.  The
// residual is taken inside the forward call as on www.pnsm.cn page sec. 2.1.
// HBM-bound: 16-byte loads and stores, consecutive threads on consecutive
// columns; for k <= 8 a thread's k row loads are in flight together.
#include "common.h"
#include "kernels.h"

namespace {

// KT > 0: k == KT and nplanes == NP fixed at compile time, so that a
// thread's KT (x NP) row loads are issued together, then summed in slot
// order; KT == 0: any k and nplanes, slot by slot.
template <int KT, int NP>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ yp,
                                                      int nplanes,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv,
                                                      const float* resid, int T, int H, int k,
                                                      float* y) {
  const int h4n = H >> 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * h4n) return;
  const int t = (int)(i / h4n), c = (int)(i % h4n) * 4;
  const int S = T * k;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  if constexpr (KT > 0) {
    float wj[KT];
    int pj[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      wj[j] = w[(size_t)t * KT + j];
      pj[j] = inv[(size_t)t * KT + j];
    }
    // each per-pair row is read once: non-temporal loads; a pair dropped by
    // the expert capacity (inv < 0) reads row 0 and adds nothing
    f32x4 v[KT][NP];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int p = min(max(pj[j], 0), S - 1);  // in range by construction
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
        v[j][pl] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(yp + ((size_t)pl * S + p) * H + c));
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      f32x4 u = v[j][0];
#pragma unroll
      for (int pl = 1; pl < NP; ++pl) u += v[j][pl];  // split-K partial sums, in plane order
      const bool kept = pj[j] >= 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = kept ? fmaf(wj[j], u[q], acc[q]) : acc[q];
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const float wj = w[(size_t)t * k + j];
      const int pi = inv[(size_t)t * k + j];
      if (pi < 0) continue;  // a pair dropped by the expert capacity
      const int p = min(pi, S - 1);  // in range by construction
      f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yp + (size_t)p * H + c));
      for (int pl = 1; pl < nplanes; ++pl)  // partial sums of a split K, in plane order
        v += __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(yp + ((size_t)pl * S + p) * H + c));
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
    }
  }
  if (resid) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(resid + (size_t)t * H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = r[q] + acc[q];
  }
  *reinterpret_cast<f32x4*>(y + (size_t)t * H + c) = acc;
}

}  // namespace

int launch_combine(const float* yp, int nplanes, const float* w, const int32_t* inv,
                   const float* resid, int T, int H, int k, float* y, hipStream_t st) {
  const int64_t n = (int64_t)T * (H / 4);
  const unsigned grid = (unsigned)((n + 255) / 256);
#define COMBINE(KT, NP) combine_kernel<KT, NP><<<grid, 256, 0, st>>>(yp, nplanes, w, inv, resid, T, H, k, y)
#define COMBINE_K(KT) \
  case KT:            \
    if (nplanes == 1) \
      COMBINE(KT, 1); \
    else              \
      COMBINE(KT, 2); \
    break
  if (nplanes < 1 || nplanes > 2) {
    COMBINE(0, 0);
  } else {
    switch (k) {
      COMBINE_K(1);
      COMBINE_K(2);
      COMBINE_K(3);
      COMBINE_K(4);
      COMBINE_K(5);
      COMBINE_K(6);
      COMBINE_K(7);
      COMBINE_K(8);
      default: COMBINE(0, 0);
    }
  }
#undef COMBINE_K
#undef COMBINE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
