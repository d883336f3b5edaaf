// expert_f32.hip -- steps 4 and 5 for fp32 layers, plain fp32 FMA, one thread
// per output element (fp32 layers are the small exactness-checked case).
//
// SwiGLU expert without bias [zskr.cn/news/2275853
// "Colibri：面向MoE架构的C语言高效推理引擎解析" sec. 3.1, sec. 3.3 stage 4]:
// act[p][f] = SiLU(g) * u with g = x[t] . Wg[f], u = x[t] . Wu[f] (t = perm[p] / k),
// then yp[p][h] = act[p] . Wd[h].
#include "common.h"
#include "kernels.h"

namespace {

__global__ __launch_bounds__(256) void f32_gate_up_kernel(
    const float* __restrict__ x, const float* __restrict__ experts, uint64_t stride_elems,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, int E, int k_top,
    int H, int F, int S, int T, float* __restrict__ act) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)S * F) return;
  const int p = (int)(i / F), f = (int)(i % F);
  const int e = upper_segment(offsets, E, p);
  const float* xr = x + (size_t)min(max(perm[p], 0) / k_top, T - 1) * H;
  const float* wg = experts + (size_t)e * stride_elems + (size_t)f * H;
  const float* wu = wg + (size_t)F * H;
  float g = 0.0f, u = 0.0f;
  for (int h = 0; h < H; ++h) {
    g = fmaf(xr[h], wg[h], g);
    u = fmaf(xr[h], wu[h], u);
  }
  act[(size_t)p * F + f] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void f32_down_kernel(
    const float* __restrict__ act, const float* __restrict__ experts, uint64_t stride_elems,
    const int32_t* __restrict__ offsets, int E, int H, int F, int S, float* __restrict__ yp) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)S * H) return;
  const int p = (int)(i / H), h = (int)(i % H);
  const int e = upper_segment(offsets, E, p);
  const float* ar = act + (size_t)p * F;
  const float* wd = experts + (size_t)e * stride_elems + 2 * (size_t)F * H + (size_t)h * F;
  float s = 0.0f;
  for (int f = 0; f < F; ++f) s = fmaf(ar[f], wd[f], s);
  yp[(size_t)p * H + h] = s;
}

}  // namespace

int launch_f32_gate_up(const ExpertArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.S * a.F;
  f32_gate_up_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
      (const float*)a.x, (const float*)a.experts, a.stride_elems, a.perm, a.offsets, a.E, a.k,
      a.H, a.F, a.S, a.T, (float*)a.act);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_f32_down(const ExpertArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.S * a.H;
  f32_down_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
      (const float*)a.act, (const float*)a.experts, a.stride_elems, a.offsets, a.E, a.H, a.F,
      a.S, a.yp);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
