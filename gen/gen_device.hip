// gen_device.hip -- device side of the seeded input generator: the same
// values as gen/gen.c, computed on the GPU from the same definition
// (gen_core.h), for inputs too large to generate on the host (the 90 GB
// stacked-layer weights).  Holds input generation only.  Built with
// floating-point contraction off, like the host side.
#include <hip/hip_runtime.h>

#include "gen_core.h"

namespace {

__global__ void normal_bf16_kernel(uint64_t state, uint64_t idx0, uint64_t n, double sigma,
                                   uint16_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = gen_f32_to_bf16(gen_to_f32(sigma * gen_normal_at(state, idx0 + i)));
}

__global__ void normal_f32_kernel(uint64_t state, uint64_t idx0, uint64_t n, double sigma,
                                  float* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = gen_to_f32(sigma * gen_normal_at(state, idx0 + i));
}

}  // namespace

extern "C" {

// Values idx0 .. idx0+n-1 of stream (seed, layer, tensor) into device memory
// `out` (bf16 bit patterns or fp32), on `stream`.  Returns 0 or a HIP error.
int gen_device_normal_bf16(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t idx0,
                           uint64_t n, double sigma, uint16_t* out, void* stream) {
  if (n == 0) return 0;
  normal_bf16_kernel<<<4096, 256, 0, (hipStream_t)stream>>>(
      gen_stream_state(seed, layer, tensor), idx0, n, sigma, out);
  return (int)hipGetLastError();
}

int gen_device_normal_f32(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t idx0,
                          uint64_t n, double sigma, float* out, void* stream) {
  if (n == 0) return 0;
  normal_f32_kernel<<<4096, 256, 0, (hipStream_t)stream>>>(
      gen_stream_state(seed, layer, tensor), idx0, n, sigma, out);
  return (int)hipGetLastError();
}

}  // extern "C"
