// quantize.hip -- conversion of bf16 expert weights to uint8 codes with one
// affine map per weight matrix (a one-time step before MOE_EXPERT_U8 layers
// run, not part of the forward pass); and the fp16 copy of a uint8 layer's
// input that its expert kernels read.
//
// The pages quantise each expert matrix after training from its minimum and
// maximum into 255 levels and read it back as (q - zero point) * scale
// [www.pnsm.cn/news/1892388.html sec. 3.1 and sec. 5.2].  Per matrix,
// in fp32 with IEEE division and rint (ties to even):
//   mn = min(0, min w), mx = max(0, max w), scale = (mx - mn) / 255 (1 if 0),
//   zero = clamp(rint(-mn / scale), 0, 255),
//   q = clamp(rint(w / scale) + zero, 0, 255).
// Four launches: clear the parameter blocks; per-matrix min/max by integer
// atomics on an order-preserving encoding of the floats (exact, so the order
// of the atomics does not matter); scale and zero point; the codes.
#include "common.h"
#include "kernels.h"

namespace {

// float -> int32 ordered like the floats; -0 is taken as +0
__device__ __forceinline__ int ord_enc(float v) {
  const int i = __float_as_int(v + 0.0f);
  return i < 0 ? i ^ 0x7FFFFFFF : i;
}
__device__ __forceinline__ float ord_dec(int i) { return __int_as_float(i < 0 ? i ^ 0x7FFFFFFF : i); }

// the 64-byte parameter block at byte 3*H*F of an expert (words: scale[3],
// zero[3], min[3], max[3], pad[4]); min and max hold ord_enc values until
// the finalize kernel
__device__ __forceinline__ uint32_t* params(uint8_t* dst, uint64_t stride, int e, size_t hf) {
  return reinterpret_cast<uint32_t*>(dst + (size_t)e * stride + 3 * hf);
}

constexpr int kChunk = 256 * 16 * 8;  // elements per workgroup and pass: 16 per thread, 8 rounds

__global__ __launch_bounds__(256) void q_clear(uint8_t* dst, uint64_t stride, size_t hf, int E) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < E * 16) params(dst, stride, i >> 4, hf)[i & 15] = 0u;  // ord_enc(0) == 0
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// grid (chunks, 3, E): min and max of matrix m of expert e
__global__ __launch_bounds__(256) void q_minmax(const uint8_t* src, uint64_t sstride,
                                                uint8_t* dst, uint64_t dstride, size_t hf) {
  const int m = blockIdx.y, e = blockIdx.z;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(src + (size_t)e * sstride) + (size_t)m * hf;
  float mn = 0.0f, mx = 0.0f;
  const size_t beg = (size_t)blockIdx.x * kChunk;
  for (int r = 0; r < 8; ++r) {
    const size_t i = beg + ((size_t)r * 256 + threadIdx.x) * 16;
    if (i >= hf) break;
    const u32x4 a = *reinterpret_cast<const u32x4*>(w + i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(w + i + 8);
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mn = fminf(mn, fminf(bf16_lo(v[j]), bf16_hi(v[j])));
      mx = fmaxf(mx, fmaxf(bf16_lo(v[j]), bf16_hi(v[j])));
    }
  }
  int lo = ord_enc(mn), hi = ord_enc(mx);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  __shared__ int red[2][4];
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = lo;
    red[1][threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lo = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    hi = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    uint32_t* p = params(dst, dstride, e, hf);
    atomicMin(reinterpret_cast<int*>(p + 6 + m), lo);
    atomicMax(reinterpret_cast<int*>(p + 9 + m), hi);
  }
}

__global__ __launch_bounds__(64) void q_finalize(uint8_t* dst, uint64_t stride, size_t hf, int E) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= E * 3) return;
  const int e = i / 3, m = i - 3 * e;
  uint32_t* p = params(dst, stride, e, hf);
  const float mn = ord_dec((int)p[6 + m]), mx = ord_dec((int)p[9 + m]);
  float scale = (mx - mn) / 255.0f;
  if (!(scale > 0.0f)) scale = 1.0f;
  int zero = (int)rintf(-mn / scale);
  zero = min(max(zero, 0), 255);
  p[m] = __float_as_uint(scale);
  p[3 + m] = (uint32_t)zero;
  p[6 + m] = __float_as_uint(mn);
  p[9 + m] = __float_as_uint(mx);
}

// grid (chunks, 3, E): the codes of matrix m of expert e
__global__ __launch_bounds__(256) void q_codes(const uint8_t* src, uint64_t sstride, uint8_t* dst,
                                               uint64_t dstride, size_t hf) {
  const int m = blockIdx.y, e = blockIdx.z;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(src + (size_t)e * sstride) + (size_t)m * hf;
  uint8_t* q = dst + (size_t)e * dstride + (size_t)m * hf;
  const uint32_t* p = params(dst, dstride, e, hf);
  const float scale = __uint_as_float(p[m]);
  const int zero = (int)p[3 + m];
  const size_t beg = (size_t)blockIdx.x * kChunk;
  for (int r = 0; r < 8; ++r) {
    const size_t i = beg + ((size_t)r * 256 + threadIdx.x) * 16;
    if (i >= hf) break;
    const u32x4 a = *reinterpret_cast<const u32x4*>(w + i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(w + i + 8);
    const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t pair = v[2 * j + (h >> 1)];
        const float x = (h & 1) ? bf16_hi(pair) : bf16_lo(pair);
        const int c = min(max((int)rintf(x / scale) + zero, 0), 255);
        word |= (uint32_t)c << (8 * h);
      }
      out[j] = word;
    }
    *reinterpret_cast<u32x4*>(q + i) = u32x4{out[0], out[1], out[2], out[3]};
  }
}

// 8 bf16 -> 8 fp16 per thread (round toward zero: exact where bf16 values
// are fp16 values)
__global__ __launch_bounds__(256) void to_f16_kernel(const uint16_t* __restrict__ src, size_t n,
                                                     uint16_t* __restrict__ dst) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i + 8 <= n) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + i);
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(d[j] << 16),
                                                                     __uint_as_float(d[j] & 0xFFFF0000u)));
    *reinterpret_cast<u32x4*>(dst + i) = u32x4{o[0], o[1], o[2], o[3]};
  } else {
    for (size_t j = i; j < n; ++j) {
      const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float((uint32_t)src[j] << 16), 0.0f);
      dst[j] = (uint16_t)__builtin_bit_cast(uint32_t, h);
    }
  }
}

}  // namespace

int launch_to_f16(const uint16_t* src, size_t n, uint16_t* dst, hipStream_t st) {
  const size_t threads = (n + 7) / 8;
  to_f16_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(src, n, dst);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize_u8(const void* src, uint64_t src_stride, int E, int H, int F, void* dst,
                       uint64_t dst_stride, hipStream_t st) {
  const size_t hf = (size_t)H * F;
  const dim3 grid((unsigned)((hf + kChunk - 1) / kChunk), 3, (unsigned)E);
  uint8_t* d = (uint8_t*)dst;
  const uint8_t* s = (const uint8_t*)src;
  q_clear<<<(E * 16 + 255) / 256, 256, 0, st>>>(d, dst_stride, hf, E);
  q_minmax<<<grid, 256, 0, st>>>(s, src_stride, d, dst_stride, hf);
  q_finalize<<<(E * 3 + 63) / 64, 64, 0, st>>>(d, dst_stride, hf, E);
  q_codes<<<grid, 256, 0, st>>>(s, src_stride, d, dst_stride, hf);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
