// Online per-tensor fp8 quantisation of Q, K or V ("FlashPrefill V2", Sec.
// 3.3 FP8 paragraph: e4m3 operands with one absmax-derived scale per
// tensor): amax = max |x|, scale = amax / 448 (1 for an all-zero tensor),
// code = e4m3(x / scale), round to nearest even, saturated at 448.  The
// scale stays on the device, where the fp8 pipeline reads it
// (bslp_problem.scales_dev), so nothing waits for the host.
//
// Four launches on the caller's stream: clear the accumulator, a grid-stride
// max over 16-byte loads, the scale, the codes.  The accumulator is the output
// float itself, holding the maximum as integer bits while it is built
// (non-negative floats order like their bit patterns).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace bslp {
namespace {

constexpr float kE4M3Max = 448.f;

template <int DT>
__device__ __forceinline__ void load8f(const void* x, int64_t i, float (&f)[8]) {
  if constexpr (DT == kBF16) {
    const uint4 w = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(u[j] << 16);
      f[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(x)[2 * i + 1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ float load1f(const void* x, int64_t i) {
  if constexpr (DT == kBF16)
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
  else
    return reinterpret_cast<const float*>(x)[i];
}

__global__ void amax_clear_kernel(float* acc) { *reinterpret_cast<uint32_t*>(acc) = 0u; }

template <int DT>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ x, int64_t n,
                                                   float* __restrict__ acc) {
  __shared__ float wmax[4];
  const int64_t n8 = n / 8;
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float f[8];
    load8f<DT>(x, i, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(f[j]));
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) m = fmaxf(m, fabsf(load1f<DT>(x, 8 * n8 + threadIdx.x)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(reinterpret_cast<unsigned int*>(acc), __float_as_uint(bm));
  }
}

__global__ void scale_kernel(float* acc) {
  const float amax = __uint_as_float(*reinterpret_cast<uint32_t*>(acc));
  *acc = amax > 0.f ? amax / kE4M3Max : 1.f;
}

// two floats -> two e4m3 codes in the low half of a word (RNE; the inputs are
// already within +-448)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

__device__ __forceinline__ float to_code_range(float x, float scale) {
  return fminf(fmaxf(x / scale, -kE4M3Max), kE4M3Max);
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ x, int64_t n,
                                                       const float* __restrict__ scale_p,
                                                       uint8_t* __restrict__ codes) {
  const float scale = *scale_p;
  const int64_t n8 = n / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float f[8];
    load8f<DT>(x, i, f);
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[j] = cvt2(to_code_range(f[4 * j], scale), to_code_range(f[4 * j + 1], scale)) |
             (cvt2(to_code_range(f[4 * j + 2], scale), to_code_range(f[4 * j + 3], scale)) << 16);
    reinterpret_cast<uint2*>(codes)[i] = make_uint2(w[0], w[1]);
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 8 * n8) {
    const int64_t j = 8 * n8 + threadIdx.x;
    codes[j] = (uint8_t)cvt2(to_code_range(load1f<DT>(x, j), scale), 0.f);
  }
}

template <int DT>
hipError_t launch_quantize_t(const void* x, int64_t n, uint8_t* codes, float* scale,
                             hipStream_t st) {
  const int64_t n8 = n / 8;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n8 + 255) / 256, 2048));
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(1), 0, st, scale);
  hipLaunchKernelGGL((amax_kernel<DT>), dim3(grid), dim3(256), 0, st, x, n, scale);
  hipLaunchKernelGGL(scale_kernel, dim3(1), dim3(1), 0, st, scale);
  hipLaunchKernelGGL((quantize_kernel<DT>), dim3(grid), dim3(256), 0, st, x, n,
                     (const float*)scale, codes);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_e4m3(int src_dtype, const void* x, int64_t n, uint8_t* codes,
                                float* scale, hipStream_t st) {
  return src_dtype == kBF16 ? launch_quantize_t<kBF16>(x, n, codes, scale, st)
                            : launch_quantize_t<kF32>(x, n, codes, scale, st);
}

}  // namespace bslp
