// BaseConv gate: y = u * conv(h, x) (blog post "Базированная модель, часть 1":
// the BaseConv block y = linear(x) * conv(h, x), an elementwise product of a
// linear map of the input with a learned filter convolved over the sequence;
// HazyResearch/based README acknowledgements: a short causal conv1d).  u =
// linear(x) is the caller's projection (a plain matrix product).
//
//   y[b, t, c] = u[b, t, c] * (bias[c] + sum_{s<K} h[c, s] x[b, t - s, c]),
//   x[b, t < 0, c] = 0.
//
// HBM-bound (a few flops per byte): each thread owns 4 consecutive channels
// of TP consecutive positions and slides a register window of K - 1 + TP rows
// of x over them, so a wavefront reads whole rows (4 channels x 64 lanes per
// instruction) and x is read 1 + (K - 1) / TP times.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int TP = 16;  // positions per thread

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
                     __uint_as_float(t.y & 0xffff0000u));
}

template <typename T, int K>
__global__ __launch_bounds__(256) void baseconv_kernel(const T* __restrict__ x, const T* __restrict__ u,
                                                      const float* __restrict__ h, const float* __restrict__ bias,
                                                      float* __restrict__ y, int L, int D, int ntile) {
  const int cg = blockIdx.y * blockDim.x + threadIdx.x;  // channel group of 4
  if (4 * cg >= D) return;
  const int c = 4 * cg;
  const size_t b = blockIdx.x / ntile;
  const int t0 = (blockIdx.x % ntile) * TP;
  float hk[K][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < K; ++s) hk[s][i] = h[(size_t)(c + i) * K + s];
  const float4 bz = bias ? *reinterpret_cast<const float4*>(bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  const T* xb = x + b * L * (size_t)D + c;
  const T* ub = u + b * L * (size_t)D + c;
  float* yb = y + b * L * (size_t)D + c;
  // window: rows t0 - (K - 1) .. t0 + TP - 1 of x
  float4 xw[K - 1 + TP];
#pragma unroll
  for (int r = 0; r < K - 1 + TP; ++r) {
    const int t = t0 - (K - 1) + r;
    xw[r] = t >= 0 && t < L ? ld4(xb + (size_t)t * D) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int p = 0; p < TP; ++p) {
    const int t = t0 + p;
    if (t < L) {
      float4 a = bz;
#pragma unroll
      for (int s = 0; s < K; ++s) {
        const float4 xv = xw[K - 1 + p - s];
        a.x = __builtin_fmaf(hk[s][0], xv.x, a.x);
        a.y = __builtin_fmaf(hk[s][1], xv.y, a.y);
        a.z = __builtin_fmaf(hk[s][2], xv.z, a.z);
        a.w = __builtin_fmaf(hk[s][3], xv.w, a.w);
      }
      const float4 g = ld4(ub + (size_t)t * D);
      *reinterpret_cast<float4*>(yb + (size_t)t * D) = make_float4(g.x * a.x, g.y * a.y, g.z * a.z, g.w * a.w);
    }
  }
}

template <typename T, int K>
hipError_t launch_k(const BaseConvArgs& a, hipStream_t s) {
  const int ntile = (a.L + TP - 1) / TP;
  const int groups = a.D / 4;
  const dim3 grid((unsigned)((size_t)a.B * ntile), (unsigned)((groups + 255) / 256));
  hipLaunchKernelGGL((baseconv_kernel<T, K>), grid, dim3(256), 0, s, (const T*)a.x, (const T*)a.u, a.h, a.bias, a.y,
                     a.L, a.D, ntile);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BaseConvArgs& a, hipStream_t s) {
  switch (a.K) {
    case 1: return launch_k<T, 1>(a, s);
    case 2: return launch_k<T, 2>(a, s);
    case 3: return launch_k<T, 3>(a, s);
    case 4: return launch_k<T, 4>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_baseconv(const BaseConvArgs& a, bool bf16, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  return bf16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace based
