// Causal sliding-window softmax attention on the vector ALUs in fp32
// (the fp32 path of based_swa_fwd).
//
// Definition (HazyResearch/based README, introduction: exact softmax attention
// over a short window): row i attends to the `window` positions
// max(0, i - window + 1) .. i with weights exp(s_j - max s) / sum, where
// s_j = scale * q_i.k_j.
//
// One workgroup of 256 threads per (batch*head, block of 32 queries).  The
// block's keys/values (positions i0-63 .. i0+31) are staged in LDS once.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int QB = 32;               // queries per workgroup
constexpr int NT = 256;              // threads: 32 queries x 8 lanes
constexpr int G = NT / QB;           // lanes per query
constexpr int WMAX = 64;             // window capacity
constexpr int KR = QB + WMAX - 1;    // staged key rows
constexpr int DMAX = 128;

template <typename T>
__global__ __launch_bounds__(NT) void swa_valu_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, float* __restrict__ y, int L,
                                                       int dqk, int dv, int window, float scale) {
  __shared__ float Qs[QB][DMAX];
  __shared__ float Ks[KR][DMAX + 1];
  __shared__ float Vs[KR][DMAX];
  __shared__ float P[QB][WMAX + 1];

  const int nblk = (L + QB - 1) / QB;
  const size_t bh = blockIdx.x / nblk;
  const int i0 = (blockIdx.x % nblk) * QB;
  const int key0 = i0 - (WMAX - 1);  // position of staged row 0
  const int tid = threadIdx.x;
  const T* qb = q + bh * L * dqk;
  const T* kb = k + bh * L * dqk;
  const T* vb = v + bh * L * dv;

  for (int e = tid; e < QB * dqk; e += NT) {
    const int r = e / dqk, d = e % dqk;
    Qs[r][d] = (i0 + r < L) ? to_f32(qb[(size_t)(i0 + r) * dqk + d]) : 0.f;
  }
  for (int e = tid; e < KR * dqk; e += NT) {
    const int r = e / dqk, d = e % dqk, p = key0 + r;
    Ks[r][d] = (p >= 0 && p < L) ? to_f32(kb[(size_t)p * dqk + d]) : 0.f;
  }
  for (int e = tid; e < KR * dv; e += NT) {
    const int r = e / dv, d = e % dv, p = key0 + r;
    Vs[r][d] = (p >= 0 && p < L) ? to_f32(vb[(size_t)p * dv + d]) : 0.f;
  }
  __syncthreads();

  const int i = tid / G, g = tid % G;
  const int qi = i0 + i;
  // window slot w holds key position qi - 63 + w, staged row i + w
  for (int w = g; w < WMAX; w += G) {
    const int p = qi - (WMAX - 1) + w;
    float s = -INFINITY;
    if (p >= 0 && w >= WMAX - window) {
      float acc = 0.f;
      for (int d = 0; d < dqk; ++d) acc += Qs[i][d] * Ks[i + w][d];
      s = scale * acc;
    }
    P[i][w] = s;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int w = 0; w < WMAX; ++w) m = fmaxf(m, P[i][w]);
  __syncthreads();
  for (int w = g; w < WMAX; w += G) P[i][w] = __expf(P[i][w] - m);  // exp(-inf) = 0
  __syncthreads();
  if (qi >= L) return;
  float sum = 0.f;
  for (int w = 0; w < WMAX; ++w) sum += P[i][w];
  const float r = 1.f / sum;
  float* yr = y + (bh * L + qi) * dv;
  for (int c = g; c < dv; c += G) {
    float acc = 0.f;
    for (int w = 0; w < WMAX; ++w) acc += P[i][w] * Vs[i + w][c];
    yr[c] = acc * r;
  }
}

}  // namespace

hipError_t launch_swa_valu(const SwaArgs& a, bool bf16, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  dim3 grid((unsigned)((a.L + QB - 1) / QB) * (unsigned)(a.B * a.H));
  if (bf16)
    hipLaunchKernelGGL(swa_valu_kernel<bf16_t>, grid, dim3(NT), 0, s, (const bf16_t*)a.q, (const bf16_t*)a.k,
                       (const bf16_t*)a.v, a.y, a.L, a.dqk, a.dv, a.window, a.scale);
  else
    hipLaunchKernelGGL(swa_valu_kernel<float>, grid, dim3(NT), 0, s, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, a.y, a.L, a.dqk, a.dv, a.window, a.scale);
  return hipGetLastError();
}

}  // namespace based
