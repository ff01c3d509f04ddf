// Causal Taylor linear attention, backward: the direct form (fp32 vector
// arithmetic, any input dtype and d_v).
//
// Gradients of y_i = sum_{j<=i} K_ij v_j / den_i, K_ij = 1 + x + x^2/2 with
// x = q_i.k_j and den_i = sum_{j<=i} K_ij (blog post "Базированная модель,
// часть 2": the Taylor kernel and its feature map; the based/train README's
// training views differentiate this forward).  With g_i = dy_i / den_i and
// h_i = -(dy_i . y_i) / den_i:
//   dK_ij = g_i . v_j + h_i,  c_ij = dK_ij (1 + x_ij)          (j <= i)
//   dq_i = sum_{j<=i} c_ij k_j,  dk_j = sum_{i>=j} c_ij q_i,  dv_j = sum_{i>=j} K_ij g_i.
//
// Two kernels, each sweeping 64-row tiles of the other side through LDS:
// per query (den, then g, h and dq; den and h go to the workspace), then per
// key (dk, dv).  Work is quadratic in L: this form serves fp32 inputs and
// widths the matrix-core passes do not take.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int TB = 64;  // rows per tile and threads per workgroup

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
                     __uint_as_float(t.y & 0xffff0000u));
}

// rows [r0, r0 + TB) of a [L, D] tensor into an fp32 LDS tile (zeros past L)
template <int D, int STRIDE, typename T>
__device__ __forceinline__ void stage(float (*dst)[STRIDE], const T* src, int r0, int L) {
  constexpr int G = D / 4;
  for (int e = threadIdx.x; e < TB * G; e += blockDim.x) {
    const int r = e / G, c = 4 * (e % G);
    const float4 x = r0 + r < L ? ld4(src + (size_t)(r0 + r) * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[r][c] = x.x; dst[r][c + 1] = x.y; dst[r][c + 2] = x.z; dst[r][c + 3] = x.w;
  }
}

// Per query i (one thread): den_i, then g_i (kept in LDS), h_i and dq_i.
template <typename T, int DV, int DEC>
__global__ __launch_bounds__(TB) void bwd_query_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const float* __restrict__ y,
                                                       const float* __restrict__ dy, float* __restrict__ gq,
                                                       float* __restrict__ den_out, float* __restrict__ h_out, int L,
                                                       int nblk, const float* __restrict__ gamma, int H) {
  __shared__ float ks[TB][DK + 1];
  __shared__ float vs[TB][DV + 1];
  __shared__ float gs[TB][DV + 1];
  const int t = threadIdx.x;
  const size_t bh = blockIdx.x / nblk;
  const int i0 = (blockIdx.x % nblk) * TB, i = i0 + t;
  const float lg = DEC ? decay_lg2_clamped(log2f(gamma[bh % H])) : 0.f;  // decay weight of (i, j): 2^(lg (i - j))
  const T* kh = k + bh * L * DK;
  const T* vh = v + bh * (size_t)L * DV;
  float qi[DK];
  if (i < L) {
    load_row<DK>(q + (bh * L + i) * DK, qi);
  } else {
#pragma unroll
    for (int e = 0; e < DK; ++e) qi[e] = 0.f;
  }
  const int jend = min(L, i0 + TB);  // keys this block's queries see

  // den_i = sum_{j<=i} K_ij
  float den = 0.f;
  for (int j0 = 0; j0 < jend; j0 += TB) {
    __syncthreads();
    stage<DK, DK + 1>(ks, kh, j0, L);
    __syncthreads();
    const int n = min(TB, i + 1 - j0);
    for (int jj = 0; jj < n; ++jj) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < DK; ++e) x = __builtin_fmaf(qi[e], ks[jj][e], x);
      const float K = 1.f + x + 0.5f * x * x;
      den += DEC ? K * exp2f(lg * (float)(i - j0 - jj)) : K;
    }
  }
  // g_i, h_i
  float h = 0.f;
  if (i < L) {
    const float rden = 1.f / den;
    float dot = 0.f;
    for (int c = 0; c < DV; c += 4) {
      const float4 a = ld4(dy + (bh * L + i) * DV + c), b = ld4(y + (bh * L + i) * DV + c);
      dot += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
      gs[t][c] = a.x * rden; gs[t][c + 1] = a.y * rden; gs[t][c + 2] = a.z * rden; gs[t][c + 3] = a.w * rden;
    }
    h = -dot * rden;
    den_out[bh * L + i] = den;
    h_out[bh * L + i] = h;
  }
  // dq_i = sum_{j<=i} (g_i . v_j + h_i)(1 + x_ij) k_j
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < jend; j0 += TB) {
    __syncthreads();
    stage<DK, DK + 1>(ks, kh, j0, L);
    stage<DV, DV + 1>(vs, vh, j0, L);
    __syncthreads();
    const int n = min(TB, i + 1 - j0);
    for (int jj = 0; jj < n; ++jj) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < DK; ++e) x = __builtin_fmaf(qi[e], ks[jj][e], x);
      float gv = h;
      for (int c = 0; c < DV; ++c) gv = __builtin_fmaf(gs[t][c], vs[jj][c], gv);
      float cij = gv * (1.f + x);
      if (DEC) cij *= exp2f(lg * (float)(i - j0 - jj));
#pragma unroll
      for (int e = 0; e < DK; ++e) acc[e] = __builtin_fmaf(cij, ks[jj][e], acc[e]);
    }
  }
  if (i < L)
#pragma unroll
    for (int e = 0; e < DK; e += 4)
      *reinterpret_cast<float4*>(gq + (bh * L + i) * DK + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

// Per key j (one thread): dk_j and dv_j over the queries i >= j.
template <typename T, int DV, int DEC>
__global__ __launch_bounds__(TB) void bwd_key_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const float* __restrict__ dy,
                                                     const float* __restrict__ den_in, const float* __restrict__ h_in,
                                                     float* __restrict__ gk, float* __restrict__ gv, int L, int nblk,
                                                     const float* __restrict__ gamma, int H) {
  __shared__ float qs[TB][DK + 1];
  __shared__ float gs[TB][DV + 1];
  __shared__ float hs[TB];
  __shared__ float vj[TB][DV + 1];
  __shared__ float dvj[TB][DV + 1];
  const int t = threadIdx.x;
  const size_t bh = blockIdx.x / nblk;
  const int j0 = (blockIdx.x % nblk) * TB, j = j0 + t;
  const float lg = DEC ? decay_lg2_clamped(log2f(gamma[bh % H])) : 0.f;
  const T* qh = q + bh * L * DK;
  float kj[DK];
  if (j < L) {
    load_row<DK>(k + (bh * L + j) * DK, kj);
  } else {
#pragma unroll
    for (int e = 0; e < DK; ++e) kj[e] = 0.f;
  }
  stage<DV, DV + 1>(vj, v + bh * (size_t)L * DV, j0, L);
  for (int c = 0; c < DV; ++c) dvj[t][c] = 0.f;
  float acc[DK];
#pragma unroll
  for (int e = 0; e < DK; ++e) acc[e] = 0.f;
  for (int i0 = j0; i0 < L; i0 += TB) {
    __syncthreads();
    stage<DK, DK + 1>(qs, qh, i0, L);
    for (int e = t; e < TB * DV; e += TB) {
      const int r = e / DV, c = e % DV, i = i0 + r;
      gs[r][c] = i < L ? dy[(bh * L + i) * DV + c] / den_in[bh * L + i] : 0.f;
    }
    hs[t] = i0 + t < L ? h_in[bh * L + i0 + t] : 0.f;
    __syncthreads();
    const int n = min(TB, L - i0);
    for (int ii = max(0, j - i0); ii < n; ++ii) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < DK; ++e) x = __builtin_fmaf(qs[ii][e], kj[e], x);
      const float wd = DEC ? exp2f(lg * (float)(i0 + ii - j)) : 1.f;
      const float K = (1.f + x + 0.5f * x * x) * wd;
      float gvv = hs[ii];
      for (int c = 0; c < DV; ++c) {
        gvv = __builtin_fmaf(gs[ii][c], vj[t][c], gvv);
        dvj[t][c] = __builtin_fmaf(K, gs[ii][c], dvj[t][c]);
      }
      const float cij = gvv * (1.f + x) * wd;
#pragma unroll
      for (int e = 0; e < DK; ++e) acc[e] = __builtin_fmaf(cij, qs[ii][e], acc[e]);
    }
  }
  if (j < L) {
#pragma unroll
    for (int e = 0; e < DK; e += 4)
      *reinterpret_cast<float4*>(gk + (bh * L + j) * DK + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    for (int c = 0; c < DV; ++c) gv[(bh * L + j) * DV + c] = dvj[t][c];
  }
}

template <typename T, int DV, int DEC>
hipError_t launch_direct_dec(const LinattnBwdArgs& a, hipStream_t s) {
  const int nblk = (a.L + TB - 1) / TB;
  const size_t BH = (size_t)a.B * a.H;
  float* den = (float*)a.workspace;
  float* h = den + BH * a.L;
  hipLaunchKernelGGL((bwd_query_kernel<T, DV, DEC>), dim3((unsigned)(BH * nblk)), dim3(TB), 0, s, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, a.y, a.dy, a.gq, den, h, a.L, nblk, a.gamma, a.H);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_key_kernel<T, DV, DEC>), dim3((unsigned)(BH * nblk)), dim3(TB), 0, s, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, a.dy, den, h, a.gk, a.gv, a.L, nblk, a.gamma, a.H);
  return hipGetLastError();
}

template <typename T, int DV>
hipError_t launch_direct(const LinattnBwdArgs& a, hipStream_t s) {
  return a.gamma ? launch_direct_dec<T, DV, 1>(a, s) : launch_direct_dec<T, DV, 0>(a, s);
}

template <typename T>
hipError_t launch_direct_dv(const LinattnBwdArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_direct<T, 16>(a, s);
    case 32: return launch_direct<T, 32>(a, s);
    case 48: return launch_direct<T, 48>(a, s);
    case 64: return launch_direct<T, 64>(a, s);
    case 80: return launch_direct<T, 80>(a, s);
    case 96: return launch_direct<T, 96>(a, s);
    case 112: return launch_direct<T, 112>(a, s);
    case 128: return launch_direct<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_linattn_bwd(const LinattnBwdArgs& a, bool bf16, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  // the decayed variant takes the matrix-core passes when the caller's
  // workspace holds theirs (it may be as small as the direct form's)
  if (bf16 && linattn_bwd_mfma_supported(a.dv) &&
      (!a.gamma || a.workspace_bytes >= linattn_bwd_mfma_workspace(a.B, a.H, a.L, a.dv)))
    return launch_linattn_bwd_mfma(a, s);
  return bf16 ? launch_direct_dv<bf16_t>(a, s) : launch_direct_dv<float>(a, s);
}

}  // namespace based
