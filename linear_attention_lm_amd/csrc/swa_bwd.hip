// Sliding-window softmax attention, backward (fp32 vector arithmetic, any
// input dtype; d_qk = 16): the form for fp32 inputs and for widths the
// matrix-core kernel does not take.
//
// Gradients of y_i = sum_j p_ij v_j, p_ij = softmax_j(scale q_i.k_j) over the
// causal band max(0, i - W + 1) <= j <= i (HazyResearch/based README intro:
// exact softmax attention over a short window; the training views of the
// based/train README differentiate this forward):
//   dP_ij = dy_i . v_j,  D_i = dy_i . y_i,  dS_ij = p_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i p_ij dy_i.
//
// One workgroup per (head, chunk c of 64 keys).  The keys of chunk c are seen
// by the queries of chunks c and c + 1 (W <= 64), so the workgroup first forms
// the log-sum-exp and D of those 128 queries (two threads per query, each over
// half of the query's window), then takes the two query chunks in turn: the
// 64 x 64 tiles P and dS in LDS (4 x 4 register tiles per thread), then
// dv_c += P^T dY, dk_c += dS^T Q and the chunk's share of dq.  dk and dv of
// chunk c are written once; dq of a query gets exactly two shares (its own
// chunk's keys and the previous chunk's), added atomically onto a zeroed dq:
// 0 + a + b and 0 + b + a round to the same value (two addends onto an exact
// zero), so the result has the same bits whichever share lands first.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int CB = 64;       // positions per chunk
constexpr int QS = DK + 1;   // fp32 row stride of q / k tiles
constexpr int PS = CB + 4;   // row stride of the P tile (16-byte rows)
constexpr int DSS = CB + 1;  // row stride of the dS tile (odd: its columns are read too)

template <int DV>
struct SwaBwdSmem {
  static constexpr int VS = DV + 4;
  alignas(16) float k[CB][QS];    // keys of chunk c
  alignas(16) float v[CB][VS];    // values of chunk c
  alignas(16) float q[CB][QS];    // queries of the current query chunk
  alignas(16) float dy[CB][VS];   // upstream gradient of the current query chunk
  alignas(16) float p[CB][PS];    // softmax weights, query x key
  float ds[CB][DSS];              // p (dP - D)
  float lse[2 * CB];              // log-sum-exp of the scaled scores, queries of chunks c, c+1
  float dd[2 * CB];               // D_i = dy_i . y_i
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
                     __uint_as_float(t.y & 0xffff0000u));
}

// rows [r0, r0 + CB) of a [L, D] tensor into an fp32 LDS tile (zeros past L)
template <int D, int STRIDE, typename T>
__device__ __forceinline__ void stage_rows(float (*dst)[STRIDE], const T* src, int r0, int L) {
  constexpr int G = D / 4;
  for (int e = threadIdx.x; e < CB * G; e += blockDim.x) {
    const int r = e / G, c = 4 * (e % G);
    const float4 x = r0 + r < L ? ld4(src + (size_t)(r0 + r) * D + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dst[r][c] = x.x; dst[r][c + 1] = x.y; dst[r][c + 2] = x.z; dst[r][c + 3] = x.w;
  }
}

template <typename T, int DV>
__global__ __launch_bounds__(256) void swa_bwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, const float* __restrict__ y,
                                                      const float* __restrict__ dy, float* __restrict__ dq,
                                                      float* __restrict__ dk, float* __restrict__ dv, int L, int nch,
                                                      int window, float scale) {
  constexpr int CW = DV / 16;  // dv columns per thread
  __shared__ SwaBwdSmem<DV> S;
  const int tid = threadIdx.x;
  const size_t bh = blockIdx.x / nch;
  const int c = blockIdx.x % nch;
  const int j0 = c * CB;
  const T* qh = q + bh * L * DK;
  const T* kh = k + bh * L * DK;
  const T* vh = v + bh * (size_t)L * DV;
  const float* yh = y + bh * (size_t)L * DV;
  const float* dyh = dy + bh * (size_t)L * DV;

  // ---- log-sum-exp and D of the queries of chunks c and c + 1
  {
    const int ql = tid >> 1, half = tid & 1;
    const int i = j0 + ql;
    float m = -INFINITY, l = 0.f, d = 0.f;
    if (i < L) {
      float qi[DK];
      load_row<DK>(qh + (size_t)i * DK, qi);
      for (int j = max(0, i - window + 1) + half; j <= i; j += 2) {
        float kj[DK];
        load_row<DK>(kh + (size_t)j * DK, kj);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DK; ++e) s = __builtin_fmaf(qi[e], kj[e], s);
        s *= scale;
        if (s > m) {
          l = l * expf(m - s) + 1.f;
          m = s;
        } else {
          l += expf(s - m);
        }
      }
      for (int cc = half * (DV / 2); cc < (half + 1) * (DV / 2); cc += 4) {
        const float4 a = ld4(dyh + (size_t)i * DV + cc), b = ld4(yh + (size_t)i * DV + cc);
        d += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
      }
    }
    const float mo = __shfl_xor(m, 1, 64), lo = __shfl_xor(l, 1, 64), dother = __shfl_xor(d, 1, 64);
    const float mm = fmaxf(m, mo);
    const float ll = (l > 0.f ? l * expf(m - mm) : 0.f) + (lo > 0.f ? lo * expf(mo - mm) : 0.f);
    if (half == 0) {
      S.lse[ql] = i < L ? mm + logf(ll) : 0.f;
      S.dd[ql] = d + dother;
    }
  }
  stage_rows<DK, QS>(S.k, kh, j0, L);
  stage_rows<DV, SwaBwdSmem<DV>::VS>(S.v, vh, j0, L);

  const int ti = tid >> 4, tj = tid & 15;  // 4 x 4 tile of (query, key) pairs
  const int kg = tid & 15, cg = tid >> 4;  // dv: keys 4kg.., columns cg * CW..
  const int jr = tid & 63, dg = tid >> 6;  // dk / dq: row jr, coordinates 4dg..
  float dva[4][CW] = {};
  float dka[4] = {0.f, 0.f, 0.f, 0.f};

  for (int sb = 0; sb < 2; ++sb) {
    const int i0 = j0 + sb * CB;
    if (i0 >= L) break;
    __syncthreads();  // previous tiles consumed; lse / dd and the key chunk staged
    stage_rows<DK, QS>(S.q, qh, i0, L);
    stage_rows<DV, SwaBwdSmem<DV>::VS>(S.dy, dyh, i0, L);
    __syncthreads();

    // ---- P and dS for queries i0 + 4ti + a, keys j0 + 4tj + b
    {
      float s[4][4] = {}, dp[4][4] = {};
#pragma unroll
      for (int e = 0; e < DK; ++e) {
        float qa[4], kb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) qa[a] = S.q[4 * ti + a][e];
#pragma unroll
        for (int b = 0; b < 4; ++b) kb[b] = S.k[4 * tj + b][e];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) s[a][b] = __builtin_fmaf(qa[a], kb[b], s[a][b]);
      }
      for (int cc = 0; cc < DV; cc += 4) {
        float4 ya[4], vb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) ya[a] = *reinterpret_cast<const float4*>(&S.dy[4 * ti + a][cc]);
#pragma unroll
        for (int b = 0; b < 4; ++b) vb[b] = *reinterpret_cast<const float4*>(&S.v[4 * tj + b][cc]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            dp[a][b] += ya[a].x * vb[b].x + ya[a].y * vb[b].y + ya[a].z * vb[b].z + ya[a].w * vb[b].w;
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int il = 4 * ti + a, i = i0 + il;
        const float lse = S.lse[sb * CB + il], dd = S.dd[sb * CB + il];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int j = j0 + 4 * tj + b;
          const bool in_band = i < L && j <= i && i - j < window;
          const float pw = in_band ? expf(scale * s[a][b] - lse) : 0.f;
          S.p[il][4 * tj + b] = pw;
          S.ds[il][4 * tj + b] = pw * (dp[a][b] - dd);
        }
      }
    }
    __syncthreads();

    // ---- dv_c += P^T dY, dk_c += dS^T Q, and this query chunk's dq share
    for (int il = 0; il < CB; ++il) {
      const float4 pw = *reinterpret_cast<const float4*>(&S.p[il][4 * kg]);
      const float pb[4] = {pw.x, pw.y, pw.z, pw.w};
      float yv[CW];
#pragma unroll
      for (int e = 0; e < CW; ++e) yv[e] = S.dy[il][cg * CW + e];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < CW; ++e) dva[b][e] = __builtin_fmaf(pb[b], yv[e], dva[b][e]);
      const float dsv = S.ds[il][jr];
#pragma unroll
      for (int e = 0; e < 4; ++e) dka[e] = __builtin_fmaf(dsv, S.q[il][4 * dg + e], dka[e]);
    }
    {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int jl = 0; jl < CB; ++jl) {
        const float dsv = S.ds[jr][jl];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(dsv, S.k[jl][4 * dg + e], acc[e]);
      }
      const int i = i0 + jr;
      if (i < L)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(dq + (bh * L + i) * DK + 4 * dg + e, scale * acc[e]);
    }
  }

  // ---- dk and dv of the chunk's keys
  {
    const int j = j0 + jr;
    if (j < L)
      *reinterpret_cast<float4*>(dk + (bh * L + j) * DK + 4 * dg) =
          make_float4(scale * dka[0], scale * dka[1], scale * dka[2], scale * dka[3]);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int j = j0 + 4 * kg + b;
    if (j < L)
#pragma unroll
      for (int e = 0; e < CW; ++e) dv[(bh * L + j) * DV + cg * CW + e] = dva[b][e];
  }
}

__global__ void zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

template <typename T, int DV>
hipError_t launch_t(const SwaBwdArgs& a, hipStream_t s) {
  const int nch = (a.L + CB - 1) / CB;
  const size_t BH = (size_t)a.B * a.H;
  const size_t n = BH * a.L * DK;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536)), dim3(256), 0,
                     s, a.gq, n);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((swa_bwd_kernel<T, DV>), dim3((unsigned)(BH * nch)), dim3(256), 0, s, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, a.y, a.dy, a.gq, a.gk, a.gv, a.L, nch, a.window, a.scale);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dv(const SwaBwdArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_t<T, 16>(a, s);
    case 32: return launch_t<T, 32>(a, s);
    case 48: return launch_t<T, 48>(a, s);
    case 64: return launch_t<T, 64>(a, s);
    case 80: return launch_t<T, 80>(a, s);
    case 96: return launch_t<T, 96>(a, s);
    case 112: return launch_t<T, 112>(a, s);
    case 128: return launch_t<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_swa_bwd(const SwaBwdArgs& a, bool bf16, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  if (bf16 && swa_bwd_mfma_supported(a.dv)) return launch_swa_bwd_mfma(a, s);
  return bf16 ? launch_dv<bf16_t>(a, s) : launch_dv<float>(a, s);
}

}  // namespace based
