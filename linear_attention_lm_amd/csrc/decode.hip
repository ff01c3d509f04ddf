// Recurrent decode of the Based layer: one token per sequence per call.
//
// Per (batch b, head h), with t = pos[b] (blog post "Базированная модель,
// часть 2", paragraph on the state: a KV-state for the numerator and a
// K-state for the denominator replace the KV cache; README intro: softmax
// attention over the last 64 tokens):
//   S += phi(k) v^T, z += phi(k), y_lin = phi(q)^T S / phi(q)^T z
//   ring slot t mod W <- (k, v); y_swa = softmax window attention over t-W+1..t.
//
// The step streams the 273 x d_v fp32 state through once (read, update,
// write back) and is bound by HBM bandwidth.  Layout of the work: one
// workgroup per sequence (so the position counter can be advanced race-free),
// one wavefront per head.  Inside a wavefront, lane (rg, cg) owns columns
// 4cg..4cg+3 of every state row with row-group rg: a wavefront instruction
// touches RG whole 16-byte-per-lane row segments, each row read and written
// exactly once with 16-byte accesses.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int MAXW = 16;  // wavefronts (heads in flight) per workgroup

template <typename T, int DV>
__global__ __launch_bounds__(64 * MAXW) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ S,
    float* __restrict__ z, T* __restrict__ ring_k, T* __restrict__ ring_v, int32_t* __restrict__ pos,
    float* __restrict__ y_lin, float* __restrict__ y_swa, int H, int window, float scale) {
  constexpr int CG = DV / 4;   // column groups of 4 floats
  constexpr int RG = 64 / CG;  // row groups per wavefront
  __shared__ float qk_s[MAXW][2][DK];
  __shared__ float4 red_s[MAXW][64];
  __shared__ float p_s[MAXW][64];
  __shared__ int t_s;

  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (threadIdx.x == 0) t_s = pos[b];
  __syncthreads();
  const int t = t_s;
  const int cg = lane % CG, rg = lane / CG;
  const bool active = rg < RG;

  for (int h = wave; h < H; h += nw) {
    const size_t bh = (size_t)b * H + h;
    float qr[DK], kr[DK];
    load_row<DK>(q + bh * DK, qr);
    load_row<DK>(k + bh * DK, kr);
    if (lane < DK) {
      qk_s[wave][0][lane] = to_f32(q[bh * DK + lane]);
      qk_s[wave][1][lane] = to_f32(k[bh * DK + lane]);
    }
    __builtin_amdgcn_wave_barrier();
    float vr[4];
    {
      const T* vp = v + bh * DV + 4 * cg;
#pragma unroll
      for (int j = 0; j < 4; ++j) vr[j] = to_f32(vp[j]);
    }

    // ---- linear attention: stream the state rows through once
    float* Sh = S + bh * DPHI * DV + 4 * cg;
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
    if (active) {
      auto row = [&](int f, float pk, float pq) {
        float4 s = *reinterpret_cast<const float4*>(Sh + (size_t)f * DV);
        s.x += pk * vr[0]; s.y += pk * vr[1]; s.z += pk * vr[2]; s.w += pk * vr[3];
        *reinterpret_cast<float4*>(Sh + (size_t)f * DV) = s;
        num.x += pq * s.x; num.y += pq * s.y; num.z += pq * s.z; num.w += pq * s.w;
      };
      for (int f = rg; f < 1 + DK; f += RG) {
        const float pk = f == 0 ? 1.f : qk_s[wave][1][f - 1];
        const float pq = f == 0 ? 1.f : qk_s[wave][0][f - 1];
        row(f, pk, pq);
      }
      for (int a = rg; a < DK; a += RG) {
        const float ka = qk_s[wave][1][a] * INV_SQRT2, qa = qk_s[wave][0][a] * INV_SQRT2;
#pragma unroll
        for (int bb = 0; bb < DK; ++bb) row(1 + DK + DK * a + bb, ka * kr[bb], qa * qr[bb]);
      }
    }
    // denominator: z rows spread over all 64 lanes
    float den = 0.f;
    {
      float* zh = z + bh * DPHI;
      for (int f = lane; f < DPHI; f += 64) {
        float pk, pq;
        if (f == 0) {
          pk = pq = 1.f;
        } else if (f < 1 + DK) {
          pk = qk_s[wave][1][f - 1];
          pq = qk_s[wave][0][f - 1];
        } else {
          const int a = (f - 1 - DK) / DK, bb = (f - 1 - DK) % DK;
          pk = qk_s[wave][1][a] * qk_s[wave][1][bb] * INV_SQRT2;
          pq = qk_s[wave][0][a] * qk_s[wave][0][bb] * INV_SQRT2;
        }
        const float zn = zh[f] + pk;
        zh[f] = zn;
        den += pq * zn;
      }
    }
    den = wave_sum(den);
    red_s[wave][lane] = make_float4(num.x, num.y, num.z, num.w);
    __builtin_amdgcn_wave_barrier();
    if (active && rg == 0) {
      float4 acc = red_s[wave][lane];
      for (int r = 1; r < RG; ++r) {
        const float4 o = red_s[wave][r * CG + cg];
        acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
      }
      const float inv = 1.f / den;
      acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
      *reinterpret_cast<float4*>(y_lin + bh * DV + 4 * cg) = acc;
    }

    // ---- window softmax attention over the ring (slot = position mod window)
    const int slot = t % window;
    T* rk = ring_k + bh * (size_t)window * DK;
    T* rv = ring_v + bh * (size_t)window * DV;
    float sc = -INFINITY;
    if (lane < window) {
      const int p = t - ((t - lane) % window + window) % window;  // position held by this slot
      if (p >= 0) {
        float kk[DK];
        if (lane == slot) {
#pragma unroll
          for (int d = 0; d < DK; ++d) kk[d] = kr[d];
        } else {
#pragma unroll
          for (int d = 0; d < DK; ++d) kk[d] = to_f32(rk[(size_t)lane * DK + d]);
        }
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < DK; ++d) acc += qr[d] * kk[d];
        sc = scale * acc;
      }
    }
    const float m = wave_max(sc);
    const float p = (sc == -INFINITY) ? 0.f : __expf(sc - m);
    const float psum = wave_sum(p);
    p_s[wave][lane] = p;
    __builtin_amdgcn_wave_barrier();
    const float inv = 1.f / psum;
    for (int c = lane; c < DV; c += 64) {
      const float vcur = to_f32(v[bh * DV + c]);
      float acc = 0.f;
      for (int j = 0; j < window; ++j) {
        const float vj = (j == slot) ? vcur : to_f32(rv[(size_t)j * DV + c]);
        acc += p_s[wave][j] * vj;
      }
      y_swa[bh * DV + c] = acc * inv;
    }
    // the new token enters the ring after every slot was read
    if (lane < DK) rk[(size_t)slot * DK + lane] = k[bh * DK + lane];
    for (int c = lane; c < DV; c += 64) rv[(size_t)slot * DV + c] = v[bh * DV + c];
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (threadIdx.x == 0) pos[b] = t + 1;
}

template <typename T>
__global__ void decode_prefill_kernel(const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ ring_k,
                                      T* __restrict__ ring_v, int32_t* __restrict__ pos, int H, int L, int dv,
                                      int window) {
  const size_t bh = blockIdx.x;
  const int p0 = L > window ? L - window : 0;
  for (int e = threadIdx.x; e < (L - p0) * DK; e += blockDim.x) {
    const int p = p0 + e / DK, d = e % DK;
    ring_k[(bh * window + p % window) * DK + d] = k[(bh * L + p) * DK + d];
  }
  for (int e = threadIdx.x; e < (L - p0) * dv; e += blockDim.x) {
    const int p = p0 + e / dv, d = e % dv;
    ring_v[(bh * window + p % window) * dv + d] = v[(bh * L + p) * dv + d];
  }
  if (bh % H == 0 && threadIdx.x == 0) pos[bh / H] = L;
}

template <typename T, int DV>
hipError_t launch_step(const DecodeArgs& a, hipStream_t s) {
  const int nw = a.H < MAXW ? a.H : MAXW;
  hipLaunchKernelGGL((decode_step_kernel<T, DV>), dim3(a.B), dim3(64 * nw), 0, s, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, a.S, a.z, (T*)a.ring_k, (T*)a.ring_v, a.pos, a.y_lin, a.y_swa, a.H, a.window,
                     a.scale);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_step_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_step<T, 16>(a, s);
    case 32: return launch_step<T, 32>(a, s);
    case 48: return launch_step<T, 48>(a, s);
    case 64: return launch_step<T, 64>(a, s);
    case 80: return launch_step<T, 80>(a, s);
    case 96: return launch_step<T, 96>(a, s);
    case 112: return launch_step<T, 112>(a, s);
    case 128: return launch_step<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_step_t<bf16_t>(a, s) : launch_step_t<float>(a, s);
}

hipError_t launch_decode_prefill(const void* k, const void* v, void* ring_k, void* ring_v, int32_t* pos, int B, int H,
                                 int L, int dv, int window, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(decode_prefill_kernel<bf16_t>, dim3(B * H), dim3(256), 0, s, (const bf16_t*)k,
                       (const bf16_t*)v, (bf16_t*)ring_k, (bf16_t*)ring_v, pos, H, L, dv, window);
  else
    hipLaunchKernelGGL(decode_prefill_kernel<float>, dim3(B * H), dim3(256), 0, s, (const float*)k, (const float*)v,
                       (float*)ring_k, (float*)ring_v, pos, H, L, dv, window);
  return hipGetLastError();
}

}  // namespace based
