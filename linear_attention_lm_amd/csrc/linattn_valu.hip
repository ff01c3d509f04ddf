// Causal Taylor linear attention, chunked, on the vector ALUs in fp32.
//
// This is the fp32 path of based_linattn_fwd: every product and sum in fp32.
// Definition followed (blog post "Базированная модель, часть 2", linear-
// attention paragraph and feature-map pseudocode; paragraph on the state):
//   y_i = (phi(q_i)^T S_i) / (phi(q_i)^T z_i),  S_i = S_0 + sum_{j<=i} phi(k_j) v_j^T.
// Chunked evaluation: for a chunk of C positions, the readout of the state
// accumulated before the chunk plus the masked in-chunk term
// sum_{j<=i in chunk} (1 + x + x^2/2) v_j with x = q_i.k_j, then the state
// update with the chunk.  The state lives in LDS in the compact form (one row
// per unordered feature pair, see based_device.h).
//
// One workgroup of 256 threads per (batch, head); chunks run in sequence.
// A per-head decay of the state (DEC) is the same pass with decay weights.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int C = 64;    // positions per chunk
constexpr int NT = 256;  // threads per workgroup

struct PairTables {
  uint8_t a[NQUAD], b[NQUAD];
};
constexpr PairTables make_pairs() {
  PairTables t{};
  int p = 0;
  for (int a = 0; a < DK; ++a)
    for (int b = a; b < DK; ++b) { t.a[p] = (uint8_t)a; t.b[p] = (uint8_t)b; ++p; }
  return t;
}
__constant__ PairTables c_pairs = make_pairs();

// Compact row f of a 273-row state (row stride ld, column c).
__device__ float compact_from_phi(const float* S, int f, int c, int ld) {
  if (f < 1 + DK) return S[(size_t)f * ld + c];
  const int p = f - 1 - DK;
  const int a = c_pairs.a[p], b = c_pairs.b[p];
  if (a == b) return SQRT2 * S[(size_t)(1 + DK + DK * a + a) * ld + c];
  return (S[(size_t)(1 + DK + DK * a + b) * ld + c] + S[(size_t)(1 + DK + DK * b + a) * ld + c]) * INV_SQRT2;
}

// 273-layout row f from the compact state row-major [NCOMPACT][ld].
__device__ float phi_from_compact(const float* T, int f, int c, int ld) {
  if (f < 1 + DK) return T[f * ld + c];
  const int a = (f - 1 - DK) / DK, b = (f - 1 - DK) % DK;
  const int lo = a < b ? a : b, hi = a < b ? b : a;
  return T[(1 + DK + pair_index(lo, hi)) * ld + c] * INV_SQRT2;
}

// DEC: the decayed variant (the based/train README's optional decay
// strategy, read as a per-head factor 0 < gamma <= 1 on the state:
// S_i = gamma S_{i-1} + phi(k_i) v_i^T, z likewise).  The state entering a
// chunk reaches its position i (0-based in the chunk) times gamma^(i+1), an
// in-chunk key j weighs gamma^(i-j), and the update is S <- gamma^n S +
// sum_j gamma^(n-1-j) phi(k_j) v_j^T over the chunk's n positions.
template <typename T, int DV, int DEC>
__global__ __launch_bounds__(NT) void linattn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ y,
    const float* S_in, const float* z_in, float* S_out, float* z_out, int L, const float* gamma, int H) {
  constexpr int CPT = DV / 4;  // readout columns per thread
  __shared__ float Ts[NCOMPACT][DV];
  __shared__ float zs[NCOMPACT];
  __shared__ float qs[C][DK];
  __shared__ float ks[C][DK];
  __shared__ float vs[C][DV];
  __shared__ float wk[C];  // decayed variant: weight gamma^(n-1-j) of the chunk's key j in the update

  const int bh = blockIdx.x;
  const float lg = DEC ? decay_lg2_clamped(log2f(gamma[bh % H])) : 0.f;
  const int tid = threadIdx.x;
  const T* qb = q + (size_t)bh * L * DK;
  const T* kb = k + (size_t)bh * L * DK;
  const T* vb = v + (size_t)bh * L * DV;
  float* yb = y + (size_t)bh * L * DV;

  for (int e = tid; e < NCOMPACT * DV; e += NT) {
    const int f = e / DV, c = e % DV;
    Ts[f][c] = S_in ? compact_from_phi(S_in + (size_t)bh * DPHI * DV, f, c, DV) : 0.f;
  }
  for (int f = tid; f < NCOMPACT; f += NT) zs[f] = z_in ? compact_from_phi(z_in + (size_t)bh * DPHI, f, 0, 1) : 0.f;

  for (int c0 = 0; c0 < L; c0 += C) {
    const int n = min(C, L - c0);
    __syncthreads();  // previous chunk's update done
    for (int e = tid; e < C * DK; e += NT) {
      const int j = e / DK, d = e % DK;
      const bool ok = j < n;
      qs[j][d] = ok ? to_f32(qb[(size_t)(c0 + j) * DK + d]) : 0.f;
      ks[j][d] = ok ? to_f32(kb[(size_t)(c0 + j) * DK + d]) : 0.f;
    }
    for (int e = tid; e < C * DV; e += NT) {
      const int j = e / DV, d = e % DV;
      vs[j][d] = j < n ? to_f32(vb[(size_t)(c0 + j) * DV + d]) : 0.f;
    }
    if (DEC && tid < C) wk[tid] = tid < n ? exp2f(lg * (float)(n - 1 - tid)) : 0.f;
    __syncthreads();

    // ---- readout of the state before the chunk + in-chunk masked term
    {
      const int i = tid % C, g = tid / C, col0 = g * CPT;
      if (i < n) {
        float qr[DK];
#pragma unroll
        for (int d = 0; d < DK; ++d) qr[d] = qs[i][d];
        float num[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) num[c] = Ts[0][col0 + c];
        float den = zs[0];
#pragma unroll
        for (int a = 0; a < DK; ++a) {
          den += qr[a] * zs[1 + a];
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[c] += qr[a] * Ts[1 + a][col0 + c];
        }
#pragma unroll
        for (int a = 0; a < DK; ++a) {
#pragma unroll
          for (int b = a; b < DK; ++b) {
            const int f = 1 + DK + pair_index(a, b);
            const float w = (a == b) ? 0.5f * qr[a] * qr[a] : qr[a] * qr[b];
            den += w * zs[f];
#pragma unroll
            for (int c = 0; c < CPT; ++c) num[c] += w * Ts[f][col0 + c];
          }
        }
        if (DEC) {  // the state before the chunk, decayed over positions c0 .. c0 + i
          const float cf = exp2f(lg * (float)(i + 1));
          den *= cf;
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[c] *= cf;
        }
        for (int j = 0; j <= i; ++j) {
          float x = 0.f;
#pragma unroll
          for (int d = 0; d < DK; ++d) x += qr[d] * ks[j][d];
          float w = 1.f + x + 0.5f * x * x;
          if (DEC) w *= exp2f(lg * (float)(i - j));
          den += w;
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[c] += w * vs[j][col0 + c];
        }
        const float r = 1.f / den;
        float* yr = yb + (size_t)(c0 + i) * DV + col0;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
          float4 o = {num[c] * r, num[c + 1] * r, num[c + 2] * r, num[c + 3] * r};
          *reinterpret_cast<float4*>(yr + c) = o;
        }
      }
    }
    __syncthreads();

    // ---- state update with the chunk: T += psi'(K)^T V, z += sum psi'(k)
    {
      constexpr int FS = NT / DV;  // features handled in parallel per column
      const int c = tid % DV;
      const float gn = DEC ? exp2f(lg * (float)n) : 1.f;  // decay of the carried state over the chunk
      auto kw = [&](int j) { return DEC ? wk[j] : 1.f; };
      for (int f = tid / DV; tid < FS * DV && f < NCOMPACT; f += FS) {
        float acc = 0.f;
        if (f == 0) {
          for (int j = 0; j < n; ++j) acc += kw(j) * vs[j][c];
        } else if (f < 1 + DK) {
          for (int j = 0; j < n; ++j) acc += kw(j) * ks[j][f - 1] * vs[j][c];
        } else {
          const int a = c_pairs.a[f - 1 - DK], b = c_pairs.b[f - 1 - DK];
          for (int j = 0; j < n; ++j) acc += kw(j) * ks[j][a] * ks[j][b] * vs[j][c];
        }
        Ts[f][c] = DEC ? gn * Ts[f][c] + acc : Ts[f][c] + acc;
      }
      for (int f = tid; f < NCOMPACT; f += NT) {
        float acc = 0.f;
        if (f == 0) {
          if (DEC)
            for (int j = 0; j < n; ++j) acc += wk[j];
          else
            acc = (float)n;
        } else if (f < 1 + DK) {
          for (int j = 0; j < n; ++j) acc += kw(j) * ks[j][f - 1];
        } else {
          const int a = c_pairs.a[f - 1 - DK], b = c_pairs.b[f - 1 - DK];
          for (int j = 0; j < n; ++j) acc += kw(j) * ks[j][a] * ks[j][b];
        }
        zs[f] = DEC ? gn * zs[f] + acc : zs[f] + acc;
      }
    }
  }
  __syncthreads();
  if (S_out) {
    float* So = S_out + (size_t)bh * DPHI * DV;
    for (int e = tid; e < DPHI * DV; e += NT) So[e] = phi_from_compact(&Ts[0][0], e / DV, e % DV, DV);
    float* zo = z_out + (size_t)bh * DPHI;
    for (int f = tid; f < DPHI; f += NT) zo[f] = phi_from_compact(zs, f, 0, 1);
  }
}

template <typename T, int DV>
hipError_t launch_dv(const LinattnArgs& a, hipStream_t s) {
  if (a.gamma)
    hipLaunchKernelGGL((linattn_valu_kernel<T, DV, 1>), dim3(a.B * a.H), dim3(NT), 0, s, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.y, a.S_in, a.z_in, a.S_out, a.z_out, a.L, a.gamma, a.H);
  else
    hipLaunchKernelGGL((linattn_valu_kernel<T, DV, 0>), dim3(a.B * a.H), dim3(NT), 0, s, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.y, a.S_in, a.z_in, a.S_out, a.z_out, a.L, a.gamma, a.H);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const LinattnArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_dv<T, 16>(a, s);
    case 32: return launch_dv<T, 32>(a, s);
    case 48: return launch_dv<T, 48>(a, s);
    case 64: return launch_dv<T, 64>(a, s);
    case 80: return launch_dv<T, 80>(a, s);
    case 96: return launch_dv<T, 96>(a, s);
    case 112: return launch_dv<T, 112>(a, s);
    case 128: return launch_dv<T, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_linattn_valu(const LinattnArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace based
