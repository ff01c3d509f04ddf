// Device-side helpers shared by the Based layer kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace based {

// Raw bf16 storage: the upper 16 bits of an fp32.
typedef uint16_t bf16_t;

struct f32x4_t { float x, y, z, w; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 r = (__bf16)x;
  return __builtin_bit_cast(uint16_t, r);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Load n consecutive elements (n a multiple of 4 for fp32, 8 for bf16, 16-byte
// aligned) as fp32.
template <int N>
__device__ __forceinline__ void load_row(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    float4 t = *reinterpret_cast<const float4*>(p + i);
    out[i] = t.x; out[i + 1] = t.y; out[i + 2] = t.z; out[i + 3] = t.w;
  }
}
template <int N>
__device__ __forceinline__ void load_row(const bf16_t* p, float* out) {
#pragma unroll
  for (int i = 0; i < N; i += 8) {
    uint4 t = *reinterpret_cast<const uint4*>(p + i);
    uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[i + 2 * j] = __uint_as_float(w[j] << 16);
      out[i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

// Feature bookkeeping.  The state crosses the ABI in the 273-row layout of
// phi = [1, x_a, x_a x_b / sqrt2 (a-major)].  Inside the kernels the
// quadratic block is kept once per unordered pair a <= b ("compact" form,
// 1 + 16 + 136 = 153 rows):
//   key side   psi'(k) = [1, k_a, k_a^2, k_a k_b (a < b)]
//   query side psi(q)  = [1, q_a, q_a^2 / 2, q_a q_b (a < b)]
// so that psi(q).psi'(k) = 1 + q.k + (q.k)^2 / 2 = phi(q).phi(k).  Conversion:
//   T[aa] = sqrt2 * S[aa],  T[ab] = (S[ab] + S[ba]) / sqrt2,  S[ab] = T[ab] / sqrt2.
constexpr int DK = 16;
constexpr int DPHI = 273;
constexpr int NQUAD = DK * (DK + 1) / 2;  // 136
constexpr int NCOMPACT = 1 + DK + NQUAD;  // 153

// State decay factors.  A head's gamma is taken clamped to [0, 1] (NaN as
// 0).  decay_lg2_clamped(log2 gamma) keeps the logarithm in [-126, 0], so
// that gamma^d = exp2(d lg) is exactly 1 at d = 0 for every gamma (0^0 = 1),
// at most 2^-126 for gamma = 0 and d >= 1, and never above 1.
__device__ __forceinline__ float decay_lg2_clamped(float lg) { return fminf(fmaxf(lg, -126.f), 0.f); }
__device__ __forceinline__ float decay_clamped(float gamma) { return fminf(fmaxf(gamma, 0.f), 1.f); }
// gamma^d from lg = log2 gamma (d >= 0)
__device__ __forceinline__ float gpow(float lg, float d) { return __builtin_amdgcn_exp2f(lg * d); }
// sum_{d < n} gamma^d, through expm1 so that gamma near 1 keeps its precision
__device__ __forceinline__ float gsum_pow(float lg, int n) {
  const float ln = lg * 0.69314718055994531f;
  return ln == 0.f ? (float)n : expm1f(ln * (float)n) / expm1f(ln);
}

// Index of the unordered pair (a <= b) in the row-major upper triangle.
__host__ __device__ constexpr int pair_index(int a, int b) { return a * DK - a * (a - 1) / 2 + (b - a); }

// Compact feature f (< padded row count) of a query or key, as
// c0 + x_a (c1 + c2 x_b): the constant feature 1, the linear ones x_a, the
// pairs x_a x_b (a <= b) -- weight 1/2 on the diagonal for a query (QUERY:
// phi'(q), so that phi'(q).psi'(k) = 1 + q.k + (q.k)^2 / 2), 1 for a key
// (psi'(k)) -- and zero past NCOMPACT.  The fp32 kernels fill the same
// features of every chunk from each thread, so they work out the
// coefficients once.
struct FeatureCoef {
  float c0, c1, c2;
  int a, b;
};
template <bool QUERY>
__device__ __forceinline__ FeatureCoef feature_coef(int f) {
  FeatureCoef r{0.f, 0.f, 0.f, 0, 0};
  if (f == 0) {
    r.c0 = 1.f;
  } else if (f < 1 + DK) {
    r.c1 = 1.f;
    r.a = f - 1;
  } else if (f < NCOMPACT) {
    int pi = f - 1 - DK, a = 0;
    while (pi >= DK - a) {  // row a of the upper triangle holds DK - a pairs
      pi -= DK - a;
      ++a;
    }
    r.a = a;
    r.b = a + pi;
    r.c2 = QUERY && r.a == r.b ? 0.5f : 1.f;
  }
  return r;
}
__device__ __forceinline__ float feature(const FeatureCoef& fc, const float* x) {
  return fc.c0 + x[fc.a] * __builtin_fmaf(fc.c2, x[fc.b], fc.c1);
}

constexpr float SQRT2 = 1.41421356237309505f;
constexpr float INV_SQRT2 = 0.70710678118654752f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Workgroups go to the chip's 8 XCDs round-robin by block index, and each XCD
// has its own L2.  Block b -> (unit u, part s) of a units x parts grid such
// that all parts of one unit run on one XCD (units 8i + x take the blocks
// whose index is x mod 8); units past the last multiple of 8 map in plain
// order.  A bijection for any units, parts.
constexpr int NXCD = 8;
__device__ __forceinline__ void xcd_unit_part(int b, int units, int parts, int& u, int& s) {
  const int units8 = units - units % NXCD;
  const int full = units8 * parts;
  if (b < full) {
    const int x = b % NXCD, local = b / NXCD;
    u = NXCD * (local / parts) + x;
    s = local % parts;
  } else {
    const int r = b - full;
    u = units8 + r / parts;
    s = r % parts;
  }
}

// Issue priority by progress.  Where two workgroups share a CU, the wavefront
// arbiter favours the older wavefronts: one workgroup of the pair runs ahead
// and ends several microseconds before the other, which then runs alone at a
// fraction of the CU's throughput.  A wavefront that lowers its priority as
// it passes each quarter of its work (done of total) lets the one behind
// catch up, so that the two end closer together.
__device__ __forceinline__ void progress_priority(long long done, long long total) {
  const int q4 = total > 0 ? (int)(4 * done / total) : 0;
  if (q4 <= 0) __builtin_amdgcn_s_setprio(3);
  else if (q4 == 1) __builtin_amdgcn_s_setprio(2);
  else if (q4 == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Segment records of the linear attention's state (workspace of the chunked
// forward, read by the backward too): the 160 x dv compact state is stored in
// the order of the matrix-core accumulator fragments, so that a lane moves its
// four values of a 16 x 16 tile with one 16-byte access.  Element (r, c):
// tile (r / 16, c / 16), lane 16 ((r % 16) / 4) + c % 16, element r % 4.  The
// constant row (index 160) follows as a plain row of dv values.
__host__ __device__ constexpr size_t record_offset(int r, int c, int dv) {
  return ((size_t)((r >> 4) * (dv >> 4) + (c >> 4)) * 64 + 16 * ((r & 15) >> 2) + (c & 15)) * 4 + (r & 3);
}

}  // namespace based
