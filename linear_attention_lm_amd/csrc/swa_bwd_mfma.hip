// Sliding-window softmax attention, backward on the matrix cores (bf16
// inputs, d_qk = 16, d_v in {32, 64, 96, 128}).
//
// The same gradients as the fp32 form (HazyResearch/based README intro:
// exact softmax over a short window; the based/train README's training views
// differentiate it): with p_ij = softmax_j(scale q_i.k_j) over the causal band,
// dP = dY V^T, D_i = dy_i . y_i and dS = P (dP - D):
//   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dY.
//
// One workgroup per (head, chunk c of 64 keys).  Its keys are seen by the
// queries of chunks c and c + 1 (window <= 64), so it stages those 128
// queries with their upstream gradients (fp16 hi + lo), D, and the keys of
// chunks c - 1 .. c + 1, from which each wavefront forms the log-sum-exp of
// two query tiles (transposed score tiles, row reductions across the four
// 16-lane rows).  Then wavefront w owns key tile w: its band meets query
// tiles w .. w + 4, whose score, P, dP and dS tiles it forms in registers
// (lane: four queries of one key), giving dk (Q^T dS) and dv (P^T dY) of its
// keys directly.  dS goes through LDS for dq (K^T dS^T over the chunk's 64
// keys); a query's dq gets exactly two shares (key chunks c - 1 and c), added
// atomically onto a zeroed dq, so the result does not depend on their order.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace swab {

typedef _Float16 half_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int C = 64;          // positions per chunk
constexpr int NTHR = 256;      // 4 wavefronts
constexpr int QH = 24;         // fp16 stride of q / k rows
constexpr int KTS = C + 8;     // fp16 stride of k^T rows (64 keys)
constexpr int QTS = 2 * C + 8; // fp16 stride of q^T rows (128 queries)
constexpr int DSS = C + 4;     // fp32 stride of the dS rows (keys)
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ f16x8 ld8(const half_t* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x8 cat44(const half_t* a, const half_t* b) {
  const uint2 x = *reinterpret_cast<const uint2*>(a), y = *reinterpret_cast<const uint2*>(b);
  return __builtin_bit_cast(f16x8, make_uint4(x.x, x.y, y.x, y.y));
}
__device__ __forceinline__ uint32_t h2_from_bf2(uint32_t w) {
  const f32x2 f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return u32(__builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ uint4 h8_from_bf8(const uint4& x) {
  return make_uint4(h2_from_bf2(x.x), h2_from_bf2(x.y), h2_from_bf2(x.z), h2_from_bf2(x.w));
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f16x2 h = __builtin_convertvector((f32x2{a, b}), f16x2);
  hi = u32(h);
  lo = u32(__builtin_convertvector((f32x2{a - (float)h[0], b - (float)h[1]}), f16x2));
}
// hi / lo operands of 8 fp32 values (K indices 0..3 from t0, 4..7 from t1)
__device__ __forceinline__ void split8(const f32x4& t0, const f32x4& t1, f16x8& hi, f16x8& lo) {
  uint32_t h[4], l[4];
  split2(t0[0], t0[1], h[0], l[0]);
  split2(t0[2], t0[3], h[1], l[1]);
  split2(t1[0], t1[1], h[2], l[2]);
  split2(t1[2], t1[3], h[3], l[3]);
  hi = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(f16x8, make_uint4(l[0], l[1], l[2], l[3]));
}
// Maximum / sum over the four 16-lane rows of a wavefront (l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct Params {
  const bf16_t* q; const bf16_t* k; const bf16_t* v; const float* y; const float* dy;
  float* gq; float* gk; float* gv;
  int L, nch, window;
  float scale;
};

template <int NT>
struct Smem {
  static constexpr int DV = 16 * NT, RV = DV + 8;
  alignas(16) half_t kh3[3 * C][QH];            // keys of chunks c - 1, c, c + 1
  alignas(16) half_t kt[DK][KTS];               // k^T of chunk c
  alignas(16) half_t vh[C][RV];                 // values of chunk c
  alignas(16) half_t qh[2 * C][QH];             // queries of chunks c, c + 1
  alignas(16) half_t qt[DK][QTS];               // q^T
  alignas(16) half_t dyh[2 * C][RV], dyl[2 * C][RV];  // upstream gradient rows, hi / lo
  alignas(16) float lse[2 * C];                 // log2-domain log-sum-exp of the scaled scores
  alignas(16) float dd[2 * C];                  // D = dy . y
  alignas(16) float dsb[2 * C][DSS];            // dS, query x key
};

template <int NT>
__global__ __launch_bounds__(NTHR) void swa_bwd_mfma_kernel(Params p) {
  constexpr int DV = 16 * NT;
  __shared__ Smem<NT> S;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int L = p.L;
  const size_t bh = blockIdx.x / p.nch;
  const int j0 = (blockIdx.x % p.nch) * C;
  const f16x8 zero8 = {};

  // ---- stage the chunk's keys (with both neighbours), values, the 128
  // queries, their dy (hi / lo) and D
  for (int e = tid; e < 3 * C * 2; e += NTHR) {
    const int row = e >> 1, half = e & 1, key = j0 - C + row;
    const uint4 x = key >= 0 && key < L
                        ? h8_from_bf8(*reinterpret_cast<const uint4*>(p.k + ((size_t)bh * L + key) * DK + 8 * half))
                        : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&S.kh3[row][8 * half]) = x;
    if (row >= C && row < 2 * C) {
      const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) S.kt[8 * half + i][row - C] = h[i];
    }
  }
  for (int e = tid; e < C * (DV / 8); e += NTHR) {
    const int row = e / (DV / 8), c8 = e % (DV / 8), key = j0 + row;
    *reinterpret_cast<uint4*>(&S.vh[row][8 * c8]) =
        key < L ? h8_from_bf8(*reinterpret_cast<const uint4*>(p.v + ((size_t)bh * L + key) * DV + 8 * c8))
                : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    const int row = tid >> 1, half = tid & 1, i = j0 + row;
    const uint4 x = i < L ? h8_from_bf8(*reinterpret_cast<const uint4*>(p.q + ((size_t)bh * L + i) * DK + 8 * half))
                          : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&S.qh[row][8 * half]) = x;
    const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) S.qt[8 * half + e][row] = h[e];
    float d = 0.f;
#pragma unroll
    for (int c = half * (DV / 2); c < (half + 1) * (DV / 2); c += 8) {
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0, b0 = a0, b1 = a0;
      if (i < L) {
        const float* dyr = p.dy + ((size_t)bh * L + i) * DV + c;
        const float* yr = p.y + ((size_t)bh * L + i) * DV + c;
        a0 = *reinterpret_cast<const float4*>(dyr);
        a1 = *reinterpret_cast<const float4*>(dyr + 4);
        b0 = *reinterpret_cast<const float4*>(yr);
        b1 = *reinterpret_cast<const float4*>(yr + 4);
      }
      d += a0.x * b0.x + a0.y * b0.y + a0.z * b0.z + a0.w * b0.w + a1.x * b1.x + a1.y * b1.y + a1.z * b1.z +
           a1.w * b1.w;
      uint32_t hi[4], lo[4];
      split2(a0.x, a0.y, hi[0], lo[0]);
      split2(a0.z, a0.w, hi[1], lo[1]);
      split2(a1.x, a1.y, hi[2], lo[2]);
      split2(a1.z, a1.w, hi[3], lo[3]);
      *reinterpret_cast<uint4*>(&S.dyh[row][c]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&S.dyl[row][c]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    d += __shfl_xor(d, 1, 64);
    if (half == 0) S.dd[row] = d;
  }
  for (int e = tid; e < 2 * C * DSS; e += NTHR) (&S.dsb[0][0])[e] = 0.f;
  __syncthreads();

  // ---- log-sum-exp of query tiles w and w + 4: keys of kh3 tiles m .. m + 4
  const float c2 = p.scale * LOG2E;
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int m = w + 4 * qq;
    const int qg = j0 + 16 * m + r16;
    const f16x8 qv = g < 2 ? ld8(&S.qh[16 * m + r16][8 * g]) : zero8;
    float xs[5][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      const f16x8 kv = g < 2 ? ld8(&S.kh3[16 * (m + t) + r16][8 * g]) : zero8;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      x = mfma(kv, qv, x);  // [key 16 (m + t) + 4g + i][query]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kg = j0 - C + 16 * (m + t) + 4 * g + i;
        const bool valid = kg >= 0 && kg <= qg && qg - kg < p.window && qg < L;
        xs[t][i] = valid ? c2 * x[i] : -INFINITY;
        mx = fmaxf(mx, xs[t][i]);
      }
    }
    mx = rows_max(mx);
    float sum = 0.f;
    if (mx > -INFINITY)
#pragma unroll
      for (int t = 0; t < 5; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(xs[t][i] - mx);
    sum = rows_sum(sum);
    if (g == 0) S.lse[16 * m + r16] = mx > -INFINITY ? mx + __log2f(sum) : 0.f;
  }
  __syncthreads();

  // ---- wavefront w: key tile w against query tiles w .. w + 4
  const int kpos = 16 * w + r16;
  const f16x8 kv = g < 2 ? ld8(&S.kh3[C + kpos][8 * g]) : zero8;
  f32x4 pt[5], st[5];
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const int m = w + t;
    const f16x8 qa = g < 2 ? ld8(&S.qh[16 * m + r16][8 * g]) : zero8;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    x = mfma(qa, kv, x);  // [query 16m + 4g + i][key kpos]
    f32x4 dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) {
      const f16x8 vb = ld8(&S.vh[kpos][32 * ks + 8 * g]);
      dp = mfma(ld8(&S.dyh[16 * m + r16][32 * ks + 8 * g]), vb, dp);
      dp = mfma(ld8(&S.dyl[16 * m + r16][32 * ks + 8 * g]), vb, dp);
    }
    const float4 l4 = *reinterpret_cast<const float4*>(&S.lse[16 * m + 4 * g]);
    const float4 d4 = *reinterpret_cast<const float4*>(&S.dd[16 * m + 4 * g]);
    const float ls[4] = {l4.x, l4.y, l4.z, l4.w}, ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ql = 16 * m + 4 * g + i;
      const bool valid = j0 + ql < L && ql >= kpos && ql - kpos < p.window;
      const float pw = valid ? __builtin_amdgcn_exp2f(c2 * x[i] - ls[i]) : 0.f;
      pt[t][i] = pw;
      st[t][i] = pw * (dp[i] - ds[i]);
      S.dsb[ql][kpos] = st[t][i];
    }
  }
  // dk = Q^T dS and dv = P^T dY over query blocks (tile pairs 2kb, 2kb + 1)
  f32x4 dka = {0.f, 0.f, 0.f, 0.f};
  f32x4 dva[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) dva[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int ta = 2 * kb - w, tb = 2 * kb + 1 - w;  // indices into pt / st
    if (tb < 0 || ta > 4) continue;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 s0 = z4, s1 = z4, p0 = z4, p1 = z4;
#pragma unroll
    for (int t = 0; t < 5; ++t) {
      if (t == ta) { s0 = st[t]; p0 = pt[t]; }
      if (t == tb) { s1 = st[t]; p1 = pt[t]; }
    }
    f16x8 sh, sl, ph, pl;
    split8(s0, s1, sh, sl);
    split8(p0, p1, ph, pl);
    const f16x8 qa = cat44(&S.qt[r16][32 * kb + 4 * g], &S.qt[r16][32 * kb + 16 + 4 * g]);
    dka = mfma(qa, sh, dka);
    dka = mfma(qa, sl, dka);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f16x8 bh8, bl8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 32 * kb + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
        bh8[i] = S.dyh[row][16 * n + r16];
        bl8[i] = S.dyl[row][16 * n + r16];
      }
      dva[n] = mfma(ph, bh8, dva[n]);
      dva[n] = mfma(ph, bl8, dva[n]);
      dva[n] = mfma(pl, bh8, dva[n]);
    }
  }
  {
    const int kg = j0 + kpos;
    if (kg < L)
      *reinterpret_cast<float4*>(p.gk + ((size_t)bh * L + kg) * DK + 4 * g) =
          make_float4(p.scale * dka[0], p.scale * dka[1], p.scale * dka[2], p.scale * dka[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 16 * w + 4 * g + i;
      if (key < L)
#pragma unroll
        for (int n = 0; n < NT; ++n) p.gv[((size_t)bh * L + key) * DV + 16 * n + r16] = dva[n][i];
    }
  }
  __syncthreads();  // dS complete

  // ---- dq share of this key chunk: query tiles 2w, 2w + 1
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int m = 2 * w + qq;
    f32x4 dqa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(&S.dsb[16 * m + r16][32 * ks + 8 * g]);
      const float4 b = *reinterpret_cast<const float4*>(&S.dsb[16 * m + r16][32 * ks + 8 * g + 4]);
      f16x8 bh8, bl8;
      split8(f32x4{a.x, a.y, a.z, a.w}, f32x4{b.x, b.y, b.z, b.w}, bh8, bl8);
      const f16x8 ka = ld8(&S.kt[r16][32 * ks + 8 * g]);
      dqa = mfma(ka, bh8, dqa);
      dqa = mfma(ka, bl8, dqa);
    }
    const int qg = j0 + 16 * m + r16;
    if (qg < L) {
      float* dst = p.gq + ((size_t)bh * L + qg) * DK + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(dst + i, p.scale * dqa[i]);
    }
  }
}

// Clears n4 float4 of p (dq, which the key chunks then add into).
__global__ void zero_kernel(float4* p, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int NT>
hipError_t launch_nt(const SwaBwdArgs& a, hipStream_t s) {
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y; p.dy = a.dy;
  p.gq = a.gq; p.gk = a.gk; p.gv = a.gv;
  p.L = a.L; p.nch = (a.L + C - 1) / C; p.window = a.window; p.scale = a.scale;
  const size_t BH = (size_t)a.B * a.H, n4 = BH * a.L * DK / 4;
  const size_t zb = (n4 + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(zb < 4096 ? zb : 4096)), dim3(256), 0, s,
                     reinterpret_cast<float4*>(a.gq), n4);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL((swa_bwd_mfma_kernel<NT>), dim3((unsigned)(BH * p.nch)), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

}  // namespace swab

bool swa_bwd_mfma_supported(int dv) { return dv == 32 || dv == 64 || dv == 96 || dv == 128; }

hipError_t launch_swa_bwd_mfma(const SwaBwdArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 32: return swab::launch_nt<2>(a, s);
    case 64: return swab::launch_nt<4>(a, s);
    case 96: return swab::launch_nt<6>(a, s);
    case 128: return swab::launch_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace based
