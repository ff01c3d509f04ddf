// Sliding-window softmax attention, backward on the matrix cores (bf16
// inputs, d_qk = 16, d_v in {32, 64, 96, 128}).
//
// The same gradients as the fp32 form (HazyResearch/based README intro:
// exact softmax over a short window; the based/train README's training views
// differentiate it): with p_ij = softmax_j(scale q_i.k_j) over the causal band,
// dP = dY V^T, D_i = dy_i . y_i and dS = P (dP - D):
//   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dY.
//
// A workgroup walks a run of 64-key chunks of one head.  With a window of at
// most 64, the keys of chunk c are seen by the queries of chunks c and c + 1
// only, so step c holds in LDS the keys of chunks c and c + 1, the values of
// chunk c, and the queries of chunks c and c + 1 with their upstream gradient
// (fp16 hi + lo) and D; the next step's chunks are loaded into registers
// meanwhile.  Step c:
//   1. log-sum-exp of the queries of chunk c + 1 (keys of chunks c, c + 1);
//   2. wavefront w takes key tile w against query tiles w .. w + 4: scores,
//      P, dP and dS in registers (lane: four queries of one key), then dk and
//      dv of its keys, complete, since both query chunks that see them are
//      here; dS goes to LDS as fp16 hi / lo band tiles [key][query];
//   3. dq of query tile w of chunk c (this key chunk's share plus the share
//      of chunk c - 1, carried in registers from the previous step) is
//      written; the share of query tile w of chunk c + 1 is carried on.
// A run starts one chunk early, without writing that chunk's dk and dv, to
// form the carried dq share of its first query chunk: nothing is added
// atomically and each input is read once per run.
//
// Operands whose contraction index runs down the rows of a row-major fp16
// array in LDS (Q^T, K^T, dY^T, dS^T) come from the transposing LDS load
// ds_read_b64_tr_b16: within each 16-lane block, lane j gives the address of
// a 4-element row segment and lane t receives element t % 4 of the segments
// of lanes t / 4 + 4i, i = 0..3.  With lane j pointing at row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3, lane t gets rows r0 .. r0 + 3 of column
// c0 + t (lane layout checked on the GPU with a probe).
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace swab {

typedef _Float16 half_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int C = 64;      // positions per chunk
constexpr int NTHR = 256;  // 4 wavefronts
constexpr int BT = 16;     // band tile side
constexpr float LOG2E = 1.4426950408889634f;
constexpr int RSRC_DW3 = 0x00020000;

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ f16x8 ld8(const half_t* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x8 cat(const uint2& a, const uint2& b) {
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
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

// Transposing read: rows r0 .. r0 + 3 of column c0 + (lane % 16) of the
// row-major fp16 array at `base` (row stride ld elements), as 4 packed halves.
__device__ __forceinline__ uint2 tr4(const half_t* base, int r0, int c0, int ld) {
  const int j = threadIdx.x & 15;
  const half_t* a = base + (r0 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
  return __builtin_bit_cast(uint2, v);
}

struct Params {
  const bf16_t* q; const bf16_t* k; const bf16_t* v; const float* y; const float* dy;
  float* gq; float* gk; float* gv;
  int L, nch, nseg, seg_chunks, window;
  float scale;
};

// Buffer descriptors of one head's inputs: reads past the end of the
// sequence return zero.
struct Rsrc {
  __amdgpu_buffer_rsrc_t q, k, v, y, dy;
};

__device__ __forceinline__ Rsrc head_rsrc(const Params& p, size_t bh, int DV) {
  const int nqk = p.L * DK * 2, nv = p.L * DV * 2, ny = p.L * DV * 4;
  Rsrc r;
  r.q = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + bh * p.L * DK), (short)0, nqk, RSRC_DW3);
  r.k = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + bh * p.L * DK), (short)0, nqk, RSRC_DW3);
  r.v = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + bh * (size_t)p.L * DV), (short)0, nv, RSRC_DW3);
  r.y = __builtin_amdgcn_make_buffer_rsrc((void*)(p.y + bh * (size_t)p.L * DV), (short)0, ny, RSRC_DW3);
  r.dy = __builtin_amdgcn_make_buffer_rsrc((void*)(p.dy + bh * (size_t)p.L * DV), (short)0, ny, RSRC_DW3);
  return r;
}
__device__ __forceinline__ uint2 bload2(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint4 bload4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int NT>
struct Smem {
  static constexpr int DV = 16 * NT, RV = DV + 8;
  alignas(16) half_t kh[3][C][DK];                  // keys; chunk c in slot (c + 3) % 3
  alignas(16) half_t qh[2][C][DK];                  // queries; chunk c in slot c & 1
  alignas(16) half_t vh[C][RV];                     // values of the current key chunk
  alignas(16) half_t dyh[2][C][RV], dyl[2][C][RV];  // upstream gradient hi / lo (slot as qh)
  alignas(16) float lse[2][C];                      // log2-domain log-sum-exp of the scaled scores
  alignas(16) float dd[2][C];                       // D = dy . y
  alignas(16) half_t bh[4][5][BT][BT], bl[4][5][BT][BT];  // dS [key tile][query tile - key tile][key][query]
};

__device__ __forceinline__ int slot3(int c) { return (c + 3) % 3; }

// One step's inputs on their way from HBM to LDS: keys of one chunk, values
// of the chunk before it, queries (with dy and y) of the keys' chunk.
// Thread t: row t / 4, part t % 4 of the row.
template <int NT>
struct Pre {
  uint2 k, q;
  uint4 v[NT / 2];
  uint4 dy[NT], y[NT];  // fp32 bits
};

template <int NT>
__device__ __forceinline__ void load_step(const Rsrc& r, int kc, int vc, Pre<NT>& p) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x, row = tid >> 2, part = tid & 3;
  p.k = kc >= 0 ? bload2(r.k, ((kc * C + row) * DK + 4 * part) * 2) : make_uint2(0u, 0u);
  p.q = bload2(r.q, ((kc * C + row) * DK + 4 * part) * 2);
#pragma unroll
  for (int i = 0; i < NT / 2; ++i) {
    const int u = tid + NTHR * i, vr = u / (DV / 8), c8 = u % (DV / 8);
    p.v[i] = vc >= 0 ? bload4(r.v, ((vc * C + vr) * DV + 8 * c8) * 2) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int off = ((kc * C + row) * DV + part * 4 * NT + 4 * j) * 4;
    p.dy[j] = bload4(r.dy, off);
    p.y[j] = bload4(r.y, off);
  }
}

template <int NT>
__device__ __forceinline__ void store_step(Smem<NT>& S, int kc, bool with_v, const Pre<NT>& p) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x, row = tid >> 2, part = tid & 3, s = kc & 1;
  *reinterpret_cast<uint2*>(&S.kh[slot3(kc)][row][4 * part]) = make_uint2(h2_from_bf2(p.k.x), h2_from_bf2(p.k.y));
  *reinterpret_cast<uint2*>(&S.qh[s][row][4 * part]) = make_uint2(h2_from_bf2(p.q.x), h2_from_bf2(p.q.y));
  if (with_v)
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) {
      const int u = tid + NTHR * i, vr = u / (DV / 8), c8 = u % (DV / 8);
      *reinterpret_cast<uint4*>(&S.vh[vr][8 * c8]) = h8_from_bf8(p.v[i]);
    }
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float4 a = __builtin_bit_cast(float4, p.dy[j]), b = __builtin_bit_cast(float4, p.y[j]);
    d += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
    uint32_t h0, l0, h1, l1;
    split2(a.x, a.y, h0, l0);
    split2(a.z, a.w, h1, l1);
    const int col = part * 4 * NT + 4 * j;
    *reinterpret_cast<uint2*>(&S.dyh[s][row][col]) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(&S.dyl[s][row][col]) = make_uint2(l0, l1);
  }
  d += __shfl_xor(d, 1, 64);
  d += __shfl_xor(d, 2, 64);
  if (part == 0) S.dd[s][row] = d;
}

template <int NT>
__global__ __launch_bounds__(NTHR, NT <= 4 ? 2 : 1) void swa_bwd_mfma_kernel(Params p) {
  constexpr int DV = 16 * NT, RV = DV + 8;
  __shared__ Smem<NT> S;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int L = p.L;
  const size_t bh = blockIdx.x / p.nseg;
  const int seg = blockIdx.x % p.nseg;
  const int c_begin = seg * p.seg_chunks, c_end = min(p.nch, c_begin + p.seg_chunks);
  const int c0 = c_begin - 1;  // the run starts one chunk early (chunk -1: keys zero, masked)
  const f16x8 zero8 = {};
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  const float c2 = p.scale * LOG2E;
  const Rsrc rs = head_rsrc(p, bh, DV);

  // ---- keys of chunks c0 and c0 + 1, values of chunk c0, queries of c0 + 1
  Pre<NT> pf;
  {
    const int row = tid >> 2, part = tid & 3;
    const uint2 kf = c0 >= 0 ? bload2(rs.k, ((c0 * C + row) * DK + 4 * part) * 2) : make_uint2(0u, 0u);
    load_step<NT>(rs, c0 + 1, c0, pf);
    *reinterpret_cast<uint2*>(&S.kh[slot3(c0)][row][4 * part]) = make_uint2(h2_from_bf2(kf.x), h2_from_bf2(kf.y));
    store_step<NT>(S, c0 + 1, c0 >= 0, pf);
  }

  f32x4 carry = z4;  // dq share of query tile w of the next chunk
  for (int c = c0; c < c_end; ++c) {
    if constexpr (NT <= 4) progress_priority(c - c0, c_end - c0);  // two workgroups per CU
    __syncthreads();  // this step's chunks staged; the previous step's reads done
    const bool more = c + 1 < c_end;
    if (more) load_step<NT>(rs, c + 2, c + 1, pf);

    // ---- 1. log-sum-exp of query tile w of chunk c + 1: key tiles w .. w + 4
    // of chunks c, c + 1 (transposed scores: lane = query, four keys)
    {
      const int s1 = (c + 1) & 1;
      const int qg = (c + 1) * C + 16 * w + r16;
      const f16x8 qv = g < 2 ? ld8(&S.qh[s1][16 * w + r16][8 * g]) : zero8;
      float xs[5][4];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        const int T = w + t, kc = c + (T >> 2), kr = 16 * (T & 3);
        const f16x8 kv = g < 2 ? ld8(&S.kh[slot3(kc)][kr + r16][8 * g]) : zero8;
        const f32x4 x = mfma(kv, qv, z4);  // [key kr + 4g + i][query]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kg = kc * C + kr + 4 * g + i;
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
      if (g == 0) S.lse[s1][16 * w + r16] = mx > -INFINITY ? mx + __log2f(sum) : 0.f;
    }
    __syncthreads();  // lse of chunk c + 1 complete
    if (c >= 0) {  // (chunk -1 has no keys: its step only forms the log-sum-exp of chunk 0)

    // ---- 2. key tile w of chunk c against query tiles m = w .. w + 4 of
    // chunks c, c + 1.  In the early step only chunk c + 1's queries count.
    const bool early = c < c_begin;
    const int kc3 = slot3(c);
    const int kpos = 16 * w + r16, kg = c * C + kpos;
    {
      const f16x8 kv = g < 2 ? ld8(&S.kh[kc3][kpos][8 * g]) : zero8;
      f32x4 pt[5], st[5];
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        const int m = w + t, qc = c + (m >> 2), s = qc & 1, qr = 16 * (m & 3);
        pt[t] = z4;
        st[t] = z4;
        if (early && m < 4) continue;
        const f16x8 qa = g < 2 ? ld8(&S.qh[s][qr + r16][8 * g]) : zero8;
        const f32x4 x = mfma(qa, kv, z4);  // [query qr + 4g + i][key kpos]
        f32x4 dp = z4;
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
          const f16x8 vb = ld8(&S.vh[kpos][32 * ks + 8 * g]);
          dp = mfma(ld8(&S.dyh[s][qr + r16][32 * ks + 8 * g]), vb, dp);
          dp = mfma(ld8(&S.dyl[s][qr + r16][32 * ks + 8 * g]), vb, dp);
        }
        const float4 l4 = *reinterpret_cast<const float4*>(&S.lse[s][qr + 4 * g]);
        const float4 d4 = *reinterpret_cast<const float4*>(&S.dd[s][qr + 4 * g]);
        const float ls[4] = {l4.x, l4.y, l4.z, l4.w}, ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qg = qc * C + qr + 4 * g + i;
          const bool valid = qg < L && qg >= kg && qg - kg < p.window;
          const float pw = valid ? __builtin_amdgcn_exp2f(c2 * x[i] - ls[i]) : 0.f;
          pt[t][i] = pw;
          st[t][i] = pw * (dp[i] - ds[i]);
        }
        uint32_t h0, l0, h1, l1;
        split2(st[t][0], st[t][1], h0, l0);
        split2(st[t][2], st[t][3], h1, l1);
        *reinterpret_cast<uint2*>(&S.bh[w][t][r16][4 * g]) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(&S.bl[w][t][r16][4 * g]) = make_uint2(l0, l1);
      }
      if (!early) {
        // dk^T = Q^T dS and dv^T = dY^T P over query tile pairs (2kb, 2kb + 1)
        f32x4 dka = z4;
        f32x4 dva[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) dva[n] = z4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int ta = 2 * kb - w, tb = ta + 1;  // indices into pt / st
          if (tb < 0 || ta > 4) continue;
          f32x4 s0 = z4, s1 = z4, p0 = z4, p1 = z4;
#pragma unroll
          for (int t = 0; t < 5; ++t) {
            if (t == ta) { s0 = st[t]; p0 = pt[t]; }
            if (t == tb) { s1 = st[t]; p1 = pt[t]; }
          }
          const int s = (c + (kb >> 1)) & 1, r0 = 16 * ((2 * kb) & 3) + 4 * g;
          const f16x8 qT = cat(tr4(&S.qh[s][0][0], r0, 0, DK), tr4(&S.qh[s][0][0], r0 + 16, 0, DK));
          f16x8 sh, sl, ph, pl;
          split8(s0, s1, sh, sl);
          split8(p0, p1, ph, pl);
          dka = mfma(qT, sh, dka);
          dka = mfma(qT, sl, dka);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const f16x8 yh = cat(tr4(&S.dyh[s][0][0], r0, 16 * n, RV), tr4(&S.dyh[s][0][0], r0 + 16, 16 * n, RV));
            const f16x8 yl = cat(tr4(&S.dyl[s][0][0], r0, 16 * n, RV), tr4(&S.dyl[s][0][0], r0 + 16, 16 * n, RV));
            dva[n] = mfma(yh, ph, dva[n]);
            dva[n] = mfma(yl, ph, dva[n]);
            dva[n] = mfma(yh, pl, dva[n]);
          }
        }
        if (kg < L) {  // lane: key kpos, dims / columns 4g .. 4g + 3
          // gradients leave non-temporally (straight to memory): 72.6 -> 71.7 us
          __builtin_nontemporal_store(dka * p.scale, reinterpret_cast<f32x4*>(p.gk + ((size_t)bh * L + kg) * DK + 4 * g));
#pragma unroll
          for (int n = 0; n < NT; ++n)
            __builtin_nontemporal_store(dva[n], reinterpret_cast<f32x4*>(p.gv + ((size_t)bh * L + kg) * DV + 16 * n + 4 * g));
        }
      }
    }
    __syncthreads();  // dS band complete

    // ---- 3. dq^T = K^T dS^T of this key chunk for query tiles w (chunk c)
    // and w + 4 (chunk c + 1): key tile pairs (2kb, 2kb + 1) inside the band
    {
      f32x4 share[2];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int m = w + 4 * qq;
        f32x4 acc = z4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int o0 = m - 2 * kb, o1 = o0 - 1;
          const bool in0 = o0 >= 0 && o0 <= 4, in1 = o1 >= 0 && o1 <= 4;
          if (!in0 && !in1) continue;
          const f16x8 kT = cat(tr4(&S.kh[kc3][0][0], 32 * kb + 4 * g, 0, DK),
                               tr4(&S.kh[kc3][0][0], 32 * kb + 16 + 4 * g, 0, DK));
          uint2 h0 = make_uint2(0u, 0u), l0 = h0, h1 = h0, l1 = h0;
          if (in0) {
            h0 = tr4(&S.bh[2 * kb][o0][0][0], 4 * g, 0, BT);
            l0 = tr4(&S.bl[2 * kb][o0][0][0], 4 * g, 0, BT);
          }
          if (in1) {
            h1 = tr4(&S.bh[2 * kb + 1][o1][0][0], 4 * g, 0, BT);
            l1 = tr4(&S.bl[2 * kb + 1][o1][0][0], 4 * g, 0, BT);
          }
          acc = mfma(kT, cat(h0, h1), acc);
          acc = mfma(kT, cat(l0, l1), acc);
        }
        share[qq] = acc;  // [dim 4g + i][query r16]
      }
      if (!early) {
        const int qg = c * C + 16 * w + r16;
        if (qg < L) {
          const f32x4 t = carry + share[0];
          __builtin_nontemporal_store(t * p.scale, reinterpret_cast<f32x4*>(p.gq + ((size_t)bh * L + qg) * DK + 4 * g));
        }
      }
      carry = share[1];
    }
    }
    // ---- the next step's chunks into the slots this step no longer reads
    if (more) store_step<NT>(S, c + 2, true, pf);
  }
}

template <int NT>
hipError_t launch_nt(const SwaBwdArgs& a, hipStream_t s) {
  constexpr int DV = 16 * NT;
  if ((size_t)a.L * DV * 4 >= (size_t)1 << 31) return hipErrorInvalidValue;  // 32-bit buffer offsets
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y; p.dy = a.dy;
  p.gq = a.gq; p.gk = a.gk; p.gv = a.gv;
  p.L = a.L; p.nch = (a.L + C - 1) / C; p.window = a.window; p.scale = a.scale;
  // runs of chunks per head: enough workgroups for two per CU (one for
  // d_v > 64), at least four chunks per run
  const int BH = a.B * a.H;
  const int slots = NT <= 4 ? 512 : 256;
  int want = (slots + BH - 1) / BH;
  const int cap = p.nch / 4 > 1 ? p.nch / 4 : 1;
  want = want < 1 ? 1 : (want > cap ? cap : want);
  p.seg_chunks = (p.nch + want - 1) / want;
  p.nseg = (p.nch + p.seg_chunks - 1) / p.seg_chunks;
  hipLaunchKernelGGL((swa_bwd_mfma_kernel<NT>), dim3((unsigned)((size_t)BH * p.nseg)), dim3(NTHR), 0, s, p);
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
