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
// One workgroup of 512 threads per (batch, head) and slice of DVS value
// columns (few heads: 16-column slices, so that more CUs share the work;
// many: the whole row); chunks run in sequence.  A per-head decay of the
// state (DEC) is the same pass with decay weights.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int C = 32;    // positions per chunk
constexpr int NFP = 160; // compact feature rows, padded (NCOMPACT used)

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

// Threads per workgroup: two wavefronts per SIMD (four measured slower: the
// tiny fp32 layer's linear attention 136 us against 94 us).
template <int DV>
constexpr int nthreads() { return 512; }

// Work split of a chunk among the NT threads: value columns in NCB blocks
// of CPT, and the other axis (the chunk's rows for the readout and the
// in-chunk term, the state's feature rows for the update) in NRB blocks.
template <int DV>
struct Split {
  static constexpr int NT = nthreads<DV>();
  static constexpr int NRB = 32;                 // row / feature blocks
  static constexpr int NCB = NT / NRB;           // column blocks
  static constexpr int CPT = DV / NCB;           // columns per thread
  static constexpr int RPT = C / NRB;            // chunk rows per thread (readout)
  static constexpr int FPT = NFP / NRB;          // feature rows per thread (update)
  static_assert(DV % NCB == 0 && C % NRB == 0 && NFP % NRB == 0, "tiling");
};


// DEC: the decayed variant (the based/train README's optional decay
// strategy, read as a per-head factor gamma in [0, 1] on the state:
// S_i = gamma S_{i-1} + phi(k_i) v_i^T, z likewise).  The state entering a
// chunk reaches its position i (0-based in the chunk) times gamma^(i+1), an
// in-chunk key j weighs gamma^(i-j), and the update is S <- gamma^n S +
// sum_j gamma^(n-1-j) phi(k_j) v_j^T over the chunk's n positions.
//
// Per chunk of C positions, with the features staged in LDS (fp32):
//   1. phi(q_i) of the chunk's queries (feature-major), and the in-chunk
//      weights W_ij = 1 + x + x^2/2 (x = q_i.k_j, j <= i < n; zero otherwise);
//   2. each thread's RPT rows x CPT columns of phi(Q) T and of W V, and the
//      rows' denominators, then y;
//   3. psi(k_j) of the chunk's keys (row-major; zero past n), and the
//      update T += psi(K)^T V, z += psi(K)^T 1, each thread FPT feature rows
//      x CPT columns.
// DVS: value columns of a workgroup (DV / DVS workgroups per head, slice
// blockIdx.x % (DV / DVS)); every slice forms the chunk's features, in-chunk
// weights and denominators itself, slice 0 writes z_out.
template <typename T, int DV, int DVS, int DEC>
__global__ __launch_bounds__(nthreads<DVS>()) void linattn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ y,
    const float* S_in, const float* z_in, float* S_out, float* z_out, int L, const float* gamma, int H) {
  static_assert(DV % DVS == 0, "whole slices");
  using SP = Split<DVS>;
  constexpr int NT = SP::NT, CPT = SP::CPT, RPT = SP::RPT, FPT = SP::FPT;
  constexpr int FT = C + 4;    // row stride of the feature-major query features
  constexpr int FK = NFP + 4;  // row stride of the row-major key features
  static_assert(NFP * FT >= C * FK, "the key features reuse the query features' buffer");
  __shared__ float Ts[NFP][DVS];  // compact state of the slice (rows NCOMPACT.. zero)
  __shared__ float zs[NFP];
  __shared__ float fbuf[NFP * FT];  // phi(q) [NFP][FT], then psi(k) [C][FK]
  __shared__ float qs[C][DK + 1];  // (odd stride: rows read down a column)
  __shared__ float ks[C][DK + 1];
  __shared__ float vs[C][DVS];
  __shared__ float wt[C][C + 1];  // in-chunk weights, [key][query]

  constexpr int NS = DV / DVS;
  const int bh = blockIdx.x / NS, col0 = (blockIdx.x % NS) * DVS;
  const float lg = DEC ? decay_lg2_clamped(log2f(gamma[bh % H])) : 0.f;
  const int tid = threadIdx.x;
  const int cb = tid % SP::NCB, ob = tid / SP::NCB;  // column block; row / feature block
  const int c0 = cb * CPT, r0 = ob * RPT, f0 = ob * FPT;
  const T* qb = q + (size_t)bh * L * DK;
  const T* kb = k + (size_t)bh * L * DK;
  const T* vb = v + (size_t)bh * L * DV + col0;
  float* yb = y + (size_t)bh * L * DV + col0;
  // feature fills: item u = tid + NT m (m < NFI; u < 2 NFP) is feature u / 2
  // over rows (u % 2) C/2 .. + C/2 - 1 of the chunk
  constexpr int HC = C / 2, NFI = (2 * NFP + NT - 1) / NT;
  FeatureCoef fq[NFI], fk[NFI];
  int fu[NFI], fr[NFI];
#pragma unroll
  for (int m = 0; m < NFI; ++m) {
    const int u = tid + NT * m;
    fu[m] = u < 2 * NFP ? u / 2 : -1;
    fr[m] = (u % 2) * HC;
    fq[m] = feature_coef<true>(fu[m] < 0 ? 0 : fu[m]);
    fk[m] = feature_coef<false>(fu[m] < 0 ? 0 : fu[m]);
  }

  for (int e = tid; e < NFP * DVS; e += NT) {
    const int f = e / DVS, c = e % DVS;
    Ts[f][c] = S_in && f < NCOMPACT ? compact_from_phi(S_in + (size_t)bh * DPHI * DV, f, col0 + c, DV) : 0.f;
  }
  for (int f = tid; f < NFP; f += NT)
    zs[f] = z_in && f < NCOMPACT ? compact_from_phi(z_in + (size_t)bh * DPHI, f, 0, 1) : 0.f;

  // the chunk's q, k, v in registers, the next chunk's loads in flight while
  // this one is processed (element e = tid + NT i of the chunk; zero past L)
  constexpr int NQK = (C * DK + NT - 1) / NT, NVV = (C * DVS + NT - 1) / NT;
  float pq[NQK], pk[NQK], pv[NVV];
  auto prefetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = tid + NT * i, j = e / DK, d = e % DK;
      const bool ok = e < C * DK && t0 + j < L;
      pq[i] = ok ? to_f32(qb[(size_t)(t0 + j) * DK + d]) : 0.f;
      pk[i] = ok ? to_f32(kb[(size_t)(t0 + j) * DK + d]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int e = tid + NT * i, j = e / DVS, d = e % DVS;
      pv[i] = e < C * DVS && t0 + j < L ? to_f32(vb[(size_t)(t0 + j) * DV + d]) : 0.f;
    }
  };
  prefetch(0);

  for (int t0 = 0; t0 < L; t0 += C) {
    const int n = min(C, L - t0);
    __syncthreads();  // the previous chunk's update done
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int e = tid + NT * i;
      if (e < C * DK) {
        qs[e / DK][e % DK] = pq[i];
        ks[e / DK][e % DK] = pk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int e = tid + NT * i;
      if (e < C * DVS) vs[e / DVS][e % DVS] = pv[i];
    }
    if (t0 + C < L) prefetch(t0 + C);
    __syncthreads();

    // ---- 1. query features and in-chunk weights
#pragma unroll
    for (int m = 0; m < NFI; ++m)
      if (fu[m] >= 0)
        for (int i = fr[m]; i < fr[m] + HC; ++i) fbuf[fu[m] * FT + i] = feature(fq[m], qs[i]);
    for (int e = tid; e < C * C; e += NT) {
      const int j = e / C, i = e % C;
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < DK; ++d) x = __builtin_fmaf(qs[i][d], ks[j][d], x);
      float w = j <= i && j < n ? 1.f + x + 0.5f * x * x : 0.f;
      if (DEC && j <= i) w *= exp2f(lg * (float)(i - j));
      wt[j][i] = w;
    }
    __syncthreads();

    // ---- 2. readout of the state before the chunk, plus the in-chunk term
    {
      float num[RPT][CPT], den[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        den[r] = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) num[r][c] = 0.f;
      }
#pragma unroll 3
      for (int f = 0; f < NCOMPACT; ++f) {
        float ph[RPT], st[CPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) ph[r] = fbuf[f * FT + r0 + r];
#pragma unroll
        for (int c = 0; c < CPT; ++c) st[c] = Ts[f][c0 + c];
        const float zf = zs[f];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          den[r] = __builtin_fmaf(ph[r], zf, den[r]);
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[r][c] = __builtin_fmaf(ph[r], st[c], num[r][c]);
        }
      }
      if (DEC) {  // the state before the chunk, decayed over positions t0 .. t0 + i
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          const float cf = exp2f(lg * (float)(r0 + r + 1));
          den[r] *= cf;
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[r][c] *= cf;
        }
      }
      const int jn = min(n, r0 + RPT);  // keys past the thread's last row weigh zero
      for (int j = 0; j < jn; ++j) {
        float w[RPT], vv[CPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) w[r] = wt[j][r0 + r];
#pragma unroll
        for (int c = 0; c < CPT; ++c) vv[c] = vs[j][c0 + c];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          den[r] += w[r];
#pragma unroll
          for (int c = 0; c < CPT; ++c) num[r][c] = __builtin_fmaf(w[r], vv[c], num[r][c]);
        }
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        if (r0 + r < n) {
          const float rd = 1.f / den[r];
          float* yr = yb + (size_t)(t0 + r0 + r) * DV + c0;
#pragma unroll
          for (int c = 0; c < CPT; ++c) yr[c] = num[r][c] * rd;
        }
      }
    }
    __syncthreads();  // every read of the query features done

    // ---- 3. key features (weighted by gamma^(n-1-j) when decayed) and the update
#pragma unroll
    for (int m = 0; m < NFI; ++m)
      if (fu[m] >= 0)
        for (int j = fr[m]; j < fr[m] + HC; ++j) {
          float x = 0.f;
          if (j < n) {
            x = feature(fk[m], ks[j]);
            if (DEC) x *= exp2f(lg * (float)(n - 1 - j));
          }
          fbuf[j * FK + fu[m]] = x;
        }
    __syncthreads();
    {
      float acc[FPT][CPT], zacc[FPT];
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        zacc[i] = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[i][c] = 0.f;
      }
      for (int j = 0; j < n; ++j) {
        float ps[FPT], vv[CPT];
#pragma unroll
        for (int i = 0; i < FPT; ++i) ps[i] = fbuf[j * FK + f0 + i];
#pragma unroll
        for (int c = 0; c < CPT; ++c) vv[c] = vs[j][c0 + c];
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
          zacc[i] += ps[i];
#pragma unroll
          for (int c = 0; c < CPT; ++c) acc[i][c] = __builtin_fmaf(ps[i], vv[c], acc[i][c]);
        }
      }
      const float gn = DEC ? exp2f(lg * (float)n) : 1.f;  // decay of the carried state over the chunk
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) Ts[f0 + i][c0 + c] = DEC ? gn * Ts[f0 + i][c0 + c] + acc[i][c]
                                                              : Ts[f0 + i][c0 + c] + acc[i][c];
        if (cb == 0) zs[f0 + i] = DEC ? gn * zs[f0 + i] + zacc[i] : zs[f0 + i] + zacc[i];
      }
    }
  }
  __syncthreads();
  if (S_out) {
    float* So = S_out + (size_t)bh * DPHI * DV + col0;
    for (int e = tid; e < DPHI * DVS; e += NT)
      So[(size_t)(e / DVS) * DV + e % DVS] = phi_from_compact(&Ts[0][0], e / DVS, e % DVS, DVS);
    if (col0 == 0) {
      float* zo = z_out + (size_t)bh * DPHI;
      for (int f = tid; f < DPHI; f += NT) zo[f] = phi_from_compact(zs, f, 0, 1);
    }
  }
}

// Short sequences without a state argument: the quadratic form of the same
// attention (the pages' views are interchangeable; every view gives
// y_i = sum_{j<=i} W_ij v_j / sum_{j<=i} W_ij with W_ij = 1 + x + x^2/2,
// x = q_i.k_j, times gamma^(i-j) when decayed).  Per position it costs
// L/2 (d_k + d_v) products against about C (d_k + d_v) + 2 * 153 d_v for the
// chunked pass, so below a few hundred positions it is the cheaper form, and
// its workgroups (one per 32 queries) run side by side instead of walking
// the chunks in order.
constexpr int QB = 32;            // queries per workgroup (and keys per block)
constexpr int QNT = 256;          // threads: 8 lanes per query
constexpr int QG = QNT / QB;
constexpr int QUAD_MAX_L = 512;   // longest sequence that takes this form
// SWA: the fused layer pass -- the window softmax of the same queries
// (scores s = scale q.k over keys i - window + 1 .. i, the window attention's
// definition: HazyResearch/based README, introduction) from the same q.k of
// the key blocks that reach into the workgroup's windows, with a running
// maximum per query (earlier sums rescaled when it grows), into y_swa.
template <typename T, int DV, int DEC, int SWA = 0>
__global__ __launch_bounds__(QNT) void linattn_quad_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          const T* __restrict__ v, float* __restrict__ y, int L,
                                                          const float* gamma, int H, float* __restrict__ y_swa = nullptr,
                                                          int window = 0, float scale = 0.f) {
  constexpr int CPL = DV / QG;  // value columns per lane, contiguous
  static_assert(DV % (2 * QG) == 0, "pairs of columns per lane");
  __shared__ float Ks[QB][DK + 1];
  __shared__ float Vs[QB][DV];
  __shared__ float W[QB][QB + 1];  // [query][key] weights of the current key block
  __shared__ float Ws[SWA ? QB : 1][QB + 1];  // window softmax weights of the block

  const int nblk = (L + QB - 1) / QB;
  const int bh = blockIdx.x / nblk, i0 = (blockIdx.x % nblk) * QB;
  const int tid = threadIdx.x, i = tid / QG, g = tid % QG, qpos = i0 + i;
  const float lg = DEC ? decay_lg2_clamped(log2f(gamma[bh % H])) : 0.f;
  const T* kb = k + (size_t)bh * L * DK;
  const T* vb = v + (size_t)bh * L * DV;
  float qr[DK];
#pragma unroll
  for (int d = 0; d < DK; ++d) qr[d] = qpos < L ? to_f32(q[((size_t)bh * L + qpos) * DK + d]) : 0.f;

  // a key block's k and v in registers (element e = tid + QNT i; zero past
  // L), the next block's loads in flight while this one is processed
  constexpr int NK = QB * DK / QNT, NV = QB * DV / QNT;
  static_assert(QB * DK % QNT == 0 && QB * DV % QNT == 0, "whole rounds");
  float pk[NK], pv[NV];
  auto prefetch = [&](int j0) {
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const int e = tid + QNT * r;
      pk[r] = j0 + e / DK < L ? to_f32(kb[(size_t)j0 * DK + e]) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int e = tid + QNT * r;
      pv[r] = j0 + e / DV < L ? to_f32(vb[(size_t)j0 * DV + e]) : 0.f;
    }
  };
  prefetch(0);

  float num[CPL], den = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) num[c] = 0.f;
  // window softmax: running maximum (base-2 scores), sum and weighted sums
  const float c2 = scale * 1.4426950408889634f;
  float msw = -INFINITY, dsw = 0.f, nsw[SWA ? CPL : 1];
#pragma unroll
  for (int c = 0; c < (SWA ? CPL : 1); ++c) nsw[c] = 0.f;
  for (int j0 = 0; j0 <= i0; j0 += QB) {
    __syncthreads();  // the previous block's reads done
#pragma unroll
    for (int r = 0; r < NK; ++r) {
      const int e = tid + QNT * r;
      Ks[e / DK][e % DK] = pk[r];
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
      const int e = tid + QNT * r;
      Vs[e / DV][e % DV] = pv[r];
    }
    if (j0 + QB <= i0) prefetch(j0 + QB);
    __syncthreads();
    // this lane's keys j = g + QG m of the block
    // (uniform: the block reaches into the window of the workgroup's first query)
    const bool swa_live = SWA && j0 + QB - 1 > i0 - window;
    float xs[QB / QG];
#pragma unroll
    for (int m = 0; m < QB / QG; ++m) {
      const int j = g + QG * m, kpos = j0 + j;
      float x = 0.f;
#pragma unroll
      for (int d = 0; d < DK; ++d) x = __builtin_fmaf(qr[d], Ks[j][d], x);
      xs[m] = x;
      float w = kpos <= qpos && kpos < L ? 1.f + x + 0.5f * x * x : 0.f;
      if (DEC && kpos <= qpos) w *= exp2f(lg * (float)(qpos - kpos));
      W[i][j] = w;
    }
    if constexpr (SWA) {
      if (swa_live) {
        float sc[QB / QG], bm = -INFINITY;
#pragma unroll
        for (int m = 0; m < QB / QG; ++m) {
          const int kpos = j0 + g + QG * m;
          sc[m] = kpos <= qpos && qpos - kpos < window && kpos < L ? c2 * xs[m] : -INFINITY;
          bm = fmaxf(bm, sc[m]);
        }
        // the maximum over the query's QG lanes (consecutive threads)
#pragma unroll
        for (int o = 1; o < QG; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
        const float mn = fmaxf(msw, bm);
        // earlier sums rescaled to the new maximum (none yet: all zero)
        const float rs = mn == -INFINITY || msw == -INFINITY ? 0.f : exp2f(msw - mn);
        dsw *= rs;
#pragma unroll
        for (int c = 0; c < CPL; ++c) nsw[c] *= rs;
        msw = mn;
#pragma unroll
        for (int m = 0; m < QB / QG; ++m) Ws[i][g + QG * m] = sc[m] == -INFINITY ? 0.f : exp2f(sc[m] - mn);
      }
    }
    __syncthreads();
    // the block's share, summed apart before it joins the running sums
    float nb[CPL], db = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) nb[c] = 0.f;
    for (int j = 0; j < QB; ++j) {
      const float w = W[i][j];
      db += w;
#pragma unroll
      for (int c = 0; c < CPL; c += 2) {
        const float2 vv = *reinterpret_cast<const float2*>(&Vs[j][CPL * g + c]);
        nb[c] = __builtin_fmaf(w, vv.x, nb[c]);
        nb[c + 1] = __builtin_fmaf(w, vv.y, nb[c + 1]);
      }
    }
    den += db;
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] += nb[c];
    if constexpr (SWA) {
      if (swa_live) {
        for (int j = 0; j < QB; ++j) {
          const float w = Ws[i][j];
          dsw += w;
#pragma unroll
          for (int c = 0; c < CPL; c += 2) {
            const float2 vv = *reinterpret_cast<const float2*>(&Vs[j][CPL * g + c]);
            nsw[c] = __builtin_fmaf(w, vv.x, nsw[c]);
            nsw[c + 1] = __builtin_fmaf(w, vv.y, nsw[c + 1]);
          }
        }
      }
    }
  }
  if (qpos < L) {
    const float rd = 1.f / den;
    float* yr = y + ((size_t)bh * L + qpos) * DV + CPL * g;
#pragma unroll
    for (int c = 0; c < CPL; c += 2) *reinterpret_cast<float2*>(yr + c) = make_float2(num[c] * rd, num[c + 1] * rd);
    if constexpr (SWA) {
      const float rw = 1.f / dsw;  // key qpos is always in its window: dsw >= 1
      float* ys = y_swa + ((size_t)bh * L + qpos) * DV + CPL * g;
#pragma unroll
      for (int c = 0; c < CPL; c += 2)
        *reinterpret_cast<float2*>(ys + c) = make_float2(nsw[c] * rw, nsw[c + 1] * rw);
    }
  }
}

template <typename T, int DV, int DEC>
hipError_t launch_quad(const LinattnArgs& a, hipStream_t s, float* y_swa = nullptr, int window = 0,
                       float scale = 0.f) {
  const unsigned nblk = (unsigned)((a.L + QB - 1) / QB);
  if (y_swa)
    hipLaunchKernelGGL((linattn_quad_kernel<T, DV, DEC, 1>), dim3(nblk * (unsigned)(a.B * a.H)), dim3(QNT), 0, s,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.y, a.L, a.gamma, a.H, y_swa, window, scale);
  else
    hipLaunchKernelGGL((linattn_quad_kernel<T, DV, DEC>), dim3(nblk * (unsigned)(a.B * a.H)), dim3(QNT), 0, s,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.y, a.L, a.gamma, a.H, nullptr, 0, 0.f);
  return hipGetLastError();
}

// The fused layer pass on the vector ALUs (both attentions from one pass
// over the key blocks): short sequences without a state argument.
template <typename T, int DV>
hipError_t launch_layer_dv(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  return a.gamma ? launch_quad<T, DV, 1>(a, s, y_swa, window, scale) : launch_quad<T, DV, 0>(a, s, y_swa, window, scale);
}
template <typename T>
hipError_t launch_layer_t(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  switch (a.dv) {
    case 16: return launch_layer_dv<T, 16>(a, y_swa, window, scale, s);
    case 32: return launch_layer_dv<T, 32>(a, y_swa, window, scale, s);
    case 48: return launch_layer_dv<T, 48>(a, y_swa, window, scale, s);
    case 64: return launch_layer_dv<T, 64>(a, y_swa, window, scale, s);
    case 80: return launch_layer_dv<T, 80>(a, y_swa, window, scale, s);
    case 96: return launch_layer_dv<T, 96>(a, y_swa, window, scale, s);
    case 112: return launch_layer_dv<T, 112>(a, y_swa, window, scale, s);
    case 128: return launch_layer_dv<T, 128>(a, y_swa, window, scale, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DV, int DVS, int DEC>
hipError_t launch_slices(const LinattnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((linattn_valu_kernel<T, DV, DVS, DEC>), dim3(a.B * a.H * (DV / DVS)), dim3(nthreads<DVS>()), 0,
                     s, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.y, a.S_in, a.z_in, a.S_out, a.z_out, a.L,
                     a.gamma, a.H);
  return hipGetLastError();
}

// Few heads: 16-column slices where they still fit one workgroup per CU
// (more, and the slices' repeated feature work costs more than they gain:
// 128 heads of 2048 positions, d_v 64: 794 -> 912 us).  Not for an in-place
// update (z_out = z_in): every slice reads z_in at its start and slice 0
// writes z_out at its end, in no fixed order.
template <typename T, int DV>
hipError_t launch_dv(const LinattnArgs& a, hipStream_t s) {
  if (!a.S_in && !a.S_out && a.L <= QUAD_MAX_L) {
    if (a.L == 0) return hipSuccess;
    return a.gamma ? launch_quad<T, DV, 1>(a, s) : launch_quad<T, DV, 0>(a, s);
  }
  const bool split = DV > 16 && (long long)a.B * a.H * (DV / 16) <= 256 && !(a.z_out && a.z_out == a.z_in);
  if (a.gamma) return split ? launch_slices<T, DV, 16, 1>(a, s) : launch_slices<T, DV, DV, 1>(a, s);
  return split ? launch_slices<T, DV, 16, 0>(a, s) : launch_slices<T, DV, DV, 0>(a, s);
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

bool layer_valu_fused(const LinattnArgs& a) { return !a.S_in && !a.S_out && a.L >= 1 && a.L <= QUAD_MAX_L; }

hipError_t launch_layer_valu(const LinattnArgs& a, float* y_swa, int window, float scale, bool bf16, hipStream_t s) {
  if (!layer_valu_fused(a) || !y_swa) return hipErrorInvalidValue;
  return bf16 ? launch_layer_t<bf16_t>(a, y_swa, window, scale, s) : launch_layer_t<float>(a, y_swa, window, scale, s);
}

}  // namespace based
