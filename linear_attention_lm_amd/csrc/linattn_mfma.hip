// Causal Taylor linear attention, chunked, on bf16 matrix cores (gfx950
// v_mfma_f32_16x16x32_bf16) with fp32 accumulation: the bf16 path of
// based_linattn_fwd.
//
// Method (blog post "Базированная модель, часть 2": exp(q.k) is replaced by
// 1 + q.k + (q.k)^2/2 = phi(q).phi(k); paragraph on the state: a numerator
// KV-state and a denominator K-state; HazyResearch/based train README,
// training views: the chunked kernels compute what the quadratic view does):
// for a chunk c of C = 64 positions,
//   num_i = phi(q_i)^T S_c + sum_{j<=i in c} (1 + x_ij + x_ij^2/2) v_j
//   den_i = phi(q_i)^T z_c + sum_{j<=i in c} (1 + x_ij + x_ij^2/2),  x_ij = q_i.k_j
//   y_i = num_i / den_i;  S_{c+1} = S_c + phi(K_c)^T V_c,  z_{c+1} likewise.
//
// Design for MI355X:
// * The quadratic block of phi is symmetric, so the state keeps one row per
//   unordered pair a <= b (136 rows instead of 256) -- 160 feature slots with
//   the 16 linear features; the constant feature (sum of v, token count) is
//   carried in fp32 on the vector ALUs.  Slot r = 32kb + 8g + s holds the
//   feature of pattern (kb, s) shifted by 4g (cyclic on the 16 coordinates):
//   the lane group g of a matrix-core operand then builds its 8 features from
//   a register copy of q rotated by 4g, with compile-time register indices.
//   The pairs {a, a+8} are fixed by the shift by 8 and appear in two slots,
//   each with query weight 1/2.
// * bf16 has an 8-bit significand: q, k, v are exact, products q_a q_b and
//   the fp32 state are not.  Every inexact operand is split into hi + lo bf16
//   (exact for a product of two bf16 values) and the matrix product takes the
//   hi*hi + hi*lo + lo*hi passes, so the result carries ~16 significant bits.
// * Workgroup = 4 wavefronts; one workgroup per (batch*head, sequence
//   segment).  Per chunk: readout + in-chunk term (wavefront w owns positions
//   16w..16w+15 and every value column), then the state update (wavefront w
//   owns a contiguous quarter of the 10 x (d_v/16) state tiles, which stay in
//   accumulator registers across chunks), then the state is re-split into
//   bf16 hi/lo in LDS for the next chunk's readout.  The next chunk's inputs
//   are loaded from HBM into registers while the current one computes.
// * Long sequences are split into segments so that the grid fills the GPU: a
//   state-only pass computes each segment's state increment into the
//   workspace, a scan turns those into prefix states, and every segment then
//   starts from its prefix.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;         // positions per chunk
constexpr int NTHR = 256;     // 4 wavefronts
constexpr int NF = 160;       // feature slots (linear + quadratic), constant kept apart
constexpr int NKB = NF / 32;  // K-blocks of 32 slots in the readout
constexpr int QS = 20;        // fp32 q row stride in LDS (floats)
constexpr int QKB = 24;       // bf16 q/k row stride in LDS (elements)
constexpr int KT = C + 4;     // fp32 k^T row stride
constexpr int VT = C + 8;     // bf16 v^T row stride
constexpr int TT = NF + 8;    // bf16 state^T row stride
constexpr int ONES = 16;      // k^T row holding 1.0 (second factor of linear features)

enum SlotType : uint8_t { LIN = 0, DIAG = 1, OFF = 2, HALF = 3 };

struct SlotTables {
  uint8_t a[NF], b[NF], type[NF];  // feature of slot r: coordinates and kind
  int16_t phi_slot[DPHI];          // slot holding phi row f (-1: constant row)
};

__host__ __device__ constexpr int slot_d(int kb, int s) { return 2 * (kb - 1) + 1 + s / 4; }

constexpr SlotTables make_tables() {
  SlotTables t{};
  for (int r = 0; r < NF; ++r) {
    const int kb = r / 32, g = (r % 32) / 8, s = r % 8;
    int A = 0, B = 0, ty = 0;
    if (kb == 0) {
      A = s % 4;
      B = A;
      ty = s < 4 ? LIN : DIAG;
    } else {
      const int d = slot_d(kb, s);
      A = s % 4;
      B = A + d;
      ty = d == 8 ? HALF : OFF;
    }
    t.a[r] = (uint8_t)((A + 4 * g) % 16);
    t.b[r] = (uint8_t)((B + 4 * g) % 16);
    t.type[r] = (uint8_t)ty;
  }
  t.phi_slot[0] = -1;
  for (int f = 1; f < DPHI; ++f) {
    int want_a = 0, want_b = 0, want_t = 0;
    if (f < 1 + DK) {
      want_a = f - 1; want_b = f - 1; want_t = LIN;
    } else {
      const int a = (f - 1 - DK) / DK, b = (f - 1 - DK) % DK;
      want_a = a < b ? a : b; want_b = a < b ? b : a;
      want_t = a == b ? DIAG : OFF;
    }
    t.phi_slot[f] = -2;
    for (int r = 0; r < NF && t.phi_slot[f] == -2; ++r) {
      const int ty = t.type[r];
      const int lo = t.a[r] < t.b[r] ? t.a[r] : t.b[r], hi = t.a[r] < t.b[r] ? t.b[r] : t.a[r];
      if (want_t == LIN ? (ty == LIN && t.a[r] == want_a)
                        : (want_t == DIAG ? (ty == DIAG && t.a[r] == want_a)
                                          : ((ty == OFF || ty == HALF) && lo == want_a && hi == want_b)))
        t.phi_slot[f] = (int16_t)r;
    }
  }
  return t;
}
constexpr SlotTables kTables = make_tables();
__constant__ SlotTables c_tab = make_tables();

constexpr bool tables_ok() {
  for (int f = 1; f < DPHI; ++f)
    if (kTables.phi_slot[f] < 0) return false;
  // every unordered pair covered exactly once (HALF pairs: twice)
  int cnt[DK][DK] = {};
  for (int r = 0; r < NF; ++r) {
    if (kTables.type[r] == LIN) continue;
    const int a = kTables.a[r], b = kTables.b[r];
    const int lo = a < b ? a : b, hi = a < b ? b : a;
    cnt[lo][hi] += kTables.type[r] == HALF ? 1 : 2;
  }
  for (int a = 0; a < DK; ++a)
    for (int b = a; b < DK; ++b)
      if (cnt[a][b] != 2) return false;
  return true;
}
static_assert(tables_ok(), "feature slot layout must cover every pair");

// Value of the compact state (key-side convention: sum over tokens of
// [k_a | k_a^2 | k_a k_b] v) for slot r, column c, from a 273-row phi state.
__device__ __forceinline__ float compact_from_phi(const float* S, int r, int c, int ld) {
  const int a = c_tab.a[r], b = c_tab.b[r], ty = c_tab.type[r];
  if (ty == LIN) return S[(size_t)(1 + a) * ld + c];
  if (ty == DIAG) return SQRT2 * S[(size_t)(1 + DK + DK * a + a) * ld + c];
  return (S[(size_t)(1 + DK + DK * a + b) * ld + c] + S[(size_t)(1 + DK + DK * b + a) * ld + c]) * INV_SQRT2;
}

struct Params {
  const bf16_t* q; const bf16_t* k; const bf16_t* v; float* y;
  const float* S_in; const float* z_in; float* S_out; float* z_out;
  float* ws;        // [BH][nseg][NF+1][DV] compact state records (row NF = constant row)
  float* wsz;       // [BH][nseg][NF+1] likewise for z (entry NF = constant: token count)
  int L, nseg, seg_chunks;
};

// LDS.  vt is v^T with the 8-position groups of row `col` XOR-swizzled by
// (col / 8) % 8, so that the transposing writes of a wavefront spread over all
// banks while 8 consecutive positions stay contiguous for 16-byte reads.
template <int NT, bool FULL>
struct Smem {
  static constexpr int DV = 16 * NT;
  alignas(16) float qs[FULL ? C : 1][QS];
  alignas(16) bf16_t qb[FULL ? C : 1][QKB];
  alignas(16) bf16_t kb[FULL ? C : 1][QKB];
  alignas(16) float kt[DK + 1][KT];
  alignas(16) bf16_t vt[DV][VT];
  // state^T, hi and lo; row DV holds the denominator state z, row DV + 1
  // zeros (the z column tile of the readout); reused as fp32 staging at the end
  alignas(16) bf16_t tt[FULL ? 2 : 1][DV + 2][TT];
  alignas(16) float t0[DV];
  alignas(16) float vpart[NTHR];  // partial column sums of v
  alignas(16) float zf[NF];
};

// Column of v^T row `col` holding position t (see Smem).
__device__ __forceinline__ int vt_pos(int col, int t) { return ((((t >> 3) ^ (col >> 3)) & 7) << 3) | (t & 7); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// hi + lo bf16 split of two fp32 values, packed: hi = RNE(x), lo = RNE(x - hi)
// (one v_cvt_pk_bf16_f32 per pair for each part; hi is widened back to fp32
// by a shift / mask).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
}

__device__ __forceinline__ void split8(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
  uint4 h, l;
  split2(p[0], p[1], h.x, l.x);
  split2(p[2], p[3], h.y, l.y);
  split2(p[4], p[5], h.z, l.z);
  split2(p[6], p[7], h.w, l.w);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split4(float a, float b, float c, float d, bf16x4& hi, bf16x4& lo) {
  uint2 h, l;
  split2(a, b, h.x, l.x);
  split2(c, d, h.y, l.y);
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, l);
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Registers holding one chunk's inputs on their way from HBM to LDS.
template <int NT>
struct Prefetch {
  static constexpr int NV = NT / 2;  // uint4 of v per thread
  uint4 qk;
  uint4 v[NV];
};

// Buffer descriptors of one head's q, k, v: reads past the end of the
// sequence return zero, which pads the last chunk.
struct HeadRsrc {
  __amdgpu_buffer_rsrc_t q, k, v;
};
constexpr int RSRC_DW3 = 0x00020000;

__device__ __forceinline__ HeadRsrc head_rsrc(const Params& p, size_t bh, int DV) {
  const int nq = p.L * DK * 2, nv = p.L * DV * 2;
  HeadRsrc r;
  r.q = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + bh * p.L * DK), (short)0, nq, RSRC_DW3);
  r.k = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + bh * p.L * DK), (short)0, nq, RSRC_DW3);
  r.v = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + bh * (size_t)p.L * DV), (short)0, nv, RSRC_DW3);
  return r;
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Thread -> (position, 8 columns) of the v loads: a wavefront covers 8
// positions x 8 column groups per load (DV = 64) so that its transposing LDS
// writes hit distinct banks after the swizzle.
template <int NT>
__device__ __forceinline__ void load_chunk(const HeadRsrc& r, int t0, bool q_too, Prefetch<NT>& pf) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x;
  {
    const int u = tid & 127, j = u >> 1, h = u & 1;
    const int off = ((t0 + j) * DK + 8 * h) * 2;
    if (tid < 128) {
      if (q_too) pf.qk = bload(r.q, off);
    } else {
      pf.qk = bload(r.k, off);
    }
  }
#pragma unroll
  for (int i = 0; i < Prefetch<NT>::NV; ++i) {
    const int u = tid + NTHR * i;
    const int j = u / (DV / 8), c8 = u % (DV / 8);
    pf.v[i] = bload(r.v, ((t0 + j) * DV + 8 * c8) * 2);
  }
}

// k^T (fp32) and v^T (bf16, swizzled) of one chunk from the prefetch registers.
template <int NT>
__device__ __forceinline__ void store_kv(float (*kt)[KT], bf16_t (*vt)[VT], const Prefetch<NT>& pf) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x;
  if (tid >= 128) {
    const int u = tid & 127, j = u >> 1, h = u & 1;
    const uint32_t w[4] = {pf.qk.x, pf.qk.y, pf.qk.z, pf.qk.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kt[8 * h + 2 * i][j] = __uint_as_float(w[i] << 16);
      kt[8 * h + 2 * i + 1][j] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < Prefetch<NT>::NV; ++i) {
    const int u = tid + NTHR * i;
    const int j = u / (DV / 8), c8 = u % (DV / 8);
    const uint32_t w[4] = {pf.v[i].x, pf.v[i].y, pf.v[i].z, pf.v[i].w};
    const int pc = vt_pos(8 * c8, j);  // the same for the 8 columns of this group
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[8 * c8 + 2 * e][pc] = (bf16_t)(w[e] & 0xffffu);
      vt[8 * c8 + 2 * e + 1][pc] = (bf16_t)(w[e] >> 16);
    }
  }
}

template <int NT, bool FULL>
__device__ __forceinline__ void store_chunk(Smem<NT, FULL>& S, const Prefetch<NT>& pf) {
  const int tid = threadIdx.x;
  if constexpr (FULL) {
    const int u = tid & 127, j = u >> 1, h = u & 1;
    if (tid < 128) {
      const uint32_t w[4] = {pf.qk.x, pf.qk.y, pf.qk.z, pf.qk.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(&S.qb[j][8 * h]) = pf.qk;
      *reinterpret_cast<float4*>(&S.qs[j][8 * h]) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(&S.qs[j][8 * h + 4]) = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      *reinterpret_cast<uint4*>(&S.kb[j][8 * h]) = pf.qk;
    }
  }
  store_kv<NT>(S.kt, S.vt, pf);
}

// The state is 10 feature tiles x NT column tiles of 16x16.  Wavefront w owns
// feature tiles w and w + 4 for every column tile (slots 0 and 1) and feature
// tile 8 + w/2 for the column-tile half w%2 (slot 2): 2.5 NT tiles each, and
// the same code shape in every wavefront (tile indices are wave-uniform values).
template <int NT>
struct Own {
  static constexpr int PPW = 2 * NT + NT / 2;
  static_assert(NT % 2 == 0, "column tiles come in pairs");
};

// Feature tile m and column tile n of owned pair j of wavefront w.
template <int NT>
__device__ __forceinline__ void pair_mn(int w, int j, int& m, int& n) {
  if (j < NT) { m = w; n = j; }
  else if (j < 2 * NT) { m = w + 4; n = j - NT; }
  else { m = 8 + (w >> 1); n = (w & 1) * (NT / 2) + (j - 2 * NT); }
}

// bf16 B operand whose column 0 is all ones (lanes of column 0), else zero:
// multiplying by it sums the A operand's rows into column 0.
__device__ __forceinline__ bf16x8 ones_col0(int r16) {
  const uint32_t one2 = r16 == 0 ? 0x3f803f80u : 0u;  // bf16 1.0 twice
  return __builtin_bit_cast(bf16x8, make_uint4(one2, one2, one2, one2));
}

// State update of one chunk: tacc += psi'(K)^T V over the chunk, and the
// denominator state of the owned feature tiles, tz[slot] += psi'(K)^T 1
// (column 0 of each tz tile; the other columns stay zero).
template <int NT>
__device__ __forceinline__ void update_chunk(const float (*kt)[KT], const bf16_t (*vt)[VT], f32x4 (&tacc)[Own<NT>::PPW],
                                             f32x4 (&tz)[3], const int (&ia_)[3], const int (&ib_)[3]) {
  constexpr int H = NT / 2;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int n2 = (w & 1) * H;  // first column tile of slot 2
  const bf16x8 ones = ones_col0(r16);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 ahi[3], alo[3];
#pragma unroll
    for (int ms = 0; ms < 3; ++ms) {
      const float4* pa = reinterpret_cast<const float4*>(&kt[ia_[ms]][32 * ks + 8 * g]);
      const float4* pb = reinterpret_cast<const float4*>(&kt[ib_[ms]][32 * ks + 8 * g]);
      const float4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
      float pr[8] = {a0.x * b0.x, a0.y * b0.y, a0.z * b0.z, a0.w * b0.w,
                     a1.x * b1.x, a1.y * b1.y, a1.z * b1.z, a1.w * b1.w};
      split8(pr, ahi[ms], alo[ms]);
    }
    bf16x8 bv[NT], bv2[H];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int col = 16 * n + r16;
      bv[n] = *reinterpret_cast<const bf16x8*>(&vt[col][vt_pos(col, 32 * ks + 8 * g)]);
    }
#pragma unroll
    for (int n = 0; n < H; ++n) {
      const int col = 16 * (n2 + n) + r16;
      bv2[n] = *reinterpret_cast<const bf16x8*>(&vt[col][vt_pos(col, 32 * ks + 8 * g)]);
    }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int n = 0; n < NT; ++n) tacc[n] = mfma(pass ? alo[0] : ahi[0], bv[n], tacc[n]);
#pragma unroll
      for (int n = 0; n < NT; ++n) tacc[NT + n] = mfma(pass ? alo[1] : ahi[1], bv[n], tacc[NT + n]);
#pragma unroll
      for (int n = 0; n < H; ++n) tacc[2 * NT + n] = mfma(pass ? alo[2] : ahi[2], bv2[n], tacc[2 * NT + n]);
      tz[0] = mfma(pass ? alo[0] : ahi[0], ones, tz[0]);
      tz[1] = mfma(pass ? alo[1] : ahi[1], ones, tz[1]);
      if ((w & 1) == 0) tz[2] = mfma(pass ? alo[2] : ahi[2], ones, tz[2]);  // z of tile 8 + w/2 kept once
    }
  }
}

// Re-split the owned state tiles (and the denominator state) into bf16 hi/lo
// rows of S.tt (the caller has synchronised: nobody reads tt meanwhile).
template <int NT, bool FULL>
__device__ __forceinline__ void publish_state(Smem<NT, FULL>& S, const f32x4 (&tacc)[Own<NT>::PPW],
                                              const f32x4 (&tz)[3]) {
  constexpr int PPW = Own<NT>::PPW;
  constexpr int DV = 16 * NT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  if constexpr (FULL) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) {
      int m, n;
      pair_mn<NT>(w, j, m, n);
      bf16x4 hi, lo;
      split4(tacc[j][0], tacc[j][1], tacc[j][2], tacc[j][3], hi, lo);
      *reinterpret_cast<bf16x4*>(&S.tt[0][16 * n + r16][16 * m + 4 * g]) = hi;
      *reinterpret_cast<bf16x4*>(&S.tt[1][16 * n + r16][16 * m + 4 * g]) = lo;
    }
    if (r16 == 0) {
      const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
      for (int ms = 0; ms < 3; ++ms) {
        if (ms < 2 || (w & 1) == 0) {
          bf16x4 hi, lo;
          split4(tz[ms][0], tz[ms][1], tz[ms][2], tz[ms][3], hi, lo);
          *reinterpret_cast<bf16x4*>(&S.tt[0][DV][16 * mt[ms] + 4 * g]) = hi;
          *reinterpret_cast<bf16x4*>(&S.tt[1][DV][16 * mt[ms] + 4 * g]) = lo;
        }
      }
    }
  }
}

// The denominator state of the owned feature tiles back into S.zf.
template <int NT>
__device__ __forceinline__ void store_z(float* zf, const f32x4 (&tz)[3]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  if (r16 != 0) return;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
  for (int ms = 0; ms < 3; ++ms)
    if (ms < 2 || (w & 1) == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[16 * mt[ms] + 4 * g + i] = tz[ms][i];
}

// Initial owned state tiles: from a compact state in the workspace
// ([NF+1][DV], row NF = constant), else from the caller's phi-layout S_in,
// else zero.
template <int NT>
__device__ __forceinline__ void init_state(const float* compact, const float* Sin, f32x4 (&tacc)[Own<NT>::PPW]) {
  constexpr int DV = 16 * NT;
  constexpr int PPW = Own<NT>::PPW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    int m, n;
    pair_mn<NT>(w, j, m, n);
    const int c = 16 * n + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g + i;
      tacc[j][i] = compact ? compact[(size_t)r * DV + c] : (Sin ? compact_from_phi(Sin, r, c, DV) : 0.f);
    }
  }
}

template <int NT>
__device__ __forceinline__ void write_compact(const float* t0, const float* zf, const f32x4 (&tacc)[Own<NT>::PPW],
                                              float z0, float* dst, float* dz) {
  constexpr int DV = 16 * NT;
  constexpr int PPW = Own<NT>::PPW;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < PPW; ++j) {
    int m, nn;
    pair_mn<NT>(w, j, m, nn);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * DV + 16 * nn + r16] = tacc[j][i];
  }
  for (int c = tid; c < DV; c += NTHR) dst[(size_t)NF * DV + c] = t0[c];
  for (int r = tid; r < NF; r += NTHR) dz[r] = zf[r];
  if (tid == 0) dz[NF] = z0;
}

// Two wavefronts per SIMD (two workgroups per CU) where the LDS footprint
// allows it (d_v <= 64), one otherwise.
template <int NT> struct Occ { static constexpr int value = NT <= 4 ? 2 : 1; };

template <int NT, bool FULL>
__global__ __launch_bounds__(NTHR, Occ<NT>::value) void linattn_mfma_kernel(Params p) {
  constexpr int DV = 16 * NT;
  constexpr int PPW = Own<NT>::PPW;
  __shared__ Smem<NT, FULL> S;

  const int nseg_here = FULL ? p.nseg : p.nseg - 1;
  const size_t bh = blockIdx.x / nseg_here;
  const int seg = blockIdx.x % nseg_here;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int tok_begin = seg * p.seg_chunks * C;
  const int tok_end = min(p.L, tok_begin + p.seg_chunks * C);

  // ---- initial state.  One segment: the caller's S_in/z_in.  Several: the
  // state-only pass (segment s < nseg-1) starts segment 0 from S_in and the
  // others from zero and records increments; the main pass starts segment s
  // from the prefix record ws[s].  So S_in is read only before the main pass
  // and S_out (written by the last segment) may alias it.
  const size_t rec = (size_t)(NF + 1) * DV;
  const float* src = nullptr;   // compact record to start from
  const float* srcz = nullptr;
  const float* Sin = nullptr;
  const float* zin = nullptr;
  if (p.nseg > 1 && FULL) {
    src = p.ws + (bh * p.nseg + seg) * rec;
    srcz = p.wsz + (bh * p.nseg + seg) * (size_t)(NF + 1);
  } else if (FULL || seg == 0) {
    Sin = p.S_in ? p.S_in + bh * DPHI * DV : nullptr;
    zin = p.z_in ? p.z_in + bh * DPHI : nullptr;
  }
  f32x4 tacc[PPW];
  init_state<NT>(src, Sin, tacc);
  for (int c = tid; c < DV; c += NTHR) S.t0[c] = src ? src[(size_t)NF * DV + c] : (Sin ? Sin[c] : 0.f);
  for (int r = tid; r < NF; r += NTHR) S.zf[r] = srcz ? srcz[r] : (zin ? compact_from_phi(zin, r, 0, 1) : 0.f);
  float z0 = srcz ? srcz[NF] : (zin ? zin[0] : 0.f);
  for (int j = tid; j < KT; j += NTHR) S.kt[ONES][j] = 1.f;
  if constexpr (FULL)
    for (int j = tid; j < 2 * TT; j += NTHR) S.tt[j / TT][DV + 1][j % TT] = (bf16_t)0;
  __syncthreads();
  f32x4 tz[3];  // denominator state of the owned feature tiles, in column 0
  {
    const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
    for (int ms = 0; ms < 3; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) tz[ms][i] = r16 == 0 ? S.zf[16 * mt[ms] + 4 * g + i] : 0.f;
  }
  if constexpr (!FULL) {
    if (seg == 0)  // record 0: the initial state of the whole sequence
      write_compact<NT>(S.t0, S.zf, tacc, z0, p.ws + bh * p.nseg * rec, p.wsz + bh * p.nseg * (size_t)(NF + 1));
  }
  publish_state<NT, FULL>(S, tacc, tz);

  // update-operand rows of this wavefront's feature tiles (loop invariant)
  int ia[3], ib[3];
  {
    const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
    for (int mm = 0; mm < 3; ++mm) {
      const int r = 16 * mt[mm] + r16;
      const int ty = c_tab.type[r];
      ia[mm] = c_tab.a[r];
      ib[mm] = ty == LIN ? ONES : (ty == DIAG ? ia[mm] : c_tab.b[r]);
    }
  }

  const HeadRsrc rs = head_rsrc(p, bh, DV);
  Prefetch<NT> pf;
  if (tok_begin < tok_end) {
    load_chunk<NT>(rs, tok_begin, FULL, pf);
    store_chunk<NT, FULL>(S, pf);
  }

  for (int t0 = tok_begin; t0 < tok_end; t0 += C) {
    const int n = min(C, tok_end - t0);
    __syncthreads();  // chunk inputs, state hi/lo, t0 and zf visible
    const int tn = t0 + C;
    if (tn < tok_end) load_chunk<NT>(rs, tn, FULL, pf);

    // ---- constant row of the state: column sums of v over the chunk, in
    // NTHR / DV partial sums per column (order within a row is irrelevant)
    {
      constexpr int PARTS = NTHR / DV, SPAN = C / PARTS;
      const int col = tid % DV, part = tid / DV;
      float vs = 0.f;
#pragma unroll
      for (int j = 0; j < SPAN; j += 8) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(&S.vt[col][part * SPAN + j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) vs += (float)x[e];
      }
      S.vpart[tid] = vs;
    }

    // normalised outputs of this chunk; stored only after the next chunk's
    // inputs have been consumed, so that waiting for those loads never waits
    // for these stores (vector memory operations complete in order)
    float yv[FULL ? NT : 1][4];
    if constexpr (FULL) {
      // ---- readout of the state before the chunk: positions 16w + r16
      f32x4 acc[NT];
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
      float qr[16];
      {
        const int tok = 16 * w + r16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 x = *reinterpret_cast<const float4*>(&S.qs[tok][4 * ((g + m) & 3)]);
          qr[4 * m] = x.x; qr[4 * m + 1] = x.y; qr[4 * m + 2] = x.z; qr[4 * m + 3] = x.w;
        }
      }
      f32x4 accz = {0.f, 0.f, 0.f, 0.f};  // column 0: denominator of each position
      const int zrow = DV + (r16 == 0 ? 0 : 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float f[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (kb == 0) {
            f[s] = s < 4 ? qr[s] : 0.5f * qr[s - 4] * qr[s - 4];
          } else {
            const int d = slot_d(kb, s), A = s % 4, B = (A + d) % 16;
            f[s] = (d == 8 ? 0.5f : 1.f) * qr[A] * qr[B];
          }
        }
        bf16x8 ahi, alo;
        split8(f, ahi, alo);
        {
          const bf16x8 zhi = *reinterpret_cast<const bf16x8*>(&S.tt[0][zrow][32 * kb + 8 * g]);
          const bf16x8 zlo = *reinterpret_cast<const bf16x8*>(&S.tt[1][zrow][32 * kb + 8 * g]);
          accz = mfma(ahi, zhi, accz);
          accz = mfma(ahi, zlo, accz);
          accz = mfma(alo, zhi, accz);
        }
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(&S.tt[0][16 * nn + r16][32 * kb + 8 * g]);
          const bf16x8 blo = *reinterpret_cast<const bf16x8*>(&S.tt[1][16 * nn + r16][32 * kb + 8 * g]);
          acc[nn] = mfma(ahi, bhi, acc[nn]);
          acc[nn] = mfma(ahi, blo, acc[nn]);
          acc[nn] = mfma(alo, bhi, acc[nn]);
        }
      }

      // ---- in-chunk causal term: X^T = K Q^T on the keys 0 .. 16w+15
      const bf16x8 zero8 = {};
      const bf16x8 qbv = g < 2 ? *reinterpret_cast<const bf16x8*>(&S.qb[16 * w + r16][8 * g]) : zero8;
      bf16x4 xh[4], xl[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xh[m] = bf16x4{};
        xl[m] = bf16x4{};
        if (m <= w) {
          const bf16x8 kav = g < 2 ? *reinterpret_cast<const bf16x8*>(&S.kb[16 * m + r16][8 * g]) : zero8;
          const f32x4 x = mfma(kav, qbv, f32x4{0.f, 0.f, 0.f, 0.f});
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = 1.f + x[i] + 0.5f * x[i] * x[i];
            if (m == w && 4 * g + i > r16) a[i] = 0.f;  // key after query
          }
          split4(a[0], a[1], a[2], a[3], xh[m], xl[m]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb <= w) {
          bf16x8 ah, al;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ah[i] = xh[2 * kb][i]; ah[4 + i] = xh[2 * kb + 1][i];
            al[i] = xl[2 * kb][i]; al[4 + i] = xl[2 * kb + 1][i];
          }
          {
            const bf16x8 ones = ones_col0(r16);  // row sums of the weights -> denominator
            accz = mfma(ah, ones, accz);
            accz = mfma(al, ones, accz);
          }
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const int col = 16 * nn + r16;
            const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(&S.vt[col][vt_pos(col, 32 * kb + 4 * g)]);
            const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(&S.vt[col][vt_pos(col, 32 * kb + 16 + 4 * g)]);
            bf16x8 bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) { bv[i] = v0[i]; bv[4 + i] = v1[i]; }
            acc[nn] = mfma(ah, bv, acc[nn]);
            acc[nn] = mfma(al, bv, acc[nn]);
          }
        }
      }

      // ---- normalise and store: acc[nn][i] is position 16w + 4g + i, column 16nn + r16
      float rden[4];  // position 16w + 4g + i: its denominator sits in column 0 (lane 16g)
#pragma unroll
      for (int i = 0; i < 4; ++i) rden[i] = __builtin_amdgcn_rcpf(z0 + __shfl(accz[i], lane & 48, 64));
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const float c0 = S.t0[16 * nn + r16];
#pragma unroll
        for (int i = 0; i < 4; ++i) yv[nn][i] = (acc[nn][i] + c0) * rden[i];
      }
    }

    // ---- state update with this chunk (registers only)
    update_chunk<NT>(S.kt, S.vt, tacc, tz, ia, ib);
    z0 += (float)n;
    __syncthreads();  // every read of tt, zf, t0 and the chunk buffers done
    if (tid < DV) {
      float vs = 0.f;
#pragma unroll
      for (int part = 0; part < NTHR / DV; ++part) vs += S.vpart[part * DV + tid];
      S.t0[tid] += vs;
    }
    publish_state<NT, FULL>(S, tacc, tz);
    if (tn < tok_end) store_chunk<NT, FULL>(S, pf);
    if constexpr (FULL) {
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const int col = 16 * nn + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = 16 * w + 4 * g + i;
          if (pos < n) p.y[(bh * p.L + t0 + pos) * DV + col] = yv[nn][i];
        }
      }
    }
  }
  __syncthreads();

  // ---- segment result: the record after segment s (state-only pass) or S_out
  store_z<NT>(S.zf, tz);
  __syncthreads();
  if constexpr (!FULL) {
    write_compact<NT>(S.t0, S.zf, tacc, z0, p.ws + (bh * p.nseg + seg + 1) * rec,
                      p.wsz + (bh * p.nseg + seg + 1) * (size_t)(NF + 1));
  } else {
    if (p.S_out && seg == p.nseg - 1) {
      float* stage = reinterpret_cast<float*>(&S.tt[0][0][0]);  // [NF][DV] fp32
#pragma unroll
      for (int j = 0; j < PPW; ++j) {
        int m, nn;
        pair_mn<NT>(w, j, m, nn);
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(16 * m + 4 * g + i) * DV + 16 * nn + r16] = tacc[j][i];
      }
      __syncthreads();
      float* So = p.S_out + bh * DPHI * DV;
      for (int e = tid; e < DPHI * DV; e += NTHR) {
        const int f = e / DV, c = e % DV;
        const int r = c_tab.phi_slot[f];
        float val;
        if (r < 0) val = S.t0[c];
        else val = c_tab.type[r] == LIN ? stage[r * DV + c] : stage[r * DV + c] * INV_SQRT2;
        So[e] = val;
      }
      float* zo = p.z_out + bh * DPHI;
      for (int f = tid; f < DPHI; f += NTHR) {
        const int r = c_tab.phi_slot[f];
        zo[f] = r < 0 ? z0 : (c_tab.type[r] == LIN ? S.zf[r] : S.zf[r] * INV_SQRT2);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// State-only pass over segment s < nseg - 1 of a (batch, head): the segment's
// increment of the compact state (segment 0 starts from S_in, so its record
// carries the initial state too).  Update only, so one barrier per chunk:
// k^T / v^T are double-buffered in LDS and the inputs are prefetched into
// registers two chunks ahead.
template <int NT>
struct StateSmem {
  static constexpr int DV = 16 * NT;
  alignas(16) float kt[2][DK + 1][KT];
  alignas(16) bf16_t vt[2][DV][VT];
  alignas(16) float vpart[NTHR];
  alignas(16) float t0[DV];
  alignas(16) float zf[NF];
};

template <int NT>
__global__ __launch_bounds__(NTHR, Occ<NT>::value) void linattn_state_kernel(Params p) {
  constexpr int DV = 16 * NT;
  constexpr int PPW = Own<NT>::PPW;
  constexpr int PARTS = NTHR / DV, SPAN = C / PARTS;
  __shared__ StateSmem<NT> S;

  const int nsm = p.nseg - 1;
  const size_t bh = blockIdx.x / nsm;
  const int seg = blockIdx.x % nsm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int tok_begin = seg * p.seg_chunks * C;
  const int tok_end = min(p.L, tok_begin + p.seg_chunks * C);
  const size_t rec = (size_t)(NF + 1) * DV;

  const float* Sin = (seg == 0 && p.S_in) ? p.S_in + bh * DPHI * DV : nullptr;
  const float* zin = (seg == 0 && p.z_in) ? p.z_in + bh * DPHI : nullptr;
  f32x4 tacc[PPW];
  init_state<NT>(nullptr, Sin, tacc);
  for (int c = tid; c < DV; c += NTHR) S.t0[c] = Sin ? Sin[c] : 0.f;
  for (int r = tid; r < NF; r += NTHR) S.zf[r] = zin ? compact_from_phi(zin, r, 0, 1) : 0.f;
  float z0 = zin ? zin[0] : 0.f;
  for (int j = tid; j < 2 * KT; j += NTHR) S.kt[j / KT][ONES][j % KT] = 1.f;
  __syncthreads();
  f32x4 tz[3];
  {
    const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
    for (int ms = 0; ms < 3; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) tz[ms][i] = r16 == 0 ? S.zf[16 * mt[ms] + 4 * g + i] : 0.f;
  }
  if (seg == 0)  // record 0: the initial state of the whole sequence
    write_compact<NT>(S.t0, S.zf, tacc, z0, p.ws + bh * p.nseg * rec, p.wsz + bh * p.nseg * (size_t)(NF + 1));
  int ia[3], ib[3];
  {
    const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
    for (int mm = 0; mm < 3; ++mm) {
      const int r = 16 * mt[mm] + r16;
      const int ty = c_tab.type[r];
      ia[mm] = c_tab.a[r];
      ib[mm] = ty == LIN ? ONES : (ty == DIAG ? ia[mm] : c_tab.b[r]);
    }
  }

  const HeadRsrc rs = head_rsrc(p, bh, DV);
  const int col = tid % DV, part = tid / DV;
  float vs = 0.f;  // this thread's share of the column sums of v (constant row)
  Prefetch<NT> pa, pb;
  if (tok_begin < tok_end) {
    load_chunk<NT>(rs, tok_begin, false, pa);
    store_kv<NT>(S.kt[0], S.vt[0], pa);
  }
  if (tok_begin + C < tok_end) load_chunk<NT>(rs, tok_begin + C, false, pb);

  // chunk at t (in LDS buffer buf); `next` holds chunk t + C, `spare` receives t + 2C
  auto step = [&](int t, int buf, const Prefetch<NT>& next, Prefetch<NT>& spare) {
    __syncthreads();
    if (t + 2 * C < tok_end) load_chunk<NT>(rs, t + 2 * C, false, spare);
#pragma unroll
    for (int j = 0; j < SPAN; j += 8) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(&S.vt[buf][col][part * SPAN + j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vs += (float)x[e];
    }
    update_chunk<NT>(S.kt[buf], S.vt[buf], tacc, tz, ia, ib);
    if (t + C < tok_end) store_kv<NT>(S.kt[buf ^ 1], S.vt[buf ^ 1], next);
  };
  for (int t = tok_begin; t < tok_end; t += 2 * C) {
    step(t, 0, pb, pa);
    if (t + C < tok_end) step(t + C, 1, pa, pb);
  }
  z0 += (float)(tok_end - tok_begin);
  __syncthreads();
  S.vpart[tid] = vs;
  store_z<NT>(S.zf, tz);
  __syncthreads();
  if (tid < DV) {
    float sum = S.t0[tid];
#pragma unroll
    for (int q = 0; q < PARTS; ++q) sum += S.vpart[q * DV + tid];
    S.t0[tid] = sum;
  }
  __syncthreads();
  write_compact<NT>(S.t0, S.zf, tacc, z0, p.ws + (bh * p.nseg + seg + 1) * rec,
                    p.wsz + (bh * p.nseg + seg + 1) * (size_t)(NF + 1));
}

// Prefix over the segment records of each (batch, head): record s holds the
// increment of segment s-1 (record 1: the initial state plus that
// increment); after the scan record s is the state at the start of segment s.
__global__ void seg_scan_kernel(float* ws, float* wsz, int nseg, int rec, int BH) {
  const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t per_head = (size_t)rec + (NF + 1);
  if (e >= per_head * BH) return;
  const size_t bh = e / per_head, o = e % per_head;
  float* base;
  size_t stride;
  if (o < (size_t)rec) {
    base = ws + bh * nseg * (size_t)rec + o;
    stride = rec;
  } else {
    base = wsz + bh * nseg * (size_t)(NF + 1) + (o - rec);
    stride = NF + 1;
  }
  float run = base[stride];
  for (int s = 2; s < nseg; ++s) {
    run += base[s * stride];
    base[s * stride] = run;
  }
}

}  // namespace mfma

using namespace mfma;

// Segments per (batch, head): enough workgroups to fill the GPU's 256
// compute units (two per CU where they fit: d_v <= 64), each segment at
// least 4 chunks long.
void linattn_mfma_plan(int BH, int L, int dv, int* nseg, int* seg_chunks) {
  const int nch = (L + C - 1) / C;
  const int slots = dv <= 64 ? 512 : 256;
  int want = (slots + BH - 1) / BH;
  int cap = nch / 4;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  const int sc = (nch + want - 1) / want;
  *seg_chunks = sc < 1 ? 1 : sc;
  *nseg = nch == 0 ? 1 : (nch + *seg_chunks - 1) / *seg_chunks;
}

bool linattn_mfma_supported(int dv) { return dv == 32 || dv == 64 || dv == 96 || dv == 128; }

size_t linattn_mfma_workspace(int B, int H, int L, int dv) {
  if (!linattn_mfma_supported(dv)) return 0;
  int nseg, sc;
  linattn_mfma_plan(B * H, L, dv, &nseg, &sc);
  if (nseg <= 1) return 0;
  return (size_t)B * H * nseg * ((size_t)(NF + 1) * dv + (NF + 1)) * sizeof(float);
}

template <int NT>
static hipError_t launch_nt(const LinattnArgs& a, hipStream_t s) {
  constexpr int DV = 16 * NT;
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y;
  p.S_in = a.S_in; p.z_in = a.z_in; p.S_out = a.S_out; p.z_out = a.z_out;
  p.L = a.L;
  linattn_mfma_plan(a.B * a.H, a.L, DV, &p.nseg, &p.seg_chunks);
  const int BH = a.B * a.H;
  if (p.nseg > 1) {
    p.ws = (float*)a.workspace;
    p.wsz = p.ws + (size_t)BH * p.nseg * (NF + 1) * DV;
    hipLaunchKernelGGL((linattn_state_kernel<NT>), dim3(BH * (p.nseg - 1)), dim3(NTHR), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (p.nseg > 2) {
      const size_t total = (size_t)BH * ((size_t)(NF + 1) * DV + NF + 1);
      hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p.ws, p.wsz,
                         p.nseg, (NF + 1) * DV, BH);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((linattn_mfma_kernel<NT, true>), dim3(BH * p.nseg), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_linattn_mfma(const LinattnArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 32: return launch_nt<2>(a, s);
    case 64: return launch_nt<4>(a, s);
    case 96: return launch_nt<6>(a, s);
    case 128: return launch_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace based
