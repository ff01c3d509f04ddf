// Causal Taylor linear attention, chunked, on the matrix cores of gfx950
// (v_mfma_f32_16x16x32_f16, fp32 accumulation): the bf16 path of
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
// * Operands are fp16 (11-bit significand; bf16 inputs convert exactly):
//   features are products of two fp16 values rounded once (v_pk_mul_f16),
//   the fp32 state is rounded once to fp16 for the readout, and the in-chunk
//   weights 1 + x + x^2/2 are split into fp16 hi + lo (two passes).  The
//   state copy is scaled by a power of two chosen from its largest entry, so
//   its fp16 range never limits the sequence length; the query weights 1/2
//   ride on that copy, so query features are plain products.  Range of the
//   inputs: |q|, |k| < 2^7 per coordinate, |q.k| < 2^8, |v| < 2^15.
// * Workgroup = 4 wavefronts; one workgroup per (batch*head, sequence
//   segment).  Per chunk: readout + in-chunk term (wavefront w owns positions
//   16w..16w+15 and every value column), then the state update (wavefront w
//   owns a contiguous quarter of the 10 x (d_v/16) state tiles, which stay in
//   accumulator registers across chunks), then the state is written to LDS
//   as scaled fp16 for the next chunk's readout.  The next chunk's inputs
//   are loaded from HBM into registers while the current one computes.
// * Long sequences are split into segments so that the grid fills the GPU: a
//   state-only pass computes each segment's state increment into the
//   workspace, a scan turns those into prefix states, and every segment then
//   starts from its prefix.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace mfma {

typedef _Float16 half_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;         // positions per chunk
constexpr int NTHR = 256;     // 4 wavefronts
constexpr int NF = 160;       // feature slots (linear + quadratic), constant kept apart
constexpr int NKB = NF / 32;  // K-blocks of 32 slots in the readout
constexpr int QH = 24;        // fp16 q / k row stride in LDS (elements)
constexpr int KT = C + 8;     // fp16 k^T row stride
constexpr int TT = NF + 8;    // fp16 state^T row stride
constexpr int ONES = 16;      // k^T row holding 1.0 (second factor of linear features)
constexpr int SCALE_TOP = 13; // the scaled fp16 state stays below 2^(SCALE_TOP + 1)
// Up to this many segments per head the main pass sums the segment
// increments before its segment itself; beyond, a scan pass writes each
// segment's starting state.
constexpr int MAX_SUM = 3;
static_assert(C == layout::CHUNK && NF == layout::FWD_SLOTS && MAX_SUM == layout::FWD_MAX_SUM,
              "planning constants (plan.cpp) must match the kernels");

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
  float* ws;        // [BH][nseg] compact state records of (NF+1) DV floats (record_offset; row NF = constant; record 0: S_in)
  float* wsz;       // [BH][nseg][NF+1] likewise for z (entry NF = constant: token count)
  int L, nseg, seg_chunks;
  float* y_swa;     // sliding-window softmax output of the fused layer pass
  int window;
  float swa_scale;
  const float* gamma;  // [H] state decay per head (decayed variant)
  int H;
  int nrec;            // state-only pass: segments per head it covers (0: nseg - 1)
};

// Decayed variant: log2 of the head's decay factor (gamma^d = gpow(lg, d)).
__device__ __forceinline__ float decay_lg2(const Params& p, size_t bh) {
  return decay_lg2_clamped(__log2f(p.gamma[bh % p.H]));
}
// a value that every lane holds alike, moved to a scalar register
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// fp16 row stride of the row-major v chunk in LDS (8 halves of padding keep
// the transposing reads of four consecutive rows on distinct banks)
template <int NT> constexpr int vrow() { return 16 * NT + 8; }

// LDS of the main pass.  With the sliding window (SWA) the row-major k and v
// keep the previous chunk too (NB = 2 buffers).
template <int NT, int SWA, int HI = 0, int DEC = 0>
struct Smem {
  static constexpr int DV = 16 * NT;
  static constexpr int NB = SWA ? 2 : 1;
  alignas(16) half_t qh[C][QH];          // q, row-major
  alignas(16) half_t kh[NB][C][QH];      // k, row-major
  alignas(16) half_t kt[DK + 1][KT];     // k^T; row ONES = 1
  alignas(16) half_t vh[NB][C][vrow<NT>()];  // v, row-major
  alignas(16) half_t tt[DV + 1][TT];     // scaled state^T; row DV: denominator state
  alignas(16) half_t tl[HI ? DV + 1 : 1][HI ? TT : 8];  // HI: the rounding remainder of tt
  alignas(16) float t0[DV];              // constant row of the state (sum of v)
  alignas(16) float vpart[NTHR];         // partial column sums of v (decayed variant)
  alignas(16) float zf[NF];              // denominator state (set-up and result)
  alignas(16) float wmax[4];             // per-wavefront largest state magnitude
  // decayed variant, fixed for the whole pass: the in-chunk weights
  // gamma^(query - key) of the 16-key tile t tiles before the query's tile,
  // as lane l of a wavefront holds them (query 16 w + l % 16 against keys
  // 16 (w - t) + 4 (l / 16) + i; zero for a key after the query), and the
  // update's key weights gamma^(C - 1 - key) of a whole chunk
  alignas(16) float dw[DEC ? 4 : 1][DEC ? 64 : 1][4];
  alignas(16) half_t wkc[DEC ? C : 8];
  alignas(16) float wvc[DEC ? C : 4];  // the same weights in fp32 (column sums of v)
};

// Wavefront index as a scalar, so that every branch on it is a uniform
// (scalar) branch: a matrix-core instruction under such a branch is skipped,
// never issued with part of EXEC cleared -- the matrix cores ignore EXEC and
// would write their result from whatever the skipped vector code left in the
// operand registers.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Transposing LDS read (ds_read_b64_tr_b16): rows r0 .. r0 + 3 of column
// c0 + (lane % 16) of the row-major fp16 array at `base` (row stride ld).
// Within each 16-lane block lane t receives element t % 4 of the 4-element
// segments addressed by lanes t / 4 + 4i, so lane j points at row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3.  Every lane of a block must take part.
__device__ __forceinline__ uint2 tr4(const half_t* base, int r0, int c0, int ld) {
  const int j = threadIdx.x & 15;
  const half_t* a = base + (r0 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
  return __builtin_bit_cast(uint2, v);
}
// matrix operand with K = rows r0 .. r0 + 7 of column c0 + (lane % 16)
__device__ __forceinline__ f16x8 tr8(const half_t* base, int r0, int c0, int ld) {
  const uint2 a = tr4(base, r0, c0, ld), b = tr4(base, r0 + 4, c0, ld);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// K = rows r0 .. r0 + 3 and r0 + 16 .. r0 + 19 (the same rows of two 16-row tiles)
__device__ __forceinline__ f16x8 tr44(const half_t* base, int r0, int c0, int ld) {
  const uint2 a = tr4(base, r0, c0, ld), b = tr4(base, r0 + 16, c0, ld);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}

__device__ __forceinline__ f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x2 h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Two bf16 packed in a word -> two fp16 packed in a word (exact in fp16's
// normal range).
__device__ __forceinline__ uint32_t h2_from_bf2(uint32_t w) {
  const f32x2 f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return u32(__builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ uint4 h8_from_bf8(const uint4& x) {
  return make_uint4(h2_from_bf2(x.x), h2_from_bf2(x.y), h2_from_bf2(x.z), h2_from_bf2(x.w));
}

// fp16 hi + lo of two fp32 values: hi = RNE(x), lo = RNE(x - hi).  The
// remainders are formed by v_fma_mix{lo,hi}_f16, which take the fp32 value
// and the fp16 half of hi as they are (x * 1 - hi in fp32, rounded once to
// fp16): one instruction per value where the compiler's form (widen hi,
// subtract, narrow) takes three.  x - hi is exact in fp32, so the result is
// the same.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f16x2 h = __builtin_convertvector((f32x2{a, b}), f16x2);
  hi = u32(h);
  uint32_t l = 0;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %3, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "+v"(l)
      : "v"(a), "v"(hi), "v"(b));
  lo = l;
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

// 16-byte loads of the chunk inputs and the segment records, with the
// non-temporal hint (cache policy bit 1): each is read by few workgroups,
// and streaming them leaves the L2 to the rest; 32k layer 147 -> 137-143 us,
// 1.3B 135 -> 133.6 us, 360M unchanged (three A/B pairs on one box)
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// Thread -> (position, 8 columns) of the v loads: consecutive threads take
// consecutive 16-byte pieces of the chunk's rows.  Threads 0..127 load q (k
// again when q is not wanted), threads 128..255 load k, 8 elements each:
// every wavefront issues the same loads, so the compiler can count the loads
// in flight exactly and a deeper prefetch is not drained early.
template <int NT, int DVS = 16 * NT>
__device__ __forceinline__ void load_chunk(const HeadRsrc& r, int t0, bool q_too, Prefetch<NT>& pf, int col0 = 0) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x;
  {
    const int u = tid & 127, j = u >> 1, h = u & 1;
    const int off = ((t0 + j) * DK + 8 * h) * 2;
    pf.qk = bload(wave_index() < 2 && q_too ? r.q : r.k, off);
  }
#pragma unroll
  for (int i = 0; i < Prefetch<NT>::NV; ++i) {
    const int u = tid + NTHR * i;
    const int j = u / (DV / 8), c8 = u % (DV / 8);
    pf.v[i] = bload(r.v, ((t0 + j) * DVS + col0 + 8 * c8) * 2);
  }
}

// One chunk from the prefetch registers into LDS as fp16: k^T and the
// row-major v, and (when given) the row-major copies of q and k.
template <int NT>
__device__ __forceinline__ void store_chunk(half_t (*kt)[KT], half_t* vh, half_t (*qh)[QH], half_t (*kh)[QH],
                                            const Prefetch<NT>& pf) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x;
  const int u = tid & 127, j = u >> 1, h = u & 1;
  if (tid >= 128) {
    const uint4 k8 = h8_from_bf8(pf.qk);
    if (kh) *reinterpret_cast<uint4*>(&kh[j][8 * h]) = k8;
    const f16x8 e = __builtin_bit_cast(f16x8, k8);
#pragma unroll
    for (int i = 0; i < 8; ++i) kt[8 * h + i][j] = e[i];
  } else if (qh) {
    *reinterpret_cast<uint4*>(&qh[j][8 * h]) = h8_from_bf8(pf.qk);
  }
#pragma unroll
  for (int i = 0; i < Prefetch<NT>::NV; ++i) {
    const int uu = tid + NTHR * i;
    const int jj = uu / (DV / 8), c8 = uu % (DV / 8);
    *reinterpret_cast<uint4*>(vh + jj * vrow<NT>() + 8 * c8) = h8_from_bf8(pf.v[i]);
  }
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

__device__ __forceinline__ f16x8 ones8() {
  const uint32_t one2 = 0x3c003c00u;  // fp16 1.0 twice
  return __builtin_bit_cast(f16x8, make_uint4(one2, one2, one2, one2));
}

// State update of one chunk: tacc += psi'(K)^T V over the chunk, and the
// denominator state of the owned feature tiles, tz[slot] += psi'(K)^T 1
// (every column of a tz tile holds it).
//
// VS: the wavefront with `vs_mine` also adds the chunk's column sums of v to
// vsum (an all-ones A operand -- the key weights in the decayed variant --
// against the v fragments the update loads anyway; every row of a vsum tile
// holds the sums of its 16 columns).
template <int NT, int DEC = 0, int FREE = 0, int VS = 0>
__device__ __forceinline__ void update_chunk(const half_t (*kt)[KT], const half_t* vh,
                                             f32x4 (&tacc)[Own<NT>::PPW], f32x4 (&tz)[3], const int (&ia)[3],
                                             const int (&ib)[3], const f16x8* wk = nullptr,
                                             f32x4* vsum = nullptr, bool vs_mine = false) {
  constexpr int H = NT / 2;
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const bool upper = (w & 1) != 0;  // slot 2 holds the upper half of the column tiles
  const f16x8 ones = ones8();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    f16x8 a[3];
#pragma unroll
    for (int ms = 0; ms < 3; ++ms) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(&kt[ia[ms]][32 * ks + 8 * g]);
      const f16x8 y = *reinterpret_cast<const f16x8*>(&kt[ib[ms]][32 * ks + 8 * g]);
      a[ms] = x * y;
      if constexpr (DEC) a[ms] *= wk[ks];  // decayed variant: each key's weight
    }
    f16x8 bv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) bv[n] = tr8(vh, 32 * ks + 8 * g, 16 * n, vrow<NT>());
#pragma unroll
    for (int n = 0; n < NT; ++n) tacc[n] = mfma(a[0], bv[n], tacc[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) tacc[NT + n] = mfma(a[1], bv[n], tacc[NT + n]);
    if (upper) {  // uniform branch (scalar wavefront index)
#pragma unroll
      for (int n = 0; n < H; ++n) tacc[2 * NT + n] = mfma(a[2], bv[H + n], tacc[2 * NT + n]);
    } else {
#pragma unroll
      for (int n = 0; n < H; ++n) tacc[2 * NT + n] = mfma(a[2], bv[n], tacc[2 * NT + n]);
    }
    tz[0] = mfma(a[0], ones, tz[0]);
    tz[1] = mfma(a[1], ones, tz[1]);
    if ((w & 1) == 0) tz[2] = mfma(a[2], ones, tz[2]);  // z of tile 8 + w/2 kept once
    if constexpr (VS) {
      if (vs_mine)  // uniform branch; decayed variant: each key's weight
#pragma unroll
        for (int n = 0; n < NT; ++n) vsum[n] = mfma(DEC ? wk[ks] : ones, bv[n], vsum[n]);
    }
    // keep the operands of the two K-steps from being live at once (FREE:
    // the caller has the registers to let the scheduler overlap them)
    if constexpr (!FREE) __builtin_amdgcn_sched_barrier(0);
  }
}

// Decayed main pass: this thread's share of the weighted column sums of the
// chunk's v (row-major in LDS), row t weighing gamma^(n-1-t) and rows past n
// none: column tid % DV, rows part * SPAN .. + SPAN - 1 with part = tid / DV,
// read four rows at a time with the transposing load (a 16-lane block covers
// 16 consecutive columns of one part).  A whole chunk takes its weights from
// the pass's table wvc[t] = gamma^(C-1-t).  (Elsewhere the update forms the
// column sums with the matrix cores.)
template <int NT>
__device__ __forceinline__ float vsum_part_decayed(const half_t* vh, int n, float lg, const float* wvc) {
  constexpr int DV = 16 * NT;
  constexpr int PARTS = NTHR / DV >= 1 ? NTHR / DV : 1, SPAN = C / PARTS;
  const int tid = threadIdx.x, col = tid % DV, part = tid / DV;
  float vs = 0.f;
  if (part < PARTS && n == C) {
#pragma unroll
    for (int j = 0; j < SPAN; j += 4) {
      const f16x4 x = __builtin_bit_cast(f16x4, tr4(vh, part * SPAN + j, col & ~15, vrow<NT>()));
      const float4 wv = *reinterpret_cast<const float4*>(&wvc[part * SPAN + j]);
      vs = __builtin_fmaf((float)x[0], wv.x, vs);
      vs = __builtin_fmaf((float)x[1], wv.y, vs);
      vs = __builtin_fmaf((float)x[2], wv.z, vs);
      vs = __builtin_fmaf((float)x[3], wv.w, vs);
    }
  } else if (part < PARTS) {  // whole wavefronts (DV divides 64 or is a multiple of 32)
    // a ragged chunk: the weight of row t from its own power (rows past n
    // are masked, whatever their weight)
#pragma unroll
    for (int j = 0; j < SPAN; j += 4) {
      const f16x4 x = __builtin_bit_cast(f16x4, tr4(vh, part * SPAN + j, col & ~15, vrow<NT>()));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = part * SPAN + j + e;
        vs = __builtin_fmaf((float)x[e], t < n ? gpow(lg, (float)(n - 1 - t)) : 0.f, vs);
      }
    }
  }
  return vs;
}

// DPP move of a lane value (row_mask / bank_mask all, out-of-row sources read 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Maximum over the four 16-lane rows of a wavefront (lanes l, l^16,
// l^32, l^48), by row swaps in registers: v_permlane16_swap pairs rows 0-1
// and 2-3, v_permlane32_swap the two halves.  Every lane applies the same
// operand order, so all four get the same bits.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Largest magnitude of this wavefront's state entries, into wmax[w]: quad and
// row reductions in DPP, then the four row results through scalar registers
// (non-negative floats order like their bit patterns).
template <int NT>
__device__ __forceinline__ void post_max(float* wmax, const f32x4 (&tacc)[Own<NT>::PPW], const f32x4 (&tz)[3]) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(tacc[j][i]));
#pragma unroll
  for (int ms = 0; ms < 3; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(tz[ms][i]));
  m = fmaxf(m, dpp<0xb1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp<0x4e>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp<0x114>(m));  // row_shr:4
  m = fmaxf(m, dpp<0x118>(m));  // row_shr:8 -> lane 15 of each row holds the row maximum
  const int b = __float_as_int(m);
  const uint32_t r0 = __builtin_amdgcn_readlane(b, 15), r1 = __builtin_amdgcn_readlane(b, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(b, 47), r3 = __builtin_amdgcn_readlane(b, 63);
  const uint32_t mx = max(max(r0, r1), max(r2, r3));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = __uint_as_float(mx);
}

// Power-of-two scale of the published state from the block's largest entry
// M (wmax, after a barrier).  No scale (e = 0) while M is in [2^-4, 2^14):
// entries then stay below fp16's largest value and those that fall below its
// normal range are negligible next to M.  Otherwise entries times 2^-e stay
// below 2^(SCALE_TOP + 1).  Returns e; down = 2^-e, up = 2^e.
__device__ __forceinline__ int state_scale(const float* wmax, float& down, float& up) {
  const uint4 mm = *reinterpret_cast<const uint4*>(wmax);
  const uint32_t mb = max(max(mm.x, mm.y), max(mm.z, mm.w));  // non-negative: order as integers
  const int E = (int)((mb >> 23) & 0xffu) - 127;                 // floor(log2 M) (-127: zero)
  int e = (E >= -4 && E < 14) ? 0 : E - SCALE_TOP;
  e = e < -126 ? -126 : e;
  down = __uint_as_float((uint32_t)(127 - e) << 23);
  up = __uint_as_float((uint32_t)(127 + e) << 23);
  return e;
}

// fp16 hi + lo of four fp32 values: hi = RNE(x), lo = RNE(x - hi).
__device__ __forceinline__ f16x4 split4(const f32x4& x, f16x4& lo) {
  const f16x4 hi = __builtin_convertvector(x, f16x4);
  lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), f16x4);
  return hi;
}

// High-precision readout (HI): the owned state tiles times `down` as fp16
// hi into tt and lo into tl.
template <int NT>
__device__ __forceinline__ void publish_state_hilo(half_t (*tt)[TT], half_t (*tl)[TT],
                                                   const f32x4 (&tacc)[Own<NT>::PPW], const f32x4 (&tz)[3],
                                                   float down) {
  constexpr int DV = 16 * NT;
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j) {
    int m, n;
    pair_mn<NT>(w, j, m, n);
    f16x4 lo;
    *reinterpret_cast<f16x4*>(&tt[16 * n + r16][16 * m + 4 * g]) = split4(tacc[j] * down, lo);
    *reinterpret_cast<f16x4*>(&tl[16 * n + r16][16 * m + 4 * g]) = lo;
  }
  if (r16 == 0)
#pragma unroll
    for (int ms = 0; ms < 3; ++ms)
      if (ms < 2 || (w & 1) == 0) {
        f16x4 lo;
        *reinterpret_cast<f16x4*>(&tt[DV][16 * mt[ms] + 4 * g]) = split4(tz[ms] * down, lo);
        *reinterpret_cast<f16x4*>(&tl[DV][16 * mt[ms] + 4 * g]) = lo;
      }
}

// Write the owned state tiles (and the denominator state) into tt as fp16,
// times `down` unless e = 0 (the caller has synchronised: nobody reads tt
// meanwhile).
template <int NT>
__device__ __forceinline__ void publish_state(half_t (*tt)[TT], const f32x4 (&tacc)[Own<NT>::PPW],
                                              const f32x4 (&tz)[3], int e, float down) {
  constexpr int DV = 16 * NT;
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
  if (e == 0) {
#pragma unroll
    for (int j = 0; j < Own<NT>::PPW; ++j) {
      int m, n;
      pair_mn<NT>(w, j, m, n);
      *reinterpret_cast<f16x4*>(&tt[16 * n + r16][16 * m + 4 * g]) = __builtin_convertvector(tacc[j], f16x4);
    }
    if (r16 == 0)
#pragma unroll
      for (int ms = 0; ms < 3; ++ms)
        if (ms < 2 || (w & 1) == 0)
          *reinterpret_cast<f16x4*>(&tt[DV][16 * mt[ms] + 4 * g]) = __builtin_convertvector(tz[ms], f16x4);
  } else {
#pragma unroll
    for (int j = 0; j < Own<NT>::PPW; ++j) {
      int m, n;
      pair_mn<NT>(w, j, m, n);
      *reinterpret_cast<f16x4*>(&tt[16 * n + r16][16 * m + 4 * g]) = __builtin_convertvector(tacc[j] * down, f16x4);
    }
    if (r16 == 0)
#pragma unroll
      for (int ms = 0; ms < 3; ++ms)
        if (ms < 2 || (w & 1) == 0)
          *reinterpret_cast<f16x4*>(&tt[DV][16 * mt[ms] + 4 * g]) = __builtin_convertvector(tz[ms] * down, f16x4);
  }
}

// The denominator state of the owned feature tiles back into zf.
template <int NT>
__device__ __forceinline__ void store_z(float* zf, const f32x4 (&tz)[3]) {
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  if (r16 != 0) return;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
  for (int ms = 0; ms < 3; ++ms)
    if (ms < 2 || (w & 1) == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) zf[16 * mt[ms] + 4 * g + i] = tz[ms][i];
}

// Initial owned state tiles from the caller's phi-layout S_in, else zero
// (one uniform branch around the whole tile loop).
template <int NT>
__device__ __forceinline__ void init_state(const float* Sin, f32x4 (&tacc)[Own<NT>::PPW], int col0 = 0,
                                           int ld = 16 * NT) {
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  if (Sin) {
#pragma unroll
    for (int j = 0; j < Own<NT>::PPW; ++j) {
      int m, n;
      pair_mn<NT>(w, j, m, n);
#pragma unroll
      for (int i = 0; i < 4; ++i) tacc[j][i] = compact_from_phi(Sin, 16 * m + 4 * g + i, col0 + 16 * n + r16, ld);
    }
  } else {
#pragma unroll
    for (int j = 0; j < Own<NT>::PPW; ++j) tacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

__device__ __forceinline__ float bload_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// Initial state of a segment from the compact records of earlier segments
// (record_offset layout, consecutive, (NF + 1) * DV floats apart; their z
// parts (NF + 1) floats apart): the sum of records 0..n-1 from `first`, record
// k weighted by wts[k], n <= MAX_SUM.  Owned tiles into tacc, the constant row
// into t0, the z entries into zf / z0.  Every read goes through a buffer
// resource that spans exactly the n records, so all MAX_SUM reads of each
// entry are issued unconditionally (those past the n-th record return zero
// without touching memory): no branch lies between them and the compiler
// keeps them in flight together.  wts[k] must be finite for every k.
template <int NT>
__device__ __forceinline__ void sum_records(const float* first, const float* firstz, int n, const float (&wts)[MAX_SUM],
                                            f32x4 (&tacc)[Own<NT>::PPW], float* t0, float* zf, float& z0) {
  constexpr int DV = 16 * NT;
  constexpr int REC = (NF + 1) * DV;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const __amdgpu_buffer_rsrc_t rr =
      __builtin_amdgcn_make_buffer_rsrc((void*)first, (short)0, n * REC * (int)sizeof(float), RSRC_DW3);
  const __amdgpu_buffer_rsrc_t rz =
      __builtin_amdgcn_make_buffer_rsrc((void*)firstz, (short)0, n * (NF + 1) * (int)sizeof(float), RSRC_DW3);
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j) {
    int m, nn;
    pair_mn<NT>(w, j, m, nn);
    const int off = (int)record_offset(16 * m + 4 * g, 16 * nn + r16, DV) * (int)sizeof(float);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < MAX_SUM; ++k) {
      const uint4 x = bload(rr, off + k * REC * (int)sizeof(float));
      sum += __builtin_bit_cast(f32x4, x) * wts[k];
    }
    tacc[j] = sum;
  }
  for (int c = tid; c < DV; c += NTHR) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < MAX_SUM; ++k) sum += wts[k] * bload_f32(rr, (k * REC + NF * DV + c) * (int)sizeof(float));
    t0[c] = sum;
  }
  for (int r = tid; r < NF; r += NTHR) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < MAX_SUM; ++k) sum += wts[k] * bload_f32(rz, (k * (NF + 1) + r) * (int)sizeof(float));
    zf[r] = sum;
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < MAX_SUM; ++k) sum += wts[k] * bload_f32(rz, (k * (NF + 1) + NF) * (int)sizeof(float));
  z0 = sum;
}

// Denominator state of the owned feature tiles from zf (every column).
__device__ __forceinline__ void load_tz(const float* zf, f32x4 (&tz)[3]) {
  const int lane = threadIdx.x & 63, w = wave_index(), g = lane >> 4;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
  for (int ms = 0; ms < 3; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) tz[ms][i] = zf[16 * mt[ms] + 4 * g + i];
}

// Loop-invariant per-lane data of the owned feature tiles: the k^T rows
// whose product is the key feature of the lane's slot (update operand rows).
__device__ __forceinline__ void slot_rows(int (&ia)[3], int (&ib)[3]) {
  const int lane = threadIdx.x & 63, w = wave_index(), r16 = lane & 15;
  const int mt[3] = {w, w + 4, 8 + (w >> 1)};
#pragma unroll
  for (int mm = 0; mm < 3; ++mm) {
    const int r = 16 * mt[mm] + r16;
    const int ty = c_tab.type[r];
    ia[mm] = c_tab.a[r];
    ib[mm] = ty == LIN ? ONES : (ty == DIAG ? ia[mm] : c_tab.b[r]);
  }
}

template <int NT, int CS = 1>
__device__ __forceinline__ void write_compact(const float* t0, const float* zf, const f32x4 (&tacc)[Own<NT>::PPW],
                                              float z0, float* dst, float* dz, int col0 = 0) {
  constexpr int DV = 16 * NT, DVF = DV * CS;
  const int tid = threadIdx.x, w = wave_index(), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j) {
    int m, nn;
    pair_mn<NT>(w, j, m, nn);
    *reinterpret_cast<float4*>(dst + record_offset(16 * m + 4 * g, col0 + 16 * nn + r16, DVF)) =
        make_float4(tacc[j][0], tacc[j][1], tacc[j][2], tacc[j][3]);
  }
  for (int c = tid; c < DV; c += NTHR) dst[(size_t)NF * DVF + col0 + c] = t0[c];
  if (col0 == 0) {
    for (int r = tid; r < NF; r += NTHR) dz[r] = zf[r];
    if (tid == 0) dz[NF] = z0;
  }
}

// Record 0 of a head: the caller's initial state in the compact record
// layout (owned tiles from s0 = init_state of Sin; the constant row and the
// z entries straight from Sin / zin).
template <int NT, int CS = 1>
__device__ __forceinline__ void write_initial_record(const float* Sin, const float* zin,
                                                     const f32x4 (&s0)[Own<NT>::PPW], float* dst, float* dz,
                                                     int col0 = 0) {
  constexpr int DV = 16 * NT, DVF = DV * CS;
  const int tid = threadIdx.x, w = wave_index(), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j) {
    int m, nn;
    pair_mn<NT>(w, j, m, nn);
    *reinterpret_cast<float4*>(dst + record_offset(16 * m + 4 * g, col0 + 16 * nn + r16, DVF)) =
        make_float4(s0[j][0], s0[j][1], s0[j][2], s0[j][3]);
  }
  for (int c = tid; c < DV; c += NTHR) dst[(size_t)NF * DVF + col0 + c] = Sin[col0 + c];
  if (col0 == 0 && zin) {
    for (int r = tid; r < NF; r += NTHR) dz[r] = compact_from_phi(zin, r, 0, 1);
    if (tid == 0) dz[NF] = zin[0];
  }
}

// The final state in the caller's 273-row phi layout, straight from the
// accumulator registers: slot r of a pair (a, b) writes rows (a, b) and
// (b, a) when it is the slot that represents that pair.
template <int NT>
__device__ __forceinline__ void write_phi_state(const float* t0, const float* zf, const f32x4 (&tacc)[Own<NT>::PPW],
                                                float z0, float* So, float* zo) {
  constexpr int DV = 16 * NT;
  const int tid = threadIdx.x, w = wave_index(), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < Own<NT>::PPW; ++j) {
    int m, nn;
    pair_mn<NT>(w, j, m, nn);
    const int c = 16 * nn + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g + i;
      const int a = c_tab.a[r], b = c_tab.b[r], ty = c_tab.type[r];
      if (ty == LIN) {
        So[(size_t)(1 + a) * DV + c] = tacc[j][i];
      } else {
        const int f1 = 1 + DK + DK * a + b, f2 = 1 + DK + DK * b + a;
        if (c_tab.phi_slot[f1] == r) {
          const float val = tacc[j][i] * INV_SQRT2;
          So[(size_t)f1 * DV + c] = val;
          if (f2 != f1) So[(size_t)f2 * DV + c] = val;
        }
      }
    }
  }
  for (int c = tid; c < DV; c += NTHR) So[c] = t0[c];
  for (int f = tid; f < DPHI; f += NTHR) {
    const int r = c_tab.phi_slot[f];
    zo[f] = r < 0 ? z0 : (c_tab.type[r] == LIN ? zf[r] : zf[r] * INV_SQRT2);
  }
}

// Two wavefronts per SIMD (two workgroups per CU) where the register budget
// allows it (d_v <= 64), one otherwise.
template <int NT> struct Occ { static constexpr int value = NT <= 4 ? 2 : 1; };

// Four outputs of a position.  The one-workgroup-per-CU kernels (d_v 96,
// 128) store them non-temporally (straight to memory, not kept in L2): the
// 1.3B-shaped layer 143 -> 137 us; the two-per-CU kernels keep plain stores
// (non-temporal ones made the 360M layer 3.5 us and the 32k layer 9 us
// slower).
template <int NT>
__device__ __forceinline__ void store_y(float* dst, const f32x4& v) {
  if constexpr (Occ<NT>::value == 1) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
  else *reinterpret_cast<f32x4*>(dst) = v;
}

// SWA: 0 = linear attention only; 1 = with the window attention, window 64;
// 2 = with the window attention, any window.
// HI: high-precision readout for an arbitrary initial state -- the query
// features and the state copy both as fp16 hi + lo, three passes (hi hi,
// hi lo, lo hi).  A state the recurrence builds is read out accurately by
// the single pass; one supplied by the caller may cancel over its 272
// feature rows, where the single rounding of either operand is too coarse.
template <int NT, int SWA, int DEC = 0, int HI = 0>
__global__ __launch_bounds__(NTHR, Occ<NT>::value) void linattn_mfma_kernel(Params p) {
  constexpr int DV = 16 * NT;
  constexpr int PARTS = NTHR / DV >= 1 ? NTHR / DV : 1, SPAN = C / PARTS;
  __shared__ Smem<NT, SWA, HI, DEC> S;

  // the segments of one (batch, head) share an XCD: the later segments read
  // the same records of the earlier ones, through that XCD's L2
  int bhi, seg;
  xcd_unit_part(blockIdx.x, gridDim.x / p.nseg, p.nseg, bhi, seg);
  const size_t bh = bhi;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int tok_begin = seg * p.seg_chunks * C;
  const int tok_end = min(p.L, tok_begin + p.seg_chunks * C);

  // ---- initial state.  One segment: the caller's S_in / z_in (or zero),
  // read by this workgroup before it writes S_out.  Several segments:
  // segment 0 starts from record 0, the state-only pass's copy of S_in (or
  // from zero), so that no workgroup of this pass reads S_in and the last
  // segment may write S_out over it; segment s > 0, with at most MAX_SUM + 1
  // segments, from the sum of records 1..s (record 1 holds S_in plus
  // segment 0's increment, record j > 1 segment j-1's increment); with more,
  // the scan has turned record s into the state at the segment's start.
  const size_t rec = (size_t)(NF + 1) * DV;
  const bool scanned = p.nseg > MAX_SUM + 1;
  const bool rec0 = p.nseg > 1 && seg == 0 && p.S_in != nullptr;
  const bool from_records = (p.nseg > 1 && seg > 0) || rec0;
  const int first = rec0 ? 0 : (scanned ? seg : 1), nsrc = rec0 ? 1 : (scanned ? 1 : seg);
  // the segment's first chunk (and, with the window, the chunk before it)
  // from HBM first, so that their latency overlaps the state set-up
  const HeadRsrc rs = head_rsrc(p, bh, DV);
  Prefetch<NT> pf, pp;
  if (SWA && tok_begin > 0) load_chunk<NT>(rs, tok_begin - C, false, pp);
  if (tok_begin < tok_end) load_chunk<NT>(rs, tok_begin, true, pf);
  // decayed variant: record 1 + k (k < seg, no scan) holds segment k's share
  // at its end, which lies seg_chunks * C * (seg - 1 - k) positions before
  // this segment's start; weights of absent records stay finite (their reads
  // return zero)
  float lg = 0.f;
  float wrec[MAX_SUM];
#pragma unroll
  for (int k2 = 0; k2 < MAX_SUM; ++k2) wrec[k2] = 1.f;
  if constexpr (DEC) {
    lg = decay_lg2(p, bh);
    if (!scanned && !rec0)
#pragma unroll
      for (int k2 = 0; k2 < MAX_SUM; ++k2)
        wrec[k2] = k2 < nsrc ? gpow(lg, (float)((seg - 1 - k2) * p.seg_chunks * C)) : 0.f;
  }
  // a whole chunk decays the carried state by gnC and adds gsC to its
  // constant denominator entry
  float gnC = 1.f, gsC = (float)C;
  if constexpr (DEC) {
    gnC = uniform(gpow(lg, (float)C));
    gsC = uniform(gsum_pow(lg, C));
    for (int j = tid; j < 4 * 64; j += NTHR) {
      const int t = j >> 6, l = j & 63, d0 = 16 * t + (l & 15) - 4 * (l >> 4);
      float4 wv;
      wv.x = d0 >= 0 ? gpow(lg, (float)d0) : 0.f;
      wv.y = d0 >= 1 ? gpow(lg, (float)(d0 - 1)) : 0.f;
      wv.z = d0 >= 2 ? gpow(lg, (float)(d0 - 2)) : 0.f;
      wv.w = d0 >= 3 ? gpow(lg, (float)(d0 - 3)) : 0.f;
      *reinterpret_cast<float4*>(&S.dw[t][l][0]) = wv;
    }
    for (int j = tid; j < C; j += NTHR) {
      S.wvc[j] = gpow(lg, (float)(C - 1 - j));
      S.wkc[j] = (half_t)S.wvc[j];
    }
  }
  f32x4 tacc[Own<NT>::PPW];
  float z0 = 0.f;
  if (from_records) {
    sum_records<NT>(p.ws + (bh * p.nseg + first) * rec, p.wsz + (bh * p.nseg + first) * (size_t)(NF + 1), nsrc,
                    wrec, tacc, S.t0, S.zf, z0);
  } else {
    const bool own_sin = p.nseg == 1 && p.S_in != nullptr;
    const float* Sin = own_sin ? p.S_in + bh * DPHI * DV : nullptr;
    const float* zin = own_sin ? p.z_in + bh * DPHI : nullptr;
    init_state<NT>(Sin, tacc);
    for (int c = tid; c < DV; c += NTHR) S.t0[c] = Sin ? Sin[c] : 0.f;
    for (int r = tid; r < NF; r += NTHR) S.zf[r] = zin ? compact_from_phi(zin, r, 0, 1) : 0.f;
    z0 = zin ? zin[0] : 0.f;
  }
  for (int j = tid; j < KT; j += NTHR) S.kt[ONES][j] = (half_t)1.f;
  int ia[3], ib[3];
  slot_rows(ia, ib);
  if constexpr (SWA) {
    // the window of the segment's first chunk reaches into the chunk before
    if (tok_begin > 0) {
      store_chunk<NT>(S.kt, &S.vh[1][0][0], nullptr, S.kh[1], pp);
    } else {
      for (int j = tid; j < C * QH / 2; j += NTHR) reinterpret_cast<uint32_t*>(&S.kh[1][0][0])[j] = 0u;
      for (int j = tid; j < C * vrow<NT>() / 2; j += NTHR) reinterpret_cast<uint32_t*>(&S.vh[1][0][0])[j] = 0u;
    }
  }
  __syncthreads();
  f32x4 tz[3];  // denominator state of the owned feature tiles
  load_tz(S.zf, tz);
  post_max<NT>(S.wmax, tacc, tz);
  __syncthreads();
  float down, up;
  int e = state_scale(S.wmax, down, up);
  if constexpr (HI) publish_state_hilo<NT>(S.tt, S.tl, tacc, tz, down);
  else publish_state<NT>(S.tt, tacc, tz, e, down);
  if (tok_begin < tok_end) store_chunk<NT>(S.kt, &S.vh[0][0][0], S.qh, S.kh[0], pf);
  int cur = 0;  // buffer of the current chunk's k and v (the other: previous chunk)

  const f16x8 ones = ones8();
  const int pos = 16 * w + r16;  // the chunk position whose outputs this lane holds
  // Diagonal tile masks (key 4g + i against query r16 of the same 16-tile),
  // kept as floats so they stay in vector registers: a weight factor for the
  // linear attention and additive 0 / -inf masks for the window's current and
  // previous-chunk diagonal tiles (the window-64 case).
  float dkeep[4], dcur[4], dprev[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool after = 4 * g + i > r16;
    dkeep[i] = after ? 0.f : 1.f;
    dcur[i] = after ? -INFINITY : 0.f;
    dprev[i] = after ? 0.f : -INFINITY;
  }
  f32x4 vacc[NT];  // wavefront 0: the chunk's column sums of v
  for (int t0 = tok_begin; t0 < tok_end; t0 += C) {
    if constexpr (Occ<NT>::value > 1) progress_priority(t0 - tok_begin, tok_end - tok_begin);
    const int n = min(C, tok_end - t0);
    __syncthreads();  // chunk inputs, published state, t0 visible
    const int tn = t0 + C;
    if (tn < tok_end) load_chunk<NT>(rs, tn, true, pf);

    // ---- constant row of the state: column sums of v over the chunk (the
    // decayed variant here, in PARTS partial sums per column; otherwise
    // wavefront 0 forms them in the update below)
    if constexpr (DEC) S.vpart[tid] = vsum_part_decayed<NT>(&S.vh[cur][0][0], n, lg, S.wvc);

    // ---- readout of the state before the chunk, transposed (value columns x
    // positions): acc[nn][i] is column 16nn + 4g + i of position `pos`; every
    // entry of accz is the denominator of `pos`
    f32x4 acc[NT];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 accz = {0.f, 0.f, 0.f, 0.f};
    {
      uint32_t q2[8];  // q of this position as fp16 pairs, rotated by 4g coordinates
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const uint2 x = *reinterpret_cast<const uint2*>(&S.qh[pos][4 * ((pc + g) & 3)]);
        q2[2 * pc] = x.x;
        q2[2 * pc + 1] = x.y;
      }
      uint32_t qo[5];  // odd pairs: (q[2j+1], q[2j+2])
#pragma unroll
      for (int j = 0; j < 5; ++j) qo[j] = (uint32_t)((((uint64_t)q2[j + 1] << 32) | q2[j]) >> 16);
      // query weight 1/2 of the square and {a, a+8} slots on the first factor
      const f16x2 half2 = {(half_t)0.5f, (half_t)0.5f};
      const uint32_t qh0 = u32(h2(q2[0]) * half2), qh1 = u32(h2(q2[1]) * half2);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        uint4 fw;
        if (kb == 0) {
          fw = make_uint4(q2[0], q2[1], u32(h2(qh0) * h2(q2[0])), u32(h2(qh1) * h2(q2[1])));
        } else {
          fw = make_uint4(u32(h2(q2[0]) * h2(qo[kb - 1])), u32(h2(q2[1]) * h2(qo[kb])),
                          u32(h2(kb == NKB - 1 ? qh0 : q2[0]) * h2(q2[kb])),
                          u32(h2(kb == NKB - 1 ? qh1 : q2[1]) * h2(q2[kb + 1])));
        }
        const f16x8 fb = __builtin_bit_cast(f16x8, fw);
        accz = mfma(*reinterpret_cast<const f16x8*>(&S.tt[DV][32 * kb + 8 * g]), fb, accz);
#pragma unroll
        for (int nn = 0; nn < NT; ++nn)
          acc[nn] = mfma(*reinterpret_cast<const f16x8*>(&S.tt[16 * nn + r16][32 * kb + 8 * g]), fb, acc[nn]);
        if constexpr (HI) {
          // the features' rounding remainders (exact fp32 products of the
          // fp16 factors, minus the fp16 features; linear features: zero)
          uint4 fx, fy;
          if (kb == 0) {
            fx = make_uint4(0u, 0u, q2[0], q2[1]);
            fy = make_uint4(0u, 0u, qh0, qh1);
          } else {
            fx = make_uint4(q2[0], q2[1], kb == NKB - 1 ? qh0 : q2[0], kb == NKB - 1 ? qh1 : q2[1]);
            fy = make_uint4(qo[kb - 1], qo[kb], q2[kb], q2[kb + 1]);
          }
          const f16x8 hx = __builtin_bit_cast(f16x8, fx), hy = __builtin_bit_cast(f16x8, fy);
          f16x8 fl;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float prod = (float)hx[i] * (float)hy[i];
            fl[i] = (half_t)(prod - (float)fb[i]);
          }
          if (kb == 0) { fl[0] = fl[1] = fl[2] = fl[3] = (half_t)0.f; }
          accz = mfma(*reinterpret_cast<const f16x8*>(&S.tl[DV][32 * kb + 8 * g]), fb, accz);
          accz = mfma(*reinterpret_cast<const f16x8*>(&S.tt[DV][32 * kb + 8 * g]), fl, accz);
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            acc[nn] = mfma(*reinterpret_cast<const f16x8*>(&S.tl[16 * nn + r16][32 * kb + 8 * g]), fb, acc[nn]);
            acc[nn] = mfma(*reinterpret_cast<const f16x8*>(&S.tt[16 * nn + r16][32 * kb + 8 * g]), fl, acc[nn]);
          }
        }
      }
    }
    if (e != 0) {
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) acc[nn] *= up;
      accz *= up;
    }
    // decayed variant: the state before the chunk reaches position pos
    // decayed by gamma^(pos + 1)
    const float cf = DEC ? gpow(lg, (float)(pos + 1)) : 1.f;
    if constexpr (DEC) {
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) acc[nn] *= cf;
      accz *= cf;
    }

    // ---- in-chunk causal term: X^T = K Q^T on the keys 0 .. 16w+15, then
    // Y^T += V^T P^T with the weights P = 1 + x + x^2/2 split into fp16 hi + lo
    const f16x8 zero8 = {};
    const f16x8 qv = g < 2 ? *reinterpret_cast<const f16x8*>(&S.qh[pos][8 * g]) : zero8;
    f32x4 xc[4];  // scores against the chunk's key tiles m <= w: key 16m + 4g + i, query `pos`
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      xc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m <= w) {
        const f16x8 kv = g < 2 ? *reinterpret_cast<const f16x8*>(&S.kh[cur][16 * m + r16][8 * g]) : zero8;
        xc[m] = mfma(kv, qv, xc[m]);
      }
    }
    {
      uint4 ah[2], al[2];  // fp16 hi / lo weights of key blocks (tiles 2kb, 2kb + 1)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ah[kb] = al[kb] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m <= w) {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = __builtin_fmaf(xc[m][i], __builtin_fmaf(xc[m][i], 0.5f, 1.f), 1.f);
          if constexpr (DEC) {  // gamma^(query - key), zero for a key after the query
            const float4 dv4 = *reinterpret_cast<const float4*>(&S.dw[w - m][lane][0]);
            a[0] *= dv4.x;
            a[1] *= dv4.y;
            a[2] *= dv4.z;
            a[3] *= dv4.w;
          } else if (m == w) {  // key after query
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] *= dkeep[i];
          }
          uint32_t h0, l0, h1, l1;
          split2(a[0], a[1], h0, l0);
          split2(a[2], a[3], h1, l1);
          if (m & 1) { ah[m >> 1].z = h0; ah[m >> 1].w = h1; al[m >> 1].z = l0; al[m >> 1].w = l1; }
          else { ah[m >> 1].x = h0; ah[m >> 1].y = h1; al[m >> 1].x = l0; al[m >> 1].y = l1; }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb <= w) {
          const f16x8 ph = __builtin_bit_cast(f16x8, ah[kb]);
          const f16x8 pl = __builtin_bit_cast(f16x8, al[kb]);
          accz = mfma(ones, ph, accz);
          accz = mfma(ones, pl, accz);
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const int col = 16 * nn + r16;
            const f16x8 va = tr44(&S.vh[cur][0][0], 32 * kb + 4 * g, 16 * nn, vrow<NT>());
            acc[nn] = mfma(va, ph, acc[nn]);
            acc[nn] = mfma(va, pl, acc[nn]);
          }
        }
      }
    }

    // ---- normalise and store.  The next chunk's loads were issued before
    // these stores, so waiting for them never waits for the stores (vector
    // memory operations complete in order).
    {
      const float rden = __builtin_amdgcn_rcpf(cf * z0 + accz[0]);
      if (pos < n) {
        float* yrow = p.y + (bh * p.L + t0 + pos) * DV + 4 * g;
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) {
          const float4 c0 = *reinterpret_cast<const float4*>(&S.t0[16 * nn + 4 * g]);
          store_y<NT>(yrow + 16 * nn, f32x4{(acc[nn][0] + cf * c0.x) * rden, (acc[nn][1] + cf * c0.y) * rden,
                                            (acc[nn][2] + cf * c0.z) * rden, (acc[nn][3] + cf * c0.w) * rden});
        }
      }
    }

    // ---- sliding-window softmax of the same q, k, v (fused layer pass): the
    // keys of query `pos` are the chunk's tiles m <= w (scores xc) and the
    // previous chunk's tiles m >= w; 5 tiles and 3 key blocks per wavefront
    if constexpr (SWA) {
      const int prev = cur ^ 1;
      f32x4 xp[4];  // scores against the previous chunk's key tiles m >= w
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        xp[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m >= w) {
          const f16x8 kv = g < 2 ? *reinterpret_cast<const f16x8*>(&S.kh[prev][16 * m + r16][8 * g]) : zero8;
          xp[m] = mfma(kv, qv, xp[m]);
        }
      }
      // Scores in the base-2 domain, s = scale * log2(e) * x, so that the
      // weights are exp2(s - max); keys outside the window get s = -inf and
      // weight 0.  Key 4g + i of tile m lies rel = 16(m - w) + 4g + i - r16
      // positions from the query in this chunk (rel - 64 in the previous
      // one); it is in the window when -window < rel <= 0 and it exists.
      // With the full window (64) only the two diagonal tiles are partial.
      const float c2 = p.swa_scale * 1.4426950408889634f;
      const bool have_prev = t0 > 0;
      if constexpr (SWA == 1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (m < w) xc[m] *= c2;
          if (m == w)
#pragma unroll
            for (int i = 0; i < 4; ++i) xc[m][i] = __builtin_fmaf(xc[m][i], c2, dcur[i]);
        }
        if (have_prev) {  // uniform: false only for the sequence's first chunk
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if (m > w) xp[m] *= c2;
            if (m == w)
#pragma unroll
              for (int i = 0; i < 4; ++i) xp[m][i] = __builtin_fmaf(xp[m][i], c2, dprev[i]);
          }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m)
            if (m >= w) xp[m] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
      } else {
        const uint32_t W = (uint32_t)p.window;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rel = 16 * (m - w) + 4 * g + i - r16;
            if (m <= w) xc[m][i] = (uint32_t)(-rel) < W ? c2 * xc[m][i] : -INFINITY;
            if (m >= w) xp[m][i] = have_prev && (uint32_t)(C - rel) < W ? c2 * xp[m][i] : -INFINITY;
          }
        }
      }
      // (chains of three-operand maxima)
      float mx = -INFINITY;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m <= w) {
          mx = fmaxf(fmaxf(mx, xc[m][0]), xc[m][1]);
          mx = fmaxf(fmaxf(mx, xc[m][2]), xc[m][3]);
        }
        if (m >= w) {
          mx = fmaxf(fmaxf(mx, xp[m][0]), xp[m][1]);
          mx = fmaxf(fmaxf(mx, xp[m][2]), xp[m][3]);
        }
      }
      mx = rows_max(mx);
      // fp16 hi / lo weights per key block: this chunk's blocks, the previous chunk's
      uint4 ch[2], cl[2], qh_[2], ql_[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ch[kb] = cl[kb] = qh_[kb] = ql_[kb] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int side = 0; side < 2; ++side) {  // 0: this chunk, 1: previous chunk
          if (side == 0 ? m <= w : m >= w) {
            const f32x4& x = side == 0 ? xc[m] : xp[m];
            float e4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e4[i] = __builtin_amdgcn_exp2f(x[i] - mx);
            uint32_t h0, l0, h1, l1;
            split2(e4[0], e4[1], h0, l0);
            split2(e4[2], e4[3], h1, l1);
            uint4& H = side == 0 ? ch[m >> 1] : qh_[m >> 1];
            uint4& Lo = side == 0 ? cl[m >> 1] : ql_[m >> 1];
            if (m & 1) { H.z = h0; H.w = h1; Lo.z = l0; Lo.w = l1; }
            else { H.x = h0; H.y = h1; Lo.x = l0; Lo.y = l1; }
          }
        }
      }
      // the weighted sums and, from an all-ones operand against the same
      // weights, the denominator (every entry of accd)
      f32x4 accs[NT];
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) accs[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 accd = {0.f, 0.f, 0.f, 0.f};
      // key blocks: previous chunk (0,1), (2,3); this chunk (0,1), (2,3)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const bool is_prev = blk < 2;
        const int kb = blk & 1;
        const bool live = is_prev ? 2 * kb + 1 >= w : 2 * kb <= w;
        if (live) {
          const f16x8 ph = __builtin_bit_cast(f16x8, is_prev ? qh_[kb] : ch[kb]);
          const f16x8 pl = __builtin_bit_cast(f16x8, is_prev ? ql_[kb] : cl[kb]);
          const int b = is_prev ? prev : cur;
          accd = mfma(ones, ph, accd);
          accd = mfma(ones, pl, accd);
#pragma unroll
          for (int nn = 0; nn < NT; ++nn) {
            const int col = 16 * nn + r16;
            const f16x8 va = tr44(&S.vh[b][0][0], 32 * kb + 4 * g, 16 * nn, vrow<NT>());
            accs[nn] = mfma(va, ph, accs[nn]);
            accs[nn] = mfma(va, pl, accs[nn]);
          }
        }
      }
      const float rs_ = __builtin_amdgcn_rcpf(accd[0]);
      if (pos < n) {
        float* yrow = p.y_swa + (bh * p.L + t0 + pos) * DV + 4 * g;
#pragma unroll
        for (int nn = 0; nn < NT; ++nn)
          store_y<NT>(yrow + 16 * nn, accs[nn] * rs_);
      }
    }

    // ---- state update with this chunk (registers only)
    float gn = 1.f;  // decay of the carried state over this chunk
    if constexpr (DEC) {
      f16x8 wk[2];  // weight gamma^(n-1-key) of this lane's keys 32 ks + 8 g + i
      float gs;
      if (n == C) {  // uniform branch: a whole chunk takes the pass's tables
        gn = gnC;
        gs = gsC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) wk[ks] = *reinterpret_cast<const f16x8*>(&S.wkc[32 * ks + 8 * g]);
      } else {
        gn = gpow(lg, (float)n);
        gs = gsum_pow(lg, n);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = 32 * ks + 8 * g + i;
            wk[ks][i] = (half_t)(key < n ? gpow(lg, (float)(n - 1 - key)) : 0.f);
          }
      }
#pragma unroll
      for (int j = 0; j < Own<NT>::PPW; ++j) tacc[j] *= gn;
#pragma unroll
      for (int ms = 0; ms < 3; ++ms) tz[ms] *= gn;
      update_chunk<NT, 1>(S.kt, &S.vh[cur][0][0], tacc, tz, ia, ib, wk);
      z0 = gn * z0 + gs;
    } else {
      // wavefront 0 (the one the causal in-chunk term leaves lightest) adds
      // the column sums of v (rows past n of a ragged chunk are zero)
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) vacc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
      update_chunk<NT, 0, 0, 1>(S.kt, &S.vh[cur][0][0], tacc, tz, ia, ib, nullptr, vacc, w == 0);
      z0 += (float)n;
    }
    post_max<NT>(S.wmax, tacc, tz);
    __syncthreads();  // every read of tt, t0 and the chunk buffers done; wmax complete
    if constexpr (DEC) {
      if (tid < DV) {
        float vs = 0.f;
#pragma unroll
        for (int part = 0; part < PARTS; ++part) vs += S.vpart[part * DV + tid];
        S.t0[tid] = gn * S.t0[tid] + vs;
      }
    } else if (w == 0 && g == 0) {
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) S.t0[16 * nn + r16] += vacc[nn][0];
    }
    e = state_scale(S.wmax, down, up);
    if constexpr (HI) publish_state_hilo<NT>(S.tt, S.tl, tacc, tz, down);
    else publish_state<NT>(S.tt, tacc, tz, e, down);
    if constexpr (SWA) cur ^= 1;  // the next chunk replaces the previous one
    if (tn < tok_end) store_chunk<NT>(S.kt, &S.vh[cur][0][0], S.qh, S.kh[cur], pf);
  }

  // ---- the last segment writes the final state
  if (p.S_out && seg == p.nseg - 1) {
    __syncthreads();  // t0 complete
    store_z<NT>(S.zf, tz);
    __syncthreads();
    write_phi_state<NT>(S.t0, S.zf, tacc, z0, p.S_out + bh * DPHI * DV, p.z_out + bh * DPHI);
  }
}

// ---------------------------------------------------------------------------
// State-only pass over segment s < nseg - 1 of a (batch, head): the segment's
// increment of the compact state (segment 0's record also carries S_in).
// Update only, in groups of chunks (SG, half that in the decayed variant):
// k^T and the row-major v of a whole group sit in LDS together, so a group
// costs two barriers and its updates run back to back, while the next
// group's inputs are in flight in registers.  The reads go through buffer resources that end at the
// segment's end: chunks past it read as zero and add nothing, so every
// update runs unconditionally.
constexpr int SG = 4;
template <int NT>
struct StateSmem {
  static constexpr int DV = 16 * NT;
  alignas(16) half_t kt[SG][DK + 1][KT];
  alignas(16) half_t vh[SG][C][vrow<NT>()];
  alignas(16) float t0[DV];
  alignas(16) float zf[NF];
  alignas(16) half_t wkc[C];  // decayed variant: key weights gamma^(C - 1 - key)
};

// CS: the value columns split over CS workgroups per segment (each takes
// DV = 16 NT of the DVF = CS DV columns of the records; the first also writes
// the denominator record).  Splitting halves a workgroup's accumulators and
// doubles the workgroups, which pays at d_v = 128 (segments too few to fill
// the chip) but not at d_v = 64.
template <int NT, int DEC = 0, int CS = 1>
__global__ __launch_bounds__(NTHR, Occ<NT>::value) void linattn_state_kernel(Params p) {
  constexpr int DV = 16 * NT, DVF = DV * CS;
  // chunks per group (the decayed variant's extra per-chunk registers leave
  // room for half the prefetches)
  constexpr int G = DEC ? SG / 2 : SG;
  __shared__ StateSmem<NT> S;

  const int nsm = p.nrec ? p.nrec : p.nseg - 1;
  int bhi, part;
  xcd_unit_part(blockIdx.x, gridDim.x / (nsm * CS), nsm * CS, bhi, part);
  const int seg = part / CS, col0 = (part % CS) * DV;
  const size_t bh = bhi;
  const int tid = threadIdx.x;
  const int tok_begin = seg * p.seg_chunks * C;
  const int tok_end = min(p.L, tok_begin + p.seg_chunks * C);
  const size_t rec = (size_t)(NF + 1) * DVF;

  // the head's k and v up to the segment's end; the first group's loads go
  // out first, overlapping the state set-up
  HeadRsrc rs;
  rs.q = rs.k = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + bh * p.L * DK), (short)0, tok_end * DK * 2, RSRC_DW3);
  rs.v = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + bh * (size_t)p.L * DVF), (short)0, tok_end * DVF * 2,
                                           RSRC_DW3);
  Prefetch<NT> pf[G];
#pragma unroll
  for (int i = 0; i < G; ++i) load_chunk<NT, DVF>(rs, tok_begin + i * C, false, pf[i], col0);
  // the segment's increment from zero; segment 0 adds the caller's initial
  // state after the loop (every term is linear in it)
  f32x4 tacc[Own<NT>::PPW];
  init_state<NT>(nullptr, tacc);
  f32x4 tz[3];
#pragma unroll
  for (int ms = 0; ms < 3; ++ms) tz[ms] = f32x4{0.f, 0.f, 0.f, 0.f};
  float z0 = 0.f;
  for (int j = tid; j < SG * KT; j += NTHR) S.kt[j / KT][ONES][j % KT] = (half_t)1.f;
  int ia[3], ib[3];
  slot_rows(ia, ib);

  // wavefront 0 carries the column sums of v (the constant row), formed in
  // the updates from the v fragments they load
  f32x4 vacc[NT];
#pragma unroll
  for (int nn = 0; nn < NT; ++nn) vacc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float lg = DEC ? decay_lg2(p, bh) : 0.f;
  const int lane = tid & 63, g = lane >> 4, w = wave_index(), r16 = lane & 15;
  // a whole chunk decays the carried sums by gnC and adds gsC to the
  // constant denominator entry
  float gnC = 1.f, gsC = (float)C;
  if constexpr (DEC) {
    gnC = uniform(gpow(lg, (float)C));
    gsC = uniform(gsum_pow(lg, C));
    for (int j = tid; j < C; j += NTHR) S.wkc[j] = (half_t)gpow(lg, (float)(C - 1 - j));
  }
  for (int t = tok_begin; t < tok_end; t += G * C) {
    __syncthreads();  // the previous group's reads of LDS done
#pragma unroll
    for (int i = 0; i < G; ++i) store_chunk<NT>(S.kt[i], &S.vh[i][0][0], nullptr, nullptr, pf[i]);
#pragma unroll
    for (int i = 0; i < G; ++i) load_chunk<NT, DVF>(rs, t + (G + i) * C, false, pf[i], col0);
    __syncthreads();  // the group in LDS
    if constexpr (DEC) {
      // (a rolled loop: the decay weights of several chunks at once would
      // not fit the register budget)
#pragma unroll 1
      for (int i = 0; i < G; ++i) {
        // the carried sums decay over the chunk; keys weigh gamma^(n-1-key);
        // a chunk past the segment (n = 0) leaves everything unchanged
        const int n = min(C, max(0, tok_end - (t + i * C)));
        f16x8 wk[2];
        float gn, gs;
        if (n == C) {  // uniform branch: a whole chunk takes the pass's tables
          gn = gnC;
          gs = gsC;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) wk[ks] = *reinterpret_cast<const f16x8*>(&S.wkc[32 * ks + 8 * g]);
        } else {
          gn = gpow(lg, (float)n);
          gs = gsum_pow(lg, n);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = 32 * ks + 8 * g + e;
              wk[ks][e] = (half_t)(key < n ? gpow(lg, (float)(n - 1 - key)) : 0.f);
            }
        }
        z0 = gn * z0 + gs;
#pragma unroll
        for (int nn = 0; nn < NT; ++nn) vacc[nn] *= gn;
#pragma unroll
        for (int j = 0; j < Own<NT>::PPW; ++j) tacc[j] *= gn;
#pragma unroll
        for (int ms = 0; ms < 3; ++ms) tz[ms] *= gn;
        update_chunk<NT, 1, 0, 1>(S.kt[i], &S.vh[i][0][0], tacc, tz, ia, ib, wk, vacc, w == 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i)
        update_chunk<NT, 0, 1, 1>(S.kt[i], &S.vh[i][0][0], tacc, tz, ia, ib, nullptr, vacc, w == 0);
    }
  }
  if constexpr (!DEC) z0 += (float)(tok_end - tok_begin);
  __syncthreads();
  store_z<NT>(S.zf, tz);
  if (w == 0 && g == 0)
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) S.t0[16 * nn + r16] = vacc[nn][0];
  __syncthreads();
  // segment 0: the caller's initial state, decayed over the segment
  const float* Sin = (seg == 0 && p.S_in) ? p.S_in + bh * DPHI * DVF : nullptr;
  const float* zin = (seg == 0 && p.z_in) ? p.z_in + bh * DPHI : nullptr;
  const float gN = DEC ? gpow(lg, (float)(tok_end - tok_begin)) : 1.f;
  if (Sin && tid < DV) S.t0[tid] += gN * Sin[col0 + tid];
  if (zin) {
    for (int r = tid; r < NF; r += NTHR) S.zf[r] += gN * compact_from_phi(zin, r, 0, 1);
    z0 += gN * zin[0];
  }
  if (Sin) {
    f32x4 s0[Own<NT>::PPW];
    init_state<NT>(Sin, s0, col0, DVF);
#pragma unroll
    for (int j = 0; j < Own<NT>::PPW; ++j) tacc[j] += gN * s0[j];
    // record 0: S_in itself, the main pass's start of segment 0 (that pass
    // then reads no S_in, so S_out may alias it)
    write_initial_record<NT, CS>(Sin, zin, s0, p.ws + bh * p.nseg * rec, p.wsz + bh * p.nseg * (size_t)(NF + 1),
                                 col0);
  }
  __syncthreads();
  write_compact<NT, CS>(S.t0, S.zf, tacc, z0, p.ws + (bh * p.nseg + seg + 1) * rec,
                        p.wsz + (bh * p.nseg + seg + 1) * (size_t)(NF + 1), col0);
}

// Prefix over the segment records of each (batch, head): record s >= 1 holds
// the increment of segment s-1 (record 1: the initial state plus that
// increment); after the scan record s is the state at the start of segment s.
// Record 0 (the initial state, when there is one) is left as it is.
__global__ void seg_scan_kernel(float* ws, float* wsz, int nseg, int rec, int BH, const float* gamma, int H,
                                int seg_len) {
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
  // records are loaded 8 at a time before any is written, so the loads of a
  // group are in flight together
  float run = base[stride];
  // decayed variant: the running state decays over each segment it crosses
  const float gseg =
      gamma ? __builtin_amdgcn_exp2f(decay_lg2_clamped(__log2f(gamma[bh % H])) * (float)seg_len) : 1.f;
  for (int s0 = 2; s0 < nseg; s0 += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = s0 + i < nseg ? base[(size_t)(s0 + i) * stride] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (s0 + i < nseg) {
        run = gseg * run + x[i];
        base[(size_t)(s0 + i) * stride] = run;
      }
    }
  }
}

}  // namespace mfma

using namespace mfma;

template <int NT, int SWA, int DEC, int HI>
static hipError_t launch_nt_hi(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  constexpr int DV = 16 * NT;
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y;
  p.S_in = a.S_in; p.z_in = a.z_in; p.S_out = a.S_out; p.z_out = a.z_out;
  p.L = a.L;
  p.y_swa = y_swa; p.window = window; p.swa_scale = scale;
  p.gamma = a.gamma; p.H = a.H;
  linattn_mfma_plan(a.B * a.H, a.L, DV, &p.nseg, &p.seg_chunks);
  const int BH = a.B * a.H;
  if (p.nseg > 1) {
    p.ws = (float*)a.workspace;
    p.wsz = p.ws + (size_t)BH * p.nseg * (NF + 1) * DV;
    if constexpr (NT == 8)
      hipLaunchKernelGGL((linattn_state_kernel<NT / 2, DEC, 2>), dim3(BH * (p.nseg - 1) * 2), dim3(NTHR), 0, s, p);
    else
      hipLaunchKernelGGL((linattn_state_kernel<NT, DEC>), dim3(BH * (p.nseg - 1)), dim3(NTHR), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (p.nseg > MAX_SUM + 1) {
      const size_t total = (size_t)BH * ((size_t)(NF + 1) * DV + NF + 1);
      hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p.ws, p.wsz,
                         p.nseg, (NF + 1) * DV, BH, DEC ? p.gamma : nullptr, a.H, p.seg_chunks * C);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((linattn_mfma_kernel<NT, SWA, DEC, HI>), dim3(BH * p.nseg), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

template <int NT, int SWA, int DEC = 0>
static hipError_t launch_nt(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  // a caller's initial state: the high-precision readout
  if (a.S_in) return launch_nt_hi<NT, SWA, DEC, 1>(a, y_swa, window, scale, s);
  return launch_nt_hi<NT, SWA, DEC, 0>(a, y_swa, window, scale, s);
}

// State-only pass on its own (zero initial state): records [BH][nseg][NF + 1][dv]
// and [BH][nseg][NF + 1] at ws / wsz, record s + 1 = the compact increment of
// segment s for s < nrec (nrec <= nseg - 1), slot values
// sum_t [k_a | k_a^2 | k_a k_b] v_t (decayed: weights gamma^(end - 1 - t) over
// the segment's positions t).
template <int NT>
static hipError_t launch_state_records_nt(const void* k, const void* v, float* ws, int BH, int L, int nseg,
                                          int seg_chunks, int nrec, const float* gamma, int H, hipStream_t s) {
  Params p{};
  p.k = (const bf16_t*)k; p.v = (const bf16_t*)v;
  p.L = L; p.nseg = nseg; p.seg_chunks = seg_chunks; p.nrec = nrec;
  p.ws = ws;
  p.wsz = ws + (size_t)BH * nseg * (NF + 1) * (16 * NT);
  p.gamma = gamma;
  p.H = H;
  // with at most one record per two CUs, each record's value columns are
  // split over two workgroups (same records)
  if constexpr (NT % 4 == 0) {
    if ((long long)BH * nrec <= 128) {
      if (gamma) hipLaunchKernelGGL((linattn_state_kernel<NT / 2, 1, 2>), dim3(BH * nrec * 2), dim3(NTHR), 0, s, p);
      else hipLaunchKernelGGL((linattn_state_kernel<NT / 2, 0, 2>), dim3(BH * nrec * 2), dim3(NTHR), 0, s, p);
      return hipGetLastError();
    }
  }
  if (gamma) hipLaunchKernelGGL((linattn_state_kernel<NT, 1>), dim3(BH * nrec), dim3(NTHR), 0, s, p);
  else hipLaunchKernelGGL((linattn_state_kernel<NT>), dim3(BH * nrec), dim3(NTHR), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_linattn_state_records(const void* k, const void* v, float* ws, int BH, int L, int dv, int nseg,
                                        int seg_chunks, int nrec, const float* gamma, int H, hipStream_t s) {
  if (nseg < 2 || nrec < 1) return hipSuccess;
  if (nrec > nseg - 1) return hipErrorInvalidValue;
  switch (dv) {
    case 32: return launch_state_records_nt<2>(k, v, ws, BH, L, nseg, seg_chunks, nrec, gamma, H, s);
    case 64: return launch_state_records_nt<4>(k, v, ws, BH, L, nseg, seg_chunks, nrec, gamma, H, s);
    case 96: return launch_state_records_nt<6>(k, v, ws, BH, L, nseg, seg_chunks, nrec, gamma, H, s);
    case 128: return launch_state_records_nt<8>(k, v, ws, BH, L, nseg, seg_chunks, nrec, gamma, H, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_linattn_decay_mfma(const LinattnArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 32: return launch_nt<2, 0, 1>(a, nullptr, 0, 0.f, s);
    case 64: return launch_nt<4, 0, 1>(a, nullptr, 0, 0.f, s);
    case 96: return launch_nt<6, 0, 1>(a, nullptr, 0, 0.f, s);
    case 128: return launch_nt<8, 0, 1>(a, nullptr, 0, 0.f, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_linattn_mfma(const LinattnArgs& a, hipStream_t s) {
  switch (a.dv) {
    case 32: return launch_nt<2, 0>(a, nullptr, 0, 0.f, s);
    case 64: return launch_nt<4, 0>(a, nullptr, 0, 0.f, s);
    case 96: return launch_nt<6, 0>(a, nullptr, 0, 0.f, s);
    case 128: return launch_nt<8, 0>(a, nullptr, 0, 0.f, s);
  }
  return hipErrorInvalidValue;
}

template <int SWA, int DEC>
static hipError_t launch_layer(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  switch (a.dv) {
    case 32: return launch_nt<2, SWA, DEC>(a, y_swa, window, scale, s);
    case 64: return launch_nt<4, SWA, DEC>(a, y_swa, window, scale, s);
    case 96: return launch_nt<6, SWA, DEC>(a, y_swa, window, scale, s);
    case 128: return launch_nt<8, SWA, DEC>(a, y_swa, window, scale, s);
  }
  return hipErrorInvalidValue;
}

// The fused layer pass; with a.gamma the linear attention's state decays
// per head (the window attention has no decay).
hipError_t launch_layer_mfma(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t s) {
  if (a.gamma)
    return window >= C ? launch_layer<1, 1>(a, y_swa, window, scale, s) : launch_layer<2, 1>(a, y_swa, window, scale, s);
  return window >= C ? launch_layer<1, 0>(a, y_swa, window, scale, s) : launch_layer<2, 0>(a, y_swa, window, scale, s);
}

}  // namespace based
