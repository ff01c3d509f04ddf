// Causal Taylor linear attention, backward on the matrix cores (bf16 inputs,
// d_v in {32, 64, 96, 128}).
//
// Gradients of the normalised forward y_i = num_i / den_i (blog post
// "Базированная модель, часть 2": Taylor kernel 1 + x + x^2/2 as the feature
// dot product phi(q).phi(k); based/train README: the training views train
// through this forward).  With g_i = dy_i / den_i and h_i = -(dy_i . y_i) / den_i
// the kernel entries' gradient is dK_ij = g_i . v_j + h_i, and in feature form
//   dq_i = J_phi(q_i)^T [ S_i g_i + z_i h_i ]            (S, z: prefix states)
//   dk_j = J_phi(k_j)^T [ R_j v_j + r_j ],  dv_j = R_j^T phi(k_j)
// with the suffix states R_j = sum_{i>=j} phi(q_i) g_i^T, r_j = sum_{i>=j} phi(q_i) h_i.
//
// Features here are the 272 non-constant rows of phi without the 1/sqrt2
// (tile 0: x_b; tile 1 + a: x_a x_b; b = 0..15 within a tile), so the
// quadratic block of every state is symmetric in (a, b) and the Jacobian
// contractions are lane-local: a lane holding u[(b, a)] for its four a and
// every b adds u[(b, a)] x_b into the gradient of x_a.  The 1/2 of the
// quadratic term sits on the side that is not differentiated.  The states
// are accumulated in the 160 compact slots of the forward's records (one per
// unordered pair) and expanded to these rows only in the fp16 copies that the
// readouts and contractions read.
//
// Passes (chunks of 64 positions; one workgroup of 4 wavefronts per (head,
// slice of 32 value columns); with several slices each writes its dq and dk
// shares to a buffer of its own, and a last pass adds them in slice order:
// float atomics onto one buffer cost far more, and their order would show in
// the last bits).
// Every term in h is linear in h, and h_i = sum over slices of
// h_i^s = -(dy_i . y_i over the slice's columns) / den_i: each slice adds the
// terms of its own h^s, so no pass needs the whole row dy_i . y_i.
//   query pass, chunks in order: den_i (state z plus the in-chunk kernel
//     sums), h_i^s and g_i; dq_i from u = S g + z h^s through the lane-local
//     contraction, plus the in-chunk term sum_j dK_ij (1 + x_ij) k_j; then the
//     state update S += phi(K)^T V, z += phi(K)^T 1.  Writes den and h^s.
//   key pass, chunks in reverse: dk_j from u = R v + r, dv_j from
//   R^T phi~(k_j) + sum_{i later} g_i, plus the in-chunk terms; then
//   R += phi(Q)^T G, r += phi(Q)^T h.
// Operands are fp16 (bf16 inputs convert exactly); g, h and the in-chunk
// weights are split into fp16 hi + lo; the state copies read by the matrix
// cores are fp16 scaled by a power of two; all sums are fp32.
#include <type_traits>

#include "based_device.h"
#include "launchers.h"

namespace based {
namespace bwdm {

typedef _Float16 half_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;                // positions per chunk
constexpr int NTHR = 256;            // 4 wavefronts
constexpr int SW = 32;               // value columns per slice
constexpr int NFT = 17;              // feature tiles: linear, then quadratic rows a = 0..15
constexpr int NF = 16 * NFT;         // 272
constexpr int NKS = (NF + 31) / 32;  // 9 steps of 32 features (the last half zero)
constexpr int QH = 24;               // fp16 stride of q / k rows
constexpr int XT = C + 8;            // fp16 stride of transposed chunk rows
constexpr int RS = SW + 8;           // fp16 stride of slice rows
constexpr int SCALE_TOP = 13;
constexpr int MAXSEG = 8;            // segments per head at most (records summed directly)
constexpr int NFC = 160;             // compact slots of the forward's state records
constexpr int RREC = NFC * SW + NFC + SW;  // floats of one suffix-state record (R, r in compact slots, sum g)
constexpr int NFP = 32 * NKS;
static_assert(C == layout::CHUNK && SW == layout::BWD_SLICE && MAXSEG == layout::BWD_MAXSEG && NF == layout::BWD_NF &&
                  NFC == layout::FWD_SLOTS && RREC == layout::BWD_RREC,
              "planning constants (plan.cpp) must match the kernels");        // feature rows of the key pass's state copy (rows NF.. zero)

// The forward's compact record layout: slot r = 32 kb + 8 g + s holds
// pattern (kb, s) with both coordinates shifted by 4g: kb = 0 gives x_a
// (s < 4) and x_a^2 (s >= 4) for a = s % 4; kb >= 1 gives x_a x_{a+d} for
// a = s % 4, d = 2 (kb - 1) + 1 + s / 4 (mod 16).  A record holds
// sum_t [k_a | k_a^2 | k_a k_b] v_t in every slot.

// The states are symmetric in (a, b), so every pass accumulates them in the
// forward's 160 compact slots and expands them to the 272 rows of this
// layout only in the fp16 copy the readouts use.  Per slot r, packed: the
// two transposed-chunk rows whose product is its feature (bits 0-4, 5-9; row
// DK holds ones, the linear slots' second factor) and the one or two rows of
// this layout that hold it (bits 10-18, 19-27; NOROW for none): x_a x_b and
// x_b x_a for a pair, one row for a linear feature, a square, or a pair at
// distance 8 (whose two orientations are both slots).
constexpr int NCT = NFC / 16;  // compact slot tiles
constexpr int MAXC = 3;        // compact slot tiles owned by a wavefront
constexpr uint32_t NOROW = 511;
struct SlotInfo {
  uint32_t x[NFC];
};
constexpr SlotInfo make_slot_info() {
  SlotInfo t{};
  for (int r = 0; r < NFC; ++r) {
    const int kb = r / 32, g = (r % 32) / 8, s2 = r % 8;
    const int A = s2 % 4, B = kb > 0 ? A + 2 * (kb - 1) + 1 + s2 / 4 : A;
    const bool lin = kb == 0 && s2 < 4;
    const uint32_t a = (uint32_t)((A + 4 * g) % 16), b = (uint32_t)((B + 4 * g) % 16);
    uint32_t r1 = 0, r2 = NOROW;
    if (lin) r1 = a;
    else {
      r1 = 16 + 16 * a + b;
      if (a != b && (b + 16 - a) % 16 != 8) r2 = 16 + 16 * b + a;
    }
    t.x[r] = a | (lin ? (uint32_t)DK : b) << 5 | r1 << 10 | r2 << 19;
  }
  return t;
}
constexpr SlotInfo kSlotInfo = make_slot_info();
// every row of this layout is written from exactly one slot
constexpr bool slot_rows_ok() {
  int hits[NF] = {};
  for (int r = 0; r < NFC; ++r) {
    const uint32_t r1 = (kSlotInfo.x[r] >> 10) & 511u, r2 = kSlotInfo.x[r] >> 19;
    if (r1 >= (uint32_t)NF) return false;
    ++hits[r1];
    if (r2 != NOROW) {
      if (r2 >= (uint32_t)NF) return false;
      ++hits[r2];
    }
  }
  for (int f = 0; f < NF; ++f)
    if (hits[f] != 1) return false;
  return true;
}
static_assert(slot_rows_ok(), "the compact slots must cover every feature row once");
__constant__ SlotInfo c_sinfo = make_slot_info();
__device__ __forceinline__ int sl_a(uint32_t x) { return (int)(x & 31u); }
__device__ __forceinline__ int sl_b(uint32_t x) { return (int)((x >> 5) & 31u); }
__device__ __forceinline__ int sl_r1(uint32_t x) { return (int)((x >> 10) & 511u); }
__device__ __forceinline__ uint32_t sl_r2(uint32_t x) { return x >> 19; }
// Compact slot tiles: wavefront w owns tiles w and w + 4, and tile
// 8 + (w & 1) if it is one of the two that the pass's causal in-chunk work
// leaves lightest (XLO: wavefronts 0 and 1, else 2 and 3).
template <bool XLO>
__device__ __forceinline__ int cown_count(int w) { return (XLO ? w < 2 : w >= 2) ? 3 : 2; }
__device__ __forceinline__ int cown_tile(int w, int j) { return j < 2 ? w + 4 * j : 8 + (w & 1); }
// the lane's slot info for its owned tiles (read once, from constant memory)
template <bool XLO>
__device__ __forceinline__ void slot_info(int w, int r16, uint32_t (&x)[MAXC]) {
#pragma unroll
  for (int j = 0; j < MAXC; ++j) x[j] = j < cown_count<XLO>(w) ? c_sinfo.x[16 * cown_tile(w, j) + r16] : 0u;
}

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
// Transposing LDS read (ds_read_b64_tr_b16): rows r0 .. r0 + 3 of column
// c0 + (lane % 16) of the row-major fp16 array at `base` (row stride ld).
// Within each 16-lane block lane t receives element t % 4 of the 4-element
// segments addressed by lanes t / 4 + 4i, so lane j points at row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3.
__device__ __forceinline__ uint2 tr4(const half_t* base, int r0, int c0, int ld) {
  const int j = threadIdx.x & 15;
  const half_t* a = base + (r0 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
  return __builtin_bit_cast(uint2, v);
}
// MFMA operand with K = rows r0 .. r0 + 7 of column c0 + (lane % 16)
__device__ __forceinline__ f16x8 tr8(const half_t* base, int r0, int c0, int ld) {
  const uint2 a = tr4(base, r0, c0, ld), b = tr4(base, r0 + 4, c0, ld);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}
// K = rows r0 .. r0 + 3 and r0 + 16 .. r0 + 19 (two 16-row tiles)
__device__ __forceinline__ f16x8 tr44(const half_t* base, int r0, int c0, int ld) {
  const uint2 a = tr4(base, r0, c0, ld), b = tr4(base, r0 + 16, c0, ld);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// The thread index as an opaque value: addresses formed from it at their use
// inside a loop are not hoisted out of it (a hoisted address stays live
// across the whole loop body, which in the key pass cost spills whose
// reloads waited for every memory operation in flight).
__device__ __forceinline__ int tid_here() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ f16x8 ones8() {
  const uint32_t one2 = 0x3c003c00u;
  return __builtin_bit_cast(f16x8, make_uint4(one2, one2, one2, one2));
}

__device__ __forceinline__ uint32_t h2_from_bf2(uint32_t w) {
  const f32x2 f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return u32(__builtin_convertvector(f, f16x2));
}
__device__ __forceinline__ uint4 h8_from_bf8(const uint4& x) {
  return make_uint4(h2_from_bf2(x.x), h2_from_bf2(x.y), h2_from_bf2(x.z), h2_from_bf2(x.w));
}

// fp16 hi + lo of two fp32 values: hi = RNE(x), lo = RNE(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f16x2 h = __builtin_convertvector((f32x2{a, b}), f16x2);
  hi = u32(h);
  lo = u32(__builtin_convertvector((f32x2{a - (float)h[0], b - (float)h[1]}), f16x2));
}
// hi / lo operands of 8 weights: tile values t0 (K indices 0..3) and t1 (4..7)
__device__ __forceinline__ void split8(const f32x4& t0, const f32x4& t1, f16x8& hi, f16x8& lo) {
  uint32_t h[4], l[4];
  split2(t0[0], t0[1], h[0], l[0]);
  split2(t0[2], t0[3], h[1], l[1]);
  split2(t1[0], t1[1], h[2], l[2]);
  split2(t1[2], t1[3], h[3], l[3]);
  hi = __builtin_bit_cast(f16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(f16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// Sum over the four 16-lane rows of a wavefront (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max_abs(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Exponent e of the fp16 state copy (entries times 2^-e): none while the
// largest magnitude M lies in [2^-4, 2^14), else M 2^-e lands in [2^13, 2^14).
__device__ __forceinline__ int scale_exp(float M) {
  if (!(M >= 0x1p-100f)) return 0;
  if (M >= 0x1p-4f && M < 0x1p14f) return 0;
  const int ex = (int)((__float_as_uint(M) >> 23) & 0xffu) - 127;
  return ex - SCALE_TOP;
}

struct Params {
  const bf16_t* q; const bf16_t* k; const bf16_t* v; const float* y; const float* dy;
  float* den; float* h; // per position, from the query pass (h: [nslice][npos], one row per slice)
  size_t npos;          // B * H * L
  float* gq; float* gk; float* gv;
  float* pq; float* pk;  // with several slices: [nslice][npos][16] shares of dq and dk
  const float* frec;    // [BH][nseg * rsplit] forward records of (NFC + 1) dvf floats, record_offset layout
                        // (record s + 1: sub-segment s, seg_chunks / rsplit chunks from s * seg_chunks / rsplit)
  const float* frecz;   // [BH][nseg * rsplit][NFC + 1]
  float* krec;          // [BH][nslice][nseg][ksplit] suffix-state increments of a segment's parts: R [NFC][SW],
                        // r [NFC] (compact slots), sum g [SW]
  int L, dvf, nslice, nseg, seg_chunks;
  int rsplit;           // forward-record sub-segments per segment
  int ksplit;           // suffix-state sub-records per segment ([BH][nslice][nseg][ksplit] records)
  const float* gamma;   // decayed variant: [H] per-head state decay
  int H;
};

// Workgroup -> (head, value slice, segment) and the segment's positions.
struct Unit {
  size_t bh;
  int s, seg, t_begin, t_end;
};
__device__ __forceinline__ Unit unit_of(const Params& p) {
  Unit u;
  // a head's workgroups share an XCD (its L2): the slices read the same q, k
  const int per_head = p.nslice * p.nseg;
  int bh, part;
  xcd_unit_part(blockIdx.x, gridDim.x / per_head, per_head, bh, part);
  u.bh = bh;
  u.s = part / p.nseg;
  u.seg = part % p.nseg;
  u.t_begin = u.seg * p.seg_chunks * C;
  u.t_end = min(p.L, u.t_begin + p.seg_chunks * C);
  return u;
}

// ---------------------------------------------------------------- slice sums
// The sum over slices of the slices' shares ([nslice][n4] float4 each), in
// slice order, for the elements first, first + step, ... below i1; four of
// them per round, so that their loads are in flight together.
__device__ __forceinline__ void sum_slices(const float4* __restrict__ part, float4* __restrict__ out, size_t n4,
                                           int nslice, size_t first, size_t i1, size_t step) {
  for (size_t i = first; i < i1; i += 4 * step) {
    float4 a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t j = i + u * step;
      a[u] = j < i1 ? part[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int s = 1; s < nslice; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t j = i + u * step;
        if (j < i1) {
          const float4 x = part[(size_t)s * n4 + j];
          a[u].x += x.x; a[u].y += x.y; a[u].z += x.z; a[u].w += x.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * step < i1) out[i + u * step] = a[u];
  }
}

// dk = sum of the slices' shares, and dq likewise unless pq is null (the
// suffix-state pass has summed dq then).
__global__ void slice_sum_kernel(const float4* __restrict__ pq, const float4* __restrict__ pk, float4* __restrict__ gq,
                                 float4* __restrict__ gk, size_t n4, int nslice) {
  const size_t first = (size_t)blockIdx.x * blockDim.x + threadIdx.x, step = (size_t)gridDim.x * blockDim.x;
  if (pq) sum_slices(pq, gq, n4, nslice, first, n4, step);
  sum_slices(pk, gk, n4, nslice, first, n4, step);
}

// ---------------------------------------------------------------- chunk loads
// Raw buffer loads through per-head descriptors (scalar registers, 32-bit
// offsets): reads past the end of the sequence return zero, with no branch
// and no 64-bit address held in vector registers across the chunk loop.
struct HeadRsrc {
  __amdgpu_buffer_rsrc_t q, k, v, dy, y;
  __amdgpu_buffer_rsrc_t f1, f2;  // per-position fp32: den and the slice's h (key passes)
};
constexpr int RSRC_DW3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_DW3);
}
__device__ __forceinline__ HeadRsrc head_rsrc(const Params& p, size_t bh, const float* f1, const float* f2) {
  const size_t L = p.L;
  HeadRsrc r;
  r.q = rsrc(p.q + bh * L * DK, L * DK * 2);
  r.k = rsrc(p.k + bh * L * DK, L * DK * 2);
  r.v = rsrc(p.v + bh * L * p.dvf, L * p.dvf * 2);
  r.dy = rsrc(p.dy + bh * L * p.dvf, L * p.dvf * 4);
  r.y = rsrc(p.y + bh * L * p.dvf, L * p.dvf * 4);
  r.f1 = rsrc(f1 + bh * L, L * 4);
  r.f2 = rsrc(f2 + bh * L, L * 4);
  return r;
}
__device__ __forceinline__ uint4 bload4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Thread -> data: q (threads 0..127) or k (128..255) row (tid & 127) / 2, 8
// coordinates; v and dy of the slice: row tid / 4, columns 8 (tid % 4) ..
struct Pre {
  uint4 qk;
  uint4 v;
  float4 dy0, dy1;
  float4 y0, y1;  // query pass: y of the same slice columns
  float aux;      // key passes: den of row tid / 4
  float aux2;     // key passes: the slice's h of position tid (tid < 64)
};

__device__ __forceinline__ void load_common(const Params& p, const HeadRsrc& rs, int s, int t0, Pre& pf) {
  const int tid = threadIdx.x;
  {
    const int r = (tid & 127) >> 1, half = tid & 1;
    pf.qk = bload4(wave_index() < 2 ? rs.q : rs.k, ((t0 + r) * DK + 8 * half) * 2);
  }
  {
    const int r = tid >> 2, cq = tid & 3;
    const int e = (t0 + r) * p.dvf + s * SW + 8 * cq;
    pf.v = bload4(rs.v, e * 2);
    pf.dy0 = __builtin_bit_cast(float4, bload4(rs.dy, e * 4));
    pf.dy1 = __builtin_bit_cast(float4, bload4(rs.dy, e * 4 + 16));
  }
}

// The query pass also reads y over the slice's columns (for dy . y).
__device__ __forceinline__ void q_load(const Params& p, const HeadRsrc& rs, int s, int t0, Pre& pf) {
  load_common(p, rs, s, t0, pf);
  const int tid = threadIdx.x, r = tid >> 2, cq = tid & 3;
  const int e = (t0 + r) * p.dvf + s * SW + 8 * cq;
  pf.y0 = __builtin_bit_cast(float4, bload4(rs.y, e * 4));
  pf.y1 = __builtin_bit_cast(float4, bload4(rs.y, e * 4 + 16));
}

// ---------------------------------------------------------------- query pass
struct QSmem {
  alignas(16) half_t qh[C][QH];            // q rows
  alignas(16) half_t kh[C][QH];            // k rows
  alignas(16) half_t kt[DK + 1][XT];       // k^T; row DK all ones
  alignas(16) half_t vh[C][RS];            // v rows (slice)
  alignas(16) half_t gh[C][RS], gl[C][RS];  // g hi / lo (slice)
  alignas(16) half_t st[NF][RS];           // state S, feature rows, scaled by 2^-e
  alignas(16) float zs[NF];                // state z (fp32)
  float dys[C];                            // dy . y over the slice's columns, per position
  float dens[C];                           // den of the chunk's positions
  float wmax[4];
  // decayed variant: the in-chunk weights gamma^(query - key) as lane l of
  // wavefront w holds them for the key tile t tiles before its query tile
  // (query 16 w + l % 16, keys 16 (w - t) + 4 (l / 16) + i; zero for a key
  // after the query), and the update's key weights gamma^(C - 1 - key)
  alignas(16) float dw[4][64][4];
  alignas(16) half_t wkc[C];
};

__device__ __forceinline__ void q_store(QSmem& S, const Pre& pf) {
  const int tid = threadIdx.x;
  {
    const int r = (tid & 127) >> 1, half = tid & 1;
    const uint4 x = h8_from_bf8(pf.qk);
    if (tid < 128) {
      *reinterpret_cast<uint4*>(&S.qh[r][8 * half]) = x;
    } else {
      *reinterpret_cast<uint4*>(&S.kh[r][8 * half]) = x;
      const f16x8 e = __builtin_bit_cast(f16x8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) S.kt[8 * half + i][r] = e[i];
    }
  }
  {
    const int r = tid >> 2, cq = tid & 3;
    *reinterpret_cast<uint4*>(&S.vh[r][8 * cq]) = h8_from_bf8(pf.v);
  }
  {
    // dy . y over the slice's columns: 8 per thread, 4 threads per row
    const float4 a0 = pf.dy0, a1 = pf.dy1, b0 = pf.y0, b1 = pf.y1;
    float d = a0.x * b0.x + a0.y * b0.y + a0.z * b0.z + a0.w * b0.w + a1.x * b1.x + a1.y * b1.y + a1.z * b1.z +
              a1.w * b1.w;
    d += __shfl_xor(d, 1, 64);
    d += __shfl_xor(d, 2, 64);
    if ((tid & 3) == 0) S.dys[tid >> 2] = d;
  }
}

// DEC: the decayed variant (a per-head gamma on the state: the kernel
// entry of (i, j) weighs gamma^(i-j)).  The state before a chunk reaches its
// position pos times gamma^(pos + 1) (readout and den), the in-chunk terms
// carry gamma^(i-j), and the update is S <- gamma^n S + sum_j gamma^(n-1-j)
// phi(k_j) v_j^T; the forward records are the segments' decayed increments,
// summed with the decay over the distance to this segment.
template <int DEC>
__global__ __launch_bounds__(NTHR, 2) void query_pass_kernel(Params p) {
  __shared__ QSmem S;
  const Unit un = unit_of(p);
  const size_t bh = un.bh;
  const int s = un.s;
  const bool first = s == 0;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int pos = 16 * w + r16;  // position (query) of the lane in transposed tiles
  const int L = p.L;
  const float lg = DEC ? decay_lg2_clamped(__log2f(p.gamma[bh % p.H])) : 0.f;
  const float cf = DEC ? gpow(lg, (float)(pos + 1)) : 1.f;  // the carried state's weight at pos
  if constexpr (DEC) {
    for (int j = tid; j < 4 * 64; j += NTHR) {
      const int t = j >> 6, l = j & 63, d0 = 16 * t + (l & 15) - 4 * (l >> 4);
      float4 wv;
      wv.x = d0 >= 0 ? gpow(lg, (float)d0) : 0.f;
      wv.y = d0 >= 1 ? gpow(lg, (float)(d0 - 1)) : 0.f;
      wv.z = d0 >= 2 ? gpow(lg, (float)(d0 - 2)) : 0.f;
      wv.w = d0 >= 3 ? gpow(lg, (float)(d0 - 3)) : 0.f;
      *reinterpret_cast<float4*>(&S.dw[t][l][0]) = wv;
    }
    for (int j = tid; j < C; j += NTHR) S.wkc[j] = (half_t)gpow(lg, (float)(C - 1 - j));
  }

  for (int e = tid; e < NF * RS / 2; e += NTHR) reinterpret_cast<uint32_t*>(&S.st[0][0])[e] = 0u;
  for (int e = tid; e < NF; e += NTHR) S.zs[e] = 0.f;
  for (int e = tid; e < XT; e += NTHR) S.kt[DK][e] = (half_t)1.f;
  // state S of the owned compact slot tiles; z as one value per lane and
  // tile (slot 16 t + r16: the rows of a z tile are all equal)
  const int nown = cown_count<true>(w);
  uint32_t si[MAXC];
  slot_info<true>(w, r16, si);
  f32x4 acc[MAXC][2];
  float zacc[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    zacc[j] = 0.f;
  }
  float up = 1.f;
  // largest state magnitude over the workgroup -> scale; state copy to LDS
  // (each slot to its one or two rows)
  auto publish = [&]() {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j)
      if (j < nown)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[j][nn][i]));
    mx = wave_max_abs(mx);
    if (lane == 0) S.wmax[w] = mx;
    __syncthreads();  // every read of the state copy and the chunk buffers done
    const int e = scale_exp(fmaxf(fmaxf(S.wmax[0], S.wmax[1]), fmaxf(S.wmax[2], S.wmax[3])));
    const float down = __builtin_amdgcn_ldexpf(1.f, -e);
    up = __builtin_amdgcn_ldexpf(1.f, e);
    // (two copies of the store loop behind one uniform branch: no scaling
    // while e = 0, the usual case)
    auto store_copy = [&](auto scaled) {
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        if (j < nown) {
          const int r1 = sl_r1(si[j]);
          const uint32_t r2 = sl_r2(si[j]);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            f32x4 a = acc[j][nn];
            if constexpr (decltype(scaled)::value) a *= down;
            const uint32_t w0 = u32(__builtin_convertvector((f32x2{a[0], a[1]}), f16x2));
            const uint32_t w1 = u32(__builtin_convertvector((f32x2{a[2], a[3]}), f16x2));
            *reinterpret_cast<uint2*>(&S.st[r1][16 * nn + 4 * g]) = make_uint2(w0, w1);
            if (r2 != NOROW) *reinterpret_cast<uint2*>(&S.st[r2][16 * nn + 4 * g]) = make_uint2(w0, w1);
          }
          if (g == 0) {
            S.zs[r1] = zacc[j];
            if (r2 != NOROW) S.zs[r2] = zacc[j];
          }
        }
      }
    };
    if (__builtin_amdgcn_readfirstlane(e) != 0) store_copy(std::true_type{});
    else store_copy(std::false_type{});
  };
  // the state before the segment: the sum of the forward records of the
  // earlier segments (slot values sum_t [k_a | k_a^2 | k_a k_b] v_t)
  // (records 1 .. nr of the head, through buffer resources that end at
  // record nr: an odd first record alone, then two records per round with
  // both records' loads in flight together)
  if (un.seg > 0) {
    const int rows = NFC + 1, nr = un.seg * p.rsplit;
    const size_t first = bh * p.nseg * p.rsplit + 1;
    // decayed variant: record k (0-based) ends (nr - 1 - k) sub-segments
    // before this segment starts
    const int sub = p.seg_chunks * C / p.rsplit;
    auto rec_w = [&](int k2) { return DEC ? gpow(lg, (float)((nr - 1 - k2) * sub)) : 1.f; };
    const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.frec + first * rows * p.dvf), (short)0, nr * rows * p.dvf * (int)sizeof(float), RSRC_DW3);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.frecz + first * rows), (short)0, nr * rows * (int)sizeof(float), RSRC_DW3);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (j < nown) {
        const int slot = 16 * cown_tile(w, j) + r16;
        float z = 0.f;
        if (nr & 1) {  // record 1 on its own
          const float wr = rec_w(0);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[j][nn][i] += wr * bload1(rf, (int)record_offset(slot, s * SW + 16 * nn + 4 * g + i, p.dvf) *
                                                   (int)sizeof(float));
          z += wr * bload1(rz, slot * (int)sizeof(float));
        }
        for (int r = nr & 1; r < nr; r += 2) {  // pairs (an odd record first, alone)
          float x[2][2][4], zz[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int nn = 0; nn < 2; ++nn)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                x[u][nn][i] = bload1(rf, ((r + u) * rows * p.dvf +
                                          (int)record_offset(slot, s * SW + 16 * nn + 4 * g + i, p.dvf)) *
                                             (int)sizeof(float));
            zz[u] = bload1(rz, ((r + u) * rows + slot) * (int)sizeof(float));
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float wr = rec_w(r + u);
#pragma unroll
            for (int nn = 0; nn < 2; ++nn)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[j][nn][i] += wr * x[u][nn][i];
            z += wr * zz[u];
          }
        }
        zacc[j] = z;
      }
    }
    publish();
  }
  const HeadRsrc rs = head_rsrc(p, bh, p.den, p.den);
  Pre pf;
  q_load(p, rs, s, un.t_begin, pf);
  __syncthreads();
  q_store(S, pf);
  const f16x8 zero8 = {};
  const f16x8 ones = ones8();

  for (int t0 = un.t_begin; t0 < un.t_end; t0 += C) {
    const int n = min(C, un.t_end - t0);
    const float4 dy0 = pf.dy0, dy1 = pf.dy1;  // this chunk's dy (the prefetch below replaces pf)
    __syncthreads();  // chunk inputs and the state copy visible
    if (t0 + C < un.t_end) q_load(p, rs, s, t0 + C, pf);

    // ---- scores X^T (keys x queries) of the chunk's key tiles m <= w, the
    // kernel weights K = 1 + x + x^2/2 below the diagonal, their row sums
    const f16x8 qv = g < 2 ? ld8(&S.qh[pos][8 * g]) : zero8;
    f32x4 xc[4];
    float dpart = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      xc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m <= w) {
        const f16x8 kv = g < 2 ? ld8(&S.kh[16 * m + r16][8 * g]) : zero8;
        xc[m] = mfma(kv, qv, xc[m]);
        if constexpr (DEC) {  // gamma^(query - key), zero for a key after the query
          const float4 dv4 = *reinterpret_cast<const float4*>(&S.dw[w - m][lane][0]);
          const float wt[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = xc[m][i];
            dpart += wt[i] * (1.f + x + 0.5f * x * x);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = xc[m][i];
            if (m < w || 4 * g + i <= r16) dpart += 1.f + x + 0.5f * x * x;
          }
        }
      }
    }
    // ---- the state's share of den: z_lin . q + q^T Z2 q / 2, this lane's four rows a
    float qf[DK];
    {
      const f16x8 q0 = ld8(&S.qh[pos][0]), q1 = ld8(&S.qh[pos][8]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qf[i] = (float)q0[i];
        qf[8 + i] = (float)q1[i];
      }
    }
    // zg[i] = z_lin[a] + sum_b z[(a, b)] q_b for a = 4g + i is also the
    // z h share of dq[a] (times h): z is symmetric in (a, b)
    f32x4 zg;
    {
      const uint2 qa2 = *reinterpret_cast<const uint2*>(&S.qh[pos][4 * g]);
      const f16x8 qa8 = __builtin_bit_cast(f16x8, make_uint4(qa2.x, qa2.y, 0u, 0u));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a = 4 * g + i;
        const float qa = (float)qa8[i];
        float zq = 0.f;
#pragma unroll
        for (int b = 0; b < DK; b += 4) {
          const float4 z4 = *reinterpret_cast<const float4*>(&S.zs[DK + DK * a + b]);
          zq += z4.x * qf[b] + z4.y * qf[b + 1] + z4.z * qf[b + 2] + z4.w * qf[b + 3];
        }
        dpart += cf * qa * (S.zs[a] + 0.5f * zq);
        zg[i] = S.zs[a] + zq;
      }
    }
    // (the constant feature: t0 earlier positions, decayed: cf sum_{d < t0} gamma^d)
    const float den = rows_sum(dpart) + (DEC ? cf * gsum_pow(lg, t0) : (float)t0);
    const float hval = -S.dys[pos] / den;
    if (g == 0) {
      S.dens[pos] = den;
      if (pos < n) {
        if (first) p.den[(size_t)bh * L + t0 + pos] = den;
        p.h[(size_t)s * p.npos + (size_t)bh * L + t0 + pos] = hval;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- g = dy / den of the wavefront's rows, fp16 hi / lo
    {
      const int row = 16 * w + (lane >> 2), cq = lane & 3;
      const float rden = 1.f / S.dens[row];
      uint32_t hi[4], lo[4];
      split2(dy0.x * rden, dy0.y * rden, hi[0], lo[0]);
      split2(dy0.z * rden, dy0.w * rden, hi[1], lo[1]);
      split2(dy1.x * rden, dy1.y * rden, hi[2], lo[2]);
      split2(dy1.z * rden, dy1.w * rden, hi[3], lo[3]);
      *reinterpret_cast<uint4*>(&S.gh[row][8 * cq]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&S.gl[row][8 * cq]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __builtin_amdgcn_wave_barrier();

    // ---- dq from the state: u^T = S^T-readout (features x this position),
    // lane-local contraction into dq[4g + i]; plus the z h share, h zg
    // (the copy's scale 2^e rides on the q factors: exact, a power of two)
    // (decayed: the carried state's weight cf at this position rides along)
    const float upc = DEC ? up * cf : up;
    f32x4 dqa = zg * (DEC ? hval * cf : hval);
    const f16x8 gbh = ld8(&S.gh[pos][8 * g]), gbl = ld8(&S.gl[pos][8 * g]);
#pragma unroll
    for (int m = 0; m < NFT; ++m) {
      const f16x8 sa = ld8(&S.st[16 * m + r16][8 * g]);
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      u = mfma(sa, gbh, u);  // g rounded once: the state copy is fp16 as well
      dqa += u * (m == 0 ? upc : qf[m - 1] * upc);
    }

    // ---- in-chunk term: dK^T = V G^T (+ h), c = dK (1 + x) below the
    // diagonal, dq += K^T c over key blocks (tiles 2kb, 2kb + 1)
    {
      f32x4 cw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        cw[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m <= w) {
          const f16x8 va = ld8(&S.vh[16 * m + r16][8 * g]);
          f32x4 da = {0.f, 0.f, 0.f, 0.f};
          da = mfma(va, gbh, da);
          da = mfma(va, gbl, da);
          if constexpr (DEC) {
            const float4 dv4 = *reinterpret_cast<const float4*>(&S.dw[w - m][lane][0]);
            const float wt[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) cw[m][i] = wt[i] * (da[i] + hval) * (1.f + xc[m][i]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float dk = da[i] + hval;
              cw[m][i] = (m < w || 4 * g + i <= r16) ? dk * (1.f + xc[m][i]) : 0.f;
            }
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb <= w) {
          f16x8 bh8, bl8;
          split8(cw[2 * kb], cw[2 * kb + 1], bh8, bl8);
          const f16x8 ka = cat44(&S.kt[r16][32 * kb + 4 * g], &S.kt[r16][32 * kb + 16 + 4 * g]);
          dqa = mfma(ka, bh8, dqa);
          dqa = mfma(ka, bl8, dqa);
        }
      }
    }
    if (pos < n) {
      float* dst = (p.nslice == 1 ? p.gq : p.pq + (size_t)s * p.npos * DK) + ((size_t)bh * L + t0 + pos) * DK + 4 * g;
      __builtin_nontemporal_store(dqa, reinterpret_cast<f32x4*>(dst));  // (see the key pass's stores)
    }

    // ---- state update with the chunk (none after the segment's last: no
    // later chunk reads it): S^T += V^T phi(K), z += phi(K)^T 1
    // (decayed: S^T <- gamma^n S^T + V^T diag(gamma^(n-1-j)) phi(K), z likewise)
    if (t0 + C >= un.t_end) break;  // uniform
    f16x8 wk[2];
    if constexpr (DEC) {
      float gn;
      if (n == C) {  // uniform branch: a whole chunk takes the table
        gn = gpow(lg, (float)C);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) wk[ks] = ld8(&S.wkc[32 * ks + 8 * g]);
      } else {
        gn = gpow(lg, (float)n);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int key = 32 * ks + 8 * g + i;
            wk[ks][i] = (half_t)(key < n ? gpow(lg, (float)(n - 1 - key)) : 0.f);
          }
      }
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        acc[j][0] *= gn;
        acc[j][1] *= gn;
        zacc[j] *= gn;
      }
    }
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (j < nown) {  // uniform branch
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 fb = ld8(&S.kt[sl_a(si[j])][32 * ks + 8 * g]) * ld8(&S.kt[sl_b(si[j])][32 * ks + 8 * g]);
          if constexpr (DEC) fb *= wk[ks];
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
            acc[j][nn] = mfma(tr8(&S.vh[0][0], 32 * ks + 8 * g, 16 * nn, RS), fb, acc[j][nn]);
          zacc[j] += mfma(ones, fb, f32x4{0.f, 0.f, 0.f, 0.f})[0];
        }
      }
    }
    publish();
    if (t0 + C < un.t_end) q_store(S, pf);
  }
}

// ---------------------------------------------------------------- key pass
struct KSmem {
  alignas(16) half_t qh[C][QH];              // q rows
  alignas(16) half_t qt[DK + 1][XT];         // q^T; row DK all ones
  alignas(16) half_t kh[C][QH];              // k rows
  alignas(16) half_t vh[C][RS];              // v rows (slice)
  alignas(16) half_t gh[C][RS], gl[C][RS];    // g rows hi / lo (slice)
  alignas(16) half_t hh[XT];                 // h over the chunk's positions, fp16
  alignas(16) half_t rf[NFP][RS];            // state R, feature rows (rows NF.. zero), scaled by 2^-e
  alignas(16) float rs[NF];                  // state r (fp32)
  alignas(16) float g0[SW];                  // sum of g over the later positions
  alignas(16) float hs[C];                   // h of the chunk's positions
  float gpart[8][SW];                        // column sums of g over 8-row groups
  float wmax[4];
  // decayed variant: the in-chunk weights gamma^(query - key) as lane l of
  // wavefront w holds them for the query tile t tiles after its key tile
  // (key 16 w + l % 16, queries 16 (w + t) + 4 (l / 16) + i; zero for a
  // query before the key), and the update's query weights gamma^p over the
  // chunk's positions p (fp16 for the features, fp32 for the sums of g)
  alignas(16) float dw[4][64][4];
  alignas(16) half_t wq[C];
  alignas(16) float wqf[C];
};

__device__ __forceinline__ void k_store(KSmem& S, const Pre& pf) {
  const int tid = threadIdx.x;
  {
    const int r = (tid & 127) >> 1, half = tid & 1;
    const uint4 x = h8_from_bf8(pf.qk);
    if (tid < 128) {
      *reinterpret_cast<uint4*>(&S.qh[r][8 * half]) = x;
      const f16x8 e = __builtin_bit_cast(f16x8, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) S.qt[8 * half + i][r] = e[i];
    } else {
      *reinterpret_cast<uint4*>(&S.kh[r][8 * half]) = x;
    }
  }
  {
    const int r = tid >> 2, cq = tid & 3;
    *reinterpret_cast<uint4*>(&S.vh[r][8 * cq]) = h8_from_bf8(pf.v);
    const float rden = 1.f / pf.aux;
    uint32_t hi[4], lo[4];
    split2(pf.dy0.x * rden, pf.dy0.y * rden, hi[0], lo[0]);
    split2(pf.dy0.z * rden, pf.dy0.w * rden, hi[1], lo[1]);
    split2(pf.dy1.x * rden, pf.dy1.y * rden, hi[2], lo[2]);
    split2(pf.dy1.z * rden, pf.dy1.w * rden, hi[3], lo[3]);
    *reinterpret_cast<uint4*>(&S.gh[r][8 * cq]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *reinterpret_cast<uint4*>(&S.gl[r][8 * cq]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  if (tid < C) {
    const float hv = pf.aux2;
    const int t = tid_here();
    S.hs[t] = hv;
    S.hh[t] = (_Float16)hv;
  }
}

__device__ __forceinline__ void k_load(const Params& p, const HeadRsrc& rs, int s, int t0, Pre& pf) {
  const int tid = threadIdx.x;
  load_common(p, rs, s, t0, pf);
  const int r = t0 + (tid >> 2);
  const float den = bload1(rs.f1, r * 4);
  pf.aux = r < p.L ? den : 1.f;  // rows past the end: g = 0
  pf.aux2 = bload1(rs.f2, (t0 + (tid & 63)) * 4);  // h (zero past the end)
}

// Suffix-state increment of one segment (>= 1): R += phi(Q)^T G,
// r += phi(Q)^T h and sum g over its positions; the key pass of segment s
// starts from the sum of the increments of the segments after it.
struct KIncSmem {
  alignas(16) half_t qt[DK + 1][XT];  // q^T; row DK all ones
  alignas(16) half_t gh[C][RS];  // g rows (slice), fp16
  alignas(16) half_t hh[XT];     // h, fp16
  alignas(16) float gsum[C][SW];  // per-thread column sums of g (row tid / 4), summed in row order
};

// DEC: the decayed variant -- position i of the segment weighs
// gamma^(i - start) in the increment (the key pass decays the increments of
// later segments over the distance to its own).
template <int DEC>
__global__ __launch_bounds__(NTHR) void key_state_kernel(Params p) {
  __shared__ KIncSmem S;
  // workgroup -> (head, slice, part): part 0 sums dq; part 1 + i is
  // sub-record i % ksplit of segment 1 + i / ksplit (sc chunks each)
  const int per_hs = 1 + (p.nseg - 1) * p.ksplit, sc = (p.seg_chunks + p.ksplit - 1) / p.ksplit;
  Unit un;
  int bhi, hp;
  xcd_unit_part(blockIdx.x, gridDim.x / (p.nslice * per_hs), p.nslice * per_hs, bhi, hp);
  un.bh = bhi;
  un.s = hp / per_hs;
  const int part = hp % per_hs;
  un.seg = part == 0 ? 0 : 1 + (part - 1) / p.ksplit;
  const int sub = part == 0 ? 0 : (part - 1) % p.ksplit;
  {
    const int seg_end = min(p.L, (un.seg + 1) * p.seg_chunks * C);
    un.t_begin = min(seg_end, un.seg * p.seg_chunks * C + sub * sc * C);
    un.t_end = min(seg_end, un.t_begin + sc * C);
  }
  if (un.seg == 0) {
    // Nothing lies before segment 0, so its workgroups have no state to
    // form: with several slices they sum the dq shares of their head (the
    // query pass that wrote them has completed), in slice order, workgroup s
    // taking the s-th part of the head's positions.
    if (p.nslice > 1) {
      const size_t n4 = p.npos * DK / 4, per_head = (size_t)p.L * DK / 4;
      const size_t i0 = un.bh * per_head + per_head * un.s / p.nslice;
      const size_t i1 = un.bh * per_head + per_head * (un.s + 1) / p.nslice;
      sum_slices(reinterpret_cast<const float4*>(p.pq), reinterpret_cast<float4*>(p.gq), n4, p.nslice,
                 i0 + threadIdx.x, i1, NTHR);
    }
    return;
  }
  const size_t bh = un.bh;
  const int s = un.s;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  // the increment in compact slots (written as such: the key pass reads them
  // into its compact accumulators)
  const int nown = cown_count<true>(w);
  uint32_t si[MAXC];
  slot_info<true>(w, r16, si);
  for (int e = tid; e < XT; e += NTHR) S.qt[DK][e] = (half_t)1.f;
  f32x4 acc[MAXC][2], racc[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    acc[j][0] = acc[j][1] = racc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float gpart[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float lg = DEC ? decay_lg2_clamped(__log2f(p.gamma[bh % p.H])) : 0.f;
  const HeadRsrc rs = head_rsrc(p, bh, p.den, p.h + (size_t)s * p.npos);
  Pre pf;
  k_load(p, rs, s, un.t_begin, pf);
  for (int t0 = un.t_begin; t0 < un.t_end; t0 += C) {
    __syncthreads();  // the previous chunk's reads done
    if (tid < 128) {
      const int r = tid >> 1, half = tid & 1;
      const f16x8 e = __builtin_bit_cast(f16x8, h8_from_bf8(pf.qk));
#pragma unroll
      for (int i = 0; i < 8; ++i) S.qt[8 * half + i][r] = e[i];
    }
    {
      const int r = tid >> 2, cq = tid & 3;
      float rden = 1.f / pf.aux;
      if constexpr (DEC) rden *= gpow(lg, (float)(t0 - un.t_begin + r));
      const float gv[8] = {pf.dy0.x * rden, pf.dy0.y * rden, pf.dy0.z * rden, pf.dy0.w * rden,
                           pf.dy1.x * rden, pf.dy1.y * rden, pf.dy1.z * rden, pf.dy1.w * rden};
      uint32_t hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hi[e] = u32(__builtin_convertvector((f32x2{gv[2 * e], gv[2 * e + 1]}), f16x2));
      *reinterpret_cast<uint4*>(&S.gh[r][8 * cq]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
#pragma unroll
      for (int i = 0; i < 8; ++i) gpart[i] += gv[i];
    }
    if (tid < C) S.hh[tid] = (_Float16)(DEC ? pf.aux2 * gpow(lg, (float)(t0 - un.t_begin + tid)) : pf.aux2);
    __syncthreads();
    if (t0 + C < un.t_end) k_load(p, rs, s, t0 + C, pf);
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (j < nown) {  // uniform branch
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 fb = ld8(&S.qt[sl_a(si[j])][32 * ks + 8 * g]) * ld8(&S.qt[sl_b(si[j])][32 * ks + 8 * g]);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
            acc[j][nn] = mfma(tr8(&S.gh[0][0], 32 * ks + 8 * g, 16 * nn, RS), fb, acc[j][nn]);
          racc[j] = mfma(ld8(&S.hh[32 * ks + 8 * g]), fb, racc[j]);
        }
      }
    }
  }
  float* rec = p.krec + (((bh * p.nslice + s) * p.nseg + un.seg) * p.ksplit + sub) * (size_t)RREC;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    if (j < nown) {
      const int slot = 16 * cown_tile(w, j) + r16;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
        *reinterpret_cast<float4*>(rec + (size_t)slot * SW + 16 * nn + 4 * g) =
            make_float4(acc[j][nn][0], acc[j][nn][1], acc[j][nn][2], acc[j][nn][3]);
      if (g == 0) rec[(size_t)NFC * SW + slot] = racc[j][0];
    }
  }
  // sum g over the segment: the threads' shares added in row order (a fixed
  // order, so that repeated runs give the same bits)
  *reinterpret_cast<float4*>(&S.gsum[tid >> 2][8 * (tid & 3)]) = make_float4(gpart[0], gpart[1], gpart[2], gpart[3]);
  *reinterpret_cast<float4*>(&S.gsum[tid >> 2][8 * (tid & 3) + 4]) = make_float4(gpart[4], gpart[5], gpart[6], gpart[7]);
  __syncthreads();
  if (tid < SW) {
    float gs = 0.f;
    for (int r = 0; r < C; ++r) gs += S.gsum[r][tid];
    rec[(size_t)NFC * SW + NFC + tid] = gs;
  }
}

// DEC: the decayed variant.  The suffix state R (and r, the sum of g) is
// kept relative to the start of the chunk after the current one: key p of
// the chunk reads it times gamma^(C - p), the in-chunk terms carry
// gamma^(i - j), and the update is R <- gamma^C R + sum_p gamma^p
// phi(q_p) g_p^T; the later segments' increments are decayed over the
// distance to this segment's end.
template <int DEC>
__global__ __launch_bounds__(NTHR, 2) void key_pass_kernel(Params p) {
  __shared__ KSmem S;
  const Unit un = unit_of(p);
  const size_t bh = un.bh;
  const int s = un.s;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_index(), g = lane >> 4, r16 = lane & 15;
  const int kpos = 16 * w + r16;  // key of the lane in transposed tiles
  const int L = p.L;
  const float lg = DEC ? decay_lg2_clamped(__log2f(p.gamma[bh % p.H])) : 0.f;
  const float wkey = DEC ? gpow(lg, (float)(C - kpos)) : 1.f;  // the suffix state's weight at this key
  if constexpr (DEC) {
    for (int j = tid; j < 4 * 64; j += NTHR) {
      const int t = j >> 6, l = j & 63, d0 = 16 * t + 4 * (l >> 4) - (l & 15);
      float4 wv;
      wv.x = d0 >= 0 ? gpow(lg, (float)d0) : 0.f;
      wv.y = d0 >= -1 ? gpow(lg, (float)(d0 + 1)) : 0.f;
      wv.z = d0 >= -2 ? gpow(lg, (float)(d0 + 2)) : 0.f;
      wv.w = d0 >= -3 ? gpow(lg, (float)(d0 + 3)) : 0.f;
      *reinterpret_cast<float4*>(&S.dw[t][l][0]) = wv;
    }
    for (int j = tid; j < C; j += NTHR) {
      S.wqf[j] = gpow(lg, (float)j);
      S.wq[j] = (half_t)S.wqf[j];
    }
  }

  for (int e = tid; e < NFP * RS / 2; e += NTHR) reinterpret_cast<uint32_t*>(&S.rf[0][0])[e] = 0u;
  for (int e = tid; e < NF; e += NTHR) S.rs[e] = 0.f;
  for (int e = tid; e < XT; e += NTHR) S.qt[DK][e] = (half_t)1.f;
  if (tid < SW) S.g0[tid] = 0.f;
  // state R of the owned compact slot tiles; r as one value per lane and
  // tile (slot 16 t + r16: the rows of an r tile are all equal)
  const int nown = cown_count<false>(w);
  uint32_t si[MAXC];
  slot_info<false>(w, r16, si);
  f32x4 acc[MAXC][2];
  float racc[MAXC];
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    racc[j] = 0.f;
  }
  float up = 1.f;
  // largest state magnitude over the workgroup -> scale; both state copies to
  // LDS (each slot to its one or two rows)
  auto publish = [&]() {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < MAXC; ++j)
      if (j < nown)
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[j][nn][i]));
    mx = wave_max_abs(mx);
    if (lane == 0) S.wmax[w] = mx;
    __syncthreads();  // every read of the state copies and the chunk buffers done
    const int e = scale_exp(fmaxf(fmaxf(S.wmax[0], S.wmax[1]), fmaxf(S.wmax[2], S.wmax[3])));
    const float down = __builtin_amdgcn_ldexpf(1.f, -e);
    up = __builtin_amdgcn_ldexpf(1.f, e);
    auto store_copy = [&](auto scaled) {  // as in the query pass
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        if (j < nown) {
          const int r1 = sl_r1(si[j]);
          const uint32_t r2 = sl_r2(si[j]);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            f32x4 a = acc[j][nn];
            if constexpr (decltype(scaled)::value) a *= down;
            const f16x2 h01 = __builtin_convertvector((f32x2{a[0], a[1]}), f16x2);
            const f16x2 h23 = __builtin_convertvector((f32x2{a[2], a[3]}), f16x2);
            *reinterpret_cast<uint2*>(&S.rf[r1][16 * nn + 4 * g]) = make_uint2(u32(h01), u32(h23));
            if (r2 != NOROW) *reinterpret_cast<uint2*>(&S.rf[r2][16 * nn + 4 * g]) = make_uint2(u32(h01), u32(h23));
          }
          if (g == 0) {
            S.rs[r1] = racc[j];
            if (r2 != NOROW) S.rs[r2] = racc[j];
          }
        }
      }
    };
    if (__builtin_amdgcn_readfirstlane(e) != 0) store_copy(std::true_type{});
    else store_copy(std::false_type{});
  };
  // the state after the segment: the sum of the increments of the later segments
  if (un.seg < p.nseg - 1) {
    float g0 = 0.f;
    const int sc = (p.seg_chunks + p.ksplit - 1) / p.ksplit;
    for (int rr = (un.seg + 1) * p.ksplit; rr < p.nseg * p.ksplit; ++rr) {
      const int r = rr / p.ksplit, sub = rr % p.ksplit;
      const float* rec = p.krec + (((bh * p.nslice + s) * p.nseg + r) * p.ksplit + sub) * (size_t)RREC;
      // decayed: part sub of segment r starts (r - seg - 1) segments and sub
      // parts after this one ends
      const float wr = DEC ? gpow(lg, (float)((r - un.seg - 1) * p.seg_chunks * C + sub * sc * C)) : 1.f;
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        if (j < nown) {
          const int slot = 16 * cown_tile(w, j) + r16;
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            const float4 x = *reinterpret_cast<const float4*>(rec + (size_t)slot * SW + 16 * nn + 4 * g);
            acc[j][nn] += wr * f32x4{x.x, x.y, x.z, x.w};
          }
          racc[j] += wr * rec[(size_t)NFC * SW + slot];
        }
      }
      if (tid < SW) g0 += wr * rec[(size_t)NFC * SW + NFC + tid];
    }
    if (tid < SW) S.g0[tid] = g0;
    publish();
  }
  const int last = un.t_begin + ((un.t_end - 1 - un.t_begin) / C) * C;
  const HeadRsrc rs = head_rsrc(p, bh, p.den, p.h + (size_t)s * p.npos);
  Pre pf;
  k_load(p, rs, s, last, pf);
  __syncthreads();
  k_store(S, pf);
  const f16x8 zero8 = {};

  for (int t0 = last; t0 >= un.t_begin; t0 -= C) {
    const int n = min(C, un.t_end - t0);
    __syncthreads();  // chunk inputs and the state copies visible
    if (t0 - C >= un.t_begin) k_load(p, rs, s, t0 - C, pf);

    float kf[DK];
    {
      const f16x8 k0 = ld8(&S.kh[kpos][0]), k1 = ld8(&S.kh[kpos][8]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kf[i] = (float)k0[i];
        kf[8 + i] = (float)k1[i];
      }
    }
    // ---- dk from the state: u^T = R-readout with v_j, lane-local contraction
    // (the r share is added before the store)
    // (the copy's scale 2^e rides on the k factors: exact, a power of two)
    // (decayed: the suffix state's weight at this key rides along)
    const float upk = DEC ? up * wkey : up;
    f32x4 dka = {0.f, 0.f, 0.f, 0.f};
    const f16x8 vb = ld8(&S.vh[kpos][8 * g]);
#pragma unroll
    for (int m = 0; m < NFT; ++m) {
      f32x4 u = {0.f, 0.f, 0.f, 0.f};
      u = mfma(ld8(&S.rf[16 * m + r16][8 * g]), vb, u);
      dka += u * (m == 0 ? upk : kf[m - 1] * upk);
    }
    // ---- dv from the state: R^T phi~(k_j) with phi~ = [k_a, k_a k_b / 2], plus sum g
    f32x4 dva[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      const f16x8 kb8 = ld8(&S.kh[kpos][8 * (g & 1)]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int mt = 2 * ks + (g >> 1);  // feature tile of this lane group's 8 features
        f16x8 fb = zero8;
        if (mt == 0) {
          fb = kb8;
        } else if (mt <= 16) {
          const _Float16 ka = S.kh[kpos][mt - 1] * (_Float16)0.5f;
          fb = kb8 * ka;
        }
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) dva[nn] = mfma(tr8(&S.rf[0][0], 32 * ks + 8 * g, 16 * nn, RS), fb, dva[nn]);
      }
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const float4 g4 = *reinterpret_cast<const float4*>(&S.g0[16 * nn + 4 * g]);
        dva[nn] = dva[nn] * up + f32x4{g4.x, g4.y, g4.z, g4.w};
        if constexpr (DEC) dva[nn] *= wkey;
      }
    }
    // ---- in-chunk terms: queries i >= j in the query tiles m >= w
    {
      const f16x8 kv = g < 2 ? ld8(&S.kh[kpos][8 * g]) : zero8;
      f32x4 cw[4], aw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        cw[m] = aw[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m >= w) {
          const f16x8 qa = g < 2 ? ld8(&S.qh[16 * m + r16][8 * g]) : zero8;
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          x = mfma(qa, kv, x);  // [query 16m + 4g + i][key]
          f32x4 da = {0.f, 0.f, 0.f, 0.f};
          da = mfma(ld8(&S.gh[16 * m + r16][8 * g]), vb, da);
          da = mfma(ld8(&S.gl[16 * m + r16][8 * g]), vb, da);
          const float4 h4 = *reinterpret_cast<const float4*>(&S.hs[16 * m + 4 * g]);
          const float hq[4] = {h4.x, h4.y, h4.z, h4.w};
          if constexpr (DEC) {  // gamma^(query - key), zero for a query before the key
            const float4 dv4 = *reinterpret_cast<const float4*>(&S.dw[m - w][lane][0]);
            const float wt[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float xx = x[i];
              aw[m][i] = wt[i] * (1.f + xx + 0.5f * xx * xx);
              cw[m][i] = wt[i] * (da[i] + hq[i]) * (1.f + xx);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool keep = m > w || 4 * g + i >= r16;
              const float xx = x[i];
              aw[m][i] = keep ? 1.f + xx + 0.5f * xx * xx : 0.f;
              cw[m][i] = keep ? (da[i] + hq[i]) * (1.f + xx) : 0.f;
            }
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb + 1 >= w) {
          f16x8 ch, cl, ah, al;
          split8(cw[2 * kb], cw[2 * kb + 1], ch, cl);
          split8(aw[2 * kb], aw[2 * kb + 1], ah, al);
          const f16x8 qa = cat44(&S.qt[r16][32 * kb + 4 * g], &S.qt[r16][32 * kb + 16 + 4 * g]);
          dka = mfma(qa, ch, dka);
          dka = mfma(qa, cl, dka);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            const f16x8 gah = tr44(&S.gh[0][0], 32 * kb + 4 * g, 16 * nn, RS);
            const f16x8 gal = tr44(&S.gl[0][0], 32 * kb + 4 * g, 16 * nn, RS);
            dva[nn] = mfma(gah, ah, dva[nn]);
            dva[nn] = mfma(gah, al, dva[nn]);
            dva[nn] = mfma(gal, ah, dva[nn]);
          }
        }
      }
    }
    // the r share of dk[a], a = 4g + i: r_lin[a] + sum_b r[(a, b)] k_b (r is
    // symmetric in (a, b)), from the fp32 copy of r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = 4 * g + i;
      float rk = S.rs[a];
#pragma unroll
      for (int b = 0; b < DK; b += 8) {
        const f16x8 k8 = ld8(&S.kh[kpos][b]);
        const float4 r0 = *reinterpret_cast<const float4*>(&S.rs[DK + DK * a + b]);
        const float4 r1 = *reinterpret_cast<const float4*>(&S.rs[DK + DK * a + b + 4]);
        rk += r0.x * (float)k8[0] + r0.y * (float)k8[1] + r0.z * (float)k8[2] + r0.w * (float)k8[3] +
              r1.x * (float)k8[4] + r1.y * (float)k8[5] + r1.z * (float)k8[6] + r1.w * (float)k8[7];
      }
      dka[i] += DEC ? rk * wkey : rk;
    }
    if (kpos < n) {
      float* dst = (p.nslice == 1 ? p.gk : p.pk + (size_t)s * p.npos * DK) + ((size_t)bh * L + t0 + kpos) * DK + 4 * g;
      // gradients leave non-temporally (straight to memory, not kept in L2):
      // 360M backward 206.7 -> 204.5 us, decayed 218.0 -> 214.9 us
      __builtin_nontemporal_store(dka, reinterpret_cast<f32x4*>(dst));
      float* dv = p.gv + ((size_t)bh * L + t0 + kpos) * p.dvf + (size_t)s * SW + 4 * g;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
        __builtin_nontemporal_store(dva[nn], reinterpret_cast<f32x4*>(dv + 16 * nn));
    }

    // ---- state update with the chunk (none after the segment's first, the
    // last one processed): R^T += G^T phi(Q), r += phi(Q)^T h
    // (decayed: R^T <- gamma^C R^T + G^T diag(gamma^p) phi(Q), r likewise)
    if (t0 - C < un.t_begin) break;  // uniform
    const float gC = DEC ? gpow(lg, (float)C) : 1.f;
    if constexpr (DEC) {
#pragma unroll
      for (int j = 0; j < MAXC; ++j) {
        acc[j][0] *= gC;
        acc[j][1] *= gC;
        racc[j] *= gC;
      }
    }
#pragma unroll
    for (int j = 0; j < MAXC; ++j) {
      if (j < nown) {  // uniform branch
        // g and h rounded once to fp16 (the state is read back as an fp16 copy)
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 fb = ld8(&S.qt[sl_a(si[j])][32 * ks + 8 * g]) * ld8(&S.qt[sl_b(si[j])][32 * ks + 8 * g]);
          if constexpr (DEC) fb *= ld8(&S.wq[32 * ks + 8 * g]);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
            acc[j][nn] = mfma(tr8(&S.gh[0][0], 32 * ks + 8 * g, 16 * nn, RS), fb, acc[j][nn]);
          t = mfma(ld8(&S.hh[32 * ks + 8 * g]), fb, t);
        }
        racc[j] += t[0];
      }
    }
    {
      // this chunk's column sums of g, eight rows per thread
      const int c = tid & (SW - 1), part = tid / SW;
      float gs = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float gr = (float)S.gh[8 * part + r][c] + (float)S.gl[8 * part + r][c];
        gs += DEC ? S.wqf[8 * part + r] * gr : gr;
      }
      S.gpart[part][c] = gs;
    }
    publish();
    if (tid < SW) {
      const int t = tid_here();
      float gsum = 0.f;
#pragma unroll
      for (int part = 0; part < 8; ++part) gsum += S.gpart[part][t];
      S.g0[t] = DEC ? gC * S.g0[t] + gsum : S.g0[t] + gsum;
    }
    if (t0 - C >= un.t_begin) k_store(S, pf);
  }
}

}  // namespace bwdm

hipError_t launch_linattn_bwd_mfma(const LinattnBwdArgs& a, hipStream_t s) {
  using namespace bwdm;
  if ((size_t)a.L * a.dv * 4 >= (size_t)1 << 31) return hipErrorInvalidValue;  // 32-bit buffer offsets
  const size_t BH = (size_t)a.B * a.H, npos = BH * a.L;
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y; p.dy = a.dy;
  p.den = (float*)a.workspace;
  p.h = p.den + npos;
  p.npos = npos;
  p.gq = a.gq; p.gk = a.gk; p.gv = a.gv;
  p.L = a.L; p.dvf = a.dv; p.nslice = a.dv / SW;
  p.gamma = a.gamma;
  p.H = a.H;
  linattn_bwd_mfma_plan((int)BH, a.L, a.dv, &p.nseg, &p.seg_chunks);
  float* part = p.h + (size_t)p.nslice * npos;
  if (p.nslice > 1) {
    p.pq = part;
    p.pk = part + (size_t)p.nslice * npos * DK;
    part += (size_t)2 * p.nslice * npos * DK;
  }
  p.rsplit = linattn_bwd_rec_split((int)BH, p.nseg, p.seg_chunks);
  p.ksplit = linattn_bwd_key_split((int)BH, a.dv, p.nseg, p.seg_chunks);
  const int nrec_seg = p.nseg * p.rsplit;  // forward-record sub-segments per head
  float* frec = part;
  p.frec = frec;
  p.frecz = frec + BH * nrec_seg * (size_t)(NFC + 1) * a.dv;
  p.krec = const_cast<float*>(p.frecz) + BH * nrec_seg * (size_t)(NFC + 1);
  const unsigned grid = (unsigned)(BH * p.nslice * p.nseg);
  const size_t n4 = npos * DK / 4, cblocks = (n4 + 255) / 256;
  if (p.nseg > 1) {
    // the sub-segments before the last segment (no segment reads the last one's)
    if (hipError_t e = launch_linattn_state_records(a.k, a.v, frec, (int)BH, a.L, a.dv, nrec_seg,
                                                    p.seg_chunks / p.rsplit, (p.nseg - 1) * p.rsplit, a.gamma,
                                                    a.H, s);
        e != hipSuccess)
      return e;
  }
  const bool dec = a.gamma != nullptr;
  if (dec) hipLaunchKernelGGL(query_pass_kernel<1>, dim3(grid), dim3(NTHR), 0, s, p);
  else hipLaunchKernelGGL(query_pass_kernel<0>, dim3(grid), dim3(NTHR), 0, s, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (p.nseg > 1) {
    const unsigned kgrid = (unsigned)(BH * p.nslice * (1 + (p.nseg - 1) * p.ksplit));
    if (dec) hipLaunchKernelGGL(key_state_kernel<1>, dim3(kgrid), dim3(NTHR), 0, s, p);
    else hipLaunchKernelGGL(key_state_kernel<0>, dim3(kgrid), dim3(NTHR), 0, s, p);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  if (dec) hipLaunchKernelGGL(key_pass_kernel<1>, dim3(grid), dim3(NTHR), 0, s, p);
  else hipLaunchKernelGGL(key_pass_kernel<0>, dim3(grid), dim3(NTHR), 0, s, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (p.nslice > 1) {
    // with several segments the suffix-state pass has summed dq
    hipLaunchKernelGGL(slice_sum_kernel, dim3((unsigned)(cblocks < 8192 ? cblocks : 8192)), dim3(256), 0, s,
                       p.nseg > 1 ? nullptr : reinterpret_cast<const float4*>(p.pq),
                       reinterpret_cast<const float4*>(p.pk),
                       reinterpret_cast<float4*>(p.gq), reinterpret_cast<float4*>(p.gk), n4, p.nslice);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace based
