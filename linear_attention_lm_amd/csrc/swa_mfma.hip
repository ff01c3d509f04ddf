// Causal sliding-window softmax attention on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation): the bf16 path of
// based_swa_fwd.
//
// Definition (HazyResearch/based README, introduction: exact softmax
// attention over a short window of recent tokens): row i attends to
// positions max(0, i - window + 1) .. i with weights exp(s_j - max s) / sum,
// s_j = scale * q_i.k_j.
//
// Layout of the work: a workgroup (4 wavefronts) walks a segment of a
// (batch, head) sequence in blocks of 64 queries.  The keys/values of the
// current and the previous block sit in an LDS ring, row-major (each K/V row
// is read from HBM once per segment); the next block's keys, values and
// queries are loaded into registers while the current block computes.
// Wavefront w owns queries 16w..16w+15 of the block, whose keys span 5 tiles
// of 16.  Scores are computed transposed (keys x queries) so that each lane
// holds 4 keys of one query: the softmax row statistics need only
// in-register work plus two cross-lane steps, and the probabilities already
// sit in the B-operand layout of the product Y^T = V^T P^T (keys permuted
// consistently in V^T, which the transposing LDS load ds_read_b64_tr_b16
// reads from the row-major ring: within each 16-lane block, lane t receives
// element t % 4 of the 4-element row segments addressed by lanes t / 4 + 4i).
// Y^T leaves each lane with 4 consecutive columns of one query: 16-byte
// stores.  P is fp32; it enters the product as hi + lo bf16 (exact to ~16
// bits), V is exact in bf16.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace swa_mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = 64;         // queries per block
constexpr int NTHR = 256;      // 4 wavefronts
constexpr int RING = 2 * QB;   // key positions held in LDS
constexpr int SEG_BLOCKS = 8;  // query blocks per workgroup

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// hi + lo bf16 split of two fp32 values, packed: hi = RNE(x), lo = RNE(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
}

constexpr int RSRC_DW3 = 0x00020000;
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Transposing read: rows r0 .. r0 + 3 of column c0 + (lane % 16) of the
// row-major 16-bit array at `base` (row stride ld); lane j of each 16-lane
// block addresses row r0 + j / 4, columns c0 + 4 (j % 4) .. + 3.
__device__ __forceinline__ uint2 tr4(const bf16_t* base, int r0, int c0, int ld) {
  const int j = threadIdx.x & 15;
  const bf16_t* a = base + (r0 + (j >> 2)) * ld + c0 + 4 * (j & 3);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)a);
  return __builtin_bit_cast(uint2, v);
}

// One block's keys, values and queries on their way from HBM to the ring
// (k and q: d_qk <= 128, at most 4 16-byte pieces per thread).
template <int NT>
struct Pre {
  static constexpr int NV = (NT + 1) / 2;  // 16-byte pieces of v per thread
  uint4 k[4];
  uint4 v[NV];
  uint4 q[4];  // the lane's query row, dims 8g .. in steps of 32
};

struct Params {
  const bf16_t* q; const bf16_t* k; const bf16_t* v; float* y;
  int L, dqk, window, nseg;
  float scale;
};

// Dynamic LDS: k ring [RING][dqk + 8] bf16, then v ring [RING][DV + 8] bf16.
template <int NT>
__global__ __launch_bounds__(NTHR, 2) void swa_mfma_kernel(Params p) {
  constexpr int DV = 16 * NT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int ks_stride = p.dqk + 8;
  bf16_t* kring = reinterpret_cast<bf16_t*>(smem);
  constexpr int VRS = DV + 8;  // v ring row stride (bf16)
  bf16_t* vring = kring + RING * ks_stride;

  const size_t bh = blockIdx.x / p.nseg;
  const int seg = blockIdx.x % p.nseg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int nblk = (p.L + QB - 1) / QB;
  const int b_begin = seg * SEG_BLOCKS, b_end = min(nblk, b_begin + SEG_BLOCKS);

  const int qbytes = p.L * p.dqk * 2;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + bh * p.L * p.dqk), (short)0, qbytes, RSRC_DW3);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + bh * p.L * p.dqk), (short)0, qbytes, RSRC_DW3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + bh * (size_t)p.L * DV), (short)0, p.L * DV * 2, RSRC_DW3);

  // Keys/values of block b (positions 64b .. 64b+63; positions outside
  // 0..L-1 read as zero and are masked later) and the lane's query row of
  // block b into registers; then into the ring.
  const int kchunks = QB * p.dqk / 8;  // 16-byte pieces of a k block
  auto load_block = [&](int b, Pre<NT>& pr) {
    const int pos0 = b * QB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + NTHR * i;
      const int j = u / (p.dqk / 8), c8 = u % (p.dqk / 8);
      pr.k[i] = u < kchunks && pos0 + j >= 0 ? bload(rk, ((pos0 + j) * p.dqk + 8 * c8) * 2) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Pre<NT>::NV; ++i) {
      const int u = tid + NTHR * i;
      const int j = u / (DV / 8), c8 = u % (DV / 8);
      pr.v[i] = u < QB * DV / 8 && pos0 + j >= 0 ? bload(rv, ((pos0 + j) * DV + 8 * c8) * 2) : make_uint4(0, 0, 0, 0);
    }
    const int qi = pos0 + 16 * w + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * i + 8 * g;
      pr.q[i] = d < p.dqk && qi >= 0 ? bload(rq, (qi * p.dqk + d) * 2) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_block = [&](int b, const Pre<NT>& pr) {
    const int pos0 = b * QB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = tid + NTHR * i;
      const int j = u / (p.dqk / 8), c8 = u % (p.dqk / 8);
      if (u < kchunks) *reinterpret_cast<uint4*>(&kring[((pos0 + j) & (RING - 1)) * ks_stride + 8 * c8]) = pr.k[i];
    }
#pragma unroll
    for (int i = 0; i < Pre<NT>::NV; ++i) {
      const int u = tid + NTHR * i;
      const int j = u / (DV / 8), c8 = u % (DV / 8);
      if (u < QB * DV / 8) *reinterpret_cast<uint4*>(&vring[((pos0 + j) & (RING - 1)) * VRS + 8 * c8]) = pr.v[i];
    }
  };

  Pre<NT> pr;
  uint4 qcur[4];
  if (b_begin < b_end) {
    load_block(b_begin - 1, pr);
    store_block(b_begin - 1, pr);
    load_block(b_begin, pr);
    store_block(b_begin, pr);
  }
  const bf16x8 zero8 = {};
  for (int b = b_begin; b < b_end; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) qcur[i] = pr.q[i];  // this block's queries (pr receives the next block)
    __syncthreads();  // block b's keys and values in the ring
    if (b + 1 < b_end) load_block(b + 1, pr);

    const int q0 = b * QB + 16 * w;  // first query of this wavefront
    const int qi = q0 + r16;         // the query column this lane holds
    // scores X^T (keys x queries) for the 5 key tiles of 16 ending at q0 + 15
    f32x4 x[5];
#pragma unroll
    for (int m = 0; m < 5; ++m) x[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * i + 8 * g;
      if (32 * i >= p.dqk) break;
      const bf16x8 qv = d < p.dqk ? __builtin_bit_cast(bf16x8, qcur[i]) : zero8;
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const int key = q0 - 64 + 16 * m + r16;
        const bf16x8 kv = d < p.dqk ? *reinterpret_cast<const bf16x8*>(&kring[(key & (RING - 1)) * ks_stride + d]) : zero8;
        x[m] = mfma(kv, qv, x[m]);
      }
    }
    // softmax statistics of query qi over its window
    float mx = -INFINITY;
    float s[5][4];
#pragma unroll
    for (int m = 0; m < 5; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = q0 - 64 + 16 * m + 4 * g + i;
        const bool ok = key <= qi && key > qi - p.window && key >= 0;
        s[m][i] = ok ? p.scale * x[m][i] : -INFINITY;
        mx = fmaxf(mx, s[m][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float den = 0.f;
    bf16x4 ph[6], pl[6];
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e[i] = s[m][i] == -INFINITY ? 0.f : __expf(s[m][i] - mx);
        den += e[i];
      }
      uint2 h, l;
      split2(e[0], e[1], h.x, l.x);
      split2(e[2], e[3], h.y, l.y);
      ph[m] = __builtin_bit_cast(bf16x4, h);
      pl[m] = __builtin_bit_cast(bf16x4, l);
    }
    ph[5] = bf16x4{};
    pl[5] = bf16x4{};
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);

    // Y^T = V^T P^T over the three 32-key blocks (tile pairs (0,1), (2,3), (4,-))
    f32x4 acc[NT];
#pragma unroll
    for (int nn = 0; nn < NT; ++nn) acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      bf16x8 ah, al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ah[i] = ph[2 * kb][i]; ah[4 + i] = ph[2 * kb + 1][i];
        al[i] = pl[2 * kb][i]; al[4 + i] = pl[2 * kb + 1][i];
      }
      // keys of K slots 0..3 and (kb < 2) 4..7, 16 later; ring rows of 4 never wrap
      const int k0 = (q0 - 64 + 32 * kb + 4 * g) & (RING - 1);
#pragma unroll
      for (int nn = 0; nn < NT; ++nn) {
        const uint2 v0 = tr4(vring, k0, 16 * nn, VRS);
        const uint2 v1 = kb < 2 ? tr4(vring, (k0 + 16) & (RING - 1), 16 * nn, VRS) : make_uint2(0u, 0u);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        acc[nn] = mfma(va, ah, acc[nn]);  // [column 16nn + 4g + i][query qi]
        acc[nn] = mfma(va, al, acc[nn]);
      }
    }
    if (qi < p.L) {
      const float rden = __builtin_amdgcn_rcpf(den);
      float* yrow = p.y + (bh * p.L + qi) * DV + 4 * g;
#pragma unroll
      for (int nn = 0; nn < NT; ++nn)
        *reinterpret_cast<float4*>(yrow + 16 * nn) =
            make_float4(acc[nn][0] * rden, acc[nn][1] * rden, acc[nn][2] * rden, acc[nn][3] * rden);
    }
    __syncthreads();  // every read of the ring slot of block b-1 done
    if (b + 1 < b_end) store_block(b + 1, pr);
  }
}

template <int NT>
static hipError_t launch_nt(const SwaArgs& a, hipStream_t s) {
  constexpr int DV = 16 * NT;
  Params p{};
  p.q = (const bf16_t*)a.q; p.k = (const bf16_t*)a.k; p.v = (const bf16_t*)a.v; p.y = a.y;
  p.L = a.L; p.dqk = a.dqk; p.window = a.window; p.scale = a.scale;
  const int nblk = (a.L + QB - 1) / QB;
  p.nseg = (nblk + SEG_BLOCKS - 1) / SEG_BLOCKS;
  const size_t lds = (size_t)RING * (a.dqk + 8) * 2 + (size_t)RING * (DV + 8) * 2;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)swa_mfma_kernel<NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(swa_mfma_kernel<NT>, dim3((unsigned)(a.B * a.H * p.nseg)), dim3(NTHR), lds, s, p);
  return hipGetLastError();
}

}  // namespace swa_mfma

hipError_t launch_swa_mfma(const SwaArgs& a, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  switch (a.dv) {
    case 16: return swa_mfma::launch_nt<1>(a, s);
    case 32: return swa_mfma::launch_nt<2>(a, s);
    case 48: return swa_mfma::launch_nt<3>(a, s);
    case 64: return swa_mfma::launch_nt<4>(a, s);
    case 80: return swa_mfma::launch_nt<5>(a, s);
    case 96: return swa_mfma::launch_nt<6>(a, s);
    case 112: return swa_mfma::launch_nt<7>(a, s);
    case 128: return swa_mfma::launch_nt<8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace based
