// Recurrent decode of the Based layer: one token per sequence per call.
//
// Per (batch b, head h), with t = pos[b] (blog post "Базированная модель,
// часть 2", paragraph on the state: a KV-state for the numerator and a
// K-state for the denominator replace the KV cache; README intro: softmax
// attention over the last 64 tokens):
//   S += phi(k) v^T, z += phi(k), y_lin = phi(q)^T S / phi(q)^T z
//   ring slot t mod W <- (k, v); y_swa = softmax window attention over t-W+1..t.
// Decayed variant (train README's decay strategy, read as a per-head factor
// on the state): S <- gamma_h S + phi(k) v^T, z <- gamma_h z + phi(k); without
// gamma the factor is 1 and the update is the same arithmetic as above.
//
// The step streams the 273 x d_v fp32 state through once (read, update,
// write back) and is bound by HBM bandwidth.  A second state layout keeps
// one row per unordered pair (a, b) of the quadratic features: 153 rows
// (constant, k_a, then the pairs a <= b), the pair row holding
// S[(a,b)] + S[(b,a)] (S[(a,a)] on the diagonal).  Every state the recurrence
// builds has S[(a,b)] = S[(b,a)], and the readout and the update only ever
// use that sum, so the compact step computes the same result from 56 % of
// the state bytes.  Layout of the work: one
// workgroup per sequence (so the position counter can be advanced race-free),
// one wavefront per head at a time (MAXW wavefronts stride over the heads).
// phi(k) and phi(q) are formed once per head into LDS.  Inside a wavefront,
// lane (rg, cg) owns columns 4cg..4cg+3 of the state rows rg + RG i: a
// wavefront instruction touches RG whole rows with 16-byte-per-lane accesses,
// each row is read and written exactly once, and rows stream in batches of NB
// with the next batch's loads in flight (the compiler would otherwise wait
// for each row's load before issuing the next, one row per round trip).  The
// ring's value rows are read the same way, four columns per lane.
#include "based_device.h"
#include "launchers.h"

namespace based {
namespace {

constexpr int MAXW = 8;  // wavefronts (heads in flight) per workgroup

// Raw buffer resources (range-checked: loads past the end read 0, stores
// past the end are dropped), so that a row's offset is a scalar operand and
// the per-lane offset stays fixed: no per-row address registers.
constexpr int RSRC_DW3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, RSRC_DW3);
}
__device__ __forceinline__ float4 bload_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Non-temporal load (cache-policy bit NT): each state row is read once per
// step, and the whole state (273 MB at 4,096 heads of d_v 64) does not fit
// the caches, so its lines are not worth keeping.  Measured 4 % faster per
// step than the default policy; non-temporal stores were slower.
__device__ __forceinline__ float4 bload_stream(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ void bstore_f4(float4 x, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, x), r, voff,
                                         soff, 0);
}

// Four consecutive elements as fp32 (one 8-byte bf16 / 16-byte fp32 load).
__device__ __forceinline__ float4 bload4(const float*, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return bload_f4(r, voff, soff);
}
__device__ __forceinline__ float4 bload4(const bf16_t*, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
                     __uint_as_float(t.y & 0xffff0000u));
}
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
                     __uint_as_float(t.y & 0xffff0000u));
}

__device__ __forceinline__ float4 fma4(float a, float4 x, float4 acc) {
  return make_float4(__builtin_fmaf(a, x.x, acc.x), __builtin_fmaf(a, x.y, acc.y), __builtin_fmaf(a, x.z, acc.z),
                     __builtin_fmaf(a, x.w, acc.w));
}

// Rows of the compact state and its pair table: compact row 1 + DK + p holds
// the pair (a, b) = (pair_a[p], pair_b[p]), a <= b, in row-major order.
constexpr int DCMP = 1 + DK + DK * (DK + 1) / 2;
struct PairTable {
  uint8_t a[DK * (DK + 1) / 2], b[DK * (DK + 1) / 2];
  constexpr PairTable() : a(), b() {
    int p = 0;
    for (int i = 0; i < DK; ++i)
      for (int j = i; j < DK; ++j) {
        a[p] = (uint8_t)i;
        b[p] = (uint8_t)j;
        ++p;
      }
  }
};
__constant__ PairTable c_pairs = PairTable();

// (key feature, query feature) of state row f, from q and k in LDS.  Full
// layout (DPHI rows): 1, x_a, then the ordered pairs x_a x_b / sqrt2.
// Compact layout (DCMP rows): 1, x_a, then the unordered pairs a <= b; a
// pair row gathers the updates of both ordered rows, so its key feature is
// sqrt2 k_a k_b off the diagonal (k_a^2 / sqrt2 on it), and the readout
// weighs it by q_a q_b / sqrt2 like either ordered row.
template <int NROW>
__device__ __forceinline__ float2 row_features(int f, const float* qv, const float* kv) {
  if (f == 0) return make_float2(1.f, 1.f);
  if (f < 1 + DK) return make_float2(kv[f - 1], qv[f - 1]);
  int a, bb;
  if constexpr (NROW == DPHI) {
    a = (f - 1 - DK) / DK;
    bb = (f - 1 - DK) % DK;
  } else {
    a = c_pairs.a[f - 1 - DK];
    bb = c_pairs.b[f - 1 - DK];
  }
  const float kf = (NROW != DPHI && a != bb) ? kv[a] * kv[bb] * SQRT2 : kv[a] * kv[bb] * INV_SQRT2;
  return make_float2(kf, qv[a] * qv[bb] * INV_SQRT2);
}

template <typename T, int DV, int NROW>
__global__ __launch_bounds__(64 * MAXW) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, float* __restrict__ S,
    float* __restrict__ z, T* __restrict__ ring_k, T* __restrict__ ring_v, int32_t* __restrict__ pos,
    float* __restrict__ y_lin, float* __restrict__ y_swa, int H, int window, float scale,
    const float* __restrict__ gamma) {
  constexpr int CG = DV / 4;                     // lanes per state row (4 columns each)
  constexpr int RG = 64 / CG;                    // rows per wavefront instruction
  constexpr int NI = (NROW + RG - 1) / RG;       // state rows per lane
  constexpr int NB = 16;                         // state rows per load batch
  constexpr int NBATCH = (NI + NB - 1) / NB;
  constexpr int NR = (64 + RG - 1) / RG;         // ring rows per lane (window <= 64)
  constexpr int RB = 8, NRB = (NR + RB - 1) / RB;  // ring rows per load batch
  constexpr int NZ = (NROW + 63) / 64;           // z rows per lane
  constexpr int ES = sizeof(T);
  __shared__ float qk_s[MAXW][2][DK];
  __shared__ float2 phi_s[MAXW][NROW];  // (phi(k)_f, phi(q)_f) of the wavefront's head
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
  const int slot = t % window;  // the ring slot of token t (it held token t - window)
  // per-lane byte offsets: row rg, columns 4cg..4cg+3 (inactive lanes past the end)
  const int voff_s = active ? (rg * DV + 4 * cg) * 4 : NROW * DV * 4;
  const int voff_r = active ? (rg * DV + 4 * cg) * ES : 64 * DV * ES;

  for (int h = wave; h < H; h += nw) {
    const size_t bh = (size_t)b * H + h;
    const float gm = gamma ? decay_clamped(gamma[h]) : 1.f;  // state decay of the head (gm * x = x exactly when 1)
    const auto rS = rsrc(S + bh * NROW * DV, NROW * DV * 4);
    const auto rZ = rsrc(z + bh * NROW, NROW * 4);
    const auto rK = rsrc(ring_k + bh * (size_t)window * DK, window * DK * ES);
    const auto rV = rsrc(ring_v + bh * (size_t)window * DV, window * DV * ES);

    // ---- loads whose latency the set-up hides: q, k, this lane's four v
    // columns, z rows lane + 64j, the ring's key rows (lane j: slot j).  The
    // slot of token t is never used: token t takes its place.
    float qr[DK], kr[DK], kk[DK];
    load_row<DK>(q + bh * DK, qr);
    load_row<DK>(k + bh * DK, kr);
    const float4 vr = active ? load4(v + bh * DV + 4 * cg) : make_float4(0.f, 0.f, 0.f, 0.f);
    float zl[NZ];
#pragma unroll
    for (int j = 0; j < NZ; ++j) zl[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rZ, lane * 4, 256 * j, 0));
#pragma unroll
    for (int d = 0; d < DK; d += 4) {
      const float4 x = bload4((const T*)nullptr, rK, lane * DK * ES, d * ES);
      kk[d] = x.x; kk[d + 1] = x.y; kk[d + 2] = x.z; kk[d + 3] = x.w;
    }
    // position held by slot `lane` (negative: never written)
    const int held = t - ((t - lane) % window + window) % window;
    const bool key_live = lane < window && held >= 0;
    if (lane == slot) {
#pragma unroll
      for (int d = 0; d < DK; ++d) kk[d] = kr[d];
    }
    // scores of the window's keys (q and the key rows are dead after this)
    float sc = -INFINITY;
    if (key_live) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < DK; ++d) acc = __builtin_fmaf(qr[d], kk[d], acc);
      sc = scale * acc;
    }
    // ring value rows rg + RG i in batches of RB: batch 0 now, the rest while summing
    auto ring_issue = [&](int bt, float4 (&buf)[RB]) {
#pragma unroll
      for (int i = 0; i < RB; ++i) buf[i] = bload4((const T*)nullptr, rV, voff_r, RG * (bt * RB + i) * DV * ES);
    };
    float4 ra[RB], rb[RB];
    ring_issue(0, ra);

    // ---- features of k and q into LDS; z += phi(k), den = phi(q).z
    if (lane < DK) {
      qk_s[wave][0][lane] = to_f32(q[bh * DK + lane]);
      qk_s[wave][1][lane] = to_f32(k[bh * DK + lane]);
    }
    __builtin_amdgcn_wave_barrier();
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < NZ; ++j) {
      const int f = lane + 64 * j;
      if (f < NROW) {
        const float2 fe = row_features<NROW>(f, qk_s[wave][0], qk_s[wave][1]);
        const float pk = fe.x, pq = fe.y;
        phi_s[wave][f] = fe;
        const float zn = gm * zl[j] + pk;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(zn), rZ, lane * 4, 256 * j, 0);
        den += pq * zn;
      }
    }
    den = wave_sum(den);

    // ---- window softmax attention over the ring
    const float m = wave_max(sc);
    const float pw = sc == -INFINITY ? 0.f : __expf(sc - m);
    const float psum = wave_sum(pw);
    p_s[wave][lane] = pw;
    __builtin_amdgcn_wave_barrier();
    {
      float4 a4 = make_float4(0.f, 0.f, 0.f, 0.f);
      auto ring_acc = [&](int bt, const float4 (&buf)[RB]) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int ii = bt * RB + i, j = rg + RG * ii;
          if (ii < NR && active && j < window) {
            const float pj = p_s[wave][j];
            // empty slots (weight 0) may hold anything
            if (pj != 0.f) a4 = fma4(pj, j == slot ? vr : buf[i], a4);
          }
        }
      };
#pragma unroll 1
      for (int bt = 0; bt < NRB; bt += 2) {
        if (bt + 1 < NRB) ring_issue(bt + 1, rb);
        ring_acc(bt, ra);
        if (bt + 1 < NRB) {
          if (bt + 2 < NRB) ring_issue(bt + 2, ra);
          ring_acc(bt + 1, rb);
        }
      }
      red_s[wave][lane] = a4;
    }
    __builtin_amdgcn_wave_barrier();
    if (active && rg == 0) {
      float4 acc = red_s[wave][lane];
      for (int r = 1; r < RG; ++r) {
        const float4 o = red_s[wave][r * CG + cg];
        acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
      }
      const float inv = 1.f / psum;
      *reinterpret_cast<float4*>(y_swa + bh * DV + 4 * cg) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    __builtin_amdgcn_wave_barrier();
    // token t enters the ring (its slot was not read above)
    if (lane < DK) ring_k[(bh * window + slot) * DK + lane] = k[bh * DK + lane];
    for (int c = lane; c < DV; c += 64) ring_v[(bh * window + slot) * DV + c] = v[bh * DV + c];

    // ---- linear attention: stream the state rows rg + RG i through once, NB
    // rows per batch with the next batch's loads in flight (rows past the end
    // read 0 and are not written)
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    {
      float4 ba[NB], bb[NB];
      auto issue = [&](int bt, float4 (&buf)[NB]) {
#pragma unroll
        for (int i = 0; i < NB; ++i) buf[i] = bload_stream(rS, voff_s, RG * (bt * NB + i) * DV * 4);
      };
      auto process = [&](int bt, const float4 (&buf)[NB]) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int f = rg + RG * (bt * NB + i);
          if (active && f < NROW) {
            const float2 ph = phi_s[wave][f];
            const float4 sd = make_float4(gm * buf[i].x, gm * buf[i].y, gm * buf[i].z, gm * buf[i].w);
            const float4 sn = fma4(ph.x, vr, sd);
            bstore_f4(sn, rS, voff_s, RG * (bt * NB + i) * DV * 4);
            num = fma4(ph.y, sn, num);
          }
        }
      };
      issue(0, ba);
#pragma unroll 1
      for (int bt = 0; bt < NBATCH; bt += 2) {
        if (bt + 1 < NBATCH) issue(bt + 1, bb);
        process(bt, ba);
        if (bt + 1 < NBATCH) {
          if (bt + 2 < NBATCH) issue(bt + 2, ba);
          process(bt + 1, bb);
        }
      }
    }
    red_s[wave][lane] = num;
    __builtin_amdgcn_wave_barrier();
    if (active && rg == 0) {
      float4 acc = red_s[wave][lane];
      for (int r = 1; r < RG; ++r) {
        const float4 o = red_s[wave][r * CG + cg];
        acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
      }
      const float inv = 1.f / den;
      *reinterpret_cast<float4*>(y_lin + bh * DV + 4 * cg) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
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
  if (a.compact)
    hipLaunchKernelGGL((decode_step_kernel<T, DV, DCMP>), dim3(a.B), dim3(64 * nw), 0, s, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.S, a.z, (T*)a.ring_k, (T*)a.ring_v, a.pos, a.y_lin, a.y_swa,
                       a.H, a.window, a.scale, a.gamma);
  else
    hipLaunchKernelGGL((decode_step_kernel<T, DV, DPHI>), dim3(a.B), dim3(64 * nw), 0, s, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.S, a.z, (T*)a.ring_k, (T*)a.ring_v, a.pos, a.y_lin, a.y_swa,
                       a.H, a.window, a.scale, a.gamma);
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

// Layout conversions of a state (n = B*H heads of rows x cols; z: cols 1).
// Compact row 1 + DK + p of pair (a, b): S[(a,b)] + S[(b,a)] (S[(a,a)]).
__global__ void state_compact_kernel(const float* __restrict__ S, float* __restrict__ Sc, size_t n, int cols) {
  const size_t total = n * DCMP * (size_t)cols;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const size_t head = e / ((size_t)DCMP * cols);
    const int r = (int)(e / cols % DCMP), c = (int)(e % cols);
    const float* src = S + head * DPHI * cols;
    float x;
    if (r < 1 + DK) {
      x = src[(size_t)r * cols + c];
    } else {
      const int a = c_pairs.a[r - 1 - DK], b = c_pairs.b[r - 1 - DK];
      x = src[(size_t)(1 + DK + DK * a + b) * cols + c];
      if (a != b) x += src[(size_t)(1 + DK + DK * b + a) * cols + c];
    }
    Sc[e] = x;
  }
}

// Full row (a, b) of a compact state: the pair row halved (the diagonal as is).
__global__ void state_expand_kernel(const float* __restrict__ Sc, float* __restrict__ S, size_t n, int cols) {
  const size_t total = n * DPHI * (size_t)cols;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
    const size_t head = e / ((size_t)DPHI * cols);
    const int r = (int)(e / cols % DPHI), c = (int)(e % cols);
    const float* src = Sc + head * DCMP * cols;
    float x;
    if (r < 1 + DK) {
      x = src[(size_t)r * cols + c];
    } else {
      const int a0 = (r - 1 - DK) / DK, b0 = (r - 1 - DK) % DK;
      const int a = a0 < b0 ? a0 : b0, b = a0 < b0 ? b0 : a0;
      const int p = a * DK - a * (a - 1) / 2 + (b - a);  // row-major index of a <= b
      x = src[(size_t)(1 + DK + p) * cols + c];
      if (a != b) x *= 0.5f;
    }
    S[e] = x;
  }
}

static unsigned conv_blocks(size_t total) {
  const size_t b = (total + 255) / 256;
  return (unsigned)(b < 16384 ? b : 16384);
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_step_t<bf16_t>(a, s) : launch_step_t<float>(a, s);
}

hipError_t launch_state_compact(const float* S, const float* z, float* Sc, float* zc, size_t n, int dv, hipStream_t s) {
  hipLaunchKernelGGL(state_compact_kernel, dim3(conv_blocks(n * DCMP * dv)), dim3(256), 0, s, S, Sc, n, dv);
  hipLaunchKernelGGL(state_compact_kernel, dim3(conv_blocks(n * DCMP)), dim3(256), 0, s, z, zc, n, 1);
  return hipGetLastError();
}

hipError_t launch_state_expand(const float* Sc, const float* zc, float* S, float* z, size_t n, int dv, hipStream_t s) {
  hipLaunchKernelGGL(state_expand_kernel, dim3(conv_blocks(n * DPHI * dv)), dim3(256), 0, s, Sc, S, n, dv);
  hipLaunchKernelGGL(state_expand_kernel, dim3(conv_blocks(n * DPHI)), dim3(256), 0, s, zc, z, n, 1);
  return hipGetLastError();
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
