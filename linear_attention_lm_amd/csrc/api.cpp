// C ABI of the Based layer: argument validation and dispatch to the kernels.
// Every check runs on the host before anything is enqueued; a failed check
// returns a negative status and touches no memory.
#include "../../include/based.h"

#include <hip/hip_runtime.h>

#include <initializer_list>

#include "launchers.h"

#define BASED_API extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dv(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Span a, Span b) { return a.lo && b.lo && a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

size_t elem_size(int dtype) { return dtype == BASED_BF16 ? 2 : 4; }

// Every per-(batch, head) block of an [L, d] tensor spans fewer than 2^31
// bytes even in fp32: the kernels address a head's rows through 32-bit
// buffer offsets.
bool head_extent_ok(long long L, long long d) { return L * d * 4 < (1LL << 31); }

// The forward's state arguments: S_out is S_in itself (in-place update) or
// shares no byte with it, z_out likewise with z_in; no other overlap among
// the four, with the workspace, or (for the outputs) with the inputs ins.
int check_states(const float* S_in, const float* z_in, const float* S_out, const float* z_out, size_t BH, int d_v,
                 const Span* ins, int nins, Span ws) {
  const Span si = span(S_in, BH * BASED_DPHI * d_v * 4), zi = span(z_in, BH * BASED_DPHI * 4);
  const Span so = span(S_out, BH * BASED_DPHI * d_v * 4), zo = span(z_out, BH * BASED_DPHI * 4);
  if (overlap(so, si) && S_out != S_in) return BASED_ERR_ALIAS;
  if (overlap(zo, zi) && z_out != z_in) return BASED_ERR_ALIAS;
  if (overlap(so, zi) || overlap(zo, si) || overlap(so, zo)) return BASED_ERR_ALIAS;
  for (int i = 0; i < nins; ++i)
    if (overlap(so, ins[i]) || overlap(zo, ins[i])) return BASED_ERR_ALIAS;
  for (const Span& s : {si, zi, so, zo})
    if (overlap(ws, s)) return BASED_ERR_ALIAS;
  for (int i = 0; i < nins; ++i)
    if (overlap(ws, ins[i])) return BASED_ERR_ALIAS;
  return BASED_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? BASED_OK : BASED_ERR_HIP; }

}  // namespace

BASED_API int based_abi_version(void) { return BASED_ABI_VERSION; }

BASED_API const char* based_status_string(int status) {
  switch (status) {
    case BASED_OK: return "ok";
    case BASED_ERR_NULL: return "a required pointer is NULL";
    case BASED_ERR_SHAPE: return "a size is out of range";
    case BASED_ERR_UNSUPPORTED: return "unsupported head dimension (d_k must be 16; d_v, d_qk multiples of 16 up to 128)";
    case BASED_ERR_DTYPE: return "dtype must be BASED_F32 or BASED_BF16";
    case BASED_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case BASED_ERR_WORKSPACE: return "workspace missing or too small";
    case BASED_ERR_WINDOW: return "window must be in 1..64";
    case BASED_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case BASED_ERR_ALIAS: return "an output overlaps an input";
  }
  return "unknown status";
}

BASED_API size_t based_linattn_workspace_bytes(int B, int H, int L, int d_k, int d_v, int dtype) {
  if (dtype != BASED_BF16 || B < 1 || H < 1 || L < 0 || d_k != BASED_DK) return 0;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return 0;
  return based::linattn_mfma_workspace(B, H, L, d_v);
}

BASED_API int based_linattn_fwd(const void* q, const void* k, const void* v, float* y, const float* S_in,
                                const float* z_in, float* S_out, float* z_out, int B, int H, int L, int d_k,
                                int d_v, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v) || !head_extent_ok(L, d_k)) return BASED_ERR_SHAPE;
  if (L > 0 && (!q || !k || !v || !y)) return BASED_ERR_NULL;
  if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr)) return BASED_ERR_NULL;
  const void* ptrs[] = {q, k, v, y, S_in, z_in, S_out, z_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t need = based_linattn_workspace_bytes(B, H, L, d_k, d_v, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BASED_ERR_WORKSPACE;
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  const Span ys = span(y, BH * L * d_v * 4);
  const Span in[] = {span(q, BH * L * d_k * es), span(k, BH * L * d_k * es), span(v, BH * L * d_v * es),
                     span(S_in, BH * BASED_DPHI * d_v * 4), span(z_in, BH * BASED_DPHI * 4)};
  for (const Span& s : in)
    if (L > 0 && overlap(ys, s)) return BASED_ERR_ALIAS;
  const Span io[] = {in[0], in[1], in[2], ys};
  if (int st = check_states(S_in, z_in, S_out, z_out, BH, d_v, io, L > 0 ? 4 : 0, span(workspace, need));
      st != BASED_OK)
    return st;

  based::LinattnArgs a{q, k, v, y, S_in, z_in, S_out, z_out, B, H, L, d_v, workspace, workspace_bytes};
  if (L == 0 && !S_out) return BASED_OK;
  if (dtype == BASED_BF16 && based::linattn_mfma_supported(d_v))
    return status_of(based::launch_linattn_mfma(a, (hipStream_t)stream));
  return status_of(based::launch_linattn_valu(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_linattn_decay_fwd(const void* q, const void* k, const void* v, const float* gamma, float* y,
                                      const float* S_in, const float* z_in, float* S_out, float* z_out, int B, int H,
                                      int L, int d_k, int d_v, int dtype, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v) || !head_extent_ok(L, d_k)) return BASED_ERR_SHAPE;
  if (!gamma || (L > 0 && (!q || !k || !v || !y))) return BASED_ERR_NULL;
  if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr)) return BASED_ERR_NULL;
  const void* ptrs[] = {q, k, v, y, S_in, z_in, S_out, z_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t need = based_linattn_workspace_bytes(B, H, L, d_k, d_v, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BASED_ERR_WORKSPACE;
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  const Span ys = span(y, BH * L * d_v * 4);
  const Span in[] = {span(q, BH * L * d_k * es), span(k, BH * L * d_k * es), span(v, BH * L * d_v * es),
                     span(S_in, BH * BASED_DPHI * d_v * 4), span(z_in, BH * BASED_DPHI * 4), span(gamma, (size_t)H * 4)};
  for (const Span& s : in)
    if (L > 0 && overlap(ys, s)) return BASED_ERR_ALIAS;
  const Span io[] = {in[0], in[1], in[2], in[5], ys};
  if (int st = check_states(S_in, z_in, S_out, z_out, BH, d_v, io, L > 0 ? 5 : 0, span(workspace, need));
      st != BASED_OK)
    return st;
  if (L == 0 && !S_out) return BASED_OK;
  based::LinattnArgs a{q, k, v, y, S_in, z_in, S_out, z_out, B, H, L, d_v, workspace, workspace_bytes, gamma};
  if (dtype == BASED_BF16 && based::linattn_mfma_supported(d_v))
    return status_of(based::launch_linattn_decay_mfma(a, (hipStream_t)stream));
  return status_of(based::launch_linattn_valu(a, dtype == BASED_BF16, (hipStream_t)stream));
}

static int layer_fwd_impl(const void* q, const void* k, const void* v, const float* gamma, float* y_lin,
                          float* y_swa, const float* S_in, const float* z_in, float* S_out, float* z_out, int B, int H,
                          int L, int d_k, int d_v, int window, float scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if ((long long)B * H * ((L + 31) / 32) > 0x7fffffffLL) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v) || !head_extent_ok(L, d_k)) return BASED_ERR_SHAPE;
  if (window < 1 || window > BASED_MAX_WINDOW) return BASED_ERR_WINDOW;
  if (L > 0 && (!q || !k || !v || !y_lin || !y_swa)) return BASED_ERR_NULL;
  if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr)) return BASED_ERR_NULL;
  const void* ptrs[] = {q, k, v, y_lin, y_swa, S_in, z_in, S_out, z_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t need = based_linattn_workspace_bytes(B, H, L, d_k, d_v, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BASED_ERR_WORKSPACE;
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  const Span outs[] = {span(y_lin, BH * L * d_v * 4), span(y_swa, BH * L * d_v * 4)};
  const Span ins[] = {span(q, BH * L * d_k * es), span(k, BH * L * d_k * es), span(v, BH * L * d_v * es),
                      span(S_in, BH * BASED_DPHI * d_v * 4), span(z_in, BH * BASED_DPHI * 4),
                      span(S_out, BH * BASED_DPHI * d_v * 4), span(z_out, BH * BASED_DPHI * 4)};
  if (L > 0) {
    if (overlap(outs[0], outs[1])) return BASED_ERR_ALIAS;
    for (const Span& o : outs)
      for (const Span& s : ins)
        if (overlap(o, s)) return BASED_ERR_ALIAS;
  }
  const Span gs = span(gamma, (size_t)H * 4);
  const Span io[] = {ins[0], ins[1], ins[2], outs[0], outs[1], gs};
  if (L > 0 && (overlap(outs[0], gs) || overlap(outs[1], gs))) return BASED_ERR_ALIAS;
  if (int st = check_states(S_in, z_in, S_out, z_out, BH, d_v, io, L > 0 ? 6 : 0, span(workspace, need));
      st != BASED_OK)
    return st;

  based::LinattnArgs a{q, k, v, y_lin, S_in, z_in, S_out, z_out, B, H, L, d_v, workspace, workspace_bytes, gamma};
  if (L == 0 && !S_out) return BASED_OK;
  if (dtype == BASED_BF16 && based::linattn_mfma_supported(d_v))
    return status_of(based::launch_layer_mfma(a, y_swa, window, scale, (hipStream_t)stream));
  if (based::layer_valu_fused(a))
    return status_of(based::launch_layer_valu(a, y_swa, window, scale, dtype == BASED_BF16, (hipStream_t)stream));
  if (int st = status_of(based::launch_linattn_valu(a, dtype == BASED_BF16, (hipStream_t)stream)); st != BASED_OK)
    return st;
  if (L == 0) return BASED_OK;
  based::SwaArgs sa{q, k, v, y_swa, B, H, L, d_k, d_v, window, scale};
  if (dtype == BASED_BF16) return status_of(based::launch_swa_mfma(sa, (hipStream_t)stream));
  return status_of(based::launch_swa_valu(sa, false, (hipStream_t)stream));
}

BASED_API int based_layer_fwd(const void* q, const void* k, const void* v, float* y_lin, float* y_swa,
                               const float* S_in, const float* z_in, float* S_out, float* z_out, int B, int H,
                               int L, int d_k, int d_v, int window, float scale, int dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return layer_fwd_impl(q, k, v, nullptr, y_lin, y_swa, S_in, z_in, S_out, z_out, B, H, L, d_k, d_v, window, scale,
                        dtype, workspace, workspace_bytes, stream);
}

BASED_API int based_layer_decay_fwd(const void* q, const void* k, const void* v, const float* gamma, float* y_lin,
                                     float* y_swa, const float* S_in, const float* z_in, float* S_out, float* z_out,
                                     int B, int H, int L, int d_k, int d_v, int window, float scale, int dtype,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!gamma) return BASED_ERR_NULL;
  return layer_fwd_impl(q, k, v, gamma, y_lin, y_swa, S_in, z_in, S_out, z_out, B, H, L, d_k, d_v, window, scale,
                        dtype, workspace, workspace_bytes, stream);
}

BASED_API int based_swa_fwd(const void* q, const void* k, const void* v, float* y, int B, int H, int L, int d_qk,
                            int d_v, int window, float scale, int dtype, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (!valid_dv(d_qk) || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if (window < 1 || window > BASED_MAX_WINDOW) return BASED_ERR_WINDOW;
  if ((long long)B * H * ((L + 31) / 32) > 0x7fffffffLL) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v) || !head_extent_ok(L, d_qk)) return BASED_ERR_SHAPE;
  if (L == 0) return BASED_OK;
  if (!q || !k || !v || !y) return BASED_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return BASED_ERR_ALIGN;
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  const Span ys = span(y, BH * L * d_v * 4);
  if (overlap(ys, span(q, BH * L * d_qk * es)) || overlap(ys, span(k, BH * L * d_qk * es)) ||
      overlap(ys, span(v, BH * L * d_v * es)))
    return BASED_ERR_ALIAS;
  based::SwaArgs a{q, k, v, y, B, H, L, d_qk, d_v, window, scale};
  if (dtype == BASED_BF16) return status_of(based::launch_swa_mfma(a, (hipStream_t)stream));
  return status_of(based::launch_swa_valu(a, false, (hipStream_t)stream));
}

// Shared checks of the two backward entry points: inputs q, k, v (dtype), y
// and dy (fp32), outputs gq, gk, gv (fp32) that overlap nothing else.
static int check_bwd(const void* q, const void* k, const void* v, const float* y, const float* dy, const float* gq,
                     const float* gk, const float* gv, int B, int H, int L, int d_v, int dtype) {
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  if (!q || !k || !v || !y || !dy || !gq || !gk || !gv) return BASED_ERR_NULL;
  const void* ptrs[] = {q, k, v, y, dy, gq, gk, gv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const Span in[] = {span(q, BH * L * BASED_DK * es), span(k, BH * L * BASED_DK * es), span(v, BH * L * d_v * es),
                     span(y, BH * L * d_v * 4), span(dy, BH * L * d_v * 4)};
  const Span out[] = {span(gq, BH * L * BASED_DK * 4), span(gk, BH * L * BASED_DK * 4), span(gv, BH * L * d_v * 4)};
  for (int o = 0; o < 3; ++o) {
    for (const Span& s : in)
      if (overlap(out[o], s)) return BASED_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(out[o], out[o2])) return BASED_ERR_ALIAS;
  }
  return BASED_OK;
}

BASED_API size_t based_linattn_bwd_workspace_bytes(int B, int H, int L, int d_k, int d_v, int dtype) {
  if ((dtype != BASED_F32 && dtype != BASED_BF16) || B < 1 || H < 1 || L < 1 || d_k != BASED_DK || !valid_dv(d_v))
    return 0;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return 0;
  return based::linattn_bwd_workspace(B, H, L, d_v, dtype == BASED_BF16);
}

BASED_API int based_linattn_bwd(const void* q, const void* k, const void* v, const float* y, const float* dy,
                                float* dq, float* dk, float* dv, int B, int H, int L, int d_k, int d_v, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if ((long long)B * H * ((L + 63) / 64) > 0x7fffffffLL) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v)) return BASED_ERR_SHAPE;
  if (L == 0) return BASED_OK;
  if (int st = check_bwd(q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, dtype); st != BASED_OK) return st;
  const size_t need = based_linattn_bwd_workspace_bytes(B, H, L, d_k, d_v, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return BASED_ERR_WORKSPACE;
  if (workspace && need > 0) {
    const Span ws = span(workspace, need);
    const size_t BH = (size_t)B * H, es = elem_size(dtype);
    const Span all[] = {span(q, BH * L * BASED_DK * es), span(k, BH * L * BASED_DK * es), span(v, BH * L * d_v * es),
                        span(y, BH * L * d_v * 4), span(dy, BH * L * d_v * 4), span(dq, BH * L * BASED_DK * 4),
                        span(dk, BH * L * BASED_DK * 4), span(dv, BH * L * d_v * 4)};
    for (const Span& s : all)
      if (overlap(ws, s)) return BASED_ERR_ALIAS;
  }
  based::LinattnBwdArgs a{q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, workspace, workspace_bytes};
  return status_of(based::launch_linattn_bwd(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_linattn_decay_bwd(const void* q, const void* k, const void* v, const float* gamma, const float* y,
                                      const float* dy, float* dq, float* dk, float* dv, int B, int H, int L, int d_k,
                                      int d_v, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30) || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if ((long long)B * H * ((L + 63) / 64) > 0x7fffffffLL) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v)) return BASED_ERR_SHAPE;
  if (!gamma) return BASED_ERR_NULL;
  if (L == 0) return BASED_OK;
  if (int st = check_bwd(q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, dtype); st != BASED_OK) return st;
  // the vector form: den and h per position (the matrix-core form takes more, see the dispatch)
  const size_t BH = (size_t)B * H, need = 2 * BH * L * sizeof(float);
  if (!workspace || workspace_bytes < need) return BASED_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const Span g = span(gamma, (size_t)H * 4), ws = span(workspace, need);
  const Span all[] = {span(q, BH * L * BASED_DK * es), span(k, BH * L * BASED_DK * es), span(v, BH * L * d_v * es),
                      span(y, BH * L * d_v * 4), span(dy, BH * L * d_v * 4), span(dq, BH * L * BASED_DK * 4),
                      span(dk, BH * L * BASED_DK * 4), span(dv, BH * L * d_v * 4), g};
  for (const Span& s : all)
    if (overlap(ws, s)) return BASED_ERR_ALIAS;
  for (int o = 5; o < 8; ++o)
    if (overlap(all[o], g)) return BASED_ERR_ALIAS;
  based::LinattnBwdArgs a{q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, workspace, workspace_bytes, gamma};
  return status_of(based::launch_linattn_bwd(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_swa_bwd(const void* q, const void* k, const void* v, const float* y, const float* dy, float* dq,
                            float* dk, float* dv, int B, int H, int L, int d_qk, int d_v, int window, float scale,
                            int dtype, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if (d_qk != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if (window < 1 || window > BASED_MAX_WINDOW) return BASED_ERR_WINDOW;
  if ((long long)B * H * ((L + 63) / 64) > 0x7fffffffLL || (long long)L > (1LL << 30)) return BASED_ERR_SHAPE;
  if (!head_extent_ok(L, d_v)) return BASED_ERR_SHAPE;
  if (L == 0) return BASED_OK;
  if (int st = check_bwd(q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, dtype); st != BASED_OK) return st;
  based::SwaBwdArgs a{q, k, v, y, dy, dq, dk, dv, B, H, L, d_v, window, scale};
  return status_of(based::launch_swa_bwd(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_baseconv_fwd(const void* x, const void* u, const float* h, const float* bias, float* y, int B,
                                 int L, int D, int K, int dtype, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || L < 0 || D < 4) return BASED_ERR_SHAPE;
  if (D % 4 != 0 || K < 1 || K > BASED_MAX_CONV) return BASED_ERR_UNSUPPORTED;
  if ((long long)B * L > (1LL << 31) || (long long)D > (1LL << 24) ||
      (long long)B * ((L + 15) / 16) > 0x7fffffffLL)
    return BASED_ERR_SHAPE;
  if (L == 0) return BASED_OK;
  if (!x || !u || !h || !y) return BASED_ERR_NULL;
  const void* ptrs[] = {x, u, h, bias, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t n = (size_t)B * L * D, es = elem_size(dtype);
  const Span ys = span(y, n * 4);
  if (overlap(ys, span(x, n * es)) || overlap(ys, span(u, n * es)) || overlap(ys, span(h, (size_t)D * K * 4)) ||
      overlap(ys, span(bias, (size_t)D * 4)))
    return BASED_ERR_ALIAS;
  based::BaseConvArgs a{x, u, h, bias, y, B, L, D, K};
  return status_of(based::launch_baseconv(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_decode_prefill(const void* k, const void* v, void* ring_k, void* ring_v, int32_t* pos, int B,
                                   int H, int L, int d_k, int d_v, int window, int dtype, void* stream) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1 || L < 0) return BASED_ERR_SHAPE;
  if ((long long)B * H > 0x7fffffffLL) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if (window < 1 || window > BASED_MAX_WINDOW) return BASED_ERR_WINDOW;
  if (!ring_k || !ring_v || !pos || (L > 0 && (!k || !v))) return BASED_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(ring_k) || !aligned16(ring_v) || !aligned16(pos))
    return BASED_ERR_ALIGN;
  return status_of(
      based::launch_decode_prefill(k, v, ring_k, ring_v, pos, B, H, L, d_v, window, dtype == BASED_BF16,
                                   (hipStream_t)stream));
}

static int decode_step_impl(const void* q, const void* k, const void* v, const float* gamma, float* S, float* z,
                            void* ring_k, void* ring_v, int32_t* pos, float* y_lin, float* y_swa, int B, int H,
                            int d_k, int d_v, int window, float scale, int dtype, void* stream,
                            bool compact = false) {
  if (dtype != BASED_F32 && dtype != BASED_BF16) return BASED_ERR_DTYPE;
  if (B < 1 || H < 1) return BASED_ERR_SHAPE;
  if ((long long)B * H > (1LL << 30) || B > 0x7fffffff) return BASED_ERR_SHAPE;
  if (d_k != BASED_DK || !valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  if (window < 1 || window > BASED_MAX_WINDOW) return BASED_ERR_WINDOW;
  const void* ptrs[] = {q, k, v, S, z, ring_k, ring_v, pos, y_lin, y_swa};
  for (const void* p : ptrs)
    if (!p) return BASED_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t BH = (size_t)B * H, es = elem_size(dtype);
  const size_t rows = compact ? BASED_DCMP : BASED_DPHI;
  const Span outs[] = {span(S, BH * rows * d_v * 4), span(z, BH * rows * 4),
                       span(ring_k, BH * window * d_k * es), span(ring_v, BH * window * d_v * es),
                       span(pos, (size_t)B * 4), span(y_lin, BH * d_v * 4), span(y_swa, BH * d_v * 4)};
  const Span ins[] = {span(q, BH * d_k * es), span(k, BH * d_k * es), span(v, BH * d_v * es)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Span& s : ins)
      if (overlap(outs[i], s)) return BASED_ERR_ALIAS;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return BASED_ERR_ALIAS;
  }
  if (gamma) {
    const Span g = span(gamma, (size_t)H * 4);
    for (const Span& o : outs)
      if (overlap(o, g)) return BASED_ERR_ALIAS;
  }
  based::DecodeArgs a{q, k, v, S, z, ring_k, ring_v, pos, y_lin, y_swa, B, H, d_v, window, scale, gamma, compact};
  return status_of(based::launch_decode_step(a, dtype == BASED_BF16, (hipStream_t)stream));
}

BASED_API int based_decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* ring_k,
                                void* ring_v, int32_t* pos, float* y_lin, float* y_swa, int B, int H, int d_k,
                                int d_v, int window, float scale, int dtype, void* stream) {
  return decode_step_impl(q, k, v, nullptr, S, z, ring_k, ring_v, pos, y_lin, y_swa, B, H, d_k, d_v, window, scale,
                          dtype, stream);
}

BASED_API int based_decode_step_decay(const void* q, const void* k, const void* v, const float* gamma, float* S,
                                      float* z, void* ring_k, void* ring_v, int32_t* pos, float* y_lin, float* y_swa,
                                      int B, int H, int d_k, int d_v, int window, float scale, int dtype,
                                      void* stream) {
  if (!gamma) return BASED_ERR_NULL;
  return decode_step_impl(q, k, v, gamma, S, z, ring_k, ring_v, pos, y_lin, y_swa, B, H, d_k, d_v, window, scale,
                          dtype, stream);
}

BASED_API int based_decode_step_compact(const void* q, const void* k, const void* v, const float* gamma, float* S,
                                        float* z, void* ring_k, void* ring_v, int32_t* pos, float* y_lin,
                                        float* y_swa, int B, int H, int d_k, int d_v, int window, float scale,
                                        int dtype, void* stream) {
  return decode_step_impl(q, k, v, gamma, S, z, ring_k, ring_v, pos, y_lin, y_swa, B, H, d_k, d_v, window, scale,
                          dtype, stream, true);
}

static int state_convert(const float* in, const float* zin, float* out, float* zout, int B, int H, int d_v,
                         bool to_compact, void* stream) {
  if (B < 1 || H < 1 || (long long)B * H > (1LL << 30)) return BASED_ERR_SHAPE;
  if (!valid_dv(d_v)) return BASED_ERR_UNSUPPORTED;
  const void* ptrs[] = {in, zin, out, zout};
  for (const void* p : ptrs)
    if (!p) return BASED_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return BASED_ERR_ALIGN;
  const size_t BH = (size_t)B * H;
  const size_t rin = to_compact ? BASED_DPHI : BASED_DCMP, rout = to_compact ? BASED_DCMP : BASED_DPHI;
  const Span ins[] = {span(in, BH * rin * d_v * 4), span(zin, BH * rin * 4)};
  const Span outs[] = {span(out, BH * rout * d_v * 4), span(zout, BH * rout * 4)};
  for (const Span& o : outs)
    for (const Span& i : ins)
      if (overlap(o, i)) return BASED_ERR_ALIAS;
  if (overlap(outs[0], outs[1])) return BASED_ERR_ALIAS;
  return status_of(to_compact ? based::launch_state_compact(in, zin, out, zout, BH, d_v, (hipStream_t)stream)
                              : based::launch_state_expand(in, zin, out, zout, BH, d_v, (hipStream_t)stream));
}

BASED_API int based_state_compact(const float* S, const float* z, float* Sc, float* zc, int B, int H, int d_v,
                                  void* stream) {
  return state_convert(S, z, Sc, zc, B, H, d_v, true, stream);
}

BASED_API int based_state_expand(const float* Sc, const float* zc, float* S, float* z, int B, int H, int d_v,
                                 void* stream) {
  return state_convert(Sc, zc, S, z, B, H, d_v, false, stream);
}
