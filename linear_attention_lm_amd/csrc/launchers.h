// Host-side launchers of the Based kernels; called by the C ABI after its
// argument checks.  Every launcher enqueues on `stream` and returns the HIP
// status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace based {

// Layout constants shared by the host-side planning (plan.cpp) and the
// kernels (each kernel file checks its own constants against these).
namespace layout {
constexpr int CHUNK = 64;          // positions per chunk
constexpr int FWD_SLOTS = 160;     // compact feature slots of the forward's state records
constexpr int FWD_MAX_SUM = 3;     // segments summed directly by the forward's main pass
constexpr int BWD_SLICE = 32;      // value columns per backward workgroup
constexpr int BWD_MAXSEG = 8;      // backward segments per head at most
constexpr int BWD_NF = 272;        // non-constant feature rows of the backward's states
constexpr int BWD_RREC = FWD_SLOTS * BWD_SLICE + FWD_SLOTS + BWD_SLICE;  // floats of one suffix-state record (compact slots)
}  // namespace layout

// Host-side planning (plan.cpp): sequence segments per (batch, head) and
// workspace sizes.
void linattn_mfma_plan(int BH, int L, int dv, int* nseg, int* seg_chunks);
void linattn_bwd_mfma_plan(int BH, int L, int dv, int* nseg, int* seg_chunks);
int linattn_bwd_rec_split(int BH, int nseg, int seg_chunks);
int linattn_bwd_key_split(int BH, int dv, int nseg, int seg_chunks);

struct LinattnArgs {
  const void* q; const void* k; const void* v; float* y;
  const float* S_in; const float* z_in; float* S_out; float* z_out;
  int B, H, L, dv;
  void* workspace; size_t workspace_bytes;
  const float* gamma = nullptr;  // [H] per-head state decay (decayed variant only)
};

// fp32 (and generic) chunked linear attention on the vector ALUs.
hipError_t launch_linattn_valu(const LinattnArgs& a, bool bf16, hipStream_t stream);
// Both attentions of the layer in one vector-ALU pass (short sequences
// without a state argument: layer_valu_fused), the window's output in y_swa.
bool layer_valu_fused(const LinattnArgs& a);
hipError_t launch_layer_valu(const LinattnArgs& a, float* y_swa, int window, float scale, bool bf16,
                             hipStream_t stream);

// bf16 chunked linear attention on the matrix cores (d_v in {32, 64, 96, 128}).
bool linattn_mfma_supported(int dv);
size_t linattn_mfma_workspace(int B, int H, int L, int dv);
hipError_t launch_linattn_mfma(const LinattnArgs& a, hipStream_t stream);
// The decayed variant (per-head gamma in a.gamma), same layouts and workspace.
hipError_t launch_linattn_decay_mfma(const LinattnArgs& a, hipStream_t stream);
// The state-only pass alone (zero initial state; bf16, d_v in {32, 64, 96, 128}):
// compact segment increments at ws, as the main pass's records, for the
// first nrec segments of each head (nrec <= nseg - 1); with a per-head decay
// gamma [H] (or null), each increment decayed to its segment's end.
hipError_t launch_linattn_state_records(const void* k, const void* v, float* ws, int BH, int L, int dv, int nseg,
                                        int seg_chunks, int nrec, const float* gamma, int H, hipStream_t stream);
// The same pass with the sliding-window softmax of the same q, k, v fused in
// (d_qk = d_k = 16), written to y_swa.
hipError_t launch_layer_mfma(const LinattnArgs& a, float* y_swa, int window, float scale, hipStream_t stream);

struct SwaArgs {
  const void* q; const void* k; const void* v; float* y;
  int B, H, L, dqk, dv, window; float scale;
};
hipError_t launch_swa_valu(const SwaArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_swa_mfma(const SwaArgs& a, hipStream_t stream);  // bf16 inputs

// Backward of the window softmax (d_qk = 16): gradients gq, gk, gv (fp32) of
// y with respect to q, k, v, given the forward output y and its gradient dy.
struct SwaBwdArgs {
  const void* q; const void* k; const void* v; const float* y; const float* dy;
  float* gq; float* gk; float* gv;
  int B, H, L, dv, window; float scale;
};
hipError_t launch_swa_bwd(const SwaBwdArgs& a, bool bf16, hipStream_t stream);
bool swa_bwd_mfma_supported(int dv);  // bf16, d_v in {32, 64, 96, 128}
hipError_t launch_swa_bwd_mfma(const SwaBwdArgs& a, hipStream_t stream);

// Backward of the linear attention (zero initial state), likewise.
struct LinattnBwdArgs {
  const void* q; const void* k; const void* v; const float* y; const float* dy;
  float* gq; float* gk; float* gv;
  int B, H, L, dv;
  void* workspace; size_t workspace_bytes;
  const float* gamma = nullptr;  // [H] per-head state decay (decayed variant)
};
size_t linattn_bwd_workspace(int B, int H, int L, int dv, bool bf16);
// bf16 on the matrix cores for d_v in {32, 64, 96, 128} (slices of 32 columns)
bool linattn_bwd_mfma_supported(int dv);
size_t linattn_bwd_mfma_workspace(int B, int H, int L, int dv);
hipError_t launch_linattn_bwd_mfma(const LinattnBwdArgs& a, hipStream_t stream);
hipError_t launch_linattn_bwd(const LinattnBwdArgs& a, bool bf16, hipStream_t stream);

// BaseConv gate: y = u * (bias + causal depthwise conv of x with h [D, K]).
struct BaseConvArgs {
  const void* x; const void* u; const float* h; const float* bias; float* y;
  int B, L, D, K;
};
hipError_t launch_baseconv(const BaseConvArgs& a, bool bf16, hipStream_t stream);

struct DecodeArgs {
  const void* q; const void* k; const void* v;
  float* S; float* z; void* ring_k; void* ring_v; int32_t* pos;
  float* y_lin; float* y_swa;
  int B, H, dv, window; float scale;
  const float* gamma = nullptr;  // [H] per-head state decay (decayed variant only)
  bool compact = false;          // S [.,153,dv], z [.,153]: one row per unordered feature pair
};
hipError_t launch_decode_step(const DecodeArgs& a, bool bf16, hipStream_t stream);

// State layout conversions over n heads: 273-row <-> compact 153-row.
hipError_t launch_state_compact(const float* S, const float* z, float* Sc, float* zc, size_t n, int dv,
                                hipStream_t stream);
hipError_t launch_state_expand(const float* Sc, const float* zc, float* S, float* z, size_t n, int dv,
                               hipStream_t stream);

hipError_t launch_decode_prefill(const void* k, const void* v, void* ring_k, void* ring_v, int32_t* pos,
                                 int B, int H, int L, int dv, int window, bool bf16, hipStream_t stream);

}  // namespace based
