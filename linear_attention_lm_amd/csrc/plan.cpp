// Host-side planning of the chunked linear-attention passes: how a (batch,
// head)'s sequence splits into segments so that the grid fills the GPU, and
// the workspace each entry point needs for that split.  Plain C++ (no device
// code), so that the C ABI's validation can be built and tested on its own.
#include "../../include/based.h"
#include "launchers.h"

namespace based {

using namespace layout;

// Forward: enough workgroups to fill the GPU's 256 compute units (two per CU
// where they fit: d_v <= 64), each segment at least 4 chunks long.
void linattn_mfma_plan(int BH, int L, int dv, int* nseg, int* seg_chunks) {
  const int nch = (L + CHUNK - 1) / CHUNK;
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

// Forward workspace: per (batch, head) and segment one compact state record
// of (FWD_SLOTS + 1) x dv floats and one denominator record of FWD_SLOTS + 1.
size_t linattn_mfma_workspace(int B, int H, int L, int dv) {
  if (!linattn_mfma_supported(dv)) return 0;
  int nseg, sc;
  linattn_mfma_plan(B * H, L, dv, &nseg, &sc);
  if (nseg <= 1) return 0;
  return (size_t)B * H * nseg * ((size_t)(FWD_SLOTS + 1) * dv + (FWD_SLOTS + 1)) * sizeof(float);
}

bool linattn_bwd_mfma_supported(int dv) { return dv == 32 || dv == 64 || dv == 96 || dv == 128; }

// Backward segments per head: enough workgroups for two per CU, at most
// BWD_MAXSEG, and at least four chunks per segment.
void linattn_bwd_mfma_plan(int BH, int L, int dv, int* nseg, int* seg_chunks) {
  const int nch = (L + CHUNK - 1) / CHUNK;
  const int units = BH * (dv / BWD_SLICE);
  int want = (512 + units - 1) / units;
  if (want > BWD_MAXSEG) want = BWD_MAXSEG;
  int cap = nch / 4;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  const int sc = nch < 1 ? 1 : (nch + want - 1) / want;
  *seg_chunks = sc;
  *nseg = nch < 1 ? 1 : (nch + sc - 1) / sc;
}

// Forward-record sub-segments per backward segment.  With two segments the
// records cover only the first, as B*H workgroups of the state-only pass;
// where that leaves most of the CUs idle (B*H <= 64) the record is split
// (down to 8 chunks, up to one workgroup per CU) and the query pass sums the
// parts.  Otherwise the extra records cost the query pass about what the
// shorter pass saves, and with more segments each one adds to that sum.
int linattn_bwd_rec_split(int BH, int nseg, int seg_chunks) {
  int r = 1;
  if (nseg != 2 || BH > 64) return r;
  while (r < 4 && (long long)BH * 2 * r <= 256 && seg_chunks % (2 * r) == 0 && seg_chunks / (2 * r) >= 8) r *= 2;
  return r;
}

// Suffix-state sub-records per segment: the suffix-state pass has one
// workgroup per (head, slice, segment >= 1, sub-record) beside the B*H*slices
// that sum dq; a segment's increment is split (down to 4 chunks) while the
// pass stays within three workgroups per CU.
int linattn_bwd_key_split(int BH, int dv, int nseg, int seg_chunks) {
  const long long units = (long long)BH * (dv / BWD_SLICE) * (nseg - 1), sum_units = (long long)BH * (dv / BWD_SLICE);
  int r = 1;
  if (nseg < 2) return r;
  while (r < 4 && units * 2 * r + sum_units <= 768 && seg_chunks % (2 * r) == 0 && seg_chunks / (2 * r) >= 4) r *= 2;
  return r;
}

size_t linattn_bwd_mfma_workspace(int B, int H, int L, int dv) {
  int nseg, sc;
  const int BH = B * H;
  linattn_bwd_mfma_plan(BH, L, dv, &nseg, &sc);
  const int nslice = dv / BWD_SLICE;
  size_t floats = (size_t)(1 + nslice) * BH * L;                          // den, h per slice
  if (nslice > 1) floats += (size_t)2 * nslice * BH * L * BASED_DK;      // dq, dk shares per slice
  if (nseg > 1) {
    const int rs = linattn_bwd_rec_split(BH, nseg, sc);
    floats += (size_t)BH * nseg * rs * ((size_t)(FWD_SLOTS + 1) * dv + (FWD_SLOTS + 1));  // forward records
    floats += (size_t)BH * nslice * nseg * linattn_bwd_key_split(BH, dv, nseg, sc) * BWD_RREC;  // suffix records
  }
  return floats * sizeof(float);
}

size_t linattn_bwd_workspace(int B, int H, int L, int dv, bool bf16) {
  if (bf16 && linattn_bwd_mfma_supported(dv)) return linattn_bwd_mfma_workspace(B, H, L, dv);
  return (size_t)B * H * L * 2 * sizeof(float);  // den and h per position
}

}  // namespace based
