// Host-side interface between the C entry points (gdn_fwd.hip) and the
// full-width chunk kernel (gdn_fwd_full.hip).  Internal header: nothing
// here is exported from the shared library.
#ifndef GDN_LAUNCH_H
#define GDN_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn_launch {

// One workgroup per (sequence segment, head), all dv = 128 value columns,
// dk = 128, 64-token chunks, bf16 storage.
struct FullParams {
  const char* q;
  const char* k;
  const char* v;
  const float* g;
  const float* beta;
  const float* h0;
  const int32_t* cu;  // packed batch offsets (B + 1), or null (dense)
  char* out;
  float* hT;
  int B, T, H;
  // A sequence of n chunks is cut into ceil(n / seg_max) segments of equal
  // length (the last one shorter); seg_max = 0 never cuts.  The cut depends
  // on the sequence alone, never on the batch or the device.
  int seg_max;
  int nslot;  // segment slots per head (the grid is nslot x H)
  // Chunk-map scan (fwd_full_scan): per (segment slot, head) three dk x dv
  // fp32 matrices, row-major: the segment's map P and Q (M_end = P M_start
  // + Q) and its exact entry state S.  Null: segments start from halos.
  float* ws = nullptr;
};

// Number of segment slots per head for a call (see FullParams).
__attribute__((visibility("hidden"))) int full_slots(int B, int T, bool packed, int seg_max);

__attribute__((visibility("hidden"))) int fwd_full(const FullParams& p, hipStream_t stream);

// Floats of workspace fwd_full_scan needs for nslot segment slots.
__attribute__((visibility("hidden"))) long long scan_ws_floats(int nslot, int H);

// Three launches: the maps of every segment but the last, the scan of the
// maps into exact entry states, then the outputs from those states.
__attribute__((visibility("hidden"))) int fwd_full_scan(const FullParams& p, hipStream_t stream);

}  // namespace gdn_launch

#endif  // GDN_LAUNCH_H
