// Host-side interface between the C entry points (gdn_fwd.hip) and the
// full-width chunk kernel (gdn_fwd_full.hip).  Internal header: nothing
// here is exported from the shared library.
#ifndef GDN_LAUNCH_H
#define GDN_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn_launch {

// Longest sequence segment, in 64-token chunks, of the full-width kernels.
constexpr int SEG_MAX_CHUNKS = 16;

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
  // length (the last one shorter), but into at most seg_cap of them when
  // seg_cap > 0; seg_max = 0 never cuts.  The cut depends on the sequence,
  // H and the device (seg_cap is the CUs per head), never on the batch.
  int seg_max;
  int seg_cap = 0;
  int nslot;  // segment slots per head (the grid is nslot x H)
  // Chunk-map scan (fwd_full_scan): per (segment slot, head) three dk x dv
  // fp32 matrices, row-major: the segment's map P and Q (M_end = P M_start
  // + Q) and its exact entry state S.  Null: segments start from halos.
  float* ws = nullptr;
  // Backward-pass records (gdn_full_kernel<2> and <3> write M and U, the
  // adjoint kernel dM and dX): one record of BWD_REC_BYTES per (chunk slot, head),
  // chunk c of the sequence whose tokens start at s taking chunk slot
  // floor(s / 64) + (sequence index) + c.  Each part is bf16 row-major.
  char* sv = nullptr;
};

// A backward record: M and dM (the chunk's entry state and the gradient
// reaching its exit state, key-major: dk rows of dv values), then U and dX
// (C token rows of dv values), at these byte offsets.
constexpr long BWD_OFF_M = 0, BWD_OFF_DM = 128 * 128 * 2, BWD_OFF_U = 2 * 128 * 128 * 2,
               BWD_OFF_DX = 2 * 128 * 128 * 2 + 64 * 128 * 2, BWD_REC_BYTES = 2 * 128 * 128 * 2 + 2 * 64 * 128 * 2;

// Backward pass, bf16, dk = dv = 128, 64-token chunks (gdn_bwd_full.hip).
struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* dO;
  const float* g;
  const float* beta;
  const float* h0;
  const float* dhT;
  const int32_t* cu;
  char* dq;
  char* dk;
  char* dv;
  float* dg;
  float* dbeta;
  float* dh0;
  char* sv;   // records, as FullParams::sv
  float* hT;  // any valid float buffer (the states pass writes no hT)
  int B, T, H;
  int seg_max, seg_cap, nslot;  // sequence segments of the two sweeps (as FullParams)
  int states_saved = 0;         // the records of M and U are already in sv (a training forward wrote them)
  int nchunk;          // chunk slots per head
};

// Bytes of records the full-width backward needs.
__attribute__((visibility("hidden"))) long long bwd_full_ws_bytes(int B, long ttot, int H);

// The states pass, the adjoint sweep and the gradient kernel.
__attribute__((visibility("hidden"))) int bwd_full(const BwdParams& p, hipStream_t stream);

// Number of segment slots per head for a call (see FullParams).
__attribute__((visibility("hidden"))) int full_slots(int B, int T, bool packed, int seg_max, int seg_cap);

// The segment cap for H heads on the current device: its CUs per head (at
// least 1), or 0 when the device cannot be queried (no cap).
__attribute__((visibility("hidden"))) int seg_cap_for(int H);

__attribute__((visibility("hidden"))) int fwd_full(const FullParams& p, hipStream_t stream);

// Floats of workspace fwd_full_scan needs for nslot segment slots.
__attribute__((visibility("hidden"))) long long scan_ws_floats(int nslot, int H);

// Three launches: the maps of every segment but the last, the scan of the
// maps into exact entry states, then the outputs from those states.
__attribute__((visibility("hidden"))) int fwd_full_scan(const FullParams& p, hipStream_t stream);

// The forward recurrence saving every chunk's entry state and U into p.sv
// (no outputs, no hT).
__attribute__((visibility("hidden"))) int fwd_full_save(const FullParams& p, hipStream_t stream);

// fwd_full and fwd_full_save in one pass: outputs, hT and the records.
__attribute__((visibility("hidden"))) int fwd_full_train(const FullParams& p, hipStream_t stream);

}  // namespace gdn_launch

#endif  // GDN_LAUNCH_H
