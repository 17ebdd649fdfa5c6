// Shapes, LDS layout constants and index helpers shared by the full-width
// chunk kernels (gdn_fwd_full.hip, gdn_bwd_full.hip): bf16 storage,
// dk = dv = 128, 64-token chunks.  Internal header: every definition sits in
// an unnamed namespace of the including file.
#ifndef GDN_FULL_COMMON_H
#define GDN_FULL_COMMON_H

#include "gdn_device.h"

namespace {

namespace fk {

constexpr int DK = 128, DV = 128, C = 64;
constexpr int NB = C / 16, NTS = C / 32;    // 16-token blocks, 32-token slabs per chunk
constexpr int NKB = DK / 16, NKS = DK / 32;  // 16-key blocks, 32-key slabs
constexpr int NCW = DV / 32;                 // column waves
constexpr int NW = NCW + 4;                  // + loader, Gram, two P waves
constexpr int W_L = NCW, W_G = NCW + 1, W_P = NCW + 2;
constexpr int KQR = DK * 2;       // bytes per q/k row
constexpr int GR = KQR / 16;      // 16-byte granules per row
constexpr int KQ_BYTES = C * KQR;  // one chunk of q or k
constexpr int KQ_INS = KQ_BYTES / 1024, KQ_RPI = 1024 / KQR;  // copies per chunk, rows per copy
constexpr int CCR = C * 2;        // bytes per row of a C x C bf16 tile
constexpr int CC_BYTES = C * CCR;
constexpr int NKR = 4, NQR = 3, NVEC = 3;  // ring depths: k, q, decay vectors
// Per-token vectors (fp32, C each): beta, lambda = gamma*log2(e), Gam,
// w = exp(gamma_C - gamma), exp(gamma_t - gamma at the start of t's block),
// and for b = 1..NB-1, exp(gamma_{16 b} - gamma_t) (t < 16 b).
constexpr int F_BETA = 0, F_LAM = 1, F_GAM = 2, F_W = 3, F_ER = 4, NF = 4 + NB;
constexpr int AD_ROW = 20, AD_BLK = 16 * AD_ROW + 4;  // padded fp32 diagonal blocks
constexpr int LDS = NKR * KQ_BYTES + NQR * KQ_BYTES + CC_BYTES + 2 * CC_BYTES + CC_BYTES +
                    NVEC * NF * C * 4 + NB * AD_BLK * 4 + 4 * C * 4 + 64;
static_assert(LDS <= 160 * 1024, "LDS budget");
static_assert(NB == 4 && NKS == 4 && NCW == 4, "shape");

// P wave o owns the 16-row blocks {o, 3 - o} (equal MFMA work).
__host__ __device__ constexpr int own_tb(int o, int i) { return i == 0 ? o : NB - 1 - o; }

// State row (key) held by accumulator block b, row r: of the 32 keys of
// slab b >> 1, block b takes the half b & 1 of each 8-key group, so that
// two stacked blocks form a bf16 fragment whose positions are the natural
// keys 32 s + 8 q .. 32 s + 8 q + 7 of lane group q.
__device__ static inline int key_of(int b, int r) {
  return 32 * (b >> 1) + 8 * (r >> 2) + 4 * (b & 1) + (r & 3);
}

// Chunk count of a sequence and its segment layout: ceil(nch / seg_max)
// segments of equal length (the last one shorter), at most seg_cap of them
// when seg_cap > 0.
__host__ __device__ static inline void seg_layout(int len, int seg_max, int seg_cap, int& nch, int& seg_len,
                                                  int& nseg) {
  nch = (len + C - 1) / C;
  if (seg_max <= 0 || nch <= seg_max) {
    seg_len = nch > 0 ? nch : 1;
    nseg = 1;
    return;
  }
  int n0 = (nch + seg_max - 1) / seg_max;
  if (seg_cap > 0 && n0 > seg_cap) n0 = seg_cap;
  seg_len = (nch + n0 - 1) / n0;
  nseg = (nch + seg_len - 1) / seg_len;
}

}  // namespace fk

}  // namespace

#endif  // GDN_FULL_COMMON_H
