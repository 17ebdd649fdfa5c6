// Token-by-token (fused recurrent) form of the gated delta rule for short
// sequences and decoding, for gfx950.
//
// Per head and token (HyMo "Model Architecture Walkthrough", sections
// 5.2.1-5.2.2; the decayed read-before-write order of section 5.3.1):
//
//   alpha = exp(g_t),  p = S_{t-1} k_t,
//   S_t   = alpha S_{t-1} + beta_t (v_t - alpha p) k_t^T,   o_t = S_t q_t,
//
// which is alpha S (I - beta k k^T) + beta v k^T rewritten with the
// prediction alpha p, one rank-1 update per token.  The pages' description
// of this form keeps the state on chip for the whole sequence and streams
// one token's q, k, v, g and beta per step ("Model Architecture
// Walkthrough", sections 6.2-6.4).
//
// Mapping: one wave per (chain, slab of up to 64 value columns); lane j owns
// value column j of the slab and holds that column of the state, all dk key
// rows, in registers (M = S^T, so the lane's column is contiguous in h0/hT
// rows).  Both reductions over the key dimension (S k and S q) therefore stay
// inside a lane; the token's k and q, g and beta are the same for every lane
// and are read through the scalar unit.  Nothing is shared between waves, so
// there is no LDS and no barrier.  The traffic is the state read and write
// (dk x dv fp32 per chain, each lane reading and writing 4 bytes of every
// 256-byte key row) plus one pass over the tokens.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace {

struct RShape {
  int T, H, dv, width, nslab, nitems;
};

constexpr int WAVES = 4;  // independent waves per workgroup

// Element i of a token's key or query row as fp32.  A bf16 row is read as
// 32-bit words (two elements each) so that the read, uniform across the
// wave, goes through the scalar unit, and widened by shifting.
template <typename TI>
__device__ static inline float row_el(const TI* __restrict__ base, long row0, int i) {
  if constexpr (sizeof(TI) == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(base + row0)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return base[row0 + i];
  }
}

// Read-only, non-aliased pointers as separate arguments: the loads of the
// token's k, q, g and beta, whose addresses are the same in every lane,
// then go through the scalar unit.  h0 and hT carry no restrict: hT may be
// h0 itself (an in-place state update; each lane reads its column of h0
// before the token loop and writes it back after).
template <typename TI, int DK>
__global__ __launch_bounds__(64 * WAVES) void gdn_recurrent_kernel(
    const TI* __restrict__ qp, const TI* __restrict__ kp, const TI* __restrict__ vp, const float* __restrict__ gp,
    const float* __restrict__ bp, const float* h0, const int32_t* __restrict__ cu, TI* __restrict__ out,
    float* hT, const RShape p) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * WAVES + (threadIdx.x >> 6));
  if (item >= p.nitems) return;  // whole waves leave together
  const int chain = item / p.nslab, slab = item % p.nslab;
  const int H = p.H, dv = p.dv;
  const int bseq = chain / H, hh = chain % H;
  long rowbase;
  int len;
  if (cu) {
    rowbase = cu[bseq];
    len = cu[bseq + 1] - cu[bseq];
  } else {
    rowbase = (long)bseq * p.T;
    len = p.T;
  }
  const bool active = lane < p.width;
  const int col = slab * p.width + (active ? lane : 0);
  const long sbase = (long)chain * DK * dv + col;

  float M[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) M[i] = 0.f;
  if (h0 && active) {
#pragma unroll
    for (int i = 0; i < DK; ++i) M[i] = h0[sbase + (long)i * dv];
  }

  for (int t = 0; t < len; ++t) {
    const long row = rowbase + t;
    const long th = row * H + hh;  // token-head index
    const float a = __builtin_amdgcn_exp2f(gp[th] * kLog2e);
    const float b = bp[th];
    const long kq = th * DK;
    // p = S_{t-1} k (four interleaved partial sums, combined in fixed order)
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DK; ++i) ps[i & 3] = __builtin_fmaf(M[i], row_el(kp, kq, i), ps[i & 3]);
    const float pk = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    const float vc = active ? (float)vp[th * dv + col] : 0.f;
    const float u = b * (vc - a * pk);
    // S_t = alpha S_{t-1} + u k^T, then o = S_t q
    float os[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DK; ++i) {
      M[i] = __builtin_fmaf(a, M[i], u * row_el(kp, kq, i));
      os[i & 3] = __builtin_fmaf(M[i], row_el(qp, kq, i), os[i & 3]);
    }
    // rounded to nearest even for bf16
    if (active) out[th * dv + col] = (TI)((os[0] + os[1]) + (os[2] + os[3]));
  }
  if (active) {
#pragma unroll
    for (int i = 0; i < DK; ++i) hT[sbase + (long)i * dv] = M[i];
  }
}

template <typename TI, int DK>
void launch_dk(const void* q, const void* k, const void* v, const float* g, const float* beta, const float* h0,
               const int32_t* cu, void* out, float* hT, const RShape& p, hipStream_t s) {
  const int nwg = (p.nitems + WAVES - 1) / WAVES;
  hipLaunchKernelGGL((gdn_recurrent_kernel<TI, DK>), dim3(nwg), dim3(64 * WAVES), 0, s, static_cast<const TI*>(q),
                     static_cast<const TI*>(k), static_cast<const TI*>(v), g, beta, h0, cu, static_cast<TI*>(out), hT,
                     p);
}

template <typename TI>
int launch_rec(const void* q, const void* k, const void* v, const float* g, const float* beta, const float* h0,
               const int32_t* cu, void* out, float* hT, const RShape& p, int dk, hipStream_t s) {
  switch (dk) {
    case 32: launch_dk<TI, 32>(q, k, v, g, beta, h0, cu, out, hT, p, s); break;
    case 64: launch_dk<TI, 64>(q, k, v, g, beta, h0, cu, out, hT, p, s); break;
    case 128: launch_dk<TI, 128>(q, k, v, g, beta, h0, cu, out, hT, p, s); break;
    default: return GDN_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" int gdn_fwd_recurrent(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const float* h0, const int32_t* cu_seqlens, void* out, float* hT, int B, int T,
                                 int H, int dk, int dv, void* stream, int dtype) {
  if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_INVALID_ARG;
  if (B > 0 && !hT) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if ((dk != 32 && dk != 64 && dk != 128) || (dv != 32 && dv != 64 && dv != 128)) return GDN_ERR_UNSUPPORTED;
  RShape p;
  p.width = dv < 64 ? dv : 64;
  p.nslab = dv / p.width;
  const long items = (long)B * H * p.nslab;
  if (items > 0x7fffffffL - WAVES) return GDN_ERR_INVALID_ARG;
  if (items == 0) return GDN_OK;
  p.T = T;
  p.H = H;
  p.dv = dv;
  p.nitems = (int)items;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == GDN_BF16 ? launch_rec<__bf16>(q, k, v, g, beta, h0, cu_seqlens, out, hT, p, dk, s)
                            : launch_rec<float>(q, k, v, g, beta, h0, cu_seqlens, out, hT, p, dk, s);
}
