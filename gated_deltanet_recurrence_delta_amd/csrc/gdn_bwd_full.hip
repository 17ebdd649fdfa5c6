// Backward pass of the gated delta rule for gfx950, full-width chunk
// kernels: bf16 q/k/v/dO, dk = dv = 128, 64-token chunks.
//
// Rule and chunk algebra as in gdn_fwd_full.hip (HyMo "Model Architecture
// Walkthrough", sections 5.2.1-5.2.2; "Optimization Quartet", section 3.2).
// The pages train through the layer with a backward pass that recomputes
// what it needs from the saved inputs ("Optimization Quartet", sections
// 3.3-3.4).  With M = S^T, a chunk's entry state M and exit state M',
// Tb = T diag(beta), X = V - diag(Gam) K M, U = Tb X, E_ij =
// exp(gamma_i - gamma_j), P = lower(Q K^T . E), and dO, dM' the gradients
// reaching the chunk's outputs and exit state, reverse mode gives
//
//   dU = P^T dO + diag(w) K dM',   dX = T^T dU  (the gradient of beta X),
//   dV = diag(beta) dX,
//   dM = Gam_C dM' + Q^T diag(Gam) dO - K^T diag(Gam) dV     (chunk to chunk),
//   dA = -strict_lower(dX U^T),    dP = lower(dO U^T),   G = dA . E . beta_i,
//   dQ = diag(Gam) dO M^T + (dP . E) K,
//   dK = -diag(beta Gam) dX M^T + diag(w) U dM'^T + (G + G^T) K + (dP . E)^T Q,
//   dbeta_i = sum_b dX_ib (V - Gam K M)_ib + sum_j dA_ij (K K^T . E)_ij,
//   dgamma = rowsum(Z) - colsum(Z) + dGam . Gam - dw . w (+ sum(dw . w) at the
//            chunk's last token),  Z = strict_lower(dA . A + dP . P),
//   dGam_i = -beta_i sum_b dX_ib (K M)_ib + sum_b dO_ib (Q M)_ib
//            (+ <M', dM'> at the last token ... see the gradient kernel),
//   dw_i = sum_b U_ib (K dM')_ib,   dg = reverse cumulative sum of dgamma.
//
// Three passes:
//   states  (gdn_full_kernel<2> of gdn_fwd_full.hip): the forward recurrence,
//           saving every chunk's entry state M and its U;
//   adjoint (gdn_adjoint_kernel below): the state gradient from dhT backwards
//           over the chunks, in the forward kernel's eight-wave pipeline with
//           the chunk order reversed, saving every chunk's dM' and dX;
//   grad    (gdn_grad_kernel below): one workgroup per (chunk, head), dq, dk,
//           dv, dg and dbeta from the saved M, dM', U and dX -- no triangular
//           solve is left in it.
// Every product runs on the bf16 matrix cores with fp32 accumulation; the
// saved matrices are bf16.  No atomics: results are deterministic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_full_common.h"
#include "gdn_launch.h"

namespace {

using namespace fk;

// ====================================================================
// adjoint sweep
//
// One workgroup per (sequence segment, head), as the forward.  A segment
// covering chunks [c0, c1) starts from a zero gradient at the earliest chunk
// boundary ce >= c1 after which the product of the per-token transition
// norms over [c1, ce) is at most e^-HALO_NATS (the gradient goes back
// through the transposed, here the same, symmetric, maps), or from dhT at
// the sequence end; chunks ce-1 down to c0 are processed, the ones at or
// after c1 (the halo) without saving anything.  Step r works chunk ce-1-r.
//
// Waves as in the forward: column waves 0..3 (32 value columns each, that
// quarter of the state gradient D in fp32 MFMA accumulators), the loader,
// the Gram wave (publishes T^T unscaled, rows in pi order, so that it is an
// MFMA row operand by plain 16-byte reads) and two P waves (publish P^T as
// lane-major row-operand fragments).  Per chunk a column wave forms
//   Y' = K D,  D <- Gam_C D + Q^T (Gam dO),  dU = P^T dO + diag(w) Y',
//   dX = T^T dU,  W = -diag(Gam beta) dX,  D <- D + K^T W.
__global__ __launch_bounds__(64 * NW, 1) void gdn_adjoint_kernel(const gdn_launch::BwdParams p) {
  using MM = Mma<__bf16>;
  using F = bf16x8;
  constexpr float kLog2e = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) char sK[NKR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sQ[NQR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sAT[CC_BYTES];     // A (off-diagonal) and T_bb^T
  __shared__ __attribute__((aligned(16))) char sT[2 * CC_BYTES];  // T^T of two chunks, rows in pi order
  __shared__ __attribute__((aligned(16))) char sP[CC_BYTES];      // P^T, lane-major fragments
  __shared__ __attribute__((aligned(16))) float sVEC[NVEC * NF * C];
  __shared__ __attribute__((aligned(16))) float sAD[NB * AD_BLK];
  __shared__ __attribute__((aligned(16))) float sGB[2 * 2 * C];  // g, beta of two chunks
  __shared__ int sFLAG[4];
  __shared__ int sPICK[2];
  __shared__ int sEND;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4, n16 = lane & 15;
  const int src = lane & 15;
  const int H = p.H;

  // ---------------------------------------------------- which segment
  const int slot = blockIdx.x / H, hh = blockIdx.x % H;
  int bseq, seg;
  long rowbase;
  int len;
  if (p.cu) {
    if (threadIdx.x == 0) sPICK[0] = -1;
    __syncthreads();
    const long segt = p.seg_max > 0 ? (long)p.seg_max * C : 0;
    for (int t = threadIdx.x; t < p.B; t += blockDim.x) {
      const int s0 = p.cu[t], s1 = p.cu[t + 1];
      int nch, seg_len, nseg;
      seg_layout(s1 - s0, p.seg_max, p.seg_cap, nch, seg_len, nseg);
      const long f = (segt > 0 ? s0 / segt : 0) + t;
      if (slot >= f && slot < f + nseg) {
        sPICK[0] = t;
        sPICK[1] = (int)(slot - f);
      }
    }
    __syncthreads();
    bseq = sPICK[0];
    if (bseq < 0) return;  // a slot no sequence uses (uniform over the workgroup)
    seg = sPICK[1];
    rowbase = p.cu[bseq];
    len = p.cu[bseq + 1] - p.cu[bseq];
  } else {
    int nch, seg_len, nseg;
    seg_layout(p.T, p.seg_max, p.seg_cap, nch, seg_len, nseg);
    bseq = slot / nseg;
    seg = slot % nseg;
    if (bseq >= p.B) return;
    rowbase = (long)bseq * p.T;
    len = p.T;
  }
  bseq = __builtin_amdgcn_readfirstlane(bseq);
  seg = __builtin_amdgcn_readfirstlane(seg);
  len = __builtin_amdgcn_readfirstlane(len);
  const int chain = bseq * H + hh;
  const long cslot0 = rowbase / C + bseq;  // chunk slot of the sequence's first chunk

  int nch, seg_len, nseg;
  seg_layout(len, p.seg_max, p.seg_cap, nch, seg_len, nseg);
  const int c0 = seg * seg_len;
  const int c1 = min(c0 + seg_len, nch);
  if (threadIdx.x < 4) sFLAG[threadIdx.x] = 0;
  if (wave == 0) {
    int ce = c1;
    float acc = 0.f;  // log of the transition-norm product over chunks [c1, ce)
    while (ce < nch && acc > -HALO_NATS) {
      const int t = ce * C + lane;  // the sequence's last chunk may be partial
      float e = 0.f;
      if (t < len) {
        const long th = (rowbase + t) * H + hh;
        const uint4* kr = reinterpret_cast<const uint4*>(p.k + th * KQR);
        float n2 = 0.f;
#pragma unroll
        for (int i = 0; i < DK / 8; ++i) {
          const uint4 w = kr[i];
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float lo = __uint_as_float(u[jj] << 16), hi = __uint_as_float(u[jj] & 0xffff0000u);
            n2 = __builtin_fmaf(lo, lo, n2);
            n2 = __builtin_fmaf(hi, hi, n2);
          }
        }
        const float f = fabsf(1.f - p.beta[th] * n2);
        e = p.g[th] + (f > 1.f ? __logf(f) : 0.f);
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) e += __shfl_xor(e, d);
      acc += e;
      ++ce;
    }
    if (lane == 0) sEND = ce;
  }
  __syncthreads();
  const int ce = sEND;
  const int NC = ce - c0;  // chunks processed, step r working chunk ce-1-r
  const int NIT = NC > 0 ? NC + 2 : 0;
  const int r_store = ce - c1;  // steps r >= r_store save their chunk
  const long kq_stride = (long)H * KQR;
  const long v_stride = (long)H * DV * 2;
  // First row of step r's chunk, and its tokens up to the sequence end (0
  // for a step past the last: empty descriptors).
  auto crow = [&](int r) { return rowbase + (long)max(ce - 1 - r, 0) * C; };
  auto cleft = [&](int r) { return r < NC ? (long)(len - (ce - 1 - r) * C) : 0L; };
  auto vec_of = [&](int r) { return sVEC + (r % NVEC) * NF * C; };

  int kq_frag[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kq_frag[s] = n16 * KQR + 16 * ((4 * s + q4) ^ swz_kq<GR>(n16));
  int cc_frag[NTS];
#pragma unroll
  for (int s = 0; s < NTS; ++s) cc_frag[s] = n16 * CCR + 16 * ((4 * s + q4) ^ swz_cc<C>(n16));

  if (wave < NCW) {
    // ========================================================= column waves
    const int j = wave;
    const long sbase = (long)chain * DK * DV;
    // K^T and Q^T (transposing reads), as the forward's K^T.
    int kt_base[NKB / 2];
#pragma unroll
    for (int bh = 0; bh < NKB / 2; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      kt_base[bh] = r * KQR + 16 * ((4 * bh + (src & 3)) ^ swz_kq<GR>(r));
    }
    // dO in accumulator layout: token 16 tb + 4 q4 + e, value columns
    // 32 j + 2 n16 .. +1 (one bf16 pair per lane).
    const int d_lane = (int)(4 * q4 * v_stride) + (32 * j + 2 * n16) * 2;

    f32x4 Dacc[NKB][2];
    {
      const bool from_dhT = p.dhT && ce == nch;
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(from_dhT ? p.dhT + sbase : p.hT, from_dhT ? (long)DK * DV * 4 : 0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(
              rh, (key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16) * 4, 0, 0);
          Dacc[kb][0][e] = __uint_as_float(h[0]);
          Dacc[kb][1][e] = __uint_as_float(h[1]);
        }
    }
    F Df[NKS][2];
    auto make_df = [&]() {
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) Df[s][cb] = MM::from_acc(Dacc[2 * s][cb], Dacc[2 * s + 1][cb]);
    };
    make_df();

    auto load_do = [&](int r, uint32_t (&Dn)[NB][4]) {
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dO + (crow(r) * H + hh) * DV * 2, cleft(r) * v_stride);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Dn[tb][e] = __builtin_amdgcn_raw_buffer_load_b32(rd, d_lane, (int)((16 * tb + e) * v_stride), 0);
    };
    auto vval = [](uint32_t pair, int cb) { return __uint_as_float(cb ? (pair & 0xffff0000u) : (pair << 16)); };

    uint32_t Db[NB][4], Dn[NB][4];
    auto process = [&](int r) {
      const int c = ce - 1 - r;
      const char* sk = sK + (r % NKR) * KQ_BYTES;
      const char* sq = sQ + (r % NQR) * KQ_BYTES;
      const char* st = sT + (r & 1) * CC_BYTES;
      const float* vec = vec_of(r);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      load_do(r + 1, Dn);  // unconditional: past the last step the descriptor is empty
      asm volatile("" ::: "memory");
      const __amdgpu_buffer_rsrc_t rrec = make_rsrc(p.sv + ((cslot0 + c) * H + hh) * gdn_launch::BWD_REC_BYTES,
                                                    r >= r_store ? gdn_launch::BWD_REC_BYTES : 0);
      // The gradient reaching this chunk's exit, key-major (key rows of 128
      // values; one bf16 pair of adjacent value columns per lane and key).
      {
        const int d_lane = (8 * q4 * DV + 32 * j + 2 * n16) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(cvt_pair(Dacc[kb][0][e], Dacc[kb][1][e]), rrec,
                                                  d_lane + (32 * (kb >> 1) + 4 * (kb & 1) + e) * DV * 2,
                                                  (int)gdn_launch::BWD_OFF_DM, 0);
      }

      // dO as B fragments (byte permutes of the bf16 pairs), and Gam dO.
      F dOf[NTS][2], GdOf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 4 * q4);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 16 + 4 * q4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const uint32_t sel = cb ? 0x07060302u : 0x05040100u;
          const u32x4 f = {__builtin_amdgcn_perm(Db[2 * s][1], Db[2 * s][0], sel),
                           __builtin_amdgcn_perm(Db[2 * s][3], Db[2 * s][2], sel),
                           __builtin_amdgcn_perm(Db[2 * s + 1][1], Db[2 * s + 1][0], sel),
                           __builtin_amdgcn_perm(Db[2 * s + 1][3], Db[2 * s + 1][2], sel)};
          dOf[s][cb] = __builtin_bit_cast(F, f);
          f32x4 x0, x1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x0[e] = g0[e] * vval(Db[2 * s][e], cb);
            x1[e] = g1[e] * vval(Db[2 * s + 1][e], cb);
          }
          GdOf[s][cb] = MM::from_acc(x0, x1);
        }
      }
      // Y' = K D.
      f32x4 Y[NB][2];
      {
        F Kf[2][NKS];
        auto read_k = [&](int tb) {
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[tb & 1][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * tb);
        };
        read_k(0);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          if (tb + 1 < NB) read_k(tb + 1);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            f32x4 y = zero4;
#pragma unroll
            for (int s = 0; s < NKS; ++s) y = MM::mma(Kf[tb & 1][s], Df[s][cb], y);
            Y[tb][cb] = y;
          }
        }
      }
      // D <- Gam_C D + Q^T (Gam dO).
      const float gC = vec[F_GAM * C + C - 1];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        F QT[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
          const char* p0 = sq + kt_base[kb >> 1] + 8 * (kb & 1) + 32 * s * KQR;
          const bf16x4 lo = lds_read_tr(p0, 0);
          const bf16x4 hi = lds_read_tr(p0, 16 * KQR);
          QT[s] = F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 m = Dacc[kb][cb];
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] *= gC;
#pragma unroll
          for (int s = 0; s < NTS; ++s) m = MM::mma(QT[s], GdOf[s][cb], m);
          Dacc[kb][cb] = m;
        }
      }
      // dU = P^T dO + diag(w) Y' once the P waves have published P^T
      // (P^T of row block tb is zero in slabs s with 2 s + 1 < tb).
      flag_wait_lds(&sFLAG[0], r + 1);
      flag_wait_lds(&sFLAG[1], r + 1);
      f32x4 dU[NB][2];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(vec + F_W * C + 16 * tb + 4 * q4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 u = zero4;
#pragma unroll
          for (int s = 0; s < NTS; ++s)
            if (2 * s + 1 >= tb) u = MM::mma(lds_at<F>(sP + ((tb * NTS + s) * 64 + lane) * 16), dOf[s][cb], u);
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = __builtin_fmaf(wv[e], Y[tb][cb][e], u[e]);
          dU[tb][cb] = u;
        }
      }
      F dUf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) dUf[s][cb] = MM::from_acc(dU[2 * s][cb], dU[2 * s + 1][cb]);
      // dX = T^T dU: row block tb of T^T is zero in the blocks left of it
      // (the low half of slab s when 2 s < tb).
      f32x4 dX[NB][2];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        F TTf[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
          if (2 * s + 1 < tb) continue;
          F f = lds_at<F>(st + cc_frag[s] + 16 * CCR * tb);
          if (2 * s < tb) {
            f[0] = (__bf16)0.f; f[1] = (__bf16)0.f; f[2] = (__bf16)0.f; f[3] = (__bf16)0.f;
          }
          TTf[s] = f;
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 x = zero4;
#pragma unroll
          for (int s = 0; s < NTS; ++s)
            if (2 * s + 1 >= tb) x = MM::mma(TTf[s], dUf[s][cb], x);
          dX[tb][cb] = x;
        }
      }
      // dX saved (bf16 token rows); W = -diag(Gam beta) dX.
      {
        const int x_lane = (4 * q4 * DV + 32 * j + 2 * n16) * 2;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, bf16x2{(__bf16)dX[tb][0][e], (__bf16)dX[tb][1][e]}), rrec, x_lane,
                (int)gdn_launch::BWD_OFF_DX + (16 * tb + e) * DV * 2, 0);
      }
      F Wf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 4 * q4);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 16 + 4 * q4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(vec + F_BETA * C + 32 * s + 4 * q4);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(vec + F_BETA * C + 32 * s + 16 + 4 * q4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 w0, w1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = -(g0[e] * b0[e]) * dX[2 * s][cb][e];
            w1[e] = -(g1[e] * b1[e]) * dX[2 * s + 1][cb][e];
          }
          Wf[s][cb] = MM::from_acc(w0, w1);
        }
      }
      // D <- D + K^T W, then the next chunk's bf16 fragments.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        F KT[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
          const char* p0 = sk + kt_base[kb >> 1] + 8 * (kb & 1) + 32 * s * KQR;
          const bf16x4 lo = lds_read_tr(p0, 0);
          const bf16x4 hi = lds_read_tr(p0, 16 * KQR);
          KT[s] = F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 m = Dacc[kb][cb];
#pragma unroll
          for (int s = 0; s < NTS; ++s) m = MM::mma(KT[s], Wf[s][cb], m);
          Dacc[kb][cb] = m;
        }
      }
      make_df();
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) Db[tb][e] = Dn[tb][e];
    };

    if (NIT > 0) {
      lds_barrier();
      load_do(0, Db);
      lds_barrier();
      for (int r = 0; r < NC; ++r) {
        process(r);
        lds_barrier();
      }
    }
    if (p.dh0 && c0 == 0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x2*>(p.dh0 + sbase + (long)key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16) =
              f32x2{Dacc[kb][0][e], Dacc[kb][1][e]};
    }
  } else if (wave == W_L) {
    // ========================================================== loader wave
    // As the forward's, with step r's chunk at crow(r).
    int kq_src[KQ_INS];
#pragma unroll
    for (int i = 0; i < KQ_INS; ++i) {
      const int r = i * KQ_RPI + lane / GR;
      kq_src[i] = (int)(r * kq_stride) + 16 * ((lane % GR) ^ swz_kq<GR>(r));
    }
    const int gb_src = lane * H * 4;
    auto issue_gb = [&](int r) {
      char* d = reinterpret_cast<char*>(sGB + (r & 1) * 2 * C);
      copy_to_lds4(make_rsrc(p.g + crow(r) * H + hh, cleft(r) * H * 4), d, gb_src);
      copy_to_lds4(make_rsrc(p.beta + crow(r) * H + hh, cleft(r) * H * 4), d + C * 4, gb_src);
    };
    auto issue = [&](const char* base, char* ring, int nring, int r) {
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + crow(r) * kq_stride + hh * KQR, cleft(r) * kq_stride);
      char* d = ring + (r % nring) * KQ_BYTES;
#pragma unroll
      for (int i = 0; i < KQ_INS; ++i) copy_to_lds(rs, d + i * 1024, kq_src[i]);
    };
    auto make_vec = [&](int r, float sg, float sb) {
      float* vec = vec_of(r);
      const float lam = wave_prefix_sum(sg * kLog2e, lane);
      const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), C - 1));
      float lb[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) lb[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 16 * b));
      const int blk = lane >> 4;
      float lown = lb[0];
#pragma unroll
      for (int b = 1; b < NB; ++b) lown = blk == b ? lb[b] : lown;
      vec[F_BETA * C + lane] = sb;
      vec[F_LAM * C + lane] = lam;
      vec[F_GAM * C + lane] = exp2_fast(lam);
      vec[F_W * C + lane] = exp2_fast(lamC - lam);
      vec[F_ER * C + lane] = exp2_fast(lam - lown);
#pragma unroll
      for (int b = 1; b < NB; ++b) vec[(F_ER + b) * C + lane] = lane < 16 * b ? exp2_fast(lb[b] - lam) : 0.f;
    };
    constexpr int NOPS = 2 * KQ_INS + 2;
    constexpr int WAIT_NOPS = (NOPS & 15) | ((NOPS >> 4) << 14) | (7 << 4);  // vmcnt(NOPS) lgkmcnt(0)
    auto step_barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(WAIT_NOPS);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    if (NIT > 0) {
      issue_gb(0);
      issue(p.k, sK, NKR, 0);
    }
    for (int it = 0; it < NIT; ++it) {
      if (it == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(KQ_INS));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * KQ_INS));
      asm volatile("" ::: "memory");
      if (it < NC) {
        const float* gb = sGB + (it & 1) * 2 * C;
        make_vec(it, gb[lane], gb[C + lane]);
      }
      issue_gb(it + 1);
      issue(p.k, sK, NKR, it + 1);
      issue(p.q, sQ, NQR, it);
      step_barrier();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (wave == W_G) {
    // ============================================================ Gram wave
    // As the forward's; T is published transposed and unscaled, each
    // 32-column slab of a row in pi order.
    int t_dst[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * q4 + n16;
      t_dst[m] = r * CCR + 16 * ((4 * (q4 >> 1) + m) ^ swz_cc<C>(r)) + 8 * (q4 & 1);
    }
    int t_base[NTS];
#pragma unroll
    for (int bh = 0; bh < NTS; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      t_base[bh] = r * CCR + 16 * ((4 * bh + (src & 3)) ^ swz_cc<C>(r));
    }
    // T^T store: row x = 16 col + n16 holds T[16 b + 4 q4 .. +3][x]: in pi
    // order the granule 4 (b >> 1) + q4, half b & 1.
    auto tt_off = [&](int b, int col) {
      const int x = 16 * col + n16;
      return x * CCR + 16 * ((4 * (b >> 1) + q4) ^ swz_cc<C>(x)) + 8 * (b & 1);
    };
    auto cat = [](bf16x4 lo, bf16x4 hi) { return F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; };

    auto gram_solve = [&](int r) {
      const char* sk = sK + (r % NKR) * KQ_BYTES;
      const float* vec = vec_of(r);
      F Kf[NB][NKS];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < NKS; ++s) Kf[b][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float li = vec[F_LAM * C + 16 * b + n16];
        const float bi0 = vec[F_BETA * C + 16 * b + n16];
        const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + F_LAM * C + 16 * b + 4 * q4);
        f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s) kk = MM::mma(Kf[b][s], Kf[b][s], kk);
        f32x4 rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = 4 * q4 + e < n16 ? bi0 * kk[e] * exp2_fast(li - lj[e]) : 0.f;
        *reinterpret_cast<f32x4*>(sAD + b * AD_BLK + n16 * AD_ROW + 4 * q4) = rr;
      }
      float bi[NB], eri[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        bi[b] = vec[F_BETA * C + 16 * b + n16];
        eri[b] = vec[F_ER * C + 16 * b + n16];
      }
#pragma unroll
      for (int b1 = 1; b1 < NB; ++b1)
#pragma unroll
        for (int b2 = 0; b2 < b1; ++b2) {
          const f32x4 ec = *reinterpret_cast<const f32x4*>(vec + (F_ER + b1) * C + 16 * b2 + 4 * q4);
          f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s) kk = MM::mma(Kf[b2][s], Kf[b1][s], kk);
          const float sc = bi[b1] * eri[b1];
          f32x4 ra;
#pragma unroll
          for (int e = 0; e < 4; ++e) ra[e] = sc * kk[e] * ec[e];
          lds_st<bf16x4>(sAT, cc_frag[b2 >> 1] + 16 * CCR * b1 + 8 * (b2 & 1), cvt4(ra));
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      {
        const float* A = sAD + q4 * AD_BLK;
        float ar[16][16];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          const float* row = A + i * AD_ROW;
#pragma unroll
          for (int l = 0; l + 4 <= i; l += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(row + l);
            ar[i][l] = v[0]; ar[i][l + 1] = v[1]; ar[i][l + 2] = v[2]; ar[i][l + 3] = v[3];
          }
          const int l0 = i & ~3;
          if (i & 2) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(row + l0);
            ar[i][l0] = v[0]; ar[i][l0 + 1] = v[1];
          }
          if (i & 1) ar[i][i - 1] = row[i - 1];
        }
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tc[i] = (i == n16) ? 1.f : 0.f;
#pragma unroll
        for (int l = 0; l < 15; ++l)
#pragma unroll
          for (int i = l + 1; i < 16; ++i) tc[i] = __builtin_fmaf(-ar[i][l], tc[l], tc[i]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          lds_st<bf16x4>(sAT, t_dst[m],
                         bf16x4{(__bf16)tc[4 * m], (__bf16)tc[4 * m + 1], (__bf16)tc[4 * m + 2], (__bf16)tc[4 * m + 3]});
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bf16x4 Tf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) Tf[b] = lds_read_tr(sAT, t_base[b >> 1] + 16 * CCR * b + 8 * (b & 1));
      F Af[NB][NTS];
#pragma unroll
      for (int b = 1; b < NB; ++b)
#pragma unroll
        for (int s = 0; 32 * s < 16 * b; ++s) Af[b][s] = lds_at<F>(sAT + cc_frag[s] + 16 * CCR * b);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      f32x4 RT[NB][NB];
      bf16x4 RH[NB][NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int col = 0; col <= b; ++col) {
          bf16x4 xh;
          if (col == b) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xh[e] = 4 * q4 + e == n16 ? (__bf16)1.f : (__bf16)0.f;
          } else {
            f32x4 rr = zero4, r16 = zero4;
#pragma unroll
            for (int s = 0; 32 * s < 16 * b; ++s) {
              if (2 * s + 1 < col) continue;
              if (2 * s + 1 >= b) r16 = MM::mma16(MM::lo(Af[b][s]), RH[2 * s][col], r16);
              else if (2 * s < col) r16 = MM::mma16(MM::hi(Af[b][s]), RH[2 * s + 1][col], r16);
              else rr = MM::mma(Af[b][s], cat(RH[2 * s][col], RH[2 * s + 1][col]), rr);
            }
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = -(rr[e] + r16[e]);
            xh = cvt4(x);
          }
          RT[b][col] = MM::mma16(Tf[b], xh, zero4);
          RH[b][col] = cvt4(RT[b][col]);
        }
      }
      char* tp = sT + (r & 1) * CC_BYTES;
#pragma unroll
      for (int col = 0; col < NB; ++col)
#pragma unroll
        for (int b = col; b < NB; ++b) lds_st<bf16x4>(tp, tt_off(b, col), RH[b][col]);
    };
    for (int it = 0; it < NIT; ++it) {
      const int r = it - 1;
      if (r >= 0 && r < NC) gram_solve(r);
      lds_barrier();
    }
  } else {
    // ============================================================= P waves
    // P^T of row block b1 (token i), column block b2 >= b1 (token j):
    // (k_i . q_j) exp(gamma_j - gamma_i), j >= i.  Lane (n16, q4) holds row
    // i = 16 b1 + n16 and columns j = 16 b2 + 4 q4 + e.
    auto p_wave = [&](auto oc) {
      constexpr int o = decltype(oc)::value;
      auto make_pt = [&](int r) {
        const char* sk = sK + (r % NKR) * KQ_BYTES;
        const char* sq = sQ + (r % NQR) * KQ_BYTES;
        const float* vec = vec_of(r);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int b1 = own_tb(o, i);
          F Kf[NKS];
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b1);
          const float li = vec[F_LAM * C + 16 * b1 + n16];
          f32x4 pb[NB];
#pragma unroll
          for (int b2 = 0; b2 < NB; ++b2) {
            pb[b2] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (b2 < b1) continue;
            F Qf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) Qf[s] = lds_at<F>(sq + kq_frag[s] + 16 * KQR * b2);
            f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) pq = MM::mma(Qf[s], Kf[s], pq);
            if (b2 > b1) {
              // exp(gamma_j - gamma_{16 b2}) exp(gamma_{16 b2} - gamma_i), both <= 1
              const f32x4 ej = *reinterpret_cast<const f32x4*>(vec + F_ER * C + 16 * b2 + 4 * q4);
              const float ei = vec[(F_ER + b2) * C + 16 * b1 + n16];
#pragma unroll
              for (int e = 0; e < 4; ++e) pb[b2][e] = pq[e] * (ej[e] * ei);
            } else {
              const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + F_LAM * C + 16 * b1 + 4 * q4);
#pragma unroll
              for (int e = 0; e < 4; ++e) pb[b2][e] = 4 * q4 + e >= n16 ? pq[e] * exp2_fast(lj[e] - li) : 0.f;
            }
          }
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            if (2 * s + 1 < b1) continue;
            lds_st<F>(sP, ((b1 * NTS + s) * 64 + lane) * 16, MM::from_acc(pb[2 * s], pb[2 * s + 1]));
          }
        }
        flag_release(&sFLAG[o], r + 1);
      };
      for (int it = 0; it < NIT; ++it) {
        const int r = it - 2;
        if (r >= 0) make_pt(r);
        lds_barrier();
      }
    };
    if (wave == W_P) p_wave(IC<0>{});
    else p_wave(IC<1>{});
  }
}

// ====================================================================
// gradient kernels
//
// gdn_grad_kernel: one workgroup per (chunk slot, head), four waves, wave w
// owning the tokens of row block w.  From the saved M and dM' (key-major,
// staged in LDS a key block at a time), U and dX (read as operands), and the
// chunk's q, k (LDS), v and dO:
//   phase 1 (the 64 x 64 blocks (w, b) of the lower triangle, b <= w): S =
//       K K^T, Q K^T, dX U^T and dO U^T; then G = dA . E . beta_i and
//       dP . E (bf16 tiles, rows in pi order), and the row and column sums
//       of Z and the row sums of dA . (S . E) per block;
//   phase 2 (dq and dk as transposed 16 x 16 tiles, keys by tokens, over
//       the eight key blocks; each block's M and dM' rows copied to LDS
//       while the previous block is worked),
//       dv, and the per-token sums over the keys;
//   phase 3 (one wave): dg (a reverse sum over the chunk) and dbeta from
//       those sums.
// A key-side operand (rows = keys) comes from
// LDS, by plain reads (M, dM') or transposing ones (q, k); a token-side
// one (rows = tokens) from the record, v and dO (natural value order) or
// from the bf16 tiles (pi token order).
//
// Two workgroups share a CU (72 KB of LDS and at most 256 VGPRs per wave):
// one's loads overlap the other's products.
namespace gk {
constexpr int NWG = 4;  // waves per gradient workgroup
// Per-token partial sums for dg and dbeta (LDS, fp32 offsets): the row sums
// of Z, its column sums and the row sums of dA . (S . E) for each 16 x 16
// block (b1, b2), 16 each; the per-token sums dO M^T . q, dX M^T . k and
// U dM'^T . k (64 each); dX . v per token; <M, dM'> over each wave's keys.
constexpr int SUM_ZR = 0, SUM_ZC = 256, SUM_BR = 512, SUM_S3 = 768, SUM_XV = 960, SUM_GC = 1024,
              SUM_FLOATS = 1028;
}  // namespace gk

// The chunk that slot sigma holds: sequence n is the largest with
// floor(start_n / C) + n <= sigma (slots of a sequence are consecutive).
struct SlotChunk {
  long t0;   // first token row
  int Lc;    // tokens of the chunk (0: a slot no chunk uses)
};
__device__ static inline SlotChunk slot_chunk(const gdn_launch::BwdParams& p, long sigma) {
  auto start_of = [&](int n) { return p.cu ? (long)p.cu[n] : (long)n * p.T; };
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start_of(mid) / C + mid <= sigma) lo = mid;
    else hi = mid - 1;
  }
  const int n = __builtin_amdgcn_readfirstlane(lo);
  const long start = start_of(n);
  const int len = p.cu ? p.cu[n + 1] - p.cu[n] : p.T;
  const int c = (int)(sigma - (start / C + n));
  if (c < 0 || (long)c * C >= len) return SlotChunk{0, 0};
  return SlotChunk{start + (long)c * C, min(C, len - c * C)};
}

__global__ __launch_bounds__(64 * gk::NWG, 2) void gdn_grad_kernel(const gdn_launch::BwdParams p) {
  using MM = Mma<__bf16>;
  using F = bf16x8;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __attribute__((aligned(16))) char sQ[KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sK[KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sPE[CC_BYTES];  // dP . E, rows in pi order
  __shared__ __attribute__((aligned(16))) char sG[CC_BYTES];   // G = dA . E . beta_i, rows in pi order
  __shared__ __attribute__((aligned(16))) float sVEC[NF * C];
  __shared__ __attribute__((aligned(16))) float sGB[2 * C];
  __shared__ float sums[gk::SUM_FLOATS];  // per-token partial sums for dg and dbeta
  // M and dM' rows of one key block (16 rows of 256 bytes each, granules
  // permuted as in the q / k tiles), double-buffered over the key blocks
  __shared__ __attribute__((aligned(16))) char sMD[2][2 * 16 * KQR];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4, n16 = lane & 15;
  const int H = p.H, hh = blockIdx.y;
  const long sigma = blockIdx.x;
  const SlotChunk sc = slot_chunk(p, sigma);
  if (sc.Lc == 0) return;  // a slot no chunk uses (uniform)
  const long t0 = sc.t0;
  const int Lc = sc.Lc;
  const long kq_stride = (long)H * KQR;
  const long v_stride = (long)H * DV * 2;
  const char* rec = p.sv + (sigma * H + hh) * gdn_launch::BWD_REC_BYTES;

  // ---------------------------------------------------- phase 0: loads
  // q and k (16 copies each; wave w issues [8 w, 8 w + 8) of the 32), g and
  // beta, then this wave's operands in registers: phase 1 starts once the
  // copies have landed in every wave.
  constexpr int GK_QK = 2 * KQ_INS / gk::NWG;
  static_assert(GK_QK * gk::NWG == 2 * KQ_INS, "copies per wave");
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (t0 * H + hh) * KQR, (long)Lc * kq_stride);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (t0 * H + hh) * KQR, (long)Lc * kq_stride);
#pragma unroll
    for (int x = 0; x < GK_QK; ++x) {
      const int i = GK_QK * wave + x;
      const int ii = i % KQ_INS, r = ii * KQ_RPI + lane / GR;
      const int so = (int)(r * kq_stride) + 16 * ((lane % GR) ^ swz_kq<GR>(r));
      copy_to_lds(i < KQ_INS ? rq : rk, (i < KQ_INS ? sQ : sK) + ii * 1024, so);
    }
    if (wave == 0) {
      copy_to_lds4(make_rsrc(p.g + t0 * H + hh, (long)Lc * H * 4), reinterpret_cast<char*>(sGB), lane * H * 4);
      copy_to_lds4(make_rsrc(p.beta + t0 * H + hh, (long)Lc * H * 4), reinterpret_cast<char*>(sGB + C),
                   lane * H * 4);
    }
  }
  asm volatile("" ::: "memory");  // the register loads below are issued after the copies
  // token-side operands of this wave: rows 16 ib + n16, values 32 s + 8 q4 .. +7
  const int ib = wave;
  const int irow = 16 * ib + n16;
  F dOr[NKS], dXr[NKS], Ur[NKS];
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, gdn_launch::BWD_REC_BYTES);
  {
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dO + (t0 * H + hh) * DV * 2, (long)Lc * v_stride);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int col = (32 * s + 8 * q4) * 2;
      dOr[s] = __builtin_bit_cast(F, __builtin_amdgcn_raw_buffer_load_b128(rd, (int)(irow * v_stride) + col, 0, 0));
      dXr[s] = __builtin_bit_cast(
          F, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)gdn_launch::BWD_OFF_DX + irow * DV * 2 + col, 0, 0));
      Ur[s] = __builtin_bit_cast(
          F, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)gdn_launch::BWD_OFF_U + irow * DV * 2 + col, 0, 0));
    }
  }
  // U rows of the phase-1 column blocks b2 < ib (past the record's end,
  // reading zeros without a fetch, for b2 >= ib; block ib is Ur)
  F Uc[NB - 1][NKS];
#pragma unroll
  for (int b2 = 0; b2 < NB - 1; ++b2) {
    const int base = b2 < ib ? (int)gdn_launch::BWD_OFF_U + (16 * b2 + n16) * DV * 2 : (int)gdn_launch::BWD_REC_BYTES;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      Uc[b2][s] = __builtin_bit_cast(F, __builtin_amdgcn_raw_buffer_load_b128(rr, base + (32 * s + 8 * q4) * 2, 0, 0));
  }
  // M and dM' rows of key block ab into buffer b: eight 1 KB copies (four
  // rows each), two per wave
  auto issue_md = [&](int ab, int b) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int i = 2 * wave + x, part = i >> 2, ii = i & 3;
      const int r = ii * KQ_RPI + lane / GR;
      const int so = (int)(part ? gdn_launch::BWD_OFF_DM : gdn_launch::BWD_OFF_M) + (16 * ab + r) * KQR +
                     16 * ((lane % GR) ^ swz_kq<GR>(r));
      copy_to_lds(rr, sMD[b] + part * 16 * KQR + ii * 1024, so);
    }
  };
  static_assert(2 * gk::NWG * 1024 == 2 * 16 * KQR, "copies per key block");
  issue_md(0, 0);
  // the q / k copies have landed, in every wave; the register loads (3 NKS
  // + (NB - 1) NKS of them) and the first key block's two copies may still
  // be in flight
  constexpr int GK_REG = (3 + NB - 1) * NKS + 2;
  static_assert(GK_REG <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(GK_REG) : "memory");
  if (wave == 0) {
    // per-token vectors (as the forward's loader)
    const float lam = wave_prefix_sum(sGB[lane] * kLog2e, lane);
    const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), C - 1));
    float lb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) lb[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 16 * b));
    const int blk = lane >> 4;
    float lown = lb[0];
#pragma unroll
    for (int b = 1; b < NB; ++b) lown = blk == b ? lb[b] : lown;
    sVEC[F_BETA * C + lane] = sGB[C + lane];
    sVEC[F_LAM * C + lane] = lam;
    sVEC[F_GAM * C + lane] = exp2_fast(lam);
    sVEC[F_W * C + lane] = exp2_fast(lamC - lam);
    sVEC[F_ER * C + lane] = exp2_fast(lam - lown);
#pragma unroll
    for (int b = 1; b < NB; ++b) sVEC[(F_ER + b) * C + lane] = lane < 16 * b ? exp2_fast(lb[b] - lam) : 0.f;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const float* vec = sVEC;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------- phase 1
  {
    int kq_frag[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) kq_frag[s] = n16 * KQR + 16 * ((4 * s + q4) ^ swz_kq<GR>(n16));
    const int b1 = ib;
    const int i = 16 * b1 + n16;
    const float li = vec[F_LAM * C + i], bi = vec[F_BETA * C + i], eri = vec[F_ER * C + i];
    F Kb1[NKS], Qb1[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      Kb1[s] = lds_at<F>(sK + kq_frag[s] + 16 * KQR * b1);
      Qb1[s] = lds_at<F>(sQ + kq_frag[s] + 16 * KQR * b1);
    }
#pragma unroll
    for (int b2 = 0; b2 < NB; ++b2) {
      if (b2 > b1) continue;
      f32x4 S = zero4, QK = zero4, XU = zero4, OU = zero4;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const F kb2 = lds_at<F>(sK + kq_frag[s] + 16 * KQR * b2);
        const F ub = (b2 == NB - 1 || b2 == b1) ? Ur[s] : Uc[b2 < NB - 1 ? b2 : 0][s];
        S = MM::mma(kb2, Kb1[s], S);
        QK = MM::mma(kb2, Qb1[s], QK);
        XU = MM::mma(ub, dXr[s], XU);
        OU = MM::mma(ub, dOr[s], OU);
      }
      // lane: row i, columns j = 16 b2 + 4 q4 + e
      f32x4 E;
      if (b2 < b1) {
        const f32x4 ec = *reinterpret_cast<const f32x4*>(vec + (F_ER + b1) * C + 16 * b2 + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) E[e] = eri * ec[e];
      } else {
        const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + F_LAM * C + 16 * b2 + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) E[e] = 4 * q4 + e <= n16 ? exp2_fast(li - lj[e]) : 0.f;
      }
      f32x4 Gv, PEv;
      float zr = 0.f, br = 0.f, zc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool strict = b2 < b1 || 4 * q4 + e < n16;
        const float se = S[e] * E[e];
        const float dA = strict ? -XU[e] : 0.f;
        const float dP = OU[e];  // E is zero above the diagonal
        Gv[e] = dA * E[e] * bi;
        PEv[e] = dP * E[e];
        const float z = strict ? __builtin_fmaf(dA, bi * se, dP * (QK[e] * E[e])) : 0.f;
        zr += z;
        zc[e] = z;
        br = __builtin_fmaf(dA, se, br);
      }
      const int toff = i * CCR + 16 * ((4 * (b2 >> 1) + q4) ^ swz_cc<C>(i)) + 8 * (b2 & 1);
      lds_st<bf16x4>(sPE, toff, cvt4(PEv));
      lds_st<bf16x4>(sG, toff, cvt4(Gv));
      {
        // row sums over the block's 16 columns (the four lane groups), column
        // sums over its 16 rows (the sixteen lanes of a group)
        zr += __shfl_xor(zr, 16);
        zr += __shfl_xor(zr, 32);
        br += __shfl_xor(br, 16);
        br += __shfl_xor(br, 32);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int d = 1; d < 16; d <<= 1) zc[e] += __shfl_xor(zc[e], d);
        const int blk = b1 * NB + b2;
        if (q4 == 0) {
          sums[gk::SUM_ZR + blk * 16 + n16] = zr;
          sums[gk::SUM_BR + blk * 16 + n16] = br;
        }
        if (n16 == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sums[gk::SUM_ZC + blk * 16 + 4 * q4 + e] = zc[e];
        }
      }
    }
  }
  // the tiles are complete
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---------------------------------------------------- phase 2
  {
    // token-side tiles for this wave's rows: dP . E and G rows (pi order),
    // G^T and (dP . E)^T rows by transposing reads; blocks outside the
    // lower (resp. upper) triangle are zero.
    F PEr[NTS], Gr[NTS], GTr[NTS], PETr[NTS];
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const int off = irow * CCR + 16 * ((4 * ts + q4) ^ swz_cc<C>(irow));
      F a = lds_at<F>(sPE + off), b = lds_at<F>(sG + off);
      if (2 * ts > ib) {
        a = F{}; b = F{};
      } else if (2 * ts + 1 > ib) {
        a[4] = a[5] = a[6] = a[7] = (__bf16)0.f;
        b[4] = b[5] = b[6] = b[7] = (__bf16)0.f;
      }
      PEr[ts] = a;
      Gr[ts] = b;
      // rows j = 32 ts + 4 q4 + (n16 >> 2) (+16), columns 16 ib + 4 (n16 & 3) .. +3
      const int jl = 32 * ts + 4 * q4 + (n16 >> 2), jh = jl + 16;
      const int cg = 4 * (ib >> 1) + (n16 & 3), ch = 8 * (ib & 1);
      const bf16x4 pl = lds_read_tr(sPE, jl * CCR + 16 * (cg ^ swz_cc<C>(jl)) + ch);
      const bf16x4 ph = lds_read_tr(sPE, jh * CCR + 16 * (cg ^ swz_cc<C>(jh)) + ch);
      const bf16x4 gl = lds_read_tr(sG, jl * CCR + 16 * (cg ^ swz_cc<C>(jl)) + ch);
      const bf16x4 gh = lds_read_tr(sG, jh * CCR + 16 * (cg ^ swz_cc<C>(jh)) + ch);
      F pt{pl[0], pl[1], pl[2], pl[3], ph[0], ph[1], ph[2], ph[3]};
      F gt{gl[0], gl[1], gl[2], gl[3], gh[0], gh[1], gh[2], gh[3]};
      if (2 * ts + 1 < ib) {
        pt = F{}; gt = F{};
      } else if (2 * ts < ib) {
        pt[0] = pt[1] = pt[2] = pt[3] = (__bf16)0.f;
        gt[0] = gt[1] = gt[2] = gt[3] = (__bf16)0.f;
      }
      PETr[ts] = pt;
      GTr[ts] = gt;
    }
    const float gi = vec[F_GAM * C + irow], wi = vec[F_W * C + irow], bgi = vec[F_BETA * C + irow] * gi;
    float sq_ = 0.f, sx_ = 0.f, sw_ = 0.f, gc = 0.f;
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc(p.dq + (t0 * H + hh) * KQR, (long)Lc * kq_stride);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(p.dk + (t0 * H + hh) * KQR, (long)Lc * kq_stride);
#pragma unroll 1
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int m = 0; m < NKB / 2; ++m) {
      const int ab = NKB / 2 * hf + m;
      // key block ab's copies have landed in every wave (after them each
      // wave issued only the previous block's two stores), and every wave
      // is done with the other buffer; then the next block's copies go out
      const int buf = m & 1;
      if (ab == 0) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
      if (ab + 1 < NKB) issue_md(ab + 1, buf ^ 1);
      // key-side operands, rows a = 16 ab + n16: M and dM' (LDS), k and q
      // (transposing reads)
      F MTa[NKS], DTa[NKS], KTa[NTS], QTa[NTS];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int fo = n16 * KQR + 16 * ((4 * s + q4) ^ swz_kq<GR>(n16));
        MTa[s] = lds_at<F>(sMD[buf] + fo);
        DTa[s] = lds_at<F>(sMD[buf] + 16 * KQR + fo);
      }
#pragma unroll
      for (int ts = 0; ts < NTS; ++ts) {
        const int jl = 32 * ts + 4 * q4 + (n16 >> 2), jh = jl + 16;
        const int mg = 2 * ab + ((n16 & 3) >> 1), mh = 8 * (n16 & 1);
        const bf16x4 kl = lds_read_tr(sK, jl * KQR + 16 * (mg ^ swz_kq<GR>(jl)) + mh);
        const bf16x4 kh = lds_read_tr(sK, jh * KQR + 16 * (mg ^ swz_kq<GR>(jh)) + mh);
        const bf16x4 ql = lds_read_tr(sQ, jl * KQR + 16 * (mg ^ swz_kq<GR>(jl)) + mh);
        const bf16x4 qh = lds_read_tr(sQ, jh * KQR + 16 * (mg ^ swz_kq<GR>(jh)) + mh);
        KTa[ts] = F{kl[0], kl[1], kl[2], kl[3], kh[0], kh[1], kh[2], kh[3]};
        QTa[ts] = F{ql[0], ql[1], ql[2], ql[3], qh[0], qh[1], qh[2], qh[3]};
      }
      f32x4 aQ = zero4, aXM = zero4, aUD = zero4;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        aQ = MM::mma(MTa[s], dOr[s], aQ);
        aXM = MM::mma(MTa[s], dXr[s], aXM);
        aUD = MM::mma(DTa[s], Ur[s], aUD);
      }
      if (m == ib) {
        // <M, dM'> over this wave's 32 keys (all four waves: all 128)
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) gc = __builtin_fmaf((float)MTa[s][e], (float)DTa[s][e], gc);
      }
      // lane: token irow, keys 16 ab + 4 q4 + e; q and k of them
      const int kgo = irow * KQR + 16 * ((2 * ab + (q4 >> 1)) ^ swz_kq<GR>(irow)) + 8 * (q4 & 1);
      const bf16x4 qv = lds_ld<bf16x4>(sQ, kgo), kv = lds_ld<bf16x4>(sK, kgo);
      f32x4 aK;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sq_ = __builtin_fmaf((float)qv[e], aQ[e], sq_);
        sx_ = __builtin_fmaf((float)kv[e], aXM[e], sx_);
        sw_ = __builtin_fmaf((float)kv[e], aUD[e], sw_);
        aQ[e] *= gi;
        aK[e] = __builtin_fmaf(-bgi, aXM[e], wi * aUD[e]);
      }
#pragma unroll
      for (int ts = 0; ts < NTS; ++ts) {
        if (2 * ts <= ib) {
          aQ = MM::mma(KTa[ts], PEr[ts], aQ);
          aK = MM::mma(KTa[ts], Gr[ts], aK);
        }
        if (2 * ts + 1 >= ib) {
          aK = MM::mma(KTa[ts], GTr[ts], aK);
          aK = MM::mma(QTa[ts], PETr[ts], aK);
        }
      }
      const int so = (int)(irow * kq_stride) + (16 * ab + 4 * q4) * 2;
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(aQ)), rdq, so, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(aK)), rdk, so, 0, 0);
    }
    // per-token sums over the keys: over the four lane groups
#pragma unroll
    for (int d = 16; d <= 32; d <<= 1) {
      sq_ += __shfl_xor(sq_, d);
      sx_ += __shfl_xor(sx_, d);
      sw_ += __shfl_xor(sw_, d);
    }
    if (q4 == 0) {
      float* s3 = sums + gk::SUM_S3;
      s3[irow] = sq_;
      s3[C + irow] = sx_;
      s3[2 * C + irow] = sw_;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) gc += __shfl_xor(gc, d);
    if (lane == 0) sums[gk::SUM_GC + ib] = gc;
    {
      // dv = diag(beta) dX (rows irow, values 32 s + 8 q4 .. +7), and dX . v
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (t0 * H + hh) * DV * 2, (long)Lc * v_stride);
      uint32_t Vr[NKS][4];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const u32x4 vv = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(irow * v_stride) + (32 * s + 8 * q4) * 2, 0, 0);
        Vr[s][0] = vv[0]; Vr[s][1] = vv[1]; Vr[s][2] = vv[2]; Vr[s][3] = vv[3];
      }
      const float bt = vec[F_BETA * C + irow];
      const __amdgpu_buffer_rsrc_t rdv = make_rsrc(p.dv + (t0 * H + hh) * DV * 2, (long)Lc * v_stride);
      float xv = 0.f;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        F o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)dXr[s][e];
          const uint32_t pr = Vr[s][e >> 1];
          const float vv = __uint_as_float((e & 1) ? (pr & 0xffff0000u) : (pr << 16));
          xv = __builtin_fmaf(x, vv, xv);
          o[e] = (__bf16)(bt * x);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rdv,
                                               (int)(irow * v_stride) + (32 * s + 8 * q4) * 2, 0, 0);
      }
      xv += __shfl_xor(xv, 16);
      xv += __shfl_xor(xv, 32);
      if (q4 == 0) sums[gk::SUM_XV + irow] = xv;
    }
  }
  // every wave's sums are in LDS (no wait for the global stores)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---------------------------------------------------- phase 3
  if (wave == 0) {
    const int t = lane;
    const long th = (t0 + t) * H + hh;
    const float Gt = vec[F_GAM * C + t], wt = vec[F_W * C + t], bt = vec[F_BETA * C + t];
    const int tb = t >> 4, tr = t & 15, last = Lc - 1;
    float rz = 0.f, cz = 0.f, b2 = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b <= tb) {
        rz += sums[gk::SUM_ZR + (tb * NB + b) * 16 + tr];
        b2 += sums[gk::SUM_BR + (tb * NB + b) * 16 + tr];
      }
      if (b >= tb) cz += sums[gk::SUM_ZC + (b * NB + tb) * 16 + tr];
    }
    float gc = 0.f;
#pragma unroll
    for (int w = 0; w < gk::NWG; ++w) gc += sums[gk::SUM_GC + w];
    const float* s3 = sums + gk::SUM_S3;
    const float sQv = s3[t], sXv = s3[C + t], sWv = s3[2 * C + t];
    const float dGam = __builtin_fmaf(-bt, sXv, sQv) + (t == last ? gc : 0.f);
    const float dbeta = __builtin_fmaf(-Gt, sXv, sums[gk::SUM_XV + t]) + b2;
    const float dgam = t < Lc ? __builtin_fmaf(dGam, Gt, rz - cz) : 0.f;  // dgamma without the w terms
    const float dww = t < Lc ? sWv * wt : 0.f;                              // dw . w
    // dg_t = sum_{u >= t} dgamma_u; the w terms (-dw_u w_u at every token,
    // +sum_u dw_u w_u at the last) enter as they add up after the reverse
    // sum, sum_{u < t} dw_u w_u, which cancels nothing large under strong
    // decay.  The suffix sum is a prefix sum over the lanes in reverse
    // order, the exclusive prefix sum an inclusive one moved up a lane:
    // neither subtracts a total (fixed addition order: deterministic).
    const float rev = __shfl(dgam, C - 1 - t);
    const float suf = __shfl(wave_prefix_sum(rev, t), C - 1 - t);
    const float inc = wave_prefix_sum(dww, t);
    // every lane takes part in the cross-lane read (a lane left out of it
    // would not supply its value to the next one), then lane 0 drops it
    const float prev = __shfl(inc, (t + C - 1) & (C - 1));
    const float exc = t > 0 ? prev : 0.f;
    const float acc = suf + exc;
    if (t < Lc) {
      p.dg[th] = acc;
      p.dbeta[th] = dbeta;
    }
  }
}

}  // namespace

namespace gdn_launch {

long long bwd_full_ws_bytes(int B, long ttot, int H) {
  return (long long)((ttot / fk::C) + B) * H * BWD_REC_BYTES;
}

int bwd_full(const BwdParams& p, hipStream_t stream) {
  if (p.B <= 0) return GDN_OK;
  // states: the forward recurrence saving M and U
  FullParams fp;
  fp.q = p.q;
  fp.k = p.k;
  fp.v = p.v;
  fp.g = p.g;
  fp.beta = p.beta;
  fp.h0 = p.h0;
  fp.cu = p.cu;
  fp.out = nullptr;
  fp.hT = p.hT;
  fp.B = p.B;
  fp.T = p.T;
  fp.H = p.H;
  fp.seg_max = p.seg_max;
  fp.seg_cap = p.seg_cap;
  fp.nslot = p.nslot;
  fp.sv = p.sv;
  const long nwg = (long)p.nslot * p.H;
  const long ngrad = (long)p.nchunk;
  if (nwg > 0x7fffffffL || ngrad > 0x7fffffffL || p.H > 65535) return GDN_ERR_INVALID_ARG;
  if (nwg > 0) {
    if (!p.states_saved) {
      const int rc = fwd_full_save(fp, stream);
      if (rc != GDN_OK) return rc;
    }
    hipLaunchKernelGGL(gdn_adjoint_kernel, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
  }
  if (ngrad > 0) {
    hipLaunchKernelGGL(gdn_grad_kernel, dim3((unsigned)ngrad, (unsigned)p.H), dim3(64 * gk::NWG), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
  }
  return GDN_OK;
}

}  // namespace gdn_launch
