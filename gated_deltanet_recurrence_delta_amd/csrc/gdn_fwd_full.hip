// Gated-delta-rule forward pass, full-width chunk kernel for gfx950:
// bf16 q/k/v/out, dk = dv = 128, 64-token chunks.
//
// Rule and chunk algebra: as in gdn_fwd.hip (HyMo "Model Architecture
// Walkthrough", sections 5.2.1-5.2.2 for the rule; "v1.0 Architecture &
// Design Spec", section 2.3 and "Optimization Quartet", section 3.2 for the
// chunkwise-parallel evaluation).  With M = S^T (dk x dv), a chunk of C
// tokens, gamma its in-chunk cumulative g, Gam = exp(gamma),
// w = exp(gamma_C - gamma):
//
//     A = strict_lower(diag(beta) (K K^T) * exp(gamma_i - gamma_j)),
//     T = (I + A)^{-1},
//     U = T diag(beta) (V - diag(Gam) K M),
//     O = diag(Gam) Q M + ((Q K^T) * exp(gamma_i - gamma_j), j <= i) U,
//     M <- Gam_C M + K^T diag(w) U.
//
// Decomposition.  One workgroup per (sequence segment, head) owns all 128
// value columns, so the state-independent work of a chunk (the Gram matrix,
// T and the masked decayed Q K^T) is done once per chunk, not once per value
// tile.  A sequence of n chunks is cut into ceil(n / seg_max) segments of
// equal length; the cut depends only on the sequence's own length, so a
// sequence inside a packed batch is computed exactly as when it runs alone.
// A segment other than the first starts from a zero state at the latest
// chunk boundary behind it from which the product of the per-token
// transition norms is at most e^-HALO_NATS (see gdn_device.h), or at the
// sequence start from h0; the chunks in between (the halo) carry the state
// but store nothing.
//
// Eight waves, two per SIMD, one LDS barrier per step.  Step `it`:
//   column waves 0..3 (one per SIMD; wave j owns value columns 32j..32j+31
//       and that quarter of the state, fp32, in MFMA accumulators for the
//       whole segment): chunk it-2 -- Y = K M, X = diag(beta)(V - Gam Y),
//       U = T X, O^T = diag-scaled M^T Q^T + U^T P^T (stored), the update
//       M <- Gam_C M + K^T diag(w) U.  v comes from HBM straight into
//       registers one step ahead;
//   loader wave 4: copies k of chunk it+1 and q of chunk it (two steps
//       ahead of their readers) from HBM into LDS rings, g and beta of chunk
//       it+1 into registers, the per-token decay vectors of chunk it;
//   Gram wave 5: chunk it-1 -- A (fp32 diagonal blocks, bf16 off-diagonal
//       blocks), the inverses of the 16x16 diagonal blocks of I + A by
//       forward substitution, then T by block substitution on the MFMA;
//   P waves 6, 7: chunk it-2 -- P = (Q K^T) * decay, two of the four 16-row
//       blocks each, published to the column waves through an LDS flag.
//
// Column permutation: state column position r of 16-column block cb holds
// value column 2r + cb (relative to the wave's 32), so that a lane's v
// values come as bf16 pairs and its eight output columns are contiguous
// (one 16-byte store per token row).  State rows are ordered (key_of below)
// so that the state's bf16 fragments come straight from its accumulators in
// natural key order.
//
// No atomics: results are deterministic and bitwise independent of the
// workgroup schedule.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_full_common.h"
#include "gdn_launch.h"

namespace {


// MODE 0: outputs and hT.  MODE 1 (maps): the affine map of one segment
// (p.ws set; see the chunk-map scan below): the recurrence over the
// segment's chunks from the identity with v = 0 (giving P) or from zero
// (from h0 for the first segment) with the real v (giving Q), no outputs.
// MODE 3 (training forward, p.sv set): MODE 0 and MODE 2 at once -- the
// outputs and hT, and every chunk's saved state and U.
// MODE 2 (states for the backward pass, p.sv set): the recurrence as in
// MODE 0 without outputs; every chunk's entry state M and its U are saved
// in bf16 (see gdn_launch.h).
template <int MODE>
__global__ __launch_bounds__(64 * fk::NW, 1) void gdn_full_kernel(const gdn_launch::FullParams p) {
  constexpr bool MAPS = MODE == 1;
  constexpr bool SAVE = MODE == 2 || MODE == 3;
  constexpr bool NOOUT = MODE == 1 || MODE == 2;  // no outputs: no q, no P waves
  using namespace fk;
  using MM = Mma<__bf16>;
  using F = bf16x8;
  constexpr float kLog2e = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) char sK[NKR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sQ[NQR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sAT[CC_BYTES];     // A (off-diagonal) and T_bb^T
  __shared__ __attribute__((aligned(16))) char sT[2 * CC_BYTES];  // (T diag(beta))^T of two chunks
  __shared__ __attribute__((aligned(16))) char sP[CC_BYTES];      // P, lane-major fragments
  __shared__ __attribute__((aligned(16))) float sVEC[NVEC * NF * C];
  __shared__ __attribute__((aligned(16))) float sAD[NB * AD_BLK];
  __shared__ __attribute__((aligned(16))) float sGB[2 * 2 * C];  // g, beta of two chunks
  // Flags, chunk index + 1: [0], [1] P published by P wave 0 / 1.
  __shared__ int sFLAG[4];
  __shared__ int sPICK[2];
  __shared__ int sSTART;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4, n16 = lane & 15;
  const int src = lane & 15;  // source lane of a transposing read
  const int H = p.H;

  // ---------------------------------------------------- which segment
  // The maps pass has two workgroups per segment slot: even ones compose
  // Q, odd ones P.
  const int wslot = blockIdx.x / H, hh = blockIdx.x % H;
  const int slot = MAPS ? wslot >> 1 : wslot;
  const bool map_p = MAPS && (wslot & 1);
  int bseq, seg;
  long rowbase;
  int len;
  if (p.cu) {
    // Slots of sequence n: [floor(cu[n] / S) + n, + its segment count),
    // S = seg_max * C tokens (slot n when sequences are never cut).  The
    // ranges are disjoint and increasing in n.
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
  // Chunk slot of the sequence's first chunk (backward records).
  const long cslot0 = rowbase / C + bseq;

  // Segment range [c0, c1) of chunks whose outputs this workgroup stores,
  // and where its recurrence starts (cs <= c0).
  int nch, seg_len, nseg;
  seg_layout(len, p.seg_max, p.seg_cap, nch, seg_len, nseg);
  const int c0 = seg * seg_len;
  const int c1 = min(c0 + seg_len, nch);
  // Maps are needed for every segment but the last; P not for the first,
  // whose Q starts from h0 and is already the next segment's entry state.
  if (MAPS && (seg >= nseg - 1 || (seg == 0 && map_p))) return;  // uniform over the workgroup
  // With the scan, a cut sequence's segments start exactly at c0 (from the
  // scanned entry state); otherwise a segment starts at its halo.
  const bool exact = p.ws != nullptr && nseg > 1;
  if (threadIdx.x < 4) sFLAG[threadIdx.x] = 0;
  if (wave == 0) {
    int cs = c0;
    float acc = 0.f;  // log of the transition-norm product over chunks [cs, c0)
    while (!exact && cs > 0 && acc > -HALO_NATS) {
      --cs;  // chunks before c0 are whole: every lane holds a token
      const long th = (rowbase + (long)cs * C + lane) * H + hh;
      const uint4* kr = reinterpret_cast<const uint4*>(p.k + th * KQR);
      float n2 = 0.f;
#pragma unroll
      for (int i = 0; i < DK / 8; ++i) {
        const uint4 w = kr[i];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = __uint_as_float(u[j] << 16), hi = __uint_as_float(u[j] & 0xffff0000u);
          n2 = __builtin_fmaf(lo, lo, n2);
          n2 = __builtin_fmaf(hi, hi, n2);
        }
      }
      const float f = fabsf(1.f - p.beta[th] * n2);
      float e = p.g[th] + (f > 1.f ? __logf(f) : 0.f);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) e += __shfl_xor(e, d);
      acc += e;
    }
    if (lane == 0) sSTART = cs;
  }
  // The loader requests the first chunk's k, g and beta while the start is
  // still being searched for, assuming the start the search usually finds:
  // c0 itself without a search, else the chunk before it (one chunk of
  // decay reaches e^-HALO_NATS).  Another start requests them again below.
  const int cs_guess = (exact || c0 == 0) ? c0 : c0 - 1;
  if (wave == W_L) {
    const int rb = (int)(rowbase + (long)cs_guess * C);
    const long ln = (long)min(len, c1 * C) - (long)cs_guess * C;
    if (ln > 0) {
      const long kq_stride = (long)H * KQR;
      char* d = reinterpret_cast<char*>(sGB);
      copy_to_lds4(make_rsrc(p.g + (long)rb * H + hh, ln * H * 4), d, lane * H * 4);
      copy_to_lds4(make_rsrc(p.beta + (long)rb * H + hh, ln * H * 4), d + C * 4, lane * H * 4);
      const __amdgpu_buffer_rsrc_t r = make_rsrc(p.k + (long)rb * kq_stride + hh * KQR, ln * kq_stride);
#pragma unroll
      for (int i = 0; i < KQ_INS; ++i) {
        const int rr = i * KQ_RPI + lane / GR;
        copy_to_lds(r, sK + i * 1024, (int)(rr * kq_stride) + 16 * ((lane % GR) ^ swz_kq<GR>(rr)));
      }
    }
  }
  __syncthreads();
  const int cs = sSTART;
  const bool write_hT = (MODE == 0 || MODE == 3) && c1 >= nch;
  // This (segment slot, head)'s P, Q and entry state S in the workspace.
  float* const wsm = p.ws ? p.ws + ((long)slot * H + hh) * 3 * DK * DV : nullptr;
  // Where the recurrence's starting state comes from (an empty descriptor
  // reads zeros): P starts from the identity (set below), the first
  // segment's Q and an uncut or halo start at the sequence start from h0,
  // an exact output start from the scanned state, anything else from zero.
  const float* st_src = p.hT;
  long st_bytes = 0;
  if (MAPS) {
    if (!map_p && seg == 0 && p.h0) {
      st_src = p.h0 + (long)chain * DK * DV;
      st_bytes = (long)DK * DV * 4;
    }
  } else if (exact) {
    st_src = wsm + 2 * DK * DV;
    st_bytes = (long)DK * DV * 4;
  } else if (p.h0 && cs == 0) {
    st_src = p.h0 + (long)chain * DK * DV;
    st_bytes = (long)DK * DV * 4;
  }
  const int store_from = c0 - cs;
  rowbase = __builtin_amdgcn_readfirstlane((int)(rowbase + (long)cs * C));
  len = __builtin_amdgcn_readfirstlane(min(len, c1 * C) - cs * C);
  const int NC = (len + C - 1) / C;
  const int NIT = NC > 0 ? NC + 2 : 0;
  const long kq_stride = (long)H * KQR;  // bytes between tokens in q/k
  const long v_stride = (long)H * DV * 2;  // bytes between tokens in v/out
  auto vec_of = [&](int c) { return sVEC + (c % NVEC) * NF * C; };

  // Lane-constant parts of fragment addresses.
  // q/k fragment (row 16 tb + n16, natural slab s): kq_frag[s] + 16*KQR*tb.
  int kq_frag[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kq_frag[s] = n16 * KQR + 16 * ((4 * s + q4) ^ swz_kq<GR>(n16));
  // A-tile fragment (row 16 b + n16, slab s) and 4-wide stores.
  int cc_frag[NTS];
#pragma unroll
  for (int s = 0; s < NTS; ++s) cc_frag[s] = n16 * CCR + 16 * ((4 * s + q4) ^ swz_cc<C>(n16));

  if (wave < NCW) {
    // ========================================================= column waves
    const int j = wave;  // value columns 32 j .. 32 j + 31
    const long sbase = (long)chain * DK * DV;
    // K^T (transposing reads): rows 32 s + 16 hi + 4 q4 + (src >> 2), the
    // 8-byte piece holding keys 32 (b>>1) + 8 (src&3) + 4 (b&1) .. +3 (two
    // lanes of each 32-lane half share a bank pair: 2-way conflicts).
    int kt_base[NKB / 2];
#pragma unroll
    for (int bh = 0; bh < NKB / 2; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      kt_base[bh] = r * KQR + 16 * ((4 * bh + (src & 3)) ^ swz_kq<GR>(r));
    }
    // T as a row operand (transposing read of T^T): rows
    // 32 s + 16 hi + 4 q4 + (src >> 2), columns 16 tb + 4 (src & 3) .. +3.
    int tp_base[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const int r = 4 * q4 + (src >> 2);
      tp_base[tb] = r * CCR + 16 * ((2 * tb + ((src & 3) >> 1)) ^ swz_cc<C>(r)) + 8 * (src & 1);
    }
    // v in accumulator layout: token 16 tb + 4 q4 + e, columns
    // 32 j + 2 n16 .. +1 (one bf16 pair per lane); the token's row offset
    // (16 tb + e) * v_stride is uniform and goes in the scalar offset.
    const int v_lane = (int)(4 * q4 * v_stride) + (32 * j + 2 * n16) * 2;
    // out: token 16 tb + n16, columns 32 j + 8 q4 .. +7.
    const int o_lane = (int)(n16 * v_stride) + (32 * j + 8 * q4) * 2;

    // State: Macc[kb][cb] lane (n16, q4) element e = M[key_of(kb, 4 q4 + e)]
    // [32 j + 2 n16 + cb].  h0 comes through a buffer descriptor that is
    // empty without an initial state (reads return zero), so the 32 loads go
    // out back to back.
    f32x4 Macc[NKB][2];
    {
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(st_src, st_bytes);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(
              rh, (key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16) * 4, 0, 0);
          Macc[kb][0][e] = __uint_as_float(h[0]);
          Macc[kb][1][e] = __uint_as_float(h[1]);
        }
      if constexpr (MAPS) {
        if (map_p) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                Macc[kb][cb][e] = key_of(kb, 4 * q4 + e) == 32 * j + 2 * n16 + cb ? 1.f : 0.f;
        }
      }
    }
    // bf16 state fragments, natural key order 32 s + 8 q4 .. +7 (key_of).
    F Mf[NKS][2];
    auto make_mf = [&]() {
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) Mf[s][cb] = MM::from_acc(Macc[2 * s][cb], Macc[2 * s + 1][cb]);
    };
    make_mf();

    // P's recurrence runs with v = 0: an empty descriptor.
    auto load_v = [&](int c, uint32_t (&Vn)[NB][4]) {
      const long row0 = rowbase + (long)c * C;
      const __amdgpu_buffer_rsrc_t rv =
          make_rsrc(p.v + (row0 * H + hh) * DV * 2, c < NC && !map_p ? (long)(len - c * C) * v_stride : 0);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Vn[tb][e] = __builtin_amdgcn_raw_buffer_load_b32(rv, v_lane, (int)((16 * tb + e) * v_stride), 0);
    };

    // v of chunk c + 1 is loaded into Vn first thing in chunk c's step (a
    // step ahead of its use) and moved to Vb at the end of it.
    uint32_t Vb[NB][4], Vn[NB][4];
    // Chunk c.  Only full-depth (32-long) products are used: where a slab's
    // upper half lies above the diagonal, the row operand holds zeros there.
    // With Tb = T diag(beta), U = Tb (V - diag(Gam) K M).  The recurrence's
    // own path is Y = K M -> Z = -diag(Gam) Y -> U = u + Tb Z ->
    // W = diag(w) U -> M <- Gam_C M + K^T W -> bf16 state; u = Tb V,
    // diag(Gam) Q M and the stores hang off it.
    auto process = [&](int c) {
      // States pass: this chunk's record (empty for halo chunks).
      __amdgpu_buffer_rsrc_t rrec;
      if constexpr (SAVE) {
        rrec = make_rsrc(p.sv + ((cslot0 + cs + c) * H + hh) * gdn_launch::BWD_REC_BYTES,
                         c >= store_from ? gdn_launch::BWD_REC_BYTES : 0);
        // entry state, key-major (key rows of 128 values): lane (n16, q4)
        // holds keys key_of(kb, 4 q4) .. +3 of value columns 32 j + 2 n16
        // (block cb = 0) and the next one (cb = 1), one bf16 pair per key
        // (one lane base; the rest is a per-instruction constant)
        const int m_lane = (int)gdn_launch::BWD_OFF_M + (8 * q4 * DV + 32 * j + 2 * n16) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(cvt_pair(Macc[kb][0][e], Macc[kb][1][e]), rrec,
                                                  m_lane + (32 * (kb >> 1) + 4 * (kb & 1) + e) * DV * 2, 0, 0);
      }
      const char* sk = sK + (c % NKR) * KQ_BYTES;
      const char* sq = sQ + (c % NQR) * KQ_BYTES;
      const char* st = sT + (c & 1) * CC_BYTES;
      const float* vec = vec_of(c);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      load_v(c + 1, Vn);  // unconditional: past the end the descriptor is empty
      asm volatile("" ::: "memory");  // issued here, not later

      // T (lower triangular) as row operands: slab s of row block tb is used
      // for 2 s <= tb, its upper half only when 2 s + 1 <= tb.
      F TPf[NB][NTS];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int s = 0; 2 * s <= tb; ++s) {
          const bf16x4 lo = lds_read_tr(st, tp_base[tb] + 32 * s * CCR);
          F f{};
          f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
          if (2 * s + 1 <= tb) {
            const bf16x4 hi = lds_read_tr(st, tp_base[tb] + (32 * s + 16) * CCR);
            f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
          }
          TPf[tb][s] = f;
        }
      // u = T diag(beta) V (independent of the state): the bf16 pairs of v
      // regroup into fragments by byte permutes (column 2 n16 + cb is the
      // low half of each pair for cb = 0, the high half for cb = 1).
      F XVf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const uint32_t sel = cb ? 0x07060302u : 0x05040100u;
          const u32x4 f = {__builtin_amdgcn_perm(Vb[2 * s][1], Vb[2 * s][0], sel),
                           __builtin_amdgcn_perm(Vb[2 * s][3], Vb[2 * s][2], sel),
                           __builtin_amdgcn_perm(Vb[2 * s + 1][1], Vb[2 * s + 1][0], sel),
                           __builtin_amdgcn_perm(Vb[2 * s + 1][3], Vb[2 * s + 1][2], sel)};
          XVf[s][cb] = __builtin_bit_cast(F, f);
        }
      f32x4 U[NB][2];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 u = zero4;
#pragma unroll
          for (int s = 0; 2 * s <= tb; ++s) u = MM::mma(TPf[tb][s], XVf[s][cb], u);
          U[tb][cb] = u;
        }

      // Y = K M (K read one row block ahead of its use).
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
            for (int s = 0; s < NKS; ++s) y = MM::mma(Kf[tb & 1][s], Mf[s][cb], y);
            Y[tb][cb] = y;
          }
        }
      }
      // Z = -diag(Gam) Y, then U = u + T diag(beta) Z.
      F Zf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 4 * q4);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 32 * s + 16 + 4 * q4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 z0, z1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z0[e] = -(g0[e] * Y[2 * s][cb][e]);
            z1[e] = -(g1[e] * Y[2 * s + 1][cb][e]);
          }
          Zf[s][cb] = MM::from_acc(z0, z1);
        }
      }
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 u = U[tb][cb];
#pragma unroll
          for (int s = 0; 2 * s <= tb; ++s) u = MM::mma(TPf[tb][s], Zf[s][cb], u);
          U[tb][cb] = u;
        }
      if constexpr (SAVE) {
        // U, bf16 row-major: tokens 16 tb + 4 q4 + e, value columns 32 j + 2 n16 + {0, 1}
        const int u_lane = (4 * q4 * DV + 32 * j + 2 * n16) * 2;
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, bf16x2{(__bf16)U[tb][0][e], (__bf16)U[tb][1][e]}), rrec, u_lane,
                (int)gdn_launch::BWD_OFF_U + (16 * tb + e) * DV * 2, 0);
      }
      F Uf[NTS][2], Wf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(vec + F_W * C + 32 * s + 4 * q4);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(vec + F_W * C + 32 * s + 16 + 4 * q4);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          Uf[s][cb] = MM::from_acc(U[2 * s][cb], U[2 * s + 1][cb]);
          f32x4 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = w0[e] * U[2 * s][cb][e];
            b[e] = w1[e] * U[2 * s + 1][cb][e];
          }
          Wf[s][cb] = MM::from_acc(a, b);
        }
      }
      // O^T = (M^T Q^T) diag(Gam), from the state before this chunk's
      // update: lane (token 16 tb + n16, q4) holds value columns
      // 32 j + 2 (4 q4 + e) + cb.
      f32x4 O[NB][2];
      if constexpr (!NOOUT) {
        F Qf[2][NKS];
        auto read_q = [&](int tb) {
#pragma unroll
          for (int s = 0; s < NKS; ++s) Qf[tb & 1][s] = lds_at<F>(sq + kq_frag[s] + 16 * KQR * tb);
        };
        read_q(0);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          if (tb + 1 < NB) read_q(tb + 1);
          const float gt = vec[F_GAM * C + 16 * tb + n16];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            f32x4 o = zero4;
#pragma unroll
            for (int s = 0; s < NKS; ++s) o = MM::mma(Mf[s][cb], Qf[tb & 1][s], o);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] *= gt;
            O[tb][cb] = o;
          }
        }
      }
      // M <- Gam_C M + K^T diag(w) U, then the next chunk's bf16 state.
      const float gC = vec[F_GAM * C + C - 1];
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
          f32x4 m = Macc[kb][cb];
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] *= gC;
#pragma unroll
          for (int s = 0; s < NTS; ++s) m = MM::mma(KT[s], Wf[s][cb], m);
          Macc[kb][cb] = m;
        }
      }
      make_mf();
      if constexpr (!NOOUT) {
        // O^T += U^T P^T once the P waves have published P.
        flag_wait_lds(&sFLAG[0], c + 1);
        flag_wait_lds(&sFLAG[1], c + 1);
        const long row0 = rowbase + (long)c * C;
        // a segment's halo chunks are computed but not stored (zero-size descriptor)
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + (row0 * H + hh) * DV * 2,
                                                    c >= store_from ? (long)(len - c * C) * v_stride : 0);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
#pragma unroll
          for (int s = 0; 2 * s <= tb; ++s) {
            const F pf = lds_at<F>(sP + ((tb * NTS + s) * 64 + lane) * 16);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) O[tb][cb] = MM::mma(Uf[s][cb], pf, O[tb][cb]);
          }
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)O[tb][0][e], (__bf16)O[tb][1][e]});
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, o_lane, (int)(16 * tb * v_stride), 0);
        }
      }
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) Vb[tb][e] = Vn[tb][e];
    };

    // No branch around the loads of v: a load whose destination register
    // meets another value at a control-flow join would have to complete
    // there.  Steps 0 and 1 fill the pipeline, step c + 2 works chunk c.
    if (NIT > 0) {
      lds_barrier();
      load_v(0, Vb);
      // Four stores that write nothing (empty descriptor), so that here, as
      // at the end of every chunk, the loads of v are followed by four
      // stores: the waits placed for v before its first use then count the
      // same operations on both ways in, and never wait for the stores.
      // (The maps and states passes store nothing here in their chunks.)
      if constexpr (!NOOUT) {
        const __amdgpu_buffer_rsrc_t none = make_rsrc(p.out, 0);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, none, o_lane, (int)(16 * tb * v_stride), 0);
      }
      lds_barrier();
      for (int c = 0; c < NC; ++c) {
        process(c);
        lds_barrier();
      }
    }
    // The final state: hT at the sequence end, or this segment's P or Q.
    float* const dst = MAPS ? wsm + (map_p ? 0 : DK * DV) : (write_hT ? p.hT + sbase : nullptr);
    if (dst) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x2*>(dst + (long)key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16) =
              f32x2{Macc[kb][0][e], Macc[kb][1][e]};
    }
  } else if (wave == W_L) {
    // ========================================================== loader wave
    // Copy i of a chunk writes LDS bytes [1024 i, 1024 i + 1024): lane l
    // fills granule l % GR of row i*RPI + l/GR with the logical granule
    // (l % GR) ^ swz(row).
    int kq_src[KQ_INS];
#pragma unroll
    for (int i = 0; i < KQ_INS; ++i) {
      const int r = i * KQ_RPI + lane / GR;
      kq_src[i] = (int)(r * kq_stride) + 16 * ((lane % GR) ^ swz_kq<GR>(r));
    }
    // g and beta: lane t copies token t of the chunk into sGB.
    const int gb_src = lane * H * 4;
    // Every copy below is issued unconditionally: a chunk past the end gets
    // empty descriptors (nothing is read, and the ring slots they fill hold
    // no live chunk), so each step issues the same number of memory
    // operations and one counted wait per step leaves exactly that step's
    // operations in flight.  Nothing is loaded into registers: a register
    // load carried from one step to the next would be made to complete at
    // the loop's control-flow joins.
    auto issue_gb = [&](int c) {
      const long row0 = rowbase + (long)c * C;
      const long left = c < NC ? (long)(len - c * C) : 0;
      char* d = reinterpret_cast<char*>(sGB + (c & 1) * 2 * C);
      copy_to_lds4(make_rsrc(p.g + row0 * H + hh, left * H * 4), d, gb_src);
      copy_to_lds4(make_rsrc(p.beta + row0 * H + hh, left * H * 4), d + C * 4, gb_src);
    };
    // q of a halo chunk is not needed (its outputs are not stored): empty.
    auto issue = [&](const char* base, char* ring, int nring, int c, bool need) {
      const long row0 = rowbase + (long)c * C;
      const long left = c < NC && need ? (long)(len - c * C) : 0;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(base + row0 * kq_stride + hh * KQR, left * kq_stride);
      char* d = ring + (c % nring) * KQ_BYTES;
#pragma unroll
      for (int i = 0; i < KQ_INS; ++i) copy_to_lds(r, d + i * 1024, kq_src[i]);
    };
    auto make_vec = [&](int c, float sg, float sb) {
      float* vec = vec_of(c);
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
    // Wait until at most the current step's loads and copies are in flight
    // and this wave's LDS stores are done, then join the barrier.  (A plain
    // LDS fence here would also wait for the copies just issued.)
    constexpr int NOPS = 2 * KQ_INS + 2;
    static_assert(NOPS < 64, "vmcnt range");
    constexpr int WAIT_NOPS = (NOPS & 15) | ((NOPS >> 4) << 14) | (7 << 4);  // vmcnt(NOPS) lgkmcnt(0)
    auto step_barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(WAIT_NOPS);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    if (NIT > 0 && cs != cs_guess) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the early copies have landed
      issue_gb(0);
      issue(p.k, sK, NKR, 0, true);
    }
    // Step it: the vectors of chunk it (its g and beta were copied one
    // step earlier, first among that step's operations), g and beta of
    // chunk it+1, k of chunk it+1, q of chunk it.
    for (int it = 0; it < NIT; ++it) {
      if (it == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(KQ_INS));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * KQ_INS));
      asm volatile("" ::: "memory");
      if (it < NC) {
        const float* gb = sGB + (it & 1) * 2 * C;
        make_vec(it, gb[lane], gb[C + lane]);
      }
      issue_gb(it + 1);
      issue(p.k, sK, NKR, it + 1, true);
      issue(p.q, sQ, NQR, it, !NOOUT && it >= store_from);
      step_barrier();
    }
    // The last steps' copies (of chunks past the end) still write LDS: let
    // them land before this wave ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (wave == W_G) {
    // ============================================================ Gram wave
    // A block result of mma(K rows b2, K rows b1): lane (n16, q4) holds row
    // i = 16 b1 + n16 and columns j = 16 b2 + 4 q4 + e.
    // Diagonal-block inverse: lane (block q4, column n16) writes row n16 of
    // Tbb^T (= column n16 of Tbb): four 4-wide pieces.
    int t_dst[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * q4 + n16;
      t_dst[m] = r * CCR + 16 * ((4 * (q4 >> 1) + m) ^ swz_cc<C>(r)) + 8 * (q4 & 1);
    }
    // Tbb as an MFMA row operand (transposing read of Tbb^T): rows
    // 16 b + 4 q4 + (src >> 2), columns 16 b + 4 (src & 3) .. +3.
    int t_base[NTS];
#pragma unroll
    for (int bh = 0; bh < NTS; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      t_base[bh] = r * CCR + 16 * ((4 * bh + (src & 3)) ^ swz_cc<C>(r));
    }
    // T^T store: row j = 16 col + n16, columns 16 b + 4 q4 .. +3.
    auto tp_off = [&](int b, int col) {
      const int jj = 16 * col + n16;
      return jj * CCR + 16 * ((2 * b + (q4 >> 1)) ^ swz_cc<C>(jj)) + 8 * (q4 & 1);
    };
    auto cat = [](bf16x4 lo, bf16x4 hi) { return F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; };

    auto gram_solve = [&](int c) {
      const char* sk = sK + (c % NKR) * KQ_BYTES;
      const float* vec = vec_of(c);
      F Kf[NB][NKS];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < NKS; ++s) Kf[b][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b);
      // Diagonal blocks of A (fp32, strictly lower).
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float li = vec[F_LAM * C + 16 * b + n16];
        const float bi0 = vec[F_BETA * C + 16 * b + n16];
        const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + F_LAM * C + 16 * b + 4 * q4);
        f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s) kk = MM::mma(Kf[b][s], Kf[b][s], kk);
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = 4 * q4 + e < n16 ? bi0 * kk[e] * exp2_fast(li - lj[e]) : 0.f;
        *reinterpret_cast<f32x4*>(sAD + b * AD_BLK + n16 * AD_ROW + 4 * q4) = r;
      }
      // Off-diagonal blocks (bf16), decay through the row block's first token.
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
      // Inverse of each 16x16 diagonal block of (I + A): lane (block q4,
      // column n16) runs forward substitution down the block.
      {
        const float* A = sAD + q4 * AD_BLK;
        // Row i holds columns 0..i-1: whole 4-wide pieces, then a 2- and/or
        // 1-wide piece, so every value read is used.
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
        // Right-looking order: once entry l is final it is folded into every
        // later row (each row still accumulates its terms in increasing l).
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
      // T by block forward substitution: column block col of row block b is
      // R_b = Tbb (X_b - sum_{j<b} A_bj R_j) with X = I; each result block
      // is rounded to bf16 once and reused by every later row block.
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
            f32x4 r = zero4, r16 = zero4;  // full- and half-depth apart (see mma16)
#pragma unroll
            for (int s = 0; 32 * s < 16 * b; ++s) {
              if (2 * s + 1 < col) continue;  // both blocks of the slab are zero
              if (2 * s + 1 >= b) r16 = MM::mma16(MM::lo(Af[b][s]), RH[2 * s][col], r16);
              else if (2 * s < col) r16 = MM::mma16(MM::hi(Af[b][s]), RH[2 * s + 1][col], r16);
              else r = MM::mma(Af[b][s], cat(RH[2 * s][col], RH[2 * s + 1][col]), r);
            }
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = -(r[e] + r16[e]);
            xh = cvt4(x);
          }
          RT[b][col] = MM::mma16(Tf[b], xh, zero4);
          RH[b][col] = cvt4(RT[b][col]);
        }
      }
      // Published as T diag(beta): row j = 16 col + n16 of the transposed
      // tile is column j of T, scaled by beta_j.
      char* tp = sT + (c & 1) * CC_BYTES;
#pragma unroll
      for (int col = 0; col < NB; ++col) {
        const float bj = vec[F_BETA * C + 16 * col + n16];
#pragma unroll
        for (int b = col; b < NB; ++b) {
          f32x4 t;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = RT[b][col][e] * bj;
          lds_st<bf16x4>(tp, tp_off(b, col), cvt4(t));
        }
      }
    };
    for (int it = 0; it < NIT; ++it) {
      const int c = it - 1;
      if (c >= 0 && c < NC) gram_solve(c);
      lds_barrier();
    }
  } else {
    // ============================================================= P waves
    auto p_wave = [&](auto oc) {
      constexpr int o = decltype(oc)::value;
      auto make_p = [&](int c) {
        const char* sk = sK + (c % NKR) * KQ_BYTES;
        const char* sq = sQ + (c % NQR) * KQ_BYTES;
        const float* vec = vec_of(c);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int b1 = own_tb(o, i);
          F Qf[NKS];
#pragma unroll
          for (int s = 0; s < NKS; ++s) Qf[s] = lds_at<F>(sq + kq_frag[s] + 16 * KQR * b1);
          const float li = vec[F_LAM * C + 16 * b1 + n16];
          const float eri = vec[F_ER * C + 16 * b1 + n16];
          // Block (b1, b2): lane (n16, q4) holds row i = 16 b1 + n16 and
          // columns j = 16 b2 + 4 q4 + e, the pi-order operand of U^T P^T.
          f32x4 pb[NB];
#pragma unroll
          for (int b2 = 0; b2 <= b1; ++b2) {
            F Kf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) Kf[s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b2);
            f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) pq = MM::mma(Kf[s], Qf[s], pq);
            if (b2 < b1) {
              const f32x4 ec = *reinterpret_cast<const f32x4*>(vec + (F_ER + b1) * C + 16 * b2 + 4 * q4);
#pragma unroll
              for (int e = 0; e < 4; ++e) pb[b2][e] = pq[e] * (eri * ec[e]);
            } else {
              const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + F_LAM * C + 16 * b1 + 4 * q4);
#pragma unroll
              for (int e = 0; e < 4; ++e) pb[b2][e] = 4 * q4 + e <= n16 ? pq[e] * exp2_fast(li - lj[e]) : 0.f;
            }
          }
#pragma unroll
          for (int s = 0; 2 * s <= b1; ++s) {
            const F pf = 2 * s + 1 <= b1 ? MM::from_acc(pb[2 * s], pb[2 * s + 1]) : MM::from_acc1(pb[2 * s]);
            lds_st<F>(sP, ((b1 * NTS + s) * 64 + lane) * 16, pf);
          }
        }
        flag_release(&sFLAG[o], c + 1);
      };
      for (int it = 0; it < NIT; ++it) {
        const int c = it - 2;
        if (c >= 0) make_p(c);
        lds_barrier();
      }
    };
    if constexpr (NOOUT) {
      for (int it = 0; it < NIT; ++it) lds_barrier();  // no outputs: nothing to form
    } else if (wave == W_P) {
      p_wave(IC<0>{});
    } else {
      p_wave(IC<1>{});
    }
  }
}

// ------------------------------------------------------------ the scan
// Exact entry states of a cut sequence's segments.  Over a segment the rule
// is affine in the state, M_end = P M_start + Q, and the maps pass above
// leaves P (for segments 1 .. nseg-2) and Q (segments 0 .. nseg-2, the first
// one from h0) in the workspace.  Here S_0 = h0, S_1 = Q_0 and
// S_{s+1} = P_s S_s + Q_s, in fp32 on the matrix cores: the chunk-to-chunk
// series of the chunked form ("Optimization Quartet", section 3.2) shrinks
// to one dk x dk by dk x dv product per segment.  One workgroup per
// (sequence, head, 16-column block); wave w owns state rows 16 w .. 16 w + 15.
namespace sk {
constexpr int NCB = fk::DV / 16;  // column blocks (workgroups per chain)
constexpr int NWS = fk::DK / 16;  // waves, one per 16-row block
constexpr int LD = fk::DK + 4;    // LDS pitch (floats) of a column of the state block
}  // namespace sk

__global__ __launch_bounds__(64 * sk::NWS, 1) void gdn_scan_kernel(const gdn_launch::FullParams p) {
  using namespace fk;
  // S_s of this column block, transposed (column-major), two steps.
  __shared__ __attribute__((aligned(16))) float sS[2][16 * sk::LD];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4, n16 = lane & 15;
  const int H = p.H;
  const int item = xcd_remap(blockIdx.x, p.B * H * sk::NCB);
  const int cb = item % sk::NCB, chain = item / sk::NCB;
  const int hh = chain % H, n = chain / H;
  int len = p.T, s0 = 0;
  if (p.cu) {
    s0 = p.cu[n];
    len = p.cu[n + 1] - s0;
  }
  int nch, seg_len, nseg;
  seg_layout(len, p.seg_max, p.seg_cap, nch, seg_len, nseg);
  if (nseg <= 1) return;  // uniform over the workgroup
  // First segment slot of the sequence (the same numbering as the kernel above).
  const long slot0 = p.cu ? (long)(s0 / (p.seg_max * C)) + n : (long)n * nseg;
  auto mat = [&](int s, int which) {  // which: 0 P, 1 Q, 2 S
    return p.ws + (((slot0 + s) * H + hh) * 3 + which) * (long)(DK * DV);
  };
  // Result lane layout (16x16 fp32 accumulator): rows 16 w + 4 q4 + r,
  // column 16 cb + n16.
  const int col = 16 * cb + n16;
  const int row = 16 * w + 4 * q4;
  auto put = [&](int s, f32x4 d) {
    float* S = mat(s, 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[(long)(row + r) * DV + col] = d[r];
    *reinterpret_cast<f32x4*>(&sS[s & 1][n16 * sk::LD + row]) = d;
  };
  {
    f32x4 h = {0.f, 0.f, 0.f, 0.f};
    if (p.h0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = p.h0[((long)chain * DK + row + r) * DV + col];
    }
    put(0, h);
    const float* Q0 = mat(0, 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = Q0[(long)(row + r) * DV + col];
    put(1, h);
  }
  // A operand of step (a, t): P[16 w + n16][16 a + 4 q4 + t]; B operand:
  // S[16 a + 4 q4 + t][col], one 16-byte LDS read per a.  The maps of
  // segment s + 1 are loaded during step s (empty descriptors past the last).
  f32x4 Pc[8], Qc, Pn[8], Qn;
  auto load = [&](int s, f32x4 (&Pd)[8], f32x4& Qd) {
    const bool live = s + 1 < nseg;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(mat(live ? s : 1, 0), live ? (long)DK * DV * 4 : 0);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(mat(live ? s : 1, 1), live ? (long)DK * DV * 4 : 0);
#pragma unroll
    for (int a = 0; a < 8; ++a)
      Pd[a] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rp, ((16 * w + n16) * DV + 16 * a + 4 * q4) * 4, 0, 0));
#pragma unroll
    for (int r = 0; r < 4; ++r)
      Qd[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, ((row + r) * DV + col) * 4, 0, 0));
  };
  load(1, Pc, Qc);
  for (int s = 1; s + 1 < nseg; ++s) {
    load(s + 1, Pn, Qn);
    __syncthreads();  // S_s complete in sS[s & 1]; sS[(s + 1) & 1] no longer read
    const float* Sb = sS[s & 1] + n16 * sk::LD + 4 * q4;
    f32x4 d = Qc;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(Sb + 16 * a);
#pragma unroll
      for (int t = 0; t < 4; ++t) d = __builtin_amdgcn_mfma_f32_16x16x4f32(Pc[a][t], b[t], d, 0, 0, 0);
    }
    put(s + 1, d);
#pragma unroll
    for (int a = 0; a < 8; ++a) Pc[a] = Pn[a];
    Qc = Qn;
  }
}

}  // namespace

namespace gdn_launch {

int full_slots(int B, int T, bool packed, int seg_max, int seg_cap) {
  if (!packed) {
    int nch, seg_len, nseg;
    fk::seg_layout(T, seg_max, seg_cap, nch, seg_len, nseg);
    return B * nseg;
  }
  // sequence n takes slots [floor(start_n / (seg_max * 64)) + n, + its
  // segments), never more than ceil(length_n / (seg_max * 64)) of them
  return (seg_max > 0 ? T / (seg_max * 64) : 0) + B;
}

int seg_cap_for(int H) {
  int dev = 0, ncu = 0;
  if (H < 1 || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    return 0;
  return ncu / H > 1 ? ncu / H : 1;
}

int fwd_full(const FullParams& p, hipStream_t stream) {
  const long nwg = (long)p.nslot * p.H;
  if (nwg <= 0) return GDN_OK;
  if (nwg > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn_full_kernel<0>, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int fwd_full_train(const FullParams& p, hipStream_t stream) {
  const long nwg = (long)p.nslot * p.H;
  if (nwg <= 0) return GDN_OK;
  if (nwg > 0x7fffffffL || !p.sv) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn_full_kernel<3>, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int fwd_full_save(const FullParams& p, hipStream_t stream) {
  const long nwg = (long)p.nslot * p.H;
  if (nwg <= 0) return GDN_OK;
  if (nwg > 0x7fffffffL || !p.sv) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn_full_kernel<2>, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

long long scan_ws_floats(int nslot, int H) { return (long long)nslot * H * 3 * fk::DK * fk::DV; }

int fwd_full_scan(const FullParams& p, hipStream_t stream) {
  const long nwg = (long)p.nslot * p.H;
  if (nwg <= 0) return GDN_OK;
  const long nscan = (long)p.B * p.H * sk::NCB;
  if (!p.ws || 2 * nwg > 0x7fffffffL || nscan > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  // Only a sequence of more than seg_max chunks is cut.
  const long seg_tokens = (long)p.seg_max * fk::C;
  const bool cut = p.seg_max > 0 && p.T > seg_tokens;
  if (cut) {
    hipLaunchKernelGGL(gdn_full_kernel<1>, dim3((unsigned)(2 * nwg)), dim3(64 * fk::NW), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
    hipLaunchKernelGGL(gdn_scan_kernel, dim3((unsigned)nscan), dim3(64 * sk::NWS), 0, stream, p);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(gdn_full_kernel<0>, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn_launch
