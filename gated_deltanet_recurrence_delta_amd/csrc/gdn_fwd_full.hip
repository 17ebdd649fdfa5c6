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
// (one 16-byte store per token row).  State rows use the key order of the
// bf16 kernel in gdn_fwd.hip (key_of below), which makes the transposing
// reads of K conflict-free and the state's bf16 fragments natural-order.
//
// No atomics: results are deterministic and bitwise independent of the
// workgroup schedule.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_launch.h"

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
                    NVEC * NF * C * 4 + NB * AD_BLK * 4 + 64;
static_assert(LDS <= 160 * 1024, "LDS budget");
static_assert(NB == 4 && NKS == 4 && NCW == 4, "shape");

// P wave o owns the 16-row blocks {o, 3 - o} (equal MFMA work).
__host__ __device__ constexpr int own_tb(int o, int i) { return i == 0 ? o : NB - 1 - o; }

// State row (key) held by accumulator block b, row r: of the 32 keys of
// slab b >> 1, block b takes from each 8-key group the half (b ^ g) & 1.
__device__ static inline int key_of(int b, int r) {
  return 32 * (b >> 1) + 8 * (r >> 2) + 4 * ((b ^ (r >> 2)) & 1) + (r & 3);
}

// Chunk count of a sequence and its segment layout.
__device__ static inline void seg_layout(int len, int seg_max, int& nch, int& seg_len, int& nseg) {
  nch = (len + C - 1) / C;
  if (seg_max <= 0 || nch <= seg_max) {
    seg_len = nch > 0 ? nch : 1;
    nseg = 1;
    return;
  }
  const int n0 = (nch + seg_max - 1) / seg_max;
  seg_len = (nch + n0 - 1) / n0;
  nseg = (nch + seg_len - 1) / seg_len;
}

}  // namespace fk

__global__ __launch_bounds__(64 * fk::NW, 1) void gdn_full_kernel(const gdn_launch::FullParams p) {
  using namespace fk;
  using MM = Mma<__bf16>;
  using F = bf16x8;
  constexpr float kLog2e = 1.4426950408889634f;

  __shared__ __attribute__((aligned(16))) char sK[NKR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sQ[NQR * KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sAT[CC_BYTES];     // A (off-diagonal) and T_bb^T
  __shared__ __attribute__((aligned(16))) char sT[2 * CC_BYTES];  // T^T of two chunks
  __shared__ __attribute__((aligned(16))) char sP[CC_BYTES];      // P, lane-major fragments
  __shared__ __attribute__((aligned(16))) float sVEC[NVEC * NF * C];
  __shared__ __attribute__((aligned(16))) float sAD[NB * AD_BLK];
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
  const int slot = blockIdx.x / H, hh = blockIdx.x % H;
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
      seg_layout(s1 - s0, p.seg_max, nch, seg_len, nseg);
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
    seg_layout(p.T, p.seg_max, nch, seg_len, nseg);
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

  // Segment range [c0, c1) of chunks whose outputs this workgroup stores,
  // and where its recurrence starts (cs <= c0).
  int nch, seg_len, nseg;
  seg_layout(len, p.seg_max, nch, seg_len, nseg);
  const int c0 = seg * seg_len;
  const int c1 = min(c0 + seg_len, nch);
  if (threadIdx.x < 4) sFLAG[threadIdx.x] = 0;
  if (wave == 0) {
    int cs = c0;
    float acc = 0.f;  // log of the transition-norm product over chunks [cs, c0)
    while (cs > 0 && acc > -HALO_NATS) {
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
  __syncthreads();
  const int cs = sSTART;
  const bool use_h0 = cs == 0;
  const bool write_hT = c1 >= nch;
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
    // 8-byte piece holding keys 32 (b>>1) + 8 (src&3) + 4 ((b^src)&1) .. +3.
    int kt_base[NKB / 2];
#pragma unroll
    for (int bh = 0; bh < NKB / 2; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      kt_base[bh] = r * KQR + 16 * ((4 * bh + (src & 3)) ^ swz_kq<GR>(r)) + 8 * (src & 1);
    }
    const int kt_flip = 8 - 16 * (src & 1);  // to the other half (odd blocks)
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
    // [32 j + 2 n16 + cb].
    f32x4 Macc[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f32x2 h = {0.f, 0.f};
        if (p.h0 && use_h0)
          h = *reinterpret_cast<const f32x2*>(p.h0 + sbase + (long)key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16);
        Macc[kb][0][e] = h[0];
        Macc[kb][1][e] = h[1];
      }
    F Mf[NKS][2];
    const bool odd = q4 & 1;
    auto make_mf = [&]() {
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const u32x4 u = __builtin_bit_cast(u32x4, MM::from_acc(Macc[2 * s][cb], Macc[2 * s + 1][cb]));
          Mf[s][cb] = __builtin_bit_cast(F, u32x4{odd ? u[2] : u[0], odd ? u[3] : u[1], odd ? u[0] : u[2], odd ? u[1] : u[3]});
        }
    };
    make_mf();

    auto load_v = [&](int c, uint32_t (&Vn)[NB][4]) {
      const long row0 = rowbase + (long)c * C;
      const __amdgpu_buffer_rsrc_t rv =
          make_rsrc(p.v + (row0 * H + hh) * DV * 2, c < NC ? (long)(len - c * C) * v_stride : 0);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Vn[tb][e] = __builtin_amdgcn_raw_buffer_load_b32(rv, v_lane, (int)((16 * tb + e) * v_stride), 0);
    };

    // v of chunk c sits in Vb from the middle of step c+1 (right after the
    // previous chunk's X consumed it) to its own X at step c+2.
    uint32_t Vb[NB][4];
    auto process = [&](int c) {
      const char* sk = sK + (c % NKR) * KQ_BYTES;
      const char* sq = sQ + (c % NQR) * KQ_BYTES;
      const char* st = sT + (c & 1) * CC_BYTES;
      const float* vec = vec_of(c);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

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
      // O^T = (M^T Q^T) diag(Gam): lane (token 16 tb + n16, q4) holds value
      // columns 32 j + 2 (4 q4 + e) + cb.
      f32x4 O[NB][2];
      {
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
      // X = diag(beta) (V - diag(Gam) Y), in place of Y.
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(vec + F_BETA * C + 16 * tb + 4 * q4);
        const f32x4 gm = *reinterpret_cast<const f32x4*>(vec + F_GAM * C + 16 * tb + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = __uint_as_float(Vb[tb][e] << 16), v1 = __uint_as_float(Vb[tb][e] & 0xffff0000u);
          Y[tb][0][e] = bt[e] * (v0 - gm[e] * Y[tb][0][e]);
          Y[tb][1][e] = bt[e] * (v1 - gm[e] * Y[tb][1][e]);
        }
      }
      if (c + 1 < NC) load_v(c + 1, Vb);
      F Xf[NTS][2];
#pragma unroll
      for (int s = 0; s < NTS; ++s)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) Xf[s][cb] = MM::from_acc(Y[2 * s][cb], Y[2 * s + 1][cb]);
      // U = T X (full- and half-depth products accumulate apart, see mma16).
      f32x4 U[NB][2];
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          f32x4 u = zero4, h = zero4;
#pragma unroll
          for (int s = 0; 2 * s <= tb; ++s) {
            if (2 * s + 1 <= tb) u = MM::mma(TPf[tb][s], Xf[s][cb], u);
            else h = MM::mma16(MM::lo(TPf[tb][s]), MM::lo(Xf[s][cb]), h);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] += h[e];
          U[tb][cb] = u;
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
      // M <- Gam_C M + K^T diag(w) U
      const float gC = vec[F_GAM * C + C - 1];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        F KT[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
          const char* p0 = sk + kt_base[kb >> 1] + ((kb & 1) ? kt_flip : 0) + 32 * s * KQR;
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
      // O^T += U^T P^T once the P waves have published P.
      flag_wait_lds(&sFLAG[0], c + 1);
      flag_wait_lds(&sFLAG[1], c + 1);
      const long row0 = rowbase + (long)c * C;
      // a segment's halo chunks are computed but not stored (zero-size descriptor)
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + (row0 * H + hh) * DV * 2,
                                                  c >= store_from ? (long)(len - c * C) * v_stride : 0);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        f32x4 h[2] = {zero4, zero4};
#pragma unroll
        for (int s = 0; 2 * s <= tb; ++s) {
          const F pf = lds_at<F>(sP + ((tb * NTS + s) * 64 + lane) * 16);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            if (2 * s + 1 <= tb) O[tb][cb] = MM::mma(Uf[s][cb], pf, O[tb][cb]);
            else h[cb] = MM::mma16(MM::lo(Uf[s][cb]), MM::lo(pf), h[cb]);
          }
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 a = (__bf16)(O[tb][0][e] + h[0][e]);
          const __bf16 b = (__bf16)(O[tb][1][e] + h[1][e]);
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
        }
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, o_lane, (int)(16 * tb * v_stride), 0);
      }
      make_mf();
    };

    for (int it = 0; it < NIT; ++it) {
      if (it == 1) load_v(0, Vb);
      if (it >= 2) process(it - 2);
      lds_barrier();
    }
    if (write_hT) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x2*>(p.hT + sbase + (long)key_of(kb, 4 * q4 + e) * DV + 32 * j + 2 * n16) =
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
    // g and beta: lane t reads token t of the chunk.
    const int gb_src = lane * H * 4;
    // Every load and copy below is issued unconditionally: a chunk past the
    // end gets empty descriptors (its loads read zeros and its copies fill
    // ring slots no live chunk occupies), so each step issues the same
    // number of memory operations and one counted wait per step leaves
    // exactly that step's operations in flight.
    auto load_gb = [&](int c, float& sg, float& sb) {
      const long row0 = rowbase + (long)c * C;
      const long left = c < NC ? (long)(len - c * C) : 0;
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + row0 * H + hh, left * H * 4);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.beta + row0 * H + hh, left * H * 4);
      sg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, gb_src, 0, 0));
      sb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, gb_src, 0, 0));
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
    float g0 = 0.f, b0 = 0.f, g1 = 0.f, b1 = 0.f;
    if (NIT > 0) {
      load_gb(0, g0, b0);
      issue(p.k, sK, NKR, 0, true);
    }
    // Step it: vectors of chunk it (from the g and beta loaded one step
    // earlier), g and beta of chunk it+1, k of chunk it+1, q of chunk it.
    auto step = [&](int it, float& gu, float& bu, float& gl, float& bl) {
      if (it < NC) make_vec(it, gu, bu);
      load_gb(it + 1, gl, bl);
      issue(p.k, sK, NKR, it + 1, true);
      issue(p.q, sQ, NQR, it, it >= store_from);
      step_barrier();
    };
    for (int it = 0; it < NIT; it += 2) {
      step(it, g0, b0, g1, b1);
      if (it + 1 < NIT) step(it + 1, g1, b1, g0, b0);
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
      char* tp = sT + (c & 1) * CC_BYTES;
#pragma unroll
      for (int col = 0; col < NB; ++col)
#pragma unroll
        for (int b = col; b < NB; ++b) lds_st<bf16x4>(tp, tp_off(b, col), RH[b][col]);
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
    if (wave == W_P) p_wave(IC<0>{});
    else p_wave(IC<1>{});
  }
}

}  // namespace

namespace gdn_launch {

int full_slots(int B, int T, bool packed, int seg_max) {
  if (!packed) {
    const int nch = (T + 63) / 64;
    int nseg = 1;
    if (seg_max > 0 && nch > seg_max) {
      const int n0 = (nch + seg_max - 1) / seg_max;
      const int seg_len = (nch + n0 - 1) / n0;
      nseg = (nch + seg_len - 1) / seg_len;
    }
    return B * nseg;
  }
  return (seg_max > 0 ? T / (seg_max * 64) : 0) + B;
}

int fwd_full(const FullParams& p, hipStream_t stream) {
  const long nwg = (long)p.nslot * p.H;
  if (nwg <= 0) return GDN_OK;
  if (nwg > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gdn_full_kernel, dim3((unsigned)nwg), dim3(64 * fk::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn_launch
