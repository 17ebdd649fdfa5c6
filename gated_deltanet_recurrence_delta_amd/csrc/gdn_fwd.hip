// Gated-delta-rule forward pass for AMD MI355X (gfx950 / CDNA4).
//
// Rule, per head and sequence (HyMo "Model Architecture Walkthrough",
// sections 5.2.1-5.2.2: the delta rule with rate beta_t, target v_t, write
// key k_t, prediction alpha_t S_{t-1} k_t, after the per-head decay
// alpha_t = exp(g_t); the read uses the updated state):
//
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t q_t.
//
// Chunkwise-parallel evaluation.  The pages' kernel cuts the sequence into
// chunks (64 by default), works inside a chunk in parallel and carries the
// state across chunks in series ("v1.0 Architecture & Design Spec",
// section 2.3; "Optimization Quartet", section 3.2).  With M = S^T
// (dk x dv, the h0/hT layout), a chunk of C tokens, gamma = in-chunk cumsum
// of g, Gam = exp(gamma), w = exp(gamma_C - gamma):
//
//     A    = strictly-lower( diag(beta) (K K^T) * exp(gamma_i - gamma_j) )
//     Tinv = (I + A)^{-1}                          (unit lower triangular)
//     X    = diag(beta) (V - diag(Gam) K M)
//     U    = Tinv X                                (corrected writes)
//     O    = diag(Gam) Q M + ((Q K^T) * exp(gamma_i - gamma_j), j <= i) U
//     M   <- Gam_C M + K^T diag(w) U
//
// This file holds the C entry points (gdn_fwd, gdn_fwd_scan, gdn_strerror,
// gdn_version) and the per-tile kernels.  Which kernel runs:
//   * bf16 storage, dk = dv = 128, 64-token chunks: the full-width kernel of
//     gdn_fwd_full.hip, one workgroup per (sequence segment, head) owning
//     all value columns (also the three launches of gdn_fwd_scan);
//   * other bf16 shapes: gdn_bf16_kernel below, one workgroup per (chain,
//     32-column value tile), eight wave roles (loader, Gram, two solve, two
//     state, two output) in a three-step software pipeline;
//   * fp32 storage: gdn_fwd_kernel below, one workgroup per (chain,
//     32-column value tile), a three-stage pipeline (Gram wave, solve wave,
//     value waves holding the tile's state in MFMA accumulators).
// Value columns never mix in the rule, so tiles are independent; each tile
// recomputes its chunk's Gram matrix and solve.  No atomics: results are
// deterministic.
//
// Operand conventions: a 16x16xSLAB MFMA "fragment" gives every lane
// (l % 16 = row/column index, q = l / 16 = lane group) E consecutive
// contraction positions [E*q, E*q+E).  The 16x16 fp32 accumulator layout
// gives lane (n = l % 16, q) rows 4q..4q+3 of column n; two vertically
// stacked accumulators therefore form a fragment whose positions map to
// rows {4q..4q+3} and {16+4q..16+4q+3} ("pi" order).  Row-major LDS
// operands that meet such a fragment are read in the same pi order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace {


// ------------------------------------------------------------ LDS tiles

// Row-major tile of COLS elements of T per row, 16-byte granules XOR-
// swizzled by row so that 16 lanes reading the same logical granule of 16
// consecutive rows hit 16 distinct bank groups.
template <typename T, int COLS>
struct Swz {
  static constexpr int RB = COLS * (int)sizeof(T);
  static constexpr int GR = RB / 16;
  static_assert(RB % 16 == 0 && GR >= 2, "row must hold >= 2 granules");
  __device__ static inline int h(int r) { return GR >= 16 ? (r & 15) : ((r * GR / 16) % GR); }
  __device__ static inline int off(int r, int c) {
    const int byte = c * (int)sizeof(T);
    return r * RB + ((((byte >> 4) ^ h(r))) << 4) + (byte & 15);
  }
  __device__ static inline int goff(int r, int granule) { return r * RB + ((granule ^ h(r)) << 4); }
};


// Fragment with natural positions from a row-major swizzled tile: row r,
// columns [c0 + E*q, c0 + E*q + E).  c0 is a multiple of SLAB.
template <typename TI, int COLS>
__device__ static inline typename Mma<TI>::frag frag_nat(const char* t, int r, int c0, int q) {
  using F = typename Mma<TI>::frag;
  return lds_ld<F>(t, Swz<TI, COLS>::off(r, c0 + Mma<TI>::E * q));
}

// Fragment in pi order from a row-major swizzled tile (row r, slab at c0).
template <typename TI, int COLS>
__device__ static inline typename Mma<TI>::frag frag_pi(const char* t, int r, int c0, int q) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x4 lo = lds_ld<bf16x4>(t, Swz<TI, COLS>::off(r, c0 + 4 * q));
    const bf16x4 hi = lds_ld<bf16x4>(t, Swz<TI, COLS>::off(r, c0 + 16 + 4 * q));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return lds_ld<f32x4>(t, Swz<TI, COLS>::off(r, c0 + 4 * q));
  }
}

// Pi-order fragment whose second half (positions 16..31) is zero: a 16-long
// contraction against a single accumulator block.
template <typename TI, int COLS>
__device__ static inline typename Mma<TI>::frag frag_pi1(const char* t, int r, int c0, int q) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x4 lo = lds_ld<bf16x4>(t, Swz<TI, COLS>::off(r, c0 + 4 * q));
    bf16x8 f{};
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    return f;
  } else {
    return lds_ld<f32x4>(t, Swz<TI, COLS>::off(r, c0 + 4 * q));
  }
}

// Store 4 consecutive elements (row r, columns c..c+3).
template <typename TI, int COLS>
__device__ static inline void st4(char* t, int r, int c, f32x4 v) {
  if constexpr (sizeof(TI) == 2) {
    lds_st<bf16x4>(t, Swz<TI, COLS>::off(r, c),
                   bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]});
  } else {
    lds_st<f32x4>(t, Swz<TI, COLS>::off(r, c), v);
  }
}

template <typename TI, int COLS>
__device__ static inline void st1(char* t, int r, int c, float v) {
  lds_st<TI>(t, Swz<TI, COLS>::off(r, c), (TI)v);
}

template <typename TI>
__device__ static inline float to_f(TI x) { return (float)x; }

// Fragment of contraction slab s from a column of stacked accumulators
// (two blocks per slab for bf16, one for fp32).
template <typename TI>
__device__ static inline typename Mma<TI>::frag acc_frag(const f32x4* a, int s) {
  if constexpr (Mma<TI>::SLAB == 32) {
    return Mma<TI>::from_acc(a[2 * s], a[2 * s + 1]);
  } else {
    return Mma<TI>::from_acc(a[s], a[s]);
  }
}


// ------------------------------------------------------------ configuration

template <typename TI, int DK, int DVT, int C>
struct Cfg {
  using MM = Mma<TI>;
  static constexpr int S = sizeof(TI);
  static constexpr int SLAB = MM::SLAB, E = MM::E, BPS = SLAB / 16;
  static constexpr int NB = C / 16;       // 16-token blocks per chunk
  static constexpr int NTS = C / SLAB;    // token slabs per chunk
  static constexpr int NKB = DK / 16;     // 16-row key blocks of the state
  static constexpr int NKS = DK / SLAB;   // key slabs
  static constexpr int NDV = DVT / 16;    // value waves
  static constexpr int W_S = NDV;         // solve wave
  static constexpr int W_G = NDV + 1;     // Gram / loader wave
  static constexpr int NW = NDV + 2;
  static constexpr int NT = 64 * NW;
  static_assert(C % SLAB == 0 && DK % SLAB == 0 && DVT % 16 == 0, "shape");
  static_assert(NB <= 4, "chunk of at most 64 tokens");

  static constexpr int KQ_BYTES = C * DK * S;
  static constexpr int V_BYTES = C * DVT * S;
  static constexpr int CC_BYTES = C * C * S;
  static constexpr int VEC_BYTES = 4 * C * 4;  // beta, gamma, exp(gamma), exp(gamma_C - gamma)
  static constexpr int AD_STRIDE = 260;        // floats per padded 16x16 fp32 block
  static constexpr int OFF_K = 0;                         // [3] K ring
  static constexpr int OFF_V = OFF_K + 3 * KQ_BYTES;      // [3] V ring (this tile's columns)
  static constexpr int OFF_A = OFF_V + 3 * V_BYTES;       // [2] A, off-diagonal blocks
  static constexpr int OFF_P = OFF_A + 2 * CC_BYTES;      // [3] masked decayed Q K^T
  static constexpr int OFF_T = OFF_P + 3 * CC_BYTES;      // [2] Tinv
  static constexpr int OFF_TT = OFF_T + 2 * CC_BYTES;     // [1] Tinv^T (solve wave only)
  static constexpr int OFF_VEC = OFF_TT + CC_BYTES;       // [3] per-token vectors
  static constexpr int OFF_AD = OFF_VEC + 3 * VEC_BYTES;  // [1] A diagonal blocks, fp32
  static constexpr int LDS = OFF_AD + NB * AD_STRIDE * 4;

  // Solve-wave staging of this tile's V: 16-byte granules per lane.
  static constexpr int GRV = DVT * S / 16;  // granules per v token row (this tile)
  static constexpr int NPV = (C * GRV + 63) / 64;
};

struct Params {
  const char* q;
  const char* k;
  const char* v;
  const float* g;
  const float* beta;
  const float* h0;
  const int32_t* cu;
  char* out;
  float* hT;
  int T, H, dv, ntile, nwg;
  int lpt;  // packed batch: longest sequences dispatched first (chunkwise bf16 kernel)
  // Dense batch with fewer chains than CUs (chunkwise bf16 kernel): each
  // chain's sequence is cut into nseg segments of seg_chunks chunks, one
  // workgroup per (chain, segment, value tile).
  int nseg, seg_chunks;
};


// Longest segment, in chunks, of the full-width kernel (gdn_fwd_full.hip):
// 16 chunks of 64 tokens cut a 4,096-token sequence into four workgroups.
constexpr int GDN_SEG_MAX_CHUNKS = gdn_launch::SEG_MAX_CHUNKS;

// Largest packed batch whose sequences the bf16 kernel orders by length.
constexpr int GDN_LPT_MAX = 512;


// Chunk c flows through three stages, one per loop iteration, with one
// LDS barrier between iterations:
//   iteration c   : Gram wave  -- stage K of chunk c into LDS, decay
//                   vectors, off-diagonal A blocks, P (its K and Q
//                   fragments were loaded two iterations earlier);
//                   solve wave -- stage this tile's V of chunk c into LDS;
//   iteration c+1 : solve wave -- diagonal A blocks, Tinv;
//   iteration c+2 : value waves -- the state-dependent products.
template <typename TI, int DK, int DVT, int C>
__global__ __launch_bounds__(64 * (DVT / 16 + 2), 1) void gdn_fwd_kernel(const Params p) {
  using CF = Cfg<TI, DK, DVT, C>;
  using MM = Mma<TI>;
  using F = typename MM::frag;
  using SK = Swz<TI, DK>;
  using SV = Swz<TI, DVT>;
  constexpr int SLAB = CF::SLAB, E = CF::E, BPS = CF::BPS;
  constexpr int NB = CF::NB, NTS = CF::NTS, NKB = CF::NKB, NKS = CF::NKS, NDV = CF::NDV;

  __shared__ __attribute__((aligned(16))) char smem[CF::LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4, n16 = lane & 15;

  const int item = xcd_remap(blockIdx.x, p.nwg);
  const int chain = item / p.ntile, tile = item % p.ntile;
  const int H = p.H;
  const int bseq = chain / H, hh = chain % H;
  long rowbase;
  int len;
  if (p.cu) {
    rowbase = p.cu[bseq];
    len = p.cu[bseq + 1] - p.cu[bseq];
  } else {
    rowbase = (long)bseq * p.T;
    len = p.T;
  }
  const int NC = (len + C - 1) / C;
  const int NIT = NC > 0 ? NC + 2 : 0;
  const long kq_stride = (long)H * DK * CF::S;  // bytes between tokens in q/k
  const long v_stride = (long)H * p.dv * CF::S;
  const char* qbase = p.q + hh * (long)DK * CF::S;
  const char* kbase = p.k + hh * (long)DK * CF::S;
  const char* vbase = p.v + ((long)hh * p.dv + tile * DVT) * CF::S;
  auto clamp_tok = [&](int t) { return t < len ? t : len - 1; };

  auto kbuf = [&](int c) { return smem + CF::OFF_K + (c % 3) * CF::KQ_BYTES; };
  auto vbuf = [&](int c) { return smem + CF::OFF_V + (c % 3) * CF::V_BYTES; };
  auto abuf = [&](int c) { return smem + CF::OFF_A + (c & 1) * CF::CC_BYTES; };
  auto pbuf = [&](int c) { return smem + CF::OFF_P + (c % 3) * CF::CC_BYTES; };
  auto tbuf = [&](int c) { return smem + CF::OFF_T + (c & 1) * CF::CC_BYTES; };
  auto vecb = [&](int c) { return reinterpret_cast<float*>(smem + CF::OFF_VEC + (c % 3) * CF::VEC_BYTES); };

  // Q or K fragments of chunk c straight from global memory: fragment
  // (tb, s) of lane (n16, q4) is row 16 tb + n16, key positions
  // s*SLAB + E*q4 .. +E-1 (16 bytes).
  auto load_frags = [&](const char* base, int c, F (&f)[NB][NKS]) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const long row = rowbase + clamp_tok(c * C + 16 * tb + n16);
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        f[tb][s] = *reinterpret_cast<const F*>(base + row * kq_stride + (s * SLAB + E * q4) * CF::S);
    }
  };

  if (wave < NDV) {
    // =========================================================== value waves
    const int dvcol = tile * DVT + wave * 16 + n16;  // this lane's state column
    const long sbase = (long)chain * DK * p.dv;      // h0/hT slab of this chain
    // Accumulator block b, element e holds M[key(b, 4q+e)][dvcol].  For bf16
    // the key order makes two stacked blocks a fragment with natural key
    // positions and lets one transposing read fetch four keys.
    auto key_of = [&](int b, int r) -> int {
      if constexpr (BPS == 2) {
        return 32 * (b >> 1) + 8 * (r >> 2) + 4 * (b & 1) + (r & 3);
      } else {
        return 16 * b + r;
      }
    };
    f32x4 Macc[NKB];
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Macc[b][e] = p.h0 ? p.h0[sbase + (long)key_of(b, 4 * q4 + e) * p.dv + dvcol] : 0.f;
    }

    // One step: chunk c = it - 2 with its Q fragments in `qcur`; Q of chunk
    // c+1 is fetched into `qnxt` for the next step.
    auto step = [&](int it, F (&qcur)[NB][NKS], F (&qnxt)[NB][NKS]) {
      const int c = it - 2;
      if (c + 1 >= 0 && c + 1 < NC) load_frags(qbase, c + 1, qnxt);
      if (c >= 0) {
        const char* sk = kbuf(c);
        const char* sv = vbuf(c);
        const char* st = tbuf(c);
        const char* sp = pbuf(c);
        const float* vec = vecb(c);

        // LDS reads for the first products: K fragments and V.
        F Kf[NB][NKS];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[tb][s] = frag_nat<TI, DK>(sk, 16 * tb + n16, s * SLAB, q4);
        // V in accumulator layout: Vc[tb][e] = V[16 tb + 4 q + e][16 wave + n16].
        f32x4 Vc[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          if constexpr (sizeof(TI) == 2) {
            const int src = lane & 15;
            const bf16x4 r = lds_read_tr(sv, SV::off(16 * tb + 4 * q4 + (src >> 2), 16 * wave + 4 * (src & 3)));
            Vc[tb] = f32x4{(float)r[0], (float)r[1], (float)r[2], (float)r[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              Vc[tb][e] = lds_ld<float>(sv, SV::off(16 * tb + 4 * q4 + e, 16 * wave + n16));
          }
        }
        F Mf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) Mf[s] = acc_frag<TI>(Macc, s);

        // Y = K M
        f32x4 Y[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s) y = MM::mma(Kf[tb][s], Mf[s], y);
          Y[tb] = y;
        }

        // LDS reads for the later products: Tinv, P.
        F Tf[NB][NTS], Pf[NB][NTS];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int s = 0; s <= (16 * tb + 15) / SLAB; ++s) {
            Tf[tb][s] = frag_pi<TI, C>(st, 16 * tb + n16, s * SLAB, q4);
            Pf[tb][s] = frag_pi<TI, C>(sp, 16 * tb + n16, s * SLAB, q4);
          }

        // O^T, first part: (M^T Q^T) diag(Gam); independent of Y, fills the
        // MFMA pipe while X is formed.
        f32x4 O[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s) o = MM::mma(Mf[s], qcur[tb][s], o);
          O[tb] = o;
        }

        // X = beta (V - Gam Y)
        f32x4 X[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(vec + 16 * tb + 4 * q4);
          const f32x4 gm = *reinterpret_cast<const f32x4*>(vec + 2 * C + 16 * tb + 4 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) X[tb][e] = bt[e] * __builtin_fmaf(-gm[e], Y[tb][e], Vc[tb][e]);
        }
        F Xf[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) Xf[s] = acc_frag<TI>(X, s);

        // U = Tinv X  (Tinv is lower triangular: slabs up to the diagonal)
        f32x4 U[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s <= (16 * tb + 15) / SLAB; ++s) u = MM::mma(Tf[tb][s], Xf[s], u);
          U[tb] = u;
        }

        // Transposed K for the state update (tokens along the contraction).
        F KT[NKB][NTS];
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            if constexpr (BPS == 2) {
              // Two transposing reads: tokens 32s + 4q + k and 32s + 16 + 4q + k
              // of keys key_of(b, n16).
              const int src = lane & 15;
              const int key0 = 32 * (b >> 1) + 8 * (src & 3) + 4 * (b & 1);
              const bf16x4 lo = lds_read_tr(sk, SK::off(32 * s + 4 * q4 + (src >> 2), key0));
              const bf16x4 hi = lds_read_tr(sk, SK::off(32 * s + 16 + 4 * q4 + (src >> 2), key0));
              KT[b][s] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
#pragma unroll
              for (int e = 0; e < E; ++e) KT[b][s][e] = lds_ld<TI>(sk, SK::off(s * 16 + 4 * q4 + e, key_of(b, n16)));
            }
          }

        F Uf[NTS], Wf[NTS];
        {
          f32x4 WU[NB];
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(vec + 3 * C + 16 * tb + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) WU[tb][e] = wv[e] * U[tb][e];
          }
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            Uf[s] = acc_frag<TI>(U, s);
            Wf[s] = acc_frag<TI>(WU, s);
          }
        }

        // M <- Gam_C M + K^T diag(w) U
        const float gC = vec[2 * C + C - 1];
#pragma unroll
        for (int b = 0; b < NKB; ++b) {
          f32x4 m = Macc[b];
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] *= gC;
#pragma unroll
          for (int s = 0; s < NTS; ++s) m = MM::mma(KT[b][s], Wf[s], m);
          Macc[b] = m;
        }

        // O^T, second part: + U^T P^T; store.
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 o = O[tb];
          const float gcol = vec[2 * C + 16 * tb + n16];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] *= gcol;
#pragma unroll
          for (int s = 0; s <= (16 * tb + 15) / SLAB; ++s) o = MM::mma(Uf[s], Pf[tb][s], o);
          const int t = c * C + 16 * tb + n16;
          if (t < len) {
            char* dst = p.out + (((rowbase + t) * H + hh) * (long)p.dv + tile * DVT + wave * 16 + 4 * q4) * CF::S;
            if constexpr (sizeof(TI) == 2) {
              *reinterpret_cast<bf16x4*>(dst) = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
            } else {
              *reinterpret_cast<f32x4*>(dst) = o;
            }
          }
        }
      }
      lds_barrier();
    };

    F qa[NB][NKS], qb[NB][NKS];
    for (int it = 0; it < NIT; it += 2) {
      step(it, qa, qb);
      if (it + 1 < NIT) step(it + 1, qb, qa);
    }

#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.hT[sbase + (long)key_of(b, 4 * q4 + e) * p.dv + dvcol] = Macc[b][e];

  } else if (wave == CF::W_S) {
    // ============================================================ solve wave
    // Also stages this tile's V two chunks ahead.
    auto load_v = [&](int c, uint4 (&st)[CF::NPV]) {
#pragma unroll
      for (int i = 0; i < CF::NPV; ++i) {
        const int gi = lane + 64 * i;
        if ((C * CF::GRV) % 64 == 0 || gi < C * CF::GRV) {
          const int row = gi / CF::GRV, gc = gi % CF::GRV;
          st[i] = *reinterpret_cast<const uint4*>(vbase + (rowbase + clamp_tok(c * C + row)) * v_stride + gc * 16);
        }
      }
    };
    auto step = [&](int it, uint4 (&vcur)[CF::NPV]) {
      if (it < NC) {
        char* sv = vbuf(it);
#pragma unroll
        for (int i = 0; i < CF::NPV; ++i) {
          const int gi = lane + 64 * i;
          if ((C * CF::GRV) % 64 == 0 || gi < C * CF::GRV) lds_st<uint4>(sv, SV::goff(gi / CF::GRV, gi % CF::GRV), vcur[i]);
        }
        if (it + 2 < NC) load_v(it + 2, vcur);
      }
      const int c = it - 1;
      if (c >= 0 && c < NC) {
        const char* sk = kbuf(c);
        const char* sa = abuf(c);
        char* st = tbuf(c);
        char* stt = smem + CF::OFF_TT;
        float* sad = reinterpret_cast<float*>(smem + CF::OFF_AD);
        const float* vec = vecb(c);

        // Diagonal blocks of A: beta_i (K K^T)_ij exp(gamma_i - gamma_j), j < i.
        F Kf[NB][NKS];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[b][s] = frag_nat<TI, DK>(sk, 16 * b + n16, s * SLAB, q4);
        float gi[NB], bi[NB];
        f32x4 gj[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          gi[b] = vec[C + 16 * b + n16];
          bi[b] = vec[16 * b + n16];
          gj[b] = *reinterpret_cast<const f32x4*>(vec + C + 16 * b + 4 * q4);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s) a = MM::mma(Kf[b][s], Kf[b][s], a);
          // a[e] = (K K^T)[i = 16 b + n16][j = 16 b + 4 q4 + e]
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool keep = 4 * q4 + e < n16;
            r[e] = keep ? bi[b] * a[e] * __expf(gi[b] - gj[b][e]) : 0.f;
          }
          *reinterpret_cast<f32x4*>(sad + b * CF::AD_STRIDE + 16 * n16 + 4 * q4) = r;
        }

        // Diagonal 16x16 blocks of Tinv: forward substitution in fp32.  Lane
        // (block q4, column n16) computes column n16 of its block's inverse;
        // the rows of A it needs are all loaded before the substitution.
        if (q4 < NB) {
          const float* ad = sad + q4 * CF::AD_STRIDE;
          f32x4 arow[16][4];
#pragma unroll
          for (int i = 1; i < 16; ++i)
#pragma unroll
            for (int l4 = 0; l4 < i; l4 += 4) arow[i][l4 >> 2] = *reinterpret_cast<const f32x4*>(ad + 16 * i + l4);
          __builtin_amdgcn_sched_barrier(0);
          float tc[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float s = (i == n16) ? 1.f : 0.f;
#pragma unroll
            for (int l = 0; l + 1 < i; ++l) s = __builtin_fmaf(-arow[i][l >> 2][l & 3], tc[l], s);
            if (i > 0) s = __builtin_fmaf(-arow[i][(i - 1) >> 2][(i - 1) & 3], tc[i - 1], s);
            tc[i] = s;
          }
          const int base = 16 * q4;
#pragma unroll
          for (int i = 0; i < 16; ++i) st1<TI, C>(st, base + i, base + n16, tc[i]);
#pragma unroll
          for (int i = 0; i < 16; i += 4)
            st4<TI, C>(stt, base + n16, base + i, f32x4{tc[i], tc[i + 1], tc[i + 2], tc[i + 3]});
        }
        if constexpr (BPS == 2) {
#pragma unroll
          for (int b1 = 0; b1 + 1 < NB; b1 += 2)
            st4<TI, C>(st, 16 * b1 + n16, 16 * (b1 + 1) + 4 * q4, f32x4{0.f, 0.f, 0.f, 0.f});
        }

        // Off-diagonal blocks, by distance from the diagonal:
        //   Tinv_ij = -Tinv_ii * sum_{j <= l < i} A_il Tinv_lj.
#pragma unroll
        for (int d = 1; d < NB; ++d) {
          f32x4 R[NB];
#pragma unroll
          for (int i = d; i < NB; ++i) {
            const int j = i - d;
            const int L = 16 * d;
            f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s * SLAB < L; ++s) {
              const bool valid = s * SLAB + E * q4 < L;
              const F fa = valid ? frag_nat<TI, C>(sa, 16 * i + n16, 16 * j + s * SLAB, q4) : MM::zero();
              const F fb = valid ? frag_nat<TI, C>(stt, 16 * j + n16, 16 * j + s * SLAB, q4) : MM::zero();
              r = MM::mma(fa, fb, r);
            }
            R[i] = r;  // R[row 16 i + 4 q4 + e][col 16 j + n16]
          }
#pragma unroll
          for (int i = d; i < NB; ++i) {
            const int j = i - d;
            f32x4 o = MM::mma(frag_pi1<TI, C>(st, 16 * i + n16, 16 * i, q4), MM::from_acc1(R[i]),
                              f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              o[e] = -o[e];
              st1<TI, C>(st, 16 * i + 4 * q4 + e, 16 * j + n16, o[e]);
            }
            st4<TI, C>(stt, 16 * j + n16, 16 * i + 4 * q4, o);
          }
        }
      }
      lds_barrier();
    };

    uint4 va[CF::NPV], vb[CF::NPV];
    if (NC > 0) load_v(0, va);
    if (NC > 1) load_v(1, vb);
    for (int it = 0; it < NIT; it += 2) {
      step(it, va);
      if (it + 1 < NIT) step(it + 1, vb);
    }
  } else {
    // ===================================================== Gram / loader wave
    // K and Q fragments (and g, beta) are fetched two chunks ahead into one
    // of two register sets and used straight from registers.
    auto load_gb = [&](int c, float& sg, float& sb) {
      sg = 0.f;
      sb = 0.f;
      const int t = c * C + lane;
      if (lane < C && t < len) {
        const long idx = (rowbase + t) * H + hh;
        sg = p.g[idx];
        sb = p.beta[idx];
      }
    };
    auto step = [&](int it, F (&Kc)[NB][NKS], F (&Qc)[NB][NKS], float& sg, float& sb) {
      const int c = it;
      if (c < NC) {
        char* sk = kbuf(c);
        char* sa = abuf(c);
        char* sp = pbuf(c);
        float* vec = vecb(c);
        // Stage K of chunk c for the solve and value waves.
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
          for (int s = 0; s < NKS; ++s) lds_st<F>(sk, SK::off(16 * tb + n16, s * SLAB + E * q4), Kc[tb][s]);

        // In-chunk cumulative log-decay and the per-token vectors.
        const float gam = wave_prefix_sum(sg, lane);
        const float bet = sb;
        const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), C - 1));
        if (lane < C) {
          vec[lane] = bet;
          vec[C + lane] = gam;
          vec[2 * C + lane] = __expf(gam);
          vec[3 * C + lane] = __expf(gC - gam);
        }
        float gi[NB], bi[NB];
        f32x4 gj[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          gi[b] = vec[C + 16 * b + n16];
          bi[b] = vec[16 * b + n16];
          gj[b] = *reinterpret_cast<const f32x4*>(vec + C + 16 * b + 4 * q4);
        }

#pragma unroll
        for (int b1 = 0; b1 < NB; ++b1) {
#pragma unroll
          for (int b2 = 0; b2 <= b1; ++b2) {
            // Decay exp(gamma_i - gamma_j), i = 16 b1 + n16, j = 16 b2 + 4 q4 + e,
            // shared by A (j < i) and P (j <= i); zero above the diagonal.
            f32x4 dec;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool keep = b2 < b1 || 4 * q4 + e <= n16;
              dec[e] = keep ? __expf(gi[b1] - gj[b2][e]) : 0.f;
            }
            f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) pq = MM::mma(Kc[b2][s], Qc[b1][s], pq);
            // pq[e] = (Q K^T)[i][j]
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = pq[e] * dec[e];
            st4<TI, C>(sp, 16 * b1 + n16, 16 * b2 + 4 * q4, r);
            if (b2 < b1) {  // off-diagonal block of A (the solve wave forms the diagonal ones)
              f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < NKS; ++s) kk = MM::mma(Kc[b2][s], Kc[b1][s], kk);
              f32x4 ra;
#pragma unroll
              for (int e = 0; e < 4; ++e) ra[e] = bi[b1] * kk[e] * dec[e];
              st4<TI, C>(sa, 16 * b1 + n16, 16 * b2 + 4 * q4, ra);
            }
          }
          if (BPS == 2 && (b1 & 1) == 0 && b1 + 1 < NB)
            st4<TI, C>(sp, 16 * b1 + n16, 16 * (b1 + 1) + 4 * q4, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (c + 2 < NC) {
          load_frags(kbase, c + 2, Kc);
          load_frags(qbase, c + 2, Qc);
          load_gb(c + 2, sg, sb);
        }
      }
      lds_barrier();
    };

    F ka[NB][NKS], qa_[NB][NKS], kb[NB][NKS], qb_[NB][NKS];
    float ga = 0.f, ba = 0.f, gb = 0.f, bb = 0.f;
    if (NC > 0) {
      load_frags(kbase, 0, ka);
      load_frags(qbase, 0, qa_);
      load_gb(0, ga, ba);
    }
    if (NC > 1) {
      load_frags(kbase, 1, kb);
      load_frags(qbase, 1, qb_);
      load_gb(1, gb, bb);
    }
    for (int it = 0; it < NIT; it += 2) {
      step(it, ka, qa_, ga, ba);
      if (it + 1 < NIT) step(it + 1, kb, qb_, gb, bb);
    }
  }
}

// ======================================================================
// bf16 kernel
//
// Same chunk algebra, reorganised for bf16 so that every global access goes
// through a per-sequence buffer descriptor (rows past the sequence end read
// as zero and stores past it are dropped, so the ragged tail needs no
// special code) and q, k and this tile's v land in LDS by direct
// buffer-to-LDS copies.  The correction is split into a state-independent
// and a state-dependent part:
//
//     U = Tinv diag(beta) V - Tinv diag(beta Gam) K M = u + T' Y,
//     u = Tinv diag(beta) V,   T' = -Tinv diag(beta Gam),   Y = K M,
//
// so that only Y, one triangular product and the update remain in the
// chunk-to-chunk recurrence.  One workgroup per (chain, 32-column value
// tile), eight waves (two per SIMD), one LDS barrier per step; chunk c is
// Gram-processed at step c, solved at step c+1, finished at step c+2:
//
//   loader wave (step c): copies v of chunk c+1 and k of chunk c+2 into the
//       LDS rings (two steps ahead of their first readers); g and beta of
//       chunk c+2; per-token vectors of chunk c+1; once the Gram wave has
//       published them (LDS flag), the inverses of the 16x16 diagonal
//       blocks of (I + A) of chunk c (fp32 forward substitution, one lane
//       per column).
//   Gram wave (step c): diagonal blocks of A of chunk c (fp32, published
//       first), then the off-diagonal blocks (bf16).
//   T and u solve waves (step c+1): block forward substitution of (I + A)
//       R = diag(beta) and of (I + A) R = diag(beta) V on the MFMA;
//       publish T' = -R diag(Gam) and u = R.
//   two state waves (step c+2), one per 16-column half: Y = K M,
//       U = u + T' Y, publish U (LDS flag), the update
//       M <- Gam_C M + K^T diag(w) U, publish the bf16 state.
//   two output waves (step c+2), each owning half of the chunk's 16-row
//       blocks: diag(Gam) Q M and the masked decayed P = (Q K^T) * D, then
//       (once U is published) P U, and the stores; q comes straight from
//       HBM into registers one step ahead.
//
// The decay exp(gamma_i - gamma_j) of an off-diagonal block (rows in block
// b1, columns in an earlier block) is the product of two factors through
// the first token of block b1, exp(gamma_i - gamma_{16 b1}) and
// exp(gamma_{16 b1} - gamma_j); for g <= 0 both are at most 1, so neither
// overflows.  Diagonal blocks use the direct exponential.
//
// LDS layouts (all chosen so that every fragment read is one instruction
// from a per-lane base register plus a compile-time offset):
//   q/k tiles: rows of 2*DK bytes, 16-byte granules XOR-permuted by row;
//   v tiles:   rows of 64 bytes, granules XOR-permuted by row;
//   A tile (off-diagonal blocks of A and the inverted diagonal blocks):
//       rows of 2*C bytes; inside each 32-column slab the columns are
//       stored in the order {0-3, 16-19, 4-7, 20-23, ...} so that the eight
//       positions a lane holds in a 16x16x32 fragment are contiguous;
//   T'^T tile: rows of 2*C bytes in natural column order (read with
//       transposing reads); both C x C tiles XOR-permute granules by row;
//   u: fp32 accumulator blocks, U and the state: bf16 fragments, all
//       stored lane-major so that each lane reads 16 contiguous bytes.
// ======================================================================


__device__ static inline int swz_v(int r) { return (r >> 2) & 1; }
// Value columns of a 32-column tile: position r (0..15) of 16-column block
// cb holds tile column 8 (r >> 2) + 4 ((cb ^ (r >> 2)) & 1) + (r & 3).  The
// two blocks' positions 4g .. 4g+3 together cover the eight columns 8g ..
// 8g+7, so an output lane writes 16 contiguous bytes, and the transposing
// reads of v alternate 8-byte halves across lanes (no bank conflicts).
__device__ static inline int tile_col(int cb, int r) { return 8 * (r >> 2) + 4 * ((cb ^ (r >> 2)) & 1) + (r & 3); }

// Issue priority (s_setprio, 0..3) of the Gram wave's diagonal phase and
// the loader's diagonal-block inverses (GL), of the state waves (S) and of
// the output waves (O); the other waves and phases stay at 0.  The Gram ->
// loader chain goes first: giving the state waves equal or higher priority
// measured ~10% slower.
#ifndef GDN_PRIO_GL
#define GDN_PRIO_GL 3
#endif
#ifndef GDN_PRIO_S
#define GDN_PRIO_S 2
#endif
#ifndef GDN_PRIO_O
#define GDN_PRIO_O 0
#endif
#ifndef GDN_ROLEMAP
#define GDN_ROLEMAP 0x54673210u
#endif

template <int DK, int C>
struct Cfg16 {
  static constexpr int DVT = 32, NCB = 2;  // value columns per workgroup, 16-column blocks
  static constexpr int NB = C / 16, NTS = C / 32, NKB = DK / 16, NKS = DK / 32;
  static constexpr int KQ_ROWB = DK * 2, V_ROWB = 64, CC_ROWB = C * 2;
  static constexpr int GR = KQ_ROWB / 16;
  static constexpr int KQ_BYTES = C * KQ_ROWB, V_BYTES = C * V_ROWB, CC_BYTES = C * CC_ROWB;
  static constexpr int UF_BYTES = NCB * NTS * 1024;  // U, bf16 fragments
  static constexpr int UU_BYTES = NB * NCB * 1024;   // u, fp32 accumulator blocks
  static constexpr int MF_BYTES = NCB * NKS * 1024;  // state, bf16 fragments
  // Per-token vectors (fp32, C each): beta, lambda = gamma*log2(e), Gam,
  // w = exp(gamma_C - gamma), exp(gamma_t - gamma at the start of t's
  // block), and for b = 1..NB-1, exp(gamma_{16 b} - gamma_t) (t < 16 b).
  static constexpr int F_BETA = 0, F_LAM = 1, F_GAM = 2, F_W = 3, F_ER = 4;
  static constexpr int NF = 4 + NB;
  // fp32 diagonal blocks: padded rows, and blocks 4 banks apart so that the
  // four blocks' rows are read without bank conflicts.
  static constexpr int AD_ROW = 20, AD_BLK = 16 * AD_ROW + 4;
  static constexpr int KQ_INS = KQ_BYTES / 1024, V_INS = V_BYTES / 1024;  // copies per chunk
  static constexpr int KQ_RPI = 1024 / KQ_ROWB, V_RPI = 1024 / V_ROWB;    // rows per copy
  // Wave roles.  ROLEMAP holds the role of wave w in bits [4w, 4w + 4);
  // waves w and w + 4 share a SIMD, so the map also places the roles on
  // SIMDs (by default: state half 0 with the Gram wave, state half 1 with
  // the loader, each output wave with one of the solve waves, whose work
  // ends early in the step).
  static constexpr int R_S0 = 0, R_S1 = 1, R_OA = 2, R_OB = 3, R_X = 4, R_XU = 5, R_L = 6, R_G = 7, NW = 8;
  static constexpr unsigned ROLEMAP = GDN_ROLEMAP;
  // Output wave o owns row blocks own_tb(o, 0..NOWN-1): {0, 3} and {1, 2}
  // for four blocks (equal MFMA work), {0} and {1} for two.
  static constexpr int NOWN = NB == 4 ? 2 : 1;
  __host__ __device__ static constexpr int own_tb(int o, int i) { return NB == 4 ? (i == 0 ? o : 3 - o) : o; }
  // Ring depths: k is copied two steps ahead of the Gram wave and read
  // until the state and output waves finish the chunk two steps later; v
  // is copied two steps ahead of the u solve.
  static constexpr int NKR = 5, NVR = 3;
  static constexpr int LDS = NKR * KQ_BYTES + NVR * V_BYTES + 3 * CC_BYTES + UU_BYTES + MF_BYTES + UF_BYTES +
                             4 * NF * C * 4 + NB * AD_BLK * 4 + 32;
  static_assert(NB >= 2 && NB <= 4 && NKS >= 1 && GR >= 4, "shape");
};


template <int DK, int C>
__global__ __launch_bounds__(512, 1) void gdn_bf16_kernel(const Params p) {
  using CF = Cfg16<DK, C>;
  static_assert(64 * CF::NW == 512, "launch bounds");
  using MM = Mma<__bf16>;
  using F = bf16x8;
  constexpr int NB = CF::NB, NTS = CF::NTS, NKB = CF::NKB, NKS = CF::NKS, NCB = CF::NCB, NF = CF::NF;
  constexpr int GR = CF::GR, KQR = CF::KQ_ROWB, CCR = CF::CC_ROWB;
  constexpr float kLog2e = 1.4426950408889634f;

  // Separate LDS objects: the loader wave's own LDS accesses (flags,
  // vectors) never alias its in-flight copies (q, k, v).
  __shared__ __attribute__((aligned(16))) char sK[CF::NKR * CF::KQ_BYTES];
  __shared__ __attribute__((aligned(16))) char sV[CF::NVR * CF::V_BYTES];
  __shared__ __attribute__((aligned(16))) char sAT[2 * CF::CC_BYTES];
  __shared__ __attribute__((aligned(16))) char sTP[CF::CC_BYTES];
  __shared__ __attribute__((aligned(16))) char sUU[CF::UU_BYTES];
  __shared__ __attribute__((aligned(16))) char sMF[CF::MF_BYTES];
  __shared__ __attribute__((aligned(16))) char sUF[CF::UF_BYTES];
  __shared__ __attribute__((aligned(16))) float sVEC[4 * NF * C];
  __shared__ __attribute__((aligned(16))) float sAD[NB * CF::AD_BLK];
  // Flags, each holding chunk index + 1:
  //   [0], [1] U published by state wave 0 / 1 (-> output waves);
  //   [2], [3] T' and u read by state wave 0 / 1 (-> solve waves, which
  //            then overwrite them);
  //   [4], [5] state read by output wave 0 / 1 (-> state waves, which then
  //            publish the next state over it);
  //   [6] diagonal blocks of A published (Gram -> loader wave).
  __shared__ int sFLAG[8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int role = (CF::ROLEMAP >> (4 * wave)) & 15;
  const int q4 = lane >> 4, n16 = lane & 15;
  const int src = lane & 15;  // source lane of a transposing read

  // Packed batch: workgroups start in dispatch order, so the longest
  // sequences are handed out first (longest-processing-time-first); chains
  // are dealt round-robin over the 8 XCDs, a chain's value tiles together
  // on one XCD.  Otherwise each XCD takes a contiguous range of items.
  __shared__ int sLEN[GDN_LPT_MAX];
  __shared__ int sPICK;
  int chain_v, tile_v, seg_v = 0;
  if (p.lpt) {
    const int nseq = p.nwg / (p.ntile * p.H);
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int k = (slot / p.ntile) * 8 + xcd;  // k-th chain in length order
    tile_v = slot % p.ntile;
    const int t = threadIdx.x;
    if (t < nseq) sLEN[t] = p.cu[t + 1] - p.cu[t];
    __syncthreads();
    if (t < nseq) {
      const int lt = sLEN[t];
      int rank = 0;  // sequences ahead of t: longer, or as long with a lower index
      for (int m = 0; m < nseq; ++m) {
        const int lm = sLEN[m];
        rank += (lm > lt || (lm == lt && m < t)) ? 1 : 0;
      }
      if (rank == k / p.H) sPICK = t;
    }
    __syncthreads();
    chain_v = sPICK * p.H + k % p.H;
  } else {
    const int item = xcd_remap(blockIdx.x, p.nwg);
    chain_v = item / (p.ntile * p.nseg);
    seg_v = (item / p.ntile) % p.nseg;
    tile_v = item % p.ntile;
  }
  const int chain = __builtin_amdgcn_readfirstlane(chain_v);
  const int tile = __builtin_amdgcn_readfirstlane(tile_v);
  const int seg = __builtin_amdgcn_readfirstlane(seg_v);
  const int H = p.H;
  const int bseq = chain / H, hh = chain % H;
  long rowbase;
  int len;
  if (p.cu) {
    rowbase = p.cu[bseq];
    len = p.cu[bseq + 1] - p.cu[bseq];
  } else {
    rowbase = (long)bseq * p.T;
    len = p.T;
  }
  rowbase = __builtin_amdgcn_readfirstlane((int)rowbase);
  len = __builtin_amdgcn_readfirstlane(len);
  // Sequence segments: find where this segment's recurrence starts (see
  // HALO_NATS), then narrow the token range to [halo start, segment end).
  int use_h0 = 1, write_hT = 1, store_from = 0;
  if (p.nseg > 1) {
    __shared__ int sSTART;
    const int c0 = seg * p.seg_chunks;                        // first chunk whose outputs are stored
    const int c1 = min(c0 + p.seg_chunks, (len + C - 1) / C);  // one past the segment's last chunk
    if (wave == 0) {
      int cs = c0;
      float acc = 0.f;  // log of the transition-norm product over chunks [cs, c0)
      while (cs > 0 && acc > -HALO_NATS) {
        --cs;  // chunks before c0 are whole: every lane < C holds a token
        float e = 0.f;
        if (lane < C) {
          const long th = (rowbase + (long)cs * C + lane) * H + hh;
          const uint4* kr = reinterpret_cast<const uint4*>(p.k + th * DK * 2);
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
          e = p.g[th] + (f > 1.f ? __logf(f) : 0.f);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) e += __shfl_xor(e, d);
        acc += e;
      }
      if (lane == 0) sSTART = cs;
    }
    __syncthreads();
    const int cs = sSTART;
    use_h0 = cs == 0;
    write_hT = seg == p.nseg - 1;
    store_from = c0 - cs;
    rowbase = __builtin_amdgcn_readfirstlane((int)(rowbase + (long)cs * C));
    len = __builtin_amdgcn_readfirstlane(min(len, c1 * C) - cs * C);
  }
  const int NC = (len + C - 1) / C;
  const int NIT = NC > 0 ? NC + 2 : 0;
  const long kq_stride = (long)H * DK * 2;  // bytes between tokens in q/k
  const long v_stride = (long)H * p.dv * 2;  // bytes between tokens in v/out
  auto vec_of = [&](int c) { return sVEC + (c & 3) * NF * C; };

  // Lane-constant parts of the fragment addresses.
  // q/k fragment (row 16 tb + n16, natural slab s): base[s] + 16*KQR*tb.
  int kq_frag[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kq_frag[s] = n16 * KQR + 16 * ((4 * s + q4) ^ swz_kq<GR>(n16));
  // A-tile fragment (row 16 b + n16, slab s) and the Gram wave's 4-wide
  // stores (slab s, half): base[s] + 16*CCR*b (+ 8 for the second half).
  int cc_frag[NTS];
#pragma unroll
  for (int s = 0; s < NTS; ++s) cc_frag[s] = n16 * CCR + 16 * ((4 * s + q4) ^ swz_cc<C>(n16));

  if (role == CF::R_L) {
    // ========================================================== loader wave
    // Copy i of a chunk writes LDS bytes [1024 i, 1024 i + 1024): lane l
    // fills granule l % GR of row i*RPI + l/GR with the logical granule
    // (l % GR) ^ swz(row).
    int kq_src[CF::KQ_INS], v_src[CF::V_INS];
#pragma unroll
    for (int i = 0; i < CF::KQ_INS; ++i) {
      const int r = i * CF::KQ_RPI + lane / GR;
      kq_src[i] = (int)(r * kq_stride) + 16 * ((lane % GR) ^ swz_kq<GR>(r));
    }
#pragma unroll
    for (int i = 0; i < CF::V_INS; ++i) {
      const int r = i * CF::V_RPI + lane / 4;
      v_src[i] = (int)(r * v_stride) + 16 * ((lane & 3) ^ swz_v(r));
    }
    // g and beta: lane t < C reads token t of the chunk; other lanes read
    // past any descriptor's end (zero).
    const int gb_src = lane < C ? lane * H * 4 : 0x7ffffff0;

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
    auto issue_k = [&](int c) {
      const long row0 = rowbase + (long)c * C;
      const long left = c < NC ? (long)(len - c * C) : 0;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0 * kq_stride + hh * DK * 2, left * kq_stride);
      char* dk = sK + (c % CF::NKR) * CF::KQ_BYTES;
#pragma unroll
      for (int i = 0; i < CF::KQ_INS; ++i) copy_to_lds(rk, dk + i * 1024, kq_src[i]);
    };
    auto issue_v = [&](int c) {
      const long row0 = rowbase + (long)c * C;
      const long left = c < NC ? (long)(len - c * C) : 0;
      const __amdgpu_buffer_rsrc_t rv =
          make_rsrc(p.v + row0 * v_stride + (hh * p.dv + tile * CF::DVT) * 2, left * v_stride);
      char* dv = sV + (c % CF::NVR) * CF::V_BYTES;
#pragma unroll
      for (int i = 0; i < CF::V_INS; ++i) copy_to_lds(rv, dv + i * 1024, v_src[i]);
    };
    auto make_vec = [&](int c, float sg, float sb) {
      float* vec = vec_of(c);
      const float lam = wave_prefix_sum(sg * kLog2e, lane);
      const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), C - 1));
      float lb[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) lb[b] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 16 * b));
      if (lane < C) {
        const int blk = lane >> 4;
        float lown = lb[0];
#pragma unroll
        for (int b = 1; b < NB; ++b) lown = blk == b ? lb[b] : lown;
        vec[CF::F_BETA * C + lane] = sb;
        vec[CF::F_LAM * C + lane] = lam;
        vec[CF::F_GAM * C + lane] = exp2_fast(lam);
        vec[CF::F_W * C + lane] = exp2_fast(lamC - lam);
        vec[CF::F_ER * C + lane] = exp2_fast(lam - lown);
#pragma unroll
        for (int b = 1; b < NB; ++b) vec[(CF::F_ER + b) * C + lane] = lane < 16 * b ? exp2_fast(lb[b] - lam) : 0.f;
      }
    };

    // Diagonal-block inverse: lane (block q4, column n16) writes row n16 of
    // Tbb^T (= column n16 of Tbb): four 4-wide pieces.
    int t_dst[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * q4 + n16;
      t_dst[m] = r * CCR + 16 * ((4 * (q4 >> 1) + m) ^ swz_cc<C>(r)) + 8 * (q4 & 1);
    }
    // Inverse of each 16x16 diagonal block of (I + A) of chunk c, once the
    // Gram wave has published them: lane (block q4, column n16) runs forward
    // substitution down the block.
    auto diag_inverse = [&](int c) {
      flag_wait_lds(&sFLAG[6], c + 1);
      if (q4 < NB) {
        const float* A = sAD + q4 * CF::AD_BLK;
        // Row i holds columns 0..i-1: whole 4-wide pieces, then a 2- and/or
        // 1-wide piece, so every value read is used.
        float ar[16][16];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          const float* row = A + i * CF::AD_ROW;
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
        // later row, so the rows' sums proceed side by side (each row still
        // accumulates its terms in increasing l).
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tc[i] = (i == n16) ? 1.f : 0.f;
#pragma unroll
        for (int l = 0; l < 15; ++l)
#pragma unroll
          for (int i = l + 1; i < 16; ++i) tc[i] = __builtin_fmaf(-ar[i][l], tc[l], tc[i]);
        char* sat = sAT + (c & 1) * CF::CC_BYTES;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          lds_st<bf16x4>(sat, t_dst[m],
                         bf16x4{(__bf16)tc[4 * m], (__bf16)tc[4 * m + 1], (__bf16)tc[4 * m + 2], (__bf16)tc[4 * m + 3]});
      }
    };

    // Wait until at most the current step's loads and copies are in flight
    // and this wave's LDS stores are done, then join the barrier.  (A plain
    // LDS fence here would also wait for the copies just issued.)
    constexpr int NOPS = CF::KQ_INS + CF::V_INS + 2;
    static_assert(NOPS < 64, "vmcnt range");
    constexpr int WAIT_NOPS = (NOPS & 15) | ((NOPS >> 4) << 14) | (7 << 4);  // vmcnt(NOPS) lgkmcnt(0)
    auto step_barrier = [&]() {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(WAIT_NOPS);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    if (lane < 8) sFLAG[lane] = 0;
    float g0 = 0.f, b0 = 0.f, g1 = 0.f, b1 = 0.f;
    if (NIT > 0) {
      load_gb(0, g0, b0);
      issue_k(0);
      make_vec(0, g0, b0);
      issue_v(0);
      load_gb(1, g1, b1);
      issue_k(1);
    }
    step_barrier();  // k of chunk 0 has landed

    // Step it: v of chunk it+1 and k of chunk it+2 (two steps ahead of
    // their first readers), g and beta of chunk it+2, the vectors of chunk
    // it+1 from the g and beta loaded one step earlier, and the diagonal-
    // block inverses of chunk it.
    auto step = [&](int it, float& gu, float& bu, float& gl, float& bl) {
      load_gb(it + 2, gl, bl);
      issue_v(it + 1);
      issue_k(it + 2);
      if (it + 1 < NC) make_vec(it + 1, gu, bu);
      if (it < NC) {
        if (GDN_PRIO_GL) __builtin_amdgcn_s_setprio(GDN_PRIO_GL);
        diag_inverse(it);
        if (GDN_PRIO_GL) __builtin_amdgcn_s_setprio(0);
      }
      step_barrier();
    };
    for (int it = 0; it < NIT; it += 2) {
      step(it, g1, b1, g0, b0);
      if (it + 1 < NIT) step(it + 1, g0, b0, g1, b1);
    }
    // The last steps' copies (of chunks past the end) still write LDS: let
    // them land before this wave ends.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (role == CF::R_G) {
    // ============================================================ Gram wave
    lds_barrier();
    for (int it = 0; it < NIT; ++it) {
      const int c = it;
      if (c < NC) {
        if (GDN_PRIO_GL) __builtin_amdgcn_s_setprio(GDN_PRIO_GL);
        const char* sk = sK + (c % CF::NKR) * CF::KQ_BYTES;
        const float* vec = vec_of(c);
        char* sat = sAT + (c & 1) * CF::CC_BYTES;
        // A block result: lane (n16, q4) holds row i = 16 b1 + n16 and
        // columns j = 16 b2 + 4 q4 + e.  Diagonal blocks first (fp32, j < i),
        // published for the loader's inverses.
        F Kf[NB][NKS];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[b][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float li = vec[CF::F_LAM * C + 16 * b + n16];
          const float bi0 = vec[CF::F_BETA * C + 16 * b + n16];
          const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + CF::F_LAM * C + 16 * b + 4 * q4);
          f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s) kk = MM::mma(Kf[b][s], Kf[b][s], kk);
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = 4 * q4 + e < n16 ? bi0 * kk[e] * exp2_fast(li - lj[e]) : 0.f;
          *reinterpret_cast<f32x4*>(sAD + b * CF::AD_BLK + n16 * CF::AD_ROW + 4 * q4) = r;
        }
        flag_release(&sFLAG[6], c + 1);
        if (GDN_PRIO_GL) __builtin_amdgcn_s_setprio(0);
        // Off-diagonal blocks (bf16).
        float bi[NB], eri[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          bi[b] = vec[CF::F_BETA * C + 16 * b + n16];
          eri[b] = vec[CF::F_ER * C + 16 * b + n16];
        }
#pragma unroll
        for (int b1 = 1; b1 < NB; ++b1)
#pragma unroll
          for (int b2 = 0; b2 < b1; ++b2) {
            const f32x4 ec = *reinterpret_cast<const f32x4*>(vec + (CF::F_ER + b1) * C + 16 * b2 + 4 * q4);
            f32x4 kk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) kk = MM::mma(Kf[b2][s], Kf[b1][s], kk);
            const float sc = bi[b1] * eri[b1];
            f32x4 ra;
#pragma unroll
            for (int e = 0; e < 4; ++e) ra[e] = sc * kk[e] * ec[e];
            lds_st<bf16x4>(sat, cc_frag[b2 >> 1] + 16 * CCR * b1 + 8 * (b2 & 1), cvt4(ra));
          }
      }
      lds_barrier();
    }
  } else if (role == CF::R_X || role == CF::R_XU) {
    // ========================================================= solve waves
    // Tbb as an MFMA row operand (transposing read of Tbb^T): rows
    // 16 b + 4 q4 + (src >> 2), columns 16 b + 4 (src & 3) .. +3.
    int t_base[NTS];
#pragma unroll
    for (int bh = 0; bh < NTS; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      t_base[bh] = r * CCR + 16 * ((4 * bh + (src & 3)) ^ swz_cc<C>(r));
    }
    // V in accumulator layout: rows 16 tb + 4 q4 + (src >> 2), block
    // positions 4 (src & 3) .. +3 of block cb (tile columns tile_col).
    int v_base[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int r = 4 * q4 + (src >> 2), g = src & 3;
      v_base[cb] = r * CF::V_ROWB + 16 * (g ^ swz_v(r)) + 8 * ((cb ^ g) & 1);
    }
    // T'^T store: row j = 16 col + n16, columns 16 b + 4 q4 .. +3.
    auto tp_off = [&](int b, int col) {
      const int j = 16 * col + n16;
      return j * CCR + 16 * ((2 * b + (q4 >> 1)) ^ swz_cc<C>(j)) + 8 * (q4 & 1);
    };
    auto cat = [](bf16x4 lo, bf16x4 hi) { return F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; };

    // Row block b of (I + A) R = X: R_b = Tbb (X_b - sum_{j<b} A_bj R_j).
    // The T wave solves for X = diag(beta) (lower blocks only) and publishes
    // T' = -R diag(Gam); the u wave solves for X = diag(beta) V and
    // publishes u = R.  Each result block is rounded to bf16 once and reused
    // as the B operand of every later row block.
    auto solve_wave = [&](auto rc) {
      constexpr bool TW = decltype(rc)::value == 0;
      lds_barrier();
      for (int it = 0; it < NIT; ++it) {
        const int c = it - 1;
        if (c >= 0 && c < NC) {
          const float* vec = vec_of(c);
          char* sat = sAT + (c & 1) * CF::CC_BYTES;
          bf16x4 Tf[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) Tf[b] = lds_read_tr(sat, t_base[b >> 1] + 16 * CCR * b + 8 * (b & 1));
          // Row blocks of A left of the diagonal as pi-order fragments;
          // where the slab's upper half is the diagonal block the matching
          // operand half is zero.
          F Af[NB][NTS];
#pragma unroll
          for (int b = 1; b < NB; ++b)
#pragma unroll
            for (int s = 0; 32 * s < 16 * b; ++s) Af[b][s] = lds_at<F>(sat + cc_frag[s] + 16 * CCR * b);
          const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

          if constexpr (TW) {
            f32x4 RT[NB][NB];
            bf16x4 RH[NB][NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
              for (int col = 0; col <= b; ++col) {
                bf16x4 xh;
                if (col == b) {
                  const __bf16 bcol = (__bf16)vec[CF::F_BETA * C + 16 * b + n16];
#pragma unroll
                  for (int e = 0; e < 4; ++e) xh[e] = 4 * q4 + e == n16 ? bcol : (__bf16)0.f;
                } else {
                  // full- and half-depth products accumulate apart (see mma16)
                  f32x4 r = zero4, r16 = zero4;
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
            // Publish T' = -R diag(Gam) as T'^T, once the state wave has
            // read the previous chunk's.
            flag_wait_lds(&sFLAG[2], c);
            flag_wait_lds(&sFLAG[3], c);
            char* tp = sTP;
#pragma unroll
            for (int col = 0; col < NB; ++col) {
              const float ng = -vec[CF::F_GAM * C + 16 * col + n16];
#pragma unroll
              for (int b = col; b < NB; ++b) {
                f32x4 t;
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = RT[b][col][e] * ng;
                lds_st<bf16x4>(tp, tp_off(b, col), cvt4(t));
              }
            }
          } else {
            const char* sv = sV + (c % CF::NVR) * CF::V_BYTES;
            bf16x4 Vr[NB][NCB];
#pragma unroll
            for (int tb = 0; tb < NB; ++tb)
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) Vr[tb][cb] = lds_read_tr(sv, v_base[cb] + 16 * CF::V_ROWB * tb);
            f32x4 RU[NB][NCB];
            bf16x4 RH[NB][NCB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const f32x4 bt = *reinterpret_cast<const f32x4*>(vec + CF::F_BETA * C + 16 * b + 4 * q4);
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = bt[e] * (float)Vr[b][cb][e];
                if (b > 0) {
                  f32x4 r = zero4, r16 = zero4;  // full- and half-depth apart (see mma16)
#pragma unroll
                  for (int s = 0; 32 * s < 16 * b; ++s) {
                    if (2 * s + 1 < b) r = MM::mma(Af[b][s], cat(RH[2 * s][cb], RH[2 * s + 1][cb]), r);
                    else r16 = MM::mma16(MM::lo(Af[b][s]), RH[2 * s][cb], r16);
                  }
#pragma unroll
                  for (int e = 0; e < 4; ++e) x[e] -= r[e] + r16[e];
                }
                RU[b][cb] = MM::mma16(Tf[b], cvt4(x), zero4);
                RH[b][cb] = cvt4(RU[b][cb]);
              }
            }
            flag_wait_lds(&sFLAG[2], c);
            flag_wait_lds(&sFLAG[3], c);
            char* uu = sUU;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int cb = 0; cb < NCB; ++cb) lds_st<f32x4>(uu, ((b * NCB + cb) * 64 + lane) * 16, RU[b][cb]);
          }
        }
        lds_barrier();
      }
    };
    if (role == CF::R_X) solve_wave(IC<0>{});
    else solve_wave(IC<1>{});
  } else if (role == CF::R_S0 || role == CF::R_S1) {
    // ========================================================== state waves
    // Two waves, one per 16-column half of the tile; each carries its half
    // of the state for the whole sequence.
    const long sbase = (long)chain * DK * p.dv;
    // Accumulator block b holds M[key(b, 4q + e)][column n16 of the half]:
    // of the 32 keys of slab b >> 1, block b takes from each 8-key group g
    // the half (b ^ g) & 1, so that the transposing reads of K alternate
    // halves across lanes.  Two stacked blocks form a fragment with natural
    // key positions once lanes with odd q4 swap the blocks.
    auto key_of = [&](int b, int r) { return 32 * (b >> 1) + 8 * (r >> 2) + 4 * ((b ^ (r >> 2)) & 1) + (r & 3); };
    // Transposing reads.  K^T: rows 32 s + 16 hi + 4 q4 + (src >> 2), the
    // 8-byte piece holding keys 32 (b>>1) + 8 (src&3) + 4 ((b^src)&1) .. +3.
    int kt_base[(NKB + 1) / 2];
#pragma unroll
    for (int bh = 0; bh < (NKB + 1) / 2; ++bh) {
      const int r = 4 * q4 + (src >> 2);
      kt_base[bh] = r * KQR + 16 * ((4 * bh + (src & 3)) ^ swz_kq<GR>(r)) + 8 * (src & 1);
    }
    const int kt_flip = 8 - 16 * (src & 1);  // to the other half (odd blocks)
    // T' as a row operand (transposing read of T'^T): rows
    // 32 s + 16 hi + 4 q4 + (src >> 2), columns 16 tb + 4 (src & 3) .. +3.
    int tp_base[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const int r = 4 * q4 + (src >> 2);
      tp_base[tb] = r * CCR + 16 * ((2 * tb + ((src & 3) >> 1)) ^ swz_cc<C>(r)) + 8 * (src & 1);
    }

    auto state_wave = [&](auto hc) {
      if (GDN_PRIO_S) __builtin_amdgcn_s_setprio(GDN_PRIO_S);
      constexpr int cb = decltype(hc)::value;  // this wave's column block
      const long col = (long)tile * CF::DVT + tile_col(cb, n16);
      f32x4 Macc[NKB];
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Macc[b][e] = (p.h0 && use_h0) ? p.h0[sbase + (long)key_of(b, 4 * q4 + e) * p.dv + col] : 0.f;

      F Mf[NKS];
      const bool odd = q4 & 1;
      auto publish_state = [&]() {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const u32x4 u = __builtin_bit_cast(u32x4, MM::from_acc(Macc[2 * s], Macc[2 * s + 1]));
          Mf[s] = __builtin_bit_cast(F, u32x4{odd ? u[2] : u[0], odd ? u[3] : u[1], odd ? u[0] : u[2], odd ? u[1] : u[3]});
          lds_st<F>(sMF, ((cb * NKS + s) * 64 + lane) * 16, Mf[s]);
        }
      };
      publish_state();
      lds_barrier();

      for (int it = 0; it < NIT; ++it) {
        const int c = it - 2;
        if (c >= 0 && c < NC) {
          const char* sk = sK + (c % CF::NKR) * CF::KQ_BYTES;
          const float* vec = vec_of(c);

          // u and T' into registers first, so that the solve waves may
          // overwrite them with the next chunk's early.
          f32x4 U[NB];
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) U[tb] = lds_at<f32x4>(sUU + ((tb * NCB + cb) * 64 + lane) * 16);
          // T' (lower triangular) as row operands: slab s2 of row block tb
          // is used for 32 s2 <= 16 tb, its upper half only when
          // 16 tb > 32 s2.
          F TPf[NB][NTS];
#pragma unroll
          for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int s = 0; 32 * s <= 16 * tb; ++s) {
              const bf16x4 lo = lds_read_tr(sTP, tp_base[tb] + 32 * s * CCR);
              F f{};
              f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
              if (32 * s + 16 <= 16 * tb) {
                const bf16x4 hi = lds_read_tr(sTP, tp_base[tb] + (32 * s + 16) * CCR);
                f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
              }
              TPf[tb][s] = f;
            }

          // K^T for the update (transposing reads, tokens in pi order to
          // match the W fragments), issued early so that they arrive while
          // Y and U are formed.
          F KT[NKB][NTS];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
              const char* p0 = sk + kt_base[kb >> 1] + ((kb & 1) ? kt_flip : 0) + 32 * s * KQR;
              const bf16x4 lo = lds_read_tr(p0, 0);
              const bf16x4 hi = lds_read_tr(p0, 16 * KQR);
              KT[kb][s] = F{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
          // Y = K M, K read one row block ahead of its use.
          F Kf[2][NKS];
          auto read_k = [&](int tb) {
#pragma unroll
            for (int s = 0; s < NKS; ++s) Kf[tb & 1][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * tb);
          };
          read_k(0);
          f32x4 Y[NB];
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) {
            if (tb + 1 < NB) read_k(tb + 1);
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) y = MM::mma(Kf[tb & 1][s], Mf[s], y);
            Y[tb] = y;
          }
          flag_release(&sFLAG[2 + cb], c + 1);
          // U = u + T' Y
          F Yf[NTS];
#pragma unroll
          for (int s = 0; s < NTS; ++s) Yf[s] = MM::from_acc(Y[2 * s], Y[2 * s + 1]);
#pragma unroll
          for (int tb = 0; tb < NB; ++tb)
#pragma unroll
            for (int s = 0; 32 * s <= 16 * tb; ++s) {
              if (32 * s + 16 <= 16 * tb) {
                U[tb] = MM::mma(TPf[tb][s], Yf[s], U[tb]);
              } else {
                const f32x4 h = MM::mma16(MM::lo(TPf[tb][s]), MM::lo(Yf[s]), f32x4{0.f, 0.f, 0.f, 0.f});  // see mma16
#pragma unroll
                for (int e = 0; e < 4; ++e) U[tb][e] += h[e];
              }
            }

          // Publish U for the output waves; W = diag(w) U for the update.
          F Wf[NTS];
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(vec + CF::F_W * C + 32 * s + 4 * q4);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(vec + CF::F_W * C + 32 * s + 16 + 4 * q4);
            lds_st<F>(sUF, ((cb * NTS + s) * 64 + lane) * 16, MM::from_acc(U[2 * s], U[2 * s + 1]));
            f32x4 a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] = w0[e] * U[2 * s][e];
              b[e] = w1[e] * U[2 * s + 1][e];
            }
            Wf[s] = MM::from_acc(a, b);
          }
          flag_release(&sFLAG[cb], c + 1);

          const float gC = vec[CF::F_GAM * C + C - 1];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) Macc[kb][e] *= gC;

          // M <- Gam_C M + K^T diag(w) U
#pragma unroll
          for (int b = 0; b < NKB; ++b) {
            f32x4 m = Macc[b];
#pragma unroll
            for (int s = 0; s < NTS; ++s) m = MM::mma(KT[b][s], Wf[s], m);
            Macc[b] = m;
          }
          // The output waves have read this chunk's state: publish the next.
          flag_wait_lds(&sFLAG[4], c + 1);
          flag_wait_lds(&sFLAG[5], c + 1);
          publish_state();
        }
        lds_barrier();
      }
      if (write_hT) {
#pragma unroll
        for (int b = 0; b < NKB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) p.hT[sbase + (long)key_of(b, 4 * q4 + e) * p.dv + col] = Macc[b][e];
      }
    };
    if (role == CF::R_S0) state_wave(IC<0>{});
    else state_wave(IC<1>{});
  } else {
    // ========================================================= output waves
    auto out_wave = [&](auto oc) {
      constexpr int OW = decltype(oc)::value;
      if (GDN_PRIO_O) __builtin_amdgcn_s_setprio(GDN_PRIO_O);
      constexpr int NOWN = CF::NOWN;
      constexpr int KMAX = CF::own_tb(OW, NOWN - 1) > CF::own_tb(OW, 0) ? CF::own_tb(OW, NOWN - 1) : CF::own_tb(OW, 0);
      // Output rows: lane (token 16 tb + n16, tile columns 8 q4 .. +7).
      int o_off[NOWN];
#pragma unroll
      for (int i = 0; i < NOWN; ++i) o_off[i] = (int)((16 * CF::own_tb(OW, i) + n16) * v_stride) + 16 * q4;
      const bool odd = q4 & 1;
      // q fragments straight from HBM into registers, one step ahead of
      // use: lane (token 16 tb + n16, keys 32 s + 8 q4 .. +7).
      int q_off[NOWN];
#pragma unroll
      for (int i = 0; i < NOWN; ++i) q_off[i] = (int)((16 * CF::own_tb(OW, i) + n16) * kq_stride) + 16 * q4;
      // Issued unconditionally (a chunk past the end gets an empty
      // descriptor and reads zeros), so that the waits for the previous
      // step's loads never cover these.
      auto load_q = [&](int c, F (&Qn)[NOWN][NKS]) {
        const long row0 = rowbase + (long)c * C;
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(p.q + row0 * kq_stride + hh * DK * 2, c < NC ? (long)(len - c * C) * kq_stride : 0);
#pragma unroll
        for (int i = 0; i < NOWN; ++i)
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            Qn[i][s] = __builtin_bit_cast(F, __builtin_amdgcn_raw_buffer_load_b128(rq, q_off[i] + 64 * s, 0, 0));
      };
      // Step it (2 <= it < NC + 2): load q of chunk it-1; finish chunk it-2
      // with the q loaded one step earlier.
      auto step = [&](int it, F (&Qf)[NOWN][NKS], F (&Qn)[NOWN][NKS]) {
        load_q(it - 1, Qn);
        const int c = it - 2;
        {
          const char* sk = sK + (c % CF::NKR) * CF::KQ_BYTES;
          const float* vec = vec_of(c);
          F Mf[NKS][NCB];
#pragma unroll
          for (int s = 0; s < NKS; ++s)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) Mf[s][cb] = lds_at<F>(sMF + ((cb * NKS + s) * 64 + lane) * 16);
          flag_release(&sFLAG[4 + OW], c + 1);
          // O^T = (M^T Q^T) diag(Gam): lane (token 16 tb + n16, q4) holds
          // columns 16 cb + 4 q4 + e.
          f32x4 Oacc[NOWN][NCB];
#pragma unroll
          for (int i = 0; i < NOWN; ++i) {
            const int tb = CF::own_tb(OW, i);
            const float gcol = vec[CF::F_GAM * C + 16 * tb + n16];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < NKS; ++s) o = MM::mma(Mf[s][cb], Qf[i][s], o);
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] *= gcol;
              Oacc[i][cb] = o;
            }
          }
          // P: lane (n16, q4) of block (b1, b2) holds row i = 16 b1 + n16 and
          // columns j = 16 b2 + 4 q4 + e, which is the pi-order B operand of
          // P U for slab b2 >> 1.
          F Kf[KMAX + 1][NKS];
#pragma unroll
          for (int b = 0; b <= KMAX; ++b)
#pragma unroll
            for (int s = 0; s < NKS; ++s) Kf[b][s] = lds_at<F>(sk + kq_frag[s] + 16 * KQR * b);
          F Pf[NOWN][NTS];
#pragma unroll
          for (int i = 0; i < NOWN; ++i) {
            const int b1 = CF::own_tb(OW, i);
            const float li = vec[CF::F_LAM * C + 16 * b1 + n16];
            const float eri = vec[CF::F_ER * C + 16 * b1 + n16];
            f32x4 pb[NB];
#pragma unroll
            for (int b2 = 0; b2 <= b1; ++b2) {
              f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < NKS; ++s) pq = MM::mma(Kf[b2][s], Qf[i][s], pq);
              if (b2 < b1) {
                const f32x4 ec = *reinterpret_cast<const f32x4*>(vec + (CF::F_ER + b1) * C + 16 * b2 + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) pb[b2][e] = pq[e] * (eri * ec[e]);
              } else {
                const f32x4 lj = *reinterpret_cast<const f32x4*>(vec + CF::F_LAM * C + 16 * b1 + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) pb[b2][e] = 4 * q4 + e <= n16 ? pq[e] * exp2_fast(li - lj[e]) : 0.f;
              }
            }
#pragma unroll
            for (int s = 0; 32 * s <= 16 * b1; ++s)
              Pf[i][s] = 2 * s + 1 <= b1 ? MM::from_acc(pb[2 * s], pb[2 * s + 1]) : MM::from_acc1(pb[2 * s]);
          }

          // Finish P and diag(Gam) Q M before spinning on U.
#pragma unroll
          for (int i = 0; i < NOWN; ++i) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) settle(Oacc[i][cb]);
#pragma unroll
            for (int s = 0; 32 * s <= 16 * CF::own_tb(OW, i); ++s) settle(Pf[i][s]);
          }
          flag_wait_lds(&sFLAG[0], c + 1);
          flag_wait_lds(&sFLAG[1], c + 1);
          constexpr int NUS = (16 * KMAX + 15) / 32 + 1;  // U slabs used
          F Uf[NUS][NCB];
#pragma unroll
          for (int s = 0; s < NUS; ++s)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) Uf[s][cb] = lds_at<F>(sUF + ((cb * NTS + s) * 64 + lane) * 16);
          const long row0 = rowbase + (long)c * C;
          // a segment's halo chunks are computed but not stored (zero-size descriptor)
          const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + row0 * v_stride + (hh * p.dv + tile * CF::DVT) * 2,
                                                      c >= store_from ? (long)(len - c * C) * v_stride : 0);
#pragma unroll
          for (int i = 0; i < NOWN; ++i) {
            const int tb = CF::own_tb(OW, i);
            u32x2 ob[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              f32x4 o = Oacc[i][cb];
#pragma unroll
              for (int s = 0; 32 * s <= 16 * tb; ++s) {
                if (2 * s + 1 <= tb) {
                  o = MM::mma(Uf[s][cb], Pf[i][s], o);
                } else {
                  const f32x4 h = MM::mma16(MM::lo(Uf[s][cb]), MM::lo(Pf[i][s]), f32x4{0.f, 0.f, 0.f, 0.f});  // see mma16
#pragma unroll
                  for (int e = 0; e < 4; ++e) o[e] += h[e];
                }
              }
              ob[cb] = __builtin_bit_cast(u32x2, cvt4(o));
            }
            // Block 0 holds columns 8 q4 .. +3 for even q4, 8 q4 + 4 .. +7 for odd.
            const u32x2 lo = odd ? ob[1] : ob[0], hi = odd ? ob[0] : ob[1];
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo[0], lo[1], hi[0], hi[1]}, ro, o_off[i], 0, 0);
          }
        }
        lds_barrier();
      };
      lds_barrier();
      F Q0[NOWN][NKS], Q1[NOWN][NKS];
      if (NIT > 0) {
        lds_barrier();  // step 0
        load_q(0, Q0);
        lds_barrier();  // step 1
      }
      for (int it = 2; it < NIT; it += 2) {
        step(it, Q0, Q1);
        if (it + 1 < NIT) step(it + 1, Q1, Q0);
      }
    };
    if (role == CF::R_OA) out_wave(IC<0>{});
    else out_wave(IC<1>{});
  }
}

template <int DK, int C>
int launch16(const Params& p, int nwg, hipStream_t stream) {
  using CF = Cfg16<DK, C>;
  static_assert(CF::LDS <= 160 * 1024, "LDS budget");
  hipLaunchKernelGGL((gdn_bf16_kernel<DK, C>), dim3(nwg), dim3(64 * CF::NW), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// Workgroups of gdn_bf16_kernel<DK, C> that fit on one CU at once (LDS and
// registers), 1 when the runtime cannot tell.
template <int DK, int C>
int occupancy16() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gdn_bf16_kernel<DK, C>, 64 * Cfg16<DK, C>::NW, 0) != hipSuccess)
    return 1;
  return n > 0 ? n : 1;
}

static int occupancy_bf16(int dk, int chunk) {
  switch (dk * 1000 + chunk) {
    case 32064: return occupancy16<32, 64>();
    case 32032: return occupancy16<32, 32>();
    case 64064: return occupancy16<64, 64>();
    case 64032: return occupancy16<64, 32>();
    case 128064: return occupancy16<128, 64>();
    case 128032: return occupancy16<128, 32>();
    default: return 1;
  }
}

template <typename TI, int DK, int DVT, int C>
int launch(const Params& p, int nwg, hipStream_t stream) {
  using CF = Cfg<TI, DK, DVT, C>;
  static_assert(CF::LDS <= 160 * 1024, "LDS budget");
  hipLaunchKernelGGL((gdn_fwd_kernel<TI, DK, DVT, C>), dim3(nwg), dim3(CF::NT), 0, stream, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename TI, int DK>
int by_chunk(const Params& p, int nwg, hipStream_t s, int chunk) {
  if constexpr (sizeof(TI) == 2) {
    if (chunk == 64) return launch16<DK, 64>(p, nwg, s);
    if (chunk == 32) return launch16<DK, 32>(p, nwg, s);
  } else {
    if (chunk == 16) return launch<TI, DK, 32, 16>(p, nwg, s);
    if (chunk == 32) return launch<TI, DK, 32, 32>(p, nwg, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <typename TI>
int by_dk(const Params& p, int nwg, hipStream_t s, int dk, int chunk) {
  switch (dk) {
    case 32: return by_chunk<TI, 32>(p, nwg, s, chunk);
    case 64: return by_chunk<TI, 64>(p, nwg, s, chunk);
    case 128: return by_chunk<TI, 128>(p, nwg, s, chunk);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

}  // namespace

extern "C" {

// Host-side checks of gdn_fwd's and gdn_fwd_scan's common arguments;
// resolves chunk 0 to the dtype's default.
static int fwd_check(const void* q, const void* k, const void* v, const float* g, const float* beta,
                     const void* out, const float* hT, const int32_t* cu_seqlens, int B, int T, int H,
                     int dk, int dv, int dtype, int& chunk) {
  if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_INVALID_ARG;
  // Token tensors may be NULL only when there are no tokens; the state
  // output is required whenever there is at least one chain.
  if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_INVALID_ARG;
  if (B > 0 && !hT) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (chunk == 0) chunk = dtype == GDN_BF16 ? 64 : 16;
  if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_INVALID_ARG;
  if ((dk != 32 && dk != 64 && dk != 128) || (dv != 32 && dv != 64 && dv != 128))
    return GDN_ERR_UNSUPPORTED;
  if (dtype == GDN_BF16 && chunk == 16) return GDN_ERR_UNSUPPORTED;
  if (dtype == GDN_F32 && chunk == 64) return GDN_ERR_UNSUPPORTED;
  if (!cu_seqlens && (long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;  // token rows are 32-bit
  return GDN_OK;
}

// The full-width kernel's shapes: bf16, dk = dv = 128, 64-token chunks.
static bool full_width(int dtype, int dk, int dv, int chunk) {
  return dtype == GDN_BF16 && dk == 128 && dv == 128 && chunk == 64;
}

static gdn_launch::FullParams full_params(const void* q, const void* k, const void* v, const float* g,
                                          const float* beta, const float* h0, const int32_t* cu_seqlens,
                                          void* out, float* hT, int B, int T, int H, int seg_max) {
  gdn_launch::FullParams fp;
  fp.q = static_cast<const char*>(q);
  fp.k = static_cast<const char*>(k);
  fp.v = static_cast<const char*>(v);
  fp.g = g;
  fp.beta = beta;
  fp.h0 = h0;
  fp.cu = cu_seqlens;
  fp.out = static_cast<char*>(out);
  fp.hT = hT;
  fp.B = B;
  fp.T = T;
  fp.H = H;
  fp.seg_max = seg_max;
  fp.seg_cap = seg_max > 0 ? gdn_launch::seg_cap_for(H) : 0;
  fp.nslot = gdn_launch::full_slots(B, T, cu_seqlens != nullptr, seg_max, fp.seg_cap);
  return fp;
}

int gdn_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
            const float* h0, const int32_t* cu_seqlens, void* out, float* hT, int B, int T, int H,
            int dk, int dv, void* stream, int dtype, int chunk, int flags) {
  const int rc = fwd_check(q, k, v, g, beta, out, hT, cu_seqlens, B, T, H, dk, dv, dtype, chunk);
  if (rc != GDN_OK) return rc;
  if (flags & ~GDN_FLAG_NO_SEGMENTS) return GDN_ERR_INVALID_ARG;
  // A segment that starts at the sequence start reads h0; when hT aliases
  // h0 the last segment may already have written over it, so such calls
  // are never cut.
  const bool alias = h0 && static_cast<const void*>(h0) == static_cast<const void*>(hT);
  const bool may_cut = !(flags & GDN_FLAG_NO_SEGMENTS) && !alias;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (full_width(dtype, dk, dv, chunk))
    return gdn_launch::fwd_full(full_params(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H,
                                            may_cut ? GDN_SEG_MAX_CHUNKS : 0),
                                s);
  const int ntile = dv / 32;
  const long nwg_l = (long)B * H * ntile;
  if (nwg_l > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  if (nwg_l == 0) return GDN_OK;
  const int nwg = (int)nwg_l;
  Params p;
  p.q = static_cast<const char*>(q);
  p.k = static_cast<const char*>(k);
  p.v = static_cast<const char*>(v);
  p.g = g;
  p.beta = beta;
  p.h0 = h0;
  p.cu = cu_seqlens;
  p.out = static_cast<char*>(out);
  p.hT = hT;
  p.T = T;
  p.H = H;
  p.dv = dv;
  p.ntile = ntile;
  p.nwg = nwg;
  p.lpt = (cu_seqlens && B <= GDN_LPT_MAX && nwg % (8 * ntile) == 0) ? 1 : 0;
  // Dense bf16 batches with fewer workgroups than CUs: cut each sequence
  // into segments of at least 8 chunks, about one workgroup per CU.  Not
  // when hT aliases h0: a segment that starts at the sequence start could
  // read h0 after the last segment has written hT over it.
  p.nseg = 1;
  p.seg_chunks = 0;
  if (dtype == GDN_BF16 && !cu_seqlens && may_cut) {
    const int nchunks = (T + chunk - 1) / chunk;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
      ncu *= occupancy_bf16(dk, chunk);  // workgroup slots
    }
    if (ncu > 0 && nwg < ncu) {
      int nseg = ncu / nwg < nchunks / 8 ? ncu / nwg : nchunks / 8;
      if (nseg >= 2) {
        p.seg_chunks = (nchunks + nseg - 1) / nseg;
        p.nseg = (nchunks + p.seg_chunks - 1) / p.seg_chunks;  // every segment holds a chunk
      }
    }
  }
  const int nwg_all = nwg * p.nseg;
  p.nwg = nwg_all;
  return dtype == GDN_BF16 ? by_dk<__bf16>(p, nwg_all, s, dk, chunk) : by_dk<float>(p, nwg, s, dk, chunk);
}

int gdn_fwd_train(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* h0, const int32_t* cu_seqlens, void* out, float* hT, int B, int T, int H,
                  int dk, int dv, void* stream, int dtype, int chunk, void* workspace,
                  long long workspace_bytes) {
  const int rc = fwd_check(q, k, v, g, beta, out, hT, cu_seqlens, B, T, H, dk, dv, dtype, chunk);
  if (rc != GDN_OK) return rc;
  if (!full_width(dtype, dk, dv, chunk)) return GDN_ERR_UNSUPPORTED;
  const long long need = gdn_bwd_workspace_size(B, T, H, dk, dv, cu_seqlens != nullptr);
  if (need < 0) return (int)need;
  if (B > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15u)))
    return GDN_ERR_INVALID_ARG;
  const long ttot = cu_seqlens ? (long)T : (long)B * T;
  if (need < gdn_launch::bwd_full_ws_bytes(B, ttot, H)) return GDN_ERR_UNSUPPORTED;
  // cut as gdn_fwd cuts (not when hT aliases h0)
  const bool alias = h0 && static_cast<const void*>(h0) == static_cast<const void*>(hT);
  gdn_launch::FullParams fp =
      full_params(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, alias ? 0 : GDN_SEG_MAX_CHUNKS);
  fp.sv = static_cast<char*>(workspace);
  return gdn_launch::fwd_full_train(fp, static_cast<hipStream_t>(stream));
}

long long gdn_fwd_scan_workspace_size(int B, int T, int H, int dk, int dv, int packed, int dtype, int chunk) {
  if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_INVALID_ARG;
  if (chunk == 0) chunk = dtype == GDN_BF16 ? 64 : 16;
  // Only the full-width kernel's shapes use the scan, and only sequences of
  // more than GDN_SEG_MAX_CHUNKS chunks are cut; the slots without a
  // segment cap bound those of any device.
  if (!full_width(dtype, dk, dv, chunk) || T <= GDN_SEG_MAX_CHUNKS * 64) return 0;
  return 4 * gdn_launch::scan_ws_floats(gdn_launch::full_slots(B, T, packed != 0, GDN_SEG_MAX_CHUNKS, 0), H);
}

int gdn_fwd_scan(const void* q, const void* k, const void* v, const float* g, const float* beta,
                 const float* h0, const int32_t* cu_seqlens, void* out, float* hT, int B, int T, int H,
                 int dk, int dv, void* stream, int dtype, int chunk, void* workspace,
                 long long workspace_bytes) {
  const int rc = fwd_check(q, k, v, g, beta, out, hT, cu_seqlens, B, T, H, dk, dv, dtype, chunk);
  if (rc != GDN_OK) return rc;
  if (!full_width(dtype, dk, dv, chunk))
    return gdn_fwd(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, dk, dv, stream, dtype, chunk,
                   GDN_FLAG_NO_SEGMENTS);
  const long long need = gdn_fwd_scan_workspace_size(B, T, H, dk, dv, cu_seqlens != nullptr, dtype, chunk);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15u)))
    return GDN_ERR_INVALID_ARG;
  gdn_launch::FullParams fp =
      full_params(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, GDN_SEG_MAX_CHUNKS);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0) return gdn_launch::fwd_full(fp, s);  // nothing is cut: one workgroup per chain
  fp.ws = static_cast<float*>(workspace);
  return gdn_launch::fwd_full_scan(fp, s);
}

const char* gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "success";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape, dtype or chunk length";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_SCRATCH: return "problem larger than the no-allocation entry point's scratch buffer";
    default: return "unknown status";
  }
}

int gdn_version(void) { return 300; }

}  // extern "C"
