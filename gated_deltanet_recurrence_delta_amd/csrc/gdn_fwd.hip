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
// Work decomposition: one workgroup per (chain, 32-wide value tile).  Value
// columns never mix in the rule, so tiles are independent.  Per workgroup:
//   * "value" waves (DVT/16 of them) each own 16 state columns: they keep M
//     in MFMA accumulators for the whole sequence and run the state-
//     dependent part of every chunk (K M, X, Tinv X, O, the state update);
//   * two "prep" waves run one chunk ahead and build everything that does
//     not depend on the state: the decay vectors, Tinv (Gram matrix, 16x16
//     diagonal inverses on the VALU, block merges on the MFMA) and the
//     masked decayed Q K^T;
//   * all waves stage the next chunk's K and Q from HBM through registers
//     into a triple-buffered, XOR-swizzled LDS ring.
// One barrier per chunk.  No atomics: results are deterministic.
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

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ operand traits

template <typename TI>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int SLAB = 32;  // contraction positions per fragment
  static constexpr int E = 8;      // positions per lane group
  using frag = bf16x8;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag zero() { return frag{}; }
  // Fragment from two stacked accumulators (pi order).
  __device__ static inline frag from_acc(f32x4 lo, f32x4 hi) {
    frag r;
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
    return r;
  }
  // Fragment from one accumulator; the second half of the slab is zero.
  __device__ static inline frag from_acc1(f32x4 lo) {
    frag r{};
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    return r;
  }
};

template <>
struct Mma<float> {
  static constexpr int SLAB = 16;
  static constexpr int E = 4;
  using frag = f32x4;
  // Four K=4 steps; step j takes element j of every lane, i.e. position
  // 4q + j, so a lane's four elements are positions 4q..4q+3.
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
  __device__ static inline frag zero() { return frag{}; }
  __device__ static inline frag from_acc(f32x4 lo, f32x4) { return lo; }
  __device__ static inline frag from_acc1(f32x4 lo) { return lo; }
};

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

template <typename V>
__device__ static inline V lds_ld(const char* base, int off) {
  return *reinterpret_cast<const V*>(base + off);
}
template <typename V>
__device__ static inline void lds_st(char* base, int off, V v) {
  *reinterpret_cast<V*>(base + off) = v;
}

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
  static constexpr int NW = NDV + 2;      // + two prep waves
  static constexpr int NT = 64 * NW;
  static_assert(C % SLAB == 0 && DK % SLAB == 0 && DVT % 16 == 0, "shape");
  static_assert(NB <= 4, "chunk of at most 64 tokens");

  static constexpr int KQ_BYTES = C * DK * S;
  static constexpr int CC_BYTES = C * C * S;
  static constexpr int VEC_BYTES = 3 * C * 4;  // beta, Gam, w
  static constexpr int AD_STRIDE = 260;        // floats per padded 16x16 block
  static constexpr int OFF_K = 0;                           // [3] K chunks
  static constexpr int OFF_Q = OFF_K + 3 * KQ_BYTES;        // [3] Q chunks
  static constexpr int OFF_T = OFF_Q + 3 * KQ_BYTES;        // [2] Tinv
  static constexpr int OFF_P = OFF_T + 2 * CC_BYTES;        // [2] masked decayed Q K^T
  static constexpr int OFF_VEC = OFF_P + 2 * CC_BYTES;      // [2] per-token vectors
  static constexpr int OFF_A = OFF_VEC + 2 * VEC_BYTES;     // A, off-diagonal blocks
  static constexpr int OFF_TT = OFF_A + CC_BYTES;           // Tinv^T
  static constexpr int OFF_AD = OFF_TT + CC_BYTES;          // A diagonal blocks, fp32
  static constexpr int LDS = OFF_AD + NB * AD_STRIDE * 4;

  // Staging of one K or Q chunk: 16-byte granules per thread.
  static constexpr int GRK = DK * S / 16;   // granules per token row
  static constexpr int NG = C * GRK;
  static constexpr int NPT = (NG + NT - 1) / NT;
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
};

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give
// each XCD a contiguous range of work items so that the value tiles of one
// chain, which re-read the same q/k, share that XCD's L2.
__device__ static inline int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int q = n >> 3, r = n & 7;
  return xcd * q + (xcd < r ? xcd : r) + slot;
}

template <typename TI, int DK, int DVT, int C>
__global__ __launch_bounds__(64 * (DVT / 16 + 2), 1) void gdn_fwd_kernel(const Params p) {
  using CF = Cfg<TI, DK, DVT, C>;
  using MM = Mma<TI>;
  using F = typename MM::frag;
  using SK = Swz<TI, DK>;
  constexpr int SLAB = CF::SLAB, E = CF::E, BPS = CF::BPS;
  constexpr int NB = CF::NB, NTS = CF::NTS, NKB = CF::NKB, NKS = CF::NKS, NDV = CF::NDV;

  __shared__ __attribute__((aligned(16))) char smem[CF::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const long kq_stride = (long)H * DK * CF::S;  // bytes between tokens in q/k
  const char* qbase = p.q + hh * (long)DK * CF::S;
  const char* kbase = p.k + hh * (long)DK * CF::S;

  // ---------------------------------------------------- K/Q staging
  uint4 stK[CF::NPT], stQ[CF::NPT];
  auto stage_load = [&](int c) {
#pragma unroll
    for (int i = 0; i < CF::NPT; ++i) {
      const int gi = tid + CF::NT * i;
      if (CF::NG % CF::NT == 0 || gi < CF::NG) {
        const int row = gi / CF::GRK, gc = gi % CF::GRK;
        int t = c * C + row;
        t = t < len ? t : len - 1;
        const long off = (rowbase + t) * kq_stride + gc * 16;
        stK[i] = *reinterpret_cast<const uint4*>(kbase + off);
        stQ[i] = *reinterpret_cast<const uint4*>(qbase + off);
      }
    }
  };
  auto stage_store = [&](int c) {
    char* sk = smem + CF::OFF_K + (c % 3) * CF::KQ_BYTES;
    char* sq = smem + CF::OFF_Q + (c % 3) * CF::KQ_BYTES;
#pragma unroll
    for (int i = 0; i < CF::NPT; ++i) {
      const int gi = tid + CF::NT * i;
      if (CF::NG % CF::NT == 0 || gi < CF::NG) {
        const int row = gi / CF::GRK, gc = gi % CF::GRK;
        lds_st<uint4>(sk, SK::goff(row, gc), stK[i]);
        lds_st<uint4>(sq, SK::goff(row, gc), stQ[i]);
      }
    }
  };

  if (NC > 0) {
    stage_load(0);
    stage_store(0);
  }
  __syncthreads();

  if (wave < NDV) {
    // =========================================================== value wave
    const int dvcol = tile * DVT + wave * 16 + n16;  // this lane's state column
    const long sbase = (long)chain * DK * p.dv;      // h0/hT slab of this chain
    // Accumulator block b, element e holds M[key(b, 4q+e)][dvcol].
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
    const char* vbase = p.v + ((long)hh * p.dv + dvcol) * CF::S;
    const long v_stride = (long)H * p.dv * CF::S;
    float Vr[NB][4];
    auto load_v = [&](int c) {
#pragma unroll
      for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int t = c * C + 16 * tb + 4 * q4 + e;
          t = t < len ? t : len - 1;
          Vr[tb][e] = to_f(*reinterpret_cast<const TI*>(vbase + (rowbase + t) * v_stride));
        }
    };
    if (NC > 0) load_v(0);

    for (int it = 0; it <= NC; ++it) {
      if (it + 1 < NC) stage_load(it + 1);
      if (it >= 1) {
        const int c = it - 1;
        const char* sk = smem + CF::OFF_K + (c % 3) * CF::KQ_BYTES;
        const char* sq = smem + CF::OFF_Q + (c % 3) * CF::KQ_BYTES;
        const char* st = smem + CF::OFF_T + (c & 1) * CF::CC_BYTES;
        const char* sp = smem + CF::OFF_P + (c & 1) * CF::CC_BYTES;
        const float* vec = reinterpret_cast<const float*>(smem + CF::OFF_VEC + (c & 1) * CF::VEC_BYTES);

        // State as MFMA fragments (key positions in natural order).
        F Mf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) Mf[s] = acc_frag<TI>(Macc, s);

        // Y = K M ; X = beta (V - Gam Y)
        f32x4 X[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            y = MM::mma(frag_nat<TI, DK>(sk, 16 * tb + n16, s * SLAB, q4), Mf[s], y);
          const f32x4 bt = *reinterpret_cast<const f32x4*>(vec + 16 * tb + 4 * q4);
          const f32x4 gm = *reinterpret_cast<const f32x4*>(vec + C + 16 * tb + 4 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) X[tb][e] = bt[e] * (Vr[tb][e] - gm[e] * y[e]);
        }
        if (c + 1 < NC) load_v(c + 1);
        F Xf[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) Xf[s] = acc_frag<TI>(X, s);

        // U = Tinv X  (Tinv is lower triangular: slabs up to the diagonal)
        f32x4 U[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s <= (16 * tb + 15) / SLAB; ++s)
            u = MM::mma(frag_pi<TI, C>(st, 16 * tb + n16, s * SLAB, q4), Xf[s], u);
          U[tb] = u;
        }
        F Uf[NTS], Wf[NTS];
        {
          f32x4 WU[NB];
#pragma unroll
          for (int tb = 0; tb < NB; ++tb) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(vec + 2 * C + 16 * tb + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) WU[tb][e] = wv[e] * U[tb][e];
          }
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            Uf[s] = acc_frag<TI>(U, s);
            Wf[s] = acc_frag<TI>(WU, s);
          }
        }

        // O^T = (M^T Q^T) diag(Gam) + U^T P^T, one 16-token block at a time.
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            o = MM::mma(Mf[s], frag_nat<TI, DK>(sq, 16 * tb + n16, s * SLAB, q4), o);
          const float gcol = vec[C + 16 * tb + n16];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] *= gcol;
#pragma unroll
          for (int s = 0; s <= (16 * tb + 15) / SLAB; ++s)
            o = MM::mma(Uf[s], frag_pi<TI, C>(sp, 16 * tb + n16, s * SLAB, q4), o);
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

        // M <- Gam_C M + K^T diag(w) U
        const float gC = vec[C + C - 1];
#pragma unroll
        for (int b = 0; b < NKB; ++b) {
          f32x4 m = Macc[b];
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] *= gC;
          const int key = key_of(b, n16);
#pragma unroll
          for (int s = 0; s < NTS; ++s) {
            F a;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              int tok;
              if constexpr (BPS == 2) {
                tok = s * 32 + 16 * (e >> 2) + 4 * q4 + (e & 3);
              } else {
                tok = s * 16 + 4 * q4 + e;
              }
              a[e] = lds_ld<TI>(sk, SK::off(tok, key));
            }
            m = MM::mma(a, Wf[s], m);
          }
          Macc[b] = m;
        }
      }
      if (it + 1 < NC) stage_store(it + 1);
      __syncthreads();
    }

#pragma unroll
    for (int b = 0; b < NKB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.hT[sbase + (long)key_of(b, 4 * q4 + e) * p.dv + dvcol] = Macc[b][e];
  } else {
    // ============================================================ prep waves
    const bool p0 = wave == NDV;
    float gv = 0.f, bv = 0.f;
    auto load_gb = [&](int c) {
      gv = 0.f;
      bv = 0.f;
      const int t = c * C + lane;
      if (lane < C && t < len) {
        const long idx = (rowbase + t) * H + hh;
        gv = p.g[idx];
        bv = p.beta[idx];
      }
    };
    if (NC > 0) load_gb(0);

    for (int it = 0; it <= NC; ++it) {
      if (it + 1 < NC) stage_load(it + 1);
      if (it < NC) {
        const int c = it;
        const char* sk = smem + CF::OFF_K + (c % 3) * CF::KQ_BYTES;
        const char* sq = smem + CF::OFF_Q + (c % 3) * CF::KQ_BYTES;
        char* st = smem + CF::OFF_T + (c & 1) * CF::CC_BYTES;
        char* sp = smem + CF::OFF_P + (c & 1) * CF::CC_BYTES;
        float* vec = reinterpret_cast<float*>(smem + CF::OFF_VEC + (c & 1) * CF::VEC_BYTES);

        // In-chunk cumulative log-decay (inclusive scan over the lanes).
        float gam = gv;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float y = __shfl_up(gam, d, 64);
          if (lane >= d) gam += y;
        }
        const float bet = bv;
        if (c + 1 < NC) load_gb(c + 1);

        // Per-lane decay of the 16-token block rows (i = 16*bi + n16) and
        // of the accumulator rows (j = 16*bj + 4*q4 + e).
        float gi[NB], bi_[NB], gj[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          gi[b] = __shfl(gam, 16 * b + n16, 64);
          bi_[b] = __shfl(bet, 16 * b + n16, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) gj[b][e] = __shfl(gam, 16 * b + 4 * q4 + e, 64);
        }

        F Kf[NB][NKS];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int s = 0; s < NKS; ++s) Kf[b][s] = frag_nat<TI, DK>(sk, 16 * b + n16, s * SLAB, q4);

        if (!p0) {
          // ---- prep wave 1: per-token vectors and P = masked decayed Q K^T
          const float gC = __shfl(gam, C - 1, 64);
          if (lane < C) {
            vec[lane] = bet;
            vec[C + lane] = __expf(gam);
            vec[2 * C + lane] = __expf(gC - gam);
          }
#pragma unroll
          for (int b1 = 0; b1 < NB; ++b1) {  // row block of P (token i)
            F Qf[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) Qf[s] = frag_nat<TI, DK>(sq, 16 * b1 + n16, s * SLAB, q4);
#pragma unroll
            for (int b2 = 0; b2 <= b1; ++b2) {  // column block (token j)
              f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < NKS; ++s) a = MM::mma(Kf[b2][s], Qf[s], a);
              // a[e] = (Q K^T)[i = 16 b1 + n16][j = 16 b2 + 4 q4 + e]
              f32x4 r;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool keep = (16 * b2 + 4 * q4 + e) <= (16 * b1 + n16);
                const float d = keep ? gi[b1] - gj[b2][e] : 0.f;
                r[e] = keep ? a[e] * __expf(d) : 0.f;
              }
              st4<TI, C>(sp, 16 * b1 + n16, 16 * b2 + 4 * q4, r);
            }
            if (BPS == 2 && (b1 & 1) == 0 && b1 + 1 < NB)
              st4<TI, C>(sp, 16 * b1 + n16, 16 * (b1 + 1) + 4 * q4, f32x4{0.f, 0.f, 0.f, 0.f});
          }
        } else {
          // ---- prep wave 0: A, then Tinv = (I + A)^{-1}
          char* sa = smem + CF::OFF_A;
          char* stt = smem + CF::OFF_TT;
          float* sad = reinterpret_cast<float*>(smem + CF::OFF_AD);
#pragma unroll
          for (int b1 = 0; b1 < NB; ++b1) {
#pragma unroll
            for (int b2 = 0; b2 <= b1; ++b2) {
              f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s < NKS; ++s) a = MM::mma(Kf[b2][s], Kf[b1][s], a);
              // a[e] = (K K^T)[i = 16 b1 + n16][j = 16 b2 + 4 q4 + e]
              f32x4 r;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool keep = (16 * b2 + 4 * q4 + e) < (16 * b1 + n16);
                const float d = keep ? gi[b1] - gj[b2][e] : 0.f;
                r[e] = keep ? bi_[b1] * a[e] * __expf(d) : 0.f;
              }
              if (b2 == b1) {
                *reinterpret_cast<f32x4*>(sad + b1 * CF::AD_STRIDE + 16 * n16 + 4 * q4) = r;
              } else {
                st4<TI, C>(sa, 16 * b1 + n16, 16 * b2 + 4 * q4, r);
              }
            }
          }

          // Diagonal 16x16 blocks: forward substitution on the VALU in fp32.
          // Lane (block q4, column n16) computes column n16 of the inverse.
          if (q4 < NB) {
            const float* ad = sad + q4 * CF::AD_STRIDE;
            float tc[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float s = (i == n16) ? 1.f : 0.f;
#pragma unroll
              for (int l4 = 0; l4 < i; l4 += 4) {
                const f32x4 arow = *reinterpret_cast<const f32x4*>(ad + 16 * i + l4);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  if (l4 + u < i) s -= arow[u] * tc[l4 + u];
              }
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

          // Off-diagonal blocks: Tinv_ij = -Tinv_ii * sum_{j<=l<i} A_il Tinv_lj.
#pragma unroll
          for (int i = 1; i < NB; ++i) {
#pragma unroll
            for (int j = 0; j < i; ++j) {
              const int L = 16 * (i - j);
              f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int s = 0; s * SLAB < L; ++s) {
                const bool valid = s * SLAB + E * q4 < L;
                const F fa = valid ? frag_nat<TI, C>(sa, 16 * i + n16, 16 * j + s * SLAB, q4) : MM::zero();
                const F fb = valid ? frag_nat<TI, C>(stt, 16 * j + n16, 16 * j + s * SLAB, q4) : MM::zero();
                r = MM::mma(fa, fb, r);
              }
              // r[e] = R[row 16 i + 4 q4 + e][col 16 j + n16]
              f32x4 o = MM::mma(frag_pi1<TI, C>(st, 16 * i + n16, 16 * i, q4), MM::from_acc1(r),
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
      }
      if (it + 1 < NC) stage_store(it + 1);
      __syncthreads();
    }
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
    if (chunk == 64) return launch<TI, DK, 32, 64>(p, nwg, s);
    if (chunk == 32) return launch<TI, DK, 32, 32>(p, nwg, s);
  } else {
    if (chunk == 16) return launch<TI, DK, 32, 16>(p, nwg, s);
    if (chunk == 32) return launch<TI, DK, 32, 32>(p, nwg, s);
    if constexpr (DK == 32) {
      if (chunk == 64) return launch<TI, DK, 32, 64>(p, nwg, s);
    }
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

int gdn_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
            const float* h0, const int32_t* cu_seqlens, void* out, float* hT, int B, int T, int H,
            int dk, int dv, void* stream, int dtype, int chunk) {
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
  if (dtype == GDN_F32 && chunk == 64 && dk != 32) return GDN_ERR_UNSUPPORTED;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == GDN_BF16 ? by_dk<__bf16>(p, nwg, s, dk, chunk) : by_dk<float>(p, nwg, s, dk, chunk);
}

const char* gdn_strerror(int status) {
  switch (status) {
    case GDN_OK: return "success";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape, dtype or chunk length";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int gdn_version(void) { return 100; }

}  // extern "C"
