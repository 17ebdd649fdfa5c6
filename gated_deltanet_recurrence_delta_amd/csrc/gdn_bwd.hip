// Backward pass of the gated delta rule, chunkwise, for gfx950.
//
// The forward rule, per chain, with the state kept as M = S^T (dk x dv) and
// alpha_t = exp(g_t) (HyMo "Model Architecture Walkthrough", sections 5.2.1
// and 5.2.2):
//
//   u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t),
//   M_t = alpha_t M_{t-1} + k_t u_t^T,      o_t = M_t^T q_t.
//
// The pages train through this layer with a backward pass that recomputes
// what it needs from the saved inputs ("Optimization Quartet", sections
// 3.3-3.4; the walkthrough's section 6.5).  Here the gradients of
// <do, out> + <dhT, hT> are formed chunk by chunk.  For a chunk of C tokens
// with entry state M, exit state M', in-chunk cumulative log-decay gamma,
// Gam = exp(gamma), w_i = exp(gamma_C - gamma_i), E_ij = exp(gamma_i - gamma_j):
//
//   A   = strict_lower(diag(beta) (K K^T) . E),   T = (I + A)^-1
//   X   = diag(beta) (V - diag(Gam) K M),         U = T X
//   P   = lower(Q K^T . E)
//   O   = diag(Gam) Q M + P U,                    M' = Gam_C M + K^T diag(w) U
//
// Reverse mode through these, given dO and dM' (the gradient reaching the
// chunk's exit state):
//
//   dU = P^T dO + diag(w) K dM',   dX = T^T dU,
//   dM = Gam_C dM' + Q^T diag(Gam) dO - K^T diag(beta Gam) dX
//
// which runs backwards over the chunks (the state's adjoint), and per chunk
//
//   dV = diag(beta) dX,  dA = -strict_lower(dX U^T),  dP = lower(dO U^T),
//   dQ = diag(Gam) dO M^T + (dP . E) K,
//   dK = -diag(beta Gam) dX M^T + G K + G^T K + (dP . E)^T Q + diag(w) U dM'^T,
//        with G = dA . E . beta_i,
//   dbeta_i = sum_j dX_ij (V - Gam K M)_ij + sum_j dA_ij (K K^T . E)_ij,
//   dgamma  = rowsum(Z) - colsum(Z) + dGam . Gam - dw . w  (+ sum(dw . w) at
//             the chunk's last token), Z = strict_lower(dA . A + dP . P),
//   dGam_i  = -beta_i sum_j dX_ij (K M)_ij + sum_j dO_ij (Q M)_ij
//             (+ <M, dM'> at the last token),  dw_i = sum_j U_ij (K dM')_ij,
//   dg      = reverse cumulative sum of dgamma within the chunk, the w terms
//             summed as sum_{u < t} dw_u w_u (what they add up to).
//
// Four kernels, all in fp32, their products on the fp32 matrix cores (bf16
// storage is widened on load, the token gradients rounded to nearest even on
// store):
//   prep     (chunk, head), parallel:  T and P of every chunk (T by 16 x 16
//            blocks: two diagonal substitutions, then the off-diagonal block);
//   states   (chain, 16-column tile), serial over chunks: the state at every
//            chunk's entry, from h0;
//   adjoint  (chain, 16-column tile), serial over chunks in reverse: the
//            gradient reaching every chunk's exit state, from dhT; dh0;
//   grad     (chunk, head), parallel: dq, dk, dv, dg, dbeta of the chunk from
//            its entry state and exit gradient, all value columns.
// T, P, the entry states and the exit gradients live in a caller-supplied
// workspace, one slot per (head, chunk).  Chunks restart at every sequence
// start; chunk c of sequence n (its tokens start at offset s_n) takes slot
// floor(s_n / C) + n + c, which is distinct for distinct (n, c) and below
// floor(total tokens / C) + B + 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

constexpr int BC = 32;  // tokens per chunk
constexpr int TW = 16;  // value columns per tile
constexpr int NT = 256; // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;

struct BShape {
  int B, T, H, dv;      // T: tokens per sequence (dense) or in total (packed)
  int nslots;           // chunk slots per head
  int ntile;            // dv / TW
  int nseg, seg_chunks; // the two serial sweeps: segments per sequence, chunks per segment
};

// Sequence segments of the two serial sweeps.  A dense batch with fewer
// (chain, tile) workgroups than two per CU runs each sequence as nseg
// segments, one workgroup per (chain, segment, tile).  A token's transition
// M -> alpha (I - beta k k^T) M has spectral norm alpha max(1, |1 - beta |k|^2|),
// and the state gradient goes back through the same (symmetric) map.  So the
// states sweep of a segment starts from a zero state at the latest chunk
// boundary behind the segment where the product of those norms is below
// e^-HALO_NATS (or from h0 at the sequence start).  The adjoint sweep starts
// from a zero gradient at the earliest chunk boundary after the segment where
// the product over the chunks in between is below that bound (or from dhT at
// the sequence end).  Either way the result differs from the unsegmented one
// by less than that factor beyond rounding.  The halo chunks are computed but
// not stored.
constexpr float HALO_NATS = 40.f;

__device__ inline float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ inline void seq_info(const int32_t* __restrict__ cu, const BShape& p, int n, long& row0, int& len) {
  if (cu) {
    row0 = cu[n];
    len = cu[n + 1] - cu[n];
  } else {
    row0 = (long)n * p.T;
    len = p.T;
  }
}

__device__ inline int slot_key(const int32_t* __restrict__ cu, const BShape& p, int n) {
  const long start = cu ? (long)cu[n] : (long)n * p.T;
  return (int)(start / BC) + n;
}

// The sequence that owns slot s: the largest n with slot_key(n) <= s.
__device__ inline int find_seq(const int32_t* __restrict__ cu, const BShape& p, int s) {
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_key(cu, p, mid) <= s)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// In-chunk cumulative log-decay: gv is token tid's g (0 past the chunk's
// length and for tid >= C); wave 0 forms the inclusive prefix sum with a
// fixed shuffle tree and writes gam.  Every kernel forms gam with this scan.
__device__ inline float chunk_scan(float gv, int tid) {
  float x = gv;
#pragma unroll
  for (int off = 1; off < BC; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (tid >= off) x += y;
  }
  return x;
}

__device__ inline void chunk_gamma(float gv, int tid, float* gam) {
  if (tid < 64) {
    const float x = chunk_scan(gv, tid);
    if (tid < BC) gam[tid] = x;
  }
}

__device__ inline float token_f(const float* __restrict__ x, long row0, int t0, int Lc, int H, int h, int tid) {
  return tid < Lc ? x[(row0 + t0 + tid) * H + h] : 0.f;
}

// Log of the product of the per-token transition-norm bounds over chunk c
// (log alpha + log max(1, |1 - beta |k|^2|) summed over its tokens), formed by
// one wave (every lane returns it).
template <typename TI, int DK>
__device__ inline float chunk_log_norm(const TI* __restrict__ k, const float* __restrict__ g,
                                       const float* __restrict__ beta, long row0, int len, int H, int h, int c,
                                       int lane) {
  const int t0 = c * BC, Lc = min(BC, len - t0);
  float e = 0.f;
  if (lane < Lc) {
    const long th = (row0 + t0 + lane) * H + h;
    const TI* kr = k + th * DK;
    float n2 = 0.f;
#pragma unroll 8
    for (int i = 0; i < DK; ++i) {
      const float x = (float)kr[i];
      n2 = __builtin_fmaf(x, x, n2);
    }
    const float f = fabsf(1.f - beta[th] * n2);
    e = g[th] + (f > 1.f ? __logf(f) : 0.f);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) e += __shfl_xor(e, d, 64);
  return e;
}

// A chunk's C rows of a (token, head, W) tensor (columns col0 .. col0+W-1 of
// rows of length ld), held in registers between a fetch and an LDS store;
// rows past the chunk's length are zero.  bf16 elements travel in pairs
// (one 32-bit load each).  Every load address is clamped into the chunk
// (Lc >= 1), so the fetch has no branches.
template <typename TI, int W>
struct RowsReg {
  static constexpr int PK = sizeof(TI) == 2 ? 2 : 1;  // elements per register
  static constexpr int N = BC * W / (NT * PK);
  uint32_t r[N];
  __device__ void fetch(const TI* __restrict__ p, long row0, int t0, int Lc, int H, int h, long ld, int col0,
                        int tid) {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int e = PK * (tid + NT * x), t = e / W, i = e % W;
      const long off = ((row0 + t0 + min(t, Lc - 1)) * H + h) * ld + col0 + i;
      uint32_t w;
      if constexpr (PK == 2)
        w = *reinterpret_cast<const uint32_t*>(p + off);
      else
        w = __float_as_uint(p[off]);
      r[x] = t < Lc ? w : 0u;
    }
  }
  template <int S>
  __device__ void store_s(float (*dst)[S], int tid) const {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int e = PK * (tid + NT * x), t = e / W, i = e % W;
      if constexpr (PK == 2) {
        dst[t][i] = __uint_as_float(r[x] << 16);
        dst[t][i + 1] = __uint_as_float(r[x] & 0xffff0000u);
      } else {
        dst[t][i] = __uint_as_float(r[x]);
      }
    }
  }
};

// One chunk's C x C matrix from the workspace, in registers.
struct CCReg {
  static constexpr int N = BC * BC / NT;
  float r[N];
  __device__ void fetch(const float* __restrict__ p, int tid) {
#pragma unroll
    for (int x = 0; x < N; ++x) r[x] = p[tid + NT * x];
  }
  template <int S>
  __device__ void store_s(float (*dst)[S], int tid) const {
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int e = tid + NT * x;
      dst[e / BC][e % BC] = r[x];
    }
  }
};

// ------------------------------------------------------- matrix cores ----
// The products run on the fp32 matrix cores: v_mfma_f32_16x16x4f32 takes
// A (16 x 4) and B (4 x 16) one element per lane -- lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16] -- and accumulates D (16 x 16), of which lane l holds
// rows 4 (l / 16) .. 4 (l / 16) + 3 of column l % 16.  LDS rows are padded to
// a stride of 8 mod 64 words, which keeps both operand read patterns (down a
// column, along a row) within two-way bank conflicts.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc + sum over the contraction of A B, in steps of four (the lane's
// element of step kk is a(kk), b(kk)).  The operands of G steps are read
// before their products are issued, so the LDS reads overlap the
// matrix-core work instead of waiting in front of every product.
template <int K, class FA, class FB>
__device__ inline f32x4 mfma_chain(f32x4 acc, FA a, FB b) {
  constexpr int G = K / 4 < 8 ? K / 4 : 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4 * G) {
    float av[G], bv[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      av[j] = a(k0 + 4 * j);
      bv[j] = b(k0 + 4 * j);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) acc = mfma4(av[j], bv[j], acc);
  }
  return acc;
}

constexpr int SC = BC + 8;  // row stride of the C x C arrays
constexpr int ST = TW + 8;  // row stride of the tile arrays

// A plain owner mapping of a DK x TW tile: thread -> row si, columns
// sj0 .. sj0 + JP - 1.
template <int DK>
struct Owner {
  static constexpr int JP = DK * TW / NT;
  int si, sj0;
  __device__ Owner(int tid) : si(tid % DK), sj0((tid / DK) * JP) {}
};

// ---------------------------------------------------------------- prep ----
template <typename TI, int DK>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                                                      const float* __restrict__ g, const float* __restrict__ beta,
                                                      const int32_t* __restrict__ cu, float* __restrict__ wsT,
                                                      float* __restrict__ wsP, const BShape p) {
  constexpr int SK = DK + 8;
  __shared__ TI qs[BC][SK], ks[BC][SK];  // stored as given (bf16 is widened on read)
  __shared__ float As[BC][SC], Ts[BC][SC];
  __shared__ float gam[BC], bet[BC];
  const int tid = threadIdx.x, s = blockIdx.x, h = blockIdx.y, H = p.H;
  const int n = find_seq(cu, p, s);
  long row0;
  int len;
  seq_info(cu, p, n, row0, len);
  const int c = s - slot_key(cu, p, n);
  if (c < 0 || (long)c * BC >= len) return;  // slot not used
  const int t0 = c * BC, Lc = min(BC, len - t0);
  for (int e = tid; e < BC * DK; e += NT) {
    const int t = e / DK, i = e % DK;
    const long off = ((row0 + t0 + t) * H + h) * DK + i;
    qs[t][i] = t < Lc ? q[off] : (TI)0.f;
    ks[t][i] = t < Lc ? k[off] : (TI)0.f;
  }
  if (tid < BC) bet[tid] = token_f(beta, row0, t0, Lc, H, h, tid);
  chunk_gamma(tid < BC ? token_f(g, row0, t0, Lc, H, h, tid) : 0.f, tid, gam);
  __syncthreads();
  const size_t base = ((size_t)h * p.nslots + s) * (BC * BC);
  {  // K K^T and Q K^T on block `wave` of the C x C outputs
    const int wave = tid >> 6, ln = tid & 15, lq = (tid >> 4) & 3;
    const int tr0 = 16 * (wave >> 1), uc = 16 * (wave & 1) + ln;
    f32x4 kk4 = {0.f, 0.f, 0.f, 0.f}, qk4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK; kk += 4) {
      const float b = (float)ks[uc][kk + lq];
      kk4 = mfma4((float)ks[tr0 + ln][kk + lq], b, kk4);
      qk4 = mfma4((float)qs[tr0 + ln][kk + lq], b, qk4);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = tr0 + 4 * lq + x;
      const float E = uc <= t ? ex(gam[t] - gam[uc]) : 0.f;
      As[t][uc] = uc < t ? bet[t] * kk4[x] * E : 0.f;
      wsP[base + t * BC + uc] = qk4[x] * E;
    }
  }
  __syncthreads();
  // (I + A)^-1 in 16 x 16 blocks: the two diagonal blocks by forward
  // substitution (one column per thread), then T21 = -T22 (A21 T11).  The
  // upper-right block of As, zero in A, holds A21 T11.
  constexpr int HB = BC / 2;
  if (tid < BC) {
    const int o = HB * (tid / HB), u = tid % HB;
    for (int t = 0; t < HB; ++t) {
      float x = t == u ? 1.f : 0.f;
      for (int r = u; r < t; ++r) x = __builtin_fmaf(-As[o + t][o + r], Ts[o + r][o + u], x);
      Ts[o + t][o + u] = x;
      Ts[t][HB + u] = 0.f;  // upper-right block of T
    }
  }
  __syncthreads();
  {
    const int i = tid / HB, j = tid % HB;  // NT = HB * HB
    float x = 0.f;
    for (int r = j; r < HB; ++r) x = __builtin_fmaf(As[HB + i][r], Ts[r][j], x);
    As[i][HB + j] = x;
  }
  __syncthreads();
  {
    const int i = tid / HB, j = tid % HB;
    float x = 0.f;
    for (int r = 0; r <= i; ++r) x = __builtin_fmaf(Ts[HB + i][HB + r], As[r][HB + j], x);
    Ts[HB + i][j] = -x;
  }
  __syncthreads();
  for (int e = tid; e < BC * BC; e += NT) wsT[base + e] = Ts[e / BC][e % BC];
}

// -------------------------------------------------------------- states ----
// The state tile M (DK x 16) is held in matrix-core accumulator layout:
// 16-row block b of it belongs to wave b mod 4, lane l holding rows
// 16 b + 4 (l / 16) .. + 3 of column l % 16.
template <int DK>
struct StateBlocks {
  static constexpr int NBM = DK / 16;            // 16-row blocks of the tile
  static constexpr int PER = (NBM + 3) / 4;      // blocks per wave (some waves may own fewer)
};

// Wave 0 forms the chunk's cumulative log-decay gam (as chunk_gamma), and
// from it Gam_t = exp(gam_t) and w_t = exp(gam_{C-1} - gam_t).
__device__ inline void chunk_decay(float gv, int tid, float* gam, float* Gam, float* wv) {
  if (tid < 64) {
    const float x = chunk_scan(gv, tid);
    const float last = __shfl(x, BC - 1, 64);
    if (tid < BC) {
      gam[tid] = x;
      Gam[tid] = ex(x);
      wv[tid] = ex(last - x);
    }
  }
}

template <typename TI, int DK>
__global__ __launch_bounds__(NT, 2) void bwd_states_kernel(const TI* __restrict__ k, const TI* __restrict__ v,
                                                           const float* __restrict__ g,
                                                           const float* __restrict__ beta,
                                                           const float* __restrict__ h0,
                                                           const int32_t* __restrict__ cu,
                                                           const float* __restrict__ wsT,
                                                           float* __restrict__ wsM, const BShape p) {
  using SBk = StateBlocks<DK>;
  constexpr int SK = DK + 8;
  __shared__ float ks[BC][SK], vs[BC][ST], Ts[BC][SC], Xs[BC][ST], Ws[BC][ST], Ms[DK][ST];
  __shared__ float gam[BC], Gam[BC], wv[BC], bet[BC];
  const int tid = threadIdx.x, H = p.H, dv = p.dv;
  const int chain = blockIdx.x / (p.ntile * p.nseg), seg = (blockIdx.x / p.ntile) % p.nseg;
  const int tile = blockIdx.x % p.ntile;
  const int n = chain / H, h = chain % H, col0 = tile * TW;
  long row0;
  int len;
  seq_info(cu, p, n, row0, len);
  const int key = slot_key(cu, p, n), nch = (len + BC - 1) / BC;
  const int wave = tid >> 6, ln = tid & 15, lq = (tid >> 4) & 3;
  // chunks [c0, c1) are stored; the sweep starts at cs <= c0 (see HALO_NATS)
  int c0 = 0, c1 = nch, cs = 0;
  if (p.nseg > 1) {
    __shared__ int sStart;
    c0 = min(seg * p.seg_chunks, nch);
    c1 = min(c0 + p.seg_chunks, nch);
    if (wave == 0) {
      int cc = c0;
      float acc = 0.f;  // log of the norm product over chunks [cc, c0)
      while (cc > 0 && acc > -HALO_NATS) {
        --cc;
        acc += chunk_log_norm<TI, DK>(k, g, beta, row0, len, H, h, cc, tid);
      }
      if (tid == 0) sStart = cc;
    }
    __syncthreads();
    cs = sStart;
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 M[SBk::PER];
#pragma unroll
  for (int m = 0; m < SBk::PER; ++m) {
    const int blk = wave + 4 * m;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      M[m][x] = (h0 && cs == 0 && blk < SBk::NBM)
                    ? h0[((long)chain * DK + 16 * blk + 4 * lq + x) * dv + col0 + ln]
                    : 0.f;
  }

  // the next chunk's inputs, fetched into registers while this one computes
  RowsReg<TI, DK> kr;
  RowsReg<TI, TW> vr;
  CCReg tr;
  float gr = 0.f, br = 0.f;
  auto fetch = [&](int c) {
    const int t0 = c * BC, Lc = min(BC, len - t0);
    kr.fetch(k, row0, t0, Lc, H, h, DK, 0, tid);
    vr.fetch(v, row0, t0, Lc, H, h, dv, col0, tid);
    tr.fetch(wsT + ((size_t)h * p.nslots + key + c) * (BC * BC), tid);
    if (tid < BC) {
      gr = token_f(g, row0, t0, Lc, H, h, tid);
      br = token_f(beta, row0, t0, Lc, H, h, tid);
    }
  };
  if (cs < c1) fetch(cs);

  for (int c = cs; c < c1; ++c) {
    const size_t sb = (size_t)h * p.nslots + key + c;
    float* mo = wsM + sb * DK * dv;
    const bool store = c >= c0;  // halo chunks are not stored
#pragma unroll
    for (int m = 0; m < SBk::PER; ++m) {
      const int blk = wave + 4 * m;
      if (blk < SBk::NBM) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 16 * blk + 4 * lq + x;
          if (store) mo[(long)i * dv + col0 + ln] = M[m][x];
          Ms[i][ln] = M[m][x];
        }
      }
    }
    kr.template store_s<SK>(ks, tid);
    vr.template store_s<ST>(vs, tid);
    tr.store_s<SC>(Ts, tid);
    if (tid < BC) bet[tid] = br;
    chunk_decay(gr, tid, gam, Gam, wv);
    if (c + 1 < c1) fetch(c + 1);
    __syncthreads();
    if (wave < 2) {  // X = beta (V - Gam K M), row block `wave`
      const int r16 = 16 * wave + ln;
      f32x4 y = zero;
#pragma unroll
      for (int kk = 0; kk < DK; kk += 4) y = mfma4(ks[r16][kk + lq], Ms[kk + lq][ln], y);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * wave + 4 * lq + x;
        Xs[t][ln] = bet[t] * (vs[t][ln] - Gam[t] * y[x]);
      }
    }
    __syncthreads();
    if (wave < 2) {  // W = diag(w) T X
      const int r16 = 16 * wave + ln;
      f32x4 u = zero;
#pragma unroll
      for (int kk = 0; kk < BC; kk += 4) u = mfma4(Ts[r16][kk + lq], Xs[kk + lq][ln], u);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * wave + 4 * lq + x;
        Ws[t][ln] = wv[t] * u[x];
      }
    }
    __syncthreads();
    {  // M <- Gam_C M + K^T W
      const float GC = Gam[BC - 1];
#pragma unroll
      for (int m = 0; m < SBk::PER; ++m) {
        const int blk = wave + 4 * m;
        if (blk < SBk::NBM) {
          f32x4 acc = GC * M[m];
#pragma unroll
          for (int kk = 0; kk < BC; kk += 4) acc = mfma4(ks[kk + lq][16 * blk + ln], Ws[kk + lq][ln], acc);
          M[m] = acc;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- adjoint ----
template <typename TI, int DK>
__global__ __launch_bounds__(NT, 2) void bwd_adjoint_kernel(const TI* __restrict__ q, const TI* __restrict__ k,
                                                            const TI* __restrict__ dO,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ beta,
                                                            const float* __restrict__ dhT,
                                                            const int32_t* __restrict__ cu,
                                                            const float* __restrict__ wsT,
                                                            const float* __restrict__ wsP,
                                                            float* __restrict__ wsD, float* __restrict__ dh0,
                                                            const BShape p) {
  using SBk = StateBlocks<DK>;
  constexpr int SK = DK + 8;
  __shared__ float qs[BC][SK], ks[BC][SK], ds[BC][ST], Ts[BC][SC], Ps[BC][SC];
  __shared__ float KDs[BC][ST], PDs[BC][ST], Zs[BC][ST], Ds[DK][ST];
  __shared__ float gam[BC], Gam[BC], wv[BC], bet[BC];
  const int tid = threadIdx.x, H = p.H, dv = p.dv;
  const int chain = blockIdx.x / (p.ntile * p.nseg), seg = (blockIdx.x / p.ntile) % p.nseg;
  const int tile = blockIdx.x % p.ntile;
  const int n = chain / H, h = chain % H, col0 = tile * TW;
  long row0;
  int len;
  seq_info(cu, p, n, row0, len);
  const int key = slot_key(cu, p, n), nch = (len + BC - 1) / BC;
  const int wave = tid >> 6, ln = tid & 15, lq = (tid >> 4) & 3;
  // chunks [c0, c1) are stored; the reverse sweep starts at ce >= c1 (see HALO_NATS)
  int c0 = 0, c1 = nch, ce = nch;
  if (p.nseg > 1) {
    __shared__ int sEnd;
    c0 = min(seg * p.seg_chunks, nch);
    c1 = min(c0 + p.seg_chunks, nch);
    if (wave == 0) {
      int cc = c1;
      float acc = 0.f;  // log of the norm product over chunks [c1, cc)
      while (cc < nch && acc > -HALO_NATS) {
        acc += chunk_log_norm<TI, DK>(k, g, beta, row0, len, H, h, cc, tid);
        ++cc;
      }
      if (tid == 0) sEnd = cc;
    }
    __syncthreads();
    ce = sEnd;
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 D[SBk::PER];
#pragma unroll
  for (int m = 0; m < SBk::PER; ++m) {
    const int blk = wave + 4 * m;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      D[m][x] = (dhT && ce == nch && blk < SBk::NBM)
                    ? dhT[((long)chain * DK + 16 * blk + 4 * lq + x) * dv + col0 + ln]
                    : 0.f;
  }

  // the previous chunk's inputs, fetched into registers while this one computes
  RowsReg<TI, DK> qr, kr;
  RowsReg<TI, TW> dr;
  CCReg tr, pr;
  float gr = 0.f, br = 0.f;
  auto fetch = [&](int c) {
    const int t0 = c * BC, Lc = min(BC, len - t0);
    qr.fetch(q, row0, t0, Lc, H, h, DK, 0, tid);
    kr.fetch(k, row0, t0, Lc, H, h, DK, 0, tid);
    dr.fetch(dO, row0, t0, Lc, H, h, dv, col0, tid);
    const size_t sb = (size_t)h * p.nslots + key + c;
    tr.fetch(wsT + sb * (BC * BC), tid);
    pr.fetch(wsP + sb * (BC * BC), tid);
    if (tid < BC) {
      gr = token_f(g, row0, t0, Lc, H, h, tid);
      br = token_f(beta, row0, t0, Lc, H, h, tid);
    }
  };
  if (ce > c0) fetch(ce - 1);

  for (int c = ce - 1; c >= c0; --c) {
    const size_t sb = (size_t)h * p.nslots + key + c;
    float* dout = wsD + sb * DK * dv;
    const bool store = c < c1;  // halo chunks are not stored
#pragma unroll
    for (int m = 0; m < SBk::PER; ++m) {
      const int blk = wave + 4 * m;
      if (blk < SBk::NBM) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 16 * blk + 4 * lq + x;
          if (store) dout[(long)i * dv + col0 + ln] = D[m][x];
          Ds[i][ln] = D[m][x];
        }
      }
    }
    qr.template store_s<SK>(qs, tid);
    kr.template store_s<SK>(ks, tid);
    dr.template store_s<ST>(ds, tid);
    tr.store_s<SC>(Ts, tid);
    pr.store_s<SC>(Ps, tid);
    if (tid < BC) bet[tid] = br;
    chunk_decay(gr, tid, gam, Gam, wv);
    if (c > c0) fetch(c - 1);
    __syncthreads();
    if (wave < 2) {  // KD = K dM' on row block `wave`
      const int r16 = 16 * wave + ln;
      f32x4 a = zero;
#pragma unroll
      for (int kk = 0; kk < DK; kk += 4) a = mfma4(ks[r16][kk + lq], Ds[kk + lq][ln], a);
#pragma unroll
      for (int x = 0; x < 4; ++x) KDs[16 * wave + 4 * lq + x][ln] = a[x];
    } else {  // P^T dO on row block `wave - 2`
      const int rb = wave - 2, r16 = 16 * rb + ln;
      f32x4 a = zero;
#pragma unroll
      for (int kk = 0; kk < BC; kk += 4) a = mfma4(Ps[kk + lq][r16], ds[kk + lq][ln], a);
#pragma unroll
      for (int x = 0; x < 4; ++x) PDs[16 * rb + 4 * lq + x][ln] = a[x];
    }
    __syncthreads();
    if (wave < 2) {  // dX = T^T dU with dU = P^T dO + diag(w) KD;  Z = diag(beta Gam) dX
      const int r16 = 16 * wave + ln;
      f32x4 a = zero;
#pragma unroll
      for (int kk = 0; kk < BC; kk += 4) {
        const int r = kk + lq;
        a = mfma4(Ts[r][r16], __builtin_fmaf(wv[r], KDs[r][ln], PDs[r][ln]), a);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * wave + 4 * lq + x;
        Zs[t][ln] = bet[t] * Gam[t] * a[x];
      }
    }
    __syncthreads();
    {  // dM <- Gam_C dM' + Q^T diag(Gam) dO - K^T Z
      const float GC = Gam[BC - 1];
#pragma unroll
      for (int m = 0; m < SBk::PER; ++m) {
        const int blk = wave + 4 * m;
        if (blk < SBk::NBM) {
          f32x4 acc = GC * D[m];
#pragma unroll
          for (int kk = 0; kk < BC; kk += 4) {
            const int r = kk + lq;
            acc = mfma4(qs[r][16 * blk + ln], Gam[r] * ds[r][ln], acc);
            acc = mfma4(-ks[r][16 * blk + ln], Zs[r][ln], acc);
          }
          D[m] = acc;
        }
      }
    }
    __syncthreads();
  }
  if (dh0 && c0 == 0) {  // the segment holding the sequence start
#pragma unroll
    for (int m = 0; m < SBk::PER; ++m) {
      const int blk = wave + 4 * m;
      if (blk < SBk::NBM) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          dh0[((long)chain * DK + 16 * blk + 4 * lq + x) * dv + col0 + ln] = D[m][x];
      }
    }
  }
}

// ---------------------------------------------------------------- grad ----
template <typename TI, int DK>
struct GradLds {
  static constexpr int SK = DK + 8;
  TI qs[BC][SK], ks[BC][SK];  // stored as given (bf16 is widened on read)
  float Ts[BC][SC], Ps[BC][SC];
  union {
    struct {
      float Mt[DK][ST], Dt[DK][ST];
    } tile;
    struct {
      float Gs[BC][SC], dPs[BC][SC], Zs[BC][SC], Bs[BC][SC];
    } fin;
  } u;
  float vt[BC][ST], dot[BC][ST], Yt[BC][ST], KDt[BC][ST], Xt[BC][ST], Ut[BC][ST], dUt[BC][ST], dXt[BC][ST];
  float gam[BC], bet[BC], sgQ[2][BC], sgB[BC], sb1[BC], sw[BC], red[NT / 64];
};

template <typename TI, int DK>
__global__ __launch_bounds__(NT, sizeof(TI) == 2 ? 2 : 1) void bwd_grad_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v, const TI* __restrict__ dO,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    const float* __restrict__ wsT, const float* __restrict__ wsP, const float* __restrict__ wsM,
    const float* __restrict__ wsD, TI* __restrict__ dq, TI* __restrict__ dk, TI* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta, const BShape p) {
  constexpr int NB = DK / 8 / 4;  // 16x16 blocks of the C x DK gradients per wave
  constexpr int JP = Owner<DK>::JP;
  __shared__ GradLds<TI, DK> L;
  const int tid = threadIdx.x, s = blockIdx.x, h = blockIdx.y, H = p.H, dvn = p.dv;
  const int n = find_seq(cu, p, s);
  long row0;
  int len;
  seq_info(cu, p, n, row0, len);
  const int c = s - slot_key(cu, p, n);
  if (c < 0 || (long)c * BC >= len) return;  // slot not used
  const int t0 = c * BC, Lc = min(BC, len - t0);
  const size_t sb = (size_t)h * p.nslots + s;
  for (int e = tid; e < BC * DK; e += NT) {
    const int t = e / DK, i = e % DK;
    const long off = ((row0 + t0 + t) * H + h) * DK + i;
    L.qs[t][i] = t < Lc ? q[off] : (TI)0.f;
    L.ks[t][i] = t < Lc ? k[off] : (TI)0.f;
  }
  for (int e = tid; e < BC * BC; e += NT) {
    L.Ts[e / BC][e % BC] = wsT[sb * (BC * BC) + e];
    L.Ps[e / BC][e % BC] = wsP[sb * (BC * BC) + e];
  }
  if (tid < BC) L.bet[tid] = token_f(beta, row0, t0, Lc, H, h, tid);
  chunk_gamma(tid < BC ? token_f(g, row0, t0, Lc, H, h, tid) : 0.f, tid, L.gam);
  auto kf = [&](int r, int i) { return (float)L.ks[r][i]; };
  auto qf = [&](int r, int i) { return (float)L.qs[r][i]; };

  const int wave = tid >> 6, ln = tid & 15, lq = (tid >> 4) & 3;
  const int rb = wave & 1;          // row block of the tile phases
  const int r16 = 16 * rb + ln;     // the lane's A-operand row in those phases
  const Owner<DK> o(tid);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 accQ[NB], accK[NB], accXU = zero, accOU = zero;
#pragma unroll
  for (int m = 0; m < NB; ++m) accQ[m] = accK[m] = zero;
  float pA[4] = {0.f, 0.f, 0.f, 0.f}, pB[4] = {0.f, 0.f, 0.f, 0.f};  // per-row partial sums
  float sGC = 0.f;
  const float* mbase = wsM + sb * DK * dvn;
  const float* dbase = wsD + sb * DK * dvn;
  // the next tile's entry state, exit gradient, v and dO, fetched into
  // registers while this one computes
  constexpr int NS = DK * TW / NT;
  float mr[NS], dr[NS];
  RowsReg<TI, TW> vr, orr;
  auto fetch = [&](int tile) {
    const int col0 = tile * TW;
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      const int e = tid + NT * x, i = e / TW, j = e % TW;
      mr[x] = mbase[(long)i * dvn + col0 + j];
      dr[x] = dbase[(long)i * dvn + col0 + j];
    }
    vr.fetch(v, row0, t0, Lc, H, h, dvn, col0, tid);
    orr.fetch(dO, row0, t0, Lc, H, h, dvn, col0, tid);
  };
  fetch(0);

  for (int tile = 0; tile < p.ntile; ++tile) {
    const int col0 = tile * TW;
    __syncthreads();  // the previous tile's readers are done
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      const int e = tid + NT * x, i = e / TW, j = e % TW;
      L.u.tile.Mt[i][j] = mr[x];
      L.u.tile.Dt[i][j] = dr[x];
    }
    vr.template store_s<ST>(L.vt, tid);
    orr.template store_s<ST>(L.dot, tid);
    if (tile + 1 < p.ntile) fetch(tile + 1);
    __syncthreads();
    // phase A.  waves 0, 1: Y = K M on row block rb, then X;
    //           waves 2, 3: KD = K dM' and P^T dO on row block rb, then dU.
    if (wave < 2) {
      const f32x4 y = mfma_chain<DK>(zero, [&](int kk) { return kf(r16, kk + lq); },
                                     [&](int kk) { return L.u.tile.Mt[kk + lq][ln]; });
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * rb + 4 * lq + x;
        L.Yt[t][ln] = y[x];
        L.Xt[t][ln] = L.bet[t] * (L.vt[t][ln] - ex(L.gam[t]) * y[x]);
      }
    } else {
      const f32x4 kd = mfma_chain<DK>(zero, [&](int kk) { return kf(r16, kk + lq); },
                                      [&](int kk) { return L.u.tile.Dt[kk + lq][ln]; });
      const f32x4 pd = mfma_chain<BC>(zero, [&](int kk) { return L.Ps[kk + lq][r16]; },
                                      [&](int kk) { return L.dot[kk + lq][ln]; });
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * rb + 4 * lq + x;
        L.KDt[t][ln] = kd[x];
        L.dUt[t][ln] = __builtin_fmaf(ex(L.gam[BC - 1] - L.gam[t]), kd[x], pd[x]);
      }
    }
    __syncthreads();
    // phase B.  waves 0, 1: U = T X;  waves 2, 3: dX = T^T dU, dV.
    if (wave < 2) {
      const f32x4 uu = mfma_chain<BC>(zero, [&](int kk) { return L.Ts[r16][kk + lq]; },
                                      [&](int kk) { return L.Xt[kk + lq][ln]; });
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * rb + 4 * lq + x;
        L.Ut[t][ln] = uu[x];
        pB[x] = __builtin_fmaf(uu[x], L.KDt[t][ln], pB[x]);  // U . KD
      }
    } else {
      const f32x4 dx = mfma_chain<BC>(zero, [&](int kk) { return L.Ts[kk + lq][r16]; },
                                      [&](int kk) { return L.dUt[kk + lq][ln]; });
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int t = 16 * rb + 4 * lq + x;
        const float bt = L.bet[t], yv = L.Yt[t][ln];
        L.dXt[t][ln] = dx[x];
        pA[x] = __builtin_fmaf(dx[x], L.vt[t][ln] - ex(L.gam[t]) * yv, pA[x]);  // dX . R
        pB[x] = __builtin_fmaf(-bt * dx[x], yv, pB[x]);                        // -beta dX . Y
        if (t < Lc) dv[((row0 + t0 + t) * H + h) * (long)dvn + col0 + ln] = (TI)(bt * dx[x]);
      }
    }
#pragma unroll
    for (int r = 0; r < JP; ++r)
      sGC = __builtin_fmaf(L.u.tile.Mt[o.si][o.sj0 + r], L.u.tile.Dt[o.si][o.sj0 + r], sGC);
    __syncthreads();
    // phase C, all waves.  dX U^T and dO U^T (C x C, block `wave`), and
    // dQ0 += dO M^T (diag(Gam) is applied after the last tile), dK +=
    // -diag(beta Gam) dX M^T + diag(w) U dM'^T (C x DK, blocks wave + 4 m).
    {
      const int cr = 16 * (wave >> 1) + ln, cc = 16 * (wave & 1) + ln;
      float xa[TW / 4], oa[TW / 4], ub[TW / 4];
#pragma unroll
      for (int j = 0; j < TW / 4; ++j) {
        xa[j] = L.dXt[cr][4 * j + lq];
        oa[j] = L.dot[cr][4 * j + lq];
        ub[j] = L.Ut[cc][4 * j + lq];
      }
#pragma unroll
      for (int j = 0; j < TW / 4; ++j) {
        accXU = mfma4(xa[j], ub[j], accXU);
        accOU = mfma4(oa[j], ub[j], accOU);
      }
    }
    {
      // the A operands' rows are the same for every block of this wave
      const int br = 16 * (wave & 1) + ln;
      const float bg = -L.bet[br] * ex(L.gam[br]), w = ex(L.gam[BC - 1] - L.gam[br]);
      float ao[TW / 4], ax[TW / 4], au[TW / 4];
#pragma unroll
      for (int j = 0; j < TW / 4; ++j) {
        ao[j] = L.dot[br][4 * j + lq];
        ax[j] = bg * L.dXt[br][4 * j + lq];
        au[j] = w * L.Ut[br][4 * j + lq];
      }
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const int bc = 16 * ((wave + 4 * m) >> 1) + ln;
        float mv[TW / 4], dd[TW / 4];
#pragma unroll
        for (int j = 0; j < TW / 4; ++j) {
          mv[j] = L.u.tile.Mt[bc][4 * j + lq];
          dd[j] = L.u.tile.Dt[bc][4 * j + lq];
        }
#pragma unroll
        for (int j = 0; j < TW / 4; ++j) {
          accQ[m] = mfma4(ao[j], mv[j], accQ[m]);
          accK[m] = mfma4(ax[j], mv[j], accK[m]);
          accK[m] = mfma4(au[j], dd[j], accK[m]);
        }
      }
    }
  }
  // dO_t . (Q M)_t summed over all value columns is q_t . (M dO_t) = q_t . dQ0_t
  // (this wave's key columns of it); then dQ0 gets its diag(Gam)
  float pQ[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int bc = 16 * ((wave + 4 * m) >> 1) + ln;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = 16 * rb + 4 * lq + x;
      pQ[x] = __builtin_fmaf(qf(t, bc), accQ[m][x], pQ[x]);
      accQ[m][x] *= ex(L.gam[t]);
    }
  }
  // per-row partial sums: reduce over the 16 lanes of a row group
#pragma unroll
  for (int x = 0; x < 4; ++x) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      pA[x] += __shfl_xor(pA[x], m);
      pB[x] += __shfl_xor(pB[x], m);
      pQ[x] += __shfl_xor(pQ[x], m);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sGC += __shfl_xor(sGC, m);
  __syncthreads();  // the last tile's readers of Mt / Dt are done (fin reuses them)
  if (ln == 0) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = 16 * rb + 4 * lq + x;
      L.sgQ[wave >> 1][t] = pQ[x];  // dO . QM, this wave's key columns
      if (wave < 2) {
        L.sw[t] = pB[x];  // U . KD
      } else {
        L.sb1[t] = pA[x];  // dX . R
        L.sgB[t] = pB[x];  // -beta dX . Y
      }
    }
  }
  if ((tid & 63) == 0) L.red[wave] = sGC;
  {  // K K^T on block `wave`, then dA, G, dP . E, Z and the second dbeta term
    const int tr0 = 16 * (wave >> 1), uc = 16 * (wave & 1) + ln;
    const f32x4 kk4 = mfma_chain<DK>(zero, [&](int kk) { return kf(tr0 + ln, kk + lq); },
                                     [&](int kk) { return kf(uc, kk + lq); });
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = tr0 + 4 * lq + x;
      const float bt = L.bet[t];
      const float E = uc <= t ? ex(L.gam[t] - L.gam[uc]) : 0.f;
      const float dA = uc < t ? -accXU[x] : 0.f;
      const float kke = kk4[x] * E;
      const float dP = uc <= t ? accOU[x] : 0.f;
      L.u.fin.Gs[t][uc] = dA * E * bt;
      L.u.fin.dPs[t][uc] = dP * E;
      // the diagonal adds to a token's row and column alike: left out
      L.u.fin.Zs[t][uc] = uc < t ? __builtin_fmaf(dA, bt * kke, dP * L.Ps[t][uc]) : 0.f;
      L.u.fin.Bs[t][uc] = dA * kke;
    }
  }
  __syncthreads();
  // dQ += (dP . E) K;  dK += (G + G^T) K + (dP . E)^T Q
  // the A operands' rows are the same for every block of this wave
  const int fbr = 16 * (wave & 1);
  float fp[BC / 4], fg[BC / 4], ft[BC / 4];
#pragma unroll
  for (int j = 0; j < BC / 4; ++j) {
    const int r = 4 * j + lq;
    fp[j] = L.u.fin.dPs[fbr + ln][r];
    fg[j] = L.u.fin.Gs[fbr + ln][r] + L.u.fin.Gs[r][fbr + ln];
    ft[j] = L.u.fin.dPs[r][fbr + ln];
  }
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int blk = wave + 4 * m, br = 16 * (blk & 1), bc = 16 * (blk >> 1) + ln;
    float kv[BC / 4], qv[BC / 4];
#pragma unroll
    for (int j = 0; j < BC / 4; ++j) {
      kv[j] = kf(4 * j + lq, bc);
      qv[j] = qf(4 * j + lq, bc);
    }
#pragma unroll
    for (int j = 0; j < BC / 4; ++j) {
      accQ[m] = mfma4(fp[j], kv[j], accQ[m]);
      accK[m] = mfma4(fg[j], kv[j], accK[m]);
      accK[m] = mfma4(ft[j], qv[j], accK[m]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t = br + 4 * lq + x;
      if (t < Lc) {
        const long off = ((row0 + t0 + t) * H + h) * DK + bc;
        dq[off] = (TI)accQ[m][x];
        dk[off] = (TI)accK[m][x];
      }
    }
  }
  if (tid < BC) {  // per-token terms
    const int t = tid, last = Lc - 1;
    float rz = 0.f, cz = 0.f, b2 = 0.f;
#pragma unroll
    for (int uu = 0; uu < BC; ++uu) {
      rz += L.u.fin.Zs[t][uu];
      cz += L.u.fin.Zs[uu][t];
      b2 += L.u.fin.Bs[t][uu];
    }
    float gc = 0.f;
    for (int wv = 0; wv < NT / 64; ++wv) gc += L.red[wv];
    const float Gt = ex(L.gam[t]), wt = ex(L.gam[BC - 1] - L.gam[t]);
    const float dGam = (L.sgQ[0][t] + L.sgQ[1][t]) + L.sgB[t] + (t == last ? gc : 0.f);
    L.sb1[t] += b2;                                   // dbeta, in place
    L.sgQ[0][t] = __builtin_fmaf(dGam, Gt, rz - cz);  // dgamma without the w terms, in place
    L.sw[t] *= wt;                                 // dw . w, in place
  }
  __syncthreads();
  // dg_t = sum_{u >= t} dgamma_u.  The w terms (-dw_u w_u at every token,
  // +sum_u dw_u w_u at the last) are summed in the form they take after the
  // reverse sum, sum_{u < t} dw_u w_u, which does not cancel large terms
  // when the decay is strong.
  if (tid < Lc) {
    const int t = tid;
    // fixed trip counts (the reads do not wait on each other); adding the
    // zeros of rows past the chunk's end first leaves the sum unchanged
    float acc = 0.f;
#pragma unroll
    for (int uu = BC - 1; uu >= 0; --uu) acc += (uu >= t && uu < Lc) ? L.sgQ[0][uu] : 0.f;
#pragma unroll
    for (int uu = 0; uu < BC; ++uu) acc += uu < t ? L.sw[uu] : 0.f;
    const long th = (row0 + t0 + t) * H + h;
    dg[th] = acc;
    dbeta[th] = L.sb1[t];
  }
}

// ---------------------------------------------------------------- host ----
size_t slots_per_head(long ttot, int B) { return (size_t)(ttot / BC) + (size_t)B + 1; }

size_t ws_floats(size_t nslots, int H, int dk, int dv) {
  return (size_t)H * nslots * (2 * (size_t)BC * BC + 2 * (size_t)dk * dv);
}

template <typename TI, int DK>
int launch_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta, const float* h0,
               const int32_t* cu, const void* dO, const float* dhT, void* dq, void* dk, void* dv, float* dg,
               float* dbeta, float* dh0, float* ws, const BShape& p, hipStream_t st) {
  const size_t cc = (size_t)p.H * p.nslots * BC * BC;
  const size_t sm = (size_t)p.H * p.nslots * DK * p.dv;
  float* wsT = ws;
  float* wsP = wsT + cc;
  float* wsM = wsP + cc;
  float* wsD = wsM + sm;
  const TI *qq = static_cast<const TI*>(q), *kk = static_cast<const TI*>(k), *vv = static_cast<const TI*>(v);
  const TI* oo = static_cast<const TI*>(dO);
  const dim3 chunks(p.nslots, p.H), chains(p.B * p.H * p.ntile * p.nseg);
  if (p.B * p.H * p.ntile == 0) return GDN_OK;
  hipLaunchKernelGGL((bwd_prep_kernel<TI, DK>), chunks, dim3(NT), 0, st, qq, kk, g, beta, cu, wsT, wsP, p);
  hipLaunchKernelGGL((bwd_states_kernel<TI, DK>), chains, dim3(NT), 0, st, kk, vv, g, beta, h0, cu, wsT, wsM, p);
  hipLaunchKernelGGL((bwd_adjoint_kernel<TI, DK>), chains, dim3(NT), 0, st, qq, kk, oo, g, beta, dhT, cu, wsT,
                     wsP, wsD, dh0, p);
  hipLaunchKernelGGL((bwd_grad_kernel<TI, DK>), chunks, dim3(NT), 0, st, qq, kk, vv, oo, g, beta, cu, wsT, wsP,
                     wsM, wsD, static_cast<TI*>(dq), static_cast<TI*>(dk), static_cast<TI*>(dv), dg, dbeta, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename TI>
int launch_dtype(int dkn, const void* q, const void* k, const void* v, const float* g, const float* beta,
                 const float* h0, const int32_t* cu, const void* dO, const float* dhT, void* dq, void* dk, void* dv,
                 float* dg, float* dbeta, float* dh0, float* ws, const BShape& p, hipStream_t st) {
  switch (dkn) {
    case 32: return launch_bwd<TI, 32>(q, k, v, g, beta, h0, cu, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws, p, st);
    case 64: return launch_bwd<TI, 64>(q, k, v, g, beta, h0, cu, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws, p, st);
    case 128: return launch_bwd<TI, 128>(q, k, v, g, beta, h0, cu, dO, dhT, dq, dk, dv, dg, dbeta, dh0, ws, p, st);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

bool bwd_sizes_ok(int B, int T, int H, int dk, int dv, int packed) {
  if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1) return false;
  if (!packed && (long)B * T > 0x7fffffffL) return false;
  return true;
}

}  // namespace

namespace {

// Workspace of gdn_bwd_noalloc: one array per GPU, in the library's device
// code object, held until the process ends.  Host code never passes this
// name to a kernel; it passes the device address that hipGetSymbolAddress
// returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
float* g_scratch[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];

// The current device's scratch address (looked up once per device, with
// that device current), or null if the lookup failed.
float* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_rc[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_rc[dev] == hipSuccess ? static_cast<float*>(ptr) : nullptr;
  });
  return g_scratch[dev];
}

}  // namespace

extern "C" long long gdn_bwd_workspace_size(int B, int T, int H, int dk, int dv, int packed) {
  if (!bwd_sizes_ok(B, T, H, dk, dv, packed)) return GDN_ERR_INVALID_ARG;
  if (H > 65535) return GDN_ERR_UNSUPPORTED;
  if ((dk != 32 && dk != 64 && dk != 128) || (dv != 32 && dv != 64 && dv != 128)) return GDN_ERR_UNSUPPORTED;
  const long ttot = packed ? (long)T : (long)B * T;
  return (long long)(ws_floats(slots_per_head(ttot, B), H, dk, dv) * sizeof(float));
}

namespace {

// Every host-side check of gdn_bwd except the workspace's.
int bwd_check(const void* q, const void* k, const void* v, const float* g, const float* beta,
              const int32_t* cu_seqlens, const void* dout, void* dq, void* dk, void* dv, float* dg,
              float* dbeta, int B, int T, int H, int dkn, int dvn, int dtype) {
  if (!bwd_sizes_ok(B, T, H, dkn, dvn, cu_seqlens != nullptr)) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
    return GDN_ERR_INVALID_ARG;
  if ((dkn != 32 && dkn != 64 && dkn != 128) || (dvn != 32 && dvn != 64 && dvn != 128)) return GDN_ERR_UNSUPPORTED;
  if (H > 65535) return GDN_ERR_UNSUPPORTED;
  const long ttot = cu_seqlens ? (long)T : (long)B * T;
  const size_t nslots = slots_per_head(ttot, B);
  if ((long long)(nslots * (size_t)H) > 0x7fffffffLL || nslots > 0x7fffffffULL) return GDN_ERR_UNSUPPORTED;
  if ((long)B * H * (dvn / TW) > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace

// The full-width backward (bf16, dk = dv = 128, a 16-byte-aligned workspace
// of gdn_bwd_workspace_size bytes): states (unless states_saved), adjoint
// and gradient kernels of gdn_bwd_full.hip.
static int bwd_full_path(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* h0, const int32_t* cu_seqlens, const void* dout, const float* dhT, void* dq,
                         void* dk, void* dv, float* dg, float* dbeta, float* dh0, void* workspace, int B, int T,
                         int H, long ttot, bool states_saved, hipStream_t st) {
  gdn_launch::BwdParams bp;
  bp.q = static_cast<const char*>(q);
  bp.k = static_cast<const char*>(k);
  bp.v = static_cast<const char*>(v);
  bp.dO = static_cast<const char*>(dout);
  bp.g = g;
  bp.beta = beta;
  bp.h0 = h0;
  bp.dhT = dhT;
  bp.cu = cu_seqlens;
  bp.dq = static_cast<char*>(dq);
  bp.dk = static_cast<char*>(dk);
  bp.dv = static_cast<char*>(dv);
  bp.dg = dg;
  bp.dbeta = dbeta;
  bp.dh0 = dh0;
  bp.sv = static_cast<char*>(workspace);
  bp.hT = dg;
  bp.B = B;
  bp.T = T;
  bp.H = H;
  bp.seg_max = gdn_launch::SEG_MAX_CHUNKS;
  bp.seg_cap = gdn_launch::seg_cap_for(H);
  bp.nslot = gdn_launch::full_slots(B, T, cu_seqlens != nullptr, bp.seg_max, bp.seg_cap);
  bp.nchunk = (int)(ttot / 64 + B);
  bp.states_saved = states_saved ? 1 : 0;
  return gdn_launch::bwd_full(bp, st);
}

// Whether gdn_bwd takes the full-width kernels for these arguments.
static bool bwd_full_width(int dtype, int dkn, int dvn, const void* workspace, size_t need, int B, long ttot, int H) {
  return dtype == GDN_BF16 && dkn == 128 && dvn == 128 && (reinterpret_cast<uintptr_t>(workspace) & 15u) == 0 &&
         (long long)need >= gdn_launch::bwd_full_ws_bytes(B, ttot, H);
}

extern "C" int gdn_bwd_saved(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* h0, const int32_t* cu_seqlens, const void* dout, const float* dhT,
                             void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, void* workspace,
                             long long workspace_bytes, int B, int T, int H, int dkn, int dvn, void* stream,
                             int dtype) {
  const int rc = bwd_check(q, k, v, g, beta, cu_seqlens, dout, dq, dk, dv, dg, dbeta, B, T, H, dkn, dvn, dtype);
  if (rc != GDN_OK) return rc;
  const long ttot = cu_seqlens ? (long)T : (long)B * T;
  const size_t need = ws_floats(slots_per_head(ttot, B), H, dkn, dvn) * sizeof(float);
  if (B > 0 && (!workspace || workspace_bytes < 0 || (size_t)workspace_bytes < need))
    return GDN_ERR_INVALID_ARG;
  if (!bwd_full_width(dtype, dkn, dvn, workspace, need, B, ttot, H)) return GDN_ERR_UNSUPPORTED;
  if (B == 0) return GDN_OK;
  return bwd_full_path(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0, workspace, B, T, H,
                       ttot, true, static_cast<hipStream_t>(stream));
}

extern "C" int gdn_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const float* h0, const int32_t* cu_seqlens, const void* dout, const float* dhT, void* dq,
                       void* dk, void* dv, float* dg, float* dbeta, float* dh0, void* workspace,
                       long long workspace_bytes, int B, int T, int H, int dkn, int dvn, void* stream, int dtype) {
  const int rc = bwd_check(q, k, v, g, beta, cu_seqlens, dout, dq, dk, dv, dg, dbeta, B, T, H, dkn, dvn, dtype);
  if (rc != GDN_OK) return rc;
  const long ttot = cu_seqlens ? (long)T : (long)B * T;
  const size_t nslots = slots_per_head(ttot, B);
  const size_t need = ws_floats(nslots, H, dkn, dvn) * sizeof(float);
  if (B > 0 && (!workspace || workspace_bytes < 0 || (size_t)workspace_bytes < need ||
                (reinterpret_cast<uintptr_t>(workspace) & 3u)))
    return GDN_ERR_INVALID_ARG;
  if (B == 0) return GDN_OK;
  BShape p;
  p.B = B;
  p.T = T;
  p.H = H;
  p.dv = dvn;
  p.nslots = (int)nslots;
  p.ntile = dvn / TW;
  // Sequence segments (see HALO_NATS) for dense batches with fewer (chain,
  // tile) workgroups than two per CU and at least 16 chunks per sequence.
  p.nseg = 1;
  p.seg_chunks = 0;
  if (!cu_seqlens) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 0;
    const long nwg = (long)B * H * p.ntile, slots = 2L * ncu;
    const int nch = (T + BC - 1) / BC;
    if (nwg > 0 && nwg < slots && nch >= 16) {
      const int nseg = (int)(slots / nwg < nch / 8 ? slots / nwg : nch / 8);
      if (nseg >= 2) {
        p.seg_chunks = (nch + nseg - 1) / nseg;
        p.nseg = (nch + p.seg_chunks - 1) / p.seg_chunks;  // every segment holds a chunk
      }
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16 with dk = dv = 128: the full-width kernels (gdn_bwd_full.hip), whose
  // records fit in the workspace sized above (a 16-byte-aligned one).
  if (bwd_full_width(dtype, dkn, dvn, workspace, need, B, ttot, H))
    return bwd_full_path(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0, workspace, B, T,
                         H, ttot, false, st);
  float* ws = static_cast<float*>(workspace);
  return dtype == GDN_BF16 ? launch_dtype<__bf16>(dkn, q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg,
                                                  dbeta, dh0, ws, p, st)
                           : launch_dtype<float>(dkn, q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg,
                                                 dbeta, dh0, ws, p, st);
}

extern "C" int gdn_bwd_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               const float* h0, const int32_t* cu_seqlens, const void* dout, const float* dhT,
                               void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0, int B, int T,
                               int H, int dkn, int dvn, void* stream, int dtype) {
  const int rc = bwd_check(q, k, v, g, beta, cu_seqlens, dout, dq, dk, dv, dg, dbeta, B, T, H, dkn, dvn, dtype);
  if (rc != GDN_OK) return rc;
  const long long need = gdn_bwd_workspace_size(B, T, H, dkn, dvn, cu_seqlens != nullptr);
  if (need < 0) return (int)need;
  if ((unsigned long long)need > kScratchBytes) return GDN_ERR_SCRATCH;
  if (B == 0) return GDN_OK;
  float* ws = device_scratch();
  if (!ws) return GDN_ERR_LAUNCH;
  return gdn_bwd(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0, ws,
                 (long long)kScratchBytes, B, T, H, dkn, dvn, stream, dtype);
}
