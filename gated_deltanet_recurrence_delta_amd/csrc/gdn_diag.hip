// The diagonal-decay additive recurrence that HyMo writes for its GDN
// layer, for gfx950.
//
// Per head, with the state H of shape (S, D) (key rows x value columns),
// A = -exp(A_log) (HyMo "Model Architecture Walkthrough", section 5.2.1;
// A_log of shape (H, S) as in "Optimization Quartet", section 3.2):
//
//   H_t = exp(g_t A) (.) H_{t-1} + b_t (x) v_t     each key row decays alone
//   o_t = c_t^T H_t                                 read after the write
//
// followed by the block's epilogue o_t <- (o_t + D_h v_t) * gate_t
// (Walkthrough, section 5.5 step 6 and section 5.6), each factor optional.
//
// Every value column of the state evolves on its own: column d only ever
// meets v_t[d].  That is what both forms below exploit.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DShape {
  int T, H, S, D, width, nslab, nitems;
};

// ---------------------------------------------------------------------------
// Token-by-token form (decoding and short sequences).
//
// One wave per (chain, slab of up to 64 value columns); lane j holds column
// j of the state, all S key rows, in registers, so the read c_t^T H_t is a
// sum inside the lane.  The token's b and c rows and its g, gate, the same
// for every lane, are read through the scalar unit; v and out are one
// element per lane.  The per-row decay rates A_s log2(e) are formed once per
// wave when they fit in registers next to the state (S <= 64).
// ---------------------------------------------------------------------------
constexpr int RWAVES = 4;

template <typename TI>
__device__ static inline float row_el(const TI* __restrict__ base, long row0, int i) {
  if constexpr (sizeof(TI) == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(base + row0)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return base[row0 + i];
  }
}

// log2 of the decay factor per unit of g for key row s: A_s log2(e), A_s = -exp(A_log).
__device__ static inline float decay_rate2(const float* __restrict__ alog, int i) {
  return -__builtin_amdgcn_exp2f(alog[i] * kLog2e) * kLog2e;
}

template <typename TI, int S>
__global__ __launch_bounds__(64 * RWAVES) void diag_recurrent_kernel(
    const TI* __restrict__ vp, const TI* __restrict__ bp, const TI* __restrict__ cp, const float* __restrict__ gp,
    const float* __restrict__ alog, const float* __restrict__ dskip, const float* __restrict__ gatep,
    const float* h0, const int32_t* __restrict__ cu, TI* __restrict__ out, float* hT,
    const DShape p) {
  // h0 and hT carry no restrict: hT may be h0 itself (each lane reads its
  // column of h0 before the token loop and writes it back after).
  constexpr bool kHoist = S <= 64;
  const int lane = threadIdx.x & 63;
  const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * RWAVES + (threadIdx.x >> 6));
  if (item >= p.nitems) return;  // whole waves leave together
  const int chain = item / p.nslab, slab = item % p.nslab;
  const int H = p.H, D = p.D;
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
  const long sbase = (long)chain * S * D + col;
  const float* __restrict__ arow = alog + (long)hh * S;

  float st[S];
#pragma unroll
  for (int s = 0; s < S; ++s) st[s] = 0.f;
  if (h0 && active) {
#pragma unroll
    for (int s = 0; s < S; ++s) st[s] = h0[sbase + (long)s * D];
  }
  float a2[kHoist ? S : 1];
  if constexpr (kHoist) {
#pragma unroll
    for (int s = 0; s < S; ++s) a2[s] = decay_rate2(arow, s);
  }
  const float dh = dskip ? dskip[hh] : 0.f;

  for (int t = 0; t < len; ++t) {
    const long th = (rowbase + t) * H + hh;  // token-head index
    const float gt = gp[th];
    const float vc = active ? (float)vp[th * D + col] : 0.f;
    const long r0 = th * S;
    float os[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float rate = kHoist ? a2[s] : decay_rate2(arow, s);
      const float a = __builtin_amdgcn_exp2f(gt * rate);
      st[s] = __builtin_fmaf(a, st[s], row_el(bp, r0, s) * vc);
      os[s & 3] = __builtin_fmaf(row_el(cp, r0, s), st[s], os[s & 3]);
    }
    float o = (os[0] + os[1]) + (os[2] + os[3]);
    if (dskip) o = __builtin_fmaf(dh, vc, o);
    if (gatep) o = o * gatep[th];
    if (active) out[th * D + col] = (TI)o;  // rounded to nearest even for bf16
  }
  if (active) {
#pragma unroll
    for (int s = 0; s < S; ++s) hT[sbase + (long)s * D] = st[s];
  }
}

template <typename TI, int S>
int launch_recurrent(const void* v, const void* b, const void* c, const float* g, const float* alog,
                     const float* dskip, const float* gate, const float* h0, const int32_t* cu, void* out, float* hT,
                     const DShape& p, hipStream_t s) {
  const int nwg = (p.nitems + RWAVES - 1) / RWAVES;
  hipLaunchKernelGGL((diag_recurrent_kernel<TI, S>), dim3(nwg), dim3(64 * RWAVES), 0, s, static_cast<const TI*>(v),
                     static_cast<const TI*>(b), static_cast<const TI*>(c), g, alog, dskip, gate, h0, cu,
                     static_cast<TI*>(out), hT, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <typename TI>
int dispatch_recurrent(const void* v, const void* b, const void* c, const float* g, const float* alog,
                       const float* dskip, const float* gate, const float* h0, const int32_t* cu, void* out,
                       float* hT, const DShape& p, hipStream_t s) {
  switch (p.S) {
    case 16: return launch_recurrent<TI, 16>(v, b, c, g, alog, dskip, gate, h0, cu, out, hT, p, s);
    case 32: return launch_recurrent<TI, 32>(v, b, c, g, alog, dskip, gate, h0, cu, out, hT, p, s);
    case 64: return launch_recurrent<TI, 64>(v, b, c, g, alog, dskip, gate, h0, cu, out, hT, p, s);
    case 128: return launch_recurrent<TI, 128>(v, b, c, g, alog, dskip, gate, h0, cu, out, hT, p, s);
    default: return GDN_ERR_UNSUPPORTED;
  }
}

bool pow2_dim(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }

// Host-side checks shared by both entry points; fills the shape on success.
int diag_validate(const void* v, const void* b, const void* c, const float* g, const float* alog, const void* out,
                  const float* hT, int B, int T, int H, int S, int D, int dtype, DShape* p) {
  if (B < 0 || T < 0 || H < 1 || S < 1 || D < 1) return GDN_ERR_INVALID_ARG;
  if (T > 0 && (!v || !b || !c || !g || !alog || !out)) return GDN_ERR_INVALID_ARG;
  if (B > 0 && !hT) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (!pow2_dim(S) || !pow2_dim(D)) return GDN_ERR_UNSUPPORTED;
  p->T = T;
  p->H = H;
  p->S = S;
  p->D = D;
  p->width = D < 64 ? D : 64;
  p->nslab = D / p->width;
  const long items = (long)B * H * p->nslab;
  if (items > 0x7fffffffL - 64) return GDN_ERR_INVALID_ARG;
  p->nitems = (int)items;
  return GDN_OK;
}


// ---------------------------------------------------------------------------
// Chunkwise form (long sequences), bf16 storage, S = D = 32.
//
// The pages run this layer as a chunked kernel with 64-token chunks
// ("Optimization Quartet", section 3.2): parallel inside a chunk, the state
// carried across chunks in series.  The algebra below follows from the
// unrolled sum of Walkthrough section 5.3.1.  Within a chunk let
// gamma_t = g_1 + ... + g_t (chunk-relative, inclusive) and x_t[s] =
// A_s gamma_t, which falls with t because A_s < 0 < g.  Then
//
//   o_t = c_t^T (e^{x_t} (.) H_c) + sum_{tau <= t} sum_s c_t[s] b_tau[s]
//                                     e^{x_t[s] - x_tau[s]} v_tau,
//   H_{c+1} = e^{x_63} (.) H_c + sum_tau (e^{x_63 - x_tau} (.) b_tau) v_tau^T.
//
// Every exponent used is <= 0 (a factor in [0, 1]), so nothing overflows;
// a factor that underflows to zero stands for a contribution below 1e-38 of
// its neighbours.
//
// Mapping: one workgroup per (chain, segment), 4 waves, two workgroups per
// CU; wave w takes chunks w, w+4, ... of its range; neighbouring chains run
// on one XCD.  Per chunk:
//   phase A (needs no state): the chunk's own write to the next state,
//     dH = sum_tau (e^{x_63 - x_tau} (.) b_tau) v_tau^T, with each key first
//     decayed to the end of its 16-token sub-chunk (kept for phase B); the
//     per-row decays e^{x} over each sub-chunk and over the chunk.
//   hand-off: wait for H_c (a counter in LDS guards two state slots), pass
//     H_{c+1} = e^{x_63} (.) H_c + dH on -- one multiply-add per element is
//     the whole serial path between waves.
//   phase B: the outputs, sub-chunk by sub-chunk with the running state Hs
//     (Hs = H_c at the first): O = Qt Hs + P V with Qt = c (.) e^{x_t -
//     x_ref} (ref = the token before the sub-chunk) and the 16x16 matrix
//     P[t][tau] = sum_s c_t[s] b_tau[s] e^{x_t[s] - x_tau[s]}, tau <= t;
//     then the epilogue and Hs <- E_k (.) Hs + Bt_k^T V_k.
// P is split at reference tokens so that no factor exceeds 1 even for rows
// that decay by e^-40 per token: pairs on the two sides of token 7, or of
// token 3 or 11 inside a half, are products X X^T of keys and queries
// decayed to the reference (fp16 matrix core); pairs inside one 4-token
// quarter are formed exactly by products of per-token decays in packed
// fp16 with fp32-accumulating dot products.  The other contractions (Bt^T V,
// Qt Hs, P V) run on the bf16 matrix core with fp32 accumulation, in one
// 16-deep accumulation chain for the outputs; the state is rounded to bf16
// only as an operand and carried in fp32.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int CW = 4;                // waves per workgroup (two workgroups per CU)
constexpr int CC = 64;               // tokens per chunk
constexpr int CS = 32;               // key rows
constexpr int CD = 32;               // value columns
constexpr int ROWB = 64;             // bytes per token row of b, c or v (32 bf16)
constexpr int SPIN_LIMIT = 1 << 26;  // bound on a wait for the previous chunk's state

struct ChunkParams {
  const __bf16* v;
  const __bf16* b;
  const __bf16* c;
  const float* g;
  const float* alog;
  const float* dskip;
  const float* gate;
  const float* h0;
  const int32_t* cu;
  __bf16* out;
  float* hT;
  int T, H, nchain, nseg, seg_chunks;
};

// Per-wave LDS region (≈17.6 KB; four waves and the shared part fit twice
// in a CU's 160 KB).
//
// The chunk rows of b, c and v are token-major, 64 bytes per token, with
// the four 16-byte granules of row r permuted: granule g sits at
// g ^ swz(r), swz(r) = the two bits of (r >> 2) & 3 reversed.  That puts
// the column reads of the c rows (sixteen rows, 8 bytes each) and the
// transposing reads of b and v (eight rows) on distinct banks.
//
// The decay-product tables of a sub-chunk are one contiguous block: the
// per-token decays e^{A_s g_t} (fp16, row t at 15 - t, i.e. stored last
// row first), then for each quarter of the sub-chunk (tokens 4 u .. 4 u + 3)
// 3 zero rows and its 4 b rows in fp16.  Rows -1 and -2 of the decay table
// fall into the first zero rows, and rows -1 ... -3 of each quarter of b
// into the zero rows before it, which is what lets every lane walk the same
// number of steps (see phase B).
constexpr int PROW = 80;  // bytes per row of P (bf16, column tau at 16 + tau)
struct WaveLds {
  alignas(16) char b[CC * ROWB];     // chunk rows of b (bf16, token-major, granules permuted)
  alignas(16) char c[CC * ROWB];
  alignas(16) char v[CC * ROWB];
  alignas(16) _Float16 ta[16 * CS];   // e^{A_s g_t}, last row first; output staging after P
  alignas(16) _Float16 tb[28 * CS];   // per quarter: 3 zero rows, then its b rows (fp16)
  alignas(16) char p[16 * PROW];     // P of the sub-chunk (bf16), row t, column tau at 16 + tau
  alignas(16) float ex[5 * CS];      // per-row decays: sub-chunk k at [32 k + s], chunk at [128 + s]
  alignas(16) float gam[CC];         // chunk-relative inclusive cumsum of g
  alignas(16) float graw[CC];
  alignas(16) float gate[CC];
};
static_assert(offsetof(WaveLds, tb) == offsetof(WaveLds, ta) + 16 * CS * 2, "tables are contiguous");
// byte offset in tb of b row t of the sub-chunk
__device__ static inline int tb_row(int t) { return 64 * (3 + t + 3 * (t >> 2)); }

// Granule permutation of the chunk rows (see WaveLds).
__device__ static inline int swz(int row) { return ((row >> 2) & 1) << 1 | ((row >> 3) & 1); }

struct ChunkLds {
  WaveLds w[CW];
  // entry states: element i of the lane's f32x4 number j at [j][lane][i]
  alignas(16) float state[2][CS * CD];
  alignas(16) float a2[CS];             // A_s log2(e)
  int ready;                            // index of the latest entry state in `state`
  int cstart;                           // first chunk this workgroup runs
};

__device__ static inline f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}

// Transposing LDS read (gfx950): within each 16-lane group, destination
// lane i, element k receives element (i & 3) of the 8 bytes addressed by
// source lane (i >> 2) + 4k.
__device__ static inline bf16x4 lds_read_tr(const char* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) char*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// a.x b.x + a.y b.y in fp32 (packed fp16 operands): the three-operand
// form with an inline zero, which needs no zeroed accumulator register.
__device__ static inline float dot2_first(h16x2 a, h16x2 b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ static inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ static inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ static inline float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ static inline float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// LDS-only ordering among the lanes of one wave.
__device__ static inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

__device__ static inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Pairs are converted as two-element vectors: that gives one packed
// conversion per pair, where a four-element vector (or one built element by
// element) is converted a value at a time and merged with permutes.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ static inline uint32_t cvt_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ static inline bf16x4 pack4(f32x4 x) {
  return __builtin_bit_cast(bf16x4, u32x2{cvt_pair(x[0], x[1]), cvt_pair(x[2], x[3])});
}

// Issue priority of the calling wave from the number r of chunks it still
// has after the current one (r is the same in every lane).  Two workgroups
// share each CU; with equal priorities the older wave of a SIMD wins every
// issue conflict, so the younger workgroup would lag and finish its last
// chunks alone.  A wave that falls behind the other wave of its SIMD by a
// chunk outranks it until it catches up.
__device__ static inline void set_prio_remaining(int r) {
  if (r >= 3) __builtin_amdgcn_s_setprio(3);
  else if (r == 2) __builtin_amdgcn_s_setprio(2);
  else if (r == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Wait until the LDS counter holds at least v (bounded: a wait that runs
// out leaves the loop so that the wave still ends).
__device__ static inline void wait_ready(const int* f, int v) {
  const unsigned addr = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) int*)f;
  for (int i = 0; i < SPIN_LIMIT; ++i) {
    int x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
    if (__builtin_amdgcn_readfirstlane(x) >= v) break;
  }
}

__global__ __launch_bounds__(64 * CW, 2) void diag_chunk_kernel(const ChunkParams p) {
  __shared__ __attribute__((aligned(16))) ChunkLds L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  // Consecutive chains (neighbouring heads, whose 64-byte token slices share
  // 128-byte cache lines) go to the same XCD: each XCD takes a contiguous
  // range of chains (the dispatcher deals workgroups round-robin over the 8).
  // A chain's segments (see below) are consecutive items.
  const int item = [](int bid, int n) {
    const int xcd = bid & 7, slot = bid >> 3, q8 = n >> 3, r8 = n & 7;
    return xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
  }(blockIdx.x, p.nchain * p.nseg);
  const int chain = item / p.nseg, seg = item % p.nseg;
  const int H = p.H;
  const int seq = chain / H, hh = chain % H;
  long row0;
  int len;
  if (p.cu) {
    row0 = p.cu[seq];
    len = p.cu[seq + 1] - p.cu[seq];
  } else {
    row0 = (long)seq * p.T;
    len = p.T;
  }
  const int nch = (len + CC - 1) / CC;
  WaveLds& W = L.w[wave];
  const long sbase = (long)chain * CS * CD;

  // ---- prologue: decay rates, where this workgroup starts, entry state -----
  // A dense batch with fewer chains than two per CU cuts each sequence into
  // segments of seg_chunks chunks, one workgroup each.  A segment's
  // recurrence starts from a zero state at the latest chunk boundary behind
  // it where the state's decay since then, prod_t max_s e^{g_t A_s} (the
  // transition's norm: it is diagonal with entries in [0, 1]), is below
  // e^-40, or at the sequence start from h0.  The state it then reaches at
  // the segment's start differs from the exact one by less than e^-40 of
  // the exact state at that boundary.  The chunks in between (the halo)
  // are computed and their outputs dropped; only the last segment writes hT.
  const int c0 = p.nseg > 1 ? seg * p.seg_chunks : 0;                  // first stored chunk
  const int c1 = p.nseg > 1 ? min(c0 + p.seg_chunks, nch) : nch;        // one past the last
  const bool write_hT = seg == p.nseg - 1;
  if (wave == 0) {
    if (lane < CS) L.a2[lane] = p.alog ? -__builtin_amdgcn_exp2f(p.alog[hh * CS + lane] * kLog2e) * kLog2e : 0.f;
    int cs = c0;
    if (cs > 0) {
      wave_lds_sync();
      float a2max = L.a2[lane & 31];  // the slowest row: its rate is the transition's norm
#pragma unroll
      for (int d = 16; d >= 1; d >>= 1) a2max = fmaxf(a2max, __shfl_xor(a2max, d));
      float acc = 0.f;  // log2 of the decay over chunks [cs, c0)
      while (cs > 0 && acc > -40.f * kLog2e) {
        --cs;  // chunks before c0 are whole: every lane holds a token
        float e = p.g[(row0 + (long)cs * CC + lane) * H + hh] * a2max;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) e += __shfl_xor(e, d);
        acc += e;
      }
    }
    // lane holds rows 16*mt + 4q + i, column 16*nt + n  (accumulator layout)
    float* slot = L.state[cs & 1] + 4 * lane;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 16 * mt + 4 * q + i, d = 16 * nt + n;
          const float x = (p.h0 && cs == 0) ? p.h0[sbase + s * CD + d] : 0.f;
          slot[256 * (2 * mt + nt) + i] = x;
          if (nch == 0) p.hT[sbase + s * CD + d] = x;
        }
    if (lane == 0) {
      L.ready = cs;
      L.cstart = cs;
    }
  }
  // the zero rows of the decay tables and the never-written part of P
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    // zero rows of tb: rows 7 u .. 7 u + 2, 12 granules per quarter u
    if (lane < 48) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(W.tb) + 448 * (lane / 12) + 16 * (lane % 12)) = z;
    *reinterpret_cast<u32x4*>(W.p + 16 * lane) = z;
    if (lane < 16) *reinterpret_cast<u32x4*>(W.p + 1024 + 16 * lane) = z;
  }
  __syncthreads();
  const int cs = L.cstart;
  if (cs + wave >= c1) return;

  // Decay rates in the lane's layouts: rows sigma(q, j) (= accumulator rows
  // 16*mt + 4q + i), rows n and n + 16, and the groups 8*(lane & 3) + j and
  // 8*q + j.
  float a2s[8], a2g[8], a2q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a2s[j] = L.a2[(j < 4 ? 0 : 16) + 4 * q + (j & 3)];
    a2g[j] = L.a2[8 * (lane & 3) + j];
    a2q[j] = L.a2[8 * q + j];
  }
  const float a2n0 = L.a2[n], a2n1 = L.a2[n + 16];
  const float dh = p.dskip ? p.dskip[hh] : 0.f;

  const long tok_stride = (long)H * ROWB;  // bytes between token rows of one head
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<const char*>(p.b) + (row0 * H + hh) * ROWB,
                                              (long)len * tok_stride);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(reinterpret_cast<const char*>(p.c) + (row0 * H + hh) * ROWB,
                                              (long)len * tok_stride);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const char*>(p.v) + (row0 * H + hh) * ROWB,
                                              (long)len * tok_stride);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(reinterpret_cast<char*>(p.out) + (row0 * H + hh) * ROWB,
                                              (long)len * tok_stride);
  // The next chunk of this wave is fetched into registers while the current
  // one is worked on (12 x 16 bytes per lane of b, c and v rows, plus the
  // lane's token gate values), and written to LDS when its turn comes.
  // Lane -> row 16*i + (lane >> 2) of the chunk, 16-byte granule lane & 3.
  u32x4 pf[12];
  float pg = 0.f, pgate = 1.f;
  // b, v and the gates first (phase A needs them), c last (phase B only).
  auto prefetch_bv = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int voff = (int)(((long)(c * CC + 16 * i + (lane >> 2))) * tok_stride) + 16 * (lane & 3);
      pf[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0);
      pf[8 + i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0);
    }
    const int tok = c * CC + lane;
    const long th = (row0 + tok) * H + hh;
    pg = tok < len ? p.g[th] : 0.f;
    pgate = (tok < len && p.gate) ? p.gate[th] : 1.f;
  };
  auto prefetch_c = [&](int c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int voff = (int)(((long)(c * CC + 16 * i + (lane >> 2))) * tok_stride) + 16 * (lane & 3);
      pf[4 + i] = __builtin_amdgcn_raw_buffer_load_b128(rc, voff, 0, 0);
    }
  };
  prefetch_bv(cs + wave);
  prefetch_c(cs + wave);
  for (int c = cs + wave; c < c1; c += CW) {
    // Lane-dependent offsets are re-derived in each iteration instead of
    // being held in registers across the whole loop.
    set_prio_remaining((c1 - 1 - c) / CW);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int nn = ln & 15, qq = ln >> 4, m4 = ln & 3, hi4 = ln >> 2;

    // ---- this chunk's rows into LDS; fetch the wave's next chunk ----------
    {
      const int wo = 64 * hi4 + 16 * (m4 ^ swz(hi4));  // row 16 i + hi4, granule m4
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(W.b + 1024 * i + wo) = pf[i];
        *reinterpret_cast<u32x4*>(W.v + 1024 * i + wo) = pf[8 + i];
      }
    }
    const float gt = pg, gate_t = pgate;
    if (c + CW < c1) prefetch_bv(c + CW);
    float gam = gt;  // inclusive scan of g over the chunk (lane = token)
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(gam, d);
      if (ln >= d) gam += y;
    }
    W.gam[ln] = gam;
    W.graw[ln] = gt;
    W.gate[ln] = gate_t;
    wave_lds_sync();
    const float gend = W.gam[CC - 1];

    // ---- phase A: the chunk's own contribution to the next state ----------
    // dH = sum_tau (e^{x_63 - x_tau} (.) b_tau) v_tau^T over the chunk.  The
    // keys are first decayed to the end of their own sub-chunk (kept for the
    // output phase), then by the row's decay from there to the chunk's end.
    f32x4 dH[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) dH[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Source row and the byte offsets of value/key columns 16 h + 4 (ln & 3)
    // (h = 0, 1) of the transposing reads; the row's granule permutation is
    // swz(trow0) = swz(4 qq).
    const int trow0 = 4 * qq + (nn >> 2);
    const int tcol0 = 16 * (((ln & 3) >> 1) ^ swz(4 * qq)) + 8 * (ln & 1);
    const int tcol1 = 16 * ((2 + ((ln & 3) >> 1)) ^ swz(4 * qq)) + 8 * (ln & 1);
    bf16x4 bsub[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t0 = 16 * k;
      const float gsub = W.gam[t0 + 15];
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(&W.gam[t0 + 4 * qq]);
      bf16x4 vf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) vf[nt] = lds_read_tr(W.v + (t0 + trow0) * ROWB + (nt ? tcol1 : tcol0));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x4 braw = lds_read_tr(W.b + (t0 + trow0) * ROWB + (mt ? tcol1 : tcol0));
        const float a2r = mt ? a2n1 : a2n0;
        const float f = __builtin_amdgcn_exp2f(a2r * (gend - gsub));
        f32x4 bt, btc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bt[j] = (float)braw[j] * __builtin_amdgcn_exp2f(a2r * (gsub - g4[j]));
          btc[j] = bt[j] * f;
        }
        bsub[k][mt] = pack4(bt);
        const bf16x4 bb = pack4(btc);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) dH[mt][nt] = mma16(bb, vf[nt], dH[mt][nt]);
      }
    }
    // This chunk's c rows into LDS (made visible by the sync below), then
    // the next chunk's c.
    {
      const int wo = 64 * hi4 + 16 * (m4 ^ swz(hi4));
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(W.c + 1024 * i + wo) = pf[4 + i];
    }
    if (c + CW < c1) prefetch_c(c + CW);
    // Per-row decays over each sub-chunk (E_k) and over the chunk (e^{x_63}),
    // one exponential per lane and value.
    float* const ex = W.ex;
    {
      const int srow = ln & 31, k0 = 2 * (ln >> 5);
      const float a2l = L.a2[srow];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = k0 + kk;
        const float gr = k ? W.gam[16 * k - 1] : 0.f;
        ex[k * 32 + srow] = __builtin_amdgcn_exp2f(a2l * (W.gam[16 * k + 15] - gr));
      }
      if (ln < 32) ex[128 + srow] = __builtin_amdgcn_exp2f(a2l * gend);
    }
    wave_lds_sync();
    float ec[8];  // e^{x_63} on the lane's accumulator rows
    {
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(&ex[128 + 4 * qq]);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(&ex[128 + 16 + 4 * qq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ec[j] = e0[j];
        ec[j + 4] = e1[j];
      }
    }

    // ---- entry state: wait for it, pass the next one on -------------------
    wait_ready(&L.ready, c);
    f32x4 hs[2][2];  // state at the start of the current sub-chunk
    {
      const f32x4* src = reinterpret_cast<const f32x4*>(L.state[c & 1]) + ln;
      hs[0][0] = src[0];
      hs[0][1] = src[64];
      hs[1][0] = src[128];
      hs[1][1] = src[192];
    }
    {
      f32x4 hn[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) hn[mt][nt][i] = __builtin_fmaf(ec[4 * mt + i], hs[mt][nt][i], dH[mt][nt][i]);
      if (c + 1 < c1) {
        f32x4* dst = reinterpret_cast<f32x4*>(L.state[(c + 1) & 1]) + ln;
        dst[0] = hn[0][0];
        dst[64] = hn[0][1];
        dst[128] = hn[1][0];
        dst[192] = hn[1][1];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        if (ln == 0) __hip_atomic_store(&L.ready, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else if (write_hT) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.hT[sbase + (16 * mt + 4 * qq + i) * CD + 16 * nt + nn] = hn[mt][nt][i];
      }
    }

    // ---- phase B: outputs, sub-chunk by sub-chunk with the running state ---
    // (a halo chunk only carries the state)
    if (c < c0) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t0 = 16 * k;
      const float gref = k ? W.gam[t0 - 1] : 0.f;
      // Tables for P in fp16, lane -> (token hi4, key rows 8*m4 + j): the
      // per-token decays e^{A_s g_t} (row t at 15 - t) and b (row t in the
      // quarter of its token).
      // The lane keeps its own token's c.  (swz(t0 + hi4) = swz(hi4).)
      h16x2 d[4];
      {
        const int gsw = 16 * (m4 ^ swz(hi4));
        const float gu = W.graw[t0 + hi4];
        h16x8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (_Float16)__builtin_amdgcn_exp2f(a2g[j] * gu);
        *reinterpret_cast<h16x8*>(reinterpret_cast<char*>(W.ta) + 64 * (15 - hi4) + 16 * m4) = x;
        const u32x4 bw = *reinterpret_cast<const u32x4*>(W.b + (t0 + hi4) * ROWB + gsw);
        h16x8 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[2 * j] = (_Float16)bf_lo(bw[j]);
          y[2 * j + 1] = (_Float16)bf_hi(bw[j]);
        }
        *reinterpret_cast<h16x8*>(reinterpret_cast<char*>(W.tb) + tb_row(hi4) + 16 * m4) = y;
        const u32x4 cw = *reinterpret_cast<const u32x4*>(W.c + (t0 + hi4) * ROWB + gsw);
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = h16x2{(_Float16)bf_lo(cw[j]), (_Float16)bf_hi(cw[j])};
      }
      // Qt = c (.) e^{x_t - x_ref}: row t0 + nn, key rows 4 qq + j (Qlo) and
      // 16 + 4 qq + j (Qhi)
      bf16x4 Qlo, Qhi;
      {
        const float gt_n = W.gam[t0 + nn];
        const int sq = swz(nn), h8 = 8 * (qq & 1);
        const u32x2 c0 = *reinterpret_cast<const u32x2*>(W.c + (t0 + nn) * ROWB + 16 * ((qq >> 1) ^ sq) + h8);
        const u32x2 c1 = *reinterpret_cast<const u32x2*>(W.c + (t0 + nn) * ROWB + 16 * ((2 + (qq >> 1)) ^ sq) + h8);
        const float cv[8] = {bf_lo(c0[0]), bf_hi(c0[0]), bf_lo(c0[1]), bf_hi(c0[1]),
                             bf_lo(c1[0]), bf_hi(c1[0]), bf_lo(c1[1]), bf_hi(c1[1])};
        f32x4 lo, hi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lo[j] = cv[j] * __builtin_amdgcn_exp2f(a2s[j] * (gt_n - gref));
          hi[j] = cv[j + 4] * __builtin_amdgcn_exp2f(a2s[j + 4] * (gt_n - gref));
        }
        Qlo = pack4(lo);
        Qhi = pack4(hi);
      }
      // v fragments and the sub-chunk's own write, decayed to its end
      bf16x4 vf[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) vf[nt] = lds_read_tr(W.v + (t0 + trow0) * ROWB + (nt ? tcol1 : tcol0));
      f32x4 dk[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) dk[mt][nt] = mma16(bsub[k][mt], vf[nt], f32x4{0.f, 0.f, 0.f, 0.f});
      wave_lds_sync();  // tables written above are visible to every lane
      // P[t][tau] for t and tau in the same quarter of the sub-chunk (tokens
      // 4 u .. 4 u + 3), tau <= t; lane -> (t = hi4, key rows 8*m4 + j).  The
      // lane walks tau = t, t - 1, t - 2, t - 3 carrying r = c_t (.) prod_{j =
      // tau+1..t} e^{A g_j}: step l multiplies r by the decays of token
      // t - l + 1 and dots it with b_{t - l}, in packed fp16 with fp32
      // accumulation (two rows per dot-product instruction), so every factor
      // stays in [0, 1] however fast a row decays.  Steps that pass the
      // quarter's first token read zero rows of b (and decays of earlier
      // tokens or zero rows, all in [0, 1]); their sums are zero and land in
      // P's columns left of the quarter.  Every lane thus runs the same 4
      // steps, at constant offsets from its own row.
      {
        const char* arow = reinterpret_cast<const char*>(W.tb) - 128 - 64 * hi4 + 16 * m4;  // + 64 l
        const char* brow = reinterpret_cast<const char*>(W.tb) + tb_row(hi4) - 192 + 16 * m4;  // + 64 (3 - l)
        float pt[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          if (l > 0) {
            const h16x8 a = *reinterpret_cast<const h16x8*>(arow + 64 * l);
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] = d[j] * h16x2{a[2 * j], a[2 * j + 1]};
          }
          const h16x8 bq = *reinterpret_cast<const h16x8*>(brow + 64 * (3 - l));
          float acc = dot2_first(h16x2{bq[0], bq[1]}, d[0]);
#pragma unroll
          for (int j = 1; j < 4; ++j) acc = __builtin_amdgcn_fdot2(h16x2{bq[2 * j], bq[2 * j + 1]}, d[j], acc, false);
          pt[l] = acc;
        }
#pragma unroll
        for (int l = 0; l < 4; ++l) {
          pt[l] += dpp_xor1(pt[l]);
          pt[l] += dpp_xor2(pt[l]);
        }
        // the four lanes of a quad hold the same sums; one of them stores
        // P[t][t - l] (bf16, the MFMA operand's precision)
        if (m4 == 0) {
          char* prow = W.p + (PROW + 2) * hi4 + 26;  // + 2 (3 - l): column t - l of row t
#pragma unroll
          for (int l = 0; l < 4; l += 2) {
            const uint32_t w = cvt_pair(pt[l + 1], pt[l]);  // columns t - l - 1, t - l
            *reinterpret_cast<uint16_t*>(prow + 2 * (2 - l)) = (uint16_t)w;
            *reinterpret_cast<uint16_t*>(prow + 2 * (3 - l)) = (uint16_t)(w >> 16);
          }
        }
      }
      // The rest of P on the matrix unit, split at reference tokens so that
      // every factor lies in [0, 1] and the split is exact:
      //   t in 8..15, tau in 0..7 (reference 7), and within each half
      //   t in 4 u' + 4 .. 4 u' + 7, tau in 4 u' .. 4 u' + 3 (reference 4 u' + 3),
      // P[t][tau] = sum_s X[t][s] X[tau][s] with X[x] = c_x (.) e^{x_x - x_r}
      // on the later side of the reference r and b_x (.) e^{x_r - x_x} on
      // the earlier side.  Each product X X^T (16x16x32, fp16 operands) leaves
      // P[t][4 qq + i] in lane (t = nn, qq), the layout of P V's row operand;
      // its entries that do not pair the two sides of one reference are
      // dropped.
      bf16x4 poff;
      {
        f32x4 x8, x4;
#pragma unroll
        for (int lev = 0; lev < 2; ++lev) {
          const int r = lev ? 4 * (nn >> 2 & ~1) + 3 : 7;  // the lane token's reference
          const bool late = lev ? (nn >> 2) & 1 : nn >= 8;
          const float dg = fabsf(W.gam[t0 + nn] - W.gam[t0 + r]);
          const u32x4 raw = *reinterpret_cast<const u32x4*>((late ? W.c : W.b) + (t0 + nn) * ROWB +
                                                            16 * (qq ^ swz(nn)));
          h16x8 xv;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[2 * j] = (_Float16)(bf_lo(raw[j]) * __builtin_amdgcn_exp2f(a2q[2 * j] * dg));
            xv[2 * j + 1] = (_Float16)(bf_hi(raw[j]) * __builtin_amdgcn_exp2f(a2q[2 * j + 1] * dg));
          }
          (lev ? x4 : x8) = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, xv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
        const bool keep8 = nn >= 8 && qq < 2;
        const bool keep4 = ((nn >> 2) & 1) && qq == 2 * (nn >> 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) x8[i] = keep8 ? x8[i] : (keep4 ? x4[i] : 0.f);
        poff = pack4(x8);
      }
      wave_lds_sync();
      // O = Qt H_start + P V, then the epilogue; the output tile is staged
      // in bf16 rows of 32 values whose 16-byte granule g of row t sits at
      // g ^ (2 ((t >> 2) & 1)), for 16-byte stores
      {
        const bf16x4 pa = *reinterpret_cast<const bf16x4*>(W.p + PROW * nn + 32 + 8 * qq);
        const f32x4 gt4 = *reinterpret_cast<const f32x4*>(&W.gate[t0 + 4 * qq]);
        __bf16* const stg = reinterpret_cast<__bf16*>(W.ta);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          // One accumulator through four 16-deep products (key rows
          // 4 qq + j, then 16 + 4 qq + j, then P V for the two parts of P).  Products of one depth
          // only: a 16-deep MFMA that takes a 32-deep MFMA's result as its
          // accumulator a few instructions later can read the register
          // before that result lands.
          f32x4 acc = mma16(Qlo, pack4(hs[0][nt]), f32x4{0.f, 0.f, 0.f, 0.f});
          acc = mma16(Qhi, pack4(hs[1][nt]), acc);
          acc = mma16(pa, vf[nt], acc);
          acc = mma16(poff, vf[nt], acc);
          const int col = 8 * ((2 * nt + (nn >> 3)) ^ (2 * (qq & 1))) + (nn & 7);
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // dh = 0 without the skip term: one form, no lane selects
            y[i] = __builtin_fmaf(dh, (float)vf[nt][i], acc[i]) * gt4[i];
          }
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const uint32_t w = cvt_pair(y[i], y[i + 1]);  // rows 4 qq + i, 4 qq + i + 1
            reinterpret_cast<uint16_t*>(stg)[(4 * qq + i) * CD + col] = (uint16_t)w;
            reinterpret_cast<uint16_t*>(stg)[(4 * qq + i + 1) * CD + col] = (uint16_t)(w >> 16);
          }
        }
      }
      // the state at the next sub-chunk's start
      if (k < 3) {
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(&ex[k * 32 + 4 * qq]);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(&ex[k * 32 + 16 + 4 * qq]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = j < 4 ? e0[j] : e1[j - 4];
          const int mt = j >> 2, i = j & 3;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) hs[mt][nt][i] = __builtin_fmaf(e, hs[mt][nt][i], dk[mt][nt][i]);
        }
      }
      wave_lds_sync();
      {
        const u32x4 ow = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(W.ta) + 64 * hi4 +
                                                          16 * (m4 ^ (2 * ((hi4 >> 2) & 1))));
        const int orow = c * CC + t0 + hi4;
        __builtin_amdgcn_raw_buffer_store_b128(ow, ro, (int)((long)orow * tok_stride) + 16 * m4, 0, 0);
      }
      wave_lds_sync();  // the tables and staging are rewritten next
    }

  }
}

int launch_chunk(const void* v, const void* b, const void* c, const float* g, const float* alog, const float* dskip,
                 const float* gate, const float* h0, const int32_t* cu, void* out, float* hT, int nchain, int T,
                 int H, int nseg, int seg_chunks, hipStream_t s) {
  ChunkParams p;
  p.v = static_cast<const __bf16*>(v);
  p.b = static_cast<const __bf16*>(b);
  p.c = static_cast<const __bf16*>(c);
  p.g = g;
  p.alog = alog;
  p.dskip = dskip;
  p.gate = gate;
  p.h0 = h0;
  p.cu = cu;
  p.out = static_cast<__bf16*>(out);
  p.hT = hT;
  p.T = T;
  p.H = H;
  p.nchain = nchain;
  p.nseg = nseg;
  p.seg_chunks = seg_chunks;
  hipLaunchKernelGGL(diag_chunk_kernel, dim3(nchain * nseg), dim3(64 * CW), 0, s, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" int gdn_diag_fwd_recurrent(const void* v, const void* b, const void* c, const float* g,
                                      const float* A_log, const float* Dskip, const float* gate, const float* h0,
                                      const int32_t* cu_seqlens, void* out, float* hT, int B, int T, int H, int S,
                                      int D, void* stream, int dtype) {
  DShape p;
  const int rc = diag_validate(v, b, c, g, A_log, out, hT, B, T, H, S, D, dtype, &p);
  if (rc != GDN_OK) return rc;
  if (p.nitems == 0) return GDN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == GDN_BF16
             ? dispatch_recurrent<__bf16>(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, p, s)
             : dispatch_recurrent<float>(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, p, s);
}

extern "C" int gdn_diag_fwd(const void* v, const void* b, const void* c, const float* g, const float* A_log,
                            const float* Dskip, const float* gate, const float* h0, const int32_t* cu_seqlens,
                            void* out, float* hT, int B, int T, int H, int S, int D, void* stream, int dtype,
                            int chunk) {
  DShape p;
  const int rc = diag_validate(v, b, c, g, A_log, out, hT, B, T, H, S, D, dtype, &p);
  if (rc != GDN_OK) return rc;
  if (chunk != 0 && chunk != CC) return GDN_ERR_UNSUPPORTED;
  if (dtype != GDN_BF16 || S != CS || D != CD) return GDN_ERR_UNSUPPORTED;
  if ((long)(T + CC) * H * ROWB > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;  // 32-bit buffer offsets
  const long nchain = (long)B * H;
  if (nchain > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  if (nchain == 0) return GDN_OK;
  // Dense batches with fewer chains than two workgroups per CU: segments of
  // at least 4 chunks, about two workgroups per CU (not when hT aliases h0:
  // a segment starting at the sequence start could read h0 after the last
  // segment has overwritten it).
  int nseg = 1, seg_chunks = 0;
  if (!cu_seqlens && !(h0 && static_cast<const void*>(h0) == static_cast<const void*>(hT))) {
    const int nchunks = (T + CC - 1) / CC;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        nchain < 2L * ncu) {
      const int want = (int)(2L * ncu / nchain);
      const int n = want < nchunks / 4 ? want : nchunks / 4;
      if (n >= 2) {
        seg_chunks = (nchunks + n - 1) / n;
        nseg = (nchunks + seg_chunks - 1) / seg_chunks;  // every segment holds a chunk
      }
    }
  }
  if ((long)nchain * nseg > 0x7fffffffL) return GDN_ERR_INVALID_ARG;
  return launch_chunk(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, (int)nchain, T, H, nseg,
                      seg_chunks, static_cast<hipStream_t>(stream));
}
