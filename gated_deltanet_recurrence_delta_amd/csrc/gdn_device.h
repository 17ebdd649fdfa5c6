// Device-side building blocks shared by the gated-delta-rule kernels of
// this library (gfx950): MFMA operand traits, LDS helpers, cross-lane
// scans, buffer descriptors and LDS flags.  Internal header: every
// definition sits in an unnamed namespace of the including file.
#ifndef GDN_DEVICE_H
#define GDN_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
  // Half-depth product: the same lane pairing as mma() restricted to the
  // first four positions of each lane group (for operands whose other half
  // is zero).  Its accumulator never comes from a full-depth product: the
  // compiler inserts no wait states between the two shapes, and a
  // half-depth MFMA issued two instructions after a full-depth one read its
  // accumulator register before the result had landed.  Mixed sums keep one
  // accumulator per depth and add them on the VALU.
  __device__ static inline f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0,
                                                     0);
  }
  __device__ static inline bf16x4 lo(frag f) { return bf16x4{f[0], f[1], f[2], f[3]}; }
  __device__ static inline bf16x4 hi(frag f) { return bf16x4{f[4], f[5], f[6], f[7]}; }
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

// ------------------------------------------------------------ cross-lane

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane
// row with DPP row shifts, then the row totals are added across rows.  The
// order of additions is fixed, so every call gives the same bits.
__device__ static inline float wave_prefix_sum(float x, int lane) {
  // DPP row_shr:n is control code 0x110 + n; lanes shifted in from outside
  // the row read 0 (bound_ctrl).
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const float off = lane < 16 ? 0.f : (lane < 32 ? r0 : (lane < 48 ? r0 + r1 : (r0 + r1) + r2));
  return x + off;
}

// Barrier that orders LDS only.  Waves share nothing through global memory
// inside the kernel, so outstanding global loads and stores may stay in
// flight across it.
__device__ static inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Transposing LDS read (gfx950): within each 16-lane group, destination
// lane i, element k receives element (i & 3) of the 8 bytes addressed by
// source lane (i >> 2) + 4k.
__device__ static inline bf16x4 lds_read_tr(const char* base, int off) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) char*)(base + off));
  return __builtin_bit_cast(bf16x4, r);
}

// A segment's workgroup starts its recurrence from a zero state at the
// latest chunk boundary behind the segment from which the product of the
// per-token transition norms, alpha_t max(1, |1 - beta_t |k_t|^2|), is at
// most e^-HALO_NATS (or at the sequence start, from h0).  Each token's
// transition M -> alpha (I - beta k k^T) M has spectral norm alpha
// max(1, |1 - beta |k|^2|), so the state the segment starts from differs
// from the exact one by at most e^-HALO_NATS times the exact state's norm
// at the halo's start.  Outputs of the halo's chunks are not stored.
constexpr float HALO_NATS = 40.f;

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give
// each XCD a contiguous range of work items, so that neighbouring items
// (for instance the value tiles of one chain, which re-read the same q/k)
// share that XCD's L2.
__device__ static inline int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int q = n >> 3, r = n & 7;
  return xcd * q + (xcd < r ? xcd : r) + slot;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Granule permutation of a q/k row (GR granules of 16 bytes).  LDS has 64
// banks of 4 bytes (a 256-byte period).  A 16-byte read is served 16 lanes
// at a time: the lanes that agree in lane bit 5 and in the parity of lane
// bits 2..4.  An 8-byte (plain or transposing) read is served 32 lanes at a
// time: the lanes that agree in lane bit 5.  For 256-byte rows the
// permutation below puts each such group of a fragment read (16 rows, one
// granule each) and of a state wave's transposing read (8 rows, four
// 8-byte pieces each, alternating halves) on distinct banks.
template <int GR>
__device__ static inline int swz_kq(int r) {
  if constexpr (GR >= 16) return 8 * (r & 1) + 4 * ((r >> 1) & 1) + 3 * ((r >> 2) & 1);
  else if constexpr (GR >= 8) return 2 * (r & 3) + ((r >> 2) & 1);
  else return (r >> 1) & 3;  // two 64-byte rows share a 128-byte bank line
}

template <int C>
__device__ static inline int swz_cc(int r) {
  if constexpr (C == 64) return r & 7;
  else return (r >> 1) & 3;
}

template <int N>
struct IC {
  static constexpr int value = N;
};

// Wait until the LDS word `f` holds at least v.  The read is issued from
// inline assembly so that the compiler does not make it wait for this
// wave's outstanding copies into LDS (which never touch the flag).  The
// wait is bounded: every producer releases its flag unconditionally, so
// the bound is never reached in a correct kernel, and if a defect ever
// left a flag unset the wave would go on (with wrong results) instead of
// holding the GPU.
constexpr unsigned FLAG_SPIN_MAX = 1u << 24;
__device__ static inline void flag_wait_lds(const int* f, int v) {
  const unsigned addr = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) int*)f;
  for (unsigned spin = 0; spin < FLAG_SPIN_MAX; ++spin) {
    int x;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
    if (__builtin_amdgcn_readfirstlane(x) >= v) break;
  }
}

// Make v's value exist at this point of the instruction stream: the work
// that produces it is then done before, not after, a following wait.
template <typename T>
__device__ static inline void settle(T& v) {
  asm volatile("" : "+v"(v));
}

__device__ static inline void flag_release(int* f, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// 16 bytes per lane from the buffer at byte offset voff into LDS at
// lds + 16 * lane.  (Kept out of the kernel body: the host compilation pass
// does not accept this builtin inside a kernel and would drop its stub.)
__device__ static inline void copy_to_lds(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// 4 bytes per lane from the buffer at byte offset voff into LDS at
// lds + 4 * lane.
__device__ static inline void copy_to_lds4(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (and nothing else).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ static inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Four values to bf16 (round to nearest even) as two packed pair
// conversions.  (A vector built element by element, or a four-element
// vector conversion feeding a bit cast, is converted a value at a time and
// merged with permutes.)
__device__ static inline uint32_t cvt_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ static inline bf16x4 cvt4(f32x4 v) {
  return __builtin_bit_cast(bf16x4, u32x2{cvt_pair(v[0], v[1]), cvt_pair(v[2], v[3])});
}

// Raw buffer descriptor over [base, base + bytes); accesses at or past the
// end read zero and write nothing.
__device__ static inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffffL ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <typename V>
__device__ static inline V lds_ld(const char* base, int off) {
  return *reinterpret_cast<const V*>(base + off);
}
template <typename V>
__device__ static inline void lds_st(char* base, int off, V v) {
  *reinterpret_cast<V*>(base + off) = v;
}
template <typename V>
__device__ static inline V lds_at(const char* p) { return *reinterpret_cast<const V*>(p); }

}  // namespace

#endif  // GDN_DEVICE_H
