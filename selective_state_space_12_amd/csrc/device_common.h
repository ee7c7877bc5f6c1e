// Device helpers shared by the gfx950 kernels: storage types, 16-byte vector
// loads/stores with conversion to fp32, and the 16x16 MFMA fragment wrapper.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mmssd {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;  // log2(e), converts exp(v) to exp2(v*log2e)

// SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)), with the hardware exp2 and
// reciprocal (about 1 ulp each): an IEEE division made the conv kernel
// VALU-bound below the HBM rate.  Large |v| saturates correctly (exp2 -> inf,
// rcp(inf) -> 0).  Every kernel that applies the conv uses this one form, so
// a fused conv rounds exactly as the standalone one.
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// softplus(v) = log(1 + exp(v)); above 20 it equals v in fp32.
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(expf(v)); }

// ---- scalar conversions -------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// ---- 16-byte vectors of storage elements --------------------------------
template <typename T> struct Vec16 {
  static constexpr int kN = 16 / sizeof(T);
  T v[kN];
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(r.v) = *reinterpret_cast<const uint4*>(p);
  return r;
}

// For data read exactly once (a streamed input): a nontemporal load.
template <typename T>
__device__ __forceinline__ Vec16<T> load16_once(const T* p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  Vec16<T> r;
  *reinterpret_cast<u32x4_t*>(r.v) = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return r;
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const Vec16<T>& r) {
  *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(r.v);
}

template <typename T>
__device__ __forceinline__ Vec16<T> zero16() {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(r.v) = make_uint4(0u, 0u, 0u, 0u);
  return r;
}

// ---- range-checked stores ------------------------------------------------
// 16 bytes per lane at byte offset `off` of [base, base + bytes), through a
// buffer resource: the hardware drops lanes whose offset lies outside the
// range, so a ragged tail needs no lane-conditional branch.  (A branch around
// a store leaves the store count of later code unknown, and the compiler then
// makes every later wait for a load also wait for all stores.)  Nontemporal:
// data written once.  Offsets are 32-bit: callers keep `bytes` below 2^32.
// Buffer resource over the byte range [addr, addr + bytes), forced uniform
// (it lives in scalar registers; `addr` and `bytes` must be the same in every
// lane).  Loads through it at an offset outside the range return 0 and stores
// there are dropped.  Buffer loads and stores address with a scalar base and
// a 32-bit per-lane offset; on gfx950 they measured ~10% faster than 64-bit
// per-lane global addressing for the scan's mix of shared-fragment loads and
// streamed rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(uint64_t addr, uint32_t bytes) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  const int nb = __builtin_amdgcn_readfirstlane((int)bytes);
  // word 3 of a gfx9 raw buffer resource: 32-bit data format, no swizzle
  return __builtin_amdgcn_make_buffer_rsrc(ub, 0, nb, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, uint32_t bytes) {
  return uniform_rsrc(reinterpret_cast<uint64_t>(base), bytes);
}

// Cache policies of the buffer operations (gfx950): 0 = default, 2 = nontemporal.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyNT = 2;

template <int POLICY>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
}
template <int POLICY>
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POLICY);
}

__device__ __forceinline__ void store16_nt_ranged(void* base, uint32_t bytes, uint32_t off,
                                                  uint4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), uniform_rsrc(base, bytes),
                                         (int)off, 0, kPolicyNT);
}

// ---- MFMA fragments -----------------------------------------------------
// A 16x16 output tile computed from a K=32 slice.  Lane l (0..63) with
// row/col index r = l % 16 and group g = l / 16 holds, for the A operand,
// A[r][g*8 + j] and, for the B operand, B[g*8 + j][r], j = 0..7.  The output
// tile D[m][n] is held as D[g*4 + i][r], i = 0..3.  Any permutation of the 32
// k indices may be used as long as A and B agree on it.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { float v[8]; };

__device__ __forceinline__ f32x4 mma(const Frag8<bf16>& a, const Frag8<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// fp32 operands: eight K=4 MFMAs; step j contracts k-slot j of every group.
__device__ __forceinline__ f32x4 mma(const Frag8<float>& a, const Frag8<float>& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

template <typename T>
__device__ __forceinline__ void frag_set(Frag8<T>& f, int j, float v) {
  f.v[j] = from_f32<T>(v);
}

template <typename T>
__device__ __forceinline__ void frag_zero(Frag8<T>& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = from_f32<T>(0.0f);
}

// Eight consecutive storage elements (16 B for bf16, 32 B for fp32).
template <typename T>
__device__ __forceinline__ void frag_load8(Frag8<T>& f, const T* p) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint4*>(&f.v) = *reinterpret_cast<const uint4*>(p);
  } else {
    *reinterpret_cast<uint4*>(&f.v[0]) = *reinterpret_cast<const uint4*>(p);
    *reinterpret_cast<uint4*>(&f.v[4]) = *reinterpret_cast<const uint4*>(p + 4);
  }
}

// Two runs of four consecutive elements into slots 0..3 and 4..7.
template <typename T>
__device__ __forceinline__ void frag_load4x2(Frag8<T>& f, const T* p0, const T* p1) {
  if constexpr (sizeof(T) == 2) {
    uint2 a = *reinterpret_cast<const uint2*>(p0);
    uint2 b = *reinterpret_cast<const uint2*>(p1);
    uint4 r = make_uint4(a.x, a.y, b.x, b.y);
    *reinterpret_cast<uint4*>(&f.v) = r;
  } else {
    *reinterpret_cast<uint4*>(&f.v[0]) = *reinterpret_cast<const uint4*>(p0);
    *reinterpret_cast<uint4*>(&f.v[4]) = *reinterpret_cast<const uint4*>(p1);
  }
}

__device__ __forceinline__ int clamp_heads(const int32_t* per_seq, int b, int cap) {
  if (!per_seq) return cap;
  int h = per_seq[b];
  return h < 0 ? 0 : (h > cap ? cap : h);
}

}  // namespace mmssd
