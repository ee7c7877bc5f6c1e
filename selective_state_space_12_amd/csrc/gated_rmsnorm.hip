// Gated RMSNorm epilogue over the first d channels of each token row
// ("MatMamba: A Matryoshka State Space Model", block paragraph: the scan
// output is gated by sigma(z) with sigma = SiLU and normalised with Norm =
// RMSNorm; the display equation is lost, and the gate is read as applied
// before the norm, the Mamba2 order):
//   g_c = y_c * SiLU(z_c),  out_c = g_c * w_c / sqrt(mean_{c<d} g_c^2 + eps)
// With a Matryoshka slice, d = d_i = h_i * d_head and w is the prefix w[0:d_i]
// (the norm over d_i is why sub-block outputs are not a prefix of the full
// block's after this step).
//
// HBM-bound (3 * d * s bytes per token, s = element size): 256-thread
// workgroups, 16-byte loads and stores, the row's gated values kept in
// registers between the sum of squares and the scaling (up to 4 chunks of 8
// per thread; wider rows recompute the gate in a second pass).  Rows of up
// to 1024 values take one wave each (four rows per workgroup, a wave-only
// sum), wider rows a whole workgroup.
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kNormThreads = 256;
constexpr int kMaxCached = 4;  // at most this many chunks of 8 values held per thread

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const Vec16<T> a = load16(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = to_f32(a.v[j]);
  } else {
    const Vec16<T> a = load16(p), b = load16(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = to_f32(a.v[j]);
      v[j + 4] = to_f32(b.v[j]);
    }
  }
}

// Eight storage elements as raw 16-byte words (one for bf16, two for fp32),
// so that several rows' loads can be issued before any value is converted.
struct Raw8 {
  uint4 a, b;
};

template <typename T>
__device__ __forceinline__ Raw8 load8raw(const T* p) {
  Raw8 r;
  r.a = *reinterpret_cast<const uint4*>(p);
  if constexpr (sizeof(T) == 4) r.b = *reinterpret_cast<const uint4*>(p + 4);
  else r.b = r.a;
  return r;
}

template <typename T>
__device__ __forceinline__ void raw8f(const Raw8& r, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    // a bf16 is the high half of its fp32
    const unsigned w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __builtin_bit_cast(float, w[j] << 16);
      v[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
    }
  } else {
    v[0] = __builtin_bit_cast(float, r.a.x);
    v[1] = __builtin_bit_cast(float, r.a.y);
    v[2] = __builtin_bit_cast(float, r.a.z);
    v[3] = __builtin_bit_cast(float, r.a.w);
    v[4] = __builtin_bit_cast(float, r.b.x);
    v[5] = __builtin_bit_cast(float, r.b.y);
    v[6] = __builtin_bit_cast(float, r.b.z);
    v[7] = __builtin_bit_cast(float, r.b.w);
  }
}

template <typename T>
__device__ __forceinline__ void store8f(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    Vec16<T> a;
#pragma unroll
    for (int j = 0; j < 8; ++j) a.v[j] = from_f32<T>(v[j]);
    store16(p, a);
  } else {
    Vec16<T> a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a.v[j] = from_f32<T>(v[j]);
      b.v[j] = from_f32<T>(v[j + 4]);
    }
    store16(p, a);
    store16(p + 4, b);
  }
}

// kRT threads per row (64, 128 or 256), each holding kCached chunks of 8
// values in registers between the sum of squares and the scaled write; a
// row longer than kRT * kCached chunks reloads the rest.
template <typename T, int kRT, int kCached>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(
    const T* __restrict__ y, int64_t ys, const T* __restrict__ z, int64_t zs,
    const float* __restrict__ w, float eps, T* out, int64_t os, int d, int64_t rows) {
  __shared__ float red[kNormThreads / 64];
  const int64_t r = (int64_t)blockIdx.x * (kNormThreads / kRT) + threadIdx.x / kRT;
  if (kRT == 64 && r >= rows) return;  // whole wave; no workgroup barrier below
  // (wider rows share a barrier: a row past the end only skips its memory)
  const int nch = r < rows ? d / 8 : 0;
  // a row past the end reads the last row (its values are never used)
  const int64_t rc = r < rows ? r : rows - 1;
  const T* yr = y + rc * ys;
  const T* zr = z + rc * zs;
  T* orow = out + r * os;
  const int tid = threadIdx.x % kRT;
  float g[kCached][8];
  float ss = 0.0f;
  auto gate = [&](int ch, float (&gv)[8]) {
    float yv[8], zv[8];
    load8f(yr + ch * 8, yv);
    load8f(zr + ch * 8, zv);
#pragma unroll
    for (int j = 0; j < 8; ++j) gv[j] = yv[j] * silu(zv[j]);
  };
  {
    // The cached chunks' loads are issued together, unconditionally at a
    // clamped chunk index, and masked afterwards: a load under a lane
    // condition is waited for at the end of its branch, which serialised
    // them.
    const int last = d / 8 - 1;
    Raw8 ry[kCached], rz[kCached];
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
      const int ch = min(tid + i * kRT, last);
      ry[i] = load8raw(yr + ch * 8);
      rz[i] = load8raw(zr + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < kCached; ++i) {
      float yv[8], zv[8];
      raw8f<T>(ry[i], yv);
      raw8f<T>(rz[i], zv);
      const bool live = tid + i * kRT < nch;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        g[i][j] = live ? yv[j] * silu(zv[j]) : 0.0f;
        ss = fmaf(g[i][j], g[i][j], ss);
      }
    }
  }
  for (int ch = tid + kCached * kRT; ch < nch; ch += kRT) {
    float gv[8];
    gate(ch, gv);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(gv[j], gv[j], ss);
  }
  // sum over the row: butterfly within each wave, then (256 threads per row)
  // the 4 wave partials
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  float tot = ss;
  if (kRT > 64) {
    const int w0 = (threadIdx.x / kRT) * (kRT / 64);  // this row's first wave slot
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    tot = red[w0];
#pragma unroll
    for (int k = 1; k < kRT / 64; ++k) tot += red[w0 + k];
  }
  const float inv = rsqrtf(tot / (float)d + eps);
  auto emit = [&](int ch, const float (&gv)[8]) {
    const float4 w0 = *reinterpret_cast<const float4*>(w + ch * 8);
    const float4 w1 = *reinterpret_cast<const float4*>(w + ch * 8 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = gv[j] * inv * wv[j];
    store8f(orow + ch * 8, o);
  };
#pragma unroll
  for (int i = 0; i < kCached; ++i) {
    const int ch = tid + i * kRT;
    if (ch < nch) emit(ch, g[i]);
  }
  for (int ch = tid + kCached * kRT; ch < nch; ch += kRT) {
    float gv[8];
    gate(ch, gv);
    emit(ch, gv);
  }
}

template <typename T, int kRT, int kCached>
void launch_rt(const NormArgs& a, hipStream_t s) {
  static_assert(kCached >= 1 && kCached <= kMaxCached, "chunks held per thread");
  constexpr int kRows = kNormThreads / kRT;
  const dim3 grid((unsigned)((a.rows + kRows - 1) / kRows));
  hipLaunchKernelGGL((gated_rmsnorm_kernel<T, kRT, kCached>), grid, dim3(kNormThreads), 0, s,
                     static_cast<const T*>(a.y), a.ys, static_cast<const T*>(a.z), a.zs, a.w, a.eps,
                     static_cast<T*>(a.out), a.os, (int)a.d, a.rows);
}

}  // namespace

template <typename T>
void launch_typed(const NormArgs& a, hipStream_t s) {
  // Threads per row and chunks per thread sized to the row, so that every
  // cached load a thread issues is one the row needs (the loads are issued
  // unconditionally; with more slots than chunks they would repeat the
  // last chunk and crowd the memory pipeline).
  // Measured at 32768 rows: one wave per row up to d = 1024 (1024: 0.072 ms
  // against 0.079 with 256 threads, half of them idle), four waves per row
  // from there (2048: one wave holding 4 chunks took 0.106 ms against 0.101).
  const int64_t nch = a.d / 8;
  if (nch <= 64) launch_rt<T, 64, 1>(a, s);
  else if (nch <= 128) launch_rt<T, 64, 2>(a, s);
  else if (nch <= 256) launch_rt<T, kNormThreads, 1>(a, s);
  else if (nch <= 512) launch_rt<T, kNormThreads, 2>(a, s);
  else launch_rt<T, kNormThreads, kMaxCached>(a, s);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, int dtype, hipStream_t s) {
  if (dtype == MM_BF16) launch_typed<bf16>(a, s);
  else launch_typed<float>(a, s);
  return hipGetLastError();
}

}  // namespace mmssd
