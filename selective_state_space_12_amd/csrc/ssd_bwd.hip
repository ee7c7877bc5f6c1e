// Chunked selective scan (SSD) backward over the first `heads` heads.
//
// "MatMamba: A Matryoshka State Space Model", training paragraph: the nested
// granularities are trained jointly, one forward pass per granularity with
// the gradients of the shared weights accumulated, and a single backward
// pass; a sub-block uses A[0:h_i] and the first h_i heads of x (nesting
// paragraph).  This file is the backward pass of the scan of one granularity:
// given the cotangents dy (and dhT of the final state) it produces dx, ddt,
// dA, dB, dC, dD and dh0 of L = sum dy.y + sum dhT.h_final, and can add them
// into existing gradients so that the granularities' passes accumulate.
//
// Chunk algebra (chunk of Q tokens, Lambda_t = sum_{r<=t} dt_r A inclusive,
// e = last token, Gc = dL/dH at the chunk's end, Hp = state before it):
//   g_s   = sum_{t>=s} exp(Lambda_t - Lambda_s) dy_t C_t^T + exp(Lambda_e - Lambda_s) Gc
//           (dL/dH_s, never formed; every term below is a product with it)
//   u_s   = g_s B_s = sum_{t>=s} exp(..)(C_t . B_s) dy_t + exp(..) Gc B_s        (P)
//   dx_s  = dt_s u_s + D dy_s,     ddt_s = x_s . u_s + A da_s
//   dB_s  = dt_s g_s^T x_s = dt_s [sum_{t>=s} exp(..)(dy_t . x_s) C_t + exp(..) Gc^T x_s]
//   dC_t  = h_t^T dy_t = exp(Lambda_t) Hp^T dy_t + sum_{s<=t} exp(..) dt_s (dy_t . x_s) B_s
//   dGp   = exp(Lambda_e) Gc + sum_t exp(Lambda_t) dy_t C_t^T       (carried to the chunk before)
// and, differentiating the exponents, dLambda_t =
//     exp(Lambda_t) dy_t . Hp C_t                                  (off-diagonal output)
//   + sum_{s<=t} W[t,s] - sum_{t'>=t} W[t',t]                      (diagonal block)
//   - dt_t exp(Lambda_e - Lambda_t) x_t^T Gc B_t + [t = e] <Gc, H_e> (the chunk's end state)
// with W[t,s] = exp(Lambda_t - Lambda_s)(C_t . B_s) dt_s (dy_t . x_s); then
// da_r = sum_{t>=r} dLambda_t, ddt_r gets A da_r, dA_h = sum_r dt_r da_r.
//
// MI355X design (gfx950, 64-wide waves, 16x16x32 bf16 / 16x16x4 fp32 MFMA):
//  - bwd_state_kernel: one workgroup per (sequence, head) walks the chunks
//    forward with the fp32 state in MFMA accumulators and stores the state
//    before every chunk (and the final one) in the storage type to the
//    workspace: the backward walk needs them in reverse order.
//  - bwd_chunk_kernel: one workgroup of 8 waves per (sequence, head) walks the
//    chunks backwards with dL/dH (P x N fp32) in accumulators.  Per chunk the
//    x, dy, B, C rows are staged in LDS in token-major form plus the
//    transposed copies the K = token products need, Hp (from the workspace)
//    and the bf16/fp32 operand copies of Gc.  Waves 0-3 own one 16-token
//    s-block each (dx, dB, the column sums of W), waves 4-7 one 16-token
//    t-block each (dC, the first dLambda term); the causal work of an
//    s-block grows as that of the matching t-block shrinks, and wave w and
//    w+4 share a SIMD.  Every wave updates its tiles of dL/dH.  The Q x Q
//    products are formed transposed where needed so that their accumulators
//    are directly the A operand of the next product (the masked decay applied
//    in registers), as in the forward kernel.
//  - dB and dC are sums over heads: fp32 atomics into the caller's buffers
//    (zeroed by a fill kernel unless the call accumulates); dA and dD are sums
//    over sequences, one atomic per workgroup.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kBQ = 64;  // tokens per backward chunk
constexpr int kBWaves = 8;
constexpr int kBThreads = kBWaves * 64;
constexpr int kXcds = 8;

struct BwdK {
  const void* x;
  int64_t xs;
  const void* dt;
  int64_t dts;
  const float* A;
  const void* B;
  int64_t bs;
  const void* C;
  int64_t cs;
  const float* D;
  const float* h0;
  const void* dy;
  int64_t dys;
  const float* dhT;
  void* dx;
  int64_t dxs;
  void* ddt;
  int64_t ddts;
  float* dA;
  float* dB;
  int64_t dbs;
  float* dC;
  int64_t dcs;
  float* dD;
  float* dh0;
  void* hst;  // (batch, heads, nchunks + 1, P, N) storage type
  // sequence split (nseg > 1): per (unit, segment) fp32 P x N blocks and
  // log2 decays; see the launch for what each holds when
  float* seg_h;
  float* seg_hd;
  float* seg_g;
  float* seg_gd;
  int64_t seqlen;
  int n_heads, heads, nchunks, accumulate;
  int nseg, seg_chunks;
};

template <typename T> constexpr int bpad() { return 16 / (int)sizeof(T); }

// (sequence, head) of this workgroup: consecutive units on one XCD so that
// the heads of a sequence share its B and C rows in that XCD's L2.
// With nsk segments per unit in the grid (segment fastest), *seg is this
// workgroup's segment among them.
__device__ __forceinline__ void unit_of_idx(int pid, int total, int heads, int nsk, int* b, int* h,
                                            int* seg) {
  const int uid = total % kXcds == 0 ? (pid % kXcds) * (total / kXcds) + pid / kXcds : pid;
  const int unit = uid / nsk;
  *seg = uid % nsk;
  *b = unit / heads;
  *h = unit % heads;
}

__device__ __forceinline__ void unit_of(int heads, int nsk, int* b, int* h, int* seg) {
  unit_of_idx(blockIdx.x, gridDim.x, heads, nsk, b, h, seg);
}

// Eight consecutive elements at p[k0..k0+7] when k0 < K, else zeros.
template <typename T>
__device__ __forceinline__ void frag_row(Frag8<T>& f, const T* p, int k0, int K) {
  if (k0 < K) frag_load8(f, p + k0);
  else frag_zero(f);
}

// Same, every element multiplied by s.
template <typename T>
__device__ __forceinline__ void frag_row_scaled(Frag8<T>& f, const T* p, int k0, int K, float s) {
  if (k0 < K) {
    Frag8<T> r;
    frag_load8(r, p + k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) frag_set(f, j, to_f32(r.v[j]) * s);
  } else {
    frag_zero(f);
  }
}

// Sum over the 16 lanes of a DPP row (lanes 16r..16r+15), in every lane of
// the row: rotate-and-add by 8 and 4 within the row, then quad swaps of 2
// and 1.  Four VALU adds with DPP operands instead of four LDS permutes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                               0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0x128>(v);  // row_ror:8
  v += dpp_f32<0x124>(v);  // row_ror:4
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  return v;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                               kRowMask, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// within each row of 16 (a lane whose source is outside its row adds 0),
// then rows 1 and 3 add lane 15 of the row before and rows 2 and 3 add lane
// 31 (the running total of rows 0-1).  Six DPP adds, no LDS permutes.
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += dpp_rows<0x111, 0xF>(v);  // row_shr:1
  v += dpp_rows<0x112, 0xF>(v);  // row_shr:2
  v += dpp_rows<0x114, 0xF>(v);  // row_shr:4
  v += dpp_rows<0x118, 0xF>(v);  // row_shr:8
  v += dpp_rows<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_rows<0x143, 0xC>(v);  // row_bcast:31
  return v;
}

// Inclusive cumsum of dt*A*log2(e) over the chunk (wave 0, one token per
// lane; tokens >= len take dt = 0 so Lambda stays at its end value).
__device__ __forceinline__ float chunk_cumsum(float a, int) { return wave_incl_scan(a); }

// Four consecutive storage elements (8 bytes of bf16, 16 of fp32).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    const bf16 v[4] = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(v);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&o)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = __builtin_bit_cast(float, u.x << 16);
    o[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
    o[2] = __builtin_bit_cast(float, u.y << 16);
    o[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
  }
}

template <typename T, int P, int N>
struct StateLds {
  static constexpr int TQ = kBQ + bpad<T>();  // pitch of the transposed x and B rows
  static constexpr size_t bytes = (size_t)(P + N) * TQ * sizeof(T) + 2 * kBQ * sizeof(float);
};

// Forward walk storing the state before every chunk and the final state.
// With the sequence split, PRE walks segments 0..nseg-2 from a zero state and
// writes each one's end state and log2 decay (seg_h, seg_hd); the main walk
// of segment s > 0 then starts from the combined state in seg_h slot s-1.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Returns v unchanged, but the compiler can no longer see where it came
// from.  Values loaded ahead pass through it where they are used, so that
// unpacking or converting them is not moved up to their load: work placed
// there makes the wave wait for the load at once, and loading ahead is lost.
template <typename V> __device__ __forceinline__ V opaque(V v) {
  if constexpr (sizeof(V) == 2) {
    unsigned u = __builtin_bit_cast(unsigned short, v);
    asm volatile("" : "+v"(u));
    return __builtin_bit_cast(V, static_cast<unsigned short>(u));
  } else {
    asm volatile("" : "+v"(v));
    return v;
  }
}

template <typename T, int P, int N, bool PRE>
__device__ __forceinline__ void state_walk(const BwdK& k, int pid, int total) {
  using L = StateLds<T, P, N>;
  constexpr int Q = kBQ, TQ = L::TQ;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= kBWaves ? NTILE / kBWaves : 1;
  static_assert(NTILE < kBWaves || NTILE % kBWaves == 0, "state tiles must split evenly");
  static_assert(TP % TPW == 0, "a wave's state tiles share one column block");
  constexpr int VB = 16 / (int)sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];
  T* XT = reinterpret_cast<T*>(smem);
  T* BT = XT + P * TQ;
  float* lam = reinterpret_cast<float*>(BT + N * TQ);
  float* wsc = lam + Q;

  int b, h, seg;
  unit_of_idx(pid, total, k.heads, PRE ? k.nseg - 1 : k.nseg, &b, &h, &seg);
  const int64_t unit = (int64_t)b * k.heads + h;
  const int c0 = seg * k.seg_chunks, c1 = min(c0 + k.seg_chunks, k.nchunks);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;
  const T* __restrict__ Xp = static_cast<const T*>(k.x);
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const T* __restrict__ Bp = static_cast<const T*>(k.B);
  T* __restrict__ Hst = static_cast<T*>(k.hst) + unit * (k.nchunks + 1) * (P * N);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah2 = k.A[h] * kLog2e;

  const int tile0 = wave * TPW;
  const bool owns = NTILE >= kBWaves || tile0 < NTILE;  // every wave when tiles >= waves
  const int nt = tile0 / TP, pt0 = tile0 % TP;
  f32x4 hacc[TPW];
  const float* hin = PRE ? nullptr
                     : seg > 0 ? k.seg_h + (unit * k.nseg + seg - 1) * (P * N)
                     : k.h0 ? k.h0 + ((int64_t)b * k.n_heads + h) * (P * N)
                            : nullptr;
  float lam_seg = 0.0f;  // log2 decay over the walked chunks
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hacc[t][i] = (hin && owns) ? hin[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] : 0.0f;
  // the start state's loads complete here, before any chunk is loaded ahead
#pragma unroll
  for (int t = 0; t < TPW; ++t) hacc[t] = opaque(hacc[t]);

  auto store_state = [&](int c) {
    if (PRE || !owns) return;
    T* dst = Hst + (int64_t)c * (P * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] = from_f32<T>(hacc[t][i]);
  };

  // The x, B rows and dt of the chunk two ahead are loaded into registers
  // while this chunk's update runs (two register sets, used alternately; a
  // thread's vector slots are fixed, so a chunk's loads are all in flight at
  // once and have two chunks of time to land).
  constexpr int NXV = (Q * (P / VB) + kBThreads - 1) / kBThreads;
  constexpr int NBV = (Q * (N / VB) + kBThreads - 1) / kBThreads;
  u32x4 px[2][NXV], pb[2][NBV];
  T pdt[2];
  int plen[2] = {0, 0};
  auto prefetch = [&](int c, auto set) {
    constexpr int S = decltype(set)::value;
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
    // Every load is issued unconditionally at a clamped address and the
    // rows past the end are zeroed afterwards: a load under a lane condition
    // is followed by a wait for it at the branch's end, which serialises
    // the whole batch.
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (P / VB) - 1), s = idx % Q;
      const int p0 = (idx / Q) * VB;
      px[S][v] = *reinterpret_cast<const u32x4*>(Xp + (row0 + min(s, len - 1)) * k.xs + (int64_t)h * P + p0);
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (N / VB) - 1), s = idx % Q;
      const int n0 = (idx / Q) * VB;
      pb[S][v] = *reinterpret_cast<const u32x4*>(Bp + (row0 + min(s, len - 1)) * k.bs + n0);
    }
    pdt[S] = DTp[(row0 + min(lane, len - 1)) * k.dts + h];
    plen[S] = len;
  };
  auto step = [&](int c, auto set) {
    constexpr int S = decltype(set)::value;
    store_state(c);
    // x^T and B^T: consecutive lanes take consecutive tokens (distinct banks)
    const int len = plen[S];
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, p0 = (idx / Q) * VB;
      const u32x4 raw = opaque(px[S][v]);
      Vec16<T> xv;
      *reinterpret_cast<u32x4*>(xv.v) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
      if (idx < Q * (P / VB))
#pragma unroll
        for (int j = 0; j < VB; ++j) XT[(p0 + j) * TQ + s] = xv.v[j];
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, n0 = (idx / Q) * VB;
      const u32x4 raw = opaque(pb[S][v]);
      Vec16<T> bv;
      *reinterpret_cast<u32x4*>(bv.v) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
      if (idx < Q * (N / VB))
#pragma unroll
        for (int j = 0; j < VB; ++j) BT[(n0 + j) * TQ + s] = bv.v[j];
    }
    if (wave == 0) {
      const float d = lane < len ? to_f32(opaque(pdt[S])) : 0.0f;
      const float lv = chunk_cumsum(d * Ah2, lane);
      const float le = __shfl(lv, 63);
      lam[lane] = lv;
      wsc[lane] = __builtin_amdgcn_exp2f(le - lv) * d;
    }
    __syncthreads();
    // issued on every step (the last two reload the final chunk) so that the
    // loop has one path and each load is waited for exactly where it is used
    prefetch(min(c + 2, c1 - 1), set);
    lam_seg += lam[Q - 1];
    if (owns) {
      const float dec = __builtin_amdgcn_exp2f(lam[Q - 1]);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) hacc[t][i] *= dec;
#pragma unroll
      for (int ks = 0; ks < Q / 32; ++ks) {
        const int s0 = ks * 32 + g * 8;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wsc + s0);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wsc + s0 + 4);
        Frag8<T> bf;
        frag_load8(bf, BT + (nt * 16 + r16) * TQ + s0);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> xr, xf;
          frag_load8(xr, XT + ((pt0 + t) * 16 + r16) * TQ + s0);
#pragma unroll
          for (int j = 0; j < 8; ++j) frag_set(xf, j, to_f32(xr.v[j]) * (j < 4 ? w0[j] : w1[j - 4]));
          hacc[t] = mma(xf, bf, hacc[t]);
        }
      }
    }
    __syncthreads();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // c1 - 1 is a valid chunk whenever there is one (c1 = min(c0 + seg_chunks,
  // nchunks) and nchunks >= 1), so the clamped loads stay in bounds
  prefetch(min(c0, c1 - 1), S0{});
  prefetch(min(c0 + 1, c1 - 1), S1{});
  int c = c0;
  for (; c + 1 < c1; c += 2) {
    step(c, S0{});
    step(c + 1, S1{});
  }
  if (c < c1) step(c, S0{});
  if (PRE) {
    float* dst = k.seg_h + (unit * k.nseg + seg) * (P * N);
    if (owns)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] = hacc[t][i];
    if (tid == 0) k.seg_hd[unit * k.nseg + seg] = lam_seg;
  } else if (c1 == k.nchunks) {
    store_state(k.nchunks);
  }
}

template <typename T, int P, int N>
__global__ __launch_bounds__(kBThreads) void bwd_state_kernel(BwdK k) {
  state_walk<T, P, N, false>(k, blockIdx.x, gridDim.x);
}

// Reverse prepass of the sequence split: segments 1..nseg-1 walk their
// chunks backwards from dL/dH = 0 at their end with the dL/dH update alone
// (dGp = exp(Lambda_e) Gc + sum_t exp(Lambda_t) dy_t C_t^T) and write the
// result at their start and their log2 decay (seg_g, seg_gd).
template <typename T, int P, int N>
__device__ __forceinline__ void gprep_walk(const BwdK& k, int pid, int total) {
  using L = StateLds<T, P, N>;
  constexpr int Q = kBQ, TQ = L::TQ;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= kBWaves ? NTILE / kBWaves : 1;
  constexpr int VB = 16 / (int)sizeof(T);
  constexpr int NYV = (Q * (P / VB) + kBThreads - 1) / kBThreads;
  constexpr int NCV = (Q * (N / VB) + kBThreads - 1) / kBThreads;
  extern __shared__ __align__(16) unsigned char smem[];
  T* YT = reinterpret_cast<T*>(smem);  // dy^T [P][TQ]
  T* CT = YT + P * TQ;                 // C^T [N][TQ]
  float* lam = reinterpret_cast<float*>(CT + N * TQ);
  float* eL = lam + Q;

  int b, h, sg;
  unit_of_idx(pid, total, k.heads, k.nseg - 1, &b, &h, &sg);
  const int seg = sg + 1;
  const int64_t unit = (int64_t)b * k.heads + h;
  const int c0 = seg * k.seg_chunks, c1 = min(c0 + k.seg_chunks, k.nchunks);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;
  const T* __restrict__ DYp = static_cast<const T*>(k.dy);
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const T* __restrict__ Cp = static_cast<const T*>(k.C);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah2 = k.A[h] * kLog2e;
  const int tile0 = wave * TPW;
  const bool owns = NTILE >= kBWaves || tile0 < NTILE;  // every wave when tiles >= waves
  const int nt = tile0 / TP, pt0 = tile0 % TP;
  f32x4 gacc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) gacc[t] = f32x4{0, 0, 0, 0};
  float lam_seg = 0.0f;
  // As in the forward state walk: dy, C rows and dt of the chunk two behind
  // (in walk order) are loaded while this chunk runs, into two register sets
  // used alternately, and pass through opaque() where they are used.
  u32x4 py[2][NYV], pc[2][NCV];
  T pdt[2];
  int plen[2];
  auto prefetch = [&](int c, auto set) {
    constexpr int S = decltype(set)::value;
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
#pragma unroll
    for (int v = 0; v < NYV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (P / VB) - 1), s = min(idx % Q, len - 1);
      py[S][v] = *reinterpret_cast<const u32x4*>(DYp + (row0 + s) * k.dys + (int64_t)h * P + (idx / Q) * VB);
    }
#pragma unroll
    for (int v = 0; v < NCV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (N / VB) - 1), s = min(idx % Q, len - 1);
      pc[S][v] = *reinterpret_cast<const u32x4*>(Cp + (row0 + s) * k.cs + (idx / Q) * VB);
    }
    pdt[S] = DTp[(row0 + min(lane, len - 1)) * k.dts + h];
    plen[S] = len;
  };
  auto step = [&](int c, auto set) {
    constexpr int S = decltype(set)::value;
    const int len = plen[S];
#pragma unroll
    for (int v = 0; v < NYV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, p0 = (idx / Q) * VB;
      const u32x4 raw = opaque(py[S][v]);
      Vec16<T> yv;
      *reinterpret_cast<u32x4*>(yv.v) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
      if (idx < Q * (P / VB))
#pragma unroll
        for (int j = 0; j < VB; ++j) YT[(p0 + j) * TQ + s] = yv.v[j];
    }
#pragma unroll
    for (int v = 0; v < NCV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, n0 = (idx / Q) * VB;
      const u32x4 raw = opaque(pc[S][v]);
      Vec16<T> cv;
      *reinterpret_cast<u32x4*>(cv.v) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
      if (idx < Q * (N / VB))
#pragma unroll
        for (int j = 0; j < VB; ++j) CT[(n0 + j) * TQ + s] = cv.v[j];
    }
    if (wave == 0) {
      const float d = lane < len ? to_f32(opaque(pdt[S])) : 0.0f;
      const float lv = chunk_cumsum(d * Ah2, lane);
      lam[lane] = lv;
      eL[lane] = __builtin_amdgcn_exp2f(lv);
    }
    __syncthreads();
    // issued on every step, clamped at the segment's first chunk
    prefetch(max(c - 2, c0), set);
    lam_seg += lam[Q - 1];
    if (owns) {
      const float dec = __builtin_amdgcn_exp2f(lam[Q - 1]);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) gacc[t][i] *= dec;
#pragma unroll
      for (int ks = 0; ks < Q / 32; ++ks) {
        const int tq = ks * 32 + g * 8;
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(eL + tq);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(eL + tq + 4);
        Frag8<T> cr, cf;
        frag_load8(cr, CT + (nt * 16 + r16) * TQ + tq);
#pragma unroll
        for (int j = 0; j < 8; ++j) frag_set(cf, j, to_f32(cr.v[j]) * (j < 4 ? e0[j] : e1[j - 4]));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> yf;
          frag_load8(yf, YT + ((pt0 + t) * 16 + r16) * TQ + tq);
          gacc[t] = mma(yf, cf, gacc[t]);
        }
      }
    }
    __syncthreads();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // segments 1..nseg-1 each hold at least one chunk (c0 < c1), so every
  // clamped chunk index below is a valid one
  prefetch(c1 - 1, S0{});
  prefetch(max(c1 - 2, c0), S1{});
  int c = c1 - 1;
  for (; c - 1 >= c0; c -= 2) {
    step(c, S0{});
    step(c - 1, S1{});
  }
  if (c >= c0) step(c, S0{});
  float* dst = k.seg_g + (unit * k.nseg + seg) * (P * N);
  if (owns)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] = gacc[t][i];
  if (tid == 0) k.seg_gd[unit * k.nseg + seg] = lam_seg;
}

// Both prepasses of the sequence split in one launch: they are independent
// and each fills fewer than all CUs.  Workgroups [0, total/2) walk segments
// 0..nseg-2 forward, the rest segments 1..nseg-1 backward.
template <typename T, int P, int N>
__global__ __launch_bounds__(kBThreads) void bwd_prepass_kernel(BwdK k) {
  const int half = gridDim.x / 2;
  if ((int)blockIdx.x < half) state_walk<T, P, N, true>(k, blockIdx.x, half);
  else gprep_walk<T, P, N>(k, blockIdx.x - half, half);
}

// Chains the segments of every unit, one thread per state element.
// Forward (seg_h): slot s <- exp2(hd_s) * start_s + end_s, the start of
// segment s+1 (start_0 = h0).  Backward (seg_g): from dL/dH = dhT at the end
// of the last segment, slot s <- exp2(gd_s) * G + slot s for s = nseg-1..1,
// the gradient at the end of segment s-1.
template <int PN>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdK k) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = blockIdx.y;
  const int b = (int)(unit / k.heads), h = (int)(unit % k.heads);
  if (e >= PN) return;
  const int64_t base = ((int64_t)b * k.n_heads + h) * PN + e;
  float st = k.h0 ? k.h0[base] : 0.0f;
  for (int s = 0; s + 1 < k.nseg; ++s) {
    float* slot = k.seg_h + (unit * k.nseg + s) * PN + e;
    st = __builtin_amdgcn_exp2f(k.seg_hd[unit * k.nseg + s]) * st + *slot;
    *slot = st;
  }
  float gr = k.dhT ? k.dhT[base] : 0.0f;
  for (int s = k.nseg - 1; s >= 1; --s) {
    float* slot = k.seg_g + (unit * k.nseg + s) * PN + e;
    gr = __builtin_amdgcn_exp2f(k.seg_gd[unit * k.nseg + s]) * gr + *slot;
    *slot = gr;
  }
}

template <typename T, int P, int N>
struct ChunkLds {
  static constexpr int NP = P + bpad<T>();   // token-major x and dy rows
  static constexpr int NN = N + bpad<T>();   // token-major B and C rows, Gc rows (p-major)
  static constexpr int TQ = kBQ + bpad<T>(); // transposed dy, B, C rows
  static constexpr int TP2 = P + bpad<T>();  // Gc^T and Hp^T rows (n-major)
  static constexpr size_t elems = (size_t)2 * kBQ * NP + (size_t)P * TQ + (size_t)2 * kBQ * NN +
                                  (size_t)2 * N * TQ + (size_t)P * NN + (size_t)2 * N * TP2;
  static constexpr int kFloats = 15 * kBQ + 2 * kBWaves;
  static constexpr size_t bytes = elems * sizeof(T) + kFloats * sizeof(float);
};

template <typename T>
__device__ __forceinline__ void grad_store(T* p, float v, int accumulate) {
  *p = from_f32<T>(accumulate ? to_f32(*p) + v : v);
}

template <typename T, int P, int N>
__global__ __launch_bounds__(kBThreads) void bwd_chunk_kernel(BwdK k) {
  using L = ChunkLds<T, P, N>;
  constexpr int Q = kBQ, NP = L::NP, NN = L::NN, TQ = L::TQ, TP2 = L::TP2;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= kBWaves ? NTILE / kBWaves : 1;
  constexpr int NKB = (N + 31) / 32;  // K=32 slices over d_state
  constexpr int PKB = P / 32;         // K=32 slices over d_head
  constexpr int VB = 16 / (int)sizeof(T);
  constexpr int NBLK = Q / 16;        // 16-token blocks per chunk
  static_assert(NBLK == 4, "four s-blocks and four t-blocks, one per wave");
  static_assert(P % 32 == 0, "d_head is a whole number of K=32 slices");
  constexpr int NXV = (Q * (P / VB) + kBThreads - 1) / kBThreads;  // x, dy vectors per thread
  constexpr int NBV = (Q * (N / VB) + kBThreads - 1) / kBThreads;  // B, C vectors per thread
  constexpr int NHV = (P * (N / VB) + kBThreads - 1) / kBThreads;  // Hp vectors per thread
  constexpr int TPH = TP / 2;                  // d_head tiles per column half
  constexpr int TNH = TN >= 2 ? TN / 2 : 1;    // d_state tiles per column half
  static_assert(TP % 2 == 0 && (TN == 1 || TN % 2 == 0), "columns split in two halves");

  extern __shared__ __align__(16) unsigned char smem[];
  T* Xn = reinterpret_cast<T*>(smem);  // [Q][NP]
  T* Yn = Xn + Q * NP;                 // dy [Q][NP]
  T* YT = Yn + Q * NP;                 // dy^T [P][TQ]
  T* Bn = YT + P * TQ;                 // [Q][NN]
  T* Cn = Bn + Q * NN;                 // [Q][NN]
  T* BT = Cn + Q * NN;                 // [N][TQ]
  T* CT = BT + N * TQ;                 // [N][TQ]
  T* Gs = CT + N * TQ;                 // Gc [P][NN]
  T* GT = Gs + P * NN;                 // Gc^T [N][TP2]
  T* HT = GT + N * TP2;                // Hp^T [N][TP2]
  float* lam = reinterpret_cast<float*>(HT + N * TP2);  // log2-scaled Lambda
  float* dtv = lam + Q;
  float* eL = dtv + Q;    // exp(Lambda_t)
  float* sc = eL + Q;     // exp(Lambda_e - Lambda_s)
  float* rpart = sc + Q;  // sum_s W[t,s] over each s-block: [4][Q]
  float* csum = rpart + 4 * Q;  // sum_t W[t,s]
  float* esum = csum + Q;     // dt_s exp(..) x_s^T Gc B_s, per column half: [2][Q]
  float* t1 = esum + 2 * Q;   // exp(Lambda_t) dy_t . Hp C_t, per column half: [2][Q]
  float* expl = t1 + 2 * Q;   // x_s . u_s, per column half: [2][Q]
  float* hgw = expl + 2 * Q;  // <Gc, H_e> over each wave's tiles: [2][8] by chunk parity

  int b, h, seg;
  unit_of(k.heads, k.nseg, &b, &h, &seg);
  const int64_t unit = (int64_t)b * k.heads + h;
  const int c0 = seg * k.seg_chunks, c1 = min(c0 + k.seg_chunks, k.nchunks);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;
  const T* __restrict__ Xp = static_cast<const T*>(k.x);
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const T* __restrict__ Bp = static_cast<const T*>(k.B);
  const T* __restrict__ Cp = static_cast<const T*>(k.C);
  const T* __restrict__ DYp = static_cast<const T*>(k.dy);
  T* __restrict__ DXp = static_cast<T*>(k.dx);
  T* __restrict__ DDTp = static_cast<T*>(k.ddt);
  const T* __restrict__ Hst =
      static_cast<const T*>(k.hst) + unit * (k.nchunks + 1) * (P * N);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah = k.A[h];
  const float Ah2 = Ah * kLog2e;
  const float Dh = k.D ? k.D[h] : 0.0f;

  // tiles of dL/dH owned by this wave: G[pt*16 + g*4 + i][nt*16 + r16]
  const int tile0 = wave * TPW;
  const bool owns = tile0 < NTILE;
  const int nt = tile0 / TP, pt0 = tile0 % TP;
  f32x4 gacc[TPW];
  {
    // dL/dH at the end of this walk: the final state's cotangent, or (split
    // sequence) the combined gradient at the end of this segment
    const float* gin = seg + 1 < k.nseg ? k.seg_g + (unit * k.nseg + seg + 1) * (P * N)
                       : k.dhT          ? k.dhT + ((int64_t)b * k.n_heads + h) * (P * N)
                                        : nullptr;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        gacc[t][i] = (gin && owns) ? gin[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] : 0.0f;
  }
  // Global rows of a chunk, into registers (all issued before any is used).
  Vec16<T> vx[NXV], vy[NXV], vb[NBV], vc[NBV];
  float pdt = 0.0f;
  auto load_rows = [&](int c) {
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
    // unconditional loads at clamped addresses (a lane-conditional load is
    // waited for at its branch's end); rows past len are zeroed at staging
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (P / VB) - 1), s = min(idx % Q, len - 1);
      const int p0 = (idx / Q) * VB;
      vx[v] = load16(Xp + (row0 + s) * k.xs + (int64_t)h * P + p0);
      vy[v] = load16(DYp + (row0 + s) * k.dys + (int64_t)h * P + p0);
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (N / VB) - 1), s = min(idx % Q, len - 1);
      const int n0 = (idx / Q) * VB;
      vb[v] = load16(Bp + (row0 + s) * k.bs + n0);
      vc[v] = load16(Cp + (row0 + s) * k.cs + n0);
    }
    pdt = to_f32(DTp[(row0 + min(lane, len - 1)) * k.dts + h]);
  };
  // <Gc, H_e> of the last chunk: Gc = dL/dh_final, H_e = the final state;
  // for every other chunk it is formed at the end of the chunk after it,
  // from the operand copy of that chunk's start state in LDS
  {
    const int cl = c1 - 1;
    const T* hn = Hst + (int64_t)c1 * (P * N);
    float hdot = 0.0f;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hdot += owns ? gacc[t][i] * to_f32(hn[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16])
                     : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) hdot += __shfl_xor(hdot, off);
    if (lane == 0) hgw[(cl & 1) * kBWaves + wave] = hdot;
  }
  float da_acc = 0.0f;  // wave 0: sum_r dt_r da_r of this lane's tokens
  float dd_acc = 0.0f;  // sum dy . x over this lane's entries

  for (int c = c1 - 1; c >= c0; --c) {
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);

    // ---- stage: the chunk's rows into LDS (every global load first: one
    // round trip): token rows (zero past len), transposed copies, Hp^T and
    // Gc.  (Loading the next chunk during this one's compute measured no
    // faster and spills registers.) ----
    load_rows(c);
    Vec16<T> vh[NHV];
    {
      const T* hp = Hst + (int64_t)c * (P * N);
#pragma unroll
      for (int v = 0; v < NHV; ++v) {
        const int idx = min(tid + v * kBThreads, P * (N / VB) - 1), p = idx % P;
        vh[v] = load16(hp + p * N + (idx / P) * VB);
      }
    }
    const float dtl = lane < len ? pdt : 0.0f;
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, p0 = (idx / Q) * VB;
      const Vec16<T> xv = s < len ? vx[v] : zero16<T>(), yv = s < len ? vy[v] : zero16<T>();
      if (idx < Q * (P / VB)) {
        store16(Xn + s * NP + p0, xv);
        store16(Yn + s * NP + p0, yv);
#pragma unroll
        for (int j = 0; j < VB; ++j) YT[(p0 + j) * TQ + s] = yv.v[j];
      }
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = tid + v * kBThreads, s = idx % Q, n0 = (idx / Q) * VB;
      const Vec16<T> bv = s < len ? vb[v] : zero16<T>(), cv = s < len ? vc[v] : zero16<T>();
      if (idx < Q * (N / VB)) {
        store16(Bn + s * NN + n0, bv);
        store16(Cn + s * NN + n0, cv);
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          BT[(n0 + j) * TQ + s] = bv.v[j];
          CT[(n0 + j) * TQ + s] = cv.v[j];
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NHV; ++v) {
      const int idx = tid + v * kBThreads, p = idx % P, n0 = (idx / P) * VB;
      if (idx < P * (N / VB))
#pragma unroll
        for (int j = 0; j < VB; ++j) HT[(n0 + j) * TP2 + p] = vh[v].v[j];
    }
    if (owns) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int p0 = (pt0 + t) * 16 + g * 4, n = nt * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) Gs[(p0 + i) * NN + n] = from_f32<T>(gacc[t][i]);
        store4(GT + n * TP2 + p0, gacc[t][0], gacc[t][1], gacc[t][2], gacc[t][3]);
      }
    }
    if (wave == 0) {
      const float d = dtl;
      const float lv = chunk_cumsum(d * Ah2, lane);
      const float le = __shfl(lv, 63);
      lam[lane] = lv;
      dtv[lane] = d;
      eL[lane] = __builtin_amdgcn_exp2f(lv);
      sc[lane] = __builtin_amdgcn_exp2f(le - lv);
#pragma unroll
      for (int j = 0; j < 4; ++j) rpart[j * Q + lane] = 0.0f;
    }
    __syncthreads();

    {
      // ---- this wave: s-block and t-block `blk`, column half `hf` (d_head
      // tiles [pb0, pb0+TPH), d_state tiles [nb0, nb0+TNH)); the two waves of
      // a block share its Q x Q products and split the outputs' columns ----
      const int blk = wave % NBLK, hf = wave / NBLK;
      const int pb0 = hf * TPH, nb0 = hf * TNH;
      const bool nlive = nb0 < TN;  // this half has d_state tiles (wave-uniform)

      // ---- s-side: rows s of the block: dx, dB, column sums of W ----
      {
        const int s0 = blk * 16, srow = s0 + r16;  // A-operand row of this lane
        const float scs = sc[srow];
        f32x4 au[TPH], ab[TNH];
#pragma unroll
        for (int i = 0; i < TPH; ++i) au[i] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < TNH; ++i) ab[i] = f32x4{0, 0, 0, 0};
        // end-state terms: u += exp(..) B_s Gc^T,  dB-part += exp(..) x_s Gc
#pragma unroll 1
        for (int kb = 0; kb < NKB; ++kb) {
          Frag8<T> bf;
          frag_row_scaled(bf, Bn + srow * NN, kb * 32 + g * 8, N, scs);
#pragma unroll
          for (int pp = 0; pp < TPH; ++pp) {
            Frag8<T> gf;
            frag_row(gf, Gs + ((pb0 + pp) * 16 + r16) * NN, kb * 32 + g * 8, N);
            au[pp] = mma(bf, gf, au[pp]);
          }
        }
        if (nlive) {
#pragma unroll 1
          for (int kp = 0; kp < PKB; ++kp) {
            Frag8<T> xf;
            frag_row_scaled(xf, Xn + srow * NP, kp * 32 + g * 8, P, scs);
#pragma unroll
            for (int nn = 0; nn < TNH; ++nn) {
              Frag8<T> gf;
              frag_load8(gf, GT + ((nb0 + nn) * 16 + r16) * TP2 + kp * 32 + g * 8);
              ab[nn] = mma(xf, gf, ab[nn]);
            }
          }
        }
        // esum_s (this half) = dt_s sum_n ab[s][n] B[s][n]  (rows s = s0 + 4g + i)
        {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = s0 + g * 4 + i;
            float v = 0.0f;
            if (nlive)
#pragma unroll
              for (int nn = 0; nn < TNH; ++nn)
                v += ab[nn][i] * to_f32(Bn[s * NN + (nb0 + nn) * 16 + r16]);
            e[i] = v;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = row16_sum(e[i]);
          if (r16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) esum[hf * Q + s0 + g * 4 + i] = e[i] * dtv[s0 + g * 4 + i];
        }
        // diagonal-block terms over t-block pairs (2ip, 2ip+1) with t >= s
        const float lam_s = lam[srow], dt_s = dtv[srow];
        float csum_l = 0.0f;
#pragma unroll 1
        for (int ip = blk / 2; ip < NBLK / 2; ++ip) {
          const int ta = 2 * ip, tb = 2 * ip + 1;
          const bool doa = ta >= blk;  // block ta has t >= s somewhere (wave-uniform)
          f32x4 gA = {0, 0, 0, 0}, gB = {0, 0, 0, 0}, qA = {0, 0, 0, 0}, qB = {0, 0, 0, 0};
#pragma unroll 2
          for (int kb = 0; kb < NKB; ++kb) {
            Frag8<T> bs, ca, cb;
            frag_row(bs, Bn + srow * NN, kb * 32 + g * 8, N);
            frag_row(cb, Cn + (tb * 16 + r16) * NN, kb * 32 + g * 8, N);
            gB = mma(cb, bs, gB);
            if (doa) {
              frag_row(ca, Cn + (ta * 16 + r16) * NN, kb * 32 + g * 8, N);
              gA = mma(ca, bs, gA);
            }
          }
#pragma unroll
          for (int kp = 0; kp < PKB; ++kp) {
            Frag8<T> xs, ya, yb;
            frag_load8(xs, Xn + srow * NP + kp * 32 + g * 8);
            frag_load8(yb, Yn + (tb * 16 + r16) * NP + kp * 32 + g * 8);
            qB = mma(yb, xs, qB);
            if (doa) {
              frag_load8(ya, Yn + (ta * 16 + r16) * NP + kp * 32 + g * 8);
              qA = mma(ya, xs, qA);
            }
          }
          // lane: G[t][s], Q[t][s] for s = srow, t = ta*16 + 4g + i (slot i)
          // and t = tb*16 + 4g + i (slot 4 + i)
          Frag8<T> mf, kf;
          float rw[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int t = (j < 4 ? ta : tb) * 16 + g * 4 + (j & 3);
            const float gv = j < 4 ? gA[j] : gB[j - 4];
            const float qv = j < 4 ? qA[j] : qB[j - 4];
            const float dec = t >= srow ? __builtin_amdgcn_exp2f(lam[t] - lam_s) : 0.0f;
            frag_set(mf, j, gv * dec);
            frag_set(kf, j, qv * dec);
            const float w = gv * qv * dec * dt_s;
            rw[j] = w;
            csum_l += w;
          }
          if (hf == 0) {
            // row sums of W over this block's 16 s (lanes r16), per t
#pragma unroll
            for (int j = 0; j < 8; ++j) rw[j] = row16_sum(rw[j]);
            if (r16 == 0) {
#pragma unroll
              for (int j = 0; j < 8; ++j)
                rpart[blk * Q + (j < 4 ? ta : tb) * 16 + g * 4 + (j & 3)] = rw[j];
            }
          }
          // u += M^T dy  (k = t in the slot order above), dB-part += K^T C
#pragma unroll
          for (int pp = 0; pp < TPH; ++pp) {
            Frag8<T> yf;
            const T* yr = YT + ((pb0 + pp) * 16 + r16) * TQ;
            frag_load4x2(yf, yr + ta * 16 + g * 4, yr + tb * 16 + g * 4);
            au[pp] = mma(mf, yf, au[pp]);
          }
          if (nlive) {
#pragma unroll
            for (int nn = 0; nn < TNH; ++nn) {
              Frag8<T> cf;
              const T* cr = CT + ((nb0 + nn) * 16 + r16) * TQ;
              frag_load4x2(cf, cr + ta * 16 + g * 4, cr + tb * 16 + g * 4);
              ab[nn] = mma(kf, cf, ab[nn]);
            }
          }
        }
        // column sums: over the 4 t-slots of each group, then the 4 groups
        csum_l += __shfl_xor(csum_l, 16);
        csum_l += __shfl_xor(csum_l, 32);
        if (hf == 0 && g == 0) csum[srow] = csum_l;
        // epilogue: dx = dt_s u + D dy, x_s . u_s and dy . x over this half's
        // d_head columns, dB atomics over its d_state columns
        float ex[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float dxv[4][TPH];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = s0 + g * 4 + i;
          const float dts = dtv[s];
          const bool live = s < len;
#pragma unroll
          for (int pp = 0; pp < TPH; ++pp) {
            const int p = (pb0 + pp) * 16 + r16;
            const float xv = to_f32(Xn[s * NP + p]), yv = to_f32(Yn[s * NP + p]);
            ex[i] += xv * au[pp][i];
            dd_acc += xv * yv;
            dxv[i][pp] = dts * au[pp][i] + Dh * yv;
          }
          if (live && nlive) {
#pragma unroll
            for (int nn = 0; nn < TNH; ++nn)
              unsafeAtomicAdd(k.dB + (row0 + s) * k.dbs + (nb0 + nn) * 16 + r16, dts * ab[nn][i]);
          }
        }
        // dx rows: when adding into the caller's dx, all of this lane's old
        // values are read (at clamped rows, under the wave-uniform flag only)
        // before any is written, so the reads are in flight together
        T* const dxrow = DXp + row0 * k.dxs + (int64_t)h * P;
        if (k.accumulate) {
          float old[4][TPH];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int pp = 0; pp < TPH; ++pp)
              old[i][pp] = to_f32(dxrow[(int64_t)min(s0 + g * 4 + i, len - 1) * k.dxs +
                                        (pb0 + pp) * 16 + r16]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (s0 + g * 4 + i < len)
#pragma unroll
              for (int pp = 0; pp < TPH; ++pp)
                dxrow[(int64_t)(s0 + g * 4 + i) * k.dxs + (pb0 + pp) * 16 + r16] =
                    from_f32<T>(old[i][pp] + dxv[i][pp]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (s0 + g * 4 + i < len)
#pragma unroll
              for (int pp = 0; pp < TPH; ++pp)
                dxrow[(int64_t)(s0 + g * 4 + i) * k.dxs + (pb0 + pp) * 16 + r16] =
                    from_f32<T>(dxv[i][pp]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ex[i] = row16_sum(ex[i]);
        if (r16 == 0)
#pragma unroll
          for (int i = 0; i < 4; ++i) expl[hf * Q + s0 + g * 4 + i] = ex[i];
      }

      // ---- t-side: rows t of the block: dC (this half's columns), Hp term ----
      {
        const int t0 = blk * 16, trow = t0 + r16;
        const float lam_t = lam[trow];
        f32x4 ac[TNH];
#pragma unroll
        for (int i = 0; i < TNH; ++i) ac[i] = f32x4{0, 0, 0, 0};
        if (nlive) {
          // off-diagonal output term: exp(Lambda_t) dy_t Hp
#pragma unroll 1
          for (int kp = 0; kp < PKB; ++kp) {
            Frag8<T> yf;
            frag_row_scaled(yf, Yn + trow * NP, kp * 32 + g * 8, P, eL[trow]);
#pragma unroll
            for (int nn = 0; nn < TNH; ++nn) {
              Frag8<T> hfr;
              frag_load8(hfr, HT + ((nb0 + nn) * 16 + r16) * TP2 + kp * 32 + g * 8);
              ac[nn] = mma(yf, hfr, ac[nn]);
            }
          }
        }
        {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + g * 4 + i;
            float v = 0.0f;
            if (nlive)
#pragma unroll
              for (int nn = 0; nn < TNH; ++nn)
                v += ac[nn][i] * to_f32(Cn[t * NN + (nb0 + nn) * 16 + r16]);
            e[i] = v;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = row16_sum(e[i]);
          if (r16 == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) t1[hf * Q + t0 + g * 4 + i] = e[i];
        }
        if (nlive) {
          // diagonal-block term over s-block pairs (2jp, 2jp+1) with s <= t
#pragma unroll 1
          for (int jp = 0; jp <= blk / 2; ++jp) {
            const int sa = 2 * jp, sb2 = 2 * jp + 1;
            const bool dob = sb2 <= blk;  // wave-uniform
            f32x4 rA = {0, 0, 0, 0}, rB = {0, 0, 0, 0};
#pragma unroll
            for (int kp = 0; kp < PKB; ++kp) {
              Frag8<T> yt, xa, xb;
              frag_load8(yt, Yn + trow * NP + kp * 32 + g * 8);
              frag_load8(xa, Xn + (sa * 16 + r16) * NP + kp * 32 + g * 8);
              rA = mma(xa, yt, rA);
              if (dob) {
                frag_load8(xb, Xn + (sb2 * 16 + r16) * NP + kp * 32 + g * 8);
                rB = mma(xb, yt, rB);
              }
            }
            // lane: (x_s . dy_t) for t = trow, s = sa*16 + 4g + i (slot i),
            // sb2*16 + 4g + i (slot 4 + i)
            Frag8<T> kf;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int s = (j < 4 ? sa : sb2) * 16 + g * 4 + (j & 3);
              const float rv = j < 4 ? rA[j] : rB[j - 4];
              const float f = s <= trow ? __builtin_amdgcn_exp2f(lam_t - lam[s]) * dtv[s] : 0.0f;
              frag_set(kf, j, rv * f);
            }
#pragma unroll
            for (int nn = 0; nn < TNH; ++nn) {
              Frag8<T> bf;
              const T* br = BT + ((nb0 + nn) * 16 + r16) * TQ;
              frag_load4x2(bf, br + sa * 16 + g * 4, br + sb2 * 16 + g * 4);
              ac[nn] = mma(kf, bf, ac[nn]);
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + g * 4 + i;
            if (t < len) {
#pragma unroll
              for (int nn = 0; nn < TNH; ++nn)
                unsafeAtomicAdd(k.dC + (row0 + t) * k.dcs + (nb0 + nn) * 16 + r16, ac[nn][i]);
            }
          }
        }
      }
    }

    // ---- every wave: dGp = exp(Lambda_e) Gc + sum_t exp(Lambda_t) dy_t C_t^T on
    // its tiles, then <dGp, Hp> for the chunk before (Hp^T is in LDS) ----
    if (owns) {
      const float dec = __builtin_amdgcn_exp2f(lam[Q - 1]);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) gacc[t][i] *= dec;
#pragma unroll
      for (int ks = 0; ks < Q / 32; ++ks) {
        const int tq = ks * 32 + g * 8;
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(eL + tq);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(eL + tq + 4);
        Frag8<T> cr, cf;
        frag_load8(cr, CT + (nt * 16 + r16) * TQ + tq);
#pragma unroll
        for (int j = 0; j < 8; ++j) frag_set(cf, j, to_f32(cr.v[j]) * (j < 4 ? e0[j] : e1[j - 4]));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> yf;
          frag_load8(yf, YT + ((pt0 + t) * 16 + r16) * TQ + tq);
          gacc[t] = mma(yf, cf, gacc[t]);
        }
      }
    }
    if (c > c0) {
      float hdot = 0.0f;
      if (owns) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          float hv[4];
          load4(HT + (nt * 16 + r16) * TP2 + (pt0 + t) * 16 + g * 4, hv);
#pragma unroll
          for (int i = 0; i < 4; ++i) hdot += gacc[t][i] * hv[i];
        }
      }
      hdot = row16_sum(hdot);
      hdot += __shfl_xor(hdot, 16);
      hdot += __shfl_xor(hdot, 32);
      // two halves by chunk parity: wave 0 reads chunk c's half below while
      // this writes chunk c-1's
      if (lane == 0) hgw[((c - 1) & 1) * kBWaves + wave] = hdot;
    }
    __syncthreads();

    // ---- wave 0: dLambda -> da (suffix sum) -> ddt, dA ----
    if (wave == 0) {
      const int t = lane;
      // fixed summation order: the result does not depend on wave timing
      float dl = (t1[t] + t1[Q + t]) +
                 (((rpart[t] + rpart[Q + t]) + rpart[2 * Q + t]) + rpart[3 * Q + t]) - csum[t] -
                 (esum[t] + esum[Q + t]);
      if (t == Q - 1) {
        float hg = 0.0f;
#pragma unroll
        for (int j = 0; j < kBWaves; ++j) hg += hgw[(c & 1) * kBWaves + j];
        dl += hg;
      }
      // suffix sum over t' >= t: the total minus the prefix before t
      const float incl = wave_incl_scan(dl);
      const float tot = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
      const float suf = (tot - incl) + dl;
      if (t < len) {
        grad_store(DDTp + (row0 + t) * k.ddts + h, (expl[t] + expl[Q + t]) + Ah * suf, k.accumulate);
        da_acc += dtv[t] * suf;
      }
    }
    // wave 0 rewrites lam/dtv/eL/sc/rpart only after its own reads above;
    // every other array is rewritten after the next barrier
  }

  // ---- per-unit results: dh0, dA, dD ----
  if (k.dh0 && owns && seg == 0) {
    float* dst = k.dh0 + ((int64_t)b * k.n_heads + h) * (P * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* q = dst + ((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16;
        *q = k.accumulate ? *q + gacc[t][i] : gacc[t][i];
      }
  }
  if (wave == 0) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) da_acc += __shfl_xor(da_acc, off);
    if (lane == 0) unsafeAtomicAdd(k.dA + h, da_acc);
  }
  if (k.dD) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) dd_acc += __shfl_xor(dd_acc, off);
    if (lane == 0) unsafeAtomicAdd(k.dD + h, dd_acc);
  }
}

// The summed gradients set to zero in one launch: dB and dC (rows x width
// fp32 values with their own row strides), dA and dD (heads values; dD may
// be null).
__global__ __launch_bounds__(256) void zero_grads_kernel(float* dB, int64_t dbs, float* dC, int64_t dcs,
                                                         int width, int64_t rows, float* dA, float* dD,
                                                         int heads) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < rows * width) {
    const int64_t r = i / width;
    const int col = (int)(i % width);
    dB[r * dbs + col] = 0.0f;
    dC[r * dcs + col] = 0.0f;
  }
  if (i < heads) {
    dA[i] = 0.0f;
    if (dD) dD[i] = 0.0f;
  }
}

template <typename T, int P, int N>
hipError_t launch_shape(const BwdK& k, int64_t batch, hipStream_t s) {
  const unsigned units = (unsigned)(batch * k.heads);
  const size_t lds1 = StateLds<T, P, N>::bytes, lds2 = ChunkLds<T, P, N>::bytes;
  static_assert(ChunkLds<T, P, N>::bytes <= 160 * 1024, "chunk tiles fit one CU's LDS");
  const void* fns[] = {reinterpret_cast<const void*>(&bwd_state_kernel<T, P, N>),
                       reinterpret_cast<const void*>(&bwd_prepass_kernel<T, P, N>),
                       reinterpret_cast<const void*>(&bwd_chunk_kernel<T, P, N>)};
  const size_t ldss[] = {lds1, lds1, lds2};
  for (int i = 0; i < 3; ++i) {
    const hipError_t e =
        hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldss[i]);
    if (e != hipSuccess) return e;
  }
  if (k.nseg > 1) {
    // segment prepasses (forward states, reverse dL/dH), then the combine
    const unsigned pre = units * (unsigned)(k.nseg - 1);
    hipLaunchKernelGGL((bwd_prepass_kernel<T, P, N>), dim3(2 * pre), dim3(kBThreads), lds1, s, k);
    hipLaunchKernelGGL((bwd_combine_kernel<P * N>), dim3((P * N + 255) / 256, units), dim3(256), 0,
                       s, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid = units * (unsigned)k.nseg;
  hipLaunchKernelGGL((bwd_state_kernel<T, P, N>), dim3(grid), dim3(kBThreads), lds1, s, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk_kernel<T, P, N>), dim3(grid), dim3(kBThreads), lds2, s, k);
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool bwd_shape_supported(int64_t d_head, int64_t d_state, int dtype) {
  if (dtype == MM_BF16) return d_head == 64 && (d_state == 64 || d_state == 128);
  return d_head == 32 && d_state == 16;
}

void bwd_plan(int64_t batch, int64_t seqlen, int64_t heads, int* nchunks, int* nseg,
              int* seg_chunks) {
  const int nc = (int)((seqlen + kBQ - 1) / kBQ);
  const int64_t units = batch * heads;
  // Each (sequence, head) walk is one latency-bound workgroup per CU; with
  // fewer than 256 walks, split the sequences into segments (at least four
  // chunks each) so that about 256 workgroups run.
  int64_t ns = 1;
  if (units < 256) ns = std::min<int64_t>((256 + units - 1) / units, nc / 4);
  if (ns < 1) ns = 1;
  const int sc = (int)((nc + ns - 1) / ns);
  *nchunks = nc;
  *seg_chunks = sc;
  *nseg = (nc + sc - 1) / sc;
}

size_t bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                           int64_t d_state, int dtype) {
  int nc, ns, sc;
  bwd_plan(batch, seqlen, heads, &nc, &ns, &sc);
  const size_t el = dtype == MM_BF16 ? 2 : 4;
  const size_t units = (size_t)(batch * heads), pn = (size_t)(d_head * d_state);
  size_t bytes = align256(units * (size_t)(nc + 1) * pn * el);
  if (ns > 1) bytes += 2 * align256(units * ns * pn * 4) + 2 * align256(units * ns * 4);
  return bytes;
}

hipError_t launch_ssd_backward(const BwdArgs& a, void* workspace, hipStream_t s) {
  BwdK k;
  k.x = a.x;
  k.xs = a.xs;
  k.dt = a.dt;
  k.dts = a.dts;
  k.A = a.A;
  k.B = a.B;
  k.bs = a.bs;
  k.C = a.C;
  k.cs = a.cs;
  k.D = a.D;
  k.h0 = a.h0;
  k.dy = a.dy;
  k.dys = a.dys;
  k.dhT = a.dhT;
  k.dx = a.dx;
  k.dxs = a.dxs;
  k.ddt = a.ddt;
  k.ddts = a.ddts;
  k.dA = a.dA;
  k.dB = a.dB;
  k.dbs = a.dbs;
  k.dC = a.dC;
  k.dcs = a.dcs;
  k.dD = a.dD;
  k.dh0 = a.dh0;
  k.seqlen = a.seqlen;
  k.n_heads = a.n_heads;
  k.heads = a.heads;
  bwd_plan(a.batch, a.seqlen, a.heads, &k.nchunks, &k.nseg, &k.seg_chunks);
  k.accumulate = a.accumulate;
  {
    const size_t el = a.dtype == MM_BF16 ? 2 : 4;
    const size_t units = (size_t)(a.batch * a.heads), pn = (size_t)(a.d_head * a.d_state);
    unsigned char* w = static_cast<unsigned char*>(workspace);
    k.hst = w;
    w += align256(units * (size_t)(k.nchunks + 1) * pn * el);
    k.seg_h = k.seg_g = k.seg_hd = k.seg_gd = nullptr;
    if (k.nseg > 1) {
      k.seg_h = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * pn * 4);
      k.seg_g = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * pn * 4);
      k.seg_hd = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * 4);
      k.seg_gd = reinterpret_cast<float*>(w);
    }
  }
  if (!a.accumulate) {
    const int64_t rows = a.batch * a.seqlen;
    const int64_t n = std::max<int64_t>(rows * a.d_state, a.heads);
    hipLaunchKernelGGL(zero_grads_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.dB, a.dbs,
                       a.dC, a.dcs, a.d_state, rows, a.dA, a.dD, a.heads);
  }
  if (a.dtype == MM_BF16) {
    if (a.d_state == 128) return launch_shape<bf16, 64, 128>(k, a.batch, s);
    return launch_shape<bf16, 64, 64>(k, a.batch, s);
  }
  return launch_shape<float, 32, 16>(k, a.batch, s);
}

}  // namespace mmssd
