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
//  - bwd_walks_kernel: two independent walks per (sequence, head) in one
//    launch, one workgroup of 8 waves each, the fp32 P x N value in MFMA
//    accumulators: forwards, storing the state before every chunk (and the
//    final one); backwards, storing Gc, dL/dH at the end of every chunk.
//    Both are stored in the storage type in MFMA fragment order: each lane
//    writes its 16 bytes of a 1 KB fragment, so a store covers whole cache
//    lines.  Token rows are read by consecutive lanes along a row.  With few
//    walks the sequences are split into segments walked in parallel, each
//    from its own start (h0 or dL/dH of the final state at the sequence's
//    ends, zero elsewhere); a combine chains the segments' end values, and
//    the chunk kernel adds to each stored value the chained value at its
//    segment's boundary, decayed to the chunk (the recurrence is linear).
//  - bwd_chunk_kernel: one workgroup of 16 waves per (sequence, chunk), every
//    chunk in parallel, looping over up to 64 heads per launch.  The B, C
//    rows, the Q x Q blocks of C_t . B_s (the same for every head) and the
//    chunk's dt, A and D of the heads are loaded once; per head the x, dy
//    rows, Hp and Gc are staged (the next head's loaded during this one),
//    then phase 1 forms the head's Q x Q blocks (one block per wave on waves
//    0-9) and the end-state and Hp terms (each wave its own u, dB and dC
//    tiles) and phase 2 the causal products into the same accumulators, with
//    dx written and dB, dC added to their sums over the heads in registers.
//    Products that need a tile's transpose read its columns with LDS
//    transpose loads.  Wave kTailWave forms the previous head's
//    dLambda, ddt, dA and dD during phase 1 and leaves them in LDS.
//  - dB and dC (sums over the heads) are written once per chunk, no atomics;
//    ddt once per chunk for all its heads; dA and dD (sums over the sequences
//    and chunks) are one fp32 atomic per (workgroup, head).
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kBQ = 64;  // tokens per backward chunk
constexpr int kBWaves = 8;  // state walks
constexpr int kBThreads = kBWaves * 64;
constexpr int kCWaves = 16;  // chunk walk
constexpr int kCThreads = kCWaves * 64;
constexpr int kTailWave = 2;  // runs each head's dLambda / ddt / dA / dD tail
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
  void* hst;  // (batch, heads, nchunks + 1, P, N) storage type, fragment order
  void* gst;  // (batch, heads, nchunks, P, N) storage type, fragment order: dL/dH at each chunk's end
  // sequence split (nseg > 1): per (unit, segment) fp32 P x N blocks,
  // n-major ([N][P]), and the segments' log2 decays (the combine describes
  // what each holds); the chained boundary values in the storage type,
  // n-major: hb slot s the state at the start of segment s+1, gb slot s
  // dL/dH at the end of segment s-1; per (unit, chunk) the log2 decay
  // between the chunk's stored value and its segment's boundary: lamh from
  // the segment start to the chunk start, lamg from the chunk end to the
  // segment end
  float* seg_h;
  float* seg_hd;
  float* seg_g;
  float* seg_gd;
  void* seg_hb;
  void* seg_gb;
  float* lamh;
  float* lamg;
  int64_t seqlen;
  int n_heads, heads, nchunks, accumulate;
  int nseg, seg_chunks;
  // chunk kernel: heads [h0g, h0g + hg) of this launch; bc_acc: add dB, dC
  // into the values an earlier launch (heads before h0g) wrote
  int h0g, hg, bc_acc;
};

template <typename T> constexpr int bpad() { return 16 / (int)sizeof(T); }

// State tiles (16 x 16 of P x N) come in pairs 2j, 2j+1 that together cover
// d_head rows 32j .. 32j+31, interleaved so that the accumulators of a pair
// are an MFMA operand fragment with K = d_head: row m of tile T is d_head row
//   prow(T, m) = 32 (T/2) + 4 (T%2) + 8 (m/4) + m%4,
// so lane (r, g) holds rows 32j + 8g + 0..7 of column r across the pair
// (slots 0-3 from tile 2j, 4-7 from tile 2j+1).  The stored chunk states use
// that fragment order: fragment (kp, nb) of a P x N state is 64 lanes x 8
// consecutive elements at ((kp * N/16 + nb) * 64 + lane) * 8.
__device__ __forceinline__ int prow(int T, int m) {
  return (T >> 1) * 32 + (T & 1) * 4 + (m >> 2) * 8 + (m & 3);
}

template <int N>
__device__ __forceinline__ int64_t state_frag(int kp, int nb, int lane) {
  return ((int64_t)(kp * (N / 16) + nb) * 64 + lane) * 8;
}

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

// Eight consecutive storage elements from two accumulator quads (16 B of
// bf16, 32 of fp32).
template <typename T>
__device__ __forceinline__ void store8(T* p, const f32x4& a, const f32x4& b) {
  if constexpr (sizeof(T) == 2) {
    bf16 v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = from_f32<bf16>(a[i]);
      v[i + 4] = from_f32<bf16>(b[i]);
    }
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(v);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a[0], a[1], a[2], a[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(b[0], b[1], b[2], b[3]);
  }
}

// One storage element through a buffer resource: loads outside the range
// read 0, stores there are dropped.
template <typename T>
__device__ __forceinline__ float buffer_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 2) {
    const unsigned short u = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    return __builtin_bit_cast(float, (uint32_t)u << 16);
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  }
}
template <typename T>
__device__ __forceinline__ void buffer_store_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<bf16>(v)), r,
                                          (int)off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
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

// Operand fragment from columns of a row-major LDS tile M (row pitch ld):
// lane (r, g) gets M[ra + j][c(r)] in slots j = 0..3 and M[rb + j][c(r)] in
// slots 4..7, where ra, rb are the row bases of its 16-lane group and
// c(r) = c0 + cs (r/4) + r%4 (cs = 4: sixteen consecutive columns; cs = 8:
// the paired d_head rows of prow()).  16-bit elements: two LDS transpose
// loads, in which lane q of a group addresses the four elements at row
// base + q/4, columns c0 + cs (q%4) .. +3, and receives in element k element
// q%4 of what lane 4k + q/4 addressed (tiles of whole K=32 slices only).
// 32-bit elements: eight element reads, zeros where live is false.
template <typename T>
__device__ __forceinline__ void frag_cols(Frag8<T>& f, const T* M, int ld, int ra, int rb, int c0,
                                          int cs, int lane, bool live = true) {
  const int q = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef short short4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) short4v lds_short4;
    const int col = c0 + (q & 3) * cs;
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4*)(const_cast<T*>(M) + (ra + (q >> 2)) * ld + col));
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4*)(const_cast<T*>(M) + (rb + (q >> 2)) * ld + col));
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    const int col = c0 + (q >> 2) * cs + (q & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = live ? M[(ra + j) * ld + col] : 0.0f;
      f.v[j + 4] = live ? M[(rb + j) * ld + col] : 0.0f;
    }
  }
}

// Rows ra..ra+3 of column c0 + lane%16 of a row-major LDS tile M (pitch
// ld), as fp32: one transpose load in 16-bit storage (frag_cols' first
// half with column step 4), four element loads in fp32.
template <typename T>
__device__ __forceinline__ f32x4 col4(const T* M, int ld, int ra, int c0, int lane) {
  const int q = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef short short4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) short4v lds_short4;
    const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4*)(const_cast<T*>(M) + (ra + (q >> 2)) * ld + c0 + (q & 3) * 4));
    const uint2 u = __builtin_bit_cast(uint2, v);
    return f32x4{__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
                 __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u)};
  } else {
    return f32x4{M[ra * ld + c0 + q], M[(ra + 1) * ld + c0 + q], M[(ra + 2) * ld + c0 + q],
                 M[(ra + 3) * ld + c0 + q]};
  }
}

// LDS of a walk: two buffers (by chunk parity), each the chunk's rows of the
// d_head stream (x forwards, dy backwards) and of the d_state stream (B
// forwards, C backwards) token-major, with Lambda and the per-token weights.
template <typename T, int P, int N>
struct WalkLds {
  static constexpr int NP = P + bpad<T>();
  static constexpr int NN = N + bpad<T>();
  static constexpr size_t buf_elems = (size_t)kBQ * NP + (size_t)kBQ * NN;
  static constexpr size_t buf_bytes = buf_elems * sizeof(T) + 2 * kBQ * sizeof(float);
  static constexpr size_t bytes = 2 * buf_bytes;
};

// One walk over the chunks of a (sequence, head) segment with the fp32 P x N
// value V in MFMA accumulators, V <- exp2(Lambda_e) V + sum_t a_t w_t b_t^T
// per chunk:
//   REV = false (states): chunks ascending, a = x, b = B, w_s = exp2(Lambda_e -
//     Lambda_s) dt_s: V is the state, stored before every chunk (and after
//     the last one) in fragment order.  Starts from h0 in the first segment,
//     from zero in the others.
//   REV = true (gradients): chunks descending, a = dy, b = C, w_t =
//     exp2(Lambda_t): V is dL/dH, stored at the end of every chunk in
//     fragment order, before the chunk's update.  Starts from dL/dH of the
//     final state in the last segment, from zero in the others; an unsplit
//     walk writes dh0.
// In a split call every walk also stores, per chunk, the log2 decay between
// the stored value and the segment boundary it started from, and writes its
// own end value (forward, all segments but the last) or start value
// (backward, every segment) with the segment's log2 decay, for the combine.
// The a and b rows are staged token-major and read as operand columns with
// transpose loads; the rows of the chunk two ahead are loaded into registers
// (two sets, used alternately) and the LDS buffers alternate by chunk, so a
// chunk needs one barrier.  Tile rows in the paired order of prow().
template <typename T, int P, int N, bool REV>
__device__ __forceinline__ void walk(const BwdK& k, int pid, int total) {
  using L = WalkLds<T, P, N>;
  constexpr int Q = kBQ, NP = L::NP, NN = L::NN;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= 2 * kBWaves ? NTILE / kBWaves : 2;
  static_assert(NTILE < 2 * kBWaves || NTILE % kBWaves == 0, "state tiles must split evenly");
  static_assert(TP % TPW == 0 && TPW % 2 == 0, "a wave's tiles are whole pairs of one column block");
  constexpr int VB = 16 / (int)sizeof(T);
  constexpr int NAV = (Q * (P / VB) + kBThreads - 1) / kBThreads;  // a vectors per thread
  constexpr int NBV = (Q * (N / VB) + kBThreads - 1) / kBThreads;  // b vectors per thread
  extern __shared__ __align__(16) unsigned char smem[];
  auto buf = [&](int parity, T*& an, T*& bn, float*& lam, float*& wt) {
    unsigned char* base = smem + parity * L::buf_bytes;
    an = reinterpret_cast<T*>(base);
    bn = an + Q * NP;
    lam = reinterpret_cast<float*>(bn + Q * NN);
    wt = lam + Q;
  };

  int b, h, seg;
  unit_of_idx(pid, total, k.heads, k.nseg, &b, &h, &seg);
  const int64_t unit = (int64_t)b * k.heads + h;
  const int c0 = seg * k.seg_chunks, c1 = min(c0 + k.seg_chunks, k.nchunks);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;
  const T* __restrict__ Ap = static_cast<const T*>(REV ? k.dy : k.x);
  const int64_t as = REV ? k.dys : k.xs;
  const T* __restrict__ Bp = static_cast<const T*>(REV ? k.C : k.B);
  const int64_t bs = REV ? k.cs : k.bs;
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah2 = k.A[h] * kLog2e;

  // this wave's tiles (pt0 + t, nt), rows in the paired order of prow()
  const int tile0 = wave * TPW;
  const bool owns = NTILE >= kBWaves * TPW || tile0 < NTILE;  // known true when every wave owns
  const int nt = tile0 / TP, pt0 = tile0 % TP;
  f32x4 acc[TPW];
  {
    const float* vin = nullptr;
    if (!REV && seg == 0 && k.h0) vin = k.h0 + ((int64_t)b * k.n_heads + h) * (P * N);
    if (REV && seg + 1 == k.nseg && k.dhT) vin = k.dhT + ((int64_t)b * k.n_heads + h) * (P * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[t][i] = (vin && owns) ? vin[prow(pt0 + t, g * 4 + i) * N + nt * 16 + r16] : 0.0f;
    // the start value's loads complete here, before any chunk is loaded ahead
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = opaque(acc[t]);
  }
  float lam_seg = 0.0f;  // log2 decay over the walked chunks
  float* const lamc = k.nseg > 1 ? (REV ? k.lamg : k.lamh) : nullptr;
  T* __restrict__ Vst = static_cast<T*>(REV ? k.gst : k.hst) +
                        unit * (REV ? k.nchunks : k.nchunks + 1) * (P * N);
  // V after chunk c (REV: before the update with chunk c), in its stored layout
  auto store_v = [&](int c) {
    if (!owns) return;
    T* dst = Vst + (int64_t)c * (P * N);
#pragma unroll
    for (int t = 0; t < TPW; t += 2) store8(dst + state_frag<N>((pt0 + t) / 2, nt, lane), acc[t], acc[t + 1]);
  };

  u32x4 pa[2][NAV], pb[2][NBV];
  float pdt[2];
  int plen[2] = {0, 0};
  auto prefetch = [&](int c, auto set) {
    constexpr int S = decltype(set)::value;
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
    // every load unconditional, at a clamped row (rows past len are zeroed
    // at staging): a load under a lane condition is waited for at its branch.
    // Consecutive lanes read along a row, so a wave reads whole rows.
#pragma unroll
    for (int v = 0; v < NAV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (P / VB) - 1), s = min(idx / (P / VB), len - 1);
      // this head's rows, not read again by the walk: nontemporal (about 1.5%
      // of the call; the B and C rows, shared by the heads, stay cached)
      pa[S][v] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(Ap + (row0 + s) * as + (int64_t)h * P + (idx % (P / VB)) * VB));
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = min(tid + v * kBThreads, Q * (N / VB) - 1), s = min(idx / (N / VB), len - 1);
      pb[S][v] = *reinterpret_cast<const u32x4*>(Bp + (row0 + s) * bs + (idx % (N / VB)) * VB);
    }
    // dt: wave 0 only (the other waves' range is empty); tokens past len read 0
    pdt[S] = buffer_elem<T>(uniform_rsrc(DTp + row0 * k.dts + h, wave == 0 ? (uint32_t)(len * k.dts * sizeof(T)) : 0u),
                            (uint32_t)(lane * k.dts * sizeof(T)));
    plen[S] = len;
  };
  auto step = [&](int c, int parity, auto set) {
    constexpr int S = decltype(set)::value;
    T *an, *bn;
    float *lam, *wt;
    buf(parity, an, bn, lam, wt);
    store_v(c);  // the state before chunk c, or dL/dH at its end
    if (lamc && tid == 0) lamc[unit * k.nchunks + c] = lam_seg;
    const int len = plen[S];
#pragma unroll
    for (int v = 0; v < NAV; ++v) {
      const int idx = tid + v * kBThreads, s = idx / (P / VB);
      const u32x4 raw = opaque(pa[S][v]);
      if (idx < Q * (P / VB))
        *reinterpret_cast<u32x4*>(an + s * NP + (idx % (P / VB)) * VB) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = tid + v * kBThreads, s = idx / (N / VB);
      const u32x4 raw = opaque(pb[S][v]);
      if (idx < Q * (N / VB))
        *reinterpret_cast<u32x4*>(bn + s * NN + (idx % (N / VB)) * VB) = s < len ? raw : u32x4{0u, 0u, 0u, 0u};
    }
    if (wave == 0) {
      const float d = opaque(pdt[S]);
      const float lv = chunk_cumsum(d * Ah2, lane);
      const float le = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), 63));
      lam[lane] = lv;
      wt[lane] = REV ? __builtin_amdgcn_exp2f(lv) : __builtin_amdgcn_exp2f(le - lv) * d;
    }
    // one barrier per chunk: this buffer is staged, and every wave is done
    // with the other one (read by the chunk before), which the next chunk
    // stages
    __syncthreads();
    // issued on every step, clamped at the segment's last chunk in walk order
    prefetch(REV ? max(c - 2, c0) : min(c + 2, c1 - 1), set);
    lam_seg += lam[Q - 1];
    if (owns) {
      const float dec = __builtin_amdgcn_exp2f(lam[Q - 1]);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] *= dec;
#pragma unroll
      for (int ks = 0; ks < Q / 32; ++ks) {
        const int tq = ks * 32 + g * 8;
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wt + tq);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wt + tq + 4);
        Frag8<T> br, bf;
        frag_cols(br, bn, NN, tq, tq + 4, nt * 16, 4, lane);
#pragma unroll
        for (int j = 0; j < 8; ++j) frag_set(bf, j, to_f32(br.v[j]) * (j < 4 ? w0[j] : w1[j - 4]));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> af;
          frag_cols(af, an, NP, tq, tq + 4, ((pt0 + t) >> 1) * 32 + ((pt0 + t) & 1) * 4, 8, lane);
          acc[t] = mma(af, bf, acc[t]);
        }
      }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // every segment walked here holds at least one chunk (c0 < c1), so every
  // clamped chunk index below is a valid one
  if (!REV) {
    prefetch(min(c0, c1 - 1), S0{});
    prefetch(min(c0 + 1, c1 - 1), S1{});
    int c = c0;
    for (; c + 1 < c1; c += 2) {
      step(c, 0, S0{});
      step(c + 1, 1, S1{});
    }
    if (c < c1) step(c, 0, S0{});
  } else {
    prefetch(c1 - 1, S0{});
    prefetch(max(c1 - 2, c0), S1{});
    int c = c1 - 1;
    for (; c - 1 >= c0; c -= 2) {
      step(c, 0, S0{});
      step(c - 1, 1, S1{});
    }
    if (c >= c0) step(c, 0, S0{});
  }
  if (!REV && c1 == k.nchunks) store_v(k.nchunks);
  if (k.nseg > 1) {
    if (REV || seg + 1 < k.nseg) {
      float* dst = (REV ? k.seg_g : k.seg_h) + (unit * k.nseg + seg) * (P * N);
      if (owns)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[(nt * 16 + r16) * P + prow(pt0 + t, g * 4 + i)] = acc[t][i];
      if (tid == 0) (REV ? k.seg_gd : k.seg_hd)[unit * k.nseg + seg] = lam_seg;
    }
  } else if (REV && k.dh0 && owns) {
    float* dst = k.dh0 + ((int64_t)b * k.n_heads + h) * (P * N);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* q = dst + prow(pt0 + t, g * 4 + i) * N + nt * 16 + r16;
        *q = k.accumulate ? *q + acc[t][i] : acc[t][i];
      }
  }
}

// Both walks of the call in one launch, independent of each other:
// workgroups [0, total/2) walk forward storing the state before every chunk,
// the rest walk backwards storing dL/dH at the end of every chunk.  dA and dD
// are sums that the chunk kernel (launched after this one) adds into with
// fp32 atomics: unless the call accumulates, the first workgroup clears them.
template <typename T, int P, int N>
__global__ __launch_bounds__(kBThreads) void bwd_walks_kernel(BwdK k) {
  const int half = gridDim.x / 2;
  if (blockIdx.x == 0 && !k.accumulate) {
    for (int i = threadIdx.x; i < k.heads; i += kBThreads) {
      k.dA[i] = 0.0f;
      if (k.dD) k.dD[i] = 0.0f;
    }
  }
  if ((int)blockIdx.x < half) walk<T, P, N, false>(k, blockIdx.x, half);
  else walk<T, P, N, true>(k, blockIdx.x - half, half);
}

// Chains the segments of every unit, one thread per state element (n-major
// index e = n P + p).  Forward: slot s holds segment s's end state from its
// own start (h0 for segment 0, zero after); the start of segment s+1 is
// exp2(hd_s) (start of s) + slot s, written to slot s of seg_hb.  Backward:
// slot s holds dL/dH at segment s's start from its own end value (dL/dH of
// the final state for the last segment, zero before); dL/dH at the end of
// segment s-1 is exp2(gd_s) (that at the end of s) + slot s, written to
// slot s of seg_gb, and dh0 is exp2(gd_0) (dL/dH at the end of segment 0) +
// slot 0.  The chains run in fp32; the boundary values are stored in the
// storage type, as the walks store theirs.  The slots of both chains are
// loaded eight at a time before their part of the chains (one load round
// trip per eight segments, not one per segment).
template <typename T, int P, int N>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdK k) {
  constexpr int kG = 8, PN = P * N;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = blockIdx.y;
  const int b = (int)(unit / k.heads), h = (int)(unit % k.heads);
  if (e >= PN) return;
  float st = 0.0f, gr = 0.0f;
  const float* hs = k.seg_h + unit * k.nseg * PN + e;
  const float* gs = k.seg_g + unit * k.nseg * PN + e;
  T* hb = static_cast<T*>(k.seg_hb) + unit * k.nseg * PN + e;
  T* gb = static_cast<T*>(k.seg_gb) + unit * k.nseg * PN + e;
  const float* hd = k.seg_hd + unit * k.nseg;
  const float* gd = k.seg_gd + unit * k.nseg;
  const int npre = k.nseg - 1;  // forward slots 0..npre-1, backward slots npre..1
  for (int i0 = 0; i0 < npre; i0 += kG) {
    float Hs[kG], Gs[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {  // (slot index clamped: every load valid)
      const int s = min(i0 + i, npre - 1);
      Hs[i] = hs[(int64_t)s * PN];
      Gs[i] = gs[(int64_t)(npre - s) * PN];
    }
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const int s = i0 + i;
      if (s < npre) {
        st = __builtin_amdgcn_exp2f(hd[s]) * st + Hs[i];
        hb[(int64_t)s * PN] = from_f32<T>(st);
        gr = __builtin_amdgcn_exp2f(gd[npre - s]) * gr + Gs[i];
        gb[(int64_t)(npre - s) * PN] = from_f32<T>(gr);
      }
    }
  }
  if (k.dh0) {
    const float v = __builtin_amdgcn_exp2f(gd[0]) * gr + gs[0];
    float* q = k.dh0 + ((int64_t)b * k.n_heads + h) * PN + (e % P) * N + e / P;
    *q = k.accumulate ? *q + v : v;
  }
}

// LDS of the chunk kernel: the chunk's x, dy, B, C rows token-major, Gc
// n-major, the start state Hp as stored (fragment order) and the masked Q x Q
// matrices M, K (rows s) and Kd (rows t); products that need another
// orientation read columns with transpose loads (frag_cols), so no
// transposed copy is kept (119 KB at d_head 64, d_state 128 in bf16).
template <typename T, int P, int N>
struct ChunkLds {
  // row pitches: 16-bit x, dy and Gc^T rows padded by 32 bytes rather than
  // 16 (fewer bank conflicts in their transpose loads: about 1% of the call)
  static constexpr int NP = P + (sizeof(T) == 2 ? 16 : bpad<T>());   // token-major x and dy rows
  static constexpr int NN = N + bpad<T>();                           // token-major B and C rows
  static constexpr int TP2 = P + (sizeof(T) == 2 ? 16 : bpad<T>());  // Gc^T rows (n-major)
  static constexpr int QP = kBQ + bpad<T>();  // M, K, Kd rows
  static constexpr size_t elems = (size_t)2 * kBQ * NP + (size_t)2 * kBQ * NN + (size_t)N * TP2 +
                                  (size_t)P * N + (size_t)3 * kBQ * QP;
  static constexpr int kHeadFloats = 4 * kBQ + 2 * 4 * kBQ + 3 * 4 * kBQ + 2 * kCWaves;
  static constexpr int kFloats = 2 * kHeadFloats;  // by head parity
  // per launch (at most kGH heads): dt of the chunk [head][token] in the
  // storage type, ddt [head][token] fp32, and per head A, D, dA, dD
  static constexpr int kGH = 64;
  static constexpr int DTP = kBQ + 2, DDP = kBQ + 1;
  static constexpr size_t bytes = elems * sizeof(T) + kFloats * sizeof(float) +
                                  ((size_t)kGH * DTP * sizeof(T) + 3) / 4 * 4 +
                                  ((size_t)kGH * DDP + 4 * kGH) * sizeof(float);
};

// Sum over the 64 lanes, in every lane: row sums by DPP, then the four rows'
// sums read from lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  auto rl = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l)); };
  return (rl(0) + rl(16)) + (rl(32) + rl(48));
}

// v of lane ^ m (an LDS permute whose address is formed from the caller's
// lane index, so that it is formed where used)
__device__ __forceinline__ float xor_lane(float v, int lane, int m) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, v)));
}

// ACC: add into the caller's dx, ddt, dB and dC (else overwrite them).
//
// One workgroup of 16 waves per (sequence, chunk) loops over heads
// [h0g, h0g + hg), at most 64; the walks have stored, per head, the state
// before the chunk (Hp) and dL/dH at its end (Gc).  Once per chunk: the B and
// C rows and the dt, A and D of the heads are staged and the Q x Q blocks of
// B_s . C_t on and below the diagonal formed (waves 0-9, one 16 x 16 block
// each, kept in registers: they do not depend on the head).
// Per head, after staging its x, dy, Hp and Gc:
//  phase 1: dy_t . x_s on the same blocks, the masked decay, and from them
//    M = G dec, K = Q dec (both [s][t]) and Kd = K dt_s ([t][s]) in LDS with
//    the row and column sums of W; the wave's u tile's end-state term
//    exp(Lambda_e - Lambda_s) B_s Gc^T, its dB tiles' exp(..) x_s Gc, its dC
//    tiles' exp(Lambda_t) dy_t Hp, and part of <Gc, Hp>;
//  phase 2: u += M dy, dB += K C, dC += Kd B; dx; dB and dC added to their
//    sums over the heads (registers);
//  tail (wave 0): dLambda from the partial sums, its suffix sum, ddt, dA and
//    dD, left in LDS.
// The chunk's end state is H_e = exp(Lambda_e) Hp + sum_s exp(Lambda_e -
// Lambda_s) dt_s x_s B_s^T, so <Gc, H_e> = exp(Lambda_e) <Gc, Hp> + the sum
// over s of the end-state dLambda terms.  After the loop: ddt is written as
// whole token rows of the group's heads, dA and dD one atomic per head, dB
// and dC once (a later group's launch adds into them): no dB/dC atomics.  Every partial sum is written by one
// wave and summed in a fixed order: the results do not depend on timing.
template <typename T, int P, int N, bool ACC, bool SPLIT>
__global__ __launch_bounds__(kCThreads) void bwd_chunk_kernel(BwdK k) {
  using L = ChunkLds<T, P, N>;
  constexpr int Q = kBQ, NP = L::NP, NN = L::NN, TP2 = L::TP2, QP = L::QP;
  constexpr int TP = P / 16, TN = N / 16;
  constexpr int NKB = (N + 31) / 32;  // K=32 slices over d_state
  constexpr int PKB = P / 32;         // K=32 slices over d_head
  constexpr int VB = 16 / (int)sizeof(T);
  constexpr int NBLK = Q / 16;        // 16-token blocks per chunk
  static_assert(NBLK == 4 && Q % 32 == 0, "four 16-token blocks per chunk");
  static_assert(P % 32 == 0 && TP % 2 == 0, "d_head is a whole number of K=32 slices");
  static_assert(sizeof(T) == 4 || N % 32 == 0, "16-bit tiles are read in whole K=32 slices");
  constexpr int NU = NBLK * TP, UPW = (NU + kCWaves - 1) / kCWaves;  // u tiles, per wave
  constexpr int ND = NBLK * TN, DPW = (ND + kCWaves - 1) / kCWaves;  // dB (and dC) tiles, per wave
  static_assert(UPW == 1 && TN % DPW == 0, "one u tile per wave; a wave's dB tiles share a block");
  constexpr int NQ = TN / DPW;                 // dB / dC partials per 16-token block
  constexpr int NFR = (P / 32) * TN;           // state fragments (for <Gc, Hp>)
  static_assert(NFR <= kCWaves, "at most one state fragment per wave");
  constexpr int NQQ = NBLK * (NBLK + 1) / 2;  // Q x Q blocks on and below the diagonal
  static_assert(NQQ <= kCWaves, "one Q x Q block per wave");
  constexpr int NXY = (2 * Q * (P / VB) + kCThreads - 1) / kCThreads;  // x, dy vectors per thread
  constexpr int NBC = (2 * Q * (N / VB) + kCThreads - 1) / kCThreads;  // B, C vectors per thread
  constexpr int NHV = (P * (N / VB) + kCThreads - 1) / kCThreads;      // Hp (and Gc) vectors per thread

  extern __shared__ __align__(16) unsigned char smem[];
  T* Xn = reinterpret_cast<T*>(smem);  // [Q][NP]
  T* Yn = Xn + Q * NP;                 // dy [Q][NP]
  T* Bn = Yn + Q * NP;                 // [Q][NN]
  T* Cn = Bn + Q * NN;                 // [Q][NN]
  T* GT = Cn + Q * NN;                 // Gc^T [N][TP2]
  T* HpF = GT + N * TP2;               // Hp, fragment order [P * N]
  T* Mq = HpF + P * N;                 // M [s][t]
  T* Kq = Mq + Q * QP;                 // K [s][t]
  T* Kd = Kq + Q * QP;                 // K dt_s, [t][s]
  // Per-head values, two sets by head parity: the tail of a head runs
  // during phase 1 of the next one.
  float* const fbase = reinterpret_cast<float*>(Kd + Q * QP);
  constexpr int kGH = L::kGH, DTP = L::DTP, DDP = L::DDP;
  T* const dtS = reinterpret_cast<T*>(fbase + L::kFloats);  // [kGH][DTP]
  float* const ddtS = reinterpret_cast<float*>(dtS) + ((size_t)kGH * DTP * sizeof(T) + 3) / 4;  // [kGH][DDP]
  float* const ADs = ddtS + kGH * DDP;  // A, D, dA, dD of the launch's heads
  struct HeadF {
    float *lam, *dtv, *eL, *sc, *rpart, *cpart, *t1p, *esp, *expl, *hgw, *ddw;
  };
  auto head_floats = [&](int parity) {
    HeadF f;
    f.lam = fbase + parity * L::kHeadFloats;  // log2-scaled Lambda
    f.dtv = f.lam + Q;
    f.eL = f.dtv + Q;              // exp(Lambda_t)
    f.sc = f.eL + Q;               // exp(Lambda_e - Lambda_s)
    f.rpart = f.sc + Q;            // [sb][t]: sum over s in block sb of W[t][s]
    f.cpart = f.rpart + NBLK * Q;  // [tb][s]: sum over t in block tb of W[t][s]
    f.t1p = f.cpart + NBLK * Q;    // [q][t]: exp(Lambda_t) dy_t . Hp C_t over d_state part q
    f.esp = f.t1p + 4 * Q;         // [q][s]: dt_s exp(..) x_s^T Gc B_s over d_state part q
    f.expl = f.esp + 4 * Q;        // [pt][s]: x_s . u_s over d_head tile pt
    f.hgw = f.expl + 4 * Q;        // [16]: <Gc, Hp> per wave
    f.ddw = f.hgw + kCWaves;       // [16]: dy . x per wave
    return f;
  };

  // (sequence, chunk) of this workgroup: consecutive chunks on one XCD, so
  // that the chunks of a segment share its boundary values in that XCD's L2
  // (split calls)
  const int total = (int)gridDim.x, pid = (int)blockIdx.x;
  const int uid = total % kXcds == 0 ? (pid % kXcds) * (total / kXcds) + pid / kXcds : pid;
  const int c = uid % k.nchunks, b = uid / k.nchunks;
  const int64_t row0 = (int64_t)b * k.seqlen + (int64_t)c * Q;
  const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;
  const T* __restrict__ Xp = static_cast<const T*>(k.x);
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const T* __restrict__ DYp = static_cast<const T*>(k.dy);
  T* __restrict__ DXp = static_cast<T*>(k.dx);
  T* __restrict__ DDTp = static_cast<T*>(k.ddt);
  const int64_t ubase = (int64_t)b * k.heads;  // unit of head 0 of this sequence

  // this wave's tiles (wave-uniform; known when the tiles divide evenly)
  const bool uown = NU >= kCWaves || wave < NU;  // u tile: s block usb, d_head tile upt
  const int usb = wave / TP, upt = wave % TP;
  const bool down = ND >= kCWaves * DPW || wave * DPW < ND;  // dB, dC tiles: block dsb, n tiles dnt0 + j
  const int dsb = (wave * DPW) / TN, dnt0 = (wave * DPW) % TN, dq = dnt0 / DPW;

  // ---- once per chunk: B and C rows (zero past len); M, K, Kd zeroed (the
  // blocks above the diagonal are never written) ----
#pragma unroll
  for (int v = 0; v < NBC; ++v) {
    const int idx = tid + v * kCThreads;
    const int which = idx / (Q * (N / VB)), r = idx % (Q * (N / VB));
    const int s = r / (N / VB), n0 = (r % (N / VB)) * VB;
    if (idx < 2 * Q * (N / VB)) {
      const T* src = static_cast<const T*>(which ? k.C : k.B) + (row0 + min(s, len - 1)) * (which ? k.cs : k.bs);
      const Vec16<T> bv = load16(src + n0);
      store16((which ? Cn : Bn) + s * NN + n0, s < len ? bv : zero16<T>());
    }
  }
  for (int i = tid; i < 3 * Q * QP; i += kCThreads) Mq[i] = from_f32<T>(0.0f);
  // dt of the launch's heads over the chunk, one 2- or 4-byte element per
  // lane, 64 consecutive heads of a token per wave (rows past len and heads
  // past hg read 0); A and D of the heads
  {
    const auto rdt = uniform_rsrc(DTp + row0 * k.dts + k.h0g, (uint32_t)(len * k.dts * sizeof(T)));
    for (int i = tid; i < Q * kGH; i += kCThreads) {
      const int t = i / kGH, hl = i % kGH;
      const uint32_t off = hl < k.hg ? (uint32_t)((t * k.dts + hl) * sizeof(T)) : 0x7ffffff0u;
      dtS[hl * DTP + t] = from_f32<T>(buffer_elem<T>(rdt, off));
    }
    if (tid < k.hg) {
      ADs[tid] = k.A[k.h0g + tid];
      ADs[kGH + tid] = k.D ? k.D[k.h0g + tid] : 0.0f;
    }
  }
  __syncthreads();
  // this wave's Q x Q block (sb, tb), tb >= sb: lane slot i is s = sb*16 + 4g + i,
  // t = tb*16 + r16; gq = B_s . C_t
  int qsb = 0, qtb = wave < NQQ ? wave : 0;
  while (qtb >= NBLK - qsb) {
    qtb -= NBLK - qsb;
    ++qsb;
  }
  qtb += qsb;
  f32x4 gq = {0, 0, 0, 0};
  if (wave < NQQ) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      Frag8<T> bs, ct;
      frag_row(bs, Bn + (qsb * 16 + r16) * NN, kb * 32 + g * 8, N);
      frag_row(ct, Cn + (qtb * 16 + r16) * NN, kb * 32 + g * 8, N);
      gq = mma(bs, ct, gq);
    }
  }

  // Per-head rows (x, dy), dt, Hp and Gc into registers (all issued before
  // any is used): loaded during the head before.  Waves 0-7 read x rows,
  // waves 8-15 dy rows, one 16-byte vector per thread, consecutive lanes
  // along a row (a wave reads whole rows: a lane per row had made every load
  // touch 64 cache lines and the vector memory unit the bottleneck of the
  // head boundary), through a range over
  // the chunk's rows of the head (rows past len read 0); Hp and Gc through
  // ranges over their blocks (threads past a block's end read 0).  Offsets
  // are 32-bit: a load costs one address add, not 64-bit row arithmetic.
  static_assert(NXY == 1 && 2 * Q * (P / VB) == kCThreads, "one x or dy vector per thread");
  static_assert(NHV == 1, "at most one Hp and one Gc vector per thread");
  Vec16<T> vxy[NXY], vh[NHV], vg[NHV];
  // split calls: the chained values at the chunk's segment boundaries at
  // this thread's Hp and Gc elements, and the log2 decays from them
  Vec16<T> vsh, vsg;
  float lsh = 0.0f, lsg = 0.0f;
  const bool is_dy = wave >= kCWaves / 2;
  const uint32_t xy_rb = (uint32_t)((is_dy ? k.dys : k.xs) * (int64_t)sizeof(T));  // row bytes
  const T* const xy0 = is_dy ? DYp + row0 * k.dys : Xp + row0 * k.xs;
  auto vec_at = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec16<T> v;
    *reinterpret_cast<uint4*>(v.v) = buffer_load16<kPolicyDefault>(r, off);
    return v;
  };
  auto load_head = [&](int hh, int tid, int lane) {
    const int64_t unit = ubase + hh;
    const unsigned r = (unsigned)tid % (Q * (P / VB)), s = r / (P / VB), p0 = (r % (P / VB)) * VB;
    vxy[0] = vec_at(uniform_rsrc(xy0 + (int64_t)hh * P, (uint32_t)len * xy_rb),
                    s * xy_rb + p0 * (unsigned)sizeof(T));
    constexpr uint32_t kHB = (uint32_t)(P * N * sizeof(T));
    const T* hp = static_cast<const T*>(k.hst) + (unit * (k.nchunks + 1) + c) * (P * N);
    const T* gp = static_cast<const T*>(k.gst) + (unit * k.nchunks + c) * (P * N);
    vh[0] = vec_at(uniform_rsrc(hp, kHB), (uint32_t)tid * 16u);
    vg[0] = vec_at(uniform_rsrc(gp, kHB), (uint32_t)tid * 16u);
    if constexpr (SPLIT) {
      // the walks of a split call start each segment from its own boundary
      // value (zero inside the sequence); the recurrence being linear, the
      // chained value at that boundary (n-major, from the combine) decayed
      // to the chunk is added here.  At the sequence's ends there is none:
      // the empty ranges read 0.
      const int sg = c / k.seg_chunks;
      const unsigned e = (unsigned)tid * VB, fid = e / 512, ln = (e / 8) % 64, j0 = e % 8;
      const unsigned n = (fid % TN) * 16 + ln % 16, p = (fid / TN) * 32 + (ln / 16) * 8 + j0;
      const uint32_t off = (n * P + p) * (uint32_t)sizeof(T);
      const T* hb = static_cast<const T*>(k.seg_hb) + (unit * k.nseg + max(sg - 1, 0)) * (P * N);
      const T* gb = static_cast<const T*>(k.seg_gb) + (unit * k.nseg + min(sg + 1, k.nseg - 1)) * (P * N);
      vsh = vec_at(uniform_rsrc(hb, sg > 0 ? kHB : 0u), off);
      vsg = vec_at(uniform_rsrc(gb, sg + 1 < k.nseg ? kHB : 0u), off);
      lsh = k.lamh[unit * k.nchunks + c];
      lsg = k.lamg[unit * k.nchunks + c];
    }
  };
  f32x4 abt[DPW], act[DPW];  // dB, dC summed over the heads
#pragma unroll
  for (int j = 0; j < DPW; ++j) abt[j] = act[j] = f32x4{0, 0, 0, 0};

  const int tid_o = tid;
  load_head(k.h0g, opaque(tid_o), opaque(tid_o) % 64);
  // Every head issues its dx stores after the next head's loads, and the
  // staging waits for those loads with the stores still in flight.  The loop
  // is entered with nothing issued after the first loads; the compiler merges
  // the two entries and would wait for every store.  So the entry issues as
  // many memory operations after them: stores through an empty range, which
  // the hardware drops (at offsets far apart, so that they are not merged).
  {
    constexpr int kOps = (ACC ? 8 : 4) * UPW;
    const auto none = uniform_rsrc(k.dA, 0u);
#pragma unroll
    for (int i = 0; i < kOps; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, i * 256, 0, 0);
  }
  // outputs of this chunk through buffer resources over its rows: lanes at
  // rows past len fall outside the range and are dropped, so no store sits
  // under a lane condition (which would make every later wait for a load
  // also wait for all earlier stores)
  const auto rdb = uniform_rsrc(k.dB + row0 * k.dbs, (uint32_t)(len * k.dbs * sizeof(float)));
  const auto rdc = uniform_rsrc(k.dC + row0 * k.dcs, (uint32_t)(len * k.dcs * sizeof(float)));

  // ---- tail of head th (one wave): dLambda -> da (suffix sum) -> ddt, dA, dD
  // of the head into LDS (written out once per chunk) ----
  auto run_tail = [&](int th, int lane) {
    const HeadF F = head_floats(th & 1);
    const int thl = th - k.h0g;
    const float Ah = ADs[thl];
    {
      const int t = lane, tb = t / 16;
      // fixed summation order: the result does not depend on wave timing
      float t1 = 0.0f, es = 0.0f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        t1 += F.t1p[q * Q + t];
        es += F.esp[q * Q + t];
      }
      float dl = t1 - es;
#pragma unroll
      for (int sb = 0; sb < NBLK; ++sb) dl += sb <= tb ? F.rpart[sb * Q + t] : 0.0f;
#pragma unroll
      for (int b2 = 0; b2 < NBLK; ++b2) dl -= b2 >= tb ? F.cpart[b2 * Q + t] : 0.0f;
      // <Gc, H_e> at the chunk's last token
      float hp = 0.0f;
#pragma unroll
      for (int j = 0; j < NFR; ++j) hp += F.hgw[j];
      const float hg = F.eL[Q - 1] * hp + wave_sum(es);
      if (t == Q - 1) dl += hg;
      // suffix sum over t' >= t: the total minus the prefix before t
      const float incl = wave_incl_scan(dl);
      const float tot = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
      const float suf = (tot - incl) + dl;
      float xu = 0.0f;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) xu += F.expl[pt * Q + t];
      // dt is 0 past len, so dA takes nothing from those tokens
      ddtS[thl * DDP + t] = xu + Ah * suf;
      const float da = wave_sum(F.dtv[t] * suf);
      float ddh = 0.0f;
#pragma unroll
      for (int j = 0; j < kCWaves; ++j) ddh += F.ddw[j];
      if (lane == 0) {
        ADs[2 * kGH + thl] = da;
        ADs[3 * kGH + thl] = ddh;
      }
    }
  };

  const int hend = k.h0g + k.hg;
  for (int hh = k.h0g; hh < hend; ++hh) {
    // The lane indices, re-derived every head from an opaque copy: the LDS
    // and global addresses built from them are then formed inside the loop
    // rather than hoisted out of it and held across it.
    const int tid = opaque(tid_o), lane = tid & 63, r16 = lane & 15, g = lane >> 4;
    const float Ah = ADs[hh - k.h0g];
    const float Dh = ADs[kGH + hh - k.h0g];
    const HeadF F = head_floats(hh & 1);

    // ---- stage this head: x, dy rows token-major (zero past len), Hp as
    // stored, Gc as n-major rows; wave 0: Lambda and its factors ----
    {
      const unsigned r = (unsigned)tid % (Q * (P / VB)), s = r / (P / VB), p0 = (r % (P / VB)) * VB;
      store16((is_dy ? Yn : Xn) + s * NP + p0, vxy[0]);
    }
    if ((unsigned)tid < P * (N / VB)) {
      const unsigned idx = tid;
      Vec16<T> hv = vh[0], gv = vg[0];
      if constexpr (SPLIT) {
        const float eh = __builtin_amdgcn_exp2f(lsh), eg = __builtin_amdgcn_exp2f(lsg);
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          hv.v[j] = from_f32<T>(to_f32(hv.v[j]) + eh * to_f32(vsh.v[j]));
          gv.v[j] = from_f32<T>(to_f32(gv.v[j]) + eg * to_f32(vsg.v[j]));
        }
      }
      store16(HpF + idx * VB, hv);
      // Gc in fragment order: element e of the block is lane ln's value j0
      // of fragment (kp, nb), i.e. row n = nb*16 + ln%16, column
      // p = kp*32 + (ln/16)*8 + j0 of Gc^T
      const unsigned e = idx * VB, fid = e / 512, ln = (e / 8) % 64, j0 = e % 8;
      const unsigned n = (fid % TN) * 16 + ln % 16, p = (fid / TN) * 32 + (ln / 16) * 8 + j0;
      store16(GT + n * TP2 + p, gv);
    }
    if (wave == 0) {
      const float dtl = to_f32(dtS[(hh - k.h0g) * DTP + lane]);  // 0 past len
      const float lv = chunk_cumsum(dtl * Ah * kLog2e, lane);
      const float le = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv), 63));
      F.lam[lane] = lv;
      F.dtv[lane] = dtl;
      F.eL[lane] = __builtin_amdgcn_exp2f(lv);
      F.sc[lane] = __builtin_amdgcn_exp2f(le - lv);
    }
    __syncthreads();
    // the next head's inputs (this one's again at the last), in flight
    // while this one is computed
    load_head(min(hh + 1, hend - 1), tid, lane);

    // ================= phase 1 =================
    // the previous head's tail on wave kTailWave: its Q x Q block leaves it
    // the most slack before the phase-1 barrier (a barrier-wait probe: waves
    // 0-3 waited ~20% of the loop there, and the tail on the last wave, whose
    // tiles fill phase 1, made that wave the one every other waited for)
    if (wave == kTailWave && hh > k.h0g) run_tail(hh - 1, lane);
    // ---- the wave's Q x Q block: x_s . dy_t, masked decay, M, K, Kd, W sums ----
    if (wave < NQQ) {
      f32x4 qq = {0, 0, 0, 0};
#pragma unroll
      for (int kp = 0; kp < PKB; ++kp) {
        Frag8<T> xs, yt;
        frag_load8(xs, Xn + (qsb * 16 + r16) * NP + kp * 32 + g * 8);
        frag_load8(yt, Yn + (qtb * 16 + r16) * NP + kp * 32 + g * 8);
        qq = mma(xs, yt, qq);
      }
      const int t = qtb * 16 + r16, s4 = qsb * 16 + g * 4;
      const float lam_t = F.lam[t];
      const f32x4 lam_s = *reinterpret_cast<const f32x4*>(F.lam + s4);
      const f32x4 dt_s = *reinterpret_cast<const f32x4*>(F.dtv + s4);
      float w[4], kd[4], rs = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dec = t >= s4 + i ? __builtin_amdgcn_exp2f(lam_t - lam_s[i]) : 0.0f;
        const float m = gq[i] * dec, kk = qq[i] * dec;
        Mq[(s4 + i) * QP + t] = from_f32<T>(m);
        Kq[(s4 + i) * QP + t] = from_f32<T>(kk);
        kd[i] = kk * dt_s[i];
        w[i] = m * qq[i] * dt_s[i];
        rs += w[i];
      }
      store4(Kd + t * QP + s4, kd[0], kd[1], kd[2], kd[3]);
      // row sums (over s, per t): over the 4 slots, then the 4 groups
      rs += xor_lane(rs, lane, 16);
      rs += xor_lane(rs, lane, 32);
      if (g == 0) F.rpart[qsb * Q + t] = rs;
      // column sums (over t, per s): over the 16 lanes of each group
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = row16_sum(w[i]);
      if (r16 == 0) *reinterpret_cast<f32x4*>(F.cpart + qtb * Q + s4) = f32x4{w[0], w[1], w[2], w[3]};
    }
    // ---- <Gc, Hp> over the wave's state fragment (kp, nb) ----
    if (NFR >= kCWaves || wave < NFR) {
      const int kp = wave / TN, nb = wave % TN;
      Frag8<T> hf, gf;
      frag_load8(hf, HpF + state_frag<N>(kp, nb, lane));
      frag_load8(gf, GT + (nb * 16 + r16) * TP2 + kp * 32 + g * 8);
      float v = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) v += to_f32(hf.v[j]) * to_f32(gf.v[j]);
      v = wave_sum(v);
      if (lane == 0) F.hgw[wave] = v;
    }
    // ---- u tile (usb, upt): exp(Lambda_e - Lambda_s) B_s Gc^T ----
    f32x4 au = {0, 0, 0, 0};
    if (uown) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        Frag8<T> bf, gf;
        frag_row(bf, Bn + (usb * 16 + r16) * NN, kb * 32 + g * 8, N);
        frag_cols(gf, GT, TP2, kb * 32 + g * 8, kb * 32 + g * 8 + 4, upt * 16, 4, lane, kb * 32 + g * 8 < N);
        au = mma(bf, gf, au);
      }
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(F.sc + usb * 16 + g * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) au[i] *= s4[i];
    }
    // ---- dB tiles (dsb, dnt0 + j): exp(..) x_s Gc, and its part of esum;
    // dC tiles (same block index as t block): exp(Lambda_t) dy_t Hp, and its
    // part of t1 ----
    f32x4 ab[DPW], ac[DPW];
#pragma unroll
    for (int j = 0; j < DPW; ++j) ab[j] = ac[j] = f32x4{0, 0, 0, 0};
    if (down) {
#pragma unroll
      for (int kp = 0; kp < PKB; ++kp) {
        Frag8<T> xf, yf;
        frag_load8(xf, Xn + (dsb * 16 + r16) * NP + kp * 32 + g * 8);
        frag_load8(yf, Yn + (dsb * 16 + r16) * NP + kp * 32 + g * 8);
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          Frag8<T> gf, hfr;
          frag_load8(gf, GT + ((dnt0 + j) * 16 + r16) * TP2 + kp * 32 + g * 8);
          frag_load8(hfr, HpF + state_frag<N>(kp, dnt0 + j, lane));
          ab[j] = mma(xf, gf, ab[j]);
          ac[j] = mma(yf, hfr, ac[j]);
        }
      }
      const int s4 = dsb * 16 + g * 4;
      const f32x4 scs = *reinterpret_cast<const f32x4*>(F.sc + s4);
      const f32x4 dts = *reinterpret_cast<const f32x4*>(F.dtv + s4);
      const f32x4 et = *reinterpret_cast<const f32x4*>(F.eL + s4);
      float e[4], f[4];
      f32x4 bc[DPW], cc[DPW];  // B, C at rows s4 + i, columns of the wave's tiles
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        bc[j] = col4(Bn, NN, s4, (dnt0 + j) * 16, lane);
        cc[j] = col4(Cn, NN, s4, (dnt0 + j) * 16, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.0f, u = 0.0f;
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          ab[j][i] *= scs[i];
          ac[j][i] *= et[i];
          v += ab[j][i] * bc[j][i];
          u += ac[j][i] * cc[j][i];
        }
        e[i] = row16_sum(v) * dts[i];
        f[i] = row16_sum(u);
      }
      if (r16 == 0) {
        *reinterpret_cast<f32x4*>(F.esp + dq * Q + s4) = f32x4{e[0], e[1], e[2], e[3]};
        *reinterpret_cast<f32x4*>(F.t1p + dq * Q + s4) = f32x4{f[0], f[1], f[2], f[3]};
      }
    }
    __syncthreads();

    // ================= phase 2 =================
    float dd = 0.0f;
    // ---- u += M dy over t >= s (K = t slices from the block's own) ----
    if (uown) {
#pragma unroll 1
      for (int ks = usb / 2; ks < Q / 32; ++ks) {
        Frag8<T> mf, yf;
        frag_load8(mf, Mq + (usb * 16 + r16) * QP + ks * 32 + g * 8);
        frag_cols(yf, Yn, NP, ks * 32 + g * 8, ks * 32 + g * 8 + 4, upt * 16, 4, lane);
        au = mma(mf, yf, au);
      }
      // dx = dt_s u + D dy; x_s . u_s over this d_head tile; dy . x
      const auto rdx = uniform_rsrc(DXp + row0 * k.dxs + (int64_t)hh * P, (uint32_t)(len * k.dxs * sizeof(T)));
      const int s4 = usb * 16 + g * 4, p = upt * 16 + r16;
      const f32x4 dts = *reinterpret_cast<const f32x4*>(F.dtv + s4);
      float ex[4], dxv[4], old[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        old[i] = ACC ? buffer_elem<T>(rdx, (uint32_t)(((s4 + i) * k.dxs + p) * sizeof(T))) : 0.0f;
      const f32x4 xc = col4(Xn, NP, s4, upt * 16, lane), yc = col4(Yn, NP, s4, upt * 16, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xv = xc[i], yv = yc[i];
        ex[i] = xv * au[i];
        dd += xv * yv;
        dxv[i] = dts[i] * au[i] + Dh * yv;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        buffer_store_elem<T>(rdx, (uint32_t)(((s4 + i) * k.dxs + p) * sizeof(T)), old[i] + dxv[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ex[i] = row16_sum(ex[i]);
      if (r16 == 0) *reinterpret_cast<f32x4*>(F.expl + upt * Q + s4) = f32x4{ex[0], ex[1], ex[2], ex[3]};
    }
    dd = wave_sum(dd);
    if (lane == 0) F.ddw[wave] = dd;
    if (down) {
      // ---- dB += K C over t >= s; dB summed over heads with dt_s ----
#pragma unroll 1
      for (int ks = dsb / 2; ks < Q / 32; ++ks) {
        Frag8<T> kf;
        frag_load8(kf, Kq + (dsb * 16 + r16) * QP + ks * 32 + g * 8);
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          Frag8<T> cf;
          frag_cols(cf, Cn, NN, ks * 32 + g * 8, ks * 32 + g * 8 + 4, (dnt0 + j) * 16, 4, lane);
          ab[j] = mma(kf, cf, ab[j]);
        }
      }
      // ---- dC += Kd B over s <= t ----
#pragma unroll 1
      for (int ks = 0; ks <= dsb / 2; ++ks) {
        Frag8<T> kf;
        frag_load8(kf, Kd + (dsb * 16 + r16) * QP + ks * 32 + g * 8);
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          Frag8<T> bf;
          frag_cols(bf, Bn, NN, ks * 32 + g * 8, ks * 32 + g * 8 + 4, (dnt0 + j) * 16, 4, lane);
          ac[j] = mma(kf, bf, ac[j]);
        }
      }
      const f32x4 dts = *reinterpret_cast<const f32x4*>(F.dtv + dsb * 16 + g * 4);
#pragma unroll
      for (int j = 0; j < DPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          abt[j][i] += dts[i] * ab[j][i];
          act[j][i] += ac[j][i];
        }
    }
    __syncthreads();

    // (the tail of this head reads its values during the next head's phase 1;
    // they are rewritten two heads later)
  }

  if (wave == kTailWave) run_tail(hend - 1, opaque(lane));
  __syncthreads();
  // ---- ddt of the launch's heads (64 consecutive heads of a token per wave,
  // rows past len and heads past hg dropped), then dA and dD, one head per
  // lane ----
  {
    const auto rdt = uniform_rsrc(DDTp + row0 * k.ddts + k.h0g, (uint32_t)(len * k.ddts * sizeof(T)));
    for (int i = tid; i < Q * kGH; i += kCThreads) {
      const int t = i / kGH, hl = i % kGH;
      const uint32_t off = hl < k.hg ? (uint32_t)((t * k.ddts + hl) * sizeof(T)) : 0x7ffffff0u;
      const float old = ACC ? buffer_elem<T>(rdt, off) : 0.0f;
      buffer_store_elem<T>(rdt, off, old + ddtS[hl * DDP + t]);
    }
    static_assert(kGH == 64, "one head per lane");
    if (wave == 0) {
      const auto rdA = uniform_rsrc(k.dA + k.h0g, (uint32_t)(k.hg * sizeof(float)));
      const auto rdD = uniform_rsrc(k.dD + k.h0g, k.dD ? (uint32_t)(k.hg * sizeof(float)) : 0u);
      const int off = lane < k.hg ? lane * 4 : 0x7ffffff0;
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(ADs[2 * kGH + lane], rdA, off, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(ADs[3 * kGH + lane], rdD, off, 0, 0);
    }
  }

  // ---- dB and dC of this chunk, summed over the heads ----
  const bool acc_bc = ACC || k.bc_acc;
  if (down) {
    const int s4 = dsb * 16 + g * 4;
#pragma unroll
    for (int j = 0; j < DPW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = (dnt0 + j) * 16 + r16;
        const uint32_t ob = (uint32_t)(((s4 + i) * k.dbs + col) * sizeof(float));
        const uint32_t oc = (uint32_t)(((s4 + i) * k.dcs + col) * sizeof(float));
        const float pb = acc_bc ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdb, (int)ob, 0, 0)) : 0.0f;
        const float pc = acc_bc ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rdc, (int)oc, 0, 0)) : 0.0f;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pb + abt[j][i]), rdb, (int)ob, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pc + act[j][i]), rdc, (int)oc, 0, 0);
      }
  }
}

template <typename T, int P, int N>
hipError_t launch_shape(const BwdK& k, int64_t batch, hipStream_t s) {
  const unsigned units = (unsigned)(batch * k.heads);
  const size_t lds1 = WalkLds<T, P, N>::bytes, lds2 = ChunkLds<T, P, N>::bytes;
  static_assert(ChunkLds<T, P, N>::bytes <= 160 * 1024, "chunk tiles fit one CU's LDS");
  const void* fns[] = {reinterpret_cast<const void*>(&bwd_walks_kernel<T, P, N>),
                       reinterpret_cast<const void*>(&bwd_chunk_kernel<T, P, N, false, false>),
                       reinterpret_cast<const void*>(&bwd_chunk_kernel<T, P, N, true, false>),
                       reinterpret_cast<const void*>(&bwd_chunk_kernel<T, P, N, false, true>),
                       reinterpret_cast<const void*>(&bwd_chunk_kernel<T, P, N, true, true>)};
  const size_t ldss[] = {lds1, lds2, lds2, lds2, lds2};
  for (int i = 0; i < 5; ++i) {
    const hipError_t e =
        hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldss[i]);
    if (e != hipSuccess) return e;
  }
  // the two walks (states before each chunk, dL/dH after each), each segment
  // from its own start; with a split, the combine chains the segments
  const unsigned walks = units * (unsigned)k.nseg;
  hipLaunchKernelGGL((bwd_walks_kernel<T, P, N>), dim3(2 * walks), dim3(kBThreads), lds1, s, k);
  if (k.nseg > 1)
    hipLaunchKernelGGL((bwd_combine_kernel<T, P, N>), dim3((P * N + 255) / 256, units), dim3(256), 0, s, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the chunks in parallel, one launch per group of at most kGH heads (the
  // per-head dt, ddt, A, D, dA, dD of a launch live in LDS); later groups
  // add their dB, dC to the earlier ones'
  const unsigned grid = (unsigned)(batch * k.nchunks);
  constexpr int kGH = ChunkLds<T, P, N>::kGH;
  const bool split = k.nseg > 1;
  for (int g0 = 0; g0 < k.heads; g0 += kGH) {
    BwdK kg = k;
    kg.h0g = g0;
    kg.hg = std::min(kGH, k.heads - g0);
    kg.bc_acc = g0 > 0;
    const void* fn = fns[1 + (k.accumulate ? 1 : 0) + (split ? 2 : 0)];
    void* args[] = {&kg};
    e = hipLaunchKernel(fn, dim3(grid), dim3(kCThreads), args, lds2, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  // Each (sequence, head) walk is a latency-bound chain over the chunks, one
  // workgroup per direction.  With fewer than 128 (sequence, head) units the
  // sequences are cut into segments (at least 8 chunks each) so that about
  // 128 units run, one walk workgroup per CU; more segments, with walks
  // sharing CUs, measured slower (the split also adds a combine and the
  // boundary correction in the chunk kernel).
  int64_t ns = 1;
  if (units < 128) ns = std::min<int64_t>(128 / units, nc / 8);
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
  size_t bytes = align256(units * (size_t)(nc + 1) * pn * el) + align256(units * (size_t)nc * pn * el);
  if (ns > 1)
    bytes += 2 * align256(units * ns * pn * 4) + 2 * align256(units * ns * 4) +
             2 * align256(units * ns * pn * el) + 2 * align256(units * (size_t)nc * 4);
  return bytes;
}

hipError_t launch_ssd_backward(const BwdArgs& a, void* workspace, hipStream_t s) {
  BwdK k{};
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
    k.gst = w;
    w += align256(units * (size_t)k.nchunks * pn * el);
    k.seg_h = k.seg_g = k.seg_hd = k.seg_gd = k.lamh = k.lamg = nullptr;
    k.seg_hb = k.seg_gb = nullptr;
    if (k.nseg > 1) {
      k.seg_h = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * pn * 4);
      k.seg_g = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * pn * 4);
      k.seg_hd = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * 4);
      k.seg_gd = reinterpret_cast<float*>(w);
      w += align256(units * k.nseg * 4);
      k.seg_hb = w;
      w += align256(units * k.nseg * pn * el);
      k.seg_gb = w;
      w += align256(units * k.nseg * pn * el);
      k.lamh = reinterpret_cast<float*>(w);
      w += align256(units * (size_t)k.nchunks * 4);
      k.lamg = reinterpret_cast<float*>(w);
    }
  }
  // dB and dC are written whole by the chunk kernel; dA and dD are sums
  // over workgroups, cleared by the walks kernel
  if (a.dtype == MM_BF16) {
    if (a.d_state == 128) return launch_shape<bf16, 64, 128>(k, a.batch, s);
    return launch_shape<bf16, 64, 64>(k, a.batch, s);
  }
  return launch_shape<float, 32, 16>(k, a.batch, s);
}

}  // namespace mmssd
