// Single-token recurrent decode step of the selective scan.
//
// "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" (digest
// page), Strengths: linear-time recurrent inference with a fixed-size state;
// Sampling Rule: the state is updated with input-dependent discretised
// parameters.  Per active (sequence b, head h):
//     H <- exp(dt*A_h) * H + dt * x (outer) B ;  y = H . C + D_h * x
// Heads beyond the sequence's Matryoshka slice h_b ("MatMamba", nesting and
// Mix'n'Match paragraphs) are skipped, so a mixed-width batch streams only the
// states it uses.
//
// Design: HBM-bound (0.6 flop per byte).  One workgroup per (head, sequence)
// streams that head's d_head x d_state fp32 state once in and once out with
// 16-byte accesses, every load of a thread issued before the first use.  Many
// small workgroups (one 32 KB state each) stream best on MI355X.  The state is
// read with plain loads and written with nontemporal stores (measured: decode
// step 110 vs 114 us; nontemporal loads are slower).  A row of the state
// (d_state floats) is spread over d_state/4 lanes; y's dot product is a
// butterfly over those lanes.
// Also here: the same step with the causal conv folded in (one launch per
// token), the multi-token pass of speculative decoding, and the conv-state
// advance that commits its accepted tokens.
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kStepThreads = 256;

template <typename T, int LPR>  // LPR = lanes per state row = d_state / 4
__global__ __launch_bounds__(kStepThreads) void ssd_step_kernel(
    float* __restrict__ state, const T* __restrict__ x, int64_t xs,
    const T* __restrict__ dt, int64_t dts, const float* __restrict__ A,
    const T* __restrict__ Bt, int64_t bs, const T* __restrict__ Ct, int64_t cs,
    const float* __restrict__ D, T* __restrict__ y, int64_t ys, int n_heads,
    int P, int heads_cap, const int32_t* __restrict__ heads_per_seq) {
  constexpr int N = LPR * 4;
  constexpr int kRowsPerPass = kStepThreads / LPR;
  constexpr int kUnroll = 8;  // state rows in flight per thread
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  if (h >= clamp_heads(heads_per_seq, b, heads_cap)) return;

  const int lane_in_row = threadIdx.x % LPR;
  const int row_in_pass = threadIdx.x / LPR;
  const int n0 = lane_in_row * 4;

  float bv[4], cv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bv[j] = to_f32(Bt[(int64_t)b * bs + n0 + j]);
    cv[j] = to_f32(Ct[(int64_t)b * cs + n0 + j]);
  }
  const float dtv = to_f32(dt[(int64_t)b * dts + h]);
  const float alpha = exp2f(dtv * A[h] * kLog2e);
  const float Dh = D ? D[h] : 0.0f;
  float* sbase = state + ((int64_t)b * n_heads + h) * (int64_t)P * N;
  const T* xrow = x + (int64_t)b * xs + (int64_t)h * P;
  T* yrow = y + (int64_t)b * ys + (int64_t)h * P;

  for (int p0 = 0; p0 < P; p0 += kRowsPerPass * kUnroll) {
    // Loads at clamped rows, unconditionally; only the stores are guarded.
    // (A load under a lane condition is waited for at the end of its branch,
    // and then every row block waited for the previous block's stores.)
    f32x4 s[kUnroll];
    float xv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = min(p0 + u * kRowsPerPass + row_in_pass, P - 1);
      s[u] = *reinterpret_cast<const f32x4*>(sbase + (int64_t)p * N + n0);
      xv[u] = to_f32(xrow[p]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * kRowsPerPass + row_in_pass;
      const float xd = dtv * xv[u];
      f32x4 hn;
#pragma unroll
      for (int j = 0; j < 4; ++j) hn[j] = fmaf(alpha, s[u][j], xd * bv[j]);
      if (p < P)
        __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(sbase + (int64_t)p * N + n0));
      float part = hn[0] * cv[0] + hn[1] * cv[1] + hn[2] * cv[2] + hn[3] * cv[3];
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, LPR);
      if (p < P && lane_in_row == 0) yrow[p] = from_f32<T>(part + Dh * xv[u]);
    }
  }
}

// One decode token with the causal conv (kernel 4) + SiLU folded in.  The
// workgroup of (head h, sequence b) reads the token's raw [x | B | C] row and
// applies the conv to its head's x channels and to the B and C channels, in
// the conv step's fp32 order, rounding each output to the storage type (as a
// conv output stored in HBM would be).  It then updates the state exactly as
// ssd_step_kernel does.  The conv state is read from cs_in, and the advanced
// state is written to cs_out, a separate buffer, so no workgroup can overwrite
// taps that another is still reading.
//  - Head h's workgroup writes the taps of its x channels.
//  - Head 0's workgroup writes the B and C taps.
//  - Workgroups of heads outside the sequence's slice copy their x channels'
//    taps unchanged.
// So cs_out ends up exactly as the in-place conv step would leave cs_in.
// Order of work: each thread first issues the loads of one or two of the
// workgroup's d_head + 2*d_state conv channels, then its state rows, so the
// conv's inputs and the state are in flight together.  The conv outputs go
// through LDS (one barrier) to the lanes that use them.  The B and C inputs,
// taps and weights are re-read by every head of a sequence: a few KB, L2
// hits after the first head.
constexpr int kFusedConvCh = 3;  // conv channels per thread: d_head + 2*d_state <= 768

template <typename T, int LPR, bool kBias>
__global__ __launch_bounds__(kStepThreads) void ssd_step_fused_kernel(
    float* __restrict__ state, const float* __restrict__ cs_in, float* __restrict__ cs_out,
    const T* __restrict__ xbc, int64_t xbcs, const float* __restrict__ w,
    const float* __restrict__ bias, const T* __restrict__ dt, int64_t dts,
    const float* __restrict__ A, const float* __restrict__ D, T* __restrict__ y, int64_t ys,
    int n_heads, int P, int heads_cap, const int32_t* __restrict__ heads_per_seq) {
  constexpr int N = LPR * 4;
  constexpr int kRowsPerPass = kStepThreads / LPR;
  constexpr int kUnroll = 8;
  __shared__ float conv_out[kFusedConvCh * kStepThreads];  // x channels, then B, then C
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t d_inner = (int64_t)n_heads * P;
  const int64_t cd = d_inner + 2 * N;  // conv_dim
  const float* ci = cs_in + (int64_t)b * 3 * cd;
  float* co = cs_out + (int64_t)b * 3 * cd;
  const T* urow = xbc + (int64_t)b * xbcs;
  const int nch = P + 2 * N;

  if (h >= clamp_heads(heads_per_seq, b, heads_cap)) {
    // Outside the slice: the x channels' taps pass through unchanged.  Head
    // 0 still advances the B and C taps (the conv step always runs them).
    for (int i = threadIdx.x; i < 3 * P; i += kStepThreads) {
      const int k = i / P;
      const int64_t c = (int64_t)h * P + (i - k * P);
      co[k * cd + c] = ci[k * cd + c];
    }
    if (h == 0) {
      for (int i = threadIdx.x; i < 2 * N; i += kStepThreads) {
        const int64_t c = d_inner + i;
        const float u = to_f32(urow[c]), t1 = ci[cd + c], t2 = ci[2 * cd + c];
        co[c] = t1;
        co[cd + c] = t2;
        co[2 * cd + c] = u;
      }
    }
    return;
  }

  // conv channel i of the workgroup: x channel h*P + i, then B and C
  auto chan = [&](int i) -> int64_t { return i < P ? (int64_t)h * P + i : d_inner + (i - P); };
  float cu[kFusedConvCh], t0[kFusedConvCh], t1[kFusedConvCh], t2[kFusedConvCh], cb[kFusedConvCh];
  float4 wk[kFusedConvCh];
#pragma unroll
  for (int q = 0; q < kFusedConvCh; ++q) {
    if (q > 0 && q * kStepThreads >= nch) break;  // uniform: no channel in this slot
    const int i = min((int)threadIdx.x + q * kStepThreads, nch - 1);  // clamped: every load valid
    const int64_t c = chan(i);
    cu[q] = to_f32(urow[c]);
    t0[q] = ci[c];
    t1[q] = ci[cd + c];
    t2[q] = ci[2 * cd + c];
    wk[q] = *reinterpret_cast<const float4*>(w + c * 4);
    cb[q] = kBias ? bias[c] : 0.0f;
  }

  const int lane_in_row = threadIdx.x % LPR;
  const int row_in_pass = threadIdx.x / LPR;
  const int n0 = lane_in_row * 4;
  const float dtv = to_f32(dt[(int64_t)b * dts + h]);
  const float alpha = exp2f(dtv * A[h] * kLog2e);
  const float Dh = D ? D[h] : 0.0f;
  float* sbase = state + ((int64_t)b * n_heads + h) * (int64_t)P * N;
  T* yrow = y + (int64_t)b * ys + (int64_t)h * P;

  // first pass of state rows in flight before the conv is formed
  f32x4 s[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int p = min(u * kRowsPerPass + row_in_pass, P - 1);
    s[u] = *reinterpret_cast<const f32x4*>(sbase + (int64_t)p * N + n0);
  }

#pragma unroll
  for (int q = 0; q < kFusedConvCh; ++q) {
    const int i = threadIdx.x + q * kStepThreads;
    if (q > 0 && q * kStepThreads >= nch) break;
    if (i < nch) {
      float pre = cb[q];
      pre = fmaf(wk[q].x, t0[q], pre);
      pre = fmaf(wk[q].y, t1[q], pre);
      pre = fmaf(wk[q].z, t2[q], pre);
      pre = fmaf(wk[q].w, cu[q], pre);
      conv_out[i] = to_f32(from_f32<T>(silu(pre)));
      if (i < P || h == 0) {  // taps of the channels this workgroup owns
        const int64_t c = chan(i);
        co[c] = t1[q];
        co[cd + c] = t2[q];
        co[2 * cd + c] = cu[q];
      }
    }
  }
  __syncthreads();

  float bv[4], cv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bv[j] = conv_out[P + n0 + j];
    cv[j] = conv_out[P + N + n0 + j];
  }
  for (int p0 = 0; p0 < P; p0 += kRowsPerPass * kUnroll) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = min(p0 + u * kRowsPerPass + row_in_pass, P - 1);
        s[u] = *reinterpret_cast<const f32x4*>(sbase + (int64_t)p * N + n0);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * kRowsPerPass + row_in_pass;
      const float xv = conv_out[min(p, P - 1)];
      const float xd = dtv * xv;
      f32x4 hn;
#pragma unroll
      for (int j = 0; j < 4; ++j) hn[j] = fmaf(alpha, s[u][j], xd * bv[j]);
      if (p < P)
        __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(sbase + (int64_t)p * N + n0));
      float part = hn[0] * cv[0] + hn[1] * cv[1] + hn[2] * cv[2] + hn[3] * cv[3];
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, LPR);
      if (p < P && lane_in_row == 0) yrow[p] = from_f32<T>(part + Dh * xv);
    }
  }
}

// k tokens per sequence in one pass over the states (speculative decoding:
// verify a draft, then commit its accepted prefix): each workgroup reads its
// (head, sequence) state once, applies the sequence's first ntok_b tokens in
// order with exactly the single-step arithmetic, writes y for those tokens
// and, when state_out is given, the advanced state (nontemporal stores; the
// state read when ntok_b = 0).  Token t of sequence b is row b*k + t of x,
// dt, B, C and y.  All rows of a workgroup's state fit in one pass
// (P <= rows per pass x kUnroll), which the launch checks.  The per-token dot
// products bound it (a 5-step butterfly per state row and token; loading all
// tokens' inputs up front measured no faster), so up to 8 tokens the partial
// sums are kept per token and reduced together: log2(k) stages that split
// the tokens between partner lanes, then the remaining stages once.
template <typename T, int LPR, int KMAX>  // KMAX > 0: tokens' dot products reduced together
__global__ __launch_bounds__(kStepThreads) void ssd_steps_kernel(
    const float* __restrict__ state_in, float* state_out, const T* __restrict__ x, int64_t xs,
    const T* __restrict__ dt, int64_t dts, const float* __restrict__ A,
    const T* __restrict__ Bt, int64_t bs, const T* __restrict__ Ct, int64_t cs,
    const float* __restrict__ D, T* __restrict__ y, int64_t ys, int n_heads, int P,
    int heads_cap, const int32_t* __restrict__ heads_per_seq, int k,
    const int32_t* __restrict__ tokens_per_seq) {
  constexpr int N = LPR * 4;
  constexpr int kRowsPerPass = kStepThreads / LPR;
  constexpr int kUnroll = 8;
  static_assert(KMAX == 0 || (KMAX <= LPR && (KMAX & (KMAX - 1)) == 0), "tokens per lane group");
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  if (h >= clamp_heads(heads_per_seq, b, heads_cap)) return;
  int ntok = k;
  if (tokens_per_seq) ntok = min(max(tokens_per_seq[b], 0), k);

  const int lane_in_row = threadIdx.x % LPR;
  const int row_in_pass = threadIdx.x / LPR;
  const int n0 = lane_in_row * 4;
  const float Ah = A[h];
  const float Dh = D ? D[h] : 0.0f;
  const int64_t soff = ((int64_t)b * n_heads + h) * (int64_t)P * N;

  f32x4 s[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {  // clamped rows, loaded unconditionally
    const int p = min(u * kRowsPerPass + row_in_pass, P - 1);
    s[u] = *reinterpret_cast<const f32x4*>(state_in + soff + (int64_t)p * N + n0);
  }
  auto load_tok = [&](int t, float (&bv)[4], float (&cv)[4], float& dtv, float (&xv)[kUnroll]) {
    const int64_t row = (int64_t)b * k + t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bv[j] = to_f32(Bt[row * bs + n0 + j]);
      cv[j] = to_f32(Ct[row * cs + n0 + j]);
    }
    dtv = to_f32(dt[row * dts + h]);
    const T* xrow = x + row * xs + (int64_t)h * P;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = u * kRowsPerPass + row_in_pass;
      const float v = to_f32(xrow[min(p, P - 1)]);
      xv[u] = p < P ? v : 0.0f;
    }
  };
  // one token's update with the single step's arithmetic, in its order; the
  // lane's part of y's dot product for each row
  auto update = [&](float dtv, const float (&bv)[4], const float (&cv)[4],
                    const float (&xv)[kUnroll], float (&part)[kUnroll]) {
    const float alpha = exp2f(dtv * Ah * kLog2e);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float xd = dtv * xv[u];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[u][j] = fmaf(alpha, s[u][j], xd * bv[j]);
      part[u] = s[u][0] * cv[0] + s[u][1] * cv[1] + s[u][2] * cv[2] + s[u][3] * cv[3];
    }
  };
  if constexpr (KMAX > 0) {
    // Token loop with local partial sums only, then one butterfly per row for
    // all KMAX tokens: the first log2(KMAX) stages each hand half of a lane's
    // tokens to its partner (the lane keeps the other half, adding the
    // partner's value of the same token), the rest are the usual stages.
    // Every sum adds the same operands in the same order as a single step.
    float part[KMAX][kUnroll], xs0[KMAX][kUnroll];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
      float bv[4], cv[4], dtv = 0.0f, xv[kUnroll];
      if (t < ntok) {
        load_tok(t, bv, cv, dtv, xv);
        update(dtv, bv, cv, xv, part[t]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) xs0[t][u] = xv[u];
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) part[t][u] = xs0[t][u] = 0.0f;
      }
    }
    int tok = 0;  // token whose sum this lane ends up holding
#pragma unroll
    for (int cnt = KMAX, off = LPR / 2; cnt > 1; cnt >>= 1, off >>= 1) {
      const int half = cnt / 2;
      const bool hi = (lane_in_row & off) != 0;
      if (hi) tok += half;
#pragma unroll
      for (int i = 0; i < half; ++i)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const float mine = hi ? part[i + half][u] : part[i][u];
          const float send = hi ? part[i][u] : part[i + half][u];
          part[i][u] = mine + __shfl_xor(send, off, LPR);
        }
    }
#pragma unroll
    for (int off = LPR / (2 * KMAX); off >= 1; off >>= 1)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) part[0][u] += __shfl_xor(part[0][u], off, LPR);
    if ((lane_in_row & (LPR / KMAX - 1)) == 0 && tok < ntok) {
      T* yrow = y + ((int64_t)b * k + tok) * ys + (int64_t)h * P;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = u * kRowsPerPass + row_in_pass;
        float xv = 0.0f;
#pragma unroll
        for (int t = 0; t < KMAX; ++t) xv = t == tok ? xs0[t][u] : xv;
        if (p < P) yrow[p] = from_f32<T>(part[0][u] + Dh * xv);
      }
    }
  } else {
    for (int t = 0; t < ntok; ++t) {
      float bv[4], cv[4], dtv, xv[kUnroll], part[kUnroll];
      load_tok(t, bv, cv, dtv, xv);
      update(dtv, bv, cv, xv, part);
      T* yrow = y + ((int64_t)b * k + t) * ys + (int64_t)h * P;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = u * kRowsPerPass + row_in_pass;
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) part[u] += __shfl_xor(part[u], m, LPR);
        if (lane_in_row == 0 && p < P) yrow[p] = from_f32<T>(part[u] + Dh * xv[u]);
      }
    }
  }
  if (state_out) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = u * kRowsPerPass + row_in_pass;
      if (p < P)
        __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4*>(state_out + soff + (int64_t)p * N + n0));
    }
  }
}

template <typename T, int LPR, int KMAX>
void launch_multi_k(const StepMultiArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.heads_cap, (unsigned)a.batch);
  hipLaunchKernelGGL((ssd_steps_kernel<T, LPR, KMAX>), grid, dim3(kStepThreads), 0, s, a.state_in,
                     a.state_out, static_cast<const T*>(a.x), a.xs, static_cast<const T*>(a.dt),
                     a.dts, a.A, static_cast<const T*>(a.B), a.bs, static_cast<const T*>(a.C),
                     a.cs, a.D, static_cast<T*>(a.y), a.ys, a.n_heads, a.d_head, a.heads_cap,
                     a.heads_per_seq, a.ntok, a.tokens_per_seq);
}

template <typename T, int LPR>
hipError_t launch_multi_lpr(const StepMultiArgs& a, hipStream_t s) {
  constexpr int kRowsMax = (kStepThreads / LPR) * 8;
  if (a.d_head > kRowsMax) return hipErrorInvalidValue;
  if (a.ntok <= 2 && LPR >= 2) launch_multi_k<T, LPR, 2>(a, s);
  else if (a.ntok <= 4 && LPR >= 4) launch_multi_k<T, LPR, 4>(a, s);
  else if (a.ntok <= 8 && LPR >= 8) launch_multi_k<T, LPR, (LPR >= 8 ? 8 : 1)>(a, s);
  else launch_multi_k<T, LPR, 0>(a, s);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_multi_typed(const StepMultiArgs& a, hipStream_t s) {
  switch (a.d_state) {
    case 16: return launch_multi_lpr<T, 4>(a, s);
    case 32: return launch_multi_lpr<T, 8>(a, s);
    case 64: return launch_multi_lpr<T, 16>(a, s);
    case 128: return launch_multi_lpr<T, 32>(a, s);
    case 256: return launch_multi_lpr<T, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// conv_state[b] advanced by the sequence's first ntok_b raw inputs (rows
// b*k + t of xbc): the new state is the last three of (old state, those
// inputs), active channels only (x slice of heads_cap heads, then B and C).
template <typename T>
__global__ __launch_bounds__(256) void conv_state_advance_kernel(
    float* __restrict__ cstate, const T* __restrict__ xbc, int64_t xbcs, int k,
    const int32_t* __restrict__ tokens_per_seq, int64_t conv_dim, int xw, int d_inner,
    int bc_dim) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= xw + bc_dim) return;
  const int64_t c = i < xw ? i : d_inner + (i - xw);
  const int ntok = tokens_per_seq ? min(max(tokens_per_seq[b], 0), k) : k;
  float* sp = cstate + (int64_t)b * 3 * conv_dim + c;
  float v[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int t = ntok - 3 + q;  // token index; below 0: the old state's slot t + 3
    v[q] = t >= 0 ? to_f32(xbc[((int64_t)b * k + t) * xbcs + c]) : sp[(t + 3) * conv_dim];
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) sp[q * conv_dim] = v[q];
}

template <typename T, int LPR>
hipError_t launch_lpr(const StepArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.heads_cap, (unsigned)a.batch);
  hipLaunchKernelGGL((ssd_step_kernel<T, LPR>), grid, dim3(kStepThreads), 0, s, a.state,
                     static_cast<const T*>(a.x), a.xs, static_cast<const T*>(a.dt), a.dts,
                     a.A, static_cast<const T*>(a.B), a.bs, static_cast<const T*>(a.C),
                     a.cs, a.D, static_cast<T*>(a.y), a.ys, a.n_heads, a.d_head,
                     a.heads_cap, a.heads_per_seq);
  return hipGetLastError();
}

template <typename T, int LPR>
hipError_t launch_fused_lpr(const StepFusedArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_heads, (unsigned)a.batch);
  auto kern = a.bias ? ssd_step_fused_kernel<T, LPR, true> : ssd_step_fused_kernel<T, LPR, false>;
  hipLaunchKernelGGL(kern, grid, dim3(kStepThreads), 0, s, a.state, a.cs_in, a.cs_out,
                     static_cast<const T*>(a.xbc), a.xbcs, a.w, a.bias,
                     static_cast<const T*>(a.dt), a.dts, a.A, a.D, static_cast<T*>(a.y), a.ys,
                     a.n_heads, a.d_head, a.heads_cap, a.heads_per_seq);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fused_typed(const StepFusedArgs& a, hipStream_t s) {
  switch (a.d_state) {
    case 16: return launch_fused_lpr<T, 4>(a, s);
    case 32: return launch_fused_lpr<T, 8>(a, s);
    case 64: return launch_fused_lpr<T, 16>(a, s);
    case 128: return launch_fused_lpr<T, 32>(a, s);
    case 256: return launch_fused_lpr<T, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_typed(const StepArgs& a, hipStream_t s) {
  switch (a.d_state) {
    case 16: return launch_lpr<T, 4>(a, s);
    case 32: return launch_lpr<T, 8>(a, s);
    case 64: return launch_lpr<T, 16>(a, s);
    case 128: return launch_lpr<T, 32>(a, s);
    case 256: return launch_lpr<T, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_ssd_step(const StepArgs& a, int dtype, hipStream_t s) {
  if (dtype == MM_BF16) return launch_typed<bf16>(a, s);
  return launch_typed<float>(a, s);
}

hipError_t launch_ssd_step_fused(const StepFusedArgs& a, int dtype, hipStream_t s) {
  if (dtype == MM_BF16) return launch_fused_typed<bf16>(a, s);
  return launch_fused_typed<float>(a, s);
}

hipError_t launch_ssd_step_multi(const StepMultiArgs& a, int dtype, hipStream_t s) {
  if (dtype == MM_BF16) return launch_multi_typed<bf16>(a, s);
  return launch_multi_typed<float>(a, s);
}

hipError_t launch_conv_state_advance(const ConvAdvanceArgs& a, int dtype, hipStream_t s) {
  const int active = a.xw + a.bc_dim;
  dim3 grid((unsigned)((active + 255) / 256), (unsigned)a.batch);
  if (dtype == MM_BF16)
    hipLaunchKernelGGL(conv_state_advance_kernel<bf16>, grid, dim3(256), 0, s, a.conv_state,
                       static_cast<const bf16*>(a.xbc), a.xbcs, a.ntok, a.tokens_per_seq,
                       a.conv_dim, a.xw, a.d_inner, a.bc_dim);
  else
    hipLaunchKernelGGL(conv_state_advance_kernel<float>, grid, dim3(256), 0, s, a.conv_state,
                       static_cast<const float*>(a.xbc), a.xbcs, a.ntok, a.tokens_per_seq,
                       a.conv_dim, a.xw, a.d_inner, a.bc_dim);
  return hipGetLastError();
}

}  // namespace mmssd
