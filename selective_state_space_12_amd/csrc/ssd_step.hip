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
    f32x4 s[kUnroll];
    float xv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * kRowsPerPass + row_in_pass;
      if (p < P) {
        s[u] = *reinterpret_cast<const f32x4*>(sbase + (int64_t)p * N + n0);
        xv[u] = to_f32(xrow[p]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + u * kRowsPerPass + row_in_pass;
      if (p < P) {
        const float xd = dtv * xv[u];
        f32x4 hn;
#pragma unroll
        for (int j = 0; j < 4; ++j) hn[j] = fmaf(alpha, s[u][j], xd * bv[j]);
        __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(sbase + (int64_t)p * N + n0));
        float part = hn[0] * cv[0] + hn[1] * cv[1] + hn[2] * cv[2] + hn[3] * cv[3];
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m, LPR);
        if (lane_in_row == 0) yrow[p] = from_f32<T>(part + Dh * xv[u]);
      }
    }
  }
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

}  // namespace mmssd
