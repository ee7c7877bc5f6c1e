// Causal depthwise conv1d (kernel 4) + SiLU over the [x | B | C] channels.
//
// "MatMamba: A Matryoshka State Space Model", block paragraph: the conv
// weights concatenate W_conv_x, W_conv_B and W_conv_C and the conv is
// followed by sigma = SiLU; nesting paragraph: a sub-block uses W_conv_x[0:d_i].
//
// Design: HBM-bound streaming.  A thread owns 16 bytes of channels (8 bf16 or
// 4 fp32) and a run of consecutive tokens; it keeps the three previous inputs
// in registers and slides, so every input element is loaded once per run
// (plus a three-token halo) and every output stored once, with 16-byte
// coalesced accesses across a wavefront.  Active channels are enumerated
// densely (x slice first, then B and C), so inactive channels cost nothing.
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kConvThreads = 64;
constexpr int kTokensPerRun = 32;

// SiLU(v) = v * sigmoid(v) = v / (1 + exp(-v)), with the hardware exp2 and
// reciprocal (about 1 ulp each): an IEEE division here made the kernel
// VALU-bound below the HBM rate.  Large |v| saturates correctly (exp2 -> inf,
// rcp(inf) -> 0).
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv1d_silu_kernel(
    const T* __restrict__ in, int64_t in_stride, T* __restrict__ out,
    int64_t out_stride, const float* __restrict__ w,
    const float* __restrict__ bias, float* __restrict__ conv_state, int seqlen,
    int d_inner, int d_head, int bc_dim, int heads_cap,
    const int32_t* __restrict__ heads_per_seq, int run_len, int state_in_kernel) {
  constexpr int V = Vec16<T>::kN;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * run_len;
  const int cg = blockIdx.x * kConvThreads + threadIdx.x;
  const int d_b = clamp_heads(heads_per_seq, b, heads_cap) * d_head;
  const int ngx = d_b / V;
  if (cg >= ngx + bc_dim / V || t0 >= seqlen) return;
  const int c = cg < ngx ? cg * V : d_inner + (cg - ngx) * V;
  const int conv_dim = d_inner + bc_dim;
  const int t1 = min(seqlen, t0 + run_len);

  float wk[4][V];
  float bv[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const float4 wj = *reinterpret_cast<const float4*>(w + (int64_t)(c + j) * 4);
    wk[0][j] = wj.x;
    wk[1][j] = wj.y;
    wk[2][j] = wj.z;
    wk[3][j] = wj.w;
    bv[j] = bias ? bias[c + j] : 0.0f;
  }

  const int64_t row0 = (int64_t)b * seqlen;
  // history u[t0-3], u[t0-2], u[t0-1]
  float h[3][V];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int tau = t0 - 3 + k;
    if (tau >= 0) {
      const Vec16<T> v = load16(in + (row0 + tau) * in_stride + c);
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = to_f32(v.v[j]);
    } else if (conv_state) {
      const float* sp = conv_state + ((int64_t)b * 3 + (tau + 3)) * conv_dim + c;
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = sp[j];
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = 0.0f;
    }
  }

  // tokens in groups of kGroup: issue the group's loads, then compute and store
  constexpr int kGroup = 4;
  for (int tg = t0; tg < t1; tg += kGroup) {
    Vec16<T> u[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      if (tg + i < t1) u[i] = load16(in + (row0 + tg + i) * in_stride + c);
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (tg + i < t1) {
        Vec16<T> o;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float ut = to_f32(u[i].v[j]);
          float pre = bv[j];
          pre = fmaf(wk[0][j], h[0][j], pre);
          pre = fmaf(wk[1][j], h[1][j], pre);
          pre = fmaf(wk[2][j], h[2][j], pre);
          pre = fmaf(wk[3][j], ut, pre);
          o.v[j] = from_f32<T>(silu(pre));
          h[0][j] = h[1][j];
          h[1][j] = h[2][j];
          h[2][j] = ut;
        }
        store16(out + (row0 + tg + i) * out_stride + c, o);
      }
    }
  }

  // Single run per sequence: this thread read the old state, so it may
  // overwrite it with the last three inputs.
  if (conv_state && state_in_kernel && t1 == seqlen) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      float* sp = conv_state + ((int64_t)b * 3 + k) * conv_dim + c;
#pragma unroll
      for (int j = 0; j < V; ++j) sp[j] = h[k][j];
    }
  }
}

// Several runs per sequence: the new state is the last three input rows
// (seqlen > run length >= 3), written after the conv kernel has read the old
// state (stream order).
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_state_update_kernel(
    const T* __restrict__ in, int64_t in_stride, float* __restrict__ conv_state,
    int seqlen, int d_inner, int d_head, int bc_dim, int heads_cap,
    const int32_t* __restrict__ heads_per_seq) {
  constexpr int V = Vec16<T>::kN;
  const int b = blockIdx.z;
  const int cg = blockIdx.x * kConvThreads + threadIdx.x;
  const int d_b = clamp_heads(heads_per_seq, b, heads_cap) * d_head;
  const int ngx = d_b / V;
  if (cg >= ngx + bc_dim / V) return;
  const int c = cg < ngx ? cg * V : d_inner + (cg - ngx) * V;
  const int conv_dim = d_inner + bc_dim;
  const int64_t row0 = (int64_t)b * seqlen;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const Vec16<T> v = load16(in + (row0 + seqlen - 3 + k) * in_stride + c);
    float* sp = conv_state + ((int64_t)b * 3 + k) * conv_dim + c;
#pragma unroll
    for (int j = 0; j < V; ++j) sp[j] = to_f32(v.v[j]);
  }
}

template <typename T>
hipError_t launch_typed(const ConvArgs& a, hipStream_t s) {
  constexpr int V = Vec16<T>::kN;
  const int max_groups = (int)((a.heads_cap * a.d_head + a.bc_dim) / V);
  // runs go on grid y (at most 65535 blocks): lengthen runs for very long sequences
  int64_t rl = (a.seqlen + 65534) / 65535;
  const int run_len = (int)(rl > kTokensPerRun ? rl : kTokensPerRun);
  const int runs = (int)((a.seqlen + run_len - 1) / run_len);
  const int single = runs == 1;
  dim3 grid((max_groups + kConvThreads - 1) / kConvThreads, runs, (unsigned)a.batch);
  hipLaunchKernelGGL(conv1d_silu_kernel<T>, grid, dim3(kConvThreads), 0, s,
                     static_cast<const T*>(a.in), a.in_stride, static_cast<T*>(a.out),
                     a.out_stride, a.w, a.bias, a.conv_state, (int)a.seqlen,
                     (int)a.d_inner, (int)a.d_head, (int)a.bc_dim, a.heads_cap,
                     a.heads_per_seq, run_len, single);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.conv_state || single) return e;
  dim3 g2((max_groups + kConvThreads - 1) / kConvThreads, 1, (unsigned)a.batch);
  hipLaunchKernelGGL(conv_state_update_kernel<T>, g2, dim3(kConvThreads), 0, s,
                     static_cast<const T*>(a.in), a.in_stride, a.conv_state,
                     (int)a.seqlen, (int)a.d_inner, (int)a.d_head, (int)a.bc_dim,
                     a.heads_cap, a.heads_per_seq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d_silu(const ConvArgs& a, int dtype, hipStream_t s) {
  if (dtype == MM_BF16) return launch_typed<bf16>(a, s);
  return launch_typed<float>(a, s);
}

}  // namespace mmssd
