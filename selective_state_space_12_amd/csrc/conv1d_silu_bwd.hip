// Backward pass of the causal depthwise conv1d (kernel 4) + SiLU over the
// [x | B | C] channels ("MatMamba: A Matryoshka State Space Model", block
// paragraph for the conv and SiLU; training paragraph for the joint backward
// pass of the nested granularities).  With pre[t] = bias + sum_k w_k u[t-3+k]
// and SiLU'(v) = s (1 + v (1 - s)), s = sigmoid(v):
//   dpre[t]   = dout[t] SiLU'(pre[t])
//   du[tau]   = sum_k w_k dpre[tau + 3 - k]       (tau = -3..-1: the conv state rows)
//   dw_k     += sum_t dpre[t] u[t - 3 + k],  dbias += sum_t dpre[t]
//
// Design: HBM-bound streaming, as the forward conv.  A thread owns four
// channels and a run of 128 tokens; it slides a window of three inputs and
// three dpre values, so du[t-3] is complete once dpre[t] is known: the run
// reads three tokens past its end (the halo whose dpre reaches back into the
// run) and three before it.  The streamed rows (inputs and dout) are read
// with nontemporal loads (measured: 0.286 -> 0.258 ms at the 1.4B full
// width; runs of 128 tokens rather than 64, 0.247 ms).  The run that starts at token 0 also emits the
// conv-state rows' gradient.  A workgroup is 4 waves over 4 consecutive
// runs of the same 64 channel groups; dw and dbias are summed over each run
// in registers, over the 4 runs through LDS, and added with one fp32 atomic
// per value and workgroup (atomics on the same few thousand addresses from
// every run had made the kernel atomic-bound).
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kLanes = 64;   // channel groups per workgroup
constexpr int kRuns = 4;     // token runs per workgroup (one wave each)
constexpr int kThreads = kLanes * kRuns;
constexpr int kRun = 128;    // tokens per thread

// Four consecutive channels of one token (8 bytes of bf16, 16 of fp32): a
// thread's share.  Four rather than a 16-byte vector of bf16 keeps the
// per-thread windows and sums small enough for several waves per SIMD.
constexpr int V = 4;

template <typename T>
__device__ __forceinline__ void load4f(const T* p, float (&o)[V]) {
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


// The same for rows streamed once: a nontemporal load.
template <typename T>
__device__ __forceinline__ void load4f_nt(const T* p, float (&o)[V]) {
  if constexpr (sizeof(T) == 2) {
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    o[0] = __builtin_bit_cast(float, u[0] << 16);
    o[1] = __builtin_bit_cast(float, u[0] & 0xffff0000u);
    o[2] = __builtin_bit_cast(float, u[1] << 16);
    o[3] = __builtin_bit_cast(float, u[1] & 0xffff0000u);
  } else {
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
  }
}

template <typename T>
__device__ __forceinline__ void add_store4(T* p, const float (&v)[V], int accumulate) {
  float o[V];
  if (accumulate) {
    float old[V];
    load4f(p, old);
#pragma unroll
    for (int j = 0; j < V; ++j) o[j] = old[j] + v[j];
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) o[j] = v[j];
  }
  if constexpr (sizeof(T) == 2) {
    const bf16 b[4] = {from_f32<bf16>(o[0]), from_f32<bf16>(o[1]), from_f32<bf16>(o[2]),
                       from_f32<bf16>(o[3])};
    *reinterpret_cast<uint2*>(p) = *reinterpret_cast<const uint2*>(b);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void conv1d_silu_bwd_kernel(
    const T* __restrict__ in, int64_t in_stride, const T* __restrict__ dout, int64_t dout_stride,
    T* __restrict__ din, int64_t din_stride, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ conv_state, float* __restrict__ dw,
    float* __restrict__ dbias, float* __restrict__ dstate, int seqlen, int d_inner, int xw,
    int bc_dim, int accumulate) {
  __shared__ float red[kRuns - 1][5 * V][kLanes];
  const int b = blockIdx.z;
  const int run = threadIdx.x / kLanes, ln = threadIdx.x % kLanes;
  const int t0 = (blockIdx.y * kRuns + run) * kRun;
  const int cg = blockIdx.x * kLanes + ln;
  const int ngx = xw / V;
  // a thread past the channels or the sequence has no run but still takes
  // part in the reduction (with zeros)
  const bool active = cg < ngx + bc_dim / V && t0 < seqlen;
  const int cgc = active ? cg : 0;
  const int c = cgc < ngx ? cgc * V : d_inner + (cgc - ngx) * V;
  const int conv_dim = d_inner + bc_dim;
  const int t1 = active ? min(seqlen, t0 + kRun) : t0;
  const int tend = active ? min(seqlen, t1 + 3) : t0;  // tokens whose dpre is needed

  float wk[4][V], bv[V];
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
  // inputs u[t-3], u[t-2], u[t-1] and dpre[t-3], dpre[t-2], dpre[t-1]
  float h[3][V], dp[3][V];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int tau = t0 - 3 + k;
    if (!active) {
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = 0.0f;
    } else if (tau >= 0) {
      load4f(in + (row0 + tau) * in_stride + c, h[k]);
    } else if (conv_state) {
      const float* sp = conv_state + ((int64_t)b * 3 + (tau + 3)) * conv_dim + c;
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = sp[j];
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j) h[k][j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) dp[k][j] = 0.0f;
  }
  float sw[4][V], sb[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    sb[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) sw[k][j] = 0.0f;
  }

  // Before the run's first token the dpre window would need dpre[t0-3..t0-1],
  // which only matter for du[t0-3..t0-1] (outside the run): the window starts
  // at zero and nothing is emitted for those tokens, except the conv-state
  // rows when the run starts the sequence (dpre before token 0 is zero).
  // Tokens past the sequence end have dpre = 0.
  constexpr int kGroup = 8;  // tokens whose loads are in flight together (measured: 8 > 4, 16)
  const int tstop = active ? t1 + 3 : t0;
  // A group's loads are issued with no lane condition, at rows clamped to a
  // valid token (a load under a lane condition is waited for at the end of
  // its branch, which would serialise them); only tokens below tend are used.
  const int tlast = max(0, min(tend, seqlen) - 1);
  for (int tg = t0; tg < tstop; tg += kGroup) {
    float u[kGroup][V], go[kGroup][V];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int tc = min(tg + i, tlast);
      load4f_nt(in + (row0 + tc) * in_stride + c, u[i]);
      load4f_nt(dout + (row0 + tc) * dout_stride + c, go[i]);
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int t = tg + i;
      if (t >= tstop) break;
      float dcur[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        float d = 0.0f;
        if (t < tend) {
          const float ut = u[i][j];
          float pre = bv[j];
          pre = fmaf(wk[0][j], h[0][j], pre);
          pre = fmaf(wk[1][j], h[1][j], pre);
          pre = fmaf(wk[2][j], h[2][j], pre);
          pre = fmaf(wk[3][j], ut, pre);
          const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-pre * kLog2e));
          d = go[i][j] * s * (1.0f + pre * (1.0f - s));
          if (t < t1) {
            sw[0][j] = fmaf(d, h[0][j], sw[0][j]);
            sw[1][j] = fmaf(d, h[1][j], sw[1][j]);
            sw[2][j] = fmaf(d, h[2][j], sw[2][j]);
            sw[3][j] = fmaf(d, ut, sw[3][j]);
            sb[j] += d;
          }
          h[0][j] = h[1][j];
          h[1][j] = h[2][j];
          h[2][j] = ut;
        }
        dcur[j] = d;
      }
      // du[t-3] = w0 dpre[t] + w1 dpre[t-1] + w2 dpre[t-2] + w3 dpre[t-3]
      const int tau = t - 3;
      if (tau >= t0 || (t0 == 0 && dstate)) {
        float g[V];
#pragma unroll
        for (int j = 0; j < V; ++j)
          g[j] = wk[0][j] * dcur[j] + wk[1][j] * dp[2][j] + wk[2][j] * dp[1][j] + wk[3][j] * dp[0][j];
        if (tau >= t0) {
          add_store4(din + (row0 + tau) * din_stride + c, g, accumulate);
        } else {  // tau = -3..-1: conv state row tau + 3 (the run starts the sequence)
          float* sp = dstate + ((int64_t)b * 3 + (tau + 3)) * conv_dim + c;
#pragma unroll
          for (int j = 0; j < V; ++j) sp[j] = accumulate ? sp[j] + g[j] : g[j];
        }
      }
#pragma unroll
      for (int j = 0; j < V; ++j) {
        dp[0][j] = dp[1][j];
        dp[1][j] = dp[2][j];
        dp[2][j] = dcur[j];
      }
    }
  }
  // sums over the workgroup's runs: runs 1.. park theirs in LDS, run 0 adds
  if (run > 0) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
#pragma unroll
      for (int k = 0; k < 4; ++k) red[run - 1][k * V + j][ln] = sw[k][j];
      red[run - 1][4 * V + j][ln] = sb[j];
    }
  }
  __syncthreads();
  if (run == 0 && cg < ngx + bc_dim / V) {
#pragma unroll
    for (int r = 0; r < kRuns - 1; ++r)
#pragma unroll
      for (int j = 0; j < V; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k) sw[k][j] += red[r][k * V + j][ln];
        sb[j] += red[r][4 * V + j][ln];
      }
#pragma unroll
    for (int j = 0; j < V; ++j) {
#pragma unroll
      for (int k = 0; k < 4; ++k) unsafeAtomicAdd(dw + (int64_t)(c + j) * 4 + k, sw[k][j]);
      if (dbias) unsafeAtomicAdd(dbias + c + j, sb[j]);
    }
  }
}

// n fp32 values at p set to zero; the x slice [0, xw) and the B/C channels
// [d_inner, conv_dim) of a per-channel array (width values per channel)
__global__ __launch_bounds__(256) void zero_channels_kernel(float* p, int width, int xw,
                                                            int d_inner, int bc_dim) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= (xw + bc_dim) * width) return;
  const int ch = i / width, k = i % width;
  const int c = ch < xw ? ch : d_inner + (ch - xw);
  p[(int64_t)c * width + k] = 0.0f;
}

template <typename T>
void launch_typed(const ConvBwdArgs& a, hipStream_t s) {
  const int groups = (a.xw + a.bc_dim) / V;
  const dim3 grid((unsigned)((groups + kLanes - 1) / kLanes),
                  (unsigned)((a.seqlen + kRun * kRuns - 1) / (kRun * kRuns)), (unsigned)a.batch);
  hipLaunchKernelGGL(conv1d_silu_bwd_kernel<T>, grid, dim3(kThreads), 0, s,
                     static_cast<const T*>(a.in), a.in_stride, static_cast<const T*>(a.dout),
                     a.dout_stride, static_cast<T*>(a.din), a.din_stride, a.w, a.bias,
                     a.conv_state, a.dw, a.dbias, a.dstate, (int)a.seqlen, (int)a.d_inner, a.xw,
                     a.bc_dim, a.accumulate);
}

}  // namespace

hipError_t launch_conv1d_silu_backward(const ConvBwdArgs& a, int dtype, hipStream_t s) {
  if (!a.accumulate) {
    const int ch = a.xw + a.bc_dim;
    hipLaunchKernelGGL(zero_channels_kernel, dim3((unsigned)((ch * 4 + 255) / 256)), dim3(256), 0,
                       s, a.dw, 4, a.xw, (int)a.d_inner, a.bc_dim);
    if (a.dbias)
      hipLaunchKernelGGL(zero_channels_kernel, dim3((unsigned)((ch + 255) / 256)), dim3(256), 0,
                         s, a.dbias, 1, a.xw, (int)a.d_inner, a.bc_dim);
  }
  if (dtype == MM_BF16) launch_typed<bf16>(a, s);
  else launch_typed<float>(a, s);
  return hipGetLastError();
}

}  // namespace mmssd
