// Fused prefill call: the causal conv1d (kernel 4) + SiLU over [x | B | C] and
// the dt transform (dt + dt_bias, optionally through softplus) applied on the
// way into the chunked scan ("MatMamba: A Matryoshka State Space Model", block
// paragraph: the conv output feeds the SSM; the conv output itself is never
// needed outside the block, so it need not reach HBM).
//
// bf16 storage with d_head 64, d_state 128 and chunk 128/256 runs the fused
// scan kernels of ssd_fwd_bf16.hip: the tile prep kernel convolves B and C and
// transforms dt per tile, the scan's staging waves convolve x, and nothing but
// y (and the final state) is written.  Every other shape runs the conv kernel
// into the workspace, the dt transform below, then the general scan.  Either
// way the conv state, if given, is rolled last, after every read of it.
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

// state[b][k][c] <- u[seqlen - 3 + k][c] for the active channels c (x slice,
// then B and C), taking the old state where that token is before the start.
// One thread per (sequence, channel); each reads its three values before it
// writes any.
template <typename T>
__global__ __launch_bounds__(256) void conv_state_roll_kernel(const T* __restrict__ in,
                                                              int64_t in_stride,
                                                              float* __restrict__ state,
                                                              int64_t seqlen, int64_t conv_dim,
                                                              int xw, int d_inner, int bc_dim) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= xw + bc_dim) return;
  const int64_t c = i < xw ? i : d_inner + (i - xw);
  float* sp = state + (int64_t)b * 3 * conv_dim + c;
  float v[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int64_t t = seqlen - 3 + k;
    v[k] = t >= 0 ? to_f32(in[((int64_t)b * seqlen + t) * in_stride + c]) : sp[(t + 3) * conv_dim];
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) sp[k * conv_dim] = v[k];
}

// out[r][h] = dt[r][h] + dt_bias[h], through softplus if asked, rounded to the
// storage type (as a stored dt would be); heads [0, heads) of every row.
template <typename T>
__global__ __launch_bounds__(256) void dt_prepare_kernel(const T* __restrict__ dt, int64_t dts,
                                                         T* __restrict__ out,
                                                         const float* __restrict__ bias,
                                                         int softplus_on, int heads, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t r = i / heads;
  const int h = (int)(i % heads);
  float v = to_f32(dt[r * dts + h]) + (bias ? bias[h] : 0.0f);
  if (softplus_on) v = softplus(v);
  out[i] = from_f32<T>(v);
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t elem_bytes(int dtype) { return dtype == MM_BF16 ? 2 : 4; }

}  // namespace

size_t fused_workspace_bytes(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t heads,
                             int64_t d_head, int64_t d_state, int64_t chunk, int dtype) {
  if (bf16_path(d_head, d_state, chunk, dtype)) return bf16_workspace_bytes(batch, seqlen, heads);
  const size_t rows = (size_t)(batch * seqlen);
  const size_t conv_dim = (size_t)(n_heads * d_head + 2 * d_state);
  return align256(rows * conv_dim * elem_bytes(dtype)) +
         align256(rows * (size_t)heads * elem_bytes(dtype)) +
         fwd_workspace_bytes(batch, seqlen, heads, d_head, d_state, chunk, dtype);
}

hipError_t launch_ssd_forward_fused(const FusedCall& f, void* ws, hipStream_t s) {
  const int64_t d_inner = (int64_t)f.n_heads * f.d_head;
  const int64_t conv_dim = d_inner + 2 * f.d_state;
  const int64_t rows = f.batch * f.seqlen;
  const size_t el = elem_bytes(f.dtype);
  const unsigned char* xbc = static_cast<const unsigned char*>(f.xbc);
  FwdArgs a;
  a.A = f.A;
  a.D = f.D;
  a.y = f.y;
  a.ys = f.ys;
  a.h0 = f.h0;
  a.hT = f.hT;
  a.batch = f.batch;
  a.seqlen = f.seqlen;
  a.n_heads = f.n_heads;
  a.d_head = f.d_head;
  a.d_state = f.d_state;
  a.heads = f.heads;
  a.chunk = f.chunk;
  hipError_t e;
  if (bf16_path(f.d_head, f.d_state, f.chunk, f.dtype)) {
    a.x = xbc;
    a.xs = f.xbcs;
    a.B = xbc + d_inner * el;
    a.bs = f.xbcs;
    a.C = xbc + (d_inner + f.d_state) * el;
    a.cs = f.xbcs;
    a.dt = f.dt;
    a.dts = f.dts;
    FuseArgs fu;
    fu.w = f.conv_w;
    fu.bias = f.conv_bias;
    fu.state = f.conv_state;
    fu.dt_bias = f.dt_bias;
    fu.conv_dim = conv_dim;
    fu.d_inner = (int)d_inner;
    fu.softplus = f.softplus;
    e = launch_ssd_forward_bf16_fused(a, fu, ws, s);
    if (e != hipSuccess || !f.conv_state) return e;
    const int xw = f.heads * f.d_head, bc = 2 * f.d_state;
    dim3 grid((unsigned)((xw + bc + 255) / 256), (unsigned)f.batch);
    hipLaunchKernelGGL(conv_state_roll_kernel<bf16>, grid, dim3(256), 0, s,
                       static_cast<const bf16*>(f.xbc), f.xbcs, f.conv_state, f.seqlen, conv_dim,
                       xw, (int)d_inner, bc);
    return hipGetLastError();
  }
  // conv into the workspace (it rolls the conv state itself), dt transform,
  // then the general scan on the workspace rows
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* conv_out = w;
  void* dt_out = w + align256((size_t)rows * conv_dim * el);
  void* scan_ws = static_cast<unsigned char*>(dt_out) + align256((size_t)rows * f.heads * el);
  ConvArgs ca;
  ca.in = f.xbc;
  ca.in_stride = f.xbcs;
  ca.out = conv_out;
  ca.out_stride = conv_dim;
  ca.w = f.conv_w;
  ca.bias = f.conv_bias;
  ca.conv_state = f.conv_state;
  ca.batch = f.batch;
  ca.seqlen = f.seqlen;
  ca.d_inner = d_inner;
  ca.d_head = f.d_head;
  ca.bc_dim = 2 * f.d_state;
  ca.heads_cap = f.heads;
  ca.heads_per_seq = nullptr;
  e = launch_conv1d_silu(ca, f.dtype, s);
  if (e != hipSuccess) return e;
  const int64_t n = rows * f.heads;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (f.dtype == MM_BF16)
    hipLaunchKernelGGL(dt_prepare_kernel<bf16>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const bf16*>(f.dt), f.dts, static_cast<bf16*>(dt_out),
                       f.dt_bias, f.softplus, f.heads, n);
  else
    hipLaunchKernelGGL(dt_prepare_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(f.dt), f.dts, static_cast<float*>(dt_out),
                       f.dt_bias, f.softplus, f.heads, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned char* co = static_cast<const unsigned char*>(conv_out);
  a.x = co;
  a.xs = conv_dim;
  a.B = co + d_inner * el;
  a.bs = conv_dim;
  a.C = co + (d_inner + f.d_state) * el;
  a.cs = conv_dim;
  a.dt = dt_out;
  a.dts = f.heads;
  return launch_ssd_forward(a, f.dtype, scan_ws, s);
}

}  // namespace mmssd
