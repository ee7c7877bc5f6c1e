// C ABI entry points of libmmssd.so (declared in include/mm_ssd.h): validate
// on the host, then enqueue the gfx950 kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include "../../include/mm_ssd.h"
#include "kernels.h"
#include "validate.h"

using namespace mmssd;

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? MM_OK : MM_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int mm_abi_version(void) { return MM_ABI_VERSION; }

const char* mm_status_string(int status) {
  switch (status) {
    case MM_OK: return "MM_OK";
    case MM_ERR_NULL: return "MM_ERR_NULL: a required pointer is NULL";
    case MM_ERR_SHAPE: return "MM_ERR_SHAPE: a size or stride is out of range or inconsistent";
    case MM_ERR_SLICE: return "MM_ERR_SLICE: Matryoshka width or active head count is invalid";
    case MM_ERR_DTYPE: return "MM_ERR_DTYPE: unknown dtype code";
    case MM_ERR_UNSUPPORTED: return "MM_ERR_UNSUPPORTED: valid request not implemented by this build";
    case MM_ERR_ALIGN: return "MM_ERR_ALIGN: a row start is not 16-byte aligned";
    case MM_ERR_WORKSPACE: return "MM_ERR_WORKSPACE: workspace missing or too small";
    case MM_ERR_HIP: return "MM_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown mm_status code";
  }
}

int mm_heads_for_dim(int64_t d_model, int64_t d_inner, int64_t d_head, int64_t m,
                     int64_t* heads_out) {
  const int st = validate_heads_for_dim(d_model, d_inner, d_head, m, heads_out);
  if (st != MM_OK) return st;
  *heads_out = (d_inner / d_model) * m / d_head;
  return MM_OK;
}

int mm_conv1d_silu(const void* xbc_in, int64_t in_row_stride, void* xbc_out,
                   int64_t out_row_stride, const float* w, const float* bias,
                   float* conv_state, int64_t batch, int64_t seqlen, int64_t d_inner,
                   int64_t d_head, int64_t d_state, int64_t ngroups,
                   int64_t n_heads_active, const int32_t* heads_active_per_seq,
                   int dtype, void* stream) {
  const int st = validate_conv(xbc_in, in_row_stride, xbc_out, out_row_stride, w, bias,
                               conv_state, batch, seqlen, d_inner, d_head, d_state, ngroups,
                               n_heads_active, dtype);
  if (st != MM_OK) return st;
  ConvArgs a;
  a.in = xbc_in;
  a.in_stride = in_row_stride;
  a.out = xbc_out;
  a.out_stride = out_row_stride;
  a.w = w;
  a.bias = bias;
  a.conv_state = conv_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.d_inner = d_inner;
  a.d_head = d_head;
  a.bc_dim = 2 * ngroups * d_state;
  a.heads_cap = (int)n_heads_active;
  a.heads_per_seq = heads_active_per_seq;
  return hip_status(launch_conv1d_silu(a, dtype, as_stream(stream)));
}

int mm_ssd_forward_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                  int64_t d_head, int64_t d_state, int64_t ngroups,
                                  int64_t n_heads_active, int64_t chunk, int dtype,
                                  size_t* bytes_out) {
  if (!bytes_out) return MM_ERR_NULL;
  const int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                    n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  *bytes_out = fwd_workspace_bytes(batch, seqlen, n_heads_active, d_head, d_state, chunk, dtype);
  return MM_OK;
}

int mm_ssd_forward_segments(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                            int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                            int64_t chunk, int dtype, int* nseg_out) {
  if (!nseg_out) return MM_ERR_NULL;
  const int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                    n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  *nseg_out = fwd_segments(batch, seqlen, n_heads_active, d_head, d_state, chunk, dtype);
  return MM_OK;
}

int mm_ssd_forward(const void* x, int64_t x_row_stride, const void* dt,
                   int64_t dt_row_stride, const float* A, const void* B,
                   int64_t b_row_stride, const void* C, int64_t c_row_stride,
                   const float* D, void* y, int64_t y_row_stride,
                   const float* initial_state, float* final_state, int64_t batch,
                   int64_t seqlen, int64_t n_heads, int64_t d_head, int64_t d_state,
                   int64_t ngroups, int64_t n_heads_active, int64_t chunk, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_ssd_forward(x, x_row_stride, dt, dt_row_stride, A, B, b_row_stride, C,
                                c_row_stride, y, y_row_stride, initial_state, final_state,
                                batch, seqlen, n_heads, d_head, d_state, ngroups,
                                n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  const size_t need = fwd_workspace_bytes(batch, seqlen, n_heads_active, d_head, d_state, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MM_ERR_WORKSPACE;
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MM_ERR_ALIGN;
  FwdArgs a;
  a.x = x;
  a.xs = x_row_stride;
  a.dt = dt;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B;
  a.bs = b_row_stride;
  a.C = C;
  a.cs = c_row_stride;
  a.D = D;
  a.y = y;
  a.ys = y_row_stride;
  a.h0 = initial_state;
  a.hT = final_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads = (int)n_heads_active;
  a.chunk = (int)chunk;
  return hip_status(launch_ssd_forward(a, dtype, workspace, as_stream(stream)));
}

int mm_ssd_forward_nested(const void* x, int64_t x_row_stride, const void* dt,
                          int64_t dt_row_stride, const float* A, const void* B,
                          int64_t b_row_stride, const void* C, int64_t c_row_stride,
                          const float* D, void* y, int64_t y_row_stride,
                          const float* initial_state, float* final_state, int64_t batch,
                          int64_t seqlen, int64_t n_heads, int64_t d_head, int64_t d_state,
                          int64_t ngroups, int64_t n_heads_active, int64_t plan_heads,
                          int64_t chunk, int dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = validate_ssd_forward(x, x_row_stride, dt, dt_row_stride, A, B, b_row_stride, C,
                                c_row_stride, y, y_row_stride, initial_state, final_state,
                                batch, seqlen, n_heads, d_head, d_state, ngroups,
                                n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  if (plan_heads < n_heads_active || plan_heads > n_heads) return MM_ERR_SLICE;
  // the workspace of a call with plan_heads active heads covers this plan
  const size_t need = fwd_workspace_bytes(batch, seqlen, plan_heads, d_head, d_state, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MM_ERR_WORKSPACE;
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MM_ERR_ALIGN;
  FwdArgs a;
  a.x = x;
  a.xs = x_row_stride;
  a.dt = dt;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B;
  a.bs = b_row_stride;
  a.C = C;
  a.cs = c_row_stride;
  a.D = D;
  a.y = y;
  a.ys = y_row_stride;
  a.h0 = initial_state;
  a.hT = final_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads = (int)n_heads_active;
  a.chunk = (int)chunk;
  a.plan_heads = (int)plan_heads;
  return hip_status(launch_ssd_forward(a, dtype, workspace, as_stream(stream)));
}

int mm_ssd_forward_mixed_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                        int64_t d_head, int64_t d_state, int64_t ngroups,
                                        const int32_t* heads_per_seq, int64_t chunk, int dtype,
                                        size_t* bytes_out) {
  if (!bytes_out) return MM_ERR_NULL;
  int64_t mx = 0;
  int st = validate_heads_per_seq(heads_per_seq, batch, n_heads, &mx);
  if (st != MM_OK) return st;
  st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups, mx, chunk, dtype);
  if (st != MM_OK) return st;
  int64_t units = 0;
  for (int64_t b = 0; b < batch; ++b) units += heads_per_seq[b];
  *bytes_out = fwd_workspace_bytes(batch, seqlen, mx, d_head, d_state, chunk, dtype, units);
  return MM_OK;
}

int mm_ssd_forward_mixed(const void* x, int64_t x_row_stride, const void* dt,
                         int64_t dt_row_stride, const float* A, const void* B,
                         int64_t b_row_stride, const void* C, int64_t c_row_stride,
                         const float* D, void* y, int64_t y_row_stride,
                         const float* initial_state, float* final_state, int64_t batch,
                         int64_t seqlen, int64_t n_heads, int64_t d_head, int64_t d_state,
                         int64_t ngroups, const int32_t* heads_per_seq, int64_t chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int64_t mx = 0;
  int st = validate_heads_per_seq(heads_per_seq, batch, n_heads, &mx);
  if (st != MM_OK) return st;
  st = validate_ssd_forward(x, x_row_stride, dt, dt_row_stride, A, B, b_row_stride, C,
                            c_row_stride, y, y_row_stride, initial_state, final_state, batch,
                            seqlen, n_heads, d_head, d_state, ngroups, mx, chunk, dtype);
  if (st != MM_OK) return st;
  int64_t units = 0;
  for (int64_t b = 0; b < batch; ++b) units += heads_per_seq[b];
  const size_t need =
      fwd_workspace_bytes(batch, seqlen, mx, d_head, d_state, chunk, dtype, units);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MM_ERR_WORKSPACE;
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MM_ERR_ALIGN;
  FwdArgs a;
  a.x = x;
  a.xs = x_row_stride;
  a.dt = dt;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B;
  a.bs = b_row_stride;
  a.C = C;
  a.cs = c_row_stride;
  a.D = D;
  a.y = y;
  a.ys = y_row_stride;
  a.h0 = initial_state;
  a.hT = final_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads = (int)mx;
  a.chunk = (int)chunk;
  a.heads_per_seq = heads_per_seq;
  return hip_status(launch_ssd_forward(a, dtype, workspace, as_stream(stream)));
}

int mm_ssd_forward_fused_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                        int64_t d_head, int64_t d_state, int64_t ngroups,
                                        int64_t n_heads_active, int64_t chunk, int dtype,
                                        size_t* bytes_out) {
  if (!bytes_out) return MM_ERR_NULL;
  const int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                    n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  *bytes_out = fused_workspace_bytes(batch, seqlen, n_heads, n_heads_active, d_head, d_state,
                                     chunk, dtype);
  return MM_OK;
}

int mm_ssd_forward_fused(const void* xbc, int64_t xbc_row_stride, const float* conv_w,
                         const float* conv_bias, float* conv_state, const void* dt,
                         int64_t dt_row_stride, const float* dt_bias, int dt_softplus,
                         const float* A, const float* D, void* y, int64_t y_row_stride,
                         const float* initial_state, float* final_state, int64_t batch,
                         int64_t seqlen, int64_t n_heads, int64_t d_head, int64_t d_state,
                         int64_t ngroups, int64_t n_heads_active, int64_t chunk, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_ssd_forward_fused(xbc, xbc_row_stride, conv_w, conv_bias, conv_state, dt,
                                      dt_row_stride, dt_bias, dt_softplus, A, y, y_row_stride,
                                      initial_state, final_state, batch, seqlen, n_heads,
                                      d_head, d_state, ngroups, n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  const size_t need = fused_workspace_bytes(batch, seqlen, n_heads, n_heads_active, d_head,
                                            d_state, chunk, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MM_ERR_WORKSPACE;
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MM_ERR_ALIGN;
  FusedCall f;
  f.xbc = xbc;
  f.xbcs = xbc_row_stride;
  f.conv_w = conv_w;
  f.conv_bias = conv_bias;
  f.conv_state = conv_state;
  f.dt = dt;
  f.dts = dt_row_stride;
  f.dt_bias = dt_bias;
  f.softplus = dt_softplus;
  f.A = A;
  f.D = D;
  f.y = y;
  f.ys = y_row_stride;
  f.h0 = initial_state;
  f.hT = final_state;
  f.batch = batch;
  f.seqlen = seqlen;
  f.n_heads = (int)n_heads;
  f.d_head = (int)d_head;
  f.d_state = (int)d_state;
  f.heads = (int)n_heads_active;
  f.chunk = (int)chunk;
  f.dtype = dtype;
  return hip_status(launch_ssd_forward_fused(f, workspace, as_stream(stream)));
}

int mm_gated_rmsnorm(const void* y, int64_t y_row_stride, const void* z, int64_t z_row_stride,
                     const float* w, float eps, void* out, int64_t out_row_stride, int64_t rows,
                     int64_t d, int dtype, void* stream) {
  const int st = validate_gated_rmsnorm(y, y_row_stride, z, z_row_stride, w, eps, out,
                                        out_row_stride, rows, d, dtype);
  if (st != MM_OK) return st;
  NormArgs a;
  a.y = y;
  a.ys = y_row_stride;
  a.z = z;
  a.zs = z_row_stride;
  a.w = w;
  a.eps = eps;
  a.out = out;
  a.os = out_row_stride;
  a.rows = rows;
  a.d = d;
  return hip_status(launch_gated_rmsnorm(a, dtype, as_stream(stream)));
}

int mm_ssd_step_multi(const float* state_in, float* state_out, const void* x, int64_t x_row_stride,
                      const void* dt, int64_t dt_row_stride, const float* A, const void* B,
                      int64_t b_row_stride, const void* C, int64_t c_row_stride, const float* D,
                      void* y, int64_t y_row_stride, int64_t batch, int64_t ntok,
                      int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                      int64_t n_heads_active, const int32_t* heads_active_per_seq,
                      const int32_t* tokens_per_seq, int dtype, void* stream) {
  const int st = validate_ssd_step_multi(state_in, state_out, x, x_row_stride, dt, dt_row_stride,
                                         A, B, b_row_stride, C, c_row_stride, y, y_row_stride,
                                         batch, ntok, n_heads, d_head, d_state, ngroups,
                                         n_heads_active, dtype);
  if (st != MM_OK) return st;
  StepMultiArgs a;
  a.state_in = state_in;
  a.state_out = state_out;
  a.x = x;
  a.xs = x_row_stride;
  a.dt = dt;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B;
  a.bs = b_row_stride;
  a.C = C;
  a.cs = c_row_stride;
  a.D = D;
  a.y = y;
  a.ys = y_row_stride;
  a.batch = batch;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads_cap = (int)n_heads_active;
  a.heads_per_seq = heads_active_per_seq;
  a.ntok = (int)ntok;
  a.tokens_per_seq = tokens_per_seq;
  return hip_status(launch_ssd_step_multi(a, dtype, as_stream(stream)));
}

int mm_conv_state_advance(float* conv_state, const void* xbc, int64_t xbc_row_stride,
                          int64_t batch, int64_t ntok, const int32_t* tokens_per_seq,
                          int64_t d_inner, int64_t d_head, int64_t d_state, int64_t ngroups,
                          int64_t n_heads_active, int dtype, void* stream) {
  const int st = validate_conv_state_advance(conv_state, xbc, xbc_row_stride, batch, ntok,
                                             d_inner, d_head, d_state, ngroups, n_heads_active,
                                             dtype);
  if (st != MM_OK) return st;
  ConvAdvanceArgs a;
  a.conv_state = conv_state;
  a.xbc = xbc;
  a.xbcs = xbc_row_stride;
  a.batch = batch;
  a.ntok = (int)ntok;
  a.tokens_per_seq = tokens_per_seq;
  a.conv_dim = d_inner + 2 * ngroups * d_state;
  a.xw = (int)(n_heads_active * d_head);
  a.d_inner = (int)d_inner;
  a.bc_dim = (int)(2 * ngroups * d_state);
  return hip_status(launch_conv_state_advance(a, dtype, as_stream(stream)));
}

int mm_conv1d_silu_backward(const void* xbc_in, int64_t in_row_stride, const void* dout,
                            int64_t dout_row_stride, void* dxbc_in, int64_t din_row_stride,
                            const float* w, const float* bias, const float* conv_state,
                            float* dw, float* dbias, float* dconv_state, int64_t batch,
                            int64_t seqlen, int64_t d_inner, int64_t d_head, int64_t d_state,
                            int64_t ngroups, int64_t n_heads_active, int dtype, int accumulate,
                            void* stream) {
  const int st = validate_conv_backward(xbc_in, in_row_stride, dout, dout_row_stride, dxbc_in,
                                        din_row_stride, w, bias, conv_state, dw, dbias,
                                        dconv_state, batch, seqlen, d_inner, d_head, d_state,
                                        ngroups, n_heads_active, dtype, accumulate);
  if (st != MM_OK) return st;
  ConvBwdArgs a;
  a.in = xbc_in;
  a.in_stride = in_row_stride;
  a.dout = dout;
  a.dout_stride = dout_row_stride;
  a.din = dxbc_in;
  a.din_stride = din_row_stride;
  a.w = w;
  a.bias = bias;
  a.conv_state = conv_state;
  a.dw = dw;
  a.dbias = dbias;
  a.dstate = dconv_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.d_inner = d_inner;
  a.xw = (int)(n_heads_active * d_head);
  a.bc_dim = (int)(2 * ngroups * d_state);
  a.accumulate = accumulate;
  return hip_status(launch_conv1d_silu_backward(a, dtype, as_stream(stream)));
}

int mm_ssd_backward_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                   int64_t d_head, int64_t d_state, int64_t ngroups,
                                   int64_t n_heads_active, int dtype, size_t* bytes_out) {
  if (!bytes_out) return MM_ERR_NULL;
  const int st = validate_ssd_backward_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                             n_heads_active, dtype);
  if (st != MM_OK) return st;
  *bytes_out = bwd_workspace_bytes(batch, seqlen, n_heads_active, d_head, d_state, dtype);
  return MM_OK;
}

int mm_ssd_backward_segments(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                             int64_t d_state, int64_t ngroups, int64_t n_heads_active, int dtype,
                             int* nseg_out) {
  if (!nseg_out) return MM_ERR_NULL;
  const int st = validate_ssd_backward_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                             n_heads_active, dtype);
  if (st != MM_OK) return st;
  int nc, sc;
  bwd_plan(batch, seqlen, n_heads_active, &nc, nseg_out, &sc);
  return MM_OK;
}

int mm_ssd_backward(const void* x, int64_t x_row_stride, const void* dt, int64_t dt_row_stride,
                    const float* A, const void* B, int64_t b_row_stride, const void* C,
                    int64_t c_row_stride, const float* D, const float* initial_state,
                    const void* dy, int64_t dy_row_stride, const float* dfinal_state, void* dx,
                    int64_t dx_row_stride, void* ddt, int64_t ddt_row_stride, float* dA,
                    float* dB, int64_t db_row_stride, float* dC, int64_t dc_row_stride,
                    float* dD, float* dinitial_state, int64_t batch, int64_t seqlen,
                    int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                    int64_t n_heads_active, int dtype, int accumulate, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const int st = validate_ssd_backward(
      x, x_row_stride, dt, dt_row_stride, A, B, b_row_stride, C, c_row_stride, D, initial_state,
      dy, dy_row_stride, dfinal_state, dx, dx_row_stride, ddt, ddt_row_stride, dA, dB,
      db_row_stride, dC, dc_row_stride, dD, dinitial_state, batch, seqlen, n_heads, d_head,
      d_state, ngroups, n_heads_active, dtype, accumulate);
  if (st != MM_OK) return st;
  const size_t need = bwd_workspace_bytes(batch, seqlen, n_heads_active, d_head, d_state, dtype);
  if (!workspace || workspace_bytes < need) return MM_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MM_ERR_ALIGN;
  BwdArgs a;
  a.x = x;
  a.xs = x_row_stride;
  a.dt = dt;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B;
  a.bs = b_row_stride;
  a.C = C;
  a.cs = c_row_stride;
  a.D = D;
  a.h0 = initial_state;
  a.dy = dy;
  a.dys = dy_row_stride;
  a.dhT = dfinal_state;
  a.dx = dx;
  a.dxs = dx_row_stride;
  a.ddt = ddt;
  a.ddts = ddt_row_stride;
  a.dA = dA;
  a.dB = dB;
  a.dbs = db_row_stride;
  a.dC = dC;
  a.dcs = dc_row_stride;
  a.dD = dD;
  a.dh0 = dinitial_state;
  a.batch = batch;
  a.seqlen = seqlen;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads = (int)n_heads_active;
  a.dtype = dtype;
  a.accumulate = accumulate;
  return hip_status(launch_ssd_backward(a, workspace, as_stream(stream)));
}

int mm_ssd_step(float* state, const void* x_t, int64_t x_row_stride, const void* dt_t,
                int64_t dt_row_stride, const float* A, const void* B_t,
                int64_t b_row_stride, const void* C_t, int64_t c_row_stride,
                const float* D, void* y_t, int64_t y_row_stride, int64_t batch,
                int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                int64_t n_heads_active, const int32_t* heads_active_per_seq, int dtype,
                void* stream) {
  const int st = validate_ssd_step(state, x_t, x_row_stride, dt_t, dt_row_stride, A, B_t,
                                   b_row_stride, C_t, c_row_stride, y_t, y_row_stride,
                                   batch, n_heads, d_head, d_state, ngroups, n_heads_active,
                                   dtype);
  if (st != MM_OK) return st;
  StepArgs a;
  a.state = state;
  a.x = x_t;
  a.xs = x_row_stride;
  a.dt = dt_t;
  a.dts = dt_row_stride;
  a.A = A;
  a.B = B_t;
  a.bs = b_row_stride;
  a.C = C_t;
  a.cs = c_row_stride;
  a.D = D;
  a.y = y_t;
  a.ys = y_row_stride;
  a.batch = batch;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads_cap = (int)n_heads_active;
  a.heads_per_seq = heads_active_per_seq;
  return hip_status(launch_ssd_step(a, dtype, as_stream(stream)));
}

int mm_ssd_step_fused(float* state, const float* conv_state_in, float* conv_state_out,
                      const void* xbc_t, int64_t xbc_row_stride, const float* conv_w,
                      const float* conv_bias, const void* dt_t, int64_t dt_row_stride,
                      const float* A, const float* D, void* y_t, int64_t y_row_stride,
                      int64_t batch, int64_t n_heads, int64_t d_head, int64_t d_state,
                      int64_t ngroups, int64_t n_heads_active,
                      const int32_t* heads_active_per_seq, int dtype, void* stream) {
  const int st = validate_ssd_step_fused(state, conv_state_in, conv_state_out, xbc_t,
                                         xbc_row_stride, conv_w, conv_bias, dt_t, dt_row_stride,
                                         A, y_t, y_row_stride, batch, n_heads, d_head, d_state,
                                         ngroups, n_heads_active, dtype);
  if (st != MM_OK) return st;
  StepFusedArgs a;
  a.state = state;
  a.cs_in = conv_state_in;
  a.cs_out = conv_state_out;
  a.xbc = xbc_t;
  a.xbcs = xbc_row_stride;
  a.w = conv_w;
  a.bias = conv_bias;
  a.dt = dt_t;
  a.dts = dt_row_stride;
  a.A = A;
  a.D = D;
  a.y = y_t;
  a.ys = y_row_stride;
  a.batch = batch;
  a.n_heads = (int)n_heads;
  a.d_head = (int)d_head;
  a.d_state = (int)d_state;
  a.heads_cap = (int)n_heads_active;
  a.heads_per_seq = heads_active_per_seq;
  return hip_status(launch_ssd_step_fused(a, dtype, as_stream(stream)));
}

}  // extern "C"
