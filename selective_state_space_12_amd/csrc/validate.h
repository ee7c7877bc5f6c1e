// Host-side argument validation for the C ABI in include/mm_ssd.h.
//
// Pure C++ with no HIP calls, so it is also built with g++ (and sanitizers) on
// machines without a GPU.  Every function returns MM_OK or the MM_ERR_* code
// the header documents; nothing is enqueued before these checks pass.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/mm_ssd.h"

namespace mmssd {

// Grid dimensions y and z of a launch are limited to this many blocks.
constexpr int64_t kMaxGridYZ = 65535;

// Sizes of one element of a token-stream dtype, 0 if unknown.
inline int64_t dtype_bytes(int dtype) {
  return dtype == MM_F32 ? 4 : dtype == MM_BF16 ? 2 : 0;
}

// True when p is 16-byte aligned and stride*elem keeps every row aligned.
bool rows_aligned(const void* p, int64_t stride, int64_t elem);

int validate_heads_for_dim(int64_t d_model, int64_t d_inner, int64_t d_head,
                           int64_t m, const int64_t* heads_out);

int validate_conv(const void* xbc_in, int64_t in_row_stride, const void* xbc_out,
                  int64_t out_row_stride, const float* w, const float* bias,
                  const float* conv_state, int64_t batch,
                  int64_t seqlen, int64_t d_inner, int64_t d_head,
                  int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                  int dtype);

// Shape-only part of the scan checks (used by the workspace query too).
int validate_ssd_shape(int64_t batch, int64_t seqlen, int64_t n_heads,
                       int64_t d_head, int64_t d_state, int64_t ngroups,
                       int64_t n_heads_active, int64_t chunk, int dtype);

int validate_ssd_forward(const void* x, int64_t x_row_stride, const void* dt,
                         int64_t dt_row_stride, const float* A, const void* B,
                         int64_t b_row_stride, const void* C,
                         int64_t c_row_stride, const void* y,
                         int64_t y_row_stride, const float* initial_state,
                         const float* final_state, int64_t batch, int64_t seqlen,
                         int64_t n_heads, int64_t d_head, int64_t d_state,
                         int64_t ngroups, int64_t n_heads_active, int64_t chunk,
                         int dtype);

// Per-sequence head counts of a mixed scan call (host array): batch <= 256
// entries, each in [1, n_heads].  On success *max_heads is the widest.
int validate_heads_per_seq(const int32_t* heads_per_seq, int64_t batch, int64_t n_heads,
                           int64_t* max_heads);

int validate_ssd_forward_fused(const void* xbc, int64_t xbc_row_stride, const float* conv_w,
                               const float* conv_bias, const float* conv_state, const void* dt,
                               int64_t dt_row_stride, const float* dt_bias, int dt_softplus,
                               const float* A, const void* y, int64_t y_row_stride,
                               const float* initial_state, const float* final_state,
                               int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                               int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                               int64_t chunk, int dtype);

int validate_gated_rmsnorm(const void* y, int64_t y_row_stride, const void* z,
                           int64_t z_row_stride, const float* w, float eps, const void* out,
                           int64_t out_row_stride, int64_t rows, int64_t d, int dtype);

// mm_ssd_step_multi: the checks of validate_ssd_step for the states (batch
// sequences) and for batch * ntok token rows, plus 1 <= ntok <= 64, d_head
// within one state pass (d_head * d_state <= 8192) and state_out equal to
// state_in, NULL, or disjoint from it.
int validate_ssd_step_multi(const float* state_in, const float* state_out, const void* x_t,
                            int64_t x_row_stride, const void* dt_t, int64_t dt_row_stride,
                            const float* A, const void* B_t, int64_t b_row_stride,
                            const void* C_t, int64_t c_row_stride, const void* y_t,
                            int64_t y_row_stride, int64_t batch, int64_t ntok, int64_t n_heads,
                            int64_t d_head, int64_t d_state, int64_t ngroups,
                            int64_t n_heads_active, int dtype);

int validate_conv_state_advance(const float* conv_state, const void* xbc, int64_t xbc_row_stride,
                                int64_t batch, int64_t ntok, int64_t d_inner, int64_t d_head,
                                int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                                int dtype);

int validate_ssd_step(const float* state, const void* x_t, int64_t x_row_stride,
                      const void* dt_t, int64_t dt_row_stride, const float* A,
                      const void* B_t, int64_t b_row_stride, const void* C_t,
                      int64_t c_row_stride, const void* y_t,
                      int64_t y_row_stride, int64_t batch, int64_t n_heads,
                      int64_t d_head, int64_t d_state, int64_t ngroups,
                      int64_t n_heads_active, int dtype);

// mm_ssd_step_fused: validate_ssd_step's checks for the state, dt and y,
// validate_conv's for the raw row and the weights (d_head a multiple of 8),
// 16-byte aligned conv states, and conv_state_out overlapping neither
// conv_state_in nor the state.
int validate_ssd_step_fused(const float* state, const float* cs_in, const float* cs_out,
                            const void* xbc_t, int64_t xbc_row_stride, const float* w,
                            const float* bias, const void* dt_t, int64_t dt_row_stride,
                            const float* A, const void* y_t, int64_t y_row_stride, int64_t batch,
                            int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                            int64_t n_heads_active, int dtype);

// mm_conv1d_silu_backward: validate_conv's checks with dxbc_in as the
// output, dout's stride and alignment, accumulate 0 or 1, and no gradient
// overlapping an input or another gradient.
int validate_conv_backward(const void* xbc_in, int64_t in_row_stride, const void* dout,
                           int64_t dout_row_stride, const void* dxbc_in, int64_t din_row_stride,
                           const float* w, const float* bias, const float* conv_state,
                           const float* dw, const float* dbias, const float* dconv_state,
                           int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_head,
                           int64_t d_state, int64_t ngroups, int64_t n_heads_active, int dtype,
                           int accumulate);

// Shape part of the backward checks (used by its workspace query too).
int validate_ssd_backward_shape(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                                int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                                int dtype);

// mm_ssd_backward: the forward's checks (chunk aside) for the inputs, the
// backward's shapes ((64, 64) and (64, 128) with bf16, (32, 16) with fp32),
// strides and alignment of the gradients, accumulate 0 or 1, and no
// gradient overlapping an input or another gradient.
int validate_ssd_backward(const void* x, int64_t x_row_stride, const void* dt,
                          int64_t dt_row_stride, const float* A, const void* B,
                          int64_t b_row_stride, const void* C, int64_t c_row_stride,
                          const float* D, const float* initial_state, const void* dy,
                          int64_t dy_row_stride, const float* dfinal_state, const void* dx,
                          int64_t dx_row_stride, const void* ddt, int64_t ddt_row_stride,
                          const float* dA, const float* dB, int64_t db_row_stride,
                          const float* dC, int64_t dc_row_stride, const float* dD,
                          const float* dinitial_state, int64_t batch, int64_t seqlen,
                          int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                          int64_t n_heads_active, int dtype, int accumulate);

}  // namespace mmssd
