// Host-side argument validation (see validate.h).
#include "validate.h"

#include <cstdint>
#include <utility>

namespace mmssd {

namespace {

// Largest element count accepted for any single dimension product; keeps all
// index arithmetic far from int64 overflow.
constexpr int64_t kMaxElems = int64_t(1) << 46;

bool pos(int64_t v) { return v > 0 && v < kMaxElems; }

bool mul_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= kMaxElems / b; }

// Supported (d_head, d_state) pairs of the chunked-scan kernel.
bool scan_shape_supported(int64_t P, int64_t N) {
  return (P == 32 && N == 16) || (P == 64 && N == 64) || (P == 64 && N == 128);
}

// Shapes of the scan backward: its LDS tiles (x, dy, B, C with their
// transposes, dL/dH and the chunk's start state) fit one CU for these.
bool bwd_supported(int64_t P, int64_t N, int dtype) {
  if (dtype == MM_BF16) return P == 64 && (N == 64 || N == 128);
  return P == 32 && N == 16;
}

// [p, p + bytes) and [q, q + bytes2) share a byte (NULL never overlaps).
bool ranges_overlap(const void* p, int64_t bytes, const void* q, int64_t bytes2) {
  if (!p || !q) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
  return a0 < b0 + uintptr_t(bytes2) && b0 < a0 + uintptr_t(bytes);
}

bool chunk_supported(int64_t q) {
  return q == 16 || q == 32 || q == 64 || q == 128 || q == 256;
}

}  // namespace

bool rows_aligned(const void* p, int64_t stride, int64_t elem) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((stride * elem) % 16 == 0);
}

int validate_heads_for_dim(int64_t d_model, int64_t d_inner, int64_t d_head,
                           int64_t m, const int64_t* heads_out) {
  if (!heads_out) return MM_ERR_NULL;
  if (!pos(d_model) || !pos(d_inner) || !pos(d_head)) return MM_ERR_SHAPE;
  if (d_inner % d_model != 0) return MM_ERR_SHAPE;
  if (m <= 0 || m > d_model) return MM_ERR_SLICE;
  const int64_t e = d_inner / d_model;
  if ((e * m) % d_head != 0) return MM_ERR_SLICE;
  return MM_OK;
}

int validate_conv(const void* xbc_in, int64_t in_row_stride, const void* xbc_out,
                  int64_t out_row_stride, const float* w, const float* bias,
                  const float* conv_state, int64_t batch,
                  int64_t seqlen, int64_t d_inner, int64_t d_head,
                  int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                  int dtype) {
  if (!xbc_in || !xbc_out || !w) return MM_ERR_NULL;
  const int64_t el = dtype_bytes(dtype);
  if (el == 0) return MM_ERR_DTYPE;
  if (!pos(batch) || !pos(seqlen) || !pos(d_inner) || !pos(d_head) ||
      !pos(d_state) || !pos(ngroups))
    return MM_ERR_SHAPE;
  if (d_inner % d_head != 0) return MM_ERR_SHAPE;
  if (d_head % 8 != 0 || d_state % 8 != 0) return MM_ERR_UNSUPPORTED;
  const int64_t n_heads = d_inner / d_head;
  if (n_heads_active < 1 || n_heads_active > n_heads) return MM_ERR_SLICE;
  if (!mul_ok(ngroups, d_state)) return MM_ERR_SHAPE;
  const int64_t conv_dim = d_inner + 2 * ngroups * d_state;
  if (in_row_stride < conv_dim || out_row_stride < conv_dim) return MM_ERR_SHAPE;
  if (!mul_ok(batch, seqlen) || !mul_ok(batch * seqlen, in_row_stride) ||
      !mul_ok(batch * seqlen, out_row_stride))
    return MM_ERR_SHAPE;
  if (batch > kMaxGridYZ) return MM_ERR_SHAPE;
  if (!rows_aligned(xbc_in, in_row_stride, el) || !rows_aligned(xbc_out, out_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(w) % 16 != 0) return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(bias) % 4 != 0 || reinterpret_cast<uintptr_t>(conv_state) % 4 != 0)
    return MM_ERR_ALIGN;
  // The output must not overlap the input (the window reads neighbours).
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(xbc_in);
  const uintptr_t i1 = i0 + uintptr_t(((batch * seqlen - 1) * in_row_stride + conv_dim) * el);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(xbc_out);
  const uintptr_t o1 = o0 + uintptr_t(((batch * seqlen - 1) * out_row_stride + conv_dim) * el);
  if (i0 < o1 && o0 < i1) return MM_ERR_SHAPE;
  return MM_OK;
}

int validate_ssd_shape(int64_t batch, int64_t seqlen, int64_t n_heads,
                       int64_t d_head, int64_t d_state, int64_t ngroups,
                       int64_t n_heads_active, int64_t chunk, int dtype) {
  if (dtype_bytes(dtype) == 0) return MM_ERR_DTYPE;
  if (!pos(batch) || !pos(seqlen) || !pos(n_heads) || !pos(d_head) ||
      !pos(d_state) || !pos(ngroups) || !pos(chunk))
    return MM_ERR_SHAPE;
  if (n_heads_active < 1 || n_heads_active > n_heads) return MM_ERR_SLICE;
  if (n_heads % ngroups != 0) return MM_ERR_SHAPE;
  if (batch > kMaxGridYZ || n_heads > kMaxGridYZ) return MM_ERR_SHAPE;
  if (ngroups != 1) return MM_ERR_UNSUPPORTED;
  if (!scan_shape_supported(d_head, d_state)) return MM_ERR_UNSUPPORTED;
  if (!chunk_supported(chunk)) return MM_ERR_UNSUPPORTED;
  // fp32 tiles of a 256-token chunk with d_state 128 exceed one CU's LDS.
  if (dtype == MM_F32 && d_state == 128 && chunk > 128) return MM_ERR_UNSUPPORTED;
  if (!mul_ok(batch, seqlen) || !mul_ok(n_heads, d_head) ||
      !mul_ok(batch * seqlen, n_heads * d_head) || !mul_ok(batch * n_heads, d_head * d_state))
    return MM_ERR_SHAPE;
  return MM_OK;
}

int validate_ssd_forward(const void* x, int64_t x_row_stride, const void* dt,
                         int64_t dt_row_stride, const float* A, const void* B,
                         int64_t b_row_stride, const void* C,
                         int64_t c_row_stride, const void* y,
                         int64_t y_row_stride, const float* initial_state,
                         const float* final_state, int64_t batch, int64_t seqlen,
                         int64_t n_heads, int64_t d_head, int64_t d_state,
                         int64_t ngroups, int64_t n_heads_active, int64_t chunk,
                         int dtype) {
  if (!x || !dt || !A || !B || !C || !y) return MM_ERR_NULL;
  int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                              n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  const int64_t el = dtype_bytes(dtype);
  // only the active prefix of each token row is read or written
  const int64_t xw = n_heads_active * d_head;
  const int64_t bw = ngroups * d_state;
  if (x_row_stride < xw || y_row_stride < xw || dt_row_stride < n_heads_active ||
      b_row_stride < bw || c_row_stride < bw)
    return MM_ERR_SHAPE;
  const int64_t rows = batch * seqlen;
  if (!mul_ok(rows, x_row_stride) || !mul_ok(rows, y_row_stride) ||
      !mul_ok(rows, dt_row_stride) || !mul_ok(rows, b_row_stride) ||
      !mul_ok(rows, c_row_stride))
    return MM_ERR_SHAPE;
  if (!rows_aligned(x, x_row_stride, el) || !rows_aligned(y, y_row_stride, el) ||
      !rows_aligned(B, b_row_stride, el) || !rows_aligned(C, c_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(dt) % el != 0) return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(initial_state) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(final_state) % 4 != 0)
    return MM_ERR_ALIGN;
  return MM_OK;
}

int validate_heads_per_seq(const int32_t* heads_per_seq, int64_t batch, int64_t n_heads,
                           int64_t* max_heads) {
  if (!heads_per_seq || !max_heads) return MM_ERR_NULL;
  if (!pos(batch) || !pos(n_heads)) return MM_ERR_SHAPE;
  if (batch > 256) return MM_ERR_UNSUPPORTED;
  int64_t mx = 0;
  for (int64_t b = 0; b < batch; ++b) {
    const int64_t h = heads_per_seq[b];
    if (h < 1 || h > n_heads) return MM_ERR_SLICE;
    if (h > mx) mx = h;
  }
  *max_heads = mx;
  return MM_OK;
}

int validate_ssd_forward_fused(const void* xbc, int64_t xbc_row_stride, const float* conv_w,
                               const float* conv_bias, const float* conv_state, const void* dt,
                               int64_t dt_row_stride, const float* dt_bias, int dt_softplus,
                               const float* A, const void* y, int64_t y_row_stride,
                               const float* initial_state, const float* final_state,
                               int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                               int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                               int64_t chunk, int dtype) {
  if (!xbc || !conv_w || !dt || !A || !y) return MM_ERR_NULL;
  int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                              n_heads_active, chunk, dtype);
  if (st != MM_OK) return st;
  if (dt_softplus != 0 && dt_softplus != 1) return MM_ERR_SHAPE;
  const int64_t el = dtype_bytes(dtype);
  const int64_t conv_dim = n_heads * d_head + 2 * ngroups * d_state;
  const int64_t xw = n_heads_active * d_head;
  if (xbc_row_stride < conv_dim || y_row_stride < xw || dt_row_stride < n_heads_active)
    return MM_ERR_SHAPE;
  const int64_t rows = batch * seqlen;
  if (!mul_ok(rows, xbc_row_stride) || !mul_ok(rows, y_row_stride) ||
      !mul_ok(rows, dt_row_stride))
    return MM_ERR_SHAPE;
  if (!rows_aligned(xbc, xbc_row_stride, el) || !rows_aligned(y, y_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(dt) % el != 0) return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(conv_w) % 16 != 0) return MM_ERR_ALIGN;
  const void* f32s[] = {conv_bias, conv_state, dt_bias, initial_state, final_state};
  for (const void* p : f32s)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) return MM_ERR_ALIGN;
  // y must not overlap the conv input (the scan reads its rows while storing y).
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(xbc);
  const uintptr_t i1 = i0 + uintptr_t(((rows - 1) * xbc_row_stride + conv_dim) * el);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(y);
  const uintptr_t o1 = o0 + uintptr_t(((rows - 1) * y_row_stride + xw) * el);
  if (i0 < o1 && o0 < i1) return MM_ERR_SHAPE;
  return MM_OK;
}

int validate_gated_rmsnorm(const void* y, int64_t y_row_stride, const void* z,
                           int64_t z_row_stride, const float* w, float eps, const void* out,
                           int64_t out_row_stride, int64_t rows, int64_t d, int dtype) {
  if (!y || !z || !w || !out) return MM_ERR_NULL;
  const int64_t el = dtype_bytes(dtype);
  if (el == 0) return MM_ERR_DTYPE;
  if (!pos(rows) || !pos(d) || rows > INT32_MAX || d > INT32_MAX) return MM_ERR_SHAPE;
  if (d % 8 != 0) return MM_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return MM_ERR_SHAPE;  // rejects NaN and inf too
  if (y_row_stride < d || z_row_stride < d || out_row_stride < d) return MM_ERR_SHAPE;
  if (!mul_ok(rows, y_row_stride) || !mul_ok(rows, z_row_stride) || !mul_ok(rows, out_row_stride))
    return MM_ERR_SHAPE;
  if (!rows_aligned(y, y_row_stride, el) || !rows_aligned(z, z_row_stride, el) ||
      !rows_aligned(out, out_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(w) % 16 != 0) return MM_ERR_ALIGN;
  // out may be y itself (same rows); any other overlap with y or z is refused
  auto span = [&](const void* p, int64_t stride) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return std::pair<uintptr_t, uintptr_t>(a, a + uintptr_t(((rows - 1) * stride + d) * el));
  };
  const auto o = span(out, out_row_stride), yy = span(y, y_row_stride), zz = span(z, z_row_stride);
  const bool same_as_y = out == y && out_row_stride == y_row_stride;
  if (!same_as_y && o.first < yy.second && yy.first < o.second) return MM_ERR_SHAPE;
  if (o.first < zz.second && zz.first < o.second) return MM_ERR_SHAPE;
  return MM_OK;
}

int validate_ssd_step_multi(const float* state_in, const float* state_out, const void* x_t,
                            int64_t x_row_stride, const void* dt_t, int64_t dt_row_stride,
                            const float* A, const void* B_t, int64_t b_row_stride,
                            const void* C_t, int64_t c_row_stride, const void* y_t,
                            int64_t y_row_stride, int64_t batch, int64_t ntok, int64_t n_heads,
                            int64_t d_head, int64_t d_state, int64_t ngroups,
                            int64_t n_heads_active, int dtype) {
  if (ntok < 1 || ntok > 64) return MM_ERR_SHAPE;
  if (!pos(batch) || !mul_ok(batch, ntok)) return MM_ERR_SHAPE;
  // the state shape and alignment with batch sequences
  int st = validate_ssd_step(state_in, x_t, x_row_stride, dt_t, dt_row_stride, A, B_t,
                             b_row_stride, C_t, c_row_stride, y_t, y_row_stride, batch, n_heads,
                             d_head, d_state, ngroups, n_heads_active, dtype);
  if (st != MM_OK) return st;
  // the token streams have batch * ntok rows
  if (!mul_ok(batch * ntok, x_row_stride) || !mul_ok(batch * ntok, y_row_stride) ||
      !mul_ok(batch * ntok, dt_row_stride) || !mul_ok(batch * ntok, b_row_stride) ||
      !mul_ok(batch * ntok, c_row_stride))
    return MM_ERR_SHAPE;
  if (d_head * d_state > 8192) return MM_ERR_UNSUPPORTED;  // one pass over a state
  if (reinterpret_cast<uintptr_t>(state_out) % 16 != 0) return MM_ERR_ALIGN;
  if (state_out && state_out != state_in) {
    const uintptr_t i0 = reinterpret_cast<uintptr_t>(state_in);
    const uintptr_t bytes = uintptr_t(batch * n_heads * d_head * d_state) * sizeof(float);
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(state_out);
    if (i0 < o0 + bytes && o0 < i0 + bytes) return MM_ERR_SHAPE;
  }
  return MM_OK;
}

int validate_conv_state_advance(const float* conv_state, const void* xbc, int64_t xbc_row_stride,
                                int64_t batch, int64_t ntok, int64_t d_inner, int64_t d_head,
                                int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                                int dtype) {
  if (!conv_state || !xbc) return MM_ERR_NULL;
  const int64_t el = dtype_bytes(dtype);
  if (el == 0) return MM_ERR_DTYPE;
  if (ntok < 1 || ntok > 64) return MM_ERR_SHAPE;
  if (!pos(batch) || !pos(d_inner) || !pos(d_head) || !pos(d_state) || !pos(ngroups))
    return MM_ERR_SHAPE;
  if (batch > kMaxGridYZ || d_inner % d_head != 0) return MM_ERR_SHAPE;
  const int64_t n_heads = d_inner / d_head;
  if (n_heads_active < 1 || n_heads_active > n_heads) return MM_ERR_SLICE;
  if (!mul_ok(ngroups, d_state)) return MM_ERR_SHAPE;
  const int64_t conv_dim = d_inner + 2 * ngroups * d_state;
  if (xbc_row_stride < conv_dim || !mul_ok(batch, ntok) || !mul_ok(batch * ntok, xbc_row_stride) ||
      !mul_ok(batch * 3, conv_dim))
    return MM_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(xbc) % el != 0 || reinterpret_cast<uintptr_t>(conv_state) % 4 != 0)
    return MM_ERR_ALIGN;
  return MM_OK;
}

int validate_ssd_step(const float* state, const void* x_t, int64_t x_row_stride,
                      const void* dt_t, int64_t dt_row_stride, const float* A,
                      const void* B_t, int64_t b_row_stride, const void* C_t,
                      int64_t c_row_stride, const void* y_t,
                      int64_t y_row_stride, int64_t batch, int64_t n_heads,
                      int64_t d_head, int64_t d_state, int64_t ngroups,
                      int64_t n_heads_active, int dtype) {
  if (!state || !x_t || !dt_t || !A || !B_t || !C_t || !y_t) return MM_ERR_NULL;
  const int64_t el = dtype_bytes(dtype);
  if (el == 0) return MM_ERR_DTYPE;
  if (!pos(batch) || !pos(n_heads) || !pos(d_head) || !pos(d_state) || !pos(ngroups))
    return MM_ERR_SHAPE;
  if (n_heads_active < 1 || n_heads_active > n_heads) return MM_ERR_SLICE;
  if (n_heads % ngroups != 0) return MM_ERR_SHAPE;
  if (batch > kMaxGridYZ) return MM_ERR_SHAPE;
  if (ngroups != 1) return MM_ERR_UNSUPPORTED;
  if (d_state != 16 && d_state != 32 && d_state != 64 && d_state != 128 && d_state != 256)
    return MM_ERR_UNSUPPORTED;
  const int64_t xw = n_heads_active * d_head;
  const int64_t bw = ngroups * d_state;
  if (x_row_stride < xw || y_row_stride < xw || dt_row_stride < n_heads_active ||
      b_row_stride < bw || c_row_stride < bw)
    return MM_ERR_SHAPE;
  if (!mul_ok(batch, x_row_stride) || !mul_ok(batch, y_row_stride) ||
      !mul_ok(batch, dt_row_stride) || !mul_ok(batch, b_row_stride) ||
      !mul_ok(batch, c_row_stride) || !mul_ok(batch * n_heads, d_head * d_state))
    return MM_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(state) % 16 != 0) return MM_ERR_ALIGN;
  if (!rows_aligned(B_t, b_row_stride, el) || !rows_aligned(C_t, c_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(x_t) % el != 0 || reinterpret_cast<uintptr_t>(y_t) % el != 0 ||
      reinterpret_cast<uintptr_t>(dt_t) % el != 0)
    return MM_ERR_ALIGN;
  return MM_OK;
}

int validate_ssd_step_fused(const float* state, const float* cs_in, const float* cs_out,
                            const void* xbc_t, int64_t xbc_row_stride, const float* w,
                            const float* bias, const void* dt_t, int64_t dt_row_stride,
                            const float* A, const void* y_t, int64_t y_row_stride, int64_t batch,
                            int64_t n_heads, int64_t d_head, int64_t d_state, int64_t ngroups,
                            int64_t n_heads_active, int dtype) {
  if (!state || !cs_in || !cs_out || !xbc_t || !w || !dt_t || !A || !y_t) return MM_ERR_NULL;
  const int64_t el = dtype_bytes(dtype);
  if (el == 0) return MM_ERR_DTYPE;
  if (!pos(batch) || !pos(n_heads) || !pos(d_head) || !pos(d_state) || !pos(ngroups))
    return MM_ERR_SHAPE;
  if (n_heads_active < 1 || n_heads_active > n_heads) return MM_ERR_SLICE;
  if (n_heads % ngroups != 0) return MM_ERR_SHAPE;
  if (batch > kMaxGridYZ || n_heads >= (int64_t(1) << 31)) return MM_ERR_SHAPE;
  if (ngroups != 1) return MM_ERR_UNSUPPORTED;
  if (d_state != 16 && d_state != 32 && d_state != 64 && d_state != 128 && d_state != 256)
    return MM_ERR_UNSUPPORTED;
  if (d_head % 8 != 0) return MM_ERR_UNSUPPORTED;  // the conv's channel groups
  if (d_head + 2 * d_state > 768) return MM_ERR_UNSUPPORTED;  // three conv channels per thread
  if (!mul_ok(n_heads, d_head)) return MM_ERR_SHAPE;
  const int64_t conv_dim = n_heads * d_head + 2 * d_state;
  const int64_t xw = n_heads_active * d_head;
  if (xbc_row_stride < conv_dim || y_row_stride < xw || dt_row_stride < n_heads_active)
    return MM_ERR_SHAPE;
  if (!mul_ok(batch, xbc_row_stride) || !mul_ok(batch, y_row_stride) ||
      !mul_ok(batch, dt_row_stride) || !mul_ok(batch * 3, conv_dim) ||
      !mul_ok(batch * n_heads, d_head * d_state))
    return MM_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(state) % 16 != 0 || reinterpret_cast<uintptr_t>(cs_in) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(cs_out) % 16 != 0 || reinterpret_cast<uintptr_t>(w) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(bias) % 4 != 0)
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(xbc_t) % el != 0 || reinterpret_cast<uintptr_t>(y_t) % el != 0 ||
      reinterpret_cast<uintptr_t>(dt_t) % el != 0)
    return MM_ERR_ALIGN;
  // The advanced conv state goes to a buffer of its own: it may overlap
  // neither the state it is advanced from nor the SSD state.
  const uintptr_t cb = uintptr_t(batch * 3 * conv_dim * 4);
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(cs_in), o0 = reinterpret_cast<uintptr_t>(cs_out);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(state);
  const uintptr_t sb = uintptr_t(batch * n_heads * d_head * d_state * 4);
  if ((i0 < o0 + cb && o0 < i0 + cb) || (s0 < o0 + cb && o0 < s0 + sb)) return MM_ERR_SHAPE;
  return MM_OK;
}

int validate_ssd_backward_shape(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t d_head,
                                int64_t d_state, int64_t ngroups, int64_t n_heads_active,
                                int dtype) {
  const int st = validate_ssd_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                    n_heads_active, 64, dtype);
  if (st != MM_OK) return st;
  // one workgroup per (sequence, head) walk, numbered in a 32-bit grid
  if (batch * n_heads_active >= (int64_t(1) << 31)) return MM_ERR_UNSUPPORTED;
  return bwd_supported(d_head, d_state, dtype) ? MM_OK : MM_ERR_UNSUPPORTED;
}

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
                          int64_t n_heads_active, int dtype, int accumulate) {
  if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC) return MM_ERR_NULL;
  const int st = validate_ssd_backward_shape(batch, seqlen, n_heads, d_head, d_state, ngroups,
                                             n_heads_active, dtype);
  if (st != MM_OK) return st;
  if (accumulate != 0 && accumulate != 1) return MM_ERR_SHAPE;
  const int64_t el = dtype_bytes(dtype);
  const int64_t xw = n_heads_active * d_head, hw = n_heads_active, bw = ngroups * d_state;
  if (x_row_stride < xw || dy_row_stride < xw || dx_row_stride < xw || dt_row_stride < hw ||
      ddt_row_stride < hw || b_row_stride < bw || c_row_stride < bw || db_row_stride < bw ||
      dc_row_stride < bw)
    return MM_ERR_SHAPE;
  const int64_t rows = batch * seqlen;
  const int64_t strides[] = {x_row_stride, dy_row_stride, dx_row_stride, dt_row_stride,
                             ddt_row_stride, b_row_stride, c_row_stride, db_row_stride,
                             dc_row_stride};
  for (int64_t v : strides)
    if (!mul_ok(rows, v)) return MM_ERR_SHAPE;
  if (!rows_aligned(x, x_row_stride, el) || !rows_aligned(dy, dy_row_stride, el) ||
      !rows_aligned(dx, dx_row_stride, el) || !rows_aligned(B, b_row_stride, el) ||
      !rows_aligned(C, c_row_stride, el))
    return MM_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(dt) % el != 0 || reinterpret_cast<uintptr_t>(ddt) % el != 0)
    return MM_ERR_ALIGN;
  const void* f32s[] = {D, initial_state, dfinal_state, dA, dB, dC, dD, dinitial_state};
  for (const void* p : f32s)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) return MM_ERR_ALIGN;
  // the written gradients must not overlap what the call reads or each other
  auto span = [&](int64_t stride, int64_t width, int64_t e) { return ((rows - 1) * stride + width) * e; };
  const int64_t sdx = span(dx_row_stride, xw, el), sddt = span(ddt_row_stride, hw, el);
  const int64_t sdb = span(db_row_stride, bw, 4), sdc = span(dc_row_stride, bw, 4);
  const int64_t sst = batch * n_heads * d_head * d_state * 4;
  struct R { const void* p; int64_t n; };
  const R outs[] = {{dx, sdx}, {ddt, sddt}, {dB, sdb}, {dC, sdc}, {dA, n_heads * 4},
                    {dD, n_heads * 4}, {dinitial_state, sst}};
  const R ins[] = {{x, span(x_row_stride, xw, el)}, {dy, span(dy_row_stride, xw, el)},
                   {dt, span(dt_row_stride, hw, el)}, {B, span(b_row_stride, bw, el)},
                   {C, span(c_row_stride, bw, el)}, {A, n_heads * 4}, {D, n_heads * 4},
                   {initial_state, sst}, {dfinal_state, sst}};
  for (const R& o : outs) {
    for (const R& i : ins)
      if (ranges_overlap(o.p, o.n, i.p, i.n)) return MM_ERR_SHAPE;
    for (const R& o2 : outs)
      if (&o2 != &o && ranges_overlap(o.p, o.n, o2.p, o2.n)) return MM_ERR_SHAPE;
  }
  return MM_OK;
}

int validate_conv_backward(const void* xbc_in, int64_t in_row_stride, const void* dout,
                           int64_t dout_row_stride, const void* dxbc_in, int64_t din_row_stride,
                           const float* w, const float* bias, const float* conv_state,
                           const float* dw, const float* dbias, const float* dconv_state,
                           int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_head,
                           int64_t d_state, int64_t ngroups, int64_t n_heads_active, int dtype,
                           int accumulate) {
  if (!dout || !dw) return MM_ERR_NULL;
  // the forward's checks with dxbc_in in the output's place (it must not
  // overlap the input either)
  const int st = validate_conv(xbc_in, in_row_stride, dxbc_in, din_row_stride, w, bias, conv_state,
                               batch, seqlen, d_inner, d_head, d_state, ngroups, n_heads_active,
                               dtype);
  if (st != MM_OK) return st;
  if (accumulate != 0 && accumulate != 1) return MM_ERR_SHAPE;
  const int64_t el = dtype_bytes(dtype);
  const int64_t conv_dim = d_inner + 2 * ngroups * d_state;
  const int64_t rows = batch * seqlen;
  if (dout_row_stride < conv_dim || !mul_ok(rows, dout_row_stride)) return MM_ERR_SHAPE;
  if ((seqlen + 63) / 64 > kMaxGridYZ) return MM_ERR_SHAPE;
  if (!rows_aligned(dout, dout_row_stride, el)) return MM_ERR_ALIGN;
  const void* f32s[] = {dw, dbias, dconv_state};
  for (const void* p : f32s)
    if (reinterpret_cast<uintptr_t>(p) % 4 != 0) return MM_ERR_ALIGN;
  const int64_t sdin = ((rows - 1) * din_row_stride + conv_dim) * el;
  const int64_t sdout = ((rows - 1) * dout_row_stride + conv_dim) * el;
  const int64_t sin = ((rows - 1) * in_row_stride + conv_dim) * el;
  const int64_t sst = batch * 3 * conv_dim * 4;
  struct R { const void* p; int64_t n; };
  const R outs[] = {{dxbc_in, sdin}, {dw, conv_dim * 16}, {dbias, conv_dim * 4},
                    {dconv_state, sst}};
  const R ins[] = {{xbc_in, sin}, {dout, sdout}, {w, conv_dim * 16}, {bias, conv_dim * 4},
                   {conv_state, sst}};
  for (const R& o : outs) {
    for (const R& i : ins)
      if (ranges_overlap(o.p, o.n, i.p, i.n)) return MM_ERR_SHAPE;
    for (const R& o2 : outs)
      if (&o2 != &o && ranges_overlap(o.p, o.n, o2.p, o2.n)) return MM_ERR_SHAPE;
  }
  return MM_OK;
}

}  // namespace mmssd
