// Host-side launchers of the gfx950 kernels.  Arguments have been validated by
// the C ABI layer (abi.cpp) before any of these is called; each returns a
// hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace mmssd {

struct ConvArgs {
  const void* in;
  int64_t in_stride;
  void* out;
  int64_t out_stride;
  const float* w;
  const float* bias;
  float* conv_state;
  int64_t batch, seqlen, d_inner, d_head, bc_dim;  // bc_dim = 2*ngroups*d_state
  int heads_cap;                                    // n_heads_active
  const int32_t* heads_per_seq;                     // device, nullable
};

hipError_t launch_conv1d_silu(const ConvArgs& a, int dtype, hipStream_t s);

struct StepArgs {
  float* state;
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
  void* y;
  int64_t ys;
  int64_t batch;
  int n_heads, d_head, d_state;
  int heads_cap;
  const int32_t* heads_per_seq;
};

hipError_t launch_ssd_step(const StepArgs& a, int dtype, hipStream_t s);

// One decode token with the conv folded in (ssd_step.hip): raw [x | B | C]
// row in, conv state read from cs_in and the advanced one written to cs_out.
struct StepFusedArgs {
  float* state;
  const float* cs_in;
  float* cs_out;
  const void* xbc;
  int64_t xbcs;
  const float* w;
  const float* bias;
  const void* dt;
  int64_t dts;
  const float* A;
  const float* D;
  void* y;
  int64_t ys;
  int64_t batch;
  int n_heads, d_head, d_state;
  int heads_cap;
  const int32_t* heads_per_seq;
};

hipError_t launch_ssd_step_fused(const StepFusedArgs& a, int dtype, hipStream_t s);

// ntok tokens per sequence in one pass over the states (ssd_step.hip).
struct StepMultiArgs {
  const float* state_in;
  float* state_out;  // may equal state_in, or NULL for outputs only
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
  void* y;
  int64_t ys;
  int64_t batch;
  int n_heads, d_head, d_state;
  int heads_cap;
  const int32_t* heads_per_seq;   // device, nullable
  int ntok;
  const int32_t* tokens_per_seq;  // device, nullable
};
hipError_t launch_ssd_step_multi(const StepMultiArgs& a, int dtype, hipStream_t s);

// Conv state advanced by each sequence's first tokens (ssd_step.hip).
struct ConvAdvanceArgs {
  float* conv_state;
  const void* xbc;
  int64_t xbcs;
  int64_t batch;
  int ntok;
  const int32_t* tokens_per_seq;  // device, nullable
  int64_t conv_dim;
  int xw, d_inner, bc_dim;
};
hipError_t launch_conv_state_advance(const ConvAdvanceArgs& a, int dtype, hipStream_t s);

// Per-sequence slices of a scan call (input-adaptive widths: each sequence
// runs its own slice): the active (sequence, head) units, numbered sequence-major, with
// start[b] the first unit of sequence b (start[batch] = units).  Passed by
// value to the kernels, so a mixed call needs no device-side table.
constexpr int kMaxMixedBatch = 256;
struct UnitMap {
  int mixed = 0;  // 0: every sequence runs the call's `heads`
  int batch = 0;
  int units = 0;
  int start[kMaxMixedBatch + 1] = {};
};

// Sequence and head of unit u (mixed maps; start[] is nondecreasing).
__host__ __device__ inline void unit_to_bh(const UnitMap& m, int u, int* b, int* h) {
  int lo = 0, hi = m.batch;  // start[lo] <= u < start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (m.start[mid] <= u) lo = mid;
    else hi = mid;
  }
  *b = lo;
  *h = u - m.start[lo];
}

struct FwdArgs {
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
  void* y;
  int64_t ys;
  const float* h0;
  float* hT;
  int64_t batch, seqlen;
  int n_heads, d_head, d_state, heads;  // heads: active heads (the widest sequence's, if mixed)
  int chunk;
  const int32_t* heads_per_seq = nullptr;  // host array (batch entries) for a mixed call
  // heads the segment plan is chosen for (>= heads; 0: heads).  Calls planned
  // for the same count cut the sequences alike, whatever their active heads.
  int plan_heads = 0;
};

// The unit map of a call (mixed when a.heads_per_seq is set).
UnitMap make_unit_map(const FwdArgs& a);

// How a scan call is cut: chunks per sequence, segments per sequence and
// chunks per segment (every segment but the last holds seg_chunks chunks).
// `units` overrides batch * heads as the count of active (sequence, head)
// units (a mixed call); 0 keeps it.
void fwd_plan(int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk, int* nchunks,
              int* nseg, int* seg_chunks, int64_t units = 0);
// Device workspace a scan call needs, 0 if none: segment states and decays
// of the plan and, on the bf16 d_head-64 d_state-128 path, the per-tile G and
// B^T fragments.
size_t fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads,
                           int64_t d_head, int64_t d_state, int64_t chunk, int dtype,
                           int64_t units = 0);

// Segments per sequence of a scan call (the plan of the path it takes).
int fwd_segments(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                 int64_t d_state, int64_t chunk, int dtype, int64_t units = 0);

// Conv and dt parameters of a fused scan call (raw conv input in, the conv
// and the dt transform applied on the way into the scan).
struct FuseArgs {
  const float* w = nullptr;        // (conv_dim, 4) conv weights, tap 3 = current token
  const float* bias = nullptr;     // (conv_dim) or NULL
  float* state = nullptr;          // (batch, 3, conv_dim) conv history or NULL (zeros)
  const float* dt_bias = nullptr;  // (n_heads) or NULL
  int64_t conv_dim = 0;
  int d_inner = 0;
  int softplus = 0;                // dt = softplus(dt + dt_bias) if set, else dt + dt_bias
};

// bf16, d_head 64, d_state 128, chunk 128 or 256 (ssd_fwd_bf16.hip).
bool bf16_path(int64_t d_head, int64_t d_state, int64_t chunk, int dtype);
// allow_pairs: the call may run its state-only pass two heads per workgroup
// (calls without the fused conv and without per-sequence widths).
size_t bf16_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t units = 0,
                            bool allow_pairs = false);
// The bf16 path's cut (128-token tiles): the segment count that minimises an
// estimate of the call's time in tile-walk units, counting workgroup rounds
// of one workgroup per CU, the per-walk start-up and the prepass and combine
// that a split adds.
void fwd_plan_bf16(int64_t batch, int64_t seqlen, int64_t heads, int* ntiles, int* nseg,
                   int* seg_tiles, int64_t units = 0, bool allow_pairs = false);
// The full plan: main segments of seg_tiles tiles; for a split call, each
// segment but the last is cut into ppseg pieces of piece_tiles tiles (the
// last piece may be shorter, none empty) for the state-only pass, which
// takes two heads per workgroup when pairs is set.
struct Bf16Plan {
  int ntiles = 0, nseg = 1, seg_tiles = 1, ppseg = 1, piece_tiles = 1;
  bool pairs = false;
  int nslot() const { return nseg > 1 ? (nseg - 1) * ppseg + 1 : 1; }
};
Bf16Plan plan_bf16(int64_t batch, int64_t seqlen, int64_t heads, int64_t units = 0,
                   bool allow_pairs = false);
hipError_t launch_ssd_forward_bf16(const FwdArgs& a, void* workspace, hipStream_t s);
// The same with the conv and dt transform fused in: a.x, a.B, a.C are the raw
// conv input's x, B and C columns and a.dt the raw dt.  The conv state, if
// any, is read, not updated (the caller rolls it afterwards).
hipError_t launch_ssd_forward_bf16_fused(const FwdArgs& a, const FuseArgs& fu, void* workspace,
                                         hipStream_t s);

hipError_t launch_ssd_forward(const FwdArgs& a, int dtype, void* workspace, hipStream_t s);

// Gated RMSNorm epilogue (gated_rmsnorm.hip): rows of y and z, d channels.
struct NormArgs {
  const void* y;
  int64_t ys;
  const void* z;
  int64_t zs;
  const float* w;
  float eps;
  void* out;
  int64_t os;
  int64_t rows, d;
};
hipError_t launch_gated_rmsnorm(const NormArgs& a, int dtype, hipStream_t s);

// A fused prefill call (fused.hip): raw [x | B | C] conv input rows in, the
// conv + SiLU and the dt transform applied on the way into the scan.
struct FusedCall {
  const void* xbc;
  int64_t xbcs;
  const float* conv_w;
  const float* conv_bias;
  float* conv_state;
  const void* dt;
  int64_t dts;
  const float* dt_bias;
  int softplus;
  const float* A;
  const float* D;
  void* y;
  int64_t ys;
  const float* h0;
  float* hT;
  int64_t batch, seqlen;
  int n_heads, d_head, d_state, heads, chunk, dtype;
};
size_t fused_workspace_bytes(int64_t batch, int64_t seqlen, int64_t n_heads, int64_t heads,
                             int64_t d_head, int64_t d_state, int64_t chunk, int dtype);
hipError_t launch_ssd_forward_fused(const FusedCall& f, void* workspace, hipStream_t s);

// Scan backward (ssd_bwd.hip): gradients of L = sum dy.y + sum dhT.h_final.
struct BwdArgs {
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
  int64_t batch, seqlen;
  int n_heads, d_head, d_state, heads, dtype, accumulate;
};
bool bwd_shape_supported(int64_t d_head, int64_t d_state, int dtype);
// Workspace: the state before every 64-token chunk and the final state, per
// active (sequence, head), in the storage type.
size_t bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                           int64_t d_state, int dtype);
hipError_t launch_ssd_backward(const BwdArgs& a, void* workspace, hipStream_t s);
// Chunks per sequence, segments per sequence and chunks per segment of a
// backward call (the split the launch, the workspace and the query share).
void bwd_plan(int64_t batch, int64_t seqlen, int64_t heads, int* nchunks, int* nseg,
              int* seg_chunks);

// Conv backward (conv1d_silu_bwd.hip): gradients of sum dout * conv1d_silu(in).
struct ConvBwdArgs {
  const void* in;
  int64_t in_stride;
  const void* dout;
  int64_t dout_stride;
  void* din;
  int64_t din_stride;
  const float* w;
  const float* bias;
  const float* conv_state;  // (batch, 3, conv_dim) history, or NULL (zeros)
  float* dw;
  float* dbias;
  float* dstate;            // (batch, 3, conv_dim) or NULL
  int64_t batch, seqlen, d_inner;
  int xw, bc_dim, accumulate;  // xw: active x channels
};
hipError_t launch_conv1d_silu_backward(const ConvBwdArgs& a, int dtype, hipStream_t s);

}  // namespace mmssd
