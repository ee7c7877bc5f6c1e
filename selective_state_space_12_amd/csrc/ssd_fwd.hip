// Chunked selective scan (SSD) forward over the first `heads` heads.
//
// "MatMamba: A Matryoshka State Space Model", block paragraph: the Mamba2
// block runs a chunk + selective scan with learnable per-head A and D;
// nesting paragraph: a sub-block uses A[0:h_i] and the first d_i = h_i*d_head
// channels of x.  The recurrence (H_t = exp(dt_t A) H_{t-1} + dt_t x_t B_t^T,
// y_t = H_t C_t + D x_t) is evaluated chunk by chunk.  For a chunk of Q
// tokens with Lambda_t = sum_{r<=t} dt_r A (inclusive, chunk-local):
//   Y_diag[t] = sum_{s<=t} exp(Lambda_t - Lambda_s) (C_t . B_s) dt_s x_s
//   Y_off[t]  = exp(Lambda_t) H_prev . C_t
//   y_t       = Y_diag[t] + Y_off[t] + D x_t
//   H_next    = exp(Lambda_end) H_prev + sum_s exp(Lambda_end - Lambda_s) dt_s x_s B_s^T
// which is the recurrence unrolled inside the chunk.
//
// MI355X design (gfx950, 64-wide waves, 16x16x32 bf16 / 16x16x4 fp32 MFMA):
//  - one workgroup of 8 waves walks the chunks of one (sequence, head,
//    segment) in order, so the fp32 state H (d_head x d_state) stays in MFMA
//    accumulator registers from chunk to chunk and never round-trips HBM;
//  - per chunk, B (Q x N, natural layout), x (transposed to d_head x Q) and
//    the decay cumsums live in LDS; C is read straight into MFMA operand
//    registers (the same fragment serves C.B^T and C.H^T);
//  - C.B^T is produced transposed so that its accumulator layout is directly
//    the A operand of the next product (masked decay applied in registers,
//    rounded to the operand type) -- no LDS round trip for the Q x Q block;
//  - 16-row output blocks are dealt to waves in a snake order so each wave
//    gets the same number of causal tiles;
//  - x and y rows of a head are 128 contiguous bytes of a token row: loads are
//    16-byte vectors, strided rows read only the active head range;
//  - long sequences with few (sequence, head) units are split into segments:
//    a prepass computes each segment's local end state, a tiny combine kernel
//    chains them, and the main pass starts every segment from its true state.
#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
// Aim for at least this many workgroups (two per CU of the 256-CU part).
#ifndef MMSSD_TARGET_UNITS
#define MMSSD_TARGET_UNITS 512
#endif

struct FwdK {
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
  float* seg_state;  // (batch, heads, nseg, P, N) fp32, or null
  float* seg_decay;  // (batch, heads, nseg) log2 decay of each segment
  int64_t seqlen;
  int n_heads, heads, Q, QA, nseg, seg_chunks, nchunks;
};

template <typename T> constexpr int pad16() { return 16 / (int)sizeof(T); }

template <typename T, int P, int N>
struct Layout {
  static constexpr int BP = N + pad16<T>();  // row pitch of B tile (elements)
  static constexpr int HP = N + pad16<T>();  // row pitch of the operand copy of H
  __host__ __device__ static int XP(int QA) { return QA + pad16<T>(); }
  __host__ __device__ static size_t bytes(int QA) {
    return (size_t)QA * BP * sizeof(T) + (size_t)P * XP(QA) * sizeof(T) +
           (size_t)P * HP * sizeof(T) + 3 * (size_t)QA * sizeof(float);
  }
};

template <typename T, int P, int N, bool OUT>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(FwdK k) {
  using L = Layout<T, P, N>;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= kWaves ? NTILE / kWaves : 1;  // state tiles per wave
  static_assert(NTILE < kWaves || NTILE % kWaves == 0, "state tiles must split evenly");
  static_assert(TP % TPW == 0, "a wave's state tiles share one column block");
  constexpr int NKB = (N + 31) / 32;  // K=32 slices over d_state
  constexpr int VB = 16 / (int)sizeof(T);

  extern __shared__ __align__(16) unsigned char smem[];
  const int Q = k.Q, QA = k.QA, XP = L::XP(QA);
  T* Bs = reinterpret_cast<T*>(smem);
  T* XT = Bs + (size_t)QA * L::BP;
  T* Hs = XT + (size_t)P * XP;
  float* lam = reinterpret_cast<float*>(Hs + (size_t)P * L::HP);
  float* dtv = lam + QA;
  float* wsc = dtv + QA;

  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int r16 = lane % 16, g = lane / 16;

  const T* __restrict__ Xp = static_cast<const T*>(k.x);
  const T* __restrict__ DTp = static_cast<const T*>(k.dt);
  const T* __restrict__ Bp = static_cast<const T*>(k.B);
  const T* __restrict__ Cp = static_cast<const T*>(k.C);
  T* __restrict__ Yp = static_cast<T*>(k.y);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah2 = k.A[h] * kLog2e;
  const float Dh = k.D ? k.D[h] : 0.0f;

  // ---- state tiles owned by this wave: H[pt*16 + g*4 + i][nt*16 + r16] ----
  const int tile0 = wave * TPW;
  const bool owns = tile0 < NTILE;
  const int nt = tile0 / TP, pt0 = tile0 % TP;
  f32x4 hacc[TPW];
  {
    const float* hin = nullptr;
    if (OUT) {
      if (k.nseg > 1)
        hin = k.seg_state + (((int64_t)b * k.heads + h) * k.nseg + seg) * (P * N);
      else if (k.h0)
        hin = k.h0 + ((int64_t)b * k.n_heads + h) * (P * N);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hacc[t][i] = (hin && owns) ? hin[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] : 0.0f;
  }

  const int c_begin = seg * k.seg_chunks;
  const int c_end = min(c_begin + k.seg_chunks, k.nchunks);
  float lam_seg = 0.0f;

  for (int c = c_begin; c < c_end; ++c) {
    const int64_t t_base = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - t_base);
    const int64_t row0 = rowb + t_base;

    // ---- phase L: dt + decay cumsum (wave 0), B and x tiles, operand copy of H
    if (wave == 0) {
      constexpr int kMaxE = 4;  // QA <= 256
      const int E = (QA + 63) / 64;
      float d[kMaxE], pre[kMaxE];
      float run = 0.0f;
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        const int s = lane * E + e;
        d[e] = (e < E && s < len) ? to_f32(DTp[(row0 + s) * k.dts + h]) : 0.0f;
        run += d[e] * Ah2;
        pre[e] = run;
      }
      float incl = run;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      const float excl = incl - run;
      const float lend = __shfl(incl, 63);
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        const int s = lane * E + e;
        if (e < E && s < QA) {
          const float lv = excl + pre[e];
          lam[s] = lv;
          dtv[s] = d[e];
          wsc[s] = exp2f(lend - lv) * d[e];
        }
      }
    }
    for (int idx = tid; idx < QA * (N / VB); idx += kThreads) {
      const int s = idx / (N / VB), col = (idx % (N / VB)) * VB;
      const Vec16<T> v = s < len ? load16(Bp + (row0 + s) * k.bs + col) : zero16<T>();
      store16(Bs + s * L::BP + col, v);
    }
    for (int idx = tid; idx < QA * (P / VB); idx += kThreads) {
      const int s = idx / (P / VB), p0 = (idx % (P / VB)) * VB;
      const Vec16<T> v = s < len ? load16(Xp + (row0 + s) * k.xs + (int64_t)h * P + p0) : zero16<T>();
#pragma unroll
      for (int j = 0; j < VB; ++j) XT[(p0 + j) * XP + s] = v.v[j];
    }
    if (OUT && owns) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Hs[((pt0 + t) * 16 + g * 4 + i) * L::HP + nt * 16 + r16] = from_f32<T>(hacc[t][i]);
    }
    __syncthreads();

    // ---- phase R: outputs of this chunk, 16-row blocks in snake order ----
    if (OUT) {
      const int RB = Q / 16;
      for (int it = 0; it * kWaves < RB; ++it) {
        const int base = it * kWaves;
        const int r = (it & 1) ? base + kWaves - 1 - wave : base + wave;
        const int t0 = r * 16;
        if (r >= RB || t0 >= len) continue;
        const int trow = t0 + r16;  // this lane's row of C and of the masked product

        Frag8<T> cf[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int n = kb * 32 + g * 8;
          if (trow < len && n < N) frag_load8(cf[kb], Cp + (row0 + trow) * k.cs + n);
          else frag_zero(cf[kb]);
        }

        // Y_off = exp(Lambda_t) * C_t . H_prev
        f32x4 acc[TP];
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          acc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const int n = kb * 32 + g * 8;
            Frag8<T> hf;
            if (n < N) frag_load8(hf, Hs + (pt * 16 + r16) * L::HP + n);
            else frag_zero(hf);
            acc[pt] = mma(cf[kb], hf, acc[pt]);
          }
        }
        {
          float sc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[i] = exp2f(lam[t0 + g * 4 + i]);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[pt][i] *= sc[i];
        }

        // Y_diag: (G o L) (x) over the causal 32-wide column blocks
        const float lam_t = lam[trow];
        const int nsb = (t0 + 15) / 32 + 1;
        for (int sb = 0; sb < nsb; ++sb) {
          const int s0 = sb * 32;
          f32x4 g0 = {0.0f, 0.0f, 0.0f, 0.0f}, g1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const int n = kb * 32 + g * 8;
            Frag8<T> b0, b1;
            if (n < N) {
              frag_load8(b0, Bs + (s0 + r16) * L::BP + n);
              frag_load8(b1, Bs + (s0 + 16 + r16) * L::BP + n);
            } else {
              frag_zero(b0);
              frag_zero(b1);
            }
            g0 = mma(b0, cf[kb], g0);  // G^T[s0 + g*4 + i][trow]
            g1 = mma(b1, cf[kb], g1);  // G^T[s0 + 16 + g*4 + i][trow]
          }
          Frag8<T> mf;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int sj = s0 + (j < 4 ? g * 4 + j : 16 + g * 4 + (j - 4));
            const float gv = j < 4 ? g0[j] : g1[j - 4];
            float v = 0.0f;
            if (sj <= trow) v = gv * exp2f(lam_t - lam[sj]) * dtv[sj];
            frag_set(mf, j, v);
          }
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            const T* xr = XT + (pt * 16 + r16) * XP + s0 + g * 4;
            Frag8<T> xf;
            frag_load4x2(xf, xr, xr + 16);
            acc[pt] = mma(mf, xf, acc[pt]);
          }
        }

        // epilogue: + D x, round, store the head's slice of each token row
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const int p = pt * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = t0 + g * 4 + i;
            if (t < len) {
              const float xv = to_f32(XT[p * XP + t]);
              Yp[(row0 + t) * k.ys + (int64_t)h * P + p] = from_f32<T>(acc[pt][i] + Dh * xv);
            }
          }
        }
      }
    }

    // ---- phase U: H <- exp(Lambda_end) H + (w o x)^T B, w_s = exp(Lambda_end - Lambda_s) dt_s
    const float lend = lam[QA - 1];
    lam_seg += lend;
    if (owns) {
      const float dec = exp2f(lend);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) hacc[t][i] *= dec;
      const int nsbu = (len + 31) / 32;
      for (int sb = 0; sb < nsbu; ++sb) {
        const int s0 = sb * 32 + g * 8;
        Frag8<T> bfv;
#pragma unroll
        for (int j = 0; j < 8; ++j) bfv.v[j] = Bs[(s0 + j) * L::BP + nt * 16 + r16];
        float wj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wj[j] = wsc[s0 + j];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> xf, af;
          frag_load8(xf, XT + ((pt0 + t) * 16 + r16) * XP + s0);
#pragma unroll
          for (int j = 0; j < 8; ++j) frag_set(af, j, to_f32(xf.v[j]) * wj[j]);
          hacc[t] = mma(af, bfv, hacc[t]);
        }
      }
    }
    __syncthreads();
  }

  // ---- write the state leaving this segment ----
  float* hout = nullptr;
  if (OUT) {
    if (k.hT && seg == k.nseg - 1) hout = k.hT + ((int64_t)b * k.n_heads + h) * (P * N);
  } else {
    hout = k.seg_state + (((int64_t)b * k.heads + h) * k.nseg + seg) * (P * N);
    if (tid == 0) k.seg_decay[((int64_t)b * k.heads + h) * k.nseg + seg] = lam_seg;
  }
  if (hout && owns) {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) hout[((pt0 + t) * 16 + g * 4 + i) * N + nt * 16 + r16] = hacc[t][i];
  }
}

// Chains segment states: slot s receives the state entering segment s,
//   H_in[0] = h0, H_in[s+1] = exp2(decay_s) H_in[s] + S_s,
// where slot s held the local end state S_s written by the prepass.
__global__ __launch_bounds__(256) void seg_combine_kernel(float* __restrict__ seg_state,
                                                          const float* __restrict__ seg_decay,
                                                          const float* __restrict__ h0,
                                                          int n_heads, int heads, int nseg, int PN) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t unit = (int64_t)b * heads + h;
  for (int e = threadIdx.x; e < PN; e += 256) {
    float H = h0 ? h0[((int64_t)b * n_heads + h) * PN + e] : 0.0f;
    for (int s = 0; s < nseg; ++s) {
      float* slot = seg_state + (unit * nseg + s) * PN + e;
      const float S = s < nseg - 1 ? *slot : 0.0f;
      *slot = H;
      if (s < nseg - 1) H = exp2f(seg_decay[unit * nseg + s]) * H + S;
    }
  }
}

template <typename T, int P, int N>
hipError_t launch_shape(const FwdArgs& a, void* ws, hipStream_t s) {
  using L = Layout<T, P, N>;
  FwdK k;
  k.x = a.x; k.xs = a.xs; k.dt = a.dt; k.dts = a.dts; k.A = a.A;
  k.B = a.B; k.bs = a.bs; k.C = a.C; k.cs = a.cs; k.D = a.D;
  k.y = a.y; k.ys = a.ys; k.h0 = a.h0; k.hT = a.hT;
  k.seqlen = a.seqlen; k.n_heads = a.n_heads; k.heads = a.heads;
  k.Q = a.chunk; k.QA = a.chunk < 32 ? 32 : a.chunk;
  fwd_plan(a.batch, a.seqlen, a.heads, a.chunk, &k.nchunks, &k.nseg, &k.seg_chunks);
  k.seg_state = nullptr;
  k.seg_decay = nullptr;
  if (k.nseg > 1) {
    k.seg_state = static_cast<float*>(ws);
    k.seg_decay = k.seg_state + (size_t)a.batch * a.heads * k.nseg * P * N;
  }
  const size_t lds = L::bytes(k.QA);
  hipError_t e;
  if (k.nseg > 1) {
    auto pre = ssd_chunk_kernel<T, P, N, false>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(pre),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pre, dim3(k.nseg - 1, a.heads, (unsigned)a.batch), dim3(kThreads), lds, s, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3(a.heads, (unsigned)a.batch), dim3(256), 0, s,
                       k.seg_state, k.seg_decay, a.h0, a.n_heads, a.heads, k.nseg, P * N);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto main_k = ssd_chunk_kernel<T, P, N, true>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(main_k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(main_k, dim3(k.nseg, a.heads, (unsigned)a.batch), dim3(kThreads), lds, s, k);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const FwdArgs& a, void* ws, hipStream_t s) {
  if (a.d_head == 32 && a.d_state == 16) return launch_shape<T, 32, 16>(a, ws, s);
  if (a.d_head == 64 && a.d_state == 64) return launch_shape<T, 64, 64>(a, ws, s);
  if (a.d_head == 64 && a.d_state == 128) return launch_shape<T, 64, 128>(a, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace

void fwd_plan(int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk, int* nchunks,
              int* nseg, int* seg_chunks) {
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  const int64_t units = batch * heads;
  int64_t want = (MMSSD_TARGET_UNITS + units - 1) / units;
  if (want > nc) want = nc;
  if (want < 1) want = 1;
  const int64_t per = (nc + want - 1) / want;  // whole chunks per segment
  *nchunks = (int)nc;
  *seg_chunks = (int)per;
  *nseg = (int)((nc + per - 1) / per);
}

size_t fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                           int64_t d_state, int64_t chunk) {
  int nc, nseg, per;
  fwd_plan(batch, seqlen, heads, chunk, &nc, &nseg, &per);
  if (nseg <= 1) return 0;
  return (size_t)(batch * heads * nseg) * (size_t)(d_head * d_state + 1) * sizeof(float);
}

hipError_t launch_ssd_forward(const FwdArgs& a, int dtype, void* ws, hipStream_t s) {
  if (dtype == MM_BF16) return launch_typed<bf16>(a, ws, s);
  return launch_typed<float>(a, ws, s);
}

}  // namespace mmssd
