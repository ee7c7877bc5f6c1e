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
constexpr int kXcds = 8;  // accelerator complex dies of the MI355X, each with its own L2
// Aim for at least this many workgroups (one per CU of the 256-CU part: the
// chunk tiles take most of a CU's LDS).
#ifndef MMSSD_TARGET_UNITS
#define MMSSD_TARGET_UNITS 256
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
  int n_heads, heads, nseg, seg_chunks, nchunks;
  UnitMap um;  // mixed: heads of sequence b = um.start[b+1] - um.start[b]
};

template <typename T> constexpr int pad16() { return 16 / (int)sizeof(T); }

template <typename T, int P, int N, int Q>
struct Layout {
  static constexpr int QA = Q < 32 ? 32 : Q;  // rows allocated (whole 32-wide column blocks)
  static constexpr int BP = N + pad16<T>();   // row pitch of the B tile (elements)
  static constexpr int HP = N + pad16<T>();   // row pitch of the operand copy of H
  static constexpr int XP = QA + pad16<T>();  // row pitch of the transposed x tile
  static constexpr size_t bytes = (size_t)QA * BP * sizeof(T) + (size_t)P * XP * sizeof(T) +
                                  (size_t)P * HP * sizeof(T) + 4 * (size_t)QA * sizeof(float);
};

template <typename T, int P, int N, int Q, bool OUT>
__global__ __launch_bounds__(kThreads) void ssd_chunk_kernel(FwdK k) {
  using L = Layout<T, P, N, Q>;
  constexpr int TP = P / 16, TN = N / 16, NTILE = TP * TN;
  constexpr int TPW = NTILE >= kWaves ? NTILE / kWaves : 1;  // state tiles per wave
  static_assert(NTILE < kWaves || NTILE % kWaves == 0, "state tiles must split evenly");
  static_assert(TP % TPW == 0, "a wave's state tiles share one column block");
  constexpr int NKB = (N + 31) / 32;  // K=32 slices over d_state
  constexpr int VB = 16 / (int)sizeof(T);
  constexpr int QA = L::QA, XP = L::XP;
  constexpr int NBV = (QA * (N / VB) + kThreads - 1) / kThreads;  // B vectors per thread
  constexpr int NXV = (QA * (P / VB) + kThreads - 1) / kThreads;  // x vectors per thread
  constexpr int kRBW = 2;                                          // row blocks per wave (Q <= 256)
  constexpr int E = (QA + 63) / 64;                                // dt values per lane of wave 0
  constexpr int RB = Q / 16;

  extern __shared__ __align__(16) unsigned char smem[];
  T* Bs = reinterpret_cast<T*>(smem);
  T* XT = Bs + (size_t)QA * L::BP;
  T* Hs = XT + (size_t)P * XP;
  float* lam = reinterpret_cast<float*>(Hs + (size_t)P * L::HP);
  float* dtv = lam + QA;
  float* wsc = dtv + QA;
  float* efac = wsc + QA;

  // XCD-aware unit mapping: workgroups are dealt round-robin to the 8 XCDs in
  // dispatch order, so give each XCD a contiguous block of (sequence, head,
  // segment) units -- heads that share a sequence's B and C tiles then share
  // one XCD's L2.
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int pid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int uid = total % kXcds == 0 ? (pid % kXcds) * (total / kXcds) + pid / kXcds : pid;
  const int seg = uid % gx, h = (uid / gx) % gy, b = uid / (gx * gy);
  if (k.um.mixed && h >= k.um.start[b + 1] - k.um.start[b]) return;  // whole workgroup
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

  // 16-row output blocks of this wave, dealt in snake order for balance
  int rb[kRBW];
#pragma unroll
  for (int i = 0; i < kRBW; ++i) rb[i] = (i & 1) ? i * kWaves + kWaves - 1 - wave : i * kWaves + wave;

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

  // ---- registers holding the next chunk's inputs (loaded during compute) ----
  Vec16<T> pb[NBV], px[NXV];
  float pdt[E];
  Frag8<T> cfa[NKB], cfb[NKB];  // C of this wave's two row blocks, loaded a chunk ahead

  // Loads are unconditional (rows past the end of the sequence are clamped to
  // its last row); the commit below zeroes them, so no lane branches here.
  // A chunk's loads are issued in kParts portions spread over the previous
  // chunk's compute: every CU runs the same program, so issuing them in one
  // burst saturates HBM for microseconds and then leaves it idle.
  constexpr int kParts = 3;
  auto prefetch = [&](int c, int part) {
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int last = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q) - 1;
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      if (v % kParts != part) continue;
      const int idx = tid + v * kThreads;
      const int s = min(idx / (N / VB), last), col = (idx % (N / VB)) * VB;
      pb[v] = load16(Bp + (row0 + s) * k.bs + col);
    }
    // x: consecutive lanes take consecutive tokens (same 16-byte column
    // group), so the transposed LDS writes of a wave hit distinct banks
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      if (v % kParts != part) continue;
      const int idx = tid + v * kThreads;
      const int s = min(idx % QA, last), p0 = ((idx / QA) % (P / VB)) * VB;
      px[v] = load16(Xp + (row0 + s) * k.xs + (int64_t)h * P + p0);
    }
    if (wave == 0 && part == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int s = min(lane * E + e, last);
        pdt[e] = to_f32(DTp[(row0 + s) * k.dts + h]);
      }
    }
  };

  // C fragments of one 16-row block: lane holds C[t0 + r16][kb*32 + g*8 + j]
  auto load_c = [&](int c, int r, Frag8<T> (&cf)[NKB]) {
    const int64_t row0 = rowb + (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - (int64_t)c * Q);
    const int trow = r * 16 + r16;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int n = kb * 32 + g * 8;
      if (r < RB && trow < len && n < N) frag_load8(cf[kb], Cp + (row0 + trow) * k.cs + n);
      else frag_zero(cf[kb]);
    }
  };

  const int c_begin = seg * k.seg_chunks;
  const int c_end = min(c_begin + k.seg_chunks, k.nchunks);
  float lam_seg = 0.0f;
  if (c_begin < c_end) {
#pragma unroll
    for (int part = 0; part < kParts; ++part) prefetch(c_begin, part);
    if (OUT) {
      load_c(c_begin, rb[0], cfa);
      load_c(c_begin, rb[1], cfb);
    }
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int64_t t_base = (int64_t)c * Q;
    const int len = (int)min((int64_t)Q, k.seqlen - t_base);
    const int64_t row0 = rowb + t_base;

    // ---- phase L: prefetched tiles -> LDS (rows >= len zeroed), decay cumsum,
    // operand copy of H
#pragma unroll
    for (int v = 0; v < NBV; ++v) {
      const int idx = tid + v * kThreads;
      if (idx < QA * (N / VB)) {
        const int s = idx / (N / VB), col = (idx % (N / VB)) * VB;
        store16(Bs + s * L::BP + col, s < len ? pb[v] : zero16<T>());
      }
    }
#pragma unroll
    for (int v = 0; v < NXV; ++v) {
      const int idx = tid + v * kThreads;
      if (idx < QA * (P / VB)) {
        const int s = idx % QA, p0 = (idx / QA) * VB;
        const Vec16<T> xv = s < len ? px[v] : zero16<T>();
#pragma unroll
        for (int j = 0; j < VB; ++j) XT[(p0 + j) * XP + s] = xv.v[j];
      }
    }
    if (wave == 0) {
      float pre[E];
      float run = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lane * E + e >= len) pdt[e] = 0.0f;
        run += pdt[e] * Ah2;
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
      for (int e = 0; e < E; ++e) {
        const int s = lane * E + e;
        if (s < QA) {
          const float lv = excl + pre[e];
          lam[s] = lv;
          dtv[s] = pdt[e];
          wsc[s] = __builtin_amdgcn_exp2f(lend - lv) * pdt[e];
        }
      }
      // efac_s = exp2(lam_e - lam_s) dt_s with e the last token of s's
      // 32-wide column block (token s | 31, held by lane (s|31)/E, slot E-1)
      static_assert(32 % E == 0, "a column block spans whole lanes");
      const float lane_last = excl + pre[E - 1];
      const float lam_blk_end = __shfl(lane_last, lane | (32 / E - 1));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int s = lane * E + e;
        if (s < QA) efac[s] = __builtin_amdgcn_exp2f(lam_blk_end - (excl + pre[e])) * pdt[e];
      }
    }
    if (OUT && owns) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Hs[((pt0 + t) * 16 + g * 4 + i) * L::HP + nt * 16 + r16] = from_f32<T>(hacc[t][i]);
    }
    __syncthreads();

    // next chunk's loads are in flight while this chunk computes
    const bool more = c + 1 < c_end;
    if (more) prefetch(c + 1, 0);  // parts 1 and 2 follow the state update and Y_off

    // ---- phase U: H <- exp(Lambda_end) H + (w o x)^T B, w_s = exp(Lambda_end - Lambda_s) dt_s
    // (registers only; the outputs below use the operand copy of H_prev in LDS)
    const float lend = lam[QA - 1];
    lam_seg += lend;
    if (owns) {
      const float dec = __builtin_amdgcn_exp2f(lend);
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) hacc[t][q] *= dec;
      const int nsbu = (len + 31) / 32;
#pragma unroll 1
      for (int sb = 0; sb < nsbu; ++sb) {
        const int s0 = sb * 32 + g * 8;
        // B operand (k = s, n): the decay weight w_s is folded in here, once
        // per column block, so the x operand is a plain tile read
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wsc + s0);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wsc + s0 + 4);
        Frag8<T> bfv;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          frag_set(bfv, j, to_f32(Bs[(s0 + j) * L::BP + nt * 16 + r16]) * (j < 4 ? w0[j] : w1[j - 4]));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          Frag8<T> xf;
          frag_load8(xf, XT + ((pt0 + t) * 16 + r16) * XP + s0);
          hacc[t] = mma(xf, bfv, hacc[t]);
        }
      }
    }
    if (more) {
      prefetch(c + 1, 1);
      if (!OUT) prefetch(c + 1, 2);
    }
    // ---- phase R: outputs of this chunk ----
    // Lane holds G^T[s0 + g*4 + q][t] (gA) and G^T[s0 + 16 + g*4 + q][t] (gB)
    // for its row t; the masked decay turns them into the A operand of M . x.
    // Column blocks left of the diagonal use the factored decay
    //   exp2(lam_t - lam_s) dt_s = exp2(lam_t - lam_e) * efac_s,
    //   efac_s = exp2(lam_e - lam_s) dt_s,  e = last token of the block,
    // both factors <= 1 when A < 0; the diagonal block uses the direct form.
    auto build_m = [&](const f32x4& gA, const f32x4& gB, int s0, int trow, float lam_t,
                       bool diag) {
      Frag8<T> mf;
      if (!diag) {
        const float et = __builtin_amdgcn_exp2f(lam_t - lam[s0 + 31]);
        const f32x4 ea = *reinterpret_cast<const f32x4*>(efac + s0 + g * 4);
        const f32x4 eb = *reinterpret_cast<const f32x4*>(efac + s0 + 16 + g * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          frag_set(mf, j, gA[j] * ea[j] * et);
          frag_set(mf, j + 4, gB[j] * eb[j] * et);
        }
      } else {
        const f32x4 la = *reinterpret_cast<const f32x4*>(lam + s0 + g * 4);
        const f32x4 lb = *reinterpret_cast<const f32x4*>(lam + s0 + 16 + g * 4);
        const f32x4 da = *reinterpret_cast<const f32x4*>(dtv + s0 + g * 4);
        const f32x4 db = *reinterpret_cast<const f32x4*>(dtv + s0 + 16 + g * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sa = s0 + g * 4 + j;
          frag_set(mf, j, sa <= trow ? gA[j] * __builtin_amdgcn_exp2f(lam_t - la[j]) * da[j] : 0.0f);
          frag_set(mf, j + 4,
                   sa + 16 <= trow ? gB[j] * __builtin_amdgcn_exp2f(lam_t - lb[j]) * db[j] : 0.0f);
        }
      }
      return mf;
    };
    // B operand rows s0 + r16 and s0 + 16 + r16 of K-slice kb (d_state)
    auto load_bpair = [&](int s0, int kb, Frag8<T>& b0, Frag8<T>& b1) {
      const int n = kb * 32 + g * 8;
      if (n < N) {
        frag_load8(b0, Bs + (s0 + r16) * L::BP + n);
        frag_load8(b1, Bs + (s0 + 16 + r16) * L::BP + n);
      } else {
        frag_zero(b0);
        frag_zero(b1);
      }
    };
    auto load_xpair = [&](int s0, int pt, Frag8<T>& xf) {
      const T* xr = XT + (pt * 16 + r16) * XP + s0 + g * 4;
      frag_load4x2(xf, xr, xr + 16);
    };
    // epilogue: + D x, round, store the head's slice of each token row
    auto store_rows = [&](const f32x4 (&acc)[TP], int t0, bool full) {
      T* ybase = Yp + (row0 + t0 + g * 4) * k.ys + (int64_t)h * P + r16;
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        // x[t0 + g*4 + q][p] for q = 0..3: four consecutive entries of XT's row p
        Frag8<T> xq;
        const T* xrow = XT + (pt * 16 + r16) * XP + t0 + g * 4;
        frag_load4x2(xq, xrow, xrow);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (full || t0 + g * 4 + q < len)
            ybase[q * k.ys + pt * 16] = from_f32<T>(acc[pt][q] + Dh * to_f32(xq.v[q]));
        }
      }
    };
    auto scale_rows = [&](f32x4 (&acc)[TP], int t0) {
      const f32x4 la = *reinterpret_cast<const f32x4*>(lam + t0 + g * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sq = __builtin_amdgcn_exp2f(la[q]);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) acc[pt][q] *= sq;
      }
    };

    if (OUT && len == Q && (RB == 16 || RB == 8)) {
      // Full chunk: every wave owns RB/8 row blocks, no bounds tests.
      constexpr bool kTwo = RB == 16;
      const int t00 = rb[0] * 16, t01 = rb[1] * 16;
      const int nsb0 = rb[0] / 2 + 1, nsb1 = rb[1] / 2 + 1;  // column blocks through the diagonal
      const float lt0 = lam[t00 + r16];
      const float lt1 = kTwo ? lam[t01 + r16] : 0.0f;
      f32x4 acc0[TP], acc1[TP];
      // Y_off = exp(Lambda_t) * C_t . H_prev
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        acc0[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        acc1[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int n = kb * 32 + g * 8;
          Frag8<T> hf;
          if (n < N) frag_load8(hf, Hs + (pt * 16 + r16) * L::HP + n);
          else frag_zero(hf);
          acc0[pt] = mma(cfa[kb], hf, acc0[pt]);
          if (kTwo) acc1[pt] = mma(cfb[kb], hf, acc1[pt]);
        }
      }
      scale_rows(acc0, t00);
      if (kTwo) scale_rows(acc1, t01);
      if (more) prefetch(c + 1, 2);
      // Y_diag over column blocks; both row blocks share each B and x fragment
      auto step = [&](int sb, bool both, bool diag0, bool diag1) {
        const int s0 = sb * 32;
        f32x4 g0A = {0, 0, 0, 0}, g0B = {0, 0, 0, 0}, g1A = {0, 0, 0, 0}, g1B = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          Frag8<T> b0, b1;
          load_bpair(s0, kb, b0, b1);
          if (both) {
            g0A = mma(b0, cfa[kb], g0A);
            g0B = mma(b1, cfa[kb], g0B);
          }
          g1A = mma(b0, cfb[kb], g1A);
          g1B = mma(b1, cfb[kb], g1B);
        }
        Frag8<T> m0, m1;
        if (both) m0 = build_m(g0A, g0B, s0, t00 + r16, lt0, diag0);
        m1 = build_m(g1A, g1B, s0, t01 + r16, lt1, diag1);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          Frag8<T> xf;
          load_xpair(s0, pt, xf);
          if (both) acc0[pt] = mma(m0, xf, acc0[pt]);
          acc1[pt] = mma(m1, xf, acc1[pt]);
        }
      };
      if (kTwo) {
        int sb = 0;
#pragma unroll 1
        for (; sb < nsb0 - 1; ++sb) step(sb, true, false, false);
        step(sb++, true, true, false);
#pragma unroll 1
        for (; sb < nsb1 - 1; ++sb) step(sb, false, false, false);
        step(sb, false, false, true);
        store_rows(acc0, t00, true);
        store_rows(acc1, t01, true);
      } else {
        // one row block per wave
        int sb = 0;
#pragma unroll 1
        for (; sb < nsb0 - 1; ++sb) {
          const int s0 = sb * 32;
          f32x4 gA = {0, 0, 0, 0}, gB = {0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            Frag8<T> b0, b1;
            load_bpair(s0, kb, b0, b1);
            gA = mma(b0, cfa[kb], gA);
            gB = mma(b1, cfa[kb], gB);
          }
          const Frag8<T> m = build_m(gA, gB, s0, t00 + r16, lt0, false);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            Frag8<T> xf;
            load_xpair(s0, pt, xf);
            acc0[pt] = mma(m, xf, acc0[pt]);
          }
        }
        {
          const int s0 = sb * 32;
          f32x4 gA = {0, 0, 0, 0}, gB = {0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            Frag8<T> b0, b1;
            load_bpair(s0, kb, b0, b1);
            gA = mma(b0, cfa[kb], gA);
            gB = mma(b1, cfa[kb], gB);
          }
          const Frag8<T> m = build_m(gA, gB, s0, t00 + r16, lt0, true);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            Frag8<T> xf;
            load_xpair(s0, pt, xf);
            acc0[pt] = mma(m, xf, acc0[pt]);
          }
        }
        store_rows(acc0, t00, true);
      }
      if (c + 1 < c_end) {  // in flight across the next commit and state update
        load_c(c + 1, rb[0], cfa);
        load_c(c + 1, rb[1], cfb);
      }
    } else if (OUT) {
      if (more) prefetch(c + 1, 2);
      // Generic path: ragged last chunk or fewer row blocks than waves.
      const int t00 = rb[0] * 16, t01 = rb[1] * 16;
      const bool v0 = rb[0] < RB && t00 < len;  // wave-uniform
      const bool v1 = rb[1] < RB && t01 < len;
      f32x4 acc0[TP], acc1[TP];

      // Y_off = exp(Lambda_t) * C_t . H_prev
#pragma unroll
      for (int pt = 0; pt < TP; ++pt) {
        acc0[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        acc1[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int n = kb * 32 + g * 8;
          Frag8<T> hf;
          if (n < N) frag_load8(hf, Hs + (pt * 16 + r16) * L::HP + n);
          else frag_zero(hf);
          if (v0) acc0[pt] = mma(cfa[kb], hf, acc0[pt]);
          if (v1) acc1[pt] = mma(cfb[kb], hf, acc1[pt]);
        }
      }
      {
        const f32x4 la0 = v0 ? *reinterpret_cast<const f32x4*>(lam + t00 + g * 4) : f32x4{0, 0, 0, 0};
        const f32x4 la1 = v1 ? *reinterpret_cast<const f32x4*>(lam + t01 + g * 4) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float s0q = __builtin_amdgcn_exp2f(la0[q]), s1q = __builtin_amdgcn_exp2f(la1[q]);
#pragma unroll
          for (int pt = 0; pt < TP; ++pt) {
            acc0[pt][q] *= s0q;
            acc1[pt][q] *= s1q;
          }
        }
      }

      // Y_diag over causal 32-wide column blocks
      const int nsb0 = v0 ? t00 / 32 + 1 : 0;  // column blocks up to the diagonal
      const int nsb1 = v1 ? t01 / 32 + 1 : 0;
      const int nsbm = nsb0 > nsb1 ? nsb0 : nsb1;
      const float lt0 = lam[t00 + r16 < QA ? t00 + r16 : QA - 1];
      const float lt1 = lam[t01 + r16 < QA ? t01 + r16 : QA - 1];
#pragma unroll 1
      for (int sb = 0; sb < nsbm; ++sb) {
        const int s0 = sb * 32;
        const bool a0 = sb < nsb0, a1 = sb < nsb1;  // wave-uniform
        f32x4 g0A = {0, 0, 0, 0}, g0B = {0, 0, 0, 0}, g1A = {0, 0, 0, 0}, g1B = {0, 0, 0, 0};
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
          if (a0) {
            g0A = mma(b0, cfa[kb], g0A);
            g0B = mma(b1, cfa[kb], g0B);
          }
          if (a1) {
            g1A = mma(b0, cfb[kb], g1A);
            g1B = mma(b1, cfb[kb], g1B);
          }
        }
        Frag8<T> m0, m1;
        if (a0) m0 = build_m(g0A, g0B, s0, t00 + r16, lt0, sb + 1 == nsb0);
        if (a1) m1 = build_m(g1A, g1B, s0, t01 + r16, lt1, sb + 1 == nsb1);
#pragma unroll
        for (int pt = 0; pt < TP; ++pt) {
          const T* xr = XT + (pt * 16 + r16) * XP + s0 + g * 4;
          Frag8<T> xf;
          frag_load4x2(xf, xr, xr + 16);
          if (a0) acc0[pt] = mma(m0, xf, acc0[pt]);
          if (a1) acc1[pt] = mma(m1, xf, acc1[pt]);
        }
      }

      if (v0) store_rows(acc0, t00, t00 + 16 <= len);
      if (v1) store_rows(acc1, t01, t01 + 16 <= len);
      if (c + 1 < c_end) {  // in flight across the next commit and state update
        load_c(c + 1, rb[0], cfa);
        load_c(c + 1, rb[1], cfb);
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
      for (int q = 0; q < 4; ++q) hout[((pt0 + t) * 16 + g * 4 + q) * N + nt * 16 + r16] = hacc[t][q];
  }
}

// Chains segment states: slot s receives the state entering segment s,
//   H_in[0] = h0, H_in[s+1] = exp2(decay_s) H_in[s] + S_s,
// where slot s held the local end state S_s written by the prepass.
__global__ __launch_bounds__(256) void seg_combine_kernel(float* __restrict__ seg_state,
                                                          const float* __restrict__ seg_decay,
                                                          const float* __restrict__ h0,
                                                          int n_heads, int heads, int nseg, int PN,
                                                          UnitMap um) {
  const int h = blockIdx.x, b = blockIdx.y;
  if (um.mixed && h >= um.start[b + 1] - um.start[b]) return;
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

template <typename T, int P, int N, int Q>
hipError_t launch_shape(const FwdArgs& a, void* ws, hipStream_t s) {
  using L = Layout<T, P, N, Q>;
  FwdK k;
  k.x = a.x; k.xs = a.xs; k.dt = a.dt; k.dts = a.dts; k.A = a.A;
  k.B = a.B; k.bs = a.bs; k.C = a.C; k.cs = a.cs; k.D = a.D;
  k.y = a.y; k.ys = a.ys; k.h0 = a.h0; k.hT = a.hT;
  k.seqlen = a.seqlen; k.n_heads = a.n_heads; k.heads = a.heads;
  k.um = make_unit_map(a);
  fwd_plan(a.batch, a.seqlen, a.plan_heads > 0 ? a.plan_heads : a.heads, Q, &k.nchunks, &k.nseg,
           &k.seg_chunks, k.um.mixed ? k.um.units : 0);
  k.seg_state = nullptr;
  k.seg_decay = nullptr;
  if (k.nseg > 1) {
    k.seg_state = static_cast<float*>(ws);
    k.seg_decay = k.seg_state + (size_t)a.batch * a.heads * k.nseg * P * N;
  }
  const size_t lds = L::bytes;
  hipError_t e;
  if (k.nseg > 1) {
    auto pre = ssd_chunk_kernel<T, P, N, Q, false>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(pre),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pre, dim3(k.nseg - 1, a.heads, (unsigned)a.batch), dim3(kThreads), lds, s, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3(a.heads, (unsigned)a.batch), dim3(256), 0, s,
                       k.seg_state, k.seg_decay, a.h0, a.n_heads, a.heads, k.nseg, P * N, k.um);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto main_k = ssd_chunk_kernel<T, P, N, Q, true>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(main_k),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(main_k, dim3(k.nseg, a.heads, (unsigned)a.batch), dim3(kThreads), lds, s, k);
  return hipGetLastError();
}

template <typename T, int P, int N>
hipError_t launch_chunk(const FwdArgs& a, void* ws, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_shape<T, P, N, 16>(a, ws, s);
    case 32: return launch_shape<T, P, N, 32>(a, ws, s);
    case 64: return launch_shape<T, P, N, 64>(a, ws, s);
    case 128: return launch_shape<T, P, N, 128>(a, ws, s);
    case 256:
      // fp32 tiles of 256 tokens with d_state 128 do not fit one CU's LDS
      if constexpr (sizeof(T) == 4 && N == 128) return hipErrorInvalidValue;
      else return launch_shape<T, P, N, 256>(a, ws, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_typed(const FwdArgs& a, void* ws, hipStream_t s) {
  if (a.d_head == 32 && a.d_state == 16) return launch_chunk<T, 32, 16>(a, ws, s);
  if (a.d_head == 64 && a.d_state == 64) return launch_chunk<T, 64, 64>(a, ws, s);
  if (a.d_head == 64 && a.d_state == 128) return launch_chunk<T, 64, 128>(a, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace

UnitMap make_unit_map(const FwdArgs& a) {
  UnitMap m;
  if (!a.heads_per_seq) return m;
  m.mixed = 1;
  m.batch = (int)a.batch;
  m.start[0] = 0;
  for (int b = 0; b < m.batch; ++b) m.start[b + 1] = m.start[b] + a.heads_per_seq[b];
  m.units = m.start[m.batch];
  return m;
}

void fwd_plan(int64_t batch, int64_t seqlen, int64_t heads, int64_t chunk, int* nchunks,
              int* nseg, int* seg_chunks, int64_t units_in) {
  const int64_t nc = (seqlen + chunk - 1) / chunk;
  const int64_t units = units_in > 0 ? units_in : batch * heads;
  int64_t want = (MMSSD_TARGET_UNITS + units - 1) / units;
  if (want > nc) want = nc;
  if (want < 1) want = 1;
  const int64_t per = (nc + want - 1) / want;  // whole chunks per segment
  *nchunks = (int)nc;
  *seg_chunks = (int)per;
  *nseg = (int)((nc + per - 1) / per);
}

int fwd_segments(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                 int64_t d_state, int64_t chunk, int dtype, int64_t units) {
  int nc, nseg, per;
  if (bf16_path(d_head, d_state, chunk, dtype))
    fwd_plan_bf16(batch, seqlen, heads, &nc, &nseg, &per, units, units == 0);
  else
    fwd_plan(batch, seqlen, heads, chunk, &nc, &nseg, &per, units);
  return nseg;
}

size_t fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t d_head,
                           int64_t d_state, int64_t chunk, int dtype, int64_t units) {
  if (bf16_path(d_head, d_state, chunk, dtype))
    return bf16_workspace_bytes(batch, seqlen, heads, units, units == 0);
  int nc, nseg, per;
  fwd_plan(batch, seqlen, heads, chunk, &nc, &nseg, &per, units);
  if (nseg <= 1) return 0;
  return (size_t)(batch * heads * nseg) * (size_t)(d_head * d_state + 1) * sizeof(float);
}

hipError_t launch_ssd_forward(const FwdArgs& a, int dtype, void* ws, hipStream_t s) {
  if (bf16_path(a.d_head, a.d_state, a.chunk, dtype)) return launch_ssd_forward_bf16(a, ws, s);
  if (dtype == MM_BF16) return launch_typed<bf16>(a, ws, s);
  return launch_typed<float>(a, ws, s);
}

}  // namespace mmssd
