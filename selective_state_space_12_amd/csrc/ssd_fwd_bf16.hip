// Chunked selective scan (SSD) forward, bf16 inputs with fp32 accumulation,
// d_head 64, d_state 128, one B/C group: the shape of the MatMamba blocks
// ("MatMamba: A Matryoshka State Space Model", block and nesting paragraphs;
// Mamba2 blocks with 64-wide heads).  Same recurrence and chunked identity as
// the general kernel in ssd_fwd.hip:
//   Y_diag[t] = sum_{s<=t} exp(Lambda_t - Lambda_s) (C_t . B_s) dt_s x_s
//   Y_off[t]  = exp(Lambda_t) H_prev . C_t,   y_t = Y_diag[t] + Y_off[t] + D x_t
//   H_next    = exp(Lambda_end) H_prev + sum_s exp(Lambda_end - Lambda_s) dt_s x_s B_s^T
// evaluated over tiles of 128 tokens (a 256-token chunk is two tiles: the
// chunked form is exact at any chunk length, so only rounding differs).
//
// MI355X design:
//  - tile_prep_kernel forms, once per (sequence, tile) and for every head,
//    the causal blocks of G = C B^T and the tiles of B^T and C, already in
//    the register order of the MFMA operands that consume them (1 KB per wave
//    load, fully coalesced), and a head-major copy of dt.  With one B/C group
//    all heads share them, so the C.B^T contraction leaves the per-head
//    kernel and every per-tile load is a few whole cache lines.
//  - ssd_bf16_kernel: one workgroup of 16 waves walks the tiles of one
//    (sequence, head, segment).  Eight waves produce outputs (one 16-token
//    block each), four own the fp32 state in MFMA accumulators, four stage x
//    and the decay cumsums; every SIMD runs waves of all three kinds, so the
//    output MFMAs overlap the state update and the staging.
//  - x and the bf16 copy of H live in LDS as MFMA operand fragments
//    (lane-major, 16 bytes per lane), so every operand read is a linear,
//    conflict-free 16-byte load.  Each staging wave transposes its 32 tokens
//    once per tile (raw rows to LDS, LDS transpose loads back) and writes two
//    x copies: plain, and times the tile-end factor exp(Lambda_end -
//    Lambda_s) dt_s (<= dt_s) for the state update.
//  - the state is decayed to the tile end once per tile, after which its
//    four 32-token MFMA blocks accumulate with no rescaling in between (a
//    per-block rescale had put a VALU step between dependent MFMAs on the
//    waves that bounded the tile time).
//  - every output block takes the plain x copy: off-diagonal 32-token blocks
//    split the factor exp(Lambda_t - Lambda_s) dt_s into exp(Lambda_t -
//    Lambda_e) (one scalar per lane, e = block end) times the block-end
//    factor exp(Lambda_e - Lambda_s) dt_s, both <= 1, applied to the G
//    fragment in registers; the diagonal block takes the direct masked form,
//    with D folded into the diagonal of the mask.
//  - output rows are dealt to the A operand in an order that leaves each lane
//    eight consecutive channels of a token, stored as one 16-byte write;
//  - LDS tiles are double-buffered and the decay cumsums triple-buffered, so
//    each tile costs one workgroup barrier; an output wave's G fragments sit
//    in two register sets, the next tile's requested a whole tile ahead.
//  - long sequences with few heads are split into segments: a state-only pass
//    (one or two heads per workgroup, pieces finer than the segments) forms
//    each piece's end state from zero, a combine chains them, and the main
//    kernel walks every segment from its chained start state.
#include <atomic>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "kernels.h"
#include "../../include/mm_ssd.h"

namespace mmssd {

namespace {

constexpr int kQ = 128;        // tokens per tile
constexpr int kP = 64;         // d_head
constexpr int kN = 128;        // d_state
constexpr int kTB = kQ / 16;   // 16-token blocks per tile
constexpr int kSB = kQ / 32;   // 32-token blocks per tile
constexpr int kPB = kP / 16;   // 16-wide d_head blocks
constexpr int kNB = kN / 16;   // 16-wide d_state blocks
constexpr int kKB = kN / 32;   // K=32 slices over d_state
constexpr int kNBW = kNB / 4;  // state column blocks per state wave
constexpr int kXcds = 8;
// 16 waves, four per SIMD: 0-7 outputs (one 16-token block each; waves w and
// w+4 share a SIMD and take blocks whose causal work adds up the same), 8-11
// state update, 12-15 x staging and decay cumsums.
constexpr int kThreads = 16 * 64;

// G fragments (tb, k) exist for the 32-token blocks k <= tb/2 (causal,
// diagonal block included), numbered tb-major.
__host__ __device__ constexpr int gbase(int tb) {
  return (tb / 2) * (tb / 2 + 1) + (tb & 1) * (tb / 2 + 1);
}
constexpr int kNG = gbase(kTB);                  // G fragments: 20
constexpr int kBT0 = kNG;                        // first B^T fragment (nb, ks): kNB * kSB
constexpr int kC0 = kBT0 + kNB * kSB;            // first C fragment (tb, kb): kTB * kKB
constexpr int kNFR = kC0 + kTB * kKB;            // fragments per (sequence, tile): 84
constexpr size_t kFragBytes = 64 * 16;           // one wave-wide fragment

// The x tiles and the bf16 copy of H live in LDS as MFMA operand fragments,
// lane-major (16 bytes per lane, 1 KB per fragment), so every operand read is
// one conflict-free linear 16-byte load:
//   x fragment (q, pb):   lane (r, g) holds x[q*32 + g*8 + j][column pb*16 + r]
//   H fragment (pb, kb):  lane (r, g) holds H[chan(pb, r)][kb*32 + g*8 + j]
constexpr int kXE = kQ * kP;   // elements of one x tile (16 fragments)
// Per buffer two x tiles: plain (output blocks) and scaled by the tile-end
// factor (the state update).
constexpr int kXBuf = 2 * kXE;
constexpr int kHF = kP * kN;   // elements of the operand copy of H (16 fragments)
// Raw token-major rows per staging wave: 4 rows before its 32 tokens (the
// conv window of a fused call) and the 32 rows themselves.
constexpr int kStgRows = 4 + 32;
constexpr int kStg = 4 * kStgRows * kP;
// floats: Lambda, dt, block-end factor exp2(Lambda_e - Lambda_s) dt_s (e the
// end of s's 32-token block), tile-end factor exp2(Lambda_end - Lambda_s) dt_s
constexpr size_t kDec = 4 * kQ;
// Output staging: each output wave's 16 tokens x 64 channels (rows laid out
// as the staged x rows, soff), so that y leaves in whole 128-byte lines.
constexpr int kYRows = 16;
constexpr size_t kYOff = (size_t)(2 * kXBuf + 2 * kHF + kStg) * sizeof(bf16) + 3 * kDec * sizeof(float);
constexpr size_t kLds = kYOff + (size_t)8 * kYRows * kP * sizeof(bf16);
// The state-only pass (segment end states, no outputs) keeps only the scaled
// x copy and no H copies or output rows: a compact layout, so that several
// of its 512-thread workgroups share a CU.
template <bool OUT> constexpr int kXBufL = OUT ? kXBuf : kXE;   // elements per x buffer
template <bool OUT> constexpr int kXFOff = OUT ? kXE : 0;       // scaled copy within a buffer
template <bool OUT> constexpr int kStgOff = 2 * kXBufL<OUT> + (OUT ? 2 * kHF : 0);  // elements
template <bool OUT> constexpr size_t kDecOff = (size_t)(kStgOff<OUT> + kStg) * sizeof(bf16);  // bytes
static_assert(kDecOff<true> + 3 * kDec * sizeof(float) == kYOff, "main layout");
constexpr size_t kLdsSeg = kDecOff<false> + 3 * kDec * sizeof(float);

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 pack4(f32x4 v) {
  return __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
}
__device__ __forceinline__ Frag8<bf16> as_frag(uint4 u) {
  Frag8<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}
__device__ __forceinline__ Frag8<bf16> lds_frag(const bf16* p) {
  return as_frag(*reinterpret_cast<const uint4*>(p));
}
// Element offset of a lane's 16 bytes of fragment f in a fragment-ordered tile
__device__ __forceinline__ int foff(int f, int lane) { return (f * 64 + lane) * 8; }

// Channel held at column c of an operand tile: tile pb = c/16, row m = c%16
// is channel (pb/2)*32 + (m/4)*8 + (pb%2)*4 + m%4.  Output tiles 2a and 2a+1
// then leave a lane eight consecutive channels (one 16-byte store).
__device__ __forceinline__ int chan(int pb, int m) {
  return (pb >> 1) * 32 + (m >> 2) * 8 + (pb & 1) * 4 + (m & 3);
}

// Raw rows staged by a staging wave: row s holds the head's 64 channels of
// one token in natural order (token s - 4 of the wave's 32), 8 chunks of 16
// bytes per 128-byte row, chunk index XOR-ed with s%8.  Element offset of
// (s, chunk):
__device__ __forceinline__ int soff(int s, int chunk) { return s * kP + ((chunk ^ (s & 7)) << 3); }

// Four consecutive staged rows sb..sb+3 for the channel chan(pb, r), read
// with one LDS transpose load: within each 16-lane group, lane i receives
// element i%4 of the 8 bytes that lane 4k + i/4 addresses, for k = 0..3.
// Lane src therefore addresses row sb + src/4 at the four channels
// chan(pb, 4*(src%4)) .. +3, which are consecutive:
// (pb/2)*32 + (src%4)*8 + (pb%2)*4.
typedef short short4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ short4v stg_rows4(const bf16* S, int sb, int pb, int lane) {
  const int src = lane & 15;
  const int chunk = (pb >> 1) * 4 + (src & 3), half = (pb & 1) * 4;
  typedef __attribute__((address_space(3))) short4v lds_short4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)(const_cast<bf16*>(S) + soff(sb + (src >> 2), chunk) + half));
}
// Operand fragment of the 8 staged rows sb..sb+7 (two transpose loads).
__device__ __forceinline__ Frag8<bf16> stg_frag(const bf16* S, int sb, int pb, int lane) {
  const short4v lo = stg_rows4(S, sb, pb, lane), hi = stg_rows4(S, sb + 4, pb, lane);
  Frag8<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

// f[j] *= sc[j] for the 8 operand values of a fragment (rounded back to bf16)
__device__ __forceinline__ Frag8<bf16> scale8(const Frag8<bf16>& f, const f32x4& a, const f32x4& b) {
  Frag8<bf16> r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.v[j] = static_cast<bf16>(static_cast<float>(f.v[j]) * a[j]);
    r.v[j + 4] = static_cast<bf16>(static_cast<float>(f.v[j + 4]) * b[j]);
  }
  return r;
}

// Lane value moved by a DPP pattern; lanes with no source (or outside the
// row mask) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}

// ---------------------------------------------------------------------------
// Per (sequence, tile), shared by every head:
//   G fragment (tb, k):    lane (r, g) holds G[tb*16 + r][k*32 + g*8 + j], j < 8
//   B^T fragment (np, e, ks): lane (r, g) holds B[ks*32 + g*8 + j][n] with
//                          n = np*32 + (r/4)*8 + e*4 + r%4 (so the state
//                          update leaves lane (p, g) eight consecutive n)
//   C fragment (tb, kb):   lane (r, g) holds C[tb*16 + r][kb*32 + g*8 + j]
// and, per head, dt of the tile's tokens as one contiguous row (dtT).  Rows
// past the end of the sequence repeat its last row (finite values that the
// scan multiplies by dt = 0 or never stores).  One workgroup per tile stages
// the B and C rows in LDS with whole-row loads and forms every fragment from
// there.
//
// Fused calls (raw conv input, FUSED): the workgroup also stages the three
// rows before the tile and applies the causal conv (kernel 4) + SiLU to the
// B and C channels in LDS, in the same fp32 operation order and rounding as
// the conv kernel, and turns raw dt into dt = softplus(dt + dt_bias) (or
// dt + dt_bias), rounded to bf16 as a stored dt would be.
// Byte offset of lane `lane`'s 16 bytes of fragment f in a tile's block.
__device__ __forceinline__ uint32_t frag_off(int f, int lane) { return (uint32_t)(f * 64 + lane) * 16; }
constexpr int kBCP = kN + 8;  // LDS row pitch (elements) of the staged B and C rows
constexpr int kBCRows = kQ + 3;  // the tile's rows and, for a fused call, three before it
// B and C rows; the dt transpose buffer reuses the C rows once the G and C
// fragments are out (71 KB: two workgroups per CU)
constexpr size_t kPrepLds = 2 * (size_t)kBCRows * kBCP * sizeof(bf16);
static_assert(64 * (kQ + 2) <= kQ * kBCP, "dt buffer fits in the C rows");

// (at most 128 VGPRs: two workgroups per CU)
template <bool FUSED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void tile_prep_kernel(const bf16* __restrict__ Bp, int64_t bs,
                                                        const bf16* __restrict__ Cp, int64_t cs,
                                                        const bf16* __restrict__ dtp, int64_t dts,
                                                        uint4* __restrict__ frags,
                                                        bf16* __restrict__ dtT, int64_t seqlen,
                                                        int ntiles, int heads, FuseArgs cv) {
  extern __shared__ __align__(16) unsigned char psm[];
  bf16 (*Bs)[kBCP] = reinterpret_cast<bf16 (*)[kBCP]>(psm);
  bf16 (*Cs)[kBCP] = reinterpret_cast<bf16 (*)[kBCP]>(psm + (size_t)kBCRows * kBCP * sizeof(bf16));
  bf16 (*Dt)[kQ + 2] = reinterpret_cast<bf16 (*)[kQ + 2]>(psm + (size_t)kBCRows * kBCP * sizeof(bf16));
  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)b * seqlen + (int64_t)c * kQ;
  const int last = (int)min((int64_t)kQ, seqlen - (int64_t)c * kQ) - 1;
  uint4* out = frags + ((int64_t)b * ntiles + c) * kNFR * 64;

  // dt of heads h0 .. h0+63: thread takes head h0 + tid%64, tokens tid/64 + 8i
  const int hh = tid & 63;
  bf16 dv[kQ / 8];
  auto load_dt = [&](int h0, int nh) {
    const int hd = h0 + min(hh, nh - 1);
#pragma unroll
    for (int i = 0; i < kQ / 8; ++i) {
      const int s = (tid >> 6) + 8 * i;
      dv[i] = dtp[(row0 + min(s, last)) * dts + hd];
    }
    if (FUSED) {
      const float db = cv.dt_bias ? cv.dt_bias[hd] : 0.0f;
#pragma unroll
      for (int i = 0; i < kQ / 8; ++i) {
        const float d = static_cast<float>(dv[i]) + db;
        dv[i] = static_cast<bf16>(cv.softplus ? softplus(d) : d);
      }
    }
  };
  if (!FUSED) load_dt(0, min(64, heads));  // in flight during the row loads
  // Row sr of Bs/Cs holds token sr - kH of the tile (kH = 3 before the conv of
  // a fused call, 0 otherwise); the rows before the sequence start are 0 (a
  // given conv state enters the conv below in fp32).
  constexpr int kH = FUSED ? 3 : 0;
  // Every row load of the tile is issued before any is written to LDS (a
  // loop that stored each pair before loading the next waited for one HBM
  // round trip per iteration).  Through buffer ranges that start kH rows
  // before the tile: rows at or past the sequence end read as 0 (finite
  // values that the scan multiplies by dt = 0 or never stores), and so do
  // the rows before the sequence start (a given conv state enters the conv
  // below in fp32).  B and C rows are read once here: nontemporal.
  {
    constexpr int kRowChunks = (kQ + kH) * (kN / 8);
    constexpr int kIt = (kRowChunks + 511) / 512;
    const int len = last + 1;
    const int64_t first = row0 - kH;  // row of staged row 0
    const uint64_t bb = reinterpret_cast<uint64_t>(Bp) + (uint64_t)(first * bs * (int64_t)sizeof(bf16));
    const uint64_t cb = reinterpret_cast<uint64_t>(Cp) + (uint64_t)(first * cs * (int64_t)sizeof(bf16));
    const uint32_t bstep = (uint32_t)(bs * sizeof(bf16)), cstep = (uint32_t)(cs * sizeof(bf16));
    const auto rb = uniform_rsrc(bb, (uint32_t)(len + kH) * bstep);
    const auto rc = uniform_rsrc(cb, (uint32_t)(len + kH) * cstep);
    uint4 bq[kIt], cq[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int v = tid + i * 512;
      const int sr = min(v, kRowChunks - 1) / (kN / 8), col = (v % (kN / 8)) * 8;
      // staged row sr; before the sequence start only in a fused call's first tile
      const bool before = c == 0 && sr < kH;
      bq[i] = buffer_load16<kPolicyNT>(rb, before ? 0xfffffff0u : (uint32_t)sr * bstep + col * 2);
      cq[i] = buffer_load16<kPolicyNT>(rc, before ? 0xfffffff0u : (uint32_t)sr * cstep + col * 2);
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int v = tid + i * 512;
      if (v < kRowChunks) {
        const int sr = v / (kN / 8), col = (v % (kN / 8)) * 8;
        *reinterpret_cast<uint4*>(&Bs[sr][col]) = bq[i];
        *reinterpret_cast<uint4*>(&Cs[sr][col]) = cq[i];
      }
    }
  }
  __syncthreads();
  if (FUSED) {
    // Thread: matrix m (B, C), 8 channels (group cg), 8 tokens (run).  It
    // takes its three history rows into registers, then (after a barrier, as
    // the previous run's thread overwrites them) turns each of its 8 raw rows
    // into the conv output in place: row sr = token sr - 3.
    const int m = tid >> 8, run = (tid >> 4) & 15, cg = tid & 15;
    bf16 (*S)[kBCP] = m ? Cs : Bs;
    const int64_t ch = cv.d_inner + m * kN + cg * 8;
    float wk[4][8], bv[8], hs[3][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 wj = *reinterpret_cast<const float4*>(cv.w + (ch + j) * 4);
      wk[0][j] = wj.x; wk[1][j] = wj.y; wk[2][j] = wj.z; wk[3][j] = wj.w;
      bv[j] = cv.bias ? cv.bias[ch + j] : 0.0f;
    }
    const bool from_state = c == 0 && run == 0 && cv.state;
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        hs[k][j] = from_state ? cv.state[((int64_t)b * 3 + k) * cv.conv_dim + ch + j]
                              : static_cast<float>(S[run * 8 + k][cg * 8 + j]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x8* row = reinterpret_cast<bf16x8*>(&S[run * 8 + 3 + i][cg * 8]);
      const bf16x8 u = *row;
      bf16x8 ov;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ut = static_cast<float>(u[j]);
        float pre = bv[j];
        pre = fmaf(wk[0][j], hs[0][j], pre);
        pre = fmaf(wk[1][j], hs[1][j], pre);
        pre = fmaf(wk[2][j], hs[2][j], pre);
        pre = fmaf(wk[3][j], ut, pre);
        ov[j] = static_cast<bf16>(silu(pre));
        hs[0][j] = hs[1][j];
        hs[1][j] = hs[2][j];
        hs[2][j] = ut;
      }
      *row = ov;
    }
    __syncthreads();
  }
  // token s of the tile at row s from here on
  Bs += kH;
  Cs += kH;
  if (FUSED) load_dt(0, min(64, heads));  // (after the conv: registers)

  // G^T tiles: A operand row m takes B row k*32 + (m/4)*8 + m%4 (tile a) or
  // that + 4 (tile b), B operand column n is C row tb*16 + n, so output slot
  // i of lane (r, g) is G[tb*16 + r][k*32 + g*8 + i] (a) and [.. + 4 + i] (b).
  // Waves 0-3 form three fragments, waves 4-7 two (f = wave + 8i), each
  // wave's fragments in one unrolled pass so that the LDS reads of all of them
  // are in flight together (one fragment at a time waited for its reads).
  // Fragments leave with nontemporal stores: they are read back from HBM by
  // the scan kernels, and streaming them out shortens the kernel's drain.
  const uint32_t fbytes = (uint32_t)(kNFR * kFragBytes);
  auto g_frags = [&](auto nf) {
    constexpr int NF = decltype(nf)::value;
    int tbs[NF], sas[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int f = wave + 8 * i;
      int tb = 0;
      while (gbase(tb + 1) <= f) ++tb;
      tbs[i] = tb;
      sas[i] = (f - gbase(tb)) * 32 + (r16 >> 2) * 8 + (r16 & 3);
    }
    f32x4 da[NF], db[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) da[i] = db[i] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int n = kb * 32 + g * 8;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const Frag8<bf16> cfr = lds_frag(&Cs[tbs[i] * 16 + r16][n]);
        da[i] = mma(lds_frag(&Bs[sas[i]][n]), cfr, da[i]);
        db[i] = mma(lds_frag(&Bs[sas[i] + 4][n]), cfr, db[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const uint2 lo = pack4(da[i]), hi = pack4(db[i]);
      store16_nt_ranged(out, fbytes, frag_off(wave + 8 * i, lane), make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
  };
  static_assert(kNG == 20, "three G fragments for waves 0-3, two for waves 4-7");
  if (wave < 4)
    g_frags(std::integral_constant<int, 3>{});
  else
    g_frags(std::integral_constant<int, 2>{});
  // B^T fragments with LDS transpose loads: within each 16-lane group lane i
  // receives element i%4 of the 8 bytes lane 4k + i/4 addresses (k = 0..3),
  // so lane src addresses row ks*32 + g*8 + src/4 (+4), columns
  // np*32 + (src%4)*8 + e*4 .. +3.
  typedef __attribute__((address_space(3))) short4v lds_short4;
  static_assert(kNB * kSB == 32 && kTB * kKB == 32, "four B^T and four C fragments per wave");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = wave + 8 * i;
    const int npe = f / kSB, ks = f % kSB;  // npe = np*2 + e
    const int src = lane & 15;
    const int col = (npe >> 1) * 32 + (src & 3) * 8 + (npe & 1) * 4;
    const int s1 = ks * 32 + g * 8 + (src >> 2);
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)&Bs[s1][col]);
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)&Bs[s1 + 4][col]);
    store16_nt_ranged(out, fbytes, frag_off(kBT0 + f, lane),
                      __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = wave + 8 * i;
    const int tb = f / kKB, kb = f % kKB;
    store16_nt_ranged(out, fbytes, frag_off(kC0 + f, lane),
                      *reinterpret_cast<const uint4*>(&Cs[tb * 16 + r16][kb * 32 + g * 8]));
  }

  // dt, 64 heads at a time: [token][head] -> LDS -> [head][token]
  bf16* dto = dtT + ((int64_t)b * ntiles + c) * heads * kQ;
  for (int h0 = 0; h0 < heads; h0 += 64) {
    const int nh = min(64, heads - h0);
    if (h0 > 0) load_dt(h0, nh);
    __syncthreads();  // C rows (aliased) consumed / previous group's rows written out
    if (hh < nh) {
#pragma unroll
      for (int i = 0; i < kQ / 8; ++i) Dt[hh][(tid >> 6) + 8 * i] = dv[i];
    }
    __syncthreads();
    for (int v2 = tid; v2 < nh * (kQ / 2); v2 += 512) {
      const int hr = v2 / (kQ / 2), s2 = v2 % (kQ / 2);
      *reinterpret_cast<uint32_t*>(dto + (int64_t)(h0 + hr) * kQ + 2 * s2) =
          *reinterpret_cast<const uint32_t*>(&Dt[hr][2 * s2]);
    }
  }
}

struct BK {
  const bf16* x;
  int64_t xs;
  const bf16* dt;
  int64_t dts;
  const float* A;
  const bf16* C;
  int64_t cs;
  const float* D;
  bf16* y;
  int64_t ys;
  const float* h0;
  float* hT;
  const uint4* frags;
  const bf16* dtT;
  float* seg_state;
  float* seg_decay;
  // fused calls: x is the raw conv input of the x channels; the staging
  // waves apply the conv (weights cw, bias cbias, history cstate)
  const float* cw;
  const float* cbias;
  const float* cstate;
  int64_t conv_dim;
  int64_t seqlen;
  int n_heads, heads, nseg, seg_chunks, ntiles;
  // split calls: each main segment but the last is cut into ppseg pieces of
  // piece_tiles tiles for the state-only pass; state slot i of a unit holds
  // the state entering piece i (nslot = (nseg - 1) * ppseg + 1 per unit)
  int ppseg, piece_tiles, nslot;
  // mixed calls: the grid is (segments x active units) on x, units numbered
  // sequence-major (heads of one sequence adjacent)
  UnitMap um;
};

// Buffer range over the fragments of tile c of sequence b, and the byte
// offset of lane `lane`'s 16 bytes of fragment f in it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_frags(const BK& k, int b, int c) {
  return uniform_rsrc(k.frags + ((int64_t)b * k.ntiles + c) * kNFR * 64, (uint32_t)(kNFR * kFragBytes));
}

// ---------------------------------------------------------------------------
// Output waves (OUT only).  Each produces one 16-token block tb of every tile
// for all 64 channels of the head; L = tb/2 is the number of 32-token blocks
// left of its diagonal block.  Output tiles are held transposed, D[m][t]:
// row m of tile pb = 2a + e is channel a*32 + (m/4)*8 + e*4 + m%4, so lane
// (r, g) holds channels a*32 + g*8 + e*4 + i of token tb*16 + r: tiles 2a and
// 2a+1 together give it eight consecutive channels, one 16-byte store.
template <int L>
__device__ void output_wave(const BK& k, unsigned char* smem, int b, int h, int c0, int c1,
                            int tb) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const bf16* xbuf = reinterpret_cast<const bf16*>(smem);
  const bf16* hbuf = xbuf + 2 * kXBuf;
  const float* dbuf = reinterpret_cast<const float*>(smem + kDecOff<true>);
  bf16* ybuf = reinterpret_cast<bf16*>(smem + kYOff) + (threadIdx.x >> 6) * kYRows * kP;
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Dh = k.D ? k.D[h] : 0.0f;
  const int t = tb * 16 + r16;  // this lane's token within a tile

  Frag8<bf16> cf[kKB];
  // G fragments in two register sets used in turn: tile c+1's are requested
  // at the start of tile c, a whole tile before its diagonal mask needs them
  // (requested at the end of tile c they arrived last, and the waves with the
  // most G blocks waited on them while the other roles idled at the barrier)
  Frag8<bf16> g0[L + 1], g1[L + 1];
  auto load_c = [&](int c) {
    const auto r = tile_frags(k, b, c);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
      cf[kb] = as_frag(buffer_load16<kPolicyDefault>(r, frag_off(kC0 + tb * kKB + kb, lane)));
  };
  auto load_g = [&](Frag8<bf16> (&g)[L + 1], int c) {
    const auto r = tile_frags(k, b, c);
#pragma unroll
    for (int q = 0; q <= L; ++q)
      g[q] = as_frag(buffer_load16<kPolicyDefault>(r, frag_off(gbase(tb) + q, lane)));
  };

  load_c(c0);
  load_g(g0, c0);
  // Two stores with an empty range (dropped by the hardware) after the
  // prologue loads, as each tile issues its two y stores after its loads:
  // the compiler's wait at the top of the loop then lets the previous tile's
  // stores stay in flight on every path into it.
  store16_nt_ranged(k.y, 0u, 0u, make_uint4(0u, 0u, 0u, 0u));
  store16_nt_ranged(k.y, 0u, 0u, make_uint4(0u, 0u, 0u, 0u));
  __syncthreads();  // decay cumsums and H_prev copy of the first tile
  __syncthreads();  // x copies of the first tile

  // one tile: G fragments of tile c in gf, tile c+1's requested into gn
  auto tile = [&](const int c, Frag8<bf16> (&gf)[L + 1], Frag8<bf16> (&gn)[L + 1]) {
    // Prefetches are unconditional (the last tile reloads itself): with a
    // fixed number of loads per tile the compiler's vmcnt waits stay exact
    // instead of draining loads that were just issued.
    const int cn = min(c + 1, c1 - 1);
    load_g(gn, cn);
    const int len = (int)min((int64_t)kQ, k.seqlen - (int64_t)c * kQ);
    const int64_t r0 = rowb + (int64_t)c * kQ;
    const bf16* Hs = hbuf + (c & 1) * kHF;
    const bf16* XT = xbuf + (c & 1) * kXBuf;
    const float* lam = dbuf + (c % 3) * kDec;
    const float* dtv = lam + kQ;
    const float* bef = lam + 2 * kQ;  // block-end factors

    f32x4 acc[kPB];
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) acc[pb] = f32x4{0, 0, 0, 0};

    // Diagonal block: M[t][s] = G[t][s] exp2(lam_t - lam_s) dt_s for s <= t,
    // plus D on s == t (the skip term D x_t).  Built in two halves dealt
    // between the Y_off MFMAs below (independent VALU work).
    const float lt = lam[t];
    Frag8<bf16> m;
    auto mask4 = [&](int j0) {
      const int sb = L * 32 + g * 8 + j0;
      const f32x4 ls = *reinterpret_cast<const f32x4*>(lam + sb);
      const f32x4 ds = *reinterpret_cast<const f32x4*>(dtv + sb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = sb + j;
        float v = static_cast<float>(gf[L].v[j0 + j]) * __builtin_amdgcn_exp2f(lt - ls[j]) * ds[j];
        v = s <= t ? v : 0.0f;
        v = s == t ? v + Dh : v;
        m.v[j0 + j] = static_cast<bf16>(v);
      }
    };

    // Y_off before scaling: D[p][t] = sum_n H_prev[p][n] C[t][n]
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const Frag8<bf16> hf = lds_frag(Hs + foff(pb * kKB + kb, lane));
        acc[pb] = mma(hf, cf[kb], acc[pb]);
      }
      if (kb == 1) mask4(0);
      if (kb == 3) mask4(4);
    }
    load_c(cn);

    // The state's contribution decays from the tile start to the token.
    {
      const float st = __builtin_amdgcn_exp2f(lt);
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) acc[pb] *= st;
    }
    // Off-diagonal blocks q < L: the exact factor exp2(lam_t - lam_s) dt_s
    // is split as exp2(lam_t - lam_e) (e = end of block q, one scalar per
    // lane, <= 1) times the block-end factor of s, and applied to the G
    // fragment in registers, so these blocks take the plain x copy.
#pragma unroll
    for (int q = 0; q < L; ++q) {
      const float f = __builtin_amdgcn_exp2f(lt - lam[q * 32 + 31]);
      const f32x4 ga = *reinterpret_cast<const f32x4*>(bef + q * 32 + g * 8);
      const f32x4 gb = *reinterpret_cast<const f32x4*>(bef + q * 32 + g * 8 + 4);
      Frag8<bf16> mq;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mq.v[j] = static_cast<bf16>(static_cast<float>(gf[q].v[j]) * (f * ga[j]));
        mq.v[j + 4] = static_cast<bf16>(static_cast<float>(gf[q].v[j + 4]) * (f * gb[j]));
      }
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const Frag8<bf16> xf = lds_frag(XT + foff(q * kPB + pb, lane));
        acc[pb] = mma(xf, mq, acc[pb]);
      }
    }
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      const Frag8<bf16> xf = lds_frag(XT + foff(L * kPB + pb, lane));
      acc[pb] = mma(xf, m, acc[pb]);
    }

    // Every load of the tile is issued before the y stores: the vmcnt
    // counter retires in order, so a load issued after the stores would make
    // its wait (early in the next tile) wait for the stores too.
    // y through the wave's LDS rows: lane (r, g) holds chunks g and 4 + g
    // (16 bytes each) of token r; read back, lane (i, j) = (lane / 8, lane % 8)
    // holds chunk j of token 8k + i, so each store instruction writes eight
    // whole 128-byte lines.  Whole-line nontemporal stores let the L2 hand
    // the lines to HBM without interleaving with the fragment loads that
    // every head repeats (measured: half-line stores cost ~20% of the
    // kernel).  One wave's LDS operations complete in order, so the reads see
    // the writes and the next tile's writes follow this tile's reads.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint2 lo = pack4(acc[2 * a]), hi = pack4(acc[2 * a + 1]);
      *reinterpret_cast<uint4*>(ybuf + soff(r16, a * 4 + g)) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int row = kk * 8 + (lane >> 3);
      const uint4 v = *reinterpret_cast<const uint4*>(ybuf + soff(row, lane & 7));
      // rows tb*16 + 8kk .. +7; those at or past the sequence end are dropped
      const int first = tb * 16 + kk * 8;
      const int nrows = min(max(len - first, 0), 8);
      store16_nt_ranged(k.y + (r0 + first) * k.ys + (int64_t)h * kP,
                        (uint32_t)(nrows * k.ys * (int64_t)sizeof(bf16)),
                        (uint32_t)((lane >> 3) * k.ys * (int64_t)sizeof(bf16) + (lane & 7) * 16), v);
    }
    __syncthreads();
  };
  for (int c = c0; c < c1; c += 2) {
    tile(c, g0, g1);
    if (c + 1 < c1) tile(c + 1, g1, g0);
  }
}

// ---------------------------------------------------------------------------
// State waves.  Wave u owns the state columns n in [32u, 32u + 32) for all
// rows: H^T tiles D[m][p] (e = 0, 1), lane (r, g) holds
// H[chan(pb, r)][32u + g*8 + e*4 + i], eight consecutive columns over the two
// tiles (the B^T fragments deal their rows in that order).
template <bool OUT>
__device__ void state_waves(const BK& k, unsigned char* smem, int b, int h, int seg, int c0,
                            int c1, int u) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const bf16* xbuf = reinterpret_cast<const bf16*>(smem);
  bf16* hbuf = reinterpret_cast<bf16*>(smem) + 2 * kXBuf;  // (OUT only)
  const float* dbuf = reinterpret_cast<const float*>(smem + kDecOff<OUT>);

  f32x4 hacc[kNBW][kPB];
  {
    const float* hin = nullptr;
    if (OUT) {
      if (k.nseg > 1)
        hin = k.seg_state + (((int64_t)b * k.heads + h) * k.nslot + seg * k.ppseg) * (kP * kN);
      else if (k.h0)
        hin = k.h0 + ((int64_t)b * k.n_heads + h) * (kP * kN);
    }
#pragma unroll
    for (int e = 0; e < kNBW; ++e)
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb)
        hacc[e][pb] = hin ? *reinterpret_cast<const f32x4*>(
                                hin + chan(pb, r16) * kN + u * 32 + g * 8 + e * 4)
                          : f32x4{0, 0, 0, 0};
  }
  Frag8<bf16> bt[kNBW][kSB];
  auto load_bt = [&](int c, int ks) {  // one 32-token slice of this wave's B^T columns
    const auto r = tile_frags(k, b, c);
#pragma unroll
    for (int j = 0; j < kNBW; ++j)
      bt[j][ks] = as_frag(
          buffer_load16<kPolicyDefault>(r, frag_off(kBT0 + (u * kNBW + j) * kSB + ks, lane)));
  };
  // this wave's columns are exactly the H fragments (pb, kb = u)
  auto write_hs = [&](int buf) {
    bf16* Hs = hbuf + buf * kHF;
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      const uint2 lo = pack4(hacc[0][pb]), hi = pack4(hacc[1][pb]);
      *reinterpret_cast<uint4*>(Hs + foff(pb * kKB + u, lane)) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };

  // The same loads in the same order every iteration (tile index clamped to
  // the last tile), and the prologue ends with that sequence, so the
  // compiler's vmcnt waits stay exact.
  const int cl = c1 - 1;
  if (OUT) write_hs(c0 & 1);
#pragma unroll
  for (int ks = 0; ks < kSB; ++ks) load_bt(c0, ks);
  __syncthreads();  // decay cumsums of the first tiles
  __syncthreads();  // x copies of the first tile

  for (int c = c0; c < c1; ++c) {
    // H <- exp2(Lambda_end) H + sum_s exp2(Lambda_end - Lambda_s) dt_s x_s B_s^T:
    // the state is decayed to the tile end once, then the four 32-token
    // blocks add B^T times the x copy that carries the tile-end factor
    // exp2(lam_end - lam_s) dt_s (<= dt_s), with no rescaling between them.
    // A operand B^T rows, B operand x; each B^T slice is reloaded for the
    // next tile as soon as its MFMAs are issued.
    const float* d = dbuf + (c % 3) * kDec;
    const bf16* XF = xbuf + (c & 1) * kXBufL<OUT> + kXFOff<OUT>;
    {
      const float rt = __builtin_amdgcn_exp2f(d[kQ - 1]);
#pragma unroll
      for (int j = 0; j < kNBW; ++j)
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) hacc[j][pb] *= rt;
    }
#pragma unroll
    for (int ks = 0; ks < kSB; ++ks) {
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const Frag8<bf16> xf = lds_frag(XF + foff(ks * kPB + pb, lane));
#pragma unroll
        for (int j = 0; j < kNBW; ++j) hacc[j][pb] = mma(bt[j][ks], xf, hacc[j][pb]);
      }
      load_bt(min(c + 1, cl), ks);
    }
    if (OUT && c + 1 < c1) write_hs((c + 1) & 1);
    __syncthreads();
  }

  float* hout = nullptr;
  if (OUT) {
    if (k.hT && seg == k.nseg - 1) hout = k.hT + ((int64_t)b * k.n_heads + h) * (kP * kN);
  } else {
    hout = k.seg_state + (((int64_t)b * k.heads + h) * k.nslot + seg) * (kP * kN);  // seg: piece
  }
  if (hout) {
#pragma unroll
    for (int e = 0; e < kNBW; ++e)
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb)
        *reinterpret_cast<f32x4*>(hout + chan(pb, r16) * kN + u * 32 + g * 8 + e * 4) =
            hacc[e][pb];
  }
}

// ---------------------------------------------------------------------------
// Stage waves.  Wave v turns tokens 32v..32v+31 of each tile, one tile ahead,
// into the x fragments (v, pb) of both LDS x tiles (plain and times the
// tile-end factor): its raw rows go to its own staging rows (layout at soff)
// and come back transposed, as operand fragments, from LDS transpose loads.
// In a fused call the wave also stages the 4 rows before its tokens and
// applies the causal conv (kernel 4) + SiLU to the transposed fragments, where
// each lane holds 8 consecutive tokens of one channel: the same fp32
// operation order and rounding as the conv kernel.
// All four also form the decay cumsum two tiles ahead (a few DPP steps) and
// each writes one of its four arrays.
template <bool OUT, bool FUSED>
__device__ void stage_waves(const BK& k, unsigned char* smem, int b, int h, int seg, int c0,
                            int c1, int v) {
  const int lane = threadIdx.x & 63;
  bf16* xbuf = reinterpret_cast<bf16*>(smem);
  bf16* stg = xbuf + kStgOff<OUT> + v * kStgRows * kP;  // this wave's staged rows
  float* dbuf = reinterpret_cast<float*>(smem + kDecOff<OUT>);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const float Ah2 = k.A[h] * kLog2e;

  // Lane: channels 8*(lane%8) .. +7 (chunk lane%8) of tokens 32v + 8i + lane/8,
  // one 16-byte load each (eight lanes read a whole 128-byte row).  x is read
  // once: nontemporal loads (measured 6% faster on the whole kernel).
  // (four named registers, not an array: the array was placed in scratch)
  const int pc = lane & 7;
  // rows r0..r3 (tokens 32v + 8i + lane/8) and, fused, the halo row
  struct XSet { uint4 r0, r1, r2, r3, h; };
  XSet xs;
  // Rows at or past the sequence end lie outside the tile's buffer range and
  // read as 0 (finite values that the scan multiplies by dt = 0 or never
  // stores), so every iteration issues the same loads with no lane condition.
  const uint32_t rowbytes = (uint32_t)(k.xs * (int64_t)sizeof(bf16));
  auto load_x = [&](int c) {
    const int len = (int)min((int64_t)kQ, k.seqlen - (int64_t)c * kQ);
    const uint64_t tile0 = reinterpret_cast<uint64_t>(k.x) +
                           (uint64_t)(((rowb + (int64_t)c * kQ) * k.xs + (int64_t)h * kP) * sizeof(bf16));
    const auto r = uniform_rsrc(tile0, (uint32_t)len * rowbytes);
    auto row = [&](int i) {
      const int s = v * 32 + i * 8 + (lane >> 3);
      return buffer_load16<kPolicyNT>(r, (uint32_t)s * rowbytes + pc * 16);
    };
    xs.r0 = row(0);
    xs.r1 = row(1);
    xs.r2 = row(2);
    xs.r3 = row(3);
    if (FUSED) {
      // the 4 tokens before the wave's first (lanes 32-63 repeat lanes 0-31),
      // through a range that starts 4 rows before the tile; before the
      // sequence start they read 0 (a conv state enters in fp32 below)
      const int s = v * 32 - 4 + ((lane >> 3) & 3);
      const auto rh = uniform_rsrc(tile0 - 4 * (uint64_t)rowbytes, (uint32_t)(len + 4) * rowbytes);
      const uint32_t off = (s >= 0 || c > 0) ? (uint32_t)(s + 4) * rowbytes + pc * 16 : 0xfffffff0u;
      xs.h = buffer_load16<kPolicyDefault>(rh, off);
    }
  };
  // conv weights and bias of the lane's channels h*64 + chan(pb, r)
  f32x4 cwk[kPB];
  float cbv[kPB];
  if (FUSED) {
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      const int64_t ch = (int64_t)h * kP + chan(pb, lane & 15);
      cwk[pb] = *reinterpret_cast<const f32x4*>(k.cw + ch * 4);
      cbv[pb] = k.cbias ? k.cbias[ch] : 0.0f;
    }
  }
  // Raw rows out, fragments back (LDS operations of one wave complete in
  // order, so the transpose loads see the rows just written), then the plain
  // fragments and the ones scaled by exp2(lam[e] - lam_s) dt_s, e the end of
  // the token's 32-token block (lane (r, g) holds tokens 32v + g*8 + j).
  auto commit = [&](int c) {
    bf16* XT = xbuf + (c & 1) * kXBufL<OUT>;  // (plain copy: OUT only)
    bf16* XF = XT + kXFOff<OUT>;
    const float* d = dbuf + (c % 3) * kDec;
    *reinterpret_cast<uint4*>(stg + soff(4 + (lane >> 3), pc)) = xs.r0;
    *reinterpret_cast<uint4*>(stg + soff(12 + (lane >> 3), pc)) = xs.r1;
    *reinterpret_cast<uint4*>(stg + soff(20 + (lane >> 3), pc)) = xs.r2;
    *reinterpret_cast<uint4*>(stg + soff(28 + (lane >> 3), pc)) = xs.r3;
    if (FUSED && lane < 32) *reinterpret_cast<uint4*>(stg + soff(lane >> 3, pc)) = xs.h;
    Frag8<bf16> f[kPB];
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) f[pb] = stg_frag(stg, 4 + (lane >> 4) * 8, pb, lane);
    if (FUSED) {
      // lanes holding a sequence's first tokens take the history from the
      // conv state in fp32 (loaded here: once per sequence)
      const bool first = c == 0 && v == 0 && (lane >> 4) == 0 && k.cstate;
      const float* hist = first ? k.cstate + (int64_t)b * 3 * k.conv_dim + (int64_t)h * kP : nullptr;
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        // tokens -4..-1 as bf16 pairs: a bf16 is the high half of its fp32,
        // so the three taps are word 0's high half and word 1's two halves
        // (element extraction through a bf16 bit_cast of the short vector
        // was lowered to element 0 for all three)
        const uint2 hw = __builtin_bit_cast(uint2, stg_rows4(stg, (lane >> 4) * 8, pb, lane));
        float h0 = __builtin_bit_cast(float, hw.x & 0xffff0000u);
        float h1 = __builtin_bit_cast(float, hw.y << 16);
        float h2 = __builtin_bit_cast(float, hw.y & 0xffff0000u);
        const int ch = chan(pb, lane & 15);
        if (first) {
          h0 = hist[ch];
          h1 = hist[k.conv_dim + ch];
          h2 = hist[2 * k.conv_dim + ch];
        }
        const f32x4 wk = cwk[pb];
        const float bias = cbv[pb];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float ut = static_cast<float>(f[pb].v[j]);
          float pre = bias;
          pre = fmaf(wk[0], h0, pre);
          pre = fmaf(wk[1], h1, pre);
          pre = fmaf(wk[2], h2, pre);
          pre = fmaf(wk[3], ut, pre);
          f[pb].v[j] = static_cast<bf16>(silu(pre));
          h0 = h1;
          h1 = h2;
          h2 = ut;
        }
      }
    }
    const float* ef = d + 3 * kQ + v * 32 + (lane >> 4) * 8;
    const f32x4 e0 = *reinterpret_cast<const f32x4*>(ef);
    const f32x4 e1 = *reinterpret_cast<const f32x4*>(ef + 4);
#pragma unroll
    for (int pb = 0; pb < kPB; ++pb) {
      if (OUT) *reinterpret_cast<uint4*>(XT + foff(v * kPB + pb, lane)) = __builtin_bit_cast(uint4, f[pb].v);
      *reinterpret_cast<uint4*>(XF + foff(v * kPB + pb, lane)) =
          __builtin_bit_cast(uint4, scale8(f[pb], e0, e1).v);
    }
  };
  // dt of tokens 2*lane, 2*lane + 1 of a tile (head-major copy), kept raw
  // until make_dec (a conversion here would make the wave wait for the load)
  auto load_dt = [&](int c) -> uint32_t {
    const auto r = uniform_rsrc(k.dtT + (((int64_t)b * k.ntiles + c) * k.heads + h) * kQ,
                                (uint32_t)(kQ * sizeof(bf16)));
    return buffer_load4<kPolicyDefault>(r, (uint32_t)lane * 4);
  };
  uint32_t dtr_raw;
  // Lambda (inclusive cumsum of dt*A, log2 units), dt, block-end factor
  // exp2(Lambda_e - Lambda_s) dt_s and tile-end factor exp2(Lambda_end -
  // Lambda_s) dt_s of tile c (dt = 0 past the end of the sequence).
  auto make_dec = [&](int c, int buf, uint32_t raw) {
    const int len = (int)min((int64_t)kQ, k.seqlen - (int64_t)c * kQ);
    float dtr[2];
    dtr[0] = 2 * lane < len ? __builtin_bit_cast(float, raw << 16) : 0.0f;
    dtr[1] = 2 * lane + 1 < len ? __builtin_bit_cast(float, raw & 0xffff0000u) : 0.0f;
    float* d = dbuf + buf * kDec;
    const float v0 = dtr[0] * Ah2, v1 = dtr[1] * Ah2;
    // inclusive scan over the wave with DPP row shifts and row broadcasts
    float incl = v0 + v1;
    incl += dpp_f<0x111, 0xf>(incl);  // row_shr:1
    incl += dpp_f<0x112, 0xf>(incl);  // row_shr:2
    incl += dpp_f<0x114, 0xf>(incl);  // row_shr:4
    incl += dpp_f<0x118, 0xf>(incl);  // row_shr:8
    incl += dpp_f<0x142, 0xa>(incl);  // row_bcast:15 into rows 1 and 3
    incl += dpp_f<0x143, 0xc>(incl);  // row_bcast:31 into rows 2 and 3
    const float l0 = incl - v1, l1 = incl;
    const float lend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
    // tokens 32q..32q+31 sit in lanes 16q..16q+15: the block end is lane 16q+15
    const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 15));
    const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 31));
    const float e2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 47));
    const int row = lane >> 4;
    const float lblk = row == 0 ? e0 : row == 1 ? e1 : row == 2 ? e2 : lend;
    if (v == 0) {
      *reinterpret_cast<float2*>(d + 2 * lane) = make_float2(l0, l1);
    } else if (v == 1) {
      *reinterpret_cast<float2*>(d + kQ + 2 * lane) = make_float2(dtr[0], dtr[1]);
    } else if (v == 2) {
      *reinterpret_cast<float2*>(d + 2 * kQ + 2 * lane) =
          make_float2(__builtin_amdgcn_exp2f(lblk - l0) * dtr[0], __builtin_amdgcn_exp2f(lblk - l1) * dtr[1]);
    } else {
      *reinterpret_cast<float2*>(d + 3 * kQ + 2 * lane) =
          make_float2(__builtin_amdgcn_exp2f(lend - l0) * dtr[0], __builtin_amdgcn_exp2f(lend - l1) * dtr[1]);
    }
    return lend;
  };

  // The same loads in the same order every iteration (x, dt; tile indices
  // clamped to the last tile), and the prologue ends with that sequence, so
  // the compiler's vmcnt waits stay exact.
  const int cl = c1 - 1;
  float lam_seg = 0.0f;
  load_x(c0);
  const uint32_t dt0 = load_dt(c0), dt1 = load_dt(min(c0 + 1, cl));  // both in flight
  lam_seg += make_dec(c0, c0 % 3, dt0);
  if (c0 + 1 < c1) lam_seg += make_dec(c0 + 1, (c0 + 1) % 3, dt1);
  __syncthreads();
  commit(c0);
  load_x(min(c0 + 1, cl));
  dtr_raw = load_dt(min(c0 + 2, cl));
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) commit(c + 1);
    load_x(min(c + 2, cl));
    if (c + 2 < c1) lam_seg += make_dec(c + 2, (c + 2) % 3, dtr_raw);
    dtr_raw = load_dt(min(c + 3, cl));
    __syncthreads();
  }
  if (!OUT && v == 0 && lane == 0)
    k.seg_decay[((int64_t)b * k.heads + h) * k.nslot + seg] = lam_seg;  // seg: piece
}

// XCD-aware unit mapping: consecutive workgroups go to different XCDs, so
// give each XCD a contiguous block of units numbered head fastest; the heads
// that walk the same tiles (same sequence and segment) then share one L2 for
// the fragments.  Grid (parts, heads, batch), or (parts * units) for mixed
// calls; returns the part (segment or piece) index.
__device__ __forceinline__ int unit_of_block(const BK& k, int* b, int* h) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int pid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int uid = total % kXcds == 0 ? (pid % kXcds) * (total / kXcds) + pid / kXcds : pid;
  if (k.um.mixed) {
    unit_to_bh(k.um, uid % k.um.units, b, h);
    return uid / k.um.units;
  }
  *h = uid % gy;
  *b = uid / (gx * gy);
  return (uid / gy) % gx;
}

template <bool FUSED>
__global__ __launch_bounds__(kThreads) void ssd_bf16_kernel(BK k) {
  extern __shared__ __align__(16) unsigned char smem[];
  int b, h;
  const int seg = unit_of_block(k, &b, &h);
  const int c0 = seg * k.seg_chunks;
  const int c1 = min(c0 + k.seg_chunks, k.ntiles);
  if (c0 >= c1) return;  // whole workgroup
  // wave index as a scalar, so the role branch below is uniform per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 12) {
    stage_waves<true, FUSED>(k, smem, b, h, seg, c0, c1, wave - 12);
  } else if (wave >= 8) {
    state_waves<true>(k, smem, b, h, seg, c0, c1, wave - 8);
  } else {
    const int tb = wave < 4 ? wave : kTB + 3 - wave;  // 0 1 2 3 7 6 5 4
    switch (tb >> 1) {
      case 0: output_wave<0>(k, smem, b, h, c0, c1, tb); break;
      case 1: output_wave<1>(k, smem, b, h, c0, c1, tb); break;
      case 2: output_wave<2>(k, smem, b, h, c0, c1, tb); break;
      default: output_wave<3>(k, smem, b, h, c0, c1, tb); break;
    }
  }
}

// State-only pass of a split call: for each unit and each piece of the
// segments before the last, the state at the piece end starting from zero
// (slot = piece) and the piece's total log2 decay.  Eight waves (four stage
// x, four update the state) in a compact LDS layout (56 KB); the pieces may
// be finer than the segments so that these workgroups fill the GPU.
template <bool FUSED>
__global__ __launch_bounds__(512) void ssd_bf16_seg_kernel(BK k) {
  extern __shared__ __align__(16) unsigned char smem[];
  int b, h;
  const int piece = unit_of_block(k, &b, &h);
  const int seg = piece / k.ppseg;
  const int c0 = seg * k.seg_chunks + (piece % k.ppseg) * k.piece_tiles;
  const int c1 = min(min(c0 + k.piece_tiles, (seg + 1) * k.seg_chunks), k.ntiles);
  if (c0 >= c1) return;  // whole workgroup (the planner makes no empty piece)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4)
    state_waves<false>(k, smem, b, h, piece, c0, c1, wave - 4);
  else
    stage_waves<false, FUSED>(k, smem, b, h, piece, c0, c1, wave);
}

// ---------------------------------------------------------------------------
// State-only pass over two heads of a sequence per workgroup (calls without
// the fused conv and without per-sequence widths).  The state waves load
// each tile's B^T fragments once and update both heads' states with them, so
// the bytes the CU reads per head and tile fall from 48 KB (16 KB of x, 32
// KB of B^T) to 32 KB; the staging waves stage both heads' x.  Same
// arithmetic per head as the one-head pass.  With an odd head count the last
// workgroup repeats its head as the second and stores it once.
constexpr int kXBuf2 = 2 * kXE;  // per parity: head 0's scaled x, then head 1's
constexpr size_t kDecOff2 = (size_t)(2 * kXBuf2 + kStg) * sizeof(bf16);
constexpr size_t kLdsSeg2 = kDecOff2 + 2 * 3 * kDec * sizeof(float);  // per head: three decay sets

__device__ void state_waves2(const BK& k, unsigned char* smem, int b, int h0, int nh, int piece,
                             int c0, int c1, int u) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const bf16* xbuf = reinterpret_cast<const bf16*>(smem);
  const float* dbuf = reinterpret_cast<const float*>(smem + kDecOff2);
  f32x4 hacc[2][kNBW][kPB];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int j = 0; j < kNBW; ++j)
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) hacc[e][j][pb] = f32x4{0, 0, 0, 0};
  Frag8<bf16> bt[kNBW][kSB];
  auto load_bt = [&](int c, int ks) {
    const auto r = tile_frags(k, b, c);
#pragma unroll
    for (int j = 0; j < kNBW; ++j)
      bt[j][ks] = as_frag(
          buffer_load16<kPolicyDefault>(r, frag_off(kBT0 + (u * kNBW + j) * kSB + ks, lane)));
  };
  const int cl = c1 - 1;
#pragma unroll
  for (int ks = 0; ks < kSB; ++ks) load_bt(c0, ks);
  __syncthreads();  // decay cumsums of the first tiles
  __syncthreads();  // x copies of the first tile

  for (int c = c0; c < c1; ++c) {
    const bf16* XF = xbuf + (c & 1) * kXBuf2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float rt = __builtin_amdgcn_exp2f(dbuf[(e * 3 + c % 3) * kDec + kQ - 1]);
#pragma unroll
      for (int j = 0; j < kNBW; ++j)
#pragma unroll
        for (int pb = 0; pb < kPB; ++pb) hacc[e][j][pb] *= rt;
    }
#pragma unroll
    for (int ks = 0; ks < kSB; ++ks) {
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const Frag8<bf16> x0 = lds_frag(XF + foff(ks * kPB + pb, lane));
        const Frag8<bf16> x1 = lds_frag(XF + kXE + foff(ks * kPB + pb, lane));
#pragma unroll
        for (int j = 0; j < kNBW; ++j) {
          hacc[0][j][pb] = mma(bt[j][ks], x0, hacc[0][j][pb]);
          hacc[1][j][pb] = mma(bt[j][ks], x1, hacc[1][j][pb]);
        }
      }
      load_bt(min(c + 1, cl), ks);
    }
    __syncthreads();
  }

#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (e >= nh) break;
    float* hout = k.seg_state + (((int64_t)b * k.heads + h0 + e) * k.nslot + piece) * (kP * kN);
#pragma unroll
    for (int j = 0; j < kNBW; ++j)
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb)
        *reinterpret_cast<f32x4*>(hout + chan(pb, r16) * kN + u * 32 + g * 8 + j * 4) = hacc[e][j][pb];
  }
}

__device__ void stage_waves2(const BK& k, unsigned char* smem, int b, int h0, int nh, int piece,
                             int c0, int c1, int v) {
  const int lane = threadIdx.x & 63;
  bf16* xbuf = reinterpret_cast<bf16*>(smem);
  bf16* stg = xbuf + 2 * kXBuf2 + v * kStgRows * kP;  // this wave's staged rows
  float* dbuf = reinterpret_cast<float*>(smem + kDecOff2);
  const int64_t rowb = (int64_t)b * k.seqlen;
  const int hs[2] = {h0, h0 + nh - 1};
  const float Ah2[2] = {k.A[hs[0]] * kLog2e, k.A[hs[1]] * kLog2e};
  const int pc = lane & 7;
  // rows of both heads: (head 0: r0..r3, head 1: r4..r7), four named
  // registers per head (an array was placed in scratch in the one-head pass)
  struct XSet { uint4 r0, r1, r2, r3; };
  XSet xs0, xs1;
  const uint32_t rowbytes = (uint32_t)(k.xs * (int64_t)sizeof(bf16));
  auto load_x = [&](int c) {
    const int len = (int)min((int64_t)kQ, k.seqlen - (int64_t)c * kQ);
    auto head_rows = [&](int hh, XSet& xs) {
      const uint64_t tile0 = reinterpret_cast<uint64_t>(k.x) +
                             (uint64_t)(((rowb + (int64_t)c * kQ) * k.xs + (int64_t)hh * kP) * sizeof(bf16));
      const auto r = uniform_rsrc(tile0, (uint32_t)len * rowbytes);
      auto row = [&](int i) {
        const int s = v * 32 + i * 8 + (lane >> 3);
        return buffer_load16<kPolicyNT>(r, (uint32_t)s * rowbytes + pc * 16);
      };
      xs.r0 = row(0);
      xs.r1 = row(1);
      xs.r2 = row(2);
      xs.r3 = row(3);
    };
    head_rows(hs[0], xs0);
    head_rows(hs[1], xs1);
  };
  // raw rows out, fragments back, times the tile-end factor, for each head
  // (LDS operations of one wave complete in order: head 1's rows are written
  // after head 0's transposed reads)
  auto commit = [&](int c) {
    auto one = [&](const XSet& xs, int e) {
      bf16* XF = xbuf + (c & 1) * kXBuf2 + e * kXE;
      const float* d = dbuf + (e * 3 + c % 3) * kDec;
      *reinterpret_cast<uint4*>(stg + soff(4 + (lane >> 3), pc)) = xs.r0;
      *reinterpret_cast<uint4*>(stg + soff(12 + (lane >> 3), pc)) = xs.r1;
      *reinterpret_cast<uint4*>(stg + soff(20 + (lane >> 3), pc)) = xs.r2;
      *reinterpret_cast<uint4*>(stg + soff(28 + (lane >> 3), pc)) = xs.r3;
      Frag8<bf16> f[kPB];
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) f[pb] = stg_frag(stg, 4 + (lane >> 4) * 8, pb, lane);
      const float* ef = d + 3 * kQ + v * 32 + (lane >> 4) * 8;
      const f32x4 e0 = *reinterpret_cast<const f32x4*>(ef);
      const f32x4 e1 = *reinterpret_cast<const f32x4*>(ef + 4);
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb)
        *reinterpret_cast<uint4*>(XF + foff(v * kPB + pb, lane)) =
            __builtin_bit_cast(uint4, scale8(f[pb], e0, e1).v);
    };
    one(xs0, 0);
    one(xs1, 1);
  };
  auto load_dt = [&](int c, int hh) -> uint32_t {
    const auto r = uniform_rsrc(k.dtT + (((int64_t)b * k.ntiles + c) * k.heads + hh) * kQ,
                                (uint32_t)(kQ * sizeof(bf16)));
    return buffer_load4<kPolicyDefault>(r, (uint32_t)lane * 4);
  };
  // the one-head pass's decay arrays (Lambda, dt, block-end and tile-end
  // factors), each stage wave writing one, for head e
  auto make_dec = [&](int c, int buf, uint32_t raw, int e) {
    const int len = (int)min((int64_t)kQ, k.seqlen - (int64_t)c * kQ);
    float dtr[2];
    dtr[0] = 2 * lane < len ? __builtin_bit_cast(float, raw << 16) : 0.0f;
    dtr[1] = 2 * lane + 1 < len ? __builtin_bit_cast(float, raw & 0xffff0000u) : 0.0f;
    float* d = dbuf + (e * 3 + buf) * kDec;
    const float v0 = dtr[0] * Ah2[e], v1 = dtr[1] * Ah2[e];
    float incl = v0 + v1;
    incl += dpp_f<0x111, 0xf>(incl);  // row_shr:1
    incl += dpp_f<0x112, 0xf>(incl);  // row_shr:2
    incl += dpp_f<0x114, 0xf>(incl);  // row_shr:4
    incl += dpp_f<0x118, 0xf>(incl);  // row_shr:8
    incl += dpp_f<0x142, 0xa>(incl);  // row_bcast:15 into rows 1 and 3
    incl += dpp_f<0x143, 0xc>(incl);  // row_bcast:31 into rows 2 and 3
    const float l0 = incl - v1, l1 = incl;
    const float lend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
    const float e0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 15));
    const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 31));
    const float e2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 47));
    const int row = lane >> 4;
    const float lblk = row == 0 ? e0 : row == 1 ? e1 : row == 2 ? e2 : lend;
    if (v == 0) {
      *reinterpret_cast<float2*>(d + 2 * lane) = make_float2(l0, l1);
    } else if (v == 1) {
      *reinterpret_cast<float2*>(d + kQ + 2 * lane) = make_float2(dtr[0], dtr[1]);
    } else if (v == 2) {
      *reinterpret_cast<float2*>(d + 2 * kQ + 2 * lane) =
          make_float2(__builtin_amdgcn_exp2f(lblk - l0) * dtr[0], __builtin_amdgcn_exp2f(lblk - l1) * dtr[1]);
    } else {
      *reinterpret_cast<float2*>(d + 3 * kQ + 2 * lane) =
          make_float2(__builtin_amdgcn_exp2f(lend - l0) * dtr[0], __builtin_amdgcn_exp2f(lend - l1) * dtr[1]);
    }
    return lend;
  };

  // the one-head pass's schedule, for two heads
  const int cl = c1 - 1;
  float lam_seg[2] = {0.0f, 0.0f};
  uint32_t dtr_raw[2];
  load_x(c0);
  {
    uint32_t d0[2], d1[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      d0[e] = load_dt(c0, hs[e]);
      d1[e] = load_dt(min(c0 + 1, cl), hs[e]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      lam_seg[e] += make_dec(c0, c0 % 3, d0[e], e);
      if (c0 + 1 < c1) lam_seg[e] += make_dec(c0 + 1, (c0 + 1) % 3, d1[e], e);
    }
  }
  __syncthreads();
  commit(c0);
  load_x(min(c0 + 1, cl));
#pragma unroll
  for (int e = 0; e < 2; ++e) dtr_raw[e] = load_dt(min(c0 + 2, cl), hs[e]);
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) commit(c + 1);
    load_x(min(c + 2, cl));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (c + 2 < c1) lam_seg[e] += make_dec(c + 2, (c + 2) % 3, dtr_raw[e], e);
      dtr_raw[e] = load_dt(min(c + 3, cl), hs[e]);
    }
    __syncthreads();
  }
  if (v == 0 && lane == 0) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (e < nh) k.seg_decay[((int64_t)b * k.heads + hs[e]) * k.nslot + piece] = lam_seg[e];
  }
}

__global__ __launch_bounds__(512) void ssd_bf16_seg2_kernel(BK k) {
  extern __shared__ __align__(16) unsigned char smem[];
  int b, hp;
  const int piece = unit_of_block(k, &b, &hp);  // grid (pieces, head pairs, batch)
  const int h0 = 2 * hp, nh = min(2, k.heads - h0);
  const int seg = piece / k.ppseg;
  const int c0 = seg * k.seg_chunks + (piece % k.ppseg) * k.piece_tiles;
  const int c1 = min(min(c0 + k.piece_tiles, (seg + 1) * k.seg_chunks), k.ntiles);
  if (c0 >= c1) return;  // whole workgroup (the planner makes no empty piece)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= 4)
    state_waves2(k, smem, b, h0, nh, piece, c0, c1, wave - 4);
  else
    stage_waves2(k, smem, b, h0, nh, piece, c0, c1, wave);
}

// Chains the pieces' states: slot i receives the state entering piece i,
//   H_in[0] = h0, H_in[i+1] = exp2(decay_i) H_in[i] + S_i,
// where slot i held the piece's own end state S_i from the state-only pass.
// One thread per state element; the loads of eight slots are issued together
// before their part of the chain.
constexpr int kCombineRegs = 8;
__global__ __launch_bounds__(256) void seg_combine_bf16_kernel(float* __restrict__ seg_state,
                                                               const float* __restrict__ seg_decay,
                                                               const float* __restrict__ h0,
                                                               int n_heads, int heads, int nslot,
                                                               UnitMap um) {
  constexpr int PN = kP * kN;
  const int e = blockIdx.x * 256 + threadIdx.x;
  int h = blockIdx.y, b = blockIdx.z;
  if (um.mixed) unit_to_bh(um, blockIdx.y, &b, &h);
  const int64_t unit = (int64_t)b * heads + h;
  float H = h0 ? h0[((int64_t)b * n_heads + h) * PN + e] : 0.0f;
  float* base = seg_state + unit * nslot * PN + e;
  const float* dec = seg_decay + unit * nslot;
  const int npre = nslot - 1;
  for (int s0 = 0; s0 < npre; s0 += kCombineRegs) {
    float S[kCombineRegs];
#pragma unroll
    for (int i = 0; i < kCombineRegs; ++i)  // (slot index clamped: every load valid)
      S[i] = base[(int64_t)min(s0 + i, npre - 1) * PN];
#pragma unroll
    for (int i = 0; i < kCombineRegs; ++i) {
      const int sg = s0 + i;
      if (sg < npre) {
        base[(int64_t)sg * PN] = H;
        H = exp2f(dec[sg]) * H + S[i];
      }
    }
  }
  base[(int64_t)npre * PN] = H;
}

size_t frag_region_bytes(int64_t batch, int64_t seqlen) {
  const int64_t nt = (seqlen + kQ - 1) / kQ;
  const size_t bytes = (size_t)(batch * nt) * kNFR * kFragBytes;
  return (bytes + 255) & ~(size_t)255;
}
size_t dt_region_bytes(int64_t batch, int64_t seqlen, int64_t heads) {
  const int64_t nt = (seqlen + kQ - 1) / kQ;
  const size_t bytes = (size_t)(batch * nt * heads) * kQ * sizeof(bf16);
  return (bytes + 255) & ~(size_t)255;
}

}  // namespace

bool bf16_path(int64_t d_head, int64_t d_state, int64_t chunk, int dtype) {
  return dtype == MM_BF16 && d_head == kP && d_state == kN && (chunk == 128 || chunk == 256);
}

Bf16Plan plan_bf16(int64_t batch, int64_t seqlen, int64_t heads, int64_t units_in,
                   bool allow_pairs) {
  // Cost in units of one tile step of a main workgroup (about 2.5 us on
  // MI355X).  Each round of up to kCus main workgroups costs its walk plus
  // ~2.5 tiles of start-up (first loads from HBM, state in, pipeline fill and
  // drain).  A split adds the state-only pass, whose workgroups walk a piece
  // at ~0.6 of a main tile step per tile plus ~2.5 of start-up (one per CU:
  // two sharing a CU measured slower per CU than one), and the combine and
  // its launch (~3, plus ~0.3 per piece: each piece's state is written and
  // read back once more; traces put the combine alone at 5-9 us).  Pieces finer than the segments pay where the
  // segments alone leave CUs idle in the state-only pass.  Two heads per
  // state-only workgroup (pairs: the B^T fragments are read once for the
  // two) take ~1.0 of a main tile step per tile for both (measured at long
  // context: 0.6 for one head), in half as many workgroups: they pay where
  // the pieces can be made fine enough to fill the CUs.
  constexpr int64_t kCus = 256, kSegPerCu = 1, kMaxPieces = 16;
  Bf16Plan pl;
  const int64_t n = (seqlen + kQ - 1) / kQ;
  const int64_t units = units_in > 0 ? units_in : batch * heads;
  pl.ntiles = (int)n;
  pl.nseg = 1;
  pl.seg_tiles = (int)(n > 0 ? n : 1);
  pl.ppseg = 1;
  pl.piece_tiles = pl.seg_tiles;
  double best = 1e300;
  for (int64_t want = 1; want <= n; ++want) {
    const int64_t per = (n + want - 1) / want;
    const int64_t seg = (n + per - 1) / per;
    if (seg != want) continue;  // the same cut as a smaller count
    const int64_t r_main = (units * seg + kCus - 1) / kCus;
    const double main_cost = (double)r_main * ((double)per + 2.5);
    if (seg == 1) {
      if (main_cost < best) {
        best = main_cost;
        pl.nseg = 1; pl.seg_tiles = (int)per; pl.ppseg = 1; pl.piece_tiles = (int)per;
      }
      continue;
    }
    for (int64_t pp = 1; pp <= kMaxPieces && pp <= per; ++pp) {
      const int64_t pt = (per + pp - 1) / pp;
      if ((pp - 1) * pt >= per) continue;  // an empty piece
      const int64_t npre = (seg - 1) * pp;
      for (int pr = 0; pr < (allow_pairs ? 2 : 1); ++pr) {
        if (!pr && pp > 8) continue;  // one head per workgroup: at most 8 pieces
        const int64_t pu = pr ? batch * ((heads + 1) / 2) : units;  // state-only workgroups per piece
        const int64_t r_pre = (pu * npre + kCus * kSegPerCu - 1) / (kCus * kSegPerCu);
        const double cost = main_cost + (double)r_pre * ((pr ? 1.0 : 0.6) * (double)pt + 2.5) + 3.0 +
                            0.3 * (double)npre;
        if (cost < best) {
          best = cost;
          pl.nseg = (int)seg; pl.seg_tiles = (int)per; pl.ppseg = (int)pp; pl.piece_tiles = (int)pt;
          pl.pairs = pr != 0;
        }
      }
    }
  }
  return pl;
}

void fwd_plan_bf16(int64_t batch, int64_t seqlen, int64_t heads, int* ntiles, int* nseg,
                   int* seg_tiles, int64_t units_in, bool allow_pairs) {
  const Bf16Plan pl = plan_bf16(batch, seqlen, heads, units_in, allow_pairs);
  *ntiles = pl.ntiles;
  *seg_tiles = pl.seg_tiles;
  *nseg = pl.nseg;
}

size_t bf16_workspace_bytes(int64_t batch, int64_t seqlen, int64_t heads, int64_t units,
                            bool allow_pairs) {
  const Bf16Plan pl = plan_bf16(batch, seqlen, heads, units, allow_pairs);
  size_t bytes = frag_region_bytes(batch, seqlen) + dt_region_bytes(batch, seqlen, heads);
  if (pl.nseg > 1) bytes += (size_t)(batch * heads * pl.nslot()) * (size_t)(kP * kN + 1) * sizeof(float);
  return bytes;
}

// hipFuncSetAttribute for the kernels that need more than 64 KB of LDS,
// once per device (bit d of the mask).
hipError_t set_lds_attributes() {
  static std::atomic<unsigned long long> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load() & bit)) return hipSuccess;
  const std::pair<const void*, size_t> attrs[] = {
      {reinterpret_cast<const void*>(tile_prep_kernel<false>), kPrepLds},
      {reinterpret_cast<const void*>(tile_prep_kernel<true>), kPrepLds},
      {reinterpret_cast<const void*>(ssd_bf16_kernel<false>), kLds},
      {reinterpret_cast<const void*>(ssd_bf16_kernel<true>), kLds},
      {reinterpret_cast<const void*>(ssd_bf16_seg_kernel<false>), kLdsSeg},
      {reinterpret_cast<const void*>(ssd_bf16_seg_kernel<true>), kLdsSeg},
      {reinterpret_cast<const void*>(ssd_bf16_seg2_kernel), kLdsSeg2}};
  for (const auto& fa : attrs) {
    e = hipFuncSetAttribute(fa.first, hipFuncAttributeMaxDynamicSharedMemorySize, (int)fa.second);
    if (e != hipSuccess) return e;
  }
  done.fetch_or(bit);
  return hipSuccess;
}

template <bool FUSED>
hipError_t launch_bf16(const FwdArgs& a, const FuseArgs& fu, void* ws, hipStream_t s) {
  BK k;
  k.x = static_cast<const bf16*>(a.x); k.xs = a.xs;
  k.dt = static_cast<const bf16*>(a.dt); k.dts = a.dts;
  k.A = a.A;
  k.C = static_cast<const bf16*>(a.C); k.cs = a.cs;
  k.D = a.D;
  k.y = static_cast<bf16*>(a.y); k.ys = a.ys;
  k.h0 = a.h0; k.hT = a.hT;
  k.cw = fu.w; k.cbias = fu.bias; k.cstate = fu.state; k.conv_dim = fu.conv_dim;
  k.seqlen = a.seqlen; k.n_heads = a.n_heads; k.heads = a.heads;
  k.um = make_unit_map(a);
  const Bf16Plan pl = plan_bf16(a.batch, a.seqlen, a.plan_heads > 0 ? a.plan_heads : a.heads,
                                k.um.mixed ? k.um.units : 0,
                                !FUSED && !k.um.mixed);
  k.ntiles = pl.ntiles;
  k.nseg = pl.nseg;
  k.seg_chunks = pl.seg_tiles;
  k.ppseg = pl.ppseg;
  k.piece_tiles = pl.piece_tiles;
  k.nslot = pl.nslot();
  if (k.um.mixed && k.um.units == 0) return hipSuccess;  // no active head anywhere
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  uint4* frags = reinterpret_cast<uint4*>(wsb);
  bf16* dtT = reinterpret_cast<bf16*>(wsb + frag_region_bytes(a.batch, a.seqlen));
  k.frags = frags;
  k.dtT = dtT;
  k.seg_state = nullptr;
  k.seg_decay = nullptr;
  if (k.nseg > 1) {
    k.seg_state = reinterpret_cast<float*>(wsb + frag_region_bytes(a.batch, a.seqlen) +
                                           dt_region_bytes(a.batch, a.seqlen, a.heads));
    k.seg_decay = k.seg_state + (size_t)a.batch * a.heads * k.nslot * kP * kN;
  }
  hipError_t e = set_lds_attributes();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tile_prep_kernel<FUSED>, dim3(k.ntiles, (unsigned)a.batch), dim3(512),
                     kPrepLds, s, static_cast<const bf16*>(a.B), a.bs, k.C, a.cs, k.dt, a.dts,
                     frags, dtT, a.seqlen, k.ntiles, a.heads, fu);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (k.nseg > 1) {
    const int npre = k.nslot - 1;
    if (pl.pairs) {
      // two heads per workgroup, sharing the B^T fragments
      hipLaunchKernelGGL(ssd_bf16_seg2_kernel, dim3(npre, (unsigned)((a.heads + 1) / 2), (unsigned)a.batch),
                         dim3(512), kLdsSeg2, s, k);
    } else {
      auto pre = ssd_bf16_seg_kernel<FUSED>;
      const dim3 gpre = k.um.mixed ? dim3((unsigned)(npre * k.um.units))
                                   : dim3(npre, a.heads, (unsigned)a.batch);
      hipLaunchKernelGGL(pre, gpre, dim3(512), kLdsSeg, s, k);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    static_assert((kP * kN) % 256 == 0, "state elements split over 256-thread blocks");
    const dim3 gcomb = k.um.mixed ? dim3(kP * kN / 256, (unsigned)k.um.units)
                                  : dim3(kP * kN / 256, a.heads, (unsigned)a.batch);
    hipLaunchKernelGGL(seg_combine_bf16_kernel, gcomb, dim3(256), 0, s, k.seg_state, k.seg_decay,
                       a.h0, a.n_heads, a.heads, k.nslot, k.um);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto main_k = ssd_bf16_kernel<FUSED>;
  const dim3 gmain = k.um.mixed ? dim3((unsigned)(k.nseg * k.um.units))
                                : dim3(k.nseg, a.heads, (unsigned)a.batch);
  hipLaunchKernelGGL(main_k, gmain, dim3(kThreads), kLds, s, k);
  return hipGetLastError();
}

hipError_t launch_ssd_forward_bf16(const FwdArgs& a, void* ws, hipStream_t s) {
  return launch_bf16<false>(a, FuseArgs{}, ws, s);
}

hipError_t launch_ssd_forward_bf16_fused(const FwdArgs& a, const FuseArgs& fu, void* ws,
                                         hipStream_t s) {
  return launch_bf16<true>(a, fu, ws, s);
}

}  // namespace mmssd
