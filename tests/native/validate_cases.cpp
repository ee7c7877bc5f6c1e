// Host-only checks of the C ABI's argument validation, built with g++ and
// AddressSanitizer/UBSan by tests/test_abi_cpu.py (no HIP, no GPU).  Every
// case states the status code include/mm_ssd.h documents for it.
#include <cstdint>
#include <cstdio>

#include "../../selective_state_space_12_amd/csrc/validate.h"

using namespace mmssd;

static int failures = 0;

static void expect(const char* name, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d\n", name, got, want);
    ++failures;
  } else {
    std::printf("ok   %s\n", name);
  }
}

int main() {
  // fake, 16-byte aligned addresses: validation never dereferences them
  const void* P = reinterpret_cast<const void*>(uintptr_t(0x100000));
  const void* P2 = reinterpret_cast<const void*>(uintptr_t(0x1000000000ull));
  const float* F = reinterpret_cast<const float*>(uintptr_t(0x200000));
  const void* MIS = reinterpret_cast<const void*>(uintptr_t(0x100008));
  int64_t h = 0;

  // slice resolution (nesting / Mix'n'Match rule)
  expect("heads ok", validate_heads_for_dim(2048, 4096, 64, 256, &h), MM_OK);
  expect("heads null", validate_heads_for_dim(2048, 4096, 64, 256, nullptr), MM_ERR_NULL);
  expect("heads m=0", validate_heads_for_dim(2048, 4096, 64, 0, &h), MM_ERR_SLICE);
  expect("heads m>d", validate_heads_for_dim(2048, 4096, 64, 2049, &h), MM_ERR_SLICE);
  expect("heads non-integer", validate_heads_for_dim(2048, 4096, 64, 100, &h), MM_ERR_SLICE);
  expect("heads e not integer", validate_heads_for_dim(3, 4, 2, 1, &h), MM_ERR_SHAPE);
  expect("heads d_head<=0", validate_heads_for_dim(2048, 4096, 0, 256, &h), MM_ERR_SHAPE);

  // conv: 4096 + 256 channels, bf16
  const int64_t cd = 4352;
  expect("conv ok", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_OK);
  expect("conv null in", validate_conv(nullptr, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_NULL);
  expect("conv null w", validate_conv(P, cd, P2, cd, nullptr, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_NULL);
  expect("conv dtype", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, 9), MM_ERR_DTYPE);
  expect("conv heads 0", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 0, MM_BF16), MM_ERR_SLICE);
  expect("conv heads > n", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 65, MM_BF16), MM_ERR_SLICE);
  expect("conv stride short", validate_conv(P, cd - 8, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_SHAPE);
  expect("conv misaligned", validate_conv(MIS, cd, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_ALIGN);
  expect("conv stride misaligned", validate_conv(P, cd + 1, P2, cd, F, nullptr, nullptr, 4, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_ALIGN);
  expect("conv overlap", validate_conv(P, cd, P, cd, F, nullptr, nullptr, 1, 2, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_SHAPE);
  expect("conv d_head%8", validate_conv(P, 40, P2, 40, F, nullptr, nullptr, 1, 2, 12, 4, 8, 1, 1, MM_F32), MM_ERR_UNSUPPORTED);
  expect("conv batch 0", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 0, 8192, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_SHAPE);
  expect("conv batch > grid", validate_conv(P, cd, P2, cd, F, nullptr, nullptr, 70000, 1, 4096, 64, 128, 1, 64, MM_BF16), MM_ERR_SHAPE);

  // scan forward: x/y rows 4096 wide, B/C 128 wide, dt 64 wide
  auto fwd = [&](const void* x, int64_t xs, const void* dt, int64_t dts, const float* A,
                 const void* B, int64_t bs, const void* C, int64_t cs, const void* y, int64_t ys,
                 int64_t batch, int64_t seqlen, int64_t nh, int64_t P_, int64_t N_, int64_t G,
                 int64_t ha, int64_t q, int dt_code) {
    return validate_ssd_forward(x, xs, dt, dts, A, B, bs, C, cs, y, ys, nullptr, nullptr, batch,
                                seqlen, nh, P_, N_, G, ha, q, dt_code);
  };
  expect("fwd ok", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_OK);
  expect("fwd ok strided", fwd(P, 4352, P, 64, F, P, 4352, P, 4352, P2, 4096, 4, 8192, 64, 64, 128, 1, 8, 256, MM_BF16), MM_OK);
  expect("fwd null A", fwd(P, 4096, P, 64, nullptr, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_NULL);
  expect("fwd dtype", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, 2), MM_ERR_DTYPE);
  expect("fwd heads 0", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 0, 256, MM_BF16), MM_ERR_SLICE);
  expect("fwd heads > n", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 65, 256, MM_BF16), MM_ERR_SLICE);
  expect("fwd ngroups 2", fwd(P, 4096, P, 64, F, P, 256, P, 256, P2, 4096, 4, 8192, 64, 64, 128, 2, 64, 256, MM_BF16), MM_ERR_UNSUPPORTED);
  expect("fwd chunk 48", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 48, MM_BF16), MM_ERR_UNSUPPORTED);
  expect("fwd shape (48,128)", fwd(P, 3072, P, 64, F, P, 128, P, 128, P2, 3072, 4, 8192, 64, 48, 128, 1, 64, 256, MM_BF16), MM_ERR_UNSUPPORTED);
  expect("fwd fp32 chunk 256 N=128", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_F32), MM_ERR_UNSUPPORTED);
  expect("fwd x stride short", fwd(P, 4088, P, 64, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fwd dt stride short", fwd(P, 4096, P, 63, F, P, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fwd B misaligned", fwd(P, 4096, P, 64, F, MIS, 128, P, 128, P2, 4096, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_ALIGN);
  expect("fwd y stride misaligned", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4100, 4, 8192, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_ALIGN);
  expect("fwd seqlen 0", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, 4, 0, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fwd huge", fwd(P, 4096, P, 64, F, P, 128, P, 128, P2, 4096, int64_t(1) << 40, 1 << 20, 64, 64, 128, 1, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fwd shape only ok", validate_ssd_shape(1, 256, 4, 32, 16, 1, 4, 64, MM_F32), MM_OK);

  // decode step
  auto step = [&](const float* st, int64_t batch, int64_t nh, int64_t P_, int64_t N_, int64_t G,
                  int64_t ha, int dt_code, const void* B) {
    return validate_ssd_step(st, P, nh * P_, P, nh, F, B, G * N_, P, G * N_, P2, nh * P_, batch, nh,
                             P_, N_, G, ha, dt_code);
  };
  expect("step ok", step(F, 256, 64, 64, 128, 1, 64, MM_F32, P), MM_OK);
  expect("step null state", step(nullptr, 256, 64, 64, 128, 1, 64, MM_F32, P), MM_ERR_NULL);
  expect("step heads 0", step(F, 256, 64, 64, 128, 1, 0, MM_F32, P), MM_ERR_SLICE);
  expect("step N=96", step(F, 256, 64, 64, 96, 1, 64, MM_F32, P), MM_ERR_UNSUPPORTED);
  expect("step ngroups 2", step(F, 256, 64, 64, 128, 2, 64, MM_F32, P), MM_ERR_UNSUPPORTED);
  expect("step B misaligned", step(F, 256, 64, 64, 128, 1, 64, MM_F32, MIS), MM_ERR_ALIGN);
  expect("step dtype", step(F, 256, 64, 64, 128, 1, 64, 5, P), MM_ERR_DTYPE);

  // fused prefill call: raw xBC rows (4352 channels) at P, y at P2
  auto fused = [&](const void* xbc, int64_t xs, const float* cw, const float* cst, int sp,
                   const void* y, int64_t heads, int64_t chunk, int dt_code) {
    return validate_ssd_forward_fused(xbc, xs, cw, nullptr, cst, P, 64, nullptr, sp, F, y, 4096,
                                      nullptr, nullptr, 4, 8192, 64, 64, 128, 1, heads, chunk,
                                      dt_code);
  };
  const float* FMIS = reinterpret_cast<const float*>(uintptr_t(0x200004));
  expect("fused ok", fused(P, cd, F, F, 1, P2, 64, 256, MM_BF16), MM_OK);
  expect("fused null conv w", fused(P, cd, nullptr, F, 1, P2, 64, 256, MM_BF16), MM_ERR_NULL);
  expect("fused stride < conv_dim", fused(P, cd - 8, F, F, 1, P2, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fused softplus flag 2", fused(P, cd, F, F, 2, P2, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fused conv w misaligned", fused(P, cd, FMIS, F, 1, P2, 64, 256, MM_BF16), MM_ERR_ALIGN);
  expect("fused y over xbc", fused(P, cd, F, F, 1, P, 64, 256, MM_BF16), MM_ERR_SHAPE);
  expect("fused heads 0", fused(P, cd, F, F, 1, P2, 0, 256, MM_BF16), MM_ERR_SLICE);
  expect("fused chunk 48", fused(P, cd, F, F, 1, P2, 64, 48, MM_BF16), MM_ERR_UNSUPPORTED);

  // gated RMSNorm: 32768 rows of 4096, y at P, z at P2, out at P3
  const void* P3 = reinterpret_cast<const void*>(uintptr_t(0x4000000000ull));
  auto norm = [&](const void* y, const void* z, const void* o, int64_t os, const float* w, float eps,
                  int64_t d, int dt_code) {
    return validate_gated_rmsnorm(y, 4096, z, 4096, w, eps, o, os, 32768, d, dt_code);
  };
  expect("norm ok", norm(P, P2, P3, 4096, F, 1e-5f, 4096, MM_BF16), MM_OK);
  expect("norm in place", norm(P, P2, P, 4096, F, 1e-5f, 4096, MM_BF16), MM_OK);
  expect("norm out over y, other stride", norm(P, P2, P, 4104, F, 1e-5f, 4096, MM_BF16), MM_ERR_SHAPE);
  expect("norm out over z", norm(P, P2, P2, 4096, F, 1e-5f, 4096, MM_BF16), MM_ERR_SHAPE);
  expect("norm d % 8", norm(P, P2, P3, 4096, F, 1e-5f, 4092, MM_BF16), MM_ERR_UNSUPPORTED);
  expect("norm eps < 0", norm(P, P2, P3, 4096, F, -1.0f, 4096, MM_BF16), MM_ERR_SHAPE);
  expect("norm w misaligned", norm(P, P2, P3, 4096, FMIS, 1e-5f, 4096, MM_BF16), MM_ERR_ALIGN);
  expect("norm null z", norm(P, nullptr, P3, 4096, F, 1e-5f, 4096, MM_BF16), MM_ERR_NULL);
  expect("norm dtype", norm(P, P2, P3, 4096, F, 1e-5f, 4096, 9), MM_ERR_DTYPE);

  // per-sequence widths of a mixed scan call
  {
    int64_t mx = 0;
    const int32_t ok4[4] = {16, 64, 32, 64}, zero[2] = {0, 3}, wide[2] = {3, 65};
    expect("mixed ok", validate_heads_per_seq(ok4, 4, 64, &mx), MM_OK);
    expect("mixed widest", (int)mx, 64);
    expect("mixed null", validate_heads_per_seq(nullptr, 4, 64, &mx), MM_ERR_NULL);
    expect("mixed 0 heads", validate_heads_per_seq(zero, 2, 64, &mx), MM_ERR_SLICE);
    expect("mixed > n_heads", validate_heads_per_seq(wide, 2, 64, &mx), MM_ERR_SLICE);
    expect("mixed batch 257", validate_heads_per_seq(ok4, 257, 64, &mx), MM_ERR_UNSUPPORTED);
  }

  // multi-token decode step: 256 sequences x 4 tokens, 64 heads x 64 x 128
  {
    float* S2 = reinterpret_cast<float*>(uintptr_t(0x8000000000ull));
    auto multi = [&](const float* out, int64_t ntok, int64_t P_, int64_t N_) {
      return validate_ssd_step_multi(F, out, P, 64 * P_, P, 64, F, P, N_, P, N_, P2, 64 * P_, 256,
                                     ntok, 64, P_, N_, 1, 64, MM_F32);
    };
    expect("multi ok", multi(nullptr, 4, 64, 128), MM_OK);
    expect("multi in place", multi(F, 4, 64, 128), MM_OK);
    expect("multi separate out", multi(S2, 4, 64, 128), MM_OK);
    expect("multi out overlaps in", multi(F + 4, 4, 64, 128), MM_ERR_SHAPE);
    expect("multi ntok 0", multi(nullptr, 0, 64, 128), MM_ERR_SHAPE);
    expect("multi ntok 65", multi(nullptr, 65, 64, 128), MM_ERR_SHAPE);
    expect("multi state too big for a pass", multi(nullptr, 4, 128, 128), MM_ERR_UNSUPPORTED);
    expect("conv advance ok",
           validate_conv_state_advance(F, P, cd, 256, 4, 4096, 64, 128, 1, 64, MM_F32), MM_OK);
    expect("conv advance stride",
           validate_conv_state_advance(F, P, cd - 4, 256, 4, 4096, 64, 128, 1, 64, MM_F32),
           MM_ERR_SHAPE);
    expect("conv advance heads",
           validate_conv_state_advance(F, P, cd, 256, 4, 4096, 64, 128, 1, 65, MM_F32),
           MM_ERR_SLICE);
    expect("conv advance null",
           validate_conv_state_advance(nullptr, P, cd, 256, 4, 4096, 64, 128, 1, 64, MM_F32),
           MM_ERR_NULL);
  }

  // scan backward: 4 x 8192 tokens, 64 heads x 64 x 128, bf16; every output
  // in a region of its own (inputs may share theirs)
  {
    auto at = [](uint64_t a) { return reinterpret_cast<float*>(uintptr_t(a)); };
    float *dx = at(0x1000000000ull), *ddt = at(0x2000000000ull), *dB = at(0x3000000000ull),
          *dC = at(0x4000000000ull), *dA = at(0x5000000000ull), *dD = at(0x6000000000ull),
          *dh0 = at(0x7000000000ull);
    auto bwd = [&](const void* dy, const void* dx_, float* dB_, float* dC_, int64_t dxs,
                   int64_t P_, int64_t N_, int64_t ha, int dt_code, int acc) {
      return validate_ssd_backward(P, 64 * P_, P, 64, F, P, N_, P, N_, F, nullptr, dy, 64 * P_,
                                   nullptr, dx_, dxs, ddt, 64, dA, dB_, N_, dC_, N_, dD, dh0, 4,
                                   8192, 64, P_, N_, 1, ha, dt_code, acc);
    };
    expect("bwd ok", bwd(P, dx, dB, dC, 4096, 64, 128, 64, MM_BF16, 0), MM_OK);
    expect("bwd ok accumulate", bwd(P, dx, dB, dC, 4096, 64, 128, 8, MM_BF16, 1), MM_OK);
    expect("bwd ok d_state 64", bwd(P, dx, dB, dC, 4096, 64, 64, 64, MM_BF16, 0), MM_OK);
    expect("bwd null dy", bwd(nullptr, dx, dB, dC, 4096, 64, 128, 64, MM_BF16, 0), MM_ERR_NULL);
    expect("bwd fp32 d_head 64", bwd(P, dx, dB, dC, 4096, 64, 128, 64, MM_F32, 0),
           MM_ERR_UNSUPPORTED);
    expect("bwd bf16 d_head 32", bwd(P, dx, dB, dC, 2048, 32, 16, 64, MM_BF16, 0),
           MM_ERR_UNSUPPORTED);
    expect("bwd dx over x", bwd(P, P, dB, dC, 4096, 64, 128, 64, MM_BF16, 0), MM_ERR_SHAPE);
    expect("bwd dB over dC", bwd(P, dx, dB, dB + 64, 4096, 64, 128, 64, MM_BF16, 0),
           MM_ERR_SHAPE);
    expect("bwd accumulate 2", bwd(P, dx, dB, dC, 4096, 64, 128, 64, MM_BF16, 2), MM_ERR_SHAPE);
    expect("bwd dx stride short", bwd(P, dx, dB, dC, 4088, 64, 128, 64, MM_BF16, 0),
           MM_ERR_SHAPE);
    expect("bwd dB misaligned", bwd(P, dx, at(0x3000000002ull), dC, 4096, 64, 128, 64, MM_BF16, 0),
           MM_ERR_ALIGN);
    expect("bwd heads 0", bwd(P, dx, dB, dC, 4096, 64, 128, 0, MM_BF16, 0), MM_ERR_SLICE);
    expect("bwd shape query ok", validate_ssd_backward_shape(4, 8192, 64, 64, 128, 1, 64, MM_BF16),
           MM_OK);
    expect("bwd shape query fp32 64x64",
           validate_ssd_backward_shape(4, 8192, 64, 64, 64, 1, 64, MM_F32), MM_ERR_UNSUPPORTED);
  }

  // conv backward: 4 x 8192 rows of 4352 channels, bf16
  {
    const void* D1 = reinterpret_cast<const void*>(uintptr_t(0x2000000000ull));
    void* G1 = reinterpret_cast<void*>(uintptr_t(0x3000000000ull));
    float* DW = reinterpret_cast<float*>(uintptr_t(0x4000000000ull));
    float* DS = reinterpret_cast<float*>(uintptr_t(0x5000000000ull));
    auto cb = [&](const void* dout, void* din, float* dw, int64_t ds, int acc) {
      return validate_conv_backward(P, cd, dout, ds, din, cd, F, nullptr, nullptr, dw, nullptr, DS,
                                    4, 8192, 4096, 64, 128, 1, 64, MM_BF16, acc);
    };
    expect("conv bwd ok", cb(D1, G1, DW, cd, 0), MM_OK);
    expect("conv bwd accumulate", cb(D1, G1, DW, cd, 1), MM_OK);
    expect("conv bwd null dout", cb(nullptr, G1, DW, cd, 0), MM_ERR_NULL);
    expect("conv bwd null dw", cb(D1, G1, nullptr, cd, 0), MM_ERR_NULL);
    expect("conv bwd din over dout", cb(D1, const_cast<void*>(D1), DW, cd, 0), MM_ERR_SHAPE);
    expect("conv bwd din over input", cb(D1, const_cast<void*>(P), DW, cd, 0), MM_ERR_SHAPE);
    expect("conv bwd dout stride short", cb(D1, G1, DW, cd - 8, 0), MM_ERR_SHAPE);
    expect("conv bwd accumulate 2", cb(D1, G1, DW, cd, 2), MM_ERR_SHAPE);
    expect("conv bwd dw misaligned", cb(D1, G1, reinterpret_cast<float*>(uintptr_t(0x4000000002ull)),
                                        cd, 0), MM_ERR_ALIGN);
    expect("conv bwd dw over dstate", cb(D1, G1, DS, cd, 0), MM_ERR_SHAPE);
  }

  // fused decode step: 256 sequences, 64 heads x 64 x 128, raw rows of 4352
  // channels at P; state at F, conv states at CI / CO, y at P2
  {
    const float* CI = reinterpret_cast<const float*>(uintptr_t(0x6000000000ull));
    const float* CO = reinterpret_cast<const float*>(uintptr_t(0x7000000000ull));
    auto sf = [&](const float* st, const float* ci, const float* co, const float* w, int64_t xs,
                  int64_t P_, int64_t N_, int64_t ha, int dt_code) {
      return validate_ssd_step_fused(st, ci, co, P, xs, w, nullptr, P, 64, F, P2, 64 * P_, 256, 64,
                                     P_, N_, 1, ha, dt_code);
    };
    expect("step fused ok", sf(F, CI, CO, F, cd, 64, 128, 64, MM_BF16), MM_OK);
    expect("step fused null conv out", sf(F, CI, nullptr, F, cd, 64, 128, 64, MM_BF16), MM_ERR_NULL);
    expect("step fused null conv w", sf(F, CI, CO, nullptr, cd, 64, 128, 64, MM_BF16), MM_ERR_NULL);
    expect("step fused in place", sf(F, CI, CI, F, cd, 64, 128, 64, MM_BF16), MM_ERR_SHAPE);
    expect("step fused out over state", sf(CO, CI, CO, F, cd, 64, 128, 64, MM_BF16), MM_ERR_SHAPE);
    expect("step fused out overlaps in",
           sf(F, CI, reinterpret_cast<const float*>(uintptr_t(0x6000000100ull)), F, cd, 64, 128, 64,
              MM_BF16), MM_ERR_SHAPE);
    expect("step fused stride < conv_dim", sf(F, CI, CO, F, cd - 8, 64, 128, 64, MM_BF16), MM_ERR_SHAPE);
    expect("step fused d_head 60", sf(F, CI, CO, F, cd, 60, 128, 64, MM_BF16), MM_ERR_UNSUPPORTED);
    expect("step fused N=96", sf(F, CI, CO, F, cd, 64, 96, 64, MM_BF16), MM_ERR_UNSUPPORTED);
    expect("step fused d_head 512 N=256", sf(F, CI, CO, F, 512 * 64 + 512, 512, 256, 64, MM_BF16),
           MM_ERR_UNSUPPORTED);
    expect("step fused heads 0", sf(F, CI, CO, F, cd, 64, 128, 0, MM_BF16), MM_ERR_SLICE);
    expect("step fused conv in misaligned",
           sf(F, reinterpret_cast<const float*>(uintptr_t(0x6000000004ull)), CO, F, cd, 64, 128, 64,
              MM_BF16), MM_ERR_ALIGN);
    expect("step fused dtype", sf(F, CI, CO, F, cd, 64, 128, 64, 3), MM_ERR_DTYPE);
  }

  std::printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
