// Drives the host code of libsvdq (C ABI and packer) under AddressSanitizer and
// UndefinedBehaviorSanitizer, against the fake runtime in fake_runtime.cpp.
// Every buffer is a heap allocation of exactly the size the header states, so
// a read or write past it is reported.  Modes:
//   full           gfx950 device: argument checks, workspace and overlap rules,
//                  launches reaching the (fake) launchers, the packers
//   arch-mismatch  the device reports another architecture (FAKE_GFX_ARCH):
//                  every device call returns ARCH_MISMATCH, nothing launches
//   no-device      no device (FAKE_DEVICE_COUNT=0): NO_DEVICE
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "svdq.h"
#include "fake_runtime.h"

static int g_failures = 0;
#define CHECK(cond)                                                                   \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      std::fprintf(stderr, "%s:%d: CHECK failed: %s (last error: %s)\n", __FILE__,    \
                   __LINE__, #cond, svdq_last_error());                               \
      ++g_failures;                                                                   \
    }                                                                                 \
  } while (0)

// exact-size, 16-byte aligned heap buffer
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t n) { p = std::aligned_alloc(16, (n + 15) / 16 * 16 == n ? n : (n + 15) / 16 * 16); }
  ~Buf() { std::free(p); }
  template <class T> T* as() const { return static_cast<T*>(p); }
};

static uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

static void run_calls(svdq_status want) {
  const int64_t M = 100, K = 256, N = 256, r = 16;
  Buf x(M * K * 2), lam(K * 4), down(r * K * 2), codes(M * K / 2), scales(M * K / 64 * 2), la(M * r * 2);
  Buf wc(N * K / 2), ws(N * K / 64 * 2), up(N * r * 2), bias(N * 2), y(M * N * 2), wsp(1 << 16);
  g_fake.quant_need = 0;
  g_fake.gemm_need = 0;
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, codes.p, scales.p, la.p,
                                    nullptr, 0, nullptr) == want);
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, wc.p, ws.p, la.p, up.p, bias.p, M, N, K, r, 64, y.p,
                               nullptr, 0, nullptr) == want);
  CHECK(svdq_fp4_gemm_lora_up(codes.p, scales.p, wc.p, ws.p, la.p, up.p, bias.p, M, N, K, r, 0, y.p,
                              nullptr, 0, nullptr) == want);
  CHECK(svdq_awq_w4a16_gemm(x.p, lam.as<float>(), wc.p, ws.p, scales.p, bias.p, 1, N, K, 64, y.p, nullptr) == want);
  Buf acc(5 * 3 * (K / 64) * 4);
  CHECK(svdq_w4a4_group_acc_debug(codes.p, wc.p, M, N, K, 37, 5, 70, 3, acc.as<int32_t>(), nullptr) == want);
  if (want == SVDQ_STATUS_SUCCESS) {
    CHECK(std::string(g_fake.last) == "dump" && g_fake.last_out == acc.p);
    // rows [37, 42) launched from the 16-row block at 32 (storage order of the
    // codes), as rows [0, 10) with the window [5, 10); columns [64, 128)
    // launched, window [6, 9)
    CHECK(g_fake.last_window[0] == 5 && g_fake.last_window[1] == 10);
    CHECK(g_fake.last_window[2] == 6 && g_fake.last_window[3] == 9);
  }
}

static void full_mode() {
  CHECK(svdq_check_device(0) == SVDQ_STATUS_SUCCESS);
  CHECK(svdq_check_device(-1) == SVDQ_STATUS_INVALID_VALUE);
  g_fake.launches = 0;
  run_calls(SVDQ_STATUS_SUCCESS);
  CHECK(g_fake.launches == 5);

  const int64_t M = 64, K = 256, N = 128, r = 16;
  Buf x(M * K * 2), lam(K * 4), down(r * K * 2), codes(M * K / 2), scales(M * K / 64 * 2), la(M * r * 2);
  Buf wc(N * K / 2), wsc(N * K / 64 * 2), up(N * r * 2), bias(N * 2), y(M * N * 2);
  // workspace: required when the planner asks for one, passed through unchanged
  g_fake.quant_need = 4096;
  g_fake.gemm_need = 8192;
  Buf work(8192);
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, codes.p, scales.p, la.p,
                                    nullptr, 0, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(std::strstr(svdq_last_error(), "workspace") != nullptr);
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, codes.p, scales.p, la.p,
                                    work.p, 4095, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, codes.p, scales.p, la.p,
                                    work.p, 8192, nullptr) == SVDQ_STATUS_SUCCESS);
  CHECK(g_fake.last_ws == work.p && g_fake.last_ws_bytes == 8192);
  CHECK(svdq_quantize_act_workspace_size(M, K, r) == 4096);
  CHECK(svdq_quantize_act_workspace_size(M, 96, r) == 0);
  CHECK(svdq_w4a4_gemm_workspace_size(M, N, K, r) == 8192);
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, y.p,
                               work.p, 8191, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, y.p,
                               work.p, 8192, nullptr) == SVDQ_STATUS_SUCCESS);
  // the workspace may not overlap the output
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, y.p,
                               y.p, 8192, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  // the no-allocation variant: no workspace argument, a plan beyond the fixed
  // 64 MiB scratch is refused before any launch
  g_fake.gemm_need = (size_t(64) << 20) + 1;
  CHECK(svdq_w4a4_gemm_lora_up_noalloc(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, 0, y.p,
                                       nullptr) == SVDQ_STATUS_NOT_SUPPORTED);
  g_fake.gemm_need = size_t(64) << 20;
  CHECK(svdq_w4a4_gemm_lora_up_noalloc(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, 1, y.p,
                                       nullptr) == SVDQ_STATUS_SUCCESS);
  CHECK(std::string(g_fake.last) == "gemm_static" && g_fake.last_out == y.p);
  CHECK(svdq_w4a4_gemm_lora_up_noalloc(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, 0, la.p,
                                       nullptr) == SVDQ_STATUS_INVALID_VALUE);
  g_fake.quant_need = g_fake.gemm_need = 0;
  // overlapping outputs and inputs
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, wc.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, wc.p,
                               nullptr, 0, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, codes.p, codes.p, la.p,
                                    nullptr, 0, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(svdq_quantize_act_lora_down(x.p, lam.as<float>(), down.p, M, K, r, 64, x.p, scales.p, la.p,
                                    nullptr, 0, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  // inputs may share memory
  CHECK(svdq_w4a4_gemm_lora_up(codes.p, scales.p, codes.p, wsc.p, la.p, up.p, bias.p, M, N, K, r, 64, y.p,
                               nullptr, 0, nullptr) == SVDQ_STATUS_SUCCESS);
  // QKV epilogue arguments
  Buf qn(256), kn(256), cs(M * 64 * 4), sn(M * 64 * 4), y3(M * 384 * 2), wc3(384 * K / 2), ws3(384 * K / 64 * 2),
      up3(384 * r * 2), b3(384 * 2);
  CHECK(svdq_w4a4_gemm_qkv_norm_rope(codes.p, scales.p, wc3.p, ws3.p, la.p, up3.p, b3.p, M, 384, K, r, 64, 128,
                                     qn.p, kn.p, 1e-6f, cs.as<float>(), sn.as<float>(), y3.p,
                                     nullptr) == SVDQ_STATUS_SUCCESS);
  CHECK(std::string(g_fake.last) == "gemm_qkv");
  CHECK(svdq_w4a4_gemm_qkv_norm_rope(codes.p, scales.p, wc3.p, ws3.p, la.p, up3.p, b3.p, M, 384, K, r, 64, 128,
                                     qn.p, kn.p, 1e-6f, cs.as<float>(), sn.as<float>(), cs.p,
                                     nullptr) == SVDQ_STATUS_INVALID_VALUE);
  // every status has a name
  for (int s = 0; s <= 7; ++s) CHECK(svdq_status_string(static_cast<svdq_status>(s)) != nullptr);

  // packers on exact-size buffers
  const int64_t PN = 96, PK = 256, PR = 16;
  std::mt19937 rng(7);
  std::normal_distribution<float> nd(0.f, 0.02f);
  std::vector<uint16_t> w(PN * PK);
  for (auto& v : w) v = bf16(nd(rng));
  std::vector<float> amax(PK);
  for (int64_t k = 0; k < PK; ++k) amax[k] = 1.0f + (float)(k % 7);
  Buf smooth(PK * 4), pc(PN * PK / 2), ps(PN * PK / 64 * 2), pd(PR * PK * 2), pu(PN * PR * 2);
  CHECK(svdq_smooth_from_absmax(amax.data(), w.data(), PN, PK, smooth.as<float>()) == SVDQ_STATUS_SUCCESS);
  for (int64_t k = 0; k < PK; ++k) CHECK(std::isfinite(smooth.as<float>()[k]) && smooth.as<float>()[k] > 0);
  CHECK(svdq_pack_weights(w.data(), smooth.as<float>(), PN, PK, PR, 64, 3, pc.as<uint8_t>(), ps.as<uint16_t>(),
                          pd.as<uint16_t>(), pu.as<uint16_t>()) == SVDQ_STATUS_SUCCESS);
  for (int64_t i = 0; i < PN * PK / 2; ++i) {
    const uint8_t b = pc.as<uint8_t>()[i];
    CHECK((b & 0xF) != 8 && (b >> 4) != 8);  // -8 is never produced
  }
  CHECK(svdq_pack_weights(w.data(), smooth.as<float>(), PN, PK, 0, 64, 3, pc.as<uint8_t>(), ps.as<uint16_t>(),
                          nullptr, nullptr) == SVDQ_STATUS_SUCCESS);
  Buf fc(PN * PK / 2), fs(PN * PK / 32);
  CHECK(svdq_pack_weights_fp4(w.data(), smooth.as<float>(), PN, PK, PR, 3, fc.as<uint8_t>(), fs.as<uint8_t>(),
                              pd.as<uint16_t>(), pu.as<uint16_t>()) == SVDQ_STATUS_SUCCESS);
  const int64_t Mc = 8, AN = 64, AK = 128;
  std::vector<uint16_t> aw(AN * AK), xc(Mc * AK);
  for (auto& v : aw) v = bf16(nd(rng));
  for (auto& v : xc) v = bf16(50.f * nd(rng));
  Buf as_(AK * 4), ac(AN * AK / 2), asc(AN * AK / 64 * 2), az(AN * AK / 64);
  float alpha = -1.f;
  CHECK(svdq_awq_pack_weights(aw.data(), xc.data(), Mc, AN, AK, 64, 20, as_.as<float>(), ac.as<uint8_t>(),
                              asc.as<uint16_t>(), az.as<uint8_t>(), &alpha) == SVDQ_STATUS_SUCCESS);
  CHECK(alpha >= 0.f && alpha < 1.f);
  for (int64_t i = 0; i < AN * AK / 64; ++i) CHECK(az.as<uint8_t>()[i] <= 15);
  // packer argument errors
  CHECK(svdq_pack_weights(w.data(), smooth.as<float>(), PN, 96, 0, 64, 3, pc.as<uint8_t>(), ps.as<uint16_t>(),
                          nullptr, nullptr) == SVDQ_STATUS_NOT_SUPPORTED);
  CHECK(svdq_pack_weights(w.data(), smooth.as<float>(), PN, PK, PR, 64, 3, pc.as<uint8_t>(), ps.as<uint16_t>(),
                          nullptr, nullptr) == SVDQ_STATUS_INVALID_VALUE);
  CHECK(svdq_awq_pack_weights(aw.data(), xc.data(), Mc, AN, AK, 64, 0, as_.as<float>(), ac.as<uint8_t>(),
                              asc.as<uint16_t>(), az.as<uint8_t>(), nullptr) == SVDQ_STATUS_INVALID_VALUE);
}

int main(int argc, char** argv) {
  const std::string mode = argc > 1 ? argv[1] : "full";
  if (mode == "full") {
    full_mode();
  } else if (mode == "arch-mismatch") {
    CHECK(svdq_check_device(0) == SVDQ_STATUS_ARCH_MISMATCH);
    CHECK(std::strstr(svdq_last_error(), "gfx950") != nullptr);
    CHECK(svdq_check_device(0) == SVDQ_STATUS_ARCH_MISMATCH);  // cached
    g_fake.launches = 0;
    run_calls(SVDQ_STATUS_ARCH_MISMATCH);
    CHECK(g_fake.launches == 0);
  } else if (mode == "no-device") {
    CHECK(svdq_check_device(0) == SVDQ_STATUS_NO_DEVICE);
    g_fake.launches = 0;
    run_calls(SVDQ_STATUS_NO_DEVICE);
    CHECK(g_fake.launches == 0);
  } else {
    std::fprintf(stderr, "unknown mode %s\n", mode.c_str());
    return 2;
  }
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed: %s\n", mode.c_str());
  return 0;
}
