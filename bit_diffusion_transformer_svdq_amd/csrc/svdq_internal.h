// Internal declarations shared by the C ABI (api.cpp) and the HIP kernel files.
// Host-only: the C ABI and the packer build without the device compiler.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

// Epilogue codes of call 2 (values of the C ABI's svdq_epilogue, plus the
// fused QKV epilogue of svdq_w4a4_gemm_qkv_norm_rope).
constexpr int kEpilogueNone = 0;
constexpr int kEpilogueGelu = 1;
constexpr int kEpilogueQkv = 2;

// Operands of the fused QKV epilogue: Y = [Q | K | V] along N, heads of 128
// channels; per-head RMSNorm with learned scales on Q and K, then the rotary
// turn of each adjacent channel pair by the token's angle.
struct QkvEpilogue {
  const uint16_t* q_norm;  // bf16 [128]
  const uint16_t* k_norm;  // bf16 [128]
  const float* cos;        // fp32 [M, 64]
  const float* sin;        // fp32 [M, 64]
  float eps;
};

// Caller-owned device workspace of a call: a fixed region of u32 arrival
// counters first, then scratch bytes (fp32 partial sums of the K-split
// reductions).  The counters are zero whenever no launch using them runs: the
// caller zero-fills the buffer once, and every kernel leaves the counters it
// used at zero.  Because the counter region has the same place and size for
// every call, one workspace serves calls of any shape in turn; the scratch
// after it is always written before it is read.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
constexpr size_t kWsCounterBytes = 1024 * 1024;         // the counter region
constexpr size_t kWsMaxCounters = kWsCounterBytes / 4;  // plans never need more
constexpr size_t ws_bytes(size_t counters, size_t scratch) {
  return (counters == 0 && scratch == 0) ? 0 : kWsCounterBytes + scratch;
}
inline uint32_t* ws_counters(const Workspace& w) { return static_cast<uint32_t*>(w.ptr); }
inline void* ws_scratch(const Workspace& w) { return static_cast<uint8_t*>(w.ptr) + kWsCounterBytes; }

// Call 2 without any allocation: the workspace is the library's fixed device
// scratch (one per device, kStaticScratchBytes, counter region first), whose
// device address is looked up once per device; the first call on a device
// also clears its counters with a fill kernel on `stream`.  Calls that may
// overlap on one device race on it.  The caller checks that the plan's
// gemm_workspace_bytes fits.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t launch_w4a4_gemm_lora_up_static(const uint8_t* act_codes, const uint16_t* act_scales,
                                           const uint8_t* w_codes, const uint16_t* w_scales,
                                           const uint16_t* lora_act, const uint16_t* lora_up,
                                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                                           int epilogue, uint16_t* y, hipStream_t stream);

// Compute units of the current device (cached; 256 when no device answers).
int current_cus();

// Call 1: smoothing + int4 group quantization + packing + fused lora_down.
// Shapes are validated by the caller: M > 0, K % 64 == 0, r % 16 == 0, r <= 128.
// fp4: MXFP4 codes with two E8M0 exponents per 64-group (stored as one u16
// per group: block 2g in the low byte) instead of int4 codes and bf16 scales.
// The workspace must hold quant_workspace_bytes(M, K, r) bytes (planned for
// the current device and the test hook's forced split).
size_t quant_workspace_bytes(int64_t M, int64_t K, int64_t r);
hipError_t launch_quant_lora_down(const uint16_t* x, const float* lam, const uint16_t* lora_down,
                                  int64_t M, int64_t K, int64_t r,
                                  uint8_t* codes, uint16_t* scales, uint16_t* lora_act,
                                  bool fp4, Workspace ws, hipStream_t stream);

// Test hook: forces call 1's work split (K-blocks, row tiles per workgroup);
// 0 keeps the automatic choice.  Affects later launches of this process.
void set_quant_plan_override(int k_blocks, int tiles_per_wg);
void set_quant_waves_override(int waves);

// Window of the accumulator dump: rows [m_lo, m_hi) and columns [n_lo, n_hi)
// of the launched problem go to acc[((m - m_lo) * (n_hi - n_lo) + n - n_lo) * G + g].
struct DumpWindow {
  int32_t* acc = nullptr;
  int m_lo = 0, m_hi = 0, n_lo = 0, n_hi = 0;
};

// Call 2: W4A4 GEMM + group dequant + fused lora_up + bias.  When `dump.acc` is
// not null the kernel writes the int32 group accumulators of the window there
// instead of Y (scales, lora and bias are then ignored).
// Shapes are validated by the caller: M > 0, N % 64 == 0, K % 64 == 0,
// r % 16 == 0, r <= 128.
// `qkv` is read only for epilogue == kEpilogueQkv (then N % 384 == 0), which
// always runs on the tiled kernel.
// The workspace must hold gemm_workspace_bytes(M, N, K, r, epilogue, fp4)
// bytes (planned for the current device and the test hooks' forced settings).
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r, int epilogue, bool fp4);
hipError_t launch_w4a4_gemm_lora_up(const uint8_t* act_codes, const uint16_t* act_scales,
                                    const uint8_t* w_codes, const uint16_t* w_scales,
                                    const uint16_t* lora_act, const uint16_t* lora_up,
                                    const uint16_t* bias,
                                    int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                                    const QkvEpilogue* qkv, uint16_t* y, const DumpWindow& dump,
                                    Workspace ws, hipStream_t stream);

// Call 2 for few tokens: K split over the waves of a workgroup, weights
// streamed once.  Same arguments and results as launch_w4a4_gemm_lora_up.
bool skinny_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a4_gemm_skinny(const uint8_t* act_codes, const uint16_t* act_scales,
                                   const uint8_t* w_codes, const uint16_t* w_scales,
                                   const uint16_t* lora_act, const uint16_t* lora_up,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                   int64_t r, int epilogue, uint16_t* y, const DumpWindow& dump,
                                   hipStream_t stream);

// Call 2 of the MXFP4 variant (tiled kernel; E8M0 scales u8 [rows, K/32],
// K % 128 == 0; epilogue none or GELU).
hipError_t launch_fp4_gemm_lora_up(const uint8_t* act_codes, const uint8_t* act_scales,
                                  const uint8_t* w_codes, const uint8_t* w_scales,
                                  const uint16_t* lora_act, const uint16_t* lora_up,
                                  const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                                  int epilogue, uint16_t* y, Workspace ws, hipStream_t stream);

// Call 2 of the MXFP4 variant on 256 x 256 tiles (one workgroup per CU, no
// K-split, no workspace); K % 1024 == 0, N % 64 == 0, epilogue none or GELU.
// launch_fp4_gemm_lora_up picks it when there are at least a quarter as many
// tiles as CUs.
int fp4_big_tiles(int64_t M, int64_t N);
hipError_t launch_fp4_gemm_big(const uint8_t* act_codes, const uint8_t* act_scales, const uint8_t* w_codes,
                               const uint8_t* w_scales, const uint16_t* lora_act, const uint16_t* lora_up,
                               const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                               uint16_t* y, hipStream_t stream);

// Test hook: output tile edge of the MXFP4 GEMM for later calls (0 = chosen by
// shape, 128 = the tiled kernel with K-splits, 256 = the 256 x 256 kernel
// wherever K % 1024 == 0).
void set_fp4_tile_override(int tile);

// Test hook: 0 = choose by shape, 1 = always the tiled kernel, 2 = the
// few-token kernel wherever it is supported.
void set_gemm_path_override(int path);

// AWQ W4A16 linear (x bf16 [M, K], unsigned 4-bit codes, bf16 scales and u8
// zero points per 64-wide group).  Shapes validated by the caller: M > 0,
// N % 32 == 0, K % 64 == 0, awq_supported(K, M): K <= 16384 for M == 1,
// K <= 8192 for M <= 4, K <= 4096 otherwise (the LDS the instances stage).
// L linears stacked at fixed strides (smooth [L][K], codes [L][N][K/2],
// scales and zeros [L][N][K/64], bias [L][N], y [L][M][N]) share x; L >= 1,
// L <= 65535.
bool awq_supported(int64_t K, int64_t M);
hipError_t launch_awq_w4a16(const uint16_t* x, const float* smooth, const uint8_t* codes,
                            const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                            int64_t L, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// Test hook: K-splits per tile of the tiled kernel (0 = choose by shape;
// clipped to the number of group pairs; ignored for the QKV epilogue).
void set_gemm_splits_override(int splits);

}  // namespace svdq
