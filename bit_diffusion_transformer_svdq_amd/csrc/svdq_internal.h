// Internal declarations shared by the C ABI (api.cpp) and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// Output epilogue of call 2: GELU with the tanh approximation (Hendrycks and
// Gimpel, 2016), 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), for the MLP
// projections the W4A4 layer serves (mind-verse.de, "Effiziente Optimierung
// von Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku
// Lite: Nahtlose Integration in Diffusers").  With e = exp(2u) the identity
// 0.5 x (1 + tanh u) = x - x / (e + 1) needs one exponential and one
// reciprocal, and gives x for e = inf and 0 for e = 0.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * x, x * x, x);
  const float e = __expf(2.0f * u);
  return x - __fdividef(x, e + 1.0f);
}

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

// The library's device scratch for `stream` on the current device: at least
// `counters` u32 counters, zero between launches (every kernel that uses one
// leaves it at zero), and at least `bytes` of scratch after them.  Allocates
// or grows on demand (never while the stream is capturing: then
// hipErrorStreamCaptureUnsupported); outgrown buffers stay allocated.
hipError_t stream_workspace(hipStream_t stream, size_t counters, size_t bytes, uint32_t** counter_ptr,
                            void** scratch_ptr);

// Call 1: smoothing + int4 group quantization + packing + fused lora_down.
// Shapes are validated by the caller: M > 0, K % 64 == 0, r % 16 == 0, r <= 128.
// fp4: MXFP4 codes with two E8M0 exponents per 64-group (stored as one u16
// per group: block 2g in the low byte) instead of int4 codes and bf16 scales.
hipError_t launch_quant_lora_down(const uint16_t* x, const float* lam, const uint16_t* lora_down,
                                  int64_t M, int64_t K, int64_t r,
                                  uint8_t* codes, uint16_t* scales, uint16_t* lora_act,
                                  bool fp4, hipStream_t stream);

// Test hook: forces call 1's work split (K-blocks, row tiles per workgroup);
// 0 keeps the automatic choice.  Affects later launches of this process.
void set_quant_plan_override(int k_blocks, int tiles_per_wg);

// Call 2: W4A4 GEMM + group dequant + fused lora_up + bias.  When `acc_dump` is
// not null the kernel writes the int32 group accumulators [M, N, K/64] there
// instead of Y (scales, lora and bias are then ignored).
// Shapes are validated by the caller: M > 0, N % 64 == 0, K % 64 == 0,
// r % 16 == 0, r <= 128.
// `qkv` is read only for epilogue == kEpilogueQkv (then N % 384 == 0), which
// always runs on the tiled kernel.
hipError_t launch_w4a4_gemm_lora_up(const uint8_t* act_codes, const uint16_t* act_scales,
                                    const uint8_t* w_codes, const uint16_t* w_scales,
                                    const uint16_t* lora_act, const uint16_t* lora_up,
                                    const uint16_t* bias,
                                    int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                                    const QkvEpilogue* qkv, uint16_t* y, int32_t* acc_dump,
                                    hipStream_t stream);

// Call 2 for few tokens: K split over the waves of a workgroup, weights
// streamed once.  Same arguments and results as launch_w4a4_gemm_lora_up.
bool skinny_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a4_gemm_skinny(const uint8_t* act_codes, const uint16_t* act_scales,
                                   const uint8_t* w_codes, const uint16_t* w_scales,
                                   const uint16_t* lora_act, const uint16_t* lora_up,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                   int64_t r, int epilogue, uint16_t* y, int32_t* acc_dump,
                                   hipStream_t stream);

// Call 2 of the MXFP4 variant (tiled kernel; E8M0 scales u8 [rows, K/32],
// K % 128 == 0; epilogue none or GELU).
hipError_t launch_fp4_gemm_lora_up(const uint8_t* act_codes, const uint8_t* act_scales,
                                  const uint8_t* w_codes, const uint8_t* w_scales,
                                  const uint16_t* lora_act, const uint16_t* lora_up,
                                  const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                                  int epilogue, uint16_t* y, hipStream_t stream);

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
