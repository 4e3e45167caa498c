// Internal declarations shared by the C ABI (api.cpp) and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// Call 1: smoothing + int4 group quantization + packing + fused lora_down.
// Shapes are validated by the caller: M > 0, K % 64 == 0, r % 16 == 0, r <= 128.
hipError_t launch_quant_lora_down(const uint16_t* x, const float* lam, const uint16_t* lora_down,
                                  int64_t M, int64_t K, int64_t r,
                                  uint8_t* codes, uint16_t* scales, uint16_t* lora_act,
                                  hipStream_t stream);

// Test hook: forces call 1's work split (K-blocks, row tiles per workgroup);
// 0 keeps the automatic choice.  Affects later launches of this process.
void set_quant_plan_override(int k_blocks, int tiles_per_wg);

// Call 2: W4A4 GEMM + group dequant + fused lora_up + bias.  When `acc_dump` is
// not null the kernel writes the int32 group accumulators [M, N, K/64] there
// instead of Y (scales, lora and bias are then ignored).
// Shapes are validated by the caller: M > 0, N % 64 == 0, K % 64 == 0,
// r % 16 == 0, r <= 128.
hipError_t launch_w4a4_gemm_lora_up(const uint8_t* act_codes, const uint16_t* act_scales,
                                    const uint8_t* w_codes, const uint16_t* w_scales,
                                    const uint16_t* lora_act, const uint16_t* lora_up,
                                    const uint16_t* bias,
                                    int64_t M, int64_t N, int64_t K, int64_t r,
                                    uint16_t* y, int32_t* acc_dump, hipStream_t stream);

// Call 2 for few tokens: K split over the waves of a workgroup, weights
// streamed once.  Same arguments and results as launch_w4a4_gemm_lora_up.
bool skinny_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a4_gemm_skinny(const uint8_t* act_codes, const uint16_t* act_scales,
                                   const uint8_t* w_codes, const uint16_t* w_scales,
                                   const uint16_t* lora_act, const uint16_t* lora_up,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                   int64_t r, uint16_t* y, int32_t* acc_dump, hipStream_t stream);

// Test hook: 0 = choose by shape, 1 = always the tiled kernel, 2 = the
// few-token kernel wherever it is supported.
void set_gemm_path_override(int path);

}  // namespace svdq
