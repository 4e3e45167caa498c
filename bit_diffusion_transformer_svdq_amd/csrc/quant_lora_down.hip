// Call 1 of the SVDQuant W4A4 linear on gfx950: smoothing, per-token per-group
// symmetric int4 quantization, nibble packing, and the fused low-rank
// down-projection lora_act = x_hat @ L1.
//
// Method: mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
// Nunchaku 4-Bit-Quantisierung", section "Nunchaku und SVDQuant" (activation
// outliers moved into the weights, W4A4); ai2day.live, "AI-Bildmodelle auf
// normalen GPUs ausführen", section "Was ist Nunchaku Lite und was macht es
// genau?" (4-bit live activations).  Fusion of lora_down into this kernel: the
// charmloop.ai news item on Nunchaku in Diffusers, paragraph on the 16-bit
// branch.  X is read from HBM once; x_hat feeds both the quantizer and the
// bf16 MFMA of the down-projection from registers.
//
// Work split.  A workgroup owns 16 rows and the full K; its 4 waves take the
// 64-wide groups round-robin (wave w: groups w, w+4, ...), each wave keeping
// three groups (X and the matching lora_down fragments) in flight.  Lane l of a wave
// covers row (l % 16) and, inside each group, the two 8-element runs
// k = 8*(l/16) + {0..7} and 32 + 8*(l/16) + {0..7}: one global load of 16 bytes
// per run, 64 contiguous bytes per row per load instruction, and exactly the
// A-operand fragment of v_mfma_f32_16x16x32_bf16.  The group maximum combines
// the four lanes of a row with two cross-lane exchanges.  The per-wave lora
// partials are summed over the 4 waves in LDS in a fixed order, so results are
// deterministic.
//
// Rounding (bit-exact by construction): mu = fl32(1/lambda) by IEEE division,
// once per workgroup and channel, kept in LDS;
// fl32(x * mu) by one multiply; bf16 by round-to-nearest-even conversion;
// s = bf16(fl32(A / 7)); iota = fl32(1 / s); q = rint(x_hat * iota) from one fma
// against 1.5 * 2^23 (the exact product is rounded once to an integer, ties to
// even).  |q| <= 7 needs no clamp: s >= (A / 7)(1 - 2^-24)(1 - 2^-8), so
// max |x_hat| * iota < 7.03.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq_internal.h"

namespace svdq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kRows = 16;
constexpr int kDepth = 3;      // groups in flight per wave (X and lora_down)
constexpr int kMuChunk = 4096; // channels whose reciprocals are staged in LDS at a time
constexpr int kRedSlots = kWaves < 4 ? kWaves : 4;  // LDS slots of the lora partial sums
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ float lo_bf16(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// two floats -> packed bf16 pair (round to nearest even), a in the low half
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

// Packed data of one group for one lane, fetched kDepth groups ahead: the two
// 16-byte runs of X and the lane's lora_down fragments (B operand of the bf16
// MFMA: rank 16t + l%16, the same k runs as X).
template <int NT>
struct Slot {
  uint4 xa, xb;
  v8bf lb[NT > 0 ? NT : 1][2];
};

template <int NT>
__device__ __forceinline__ void fetch(Slot<NT>& sl, const uint16_t* xrow, const uint16_t* lrow,
                                      int K, int g) {
  sl.xa = *reinterpret_cast<const uint4*>(xrow + 64 * g);
  sl.xb = *reinterpret_cast<const uint4*>(xrow + 64 * g + 32);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint16_t* l = lrow + (size_t)16 * t * K + 64 * g;
    sl.lb[t][0] = *reinterpret_cast<const v8bf*>(l);
    sl.lb[t][1] = *reinterpret_cast<const v8bf*>(l + 32);
  }
}

// One 64-wide group of one wave: smooth, quantize, pack, store, and accumulate
// the lora_down partial.  mu_g points at the 64 reciprocals of this group.
template <int NT>
__device__ __forceinline__ void quant_group(const Slot<NT>& sl, const float* mu_g, int g, int seg,
                                            bool row_ok, uint8_t* crow, uint16_t* srow_out,
                                            v4f* lacc) {
  const v4f m0a = *reinterpret_cast<const v4f*>(mu_g + 8 * seg);
  const v4f m0b = *reinterpret_cast<const v4f*>(mu_g + 8 * seg + 4);
  const v4f m1a = *reinterpret_cast<const v4f*>(mu_g + 32 + 8 * seg);
  const v4f m1b = *reinterpret_cast<const v4f*>(mu_g + 32 + 8 * seg + 4);
  const float mu[16] = {m0a[0], m0a[1], m0a[2], m0a[3], m0b[0], m0b[1], m0b[2], m0b[3],
                        m1a[0], m1a[1], m1a[2], m1a[3], m1b[0], m1b[1], m1b[2], m1b[3]};
  const u32 xw[8] = {sl.xa.x, sl.xa.y, sl.xa.z, sl.xa.w, sl.xb.x, sl.xb.y, sl.xb.z, sl.xb.w};

  // x_hat = bf16(fl32(x * mu)) as packed pairs (also the MFMA A operand)
  u32 xh[8];
  float xf[16];
  float amax = 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const float p0 = lo_bf16(xw[d]) * mu[2 * d];
    const float p1 = hi_bf16(xw[d]) * mu[2 * d + 1];
    xh[d] = pack_bf16(p0, p1);
    xf[2 * d] = lo_bf16(xh[d]);
    xf[2 * d + 1] = hi_bf16(xh[d]);
    amax = fmaxf(amax, fmaxf(fabsf(xf[2 * d]), fabsf(xf[2 * d + 1])));
  }
  // the four lanes that hold this row's group: lanes l, l^16, l^32, l^48
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));

  const u32 sbits = pack_bf16(amax / 7.0f, 0.f) & 0xFFFFu;
  const float s = __builtin_bit_cast(float, sbits << 16);
  const float iota = s > 0.f ? 1.0f / s : 0.f;

  // quantize and pack 8 nibbles per dword (element 2i low nibble)
  u32 packed[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    u32 pk = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32 qb = __builtin_bit_cast(u32, fmaf(xf[8 * i + e], iota, kRoundMagic));
      pk |= (qb & 0xFu) << (4 * e);
    }
    packed[i] = pk;
  }

  // fused lora_down: lacc[t] += x_hat[16 rows, 64] @ L1[64, 16 ranks]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v4u av = {xh[4 * i], xh[4 * i + 1], xh[4 * i + 2], xh[4 * i + 3]};
      lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av), sl.lb[t][i],
                                                        lacc[t], 0, 0, 0);
    }
  }
  if (row_ok) {
    uint8_t* c = crow + 32 * g + 4 * seg;
    *reinterpret_cast<u32*>(c) = packed[0];
    *reinterpret_cast<u32*>(c + 16) = packed[1];
    if (seg == 0) srow_out[g] = (uint16_t)sbits;
  }
}

template <int NT>  // NT = r / 16 rank tiles of 16
__global__ __launch_bounds__(kWaves * 64) void quant_lora_down_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ lam,
    const uint16_t* __restrict__ lora_down, int M, int K,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ lora_act) {
  constexpr int R = NT * 16;
  __shared__ float mu_s[kMuChunk];
  __shared__ float red[kRedSlots][kRows][NT > 0 ? R : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rho = lane & 15;
  const int seg = lane >> 4;
  const int row0 = blockIdx.x * kRows;
  const int row = row0 + rho;
  const bool row_ok = row < M;
  const int G = K >> 6;
  const uint16_t* xrow = x + (size_t)(row_ok ? row : M - 1) * K + 8 * seg;
  const uint16_t* lrow = lora_down + (size_t)rho * K + 8 * seg;
  uint8_t* crow = codes + (size_t)row * (K >> 1);
  uint16_t* srow = scales + (size_t)row * G;

  v4f lacc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) lacc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // K is processed in chunks of kMuChunk channels whose reciprocals mu sit in
  // LDS.  Inside a chunk, wave w takes groups w, w + kWaves, ... through a ring
  // of kDepth slots: each slot is refilled with the group kDepth steps ahead as
  // soon as it is consumed, and every global load a step waits for was issued
  // kDepth steps earlier (vector memory counters retire in issue order).
  for (int k0 = 0; k0 < K; k0 += kMuChunk) {
    const int kc = min(kMuChunk, K - k0);
    const int g0 = k0 >> 6;
    const int gc = kc >> 6;
    __syncthreads();  // previous chunk's mu fully consumed
    {
      // all loads of lambda first (16 bytes per thread and step), then the
      // divisions: one memory round trip instead of one per element
      constexpr int kPer = (kMuChunk / 4 + kWaves * 64 - 1) / (kWaves * 64);
      const float4* lam4 = reinterpret_cast<const float4*>(lam + k0);
      float4 lv[kPer];
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        const int i = threadIdx.x + c * kWaves * 64;
        if (i < (kc >> 2)) lv[c] = lam4[i];
      }
#pragma unroll
      for (int c = 0; c < kPer; ++c) {
        const int i = threadIdx.x + c * kWaves * 64;
        if (i < (kc >> 2))
          reinterpret_cast<float4*>(mu_s)[i] =
              float4{1.0f / lv[c].x, 1.0f / lv[c].y, 1.0f / lv[c].z, 1.0f / lv[c].w};
      }
    }
    __syncthreads();

    Slot<NT> ring[kDepth];
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      const int gl = wave + kWaves * s;
      if (gl < gc) fetch<NT>(ring[s], xrow, lrow, K, g0 + gl);
    }
    for (int base = wave; base < gc; base += kWaves * kDepth) {
#pragma unroll
      for (int s = 0; s < kDepth; ++s) {
        const int gl = base + kWaves * s;
        if (gl < gc) {
          // consume the slot in place, then refill it: refilling first would
          // make the compiler copy the slot, and the copy waits for every load
          // in flight (loads retire in issue order), draining the ring
          quant_group<NT>(ring[s], mu_s + 64 * gl, g0 + gl, seg, row_ok, crow, srow, lacc);
          const int gn = gl + kWaves * kDepth;
          if (gn < gc) fetch<NT>(ring[s], xrow, lrow, K, g0 + gn);
        }
      }
    }
  }

  if constexpr (NT > 0) {
    // lane l holds rows 4*(l/16)+v, rank 16t + l%16.  Waves w, w + kRedSlots,
    // ... are added into slot w in a fixed order (highest first), then the
    // slots are summed in order: the result does not depend on timing.
    constexpr int kPhases = kWaves / kRedSlots;
#pragma unroll
    for (int ph = kPhases - 1; ph >= 0; --ph) {
      if (wave / kRedSlots == ph) {
        float(*dst)[NT > 0 ? R : 1] = red[wave % kRedSlots];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float& d = dst[4 * seg + v][16 * t + rho];
            d = (ph == kPhases - 1) ? lacc[t][v] : d + lacc[t][v];
          }
      }
      __syncthreads();
    }
    for (int idx = threadIdx.x; idx < kRows * R; idx += kWaves * 64) {
      const int rr = idx / R;
      const int j = idx - rr * R;
      float sum = red[0][rr][j];
#pragma unroll
      for (int w = 1; w < kRedSlots; ++w) sum += red[w][rr][j];
      if (row0 + rr < M) lora_act[(size_t)(row0 + rr) * R + j] = (uint16_t)(pack_bf16(sum, 0.f) & 0xFFFFu);
    }
  }
}

template <int NT>
hipError_t launch_nt(const uint16_t* x, const float* lam, const uint16_t* lora_down, int M, int K,
                     uint8_t* codes, uint16_t* scales, uint16_t* lora_act, hipStream_t stream) {
  const dim3 grid((M + kRows - 1) / kRows);
  hipLaunchKernelGGL(quant_lora_down_kernel<NT>, grid, dim3(kWaves * 64), 0, stream, x, lam,
                     lora_down, M, K, codes, scales, lora_act);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_lora_down(const uint16_t* x, const float* lam, const uint16_t* lora_down,
                                  int64_t M, int64_t K, int64_t r, uint8_t* codes,
                                  uint16_t* scales, uint16_t* lora_act, hipStream_t stream) {
  const int m = (int)M, k = (int)K;
  switch (r / 16) {
    case 0: return launch_nt<0>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 1: return launch_nt<1>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 2: return launch_nt<2>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 3: return launch_nt<3>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 4: return launch_nt<4>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 5: return launch_nt<5>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 6: return launch_nt<6>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 7: return launch_nt<7>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    case 8: return launch_nt<8>(x, lam, lora_down, m, k, codes, scales, lora_act, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace svdq
