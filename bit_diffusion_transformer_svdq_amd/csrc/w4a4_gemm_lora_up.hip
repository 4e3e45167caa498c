// Call 2 of the SVDQuant W4A4 linear on gfx950: int4 x int4 GEMM with int32
// accumulation per 64-wide quant group, per-group dequantization, the fused
// low-rank up-projection (lora_act @ L2) and the bias.
//
// Method: mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
// Nunchaku 4-Bit-Quantisierung", section "Nunchaku und SVDQuant" (4-bit weights
// and activations, a 16-bit low-rank branch, fused kernels for both).  Fusion of
// lora_up into this kernel: the charmloop.ai news item on Nunchaku in Diffusers,
// paragraph on the 16-bit branch.
//
// The kernel computes Y^T tiles: the MFMA A operand is the weight tile (rows n),
// the B operand the activation tile (columns m).  With the 16x16 MFMA output
// layout (lane l: column l%16, rows 4*(l/16) + v) every lane then owns four
// consecutive n of one token row m, so Y rows are written 8 bytes at a time.
//
// Main loop, per 64-wide group g:
//  * staging: each thread loads 16 packed bytes (32 nibbles) of the weight tile
//    and 16 of the activation tile, widens nibbles to int8 as 16*q with
//    (x & 0xF0F0F0F0) and ((x << 4) & 0xF0F0F0F0) (no sign extension needed),
//    and writes them to a double-buffered LDS stage.  Weights and activations
//    go through the same code, so the K permutation this introduces is the same
//    on both sides and the dot products are unchanged; the products are 256 *
//    q_x * q_w.
//  * MFMA: v_mfma_i32_16x16x64_i8 covers one whole group per instruction.  Its
//    C operand is the constant 0x4B400000 (the bits of 1.5 * 2^23), so the int32
//    result read as fp32 is exactly 1.5 * 2^23 + 256 * acc (|256 acc| <= 802816
//    < 2^22): the int->float conversion is free.
//  * dequant: t = fma(F, s_x/256, -1.5*2^23 * s_x/256) = fl32(acc * s_x) exactly
//    (s_x is bf16, so both constants are exact), then y = fma(t, s_w, y).
// The int32 group accumulator itself is exact; the debug variant of this
// kernel stores (bits - 0x4B400000) >> 8 instead of dequantizing.
//
// Workgroup: 256 threads (4 waves as 2 x 2), tile 128 n x 128 m, wave tile
// 64 x 64 = 4 x 4 MFMA tiles.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;

constexpr int kBN = 128;            // weight rows (n) per workgroup
constexpr int kBM = 128;            // token rows (m) per workgroup
constexpr int kThreads = 256;
constexpr int kStride = 80;         // LDS bytes per int8 row of one group (64 + 16 pad)
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

struct Stage {
  uint8_t w[kBN * kStride];
  uint8_t a[kBM * kStride];
  float sxm[kBM * 2];   // per token m (permuted, see below): (s_x / 256, -1.5*2^23 * s_x / 256)
  float sw[kBN];        // per weight row n: s_w
};

__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (u32)h << 16);
}

// Token m (0..127) of the tile -> slot in sxm, so that lane l of wave column wm
// finds its four m = wm*64 + 16j + l%16 (j = 0..3) as 8 consecutive floats.
__device__ __forceinline__ int sx_slot(int m) {
  return (m >> 6) * 64 + (m & 15) * 4 + ((m >> 4) & 3);
}

// widen 16 packed bytes (32 nibbles) to 32 int8 bytes holding 16*q
__device__ __forceinline__ void widen(const uint4 p, uint4& lo, uint4& hi) {
  lo.x = (p.x << 4) & 0xF0F0F0F0u;  hi.x = p.x & 0xF0F0F0F0u;
  lo.y = (p.y << 4) & 0xF0F0F0F0u;  hi.y = p.y & 0xF0F0F0F0u;
  lo.z = (p.z << 4) & 0xF0F0F0F0u;  hi.z = p.z & 0xF0F0F0F0u;
  lo.w = (p.w << 4) & 0xF0F0F0F0u;  hi.w = p.w & 0xF0F0F0F0u;
}

template <bool kDump>
struct GemmArgs {
  const uint8_t* act_codes;
  const uint16_t* act_scales;
  const uint8_t* w_codes;
  const uint16_t* w_scales;
  const uint16_t* lora_act;
  const uint16_t* lora_up;
  const uint16_t* bias;
  uint16_t* y;
  int32_t* acc;
  int M, N, K, r;
};

template <bool kDump>
__global__ __launch_bounds__(kThreads, 2) void w4a4_gemm_kernel(const GemmArgs<kDump> p) {
  __shared__ Stage st[2];

  const int M = p.M, N = p.N, K = p.K;
  const int G = K >> 6;
  const int KB = K >> 1;  // bytes per packed row
  const int tiles_n = (N + kBN - 1) / kBN;
  const int tn = blockIdx.x % tiles_n;
  const int tm = blockIdx.x / tiles_n;
  const int n0 = tn * kBN;
  const int m0 = tm * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave >> 1;  // n half of the tile
  const int wm = wave & 1;   // m half of the tile
  const int l16 = lane & 15;
  const int lseg = lane >> 4;

  // staging roles: thread -> (row, half) of the 128 x 32-byte packed group tile
  const int srow = tid >> 1;
  const int shalf = tid & 1;
  const int wrow_g = min(n0 + srow, N - 1);
  const int arow_g = min(m0 + srow, M - 1);
  const uint8_t* wsrc = p.w_codes + (size_t)wrow_g * KB + 16 * shalf;
  const uint8_t* asrc = p.act_codes + (size_t)arow_g * KB + 16 * shalf;
  // scale staging: threads 0..127 -> token scales, 128..255 -> weight scales
  const bool s_is_act = tid < kBM;
  const int s_idx = s_is_act ? tid : tid - kBM;
  const uint16_t* ssrc = s_is_act ? p.act_scales + (size_t)min(m0 + s_idx, M - 1) * G
                                  : p.w_scales + (size_t)min(n0 + s_idx, N - 1) * G;

  uint4 wpk = *reinterpret_cast<const uint4*>(wsrc);
  uint4 apk = *reinterpret_cast<const uint4*>(asrc);
  uint16_t spk = kDump ? 0 : ssrc[0];

  auto stage_store = [&](Stage& s, uint4 wv, uint4 av, uint16_t sv) {
    uint4 lo, hi;
    widen(wv, lo, hi);
    uint4* wd = reinterpret_cast<uint4*>(s.w + srow * kStride + 32 * shalf);
    wd[0] = uint4{lo.x, hi.x, lo.y, hi.y};
    wd[1] = uint4{lo.z, hi.z, lo.w, hi.w};
    widen(av, lo, hi);
    uint4* ad = reinterpret_cast<uint4*>(s.a + srow * kStride + 32 * shalf);
    ad[0] = uint4{lo.x, hi.x, lo.y, hi.y};
    ad[1] = uint4{lo.z, hi.z, lo.w, hi.w};
    if (!kDump) {
      const float f = bf16_to_f32(sv);
      if (s_is_act) {
        const float sp = f * (1.0f / 256.0f);
        const int slot = sx_slot(s_idx);
        s.sxm[2 * slot] = sp;
        s.sxm[2 * slot + 1] = -kMagic * sp;
      } else {
        s.sw[s_idx] = f;
      }
    }
  };

  stage_store(st[0], wpk, apk, spk);
  __syncthreads();

  v4f y[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) y[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (more) {
      wpk = *reinterpret_cast<const uint4*>(wsrc + 32 * (g + 1));
      apk = *reinterpret_cast<const uint4*>(asrc + 32 * (g + 1));
      if (!kDump) spk = ssrc[g + 1];
    }
    const Stage& s = st[buf];
    v4i wf[4], af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wf[i] = *reinterpret_cast<const v4i*>(s.w + (wn * 64 + 16 * i + l16) * kStride + 16 * lseg);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      af[j] = *reinterpret_cast<const v4i*>(s.a + (wm * 64 + 16 * j + l16) * kStride + 16 * lseg);

    if constexpr (kDump) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], af[j], magic, 0, 0, 0);
          const int m = m0 + wm * 64 + 16 * j + l16;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = n0 + wn * 64 + 16 * i + 4 * lseg + v;
            if (m < M && n < N) p.acc[((size_t)m * N + n) * G + g] = (acc[v] - kMagicBits) >> 8;
          }
        }
    } else {
      const v4f sxa = *reinterpret_cast<const v4f*>(&s.sxm[2 * (wm * 64 + l16 * 4)]);
      const v4f sxb = *reinterpret_cast<const v4f*>(&s.sxm[2 * (wm * 64 + l16 * 4) + 4]);
      const float sxp[4] = {sxa[0], sxa[2], sxb[0], sxb[2]};
      const float sxc[4] = {sxa[1], sxa[3], sxb[1], sxb[3]};
      v4f swv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        swv[i] = *reinterpret_cast<const v4f*>(&s.sw[wn * 64 + 16 * i + 4 * lseg]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], af[j], magic, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // element copied to a scalar first: a bit-cast applied directly to
            // an ext-vector element is lowered as a cast of element 0
            const int bits = acc[v];
            const float t = fmaf(__int_as_float(bits), sxp[j], sxc[j]);
            y[i][j][v] = fmaf(t, swv[i][v], y[i][j][v]);
          }
        }
    }
    if (more) stage_store(st[buf ^ 1], wpk, apk, spk);
    __syncthreads();
  }

  if constexpr (!kDump) {
    const int r = p.r;
    // fused lora_up: Y^T[n, m] += lora_up[n, :] . lora_act[m, :]
    if (r > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = min(n0 + wn * 64 + 16 * i + l16, N - 1);
        const uint16_t* up = p.lora_up + (size_t)n * r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = min(m0 + wm * 64 + 16 * j + l16, M - 1);
          const uint16_t* la = p.lora_act + (size_t)m * r;
          int k0 = 0;
          for (; k0 + 32 <= r; k0 += 32) {
            const v8bf a = *reinterpret_cast<const v8bf*>(up + k0 + 8 * lseg);
            const v8bf b = *reinterpret_cast<const v8bf*>(la + k0 + 8 * lseg);
            y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, y[i][j], 0, 0, 0);
          }
          if (k0 < r) {
            const v4bf a = *reinterpret_cast<const v4bf*>(up + k0 + 4 * lseg);
            const v4bf b = *reinterpret_cast<const v4bf*>(la + k0 + 4 * lseg);
            y[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, y[i][j], 0, 0, 0);
          }
        }
      }
    }
    // bias and store: lane owns Y[m, n .. n+3]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + 16 * i + 4 * lseg;
      float b[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr && n < N) {
        const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
        b[0] = __builtin_bit_cast(float, bb.x << 16);
        b[1] = __builtin_bit_cast(float, bb.x & 0xFFFF0000u);
        b[2] = __builtin_bit_cast(float, bb.y << 16);
        b[3] = __builtin_bit_cast(float, bb.y & 0xFFFF0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 64 + 16 * j + l16;
        if (m < M && n < N) {
          uint2 o;
          o.x = pack_bf16(y[i][j][0] + b[0], y[i][j][1] + b[1]);
          o.y = pack_bf16(y[i][j][2] + b[2], y[i][j][3] + b[3]);
          *reinterpret_cast<uint2*>(p.y + (size_t)m * N + n) = o;
        }
      }
    }
  }
}

template <bool kDump>
hipError_t launch(const GemmArgs<kDump>& a, hipStream_t stream) {
  const int tiles = ((a.N + kBN - 1) / kBN) * ((a.M + kBM - 1) / kBM);
  hipLaunchKernelGGL(w4a4_gemm_kernel<kDump>, dim3(tiles), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w4a4_gemm_lora_up(const uint8_t* act_codes, const uint16_t* act_scales,
                                    const uint8_t* w_codes, const uint16_t* w_scales,
                                    const uint16_t* lora_act, const uint16_t* lora_up,
                                    const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                    int64_t r, uint16_t* y, int32_t* acc_dump,
                                    hipStream_t stream) {
  if (acc_dump != nullptr) {
    GemmArgs<true> a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                     y, acc_dump, (int)M, (int)N, (int)K, (int)r};
    return launch<true>(a, stream);
  }
  GemmArgs<false> a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                    y, nullptr, (int)M, (int)N, (int)K, (int)r};
  return launch<false>(a, stream);
}

}  // namespace svdq
