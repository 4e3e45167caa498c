// AWQ W4A16 linear on gfx950: unsigned 4-bit weights with a bf16 scale and a
// zero point per 64-wide group, 16-bit activations divided by the
// activation-aware scale s.  The kernel family the Nunchaku Lite integration
// uses for the adaptive-normalization and modulation projections
// (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch Nunchaku
// 4-Bit-Quantisierung", section "Nunchaku Lite: Nahtlose Integration in
// Diffusers"; int4 with group_size 64 in the config of section "Native
// Ladefunktion in Diffusers"); the quantization is AWQ's (Lin et al., 2023).
//
//   x_hat = bf16(fl32(x * fl32(1/s)))
//   Y[m,n] = bf16( sum_g Delta[n,g] * sum_{k in g} x_hat[m,k] (q[n,k] - z[n,g]) + b[n] )
//
// These layers see one conditioning vector per image (M = batch), so the
// kernel streams the packed weights once: a workgroup owns 32 output channels
// (two MFMA n-tiles) and one tile of 16 tokens, its four waves split K, and
// their fp32 partials are added in wave order through LDS.
//
// Per group and n-tile a wave runs two v_mfma_f32_16x16x32_bf16 with A =
// x_hat and B = 128 + q in bf16: ((w >> 4j) & 0x000F000F) | 0x43004300 turns
// nibbles j and j+4 of a code dword into the bf16 pair (128 + q_j, 128 + q_{j+4})
// in two VALU ops, and the activations are packed in the same (j, j+4) pair
// order, so every product is exact.  One more MFMA pair with B = 1 gives
// xs = sum_{k in g} x_hat; the group then adds Delta * (acc - (128 + z) xs).
// Lane k-slots: in the group's 64 k, lane segment seg takes k = 16 seg + 8 h +
// (0..7) for chunk h = 0, 1, so its code bytes are one aligned 8-byte run
// (32 contiguous bytes per row) and its activations one 32-byte run.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svdq_internal.h"

namespace svdq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kNT = 2;       // n-tiles of 16 per workgroup
constexpr int kBlock = 4;    // groups whose loads are issued together

struct AwqArgs {
  const uint16_t* x;
  const float* smooth;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint16_t* bias;
  uint16_t* y;
  int M, N, K, G;
};

__device__ __forceinline__ float bf_lo(u32 v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf_hi(u32 v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

// one group's loads for this lane: 16 activations (2 x 16 B), 8 code bytes per
// n-tile, Delta and z per n-tile
struct GroupLoads {
  uint4 xa, xb;
  uint2 w[kNT];
  uint16_t d[kNT];
  uint8_t z[kNT];
};

__global__ __launch_bounds__(kThreads) void awq_w4a16_kernel(const AwqArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* mu_s = smem;                 // [K]   fl32(1/s)
  v4f* red = reinterpret_cast<v4f*>(smem + a.K);  // [kWaves][kNT][64]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, seg = lane >> 4;
  const int n0 = blockIdx.x * 16 * kNT;
  const int m0 = blockIdx.y * 16;

  for (int k = threadIdx.x; k < a.K; k += kThreads) mu_s[k] = 1.0f / a.smooth[k];
  __syncthreads();

  const int g_lo = (int)(((long)wave * a.G) / kWaves);
  const int g_hi = (int)(((long)(wave + 1) * a.G) / kWaves);
  const uint16_t* xrow = a.x + (size_t)min(m0 + l16, a.M - 1) * a.K + 16 * seg;
  const int KB = a.K >> 1;
  const uint8_t* wrow[kNT];
  int nrow[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    nrow[t] = min(n0 + 16 * t + l16, a.N - 1);
    wrow[t] = a.codes + (size_t)nrow[t] * KB + 8 * seg;
  }
  auto load = [&](GroupLoads& L, int g) {
    L.xa = *reinterpret_cast<const uint4*>(xrow + 64 * g);
    L.xb = *reinterpret_cast<const uint4*>(xrow + 64 * g + 8);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      L.w[t] = *reinterpret_cast<const uint2*>(wrow[t] + 32 * g);
      L.d[t] = a.scales[(size_t)nrow[t] * a.G + g];
      L.z[t] = a.zeros[(size_t)nrow[t] * a.G + g];
    }
  };

  const v8bf ones = __builtin_bit_cast(v8bf, v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f yacc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) yacc[t] = zero4;

  auto compute = [&](const GroupLoads& L, int g) {
    // A: x_hat of k = 64g + 16 seg + 8h + (j, j+4) pairs
    const float* mu = mu_s + 64 * g + 16 * seg;
    v8bf af[2];
    const u32 xw[2][4] = {{L.xa.x, L.xa.y, L.xa.z, L.xa.w}, {L.xb.x, L.xb.y, L.xb.z, L.xb.w}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4f m0v = *reinterpret_cast<const v4f*>(mu + 8 * h);
      const v4f m1v = *reinterpret_cast<const v4f*>(mu + 8 * h + 4);
      float p[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float mlo = d < 2 ? m0v[2 * d] : m1v[2 * d - 4];
        const float mhi = d < 2 ? m0v[2 * d + 1] : m1v[2 * d - 3];
        p[2 * d] = bf_lo(xw[h][d]) * mlo;
        p[2 * d + 1] = bf_hi(xw[h][d]) * mhi;
      }
      const v4u pk = {pack_bf16(p[0], p[4]), pack_bf16(p[1], p[5]), pack_bf16(p[2], p[6]),
                      pack_bf16(p[3], p[7])};
      af[h] = __builtin_bit_cast(v8bf, pk);
    }
    v4f xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], ones, zero4, 0, 0, 0);
    xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], ones, xs, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      v8bf bf[2];
      const u32 wd[2] = {L.w[t].x, L.w[t].y};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4u b = {(wd[h] & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 4) & 0x000F000Fu) | 0x43004300u,
                       ((wd[h] >> 8) & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 12) & 0x000F000Fu) | 0x43004300u};
        bf[h] = __builtin_bit_cast(v8bf, b);
      }
      v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], bf[0], zero4, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], bf[1], acc, 0, 0, 0);
      const float dl = __builtin_bit_cast(float, (u32)L.d[t] << 16);
      const float c = -(128.0f + (float)L.z[t]);
#pragma unroll
      for (int v = 0; v < 4; ++v) yacc[t][v] = fmaf(dl, fmaf(c, xs[v], acc[v]), yacc[t][v]);
    }
    (void)g;
  };

  // groups in blocks of kBlock: the next block's loads are in flight while
  // the current one is computed (two register sets, unrolled by two)
  GroupLoads A[kBlock], B[kBlock];
  auto load_block = [&](GroupLoads* L, int gb) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) load(L[i], min(gb + i, max(g_hi - 1, 0)));
  };
  auto compute_block = [&](const GroupLoads* L, int gb) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i)
      if (gb + i < g_hi) compute(L[i], gb + i);
  };
  if (g_lo < g_hi) {
    load_block(A, g_lo);
    for (int gb = g_lo; gb < g_hi; gb += 2 * kBlock) {
      load_block(B, gb + kBlock);
      compute_block(A, gb);
      if (gb + kBlock >= g_hi) break;
      load_block(A, gb + 2 * kBlock);
      compute_block(B, gb + kBlock);
    }
  }

  // partials of the four waves added in wave order
#pragma unroll
  for (int t = 0; t < kNT; ++t) red[(wave * kNT + t) * 64 + lane] = yacc[t];
  __syncthreads();
  if (wave < kNT) {
    const int t = wave;
    v4f s = red[t * 64 + lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[(w * kNT + t) * 64 + lane];
    const int n = n0 + 16 * t + l16;
    if (n < a.N) {
      const float b = a.bias ? __builtin_bit_cast(float, (u32)a.bias[n] << 16) : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 4 * seg + v;
        if (m < a.M) a.y[(size_t)m * a.N + n] = (uint16_t)(pack_bf16(s[v] + b, 0.f) & 0xFFFFu);
      }
    }
  }
}

}  // namespace

size_t awq_lds_bytes(int64_t K) { return (size_t)K * 4 + (size_t)kWaves * kNT * 64 * 16; }

hipError_t launch_awq_w4a16(const uint16_t* x, const float* smooth, const uint8_t* codes,
                            const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                            int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  AwqArgs a{x, smooth, codes, scales, zeros, bias, y, (int)M, (int)N, (int)K, (int)(K / 64)};
  const size_t lds = awq_lds_bytes(K);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(awq_w4a16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((N + 16 * kNT - 1) / (16 * kNT)), (unsigned)((M + 15) / 16));
  hipLaunchKernelGGL(awq_w4a16_kernel, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
