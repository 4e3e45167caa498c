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
// kernel is a weight stream: a workgroup owns 16 output channels (one MFMA
// n-tile) and one tile of up to 16 tokens, and its four waves split K.  The
// workgroup's 16 rows of codes, and their Delta and z (contiguous in [N, G]
// layout), go into LDS with global_load_lds_dwordx4, each instruction moving
// 1 KB (reads of 32-byte pieces of 16 rows per instruction were request-bound
// at ~1.1 TB/s); piece c of row r sits at slot r P + (c ^ r) within its
// 16-piece block, which keeps the fragment reads free of bank conflicts.
// Meanwhile x_hat of the tile's tokens is written to LDS in the operand order
// below, with the per-group sums xs = sum_{k in g} x_hat; the fp32 partials of
// the waves are added in wave order through LDS.
//
// Per group a wave runs two v_mfma_f32_16x16x32_bf16 with A = x_hat and B =
// 128 + q in bf16: ((w >> 4j) & 0x000F000F) | 0x43004300 turns nibbles j and
// j+4 of a code dword into the bf16 pair (128 + q_j, 128 + q_{j+4}) in two
// VALU ops, and x_hat is stored in the same (j, j+4) pair order, so every
// product is exact.  The group then adds Delta * (acc - (128 + z) xs).  Lane
// k-slots: in the group's 64 k, lane segment seg takes k = 16 seg + 8 h +
// (0..7) for chunk h = 0, 1, so its code bytes are one aligned 8-byte run (32
// contiguous bytes per row).  Groups go two at a time (independent MFMA
// chains) with the next two groups' operands read from LDS ahead.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "svdq_internal.h"

namespace svdq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct AwqArgs {
  const uint16_t* x;
  const float* smooth;
  const uint8_t* codes;
  const uint16_t* scales;
  const uint8_t* zeros;
  const uint16_t* bias;
  uint16_t* y;
  int M, N, K, G, rows;  // rows: token rows staged per workgroup (min(16, M))
};

__device__ __forceinline__ float bf_lo(u32 v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf_hi(u32 v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

__global__ __launch_bounds__(kThreads) void awq_w4a16_kernel(const AwqArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int P = a.K >> 5;                          // 16-byte code pieces per row
  const int G = a.G;
  const int ncode = 16 * P;                        // code slots of the 16 rows
  const int nslots = ncode + 3 * G;                // + Delta (2G slots) + z (G slots)
  const int wslots = (nslots + 63) & ~63;          // whole 1 KB DMA blocks
  uint8_t* w_s = smem;                                                        // [ncode][16 B]
  const uint16_t* d_s = reinterpret_cast<const uint16_t*>(smem + 16 * ncode);  // [16][G] Delta
  const uint8_t* z_s = smem + 16 * ncode + 32 * G;                             // [16][G] z
  float* xs_s = reinterpret_cast<float*>(smem + 16 * wslots);                  // [G][16] sum x_hat
  v4f* red = reinterpret_cast<v4f*>(smem + 16 * wslots + 64 * G);              // [kWaves][64]
  uint4* xh_s = reinterpret_cast<uint4*>(smem + 16 * wslots + 64 * G + kWaves * 64 * 16);  // [rows][K/8]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, seg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16;
  const int rows = min(a.rows, a.M - m0);
  const int runs = a.K >> 3;

  // 1. Loads, in issue order (vector-memory counters retire in issue order):
  //    1/s and x of the thread's first two runs (up to 4 token rows), then the
  //    workgroup's weight block, so staging x_hat waits only for the small loads.
  uint4 xv[2][4];
  v4f sv[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = min(tid + u * kThreads, runs - 1);
    sv[u][0] = *reinterpret_cast<const v4f*>(a.smooth + 8 * c);
    sv[u][1] = *reinterpret_cast<const v4f*>(a.smooth + 8 * c + 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      xv[u][rr] = *reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + min(rr, rows - 1)) * a.K + 8 * c);
  }
  __asm__ volatile("" ::: "memory");  // these small loads go out first
  // Weight block, one 16-byte slot per lane: slots [0, 16P) are the codes,
  // piece c of row r at r P + (c ^ r) inside complete 16-piece blocks (keeps
  // the fragment reads free of bank conflicts); then the 16 rows' Delta and z,
  // contiguous in [N, G] layout (n0 is a multiple of 16, so both start on a
  // 16-byte boundary).  Pad lanes of the last block repeat the last slot.
  auto swz = [&](int c, int r) { return ((c | 15) < P) ? (c ^ (r & 15)) : c; };
  for (int j0 = 64 * wave; j0 < wslots; j0 += 64 * kWaves) {
    const int j = min(j0 + lane, nslots - 1);
    const uint8_t* src;
    if (j < ncode) {
      const int r = j / P, c = swz(j - r * P, r);
      src = a.codes + (size_t)(n0 + r) * (a.K >> 1) + 16 * c;
    } else if (j < ncode + 2 * G) {
      src = reinterpret_cast<const uint8_t*>(a.scales) + (size_t)n0 * G * 2 + 16 * (j - ncode);
    } else {
      src = a.zeros + (size_t)n0 * G + 16 * (j - ncode - 2 * G);
    }
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(w_s + 16 * j0), 16, 0, 0);
  }
  __asm__ volatile("" ::: "memory");

  // 2. x_hat = bf16(fl32(x mu)), mu = fl32(1/s), each run of 8 stored in the
  //    pair order (0,4), (1,5), (2,6), (3,7); xs[g][row] = sum of the group's
  //    x_hat (the 8 runs of a group sit in 8 consecutive lanes, since runs and
  //    the thread count are multiples of 8).
  auto stage = [&](const uint4 xw4, const float* mu, int rr, int c) {
    const u32 xw[4] = {xw4.x, xw4.y, xw4.z, xw4.w};
    float pv[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      pv[2 * d] = bf_lo(xw[d]) * mu[2 * d];
      pv[2 * d + 1] = bf_hi(xw[d]) * mu[2 * d + 1];
    }
    const uint4 h = {pack_bf16(pv[0], pv[4]), pack_bf16(pv[1], pv[5]), pack_bf16(pv[2], pv[6]),
                     pack_bf16(pv[3], pv[7])};
    xh_s[rr * runs + c] = h;
    const u32 hw[4] = {h.x, h.y, h.z, h.w};
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) s += bf_lo(hw[d]) + bf_hi(hw[d]);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if ((c & 7) == 0) xs_s[(c >> 3) * 16 + rr] = s;
  };
  auto recip = [&](const v4f s0, const v4f s1, float* mu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mu[e] = 1.0f / s0[e];
      mu[4 + e] = 1.0f / s1[e];
    }
  };
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * kThreads;
    if (c < runs) {  // uniform over each aligned 8 lanes
      float mu[8];
      recip(sv[u][0], sv[u][1], mu);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        if (rr < rows) stage(xv[u][rr], mu, rr, c);
      for (int rr = 4; rr < rows; ++rr)
        stage(*reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + rr) * a.K + 8 * c), mu, rr, c);
    }
  }
  for (int c = tid + 2 * kThreads; c < runs; c += kThreads) {  // K > 4096
    float mu[8];
    recip(*reinterpret_cast<const v4f*>(a.smooth + 8 * c), *reinterpret_cast<const v4f*>(a.smooth + 8 * c + 4), mu);
    for (int rr = 0; rr < rows; ++rr)
      stage(*reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + rr) * a.K + 8 * c), mu, rr, c);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's DMAs have landed
  __syncthreads();

  // 3. Groups [g_lo, g_hi) of this wave (wave-uniform bounds).  Rows of A past
  //    the tile's tokens repeat its last row: their outputs are not stored.
  const int g_lo = (wave * G) / kWaves;
  const int g_hi = ((wave + 1) * G) / kWaves;
  const uint4* xr = xh_s + (size_t)min(l16, rows - 1) * runs + 2 * seg;
  const uint8_t* wrow = w_s + 16 * l16 * P + 8 * (seg & 1);
  const uint16_t* drow = d_s + l16 * G;
  const uint8_t* zrow = z_s + l16 * G;
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f yacc = zero4;
  // operands of one group, read from LDS one step ahead of their use
  struct Ops {
    uint4 r0, r1;
    uint2 wv;
    v4f xs;
    u32 dl, z;
  };
  auto read_ops = [&](Ops& o, int g) {
    o.r0 = xr[8 * g];
    o.r1 = xr[8 * g + 1];
    o.wv = *reinterpret_cast<const uint2*>(wrow + 16 * swz(2 * g + (seg >> 1), l16));
    o.xs = *reinterpret_cast<const v4f*>(xs_s + 16 * g + 4 * seg);
    o.dl = drow[g];
    o.z = zrow[g];
  };
  auto mfma_ops = [&](const Ops& o) {
    const v8bf af0 = __builtin_bit_cast(v8bf, v4u{o.r0.x, o.r0.y, o.r0.z, o.r0.w});
    const v8bf af1 = __builtin_bit_cast(v8bf, v4u{o.r1.x, o.r1.y, o.r1.z, o.r1.w});
    const u32 wd[2] = {o.wv.x, o.wv.y};
    v8bf bf[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4u b = {(wd[h] & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 4) & 0x000F000Fu) | 0x43004300u,
                     ((wd[h] >> 8) & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 12) & 0x000F000Fu) | 0x43004300u};
      bf[h] = __builtin_bit_cast(v8bf, b);
    }
    const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af0, bf[0], zero4, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1, bf[1], acc, 0, 0, 0);
  };
  auto finish = [&](const Ops& o, const v4f acc) {
    const float dl = __builtin_bit_cast(float, o.dl << 16);
    const float cz = -(128.0f + (float)o.z);
#pragma unroll
    for (int v = 0; v < 4; ++v) yacc[v] = fmaf(dl, fmaf(cz, o.xs[v], acc[v]), yacc[v]);
  };
  // two groups per step (independent MFMA chains), the next two read ahead;
  // indexes past the wave's range are clamped (read, never used)
  const int glast = G - 1;
  Ops o0, o1;
  read_ops(o0, min(g_lo, glast));
  read_ops(o1, min(g_lo + 1, glast));
  for (int g = g_lo; g < g_hi; g += 2) {
    Ops n0, n1;
    read_ops(n0, min(g + 2, glast));
    read_ops(n1, min(g + 3, glast));
    const v4f acc0 = mfma_ops(o0);
    const v4f acc1 = mfma_ops(o1);
    finish(o0, acc0);
    if (g + 1 < g_hi) finish(o1, acc1);
    o0 = n0;
    o1 = n1;
  }

  // 4. partials of the four waves added in wave order
  red[wave * 64 + lane] = yacc;
  __syncthreads();
  if (wave == 0) {
    v4f sum = red[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w * 64 + lane];
    const int n = n0 + l16;
    const float b = a.bias ? __builtin_bit_cast(float, (u32)a.bias[n] << 16) : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 4 * seg + v;
      if (m < a.M) a.y[(size_t)m * a.N + n] = (uint16_t)(pack_bf16(sum[v] + b, 0.f) & 0xFFFFu);
    }
  }
}

}  // namespace

size_t awq_lds_bytes(int64_t K, int64_t rows) {
  const size_t G = (size_t)K / 64;
  const size_t wslots = ((size_t)16 * (K / 32) + 3 * G + 63) & ~(size_t)63;
  return 16 * wslots + 64 * G + (size_t)kWaves * 64 * 16 + (size_t)rows * K * 2;
}

hipError_t launch_awq_w4a16(const uint16_t* x, const float* smooth, const uint8_t* codes,
                            const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                            int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int rows = (int)std::min<int64_t>(16, M);
  AwqArgs a{x, smooth, codes, scales, zeros, bias, y, (int)M, (int)N, (int)K, (int)(K / 64), rows};
  const size_t lds = awq_lds_bytes(K, rows);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(awq_w4a16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
  hipLaunchKernelGGL(awq_w4a16_kernel, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
