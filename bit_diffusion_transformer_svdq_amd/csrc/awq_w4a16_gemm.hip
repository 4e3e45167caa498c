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
// workgroup's 16 rows of codes go into LDS with global_load_lds_dwordx4, each
// instruction moving 1 KB of contiguous rows (reads of 32-byte pieces of 16
// rows per instruction were request-bound at ~1.1 TB/s); piece c of row r sits
// at slot r P + (c ^ r) within its 16-piece block, which keeps the fragment
// reads free of bank conflicts.  Meanwhile x_hat of the tile's tokens is
// written to LDS in the operand order below; the fp32 partials of the waves
// are added in wave order through LDS.
//
// Per group a wave runs two v_mfma_f32_16x16x32_bf16 with A = x_hat and B =
// 128 + q in bf16: ((w >> 4j) & 0x000F000F) | 0x43004300 turns nibbles j and
// j+4 of a code dword into the bf16 pair (128 + q_j, 128 + q_{j+4}) in two
// VALU ops, and x_hat is stored in the same (j, j+4) pair order, so every
// product is exact.  One more MFMA pair with B = 1 gives xs = sum_{k in g}
// x_hat; the group then adds Delta * (acc - (128 + z) xs).  Lane k-slots: in
// the group's 64 k, lane segment seg takes k = 16 seg + 8 h + (0..7) for
// chunk h = 0, 1, so its code bytes are one aligned 8-byte run (32 contiguous
// bytes per row).

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
constexpr int kChunk = 16;   // groups whose loads one wave issues together

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
  const int nslots = 16 * P;
  const int wslots = (nslots + 63) & ~63;          // whole 1 KB DMA blocks
  uint8_t* w_s = smem;                                                  // [wslots][16 B]
  float* mu_s = reinterpret_cast<float*>(smem + 16 * wslots);           // [K]
  v4f* red = reinterpret_cast<v4f*>(smem + 16 * wslots + 4 * a.K);      // [kWaves][64]
  uint4* xh_s = reinterpret_cast<uint4*>(smem + 16 * wslots + 4 * a.K + kWaves * 64 * 16);  // [rows][K/8]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, seg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * 16;
  const int rows = min(a.rows, a.M - m0);
  const int runs = a.K >> 3;

  // Load order (vector-memory counters retire in issue order): the first
  // activation runs and 1/s quads of this thread, then the weights of the
  // wave's first chunk; so computing mu and x_hat waits only for the small
  // loads, and the weight stream overlaps the staging.
  const int g_lo = (int)(((long)wave * a.G) / kWaves);
  const int g_hi = (int)(((long)(wave + 1) * a.G) / kWaves);
  const int nrow = min(n0 + l16, a.N - 1);
  const uint16_t* drow = a.scales + (size_t)nrow * a.G;
  const uint8_t* zrow = a.zeros + (size_t)nrow * a.G;
  const int quads = a.K >> 2;
  const int total = rows * runs;
  auto load_runs = [&](uint4* xv, int t0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(t0 + u * kThreads, total - 1);
      const int rr = t / runs, c = t - rr * runs;
      xv[u] = *reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + rr) * a.K + 8 * c);
    }
  };
  auto load_quads = [&](v4f* sv, int q0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      sv[u] = *reinterpret_cast<const v4f*>(a.smooth + 4 * min(q0 + u * kThreads, quads - 1));
  };
  uint4 xv[4];
  v4f sv[4];
  load_runs(xv, threadIdx.x);
  load_quads(sv, threadIdx.x);
  __asm__ volatile("" ::: "memory");  // these small loads go out first
  // the workgroup's code block: slot j (16 B) <- piece c of row r with
  // r = j / P, c = (j % P) ^ (r & 15) inside complete 16-piece blocks
  auto swz = [&](int c, int r) { return ((c | 15) < P) ? (c ^ (r & 15)) : c; };
  for (int j0 = 64 * wave; j0 < wslots; j0 += 64 * kWaves) {
    const int j = min(j0 + lane, nslots - 1);
    const int r = j / P, c = swz(j - r * P, r);
    const uint8_t* src = a.codes + (size_t)min(n0 + r, a.N - 1) * (a.K >> 1) + 16 * c;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(w_s + 16 * j0), 16, 0, 0);
  }
  // scales and zero points of the wave's first chunk of groups (not combined
  // here: arithmetic on them would make the compiler wait for them early)
  uint16_t dl16[kChunk];
  uint8_t zz[kChunk];
  auto load_chunk = [&](int gb) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int g = min(gb + i, max(g_hi - 1, 0));
      dl16[i] = drow[g];
      zz[i] = zrow[g];
    }
  };
  load_chunk(g_lo);
  __asm__ volatile("" ::: "memory");

  // 2. mu = fl32(1/s) into LDS, then x_hat = bf16(fl32(x mu)) of the staged
  //    rows, each run of 8 in the pair order (0,4), (1,5), (2,6), (3,7)
  auto put_mu = [&](int q0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kThreads;
      if (q < quads) {
        const v4f m = {1.0f / sv[u][0], 1.0f / sv[u][1], 1.0f / sv[u][2], 1.0f / sv[u][3]};
        *reinterpret_cast<v4f*>(mu_s + 4 * q) = m;
      }
    }
  };
  // first pass straight-line (its loads are the ones issued above), later
  // passes (K > 4096) load and store in a loop
  put_mu(threadIdx.x);
  for (int q0 = threadIdx.x + 4 * kThreads; q0 < quads; q0 += 4 * kThreads) {
    load_quads(sv, q0);
    put_mu(q0);
  }
  __syncthreads();
  auto put_runs = [&](int t0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kThreads;
      if (t < total) {
        const int rr = t / runs, c = t - rr * runs;
        const float* mu = mu_s + 8 * c;
        const u32 xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
        float pv[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          pv[2 * d] = bf_lo(xw[d]) * mu[2 * d];
          pv[2 * d + 1] = bf_hi(xw[d]) * mu[2 * d + 1];
        }
        xh_s[rr * runs + c] = uint4{pack_bf16(pv[0], pv[4]), pack_bf16(pv[1], pv[5]),
                                    pack_bf16(pv[2], pv[6]), pack_bf16(pv[3], pv[7])};
      }
    }
  };
  put_runs(threadIdx.x);
  for (int t0 = threadIdx.x + 4 * kThreads; t0 < total; t0 += 4 * kThreads) {
    load_runs(xv, t0);
    put_runs(t0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this wave's code DMAs have landed
  __syncthreads();

  const v8bf ones = __builtin_bit_cast(v8bf, v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f yacc = zero4;
  const bool row_ok = l16 < rows;
  const uint4* xr = xh_s + (size_t)(row_ok ? l16 : 0) * runs + 2 * seg;

  for (int gb = g_lo; gb < g_hi; gb += kChunk) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int g = gb + i;
      if (g < g_hi) {
        // A: the lane's two runs of x_hat (k = 64g + 16 seg + 8h), zero past the tokens
        uint4 r0 = xr[8 * g], r1 = xr[8 * g + 1];
        if (!row_ok) r0 = r1 = uint4{0u, 0u, 0u, 0u};
        const v8bf af0 = __builtin_bit_cast(v8bf, v4u{r0.x, r0.y, r0.z, r0.w});
        const v8bf af1 = __builtin_bit_cast(v8bf, v4u{r1.x, r1.y, r1.z, r1.w});
        v4f xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af0, ones, zero4, 0, 0, 0);
        xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1, ones, xs, 0, 0, 0);
        const int cpiece = 2 * g + (seg >> 1);
        const uint2 wv = *reinterpret_cast<const uint2*>(w_s + 16 * (l16 * P + swz(cpiece, l16)) + 8 * (seg & 1));
        const u32 wd[2] = {wv.x, wv.y};
        v8bf bf[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4u b = {(wd[h] & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 4) & 0x000F000Fu) | 0x43004300u,
                         ((wd[h] >> 8) & 0x000F000Fu) | 0x43004300u, ((wd[h] >> 12) & 0x000F000Fu) | 0x43004300u};
          bf[h] = __builtin_bit_cast(v8bf, b);
        }
        v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af0, bf[0], zero4, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1, bf[1], acc, 0, 0, 0);
        const float dl = __builtin_bit_cast(float, (u32)dl16[i] << 16);
        const float c = -(128.0f + (float)zz[i]);
#pragma unroll
        for (int v = 0; v < 4; ++v) yacc[v] = fmaf(dl, fmaf(c, xs[v], acc[v]), yacc[v]);
      }
    }
    if (gb + kChunk < g_hi) load_chunk(gb + kChunk);
  }

  // partials of the four waves added in wave order
  red[wave * 64 + lane] = yacc;
  __syncthreads();
  if (wave == 0) {
    v4f sum = red[lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w * 64 + lane];
    const int n = n0 + l16;
    if (n < a.N) {
      const float b = a.bias ? __builtin_bit_cast(float, (u32)a.bias[n] << 16) : 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 4 * seg + v;
        if (m < a.M) a.y[(size_t)m * a.N + n] = (uint16_t)(pack_bf16(sum[v] + b, 0.f) & 0xFFFFu);
      }
    }
  }
}

}  // namespace

size_t awq_lds_bytes(int64_t K, int64_t rows) {
  const size_t wslots = ((size_t)16 * (K / 32) + 63) & ~(size_t)63;
  return 16 * wslots + (size_t)K * 4 + (size_t)kWaves * 64 * 16 + (size_t)rows * K * 2;
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
