// Call 2 of the SVDQuant W4A4 linear for few tokens (M up to a few hundred):
// the same arithmetic as the main GEMM kernel (int8 MFMA per 64-wide group with
// the magic-bias C operand, exact per-group dequantization, fused lora_up and
// bias), organised for a weight stream instead of a compute-bound tile grid.
//
// Method: mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
// Nunchaku 4-Bit-Quantisierung", section "Nunchaku und SVDQuant" (4-bit weights
// and activations, a 16-bit low-rank branch); fusion of lora_up: the
// charmloop.ai news item on Nunchaku in Diffusers, paragraph on the 16-bit
// branch.
//
// With few tokens the 128 x 128 tiles of the main kernel leave most compute
// units idle (at M = 64, N = 12288: 96 half-empty tiles) and each of them walks
// all of K at one wave per SIMD.  Here a workgroup owns 16*N16 weight rows and
// a chunk of up to 64 tokens, and its 8 waves split K: wave w takes groups
// [w*G/8, (w+1)*G/8).  Every weight byte is read from HBM once, by one wave,
// straight into registers (16 rows x 64 bytes, a group pair, per load
// instruction), one pair in flight per wave: with two or three in flight (all
// of a wave's pairs at 64 tokens) every shape ran 1-8 % slower, since the
// chip's memory system then holds more requests than it serves well.  The
// token rows are small and shared by every workgroup (L2).  At the end the 8 partial tiles
// are added in a fixed order through LDS, so results do not depend on timing.
//
// Per group and wave: N16 weight fragments and up to 4 activation fragments
// (8 bytes per lane), nibbles widened to 16*q as in the main kernel, one
// v_mfma_i32_16x16x64_i8 per (16 n x 16 m) tile with C = 0x4B400000, then
// t = fma(F, s_x/256, -1.5*2^23 * s_x/256) = fl32(acc * s_x) exactly and
// y = fma(t, s_w, y).  Lane l holds the tile's rows n = 4*(l/16) + v and column
// m = l % 16.  The scales of the workgroup's rows and tokens are staged in LDS
// (transposed, 8 bytes per lane per group).  lora_up is added after the main
// loop, as bf16 MFMAs from LDS with a partial tile as the C operand.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "svdq_device.h"

namespace svdq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v2u32 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMC = 64;              // token rows per chunk (4 MFMA columns of 16)
constexpr int kDepth = 1;            // group pairs in flight per wave (ring slots)
constexpr int kSlotStride = 65;      // floats per (tile, v) row of a reduction slot (bank padding)
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr u32 kNib = 0xF0F0F0F0u;
constexpr int kLdsLimit = 160 * 1024;

__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}
__device__ __forceinline__ float bf16_at(u32 w, int hi) {
  return __builtin_bit_cast(float, hi ? (w & 0xFFFF0000u) : (w << 16));
}
__device__ __forceinline__ v4i widen(uint2 p) {
  return v4i{(int)((p.x << 4) & kNib), (int)(p.x & kNib), (int)((p.y << 4) & kNib), (int)(p.y & kNib)};
}

template <bool kDump>
struct SkinnyArgs {
  const uint8_t* ac;      // act codes [M, K/2]
  const uint16_t* as;     // act scales [M, G] bf16
  const uint8_t* wc;      // weight codes [N, K/2]
  const uint16_t* ws;     // weight scales [N, G] bf16
  const uint16_t* la;     // lora_act [M, r] bf16
  const uint16_t* lu;     // lora_up [N, r] bf16
  const uint16_t* bias;   // [N] bf16 or null
  uint16_t* y;            // [M, N] bf16
  int32_t* dump;          // window [m_hi - m_lo, n_hi - n_lo, G] int32 (debug variant)
  int m_lo, m_hi, n_lo, n_hi;
  int M, N, K, G, r;
  int epilogue;           // 0: none, 1: GELU (tanh form) after the bias
};

// LDS: [G][16*N16] weight scales and [G][16][4] token scales (bf16), then the
// lora tiles [16*N16][r] and [64][r] (bf16), then four reduction slots of
// N16*4*4 rows x kSlotStride floats.
template <int N16>
constexpr size_t slot_floats() { return (size_t)N16 * 16 * kSlotStride; }
__host__ __device__ constexpr size_t align16(size_t b) { return (b + 15) & ~(size_t)15; }
template <int N16>
__host__ __device__ constexpr size_t scales_bytes(int G) { return align16((size_t)G * (16 * N16 + kMC) * 2); }
template <int N16>
__host__ __device__ constexpr size_t lora_bytes(int r) { return align16((size_t)(16 * N16 + kMC) * r * 2); }

template <int N16, bool kDump>
__global__ __launch_bounds__(kThreads, 1) void skinny_kernel(SkinnyArgs<kDump> a) {
  constexpr int NT = 16 * N16;
  constexpr int kRows = NT + kMC;          // scale rows: weight rows, then token rows
  constexpr int kRowsPerWave = kRows / kWaves;
  static_assert(kRows % kWaves == 0, "scale rows per wave");
  extern __shared__ __align__(16) uint8_t smem[];
  const int G = a.G;
  uint16_t* sw_s = reinterpret_cast<uint16_t*>(smem);                 // [G][NT]
  uint16_t* sx_s = sw_s + (size_t)G * NT;                              // [G][16][4]
  uint16_t* lu_s = reinterpret_cast<uint16_t*>(smem + scales_bytes<N16>(G));   // [NT][r]
  uint16_t* la_s = lu_s + (size_t)NT * a.r;                                     // [64][r]
  float* red = reinterpret_cast<float*>(smem + scales_bytes<N16>(G) + lora_bytes<N16>(a.r));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int n0 = blockIdx.x * NT;
  const int m0 = blockIdx.y * kMC;
  const int mt = min(4, (a.M - m0 + 15) >> 4);   // token tiles of 16 in this chunk (>= 1)
  const int K2 = a.K >> 1;
  const int P = (G + 1) >> 1;                     // group pairs
  const int p_begin = (wave * P) / kWaves, p_end = ((wave + 1) * P) / kWaves;
  const int np = p_end - p_begin;                 // >= 0

  v4f y[N16][4];
#pragma unroll
  for (int j = 0; j < N16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) y[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

  // 1. the wave's group pairs: fragments in a ring of kDepth pairs.  The
  //    first is issued after the scale and lora staging below: those short
  //    loads then do not queue behind the chip-wide weight stream, and the
  //    first pair lands about when the staging barrier is passed (2-7 %
  //    faster than issuing the pair first, on every few-token shape measured).
  //    A lane loads 16 bytes, so each instruction moves 64 contiguous bytes of
  //    each of 16 rows (runs of 32 bytes halve what the memory system
  //    delivers): lanes 0-31
  //    get group 2p, lanes 32-63 group 2p+1.  Rows past N or M re-read the
  //    last row, pairs past the wave's range re-read its last pair, and the
  //    missing half of a last odd pair re-reads the group before it, so every
  //    load is unconditional and every wait exact.
  const uint8_t* wrow[N16];
#pragma unroll
  for (int j = 0; j < N16; ++j) wrow[j] = a.wc + (size_t)min(n0 + 16 * j + l16, a.N - 1) * K2;
  const uint8_t* arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = a.ac + (size_t)min(m0 + 16 * i + l16, a.M - 1) * K2;

  uint4 rw[kDepth][N16], ra[kDepth][4];
  const int plast = max(p_end - 1, 0);
  auto fetch = [&](int s, int pp) {
    const int off = min(64 * pp + 16 * lq, K2 - 16);
#pragma unroll
    for (int j = 0; j < N16; ++j) rw[s][j] = *reinterpret_cast<const uint4*>(wrow[j] + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[s][i] = *reinterpret_cast<const uint4*>(arow[i] + off);
  };

  // 2. scales (16-byte row chunks, or for G not a multiple of 8 wave: rows
  //    wave, wave+8, ...; lane: group) and lora tiles
  //    (16 bytes per thread) into LDS; the debug variant needs neither.  They
  //    are issued before any pair; the ring follows them.
  if constexpr (!kDump) {
    // With G a multiple of 8 every scale row starts on a 16-byte boundary and
    // is read in 16-byte chunks of 8 groups (thread c: row c / (G/8)): a few
    // load instructions per workgroup instead of one 2-byte gather per scale
    // row and wave, which shortens the staging that the weight stream waits
    // for (1.4-3.6 % on the few-token shapes measured).  Other G: the gathers.
    const int gc = (G & 7) == 0 ? G >> 3 : 0;     // 16-byte chunks per row
    const int nch = kRows * gc;
    for (int c0 = 0; c0 < nch; c0 += 4 * kThreads) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = min(c0 + u * kThreads + tid, nch - 1);  // past the end: the last chunk again
        const int row = c / gc, part = c - row * gc;
        const uint16_t* src = row < NT ? a.ws + (size_t)min(n0 + row, a.N - 1) * G
                                       : a.as + (size_t)min(m0 + row - NT, a.M - 1) * G;
        v[u] = *reinterpret_cast<const uint4*>(src + 8 * part);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * kThreads + tid;
        if (c < nch) {
          const int row = c / gc, g8 = 8 * (c - row * gc);
          const u32 w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t sv = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            if (row < NT) {
              sw_s[(g8 + e) * NT + row] = sv;
            } else {
              const int m = row - NT;
              sx_s[((g8 + e) * 16 + (m & 15)) * 4 + (m >> 4)] = sv;
            }
          }
        }
      }
    }
    for (int g0 = 0; gc == 0 && g0 < G; g0 += 64) {
      const int g = min(g0 + lane, G - 1);
      uint16_t v[kRowsPerWave];
#pragma unroll
      for (int q = 0; q < kRowsPerWave; ++q) {
        const int row = wave + kWaves * q;
        v[q] = row < NT ? a.ws[(size_t)min(n0 + row, a.N - 1) * G + g]
                        : a.as[(size_t)min(m0 + row - NT, a.M - 1) * G + g];
      }
      if (g0 + lane < G) {
#pragma unroll
        for (int q = 0; q < kRowsPerWave; ++q) {
          const int row = wave + kWaves * q;
          if (row < NT) {
            sw_s[g * NT + row] = v[q];
          } else {
            const int m = row - NT;
            sx_s[(g * 16 + (m & 15)) * 4 + (m >> 4)] = v[q];
          }
        }
      }
    }
    // lora_up rows n0.., then lora_act rows m0.., 8 bf16 per chunk
    const int per_row = a.r >> 3;
    const int nchunk = kRows * per_row;
    for (int c = tid; c < nchunk; c += kThreads) {
      const int row = c / per_row, k = (c - row * per_row) * 8;
      const uint16_t* src = row < NT ? a.lu + (size_t)min(n0 + row, a.N - 1) * a.r + k
                                     : a.la + (size_t)min(m0 + row - NT, a.M - 1) * a.r + k;
      *reinterpret_cast<uint4*>(lu_s + (size_t)row * a.r + k) = *reinterpret_cast<const uint4*>(src);
    }
  }
  fetch(0, min(p_begin, plast));
#pragma unroll
  for (int s = 1; s < kDepth; ++s) fetch(s, min(p_begin + s, plast));

  // scales and lora tiles in LDS (this wave's writes done, then the barrier;
  // no __syncthreads, whose fence would also wait for the ring)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");

  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  // one group g: wf / af are the 8-byte fragments (per lane) of its weight and
  // token tiles
  auto compute = [&](const uint2 (&wf)[N16], const uint2 (&af)[4], int g) {
    // scales: 4 consecutive weight rows per tile j, one token per tile i
    float sxs[4] = {0.f, 0.f, 0.f, 0.f}, sxc[4] = {0.f, 0.f, 0.f, 0.f};
    float swv[N16][4];
    v4i wa[N16];
#pragma unroll
    for (int j = 0; j < N16; ++j) wa[j] = widen(wf[j]);
    if constexpr (!kDump) {
      const uint2 sxw = *reinterpret_cast<const uint2*>(sx_s + (g * 16 + l16) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sxs[i] = bf16_at(i < 2 ? sxw.x : sxw.y, i & 1) * 0.00390625f;  // s_x / 256
        sxc[i] = -kMagic * sxs[i];
      }
#pragma unroll
      for (int j = 0; j < N16; ++j) {
        const uint2 sww = *reinterpret_cast<const uint2*>(sw_s + g * NT + 16 * j + 4 * lq);
        swv[j][0] = bf16_at(sww.x, 0);
        swv[j][1] = bf16_at(sww.x, 1);
        swv[j][2] = bf16_at(sww.y, 0);
        swv[j][3] = bf16_at(sww.y, 1);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < mt) {
        const v4i xb = widen(af[i]);
#pragma unroll
        for (int j = 0; j < N16; ++j) {
          const v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[j], xb, magic, 0, 0, 0);
          if constexpr (kDump) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int m = m0 + 16 * i + l16, n = n0 + 16 * j + 4 * lq + v;
              if (m >= a.m_lo && m < a.m_hi && n >= a.n_lo && n < a.n_hi)
                a.dump[((size_t)(m - a.m_lo) * (size_t)(a.n_hi - a.n_lo) + (size_t)(n - a.n_lo)) * G + g] =
                    (acc[v] - kMagicBits) >> 8;
            }
          } else {
            // bit_cast the whole vector: a bit_cast of one ext-vector element
            // is lowered as element 0 by this compiler
            const v4f F = __builtin_bit_cast(v4f, acc);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float t = __builtin_fmaf(F[v], sxs[i], sxc[i]);
              y[j][i][v] = __builtin_fmaf(t, swv[j][v], y[j][i][v]);
            }
          }
        }
      }
    }
  };
  // A pair slot -> the two groups' fragments.  Lanes 0-31 hold group 2p
  // (bytes 0-15 / 16-31 of the row's group), lanes 32-63 group 2p+1; two lane
  // swaps per 16-byte fragment give every lane 8 bytes of each group: for group
  // 2p, lane groups 0..3 hold bytes 0-7, 16-23, 8-15, 24-31.  Both operands go
  // through the same swaps, so the order of k within the group cancels in the
  // dot products.
  // The swaps are done in place on the ring registers (x <-> z, y <-> w
  // halves), which keeps the compiler from copying ring slots (a copy of a
  // register still being loaded waits for it).
  // Rows with bit 3 set arrive in the int4 storage order (the two 8-byte
  // halves of every 16-byte granule exchanged) and are put back first; the
  // lane's row has bit 3 of l16 (row bases are multiples of 16; clamped rows
  // past N or M only feed outputs that are not stored).
  const bool half_swapped = (l16 & 8) != 0;
  auto split = [&](uint4& f, uint2& g0, uint2& g1) {
    const u32 x = f.x, y = f.y;
    f.x = half_swapped ? f.z : f.x;
    f.y = half_swapped ? f.w : f.y;
    f.z = half_swapped ? x : f.z;
    f.w = half_swapped ? y : f.w;
    __asm__ volatile("v_permlane32_swap_b32 %0, %1" : "+v"(f.x), "+v"(f.z));
    __asm__ volatile("v_permlane32_swap_b32 %0, %1" : "+v"(f.y), "+v"(f.w));
    g0 = uint2{f.x, f.y};
    g1 = uint2{f.z, f.w};
  };
  auto compute_pair = [&](int s, int pp) {
    uint2 w0[N16], w1[N16], a0[4], a1[4];
#pragma unroll
    for (int j = 0; j < N16; ++j) split(rw[s][j], w0[j], w1[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) split(ra[s][i], a0[i], a1[i]);
    compute(w0, a0, 2 * pp);
    if (2 * pp + 1 < G) compute(w1, a1, 2 * pp + 1);
  };

  // 3. the pairs, each slot consumed in place and refilled with the pair
  //    kDepth ahead (past the end: the last pair again, left unused)
  const int nrounds = (np + kDepth - 1) / kDepth;
  for (int rnd = 0; rnd < nrounds; ++rnd) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      const int pp = p_begin + rnd * kDepth + s;
      if (pp < p_end) compute_pair(s, pp);
      fetch(s, min(pp + kDepth, plast));
    }
  }
  if constexpr (kDump) return;

  // 4. lora_act @ L2 from the LDS tiles (bf16 MFMA with the partial tile as
  //    the C operand); tile t = 4j + i goes to wave t % 8
  if (a.r > 0) {
#pragma unroll
    for (int j = 0; j < N16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (((4 * j + i) & (kWaves - 1)) == wave && i < mt) {
          const uint16_t* up = lu_s + (size_t)(16 * j + l16) * a.r;
          const uint16_t* ac = la_s + (size_t)(16 * i + l16) * a.r;
          int k0 = 0;
          for (; k0 + 32 <= a.r; k0 += 32)  // lane l holds k0 + 8*(l/16) + 0..7
            y[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(up + k0 + 8 * lq),
                                                              *reinterpret_cast<const v8bf*>(ac + k0 + 8 * lq),
                                                              y[j][i], 0, 0, 0);
          if (k0 < a.r)  // r % 32 == 16: lane l holds k0 + 4*(l/16) + 0..3
            y[j][i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*reinterpret_cast<const v4bf*>(up + k0 + 4 * lq),
                                                                *reinterpret_cast<const v4bf*>(ac + k0 + 4 * lq),
                                                                y[j][i], 0, 0, 0);
        }
      }
  }

  // The thread's output items e = tid + it * kThreads (it < N16, since a chunk
  // has at most 64 * NT / 2 items): their bias pairs are loaded here, so that
  // the loads' round trip passes during the reduction instead of after it.
  static_assert(kMC * (NT / 2) <= kThreads * N16, "output items per thread");
  const int rows = min(kMC, a.M - m0);
  u32 bpair[N16];
#pragma unroll
  for (int it = 0; it < N16; ++it) {
    const int e = tid + it * kThreads;
    const int m = e / (NT / 2), nl = 2 * (e - m * (NT / 2));
    const int gn = min(n0 + nl, a.N - 2);  // N is a multiple of 16: gn, gn + 1 < N
    bpair[it] = a.bias ? *reinterpret_cast<const u32*>(a.bias + gn) : 0u;
  }

  // 5. fixed-order reduction: slot w' = y(w') + y(w'+4), then
  //    out = ((slot0 + slot1) + slot2) + slot3, plus the bias
  constexpr size_t kSlot = slot_floats<N16>();
  auto slot_at = [&](int w, int j, int i, int v) -> float* {
    return red + (size_t)w * kSlot + (size_t)(((j * 4 + i) * 4 + v) * kSlotStride) + lane;
  };
  // (barriers on LDS only: the ring's last refills may still be in flight)
  auto lds_barrier = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };
  if (wave >= 4) {
#pragma unroll
    for (int j = 0; j < N16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) *slot_at(wave - 4, j, i, v) = y[j][i][v];
  }
  lds_barrier();
  if (wave < 4) {
#pragma unroll
    for (int j = 0; j < N16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float* p = slot_at(wave, j, i, v);
          *p = y[j][i][v] + *p;
        }
  }
  lds_barrier();
#pragma unroll
  for (int it = 0; it < N16; ++it) {  // two consecutive n per item
    const int e = tid + it * kThreads;
    const int m = e / (NT / 2), nl = 2 * (e - m * (NT / 2));
    const int gm = m0 + m, gn = n0 + nl;
    if (m < rows && gn < a.N) {  // N is a multiple of 16, so gn + 1 < N too
      float o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nn = nl + h;
        const int j = nn >> 4, v = nn & 3, q = (nn >> 2) & 3, i = m >> 4, ln = q * 16 + (m & 15);
        const size_t off = (size_t)(((j * 4 + i) * 4 + v) * kSlotStride) + ln;
        o[h] = ((red[off] + red[kSlot + off]) + red[2 * kSlot + off]) + red[3 * kSlot + off];
        if (a.bias) o[h] += __builtin_bit_cast(float, h == 0 ? bpair[it] << 16 : bpair[it] & 0xFFFF0000u);
        if (a.epilogue == 1) o[h] = gelu_tanh(o[h]);
      }
      *reinterpret_cast<u32*>(a.y + (size_t)gm * a.N + gn) = pack_bf16(o[0], o[1]);
    }
  }
}

template <int N16>
size_t lds_for(int G, int r) {
  return scales_bytes<N16>(G) + lora_bytes<N16>(r) + 4 * slot_floats<N16>() * 4;
}

template <int N16, bool kDump>
hipError_t launch_n16(const SkinnyArgs<kDump>& a, hipStream_t stream) {
  const size_t lds = lds_for<N16>(a.G, kDump ? 0 : a.r);
  auto kern = skinny_kernel<N16, kDump>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((a.N + 16 * N16 - 1) / (16 * N16), (a.M + kMC - 1) / kMC);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// rows of 16 per workgroup: one wave of workgroups over the CUs where possible,
// fewer rows per workgroup cost more activation re-reads
int pick_n16(int N, int M, int G, int r, int cus) {
  const int n16s = N / 16, chunks = (M + kMC - 1) / kMC;
  int best = 1;
  double best_cost = 1e300;
  for (int c = 1; c <= 3; ++c) {  // 4 rows of 16 would need more than 256 VGPRs
    size_t lds = 0;
    switch (c) {
      case 1: lds = lds_for<1>(G, r); break;
      case 2: lds = lds_for<2>(G, r); break;
      default: lds = lds_for<3>(G, r); break;
    }
    if (lds > (size_t)kLdsLimit) continue;
    const long wgs = (long)((n16s + c - 1) / c) * chunks;
    const long rounds = (wgs + cus - 1) / cus;
    const double cost = rounds * (c + 1.5);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

template <bool kDump>
hipError_t launch_skinny(const SkinnyArgs<kDump>& a, hipStream_t stream) {
  if constexpr (kDump) {
    return launch_n16<1, true>(a, stream);  // debug path: smallest register set
  } else {
    switch (pick_n16(a.N, a.M, a.G, a.r, current_cus())) {
      case 1: return launch_n16<1, false>(a, stream);
      case 2: return launch_n16<2, false>(a, stream);
      default: return launch_n16<3, false>(a, stream);
    }
  }
}

}  // namespace

bool skinny_supported(int64_t M, int64_t N, int64_t K) {
  (void)M;
  const int G = (int)(K / 64);
  return N % 16 == 0 && lds_for<1>(G, 128) <= (size_t)kLdsLimit;
}

hipError_t launch_w4a4_gemm_skinny(const uint8_t* act_codes, const uint16_t* act_scales,
                                   const uint8_t* w_codes, const uint16_t* w_scales,
                                   const uint16_t* lora_act, const uint16_t* lora_up,
                                   const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                   int64_t r, int epilogue, uint16_t* y, const DumpWindow& dump,
                                   hipStream_t stream) {
  if (dump.acc != nullptr) {
    SkinnyArgs<true> a{act_codes, act_scales, w_codes, w_scales, nullptr, nullptr, nullptr,
                       nullptr, dump.acc, dump.m_lo, dump.m_hi, dump.n_lo, dump.n_hi,
                       (int)M, (int)N, (int)K, (int)(K / 64), 0, 0};
    return launch_skinny<true>(a, stream);
  }
  SkinnyArgs<false> a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                      y, nullptr, 0, 0, 0, 0, (int)M, (int)N, (int)K, (int)(K / 64), (int)r, epilogue};
  return launch_skinny<false>(a, stream);
}

}  // namespace svdq
