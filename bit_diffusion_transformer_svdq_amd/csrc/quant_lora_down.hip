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
// Work split.  The [M, K] problem is cut into cells of 16 rows (a row tile) by
// one 64-wide group.  A workgroup owns a block of TB row tiles by GB
// consecutive groups (one K-block); wave w of the workgroup owns row tile w of
// the block and walks the block's groups with a ring of X loads in flight.
// The host picks (TB, GB) so that the blocks spread evenly over the compute
// units: at M = 4608, K = 3072 that is 7 tiles x 8 groups, 252 workgroups with
// 56 cells each.  A row-only split (16 rows x all of K per workgroup) gives 288
// equal workgroups on 256 CUs, and the 32 CUs that get two of them set the
// kernel time.  The K-block's lora_down slice (GB groups x r ranks, in MFMA
// B-fragment order) and its reciprocals mu sit in LDS and serve all TB waves,
// so L1 is read once per workgroup instead of once per 16 rows.
//
// Lane l of a wave covers row (l % 16) and, inside each group, the two
// 8-element runs k = 8*(l/16) + {0..7} and 32 + 8*(l/16) + {0..7}: one 16-byte
// load per run, 64 contiguous bytes per row per load instruction, and exactly
// the A-operand fragment of v_mfma_f32_16x16x32_bf16.  The group maximum
// combines the four lanes of a row with two cross-lane exchanges.
//
// lora reduction over K-blocks.  With more than one K-block, each wave writes
// its fp32 partial (16 rows x r) to a workspace slot of its own with
// agent-coherent stores, waits for them to complete, then bumps the tile's
// arrival counter.  The wave that arrives last reads the tile's partials with
// agent-coherent loads, adds them in K-block order and writes lora_act, so the
// result does not depend on timing; the counter wraps back to zero.
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

#include <algorithm>
#include <atomic>

#include "svdq_device.h"

namespace svdq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));
typedef u32 v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int kMaxTiles = 12;     // row tiles (= waves) per workgroup
constexpr int kMaxGB = 64;        // groups per K-block (reciprocals held in LDS)
constexpr int kLdsLimit = 160 * 1024;
constexpr int kMuBytes = kMaxGB * 64 * 4;
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kRcp7 = 1.0f / 7.0f;        // fl32(1/7)

// groups of X in flight per wave.  At r <= 32, 3 measured faster than 6 (the
// headline 16.1 -> 14.8 us; more requests in flight only queue) and than 2;
// larger ranks keep the depths their fragment registers allow.
template <int NT>
constexpr int depth_for() { return NT <= 2 ? 3 : (NT <= 4 ? 4 : 3); }

__device__ __forceinline__ float lo_bf16(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// two floats -> packed bf16 pair (round to nearest even), a in the low half
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

struct QuantArgs {
  const uint16_t* x;
  const float* lam;
  const uint16_t* lora_down;
  uint8_t* codes;
  uint16_t* scales;
  uint16_t* lora_act;
  float* part;      // [KB][T][NT][4][64 lanes] partial sums (KB > 1 and r > 0)
  u32* count;       // [T] arrival counters, zero between launches
  int M, K, T, G;   // T = row tiles, G = groups of 64
  int GB, TB, KB;   // groups per K-block, row tiles per workgroup, K-blocks
};

// One 64-wide group of one wave: smooth, quantize, pack, and accumulate the
// lora_down partial.  mu_g points at the group's 64 reciprocals in LDS; the
// lora_down fragment of rank tile t, half i is lf_g[(2t + i) * fstride + flane]
// (in LDS: [NT][2 halves][64 lanes], fstride 64, flane the lane; in registers:
// an array of 2 NT fragments, fstride 1, flane 0).  Returns
// the row's codes as bytes 4*seg..+3 (code_a) and 16+4*seg..+3 (code_b) of
// the group's 32, and the scale's bf16 bits (int4), or the two E8M0 exponents
// of the group's 32-blocks (MXFP4: block 2g in the low byte).
template <int NT, bool kFp4>
__device__ __forceinline__ void quant_group(const uint4& xa, const uint4& xb, const float* mu_g,
                                            const v8bf* lf_g, int fstride, int flane, int lane,
                                            v4f* lacc, u32& code_a, u32& code_b, u32& scale) {
  const int seg = lane >> 4;
  const v4f m0a = *reinterpret_cast<const v4f*>(mu_g + 8 * seg);
  const v4f m0b = *reinterpret_cast<const v4f*>(mu_g + 8 * seg + 4);
  const v4f m1a = *reinterpret_cast<const v4f*>(mu_g + 32 + 8 * seg);
  const v4f m1b = *reinterpret_cast<const v4f*>(mu_g + 32 + 8 * seg + 4);
  const float mu[16] = {m0a[0], m0a[1], m0a[2], m0a[3], m0b[0], m0b[1], m0b[2], m0b[3],
                        m1a[0], m1a[1], m1a[2], m1a[3], m1b[0], m1b[1], m1b[2], m1b[3]};
  const u32 xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};

  // x_hat = bf16(fl32(x * mu)) as packed pairs (also the MFMA A operand)
  u32 xh[8];
  float xf[16];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const float p0 = lo_bf16(xw[d]) * mu[2 * d];
    const float p1 = hi_bf16(xw[d]) * mu[2 * d + 1];
    xh[d] = pack_bf16(p0, p1);
    xf[2 * d] = lo_bf16(xh[d]);
    xf[2 * d + 1] = hi_bf16(xh[d]);
  }
  if constexpr (kFp4) {
    // MXFP4 (OCP Microscaling v1.0): per 32-block, shared exponent
    // floor(log2 amax) - 2 as a biased E8M0 byte, which from the bf16 bits of
    // the block maximum is max(E - 2, 0) (E its exponent field; a zero or
    // subnormal maximum gives 0, the clamped -127).  Elements 0-7 of this lane
    // are in block 0 (k = 8 seg + 0..7), elements 8-15 in block 1.  Each
    // element is scaled by 2^(127 - e) (exact) and rounded to the nearest
    // E2M1 value, i.e. the midpoint ladder 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
    // (a midpoint to the even code), above 6 saturating; zero has no sign.
    v2u16 mb0 = __builtin_bit_cast(v2u16, xh[0] & 0x7FFF7FFFu);
    v2u16 mb1 = __builtin_bit_cast(v2u16, xh[4] & 0x7FFF7FFFu);
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      mb0 = __builtin_elementwise_max(mb0, __builtin_bit_cast(v2u16, xh[d] & 0x7FFF7FFFu));
      mb1 = __builtin_elementwise_max(mb1, __builtin_bit_cast(v2u16, xh[4 + d] & 0x7FFF7FFFu));
    }
    u32 a0 = max((u32)mb0[0], (u32)mb0[1]);
    u32 a1 = max((u32)mb1[0], (u32)mb1[1]);
    {
      const v2u32 s0 = __builtin_amdgcn_permlane16_swap(a0, a0, false, false);
      const v2u32 s1 = __builtin_amdgcn_permlane16_swap(a1, a1, false, false);
      a0 = max(s0[0], s0[1]);
      a1 = max(s1[0], s1[1]);
      const v2u32 t0 = __builtin_amdgcn_permlane32_swap(a0, a0, false, false);
      const v2u32 t1 = __builtin_amdgcn_permlane32_swap(a1, a1, false, false);
      a0 = max(t0[0], t0[1]);
      a1 = max(t1[0], t1[1]);
    }
    const u32 e0 = (u32)max((int)(a0 >> 7) - 2, 0);
    const u32 e1 = (u32)max((int)(a1 >> 7) - 2, 0);
    const float inv[2] = {__builtin_bit_cast(float, (254u - e0) << 23),
                          __builtin_bit_cast(float, (254u - e1) << 23)};
    // The hardware converter (v_cvt_scalef32_pk_fp4_f32, scale 1) rounds to
    // the nearest E2M1 value with midpoints to the even code and saturates,
    // as the ladder does (checked on the device against the ladder for every
    // midpoint, its neighbours and 200k random values); it keeps the sign of
    // negative values that round to zero, which the fixup below clears:
    // (magnitude + 7) sets a nibble's bit 3 exactly when its magnitude is
    // nonzero, with no carry into the next nibble.
    u32 packed[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float* xq = xf + 8 * i;
      const float sc = inv[i];
      u32 w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xq[0] * sc, xq[1] * sc, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xq[2] * sc, xq[3] * sc, 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xq[4] * sc, xq[5] * sc, 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xq[6] * sc, xq[7] * sc, 1.0f, 3);
      const u32 nz = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
      packed[i] = w & (~0x88888888u | nz);
    }
    code_a = packed[0];
    code_b = packed[1];
    scale = e0 | (e1 << 8);
  } else {
    // A = max |x_hat| over the group.  With the sign bit cleared, bf16 bit
    // patterns of non-negative values order like the values, so the maximum is
    // taken on 16-bit integers, two per instruction; the four lanes holding the
    // row's group (l, l^16, l^32, l^48) are combined with two lane swaps.
    v2u16 mm = __builtin_bit_cast(v2u16, xh[0] & 0x7FFF7FFFu);
  #pragma unroll
    for (int d = 1; d < 8; ++d) mm = __builtin_elementwise_max(mm, __builtin_bit_cast(v2u16, xh[d] & 0x7FFF7FFFu));
    u32 am = max((u32)mm[0], (u32)mm[1]);
    {
      const v2u32 sw = __builtin_amdgcn_permlane16_swap(am, am, false, false);
      am = max(sw[0], sw[1]);
      const v2u32 sw2 = __builtin_amdgcn_permlane32_swap(am, am, false, false);
      am = max(sw2[0], sw2[1]);
    }
    const float amax = __builtin_bit_cast(float, am << 16);

    // s = bf16(fl32(A / 7)) equals bf16(fl32(A * fl32(1/7))) for every
    // non-negative bf16 A (checked exhaustively: the two fp32 values differ in
    // the last bit at times, never across a bf16 rounding boundary).
    const u32 sbits = pack_bf16(amax * kRcp7, 0.f) & 0xFFFFu;
    const float s = __builtin_bit_cast(float, sbits << 16);
    // iota = fl32(1/s): hardware reciprocal and one Newton step, exact for bf16
    // s in [2^-100, 2^100] (checked exhaustively on the device); outside that
    // range (never for real activations) the IEEE division.
    float iota;
    const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
    if (__builtin_amdgcn_ballot_w64(!fast && s > 0.f) == 0) {
      const float r = __builtin_amdgcn_rcpf(s);
      iota = fast ? __builtin_fmaf(__builtin_fmaf(-s, r, 1.0f), r, r) : 0.f;
    } else {
      // a reciprocal that overflows (s < 2^-128) makes the group a zero group,
      // like s = 0
      const float r = 1.0f / s;
      iota = (s > 0.f && r <= 0x1.fffffep127f) ? r : 0.f;
    }

    // q = rint(x_hat * iota): the low byte of fma(x_hat, iota, 1.5 * 2^23) is q
    // in two's complement.  Bytes are gathered with byte permutes (even and odd
    // elements apart) and merged into nibbles (element 2i low).
    u32 packed[2];
  #pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32 qb[8];
  #pragma unroll
      for (int e = 0; e < 8; ++e) qb[e] = __builtin_bit_cast(u32, fmaf(xf[8 * i + e], iota, kRoundMagic));
      const u32 ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(qb[6], qb[4], 0x0C0C0400u),
                                           __builtin_amdgcn_perm(qb[2], qb[0], 0x0C0C0400u), 0x05040100u);
      const u32 od = __builtin_amdgcn_perm(__builtin_amdgcn_perm(qb[7], qb[5], 0x0C0C0400u),
                                           __builtin_amdgcn_perm(qb[3], qb[1], 0x0C0C0400u), 0x05040100u);
      packed[i] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
    }
    code_a = packed[0];
    code_b = packed[1];
    scale = sbits;
  }

  // fused lora_down: lacc[t] += x_hat[16 rows, 64] @ L1[64, 16 ranks]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const v4u av = {xh[4 * i], xh[4 * i + 1], xh[4 * i + 2], xh[4 * i + 3]};
      lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                        lf_g[(2 * t + i) * fstride + flane], lacc[t],
                                                        0, 0, 0);
    }
  }
}

// Codes and scales of two consecutive groups g, g+1 of a row leave in 16-byte
// and 4-byte stores.  The row's four lanes (seg = 0..3, lanes 16 apart) hold
// dwords seg and 4+seg of each group's 32 bytes; a 4 x 4 transpose over seg
// (two 32-lane swaps, then two 16-lane swaps) gives lane seg the dwords of
// 16 contiguous bytes: group g bytes 0-15, 16-31, group g+1 bytes 0-15, 16-31.
// Each store instruction then writes 64 contiguous bytes per row instead of
// four separate 4-byte pieces, and scale stores halve.  `swap`: the row is
// stored with the two 8-byte halves of every 16-byte granule exchanged (the
// int4 storage order for rows with bit 3 set; see the GEMM kernel).
__device__ __forceinline__ void store_group_pair(u32 a0, u32 b0, u32 s0, u32 a1, u32 b1, u32 s1, int g,
                                                 int seg, bool row_ok, bool scale_pair_aligned, bool swap,
                                                 uint8_t* crow, uint16_t* srow) {
  const v2u32 t02 = __builtin_amdgcn_permlane32_swap(a0, a1, false, false);
  const v2u32 t13 = __builtin_amdgcn_permlane32_swap(b0, b1, false, false);
  const v2u32 u01 = __builtin_amdgcn_permlane16_swap(t02[0], t13[0], false, false);
  const v2u32 u23 = __builtin_amdgcn_permlane16_swap(t02[1], t13[1], false, false);
  if (row_ok) {
    *reinterpret_cast<uint4*>(crow + 32 * g + 16 * seg) =
        swap ? uint4{u23[0], u23[1], u01[0], u01[1]} : uint4{u01[0], u01[1], u23[0], u23[1]};
    if (seg == 0) {
      if (scale_pair_aligned) {
        *reinterpret_cast<u32*>(srow + g) = s0 | (s1 << 16);
      } else {
        srow[g] = (uint16_t)s0;
        srow[g + 1] = (uint16_t)s1;
      }
    }
  }
}

// the last group of an odd-sized block: 4-byte code stores
__device__ __forceinline__ void store_group(u32 a, u32 b, u32 sc, int g, int seg, bool row_ok, bool swap,
                                            uint8_t* crow, uint16_t* srow) {
  if (row_ok) {
    uint8_t* c = crow + 32 * g + ((4 * seg) ^ (swap ? 8 : 0));
    *reinterpret_cast<u32*>(c) = a;
    *reinterpret_cast<u32*>(c + 16) = b;
    if (seg == 0) srow[g] = (uint16_t)sc;
  }
}

template <int NT, bool kFp4>  // NT = r / 16 rank tiles of 16; kFp4: MXFP4 codes instead of int4
__global__ __launch_bounds__(64 * kMaxTiles) void quant_lora_down_kernel(QuantArgs a) {
  constexpr int R = NT * 16;
  constexpr int kDepth = depth_for<NT>();
  __shared__ __align__(16) float mu_s[kMaxGB * 64];             // [GB * 64]
  extern __shared__ __align__(16) uint8_t smem[];
  v8bf* lf_s = reinterpret_cast<v8bf*>(smem);                   // [GB][NT][2][64]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int kb = blockIdx.y;
  const int g0 = kb * a.GB;
  const int gc = min(a.GB, a.G - g0);  // groups in this K-block (> 0 by the plan)
  const int tile = blockIdx.x * a.TB + wave;
  const bool tile_ok = tile < a.T;     // wave-uniform
  const int rho = lane & 15;
  const int row = tile * 16 + rho;
  const bool row_ok = tile_ok && row < a.M;
  const int K = a.K;

  // 1. the K-block's lora_down fragments (1 KB chunks (group, rank tile,
  //    half), 16 bytes per lane, spread over the waves) and this thread's
  //    lambda values: short L2 round trips, issued ahead of the long X stream
  //    so that waiting for them leaves X in flight (vector memory counters
  //    retire in issue order).  The first kChunks chunks of each wave are
  //    loaded unconditionally (an index past the end repeats the last chunk:
  //    same bytes to the same place), so that the compiler counts the loads
  //    in flight exactly; further chunks (large blocks only) come after X.
  //    Plain loads, not LDS DMA: the compiler does not order DMA against
  //    plain loads and would wait for X before the first use of lambda.
  constexpr int kChunks = 4;
  constexpr int nt1 = NT > 0 ? NT : 1;
  const int nchunk = NT * 2 * gc;
  auto chunk_src = [&](int c) {
    const int h = c & 1, t = (c >> 1) % nt1, gi = (c >> 1) / nt1;
    return reinterpret_cast<const v8bf*>(a.lora_down + (size_t)(16 * t + rho) * K + 64 * (g0 + gi) +
                                         32 * h + 8 * (lane >> 4));
  };
  v8bf fr[NT > 0 ? kChunks : 1];
  if constexpr (NT > 0) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) fr[j] = *chunk_src(min(wave + j * a.TB, nchunk - 1));
  }
  constexpr int kMu = 4;  // lambda values per thread in the fast path
  const int nmu = 64 * gc;
  float lv[kMu];
#pragma unroll
  for (int j = 0; j < kMu; ++j) lv[j] = a.lam[64 * g0 + min(j * nthr + (int)threadIdx.x, nmu - 1)];

  // 2. X: the first group of the ring, then the fragments and mu go to LDS
  //    (waiting for them leaves that group in flight), then the rest of the
  //    ring.  Under the full X stream the small loads above would take as
  //    long as the bulk of X, which would then wait for them.  All X loads
  //    are unconditional (rows past M re-read row M-1, groups past the block
  //    re-read its last group), so the number of loads in flight is the same
  //    on every path and each wait is a precise vmcnt.
  const uint16_t* xrow = a.x + (size_t)(row_ok ? row : a.M - 1) * K + 8 * (lane >> 4);
  uint4 ra[kDepth], rb[kDepth];
  ra[0] = *reinterpret_cast<const uint4*>(xrow + 64 * g0);
  rb[0] = *reinterpret_cast<const uint4*>(xrow + 64 * g0 + 32);

  // 3. fragments and mu = fl32(1 / lambda) into LDS.  Every lane divides and
  //    stores (lanes past the block store the last channel's value again), so
  //    that nothing is predicated.
  if constexpr (NT > 0) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) lf_s[min(wave + j * a.TB, nchunk - 1) * 64 + lane] = fr[j];
  }
#pragma unroll
  for (int j = 0; j < kMu; ++j) mu_s[min(j * nthr + (int)threadIdx.x, nmu - 1)] = 1.0f / lv[j];

#pragma unroll
  for (int s = 1; s < kDepth; ++s) {
    const int gs = g0 + min(s, gc - 1);
    ra[s] = *reinterpret_cast<const uint4*>(xrow + 64 * gs);
    rb[s] = *reinterpret_cast<const uint4*>(xrow + 64 * gs + 32);
  }
  for (int c = kMu * nthr + (int)threadIdx.x; c < nmu; c += nthr) mu_s[c] = 1.0f / a.lam[64 * g0 + c];
  if constexpr (NT > 0) {
    for (int c = wave + kChunks * a.TB; c < nchunk; c += a.TB) lf_s[c * 64 + lane] = *chunk_src(c);
  }
  // LDS writes done; no __syncthreads, whose fence would wait for X as well
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  if (!tile_ok) return;  // no barrier follows

  uint8_t* crow = a.codes + (size_t)row * (K >> 1);
  const bool swap = !kFp4 && (row & 8) != 0;  // int4 storage order of the row
  uint16_t* srow = a.scales + (size_t)row * a.G;
  v4f lacc[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) lacc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // 4. walk the block's groups in full rounds of kDepth: each slot is consumed
  //    in place and then refilled with the group kDepth ahead (refilling first
  //    would make the compiler copy the slot and wait for every load in
  //    flight); the last round's refills past the block re-read its last group.
  //    The codes of an even group (counted from the block start) wait in
  //    registers for the next group; the pair is then stored together.
  const int seg = lane >> 4;
  const bool pair_aligned = (((size_t)row * a.G + g0) & 1) == 0;  // 4-byte scale pairs
  u32 pa = 0, pb = 0, ps = 0;
  auto emit = [&](int gl, u32 ca, u32 cb, u32 sc) {
    if ((gl & 1) == 0) {
      pa = ca;
      pb = cb;
      ps = sc;
    } else {
      store_group_pair(pa, pb, ps, ca, cb, sc, g0 + gl - 1, seg, row_ok, pair_aligned, swap, crow, srow);
    }
  };
  const int nfull = gc / kDepth;
  for (int rnd = 0; rnd < nfull; ++rnd) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      const int gl = rnd * kDepth + s;
      u32 ca, cb, sc;
      quant_group<NT, kFp4>(ra[s], rb[s], mu_s + 64 * gl, lf_s + gl * NT * 128, 64, lane, lane, lacc, ca, cb,
                            sc);
      const int gn = g0 + min(gl + kDepth, gc - 1);
      ra[s] = *reinterpret_cast<const uint4*>(xrow + 64 * gn);
      rb[s] = *reinterpret_cast<const uint4*>(xrow + 64 * gn + 32);
      emit(gl, ca, cb, sc);
    }
  }
  // the remaining gc % kDepth groups sit in the first slots
#pragma unroll
  for (int s = 0; s < kDepth; ++s) {
    const int gl = nfull * kDepth + s;
    if (gl < gc) {
      u32 ca, cb, sc;
      quant_group<NT, kFp4>(ra[s], rb[s], mu_s + 64 * gl, lf_s + gl * NT * 128, 64, lane, lane, lacc, ca, cb,
                            sc);
      emit(gl, ca, cb, sc);
    }
  }
  if (gc & 1) store_group(pa, pb, ps, g0 + gc - 1, seg, row_ok, swap, crow, srow);

  if constexpr (NT > 0) {
    // lane l holds rows 4*(l/16)+v of the tile, rank 16t + l%16
    v4f sum[NT];
    if (a.KB == 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) sum[t] = lacc[t];
    } else {
      // Partials travel as agent-scope relaxed atomics (coherent across the
      // XCDs' L2s without writing back or invalidating whole caches, which a
      // fence would do); the store completion wait orders them before the
      // counter increment, and the reader loads them the same way.
      // Layout [t][v][lane]: each store instruction writes 256 contiguous bytes.
      float* mine = a.part + ((size_t)kb * a.T + tile) * NT * 256;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __hip_atomic_store(mine + (t * 4 + v) * 64 + lane, lacc[t][v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the partial is visible to the agent
      __asm__ volatile("" ::: "memory");
      u32 old = 0;
      if (lane == 0) old = atomicInc(a.count + tile, (u32)(a.KB - 1));
      old = __shfl(old, 0);
      if (old != (u32)(a.KB - 1)) return;  // another K-block of this tile is still running
      __asm__ volatile("" ::: "memory");
      // read the other K-blocks' partials kRd at a time, all loads of a batch
      // before any add (one memory round trip per batch); add in K-block order
      constexpr int kRd = 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        for (int j0 = 0; j0 < a.KB; j0 += kRd) {
          v4f pv[kRd];
#pragma unroll
          for (int i = 0; i < kRd; ++i) {
            const int j = min(j0 + i, a.KB - 1);
            const float* p = a.part + (((size_t)j * a.T + tile) * NT + t) * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              pv[i][e] = __hip_atomic_load(p + e * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int i = 0; i < kRd; ++i) {
            const int j = j0 + i;
            if (j < a.KB) {
              const v4f v = (j == kb) ? lacc[t] : pv[i];
              sum[t] = (j == 0) ? v : sum[t] + v;
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = tile * 16 + 4 * (lane >> 4) + v;
        if (rr < a.M)
          a.lora_act[(size_t)rr * R + 16 * t + rho] = (uint16_t)(pack_bf16(sum[t][v], 0.f) & 0xFFFFu);
      }
  }
}

// Few row tiles (a few hundred tokens): a workgroup owns ONE row tile and one
// K-block, and its KW waves split the block's groups into KW consecutive runs.
// With one wave per row tile (the kernel above) a short row count leaves most
// compute units idle unless K is cut into many blocks, whose partials then meet
// through memory (a store, its completion, an atomic and the loads: several
// round trips on the critical path).  Here the waves' lora partials are added
// in LDS, in wave order, and only the K-blocks (few or one) meet through the
// workspace as above.  No wave shares a group with another, so each loads its
// own lora_down fragments with its X (a ring of row_depth groups in registers)
// and only the reciprocals mu of the block, computed once per workgroup, go
// through LDS.
constexpr int kMaxKW = 8;  // waves per workgroup in the row-tile kernel

// groups in flight per wave in the row-tile kernel: at r <= 32, 2 measured
// faster than 4, 3 and 1 (64 x 3072 6.8 -> 6.2 us, 1024 x 12288 20.1 -> 18.9)
template <int NT>
constexpr int row_depth() { return NT <= 2 ? 2 : (NT <= 4 ? 3 : 2); }

template <int NT, bool kFp4>
__global__ __launch_bounds__(64 * kMaxKW) void quant_lora_down_rows_kernel(QuantArgs a) {
  constexpr int R = NT * 16;
  constexpr int kD = row_depth<NT>();
  constexpr int nt1 = NT > 0 ? NT : 1;
  extern __shared__ __align__(16) float rsm[];
  float* mu_s = rsm;                   // [GB * 64]
  v4f* red_s = reinterpret_cast<v4f*>(rsm + a.GB * 64);  // [KW][NT][64 lanes]

  const int lane = threadIdx.x & 63;
  const int kw = threadIdx.x >> 6;
  const int KW = blockDim.x >> 6;
  const int nthr = blockDim.x;
  const int tile = blockIdx.x;
  const int kb = blockIdx.y;
  const int g0 = kb * a.GB;
  const int gc = min(a.GB, a.G - g0);
  const int wb = gc * kw / KW;         // this wave's groups: [wb, we) of the block
  const int n = gc * (kw + 1) / KW - wb;
  const int rho = lane & 15;
  const int seg = lane >> 4;
  const int row = tile * 16 + rho;
  const bool row_ok = row < a.M;
  const int K = a.K;

  // 1. lambda of the block (short loads, first, so that waiting for them
  //    leaves the ring in flight), then the ring: X and the lora_down
  //    fragments of the wave's first kD groups.  Every load is unconditional
  //    (indexes past the end repeat the last one), so each wait is an exact
  //    vmcnt.
  constexpr int kMu = 8;
  const int nmu = 64 * gc;
  float lv[kMu];
#pragma unroll
  for (int j = 0; j < kMu; ++j) lv[j] = a.lam[64 * g0 + min(j * nthr + (int)threadIdx.x, nmu - 1)];

  const int gw = g0 + wb;              // first group of the wave
  const int nl = max(n, 1) - 1;        // last valid local index
  const uint16_t* xrow = a.x + (size_t)(row_ok ? row : a.M - 1) * K + 8 * seg;
  const uint16_t* lrow = a.lora_down + (size_t)rho * K + 8 * seg;
  uint4 ra[kD], rb[kD];
  v8bf lf[kD][2 * nt1];
  auto load_slot = [&](int s, int j) __attribute__((always_inline)) {
    const int g = gw + min(j, nl);
    ra[s] = *reinterpret_cast<const uint4*>(xrow + 64 * g);
    rb[s] = *reinterpret_cast<const uint4*>(xrow + 64 * g + 32);
    if constexpr (NT > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          lf[s][2 * t + h] = *reinterpret_cast<const v8bf*>(lrow + (size_t)16 * t * K + 64 * g + 32 * h);
    }
  };
#pragma unroll
  for (int s = 0; s < kD; ++s) load_slot(s, s);

  // 2. mu = fl32(1 / lambda) into LDS; no __syncthreads, whose fence would wait
  //    for the ring as well
#pragma unroll
  for (int j = 0; j < kMu; ++j) mu_s[min(j * nthr + (int)threadIdx.x, nmu - 1)] = 1.0f / lv[j];
  for (int c = kMu * nthr + (int)threadIdx.x; c < nmu; c += nthr) mu_s[c] = 1.0f / a.lam[64 * g0 + c];
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");

  uint8_t* crow = a.codes + (size_t)row * (K >> 1);
  const bool swap = !kFp4 && (row & 8) != 0;  // int4 storage order of the row
  uint16_t* srow = a.scales + (size_t)row * a.G;
  v4f lacc[nt1];
#pragma unroll
  for (int t = 0; t < nt1; ++t) lacc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // 3. the wave's groups in rounds of kD, each slot consumed and refilled in
  //    place; codes of groups 2i and 2i+1 (counted from the wave's first group)
  //    leave together
  if (n > 0) {
    const bool pair_aligned = (((size_t)row * a.G + gw) & 1) == 0;
    u32 pa = 0, pb = 0, ps = 0;
    auto emit = [&](int j, u32 ca, u32 cb, u32 sc) __attribute__((always_inline)) {
      if ((j & 1) == 0) {
        pa = ca;
        pb = cb;
        ps = sc;
      } else {
        store_group_pair(pa, pb, ps, ca, cb, sc, gw + j - 1, seg, row_ok, pair_aligned, swap, crow, srow);
      }
    };
    const int nfull = n / kD;
    for (int rnd = 0; rnd < nfull; ++rnd) {
#pragma unroll
      for (int s = 0; s < kD; ++s) {
        const int j = rnd * kD + s;
        u32 ca, cb, sc;
        quant_group<NT, kFp4>(ra[s], rb[s], mu_s + 64 * (wb + j), lf[s], 1, 0, lane, lacc, ca, cb, sc);
        load_slot(s, j + kD);
        emit(j, ca, cb, sc);
      }
    }
#pragma unroll
    for (int s = 0; s < kD; ++s) {
      const int j = nfull * kD + s;
      if (j < n) {
        u32 ca, cb, sc;
        quant_group<NT, kFp4>(ra[s], rb[s], mu_s + 64 * (wb + j), lf[s], 1, 0, lane, lacc, ca, cb, sc);
        emit(j, ca, cb, sc);
      }
    }
    if (n & 1) store_group(pa, pb, ps, gw + n - 1, seg, row_ok, swap, crow, srow);
  }

  if constexpr (NT > 0) {
    // 4. the waves' partials, added in wave order by wave 0 (lane l holds rows
    //    4*(l/16)+v of the tile, rank 16t + l%16)
#pragma unroll
    for (int t = 0; t < NT; ++t) red_s[(kw * NT + t) * 64 + lane] = lacc[t];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS writes done, code stores may fly
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (kw != 0) return;
    v4f sum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) sum[t] = lacc[t];
    for (int w = 1; w < KW; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t) sum[t] += red_s[(w * NT + t) * 64 + lane];

    if (a.KB > 1) {
      // 5. K-blocks meet through the workspace, as in the kernel above
      float* mine = a.part + ((size_t)kb * a.T + tile) * NT * 256;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __hip_atomic_store(mine + (t * 4 + v) * 64 + lane, sum[t][v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the partial is visible to the agent
      __asm__ volatile("" ::: "memory");
      u32 old = 0;
      if (lane == 0) old = atomicInc(a.count + tile, (u32)(a.KB - 1));
      old = __shfl(old, 0);
      if (old != (u32)(a.KB - 1)) return;
      __asm__ volatile("" ::: "memory");
      v4f tot[NT];
      constexpr int kRd = 8;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        tot[t] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < a.KB; j0 += kRd) {
          v4f pv[kRd];
#pragma unroll
          for (int i = 0; i < kRd; ++i) {
            const int j = min(j0 + i, a.KB - 1);
            const float* p = a.part + (((size_t)j * a.T + tile) * NT + t) * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              pv[i][e] = __hip_atomic_load(p + e * 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int i = 0; i < kRd; ++i) {
            const int j = j0 + i;
            if (j < a.KB) {
              const v4f v = (j == kb) ? sum[t] : pv[i];
              tot[t] = (j == 0) ? v : tot[t] + v;
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) sum[t] = tot[t];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = tile * 16 + 4 * (lane >> 4) + v;
        if (rr < a.M)
          a.lora_act[(size_t)rr * R + 16 * t + rho] = (uint16_t)(pack_bf16(sum[t][v], 0.f) & 0xFFFFu);
      }
  }
}

// ---------------------------------------------------------------- host side

struct Plan {
  int TB, GB, KB, nrb;
  size_t lds;
  int KW = 0;  // 0: one wave per row tile (TB tiles per workgroup); else the row-tile kernel's waves
};

size_t lds_bytes(int GB, int NT) { return (size_t)GB * NT * 2048; }  // dynamic part

// Balance cells (16 rows x 64 k) over the compute units, in units of one
// cell's X bytes (2 KB from HBM) per compute unit:
//  - the X stream: 1 per cell; the quantizer's VALU work: ~3.5 per cell of
//    each wave on the busiest SIMD (TB waves share 4 SIMDs; measured: ~750
//    cycles per wave and group against ~210 for a cell's share of HBM); the
//    larger one counts;
//  - the K-block's lora_down slice, read from L2 by each workgroup: GB * NT
//    KB-sized fragments, at half weight (L2, not HBM);
//  - with K split, each row tile's fp32 partial is written and read back
//    through the last-level cache: ~NT per tile, at half weight;
//  - the workgroup's prologue (lambda, reciprocals, barrier): ~1;
// times the number of workgroups that share a compute unit; plus, with more
// than 8 K-blocks, the last wave of each row tile adding the tile's KB
// partials (NT fragments each) on the critical path: 0.2 per fragment.
// Without that term a few hundred tokens got 24-192 K-blocks of a single
// group, and call 1 took 12-40 us where 16-48 blocks of 2-4 groups take
// 9-16 us.
Plan make_plan(int T, int G, int NT, int cus) {
  const int GB0 = std::min(G, 8);
  Plan best{1, GB0, (G + GB0 - 1) / GB0, T, lds_bytes(GB0, NT)};
  double best_cost = 1e300;
  for (int TB = 1; TB <= kMaxTiles; ++TB) {
    const int nrb = (T + TB - 1) / TB;
    for (int KB = (G + kMaxGB - 1) / kMaxGB; KB <= G; ++KB) {
      const int GB = (G + KB - 1) / KB;
      if ((G + GB - 1) / GB != KB) continue;  // same blocks as a smaller KB
      const size_t lds = lds_bytes(GB, NT);
      if (lds + kMuBytes > (size_t)kLdsLimit) continue;
      if (KB > 4 * cus) break;
      const long wgs = (long)nrb * KB;
      const long per_cu = (wgs + cus - 1) / cus;
      const double mem = (double)TB * GB;
      const double valu = 3.5 * ((TB + 3) / 4) * GB;
      const double lora = 0.5 * GB * NT + (KB > 1 ? 0.5 * TB * NT : 0.0);
      const double reduce = KB > 8 ? 0.2 * KB * NT : 0.0;
      const double cost = per_cu * (std::max(mem, valu) + lora + 1.0) + reduce;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = Plan{TB, GB, KB, nrb, lds};
      }
    }
  }
  return best;
}

// The row-tile kernel's plan: KB K-blocks of GB groups (at most kMaxGB, for
// the reciprocals in LDS), KW waves per workgroup splitting each block.
Plan rows_plan(int T, int G, int NT, int KB, int KW) {
  KB = std::max(KB, (G + kMaxGB - 1) / kMaxGB);
  const int GB = (G + KB - 1) / KB;
  KB = (G + GB - 1) / GB;
  KW = std::max(1, std::min({KW, kMaxKW, GB}));
  Plan p{1, GB, KB, T, (size_t)GB * 256 + (size_t)KW * NT * 1024};
  p.KW = KW;
  return p;
}

// Row-tile plans are used up to this many row tiles, while what they read (X
// and, per row tile, the lora_down slices: T G (2 + 2 NT) KB) stays below
// kRowsMaxKB, and with a low-rank branch (without one the kernel above has no
// partials to add either).  Measured against the kernel above (HIP graph
// replays, r = 32): faster at 64 to 2048 tokens for K = 3072 (6.8 / 7.7 /
// 8.2 / 9.2 / 12.0 us at 64 / 256 / 512 / 1024 / 2048 tokens against 9.7 /
// 12.2 / 11.3 / 13.8 / 13.5) and at 64 to 1024 tokens for K = 12288 (9.4 /
// 12.9 / 19.9 against 16.7 / 20.9 / 22.8 us); slower at 2048 tokens for
// K = 12288 (31.0 against 25.1 us), where 128 row tiles each reading the
// whole 768 KiB lora_down make 151 MB with X.
constexpr int kRowsMaxTiles = 128;
constexpr double kRowsMaxKB = 96.0 * 1024;

// Estimated time (us) of a row-tile plan, fitted (least squares) to a sweep of
// HIP-graph-replayed launches on MI355X: 64 to 2048 tokens, K = 3072, 12288
// and 15360, r = 32, KW in {2, 3, 4, 6, 8} and 1 to 24 K-blocks (rms error
// 1.3 us; on each of the twelve swept shapes its pick is within 1.3 us of the
// measured best, and is the best on seven).  Terms: launch and first round
// trip; each group a wave walks, per workgroup sharing a compute unit (the
// quantizer's dependency chain, ~0.25 us); the KB of X and lora_down a compute
// unit reads; waves per compute unit; and with split K, the workspace round
// trips and each batch of 8 partial reads.
double rows_cost(int T, int G, int NT, int KW, int KB, int cus) {
  const Plan p = rows_plan(T, G, NT, KB, KW);
  const int gpw = (p.GB + p.KW - 1) / p.KW;
  const long wgs = (long)T * p.KB;
  const long per_cu = (wgs + cus - 1) / cus;
  const double kb_per_cu = (double)p.GB * (2 + 2 * NT) * per_cu;
  const int batches = p.KB == 1 ? 0 : 1 + (p.KB - 1) / 8;
  return 1.74 + 0.252 * gpw * per_cu + 0.028 * kb_per_cu + 0.539 * p.KW * per_cu + 1.214 * batches +
         (p.KB > 1 ? 1.462 : 0.0);
}

Plan best_rows_plan(int T, int G, int NT, int cus) {
  Plan best = rows_plan(T, G, NT, 1, 2);
  double best_cost = 1e300;
  for (int KW : {2, 3, 4, 6, 8}) {
    for (int KB = 1; KB <= std::min(G, 32); ++KB) {
      const Plan p = rows_plan(T, G, NT, KB, KW);
      if (p.KB != KB || p.KW != KW) continue;  // clipped: the same plan as another (KB, KW)
      const double c = rows_cost(T, G, NT, KW, KB, cus);
      if (c < best_cost - 1e-9) {
        best_cost = c;
        best = p;
      }
    }
  }
  return best;
}

std::atomic<int> g_force_tb{0}, g_force_kb{0}, g_force_kw{0};  // test hooks (0 = automatic)

// The plan of a call on the current device, with the test hook's forced split.
Plan plan_for(int64_t M, int64_t K, int64_t r) {
  const int NT = (int)(r / 16);
  const int T = (int)((M + 15) / 16);
  const int G = (int)(K / 64);
  const int cus = current_cus();
  const int force_kb = g_force_kb.load(), force_tb = g_force_tb.load(), force_kw = g_force_kw.load();
  Plan p = make_plan(T, G, NT, cus);
  if (force_kw > 1) {
    p = rows_plan(T, G, NT, force_kb > 0 ? std::min(force_kb, G) : 1, force_kw);
  } else if (force_kw == 0 && force_kb == 0 && force_tb == 0 && NT > 0 && T <= kRowsMaxTiles &&
             (double)T * G * (2 + 2 * NT) <= kRowsMaxKB) {
    p = best_rows_plan(T, G, NT, cus);
  } else if (force_kb > 0 || force_tb > 0) {
    const int TB = force_tb > 0 ? std::min(force_tb, kMaxTiles) : p.TB;
    const int KB0 = force_kb > 0 ? std::min(force_kb, G) : p.KB;
    const int GB = (G + KB0 - 1) / KB0;
    if (GB <= kMaxGB && lds_bytes(GB, NT) + kMuBytes <= (size_t)kLdsLimit)
      p = Plan{TB, GB, (G + GB - 1) / GB, (T + TB - 1) / TB, lds_bytes(GB, NT)};
  }
  // a split K needs one workspace counter per row tile: beyond that many row
  // tiles K is split only where the LDS requires it (K > 64 groups), and the
  // C ABI rejects such shapes
  if (p.KB > 1 && NT > 0 && (size_t)T > kWsMaxCounters) {
    const int GB = std::min(G, kMaxGB);
    p = p.KW > 0 ? rows_plan(T, G, NT, 1, p.KW) : Plan{p.TB, GB, (G + GB - 1) / GB, p.nrb, lds_bytes(GB, NT)};
  }
  return p;
}

// With K split over several blocks, T arrival counters and the fp32 lora
// partials [KB][T][NT][4][64].
size_t part_counters(const Plan& p, int64_t M, int64_t r) {
  return (r > 0 && p.KB > 1) ? (size_t)((M + 15) / 16) : 0;
}
size_t part_bytes(const Plan& p, int64_t M, int64_t r) {
  return (r > 0 && p.KB > 1) ? (size_t)p.KB * (size_t)((M + 15) / 16) * (size_t)(r / 16) * 64 * 16 : 0;
}

template <int NT, bool kFp4>
hipError_t launch_nt(const QuantArgs& a, const Plan& p, hipStream_t stream) {
  const dim3 grid(p.nrb, p.KB);
  if (p.KW > 0) {
    auto kern = quant_lora_down_rows_kernel<NT, kFp4>;
    if (p.lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * p.KW), p.lds, stream, a);
    return hipGetLastError();
  }
  const dim3 block(64 * p.TB);
  auto kern = quant_lora_down_kernel<NT, kFp4>;
  if (p.lds + kMuBytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, block, p.lds, stream, a);
  return hipGetLastError();
}

}  // namespace

void set_quant_plan_override(int k_blocks, int tiles_per_wg) {
  g_force_kb.store(std::max(0, k_blocks));
  g_force_tb.store(std::max(0, tiles_per_wg));
}

void set_quant_waves_override(int waves) { g_force_kw.store(std::max(0, waves)); }

size_t quant_workspace_bytes(int64_t M, int64_t K, int64_t r) {
  if (M <= 0) return 0;
  const Plan p = plan_for(M, K, r);
  return ws_bytes(part_counters(p, M, r), part_bytes(p, M, r));
}

hipError_t launch_quant_lora_down(const uint16_t* x, const float* lam, const uint16_t* lora_down,
                                  int64_t M, int64_t K, int64_t r, uint8_t* codes,
                                  uint16_t* scales, uint16_t* lora_act, bool fp4, Workspace ws,
                                  hipStream_t stream) {
  const int NT = (int)(r / 16);
  const Plan p = plan_for(M, K, r);

  QuantArgs a;
  a.x = x; a.lam = lam; a.lora_down = lora_down;
  a.codes = codes; a.scales = scales; a.lora_act = lora_act;
  a.part = nullptr; a.count = nullptr;
  a.M = (int)M; a.K = (int)K; a.T = (int)((M + 15) / 16); a.G = (int)(K / 64);
  a.GB = p.GB; a.TB = p.TB; a.KB = p.KB;

  const size_t nc = part_counters(p, M, r);
  if (nc > 0) {
    if (ws.bytes < ws_bytes(nc, part_bytes(p, M, r))) return hipErrorInvalidValue;
    a.count = ws_counters(ws);
    a.part = static_cast<float*>(ws_scratch(ws));
  }

  switch (NT) {
    case 0: return fp4 ? launch_nt<0, true>(a, p, stream) : launch_nt<0, false>(a, p, stream);
    case 1: return fp4 ? launch_nt<1, true>(a, p, stream) : launch_nt<1, false>(a, p, stream);
    case 2: return fp4 ? launch_nt<2, true>(a, p, stream) : launch_nt<2, false>(a, p, stream);
    case 3: return fp4 ? launch_nt<3, true>(a, p, stream) : launch_nt<3, false>(a, p, stream);
    case 4: return fp4 ? launch_nt<4, true>(a, p, stream) : launch_nt<4, false>(a, p, stream);
    case 5: return fp4 ? launch_nt<5, true>(a, p, stream) : launch_nt<5, false>(a, p, stream);
    case 6: return fp4 ? launch_nt<6, true>(a, p, stream) : launch_nt<6, false>(a, p, stream);
    case 7: return fp4 ? launch_nt<7, true>(a, p, stream) : launch_nt<7, false>(a, p, stream);
    case 8: return fp4 ? launch_nt<8, true>(a, p, stream) : launch_nt<8, false>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace svdq
