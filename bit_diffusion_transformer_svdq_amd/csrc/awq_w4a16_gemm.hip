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
// kernel is a weight stream: an n-tile of 16 output channels (one MFMA tile)
// and a tile of up to 16 tokens are served by four waves that split K into
// quarters; a workgroup holds one to three n-tiles, which share the staged
// x_hat (the host picks the count per shape).  The 16 rows' Delta and z go into LDS by global_load_lds_dwordx4,
// and each wave streams its quarter of the 16 code rows through a ring of its
// own: a chunk is 2 groups x 16 rows x 32 bytes = 1 KB, one DMA instruction,
// two chunks in flight.  These DMAs are issued first; while they stream,
// x_hat of the tile's tokens is written to LDS in the operand order below,
// with the per-group sums xs = sum_{k in g} x_hat.  The fp32 partials of the
// waves are added in wave order through LDS.
//
// Per group a wave runs two v_mfma_f32_16x16x32_bf16 with A = x_hat and B =
// 128 + q in bf16: ((w >> 4j) & 0x000F000F) | 0x43004300 turns nibbles j and
// j+4 of a code dword into the bf16 pair (128 + q_j, 128 + q_{j+4}) in two
// VALU ops, and x_hat is stored in the same (j, j+4) pair order, so every
// product is exact.  The group then adds Delta * (acc - (128 + z) xs).  Lane
// k-slots: in the group's 64 k, lane segment seg takes k = 16 seg + 8 h +
// (0..7) for chunk h = 0, 1, so its code bytes are one aligned 8-byte run (32
// contiguous bytes per row).  The two groups of a chunk are independent MFMA
// chains.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "svdq_device.h"

namespace svdq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                // waves per n-tile (they split K)
constexpr int kRing = 2;                 // code chunks in flight per wave (3 and 1: slower)
// workgroups per CU an instance fits in (LDS), at most 5 (registers)
constexpr int awq_occupancy(int rows, int kmax, int tiles) {
  const int g = kmax / 64;
  const int lds = tiles * (kRing * 1024 * kWaves + 16 * ((3 * g + 63) & ~63)) + 64 * g + 2 * rows * kmax;
  return 160 * 1024 / lds < 5 ? 160 * 1024 / lds : 5;
}

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

// wait until at most n vector-memory operations of this wave are outstanding
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14));
}
// wait until all LDS operations of this wave are done
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14)); }

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// kRowsMax x kKMax: the largest token tile and K the instance stages;
// kTiles: n-tiles per workgroup, each served by its own 4 waves, all sharing
// the staged x_hat (several tiles per workgroup let a grid with more tiles
// than one wave of workgroups run in one, and re-read x and 1/s once per 32
// or 48 rows instead of once per 16).  Every LDS area is a static
// object: the compiler then tracks which of them a DMA in flight writes, and
// waits only for the ring stage a read depends on (an access to dynamic LDS
// would wait for every DMA in flight).
template <int kRowsMax, int kKMax, int kTiles>
__global__ __launch_bounds__(64 * kWaves * kTiles, awq_occupancy(kRowsMax, kKMax, kTiles))
void awq_w4a16_kernel(const AwqArgs args) {
  constexpr int kThr = 64 * kWaves * kTiles;
  // layer blockIdx.z of a stack of L linears that share x: its own 1/s,
  // codes, Delta, z, bias and output, at fixed strides
  AwqArgs a = args;
  {
    const size_t l = blockIdx.z, N = (size_t)args.N, K = (size_t)args.K, G = (size_t)args.G;
    a.smooth += l * K;
    a.codes += l * N * (K / 2);
    a.scales += l * N * G;
    a.zeros += l * N * G;
    if (a.bias) a.bias += l * N;
    a.y += l * (size_t)args.M * N;
  }
  constexpr int kGMax = kKMax / 64;
  constexpr int kDzSlots = (3 * kGMax + 63) & ~63;  // Delta + z, whole 1 KB blocks
  constexpr int kRingStage = 1024 * kWaves * kTiles;
  // Code ring: stage s holds, for each wave w, one chunk (2 groups x 16 rows
  // x 32 bytes = 1 KB) at 1024 w.
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kRingStage], ring1[kRingStage], ring2[kRing > 2 ? kRingStage : 16];
  __shared__ __attribute__((aligned(16))) uint8_t dz_s[kTiles * 16 * kDzSlots];  // per tile [16][G] Delta, z
  __shared__ __attribute__((aligned(16))) float xs_s[16 * kGMax];                 // [G][16] sum x_hat
  __shared__ __attribute__((aligned(16))) uint4 xh_s[kRowsMax * kKMax / 8];       // [rows][K/8]
  auto stage_of = [&](int s) -> uint8_t* { return s == 0 ? ring0 : s == 1 ? ring1 : ring2; };
  static_assert(kRing == 2 || kRing == 3, "one LDS object per ring stage");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = wave / kWaves, wq = wave % kWaves;  // n-tile of the workgroup, K quarter
  const int l16 = lane & 15, seg = lane >> 4;
  const int n0u = (blockIdx.x * kTiles + tg) * 16;   // past N only in a last, partial workgroup
  const bool tile_ok = n0u < a.N;
  const int n0 = tile_ok ? n0u : a.N - 16;           // loads of a missing tile repeat the last one
  const int m0 = blockIdx.y * 16;
  const int rows = min(a.rows, a.M - m0);
  const int runs = a.K >> 3;

  const int G = a.G;
  const int dzslots = (3 * G + 63) & ~63;
  uint8_t* dzt = dz_s + tg * 16 * kDzSlots;
  const uint16_t* d_s = reinterpret_cast<const uint16_t*>(dzt);
  const uint8_t* z_s = dzt + 32 * G;
  const int g_lo = (wq * G) / kWaves;               // groups [g_lo, g_hi) of this wave
  const int g_hi = ((wq + 1) * G) / kWaves;
  const int nch = (g_hi - g_lo + 1) >> 1;           // chunks of 2 groups

  // 1. 1/s and x of the thread's first two runs (up to 4 token rows), issued
  //    before any DMA.
  uint4 xv[2][4];
  v4f sv[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = min(tid + u * kThr, runs - 1);
    sv[u][0] = *reinterpret_cast<const v4f*>(a.smooth + 8 * c);
    sv[u][1] = *reinterpret_cast<const v4f*>(a.smooth + 8 * c + 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      xv[u][rr] = *reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + min(rr, rows - 1)) * a.K + 8 * c);
  }
  __asm__ volatile("" ::: "memory");  // all of them issued before the staging uses the first
  // Chunk i of the wave: groups g_lo + 2i, +1.  Lane l moves 16 bytes to
  // slot l of the wave's 1 KB: row l / 4, position l % 4, which holds piece
  // p = (l % 4) ^ (row / 4 % 4) of the row's 64 bytes (so the fragment reads
  // of 16 rows hit distinct banks).  Chunks past the wave's last one repeat
  // its last chunk (an L2 hit), keeping the count of DMAs per wave fixed.
  const int drow_ = lane >> 2;
  const int dpiece = (lane & 3) ^ ((drow_ >> 2) & 3);
  const uint8_t* dsrc = a.codes + (size_t)(n0 + drow_) * (a.K >> 1) + 16 * (dpiece & 1);
  auto dma_chunk = [&](int i, int s) {
    const int g = min(g_lo + 2 * min(i, max(nch - 1, 0)) + (dpiece >> 1), G - 1);
    dma16(dsrc + 32 * g, stage_of(s) + 1024 * wave);
  };

  // 2. The 16 rows' Delta and z (contiguous in [N, G] layout; n0 is a
  //    multiple of 16, so both start on a 16-byte boundary), a fixed count of
  //    DMAs per wave (blocks past the last repeat it, pad lanes the last
  //    slot); then exactly kRing code chunks of this wave, so "at most
  //    kRing outstanding" means everything before has landed.  They go out before
  //    x_hat is staged, so the weight stream starts at once; the staging
  //    waits for the x and 1/s loads with an explicit count of the DMAs
  //    issued after them (vector-memory counters retire in issue order).
  constexpr int kDzDmas = kDzSlots / (64 * kWaves) + (kDzSlots % (64 * kWaves) != 0);
#pragma unroll
  for (int t = 0; t < kDzDmas; ++t) {
    const int j0 = min(64 * (wq + kWaves * t), dzslots - 64);
    const int j = min(j0 + lane, 3 * G - 1);
    const uint8_t* src = j < 2 * G ? reinterpret_cast<const uint8_t*>(a.scales) + (size_t)n0 * G * 2 + 16 * j
                                   : a.zeros + (size_t)n0 * G + 16 * (j - 2 * G);
    dma16(src, dzt + 16 * j0);
  }
#pragma unroll
  for (int s = 0; s < kRing; ++s) dma_chunk(s, s);
  wait_vm<kDzDmas + kRing>();  // the x and 1/s loads of this thread have landed

  // 3. x_hat = bf16(fl32(x mu)), mu = fl32(1/s), each run of 8 stored in the
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
    const int c = tid + u * kThr;
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
  for (int c = tid + 2 * kThr; c < runs; c += kThr) {  // more than two runs per thread
    float mu[8];
    recip(*reinterpret_cast<const v4f*>(a.smooth + 8 * c), *reinterpret_cast<const v4f*>(a.smooth + 8 * c + 4), mu);
    for (int rr = 0; rr < rows; ++rr)
      stage(*reinterpret_cast<const uint4*>(a.x + (size_t)(m0 + rr) * a.K + 8 * c), mu, rr, c);
  }
  wait_vm<kRing>();  // Delta and z of this wave have landed
  __syncthreads();

  // 4. The wave's chunks through the ring: wait for chunk i (the ring is the
  //    wave's own, so no barrier), compute its two groups (independent MFMA
  //    chains), refill the stage with chunk i + 3.  Rows of A past the tile's
  //    tokens repeat its last row: their outputs are not stored.
  const uint4* xr = xh_s + (size_t)min(l16, rows - 1) * runs + 2 * seg;
  const uint16_t* drow = d_s + l16 * G;
  const uint8_t* zrow = z_s + l16 * G;
  const int fsw = (l16 >> 2) & 3;
  const int foff = 1024 * wave + 64 * l16 + 8 * (seg & 1);
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  v4f yacc = zero4;
  // the two masks in registers (opaque to the compiler), so each nibble pair
  // costs a shift and one v_and_or_b32 instead of separate and / or with literals
  u32 kNibs = 0x000F000Fu, kBias = 0x43004300u;
  __asm__ volatile("" : "+v"(kNibs), "+v"(kBias));
  auto group = [&](const uint8_t* st, int h, int g) {
    const int gr = min(g, G - 1);  // the second group of an odd tail is computed, not added
    const uint4 r0 = xr[8 * gr], r1 = xr[8 * gr + 1];
    // one 64-bit load (split into two 32-bit loads, the second lost the
    // LDS-object information the waits depend on)
    const uint64_t w64 = *reinterpret_cast<const uint64_t*>(st + foff + 16 * ((2 * h + (seg >> 1)) ^ fsw));
    const v8bf af0 = __builtin_bit_cast(v8bf, v4u{r0.x, r0.y, r0.z, r0.w});
    const v8bf af1 = __builtin_bit_cast(v8bf, v4u{r1.x, r1.y, r1.z, r1.w});
    const u32 wd[2] = {(u32)w64, (u32)(w64 >> 32)};
    v8bf bf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const v4u b = {(wd[hh] & kNibs) | kBias, ((wd[hh] >> 4) & kNibs) | kBias, ((wd[hh] >> 8) & kNibs) | kBias,
                     ((wd[hh] >> 12) & kNibs) | kBias};
      bf[hh] = __builtin_bit_cast(v8bf, b);
    }
    const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af0, bf[0], zero4, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1, bf[1], acc, 0, 0, 0);
  };
  auto finish = [&](int g, const v4f acc) {
    const float dl = __builtin_bit_cast(float, (u32)drow[g] << 16);
    const float cz = -(128.0f + (float)zrow[g]);
    const v4f xs = *reinterpret_cast<const v4f*>(xs_s + 16 * g + 4 * seg);
#pragma unroll
    for (int v = 0; v < (kRowsMax < 4 ? kRowsMax : 4); ++v)  // rows 4 seg + v of A beyond kRowsMax are not stored
      yacc[v] = fmaf(dl, fmaf(cz, xs[v], acc[v]), yacc[v]);
  };
  for (int i0 = 0; i0 < nch; i0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      // every step runs the same instructions (past the last chunk on
      // repeated data), so the count of DMAs in flight is the same on every
      // path and the compiler's own waits stay at one stage
      const int i = i0 + u;
      wait_vm<kRing - 1>();
      const uint8_t* st = stage_of(u);
      const int g = g_lo + 2 * i;
      const v4f acc0 = group(st, 0, g);  // past the last chunk: computed, not added
      const v4f acc1 = group(st, 1, g + 1);
      wait_lds();  // the stage's reads are done before it is refilled
      dma_chunk(i + kRing, u);
      if (i < nch) {
        finish(g, acc0);
        if (g + 1 < g_hi) finish(g + 1, acc1);
      }
    }
  }

  // 5. partials of each tile's four waves added in wave order, through the
  //    wave's own 1 KB of ring stage 0 once its DMAs have landed
  wait_vm<0>();
  v4f* red = reinterpret_cast<v4f*>(ring0);
  red[wave * 64 + lane] = yacc;
  __syncthreads();
  if (wq == 0 && tile_ok) {
    v4f sum = red[wave * 64 + lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[(wave + w) * 64 + lane];
    const int n = n0 + l16;
    const float b = a.bias ? __builtin_bit_cast(float, (u32)a.bias[n] << 16) : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + 4 * seg + v;
      if (m < a.M) a.y[(size_t)m * a.N + n] = (uint16_t)(pack_bf16(sum[v] + b, 0.f) & 0xFFFFu);
    }
  }
}

// instances: (token rows, K) classes, smallest first, one n-tile per
// workgroup; up to four tokens with K <= 3072 also with three n-tiles per
// workgroup, for grids that one tile per workgroup would run in more than one
// wave of workgroups
struct AwqClass {
  int rows, kmax, tiles;
  void (*kernel)(AwqArgs);
};
constexpr AwqClass kClasses[] = {
    {1, 4096, 1, awq_w4a16_kernel<1, 4096, 1>},  {1, 16384, 1, awq_w4a16_kernel<1, 16384, 1>},
    {4, 4096, 1, awq_w4a16_kernel<4, 4096, 1>},  {4, 8192, 1, awq_w4a16_kernel<4, 8192, 1>},
    {16, 4096, 1, awq_w4a16_kernel<16, 4096, 1>},
};
constexpr AwqClass kWide = {4, 3072, 3, awq_w4a16_kernel<4, 3072, 3>};
// one token, K <= 4096: two or three n-tiles per workgroup (the tiles share the
// x_hat staging, so a workgroup re-reads x and 1/s once per 32 or 48 rows)
constexpr AwqClass kOne2 = {1, 4096, 2, awq_w4a16_kernel<1, 4096, 2>};
constexpr AwqClass kOne3 = {1, 4096, 3, awq_w4a16_kernel<1, 4096, 3>};
constexpr int kCus = 256;
const AwqClass* awq_class(int64_t K, int64_t rows) {
  for (const AwqClass& c : kClasses)
    if (rows <= c.rows && K <= c.kmax) return &c;
  return nullptr;
}

}  // namespace

bool awq_supported(int64_t K, int64_t M) { return awq_class(K, std::min<int64_t>(M, 16)) != nullptr; }

hipError_t launch_awq_w4a16(const uint16_t* x, const float* smooth, const uint8_t* codes,
                            const uint16_t* scales, const uint8_t* zeros, const uint16_t* bias,
                            int64_t L, int64_t M, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
  const int rows = (int)std::min<int64_t>(16, M);
  AwqArgs a{x, smooth, codes, scales, zeros, bias, y, (int)M, (int)N, (int)K, (int)(K / 64), rows};
  const AwqClass* c = awq_class(K, rows);
  if (!c) return hipErrorInvalidValue;  // excluded by the caller's awq_supported check
  const int64_t ntiles = N / 16, mtiles = (M + 15) / 16;
  // Two to four tokens: three tiles per workgroup when one tile per workgroup
  // would need more than one wave of workgroups, and always for stacked
  // launches (their grids are L times larger: 38 x 3072 -> 9216 at four tokens
  // 219 -> 163 us, at two 181 -> 149 us, HIP-graph replays on MI355X)
  if (rows > 1 && rows <= kWide.rows && K <= kWide.kmax &&
      (L > 1 || ntiles * mtiles > (int64_t)awq_occupancy(c->rows, c->kmax, 1) * kCus) &&
      (ntiles + kWide.tiles - 1) / kWide.tiles * mtiles <= (int64_t)awq_occupancy(4, 3072, 3) * kCus)
    c = &kWide;
  // One token (measured on MI355X, HIP-graph replays): stacked launches run
  // two tiles per workgroup (38 x 3072 -> 18432 276 -> 255 us, 38 x 3072 ->
  // 9216 139 -> 129 us); a single launch takes the fewest tiles per workgroup
  // (2 or 3) that bring the grid within one workgroup per CU (3072 -> 9216:
  // 3 tiles, 8.47 -> 7.93 us; 3072 -> 6144: 2 tiles, 7.26 -> 6.70 us), else
  // one (3072 -> 18432 with 2 or 3 tiles: 12.1 / 12.2 against 11.8 us).
  if (rows == 1 && K <= kOne2.kmax && c->tiles == 1) {
    if (L > 1) c = &kOne2;
    else if ((ntiles + 1) / 2 <= kCus) c = &kOne2;
    else if ((ntiles + 2) / 3 <= kCus) c = &kOne3;
  }
  const dim3 grid((unsigned)((ntiles + c->tiles - 1) / c->tiles), (unsigned)mtiles, (unsigned)L);
  hipLaunchKernelGGL(c->kernel, grid, dim3(64 * kWaves * c->tiles), 0, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
