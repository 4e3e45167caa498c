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
// consecutive n of one token row m; the epilogue stages each wave's sub-tile
// in LDS so that Y leaves in 128-byte row runs.
//
// Data movement.  The packed int4 codes go from memory straight into LDS with
// global_load_lds_dwordx4 (no registers involved), two quant groups at a time:
// each instruction moves 64 contiguous bytes of each of 16 rows.  Runs of 32
// bytes per row halve what the L2 delivers (measured on the whole chip: about
// 7 TB/s against 14 TB/s for 64-byte runs), so a ring stage holds a pair of
// groups (128 rows x 64 bytes per operand).  Pairs q+1 and q+2 are in flight
// while pair q is computed, with one barrier per pair.  Vector-memory counters
// retire in issue order, so the wait for stage q is an explicit
// s_waitcnt vmcnt(4): the four DMAs of the next pair, issued last in every
// iteration, may stay in flight.  Inside a stage, the 16-byte granule gg (0..3)
// of row r sits at slot 4r + (gg ^ r[2:1]).  An 8-byte fragment read of a
// 16-lane phase (16 rows, one 8-byte piece of each) then finds no two lanes on
// one bank pair: a 64-byte stage row covers 16 of the 32 four-byte banks, so a
// piece's bank pair is set by r[0], the granule slot (r[2:1]) and its half in
// the granule, and the half is r[3] because of the int4 storage order of the
// codes (rows with bit 3 set hold the two 8-byte halves of every 16-byte
// granule exchanged; calls 1 and the packer write them so).  With the plain
// order and a granule swizzle alone, rows r and r + 8 met on every bank pair,
// which no swizzle of whole 16-byte DMA granules avoids.  The 16-byte reads of
// the MXFP4 variant (8-lane phases) are conflict-free with the same swizzle.
// Each thread owns the scales of one token or weight row and
// reads them three group pairs at a time (one 16-byte buffer load), ahead of
// the pairs' DMAs, then stores the converted scales of pair q+1 into the
// second of two scale areas.  The epilogue reads the lora_up and lora_act
// fragments straight from memory (they are L2-resident), which keeps the LDS
// at 52 KB per workgroup.
//
// Main loop, per 64-wide group g and wave (64 n x 64 m, 4 x 4 MFMA tiles):
//  * fragments: 8-byte LDS reads; nibbles widened to int8 as 16*q with
//    (x & 0xF0F0F0F0) and ((x << 4) & 0xF0F0F0F0), identically for weights and
//    activations, so the K permutation this introduces cancels in the dot
//    products; the products are 256 * q_x * q_w.
//  * MFMA: v_mfma_i32_16x16x64_i8 covers one whole group per instruction.  Its
//    C operand is the constant 0x4B400000 (the bits of 1.5 * 2^23), so the int32
//    result read as fp32 is exactly 1.5 * 2^23 + 256 * acc (|256 acc| <= 802816
//    < 2^22): the int->float conversion is free.
//  * dequant: t = fma(F, s_x/256, -1.5*2^23 * s_x/256) = fl32(acc * s_x) exactly
//    (s_x is bf16, so both constants are exact), then y = fma(t, s_w, y); each
//    MFMA is followed by the 8 FMAs of the previous tile.
// The int32 group accumulator itself is exact; the debug variant of this
// kernel stores (bits - 0x4B400000) >> 8 instead of dequantizing.
//
// Workgroup: 256 threads (4 waves as 2 x 2), tile 128 n x 128 m, under 168
// VGPRs, so three workgroups fit a CU; the launch picks two or three per CU
// from the tile count.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "svdq_device.h"

namespace svdq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32;
typedef u32 v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kBN = 128;            // weight rows (n) per workgroup
constexpr int kBM = 128;            // token rows (m) per workgroup
constexpr int kThreads = 256;
constexpr int kStages = 3;          // LDS ring depth, in group pairs
constexpr int kTile = 128 * 64;     // packed bytes of one operand tile for one group pair
constexpr int kScale = 512;         // floats per stage: per group, s_x/256 (128) and s_w (128)
constexpr int kStaticLds = kStages * 2 * kTile + 2 * 4 * kScale;  // 3 tile stages, 2 scale areas
constexpr int kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr u32 kNib = 0xF0F0F0F0u;
// Few tokens go to the few-token kernel up to 64 (one token chunk), and up to
// 160 for layers of at most 2^24 weights; measured on MI355X (rocprofv3):
// 3072 -> 12288 at 96 / 128 / 160 tokens 30.6 / 33.4 / 44.9 us there against
// 25.4 / 25.6 / 35.4 us on the tiled kernel with K-splits, 12288 -> 3072 at 128
// tokens 33.8 against 32.5 us, while 3072 -> 3072 stays faster there up to 160
// tokens (16.4 against 19.8 us) and every shape at 64 tokens (19.2 against 25.0
// us for 3072 -> 12288).
constexpr int64_t kSkinnyMaxM = 160;
bool skinny_preferred(int64_t M, int64_t N, int64_t K) {
  return M <= 64 || (M <= kSkinnyMaxM && N * K <= ((int64_t)1 << 24));
}

__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

// Slot p (0..127) of the token-scale arrays -> token m of the tile.  Lane l of
// wave column wm reads slots wm*64 + 4*(l%16) + j (j = 0..3), i.e. the tokens
// m = wm*64 + 16j + l%16 it owns, as one contiguous 16-byte LDS read.
__device__ __forceinline__ int sx_token(int p) {
  return (p >> 6) * 64 + (p & 3) * 16 + ((p >> 2) & 15);
}

// wait until at most n vector-memory operations of this wave are outstanding
// (and, with kLds, until all of its LDS operations are done)
template <int n, bool kLds>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | ((kLds ? 0 : 0xF) << 8) | ((n >> 4) << 14));
}

// workgroup barrier without the memory fences of __syncthreads (the waits it
// needs are explicit above); the empty asm keeps LDS accesses on their side
__device__ __forceinline__ void barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* gptr, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)gptr, (lds_void*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ v4i widen(uint2 p) {
  return v4i{(int)((p.x << 4) & kNib), (int)(p.x & kNib), (int)((p.y << 4) & kNib), (int)(p.y & kNib)};
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
  int acc_m_lo, acc_m_hi, acc_n_lo, acc_n_hi;  // dump window (kDump)
  int M, N, K, r;
  int epilogue;  // kEpilogueNone, kEpilogueGelu (after the bias) or kEpilogueQkv
  QkvEpilogue qkv;
  int splits;         // K-splits per tile (gridDim.y); > 1 needs part and count
  float* part;        // fp32 partial sub-tiles [tiles][splits][4 waves][16][4][64]
  uint32_t* count;    // arrival counters [tiles][4 waves], zero between launches
  // Tail split (whole >= 0, one-dimensional grid): workgroups [0, whole) run
  // the first `whole` tiles of the list unsplit, and each later tile runs as
  // `tsplit` workgroups, one per K-split; partials and counters are indexed
  // by the tile's place after `whole` ([tail tiles][tsplit][4 waves]...).
  int whole, tsplit;
};

// Workgroup id -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs (id % 8), each XCD with its own L2.  The ids of one XCD are mapped
// onto one contiguous chunk of the tile list, and the tile list is ordered in
// bands of kBandM tile rows, so the tiles an XCD runs at the same time share a
// few activation tiles and a few weight tiles in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kBandM = 8;
__device__ __forceinline__ int xcd_pos(int bid, int T) {
  const int x = bid % kXcds;
  const int i = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  return x * per + min(x, rem) + i;
}
// position t of the tile list -> (tile_m, tile_n)
__device__ __forceinline__ void tile_at(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int band = t / (kBandM * tiles_n);
  const int first = band * kBandM;
  const int rows = min(tiles_m - first, kBandM);
  const int in = t - band * kBandM * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

// kOcc: waves per SIMD the register budget is sized for (main kernel); the
// accumulator-dump test hook uses 1 so it never spills.  kFp4: the MXFP4
// variant (codes are E2M1 nibbles, scales E8M0 bytes per 32-block); a ring
// stage (128 k) is then one v_mfma_scale_f32_16x16x128_f8f6f4 per tile, the
// block scales applied inside the matrix core, with no dequantization work.
template <bool kDump, int kOcc, bool kFp4 = false>
__global__ __launch_bounds__(kThreads, kOcc) void w4a4_gemm_kernel(const GemmArgs<kDump> p) {
  // One LDS object per operand tile and scale area of every ring stage: the
  // compiler then sees that a DMA in flight into one object cannot alias the
  // accesses to another and waits only for the DMA a read really depends on,
  // instead of draining the ring before every LDS access.
  __shared__ __attribute__((aligned(16))) uint8_t w0[kTile], w1[kTile], w2[kTile];
  __shared__ __attribute__((aligned(16))) uint8_t a0[kTile], a1[kTile], a2[kTile];
  __shared__ __attribute__((aligned(16))) float s0[kScale], s1[kScale];
  extern __shared__ __attribute__((aligned(16))) uint8_t lora_smem[];  // 2 per CU only
  auto wtile = [&](int buf) -> uint8_t* { return buf == 0 ? w0 : buf == 1 ? w1 : w2; };
  auto atile = [&](int buf) -> uint8_t* { return buf == 0 ? a0 : buf == 1 ? a1 : a2; };
  auto sarea = [&](int buf) -> float* { return buf == 0 ? s0 : s1; };

  const int M = p.M, N = p.N, K = p.K, r = p.r;
  const int G = K >> 6;
  const int P = (G + 1) >> 1;  // group pairs
  // Which tile and K-split this workgroup runs: with a uniform split, tile
  // blockIdx.x (in XCD order) and split blockIdx.y of p.splits; with a tail
  // split, the first p.whole workgroups run whole tiles and the rest run the
  // later tiles p.tsplit workgroups each.  `sub0` indexes the tile's partials
  // and counters.  Workgroup (tile, split) runs pairs [qb, qb + Pl) of the
  // tile (splits == 1: the whole K); pair indices below are local to it.
  const int tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
  const int bid = blockIdx.x;
  int pos, split, nsplit;
  size_t sub0;
  if (p.whole < 0) {
    pos = xcd_pos(bid, tiles_m * tiles_n);
    split = blockIdx.y;
    nsplit = p.splits;
    sub0 = (size_t)bid * 4;
  } else if (bid < p.whole) {
    pos = xcd_pos(bid, p.whole);
    split = 0;
    nsplit = 1;
    sub0 = 0;
  } else {
    const int u = bid - p.whole;
    pos = p.whole + u / p.tsplit;
    split = u - (pos - p.whole) * p.tsplit;
    nsplit = p.tsplit;
    sub0 = (size_t)(pos - p.whole) * 4;
  }
  const int qb = (int)(((long)split * P) / nsplit);
  const int Pl = (int)(((long)(split + 1) * P) / nsplit) - qb;
  const int KB = K >> 1;       // bytes per packed row
  int tm, tn;
  tile_at(pos, tiles_m, tiles_n, tm, tn);
  const int n0 = tn * kBN;
  const int m0 = tm * kBM;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1;  // n half of the tile
  const int wm = wave & 1;   // m half of the tile
  const int l16 = lane & 15;
  const int lseg = lane >> 4;

  // DMA role: instruction k (0, 1) of a wave fills slots 256k + 64*wave + lane
  // of each operand tile, i.e. row s >> 2, granule (s & 3) ^ r[2:1]: four lanes
  // cover the 64 bytes of one row.  The workgroup's first row is a 64-bit base
  // pointer; lane offsets within its 128 rows fit 32 bits for every K.
  const uint8_t* wbase = p.w_codes + (size_t)n0 * (size_t)KB;
  const uint8_t* abase = p.act_codes + (size_t)m0 * (size_t)KB;
  u32 woff[2], aoff[2], gsel[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = 256 * k + 64 * wave + lane;
    const int row = s >> 2;
    gsel[k] = (u32)((s & 3) ^ ((row >> 1) & 3));
    woff[k] = (u32)(min(n0 + row, N - 1) - n0) * (u32)KB + 16u * (gsel[k] & 1u);
    aoff[k] = (u32)(min(m0 + row, M - 1) - m0) * (u32)KB + 16u * (gsel[k] & 1u);
  }
  // group pair q -> stage buffer buf (the second group clamped to the last one)
  auto dma_pair = [&](int q, int buf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32 col = 32u * (u32)min(2 * (qb + q) + (int)(gsel[k] >> 1), G - 1);
      dma16(wbase + (woff[k] + col), wtile(buf) + 4096 * k + 1024 * wave);
      dma16(abase + (aoff[k] + col), atile(buf) + 4096 * k + 1024 * wave);
    }
  };

  // Fragment read offsets for the first group of a pair: row R, granule
  // lseg >> 1, 8-byte half (lseg & 1) ^ R[3] (the storage order).  The rows of
  // fragment i (R + 16i) share R[3:1] of R = wX*64 + l16, and the second group
  // of the pair sits 32 bytes away (granule + 2 flips bit 1 of the slot):
  // offset ^ 32.
  const int fsw = (l16 >> 1) & 3;
  const int fw = 64 * (wn * 64 + l16) + 16 * ((lseg >> 1) ^ fsw) + 8 * ((lseg & 1) ^ ((l16 >> 3) & 1));
  const int fa = 64 * (wm * 64 + l16) + 16 * ((lseg >> 1) ^ fsw) + 8 * ((lseg & 1) ^ ((l16 >> 3) & 1));

  // scale role: threads 0..127 (waves 0, 1) -> token slot tid, 128..255 ->
  // weight row tid-128 (wave-uniform, so the buffer resource below is scalar)
  const bool s_is_act = wave < 2;
  const int s_idx = s_is_act ? tid : tid - kBM;
  // The thread's row of scales is read 3 group pairs at a time: one load
  // instruction per wave every 3 pairs instead of two 2-byte gathers per pair
  // (each instruction touches 64 rows, whatever it moves per lane).  With an
  // odd group count a row starts 2 bytes into a dword, so 16 bytes are read
  // from the dword boundary below and each pair's dword is realigned.  A
  // buffer load bounded by the end of the scale array returns zeros past it
  // (the last block of a row may run into the next row or past the array;
  // those groups are never used).  The wave-uniform base is the workgroup's
  // first row; offsets within fit 32 bits.
  const uint16_t* sbase = s_is_act ? p.act_scales + (size_t)m0 * (size_t)G : p.w_scales + (size_t)n0 * (size_t)G;
  const u32 soff = (u32)(s_is_act ? min(m0 + (kFp4 ? s_idx : sx_token(s_idx)), M - 1) - m0
                                  : min(n0 + s_idx, N - 1) - n0) * (u32)G * 2u;
  // bytes from sbase to the end of the array, rounded up to a whole dword: the
  // range check drops any dword that reaches past it, and with an odd group
  // count the array ends 2 bytes into a dword (whose other half is never used;
  // an aligned dword never crosses a page)
  const size_t s_left = (2 * (size_t)G * (size_t)(s_is_act ? M - m0 : N - n0) + 3) & ~(size_t)3;
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(sbase), (short)0, (int)min(s_left, (size_t)0x7FFFFFFF), 0x00020000);
  const u32 sshift = (soff & 2u) * 8u;  // 0, or 16 bits for a row that starts mid-dword
  // register ring of raw scales: block c (pairs 3c .. 3c+2 of the split,
  // pair d in bits [32d + sshift, 32d + sshift + 32): group 2q in the low
  // half) in slot c % 2
  v4u sblk[2];
  auto load_scales = [&](int c, int slot) {
    if (kDump) return;
    sblk[slot] = __builtin_amdgcn_raw_buffer_load_b128(srsrc, (int)((soff & ~3u) + 4u * (u32)(qb + 3 * c)), 0, 0);
  };
  // converted scales of pair q (block slot `slot`, dword d) -> stage buffer
  // `buf`: per group h, s_x/256 of the token slot (floats 256h + 0..127) or
  // s_w of the weight row (256h + 128..255)
  auto put_scale = [&](int slot, int d, int buf) {
    if (kDump) return;
    u32 o = 4u * (u32)(s_is_act ? s_idx : 128 + s_idx);
    __asm__ volatile("" : "+v"(o));  // keeps the per-stage addresses out of registers
    uint8_t* sp = reinterpret_cast<uint8_t*>(sarea(buf)) + o;
    const u32 w = __builtin_amdgcn_alignbit(sblk[slot][d + 1], sblk[slot][d], sshift);
    if constexpr (kFp4) {
      // the row's four E8M0 bytes of the stage (blocks 4q .. 4q+3), as loaded
      *reinterpret_cast<u32*>(sp) = w;
      return;
    }
    const float f0 = __builtin_bit_cast(float, w << 16);
    const float f1 = __builtin_bit_cast(float, w & 0xFFFF0000u);
    *reinterpret_cast<float*>(sp) = s_is_act ? f0 * (1.0f / 256.0f) : f0;
    *reinterpret_cast<float*>(sp + 1024) = s_is_act ? f1 * (1.0f / 256.0f) : f1;
  };

  // With 2 workgroups per CU the LDS has room for the lora tiles: they are
  // loaded at kernel start (before anything else, so every later wait covers
  // them) and the epilogue does not wait for memory.
  constexpr bool kLoraLds = !kDump && kOcc <= 2;
  if (kLoraLds && r > 0) {
    const int tile_bytes = kBN * r * 2;  // same for lora_act (kBM == kBN)
    for (int off = 1024 * wave; off < tile_bytes; off += 4096) {
      const int byte = off + 16 * lane;
      const int row = byte / (2 * r), col = byte - row * 2 * r;
      dma16(reinterpret_cast<const uint8_t*>(p.lora_up) + (size_t)min(n0 + row, N - 1) * 2 * r + col,
            lora_smem + off);
      dma16(reinterpret_cast<const uint8_t*>(p.lora_act) + (size_t)min(m0 + row, M - 1) * 2 * r + col,
            lora_smem + tile_bytes + off);
    }
  }

  v4f y[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) y[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i magic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  // Operand fragments (packed) and scales of one group, read from LDS.
  struct GroupRegs {
    uint2 w[4], a[4];
    v4f sx, sw[4];
  };
  // group h (0, 1) of the pair in tile stage `buf` and scale area `sbuf`
  auto read_group = [&](GroupRegs& d, int buf, int sbuf, int h) {
    const uint8_t* wt = wtile(buf);
    const uint8_t* at = atile(buf);
#pragma unroll
    for (int i = 0; i < 4; ++i) d.w[i] = *reinterpret_cast<const uint2*>(wt + (fw ^ (32 * h)) + 1024 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) d.a[j] = *reinterpret_cast<const uint2*>(at + (fa ^ (32 * h)) + 1024 * j);
    if constexpr (!kDump) {
      const float* sp = sarea(sbuf) + 256 * h;
      d.sx = *reinterpret_cast<const v4f*>(sp + wm * 64 + l16 * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) d.sw[i] = *reinterpret_cast<const v4f*>(sp + 128 + wn * 64 + 16 * i + 4 * lseg);
    }
  };
  // one group g from its registers
  auto compute = [&](const GroupRegs& d, int g) {
    v4i wf[4], af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[i] = widen(d.w[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) af[j] = widen(d.a[j]);
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
            const int a = acc[v];
            if (m >= p.acc_m_lo && m < p.acc_m_hi && n >= p.acc_n_lo && n < p.acc_n_hi)
              p.acc[((size_t)(m - p.acc_m_lo) * (size_t)(p.acc_n_hi - p.acc_n_lo) + (size_t)(n - p.acc_n_lo)) * G + g] =
                  (a - kMagicBits) >> 8;
          }
        }
    } else {
      (void)g;
      const v4f sx = d.sx;
      const v4f sc = sx * -kMagic;
      auto dequant = [&](int i, int j, const v4i acc) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // element copied to a scalar first: a bit-cast applied directly to
          // an ext-vector element is lowered as a cast of element 0
          const int bits = acc[v];
          const float t = fmaf(__int_as_float(bits), sx[j], sc[j]);
          y[i][j][v] = fmaf(t, d.sw[i][v], y[i][j][v]);
        }
      };
      // each tile is dequantized two MFMAs after its own, so its result has
      // long landed when the FMAs read it
      v4i p2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[0], af[0], magic, 0, 0, 0);
      v4i p1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[0], af[1], magic, 0, 0, 0);
#pragma unroll
      for (int idx = 2; idx < 16; ++idx) {
        const int i = idx >> 2, j = idx & 3;
        const v4i cur = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[i], af[j], magic, 0, 0, 0);
        dequant((idx - 2) >> 2, (idx - 2) & 3, p2);
        p2 = p1;
        p1 = cur;
      }
      dequant(3, 2, p2);
      dequant(3, 3, p1);
      // the accumulators are complete here: keeps the compiler from deferring
      // the dequant FMAs past the next barrier (which doubles the live registers)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) __asm__ volatile("" : "+v"(y[i][j]));
      // keep the MFMA pipe fed while the VALU dequantizes: 1 MFMA, then 8 FMAs
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
  };
  // One pair: with registers to spare (2 workgroups per CU) both groups' LDS
  // reads are issued up front, so the second group's land during the first
  // one's compute; under the 3-per-CU register budget each group reads its own.
  // MXFP4 stage: lane (l16, lseg) reads k-block lseg of its rows (granule
  // lseg, 16 bytes = 32 codes) and the rows' E8M0 byte of that block
  const int fw4 = 64 * (wn * 64 + l16) + 16 * (lseg ^ fsw);
  const int fa4 = 64 * (wm * 64 + l16) + 16 * (lseg ^ fsw);
  auto compute_stage_fp4 = [&](int buf, int sbuf) {
    const uint8_t* wt = wtile(buf);
    const uint8_t* at = atile(buf);
    const uint8_t* sp = reinterpret_cast<const uint8_t*>(sarea(sbuf));
    uint4 wq[4], aq[4];
    int sw[4], sx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wq[i] = *reinterpret_cast<const uint4*>(wt + fw4 + 1024 * i);
      sw[i] = sp[4 * (128 + wn * 64 + 16 * i + l16) + lseg];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      aq[j] = *reinterpret_cast<const uint4*>(at + fa4 + 1024 * j);
      sx[j] = sp[4 * (wm * 64 + 16 * j + l16) + lseg];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8i wa = {(int)wq[i].x, (int)wq[i].y, (int)wq[i].z, (int)wq[i].w, 0, 0, 0, 0};
        const v8i ab = {(int)aq[j].x, (int)aq[j].y, (int)aq[j].z, (int)aq[j].w, 0, 0, 0, 0};
        y[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa, ab, y[i][j], 4, 4, 0, sw[i], 0, sx[j]);
      }
  };
  auto compute_pair = [&](int buf, int sbuf, int q) {
    if constexpr (kFp4) {
      compute_stage_fp4(buf, sbuf);
      (void)q;
      return;
    }
    const int g0 = 2 * (qb + q);
    const bool two = g0 + 1 < G;
    if constexpr (kOcc <= 2) {
      GroupRegs d0, d1;
      read_group(d0, buf, sbuf, 0);
      if (two) read_group(d1, buf, sbuf, 1);
      compute(d0, g0);
      if (two) compute(d1, g0 + 1);
    } else {
      GroupRegs d;
      read_group(d, buf, sbuf, 0);
      compute(d, g0);
      if (two) {
        read_group(d, buf, sbuf, 1);
        compute(d, g0 + 1);
      }
    }
  };

  // Prologue, in issue order: scale block 0 (pairs 0-2), pair 0, pair 1.
  // Iteration q issues scale block q/3 + 1 when q % 3 == 0 and, last, the 4
  // DMAs of pair q+2, so at the top of iteration q the wait for pair q (4
  // younger operations, 5 after an iteration that loaded a block) also covers
  // every block that put_scale can ask for there.
  load_scales(0, 0);
  dma_pair(0, 0);
  dma_pair(min(1, Pl - 1), 1);
  wait_vm<8, false>();  // block 0
  put_scale(0, 0, 0);

  // Iteration q: stage q complete (own loads: vmcnt, everyone's: barrier);
  // every third pair, the next scale block goes into the ring slot the block
  // before has freed; pair q+2 starts loading into the stage freed by pair
  // q-1; the scales of pair q+1 are staged into the scale area pair q-1 has
  // freed; pair q is computed.  The body is unrolled over 6 pairs (3 tile
  // stages x 2 scale areas x 2 scale blocks) so every LDS buffer and
  // register index is a compile-time constant.
  for (int q0 = 0; q0 < Pl; q0 += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int q = q0 + u;
      if (!kDump && (u == 1 || u == 4)) wait_vm<5, true>(); else wait_vm<4, true>();
      barrier();
      if (u % 3 == 0) load_scales((q / 3) + 1, (u / 3 + 1) % 2);
      dma_pair(min(q + 2, Pl - 1), (u + 2) % 3);
      put_scale(((u + 1) / 3) % 2, (u + 1) % 3, (u + 1) % 2);
      if (q < Pl) compute_pair(u % 3, u % 2, q);
    }
  }
  wait_vm<0, true>();
  // every wave is done with the ring stages before any wave stages its Y
  // tile there (after this point a wave may leave early: K-split partials)
  barrier();

  if constexpr (!kDump) {
    // K-split: each wave reduces its own 64 x 64 sub-tile.  It stores its fp32
    // partial with agent-coherent stores (visible across the XCDs' L2s without
    // a cache-wide write-back), waits for them, and bumps the sub-tile's
    // counter; the wave that arrives last loads the other partials the same
    // way, adds all of them in split order (the result does not depend on
    // timing) and runs the epilogue.  The counter wraps back to zero.
    if (nsplit > 1) {
      const size_t sub = sub0 + wave;
      float* mine = p.part + ((sub * nsplit + split) << 12);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            __hip_atomic_store(mine + (((i * 4 + j) * 4 + v) << 6) + lane, y[i][j][v], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the partial is visible to the agent
      __asm__ volatile("" ::: "memory");
      u32 old = 0;
      if (lane == 0) old = atomicInc(p.count + sub, (u32)(nsplit - 1));
      old = __shfl(old, 0);
      if (old != (u32)(nsplit - 1)) return;  // another split of this sub-tile is still running
      __asm__ volatile("" ::: "memory");
      // two halves of the sub-tile (n tiles i = 2h, 2h + 1); per half, the
      // partials of two splits are loaded together (64 loads in flight) and
      // added in split order
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4f acc[2][4];
        for (int s0 = 0; s0 < nsplit; s0 += 2) {
          v4f t[2][2][4];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int s2 = min(s0 + e, nsplit - 1);
            const float* src = p.part + ((sub * nsplit + s2) << 12);
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
              for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  t[e][ii][j][v] = __hip_atomic_load(src + ((((2 * h + ii) * 4 + j) * 4 + v) << 6) + lane,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int s2 = s0 + e;
            if (s2 < nsplit) {
#pragma unroll
              for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const v4f v = (s2 == split) ? y[2 * h + ii][j] : t[e][ii][j];
                  acc[ii][j] = (s2 == 0) ? v : acc[ii][j] + v;
                }
            }
          }
        }
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < 4; ++j) y[2 * h + ii][j] = acc[ii][j];
      }
    }
    // fused lora_up: Y^T[n, m] += lora_up[n, :] . lora_act[m, :], fragments
    // from the LDS tiles, or else straight from memory (L2), all loads of a
    // 32-wide rank chunk first
    if (r > 0) {
      const uint16_t* up[4];
      const uint16_t* ac[4];
      const uint16_t* lu = reinterpret_cast<const uint16_t*>(lora_smem);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        up[i] = kLoraLds ? lu + (wn * 64 + 16 * i + l16) * r
                         : p.lora_up + (size_t)min(n0 + wn * 64 + 16 * i + l16, N - 1) * r;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ac[j] = kLoraLds ? lu + kBN * r + (wm * 64 + 16 * j + l16) * r
                         : p.lora_act + (size_t)min(m0 + wm * 64 + 16 * j + l16, M - 1) * r;
      int k0 = 0;
      for (; k0 + 32 <= r; k0 += 32) {
        v8bf fu[4], fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fu[i] = *reinterpret_cast<const v8bf*>(up[i] + k0 + 8 * lseg);
#pragma unroll
        for (int j = 0; j < 4; ++j) fa[j] = *reinterpret_cast<const v8bf*>(ac[j] + k0 + 8 * lseg);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) y[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fu[i], fa[j], y[i][j], 0, 0, 0);
      }
      if (k0 < r) {
        v4bf fu[4], fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fu[i] = *reinterpret_cast<const v4bf*>(up[i] + k0 + 4 * lseg);
#pragma unroll
        for (int j = 0; j < 4; ++j) fa[j] = *reinterpret_cast<const v4bf*>(ac[j] + k0 + 4 * lseg);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) y[i][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fu[i], fa[j], y[i][j], 0, 0, 0);
      }
    }
    // Fused QKV epilogue on a Q or K tile.  The 128 columns of the tile are one
    // head (tiles and thirds are 128-aligned), held by the two waves of a wave
    // row: sum of squares per token over the lane's 16 channels, then over the
    // 4 lanes of the token (lane xor 16, 32), then over the two waves through
    // the free scale area; then scale, learned weight and the pair rotation.
    const int third = (p.epilogue == kEpilogueQkv) ? n0 / (N / 3) : 2;  // workgroup-uniform
    if (p.epilogue == kEpilogueQkv && third < 2) {
      const uint16_t* nw = third == 0 ? p.qkv.q_norm : p.qkv.k_norm;
      float wgt[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * 64 + 16 * i + 4 * lseg;
        const int nl = wn * 64 + 16 * i + 4 * lseg;
        float bb4[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.bias != nullptr) {
          const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
          bb4[0] = __builtin_bit_cast(float, bb.x << 16);
          bb4[1] = __builtin_bit_cast(float, bb.x & 0xFFFF0000u);
          bb4[2] = __builtin_bit_cast(float, bb.y << 16);
          bb4[3] = __builtin_bit_cast(float, bb.y & 0xFFFF0000u);
        }
        const uint2 ww = *reinterpret_cast<const uint2*>(nw + nl);
        wgt[i][0] = __builtin_bit_cast(float, ww.x << 16);
        wgt[i][1] = __builtin_bit_cast(float, ww.x & 0xFFFF0000u);
        wgt[i][2] = __builtin_bit_cast(float, ww.y << 16);
        wgt[i][3] = __builtin_bit_cast(float, ww.y & 0xFFFF0000u);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) y[i][j][v] += bb4[v];
      }
      float ss[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) a = fmaf(y[i][j][v], y[i][j][v], a);
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        ss[j] = a;
      }
      float* red = s0;  // the scale areas are free once every wave has left the loop
      barrier();
      if (lseg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wn * 128 + wm * 64 + 16 * j + l16] = ss[j];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float tot = ss[j] + red[(1 - wn) * 128 + wm * 64 + 16 * j + l16];
        ss[j] = 1.0f / sqrtf(tot * (1.0f / 128.0f) + p.qkv.eps);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wn * 64 + 16 * i + 4 * lseg;
        const int pair = (wn * 64 + 16 * i + 4 * lseg) >> 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + wm * 64 + 16 * j + l16;
          const size_t t = (size_t)min(m, M - 1) * 64 + pair;
          const float2 c = *reinterpret_cast<const float2*>(p.qkv.cos + t);
          const float2 sn = *reinterpret_cast<const float2*>(p.qkv.sin + t);
          float z[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) z[v] = y[i][j][v] * ss[j] * wgt[i][v];
          if (m < M) {
            uint2 o;
            o.x = pack_bf16(z[0] * c.x - z[1] * sn.x, z[0] * sn.x + z[1] * c.x);
            o.y = pack_bf16(z[2] * c.y - z[3] * sn.y, z[2] * sn.y + z[3] * c.y);
            *reinterpret_cast<uint2*>(p.y + (size_t)m * N + n) = o;
          }
        }
      }
      return;
    }
    // Bias and optional GELU in fp32, then Y goes out through LDS (this
    // wave's ring stage, free since the barrier after the main loop): the wave
    // writes its 64 x 64 bf16 sub-tile as rows m of 128 bytes, 16-byte chunk
    // c of row m at chunk c ^ (m % 8), and reads it back so that each store
    // instruction writes 8 rows x 128 contiguous bytes instead of 16 rows x
    // 32 bytes.  N % 64 == 0, so the wave's 64 columns are all in range or
    // all out of it.
    uint8_t* stg = wave == 0 ? w0 : wave == 1 ? w1 : wave == 2 ? w2 : a0;
    const int nw = n0 + wn * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nl = 16 * i + 4 * lseg;  // within the wave's 64 columns
      float bb4[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr && nw < N) {
        const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + nw + nl);
        bb4[0] = __builtin_bit_cast(float, bb.x << 16);
        bb4[1] = __builtin_bit_cast(float, bb.x & 0xFFFF0000u);
        bb4[2] = __builtin_bit_cast(float, bb.y << 16);
        bb4[3] = __builtin_bit_cast(float, bb.y & 0xFFFF0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float o4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o4[v] = y[i][j][v] + bb4[v];
        if (p.epilogue == kEpilogueGelu) {
#pragma unroll
          for (int v = 0; v < 4; ++v) o4[v] = gelu_tanh(o4[v]);
        }
        uint2 o;
        o.x = pack_bf16(o4[0], o4[1]);
        o.y = pack_bf16(o4[2], o4[3]);
        const int ml = 16 * j + l16;  // row within the wave's 64
        *reinterpret_cast<uint2*>(stg + ml * 128 + (((nl >> 3) ^ (ml & 7)) << 4) + 8 * (lseg & 1)) = o;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __asm__ volatile("" ::: "memory");
    if (nw < N) {
      const int c = lane & 7;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ml = 8 * t + (lane >> 3);
        const int m = m0 + wm * 64 + ml;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + ml * 128 + ((c ^ (ml & 7)) << 4));
        // streaming (non-temporal) stores: Y is not read again by this launch
        if (m < M)
          __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p.y + (size_t)m * N + nw + 8 * c));
      }
    }
  }
}

// Workgroups per CU: the kernel fits 3 (under 168 VGPRs, 52 KB of LDS each),
// which retires about 16 % more tiles per unit time than 2, but the tile
// count then quantizes over 3 x CUs slots instead of 2 x CUs (measured on the
// 4608 x 3072 x 12288 and 4608 x 12288 x 3072 linears).  Pick the one with
// fewer rounds x time per round; 2 per CU is enforced by padding the LDS.
int pick_occupancy(int tiles, int cus) {
  const long r2 = (tiles + 2L * cus - 1) / (2L * cus);
  const long r3 = (tiles + 3L * cus - 1) / (3L * cus);
  return (r3 * 260 < r2 * 200) ? 3 : 2;
}

// K-splits per tile.  A launch runs in rounds of 3 workgroups per CU; a last,
// partial round with r workgroups takes a fraction of a full round that
// depends on how many share a CU (1: 0.55, 2: 0.7, 3: 1).  A workgroup costs
// its group pairs plus a fixed overhead (pipeline fill and epilogue, about 2
// pairs; with splits also the fp32 partial write and the in-order reduction,
// about 4 + S/2 pairs).  The split count with the least estimated time wins.
// Fitted to forced-split sweeps on MI355X (rocprofv3 kernel times, S = 1..12):
// 512 x 3072 -> 3072 (96 tiles) best at S = 4 (25.3 us; S = 2: 27.0), 192 tiles
// of 256 x 3072 -> 12288 and 1024 x 3072 -> 3072 best at S = 2 (35.8 and 35.4
// us; S = 4: 39.0 and 36.7), 512 x 12288 -> 3072 at S = 8 (53.8 us; S = 1:
// 131), 384 tiles equal at S = 1 and 2.
// rounds of `units` workgroups over 3 slots per CU, the last one partial
double split_rounds(long units, int cus) {
  const long slots = 3L * cus;
  const long full = units / slots;
  const long rest = units - full * slots;
  const long load = (rest + cus - 1) / cus;
  return (double)full + (load == 0 ? 0.0 : load == 1 ? 0.55 : load == 2 ? 0.7 : 1.0);
}
double split_cost(int pairs, int S) { return (double)pairs / S + (S == 1 ? 2.0 : 4.0 + 0.5 * S); }

int pick_splits(int tiles, int pairs, int cus) {
  auto est = [&](int S) { return split_cost(pairs, S) * split_rounds((long)tiles * S, cus); };
  int best = 1;
  double bt = est(1);
  for (int S = 2; S <= std::min(pairs, 16); S *= 2) {  // the measured counts (odd ones leave the
    const double t = est(S);                                 // 6-pair unrolled loop partly idle)
    if (t < bt * 0.97) {  // a split has to win clearly
      bt = t;
      best = S;
    }
  }
  return best;
}

// Tail split: the tiles of the first round run unsplit and only the tiles
// after it are split in two, which fills the second round without the
// partial traffic of a uniform split.  Returns 2, or 0 where it does not beat
// `uniform_cost` clearly.  Only for launches of one full round
// and a partial one: measured on MI355X, 864 tiles of 4608 x 3072 -> 3072 run
// 9-11 % faster (102-104 -> 93-96 us), while after 3 or 4 full rounds
// (4608 x 3072 -> 9216 and -> 12288) a split tail was 1-2 % slower, the
// workgroups having drifted apart by then.
int pick_tail_split(int tiles, int pairs, int cus, double uniform_cost) {
  const long slots = 3L * cus;
  const long whole = (tiles / slots) * slots;
  const long tail = tiles - whole;
  if (whole != slots || tail == 0) return 0;
  // two parts per tail tile, the measured configuration
  const double t = split_cost(pairs, 1) + split_cost(pairs, 2) * split_rounds(tail * 2, cus);
  return t < uniform_cost * 0.97 ? 2 : 0;
}

std::atomic<int> g_splits{0};  // test hook (0 = automatic)
std::atomic<int> g_path{0};    // test hook: 0 = by shape, 1 = tiled, 2 = few-token kernel
std::atomic<int> g_fp4_tile{0};  // test hook: 0 = by shape, 128, 256

// How call 2 runs a shape on the current device.
struct GemmPlan {
  bool skinny;  // the few-token kernel
  bool big;     // MXFP4 on 256 x 256 tiles
  int tiles;    // 128 x 128 output tiles (tiled kernel)
  int splits;   // K-splits per tile (uniform split)
  int occ;      // workgroups per CU the tiled kernel is built for (2 or 3)
  int whole;    // tail split: tiles run unsplit (-1: uniform split)
  int tsplit;   // tail split: K-splits of each later tile
  int wgs() const { return whole < 0 ? tiles * splits : whole + (tiles - whole) * tsplit; }
};

GemmPlan gemm_plan(int64_t M, int64_t N, int64_t K, int epilogue, bool fp4) {
  GemmPlan g{false, false, (int)(((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM)), 1, 3, -1, 1};
  const int path = g_path.load(std::memory_order_relaxed);
  if (!fp4 && epilogue != kEpilogueQkv && path != 1 && skinny_supported(M, N, K) &&
      (path == 2 || skinny_preferred(M, N, K))) {
    g.skinny = true;
    return g;
  }
  const int cus = current_cus();
  // MXFP4: 256 x 256 tiles once there are at least a quarter as many as CUs
  // (measured on MI355X: 96 tiles of 512 x 3072 -> 12288 and 216 tiles of
  // 4608 x 12288 -> 3072 run 1.2x and 2.2x faster than 128 x 128 tiles with
  // K-splits; 24 tiles of 512 x 3072 -> 3072 and 48 of 1024 x 12288 -> 3072
  // run 1.8x and 1.4x slower); the test hooks can force either, and a forced
  // split count forces the 128 x 128 kernel
  if (fp4 && K % 1024 == 0 && g_splits.load(std::memory_order_relaxed) == 0) {
    const int tile = g_fp4_tile.load(std::memory_order_relaxed);
    if (tile == 256 || (tile == 0 && 4 * fp4_big_tiles(M, N) >= cus)) {
      g.big = true;
      return g;
    }
  }
  const int pairs = (int)((K / 64 + 1) / 2);
  if (epilogue != kEpilogueQkv) {
    const int forced = g_splits.load(std::memory_order_relaxed);
    g.splits = forced > 0 ? std::min(forced, pairs) : pick_splits(g.tiles, pairs, cus);
    if ((size_t)g.tiles * 4 > kWsMaxCounters) g.splits = 1;  // one workspace counter per wave sub-tile
    if (forced == 0) {
      const int St = pick_tail_split(g.tiles, pairs, cus,
                                     split_cost(pairs, g.splits) * split_rounds((long)g.tiles * g.splits, cus));
      if (St > 0) {
        g.splits = 1;
        g.whole = (int)((g.tiles / (3L * cus)) * 3L * cus);
        g.tsplit = St;
      }
    }
  }
  // a tail split assumes the whole tiles fill exactly one round of 3 per CU
  g.occ = g.whole >= 0 ? 3 : pick_occupancy(g.wgs(), cus);
  return g;
}

// K-split partials: one arrival counter per wave sub-tile, and per tile and
// split four 64 x 64 fp32 sub-tiles.
size_t split_counters(const GemmPlan& g) {
  if (g.whole >= 0) return (size_t)(g.tiles - g.whole) * 4;
  return g.splits > 1 ? (size_t)g.tiles * 4 : 0;
}
size_t split_bytes(const GemmPlan& g) {
  if (g.whole >= 0) return (size_t)(g.tiles - g.whole) * g.tsplit * 4 * 4096 * 4;
  return g.splits > 1 ? (size_t)g.tiles * g.splits * 4 * 4096 * 4 : 0;
}

template <bool kDump, bool kFp4 = false>
hipError_t launch(GemmArgs<kDump> a, const GemmPlan& g, Workspace ws, hipStream_t stream) {
  auto kern = w4a4_gemm_kernel<kDump, kDump ? 1 : 3, kFp4>;
  size_t pad = 0;
  a.splits = kDump ? 1 : g.splits;
  a.whole = kDump ? -1 : g.whole;
  a.tsplit = g.tsplit;
  if constexpr (!kDump) {
    const size_t nc = split_counters(g);
    if (nc > 0) {
      if (ws.bytes < ws_bytes(nc, split_bytes(g))) return hipErrorInvalidValue;
      a.count = ws_counters(ws);
      a.part = static_cast<float*>(ws_scratch(ws));
    }
    if (g.occ == 2) {
      kern = w4a4_gemm_kernel<kDump, 2, kFp4>;
      // the lora tiles, and at least enough that only 2 workgroups fit a CU
      pad = max((size_t)(80 * 1024 - kStaticLds), (size_t)2 * kBN * a.r * 2);
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)pad);
      if (e != hipSuccess) return e;
    }
  }
  const dim3 grid = a.whole >= 0 ? dim3(g.wgs(), 1) : dim3(g.tiles, a.splits);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), pad, stream, a);
  return hipGetLastError();
}

// Fixed device scratch of the no-allocation entry point: a counter region and
// partial sums, as in a caller's workspace.  Each device holds its own copy
// until the process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

__global__ void clear_counters(uint32_t* c, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) c[i] = 0;
}

constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
  void* ptr = nullptr;  // device address of `scratch` on that device
  bool cleared = false; // counters cleared by an eager (not captured) launch
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxScratchDevices];

// The current device's scratch as a workspace; the first use on a device
// looks up its address and clears the counter region on `stream` (a fill
// kernel: captured into a graph, it runs before the call on every replay,
// and a later eager call clears once more).
hipError_t static_workspace(hipStream_t stream, Workspace* ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (sl.ptr == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    sl.ptr = p;
  }
  if (!sl.cleared) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return e;
    const int n = (int)(kWsCounterBytes / 4);
    hipLaunchKernelGGL(clear_counters, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(sl.ptr),
                       n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (cs == hipStreamCaptureStatusNone) sl.cleared = true;
  }
  *ws = Workspace{sl.ptr, kStaticScratchBytes};
  return hipSuccess;
}

}  // namespace

hipError_t launch_w4a4_gemm_lora_up_static(const uint8_t* act_codes, const uint16_t* act_scales,
                                           const uint8_t* w_codes, const uint16_t* w_scales,
                                           const uint16_t* lora_act, const uint16_t* lora_up,
                                           const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                                           int epilogue, uint16_t* y, hipStream_t stream) {
  if (gemm_workspace_bytes(M, N, K, r, epilogue, false) > kStaticScratchBytes) return hipErrorInvalidValue;
  Workspace ws;
  hipError_t e = static_workspace(stream, &ws);
  if (e != hipSuccess) return e;
  return launch_w4a4_gemm_lora_up(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, r,
                                  epilogue, nullptr, y, DumpWindow{}, ws, stream);
}

void set_gemm_path_override(int path) { g_path.store(path, std::memory_order_relaxed); }

void set_fp4_tile_override(int tile) { g_fp4_tile.store(tile, std::memory_order_relaxed); }

void set_gemm_splits_override(int splits) { g_splits.store(std::max(0, splits), std::memory_order_relaxed); }

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r, int epilogue, bool fp4) {
  (void)r;
  if (M <= 0) return 0;
  const GemmPlan g = gemm_plan(M, N, K, epilogue, fp4);
  if (g.skinny || g.big) return 0;
  return ws_bytes(split_counters(g), split_bytes(g));
}

hipError_t launch_fp4_gemm_lora_up(const uint8_t* act_codes, const uint8_t* act_scales,
                                  const uint8_t* w_codes, const uint8_t* w_scales,
                                  const uint16_t* lora_act, const uint16_t* lora_up,
                                  const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                                  int epilogue, uint16_t* y, Workspace ws, hipStream_t stream) {
  if (K % 128 != 0 || epilogue == kEpilogueQkv) return hipErrorInvalidValue;
  const GemmPlan g = gemm_plan(M, N, K, epilogue, true);
  if (g.big)
    return launch_fp4_gemm_big(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, r,
                               epilogue, y, stream);
  // the E8M0 byte pairs of a 64-group travel like the int4 path's bf16 scale
  GemmArgs<false> a{act_codes, reinterpret_cast<const uint16_t*>(act_scales), w_codes,
                    reinterpret_cast<const uint16_t*>(w_scales), lora_act, lora_up, bias,
                    y, nullptr, 0, 0, 0, 0, (int)M, (int)N, (int)K, (int)r, epilogue, QkvEpilogue{}, 1,
                    nullptr, nullptr, -1, 1};
  return launch<false, true>(a, g, ws, stream);
}

hipError_t launch_w4a4_gemm_lora_up(const uint8_t* act_codes, const uint16_t* act_scales,
                                    const uint8_t* w_codes, const uint16_t* w_scales,
                                    const uint16_t* lora_act, const uint16_t* lora_up,
                                    const uint16_t* bias, int64_t M, int64_t N, int64_t K,
                                    int64_t r, int epilogue, const QkvEpilogue* qkv, uint16_t* y,
                                    const DumpWindow& dump, Workspace ws, hipStream_t stream) {
  // Few tokens: the 128 x 128 tile grid leaves most CUs idle; the K-split
  // kernel streams the weights with every CU instead.
  const GemmPlan g = gemm_plan(M, N, K, epilogue, false);
  if (g.skinny)
    return launch_w4a4_gemm_skinny(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up,
                                   bias, M, N, K, r, epilogue, y, dump, stream);
  if (dump.acc != nullptr) {
    GemmArgs<true> a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                     y, dump.acc, dump.m_lo, dump.m_hi, dump.n_lo, dump.n_hi, (int)M, (int)N, (int)K, 0,
                     kEpilogueNone, QkvEpilogue{}, 1, nullptr, nullptr, -1, 1};
    return launch<true>(a, g, Workspace{}, stream);
  }
  GemmArgs<false> a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                    y, nullptr, 0, 0, 0, 0, (int)M, (int)N, (int)K, (int)r, epilogue, QkvEpilogue{}, 1,
                    nullptr, nullptr, -1, 1};
  if (epilogue == kEpilogueQkv) {
    if (qkv == nullptr || N % 384 != 0) return hipErrorInvalidValue;
    a.qkv = *qkv;
  }
  return launch<false>(a, g, ws, stream);
}

}  // namespace svdq
