// Call 2 of the MXFP4 variant on gfx950 for launches with at least one full
// round of 256 x 256 output tiles: block-scaled FP4 GEMM inside the matrix
// core, then the fused low-rank up-projection and the bias.
//
// Method: mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
// Nunchaku 4-Bit-Quantisierung", sections "Nunchaku Lite: Nahtlose Integration
// in Diffusers" and "Hardware-Unterstützung" (the 4-bit floating-point
// precision of the W4A4 layer); element format OCP MXFP4 (Microscaling
// Formats v1.0: E2M1 codes, one E8M0 exponent per 32 values along K).
//
// Why a second kernel.  With the block scales applied inside
// v_mfma_scale_f32_16x16x128_f8f6f4 there is no dequantization work left, so
// a 128-wide k stage costs a wave of the 128 x 128 int4 kernel only 16 MFMAs
// (256 cycles) instead of about 1000 cycles: that kernel's ring of three
// stages then covers too little memory latency, and its LDS traffic (every
// operand row is read by two waves) approaches the MFMA time.  Here:
//  * workgroup tile 256 n x 256 m, 4 waves as 2 x 2, each 128 n x 128 m =
//    4 x 4 tiles of v_mfma_scale_f32_32x32x64_f8f6f4; the 256 fp32
//    accumulators per lane live in the accumulation registers (one wave per
//    SIMD), so a stage is 32 MFMAs (1024 cycles) for 32 KB of operand data:
//    half the LDS and L2 bytes per MFMA of the 128 x 128 tile;
//  * a ring of four 128-wide k stages in LDS (32 KB each), filled by
//    global_load_lds_dwordx4 three stages ahead (four ahead, and two, were
//    slower: more requests in flight than the memory system serves well only
//    queue, fewer leave too little time), with one barrier per stage;
//  * the fragments of stage q+1 are read from LDS while the MFMAs of stage q
//    run (two register sets), so the matrix core does not wait on LDS latency;
//  * the E8M0 exponents move like the codes, 16 bytes (4 stages) per row at
//    a time, into two alternating LDS areas.  The two MFMAs of a stage take
//    the 32-blocks {h, 2 + h} (h = 0, 1): lane half p supplies block 2p + h,
//    so one 2-byte LDS read gives a lane both exponents it needs in the
//    stage, and the MFMA's byte select (h) picks one.  Any order of the
//    blocks along K, the same for both operands, gives the same dot product.
// Within a stage, 16-byte granule g of row R sits at slot 4R + (g ^ R[3:2]),
// which keeps the 16-byte fragment reads free of bank conflicts.
//
// The MFMA A operand is the weight tile (rows n), B the token tile (columns
// m), so lane l holds Y[m = l % 32][n = 8k + 4 (l / 32) + v], k, v = 0..3, of
// each 32 x 32 tile; Y leaves through LDS in 256-byte row segments.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "svdq_device.h"

namespace svdq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned int u32;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kT = 256;                 // tile edge: weight rows n and token rows m
constexpr int kThreads = 256;           // 4 waves
constexpr int kRing = 4;                // LDS stages (128 k each)
constexpr int kStage = kT * 64;         // bytes of one operand in one stage
constexpr int kExpBlock = 2 * kT * 16;  // exponents of 4 stages: 16 bytes per weight row, then per token row
constexpr int kXcds = 8;
constexpr int kBandM = 4;

struct Fp4BigArgs {
  const uint8_t* act_codes;   // u8 [M, K/2]
  const uint8_t* act_scales;  // u8 [M, K/32]
  const uint8_t* w_codes;     // u8 [N, K/2]
  const uint8_t* w_scales;    // u8 [N, K/32]
  const uint16_t* lora_act;   // bf16 [M, r]
  const uint16_t* lora_up;    // bf16 [N, r]
  const uint16_t* bias;       // bf16 [N] or null
  uint16_t* y;                // bf16 [M, N]
  int M, N, K, r, epilogue;
};

__device__ __forceinline__ u32 pack_bf16(float a, float b) {
  v2f f = {a, b};
  return __builtin_bit_cast(u32, __builtin_convertvector(f, v2bf));
}

// wait until at most n vector-memory operations of this wave are outstanding
// and all of its LDS operations are done
template <int n>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | ((n >> 4) << 14));
}

// workgroup barrier without the memory fences of __syncthreads (the waits it
// needs are explicit); the empty asm keeps LDS accesses on their side
__device__ __forceinline__ void barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* gptr, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_void*)gptr, (lds_void*)lds_wave_base, 16, 0, 0);
}

// One block-scaled FP4 MFMA, 32 x 32 x 64 (E2M1 x E2M1), the E8M0
// exponents in byte H of sa and sb.
template <int H>
__device__ __forceinline__ v16f mfma_fp4(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, H, sa, H, sb);
}

// Workgroup id -> (tile_m, tile_n).  Workgroups go round-robin over the 8
// XCDs (id % 8), each with its own L2; the ids of one XCD take one contiguous
// chunk of the tile list, ordered in bands of kBandM tile rows, so the
// workgroups an XCD runs together share few weight and token tiles.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int x = bid % kXcds;
  const int i = bid / kXcds;
  const int per = T / kXcds, rem = T % kXcds;
  const int t = x * per + min(x, rem) + i;
  const int band = t / (kBandM * tiles_n);
  const int first = band * kBandM;
  const int rows = min(tiles_m - first, kBandM);
  const int in = t - band * kBandM * tiles_n;
  tm = first + in % rows;
  tn = in / rows;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fp4_gemm_big_kernel(const Fp4BigArgs p) {
  // one LDS object per operand stage and exponent area, so the compiler sees
  // that a DMA into one cannot alias reads of another
  __shared__ __attribute__((aligned(16))) uint8_t w0[kStage], w1[kStage], w2[kStage], w3[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t a0[kStage], a1[kStage], a2[kStage], a3[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t x0[kExpBlock], x1[kExpBlock];
  auto wtile = [&](int b) -> uint8_t* { return b == 0 ? w0 : b == 1 ? w1 : b == 2 ? w2 : w3; };
  auto atile = [&](int b) -> uint8_t* { return b == 0 ? a0 : b == 1 ? a1 : b == 2 ? a2 : a3; };
  auto xarea = [&](int b) -> uint8_t* { return b == 0 ? x0 : x1; };

  const int M = p.M, N = p.N, K = p.K, r = p.r;
  const int S = K >> 7;   // k stages
  const int KB = K >> 1;  // code bytes per row
  const int KE = K >> 5;  // exponent bytes per row
  int tm, tn;
  tile_of(blockIdx.x, (M + kT - 1) / kT, (N + kT - 1) / kT, tm, tn);
  const int n0 = tn * kT;
  const int m0 = tm * kT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave >> 1;  // n half of the tile
  const int wm = wave & 1;   // m half of the tile
  const int l32 = lane & 31;
  const int lp = lane >> 5;

  // DMA role: instruction k (0..3) of a wave fills the 16-byte slots
  // s = 64 (4k + wave) + lane of each operand stage: row s >> 2, granule
  // (s & 3) ^ row[3:2].  Rows past the end repeat the last row (never stored).
  const uint8_t* wbase = p.w_codes + (size_t)n0 * (size_t)KB;
  const uint8_t* abase = p.act_codes + (size_t)m0 * (size_t)KB;
  u32 woff[4], aoff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s = 64 * (4 * k + wave) + lane;
    const int row = s >> 2;
    const u32 g = (u32)((s & 3) ^ ((row >> 2) & 3));
    woff[k] = (u32)(min(n0 + row, N - 1) - n0) * (u32)KB + 16u * g;
    aoff[k] = (u32)(min(m0 + row, M - 1) - m0) * (u32)KB + 16u * g;
  }

  // Exponents: the 16-byte run (blocks 16c .. 16c+15, i.e. stages 4c .. 4c+3)
  // of every weight row, then of every token row, moved like the codes, one
  // such block ahead into the other of two areas: 2 instructions per wave
  // for rows 64 (2 (wave & 1) + k) + lane of operand wave >> 1.
  const bool e_act = wave >= 2;
  const uint8_t* ebase = e_act ? p.act_scales + (size_t)m0 * (size_t)KE : p.w_scales + (size_t)n0 * (size_t)KE;
  const int elim = e_act ? M - 1 - m0 : N - 1 - n0;
  u32 eoff[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) eoff[k] = (u32)min(64 * (2 * (wave & 1) + k) + lane, elim) * (u32)KE;
  const int edst = (e_act ? kExpBlock / 2 : 0) + 2048 * (wave & 1);
  auto dma_stage = [&](int q, int buf) {
    const u32 col = 64u * (u32)q;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      dma16(wbase + (woff[k] + col), wtile(buf) + 1024 * (4 * k + wave));
      dma16(abase + (aoff[k] + col), atile(buf) + 1024 * (4 * k + wave));
    }
  };
  auto dma_exps = [&](int c, int area) {
#pragma unroll
    for (int k = 0; k < 2; ++k) dma16(ebase + (eoff[k] + 16u * (u32)c), xarea(area) + edst + 1024 * k);
  };

  // Fragment reads: for MFMA h of a stage, lane (l32, p) takes granule
  // 2p + h (32-block 2p + h, 32 codes) of rows 32 i + l32 of its wave's 128
  // weight rows and 128 token rows; and, for both MFMAs at once, the two
  // exponent bytes 2p, 2p + 1 of the stage's 4-byte word of the same rows.
  const int fsw = (l32 >> 2) & 3;
  int fw[2], fa[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    fw[h] = 64 * (wn * 128 + l32) + 16 * ((2 * lp + h) ^ fsw);
    fa[h] = 64 * (wm * 128 + l32) + 16 * ((2 * lp + h) ^ fsw);
  }
  const int ew = 16 * (wn * 128 + l32) + 2 * lp;
  const int ea = kExpBlock / 2 + 16 * (wm * 128 + l32) + 2 * lp;
  struct Frags {
    uint4 w[2][4], a[2][4];
    u32 sw[4], sx[4];
  };
  // stage in LDS buffer `buf`, its exponents in area `area` at stage slot s (0..3)
  auto read_stage = [&](Frags& f, int buf, int area, int s) {
    const uint8_t* wt = wtile(buf);
    const uint8_t* at = atile(buf);
    const uint8_t* et = xarea(area) + 4 * s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.sw[i] = *reinterpret_cast<const uint16_t*>(et + ew + 512 * i);
      f.sx[i] = *reinterpret_cast<const uint16_t*>(et + ea + 512 * i);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f.w[h][i] = *reinterpret_cast<const uint4*>(wt + fw[h] + 2048 * i);
        f.a[h][i] = *reinterpret_cast<const uint4*>(at + fa[h] + 2048 * i);
      }
  };

  v16f y[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) y[i][j][e] = 0.f;

  auto mfma_stage = [&](const Frags& f) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v8i wa = {(int)f.w[h][i].x, (int)f.w[h][i].y, (int)f.w[h][i].z, (int)f.w[h][i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8i ab = {(int)f.a[h][j].x, (int)f.a[h][j].y, (int)f.a[h][j].z, (int)f.a[h][j].w, 0, 0, 0, 0};
          y[i][j] = h == 0 ? mfma_fp4<0>(wa, ab, y[i][j], (int)f.sw[i], (int)f.sx[j])
                           : mfma_fp4<1>(wa, ab, y[i][j], (int)f.sw[i], (int)f.sx[j]);
        }
      }
  };

  // Stage q goes into LDS buffer q % 4, three stages ahead of its MFMAs
  // (issued in iteration q - 3), and the exponents of stages 4c .. 4c+3 into
  // area c % 2, issued right after stage 4c (in iteration 4c - 3); past the
  // end the loads repeat the last stage or block (into a buffer nobody reads
  // again), so every iteration issues the same operations and the loop body
  // has no branch.  At the top of iteration q, the wait leaves only what
  // iteration q-1 issued in flight (stage q+2, and an exponent block when
  // q % 4 == 2), which with the barrier means stage q+1 and its exponents
  // are in LDS for every wave; stage q's fragments are already in registers,
  // and stage q-1's buffer, read in iteration q-2, is free for stage q+3.
  // The fragments of stage q+1 are then
  // read while stage q's MFMAs run.  Unrolled by 8 (two exponent areas x four
  // stages), so every buffer, area and register-set index is a constant.
  Frags f[2];
  const int C = S >> 2;  // exponent blocks
  dma_stage(0, 0);
  dma_exps(0, 0);
  dma_stage(min(1, S - 1), 1);
  dma_stage(min(2, S - 1), 2);
  wait_vm_lds<16>();
  barrier();
  read_stage(f[0], 0, 0, 0);
  auto iteration = [&](int q, auto uc) {
    constexpr int u = decltype(uc)::value;  // q % 8
    // vector-memory operations issued after the ones that must have landed:
    // 8 per stage, plus 2 for an exponent block issued after them
    if constexpr ((u & 3) == 2) wait_vm_lds<10>(); else wait_vm_lds<8>();
    barrier();
    dma_stage(min(q + 3, S - 1), (u + 3) & 3);
    if constexpr ((u & 3) == 1) dma_exps(min((q >> 2) + 1, C - 1), ((u >> 2) + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    read_stage(f[(u + 1) & 1], (u + 1) & 3, ((u + 1) >> 2) & 1, (u + 1) & 3);
    mfma_stage(f[u & 1]);
    // one LDS read (8 exponent pairs first, then the 16 fragments) after
    // each of the first 24 MFMAs: the LDS delivers the next stage while the
    // matrix core works through this one
#pragma unroll
    for (int k = 0; k < 24; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int q = 0; q < S; q += 8) {  // S % 8 == 0
    iteration(q, std::integral_constant<int, 0>{});
    iteration(q + 1, std::integral_constant<int, 1>{});
    iteration(q + 2, std::integral_constant<int, 2>{});
    iteration(q + 3, std::integral_constant<int, 3>{});
    iteration(q + 4, std::integral_constant<int, 4>{});
    iteration(q + 5, std::integral_constant<int, 5>{});
    iteration(q + 6, std::integral_constant<int, 6>{});
    iteration(q + 7, std::integral_constant<int, 7>{});
  }
  wait_vm_lds<0>();  // no LDS write may land after the workgroup ends

  // fused lora_up: Y^T[n, m] += lora_up[n, :] . lora_act[m, :], bf16
  // 32 x 32 x 16 MFMAs with fragments straight from memory (L2), all loads
  // of a 32-wide rank chunk first
  if (r > 0) {
    const uint16_t* up[4];
    const uint16_t* ac[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) up[i] = p.lora_up + (size_t)min(n0 + wn * 128 + 32 * i + l32, N - 1) * r + 8 * lp;
#pragma unroll
    for (int j = 0; j < 4; ++j) ac[j] = p.lora_act + (size_t)min(m0 + wm * 128 + 32 * j + l32, M - 1) * r + 8 * lp;
    for (int k0 = 0; k0 < r; k0 += 32) {
      const int nh = min(2, (r - k0) >> 4);  // 16-wide halves in this chunk (r % 16 == 0)
      v8bf fu[2][4], fv[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = k0 + 16 * min(h, nh - 1);
          fu[h][i] = *reinterpret_cast<const v8bf*>(up[i] + k);
          fv[h][i] = *reinterpret_cast<const v8bf*>(ac[i] + k);
        }
      __builtin_amdgcn_sched_barrier(0);  // all 16 loads in flight together
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h < nh) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              y[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fu[h][i], fv[h][j], y[i][j], 0, 0, 0);
        }
      }
    }
  }

  // Bias and optional GELU in fp32, then Y goes out through LDS (the ring is
  // free now): each wave writes its 128 x 128 bf16 sub-tile as rows m of 256
  // bytes, 16-byte chunk c of row m at chunk c ^ (m % 16) (two 8-byte halves
  // per chunk from the lanes p = 0, 1), then reads it back a row segment at
  // a time, so every store instruction writes 4 rows x 256 contiguous bytes
  // instead of 32 rows x 16 bytes (a quarter of the L2 write requests).
  barrier();  // every wave has finished its last LDS reads of the ring
  uint8_t* stage_lo = wave == 0 ? w0 : wave == 1 ? w2 : wave == 2 ? a0 : a2;  // rows m 0..63
  uint8_t* stage_hi = wave == 0 ? w1 : wave == 1 ? w3 : wave == 2 ? a1 : a3;  // rows m 64..127
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int nl = 32 * i + 8 * k + 4 * lp;  // within the wave's 128 columns
      const int n = n0 + wn * 128 + nl;
      float bb4[4] = {0.f, 0.f, 0.f, 0.f};
      if (p.bias != nullptr && n < N) {
        const uint2 bb = *reinterpret_cast<const uint2*>(p.bias + n);
        bb4[0] = __builtin_bit_cast(float, bb.x << 16);
        bb4[1] = __builtin_bit_cast(float, bb.x & 0xFFFF0000u);
        bb4[2] = __builtin_bit_cast(float, bb.y << 16);
        bb4[3] = __builtin_bit_cast(float, bb.y & 0xFFFF0000u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float o4[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o4[v] = y[i][j][4 * k + v] + bb4[v];
        if (p.epilogue == kEpilogueGelu) {
#pragma unroll
          for (int v = 0; v < 4; ++v) o4[v] = gelu_tanh(o4[v]);
        }
        uint2 o;
        o.x = pack_bf16(o4[0], o4[1]);
        o.y = pack_bf16(o4[2], o4[3]);
        const int ml = 32 * (j & 1) + l32;  // row within the 64-row half
        uint8_t* dst = (j < 2 ? stage_lo : stage_hi) + ml * 256 + (((nl >> 3) ^ (ml & 15)) << 4) + 8 * lp;
        *reinterpret_cast<uint2*>(dst) = o;
      }
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __asm__ volatile("" ::: "memory");
  const int c = lane & 15;
  const int n = n0 + wn * 128 + 8 * c;
  if (n < N) {  // N % 64 == 0: n < N covers n + 7
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int ml = 4 * t + (lane >> 4);  // row within the wave's 128
      const int m = m0 + wm * 128 + ml;
      const uint4 v = *reinterpret_cast<const uint4*>((ml < 64 ? stage_lo : stage_hi) + (ml & 63) * 256 +
                                                      ((c ^ (ml & 15)) << 4));
      // streaming (non-temporal) stores: Y is not read again by this launch
      if (m < M) __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p.y + (size_t)m * N + n));
    }
  }
}

}  // namespace

int fp4_big_tiles(int64_t M, int64_t N) { return (int)(((M + kT - 1) / kT) * ((N + kT - 1) / kT)); }

hipError_t launch_fp4_gemm_big(const uint8_t* act_codes, const uint8_t* act_scales, const uint8_t* w_codes,
                               const uint8_t* w_scales, const uint16_t* lora_act, const uint16_t* lora_up,
                               const uint16_t* bias, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                               uint16_t* y, hipStream_t stream) {
  if (M <= 0 || N % 64 != 0 || K % 1024 != 0 || epilogue == kEpilogueQkv) return hipErrorInvalidValue;
  const Fp4BigArgs a{act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, y,
                     (int)M, (int)N, (int)K, (int)r, epilogue};
  hipLaunchKernelGGL(fp4_gemm_big_kernel, dim3(fp4_big_tiles(M, N)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace svdq
