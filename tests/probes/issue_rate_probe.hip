// Issue-rate probe for the two GEMM designs of call 2 on MI355X (gfx950).
// Not part of the library or the tests: a measurement program whose printed
// figures back the performance ceilings stated for the kernels.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature \
//         -Xclang -packed-fp32-ops tests/probes/issue_rate_probe.hip -o /tmp/issue_rate_probe
//   /tmp/issue_rate_probe
//
// Every wave of a full-chip launch (256 workgroups x 4 waves per SIMD group)
// runs a fixed loop; each line gives the shader-clock cycles per loop
// iteration (clock64 over the loop, averaged over the waves), the shader clock
// itself (clock64 against the 100 MHz wall clock) and, for MFMA-only loops,
// the chip-wide rate.
//  * int4 design: one v_mfma_i32_16x16x64_i8 against 8 independent fp32 FMAs
//    (the dequantization of one 16x16 tile is 8 FMAs per lane), alone and
//    interleaved in one wave, at 1, 2 and 4 waves per SIMD;
//  * MXFP4 design: independent block-scaled v_mfma_scale_f32_16x16x128 and
//    32x32x64 with E2M1 operands (and 16x16x128 with FP8 for comparison).
// Operands are opaque to the compiler (empty asm), so no MFMA is folded.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define CK(x)                                                                                 \
  do {                                                                                        \
    hipError_t e_ = (x);                                                                      \
    if (e_ != hipSuccess) {                                                                   \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);             \
      return 1;                                                                               \
    }                                                                                         \
  } while (0)

enum Mode { kI8Mfma = 0, kFma = 1, kI8MfmaFma = 2, kFp4_16 = 3, kFp4_32 = 4, kFp8_16 = 5 };

// per iteration: kI8Mfma 4 MFMAs; kFma 32 FMAs; kI8MfmaFma 4 MFMAs + 32 FMAs
// (1 MFMA then 8 FMAs); kFp4_16 / kFp8_16 16 MFMAs; kFp4_32 8 MFMAs
template <int MODE>
__global__ __launch_bounds__(512) void probe(int iters, float* out, long long* cyc, long long* wall) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  v4i a0 = {lane, lane * 3, lane ^ 5, 7}, b = {lane * 7, 1, 2, lane};
  v4i a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3;
  v4i acc0 = {0, 0, 0, 0}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
  v8i fa = {lane, lane + 1, lane + 2, lane + 3, 0, 0, 0, 0};
  v8i fb = {lane * 3, lane + 7, lane ^ 5, lane + 11, 0, 0, 0, 0};
  v4f q[16];
  v16f r[4];
#pragma unroll
  for (int k = 0; k < 16; ++k) q[k] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) r[k][e] = 0.f;
  float f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = lane * 0.001f + i;
  const float s = 1.0001f, t = 0.999f;
  const long long t0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
    __asm__ volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b), "+v"(fa), "+v"(fb));
    if constexpr (MODE == kI8Mfma) {
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b, acc3, 0, 0, 0);
    } else if constexpr (MODE == kFma) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = fmaf(f[i], s, t);
    } else if constexpr (MODE == kI8MfmaFma) {
      acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(f[i], s, t);
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc1, 0, 0, 0);
#pragma unroll
      for (int i = 8; i < 16; ++i) f[i] = fmaf(f[i], s, t);
      acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b, acc2, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = fmaf(f[i], s, t);
      acc3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b, acc3, 0, 0, 0);
#pragma unroll
      for (int i = 8; i < 16; ++i) f[i] = fmaf(f[i], s, t);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    } else if constexpr (MODE == kFp4_16 || MODE == kFp8_16) {
      constexpr int fmt = MODE == kFp4_16 ? 4 : 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) q[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, q[k], fmt, fmt, 0, 127, 0, 126);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, r[k], 4, 4, 0, 127, 0, 126);
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, r[k], 4, 4, 0, 127, 0, 126);
    }
  }
  const long long t1 = clock64(), w1 = wall_clock64();
  float sum = (float)(acc0[0] + acc1[1] + acc2[2] + acc3[3]);
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += f[i] + q[i][0];
#pragma unroll
  for (int k = 0; k < 4; ++k) sum += r[k][0] + r[k][15];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (lane == 0) {
    cyc[blockIdx.x * 8 + wave] = t1 - t0;
    wall[blockIdx.x * 8 + wave] = w1 - w0;
  }
}

// waves per SIMD w: 256 threads per workgroup for w = 1, else 512 threads and
// w / 2 workgroups per CU; mfma_per_iter / flops_per_mfma give the chip rate
template <int MODE>
int run(const char* name, int w, int iters, int cus, int mfma_per_iter, double flops_per_mfma) {
  const int threads = w >= 2 ? 512 : 256;
  const int blocks = cus * (w >= 2 ? w / 2 : 1);
  float* out;
  long long *cyc, *wall;
  CK(hipMalloc(&out, sizeof(float) * blocks * threads));
  CK(hipMalloc(&cyc, sizeof(long long) * blocks * 8));
  CK(hipMalloc(&wall, sizeof(long long) * blocks * 8));
  CK(hipMemset(cyc, 0, sizeof(long long) * blocks * 8));
  hipLaunchKernelGGL(probe<MODE>, dim3(blocks), dim3(threads), 0, 0, 10, out, cyc, wall);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  CK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(probe<MODE>, dim3(blocks), dim3(threads), 0, 0, iters, out, cyc, wall);
  CK(hipGetLastError());
  CK(hipEventRecord(e1, 0));
  CK(hipEventSynchronize(e1));
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, e0, e1));
  std::vector<long long> c(blocks * 8), wl(blocks * 8);
  CK(hipMemcpy(c.data(), cyc, sizeof(long long) * blocks * 8, hipMemcpyDeviceToHost));
  CK(hipMemcpy(wl.data(), wall, sizeof(long long) * blocks * 8, hipMemcpyDeviceToHost));
  double cs = 0, ws = 0;
  int n = 0;
  for (int i = 0; i < blocks * 8; ++i)
    if (c[i] > 0) {
      cs += (double)c[i];
      ws += (double)wl[i];
      ++n;
    }
  const double mhz = cs / (ws / 100.0);  // the wall clock runs at 100 MHz
  std::printf("%-30s waves/SIMD=%d  cycles/iter=%7.1f  clock=%5.0f MHz", name, w, cs / n / iters, mhz);
  if (mfma_per_iter > 0)
    std::printf("  chip=%6.0f TFLOP/s", flops_per_mfma * mfma_per_iter * iters * (double)blocks * threads / 64.0 /
                                             (ms * 1e-3) / 1e12);
  std::printf("\n");
  CK(hipFree(out));
  CK(hipFree(cyc));
  CK(hipFree(wall));
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return 0;
}

int main() {
  int cus = 0;
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  std::printf("compute units: %d\n", cus);
  const int it = 20000;
  for (int w : {1, 2, 4}) {
    if (run<kI8Mfma>("int8 16x16x64 MFMA x4", w, it, cus, 4, 32768.0)) return 1;
    if (run<kFma>("fp32 FMA x32", w, it, cus, 0, 0.0)) return 1;
    if (run<kI8MfmaFma>("int8 MFMA x4 + FMA x32 (1:8)", w, it, cus, 4, 32768.0)) return 1;
  }
  for (int w : {1, 2}) {
    if (run<kFp4_16>("FP4 scaled 16x16x128 x16", w, it / 2, cus, 16, 65536.0)) return 1;
    if (run<kFp4_32>("FP4 scaled 32x32x64 x8", w, it / 2, cus, 8, 131072.0)) return 1;
    if (run<kFp8_16>("FP8 scaled 16x16x128 x16", w, it / 2, cus, 16, 65536.0)) return 1;
  }
  return 0;
}
