// Launch and read floors of MI355X (gfx950) for the few-token kernels.
// Not part of the library or the tests: a measurement program whose printed
// figures back the floors stated for the weight-streaming kernels (the
// few-token GEMM, the AWQ W4A16 linear) and for call 1's activation stream.
//
//   hipcc --offload-arch=gfx950 -O3 -std=c++17 -Xclang -target-feature \
//         -Xclang -packed-fp32-ops tests/probes/read_floor_probe.hip -o /tmp/read_floor_probe
//   /tmp/read_floor_probe
//
// Three kernels, each timed over 50 back-to-back launches with HIP events
// (average per launch, launch gaps included) and meant to be run under
// rocprofv3 --kernel-trace --stats as well (kernel durations alone):
//  * empty: workgroups of 256 threads that do nothing (the cost of a launch
//    and of dispatching its waves);
//  * rows<R, D>: the weight-stream pattern of the few-token kernels.  A
//    workgroup of 4 waves owns 16R rows of `row_bytes` bytes; its waves split
//    each row's 64-byte pieces; lane (l % 16, l / 16) reads 16 bytes of row
//    l % 16 of each 16-row tile, so an instruction reads 64 contiguous bytes
//    of 16 rows; D instructions per tile in flight;
//  * flat<D>: the same bytes read as contiguous 1 KB per wave instruction,
//    grid-stride over the buffer, D instructions in flight.
// Every launch reads a different buffer of a set larger than the 256 MB
// last-level cache, so the bytes come from HBM.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

__global__ __launch_bounds__(256) void empty_kernel(unsigned* out, int never) {
  if ((int)threadIdx.x == never) out[blockIdx.x] = 0;  // never true: never >= 256
}

template <int R, int D>
__global__ __launch_bounds__(256) void rows_kernel(const uint8_t* w, int row_bytes, unsigned* out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lq = lane >> 4;
  const size_t r0 = (size_t)blockIdx.x * 16 * R;
  const int P = row_bytes / 64;  // 64-byte pieces per row
  const int pb = P * wave / 4, pe = P * (wave + 1) / 4;
  unsigned acc = 0;
  uint4 ring[D][R];
  for (int p0 = pb; p0 < pe; p0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int i = 0; i < R; ++i)
        ring[d][i] = *reinterpret_cast<const uint4*>(w + (r0 + 16 * i + l16) * (size_t)row_bytes +
                                                     64 * (size_t)min(p0 + d, pe - 1) + 16 * lq);
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int i = 0; i < R; ++i) acc ^= ring[d][i].x ^ ring[d][i].y ^ ring[d][i].z ^ ring[d][i].w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int D>
__global__ __launch_bounds__(256) void flat_kernel(const uint8_t* w, size_t chunks, unsigned* out) {
  const int lane = threadIdx.x & 63;
  const size_t wid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6), nw = (size_t)gridDim.x * 4;
  unsigned acc = 0;
  uint4 ring[D];
  for (size_t c0 = wid; c0 < chunks; c0 += nw * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const size_t c = c0 + nw * d < chunks ? c0 + nw * d : c0;
      ring[d] = *reinterpret_cast<const uint4*>(w + c * 1024 + 16 * lane);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) acc ^= ring[d].x ^ ring[d].y ^ ring[d].z ^ ring[d].w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

struct Bufs {
  std::vector<uint8_t*> p;
  size_t bytes = 0;
};

template <typename F>
int timeit(const char* name, size_t bytes, const Bufs& b, F launch) {
  for (int i = 0; i < 4; ++i) launch(b.p[i % b.p.size()]);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const int reps = 50;
  CK(hipEventRecord(e0, 0));
  for (int i = 0; i < reps; ++i) launch(b.p[(i + 4) % b.p.size()]);
  CK(hipEventRecord(e1, 0));
  CK(hipEventSynchronize(e1));
  CK(hipGetLastError());
  float ms = 0.f;
  CK(hipEventElapsedTime(&ms, e0, e1));
  const double us = ms * 1e3 / reps;
  if (bytes > 0)
    std::printf("%-44s %8.2f us  %6.2f TB/s\n", name, us, (double)bytes / us / 1e6);
  else
    std::printf("%-44s %8.2f us\n", name, us);
  CK(hipEventDestroy(e0));
  CK(hipEventDestroy(e1));
  return 0;
}

int main() {
  int cus = 0;
  CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  std::printf("compute units: %d\n", cus);
  // the largest stream (call 1's X at 4608 x 3072 bf16) in a rotation above 256 MB
  const size_t max_bytes = (size_t)4608 * 3072 * 2;
  Bufs b;
  b.bytes = max_bytes;
  for (int i = 0; i < 12; ++i) {
    uint8_t* q = nullptr;
    CK(hipMalloc(&q, max_bytes));
    CK(hipMemset(q, 1, max_bytes));
    b.p.push_back(q);
  }
  unsigned* out = nullptr;
  CK(hipMalloc(&out, (size_t)16 << 20));

  for (int g : {256, 1024, 2048}) {
    char name[64];
    std::snprintf(name, sizeof name, "empty grid=%d x 256", g);
    if (timeit(name, 0, b, [&](uint8_t*) { hipLaunchKernelGGL(empty_kernel, dim3(g), dim3(256), 0, 0, out, 1 << 20); }))
      return 1;
  }
  struct RowCase {
    const char* what;
    int rows, row_bytes;
  };
  // weight codes: few-token GEMM 3072 -> 12288 and AWQ 3072 -> 9216, 3072 -> 18432
  const RowCase rc[] = {{"weights 12288 x 1536 B", 12288, 1536},
                        {"weights 9216 x 1536 B", 9216, 1536},
                        {"weights 18432 x 1536 B", 18432, 1536}};
  for (const RowCase& c : rc) {
    const size_t bytes = (size_t)c.rows * c.row_bytes;
    char name[96];
#define SVDQ_ROWS(R, D)                                                                               \
  std::snprintf(name, sizeof name, "rows R=%d D=%d grid=%d %s", R, D, c.rows / (16 * R), c.what);       \
  if (c.rows % (16 * R) == 0 &&                                                                       \
      timeit(name, bytes, b, [&](uint8_t* w) {                                                        \
        hipLaunchKernelGGL((rows_kernel<R, D>), dim3(c.rows / (16 * R)), dim3(256), 0, 0, w, c.row_bytes, out); \
      }))                                                                                             \
    return 1;
    SVDQ_ROWS(1, 3)
    SVDQ_ROWS(1, 6)
    SVDQ_ROWS(3, 3)
    SVDQ_ROWS(3, 6)
#undef SVDQ_ROWS
    for (int g : {cus, 4 * cus}) {
      std::snprintf(name, sizeof name, "flat D=4 grid=%d %s", g, c.what);
      if (timeit(name, bytes, b, [&](uint8_t* w) {
            hipLaunchKernelGGL((flat_kernel<4>), dim3(g), dim3(256), 0, 0, w, bytes / 1024, out);
          }))
        return 1;
    }
  }
  // call 1's activation stream, contiguous
  for (int g : {cus, 4 * cus}) {
    char name[96];
    std::snprintf(name, sizeof name, "flat D=4 grid=%d X 4608 x 3072 bf16", g);
    if (timeit(name, max_bytes, b, [&](uint8_t* w) {
          hipLaunchKernelGGL((flat_kernel<4>), dim3(g), dim3(256), 0, 0, w, max_bytes / 1024, out);
        }))
      return 1;
  }
  for (uint8_t* q : b.p) CK(hipFree(q));
  CK(hipFree(out));
  return 0;
}
