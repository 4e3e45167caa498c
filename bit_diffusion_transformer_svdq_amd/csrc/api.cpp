// C ABI of libsvdq (declarations and the contract: include/svdq.h).
//
// Every entry point validates its arguments before touching the HIP runtime,
// so shape and pointer errors are reported synchronously and also on a machine
// without a GPU.  The device check mirrors the load-time GPU validation of the
// integration described on mind-verse.de ("Effiziente Optimierung von
// Diffusionsmodellen durch Nunchaku 4-Bit-Quantisierung", section
// "Hardware-Unterstützung"): unsupported GPU generations are refused.

#include <cmath>
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstddef>
#include <initializer_list>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "svdq.h"
#include "svdq_internal.h"

namespace {

thread_local char g_err[512] = {0};

svdq_status fail(svdq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

svdq_status ok() {
  g_err[0] = 0;
  return SVDQ_STATUS_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxDevices = 64;
// 0 = unknown, otherwise 1 + svdq_status
std::atomic<int> g_dev_state[kMaxDevices];

svdq_status check_device_uncached(int device) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(SVDQ_STATUS_NO_DEVICE, "no HIP device visible (%s)", hipGetErrorString(e));
  }
  if (device < 0 || device >= count)
    return fail(SVDQ_STATUS_INVALID_VALUE, "device index %d out of range [0, %d)", device, count);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SVDQ_STATUS_ARCH_MISMATCH, "device %d is %s; this library is built for gfx950 (MI355X)",
                device, prop.gcnArchName);
  return ok();
}

svdq_status check_current_device() {
  int dev = 0;
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(SVDQ_STATUS_NO_DEVICE, "no HIP device visible");
  }
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
  return svdq_check_device(dev);
}

bool rank_supported(int64_t r) { return r >= 0 && r <= 128 && r % 16 == 0; }

// A device byte range an entry point reads or writes.  Inputs may share memory
// with each other; an output may share memory with nothing else the call
// touches (the kernels read inputs while other workgroups already write).
struct Span {
  const void* p;
  size_t n;
  const char* name;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

svdq_status check_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (auto i = ins.begin(); i != ins.end(); ++i)
      if (overlap(*o, *i)) return fail(SVDQ_STATUS_INVALID_VALUE, "output %s overlaps input %s", o->name, i->name);
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return fail(SVDQ_STATUS_INVALID_VALUE, "outputs %s and %s overlap", o->name, o2->name);
  }
  return SVDQ_STATUS_SUCCESS;
}

// A call that needs `need` bytes of workspace gets them from the caller.
svdq_status check_workspace(const void* ws, size_t ws_bytes, size_t need, const char* query) {
  if (need == 0) return SVDQ_STATUS_SUCCESS;
  if (!ws) return fail(SVDQ_STATUS_INVALID_VALUE, "this shape needs a workspace of %zu bytes (%s)", need, query);
  if (ws_bytes < need)
    return fail(SVDQ_STATUS_INVALID_VALUE, "workspace of %zu bytes, this shape needs %zu (%s)", ws_bytes, need, query);
  if (!aligned16(ws)) return fail(SVDQ_STATUS_INVALID_VALUE, "workspace must be 16-byte aligned");
  return SVDQ_STATUS_SUCCESS;
}

size_t sz(int64_t a, int64_t b = 1, int64_t c = 1) { return (size_t)a * (size_t)b * (size_t)c; }

}  // namespace

namespace svdq {
int current_cus() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}
}  // namespace svdq

extern "C" {

const char* svdq_status_string(svdq_status s) {
  switch (s) {
    case SVDQ_STATUS_SUCCESS: return "SVDQ_STATUS_SUCCESS";
    case SVDQ_STATUS_INVALID_VALUE: return "SVDQ_STATUS_INVALID_VALUE";
    case SVDQ_STATUS_NOT_SUPPORTED: return "SVDQ_STATUS_NOT_SUPPORTED";
    case SVDQ_STATUS_ARCH_MISMATCH: return "SVDQ_STATUS_ARCH_MISMATCH";
    case SVDQ_STATUS_NO_DEVICE: return "SVDQ_STATUS_NO_DEVICE";
    case SVDQ_STATUS_HIP_ERROR: return "SVDQ_STATUS_HIP_ERROR";
    case SVDQ_STATUS_INTERNAL: return "SVDQ_STATUS_INTERNAL";
  }
  return "SVDQ_STATUS_UNKNOWN";
}

const char* svdq_last_error(void) { return g_err; }

int svdq_version(void) { return 200; }

svdq_status svdq_check_device(int device) {
  if (device < 0) return fail(SVDQ_STATUS_INVALID_VALUE, "negative device index %d", device);
  if (device < kMaxDevices) {
    const int st = g_dev_state[device].load(std::memory_order_acquire);
    if (st != 0) {
      const svdq_status s = static_cast<svdq_status>(st - 1);
      if (s == SVDQ_STATUS_SUCCESS) return ok();
      return fail(s, "device %d failed the gfx950 check earlier", device);
    }
  }
  const svdq_status s = check_device_uncached(device);
  if (device < kMaxDevices && (s == SVDQ_STATUS_SUCCESS || s == SVDQ_STATUS_ARCH_MISMATCH))
    g_dev_state[device].store(1 + static_cast<int>(s), std::memory_order_release);
  return s;
}

static svdq_status validate_quant(int64_t M, int64_t K, int64_t r, int64_t group_size) {
  if (M < 0 || K <= 0 || r < 0 || group_size <= 0)
    return fail(SVDQ_STATUS_INVALID_VALUE, "bad dims M=%lld K=%lld r=%lld group_size=%lld",
                (long long)M, (long long)K, (long long)r, (long long)group_size);
  if (group_size != 64) return fail(SVDQ_STATUS_NOT_SUPPORTED, "group_size %lld (only 64)", (long long)group_size);
  if (K % 64 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "K=%lld is not a multiple of 64", (long long)K);
  if (!rank_supported(r)) return fail(SVDQ_STATUS_NOT_SUPPORTED, "rank %lld (need 0..128, multiple of 16)", (long long)r);
  if (M > (1ll << 24) || K > (1ll << 20) || M * K > (1ll << 40))
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "problem too large M=%lld K=%lld", (long long)M, (long long)K);
  // K beyond 64 groups is always split over workgroups, one workspace counter per 16 rows
  if (r > 0 && K > 64 * 64 && (size_t)((M + 15) / 16) > svdq::kWsMaxCounters)
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "M=%lld with K=%lld > 4096 and r > 0 (at most %zu rows)", (long long)M,
                (long long)K, svdq::kWsMaxCounters * 16);
  return SVDQ_STATUS_SUCCESS;
}

static svdq_status quantize_common(const void* x, const float* smooth, const void* lora_down,
                                   int64_t M, int64_t K, int64_t r, int64_t group_size,
                                   void* act_codes, void* act_scales, void* lora_act, bool fp4,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  svdq_status s = validate_quant(M, K, r, group_size);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (M == 0) return ok();  // empty batch: nothing is read or written, pointers may be null
  if (!x || !smooth || !act_codes || !act_scales)
    return fail(SVDQ_STATUS_INVALID_VALUE, "null x/smooth/act_codes/act_scales");
  if (r > 0 && (!lora_down || !lora_act))
    return fail(SVDQ_STATUS_INVALID_VALUE, "r=%lld needs lora_down and lora_act", (long long)r);
  if (!aligned16(x) || !aligned16(smooth) || !aligned16(act_codes) || !aligned16(act_scales) ||
      (r > 0 && (!aligned16(lora_down) || !aligned16(lora_act))))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  const size_t need = svdq::quant_workspace_bytes(M, K, r);
  s = check_workspace(workspace, workspace_bytes, need, "svdq_quantize_act_workspace_size");
  if (s != SVDQ_STATUS_SUCCESS) return s;
  const Span ws{need ? workspace : nullptr, need, "workspace"};
  s = check_disjoint({{act_codes, sz(M, K / 2), "act_codes"},
                      {act_scales, fp4 ? sz(M, K / 32) : sz(M, K / 64, 2), "act_scales"},
                      {r > 0 ? lora_act : nullptr, sz(M, r, 2), "lora_act"}, ws},
                     {{x, sz(M, K, 2), "x"}, {smooth, sz(K, 4), "smooth"},
                      {r > 0 ? lora_down : nullptr, sz(r, K, 2), "lora_down"}});
  if (s != SVDQ_STATUS_SUCCESS) return s;
  s = check_current_device();
  if (s != SVDQ_STATUS_SUCCESS) return s;
  hipError_t e = svdq::launch_quant_lora_down(
      static_cast<const uint16_t*>(x), smooth, static_cast<const uint16_t*>(lora_down), M, K, r,
      static_cast<uint8_t*>(act_codes), static_cast<uint16_t*>(act_scales),
      static_cast<uint16_t*>(lora_act), fp4, svdq::Workspace{workspace, workspace_bytes},
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

size_t svdq_quantize_act_workspace_size(int64_t M, int64_t K, int64_t r) {
  if (validate_quant(M, K, r, 64) != SVDQ_STATUS_SUCCESS || M == 0) return 0;
  return svdq::quant_workspace_bytes(M, K, r);
}

svdq_status svdq_quantize_act_lora_down(const void* x, const float* smooth, const void* lora_down,
                                        int64_t M, int64_t K, int64_t r, int64_t group_size,
                                        void* act_codes, void* act_scales, void* lora_act,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_common(x, smooth, lora_down, M, K, r, group_size, act_codes, act_scales, lora_act, false,
                         workspace, workspace_bytes, stream);
}

svdq_status svdq_quantize_act_lora_down_fp4(const void* x, const float* smooth, const void* lora_down,
                                            int64_t M, int64_t K, int64_t r, void* act_codes,
                                            void* act_scales, void* lora_act, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (K > 0 && K % 128 != 0)
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  return quantize_common(x, smooth, lora_down, M, K, r, 64, act_codes, act_scales, lora_act, true,
                         workspace, workspace_bytes, stream);
}

svdq_status svdq_debug_set_quant_plan(int k_blocks, int tiles_per_wg) {
  if (k_blocks < 0 || tiles_per_wg < 0 || tiles_per_wg > 12)
    return fail(SVDQ_STATUS_INVALID_VALUE, "bad plan k_blocks=%d tiles_per_wg=%d (need >= 0, tiles <= 12)",
                k_blocks, tiles_per_wg);
  svdq::set_quant_plan_override(k_blocks, tiles_per_wg);
  return ok();
}

svdq_status svdq_debug_set_quant_waves(int waves) {
  if (waves < 0 || waves > 8) return fail(SVDQ_STATUS_INVALID_VALUE, "bad wave count %d (0..8)", waves);
  svdq::set_quant_waves_override(waves);
  return ok();
}

svdq_status svdq_debug_set_gemm_path(int path) {
  if (path < 0 || path > 2) return fail(SVDQ_STATUS_INVALID_VALUE, "bad gemm path %d (0, 1 or 2)", path);
  svdq::set_gemm_path_override(path);
  return ok();
}

svdq_status svdq_debug_set_fp4_tile(int tile) {
  if (tile != 0 && tile != 128 && tile != 256)
    return fail(SVDQ_STATUS_INVALID_VALUE, "bad fp4 tile %d (0, 128 or 256)", tile);
  svdq::set_fp4_tile_override(tile);
  return ok();
}

svdq_status svdq_debug_set_gemm_splits(int splits) {
  if (splits < 0 || splits > 64) return fail(SVDQ_STATUS_INVALID_VALUE, "bad split count %d (0..64)", splits);
  svdq::set_gemm_splits_override(splits);
  return ok();
}

static svdq_status validate_gemm_dims(int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size) {
  if (M < 0 || N <= 0 || K <= 0 || r < 0 || group_size <= 0)
    return fail(SVDQ_STATUS_INVALID_VALUE, "bad dims M=%lld N=%lld K=%lld r=%lld group_size=%lld",
                (long long)M, (long long)N, (long long)K, (long long)r, (long long)group_size);
  if (group_size != 64) return fail(SVDQ_STATUS_NOT_SUPPORTED, "group_size %lld (only 64)", (long long)group_size);
  if (K % 64 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "K=%lld is not a multiple of 64", (long long)K);
  if (N % 64 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "N=%lld is not a multiple of 64", (long long)N);
  if (!rank_supported(r)) return fail(SVDQ_STATUS_NOT_SUPPORTED, "rank %lld (need 0..128, multiple of 16)", (long long)r);
  if (M > (1ll << 24) || N > (1ll << 20) || K > (1ll << 20))
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "problem too large M=%lld N=%lld K=%lld", (long long)M,
                (long long)N, (long long)K);
  return SVDQ_STATUS_SUCCESS;
}

static svdq_status validate_gemm(const void* act_codes, const void* w_codes, int64_t M, int64_t N,
                                 int64_t K, int64_t r, int64_t group_size) {
  svdq_status s = validate_gemm_dims(M, N, K, r, group_size);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (M == 0) return SVDQ_STATUS_SUCCESS;  // empty batch: the caller returns before any pointer check
  if (!act_codes || !w_codes) return fail(SVDQ_STATUS_INVALID_VALUE, "null act_codes/w_codes");
  if (!aligned16(act_codes) || !aligned16(w_codes))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  return SVDQ_STATUS_SUCCESS;
}

// pointer checks and launch shared by the call-2 entry points (dims validated)
static svdq_status gemm_launch(const void* act_codes, const void* act_scales, const void* w_codes,
                               const void* w_scales, const void* lora_act, const void* lora_up,
                               const void* bias, int64_t M, int64_t N, int64_t K, int64_t r,
                               int epilogue, const svdq::QkvEpilogue* qkv, bool fp4, void* y,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!act_scales || !w_scales || !y) return fail(SVDQ_STATUS_INVALID_VALUE, "null act_scales/w_scales/y");
  if (r > 0 && (!lora_act || !lora_up))
    return fail(SVDQ_STATUS_INVALID_VALUE, "r=%lld needs lora_act and lora_up", (long long)r);
  if (!aligned16(act_scales) || !aligned16(w_scales) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  const size_t need = svdq::gemm_workspace_bytes(M, N, K, r, epilogue, fp4);
  svdq_status s = check_workspace(workspace, workspace_bytes, need,
                                  fp4 ? "svdq_fp4_gemm_workspace_size" : "svdq_w4a4_gemm_workspace_size");
  if (s != SVDQ_STATUS_SUCCESS) return s;
  const size_t sc_x = fp4 ? sz(M, K / 32) : sz(M, K / 64, 2), sc_w = fp4 ? sz(N, K / 32) : sz(N, K / 64, 2);
  const bool q = qkv != nullptr;
  s = check_disjoint({{y, sz(M, N, 2), "y"}, {need ? workspace : nullptr, need, "workspace"}},
                     {{act_codes, sz(M, K / 2), "act_codes"}, {act_scales, sc_x, "act_scales"},
                      {w_codes, sz(N, K / 2), "w_codes"}, {w_scales, sc_w, "w_scales"},
                      {r > 0 ? lora_act : nullptr, sz(M, r, 2), "lora_act"},
                      {r > 0 ? lora_up : nullptr, sz(N, r, 2), "lora_up"}, {bias, sz(N, 2), "bias"},
                      {q ? qkv->q_norm : nullptr, 256, "q_norm"}, {q ? qkv->k_norm : nullptr, 256, "k_norm"},
                      {q ? qkv->cos : nullptr, sz(M, 64, 4), "rope_cos"},
                      {q ? qkv->sin : nullptr, sz(M, 64, 4), "rope_sin"}});
  if (s != SVDQ_STATUS_SUCCESS) return s;
  s = check_current_device();
  if (s != SVDQ_STATUS_SUCCESS) return s;
  const svdq::Workspace ws{workspace, workspace_bytes};
  hipError_t e;
  if (fp4)
    e = svdq::launch_fp4_gemm_lora_up(
        static_cast<const uint8_t*>(act_codes), static_cast<const uint8_t*>(act_scales),
        static_cast<const uint8_t*>(w_codes), static_cast<const uint8_t*>(w_scales),
        static_cast<const uint16_t*>(lora_act), static_cast<const uint16_t*>(lora_up),
        static_cast<const uint16_t*>(bias), M, N, K, r, epilogue, static_cast<uint16_t*>(y), ws,
        static_cast<hipStream_t>(stream));
  else
    e = svdq::launch_w4a4_gemm_lora_up(
        static_cast<const uint8_t*>(act_codes), static_cast<const uint16_t*>(act_scales),
        static_cast<const uint8_t*>(w_codes), static_cast<const uint16_t*>(w_scales),
        static_cast<const uint16_t*>(lora_act), static_cast<const uint16_t*>(lora_up),
        static_cast<const uint16_t*>(bias), M, N, K, r, epilogue, qkv, static_cast<uint16_t*>(y),
        svdq::DumpWindow{}, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "gemm launch: %s", hipGetErrorString(e));
  return ok();
}

size_t svdq_w4a4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (validate_gemm_dims(M, N, K, r, 64) != SVDQ_STATUS_SUCCESS || M == 0) return 0;
  return std::max(svdq::gemm_workspace_bytes(M, N, K, r, svdq::kEpilogueNone, false),
                  svdq::gemm_workspace_bytes(M, N, K, r, svdq::kEpilogueGelu, false));
}

size_t svdq_fp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (validate_gemm_dims(M, N, K, r, 64) != SVDQ_STATUS_SUCCESS || M == 0 || K % 128 != 0) return 0;
  return std::max(svdq::gemm_workspace_bytes(M, N, K, r, svdq::kEpilogueNone, true),
                  svdq::gemm_workspace_bytes(M, N, K, r, svdq::kEpilogueGelu, true));
}

svdq_status svdq_w4a4_gemm_lora_up_ex(const void* act_codes, const void* act_scales,
                                      const void* w_codes, const void* w_scales,
                                      const void* lora_act, const void* lora_up, const void* bias,
                                      int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
                                      int epilogue, void* y, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  svdq_status s = validate_gemm(act_codes, w_codes, M, N, K, r, group_size);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (epilogue != SVDQ_EPILOGUE_NONE && epilogue != SVDQ_EPILOGUE_GELU_TANH)
    return fail(SVDQ_STATUS_INVALID_VALUE, "unknown epilogue %d", epilogue);
  if (M == 0) return ok();
  return gemm_launch(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, r,
                     epilogue, nullptr, false, y, workspace, workspace_bytes, stream);
}

svdq_status svdq_w4a4_gemm_lora_up_noalloc(const void* act_codes, const void* act_scales,
                                           const void* w_codes, const void* w_scales,
                                           const void* lora_act, const void* lora_up, const void* bias,
                                           int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
                                           int epilogue, void* y, void* stream) {
  svdq_status s = validate_gemm(act_codes, w_codes, M, N, K, r, group_size);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (epilogue != SVDQ_EPILOGUE_NONE && epilogue != SVDQ_EPILOGUE_GELU_TANH)
    return fail(SVDQ_STATUS_INVALID_VALUE, "unknown epilogue %d", epilogue);
  if (M == 0) return ok();
  if (!act_scales || !w_scales || !y) return fail(SVDQ_STATUS_INVALID_VALUE, "null act_scales/w_scales/y");
  if (r > 0 && (!lora_act || !lora_up))
    return fail(SVDQ_STATUS_INVALID_VALUE, "r=%lld needs lora_act and lora_up", (long long)r);
  if (!aligned16(act_scales) || !aligned16(w_scales) || !aligned16(y) ||
      (bias && !aligned16(bias)) || (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  const size_t need = svdq::gemm_workspace_bytes(M, N, K, r, epilogue, false);
  if (need > svdq::kStaticScratchBytes)
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "this shape needs %zu bytes of scratch; the fixed scratch holds %zu",
                need, svdq::kStaticScratchBytes);
  s = check_disjoint({{y, sz(M, N, 2), "y"}},
                     {{act_codes, sz(M, K / 2), "act_codes"}, {act_scales, sz(M, K / 64, 2), "act_scales"},
                      {w_codes, sz(N, K / 2), "w_codes"}, {w_scales, sz(N, K / 64, 2), "w_scales"},
                      {r > 0 ? lora_act : nullptr, sz(M, r, 2), "lora_act"},
                      {r > 0 ? lora_up : nullptr, sz(N, r, 2), "lora_up"}, {bias, sz(N, 2), "bias"}});
  if (s != SVDQ_STATUS_SUCCESS) return s;
  s = check_current_device();
  if (s != SVDQ_STATUS_SUCCESS) return s;
  hipError_t e = svdq::launch_w4a4_gemm_lora_up_static(
      static_cast<const uint8_t*>(act_codes), static_cast<const uint16_t*>(act_scales),
      static_cast<const uint8_t*>(w_codes), static_cast<const uint16_t*>(w_scales),
      static_cast<const uint16_t*>(lora_act), static_cast<const uint16_t*>(lora_up),
      static_cast<const uint16_t*>(bias), M, N, K, r, epilogue, static_cast<uint16_t*>(y),
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "gemm launch (fixed scratch): %s", hipGetErrorString(e));
  return ok();
}

svdq_status svdq_w4a4_gemm_qkv_norm_rope(const void* act_codes, const void* act_scales,
                                         const void* w_codes, const void* w_scales,
                                         const void* lora_act, const void* lora_up, const void* bias,
                                         int64_t M, int64_t N, int64_t K, int64_t r,
                                         int64_t group_size, int64_t head_dim, const void* q_norm,
                                         const void* k_norm, float eps, const float* rope_cos,
                                         const float* rope_sin, void* y, void* stream) {
  svdq_status s = validate_gemm(act_codes, w_codes, M, N, K, r, group_size);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (head_dim != 128) return fail(SVDQ_STATUS_NOT_SUPPORTED, "head_dim %lld (only 128)", (long long)head_dim);
  if (N % (3 * head_dim) != 0)
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "N=%lld is not 3 x a multiple of head_dim", (long long)N);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(SVDQ_STATUS_INVALID_VALUE, "eps must be finite and >= 0");
  if (M == 0) return ok();
  if (!q_norm || !k_norm || !rope_cos || !rope_sin)
    return fail(SVDQ_STATUS_INVALID_VALUE, "null q_norm/k_norm/rope_cos/rope_sin");
  if (!aligned16(q_norm) || !aligned16(k_norm) || !aligned16(rope_cos) || !aligned16(rope_sin))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  const svdq::QkvEpilogue qkv{static_cast<const uint16_t*>(q_norm), static_cast<const uint16_t*>(k_norm),
                              rope_cos, rope_sin, eps};
  // runs unsplit on the tiled kernel: no workspace
  return gemm_launch(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, r,
                     svdq::kEpilogueQkv, &qkv, false, y, nullptr, 0, stream);
}

svdq_status svdq_w4a4_gemm_lora_up(const void* act_codes, const void* act_scales,
                                   const void* w_codes, const void* w_scales,
                                   const void* lora_act, const void* lora_up, const void* bias,
                                   int64_t M, int64_t N, int64_t K, int64_t r, int64_t group_size,
                                   void* y, void* workspace, size_t workspace_bytes, void* stream) {
  return svdq_w4a4_gemm_lora_up_ex(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias,
                                   M, N, K, r, group_size, SVDQ_EPILOGUE_NONE, y, workspace,
                                   workspace_bytes, stream);
}

svdq_status svdq_fp4_gemm_lora_up(const void* act_codes, const void* act_scales, const void* w_codes,
                                  const void* w_scales, const void* lora_act, const void* lora_up,
                                  const void* bias, int64_t M, int64_t N, int64_t K, int64_t r, int epilogue,
                                  void* y, void* workspace, size_t workspace_bytes, void* stream) {
  svdq_status s = validate_gemm(act_codes, w_codes, M, N, K, r, 64);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (K % 128 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  if (epilogue != SVDQ_EPILOGUE_NONE && epilogue != SVDQ_EPILOGUE_GELU_TANH)
    return fail(SVDQ_STATUS_INVALID_VALUE, "unknown epilogue %d", epilogue);
  if (M == 0) return ok();
  return gemm_launch(act_codes, act_scales, w_codes, w_scales, lora_act, lora_up, bias, M, N, K, r,
                     epilogue, nullptr, true, y, workspace, workspace_bytes, stream);
}

namespace {
// the AWQ linear, one or L stacked layers sharing x
svdq_status awq_call(const void* x, const float* smooth, const void* w_codes, const void* w_scales,
                     const void* w_zeros, const void* bias, int64_t L, int64_t M, int64_t N, int64_t K,
                     int64_t group_size, void* y, void* stream) {
  if (L < 0 || M < 0 || N <= 0 || K <= 0 || group_size <= 0)
    return fail(SVDQ_STATUS_INVALID_VALUE, "bad dims L=%lld M=%lld N=%lld K=%lld group_size=%lld", (long long)L,
                (long long)M, (long long)N, (long long)K, (long long)group_size);
  if (group_size != 64) return fail(SVDQ_STATUS_NOT_SUPPORTED, "group_size %lld (only 64)", (long long)group_size);
  if (K % 64 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "K=%lld is not a multiple of 64", (long long)K);
  if (N % 32 != 0) return fail(SVDQ_STATUS_NOT_SUPPORTED, "N=%lld is not a multiple of 32", (long long)N);
  if (L > 65535 || M > (1ll << 20) || N > (1ll << 20) || (M > 0 && !svdq::awq_supported(K, M)))
    return fail(SVDQ_STATUS_NOT_SUPPORTED, "problem too large L=%lld M=%lld N=%lld K=%lld", (long long)L,
                (long long)M, (long long)N, (long long)K);
  if (M == 0 || L == 0) return ok();
  if (!x || !smooth || !w_codes || !w_scales || !w_zeros || !y)
    return fail(SVDQ_STATUS_INVALID_VALUE, "null x/smooth/w_codes/w_scales/w_zeros/y");
  if (!aligned16(x) || !aligned16(smooth) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(w_zeros) || !aligned16(y) || (bias && !aligned16(bias)))
    return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  svdq_status s = check_disjoint({{y, sz(L, M, N) * 2, "y"}},
                                 {{x, sz(M, K, 2), "x"}, {smooth, sz(L, K, 4), "smooth"},
                                  {w_codes, sz(L, N, K / 2), "w_codes"}, {w_scales, sz(L, N, K / 64) * 2, "w_scales"},
                                  {w_zeros, sz(L, N, K / 64), "w_zeros"}, {bias, sz(L, N, 2), "bias"}});
  if (s != SVDQ_STATUS_SUCCESS) return s;
  s = check_current_device();
  if (s != SVDQ_STATUS_SUCCESS) return s;
  hipError_t e = svdq::launch_awq_w4a16(
      static_cast<const uint16_t*>(x), smooth, static_cast<const uint8_t*>(w_codes),
      static_cast<const uint16_t*>(w_scales), static_cast<const uint8_t*>(w_zeros),
      static_cast<const uint16_t*>(bias), L, M, N, K, static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "awq launch: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

svdq_status svdq_awq_w4a16_gemm(const void* x, const float* smooth, const void* w_codes,
                               const void* w_scales, const void* w_zeros, const void* bias, int64_t M,
                               int64_t N, int64_t K, int64_t group_size, void* y, void* stream) {
  return awq_call(x, smooth, w_codes, w_scales, w_zeros, bias, 1, M, N, K, group_size, y, stream);
}

svdq_status svdq_awq_w4a16_gemm_stacked(const void* x, const float* smooth, const void* w_codes,
                                       const void* w_scales, const void* w_zeros, const void* bias,
                                       int64_t L, int64_t M, int64_t N, int64_t K, int64_t group_size,
                                       void* y, void* stream) {
  return awq_call(x, smooth, w_codes, w_scales, w_zeros, bias, L, M, N, K, group_size, y, stream);
}

svdq_status svdq_w4a4_group_acc_debug(const void* act_codes, const void* w_codes, int64_t M, int64_t N,
                                      int64_t K, int64_t m0, int64_t mc, int64_t n0, int64_t nc, int32_t* acc,
                                      void* stream) {
  svdq_status s = validate_gemm(act_codes, w_codes, M, N, K, 0, 64);
  if (s != SVDQ_STATUS_SUCCESS) return s;
  if (m0 < 0 || mc < 0 || n0 < 0 || nc < 0 || m0 + mc > M || n0 + nc > N)
    return fail(SVDQ_STATUS_INVALID_VALUE, "window rows [%lld, +%lld) cols [%lld, +%lld) outside %lld x %lld",
                (long long)m0, (long long)mc, (long long)n0, (long long)nc, (long long)M, (long long)N);
  if (M == 0 || mc == 0 || nc == 0) return ok();
  if (!acc) return fail(SVDQ_STATUS_INVALID_VALUE, "null acc");
  if (!aligned16(acc)) return fail(SVDQ_STATUS_INVALID_VALUE, "device pointers must be 16-byte aligned");
  if (mc * nc * (K / 64) > (1ll << 31)) return fail(SVDQ_STATUS_NOT_SUPPORTED, "accumulator window too large");
  s = check_disjoint({{acc, sz(mc, nc, K / 64) * 4, "acc"}},
                     {{act_codes, sz(M, K / 2), "act_codes"}, {w_codes, sz(N, K / 2), "w_codes"}});
  if (s != SVDQ_STATUS_SUCCESS) return s;
  s = check_current_device();
  if (s != SVDQ_STATUS_SUCCESS) return s;
  // the launched problem: the rows from the 16-row block holding m0 (codes
  // arrays keep their storage order only in views at multiples of 16 rows) to
  // m0 + mc, and the 64-aligned column range around the window; the window is
  // then relative to it
  const int64_t mb = m0 / 16 * 16;
  const int64_t nb = n0 / 64 * 64, ne = (n0 + nc + 63) / 64 * 64;
  const uint8_t* ac = static_cast<const uint8_t*>(act_codes) + (size_t)mb * (size_t)(K / 2);
  const uint8_t* wc = static_cast<const uint8_t*>(w_codes) + (size_t)nb * (size_t)(K / 2);
  const svdq::DumpWindow win{acc, (int)(m0 - mb), (int)(m0 - mb + mc), (int)(n0 - nb), (int)(n0 - nb + nc)};
  hipError_t e = svdq::launch_w4a4_gemm_lora_up(ac, nullptr, wc, nullptr, nullptr, nullptr, nullptr,
                                                m0 + mc - mb, ne - nb,
                                                K, 0, SVDQ_EPILOGUE_NONE, nullptr, nullptr, win, svdq::Workspace{},
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SVDQ_STATUS_HIP_ERROR, "gemm debug launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// host packer entry points live in packer.cpp; they use these helpers for errors
svdq_status svdq_internal_fail(svdq_status s, const char* msg) { return fail(s, "%s", msg); }
svdq_status svdq_internal_ok() { return ok(); }
