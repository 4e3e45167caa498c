// A stand-in for the HIP runtime and for the library's kernel launchers, so
// that the host code of libsvdq (the C ABI in api.cpp and the packer) can be
// built with AddressSanitizer / UndefinedBehaviorSanitizer and driven on a
// machine without a GPU.  The fake device's architecture name comes from the
// FAKE_GFX_ARCH environment variable (default gfx950), so the load-time
// architecture check can be forced to fail.  Launchers record their last call
// instead of launching anything; workspace needs are set by the driver.
#include <hip/hip_runtime_api.h>

#include <cstdlib>
#include <cstring>

#include "svdq_internal.h"
#include "fake_runtime.h"

FakeState g_fake;

extern "C" {

hipError_t hipGetDeviceCount(int* count) {
  const char* n = std::getenv("FAKE_DEVICE_COUNT");
  *count = n ? std::atoi(n) : 1;
  return *count > 0 ? hipSuccess : hipErrorNoDevice;
}

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int device) {
  (void)device;
  std::memset(prop, 0, sizeof(*prop));
  const char* arch = std::getenv("FAKE_GFX_ARCH");
  std::strncpy(prop->gcnArchName, arch ? arch : "gfx950", sizeof(prop->gcnArchName) - 1);
  prop->multiProcessorCount = 256;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  (void)device;
  *value = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "fake HIP error"; }

}  // extern "C"

namespace svdq {

size_t quant_workspace_bytes(int64_t, int64_t, int64_t) { return g_fake.quant_need; }
size_t gemm_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int, bool) { return g_fake.gemm_need; }
bool awq_supported(int64_t K, int64_t M) { return K <= (M == 1 ? 16384 : M <= 4 ? 8192 : 4096); }
void set_quant_plan_override(int, int) {}
void set_quant_waves_override(int) {}
void set_gemm_path_override(int) {}
void set_gemm_splits_override(int) {}
void set_fp4_tile_override(int) {}

static void record(const char* name, const void* out, Workspace ws) {
  ++g_fake.launches;
  g_fake.last = name;
  g_fake.last_out = out;
  g_fake.last_ws = ws.ptr;
  g_fake.last_ws_bytes = ws.bytes;
}

hipError_t launch_quant_lora_down(const uint16_t*, const float*, const uint16_t*, int64_t, int64_t, int64_t,
                                  uint8_t* codes, uint16_t*, uint16_t*, bool fp4, Workspace ws, hipStream_t) {
  record(fp4 ? "quant_fp4" : "quant", codes, ws);
  return hipSuccess;
}

hipError_t launch_w4a4_gemm_lora_up(const uint8_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                                    const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t,
                                    int64_t, int epilogue, const QkvEpilogue*, uint16_t* y, const DumpWindow& dump,
                                    Workspace ws, hipStream_t) {
  record(dump.acc ? "dump" : epilogue == kEpilogueQkv ? "gemm_qkv" : "gemm",
         dump.acc ? static_cast<const void*>(dump.acc) : y, ws);
  g_fake.last_window[0] = dump.m_lo;
  g_fake.last_window[1] = dump.m_hi;
  g_fake.last_window[2] = dump.n_lo;
  g_fake.last_window[3] = dump.n_hi;
  return hipSuccess;
}

hipError_t launch_w4a4_gemm_lora_up_static(const uint8_t*, const uint16_t*, const uint8_t*, const uint16_t*,
                                           const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                                           int64_t, int64_t, int, uint16_t* y, hipStream_t) {
  record("gemm_static", y, Workspace{});
  return hipSuccess;
}

hipError_t launch_fp4_gemm_lora_up(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, const uint16_t*,
                                  const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t, int,
                                  uint16_t* y, Workspace ws, hipStream_t) {
  record("gemm_fp4", y, ws);
  return hipSuccess;
}

hipError_t launch_awq_w4a16(const uint16_t*, const float*, const uint8_t*, const uint16_t*, const uint8_t*,
                            const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint16_t* y, hipStream_t) {
  record("awq", y, Workspace{});
  return hipSuccess;
}

}  // namespace svdq
