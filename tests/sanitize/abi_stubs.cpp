// Host-only stand-ins for what abi.cpp calls beyond itself: the kernel
// launchers and size functions of the library (which need the device
// compiler) and the three HIP runtime calls it makes.  They let the C-ABI
// layer be built with g++ under AddressSanitizer and UBSan and driven by
// abi_cases.cpp on a machine without a GPU.  Launchers only count calls;
// sizes are fixed so that the driver knows what the validation compares.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "stub_control.h"

int g_stub_devices = 1;
int g_stub_launches = 0;
const size_t kStubWorkspace = 4096;

extern "C" {
hipError_t hipGetDeviceCount(int *count) {
  *count = g_stub_devices;
  return g_stub_devices > 0 ? hipSuccess : hipErrorNoDevice;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
}

namespace kvpop {

long long fwd_grid_blocks(const ShapeInfo &s) { return (long long)s.B * s.Hq * ((s.S + 127) / 128); }
long long tgt_grid_blocks(const ShapeInfo &s, int) { return (long long)s.B * s.Hkv * ((s.S + 255) / 256); }

hipError_t launch_fwd(const ShapeInfo &, const void *, const void *, const void *, void *, float *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
size_t tgt_workspace_bytes(const ShapeInfo &) { return kStubWorkspace; }
size_t tgt_workspace_bytes_for(const ShapeInfo &s, int agg) {
  // grows with the shape so that the driver can ask for more than the scratch holds
  return (size_t)s.B * (agg == 0 ? s.Hkv : s.Hq) * (size_t)s.S * 64;
}
hipError_t noalloc_scratch(void **out) {
  static unsigned char fake[256];
  *out = fake;
  return hipSuccess;
}
hipError_t launch_future_target(const ShapeInfo &, const void *, const void *, const float *, int, int, int, float,
                                float *, void *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
size_t budget_workspace_bytes(const ShapeInfo &, int, int, int) { return kStubWorkspace; }
BudgetListsInfo budget_lists_info(const ShapeInfo &s, int sinks, int window, int topk) {
  BudgetListsInfo li{};
  li.lists = 256;
  li.spans = 384;
  li.lens = 512;
  li.lens_full = 768;
  li.status = 1024;
  li.QB = 32;
  li.nqb = (s.S + 31) / 32;
  li.cap = sinks + window + topk + 32;
  li.tile = 32;
  return li;
}
hipError_t launch_budget(const ShapeInfo &, const void *, const void *, const void *, const float *, int, int, int,
                         void *, float *, int *, int *, void *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
size_t teacher_workspace_bytes(int, int, int) { return kStubWorkspace; }
hipError_t launch_teacher(int, int, int, const float *, const float *, int, int, int, int, int *, int *, int *, int *,
                          void *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
size_t boundary_loss_workspace_bytes(int, int, int) { return kStubWorkspace; }
hipError_t launch_boundary_loss(int, int, int, const float *, const int *, const int *, int, int, int, float,
                                const float *, float *, float *, void *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
size_t decode_state_bytes(const DecodeShapeInfo &) { return kStubWorkspace; }
hipError_t launch_decode_init(const DecodeShapeInfo &, void *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}
hipError_t launch_decode_step(const DecodeShapeInfo &, void *, int, const void *, const void *, const void *,
                              const float *, void *, float *, hipStream_t) {
  ++g_stub_launches;
  return hipSuccess;
}

}  // namespace kvpop
