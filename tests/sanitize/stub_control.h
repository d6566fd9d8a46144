// Knobs of the host-only stand-ins in abi_stubs.cpp.
#pragma once
#include <stddef.h>

extern int g_stub_devices;   // devices hipGetDeviceCount reports (0: "no device")
extern int g_stub_launches;  // launcher calls so far
extern const size_t kStubWorkspace;  // every workspace / state size the stand-ins report
