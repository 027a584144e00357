// Library-wide entry points: version, error text, device check.
#include "kvz_internal.h"

#include <atomic>
#include <cstring>
#include <string>

namespace kvz {

namespace {
thread_local std::string g_last_error;
}

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVZ_OK;
  return set_error(KVZ_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Compute units of the current device, queried once per device (threads may race to fill an
// entry; they store the same value).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace kvz

using namespace kvz;

extern "C" int kvz_version(void) { return KVZ_VERSION; }

extern "C" const char* kvz_last_error(void) { return g_last_error.c_str(); }

extern "C" int kvz_device_check(int device) {
  hipDeviceProp_t prop;
  int rc = check_hip(hipGetDeviceProperties(&prop, device), "hipGetDeviceProperties");
  if (rc != KVZ_OK) return rc;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_error(KVZ_EUNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");
  return KVZ_OK;
}
