// C ABI shell: argument validation, error text, small helpers.  Kernels live in the .hip files.
#include <cstdarg>
#include <cstdio>

#include "common.hpp"

namespace echo {

static thread_local char g_err[1024] = "";

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ECHO_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ECHO_OK;
}

const char *last_error() { return g_err; }

}  // namespace echo

using namespace echo;

extern "C" {

const char *echo_last_error(void) { return echo::last_error(); }

const char *echo_version(void) { return "echo-mi355x 0.1 (gfx950, H=64, D=128)"; }

size_t echo_pool_metadata_bytes(int32_t n_host, int32_t n_gpu) {
  // HostTokenToGPU (4 B) per host token; free (1) + priority (4) + to_host (4) +
  // indices buffer (4) per GPU slot
  return 4u * static_cast<size_t>(n_host < 0 ? 0 : n_host) +
         13u * static_cast<size_t>(n_gpu < 0 ? 0 : n_gpu);
}

int echo_host_alloc(size_t bytes, int coherent, void **host, void **dev) {
  if (!host || !dev) return fail(ECHO_EINVAL, "echo_host_alloc: NULL output pointer");
  *host = nullptr;
  *dev = nullptr;
  if (bytes == 0) return fail(ECHO_EINVAL, "echo_host_alloc: zero bytes");
  unsigned flags = hipHostMallocMapped | (coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
  void *p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, flags);
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
  void *d = nullptr;
  e = hipHostGetDevicePointer(&d, p, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(p);
    return fail(ECHO_EHIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  }
  *host = p;
  *dev = d;
  return ECHO_OK;
}

int echo_host_free(void *host) {
  if (!host) return ECHO_OK;
  hipError_t e = hipHostFree(host);
  if (e != hipSuccess) return fail(ECHO_EHIP, "hipHostFree: %s", hipGetErrorString(e));
  return ECHO_OK;
}

}  // extern "C"
