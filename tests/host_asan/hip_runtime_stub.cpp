// Stand-ins for the HIP runtime entry points that a host-only build of libbd
// references, so that the C ABI layer and the host side of every launcher run,
// under the host sanitizers, on a machine without a GPU.  Kernel launches are
// checked for a launchable shape and counted, never run.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>

long long g_stub_launches = 0;   // launches accepted so far (read by the driver)

namespace {
struct CallConfig {
  dim3 grid, block;
  size_t shmem;
  hipStream_t stream;
};
CallConfig g_config;
char g_symbol_stand_in[64];
}  // namespace

extern "C" {

// Code-object registration (called from static constructors): nothing to register.
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, void*, void*, void*, void*,
                           int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}

// The <<<grid, block, shmem, stream>>> configuration handed from the call site to the kernel stub.
hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  g_config = CallConfig{grid, block, shmem, stream};
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shmem, hipStream_t* stream) {
  *grid = g_config.grid;
  *block = g_config.block;
  *shmem = g_config.shmem;
  *stream = g_config.stream;
  return hipSuccess;
}

hipError_t hipLaunchKernel(const void* function, dim3 grid, dim3 block, void** args, size_t shmem,
                           hipStream_t stream) {
  (void)stream;
  const unsigned long long threads = (unsigned long long)block.x * block.y * block.z;
  if (!function || !args || grid.x == 0 || grid.y == 0 || grid.z == 0 || threads == 0 || threads > 1024 ||
      shmem > 160 * 1024) {
    std::fprintf(stderr, "stub: unlaunchable kernel: grid %u x %u x %u, block %u x %u x %u, %zu bytes of LDS\n",
                 grid.x, grid.y, grid.z, block.x, block.y, block.z, shmem);
    std::abort();
  }
  ++g_stub_launches;
  return hipSuccess;
}

hipError_t hipFuncSetAttribute(const void* function, hipFuncAttribute, int value) {
  return function && value >= 0 ? hipSuccess : hipErrorInvalidValue;
}

hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

// The compute units of an MI355X; other attributes are not asked for.
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
  if (!value || device != 0 || attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *value = 256;
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

// A host stand-in address (no launch is run, so it is never dereferenced).
hipError_t hipGetSymbolAddress(void** address, const void* symbol) {
  if (!address || !symbol) return hipErrorInvalidValue;
  *address = g_symbol_stand_in;
  return hipSuccess;
}

}  // extern "C"
