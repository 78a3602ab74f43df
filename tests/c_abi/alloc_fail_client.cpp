// Allocation failures at the C interface, without a GPU.
//
// The executable defines its own global operator new / delete (counting live blocks
// and throwing std::bad_alloc once an armed countdown runs out) and the device calls
// gemm_create makes (one visible gfx950 device, the address of the scratch array).
// Linked with -rdynamic, these definitions take the place of libstdc++'s and the HIP
// runtime's for every caller in the process, libtgemm.so included. Each entry point that allocates host memory must
// then return GEMM_ERR_OUT_OF_MEMORY, with no exception escaping and nothing leaked.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "tgemm.h"

static long g_countdown = -1;  // < 0: never fail; n >= 0: the allocation after n more succeeds fails
static long g_live = 0;        // blocks allocated and not yet freed

void* operator new(std::size_t n) {
  if (g_countdown == 0) throw std::bad_alloc();
  if (g_countdown > 0) --g_countdown;
  void* p = std::malloc(n ? n : 1);
  if (p == nullptr) throw std::bad_alloc();
  ++g_live;
  return p;
}
void* operator new[](std::size_t n) { return operator new(n); }
void* operator new(std::size_t n, const std::nothrow_t&) noexcept {
  try {
    return operator new(n);
  } catch (...) {
    return nullptr;
  }
}
void* operator new[](std::size_t n, const std::nothrow_t& t) noexcept { return operator new(n, t); }
void operator delete(void* p) noexcept {
  if (p != nullptr) {
    --g_live;
    std::free(p);
  }
}
void operator delete[](void* p) noexcept { operator delete(p); }
void operator delete(void* p, std::size_t) noexcept { operator delete(p); }
void operator delete[](void* p, std::size_t) noexcept { operator delete(p); }

// One gfx950 device with 256 compute units.
extern "C" hipError_t hipGetDeviceCount(int* count) {
  *count = 1;
  return hipSuccess;
}
extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  prop->multiProcessorCount = 256;
  return hipSuccess;
}

// The device address of the library's scratch array (resolved by gemm_create).
extern "C" hipError_t hipGetSymbolAddress(void** ptr, const void*) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(0x200000));
  return hipSuccess;
}

#define EXPECT(c)                                                               \
  do {                                                                          \
    if (!(c)) {                                                                 \
      std::fprintf(stderr, "alloc_fail_client: line %d: %s\n", __LINE__, #c); \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

int main() {
  gemm_handle_t h = nullptr;
  // the handle itself, then its entry in the registry of live handles
  for (long n = 0; n < 2; ++n) {
    const long before = g_live;
    g_countdown = n;
    const gemm_status_t st = gemm_create(&h);
    g_countdown = -1;
    EXPECT(st == GEMM_ERR_OUT_OF_MEMORY);
    EXPECT(h == nullptr);
    EXPECT(g_live == before);  // a handle made before the failure is freed again
  }
  EXPECT(gemm_create(&h) == GEMM_OK && h != nullptr);
  EXPECT(gemm_set_tile(h, 64, 64, 64) == GEMM_OK && gemm_set_tile(h, 0, 0, 0) == GEMM_OK);

  // gemm_tune lists its candidate plans before it touches the device
  const void* p = reinterpret_cast<const void*>(static_cast<uintptr_t>(0x100000));
  gemm_plan_t best;
  const long before = g_live;
  g_countdown = 0;
  gemm_status_t st = gemm_tune(h, GEMM_OP_N, GEMM_OP_N, 1024, 1024, 1024, p, 1024, p, 1024, const_cast<void*>(p),
                               1024, GEMM_BF16_BF16, nullptr, 1, &best);
  g_countdown = -1;
  EXPECT(st == GEMM_ERR_OUT_OF_MEMORY);
  EXPECT(g_live == before);
  // planning does not allocate, and the handle still works
  g_countdown = 0;
  st = gemm_plan(h, 1024, 1024, 1024, p, 1024, p, 1024, p, 1024, GEMM_BF16_BF16, &best);
  g_countdown = -1;
  EXPECT(st == GEMM_OK && best.kernel == 4);
  EXPECT(gemm_destroy(h) == GEMM_OK);
  EXPECT(gemm_destroy(h) == GEMM_ERR_INVALID_ARG);
  std::printf("alloc_fail_client: ok\n");
  return 0;
}
