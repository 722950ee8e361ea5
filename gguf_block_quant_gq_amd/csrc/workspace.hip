// workspace.hip -- stream-ordered device scratch for the kernels that need
// it (the matrix-core GEMM's prepared activations and split-K partials).
//
// Each device gets one private HIP memory pool whose release threshold is
// unbounded, so memory freed on a stream goes back to the pool and is handed
// out again without a trip to the driver. Allocation and release are both
// enqueued on the caller's stream: the call stays asynchronous, concurrent
// calls on different streams get disjoint blocks, and the pool keeps its
// memory until the process ends.
#include <mutex>

#include "gq_internal.h"

namespace gq {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
hipMemPool_t g_pool[kMaxDevices];
bool g_ready[kMaxDevices];

hipError_t device_pool(hipMemPool_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ready[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pool[dev] = pool;
    g_ready[dev] = true;
  }
  *out = g_pool[dev];
  return hipSuccess;
}

}  // namespace

hipError_t ws_alloc(size_t bytes, hipStream_t s, void** p) {
  // Requests are rounded up to a power of two (at least 1 MiB): measured on
  // MI355X, consecutive requests of different sizes (prompt chunks of
  // different lengths, the groups of gq_matmul_experts) were not served
  // from the pool's freed blocks and cost hundreds of microseconds each
  // (eight Q4_K products of 50..230 rows: 2.8 ms, against 0.69 ms rounded).
  size_t b = (size_t)1 << 20;
  while (b < bytes && b <= (SIZE_MAX >> 1)) b <<= 1;
  if (b < bytes) return hipErrorOutOfMemory;
  bytes = b;
  hipMemPool_t pool;
  hipError_t e = device_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(p, bytes, pool, s);
}

hipError_t ws_free(void* p, hipStream_t s) { return hipFreeAsync(p, s); }

}  // namespace gq
