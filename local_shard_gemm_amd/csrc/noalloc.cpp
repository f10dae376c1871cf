// sm_local_gemm_reduce_noalloc: sm_local_gemm_reduce_ws with the workspace
// in a static device array of the library, for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid allocation). The call makes no hipMalloc / hipFree and calls
// no allocating routine.
//
// The array `scratch` is a file-scope __device__ variable: each GPU the
// library runs on holds its own copy until the process ends. Host code never
// uses the array's name as an address (on the host it is a stand-in, not a
// device pointer); once per device, with that device current, its device
// address is fetched with hipGetSymbolAddress and kept, and only that
// address is passed to kernels.
//
// What must start at zero: the arrival counters at the front of the array.
// A device's copy is cleared by a fill kernel on the first call on that
// device (on the caller's stream, before the first use), and every call
// that completes leaves its counters at zero again. The partials behind
// them are fully written before they are read in every call, so the
// previous call's contents never leak into a result. Calls on one GPU share
// the array: calls that overlap in time (different streams without
// synchronisation, or several threads) race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"
#include "kernels.h"

// Room for the partials of one call: 32 MiB (for example N = 8 ranks x 128
// rows x 8192 float32 columns), behind 64 KiB of counters (16384 column
// blocks over all groups of the call).
constexpr int64_t kScratchCounterBytes = int64_t{64} << 10;
constexpr int64_t kScratchPartBytes = int64_t{32} << 20;
constexpr int64_t kScratchBytes = kScratchCounterBytes + kScratchPartBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace shardmm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, set up (address
// fetched, counters cleared on `stream`) on the first call on the device.
int32_t device_scratch(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SM_ERR_ARG, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SM_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    e = launch_zero_words(static_cast<uint32_t*>(p), kScratchCounterBytes / 4, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "clearing the scratch counters");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SM_OK;
}

}  // namespace
}  // namespace shardmm

using namespace shardmm;

extern "C" int32_t sm_local_gemm_reduce_noalloc(const sm_plan_t* plan, const sm_buf* A, const sm_buf* B,
                                                const sm_buf* out, int32_t mode, int32_t group_begin,
                                                int32_t group_count, void* stream) {
  clear_error();
  // Every host check first, so that a refused call touches no device state
  // (and sets up no scratch); a call too large for the scratch is refused
  // here with SM_ERR_SHAPE.
  ReduceScratch sc;
  sc.kind = ReduceScratch::kValidate;
  int32_t st = gemm_reduce_impl(plan, A, B, out, mode, group_begin, group_count, sc, stream, nullptr);
  if (st) return st;
  const bool skinny = plan->c_local[0] <= kSkinnyMaxM;
  const ReduceWorkspace w = reduce_workspace(*plan, group_count);
  if (skinny || (w.two_pass && w.part_bytes <= kScratchPartBytes)) {
    if (skinny && (w.counter_bytes > kScratchCounterBytes || w.part_bytes > kScratchPartBytes))
      return fail(SM_ERR_SHAPE, "the call needs " + std::to_string(w.counter_bytes) + " bytes of counters and " +
                                    std::to_string(w.part_bytes) + " bytes of partials; the static scratch holds " +
                                    std::to_string(kScratchCounterBytes) + " and " +
                                    std::to_string(kScratchPartBytes) + " (use sm_local_gemm_reduce_ws)");
    void* base = nullptr;
    if ((st = device_scratch(stream, &base))) return st;
    // counters always at the front, partials always behind the whole
    // counter region: no call's partials overlap another call's counters
    sc.kind = ReduceScratch::kFixed;
    sc.counters = static_cast<uint32_t*>(base);
    sc.counter_cap = kScratchCounterBytes;
    sc.parts = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + kScratchCounterBytes);
    sc.part_cap = kScratchPartBytes;
  } else {
    // taller products: one launch over the whole J, no scratch (also when a
    // few-tile product's partials do not fit the scratch)
    sc.kind = ReduceScratch::kNone;
  }
  return gemm_reduce_impl(plan, A, B, out, mode, group_begin, group_count, sc, stream,
                          "sm_local_gemm_reduce_noalloc launch");
}
