// gptq_dequant_matmul_noalloc: the dequantize-on-the-fly product for callers
// that cannot allocate device memory (code under stream capture, tight
// serving loops).  Its scratch space (the split partial sums, the gathered X
// of an act-order layer) is a fixed device array of this file instead of a
// caller workspace.
//
// Each device holds its own copy of `scratch` for the life of the process.
// On host code the array's name is only a stand-in: its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept; kernels get that address, as they get the workspace in
// gptq_dequant_matmul.  Every call on a device shares the device's copy, so
// calls that overlap on one device (two streams, or host threads) race on
// it.  The kernels write every partial they later read, so nothing has to be
// cleared between calls.
#include <map>
#include <mutex>
#include <string>

#include "../../include/gptq.h"
#include "common.hpp"

namespace gptq {
namespace {

static_assert(GPTQ_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
__device__ __align__(256) unsigned char scratch[GPTQ_NOALLOC_SCRATCH_BYTES];

std::mutex& scratch_mutex() {
  static std::mutex mu;
  return mu;
}

// Device address of device `dev`'s copy of the scratch array (dev current).
hipError_t scratch_address(int dev, void** out) {
  static std::map<int, void*> per_dev;  // guarded by scratch_mutex()
  std::lock_guard<std::mutex> lock(scratch_mutex());
  auto it = per_dev.find(dev);
  if (it == per_dev.end()) {
    void* p = nullptr;
    GPTQ_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return hipErrorInvalidSymbol;
    it = per_dev.emplace(dev, p).first;
  }
  *out = it->second;
  return hipSuccess;
}

int noalloc_fail(int status, const std::string& msg) {
  set_error(msg);
  return status;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" int gptq_dequant_matmul_noalloc(const void* X, int x_dtype, int64_t M, int64_t in,
                                           int64_t ldx, const int32_t* qweight,
                                           const float* scales, const int32_t* zeros,
                                           const int32_t* g_idx, const int32_t* x_order,
                                           int64_t n_groups, int64_t out, int bits, void* Y,
                                           int y_dtype, int64_t ldy, void* stream) {
  clear_error();
  const int st = dequant_check(X, x_dtype, M, in, ldx, qweight, scales, zeros, g_idx, n_groups,
                               out, bits, Y, y_dtype, ldy);
  if (st != GPTQ_OK || M == 0) return st;
  const size_t need = dequant_matmul_workspace_bytes(M, in, out, x_order ? 1 : 0);
  if (need > (size_t)GPTQ_NOALLOC_SCRATCH_BYTES)
    return noalloc_fail(GPTQ_ERR_WORKSPACE,
                        "gptq_dequant_matmul_noalloc: this product needs " + std::to_string(need) +
                            " bytes of scratch, more than the fixed " +
                            std::to_string((size_t)GPTQ_NOALLOC_SCRATCH_BYTES) +
                            "; use gptq_dequant_matmul with a workspace");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess)
    return noalloc_fail(GPTQ_ERR_HIP, std::string("gptq_dequant_matmul_noalloc: ") +
                                          hipGetErrorString(e));
  if (dev != cur)
    return noalloc_fail(GPTQ_ERR_INVALID_ARG,
                        "gptq_dequant_matmul_noalloc: the stream belongs to device " +
                            std::to_string(dev) + ", not to the current device " +
                            std::to_string(cur));
  void* ws = nullptr;
  if (need > 0) {
    e = scratch_address(dev, &ws);
    if (e != hipSuccess)
      return noalloc_fail(GPTQ_ERR_HIP, std::string("gptq_dequant_matmul_noalloc: ") +
                                            hipGetErrorString(e));
  }
  e = run_dequant_matmul(X, M, in, ldx, qweight, scales, zeros, g_idx, x_order, out, bits, Y,
                         y_dtype == GPTQ_F16 ? 1 : 0, ldy, ws, GPTQ_NOALLOC_SCRATCH_BYTES, s);
  if (e != hipSuccess)
    return noalloc_fail(GPTQ_ERR_HIP, std::string("gptq_dequant_matmul_noalloc: ") +
                                          hipGetErrorString(e));
  return GPTQ_OK;
}
