// noalloc.hip -- flare_qkv_prologue_bwd_noalloc: the reverse mode of the QKV
// prologue with its weight-gradient partials in a fixed device array of the
// library instead of a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight training or serving
// loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the first call on a device, with that
// device current, looks the address up with hipGetSymbolAddress and keeps it
// per device; kernels receive that pointer, as they receive the caller's
// workspace in flare_qkv_prologue_bwd.
//
// The partials are written in full before they are read (every token block
// writes all of its channels, the reduce reads only those blocks), so nothing
// has to be cleared between calls.  All calls on one GPU share its array:
// calls that overlap in time on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_plan.h"

using namespace flare;

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // the array's device address, per device, once looked up

flare_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FLARE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FLARE_ERR_UNSUPPORTED, "device index %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FLARE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLARE_OK;
}

}  // namespace

extern "C" {

size_t flare_noalloc_scratch_bytes(void) { return kScratchBytes; }

flare_status flare_qkv_prologue_bwd_noalloc(const flare_varlen *varlen, int32_t block_size, int32_t heads,
                                            int32_t head_dim, int32_t width, int32_t io_dtype,
                                            const void *const x[3], const void *const xn[3],
                                            const float *const weight[3], int32_t activation, int32_t qk_l2norm,
                                            const void *const dy[3], const void *const dyn[3], void *const dx[3],
                                            void *const dxn[3], float *const dweight[3], void *stream) {
  clear_error();
  const size_t need = flare_qkv_prologue_bwd_workspace_size(varlen, block_size, heads, head_dim, width);
  if (need == 0) {
    // invalid arguments: the workspace entry point names the reason
    return flare_qkv_prologue_bwd(varlen, block_size, heads, head_dim, width, io_dtype, x, xn, weight, activation,
                                  qk_l2norm, dy, dyn, dx, dxn, dweight, nullptr, 0, stream);
  }
  if (need > kScratchBytes)
    return fail(FLARE_ERR_WORKSPACE,
                "qkv_prologue_bwd_noalloc: this batch needs %zu bytes of weight-gradient partials, the static "
                "scratch holds %zu (use flare_qkv_prologue_bwd with a workspace)",
                need, kScratchBytes);
  void *ptr = nullptr;
  const flare_status st = scratch_address(&ptr);
  if (st != FLARE_OK) return st;
  return flare_qkv_prologue_bwd(varlen, block_size, heads, head_dim, width, io_dtype, x, xn, weight, activation,
                                qk_l2norm, dy, dyn, dx, dxn, dweight, ptr, kScratchBytes, stream);
}

}  // extern "C"
