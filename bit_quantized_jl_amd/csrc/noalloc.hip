// Allocation-free decode attention: qjl_decode_attention with its workspace
// taken from a file-scope device array instead of a caller buffer, for
// callers that cannot allocate device memory.
//
// The array lives in the library's code object, so every GPU the library
// runs on holds its own copy from the time the code object is loaded until
// the process ends.  In host code the name `scratch` only stands in for the
// device variable; the device address of this GPU's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// on the entry point's first call there, and that address is what the
// kernels receive.  Every workspace byte the kernels read in a call was
// written earlier in the same call (softmax partials, or the scores of the
// plain path), so nothing is cleared between calls; calls that overlap on
// one GPU share the array and race.
#include <mutex>

#include "device_common.h"

namespace {

static __device__ __align__(256) unsigned char scratch[QJL_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = qjl::PerDevice::MAX_DEVICES;
std::mutex scratch_mu;
void *scratch_ptr[MAX_DEVICES];

// Device address of the current device's copy of `scratch` (dev is the
// current device).
qjl_status scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= MAX_DEVICES) return QJL_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return QJL_ERR_DEVICE;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return QJL_OK;
}

}  // namespace

extern "C" qjl_status qjl_decode_attention_noalloc(const qjl_sketch *sk, const float *Sq,
                                                   const uint32_t *bits, const float *norms,
                                                   const void *V, int32_t v_dtype, int32_t d_v,
                                                   int64_t n_groups, int64_t n_q_per_group,
                                                   int64_t n_k_per_group, float softmax_scale,
                                                   float *out, void *stream) {
  bool noop = false;
  qjl_status st = qjl::attention_check_args(sk, Sq, bits, norms, V, v_dtype, d_v, n_groups,
                                            n_q_per_group, n_k_per_group, softmax_scale, out,
                                            &noop);
  if (st != QJL_OK || noop) return st;
  const size_t need =
      qjl::attention_workspace_bytes(sk, n_groups, n_q_per_group, n_k_per_group, d_v);
  if (need > (size_t)QJL_NOALLOC_SCRATCH_BYTES) return QJL_ERR_UNSUPPORTED;
  void *ws = nullptr;
  st = scratch_address(sk->device, &ws);  // attention_check_args made sk->device current
  if (st != QJL_OK) return st;
  return qjl::attention_run(sk, Sq, bits, norms, V, v_dtype, d_v, n_groups, n_q_per_group,
                            n_k_per_group, softmax_scale, static_cast<float *>(ws), out, stream);
}
