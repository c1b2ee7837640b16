// isd_verify_noalloc: verification for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Its
// scratch space is a fixed array in device memory that the library holds on each GPU it
// runs on until the process ends; the kernels are isd_verify's, handed the array's
// address in place of a caller workspace.
#include <mutex>

#include "isd.h"
#include "launch.h"
#include "validate.h"

namespace {

constexpr size_t SCRATCH_BYTES = ISD_VERIFY_NOALLOC_MAX_BYTES;
constexpr int MAX_DEVICES = 64;

// The scratch array.  Host code never uses this name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress (below) and is what the kernels receive.
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch_of_device[MAX_DEVICES] = {};

// Device address of the current device's copy of the array, looked up once per device
// (with that device current) and kept.
isd_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return isd::set_error(ISD_ERR_HIP, "verify_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return isd::set_error(ISD_ERR_UNSUPPORTED, "verify_noalloc: device %d (at most %d devices)", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_of_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return isd::set_error(ISD_ERR_HIP, "verify_noalloc: hipGetSymbolAddress on device %d: %s", dev,
                            hipGetErrorString(e));
    g_scratch_of_device[dev] = p;
  }
  *out = g_scratch_of_device[dev];
  return ISD_OK;
}

}  // namespace

extern "C" isd_status isd_verify_noalloc(isd_dtype dt, const void* logits, const void* draft_logits,
                                         const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                                         float temperature, int32_t* n_accept, uint8_t* accept,
                                         int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                                         float* p_draft, float* q_draft, float* row_lse, void* stream) {
  // arguments first, against a stand-in address: nothing touches the GPU for a bad call
  isd::VerifyLaunch v;
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  isd_status st = isd::prepare_verify(dt, logits, draft_logits, draft_ids, uniforms, B, N, V, temperature, n_accept,
                                      accept, next_token, argmax_ids, sampled_ids, p_draft, q_draft, row_lse,
                                      stand_in, SCRATCH_BYTES, &v);
  if (st == ISD_ERR_WORKSPACE)
    return isd::set_error(ISD_ERR_UNSUPPORTED,
                          "verify_noalloc: B=%d N=%d V=%d needs %zu bytes of scratch, the fixed array holds %zu",
                          B, N, V, isd::verify_workspace_bytes(B, N, V), SCRATCH_BYTES);
  if (st != ISD_OK) return st;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != ISD_OK) return st;
  st = isd::prepare_verify(dt, logits, draft_logits, draft_ids, uniforms, B, N, V, temperature, n_accept, accept,
                           next_token, argmax_ids, sampled_ids, p_draft, q_draft, row_lse, ws, SCRATCH_BYTES, &v);
  if (st != ISD_OK) return st;
  const hipError_t e = isd::launch_verify(v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return isd::set_error(ISD_ERR_HIP, "verify_noalloc launch: %s", hipGetErrorString(e));
  return isd::clear_error();
}
