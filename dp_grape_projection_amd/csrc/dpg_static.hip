// The one-call step without a caller workspace: dpg_private_step_static runs
// dpg_private_step in a scratch array the library holds in each GPU's memory,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc). It calls no
// hipMalloc, hipFree or other allocating routine.
//
// Nothing in the scratch has to start at zero: every region the step reads
// (P, Xt, split and group partials, norm partials, clip factors, U) is
// written by an earlier kernel of the same call. All calls on one GPU share
// that GPU's array, so calls that overlap in time on one GPU (two host
// threads, or two streams without an ordering between them) race on it.
#include <mutex>
#include <string>

#include "dpg.h"
#include "dpg_internal.hpp"

namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // 64 MiB per GPU

// One array per GPU, allocated when the code object is loaded on that GPU
// and held until the process ends. In host code its name is only a stand-in
// for the symbol: the device address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current, and only that address is handed
// to kernels.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's scratch address, taken on the first call on that
// device; nullptr (with the error recorded in *status) on failure.
void* device_scratch(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = dpg::record_error(DPG_ERR_HIP,
                                (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = dpg::record_error(DPG_ERR_UNSUPPORTED,
                                "device index beyond the static scratch table");
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *status = dpg::record_error(
          DPG_ERR_HIP,
          (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e)).c_str());
      return nullptr;
    }
    g_ptr[dev] = ptr;
  }
  *status = DPG_OK;
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t dpg_static_scratch_bytes(void) { return kStaticScratchBytes; }

int dpg_private_step_static(const dpg_layer_grad* layers, const dpg_layer_param* params,
                            int32_t n_layers, int64_t B, int64_t T, int32_t r,
                            int32_t dtype, double clip_C, double sigma, double lr,
                            double beta1, double beta2, double eps, uint64_t seed,
                            uint64_t step, uint64_t proj_step, float* sample_norms,
                            void* stream) {
  size_t need = 0;
  int st = dpg_step_workspace_size(layers, n_layers, B, T, r, dtype, &need);
  if (st) return st;
  if (need > kStaticScratchBytes)
    return dpg::record_error(
        DPG_ERR_WORKSPACE,
        ("this step needs " + std::to_string(need) + " bytes of scratch, more than the " +
         std::to_string(kStaticScratchBytes) +
         " bytes of the static scratch; call dpg_private_step with a workspace")
            .c_str());
  void* ws = device_scratch(&st);
  if (!ws) return st;
  return dpg_private_step(layers, params, n_layers, B, T, r, dtype, clip_C, sigma, lr,
                          beta1, beta2, eps, seed, step, proj_step, sample_norms, ws,
                          kStaticScratchBytes, stream);
}

}  // extern "C"
