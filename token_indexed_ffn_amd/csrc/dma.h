// Copies on the GPU's DMA (SDMA) engines through the HSA runtime, between
// device memory and pinned host memory, completed into HSA signals that the
// host waits on.  A hipMemcpyAsync between pinned host memory and the device
// may be carried out by a copy kernel, whose workgroups take compute units
// from the kernels beside it; the DMA engines take none.
#pragma once

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>
#include <stdint.h>
#include <stddef.h>

namespace staple {

struct SdmaCopier {
  bool ready = false;
  hsa_agent_t gpu{}, cpu{};
  static constexpr int kMaxSignals = 16;
  hsa_signal_t sig[kMaxSignals] = {};
  int n_sig = 0;

  struct Find {
    uint32_t bdf = 0;        // bus << 8 | device << 3 of the GPU to find
    hsa_agent_t gpu{}, cpu{};
    bool got_gpu = false, got_cpu = false;
  };
  static hsa_status_t visit(hsa_agent_t a, void* data) {
    Find* f = static_cast<Find*>(data);
    hsa_device_type_t t;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) != HSA_STATUS_SUCCESS) return HSA_STATUS_SUCCESS;
    if (t == HSA_DEVICE_TYPE_CPU && !f->got_cpu) {
      f->cpu = a;
      f->got_cpu = true;
    } else if (t == HSA_DEVICE_TYPE_GPU && !f->got_gpu) {
      uint32_t bdf = 0;
      if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) ==
              HSA_STATUS_SUCCESS && (bdf & ~7u) == f->bdf) {
        f->gpu = a;
        f->got_gpu = true;
      }
    }
    return HSA_STATUS_SUCCESS;
  }

  // For HIP device `device`, with `n` completion signals; on any failure the
  // copier stays unready.
  void init(int device, int n) {
    if (n > kMaxSignals) return;
    int bus = -1, dev = -1;
    if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, device) != hipSuccess ||
        hipDeviceGetAttribute(&dev, hipDeviceAttributePciDeviceId, device) != hipSuccess)
      return;
    if (hsa_init() != HSA_STATUS_SUCCESS) return;
    Find f;
    f.bdf = (static_cast<uint32_t>(bus) << 8) | (static_cast<uint32_t>(dev) << 3);
    if (hsa_iterate_agents(&SdmaCopier::visit, &f) != HSA_STATUS_SUCCESS || !f.got_gpu || !f.got_cpu) {
      (void)hsa_shut_down();
      return;
    }
    gpu = f.gpu;
    cpu = f.cpu;
    for (n_sig = 0; n_sig < n; ++n_sig)
      if (hsa_signal_create(0, 0, nullptr, &sig[n_sig]) != HSA_STATUS_SUCCESS) break;
    ready = n_sig == n;
    if (!ready) release();
  }
  void release() {
    for (int i = 0; i < n_sig; ++i) (void)hsa_signal_destroy(sig[i]);
    if (n_sig > 0 || ready) (void)hsa_shut_down();
    n_sig = 0;
    ready = false;
  }
  // Starts copy i: device src -> pinned host dst.
  bool start_d2h(int i, void* dst, const void* src, size_t bytes) {
    hsa_signal_store_screlease(sig[i], 1);
    return hsa_amd_memory_async_copy(dst, cpu, src, gpu, bytes, 0, nullptr, sig[i]) == HSA_STATUS_SUCCESS;
  }
  // Starts copy i: pinned host src -> device dst.
  bool start_h2d(int i, void* dst, const void* src, size_t bytes) {
    hsa_signal_store_screlease(sig[i], 1);
    return hsa_amd_memory_async_copy(dst, gpu, src, cpu, bytes, 0, nullptr, sig[i]) == HSA_STATUS_SUCCESS;
  }
  // Waits for copy i; false when the engine reported an error.
  bool wait(int i) {
    hsa_signal_value_t v;
    do {
      v = hsa_signal_wait_scacquire(sig[i], HSA_SIGNAL_CONDITION_LT, 1, UINT64_MAX, HSA_WAIT_STATE_BLOCKED);
    } while (v >= 1);
    return v == 0;
  }
};

}  // namespace staple
