// Host-side dispatch of the prefill, gate-sweep and calibration kernels: picks the instantiation
// for the head dimension, query tile, workgroup width, gate and K/V layout.
#include "bsfa_internal.h"

#include <mutex>
#include <utility>
#include <vector>

namespace bsfa {
namespace {

__global__ void zero_u64_kernel(unsigned long long* p) { *p = 0ull; }
__global__ void zero_words_kernel(unsigned* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

}  // namespace

int gate_sweep_heads(int block_q, int group, bool fp8) {
  (void)block_q;
  // the FP8 sweep takes a whole group of four (its K stream then leaves L2 half as often)
  if (fp8 && group % 4 == 0) return 4;
  return group % 2 == 0 ? 2 : 1;
}

hipError_t launch_gate_sweep(const PrefillArgs& a, int head_dim, int block_q, hipStream_t stream) {
  const int hpw = gate_sweep_heads(block_q, a.G, a.q8 != nullptr);
  if (a.q8) {
    if (head_dim == 128)
      return block_q == 128 ? launch_sweep_fp8_tile<128, 128>(a, hpw, stream)
                            : launch_sweep_fp8_tile<128, 64>(a, hpw, stream);
    return block_q == 128 ? launch_sweep_fp8_tile<64, 128>(a, hpw, stream)
                          : launch_sweep_fp8_tile<64, 64>(a, hpw, stream);
  }
  if (head_dim == 128)
    return block_q == 128 ? launch_sweep_tile<128, 128>(a, hpw, stream)
                          : launch_sweep_tile<128, 64>(a, hpw, stream);
  return block_q == 128 ? launch_sweep_tile<64, 128>(a, hpw, stream)
                        : launch_sweep_tile<64, 64>(a, hpw, stream);
}

int waves_per_workgroup(int block_q, int group) {
  const int wph = block_q / kRowsPerWave;
  int hpw = 4 / wph;
  while (hpw > 1 && group % hpw != 0) hpw >>= 1;
  return hpw * wph;
}

int prefill_waves_per_workgroup(int block_q, int group, int gate) {
  return gate == kAbsolute || gate == kAbsVote ? block_q / kRowsPerWave
                                               : waves_per_workgroup(block_q, group);
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_q, int gate,
                          hipStream_t stream) {
  const int nw = prefill_waves_per_workgroup(block_q, a.G, gate);
  if (a.pages) {
    if (head_dim == 128)
      return block_q == 128 ? launch_prefill_tile<128, 128, true>(a, nw, gate, stream)
                            : launch_prefill_tile<128, 64, true>(a, nw, gate, stream);
    return block_q == 128 ? launch_prefill_tile<64, 128, true>(a, nw, gate, stream)
                          : launch_prefill_tile<64, 64, true>(a, nw, gate, stream);
  }
  if (head_dim == 128)
    return block_q == 128 ? launch_prefill_tile<128, 128, false>(a, nw, gate, stream)
                          : launch_prefill_tile<128, 64, false>(a, nw, gate, stream);
  return block_q == 128 ? launch_prefill_tile<64, 128, false>(a, nw, gate, stream)
                        : launch_prefill_tile<64, 64, false>(a, nw, gate, stream);
}

hipError_t launch_calibrate(const CalibArgs& a, int head_dim, int block_q, hipStream_t stream) {
  const int nw = waves_per_workgroup(block_q, a.G);
  if (head_dim == 128) {
    return block_q == 128 ? launch_calibrate_tile<128, 128>(a, nw, stream)
                          : launch_calibrate_tile<128, 64>(a, nw, stream);
  }
  return block_q == 128 ? launch_calibrate_tile<64, 128>(a, nw, stream)
                        : launch_calibrate_tile<64, 64>(a, nw, stream);
}

hipError_t launch_block_means(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  if (a.pages)
    return head_dim == 128 ? launch_means_tile<128, true>(a, stream)
                           : launch_means_tile<64, true>(a, stream);
  return head_dim == 128 ? launch_means_tile<128, false>(a, stream)
                         : launch_means_tile<64, false>(a, stream);
}

hipError_t launch_quantize_qk(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  if (a.pages)
    return head_dim == 128 ? launch_quant_tile<128, true>(a, stream)
                           : launch_quant_tile<64, true>(a, stream);
  return head_dim == 128 ? launch_quant_tile<128, false>(a, stream)
                         : launch_quant_tile<64, false>(a, stream);
}

int resident_workgroups(const void* kernel, int block, int fallback) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<int, const void*>, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fallback;
  const std::pair<int, const void*> key(dev, kernel);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& e : cache)
      if (e.first == key) return e.second;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
      cus < 1 || per_cu < 1) {
    (void)hipGetLastError();
    return fallback;
  }
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace_back(key, cus * per_cu);
  return cus * per_cu;
}

hipError_t launch_zero_u64(unsigned long long* p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_zero_words(unsigned* p, int n, hipStream_t stream) {
  if (n < 1 || n > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace bsfa
