// Device check of the gate preconditions: every g in [-5, 0] (the lower bound on the
// per-step log-decay from the orkas.ai Kimi K3 page, section "Eine Untergrenze, die einen
// GPU-Codepfad beseitigte") and every beta in [0, 1]. NaN counts as a violation.
// Each block writes its own count (no atomics); the host adds them up.
#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {
constexpr int kCheckBlocks = 1024;

template <typename T>
__global__ __launch_bounds__(256) void check_gates_kernel(const T* __restrict__ g, int64_t n_g,
                                                          const T* __restrict__ beta,
                                                          int64_t n_beta,
                                                          int64_t* __restrict__ counts) {
  __shared__ int64_t part[256];
  int64_t bad = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_g; i += stride) {
    const float x = ld(g, i);
    bad += !(x >= -5.0f && x <= 0.0f);
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_beta; i += stride) {
    const float x = ld(beta, i);
    bad += !(x >= 0.0f && x <= 1.0f);
  }
  part[threadIdx.x] = bad;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = part[0];
}
}  // namespace

int check_blocks() { return kCheckBlocks; }

hipError_t launch_check_gates(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                              bool bf16, int64_t* counts, int n_blocks, hipStream_t stream) {
  const dim3 grid((unsigned)std::min(std::max(n_blocks, 1), kCheckBlocks));
  if (bf16)
    hipLaunchKernelGGL(check_gates_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(g), n_g, static_cast<const uint16_t*>(beta),
                       n_beta, counts);
  else
    hipLaunchKernelGGL(check_gates_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(g), n_g, static_cast<const float*>(beta), n_beta,
                       counts);
  return hipGetLastError();
}

}  // namespace kda
