// Host side of the Q8_0 matvec kernels: instance selection and launch.
#include <map>
#include <mutex>
#include <utility>

#include "q8_gemv_kernel.h"

namespace q8 {
namespace {

__global__ void zero_fill_kernel(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// Records the XCD each workgroup runs on (the XCC_ID hardware register, low
// four bits); written with a vector store by lane 0.
__global__ void xcc_probe_kernel(uint32_t *out) {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  if (threadIdx.x == 0) out[blockIdx.x] = x & 15u;
}

__global__ void empty_product_kernel(float *C, int M, int N, float alpha, const float *corr) {
  const size_t total = (size_t)M * N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    float y = alpha * 0.f;
    if (corr != nullptr) y = fmaf(corr[i / N], C[i], y);
    C[i] = y;
  }
}

// Dynamic LDS each (kernel instance, device) has opted in to.
std::mutex g_lds_mu;
std::map<std::pair<const void *, int>, size_t> g_lds_granted;

GemvKernel pick(int vec, int m_tile) {
  switch (vec) {
    case 16: return gemv_kernel_v16(m_tile);
    case 8: return gemv_kernel_v8(m_tile);
    case 4: return gemv_kernel_v4(m_tile);
    case 2: return gemv_kernel_v2(m_tile);
    case 1: return gemv_kernel_v1(m_tile);
    default: return nullptr;
  }
}

}  // namespace

hipError_t launch_gemv(int vec, int m_tile, const GemvArgs &args, int m_chunks, size_t lds_bytes,
                       hipStream_t stream) {
  GemvKernel k = pick(vec, m_tile);
  if (k == nullptr) return hipErrorInvalidValue;
  // A wave's activations must fit the staging registers.
  const int count_max = args.upw + (args.rem > 0 ? 1 : 0);
  if ((size_t)m_tile * count_max * kBlock > (size_t)64 * kStageRegs) return hipErrorInvalidValue;
  if (lds_bytes > kMaxGemvLds) return hipErrorInvalidValue;
  if (lds_bytes > 64 * 1024) {
    // Above the default dynamic LDS limit the launch must opt in, once per
    // kernel instance and device, to the largest size it is launched with.
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_lds_mu);
    size_t &granted = g_lds_granted[std::make_pair(reinterpret_cast<const void *>(k), dev)];
    if (granted < lds_bytes) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds_bytes);
      if (e != hipSuccess) {
        (void)hipGetLastError();  // do not leave the error for the caller's next HIP call
        return e;
      }
      granted = lds_bytes;
    }
  }
  hipLaunchKernelGGL(k, dim3((unsigned)args.n_wg, (unsigned)m_chunks, 1), dim3(kThreads), lds_bytes, stream, args);
  return hipGetLastError();
}

hipError_t launch_empty_product(float *C, int M, int N, float alpha, const float *corr, hipStream_t stream) {
  const size_t total = (size_t)M * N;
  if (total == 0) return hipSuccess;
  size_t blocks = (total + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(empty_product_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, M, N, alpha, corr);
  return hipGetLastError();
}

hipError_t launch_xcc_probe(uint32_t *out, int n_wg, hipStream_t stream) {
  if (n_wg < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xcc_probe_kernel, dim3((unsigned)n_wg), dim3(64), 0, stream, out);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void *p, size_t n_words, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t *)p, n_words);
  return hipGetLastError();
}

}  // namespace q8
