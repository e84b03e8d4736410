// Quantisation of compressed-KV rows into the FP4 E2M1 latent / FP8 E4M3
// tail cache format ("Lab tổng hợp DeepSeek-V4.1-Flash", section "3 Giải
// pháp"; the format itself is described in kv4.h).  One wave per row.
#include "common.h"
#include "kernels.h"
#include "kv4.h"

namespace csa {
namespace {

// grid: rows / 4, 4 waves per block, one row per wave
__global__ __launch_bounds__(256) void kv4_quantize(Kv4Args a) {
  const int64_t r = int64_t(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (r >= a.rows) return;
  extern __shared__ float ybuf[];  // one row per wave
  float* y = ybuf + (threadIdx.x / kWave) * a.D;
  const int lane = threadIdx.x % kWave;
  for (int c = lane; c < a.D; c += kWave) y[c] = load_elem(a.x, a.x_dtype, r * a.D + c);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  kv4_store_row(y, a.D, a.rope_dim, static_cast<unsigned char*>(a.out) + r * a.row_bytes);
}

}  // namespace

hipError_t launch_kv4_quantize(const Kv4Args& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(kv4_quantize, dim3(unsigned((a.rows + 3) / 4)), dim3(256), size_t(4) * a.D * sizeof(float),
                     stream, a);
  return hipGetLastError();
}

}  // namespace csa
