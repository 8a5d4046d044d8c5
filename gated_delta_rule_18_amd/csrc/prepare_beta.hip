// The prologue of the chunkwise forward on its own: the Kaczmarz step size
// beta_t = eta_t / (||k_t||^2 + eps) ("Kaczmarz Linear Attention", Abstract) and the
// chunk-local inclusive prefix sum of log(alpha) ("Deep Dive into KDA", section 3: the
// intra-chunk accumulated decay is computed once by prefix sums; section 5: in the log
// domain). One wave per (b, h, chunk): lane r owns token chunk_start + r.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {
namespace {

template <typename E, int DK>
__global__ __launch_bounds__(kWave) void prepare_beta_kernel(
    const E* __restrict__ k, const float* __restrict__ eta, const float* __restrict__ log_alpha,
    float* __restrict__ beta, float* __restrict__ gcum, int64_t T, int64_t H, int64_t nchunks, float eps) {
  typedef typename Vec16<E>::type V;
  constexpr int N = Vec16<E>::N;
  const int64_t c = blockIdx.x % nchunks;
  const int64_t bh = blockIdx.x / nchunks;
  const int64_t h = bh % H;
  const int64_t b = bh / H;
  const int64_t t = c * kChunk + threadIdx.x;
  const bool valid = t < T;
  const int64_t idx = (b * T + t) * H + h;
  float n = 0.f, la = 0.f, e = 0.f;
  if (valid) {
    const V* kr = reinterpret_cast<const V*>(k + idx * DK);
#pragma unroll
    for (int i = 0; i < DK / N; ++i) {
      const V x = kr[i];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float f = to_f32(x[j]);
        n += f * f;
      }
    }
    la = log_alpha[idx];
    e = eta[idx];
  }
  const float G = wave_inclusive_scan(la);
  if (valid) {
    beta[idx] = e / (n + eps);
    if (gcum) gcum[idx] = G;
  }
}

template <typename E>
hipError_t launch_e(const PrepareArgs& a, hipStream_t stream) {
  const int64_t nchunks = (a.T + kChunk - 1) / kChunk;
  const int64_t grid = a.B * a.H * nchunks;
  if (a.d_k == 128)
    hipLaunchKernelGGL((prepare_beta_kernel<E, 128>), dim3((unsigned)grid), dim3(kWave), 0, stream,
                       (const E*)a.k, a.eta, a.log_alpha, a.beta, a.gcum, a.T, a.H, nchunks, a.eps);
  else
    hipLaunchKernelGGL((prepare_beta_kernel<E, 64>), dim3((unsigned)grid), dim3(kWave), 0, stream,
                       (const E*)a.k, a.eta, a.log_alpha, a.beta, a.gcum, a.T, a.H, nchunks, a.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare_beta(const PrepareArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_e<bf16>(a, stream) : launch_e<float>(a, stream);
}

}  // namespace kla
