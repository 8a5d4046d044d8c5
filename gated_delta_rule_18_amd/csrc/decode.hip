// Single-token recurrent decode step of Kaczmarz Linear Attention.
//
// Token update: "Deep Dive into KDA", section 2.2 (gated delta rule) with the Kaczmarz
// step size of "Kaczmarz Linear Attention", Abstract; state stored [d_k][d_v] (S = M^T).
// Per head:  n = ||k||^2, kappa = k.q, beta = eta / (n + eps), alpha = exp(log_alpha)
//            u = alpha S^T k,  p = alpha S^T q            (one pass over S)
//            delta = beta (v - u),  o = p + kappa delta    (= S_new^T q)
//            S <- alpha S + k delta^T                      (in place)
// The kernel is HBM-bound: it reads and writes the fp32 state once. One workgroup owns
// one d_v slice of one head and keeps that slice in registers between the read and the
// write, so the state crosses HBM exactly twice per step.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {
namespace {

constexpr int kDecodeThreads = 256;

// DVS: width of the d_v slice one workgroup owns. Thread t owns columns
// [4*(t % CG), +4) of the slice (one float4) and rows rg, rg + RG, rg + 2 RG, ...
template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ eta, const float* __restrict__ log_alpha, float* __restrict__ state,
    E* __restrict__ o, int64_t heads, float eps) {
  constexpr int CG = DVS / 4;               // float4 column groups per slice
  constexpr int RG = kDecodeThreads / CG;   // row groups
  constexpr int RPT = DK / RG;              // rows per thread
  constexpr int NSLICE = DV / DVS;
  constexpr int WAVES = kDecodeThreads / kWave;
  constexpr int RG_PER_WAVE = kWave / CG;   // row groups inside one wave
  static_assert(RPT >= 1 && DK % RG == 0, "slice too narrow for this d_k");

  const int64_t head = blockIdx.x / NSLICE;
  const int slice = blockIdx.x % NSLICE;
  if (head >= heads) return;
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int wave = tid / kWave;
  const int col0 = slice * DVS + 4 * cg;

  __shared__ float s_k[DK];
  __shared__ float s_q[DK];
  __shared__ float s_red[WAVES][2][DVS];
  __shared__ float s_delta[DVS];
  __shared__ float s_scalar[2];

  // Issue the state loads first: they are the bulk of the traffic.
  float* S = state + head * (int64_t)DK * DV;
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    s[m] = *reinterpret_cast<const f32x4*>(S + (int64_t)row * DV + col0);
  }

  // q and k of this head, as fp32, plus the two reductions ||k||^2 and k.q (wave 0).
  if (tid < DK) {
    s_k[tid] = to_f32(k[head * DK + tid]);
    s_q[tid] = to_f32(q[head * DK + tid]);
  }
  __syncthreads();
  if (wave == 0) {
    float nk = 0.f, kq = 0.f;
    for (int i = tid; i < DK; i += kWave) {
      nk += s_k[i] * s_k[i];
      kq += s_k[i] * s_q[i];
    }
    nk = wave_sum(nk);
    kq = wave_sum(kq);
    if (tid == 0) {
      s_scalar[0] = nk;
      s_scalar[1] = kq;
    }
  }

  // Partial S^T k and S^T q over this thread's rows.
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const float kr = s_k[row], qr = s_q[row];
    u += s[m] * kr;
    p += s[m] * qr;
  }
  // Reduce over the row groups of this wave (lanes that share cg), then across waves.
#pragma unroll
  for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] += __shfl_xor(u[e], off, kWave);
      p[e] += __shfl_xor(p[e], off, kWave);
    }
  }
  if ((tid % kWave) < CG) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s_red[wave][0][4 * cg + e] = u[e];
      s_red[wave][1][4 * cg + e] = p[e];
    }
  }
  __syncthreads();

  const float alpha = __expf(log_alpha[head]);
  const float beta = eta[head] / (s_scalar[0] + eps);
  const float kappa = s_scalar[1];
  if (tid < DVS) {
    float uu = 0.f, pp = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      uu += s_red[w][0][tid];
      pp += s_red[w][1][tid];
    }
    const int j = slice * DVS + tid;
    const float delta = beta * (to_f32(v[head * DV + j]) - alpha * uu);
    s_delta[tid] = delta;
    o[head * DV + j] = from_f32<E>(alpha * pp + kappa * delta);
  }
  __syncthreads();

  const f32x4 d = *reinterpret_cast<const f32x4*>(&s_delta[4 * cg]);
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const f32x4 snew = s[m] * alpha + d * s_k[row];
    *reinterpret_cast<f32x4*>(S + (int64_t)row * DV + col0) = snew;
  }
  (void)RG_PER_WAVE;
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t stream) {
  // Narrow slices when there are few heads, so that the grid still fills 256 CUs.
  const int64_t heads = a.B * a.H;
  if (heads >= 1024 || DV == 64) {
    constexpr int DVS = DV;
    const int64_t grid = heads * (DV / DVS);
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, DVS>), dim3((unsigned)grid), dim3(kDecodeThreads), 0,
                       stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.eta, a.log_alpha, a.state,
                       (E*)a.o, heads, a.eps);
  } else {
    constexpr int DVS = 32;
    const int64_t grid = heads * (DV / DVS);
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, DVS>), dim3((unsigned)grid), dim3(kDecodeThreads), 0,
                       stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.eta, a.log_alpha, a.state,
                       (E*)a.o, heads, a.eps);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const DecodeArgs& a, hipStream_t stream) {
  if (a.d_k == 128 && a.d_v == 128) return launch_dk_dv<E, 128, 128>(a, stream);
  if (a.d_k == 64 && a.d_v == 64) return launch_dk_dv<E, 64, 64>(a, stream);
  if (a.d_k == 128 && a.d_v == 64) return launch_dk_dv<E, 128, 64>(a, stream);
  return launch_dk_dv<E, 64, 128>(a, stream);
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_e<bf16>(a, stream) : launch_e<float>(a, stream);
}

}  // namespace kla
