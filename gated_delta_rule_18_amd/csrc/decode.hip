// Single-token recurrent decode step of Kaczmarz Linear Attention.
//
// Token update: "Deep Dive into KDA", section 2.2 (gated delta rule) with the Kaczmarz
// step size of "Kaczmarz Linear Attention", Abstract; state stored [d_k][d_v] (S = M^T).
// Per head:  n = ||k||^2, kappa = k.q, beta = eta / (n + eps), alpha = exp(log_alpha)
//            u = alpha S^T k,  p = alpha S^T q            (one pass over S)
//            delta = beta (v - u),  o = p + kappa delta    (= S_new^T q)
//            S <- alpha S + k delta^T                      (in place)
// The kernel is HBM-bound: it reads and writes the fp32 state once. One wave owns one d_v
// slice (DVS columns) of one head: lane (rg, cg) holds rows rg, rg + RG, ... of columns
// [4 cg, 4 cg + 4) in registers between the read and the write, and every reduction (over
// d_k for S^T k and S^T q, and for ||k||^2 and k.q) is a wave shuffle. No LDS, no barrier:
// the only latency is one round trip to memory.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {
namespace {

constexpr int kXcdCount = 8;  // MI355X

template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kWave) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ eta, const float* __restrict__ log_alpha, float* __restrict__ state,
    E* __restrict__ o, int64_t heads, float eps) {
  constexpr int CG = DVS / 4;        // float4 column groups of the slice
  constexpr int RG = kWave / CG;     // row groups
  constexpr int RPT = DK / RG;       // rows per lane
  constexpr int NS = DV / DVS;       // slices per head
  constexpr int KPL = DK / kWave;    // elements of k (and q) per lane for the norms
  static_assert(RG * CG == kWave && RPT * RG == DK && KPL * kWave == DK, "shape");

  // Workgroups are dealt round-robin to the 8 XCDs: give the NS slices of one head ids that are
  // congruent mod 8, so they share one XCD's L2 (slices narrower than a 128-byte line share lines).
  const int xcd = blockIdx.x % kXcdCount;
  const int local = blockIdx.x / kXcdCount;
  const int64_t head = (int64_t)(local / NS) * kXcdCount + xcd;
  const int slice = local % NS;
  if (head >= heads) return;
  const int lane = threadIdx.x;
  const int cg = lane % CG, rg = lane / CG;
  const int col0 = slice * DVS + 4 * cg;

  // State first: it is the bulk of the traffic.
  float* S = state + head * (int64_t)DK * DV;
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = *reinterpret_cast<const f32x4*>(S + (int64_t)(rg + RG * m) * DV + col0);

  float kk[KPL], qq[KPL];
  float nk = 0.f, kq = 0.f;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    kk[j] = to_f32(k[head * DK + lane + kWave * j]);
    qq[j] = to_f32(q[head * DK + lane + kWave * j]);
    nk += kk[j] * kk[j];
    kq += kk[j] * qq[j];
  }
  nk = wave_sum(nk);
  kq = wave_sum(kq);
  const float alpha = __expf(log_alpha[head]);
  const float beta = eta[head] / (nk + eps);
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[head * DV + col0 + e]);

  // Partial S^T k and S^T q over this lane's rows; row r's k and q come from lane r % 64.
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
  float krow[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int r = rg + RG * m;            // (RG * m) / 64 is this row's slot: RG divides 64
    const int slot = (RG * m) / kWave;
    krow[m] = __shfl(kk[slot], r % kWave, kWave);
    const float qr = __shfl(qq[slot], r % kWave, kWave);
    u += s[m] * krow[m];
    pq += s[m] * qr;
  }
#pragma unroll
  for (int off = CG; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[e] += __shfl_xor(u[e], off, kWave);
      pq[e] += __shfl_xor(pq[e], off, kWave);
    }
  }
  const f32x4 delta = beta * (vv - alpha * u);
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[head * DV + col0 + e] = from_f32<E>(alpha * pq[e] + kq * delta[e]);
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    *reinterpret_cast<f32x4*>(S + (int64_t)(rg + RG * m) * DV + col0) = s[m] * alpha + delta * krow[m];
}

template <typename E, int DK, int DV, int DVS>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  const int64_t heads = a.B * a.H;
  const int64_t grid = (heads + kXcdCount - 1) / kXcdCount * kXcdCount * (DV / DVS);
  hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, DVS>), dim3((unsigned)grid), dim3(kWave), 0, stream,
                     (const E*)a.q, (const E*)a.k, (const E*)a.v, a.eta, a.log_alpha, a.state, (E*)a.o, heads,
                     a.eps);
  return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t stream) {
  // Many heads: 32-column slices (16 rows of float4 per lane). Few heads: 16-column slices, so
  // that the grid still puts a couple of waves on every CU.
  if (a.B * a.H >= 512) return launch<E, DK, DV, 32>(a, stream);
  return launch<E, DK, DV, 16>(a, stream);
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
