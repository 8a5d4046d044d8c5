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
// [4 cg, 4 cg + 4) in registers between the read and the write, with the k and q entries of
// those rows. ||k||^2, k.q, S^T k and S^T q are summed over the lane's rows and then reduced in
// one pass over the row groups (DPP rotations within 16-lane rows, two exchanges across rows).
// No LDS storage, no barrier, and no source-level branch ahead of the stores: every load, the
// per-head scalars included, is issued at the top, so the only latency is one round trip to
// memory.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {
namespace {

// States of at least this many bytes (twice the MI355X's 256 MB last-level cache) are rewritten
// with streaming stores: cache policy bits SC1 | NT of the buffer store (system scope,
// non-temporal).
constexpr int64_t kStreamStateBytes = int64_t(512) << 20;
constexpr int kStreamStore = 16 | 2;

// Sum of x over the lanes of the wave whose index is congruent to this lane's mod CG (CG a power
// of two, 4 <= CG <= 16): DPP row rotations inside each 16-lane row, then exchanges across rows.
// (The gfx950 row swaps v_permlane16/32_swap would avoid the LDS crossbar here, but this
// compiler folds the sum of the two results of one swap into twice the first one.)
template <int CG>
__device__ __forceinline__ float class_sum(float x) {
  static_assert(CG == 4 || CG == 8 || CG == 16, "class width");
  if constexpr (CG == 4)  // row_ror:4
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  if constexpr (CG <= 8)  // row_ror:8
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __shfl_xor(x, 16, kWave);
  x += __shfl_xor(x, 32, kWave);
  return x;
}

// KDA: log_alpha holds log a [heads][DK], a per-channel decay of the state's rows
// ("Deep Dive into KDA", section 2.3): u = (Diag(a) S)^T k, p = (Diag(a) S)^T q,
// delta = beta (v - u), o = p + (k.q) delta, S <- Diag(a) S + k delta^T.
// BG: eta holds beta itself (gated DeltaNet). The arguments (seven pointers, heads_x and eps)
// fill one 64-byte line, so all their scalar loads hit the line the first one brings in.
// heads_x packs the head count (bits 0..27; the C ABI bounds it below 2^28) and log2 of the
// XCD grouping width X (bits 28..31), X the largest power of two not above the device's XCDs.
// STREAM: the state is far larger than the last-level cache, so its rewrite is stored
// non-temporally at system scope (it would only evict the next step's reads): measured on a
// 512 MiB state 208 -> 196 us per step; on states the cache holds it is slower (64 MiB: 19.9 ->
// 27.2 us), so it is chosen by state size.
template <typename E, int DK, int DV, int DVS, bool KDA, bool BG, bool STREAM = false>
__global__ __launch_bounds__(kWave) void decode_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ eta, const float* __restrict__ log_alpha, float* __restrict__ state,
    E* __restrict__ o, unsigned heads_x, float eps) {
  constexpr int CG = DVS / 4;        // float4 column groups of the slice
  constexpr int RG = kWave / CG;     // row groups
  constexpr int RPT = DK / RG;       // rows per lane
  constexpr int NS = DV / DVS;       // slices per head
  static_assert(RG * CG == kWave && RPT * RG == DK, "shape");

  // Workgroups are dealt round-robin to the XCDs: within each full group of X heads, give the
  // NS slices of one head ids that are congruent mod X, so they share one XCD's L2 (slices
  // narrower than a 128-byte line share lines). The heads past the last full group take the
  // remaining ids in order. The grid is exactly heads x NS, so no workgroup idles and nothing
  // branches ahead of the loads.
  const unsigned heads = heads_x & 0x0fffffffu, xs = heads_x >> 28;
  const unsigned b = blockIdx.x;
  const unsigned full = (heads >> xs << xs) * NS;
  const bool grouped = b < full;
  const unsigned r = grouped ? b >> xs : b - full;  // rank within the group / the tail
  const int64_t head = grouped ? ((r / NS) << xs) + (b & ((1u << xs) - 1)) : full / NS + r / NS;
  const int slice = r % NS;
  const int lane = threadIdx.x;
  const int cg = lane % CG, rg = lane / CG;
  const int col0 = slice * DVS + 4 * cg;

  // Everything is loaded up front: the state rows rg + RG m of this lane's four columns (the bulk
  // of the traffic), and the k and q entries of those same rows (read directly when a lane has
  // few rows, which keeps them off the critical path).
  float* S = state + head * (int64_t)DK * DV;
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) s[m] = *reinterpret_cast<const f32x4*>(S + (int64_t)(rg + RG * m) * DV + col0);
  float kr[RPT], qr[RPT], lr_[RPT];
  if constexpr (RPT <= 8) {
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      kr[m] = to_f32(k[head * DK + rg + RG * m]);
      qr[m] = to_f32(q[head * DK + rg + RG * m]);
      if constexpr (KDA) lr_[m] = log_alpha[head * DK + rg + RG * m];
    }
  } else {
    // Many rows per lane: load k and q once across the wave and pass row r's values from lane
    // r % 64 (fewer memory instructions for a kernel that is bound by memory).
    constexpr int KPL = DK / kWave;
    float kk[KPL], qq[KPL], ll[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      kk[j] = to_f32(k[head * DK + lane + kWave * j]);
      qq[j] = to_f32(q[head * DK + lane + kWave * j]);
      if constexpr (KDA) ll[j] = log_alpha[head * DK + lane + kWave * j];
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int r = rg + RG * m, slot = (RG * m) / kWave;  // RG divides 64
      kr[m] = __shfl(kk[slot], r % kWave, kWave);
      qr[m] = __shfl(qq[slot], r % kWave, kWave);
      if constexpr (KDA) lr_[m] = __shfl(ll[slot], r % kWave, kWave);
    }
  }
  f32x4 vv;
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = to_f32(v[head * DV + col0 + e]);
  // Without a gate (log_alpha null) the load reads eta's entry instead and alpha = exp(0) = 1:
  // the load is unconditional, so it need not wait behind a branch.
  const float la_h = KDA ? 0.f : *(log_alpha ? log_alpha + head : eta + head);
  const float alpha = KDA ? 1.f : __expf(log_alpha ? la_h : 0.f);
  float ar[RPT];  // per-row decay (KDA)
#pragma unroll
  for (int m = 0; m < RPT; ++m) ar[m] = KDA ? __expf(lr_[m]) : 1.f;
  const float et = eta[head];  // eta, or beta itself when beta_given

  // Partial sums over this lane's rows, then one joint reduction over the row groups (the lanes
  // congruent mod CG): ||k||^2, k.q, (S^T k) and (S^T q) for the four columns.
  float nk = 0.f, kq = 0.f;
  f32x4 u = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    nk += kr[m] * kr[m];
    kq += kr[m] * qr[m];
    if constexpr (KDA) {
      u += s[m] * (ar[m] * kr[m]);
      pq += s[m] * (ar[m] * qr[m]);
    } else {
      u += s[m] * kr[m];
      pq += s[m] * qr[m];
    }
  }
  nk = class_sum<CG>(nk);
  kq = class_sum<CG>(kq);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] = class_sum<CG>(u[e]);
    pq[e] = class_sum<CG>(pq[e]);
  }
  const float beta = BG ? et : et / (nk + eps);
  const f32x4 delta = beta * (vv - alpha * u);
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[head * DV + col0 + e] = from_f32<E>(alpha * pq[e] + kq * delta[e]);
  }
  if constexpr (STREAM) {
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(S, (short)0, DK * DV * 4, 0x00020000);
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4v, s[m] * (alpha * ar[m]) + delta * kr[m]), rs,
                                             (int)(((rg + RG * m) * DV + col0) * 4), 0, kStreamStore);
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      *reinterpret_cast<f32x4*>(S + (int64_t)(rg + RG * m) * DV + col0) = s[m] * (alpha * ar[m]) + delta * kr[m];
  }
}

template <typename E, int DK, int DV, int DVS, bool KDA, bool BG>
void launch_kernel(const DecodeArgs& a, unsigned heads_x, int64_t grid, hipStream_t stream) {
  const bool stream_state = DVS == 64 && (a.B * a.H) * (int64_t)DK * DV * 4 >= kStreamStateBytes;
  if (stream_state)
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, DVS, KDA, BG, DVS == 64>), dim3((unsigned)grid), dim3(kWave),
                       0, stream, (const E*)a.q, (const E*)a.k, (const E*)a.v, a.eta, a.log_alpha, a.state, (E*)a.o,
                       heads_x, a.eps);
  else
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, DVS, KDA, BG>), dim3((unsigned)grid), dim3(kWave), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.eta, a.log_alpha, a.state, (E*)a.o, heads_x,
                       a.eps);
}

template <typename E, int DK, int DV, int DVS>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
  // 1 <= heads < 2^28 and the grid below fit in an int (checked at the C ABI).
  const int64_t heads = a.B * a.H;
  const int64_t grid = heads * (DV / DVS);
  unsigned xs = 0;
  for (int x = device_info().xcds; x > 1 && xs < 7; x >>= 1) ++xs;
  const unsigned heads_x = (unsigned)heads | (xs << 28);
  if (a.kda)
    a.beta_given ? launch_kernel<E, DK, DV, DVS, true, true>(a, heads_x, grid, stream)
                 : launch_kernel<E, DK, DV, DVS, true, false>(a, heads_x, grid, stream);
  else
    a.beta_given ? launch_kernel<E, DK, DV, DVS, false, true>(a, heads_x, grid, stream)
                 : launch_kernel<E, DK, DV, DVS, false, false>(a, heads_x, grid, stream);
  return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const DecodeArgs& a, hipStream_t stream) {
  // Many heads: wide slices (more rows per lane, fewer waves per byte). Few heads: 16-column
  // slices, so that the grid still puts a couple of waves on every CU. Measured crossovers
  // (d = 128, bf16): 64 columns win from 1024 heads on, 32 at 512.
  if (a.B * a.H >= 1024) return launch<E, DK, DV, 64>(a, stream);
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
