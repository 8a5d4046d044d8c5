// Chunkwise forward, part 2 of 2: the inter-chunk state scan and the outputs.
//
// Sources: "Deep Dive into KDA", section 3 (inter-chunk state update
// S[n+1] = Diag(gamma) S[n] + (Gamma o K[n])^T (U[n] - W[n] S[n]) and intra-chunk output
// O[n] = (Gamma o Q[n]) S[n] + Tril(...)(U[n] - W[n] S[n]); only the d_k x d_v state passes
// between chunks), specialised to the scalar gate of "Kaczmarz Linear Attention", Abstract.
//
// State S is stored [d_k][d_v] (S = M^T of the pages). For chunk n with entering state S and
// the prep kernel's T, P and per-token factors (chunk_common.h):
//   X = K S;  R[r,:] = eta_r rs_r (v_r - e^{G_r} X[r,:])
//   D = T R;  D'[r,:] = rs_r D[r,:]              (D' is the page's U - W S)
//   O = diag(e^G) Q S + P D'
//   S <- e^{G_C} S + K^T diag(e^{G_C - G}) D'
// W S is never formed: W S = T diag(beta e^G) K S, folded into the single product T R.
//
// One workgroup (4 waves) owns one d_v slice (DVS columns) of one head and walks its chunks in
// order. The slice of S stays in fp32 MFMA accumulators for the whole sequence; a bf16 copy
// of S^T in LDS is the operand of the next chunk's K S and Q S. While chunk n is computed, the
// inputs of chunk n+1 (K, Q, V slice, T, P, factors) are already in flight into registers.
// The slices of one head get workgroup ids congruent mod 8, so they run on one XCD and share
// its L2 for K, Q, T and P.
#include "chunk_common.h"

namespace kla {

hipError_t launch_chunk_prep(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);

namespace {

template <typename E, int DK, int DVS>
struct ScanSmem {
  static constexpr bool BF = is_bf16<E>();
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int LDK = DK + PAD;      // Ks, Qs, STs rows
  static constexpr int LDC = kChunk + PAD;  // KTs, Tb, Pb, RTs, DTs, DTs2 rows
  static constexpr int LDO = DVS + PAD;     // Vs, Os rows
  alignas(16) E Ks[kChunk][LDK];
  alignas(16) E Qs[kChunk][LDK];
  alignas(16) E KTs[BF ? DK : 1][LDC];      // K^T (bf16 path; fp32 reads Ks transposed)
  alignas(16) E Vs[kChunk][LDO];
  alignas(16) E Tb[kChunk][LDC];
  alignas(16) E Pb[kChunk][LDC];
  alignas(16) float sc[kScRows][kChunk];
  alignas(16) E STs[DVS][LDK];
  alignas(16) E RTs[DVS][LDC];
  alignas(16) E DTs[DVS][LDC];
  alignas(16) E DTs2[DVS][LDC];
  alignas(16) E Os[kChunk][LDO];
};

template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(ChunkParams p) {
  constexpr bool BF = is_bf16<E>();
  constexpr int NS = DV / DVS;     // d_v slices per head
  constexpr int TJ = DVS / 16;     // 16-column tiles per slice
  constexpr int RT = DK / 64;      // 16-row tiles of S per wave
  constexpr int VN = Vec16<E>::N;  // elements per 16-byte vector
  typedef typename Vec16<E>::type V16;
  typedef ScanSmem<E, DK, DVS> Sm;
  constexpr int LDK = Sm::LDK, LDC = Sm::LDC;
  __shared__ Sm sm;

  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int64_t head = (int64_t)(local / NS) * kXcds + xcd;
  const int slice = local % NS;
  if (head >= p.heads) return;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, nchunks = p.nchunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int j0 = slice * DVS;
  const E* __restrict__ gq = static_cast<const E*>(p.q);
  const E* __restrict__ gk = static_cast<const E*>(p.k);
  const E* __restrict__ gv = static_cast<const E*>(p.v);
  E* __restrict__ go = static_cast<E*>(p.o);
  auto row_index = [&](int64_t t) { return (bb * T + t) * p.H + hh; };
  const Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * nchunks);
  const int64_t chunk0 = head * nchunks;

  // ---- register prefetch of one chunk's inputs ----
  constexpr int KVPR = DK / VN;                                   // vectors per K/Q row
  constexpr int NKV = kChunk * KVPR / kThreads;                   // K (and Q) vectors per thread
  constexpr int VVPR = DVS / VN;                                  // vectors per V-slice row
  constexpr int NVV = (kChunk * VVPR + kThreads - 1) / kThreads;  // V vectors per thread (ceil)
  constexpr int TVPR = kChunk / VN;                               // vectors per T/P row
  constexpr int NTV = kChunk * TVPR / kThreads;                   // T (and P) vectors per thread
  static_assert(NKV * kThreads == kChunk * KVPR && NTV * kThreads == kChunk * TVPR, "tiling");
  V16 pk[NKV], pq[NKV], pv[NVV], pt[NTV], pp[NTV];
  float psc;

  auto prefetch = [&](int64_t c) {
    const int64_t t0 = c * kChunk;
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
      const int idx = tid + i * kThreads, r = idx / KVPR, vc = idx % KVPR;
      if (t0 + r < T) {
        pk[i] = *reinterpret_cast<const V16*>(gk + row_index(t0 + r) * DK + vc * VN);
        pq[i] = *reinterpret_cast<const V16*>(gq + row_index(t0 + r) * DK + vc * VN);
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) pk[i][e] = pq[i][e] = from_f32<E>(0.f);
      }
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int idx = tid + i * kThreads, r = idx / VVPR, vc = idx % VVPR;
      if (idx < kChunk * VVPR && t0 + r < T) {
        pv[i] = *reinterpret_cast<const V16*>(gv + row_index(t0 + r) * DV + j0 + vc * VN);
      } else {
#pragma unroll
        for (int e = 0; e < VN; ++e) pv[i][e] = from_f32<E>(0.f);
      }
    }
    const E* gT = ws.T + (chunk0 + c) * kChunk * kChunk;
    const E* gP = ws.P + (chunk0 + c) * kChunk * kChunk;
#pragma unroll
    for (int i = 0; i < NTV; ++i) {
      const int idx = tid + i * kThreads;
      pt[i] = *reinterpret_cast<const V16*>(gT + idx * VN);
      pp[i] = *reinterpret_cast<const V16*>(gP + idx * VN);
    }
    psc = ws.SC[(chunk0 + c) * kScRows * kChunk + tid];
  };

  auto commit = [&]() {
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
      const int idx = tid + i * kThreads, r = idx / KVPR, vc = idx % KVPR;
      *reinterpret_cast<V16*>(&sm.Ks[r][vc * VN]) = pk[i];
      *reinterpret_cast<V16*>(&sm.Qs[r][vc * VN]) = pq[i];
      if constexpr (BF) {
#pragma unroll
        for (int e = 0; e < VN; ++e) sm.KTs[vc * VN + e][r] = pk[i][e];
      }
    }
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
      const int idx = tid + i * kThreads, r = idx / VVPR, vc = idx % VVPR;
      if (idx < kChunk * VVPR) *reinterpret_cast<V16*>(&sm.Vs[r][vc * VN]) = pv[i];
    }
#pragma unroll
    for (int i = 0; i < NTV; ++i) {
      const int idx = tid + i * kThreads, r = idx / TVPR, vc = idx % TVPR;
      *reinterpret_cast<V16*>(&sm.Tb[r][vc * VN]) = pt[i];
      *reinterpret_cast<V16*>(&sm.Pb[r][vc * VN]) = pp[i];
    }
    (&sm.sc[0][0])[tid] = psc;
  };

  auto store_output = [&](int64_t t0) {
    for (int i = tid; i < kChunk * VVPR; i += kThreads) {
      const int r = i / VVPR, vc = i % VVPR;
      if (t0 + r < T)
        *reinterpret_cast<V16*>(go + row_index(t0 + r) * DV + j0 + vc * VN) =
            *reinterpret_cast<const V16*>(&sm.Os[r][vc * VN]);
    }
  };

  // ---- state slice -> accumulators; wave w owns S rows [w DK/4, (w+1) DK/4) ----
  f32x4 accS[RT][TJ];
  {
    const float* Sin = p.state_in ? p.state_in + head * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        const int row0 = wave * (DK / 4) + rt * 16 + 4 * lq;
        const int col = j0 + tj * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[rt][tj][e] = Sin ? Sin[(int64_t)(row0 + e) * DV + col] : 0.f;
        store4<E>(&sm.STs[tj * 16 + lr][row0], accS[rt][tj][0], accS[rt][tj][1], accS[rt][tj][2],
                  accS[rt][tj][3]);
      }
  }

  if (nchunks > 0) prefetch(0);
  // Row block w of T and P is zero past column 16 (w + 1).
  const int kend = BF ? (wave < 2 ? 32 : 64) : 16 * (wave + 1);

  for (int64_t c = 0; c < nchunks; ++c) {
    if (c > 0) store_output((c - 1) * kChunk);
    commit();
    __syncthreads();
    if (c + 1 < nchunks) prefetch(c + 1);

    // ---- X = K S -> R^T;  Y = e^G (Q S) stays in registers ----
    f32x4 accY[TJ];
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) {
      f32x4 accX = {0.f, 0.f, 0.f, 0.f};
      accY[tj] = accX;
      const int r = lane & 15, kq = lane >> 4;
      if constexpr (BF) {
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32) {
          const bf16x8 s = *reinterpret_cast<const bf16x8*>(&sm.STs[tj * 16 + r][k0 + 8 * kq]);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.Ks[wave * 16 + r][k0 + 8 * kq]);
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(&sm.Qs[wave * 16 + r][k0 + 8 * kq]);
          accX = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, s, accX, 0, 0, 0);
          accY[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, s, accY[tj], 0, 0, 0);
        }
      } else {
        mma16<E>(accX, &sm.Ks[wave * 16][0], LDK, &sm.STs[tj * 16][0], LDK, DK, lane);
        mma16<E>(accY[tj], &sm.Qs[wave * 16][0], LDK, &sm.STs[tj * 16][0], LDK, DK, lane);
      }
      const int jj = tj * 16 + lr;
      float R[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wave * 16 + 4 * lq + e;
        const float eg = sm.sc[kScEG][row];
        R[e] = sm.sc[kScCoefR][row] * (to_f32(sm.Vs[row][jj]) - eg * accX[e]);
        accY[tj][e] *= eg;
      }
      store4<E>(&sm.RTs[jj][wave * 16 + 4 * lq], R[0], R[1], R[2], R[3]);
    }
    __syncthreads();

    // ---- D = T R;  D' = rs D (-> DTs);  diag(e^{G_C - G}) D' (-> DTs2) ----
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma16<E>(acc, &sm.Tb[wave * 16][0], LDC, &sm.RTs[tj * 16][0], LDC, kend, lane);
      const int jj = tj * 16 + lr;
      float d1[4], d2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wave * 16 + 4 * lq + e;
        d1[e] = sm.sc[kScRs][row] * acc[e];
        d2[e] = sm.sc[kScD2][row] * acc[e];
      }
      store4<E>(&sm.DTs[jj][wave * 16 + 4 * lq], d1[0], d1[1], d1[2], d1[3]);
      store4<E>(&sm.DTs2[jj][wave * 16 + 4 * lq], d2[0], d2[1], d2[2], d2[3]);
    }
    __syncthreads();

    // ---- O = Y + P D';  S <- e^{G_C} S + K^T DTs2 ----
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) {
      mma16<E>(accY[tj], &sm.Pb[wave * 16][0], LDC, &sm.DTs[tj * 16][0], LDC, kend, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Os[wave * 16 + 4 * lq + e][tj * 16 + lr] = from_f32<E>(accY[tj][e]);
    }
    const float eGC = sm.sc[kScEG][kChunk - 1];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        const int row0 = wave * (DK / 4) + rt * 16;
        accS[rt][tj] *= eGC;
        if constexpr (BF)
          mma16<E>(accS[rt][tj], &sm.KTs[row0][0], LDC, &sm.DTs2[tj * 16][0], LDC, kChunk, lane);
        else
          mma16_f32s(accS[rt][tj], reinterpret_cast<const float*>(&sm.Ks[0][row0]), 1, LDK,
                     reinterpret_cast<const float*>(&sm.DTs2[tj * 16][0]), 1, LDC, 0, kChunk, lane);
        store4<E>(&sm.STs[tj * 16 + lr][row0 + 4 * lq], accS[rt][tj][0], accS[rt][tj][1], accS[rt][tj][2],
                  accS[rt][tj][3]);
      }
    __syncthreads();
  }
  if (nchunks > 0) store_output((nchunks - 1) * kChunk);

  if (p.state_out) {
    float* Sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        const int row0 = wave * (DK / 4) + rt * 16 + 4 * lq;
        const int col = j0 + tj * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sout[(int64_t)(row0 + e) * DV + col] = accS[rt][tj][e];
      }
  }
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const ChunkParams& p, hipStream_t stream) {
  constexpr int DVS = is_bf16<E>() ? 32 : 16;
  constexpr int NS = DV / DVS;
  const int64_t heads8 = (p.heads + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((chunk_scan_kernel<E, DK, DV, DVS>), dim3((unsigned)(heads8 * NS)), dim3(kThreads), 0, stream,
                     p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_scan(const ChunkParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_dk_dv<E, 128, 128>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_dk_dv<E, 64, 64>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_dk_dv<E, 128, 64>(p, stream);
  return launch_dk_dv<E, 64, 128>(p, stream);
}

}  // namespace

size_t chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t, int64_t, bool bf16_io) {
  const int64_t n = B * H * ((T + kChunk - 1) / kChunk);
  return bf16_io ? Workspace<bf16>::bytes(n) : Workspace<float>::bytes(n);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream) {
  ChunkParams p{a.q, a.k, a.v, a.eta, a.log_alpha, a.state_in, a.state_out, a.o, a.workspace,
                a.B * a.H, a.H, a.T, (a.T + kChunk - 1) / kChunk, a.eps};
  if (p.nchunks > 0) {
    const hipError_t e = launch_chunk_prep(p, a.d_k, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  return a.bf16 ? launch_scan<bf16>(p, a.d_k, a.d_v, stream) : launch_scan<float>(p, a.d_k, a.d_v, stream);
}

}  // namespace kla
