// Chunkwise backward, the reverse state scan: the gradient of the state, carried from the
// last chunk to the first.
//
// Sources: "Deep Dive into KDA", section 3 (the chunkwise forward that this differentiates:
// S[n+1] = gamma S[n] + (Gamma o K[n])^T (U[n] - W[n] S[n]) and
// O[n] = (Gamma o Q[n]) S[n] + Tril(...)(U[n] - W[n] S[n])); "Kaczmarz Linear Attention",
// Abstract (the chunkwise form serves prefill and training).
//
// Per chunk, in the balanced factors of the forward (chunk_prep.hip): Delta = diag(rs) T R with
// R = diag(eta rs)(V - diag(e^G) K S), O = diag(e^G) Q S + P Delta and
// S' = e^{G_C} S + K^T diag(e^{G_C - G}) Delta. Given dS' (the gradient of the state leaving the
// chunk) and dO:
//   dDelta = P^T dO + diag(e^{G_C - G}) K dS'
//   Zb     = T^T (rs o dDelta)                      (= diag(rs) dR with dR = (I + A)^-T dDelta)
//   dS     = e^{G_C} dS' + Q^T diag(e^G) dO - K^T diag(eta rs e^G) Zb
// With the forward's factors that is X = K dS', R' = (rs e^{G_C - G}) o X + rs o (P^T dO),
// Zb = T^T R'. Every chunk's dS' and Zb go to the backward workspace for the chunk-parallel
// gradient kernel; dS after the first chunk is dL/dS_0.
//
// With the per-channel decay (KDA, "Deep Dive into KDA", sections 2.3 and 3) the decays sit in
// the operands that the KDA prep wrote (K1 = K o e^G, Q1 = Q o e^G, K2 = K o e^{G_C - G}, gamma =
// e^{G_C} per d_k row; its factor rows carry e^G = 1 and rs e^{G_C - G} = rs):
//   X = K2 dS',  R' = rs o X + rs o (P^T dO),  Zb = T^T R',
//   dS = Diag(gamma) dS' + Q1^T dO - K1^T diag(eta rs) Zb.
//
// The structure mirrors the forward scan (chunk_scan.hip): a workgroup of W waves owns DVS
// columns of one head's dS for every d_k row, each wave 16 NT of them, in fp32 MFMA
// accumulators; the chain dS -> X -> R' -> Zb -> dS never leaves the wave. Operands (K, Q, T, P,
// dO and the per-token factors) arrive by direct-to-LDS loads a chunk ahead, chunks in
// descending order. P^T, T^T, K^T and Q^T are read with the transposing LDS read.
#include "tile_ops.h"

namespace kla {

hipError_t launch_chunk_prep(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);
hipError_t launch_chunk_prep_kda(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);
hipError_t launch_scan_recompute(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream);
hipError_t launch_scan_recompute_kda(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io,
                                     hipStream_t stream);
hipError_t launch_chunk_grad(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream);
hipError_t launch_chunk_grad_kda(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, bool bf16_io,
                                 hipStream_t stream);

namespace {

// Producer waves (bf16): as in the forward scan, two more waves per workgroup on the idle SIMDs
// issue all direct-to-LDS loads.
template <typename E, int DK, int DV, int W, int NT, bool KDA>
constexpr int rscan_producers() {
  return (is_bf16<E>() && scan_ring<E, DK, W * 16 * NT, KDA>() == 2) ? 2 : 0;
}

// KDA: the buffer's K holds K2 (the rows of X = K2 dS'), its K2 slot K1 (read transposed for the
// state update), Q holds Q1, and gam the chunk's gamma.
template <typename E, int DK, int DV, int W, int NT, bool KDA>
__global__ __launch_bounds__((W + 2) * kWave) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_rscan_kernel(
    ChunkBwdParams p) {
  constexpr int GK = Grp<E>::K;
  typedef typename Grp<E>::V GV;
  constexpr int NC = 16 * NT;        // state columns per wave
  constexpr int DVS = W * NC;        // state columns per workgroup
  constexpr int NS = DV / DVS;       // workgroups per head
  constexpr int RTK = DK / 16;       // 16-row tiles of dS
  constexpr int NGD = DK / GK;       // groups over d_k
  constexpr int NGT = kChunk / GK;   // groups over the chunk's tokens
  constexpr int PER = 16 / sizeof(E);
  typedef ScanBuf<E, DK, DVS, KDA> Buf;
  constexpr int NB = scan_ring<E, DK, DVS, KDA>();
  constexpr int DIST = NB > 1 ? NB - 1 : 1;
  static_assert(NB <= 2, "ring of at most two buffers");
  static_assert(DV % DVS == 0, "shape");
  __shared__ Buf buf0;
  __shared__ typename std::conditional<(NB >= 2), Buf, int>::type buf1;

  const int bid = blockIdx.x;
  const int xcd = bid % p.xcds;
  const int local = bid / p.xcds;
  const int64_t head = (int64_t)(local / NS) * p.xcds + xcd;
  const int slice = local % NS;
  if (head >= p.heads) return;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, nchunks = p.nchunks, H = p.H;
  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int c16 = lane & 15, g = lane >> 4;
  const int j0 = slice * DVS;
  const int cw = wave * NC;
  const int ct0 = (j0 + cw) / 16;  // first global 16-column tile of this wave

  const int64_t brow = bb * T * H;
  const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E);
  const rsrc_t rdo = make_rsrc(static_cast<const E*>(p.dout) + brow * DV, (uint32_t)(T * vrow));
  const Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * nchunks);
  const BwdSpace<E> bw = BwdSpace<E>::at(p.ws, p.bwd_off, p.heads * nchunks, DK, DV);
  const int64_t chunk0 = head * nchunks;
  // K and Q rows: the k/q tensors (token stride H DK), or with KDA the decayed operands of the
  // KDA workspace (chunk-contiguous rows of DK): K2 in K's place, Q1 in Q's, K1 for the update.
  const KdaSpace<E> kw = KdaSpace<E>::at(p.ws, p.heads * nchunks, DK);
  const uint32_t krow = KDA ? DK * sizeof(E) : xrow;
  const uint32_t kspan = KDA ? (uint32_t)(nchunks * kChunk * DK * sizeof(E)) : (uint32_t)(T * xrow);
  const rsrc_t rk = make_rsrc(KDA ? (const void*)(kw.K2 + chunk0 * kChunk * DK)
                                  : (const void*)(static_cast<const E*>(p.k) + brow * DK), kspan);
  const rsrc_t rq = make_rsrc(KDA ? (const void*)(kw.Q1 + chunk0 * kChunk * DK)
                                  : (const void*)(static_cast<const E*>(p.q) + brow * DK), kspan);
  const rsrc_t rk1 = make_rsrc(kw.K1 + chunk0 * kChunk * DK, KDA ? kspan : 0u);
  const rsrc_t rgam = make_rsrc(kw.gamma + chunk0 * DK, KDA ? (uint32_t)(nchunks * DK * 4) : 0u);
  constexpr uint32_t kMatBytes = kChunk * kChunk * sizeof(E), kScBytes = kScRows * kChunk * sizeof(float);
  constexpr uint32_t kSBytes = DK * DV * sizeof(E), kDBytes = kChunk * DV * sizeof(E);
  const rsrc_t rt = make_rsrc(ws.T + chunk0 * kChunk * kChunk, (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rp = make_rsrc(ws.P + chunk0 * kChunk * kChunk, (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rsc = make_rsrc(ws.SC + chunk0 * kScRows * kChunk, (uint32_t)(nchunks * kScBytes));
  const rsrc_t rds = make_rsrc(bw.dSn + chunk0 * DK * DV, (uint32_t)(nchunks * kSBytes));
  const rsrc_t rzb = make_rsrc(bw.Zb + chunk0 * kChunk * DV, (uint32_t)(nchunks * kDBytes));
  const uint32_t hcol_x = KDA ? 0u : hh * DK * sizeof(E), hcol_v = (hh * DV + j0) * sizeof(E);

  // ---- DMA of one chunk's operands (as in the forward scan; dO takes V's place), by the
  //      producer waves if there are any, else by the scan waves ----
  constexpr int NP = rscan_producers<E, DK, DV, W, NT, KDA>();
  constexpr int WD = NP ? NP : W;
  const int dw = NP ? wave - W : wave;
  constexpr int CK = DK / PER, CT = kChunk / PER, CV = DVS / PER;
  constexpr int BK = kChunk * CK / 64, BT = kChunk * CT / 64, BV = kChunk * CV / 64;
  static_assert(BK % WD == 0 && BT % WD == 0 && BV % WD == 0, "block split");
  constexpr int NBK = BK / WD, NBT = BT / WD, NBV = BV / WD;
  uint32_t offk[NBK], offt[NBT], offv[NBV];
#pragma unroll
  for (int i = 0; i < NBK; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CK;
    offk[i] = r * krow + hcol_x + 16 * swz<E, CK>(r, ph % CK);
  }
#pragma unroll
  for (int i = 0; i < NBT; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CT;
    offt[i] = (r * CT + swz<E, CT>(r, ph % CT)) * 16;
  }
#pragma unroll
  for (int i = 0; i < NBV; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CV;
    offv[i] = r * vrow + hcol_v + 16 * swz<E, CV>(r, ph % CV);
  }
  constexpr int NDMA = (2 + KDA) * NBK + 2 * NBT + NBV + 1 + KDA;
  constexpr int NST = (RTK + 4) * NT;  // stores per chunk and wave: dS' tiles, Zb tiles
  auto fetch = [&](Buf& B, int64_t c) {
    c = c < 0 ? 0 : c;  // a chunk before the first is clamped (loaded again, never read)
    const uint32_t t0 = (uint32_t)(c * kChunk);
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = dw + WD * i;
      dma16(rk, B.K + blk * 64 * PER, t0 * krow + offk[i]);
      dma16(rq, B.Q + blk * 64 * PER, t0 * krow + offk[i]);
      if constexpr (KDA) dma16(rk1, B.K2 + blk * 64 * PER, t0 * krow + offk[i]);
    }
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int blk = dw + WD * i;
      dma16(rt, B.T + blk * 64 * PER, (uint32_t)c * kMatBytes + offt[i]);
      dma16(rp, B.P + blk * 64 * PER, (uint32_t)c * kMatBytes + offt[i]);
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int blk = dw + WD * i;
      dma16(rdo, B.V + blk * 64 * PER, t0 * vrow + offv[i]);
    }
    dma16(rsc, B.sc, (uint32_t)c * kScBytes + 16 * lane);
    if constexpr (KDA) dma16(rgam, B.gam, (uint32_t)c * DK * 4 + 16 * lane);
  };

  if constexpr (NP > 0) {
    static_assert(NB == 2, "producers serve a two-buffer ring");
    if (wave >= W) {  // producer: every chunk's loads, one chunk ahead, descending, one barrier per chunk
      if (nchunks > 0) fetch(buf0, nchunks - 1);
      for (int64_t c = nchunks - 1; c >= 0; c -= 2) {
        wait_vmem<0>();
        __syncthreads();  // chunk c is in buf0; every wave is done with chunk c + 1 (buf1)
        fetch(buf1, c - 1);
        if (c - 1 >= 0) {
          wait_vmem<0>();
          __syncthreads();
          fetch(buf0, c - 2);
        }
      }
      wait_vmem<0>();  // no load into LDS outlives the workgroup
      return;
    }
  }

  // ---- this wave's columns of dS: lane (g, c) = dS[16 rt + 4g + e][j0 + cw + 16 ct + c] ----
  f32x4 dS[RTK][NT];
  if (p.dstate_out) {
    const float* src = p.dstate_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dS[r][ct][e] = src[(int64_t)(16 * r + 4 * g + e) * DV + j0 + cw + 16 * ct + c16];
  } else {
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) dS[r][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // One chunk (chunks in descending order; `done` chunks were processed before this one). Issue
  // order per wave: the loads of the first chunk, then per chunk the loads of the next one and
  // this chunk's stores, so at most (DIST - 1) chunks of loads and DIST chunks of stores are
  // younger than this chunk's loads when it starts.
  auto step = [&](Buf& B, Buf& Bn, int64_t c, int64_t done) __attribute__((always_inline)) {
    if constexpr (!is_bf16<E>() && DK == 128) {
      // fp32 with d_k = 128: per-lane index arithmetic is redone every chunk (the lane id passed
      // through an empty asm) rather than hoisted out of the chunk loop: hoisted, it stayed live
      // across the loop and spilled 136-169 VGPRs; now none (B2 H8 T4096 backward 2.06 ->
      // 1.54 ms). At d_k = 64 (15 spilled) the redone arithmetic cost more than it saved.
      asm volatile("" : "+v"(tid));
      lane = tid & 63;
      c16 = lane & 15;
      g = lane >> 4;
    }
    if constexpr (NP > 0) {
      // the producers waited for chunk c's loads before this barrier
    } else if constexpr (NB == 1) {
      wait_vmem<0>();
    } else {
      if (done < DIST)
        wait_vmem<(DIST - 1) * NDMA>();
      else
        wait_vmem<(DIST - 1) * NDMA + DIST * NST>();
    }
    __syncthreads();
    if constexpr (NB > 1 && NP == 0) fetch(Bn, c - DIST);

    // dS' of this chunk (the gradient of the state leaving it)
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        store4_rsrc<E>(rds, (uint32_t)c * kSBytes + tile_off(r, ct0 + ct, DV / 16, lane) * sizeof(E), dS[r][ct]);

    // ---- X = K dS' (token rows x this wave's columns) ----
    GV sb[NGD][NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 tiles[RTK];
#pragma unroll
      for (int r = 0; r < RTK; ++r) tiles[r] = dS[r][ct];
#pragma unroll
      for (int s = 0; s < NGD; ++s) sb[s][ct] = acc_grp<E>(tiles, s);
    }
    f32x4 X[4][NT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) X[r][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NGD; ++s) {
        const GV ak = row_grp<E, DK>(B.K, 16 * r + c16, s, g);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) X[r][ct] = mma<E>(ak, sb[s][ct], X[r][ct]);
      }
    }

    // ---- dO as B operands over the tokens (group s: this wave's columns), and e^G o dO ----
    GV bo[NT][NGT], boe[NT][NGT];
#pragma unroll
    for (int s = 0; s < NGT; ++s) {
      f32x4 eg0, eg1;
      if constexpr (is_bf16<E>()) {
        eg0 = *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + 32 * s + 4 * g]);
        eg1 = *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + 32 * s + 16 + 4 * g]);
      } else {
        eg0 = *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + 16 * s + 4 * g]);
        eg1 = eg0;
      }
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        bo[ct][s] = kt_grp<E, DVS>(B.V, cw / 16 + ct, s, g, c16);
        if constexpr (is_bf16<E>()) {
          bf16x8 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = from_f32<bf16>(eg0[e] * to_f32(bo[ct][s][e]));
            x[4 + e] = from_f32<bf16>(eg1[e] * to_f32(bo[ct][s][4 + e]));
          }
          boe[ct][s] = x;
        } else {
          boe[ct][s] = eg0 * bo[ct][s];
        }
      }
    }

    // ---- R' = (rs e^{G_C - G}) o X + rs o (P^T dO), in place of X (P^T upper triangular) ----
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 y[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) y[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * (s + 1) > 16 * r) {
          const GV ap = kt_grp<E, kChunk>(B.P, r, s, g, c16);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) y[ct] = mma<E>(ap, bo[ct][s], y[ct]);
        }
      }
      const f32x4 rs = *reinterpret_cast<const f32x4*>(&B.sc[kScRs * kChunk + 16 * r + 4 * g]);
      const f32x4 dd = *reinterpret_cast<const f32x4*>(&B.sc[kScD2 * kChunk + 16 * r + 4 * g]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) X[r][ct] = dd * X[r][ct] + rs * y[ct];
    }

    // ---- Zb = T^T R' (T^T upper triangular: row tile r needs tokens from 16 r on) ----
    GV rb[NT][NGT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const f32x4 tiles[4] = {X[0][ct], X[1][ct], X[2][ct], X[3][ct]};
#pragma unroll
      for (int s = 0; s < NGT; ++s) rb[ct][s] = acc_grp<E>(tiles, s);
    }
    f32x4 Z2[NT][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 z[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) z[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * (s + 1) > 16 * r) {
          const GV at_ = kt_grp<E, kChunk>(B.T, r, s, g, c16);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) z[ct] = mma<E>(at_, rb[ct][s], z[ct]);
        }
      }
      const f32x4 cr = *reinterpret_cast<const f32x4*>(&B.sc[kScCoefR * kChunk + 16 * r + 4 * g]);
      const f32x4 eg = *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + 16 * r + 4 * g]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        store4_rsrc<E>(rzb, (uint32_t)c * kDBytes + tile_off(r, ct0 + ct, DV / 16, lane) * sizeof(E), z[ct]);
        Z2[ct][r] = -(cr * eg) * z[ct];
      }
    }
    GV b2[NT][NGT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int s = 0; s < NGT; ++s) b2[ct][s] = acc_grp<E>(Z2[ct], s);

    // ---- dS <- e^{G_C} dS' + Q^T (e^G o dO) - K^T (eta rs e^G o Zb)
    //      (KDA: Diag(gamma) dS' + Q1^T dO - K1^T (eta rs o Zb)) ----
    const float eGC = B.sc[kScEG * kChunk + kChunk - 1];
#pragma unroll
    for (int r = 0; r < RTK; ++r) {
      if constexpr (KDA) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&B.gam[16 * r + 4 * g]);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) dS[r][ct] *= gm;
      } else {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) dS[r][ct] *= eGC;
      }
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        const GV aq = kt_grp<E, DK>(B.Q, r, s, g, c16);
        const GV ak = kt_grp<E, DK>(KDA ? B.K2 : B.K, r, s, g, c16);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          dS[r][ct] = mma<E>(aq, boe[ct][s], dS[r][ct]);
          dS[r][ct] = mma<E>(ak, b2[ct][s], dS[r][ct]);
        }
      }
    }
    if constexpr (NB == 1) {
      __syncthreads();
      if (c > 0) fetch(B, c - 1);
    }
  };

  if (NP == 0 && nchunks > 0) fetch(buf0, nchunks - 1);
  if constexpr (NB == 2) {
    int64_t done = 0;
    for (int64_t c = nchunks - 1; c >= 0; c -= 2, done += 2) {
      step(buf0, buf1, c, done);
      if (c - 1 >= 0) step(buf1, buf0, c - 1, done + 1);
    }
  } else {
    for (int64_t c = nchunks - 1; c >= 0; --c) step(buf0, buf0, c, 0);
  }

  wait_vmem<0>();  // no load into LDS outlives the workgroup
  if (p.dstate_in) {
    float* dst = p.dstate_in + head * (int64_t)DK * DV;
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(int64_t)(16 * r + 4 * g + e) * DV + j0 + cw + 16 * ct + c16] = dS[r][ct][e];
  }
}

template <typename E, int DK, int DV, int W, int NT, bool KDA>
hipError_t launch_wnt(const ChunkBwdParams& p, hipStream_t stream) {
  constexpr int NS = DV / (W * 16 * NT);
  const int64_t heads8 = (p.heads + p.xcds - 1) / p.xcds * p.xcds;
  constexpr int NP = rscan_producers<E, DK, DV, W, NT, KDA>();
  hipLaunchKernelGGL((chunk_rscan_kernel<E, DK, DV, W, NT, KDA>), dim3((unsigned)(heads8 * NS)),
                     dim3((W + NP) * kWave), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int DK, int DV, bool KDA>
hipError_t launch_dk_dv(const ChunkBwdParams& p, hipStream_t stream) {
  // The forward scan's split: bf16 two waves of 16 columns, fp32 four.
  if constexpr (is_bf16<E>())
    return launch_wnt<E, DK, DV, 2, 1, KDA>(p, stream);
  else
    return launch_wnt<E, DK, DV, 4, 1, KDA>(p, stream);
}

template <typename E, bool KDA>
hipError_t launch_e(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_dk_dv<E, 128, 128, KDA>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_dk_dv<E, 64, 64, KDA>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_dk_dv<E, 128, 64, KDA>(p, stream);
  return launch_dk_dv<E, 64, 128, KDA>(p, stream);
}

}  // namespace

hipError_t launch_reverse_scan(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, bool bf16_io, bool kda,
                               hipStream_t stream) {
  if (kda) return bf16_io ? launch_e<bf16, true>(p, d_k, d_v, stream) : launch_e<float, true>(p, d_k, d_v, stream);
  return bf16_io ? launch_e<bf16, false>(p, d_k, d_v, stream) : launch_e<float, false>(p, d_k, d_v, stream);
}

size_t chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16_io) {
  const int64_t n = B * H * ((T + kChunk - 1) / kChunk);
  return bf16_io ? Workspace<bf16>::bytes(n) + BwdSpace<bf16>::bytes(n, (int)d_k, (int)d_v)
                 : Workspace<float>::bytes(n) + BwdSpace<float>::bytes(n, (int)d_k, (int)d_v);
}

size_t chunk_kda_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16_io) {
  const int64_t n = B * H * ((T + kChunk - 1) / kChunk);
  return bf16_io ? KdaSpace<bf16>::bytes(n, (int)d_k) + BwdSpace<bf16>::bytes(n, (int)d_k, (int)d_v)
                 : KdaSpace<float>::bytes(n, (int)d_k) + BwdSpace<float>::bytes(n, (int)d_k, (int)d_v);
}

// The backward: the forward's per-chunk factors again (prep), the forward scan once more to
// record every chunk's entering state and Delta, the reverse scan for the state gradients, then
// the chunk-parallel gradients. With beta given the factors are taken unbalanced (rs = 1).
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, hipStream_t stream) {
  const int64_t nchunks = (a.T + kChunk - 1) / kChunk, n = a.B * a.H * nchunks;
  ChunkBwdParams bp{a.q,  a.k,    a.v,         a.eta,      a.log_alpha, a.state_in, a.dout, a.dstate_out,
                    a.dq, a.dk,   a.dv,        a.deta,     a.dlog_alpha, a.dstate_in, a.workspace,
                    a.B * a.H, a.H, a.T, nchunks, a.eps, a.beta_given};
  bp.xcds = device_info().xcds;
  bp.bwd_off = a.kda ? (a.bf16 ? KdaSpace<bf16>::bytes(n, (int)a.d_k) : KdaSpace<float>::bytes(n, (int)a.d_k))
                     : (a.bf16 ? Workspace<bf16>::bytes(n) : Workspace<float>::bytes(n));
  if (nchunks > 0 && !a.saved) {  // (saved: the training forward left all of this in the workspace)
    ChunkParams fp{a.q,   a.k,       a.v, a.eta,    a.log_alpha, a.state_in, nullptr, nullptr, a.workspace,
                   a.B * a.H, a.H, a.T, nchunks, a.eps, a.beta_given, a.beta_given};
    fp.xcds = bp.xcds;
    fp.bwd_off = bp.bwd_off;
    hipError_t e = a.kda ? launch_chunk_prep_kda(fp, a.d_k, a.bf16, stream) : launch_chunk_prep(fp, a.d_k, a.bf16, stream);
    if (e == hipSuccess)
      e = a.kda ? launch_scan_recompute_kda(fp, a.d_k, a.d_v, a.bf16, stream)
                : launch_scan_recompute(fp, a.d_k, a.d_v, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_reverse_scan(bp, a.d_k, a.d_v, a.bf16, a.kda, stream);
  if (e == hipSuccess && nchunks > 0)
    e = a.kda ? launch_chunk_grad_kda(bp, a.d_k, a.d_v, a.bf16, stream) : launch_chunk_grad(bp, a.d_k, a.d_v, a.bf16, stream);
  return e;
}

}  // namespace kla
