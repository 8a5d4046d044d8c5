// Chunkwise backward, the chunk-parallel gradients for fp32 inputs with a 128-wide head (d_k or
// d_v = 128), whose operands do not fit the LDS of the gradient kernel in chunk_bwd_grad.hip.
// The same quantities, formulas and partial-sum order as that kernel (its header gives them);
// the products over d_v (Zb Delta^T, dO Delta^T, Zb V^T, Zb S^T, dO S^T, Delta dS'^T) are
// accumulated over NH parts of d_v (two when d_v = 128), each part's operands in LDS in turn,
// and the C x C weights Ma, Mp then take the parts' space.
//
// Sources: "Deep Dive into KDA", section 3 (the chunkwise forward differentiated here);
// "Kaczmarz Linear Attention", Abstract (beta = eta / (||k||^2 + eps)).
#include "tile_ops.h"

namespace kla {

namespace {

constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = kSplitWaves * kWave;

// Parts of d_v: a part's rows of dO, S^T / dS'^T, Delta^T and Zb^T must fit beside K and Q.
template <int DK, int DV>
constexpr int split_parts() {
  return DV == 128 ? 2 : 1;
}

template <int DK, int DV>
struct SplitSmem {
  static constexpr int DVH = DV / split_parts<DK, DV>();
  alignas(16) float Ks[kChunk * DK];
  alignas(16) float Qs[kChunk * DK];
  struct Half {
    alignas(16) float dOs[kChunk * DVH];
    alignas(16) float St[DVH * DK];  // V_h ([64][DVH]) while the C x C tiles are formed, then S_h^T, then dS'_h^T
    alignas(16) float Dt[DVH * kChunk];
    alignas(16) float Zt[DVH * kChunk];
  };
  struct Weights {
    alignas(16) float Ma[kChunk * kChunk];
    alignas(16) float Mp[kChunk * kChunk];
  };
  union {
    Half h;
    Weights w;
  } u;
  float G[kChunk], eG[kChunk], cr[kChunk], rs[kChunk], zv[kChunk], kcoef[kChunk];
  float rowA[10][16], rowE[10][16], colE[10][16];
  float kzs[DK / 16][kChunk], qos[DK / 16][kChunk], kds[DK / 16][kChunk], sds[kSplitWaves];
};

template <int DK, int DV>
__global__ __launch_bounds__(kSplitThreads) void chunk_grad_split_kernel(ChunkBwdParams p) {
  typedef float E;
  constexpr int NH = split_parts<DK, DV>(), DVH = DV / NH;
  constexpr int NGD = DK / 16, NGH = DVH / 16, NGT = kChunk / 16;  // fp32 groups of 16
  constexpr int NW = kSplitWaves, NT_ = kSplitThreads;
  constexpr int NIT = DK / 16;
  constexpr int TPW = NIT * 4 / NW;
  static_assert(TPW * NW == NIT * 4 && 4 % TPW == 0, "tile split: a wave's tiles share one d_k tile");
  typedef SplitSmem<DK, DV> Sm;
  __shared__ Sm sm;

  int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int c16 = lane & 15, g = lane >> 4;
  const int itw = wave * TPW / 4;  // the d_k tile of this wave's output tiles
  const int64_t total = p.heads * p.nchunks, chunk_id = blockIdx.x;
  if (chunk_id >= total) return;
  const int64_t head = chunk_id / p.nchunks, c = chunk_id % p.nchunks;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, H = p.H, t0 = c * kChunk;
  const Workspace<E> ws = Workspace<E>::at(p.ws, total);
  const BwdSpace<E> bw = BwdSpace<E>::at(p.ws, p.bwd_off, total, DK, DV);

  const int64_t brow = bb * T * H;
  const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E);
  const rsrc_t rk = make_rsrc(static_cast<const E*>(p.k) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rq = make_rsrc(static_cast<const E*>(p.q) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rv = make_rsrc(static_cast<const E*>(p.v) + brow * DV, (uint32_t)(T * vrow));
  const rsrc_t rdo = make_rsrc(static_cast<const E*>(p.dout) + brow * DV, (uint32_t)(T * vrow));
  const rsrc_t rdq = make_rsrc(static_cast<E*>(p.dq) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rdk = make_rsrc(static_cast<E*>(p.dk) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rdv = make_rsrc(static_cast<E*>(p.dv) + brow * DV, (uint32_t)(T * vrow));
  const uint32_t hcol_x = hh * DK * sizeof(E), hcol_v = hh * DV * sizeof(E);
  const uint32_t x0 = (uint32_t)t0 * xrow, v0 = (uint32_t)t0 * vrow;

  // rows of a [64][NCOL] block (columns col0 .. col0 + NCOL of the source rows) straight into LDS
  auto dma_rows = [&](rsrc_t r, E* dst, uint32_t rowb, uint32_t hcol, uint32_t base, auto ncol_tag)
      __attribute__((always_inline)) {
    constexpr int NCOL = decltype(ncol_tag)::value;
    constexpr int CPR = NCOL / 4, NBLK = kChunk * CPR / 64;
    static_assert(NBLK % NW == 0, "block split");
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) {
      const int blk = wave + NW * i, ph = 64 * blk + lane, row = ph / CPR;
      dma16(r, dst + blk * 64 * 4, base + row * rowb + hcol + 16 * swz<E, CPR>(row, ph % CPR));
    }
  };
  dma_rows(rk, sm.Ks, xrow, hcol_x, x0, std::integral_constant<int, DK>());
  dma_rows(rq, sm.Qs, xrow, hcol_x, x0, std::integral_constant<int, DK>());
  if (wave == 0) {
    const bool valid = t0 + lane < T;
    const float la = valid && p.log_alpha ? p.log_alpha[(bb * T + t0 + lane) * H + hh] : 0.f;
    const float* sc = ws.SC + chunk_id * kScRows * kChunk;
    sm.G[lane] = wave_inclusive_scan(la);
    sm.cr[lane] = sc[kScCoefR * kChunk + lane];
    sm.eG[lane] = sc[kScEG * kChunk + lane];
    sm.rs[lane] = sc[kScRs * kChunk + lane];
  }

  // Tile-ordered workspace blocks (16 x 16 tiles, NCT = DV / 16 per row of tiles; lane piece l of
  // tile (rt, ct) = rows 4 (l / 16) .. + 3 of column l % 16), half h: the tiles with ct in the half.
  constexpr int NCT = DV / 16, NCTH = NCT / NH;
  // [64 x DV] (Delta, Zb): transposed into [DVH][64]
  auto put_t64 = [&](const E* src, E* dst, int h) __attribute__((always_inline)) {
    constexpr int NPC = 4 * NCTH * 64 / NT_;  // lane pieces per thread
    static_assert(NPC * NT_ == 4 * NCTH * 64, "piece split");
    f32x4 x[NPC];
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int pi = tid + NT_ * i, ti = pi >> 6, l = pi & 63, rt = ti / NCTH, ct = h * NCTH + ti % NCTH;
      x[i] = *reinterpret_cast<const f32x4*>(src + tile_off(rt, ct, NCT, l));
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int pi = tid + NT_ * i, ti = pi >> 6, l = pi & 63, rt = ti / NCTH, ctl = ti % NCTH;
      *reinterpret_cast<f32x4*>(dst + at<E, kChunk>(16 * ctl + (l & 15), 16 * rt + 4 * (l >> 4))) = x[i];
    }
  };
  // [DK x DV] (S, dS'): transposed into [DVH][DK]
  auto put_state = [&](const E* src, int h) __attribute__((always_inline)) {
    constexpr int NPS = NGD * NCTH * 64 / NT_;
    static_assert(NPS * NT_ == NGD * NCTH * 64, "piece split");
    f32x4 x[NPS];
#pragma unroll
    for (int i = 0; i < NPS; ++i) {
      const int pi = tid + NT_ * i, ti = pi >> 6, l = pi & 63, rt = ti / NCTH, ct = h * NCTH + ti % NCTH;
      x[i] = *reinterpret_cast<const f32x4*>(src + tile_off(rt, ct, NCT, l));
    }
#pragma unroll
    for (int i = 0; i < NPS; ++i) {
      const int pi = tid + NT_ * i, ti = pi >> 6, l = pi & 63, rt = ti / NCTH, ctl = ti % NCTH;
      *reinterpret_cast<f32x4*>(sm.u.h.St + at<E, DK>(16 * ctl + (l & 15), 16 * rt + 4 * (l >> 4))) = x[i];
    }
  };
  // <S, dS'> of this thread's pieces of half h (same positions in both)
  auto sds_part = [&](int h) __attribute__((always_inline)) {
    constexpr int NPS = NGD * NCTH * 64 / NT_;
    const E* gS = bw.Sn + chunk_id * DK * DV;
    const E* gdS = bw.dSn + chunk_id * DK * DV;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NPS; ++i) {
      const int pi = tid + NT_ * i, ti = pi >> 6, l = pi & 63, rt = ti / NCTH, ct = h * NCTH + ti % NCTH;
      const f32x4 a = *reinterpret_cast<const f32x4*>(gS + tile_off(rt, ct, NCT, l));
      const f32x4 b = *reinterpret_cast<const f32x4*>(gdS + tile_off(rt, ct, NCT, l));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += a[e] * b[e];
    }
    return acc;
  };

  // per-wave C x C tiles: tile k keeps its slot k in the partial sums
  constexpr int MAXC = (10 + NW - 1) / NW;
  f32x4 aF[MAXC], aP[MAXC], aZV[MAXC];
#pragma unroll
  for (int q = 0; q < MAXC; ++q) aF[q] = aP[q] = aZV[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
  f32x4 accZS[TPW], accOS[TPW], accDS[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) accZS[t] = accOS[t] = accDS[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float sdsum = 0.f;

  // ---- the products over d_v, one part at a time (a loop, not unrolled: unrolled, the
  //      compiler hoisted the second part's loads and spilled) ----
#pragma unroll 1
  for (int h = 0; h < NH; ++h) {
    // Per-lane index arithmetic is redone in every part rather than hoisted out of the loop and
    // kept live across it (hoisted, it spilled).
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    c16 = lane & 15;
    g = lane >> 4;
    const uint32_t hc = hcol_v + h * DVH * sizeof(E);
    dma_rows(rdo, sm.u.h.dOs, vrow, hc, v0, std::integral_constant<int, DVH>());
    dma_rows(rv, sm.u.h.St, vrow, hc, v0, std::integral_constant<int, DVH>());
    put_t64(bw.Dl + chunk_id * kChunk * DV, sm.u.h.Dt, h);
    put_t64(bw.Zb + chunk_id * kChunk * DV, sm.u.h.Zt, h);
    wait_vmem<0>();
    __syncthreads();
    // C x C tiles: Zb Delta^T, dO Delta^T; on diagonal tiles Zb V^T
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      const int j = wave + NW * q;
      if (j < 10) {
        int ti, tj;
        tri_tile(j, ti, tj);
#pragma unroll
        for (int s = 0; s < NGH; ++s) {
          const f32x4 bd = kt_grp<E, kChunk>(sm.u.h.Dt, tj, s, g, c16);
          const f32x4 az = kt_grp<E, kChunk>(sm.u.h.Zt, ti, s, g, c16);
          aF[q] = mma<E>(az, bd, aF[q]);
          aP[q] = mma<E>(row_grp<E, DVH>(sm.u.h.dOs, 16 * ti + c16, s, g), bd, aP[q]);
          if (ti == tj) aZV[q] = mma<E>(az, row_grp<E, DVH>(sm.u.h.St, 16 * tj + c16, s, g), aZV[q]);
        }
      }
    }
    // dv = diag(eta rs) Zb for this half's columns
    {
      constexpr int NJT = DVH / 16;
#pragma unroll
      for (int t = 0; t < (4 * NJT + NW - 1) / NW; ++t) {
        const int q = wave + NW * t;
        if (q < 4 * NJT) {
          const int rt = q % 4, jt = q / 4, r = 16 * rt + c16;
          const f32x4 z = col4<E, kChunk>(sm.u.h.Zt, 16 * jt, 16 * rt, g, c16);
          store4_rsrc<E>(rdv, v0 + r * vrow + hc + (16 * jt + 4 * g) * sizeof(E), sm.cr[r] * z);
        }
      }
    }
    __syncthreads();
    put_state(bw.Sn + chunk_id * DK * DV, h);
    sdsum += sds_part(h);
    __syncthreads();
    // All of a wave's output tiles share one d_k tile (itw): its S^T fragments serve them all.
#pragma unroll
    for (int s = 0; s < NGH; ++s) {
      const f32x4 as = kt_grp<E, DK>(sm.u.h.St, itw, s, g, c16);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = (wave * TPW + t) % 4;
        accZS[t] = mma<E>(as, kt_grp<E, kChunk>(sm.u.h.Zt, rt, s, g, c16), accZS[t]);
        accOS[t] = mma<E>(as, row_grp<E, DVH>(sm.u.h.dOs, 16 * rt + c16, s, g), accOS[t]);
      }
    }
    __syncthreads();
    put_state(bw.dSn + chunk_id * DK * DV, h);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NGH; ++s) {
      const f32x4 ad = kt_grp<E, DK>(sm.u.h.St, itw, s, g, c16);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int rt = (wave * TPW + t) % 4;
        accDS[t] = mma<E>(ad, kt_grp<E, kChunk>(sm.u.h.Dt, rt, s, g, c16), accDS[t]);
      }
    }
    __syncthreads();  // the half's operands are read no more
  }
  {
    const float a = wave_sum(sdsum);
    if (lane == 0) sm.sds[wave] = a;
  }

  asm volatile("" : "+v"(tid));
  lane = tid & 63;
  c16 = lane & 15;
  g = lane >> 4;
  // ---- the C x C weights: K K^T and Q K^T, then Ma, Mp and the decay sums ----
#pragma unroll
  for (int q = 0; q < MAXC; ++q) {
    const int j = wave + NW * q;
    if (j < 10) {
      int ti, tj;
      tri_tile(j, ti, tj);
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
#pragma unroll
      for (int s = 0; s < NGD; ++s) {
        const f32x4 bk = row_grp<E, DK>(sm.Ks, 16 * tj + c16, s, g);
        kk = mma<E>(row_grp<E, DK>(sm.Ks, 16 * ti + c16, s, g), bk, kk);
        qk = mma<E>(row_grp<E, DK>(sm.Qs, 16 * ti + c16, s, g), bk, qk);
      }
      if (ti == tj && (c16 >> 2) == g) {
        const int e = c16 & 3;
        sm.zv[16 * ti + c16] = e == 0 ? aZV[q][0] : e == 1 ? aZV[q][1] : e == 2 ? aZV[q][2] : aZV[q][3];
      }
      const int s = 16 * tj + c16;
      const float Gs = sm.G[s];
      float csum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + 4 * g + e;
        const float L = s <= r ? __expf(sm.G[r] - Gs) : 0.f;
        const float na = s < r ? -aF[q][e] * L : 0.f;
        const float naKK = na * kk[e];
        const float crr = sm.cr[r];
        const float mp = aP[q][e] * L;
        const float ee = crr * naKK + mp * qk[e];
        sm.u.w.Ma[at<E, kChunk>(r, s)] = crr * na;
        sm.u.w.Mp[at<E, kChunk>(r, s)] = mp;
        csum += ee;
        const float ra = row16_sum(naKK), re = row16_sum(ee);
        if (c16 == 0) {
          sm.rowA[j][4 * g + e] = ra;
          sm.rowE[j][4 * g + e] = re;
        }
      }
      csum = col4_sum(csum);
      if (g == 0) sm.colE[j][c16] = csum;
    }
  }
  // the upper tiles are zero (fp32 groups are 16 tokens wide: only tiles at or below the diagonal
  // are read, and those are all written above)
  __syncthreads();

  // ---- d_k x C products with the weights, transposed outputs; token-row dot products ----
  f32x4 accK[TPW], accQ[TPW], kv[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = (wave * TPW + t) / 4, rt = (wave * TPW + t) % 4;
    f32x4 k_ = {0.f, 0.f, 0.f, 0.f}, q_ = k_;
#pragma unroll
    for (int s = 0; s < NGT; ++s) {
      const f32x4 ak = kt_grp<E, DK>(sm.Ks, it, s, g, c16);
      if (16 * s < 16 * (rt + 1)) {  // Ma[r][s], Mp[r][s] vanish for s > r
        k_ = mma<E>(ak, row_grp<E, kChunk>(sm.u.w.Ma, 16 * rt + c16, s, g), k_);
        q_ = mma<E>(ak, row_grp<E, kChunk>(sm.u.w.Mp, 16 * rt + c16, s, g), q_);
      }
      if (16 * (s + 1) > 16 * rt) {  // Ma[r][s], Mp[r][s] over r >= s
        const f32x4 aq = kt_grp<E, DK>(sm.Qs, it, s, g, c16);
        k_ = mma<E>(ak, kt_grp<E, kChunk>(sm.u.w.Ma, rt, s, g, c16), k_);
        k_ = mma<E>(aq, kt_grp<E, kChunk>(sm.u.w.Mp, rt, s, g, c16), k_);
      }
    }
    accK[t] = k_;
    accQ[t] = q_;
    const int r = 16 * rt + c16, i0 = 16 * it + 4 * g;
    const f32x4 kx = *reinterpret_cast<const f32x4*>(&sm.Ks[at<E, DK>(r, i0)]);
    const f32x4 qx = *reinterpret_cast<const f32x4*>(&sm.Qs[at<E, DK>(r, i0)]);
    kv[t] = kx;
    float a = 0.f, b = 0.f, d = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += kx[e] * accZS[t][e];
      b += qx[e] * accOS[t][e];
      d += kx[e] * accDS[t][e];
    }
    a = col4_sum(a);
    b = col4_sum(b);
    d = col4_sum(d);
    if (g == 0) {
      sm.kzs[it][r] = a;
      sm.qos[it][r] = b;
      sm.kds[it][r] = d;
    }
  }
  __syncthreads();

  // ---- per token: deta, dG, and dlog(alpha) as the within-chunk suffix sum of dG ----
  if (wave == 0) {
    const int r = lane, ti = r >> 4, rr = r & 15;
    float rowA = 0.f, rowE = 0.f, colE = 0.f;
    for (int tj = 0; tj <= ti; ++tj) {
      rowA += sm.rowA[ti * (ti + 1) / 2 + tj][rr];
      rowE += sm.rowE[ti * (ti + 1) / 2 + tj][rr];
    }
    for (int tk = ti; tk < 4; ++tk) colE += sm.colE[tk * (tk + 1) / 2 + ti][rr];
    float kzs = 0.f, qos = 0.f, kds = 0.f, sds = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      kzs += sm.kzs[it][r];
      qos += sm.qos[it][r];
      kds += sm.kds[it][r];
    }
#pragma unroll
    for (int w = 0; w < NW; ++w) sds += sm.sds[w];
    const float crr = sm.cr[r], eGr = sm.eG[r], GC = sm.G[kChunk - 1];
    const float de = sm.rs[r] * (sm.zv[r] - eGr * kzs + rowA);
    const float wsr = __expf(GC - sm.G[r]) * kds;
    float dG = -crr * eGr * kzs + rowE - colE + eGr * qos - wsr;
    const float wtot = wave_sum(wsr);
    if (r == kChunk - 1) dG += __expf(GC) * sds + wtot;
    const float incl = wave_inclusive_scan(dG);
    const float tot = __shfl(incl, kChunk - 1, kWave);
    const int64_t row = (bb * T + t0 + r) * H + hh;
    if (t0 + r < T) {
      p.deta[row] = de;
      if (p.dlog_alpha) p.dlog_alpha[row] = tot - incl + dG;
    }
    sm.kcoef[r] = p.beta_given ? 0.f : -2.f * crr * sm.rs[r] * de;
  }
  __syncthreads();

  // ---- dk, dq: four consecutive d_k entries of one token per lane ----
  const float GC = sm.G[kChunk - 1];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = (wave * TPW + t) / 4, rt = (wave * TPW + t) % 4;
    const int r = 16 * rt + c16, i0 = 16 * it + 4 * g;
    const float crr = sm.cr[r], eGr = sm.eG[r], dec = __expf(GC - sm.G[r]), kc = sm.kcoef[r];
    const f32x4 dk = accK[t] - (crr * eGr) * accZS[t] + dec * accDS[t] + kc * kv[t];
    const f32x4 dq = accQ[t] + eGr * accOS[t];
    const uint32_t off = x0 + r * xrow + hcol_x + i0 * sizeof(E);
    store4_rsrc<E>(rdk, off, dk);
    store4_rsrc<E>(rdq, off, dq);
  }
}

template <int DK, int DV>
hipError_t launch_dk_dv(const ChunkBwdParams& p, hipStream_t stream) {
  static_assert(sizeof(SplitSmem<DK, DV>) <= 160 * 1024, "LDS");
  hipLaunchKernelGGL((chunk_grad_split_kernel<DK, DV>), dim3((unsigned)(p.heads * p.nchunks)), dim3(kSplitThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

// fp32 gradients with d_k or d_v = 128 (the other fp32 shape and every bf16 one take
// chunk_grad_kernel).
hipError_t launch_chunk_grad_split(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_dk_dv<128, 128>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_dk_dv<128, 64>(p, stream);
  if (d_k == 64 && d_v == 128) return launch_dk_dv<64, 128>(p, stream);
  return hipErrorInvalidConfiguration;
}

}  // namespace kla
