// Chunkwise backward with the per-channel decay (KDA), the chunk-parallel part: dq, dk, dv,
// deta (or dbeta) and dlog a of every chunk, one workgroup per chunk of one head, from the
// states and gradients that the two scans left in the workspace.
//
// Sources: "Deep Dive into KDA", section 2.3 (the per-channel decay Diag(a_t)) and section 3
// (the chunkwise form differentiated here: the decays inside the Q and K operands, ratios of
// decays taken in the log domain and never divided by); "Kaczmarz Linear Attention", Abstract
// (the step size beta = eta / (||k||^2 + eps)).
//
// The forward, per chunk, in the balanced factors of the KDA prep (chunk_prep.hip; cr = eta rs,
// rs, G [64][d_k] the chunk-local prefix of log a, E_rs = e^{G_r - G_s} per channel for s <= r):
//   A_rs = k_r.(k_s o E_rs) (s < r),  P_rs = q_r.(k_s o E_rs) (s <= r),  T = (I + diag(cr) A diag(rs))^-1
//   Delta = diag(rs) T diag(cr) (V - (e^G o K) S),   O = (e^G o Q) S + P Delta,
//   S' = Diag(e^{G_C}) S + (e^{G_C - G} o K)^T Delta.
// With S, dS' (gradient of the state leaving the chunk), Delta and Zb from the workspace:
//   Na = -(Zb Delta^T) (s < r),  Mp = dO Delta^T (s <= r)
//   R1_r = sum_s Na_rs k_s o E_rs,       R2_r = sum_s Mp_rs k_s o E_rs          (row side)
//   C1_s = sum_r cr_r Na_rs k_r o E_rs,  C2_s = sum_r Mp_rs q_r o E_rs          (column side)
//   ZS = Zb S^T,  OS = dO S^T,  DS = Delta dS'^T
//   deta_r = rs_r (Zb_r.v_r - (e^{G_r} o k_r).ZS_r + k_r.R1_r)
//   dk = cr R1 + C1 + C2 - cr e^G o ZS + e^{G_C - G} o DS - 2 cr rs deta k      (last term: KLA only)
//   dq = R2 + e^G o OS,   dv = cr Zb
//   dG = cr k o R1 - k o C1 + q o R2 - k o C2 - cr e^G o k o ZS + e^G o q o OS - e^{G_C - G} o k o DS
//   dG_C = sum_r e^{G_C - G_r} o k_r o DS_r + e^{G_C} o rowsum(S o dS')
//   dlog a_j = sum_{r >= j} dG_r + dG_C      (G is the chunk-local prefix; G_C = G_63)
// With beta given (factors cr = beta, rs = 1) deta is d(beta) and dk has no step-size term.
//
// The decayed products R1, R2, C1, C2. Off the diagonal 16 x 16 token blocks the ratio factors
// through a reference token between the two blocks, both factors at most 1: on the row side the
// first token b of the output's block (E_rs = e^{G_r - G_b} e^{G_b - G_s}, s < b <= r), on the
// column side its last token c (E_rs = e^{G_r - G_c} e^{G_c - G_s}, s <= c < r). The factor of the
// contracted token scales the MFMA operand, the factor of the output token the accumulator. On
// the diagonal blocks each lane walks its own token's block with a running product of the
// per-token decays a = e^{log a}. No exponent is ever positive.
//
// Outputs are computed transposed (d_k rows x tokens, as in the scalar gate's gradient kernel):
// lane (g, c) of output tile (it, rt) holds channels 16 it + 4 g .. + 3 of token 16 rt + c.
#include "tile_ops.h"

namespace kla {

namespace {

constexpr int kKgWaves = 8;
constexpr int kKgThreads = kKgWaves * kWave;
// Largest decay span (in log units, per channel) over a 16-token diagonal block that the MFMA
// path takes: its operands are then at most e^32 (about 8e13) times the keys or queries, far
// inside bf16's range for any key whose squares fit fp32 (which the recurrence itself needs).
constexpr float kSpan = 32.f;

template <typename E, int DK, int DV>
struct KgSmem {
  static constexpr int LDG = DK + 4;  // fp32 rows of G and a, padded
  alignas(16) E Ks[kChunk * DK];
  alignas(16) E Qs[kChunk * DK];
  alignas(16) E Zt[DV * kChunk];      // Zb^T
  alignas(16) E Na[kChunk * kChunk];  // -(Zb Delta^T), strictly lower
  alignas(16) E Mp[kChunk * kChunk];  // dO Delta^T, lower
  struct OpsA {                       // the products over d_v
    alignas(16) E dOs[kChunk * DV];
    alignas(16) E St[DV * DK];        // V ([64][DV]) while the C x C tiles are formed, then S^T, then dS'^T
    alignas(16) E Dt[DV * kChunk];    // Delta^T
  };
  struct OpsB {                       // the decayed products and the per-channel sums
    alignas(16) float G[kChunk * LDG];  // log a, then its chunk-local prefix
    alignas(16) float A[kChunk * LDG];  // a = e^{log a}, then dG
  };
  union {
    OpsA a;
    OpsB b;
  } u;
  float cr[kChunk], rs[kChunk], zv[kChunk], kcoef[kChunk];
  // Partial sums, one slot per producer, added in a fixed order (bitwise reproducible):
  float kr[DK / 16][kChunk], kzs[DK / 16][kChunk];  // per d_k tile: k.R1 and (e^G o k).ZS per token
  float gcp[4][DK];                                 // per token tile: sum_r e^{G_C - G_r} k_r DS_r
  float sds[DK];                                    // rowsum(S o dS')
  float gpart[kKgThreads / DK][DK];                 // per token run: prefix / suffix totals
  float dgc[DK];                                    // dG_C
};

template <typename E, int DK, int DV>
constexpr bool kda_grad_fits() {
  return sizeof(KgSmem<E, DK, DV>) <= 160 * 1024;
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kKgThreads) void chunk_grad_kda_kernel(ChunkBwdParams p) {
  constexpr bool BF = is_bf16<E>();
  constexpr int GK = Grp<E>::K;
  typedef typename Grp<E>::V GV;
  constexpr int PER = 16 / sizeof(E);
  typedef typename Vec16<E>::type V16;
  constexpr int NGV = DV / GK, NGT = kChunk / GK;
  constexpr int NW = kKgWaves, NT_ = kKgThreads;
  constexpr int NIT = DK / 16;       // 16-channel tiles of d_k
  constexpr int TPW = NIT * 4 / NW;  // (d_k tile, token tile) output tiles per wave
  static_assert(TPW * NW == NIT * 4, "tile split");
  typedef KgSmem<E, DK, DV> Sm;
  constexpr int LDG = Sm::LDG;
  __shared__ Sm sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t total = p.heads * p.nchunks, chunk_id = blockIdx.x;
  if (chunk_id >= total) return;
  const int64_t head = chunk_id / p.nchunks, c = chunk_id % p.nchunks;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, H = p.H, t0 = c * kChunk;
  const Workspace<E> ws = Workspace<E>::at(p.ws, total);
  const BwdSpace<E> bw = BwdSpace<E>::at(p.ws, p.bwd_off, total, DK, DV);

  // Rows of this batch entry through buffer resources: rows past T read as zero (log a = 0 there,
  // so the padded rows decay by 1 and G_C is the last real token's prefix), stores past T are
  // dropped.
  const int64_t brow = bb * T * H;
  const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E), lrow = H * DK * 4;
  const rsrc_t rk = make_rsrc(static_cast<const E*>(p.k) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rq = make_rsrc(static_cast<const E*>(p.q) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rv = make_rsrc(static_cast<const E*>(p.v) + brow * DV, (uint32_t)(T * vrow));
  const rsrc_t rdo = make_rsrc(static_cast<const E*>(p.dout) + brow * DV, (uint32_t)(T * vrow));
  const rsrc_t rla = make_rsrc(p.log_alpha + brow * DK, (uint32_t)(T * lrow));
  const rsrc_t rdq = make_rsrc(static_cast<E*>(p.dq) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rdk = make_rsrc(static_cast<E*>(p.dk) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rdv = make_rsrc(static_cast<E*>(p.dv) + brow * DV, (uint32_t)(T * vrow));
  const uint32_t hcol_x = hh * DK * sizeof(E), hcol_v = hh * DV * sizeof(E);
  const uint32_t x0 = (uint32_t)t0 * xrow, v0 = (uint32_t)t0 * vrow;

  // ---- loads: K, Q, dO, V rows straight into LDS; Delta, Zb, S, dS' and log a into registers ----
  auto dma_rows = [&](rsrc_t r, E* dst, uint32_t base, uint32_t rowb, uint32_t hcol, auto ncol_tag)
      __attribute__((always_inline)) {
    constexpr int NCOL = decltype(ncol_tag)::value;
    constexpr int CPR = NCOL / PER, NBLK = kChunk * CPR / 64;
    static_assert(NBLK % NW == 0, "block split");
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) {
      const int blk = wave + NW * i, ph = 64 * blk + lane, row = ph / CPR;
      dma16(r, dst + blk * 64 * PER, base + row * rowb + hcol + 16 * swz<E, CPR>(row, ph % CPR));
    }
  };
  // Issue order: what the C x C tiles need first (dO and V into LDS, Delta and Zb into
  // registers), then K and Q (first read by the decayed products), S, dS' and log a, so that the
  // first phase waits only for its own operands.
  dma_rows(rdo, sm.u.a.dOs, v0, vrow, hcol_v, std::integral_constant<int, DV>());
  dma_rows(rv, sm.u.a.St, v0, vrow, hcol_v, std::integral_constant<int, DV>());

  constexpr int NSR = DK * DV / PER / NT_;      // 16-byte pieces of S (and of dS') per thread
  constexpr int NCH = kChunk * DV / PER / NT_;  // 16-byte pieces of Delta (and of Zb) per thread
  constexpr int NL = kChunk * DK / 4 / NT_;     // 16-byte pieces of log a per thread
  constexpr int NKQ = kChunk * DK / PER / 64 / NW;  // direct-to-LDS loads per wave for K (and Q)
  static_assert(NSR >= 1 && NCH >= 1 && NL >= 1, "piece split");
  V16 sreg[NSR], dsreg[NSR], dlreg[NCH], zbreg[NCH];
  i32x4 lx[NL];
  {
    const E* gD = bw.Dl + chunk_id * kChunk * DV;
    const E* gZ = bw.Zb + chunk_id * kChunk * DV;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      dlreg[i] = *reinterpret_cast<const V16*>(gD + (tid + NT_ * i) * PER);
      zbreg[i] = *reinterpret_cast<const V16*>(gZ + (tid + NT_ * i) * PER);
    }
  }
  dma_rows(rk, sm.Ks, x0, xrow, hcol_x, std::integral_constant<int, DK>());
  dma_rows(rq, sm.Qs, x0, xrow, hcol_x, std::integral_constant<int, DK>());
  {
    const E* gS = bw.Sn + chunk_id * DK * DV;
    const E* gdS = bw.dSn + chunk_id * DK * DV;
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
      sreg[i] = *reinterpret_cast<const V16*>(gS + (tid + NT_ * i) * PER);
      dsreg[i] = *reinterpret_cast<const V16*>(gdS + (tid + NT_ * i) * PER);
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int i = tid + NT_ * j, r = i / (DK / 4), c4 = (i % (DK / 4)) * 4;
      lx[j] = __builtin_amdgcn_raw_buffer_load_b128(rla, (uint32_t)((t0 + r) * lrow + (hh * DK + c4) * 4), 0, 0);
    }
  }
  constexpr int NLATER = 2 * NKQ + 2 * NSR + NL;  // loads issued after Zb, per wave (wave 0 adds two)
  if (wave == 0) {
    const float* sc = ws.SC + chunk_id * kScRows * kChunk;
    sm.cr[lane] = sc[kScCoefR * kChunk + lane];
    sm.rs[lane] = sc[kScRs * kChunk + lane];
  }

  // tile-ordered [64 x DV] blocks, transposed into LDS: lane piece (rows 4g..4g+3 of column c of
  // tile (rt, ct)) -> row 16 ct + c, columns 16 rt + 4g .. + 3
  auto put_t64 = [&](const V16* x, E* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = tid + NT_ * i;
#pragma unroll
      for (int h = 0; h < PER / 4; ++h) {
        const int pi = ci * (PER / 4) + h, ti = pi >> 6, l = pi & 63;
        const int rt = ti / (DV / 16), ct = ti % (DV / 16);
        E* d = dst + at<E, kChunk>(16 * ct + (l & 15), 16 * rt + 4 * (l >> 4));
        if constexpr (BF)
          *reinterpret_cast<bf16x4*>(d) = half4(x[i], h);
        else
          *reinterpret_cast<f32x4*>(d) = x[i];
      }
    }
  };
  // tile-ordered [DK x DV] registers -> transposed LDS [DV][DK]
  auto put_state = [&](const V16* regs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
      const int ci = tid + NT_ * i;
#pragma unroll
      for (int h = 0; h < PER / 4; ++h) {
        const int pi = ci * (PER / 4) + h, ti = pi >> 6, l = pi & 63;
        const int rt = ti / (DV / 16), ct = ti % (DV / 16);
        E* d = sm.u.a.St + at<E, DK>(16 * ct + (l & 15), 16 * rt + 4 * (l >> 4));
        if constexpr (BF)
          *reinterpret_cast<bf16x4*>(d) = half4(regs[i], h);
        else
          *reinterpret_cast<f32x4*>(d) = regs[i];
      }
    }
  };
  put_t64(dlreg, sm.u.a.Dt);
  put_t64(zbreg, sm.Zt);
  // Upper off-diagonal tiles of Na and Mp that the 32-token contraction groups reach, (0, 1) and
  // (2, 3), are zero (fp32 groups are 16 tokens wide and reach none).
  {
    constexpr int CPT = 16 / PER;  // 16-byte chunks per tile row
    if (tid < 2 * 2 * 16 * CPT) {
      const int cc = tid % CPT, rr = (tid / CPT) % 16, tile = (tid / (16 * CPT)) % 2, arr = tid / (32 * CPT);
      const int r = 16 * (2 * tile) + rr, col = 16 * (2 * tile + 1) + PER * cc;
      V16 z;
#pragma unroll
      for (int e = 0; e < PER; ++e) z[e] = from_f32<E>(0.f);
      *reinterpret_cast<V16*>((arr ? sm.Mp : sm.Na) + at<E, kChunk>(r, col)) = z;
    }
  }
  wait_vmem<NLATER>();  // dO and V are in LDS (the loads complete in issue order)
  __syncthreads();

  // ---- C x C tiles: Na = -(Zb Delta^T), Mp = dO Delta^T; on diagonal tiles Zb V^T for Zb_r.v_r ----
  for (int j = wave; j < 10; j += NW) {
    int ti, tj;
    tri_tile(j, ti, tj);
    f32x4 F = {0.f, 0.f, 0.f, 0.f}, dp = F, zvv = F;
#pragma unroll
    for (int s = 0; s < NGV; ++s) {
      const GV bd = kt_grp<E, kChunk>(sm.u.a.Dt, tj, s, g, c16);
      const GV az = kt_grp<E, kChunk>(sm.Zt, ti, s, g, c16);
      F = mma<E>(az, bd, F);
      dp = mma<E>(row_grp<E, DV>(sm.u.a.dOs, 16 * ti + c16, s, g), bd, dp);
      if (ti == tj) zvv = mma<E>(az, row_grp<E, DV>(sm.u.a.St, 16 * tj + c16, s, g), zvv);
    }
    if (ti == tj && (c16 >> 2) == g) {
      const int e = c16 & 3;
      sm.zv[16 * ti + c16] = e == 0 ? zvv[0] : e == 1 ? zvv[1] : e == 2 ? zvv[2] : zvv[3];
    }
    const int s = 16 * tj + c16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * g + e;
      sm.Na[at<E, kChunk>(r, s)] = from_f32<E>(s < r ? -F[e] : 0.f);
      sm.Mp[at<E, kChunk>(r, s)] = from_f32<E>(s <= r ? dp[e] : 0.f);
    }
  }
  __syncthreads();

  // ---- products with the state: ZS = Zb S^T, OS = dO S^T, then DS = Delta dS'^T. All of a
  //      wave's output tiles share one d_k tile itw, whose S rows the wave keeps as operands, so
  //      that the diagonal of S dS'^T over that tile (the per-channel sums of S o dS') is one
  //      more product ----
  const int itw = wave * TPW / 4;
  put_state(sreg);
  __syncthreads();
  f32x4 aZS[TPW], aOS[TPW], aDS[TPW];
  GV sop[NGV];
#pragma unroll
  for (int s = 0; s < NGV; ++s) sop[s] = kt_grp<E, DK>(sm.u.a.St, itw, s, g, c16);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int rt = (wave * TPW + t) % 4;
    f32x4 zs = {0.f, 0.f, 0.f, 0.f}, os = zs;
#pragma unroll
    for (int s = 0; s < NGV; ++s) {
      zs = mma<E>(sop[s], kt_grp<E, kChunk>(sm.Zt, rt, s, g, c16), zs);
      os = mma<E>(sop[s], row_grp<E, DV>(sm.u.a.dOs, 16 * rt + c16, s, g), os);
    }
    aZS[t] = zs;
    aOS[t] = os;
  }
  __syncthreads();
  put_state(dsreg);
  __syncthreads();
  {
    f32x4 dd = {0.f, 0.f, 0.f, 0.f};
    GV dop[NGV];
#pragma unroll
    for (int s = 0; s < NGV; ++s) {
      dop[s] = kt_grp<E, DK>(sm.u.a.St, itw, s, g, c16);
      dd = mma<E>(sop[s], dop[s], dd);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int rt = (wave * TPW + t) % 4;
      f32x4 ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NGV; ++s) ds = mma<E>(dop[s], kt_grp<E, kChunk>(sm.u.a.Dt, rt, s, g, c16), ds);
      aDS[t] = ds;
    }
    if ((c16 >> 2) == g && (wave * TPW) % 4 == 0) {  // one wave per d_k tile writes its diagonal
      const int e = c16 & 3;
      sm.sds[16 * itw + c16] = e == 0 ? dd[0] : e == 1 ? dd[1] : e == 2 ? dd[2] : dd[3];
    }
  }
  // dv = diag(cr) Zb: the transposing read of Zb^T gives four consecutive d_v entries of one
  // token per lane
  {
    constexpr int NJT = DV / 16;
#pragma unroll
    for (int t = 0; t < 4 * NJT / NW; ++t) {
      const int q = wave * (4 * NJT / NW) + t, rt = q % 4, jt = q / 4;
      const int r = 16 * rt + c16;
      const f32x4 z = col4<E, kChunk>(sm.Zt, 16 * jt, 16 * rt, g, c16);
      store4_rsrc<E>(rdv, v0 + r * vrow + hcol_v + (16 * jt + 4 * g) * sizeof(E), sm.cr[r] * z);
    }
  }
  wait_vmem<0>();   // K and Q are in LDS
  __syncthreads();  // the d_v products are done: their LDS now holds G and a

  // ---- G = chunk-local prefix of log a per channel (NPART threads per channel, each a run of
  //      tokens), and the per-token decays a = e^{log a} ----
  float* Gm = sm.u.b.G;
  float* Am = sm.u.b.A;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int i = tid + NT_ * j, r = i / (DK / 4), c4 = (i % (DK / 4)) * 4;
    *reinterpret_cast<i32x4*>(&Gm[r * LDG + c4]) = lx[j];
  }
  __syncthreads();
  constexpr int NPART = NT_ / DK, RUN = kChunk / NPART;
  const int pch = tid % DK, part = tid / DK;
  {
    float run[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      run[j] = Gm[(part * RUN + j) * LDG + pch];
      Am[(part * RUN + j) * LDG + pch] = __expf(run[j]);
    }
#pragma unroll
    for (int j = 1; j < RUN; ++j) run[j] += run[j - 1];
    sm.gpart[part][pch] = run[RUN - 1];
    __syncthreads();
    float off = 0.f;
    for (int q = 0; q < part; ++q) off += sm.gpart[q][pch];
#pragma unroll
    for (int j = 0; j < RUN; ++j) Gm[(part * RUN + j) * LDG + pch] = run[j] + off;
  }
  __syncthreads();

  // ---- per output tile (it, rt): the decayed products, then everything of the tile that does
  //      not wait for deta: dq (stored), dG and dk without its step-size term (kept) ----
  const f32x4 one4 = {1.f, 1.f, 1.f, 1.f};
  f32x4 dkp[TPW], dGr[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = itw, rt = (wave * TPW + t) % 4;
    const int chA = 16 * it + c16;    // channel of this lane's operand fragments
    const int ch0 = 16 * it + 4 * g;  // first of this lane's four output channels
    const int b = 16 * rt, ce = 16 * rt + 15;
    const int tok = b + c16;          // this lane's output token
    f32x4 r1 = {0.f, 0.f, 0.f, 0.f}, r2 = r1, cc = r1;  // R1, R2, C1 + C2
    // The diagonal block joins the MFMA products when the block's decay span (G_b - G_{b+15}, per
    // channel) is at most kSpan on every channel of the tile: its operand factors then lie in
    // [1, e^kSpan] (row side e^{G_b - G_s}, column side e^{G_r - G_ce}) and the output factors
    // stay at most 1. Otherwise (channels that forget faster) the block is walked exactly.
    const bool fast = __all(Gm[b * LDG + chA] - Gm[ce * LDG + chA] <= kSpan);
    const int rlim = fast ? ce : b - 1;   // row side: contracted tokens s <= rlim
    const int clim = fast ? b : ce + 1;   // column side: contracted tokens r >= clim

    // row side: reference token b
    {
      const float Gb = Gm[b * LDG + chA];
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * s <= rlim) {
          GV a = kt_grp<E, DK>(sm.Ks, it, s, g, c16), alo;
#pragma unroll
          for (int j = 0; j < (BF ? 8 : 4); ++j) {
            const int sk = grp_index<E>(s, g, j);
            const float f = sk <= rlim ? __expf(Gb - Gm[sk * LDG + chA]) : 0.f;
            const float x = to_f32(a[j]) * f;
            a[j] = from_f32<E>(x);
            if constexpr (BF) alo[j] = from_f32<E>(x - to_f32(a[j]));
          }
          const GV bn = row_grp<E, kChunk>(sm.Na, 16 * rt + c16, s, g);
          const GV bm = row_grp<E, kChunk>(sm.Mp, 16 * rt + c16, s, g);
          r1 = mma<E>(a, bn, r1);
          r2 = mma<E>(a, bm, r2);
          if constexpr (BF) {
            r1 = mma<E>(alo, bn, r1);
            r2 = mma<E>(alo, bm, r2);
          }
        }
      }
      const f32x4 Gr = *reinterpret_cast<const f32x4*>(&Gm[tok * LDG + ch0]);
      const f32x4 Gbv = *reinterpret_cast<const f32x4*>(&Gm[b * LDG + ch0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = __expf(Gr[e] - Gbv[e]);
        r1[e] *= f;
        r2[e] *= f;
      }
    }
    // row side, the diagonal block walked: token tok goes s = b + 15 .. b with
    // E = prod_{s < j <= tok} a_j (a loop with per-step LDS reads, partly unrolled: fully
    // unrolled, the reads of all steps were hoisted and spilled)
    if (!fast) {
      f32x4 Ew = {0.f, 0.f, 0.f, 0.f}, w1 = Ew, w2 = Ew;
#pragma unroll 4
      for (int j = 15; j >= 0; --j) {
        const int s = b + j;
        if (j < 15) Ew = Ew * *reinterpret_cast<const f32x4*>(&Am[(s + 1) * LDG + ch0]);
        Ew = j == c16 ? one4 : Ew;
        const f32x4 u = row4<E, DK>(sm.Ks, s, ch0) * Ew;
        w1 += to_f32(sm.Na[at<E, kChunk>(tok, s)]) * u;
        w2 += to_f32(sm.Mp[at<E, kChunk>(tok, s)]) * u;
      }
      r1 += w1;
      r2 += w2;
    }

    // column side: reference token ce
    {
      const float Gc = Gm[ce * LDG + chA];
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * (s + 1) > clim) {
          GV ak = kt_grp<E, DK>(sm.Ks, it, s, g, c16), aq = kt_grp<E, DK>(sm.Qs, it, s, g, c16), aklo, aqlo;
#pragma unroll
          for (int j = 0; j < (BF ? 8 : 4); ++j) {
            const int rk_ = grp_index<E>(s, g, j);
            const float f = rk_ >= clim ? __expf(Gm[rk_ * LDG + chA] - Gc) : 0.f;
            const float xk = to_f32(ak[j]) * (f * sm.cr[rk_]), xq = to_f32(aq[j]) * f;
            ak[j] = from_f32<E>(xk);
            aq[j] = from_f32<E>(xq);
            if constexpr (BF) {
              aklo[j] = from_f32<E>(xk - to_f32(ak[j]));
              aqlo[j] = from_f32<E>(xq - to_f32(aq[j]));
            }
          }
          const GV bn = kt_grp<E, kChunk>(sm.Na, rt, s, g, c16);
          const GV bm = kt_grp<E, kChunk>(sm.Mp, rt, s, g, c16);
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
          c = mma<E>(ak, bn, c);
          c = mma<E>(aq, bm, c);
          if constexpr (BF) {
            c = mma<E>(aklo, bn, c);
            c = mma<E>(aqlo, bm, c);
          }
          cc += c;
        }
      }
      const f32x4 Gs = *reinterpret_cast<const f32x4*>(&Gm[tok * LDG + ch0]);
      const f32x4 Gcv = *reinterpret_cast<const f32x4*>(&Gm[ce * LDG + ch0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) cc[e] *= __expf(Gcv[e] - Gs[e]);
    }
    // column side, the diagonal block walked: token tok goes r = b .. b + 15 with
    // E = prod_{tok < j <= r} a_j
    if (!fast) {
      f32x4 Ew = {0.f, 0.f, 0.f, 0.f}, w = Ew;
#pragma unroll 4
      for (int j = 0; j < 16; ++j) {
        const int r = b + j;
        Ew = Ew * *reinterpret_cast<const f32x4*>(&Am[r * LDG + ch0]);
        Ew = j == c16 ? one4 : Ew;
        const float na = to_f32(sm.Na[at<E, kChunk>(r, tok)]) * sm.cr[r];
        const float mp = to_f32(sm.Mp[at<E, kChunk>(r, tok)]);
        w += (na * row4<E, DK>(sm.Ks, r, ch0) + mp * row4<E, DK>(sm.Qs, r, ch0)) * Ew;
      }
      cc += w;
    }

    // the tile's outputs, token dot products and per-channel partial sums
    const f32x4 kx = row4<E, DK>(sm.Ks, tok, ch0), qx = row4<E, DK>(sm.Qs, tok, ch0);
    const f32x4 Gr = *reinterpret_cast<const f32x4*>(&Gm[tok * LDG + ch0]);
    const f32x4 GC = *reinterpret_cast<const f32x4*>(&Gm[(kChunk - 1) * LDG + ch0]);
    f32x4 eG, eGC;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      eG[e] = __expf(Gr[e]);
      eGC[e] = __expf(GC[e] - Gr[e]);
    }
    const float crr = sm.cr[tok];
    const f32x4 ZS = aZS[t], OS = aOS[t], DS = aDS[t];
    const f32x4 dq = r2 + eG * OS;
    store4_rsrc<E>(rdq, x0 + tok * xrow + hcol_x + ch0 * sizeof(E), dq);
    dkp[t] = crr * r1 + cc - crr * eG * ZS + eGC * DS;
    dGr[t] = kx * (crr * r1 - cc - crr * eG * ZS - eGC * DS) + qx * dq;
    float kR = 0.f, kz = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kR += kx[e] * r1[e];
      kz += eG[e] * kx[e] * ZS[e];
    }
    kR = col4_sum(kR);
    kz = col4_sum(kz);
    if (g == 0) {
      sm.kr[it][tok] = kR;
      sm.kzs[it][tok] = kz;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float w = row16_sum(eGC[e] * kx[e] * DS[e]);
      if (c16 == 0) sm.gcp[rt][ch0 + e] = w;
    }
  }
  __syncthreads();

  // ---- per token: deta and the step-size coefficient of dk; per channel: dG_C ----
  if (wave == 0) {
    const int r = lane;
    float kR = 0.f, kz = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      kR += sm.kr[it][r];
      kz += sm.kzs[it][r];
    }
    const float de = sm.rs[r] * (sm.zv[r] - kz + kR);
    if (t0 + r < T) p.deta[(bb * T + t0 + r) * H + hh] = de;
    sm.kcoef[r] = p.beta_given ? 0.f : -2.f * sm.cr[r] * sm.rs[r] * de;
  }
  if (tid < DK) {
    float w = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) w += sm.gcp[rt][tid];
    sm.dgc[tid] = w + __expf(Gm[(kChunk - 1) * LDG + tid]) * sm.sds[tid];
  }
  __syncthreads();

  // ---- dk (four consecutive d_k entries of one token per lane); dG into LDS ----
  float* dGm = sm.u.b.A;  // the decays are read no more
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int rt = (wave * TPW + t) % 4;
    const int r = 16 * rt + c16, ch0 = 16 * itw + 4 * g;
    const f32x4 dk = dkp[t] + sm.kcoef[r] * row4<E, DK>(sm.Ks, r, ch0);
    store4_rsrc<E>(rdk, x0 + r * xrow + hcol_x + ch0 * sizeof(E), dk);
    *reinterpret_cast<f32x4*>(&dGm[r * LDG + ch0]) = dGr[t];
  }
  __syncthreads();

  // ---- dlog a_j = sum_{r >= j} dG_r + dG_C: suffix sums per run, then the later runs' totals ----
  {
    float run[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) run[j] = dGm[(part * RUN + j) * LDG + pch];
#pragma unroll
    for (int j = RUN - 2; j >= 0; --j) run[j] += run[j + 1];
    sm.gpart[part][pch] = run[0];
    __syncthreads();
    float off = sm.dgc[pch];
    for (int q = part + 1; q < NPART; ++q) off += sm.gpart[q][pch];
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int64_t tr = t0 + part * RUN + j;
      if (tr < T) p.dlog_alpha[((bb * T + tr) * H + hh) * DK + pch] = run[j] + off;
    }
  }
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const ChunkBwdParams& p, hipStream_t stream) {
  if constexpr (kda_grad_fits<E, DK, DV>()) {
    hipLaunchKernelGGL((chunk_grad_kda_kernel<E, DK, DV>), dim3((unsigned)(p.heads * p.nchunks)), dim3(kKgThreads),
                       0, stream, p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;
  }
}

template <typename E>
hipError_t launch_e(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_dk_dv<E, 128, 128>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_dk_dv<E, 64, 64>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_dk_dv<E, 128, 64>(p, stream);
  return launch_dk_dv<E, 64, 128>(p, stream);
}

}  // namespace

bool chunk_grad_kda_supported(int64_t d_k, int64_t d_v, bool bf16_io) {
  if (bf16_io) return true;
  return d_k == 64 && d_v == 64;  // fp32 operands of 128-wide heads exceed 160 KiB of LDS
}

hipError_t launch_chunk_grad_kda(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, bool bf16_io,
                                 hipStream_t stream) {
  return bf16_io ? launch_e<bf16>(p, d_k, d_v, stream) : launch_e<float>(p, d_k, d_v, stream);
}

}  // namespace kla
