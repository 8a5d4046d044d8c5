// Chunkwise backward, the chunk-parallel part: dq, dk, dv, deta (or dbeta) and dlog(alpha)
// of every chunk, all chunks at once (one workgroup per chunk of one head), from the states
// and gradients the two scans left in the workspace.
//
// Sources: "Deep Dive into KDA", section 3 (the chunkwise forward differentiated here: the
// WY/UT solve, the triangular-masked intra-chunk scores and the log-domain decay ratios,
// never a division by a decayed quantity); "Kaczmarz Linear Attention", Abstract (the step
// size beta = eta / (||k||^2 + eps)).
//
// For a chunk with entering state S, leaving-state gradient dS', Delta and Zb (chunk_common.h),
// the forward's factors (eta rs, e^G, rs) and L[r][s] = e^{G_r - G_s} (s <= r):
//   Na = -(Zb Delta^T) o L (s < r);  Ma = diag(eta rs) Na;  Mp = (dO Delta^T) o L (s <= r)
//   dq = Mp K + diag(e^G) dO S^T
//   dk = Ma K + Ma^T K + Mp^T Q - diag(eta rs e^G) Zb S^T + diag(e^{G_C - G}) Delta dS'^T
//        - 2 eta rs^2 deta k                                    (the last term: KLA only)
//   dv = diag(eta rs) Zb
//   deta_r = rs_r (Zb_r.v_r - e^{G_r} k_r.(Zb S^T)_r + sum_s (Na o K K^T)[r][s])
//   dG_r   = -eta_r rs_r e^{G_r} k_r.(Zb S^T)_r + e^{G_r} q_r.(dO S^T)_r
//            + rowsum_r(E) - colsum_r(E) - e^{G_C - G_r} k_r.(Delta dS'^T)_r,
//            E = diag(eta rs) (Na o K K^T) + Mp o Q K^T,
//   plus, on the last row (G_C), e^{G_C} <S, dS'> + sum_r e^{G_C - G_r} k_r.(Delta dS'^T)_r;
//   dlog(alpha)_j = sum over r >= j of dG_r within the chunk (G is the chunk-local prefix).
// With beta given (gated DeltaNet; factors eta = beta, rs = 1) deta is d(beta) and dk has no
// step-size term.
//
// Products. The C x C products (K K^T, Q K^T, Zb Delta^T, dO Delta^T) are spread over the
// waves by lower-triangular 16 x 16 tile; the d_k x C outputs are computed transposed
// (dk^T = K^T Ma^T + ..., one d_k row block per wave) so that each lane holds four consecutive
// d_k entries of one token and stores them in one 8-byte (bf16) or 16-byte (fp32) store. The
// workspace's tile-ordered Delta, Zb, S and dS' are transposed into LDS on the way in (one
// 8- or 16-byte LDS write per lane piece) and read back with the transposing LDS read.
#include "tile_ops.h"

namespace kla {

namespace {

constexpr int kGradWaves = 8;
constexpr int kGradThreads = kGradWaves * kWave;

// The row-major operands, loaded straight into LDS: an LDS object of their own, so that the
// compiler can tell them apart from the rest when the next chunk's loads are in flight.
template <typename E, int DK, int DV>
struct GradOps {
  alignas(16) E Ks[kChunk * DK];
  alignas(16) E Qs[kChunk * DK];
  alignas(16) E dOs[kChunk * DV];
  alignas(16) E St[DV * DK];      // V ([64][DV]) while the C x C tiles are formed, then S^T, then dS'^T
};

template <typename E, int DK, int DV>
struct GradSmem {
  alignas(16) E Dt[DV * kChunk];  // Delta^T
  alignas(16) E Zt[DV * kChunk];  // Zb^T
  alignas(16) E Ma[kChunk * kChunk];
  alignas(16) E Mp[kChunk * kChunk];
  float G[kChunk], eG[kChunk], cr[kChunk], rs[kChunk], zv[kChunk], kcoef[kChunk];
  // Partial sums, one slot per producer, added in a fixed order (bitwise reproducible):
  // per lower-triangular C x C tile (row sums of its 16 rows, column sums of its 16 columns) ...
  float rowA[10][16], rowE[10][16], colE[10][16];
  // ... per 16-row d_k tile (token-row dot products), and per wave (<S, dS'>).
  float kzs[DK / 16][kChunk], qos[DK / 16][kChunk], kds[DK / 16][kChunk], sds[kGradWaves];
};

template <typename E, int DK, int DV>
constexpr bool grad_fits() {
  return sizeof(GradOps<E, DK, DV>) + sizeof(GradSmem<E, DK, DV>) <= 160 * 1024;
}

// One workgroup per CU by its LDS footprint: the kernel then runs persistently and loads the
// next chunk's register operands during the current chunk.
template <typename E, int DK, int DV>
constexpr bool grad_prefetch() {
  return 2 * (sizeof(GradOps<E, DK, DV>) + sizeof(GradSmem<E, DK, DV>)) > 160 * 1024;
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kGradThreads) void chunk_grad_kernel(ChunkBwdParams p) {
  constexpr bool BF = is_bf16<E>();
  constexpr int GK = Grp<E>::K;
  typedef typename Grp<E>::V GV;
  constexpr int PER = 16 / sizeof(E);
  typedef typename Vec16<E>::type V16;
  constexpr int NGD = DK / GK, NGV = DV / GK, NGT = kChunk / GK;
  constexpr int NW = kGradWaves, NT_ = kGradThreads;
  constexpr int NIT = DK / 16;           // 16-row tiles of d_k
  constexpr int TPW = NIT * 4 / NW;      // (d_k tile, token tile) output tiles per wave
  static_assert(TPW * NW == NIT * 4, "tile split");
  typedef GradSmem<E, DK, DV> Sm;
  __shared__ Sm sm;
  __shared__ GradOps<E, DK, DV> op;

  const int tid0 = threadIdx.x;
  const int64_t T = p.T, H = p.H, total = p.heads * p.nchunks;
  const Workspace<E> ws = Workspace<E>::at(p.ws, total);
  const BwdSpace<E> bw = BwdSpace<E>::at(p.ws, p.bwd_off, total, DK, DV);

  // Where the LDS footprint leaves one workgroup per CU, nothing else hides a chunk's load
  // latency: the kernel is persistent (workgroup b works on chunks b, b + gridDim.x, ...; chunk
  // id = head * nchunks + c) and the register-borne operands of the next chunk go into the
  // registers of the current one as soon as those are spent: Delta and Zb once they sit in LDS,
  // S and dS' once both have been put into LDS. With two or more workgroups per CU they overlap
  // each other instead, the extra live registers would cost that occupancy, and each workgroup
  // takes one chunk.
  constexpr bool PF = grad_prefetch<E, DK, DV>();
  constexpr int NSR = DK * DV / PER / NT_;      // 16-byte pieces of S (and of dS') per thread
  constexpr int NCH = kChunk * DV / PER / NT_;  // 16-byte pieces of Delta (and of Zb) per thread
  V16 sreg[NSR], dsreg[NSR], dlreg[NCH], zbreg[NCH];
  auto load_state = [&](int64_t id) __attribute__((always_inline)) {
    const E* gS = bw.Sn + id * DK * DV;
    const E* gdS = bw.dSn + id * DK * DV;
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
      sreg[i] = *reinterpret_cast<const V16*>(gS + (tid0 + NT_ * i) * PER);
      dsreg[i] = *reinterpret_cast<const V16*>(gdS + (tid0 + NT_ * i) * PER);
    }
  };
  auto load_t64 = [&](int64_t id) __attribute__((always_inline)) {
    const E* gD = bw.Dl + id * kChunk * DV;
    const E* gZ = bw.Zb + id * kChunk * DV;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      dlreg[i] = *reinterpret_cast<const V16*>(gD + (tid0 + NT_ * i) * PER);
      zbreg[i] = *reinterpret_cast<const V16*>(gZ + (tid0 + NT_ * i) * PER);
    }
  };
  // The row-major operands of chunk id straight into LDS (K, Q, dO, V), and (wave 0) the chunk's
  // per-token factors into registers.
  auto dma_rows = [&](rsrc_t r, E* dst, uint32_t base, uint32_t rowb, uint32_t hcol, int wave_, int lane_, auto ncol_tag)
      __attribute__((always_inline)) {
    constexpr int NCOL = decltype(ncol_tag)::value;
    constexpr int CPR = NCOL / PER, NBLK = kChunk * CPR / 64;
    static_assert(NBLK % NW == 0, "block split");
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) {
      const int blk = wave_ + NW * i, ph = 64 * blk + lane_, row = ph / CPR;
      dma16(r, dst + blk * 64 * PER, base + row * rowb + hcol + 16 * swz<E, CPR>(row, ph % CPR));
    }
  };
  float fla = 0.f, fcr = 0.f, feG = 0.f, frs = 0.f;
  auto issue_ops = [&](int64_t id, int wave_, int lane_) __attribute__((always_inline)) {
    const int64_t head = id / p.nchunks, t0 = (id % p.nchunks) * kChunk;
    const int64_t bb = head / p.H, hh = head % p.H, brow = bb * T * H;
    const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E);
    const uint32_t hcol_x = hh * DK * sizeof(E), hcol_v = hh * DV * sizeof(E);
    const uint32_t x0 = (uint32_t)t0 * xrow, v0 = (uint32_t)t0 * vrow;
    dma_rows(make_rsrc(static_cast<const E*>(p.k) + brow * DK, (uint32_t)(T * xrow)), op.Ks, x0, xrow, hcol_x, wave_,
             lane_, std::integral_constant<int, DK>());
    dma_rows(make_rsrc(static_cast<const E*>(p.q) + brow * DK, (uint32_t)(T * xrow)), op.Qs, x0, xrow, hcol_x, wave_,
             lane_, std::integral_constant<int, DK>());
    dma_rows(make_rsrc(static_cast<const E*>(p.dout) + brow * DV, (uint32_t)(T * vrow)), op.dOs, v0, vrow, hcol_v,
             wave_, lane_, std::integral_constant<int, DV>());
    dma_rows(make_rsrc(static_cast<const E*>(p.v) + brow * DV, (uint32_t)(T * vrow)), op.St, v0, vrow, hcol_v, wave_,
             lane_, std::integral_constant<int, DV>());
    if (wave_ == 0) {
      const bool valid = t0 + lane_ < T;
      fla = valid && p.log_alpha ? p.log_alpha[(bb * T + t0 + lane_) * H + hh] : 0.f;
      const float* sc = ws.SC + id * kScRows * kChunk;
      fcr = sc[kScCoefR * kChunk + lane_];
      feG = sc[kScEG * kChunk + lane_];
      frs = sc[kScRs * kChunk + lane_];
    }
  };
  // A barrier over this wave's LDS operations only: with the next chunk's loads into LDS in
  // flight, a workgroup fence would make the compiler wait for them.
  auto lds_barrier = [] __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Stores issued after the next chunk's loads (dk, dq; wave 0's per-token stores come on top,
  // and waiting for fewer younger operations than there are is still correct).
  constexpr int NSTO = 2 * TPW;
  if ((int64_t)blockIdx.x >= total) return;
  if constexpr (PF) {
    load_state(blockIdx.x);
    load_t64(blockIdx.x);
    issue_ops(blockIdx.x, __builtin_amdgcn_readfirstlane(tid0 >> 6), tid0 & 63);
    wait_vmem<0>();
  }
  for (int64_t chunk_id = blockIdx.x; chunk_id < total; chunk_id += gridDim.x) {
  // Per-thread index arithmetic is redone every chunk rather than kept live across the loop.
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t nid = chunk_id + gridDim.x;
  const bool more = nid < total;
  const int64_t head = chunk_id / p.nchunks, c = chunk_id % p.nchunks;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t t0 = c * kChunk;

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

  // ---- the row-major operands straight into LDS; Delta and Zb from registers (transposed on
  //      the way into LDS); S and dS' stay in registers until they are needed ----
  if constexpr (!PF) {
    load_state(chunk_id);
    issue_ops(chunk_id, wave, lane);
  }

  // tile-ordered [64 x DV] blocks, transposed into LDS: lane piece (rows 4g..4g+3 of column c of
  // tile (rt, ct)) -> row 16 ct + c, columns 16 rt + 4g .. + 3
  auto put_t64 = [&](const V16* x, E* dst) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ci = tid + NT_ * i;
#pragma unroll
      for (int h = 0; h < PER / 4; ++h) {
        const int pi = ci * (PER / 4) + h, ti = pi >> 6, l = pi & 63;
        const int rt = ti / (DV / 16), ct = ti % (DV / 16);
        E* d = dst + at<E, kChunk>(16 * ct + (l & 15), 16 * rt + 4 * (l >> 4));
        if constexpr (BF) {
          *reinterpret_cast<bf16x4*>(d) = half4(x[i], h);
        } else {
          *reinterpret_cast<f32x4*>(d) = x[i];
        }
      }
    }
  };
  if constexpr (!PF) load_t64(chunk_id);
  put_t64(dlreg, sm.Dt);
  put_t64(zbreg, sm.Zt);

  // per-token factors; the chunk-local decay prefix G as the forward forms it
  if (wave == 0) {
    sm.G[lane] = wave_inclusive_scan(fla);
    sm.cr[lane] = fcr;
    sm.eG[lane] = feG;
    sm.rs[lane] = frs;
  }
  // Upper off-diagonal tiles of Ma and Mp that the 32-token contraction groups below reach,
  // (0, 1) and (2, 3), are zero (fp32 groups are 16 tokens wide and reach none).
  {
    constexpr int CPT = 16 / PER;  // 16-byte chunks per tile row
    const int i = tid;
    if (i < 2 * 2 * 16 * CPT) {
      const int cc = i % CPT, rr = (i / CPT) % 16, tile = (i / (16 * CPT)) % 2, arr = i / (32 * CPT);
      const int r = 16 * (2 * tile) + rr, col = 16 * (2 * tile + 1) + PER * cc;
      V16 z;
#pragma unroll
      for (int e = 0; e < PER; ++e) z[e] = from_f32<E>(0.f);
      *reinterpret_cast<V16*>((arr ? sm.Mp : sm.Ma) + at<E, kChunk>(r, col)) = z;
    }
  }
  if constexpr (PF) {
    // this chunk's operands were loaded during the previous one: younger are its NSTO stores
    wait_vmem<NSTO>();
    lds_barrier();
  } else {
    wait_vmem<0>();
    __syncthreads();
  }
  // Issued after the barrier: with no load to LDS outstanding, the reads below need no wait.
  if (PF && more) load_t64(nid);

  // ---- C x C tiles: K K^T, Q K^T, Zb Delta^T, dO Delta^T -> Ma, Mp and the decay sums;
  //      on diagonal tiles also Zb V^T, whose diagonal is Zb_r . v_r ----
  // Ten tiles on eight waves: waves 0 and 1 take two each, so they get off-diagonal tiles (16
  // MFMAs; a diagonal tile adds the 4 of Zb V^T). Tile k keeps its slot k in the sums below.
  for (int j = wave; j < 10; j += NW) {
    const int k = j == 0 ? 1 : j == 1 ? 3 : j == 2 ? 0 : j == 3 ? 2 : j == 7 ? 9 : j == 8 ? 7 : j == 9 ? 8 : j;
    int ti, tj;
    tri_tile(k, ti, tj);
    f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk, F = kk, dp = kk, zvv = kk;
#pragma unroll
    for (int s = 0; s < NGD; ++s) {
      const GV bk = row_grp<E, DK>(op.Ks, 16 * tj + c16, s, g);
      kk = mma<E>(row_grp<E, DK>(op.Ks, 16 * ti + c16, s, g), bk, kk);
      qk = mma<E>(row_grp<E, DK>(op.Qs, 16 * ti + c16, s, g), bk, qk);
    }
#pragma unroll
    for (int s = 0; s < NGV; ++s) {
      const GV bd = kt_grp<E, kChunk>(sm.Dt, tj, s, g, c16);
      const GV az = kt_grp<E, kChunk>(sm.Zt, ti, s, g, c16);
      F = mma<E>(az, bd, F);
      dp = mma<E>(row_grp<E, DV>(op.dOs, 16 * ti + c16, s, g), bd, dp);
      if (ti == tj) zvv = mma<E>(az, row_grp<E, DV>(op.St, 16 * tj + c16, s, g), zvv);
    }
    if (ti == tj && (c16 >> 2) == g) {
      const int e = c16 & 3;
      sm.zv[16 * ti + c16] = e == 0 ? zvv[0] : e == 1 ? zvv[1] : e == 2 ? zvv[2] : zvv[3];
    }
    const int s = 16 * tj + c16;
    const float Gs = sm.G[s];
    float csum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * g + e;
      const float L = s <= r ? __expf(sm.G[r] - Gs) : 0.f;
      const float na = s < r ? -F[e] * L : 0.f;
      const float naKK = na * kk[e];
      const float crr = sm.cr[r];
      const float mp = dp[e] * L;
      const float ee = crr * naKK + mp * qk[e];
      sm.Ma[at<E, kChunk>(r, s)] = from_f32<E>(crr * na);
      sm.Mp[at<E, kChunk>(r, s)] = from_f32<E>(mp);
      csum += ee;
      const float ra = row16_sum(naKK), re = row16_sum(ee);
      if (c16 == 0) {
        sm.rowA[k][4 * g + e] = ra;
        sm.rowE[k][4 * g + e] = re;
      }
    }
    csum = col4_sum(csum);
    if (g == 0) sm.colE[k][c16] = csum;
  }
  // <S, dS'> over this thread's pieces (same positions in both)
  {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NSR; ++i)
#pragma unroll
      for (int e = 0; e < PER; ++e) acc += to_f32(sreg[i][e]) * to_f32(dsreg[i][e]);
    acc = wave_sum(acc);
    if (lane == 0) sm.sds[wave] = acc;
  }
  __syncthreads();

  // tile-ordered [DK x DV] registers -> transposed LDS [DV][DK]
  auto put_state = [&](const V16* regs) {
#pragma unroll
    for (int i = 0; i < NSR; ++i) {
      const int ci = tid + NT_ * i;
#pragma unroll
      for (int h = 0; h < PER / 4; ++h) {
        const int pi = ci * (PER / 4) + h, ti = pi >> 6, l = pi & 63;
        const int rt = ti / (DV / 16), ct = ti % (DV / 16);
        E* d = op.St + at<E, DK>(16 * ct + (l & 15), 16 * rt + 4 * (l >> 4));
        if constexpr (BF) {
          *reinterpret_cast<bf16x4*>(d) = half4(regs[i], h);
        } else {
          *reinterpret_cast<f32x4*>(d) = regs[i];
        }
      }
    }
  };
  put_state(sreg);
  __syncthreads();

  // ---- d_k x C products, transposed outputs; this wave's tiles (it, rt) ----
  f32x4 accK[TPW], accQ[TPW], accZS[TPW], accOS[TPW], accDS[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = (wave * TPW + t) / 4, rt = (wave * TPW + t) % 4;
    f32x4 k_ = {0.f, 0.f, 0.f, 0.f}, q_ = k_, zs = k_, os = k_;
#pragma unroll
    for (int s = 0; s < NGT; ++s) {
      const GV ak = kt_grp<E, DK>(op.Ks, it, s, g, c16);
      if (GK * s < 16 * (rt + 1)) {  // Ma[r][s], Mp[r][s] vanish for s > r
        k_ = mma<E>(ak, row_grp<E, kChunk>(sm.Ma, 16 * rt + c16, s, g), k_);
        q_ = mma<E>(ak, row_grp<E, kChunk>(sm.Mp, 16 * rt + c16, s, g), q_);
      }
      if (GK * (s + 1) > 16 * rt) {  // Ma[r][s], Mp[r][s] over r >= s
        const GV aq = kt_grp<E, DK>(op.Qs, it, s, g, c16);
        k_ = mma<E>(ak, kt_grp<E, kChunk>(sm.Ma, rt, s, g, c16), k_);
        k_ = mma<E>(aq, kt_grp<E, kChunk>(sm.Mp, rt, s, g, c16), k_);
      }
    }
#pragma unroll
    for (int s = 0; s < NGV; ++s) {
      const GV as = kt_grp<E, DK>(op.St, it, s, g, c16);
      zs = mma<E>(as, kt_grp<E, kChunk>(sm.Zt, rt, s, g, c16), zs);
      os = mma<E>(as, row_grp<E, DV>(op.dOs, 16 * rt + c16, s, g), os);
    }
    accK[t] = k_;
    accQ[t] = q_;
    accZS[t] = zs;
    accOS[t] = os;
  }
  __syncthreads();
  put_state(dsreg);
  if (PF && more) load_state(nid);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = (wave * TPW + t) / 4, rt = (wave * TPW + t) % 4;
    f32x4 ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NGV; ++s)
      ds = mma<E>(kt_grp<E, DK>(op.St, it, s, g, c16), kt_grp<E, kChunk>(sm.Dt, rt, s, g, c16), ds);
    accDS[t] = ds;
  }

  // ---- token-row dot products over each d_k tile: k.(Zb S^T), q.(dO S^T), k.(Delta dS'^T) ----
  f32x4 kv[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int it = (wave * TPW + t) / 4, rt = (wave * TPW + t) % 4;
    const int r = 16 * rt + c16, i0 = 16 * it + 4 * g;
    f32x4 kx, qx;
    if constexpr (BF) {
      const bf16x4 kb = *reinterpret_cast<const bf16x4*>(&op.Ks[at<E, DK>(r, i0)]);
      const bf16x4 qb = *reinterpret_cast<const bf16x4*>(&op.Qs[at<E, DK>(r, i0)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kx[e] = to_f32(kb[e]);
        qx[e] = to_f32(qb[e]);
      }
    } else {
      kx = *reinterpret_cast<const f32x4*>(&op.Ks[at<E, DK>(r, i0)]);
      qx = *reinterpret_cast<const f32x4*>(&op.Qs[at<E, DK>(r, i0)]);
    }
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
  // ---- dv = diag(eta rs) Zb: the transposing read of Zb^T gives four consecutive d_v
  //      entries of one token per lane. Waves 1 .. NW - 1 take its tiles, so that wave 0 can
  //      form the per-token sums below meanwhile (which the others would wait for). ----
  constexpr int NJT = DV / 16;
  if (wave != 0) {
#pragma unroll
    for (int t = 0; t < (4 * NJT + NW - 2) / (NW - 1); ++t) {
      const int q = wave - 1 + (NW - 1) * t, rt = q % 4, jt = q / 4;
      if (q < 4 * NJT) {
        const int r = 16 * rt + c16;
        const f32x4 z = col4<E, kChunk>(sm.Zt, 16 * jt, 16 * rt, g, c16);
        store4_rsrc<E>(rdv, v0 + r * vrow + hcol_v + (16 * jt + 4 * g) * sizeof(E), sm.cr[r] * z);
      }
    }
  }
  // The row-major operands are read no more in this chunk: the next chunk's go into LDS now.
  // (After the transposing reads of Zb^T above: the compiler cannot tell those from the loads'
  // destination and would wait for the loads before them.)
  if (PF && more) issue_ops(nid, wave, lane);

  // ---- per token: deta, dG, and dlog(alpha) as the within-chunk suffix sum of dG ----
  if (wave == 0) {
    const int r = lane, ti = r >> 4, rr = r & 15;
    float rowA = 0.f, rowE = 0.f, colE = 0.f;
    for (int tj = 0; tj <= ti; ++tj) {  // tiles (ti, tj): row r
      rowA += sm.rowA[ti * (ti + 1) / 2 + tj][rr];
      rowE += sm.rowE[ti * (ti + 1) / 2 + tj][rr];
    }
    for (int tk = ti; tk < 4; ++tk) colE += sm.colE[tk * (tk + 1) / 2 + ti][rr];  // tiles (tk, ti): column r
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
  if constexpr (PF)
    lds_barrier();
  else
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
  // the next chunk overwrites the LDS this one reads
  if constexpr (PF)
    lds_barrier();
  else
    __syncthreads();
  if constexpr (!PF) break;
  }  // chunk loop
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const ChunkBwdParams& p, hipStream_t stream) {
  if constexpr (grad_fits<E, DK, DV>()) {
    // Workgroups resident per compute unit (the same on every gfx950 device), times the device's CUs.
    static const int64_t per = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, chunk_grad_kernel<E, DK, DV>, kGradThreads, 0) !=
              hipSuccess || n <= 0)
        return (int64_t)1;
      return (int64_t)n;
    }();
    const int64_t resident = device_info().cus * per;
    const int64_t total = p.heads * p.nchunks;
    const int64_t grid = grad_prefetch<E, DK, DV>() && resident < total ? resident : total;
    hipLaunchKernelGGL((chunk_grad_kernel<E, DK, DV>), dim3((unsigned)grid), dim3(kGradThreads), 0, stream, p);
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

bool chunk_grad_supported(int64_t, int64_t, bool) { return true; }

hipError_t launch_chunk_grad_split(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, hipStream_t stream);

// fp32 operands of 128-wide heads exceed 160 KiB of LDS in this kernel: those shapes take the
// kernel of chunk_bwd_grad_f32.hip, which forms the products over d_v in parts.
hipError_t launch_chunk_grad(const ChunkBwdParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream) {
  if (!bf16_io && !(d_k == 64 && d_v == 64)) return launch_chunk_grad_split(p, d_k, d_v, stream);
  return bf16_io ? launch_e<bf16>(p, d_k, d_v, stream) : launch_e<float>(p, d_k, d_v, stream);
}

}  // namespace kla
