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
// Work split. A workgroup of W waves owns DVS = 16 W NT columns of one head's state and walks
// the chunks in order; each wave owns 16 NT of those columns for every d_k row and every token,
// so the chain S -> X -> R -> D -> S of its columns never leaves the wave and needs no barrier.
// The outputs O of its columns are formed by the wave itself, or, in the one-pass bf16 forward,
// by an output wave of its own from the state fragments and D' handed over in LDS. The slice of
// S lives in fp32 MFMA accumulators for the whole sequence. The workgroups of one head get ids
// congruent mod 8, so they run on one XCD and share its L2.
//
// Chaining without data movement. The contraction index of every product is enumerated in
// the order in which an MFMA accumulator holds its rows, so that the accumulators of one
// product are, register for register, an operand of the next. In a 16 x 16 accumulator tile,
// lane (g, c) (g = lane / 16, c = lane % 16) holds rows 4g .. 4g + 3 of column c. A "group" of
// the contraction is 32 indices for v_mfma_f32_16x16x32_bf16 (one instruction: lane group g
// feeds indices 32s + 4g + 0..3 from tile 2s and 32s + 16 + 4g + 0..3 from tile 2s + 1) and 16
// indices for v_mfma_f32_16x16x4_f32 (four instructions: instruction i feeds index
// 16s + 4g + i from tile s). A and B fragments of these MFMAs have the same lane layout, so an
// accumulator block serves as B (contracting its rows) or, for a transposed product, as A. The
// outputs are computed transposed (O^T = S^T Q^T + D'^T P^T), which leaves each lane four
// consecutive columns of one token row: they go to global memory without a transpose.
//
// For bf16 the forward modes enumerate the contraction differently (tile_ops.h, whole-chunk
// layout): lane group g feeds the 8 consecutive indices 32s + 8g + 0..7, the token tiles and
// state tiles holding their rows in the matching order, so that a fragment along a row is one
// 16-byte LDS read and needs no register moves; the backward recompute keeps the order above.
//
// Operands in LDS. K, Q, T and P are read as A fragments along their rows, K also transposed
// for K^T with the transposing read of gfx950, and V as four rows of one column (transposing
// read). All are row-major without padding, their 16-byte chunks XOR-swizzled by row so that
// these reads are free of bank conflicts.
// They arrive by direct-to-LDS buffer loads (no registers) into a ring of LDS buffers, one
// workgroup barrier per chunk (two in the one-pass bf16 forward, the second handing D' to the
// output waves): for bf16 issued by producer waves of the workgroup (two chunks ahead by four
// producers in the one-pass forward, P there one chunk ahead in a ring of its own; a chunk ahead
// by two elsewhere), for fp32 a chunk ahead by the scan waves themselves. Every global access goes through a buffer resource
// (rows past T read as zeros, stores past T are dropped), so there are no per-lane branches
// around memory operations.
#include "tile_ops.h"

namespace kla {

hipError_t launch_chunk_prep(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);

namespace {

// Producer waves. For bf16, more waves per workgroup, on the two SIMDs the scan waves leave
// idle, issue all direct-to-LDS loads; the scan waves then spend no issue cycles on them (about
// a fifth of a chunk's step when they issued them themselves). The one-pass bf16 forward loads
// two chunks ahead into three buffers where they fit, with four producers: a chunk's loads take
// about a step to issue and as long again to arrive, and each wave can have at most 63 memory
// operations outstanding (two chunks of loads are 2 x 27 for two producers, 2 x 14 for four).
// Elsewhere two producers load one chunk ahead.
//
// Output waves (the same one-pass forward): one more wave per scan wave, on the SIMDs the scan
// waves leave idle, forms that scan wave's outputs, Y^T = S^T Q^T and O^T = e^G Y^T + D'^T P^T
// (a third of its products), from the bf16 state fragments and D' the scan wave hands over in
// LDS. The scan wave's chain then holds only X, R, D and the state update. The hand-over needs
// a second barrier per chunk and room in LDS: P then has a two-slot ring of its own, loaded a
// chunk ahead, instead of a slot in each of the three operand buffers; D' goes into the scan
// wave's own V bytes of the chunk's buffer, dead once R is formed. (Measured: the B4 H16 T32768
// prefill 1.19 -> 1.17 ms, B8 H8 T4096 192 -> 185 us from cold caches; outputs bit-identical.)
template <typename E, int DK, int W, int NT>
constexpr size_t deep_lds() {
  return 3 * sizeof(ScanBuf<E, DK, W * 16 * NT, false, false>) + 2 * kChunk * kChunk * sizeof(E) +
         (size_t)W * NT * (DK / 32) * kWave * 16;
}
template <typename E, int DK, int DV, int W, int NT, int MODE>
constexpr bool scan_deep() {
  return is_bf16<E>() && (MODE == kScanFwd || MODE == kScanFwdSave) && NT == 1 && deep_lds<E, DK, W, NT>() <= 160 * 1024;
}
template <typename E, int DK, int DV, int W, int NT, int MODE>
constexpr int scan_outwaves() {
  return scan_deep<E, DK, DV, W, NT, MODE>() ? W : 0;
}
template <typename E, int DK, int DV, int W, int NT, int MODE>
constexpr int scan_producers() {
  return scan_deep<E, DK, DV, W, NT, MODE>() ? 4
         : (is_bf16<E>() && scan_ring<E, DK, W * 16 * NT, scan_kda(MODE)>() == 2) ? 2
                                                                                    : 0;
}

// MODE kScanRec (backward recompute): no outputs; instead every chunk's entering state S and its
// Delta (rs D) are stored to the backward workspace, and Q and P are not loaded.
// MODE kScanSeg (segment scan, pass 1): workgroups cover (head, segment) pairs and, besides the
// DV / DVS slices of the state, DK / DVS slices of identity columns (chunk_common.h).
// MODE kScanKda (per-channel decay): K, Q and the update's K2 are the decayed operands of the
// KDA workspace, the factor rows carry no decay, and the state decays per row by gamma.
// MODE kScanKdaSeg: the segment pass with the per-channel decay (both of the above).
// MODE kScanKdaRec: the backward's recompute with the per-channel decay.
// MODE kScanFwdSave: kScanFwd, and, as kScanRec, every chunk's entering state and Delta are
// stored (in kScanRec's tile order, which the backward reads) for a backward without recompute.
// MODE kScanKdaSave: the same for kScanKda (kScanKdaRec's order).
// (With four producers, two waves share each of their SIMDs: at most 256 registers per wave.)
template <typename E, int DK, int DV, int W, int NT, int MODE>
__global__ __launch_bounds__((W + scan_producers<E, DK, DV, W, NT, MODE>() + scan_outwaves<E, DK, DV, W, NT, MODE>()) *
                             kWave) __attribute__((
    amdgpu_waves_per_eu(scan_deep<E, DK, DV, W, NT, MODE>() ? 2 : 1, scan_deep<E, DK, DV, W, NT, MODE>() ? 2 : 1))) void
chunk_scan_kernel(ChunkParams p) {
  constexpr bool REC = scan_rec(MODE), SEG = scan_seg(MODE), KDA = scan_kda(MODE), SAVE = scan_save(MODE);
  constexpr bool BF = is_bf16<E>();
  // bf16 outside the backward recompute uses the whole-chunk operand layout (tile_ops.h): every
  // fragment along a row is one 16-byte LDS read. The recompute keeps the row-split layout, in
  // which the backward kernels read the states and Deltas it stores.
  constexpr bool PERM = BF && !REC;
  constexpr int LT = PERM ? kLayTok : kLaySplit, LL = PERM ? kLayLin : kLaySplit;  // K, T, V / Q, P
  constexpr int GK = Grp<E>::K;
  typedef typename Grp<E>::V GV;
  constexpr int NC = 16 * NT;        // state columns per wave
  constexpr int DVS = W * NC;        // state columns per workgroup
  constexpr int NS = DV / DVS;       // workgroups per head
  constexpr int RTK = DK / 16;       // 16-row tiles of S
  constexpr int NGD = DK / GK;       // groups over d_k
  constexpr int NGT = kChunk / GK;   // groups over the chunk's tokens
  constexpr int PER = 16 / sizeof(E);
  constexpr bool DEEP = scan_deep<E, DK, DV, W, NT, MODE>();
  typedef ScanBuf<E, DK, DVS, KDA, !DEEP> Buf;  // (DEEP: P in a ring of its own)
  constexpr int NB = DEEP ? 3 : scan_ring<E, DK, DVS, KDA>();  // LDS buffers: chunks c .. c + NB - 1 in flight
  constexpr int DIST = NB > 1 ? NB - 1 : 1;     // prefetch distance
  static_assert(DV % DVS == 0, "shape");
  // Distinct LDS objects (not an array indexed by chunk), so that the compiler can tell the
  // buffer being read from the ones later chunks are loaded into.
  __shared__ Buf buf0;
  __shared__ typename std::conditional<(NB >= 2), Buf, int>::type buf1;
  __shared__ typename std::conditional<(NB >= 3), Buf, int>::type buf2;
  // DEEP: the two slots of P's ring, and the scan waves' state fragments for their output waves
  // (wave w's fragment (s, ct) of lane l at v[((w NT + ct) NGD + s) 64 + l]).
  struct PSlot {
    alignas(16) E P[kChunk * kChunk];
  };
  struct HSlot {
    alignas(16) GV v[W * NT * NGD * kWave];
  };
  __shared__ typename std::conditional<DEEP, PSlot, int>::type pr0, pr1;
  __shared__ typename std::conditional<DEEP, HSlot, int>::type hs;

  // Workgroup -> (head, segment) and slice. The workgroups of one (head, segment) get ids
  // congruent mod 8, so they run on one XCD and share its L2.
  constexpr int NSK = SEG ? DK / DVS : 0;  // identity-column slices (segment scan)
  constexpr int NSA = NS + NSK;
  static_assert(!SEG || DK % DVS == 0, "shape");
  const int64_t nseg = SEG ? p.nseg : 1;
  const int bid = blockIdx.x;
  const int xcd = bid % p.xcds;
  const int local = bid / p.xcds;
  const int64_t vh = (int64_t)(local / NSA) * p.xcds + xcd;  // head * nseg + segment
  const int slice = local % NSA;
  if (vh >= p.heads * nseg) return;
  const int64_t head = vh / nseg, seg = vh % nseg;
  const bool mpart = slice >= NS;  // identity columns: segments after the first only
  if (mpart && seg == 0) return;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, nchunks = p.nchunks, H = p.H;
  const int64_t cb = SEG ? seg * p.seg_len : 0;                                     // first chunk
  const int64_t ce = SEG ? (cb + p.seg_len < nchunks ? cb + p.seg_len : nchunks) : nchunks;  // end
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int j0 = (mpart ? slice - NS : slice) * DVS;  // first state (or identity) column of this workgroup
  constexpr int NP = scan_producers<E, DK, DV, W, NT, MODE>();  // producer waves W .. W + NP - 1
  constexpr int NO = scan_outwaves<E, DK, DV, W, NT, MODE>();   // output waves W + NP .. W + NP + NO - 1
  const bool outw = NO > 0 && wave >= W + NP;                   // output wave of scan wave wave - W - NP
  const int cw = (outw ? wave - W - NP : wave) * NC;  // first column of this (or its scan) wave within the slice

  // ---- resources: this batch's rows of q/k/v/o, this head's workspace chunks ----
  const int64_t brow = bb * T * H;
  const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E);  // bytes per token
  const Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * nchunks);
  const int64_t chunk0 = head * nchunks;
  // K and Q rows: the q/k tensors (token stride H DK), or with KDA the decayed operands of the
  // workspace (chunk-contiguous rows of DK).
  const KdaSpace<E> kw = KdaSpace<E>::at(p.ws, p.heads * nchunks, DK);
  const uint32_t krow = KDA ? DK * sizeof(E) : xrow;
  const uint32_t kspan = KDA ? (uint32_t)(nchunks * kChunk * DK * sizeof(E)) : (uint32_t)(T * xrow);
  const rsrc_t rk = make_rsrc(KDA ? (const void*)(kw.K1 + chunk0 * kChunk * DK) : (const void*)(static_cast<const E*>(p.k) + brow * DK), kspan);
  const rsrc_t rq = make_rsrc(KDA ? (const void*)(kw.Q1 + chunk0 * kChunk * DK) : (const void*)(static_cast<const E*>(p.q) + brow * DK), kspan);
  const rsrc_t rk2 = make_rsrc(kw.K2 + chunk0 * kChunk * DK, KDA ? kspan : 0u);
  const rsrc_t rgam = make_rsrc(kw.gamma + chunk0 * DK, KDA ? (uint32_t)(nchunks * DK * 4) : 0u);
  const rsrc_t rv = make_rsrc(static_cast<const E*>(p.v) + brow * DV, (uint32_t)(T * vrow));
  const rsrc_t ro = make_rsrc(static_cast<const E*>(p.o) + brow * DV, (uint32_t)(T * vrow));
  constexpr uint32_t kMatBytes = kChunk * kChunk * sizeof(E), kScBytes = kScRows * kChunk * sizeof(float);
  const rsrc_t rt = make_rsrc(ws.T + chunk0 * kChunk * kChunk, (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rp = make_rsrc(ws.P + chunk0 * kChunk * kChunk, (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rsc = make_rsrc(ws.SC + chunk0 * kScRows * kChunk, (uint32_t)(nchunks * kScBytes));
  const uint32_t hcol_x = KDA ? 0u : hh * DK * sizeof(E), hcol_v = (hh * DV + (mpart ? 0 : j0)) * sizeof(E);
  // Backward recompute: this head's state and Delta blocks, tile-ordered (chunk_common.h).
  constexpr uint32_t kSBytes = DK * DV * sizeof(E), kDBytes = kChunk * DV * sizeof(E);
  const BwdSpace<E> bw = BwdSpace<E>::at(p.ws, p.bwd_off, p.heads * nchunks, DK, DV);
  const rsrc_t rsn = make_rsrc(bw.Sn + chunk0 * DK * DV, REC || SAVE ? (uint32_t)(nchunks * kSBytes) : 0u);
  const rsrc_t rdl = make_rsrc(bw.Dl + chunk0 * kChunk * DV, REC || SAVE ? (uint32_t)(nchunks * kDBytes) : 0u);
  const int ct0 = (j0 + cw) / 16;  // first global 16-column tile of this wave
  // Output rows: o (the state columns; after the first segment of a segment scan these are
  // outputs from a zero entering state, corrected in place later), or, for identity columns, Y
  // in the segment workspace ([chunk][64][DK] per head). One store form for both.
  const SegSpace<E> sg = SegSpace<E>::at(p.ws, p.seg_off, p.heads * nchunks, p.heads * nseg, DK, DV);
  const rsrc_t rout = mpart ? make_rsrc(sg.Y + chunk0 * kChunk * DK, (uint32_t)(nchunks * kChunk * DK * sizeof(E))) : ro;
  const uint32_t orow = mpart ? DK * sizeof(E) : vrow;                       // bytes per output row
  const uint32_t ocol = mpart ? (j0 + cw) * sizeof(E) : hcol_v + cw * sizeof(E);  // this wave's first column

  // ---- DMA of one chunk's operands: 1 KiB LDS blocks dealt round-robin to the loading waves (the
  // producers, else the scan waves). Lane l of block b fills physical chunk 64 b + l; its source
  // is the logical chunk stored there. ----
  constexpr int WD = NP ? NP : W;         // loading waves
  const int dw = NP ? wave - W : wave;    // this wave's index among them (producers only, if any)
  constexpr int CK = DK / PER, CT = kChunk / PER, CV = DVS / PER;  // 16-byte chunks per row
  constexpr int BK = kChunk * CK / 64, BT = kChunk * CT / 64, BV = kChunk * CV / 64;  // blocks
  static_assert(BK % WD == 0 && BT % WD == 0 && BV % WD == 0, "block split");
  constexpr int NBK = BK / WD, NBT = BT / WD, NBV = BV / WD;
  // Per-lane byte offsets within a row-block, excluding the chunk's base (fixed for the kernel).
  uint32_t offk[NBK], offq[NBK], offt[NBT], offp[NBT], offv[NBV];
#pragma unroll
  for (int i = 0; i < NBK; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CK;
    offk[i] = r * krow + hcol_x + 16 * swz<E, CK, LT>(r, ph % CK);
    offq[i] = r * krow + hcol_x + 16 * swz<E, CK, LL>(r, ph % CK);
  }
#pragma unroll
  for (int i = 0; i < NBT; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CT;
    offt[i] = (r * CT + swz<E, CT, LT>(r, ph % CT)) * 16;
    offp[i] = (r * CT + swz<E, CT, LL>(r, ph % CT)) * 16;
  }
#pragma unroll
  for (int i = 0; i < NBV; ++i) {
    const int ph = 64 * (dw + WD * i) + lane, r = ph / CV;
    offv[i] = r * vrow + hcol_v + 16 * swz<E, CV, LT>(r, ph % CV);
  }
  // Every loading wave issues the same NDMA loads per chunk (the factor block is loaded by all of
  // them, identical bytes), so that the wait counts below are compile-time constants. A chunk
  // past the end is clamped to the last one (loaded again, never read).
  constexpr int NDMA = (1 + !REC + KDA) * NBK + (1 + (!REC && !DEEP)) * NBT + NBV + 1 + KDA;
  constexpr int NST = REC ? (RTK + 4) * NT : SAVE ? (RTK + 8) * NT : 4 * NT;  // stores per chunk and wave
  auto fetch = [&](Buf& B, int64_t c) {
    c = c < ce ? c : ce - 1;
    const uint32_t t0 = (uint32_t)(c * kChunk);
#pragma unroll
    for (int i = 0; i < NBK; ++i) {
      const int blk = dw + WD * i;
      dma16(rk, B.K + blk * 64 * PER, t0 * krow + offk[i]);
      if constexpr (!REC) dma16(rq, B.Q + blk * 64 * PER, t0 * krow + offq[i]);
      if constexpr (KDA) dma16(rk2, B.K2 + blk * 64 * PER, t0 * krow + offk[i]);
    }
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int blk = dw + WD * i;
      dma16(rt, B.T + blk * 64 * PER, (uint32_t)c * kMatBytes + offt[i]);
      if constexpr (!REC && !DEEP) dma16(rp, B.P + blk * 64 * PER, (uint32_t)c * kMatBytes + offp[i]);
    }
#pragma unroll
    for (int i = 0; i < NBV; ++i) {
      const int blk = dw + WD * i;
      dma16(rv, B.V + blk * 64 * PER, t0 * vrow + offv[i]);
    }
    dma16(rsc, B.sc, (uint32_t)c * kScBytes + 16 * lane);
    if constexpr (KDA) dma16(rgam, B.gam, (uint32_t)c * DK * 4 + 16 * lane);
  };
  // DEEP: chunk c's P into a slot of P's ring (NBT loads per producer).
  auto fetch_p = [&](E* Pd, int64_t c) {
    c = c < ce ? c : ce - 1;
#pragma unroll
    for (int i = 0; i < NBT; ++i) {
      const int blk = dw + WD * i;
      dma16(rp, Pd + blk * 64 * PER, (uint32_t)c * kMatBytes + offp[i]);
    }
  };

  // DEEP: element offset in V of hand-over piece idx (0 .. 64 NGT - 1) of scan wave wv's D': the
  // 16-byte chunks of the wave's own columns (2 per row), dead in V once the wave has formed R.
  auto dpos = [&](int wv, int idx) { return at<E, DVS, LT>(idx >> 1, 16 * wv + 8 * (idx & 1)); };
  // Slot of the T and P fragments (row tile r, group s) read early: row tiles 0, 1 need group 0.
  auto tp_slot = [](int r, int s) { return r < 2 ? r : 2 + 2 * (r - 2) + s; };
  // A barrier without a workgroup fence, for waves with stores of their own in flight (the fence
  // would wait for them; the output waves): this wave's LDS accesses are complete before it.
  auto raw_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Tile-ordered offsets (elements, kScanRec's order: tile r lane (g, c) holds rows 16 r + 4 g
  // + 0..3 of column c) of the four state rows / four tokens this lane holds in its state tile
  // rt / token tile r of column tile ct.
  auto save_off_s = [&](int rt, int ct) {
    const int r0 = PERM ? k_row(rt, g, 0) : 16 * rt + 4 * g;
    return tile_off(r0 >> 4, ct0 + ct, DV / 16, ((r0 & 15) >> 2) * 16 + c16);
  };
  auto save_off_t = [&](int r, int ct) {
    const int t = PERM ? tok_row(r, 4 * g) : 16 * r + 4 * g;
    return tile_off(t >> 4, ct0 + ct, DV / 16, ((t & 15) >> 2) * 16 + c16);
  };

  if constexpr (DEEP) {
    static_assert(NB == 3 && NP == 4 && NO == W, "four producers serve a three-buffer ring and P's ring");
    if (wave >= W && !outw) {  // producer: the loads of every chunk, two chunks ahead (P one)
      // Issue order: after chunk c's first barrier, chunk c + 1's P, then the rest of chunk
      // c + 2. Before chunk c's first barrier, chunk c's loads and its P are complete and younger
      // are only the rest of chunk c + 1 (the same count for every chunk: a fetch past the end
      // loads the last chunk again). This wave writes LDS only by these loads, and the wait is all
      // the barrier needs of them: a workgroup fence there would make the compiler wait for chunk
      // c + 1's loads as well.
      auto pstep = [&](Buf& Bt, E* Pn, int64_t c) __attribute__((always_inline)) {
        wait_vmem<NDMA>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // chunk c is in LDS; every wave is done with chunk c - 1 (Bt, Pn)
        asm volatile("" ::: "memory");
        fetch_p(Pn, c + 1);
        fetch(Bt, c + 2);
        __builtin_amdgcn_s_barrier();  // chunk c's second barrier (D' handed to the output waves)
      };
      if (ce > cb) {
        fetch_p(pr0.P, cb);
        fetch(buf0, cb);
        fetch(buf1, cb + 1);
      }
      int k = 0;
      for (int64_t c = cb; c < ce; ++c) {
        Buf& Bt = k == 0 ? buf2 : k == 1 ? buf0 : buf1;  // held chunk c - 1, receives chunk c + 2
        pstep(Bt, ((c + 1 - cb) & 1) ? pr1.P : pr0.P, c);
        k = k == 2 ? 0 : k + 1;
      }
      wait_vmem<0>();  // no load into LDS outlives the workgroup
      return;
    }
    if (outw) {  // output wave of scan wave ow: two barriers per chunk, as every wave
      const int ow = wave - W - NP;
      // Its LDS reads are complete before each barrier (the scan wave overwrites what it read
      // after the next one); no workgroup fence, which would also wait for its output stores.
      auto obarrier = raw_barrier;
      int k = 0;
      for (int64_t c = cb; c < ce; ++c) {
        const Buf& B = k == 0 ? buf0 : k == 1 ? buf1 : buf2;
        const E* Pc = ((c - cb) & 1) ? pr1.P : pr0.P;
        obarrier();  // chunk c's operands, its P and the scan wave's state fragments are in LDS
        GV so[NGD];
#pragma unroll
        for (int s = 0; s < NGD; ++s) so[s] = hs.v[(ow * NGD + s) * kWave + lane];
        // Y^T = S^T Q^T over the four token tiles, the Q fragments of tile r + 1 read during the
        // products of tile r; P's fragments and e^G with the last tile.
        GV fq[2][NGD], fp[6];
        float eGt[4];
        f32x4 Y[4];
        auto load_q = [&](int r, int slot) __attribute__((always_inline)) {
#pragma unroll
          for (int s = 0; s < NGD; ++s) fq[slot][s] = row8_grp<DK, kLayLin>(B.Q, 16 * r + c16, s, g);
        };
        load_q(0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r + 1 < 4) {
            load_q(r + 1, (r + 1) & 1);
          } else {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              eGt[rr] = B.sc[kScEG * kChunk + 16 * rr + c16];
#pragma unroll
              for (int s2 = 0; s2 < 2; ++s2)
                if (GK * s2 < 16 * (rr + 1)) fp[tp_slot(rr, s2)] = row8_grp<kChunk, kLayLin>(Pc, 16 * rr + c16, s2, g);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          Y[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NGD; ++s) Y[r] = mma<E>(so[s], fq[r & 1][s], Y[r]);
          __builtin_amdgcn_sched_barrier(0);
        }
        obarrier();  // chunk c's D' is in the scan wave's V bytes
        GV d1[NGT];
#pragma unroll
        for (int s = 0; s < NGT; ++s) d1[s] = *reinterpret_cast<const GV*>(B.V + dpos(ow, s * kWave + lane));
        if constexpr (SAVE) {
          // The chunk's entering state and Delta for the backward, from the hand-over: group s of
          // so / d1 holds state rows / tokens 32 s + 8 g + 0..7 of the lane's column, the bf16
          // values the scan wave would store; each half goes to its place in kScanRec's order.
#pragma unroll
          for (int s = 0; s < NGD; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int r0 = 32 * s + 8 * g + 4 * h;
              const uint32_t off = (uint32_t)c * kSBytes +
                                   tile_off(r0 >> 4, ct0, DV / 16, ((r0 & 15) >> 2) * 16 + c16) * sizeof(E);
              __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, half4(so[s], h)), rsn, off, 0, 0);
            }
#pragma unroll
          for (int s = 0; s < NGT; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int r0 = 32 * s + 8 * g + 4 * h;
              const uint32_t off = (uint32_t)c * kDBytes +
                                   tile_off(r0 >> 4, ct0, DV / 16, ((r0 & 15) >> 2) * 16 + c16) * sizeof(E);
              __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, half4(d1[s], h)), rdl, off, 0, 0);
            }
        }
        // O^T = e^G Y^T + D'^T P^T, each lane four consecutive columns of one token row
        const uint32_t t0 = (uint32_t)(c * kChunk);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 o = eGt[r] * Y[r];
#pragma unroll
          for (int s = 0; s < NGT; ++s)
            if (GK * s < 16 * (r + 1)) o = mma<E>(d1[s], fp[tp_slot(r, s)], o);
          store4_rsrc<E>(rout, (t0 + 16 * r + c16) * orow + ocol + 4 * g * sizeof(E), o);
        }
        k = k == 2 ? 0 : k + 1;
      }
      wait_vmem<0>();
      return;
    }
  } else if constexpr (NP > 0) {
    static_assert(NB == 2, "producers serve a two-buffer ring");
    if (wave >= W) {  // producer: the loads of every chunk, one chunk ahead, one barrier per chunk
      if (ce > cb) fetch(buf0, cb);
      for (int64_t c = cb; c < ce; c += 2) {
        wait_vmem<0>();
        __syncthreads();  // chunk c is in buf0; every wave is done with chunk c - 1 (buf1)
        fetch(buf1, c + 1);
        if (c + 1 < ce) {
          wait_vmem<0>();
          __syncthreads();
          fetch(buf0, c + 2);
        }
      }
      wait_vmem<0>();  // no load into LDS outlives the workgroup
      return;
    }
  }

  // ---- this wave's state columns: S[rt][ct] lane (g, c) = S[srow(rt, e)][j0 + cw + 16 ct + c] ----
  auto srow = [&](int rt, int e) { return PERM ? k_row(rt, g, e) : 16 * rt + 4 * g + e; };
  // First token of the four (consecutive) tokens that lane group g holds in token tile r.
  auto trow4 = [&](int r) { return PERM ? tok_row(r, 4 * g) : 16 * r + 4 * g; };
  f32x4 S[RTK][NT];
  if (mpart) {  // identity columns
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][ct][e] = srow(r, e) == j0 + cw + 16 * ct + c16 ? 1.f : 0.f;
  } else if (p.state_in && seg == 0) {
    const float* Sin = p.state_in + head * (int64_t)DK * DV;
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][ct][e] = Sin[(int64_t)srow(r, e) * DV + j0 + cw + 16 * ct + c16];
  } else {
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) S[r][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // The state's bf16 fragments (operand of X; DEEP: formed at the end of the previous chunk's
  // step and handed to the output wave through hs).
  GV sb[NGD][NT];
  auto state_frags = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 tiles[RTK];
#pragma unroll
      for (int r = 0; r < RTK; ++r) tiles[r] = S[r][ct];
#pragma unroll
      for (int s = 0; s < NGD; ++s) {
        if constexpr (PERM)
          sb[s][ct] = state_grp(tiles, s, g);
        else
          sb[s][ct] = acc_grp<E>(tiles, s);
      }
    }
  };
  // One chunk: B holds its operands; chunk c + DIST is loaded into Bn meanwhile (Bn held chunk
  // c - 1). Issue order per wave: the loads of chunks 0 .. DIST - 1, then per chunk k the loads
  // of chunk k + DIST and the k's output stores. Before chunk c's barrier the loads of chunk c
  // must be complete: younger are (DIST - 1) chunks of loads and, from c >= DIST on, the stores
  // of DIST chunks (fewer stores before that: waiting for more is still correct).
  auto step = [&](Buf& B, Buf& Bn, int64_t c) __attribute__((always_inline)) {
    if constexpr (NP > 0) {
      // the producers waited for chunk c's loads before this barrier
    } else if constexpr (NB == 1) {
      wait_vmem<0>();
    } else {
      if (c - cb < DIST)
        wait_vmem<(DIST - 1) * NDMA>();
      else
        wait_vmem<(DIST - 1) * NDMA + DIST * NST>();
    }
    __syncthreads();  // chunk c's operands are in LDS; every wave is done with chunk c - 1
    if constexpr (NB > 1 && NP == 0) fetch(Bn, c + DIST);
    const uint32_t t0 = (uint32_t)(c * kChunk);
    if constexpr (REC || (SAVE && !DEEP)) {  // the state entering chunk c (DEEP: the output wave stores it)
#pragma unroll
      for (int r = 0; r < RTK; ++r)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          store4_rsrc<E>(rsn, (uint32_t)c * kSBytes + save_off_s(r, ct) * sizeof(E), S[r][ct]);
    }

    // ---- X = K S (token rows x this wave's columns) and Y^T = S^T Q^T (DEEP: the output wave's) ----
    if constexpr (!DEEP) state_frags();
    f32x4 X[4][NT], Y[NT][4];
    // One-pass bf16 forward, scalar gate or per-channel decay (EARLY): the operands of the later
    // products are read early: T and P fragments (the groups below the diagonal), the V columns
    // and the per-token factors. (The segment pass keeps its reads beside its products: it would
    // spill. With the per-channel decay: bit-identical outputs, within noise on B8 H8 T4096 and
    // the B4 H16 T32768 prefill.)
    constexpr bool EARLY = PERM && (MODE == kScanFwd || MODE == kScanFwdSave || MODE == kScanKda || MODE == kScanKdaSave);
    constexpr int NTF = EARLY ? 6 : 1;  // T / P fragments: row tiles 0, 1 need group 0; 2, 3 groups 0, 1
    GV ft[NTF], fp[NTF];
    f32x4 fv[4][NT], fcoef[4], feg[4];
    if constexpr (EARLY) {
      // X = K S and Y^T = S^T Q^T as a two-stage pipeline over the four token tiles: the eight
      // fragment reads of tile r + 1 are issued before the eight products of tile r, so that each
      // product finds its operands in registers (issued one or two ahead, every product waited
      // for its read). The fences keep the scheduler from pulling the reads back to their uses.
      GV fk[2][NGD], fq[2][NGD];
      auto load_xy = [&](int r, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NGD; ++s) {
          fk[slot][s] = row8_grp<DK, kLayTok>(B.K, tok_row(r, c16), s, g);
          if constexpr (!REC && !DEEP) fq[slot][s] = row8_grp<DK, kLayLin>(B.Q, 16 * r + c16, s, g);
        }
      };
      load_xy(0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r + 1 < 4) {
          load_xy(r + 1, (r + 1) & 1);
        } else {
          // The last tile's products cover the reads of everything the rest of the step reads
          // from this chunk's buffer, except K^T for the state update (read with its products).
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            fcoef[rr] = *reinterpret_cast<const f32x4*>(&B.sc[kScCoefR * kChunk + trow4(rr)]);
            feg[rr] = *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + trow4(rr)]);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) fv[rr][ct] = col4<E, DVS, LT>(B.V, tok_row(rr, 0), cw + 16 * ct, g, c16);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
              if (GK * s2 < 16 * (rr + 1)) {
                ft[tp_slot(rr, s2)] = row8_grp<kChunk, kLayTok>(B.T, tok_row(rr, c16), s2, g);
                if constexpr (!REC && !DEEP) fp[tp_slot(rr, s2)] = row8_grp<kChunk, kLayLin>(B.P, 16 * rr + c16, s2, g);
              }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) X[r][ct] = Y[ct][r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NGD; ++s) {
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) X[r][ct] = mma<E>(fk[r & 1][s], sb[s][ct], X[r][ct]);
          if constexpr (!REC && !DEEP) {
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) Y[ct][r] = mma<E>(sb[s][ct], fq[r & 1][s], Y[ct][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) X[r][ct] = Y[ct][r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NGD; ++s) {
          GV ak;
          if constexpr (PERM)
            ak = row8_grp<DK, kLayTok>(B.K, tok_row(r, c16), s, g);
          else
            ak = row_grp<E, DK>(B.K, 16 * r + c16, s, g);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) X[r][ct] = mma<E>(ak, sb[s][ct], X[r][ct]);
          if constexpr (!REC) {
            GV aq;
            if constexpr (PERM)
              aq = row8_grp<DK, kLayLin>(B.Q, 16 * r + c16, s, g);
            else
              aq = row_grp<E, DK>(B.Q, 16 * r + c16, s, g);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) Y[ct][r] = mma<E>(sb[s][ct], aq, Y[ct][r]);
          }
        }
      }
    }

    // Scheduling fences around the middle of the step: without them the scheduler, working on
    // the whole step at once, issues each LDS fragment read right before its MFMA and waits on it
    // (measured 30 % slower); fenced, it keeps several reads in flight in every part.
    __builtin_amdgcn_sched_barrier(0);
    // ---- R = eta rs (V - e^G X), in place of X (identity columns carry no values) ----
    const float vscale = mpart ? 0.f : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 coefR = EARLY ? fcoef[r] : *reinterpret_cast<const f32x4*>(&B.sc[kScCoefR * kChunk + trow4(r)]);
      const f32x4 eG = EARLY ? feg[r] : *reinterpret_cast<const f32x4*>(&B.sc[kScEG * kChunk + trow4(r)]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const f32x4 v = vscale * (EARLY ? fv[r][ct]
                                        : col4<E, DVS, LT>(B.V, PERM ? tok_row(r, 0) : 16 * r, cw + 16 * ct, g, c16));
        X[r][ct] = coefR * (v - eG * X[r][ct]);
      }
    }

    // ---- D = T R (T lower triangular: row tile r needs tokens below 16 (r + 1)) ----
    GV rb[NT][NGT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const f32x4 tiles[4] = {X[0][ct], X[1][ct], X[2][ct], X[3][ct]};
#pragma unroll
      for (int s = 0; s < NGT; ++s) rb[ct][s] = acc_grp<E>(tiles, s);
    }
    f32x4 D1[NT][4], D2[NT][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 d[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) d[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * s < 16 * (r + 1)) {
          GV at_;
          if constexpr (EARLY)
            at_ = ft[tp_slot(r, s)];
          else if constexpr (PERM)
            at_ = row8_grp<kChunk, kLayTok>(B.T, tok_row(r, c16), s, g);
          else
            at_ = row_grp<E, kChunk>(B.T, 16 * r + c16, s, g);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) d[ct] = mma<E>(at_, rb[ct][s], d[ct]);
        }
      }
      const f32x4 rs = *reinterpret_cast<const f32x4*>(&B.sc[kScRs * kChunk + trow4(r)]);
      const f32x4 dd = *reinterpret_cast<const f32x4*>(&B.sc[kScD2 * kChunk + trow4(r)]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        D1[ct][r] = rs * d[ct];
        D2[ct][r] = dd * d[ct];
      }
    }
    GV b1[NT][NGT], b2[NT][NGT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        b1[ct][s] = acc_grp<E>(D1[ct], s);
        b2[ct][s] = acc_grp<E>(D2[ct], s);
      }

    // ---- O^T = (Y^T scaled by e^G per token) + D'^T P^T; or, recomputing, Delta = D' ----
    if constexpr (REC || (SAVE && !DEEP)) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          store4_rsrc<E>(rdl, (uint32_t)c * kDBytes + save_off_t(r, ct) * sizeof(E), D1[ct][r]);
    }
    if constexpr (DEEP) {
      // D' to this wave's own V bytes of the chunk's buffer, then the chunk's second barrier: the
      // output wave forms O from it.
#pragma unroll
      for (int s = 0; s < NGT; ++s) *reinterpret_cast<GV*>(B.V + dpos(wave, s * kWave + lane)) = b1[0][s];
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4 && !REC && !DEEP; ++r) {
      const float eGt = B.sc[kScEG * kChunk + 16 * r + c16];
      f32x4 o[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) o[ct] = eGt * Y[ct][r];
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        if (GK * s < 16 * (r + 1)) {
          GV ap;
          if constexpr (EARLY)
            ap = fp[tp_slot(r, s)];
          else if constexpr (PERM)
            ap = row8_grp<kChunk, kLayLin>(B.P, 16 * r + c16, s, g);
          else
            ap = row_grp<E, kChunk>(B.P, 16 * r + c16, s, g);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) o[ct] = mma<E>(b1[ct][s], ap, o[ct]);
        }
      }
      const uint32_t off = (t0 + 16 * r + c16) * orow + ocol + 4 * g * sizeof(E);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) store4_rsrc<E>(rout, off + 16 * ct * sizeof(E), o[ct]);
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- S <- e^{G_C} S + K^T diag(e^{G_C - G}) D' (KDA: Diag(gamma) S + K2^T D') ----
    const float eGC = B.sc[kScEG * kChunk + kChunk - 1];
#pragma unroll
    for (int r = 0; r < RTK; ++r) {
      if constexpr (KDA) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&B.gam[srow(r, 0)]);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) S[r][ct] *= gm;
      } else {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) S[r][ct] *= eGC;
      }
#pragma unroll
      for (int s = 0; s < NGT; ++s) {
        GV ak;
        if constexpr (PERM)
          ak = kt8_grp<DK>(KDA ? B.K2 : B.K, r, s, g, c16);
        else
          ak = kt_grp<E, DK>(KDA ? B.K2 : B.K, r, s, g, c16);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) S[r][ct] = mma<E>(ak, b2[ct][s], S[r][ct]);
      }
    }
    if constexpr (DEEP) {  // the next chunk's state fragments, also to the output wave
      state_frags();
#pragma unroll
      for (int s = 0; s < NGD; ++s) hs.v[(wave * NGD + s) * kWave + lane] = sb[s][0];
    }
    if constexpr (NB == 1) {
      __syncthreads();
      if (c + 1 < ce) fetch(B, c + 1);
    }
  };

  if (NP == 0 && ce > cb) fetch(buf0, cb);  // chunk cb (one chunk ahead)
  if constexpr (NB == 3) {
    if constexpr (DEEP) {  // the first chunk's state fragments, for X and the output wave
      state_frags();
#pragma unroll
      for (int s = 0; s < NGD; ++s) hs.v[(wave * NGD + s) * kWave + lane] = sb[s][0];
    }
    // One copy of the step, its buffer chosen per chunk: unrolled three ways (a copy per buffer)
    // the forward measured 20-25 % slower.
    int k = 0;
    for (int64_t c = cb; c < ce; ++c) {
      Buf& B = k == 0 ? buf0 : k == 1 ? buf1 : buf2;
      step(B, B, c);  // (the producers load; no next buffer is needed here)
      k = k == 2 ? 0 : k + 1;
    }
  } else if constexpr (NB == 2) {
    for (int64_t c = cb; c < ce; c += 2) {
      step(buf0, buf1, c);
      if (c + 1 < ce) step(buf1, buf0, c + 1);
    }
  } else {
    for (int64_t c = cb; c < ce; ++c) step(buf0, buf0, c);
  }

  wait_vmem<0>();  // no load into LDS outlives the workgroup
  if (SEG) {  // end state of the segment, or its transition (identity columns)
    float* dst = mpart ? sg.Mseg + vh * DK * DK : sg.Send + vh * DK * DV;
    const int ld = mpart ? DK : DV;
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(int64_t)srow(r, e) * ld + j0 + cw + 16 * ct + c16] = S[r][ct][e];
  } else if (p.state_out) {
    float* Sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int r = 0; r < RTK; ++r)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sout[(int64_t)srow(r, e) * DV + j0 + cw + 16 * ct + c16] = S[r][ct][e];
  }
}

template <typename E, int DK, int DV, int W, int NT, int MODE>
hipError_t launch_wnt(const ChunkParams& p, hipStream_t stream) {
  constexpr int DVS = W * 16 * NT;
  constexpr bool SEG = scan_seg(MODE);
  static_assert(DVS == scan_cols(is_bf16<E>(), SEG), "column split as planned");
  constexpr int NSA = DV / DVS + (SEG ? DK / DVS : 0);
  const int64_t units = p.heads * (SEG ? p.nseg : 1);  // (head, segment) pairs
  const int64_t units8 = (units + p.xcds - 1) / p.xcds * p.xcds;
  constexpr int NP = scan_producers<E, DK, DV, W, NT, MODE>();
  constexpr int NO = scan_outwaves<E, DK, DV, W, NT, MODE>();
  hipLaunchKernelGGL((chunk_scan_kernel<E, DK, DV, W, NT, MODE>), dim3((unsigned)(units8 * NSA)),
                     dim3((W + NP + NO) * kWave), 0, stream, p);
  return hipGetLastError();
}

template <typename E, int DK, int DV, int MODE>
hipError_t launch_dk_dv(const ChunkParams& p, hipStream_t stream) {
  // bf16: two waves of 16 columns per workgroup (32 columns; four workgroups per 128-column
  // head). This split measured fastest: a wave's time per chunk is set by latency, not by
  // throughput, so more workgroups per head beat wider ones. fp32: four waves (its operands
  // need a single LDS buffer, whose load is not overlapped, so more columns share it).
  // The segment scan's first pass uses four waves for bf16 too (scan_cols).
  if constexpr (is_bf16<E>() && !scan_seg(MODE))
    return launch_wnt<E, DK, DV, 2, 1, MODE>(p, stream);
  else
    return launch_wnt<E, DK, DV, 4, 1, MODE>(p, stream);
}

template <typename E, int MODE = kScanFwd>
hipError_t launch_scan(const ChunkParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_dk_dv<E, 128, 128, MODE>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_dk_dv<E, 64, 64, MODE>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_dk_dv<E, 128, 64, MODE>(p, stream);
  return launch_dk_dv<E, 64, 128, MODE>(p, stream);
}

}  // namespace

hipError_t launch_seg_combine(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream);
hipError_t launch_seg_fix(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream);

hipError_t launch_scan_recompute(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream) {
  return bf16_io ? launch_scan<bf16, kScanRec>(p, d_k, d_v, stream) : launch_scan<float, kScanRec>(p, d_k, d_v, stream);
}

hipError_t launch_scan_recompute_kda(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io,
                                     hipStream_t stream) {
  return bf16_io ? launch_scan<bf16, kScanKdaRec>(p, d_k, d_v, stream)
                 : launch_scan<float, kScanKdaRec>(p, d_k, d_v, stream);
}

// Segments for a forward of `heads` heads and `nchunks` chunks on a device with `dev.cus` compute
// units. One segment while the one-pass scan's workgroups (heads x column slices) fill the
// compute units; else enough segments for one workgroup per compute unit over both column kinds,
// at least eight chunks each. (One scan workgroup fills a compute unit's LDS, and the output
// correction grows with the number of segments: on B1 H16 T65536 with two-wave segment
// workgroups, 2 segments measured 1.29 ms, 4 1.32 ms, 8 1.37 ms, against 1.90 ms unsegmented;
// with the four-wave bf16 segment workgroups the plan gives 4 segments in 224 workgroups,
// 0.89 ms against 1.14 ms for 2 two-wave ones.) `forced` > 0 fixes the number of segments
// instead (the caller's explicit plan), clipped to the chunks.
SegPlan seg_plan(int64_t heads, int64_t nchunks, int64_t d_k, int64_t d_v, bool bf16_io, int64_t forced,
                 const DeviceInfo& dev) {
  if (nchunks < 2) return SegPlan{1, nchunks};
  const int64_t cols = scan_cols(bf16_io);
  const int64_t units = (heads + dev.xcds - 1) / dev.xcds * dev.xcds;
  int64_t nseg = 1;
  if (forced > 0) {
    nseg = forced;
  } else if (units * (d_v / cols) < dev.cus && nchunks >= 32) {
    const int64_t scols = scan_cols(bf16_io, true);
    const int64_t per = heads * ((d_v + d_k) / scols);  // workgroups per segment
    nseg = (dev.cus + per - 1) / per;
    if (nseg > nchunks / 8) nseg = nchunks / 8;
  }
  if (nseg < 1) nseg = 1;
  if (nseg > nchunks) nseg = nchunks;
  const int64_t len = (nchunks + nseg - 1) / nseg;
  return SegPlan{(nchunks + len - 1) / len, len};
}

hipError_t launch_chunk_prep_kda(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);

// Bytes of the forward's workspace: the per-chunk factors (scalar gate) or the KDA prep's
// operands, followed by the segment buffers when the plan has more than one segment.
template <typename E>
size_t fwd_space_bytes(int64_t n, int64_t heads, const SegPlan& sp, int d_k, int d_v, bool kda) {
  const size_t head = kda ? KdaSpace<E>::bytes(n, d_k) : Workspace<E>::bytes(n);
  return head + (sp.nseg > 1 ? SegSpace<E>::bytes(n, heads * sp.nseg, d_k, d_v) : 0);
}

size_t chunk_kda_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16_io,
                                     int64_t segments) {
  const int64_t nch = (T + kChunk - 1) / kChunk, n = B * H * nch;
  const SegPlan sp = seg_plan(B * H, nch, d_k, d_v, bf16_io, segments, device_info());
  return bf16_io ? fwd_space_bytes<bf16>(n, B * H, sp, (int)d_k, (int)d_v, true)
                 : fwd_space_bytes<float>(n, B * H, sp, (int)d_k, (int)d_v, true);
}

size_t chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16_io,
                                 int64_t segments) {
  const int64_t nch = (T + kChunk - 1) / kChunk, n = B * H * nch;
  const SegPlan sp = seg_plan(B * H, nch, d_k, d_v, bf16_io, segments, device_info());
  return bf16_io ? fwd_space_bytes<bf16>(n, B * H, sp, (int)d_k, (int)d_v, false)
                 : fwd_space_bytes<float>(n, B * H, sp, (int)d_k, (int)d_v, false);
}

// Launches the scan (one pass, or the segment passes when the plan has several segments) after
// the prep. KDA selects the per-channel decay's scan modes and workspace.
template <bool KDA>
hipError_t launch_scan_plan(ChunkParams& p, const ChunkArgs& a, const SegPlan& sp, hipStream_t stream) {
  constexpr int ONE = KDA ? kScanKda : kScanFwd, SEGM = KDA ? kScanKdaSeg : kScanSeg;
  if (sp.nseg <= 1)
    return a.bf16 ? launch_scan<bf16, ONE>(p, a.d_k, a.d_v, stream) : launch_scan<float, ONE>(p, a.d_k, a.d_v, stream);
  const int64_t n = p.heads * p.nchunks;
  p.nseg = sp.nseg;
  p.seg_len = sp.seg_len;
  p.seg_off = KDA ? (a.bf16 ? KdaSpace<bf16>::bytes(n, (int)a.d_k) : KdaSpace<float>::bytes(n, (int)a.d_k))
                  : (a.bf16 ? Workspace<bf16>::bytes(n) : Workspace<float>::bytes(n));
  hipError_t e = a.bf16 ? launch_scan<bf16, SEGM>(p, a.d_k, a.d_v, stream)
                        : launch_scan<float, SEGM>(p, a.d_k, a.d_v, stream);
  if (e == hipSuccess) e = launch_seg_combine(p, a.d_k, a.d_v, a.bf16, stream);
  if (e == hipSuccess) e = launch_seg_fix(p, a.d_k, a.d_v, a.bf16, stream);
  return e;
}

// KDA forward: the per-channel prep, then the scan in its KDA modes (segmented like the scalar
// gate's when few heads would leave compute units idle).
hipError_t launch_chunk_kda_fwd(const ChunkArgs& a, hipStream_t stream) {
  ChunkParams p{a.q, a.k, a.v, a.eta, a.log_alpha, a.state_in, a.state_out, a.o, a.workspace,
                a.B * a.H, a.H, a.T, (a.T + kChunk - 1) / kChunk, a.eps, a.beta_given, false};
  const DeviceInfo dev = device_info();
  p.xcds = dev.xcds;
  if (p.nchunks > 0) {
    const hipError_t e = launch_chunk_prep_kda(p, a.d_k, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  return launch_scan_plan<true>(p, a, seg_plan(p.heads, p.nchunks, a.d_k, a.d_v, a.bf16, a.segments, dev), stream);
}

// The KDA forward for training (as launch_chunk_fwd_train, with the per-channel decay's prep and
// workspace).
hipError_t launch_chunk_kda_fwd_train(const ChunkArgs& a, hipStream_t stream) {
  const int64_t nchunks = (a.T + kChunk - 1) / kChunk, n = a.B * a.H * nchunks;
  ChunkParams p{a.q, a.k, a.v, a.eta, a.log_alpha, a.state_in, a.state_out, a.o, a.workspace,
                a.B * a.H, a.H, a.T, nchunks, a.eps, a.beta_given, a.beta_given};
  p.xcds = device_info().xcds;
  p.bwd_off = a.bf16 ? KdaSpace<bf16>::bytes(n, (int)a.d_k) : KdaSpace<float>::bytes(n, (int)a.d_k);
  if (nchunks > 0) {
    const hipError_t e = launch_chunk_prep_kda(p, a.d_k, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  return a.bf16 ? launch_scan<bf16, kScanKdaSave>(p, a.d_k, a.d_v, stream)
                : launch_scan<float, kScanKdaSave>(p, a.d_k, a.d_v, stream);
}

// The forward for training: the prep with the backward's factors (beta given: unbalanced, rs =
// 1), then the one-pass scan in its saving mode, into the backward's workspace layout.
hipError_t launch_chunk_fwd_train(const ChunkArgs& a, hipStream_t stream) {
  const int64_t nchunks = (a.T + kChunk - 1) / kChunk, n = a.B * a.H * nchunks;
  ChunkParams p{a.q, a.k, a.v, a.eta, a.log_alpha, a.state_in, a.state_out, a.o, a.workspace,
                a.B * a.H, a.H, a.T, nchunks, a.eps, a.beta_given, a.beta_given};
  p.xcds = device_info().xcds;
  p.bwd_off = a.bf16 ? Workspace<bf16>::bytes(n) : Workspace<float>::bytes(n);
  if (nchunks > 0) {
    const hipError_t e = launch_chunk_prep(p, a.d_k, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  return a.bf16 ? launch_scan<bf16, kScanFwdSave>(p, a.d_k, a.d_v, stream)
                : launch_scan<float, kScanFwdSave>(p, a.d_k, a.d_v, stream);
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream) {
  ChunkParams p{a.q, a.k, a.v, a.eta, a.log_alpha, a.state_in, a.state_out, a.o, a.workspace,
                a.B * a.H, a.H, a.T, (a.T + kChunk - 1) / kChunk, a.eps, a.beta_given, false};
  const DeviceInfo dev = device_info();
  p.xcds = dev.xcds;
  if (p.nchunks > 0) {
    const hipError_t e = launch_chunk_prep(p, a.d_k, a.bf16, stream);
    if (e != hipSuccess) return e;
  }
  return launch_scan_plan<false>(p, a, seg_plan(p.heads, p.nchunks, a.d_k, a.d_v, a.bf16, a.segments, dev), stream);
}

}  // namespace kla
