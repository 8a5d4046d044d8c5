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
// One workgroup of 8 waves owns one d_v slice (DVS columns) of one head and walks its chunks
// in order. Waves 0-3 ("K waves") own token rows 16h of K, X and R, and S rows
// [h DK/4, (h+1) DK/4); waves 4-7 ("Q waves") own token rows 16h of Q, Y and O. Every wave
// computes one 16 x 16 tile of D. The slice of S stays in fp32 MFMA accumulators of the K
// waves for the whole sequence; a bf16 copy of S^T in LDS is the B operand of K S and Q S.
// A operands that belong to one wave's rows (K, Q, T, P) come from global memory straight
// into MFMA fragment registers, one to two chunks ahead; K is also kept in LDS (double-buffered) so
// that the K waves can read K^T fragments with the transposing LDS read of gfx950. The
// slices of one head get workgroup ids congruent mod 8, so they run on one XCD and share its
// L2 for K, Q, T and P. Three workgroup barriers per chunk.
#include "chunk_common.h"

namespace kla {

hipError_t launch_chunk_prep(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream);

namespace {

constexpr int kScanWaves = 8;
constexpr int kScanThreads = kScanWaves * kWave;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resources: a load whose byte offset is at or past `bytes` returns zeros and such a
// store is dropped, so rows past T need no branches (and no branch breaks the compiler's
// counting of outstanding loads).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Make this wave's LDS writes visible to its own later reads (other lanes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename E>
__device__ __forceinline__ typename Vec16<E>::type load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(typename Vec16<E>::type, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename E>
__device__ __forceinline__ E load1(rsrc_t r, uint32_t off) {
  if constexpr (is_bf16<E>())
    return __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  else
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <typename E>
__device__ __forceinline__ void store1(E x, rsrc_t r, uint32_t off) {
  if constexpr (is_bf16<E>())
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, x), r, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, off, 0, 0);
}

template <typename E, int DK, int DVS>
struct ScanSmem {
  static constexpr int PAD = 16 / sizeof(E);
  // Ks/STs rows: a 32-byte row skew, so the four rows a 16-lane group reads with the
  // transposing LDS read fall in disjoint bank ranges.
  static constexpr int LDK = DK + 2 * PAD;
  static constexpr int LDC = kChunk + PAD;  // RTs, DTs, DTs2 rows
  alignas(16) E Ks[2][kChunk][LDK];         // K of chunks n (buffer n & 1)
  alignas(16) E STs[DVS][LDK];              // S^T slice (bf16 operand copy of the state)
  alignas(16) E RTs[DVS][LDC];              // R^T
  alignas(16) E DTs[DVS][LDC];              // D'^T
  alignas(16) E DTs2[DVS][LDC];             // (diag(e^{G_C - G}) D')^T
  alignas(16) E Xs[8][16][DVS + PAD];       // per wave: its V tile (K waves) or O tile (Q waves)
};

// Per-lane MFMA fragments of 16 rows over a contraction of K elements.
template <typename E, int K>
struct Frag {
  static constexpr int STEP = is_bf16<E>() ? 32 : 4;
  static constexpr int N = K / STEP;
  typedef typename std::conditional<is_bf16<E>(), bf16x8, float>::type V;
  V v[N];
  // Row r = lane % 16 of the tile lies at byte offset off0 + r * ld_bytes of the resource.
  __device__ __forceinline__ void load(rsrc_t rs, uint32_t off0, uint32_t ld_bytes, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const uint32_t off = off0 + r * ld_bytes;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (is_bf16<E>())
        v[i] = load16<E>(rs, off + (i * 32 + 8 * kq) * sizeof(E));
      else
        v[i] = load1<E>(rs, off + (i * 4 + kq) * sizeof(E));
    }
  }
};

template <typename E, int K>
__device__ __forceinline__ void mma_frag(f32x4& acc, const Frag<E, K>& a, const E* B, int ldb, int nsteps,
                                         int lane) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int i = 0; i < Frag<E, K>::N; ++i) {
    if (i < nsteps) {
      if constexpr (is_bf16<E>()) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(B + r * ldb + i * 32 + 8 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[i], b, acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], B[r * ldb + i * 4 + kq], acc, 0, 0, 0);
      }
    }
  }
}

// acc += K^T[m0 .. m0+16) [tokens 0..64) * B^T, with K row-major in LDS (Ks[token][d]) and B
// stored [16 cols][ldb] token-contiguous. bf16: the A fragments come from two transposing
// LDS reads (ds_read_b64_tr_b16) per 32-token step.
template <typename E, int LDK>
__device__ __forceinline__ void mma_kt(f32x4& acc, const E* Ks, int m0, const E* B, int ldb, int lane) {
  const int r = lane & 15, kq = lane >> 4;
  if constexpr (is_bf16<E>()) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // lane (kq, r) supplies row 32s + 8kq + (r >> 2) (+4), columns m0 + 4 (r & 3) .. +3; it receives
      // K[32s + 8kq + j][m0 + r] for j = 0..3 (and 4..7).
      const E* p0 = Ks + (32 * s + 8 * kq + (r >> 2)) * LDK + m0 + 4 * (r & 3);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * LDK));
      const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 a = __builtin_bit_cast(bf16x8, both);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(B + r * ldb + 32 * s + 8 * kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k0 = 0; k0 < kChunk; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[(k0 + kq) * LDK + m0 + r], B[r * ldb + k0 + kq], acc, 0, 0, 0);
  }
}

template <typename E, int DK, int DV, int DVS>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(ChunkParams p) {
  constexpr int NS = DV / DVS;   // d_v slices per head
  constexpr int TJ = DVS / 16;   // 16-column tiles per slice
  constexpr int RT = DK / 64;    // 16-row tiles of S per K wave
  typedef ScanSmem<E, DK, DVS> Sm;
  constexpr int LDK = Sm::LDK, LDC = Sm::LDC;
  constexpr int STEP = is_bf16<E>() ? 32 : 4;
  __shared__ Sm sm;

  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int64_t head = (int64_t)(local / NS) * kXcds + xcd;
  const int slice = local % NS;
  if (head >= p.heads) return;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, nchunks = p.nchunks, H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool kwave = wave < 4;
  const int h = wave & 3;  // token-row tile of this wave
  const int lr = lane & 15, lq = lane >> 4;
  const int j0 = slice * DVS;
  // Tile of D = T R this wave computes: row tile h, column tile dtj (all waves when TJ = 2).
  const int dtj = wave >> 2;
  const bool dwave = dtj < TJ;
  const int kend = is_bf16<E>() ? (h < 2 ? 32 : 64) : 16 * (h + 1);  // T, P row block h: zero past 16(h+1)
  const int tsteps = kend / STEP;
  // A wave's 16 x DVS tile of V or O moves as 16-byte pieces: LPR lanes per row, RPL rows per
  // instruction, VPL instructions.
  constexpr int VN = Vec16<E>::N, LPR = DVS / VN, RPL = kWave / LPR, VPL = 16 / RPL;
  const int prow = lane / LPR, pcol = (lane % LPR) * VN;

  // Resources over this batch's rows of q/k, v and o, and over this head's workspace chunks.
  // Byte offsets fit in 32 bits (checked on the host). The K waves store O, and load P, through
  // resources of size 0 (and the Q waves load V so), so both wave roles issue the same memory
  // operations while only the role that needs the data moves it.
  const int64_t brow = bb * T * H;  // first (token, head) row of this batch
  const uint32_t xrow = H * DK * sizeof(E), vrow = H * DV * sizeof(E);  // bytes per token
  const rsrc_t rx = make_rsrc(static_cast<const E*>(kwave ? p.k : p.q) + brow * DK, (uint32_t)(T * xrow));
  const rsrc_t rv = make_rsrc(static_cast<const E*>(p.v) + brow * DV, kwave ? (uint32_t)(T * vrow) : 0u);
  const rsrc_t ro = make_rsrc(static_cast<const E*>(p.o) + brow * DV, kwave ? 0u : (uint32_t)(T * vrow));
  const Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * nchunks);
  const int64_t chunk0 = head * nchunks;
  constexpr uint32_t kMatBytes = kChunk * kChunk * sizeof(E), kScBytes = kScRows * kChunk * sizeof(float);
  const rsrc_t rt = make_rsrc(ws.T + chunk0 * kChunk * kChunk, (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rp = make_rsrc(ws.P + chunk0 * kChunk * kChunk, kwave ? 0u : (uint32_t)(nchunks * kMatBytes));
  const rsrc_t rsc = make_rsrc(ws.SC + chunk0 * kScRows * kChunk, (uint32_t)(nchunks * kScBytes));
  const uint32_t hcol_x = hh * DK * sizeof(E), hcol_v = (hh * DV + j0) * sizeof(E);  // head's column offset

  // ---- prefetched inputs (per wave: its own rows) ----
  // InX (K or Q fragments, V, per-token factors) is used up by the D phase of its chunk and is
  // refilled with chunk c+2 right after; two sets alternate. InT (T, P, e^{G_C}) is refilled
  // with chunk c+1 right after each part's last use. Loads thus stay in flight for one to two
  // chunks.
  struct InX {
    Frag<E, DK> x;      // K rows (K waves) or Q rows (Q waves) 16h .. 16h + 15
    typename Vec16<E>::type vv[VPL];  // V rows 16h.. of the slice, row-major pieces (K waves)
    f32x4 sc[kScRows];  // per-token factors of rows 16h + 4lq .. +3
  };
  struct InT {
    Frag<E, 64> t;      // T rows 16h (first tsteps steps)
    Frag<E, 64> pm;     // P rows 16h (Q waves)
    float eGC;
  };
  // Fetches never branch: chunk indices past the end are clamped to the last chunk (the data
  // is then unused) and rows past T read as zeros.
  auto fetch_x = [&](InX& in, int64_t c) {
    c = c < nchunks ? c : nchunks - 1;
    const uint32_t t0 = (uint32_t)(c * kChunk);
    in.x.load(rx, (t0 + 16 * h) * xrow + hcol_x, xrow, lane);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      in.vv[i] = load16<E>(rv, (t0 + 16 * h + i * RPL + prow) * vrow + hcol_v + pcol * sizeof(E));
    const uint32_t so = (uint32_t)c * kScBytes + (16 * h + 4 * lq) * sizeof(float);
#pragma unroll
    for (int q = 0; q < kScRows; ++q) in.sc[q] = load16<float>(rsc, so + q * kChunk * sizeof(float));
  };
  auto fetch_rows = [&](Frag<E, 64>& f, rsrc_t rs, int64_t c) {  // rows 16h of a [64][64] matrix
    c = c < nchunks ? c : nchunks - 1;
    f.load(rs, (uint32_t)c * kMatBytes + 16 * h * kChunk * sizeof(E), kChunk * sizeof(E), lane);
  };
  auto fetch_t = [&](InT& in, int64_t c) { fetch_rows(in.t, rt, c); };
  auto fetch_p = [&](InT& in, int64_t c) {
    fetch_rows(in.pm, rp, c);
    const int64_t cc = c < nchunks ? c : nchunks - 1;
    in.eGC = load1<float>(rsc, (uint32_t)cc * kScBytes + (kScEG * kChunk + kChunk - 1) * sizeof(float));
  };

  // ---- state slice -> accumulators of the K waves (rows h DK/4 + 16 rt + ...) ----
  f32x4 accS[RT][TJ];
  if (kwave) {
    const float* Sin = p.state_in ? p.state_in + head * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        const int row0 = h * (DK / 4) + rt * 16 + 4 * lq;
        const int col = j0 + tj * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) accS[rt][tj][e] = Sin ? Sin[(int64_t)(row0 + e) * DV + col] : 0.f;
        store4<E>(&sm.STs[tj * 16 + lr][row0], accS[rt][tj][0], accS[rt][tj][1], accS[rt][tj][2],
                  accS[rt][tj][3]);
      }
  }
  __syncthreads();

  InX x0, x1;
  InT ct;
  if (nchunks > 0) {
    fetch_x(x0, 0);
    fetch_t(ct, 0);
    fetch_p(ct, 0);
    fetch_x(x1, 1);
  }

  auto step = [&](int64_t c, InX& cx) {
    const int buf = c & 1;
    const int64_t t0 = c * kChunk;

    // ---- K waves: K rows -> LDS (for K^T later), X = K S -> R^T.  Q waves: Y = e^G (Q S) ----
    f32x4 acc[TJ];
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) {
      acc[tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
      mma_frag(acc[tj], cx.x, &sm.STs[tj * 16][0], LDK, Frag<E, DK>::N, lane);
    }
    if (kwave) {
      const int r = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int i = 0; i < Frag<E, DK>::N; ++i) {
        if constexpr (is_bf16<E>())
          *reinterpret_cast<bf16x8*>(&sm.Ks[buf][16 * h + r][i * 32 + 8 * kq]) = cx.x.v[i];
        else
          sm.Ks[buf][16 * h + r][i * 4 + kq] = cx.x.v[i];
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        *reinterpret_cast<typename Vec16<E>::type*>(&sm.Xs[wave][i * RPL + prow][pcol]) = cx.vv[i];
      wave_lds_sync();
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        float R[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          R[e] = cx.sc[kScCoefR][e] * (to_f32(sm.Xs[wave][4 * lq + e][16 * tj + lr]) - cx.sc[kScEG][e] * acc[tj][e]);
        store4<E>(&sm.RTs[tj * 16 + lr][16 * h + 4 * lq], R[0], R[1], R[2], R[3]);
      }
    } else {
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tj][e] *= cx.sc[kScEG][e];
    }
    __syncthreads();

    // ---- D = T R, tile (h, dtj);  D' = rs D -> DTs;  e^{G_C - G} D' -> DTs2 ----
    if (dwave) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      mma_frag(d, ct.t, &sm.RTs[dtj * 16][0], LDC, tsteps, lane);
      float d1[4], d2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d1[e] = cx.sc[kScRs][e] * d[e];
        d2[e] = cx.sc[kScD2][e] * d[e];
      }
      store4<E>(&sm.DTs[dtj * 16 + lr][16 * h + 4 * lq], d1[0], d1[1], d1[2], d1[3]);
      store4<E>(&sm.DTs2[dtj * 16 + lr][16 * h + 4 * lq], d2[0], d2[1], d2[2], d2[3]);
    }
    fetch_x(cx, c + 2);
    fetch_t(ct, c + 1);
    __syncthreads();

    if (kwave) {
      // ---- S <- e^{G_C} S + K^T DTs2 -> STs ----
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tj = 0; tj < TJ; ++tj) {
          const int row0 = h * (DK / 4) + rt * 16;
          accS[rt][tj] *= ct.eGC;
          mma_kt<E, LDK>(accS[rt][tj], &sm.Ks[buf][0][0], row0, &sm.DTs2[tj * 16][0], LDC, lane);
          store4<E>(&sm.STs[tj * 16 + lr][row0 + 4 * lq], accS[rt][tj][0], accS[rt][tj][1], accS[rt][tj][2],
                    accS[rt][tj][3]);
        }
    } else {
      // ---- O = Y + P D' ----
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) mma_frag(acc[tj], ct.pm, &sm.DTs[tj * 16][0], LDC, tsteps, lane);
    }
    // O -> global by both roles (the K waves' resource has size 0: their stores are dropped),
    // transposed to row-major 16-byte pieces through this wave's LDS slot.
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Xs[wave][4 * lq + e][16 * tj + lr] = from_f32<E>(acc[tj][e]);
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(i32x4, *reinterpret_cast<const typename Vec16<E>::type*>(&sm.Xs[wave][i * RPL + prow][pcol])),
          ro, (uint32_t)(t0 + 16 * h + i * RPL + prow) * vrow + hcol_v + pcol * sizeof(E), 0, 0);
    fetch_p(ct, c + 1);
    __syncthreads();
  };
  for (int64_t c = 0; c < nchunks; c += 2) {
    step(c, x0);
    if (c + 1 < nchunks) step(c + 1, x1);
  }

  if (p.state_out && kwave) {
    float* Sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        const int row0 = h * (DK / 4) + rt * 16 + 4 * lq;
        const int col = j0 + tj * 16 + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sout[(int64_t)(row0 + e) * DV + col] = accS[rt][tj][e];
      }
  }
}

template <typename E, int DK, int DV>
hipError_t launch_dk_dv(const ChunkParams& p, hipStream_t stream) {
  constexpr int DVS = 32;
  constexpr int NS = DV / DVS;
  const int64_t heads8 = (p.heads + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((chunk_scan_kernel<E, DK, DV, DVS>), dim3((unsigned)(heads8 * NS)), dim3(kScanThreads), 0,
                     stream, p);
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
