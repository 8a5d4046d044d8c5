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
// into MFMA fragment registers, one chunk ahead; K is also kept in LDS (double-buffered) so
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

template <typename E, int DK, int DVS>
struct ScanSmem {
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int LDK = DK + PAD;      // Ks, STs rows
  static constexpr int LDC = kChunk + PAD;  // RTs, DTs, DTs2 rows
  alignas(16) E Ks[2][kChunk][LDK];         // K of chunks n (buffer n & 1)
  alignas(16) E STs[DVS][LDK];              // S^T slice (bf16 operand copy of the state)
  alignas(16) E RTs[DVS][LDC];              // R^T
  alignas(16) E DTs[DVS][LDC];              // D'^T
  alignas(16) E DTs2[DVS][LDC];             // (diag(e^{G_C - G}) D')^T
};

// Per-lane MFMA fragments of 16 rows over a contraction of K elements.
template <typename E, int K>
struct Frag {
  static constexpr int STEP = is_bf16<E>() ? 32 : 4;
  static constexpr int N = K / STEP;
  typedef typename std::conditional<is_bf16<E>(), bf16x8, float>::type V;
  V v[N];
  // rows base[r * ld + ...], r = lane % 16; valid = whether this lane's row exists
  __device__ __forceinline__ void load(const E* base, int64_t ld, bool valid, int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (is_bf16<E>()) {
        if (valid) {
          v[i] = *reinterpret_cast<const bf16x8*>(base + r * ld + i * 32 + 8 * kq);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[i][e] = from_f32<bf16>(0.f);
        }
      } else {
        v[i] = valid ? base[r * ld + i * 4 + kq] : 0.f;
      }
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool kwave = wave < 4;
  const int h = wave & 3;  // token-row tile of this wave
  const int lr = lane & 15, lq = lane >> 4;
  const int j0 = slice * DVS;
  // Tile of D = T R this wave computes: row tile h, column tile dtj (all waves when TJ = 2).
  const int dtj = wave >> 2;
  const bool dwave = dtj < TJ;
  const int kend = is_bf16<E>() ? (h < 2 ? 32 : 64) : 16 * (h + 1);  // T, P row block h: zero past 16(h+1)
  const int tsteps = kend / STEP;

  const E* gx = static_cast<const E*>(kwave ? p.k : p.q) + (bb * T * H + hh) * DK;  // token t at + t H DK
  const E* gv = static_cast<const E*>(p.v) + (bb * T * H + hh) * DV + j0;
  E* go = static_cast<E*>(p.o) + (bb * T * H + hh) * DV + j0;
  const Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * nchunks);
  const int64_t chunk0 = head * nchunks;

  // ---- prefetched inputs of one chunk (per wave: its own rows) ----
  struct In {
    Frag<E, DK> x;      // K rows (K waves) or Q rows (Q waves) 16h .. 16h + 15
    Frag<E, 64> t;      // T rows 16h (first tsteps steps)
    Frag<E, 64> pm;     // P rows 16h (Q waves)
    E v[TJ][4];         // V[16h + 4lq + e][16 tj + lr] (K waves)
    f32x4 sc[kScRows];  // per-token factors of rows 16h + 4lq .. +3
    float eGC;
  };
  auto fetch = [&](In& in, int64_t c) {
    const int64_t t0 = c * kChunk;
    // Frag::load adds this lane's row (lane % 16) to the tile's first row t0 + 16h.
    in.x.load(gx + (t0 + 16 * h) * H * DK, H * DK, t0 + 16 * h + lr < T, lane);
    const E* gT = ws.T + (chunk0 + c) * kChunk * kChunk + 16 * h * kChunk;
    const E* gP = ws.P + (chunk0 + c) * kChunk * kChunk + 16 * h * kChunk;
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < Frag<E, 64>::N; ++i) {
      if (i < tsteps) {
        if constexpr (is_bf16<E>()) {
          in.t.v[i] = *reinterpret_cast<const bf16x8*>(gT + r * kChunk + i * 32 + 8 * kq);
          if (!kwave) in.pm.v[i] = *reinterpret_cast<const bf16x8*>(gP + r * kChunk + i * 32 + 8 * kq);
        } else {
          in.t.v[i] = gT[r * kChunk + i * 4 + kq];
          if (!kwave) in.pm.v[i] = gP[r * kChunk + i * 4 + kq];
        }
      }
    }
    if (kwave) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = t0 + 16 * h + 4 * lq + e;
#pragma unroll
        for (int tj = 0; tj < TJ; ++tj) in.v[tj][e] = t < T ? gv[t * H * DV + 16 * tj + lr] : from_f32<E>(0.f);
      }
    }
    const float* gs = ws.SC + (chunk0 + c) * kScRows * kChunk + 16 * h + 4 * lq;
#pragma unroll
    for (int q = 0; q < kScRows; ++q) in.sc[q] = *reinterpret_cast<const f32x4*>(gs + q * kChunk);
    in.eGC = ws.SC[(chunk0 + c) * kScRows * kChunk + kScEG * kChunk + kChunk - 1];
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

  In cur, nxt;
  if (nchunks > 0) fetch(nxt, 0);

  for (int64_t c = 0; c < nchunks; ++c) {
    cur = nxt;
    if (c + 1 < nchunks) fetch(nxt, c + 1);
    const int buf = c & 1;
    const int64_t t0 = c * kChunk;

    // ---- K waves: K rows -> LDS (for K^T later), X = K S -> R^T.  Q waves: Y = e^G (Q S) ----
    f32x4 acc[TJ];
#pragma unroll
    for (int tj = 0; tj < TJ; ++tj) {
      acc[tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
      mma_frag(acc[tj], cur.x, &sm.STs[tj * 16][0], LDK, Frag<E, DK>::N, lane);
    }
    if (kwave) {
      const int r = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int i = 0; i < Frag<E, DK>::N; ++i) {
        if constexpr (is_bf16<E>())
          *reinterpret_cast<bf16x8*>(&sm.Ks[buf][16 * h + r][i * 32 + 8 * kq]) = cur.x.v[i];
        else
          sm.Ks[buf][16 * h + r][i * 4 + kq] = cur.x.v[i];
      }
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        float R[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          R[e] = cur.sc[kScCoefR][e] * (to_f32(cur.v[tj][e]) - cur.sc[kScEG][e] * acc[tj][e]);
        store4<E>(&sm.RTs[tj * 16 + lr][16 * h + 4 * lq], R[0], R[1], R[2], R[3]);
      }
    } else {
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tj][e] *= cur.sc[kScEG][e];
    }
    __syncthreads();

    // ---- D = T R, tile (h, dtj);  D' = rs D -> DTs;  e^{G_C - G} D' -> DTs2 ----
    if (dwave) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      mma_frag(d, cur.t, &sm.RTs[dtj * 16][0], LDC, tsteps, lane);
      float d1[4], d2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d1[e] = cur.sc[kScRs][e] * d[e];
        d2[e] = cur.sc[kScD2][e] * d[e];
      }
      store4<E>(&sm.DTs[dtj * 16 + lr][16 * h + 4 * lq], d1[0], d1[1], d1[2], d1[3]);
      store4<E>(&sm.DTs2[dtj * 16 + lr][16 * h + 4 * lq], d2[0], d2[1], d2[2], d2[3]);
    }
    __syncthreads();

    if (kwave) {
      // ---- S <- e^{G_C} S + K^T DTs2 -> STs ----
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tj = 0; tj < TJ; ++tj) {
          const int row0 = h * (DK / 4) + rt * 16;
          accS[rt][tj] *= cur.eGC;
          mma_kt<E, LDK>(accS[rt][tj], &sm.Ks[buf][0][0], row0, &sm.DTs2[tj * 16][0], LDC, lane);
          store4<E>(&sm.STs[tj * 16 + lr][row0 + 4 * lq], accS[rt][tj][0], accS[rt][tj][1], accS[rt][tj][2],
                    accS[rt][tj][3]);
        }
    } else {
      // ---- O = Y + P D' -> global ----
#pragma unroll
      for (int tj = 0; tj < TJ; ++tj) {
        mma_frag(acc[tj], cur.pm, &sm.DTs[tj * 16][0], LDC, tsteps, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = t0 + 16 * h + 4 * lq + e;
          if (t < T) go[t * H * DV + 16 * tj + lr] = from_f32<E>(acc[tj][e]);
        }
      }
    }
    __syncthreads();
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
