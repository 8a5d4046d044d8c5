// Chunkwise forward, part 1 of 2: the state-independent work of every chunk, all chunks in
// parallel (one workgroup per chunk of one head).
//
// Sources: "Kaczmarz Linear Attention", Abstract (beta_t = eta_t / (||k_t||^2 + eps));
// "Deep Dive into KDA", section 3 (intra-chunk accumulated decays by prefix sums; the
// intra-chunk part as matrix products; the triangular-masked causal scores) and section 5
// (decay prefixes in the log domain, never dividing by a decayed quantity).
//
// For the chunk's tokens r, s (chunk-local, C = 64), with G the inclusive prefix of log(alpha)
// and rs_r = 1/sqrt(||k_r||^2 + eps):
//   A[r][s] = eta_r rs_r rs_s exp(G_r - G_s) k_r.k_s  (s < r)   -- a diagonal similarity of
//             beta_r exp(G_r - G_s) k_r.k_s that keeps |A| <= eta
//   T       = (I + A)^-1                                          (fp32)
//   P[r][s] = exp(G_r - G_s) q_r.k_s                  (s <= r)
// and the per-token factors the scan needs (see chunk_common.h).
//
// T is found blockwise on 16 x 16 blocks: the four diagonal blocks by forward substitution in
// registers (one wave, a lane per column), then the off-diagonal blocks by block forward
// substitution down each block column on fp32 MFMA, one wave per column:
// T[i][j] = -T[i][i] sum_{j<=k<i} A[i][k] T[k][j]. One barrier separates the two steps.
#include "tile_ops.h"

namespace kla {
namespace {

// Ks is dead once every wave holds its B fragments in registers (a barrier follows their
// loads), so P is staged in the same bytes; once P is stored, T's off-diagonal blocks use them.
// At 35 KiB (bf16, d_k = 128) four workgroups share a CU.
template <typename E, int DK>
struct PrepSmem {
  static constexpr int PAD = 16 / sizeof(E);
  // bf16, d_k = 128: K rows unpadded, their 16-byte chunks XOR-swizzled by row (chunk ^ row % 16)
  // so that the fragment writes and reads (16 rows x 4 chunks per instruction) are free of bank
  // conflicts; otherwise rows padded by 16 bytes.
  static constexpr bool KSW = is_bf16<E>() && DK == 128;
  static constexpr int LDK = KSW ? DK : DK + PAD;
  static constexpr int LDP = kChunk + PAD;
  static constexpr int LDF = kChunk + 4;
  union {
    alignas(16) E Ks[kChunk][LDK];  // K chunk (B operand of K K^T and Q K^T)
    alignas(16) E Ps[kChunk][LDP];
    alignas(16) float Tx[6][16][20];  // T's lower off-diagonal blocks (tx_block)
  };
  alignas(16) float Af[kChunk][LDF];  // A, then T in place
  alignas(16) float sc[kScRows][kChunk];
  float n[kChunk], eta[kChunk], la[kChunk], G[kChunk];
};

// A-operand or B-operand fragments of one 16-row tile over the contraction [0, K).
template <typename E, int K>
struct Frag {
  static constexpr int STEP = is_bf16<E>() ? 32 : 4;
  static constexpr int N = K / STEP;
  typedef typename std::conditional<is_bf16<E>(), bf16x8, float>::type V;
  V v[N];
  __device__ __forceinline__ void load(const E* base, int64_t ld, int lane, bool valid = true) {
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
  // bf16 rows of K 16-byte chunks each, chunk cc of row r stored at cc ^ (r % 16) (16 rows from
  // base, whose row index is a multiple of 16).
  __device__ __forceinline__ void load_swz(const E* base, int lane) {
    static_assert(is_bf16<E>(), "bf16 only");
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = *reinterpret_cast<const bf16x8*>(base + r * K + 8 * ((4 * i + kq) ^ r));
  }
};

template <typename E, int K>
__device__ __forceinline__ void mma_frag(f32x4& acc, const Frag<E, K>& a, const Frag<E, K>& b) {
#pragma unroll
  for (int i = 0; i < Frag<E, K>::N; ++i) {
    if constexpr (is_bf16<E>())
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[i], b.v[i], acc, 0, 0, 0);
    else
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
  }
}

// Make this wave's LDS writes visible to its own later reads (other lanes).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Index of the lower off-diagonal 16 x 16 block (i, j), i > j, of T in sm.Tx.
__device__ __forceinline__ int tx_block(int i, int j) { return i * (i - 1) / 2 + j; }

// acc += A B for 16 x 16 blocks: A row-major in LDS (leading dimension lda), B an accumulator
// tile in registers (lane (g, c) holds rows 4g .. 4g + 3 of column c). Step s contracts index
// 4g + s, so B's registers are the MFMA operands as they are.
__device__ __forceinline__ void mma16_lds_acc(f32x4& acc, const float* A, int lda, const f32x4& b, int lane) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + 4 * kq + s], b[s], acc, 0, 0, 0);
}

// Block column J of T below the diagonal (the diagonal blocks of T and the blocks of A in sm.Af).
template <int J, typename Sm>
__device__ __forceinline__ void t_column(Sm& sm, int lane) {
  constexpr int LDF = Sm::LDF;
  const int lr = lane & 15, lq = lane >> 4;
  f32x4 tk[3];
#pragma unroll
  for (int i = J + 1; i < 4; ++i) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma16_f32s(acc, &sm.Af[16 * i][16 * J], LDF, 1, &sm.Af[16 * J][16 * J], LDF, 1, 0, 16, lane);
#pragma unroll
    for (int k = J + 1; k < i; ++k) mma16_lds_acc(acc, &sm.Af[16 * i][16 * k], LDF, tk[k - J - 1], lane);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    mma16_lds_acc(t, &sm.Af[16 * i][16 * i], LDF, acc, lane);
    t = -t;
    tk[i - J - 1] = t;
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.Tx[tx_block(i, J)][4 * lq + e][lr] = t[e];
  }
}

// Diagonal 16 x 16 blocks of T = (I + A)^-1 by forward substitution, in place of A's in sm.Af
// (wave 0: lane group g takes block g, lane c of it column c).
template <typename Sm>
__device__ __forceinline__ void t_diag(Sm& sm, int lane) {
  const int base = (lane >> 4) * 16, col = lane & 15;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    // sum_{m < i} A[i][m] x[m] as four interleaved partial sums over m < i - 1 plus the last
    // term, so that each row waits on the one before it for a single fma
    const float* arow = &sm.Af[base + i][base];
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m + 1 < i; ++m) ps[m & 3] = fmaf(arow[m], x[m], ps[m & 3]);
    float s = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    if (i > 0) s = fmaf(arow[i - 1], x[i - 1], s);
    x[i] = (i == col) ? 1.f : -s;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) sm.Af[base + i][base + col] = x[i];
}

// Cache policy of the streaming stores: SC1 | NT (system scope, non-temporal). Workspace blocks
// that the scan reads only after the whole prep has written far more than the caches hold go
// out this way.
constexpr int kStreamPolicy = 16 | 2;

// 16 bytes at byte offset off of the block at base (block_bytes long), with the streaming policy.
template <typename V>
__device__ __forceinline__ void store16_stream(void* base, uint32_t block_bytes, uint32_t off, const V& v) {
  static_assert(sizeof(V) == 16, "16-byte vectors");
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), make_rsrc(base, block_bytes), off, 0,
                                         kStreamPolicy);
}

// P (sm.Ps; upper off-diagonal blocks written as zero) and the factor rows (sm.sc) of chunk
// chunk_id to the workspace, by threads t = 0 .. nt - 1 (P with streaming stores if STREAM).
template <typename E, bool STREAM = false, typename Sm>
__device__ __forceinline__ void store_p_sc(const Sm& sm, const Workspace<E>& ws, int64_t chunk_id, int t, int nt) {
  constexpr int VN = Vec16<E>::N;
  typedef typename Vec16<E>::type V16;
  constexpr int VPR = kChunk / VN;
  E* gP = ws.P + chunk_id * kChunk * kChunk;
  for (int i = t; i < kChunk * VPR; i += nt) {
    const int r = i / VPR, c0 = (i % VPR) * VN;
    V16 out = *reinterpret_cast<const V16*>(&sm.Ps[r][c0]);
    if ((c0 >> 4) > (r >> 4)) {  // upper off-diagonal blocks were never computed
#pragma unroll
      for (int e = 0; e < VN; ++e) out[e] = from_f32<E>(0.f);
    }
    if constexpr (STREAM)
      store16_stream(gP, kChunk * kChunk * sizeof(E), (uint32_t)((r * kChunk + c0) * sizeof(E)), out);
    else
      *reinterpret_cast<V16*>(gP + r * kChunk + c0) = out;
  }
  float* gS = ws.SC + chunk_id * kScRows * kChunk;
  for (int i = t; i < kScRows * kChunk; i += nt) gS[i] = (&sm.sc[0][0])[i];
}

// T of chunk chunk_id to the workspace (diagonal blocks from sm.Af, lower off-diagonal ones
// from sm.Tx, upper ones zero), by all NTH threads (with streaming stores if STREAM).
template <typename E, int NTH, bool STREAM = false, typename Sm>
__device__ __forceinline__ void store_t(const Sm& sm, const Workspace<E>& ws, int64_t chunk_id) {
  constexpr int VN = Vec16<E>::N;
  typedef typename Vec16<E>::type V16;
  constexpr int VPR = kChunk / VN;
  E* gT = ws.T + chunk_id * kChunk * kChunk;
  for (int i = threadIdx.x; i < kChunk * VPR; i += NTH) {
    const int r = i / VPR, c0 = (i % VPR) * VN;
    V16 out;
    const int bi = r >> 4, bj = c0 >> 4;
    const bool zero = bj > bi;  // upper off-diagonal block
    const float* src = bj == bi ? &sm.Af[r][c0] : &sm.Tx[zero ? 0 : tx_block(bi, bj)][r & 15][c0 & 15];
#pragma unroll
    for (int e4 = 0; e4 < VN; e4 += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + e4);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e4 + e] = from_f32<E>(zero ? 0.f : x[e]);
    }
    if constexpr (STREAM)
      store16_stream(gT, kChunk * kChunk * sizeof(E), (uint32_t)((r * kChunk + c0) * sizeof(E)), out);
    else
      *reinterpret_cast<V16*>(gT + r * kChunk + c0) = out;
  }
}

// T = (I + A)^-1 (diagonal blocks in place of A in sm.Af, the others in sm.Tx), and the chunk's
// P, T and factor rows to the workspace (P and T with streaming stores if STREAM).
// Called by all threads of the workgroup once A (sm.Af, fp32, zero on and above the diagonal),
// P (sm.Ps) and the factor rows (sm.sc) are in LDS and published by a barrier.
template <typename E, bool STREAM, int NTH = kThreads, typename Sm>
__device__ __forceinline__ void solve_and_store(Sm& sm, const Workspace<E>& ws, int64_t chunk_id) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- diagonal blocks of T (wave 0, as t_diag; written out here: through the helper the
  //      scheduler hoists all of the blocks' LDS reads ahead of the substitution, 92 -> 140 VGPRs
  //      at bf16 d_k = 128) while the other waves store P and the factors ----
  if (wave == 0) {
    const int base = (lane >> 4) * 16, col = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* arow = &sm.Af[base + i][base];
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(arow[m], x[m], s);
      x[i] = (i == col) ? 1.f : -s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.Af[base + i][base + col] = x[i];
  } else {
    store_p_sc<E, STREAM>(sm, ws, chunk_id, tid - kWave, NTH - kWave);
  }
  __syncthreads();

  // ---- off-diagonal blocks, down each block column: wave j forms, for i = j+1 .. 3,
  //      T[i][j] = -T[i][i] (A[i][j] T[j][j] + sum_{j<k<i} A[i][k] T[k][j]),
  //      keeping its T[k][j] in registers as operands; results go to sm.Tx ----
  if (wave == 0) t_column<0>(sm, lane);
  if (wave == 1) t_column<1>(sm, lane);
  if (wave == 2) t_column<2>(sm, lane);
  __syncthreads();

  // ---- T to the workspace (upper off-diagonal blocks are zero) ----
  store_t<E, NTH, STREAM>(sm, ws, chunk_id);
}

// Waves per SIMD that the LDS of one workgroup a chunk lets a CU hold (160 KiB per CU, four SIMDs,
// kThreads / 64 waves per workgroup).
template <typename E, int DK>
constexpr int prep_waves_per_simd() {
  const int wg = (160 * 1024) / (int)sizeof(PrepSmem<E, DK>);
  const int w = wg * (kThreads / kWave) / 4;
  return w < 1 ? 1 : w > 8 ? 8 : w;
}

// STREAM: the launch's T and P blocks are larger than the last-level cache, so they go out with
// streaming stores (the scan reads them only after the whole prep has written far more than the
// caches hold).
template <typename E, int DK, bool STREAM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(prep_waves_per_simd<E, DK>())))
void chunk_prep_kernel(ChunkParams p) {
  constexpr bool BF = is_bf16<E>();
  constexpr int VN = Vec16<E>::N;
  typedef typename Vec16<E>::type V16;
  typedef PrepSmem<E, DK> Sm;
  constexpr int LDF = Sm::LDF;
  __shared__ Sm sm;

  const int64_t chunk_id = blockIdx.x;  // head * nchunks + c
  const int64_t head = chunk_id / p.nchunks, c = chunk_id % p.nchunks;
  const int64_t bb = head / p.H, hh = head % p.H;
  const int64_t T = p.T, t0 = c * kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const E* __restrict__ gk = static_cast<const E*>(p.k);
  const E* __restrict__ gq = static_cast<const E*>(p.q);
  auto row_index = [&](int64_t t) { return (bb * T + t) * p.H + hh; };
  Workspace<E> ws = Workspace<E>::at(p.ws, p.heads * p.nchunks);

  // ---- K rows (waves 0, 1) and Q rows (waves 2, 3) straight into MFMA A fragments: waves 0 and 2
  //      take row tiles {0, 3}, waves 1 and 3 take {1, 2}. The K waves also put K into LDS (the
  //      B operand of both products) and form the squared key norms. ----
  const bool qwave = wave >= 2;
  const int ti0 = (wave & 1) ? 1 : 0, ti1 = (wave & 1) ? 2 : 3;
  const E* gx = (qwave ? gq : gk) + (bb * T * p.H + hh) * DK;  // token t at + t H DK
  Frag<E, DK> a0, a1;
  a0.load(gx + (t0 + 16 * ti0) * p.H * DK, p.H * DK, lane, t0 + 16 * ti0 + lr < T);
  a1.load(gx + (t0 + 16 * ti1) * p.H * DK, p.H * DK, lane, t0 + 16 * ti1 + lr < T);
  if (tid < kChunk) {
    const bool valid = t0 + tid < T;
    sm.eta[tid] = valid ? p.eta[row_index(t0 + tid)] : 0.f;  // eta, or beta when beta_given
    sm.la[tid] = valid && p.log_alpha ? p.log_alpha[row_index(t0 + tid)] : 0.f;
  }
  if (!qwave) {
    const int kq = lane >> 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const Frag<E, DK>& a = half ? a1 : a0;
      const int row = 16 * (half ? ti1 : ti0) + lr;
      float nn = 0.f;
#pragma unroll
      for (int i = 0; i < Frag<E, DK>::N; ++i) {
        if constexpr (BF) {
          const int cc = Sm::KSW ? (4 * i + kq) ^ (row & 15) : 4 * i + kq;
          *reinterpret_cast<bf16x8*>(&sm.Ks[row][8 * cc]) = a.v[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = to_f32(a.v[i][e]);
            nn += x * x;
          }
        } else {
          sm.Ks[row][i * 4 + kq] = a.v[i];
          nn += a.v[i] * a.v[i];
        }
      }
      nn += __shfl_xor(nn, 16, kWave);
      nn += __shfl_xor(nn, 32, kWave);
      if (kq == 0) sm.n[row] = nn;
    }
  }
  __syncthreads();

  // ---- A from K K^T (waves 0, 1) and P from Q K^T (waves 2, 3): the lower 16 x 16 tiles of
  //      this wave's two row tiles (five tiles per wave) ----
  {
    // All products first (one tile of K in registers at a time), then the scaled entries. The
    // products are formed transposed (K's rows as the A operand): lane (c, g) holds entries
    // [16 ti + c][16 tj + 4 g + e], four consecutive columns of one row, written as one vector.
    f32x4 acc[2][4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
      acc[0][tj] = acc[1][tj] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (tj > ti1) continue;
      Frag<E, DK> bk;
      if constexpr (Sm::KSW)
        bk.load_swz(&sm.Ks[tj * 16][0], lane);
      else
        bk.load(&sm.Ks[tj * 16][0], Sm::LDK, lane);
      if (tj <= ti0) mma_frag(acc[0][tj], bk, a0);
      mma_frag(acc[1][tj], bk, a1);
    }
    // ---- per-token factors (wave 0, after its products; the other waves' products overlap) ----
    if (wave == 0) {
      const int r = lane;
      const float G = wave_inclusive_scan(sm.la[r]);
      const float GC = __shfl(G, kChunk - 1, kWave);  // padded rows add log 1 = 0
      // Balanced factors: A[r][s] = eta_r rs_r rs_s e^{G_r - G_s} k_r.k_s is a diagonal similarity of
      // beta_r e^{G_r - G_s} k_r.k_s when beta_r = eta_r rs_r^2. Kaczmarz step: rs = 1/sqrt(|k|^2 + eps).
      // Given beta (gated DeltaNet): rs = sqrt(|beta|), eta = sign(beta); or, for the backward,
      // rs = 1, eta = beta.
      const bool valid = t0 + r < T;
      float rs, et;
      if (p.beta_given && p.unit_rs) {
        rs = valid ? 1.f : 0.f;
        et = sm.eta[r];
      } else if (p.beta_given) {
        const float b = sm.eta[r];
        rs = valid ? sqrtf(fabsf(b)) : 0.f;
        et = b < 0.f ? -1.f : 1.f;
        sm.eta[r] = et;
      } else {
        rs = valid ? 1.f / sqrtf(sm.n[r] + p.eps) : 0.f;
        et = sm.eta[r];
      }
      sm.G[r] = G;
      sm.sc[kScCoefR][r] = et * rs;
      sm.sc[kScEG][r] = __expf(G);
      sm.sc[kScRs][r] = rs;
      sm.sc[kScD2][r] = rs * __expf(GC - G);
    }
    __syncthreads();  // factors in LDS; K no longer read: P may now overwrite it
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ti = half ? ti1 : ti0;
      const int r = ti * 16 + lr;  // this lane's row
      const float Gr = sm.G[r], cr = sm.eta[r] * sm.sc[kScRs][r];
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        if (tj > ti) continue;
        const int s0 = tj * 16 + 4 * lq;  // this lane's first column
        const f32x4 Gs = *reinterpret_cast<const f32x4*>(&sm.G[s0]);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float dec = __expf(Gr - Gs[e]) * acc[half][tj][e];
          x[e] = qwave ? (s0 + e <= r ? dec : 0.f) : (s0 + e < r ? dec : 0.f);
        }
        if (qwave) {
          if constexpr (BF) {
            const bf16x4 b = {from_f32<bf16>(x[0]), from_f32<bf16>(x[1]), from_f32<bf16>(x[2]), from_f32<bf16>(x[3])};
            *reinterpret_cast<bf16x4*>(&sm.Ps[r][s0]) = b;
          } else {
            *reinterpret_cast<f32x4*>(&sm.Ps[r][s0]) = x;
          }
        } else {
          const f32x4 rss = *reinterpret_cast<const f32x4*>(&sm.sc[kScRs][s0]);
          *reinterpret_cast<f32x4*>(&sm.Af[r][s0]) = cr * rss * x;
        }
      }
    }
  }
  __syncthreads();

  solve_and_store<E, STREAM>(sm, ws, chunk_id);
  (void)BF;
}

// ---- KDA: per-channel decay ("Deep Dive into KDA", sections 2.3 and 3) ----
// With G [64][d_k] the chunk-local prefix of log a per channel:
//   A[r][s] = eta_r rs_r rs_s sum_i k_r[i] k_s[i] e^{G_r[i] - G_s[i]}   (s < r)
//   P[r][s] = sum_i q_r[i] k_s[i] e^{G_r[i] - G_s[i]}                   (s <= r)
// Off the diagonal 16 x 16 blocks the sum is one MFMA product of decayed operands referenced to
// the row block's first token b: (k_r o e^{G_r - G_b}) . (k_s o e^{G_b - G_s}), both exponents
// <= 0 since s < b <= r. Inside a diagonal block it is summed per element, each ratio formed as
// one exponential of a non-positive difference, or (bf16) as a running product of the per-token
// decays a_j = e^{G_j - G_{j-1}} <= 1 (no prefix product is ever divided by). The scan's
// operands K o e^G, Q o e^G, K o e^{G_C - G} and gamma = e^{G_C} go to the workspace, and the
// factor rows carry e^G = 1 and rs e^{G_C - G} = rs (the decay lives in the operands).
// Sum over the 16 lanes of a DPP row (lanes with equal lane / 16), in every lane of the row.
__device__ __forceinline__ float dpp_row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

// The KDA prep keeps the prefixes of log a in log2 units, so that every decay factor is one
// hardware exp2 of a difference.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight waves per KDA workgroup: its LDS (about 136 KiB) holds one workgroup per CU, so the
// waves of the one chunk cover all four SIMDs twice.
constexpr int kKdaThreads = 512;
// Largest decay span (log units, per channel) of a 16-token diagonal block that its MFMA path
// takes: its column operands are then at most e^32 (about 8e13) times the keys, far inside
// bf16's range for any key whose squares fit fp32 (which the recurrence itself needs).
constexpr float kKdaSpan = 32.f;

template <typename E, int DK>
struct PrepKdaSmem {
  static constexpr int PAD = 16 / sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDG = DK + 4;
  static constexpr int LDP = kChunk + PAD;
  static constexpr int LDF = kChunk + 4;
  alignas(16) E Ks[kChunk][LDK];
  alignas(16) E Qs[kChunk][LDK];
  alignas(16) float Gm[kChunk][LDG];  // log a, then its chunk-local prefix per channel in log2 units
  // bf16: the row factors e^{G_r - G_b} of the 16 x 16 blocks' MFMA products (b = the row's
  // block start), formed once per chunk (fp32 forms them in the products: its LDS has no room)
  alignas(16) float FR[is_bf16<E>() ? kChunk : 1][LDG];
  float part[kKdaThreads / DK][DK];   // prefix-scan partial totals
  float EB[4][DK];                    // e^{G_b} at the four block starts b
  alignas(16) float Af[kChunk][LDF];  // A, then T in place
  alignas(16) E Ps[kChunk][LDP];
  alignas(16) float Tx[6][16][20];  // T's lower off-diagonal blocks (tx_block)
  alignas(16) float sc[kScRows][kChunk];
  float n[kChunk], eta[kChunk];
  int fast[4];  // diagonal block I within the decay span of its MFMA path (see kKdaSpan)
};

template <typename E, int DK>
__global__ __launch_bounds__(kKdaThreads) void chunk_prep_kda_kernel(ChunkParams p) {
  constexpr int NTH = kKdaThreads, NW = NTH / kWave;
  constexpr bool BF = is_bf16<E>();
  constexpr int VN = Vec16<E>::N;
  typedef typename Vec16<E>::type V16;
  typedef PrepKdaSmem<E, DK> Sm;
  __shared__ Sm sm;

  const int64_t T = p.T, total = p.heads * p.nchunks;
  const Workspace<E> ws = Workspace<E>::at(p.ws, total);
  const KdaSpace<E> kw = KdaSpace<E>::at(p.ws, total, DK);

  // Persistent: workgroup b takes chunks b, b + gridDim.x, ... (chunk id = head * nchunks + c).
  // Its LDS holds one workgroup per CU, so nothing else would hide a chunk's loads: the K, Q and
  // log a rows and eta of the next chunk are loaded into registers (through buffer resources
  // over the batch entry's rows; rows past T read as zero) as soon as the current chunk's are
  // in LDS, and arrive during the rest of its work.
  constexpr int CPR = DK / VN, NKQ = kChunk * CPR / NTH, NL = kChunk * DK / 4 / NTH;
  const int tid0 = threadIdx.x;
  i32x4 kx[NKQ], qx[NKQ], lx[NL];
  float et = 0.f;
  auto load_chunk = [&](int64_t id, int tid_) __attribute__((always_inline)) {
    // (chunk ids and head counts fit 32 bits: the entry points reject larger grids)
    const uint32_t idu = (uint32_t)id, ncu = (uint32_t)p.nchunks, Hu = (uint32_t)p.H;
    const uint32_t head = idu / ncu, bbu = head / Hu;
    const int64_t t0 = (int64_t)(idu - head * ncu) * kChunk;
    const int64_t bb = bbu, hh = head - bbu * Hu, brow = bb * T * p.H;
    const uint32_t xrow = p.H * DK * sizeof(E), lrow = p.H * DK * 4;  // bytes per token
    const rsrc_t rk = make_rsrc(static_cast<const E*>(p.k) + brow * DK, (uint32_t)(T * xrow));
    const rsrc_t rq = make_rsrc(static_cast<const E*>(p.q) + brow * DK, (uint32_t)(T * xrow));
    const rsrc_t rl = make_rsrc(p.log_alpha + brow * DK, (uint32_t)(T * lrow));
#pragma unroll
    for (int j = 0; j < NKQ; ++j) {
      const int i = tid_ + NTH * j, r = i / CPR, c0 = (i % CPR) * VN;
      const uint32_t off = (uint32_t)((t0 + r) * xrow + (hh * DK + c0) * sizeof(E));
      kx[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      qx[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int i = tid_ + NTH * j, r = i / (DK / 4), c4 = (i % (DK / 4)) * 4;
      lx[j] = __builtin_amdgcn_raw_buffer_load_b128(rl, (uint32_t)((t0 + r) * lrow + (hh * DK + c4) * 4), 0, 0);
    }
    et = tid_ < kChunk && t0 + tid_ < T ? p.eta[(bb * T + t0 + tid_) * p.H + hh] : 0.f;
  };
  if ((int64_t)blockIdx.x >= total) return;
  load_chunk(blockIdx.x, tid0);
  int64_t prev_id = -1;  // the previous chunk, whose P, factor rows and T are still in LDS
  for (int64_t chunk_id = blockIdx.x; chunk_id < total; chunk_id += gridDim.x) {
  // Per-thread index arithmetic is redone every chunk rather than kept live across the loop.
  int tid = tid0;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t t0 = (int64_t)((uint32_t)chunk_id % (uint32_t)p.nchunks) * kChunk;

  // ---- K, Q rows, log a and eta of the chunk into LDS, then the next chunk's loads ----
  {
#pragma unroll
    for (int j = 0; j < NKQ; ++j) {
      const int i = tid + NTH * j, r = i / CPR, c0 = (i % CPR) * VN;
      *reinterpret_cast<i32x4*>(&sm.Ks[r][c0]) = kx[j];
      *reinterpret_cast<i32x4*>(&sm.Qs[r][c0]) = qx[j];
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int i = tid + NTH * j, r = i / (DK / 4), c4 = (i % (DK / 4)) * 4;
      *reinterpret_cast<i32x4*>(&sm.Gm[r][c4]) = lx[j];
    }
    if (tid < kChunk) sm.eta[tid] = et;
    if (chunk_id + gridDim.x < total) load_chunk(chunk_id + gridDim.x, tid);
  }
  __syncthreads();
  // ---- the previous chunk's P, factor rows and T to the workspace: stored here, behind the
  //      loads just issued, so that waiting for those loads does not wait for these stores ----
  if (prev_id >= 0) {
    store_p_sc<E, true>(sm, ws, prev_id, tid, NTH);
    store_t<E, NTH, true>(sm, ws, prev_id);
  }

  // ---- per-channel prefix of log a over the chunk's tokens, in log2 units (every exponential
  //      below is one exp2 of a difference of these): NPART threads per channel, each a run of
  //      tokens in registers, then the runs' totals; squared key norms, TPR threads per token ----
  constexpr int NPART = NTH / DK, RUN = kChunk / NPART;
  const int ch = tid % DK, part = tid / DK;
  float run[RUN];
#pragma unroll
  for (int j = 0; j < RUN; ++j) run[j] = sm.Gm[part * RUN + j][ch] * kLog2e;
#pragma unroll
  for (int j = 1; j < RUN; ++j) run[j] += run[j - 1];
  sm.part[part][ch] = run[RUN - 1];
  {
    constexpr int TPR = NTH / kChunk, CPT = DK / TPR;
    static_assert(TPR == 8 && CPT % VN == 0, "eight threads per token");
    const int r = tid / TPR, c0 = (tid % TPR) * CPT;
    float nn = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; i += VN) {
      const V16 x = *reinterpret_cast<const V16*>(&sm.Ks[r][c0 + i]);
#pragma unroll
      for (int e = 0; e < VN; ++e) nn += to_f32(x[e]) * to_f32(x[e]);
    }
    nn += __shfl_xor(nn, 1);
    nn += __shfl_xor(nn, 2);
    nn += __shfl_xor(nn, 4);
    if (tid % TPR == 0) sm.n[r] = nn;
  }
  __syncthreads();
  {
    float off = 0.f;
    for (int j = 0; j < part; ++j) off += sm.part[j][ch];
#pragma unroll
    for (int j = 0; j < RUN; ++j) sm.Gm[part * RUN + j][ch] = run[j] + off;
    if ((part * RUN) % 16 == 0) sm.EB[part * RUN / 16][ch] = exp2_fast(run[0] + off);
  }

  // ---- factors (wave 0): as for the scalar gate, with e^G = 1 and rs e^{G_C - G} = rs ----
  if (wave == 0) {
    const int r = lane;
    const bool valid = t0 + r < T;
    float rs, et;
    if (p.beta_given && p.unit_rs) {
      rs = valid ? 1.f : 0.f;
      et = sm.eta[r];
    } else if (p.beta_given) {
      const float b = sm.eta[r];
      rs = valid ? sqrtf(fabsf(b)) : 0.f;
      et = b < 0.f ? -1.f : 1.f;
      sm.eta[r] = et;
    } else {
      rs = valid ? 1.f / sqrtf(sm.n[r] + p.eps) : 0.f;
      et = sm.eta[r];
    }
    sm.sc[kScCoefR][r] = et * rs;
    sm.sc[kScEG][r] = 1.f;
    sm.sc[kScRs][r] = rs;
    sm.sc[kScD2][r] = rs;
  }
  __syncthreads();

  // ---- decayed scan operands (streaming stores) and gamma to the workspace; (bf16) the row
  //      factors ----
  {
    constexpr int CPR = DK / VN;
    E* k1 = kw.K1 + chunk_id * kChunk * DK;
    E* q1 = kw.Q1 + chunk_id * kChunk * DK;
    E* k2 = kw.K2 + chunk_id * kChunk * DK;
    for (int i = tid; i < kChunk * CPR; i += NTH) {
      const int r = i / CPR, c0 = (i % CPR) * VN, b = r & ~15;
      const V16 kx = *reinterpret_cast<const V16*>(&sm.Ks[r][c0]);
      const V16 qx = *reinterpret_cast<const V16*>(&sm.Qs[r][c0]);
      V16 a, bq, d;
      float fr[VN];
#pragma unroll
      for (int e4 = 0; e4 < VN; e4 += 4) {
        const f32x4 G = *reinterpret_cast<const f32x4*>(&sm.Gm[r][c0 + e4]);
        const f32x4 GC = *reinterpret_cast<const f32x4*>(&sm.Gm[kChunk - 1][c0 + e4]);
        const f32x4 Gb = *reinterpret_cast<const f32x4*>(&sm.Gm[b][c0 + e4]);
        const f32x4 eb = *reinterpret_cast<const f32x4*>(&sm.EB[b >> 4][c0 + e4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // e^G = e^{G - G_b} e^{G_b}, both factors <= 1
          fr[e4 + e] = exp2_fast(G[e] - Gb[e]);
          const float eg = fr[e4 + e] * eb[e], ed = exp2_fast(GC[e] - G[e]);
          a[e4 + e] = from_f32<E>(to_f32(kx[e4 + e]) * eg);
          bq[e4 + e] = from_f32<E>(to_f32(qx[e4 + e]) * eg);
          d[e4 + e] = from_f32<E>(to_f32(kx[e4 + e]) * ed);
        }
      }
      const uint32_t off = (uint32_t)((r * DK + c0) * sizeof(E)), blk = kChunk * DK * sizeof(E);
      store16_stream(k1, blk, off, a);
      store16_stream(q1, blk, off, bq);
      store16_stream(k2, blk, off, d);
      if constexpr (BF) {
#pragma unroll
        for (int e4 = 0; e4 < VN; e4 += 4)
          *reinterpret_cast<f32x4*>(&sm.FR[r][c0 + e4]) = f32x4{fr[e4], fr[e4 + 1], fr[e4 + 2], fr[e4 + 3]};
      }
    }
    if (tid < DK) kw.gamma[chunk_id * DK + tid] = exp2_fast(sm.Gm[kChunk - 1][tid]);
  }
  // Waves 4..7: whether diagonal block I = wave - 4 decays by at most kKdaSpan (log units) over
  // its 16 tokens on every channel.
  if (wave >= 4 && wave < 8) {
    const int b = 16 * (wave - 4);
    bool ok = true;
    for (int ch = lane; ch < DK; ch += kWave) ok = ok && sm.Gm[b][ch] - sm.Gm[b + 15][ch] <= kKdaSpan * kLog2e;
    const bool all = __all(ok);
    if (lane == 0) sm.fast[wave - 4] = all;
  }
  __syncthreads();

  // ---- 16 x 16 blocks (I, J), J <= I, as MFMA products of operands decayed to b = 16 I: the
  //      six off the diagonal (row factors e^{G_r - G_b} <= 1, column factors e^{G_b - G_s} <= 1),
  //      and the four diagonal ones whose decay span is bounded (column factors then in
  //      [1, e^kKdaSpan]; in bf16 both operands are split into high and low parts, so that these
  //      blocks, which dominate A and P, keep fp32-level accuracy). The other diagonal blocks are
  //      walked below. ----
  // Block (I, J) over channel steps [i0, i1) (32 channels a step in bf16, 4 in fp32) into kk
  // (K K^T) and qk (Q K^T), accumulated.
  constexpr int NI = BF ? DK / 32 : DK / 4;
  auto block = [&](auto diag_c, int I, int J, int i0, int i1, f32x4& kk, f32x4& qk) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const int b = 16 * I;
    const int ra = 16 * I + lr, rb = 16 * J + lr;  // this lane's A row and B row
    if constexpr (BF) {
#pragma unroll
      for (int i = i0; i < i1; ++i) {
        const int c = 32 * i + 8 * lq;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sm.Ks[ra][c]);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&sm.Qs[ra][c]);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&sm.Ks[rb][c]);
        bf16x8 ak, aq, bk, akl, aql, bkl;
#pragma unroll
        for (int h = 0; h < 8; h += 4) {
          const f32x4 fa = *reinterpret_cast<const f32x4*>(&sm.FR[ra][c + h]);
          const f32x4 gb = *reinterpret_cast<const f32x4*>(&sm.Gm[b][c + h]);
          const f32x4 gs = *reinterpret_cast<const f32x4*>(&sm.Gm[rb][c + h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float fb = exp2_fast(gb[e] - gs[e]);
            const float xa = to_f32(ka[h + e]) * fa[e], xq = to_f32(qa[h + e]) * fa[e];
            const float xb = to_f32(kb[h + e]) * fb;
            ak[h + e] = from_f32<bf16>(xa);
            aq[h + e] = from_f32<bf16>(xq);
            bk[h + e] = from_f32<bf16>(xb);
            if constexpr (DIAG) {
              akl[h + e] = from_f32<bf16>(xa - to_f32(ak[h + e]));
              aql[h + e] = from_f32<bf16>(xq - to_f32(aq[h + e]));
              bkl[h + e] = from_f32<bf16>(xb - to_f32(bk[h + e]));
            }
          }
        }
        kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bk, kk, 0, 0, 0);
        qk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, qk, 0, 0, 0);
        if constexpr (DIAG) {
          kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(akl, bk, kk, 0, 0, 0);
          kk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bkl, kk, 0, 0, 0);
          qk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aql, bk, qk, 0, 0, 0);
          qk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bkl, qk, 0, 0, 0);
        }
      }
    } else {
#pragma unroll 4
      for (int i = i0; i < i1; ++i) {
        const int ch = 4 * i + lq;
        const float Gb = sm.Gm[b][ch];
        const float fa = exp2_fast(sm.Gm[ra][ch] - Gb), fb = exp2_fast(Gb - sm.Gm[rb][ch]);
        const float bk = sm.Ks[rb][ch] * fb;
        kk = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.Ks[ra][ch] * fa, bk, kk, 0, 0, 0);
        qk = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.Qs[ra][ch] * fa, bk, qk, 0, 0, 0);
      }
    }
  };
  // A and P of block (I, J) from its products.
  auto block_out = [&](int I, int J, const f32x4& kk, const f32x4& qk) __attribute__((always_inline)) {
    const int s = 16 * J + lr;
    const float rss = sm.sc[kScRs][s];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * I + 4 * lq + e;
      sm.Af[r][s] = s < r ? sm.eta[r] * sm.sc[kScRs][r] * rss * kk[e] : 0.f;
      sm.Ps[r][s] = from_f32<E>(s <= r ? qk[e] : 0.f);
    }
  };
  auto off_ij = [](int t, int& I, int& J) __attribute__((always_inline)) {
    I = t >= 3 ? 3 : t >= 1 ? 2 : 1;
    J = t - (I * (I - 1)) / 2;
  };
  // Waves 0..3 take diagonal block I = wave; waves 4..7 off-diagonal block t = wave - 4 and one
  // half of the channels of block 4 + (t & 1) (waves 4, 5 the first, 6, 7 the second), so that
  // each SIMD (waves w and w + 4) carries one diagonal block and one and a half off-diagonal
  // ones. Off-diagonal block t is (I, J) = (1,0), (2,0), (2,1), (3,0), (3,1), (3,2). The second
  // halves go through sm.Tx (free until T's blocks are formed) and are added by waves 4, 5 after
  // the barrier below.
  f32x4 hk = {0.f, 0.f, 0.f, 0.f}, hq = hk;
  if (wave < 4) {
    if (sm.fast[wave]) {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
      block(std::true_type{}, wave, wave, 0, NI, kk, qk);
      block_out(wave, wave, kk, qk);
    }
  } else if (wave < 8) {
    const int t = wave - 4;
    int I, J;
    off_ij(t, I, J);
    {
      f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
      block(std::false_type{}, I, J, 0, NI, kk, qk);
      block_out(I, J, kk, qk);
    }
    off_ij(4 + (t & 1), I, J);
    const int h = t >> 1;
    block(std::false_type{}, I, J, h * (NI / 2), (h + 1) * (NI / 2), hk, hq);
    if (h == 1) {
      float* part2 = &sm.Tx[0][0][0] + (t & 1) * 8 * kWave;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part2[e * kWave + lane] = hk[e];
        part2[(4 + e) * kWave + lane] = hq[e];
      }
    }
  }
  // ---- diagonal 16 x 16 blocks ----
  if constexpr (BF) {
    // Thread (block, row pair, channel slice): the rows r2 = 15 - pair and then r1 = pair of a
    // diagonal block, each summed against s = r, r - 1, .., 0 while the ratio
    // w = prod_{j = s+1..r} a_j is carried down by one multiply per channel (w *= a_s). Every row
    // pair takes 17 steps, so no lane idles on the upper triangle; the 16 channel slices of a row
    // share a DPP row and are summed there. Everything a step reads from LDS (the K row, the
    // decays, the column's factor) is read a step ahead, and the rows' factors before the walk,
    // so that no step waits on LDS.
    constexpr int CS = DK / 16;  // channels per slice: 8 or 4
    typedef typename std::conditional<CS == 8, bf16x8, bf16x4>::type KV;
    const int sl = tid & 15, pair = (tid >> 4) & 7, hb = tid >> 7, c0 = CS * sl;
    static_assert(NTH % 128 == 0 && NTH <= 512, "blocks of eight row pairs of sixteen slices");
    for (int I = hb; I < 4; I += NTH / 128) {
      if (sm.fast[I]) continue;
      const int b = 16 * I, r2 = 15 - pair;
      // the rows' factors eta_R rs_R
      const float f2 = sm.eta[b + r2] * sm.sc[kScRs][b + r2], f1 = sm.eta[b + pair] * sm.sc[kScRs][b + pair];
      int r = r2, s = r;
      float fr = f2;
      float kr[CS], qr[CS], w[CS], ad[CS];
      auto row_start = [&]() __attribute__((always_inline)) {
        const KV kx = *reinterpret_cast<const KV*>(&sm.Ks[b + r][c0]);
        const KV qx = *reinterpret_cast<const KV*>(&sm.Qs[b + r][c0]);
#pragma unroll
        for (int c = 0; c < CS; ++c) {
          kr[c] = to_f32(kx[c]);
          qr[c] = to_f32(qx[c]);
          w[c] = 1.f;
        }
      };
      // a_sr = e^{G_sr - G_{sr-1}} (unused for sr = 0, where it reads as 1)
      auto read_ad = [&](int sr, float* dst) __attribute__((always_inline)) {
        const int sp = sr > 0 ? sr - 1 : 0;
#pragma unroll
        for (int c = 0; c < CS; c += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.Gm[b + sr][c0 + c]);
          const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.Gm[b + sp][c0 + c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[c + e] = exp2_fast(x[e] - y[e]);
        }
      };
      row_start();
      KV ks = *reinterpret_cast<const KV*>(&sm.Ks[b + s][c0]);
      float rsc = sm.sc[kScRs][b + s];
      read_ad(s, ad);
      for (int it = 0; it < 17; ++it) {
        // next step's row and column (the pair's second row after s = 0), read early
        const bool sw = s == 0;
        const int s_n = sw ? pair : s - 1;
        const KV ks_n = *reinterpret_cast<const KV*>(&sm.Ks[b + s_n][c0]);
        const float rsc_n = sm.sc[kScRs][b + s_n];
        float ad_n[CS];
        read_ad(s_n, ad_n);
        float a = 0.f, pq = 0.f;
#pragma unroll
        for (int c = 0; c < CS; ++c) {
          const float x = to_f32(ks[c]) * w[c];
          a += kr[c] * x;
          pq += qr[c] * x;
        }
        a = dpp_row16_sum(a);
        pq = dpp_row16_sum(pq);
        if (sl == 0) {
          const int R = b + r, Sc = b + s;
          sm.Af[R][Sc] = s < r ? fr * rsc * a : 0.f;
          sm.Ps[R][Sc] = from_f32<E>(pq);
        }
        if (sw) {  // the row pair's second row
          r = pair;
          fr = f1;
          row_start();
        } else {  // w for s - 1: times a_s
#pragma unroll
          for (int c = 0; c < CS; ++c) w[c] *= ad[c];
        }
        s = s_n;
        ks = ks_n;
        rsc = rsc_n;
#pragma unroll
        for (int c = 0; c < CS; ++c) ad[c] = ad_n[c];
      }
    }
    // the upper triangles of the walked diagonal blocks
    for (int i = tid; i < 4 * 256; i += NTH) {
      const int b = 16 * (i >> 8), rr = (i >> 4) & 15, ss = i & 15;
      if (ss > rr && !sm.fast[i >> 8]) {
        sm.Af[b + rr][b + ss] = 0.f;
        sm.Ps[b + rr][b + ss] = from_f32<E>(0.f);
      }
    }
  } else {  // one thread per (r, s), summed per channel
    const int rr = (tid >> 4) & 15, ss = tid & 15;
    static_assert(NTH % 256 == 0, "whole blocks of 16 x 16 threads");
    for (int I = tid >> 8; I < 4; I += NTH / 256) {
      if (sm.fast[I]) continue;
      const int r = 16 * I + rr, s = 16 * I + ss;
      float a = 0.f, pq = 0.f;
      if (s <= r) {
        for (int i = 0; i < DK; i += 4) {
          const f32x4 Gr = *reinterpret_cast<const f32x4*>(&sm.Gm[r][i]);
          const f32x4 Gs = *reinterpret_cast<const f32x4*>(&sm.Gm[s][i]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w = exp2_fast(Gr[e] - Gs[e]) * to_f32(sm.Ks[s][i + e]);
            a += to_f32(sm.Ks[r][i + e]) * w;
            pq += to_f32(sm.Qs[r][i + e]) * w;
          }
        }
      }
      sm.Af[r][s] = s < r ? sm.eta[r] * sm.sc[kScRs][r] * sm.sc[kScRs][s] * a : 0.f;
      sm.Ps[r][s] = from_f32<E>(s <= r ? pq : 0.f);
    }
  }
  __syncthreads();
  // the split blocks: second halves (from waves 6, 7) added to the first (waves 4, 5)
  if (wave == 4 || wave == 5) {
    const float* part2 = &sm.Tx[0][0][0] + (wave - 4) * 8 * kWave;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hk[e] += part2[e * kWave + lane];
      hq[e] += part2[(4 + e) * kWave + lane];
    }
    int I, J;
    off_ij(wave, I, J);
    block_out(I, J, hk, hq);
  }

  // ---- T = (I + A)^-1 in LDS: diagonal blocks (wave 0), then the blocks below them (waves
  //      0..2, as in solve_and_store). The other waves go on to the next chunk's rows, which
  //      t_column does not read; its results are read after the next chunk's first barrier. ----
  if (wave == 0) t_diag(sm, lane);
  __syncthreads();
  if (wave == 0) t_column<0>(sm, lane);
  if (wave == 1) t_column<1>(sm, lane);
  if (wave == 2) t_column<2>(sm, lane);
  prev_id = chunk_id;
  }  // chunk loop
  __syncthreads();
  if (prev_id >= 0) {
    store_p_sc<E, true>(sm, ws, prev_id, threadIdx.x, NTH);
    store_t<E, NTH, true>(sm, ws, prev_id);
  }
}

// Workgroups of a kernel resident at once per compute unit (the same on every gfx950 device).
template <typename K>
int64_t blocks_per_cu(K kernel, int threads) {
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess || per <= 0) return 1;
  return per;
}

template <typename E>
hipError_t launch_kda_e(const ChunkParams& p, int64_t d_k, hipStream_t stream) {
  const int64_t total = p.heads * p.nchunks, cus = device_info().cus;
  if (d_k == 128) {
    static const int64_t per = blocks_per_cu(chunk_prep_kda_kernel<E, 128>, kKdaThreads);
    const int64_t res = cus * per;
    hipLaunchKernelGGL((chunk_prep_kda_kernel<E, 128>), dim3((unsigned)(total < res ? total : res)), dim3(kKdaThreads), 0,
                       stream, p);
  } else {
    static const int64_t per = blocks_per_cu(chunk_prep_kda_kernel<E, 64>, kKdaThreads);
    const int64_t res = cus * per;
    hipLaunchKernelGGL((chunk_prep_kda_kernel<E, 64>), dim3((unsigned)(total < res ? total : res)), dim3(kKdaThreads), 0,
                       stream, p);
  }
  return hipGetLastError();
}

// T and P of a launch (two C x C blocks of E per chunk) from this many bytes on are stored with
// streaming stores: the MI355X's last-level cache holds 256 MB. Measured (bf16, d = 128): the
// B4 H16 T32768 prefill forward (512 MB of T and P) 1.13 -> 1.11 ms; B8 H8 T4096 (64 MB) and its
// backward are 1-2 % slower with them.
constexpr int64_t kStreamPrepBytes = int64_t(256) << 20;

template <typename E, int DK>
void launch_dk(const ChunkParams& p, int64_t grid, hipStream_t stream) {
  const bool stream_tp = grid * 2 * kChunk * kChunk * (int64_t)sizeof(E) >= kStreamPrepBytes;
  if (stream_tp)
    hipLaunchKernelGGL((chunk_prep_kernel<E, DK, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<E, DK, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
}

template <typename E>
hipError_t launch_e(const ChunkParams& p, int64_t d_k, hipStream_t stream) {
  const int64_t grid = p.heads * p.nchunks;
  if (d_k == 128)
    launch_dk<E, 128>(p, grid, stream);
  else
    launch_dk<E, 64>(p, grid, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prep(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream) {
  return bf16_io ? launch_e<bf16>(p, d_k, stream) : launch_e<float>(p, d_k, stream);
}

hipError_t launch_chunk_prep_kda(const ChunkParams& p, int64_t d_k, bool bf16_io, hipStream_t stream) {
  return bf16_io ? launch_kda_e<bf16>(p, d_k, stream) : launch_kda_e<float>(p, d_k, stream);
}

}  // namespace kla
