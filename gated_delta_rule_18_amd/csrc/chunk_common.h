// Pieces shared by the two kernels of the chunkwise forward (chunk_prep.hip, chunk_scan.hip):
// MFMA tile products over LDS operands and the workspace layout that connects the kernels.
#pragma once

#include <type_traits>

#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

template <typename E>
constexpr bool is_bf16() { return std::is_same<E, bf16>::value; }

constexpr int kThreads = 256;  // 4 waves per workgroup

// acc += A[16 x k] * B[k x 16] over k in [0, kend), A stored row-major [16][lda] and B stored
// as its transpose [16][ldb] (both K-contiguous, in LDS). bf16: v_mfma_f32_16x16x32_bf16
// (kend a multiple of 32); fp32: v_mfma_f32_16x16x4_f32 (kend a multiple of 4).
template <typename E>
__device__ __forceinline__ void mma16(f32x4& acc, const E* A, int lda, const E* B, int ldb, int kend, int lane) {
  const int r = lane & 15, kq = lane >> 4;
  if constexpr (is_bf16<E>()) {
    for (int k0 = 0; k0 < kend; k0 += 32) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + k0 + 8 * kq);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(B + r * ldb + k0 + 8 * kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  } else {
    for (int k0 = 0; k0 < kend; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kq], B[r * ldb + k0 + kq], acc, 0, 0, 0);
  }
}

// fp32 product with arbitrary strides: acc += A(m, k) B(k, n) for k in [k0, k1), where
// A(m, k) = A[m*sam + k*sak] and B(k, n) = B[k*sbk + n*sbn]; k0, k1 multiples of 4.
__device__ __forceinline__ void mma16_f32s(f32x4& acc, const float* A, int sam, int sak, const float* B, int sbk,
                                           int sbn, int k0, int k1, int lane) {
  const int r = lane & 15, kq = lane >> 4;
  for (int k = k0; k < k1; k += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * sam + (k + kq) * sak], B[(k + kq) * sbk + r * sbn], acc, 0, 0,
                                               0);
}

// Four consecutive elements (the four accumulator rows of one lane) to LDS.
template <typename E>
__device__ __forceinline__ void store4(E* dst, float a, float b, float c, float d) {
  if constexpr (is_bf16<E>()) {
    bf16x4 v = {from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c), from_f32<bf16>(d)};
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4*>(dst) = v;
  }
}

// Workspace written by the prep kernel and read by the scan kernel, per chunk
// (chunk id = head * nchunks + c, so one head's chunks are contiguous):
//   T  [64][64] of E : T = (I + A)^-1 for the scaled A (see chunk_prep.hip)
//   P  [64][64] of E : P[r][s] = exp(G_r - G_s) q_r.k_s for s <= r, else 0
//   SC [4][64] fp32  : per token r: eta_r rs_r, e^{G_r}, rs_r, rs_r e^{G_C - G_r}
// where G is the chunk-local inclusive log-decay prefix and rs_r = 1/sqrt(||k_r||^2 + eps)
// (0 on padded rows). e^{G_C} is SC[1][63] (padded rows add log 1 = 0).
enum { kScCoefR = 0, kScEG = 1, kScRs = 2, kScD2 = 3, kScRows = 4 };

template <typename E>
struct Workspace {
  E* T;
  E* P;
  float* SC;
  __host__ __device__ static size_t bytes(int64_t nchunks_total) {
    return (size_t)nchunks_total * (2 * kChunk * kChunk * sizeof(E) + kScRows * kChunk * sizeof(float));
  }
  __host__ __device__ static Workspace at(void* base, int64_t nchunks_total) {
    char* p = static_cast<char*>(base);
    Workspace w;
    w.T = reinterpret_cast<E*>(p);
    w.P = reinterpret_cast<E*>(p + (size_t)nchunks_total * kChunk * kChunk * sizeof(E));
    w.SC = reinterpret_cast<float*>(p + (size_t)nchunks_total * 2 * kChunk * kChunk * sizeof(E));
    return w;
  }
};

// Modes of the scan kernel: the forward; the backward's recompute (entering states and Delta
// to the backward workspace, no outputs); the first pass of the segment scan (below); the
// forward with the per-channel decay (KDA); the first segment pass with that decay; and the
// backward's recompute with that decay.
enum {
  kScanFwd = 0, kScanRec = 1, kScanSeg = 2, kScanKda = 3, kScanKdaSeg = 4, kScanKdaRec = 5, kScanFwdSave = 6,
  kScanKdaSave = 7
};
__host__ __device__ constexpr bool scan_kda(int mode) {
  return mode == kScanKda || mode == kScanKdaSeg || mode == kScanKdaRec || mode == kScanKdaSave;
}
__host__ __device__ constexpr bool scan_rec(int mode) { return mode == kScanRec || mode == kScanKdaRec; }
__host__ __device__ constexpr bool scan_seg(int mode) { return mode == kScanSeg || mode == kScanKdaSeg; }
// kScanFwdSave, kScanKdaSave: the forward for training, which also stores what the backward's
// recompute would.
__host__ __device__ constexpr bool scan_save(int mode) { return mode == kScanFwdSave || mode == kScanKdaSave; }

// State columns per scan workgroup (bf16: two waves of 16 columns; fp32: four). The bf16
// segment scan uses four waves (64 columns): with half the workgroups per segment, twice the
// segments fit the compute units.
__host__ __device__ constexpr int scan_cols(bool bf16, bool seg = false) { return bf16 && !seg ? 32 : 64; }

// Segment scan of the forward, for few heads and long sequences (where one workgroup per head
// and column slice leaves most compute units idle). The chunks of a head are cut into nseg
// segments of seg_len chunks that are scanned at the same time:
//   pass 1  every segment from a zero entering state (the first from S_0), giving its outputs
//           O0 (written to o) and end state; after the first segment also the d_k "identity"
//           columns (state I, no values), giving the segment's state transition M and, per
//           chunk, Y = (e^G o Q) M_n - P W M_n, the response of the chunk's output to the
//           entering state;
//   pass 2  S_1 = end state of segment 0, S_{j+1} = M_j S_j + (end state of segment j);
//   pass 3  o += Y S_j on every chunk after the first segment.
// Every step is the same linear algebra as the one-pass scan (the state recursion is linear
// in the entering state).
struct SegPlan {
  int64_t nseg, seg_len;
};

// The segment buffers follow the forward's workspace (ChunkParams::seg_off bytes into it: the
// scalar gate's Workspace, or with the per-channel decay the KdaSpace below).
template <typename E>
struct SegSpace {
  E* Y;         // [n][64][DK]: outputs of the identity columns
  float* Send;  // [heads * nseg][DK][DV]: end state of each segment from its own entering state
  float* Mseg;  // [heads * nseg][DK][DK]: state transition of each segment
  E* SinT;      // [heads * nseg][DV][DK]: entering state of each segment, transposed (pass 2)
  __host__ __device__ static size_t bytes(int64_t n, int64_t nsegs, int dk, int dv) {
    return (size_t)n * kChunk * dk * sizeof(E) + (size_t)nsegs * ((dk * dv + dk * dk) * sizeof(float) + dk * dv * sizeof(E));
  }
  __host__ __device__ static SegSpace at(void* base, size_t off, int64_t n, int64_t nsegs, int dk, int dv) {
    char* p = static_cast<char*>(base) + off;
    SegSpace w;
    w.Y = reinterpret_cast<E*>(p);
    p += (size_t)n * kChunk * dk * sizeof(E);
    w.Send = reinterpret_cast<float*>(p);
    w.Mseg = w.Send + (size_t)nsegs * dk * dv;
    w.SinT = reinterpret_cast<E*>(w.Mseg + (size_t)nsegs * dk * dk);
    return w;
  }
};

// KDA (per-channel decay) workspace: the forward workspace above, then per chunk the decayed
// operands of the scan, in the input dtype, rows of d_k:
//   K1 [64][DK] = K o e^G,  Q1 [64][DK] = Q o e^G,  K2 [64][DK] = K o e^{G_C - G}
// and the chunk's state decay gamma [DK] = e^{G_C} (fp32), where G [64][DK] is the chunk-local
// inclusive prefix of log a per channel. Every exponent is <= 0.
template <typename E>
struct KdaSpace {
  E* K1;
  E* Q1;
  E* K2;
  float* gamma;
  __host__ __device__ static size_t bytes(int64_t n, int dk) {
    return Workspace<E>::bytes(n) + (size_t)n * dk * (3 * kChunk * sizeof(E) + sizeof(float));
  }
  __host__ __device__ static KdaSpace at(void* base, int64_t n, int dk) {
    E* p = reinterpret_cast<E*>(static_cast<char*>(base) + Workspace<E>::bytes(n));
    KdaSpace w;
    w.K1 = p;
    w.Q1 = w.K1 + (size_t)n * kChunk * dk;
    w.K2 = w.Q1 + (size_t)n * kChunk * dk;
    w.gamma = reinterpret_cast<float*>(w.K2 + (size_t)n * kChunk * dk);
    return w;
  }
};

struct ChunkParams {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* log_alpha;
  const float* state_in;
  float* state_out;
  void* o;
  void* ws;
  int64_t heads, H, T, nchunks;
  float eps;
  bool beta_given;  // eta holds beta itself (gated DeltaNet); log_alpha may then be null (alpha = 1)
  // With beta_given: factor beta as eta_r = beta_r, rs_r = 1 (no balancing) instead of
  // eta_r = sign(beta_r), rs_r = sqrt(|beta_r|). The backward needs the unbalanced factors to
  // form d(beta) on tokens whose beta is zero.
  bool unit_rs;
  int64_t nseg = 1, seg_len = 0;  // segment scan (kScanSeg): segments per head, chunks per segment
  size_t seg_off = 0;             // bytes of the workspace ahead of the segment buffers (SegSpace)
  size_t bwd_off = 0;             // bytes of the workspace ahead of the backward buffers (BwdSpace)
  int xcds = 1;  // XCDs of the device: the scan launches keep the workgroups of one head on one XCD
};

// Backward workspace: the forward workspace above (the scalar gate's Workspace, or with the
// per-channel decay the KdaSpace), then, bwd_off bytes into it, per chunk (same chunk ids)
//   Sn  [DK x DV] of E : the state entering the chunk
//   dSn [DK x DV] of E : the gradient of the state leaving the chunk
//   Dl  [64 x DV] of E : Delta = U - W S of the chunk (the page's new-value term)
//   Zb  [64 x DV] of E : diag(rs) (I + A)^-T dDelta, the gradient of the solve's right side
// each in MFMA accumulator order: 16 x 16 tiles (row tile major, then column tile), 64 lanes
// per tile, four consecutive rows of one column per lane (lane = 16 g + c holds rows
// 4g .. 4g + 3 of column c). Producers store whole tiles with one coalesced store per lane.
template <typename E>
struct BwdSpace {
  E* Sn;
  E* dSn;
  E* Dl;
  E* Zb;
  __host__ __device__ static size_t bytes(int64_t n, int dk, int dv) {
    return (size_t)n * (2 * dk * dv + 2 * kChunk * dv) * sizeof(E);
  }
  __host__ __device__ static BwdSpace at(void* base, size_t off, int64_t n, int dk, int dv) {
    E* p = reinterpret_cast<E*>(static_cast<char*>(base) + off);
    BwdSpace w;
    w.Sn = p;
    w.dSn = w.Sn + (size_t)n * dk * dv;
    w.Dl = w.dSn + (size_t)n * dk * dv;
    w.Zb = w.Dl + (size_t)n * kChunk * dv;
    return w;
  }
};

// Offset (elements) of tile (rt, ct) lane `lane` in a tile-ordered block with NCT column tiles.
__host__ __device__ constexpr int tile_off(int rt, int ct, int nct, int lane) { return ((rt * nct + ct) * 64 + lane) * 4; }

struct ChunkBwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* log_alpha;
  const float* state_in;    // may be null
  const void* dout;         // dL/do
  const float* dstate_out;  // dL/dS_T, may be null
  void* dq;
  void* dk;
  void* dv;
  float* deta;        // dL/deta, or dL/dbeta when beta_given
  float* dlog_alpha;  // may be null when log_alpha is
  float* dstate_in;   // dL/dS_0, may be null
  void* ws;
  int64_t heads, H, T, nchunks;
  float eps;
  bool beta_given;
  int xcds = 1;        // as ChunkParams::xcds
  size_t bwd_off = 0;  // as ChunkParams::bwd_off
};

}  // namespace kla
