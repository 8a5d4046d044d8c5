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
constexpr int kXcds = 8;       // MI355X: workgroups are dealt round-robin to 8 XCDs

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
  static size_t bytes(int64_t nchunks_total) {
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
};

}  // namespace kla
