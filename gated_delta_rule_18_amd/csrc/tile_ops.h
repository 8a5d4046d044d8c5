// MFMA tile operands over LDS and buffer-resource memory access, shared by the scan kernels
// (forward and reverse) and the chunk-parallel gradient kernel.
//
// Contraction groups. The contraction index of every product is enumerated in the order in
// which an MFMA accumulator holds its rows, so that the accumulators of one product are,
// register for register, an operand of the next. In a 16 x 16 accumulator tile, lane (g, c)
// (g = lane / 16, c = lane % 16) holds rows 4g .. 4g + 3 of column c. A "group" of the
// contraction is 32 indices for v_mfma_f32_16x16x32_bf16 (one instruction: lane group g feeds
// indices 32s + 4g + 0..3 from tile 2s and 32s + 16 + 4g + 0..3 from tile 2s + 1) and 16
// indices for v_mfma_f32_16x16x4_f32 (four instructions: instruction i feeds index 16s + 4g + i
// from tile s). A and B fragments of these MFMAs have the same lane layout, so an accumulator
// block serves as B (contracting its rows) or, for a transposed product, as A.
//
// LDS matrices are row-major without padding, their 16-byte chunks XOR-swizzled by row (swz)
// so that row reads, transposing reads and direct-to-LDS loads are free of bank conflicts.
#pragma once

#include "chunk_common.h"

namespace kla {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(rsrc_t r, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, 0, 0, 0);
}

// Wait until at most M of the vector memory operations this wave issued are outstanding, the
// direct-to-LDS loads included (s_waitcnt vmcnt(M); expcnt and lgkmcnt left at their maxima;
// these operations complete in issue order). Placed before each barrier that publishes such
// loads: the compiler's own wait placement does not cover LDS written by them on every path.
template <int M>
__device__ __forceinline__ void wait_vmem() {
  static_assert(M >= 0 && M < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((M & 15) | ((M >> 4) << 14) | 0x0F70);
}

// ---- contraction groups ----------------------------------------------------------------------
template <typename E>
struct Grp {
  static constexpr int K = is_bf16<E>() ? 32 : 16;  // contraction indices per group
  typedef typename std::conditional<is_bf16<E>(), bf16x8, f32x4>::type V;
};

template <typename E>
__device__ __forceinline__ f32x4 mma(typename Grp<E>::V a, typename Grp<E>::V b, f32x4 c) {
  if constexpr (is_bf16<E>()) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
}

template <typename E>
__device__ __forceinline__ typename Grp<E>::V acc_grp(const f32x4* tiles, int s) {
  if constexpr (is_bf16<E>()) {
    const f32x4 a = tiles[2 * s], b = tiles[2 * s + 1];
    bf16x8 v = {from_f32<bf16>(a[0]), from_f32<bf16>(a[1]), from_f32<bf16>(a[2]), from_f32<bf16>(a[3]),
                from_f32<bf16>(b[0]), from_f32<bf16>(b[1]), from_f32<bf16>(b[2]), from_f32<bf16>(b[3])};
    return v;
  } else {
    return tiles[s];
  }
}

// Layouts of an operand matrix in LDS (its rows' 16-byte chunks XOR-swizzled by row):
//   kLaySplit  fragments along a row read as two 8-byte halves (see Grp);
//   kLayTok    bf16 whole-chunk layout for matrices whose fragments are read along the rows
//              tok_row(r, 0..15) of a token tile (K, T) or transposed (K for the state update, V);
//   kLayLin    bf16 whole-chunk layout for matrices read along 16 consecutive rows (Q, P).
// Each swizzle keeps that matrix's reads free of bank conflicts (measured with the LDS
// bank-conflict counter on every access pattern of the scan), and depends on as few row bits
// as that allows, so that reads of different tiles differ by constant offsets.
enum { kLaySplit = 0, kLayTok = 1, kLayLin = 2 };

// Physical 16-byte chunk of logical chunk cc in row r of a matrix with CPR chunks per row.
template <typename E, int CPR, int LAY = kLaySplit>
__device__ __forceinline__ int swz(int r, int cc) {
  if constexpr (LAY != kLaySplit) {
    static_assert(is_bf16<E>(), "whole-chunk layouts are bf16 only");
    static_assert(CPR == 16 || CPR == 8 || CPR == 4, "bf16 row width");
    const int r0 = r & 1, r1 = (r >> 1) & 1, r3 = (r >> 3) & 1, r4 = (r >> 4) & 1;
    if constexpr (LAY == kLayLin)
      return CPR == 16 ? cc ^ (r & 15) : CPR == 8 ? cc ^ ((r >> 1) & 7) : cc ^ (r3 << 1);
    else if constexpr (CPR == 16)
      return cc ^ (r0 | (r4 << 1) | (r1 << 2) | (r3 << 3));
    else if constexpr (CPR == 8)
      return cc ^ (r1 | (r3 << 1) | (r4 << 2));
    else
      return cc ^ (r3 << 1);
  } else if constexpr (is_bf16<E>()) {
    static_assert(CPR == 16 || CPR == 8 || CPR == 4, "bf16 row width");
    if constexpr (CPR == 16) return cc ^ (((r & 7) << 1) | ((r >> 3) & 1));
    if constexpr (CPR == 8) return cc ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
    return cc ^ (((r >> 2) & 1) << 1);
  } else {
    static_assert(CPR >= 16, "fp32 row width");
    return cc ^ (r & 15);
  }
}

// Element offset of (r, col) in a swizzled row-major matrix of NCOL columns.
template <typename E, int NCOL, int LAY = kLaySplit>
__device__ __forceinline__ int at(int r, int col) {
  constexpr int PER = 16 / sizeof(E), CPR = NCOL / PER;
  return r * NCOL + PER * swz<E, CPR, LAY>(r, col / PER) + col % PER;
}

// ---- whole-chunk layout (bf16) ---------------------------------------------------------------
// Contraction group s of v_mfma_f32_16x16x32_bf16 feeds lane group g the 8 consecutive indices
// 32 s + 8 g + 0..7, so a fragment along a row is one 16-byte LDS read. The accumulator tiles
// that serve as the other operand hold, per lane group g, four consecutive indices each:
//   token tiles (products over the chunk's tokens), tile r, row m:
//     tok(r, m) = 32 (r / 2) + 8 (m / 4) + 4 (r % 2) + m % 4
//   state tiles (products over d_k), tile r, row m = 4 g + e:
//     krow(r, g, e) = 32 (r / 2) + 8 g + 4 ((g % 2) ^ (r % 2)) + e
// The state tiles alternate their halves with g, so that the transposing reads of K for the
// state update touch both 8-byte halves of the 16-byte chunks (no bank conflicts).
__device__ __forceinline__ int tok_row(int r, int m) { return 32 * (r >> 1) + 8 * (m >> 2) + 4 * (r & 1) + (m & 3); }
__device__ __forceinline__ int k_row(int r, int g, int e) {
  return 32 * (r >> 1) + 8 * g + 4 * ((g & 1) ^ (r & 1)) + e;
}

// A or B operand of group s along row `row`: one 16-byte read.
template <int NCOL, int LAY>
__device__ __forceinline__ bf16x8 row8_grp(const bf16* M, int row, int s, int g) {
  return *reinterpret_cast<const bf16x8*>(M + at<bf16, NCOL, LAY>(row, 32 * s + 8 * g));
}

// Operand of group s from state tiles 2s and 2s + 1 (the lane's indices 32 s + 8 g + 0..7, in
// order: the tile holding the lower four depends on g).
__device__ __forceinline__ bf16x8 state_grp(const f32x4* tiles, int s, int g) {
  const f32x4 a = tiles[2 * s], b = tiles[2 * s + 1];
  const bf16x4 ca = {from_f32<bf16>(a[0]), from_f32<bf16>(a[1]), from_f32<bf16>(a[2]), from_f32<bf16>(a[3])};
  const bf16x4 cb = {from_f32<bf16>(b[0]), from_f32<bf16>(b[1]), from_f32<bf16>(b[2]), from_f32<bf16>(b[3])};
  const bool swap = g & 1;
  const bf16x4 lo = swap ? cb : ca, hi = swap ? ca : cb;
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand of group s of K^T for state tile rt: A(m, k) = K[k][krow(rt, m / 4, m % 4)],
// k = tokens 32 s + 8 g + 0..7 (two transposing reads of four tokens each).
template <int DK>
__device__ __forceinline__ bf16x8 kt8_grp(const bf16* Ks, int rt, int s, int g, int c) {
  const int j = c & 3, r0 = 32 * s + 8 * g + (c >> 2);
  const int col = 32 * (rt >> 1) + 8 * j + 4 * ((j & 1) ^ (rt & 1));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ks + at<bf16, DK, kLayTok>(r0, col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ks + at<bf16, DK, kLayTok>(r0 + 4, col)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of group s along row `row` (k = column index).
template <typename E, int NCOL>
__device__ __forceinline__ typename Grp<E>::V row_grp(const E* M, int row, int s, int g) {
  if constexpr (is_bf16<E>()) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(M + at<E, NCOL>(row, 32 * s + 4 * g));
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(M + at<E, NCOL>(row, 32 * s + 16 + 4 * g));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return *reinterpret_cast<const f32x4*>(M + at<E, NCOL>(row, 16 * s + 4 * g));
  }
}

// A operand of group s of K^T for state row tile rt: A(m, k) = K[k][16 rt + m], k = token.
template <typename E, int DK>
__device__ __forceinline__ typename Grp<E>::V kt_grp(const E* Ks, int rt, int s, int g, int c) {
  if constexpr (is_bf16<E>()) {
    const int r0 = 32 * s + 4 * g + (c >> 2), col = 16 * rt + 4 * (c & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ks + at<E, DK>(r0, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Ks + at<E, DK>(r0 + 16, col)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  } else {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = Ks[at<E, DK>(16 * s + 4 * g + i, 16 * rt + c)];
    return v;
  }
}

// Rows r0 + GS g + 0..3 of column col0 + c, as fp32 (GS = 4; 8 in the token-tile layout).
template <typename E, int NCOL, int LAY = kLaySplit>
__device__ __forceinline__ f32x4 col4(const E* M, int r0, int col0, int g, int c) {
  constexpr int GS = LAY == kLayTok ? 8 : 4;
  f32x4 out;
  if constexpr (is_bf16<E>()) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(M + at<E, NCOL, LAY>(r0 + GS * g + (c >> 2), col0 + 4 * (c & 3))));
    const bf16x4 b = __builtin_bit_cast(bf16x4, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = to_f32(b[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = M[at<E, NCOL>(r0 + 4 * g + j, col0 + c)];
  }
  return out;
}


// Four accumulator rows of one lane (fp32) to global memory through a buffer resource, in the
// element type E: 8 bytes for bf16, 16 for fp32. Stores past the resource's end are dropped.
template <typename E>
__device__ __forceinline__ void store4_rsrc(rsrc_t r, uint32_t off, f32x4 v) {
  if constexpr (is_bf16<E>()) {
    const bf16x4 b = {from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]), from_f32<bf16>(v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, b), r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 0);
  }
}

// ---- helpers of the chunk-parallel gradient kernels --------------------------------------------
// Elements 4h .. 4h + 3 of eight bf16.
__device__ __forceinline__ bf16x4 half4(bf16x8 x, int h) {
  return h ? __builtin_shufflevector(x, x, 4, 5, 6, 7) : __builtin_shufflevector(x, x, 0, 1, 2, 3);
}

// Sum over the 16 lanes of a DPP row (lanes with equal lane / 16), in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

// Sum over the four lanes c, c + 16, c + 32, c + 48.
__device__ __forceinline__ float col4_sum(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}

// lower-triangular tile k (0..9) -> (ti, tj), ti >= tj
__device__ __forceinline__ void tri_tile(int k, int& ti, int& tj) {
  ti = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0;
  tj = k - ti * (ti + 1) / 2;
}

// Contraction index of element j of a lane's operand in group s (lane group g): see Grp.
template <typename E>
__device__ __forceinline__ int grp_index(int s, int g, int j) {
  if constexpr (is_bf16<E>())
    return 32 * s + 4 * g + (j & 3) + 16 * (j >> 2);
  else
    return 16 * s + 4 * g + j;
}

// Four consecutive entries col .. col + 3 (col a multiple of 4) of row r of a swizzled
// row-major matrix of NCOL columns, as fp32.
template <typename E, int NCOL>
__device__ __forceinline__ f32x4 row4(const E* M, int r, int col) {
  if constexpr (is_bf16<E>()) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(M + at<E, NCOL>(r, col));
    return (f32x4){to_f32(v[0]), to_f32(v[1]), to_f32(v[2]), to_f32(v[3])};
  } else {
    return *reinterpret_cast<const f32x4*>(M + at<E, NCOL>(r, col));
  }
}

// One chunk's operands in LDS (16-byte chunks of every row XOR-swizzled; see swz). With the
// per-channel decay (KDA) the buffer also holds the state-update operand K2 and the chunk's
// state decay gamma (a 1 KiB block, of which the first DK entries are this chunk's).
// HASP = false: P has a ring of its own (the one-pass bf16 forward with output waves).
template <typename E, int DK, int DVS, bool KDA = false, bool HASP = true>
struct ScanBuf {
  alignas(16) E K[kChunk * DK];
  alignas(16) E Q[kChunk * DK];
  alignas(16) E T[kChunk * kChunk];
  alignas(16) E P[HASP ? kChunk * kChunk : 8];
  alignas(16) E V[kChunk * DVS];
  alignas(16) float sc[kScRows * kChunk];
  alignas(16) E K2[KDA ? kChunk * DK : 8];
  alignas(16) float gam[KDA ? 256 : 4];
};

// Buffers in the ring: two where they fit in 160 KiB of LDS, else one. (The one-pass bf16
// forward scan uses three, with its own producer count; chunk_scan.hip.)
template <typename E, int DK, int DVS, bool KDA = false>
constexpr int scan_ring() {
  return 2 * sizeof(ScanBuf<E, DK, DVS, KDA>) <= 160 * 1024 ? 2 : 1;
}

}  // namespace kla
