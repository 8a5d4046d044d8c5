// Segment scan of the chunkwise forward, passes 2 and 3 (pass 1 is the scan kernel in its
// segment mode; the scheme is described with SegPlan in chunk_common.h).
//
// Sources: "Deep Dive into KDA", section 3: only the d_k x d_v state passes between chunks, and
// S[n+1] = Diag(gamma) S[n] + (Gamma o K[n])^T (U[n] - W[n] S[n]) is affine in S[n]; so is the
// chunk output O[n] = (Gamma o Q[n]) S[n] + Tril(...)(U[n] - W[n] S[n]). A run of chunks therefore
// maps its entering state S to M S + (its end state from zero), and its outputs to
// Y S + (its outputs from zero), with M and Y the responses to the identity.
#include "tile_ops.h"

namespace kla {

namespace {

// ---- pass 2: S_1 = end state of segment 0; S_{j+1} = M_j S_j + (end state of segment j) ----
// One workgroup per (head, 32-column slice of the state); fp32 throughout. Each S_j (j >= 1)
// is also stored transposed in the element type E, [DV][DK], the A operand layout of pass 3.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void seg_combine_kernel(ChunkParams p) {
  constexpr int CW = 32;
  constexpr int LDM = DK + 4, LDC = CW + 4;  // padded rows: no bank conflicts on the MFMA reads
  constexpr int NM = DK * DK / 4 / kThreads;  // 16-byte pieces of M per thread
  constexpr int NTILE = (DK / 16) * (CW / 16), TPW = NTILE / 4;
  __shared__ float Ms[DK * LDM];
  __shared__ float Sc[DK * LDC];
  const int64_t head = blockIdx.x / (DV / CW);
  const int cs = (int)(blockIdx.x % (DV / CW)) * CW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t nseg = p.nseg, u0 = head * nseg;
  const SegSpace<E> sg = SegSpace<E>::at(p.ws, p.seg_off, p.heads * p.nchunks, p.heads * nseg, DK, DV);

  {
    float x[DK * CW / kThreads];
#pragma unroll
    for (int i = 0; i < DK * CW / kThreads; ++i) {
      const int q = tid + kThreads * i, r = q / CW, cc = q % CW;
      x[i] = sg.Send[u0 * DK * DV + r * DV + cs + cc];
    }
#pragma unroll
    for (int i = 0; i < DK * CW / kThreads; ++i) {
      const int q = tid + kThreads * i, r = q / CW, cc = q % CW;
      Sc[r * LDC + cc] = x[i];
    }
  }
  __syncthreads();
  for (int64_t j = 1; j < nseg; ++j) {
    const float* m = sg.Mseg + (u0 + j) * DK * DK;
    const float* send = sg.Send + (u0 + j) * DK * DV;
    f32x4 mx[NM];
#pragma unroll
    for (int i = 0; i < NM; ++i) mx[i] = *reinterpret_cast<const f32x4*>(m + 4 * (tid + kThreads * i));
    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int q = wave * TPW + t, ti = q / (CW / 16), tj = q % (CW / 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = send[(16 * ti + 4 * g + e) * DV + cs + 16 * tj + c16];
    }
    // S_j, the entering state of segment j, transposed: this slice's rows of S_j^T
    E* sin = sg.SinT + (u0 + j) * DV * DK;
    for (int i = tid; i < CW * DK / 4; i += kThreads) {
      const int jj = i / (DK / 4), r = 4 * (i % (DK / 4));
      typename std::conditional<is_bf16<E>(), bf16x4, f32x4>::type y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = from_f32<E>(Sc[(r + e) * LDC + jj]);
      *reinterpret_cast<decltype(y)*>(sin + (int64_t)(cs + jj) * DK + r) = y;
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int q = 4 * (tid + kThreads * i), r = q / DK, k = q % DK;
      *reinterpret_cast<f32x4*>(&Ms[r * LDM + k]) = mx[i];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int q = wave * TPW + t, ti = q / (CW / 16), tj = q % (CW / 16);
      mma16_f32s(acc[t], &Ms[16 * ti * LDM], LDM, 1, &Sc[16 * tj], LDC, 1, 0, DK, lane);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int q = wave * TPW + t, ti = q / (CW / 16), tj = q % (CW / 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) Sc[(16 * ti + 4 * g + e) * LDC + 16 * tj + c16] = acc[t][e];
    }
    __syncthreads();
  }
  if (p.state_out) {
    float* out = p.state_out + head * DK * DV;
    for (int i = tid; i < DK * CW; i += kThreads) {
      const int r = i / CW, cc = i % CW;
      out[r * DV + cs + cc] = Sc[r * LDC + cc];
    }
  }
}

// ---- pass 3: o += Y S_j on the chunks of segments j >= 1 (in place: o holds O0) ----
// One workgroup per run of up to kFixChunks chunks of one segment; wave w takes token tile w of
// every chunk. The outputs are computed transposed, o^T = S_j^T Y^T, so that each lane holds four
// consecutive d_v entries of a token; S_j^T (the combine's transposed copy) sits in LDS.
// Eight chunks per workgroup: more workgroups in flight than with 16 (the pass is bound by
// memory latency, 46 % of HBM bandwidth at 16), for one more 32 KiB read of S_j^T per 8 chunks.
constexpr int kFixChunks = 8;

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void seg_fix_kernel(ChunkParams p) {
  typedef typename Grp<E>::V GV;
  constexpr int GK = Grp<E>::K, NGD = DK / GK, NJT = DV / 16;
  const int64_t nseg = p.nseg, L = p.seg_len, nchunks = p.nchunks;
  const int64_t gps = (L + kFixChunks - 1) / kFixChunks;  // workgroups per segment
  const int64_t per_head = (nseg - 1) * gps;
  const int64_t head = blockIdx.x / per_head, rem = blockIdx.x % per_head;
  const int64_t seg = 1 + rem / gps, grp = rem % gps;
  const int64_t c0 = seg * L + grp * kFixChunks;
  const int64_t send_ = (seg + 1) * L < nchunks ? (seg + 1) * L : nchunks;
  const int64_t c1 = c0 + kFixChunks < send_ ? c0 + kFixChunks : send_;
  if (c0 >= c1) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t bb = head / p.H, hh = head % p.H, T = p.T, H = p.H;
  const SegSpace<E> sg = SegSpace<E>::at(p.ws, p.seg_off, p.heads * nchunks, p.heads * nseg, DK, DV);

  // S_j^T into LDS (rows swizzled for conflict-free fragment reads), from the combine's copy
  constexpr int PER = 16 / sizeof(E), NCH = DV * DK / PER / kThreads;
  typedef typename Vec16<E>::type V16;
  __shared__ E St[DV * DK];
  {
    const E* st = sg.SinT + (head * nseg + seg) * DV * DK;
    V16 x[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) x[i] = *reinterpret_cast<const V16*>(st + (tid + kThreads * i) * PER);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = (tid + kThreads * i) * PER, r = q / DK, col = q % DK;
      *reinterpret_cast<V16*>(&St[at<E, DK>(r, col)]) = x[i];
    }
  }
  __syncthreads();

  const uint32_t vrow = H * DV * sizeof(E);
  const rsrc_t ro = make_rsrc(static_cast<E*>(p.o) + bb * T * H * DV, (uint32_t)(T * vrow));
  const E* Yh = sg.Y + head * nchunks * kChunk * DK;
  const int rt = wave;  // token tile
  // Y fragments and the O0 rows of one chunk (rows past T read zeros; their stores are dropped)
  auto load = [&](int64_t c, GV* yb, f32x4* acc) {
    const int64_t row = c * kChunk + 16 * rt + c16;  // this lane's token (head-local)
    const E* y = Yh + row * DK;
#pragma unroll
    for (int s = 0; s < NGD; ++s) {
      if constexpr (is_bf16<E>()) {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(y + 32 * s + 4 * g);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(y + 32 * s + 16 + 4 * g);
        yb[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        yb[s] = *reinterpret_cast<const f32x4*>(y + 16 * s + 4 * g);
      }
    }
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      const uint32_t off = (uint32_t)(row * vrow + (hh * DV + 16 * jt + 4 * g) * sizeof(E));
      if constexpr (is_bf16<E>()) {
        const bf16x4 x = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(ro, off, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jt][e] = to_f32(x[e]);
      } else {
        acc[jt] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
      }
    }
  };
  GV yb[3][NGD];
  f32x4 acc[3][NJT];
  load(c0, yb[0], acc[0]);
  if (c0 + 1 < c1) load(c0 + 1, yb[1], acc[1]);
  // three chunks per iteration, the next two chunks' loads in flight while one is computed
  for (int64_t c = c0; c < c1; c += 3) {
#pragma unroll
    for (int h = 0; h < 3; ++h) {
      const int64_t cc = c + h;
      if (cc >= c1) break;
      if (cc + 2 < c1) load(cc + 2, yb[(h + 2) % 3], acc[(h + 2) % 3]);
      const int64_t row = cc * kChunk + 16 * rt + c16;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x4 a = acc[h][jt];
#pragma unroll
        for (int s = 0; s < NGD; ++s) a = mma<E>(row_grp<E, DK>(St, 16 * jt + c16, s, g), yb[h][s], a);
        store4_rsrc<E>(ro, (uint32_t)(row * vrow + (hh * DV + 16 * jt + 4 * g) * sizeof(E)), a);
      }
    }
  }
}

template <typename E, int DK, int DV>
hipError_t launch_combine(const ChunkParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((seg_combine_kernel<E, DK, DV>), dim3((unsigned)(p.heads * (DV / 32))), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename E, int DK, int DV>
hipError_t launch_fix(const ChunkParams& p, hipStream_t stream) {
  const int64_t gps = (p.seg_len + kFixChunks - 1) / kFixChunks;
  hipLaunchKernelGGL((seg_fix_kernel<E, DK, DV>), dim3((unsigned)(p.heads * (p.nseg - 1) * gps)), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename E>
hipError_t combine_e(const ChunkParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_combine<E, 128, 128>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_combine<E, 64, 64>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_combine<E, 128, 64>(p, stream);
  return launch_combine<E, 64, 128>(p, stream);
}

template <typename E>
hipError_t fix_e(const ChunkParams& p, int64_t d_k, int64_t d_v, hipStream_t stream) {
  if (d_k == 128 && d_v == 128) return launch_fix<E, 128, 128>(p, stream);
  if (d_k == 64 && d_v == 64) return launch_fix<E, 64, 64>(p, stream);
  if (d_k == 128 && d_v == 64) return launch_fix<E, 128, 64>(p, stream);
  return launch_fix<E, 64, 128>(p, stream);
}

}  // namespace

hipError_t launch_seg_combine(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream) {
  return bf16_io ? combine_e<bf16>(p, d_k, d_v, stream) : combine_e<float>(p, d_k, d_v, stream);
}

hipError_t launch_seg_fix(const ChunkParams& p, int64_t d_k, int64_t d_v, bool bf16_io, hipStream_t stream) {
  return bf16_io ? fix_e<bf16>(p, d_k, d_v, stream) : fix_e<float>(p, d_k, d_v, stream);
}

}  // namespace kla
