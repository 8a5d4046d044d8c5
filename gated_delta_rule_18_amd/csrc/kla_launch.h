// Host-side launch interface between the C ABI (kla_abi.hip) and the kernel files.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kla {

constexpr int kChunk = 64;  // chunk length of the chunkwise algorithm

// Compute units and XCDs of the current device, queried once per device ordinal (the full
// MI355X's 256 and 8 when there is no device to ask, e.g. for a host-only size query).
// Workgroups are dealt round-robin to the XCDs; the launches use the count to keep the
// workgroups of one head on one XCD (one L2), and the plans size grids to the compute units.
struct DeviceInfo {
  int cus;
  int xcds;
};
DeviceInfo device_info();

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* log_alpha;
  float* state;
  void* o;
  int64_t B, H, d_k, d_v;
  float eps;
  bool bf16;
  bool beta_given;  // eta holds beta itself; log_alpha may be null (alpha = 1)
  bool kda = false;  // log_alpha holds log a [B, H, d_k] (per-channel decay)
};

struct PrepareArgs {
  const void* k;
  const float* eta;
  const float* log_alpha;
  float* beta;
  float* gcum;  // may be null
  int64_t B, T, H, d_k;
  float eps;
  bool bf16;
};

struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* log_alpha;
  const float* state_in;  // may be null: S_0 = 0
  float* state_out;       // may be null
  void* o;
  int64_t B, T, H, d_k, d_v;
  float eps;
  bool bf16;
  void* workspace;
  size_t workspace_bytes;
  bool beta_given;  // eta holds beta itself; log_alpha may be null (alpha = 1)
  int64_t segments = 0;  // sequence segments of the scan; 0: the library's plan
};

struct ChunkBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* eta;
  const float* log_alpha;   // may be null when beta_given (alpha = 1)
  const float* state_in;    // may be null: S_0 = 0
  const void* dout;         // dL/do
  const float* dstate_out;  // dL/dS_T, may be null (zero)
  void* dq;
  void* dk;
  void* dv;
  float* deta;        // dL/deta, or dL/dbeta when beta_given
  float* dlog_alpha;  // may be null only when log_alpha is
  float* dstate_in;   // dL/dS_0, may be null
  int64_t B, T, H, d_k, d_v;
  float eps;
  bool bf16;
  void* workspace;
  size_t workspace_bytes;
  bool beta_given;
  bool kda = false;  // per-channel decay: log_alpha holds log a [B, T, H, d_k], dlog_alpha d log a
  bool saved = false;  // the workspace holds what launch_chunk_fwd_train left for these inputs
};

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prepare_beta(const PrepareArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream);
// segments: as ChunkArgs::segments (0: the library's plan for the current device).
size_t chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16,
                                 int64_t segments = 0);
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, hipStream_t stream);
// The forward for training (scalar gate, one pass): as launch_chunk_fwd, and a.workspace
// (chunk_bwd_workspace_bytes) is left holding the prep's per-chunk factors, made as the
// backward makes them, and every chunk's entering state and Delta, so that launch_chunk_bwd with
// saved skips its prep and its recompute of the forward.
hipError_t launch_chunk_fwd_train(const ChunkArgs& a, hipStream_t stream);
// The same for the per-channel decay (chunk_kda_bwd_workspace_bytes; launch_chunk_bwd with kda).
hipError_t launch_chunk_kda_fwd_train(const ChunkArgs& a, hipStream_t stream);
// Per-channel decay (KDA): ChunkArgs.log_alpha / DecodeArgs.log_alpha hold log a [.., d_k].
hipError_t launch_chunk_kda_fwd(const ChunkArgs& a, hipStream_t stream);
size_t chunk_kda_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16,
                                     int64_t segments = 0);
size_t chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16);
size_t chunk_kda_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, bool bf16);
bool chunk_grad_supported(int64_t d_k, int64_t d_v, bool bf16);
bool chunk_grad_kda_supported(int64_t d_k, int64_t d_v, bool bf16);

}  // namespace kla
