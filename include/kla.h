/*
 * kla.h — C ABI of the Kaczmarz Linear Attention (KLA) hot path for AMD Instinct
 * MI355X (CDNA4, gfx950).
 *
 * The method ("Kaczmarz Linear Attention", Abstract) is Gated DeltaNet's recurrence
 * ("Deep Dive into KDA", section 2.2) with the Kaczmarz step size
 *     beta_t = eta_t / (||k_t||_2^2 + eps).
 * The state of one head is stored as S = M^T with shape [d_k][d_v] (d_v contiguous),
 * where M is the d_v x d_k map of the pages:
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t.
 * (The erase acts on the key side so that, with alpha = eta = 1 and eps = 0, the new
 * state maps k_t to v_t exactly — the projection the pages describe.)
 * The decay is passed as log(alpha_t); alpha_t = exp(log_alpha_t).
 *
 * Conventions shared by every entry point
 *   Layouts (row-major, contiguous, no strides):
 *     q, k        [B, T, H, d_k]      (decode: [B, H, d_k])
 *     v, o        [B, T, H, d_v]      (decode: [B, H, d_v])
 *     eta, log_alpha, beta, gcum  [B, T, H] fp32   (decode: [B, H])
 *     state       [B, H, d_k, d_v] fp32
 *   dt selects the element type of q, k, v and o: KLA_BF16 (bfloat16) or KLA_F32.
 *   State, gates and all accumulation are fp32 in both cases.
 *   Pointers are device pointers (HIP device memory of the current device) unless
 *   stated otherwise; q/k/v/o/state must be 16-byte aligned, gate arrays 4-byte aligned.
 *   Supported head sizes: d_k, d_v in {64, 128}. The chunk length must be 64.
 *   eta is used as given (any finite value >= 0; the pages' eta is a sigmoid output).
 *   eps must be finite and >= 0. With eps = 0 a zero key gives beta = inf and NaNs,
 *   exactly as the recurrence does.
 *   stream is a hipStream_t (NULL: the legacy default stream). Every call only
 *   enqueues work on that stream and returns; nothing waits on the host.
 *   Ownership: the caller allocates and owns every buffer. The library allocates
 *   nothing and keeps no pointer after a call returns.
 *   Errors: arguments are checked before anything is enqueued; on a bad argument the
 *   call returns KLA_ERR_INVALID_VALUE or KLA_ERR_NOT_SUPPORTED and enqueues nothing.
 *   A failed launch returns KLA_ERR_LAUNCH; kla_last_error() then holds the HIP text.
 *   Calls with B, H or (where present) T equal to 0 do no work beyond what is stated.
 */
#ifndef KLA_H
#define KLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kla_status {
  KLA_OK = 0,
  KLA_ERR_INVALID_VALUE = 1, /* null/misaligned pointer, negative size, bad eps, overlap */
  KLA_ERR_NOT_SUPPORTED = 2, /* head size or chunk length this build does not provide */
  KLA_ERR_LAUNCH = 3         /* the HIP runtime refused a launch; see kla_last_error() */
} kla_status_t;

typedef enum kla_dtype { KLA_F32 = 0, KLA_BF16 = 1 } kla_dtype_t;

/*
 * kla_prepare_beta — the prologue on its own.
 * Source: "Kaczmarz Linear Attention", Abstract (beta_t = eta_t / (||k_t||^2 + eps));
 * "Deep Dive into KDA", section 3 (intra-chunk accumulated decay computed once by
 * prefix sums) and section 5 (log-domain prefixes).
 *   beta_out[b,t,h] = eta[b,t,h] / (sum_i k[b,t,h,i]^2 + eps)        (fp32 accumulation)
 *   gcum_out[b,t,h] = sum of log_alpha[b,s,h] over s in t's chunk with s <= t,
 *                     chunks being [0,chunk), [chunk,2 chunk), ... along T.
 * gcum_out may be NULL (not computed). kla_chunk_fwd computes the same values
 * internally; this entry point exists for callers who want beta itself.
 */
kla_status_t kla_prepare_beta(const void* k, const float* eta, const float* log_alpha,
                              float* beta_out, float* gcum_out,
                              int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t chunk,
                              float eps, kla_dtype_t dt, void* stream);

/*
 * kla_chunk_fwd_workspace_size — bytes of device workspace kla_chunk_fwd needs for
 * these sizes on the current device (0 when it needs none). The amount depends on the scan's
 * plan, which the library sizes to the current device's compute units (the full MI355X's when
 * no device is present). Host-only; never fails.
 */
size_t kla_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                    int64_t chunk, kla_dtype_t dt);

/*
 * kla_chunk_fwd — chunkwise-parallel forward over a whole sequence (prefill / training).
 * Source: "Kaczmarz Linear Attention", Abstract (KLA keeps GDN's chunkwise parallel
 * algorithm); "Deep Dive into KDA", section 3 (inter-chunk state update
 * S[n+1] = Diag(gamma) S[n] + (Gamma o K[n])^T (U[n] - W[n] S[n]) and intra-chunk output
 * O[n] = (Gamma o Q[n]) S[n] + Tril(...)(U[n] - W[n] S[n])), with a scalar gate.
 * Computes, for every head, o_t = S_t^T q_t for t = 0..T-1 starting from S_0, and the
 * final state S_T. Numerically it equals the token recurrence up to rounding.
 *   state_in   [B,H,d_k,d_v] fp32, or NULL for S_0 = 0.
 *   state_out  [B,H,d_k,d_v] fp32, or NULL if the final state is not wanted.
 *              state_out may equal state_in (in-place update); any other overlap is an error.
 *   o          [B,T,H,d_v] of type dt; must not overlap any input.
 *   T          any length >= 0; a last partial chunk is handled. T = 0 writes
 *              state_out = S_0 and no output. One batch entry's q/k/v/o rows must stay
 *              below 2 GiB ((T + 64) * H * max(d_k, d_v) * element size < 2^31), else
 *              KLA_ERR_NOT_SUPPORTED.
 *   workspace  device buffer of at least kla_chunk_fwd_workspace_size(...) bytes, or NULL
 *              when that size is 0.
 */
kla_status_t kla_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* eta, const float* log_alpha,
                           const float* state_in, float* state_out, void* o,
                           int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                           float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * kla_chunk_fwd_noalloc — kla_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. The caller passes
 * inputs and outputs only; the workspace is a static device array of KLA_NOALLOC_SCRATCH_BYTES
 * (128 MiB) inside the library, one per device, held from the first call on that device until the
 * process ends. The call allocates nothing (no hipMalloc, no hipFree, no allocating routine).
 *   Sizes: accepted while kla_chunk_fwd_workspace_size(...) <= KLA_NOALLOC_SCRATCH_BYTES (for bf16
 *   and d_k = d_v = 128 about 17 KiB per 64-token chunk of one head: B * H * ceil(T / 64) up to
 *   7 710 on the one-pass plan); larger ones return KLA_ERR_NOT_SUPPORTED, with both sizes in
 *   kla_last_error(), and enqueue nothing.
 *   Every call on one device shares that device's array, which keeps the last call's contents (no
 *   part of it needs clearing: a call writes every byte it reads). Calls that overlap in time on
 *   one device (on different streams, or from different host threads) race on it and give wrong
 *   results: serialise them.
 * Otherwise exactly kla_chunk_fwd (same plan, same kernels, the same results bit for bit).
 */
#define KLA_NOALLOC_SCRATCH_BYTES (128u << 20)
kla_status_t kla_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* eta, const float* log_alpha,
                                   const float* state_in, float* state_out, void* o,
                                   int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                   float eps, kla_dtype_t dt, void* stream);

/*
 * kla_chunk_fwd_seg_workspace_size / kla_chunk_fwd_seg — kla_chunk_fwd with the scan's plan given
 * by the caller instead of chosen by the library.
 * Source: "Deep Dive into KDA", section 3 (each chunk maps the entering state to an affine
 * function of it, so a head's chunks can be cut into segments scanned at the same time and joined
 * by composing those maps); "Kaczmarz Linear Attention", Abstract (KLA keeps the chunkwise
 * parallel algorithm). Segments change the result only by rounding.
 *   segments   0: the library's plan for the current device (exactly kla_chunk_fwd);
 *              n >= 1: the chunks of every head are cut into about n segments of equal length
 *              (n is clipped to the number of chunks; segments of ceil(chunks / n) chunks, so the
 *              count actually used may be lower); n = 1 is the one-pass scan. Negative:
 *              KLA_ERR_INVALID_VALUE (the size query returns 0).
 * The workspace size depends on the plan: size it with kla_chunk_fwd_seg_workspace_size for the
 * same segments and current device. Everything else is as for kla_chunk_fwd. For tuning and for
 * tests that force the segmented scan; kla_chunk_fwd is the entry point for other callers.
 */
size_t kla_chunk_fwd_seg_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                        int64_t chunk, int64_t segments, kla_dtype_t dt);
kla_status_t kla_chunk_fwd_seg(const void* q, const void* k, const void* v,
                               const float* eta, const float* log_alpha,
                               const float* state_in, float* state_out, void* o,
                               int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                               int64_t segments, float eps, kla_dtype_t dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * kla_decode_step — one recurrent decode step for B x H heads (one new token each).
 * Source: "Kaczmarz Linear Attention", Abstract (recurrent decoding with a fixed-size
 * state); "Deep Dive into KDA", section 2.2 (the token update) and section 3 (memory
 * decoupled from sequence length).
 * Per head: n = ||k||^2, beta = eta / (n + eps), alpha = exp(log_alpha);
 *   u = alpha S^T k,  p = alpha S^T q,  delta = beta (v - u),
 *   o = p + (k.q) delta  (= S_new^T q),   S <- alpha S + k delta^T   (in place).
 *   q, k [B,H,d_k], v [B,H,d_v], o [B,H,d_v] of type dt; eta, log_alpha [B,H] fp32;
 *   state [B,H,d_k,d_v] fp32, read and overwritten. o must not overlap the state.
 */
kla_status_t kla_decode_step(const void* q, const void* k, const void* v,
                             const float* eta, const float* log_alpha,
                             float* state, void* o,
                             int64_t B, int64_t H, int64_t d_k, int64_t d_v,
                             float eps, kla_dtype_t dt, void* stream);

/*
 * kla_gdn_chunk_fwd — kla_chunk_fwd with the step size supplied by the caller: the gated
 * DeltaNet recurrence this method modifies, and DeltaNet itself.
 * Source: "Deep Dive into KDA", section 2.2 (Gated DeltaNet,
 * S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t v_t k_t^T, with the same state layout
 * as above) and section 2.1 (DeltaNet: the same without the gate); "Kaczmarz Linear
 * Attention", Abstract (KLA changes only how beta_t is obtained, not the recurrence or its
 * chunkwise algorithm).
 *   beta       [B,T,H] fp32, beta_t used as given (any finite value; no eps, no key norm).
 *   log_alpha  [B,T,H] fp32, or NULL for alpha_t = 1 (DeltaNet).
 * Everything else (layouts, T, state_in/state_out, workspace, kla_chunk_fwd_workspace_size,
 * errors) is as for kla_chunk_fwd.
 */
kla_status_t kla_gdn_chunk_fwd(const void* q, const void* k, const void* v,
                               const float* beta, const float* log_alpha,
                               const float* state_in, float* state_out, void* o,
                               int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                               kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kla_gdn_decode_step — kla_decode_step with beta supplied by the caller (gated DeltaNet;
 * DeltaNet when log_alpha is NULL). Source: "Deep Dive into KDA", sections 2.1 and 2.2.
 *   beta [B,H] fp32 as given; log_alpha [B,H] fp32 or NULL (alpha = 1). Otherwise as
 *   kla_decode_step: u = alpha S^T k, p = alpha S^T q, delta = beta (v - u),
 *   o = p + (k.q) delta, S <- alpha S + k delta^T (in place).
 */
kla_status_t kla_gdn_decode_step(const void* q, const void* k, const void* v,
                                 const float* beta, const float* log_alpha,
                                 float* state, void* o,
                                 int64_t B, int64_t H, int64_t d_k, int64_t d_v,
                                 kla_dtype_t dt, void* stream);

/*
 * kla_kda_chunk_fwd_workspace_size — bytes of device workspace kla_kda_chunk_fwd needs (0 when
 * T = 0 or the sizes are not supported). Host-only; never fails. About 65 KiB per chunk of 64
 * tokens per head for bf16 and d_k = 128: the forward's per-chunk factors plus the decayed
 * operands K o e^G, Q o e^G, K o e^{G_C - G} and the chunk's decay e^{G_C}.
 */
size_t kla_kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                        int64_t chunk, kla_dtype_t dt);

/*
 * kla_kda_chunk_fwd — chunkwise forward with a per-channel (diagonal) decay, KDA's gate.
 * Source: "Deep Dive into KDA", section 2.3 (S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1}
 * + beta_t v_t k_t^T) and section 3 (the chunkwise form with per-channel Gamma; decay prefixes in
 * the log domain, section 5). In this library's [d_k, d_v] state orientation Diag(a_t) scales
 * the state's d_k rows: S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1} + beta_t k_t v_t^T,
 * o_t = S_t^T q_t.
 *   log_a      [B,T,H,d_k] fp32, log of the per-channel decay (<= 0 in use; any finite value is
 *              accepted), 16-byte aligned.
 *   eta        [B,T,H] fp32: eta of the Kaczmarz step beta = eta / (||k||^2 + eps)
 *              ("Kaczmarz Linear Attention", Abstract) when beta_given = 0, else beta itself
 *              (eps is then ignored).
 *   Everything else (layouts, T, state_in/state_out aliasing, workspace, errors) as for
 *   kla_chunk_fwd, with the size limit also applied to log a's rows:
 *   (T + 64) * H * max(d_k, d_v) * element size and (T + 64) * H * d_k * 4 both below 2^31,
 *   else KLA_ERR_NOT_SUPPORTED. The scan is planned as kla_chunk_fwd's: cut into sequence
 *   segments when few heads would leave compute units idle (kla_kda_chunk_fwd_workspace_size
 *   includes the segment buffers then).
 */
kla_status_t kla_kda_chunk_fwd(const void* q, const void* k, const void* v,
                               const float* eta, const float* log_a,
                               const float* state_in, float* state_out, void* o,
                               int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                               float eps, int beta_given, kla_dtype_t dt,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * kla_kda_decode_step — one recurrent decode step with the per-channel decay (section 2.3):
 * u = (Diag(a) S)^T k, p = (Diag(a) S)^T q, delta = beta (v - u), o = p + (k.q) delta,
 * S <- Diag(a) S + k delta^T (in place).
 *   log_a [B,H,d_k] fp32; eta / beta_given / eps as for kla_kda_chunk_fwd; the rest as for
 *   kla_decode_step.
 */
kla_status_t kla_kda_decode_step(const void* q, const void* k, const void* v,
                                 const float* eta, const float* log_a,
                                 float* state, void* o,
                                 int64_t B, int64_t H, int64_t d_k, int64_t d_v,
                                 float eps, int beta_given, kla_dtype_t dt, void* stream);

/*
 * kla_chunk_bwd_workspace_size — bytes of device workspace kla_chunk_bwd and
 * kla_gdn_chunk_bwd need for these sizes (0 when T = 0 or the sizes are not supported).
 * Host-only; never fails. For bf16 and d_k = d_v = 128 it is about 113 KiB per chunk of
 * 64 tokens per head: the forward's per-chunk factors plus every chunk's entering state,
 * state gradient, Delta and solve gradient.
 */
size_t kla_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                    int64_t chunk, kla_dtype_t dt);

/*
 * kla_chunk_bwd — gradients of the chunkwise forward (training).
 * Source: "Kaczmarz Linear Attention", Abstract (the chunkwise form serves training, with the
 * step size beta_t = eta_t / (||k_t||^2 + eps)); "Deep Dive into KDA", section 3 (the
 * chunkwise forward that is differentiated). The pages give no backward formulas: the result
 * is the exact gradient of the token recurrence, up to rounding.
 * For the scalar loss L = sum(do * o) + sum(dstate_out * S_T), with o and S_T the outputs of
 * kla_chunk_fwd on the same inputs, computes
 *   dq, dk     [B,T,H,d_k] of type dt   dL/dq, dL/dk (dk includes the path through beta)
 *   dv         [B,T,H,d_v] of type dt   dL/dv
 *   deta       [B,T,H] fp32             dL/deta
 *   dlog_alpha [B,T,H] fp32             dL/dlog(alpha)
 *   dstate_in  [B,H,d_k,d_v] fp32       dL/dS_0, or NULL if not wanted
 * Inputs: q, k, v, eta, log_alpha, state_in (NULL for S_0 = 0) exactly as given to
 * kla_chunk_fwd; do [B,T,H,d_v] of type dt; dstate_out [B,H,d_k,d_v] fp32 or NULL (zero).
 * The forward is recomputed inside; o is not needed.
 *   Supported: d_k, d_v in {64, 128}, bf16 or fp32 (else KLA_ERR_NOT_SUPPORTED). chunk must
 *   be 64. Any T >= 0 (a last partial chunk is handled); T = 0 writes dstate_in = dstate_out (or
 *   zeros) and nothing else.
 *   No output may overlap an input or another output (KLA_ERR_INVALID_VALUE).
 *   workspace  device buffer of at least kla_chunk_bwd_workspace_size(...) bytes (NULL when
 *              T = 0); its contents on entry do not matter.
 * Stream-ordered and asynchronous; the library allocates nothing and keeps no pointer.
 */
kla_status_t kla_chunk_bwd(const void* q, const void* k, const void* v,
                           const float* eta, const float* log_alpha, const float* state_in,
                           const void* dout, const float* dstate_out,
                           void* dq, void* dk, void* dv, float* deta, float* dlog_alpha,
                           float* dstate_in,
                           int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                           float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * kla_gdn_chunk_bwd — kla_chunk_bwd with beta supplied by the caller (gated DeltaNet;
 * DeltaNet when log_alpha is NULL). Source: "Deep Dive into KDA", sections 2.1-3.
 *   beta [B,T,H] fp32 as given; dbeta [B,T,H] fp32 receives dL/dbeta (the key norm does not
 *   enter beta, so dk has no step-size path). log_alpha may be NULL (alpha = 1), and then
 *   dlog_alpha may be NULL too. Otherwise as kla_chunk_bwd.
 */
kla_status_t kla_gdn_chunk_bwd(const void* q, const void* k, const void* v,
                               const float* beta, const float* log_alpha, const float* state_in,
                               const void* dout, const float* dstate_out,
                               void* dq, void* dk, void* dv, float* dbeta, float* dlog_alpha,
                               float* dstate_in,
                               int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                               kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kla_chunk_fwd_train — the chunkwise forward for training: kla_chunk_fwd, which also leaves in
 * `workspace` what kla_chunk_bwd would otherwise recompute, so that kla_chunk_bwd_saved can skip
 * that. Source: "Kaczmarz Linear Attention", Abstract (the chunkwise form serves training);
 * "Deep Dive into KDA", section 3 (the chunkwise forward; its per-chunk states S[n] are what
 * passes between chunks).
 *   Arguments as kla_chunk_fwd (o, state_out and all inputs alike; the outputs agree with
 *   kla_chunk_fwd's up to rounding), except:
 *   workspace  device buffer of at least kla_chunk_bwd_workspace_size(...) bytes (NULL when
 *              T = 0). On return it holds the per-chunk factors and every chunk's entering state
 *              and Delta; the caller keeps it unchanged for kla_chunk_bwd_saved.
 *   Always one pass over the sequence (no segments). Errors as kla_chunk_fwd.
 */
kla_status_t kla_chunk_fwd_train(const void* q, const void* k, const void* v,
                                 const float* eta, const float* log_alpha, const float* state_in,
                                 float* state_out, void* o,
                                 int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                 float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * kla_gdn_chunk_fwd_train — kla_chunk_fwd_train with beta supplied by the caller (gated
 * DeltaNet; DeltaNet when log_alpha is NULL), as kla_gdn_chunk_fwd. Source: "Deep Dive into
 * KDA", sections 2.1-3.
 */
kla_status_t kla_gdn_chunk_fwd_train(const void* q, const void* k, const void* v,
                                     const float* beta, const float* log_alpha, const float* state_in,
                                     float* state_out, void* o,
                                     int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                     kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kla_chunk_bwd_saved — kla_chunk_bwd from the workspace kla_chunk_fwd_train filled: the
 * forward is not recomputed. Source: as kla_chunk_bwd.
 *   Arguments and results as kla_chunk_bwd. The inputs (q, k, v, eta, log_alpha, state_in,
 *   sizes, eps, dt) must be those of the kla_chunk_fwd_train call that filled `workspace`, and
 *   the workspace unchanged since; the library cannot check this, and results are undefined
 *   otherwise. The workspace's saved part is still valid after the call (it may be called again
 *   for another do / dstate_out).
 */
kla_status_t kla_chunk_bwd_saved(const void* q, const void* k, const void* v,
                                 const float* eta, const float* log_alpha, const float* state_in,
                                 const void* dout, const float* dstate_out,
                                 void* dq, void* dk, void* dv, float* deta, float* dlog_alpha,
                                 float* dstate_in,
                                 int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                 float eps, kla_dtype_t dt, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * kla_gdn_chunk_bwd_saved — kla_gdn_chunk_bwd from the workspace kla_gdn_chunk_fwd_train filled
 * (as kla_chunk_bwd_saved). Source: "Deep Dive into KDA", sections 2.1-3.
 */
kla_status_t kla_gdn_chunk_bwd_saved(const void* q, const void* k, const void* v,
                                     const float* beta, const float* log_alpha, const float* state_in,
                                     const void* dout, const float* dstate_out,
                                     void* dq, void* dk, void* dv, float* dbeta, float* dlog_alpha,
                                     float* dstate_in,
                                     int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                     kla_dtype_t dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kla_kda_chunk_bwd_workspace_size — bytes of device workspace kla_kda_chunk_bwd needs (0 when
 * T = 0 or the sizes are not supported). Host-only; never fails. For bf16 and d_k = d_v = 128 it
 * is about 162 KiB per chunk of 64 tokens per head: the KDA forward's per-chunk factors and
 * decayed operands plus every chunk's entering state, state gradient, Delta and solve gradient.
 */
size_t kla_kda_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                        int64_t chunk, kla_dtype_t dt);

/*
 * kla_kda_chunk_bwd — gradients of kla_kda_chunk_fwd (training with the per-channel decay).
 * Source: "Deep Dive into KDA", section 2.3 (S_t = (I - beta_t k_t k_t^T) Diag(a_t) S_{t-1}
 * + beta_t v_t k_t^T, here with the state stored [d_k, d_v]) and section 3 (the chunkwise form
 * that is differentiated, decay ratios in the log domain); "Kaczmarz Linear Attention",
 * Abstract (beta_t = eta_t / (||k_t||^2 + eps)). The pages give no backward formulas: the result
 * is the exact gradient of the token recurrence, up to rounding.
 * For L = sum(do * o) + sum(dstate_out * S_T), with o and S_T the outputs of kla_kda_chunk_fwd on
 * the same inputs, computes
 *   dq, dk     [B,T,H,d_k] of type dt   (dk includes the path through beta unless beta_given)
 *   dv         [B,T,H,d_v] of type dt
 *   deta       [B,T,H] fp32             dL/deta, or dL/dbeta when beta_given
 *   dlog_a     [B,T,H,d_k] fp32         dL/dlog a, per channel
 *   dstate_in  [B,H,d_k,d_v] fp32       dL/dS_0, or NULL if not wanted
 * Inputs: q, k, v, eta, log_a (16-byte aligned), state_in (NULL for S_0 = 0), eps and beta_given
 * exactly as given to kla_kda_chunk_fwd; do [B,T,H,d_v] of type dt; dstate_out [B,H,d_k,d_v]
 * fp32 or NULL (zero). The forward is recomputed inside.
 *   Supported: bf16 with d_k, d_v in {64, 128}; fp32 with d_k = d_v = 64 (else
 *   KLA_ERR_NOT_SUPPORTED). chunk must be 64. Any T >= 0; T = 0 writes dstate_in = dstate_out
 *   (or zeros) and nothing else. Size limits as kla_kda_chunk_fwd. No output may overlap an
 *   input or another output (KLA_ERR_INVALID_VALUE).
 *   workspace  device buffer of at least kla_kda_chunk_bwd_workspace_size(...) bytes (NULL when
 *              T = 0); its contents on entry do not matter.
 * Stream-ordered and asynchronous; the library allocates nothing and keeps no pointer.
 */
kla_status_t kla_kda_chunk_bwd(const void* q, const void* k, const void* v,
                               const float* eta, const float* log_a, const float* state_in,
                               const void* dout, const float* dstate_out,
                               void* dq, void* dk, void* dv, float* deta, float* dlog_a,
                               float* dstate_in,
                               int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                               float eps, int beta_given, kla_dtype_t dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * kla_kda_chunk_fwd_train — kla_kda_chunk_fwd for training (as kla_chunk_fwd_train): the
 * workspace, of at least kla_kda_chunk_bwd_workspace_size(...) bytes, is left holding what
 * kla_kda_chunk_bwd would recompute. Source: "Deep Dive into KDA", sections 2.3 and 3.
 *   Supported as kla_kda_chunk_bwd (fp32 only with d_k = d_v = 64; else KLA_ERR_NOT_SUPPORTED);
 *   one pass over the sequence. Otherwise arguments and errors as kla_kda_chunk_fwd.
 */
kla_status_t kla_kda_chunk_fwd_train(const void* q, const void* k, const void* v,
                                     const float* eta, const float* log_a, const float* state_in,
                                     float* state_out, void* o,
                                     int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                     float eps, int beta_given, kla_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * kla_kda_chunk_bwd_saved — kla_kda_chunk_bwd from the workspace kla_kda_chunk_fwd_train filled
 * for the same inputs (as kla_chunk_bwd_saved). Source: "Deep Dive into KDA", sections 2.3 and 3.
 */
kla_status_t kla_kda_chunk_bwd_saved(const void* q, const void* k, const void* v,
                                     const float* eta, const float* log_a, const float* state_in,
                                     const void* dout, const float* dstate_out,
                                     void* dq, void* dk, void* dv, float* deta, float* dlog_a,
                                     float* dstate_in,
                                     int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, int64_t chunk,
                                     float eps, int beta_given, kla_dtype_t dt, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* kla_status_string(kla_status_t status);

/* Text of the last error on the calling host thread ("" if none). */
const char* kla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H */
