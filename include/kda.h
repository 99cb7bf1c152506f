/*
 * kda.h -- C ABI of libkda.so, the MI355X (gfx950) implementation of the
 * Kimi Delta Attention (KDA) gated delta-rule recurrence.
 *
 * The recurrence (Kimi Linear summary page, "recurrent layers" paragraph:
 * each step decays the state per channel, removes the old state's projection
 * onto the current key, then writes the new key/value pair; the remio.ai page,
 * section on KDA's recurrent memory: a per-channel forget gate on top of Gated
 * DeltaNet's delta rule).  Per batch row b and head h the state S is a dk x dv
 * fp32 matrix whose rows are key channels.  For each valid token t:
 *
 *     S'  = Diag(exp(log_alpha_t)) S
 *     u   = beta_t (v_t - S'^T k_t)
 *     S   = S' + k_t u^T
 *     o_t = S^T q_t                       (no 1/sqrt(dk) scale; callers pre-scale q)
 *
 * Masks (Transformers issue report on Kimi Linear cached continuation:
 * padding must advance neither the convolution state nor the recurrent
 * state).  A position with mask == 0 behaves as alpha = 1, beta = 0: it leaves
 * S untouched, produces o_t = 0, and its q/k/v/log_alpha/beta values are never
 * read into the arithmetic (NaN or garbage there cannot leak).
 *
 * Conventions for every entry point
 *   - All tensor pointers are device pointers (HBM), dense, row-major, owned by
 *     the caller, and aligned to their element size; the tensors each entry
 *     point reads with 16-byte vector accesses (listed there) must be 16-byte
 *     aligned.  The library allocates nothing, keeps no pointer after
 *     returning, and holds no global state, except the per-GPU scratch array
 *     of kda_chunk_prefill_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it; nothing synchronises the host.
 *   - Arguments are validated on the host before any HIP call.  A failing call
 *     returns a negative kda_status and has no side effect.  KDA_ERR_HIP means
 *     a launch failed; kda_last_hip_error() then gives the hipError_t value
 *     (per calling thread).
 *   - `dtype` is the element type of q, k, v, o (and x, y, conv_cache for the
 *     short convolution).  log_alpha, beta, weights and states are always fp32.
 *   - Results are bitwise deterministic for identical inputs and arguments
 *     (no atomics, fixed reduction orders).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 4

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = -1,  /* null pointer where one is required, negative size, bad alignment */
  KDA_ERR_UNSUPPORTED = -2,  /* well-formed but outside the supported set (head size, chunk, width) */
  KDA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the size query returned */
  KDA_ERR_HIP = -4           /* a HIP launch failed; see kda_last_hip_error() */
} kda_status;

typedef enum { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

enum {
  /* normalise q and k per (b,t,h) to x / sqrt(sum x^2 + 1e-6) before use */
  KDA_FLAG_L2NORM_QK = 1u,
  /* short convolution: apply SiLU, y = z / (1 + exp(-z)) */
  KDA_FLAG_SILU = 2u,
  /* Gated DeltaNet's gate: one log forget gate per (token, head), applied to every key
   * channel; log_alpha is then [B,T,H] in a prefill and [B,H] in a decode step (Kimi
   * Linear summary page, recurrent-layers paragraph: earlier variants gate whole heads,
   * KDA each channel; remio.ai page, KDA section: KDA extends Gated DeltaNet).  With bf16
   * inputs the prefill forms the chunk's decay-weighted products as Gram products of the
   * raw rows times a per-row decay mask, so its results differ from those of the
   * per-channel call fed the broadcast gate by rounding; with fp32 inputs, and in the decode
   * steps, they are the same bit for bit. */
  KDA_FLAG_SCALAR_GATE = 4u,
  /* prefill: scan each (b, h) or packed sequence as one chain of chunks, never in
   * segments (see kda_chunk_prefill); calls that save states, and the backward, always do */
  KDA_FLAG_SERIAL_SCAN = 8u
};

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

/* Static, human-readable name of a kda_status value (never NULL). */
const char* kda_status_string(int status);

/* hipError_t of the last KDA_ERR_HIP returned on this thread (0 if none). */
int kda_last_hip_error(void);

/*
 * Bytes of device workspace kda_chunk_prefill needs for these arguments
 * (0 when none is needed).  Returns 0 as well for arguments that the call
 * itself would reject.
 */
size_t kda_chunk_prefill_workspace_size(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/*
 * Chunked prefill of T tokens for B sequences and H heads (Kimi Linear
 * summary page, paragraph on the kernels: sequences are split into chunks and
 * the chunk's rank-1 updates are batched through a WY representation, i.e. a
 * triangular solve).  Computes exactly the token recurrence above; `chunk` is
 * a tuning parameter that changes rounding only.
 *
 *   q, k        [B,T,H,dk]   dtype
 *   v           [B,T,H,dv]   dtype
 *   log_alpha   [B,T,H,dk]   fp32, finite, <= 0 (per-channel log forget gate);
 *                            [B,T,H] with KDA_FLAG_SCALAR_GATE
 *   beta        [B,T,H]      fp32 in [0,1]
 *   mask        [B,T]        uint8 0/1, NULL = every position valid
 *   init_state  [B,H,dk,dv]  fp32, NULL = zeros
 *   o           [B,T,H,dv]   dtype, written (0 at masked positions)
 *   final_state [B,H,dk,dv]  fp32, written; may be the same pointer as init_state
 *
 * Supported: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64} (128 and 256,
 * the pages' 256-token chunks included, return KDA_ERR_UNSUPPORTED: their decay
 * factors leave the fp32 range with this kernel's chunk-start factorisation and
 * their inverse does not fit the LDS; chunk 16 runs its 16-token chunks in the
 * 32-row tiles of chunk 32, the upper rows masked, so it costs a chunk-32 step per
 * 16 tokens and exists for chunk-size audits rather than speed); B, H <= 65535; H times the number of
 * chunks < 2^24 and B*H <= 2^20 - 8, so every launch's extent in threads fits 32
 * bits (KDA_ERR_UNSUPPORTED otherwise, and a workspace size of 0);
 * T >= 0 (T = 0 copies init_state to final_state).  16-byte aligned: q, k, v,
 * and log_alpha unless KDA_FLAG_SCALAR_GATE is set.  The ragged tail of the last chunk is handled as masked
 * positions.  `flags` may hold KDA_FLAG_L2NORM_QK, KDA_FLAG_SCALAR_GATE and KDA_FLAG_SERIAL_SCAN.
 *
 * Segmented scan.  With bf16 inputs, dv = 128 and fewer than 64 (b, h) pairs, a long
 * enough sequence (at least 128 chunks) is scanned as G = 2, 4, ... segments side by side
 * when its gates forget fast enough: the state entering segment g is taken as the run from a
 * zero state over the shortest tail of chunks before it whose per-token contraction bounds
 * (max over the key channels of alpha, times max(1, |1 - beta |k|^2|): the norm of one
 * step's state map) multiply to at most 2^-160, which changes that state by at most 2^-160
 * of the norm of the state entering the tail, below 2^-25 in absolute value for any finite
 * fp32 state.  A head for which some boundary has no such tail inside the segment before
 * it is scanned as one chain, so every input gets a result within rounding of the token
 * recurrence; the segmented one differs from the single chain's by rounding only.  A
 * non-finite value at a valid position (outside this contract) turns the single chain's
 * state into NaN from that token on, while a later segment whose tail does not reach it
 * starts from zero and stays finite: callers that detect bad inputs through the final
 * state set KDA_FLAG_SERIAL_SCAN.  Masked positions count as the identity in the bound and
 * their values are never read.  The call stays asynchronous (the choice is made on the
 * device).  KDA_FLAG_SERIAL_SCAN turns
 * it off, e.g. to get results equal bit for bit to the state-saving calls.
 * workspace/workspace_bytes: at least kda_chunk_prefill_workspace_size(...)
 * bytes of device memory (may be NULL when that size is 0).
 */
int kda_chunk_prefill(const void* q, const void* k, const void* v,
                      const float* log_alpha, const float* beta, const uint8_t* mask,
                      const float* init_state, void* o, float* final_state,
                      int B, int T, int H, int dk, int dv, int chunk, int dtype,
                      unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill that also saves the state every state_interval tokens of each row,
 * for prefix caching in the batch layout and for training: with state_interval = 64 these
 * are the chunk-end states kda_chunk_prefill_backward takes instead of running the
 * forward again (the state recurrence of the Kimi Linear summary page, read at chunk
 * boundaries).  Arguments, results, supported sizes and the workspace are those of
 * kda_chunk_prefill (kda_chunk_prefill_workspace_size), with each (b, h) scanned as one
 * chain (as with KDA_FLAG_SERIAL_SCAN), plus:
 *
 *   chunk_states [M,H,dk,dv] fp32, written, or NULL (then the call is kda_chunk_prefill):
 *                            row b's state after its first j * state_interval tokens,
 *                            j = 1 .. floor(T / state_interval), at entry
 *                            b * floor(T / state_interval) + j - 1; masked positions leave
 *                            the state as it is, so the saved states count them as tokens
 *   num_states               entries chunk_states holds (>= 0); entries past it are not
 *                            written (M = B * floor(T / state_interval) holds them all)
 *   state_interval           a positive multiple of chunk
 *
 * chunk_states 4-byte aligned (16-byte when handed to kda_chunk_prefill_backward);
 * KDA_ERR_INVALID_ARG for a bad interval or a negative num_states.
 */
int kda_chunk_prefill_states(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const uint8_t* mask,
                             const float* init_state, void* o, float* final_state,
                             float* chunk_states, int num_states, int state_interval,
                             int B, int T, int H, int dk, int dv, int chunk, int dtype,
                             unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * results and supported sizes are those of kda_chunk_prefill, without the workspace:
 * the call uses a scratch array that the library holds on each GPU (allocated with the
 * library's code on that device, kept until the process ends) and calls no allocating
 * routine.  Its size is kda_noalloc_scratch_bytes() (256 MiB); a call whose
 * kda_chunk_prefill_workspace_size(...) exceeds it returns KDA_ERR_WORKSPACE before any
 * HIP call.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress, no allocation); make that first call outside graph capture.
 * Every call on one GPU shares that GPU's array: calls that can overlap on one GPU
 * (different streams, or different host threads without ordering) race and must not be
 * issued; calls in order on one stream are fine.  Nothing in the array needs clearing
 * between calls (every byte a call reads there was written earlier in that call).
 */
int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta, const uint8_t* mask,
                              const float* init_state, void* o, float* final_state,
                              int B, int T, int H, int dk, int dv, int chunk, int dtype,
                              unsigned flags, void* stream);

/* Bytes of the per-GPU scratch array of kda_chunk_prefill_noalloc. */
size_t kda_noalloc_scratch_bytes(void);

/*
 * Bytes of device workspace kda_chunk_prefill_varlen needs for N packed
 * sequences of T tokens in total (0 when none is needed; 0 as well for
 * arguments that the call itself would reject).  It depends on N and T only,
 * not on how the tokens are split between the sequences.
 */
size_t kda_chunk_prefill_varlen_workspace_size(int N, int T, int H, int dk, int dv, int chunk,
                                               int dtype);

/*
 * Chunked prefill of N sequences of different lengths packed end to end
 * without padding (continuous batching and prefix reuse are what serving
 * stacks must support without breaking KDA: remio.ai page, sections on the
 * software-stack risk and on what to watch after the release).  Sequence i
 * owns tokens [cu_seqlens[i], cu_seqlens[i+1]) of the packed arrays and runs
 * the recurrence above from init_state[i] over those tokens only: no state or
 * output crosses a boundary (dev.to prefix-invariance page: the output at a
 * position depends on its own prefix and nothing else).  Each sequence's
 * chunks start at its first token.  With fewer than 64 (sequence, head) pairs a long
 * sequence is cut into segments exactly as kda_chunk_prefill would cut it run alone (the
 * same rule on its chunk count and H, the same plan from its own inputs; see the segmented
 * scan of kda_chunk_prefill), so its results equal those of kda_chunk_prefill on that
 * sequence alone with the same chunk and flags, bit for bit.  With 64 pairs or more, with
 * checkpoints (state_interval > 0) or with KDA_FLAG_SERIAL_SCAN every sequence is scanned as
 * one chain, equal to its lone run with KDA_FLAG_SERIAL_SCAN.
 *
 *   q, k        [T,H,dk]     dtype (T = total tokens)
 *   v           [T,H,dv]     dtype
 *   log_alpha   [T,H,dk]     fp32, finite, <= 0; [T,H] with KDA_FLAG_SCALAR_GATE
 *   beta        [T,H]        fp32 in [0,1]
 *   cu_seqlens  [N+1]        int32 device array, cu_seqlens[0] = 0,
 *                            non-decreasing, cu_seqlens[N] = T
 *   init_state  [N,H,dk,dv]  fp32, NULL = zeros ([num_slots,H,dk,dv] with slot)
 *   o           [T,H,dv]     dtype, written
 *   final_state [N,H,dk,dv]  fp32, written; may be the same pointer as init_state
 *                            ([num_slots,H,dk,dv] with slot)
 *   slot        [N]          int32 device array, or NULL: with it init_state and
 *                            final_state are a pool of num_slots states (usually one
 *                            pointer, as for kda_decode_step_fused) and sequence i
 *                            reads and writes entry slot[i].  A slot outside
 *                            [0, num_slots) starts from zero and keeps no final state.
 *                            Two sequences must not share a slot (they would race).
 *   chunk_states [M,H,dk,dv] fp32, written, or NULL: state checkpoints for prefix
 *                            caching (remio.ai page, software-stack section: prefix
 *                            caching and the state at chunk boundaries are named among
 *                            what to test).  Sequence i of length L_i saves the state
 *                            after each of its first j * state_interval tokens,
 *                            j = 1 .. floor(L_i / state_interval), in that order, at
 *                            entries sum_{i' < i} floor(L_i' / state_interval) + j - 1;
 *                            M is that sum over all sequences.  Passing checkpoint j as
 *                            init_state for the rest of the sequence continues it bit
 *                            for bit.
 *   num_states               entries chunk_states holds (>= M); checkpoints past it
 *                            are not written
 *   state_interval           tokens between checkpoints: a positive multiple of chunk
 *   (num_states and state_interval are ignored when chunk_states is NULL)
 *
 * Every token is valid (there is no mask: a packed batch has no padding).  A
 * sequence of length 0 copies its init_state to final_state.  cu_seqlens is
 * read on the device, not on the host: entries outside [0, T] are clamped
 * into it and a decreasing entry gives an empty sequence, so a malformed
 * array gives wrong results but no out-of-bounds access (checkpoints included,
 * as num_states bounds them; slots, as num_slots bounds them).  Supported: as
 * kda_chunk_prefill with B = N (N <= 65535), H times (ceil(T/chunk) + N)
 * < 2^24 and N*H <= 2^20 - 8.  16-byte aligned: q, k, v, and log_alpha unless KDA_FLAG_SCALAR_GATE
 * is set; chunk_states and slot 4-byte aligned.  `flags` may hold
 * KDA_FLAG_L2NORM_QK and KDA_FLAG_SCALAR_GATE.
 */
int kda_chunk_prefill_varlen(const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const int32_t* cu_seqlens,
                             const float* init_state, void* o, float* final_state,
                             const int32_t* slot, int num_slots,
                             float* chunk_states, int num_states, int state_interval,
                             int N, int T, int H, int dk, int dv, int chunk, int dtype,
                             unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace kda_chunk_prefill_backward needs (0 when none is needed or
 * the arguments would be rejected): flags as for the call; states_given != 0 for calls that
 * pass chunk_states (the forward's workspace, outputs and states are then not needed).
 */
size_t kda_chunk_prefill_backward_workspace_size(int B, int T, int H, int dk, int dv, int dtype,
                                                 unsigned flags, int states_given);

/*
 * Gradients of kda_chunk_prefill for training (remio.ai page, KDA section: the model is
 * trained with a blockwise algorithm).  For the scalar loss
 *     L = sum_t <d_o[t], o[t]> + <d_final_state, final_state>
 * of one prefill with the same inputs, writes dL/dq, dL/dk, dL/dv, dL/dlog_alpha,
 * dL/dbeta and dL/dinit_state.  Masked positions get zero gradients and pass the state's
 * gradient through.
 *
 *   q, k, v, log_alpha, beta, mask, init_state   as for kda_chunk_prefill
 *   chunk_states  [B*floor(T/64),H,dk,dv]  fp32, or NULL: the state at every 64-token
 *                              boundary as kda_chunk_prefill_states writes it with
 *                              state_interval = 64 on the same inputs (any chunk; with
 *                              chunk = 64 the gradients equal those of a NULL call bit for
 *                              bit).  NULL: the call runs the forward again to form them.
 *   d_o           [B,T,H,dv]   dtype
 *   d_final_state [B,H,dk,dv]  fp32, or NULL (zero)
 *   dq, dk        [B,T,H,dk]   fp32, written
 *   dv            [B,T,H,dv]   fp32, written
 *   d_log_alpha   [B,T,H,dk]   fp32, written ([B,T,H] with KDA_FLAG_SCALAR_GATE)
 *   d_beta        [B,T,H]      fp32, written
 *   d_init_state  [B,H,dk,dv]  fp32, written (also when init_state is NULL: the gradient
 *                              with respect to the zero state)
 *
 * Without chunk_states it runs the forward again in 64-token chunks, keeping the state at
 * each chunk end; then a reverse scan over the chunks carries dL/dS (the chunk recurrence
 * differentiated)
 * and chunk-parallel kernels form the gradients; every sum accumulates in fp32, with
 * MFMA operands split into bf16 high and low parts (single bf16 for the reverse scan's
 * key, query and W operands with bf16 inputs, as in the forward scan).  The workspace
 * holds about 250 KB of chunk operands per (b, h, chunk) at dk = dv = 128; without
 * chunk_states, the forward's own workspace, outputs and chunk-end states; with
 * KDA_FLAG_SCALAR_GATE, the gate's per-channel gradient before the sum over the channels
 * (dk floats per token and head).
 *
 * Supported: dk, dv in {16, 32, 64, 128}; B, H <= 65535, H ceil(T/64) < 2^24, B*H <= 2^20 - 8
 * and B*H*ceil(T/64) <= 2^22 - 8 (launch extents in threads fit 32 bits);
 * flags may hold KDA_FLAG_SCALAR_GATE (Gated DeltaNet's gate, one value per (token, head):
 * the gate is applied to every channel and its gradient is the sum over the channels, so
 * given the same chunk_states the other gradients equal those of a per-channel call fed the
 * broadcast gate bit for bit; without them the call runs the per-head prefill)
 * and KDA_FLAG_L2NORM_QK (the gradients of the prefill that normalises q and k with that
 * flag: the pass runs on the normalised rows, formed as the forward forms them, and dq, dk
 * are taken back to the raw rows at the end, dx = s dx_hat - s^3 x (x . dx_hat) with
 * s = (|x|^2 + 1e-6)^-1/2; the workspace holds the two row scales, 8 bytes per token and
 * head; chunk_states must then come from a forward with the flag); other bits
 * KDA_ERR_INVALID_ARG.
 * 16-byte aligned: q, k, v, d_o, init_state, chunk_states, dq, dk, dv, and log_alpha and
 * d_log_alpha unless KDA_FLAG_SCALAR_GATE is set (then 4-byte); 4-byte: beta, d_beta,
 * d_final_state, d_init_state; workspace 256-byte aligned.
 * Outputs must not overlap inputs.
 */
int kda_chunk_prefill_backward(const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const uint8_t* mask,
                               const float* init_state, const float* chunk_states,
                               const void* d_o, const float* d_final_state,
                               float* dq, float* dk, float* dv, float* d_log_alpha, float* d_beta,
                               float* d_init_state, int B, int T, int H, int dk_, int dv_, int dtype,
                               unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace kda_chunk_prefill_varlen_backward needs for N packed sequences of
 * T tokens in total (0 when none is needed or the arguments would be rejected); flags and
 * states_given as for kda_chunk_prefill_backward_workspace_size.  It depends on N and T only,
 * not on how the tokens are split between the sequences.
 */
size_t kda_chunk_prefill_varlen_backward_workspace_size(int N, int T, int H, int dk, int dv, int dtype,
                                                        unsigned flags, int states_given);

/*
 * Gradients of kda_chunk_prefill_varlen (without slots) for training on packed sequences: the
 * backward above for N sequences of different lengths packed end to end (the remio.ai page
 * names continuous batching among what a serving and training stack must support for KDA;
 * its KDA section, the blockwise training algorithm).  For the loss
 *     L = sum_t <d_o[t], o[t]> + sum_i <d_final_state[i], final_state[i]>
 * sequence i's gradients depend on its own tokens, d_o rows and d_final_state[i] only, and
 * equal those of kda_chunk_prefill_backward on that sequence alone (B = 1, same inputs) bit for
 * bit: each sequence's 64-token chunks start at its first token.
 *
 *   q, k, v, log_alpha, beta, cu_seqlens, init_state   as for kda_chunk_prefill_varlen
 *                              ([T,H,...] packed; init_state [N,H,dk,dv] or NULL)
 *   chunk_states  [M,H,dk,dv]  fp32, or NULL: the checkpoints kda_chunk_prefill_varlen writes
 *                              with state_interval = 64 on the same inputs (sequence i's state
 *                              after each of its first j * 64 tokens at entry
 *                              sum_{i' < i} floor(L_i' / 64) + j - 1).  NULL: the call runs the
 *                              forward again to form them.
 *   num_states                 entries chunk_states holds (>= M; ignored when it is NULL); an
 *                              entry past it is read as a zero state
 *   d_o           [T,H,dv]     dtype
 *   d_final_state [N,H,dk,dv]  fp32, or NULL (zero)
 *   dq, dk        [T,H,dk]     fp32, written
 *   dv            [T,H,dv]     fp32, written
 *   d_log_alpha   [T,H,dk]     fp32, written ([T,H] with KDA_FLAG_SCALAR_GATE)
 *   d_beta        [T,H]        fp32, written
 *   d_init_state  [N,H,dk,dv]  fp32, written
 *
 * A sequence of length 0 gets d_init_state[i] = d_final_state[i].  cu_seqlens is read on the
 * device: entries are clamped as for kda_chunk_prefill_varlen, so a malformed array gives
 * wrong (or unwritten) gradients but no access outside a buffer.  The workspace adds to that
 * of kda_chunk_prefill_backward a sequence table (16 bytes per sequence) and a chunk table
 * (8 bytes per chunk slot), and holds ceil(T/64) + N chunk slots per head.
 * Supported: as kda_chunk_prefill_backward with B = N (N <= 65535, N*H <= 2^20 - 8) and
 * H (ceil(T/64) + N) <= 2^22 - 8 in place of its chunk bounds; flags and alignment as there,
 * cu_seqlens 4-byte aligned.
 * Outputs must not overlap inputs.
 */
int kda_chunk_prefill_varlen_backward(const void* q, const void* k, const void* v,
                                      const float* log_alpha, const float* beta,
                                      const int32_t* cu_seqlens, const float* init_state,
                                      const float* chunk_states, int num_states,
                                      const void* d_o, const float* d_final_state,
                                      float* dq, float* dk, float* dv, float* d_log_alpha,
                                      float* d_beta, float* d_init_state, int N, int T, int H,
                                      int dk_, int dv_, int dtype, unsigned flags,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step: a single new token per sequence, state updated in place
 * (remio.ai page, decode section: KDA keeps a fixed-size state, so each
 * generated token reads and rewrites that state once).
 *
 *   q, k        [B,H,dk]     dtype
 *   v           [B,H,dv]     dtype
 *   log_alpha   [B,H,dk]     fp32 ([B,H] with KDA_FLAG_SCALAR_GATE)
 *   beta        [B,H]        fp32
 *   mask        [B]          uint8 0/1, NULL = all valid (0 leaves S untouched, o = 0)
 *   state       [B,H,dk,dv]  fp32, read and written in place
 *   o           [B,H,dv]     dtype, written
 *
 * Supported: dk, dv in {16, 32, 64, 128}; B, H >= 0.  `flags` may hold
 * KDA_FLAG_L2NORM_QK and KDA_FLAG_SCALAR_GATE.  16-byte aligned: state.
 */
int kda_decode_step(const void* q, const void* k, const void* v,
                    const float* log_alpha, const float* beta, const uint8_t* mask,
                    float* state, void* o, int B, int H, int dk, int dv, int dtype,
                    unsigned flags, void* stream);

/*
 * Depthwise causal short convolution with a cache, over the compacted
 * sequence of valid positions (Transformers issue report on Kimi Linear:
 * padded entries must not enter the convolution window).  Per sequence b and
 * channel c, let x~ be [the W-1 cached inputs (oldest first), then x at the
 * valid positions in order].  At a valid position t that is the m-th valid one,
 *     y[b,t,c] = bias[c] + sum_{j=0}^{W-1} weight[c,j] * x~[m + j]
 * (weight[c,W-1] multiplies the current input), optionally passed through SiLU;
 * y = 0 at masked positions.  The cache then holds the last W-1 entries of x~.
 *
 *   x           [B,T,D]      dtype
 *   weight      [D,W]        fp32
 *   bias        [D]          fp32 or NULL
 *   mask        [B,T]        uint8 0/1 or NULL
 *   conv_cache  [B,W-1,D]    dtype, read then overwritten; NULL = zero history, not written
 *   y           [B,T,D]      dtype, written; must not overlap x or conv_cache
 *
 * Supported: W in {2, 3, 4}; D >= 1, D a multiple of 8; T >= 0.  `flags` may
 * hold KDA_FLAG_SILU.  16-byte aligned: x, y, conv_cache.
 */
int kda_short_conv(const void* x, const float* weight, const float* bias, const uint8_t* mask,
                   void* conv_cache, void* y, int B, int T, int D, int W, int dtype,
                   unsigned flags, void* stream);

/*
 * Fused decode step for a serving loop: per sequence b (one new token) the three
 * short convolutions at T = 1 of kda_short_conv (with their caches), the optional
 * q/k L2 norm and the state update of kda_decode_step, in one launch; sequence b's
 * state is slot[b] of a pool (remio.ai page on Kimi Linear, decode section: each KDA
 * layer keeps a fixed-size recurrent state per sequence; closing paragraphs: serving
 * stacks need continuous batching that keeps KDA's state handling correct).  The conv
 * outputs are rounded to `dtype` before the update, as kda_short_conv stores them, so
 * the result equals three kda_short_conv calls followed by kda_decode_step bit for bit.
 *
 *   xq, xk      [B,H*dk]     dtype, raw inputs of the q and k convolutions
 *   xv          [B,H*dv]     dtype, raw input of the v convolution
 *   wq, wk      [H*dk,W]     fp32;  wv [H*dv,W] fp32
 *   bq, bk, bv  [H*dk], [H*dk], [H*dv]  fp32 or NULL (no bias)
 *   cache_q, cache_k [B,W-1,H*dk], cache_v [B,W-1,H*dv]   dtype, read then shifted
 *   log_alpha   [B,H,dk]     fp32 ([B,H] with KDA_FLAG_SCALAR_GATE)
 *   beta        [B,H]        fp32
 *   mask        [B]          uint8 0/1 or NULL; 0 leaves caches and state untouched, o = 0
 *   state       [S,H,dk,dv]  fp32 pool, slot slot[b] read and written in place
 *   slot        [B]          int32 or NULL (sequence b uses slot b; then S >= B).  The
 *                            slots of the valid sequences must be distinct; a slot
 *                            outside [0, S) is treated like a masked sequence.
 *   o           [B,H,dv]     dtype, written
 * No output may overlap an input.  Supported: dk, dv in {16, 32, 64, 128};
 * W in {2, 3, 4}.  `flags` may hold KDA_FLAG_L2NORM_QK, KDA_FLAG_SILU (SiLU after
 * each convolution) and KDA_FLAG_SCALAR_GATE.  16-byte aligned: state.
 */
int kda_decode_step_fused(const void* xq, const void* xk, const void* xv,
                          const float* wq, const float* wk, const float* wv,
                          const float* bq, const float* bk, const float* bv,
                          void* cache_q, void* cache_k, void* cache_v,
                          const float* log_alpha, const float* beta, const uint8_t* mask,
                          float* state, const int32_t* slot, void* o,
                          int B, int H, int S, int dk, int dv, int W, int dtype,
                          unsigned flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
