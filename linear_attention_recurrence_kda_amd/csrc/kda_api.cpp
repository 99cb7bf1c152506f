// C ABI of libkda (declared in include/kda.h): argument validation on the
// host, then dispatch to the gfx950 kernel launchers.  Nothing here allocates
// or synchronises; a rejected call makes no HIP call at all.
#include "kda.h"

#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }
uintptr_t elem_bytes(int dt) { return dt == KDA_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == KDA_BF16 || dt == KDA_F32; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  g_last_hip_error = (int)e;
  return KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null, negative or misaligned argument";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size, chunk or width outside the supported set";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed (see kda_last_hip_error)";
    default: return "unknown kda_status";
  }
}

int kda_last_hip_error(void) { return g_last_hip_error; }

size_t kda_chunk_prefill_workspace_size(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (B < 0 || T < 0 || H < 0 || !dtype_ok(dtype)) return 0;
  if (!head_dim_ok(dk) || !head_dim_ok(dv) || !kda::prefill_supported(dk, dv, chunk) || H > 65535 || B > 65535 ||
      !kda::prefill_grid_ok(B, T, H, chunk, false))
    return 0;
  return kda::prefill_workspace_bytes(B, T, H, dk, dv, chunk, dtype, false);
}

size_t kda_chunk_prefill_varlen_workspace_size(int N, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (N < 0 || T < 0 || H < 0 || !dtype_ok(dtype)) return 0;
  if (!head_dim_ok(dk) || !head_dim_ok(dv) || !kda::prefill_supported(dk, dv, chunk) || H > 65535 || N > 65535 ||
      !kda::prefill_grid_ok(N, T, H, chunk, true))
    return 0;
  return kda::prefill_workspace_bytes(N, T, H, dk, dv, chunk, dtype, true);
}

// The checks and the launch shared by the batch layout (B rows of T tokens, optional mask)
// and the packed layout (B sequences of T tokens in total, cu_seqlens given).
static int prefill_entry(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const uint8_t* mask, const int32_t* cu_seqlens, bool varlen,
                         const float* init_state, void* o, float* final_state, const int32_t* slot,
                         int num_slots, float* chunk_states, int num_states, int state_interval, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                         unsigned flags, void* workspace, size_t workspace_bytes, void* stream,
                         bool use_scratch = false) {
  if (B < 0 || T < 0 || H < 0 || !dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
  if ((flags & ~(unsigned)(KDA_FLAG_L2NORM_QK | KDA_FLAG_SCALAR_GATE | KDA_FLAG_SERIAL_SCAN)) != 0)
    return KDA_ERR_INVALID_ARG;
  if (!head_dim_ok(dk) || !head_dim_ok(dv) || !kda::prefill_supported(dk, dv, chunk) || H > 65535 || B > 65535 ||
      !kda::prefill_grid_ok(B, T, H, chunk, varlen))
    return KDA_ERR_UNSUPPORTED;
  const bool work = (size_t)B * H > 0;
  if (work) {
    if (final_state == nullptr || !aligned(final_state, 4)) return KDA_ERR_INVALID_ARG;
    if (init_state != nullptr && !aligned(init_state, 4)) return KDA_ERR_INVALID_ARG;
    if (varlen && (cu_seqlens == nullptr || !aligned(cu_seqlens, 4))) return KDA_ERR_INVALID_ARG;
    if (slot != nullptr && (!aligned(slot, 4) || num_slots < 0)) return KDA_ERR_INVALID_ARG;
    if (chunk_states != nullptr && (!aligned(chunk_states, 4) || num_states < 0 || state_interval <= 0 ||
                                    state_interval % chunk != 0))
      return KDA_ERR_INVALID_ARG;
    if (T > 0) {
      // q, k, v and the per-channel log_alpha are read with 16-byte vector loads; the rest,
      // the per-head gate included, element by element
      const void* vec[] = {q, k, v};
      for (const void* p : vec)
        if (p == nullptr || !aligned16(p)) return KDA_ERR_INVALID_ARG;
      if (o == nullptr || beta == nullptr || log_alpha == nullptr) return KDA_ERR_INVALID_ARG;
      if (!aligned(log_alpha, (flags & KDA_FLAG_SCALAR_GATE) ? 4 : 16)) return KDA_ERR_INVALID_ARG;
      if (!aligned(o, elem_bytes(dtype)) || !aligned(beta, 4)) return KDA_ERR_INVALID_ARG;
    }
  }
  const size_t need = kda::prefill_workspace_bytes(B, T, H, dk, dv, chunk, dtype, varlen);
  if (use_scratch) {
    // the library's per-device scratch array stands in for the workspace: no allocation
    if (need > kda::kNoallocScratchBytes) return KDA_ERR_WORKSPACE;
    if (need > 0 && work) {
      void* p = nullptr;
      const hipError_t e = kda::noalloc_scratch(&p);
      if (e != hipSuccess) return hip_status(e);
      workspace = p;
      workspace_bytes = kda::kNoallocScratchBytes;
    }
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return KDA_ERR_WORKSPACE;
  if (!work) return KDA_OK;
  kda::PrefillArgs a{q, k, v, log_alpha, beta, mask, init_state, o, final_state,
                     B, T, H, dk, dv, chunk, dtype, (flags & KDA_FLAG_L2NORM_QK) ? 1 : 0,
                     (flags & KDA_FLAG_SCALAR_GATE) ? 1 : 0, workspace, workspace_bytes, stream,
                     varlen ? cu_seqlens : nullptr, chunk_states, chunk_states != nullptr ? num_states : 0,
                     chunk_states != nullptr ? state_interval : 0, slot, slot != nullptr ? num_slots : 0,
                     (flags & KDA_FLAG_SERIAL_SCAN) ? 1 : 0};
  return hip_status(kda::launch_prefill(a));
}

int kda_chunk_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const uint8_t* mask, const float* init_state, void* o,
                      float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                      unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry(q, k, v, log_alpha, beta, mask, nullptr, false, init_state, o, final_state, nullptr, 0, nullptr, 0, 0,
                       B, T, H, dk, dv, chunk, dtype, flags, workspace, workspace_bytes, stream);
}

int kda_chunk_prefill_states(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const uint8_t* mask, const float* init_state, void* o,
                             float* final_state, float* chunk_states, int num_states, int state_interval,
                             int B, int T, int H, int dk, int dv, int chunk, int dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry(q, k, v, log_alpha, beta, mask, nullptr, false, init_state, o, final_state, nullptr, 0,
                       chunk_states, num_states, state_interval, B, T, H, dk, dv, chunk, dtype, flags, workspace,
                       workspace_bytes, stream);
}

int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* beta, const uint8_t* mask, const float* init_state, void* o,
                              float* final_state, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                              unsigned flags, void* stream) {
  return prefill_entry(q, k, v, log_alpha, beta, mask, nullptr, false, init_state, o, final_state, nullptr, 0, nullptr, 0, 0,
                       B, T, H, dk, dv, chunk, dtype, flags, nullptr, 0, stream, true);
}

size_t kda_noalloc_scratch_bytes(void) { return kda::kNoallocScratchBytes; }

int kda_chunk_prefill_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const int32_t* cu_seqlens, const float* init_state,
                             void* o, float* final_state, const int32_t* slot, int num_slots,
                             float* chunk_states, int num_states, int state_interval, int N, int T, int H, int dk, int dv, int chunk, int dtype, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry(q, k, v, log_alpha, beta, nullptr, cu_seqlens, true, init_state, o, final_state,
                       slot, num_slots, chunk_states, num_states, state_interval, N, T, H, dk, dv, chunk, dtype, flags, workspace,
                       workspace_bytes, stream);
}

// the batch and packed backward calls: the same checks, the packed one with cu_seqlens
// (B = sequences, T = packed tokens, no mask) and the count of the checkpoints it is given
static bool backward_shape_ok(int B, int T, int H, int dk, int dv, bool varlen) {
  return head_dim_ok(dk) && head_dim_ok(dv) && B <= 65535 && H <= 65535 &&
         kda::prefill_grid_ok(B, T, H, 64, varlen) && kda::backward_grid_ok(B, T, H, varlen);
}

static size_t backward_size(int B, int T, int H, int dk, int dv, int dtype, unsigned flags, int states_given,
                            bool varlen) {
  if (B < 0 || T < 0 || H < 0 || !dtype_ok(dtype) || !backward_shape_ok(B, T, H, dk, dv, varlen) ||
      (flags & ~(unsigned)(KDA_FLAG_SCALAR_GATE | KDA_FLAG_L2NORM_QK)) != 0)
    return 0;
  return kda::backward_workspace_bytes(B, T, H, dk, dv, dtype, states_given != 0,
                                       (flags & KDA_FLAG_SCALAR_GATE) != 0, varlen,
                                       (flags & KDA_FLAG_L2NORM_QK) != 0);
}

static int backward_entry(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const uint8_t* mask, const int32_t* cu_seqlens, bool varlen,
                          const float* init_state, const float* chunk_states, int num_states, const void* d_o,
                          const float* d_final_state, float* dq, float* dk, float* dv, float* d_log_alpha,
                          float* d_beta, float* d_init_state, int B, int T, int H, int dk_, int dv_, int dtype,
                          unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || H < 0 || !dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
  if ((flags & ~(unsigned)(KDA_FLAG_L2NORM_QK | KDA_FLAG_SCALAR_GATE)) != 0) return KDA_ERR_INVALID_ARG;
  const bool sg = (flags & KDA_FLAG_SCALAR_GATE) != 0, l2 = (flags & KDA_FLAG_L2NORM_QK) != 0;
  if (!backward_shape_ok(B, T, H, dk_, dv_, varlen)) return KDA_ERR_UNSUPPORTED;
  if ((size_t)B * H == 0) return KDA_OK;
  if (d_init_state == nullptr || !aligned(d_init_state, 4)) return KDA_ERR_INVALID_ARG;
  if (init_state != nullptr && !aligned(init_state, 16)) return KDA_ERR_INVALID_ARG;
  if (d_final_state != nullptr && !aligned(d_final_state, 4)) return KDA_ERR_INVALID_ARG;
  if (varlen && (cu_seqlens == nullptr || !aligned(cu_seqlens, 4))) return KDA_ERR_INVALID_ARG;
  if (varlen && chunk_states != nullptr && num_states < 0) return KDA_ERR_INVALID_ARG;
  if (T > 0) {
    const void* req[] = {q, k, v, log_alpha, beta, d_o, dq, dk, dv, d_log_alpha, d_beta};
    for (const void* ptr : req)
      if (ptr == nullptr) return KDA_ERR_INVALID_ARG;
    const void* a16[] = {q, k, v, d_o, dq, dk, dv};
    for (const void* ptr : a16)
      if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    // the per-channel gate and its gradient move in 16-byte vectors; one per head, as scalars
    if (!aligned(log_alpha, sg ? 4 : 16) || !aligned(d_log_alpha, sg ? 4 : 16)) return KDA_ERR_INVALID_ARG;
    if (!aligned(beta, 4) || !aligned(d_beta, 4)) return KDA_ERR_INVALID_ARG;
    // the chunk-end states are read with 16-byte vector loads
    if (chunk_states != nullptr && !aligned(chunk_states, 16)) return KDA_ERR_INVALID_ARG;
  }
  const size_t need =
      kda::backward_workspace_bytes(B, T, H, dk_, dv_, dtype, chunk_states != nullptr, sg, varlen, l2);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
    return KDA_ERR_WORKSPACE;
  kda::BackwardArgs a{q, k, v, d_o, log_alpha, beta, init_state, d_final_state, varlen ? nullptr : mask,
                      chunk_states, dq, dk, dv, d_log_alpha, d_beta, d_init_state, B, T, H, dk_, dv_, dtype,
                      sg ? 1 : 0, workspace, stream, varlen ? cu_seqlens : nullptr, num_states, l2 ? 1 : 0};
  return hip_status(kda::launch_backward(a));
}

size_t kda_chunk_prefill_backward_workspace_size(int B, int T, int H, int dk, int dv, int dtype,
                                                 unsigned flags, int states_given) {
  return backward_size(B, T, H, dk, dv, dtype, flags, states_given, false);
}

int kda_chunk_prefill_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const uint8_t* mask, const float* init_state,
                               const float* chunk_states, const void* d_o, const float* d_final_state, float* dq, float* dk,
                               float* dv, float* d_log_alpha, float* d_beta, float* d_init_state,
                               int B, int T, int H, int dk_, int dv_, int dtype, unsigned flags,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return backward_entry(q, k, v, log_alpha, beta, mask, nullptr, false, init_state, chunk_states, 0, d_o,
                        d_final_state, dq, dk, dv, d_log_alpha, d_beta, d_init_state, B, T, H, dk_, dv_, dtype,
                        flags, workspace, workspace_bytes, stream);
}

size_t kda_chunk_prefill_varlen_backward_workspace_size(int N, int T, int H, int dk, int dv, int dtype,
                                                        unsigned flags, int states_given) {
  return backward_size(N, T, H, dk, dv, dtype, flags, states_given, true);
}

int kda_chunk_prefill_varlen_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                                      const float* beta, const int32_t* cu_seqlens, const float* init_state,
                                      const float* chunk_states, int num_states, const void* d_o,
                                      const float* d_final_state, float* dq, float* dk, float* dv,
                                      float* d_log_alpha, float* d_beta, float* d_init_state, int N, int T, int H,
                                      int dk_, int dv_, int dtype, unsigned flags, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return backward_entry(q, k, v, log_alpha, beta, nullptr, cu_seqlens, true, init_state, chunk_states, num_states,
                        d_o, d_final_state, dq, dk, dv, d_log_alpha, d_beta, d_init_state, N, T, H, dk_, dv_,
                        dtype, flags, workspace, workspace_bytes, stream);
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, const uint8_t* mask, float* state, void* o, int B, int H,
                    int dk, int dv, int dtype, unsigned flags, void* stream) {
  if (B < 0 || H < 0 || !dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
  if ((flags & ~(unsigned)(KDA_FLAG_L2NORM_QK | KDA_FLAG_SCALAR_GATE)) != 0) return KDA_ERR_INVALID_ARG;
  if (!head_dim_ok(dk) || !head_dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if ((size_t)B * H == 0) return KDA_OK;
  const void* req[] = {q, k, v, log_alpha, beta, state, o};
  for (const void* p : req)
    if (p == nullptr) return KDA_ERR_INVALID_ARG;
  // the state is streamed with 16-byte vector accesses; the rest element by element
  if (!aligned16(state) || !aligned(log_alpha, 4) || !aligned(beta, 4)) return KDA_ERR_INVALID_ARG;
  const void* el[] = {q, k, v, o};
  for (const void* p : el)
    if (!aligned(p, elem_bytes(dtype))) return KDA_ERR_INVALID_ARG;
  kda::DecodeArgs a{q, k, v, log_alpha, beta, mask, state, o, B, H, dk, dv, dtype,
                    (flags & KDA_FLAG_L2NORM_QK) ? 1 : 0, (flags & KDA_FLAG_SCALAR_GATE) ? 1 : 0, stream};
  return hip_status(kda::launch_decode(a));
}

int kda_decode_step_fused(const void* xq, const void* xk, const void* xv, const float* wq,
                          const float* wk, const float* wv, const float* bq, const float* bk,
                          const float* bv, void* cache_q, void* cache_k, void* cache_v,
                          const float* log_alpha, const float* beta, const uint8_t* mask,
                          float* state, const int32_t* slot, void* o, int B, int H, int S, int dk,
                          int dv, int W, int dtype, unsigned flags, void* stream) {
  if (B < 0 || H < 0 || S < 0 || !dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
  if ((flags & ~(unsigned)(KDA_FLAG_L2NORM_QK | KDA_FLAG_SILU | KDA_FLAG_SCALAR_GATE)) != 0) return KDA_ERR_INVALID_ARG;
  if (!head_dim_ok(dk) || !head_dim_ok(dv) || W < 2 || W > 4) return KDA_ERR_UNSUPPORTED;
  if ((size_t)B * H == 0) return KDA_OK;
  if (slot == nullptr && S < B) return KDA_ERR_INVALID_ARG;          // sequence b uses slot b
  const void* req[] = {xq, xk, xv, wq, wk, wv, cache_q, cache_k, cache_v, log_alpha, beta, state, o};
  for (const void* p : req)
    if (p == nullptr) return KDA_ERR_INVALID_ARG;
  if (!aligned16(state) || !aligned(slot, 4)) return KDA_ERR_INVALID_ARG;
  const void* f32[] = {wq, wk, wv, bq, bk, bv, log_alpha, beta};
  for (const void* p : f32)
    if (!aligned(p, 4)) return KDA_ERR_INVALID_ARG;
  const void* el[] = {xq, xk, xv, cache_q, cache_k, cache_v, o};
  for (const void* p : el)
    if (!aligned(p, elem_bytes(dtype))) return KDA_ERR_INVALID_ARG;
  kda::FusedDecodeArgs a{xq, xk, xv, wq, wk, wv, bq, bk, bv, cache_q, cache_k, cache_v,
                         log_alpha, beta, mask, state, slot, o, B, H, S, dk, dv, W, dtype,
                         (flags & KDA_FLAG_L2NORM_QK) ? 1 : 0, (flags & KDA_FLAG_SILU) ? 1 : 0,
                         (flags & KDA_FLAG_SCALAR_GATE) ? 1 : 0, stream};
  return hip_status(kda::launch_decode_fused(a));
}

int kda_short_conv(const void* x, const float* weight, const float* bias, const uint8_t* mask,
                   void* conv_cache, void* y, int B, int T, int D, int W, int dtype, unsigned flags,
                   void* stream) {
  if (B < 0 || T < 0 || D <= 0 || !dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
  if ((flags & ~(unsigned)KDA_FLAG_SILU) != 0) return KDA_ERR_INVALID_ARG;
  if (W < 2 || W > 4 || D % 8 != 0) return KDA_ERR_UNSUPPORTED;
  if (B == 0) return KDA_OK;
  if (weight == nullptr) return KDA_ERR_INVALID_ARG;
  if (conv_cache != nullptr && !aligned16(conv_cache)) return KDA_ERR_INVALID_ARG;
  if (T > 0 && (x == nullptr || y == nullptr || !aligned16(x) || !aligned16(y))) return KDA_ERR_INVALID_ARG;
  if (T == 0) return KDA_OK;   // nothing to convolve; the cache keeps its contents
  kda::ConvArgs a{x, weight, bias, mask, conv_cache, y, B, T, D, W, dtype,
                  (flags & KDA_FLAG_SILU) ? 1 : 0, stream};
  return hip_status(kda::launch_short_conv(a));
}

}  // extern "C"
