// Internal interface between the C ABI (kda_api.cpp) and the kernel launchers.
// Every pointer here has already been validated by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  float* state;
  void* o;
  int B, H, dk, dv, dtype, l2norm, scalar_gate;
  void* stream;
};

// the three short convs at T = 1, the optional q/k L2 norm and the state update of one
// decode step, with the state taken from a pool of slots
struct FusedDecodeArgs {
  const void *xq, *xk, *xv;                // raw conv inputs [B, H*dk] / [B, H*dv]
  const float *wq, *wk, *wv;               // conv weights [D, W]
  const float *bq, *bk, *bv;               // conv biases [D] or null
  void *cq, *ck, *cv;                      // conv caches [B, W-1, D], updated
  const float *log_alpha, *beta;
  const uint8_t* mask;
  float* state;                            // [S, H, dk, dv]
  const int32_t* slot;                     // [B] or null (slot b)
  void* o;
  int B, H, S, dk, dv, W, dtype, l2norm, silu, scalar_gate;
  void* stream;
};

struct ConvArgs {
  const void* x;
  const float *weight, *bias;
  const uint8_t* mask;
  void* cache;
  void* y;
  int B, T, D, W, dtype, silu;
  void* stream;
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  const float* init_state;
  void* o;
  float* final_state;
  int B, T, H, dk, dv, chunk, dtype, l2norm, scalar_gate;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  const int32_t* cu_seqlens;               // packed sequences (then B = their number), or null
  float* chunk_states;                     // the state every state_interval tokens, or null (the batch
                                           // layout saves entry b * (T / state_interval) + j - 1)
  int num_states;                          // entries chunk_states holds
  int state_interval;                      // a multiple of chunk
  const int32_t* slot;                     // packed only: each sequence's slot in a state pool, or null
  int num_slots;                           // slots in the pool
  int serial_scan;                         // 1: each (b, h) as one chain, never segmented
};

// gradients of the prefill (see kda_backward.hip)
struct BackwardArgs {
  const void *q, *k, *v, *dout;
  const float *log_alpha, *beta, *init_state, *dfinal;
  const uint8_t* mask;
  const float* chunk_states;               // the forward's state at every 64-token chunk end, or
                                           // null (the forward runs again inside the call)
  float *dq, *dk, *dv, *dla, *dbeta, *dinit;
  int B, T, H, dk_, dv_, dtype;
  int scalar_gate;                         // log_alpha and dla are [B,T,H]: one gate per head
  void* workspace;
  void* stream;
  const int32_t* cu_seqlens;               // packed sequences (then B = their number, no mask), or null
  int num_states;                          // packed: entries chunk_states holds
  int l2norm;                              // q and k normalised inside the call (as the forward's flag)
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_backward(const BackwardArgs& a);
// varlen: B packed sequences of T tokens in total
size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype, bool states_given,
                                bool scalar_gate, bool varlen, bool l2);
// every backward launch's grid fits (the forward inside it is checked by prefill_grid_ok)
bool backward_grid_ok(int B, int T, int H, bool varlen);
hipError_t launch_short_conv(const ConvArgs& a);
hipError_t launch_decode_fused(const FusedDecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
// bytes of the per-device scratch array of kda_chunk_prefill_noalloc
constexpr size_t kNoallocScratchBytes = (size_t)256 << 20;
// the current device's scratch array (device address), resolved on first use per device
hipError_t noalloc_scratch(void** ptr);
// varlen: B packed sequences of T tokens in total (cu_seqlens given)
size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype, bool varlen);
bool prefill_supported(int dk, int dv, int chunk);
// every prefill launch's grid fits: H times the chunks, and the scan's B*H workgroup rows
bool prefill_grid_ok(int B, int T, int H, int chunk, bool varlen);

}  // namespace kda
