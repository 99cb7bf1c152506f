// Chunked prefill of the KDA recurrence on gfx950 (Kimi Linear summary page,
// paragraph on the kernels: sequences are split into chunks and each chunk's
// batch of rank-1 updates goes through a WY representation, i.e. a triangular
// solve; remio.ai page, KDA section: the diagonal-plus-low-rank transition is
// what makes the blockwise form efficient).
//
// Chunk form used here (derived from the token recurrence).  Inside a chunk
// starting from state S0, G is the inclusive cumulative sum of log_alpha from
// the chunk start (per key channel), Gam = exp(G), Kt = K*Gam, Ki = K/Gam,
// Qt = Q*Gam, Kh = K*Gam_last/Gam:
//   A  = strict_lower(Diag(beta) Kt Ki^T)      P = lower(Qt Ki^T)
//   T' = (I + A)^-1 Diag(beta)                 (unit lower-triangular solve, fp32)
//   Wn = -T' Kt
//   U  = T' V + Wn S0                          (per-token corrections)
//   O  = Qt S0 + P U
//   S1 = Diag(Gam_last) S0 + Kh^T U
// (O = Qt S0 + P U is the token read-out q_t^T S_t summed up: P U adds the chunk's own
// updates to what the decayed entry state gives.)  Nothing before the last three lines
// depends on the state or on V, so the work splits into:
//   prep_kernel: one workgroup per (b, h, chunk), fully parallel; writes Wn, Qt and
//     Kh^T, the lower-triangular fragments of P and -T' (bf16, MFMA operand order),
//     Gam_last and the validity bits of the chunk's rows to a workspace;
//   scan_kernel: one workgroup per (b, h, 16- or 32-column dv tile); a loop over the
//     chunks in order with the fp32 state tile in registers.  Each chunk's operands
//     are loaded into registers one chunk ahead of their use, and T' V for the next
//     chunk is formed from V read straight from the input.
// The factorisation Kt Ki^T (decay relative to the chunk start) is used when
// every channel's decay over the chunk stays above 2^-120 (then no factor
// over- or under-flows); otherwise that chunk computes A and P entry by entry
// with exp2(G_t - G_j).  Entries above the diagonal come from a select, never
// from a product, so nothing from a later position can reach an earlier one.
//
// Precision: bf16 MFMA operands that are not exactly bf16 are split into a
// bf16 high part and a bf16 residual where that matters (A, P, T', S, U);
// with fp32 inputs every operand is split.
#include <mutex>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kPrepThreads = 256;
constexpr int kScanThreads = 512;
constexpr int kVT = 16;                  // dv columns per MFMA tile (a scan workgroup takes 1 or 2)
constexpr float kFastLimit = -120.0f;    // log2 decay over one chunk for the factorised path
constexpr size_t kSinkBytes = 16384;     // workspace tail that absorbs the stores of rows past T

// ---------------------------------------------------------------- workspace layout
// Per (b, h, chunk), in 2-byte units.  Wn, Qt and Kh^T are in A-operand order of
// v_mfma_f32_16x16x32_bf16: fragment (row tile rt, k step ks) is 64 lanes x 8 bf16
// (1 KB), lane l holding M[16 rt + l%16][32 ks + 8 (l/16) .. +7]; with fp32 inputs
// the bf16 residual parts follow the high parts.  P and -T' (C x C, lower
// triangular) keep only the fragments of k steps that reach the diagonal, packed
// row tile by row tile, as a high part followed by a residual part.
// Number of k steps (32 columns) that row tile I of a lower-triangular C x C matrix
// needs, and the packed fragments before row tile I.
// (row tile I ends at column 16 I + 15, i.e. in k step I/2; the sum of i/2 + 1 over i < I
// is I + (I/2) ((I-1)/2).)
__host__ __device__ constexpr int tri_steps(int I) { return I / 2 + 1; }
__host__ __device__ constexpr int tri_before(int I) { return I + (I / 2) * ((I - 1) / 2); }

template <int K, int V, int C, bool SPLIT>
struct WsLayout {
  static constexpr size_t kCK = (size_t)C * K;
  static constexpr size_t kSplitCK = SPLIT ? 2 * kCK : kCK;
  static constexpr size_t kPF = (size_t)tri_before(C / 16) * 512;  // packed C x C, one part
  static constexpr size_t off_wn = 0;                    // -T' Kt          [C x K]
  static constexpr size_t off_qt = off_wn + kSplitCK;    // Qt              [C x K]
  static constexpr size_t off_kh = off_qt + kSplitCK;    // Kh^T            [K x C]
  static constexpr size_t off_p = off_kh + kSplitCK;     // P   hi, lo      packed
  static constexpr size_t off_tn = off_p + 2 * kPF;      // -T' hi, lo      packed
  static constexpr size_t off_gam = off_tn + 2 * kPF;    // Gam_last        [K] fp32
  static constexpr size_t off_valid = off_gam + 2 * (size_t)K;   // 4 x 16 row-valid bits, then
                                                                 // the contraction bound (fp32)
  static constexpr size_t kElems = off_valid + 8;
};

__device__ __forceinline__ size_t frag_off(int rt, int ks, int lane, int kk) {
  return ((size_t)(rt * (kk / 32) + ks) * 64 + lane) * 8;
}
// fragment (row tile I, k step ks) of a packed lower-triangular C x C matrix
__device__ __forceinline__ size_t tri_off(int I, int ks, int lane) {
  return ((size_t)(tri_before(I) + ks) * 64 + lane) * 8;
}

// Packed sequences of different lengths (varlen): chunk g of the packed layout spans tokens
// [span[g].x, span[g].y), its first token and the end of its sequence; x < 0 past the last
// chunk.  Sequence i owns chunks first[i] .. first[i + 1] - 1, tokens [seq[i].x, seq[i].y),
// and its saved states start at entry seq[i].z of the state checkpoints.
struct PrepParams {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  uint16_t* ws;
  const int2* span;                        // varlen chunk spans, or null (batch layout)
  int B, T, H, dk, dv, chunk, NC, l2norm, scalar_gate;
  int bound;                               // 1: store each chunk's contraction bound (segmented scan)
};

struct ScanParams {
  const void* v;
  const float* init_state;
  float* final_state;
  void* o;
  const uint16_t* ws;
  void* sink;
  const int4* seq;                         // varlen: each sequence's first token, end, first checkpoint
  const int32_t* first;                    // varlen: each sequence's first chunk (N + 1 entries)
  float* ckpt;                             // states saved every ck_every chunks, or null
  int ck_every, ck_cap;                    // ck_cap: entries ckpt holds
  const int32_t* slot;                     // varlen: state slot of each sequence in a pool of S, or null
  int S;
  int B, T, H, dk, dv, chunk, NC, NT, nbh;
  // Segmented scan (batch layout): each (b, h) cut into G segments of seg_nc chunks.
  // plan[(b H + h) G + g]: g = 0 the head's flag (1: every boundary has a forgetting tail),
  // g >= 1 the first chunk of boundary g's tail.  seg_states [B H][G][dk][dv]: segment g's
  // entry state (only g = 0 is used: a copy of the initial state).  pass 2: the segments,
  // each from the start of its boundary's tail; pass 0: every head that is not segmented,
  // as one chain.
  const int32_t* plan;
  float* seg_states;
  int G, seg_nc, pass;
};

__device__ __forceinline__ void store_frag(uint16_t* dst, const bf16x8& v) {
  *reinterpret_cast<bf16x8*>(dst) = v;
}
// Materialise a packed value in registers here.  Without this the compiler sinks the
// conversions into the later, conditional uses and keeps their fp32 inputs alive in
// the meantime (about twice the registers).
__device__ __forceinline__ void pin8(bf16x8& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 u = __builtin_bit_cast(u32x4, v);
  asm volatile("" : "+v"(u));
  v = __builtin_bit_cast(bf16x8, u);
}
// The raw words of a row slice, hidden from the optimiser (no value computed from them is
// shared with a later conversion of the same words)
__device__ __forceinline__ void opaque(Raw8<0>& r) {
  asm volatile("" : "+v"(r.u.x), "+v"(r.u.y), "+v"(r.u.z), "+v"(r.u.w));
}
__device__ __forceinline__ void opaque(Raw8<1>& r) {
  asm volatile("" : "+v"(r.a.x), "+v"(r.a.y), "+v"(r.a.z), "+v"(r.a.w));
  asm volatile("" : "+v"(r.b.x), "+v"(r.b.y), "+v"(r.b.z), "+v"(r.b.w));
}
// 8 consecutive floats from 16-byte aligned LDS
__device__ __forceinline__ void ld8f(const float* src, float* out) {
  const float4 a = reinterpret_cast<const float4*>(src)[0];
  const float4 b = reinterpret_cast<const float4*>(src)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
// Cross-lane exchange through LDS inside one wave: the wave's LDS operations execute
// in order in hardware, so no wait is needed, but the compiler must neither move LDS
// accesses across this point nor split an all-lane store into divergent branches.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// Element (n, j) of an n-major LDS matrix with C bf16 per row and no padding: the
// 16-byte blocks of row n are permuted by an XOR with bits of n, so 16 lanes that
// read one block column of 16 consecutive rows, or 64 lanes that write 16-byte
// blocks of rows 4 apart, spread over the banks.
template <int C>
__device__ __forceinline__ int swz(int n, int j) {
  return n * C + ((((j >> 3) ^ ((n ^ (n >> 3)) & (C / 8 - 1)))) << 3) + (j & 7);
}

// ================================================================ prep kernel
// LDS of one prep workgroup, sized so that three workgroups share a CU: two regions,
// each reused by a later phase once the barrier after its last read has passed.
// Rows are unpadded; bank conflicts are avoided by permuting the 16-byte blocks of
// each row with an XOR of the row index (swz, swzk, swzf).
//   R1: Ki hi, lo (fast path) or G (other path); then T (fp32 C x C) and Kt^T.
//   R3: Kh^T until stored; then A.
//   R4: the per-channel decay sums, eight zeros and eight ones, the key row scales of
//       the other path (0 for rows that are not valid); then one 16 x 17 fp32 staging tile for each wave of the inversion's
//       block steps (waves 0 .. C/16 - 2).
template <int DT, int K, int V, int C>
struct PrepLds {
  static constexpr bool SPLIT = DT == 1;
  static constexpr int RT = C / 16;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int kParts = SPLIT ? 2 : 1;
  static constexpr int kT = C * C * 4;                   // bytes of T
  static constexpr int r1 = cmax(cmax(2 * C * K * 2, C * K * 4), kT + kParts * K * C * 2);
  static constexpr int r3 = cmax(kParts * K * C * 2, C * C * 4);
  // R4 in floats: s_tot [RT][K], s_gc [K], s_gce [K], 8 zeros, 8 ones, s_ks [C], s_grow [C]
  static constexpr int off_gc = RT * K, off_gce = off_gc + K, off_zero = off_gce + K, off_one = off_zero + 8;
  static constexpr int off_ks = off_one + 8, off_grow = off_ks + C;
  static constexpr int kStage = 16 * 17;
  static constexpr int r4 = cmax(off_grow + C, cmax(RT - 1, 1) * kStage);
};

// Element (r, c) of an r-major bf16 matrix with K per row: 16-byte blocks permuted by
// an XOR with the row, so 16 lanes reading one block column of 16 rows hit all banks.
template <int K>
__device__ __forceinline__ int swzk(int r, int c) {
  return r * K + ((((c >> 3) ^ (r & (K / 8 - 1)))) << 3) + (c & 7);
}
// Element (r, c) of an r-major fp32 C x C matrix, 16-byte blocks permuted likewise.
template <int C>
__device__ __forceinline__ int swzf(int r, int c) {
  return r * C + ((((c >> 2) ^ (r & (C / 4 - 1)))) << 2) + (c & 3);
}
// 8 consecutive floats of row r from column c (c a multiple of 8) of a swzf matrix
template <int C>
__device__ __forceinline__ void ld8t(const float* m, int r, int c, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(&m[swzf<C>(r, c)]);
  const float4 b = *reinterpret_cast<const float4*>(&m[swzf<C>(r, c + 4)]);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// One workgroup per (chunk, head) and batch row; wave I owns rows 16 I .. 16 I + 15 of
// the chunk.  Lane l of wave I holds row 16 I + l%16 and channels 32 ks + 8 (l/16) .. +7
// for every k step ks: the A-operand layout of the MFMA, so Kt and Qt never leave
// registers on their way into A and P.  All global loads are issued up front,
// unconditionally, from in-bounds rows; validity (mask, ragged tail) is applied by
// select afterwards.
// SGP: one gate per (token, head) with bf16 inputs.  Every channel of a row then decays
// alike, so the decay factors are per row, and A and P are Gram products of the raw bf16
// rows (exact MFMA operands, one product per k step instead of three) times the scalar
// mask exp2(g_i - g_j) <= 1: no 1/Gam factor, and so no exact path.
template <int DT, int K, int V, int C, bool SGP = false>
__global__ void __launch_bounds__(kPrepThreads, DT == 0 ? 3 : 1)
prep_kernel(PrepParams p) {
  using E = Elem<DT>;
  using Raw = typename E::T;
  using Lds = PrepLds<DT, K, V, C>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, V, C, SPLIT>;
  constexpr int RT = C / 16;          // row tiles of the chunk
  constexpr int CS = C / 32;          // k steps over chunk rows
  constexpr int KS = K / 32;          // k steps over key channels
  static_assert(RT <= 4, "one row tile per wave");

  __shared__ __attribute__((aligned(16))) unsigned char s_r1[Lds::r1];
  __shared__ __attribute__((aligned(16))) unsigned char s_r3[Lds::r3];
  __shared__ __attribute__((aligned(16))) float s_r4[Lds::r4];
  __shared__ float s_beta[C];
  __shared__ float s_bnd[4];                                         // per wave: bound over its rows
  __bf16* s_ki = reinterpret_cast<__bf16*>(s_r1);                    // [hi, lo][C][K] swzk (fast path)
  float* s_G = reinterpret_cast<float*>(s_r1);                       // [C][K] (other path)
  float* s_T = reinterpret_cast<float*>(s_r1);                       // [C][C] swzf
  __bf16* s_kt = reinterpret_cast<__bf16*>(s_r1 + Lds::kT);          // Kt^T [hi(, lo)][K][C] swz
  __bf16* s_khs = reinterpret_cast<__bf16*>(s_r3);                   // Kh^T [hi(, lo)][K][C] swz
  float* s_A = reinterpret_cast<float*>(s_r3);                       // [C][C] swzf
  float* s_tot = s_r4;                                               // per-tile sums of log2 decay, then
                                                                     // the sums of the earlier tiles
  float* s_gc = s_r4 + Lds::off_gc;                                  // chunk total Gc per channel
  float* s_gce = s_r4 + Lds::off_gce;                                // exp2(Gc)
  float* s_zero = s_r4 + Lds::off_zero;                              // 8 x 0
  float* s_one = s_r4 + Lds::off_one;                                // 8 x 1
  float* s_ks = s_r4 + Lds::off_ks;                                  // key row scales, 0: row not valid
  float* s_grow = s_r4 + Lds::off_grow;                              // SGP: g of each row (log2)
  float* s_scratch = s_r4;                                           // staging tiles, in the inversion

  // heads vary fastest across workgroups, so the ones running together read whole token
  // rows of q, k and log_alpha (all heads side by side) instead of one head's slice of each
  const int n = blockIdx.x / p.H, h = blockIdx.x % p.H, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);          // uniform: loops over row tiles stay scalar
  // the chunk's first token and the end of its sequence
  int t0 = n * p.chunk, tend = p.T;
  if (p.span != nullptr) {
    const int2 sp = p.span[n];
    if (sp.x < 0) return;                                            // past the last packed chunk
    t0 = sp.x;
    tend = sp.y;
  }
  const int dk = p.dk, dv = p.dv;
  const Raw* qg = (const Raw*)p.q;
  const Raw* kg = (const Raw*)p.k;
  uint16_t* wsb = p.ws + ((size_t)(b * p.H + h) * p.NC + n) * L::kElems;
  auto grow = [&](int t) -> size_t { return ((size_t)b * p.T + t) * p.H + h; };
  auto tsafe = [&](int r) -> int { const int t = t0 + r; return t < tend ? t : tend - 1; };
  // any readable bytes stand in for the mask when there is none (the value is ignored)
  const uint8_t* mp = p.mask != nullptr ? p.mask : reinterpret_cast<const uint8_t*>(p.beta);

  const int I = wave;
  const bool rows = I < RT;                                          // wave-uniform
  const int rq = 16 * (rows ? I : 0) + (lane % 16);                  // this lane's row
  const int cg = 8 * (lane / 16);                                    // channel offset inside a k step

  // ---- phase 1: issue the loads of this lane's row (q, k, log_alpha, beta, mask)
  Raw8<1> la_r[KS];
  Raw8<DT> k_r[KS], q_r[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = 32 * ks + cg, cs = c < dk ? c : 0;
    const size_t row = grow(tsafe(rq)) * dk + cs;
    if (p.scalar_gate) la_r[ks].fill(p.log_alpha[grow(tsafe(rq))]);   // one gate per (t, h)
    else la_r[ks].load(p.log_alpha, row);
    k_r[ks].load(kg, row);
    q_r[ks].load(qg, row);
  }
  const float beta_r = p.beta[grow(tsafe(rq))];
  const uint8_t m_r = mp[(size_t)b * p.T + tsafe(rq)];
  const bool rok = rows && rq < p.chunk && t0 + rq < tend && (p.mask == nullptr || m_r != 0);
  // q and k of rows that are not valid and of channels past dk become 0 here
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bool cok = rok && 32 * ks + cg < dk;
    k_r[ks].keep(cok);
    q_r[ks].keep(cok);
  }

  // ---- the key row's squared norm (for the contraction bound below, and the L2 norm);
  //      converted from an opaque copy of the raw words, so that the compiler does not keep
  //      these floats alive until the decay pass converts the same words again
  float sk = 0.f;
  if (p.l2norm || p.bound) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Raw8<DT> kc = k_r[ks];
      opaque(kc);
      float kf[8];
      kc.to_float(kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) sk += kf[e] * kf[e];
    }
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
  }
  // ---- row scales of the optional L2 normalisation
  float qs = 1.f, ksc = 1.f;
  if (p.l2norm) {
    float sq = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float qf[8];
      q_r[ks].to_float(qf);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq += qf[e] * qf[e];
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    qs = rsqrtf(sq + 1e-6f);
    ksc = rsqrtf(sk + 1e-6f);
  }
  // ---- the chunk's contraction bound, log2 of an upper bound on the spectral norm of the
  //      state transition over the chunk's valid rows.  A row's step S -> (I - b k k^T)
  //      Diag(alpha) S + ... has norm at most max_c alpha_c times max(1, |1 - b |k|^2|)
  //      (the projection is symmetric with eigenvalues 1 and 1 - b |k|^2), and a chunk's
  //      transition is the product of its rows'.  A row that is not valid is the identity
  //      (0).  A non-finite input gives a NaN bound, which no test of it accepts.  Only a
  //      launch whose scan is segmented reads it.
  if (p.bound) {
    float lm, lc;                                                    // max and sum of log2 alpha
    if constexpr (SGP) {
      float laf[8];
      la_r[0].to_float(laf);                                         // the row's one gate
      lm = laf[0] * kLog2e;
      lc = lm;
    } else {
      lm = -INFINITY;
      lc = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // channels past dk exist only in the 32-channel tile of dk = 16
        const bool cin = (K > 32) || (32 * ks + cg < dk);
        float laf[8];
        la_r[ks].to_float(laf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          lm = fmaxf(lm, cin ? laf[e] : -INFINITY);
          lc += cin ? laf[e] : 0.f;
        }
      }
      lm = fmaxf(lm, __shfl_xor(lm, 16, 64));
      lm = fmaxf(lm, __shfl_xor(lm, 32, 64));
      lc += __shfl_xor(lc, 16, 64);
      lc += __shfl_xor(lc, 32, 64);
      lm *= kLog2e;
    }
    const float kk = ksc * ksc * sk;
    float f = fabsf(1.f - beta_r * kk);
    f = f <= 1.f ? 1.f : f;                                          // (a NaN stays NaN)
    float l = rok ? lm + __log2f(f) + 0.f * lc : 0.f;
    l += __shfl_xor(l, 1, 64);                                       // lanes 0-15: the tile's rows
    l += __shfl_xor(l, 2, 64);
    l += __shfl_xor(l, 4, 64);
    l += __shfl_xor(l, 8, 64);
    if (lane == 0) s_bnd[I] = rows ? l : 0.f;
  }
  if (tid < 8) { s_zero[tid] = 0.f; s_one[tid] = 1.f; }
  if (rows && lane < 16) {
    s_beta[rq] = rok ? beta_r : 0.f;
    s_ks[rq] = rok ? ksc : 0.f;
  }

  // ---- inclusive cumulative sum of log2 decay over the tile's 16 rows (DPP row scan);
  //      invalid rows and channels past dk contribute 0
  float g_r[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bool cok = rok && 32 * ks + cg < dk;
    float laf[8];
    la_r[ks].to_float(laf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = cok ? laf[e] * kLog2e : 0.f;
      x += row_shr<1>(x);
      x += row_shr<2>(x);
      x += row_shr<4>(x);
      x += row_shr<8>(x);
      g_r[ks][e] = x;
    }
  }
  if (rows && (lane % 16) == 15) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float4* dst = reinterpret_cast<float4*>(&s_tot[I * K + 32 * ks + cg]);
      dst[0] = make_float4(g_r[ks][0], g_r[ks][1], g_r[ks][2], g_r[ks][3]);
      dst[1] = make_float4(g_r[ks][4], g_r[ks][5], g_r[ks][6], g_r[ks][7]);
    }
  }
  __syncthreads();

  // ---- per channel (one thread each): the sums of the earlier tiles (in place of the tile
  //      totals), the chunk total Gc, Gam_last = exp2(Gc) (also to the workspace), and the
  //      test for the factorised path: every Gc >= -120
  bool ch_fast = true;
  if (tid < K) {
    float run = 0.f;
#pragma unroll
    for (int J = 0; J < RT; ++J) {
      const float t = s_tot[J * K + tid];
      s_tot[J * K + tid] = run;
      run += t;
    }
    const float ge = exp2f(run);
    s_gc[tid] = run;
    s_gce[tid] = ge;
    reinterpret_cast<float*>(wsb + L::off_gam)[tid] = ge;
    ch_fast = run >= kFastLimit;
  }
  bool fast = true;
  if constexpr (SGP) {
    static_assert(DT == 0, "the per-head specialisation takes bf16 rows as exact MFMA operands");
    __syncthreads();
  } else {
    fast = __syncthreads_and(ch_fast);
  }

  // ---- decay factors for this lane's row.  On the fast path every factor lies in
  //      [2^-120, 2^120], so the bare hardware exp2 is exact enough, and
  //      Gam_last / Gam = (1 / Gam) Gam_last.
  // One exp2 besides Gam per element on either path: e = k exp2(X - G) with X = 0 on
  // the fast path (e is Ki, and Kh = e Gam_last), X = Gc on the other (Kh = e; Ki is not
  // used there).  X and the factor after it are read from Gc / Gam_last or from blocks
  // of eight zeros / ones, chosen per k step, so the elementwise work has no selects.
  bf16x8 kth[KS], ktl[KS], qth[KS], qtl[KS];
  // SGP: the row's factors Gam and Gam_last / Gam, from this lane's first channel (a channel
  // past dk holds g = 0 there, and its k and q are 0 as well); lanes 0-15 hold channel 0
  // and publish the row's g for the mask of A and P
  float gam_r = 1.f, khf_r = 1.f;
  if constexpr (SGP) {
    const float g0 = g_r[0][0] + s_tot[(rows ? I : 0) * K + cg];
    gam_r = exp2f(g0);
    khf_r = exp2f(s_gc[cg] - g0);
    if (rows && lane < 16) s_grow[rq] = g0;
  }
  {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + cg;
      float pre[8], xv[8], mv[8];
      ld8f(&s_tot[(rows ? I : 0) * K + c0], pre);
      ld8f(fast ? s_zero : &s_gc[c0], xv);
      ld8f(fast ? &s_gce[c0] : s_one, mv);
      float kt[8], ki[8], kh[8], qt[8], kv[8], qv[8], g[8];
      k_r[ks].to_float(kv);
      q_r[ks].to_float(qv);
      if (p.l2norm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { kv[e] *= ksc; qv[e] *= qs; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        g[e] = g_r[ks][e] + pre[e];
        if constexpr (SGP) {
          kt[e] = kv[e] * gam_r;
          qt[e] = qv[e] * gam_r;
          ki[e] = 0.f;
          kh[e] = kv[e] * khf_r;
        } else {
          const float gam = __builtin_amdgcn_exp2f(g[e]);
          kt[e] = kv[e] * gam;
          qt[e] = qv[e] * gam;
          ki[e] = kv[e] * __builtin_amdgcn_exp2f(xv[e] - g[e]);
          kh[e] = ki[e] * mv[e];
        }
      }
      split8(kt, kth[ks], ktl[ks]);
      split8(qt, qth[ks], qtl[ks]);
      pin8(kth[ks]); pin8(ktl[ks]); pin8(qth[ks]);
      if constexpr (!SGP) pin8(qtl[ks]);                          // (SGP: P takes the raw q rows)
      if (rows) {
        // Qt rows to the workspace (invalid rows are 0)
        const size_t off = frag_off(I, ks, lane, K);
        store_frag(wsb + L::off_qt + off, qth[ks]);
        if (SPLIT) store_frag(wsb + L::off_qt + L::kCK + off, qtl[ks]);
        bf16x8 hi, lo;
        split8(kh, hi, lo);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s_khs[swz<C>(c0 + e, rq)] = hi[e];
          if (SPLIT) s_khs[K * C + swz<C>(c0 + e, rq)] = lo[e];
        }
        if constexpr (SGP) {
          // the raw k row (bf16, exact) is the A operand of the Gram products
          *reinterpret_cast<bf16x8*>(&s_ki[swzk<K>(rq, c0)]) = __builtin_bit_cast(bf16x8, k_r[ks].u);
        } else if (fast) {
          split8(ki, hi, lo);
          *reinterpret_cast<bf16x8*>(&s_ki[swzk<K>(rq, c0)]) = hi;
          *reinterpret_cast<bf16x8*>(&s_ki[C * K + swzk<K>(rq, c0)]) = lo;
        } else {                                                     // exact pairwise decays need G
          float4* gp = reinterpret_cast<float4*>(&s_G[rq * K + c0]);
          gp[0] = make_float4(g[0], g[1], g[2], g[3]);
          gp[1] = make_float4(g[4], g[5], g[6], g[7]);
        }
      }
    }
  }

  // ---- validity of the chunk's rows, 16 bits per row tile (bit r: row 16 I + r)
  {
    const unsigned long long bal = __ballot(rok);
    if (lane == 0) wsb[L::off_valid + I] = rows ? (uint16_t)(bal & 0xffffu) : (uint16_t)0;
  }
  __syncthreads();
  if (p.bound && tid == 0)                                           // after the valid bits
    *reinterpret_cast<float*>(wsb + L::off_valid + 4) = (s_bnd[0] + s_bnd[1]) + (s_bnd[2] + s_bnd[3]);

  // ---- Kh^T fragments: row c, contraction over rows 8*oct .. +7
  for (int idx = tid; idx < K * (C / 8); idx += kPrepThreads) {
    const int c = idx % K, oct = idx / K;
    const int rt = c / 16, ks = oct / 4, ln = (c % 16) + 16 * (oct % 4);
    store_frag(wsb + L::off_kh + frag_off(rt, ks, ln, C), *reinterpret_cast<const bf16x8*>(&s_khs[swz<C>(c, 8 * oct)]));
    if (SPLIT)
      store_frag(wsb + L::off_kh + L::kCK + frag_off(rt, ks, ln, C),
                 *reinterpret_cast<const bf16x8*>(&s_khs[K * C + swz<C>(c, 8 * oct)]));
  }
  __syncthreads();                                                   // Kh rows read: R3 takes A

  // ---- A into LDS (shared by the inversion), P as this wave's A-fragments (hi, lo)
  bf16x8 ph[CS], pl[CS];
#pragma unroll
  for (int ks = 0; ks < CS; ++ks) { ph[ks] = zero8(); pl[ks] = zero8(); }
  if constexpr (SGP) {
    if (rows) {
      // Gram products of the raw rows (A operand: k rows of column tile J from LDS; B: this
      // lane's raw k and q rows), then per entry the decay mask exp2(g_i - g_j) <= 1 and
      // the rows' L2 scales (s_ks is 0 for a row that is not valid)
      const float beta_row = s_beta[rq], g_i = s_grow[rq];
#pragma unroll
      for (int s2 = 0; s2 < CS; ++s2) {
        f32x4 pt[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int J = 2 * s2 + t;
          f32x4 accA = zero4(), accP = zero4();
          if (J <= I) {
            const int j = 16 * J + (lane % 16);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const bf16x8 kj = *reinterpret_cast<const bf16x8*>(&s_ki[swzk<K>(j, 32 * ks + cg)]);
              accA = mfma16(kj, __builtin_bit_cast(bf16x8, k_r[ks].u), accA);
              accP = mfma16(kj, __builtin_bit_cast(bf16x8, q_r[ks].u), accP);
            }
          }
          float av[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = 16 * J + 4 * (lane / 16) + i;
            const float d = exp2f(fminf(g_i - s_grow[jj], 0.f)) * s_ks[jj];
            av[i] = (jj < rq) ? beta_row * (accA[i] * (d * ksc)) : 0.f;
            pt[t][i] = (jj <= rq) ? accP[i] * (d * qs) : 0.f;
          }
          *reinterpret_cast<float4*>(&s_A[swzf<C>(rq, 16 * J + 4 * (lane / 16))]) = make_float4(av[0], av[1], av[2], av[3]);
        }
        float pv[8];
        pair_to_afrag(pt[0], pt[1], pv);
        split8(pv, ph[s2], pl[s2]);
      }
    }
  } else if (fast) {
    if (rows) {
      // transposed products: A-operand rows are Ki rows of column tile J (LDS), B-operand
      // columns are this wave's Kt and Qt rows (registers); lane (g, r) gets columns
      // 16 J + 4 g .. +3 of row rq of A and P
      const float beta_row = s_beta[rq];
#pragma unroll
      for (int s2 = 0; s2 < CS; ++s2) {
        f32x4 pt[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int J = 2 * s2 + t;
          f32x4 accA = zero4(), accP = zero4();
          if (J <= I) {
            const int j = 16 * J + (lane % 16);
            f32x4 a[3] = {zero4(), zero4(), zero4()}, pq[3] = {zero4(), zero4(), zero4()};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const int c = 32 * ks + cg;
              const bf16x8 kih = *reinterpret_cast<const bf16x8*>(&s_ki[swzk<K>(j, c)]);
              const bf16x8 kil = *reinterpret_cast<const bf16x8*>(&s_ki[C * K + swzk<K>(j, c)]);
              a[0] = mfma16(kih, kth[ks], a[0]);
              a[1] = mfma16(kil, kth[ks], a[1]);
              a[2] = mfma16(kih, ktl[ks], a[2]);
              pq[0] = mfma16(kih, qth[ks], pq[0]);
              pq[1] = mfma16(kil, qth[ks], pq[1]);
              pq[2] = mfma16(kih, qtl[ks], pq[2]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              accA[i] = a[0][i] + (a[1][i] + a[2][i]);
              accP[i] = pq[0][i] + (pq[1][i] + pq[2][i]);
            }
          }
          float av[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = 16 * J + 4 * (lane / 16) + i;
            av[i] = (jj < rq) ? beta_row * accA[i] : 0.f;
            pt[t][i] = (jj <= rq) ? accP[i] : 0.f;
          }
          *reinterpret_cast<float4*>(&s_A[swzf<C>(rq, 16 * J + 4 * (lane / 16))]) = make_float4(av[0], av[1], av[2], av[3]);
        }
        float pv[8];
        pair_to_afrag(pt[0], pt[1], pv);
        split8(pv, ph[s2], pl[s2]);
      }
    }
  } else if (rows) {
    // exact pairwise decays, computed by each lane for its row and A-fragment columns
    const size_t tr = grow(tsafe(rq)) * dk;
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jj = 32 * ks + cg + e;
        float sa = 0.f, sp = 0.f;
        if (jj <= rq && rok && s_ks[jj] > 0.f) {
          const size_t tj = grow(t0 + jj) * dk;
          for (int c = 0; c < dk; ++c) {
            const float d = exp2f(s_G[rq * K + c] - s_G[jj * K + c]);
            const float kj = E::ld(kg, tj + c) * s_ks[jj];
            sa += E::ld(kg, tr + c) * ksc * kj * d;
            sp += E::ld(qg, tr + c) * qs * kj * d;
          }
        }
        s_A[swzf<C>(rq, jj)] = (jj < rq) ? beta_r * sa : 0.f;
        pv[e] = sp;
      }
      split8(pv, ph[ks], pl[ks]);
    }
  }
  // P rows of this wave to the workspace: the k steps that reach the diagonal
  if (rows) {
#pragma unroll
    for (int s2 = 0; s2 < CS; ++s2) {
      if (s2 >= tri_steps(I)) continue;
      const size_t off = tri_off(I, s2, lane);
      store_frag(wsb + L::off_p + off, ph[s2]);
      store_frag(wsb + L::off_p + L::kPF + off, pl[s2]);
    }
  }
  __syncthreads();                                                   // A complete; Ki or G read

  // ---- Kt^T into R1 after T: row c holds channel c of every row of the chunk
  if (rows) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_kt[swz<C>(32 * ks + cg + e, rq)] = kth[ks][e];
        if (SPLIT) s_kt[K * C + swz<C>(32 * ks + cg + e, rq)] = ktl[ks][e];
      }
    }
  }

  // ---- T = (I + A)^-1, blocked: diagonal 16x16 blocks by forward substitution (two
  //      partial sums per row keep the dependency chain short)
  if (tid < RT * 16) {
    const int Ib = tid / 16, cc = tid % 16;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float arow[16];
      ld8t<C>(s_A, 16 * Ib + rr, 16 * Ib, arow);
      ld8t<C>(s_A, 16 * Ib + rr, 16 * Ib + 8, arow + 8);
      float v0 = (rr == cc) ? 1.f : 0.f, v1 = 0.f;
#pragma unroll
      for (int jj = 0; jj < rr; ++jj) {
        if (jj & 1) v1 -= arow[jj] * x[jj];
        else v0 -= arow[jj] * x[jj];
      }
      x[rr] = v0 + v1;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s_T[swzf<C>(16 * Ib + rr, 16 * Ib + cc)] = x[rr];
  }
  for (int idx = tid; idx < C * C; idx += kPrepThreads) {
    const int rr = idx / C, jj = idx % C;
    if (jj / 16 != rr / 16) s_T[swzf<C>(rr, jj)] = 0.f;
  }
  __syncthreads();
  // off-diagonal blocks by distance d, one block per wave on the MFMA:
  //   X = sum_{L=J}^{I-1} A_IL T_LJ,   T_IJ = -T_II X      (I = J + d, wave J)
  for (int d = 1; d < RT; ++d) {
    const int J = wave, Ib = J + d;
    if (Ib < RT) {
      const int r = lane % 16, g = lane / 16;
      f32x4 xa = zero4(), xb = zero4();
#pragma unroll
      for (int st = 0; st < (RT / 2); ++st) {
        if (st >= (d + 1) / 2) break;
        const int k0 = 16 * J + 32 * st + 8 * g;                     // contraction rows of T
        const bool kin = k0 < 16 * Ib;                               // L < I only
        float av[8], tv[8];
        ld8t<C>(s_A, 16 * Ib + r, kin ? k0 : 0, av);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          av[e] = kin ? av[e] : 0.f;
          tv[e] = kin ? s_T[swzf<C>(k0 + e, 16 * J + r)] : 0.f;
        }
        bf16x8 ah, al, th, tl;
        split8(av, ah, al);
        split8(tv, th, tl);
        xa = mfma16(ah, th, xa);
        xb = mfma16(ah, tl, xb);
        xb = mfma16(al, th, xb);
      }
      // X (D layout) through the wave's staging tile into B-operand order
      float* stage = s_scratch + wave * 16 * 17;
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[(4 * g + i) * 17 + r] = xa[i] + xb[i];
      wave_lds_sync();
      float xv[8], tiv[8];
      const bool klo = g < 2;                                        // contraction over 16 rows only
      ld8t<C>(s_T, 16 * Ib + r, 16 * Ib + (klo ? 8 * g : 0), tiv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xv[e] = klo ? stage[(8 * g + e) * 17 + r] : 0.f;
        tiv[e] = klo ? tiv[e] : 0.f;
      }
      bf16x8 xh, xl, tih, til;
      split8(xv, xh, xl);
      split8(tiv, tih, til);
      f32x4 ya = zero4(), yb = zero4();
      ya = mfma16(tih, xh, ya);
      yb = mfma16(tih, xl, yb);
      yb = mfma16(til, xh, yb);
#pragma unroll
      for (int i = 0; i < 4; ++i) s_T[swzf<C>(16 * Ib + 4 * g + i, 16 * J + r)] = -(ya[i] + yb[i]);
    }
    __syncthreads();
  }

  // ---- -T' rows of this wave as A-operand fragments: to registers and the workspace
  bf16x8 tnh[CS], tnl[CS];
  if (rows) {
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + cg;
      float tv[8];
      ld8t<C>(s_T, rq, j0, tv);
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = -tv[e] * s_beta[j0 + e];
      split8(tv, tnh[ks], tnl[ks]);
      if (ks < tri_steps(I)) {
        const size_t off = tri_off(I, ks, lane);
        store_frag(wsb + L::off_tn + off, tnh[ks]);
        store_frag(wsb + L::off_tn + L::kPF + off, tnl[ks]);
      }
    }
  }

  // ---- Wn = -T' Kt for this wave's 16 rows, computed transposed (A operand: Kt^T rows
  //      from LDS, B operand: -T' rows in registers) and turned into A-operand
  //      fragments by lane swaps
  if (rows) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x4 dw[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int cn = 32 * ks + 16 * t + (lane % 16);
        f32x4 aw = zero4();
#pragma unroll
        for (int js = 0; js < CS; ++js) {
          if (js >= tri_steps(I)) continue;                          // T' is lower triangular
          const int j0 = 32 * js + cg;
          const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&s_kt[swz<C>(cn, j0)]);
          aw = mfma16(kt, tnh[js], aw);
          if (SPLIT) {
            const bf16x8 ktl_b = *reinterpret_cast<const bf16x8*>(&s_kt[K * C + swz<C>(cn, j0)]);
            aw = mfma16(ktl_b, tnh[js], aw);
            aw = mfma16(kt, tnl[js], aw);
          }
        }
        dw[t] = aw;
      }
      float wv[8];
      pair_to_afrag(dw[0], dw[1], wv);
      bf16x8 hi, lo;
      split8(wv, hi, lo);
      const size_t off = frag_off(I, ks, lane, K);
      store_frag(wsb + L::off_wn + off, hi);
      if (SPLIT) store_frag(wsb + L::off_wn + L::kCK + off, lo);
    }
  }
}

// ================================================================ scan kernel
// One workgroup per (b, h, dv tile of 16 columns, or of 32 as two 16-column halves),
// eight waves in two roles.
//   Waves 0-3 carry the state: wave w owns state row tiles w, w+4, ... and row tile w of
//   U.  Per chunk: T' V and U = T' V + Wn S, U exchanged through LDS, then
//   S <- Diag(Gam_last) S + Kh^T U, published to LDS for the next chunk.
//   Waves 4-7 form the output: wave 4 + I computes O = Qt S + P U for row tile I from
//   the same S and U in LDS and stores it.  Nothing of O feeds the next chunk, so it
//   runs beside the state chain instead of lengthening it.
// Every wave loads what it needs for the next chunk into registers during the current
// one, in small groups spread over the step (the CU moves about 75 KB of operands per
// step from L2, and a wave that issues a burst of loads waits for room in the load
// queue), with an L2 warm-up two chunks ahead.  Each step has two barriers, which all
// eight waves join: one when U is in LDS, one when the next state and V^T are.
// With a segment plan (ScanParams::plan) the same kernel runs a chain per (b, h, segment):
// pass 2 a segment from a zero state at the start of its boundary's tail, with the output
// of the tail's chunks sent to the sink (segment 0 from the initial state), pass 0 the
// heads the plan left to one chain.
template <int K, int C, bool SPLIT>
struct ChainOps {
  static constexpr int KS = K / 32, CS = C / 32, SPW = (K / 16 + 3) / 4;
  bf16x8 wn[KS];
  bf16x8 wnl[SPLIT ? KS : 1];
  bf16x8 kh[SPW][CS];
  bf16x8 khl[SPLIT ? SPW : 1][CS];
  bf16x8 th[CS], tl[CS];                             // -T', this wave's rows
};
template <int K, int C, bool SPLIT>
struct OutOps {
  static constexpr int KS = K / 32, CS = C / 32;
  bf16x8 qt[KS];
  bf16x8 qtl[SPLIT ? KS : 1];
  bf16x8 ph[CS], pl[CS];                             // P, this wave's rows
};

// Word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle, raw addressing.
constexpr int kBufWord3 = 0x00020000;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// V of one chunk in a TW-column tile, split evenly over the four state waves: lane l of
// wave w holds row (C/4) w + l / (256/C), columns (C TW/256) (l % (256/C)) .. + C TW/256 - 1.
template <int C, int TW>
struct VTile {
  static constexpr int kPerLane = C * TW / 256;      // elements per lane
  static constexpr int kLanesPerRow = 256 / C;
  __device__ __forceinline__ static int row(int w, int l) { return (C / 4) * w + l / kLanesPerRow; }
  __device__ __forceinline__ static int col(int l) { return kPerLane * (l % kLanesPerRow); }
};
// 4, 8 or 16 bytes at byte offset off of a buffer resource, zero-extended
template <int BYTES>
__device__ __forceinline__ u32x4 buffer_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  u32x4 x = {0u, 0u, 0u, 0u};
  if (BYTES == 16) {
    x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  } else if (BYTES == 8) {
    const auto y = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    x[0] = y[0]; x[1] = y[1];
  } else {
    x[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
  }
  return x;
}

// Four consecutive values as bf16 high parts and residuals (round to nearest even, as
// a single conversion would), each part stored to LDS with one 8-byte write.
__device__ __forceinline__ void store_split4(const float* v, __bf16* hi, __bf16* lo) {
  uint32_t h[2], l[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x2 hh = __builtin_convertvector((f32x2){v[2 * j], v[2 * j + 1]}, bf16x2);
    const uint32_t u = __builtin_bit_cast(uint32_t, hh);
    const bf16x2 ll = __builtin_convertvector(
        (f32x2){v[2 * j] - __uint_as_float(u << 16), v[2 * j + 1] - __uint_as_float(u & 0xffff0000u)}, bf16x2);
    h[j] = u;
    l[j] = __builtin_bit_cast(uint32_t, ll);
  }
  *reinterpret_cast<uint2*>(hi) = make_uint2(h[0], h[1]);
  *reinterpret_cast<uint2*>(lo) = make_uint2(l[0], l[1]);
}

// s_barrier with compiler-only fences around it: no memory access moves across
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// wait for this wave's LDS operations (not for its global loads)
__device__ __forceinline__ void wait_lgkm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
}
// wait for every global load of this wave (not for its LDS operations).  Used once
// before each chunk loop: the compiler derives the waits at the top of the loop from
// every path into it, and without this the first chunk's loads, issued in the compiler's
// own order, would set them for every later chunk too: the first step of each unrolled
// pair would then wait for nearly all loads in flight, the L2 warm-up included.
__device__ __forceinline__ void drain_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);
  asm volatile("" ::: "memory");
}
// loads issued in place: the scheduler moves nothing across either side
template <typename F>
__device__ __forceinline__ void pinned(F&& f) {
  __builtin_amdgcn_sched_barrier(0);
  f();
  __builtin_amdgcn_sched_barrier(0);
}

// TW = 16 or 32 dv columns per workgroup.  With 32 every operand fragment loaded from the
// workspace feeds two 16-column MFMA tiles ("halves"), so a CU streams half the operand
// bytes per output column; that pays when there are enough (b, h) pairs to fill the chip
// with half as many workgroups.
template <int DT, int K, int V, int C, int TW>
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(ScanParams p) {
  using E = Elem<DT>;
  using Tv = typename E::T;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, V, C, SPLIT>;
  using Ch = ChainOps<K, C, SPLIT>;
  using Ou = OutOps<K, C, SPLIT>;
  using VT = VTile<C, TW>;
  constexpr int NH = TW / kVT;                      // 16-column halves per workgroup
  constexpr int RT = C / 16, CS = C / 32, KS = K / 32, SRT = K / 16;
  constexpr int SPW = Ch::SPW;                      // state row tiles per state wave
  constexpr int KB = K + 8, CB = C + 8;
  constexpr int kStores = 4;                        // global stores per lane and chunk, always
  constexpr int kParts = SPLIT ? 2 : 1;
  static_assert(RT <= 4, "one U/O row tile per wave");

  __shared__ __attribute__((aligned(16))) __bf16 s_S[2][TW * KB];     // state hi, lo; B-operand rows = dv column
  __shared__ __attribute__((aligned(16))) __bf16 s_U[2][TW * CB];     // U hi, lo
  __shared__ __attribute__((aligned(16))) __bf16 s_vT[kParts][TW * C];  // V^T (hi, lo) of the next chunk, swizzled
  // Gam_last (K floats) and the row-valid bits (the next 16 bytes) of chunk c in slot c % 3,
  // written two chunk steps ahead by one output wave with a single load (a load per state
  // wave would have sixteen lanes on each address)
  __shared__ __attribute__((aligned(16))) float s_gv[3][K + 4];

  // XCD-aware mapping: all dv tiles of one head share blockIdx.x % 8 (one L2)
  const int L_id = blockIdx.x;
  const int xcd = L_id % 8, slot = L_id / 8;
  const int vbh = (slot / p.NT) * 8 + xcd, tile = slot % p.NT;
  if (vbh >= p.nbh) return;
  const int pass = p.pass;
  // pass 2 of a segmented scan runs one chain per (b, h, segment): in the batch
  // layout G per (b, h); packed, sequence b has seq[b].w segments (0: too short for any)
  // and its (head, segment) jobs start at H * seq[b].z
  const bool seg_pass = p.plan != nullptr && pass != 0;
  int bh = vbh, seg = 0, Gb = p.G;
  if (seg_pass) {
    if (p.seq == nullptr) {
      bh = vbh / p.G;
      seg = vbh % p.G;
    } else {
      // past the last job (the grid is an upper bound): leave after one load
      const int4 sl = p.seq[p.B - 1];
      if ((long long)(sl.z + sl.w) * p.H <= vbh) return;
      int lo = 0, hi = p.B - 1;                      // the last sequence whose jobs start at or before vbh
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((long long)p.seq[mid].z * p.H <= vbh) lo = mid;
        else hi = mid - 1;
      }
      const int4 sq = p.seq[lo];
      if ((long long)(sq.z + sq.w) * p.H <= vbh) return;   // past the last job
      Gb = sq.w;
      const int r = vbh - sq.z * p.H;
      bh = lo * p.H + r / Gb;
      seg = r % Gb;
    }
  }
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = tile * TW;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);        // uniform: addresses stay scalar
  const int I = wave & 3;                            // row tile (and first state row tile)
  const int nsteps = tri_steps(I);                   // k steps of row tile I that reach the diagonal
  // predicates that the tiling makes always true are compile-time constants, so the
  // loads below are straight-line code and the compiler's waits stay exact
  const bool has_rows = (RT >= 4) || (I < RT);
  auto srow = [&](int M) __attribute__((always_inline)) { return (SRT % 4 == 0) || (M < SRT); };
  auto tri = [&](int ks) __attribute__((always_inline)) { return ks == 0 || ks < nsteps; };
  const int dk = p.dk, dv = p.dv;
  // the sequence this workgroup scans: its first token, its length, its first chunk in
  // the workspace and its number of chunks (row b of the batch, or packed sequence b)
  size_t seq_tok0 = (size_t)b * p.T, ws_chunk0 = (size_t)bh * p.NC;
  int seq_T = p.T, NCs = p.NC, ck0 = 0;
  if (p.ckpt != nullptr && p.seq == nullptr) ck0 = b * (p.T / (p.chunk * p.ck_every));
  if (p.seq != nullptr) {
    const int4 sq = p.seq[b];
    seq_tok0 = (size_t)sq.x;
    seq_T = sq.y - sq.x;
    ck0 = sq.z;
    ws_chunk0 = (size_t)h * p.NC + p.first[b];
    NCs = p.first[b + 1] - p.first[b];
  }
  // where this (sequence, head) keeps its state: its own row, or its slot of a pool (a
  // slot outside the pool: no state is read or kept, the sequence starts from zero)
  int sbh = bh;
  if (p.slot != nullptr) {
    const int sl = p.slot[b];
    sbh = (sl >= 0 && sl < p.S) ? sl * p.H + h : -1;
  }
  const size_t mat = (size_t)dk * dv;
  const float* init_ptr = (p.init_state != nullptr && sbh >= 0) ? p.init_state + (size_t)sbh * mat : nullptr;
  float* fin_ptr = (p.final_state != nullptr && sbh >= 0) ? p.final_state + (size_t)sbh * mat : nullptr;
  int out0 = 0;                                      // the chain's first chunk with output
  // a packed sequence too short for segments has no plan (pass 0 runs it)
  if (p.plan != nullptr && p.seq != nullptr && !seg_pass) Gb = p.seq[b].w;
  if (p.plan != nullptr && Gb > 0) {
    // segmented scan: this chain's chunks [c0, c1), where its state comes from and goes to;
    // the (b, h)'s plan and segment-0 entry state (the initial state when there is one,
    // copied by the plan kernel so that the last segment may write the final state over
    // it) are at pbase
    const size_t pbase = p.seq == nullptr ? (size_t)bh * Gb : ((size_t)p.seq[b].z * p.H + (size_t)h * Gb);
    const int32_t* pl = p.plan + pbase;
    const bool seg_ok = pl[0] != 0;
    if (seg_ok != seg_pass) return;                  // pass 0 takes the heads pass 2 leaves
    if (seg_pass) {
      // segment 0 from the initial state; segment g from a zero state at the first chunk of
      // boundary g's tail, with output from the segment's first chunk on
      const int seg_nc = (NCs + Gb - 1) / Gb;
      const int s0 = seg * seg_nc, c1 = min(s0 + seg_nc, NCs);
      const int c0 = seg == 0 ? 0 : min(max(pl[seg], 0), s0);
      init_ptr = (seg == 0 && init_ptr != nullptr) ? p.seg_states + pbase * mat : nullptr;
      if (seg + 1 < Gb) fin_ptr = nullptr;
      out0 = s0 - c0;
      seq_tok0 += (size_t)c0 * p.chunk;
      ws_chunk0 += (size_t)c0;
      seq_T = min(seq_T - c0 * p.chunk, (c1 - c0) * p.chunk);
      NCs = c1 - c0;
    }
  } else if (seg_pass) {
    return;
  }
  const uint16_t* wsh = p.ws + ws_chunk0 * L::kElems;
  const int last = NCs - 1;
  // tokens are H * dv elements apart in q, k, v and o; byte offsets inside a chunk stay
  // below 2^32 (checked on the host)
  const size_t row_bytes = (size_t)p.H * dv * sizeof(Tv);
  const uint32_t col_bytes = (uint32_t)(((size_t)h * dv + v0 + lane % 16) * sizeof(Tv));
  auto token_base = [&](int t0) __attribute__((always_inline)) {
    return (seq_tok0 + t0) * row_bytes;
  };
  auto ld16 = [&](const uint16_t* src) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(src);
  };
  // the state entering the chunk and U, as B-operand fragments (hi, lo) from LDS
  auto read_state = [&](int hf, bf16x8* sh, bf16x8* slo) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = 32 * ks + 8 * (lane / 16);
      sh[ks] = *reinterpret_cast<const bf16x8*>(&s_S[0][(kVT * hf + lane % 16) * KB + k0]);
      slo[ks] = *reinterpret_cast<const bf16x8*>(&s_S[1][(kVT * hf + lane % 16) * KB + k0]);
    }
  };
  auto read_u = [&](int hf, bf16x8* uh, bf16x8* ul) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + 8 * (lane / 16);
      uh[ks] = *reinterpret_cast<const bf16x8*>(&s_U[0][(kVT * hf + lane % 16) * CB + j0]);
      ul[ks] = *reinterpret_cast<const bf16x8*>(&s_U[1][(kVT * hf + lane % 16) * CB + j0]);
    }
  };

  if (wave >= 4) {
    // ================= output waves: O = Qt S + P U for row tile I
    // Loads in the order the next step uses them, except that the P fragments past this
    // wave's diagonal are not loaded at all, and the ones that may be skipped come first
    // (so the waits for the others do not depend on the branch).
    auto load_out = [&](int part, int n, Ou& o) __attribute__((always_inline)) {
      const uint16_t* cb = wsh + (size_t)n * L::kElems;
      if (!has_rows) return;
      if (part == 0) {
#pragma unroll
        for (int ks = 1; ks < CS; ++ks) {
          if (!tri(ks)) continue;
          o.ph[ks] = ld16(cb + L::off_p + tri_off(I, ks, lane));
          o.pl[ks] = ld16(cb + L::off_p + L::kPF + tri_off(I, ks, lane));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) o.qt[ks] = ld16(cb + L::off_qt + frag_off(I, ks, lane, K));
      } else {
        o.ph[0] = ld16(cb + L::off_p + tri_off(I, 0, lane));
        o.pl[0] = ld16(cb + L::off_p + L::kPF + tri_off(I, 0, lane));
        if (SPLIT) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) o.qtl[ks] = ld16(cb + L::off_qt + L::kCK + frag_off(I, ks, lane, K));
        }
      }
    };
    // Gam_last and the valid bits of chunk c: lane l < K/4 takes Gam_last[4 l .. 4 l + 3],
    // lane K/4 the 16 bytes of valid bits (the workspace tail of the chunk)
    auto load_gv = [&](int c) __attribute__((always_inline)) -> float4 {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      const uint16_t* cb = wsh + (size_t)(c <= last ? c : last) * L::kElems;
      if (lane <= K / 4)
        x = *reinterpret_cast<const float4*>(lane < K / 4 ? cb + L::off_gam + 8 * lane : cb + L::off_valid);
      return x;
    };
    auto store_gv = [&](int c, const float4& x) __attribute__((always_inline)) {
      if (lane <= K / 4) *reinterpret_cast<float4*>(&s_gv[c % 3][4 * lane]) = x;
    };
    Tv* og = (Tv*)p.o;
    constexpr int kSinkSlot = 64 * NH;               // elements of the sink per workgroup
    Tv* sink = (Tv*)p.sink + (L_id & (4096 / kSinkSlot - 1)) * kSinkSlot;
    uint32_t o_lane[kStores];
#pragma unroll
    for (int i = 0; i < kStores; ++i)
      o_lane[i] = (uint32_t)((16 * I + 4 * (lane / 16) + i) * row_bytes) + col_bytes;
    auto out_step = [&](const Ou& o, int n, auto&& loads) __attribute__((always_inline)) {
      const int t0 = n * p.chunk;
      const bool full = (p.chunk == C) && (t0 + C <= seq_T);       // every row in range
      unsigned char* ochunk = reinterpret_cast<unsigned char*>(og) + token_base(t0);
      float4 gv;
      if (wave == 4) gv = load_gv(n + 2);
      f32x4 o4[NH][2];
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        o4[hf][0] = zero4();
        o4[hf][1] = zero4();
        bf16x8 sh[KS], slo[KS];
        read_state(hf, sh, slo);
        if (has_rows) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            o4[hf][ks & 1] = mfma16(o.qt[ks], sh[ks], o4[hf][ks & 1]);
            o4[hf][ks & 1] = mfma16(o.qt[ks], slo[ks], o4[hf][ks & 1]);
            if (SPLIT) o4[hf][ks & 1] = mfma16(o.qtl[ks], sh[ks], o4[hf][ks & 1]);
          }
        }
      }
      // the loads for the next step go after this wave's products, when the state waves'
      // loads have had time to drain from the CU's queue
      pinned([&] { loads(0); });
      wait_lgkm();
      wg_barrier();                                  // U in LDS
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        bf16x8 uh[CS], ul[CS];
        read_u(hf, uh, ul);
        if (has_rows) {
#pragma unroll
          for (int ks = 0; ks < CS; ++ks) {
            if (!tri(ks)) continue;                  // P is lower triangular
            o4[hf][ks & 1] = mfma16(o.ph[ks], uh[ks], o4[hf][ks & 1]);
            o4[hf][ks & 1] = mfma16(o.ph[ks], ul[ks], o4[hf][ks & 1]);
            o4[hf][ks & 1] = mfma16(o.pl[ks], uh[ks], o4[hf][ks & 1]);
          }
        }
      }
      if (has_rows) {
        pinned([&] { loads(1); });
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
          for (int i = 0; i < kStores; ++i) {
            const int rr = 16 * I + 4 * (lane / 16) + i;
            Tv* dst = reinterpret_cast<Tv*>(ochunk + o_lane[i] + kVT * hf * (uint32_t)sizeof(Tv));
            if (n < out0 || (!full && !(rr < p.chunk && t0 + rr < seq_T)))
              dst = sink + 64 * hf + 16 * i + (lane % 16);
            E::st(dst, 0, o4[hf][0][i] + o4[hf][1][i]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kStores * NH; ++i) {                      // keep the store count uniform
          volatile Tv* dst = sink + 16 * i + (lane % 16);
          *dst = (Tv)0;
        }
      }
      if (wave == 4) store_gv(n + 2, gv);
      wait_lgkm();
      wg_barrier();                                  // next state and V^T in LDS
    };

    Ou oA, oB;
    if (NCs > 0) { load_out(0, 0, oA); load_out(1, 0, oA); }
    if (wave == 4 && NCs > 0) {
      const float4 g0 = load_gv(0), g1 = load_gv(1);
      store_gv(0, g0);
      store_gv(1, g1);
    }
    wait_lgkm();
    wg_barrier();                                    // initial state and V^T in LDS
    drain_loads();
    int n = 0;
    for (; n + 1 < NCs; n += 2) {
      out_step(oA, n, [&](int part) __attribute__((always_inline)) { load_out(part, n + 1, oB); });
      const int nn = n + 2 <= last ? n + 2 : last;
      out_step(oB, n + 1, [&](int part) __attribute__((always_inline)) { load_out(part, nn, oA); });
    }
    if (n < NCs) out_step(oA, n, [](int) {});
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // ================= state waves
  __builtin_amdgcn_s_setprio(2);                     // issue ahead of the output waves
  const Tv* vg = (const Tv*)p.v;
  const int v_row = VT::row(wave, lane), v_col = VT::col(lane);
  const uint32_t v_off = (uint32_t)v_row * (uint32_t)row_bytes +
                         (uint32_t)(((size_t)h * dv + v0 + v_col) * sizeof(Tv));
  // chunk n's V in the tile's columns (this lane's part), through a buffer resource whose
  // range ends at token T: rows past T read as 0
  auto load_v = [&](int n) __attribute__((always_inline)) -> u32x4 {
    const int t0 = n * p.chunk;
    const unsigned long long span = (unsigned long long)(seq_T - t0) * row_bytes;
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<Tv*>(vg) + token_base(t0) / sizeof(Tv), (short)0,
        (int)(uint32_t)(span < 0xffffffffull ? span : 0xffffffffull), kBufWord3);
    return buffer_load_words<VT::kPerLane * (int)sizeof(Tv)>(vr, v_off);
  };
  // the chunk's row-valid bits (a vector load: a scalar one would share its counter with
  // the LDS reads, and every wait for those would also wait for it)
  auto load_valid = [&](int n) __attribute__((always_inline)) -> unsigned long long {
    return *reinterpret_cast<const unsigned long long*>(wsh + (size_t)n * L::kElems + L::off_valid);
  };
  // V^T of a chunk into LDS, rows that are not valid as 0 (their values may be anything)
  auto write_vt = [&](const u32x4& x, unsigned long long valid) __attribute__((always_inline)) {
    const bool ok = (valid >> v_row) & 1ull;
#pragma unroll
    for (int e = 0; e < VT::kPerLane; ++e) {
      if (!SPLIT) {
        const uint32_t w = ok ? x[e / 2] : 0u;
        const uint16_t hv = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
        s_vT[0][swz<C>(v_col + e, v_row)] = __builtin_bit_cast(__bf16, hv);
      } else {
        const float f = ok ? __uint_as_float(x[e]) : 0.f;
        const __bf16 hi = (__bf16)f;
        s_vT[0][swz<C>(v_col + e, v_row)] = hi;
        s_vT[kParts - 1][swz<C>(v_col + e, v_row)] = (__bf16)(f - (float)hi);
      }
    }
  };
  // Chunk n's operands for this wave, into registers, numbered in the order the next
  // step uses them; the -T' fragments past this wave's diagonal are not loaded, and the
  // ones that may be skipped come right after V (so the waits for everything later do
  // not depend on the branch).
  constexpr int kLoads = 1 + 2 * CS + KS + SPW * CS + (SPLIT ? KS + SPW * CS : 0);
  auto issue_load = [&](int idx, int n, Ch& op, u32x4& v) __attribute__((always_inline)) {
    const uint16_t* cb = wsh + (size_t)n * L::kElems;
    int k = idx;
    if (k == 0) {
      v = load_v(n);
      if (has_rows) {
#pragma unroll
        for (int ks = 1; ks < CS; ++ks) {
          if (!tri(ks)) continue;
          op.th[ks] = ld16(cb + L::off_tn + tri_off(I, ks, lane));
          op.tl[ks] = ld16(cb + L::off_tn + L::kPF + tri_off(I, ks, lane));
        }
      }
      return;
    }
    k -= 1;
    if (k < 2 * CS) {                                // k steps >= 1 were loaded with V
      if (has_rows && k < 2) {
        if (k & 1) op.tl[0] = ld16(cb + L::off_tn + L::kPF + tri_off(I, 0, lane));
        else op.th[0] = ld16(cb + L::off_tn + tri_off(I, 0, lane));
      }
      return;
    }
    k -= 2 * CS;
    if (k < KS) { if (has_rows) op.wn[k] = ld16(cb + L::off_wn + frag_off(I, k, lane, K)); return; }
    k -= KS;
    if (k < SPW * CS) {                              // Kh^T of this wave's state rows
      const int m = k / CS, ks = k % CS, M = wave + 4 * m;
      if (srow(M)) op.kh[m][ks] = ld16(cb + L::off_kh + frag_off(M, ks, lane, C));
      return;
    }
    k -= SPW * CS;
    if (SPLIT) {                                     // residual parts (fp32 inputs)
      if (k < KS) { if (has_rows) op.wnl[k] = ld16(cb + L::off_wn + L::kCK + frag_off(I, k, lane, K)); return; }
      k -= KS;
      const int m = k / CS, ks = k % CS, M = wave + 4 * m;
      if (srow(M)) op.khl[m][ks] = ld16(cb + L::off_kh + L::kCK + frag_off(M, ks, lane, C));
    }
  };
  constexpr int kGroups = 7;
  auto load_group = [&](int g, int n, Ch& op, u32x4& v) __attribute__((always_inline)) {
    pinned([&] {
#pragma unroll
      for (int idx = 0; idx < kLoads; ++idx)
        if (idx * kGroups / kLoads == g) issue_load(idx, n, op, v);
    });
  };

  // L2 warm-up two chunks ahead: one 4-byte load per 128-byte line that the workgroup's
  // loads will read, so they hit in L2.  It is the last load of its chunk step (waits
  // complete in issue order, so nothing waits behind its miss), and the loaded word is
  // consumed by an empty asm statement at the end of the next chunk step, when it has
  // long arrived: that keeps the load alive without a wait on anything recent.  Thread g
  // of the state waves takes line g of the list [its 1/NT share of the chunk's workspace
  // lines (every tile reads all of them); the lines of the chunk's V rows that hold the
  // tile's columns]; threads past the end repeat the first line.
  constexpr int kNT = V / TW;
  constexpr int kShLines = (int)((L::kElems * 2 + 127) / 128);
  size_t pf_off = 0;                                                   // bytes from the chunk base
  int pf_row = -1;                                                     // V row, or -1
  {
    const int sh_mine = (kShLines - tile + kNT - 1) / kNT;
    const int g = tid;
    if (g < sh_mine) pf_off = (size_t)(tile + kNT * g) * 128;
    else if (g - sh_mine < C) pf_row = g - sh_mine;
  }
  const uint32_t tile_bytes = (uint32_t)(((size_t)h * dv + v0) * sizeof(Tv));
  auto warm_chunk = [&](int n) __attribute__((always_inline)) -> uint32_t {
    const unsigned char* ws_line = reinterpret_cast<const unsigned char*>(wsh + (size_t)n * L::kElems) + pf_off;
    const int t0 = n * p.chunk, tmax = seq_T - 1 - t0;
    const unsigned char* v_line = reinterpret_cast<const unsigned char*>(vg) + token_base(t0) +
                                  (uint32_t)(pf_row < tmax ? pf_row : tmax) * (uint32_t)row_bytes + tile_bytes;
    return *reinterpret_cast<const uint32_t*>(pf_row >= 0 ? v_line : ws_line);
  };

  // state tiles in registers: wave w owns state row tiles w, w+4, ...
  f32x4 S[NH][SPW];
#pragma unroll
  for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * M + 4 * (lane / 16) + i, col = v0 + kVT * hf + (lane % 16);
        S[hf][m][i] = (M < SRT && row < dk && init_ptr != nullptr) ? init_ptr[(size_t)row * dv + col] : 0.f;
      }
    }
  }
  // this workgroup's columns of the state to a dk x dv fp32 matrix in HBM
  auto store_state = [&](float* dst) __attribute__((always_inline)) {
    // the lane index passes through an empty asm so the addresses are formed here, not
    // hoisted out of the chunk loop into registers held across it
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
      for (int m = 0; m < SPW; ++m) {
        const int M = wave + 4 * m;
        if (M >= SRT) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * M + 4 * (ln / 16) + i;
          if (row < dk) dst[(size_t)row * dv + v0 + kVT * hf + (ln % 16)] = S[hf][m][i];
        }
      }
    }
  };
  auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
      for (int m = 0; m < SPW; ++m) {
        const int M = wave + 4 * m;
        if (srow(M)) {                               // rows 16 M + 4 (lane / 16) .. + 3: consecutive
          const float v4[4] = {S[hf][m][0], S[hf][m][1], S[hf][m][2], S[hf][m][3]};
          const int at = (kVT * hf + lane % 16) * KB + 16 * M + 4 * (lane / 16);
          store_split4(v4, &s_S[0][at], &s_S[1][at]);
        }
      }
    }
  };

  // One chunk step: operands in registers, V^T and S in LDS.  Writes the next chunk's
  // V^T (when there is one) after every wave has read this one.
  auto chain_step = [&](const Ch& op, int n, bool write_next, const u32x4& vnext,
                        uint32_t warm_old, auto&& group)
                        __attribute__((always_inline)) {
    // this chunk's Gam_last rows and the next chunk's valid bits, from their LDS slots
    float4 gam[SPW];
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
      if (srow(M)) gam[m] = *reinterpret_cast<const float4*>(&s_gv[n % 3][16 * M + 4 * (lane / 16)]);
    }
    const unsigned long long valid_next = *reinterpret_cast<const unsigned long long*>(&s_gv[(n + 1) % 3][K]);
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      // V^T first: T' V needs nothing else and can start while the state arrives
      bf16x8 vth[CS], vtl[SPLIT ? CS : 1];
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        const int j0 = 32 * ks + 8 * (lane / 16);
        vth[ks] = *reinterpret_cast<const bf16x8*>(&s_vT[0][swz<C>(kVT * hf + lane % 16, j0)]);
        if (SPLIT) vtl[ks] = *reinterpret_cast<const bf16x8*>(&s_vT[kParts - 1][swz<C>(kVT * hf + lane % 16, j0)]);
      }
      bf16x8 sh[KS], slo[KS];
      read_state(hf, sh, slo);
      if (hf == 0) group(0);
      if (has_rows) {
        // ---- U = T' V + Wn S for this wave's 16 rows (independent accumulators keep the
        //      chains short; -T' is stored, so T' V enters with a minus sign)
        f32x4 u[4] = {zero4(), zero4(), zero4(), zero4()};
        f32x4 tv[2] = {zero4(), zero4()};
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          if (!tri(ks)) continue;                    // T' is lower triangular
          tv[0] = mfma16(op.th[ks], vth[ks], tv[0]);
          tv[1] = mfma16(op.tl[ks], vth[ks], tv[1]);
          if (SPLIT) tv[1] = mfma16(op.th[ks], vtl[ks], tv[1]);
        }
        if (hf == 0) group(1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u[(ks & 1) * 2] = mfma16(op.wn[ks], sh[ks], u[(ks & 1) * 2]);
          u[(ks & 1) * 2 + 1] = mfma16(op.wn[ks], slo[ks], u[(ks & 1) * 2 + 1]);
          if (SPLIT) u[(ks & 1) * 2 + 1] = mfma16(op.wnl[ks], sh[ks], u[(ks & 1) * 2 + 1]);
        }
        if (hf == 0) group(2);
        float uv[4];                                 // rows 16 I + 4 (lane / 16) .. + 3
#pragma unroll
        for (int i = 0; i < 4; ++i) uv[i] = ((u[0][i] + u[2][i]) + (u[1][i] + u[3][i])) - (tv[0][i] + tv[1][i]);
        const int at = (kVT * hf + lane % 16) * CB + 16 * I + 4 * (lane / 16);
        store_split4(uv, &s_U[0][at], &s_U[1][at]);
      } else if (hf == 0) {
        group(1); group(2);
      }
    }
    group(3);
    wait_lgkm();
    wg_barrier();                                    // U in LDS; S and V^T reads done
    // ---- S = Diag(Gam_last) S + Kh^T U  (the chain that carries to the next chunk)
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      bf16x8 uh[CS], ul[CS];
      read_u(hf, uh, ul);
      if (hf == 0) group(4);
#pragma unroll
      for (int m = 0; m < SPW; ++m) {
        const int M = wave + 4 * m;
        if (!srow(M)) continue;
        f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          a0 = mfma16(op.kh[m][ks], uh[ks], a0);
          a1 = mfma16(op.kh[m][ks], ul[ks], a1);
          if (SPLIT) a1 = mfma16(op.khl[m][ks], uh[ks], a1);
        }
        const float gg[4] = {gam[m].x, gam[m].y, gam[m].z, gam[m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) S[hf][m][i] = gg[i] * S[hf][m][i] + (a0[i] + a1[i]);
      }
    }
    group(5);
    publish_state();
    if (write_next) write_vt(vnext, valid_next);
    group(6);
    group(7);                                        // the L2 warm-up: always the last load
    asm volatile("" :: "v"(warm_old));               // the warm-up load of two steps back
    wait_lgkm();
    wg_barrier();                                    // next state and V^T in LDS
  };

  // the state after chunk n when it closes a checkpoint interval (every ck_every full
  // chunks), for prefix caching
  auto checkpoint = [&](int n) __attribute__((always_inline)) {
    if (p.ckpt != nullptr && (n + 1) % p.ck_every == 0 && (n + 1) * p.chunk <= seq_T) {
      const int idx = ck0 + (n + 1) / p.ck_every - 1;
      if (idx < p.ck_cap) store_state(p.ckpt + ((size_t)idx * p.H + h) * dk * dv);
    }
  };

  publish_state();
  Ch opA, opB;
  uint32_t warmA = 0, warmB = 0;
  if (NCs > 0) {
    u32x4 v;
#pragma unroll
    for (int idx = 0; idx < kLoads; ++idx) issue_load(idx, 0, opA, v);
    write_vt(v, load_valid(0));
  }
  if (NCs > 1) warmB = warm_chunk(1);
  wait_lgkm();
  wg_barrier();                                      // initial state and V^T in LDS
  drain_loads();
  int n = 0;
  for (; n + 1 < NCs; n += 2) {
    u32x4 vB;
    chain_step(opA, n, true, vB, warmB, [&](int g) __attribute__((always_inline)) {
      if (g < kGroups) load_group(g, n + 1, opB, vB);
      else warmA = warm_chunk(n + 2 <= last ? n + 2 : last);
    });
    checkpoint(n);
    const int nn = n + 2 <= last ? n + 2 : last;
    u32x4 vA;
    chain_step(opB, n + 1, true, vA, warmA, [&](int g) __attribute__((always_inline)) {
      if (g < kGroups) load_group(g, nn, opA, vA);
      else warmB = warm_chunk(n + 3 <= last ? n + 3 : last);
    });
    checkpoint(n + 1);
  }
  if (n < NCs) {                                    // odd chunk count: the last one
    const u32x4 none = {0u, 0u, 0u, 0u};
    chain_step(opA, n, false, none, warmB, [](int) {});
    checkpoint(n);
  }
  asm volatile("" :: "v"(warmA), "v"(warmB));
  __builtin_amdgcn_s_waitcnt(0);

  if (fin_ptr != nullptr) store_state(fin_ptr);
}

// ================================================================ segmented scan plan
// One workgroup per (b, h).  Thread g - 1 takes boundary g (chunk g * seg_nc): walking back
// over the segment before it, it looks for the shortest tail of chunks ending at the
// boundary whose contraction bounds sum to at most kForgetLog2.  The exact map from the
// state entering the tail to the state at the boundary then has spectral norm at most
// 2^-160, so the tail run from a zero state gives the boundary state to within 2^-160 of the
// Frobenius norm of the state entering the tail; that state is finite fp32 (norm below
// 2^135), so the difference is below 2^-25 in absolute value whatever the inputs.  A head
// is segmented only if every boundary has such a tail; the others run as one chain, as
// without a plan.
constexpr float kForgetLog2 = -160.f;
constexpr int kMinSegChunks = 64;                   // chunks per segment, at least
constexpr int kPlanThreads = 256;                   // boundaries per (b, h): G - 1 <= 63

// Packed sequences (seq, first given): one workgroup per (sequence, head); a sequence with
// seq[b].w = G segments has its boundaries in its own chunks (head h's run of the packed
// workspace) and its plan at H seq[b].z + h G.
template <int K, int V, int C, bool SPLIT>
__global__ void __launch_bounds__(kPlanThreads)
seg_plan_kernel(const uint16_t* __restrict__ ws, int NC, int G, int seg_nc, int32_t* __restrict__ plan,
                int H, const int4* __restrict__ seq, const int32_t* __restrict__ first,
                const float* __restrict__ init, const int32_t* __restrict__ slot, int S, int mat,
                float* __restrict__ seg_states) {
  using L = WsLayout<K, V, C, SPLIT>;
  const int g = threadIdx.x + 1;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  size_t chunk0 = (size_t)blockIdx.x * NC, pbase = (size_t)blockIdx.x * G;
  if (seq != nullptr) {
    const int4 sq = seq[b];
    G = sq.w;
    if (G == 0) return;                              // too short for segments
    const int ncb = first[b + 1] - first[b];
    seg_nc = (ncb + G - 1) / G;
    chunk0 = (size_t)h * NC + first[b];
    pbase = (size_t)sq.z * H + (size_t)h * G;
  }
  int start = -1;
  if (g < G) {
    const int end = g * seg_nc, lo = end - seg_nc;
    const uint16_t* base = ws + chunk0 * L::kElems + L::off_valid + 4;
    float acc = 0.f;
    for (int j0 = end - 1; j0 >= lo && start < 0; j0 -= 8) {
      float bnd[8];                                  // eight loads in flight, then the walk
#pragma unroll
      for (int u = 0; u < 8; ++u)
        bnd[u] = j0 - u >= lo ? *reinterpret_cast<const float*>(base + (size_t)(j0 - u) * L::kElems) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (start < 0 && j0 - u >= lo) {
          acc += bnd[u];
          if (acc <= kForgetLog2) start = j0 - u;      // a NaN bound never passes
        }
      }
    }
  }
  const bool ok = __syncthreads_and(g >= G || start >= 0);
  if (g < G) plan[pbase + g] = start;
  if (threadIdx.x == 0) plan[pbase] = ok ? 1 : 0;
  // a segmented (b, h) with an initial state (its row, or its slot of a pool): that state
  // copied to the segment-0 entry, so that the last segment may overwrite it in place
  // (without one, segment 0 starts from zero and the entry is not used)
  if (!ok) return;
  int row = blockIdx.x;
  if (slot != nullptr) {
    const int sl = slot[b];
    row = (sl >= 0 && sl < S) ? sl * H + h : -1;
  }
  if (init == nullptr || row < 0) return;
  const float* src = init + (size_t)row * mat;
  float* dst = seg_states + pbase * mat;
  for (int i = threadIdx.x; i < mat; i += kPlanThreads) dst[i] = src[i];
}

// ================================================================ packed sequences
// The chunk table of N packed sequences cu[i] .. cu[i + 1] - 1, built by one workgroup:
// first[i] = the number of chunks of the sequences before i (i = 0 .. N); seq[i] = the
// sequence's first token, its end and the number of state checkpoints (one per `interval`
// tokens, 0 when interval is 0) of the sequences before it; span[g] = (first token, end of
// its sequence) of every chunk g, (-1, -1) past the last.  Token bounds are clamped into
// [0, T] and chunk indexes to the NCmax chunks the workspace holds, so a malformed cu cannot
// send any kernel outside its buffers.
constexpr int kSetupThreads = 1024;
__global__ void __launch_bounds__(kSetupThreads)
varlen_setup_kernel(const int32_t* __restrict__ cu, int N, int T, int C, int NCmax, int interval,
                    int2* __restrict__ span, int4* __restrict__ seq, int32_t* __restrict__ first, int seg_H) {
  // chunk counts in the low 32 bits, checkpoint counts in the high ones: both totals stay
  // below 2^31, so one 64-bit scan carries the two.  With seg_H > 0 (a segmented scan, which
  // saves no checkpoints) the high half counts each sequence's segments instead, by the rule
  // a lone run of the sequence with seg_H heads follows (0 for a sequence too short to cut):
  // seq[i].z is then the first (head, segment) job of the sequence over H and seq[i].w its
  // segment count.
  __shared__ long long s_scan[kSetupThreads];
  __shared__ long long s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base <= N; base += kSetupThreads) {
    const int i = base + tid;
    int start = 0, end = 0, nc = 0, ck = 0;
    if (i < N) {
      start = min(max(cu[i], 0), T);
      end = min(max(cu[i + 1], start), T);
      nc = (end - start + C - 1) / C;
      ck = interval > 0 ? (end - start) / interval : 0;
      if (seg_H > 0) {
        int G = 1;
        while (seg_H * G < 64 && nc / (2 * G) >= kMinSegChunks) G *= 2;
        ck = G > 1 ? G : 0;
      }
    }
    const long long mine = ((long long)ck << 32) | (unsigned)nc;
    s_scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kSetupThreads; off <<= 1) {     // inclusive scan of the counts
      const long long v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const long long before = s_carry + s_scan[tid] - mine;
    const int excl = min((int)(before & 0xffffffffll), NCmax);
    if (i < N) seq[i] = make_int4(start, end, (int)(before >> 32), seg_H > 0 ? ck : 0);
    if (i <= N) first[i] = excl;
    for (int j = 0; j < nc && excl + j < NCmax; ++j) span[excl + j] = make_int2(start + j * C, end);
    __syncthreads();
    if (tid == kSetupThreads - 1) s_carry += s_scan[tid];
    __syncthreads();
  }
  for (int g = min((int)(s_carry & 0xffffffffll), NCmax) + tid; g < NCmax; g += kSetupThreads)
    span[g] = make_int2(-1, -1);
}

// ================================================================ host side
// Chunks of 16, 32 and 64 tokens.  The pages' kernel uses 256-token chunks; this one does
// not accept 128 or 256: with the chunk-start factorisation the decay factors of such a
// chunk leave the fp32 range for ordinary gates, its fp32 C x C inverse alone would take
// 64 KB (C = 128) or 256 KB (C = 256) of the 160 KB LDS, and the scan's per-token operand
// stream (P and T' grow with C) would grow by a fifth at C = 128.
static int tile_chunk(int chunk) { return chunk <= 32 ? 32 : 64; }
static int pad_k(int dk) { return dk < 32 ? 32 : dk; }

bool prefill_supported(int dk, int dv, int chunk) {
  (void)dk; (void)dv;
  return chunk == 16 || chunk == 32 || chunk == 64;
}

// (padded dk, dv, tile chunk) instantiated
#define KDA_FOR_SHAPES(X)                                                  \
  X(32, 16, 32) X(32, 32, 32) X(32, 64, 32) X(32, 128, 32)                 \
  X(64, 16, 32) X(64, 32, 32) X(64, 64, 32) X(64, 128, 32)                 \
  X(128, 16, 32) X(128, 32, 32) X(128, 64, 32) X(128, 128, 32)             \
  X(32, 16, 64) X(32, 32, 64) X(32, 64, 64) X(32, 128, 64)                 \
  X(64, 16, 64) X(64, 32, 64) X(64, 64, 64) X(64, 128, 64)                 \
  X(128, 16, 64) X(128, 32, 64) X(128, 64, 64) X(128, 128, 64)

static size_t chunk_ws_elems(int K, int V, int C, int dtype) {
#define KDA_WS(KK, VV, CC)                                                             \
  if (K == KK && V == VV && C == CC)                                                   \
    return dtype == 1 ? WsLayout<KK, VV, CC, true>::kElems : WsLayout<KK, VV, CC, false>::kElems;
  KDA_FOR_SHAPES(KDA_WS)
#undef KDA_WS
  return 0;
}

// chunks the workspace holds: per batch row, or for N packed sequences the bound
// T / chunk + N (each sequence adds at most one partial chunk)
static long long prefill_chunks(int B, int T, int chunk, bool varlen) {
  const int c = chunk;
  const long long nc = T > 0 ? ((long long)T + c - 1) / c : 0;
  return varlen ? nc + B : nc;
}

// a launch's x extent in threads is a 32-bit number: the chunk-local grid holds H times the
// chunks workgroups, the scan (B*H rounded up to 8) times up to dv / 16 = 8 column tiles
bool prefill_grid_ok(int B, int T, int H, int chunk, bool varlen) {
  const long long kMax = 0xffffffffll;
  const long long nbh = (long long)B * H;
  return prefill_chunks(B, T, chunk, varlen) * H * kPrepThreads <= kMax &&
         (nbh + 7) / 8 * 8 * 8 * kScanThreads <= kMax;
}

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segments per (b, h) of a segmented scan (1: none).  It pays where the 32-column scan
// tiles (bf16, dv = 128) would not otherwise fill the chip, i.e. with fewer than 64 (b, h)
// pairs: segments double until there are 64 chains, each of at least kMinSegChunks chunks
// (the tails that precede the boundaries stay a small fraction of the work).
static int seg_count(int nbh, long long NC, int dv, int dtype) {
  if (dtype != 0 || dv != 128 || nbh <= 0) return 1;
  int G = 1;
  while ((long long)nbh * G < 64 && NC / (2LL * G) >= kMinSegChunks) G *= 2;
  return G;
}

// Packed sequences are segmented one by one, each as a lone run of it would be (so such a
// packed sequence equals that run bit for bit), when the call has fewer than 64 (sequence,
// head) pairs, as the batch call needs fewer than 64 (b, h) pairs: with more the chip is
// full of single chains already.  Possible once some sequence can hold 128 chunks.
static bool varlen_may_segment(int N, int H, long long NC, int dv, int dtype) {
  return dtype == 0 && dv == 128 && H > 0 && (long long)N * H < 64 && NC >= 2 * kMinSegChunks;
}
// at most H * (NC / 64) (head, segment) jobs (a sequence of n chunks has at most n / 64
// segments), and at most N * H * Gmax (a sequence has at most Gmax segments with H heads)
static size_t varlen_jobs(int N, int H, long long NC) {
  long long gmax = 1;
  while ((long long)H * gmax < 64) gmax *= 2;
  const long long a = NC / kMinSegChunks, b = (long long)N * gmax;
  return (size_t)H * (size_t)(a < b ? a : b);
}

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype, bool varlen) {
  if (B == 0 || H == 0 || (T == 0 && !varlen)) return 0;
  const long long NC = prefill_chunks(B, T, chunk, varlen);
  const size_t per_chunk = chunk_ws_elems(pad_k(dk), dv, tile_chunk(chunk), dtype) * 2;
  if (!varlen) {
    // a segmented scan adds the segments' entry states and the plan after the sink
    const size_t base = (size_t)B * H * NC * per_chunk + kSinkBytes;
    const int G = seg_count(B * H, NC, dv, dtype);
    if (G == 1) return base;
    const size_t chains = (size_t)B * H * G;
    return align256(base) + chains * dk * dv * 4 + chains * 4;
  }
  // packed: H x NC chunks, the sink, then the chunk table (span, seq, first); a segmented
  // scan then adds entry states and plan entries for its (sequence, head, segment) jobs
  const size_t base = (size_t)H * NC * per_chunk + kSinkBytes + align16((size_t)NC * 8) + (size_t)B * 16 +
                      align16((size_t)(B + 1) * 4);
  if (!varlen_may_segment(B, H, NC, dv, dtype)) return base;
  const size_t jobs = varlen_jobs(B, H, NC);
  return align256(base) + jobs * dk * dv * 4 + jobs * 4;
}

template <int DT, int K, int V, int C>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  if ((size_t)(C + 1) * a.H * a.dv * 4 > 0xffffffffull) return hipErrorInvalidValue;   // 32-bit output offsets
  const bool varlen = a.cu_seqlens != nullptr;
  const int NC = (int)prefill_chunks(a.B, a.T, a.chunk, varlen);
  const int nbh = a.B * a.H;
  // 32-column scan tiles (bf16, dv = 128) once there are enough (b, h) pairs for one such
  // workgroup per CU: each streams the chunk operands once for twice the columns
  constexpr bool kWideOk = (DT == 0 && V == 128);
  const bool wide = kWideOk && nbh >= 64;
  const int NT = a.dv / (wide ? 2 * kVT : kVT);
  const size_t chunks_bytes = (size_t)(varlen ? a.H : nbh) * NC * WsLayout<K, V, C, DT == 1>::kElems * 2;
  int2* span = nullptr;
  int4* seq = nullptr;
  int32_t* first = nullptr;
  const bool ckpt = a.chunk_states != nullptr;
  if (varlen) {
    unsigned char* tail = (unsigned char*)a.workspace + chunks_bytes + kSinkBytes;
    span = reinterpret_cast<int2*>(tail);
    seq = reinterpret_cast<int4*>(tail + align16((size_t)NC * 8));
    first = reinterpret_cast<int32_t*>(tail + align16((size_t)NC * 8) + (size_t)a.B * 16);
  }
  // segments per (b, h) of a segmented scan (1: one chain each); packed sequences are
  // segmented one by one on the device (vseg), never when checkpoints are saved
  const int G = (!kWideOk || varlen || ckpt || a.serial_scan) ? 1 : seg_count(nbh, NC, a.dv, DT);
  const bool vseg = kWideOk && varlen && !ckpt && !a.serial_scan && varlen_may_segment(a.B, a.H, NC, a.dv, DT);
  if (varlen) {
    hipLaunchKernelGGL(varlen_setup_kernel, dim3(1), dim3(kSetupThreads), 0, st, a.cu_seqlens, a.B, a.T,
                       a.chunk, NC, ckpt ? a.state_interval : 0, span, seq, first, vseg ? a.H : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (NC > 0) {
    PrepParams pp{a.q, a.k, a.v, a.log_alpha, a.beta, a.mask, (uint16_t*)a.workspace, span,
                  a.B, a.T, a.H, a.dk, a.dv, a.chunk, NC, a.l2norm, a.scalar_gate, (G > 1 || vseg) ? 1 : 0};
    const dim3 pgrid(NC * a.H, varlen ? 1 : a.B);
    if (DT == 0 && a.scalar_gate)
      hipLaunchKernelGGL((prep_kernel<DT, K, V, C, DT == 0>), pgrid, dim3(kPrepThreads), 0, st, pp);
    else
      hipLaunchKernelGGL((prep_kernel<DT, K, V, C>), pgrid, dim3(kPrepThreads), 0, st, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanParams sp{a.v, a.init_state, a.final_state, a.o, (const uint16_t*)a.workspace,
                NC > 0 ? (void*)((unsigned char*)a.workspace + chunks_bytes) : nullptr, seq, first,
                ckpt ? a.chunk_states : nullptr, ckpt ? a.state_interval / a.chunk : 0, ckpt ? a.num_states : 0,
                varlen ? a.slot : nullptr, a.num_slots, a.B, a.T, a.H, a.dk, a.dv, a.chunk, NC, NT, nbh,
                nullptr, nullptr, 1, NC, 0};
  if constexpr (kWideOk) {
    // segmented scan: plan (and the copies of the initial states), then the segments
    // (pass 2) as chains of 32-column tiles, then (below, pass 0) the heads without a plan
    // as single chains
    if (G > 1 || vseg) {
      // chains of pass 2: every (b, h, segment), or packed an upper bound on the
      // (sequence, head, segment) jobs, past which workgroups exit
      const size_t chains = vseg ? varlen_jobs(a.B, a.H, NC) : (size_t)nbh * G;
      const size_t base = vseg ? chunks_bytes + kSinkBytes + align16((size_t)NC * 8) + (size_t)a.B * 16 +
                                     align16((size_t)(a.B + 1) * 4)
                               : chunks_bytes + kSinkBytes;
      unsigned char* tail = (unsigned char*)a.workspace + align256(base);
      sp.seg_states = reinterpret_cast<float*>(tail);
      sp.plan = reinterpret_cast<const int32_t*>(tail + chains * a.dk * a.dv * 4);
      sp.G = vseg ? 0 : G;
      sp.seg_nc = vseg ? 0 : (NC + G - 1) / G;
      hipLaunchKernelGGL((seg_plan_kernel<K, V, C, DT == 1>), dim3(nbh), dim3(kPlanThreads), 0, st,
                         (const uint16_t*)a.workspace, NC, sp.G, sp.seg_nc, const_cast<int32_t*>(sp.plan), a.H,
                         vseg ? seq : nullptr, vseg ? first : nullptr, a.init_state, varlen ? a.slot : nullptr,
                         a.num_slots, a.dk * a.dv, sp.seg_states);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      // the segments, each after its boundary's tail, as chains of 32-column tiles
      ScanParams sw = sp;
      sw.NT = a.dv / (2 * kVT);
      sw.pass = 2;
      sw.nbh = (int)chains;
      hipLaunchKernelGGL((scan_kernel<DT, K, V, C, 2 * kVT>), dim3(((int)chains + 7) / 8 * 8 * sw.NT),
                         dim3(kScanThreads), 0, st, sw);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      sp.pass = 0;
    }
  }
  const int groups = (nbh + 7) / 8;
  if constexpr (kWideOk) {
    if (wide) {
      hipLaunchKernelGGL((scan_kernel<DT, K, V, C, 2 * kVT>), dim3(groups * 8 * NT), dim3(kScanThreads), 0, st, sp);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((scan_kernel<DT, K, V, C, kVT>), dim3(groups * 8 * NT), dim3(kScanThreads), 0, st, sp);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_prefill_dt(const PrefillArgs& a) {
  const int K = pad_k(a.dk), V = a.dv, C = tile_chunk(a.chunk);
#define KDA_PF(KK, VV, CC) \
  if (K == KK && V == VV && C == CC) return launch_prefill_t<DT, KK, VV, CC>(a);
  KDA_FOR_SHAPES(KDA_PF)
#undef KDA_PF
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- scratch for callers that cannot allocate
// The workspace of kda_chunk_prefill_noalloc: one array per GPU, resident from the first
// use of the library's code on that device until the process ends.  Host code never
// passes the array's name to a kernel (on the host that name is only a stand-in for the
// symbol); it uses the device address hipGetSymbolAddress returns, resolved once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& args) {
  return args.dtype == 0 ? launch_prefill_dt<0>(args) : launch_prefill_dt<1>(args);
}

}  // namespace kda
