// Gradients of the KDA prefill (remio.ai page, KDA section: the model is trained with a
// blockwise algorithm, which needs them): for L = sum_t <do_t, o_t> + <dfinal, S_T>, the
// derivatives with respect to q, k, v, log_alpha, beta and the initial state, in fp32.
//
// Chunk form (64-token chunks; the same quantities as the forward's chunk form, derived
// from the token recurrence).  In a chunk with entry state S0, g the inclusive cumulative
// sum of log_alpha over the chunk's rows, Gam = exp(g), Kt = K*Gam, Ki = K/Gam, Qt = Q*Gam,
// Kh = K*Gam_last/Gam:
//   G  = Kt Ki^T (strictly lower)   A = Diag(beta) G     M = (I + A)^-1   T' = M Diag(beta)
//   P  = lower(Qt Ki^T)             W = -T' Kt           R = V - Kt S0    U = T' R
//   O  = Qt S0 + P U                S1 = Diag(Gam_last) S0 + Kh^T U
// Reverse-mode differentiation of these lines, chunk by chunk from the last, with
// dS1 = dL/dS1 (dfinal for the last chunk):
//   dU  = P^T dO + Kh dS1                         dS0 = Diag(Gam_last) dS1 + Qt^T dO + W^T dU
//   dP  = lower(dO U^T)    dR = T'^T dU = dV      dT' = dU R^T
//   dbeta = colsum(dT' * M) + rowsum(dA * G)      dA = -strict_lower(M^T dT' Diag(beta) M^T)
//   dG  = Diag(beta) dA    dKt = -dR S0^T + dG Ki   dKi = dP^T Qt + dG^T Kt   dQt = dO S0^T + dP Ki
//   dKh = U dS1^T
// and through the decays: dq = Gam dQt, dk = Gam dKt + dKi/Gam + dKh Gam_last/Gam, and per
// row d(ln Gam) = dKt Kt - dKi Ki + dQt Qt - dKh Kh, plus for ln Gam_last the sum of dKh Kh
// over the rows and Gam_last rowsum(dS1 * S0); dlog_alpha_t is the sum of these over the
// rows at or after t.  Padded and masked rows enter as zero (an identity step) and get zero
// gradients.
//
// The pass runs as four launches on the caller's stream, after the forward prefill that saves
// the state at every chunk end (its own kernels) unless the caller hands those states in:
//   1. bwd_prep_kernel, one workgroup per (chunk, head): G, P, M = (I + A)^-1 and W, and the
//      reverse scan's operands Kh, W^T, Qt^T and P^T as bf16 MFMA fragments;
//   2. bwd_scan_kernel, one workgroup per (b, h, 16- or 32-column dv tile), over the chunks
//      from the last: dS1 and dU of every chunk, and dinit;
//   3. bwd_cc_kernel, one workgroup per (chunk, head): R, U, dv, dT', dbeta, dA, dG and dP;
//   4. bwd_ck_kernel, one workgroup per (chunk, head, 32 key channels): the products over dv
//      (dO S0^T, dR S0^T, U dS1^T) for its channels, then dq, dk and dlog_alpha.
// For sequences packed end to end (cu_seqlens) a one-workgroup setup kernel first writes a
// sequence table and a chunk table; each sequence's chunks start at its own first token, and
// the same four kernels find their rows, entry states and workspace slots through them.
// Products run on the bf16 MFMA with fp32 operands split into a bf16 high part and residual
// (three MFMAs per product), except the reverse scan's Kh, W^T and Qt^T, which are single
// bf16 with bf16 inputs (as the forward scan's Wn, Qt and Kh^T are).  A chunk in which some
// channel decays below 2^-120 cannot use the factorised products (Gam and 1/Gam would leave
// the fp32 range); it computes the decay-weighted C x C terms entry by entry instead.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kC = 64;                   // tokens per chunk
constexpr int kThreads = 256;
constexpr float kFastLimit = -120.0f;    // log2 decay over a chunk for the factorised path

__host__ __device__ constexpr int kpad(int k) { return k < 32 ? 32 : k; }

// bf16 elements before fragment (row tile rt, k step ks) of an A-operand matrix with kk
// columns: 64 lanes x 8 values, lane l holding row 16 rt + l%16, columns 32 ks + 8 (l/16) .. +7
__device__ __forceinline__ size_t afrag(int rt, int ks, int lane, int kk) {
  return ((size_t)(rt * (kk / 32) + ks) * 64 + lane) * 8;
}

// per-(b, h, chunk) workspace regions
struct Ws {
  uint16_t *kh, *wt, *qt, *pt;           // reverse-scan operands (fragments; high parts, then residuals)
  float *gam, *G, *M;                    // Gam_last [KP], G and M [C][C]
  uint64_t* vbits;                       // bit r: row r of the chunk is valid (in range, unmasked)
  float *dS1, *dU;                       // dL/dS at the chunk end [KP][V], dL/dU [C][V]
  float *U, *dP, *dG;                    // U [C][V]; dP and dG [C][C]
  const float* ck;                       // forward states at chunk ends [B * NCf][H][K][V]
};

struct Params {
  const void *q, *k, *v, *dout;
  const float *la, *beta, *init, *dfinal;
  const uint8_t* mask;
  float *dq, *dk, *dv, *dla, *dbeta, *dinit;
  Ws w;
  // packed sequences: per sequence (start, end, first checkpoint, first chunk) and per chunk
  // (sequence, chunk within it), (-1, -1) past the last; both null for a padded batch
  const int4* seqs;
  const int2* cmap;
  // with the q/k L2 norm: per token and head the row scales (q, k) = (|x|^2 + 1e-6)^-1/2,
  // written by the prep, (0, 0) where the row is not valid; null without the norm
  float2* qks;
  int sgate;                               // la holds one gate per (token, head), read into every channel
  int B, T, H, K, V, NC, NCf;              // packed: B = sequences, T = tokens, NC = chunk slots
  int num_states;                          // checkpoints ck holds (entries past it read as zero)
};

// Where sequence s lies for head h.  A padded batch: row s of [B, T], its chunks consecutive
// in the workspace.  Packed sequences: tokens [start, end) of the packed arrays, its chunks at
// consecutive entries of the chunk table, the workspace holding each entry's heads together.
struct SeqLoc {
  size_t t0;       // token (row of the [tokens][H] arrays) at the sequence's start
  int len, nc;     // tokens and chunks
  size_t ch0, chs; // workspace index of chunk 0 and the step between chunks
  long long ck0;   // checkpoint entry holding the state after the first chunk
};

__device__ __forceinline__ SeqLoc seq_loc(const Params& p, int s, int h) {
  if (p.seqs == nullptr)
    return {(size_t)s * p.T, p.T, p.NC, ((size_t)s * p.H + h) * p.NC, 1, (long long)s * p.NCf};
  const int4 q = p.seqs[s];
  const int len = q.y - q.x;
  return {(size_t)q.x, len, (len + kC - 1) / kC, (size_t)q.w * p.H + h, (size_t)p.H, q.z};
}

// chunk n of a sequence: its first token, the rows in range (1 .. 64) and its workspace index
struct ChunkLoc {
  size_t t0;
  int rows;
  size_t ch;
};

__device__ __forceinline__ ChunkLoc chunk_loc(const SeqLoc& S, int n) {
  const int left = S.len - n * kC;
  return {S.t0 + (size_t)n * kC, left < kC ? left : kC, S.ch0 + (size_t)n * S.chs};
}

// the (sequence, chunk) of a chunk-parallel workgroup: row b's chunk n in a padded batch, entry
// n of the chunk table for packed sequences (b = 0), where false means past the last chunk
__device__ __forceinline__ bool find_chunk(const Params& p, int b, int n, int& s, int& j) {
  if (p.cmap == nullptr) {
    s = b;
    j = n;
    return true;
  }
  const int2 m = p.cmap[n];
  s = m.x;
  j = m.y;
  return m.x >= 0;
}

// 8 consecutive floats from 8-byte aligned LDS
__device__ __forceinline__ void lds8(const float* src, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 x = reinterpret_cast<const float2*>(src)[j];
    out[2 * j] = x.x;
    out[2 * j + 1] = x.y;
  }
}
__device__ __forceinline__ void gld8(const float* src, float* out) { Elem<1>::ld8(src, 0, out); }

// D += A B for one 16 x 16 tile and one k step, both operands split (three MFMAs)
__device__ __forceinline__ f32x4 mm3(const float* a, const float* b, f32x4 acc) {
  bf16x8 ah, al, bh, bl;
  split8(a, ah, al);
  split8(b, bh, bl);
  acc = mfma16(ah, bh, acc);
  acc = mfma16(al, bh, acc);
  return mfma16(ah, bl, acc);
}

// D += A B, one k step, operands already split (three MFMAs; two when A is exact in bf16)
template <bool A_EXACT>
__device__ __forceinline__ f32x4 mma(const bf16x8& ah, const bf16x8& al, const bf16x8& bh, const bf16x8& bl, f32x4 acc) {
  acc = mfma16(ah, bh, acc);
  if (!A_EXACT) acc = mfma16(al, bh, acc);
  return mfma16(ah, bl, acc);
}

// four consecutive values as bf16 high parts and residuals, 8-byte writes to LDS
__device__ __forceinline__ void split4_to_lds(const float* v, __bf16* hi, __bf16* lo) {
  float x[8] = {v[0], v[1], v[2], v[3], 0.f, 0.f, 0.f, 0.f};
  bf16x8 h, l;
  split8(x, h, l);
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 hu = __builtin_bit_cast(u32x4, h), lu = __builtin_bit_cast(u32x4, l);
  *reinterpret_cast<uint2*>(hi) = make_uint2(hu[0], hu[1]);
  *reinterpret_cast<uint2*>(lo) = make_uint2(lu[0], lu[1]);
}

// LDS written by this wave is visible to its other lanes after this point: a wave's LDS
// operations execute in order, so the compiler only must not move accesses across it
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

// One lane's view of a chunk: row 16 w + l%16 (w = wave), channels c_base + 32 ks + 8 (l/16)
// .. +7 of a window of KW channels (the A-operand layout).  q, k and log_alpha of rows that
// are not valid (masked or past the sequence) and of channels past K are 0.  g becomes the
// inclusive cumulative sum of log2 decay over the chunk's rows and s_gl the chunk's totals
// per channel of the window.  Every thread must call it (it holds two barriers).
template <int DT, int KW>
struct Rows {
  static constexpr int KS = KW / 32;
  float k[KS][8], q[KS][8], g[KS][8];
  float beta;
  float qsc, ksc;                          // the row's L2 scales (1 without the norm)
  bool ok;
};

// With the q/k L2 norm, OWN_SCALE (the full channel window, q loaded) forms the row scales
// as the forward prep does (the same per-lane sums in the same order, so the same values)
// and stores them; the other callers read them.
template <int DT, int KW, bool WANT_Q, bool OWN_SCALE = false>
__device__ __forceinline__ void load_rows(const Params& p, const ChunkLoc& L, int h, int c_base, Rows<DT, KW>& R,
                                          float* s_tot, float* s_gl) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KW / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = 16 * w + (lane & 15), cg = 8 * (lane >> 4);
  const int rs = r < L.rows ? r : L.rows - 1;
  const size_t tk = (L.t0 + rs) * p.H + h;
  // every load is issued unconditionally from an in-bounds row and channel; what is not
  // valid is replaced by 0 with a select afterwards (a branch on the loaded mask would wait
  // for it before issuing the rest)
  const uint8_t mk = p.mask == nullptr ? (uint8_t)1 : p.mask[L.t0 + rs];
  const float bt = p.beta[tk];
  Raw8<DT> kr[KS], qr[KS];
  Raw8<1> lr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = c_base + 32 * ks + cg, cs = c0 < p.K ? c0 : 0;
    kr[ks].load((const Tp*)p.k, tk * p.K + cs);
    if (WANT_Q) qr[ks].load((const Tp*)p.q, tk * p.K + cs);
    if (p.sgate) lr[ks].fill(p.la[tk]);   // one gate per (t, h), the same in every channel
    else lr[ks].load(p.la, tk * p.K + cs);
  }
  R.ok = r < L.rows && mk != 0;
  R.beta = R.ok ? bt : 0.f;
  R.qsc = 1.f;
  R.ksc = 1.f;
  float2 sc = make_float2(1.f, 1.f);
  if (!OWN_SCALE && p.qks != nullptr) sc = p.qks[tk];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bool cok = R.ok && c_base + 32 * ks + cg < p.K;
    kr[ks].keep(cok);
    lr[ks].keep(cok);
    kr[ks].to_float(R.k[ks]);
    lr[ks].to_float(R.g[ks]);
    if (WANT_Q) {
      qr[ks].keep(cok);
      qr[ks].to_float(R.q[ks]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) R.q[ks][e] = 0.f;
    }
  }
  if (p.qks != nullptr) {
    if constexpr (OWN_SCALE) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) { sq += R.q[ks][e] * R.q[ks][e]; sk += R.k[ks][e] * R.k[ks][e]; }
      sq += __shfl_xor(sq, 16, 64); sk += __shfl_xor(sk, 16, 64);
      sq += __shfl_xor(sq, 32, 64); sk += __shfl_xor(sk, 32, 64);
      sc = make_float2(rsqrtf(sq + 1e-6f), rsqrtf(sk + 1e-6f));
      if (lane < 16 && r < L.rows) p.qks[tk] = R.ok ? sc : make_float2(0.f, 0.f);
    }
    R.qsc = R.ok ? sc.x : 0.f;
    R.ksc = R.ok ? sc.y : 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) { R.k[ks][e] *= R.ksc; R.q[ks][e] *= R.qsc; }
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = R.g[ks][e] * kLog2e;
      x += row_shr<1>(x);
      x += row_shr<2>(x);
      x += row_shr<4>(x);
      x += row_shr<8>(x);
      R.g[ks][e] = x;
    }
  }
  if ((lane & 15) == 15) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_tot[w * KW + 32 * ks + cg + e] = R.g[ks][e];
  }
  __syncthreads();
  if (tid < KW) {
    float run = 0.f;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const float x = s_tot[J * KW + tid];
      s_tot[J * KW + tid] = run;
      run += x;
    }
    s_gl[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) R.g[ks][e] += s_tot[w * KW + 32 * ks + cg + e];
}

// the entry state of chunk n of sequence s: the initial state for the first chunk, else the
// forward's state at the end of the chunk before (null: zero)
__device__ __forceinline__ const float* entry_state(const Params& p, const SeqLoc& S, int s, int h, int n) {
  if (n == 0) return p.init == nullptr ? nullptr : p.init + ((size_t)s * p.H + h) * p.K * p.V;
  const long long e = S.ck0 + n - 1;
  if (e < 0 || e >= p.num_states) return nullptr;
  return p.w.ck + ((size_t)e * p.H + h) * p.K * p.V;
}

// ================================================================ 2. prep
// One workgroup per (chunk, head); wave w holds rows 16 w .. +15 of the chunk in the
// A-operand layout.  One LDS region of C x (KP + 4) floats is reused, phase by phase, for Qt
// (to transpose it into Qt^T fragments), Ki (the B operand of G and P), A and P (the
// inverse and the P^T fragments), and Kt (the B operand of W = -T' Kt); with M and a small
// staging area that is about 58 KB, so two workgroups share a CU.
template <int DT, int KP>
__global__ void __launch_bounds__(kThreads, 2) bwd_prep_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32, CT = KP / 16, LD = KP + 4, LC = kC + 2;
  constexpr bool SPLIT = DT == 1;
  constexpr int parts = SPLIT ? 2 : 1;
  constexpr int RS = LD > 2 * LC ? LD : 2 * LC;                   // region floats per row
  __shared__ __attribute__((aligned(16))) float s_x[kC * RS];    // Qt; Ki or g; A and P; Kt
  __shared__ __attribute__((aligned(16))) float s_M[kC * LC];
  __shared__ __attribute__((aligned(16))) float s_stage[4 * 256];
  __shared__ float s_tot[4 * KP], s_gl[KP], s_beta[kC], s_ok[kC], s_qsc[kC], s_ksc[kC];
  __shared__ uint32_t s_vb[4];
  float* s_A = s_x;                                              // after G and P are formed
  float* s_P = s_x + kC * LC;

  const int h = blockIdx.x % p.H;
  int s, n;
  if (!find_chunk(p, blockIdx.y, blockIdx.x / p.H, s, n)) return;
  const ChunkLoc L = chunk_loc(seq_loc(p, s, h), n);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = L.ch;

  Rows<DT, KP> R;
  load_rows<DT, KP, true, true>(p, L, h, 0, R, s_tot, s_gl);
  if (lane < 16) { s_beta[r] = R.beta; s_ok[r] = R.ok ? 1.f : 0.f; s_qsc[r] = R.qsc; s_ksc[r] = R.ksc; }
  {
    // validity of the chunk's rows as one 64-bit word (wave w holds rows 16 w .. +15)
    const unsigned long long bal = __ballot(R.ok) & 0xffffull;
    if (lane == 0) s_vb[w] = (uint32_t)bal;
  }
  const bool fast = __syncthreads_and(tid >= KP || s_gl[tid] >= kFastLimit);
  if (tid == 0)
    p.w.vbits[ch] = (uint64_t)s_vb[0] | ((uint64_t)s_vb[1] << 16) | ((uint64_t)s_vb[2] << 32) | ((uint64_t)s_vb[3] << 48);

  // ---- decayed rows in registers; Kh fragments to the workspace; Qt to LDS
  uint16_t* kh = p.w.kh + ch * (size_t)(kC * KP * parts);
  float kt[KS][8];
  bf16x8 kth[KS], ktl[KS], qth[KS], qtl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float qt[8], khv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * ks + cg + e;
      const float gv = R.g[ks][e], gam = exp2f(gv);
      kt[ks][e] = R.k[ks][e] * gam;
      qt[e] = R.q[ks][e] * gam;
      khv[e] = R.k[ks][e] * exp2f(s_gl[c] - gv);
      s_x[r * LD + c] = qt[e];
    }
    split8(kt[ks], kth[ks], ktl[ks]);
    split8(qt, qth[ks], qtl[ks]);
    bf16x8 hi, lo;
    split8(khv, hi, lo);
    *reinterpret_cast<bf16x8*>(kh + afrag(w, ks, lane, KP)) = hi;
    if (SPLIT) *reinterpret_cast<bf16x8*>(kh + kC * KP + afrag(w, ks, lane, KP)) = lo;
  }
  __syncthreads();
  // ---- Qt^T fragments (rows: channels, contraction over chunk rows) and Gam_last
  {
    uint16_t* qtw = p.w.qt + ch * (size_t)(kC * KP * parts);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ct = w + 4 * m;
      if (ct >= CT) continue;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = s_x[(32 * s + cg + e) * LD + 16 * ct + col];
        bf16x8 hi, lo;
        split8(qv, hi, lo);
        *reinterpret_cast<bf16x8*>(qtw + afrag(ct, s, lane, kC)) = hi;
        if (SPLIT) *reinterpret_cast<bf16x8*>(qtw + kC * KP + afrag(ct, s, lane, kC)) = lo;
      }
    }
    if (tid < KP) p.w.gam[ch * KP + tid] = exp2f(s_gl[tid]);
  }
  __syncthreads();
  // ---- Ki (factorised path) or g (exact path) to LDS
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      s_x[r * LD + 32 * ks + cg + e] = fast ? R.k[ks][e] * exp2f(-R.g[ks][e]) : R.g[ks][e];
  __syncthreads();

  // ---- G (strictly lower) and P (lower) for row tile w, in registers in the D layout
  //      (lane: rows 16 w + 4 (l/16) .. +3, column 16 J + l%16)
  f32x4 gt[4], ptl[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) { gt[J] = zero4(); ptl[J] = zero4(); }
  if (fast) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > w) continue;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float bv[8];
        lds8(&s_x[(16 * J + col) * LD + 32 * ks + cg], bv);
        bf16x8 bh, bl;
        split8(bv, bh, bl);
        gt[J] = mfma16(kth[ks], bh, gt[J]);
        gt[J] = mfma16(ktl[ks], bh, gt[J]);
        gt[J] = mfma16(kth[ks], bl, gt[J]);
        ptl[J] = mfma16(qth[ks], bh, ptl[J]);
        ptl[J] = mfma16(qtl[ks], bh, ptl[J]);
        ptl[J] = mfma16(qth[ks], bl, ptl[J]);
      }
    }
  } else {
    // exact pairwise decays exp2(g_i - g_j) <= 1, entry by entry for the lane's D positions
    const Tp* kg = (const Tp*)p.k;
    const Tp* qg = (const Tp*)p.q;
    for (int J = 0; J <= w; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = 16 * w + 4 * g4 + i, jj = 16 * J + col;
        float gs = 0.f, ps = 0.f;
        if (jj <= ii && s_ok[ii] != 0.f && s_ok[jj] != 0.f) {
          const size_t ti = ((L.t0 + ii) * p.H + h) * p.K;
          const size_t tj = ((L.t0 + jj) * p.H + h) * p.K;
          // the L2 scales are 1 without the norm (an exact product)
          const float ski = s_ksc[ii], sqi = s_qsc[ii], skj = s_ksc[jj];
          for (int c = 0; c < p.K; ++c) {
            const float d = exp2f(s_x[ii * LD + c] - s_x[jj * LD + c]);
            const float kj = E::ld(kg, tj + c) * skj * d;
            gs += E::ld(kg, ti + c) * ski * kj;
            ps += E::ld(qg, ti + c) * sqi * kj;
          }
        }
        gt[J][i] = gs;
        ptl[J][i] = ps;
      }
  }
  __syncthreads();                                   // Ki / g read: the region takes A and P
  {
    float* Gg = p.w.G + ch * (size_t)(kC * kC);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const float gv = (J <= w && cl < row) ? gt[J][i] : 0.f;
        s_A[row * LC + cl] = s_beta[row] * gv;
        s_P[row * LC + cl] = (J <= w && cl <= row) ? ptl[J][i] : 0.f;
        Gg[row * kC + cl] = gv;
      }
  }
  __syncthreads();

  // ---- P^T fragments (rows: P's columns, contraction over P's rows)
  {
    uint16_t* pt = p.w.pt + ch * (size_t)(2 * kC * kC);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = s_P[(32 * s + cg + e) * LC + 16 * w + col];
      bf16x8 hi, lo;
      split8(pv, hi, lo);
      *reinterpret_cast<bf16x8*>(pt + afrag(w, s, lane, kC)) = hi;
      *reinterpret_cast<bf16x8*>(pt + kC * kC + afrag(w, s, lane, kC)) = lo;
    }
  }

  // ---- M = (I + A)^-1, blocked by 16 rows, fp32: wave I inverts diagonal block I by forward
  //      substitution (one column per lane of its first 16 lanes) and clears the blocks right
  //      of it; then the blocks below the diagonal by distance d, M_IJ = -M_II sum_{L=J}^{I-1}
  //      A_IL M_LJ with I = J + d (wave J, four values per lane, through a 16 x 16 staging tile)
  {
    const int I = w;
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float a0 = (rr == lane) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < rr; ++jj) {
          const float av = s_A[(16 * I + rr) * LC + 16 * I + jj];
          if (jj & 1) a1 -= av * x[jj];
          else a0 -= av * x[jj];
        }
        x[rr] = a0 + a1;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s_M[(16 * I + rr) * LC + 16 * I + lane] = x[rr];
    }
    for (int idx = lane; idx < (3 - I) * 256; idx += 64) {
      const int J = I + 1 + idx / 256, rr = (idx % 256) / 16, cc = idx % 16;
      s_M[(16 * I + rr) * LC + 16 * J + cc] = 0.f;
    }
    __syncthreads();
    float* stage = s_stage + w * 256;
    const int rr = lane >> 2, c0 = 4 * (lane & 3);
    for (int d = 1; d < 4; ++d) {
      const int J = w, Ib = J + d;
      if (Ib < 4) {
        float xv[4] = {0.f, 0.f, 0.f, 0.f};
        for (int L = J; L < Ib; ++L) {
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const float av = s_A[(16 * Ib + rr) * LC + 16 * L + t];
            const float2 m0 = *reinterpret_cast<const float2*>(&s_M[(16 * L + t) * LC + 16 * J + c0]);
            const float2 m1 = *reinterpret_cast<const float2*>(&s_M[(16 * L + t) * LC + 16 * J + c0 + 2]);
            xv[0] += av * m0.x; xv[1] += av * m0.y; xv[2] += av * m1.x; xv[3] += av * m1.y;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[rr * 16 + c0 + e] = xv[e];
        wave_lds_fence();
        float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float mv = s_M[(16 * Ib + rr) * LC + 16 * Ib + t];
#pragma unroll
          for (int e = 0; e < 4; ++e) yv[e] -= mv * stage[t * 16 + c0 + e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s_M[(16 * Ib + rr) * LC + 16 * J + c0 + e] = yv[e];
      }
      __syncthreads();                               // (the last one also ends the reads of A and P)
    }
    float* Mg = p.w.M + ch * (size_t)(kC * kC);
    for (int idx = tid; idx < kC * kC; idx += kThreads) Mg[idx] = s_M[(idx / kC) * LC + idx % kC];
  }

  // ---- Kt to LDS, then W = -T' Kt per channel tile, turned into W^T fragments by lane swaps
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_x[r * LD + 32 * ks + cg + e] = kt[ks][e];
  __syncthreads();
  {
    uint16_t* wt = p.w.wt + ch * (size_t)(kC * KP * parts);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ct = w + 4 * m;
      if (ct >= CT) continue;
      f32x4 wtile[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s > I / 2) continue;                   // T' is lower triangular
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 32 * s + cg + e;
            av[e] = s_M[(16 * I + col) * LC + j] * s_beta[j];
            bv[e] = s_x[j * LD + 16 * ct + col];
          }
          acc = mm3(av, bv, acc);
        }
        wtile[I] = -acc;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float wv[8];
        pair_to_afrag(wtile[2 * s], wtile[2 * s + 1], wv);
        bf16x8 hi, lo;
        split8(wv, hi, lo);
        *reinterpret_cast<bf16x8*>(wt + afrag(ct, s, lane, kC)) = hi;
        if (SPLIT) *reinterpret_cast<bf16x8*>(wt + kC * KP + afrag(ct, s, lane, kC)) = lo;
      }
    }
  }
}

// ================================================================ 3. reverse scan
// Wave w holds state row tiles w and w + 4 of lam = dL/dS (rows 16 rt + 4 (l/16) .. +3,
// column l%16 of the tile); per chunk: lam is saved as that chunk's dS1, dU's row tile w
// is formed and exchanged through LDS, then lam <- Diag(Gam_last) lam + W^T dU + Qt^T dO.
// A chunk's operands are loaded into registers while the chunk after it (in scan order:
// the one before it in time) is processed; the loop is unrolled by two so that the
// compiler's load waits are exact.
template <int DT, int KP, int NH>
struct ScanOps {
  static constexpr bool SPLIT = DT == 1;
  static constexpr int KS = KP / 32, MPW = (KP / 16 + 3) / 4, P = SPLIT ? 2 : 1;
  bf16x8 kh[P][KS];                  // Kh, row tile w
  bf16x8 pt[2][2];                   // P^T (high, residual), row tile w
  bf16x8 wt[P][MPW][2], qt[P][MPW][2];
  float4 gam[MPW];
  // dO as loaded: row tid / 4, 4 NH columns from 4 NH (tid % 4)
  typename std::conditional<DT == 1, float4, typename std::conditional<NH == 2, uint4, uint2>::type>::type dor[DT == 1 ? NH : 1];
  uint64_t vb;                       // the chunk's row-validity bits
};

// NH = 2: the workgroup takes 32 dv columns as two 16-column halves, so each chunk's
// operands, the dominant per-step traffic of the CU, serve twice the columns.  At
// dk = dv = 128 (bf16) that instance is held to 256 registers so that two workgroups share
// a CU (a 4-register spill outside the chunk loop; the other shapes spill far more under
// that bound and keep the compiler's choice)
template <int DT, int KP, int V, int NH>
__global__ void __launch_bounds__(kThreads, (DT == 0 && KP == 128 && V == 128 && NH == 2) ? 2 : 1)
    bwd_scan_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  using Ops = ScanOps<DT, KP, NH>;
  constexpr bool SPLIT = DT == 1;
  constexpr int parts = SPLIT ? 2 : 1;
  constexpr int RTK = KP / 16, MPW = Ops::MPW, KS = KP / 32, NT = V / (16 * NH), TW = 16 * NH;
  // [part][column][row], columns padded by 8 so the 16 columns a fragment read touches
  // start in different banks
  constexpr int LK = KP + 8, LR = kC + 8;
  __shared__ __attribute__((aligned(16))) __bf16 s_lam[2][TW * LK];
  __shared__ __attribute__((aligned(16))) __bf16 s_du[2][TW * LR];
  __shared__ __attribute__((aligned(16))) __bf16 s_do[2][TW * LR];

  // XCD-aware mapping: the NT column tiles of one (b, h) share blockIdx.x % 8, so they run
  // on one XCD and read each chunk's operands through one L2
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int bh = (slot / NT) * 8 + xcd, vt = slot % NT;
  if (bh >= p.B * p.H) return;
  const int h = bh % p.H;
  const SeqLoc S = seq_loc(p, bh / p.H, h);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4, v0 = TW * vt;

  auto load_ops = [&](int n, Ops& o) __attribute__((always_inline)) {
    const ChunkLoc L = chunk_loc(S, n);
    const size_t ch = L.ch;
    const uint16_t* kh = p.w.kh + ch * (size_t)(kC * KP * parts);
    const uint16_t* pt = p.w.pt + ch * (size_t)(2 * kC * kC);
    const uint16_t* wt = p.w.wt + ch * (size_t)(kC * KP * parts);
    const uint16_t* qt = p.w.qt + ch * (size_t)(kC * KP * parts);
#pragma unroll
    for (int q = 0; q < parts; ++q)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        o.kh[q][ks] = *reinterpret_cast<const bf16x8*>(kh + q * kC * KP + afrag(w, ks, lane, KP));
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int s = 0; s < 2; ++s) o.pt[q][s] = *reinterpret_cast<const bf16x8*>(pt + q * kC * kC + afrag(w, s, lane, kC));
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int rt = w + 4 * m < RTK ? w + 4 * m : 0;
#pragma unroll
      for (int q = 0; q < parts; ++q)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          o.wt[q][m][s] = *reinterpret_cast<const bf16x8*>(wt + q * kC * KP + afrag(rt, s, lane, kC));
          o.qt[q][m][s] = *reinterpret_cast<const bf16x8*>(qt + q * kC * KP + afrag(rt, s, lane, kC));
        }
      o.gam[m] = *reinterpret_cast<const float4*>(p.w.gam + ch * KP + 16 * rt + 4 * g4);
    }
    const int row = tid >> 2, c4 = 4 * NH * (tid & 3), rs = row < L.rows ? row : L.rows - 1;
    const Tp* dp = (const Tp*)p.dout + ((L.t0 + rs) * p.H + h) * V + v0 + c4;
#pragma unroll
    for (int j = 0; j < (DT == 1 ? NH : 1); ++j)
      o.dor[j] = *reinterpret_cast<const typename std::remove_reference<decltype(o.dor[0])>::type*>(dp + 4 * j);
    o.vb = p.w.vbits[ch];
  };

  float lam[NH][MPW][4];
#pragma unroll
  for (int hf = 0; hf < NH; ++hf)
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rt = w + 4 * m, row = 16 * rt + 4 * g4 + i;
        lam[hf][m][i] = (rt < RTK && row < p.K && p.dfinal != nullptr)
                            ? p.dfinal[((size_t)bh * p.K + row) * V + v0 + 16 * hf + col] : 0.f;
      }

  auto step = [&](int n, const Ops& o) __attribute__((always_inline)) {
    const size_t ch = S.ch0 + (size_t)n * S.chs;
    float* dS1 = p.w.dS1 + ch * (size_t)(KP * V);
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        const int rt = w + 4 * m;
        if (RTK % 4 != 0 && rt >= RTK) continue;     // (never taken when every wave has rows)
        const int cc = 16 * hf + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) dS1[(16 * rt + 4 * g4 + i) * V + v0 + cc] = lam[hf][m][i];
        split4_to_lds(lam[hf][m], &s_lam[0][cc * LK + 16 * rt + 4 * g4], &s_lam[1][cc * LK + 16 * rt + 4 * g4]);
      }
    {
      const int row = tid >> 2, c4 = 4 * NH * (tid & 3);
      // row valid (in range and unmasked); the empty asm keeps the test here, after the
      // loads of the next chunk have been issued, instead of right behind its own load
      uint64_t vb = o.vb;
      asm volatile("" : "+v"(vb));
      const bool rv = ((vb >> row) & 1ull) != 0ull;
      float dov[4 * NH];
      if constexpr (DT == 1) {
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          dov[4 * j] = o.dor[j].x; dov[4 * j + 1] = o.dor[j].y; dov[4 * j + 2] = o.dor[j].z; dov[4 * j + 3] = o.dor[j].w;
        }
      } else {
        uint32_t wd[2 * NH];
        if constexpr (NH == 2) {
          wd[0] = o.dor[0].x; wd[1] = o.dor[0].y; wd[2] = o.dor[0].z; wd[3] = o.dor[0].w;
        } else {
          wd[0] = o.dor[0].x; wd[1] = o.dor[0].y;
        }
#pragma unroll
        for (int j = 0; j < 2 * NH; ++j) {
          dov[2 * j] = __uint_as_float(wd[j] << 16);
          dov[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 4 * NH; ++e) {
        const float x = rv ? dov[e] : 0.f;
        const __bf16 hi = (__bf16)x;
        s_do[0][(c4 + e) * LR + row] = hi;
        if (SPLIT) s_do[1][(c4 + e) * LR + row] = (__bf16)(x - (float)hi);
      }
    }
    __syncthreads();

    // ---- dU, row tile w: Kh dS1 + P^T dO
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      const int cc = 16 * hf + col;
      f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&s_lam[0][cc * LK + 32 * ks + 8 * g4]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&s_lam[1][cc * LK + 32 * ks + 8 * g4]);
        a0 = mfma16(o.kh[0][ks], bh, a0);
        a1 = mfma16(o.kh[0][ks], bl, a1);
        if (SPLIT) a2 = mfma16(o.kh[parts - 1][ks], bh, a2);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s + 31 < 16 * w) continue;          // P^T is upper triangular
        const bf16x8 dh = *reinterpret_cast<const bf16x8*>(&s_do[0][cc * LR + 32 * s + 8 * g4]);
        a0 = mfma16(o.pt[0][s], dh, a0);
        a1 = mfma16(o.pt[1][s], dh, a1);
        if (SPLIT) a2 = mfma16(o.pt[0][s], *reinterpret_cast<const bf16x8*>(&s_do[1][cc * LR + 32 * s + 8 * g4]), a2);
      }
      float du[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = a0[i] + (a1[i] + a2[i]);
      float* dU = p.w.dU + ch * (size_t)(kC * V);
#pragma unroll
      for (int i = 0; i < 4; ++i) dU[(16 * w + 4 * g4 + i) * V + v0 + cc] = du[i];
      split4_to_lds(du, &s_du[0][cc * LR + 16 * w + 4 * g4], &s_du[1][cc * LR + 16 * w + 4 * g4]);
    }
    __syncthreads();

    // ---- lam <- Diag(Gam_last) lam + W^T dU + Qt^T dO
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int rt = w + 4 * m;
      if (RTK % 4 != 0 && rt >= RTK) continue;
      const float gg[4] = {o.gam[m].x, o.gam[m].y, o.gam[m].z, o.gam[m].w};
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const int cc = 16 * hf + col;
        f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&s_du[0][cc * LR + 32 * s + 8 * g4]);
          const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&s_du[1][cc * LR + 32 * s + 8 * g4]);
          const bf16x8 dh = *reinterpret_cast<const bf16x8*>(&s_do[0][cc * LR + 32 * s + 8 * g4]);
          a0 = mfma16(o.wt[0][m][s], uh, a0);
          a1 = mfma16(o.wt[0][m][s], ul, a1);
          a0 = mfma16(o.qt[0][m][s], dh, a0);
          if (SPLIT) {
            const bf16x8 dl = *reinterpret_cast<const bf16x8*>(&s_do[1][cc * LR + 32 * s + 8 * g4]);
            a2 = mfma16(o.wt[parts - 1][m][s], uh, a2);
            a2 = mfma16(o.qt[parts - 1][m][s], dh, a2);
            a1 = mfma16(o.qt[0][m][s], dl, a1);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[hf][m][i] = gg[i] * lam[hf][m][i] + (a0[i] + (a1[i] + a2[i]));
      }
    }
    __syncthreads();
  };

  // (loads are never conditional inside the loop, so every wait the compiler places on
  // them counts exactly the memory operations issued since)
  Ops A, B;
  int n = S.nc - 1;
  if (n >= 0) load_ops(n, A);
  __builtin_amdgcn_s_waitcnt(0);
  for (; n >= 1; n -= 2) {
    load_ops(n - 1, B);
    step(n, A);
    load_ops(n >= 2 ? n - 2 : 0, A);
    step(n - 1, B);
  }
  if (n == 0) step(0, A);
#pragma unroll
  for (int hf = 0; hf < NH; ++hf)
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rt = w + 4 * m, row = 16 * rt + 4 * g4 + i;
        if (rt < RTK && row < p.K) p.dinit[((size_t)bh * p.K + row) * V + v0 + 16 * hf + col] = lam[hf][m][i];
      }
}

// ================================================================ 4. C x C gradients
// dv runs in slabs of 32 columns: per slab R = V - Kt S0 (wave w: row tile w, Kt rows as
// A operands from registers), U = T' R and dR = T'^T dU, while dT' = dU R^T and
// dP = dO U^T accumulate in registers over the slabs (wave w: row tile w).  Then
// X = dT' Diag(beta) M^T and dA = -strict_lower(M^T X).  About 78 KB of LDS: two
// workgroups share a CU.
template <int DT, int KP, int V>
__global__ void __launch_bounds__(kThreads, 2) bwd_cc_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32, LC = kC + 2, LS = 34, VS = (V + 31) / 32;
  __shared__ __attribute__((aligned(16))) float s_R[kC * LS];    // one 32-column slab of R
  __shared__ __attribute__((aligned(16))) float s_U[kC * LS];    // ... of U
  __shared__ __attribute__((aligned(16))) float s_dU[kC * LS];   // ... of dU
  __shared__ __attribute__((aligned(16))) float s_M[kC * LC];
  // dT' and X (after the slab loop); during the loop the same bytes hold the slab of S0 as
  // split bf16 pairs, column-major ([column][k], k padded by 8): staged once per workgroup
  // with 16-byte loads and read as MFMA B operands by every wave
  constexpr int LK = KP + 8;
  static_assert(2 * 32 * LK * 2 <= 2 * kC * LC * 4, "the S0 slab does not fit the dT'/X region");
  __shared__ __attribute__((aligned(16))) float s_tx[2 * kC * LC];
  float* const s_dT = s_tx;
  float* const s_X = s_tx + kC * LC;
  __bf16* const s_Sh = reinterpret_cast<__bf16*>(s_tx);
  __bf16* const s_Sl = s_Sh + 32 * LK;
  __shared__ float s_tot[4 * KP], s_gl[KP], s_beta[kC], s_ok[kC], s_db[kC];

  const int h = blockIdx.x % p.H;
  int s, n;
  if (!find_chunk(p, blockIdx.y, blockIdx.x / p.H, s, n)) return;
  const SeqLoc S = seq_loc(p, s, h);
  const ChunkLoc L = chunk_loc(S, n);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = L.ch;
  auto tok = [&](int row) -> size_t { return (L.t0 + row) * p.H + h; };
  // the same row clamped into the sequence: an in-bounds address for unconditional loads
  auto tokc = [&](int row) -> size_t { return (L.t0 + (row < L.rows ? row : L.rows - 1)) * p.H + h; };

  Rows<DT, KP> R;
  load_rows<DT, KP, false>(p, L, h, 0, R, s_tot, s_gl);
  if (lane < 16) { s_beta[r] = R.beta; s_ok[r] = R.ok ? 1.f : 0.f; }
  // Kt of this lane's row: the A operand of R = V - Kt S0 for row tile w
  bf16x8 kth[KS], ktl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float kt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kt[e] = R.k[ks][e] * exp2f(R.g[ks][e]);
    split8(kt, kth[ks], ktl[ks]);
  }
  {
    const float4* Mg = reinterpret_cast<const float4*>(p.w.M + ch * (size_t)(kC * kC));
    float4 mv[kC * kC / 4 / kThreads];
#pragma unroll
    for (int j = 0; j < kC * kC / 4 / kThreads; ++j) mv[j] = Mg[tid + j * kThreads];
#pragma unroll
    for (int j = 0; j < kC * kC / 4 / kThreads; ++j) {
      const int idx = 4 * (tid + j * kThreads), row = idx / kC, cl = idx % kC;
      *reinterpret_cast<float2*>(&s_M[row * LC + cl]) = make_float2(mv[j].x, mv[j].y);
      *reinterpret_cast<float2*>(&s_M[row * LC + cl + 2]) = make_float2(mv[j].z, mv[j].w);
    }
  }
  __syncthreads();

  const float* S0 = entry_state(p, S, s, h, n);
  const float* dUg = p.w.dU + ch * (size_t)(kC * V);
  float* Ug = p.w.U + ch * (size_t)(kC * V);
  const bool rok = s_ok[r] != 0.f;
  f32x4 dT[4], dPa[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) { dT[J] = zero4(); dPa[J] = zero4(); }

  constexpr int SQ = KP * 8 / kThreads;           // float4 loads per thread of one S0 slab
#pragma unroll
  for (int vs = 0; vs < VS; ++vs) {
    // ---- loads of the slab: S0 rows (KP x 32, 8 float4 per row), V, dU, dO rows; the
    //      addresses are clamped in range and the values selected, so no load is conditional
    float4 s4[SQ];
    float vv[2][4], duv[2][4];
#pragma unroll
    for (int j = 0; j < SQ; ++j) {
      const int idx = tid + kThreads * j, row = idx >> 3, vc = 32 * vs + 4 * (idx & 7);
      const int vcc = vc < V ? vc : 0;
      const float* src = S0 != nullptr ? S0 + (size_t)(row < p.K ? row : 0) * V + vcc : dUg + vcc;
      const float4 x = *reinterpret_cast<const float4*>(src);
      const bool ok = S0 != nullptr && row < p.K && vc < V;
      s4[j] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int vc = 32 * vs + 16 * t2 + col, vcs = vc < V ? vc : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[t2][i] = E::ld((const Tp*)p.v, tokc(16 * w + 4 * g4 + i) * V + vcs);
    }
    {
      // dU rows 2 (tid / 16) .. +1 ... : 64 x 32 values, eight per thread
      const int row = tid >> 2, c8 = 8 * (tid & 3), vc = 32 * vs + c8;
      float x[8];
      gld8(dUg + row * V + (vc < V ? vc : 0), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) duv[e >> 2][e & 3] = vc < V ? x[e] : 0.f;
    }
    float dov[8];
    E::ld8((const Tp*)p.dout, tokc(r) * V + (32 * vs + cg < V ? 32 * vs + cg : 0), dov);
    // ---- the S0 slab split into LDS (the previous slab's readers passed the loop's last barrier)
#pragma unroll
    for (int j = 0; j < SQ; ++j) {
      const int idx = tid + kThreads * j, row = idx >> 3, c4 = 4 * (idx & 7);
      float x[8] = {s4[j].x, s4[j].y, s4[j].z, s4[j].w, 0.f, 0.f, 0.f, 0.f};
      bf16x8 hv, lv;
      split8(x, hv, lv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_Sh[(c4 + e) * LK + row] = hv[e];
        s_Sl[(c4 + e) * LK + row] = lv[e];
      }
    }
    __syncthreads();
    // ---- R slab, row tile w
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int vc = 32 * vs + 16 * t2 + col;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&s_Sh[(16 * t2 + col) * LK + 32 * ks + cg]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&s_Sl[(16 * t2 + col) * LK + 32 * ks + cg]);
        acc = mma<false>(kth[ks], ktl[ks], bh, bl, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i;
        const float vvv = (s_ok[row] != 0.f && vc < V) ? vv[t2][i] : 0.f;
        s_R[row * LS + 16 * t2 + col] = vc < V ? vvv - acc[i] : 0.f;
      }
    }
    {
      const int row = tid >> 2, c8 = 8 * (tid & 3);
      *reinterpret_cast<float2*>(&s_dU[row * LS + c8]) = make_float2(duv[0][0], duv[0][1]);
      *reinterpret_cast<float2*>(&s_dU[row * LS + c8 + 2]) = make_float2(duv[0][2], duv[0][3]);
      *reinterpret_cast<float2*>(&s_dU[row * LS + c8 + 4]) = make_float2(duv[1][0], duv[1][1]);
      *reinterpret_cast<float2*>(&s_dU[row * LS + c8 + 6]) = make_float2(duv[1][2], duv[1][3]);
    }
    __syncthreads();
    // ---- U = T' R and dR = T'^T dU for row tile w of the slab
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int vc = 32 * vs + 16 * t2 + col;
      f32x4 au = zero4(), ad = zero4();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        if (s2 <= w / 2) {                           // T' is lower triangular
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 32 * s2 + cg + e;
            av[e] = s_M[r * LC + j] * s_beta[j];
            bv[e] = s_R[j * LS + 16 * t2 + col];
          }
          au = mm3(av, bv, au);
        }
        if (32 * s2 + 31 >= 16 * w) {                // T'^T is upper triangular
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = 32 * s2 + cg + e;
            av[e] = s_M[rr * LC + r] * s_beta[r];
            bv[e] = s_dU[rr * LS + 16 * t2 + col];
          }
          ad = mm3(av, bv, ad);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i;
        s_U[row * LS + 16 * t2 + col] = au[i];
        if (vc < V) {
          Ug[row * V + vc] = au[i];
          if (row < L.rows) p.dv[tok(row) * V + vc] = s_ok[row] != 0.f ? ad[i] : 0.f;
        }
      }
    }
    __syncthreads();
    // ---- dT' += dU R^T and dP += dO U^T over the slab's columns: row tile w
    {
      float du[8];
      lds8(&s_dU[r * LS + cg], du);
#pragma unroll
      for (int e = 0; e < 8; ++e) dov[e] = (rok && 32 * vs + cg < V) ? dov[e] : 0.f;
      bf16x8 duh, dul, doh, dol;
      split8(du, duh, dul);
      split8(dov, doh, dol);
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        if (J > w) continue;
        float rv[8], uv[8];
        lds8(&s_R[(16 * J + col) * LS + cg], rv);
        lds8(&s_U[(16 * J + col) * LS + cg], uv);
        bf16x8 bh, bl;
        split8(rv, bh, bl);
        dT[J] = mma<false>(duh, dul, bh, bl, dT[J]);
        split8(uv, bh, bl);
        dPa[J] = mma<DT == 0>(doh, dol, bh, bl, dPa[J]);
      }
    }
    __syncthreads();
  }
  // ---- dT' (lower) to LDS, dP (lower) to the workspace
  {
    float* dP = p.w.dP + ch * (size_t)(kC * kC);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const bool lo = J <= w && cl <= row;
        s_dT[row * LC + cl] = lo ? dT[J][i] : 0.f;
        dP[row * kC + cl] = lo ? dPa[J][i] : 0.f;
      }
  }
  __syncthreads();

  // ---- dbeta through T' (column sums of dT' * M) and X = dT' Diag(beta) M^T; G of this
  //      wave's rows is loaded now for the dA step
  float gpre[4][4];
  {
    const float* Gg = p.w.G + ch * (size_t)(kC * kC);
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
      for (int i = 0; i < 4; ++i) gpre[J][i] = Gg[(16 * w + 4 * g4 + i) * kC + 16 * J + col];
  }
  float db = 0.f;
  if (tid < kC)
    for (int rr = tid; rr < kC; ++rr) db += s_dT[rr * LC + tid] * s_M[rr * LC + tid];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      if (s2 > w / 2 || s2 > J / 2) continue;
      float av[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 32 * s2 + cg + e;
        av[e] = s_dT[r * LC + kk] * s_beta[kk];
        bv[e] = s_M[(16 * J + col) * LC + kk];
      }
      acc = mm3(av, bv, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s_X[(16 * w + 4 * g4 + i) * LC + 16 * J + col] = acc[i];
  }
  __syncthreads();

  // ---- dA = -strict_lower(M^T X); dG = Diag(beta) dA; dbeta through A (row sums of dA * G)
  {
    float* dG = p.w.dG + ch * (size_t)(kC * kC);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 acc = zero4();
      if (J <= w) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (32 * s2 + 31 < 16 * w) continue;       // M^T is upper triangular
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = 32 * s2 + cg + e;
            av[e] = s_M[rr * LC + r];
            bv[e] = s_X[rr * LC + 16 * J + col];
          }
          acc = mm3(av, bv, acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const float da = (J <= w && cl < row) ? -acc[i] : 0.f;
        part[i] += da * gpre[J][i];
        dG[row * kC + cl] = s_beta[row] * da;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sum16(part[i]);
      if (col == 0) s_db[16 * w + 4 * g4 + i] = x;
    }
  }
  __syncthreads();
  if (tid < L.rows) p.dbeta[tok(tid)] = s_ok[tid] != 0.f ? db + s_db[tid] : 0.f;
}

// ================================================================ 5. q, k and decay gradients
// Every term here is separable by key channel, so a workgroup takes a slice of 32 channels
// and wave w channel tile w%2 of it over rows 32 (w/2) .. +31 (two row tiles): each lane
// holds the rows of one channel, and the reverse sum over rows for dlog_alpha is lane
// shuffles plus one exchange between the two halves.  dP and dG are staged in LDS as packed
// lower triangles (both are zero above the diagonal; their transposes are read from there by
// column): about 53 KB of LDS, three workgroups per CU.
constexpr int kCkSlice = 32;
constexpr int kTri = kC * (kC + 1) / 2;
// entry (i, j), j <= i, of a packed lower-triangular C x C matrix
__device__ __forceinline__ int tix(int i, int j) { return i * (i + 1) / 2 + j; }

template <int DT, int KP, int V>
__global__ void __launch_bounds__(kThreads, 3) bwd_ck_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int SW = kCkSlice, LD = SW + 2, VS = (V + 31) / 32, LA = 40;
  // One LDS region used twice: first for the dv slabs of the products (split bf16 rows of
  // dO, dR and U, and of S0 and dS1 for this slice's channels, rows padded to LA), then for
  // Kt, Ki, Qt, g and the packed dP and dG.
  constexpr int kX = 4 * kC * LD + 2 * kTri;                   // floats
  constexpr int kYA = kC * LA, kYB = SW * LA;                  // bf16 per part
  static_assert((3 * 2 * kYA + 2 * 2 * kYB) * 2 <= kX * 4, "the dv slabs do not fit the region");
  __shared__ __attribute__((aligned(16))) float s_x[kX];
  float* const s_a = s_x;                  // Kt, or k on the exact path
  float* const s_b = s_a + kC * LD;        // Ki (fast path)
  float* const s_c = s_b + kC * LD;        // Qt, or q on the exact path
  float* const s_g = s_c + kC * LD;        // g (log2)
  float* const s_dP = s_g + kC * LD;
  float* const s_dG = s_dP + kTri;
  __bf16* const s_ya = reinterpret_cast<__bf16*>(s_x);   // [dO, dR, U][high, residual][row][v]
  __bf16* const s_yb = s_ya + 3 * 2 * kYA;                // [S0, dS1][high, residual][channel][v]
  __shared__ float s_tot[4 * SW], s_gl[SW], s_ok[kC], s_half[2][2][SW], s_ss[SW], s_qsc[kC], s_ksc[kC];

  // XCD-aware mapping: the KP / SW channel slices of one chunk share blockIdx.x % 8 and are
  // dispatched 8 blocks apart, so the rows every slice reads (dO, dR, U, dP, dG) come from one L2
  constexpr int NS = KP / SW;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const long long cid = (long long)(slot / NS) * 8 + xcd;       // (b * NC + n) * H + h
  const int rows_b = p.cmap == nullptr ? p.B : 1;                // packed: one row of NC slots
  if (cid >= (long long)rows_b * p.NC * p.H) return;
  const int bn = (int)(cid / p.H), h = (int)(cid % p.H);
  int s, n;
  if (!find_chunk(p, bn / p.NC, bn % p.NC, s, n)) return;
  const SeqLoc S = seq_loc(p, s, h);
  const ChunkLoc L = chunk_loc(S, n);
  const int c_base = SW * (slot % NS);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = L.ch;
  auto tok = [&](int row) -> size_t { return (L.t0 + row) * p.H + h; };
  auto tokc = [&](int row) -> size_t { return (L.t0 + (row < L.rows ? row : L.rows - 1)) * p.H + h; };
  const int hw = w >> 1, lc = 16 * (w & 1) + col, c = c_base + lc;   // row half; channel
  const bool cin = c < p.K;

  // ---- the products over dv for this wave's tiles (rows 32 hw .. +31, channels
  //      c_base + 16 (w & 1) .. +15), kept in registers in MFMA output order:
  //      Y1 = dO S0^T, Y2 = dR S0^T and Z = U dS1^T; and rowsum(dS1 * S0) of the slice
  f32x4 y1a[2], y2a[2], za[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) { y1a[ii] = zero4(); y2a[ii] = zero4(); za[ii] = zero4(); }
  const int bch = tid >> 3, bc = c_base + bch;           // B piece: channel, 4 columns
  float ssp = 0.f;
  {
    const uint64_t vb = p.w.vbits[ch];
    const float* S0 = entry_state(p, S, s, h, n);
    const float* dS1 = p.w.dS1 + ch * (size_t)(KP * V);
    const float* Ug = p.w.U + ch * (size_t)(kC * V);
    const int arow = tid >> 2, ac8 = 8 * (tid & 3), bc4 = 4 * (tid & 7);   // A piece: row, 8 columns
    const bool arv = ((vb >> arow) & 1ull) != 0ull;
    // one slab's loads as they arrive, from addresses clamped in range (no load is
    // conditional); the next slab's are issued before this one is split into LDS
    struct Slab {
      Raw8<DT> dor;
      float4 dr[2], u[2], sv, dsv;
    };
    auto load_slab = [&](int vs, Slab& L) __attribute__((always_inline)) {
      const int va = 32 * vs + ac8, vas = va < V ? va : 0;
      L.dor.load((const Tp*)p.dout, tokc(arow) * V + vas);
      const float4* dr = reinterpret_cast<const float4*>(p.dv + tokc(arow) * V + vas);
      const float4* u = reinterpret_cast<const float4*>(Ug + arow * V + vas);
      L.dr[0] = dr[0]; L.dr[1] = dr[1];
      L.u[0] = u[0]; L.u[1] = u[1];
      const int vb4 = 32 * vs + bc4, vbs = vb4 < V ? vb4 : 0;
      L.sv = *reinterpret_cast<const float4*>(S0 != nullptr ? S0 + (size_t)(bc < p.K ? bc : 0) * V + vbs : dS1 + vbs);
      L.dsv = *reinterpret_cast<const float4*>(dS1 + (size_t)bc * V + vbs);
    };
    Slab cur, nxt;
    load_slab(0, cur);
#pragma unroll
    for (int vs = 0; vs < VS; ++vs) {
      if (vs + 1 < VS) load_slab(vs + 1, nxt);
      {
        const int v = 32 * vs + ac8;
        const bool vin = v < V, rok = vin && arv;
        float a[3][8];
        cur.dor.to_float(a[0]);
        const float4 q4[4] = {cur.dr[0], cur.dr[1], cur.u[0], cur.u[1]};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          a[1 + m][0] = q4[2 * m].x; a[1 + m][1] = q4[2 * m].y; a[1 + m][2] = q4[2 * m].z; a[1 + m][3] = q4[2 * m].w;
          a[1 + m][4] = q4[2 * m + 1].x; a[1 + m][5] = q4[2 * m + 1].y;
          a[1 + m][6] = q4[2 * m + 1].z; a[1 + m][7] = q4[2 * m + 1].w;
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[m][e] = (m == 2 ? vin : rok) ? a[m][e] : 0.f;
          bf16x8 hi, lo;
          split8(a[m], hi, lo);
          *reinterpret_cast<bf16x8*>(&s_ya[(2 * m) * kYA + arow * LA + ac8]) = hi;
          *reinterpret_cast<bf16x8*>(&s_ya[(2 * m + 1) * kYA + arow * LA + ac8]) = lo;
        }
      }
      {
        const int v = 32 * vs + bc4;
        const bool vin = v < V, sin = vin && S0 != nullptr && bc < p.K;
        const float4 s4 = cur.sv, d4 = cur.dsv;
        const float sv[4] = {sin ? s4.x : 0.f, sin ? s4.y : 0.f, sin ? s4.z : 0.f, sin ? s4.w : 0.f};
        const float dv[4] = {vin ? d4.x : 0.f, vin ? d4.y : 0.f, vin ? d4.z : 0.f, vin ? d4.w : 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) ssp += sv[e] * dv[e];
        split4_to_lds(sv, &s_yb[0 * kYB + bch * LA + bc4], &s_yb[1 * kYB + bch * LA + bc4]);
        split4_to_lds(dv, &s_yb[2 * kYB + bch * LA + bc4], &s_yb[3 * kYB + bch * LA + bc4]);
      }
      __syncthreads();
      const int br = (16 * (w & 1) + col) * LA + cg;
      const bf16x8 sh = *reinterpret_cast<const bf16x8*>(&s_yb[0 * kYB + br]);
      const bf16x8 sl = *reinterpret_cast<const bf16x8*>(&s_yb[1 * kYB + br]);
      const bf16x8 dsh = *reinterpret_cast<const bf16x8*>(&s_yb[2 * kYB + br]);
      const bf16x8 dsl = *reinterpret_cast<const bf16x8*>(&s_yb[3 * kYB + br]);
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int ar = (16 * (2 * hw + ii) + col) * LA + cg;
        bf16x8 ah[3], al[3];
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          ah[m] = *reinterpret_cast<const bf16x8*>(&s_ya[(2 * m) * kYA + ar]);
          al[m] = *reinterpret_cast<const bf16x8*>(&s_ya[(2 * m + 1) * kYA + ar]);
        }
        y1a[ii] = mma<DT == 0>(ah[0], al[0], sh, sl, y1a[ii]);
        y2a[ii] = mma<false>(ah[1], al[1], sh, sl, y2a[ii]);
        za[ii] = mma<false>(ah[2], al[2], dsh, dsl, za[ii]);
      }
      __syncthreads();
      if (vs + 1 < VS) cur = nxt;
    }
  }
  // rowsum(dS1 * S0): the eight threads of a channel are neighbouring lanes
  ssp += __shfl_xor(ssp, 1, 64);
  ssp += __shfl_xor(ssp, 2, 64);
  ssp += __shfl_xor(ssp, 4, 64);
  if ((tid & 7) == 0) s_ss[bch] = ssp;

  {
    // dP and dG into LDS (4096 values each, 16 per thread; the lower triangles kept)
    const float4* dPg = reinterpret_cast<const float4*>(p.w.dP + ch * (size_t)(kC * kC));
    const float4* dGg = reinterpret_cast<const float4*>(p.w.dG + ch * (size_t)(kC * kC));
    float4 pv[4], gv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { pv[j] = dPg[tid + j * kThreads]; gv[j] = dGg[tid + j * kThreads]; }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = 4 * (tid + j * kThreads), row = idx / kC, cl = idx % kC;
      const float pe[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w}, ge[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (cl + e <= row) {
          s_dP[tix(row, cl + e)] = pe[e];
          s_dG[tix(row, cl + e)] = ge[e];
        }
    }
  }
  Rows<DT, SW> R;
  load_rows<DT, SW, true>(p, L, h, c_base, R, s_tot, s_gl);
  if (lane < 16) { s_ok[r] = R.ok ? 1.f : 0.f; s_qsc[r] = R.qsc; s_ksc[r] = R.ksc; }
  const bool fast = __syncthreads_and(tid >= SW || s_gl[tid] >= kFastLimit);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int at = r * LD + cg + e;
    const float gv = R.g[0][e];
    s_g[at] = gv;
    if (fast) {
      const float gam = exp2f(gv);
      s_a[at] = R.k[0][e] * gam;
      s_b[at] = R.k[0][e] * exp2f(-gv);
      s_c[at] = R.q[0][e] * gam;
    } else {
      s_a[at] = R.k[0][e];
      s_b[at] = 0.f;
      s_c[at] = R.q[0][e];
    }
  }
  __syncthreads();
  const float ss = s_ss[lc];

  const float gl = s_gl[lc];
  float dl[2][4];
  float zk = 0.f;
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    const int I = 2 * hw + ii;
    // ---- the products over dv for tile I, and the raw k, q of the lane's rows
    const float y1[4] = {y1a[ii][0], y1a[ii][1], y1a[ii][2], y1a[ii][3]};
    const float y2[4] = {y2a[ii][0], y2a[ii][1], y2a[ii][2], y2a[ii][3]};
    const float z[4] = {za[ii][0], za[ii][1], za[ii][2], za[ii][3]};
    float kr[4], qr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t kat = tokc(16 * I + 4 * g4 + i) * p.K + (cin ? c : 0);
      kr[i] = E::ld((const Tp*)p.k, kat);
      qr[i] = E::ld((const Tp*)p.q, kat);
    }
    // ---- the decay-weighted C x C terms: Gam_i (dP Ki)_i, Gam_i (dG Ki)_i, (dP^T Qt)_j / Gam_j,
    //      (dG^T Kt)_j / Gam_j
    f32x4 xq = zero4(), xk1 = zero4(), xk2 = zero4(), xk3 = zero4();
    if (fast) {
      const int ra = 16 * I + col;                   // A-operand row
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int k0 = 32 * s2 + cg;
        if (s2 <= I / 2) {                           // columns j <= i
          float ap[8], ag[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool lo = k0 + e <= ra;
            const int at = tix(ra, lo ? k0 + e : 0);
            ap[e] = lo ? s_dP[at] : 0.f;
            ag[e] = lo ? s_dG[at] : 0.f;
            bv[e] = s_b[(k0 + e) * LD + lc];
          }
          bf16x8 bh, bl, hh, ll;
          split8(bv, bh, bl);
          split8(ap, hh, ll);
          xq = mma<false>(hh, ll, bh, bl, xq);
          split8(ag, hh, ll);
          xk3 = mma<false>(hh, ll, bh, bl, xk3);
        }
        if (32 * s2 + 31 >= 16 * I) {                // rows i >= j
          float ap[8], ag[8], bq[8], bk[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool lo = k0 + e >= ra;
            const int at = lo ? tix(k0 + e, ra) : 0;
            ap[e] = lo ? s_dP[at] : 0.f;
            ag[e] = lo ? s_dG[at] : 0.f;
            bq[e] = s_c[(k0 + e) * LD + lc];
            bk[e] = s_a[(k0 + e) * LD + lc];
          }
          bf16x8 bh, bl, hh, ll;
          split8(bq, bh, bl);
          split8(ap, hh, ll);
          xk1 = mma<false>(hh, ll, bh, bl, xk1);
          split8(bk, bh, bl);
          split8(ag, hh, ll);
          xk2 = mma<false>(hh, ll, bh, bl, xk2);
        }
      }
    }
    // ---- per element: dq, dk and the per-row decay gradient
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * I + 4 * g4 + i;
      const float gv = s_g[row * LD + lc];
      const bool ok = s_ok[row] != 0.f && cin;
      float kv = ok ? kr[i] : 0.f, qv = ok ? qr[i] : 0.f;
      if (p.qks != nullptr) {                        // the normalised rows
        kv *= s_ksc[row];
        qv *= s_qsc[row];
      }
      float Xq, Xk1, Xk2, Xk3;
      if (fast) {
        const float gm = exp2f(gv), gi = exp2f(-gv);
        Xq = gm * xq[i];
        Xk3 = gm * xk3[i];
        Xk1 = gi * xk1[i];
        Xk2 = gi * xk2[i];
      } else {
        Xq = 0.f; Xk1 = 0.f; Xk2 = 0.f; Xk3 = 0.f;
        for (int j = 0; j < kC; ++j) {
          const float gj = s_g[j * LD + lc];
          if (j <= row) {
            const float wgt = s_a[j * LD + lc] * exp2f(gv - gj);
            Xq += s_dP[tix(row, j)] * wgt;
            Xk3 += s_dG[tix(row, j)] * wgt;
          }
          if (j >= row) {
            const float d = exp2f(gj - gv);
            Xk1 += s_dP[tix(j, row)] * s_c[j * LD + lc] * d;
            Xk2 += s_dG[tix(j, row)] * s_a[j * LD + lc] * d;
          }
        }
      }
      const float gm = exp2f(gv), ekh = exp2f(gl - gv);
      const float a = Xk3 - gm * y2[i];              // Gam dKt
      const float bb = Xk1 + Xk2;                    // dKi / Gam
      const float dqv = gm * y1[i] + Xq;
      const float dkv = a + bb + z[i] * ekh;
      const float khv = kv * ekh;
      dl[ii][i] = ok ? kv * a - kv * bb + qv * dqv - z[i] * khv : 0.f;
      zk += ok ? z[i] * khv : 0.f;
      if (row < L.rows && cin) {
        p.dq[tok(row) * p.K + c] = ok ? dqv : 0.f;
        p.dk[tok(row) * p.K + c] = ok ? dkv : 0.f;
      }
    }
  }
  // ---- dlog_alpha: reverse sums over the rows, plus the Gam_last term; the two row halves
  //      of a channel exchange their totals through LDS
  zk += __shfl_xor(zk, 16, 64);
  zk += __shfl_xor(zk, 32, 64);
  float tile[2], after[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) tile[ii] = (dl[ii][0] + dl[ii][1]) + (dl[ii][2] + dl[ii][3]);
  // sums of the lanes holding later rows of the same tile (same column, larger l/16)
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    float later = 0.f, total = 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float x = __shfl(tile[ii], col + 16 * q4, 64);
      total += x;
      later += q4 > g4 ? x : 0.f;
    }
    after[ii] = later;
    tile[ii] = total;
  }
  if (g4 == 0) {
    s_half[hw][0][lc] = tile[0] + tile[1];
    s_half[hw][1][lc] = zk;
  }
  __syncthreads();
  const float dlast = s_half[0][1][lc] + s_half[1][1][lc] + exp2f(gl) * (cin ? ss : 0.f);
  float carry = dlast + (hw == 0 ? s_half[1][0][lc] : 0.f);
#pragma unroll
  for (int ii = 1; ii >= 0; --ii) {
    const int I = 2 * hw + ii;
    float run = carry + after[ii];
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const int row = 16 * I + 4 * g4 + i;
      run += dl[ii][i];
      if (row < L.rows && cin) p.dla[tok(row) * p.K + c] = s_ok[row] != 0.f ? run : 0.f;
    }
    carry += tile[ii];
  }
}

// ---------------------------------------------------------------- per-head gate (Gated DeltaNet)
// With one gate per (token, head) every channel decays alike: the kernels read the one value
// into every channel's registers, the per-channel pass runs unchanged on it (the forward that
// forms the chunk-end states runs the per-head prefill), and the gate's gradient is the sum
// of the per-channel ones (the chain rule through the broadcast), taken in a fixed order.
constexpr int kGateThreads = 256;
constexpr unsigned kGateMaxBlocks = 1u << 16;     // grid-stride loops past this

// K/8 neighbouring lanes per row, eight channels each (contiguous across the lanes of a
// row), then a butterfly over those lanes; every lane of a wave runs the same iterations, so
// the shuffles stay uniform, and the order of the sum is fixed
__global__ void __launch_bounds__(kGateThreads)
gate_reduce_kernel(const float* __restrict__ dla_pc, float* __restrict__ dla, size_t rows, int K) {
  const int lpr = K / 8;
  const size_t stride = (size_t)gridDim.x * kGateThreads;
  for (size_t base = (size_t)blockIdx.x * kGateThreads; base < rows * lpr; base += stride) {
    const size_t g = base + threadIdx.x, row = g / lpr;
    const int part = (int)(g % lpr);
    float s = 0.f;
    if (row < rows) {
      const float4* src = reinterpret_cast<const float4*>(dla_pc + row * K + part * 8);
      const float4 a = src[0], b = src[1];
      s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    }
    for (int o = 1; o < lpr; o <<= 1) s += __shfl_xor(s, o, 64);
    if (row < rows && part == 0) dla[row] = s;
  }
}

// ---------------------------------------------------------------- q/k L2 norm
// With the norm inside the call the pass differentiates with respect to the normalised rows
// x_hat = s x, s = (|x|^2 + 1e-6)^-1/2; this maps each row's gradient back to the raw row,
// in place: dx = s dx_hat - s^3 x (x . dx_hat).  A row is spread over K/8 neighbouring
// lanes, eight channels each, so every load and store is contiguous across the lanes of a
// row and the row is read once; the dot product is a butterfly over those lanes (every lane
// of a wave runs the same iterations).  A row whose scale is 0 (not valid) gets 0.
template <int DT>
__global__ void __launch_bounds__(kGateThreads)
l2_grad_kernel(const void* __restrict__ q, const void* __restrict__ k, const float2* __restrict__ qks,
               float* __restrict__ dq, float* __restrict__ dk, size_t rows, int K) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  const int lpr = K / 8;                                    // lanes per row: 2, 4, 8 or 16
  const size_t stride = (size_t)gridDim.x * kGateThreads;
  for (size_t base = (size_t)blockIdx.x * kGateThreads; base < rows * lpr; base += stride) {
    const size_t g = base + threadIdx.x, row = g / lpr;
    const bool in = row < rows;
    const size_t off = (in ? row : 0) * K + (size_t)(g % lpr) * 8;
    const float2 sc = qks[in ? row : 0];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const Tp* x = (const Tp*)(which == 0 ? q : k);
      float* d = which == 0 ? dq : dk;
      const float s = which == 0 ? sc.x : sc.y;
      float xv[8], gv[8];
      E::ld8(x, off, xv);
      Elem<1>::ld8(d, off, gv);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += xv[e] * gv[e];
      for (int o = 1; o < lpr; o <<= 1) dot += __shfl_xor(dot, o, 64);
      const float t = s * s * s * dot;
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = s != 0.f ? s * gv[e] - t * xv[e] : 0.f;
      if (in) Elem<1>::st8(d, off, out);
    }
  }
}

static unsigned gate_blocks(size_t items) {
  const size_t b = (items + kGateThreads - 1) / kGateThreads;
  return (unsigned)(b < kGateMaxBlocks ? b : kGateMaxBlocks);
}

// ---------------------------------------------------------------- packed sequences
// The sequence table (start, end, first checkpoint, first chunk) and the chunk table
// (sequence, chunk within it) from cu_seqlens: one workgroup scans the chunk counts and the
// 64-token checkpoint counts together (low and high 32 bits of one 64-bit sum).  Token bounds
// are clamped into [0, T]; a sequence whose chunks would pass the NC slots of the workspace is
// cut short, so a malformed cu_seqlens gives wrong results but no access outside a buffer.
constexpr int kSetupThreads = 1024;
__global__ void __launch_bounds__(kSetupThreads)
bwd_setup_kernel(const int32_t* __restrict__ cu, int N, int T, int NC, int4* __restrict__ seqs,
                 int2* __restrict__ cmap) {
  __shared__ long long s_scan[kSetupThreads];
  __shared__ long long s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < N; base += kSetupThreads) {
    const int i = base + tid;
    int start = 0, end = 0, nc = 0, nk = 0;
    if (i < N) {
      start = min(max(cu[i], 0), T);
      end = min(max(cu[i + 1], start), T);
      nc = (end - start + kC - 1) / kC;
      nk = (end - start) / kC;
    }
    const long long mine = ((long long)nk << 32) | (unsigned)nc;
    s_scan[tid] = mine;
    __syncthreads();
    for (int off = 1; off < kSetupThreads; off <<= 1) {      // inclusive scan of the counts
      const long long v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    const long long before = s_carry + s_scan[tid] - mine;
    const int first = (int)min(before & 0xffffffffll, (long long)NC);
    const int fit = min(nc, NC - first);
    if (i < N) {
      seqs[i] = make_int4(start, fit < nc ? start + fit * kC : end, (int)(before >> 32), first);
      for (int j = 0; j < fit; ++j) cmap[first + j] = make_int2(i, j);
    }
    __syncthreads();
    if (tid == kSetupThreads - 1) s_carry += s_scan[tid];
    __syncthreads();
  }
  for (int g = (int)min(s_carry & 0xffffffffll, (long long)NC) + tid; g < NC; g += kSetupThreads)
    cmap[g] = make_int2(-1, -1);
}

// ---------------------------------------------------------------- host side
// The chunk operands and gradients first, then what running the forward again needs (its
// workspace, its discarded outputs and the chunk-end states): `own` bytes suffice when the
// caller hands the states in.
struct Layout {
  size_t kh, wt, qt, pt, gam, vbits, G, M, dS1, dU, U, dP, dG, dlab, qks, seqs, cmap, own, fwd, o, fin, ck, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// chunk slots of the workspace per head: ceil(T / 64) per batch row, or for B packed
// sequences the bound ceil(T / 64) + B (each sequence adds at most one partial chunk)
long long chunk_slots(int B, int T, bool varlen) {
  const long long nc = T > 0 ? ((long long)T + kC - 1) / kC : 0;
  return varlen && T > 0 ? nc + B : nc;
}

Layout layout(int B, int T, int H, int dk, int dv, int dtype, bool scalar_gate, bool varlen, bool l2) {
  Layout L{};
  if (B == 0 || H == 0 || (T <= 0 && !varlen)) return L;
  const int KP = kpad(dk);
  const long long NC = chunk_slots(B, T, varlen);
  const size_t rows_b = varlen ? 1 : B, tokens = rows_b * (size_t)T;
  const size_t nch = rows_b * H * NC, parts = dtype == 1 ? 2 : 1, es = dtype == 1 ? 4 : 2;
  // checkpoints: B floor(T / 64) for a batch, at most floor(T / 64) for packed sequences
  const size_t nck = varlen ? (size_t)(T / kC) : (size_t)B * (T / kC);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  L.kh = take(nch * kC * KP * 2 * parts);
  L.wt = take(nch * kC * KP * 2 * parts);
  L.qt = take(nch * kC * KP * 2 * parts);
  L.pt = take(nch * kC * kC * 2 * 2);
  L.gam = take(nch * KP * 4);
  L.vbits = take(nch * 8);
  L.G = take(nch * kC * kC * 4);
  L.M = take(nch * kC * kC * 4);
  L.dS1 = take(nch * KP * dv * 4);
  L.dU = take(nch * kC * dv * 4);
  L.U = take(nch * kC * dv * 4);
  L.dP = take(nch * kC * kC * 4);
  L.dG = take(nch * kC * kC * 4);
  if (scalar_gate) {                        // the gate on every channel, and its per-channel gradient
    L.dlab = take(tokens * H * dk * 4);
  }
  if (l2) L.qks = take(tokens * H * 8);     // the row scales of q and k
  if (varlen) {
    L.seqs = take((size_t)B * 16);
    L.cmap = take((size_t)NC * 8);
  }
  L.own = off;
  L.fwd = take(T > 0 ? prefill_workspace_bytes(B, T, H, dk, dv, kC, dtype, varlen) : 0);
  L.o = take(tokens * H * dv * es);
  L.fin = take((size_t)B * H * dk * dv * 4);
  L.ck = take(nck * H * dk * dv * 4);
  L.total = off;
  return L;
}

template <int DT, int KP, int V>
hipError_t launch_t(const Params& p, hipStream_t st) {
  const int rows_b = p.cmap != nullptr ? 1 : p.B;     // packed: one row of chunk slots
  const dim3 cgrid(p.NC * p.H, rows_b);
  if (p.NC > 0) {
    hipLaunchKernelGGL((bwd_prep_kernel<DT, KP>), cgrid, dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 32-column scan workgroups (bf16) once there are enough (b, h) pairs to fill the chip with them
  constexpr bool kWideOk = DT == 0 && V >= 32;
  const int groups = (p.B * p.H + 7) / 8;
  if (kWideOk && p.B * p.H >= 64)
    hipLaunchKernelGGL((bwd_scan_kernel<DT, KP, V, kWideOk ? 2 : 1>), dim3(groups * 8 * (V / 32)), dim3(kThreads),
                       0, st, p);
  else
    hipLaunchKernelGGL((bwd_scan_kernel<DT, KP, V, 1>), dim3(groups * 8 * (V / 16)), dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.NC == 0) return e;
  hipLaunchKernelGGL((bwd_cc_kernel<DT, KP, V>), cgrid, dim3(kThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long cgroups = ((long long)rows_b * p.NC * p.H + 7) / 8;
  hipLaunchKernelGGL((bwd_ck_kernel<DT, KP, V>), dim3((unsigned)(cgroups * 8 * (KP / kCkSlice))), dim3(kThreads), 0,
                     st, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const Params& p, hipStream_t st) {
  const int KP = kpad(p.K);
#define KDA_BWD(KK, VV) \
  if (KP == KK && p.V == VV) return launch_t<DT, KK, VV>(p, st);
  KDA_BWD(32, 16) KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
  KDA_BWD(64, 16) KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
  KDA_BWD(128, 16) KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
  return hipErrorInvalidValue;
}

}  // namespace

// the x extent of every backward launch in threads fits 32 bits (the forward's own grids are
// checked by prefill_grid_ok): the chunk-local grid (H times the chunk slots workgroups), the
// scan (B H rounded up to 8, times up to 8 column tiles) and the channel-slice grid (the
// chunk-local workgroups rounded up to 8, times up to 4 slices)
bool backward_grid_ok(int B, int T, int H, bool varlen) {
  const long long kMax = 0xffffffffll, NC = chunk_slots(B, T, varlen);
  const long long nbh = (long long)B * H, chunks = (varlen ? 1 : B) * NC * H;
  return NC * H * kThreads <= kMax && (nbh + 7) / 8 * 8 * 8 * kThreads <= kMax &&
         (chunks + 7) / 8 * 8 * (128 / kCkSlice) * kThreads <= kMax;
}

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype, bool states_given,
                                bool scalar_gate, bool varlen, bool l2) {
  const Layout L = layout(B, T, H, dk, dv, dtype, scalar_gate, varlen, l2);
  return states_given ? L.own : L.total;
}

hipError_t launch_backward(const BackwardArgs& a) {
  const bool varlen = a.cu_seqlens != nullptr;
  const bool l2 = a.l2norm != 0;
  const Layout L = layout(a.B, a.T, a.H, a.dk_, a.dv_, a.dtype, a.scalar_gate != 0, varlen, l2);
  unsigned char* ws = (unsigned char*)a.workspace;
  hipStream_t st = (hipStream_t)a.stream;
  const int NC = (int)chunk_slots(a.B, a.T, varlen), NCf = a.T / kC;
  const size_t rows = (size_t)(varlen ? 1 : a.B) * a.T * a.H;
  if (varlen) {
    hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), dim3(kSetupThreads), 0, st, a.cu_seqlens, a.B, a.T, NC,
                       (int4*)(ws + L.seqs), (int2*)(ws + L.cmap));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the per-head gate's per-channel gradient goes to the workspace, then is summed
  const float* la = a.log_alpha;
  float* dla = a.dla;
  if (a.scalar_gate && rows > 0) dla = (float*)(ws + L.dlab);
  // checkpoints the pass may read: the caller's count, or what the forward below writes
  const int own_states = varlen ? NCf : a.B * NCf;
  if (a.T > 0 && a.chunk_states == nullptr) {
    // the forward pass again, keeping the state at every chunk end
    PrefillArgs f{};
    // (with the per-head gate, the per-head forward the caller runs: its chunk-end states
    // are the ones that call saves, bit for bit)
    f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.scalar_gate = a.scalar_gate;
    f.beta = a.beta; f.mask = a.mask;
    f.init_state = a.init_state;
    f.o = ws + L.o;
    f.final_state = (float*)(ws + L.fin);
    f.B = a.B; f.T = a.T; f.H = a.H; f.dk = a.dk_; f.dv = a.dv_; f.chunk = kC; f.dtype = a.dtype;
    f.workspace = ws + L.fwd;
    f.workspace_bytes = L.o - L.fwd;
    f.stream = a.stream;
    f.cu_seqlens = a.cu_seqlens;
    f.l2norm = l2 ? 1 : 0;
    f.chunk_states = own_states > 0 ? (float*)(ws + L.ck) : nullptr;
    f.num_states = own_states;
    f.state_interval = kC;
    f.serial_scan = 1;
    const hipError_t e = launch_prefill(f);
    if (e != hipSuccess) return e;
  }
  Params p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
  p.la = la; p.beta = a.beta; p.init = a.init_state; p.dfinal = a.dfinal; p.mask = a.mask;
  p.sgate = a.scalar_gate != 0;
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dla = dla; p.dbeta = a.dbeta; p.dinit = a.dinit;
  if (a.T > 0) {
    p.w.kh = (uint16_t*)(ws + L.kh); p.w.wt = (uint16_t*)(ws + L.wt); p.w.qt = (uint16_t*)(ws + L.qt);
    p.w.pt = (uint16_t*)(ws + L.pt);
    p.w.gam = (float*)(ws + L.gam); p.w.G = (float*)(ws + L.G); p.w.M = (float*)(ws + L.M);
    p.w.vbits = (uint64_t*)(ws + L.vbits);
    p.w.dS1 = (float*)(ws + L.dS1); p.w.dU = (float*)(ws + L.dU); p.w.U = (float*)(ws + L.U);
    p.w.dP = (float*)(ws + L.dP); p.w.dG = (float*)(ws + L.dG);
    p.w.ck = a.chunk_states != nullptr ? a.chunk_states : (const float*)(ws + L.ck);
  }
  if (varlen) {
    p.seqs = (const int4*)(ws + L.seqs);
    p.cmap = (const int2*)(ws + L.cmap);
  }
  if (l2 && rows > 0) p.qks = (float2*)(ws + L.qks);
  p.num_states = a.chunk_states != nullptr ? (varlen ? a.num_states : a.B * NCf) : own_states;
  p.B = a.B; p.T = a.T; p.H = a.H; p.K = a.dk_; p.V = a.dv_; p.NC = NC; p.NCf = NCf;
  hipError_t e = a.dtype == 0 ? launch_dt<0>(p, st) : launch_dt<1>(p, st);
  if (e != hipSuccess || rows == 0) return e;
  if (l2) {
    // dq and dk so far are with respect to the normalised rows
    if (a.dtype == 0)
      hipLaunchKernelGGL(l2_grad_kernel<0>, dim3(gate_blocks(rows * (a.dk_ / 8))), dim3(kGateThreads), 0, st, a.q,
                         a.k, (const float2*)p.qks, a.dq, a.dk, rows, a.dk_);
    else
      hipLaunchKernelGGL(l2_grad_kernel<1>, dim3(gate_blocks(rows * (a.dk_ / 8))), dim3(kGateThreads), 0, st, a.q,
                         a.k, (const float2*)p.qks, a.dq, a.dk, rows, a.dk_);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!a.scalar_gate) return hipSuccess;
  hipLaunchKernelGGL(gate_reduce_kernel, dim3(gate_blocks(rows * (a.dk_ / 8))), dim3(kGateThreads), 0, st,
                     (const float*)dla, a.dla, rows, a.dk_);
  return hipGetLastError();
}

}  // namespace kda
