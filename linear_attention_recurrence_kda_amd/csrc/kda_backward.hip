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
// The pass runs as five launches on the caller's stream:
//   1. the forward prefill, saving the state at every chunk end (its own kernels);
//   2. bwd_prep_kernel, one workgroup per (chunk, head): G, P, M = (I + A)^-1 and W, and the
//      reverse scan's operands Kh, W^T, Qt^T and P^T as bf16 MFMA fragments;
//   3. bwd_scan_kernel, one workgroup per (b, h, 16-column dv tile), over the chunks from the
//      last: dS1 and dU of every chunk, and dinit;
//   4. bwd_cc_kernel, one workgroup per (chunk, head): R, U, dv, dT', dbeta, dA, dG and dP;
//   5. bwd_ck_kernel, one workgroup per (chunk, head): dq, dk and dlog_alpha.
// Products run on the bf16 MFMA with fp32 operands split into a bf16 high part and residual
// (three MFMAs per product), except the reverse scan's Kh, W^T and Qt^T, which are single
// bf16 with bf16 inputs (as the forward scan's Wn, Qt and Kh^T are).  A chunk in which some
// channel decays below 2^-120 cannot use the factorised products (Gam and 1/Gam would leave
// the fp32 range); it computes the decay-weighted C x C terms entry by entry instead.
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
  float *dS1, *dU;                       // dL/dS at the chunk end [KP][V], dL/dU [C][V]
  float *U, *dP, *dPt, *dG, *dGt;        // U [C][V]; dP, dG and their transposes [C][C]
  const float* ck;                       // forward states at chunk ends [B * NCf][H][K][V]
};

struct Params {
  const void *q, *k, *v, *dout;
  const float *la, *beta, *init, *dfinal;
  const uint8_t* mask;
  float *dq, *dk, *dv, *dla, *dbeta, *dinit;
  Ws w;
  int B, T, H, K, V, NC, NCf;
};

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

__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

// One lane's view of chunk n: row 16 w + l%16 (w = wave), channels 32 ks + 8 (l/16) .. +7
// (the A-operand layout).  q, k and log_alpha of rows that are not valid (masked or past T)
// and of channels past K are 0.  g becomes the inclusive cumulative sum of log2 decay over
// the chunk's rows and s_gl the chunk's totals per channel.  Every thread must call it (it
// holds two barriers).
template <int DT, int KP>
struct Rows {
  static constexpr int KS = KP / 32;
  float k[KS][8], q[KS][8], g[KS][8];
  float beta;
  bool ok;
};

template <int DT, int KP, bool WANT_Q>
__device__ __forceinline__ void load_rows(const Params& p, int b, int h, int n, Rows<DT, KP>& R,
                                          float* s_tot, float* s_gl) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = 16 * w + (lane & 15), cg = 8 * (lane >> 4);
  const int t = n * kC + r;
  const int ts = t < p.T ? t : p.T - 1;
  const size_t tk = ((size_t)b * p.T + ts) * p.H + h;
  R.ok = t < p.T && (p.mask == nullptr || p.mask[(size_t)b * p.T + ts] != 0);
  R.beta = R.ok ? p.beta[tk] : 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = 32 * ks + cg;
    if (R.ok && c0 < p.K) {
      E::ld8((const Tp*)p.k, tk * p.K + c0, R.k[ks]);
      if (WANT_Q) E::ld8((const Tp*)p.q, tk * p.K + c0, R.q[ks]);
      Elem<1>::ld8(p.la, tk * p.K + c0, R.g[ks]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { R.k[ks][e] = 0.f; R.q[ks][e] = 0.f; R.g[ks][e] = 0.f; }
    }
    if (!WANT_Q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) R.q[ks][e] = 0.f;
    }
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
      for (int e = 0; e < 8; ++e) s_tot[w * KP + 32 * ks + cg + e] = R.g[ks][e];
  }
  __syncthreads();
  if (tid < KP) {
    float run = 0.f;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      const float x = s_tot[J * KP + tid];
      s_tot[J * KP + tid] = run;
      run += x;
    }
    s_gl[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) R.g[ks][e] += s_tot[w * KP + 32 * ks + cg + e];
}

// the chunk's entry state: the initial state for the first chunk, else the forward's
// state at the end of the chunk before (null: zero)
__device__ __forceinline__ const float* entry_state(const Params& p, int b, int h, int n) {
  if (n == 0) return p.init == nullptr ? nullptr : p.init + ((size_t)b * p.H + h) * p.K * p.V;
  return p.w.ck + (((size_t)b * p.NCf + n - 1) * p.H + h) * p.K * p.V;
}

// ================================================================ 2. prep
template <int DT, int KP>
__global__ void __launch_bounds__(kThreads) bwd_prep_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32, CT = KP / 16, LD = KP + 2, LC = kC + 2;
  constexpr bool SPLIT = DT == 1;
  constexpr int parts = SPLIT ? 2 : 1;
  __shared__ __attribute__((aligned(16))) float s_kt[kC * LD];   // Kt
  __shared__ __attribute__((aligned(16))) float s_qt[kC * LD];   // Qt
  __shared__ __attribute__((aligned(16))) float s_x[kC * LD];    // Ki, or g on the exact path
  __shared__ __attribute__((aligned(16))) float s_A[kC * LC];
  __shared__ __attribute__((aligned(16))) float s_M[kC * LC];    // P, then M
  __shared__ float s_tot[4 * KP], s_gl[KP], s_beta[kC], s_ok[kC];

  const int n = blockIdx.x / p.H, h = blockIdx.x % p.H, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = ((size_t)b * p.H + h) * p.NC + n;

  Rows<DT, KP> R;
  load_rows<DT, KP, true>(p, b, h, n, R, s_tot, s_gl);
  if (lane < 16) { s_beta[r] = R.beta; s_ok[r] = R.ok ? 1.f : 0.f; }
  const bool fast = __syncthreads_and(tid >= KP || s_gl[tid] >= kFastLimit);

  // ---- decayed rows: Kt, Qt (and Ki or g) to LDS, Kh fragments to the workspace
  uint16_t* kh = p.w.kh + ch * (size_t)(kC * KP * parts);
  bf16x8 kth[KS], ktl[KS], qth[KS], qtl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float kt[8], qt[8], khv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = 32 * ks + cg + e;
      const float gv = R.g[ks][e], gam = exp2f(gv);
      kt[e] = R.k[ks][e] * gam;
      qt[e] = R.q[ks][e] * gam;
      khv[e] = R.k[ks][e] * exp2f(s_gl[c] - gv);
      s_kt[r * LD + c] = kt[e];
      s_qt[r * LD + c] = qt[e];
      s_x[r * LD + c] = fast ? R.k[ks][e] * exp2f(-gv) : gv;
    }
    split8(kt, kth[ks], ktl[ks]);
    split8(qt, qth[ks], qtl[ks]);
    bf16x8 hi, lo;
    split8(khv, hi, lo);
    *reinterpret_cast<bf16x8*>(kh + afrag(w, ks, lane, KP)) = hi;
    if (SPLIT) *reinterpret_cast<bf16x8*>(kh + kC * KP + afrag(w, ks, lane, KP)) = lo;
  }
  __syncthreads();

  // ---- G (strictly lower), A = Diag(beta) G and P (lower, staged in s_M): wave w, row tile w
  float* Gg = p.w.G + ch * (size_t)(kC * kC);
  if (fast) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 ga = zero4(), pa = zero4();
      if (J <= w) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float bv[8];
          lds8(&s_x[(16 * J + col) * LD + 32 * ks + cg], bv);
          bf16x8 bh, bl;
          split8(bv, bh, bl);
          ga = mfma16(kth[ks], bh, ga);
          ga = mfma16(ktl[ks], bh, ga);
          ga = mfma16(kth[ks], bl, ga);
          pa = mfma16(qth[ks], bh, pa);
          pa = mfma16(qtl[ks], bh, pa);
          pa = mfma16(qth[ks], bl, pa);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const float gv = (J <= w && cl < row) ? ga[i] : 0.f;
        const float pv = (J <= w && cl <= row) ? pa[i] : 0.f;
        s_A[row * LC + cl] = s_beta[row] * gv;
        s_M[row * LC + cl] = pv;
        Gg[row * kC + cl] = gv;
      }
    }
  } else {
    // exact pairwise decays exp2(g_i - g_j) <= 1, entry by entry
    const Tp* kg = (const Tp*)p.k;
    const Tp* qg = (const Tp*)p.q;
    for (int idx = tid; idx < kC * kC; idx += kThreads) {
      const int i = idx / kC, j = idx % kC;
      float gs = 0.f, ps = 0.f;
      if (j <= i && s_ok[i] != 0.f && s_ok[j] != 0.f) {
        const size_t ti = (((size_t)b * p.T + n * kC + i) * p.H + h) * p.K;
        const size_t tj = (((size_t)b * p.T + n * kC + j) * p.H + h) * p.K;
        for (int c = 0; c < p.K; ++c) {
          const float d = exp2f(s_x[i * LD + c] - s_x[j * LD + c]);
          const float kj = E::ld(kg, tj + c) * d;
          gs += E::ld(kg, ti + c) * kj;
          ps += E::ld(qg, ti + c) * kj;
        }
      }
      gs = j < i ? gs : 0.f;
      s_A[i * LC + j] = s_beta[i] * gs;
      s_M[i * LC + j] = ps;
      Gg[i * kC + j] = gs;
    }
  }
  __syncthreads();

  // ---- P^T and Qt^T fragments (rows of P^T / channels, contraction over chunk rows), Gam_last
  {
    uint16_t* pt = p.w.pt + ch * (size_t)(2 * kC * kC);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = s_M[(32 * s + cg + e) * LC + 16 * w + col];
      bf16x8 hi, lo;
      split8(pv, hi, lo);
      *reinterpret_cast<bf16x8*>(pt + afrag(w, s, lane, kC)) = hi;
      *reinterpret_cast<bf16x8*>(pt + kC * kC + afrag(w, s, lane, kC)) = lo;
    }
    uint16_t* qtw = p.w.qt + ch * (size_t)(kC * KP * parts);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ct = w + 4 * m;
      if (ct >= CT) continue;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = s_qt[(32 * s + cg + e) * LD + 16 * ct + col];
        bf16x8 hi, lo;
        split8(qv, hi, lo);
        *reinterpret_cast<bf16x8*>(qtw + afrag(ct, s, lane, kC)) = hi;
        if (SPLIT) *reinterpret_cast<bf16x8*>(qtw + kC * KP + afrag(ct, s, lane, kC)) = lo;
      }
    }
    if (tid < KP) p.w.gam[ch * KP + tid] = exp2f(s_gl[tid]);
  }
  __syncthreads();

  // ---- M = (I + A)^-1 by forward substitution, one column per lane of wave 0 (fp32)
  if (w == 0) {
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float a0 = (i == lane) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < i; ++s2) {
        const float av = s_A[i * LC + s2];
        if (s2 & 1) a1 -= av * x[s2];
        else a0 -= av * x[s2];
      }
      x[i] = a0 + a1;
    }
    float* Mg = p.w.M + ch * (size_t)(kC * kC);
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      s_M[i * LC + lane] = x[i];
      Mg[i * kC + lane] = x[i];
    }
  }
  __syncthreads();

  // ---- W = -T' Kt, computed per channel tile and turned into W^T fragments by lane swaps
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
            bv[e] = s_kt[j * LD + 16 * ct + col];
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
template <int DT, int KP, int V>
__global__ void __launch_bounds__(kThreads) bwd_scan_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr bool SPLIT = DT == 1;
  constexpr int parts = SPLIT ? 2 : 1;
  constexpr int RTK = KP / 16, MPW = (RTK + 3) / 4, KS = KP / 32, NT = V / 16;
  __shared__ __attribute__((aligned(16))) __bf16 s_lam[2][16 * KP];   // [part][column][row]
  __shared__ __attribute__((aligned(16))) __bf16 s_du[2][16 * kC];
  __shared__ __attribute__((aligned(16))) __bf16 s_do[2][16 * kC];

  const int vt = blockIdx.x % NT, bh = blockIdx.x / NT, b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g4 = lane >> 4, vc = 16 * vt + col;

  float lam[MPW][4];
#pragma unroll
  for (int m = 0; m < MPW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = w + 4 * m, row = 16 * rt + 4 * g4 + i;
      lam[m][i] = (rt < RTK && row < p.K && p.dfinal != nullptr) ? p.dfinal[((size_t)bh * p.K + row) * V + vc] : 0.f;
    }

  for (int n = p.NC - 1; n >= 0; --n) {
    const size_t ch = (size_t)bh * p.NC + n;
    float* dS1 = p.w.dS1 + ch * (size_t)(KP * V);
#pragma unroll
    for (int m = 0; m < MPW; ++m) {
      const int rt = w + 4 * m;
      if (rt >= RTK) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) dS1[(16 * rt + 4 * g4 + i) * V + vc] = lam[m][i];
      split4_to_lds(lam[m], &s_lam[0][col * KP + 16 * rt + 4 * g4], &s_lam[1][col * KP + 16 * rt + 4 * g4]);
    }
    {
      // dO of the chunk's rows (0 where not valid), transposed into [column][row]
      const int row = tid >> 2, c4 = 4 * (tid & 3), t = n * kC + row;
      float vals[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < p.T && (p.mask == nullptr || p.mask[(size_t)b * p.T + t] != 0))
        E::ld4((const Tp*)p.dout, (((size_t)b * p.T + t) * p.H + h) * V + 16 * vt + c4, vals);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const __bf16 hi = (__bf16)vals[e];
        s_do[0][(c4 + e) * kC + row] = hi;
        if (SPLIT) s_do[1][(c4 + e) * kC + row] = (__bf16)(vals[e] - (float)hi);
      }
    }
    __syncthreads();

    // ---- dU, row tile w: Kh dS1 + P^T dO
    {
      const uint16_t* kh = p.w.kh + ch * (size_t)(kC * KP * parts);
      const uint16_t* pt = p.w.pt + ch * (size_t)(2 * kC * kC);
      f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(kh + afrag(w, ks, lane, KP));
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&s_lam[0][col * KP + 32 * ks + 8 * g4]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&s_lam[1][col * KP + 32 * ks + 8 * g4]);
        a0 = mfma16(ah, bh, a0);
        a1 = mfma16(ah, bl, a1);
        if (SPLIT) a2 = mfma16(*reinterpret_cast<const bf16x8*>(kh + kC * KP + afrag(w, ks, lane, KP)), bh, a2);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s + 31 < 16 * w) continue;          // P^T is upper triangular
        const bf16x8 ph = *reinterpret_cast<const bf16x8*>(pt + afrag(w, s, lane, kC));
        const bf16x8 pl = *reinterpret_cast<const bf16x8*>(pt + kC * kC + afrag(w, s, lane, kC));
        const bf16x8 dh = *reinterpret_cast<const bf16x8*>(&s_do[0][col * kC + 32 * s + 8 * g4]);
        a0 = mfma16(ph, dh, a0);
        a1 = mfma16(pl, dh, a1);
        if (SPLIT) a2 = mfma16(ph, *reinterpret_cast<const bf16x8*>(&s_do[1][col * kC + 32 * s + 8 * g4]), a2);
      }
      float du[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = a0[i] + (a1[i] + a2[i]);
      float* dU = p.w.dU + ch * (size_t)(kC * V);
#pragma unroll
      for (int i = 0; i < 4; ++i) dU[(16 * w + 4 * g4 + i) * V + vc] = du[i];
      split4_to_lds(du, &s_du[0][col * kC + 16 * w + 4 * g4], &s_du[1][col * kC + 16 * w + 4 * g4]);
    }
    __syncthreads();

    // ---- lam <- Diag(Gam_last) lam + W^T dU + Qt^T dO
    {
      const uint16_t* wt = p.w.wt + ch * (size_t)(kC * KP * parts);
      const uint16_t* qt = p.w.qt + ch * (size_t)(kC * KP * parts);
      const float* gam = p.w.gam + ch * KP;
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        const int rt = w + 4 * m;
        if (rt >= RTK) continue;
        f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const size_t fo = afrag(rt, s, lane, kC);
          const bf16x8 wh = *reinterpret_cast<const bf16x8*>(wt + fo);
          const bf16x8 qh = *reinterpret_cast<const bf16x8*>(qt + fo);
          const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&s_du[0][col * kC + 32 * s + 8 * g4]);
          const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&s_du[1][col * kC + 32 * s + 8 * g4]);
          const bf16x8 dh = *reinterpret_cast<const bf16x8*>(&s_do[0][col * kC + 32 * s + 8 * g4]);
          a0 = mfma16(wh, uh, a0);
          a1 = mfma16(wh, ul, a1);
          a0 = mfma16(qh, dh, a0);
          if (SPLIT) {
            const bf16x8 dl = *reinterpret_cast<const bf16x8*>(&s_do[1][col * kC + 32 * s + 8 * g4]);
            a2 = mfma16(*reinterpret_cast<const bf16x8*>(wt + kC * KP + fo), uh, a2);
            a2 = mfma16(*reinterpret_cast<const bf16x8*>(qt + kC * KP + fo), dh, a2);
            a1 = mfma16(qh, dl, a1);
          }
        }
        const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * rt + 4 * g4);
        const float gg[4] = {gm.x, gm.y, gm.z, gm.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) lam[m][i] = gg[i] * lam[m][i] + (a0[i] + (a1[i] + a2[i]));
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < MPW; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = w + 4 * m, row = 16 * rt + 4 * g4 + i;
      if (rt < RTK && row < p.K) p.dinit[((size_t)bh * p.K + row) * V + vc] = lam[m][i];
    }
}

// ================================================================ 4. C x C gradients
template <int DT, int KP, int V>
__global__ void __launch_bounds__(kThreads) bwd_cc_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32, LD = KP + 2, LV = V + 2, LC = kC + 2, VT = V / 16, VS = (V + 31) / 32;
  constexpr int LB = LD > LV ? LD : LV;
  __shared__ __attribute__((aligned(16))) float s_big[kC * LB];  // Kt (stride LD), then dU (stride LV)
  __shared__ __attribute__((aligned(16))) float s_R[kC * LV];
  __shared__ __attribute__((aligned(16))) float s_U[kC * LV];
  __shared__ __attribute__((aligned(16))) float s_M[kC * LC];
  __shared__ __attribute__((aligned(16))) float s_dT[kC * LC];
  __shared__ __attribute__((aligned(16))) float s_X[kC * LC];
  __shared__ float s_tot[4 * KP], s_gl[KP], s_beta[kC], s_ok[kC], s_db[kC];

  const int n = blockIdx.x / p.H, h = blockIdx.x % p.H, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = ((size_t)b * p.H + h) * p.NC + n;
  auto tok = [&](int row) -> size_t { return ((size_t)b * p.T + n * kC + row) * p.H + h; };

  Rows<DT, KP> R;
  load_rows<DT, KP, false>(p, b, h, n, R, s_tot, s_gl);
  if (lane < 16) { s_beta[r] = R.beta; s_ok[r] = R.ok ? 1.f : 0.f; }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_big[r * LD + 32 * ks + cg + e] = R.k[ks][e] * exp2f(R.g[ks][e]);
  const float* Mg = p.w.M + ch * (size_t)(kC * kC);
  for (int idx = tid; idx < kC * kC; idx += kThreads) s_M[(idx / kC) * LC + idx % kC] = Mg[idx];
  __syncthreads();

  // ---- R = V - Kt S0: wave w takes column tiles w and w + 4, all row tiles
  const float* S0 = entry_state(p, b, h, n);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int vt = w + 4 * m;
    if (vt >= VT) continue;
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = 32 * ks + cg + e;
        bv[e] = (S0 != nullptr && c < p.K) ? S0[(size_t)c * V + 16 * vt + col] : 0.f;
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        float av[8];
        lds8(&s_big[(16 * I + col) * LD + 32 * ks + cg], av);
        acc[I] = mm3(av, bv, acc[I]);
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * g4 + i;
        const float vv = s_ok[row] != 0.f ? E::ld((const Tp*)p.v, tok(row) * V + 16 * vt + col) : 0.f;
        s_R[row * LV + 16 * vt + col] = vv - acc[I][i];
      }
  }
  __syncthreads();

  // ---- U = T' R (to LDS and the workspace); dU of the chunk into s_big
  {
    float* Ug = p.w.U + ch * (size_t)(kC * V);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int vt = w + 4 * m;
      if (vt >= VT) continue;
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s > I / 2) continue;
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 32 * s + cg + e;
            av[e] = s_M[(16 * I + col) * LC + j] * s_beta[j];
            bv[e] = s_R[j * LV + 16 * vt + col];
          }
          acc = mm3(av, bv, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * I + 4 * g4 + i;
          s_U[row * LV + 16 * vt + col] = acc[i];
          Ug[row * V + 16 * vt + col] = acc[i];
        }
      }
    }
    const float* dUg = p.w.dU + ch * (size_t)(kC * V);
    for (int idx = tid; idx < kC * V; idx += kThreads) s_big[(idx / V) * LV + idx % V] = dUg[idx];
  }
  __syncthreads();

  // ---- dV = dR = T'^T dU
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int vt = w + 4 * m;
    if (vt >= VT) continue;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (32 * s + 31 < 16 * I) continue;          // T'^T is upper triangular
        float av[8], bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = 32 * s + cg + e;
          av[e] = s_M[rr * LC + 16 * I + col] * s_beta[16 * I + col];
          bv[e] = s_big[rr * LV + 16 * vt + col];
        }
        acc = mm3(av, bv, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * g4 + i;
        if (n * kC + row < p.T) p.dv[tok(row) * V + 16 * vt + col] = s_ok[row] != 0.f ? acc[i] : 0.f;
      }
    }
  }
  // ---- dT' = dU R^T (lower) and dP = lower(dO U^T): row tile w
  {
    float* dP = p.w.dP + ch * (size_t)(kC * kC);
    float* dPt = p.w.dPt + ch * (size_t)(kC * kC);
    float dov[VS][8];
    const bool rok = s_ok[r] != 0.f;
#pragma unroll
    for (int vs = 0; vs < VS; ++vs) {
      const int v0 = 32 * vs + cg;
      if (rok && v0 < V) E::ld8((const Tp*)p.dout, tok(r) * V + v0, dov[vs]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) dov[vs][e] = 0.f;
      }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 at = zero4(), ap = zero4();
      if (J <= w) {
#pragma unroll
        for (int vs = 0; vs < VS; ++vs) {
          const int v0 = 32 * vs + cg;
          float du[8], rv[8], uv[8];
          if (v0 < V) {
            lds8(&s_big[r * LV + v0], du);
            lds8(&s_R[(16 * J + col) * LV + v0], rv);
            lds8(&s_U[(16 * J + col) * LV + v0], uv);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { du[e] = 0.f; rv[e] = 0.f; uv[e] = 0.f; }
          }
          at = mm3(du, rv, at);
          ap = mm3(dov[vs], uv, ap);
        }
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const bool lo = J <= w && cl <= row;
        s_dT[row * LC + cl] = lo ? at[i] : 0.f;
        pv[i] = lo ? ap[i] : 0.f;
        dP[row * kC + cl] = pv[i];
      }
      *reinterpret_cast<float4*>(&dPt[(16 * J + col) * kC + 16 * w + 4 * g4]) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    }
  }
  __syncthreads();

  // ---- dbeta through T' (column sums of dT' * M) and X = dT' Diag(beta) M^T
  float db = 0.f;
  if (tid < kC)
    for (int rr = tid; rr < kC; ++rr) db += s_dT[rr * LC + tid] * s_M[rr * LC + tid];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s > w / 2 || s > J / 2) continue;
      float av[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 32 * s + cg + e;
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
    const float* Gg = p.w.G + ch * (size_t)(kC * kC);
    float* dG = p.w.dG + ch * (size_t)(kC * kC);
    float* dGt = p.w.dGt + ch * (size_t)(kC * kC);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 acc = zero4();
      if (J <= w) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (32 * s + 31 < 16 * w) continue;        // M^T is upper triangular
          float av[8], bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = 32 * s + cg + e;
            av[e] = s_M[rr * LC + r];
            bv[e] = s_X[rr * LC + 16 * J + col];
          }
          acc = mm3(av, bv, acc);
        }
      }
      float gv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * w + 4 * g4 + i, cl = 16 * J + col;
        const float da = (J <= w && cl < row) ? -acc[i] : 0.f;
        part[i] += da * Gg[row * kC + cl];
        gv[i] = s_beta[row] * da;
        dG[row * kC + cl] = gv[i];
      }
      *reinterpret_cast<float4*>(&dGt[(16 * J + col) * kC + 16 * w + 4 * g4]) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sum16(part[i]);
      if (col == 0) s_db[16 * w + 4 * g4 + i] = x;
    }
  }
  __syncthreads();
  if (tid < kC && n * kC + tid < p.T) p.dbeta[tok(tid)] = s_ok[tid] != 0.f ? db + s_db[tid] : 0.f;
}

// ================================================================ 5. q, k and decay gradients
// Wave w takes channel tiles w and w + 4 with all four row tiles, so each lane holds 16 rows
// of one channel and the reverse sum over rows for dlog_alpha stays in registers and lane
// shuffles.
template <int DT, int KP, int V>
__global__ void __launch_bounds__(kThreads) bwd_ck_kernel(Params p) {
  using E = Elem<DT>;
  using Tp = typename E::T;
  constexpr int KS = KP / 32, CT = KP / 16, LD = KP + 2, VS = (V + 31) / 32;
  __shared__ __attribute__((aligned(16))) float s_a[kC * LD];    // Kt, or k on the exact path
  __shared__ __attribute__((aligned(16))) float s_b[kC * LD];    // Ki (fast path)
  __shared__ __attribute__((aligned(16))) float s_c[kC * LD];    // Qt, or q on the exact path
  __shared__ __attribute__((aligned(16))) float s_g[kC * LD];    // g (log2)
  __shared__ float s_tot[4 * KP], s_gl[KP], s_ok[kC];

  const int n = blockIdx.x / p.H, h = blockIdx.x % p.H, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, g4 = lane >> 4, r = 16 * w + col, cg = 8 * g4;
  const size_t ch = ((size_t)b * p.H + h) * p.NC + n;
  auto tok = [&](int row) -> size_t { return ((size_t)b * p.T + n * kC + row) * p.H + h; };

  Rows<DT, KP> R;
  load_rows<DT, KP, true>(p, b, h, n, R, s_tot, s_gl);
  if (lane < 16) s_ok[r] = R.ok ? 1.f : 0.f;
  const bool fast = __syncthreads_and(tid >= KP || s_gl[tid] >= kFastLimit);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int at = r * LD + 32 * ks + cg + e;
      const float gv = R.g[ks][e];
      s_g[at] = gv;
      if (fast) {
        const float gam = exp2f(gv);
        s_a[at] = R.k[ks][e] * gam;
        s_b[at] = R.k[ks][e] * exp2f(-gv);
        s_c[at] = R.q[ks][e] * gam;
      } else {
        s_a[at] = R.k[ks][e];
        s_b[at] = 0.f;
        s_c[at] = R.q[ks][e];
      }
    }
  __syncthreads();

  const float* S0 = entry_state(p, b, h, n);
  const float* dS1 = p.w.dS1 + ch * (size_t)(KP * V);
  const float* Ug = p.w.U + ch * (size_t)(kC * V);
  const float* dP = p.w.dP + ch * (size_t)(kC * kC);
  const float* dPt = p.w.dPt + ch * (size_t)(kC * kC);
  const float* dG = p.w.dG + ch * (size_t)(kC * kC);
  const float* dGt = p.w.dGt + ch * (size_t)(kC * kC);

  for (int m = 0; m < 2; ++m) {
    const int ct = w + 4 * m;
    if (ct >= CT) continue;
    const int c = 16 * ct + col;                     // this lane's channel
    // ---- Y1 = dO S0^T, Y2 = dR S0^T, Z = U dS1^T (contraction over dv), rowsum(dS1 * S0)
    f32x4 y1[4], y2[4], z[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) { y1[I] = zero4(); y2[I] = zero4(); z[I] = zero4(); }
    float ss = 0.f;
#pragma unroll
    for (int vs = 0; vs < VS; ++vs) {
      const int v0 = 32 * vs + cg;
      float sb[8], db[8];
      if (v0 < V) {
        if (S0 != nullptr && c < p.K) gld8(S0 + (size_t)c * V + v0, sb);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) sb[e] = 0.f;
        }
        gld8(dS1 + (size_t)c * V + v0, db);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { sb[e] = 0.f; db[e] = 0.f; }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += sb[e] * db[e];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int row = 16 * I + col;
        float a1[8], a2[8], a3[8];
        if (s_ok[row] != 0.f && v0 < V) {
          E::ld8((const Tp*)p.dout, tok(row) * V + v0, a1);
          gld8(p.dv + tok(row) * V + v0, a2);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { a1[e] = 0.f; a2[e] = 0.f; }
        }
        if (v0 < V) gld8(Ug + row * V + v0, a3);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) a3[e] = 0.f;
        }
        y1[I] = mm3(a1, sb, y1[I]);
        y2[I] = mm3(a2, sb, y2[I]);
        z[I] = mm3(a3, db, z[I]);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);

    // ---- the decay-weighted C x C terms, as Gam_i (dP Ki)_i, Gam_i (dG Ki)_i, (dP^T Qt)_j / Gam_j
    //      and (dG^T Kt)_j / Gam_j
    f32x4 xq[4], xk1[4], xk2[4], xk3[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) { xq[I] = zero4(); xk1[I] = zero4(); xk2[I] = zero4(); xk3[I] = zero4(); }
    if (fast) {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int k0 = 32 * s + cg;
          float bv[8];
          if (s <= I / 2) {                          // columns j <= i
            float ap[8], ag[8];
            gld8(dP + (16 * I + col) * kC + k0, ap);
            gld8(dG + (16 * I + col) * kC + k0, ag);
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = s_b[(k0 + e) * LD + c];
            xq[I] = mm3(ap, bv, xq[I]);
            xk3[I] = mm3(ag, bv, xk3[I]);
          }
          if (32 * s + 31 >= 16 * I) {               // rows i >= j
            float ap[8], ag[8], bq[8];
            gld8(dPt + (16 * I + col) * kC + k0, ap);
            gld8(dGt + (16 * I + col) * kC + k0, ag);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              bq[e] = s_c[(k0 + e) * LD + c];
              bv[e] = s_a[(k0 + e) * LD + c];
            }
            xk1[I] = mm3(ap, bq, xk1[I]);
            xk2[I] = mm3(ag, bv, xk2[I]);
          }
        }
      }
    }

    // ---- per element: dq, dk and the per-row decay gradient
    const float gl = s_gl[c];
    float dl[4][4];
    float zk = 0.f;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * I + 4 * g4 + i;
        const float gv = s_g[row * LD + c];
        const bool ok = s_ok[row] != 0.f && c < p.K;
        float kr = 0.f, qr = 0.f;
        if (ok) {
          kr = E::ld((const Tp*)p.k, tok(row) * p.K + c);
          qr = E::ld((const Tp*)p.q, tok(row) * p.K + c);
        }
        float Xq, Xk1, Xk2, Xk3;
        if (fast) {
          const float gm = exp2f(gv), gi = exp2f(-gv);
          Xq = gm * xq[I][i];
          Xk3 = gm * xk3[I][i];
          Xk1 = gi * xk1[I][i];
          Xk2 = gi * xk2[I][i];
        } else {
          Xq = 0.f; Xk1 = 0.f; Xk2 = 0.f; Xk3 = 0.f;
          for (int j = 0; j < kC; ++j) {
            const float gj = s_g[j * LD + c];
            if (j <= row) {
              const float wgt = s_a[j * LD + c] * exp2f(gv - gj);
              Xq += dP[row * kC + j] * wgt;
              Xk3 += dG[row * kC + j] * wgt;
            }
            if (j >= row) {
              const float d = exp2f(gj - gv);
              Xk1 += dPt[row * kC + j] * s_c[j * LD + c] * d;
              Xk2 += dGt[row * kC + j] * s_a[j * LD + c] * d;
            }
          }
        }
        const float gm = exp2f(gv), ekh = exp2f(gl - gv);
        const float a = Xk3 - gm * y2[I][i];           // Gam dKt
        const float bb = Xk1 + Xk2;                    // dKi / Gam
        const float dqv = gm * y1[I][i] + Xq;
        const float dkv = a + bb + z[I][i] * ekh;
        const float khv = kr * ekh;
        dl[I][i] = ok ? kr * a - kr * bb + qr * dqv - z[I][i] * khv : 0.f;
        zk += ok ? z[I][i] * khv : 0.f;
        if (n * kC + row < p.T && c < p.K) {
          p.dq[tok(row) * p.K + c] = ok ? dqv : 0.f;
          p.dk[tok(row) * p.K + c] = ok ? dkv : 0.f;
        }
      }
    // ---- dlog_alpha: reverse sums over the rows, plus the Gam_last term
    zk += __shfl_xor(zk, 16, 64);
    zk += __shfl_xor(zk, 32, 64);
    const float dlast = zk + exp2f(gl) * ss;
    float tile[4], after[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) tile[I] = (dl[I][0] + dl[I][1]) + (dl[I][2] + dl[I][3]);
    // sums of the lanes holding later rows of the same tile (same column, larger l/16)
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      float later = 0.f, total = 0.f;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float x = __shfl(tile[I], col + 16 * q4, 64);
        total += x;
        later += q4 > g4 ? x : 0.f;
      }
      after[I] = later;
      tile[I] = total;
    }
    float carry = dlast;
#pragma unroll
    for (int I = 3; I >= 0; --I) {
      float run = carry + after[I];
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const int row = 16 * I + 4 * g4 + i;
        run += dl[I][i];
        if (n * kC + row < p.T && c < p.K) p.dla[tok(row) * p.K + c] = s_ok[row] != 0.f ? run : 0.f;
      }
      carry += tile[I];
    }
  }
}

// ---------------------------------------------------------------- host side
struct Layout {
  size_t fwd, o, fin, ck, kh, wt, qt, pt, gam, G, M, dS1, dU, U, dP, dPt, dG, dGt, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout layout(int B, int T, int H, int dk, int dv, int dtype) {
  Layout L{};
  if (T <= 0 || B == 0 || H == 0) return L;
  const int KP = kpad(dk), NC = (T + kC - 1) / kC, NCf = T / kC;
  const size_t nch = (size_t)B * H * NC, parts = dtype == 1 ? 2 : 1, es = dtype == 1 ? 4 : 2;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align256(bytes); return at; };
  L.fwd = take(prefill_workspace_bytes(B, T, H, dk, dv, kC, dtype, false));
  L.o = take((size_t)B * T * H * dv * es);
  L.fin = take((size_t)B * H * dk * dv * 4);
  L.ck = take((size_t)B * NCf * H * dk * dv * 4);
  L.kh = take(nch * kC * KP * 2 * parts);
  L.wt = take(nch * kC * KP * 2 * parts);
  L.qt = take(nch * kC * KP * 2 * parts);
  L.pt = take(nch * kC * kC * 2 * 2);
  L.gam = take(nch * KP * 4);
  L.G = take(nch * kC * kC * 4);
  L.M = take(nch * kC * kC * 4);
  L.dS1 = take(nch * KP * dv * 4);
  L.dU = take(nch * kC * dv * 4);
  L.U = take(nch * kC * dv * 4);
  L.dP = take(nch * kC * kC * 4);
  L.dPt = take(nch * kC * kC * 4);
  L.dG = take(nch * kC * kC * 4);
  L.dGt = take(nch * kC * kC * 4);
  L.total = off;
  return L;
}

template <int DT, int KP, int V>
hipError_t launch_t(const Params& p, hipStream_t st) {
  const dim3 cgrid(p.NC * p.H, p.B);
  if (p.NC > 0) {
    hipLaunchKernelGGL((bwd_prep_kernel<DT, KP>), cgrid, dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_scan_kernel<DT, KP, V>), dim3(p.B * p.H * (V / 16)), dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.NC == 0) return e;
  hipLaunchKernelGGL((bwd_cc_kernel<DT, KP, V>), cgrid, dim3(kThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_ck_kernel<DT, KP, V>), cgrid, dim3(kThreads), 0, st, p);
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

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype) {
  return layout(B, T, H, dk, dv, dtype).total;
}

hipError_t launch_backward(const BackwardArgs& a) {
  const Layout L = layout(a.B, a.T, a.H, a.dk_, a.dv_, a.dtype);
  unsigned char* ws = (unsigned char*)a.workspace;
  const int NC = a.T > 0 ? (a.T + kC - 1) / kC : 0, NCf = a.T / kC;
  if (a.T > 0) {
    // the forward pass again, keeping the state at every chunk end
    PrefillArgs f{};
    f.q = a.q; f.k = a.k; f.v = a.v; f.log_alpha = a.log_alpha; f.beta = a.beta; f.mask = a.mask;
    f.init_state = a.init_state;
    f.o = ws + L.o;
    f.final_state = (float*)(ws + L.fin);
    f.B = a.B; f.T = a.T; f.H = a.H; f.dk = a.dk_; f.dv = a.dv_; f.chunk = kC; f.dtype = a.dtype;
    f.workspace = ws + L.fwd;
    f.workspace_bytes = L.o - L.fwd;
    f.stream = a.stream;
    f.chunk_states = NCf > 0 ? (float*)(ws + L.ck) : nullptr;
    f.num_states = a.B * NCf;
    f.state_interval = kC;
    const hipError_t e = launch_prefill(f);
    if (e != hipSuccess) return e;
  }
  Params p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
  p.la = a.log_alpha; p.beta = a.beta; p.init = a.init_state; p.dfinal = a.dfinal; p.mask = a.mask;
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dla = a.dla; p.dbeta = a.dbeta; p.dinit = a.dinit;
  if (a.T > 0) {
    p.w.kh = (uint16_t*)(ws + L.kh); p.w.wt = (uint16_t*)(ws + L.wt); p.w.qt = (uint16_t*)(ws + L.qt);
    p.w.pt = (uint16_t*)(ws + L.pt);
    p.w.gam = (float*)(ws + L.gam); p.w.G = (float*)(ws + L.G); p.w.M = (float*)(ws + L.M);
    p.w.dS1 = (float*)(ws + L.dS1); p.w.dU = (float*)(ws + L.dU); p.w.U = (float*)(ws + L.U);
    p.w.dP = (float*)(ws + L.dP); p.w.dPt = (float*)(ws + L.dPt);
    p.w.dG = (float*)(ws + L.dG); p.w.dGt = (float*)(ws + L.dGt);
    p.w.ck = (const float*)(ws + L.ck);
  }
  p.B = a.B; p.T = a.T; p.H = a.H; p.K = a.dk_; p.V = a.dv_; p.NC = NC; p.NCf = NCf;
  hipStream_t st = (hipStream_t)a.stream;
  return a.dtype == 0 ? launch_dt<0>(p, st) : launch_dt<1>(p, st);
}

}  // namespace kda
