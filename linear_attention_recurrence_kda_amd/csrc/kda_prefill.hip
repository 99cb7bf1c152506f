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
//   Wn = -T' Kt,   Qh = Qt - (P T') Kt
//   U  = T' V + Wn S0                          (per-token corrections)
//   O  = Qh S0 + P (T' V)
//   S1 = Diag(Gam_last) S0 + Kh^T U
// Only the last three lines depend on the state, so the work splits into:
//   prep_kernel: one workgroup per (b, h, chunk), fully parallel; writes Wn, Qh,
//     Kh^T, T', P and Gam_last to a workspace in MFMA operand order;
//   scan_kernel: one workgroup per (b, h, dv-tile), a loop over the chunks in
//     order with the fp32 state tile held in registers across chunks.
// The factorisation Kt Ki^T (decay relative to the chunk start) is used when
// every channel's decay over the chunk stays above 2^-100 (then no factor
// over- or under-flows); otherwise that chunk computes A and P entry by entry
// with exp2(G_t - G_j).  Entries above the diagonal come from a select, never
// from a product, so nothing from a later position can reach an earlier one.
//
// Precision: bf16 MFMA operands that are not exactly bf16 are split into a
// bf16 high part and a bf16 residual where that matters (A, P, T', S, U and
// T'V); with fp32 inputs every operand is split.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kPrepThreads = 256;
constexpr int kScanThreads = 256;
constexpr int kVT = 16;                 // dv columns per scan workgroup
constexpr float kFastLimit = -100.0f;   // log2 decay over one chunk for the factorised path

// ---------------------------------------------------------------- workspace layout
// Per (b, h, chunk), in 2-byte units.  Every matrix is stored in A-operand order
// of v_mfma_f32_16x16x32_bf16: fragment (row tile rt, k step ks) is 64 lanes x
// 8 bf16, lane l holding M[16 rt + l%16][32 ks + 8 (l/16) .. +7].
template <int K, int C, bool SPLIT>
struct WsLayout {
  static constexpr size_t kCK = (size_t)C * K;
  static constexpr size_t kCC = (size_t)C * C;
  static constexpr size_t kSplitCK = SPLIT ? 2 * kCK : kCK;
  static constexpr size_t off_wn = 0;                    // -T' Kt           [C x K] (hi, lo)
  static constexpr size_t off_qh = off_wn + kSplitCK;    // Qt - P T' Kt     [C x K]
  static constexpr size_t off_kh = off_qh + kSplitCK;    // Kh^T             [K x C]
  static constexpr size_t off_tp = off_kh + kSplitCK;    // T' hi, lo        [C x C]
  static constexpr size_t off_p = off_tp + 2 * kCC;      // P hi, lo         [C x C]
  static constexpr size_t off_gam = off_p + 2 * kCC;     // Gam_last, K fp32
  static constexpr size_t kElems = off_gam + 2 * (size_t)K;
};

__device__ __forceinline__ size_t frag_off(int rt, int ks, int lane, int kk) {
  return ((size_t)(rt * (kk / 32) + ks) * 64 + lane) * 8;
}

struct PrepParams {
  const void *q, *k;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  uint16_t* ws;
  int B, T, H, dk, chunk, NC, l2norm;
};

struct ScanParams {
  const void* v;
  const uint8_t* mask;
  const float* init_state;
  float* final_state;
  void* o;
  const uint16_t* ws;
  int B, T, H, dk, dv, chunk, NC, NT, nbh;
};

__device__ __forceinline__ bool row_valid(const uint8_t* mask, int b, int T, int chunk, int r, int t) {
  return r < chunk && t < T && (mask == nullptr || mask[(size_t)b * T + t] != 0);
}

__device__ __forceinline__ void store_frag(uint16_t* dst, const bf16x8& v) {
  *reinterpret_cast<bf16x8*>(dst) = v;
}
__device__ __forceinline__ bf16x8 load_frag(const uint16_t* src) {
  return *reinterpret_cast<const bf16x8*>(src);
}

// ================================================================ prep kernel
template <int DT, int K, int C>
__global__ void __launch_bounds__(kPrepThreads)
prep_kernel(PrepParams p) {
  using E = Elem<DT>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, C, SPLIT>;
  constexpr int RT = C / 16;          // row tiles of the chunk
  constexpr int CS = C / 32;          // k steps over chunk rows
  constexpr int KS = K / 32;          // k steps over key channels
  constexpr int KP = K + 4;           // fp32 row stride
  constexpr int KB = K + 8;           // bf16 row stride (16-byte aligned rows)

  __shared__ float s_G[C * KP];                        // G (log2), then Gam in the fast path
  __shared__ __attribute__((aligned(16))) __bf16 s_kt[2][C * KB];   // Kt hi, lo
  __shared__ __attribute__((aligned(16))) __bf16 s_ki[2][C * KB];   // Ki hi, lo
  __shared__ float s_A[C * C];                         // A, later M = P T'
  __shared__ float s_T[C * C];
  __shared__ float s_P[C * C];
  __shared__ float s_X[(RT > 1 ? RT - 1 : 1) * 16 * 17];
  __shared__ float s_stage[4][16 * 17];
  __shared__ float s_beta[C], s_qs[C], s_ks[C], s_gc[K];

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = n * p.chunk;
  const int dk = p.dk;
  const typename E::T* qg = (const typename E::T*)p.q;
  const typename E::T* kg = (const typename E::T*)p.k;
  uint16_t* wsb = p.ws + ((size_t)(b * p.H + h) * p.NC + n) * L::kElems;
  auto grow = [&](int t) -> size_t { return ((size_t)b * p.T + t) * p.H + h; };

  // ---- load log_alpha (log2 units) and beta, masked rows as no-ops
  for (int idx = tid; idx < C * (K / 4); idx += kPrepThreads) {
    const int r = idx / (K / 4), c = (idx % (K / 4)) * 4, t = t0 + r;
    float4 la = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < dk && row_valid(p.mask, b, p.T, p.chunk, r, t))
      la = *reinterpret_cast<const float4*>(p.log_alpha + grow(t) * dk + c);
    float* g = s_G + r * KP + c;
    g[0] = la.x * kLog2e; g[1] = la.y * kLog2e; g[2] = la.z * kLog2e; g[3] = la.w * kLog2e;
  }
  if (tid < C) {
    const int t = t0 + tid;
    s_beta[tid] = row_valid(p.mask, b, p.T, p.chunk, tid, t) ? p.beta[grow(t)] : 0.f;
  }
  // ---- row scales for the optional L2 normalisation of q and k
  for (int r = wave; r < C; r += 4) {
    const int t = t0 + r;
    float sq = 0.f, sk = 0.f;
    if (p.l2norm && row_valid(p.mask, b, p.T, p.chunk, r, t)) {
      for (int c = lane; c < dk; c += 64) {
        const float a = E::ld(qg, grow(t) * dk + c), kk = E::ld(kg, grow(t) * dk + c);
        sq += a * a; sk += kk * kk;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) { sq += __shfl_xor(sq, off, 64); sk += __shfl_xor(sk, off, 64); }
    }
    if (lane == 0) {
      s_qs[r] = p.l2norm ? rsqrtf(sq + 1e-6f) : 1.0f;
      s_ks[r] = p.l2norm ? rsqrtf(sk + 1e-6f) : 1.0f;
    }
  }
  __syncthreads();

  // ---- inclusive cumulative sum over the chunk, per channel
  if (tid < K) {
    float acc = 0.f;
    for (int r = 0; r < C; ++r) { acc += s_G[r * KP + tid]; s_G[r * KP + tid] = acc; }
    s_gc[tid] = acc;
  }
  const int fast = __syncthreads_and(tid >= K || s_gc[tid] >= kFastLimit);

  // ---- elementwise decay factors; item = (channel c, 8 consecutive rows)
  for (int idx = tid; idx < K * (C / 8); idx += kPrepThreads) {
    const int c = idx % K, oct = idx / K;
    const float gc = s_gc[c];
    float kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = oct * 8 + e, t = t0 + r;
      float kv = 0.f;
      if (c < dk && row_valid(p.mask, b, p.T, p.chunk, r, t)) kv = E::ld(kg, grow(t) * dk + c) * s_ks[r];
      const float g = s_G[r * KP + c];
      const float gam = exp2f(g);
      const float kt = kv * gam;
      const __bf16 kth = (__bf16)kt;
      s_kt[0][r * KB + c] = kth;
      s_kt[1][r * KB + c] = (__bf16)(kt - (float)kth);
      const float ki = fast ? kv * exp2f(-g) : 0.f;
      const __bf16 kih = (__bf16)ki;
      s_ki[0][r * KB + c] = kih;
      s_ki[1][r * KB + c] = (__bf16)(ki - (float)kih);
      kh[e] = kv * exp2f(gc - g);
      if (fast) s_G[r * KP + c] = gam;       // slow path keeps G for the exact pairwise decays
    }
    // Kh^T fragment: row c, contraction over rows 8*oct .. +7
    const int rt = c / 16, ks = oct / 4, ln = (c % 16) + 16 * (oct % 4);
    bf16x8 hi, lo;
    split8(kh, hi, lo);
    store_frag(wsb + L::off_kh + frag_off(rt, ks, ln, C), hi);
    if (SPLIT) store_frag(wsb + L::off_kh + L::kCK + frag_off(rt, ks, ln, C), lo);
  }
  if (tid < K) reinterpret_cast<float*>(wsb + L::off_gam)[tid] = exp2f(s_gc[tid]);
  __syncthreads();

  // Qt = q * qscale * Gam for row r, channels c..c+7
  auto qt8 = [&](int r, int c, float* out) {
    const int t = t0 + r;
    if (c < dk && row_valid(p.mask, b, p.T, p.chunk, r, t)) {
      E::ld8(qg, grow(t) * dk + c, out);
      const float s = s_qs[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = s_G[r * KP + c + e];
        out[e] *= s * (fast ? g : exp2f(g));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
    }
  };

  // ---- A and P
  if (fast) {
    for (int I = wave; I < RT; I += 4) {
      bf16x8 kth[KS], ktl[KS], qth[KS], qtl[KS];
      const int r = 16 * I + (lane % 16);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 32 * ks + 8 * (lane / 16);
        kth[ks] = *reinterpret_cast<const bf16x8*>(&s_kt[0][r * KB + c]);
        ktl[ks] = *reinterpret_cast<const bf16x8*>(&s_kt[1][r * KB + c]);
        float qv[8];
        qt8(r, c, qv);
        split8(qv, qth[ks], qtl[ks]);
      }
      for (int J = 0; J < RT; ++J) {
        f32x4 accA = zero4(), accP = zero4();
        if (J <= I) {
          const int j = 16 * J + (lane % 16);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int c = 32 * ks + 8 * (lane / 16);
            const bf16x8 kih = *reinterpret_cast<const bf16x8*>(&s_ki[0][j * KB + c]);
            const bf16x8 kil = *reinterpret_cast<const bf16x8*>(&s_ki[1][j * KB + c]);
            accA = mfma16(kth[ks], kih, accA);
            accA = mfma16(kth[ks], kil, accA);
            accA = mfma16(ktl[ks], kih, accA);
            accP = mfma16(qth[ks], kih, accP);
            accP = mfma16(qth[ks], kil, accP);
            accP = mfma16(qtl[ks], kih, accP);
          }
        }
        const int jj = 16 * J + (lane % 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * I + 4 * (lane / 16) + i;
          s_A[rr * C + jj] = (jj < rr) ? s_beta[rr] * accA[i] : 0.f;
          s_P[rr * C + jj] = (jj <= rr) ? accP[i] : 0.f;
        }
      }
    }
  } else {
    // exact pairwise decays (chunks whose total decay in some channel is below 2^-100)
    for (int idx = tid; idx < C * C; idx += kPrepThreads) {
      const int rr = idx / C, jj = idx % C;
      float sa = 0.f, sp = 0.f;
      const int tr = t0 + rr, tj = t0 + jj;
      if (jj <= rr && row_valid(p.mask, b, p.T, p.chunk, rr, tr) &&
          row_valid(p.mask, b, p.T, p.chunk, jj, tj)) {
        for (int c = 0; c < dk; ++c) {
          const float d = exp2f(s_G[rr * KP + c] - s_G[jj * KP + c]);
          const float kj = E::ld(kg, grow(tj) * dk + c) * s_ks[jj];
          sa += E::ld(kg, grow(tr) * dk + c) * s_ks[rr] * kj * d;
          sp += E::ld(qg, grow(tr) * dk + c) * s_qs[rr] * kj * d;
        }
      }
      s_A[idx] = (jj < rr) ? s_beta[rr] * sa : 0.f;
      s_P[idx] = (jj <= rr) ? sp : 0.f;
    }
  }
  __syncthreads();

  // ---- T = (I + A)^-1, blocked: diagonal 16x16 blocks by forward substitution
  if (tid < RT * 16) {
    const int I = tid / 16, cc = tid % 16;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float v = (rr == cc) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < rr; ++jj) v -= s_A[(16 * I + rr) * C + 16 * I + jj] * x[jj];
      x[rr] = v;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s_T[(16 * I + rr) * C + 16 * I + cc] = x[rr];
  }
  for (int idx = tid; idx < C * C; idx += kPrepThreads) {
    const int rr = idx / C, jj = idx % C;
    if (jj / 16 != rr / 16) s_T[idx] = 0.f;
  }
  __syncthreads();
  // off-diagonal blocks by distance d: T_IJ = -T_II * sum_{L=J}^{I-1} A_IL T_LJ
  for (int d = 1; d < RT; ++d) {
    const int nblk = RT - d;
    for (int e = tid; e < nblk * 256; e += kPrepThreads) {
      const int J = e / 256, I = J + d, rr = (e % 256) / 16, cc = e % 16;
      float x = 0.f;
      for (int Lb = J; Lb < I; ++Lb)
#pragma unroll
        for (int m = 0; m < 16; ++m) x += s_A[(16 * I + rr) * C + 16 * Lb + m] * s_T[(16 * Lb + m) * C + 16 * J + cc];
      s_X[J * 272 + rr * 17 + cc] = x;
    }
    __syncthreads();
    for (int e = tid; e < nblk * 256; e += kPrepThreads) {
      const int J = e / 256, I = J + d, rr = (e % 256) / 16, cc = e % 16;
      float x = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) x += s_T[(16 * I + rr) * C + 16 * I + m] * s_X[J * 272 + m * 17 + cc];
      s_T[(16 * I + rr) * C + 16 * J + cc] = -x;
    }
    __syncthreads();
  }

  // ---- T' = T Diag(beta) and P to the workspace (hi, lo), A-operand order
  for (int idx = tid; idx < RT * CS * 64; idx += kPrepThreads) {
    const int ln = idx % 64, ks = (idx / 64) % CS, rt = idx / (64 * CS);
    const int r = 16 * rt + (ln % 16), j0 = 32 * ks + 8 * (ln / 16);
    float tv[8], pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tv[e] = s_T[r * C + j0 + e] * s_beta[j0 + e];
      pv[e] = s_P[r * C + j0 + e];
    }
    bf16x8 hi, lo;
    split8(tv, hi, lo);
    store_frag(wsb + L::off_tp + frag_off(rt, ks, ln, C), hi);
    store_frag(wsb + L::off_tp + L::kCC + frag_off(rt, ks, ln, C), lo);
    split8(pv, hi, lo);
    store_frag(wsb + L::off_p + frag_off(rt, ks, ln, C), hi);
    store_frag(wsb + L::off_p + L::kCC + frag_off(rt, ks, ln, C), lo);
  }

  // ---- M = P T' (lower triangular), into s_A
  for (int I = wave; I < RT; I += 4) {
    const int r = 16 * I + (lane % 16);
    bf16x8 ph[CS], pl[CS];
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      float pv[8];
      const int j0 = 32 * ks + 8 * (lane / 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = s_P[r * C + j0 + e];
      split8(pv, ph[ks], pl[ks]);
    }
    for (int N = 0; N < RT; ++N) {
      f32x4 acc = zero4();
      if (N <= I) {
        const int jn = 16 * N + (lane % 16);
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          float tv[8];
          const int m0 = 32 * ks + 8 * (lane / 16);
#pragma unroll
          for (int e = 0; e < 8; ++e) tv[e] = s_T[(m0 + e) * C + jn] * s_beta[jn];
          bf16x8 th, tl;
          split8(tv, th, tl);
          acc = mfma16(ph[ks], th, acc);
          if (SPLIT) { acc = mfma16(ph[ks], tl, acc); acc = mfma16(pl[ks], th, acc); }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s_A[(16 * I + 4 * (lane / 16) + i) * C + 16 * N + (lane % 16)] = acc[i];
    }
  }
  __syncthreads();

  // ---- Wn = -T' Kt and Qh = Qt - M Kt; wave w owns channel tiles N = w, w+4, ...
  float* stage = s_stage[wave];
  for (int N = wave; N < K / 16; N += 4) {
    bf16x8 kth[CS], ktl[CS];
    const int cn = 16 * N + (lane % 16);
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + 8 * (lane / 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kth[ks][e] = s_kt[0][(j0 + e) * KB + cn];
        ktl[ks][e] = s_kt[1][(j0 + e) * KB + cn];
      }
    }
    for (int I = 0; I < RT; ++I) {
      f32x4 accW = zero4(), accQ = zero4();
      const int r = 16 * I + (lane % 16);
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;          // T' and M are lower triangular
        const int j0 = 32 * ks + 8 * (lane / 16);
        float tv[8], mv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tv[e] = -s_T[r * C + j0 + e] * s_beta[j0 + e];
          mv[e] = -s_A[r * C + j0 + e];
        }
        bf16x8 th, tl, mh, ml;
        split8(tv, th, tl);
        split8(mv, mh, ml);
        accW = mfma16(th, kth[ks], accW);
        accQ = mfma16(mh, kth[ks], accQ);
        if (SPLIT) {
          accW = mfma16(th, ktl[ks], accW); accW = mfma16(tl, kth[ks], accW);
          accQ = mfma16(mh, ktl[ks], accQ); accQ = mfma16(ml, kth[ks], accQ);
        }
      }
      // D layout -> rows of 8 channels via a per-wave staging tile, then A-operand order
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const f32x4& acc = pass == 0 ? accW : accQ;
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(4 * (lane / 16) + i) * 17 + (lane % 16)] = acc[i];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): staging writes landed
        if (lane < 32) {
          const int rr = lane % 16, half = lane / 16;
          float vals[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vals[e] = stage[rr * 17 + 8 * half + e];
          if (pass == 1) {
            float qv[8];
            qt8(16 * I + rr, 16 * N + 8 * half, qv);
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] += qv[e];
          }
          bf16x8 hi, lo;
          split8(vals, hi, lo);
          const int ln = rr + 16 * (2 * (N % 2) + half);
          const size_t off = (pass == 0 ? L::off_wn : L::off_qh) + frag_off(I, N / 2, ln, K);
          store_frag(wsb + off, hi);
          if (SPLIT) store_frag(wsb + off + L::kCK, lo);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0xc07f);
      }
    }
  }
}

// ================================================================ scan kernel
template <int DT, int K, int C>
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(ScanParams p) {
  using E = Elem<DT>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, C, SPLIT>;
  constexpr int RT = C / 16;
  constexpr int CS = C / 32;
  constexpr int KS = K / 32;
  constexpr int SRT = K / 16;                       // state row tiles
  constexpr int SPW = (SRT + 3) / 4;                // state row tiles per wave
  constexpr int UPW = (RT + 3) / 4;                 // U/O row tiles per wave
  constexpr int KB = K + 8, CB = C + 8;

  __shared__ __attribute__((aligned(16))) __bf16 s_S[2][kVT * KB];    // state, B-operand rows = dv column
  __shared__ __attribute__((aligned(16))) __bf16 s_U[2][kVT * CB];    // U
  __shared__ __attribute__((aligned(16))) __bf16 s_Ut[2][kVT * CB];   // T'V
  __shared__ __attribute__((aligned(16))) __bf16 s_V[2][kVT * CB];    // V tile, transposed

  // XCD-aware mapping: all dv tiles of one head share blockIdx.x % 8 (one L2)
  const int L_id = blockIdx.x;
  const int xcd = L_id % 8, slot = L_id / 8;
  const int bh = (slot / p.NT) * 8 + xcd, tile = slot % p.NT;
  if (bh >= p.nbh) return;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = tile * kVT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dk = p.dk, dv = p.dv;
  const typename E::T* vg = (const typename E::T*)p.v;
  typename E::T* og = (typename E::T*)p.o;
  const uint16_t* wsh = p.ws + (size_t)bh * p.NC * L::kElems;

  // state tiles in registers: wave w owns state row tiles w, w+4, ...
  f32x4 S[SPW];
#pragma unroll
  for (int m = 0; m < SPW; ++m) {
    const int M = wave + 4 * m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * M + 4 * (lane / 16) + i, col = v0 + (lane % 16);
      S[m][i] = (M < SRT && row < dk && p.init_state != nullptr)
                    ? p.init_state[((size_t)bh * dk + row) * dv + col] : 0.f;
    }
  }
  auto publish_state = [&]() {
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
      if (M < SRT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * M + 4 * (lane / 16) + i;
          const __bf16 hi = (__bf16)S[m][i];
          s_S[0][(lane % 16) * KB + row] = hi;
          s_S[1][(lane % 16) * KB + row] = (__bf16)(S[m][i] - (float)hi);
        }
      }
    }
  };
  publish_state();

  for (int n = 0; n < p.NC; ++n) {
    const uint16_t* wsb = wsh + (size_t)n * L::kElems;
    const int t0 = n * p.chunk;
    // ---- V tile -> LDS (transposed), masked rows as zeros
    for (int idx = tid; idx < C * kVT; idx += kScanThreads) {
      const int r = idx / kVT, cidx = idx % kVT, t = t0 + r;
      float x = 0.f;
      if (row_valid(p.mask, b, p.T, p.chunk, r, t)) x = E::ld(vg, (((size_t)b * p.T + t) * p.H + h) * dv + v0 + cidx);
      const __bf16 hi = (__bf16)x;
      s_V[0][cidx * CB + r] = hi;
      s_V[1][cidx * CB + r] = (__bf16)(x - (float)hi);
    }
    __syncthreads();                                                   // (a) V and S visible

    // ---- Ut = T' V for this wave's rows; then U = Ut + Wn S and O = Qh S + P Ut
    bf16x8 sh[KS], sl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = 32 * ks + 8 * (lane / 16);
      sh[ks] = *reinterpret_cast<const bf16x8*>(&s_S[0][(lane % 16) * KB + k0]);
      sl[ks] = *reinterpret_cast<const bf16x8*>(&s_S[1][(lane % 16) * KB + k0]);
    }
    f32x4 Uacc[UPW];
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int I = wave + 4 * u;
      f32x4 ut = zero4();
      if (I < RT) {
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          if (32 * ks > 16 * I + 15) continue;
          const int j0 = 32 * ks + 8 * (lane / 16);
          const bf16x8 th = load_frag(wsb + L::off_tp + frag_off(I, ks, lane, C));
          const bf16x8 tl = load_frag(wsb + L::off_tp + L::kCC + frag_off(I, ks, lane, C));
          const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&s_V[0][(lane % 16) * CB + j0]);
          ut = mfma16(th, vh, ut);
          ut = mfma16(tl, vh, ut);
          if (SPLIT) {
            const bf16x8 vl = *reinterpret_cast<const bf16x8*>(&s_V[1][(lane % 16) * CB + j0]);
            ut = mfma16(th, vl, ut);
          }
        }
        // Ut to LDS as a B operand (rows = dv column, contraction over chunk rows)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * I + 4 * (lane / 16) + i;
          const __bf16 hi = (__bf16)ut[i];
          s_Ut[0][(lane % 16) * CB + rr] = hi;
          s_Ut[1][(lane % 16) * CB + rr] = (__bf16)(ut[i] - (float)hi);
        }
        f32x4 acc = ut;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 wh = load_frag(wsb + L::off_wn + frag_off(I, ks, lane, K));
          acc = mfma16(wh, sh[ks], acc);
          acc = mfma16(wh, sl[ks], acc);
          if (SPLIT) acc = mfma16(load_frag(wsb + L::off_wn + L::kCK + frag_off(I, ks, lane, K)), sh[ks], acc);
        }
        Uacc[u] = acc;
      }
    }
    __syncthreads();                                                   // (b) Ut visible

#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const int I = wave + 4 * u;
      if (I >= RT) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qh = load_frag(wsb + L::off_qh + frag_off(I, ks, lane, K));
        acc = mfma16(qh, sh[ks], acc);
        acc = mfma16(qh, sl[ks], acc);
        if (SPLIT) acc = mfma16(load_frag(wsb + L::off_qh + L::kCK + frag_off(I, ks, lane, K)), sh[ks], acc);
      }
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;
        const int j0 = 32 * ks + 8 * (lane / 16);
        const bf16x8 ph = load_frag(wsb + L::off_p + frag_off(I, ks, lane, C));
        const bf16x8 pl = load_frag(wsb + L::off_p + L::kCC + frag_off(I, ks, lane, C));
        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&s_Ut[0][(lane % 16) * CB + j0]);
        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&s_Ut[1][(lane % 16) * CB + j0]);
        acc = mfma16(ph, uh, acc);
        acc = mfma16(ph, ul, acc);
        acc = mfma16(pl, uh, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i, t = t0 + rr;
        if (rr < p.chunk && t < p.T) E::st(og, (((size_t)b * p.T + t) * p.H + h) * dv + v0 + (lane % 16), acc[i]);
      }
      // U to LDS as a B operand
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i;
        const __bf16 hi = (__bf16)Uacc[u][i];
        s_U[0][(lane % 16) * CB + rr] = hi;
        s_U[1][(lane % 16) * CB + rr] = (__bf16)(Uacc[u][i] - (float)hi);
      }
    }
    __syncthreads();                                                   // (c) U visible, S reads done

    // ---- S = Diag(Gam_last) S + Kh^T U
    const float* gam = reinterpret_cast<const float*>(wsb + L::off_gam);
    bf16x8 uh[CS], ul[CS];
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + 8 * (lane / 16);
      uh[ks] = *reinterpret_cast<const bf16x8*>(&s_U[0][(lane % 16) * CB + j0]);
      ul[ks] = *reinterpret_cast<const bf16x8*>(&s_U[1][(lane % 16) * CB + j0]);
    }
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
      if (M >= SRT) continue;
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = gam[16 * M + 4 * (lane / 16) + i] * S[m][i];
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        const bf16x8 kh = load_frag(wsb + L::off_kh + frag_off(M, ks, lane, C));
        acc = mfma16(kh, uh[ks], acc);
        acc = mfma16(kh, ul[ks], acc);
        if (SPLIT) acc = mfma16(load_frag(wsb + L::off_kh + L::kCK + frag_off(M, ks, lane, C)), uh[ks], acc);
      }
      S[m] = acc;
    }
    publish_state();
  }

  // ---- final state
#pragma unroll
  for (int m = 0; m < SPW; ++m) {
    const int M = wave + 4 * m;
    if (M >= SRT) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * M + 4 * (lane / 16) + i;
      if (row < dk) p.final_state[((size_t)bh * dk + row) * dv + v0 + (lane % 16)] = S[m][i];
    }
  }
}

// ================================================================ host side
static int tile_chunk(int chunk) { return chunk <= 32 ? 32 : 64; }
static int pad_k(int dk) { return dk < 32 ? 32 : dk; }

bool prefill_supported(int dk, int dv, int chunk) {
  (void)dk; (void)dv;
  return chunk == 16 || chunk == 32 || chunk == 64;
}

template <int K, int C>
static size_t ws_elems(int dtype) {
  return dtype == 1 ? WsLayout<K, C, true>::kElems : WsLayout<K, C, false>::kElems;
}

static size_t chunk_ws_elems(int K, int C, int dtype) {
#define KDA_WS(KK, CC) if (K == KK && C == CC) return ws_elems<KK, CC>(dtype);
  KDA_WS(32, 32) KDA_WS(32, 64) KDA_WS(64, 32) KDA_WS(64, 64) KDA_WS(128, 32) KDA_WS(128, 64)
#undef KDA_WS
  return 0;
}

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  (void)dv;
  if (T == 0 || B == 0 || H == 0) return 0;
  const int NC = (T + chunk - 1) / chunk;
  return (size_t)B * H * NC * chunk_ws_elems(pad_k(dk), tile_chunk(chunk), dtype) * 2;
}

template <int DT, int K, int C>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const int NC = (a.T + a.chunk - 1) / a.chunk;
  const int NT = a.dv / kVT;
  const int nbh = a.B * a.H;
  if (NC > 0) {
    PrepParams pp{a.q, a.k, a.log_alpha, a.beta, a.mask, (uint16_t*)a.workspace,
                  a.B, a.T, a.H, a.dk, a.chunk, NC, a.l2norm};
    hipLaunchKernelGGL((prep_kernel<DT, K, C>), dim3(NC, a.H, a.B), dim3(kPrepThreads), 0, st, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanParams sp{a.v, a.mask, a.init_state, a.final_state, a.o, (const uint16_t*)a.workspace,
                a.B, a.T, a.H, a.dk, a.dv, a.chunk, NC, NT, nbh};
  const int groups = (nbh + 7) / 8;
  hipLaunchKernelGGL((scan_kernel<DT, K, C>), dim3(groups * 8 * NT), dim3(kScanThreads), 0, st, sp);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_prefill_dt(const PrefillArgs& a) {
  const int K = pad_k(a.dk), C = tile_chunk(a.chunk);
#define KDA_PF(KK, CC) if (K == KK && C == CC) return launch_prefill_t<DT, KK, CC>(a);
  KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(128, 32) KDA_PF(128, 64)
#undef KDA_PF
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  return a.dtype == 0 ? launch_prefill_dt<0>(a) : launch_prefill_dt<1>(a);
}

}  // namespace kda
