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
// every channel's decay over the chunk stays above 2^-120 (then no factor
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
constexpr float kFastLimit = -120.0f;   // log2 decay over one chunk for the factorised path

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
// 8 consecutive floats from 16-byte aligned LDS
__device__ __forceinline__ void ld8f(const float* src, float* out) {
  const float4 a = reinterpret_cast<const float4*>(src)[0];
  const float4 b = reinterpret_cast<const float4*>(src)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ================================================================ prep kernel
// One workgroup per (chunk, head, batch row).  Every global load of the chunk is
// issued first, unconditionally, from in-bounds rows; row validity (mask, ragged
// tail) is applied afterwards by select, so no load waits on another.
template <int DT, int K, int C>
__global__ void __launch_bounds__(kPrepThreads)
prep_kernel(PrepParams p) {
  using E = Elem<DT>;
  using Raw = typename E::T;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, C, SPLIT>;
  constexpr int RT = C / 16;          // row tiles of the chunk
  constexpr int CS = C / 32;          // k steps over chunk rows
  constexpr int KS = K / 32;          // k steps over key channels
  constexpr int KP = K + 4;           // fp32 row stride
  constexpr int KB = K + 8;           // bf16 row stride (16-byte aligned rows)
  constexpr int CP = C + 4;           // fp32 row stride of the C x C matrices (16 rows -> 16 bank groups)
  constexpr int NLA = C * (K / 4) / kPrepThreads;                        // float4 of log_alpha per thread
  constexpr int NKI = (C * (K / 8) + kPrepThreads - 1) / kPrepThreads;   // (row, 8 channels) items per thread
  static_assert(NLA >= 1 && C * (K / 4) % kPrepThreads == 0, "log_alpha tiling");

  __shared__ __attribute__((aligned(16))) float s_G[C * KP];   // G (log2), then Gam in the fast path
  __shared__ __attribute__((aligned(16))) __bf16 s_kt[2][C * KB];   // Kt hi, lo
  __shared__ __attribute__((aligned(16))) __bf16 s_ki[2][C * KB];   // Ki hi, lo
  // A (later M = P T'), T and P, carved from one buffer that first stages Kh rows
  constexpr int kMatBytes = 3 * C * CP * 4, kKhStageBytes = C * KB * 2 * (SPLIT ? 2 : 1);
  __shared__ __attribute__((aligned(16))) unsigned char s_mat[kMatBytes > kKhStageBytes ? kMatBytes : kKhStageBytes];
  float* s_A = reinterpret_cast<float*>(s_mat);
  float* s_T = s_A + C * CP;
  float* s_P = s_T + C * CP;
  // inversion temporaries and (later) per-wave staging tiles share one buffer
  constexpr int kXSize = (RT > 1 ? RT - 1 : 1) * 16 * 17, kStageSize = 4 * 16 * 17;
  __shared__ float s_scratch[kXSize > kStageSize ? kXSize : kStageSize];
  float* s_X = s_scratch;
  __shared__ float s_beta[C], s_qs[C], s_ks[C];
  __shared__ __attribute__((aligned(16))) float s_gc[K];
  __shared__ int s_valid[C];

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = n * p.chunk;
  const int dk = p.dk;
  const Raw* qg = (const Raw*)p.q;
  const Raw* kg = (const Raw*)p.k;
  uint16_t* wsb = p.ws + ((size_t)(b * p.H + h) * p.NC + n) * L::kElems;
  auto grow = [&](int t) -> size_t { return ((size_t)b * p.T + t) * p.H + h; };
  auto tsafe = [&](int r) -> int { const int t = t0 + r; return t < p.T ? t : p.T - 1; };
  // any readable bytes stand in for the mask when there is none (the value is ignored)
  const uint8_t* mp = p.mask != nullptr ? p.mask : reinterpret_cast<const uint8_t*>(p.beta);

  // ---- phase 1: issue every load of the chunk
  float4 la_r[NLA];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int idx = tid + kPrepThreads * i;
    const int r = idx / (K / 4), c = (idx % (K / 4)) * 4;
    la_r[i] = *reinterpret_cast<const float4*>(p.log_alpha + grow(tsafe(r)) * dk + (c < dk ? c : 0));
  }
  float k_r[NKI][8];
#pragma unroll
  for (int it = 0; it < NKI; ++it) {
    const int idx = (tid + kPrepThreads * it) % (C * (K / 8));
    const int r = idx / (K / 8), c0 = (idx % (K / 8)) * 8;
    E::ld8(kg, grow(tsafe(r)) * dk + (c0 < dk ? c0 : 0), k_r[it]);
  }
  const int I = wave;                                   // this wave's row tile in the A/P and W phases
  const int rq = 16 * (I < RT ? I : 0) + (lane % 16);
  float qtf[KS][8];                                     // raw q now, Qt = q * scale * Gam later
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = 32 * ks + 8 * (lane / 16);
    E::ld8(qg, grow(tsafe(rq)) * dk + (c < dk ? c : 0), qtf[ks]);
  }
  float beta_r = 0.f;
  uint8_t m_r = 1;
  if (tid < C) {
    beta_r = p.beta[grow(tsafe(tid))];
    m_r = mp[(size_t)b * p.T + tsafe(tid)];
  }
  if (tid < C) {
    const int ok = tid < p.chunk && t0 + tid < p.T && (p.mask == nullptr || m_r != 0);
    s_valid[tid] = ok;
    s_beta[tid] = ok ? beta_r : 0.f;
  }
  __syncthreads();

  // ---- log_alpha (log2 units) into LDS, masked rows and padded channels as 0
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int idx = tid + kPrepThreads * i;
    const int r = idx / (K / 4), c = (idx % (K / 4)) * 4;
    const bool ok = c < dk && s_valid[r];
    float* g = s_G + r * KP + c;
    g[0] = ok ? la_r[i].x * kLog2e : 0.f; g[1] = ok ? la_r[i].y * kLog2e : 0.f;
    g[2] = ok ? la_r[i].z * kLog2e : 0.f; g[3] = ok ? la_r[i].w * kLog2e : 0.f;
  }
  // ---- row scales for the optional L2 normalisation of q and k
  if (p.l2norm) {
    for (int r = wave; r < C; r += 4) {
      float sq = 0.f, sk = 0.f;
      const size_t row = grow(tsafe(r)) * dk;
      for (int c = lane; c < dk; c += 64) {
        const float a = E::ld(qg, row + c), kk = E::ld(kg, row + c);
        sq += a * a; sk += kk * kk;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) { sq += __shfl_xor(sq, off, 64); sk += __shfl_xor(sk, off, 64); }
      if (lane == 0) { s_qs[r] = rsqrtf(sq + 1e-6f); s_ks[r] = rsqrtf(sk + 1e-6f); }
    }
  } else if (tid < C) {
    s_qs[tid] = 1.0f;
    s_ks[tid] = 1.0f;
  }
  __syncthreads();

  // ---- inclusive cumulative sum over the chunk, per channel
  if (tid < K) {
    float g[C];
#pragma unroll
    for (int r = 0; r < C; ++r) g[r] = s_G[r * KP + tid];
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) { acc += g[r]; s_G[r * KP + tid] = acc; }
    s_gc[tid] = acc;
  }
  const int fast = __syncthreads_and(tid >= K || s_gc[tid] >= kFastLimit);

  // ---- elementwise decay factors; item = (row r, 8 consecutive channels).  Factors are
  //      at least 2^-120 on the fast path, so the bare hardware exp2 is exact enough.
  {
    __bf16* kh_stage = reinterpret_cast<__bf16*>(s_mat);          // Kh rows, transposed below
    __bf16* kh_stage_lo = kh_stage + C * KB;
#pragma unroll
    for (int it = 0; it < NKI; ++it) {
      const int idx = tid + kPrepThreads * it;
      if (idx < C * (K / 8)) {
        const int r = idx / (K / 8), c0 = (idx % (K / 8)) * 8;
        const float sc = (c0 < dk && s_valid[r]) ? s_ks[r] : 0.f;
        float g[8], gc[8], kt[8], ki[8], kh[8], gam[8];
        ld8f(&s_G[r * KP + c0], g);
        ld8f(&s_gc[c0], gc);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kv = k_r[it][e] * sc;
          gam[e] = __builtin_amdgcn_exp2f(g[e]);
          kt[e] = kv * gam[e];
          ki[e] = fast ? kv * __builtin_amdgcn_exp2f(-g[e]) : 0.f;
          kh[e] = kv * __builtin_amdgcn_exp2f(gc[e] - g[e]);
        }
        bf16x8 hi, lo;
        split8(kt, hi, lo);
        *reinterpret_cast<bf16x8*>(&s_kt[0][r * KB + c0]) = hi;
        *reinterpret_cast<bf16x8*>(&s_kt[1][r * KB + c0]) = lo;
        split8(ki, hi, lo);
        *reinterpret_cast<bf16x8*>(&s_ki[0][r * KB + c0]) = hi;
        *reinterpret_cast<bf16x8*>(&s_ki[1][r * KB + c0]) = lo;
        split8(kh, hi, lo);
        *reinterpret_cast<bf16x8*>(&kh_stage[r * KB + c0]) = hi;
        if (SPLIT) *reinterpret_cast<bf16x8*>(&kh_stage_lo[r * KB + c0]) = lo;
        if (fast) {                         // slow path keeps G for the exact pairwise decays
          float4* gp = reinterpret_cast<float4*>(&s_G[r * KP + c0]);
          gp[0] = make_float4(gam[0], gam[1], gam[2], gam[3]);
          gp[1] = make_float4(gam[4], gam[5], gam[6], gam[7]);
        }
      }
    }
    __syncthreads();
    // Kh^T fragments: row c, contraction over rows 8*oct .. +7
    for (int idx = tid; idx < K * (C / 8); idx += kPrepThreads) {
      const int c = idx % K, oct = idx / K;
      const int rt = c / 16, ks = oct / 4, ln = (c % 16) + 16 * (oct % 4);
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = kh_stage[(8 * oct + e) * KB + c];
      store_frag(wsb + L::off_kh + frag_off(rt, ks, ln, C), v);
      if (SPLIT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = kh_stage_lo[(8 * oct + e) * KB + c];
        store_frag(wsb + L::off_kh + L::kCK + frag_off(rt, ks, ln, C), v);
      }
    }
  }
  if (tid < K) reinterpret_cast<float*>(wsb + L::off_gam)[tid] = exp2f(s_gc[tid]);
  __syncthreads();

  // ---- Qt = q * scale * Gam for this wave's rows (kept in registers for the W phase)
  if (I < RT) {
    const bool rok = s_valid[rq] != 0;
    const float sc = s_qs[rq];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 32 * ks + 8 * (lane / 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = s_G[rq * KP + c + e];
        qtf[ks][e] = (rok && c < dk) ? qtf[ks][e] * sc * (fast ? g : exp2f(g)) : 0.f;
      }
    }
  }

  // ---- A and P
  if (fast) {
    if (I < RT) {
      bf16x8 kth[KS], ktl[KS], qth[KS], qtl[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 32 * ks + 8 * (lane / 16);
        kth[ks] = *reinterpret_cast<const bf16x8*>(&s_kt[0][rq * KB + c]);
        ktl[ks] = *reinterpret_cast<const bf16x8*>(&s_kt[1][rq * KB + c]);
        split8(qtf[ks], qth[ks], qtl[ks]);
      }
      for (int J = 0; J < RT; ++J) {
        f32x4 accA = zero4(), accP = zero4();
        if (J <= I) {
          const int j = 16 * J + (lane % 16);
          f32x4 a[3] = {zero4(), zero4(), zero4()}, pq[3] = {zero4(), zero4(), zero4()};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int c = 32 * ks + 8 * (lane / 16);
            const bf16x8 kih = *reinterpret_cast<const bf16x8*>(&s_ki[0][j * KB + c]);
            const bf16x8 kil = *reinterpret_cast<const bf16x8*>(&s_ki[1][j * KB + c]);
            a[0] = mfma16(kth[ks], kih, a[0]);
            a[1] = mfma16(kth[ks], kil, a[1]);
            a[2] = mfma16(ktl[ks], kih, a[2]);
            pq[0] = mfma16(qth[ks], kih, pq[0]);
            pq[1] = mfma16(qth[ks], kil, pq[1]);
            pq[2] = mfma16(qtl[ks], kih, pq[2]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            accA[i] = a[0][i] + (a[1][i] + a[2][i]);
            accP[i] = pq[0][i] + (pq[1][i] + pq[2][i]);
          }
        }
        const int jj = 16 * J + (lane % 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * I + 4 * (lane / 16) + i;
          s_A[rr * CP + jj] = (jj < rr) ? s_beta[rr] * accA[i] : 0.f;
          s_P[rr * CP + jj] = (jj <= rr) ? accP[i] : 0.f;
        }
      }
    }
  } else {
    // exact pairwise decays (chunks whose total decay in some channel is below 2^-120)
    for (int idx = tid; idx < C * C; idx += kPrepThreads) {
      const int rr = idx / C, jj = idx % C;
      float sa = 0.f, sp = 0.f;
      if (jj <= rr && s_valid[rr] && s_valid[jj]) {
        const size_t tr = grow(t0 + rr) * dk, tj = grow(t0 + jj) * dk;
        for (int c = 0; c < dk; ++c) {
          const float d = exp2f(s_G[rr * KP + c] - s_G[jj * KP + c]);
          const float kj = E::ld(kg, tj + c) * s_ks[jj];
          sa += E::ld(kg, tr + c) * s_ks[rr] * kj * d;
          sp += E::ld(qg, tr + c) * s_qs[rr] * kj * d;
        }
      }
      s_A[rr * CP + jj] = (jj < rr) ? s_beta[rr] * sa : 0.f;
      s_P[rr * CP + jj] = (jj <= rr) ? sp : 0.f;
    }
  }
  __syncthreads();

  // ---- T = (I + A)^-1, blocked: diagonal 16x16 blocks by forward substitution
  if (tid < RT * 16) {
    const int Ib = tid / 16, cc = tid % 16;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      float arow[16];
      ld8f(&s_A[(16 * Ib + rr) * CP + 16 * Ib], arow);
      ld8f(&s_A[(16 * Ib + rr) * CP + 16 * Ib + 8], arow + 8);
      float v = (rr == cc) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < rr; ++jj) v -= arow[jj] * x[jj];
      x[rr] = v;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s_T[(16 * Ib + rr) * CP + 16 * Ib + cc] = x[rr];
  }
  for (int idx = tid; idx < C * C; idx += kPrepThreads) {
    const int rr = idx / C, jj = idx % C;
    if (jj / 16 != rr / 16) s_T[rr * CP + jj] = 0.f;
  }
  __syncthreads();
  // off-diagonal blocks by distance d: T_IJ = -T_II * sum_{L=J}^{I-1} A_IL T_LJ
  for (int d = 1; d < RT; ++d) {
    const int nblk = RT - d;
    for (int e = tid; e < nblk * 256; e += kPrepThreads) {
      const int J = e / 256, Ib = J + d, rr = (e % 256) / 16, cc = e % 16;
      float x = 0.f;
      for (int Lb = J; Lb < Ib; ++Lb)
#pragma unroll
        for (int m = 0; m < 16; ++m) x += s_A[(16 * Ib + rr) * CP + 16 * Lb + m] * s_T[(16 * Lb + m) * CP + 16 * J + cc];
      s_X[J * 272 + rr * 17 + cc] = x;
    }
    __syncthreads();
    for (int e = tid; e < nblk * 256; e += kPrepThreads) {
      const int J = e / 256, Ib = J + d, rr = (e % 256) / 16, cc = e % 16;
      float x = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) x += s_T[(16 * Ib + rr) * CP + 16 * Ib + m] * s_X[J * 272 + m * 17 + cc];
      s_T[(16 * Ib + rr) * CP + 16 * J + cc] = -x;
    }
    __syncthreads();
  }

  // ---- T' = T Diag(beta) and P to the workspace (hi, lo), A-operand order
  for (int idx = tid; idx < RT * CS * 64; idx += kPrepThreads) {
    const int ln = idx % 64, ks = (idx / 64) % CS, rt = idx / (64 * CS);
    const int r = 16 * rt + (ln % 16), j0 = 32 * ks + 8 * (ln / 16);
    float tv[8], pv[8];
    ld8f(&s_T[r * CP + j0], tv);
    ld8f(&s_P[r * CP + j0], pv);
#pragma unroll
    for (int e = 0; e < 8; ++e) tv[e] *= s_beta[j0 + e];
    bf16x8 hi, lo;
    split8(tv, hi, lo);
    store_frag(wsb + L::off_tp + frag_off(rt, ks, ln, C), hi);
    store_frag(wsb + L::off_tp + L::kCC + frag_off(rt, ks, ln, C), lo);
    split8(pv, hi, lo);
    store_frag(wsb + L::off_p + frag_off(rt, ks, ln, C), hi);
    store_frag(wsb + L::off_p + L::kCC + frag_off(rt, ks, ln, C), lo);
  }

  // ---- M = P T' (lower triangular), into s_A; T' and -M A-fragments kept for the W phase
  bf16x8 tnh[CS], tnl[CS], mnh[CS], mnl[CS];
  if (I < RT) {
    bf16x8 ph[CS], pl[CS];
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      float pv[8];
      ld8f(&s_P[rq * CP + 32 * ks + 8 * (lane / 16)], pv);
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
          for (int e = 0; e < 8; ++e) tv[e] = s_T[(m0 + e) * CP + jn] * s_beta[jn];
          bf16x8 th, tl;
          split8(tv, th, tl);
          acc = mfma16(ph[ks], th, acc);
          if (SPLIT) { acc = mfma16(ph[ks], tl, acc); acc = mfma16(pl[ks], th, acc); }
        }
      }
      // each wave reads back only its own rows of M, so a wave-local order suffices
#pragma unroll
      for (int i = 0; i < 4; ++i) s_A[(16 * I + 4 * (lane / 16) + i) * CP + 16 * N + (lane % 16)] = acc[i];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);                 // lgkmcnt(0): this wave's M rows landed
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + 8 * (lane / 16);
      float tv[8], mv[8];
      ld8f(&s_T[rq * CP + j0], tv);
      ld8f(&s_A[rq * CP + j0], mv);
#pragma unroll
      for (int e = 0; e < 8; ++e) { tv[e] = -tv[e] * s_beta[j0 + e]; mv[e] = -mv[e]; }
      split8(tv, tnh[ks], tnl[ks]);
      split8(mv, mnh[ks], mnl[ks]);
    }
  }

  // ---- Wn = -T' Kt and Qh = Qt - M Kt for this wave's 16 rows, all channel tiles
  if (I < RT) {
    float* stage = s_scratch + wave * 16 * 17;
#pragma unroll
    for (int N = 0; N < K / 16; ++N) {
      f32x4 accW = zero4(), accQ = zero4();
      const int cn = 16 * N + (lane % 16);
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;          // T' and M are lower triangular
        const int j0 = 32 * ks + 8 * (lane / 16);
        bf16x8 kth, ktl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kth[e] = s_kt[0][(j0 + e) * KB + cn];
          if (SPLIT) ktl[e] = s_kt[1][(j0 + e) * KB + cn];
        }
        accW = mfma16(tnh[ks], kth, accW);
        accQ = mfma16(mnh[ks], kth, accQ);
        if (SPLIT) {
          accW = mfma16(tnh[ks], ktl, accW); accW = mfma16(tnl[ks], kth, accW);
          accQ = mfma16(mnh[ks], ktl, accQ); accQ = mfma16(mnl[ks], kth, accQ);
        }
      }
      // D layout -> A-operand order: lane L holds row L%16, channels 16N + 8*half .. +7
      // where L/16 = 2*(N%2) + half; that lane also holds those Qt values.
      const int half = (lane / 16) - 2 * (N % 2);
      const bool mine = half == 0 || half == 1;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const f32x4& acc = pass == 0 ? accW : accQ;
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(4 * (lane / 16) + i) * 17 + (lane % 16)] = acc[i];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0): staging writes landed
        if (mine) {
          const int rr = lane % 16;
          float vals[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vals[e] = stage[rr * 17 + 8 * half + e];
          if (pass == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vals[e] += qtf[N / 2][e];
          }
          bf16x8 hi, lo;
          split8(vals, hi, lo);
          const size_t off = (pass == 0 ? L::off_wn : L::off_qh) + frag_off(I, N / 2, lane, K);
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
// Operands of one chunk that a thread needs, loaded from the workspace one chunk
// ahead so that the serial chain of chunks never waits on HBM.
template <int K, int C, bool SPLIT>
struct ScanOps {
  static constexpr int CS = C / 32, KS = K / 32;
  static constexpr int SPW = (K / 16 + 3) / 4;
  static constexpr int VPT = C * 16 / 256;           // V-tile elements per thread
  bf16x8 tph[CS], tpl[CS], ph[CS], pl[CS];
  bf16x8 wn[KS], qh[KS];
  bf16x8 wnl[SPLIT ? KS : 1], qhl[SPLIT ? KS : 1];
  bf16x8 kh[SPW][CS];
  bf16x8 khl[SPLIT ? SPW : 1][CS];
  float gam[SPW][4];
  uint32_t vraw[VPT];                                // V elements as stored (bf16 bits or fp32 bits)
  uint8_t mraw[VPT];                                 // mask bytes of their rows
};

template <int DT, int K, int C>
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(ScanParams p) {
  using E = Elem<DT>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, C, SPLIT>;
  using Ops = ScanOps<K, C, SPLIT>;
  constexpr int RT = C / 16;
  constexpr int CS = C / 32;
  constexpr int KS = K / 32;
  constexpr int SRT = K / 16;                       // state row tiles
  constexpr int SPW = Ops::SPW;                     // state row tiles per wave
  constexpr int KB = K + 8, CB = C + 8;
  static_assert(RT <= 4, "one U/O row tile per wave");

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
  const int I = wave;                                // this wave's U/O row tile
  // predicates the tiling makes always true are compile-time constants, so the
  // prefetch below is straight-line code and its waits stay exact
  const bool has_rows = (RT >= 4) || (I < RT);
  auto srow = [&](int M) { return (SRT % 4 == 0) || (M < SRT); };
  const int dk = p.dk, dv = p.dv;
  const typename E::T* vg = (const typename E::T*)p.v;
  typename E::T* og = (typename E::T*)p.o;
  const uint16_t* wsh = p.ws + (size_t)bh * p.NC * L::kElems;
  // any readable bytes stand in for the mask when there is none (the value is ignored)
  const uint8_t* mp = p.mask != nullptr ? p.mask : reinterpret_cast<const uint8_t*>(p.v);

  auto load_ops = [&](int n, Ops& op) {
    const uint16_t* wsb = wsh + (size_t)n * L::kElems;
    if (has_rows) {
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        op.tph[ks] = load_frag(wsb + L::off_tp + frag_off(I, ks, lane, C));
        op.tpl[ks] = load_frag(wsb + L::off_tp + L::kCC + frag_off(I, ks, lane, C));
        op.ph[ks] = load_frag(wsb + L::off_p + frag_off(I, ks, lane, C));
        op.pl[ks] = load_frag(wsb + L::off_p + L::kCC + frag_off(I, ks, lane, C));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        op.wn[ks] = load_frag(wsb + L::off_wn + frag_off(I, ks, lane, K));
        op.qh[ks] = load_frag(wsb + L::off_qh + frag_off(I, ks, lane, K));
        if (SPLIT) {
          op.wnl[ks] = load_frag(wsb + L::off_wn + L::kCK + frag_off(I, ks, lane, K));
          op.qhl[ks] = load_frag(wsb + L::off_qh + L::kCK + frag_off(I, ks, lane, K));
        }
      }
    }
    const float* gam = reinterpret_cast<const float*>(wsb + L::off_gam);
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
      if (srow(M)) {
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          op.kh[m][ks] = load_frag(wsb + L::off_kh + frag_off(M, ks, lane, C));
          if (SPLIT) op.khl[m][ks] = load_frag(wsb + L::off_kh + L::kCK + frag_off(M, ks, lane, C));
        }
        const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * M + 4 * (lane / 16));
        op.gam[m][0] = g4.x; op.gam[m][1] = g4.y; op.gam[m][2] = g4.z; op.gam[m][3] = g4.w;
      }
    }
    // unconditional loads from in-bounds rows; validity is applied when the chunk is used
    const int t0 = n * p.chunk;
#pragma unroll
    for (int i = 0; i < Ops::VPT; ++i) {
      const int idx = tid + kScanThreads * i;
      const int r = idx / kVT, cidx = idx % kVT, t = t0 + r;
      const int ts = t < p.T ? t : p.T - 1;
      const size_t off = (((size_t)b * p.T + ts) * p.H + h) * dv + v0 + cidx;
      if (DT == 0) op.vraw[i] = reinterpret_cast<const uint16_t*>(vg)[off];
      else op.vraw[i] = __float_as_uint(reinterpret_cast<const float*>(vg)[off]);
      op.mraw[i] = mp[(size_t)b * p.T + ts];
    }
  };

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
      if (srow(M)) {
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

  auto process = [&](const Ops& op, Ops& next, int n, int n_next) {
    const int t0 = n * p.chunk;
    // ---- V tile -> LDS (transposed, hi/lo)
#pragma unroll
    for (int i = 0; i < Ops::VPT; ++i) {
      const int idx = tid + kScanThreads * i;
      const int r = idx / kVT, cidx = idx % kVT, t = t0 + r;
      const bool ok = r < p.chunk && t < p.T && (p.mask == nullptr || op.mraw[i] != 0);
      const float x = ok ? (DT == 0 ? __uint_as_float(op.vraw[i] << 16) : __uint_as_float(op.vraw[i])) : 0.f;
      const __bf16 hi = (__bf16)x;
      s_V[0][cidx * CB + r] = hi;
      s_V[1][cidx * CB + r] = (__bf16)(x - (float)hi);
    }
    load_ops(n_next, next);                                            // prefetch the next chunk
    __syncthreads();                                                   // (a) V and S visible

    bf16x8 sh[KS], sl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = 32 * ks + 8 * (lane / 16);
      sh[ks] = *reinterpret_cast<const bf16x8*>(&s_S[0][(lane % 16) * KB + k0]);
      sl[ks] = *reinterpret_cast<const bf16x8*>(&s_S[1][(lane % 16) * KB + k0]);
    }
    // ---- Ut = T' V and U = Ut + Wn S for this wave's 16 rows (independent accumulators
    //      keep the MFMA dependency chains short)
    if (has_rows) {
      f32x4 ut0 = zero4(), ut1 = zero4();
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;
        const int j0 = 32 * ks + 8 * (lane / 16);
        const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&s_V[0][(lane % 16) * CB + j0]);
        ut0 = mfma16(op.tph[ks], vh, ut0);
        ut1 = mfma16(op.tpl[ks], vh, ut1);
        if (SPLIT) {
          const bf16x8 vl = *reinterpret_cast<const bf16x8*>(&s_V[1][(lane % 16) * CB + j0]);
          ut1 = mfma16(op.tph[ks], vl, ut1);
        }
      }
      f32x4 u[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u[(ks & 1) * 2] = mfma16(op.wn[ks], sh[ks], u[(ks & 1) * 2]);
        u[(ks & 1) * 2 + 1] = mfma16(op.wn[ks], sl[ks], u[(ks & 1) * 2 + 1]);
        if (SPLIT) u[(ks & 1) * 2 + 1] = mfma16(op.wnl[ks], sh[ks], u[(ks & 1) * 2 + 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i;
        const float utv = ut0[i] + ut1[i];
        const float uv = utv + ((u[0][i] + u[2][i]) + (u[1][i] + u[3][i]));
        __bf16 hi = (__bf16)utv;
        s_Ut[0][(lane % 16) * CB + rr] = hi;
        s_Ut[1][(lane % 16) * CB + rr] = (__bf16)(utv - (float)hi);
        hi = (__bf16)uv;
        s_U[0][(lane % 16) * CB + rr] = hi;
        s_U[1][(lane % 16) * CB + rr] = (__bf16)(uv - (float)hi);
      }
    }
    __syncthreads();                                                   // (b) Ut, U visible; S reads done

    // ---- S = Diag(Gam_last) S + Kh^T U  (the chain that carries to the next chunk)
    {
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
        if (!srow(M)) continue;
        f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          a0 = mfma16(op.kh[m][ks], uh[ks], a0);
          a1 = mfma16(op.kh[m][ks], ul[ks], a1);
          if (SPLIT) a1 = mfma16(op.khl[m][ks], uh[ks], a1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) S[m][i] = op.gam[m][i] * S[m][i] + (a0[i] + a1[i]);
      }
    }

    // ---- O = Qh S + P Ut (reads the previous state from registers)
    if (has_rows) {
      f32x4 o4[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        o4[ks & 1] = mfma16(op.qh[ks], sh[ks], o4[ks & 1]);
        o4[ks & 1] = mfma16(op.qh[ks], sl[ks], o4[ks & 1]);
        if (SPLIT) o4[ks & 1] = mfma16(op.qhl[ks], sh[ks], o4[ks & 1]);
      }
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;
        const int j0 = 32 * ks + 8 * (lane / 16);
        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&s_Ut[0][(lane % 16) * CB + j0]);
        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&s_Ut[1][(lane % 16) * CB + j0]);
        o4[2] = mfma16(op.ph[ks], uh, o4[2]);
        o4[3] = mfma16(op.ph[ks], ul, o4[3]);
        o4[3] = mfma16(op.pl[ks], uh, o4[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i, t = t0 + rr;
        const float ov = (o4[0][i] + o4[1][i]) + (o4[2][i] + o4[3][i]);
        if (rr < p.chunk && t < p.T) E::st(og, (((size_t)b * p.T + t) * p.H + h) * dv + v0 + (lane % 16), ov);
      }
    }
    publish_state();
  };

  publish_state();
  // chunk n is processed from registers loaded one chunk earlier; the load for the
  // chunk after the last one re-reads the last chunk (in bounds, unused)
  const int last = p.NC - 1;
  Ops opA, opB;
  if (p.NC > 0) load_ops(0, opA);
  for (int n = 0; n < p.NC; n += 2) {
    process(opA, opB, n, n + 1 <= last ? n + 1 : last);
    if (n + 1 < p.NC) process(opB, opA, n + 1, n + 2 <= last ? n + 2 : last);
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
