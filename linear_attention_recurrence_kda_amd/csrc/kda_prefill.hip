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
//   Wn = -T' Kt,  Qh = Qt - (P T') Kt,  Ut = T' V,  O0 = P Ut
//   U  = Ut + Wn S0                            (per-token corrections)
//   O  = O0 + Qh S0
//   S1 = Diag(Gam_last) S0 + Kh^T U
// Only the last three lines depend on the state, so the work splits into:
//   prep_kernel: one workgroup per (b, h, chunk), fully parallel; writes Wn, Qh,
//     Kh^T (bf16, MFMA operand order), Ut and O0 (fp32, MFMA accumulator order)
//     and Gam_last to a workspace;
//   scan_kernel: one workgroup per (b, h, 16-column dv tile); a loop over the
//     chunks in order with the fp32 state tile in registers, each chunk's
//     operands streamed into an LDS ring by direct global->LDS copies issued one
//     chunk ahead of their use.
// The factorisation Kt Ki^T (decay relative to the chunk start) is used when
// every channel's decay over the chunk stays above 2^-120 (then no factor
// over- or under-flows); otherwise that chunk computes A and P entry by entry
// with exp2(G_t - G_j).  Entries above the diagonal come from a select, never
// from a product, so nothing from a later position can reach an earlier one.
//
// Precision: bf16 MFMA operands that are not exactly bf16 are split into a
// bf16 high part and a bf16 residual where that matters (A, P, T', S, U, Ut);
// with fp32 inputs every operand is split.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kPrepThreads = 256;
constexpr int kScanThreads = 256;
constexpr int kVT = 16;                  // dv columns per scan workgroup
constexpr float kFastLimit = -120.0f;    // log2 decay over one chunk for the factorised path
constexpr size_t kSinkBytes = 16384;     // workspace tail that absorbs the stores of rows past T

// ---------------------------------------------------------------- workspace layout
// Per (b, h, chunk), in 2-byte units.  Wn, Qh and Kh^T are in A-operand order of
// v_mfma_f32_16x16x32_bf16: fragment (row tile rt, k step ks) is 64 lanes x 8 bf16
// (1 KB), lane l holding M[16 rt + l%16][32 ks + 8 (l/16) .. +7]; with fp32 inputs
// the bf16 residual parts follow the high parts.  Ut and O0 are in accumulator
// order: block (row tile rt, column tile ct) is 64 lanes x 4 fp32 (1 KB), lane l
// holding M[16 rt + 4 (l/16) .. +3][16 ct + l%16].
template <int K, int V, int C, bool SPLIT>
struct WsLayout {
  static constexpr size_t kCK = (size_t)C * K;
  static constexpr size_t kSplitCK = SPLIT ? 2 * kCK : kCK;
  static constexpr size_t kCV = (size_t)C * V * 2;       // fp32 C x V in 2-byte units
  static constexpr size_t off_wn = 0;                    // -T' Kt          [C x K]
  static constexpr size_t off_qh = off_wn + kSplitCK;    // Qt - P T' Kt    [C x K]
  static constexpr size_t off_kh = off_qh + kSplitCK;    // Kh^T            [K x C]
  static constexpr size_t off_ut = off_kh + kSplitCK;    // T' V            [C x V] fp32
  static constexpr size_t off_o0 = off_ut + kCV;         // P T' V          [C x V] fp32
  static constexpr size_t off_gam = off_o0 + kCV;        // Gam_last        [K] fp32
  static constexpr size_t kElems = off_gam + 2 * (size_t)K;
};

__device__ __forceinline__ size_t frag_off(int rt, int ks, int lane, int kk) {
  return ((size_t)(rt * (kk / 32) + ks) * 64 + lane) * 8;
}
template <int V>
__device__ __forceinline__ size_t acc_off(int rt, int ct, int lane) {
  return ((size_t)(rt * (V / 16) + ct) * 64 + lane) * 8;
}

struct PrepParams {
  const void *q, *k, *v;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  uint16_t* ws;
  int B, T, H, dk, dv, chunk, NC, l2norm;
};

struct ScanParams {
  const float* init_state;
  float* final_state;
  void* o;
  const uint16_t* ws;
  void* sink;
  int B, T, H, dk, dv, chunk, NC, NT, nbh;
};

__device__ __forceinline__ void store_frag(uint16_t* dst, const bf16x8& v) {
  *reinterpret_cast<bf16x8*>(dst) = v;
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
// Two 16x16 products computed transposed, so lane l holds columns 4 (l/16) .. +3 of row
// l%16 of column tiles 2s (t0) and 2s + 1 (t1), become the A-operand fragment of k step s
// (lane l: columns 32 s + 8 (l/16) .. +7 of row l%16) with two cross-lane swaps per
// register: the 32-lane swap pairs the tiles' halves, the 16-lane swap interleaves them.
__device__ __forceinline__ void pair_to_afrag(const f32x4& t0, const f32x4& t1, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(t0[i]), __float_as_uint(t1[i]), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
    out[i] = __uint_as_float(b[0]);
    out[4 + i] = __uint_as_float(b[1]);
  }
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
// LDS of one prep workgroup: three regions, each reused by a later phase once the
// barrier after its last read has passed (bf16 rows padded to K + 8, fp32 C x C rows
// to C + 4, so 16 consecutive rows fall into different banks).
template <int DT, int K, int V, int C>
struct PrepLds {
  static constexpr bool SPLIT = DT == 1;
  static constexpr int KP = K + 4, KB = K + 8, CP = C + 4, RT = C / 16;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int kParts = SPLIT ? 2 : 1;
  // R1: Ki hi, lo (fast path) or G (slow path); then T and V^T
  static constexpr int kTBytes = C * CP * 4;
  static constexpr int r1 = cmax(cmax(2 * C * KB * 2, C * KP * 4), kTBytes + kParts * V * C * 2);
  // R2: Kt^T; then Ut^T hi (and lo when it fits)
  static constexpr int kUtPart = V * C * 2;
  static constexpr int kKtBytes = kParts * K * C * 2;
  static constexpr bool kUtLoInR2 = kKtBytes >= 2 * kUtPart;
  static constexpr int r2 = cmax(kKtBytes, kUtLoInR2 ? 2 * kUtPart : kUtPart);
  // R3: Kh^T until stored; then A; then Ut^T lo
  static constexpr int r3 = cmax(cmax(kParts * K * C * 2, C * CP * 4), kUtLoInR2 ? 0 : kUtPart);
  // one 16 x 17 fp32 staging tile per wave (the inversion's block exchange)
  static constexpr int kScratch = 4 * 16 * 17;
};

// x shifted down by n lanes inside each row of 16 lanes (lanes below n read 0)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, false));
}

// One workgroup per (chunk, head, batch row); wave I owns rows 16 I .. 16 I + 15 of
// the chunk.  Lane l of wave I holds row 16 I + l%16 and channels 32 ks + 8 (l/16) .. +7
// for every k step ks: the A-operand layout of the MFMA, so Kt and Qt never leave
// registers on their way into A and P.  All global loads are issued up front,
// unconditionally, from in-bounds rows; validity (mask, ragged tail) is applied by
// select afterwards.
template <int DT, int K, int V, int C>
__global__ void __launch_bounds__(kPrepThreads, DT == 0 ? 2 : 1)
prep_kernel(PrepParams p) {
  using E = Elem<DT>;
  using Raw = typename E::T;
  using Lds = PrepLds<DT, K, V, C>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, V, C, SPLIT>;
  constexpr int RT = C / 16;          // row tiles of the chunk
  constexpr int CS = C / 32;          // k steps over chunk rows
  constexpr int KS = K / 32;          // k steps over key channels
  constexpr int KP = Lds::KP, KB = Lds::KB, CP = Lds::CP;
  constexpr int NVB = (C / 8) * (V / 4);                                 // (8 rows, 4 columns) blocks of V
  constexpr int NVI = (NVB + kPrepThreads - 1) / kPrepThreads;
  static_assert(RT <= 4, "one row tile per wave");

  __shared__ __attribute__((aligned(16))) unsigned char s_r1[Lds::r1];
  __shared__ __attribute__((aligned(16))) unsigned char s_r2[Lds::r2];
  __shared__ __attribute__((aligned(16))) unsigned char s_r3[Lds::r3];
  __shared__ __attribute__((aligned(16))) float s_scratch[Lds::kScratch];
  __shared__ __attribute__((aligned(16))) float s_tot[RT * K];       // per-tile sums of log2 decay
  __shared__ float s_beta[C], s_qs[C], s_ks[C];
  __shared__ int s_valid[C];
  __bf16* s_ki = reinterpret_cast<__bf16*>(s_r1);                    // [hi, lo][C][KB]
  float* s_G = reinterpret_cast<float*>(s_r1);                       // [C][KP] (slow path)
  float* s_T = reinterpret_cast<float*>(s_r1);                       // [C][CP]
  __bf16* s_vT = reinterpret_cast<__bf16*>(s_r1 + Lds::kTBytes);     // [hi(, lo)][V][C] swizzled
  __bf16* s_kt = reinterpret_cast<__bf16*>(s_r2);                    // Kt^T [hi(, lo)][K][C] swizzled
  __bf16* s_uth = reinterpret_cast<__bf16*>(s_r2);                   // [V][C] swizzled
  __bf16* s_utl = Lds::kUtLoInR2 ? s_uth + V * C : reinterpret_cast<__bf16*>(s_r3);
  __bf16* s_khs = reinterpret_cast<__bf16*>(s_r3);                   // Kh^T [hi(, lo)][K][C] swizzled
  float* s_A = reinterpret_cast<float*>(s_r3);                       // [C][CP]

  const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = n * p.chunk;
  const int dk = p.dk, dv = p.dv;
  const Raw* qg = (const Raw*)p.q;
  const Raw* kg = (const Raw*)p.k;
  const Raw* vg = (const Raw*)p.v;
  uint16_t* wsb = p.ws + ((size_t)(b * p.H + h) * p.NC + n) * L::kElems;
  auto grow = [&](int t) -> size_t { return ((size_t)b * p.T + t) * p.H + h; };
  auto tsafe = [&](int r) -> int { const int t = t0 + r; return t < p.T ? t : p.T - 1; };
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
    la_r[ks].load(p.log_alpha, row);
    k_r[ks].load(kg, row);
    q_r[ks].load(qg, row);
  }
  const float beta_r = p.beta[grow(tsafe(rq))];
  const uint8_t m_r = mp[(size_t)b * p.T + tsafe(rq)];
  const bool rok = rows && rq < p.chunk && t0 + rq < p.T && (p.mask == nullptr || m_r != 0);

  // ---- row scales of the optional L2 normalisation (channels past dk read as 0)
  float qs = 1.f, ksc = 1.f;
  if (p.l2norm) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bool cok = 32 * ks + cg < dk;
      float qf[8], kf[8];
      q_r[ks].to_float(qf);
      k_r[ks].to_float(kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = cok ? qf[e] : 0.f, kk = cok ? kf[e] : 0.f;
        sq += a * a; sk += kk * kk;
      }
    }
    sq += __shfl_xor(sq, 16, 64); sk += __shfl_xor(sk, 16, 64);
    sq += __shfl_xor(sq, 32, 64); sk += __shfl_xor(sk, 32, 64);
    qs = rsqrtf(sq + 1e-6f);
    ksc = rsqrtf(sk + 1e-6f);
  }
  if (rows && lane < 16) {
    s_valid[rq] = rok;
    s_beta[rq] = rok ? beta_r : 0.f;
    s_qs[rq] = qs;
    s_ks[rq] = ksc;
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

  // ---- chunk totals Gc of this lane's channels: factorised path when every Gc >= -120
  //      (each wave covers every channel, so all waves reach the same answer)
  // sums of the earlier tiles (pre) and of all tiles (tot); the loop bounds are
  // wave-uniform, so no per-element selects are needed
  auto tile_sums = [&](int ks, float* pre, float* tot) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pre[e] = 0.f;
    const int ilim = rows ? I : 0;
    for (int J = 0; J < ilim; ++J) {
      float t[8];
      ld8f(&s_tot[J * K + 32 * ks + cg], t);
#pragma unroll
      for (int e = 0; e < 8; ++e) pre[e] += t[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tot[e] = pre[e];
    for (int J = ilim; J < RT; ++J) {
      float t[8];
      ld8f(&s_tot[J * K + 32 * ks + cg], t);
#pragma unroll
      for (int e = 0; e < 8; ++e) tot[e] += t[e];
    }
  };
  bool lane_fast = true;
#pragma unroll
  for (int c = lane; c < K; c += 64) {
    float tot = 0.f;
#pragma unroll
    for (int J = 0; J < RT; ++J) tot += s_tot[J * K + c];
    lane_fast = lane_fast && tot >= kFastLimit;
  }
  const bool fast = __all(lane_fast);

  // ---- decay factors for this lane's row.  On the fast path every factor lies in
  //      [2^-120, 2^120], so the bare hardware exp2 is exact enough.
  bf16x8 kth[KS], ktl[KS];
  float qtf[KS][8];                                                  // Qt, fp32 (A and P take its hi, lo split)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c0 = 32 * ks + cg;
    const bool cok = rok && c0 < dk;
    float pre[8], gc[8];
    tile_sums(ks, pre, gc);
    float kt[8], ki[8], kh[8], kf[8], qf[8];
    k_r[ks].to_float(kf);
    q_r[ks].to_float(qf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = g_r[ks][e] + pre[e];
      g_r[ks][e] = g;
      const float kv = cok ? kf[e] * ksc : 0.f;
      const float qv = cok ? qf[e] * qs : 0.f;
      const float gam = __builtin_amdgcn_exp2f(g);
      kt[e] = kv * gam;
      ki[e] = fast ? kv * __builtin_amdgcn_exp2f(-g) : 0.f;
      kh[e] = kv * __builtin_amdgcn_exp2f(gc[e] - g);
      qtf[ks][e] = qv * gam;
    }
    split8(kt, kth[ks], ktl[ks]);
    if (rows) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_kt[swz<C>(c0 + e, rq)] = kth[ks][e];
        if (SPLIT) s_kt[K * C + swz<C>(c0 + e, rq)] = ktl[ks][e];
      }
      bf16x8 hi, lo;
      split8(kh, hi, lo);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_khs[swz<C>(c0 + e, rq)] = hi[e];
        if (SPLIT) s_khs[K * C + swz<C>(c0 + e, rq)] = lo[e];
      }
      if (fast) {
        split8(ki, hi, lo);
        *reinterpret_cast<bf16x8*>(&s_ki[rq * KB + c0]) = hi;
        *reinterpret_cast<bf16x8*>(&s_ki[C * KB + rq * KB + c0]) = lo;
      } else {                                                       // exact pairwise decays need G
        float4* gp = reinterpret_cast<float4*>(&s_G[rq * KP + c0]);
        gp[0] = make_float4(g_r[ks][0], g_r[ks][1], g_r[ks][2], g_r[ks][3]);
        gp[1] = make_float4(g_r[ks][4], g_r[ks][5], g_r[ks][6], g_r[ks][7]);
      }
    }
    if (I == 0 && (lane % 16) == 0) {
      // Gam_last: lanes 0, 16, 32, 48 of wave 0 cover every channel group once
      float gl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) gl[e] = exp2f(gc[e]);
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(wsb + L::off_gam) + c0);
      dst[0] = make_float4(gl[0], gl[1], gl[2], gl[3]);
      dst[1] = make_float4(gl[4], gl[5], gl[6], gl[7]);
    }
  }

  // ---- V: issued now, used after A and P
  float v_r[NVI][8][4];                                              // rows 8 rb .. +7, columns 4 cb .. +3
#pragma unroll
  for (int it = 0; it < NVI; ++it) {
    const int idx = (tid + kPrepThreads * it) % NVB;
    const int rb = idx / (V / 4), cb = idx % (V / 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) E::ld4(vg, grow(tsafe(8 * rb + e)) * dv + 4 * cb, v_r[it][e]);
  }
  __syncthreads();

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
  if (fast) {
    if (rows) {
      // transposed products: A-operand rows are Ki rows of column tile J (LDS), B-operand
      // columns are this wave's Kt and Qt rows (registers); lane (g, r) gets columns
      // 16 J + 4 g .. +3 of row rq of A and P
      bf16x8 qth[KS], qtl[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) split8(qtf[ks], qth[ks], qtl[ks]);
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
              const bf16x8 kih = *reinterpret_cast<const bf16x8*>(&s_ki[j * KB + c]);
              const bf16x8 kil = *reinterpret_cast<const bf16x8*>(&s_ki[C * KB + j * KB + c]);
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
          *reinterpret_cast<float4*>(&s_A[rq * CP + 16 * J + 4 * (lane / 16)]) = make_float4(av[0], av[1], av[2], av[3]);
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
        if (jj <= rq && rok && s_valid[jj]) {
          const size_t tj = grow(t0 + jj) * dk;
          for (int c = 0; c < dk; ++c) {
            const float d = exp2f(s_G[rq * KP + c] - s_G[jj * KP + c]);
            const float kj = E::ld(kg, tj + c) * s_ks[jj];
            sa += E::ld(kg, tr + c) * ksc * kj * d;
            sp += E::ld(qg, tr + c) * qs * kj * d;
          }
        }
        s_A[rq * CP + jj] = (jj < rq) ? beta_r * sa : 0.f;
        pv[e] = sp;
      }
      split8(pv, ph[ks], pl[ks]);
    }
  }
  __syncthreads();                                                   // A complete; Ki or G read

  // ---- V^T (hi, and lo for fp32 inputs) behind T in R1; masked rows as 0
#pragma unroll
  for (int it = 0; it < NVI; ++it) {
    const int idx = tid + kPrepThreads * it;
    if (idx < NVB) {
      const int rb = idx / (V / 4), cb = idx % (V / 4);
      bool ok[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ok[e] = s_valid[8 * rb + e] != 0;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ok[e] ? v_r[it][e][cc] : 0.f;
        bf16x8 hi, lo;
        split8(x, hi, lo);
        const int at = swz<C>(4 * cb + cc, 8 * rb);
        *reinterpret_cast<bf16x8*>(&s_vT[at]) = hi;
        if (SPLIT) *reinterpret_cast<bf16x8*>(&s_vT[V * C + at]) = lo;
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
      ld8f(&s_A[(16 * Ib + rr) * CP + 16 * Ib], arow);
      ld8f(&s_A[(16 * Ib + rr) * CP + 16 * Ib + 8], arow + 8);
      float v0 = (rr == cc) ? 1.f : 0.f, v1 = 0.f;
#pragma unroll
      for (int jj = 0; jj < rr; ++jj) {
        if (jj & 1) v1 -= arow[jj] * x[jj];
        else v0 -= arow[jj] * x[jj];
      }
      x[rr] = v0 + v1;
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s_T[(16 * Ib + rr) * CP + 16 * Ib + cc] = x[rr];
  }
  for (int idx = tid; idx < C * C; idx += kPrepThreads) {
    const int rr = idx / C, jj = idx % C;
    if (jj / 16 != rr / 16) s_T[rr * CP + jj] = 0.f;
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
        ld8f(&s_A[(16 * Ib + r) * CP + (kin ? k0 : 0)], av);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          av[e] = kin ? av[e] : 0.f;
          tv[e] = kin ? s_T[(k0 + e) * CP + 16 * J + r] : 0.f;
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
      ld8f(&s_T[(16 * Ib + r) * CP + 16 * Ib + (klo ? 8 * g : 0)], tiv);
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
      for (int i = 0; i < 4; ++i) s_T[(16 * Ib + 4 * g + i) * CP + 16 * J + r] = -(ya[i] + yb[i]);
    }
    __syncthreads();
  }

  // ---- -T' rows of this wave, and M = P T' computed transposed (A operand: columns of
  //      T', B operand: this wave's P rows), both as A-operand fragments in registers
  bf16x8 tnh[CS], tnl[CS], mnh[CS], mnl[CS];
  if (rows) {
#pragma unroll
    for (int ks = 0; ks < CS; ++ks) {
      const int j0 = 32 * ks + cg;
      float tv[8];
      ld8f(&s_T[rq * CP + j0], tv);
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = -tv[e] * s_beta[j0 + e];
      split8(tv, tnh[ks], tnl[ks]);
    }
#pragma unroll
    for (int s2 = 0; s2 < CS; ++s2) {
      f32x4 mt[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int N = 2 * s2 + t;
        f32x4 acc = zero4();
        if (N <= I) {
          const int jn = 16 * N + (lane % 16);
#pragma unroll
          for (int ms = 0; ms < CS; ++ms) {
            if (32 * ms > 16 * I + 15) continue;                   // P is lower triangular
            const int m0 = 32 * ms + cg;
            float tv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[e] = s_T[(m0 + e) * CP + jn] * s_beta[jn];
            bf16x8 th, tl;
            split8(tv, th, tl);
            acc = mfma16(th, ph[ms], acc);
            if (SPLIT) { acc = mfma16(tl, ph[ms], acc); acc = mfma16(th, pl[ms], acc); }
          }
        }
        mt[t] = acc;
      }
      float mv[8];
      pair_to_afrag(mt[0], mt[1], mv);
#pragma unroll
      for (int e = 0; e < 8; ++e) mv[e] = -mv[e];
      split8(mv, mnh[s2], mnl[s2]);
    }
  }

  // ---- Wn = -T' Kt and Qh = Qt - M Kt for this wave's 16 rows, computed transposed
  //      (A operand: Kt^T rows from LDS, B operand: -T' and -M rows in registers) and
  //      turned into A-operand fragments by lane swaps
  if (rows) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f32x4 dw[2], dq[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int cn = 32 * ks + 16 * t + (lane % 16);
        f32x4 aw = zero4(), aq = zero4();
#pragma unroll
        for (int js = 0; js < CS; ++js) {
          if (32 * js > 16 * I + 15) continue;                     // T' and M are lower triangular
          const int j0 = 32 * js + cg;
          const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&s_kt[swz<C>(cn, j0)]);
          aw = mfma16(kt, tnh[js], aw);
          aq = mfma16(kt, mnh[js], aq);
          if (SPLIT) {
            const bf16x8 ktl_b = *reinterpret_cast<const bf16x8*>(&s_kt[K * C + swz<C>(cn, j0)]);
            aw = mfma16(ktl_b, tnh[js], aw); aw = mfma16(kt, tnl[js], aw);
            aq = mfma16(ktl_b, mnh[js], aq); aq = mfma16(kt, mnl[js], aq);
          }
        }
        dw[t] = aw;
        dq[t] = aq;
      }
      float wv[8], qv[8];
      pair_to_afrag(dw[0], dw[1], wv);
      pair_to_afrag(dq[0], dq[1], qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] += qtf[ks][e];
      bf16x8 hi, lo;
      const size_t off = frag_off(I, ks, lane, K);
      split8(wv, hi, lo);
      store_frag(wsb + L::off_wn + off, hi);
      if (SPLIT) store_frag(wsb + L::off_wn + L::kCK + off, lo);
      split8(qv, hi, lo);
      store_frag(wsb + L::off_qh + off, hi);
      if (SPLIT) store_frag(wsb + L::off_qh + L::kCK + off, lo);
    }
  }
  __syncthreads();                                                   // Kt and A read: R2, R3 take Ut^T

  // ---- Ut = T' V for this wave's rows, every dv tile: to the workspace, and (hi, lo)
  //      transposed into LDS
  if (rows) {
#pragma unroll
    for (int N = 0; N < V / 16; ++N) {
      const int vn = 16 * N + (lane % 16);
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;
        const int j0 = 32 * ks + cg;
        const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&s_vT[swz<C>(vn, j0)]);
        a0 = mfma16(tnh[ks], vh, a0);
        a1 = mfma16(tnl[ks], vh, a1);
        if (SPLIT) a1 = mfma16(tnh[ks], *reinterpret_cast<const bf16x8*>(&s_vT[V * C + swz<C>(vn, j0)]), a1);
      }
      f32x4 ut;
#pragma unroll
      for (int i = 0; i < 4; ++i) ut[i] = -(a0[i] + a1[i]);
      *reinterpret_cast<f32x4*>(wsb + L::off_ut + acc_off<V>(I, N, lane)) = ut;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jr = 16 * I + 4 * (lane / 16) + i;
        const __bf16 hi = (__bf16)ut[i];
        s_uth[swz<C>(vn, jr)] = hi;
        s_utl[swz<C>(vn, jr)] = (__bf16)(ut[i] - (float)hi);
      }
    }
  }
  __syncthreads();

  // ---- O0 = P Ut for this wave's rows, every dv tile
  if (rows) {
#pragma unroll
    for (int N = 0; N < V / 16; ++N) {
      const int vn = 16 * N + (lane % 16);
      f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < CS; ++ks) {
        if (32 * ks > 16 * I + 15) continue;          // P is lower triangular
        const int j0 = 32 * ks + cg;
        const bf16x8 uh = *reinterpret_cast<const bf16x8*>(&s_uth[swz<C>(vn, j0)]);
        const bf16x8 ul = *reinterpret_cast<const bf16x8*>(&s_utl[swz<C>(vn, j0)]);
        a0 = mfma16(ph[ks], uh, a0);
        a1 = mfma16(ph[ks], ul, a1);
        a1 = mfma16(pl[ks], uh, a1);
      }
      f32x4 o0;
#pragma unroll
      for (int i = 0; i < 4; ++i) o0[i] = a0[i] + a1[i];
      *reinterpret_cast<f32x4*>(wsb + L::off_o0 + acc_off<V>(I, N, lane)) = o0;
    }
  }
}

// ================================================================ scan kernel
// One workgroup per (b, h, 16-column dv tile).  Each wave loads the operands it needs for
// a chunk (its row tile of Wn and Qh, its state row tiles of Kh^T, the tile's Ut and O0
// blocks, Gam_last) straight into registers one chunk ahead of their use, with an L2
// warm-up two chunks ahead; LDS only carries the state and U between the waves.
template <int K, int C, bool SPLIT>
struct ScanOps {
  static constexpr int KS = K / 32, CS = C / 32, SPW = (K / 16 + 3) / 4;
  bf16x8 wn[KS], qh[KS];
  bf16x8 wnl[SPLIT ? KS : 1], qhl[SPLIT ? KS : 1];
  bf16x8 kh[SPW][CS];
  bf16x8 khl[SPLIT ? SPW : 1][CS];
  f32x4 ut, o0;
  float4 gam[SPW];
};

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

typedef __attribute__((address_space(3))) void lds_void_t;

template <int DT, int K, int V, int C>
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(ScanParams p) {
  using E = Elem<DT>;
  constexpr bool SPLIT = (DT == 1);
  using L = WsLayout<K, V, C, SPLIT>;
  using Ops = ScanOps<K, C, SPLIT>;
  constexpr int RT = C / 16, CS = C / 32, KS = K / 32, SRT = K / 16;
  constexpr int SPW = Ops::SPW;                     // state row tiles per wave
  constexpr int KB = K + 8, CB = C + 8;
  constexpr int kStores = 4;                        // global stores per lane and chunk, always
  static_assert(RT <= 4, "one U/O row tile per wave");

  __shared__ __attribute__((aligned(16))) __bf16 s_S[2][kVT * KB];    // state hi, lo; B-operand rows = dv column
  __shared__ __attribute__((aligned(16))) __bf16 s_U[2][kVT * CB];    // U hi, lo

  // XCD-aware mapping: all dv tiles of one head share blockIdx.x % 8 (one L2)
  const int L_id = blockIdx.x;
  const int xcd = L_id % 8, slot = L_id / 8;
  const int bh = (slot / p.NT) * 8 + xcd, tile = slot % p.NT;
  if (bh >= p.nbh) return;
  const int b = bh / p.H, h = bh % p.H;
  const int v0 = tile * kVT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);        // uniform: addresses stay scalar
  const int I = wave;                                // this wave's U/O row tile
  // predicates that the tiling makes always true are compile-time constants, so the
  // loads below are straight-line code and the compiler's waits stay exact
  const bool has_rows = (RT >= 4) || (I < RT);
  auto srow = [&](int M) __attribute__((always_inline)) { return (SRT % 4 == 0) || (M < SRT); };
  const int dk = p.dk, dv = p.dv;
  typename E::T* og = (typename E::T*)p.o;
  typename E::T* sink = (typename E::T*)p.sink + (L_id & 63) * 64;
  const uint16_t* wsh = p.ws + (size_t)bh * p.NC * L::kElems;
  const int last = p.NC - 1;

  auto ld16 = [&](const uint16_t* src) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(src);
  };
  // chunk n's operands for this wave, into registers
  auto load_ops = [&](int n, Ops& op) __attribute__((always_inline)) {
    const uint16_t* cb = wsh + (size_t)n * L::kElems;
    if (has_rows) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        op.wn[ks] = ld16(cb + L::off_wn + frag_off(I, ks, lane, K));
        op.qh[ks] = ld16(cb + L::off_qh + frag_off(I, ks, lane, K));
        if (SPLIT) {
          op.wnl[ks] = ld16(cb + L::off_wn + L::kCK + frag_off(I, ks, lane, K));
          op.qhl[ks] = ld16(cb + L::off_qh + L::kCK + frag_off(I, ks, lane, K));
        }
      }
      op.ut = *reinterpret_cast<const f32x4*>(cb + L::off_ut + acc_off<V>(I, tile, lane));
      op.o0 = *reinterpret_cast<const f32x4*>(cb + L::off_o0 + acc_off<V>(I, tile, lane));
    }
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
      const int M = wave + 4 * m;
      if (srow(M)) {
#pragma unroll
        for (int ks = 0; ks < CS; ++ks) {
          op.kh[m][ks] = ld16(cb + L::off_kh + frag_off(M, ks, lane, C));
          if (SPLIT) op.khl[m][ks] = ld16(cb + L::off_kh + L::kCK + frag_off(M, ks, lane, C));
        }
        op.gam[m] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(cb + L::off_gam) + 16 * M + 4 * (lane / 16));
      }
    }
  };

  // L2 warm-up two chunks ahead: one 4-byte load per 128-byte line that this workgroup's
  // loads will read, so they hit in L2.  The loaded word is consumed by an empty asm
  // statement one chunk later, when it has long arrived, which keeps the load alive
  // without a wait anywhere else.  Thread g takes line g of the list [its
  // 1/NT share of the lines every tile reads (Wn, Qh, Kh^T); its tile's Ut and O0 lines; the
  // Gam_last lines]; threads past the end repeat the first line.
  constexpr int kNT = V / kVT;
  constexpr int kShLines = (int)(L::off_ut * 2 / 128);
  constexpr int kOwnLines = 2 * (C / 16) * 8 + (4 * K + 127) / 128;
  size_t pf_off = 0;                                                   // bytes from the chunk base
  {
    const int sh_mine = (kShLines - tile + kNT - 1) / kNT;
    const int g = tid;
    if (g < sh_mine) {
      pf_off = (size_t)(tile + kNT * g) * 128;
    } else if (g - sh_mine < kOwnLines) {
      const int j = g - sh_mine;
      if (j < 2 * (C / 16) * 8) {
        const int blk = j / 8, line = j % 8;
        const size_t base = blk < C / 16 ? L::off_ut + acc_off<V>(blk, tile, 0)
                                         : L::off_o0 + acc_off<V>(blk - C / 16, tile, 0);
        pf_off = base * 2 + (size_t)line * 128;
      } else {
        pf_off = L::off_gam * 2 + (size_t)(j - 2 * (C / 16) * 8) * 128;
      }
    }
  }
  uint32_t warm_word = 0;
  auto warm_chunk = [&](int n) __attribute__((always_inline)) {
    const unsigned char* cb = reinterpret_cast<const unsigned char*>(wsh + (size_t)n * L::kElems);
    asm volatile("" :: "v"(warm_word));
    warm_word = *reinterpret_cast<const uint32_t*>(cb + pf_off);
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
  // byte offsets of this lane's output elements from token t0 of the chunk (tokens are
  // H * dv elements apart; the host keeps these below 2^32)
  const size_t o_row_bytes = (size_t)p.H * dv * sizeof(typename E::T);
  uint32_t o_lane[kStores];
#pragma unroll
  for (int i = 0; i < kStores; ++i)
    o_lane[i] = (uint32_t)((16 * I + 4 * (lane / 16) + i) * o_row_bytes +
                           ((size_t)h * dv + v0 + lane % 16) * sizeof(typename E::T));
  auto publish_state = [&]() __attribute__((always_inline)) {
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

  // one chunk with its operands in registers; ends with exactly kStores global stores per lane
  auto process = [&](const Ops& op, int n) __attribute__((always_inline)) {
    const int t0 = n * p.chunk;
    // every row of a full chunk is in range: its stores need no check
    const bool full = (p.chunk == C) && (t0 + C <= p.T);
    unsigned char* ochunk = reinterpret_cast<unsigned char*>(og) + ((size_t)b * p.T + t0) * o_row_bytes;
    bf16x8 sh[KS], slo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k0 = 32 * ks + 8 * (lane / 16);
      sh[ks] = *reinterpret_cast<const bf16x8*>(&s_S[0][(lane % 16) * KB + k0]);
      slo[ks] = *reinterpret_cast<const bf16x8*>(&s_S[1][(lane % 16) * KB + k0]);
    }
    // ---- U = Ut + Wn S for this wave's 16 rows (independent accumulators keep the chains short)
    if (has_rows) {
      f32x4 u[4] = {op.ut, zero4(), zero4(), zero4()};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u[(ks & 1) * 2] = mfma16(op.wn[ks], sh[ks], u[(ks & 1) * 2]);
        u[(ks & 1) * 2 + 1] = mfma16(op.wn[ks], slo[ks], u[(ks & 1) * 2 + 1]);
        if (SPLIT) u[(ks & 1) * 2 + 1] = mfma16(op.wnl[ks], sh[ks], u[(ks & 1) * 2 + 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i;
        const float uv = (u[0][i] + u[2][i]) + (u[1][i] + u[3][i]);
        const __bf16 hi = (__bf16)uv;
        s_U[0][(lane % 16) * CB + rr] = hi;
        s_U[1][(lane % 16) * CB + rr] = (__bf16)(uv - (float)hi);
      }
    }
    wait_lgkm();
    wg_barrier();                                                      // U visible; S reads done

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
        const float gg[4] = {op.gam[m].x, op.gam[m].y, op.gam[m].z, op.gam[m].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) S[m][i] = gg[i] * S[m][i] + (a0[i] + a1[i]);
      }
    }
    publish_state();

    // ---- O = O0 + Qh S (the state entering the chunk, still in fragments)
    if (has_rows) {
      f32x4 o4[2] = {op.o0, zero4()};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        o4[ks & 1] = mfma16(op.qh[ks], sh[ks], o4[ks & 1]);
        o4[ks & 1] = mfma16(op.qh[ks], slo[ks], o4[ks & 1]);
        if (SPLIT) o4[ks & 1] = mfma16(op.qhl[ks], sh[ks], o4[ks & 1]);
      }
#pragma unroll
      for (int i = 0; i < kStores; ++i) {
        const int rr = 16 * I + 4 * (lane / 16) + i;
        typename E::T* dst = reinterpret_cast<typename E::T*>(ochunk + o_lane[i]);
        if (!full && !(rr < p.chunk && t0 + rr < p.T)) dst = sink + 16 * i + (lane % 16);
        E::st(dst, 0, o4[0][i] + o4[1][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kStores; ++i) {                             // keep the store count uniform
        volatile typename E::T* dst = sink + 16 * i + (lane % 16);
        *dst = (typename E::T)0;
      }
    }
  };

  publish_state();
  // Operands of chunk n are loaded at the top of chunk n - 1 (the first ones here), the
  // L2 warm-up for chunk n + 1 beside them; loads into the registers of one buffer are
  // issued only after the previous chunk that used that buffer is done with it.
  // The loop body holds two chunks with no condition between them, so each buffer keeps
  // its own registers and the compiler's waits stay exact.
  Ops opA, opB;
  if (p.NC > 0) load_ops(0, opA);
  if (p.NC > 1) warm_chunk(1);
  int n = 0;
  for (; n + 1 < p.NC; n += 2) {
    wait_lgkm();
    wg_barrier();                                                      // state visible
    load_ops(n + 1, opB);
    warm_chunk(n + 2 <= last ? n + 2 : last);
    process(opA, n);
    wait_lgkm();
    wg_barrier();
    load_ops(n + 2 <= last ? n + 2 : last, opA);
    warm_chunk(n + 3 <= last ? n + 3 : last);
    process(opB, n + 1);
  }
  if (n < p.NC) {                                                      // odd chunk count: the last one
    wait_lgkm();
    wg_barrier();
    process(opA, n);
  }
  asm volatile("" :: "v"(warm_word));
  __builtin_amdgcn_s_waitcnt(0);

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
// The chunk size only changes rounding (the result is the token recurrence for any
// chunk), so chunks above 64 tokens run as 64-token chunks: a 128- or 256-token WY
// block would not fit the LDS of a workgroup, and its decay factors would leave the fp32
// range for ordinary gates.
static int run_chunk(int chunk) { return chunk > 64 ? 64 : chunk; }
static int tile_chunk(int chunk) { return chunk <= 32 ? 32 : 64; }
static int pad_k(int dk) { return dk < 32 ? 32 : dk; }

bool prefill_supported(int dk, int dv, int chunk) {
  (void)dk; (void)dv;
  return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256;
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

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
  if (T == 0 || B == 0 || H == 0) return 0;
  chunk = run_chunk(chunk);
  const int NC = (T + chunk - 1) / chunk;
  return (size_t)B * H * NC * chunk_ws_elems(pad_k(dk), dv, tile_chunk(chunk), dtype) * 2 + kSinkBytes;
}

template <int DT, int K, int V, int C>
static hipError_t launch_prefill_t(const PrefillArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  if ((size_t)(C + 1) * a.H * a.dv * 4 > 0xffffffffull) return hipErrorInvalidValue;   // 32-bit output offsets
  const int NC = (a.T + a.chunk - 1) / a.chunk;
  const int NT = a.dv / kVT;
  const int nbh = a.B * a.H;
  const size_t chunks_bytes = (size_t)nbh * NC * WsLayout<K, V, C, DT == 1>::kElems * 2;
  if (NC > 0) {
    PrepParams pp{a.q, a.k, a.v, a.log_alpha, a.beta, a.mask, (uint16_t*)a.workspace,
                  a.B, a.T, a.H, a.dk, a.dv, a.chunk, NC, a.l2norm};
    hipLaunchKernelGGL((prep_kernel<DT, K, V, C>), dim3(NC, a.H, a.B), dim3(kPrepThreads), 0, st, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanParams sp{a.init_state, a.final_state, a.o, (const uint16_t*)a.workspace,
                NC > 0 ? (void*)((unsigned char*)a.workspace + chunks_bytes) : nullptr,
                a.B, a.T, a.H, a.dk, a.dv, a.chunk, NC, NT, nbh};
  const int groups = (nbh + 7) / 8;
  hipLaunchKernelGGL((scan_kernel<DT, K, V, C>), dim3(groups * 8 * NT), dim3(kScanThreads), 0, st, sp);
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

hipError_t launch_prefill(const PrefillArgs& args) {
  PrefillArgs a = args;
  a.chunk = run_chunk(a.chunk);
  return a.dtype == 0 ? launch_prefill_dt<0>(a) : launch_prefill_dt<1>(a);
}

}  // namespace kda
