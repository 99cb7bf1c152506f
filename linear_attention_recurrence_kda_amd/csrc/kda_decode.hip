// Decode step of the KDA recurrence: one new token per (b, h), the fp32 state
// updated in place (Kimi Linear summary page, recurrent-layers paragraph: decay
// per channel, remove the old projection onto k, write the new pair; remio.ai
// page, decode section: each generated token reads and rewrites the fixed-size
// state once).  Bandwidth-bound: 8*dk*dv bytes of state traffic per (b, h),
// no MFMA.  With s_j the j-th column of S (rows = key channels):
//   s'_j = alpha * s_j,  a_j = k . s'_j,  c_j = q . s'_j,  u_j = beta (v_j - a_j),
//   s_j <- s'_j + k u_j,  o_j = q . s_j = c_j + (q . k) u_j.
// Two kernels share the step: decode_step_kernel reads q, k, v; fused_decode_kernel
// first forms them with the three short convolutions at T = 1 (and updates their
// caches), so a serving loop needs one launch per step.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int K, int V>
struct DecodeShape {
  static constexpr int kColQuads = V / 4;                     // threads along dv
  static constexpr int kThreads = (K * V / 4) < 256 ? (K * V / 4) : 256;
  static constexpr int kRowGroups = kThreads / kColQuads;     // threads along dk
  static constexpr int kRows = K / kRowGroups;                // rows per thread
  static_assert(kThreads % kColQuads == 0, "shape");
  static_assert(K % kRowGroups == 0, "shape");
};

// LDS of one (b, h) step: its q, k, alpha = exp(log_alpha), v, u and the partial sums
template <int K, int V>
struct DecodeLds {
  float q[K], k[K], alpha[K], v[V], u[V];
  float red[2][DecodeShape<K, V>::kRowGroups][V];
  float scal[4];
};

// This thread's rows of the state (the loads that carry all of the traffic: issued
// before anything waits).  Thread tid holds rows r0 .. r0 + kRows - 1, columns 4 cq .. + 3.
template <int K, int V>
__device__ __forceinline__ void load_state_rows(const float* sp, f32x4* s, int tid) {
  using Sh = DecodeShape<K, V>;
  const int cq = tid % Sh::kColQuads, r0 = (tid / Sh::kColQuads) * Sh::kRows;
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r)
    s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)(r0 + r) * V + 4 * cq));
}

// The step from q, k, alpha and v in LDS (written before a barrier): o to ob, the new
// state back to sp.
template <int DT, int K, int V>
__device__ __forceinline__ void decode_update(DecodeLds<K, V>& L, f32x4* s, float* sp,
                                              typename Elem<DT>::T* ob, float bt, int l2norm, int tid) {
  using Sh = DecodeShape<K, V>;
  using E = Elem<DT>;
  const int cq = tid % Sh::kColQuads;
  const int rg = tid / Sh::kColQuads;
  const int r0 = rg * Sh::kRows;

  // q.k and (optionally) the L2 norms, reduced by the first wavefront
  if (tid < 64) {
    float qq = 0.f, kk = 0.f, qk = 0.f;
    for (int i = tid; i < K; i += 64) {
      float a = L.q[i], c = L.k[i];
      qq += a * a; kk += c * c; qk += a * c;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      qq += __shfl_xor(qq, off, 64);
      kk += __shfl_xor(kk, off, 64);
      qk += __shfl_xor(qk, off, 64);
    }
    if (tid == 0) {
      float rq = l2norm ? rsqrtf(qq + 1e-6f) : 1.0f;
      float rk = l2norm ? rsqrtf(kk + 1e-6f) : 1.0f;
      L.scal[0] = rq; L.scal[1] = rk; L.scal[2] = qk * rq * rk;
    }
  }
  __syncthreads();
  const float rq = L.scal[0], rk = L.scal[1], qk = L.scal[2];

  float pa[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r) {
    const float al = L.alpha[r0 + r];
    const float kr = L.k[r0 + r] * rk, qr = L.q[r0 + r] * rq;
    s[r].x *= al; s[r].y *= al; s[r].z *= al; s[r].w *= al;
    pa[0] += kr * s[r].x; pa[1] += kr * s[r].y; pa[2] += kr * s[r].z; pa[3] += kr * s[r].w;
    pc[0] += qr * s[r].x; pc[1] += qr * s[r].y; pc[2] += qr * s[r].z; pc[3] += qr * s[r].w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    L.red[0][rg][4 * cq + i] = pa[i];
    L.red[1][rg][4 * cq + i] = pc[i];
  }
  __syncthreads();

  for (int j = tid; j < V; j += Sh::kThreads) {
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int g = 0; g < Sh::kRowGroups; ++g) { a += L.red[0][g][j]; c += L.red[1][g][j]; }
    const float u = bt * (L.v[j] - a);
    L.u[j] = u;
    E::st(ob, j, c + qk * u);
  }
  __syncthreads();

  const float u0 = L.u[4 * cq], u1 = L.u[4 * cq + 1], u2 = L.u[4 * cq + 2], u3 = L.u[4 * cq + 3];
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r) {
    const float kr = L.k[r0 + r] * rk;
    f32x4 n;
    n.x = s[r].x + kr * u0; n.y = s[r].y + kr * u1; n.z = s[r].z + kr * u2; n.w = s[r].w + kr * u3;
    __builtin_nontemporal_store(n, reinterpret_cast<f32x4*>(sp + (size_t)(r0 + r) * V + 4 * cq));
  }
}

template <int DT, int K, int V>
__global__ void __launch_bounds__((DecodeShape<K, V>::kThreads))
decode_step_kernel(const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k,
                   const typename Elem<DT>::T* __restrict__ v, const float* __restrict__ log_alpha,
                   const float* __restrict__ beta, const uint8_t* __restrict__ mask,
                   float* __restrict__ state, typename Elem<DT>::T* __restrict__ o, int H, int l2norm,
                   int scalar_gate) {
  using Sh = DecodeShape<K, V>;
  using E = Elem<DT>;
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int tid = threadIdx.x;
  typename E::T* ob = o + (size_t)bh * V;

  if (mask != nullptr && mask[b] == 0) {           // padded step: state untouched, o = 0
    for (int j = tid; j < V; j += Sh::kThreads) E::st(ob, j, 0.0f);
    return;
  }

  __shared__ DecodeLds<K, V> L;
  float* sp = state + (size_t)bh * K * V;
  // q, k, log_alpha and v first (one element per thread, index clamped so that no load
  // sits under a branch), then the state rows: the waits for the small loads then do
  // not wait behind the state traffic
  static_assert(K <= Sh::kThreads && V <= Sh::kThreads, "one element per thread");
  const int ik = tid < K ? tid : K - 1, iv = tid < V ? tid : V - 1;
  const float qv = E::ld(q, (size_t)bh * K + ik), kv = E::ld(k, (size_t)bh * K + ik);
  // Gated DeltaNet's gate: one log_alpha per (b, h) for every channel
  const float la = log_alpha[scalar_gate ? (size_t)bh : (size_t)bh * K + ik], vv = E::ld(v, (size_t)bh * V + iv);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 s[Sh::kRows];
  load_state_rows<K, V>(sp, s, tid);
  if (tid < K) { L.q[tid] = qv; L.k[tid] = kv; L.alpha[tid] = __expf(la); }
  if (tid < V) L.v[tid] = vv;
  __syncthreads();
  decode_update<DT, K, V>(L, s, sp, ob, beta[bh], l2norm, tid);
}

// One channel of a short convolution at T = 1: the causal window is the W - 1 cached
// inputs, then x.  Loaded first (the values are small and needed before the state is),
// then formed with the same operations in the same order as the convolution kernel's,
// and the cache shifted by one.
template <int DT>
struct ConvChannel {
  float hist[3], x, w[3], wl, bias;                  // wl: the tap on the current input
  __device__ __forceinline__ void load(const typename Elem<DT>::T* xp, const float* wp, const float* bp,
                                       const typename Elem<DT>::T* cache, int b, int D, int c, int W) {
    using E = Elem<DT>;
    // indexes clamped into range instead of branches: every load is issued, in bounds,
    // and the values past W are never used
#pragma unroll
    for (int j = 0; j < 3; ++j)
      hist[j] = E::ld(cache, ((size_t)b * (W - 1) + (j < W - 1 ? j : W - 2)) * D + c);
    x = E::ld(xp, (size_t)b * D + c);
#pragma unroll
    for (int j = 0; j < 3; ++j) w[j] = wp[(size_t)c * W + (j < W - 1 ? j : W - 2)];
    wl = wp[(size_t)c * W + W - 1];
    const float bl = *(bp != nullptr ? bp + c : wp + (size_t)c * W);
    bias = bp != nullptr ? bl : 0.f;
  }
  // y as it reads back after a store; the cache shifted by one
  __device__ __forceinline__ float apply(typename Elem<DT>::T* cache, int b, int D, int c, int W, int silu) const {
    using E = Elem<DT>;
    float acc = bias;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < W - 1) acc += w[j] * hist[j];
    acc += wl * x;
    if (silu) acc = acc / (1.0f + __expf(-acc));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < W - 2) E::st(cache, ((size_t)b * (W - 1) + j) * D + c, hist[j + 1]);
    E::st(cache, ((size_t)b * (W - 1) + (W - 2)) * D + c, x);
    return E::round(acc);
  }
};

struct FusedDecodeParams {
  const void *xq, *xk, *xv;
  const float *wq, *wk, *wv, *bq, *bk, *bv;
  void *cq, *ck, *cv;
  const float *log_alpha, *beta;
  const uint8_t* mask;
  float* state;
  const int32_t* slot;
  void* o;
  int H, S, W, l2norm, silu, scalar_gate;
};

template <int DT, int K, int V>
__global__ void __launch_bounds__((DecodeShape<K, V>::kThreads))
fused_decode_kernel(FusedDecodeParams p) {
  using Sh = DecodeShape<K, V>;
  using E = Elem<DT>;
  using Tp = typename E::T;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x;
  Tp* ob = (Tp*)p.o + (size_t)bh * V;
  const int slot = p.slot != nullptr ? p.slot[b] : b;

  // padded step (or a slot outside the pool): state and caches untouched, o = 0
  if ((p.mask != nullptr && p.mask[b] == 0) || slot < 0 || slot >= p.S) {
    for (int j = tid; j < V; j += Sh::kThreads) E::st(ob, j, 0.0f);
    return;
  }

  __shared__ DecodeLds<K, V> L;
  float* sp = p.state + ((size_t)slot * p.H + h) * K * V;

  // this head's channels of the three convolutions, q (K), then k (K), then v (V): thread
  // tid takes channels tid, tid + kThreads, ...  Their inputs are loaded before the state
  // rows, so the convolutions do not wait behind the state traffic; no load sits under a
  // branch (a thread past the last channel loads the last one and discards it).
  constexpr int kCh = 2 * K + V, kPer = (kCh + Sh::kThreads - 1) / Sh::kThreads;
  const int Dk = p.H * K, Dv = p.H * V;
  auto which = [&](int i, const Tp*& xp, const float*& wp, const float*& bp, Tp*& cp, int& D, int& c) {
    if (i < K) { xp = (const Tp*)p.xq; wp = p.wq; bp = p.bq; cp = (Tp*)p.cq; D = Dk; c = h * K + i; }
    else if (i < 2 * K) { xp = (const Tp*)p.xk; wp = p.wk; bp = p.bk; cp = (Tp*)p.ck; D = Dk; c = h * K + i - K; }
    else { xp = (const Tp*)p.xv; wp = p.wv; bp = p.bv; cp = (Tp*)p.cv; D = Dv; c = h * V + i - 2 * K; }
  };
  ConvChannel<DT> ch[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int i = min(tid + t * Sh::kThreads, kCh - 1);
    const Tp* xp; const float *wp, *bp; Tp* cp; int D, c;
    which(i, xp, wp, bp, cp, D, c);
    ch[t].load(xp, wp, bp, cp, b, D, c, p.W);
  }
  static_assert(K <= Sh::kThreads, "one log_alpha per thread");
  const float la = p.log_alpha[p.scalar_gate ? (size_t)bh : (size_t)bh * K + (tid < K ? tid : K - 1)];
  __builtin_amdgcn_sched_barrier(0);                // every small load ahead of the state's
  f32x4 s[Sh::kRows];
  load_state_rows<K, V>(sp, s, tid);
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int i = tid + t * Sh::kThreads;
    if (i < kCh) {
      const Tp* xp; const float *wp, *bp; Tp* cp; int D, c;
      which(i, xp, wp, bp, cp, D, c);
      const float y = ch[t].apply(cp, b, D, c, p.W, p.silu);
      if (i < K) L.q[i] = y;
      else if (i < 2 * K) L.k[i - K] = y;
      else L.v[i - 2 * K] = y;
    }
  }
  if (tid < K) L.alpha[tid] = __expf(la);
  __syncthreads();
  decode_update<DT, K, V>(L, s, sp, ob, p.beta[bh], p.l2norm, tid);
}

template <int DT, int K, int V>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  using T = typename Elem<DT>::T;
  const int nbh = a.B * a.H;
  if (nbh == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_step_kernel<DT, K, V>), dim3(nbh), dim3(DecodeShape<K, V>::kThreads), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha,
                     a.beta, a.mask, a.state, (T*)a.o, a.H, a.l2norm, a.scalar_gate);
  return hipGetLastError();
}

template <int DT, int K, int V>
static hipError_t launch_fused_t(const FusedDecodeArgs& a) {
  const int nbh = a.B * a.H;
  if (nbh == 0) return hipSuccess;
  FusedDecodeParams p{a.xq, a.xk, a.xv, a.wq, a.wk, a.wv, a.bq, a.bk, a.bv, a.cq, a.ck, a.cv,
                      a.log_alpha, a.beta, a.mask, a.state, a.slot, a.o, a.H, a.S, a.W, a.l2norm, a.silu,
                      a.scalar_gate};
  hipLaunchKernelGGL((fused_decode_kernel<DT, K, V>), dim3(nbh), dim3(DecodeShape<K, V>::kThreads), 0,
                     (hipStream_t)a.stream, p);
  return hipGetLastError();
}

#define KDA_DEC_ROW(CASE, KK) CASE(KK, 16) CASE(KK, 32) CASE(KK, 64) CASE(KK, 128)
#define KDA_DEC_ALL(CASE) KDA_DEC_ROW(CASE, 16) KDA_DEC_ROW(CASE, 32) KDA_DEC_ROW(CASE, 64) KDA_DEC_ROW(CASE, 128)

template <int DT>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
#define KDA_DEC_CASE(KK, VV) \
  if (a.dk == KK && a.dv == VV) return launch_decode_t<DT, KK, VV>(a);
  KDA_DEC_ALL(KDA_DEC_CASE)
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_fused_dt(const FusedDecodeArgs& a) {
#define KDA_DEC_CASE(KK, VV) \
  if (a.dk == KK && a.dv == VV) return launch_fused_t<DT, KK, VV>(a);
  KDA_DEC_ALL(KDA_DEC_CASE)
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 0 ? launch_decode_dt<0>(a) : launch_decode_dt<1>(a);
}

hipError_t launch_decode_fused(const FusedDecodeArgs& a) {
  return a.dtype == 0 ? launch_fused_dt<0>(a) : launch_fused_dt<1>(a);
}

}  // namespace kda
