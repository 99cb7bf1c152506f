// Decode step of the KDA recurrence: one new token per (b, h), the fp32 state
// updated in place (Kimi Linear summary page, recurrent-layers paragraph: decay
// per channel, remove the old projection onto k, write the new pair; remio.ai
// page, decode section: each generated token reads and rewrites the fixed-size
// state once).  Bandwidth-bound: 8*dk*dv bytes of state traffic per (b, h),
// no MFMA.  With s_j the j-th column of S (rows = key channels):
//   s'_j = alpha * s_j,  a_j = k . s'_j,  c_j = q . s'_j,  u_j = beta (v_j - a_j),
//   s_j <- s'_j + k u_j,  o_j = q . s_j = c_j + (q . k) u_j.
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

template <int DT, int K, int V>
__global__ void __launch_bounds__((DecodeShape<K, V>::kThreads))
decode_step_kernel(const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k,
                   const typename Elem<DT>::T* __restrict__ v, const float* __restrict__ log_alpha,
                   const float* __restrict__ beta, const uint8_t* __restrict__ mask,
                   float* __restrict__ state, typename Elem<DT>::T* __restrict__ o, int H, int l2norm) {
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

  __shared__ float s_q[K], s_k[K], s_alpha[K], s_v[V], s_u[V];
  __shared__ float s_red[2][Sh::kRowGroups][V];
  __shared__ float s_scal[4];

  // the state loads carry all of the traffic: issue them before anything waits
  const int cq = tid % Sh::kColQuads;
  const int rg = tid / Sh::kColQuads;
  const int r0 = rg * Sh::kRows;
  float* sp = state + (size_t)bh * K * V;
  f32x4 s[Sh::kRows];
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r)
    s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + (size_t)(r0 + r) * V + 4 * cq));

  for (int i = tid; i < K; i += Sh::kThreads) {
    s_q[i] = E::ld(q, (size_t)bh * K + i);
    s_k[i] = E::ld(k, (size_t)bh * K + i);
    s_alpha[i] = __expf(log_alpha[(size_t)bh * K + i]);
  }
  for (int j = tid; j < V; j += Sh::kThreads) s_v[j] = E::ld(v, (size_t)bh * V + j);
  __syncthreads();

  // q.k and (optionally) the L2 norms, reduced by the first wavefront
  if (tid < 64) {
    float qq = 0.f, kk = 0.f, qk = 0.f;
    for (int i = tid; i < K; i += 64) {
      float a = s_q[i], c = s_k[i];
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
      s_scal[0] = rq; s_scal[1] = rk; s_scal[2] = qk * rq * rk;
    }
  }
  __syncthreads();
  const float rq = s_scal[0], rk = s_scal[1], qk = s_scal[2];

  float pa[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r) {
    const float al = s_alpha[r0 + r];
    const float kr = s_k[r0 + r] * rk, qr = s_q[r0 + r] * rq;
    s[r].x *= al; s[r].y *= al; s[r].z *= al; s[r].w *= al;
    pa[0] += kr * s[r].x; pa[1] += kr * s[r].y; pa[2] += kr * s[r].z; pa[3] += kr * s[r].w;
    pc[0] += qr * s[r].x; pc[1] += qr * s[r].y; pc[2] += qr * s[r].z; pc[3] += qr * s[r].w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s_red[0][rg][4 * cq + i] = pa[i];
    s_red[1][rg][4 * cq + i] = pc[i];
  }
  __syncthreads();

  const float bt = beta[bh];
  for (int j = tid; j < V; j += Sh::kThreads) {
    float a = 0.f, c = 0.f;
#pragma unroll
    for (int g = 0; g < Sh::kRowGroups; ++g) { a += s_red[0][g][j]; c += s_red[1][g][j]; }
    const float u = bt * (s_v[j] - a);
    s_u[j] = u;
    E::st(ob, j, c + qk * u);
  }
  __syncthreads();

  const float u0 = s_u[4 * cq], u1 = s_u[4 * cq + 1], u2 = s_u[4 * cq + 2], u3 = s_u[4 * cq + 3];
#pragma unroll
  for (int r = 0; r < Sh::kRows; ++r) {
    const float kr = s_k[r0 + r] * rk;
    f32x4 n;
    n.x = s[r].x + kr * u0; n.y = s[r].y + kr * u1; n.z = s[r].z + kr * u2; n.w = s[r].w + kr * u3;
    __builtin_nontemporal_store(n, reinterpret_cast<f32x4*>(sp + (size_t)(r0 + r) * V + 4 * cq));
  }
}

template <int DT, int K, int V>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  using T = typename Elem<DT>::T;
  const int nbh = a.B * a.H;
  if (nbh == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_step_kernel<DT, K, V>), dim3(nbh), dim3(DecodeShape<K, V>::kThreads), 0,
                     (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.log_alpha,
                     a.beta, a.mask, a.state, (T*)a.o, a.H, a.l2norm);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_decode_dt(const DecodeArgs& a) {
#define KDA_DEC_CASE(KK, VV) \
  if (a.dk == KK && a.dv == VV) return launch_decode_t<DT, KK, VV>(a);
#define KDA_DEC_ROW(KK) KDA_DEC_CASE(KK, 16) KDA_DEC_CASE(KK, 32) KDA_DEC_CASE(KK, 64) KDA_DEC_CASE(KK, 128)
  KDA_DEC_ROW(16) KDA_DEC_ROW(32) KDA_DEC_ROW(64) KDA_DEC_ROW(128)
#undef KDA_DEC_ROW
#undef KDA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 0 ? launch_decode_dt<0>(a) : launch_decode_dt<1>(a);
}

}  // namespace kda
