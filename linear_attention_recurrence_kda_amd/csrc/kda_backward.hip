// Gradients of the KDA prefill (remio.ai page, KDA section: the blockwise training algorithm
// needs them): for L = sum_t <do_t, o_t> + <dfinal, S_T>, the derivatives with respect to q,
// k, v, log_alpha, beta and the initial state, in fp32.
//
// Per token (mask = 1), with S' = Diag(a) S_{t-1}, a = exp(log_alpha_t), r = v_t - S'^T k_t,
// u = beta_t r, S_t = S' + k_t u^T and lam = dL/dS_t (reverse-mode differentiation of the
// recurrence):
//   L    = lam + q_t do_t^T            dq_t = S_t do_t
//   du   = L^T k_t                     dk_t = L u - S' (beta_t du)
//   dbeta_t = du . r                   dv_t = beta_t du
//   dS'  = L - k_t (beta_t du)^T       dlog_alpha_t = rowsum(dS' * S')
//   lam <- Diag(a) dS'
// A masked position passes lam through unchanged and gets zero gradients.
//
// One workgroup per (b, h) walks the sequence twice.  Forward: the state every kSeg tokens
// goes to the workspace.  Backward: for each kSeg-token segment, last first, the segment's
// states are recomputed from its checkpoint into the workspace, then the adjoint runs back
// over the segment.  Each of the 256 threads holds a (dk/16) x (dv/16) block of S and of lam;
// sums over a row of the block grid (16 neighbouring lanes) use lane shuffles, sums over a
// column (16 row blocks in four waves) shuffles and then LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kBwdThreads = 256;
constexpr int kSeg = 16;                 // tokens between saved forward states

struct BwdParams {
  const void *q, *k, *v, *dout;
  const float *log_alpha, *beta, *init_state, *dfinal;
  const uint8_t* mask;
  float *dq, *dk, *dv, *dla, *dbeta, *dinit;
  float* ws;
  int B, T, H, dk_, dv_, nseg;
};

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv) {
  if (T <= 0) return 0;                          // no token: dinit = dfinal, nothing saved
  const size_t nseg = ((size_t)T + kSeg - 1) / kSeg;
  return (size_t)B * H * (nseg + kSeg) * dk * dv * sizeof(float);
}

template <int DT, int K, int V>
__global__ void __launch_bounds__(kBwdThreads) backward_kernel(BwdParams p) {
  using E = Elem<DT>;
  using Tv = typename E::T;
  constexpr int RB = K / 16, CB = V / 16;          // rows and columns of this thread's block
  __shared__ float s_col[2][4][V];                 // per-wave column partial sums, two slots

  const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = tid / 16, cb = tid % 16;
  const int r0 = rb * RB, c0 = cb * CB;
  const int T = p.T;
  float* ckpt = p.ws + (size_t)bh * (p.nseg + kSeg) * K * V;   // nseg checkpoints
  float* segbuf = ckpt + (size_t)p.nseg * K * V;                // kSeg states of one segment
  auto tok = [&](int t) -> size_t { return ((size_t)b * T + t) * p.H + h; };
  auto valid = [&](int t) -> bool { return p.mask == nullptr || p.mask[(size_t)b * T + t] != 0; };

  float S[RB][CB], lam[RB][CB];
  auto store_block = [&](float* dst, const float (&x)[RB][CB]) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) dst[(size_t)(r0 + i) * V + c0 + j] = x[i][j];
  };
  auto load_block = [&](const float* src, float (&x)[RB][CB]) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) x[i][j] = src[(size_t)(r0 + i) * V + c0 + j];
  };
  // sum over the 16 row blocks of a per-column partial (all 16 threads of each column get it)
  int slot = 0;
  auto colsum = [&](float (&part)[CB], float (&out)[CB]) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      float x = part[j];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      part[j] = x;
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < CB; ++j) s_col[slot][wave][c0 + j] = part[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CB; ++j)
      out[j] = (s_col[slot][0][c0 + j] + s_col[slot][1][c0 + j]) + (s_col[slot][2][c0 + j] + s_col[slot][3][c0 + j]);
    slot ^= 1;                                     // the next call writes the other slot
  };
  // sum over the 16 column blocks (16 neighbouring lanes)
  auto rowsum = [&](float x) -> float {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
  };
  struct Tok {
    float q[RB], k[RB], a[RB], la[RB], v[CB], d[CB], beta;
  };
  auto load_tok = [&](int t, Tok& x, bool with_grad) {
    const size_t row_k = tok(t) * K, row_v = tok(t) * V;
    const Tv* qg = (const Tv*)p.q;
    const Tv* kg = (const Tv*)p.k;
    const Tv* vg = (const Tv*)p.v;
    const Tv* dg = (const Tv*)p.dout;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      x.k[i] = E::ld(kg, row_k + r0 + i);
      x.la[i] = p.log_alpha[row_k + r0 + i];
      x.a[i] = expf(x.la[i]);
      x.q[i] = with_grad ? E::ld(qg, row_k + r0 + i) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      x.v[j] = E::ld(vg, row_v + c0 + j);
      x.d[j] = with_grad ? E::ld(dg, row_v + c0 + j) : 0.f;
    }
    x.beta = p.beta[tok(t)];
  };
  // one forward token step on S (valid token)
  auto fwd_step = [&](const Tok& x) {
    float pp[CB], pred[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) pp[j] = 0.f;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        S[i][j] *= x.a[i];
        pp[j] += S[i][j] * x.k[i];
      }
    colsum(pp, pred);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float u = x.beta * (x.v[j] - pred[j]);
#pragma unroll
      for (int i = 0; i < RB; ++i) S[i][j] += x.k[i] * u;
    }
  };

  // ---- forward: checkpoint the state every kSeg tokens
  if (p.init_state != nullptr) load_block(p.init_state + (size_t)bh * K * V, S);
  else {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) S[i][j] = 0.f;
  }
  for (int t = 0; t < T; ++t) {
    if (t % kSeg == 0) store_block(ckpt + (size_t)(t / kSeg) * K * V, S);
    if (!valid(t)) continue;                       // uniform across the workgroup
    Tok x;
    load_tok(t, x, false);
    fwd_step(x);
  }

  // ---- backward, segment by segment
  if (p.dfinal != nullptr) load_block(p.dfinal + (size_t)bh * K * V, lam);
  else {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) lam[i][j] = 0.f;
  }
  for (int sg = p.nseg - 1; sg >= 0; --sg) {
    const int t0 = sg * kSeg, t1 = min(T, t0 + kSeg);
    // recompute the segment's states: segbuf[t - t0] = S_{t-1} (the state before token t)
    load_block(ckpt + (size_t)sg * K * V, S);
    for (int t = t0; t < t1; ++t) {
      store_block(segbuf + (size_t)(t - t0) * K * V, S);
      if (!valid(t)) continue;
      Tok x;
      load_tok(t, x, false);
      fwd_step(x);
    }
    __syncthreads();                               // (the stores above are read by this thread only)
    for (int t = t1 - 1; t >= t0; --t) {
      const size_t row_k = tok(t) * K, row_v = tok(t) * V;
      if (!valid(t)) {                             // zero gradients; lam passes through
        if (cb == 0) {
#pragma unroll
          for (int i = 0; i < RB; ++i) { p.dq[row_k + r0 + i] = 0.f; p.dk[row_k + r0 + i] = 0.f; p.dla[row_k + r0 + i] = 0.f; }
        }
        if (rb == 0) {
#pragma unroll
          for (int j = 0; j < CB; ++j) p.dv[row_v + c0 + j] = 0.f;
        }
        if (tid == 0) p.dbeta[tok(t)] = 0.f;
        continue;
      }
      Tok x;
      load_tok(t, x, true);
      float Sp[RB][CB];
      load_block(segbuf + (size_t)(t - t0) * K * V, Sp);
      float pp[CB], pred[CB], r[CB], u[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) pp[j] = 0.f;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          Sp[i][j] *= x.a[i];
          pp[j] += Sp[i][j] * x.k[i];
        }
      colsum(pp, pred);
#pragma unroll
      for (int j = 0; j < CB; ++j) { r[j] = x.v[j] - pred[j]; u[j] = x.beta * r[j]; }
      // L = lam + q do^T; dq = S_t do; du = L^T k
      float dup[CB], du[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) dup[j] = 0.f;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        float dqp = 0.f;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          lam[i][j] += x.q[i] * x.d[j];
          dqp += (Sp[i][j] + x.k[i] * u[j]) * x.d[j];
          dup[j] += lam[i][j] * x.k[i];
        }
        const float dq = rowsum(dqp);
        if (cb == 0) p.dq[row_k + r0 + i] = dq;
      }
      colsum(dup, du);
      // dbeta = du . r over all columns (the row-block-0 threads hold each column once)
      float dbp = 0.f;
#pragma unroll
      for (int j = 0; j < CB; ++j) dbp += du[j] * r[j];
      dbp = rowsum(dbp);
      if (tid == 0) p.dbeta[tok(t)] = dbp;
      float dr[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) dr[j] = x.beta * du[j];
      if (rb == 0) {
#pragma unroll
        for (int j = 0; j < CB; ++j) p.dv[row_v + c0 + j] = dr[j];
      }
      // dk = L u - S' dr;  dS' = L - k dr^T;  dlog_alpha = rowsum(dS' * S');  lam = a dS'
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        float dkp = 0.f, dlp = 0.f;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          dkp += lam[i][j] * u[j] - Sp[i][j] * dr[j];
          const float dsp = lam[i][j] - x.k[i] * dr[j];
          dlp += dsp * Sp[i][j];
          lam[i][j] = x.a[i] * dsp;
        }
        const float dk = rowsum(dkp), dl = rowsum(dlp);
        if (cb == 0) {
          p.dk[row_k + r0 + i] = dk;
          p.dla[row_k + r0 + i] = dl;
        }
      }
    }
    __syncthreads();                               // segbuf is rewritten by the next segment
  }
  store_block(p.dinit + (size_t)bh * K * V, lam);
}

template <int DT, int K, int V>
static hipError_t launch_bwd_t(const BwdParams& bp, hipStream_t st) {
  hipLaunchKernelGGL((backward_kernel<DT, K, V>), dim3(bp.B * bp.H), dim3(kBwdThreads), 0, st, bp);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_bwd_dt(const BwdParams& bp, hipStream_t st) {
#define KDA_BWD(KK, VV) \
  if (bp.dk_ == KK && bp.dv_ == VV) return launch_bwd_t<DT, KK, VV>(bp, st);
  KDA_BWD(16, 16) KDA_BWD(16, 32) KDA_BWD(16, 64) KDA_BWD(16, 128)
  KDA_BWD(32, 16) KDA_BWD(32, 32) KDA_BWD(32, 64) KDA_BWD(32, 128)
  KDA_BWD(64, 16) KDA_BWD(64, 32) KDA_BWD(64, 64) KDA_BWD(64, 128)
  KDA_BWD(128, 16) KDA_BWD(128, 32) KDA_BWD(128, 64) KDA_BWD(128, 128)
#undef KDA_BWD
  return hipErrorInvalidValue;
}

hipError_t launch_backward(const BackwardArgs& a) {
  BwdParams bp{a.q, a.k, a.v, a.dout, a.log_alpha, a.beta, a.init_state, a.dfinal, a.mask,
               a.dq, a.dk, a.dv, a.dla, a.dbeta, a.dinit, (float*)a.workspace,
               a.B, a.T, a.H, a.dk_, a.dv_, a.T > 0 ? (a.T + kSeg - 1) / kSeg : 0};
  hipStream_t st = (hipStream_t)a.stream;
  return a.dtype == 0 ? launch_bwd_dt<0>(bp, st) : launch_bwd_dt<1>(bp, st);
}

}  // namespace kda
