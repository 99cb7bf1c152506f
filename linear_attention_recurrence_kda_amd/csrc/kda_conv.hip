// Masked depthwise causal short convolution with a conv cache (Transformers
// issue report on Kimi Linear cached continuation: padded entries entering the
// convolution window were one of the two causes of the state defect, so the
// taps here run over the compacted sequence of valid positions only).
//
// For sequence b and channel c, x~ = [cache[b,0..W-2,c], x at the valid
// positions of b in order]; the m-th valid position gets
//   y = bias[c] + sum_j w[c,j] * x~[m + j]      (w[c,W-1] on the current input)
// and masked positions get y = 0.  The new cache is the last W-1 entries of x~.
//
// Two launches on the caller's stream: conv_y_kernel reads the old cache,
// conv_cache_kernel then overwrites it (stream order separates the two).  When the
// whole sequence is one token segment (decode: T = 1), the thread that forms y for a
// channel group has read that group's old cache before anything else and ends holding
// the new one, so it writes the cache itself and the second launch is skipped.
// Each thread owns 8 consecutive channels (one 16-byte bf16 vector) and a
// segment of tokens; the segment's window history (the last W-1 valid positions before
// it) is found once per workgroup by a parallel search back over the mask.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kConvThreads = 256;
constexpr int kConvSeg = 32;   // tokens per thread

__device__ __forceinline__ bool conv_valid(const uint8_t* mask, int b, int T, int t) {
  return mask == nullptr || mask[(size_t)b * T + t] != 0;
}

// The last W-1 valid positions before t_before, newest first, into s_pos[0 .. W-2] (-1
// where fewer exist: those entries come from the cache).  Found by the whole workgroup at
// once: each pass looks at the 16 x 256 positions below the previous pass, every thread
// taking 16 consecutive ones, and a block prefix count over the threads (highest
// positions first) gives each valid position its rank.  A pad of any length costs
// pad / 4096 passes, not a walk per thread.  Every thread of the block must call this.
template <int W>
__device__ void find_history(const uint8_t* __restrict__ mask, int b, int T, int t_before, int* s_pos,
                             int* s_wsum) {
  constexpr int kSpan = 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kWaves = kConvThreads / 64;
  if (mask == nullptr) {                 // every position valid
    if (tid < W - 1) s_pos[tid] = t_before - 1 - tid >= 0 ? t_before - 1 - tid : -1;
    __syncthreads();
    return;
  }
  if (tid < W - 1) s_pos[tid] = -1;
  __syncthreads();
  const uint8_t* mrow = mask + (size_t)b * T;
  int need = W - 1, hi = t_before - 1;   // the same in every thread
  while (need > 0 && hi >= 0) {
    const int top = hi - kSpan * tid;
    unsigned bits = 0;                   // bit j: position top - j is valid
#pragma unroll
    for (int j = 0; j < kSpan; ++j) {
      const int t = top - j;
      if (t >= 0 && mrow[t] != 0) bits |= 1u << j;
    }
    const int cnt = __popc(bits);
    int x = cnt;                         // inclusive prefix count inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = s_wsum[w];
      before += w < wave ? v : 0;
      total += v;
    }
    int r = before + x - cnt;            // rank of this thread's highest valid position
    const int base = (W - 1) - need;
    for (int j = 0; j < kSpan && r < need; ++j) {
      if ((bits >> j) & 1u) {
        s_pos[base + r] = top - j;
        ++r;
      }
    }
    __syncthreads();
    need -= total < need ? total : need;
    hi -= kSpan * kConvThreads;
  }
}

// History entries preceding a segment: hist[0] oldest ... hist[W-2] newest, from the
// positions find_history left in s_pos, then from the cache (newest cache entry first),
// then zeros.
template <int DT, int W>
__device__ __forceinline__ void load_history(const typename Elem<DT>::T* x, const typename Elem<DT>::T* cache,
                                             const int* s_pos, int b, int T, int D, int c0,
                                             float (&hist)[W > 1 ? W - 1 : 1][8]) {
  using E = Elem<DT>;
  int used_cache = 0;
#pragma unroll
  for (int s = 0; s < W - 1; ++s) {
    const int t = s_pos[s];
    if (t >= 0) {
      E::ld8(x, ((size_t)b * T + t) * D + c0, hist[W - 2 - s]);
    } else if (cache != nullptr) {
      E::ld8(cache, ((size_t)b * (W - 1) + (W - 2 - used_cache)) * D + c0, hist[W - 2 - s]);
      ++used_cache;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) hist[W - 2 - s][i] = 0.f;
    }
  }
}

template <int DT, int W>
__global__ void __launch_bounds__(kConvThreads)
conv_y_kernel(const typename Elem<DT>::T* __restrict__ x, const float* __restrict__ w,
              const float* __restrict__ bias, const uint8_t* __restrict__ mask,
              typename Elem<DT>::T* __restrict__ cache, typename Elem<DT>::T* __restrict__ y,
              int T, int D, int silu, int write_cache) {
  using E = Elem<DT>;
  __shared__ int s_pos[W > 1 ? W - 1 : 1];
  __shared__ int s_wsum[kConvThreads / 64];
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * 8;
  const bool active = c0 < D;            // inactive threads still join the block's search
  const int b = blockIdx.z;
  const int t_start = blockIdx.y * kConvSeg;
  const int t_end = min(T, t_start + kConvSeg);

  // a segment with no valid position writes zeros and needs no history (unless it is the
  // whole sequence and writes the cache, which then keeps its contents)
  const bool any_valid = __syncthreads_or(threadIdx.x < t_end - t_start && conv_valid(mask, b, T, t_start + threadIdx.x));
  if (!any_valid && !write_cache) {
    if (active) {
      float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int t = t_start; t < t_end; ++t) E::st8(y, ((size_t)b * T + t) * D + c0, zero);
    }
    return;
  }
  find_history<W>(mask, b, T, t_start, s_pos, s_wsum);
  if (!active) return;

  float wt[8][W], bs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) wt[i][j] = w[(size_t)(c0 + i) * W + j];
    bs[i] = bias != nullptr ? bias[c0 + i] : 0.f;
  }
  float hist[W > 1 ? W - 1 : 1][8];
  load_history<DT, W>(x, cache, s_pos, b, T, D, c0, hist);

  for (int t = t_start; t < t_end; ++t) {
    const size_t off = ((size_t)b * T + t) * D + c0;
    float out[8];
    if (conv_valid(mask, b, T, t)) {
      float xt[8];
      E::ld8(x, off, xt);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float acc = bs[i];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) acc += wt[i][j] * hist[j][i];
        acc += wt[i][W - 1] * xt[i];
        if (silu) acc = acc / (1.0f + __expf(-acc));
        out[i] = acc;
      }
#pragma unroll
      for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) hist[j][i] = hist[j + 1][i];
      if (W > 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) hist[W > 1 ? W - 2 : 0][i] = xt[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = 0.f;
    }
    E::st8(y, off, out);
  }
  if (write_cache) {                     // one segment from t = 0: hist is the new cache
#pragma unroll
    for (int j = 0; j < W - 1; ++j) E::st8(cache, ((size_t)b * (W - 1) + j) * D + c0, hist[j]);
  }
}

template <int DT, int W>
__global__ void __launch_bounds__(kConvThreads)
conv_cache_kernel(const typename Elem<DT>::T* __restrict__ x, const uint8_t* __restrict__ mask,
                  typename Elem<DT>::T* __restrict__ cache, int T, int D) {
  __shared__ int s_pos[W > 1 ? W - 1 : 1];
  __shared__ int s_wsum[kConvThreads / 64];
  using E = Elem<DT>;
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * 8;
  const int b = blockIdx.z;
  find_history<W>(mask, b, T, T, s_pos, s_wsum);
  if (c0 >= D) return;
  float hist[W > 1 ? W - 1 : 1][8];
  load_history<DT, W>(x, cache, s_pos, b, T, D, c0, hist);     // reads the old cache first
#pragma unroll
  for (int j = 0; j < W - 1; ++j) E::st8(cache, ((size_t)b * (W - 1) + j) * D + c0, hist[j]);
}

template <int DT, int W>
static hipError_t launch_conv_t(const ConvArgs& a) {
  using T = typename Elem<DT>::T;
  if (a.B == 0 || a.T == 0) return hipSuccess;
  const int cblocks = (a.D / 8 + kConvThreads - 1) / kConvThreads;
  const int segs = (a.T + kConvSeg - 1) / kConvSeg;
  hipStream_t st = (hipStream_t)a.stream;
  const int fused = (segs == 1 && a.cache != nullptr) ? 1 : 0;
  hipLaunchKernelGGL((conv_y_kernel<DT, W>), dim3(cblocks, segs, a.B), dim3(kConvThreads), 0, st,
                     (const T*)a.x, a.weight, a.bias, a.mask, (T*)a.cache, (T*)a.y, a.T, a.D, a.silu, fused);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.cache == nullptr || fused) return e;
  hipLaunchKernelGGL((conv_cache_kernel<DT, W>), dim3(cblocks, 1, a.B), dim3(kConvThreads), 0, st,
                     (const T*)a.x, a.mask, (T*)a.cache, a.T, a.D);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_conv_dt(const ConvArgs& a) {
  switch (a.W) {
    case 2: return launch_conv_t<DT, 2>(a);
    case 3: return launch_conv_t<DT, 3>(a);
    case 4: return launch_conv_t<DT, 4>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_short_conv(const ConvArgs& a) {
  return a.dtype == 0 ? launch_conv_dt<0>(a) : launch_conv_dt<1>(a);
}

}  // namespace kda
