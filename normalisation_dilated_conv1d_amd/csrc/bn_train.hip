// BatchNorm1d in training mode for the pre-norm block: the batch statistics of x per
// channel over (N, L), folded into the same scale/shift the conv kernels read, plus the
// running-statistics update.
//
// Semantics (POPCORNBENCH "Kimi-K2.6__l2_p97", first turn; "Kimi-K2.6__l2_p12",
// correctness-debugging turn): normalise with the batch mean and the biased batch
// variance (divide by n = N*L); update
//   running_mean <- (1 - momentum)*running_mean + momentum*mean
//   running_var  <- (1 - momentum)*running_var  + momentum*var*n/(n - 1).
//
// Two kernels, both deterministic (fixed reduction order for a given shape):
//
// 1. bn_stats_kernel: one workgroup per (n, c, segment of up to STAT_SEG time steps),
//    in memory order so consecutive workgroups stream consecutive rows of x. Every
//    element is taken in double as (x - K), with K = x[0][c][0] a per-channel shift,
//    and the workgroup writes its (sum, sum of squares) pair, reduced by a fixed
//    butterfly, to partials[c][n*n_seg + s]. The shift keeps the one-pass variance
//    free of cancellation when |mean| >> std.
// 2. bn_finalize_kernel: one wave per channel merges its P partials (lane-strided
//    sums, then a fixed butterfly), forms mean = K + S/n and var = Q/n - (S/n)^2,
//    and writes scale = gamma/sqrt(var+eps), shift = beta - mean*scale (double,
//    rounded once, zero for padded channels), the running update and, when asked,
//    the batch mean and 1/sqrt(var+eps).
//
// HBM: the statistics pass reads x once (the conv then reads it again); it is bound by
// that read.

#include "internal.h"

namespace dconv1d {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double to_double(float v) { return (double)v; }
__device__ __forceinline__ double to_double(uint16_t v) {
  return (double)__uint_as_float((uint32_t)v << 16);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Reduces (s, q) over the 256 threads in a fixed order; thread 0 gets the result.
__device__ __forceinline__ void block_sum2(double& s, double& q) {
  __shared__ double red[2][4];
  s = wave_sum(s);
  q = wave_sum(q);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = s;
    red[1][w] = q;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    s = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    q = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// VEC: every row starts 16-byte aligned and L is a multiple of the elements per 16 bytes
template <typename XT, bool VEC>
__global__ void __launch_bounds__(256)
bn_stats_kernel(const XT* __restrict__ x, int C, int L, int n_seg, int P,
                double2* __restrict__ partials) {
  constexpr int EPV = 16 / sizeof(XT);                 // elements per 16-byte load
  constexpr int ITERS = STAT_SEG / (256 * (VEC ? EPV : 1));
  const long long b = blockIdx.x;                      // ((n*C + c)*n_seg + s)
  const int s = (int)(b % n_seg);
  const long long row = b / n_seg;                     // n*C + c
  const int c = (int)(row % C);
  const int n = (int)(row / C);
  const XT* xr = x + row * (long long)L;
  const double K = to_double(x[(size_t)c * L]);        // x[0][c][0]
  const int t0 = s * STAT_SEG;
  const int t1 = min(L, t0 + STAT_SEG);
  double sum = 0.0, sq = 0.0;
  if constexpr (VEC) {
    typedef typename std::conditional<sizeof(XT) == 4, f32x4, u32x4>::type V;
    V v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int t = t0 + EPV * (threadIdx.x + 256 * i);
      if (t < t1) v[i] = *reinterpret_cast<const V*>(xr + t);
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int t = t0 + EPV * (threadIdx.x + 256 * i);
      if (t < t1) {
        if constexpr (sizeof(XT) == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const double dv = (double)v[i][e] - K;
            sum += dv;
            sq = fma(dv, dv, sq);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const double lo = (double)__uint_as_float(v[i][e] << 16) - K;
            const double hi = (double)__uint_as_float(v[i][e] & 0xffff0000u) - K;
            sum += lo;
            sq = fma(lo, lo, sq);
            sum += hi;
            sq = fma(hi, hi, sq);
          }
        }
      }
    }
  } else {
    XT v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int t = t0 + threadIdx.x + 256 * i;
      if (t < t1) v[i] = xr[t];
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int t = t0 + threadIdx.x + 256 * i;
      if (t < t1) {
        const double dv = to_double(v[i]) - K;
        sum += dv;
        sq = fma(dv, dv, sq);
      }
    }
  }
  block_sum2(sum, sq);
  if (threadIdx.x == 0) partials[(size_t)c * P + (size_t)n * n_seg + s] = make_double2(sum, sq);
}

template <typename XT>
__global__ void __launch_bounds__(256)
bn_finalize_kernel(const XT* __restrict__ x, int C, int L, int Cin_pad,
                   const double2* __restrict__ partials, int P, double count,
                   const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                   float momentum, float* __restrict__ running_mean,
                   float* __restrict__ running_var, float* __restrict__ save_mean,
                   float* __restrict__ save_invstd, float* __restrict__ scale,
                   float* __restrict__ shift) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= Cin_pad) return;                            // uniform per wave
  if (c >= C) {
    if (lane == 0) {
      scale[c] = 0.f;
      shift[c] = 0.f;
    }
    return;
  }
  double s = 0.0, q = 0.0;
  const double2* pc = partials + (size_t)c * P;
  for (int j = lane; j < P; j += 64) {
    const double2 v = pc[j];
    s += v.x;
    q += v.y;
  }
  s = wave_sum(s);
  q = wave_sum(q);
  if (lane != 0) return;
  const double K = to_double(x[(size_t)c * L]);
  const double m1 = s / count;                         // mean of x - K
  const double mean = K + m1;
  const double var = fmax(q / count - m1 * m1, 0.0);   // biased
  const double inv = 1.0 / sqrt(var + (double)eps);
  const double sc = (double)gamma[c] * inv;
  scale[c] = (float)sc;
  shift[c] = (float)((double)beta[c] - mean * sc);
  if (running_mean != nullptr) {
    const double m = (double)momentum;
    running_mean[c] = (float)((1.0 - m) * (double)running_mean[c] + m * mean);
    running_var[c] =
        (float)((1.0 - m) * (double)running_var[c] + m * var * count / (count - 1.0));
  }
  if (save_mean != nullptr) save_mean[c] = (float)mean;
  if (save_invstd != nullptr) save_invstd[c] = (float)inv;
}

template <typename XT>
hipError_t launch_bn_train_impl(const XT* x, int N, int C, int L, int Cin_pad,
                                double2* partials, const float* gamma, const float* beta,
                                float eps, float momentum, float* running_mean,
                                float* running_var, float* save_mean, float* save_invstd,
                                float* scale, float* shift, hipStream_t stream) {
  const int n_seg = (L + STAT_SEG - 1) / STAT_SEG;
  const int P = N * n_seg;
  const long long nwg = (long long)N * C * n_seg;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  constexpr int EPV = 16 / sizeof(XT);
  const bool vec = L % EPV == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((bn_stats_kernel<XT, true>), dim3((unsigned)nwg), dim3(256), 0, stream, x,
                       C, L, n_seg, P, partials);
  else
    hipLaunchKernelGGL((bn_stats_kernel<XT, false>), dim3((unsigned)nwg), dim3(256), 0, stream,
                       x, C, L, n_seg, P, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const double count = (double)N * (double)L;
  hipLaunchKernelGGL(bn_finalize_kernel<XT>, dim3((Cin_pad + 3) / 4), dim3(256), 0, stream, x, C,
                     L, Cin_pad, partials, P, count, gamma, beta, eps, momentum, running_mean,
                     running_var, save_mean, save_invstd, scale, shift);
  return hipGetLastError();
}

}  // namespace

size_t bn_train_partials_bytes(int N, int C, int L) {
  return sizeof(double2) * (size_t)C * N * ((L + STAT_SEG - 1) / STAT_SEG);
}

hipError_t launch_bn_train(const void* x, bool bf16, int N, int C, int L, int Cin_pad,
                           void* partials, const float* gamma, const float* beta, float eps,
                           float momentum, float* running_mean, float* running_var,
                           float* save_mean, float* save_invstd, float* scale, float* shift,
                           hipStream_t stream) {
  double2* p = static_cast<double2*>(partials);
  if (bf16)
    return launch_bn_train_impl(static_cast<const uint16_t*>(x), N, C, L, Cin_pad, p, gamma, beta,
                                eps, momentum, running_mean, running_var, save_mean, save_invstd,
                                scale, shift, stream);
  return launch_bn_train_impl(static_cast<const float*>(x), N, C, L, Cin_pad, p, gamma, beta, eps,
                              momentum, running_mean, running_var, save_mean, save_invstd, scale,
                              shift, stream);
}

}  // namespace dconv1d
