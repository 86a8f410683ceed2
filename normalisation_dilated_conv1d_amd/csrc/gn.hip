// GroupNorm finalize + normalize (POPCORNBENCH "FW-GLM-5-1__l2_p35": its second kernel
// turns per-group sums into mean, biased variance and inverse standard deviation, then
// normalises the conv output in place and applies gamma/beta when present).
//
// Here the conv kernel has already written, per (sample n, channel co, time tile),
// the tile sum S, the tile-centred sum of squares M2 (two-pass inside the tile, in
// registers) and the tile's count of outputs (direct kernel: a run of time steps;
// Winograd kernel: the in-range outputs of its 32 output pairs). Each workgroup of this kernel first merges the partials of its (n, group)
// in a fixed order, in double precision:
//     mean = sum S / count
//     M2   = sum over tiles of [ M2_tile + cnt_tile * (S_tile/cnt_tile - mean)^2 ]
//     var  = M2 / count   (biased, as on the page),  rstd = 1/sqrt(var + eps)
// (the exact decomposition of the group's sum of squared deviations over its tiles, so
// no large-mean cancellation), and then rewrites its rows of the group as
//     out = y * (rstd*gamma) + (beta - mean*rstd*gamma).
// The merge is a fixed-shape tree (per-lane strided sums, then ds_swizzle butterflies
// inside each half-wave and one add across the halves), so results are bitwise
// reproducible from run to run.

#include "internal.h"

namespace dconv1d {

template <int XOR>
__device__ __forceinline__ double swz_xor_d(double v) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_ds_swizzle((int)(bits & 0xffffffffLL), (XOR << 10) | 0x1F);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(bits >> 32), (XOR << 10) | 0x1F);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over the 64 lanes of wave 0; the result is valid in every lane.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += swz_xor_d<16>(v);
  v += swz_xor_d<8>(v);
  v += swz_xor_d<4>(v);
  v += swz_xor_d<2>(v);
  v += swz_xor_d<1>(v);
  const long long bits = __double_as_longlong(v);
  const int lo0 = __builtin_amdgcn_readlane((int)(bits & 0xffffffffLL), 0);
  const int hi0 = __builtin_amdgcn_readlane((int)(bits >> 32), 0);
  const int lo1 = __builtin_amdgcn_readlane((int)(bits & 0xffffffffLL), 32);
  const int hi1 = __builtin_amdgcn_readlane((int)(bits >> 32), 32);
  const double a = __longlong_as_double(((long long)hi0 << 32) | (unsigned int)lo0);
  const double b = __longlong_as_double(((long long)hi1 << 32) | (unsigned int)lo1);
  return a + b;
}

constexpr int GN_MAX_ROWS = 256;

__global__ void __launch_bounds__(256)
gn_normalize_kernel(float* __restrict__ out, const float* __restrict__ partials,
                    const float* __restrict__ gamma, const float* __restrict__ beta, float eps,
                    int C_out, int L_out, int G, int n_tt, int rows_per_wg,
                    int chunks, int vec4) {
  const int ng = blockIdx.x / chunks;
  const int chunk = blockIdx.x - ng * chunks;
  const int n = ng / G, g = ng - (ng / G) * G;
  const int cpg = C_out / G;
  const int r_begin = chunk * rows_per_wg;
  const int r_end = min(cpg, r_begin + rows_per_wg);

  __shared__ float s_mul[GN_MAX_ROWS], s_add[GN_MAX_ROWS];

  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int P = cpg * n_tt;  // partial entries of this group, e = c_local*n_tt + tt
    const float* pp = partials + ((size_t)n * C_out + (size_t)g * cpg) * n_tt * 3;
    const double count = (double)cpg * (double)L_out;
    double s = 0.0;
    for (int e = lane; e < P; e += 64) s += (double)pp[3 * e];
    const double mean = wave_sum_d(s) / count;
    double m2 = 0.0;
    for (int e = lane; e < P; e += 64) {
      const double cnt = (double)pp[3 * e + 2];   // 0 for a tile with no output in range
      if (cnt > 0.0) {
        const double dm = (double)pp[3 * e] / cnt - mean;
        m2 += (double)pp[3 * e + 1] + cnt * dm * dm;
      }
    }
    const double var = wave_sum_d(m2) / count;
    const double rstd = 1.0 / sqrt(var + (double)eps);
    for (int r = r_begin + lane; r < r_end; r += 64) {
      const int co = g * cpg + r;
      const double ga = gamma ? (double)gamma[co] : 1.0;
      const double be = beta ? (double)beta[co] : 0.0;
      s_mul[r - r_begin] = (float)(rstd * ga);
      s_add[r - r_begin] = (float)(be - mean * rstd * ga);
    }
  }
  __syncthreads();

  float* base = out + ((size_t)n * C_out + (size_t)g * cpg + r_begin) * L_out;
  const int rows = r_end - r_begin;
  if (vec4) {
    // L_out % 4 == 0 and out is 16-byte aligned: every row is whole, aligned float4s
    const int q_per_row = L_out >> 2;
    const long long total = (long long)rows * q_per_row;
    float4* b4 = reinterpret_cast<float4*>(base);
    for (long long i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = (int)(i / q_per_row);
      const float m = s_mul[r], ad = s_add[r];
      float4 v = b4[i];
      v.x = fmaf(v.x, m, ad);
      v.y = fmaf(v.y, m, ad);
      v.z = fmaf(v.z, m, ad);
      v.w = fmaf(v.w, m, ad);
      b4[i] = v;
    }
  } else {
    const long long total = (long long)rows * L_out;
    for (long long i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = (int)(i / L_out);
      base[i] = fmaf(base[i], s_mul[r], s_add[r]);
    }
  }
}

hipError_t launch_gn_normalize(float* out, const float* partials, const float* gamma,
                               const float* beta, float eps, int N, int C_out, int L_out,
                               int num_groups, int n_tt, hipStream_t stream) {
  const int cpg = C_out / num_groups;
  int rows = 8192 / L_out;
  if (rows < 1) rows = 1;
  if (rows > cpg) rows = cpg;
  if (rows > GN_MAX_ROWS) rows = GN_MAX_ROWS;
  const int chunks = (cpg + rows - 1) / rows;
  const long long nwg = (long long)N * num_groups * chunks;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gn_normalize_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, out,
                     partials, gamma, beta, eps, C_out, L_out, num_groups, n_tt, rows,
                     chunks, (int)(((L_out & 3) == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0)));
  return hipGetLastError();
}

}  // namespace dconv1d
