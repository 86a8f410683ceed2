// Per-call preparation for the float32 conv kernel, in one launch:
//
// 1. BN fold (POPCORNBENCH "Kimi-K2.6__l2_p12", first turn: eval-mode BN per channel,
//    with the inverse standard deviation precomputed once per channel as on that page):
//      scale[c] = gamma[c] / sqrt(running_var[c] + eps)
//      shift[c] = beta[c] - running_mean[c] * scale[c]
//    computed in double and rounded once to float, so the staged activation is
//    ReLU(fma(x, scale, shift)). Channels in [C_in, Cin_pad) get scale = shift = 0.
//    With gamma null (the caller normalised already) scale = 1 and shift = 0, so the
//    stage computes ReLU(x) exactly; with scale null the fold is skipped.
//
// 2. Weight repack from PyTorch's [C_out][C_in][3] into the register order of the MFMA
//    A operand (the first page's design turn proposes a transposed weight layout so the
//    output-channel loop is contiguous; this goes one step further, to lane order).
//    Index, in 16-byte units:   (G*NCB + cb)*64 + lane
//      G    = 2*q + g     16-row group g (0, 1) of K-chunk q = 3*c + k
//                         (input-channel block c of 32 channels, tap k)
//      cb   = 0..NCB-1    block of 16 output channels
//      lane = 0..63       co = 16*cb + lane%16, rows 16g + 4*(lane/16) + u, u = 0..3
//    and the 4 floats of the unit are u = 0..3:
//      Wp[unit][u] = W[co][32c + 16g + 4*(lane/16) + u][k]   (0 outside C_out x C_in).
//    A wave of the conv kernel then loads 1 KB contiguous per (G, cb) and each lane
//    holds its A values for four consecutive MFMA steps.

#include "internal.h"

namespace dconv1d {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Step 1 for channel idx (every launch covers [0, Cin_pad) with its first threads).
__device__ __forceinline__ void fold_bn(int idx, int C_in, int Cin_pad,
                                        const float* __restrict__ mean,
                                        const float* __restrict__ var,
                                        const float* __restrict__ gamma,
                                        const float* __restrict__ beta, float eps,
                                        float* __restrict__ scale, float* __restrict__ shift) {
  if (scale != nullptr && idx < Cin_pad) {
    float sc = 0.f, sh = 0.f;
    if (idx < C_in && gamma == nullptr) {
      sc = 1.f;                          // no normalisation: the stage applies ReLU only
    } else if (idx < C_in) {
      const double s = (double)gamma[idx] / sqrt((double)var[idx] + (double)eps);
      sc = (float)s;
      sh = (float)((double)beta[idx] - (double)mean[idx] * s);
    }
    scale[idx] = sc;
    shift[idx] = sh;
  }
}

__global__ void __launch_bounds__(256)
prep_f32_kernel(const float* __restrict__ W, int C_out, int C_in, int NCB, int total4,
                f32x4* __restrict__ Wp, const float* __restrict__ mean,
                const float* __restrict__ var, const float* __restrict__ gamma,
                const float* __restrict__ beta, float eps, float* __restrict__ scale,
                float* __restrict__ shift, int Cin_pad) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < total4) {
    const int lane = idx & 63;
    int rest = idx >> 6;
    const int cb = rest % NCB;          // 16-channel block
    const int G = rest / NCB;           // 16-row group: chunk G/2, half G%2
    const int q = G >> 1, g = G & 1;
    const int c = q / 3, k = q - 3 * c;
    const int co = 16 * cb + (lane & 15);
    const int ci0 = 32 * c + 16 * g + 4 * (lane >> 4);
    f32x4 v;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ci = ci0 + u;
      v[u] = (co < C_out && ci < C_in) ? W[((size_t)co * C_in + ci) * 3 + k] : 0.f;
    }
    Wp[idx] = v;
  }
  fold_bn(idx, C_in, Cin_pad, mean, var, gamma, beta, eps, scale, shift);
}

hipError_t launch_prep_f32(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                           float* Wp, const float* running_mean, const float* running_var,
                           const float* gamma, const float* beta, float eps, float* scale,
                           float* shift, hipStream_t stream) {
  const int NCB = Cout_pad / 16;
  const long long total4 = 3LL * Cin_pad * Cout_pad / 4;
  const long long threads = total4 > Cin_pad ? total4 : Cin_pad;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(prep_f32_kernel, dim3(blocks), dim3(256), 0, stream, W, C_out, C_in, NCB,
                     (int)total4, reinterpret_cast<f32x4*>(Wp), running_mean, running_var,
                     gamma, beta, eps, scale, shift, Cin_pad);
  return hipGetLastError();
}

// Weight transform of the Winograd F(2,3) kernel (conv_wino.hip) with step 1 in the same
// launch. For taps g0, g1, g2 = W[co][ci][0..2] the four transformed weights are
//   U0 = g0,  U1 = (g0 + g1 + g2) / 2,  U2 = (g0 - g1 + g2) / 2,  U3 = g2
// (in double, rounded once). Index, in 16-byte units:   (S*NCB + cb)*64 + lane
//   S    = 8*q + s     MFMA step s (0..7) of K-chunk q (input channels 32q .. 32q + 31)
//   cb   = 0..NCB-1    block of 16 output channels
//   lane = 0..63       co = 16*cb + lane%16, ci = 32q + 16*(s/4) + 4*(lane/16) + s%4
// and the 4 floats of the unit are U0..U3 of (co, ci), 0 outside C_out x C_in.
__global__ void __launch_bounds__(256)
prep_wino_kernel(const float* __restrict__ W, int C_out, int C_in, int NCB, int total4,
                 f32x4* __restrict__ Up, const float* __restrict__ mean,
                 const float* __restrict__ var, const float* __restrict__ gamma,
                 const float* __restrict__ beta, float eps, float* __restrict__ scale,
                 float* __restrict__ shift, int Cin_pad) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < total4) {
    const int lane = idx & 63;
    const int rest = idx >> 6;
    const int cb = rest % NCB;
    const int S = rest / NCB;
    const int q = S >> 3, s = S & 7;
    const int co = 16 * cb + (lane & 15);
    const int ci = 32 * q + 16 * (s >> 2) + 4 * (lane >> 4) + (s & 3);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (co < C_out && ci < C_in) {
      const float* g = W + ((size_t)co * C_in + ci) * 3;
      const double g0 = g[0], g1 = g[1], g2 = g[2];
      v[0] = (float)g0;
      v[1] = (float)(0.5 * (g0 + g1 + g2));
      v[2] = (float)(0.5 * (g0 - g1 + g2));
      v[3] = (float)g2;
    }
    Up[idx] = v;
  }
  fold_bn(idx, C_in, Cin_pad, mean, var, gamma, beta, eps, scale, shift);
}

hipError_t launch_prep_wino(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                            float* Up, const float* running_mean, const float* running_var,
                            const float* gamma, const float* beta, float eps, float* scale,
                            float* shift, hipStream_t stream) {
  const int NCB = Cout_pad / 16;
  const long long total4 = (long long)Cin_pad * Cout_pad;
  const long long threads = total4 > Cin_pad ? total4 : Cin_pad;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(prep_wino_kernel, dim3(blocks), dim3(256), 0, stream, W, C_out, C_in,
                     NCB, (int)total4, reinterpret_cast<f32x4*>(Up), running_mean,
                     running_var, gamma, beta, eps, scale, shift, Cin_pad);
  return hipGetLastError();
}

}  // namespace dconv1d
