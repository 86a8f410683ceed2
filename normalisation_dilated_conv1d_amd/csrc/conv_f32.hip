// Float32 implicit-GEMM kernel for a kernel-3, stride-1 Conv1d on MI355X (gfx950).
//
// It serves both operations of the library:
//   * the pre-norm residual block (POPCORNBENCH "Kimi-K2.6__l2_p12", first turn): each
//     conv input value is ReLU(BN_eval(x)) applied while the tile is staged, padded taps
//     are exact zeros, and the epilogue adds the conv bias and the raw x residual;
//   * Conv1d + GroupNorm (POPCORNBENCH "FW-GLM-5-1__l2_p35"): the staged value is x
//     itself, and the epilogue stores the conv output together with per-channel tile
//     statistics for the GroupNorm pass.
//
// GEMM view (the three-tap decomposition of the first page's design turn): for one
// sample, out[co][t] = sum over K = (tap k, input channel ci) of
// W[co][ci][k] * z[ci][t - pad + k*dil], i.e. M = C_out, N = time, K = 3*C_in.
//
// Work split
//   workgroup  = one sample n, 64*MB output channels (co tile: 256, 128 or 64), TT time
//                steps (t tile: 128 or 64); 4 waves, wave w owns output channels
//                [16*MB*w, 16*MB*(w+1)) of the co tile and all TT time steps: MB x (TT/16)
//                MFMA 16x16 accumulator blocks.
//   K loop     = chunks of 32 input channels of one tap, ordered (ci-block, tap) so
//                that the three taps of a channel block are staged back to back and hit
//                the same L2 lines.
//   B operand  = the activation tile z[32][TT], staged through LDS once per chunk by
//                all 256 threads (global loads coalesced along t, BN+ReLU applied in
//                registers as one med3, zero outside [0, L_in)), double-buffered, one
//                barrier per chunk; the staging of chunk q+1 runs in the middle of chunk
//                q's MFMAs.
//   A operand  = the weights, read straight from global memory into registers: the
//                repack kernel stores them in the exact lane order of the MFMA A operand,
//                so each lane fetches 4 consecutive K values with one 16-byte load and
//                each wave reads 1 KB contiguous per load. No LDS for W: no two waves of
//                a workgroup use the same weights.
//   MFMA       = v_mfma_f32_16x16x4_f32 (full float32 products and accumulation). On
//                MI355X it sustains a higher clock under load than the 32x32x2 form
//                (measured ~155 vs ~145 TFLOP/s in a register-only loop).
//   Occupancy  = at most 256 VGPRs, so two workgroups share each CU (two waves per
//                SIMD) and hide each other's barriers, staging and epilogue.
//
// K permutation inside a chunk: the 32 rows r of a chunk are split as r = 16g + 4q + u
// (g: two 16-row groups, q = lane/16: the lane's quarter-wave, u: 4 steps). MFMA step
// (g, u) gives quarter-wave q row 16g + 4q + u as its K value, so a lane's four A
// values for steps u = 0..3 are contiguous in the repacked weights. A and B use the
// same permutation, so the sum over K is unchanged.
//
// Workgroup order is XCD-aware: the hardware sends workgroup b to XCD b % 8, so the
// logical tile index is remapped to give every XCD one contiguous range of tiles; the
// neighbouring time tiles whose tap windows overlap then share that XCD's L2.

#include "internal.h"

namespace dconv1d {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Sum over the 16 lanes of each quarter-wave with ds_swizzle butterflies (xor 8..1).
// Every lane ends with the same, order-fixed value.
template <int XOR>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (XOR << 10) | 0x1F));
}
__device__ __forceinline__ float quarterwave_sum(float v) {
  v += swz_xor<8>(v);
  v += swz_xor<4>(v);
  v += swz_xor<2>(v);
  v += swz_xor<1>(v);
  return v;
}

// Storage type hooks (the kernel is instantiated for float storage).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ void from_f32(float v, float* dst) { *dst = v; }

template <int TT, int MB, bool BN, int EPI, typename XT>
__global__ void __launch_bounds__(NTHREADS, 2)
conv_f32_kernel(ConvF32Args a) {
  constexpr int CO_TILE = 4 * 16 * MB;           // output channels per workgroup
  constexpr int NB = TT / 16;                    // 16-column MFMA blocks per wave
  constexpr int NQ = NB / 4;                     // 16-byte LDS reads per MFMA step
  constexpr int CPT = TT / 64;                   // staged columns per thread
  constexpr int RPW = KC / 4;                    // staged rows per wave (8)
  constexpr int XPT = RPW * CPT;                 // staged values per thread per chunk
  // LDS row layout: within each 64-column quarter, column c lives at
  // (c % 16) * 4 + (c % 64) / 16, so lane l reads its 4 B values (columns l%16 + 16*nb)
  // with one 16-byte load and the 16 lanes of a quarter-wave read 256 contiguous bytes.
  constexpr int PITCH = TT + 4;
  __shared__ __attribute__((aligned(16))) float zs[2][KC * PITCH];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lq = l >> 4;     // quarter-wave: selects the K row inside an MFMA step
  const int l16 = l & 15;

  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = b & 7;
  const int logical = xcd * per + min(xcd, rem) + (b >> 3);
  // the tile indices are wave-uniform: readfirstlane keeps them (and the addresses
  // derived from them, such as the buffer resource of x) in scalar registers
  const int ct = __builtin_amdgcn_readfirstlane(logical % a.n_ct);
  const int rest = logical / a.n_ct;
  const int tt = __builtin_amdgcn_readfirstlane(rest % a.n_tt);
  const int n = __builtin_amdgcn_readfirstlane(rest / a.n_tt);
  const int t0 = tt * TT;

  const XT* __restrict__ xn = reinterpret_cast<const XT*>(a.x) + (size_t)n * a.C_in * a.L_in;
  const f32x4* __restrict__ Wp4 = reinterpret_cast<const f32x4*>(a.Wp);
  const int cb0 = (ct * CO_TILE) / 16 + MB * w;   // first 16-channel block of the wave

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][nb][r] = 0.f;

  float xr[XPT];
  float sc[RPW], sh[RPW];

  auto load_x = [&](int q) {
    const int c = q / 3, k = q - 3 * c;
    const int off = k * a.dil - a.pad;
    // a row's base address is wave-uniform (scalar registers) and a lane's byte offset
    // inside the row is one 32-bit register per column block (L_in < 2^30)
    uint32_t boff[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      // a padded tap may read any in-range step: store_z masks it to zero
      const uint32_t ts = tap_step(t0 + l + 64 * j, off);
      boff[j] = (ts < (uint32_t)a.L_in ? ts : 0u) * (uint32_t)sizeof(XT);
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int ci = min(c * KC + RPW * w + i, a.C_in - 1);
      const char* rowp = reinterpret_cast<const char*>(xn + (size_t)ci * a.L_in);
#pragma unroll
      for (int j = 0; j < CPT; ++j)
        xr[i * CPT + j] = to_f32(*reinterpret_cast<const XT*>(rowp + boff[j]));
    }
    if (BN) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        sc[i] = a.scale[c * KC + RPW * w + i];
        sh[i] = a.shift[c * KC + RPW * w + i];
      }
    }
  };
  auto store_z = [&](int q, float* dst) {
    const int c = q / 3, k = q - 3 * c;
    const int off = k * a.dil - a.pad;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int col = l + 64 * j;
      const bool in_tap = tap_step(t0 + col, off) < (uint32_t)a.L_in;
      // With BN the staged value is med3(fma(x, scale, shift), 0, cap), cap = +inf inside
      // the input and 0 on a padded tap: ReLU in one instruction, and an exact zero for
      // padding. Without BN the value is x AND a mask. Both stay opaque to the optimiser.
      uint32_t tkeep = in_tap ? 0xffffffffu : 0u;
      float cap = in_tap ? __builtin_huge_valf() : 0.f;
      asm volatile("" : "+v"(tkeep), "+v"(cap));
      const int pos = 64 * j + (col & 15) * 4 + ((col & 63) >> 4);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int row = RPW * w + i;
        const float v = xr[i * CPT + j];
        if (BN) {
          // a padded input channel has scale = shift = 0 (every fold writes that), so its
          // value is med3(fma(x, 0, 0), 0, cap) = 0, also for an infinite or NaN x: med3
          // with a NaN operand returns the smallest of the other two
          dst[row * PITCH + pos] = __builtin_amdgcn_fmed3f(fmaf(v, sc[i], sh[i]), 0.f, cap);
        } else {
          const uint32_t keep = (c * KC + row < a.C_in) ? tkeep : 0u;
          dst[row * PITCH + pos] = __uint_as_float(__float_as_uint(v) & keep);
        }
      }
    }
  };
  // A operands of 16-row group G = 2*chunk + g: 4 float4 (one per 16-channel block),
  // each holding the lane's 4 MFMA steps.
  const int n_groups = 2 * a.Q;
  auto load_w = [&](int G, f32x4 (&dst)[MB]) {
    G = min(G, n_groups - 1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // wave-uniform base (scalar registers) plus the lane's 16-byte slot
      const f32x4* wb = Wp4 + (size_t)(G * a.NCB + cb0 + mb) * 64;
      dst[mb] = wb[l];
    }
  };
  // B operands of MFMA step s (row 16*(s/4) + 4*lq + s%4).
  auto load_b = [&](const float* zb, int s, f32x4 (&dst)[NQ]) {
    const float* p = zb + (16 * (s >> 2) + 4 * lq + (s & 3)) * PITCH + l16 * 4;
#pragma unroll
    for (int m = 0; m < NQ; ++m) dst[m] = *reinterpret_cast<const f32x4*>(p + 64 * m);
  };

  f32x4 wr[2][MB];
  f32x4 bv[2][NQ];

  auto compute = [&](const float* zb, int q, auto&& mid) {
    load_b(zb, 0, bv[0]);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      load_w(2 * q + g + 1, wr[(g + 1) & 1]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = 4 * g + u;
        if (s + 1 < 8) load_b(zb, s + 1, bv[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float av = wr[g][mb][u];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[s & 1][nb >> 2][nb & 3],
                                                               acc[mb][nb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (s == 3) {
          mid();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  const int Q = a.Q;
  load_w(0, wr[0]);
  load_x(0);
  store_z(0, zs[0]);
  __syncthreads();
  int q = 0;
  for (; q + 1 < Q; q += 2) {
    load_x(q + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(zs[0], q, [&] { store_z(q + 1, zs[1]); });
    __syncthreads();
    const int qn = min(q + 2, Q - 1);
    load_x(qn);
    __builtin_amdgcn_sched_barrier(0);
    compute(zs[1], q + 1, [&] { store_z(qn, zs[0]); });
    __syncthreads();
  }
  if (q < Q) compute(zs[0], q, [] {});

  // Epilogue. Accumulator register r of block (mb, nb) holds output channel
  // 16*mb + 4*lq + r (within the wave's 64) and time 16*nb + l16.
  // not restrict: the residual may be out itself (in-place residual add)
  XT* outn = reinterpret_cast<XT*>(a.out) + (size_t)n * a.C_out * a.L_out;
  const int co_base = ct * CO_TILE + 16 * MB * w + 4 * lq;
  if (EPI == EPI_RESIDUAL) {
    const XT* resn = reinterpret_cast<const XT*>(a.residual) + (size_t)n * a.C_out * a.L_out;
    const bool vec_epi = sizeof(XT) == 4 && ((a.L_out & 3) == 0) &&
                         (((reinterpret_cast<uintptr_t>(a.out) |
                            reinterpret_cast<uintptr_t>(a.residual)) & 15) == 0);
    if (vec_epi) {
      // Each 16-channel block of accumulators goes through the staging LDS so that a
      // lane then owns 4 consecutive time steps of one channel: 16-byte residual loads
      // and stores. The barrier makes sure every wave has finished reading its last B
      // operands (with an odd chunk count the loop ends without one). Every wave then
      // uses its own 16 x (TT+4) float tile; the LDS accesses of a wave complete in
      // order, so no further barrier is needed.
      __syncthreads();
      constexpr int EP = TT + 4;
      constexpr int CH = TT / 4;              // float4 chunks per row
      constexpr int IPL = 16 * CH / 64;       // (row, chunk) items per lane per block
      float* ep = &zs[0][0] + w * (16 * EP);
      const int co_w = ct * CO_TILE + 16 * MB * w;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) ep[(4 * lq + r) * EP + 16 * nb + l16] = acc[mb][nb][r];
        // residual and bias loads (clamped in-bounds; L_out is a multiple of 4, so a
        // clamped chunk start is too) go out before any use
        f32x4 rv[IPL];
        float bia[IPL];
#pragma unroll
        for (int i = 0; i < IPL; ++i) {
          const int item = l + 64 * i;
          const int row = item / CH, ch = item % CH;
          const int coc = min(co_w + 16 * mb + row, a.C_out - 1);
          const int tcl = min(t0 + 4 * ch, a.L_out - 4);
          rv[i] = *reinterpret_cast<const f32x4*>(resn + (size_t)coc * a.L_out + tcl);
          bia[i] = a.bias ? a.bias[coc] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < IPL; ++i) {
          const int item = l + 64 * i;
          const int row = item / CH, ch = item % CH;
          const int co = co_w + 16 * mb + row;
          const int t = t0 + 4 * ch;
          const f32x4 v = *reinterpret_cast<const f32x4*>(ep + row * EP + 4 * ch);
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = v[e] + bia[i] + rv[i][e];
          // t and L_out are multiples of 4: the 4 steps are all in range or all out.
          // Non-temporal: out is not read again here, and the stores then pass the
          // caches without allocating, which shortens the end-of-round write bursts.
          if (co < a.C_out && t < a.L_out)
            __builtin_nontemporal_store(
                o, reinterpret_cast<f32x4*>(outn + (size_t)co * a.L_out + t));
        }
      }
    } else
    // Residual and bias loads use clamped (always in-bounds) addresses and are issued
    // a 16-channel block at a time before any use, so each block pays the memory
    // latency once; only the stores are predicated.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float res[4][NB], bco[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int coc = min(co_base + 16 * mb + r, a.C_out - 1);
        bco[r] = a.bias ? a.bias[coc] : 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int tc = min(t0 + 16 * nb + l16, a.L_out - 1);
          res[r][nb] = to_f32(resn[coc * a.L_out + tc]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co_base + 16 * mb + r;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int t = t0 + 16 * nb + l16;
          if (co < a.C_out && t < a.L_out)
            __builtin_nontemporal_store(acc[mb][nb][r] + bco[r] + res[r][nb],
                                        &outn[co * a.L_out + t]);
        }
      }
    }
  } else {
    const int cnt = min(TT, a.L_out - t0);
    const float inv_cnt = 1.f / (float)cnt;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co_base + 16 * mb + r;
        const bool cok = co < a.C_out;
        const float bco = (cok && a.bias) ? a.bias[co] : 0.f;
        float y[NB];
        float s = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          y[nb] = acc[mb][nb][r] + bco;
          s += (t0 + 16 * nb + l16 < a.L_out) ? y[nb] : 0.f;
        }
        s = quarterwave_sum(s);
        const float mean = s * inv_cnt;
        float m2 = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float dv = y[nb] - mean;
          m2 += (t0 + 16 * nb + l16 < a.L_out) ? dv * dv : 0.f;
        }
        m2 = quarterwave_sum(m2);
        if (cok) {
          if (l16 == 0) {
            float* p = a.partials + (((size_t)n * a.C_out + co) * a.n_tt + tt) * 3;
            p[0] = s;
            p[1] = m2;
            p[2] = (float)cnt;
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int t = t0 + 16 * nb + l16;
            if (t < a.L_out) from_f32(y[nb], &outn[co * a.L_out + t]);
          }
        }
      }
  }
}

template <int TT, int MB, bool BN, int EPI, typename XT>
static hipError_t launch_one(const ConvF32Args& a, int nwg, hipStream_t stream) {
  hipLaunchKernelGGL((conv_f32_kernel<TT, MB, BN, EPI, XT>), dim3(nwg), dim3(NTHREADS), 0, stream,
                     a);
  return hipGetLastError();
}

template <bool BN, int EPI>
static hipError_t launch_shape(const ConvF32Args& a, ConvTile tile, int nwg, hipStream_t stream) {
  if (tile.tt == 128 && tile.mb == 4) return launch_one<128, 4, BN, EPI, float>(a, nwg, stream);
  if (tile.tt == 64 && tile.mb == 4) return launch_one<64, 4, BN, EPI, float>(a, nwg, stream);
  if (tile.tt == 64 && tile.mb == 2) return launch_one<64, 2, BN, EPI, float>(a, nwg, stream);
  if (tile.tt == 128 && tile.mb == 2) return launch_one<128, 2, BN, EPI, float>(a, nwg, stream);
  if (tile.tt == 128 && tile.mb == 1) return launch_one<128, 1, BN, EPI, float>(a, nwg, stream);
  if (tile.tt == 64 && tile.mb == 1) return launch_one<64, 1, BN, EPI, float>(a, nwg, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_conv_f32(const ConvF32Args& a, ConvTile tile, int epilogue, hipStream_t stream) {
  const long long nwg = (long long)a.N * a.n_tt * a.n_ct;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool bn = a.scale != nullptr;
  if (epilogue == EPI_RESIDUAL) {
    if (!bn) return hipErrorInvalidValue;
    return launch_shape<true, EPI_RESIDUAL>(a, tile, (int)nwg, stream);
  }
  if (bn) return hipErrorInvalidValue;
  return launch_shape<false, EPI_GN_STATS>(a, tile, (int)nwg, stream);
}

}  // namespace dconv1d

