// Float32 kernel for the pre-norm residual block (POPCORNBENCH "Kimi-K2.6__l2_p12", first
// turn: out = x + b + Conv1d_{k=3, dilation d, padding d}(ReLU(BN(x)))) by Winograd
// F(2,3) along the dilation lattice.
//
// Two outputs d apart share three of their four inputs. With z = ReLU(BN(x)) (zero
// outside [0, L)), taps g0, g1, g2 and the inputs v0..v3 = z(t - d), z(t), z(t + d),
// z(t + 2d) of the output pair (t, t + d):
//   V0 = v0 - v2,  V1 = v1 + v2,  V2 = v2 - v1,  V3 = v1 - v3
//   U0 = g0,  U1 = (g0 + g1 + g2) / 2,  U2 = (g0 - g1 + g2) / 2,  U3 = g2
//   M_j = sum over input channels of U_j * V_j
//   y(t) = M0 + M1 + M2,  y(t + d) = M1 - M2 - M3,
// which is the direct three-tap sum exactly (up to rounding), with four products per pair
// and input channel instead of six: the four M_j are four GEMMs of K = C_in, so the
// kernel runs 2/3 of the direct conv's MFMA work.
//
// Pairs. Output step t = 2d*b + r (r < d) pairs with t + d; pair p = d*b + r. A tile is
// 32 consecutive pairs, so pair c of tile pt has first step t0 = 2d*(p / d) + p % d with
// p = 32*pt + c. When d is a multiple of 32 the tile is 32 consecutive r of one
// super-block (outputs [T0, T0 + 32) and [T0 + d, T0 + d + 32)); when d divides 32 it is
// 32/d whole super-blocks (outputs [T0, T0 + 64)); with D = min(d, 32) both cases read
//   t0(c) = T0 + 2D*(c / D) + c % D,
// and the epilogue goes through LDS. Any other dilation takes the per-element epilogue.
//
// Work split
//   workgroup  = one sample n, 64*WMB output channels (WMB = 4, 2 or 1: 256, 128 or 64),
//                32 pairs (64 output steps); 4 waves, wave w owns output channels
//                [16*WMB*w, 16*WMB*(w + 1)): for each of the four transforms j, WMB x 2
//                MFMA 16x16 accumulator blocks (128 registers at WMB = 4).
//   K loop     = chunks of 32 input channels (no taps: they are inside the transform),
//                8 MFMA steps of K = 4 each, 32 MFMAs per step.
//   B operand  = V_j[32 rows][32 pairs] staged through LDS per chunk by all 256 threads:
//                each thread loads the four lattice inputs of 4 (row, pair) items: one
//                row and four consecutive pairs by four 16-byte loads when L is a
//                multiple of 4 and x 16-byte aligned (one load per lattice step when d is
//                4, 8, 16 or a multiple of 32; the 16 steps around the pairs when d is 1
//                or 2), else 4 rows of one pair by sixteen 4-byte loads. It applies
//                BN+ReLU (med3(fma(x, scale, shift), 0, cap), cap = 0 outside the input),
//                forms V0..V3 and writes each item's with one 16-byte store;
//                double-buffered, one barrier per chunk, the next chunk staged in the
//                middle of the current one's MFMAs. A row holds, for pair c, the four V_j at
//                64*(c/16) + 4*(c%16) + j, so a lane's B values of one MFMA step (pairs
//                l%16 and 16 + l%16, all four j) are two 16-byte LDS reads.
//   A operand  = U_j from the repack of prep_wino_kernel, one 16-byte load per (step,
//                16-channel block) holding the four j, two steps ahead: the MFMAs of a
//                step run block by block, and each block's register slot is refilled for
//                the step after next as soon as its MFMAs have issued. One step ahead was
//                too short for a workgroup alone on its CU (its step takes half as long
//                as with a partner): 9% slower overall.
//   Epilogue   = y(t0), y(t0 + d) from the four accumulator sets in registers, then as in
//                the direct kernel: through LDS so that a lane owns 4 consecutive steps,
//                + bias + residual (16-byte loads), non-temporal 16-byte stores.
//   MFMA       = v_mfma_f32_16x16x4_f32 (float32 products and accumulation).
//
// The K-row permutation inside a chunk (r = 16g + 4q + u) and the XCD-aware workgroup order
// are those of the direct kernel (conv_f32.hip).

#include "internal.h"

namespace dconv1d {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WPAIRS = WINO_PAIRS;        // output pairs per workgroup
constexpr int WPITCH = 4 * WPAIRS + 4;    // floats per staged row (four V_j per pair)
constexpr int WEP = 2 * WPAIRS + 4;       // floats per epilogue row (64 output steps)
constexpr int WNB = WPAIRS / 16;          // 16-pair blocks per wave
constexpr int WRPL = KC * WPAIRS / NTHREADS;   // staged (row, pair) items per thread (4)

// v of the lane K places further along its DPP row of 16 lanes (row_ror:K)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 | K, 0xF, 0xF, false));
}

// sum over the 16 lanes of each quarter-wave (a DPP row); lanes associate the terms
// differently, so where the bits matter one lane's value is used
__device__ __forceinline__ float quarterwave_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

// first output step of pair p
__device__ __forceinline__ int wino_pair_step(int p, int d) {
  const int b = p / d;
  return 2 * d * b + (p - b * d);
}

// first output step of pair tile pt, for a dilation that divides 32 or is a multiple of it
__device__ __forceinline__ int wino_tile_start(int pt, int d) {
  if (d >= 32) {
    const int per = d >> 5;
    return 2 * d * (pt / per) + 32 * (pt % per);
  }
  return 64 * pt;
}

}  // namespace

// WMB: 16-channel blocks per wave (the workgroup's channel tile is 64*WMB: 256, 128 or 64).
// BN: the staged value is ReLU(BN(x)) (the block) or x itself (the conv of Conv1d +
// GroupNorm). EPI: EPI_RESIDUAL (the block: + bias + residual) or EPI_GN_STATS (y = conv
// + bias into out, and per (channel, pair tile) the sum, the tile-centred sum of squares
// and the count of y for the GroupNorm pass).
// SX: the staging form (below): SX_SCALAR for any shape; SX_LATTICE for d = 4, 8, 16 or
// a multiple of 32, SX_WINDOW1 for d = 1 and SX_WINDOW2 for d = 2, each with L a multiple
// of 4 and x 16-byte aligned.
enum { SX_SCALAR = 0, SX_LATTICE = 1, SX_WINDOW1 = 2, SX_WINDOW2 = 3 };
template <int WMB, bool BN, int EPI, int SX>
__global__ void __launch_bounds__(NTHREADS, 2)
conv_wino_kernel(ConvF32Args a) {
  constexpr int CO_TILE = 64 * WMB;
  // two named staging buffers (see conv_f32.hip); the epilogue reuses them
  __shared__ __attribute__((aligned(16))) float zs0[KC * WPITCH];
  __shared__ __attribute__((aligned(16))) float zs1[KC * WPITCH];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lq = l >> 4;
  const int l16 = l & 15;

  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = b & 7;
  const int logical = xcd * per + min(xcd, rem) + (b >> 3);
  const int ct = __builtin_amdgcn_readfirstlane(logical % a.n_ct);
  const int rest = logical / a.n_ct;
  const int pt = __builtin_amdgcn_readfirstlane(rest % a.n_tt);
  const int n = __builtin_amdgcn_readfirstlane(rest / a.n_tt);

  const int d = a.dil;
  const int L = a.L_in;
  // regular: d divides 32 or is a multiple of it (the tile's outputs form one or two runs)
  const bool regular = (d & 31) == 0 || (32 % d) == 0;
  const int T0 = __builtin_amdgcn_readfirstlane(regular ? wino_tile_start(pt, d) : 0);
  const int D = regular ? min(d, 32) : 1;   // a power of two
  const int lgD = __builtin_ctz(D);

  const float* __restrict__ xn = reinterpret_cast<const float*>(a.x) + (size_t)n * a.C_in * L;
  const f32x4* __restrict__ Up4 = reinterpret_cast<const f32x4*>(a.Wp);
  const int cb0 = (ct * CO_TILE) / 16 + WMB * w;

  f32x4 acc[4][WMB][WNB];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][mb][nb][r] = 0.f;

  // Staging geometry of this lane. Scalar form: pair c = l % 32 of the tile, rows
  // 8w + 2i + l/32 (i = 0..3) of each chunk, one 4-byte load per lattice step. The other
  // two: row 8w + l/8 of each chunk and the four pairs c .. c + 3, c = 4(l % 8), with
  // 16-byte loads of 4 steps from a multiple of 4, which lie all inside the input or all
  // outside (0 and L are multiples of 4 too). Lattice form: the four pairs' steps are
  // consecutive, so one load per lattice step brings all four. Window form (d = 1 or 2):
  // the four pairs' 16 lattice inputs lie in the 16 steps from t0c - 4 on, four loads.
  // The loaded steps and their caps are the same for every chunk.
  const int c = SX != SX_SCALAR ? 4 * (l & 7) : (l & 31);
  const int hrow = SX != SX_SCALAR ? (l >> 3) : (l >> 5);
  const int t0c = regular ? T0 + ((c >> lgD) << (lgD + 1)) + (c & (D - 1))
                          : wino_pair_step(WPAIRS * pt + c, d);
  uint32_t toff[4];                         // byte offsets inside a row
  float cap[4];                             // BN: +inf inside the input, 0 on padding
  uint32_t keep[4];                         // no BN: all ones inside the input, 0 on padding
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    // lattice step m, or window group m; |t| < 2^30: L, d < 2^28
    const int t = SX >= SX_WINDOW1 ? t0c - 4 + 4 * m : t0c + (m - 1) * d;
    const bool in = t >= 0 && t < L;
    // an outside step loads any in-range step: its cap makes it zero
    toff[m] = 4u * (uint32_t)(in ? t : 0);
    cap[m] = in ? __builtin_huge_valf() : 0.f;
    keep[m] = in ? 0xffffffffu : 0u;
    if (BN)
      asm volatile("" : "+v"(cap[m]));
    else
      asm volatile("" : "+v"(keep[m]));
  }
  const int zpos = 64 * (c >> 4) + 4 * (c & 15);   // LDS position of the pair in a row

  float xr[WRPL][4];   // scalar form: row i, lattice step m
  f32x4 xv[4];         // lattice form: step m of pairs c .. c + 3; window form: group m
  float sc[WRPL], sh[WRPL];
  auto load_x = [&](int q) {
    if constexpr (SX != SX_SCALAR) {
      const int rl = min(KC * q + 8 * w + hrow, a.C_in - 1);
      const char* rowp = reinterpret_cast<const char*>(xn + (size_t)rl * L);
#pragma unroll
      for (int m = 0; m < 4; ++m) xv[m] = *reinterpret_cast<const f32x4*>(rowp + toff[m]);
      if (BN) {
        sc[0] = a.scale[KC * q + 8 * w + hrow];
        sh[0] = a.shift[KC * q + 8 * w + hrow];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < WRPL; ++i) {
      // a padded input channel loads the last real row: its scale and shift are 0
      const int rb = min(KC * q + 8 * w + 2 * i, a.C_in - 1);            // wave-uniform
      const int rl = min(KC * q + 8 * w + 2 * i + hrow, a.C_in - 1);     // this lane's
      // the row's base address is wave-uniform (scalar registers); the lane adds one row
      // (or none) and its step, in bytes: below 2^31 as L < 2^28
      const char* rowp = reinterpret_cast<const char*>(xn + (size_t)rb * L);
      const uint32_t ro = (uint32_t)(rl - rb) * 4u * (uint32_t)L;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xr[i][m] = *reinterpret_cast<const float*>(rowp + (ro + toff[m]));
      if (BN) {
        sc[i] = a.scale[KC * q + 8 * w + 2 * i + hrow];
        sh[i] = a.shift[KC * q + 8 * w + 2 * i + hrow];
      }
    }
  };
  // chunk q's staged values: with BN, med3(fma(x, scale, shift), 0, cap) (a padded input
  // channel has scale = shift = 0); without, x AND a mask that is zero on a padded tap
  // or a padded input channel
  auto store_z = [&](int q, float* dst) {
    if constexpr (SX != SX_SCALAR) {
      const uint32_t rkeep = KC * q + 8 * w + hrow < a.C_in ? 0xffffffffu : 0u;
      float* drow = dst + (8 * w + hrow) * WPITCH + zpos;
      // the four pairs, with the loaded value (group g, element e) of lattice step m of
      // pair u given by pos(u, m) = 4g + e
      auto stage = [&](auto pos) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float z[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int g = pos(u, m) >> 2, e = pos(u, m) & 3;
            z[m] = BN ? __builtin_amdgcn_fmed3f(fmaf(xv[g][e], sc[0], sh[0]), 0.f, cap[g])
                      : __uint_as_float(__float_as_uint(xv[g][e]) & keep[g] & rkeep);
          }
          f32x4 v;
          v[0] = z[0] - z[2];
          v[1] = z[1] + z[2];
          v[2] = z[2] - z[1];
          v[3] = z[1] - z[3];
          *reinterpret_cast<f32x4*>(drow + 4 * u) = v;
        }
      };
      if constexpr (SX == SX_LATTICE) {
        stage([](int u, int m) { return 4 * m + u; });
      } else if constexpr (SX == SX_WINDOW1) {
        // pair u is (t0c + 2u, t0c + 2u + 1): step m at t0c + 2u + m - 1
        stage([](int u, int m) { return 2 * u + m + 3; });
      } else {
        // d = 2: pair u is (t0c + 4(u/2) + u%2, + 2): step m at that + 2(m - 1)
        stage([](int u, int m) { return 4 * (u >> 1) + (u & 1) + 2 * m + 2; });
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < WRPL; ++i) {
      float z[4];
      const uint32_t rkeep = KC * q + 8 * w + 2 * i + hrow < a.C_in ? 0xffffffffu : 0u;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        z[m] = BN ? __builtin_amdgcn_fmed3f(fmaf(xr[i][m], sc[i], sh[i]), 0.f, cap[m])
                  : __uint_as_float(__float_as_uint(xr[i][m]) & keep[m] & rkeep);
      f32x4 v;
      v[0] = z[0] - z[2];
      v[1] = z[1] + z[2];
      v[2] = z[2] - z[1];
      v[3] = z[1] - z[3];
      *reinterpret_cast<f32x4*>(dst + (8 * w + 2 * i + hrow) * WPITCH + zpos) = v;
    }
  };
  // A operands of MFMA step s of chunk q: one float4 (U0..U3) per 16-channel block
  const int Q = a.Q;
  auto load_a1 = [&](int q, int s, int mb, f32x4& dst) {
    q = min(q, Q - 1);
    dst = Up4[(size_t)((8 * q + s) * a.NCB + cb0 + mb) * 64 + l];
  };
  auto load_a = [&](int q, int s, f32x4 (&dst)[WMB]) {
    q = min(q, Q - 1);
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const f32x4* ub = Up4 + (size_t)((8 * q + s) * a.NCB + cb0 + mb) * 64;
      dst[mb] = ub[l];
    }
  };
  // B operands of MFMA step s (row 16*(s/4) + 4*lq + s%4): pairs l16 and 16 + l16
  auto load_b = [&](const float* zb, int s, f32x4 (&dst)[WNB]) {
    const float* p = zb + (16 * (s >> 2) + 4 * lq + (s & 3)) * WPITCH + 4 * l16;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) dst[nb] = *reinterpret_cast<const f32x4*>(p + 64 * nb);
  };

  f32x4 au[2][WMB];
  f32x4 bv[2][WNB];

  auto compute = [&](const float* zb, int q, auto&& mid) {
    load_b(zb, 0, bv[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s + 1 < 8) load_b(zb, s + 1, bv[(s + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int nb = 0; nb < WNB; ++nb)
            acc[j][mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                au[s & 1][mb][j], bv[s & 1][nb][j], acc[j][mb][nb], 0, 0, 0);
        // the block's slot now holds what step s + 2 needs
        load_a1(s + 2 < 8 ? q : q + 1, (s + 2) & 7, mb, au[s & 1][mb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s == 3) {
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  load_a(0, 0, au[0]);
  load_a(0, 1, au[1]);
  load_x(0);
  store_z(0, zs0);
  __syncthreads();
  int q = 0;
  for (; q + 1 < Q; q += 2) {
    load_x(q + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(zs0, q, [&] { store_z(q + 1, zs1); });
    __syncthreads();
    const int qn = min(q + 2, Q - 1);
    load_x(qn);
    __builtin_amdgcn_sched_barrier(0);
    compute(zs1, q + 1, [&] { store_z(qn, zs0); });
    __syncthreads();
  }
  if (q < Q) compute(zs0, q, [] {});

  // Epilogue. Register r of block (j, mb, nb) holds M_j of output channel 16mb + 4lq + r
  // (within the wave's 64) and pair 16nb + l16; y(t0) = (M0 + M1) + M2 and
  // y(t0 + d) = (M1 - M2) - M3. Output column o of the tile (0..63, increasing step) of
  // pair c: o0 = 2D*(c / D) + c % D and o0 + D; its step is T0 + o, or T0 + d + (o - 32)
  // for o >= 32 when d > 32.
  float* outn = reinterpret_cast<float*>(a.out) + (size_t)n * a.C_out * L;
  const int co_w = ct * CO_TILE + 16 * WMB * w;
  if (EPI == EPI_GN_STATS) {
    // y = conv + bias into out, and per output channel the tile's sum S of y, the sum of
    // squares about the tile mean and the count, at partials[((n*C_out + co)*n_tt + pt)*3].
    // Registers (j, mb, nb, r) of the 16 lanes of quarter-wave lq hold channel
    // 16mb + 4lq + r at all 32 pairs of the tile, so each sum runs over those 16 lanes
    // (DPP row rotations), and lane 0 of the row gives S to the row before the second
    // pass.
    int ta[WNB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int cc = 16 * nb + l16;
      ta[nb] = regular ? T0 + ((cc >> lgD) << (lgD + 1)) + (cc & (D - 1))
                       : wino_pair_step(WPAIRS * pt + cc, d);
    }
    float cnt = 0.f;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) cnt += (ta[nb] < L ? 1.f : 0.f) + (ta[nb] + d < L ? 1.f : 0.f);
    // whole numbers up to 64, exact in every lane; 0 for a tile whose pairs all lie past
    // the end (the last tile of a dilation that does not divide its super-blocks evenly)
    cnt = quarterwave_sum(cnt);
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co_w + 16 * mb + 4 * lq + r;
        const float bco = (co < a.C_out && a.bias) ? a.bias[co] : 0.f;
        float y[WNB][2];
        float sum = 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) {
          const float m0 = acc[0][mb][nb][r], m1 = acc[1][mb][nb][r];
          const float m2 = acc[2][mb][nb][r], m3 = acc[3][mb][nb][r];
          y[nb][0] = ((m0 + m1) + m2) + bco;
          y[nb][1] = ((m1 - m2) - m3) + bco;
          sum += (ta[nb] < L ? y[nb][0] : 0.f) + (ta[nb] + d < L ? y[nb][1] : 0.f);
        }
        sum = __shfl(quarterwave_sum(sum), 16 * lq);
        const float mean = cnt > 0.f ? sum / cnt : 0.f;
        float m2s = 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) {
          const float d0 = y[nb][0] - mean, d1 = y[nb][1] - mean;
          m2s += (ta[nb] < L ? d0 * d0 : 0.f) + (ta[nb] + d < L ? d1 * d1 : 0.f);
        }
        m2s = quarterwave_sum(m2s);
        if (co < a.C_out) {
#pragma unroll
          for (int nb = 0; nb < WNB; ++nb) {
            if (ta[nb] < L) outn[(size_t)co * L + ta[nb]] = y[nb][0];
            if (ta[nb] + d < L) outn[(size_t)co * L + ta[nb] + d] = y[nb][1];
          }
          if (l16 == 0) {
            float* pp = a.partials + (((size_t)n * a.C_out + co) * a.n_tt + pt) * 3;
            pp[0] = sum;
            pp[1] = m2s;
            pp[2] = cnt;
          }
        }
      }
    }
    return;
  }
  const float* resn = reinterpret_cast<const float*>(a.residual) + (size_t)n * a.C_out * L;
  const int skip = d > 32 ? d - 32 : 0;
  const bool vec_epi = regular && ((L & 3) == 0) &&
                       (((reinterpret_cast<uintptr_t>(a.out) |
                          reinterpret_cast<uintptr_t>(a.residual)) & 15) == 0);
  if (vec_epi) {
    // every wave has finished reading its last B operands; each wave then uses its own
    // 16 x WEP tile, and its LDS accesses complete in order
    __syncthreads();
    float* ep = (w < 2 ? zs0 : zs1) + (w & 1) * (16 * WEP);
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int cc = 16 * nb + l16;
        const int o0 = ((cc >> lgD) << (lgD + 1)) + (cc & (D - 1));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float m0 = acc[0][mb][nb][r], m1 = acc[1][mb][nb][r];
          const float m2 = acc[2][mb][nb][r], m3 = acc[3][mb][nb][r];
          ep[(4 * lq + r) * WEP + o0] = (m0 + m1) + m2;
          ep[(4 * lq + r) * WEP + o0 + D] = (m1 - m2) - m3;
        }
      }
      // 16 rows x 16 four-step chunks, 4 per lane; residual and bias loads (clamped
      // in-bounds; L is a multiple of 4, so a clamped chunk start is too) before any use
      f32x4 rv[4];
      float bia[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int item = l + 64 * i;
        const int row = item >> 4, o = 4 * (item & 15);
        const int t = T0 + o + (o >= 32 ? skip : 0);
        const int coc = min(co_w + 16 * mb + row, a.C_out - 1);
        const int tcl = min(t, L - 4);
        rv[i] = *reinterpret_cast<const f32x4*>(resn + (size_t)coc * L + tcl);
        bia[i] = a.bias ? a.bias[coc] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int item = l + 64 * i;
        const int row = item >> 4, o = 4 * (item & 15);
        const int t = T0 + o + (o >= 32 ? skip : 0);
        const int co = co_w + 16 * mb + row;
        const f32x4 v = *reinterpret_cast<const f32x4*>(ep + row * WEP + o);
        f32x4 res;
#pragma unroll
        for (int e = 0; e < 4; ++e) res[e] = v[e] + bia[i] + rv[i][e];
        // t and L are multiples of 4: the 4 steps are all in range or all out
        if (co < a.C_out && t < L)
          __builtin_nontemporal_store(res, reinterpret_cast<f32x4*>(outn + (size_t)co * L + t));
      }
    }
  } else {
    int ta[WNB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int cc = 16 * nb + l16;
      ta[nb] = regular ? T0 + ((cc >> lgD) << (lgD + 1)) + (cc & (D - 1))
                       : wino_pair_step(WPAIRS * pt + cc, d);
    }
    float rs[WMB][4][WNB][2], bco[WMB][4];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int coc = min(co_w + 16 * mb + 4 * lq + r, a.C_out - 1);
        bco[mb][r] = a.bias ? a.bias[coc] : 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) {
          rs[mb][r][nb][0] = resn[(size_t)coc * L + min(ta[nb], L - 1)];
          rs[mb][r][nb][1] = resn[(size_t)coc * L + min(ta[nb] + d, L - 1)];
        }
      }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co_w + 16 * mb + 4 * lq + r;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) {
          const int tb = ta[nb] + d;
          const float m0 = acc[0][mb][nb][r], m1 = acc[1][mb][nb][r];
          const float m2 = acc[2][mb][nb][r], m3 = acc[3][mb][nb][r];
          if (co < a.C_out && ta[nb] < L)
            __builtin_nontemporal_store(((m0 + m1) + m2) + bco[mb][r] + rs[mb][r][nb][0],
                                        &outn[(size_t)co * L + ta[nb]]);
          if (co < a.C_out && tb < L)
            __builtin_nontemporal_store(((m1 - m2) - m3) + bco[mb][r] + rs[mb][r][nb][1],
                                        &outn[(size_t)co * L + tb]);
        }
      }
    }
  }
}

template <bool BN, int EPI, int SX>
static void launch_wmb(const ConvF32Args& a, int wmb, dim3 grid, dim3 block,
                       hipStream_t stream) {
  if (wmb == 4)
    hipLaunchKernelGGL((conv_wino_kernel<4, BN, EPI, SX>), grid, block, 0, stream, a);
  else if (wmb == 2)
    hipLaunchKernelGGL((conv_wino_kernel<2, BN, EPI, SX>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((conv_wino_kernel<1, BN, EPI, SX>), grid, block, 0, stream, a);
}

hipError_t launch_conv_wino(const ConvF32Args& a, int wmb, int epilogue, hipStream_t stream) {
  const long long nwg = (long long)a.N * a.n_tt * a.n_ct;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // the block: BN folded into scale/shift, a residual of the output's shape; Conv1d +
  // GroupNorm: no BN, the partials array
  const bool block_ok = epilogue == EPI_RESIDUAL && a.scale != nullptr && a.C_in == a.C_out;
  const bool gn_ok = epilogue == EPI_GN_STATS && a.scale == nullptr && a.partials != nullptr;
  if (!(block_ok || gn_ok) || a.L_in != a.L_out || a.pad != a.dil ||
      !wino_supported(a.L_in) || a.dil < 1 || a.dil > a.L_in ||
      a.n_tt != wino_pair_tiles(a.L_in, a.dil) ||
      (wmb != 1 && wmb != 2 && wmb != 4) || a.n_ct != (a.C_out + 64 * wmb - 1) / (64 * wmb) ||
      a.NCB * 16 < a.n_ct * 64 * wmb || a.Q * KC < a.C_in)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg), block(NTHREADS);
  // the staging form: 16-byte loads need L a multiple of 4 and x 16-byte aligned
  const int d = a.dil;
  const bool v16 = a.L_in % 4 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0;
  const int sx = !v16 ? SX_SCALAR
                 : d % 32 == 0 || (d >= 4 && 32 % d == 0) ? SX_LATTICE
                 : d == 1 ? SX_WINDOW1 : d == 2 ? SX_WINDOW2 : SX_SCALAR;
  if (block_ok) {
    if (sx == SX_LATTICE)
      launch_wmb<true, EPI_RESIDUAL, SX_LATTICE>(a, wmb, grid, block, stream);
    else if (sx == SX_WINDOW1)
      launch_wmb<true, EPI_RESIDUAL, SX_WINDOW1>(a, wmb, grid, block, stream);
    else if (sx == SX_WINDOW2)
      launch_wmb<true, EPI_RESIDUAL, SX_WINDOW2>(a, wmb, grid, block, stream);
    else
      launch_wmb<true, EPI_RESIDUAL, SX_SCALAR>(a, wmb, grid, block, stream);
  } else {
    if (sx == SX_LATTICE)
      launch_wmb<false, EPI_GN_STATS, SX_LATTICE>(a, wmb, grid, block, stream);
    else if (sx == SX_WINDOW1)
      launch_wmb<false, EPI_GN_STATS, SX_WINDOW1>(a, wmb, grid, block, stream);
    else if (sx == SX_WINDOW2)
      launch_wmb<false, EPI_GN_STATS, SX_WINDOW2>(a, wmb, grid, block, stream);
    else
      launch_wmb<false, EPI_GN_STATS, SX_SCALAR>(a, wmb, grid, block, stream);
  }
  return hipGetLastError();
}

}  // namespace dconv1d
