// Conv1d + GroupNorm in one launch, for shapes whose groups fit in one workgroup
// (POPCORNBENCH "FW-GLM-5-1__l2_p35", its single turn: the conv with zero padding, then
// per (sample, group) the mean and the biased variance over the group's channels and
// time steps, normalisation with eps inside the square root, optional affine).
//
// Work split
//   workgroup  = one sample n and 16 output channels [co0, co0 + 16) over every output
//                time step (T_out <= 1024). Channels per group divides 16, so every group
//                lies inside one workgroup: the conv result stays in registers, the group
//                statistics are reduced inside the workgroup in a fixed order, and `out`
//                is written once, already normalised. No second pass over HBM, no weight
//                repack launch.
//   waves      = 8; wave w owns output steps [128w, 128w + 128): 8 accumulator blocks of
//                16 x 16 (v_mfma_f32_16x16x4_f32, float32 products and accumulation).
//   K loop     = chunks of 16 input channels. A chunk stages x[n][16c .. 16c + 16) over the
//                window of input steps [ws, ws + 64*MG), ws = -pad - delta, that every tap
//                of every output step reads, once, into LDS: tap k of output step t reads
//                window column t + k*dil + delta, so the three taps share one staged copy
//                and x crosses L2 -> LDS once per workgroup. Wave w stages channels
//                16c + w and 16c + w + 8 with buffer loads into registers (16 bytes per
//                lane when T is a multiple of 4 and x is 16-byte aligned, else 4), two
//                chunks ahead (chunk c + 2 loads while chunk c computes; chunk c + 1,
//                loaded during chunk c - 1, goes to LDS after chunk c's MFMAs), then one
//                ds_write per load. Steps outside [0, T) get an offset past the end of the
//                row's buffer range, so the hardware range check delivers exact zeros.
//                With 16-byte loads delta (0..3) puts ws on a multiple of 4, so a load lies
//                entirely inside or entirely outside [0, T); with 4-byte loads delta = 0.
//                Two LDS buffers, one barrier per chunk.
//   LDS layout = row r (channel 16c + r) at r*RS floats, RS = 64*MG + 8: RS = 8 mod 16
//                puts the rows 2lq of the four quarter-waves of a B read on different
//                banks.
//   private    = (MG = GN_PRIVATE, when 128 + 2*dil + delta <= GN_PW) every wave stages
//   windows      all 16 rows of a chunk itself, over only the GN_PW input steps from
//                128w - pad - delta on that its own 128 output steps read, into an LDS
//                area of its own (row pitch GN_PW, also 8 mod 16). The neighbouring waves'
//                windows overlap by 2*dil + delta steps (about 6% more L2 -> LDS traffic
//                for dil = 1), and no wave reads another's area, so the chunk loop has no
//                workgroup barrier: a wave's LDS accesses complete in program order, and
//                the two waves of a SIMD drift apart, one in its MFMAs while the other
//                loads. Here x goes straight into LDS: item i of the window (row i / IPR,
//                VW floats from column VW*(i % IPR) on, IPR = GN_PW / VW) lands at float
//                VW*i of the wave's area, which is exactly where a buffer->LDS load puts
//                lane i % 64 of load i / 64, so chunk c + 1's window is fetched by such
//                loads while chunk c computes, and x never passes through VGPRs
//                (measured 3% faster than register staging two chunks ahead: loads that
//                return into VGPRs slow the matrix pipe of their SIMD). Items past the 16
//                rows land in the padding of the wave's area; steps outside [0, T) get the
//                rejected offset and arrive as zeros. Both buffers are separate named
//                arrays, so the compiler's wait before a read of one buffer does not wait
//                for the loads into the other.
//   operands   = MFMA K-step (tap k, half g, e): quarter-wave lq = lane/16 supplies input
//                channel 16c + 8g + 2lq + e. A = W[co0 + lane%16][16c + 8g + 2lq + e][k]:
//                per half, six consecutive floats of the [C_out][C_in][3] layout per lane.
//                B = window column t + k*dil + delta of row 8g + 2lq + e. 96 MFMAs per
//                wave per chunk between barriers.
//   statistics = two passes over the registers: per-row sums (DPP row rotations over each
//                quarter-wave), then per group, in double, over (wave, row) in a fixed
//                butterfly order across a wave's lanes -> mean; the same for the sum of
//                squared deviations from that mean -> biased variance. Every wave forms
//                the group totals itself, in the same order, so each pass needs one
//                barrier. Bitwise reproducible: no atomics, no order that depends on
//                timing.

#include <type_traits>

#include "conv_gn.h"

namespace dconv1d {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int GN_WAVES = 8;
constexpr int GN_CI = 16;     // input channels per chunk
constexpr int GN_NB = 8;      // 16-column blocks per wave
// buffer resource word 3 for raw (untyped, unswizzled) buffers on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;
// voffset that fails the range check of any row (rows are < 2^31 bytes)
constexpr uint32_t kOutOfRange = 0x80000000u;

// v of the lane K places further along its DPP row of 16 lanes (row_ror:K)
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 | K, 0xF, 0xF, false));
}
// sum over the 16 lanes of each quarter-wave (a DPP row), with VALU row rotations rather
// than LDS swizzles; every lane ends with the sum (lanes associate the terms differently,
// so only one lane's value is used: the first lane of the row, always the same one)
__device__ __forceinline__ float quarterwave_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

// Sum, in double, of a group's per-(wave, row) partials red[16*ww + row] (8 waves x 16
// rows; the group of row r is r / cpg), over the 64 lanes of one wave in a fixed order:
// lane l adds the partials of waves l/16 and l/16 + 4 at row l%16, then butterflies over
// the row bits below cpg and over the wave bits. Every lane ends with the total of the
// group of row l%16; the order of additions does not depend on timing.
__device__ __forceinline__ double group_total(const float* red, int l, int cpg) {
  double v = (double)red[l] + (double)red[l + 64];
  for (int m = 1; m < cpg; m <<= 1) v += __shfl_xor(v, m);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// One buffer->LDS load of VW floats per lane: lane l's data lands at lds + VW*l. (A
// device-only function: lambdas in a kernel are compiled for the host too, where the
// 16-byte form of the builtin is not available.)
template <int VW>
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t rs, float* lds,
                                              uint32_t voffset) {
  auto* dst = (__attribute__((address_space(3))) void*)lds;
  if constexpr (VW == 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voffset, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voffset, 0, 0, 0);
}

}  // namespace

// MG: 64-step groups of the shared staged window (the window is 64*MG steps wide), or
// GN_PRIVATE for per-wave windows; VW: floats per lane per load (1 or 4); WINO: the
// Winograd form of the conv (per-wave windows only)
template <int MG, int VW, bool WINO>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * GN_WAVES, 64 * GN_WAVES)))
conv_gn_fused_kernel(GnFusedArgs a) {
  // MG == GN_PRIVATE: each wave stages its own window (see the file comment)
  constexpr bool PRIV = MG == GN_PRIVATE;
  static_assert(PRIV || !WINO, "the Winograd form runs with per-wave windows");
  constexpr int RS = PRIV ? GN_PW : 64 * MG + 8;               // floats per staged row
  // private windows: a wave's area holds its 16 rows and the tail of its last load
  constexpr int WAREA = PRIV ? (GN_CI * (RS / VW) + 63) / 64 * 64 * VW : GN_CI * RS;
  constexpr int BUF = (PRIV ? GN_WAVES : 1) * WAREA;           // floats per chunk buffer
  __shared__ __attribute__((aligned(16))) float zA[BUF];
  __shared__ __attribute__((aligned(16))) float zB[BUF];
  __shared__ float red[GN_WAVES * 16];    // per (wave, row) partials: sums
  __shared__ float red2[GN_WAVES * 16];   // and sums of squared deviations

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lq = l >> 4;
  const int l16 = l & 15;

  // XCD-aware order: workgroup b runs on XCD b % 8; consecutive logical indices (the
  // channel blocks of one sample, which read the same x) land on one XCD and its L2
  const int nwg = gridDim.x;
  const int b = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = b & 7;
  const int logical = xcd * per + min(xcd, rem) + (b >> 3);
  const int cb = __builtin_amdgcn_readfirstlane(logical % a.n_cb);
  const int n = __builtin_amdgcn_readfirstlane(logical / a.n_cb);
  const int co0 = 16 * cb;
  const int tw = 128 * w;                 // first output step of this wave
  const bool active = tw < a.T_out;       // waves past the end only stage (shared window)
  const int wz = PRIV ? w * WAREA : 0;        // this wave's LDS area (private windows)
  const int tz = PRIV ? 0 : tw;               // LDS column of the wave's first output step

  const float* xn = a.x + (size_t)n * a.C_in * a.T;
  // this lane's weight row: W[co0 + l16][2lq][0], or W[co0 + l16][4lq][0] in the
  // Winograd form (see load_w)
  const float* __restrict__ wrow =
      a.W + ((size_t)(co0 + l16) * a.C_in + (WINO ? 4 : 2) * lq) * 3;

  // three-tap form: block nb is output steps 16nb + l16 of the wave; Winograd form: block
  // 4j + nb is M_j of pairs 16nb + l16
  constexpr int NACC = WINO ? 16 : GN_NB;
  f32x4 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][r] = 0.f;
  // Winograd form: with d = dil (1, 2 or 4), wave-local pair p has first output step
  // 2d*(p/d) + p%d and second one d later; the lane's pair 16nb + l16 starts at 32nb + tl
  const int lgd = __builtin_ctz(a.dil);
  const int tl = WINO ? ((l16 >> lgd) << (lgd + 1)) + (l16 & (a.dil - 1)) : 0;

  // Load i of a row covers window columns [64*VW*i + VW*l, +VW), input steps from
  // ws = -pad - delta on. Its byte offset, or one the range check rejects (t < 0 or past
  // the window; t >= T is past the row's range by itself). Opaque, so that no constant
  // part is folded into the instruction offset (which could bring a rejected offset back
  // into range).
  static_assert(VW == 1 || VW == 4, "4- or 16-byte loads");
  using XV = typename std::conditional<VW == 4, f32x4, float>::type;
  // Private windows: item i of the 16 x GN_PW window is row i / IPR, columns
  // VW * (i % IPR) on, and lane l takes items l, l + 64, ... Shared window: loads per row.
  constexpr int IPR = RS / VW;                                  // items per private row
  constexpr int NL = PRIV ? (GN_CI * IPR + 63) / 64 : (64 * MG + 64 * VW - 1) / (64 * VW);
  constexpr int NX = PRIV ? NL : 2 * NL;                        // loads per lane per chunk
  const int ws = (PRIV ? tw : 0) - a.pad - a.delta;
  uint32_t voff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if constexpr (PRIV) {
      // byte offset within the chunk's 16 rows (one buffer range of 16*T floats), so
      // steps past T are rejected here rather than by the range check
      const int item = l + 64 * i, row = item / IPR, j = VW * (item % IPR);
      const int t = ws + j;
      voff[i] = (item < GN_CI * IPR && t >= 0 && t < a.T) ? 4u * (uint32_t)(row * a.T + t)
                                                          : kOutOfRange;
    } else {
      const int j = 64 * VW * i + VW * l;
      const int t = ws + j;
      voff[i] = (t >= 0 && j < 64 * MG) ? 4u * (uint32_t)t : kOutOfRange;
    }
    asm volatile("" : "+v"(voff[i]));
  }
  auto load_one = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo) -> XV {
    if constexpr (VW == 4)
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
    else
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo, 0, 0));
  };
  // Shared window: this wave's rows 16c + w (dst[0 .. NL)) and 16c + w + 8 (dst[NL .. 2NL))
  // of chunk c into registers (private windows go straight into LDS: dma_x below).
  XV xa[NX], xb[NX];
  auto load_x = [&](int c, XV (&dst)[NX]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(xn + (size_t)(GN_CI * c + w + 8 * h) * a.T), (short)0, 4 * a.T,
          kBufferFlags);
#pragma unroll
      for (int i = 0; i < NL; ++i) dst[h * NL + i] = load_one(rs, voff[i]);
    }
  };
  // columns past 64*MG (the tail of the last 16-byte load) are not stored
  auto store_x = [&](const XV (&src)[NX], float* zb) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int j = 64 * VW * i + VW * l;
        if (64 * VW * (i + 1) <= 64 * MG || j < 64 * MG)
          *reinterpret_cast<XV*>(zb + (w + 8 * h) * RS + j) = src[h * NL + i];
      }
  };
  // End of a chunk: the next chunk reads what this one staged. Shared window: every wave's
  // rows, so a workgroup barrier. Private: only this wave's own area; the wave's LDS
  // accesses complete in program order, so the fence only keeps the compiler from moving
  // them across.
  auto chunk_sync = [&] {
    if constexpr (PRIV)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    else
      __syncthreads();
  };
  const int nC = a.C_in / GN_CI;
  // A operands of chunk c: W[co0 + l16][16c + 8g + 2lq + e][k] at wrow + 48c + 24g + 3e + k,
  // stored at index 6g + 3e + k. Winograd form: the taps W[co0 + l16][16c + 4lq + s][k]
  // of K-step s at index 3s + k, twelve consecutive floats (16-byte aligned: C_in is a
  // multiple of 16 and W 16-byte aligned)
  auto load_w = [&](int c, float (&dst)[12]) {
    c = min(c, nC - 1);
    if constexpr (WINO) {
      const f32x4* p = reinterpret_cast<const f32x4*>(wrow + 48 * c);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const f32x4 v = p[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * i + e] = v[e];
      }
      return;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const f32x2* p = reinterpret_cast<const f32x2*>(wrow + 48 * c + 24 * g);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const f32x2 v = p[i];
        dst[6 * g + 2 * i] = v[0];
        dst[6 * g + 2 * i + 1] = v[1];
      }
    }
  };
  // B operand base of this lane: row 2lq, window column tz + l16 + delta
  const int boff = wz + 2 * lq * RS + tz + l16 + a.delta;
  // Winograd form: row 4lq, window column tl + delta (per-wave windows: tz = 0). Kept as
  // one integer offset from the buffer: written as a chain of pointer additions, the
  // compiler lost track of which buffer the reads use and waited for every buffer->LDS
  // load in flight, the next chunk's included, before each chunk.
  const int boffw = wz + 4 * lq * RS + a.delta + tl;
  // the chunk's 96 MFMAs of this wave on buffer zb, in six steps (tap k, half g); the B
  // operands of the next step are read while the current step's MFMAs run
  // Winograd form, the chunk's 64 MFMAs in four K-steps: step s takes input channel
  // 16c + 4lq + s (row 4lq + s). With the lattice inputs v0..v3 = x(t - pad + m*d) of a
  // pair (t, t + d) and its taps g:
  //   V = (v0 - v2, v1 + v2, v2 - v1, v1 - v3),  U = (g0, (g0 + g1 + g2)/2, (g0 - g1 + g2)/2, g2),
  //   M_j += U_j V_j;  y(t) = (M0 + M1) + M2,  y(t + d) = (M1 - M2) - M3.
  // Input step t - pad + m*d of the wave's output step t sits at window column
  // t + m*d + delta.
  auto compute_w = [&](const float* zb, const float (&gv)[12]) {
    const float* bp = zb + boffw;
    const int d = a.dil;
    auto read_b = [&](int st, float (&dst)[4][4]) {
      const float* p = bp + st * RS;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) dst[nb][m] = p[32 * nb + m * d];
    };
    float bx[2][4][4];
    read_b(0, bx[0]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (st + 1 < 4) read_b(st + 1, bx[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const float g0 = gv[3 * st], g1 = gv[3 * st + 1], g2 = gv[3 * st + 2];
      const float e02 = g0 + g2;
      const float u[4] = {g0, 0.5f * (e02 + g1), 0.5f * (e02 - g1), g2};
      // all of the step's transforms first, then its MFMAs back to back: interleaved,
      // each MFMA waited on the VALU op that formed its operand (about 10% slower)
      float vv[4][4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float* v = bx[st & 1][nb];
        vv[nb][0] = v[0] - v[2];
        vv[nb][1] = v[1] + v[2];
        vv[nb][2] = v[2] - v[1];
        vv[nb][3] = v[1] - v[3];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[4 * j + nb] =
              __builtin_amdgcn_mfma_f32_16x16x4f32(u[j], vv[nb][j], acc[4 * j + nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute = [&](const float* zb, const float (&wv)[12]) {
    if (!active) return;
    if constexpr (WINO) {
      compute_w(zb, wv);
      return;
    }
    const float* base = zb + boff;
    auto read_b = [&](int st, f32x2 (&dst)[GN_NB]) {
      const float* p = base + 8 * (st & 1) * RS + (st >> 1) * a.dil;
#pragma unroll
      for (int nb = 0; nb < GN_NB; ++nb) {
        dst[nb][0] = p[16 * nb];
        dst[nb][1] = p[16 * nb + RS];
      }
    };
    f32x2 bv[2][GN_NB];
    read_b(0, bv[0]);
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      if (st + 1 < 6) read_b(st + 1, bv[(st + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int k = st >> 1, g = st & 1;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int nb = 0; nb < GN_NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[6 * g + 3 * e + k], bv[st & 1][nb][e],
                                                         acc[nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // private windows: chunk c's window straight into this wave's area of buffer zb by
  // buffer->LDS loads; load i covers items 64i .. 64i + 63, i.e. floats VW*64*i on
  auto dma_x = [&](int c, float* zb) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(xn + (size_t)GN_CI * c * a.T), (short)0, 4 * GN_CI * a.T,
        kBufferFlags);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_to_lds<VW>(rs, zb + wz + 64 * VW * i, voff[i]);
  };
  // private windows, one chunk: the weights of chunk c + 1 and, into buffer zn (last read
  // by chunk c - 1), the window of chunk c + 1 go out; chunk c computes from buffer zc
  auto chunk_dma = [&](int c, const float* zc, float* zn, const float (&wc)[12],
                       float (&w1)[12]) {
    load_w(c + 1, w1);
    if (c + 1 < nC) dma_x(c + 1, zn);
    __builtin_amdgcn_sched_barrier(0);
    compute(zc, wc);
    chunk_sync();
  };
  // shared window, one chunk: the weights of chunk c + 1 and the x of chunk c + 2 go out,
  // chunk c computes from buffer zc, then chunk c + 1's x (loaded a chunk ago) goes to
  // buffer zn (last read by chunk c - 1, finished before the previous chunk_sync)
  auto chunk = [&](int c, const float* zc, float* zn, const float (&wc)[12], float (&w1)[12],
                   XV (&x2)[NX], const XV (&x1)[NX]) {
    load_w(c + 1, w1);
    load_x(min(c + 2, nC - 1), x2);
    __builtin_amdgcn_sched_barrier(0);
    compute(zc, wc);
    if (c + 1 < nC) store_x(x1, zn);
    chunk_sync();
  };

  // private windows: a wave past the end has nothing to stage for anyone
  if (PRIV && active) {
    float wA[12], wB[12];
    load_w(0, wA);
    dma_x(0, zA);
    int c = 0;
    for (; c + 1 < nC; c += 2) {
      chunk_dma(c, zA, zB, wA, wB);
      chunk_dma(c + 1, zB, zA, wB, wA);
    }
    if (c < nC) chunk_dma(c, zA, zB, wA, wB);
    // every buffer->LDS load has landed before the epilogue reuses the buffers
    __builtin_amdgcn_s_waitcnt(0x0f70);
  } else if (!PRIV) {
    float wA[12], wB[12];
    load_w(0, wA);
    load_x(0, xa);
    load_x(min(1, nC - 1), xb);
    store_x(xa, zA);
    chunk_sync();
    int c = 0;
    for (; c + 1 < nC; c += 2) {
      chunk(c, zA, zB, wA, wB, xa, xb);
      chunk(c + 1, zB, zA, wB, wA, xb, xa);
    }
    if (c < nC) chunk(c, zA, zB, wA, wB, xa, xb);
  }

  // Epilogue. Value y[i][r] of the lane is channel co0 + 4lq + r at step tw + col[i]: in
  // the three-tap form block i, step 16i + l16; in the Winograd form output h = i % 2 of the
  // pair in block nb = i / 2, step 32nb + tl + h*d.
  const int cpg = a.cpg;
  const double cnt = (double)cpg * (double)a.T_out;
  float y[GN_NB][4];
  int col[GN_NB];
  bool valid[GN_NB];
#pragma unroll
  for (int i = 0; i < GN_NB; ++i) {
    col[i] = WINO ? 32 * (i >> 1) + tl + (i & 1) * a.dil : 16 * i + l16;
    valid[i] = tw + col[i] < a.T_out;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float bco = a.bias ? a.bias[co0 + 4 * lq + r] : 0.f;
#pragma unroll
    for (int i = 0; i < GN_NB; ++i) {
      if constexpr (WINO) {
        const int nb = i >> 1;
        const float m0 = acc[nb][r], m1 = acc[4 + nb][r];
        const float m2 = acc[8 + nb][r], m3 = acc[12 + nb][r];
        y[i][r] = ((i & 1) ? (m1 - m2) - m3 : (m0 + m1) + m2) + bco;
      } else {
        y[i][r] = acc[i][r] + bco;
      }
    }
  }

  // pass 1: the group means. Every wave adds up the same partials in the same order
  // (group_total), so no further barrier is needed to share the result; lane l ends with
  // the total of the group of row l % 16, and a lane takes its rows' from lanes 0..15.
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float s = 0.f;
#pragma unroll
    for (int nb = 0; nb < GN_NB; ++nb) s += valid[nb] ? y[nb][r] : 0.f;
    s = quarterwave_sum(s);
    if (l16 == 0) red[w * 16 + 4 * lq + r] = s;
  }
  __syncthreads();
  const float gm = (float)(group_total(red, l, cpg) / cnt);
  float mean[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) mean[r] = __shfl(gm, 4 * lq + r);

  // pass 2: the biased variances, from the deviations about those means (into a second
  // partials array: other waves may still be reading the first)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float s = 0.f;
#pragma unroll
    for (int nb = 0; nb < GN_NB; ++nb) {
      const float dv = y[nb][r] - mean[r];
      s += valid[nb] ? dv * dv : 0.f;
    }
    s = quarterwave_sum(s);
    if (l16 == 0) red2[w * 16 + 4 * lq + r] = s;
  }
  __syncthreads();
  const float gr = (float)(1.0 / sqrt(group_total(red2, l, cpg) / cnt + (double)a.eps));
  float rstd[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rstd[r] = __shfl(gr, 4 * lq + r);

  // normalise and store: out = (y - mean) * rstd * gamma + beta
  float* __restrict__ outn = a.out + (size_t)n * a.C_out * a.T_out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int co = co0 + 4 * lq + r;
    const float ga = a.gamma ? a.gamma[co] : 1.f;
    const float be = a.beta ? a.beta[co] : 0.f;
    const float sc = rstd[r] * ga;
#pragma unroll
    for (int nb = 0; nb < GN_NB; ++nb) y[nb][r] = fmaf(y[nb][r] - mean[r], sc, be);
  }
  // Non-temporal stores: out is not read again here, and all workgroups write it at once.
  const bool vec_out = (a.T_out & 3) == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
  if (vec_out) {
    // Through the idle staging buffer zA, so that a lane stores 4 consecutive steps of one
    // channel (16 bytes) and 32 lanes one row's 128 steps (whole lines): each wave writes
    // and reads back only its own 16 x 128 block (rows 0..15 of its area, columns
    // tz..tz+127, inside a row of RS for an active wave); the statistics passes ended with
    // barriers, and a wave's LDS accesses complete in order. T_out is a multiple of 4, so
    // the 4 steps are all in range or all out.
    if (!active) return;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nb = 0; nb < GN_NB; ++nb) zA[wz + (4 * lq + r) * RS + tz + col[nb]] = y[nb][r];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int item = l + 64 * i;
      const int row = item >> 5, j = 4 * (item & 31), t = tw + j;
      const f32x4 v = *reinterpret_cast<const f32x4*>(&zA[wz + row * RS + tz + j]);
      if (t < a.T_out)
        __builtin_nontemporal_store(
            v, reinterpret_cast<f32x4*>(outn + (size_t)(co0 + row) * a.T_out + t));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* __restrict__ orow = outn + (size_t)(co0 + 4 * lq + r) * a.T_out;
#pragma unroll
      for (int nb = 0; nb < GN_NB; ++nb) {
        const int t = tw + col[nb];
        if (valid[nb]) __builtin_nontemporal_store(y[nb][r], &orow[t]);
      }
    }
  }
}

int gn_fused_groups(int T_out, int dil, int delta) {
  if (128LL + 2LL * dil + delta <= GN_PW) return GN_PRIVATE;
  const long long span = 128LL * ((T_out + 127) / 128) + 2LL * dil + delta;
  const int need = (int)((span + 63) / 64);
  for (int mg : {4, 8, 12, 17, 19})
    if (need <= mg) return mg;
  return 0;
}

bool gn_fused_vec4(int T, const void* x) {
  return T % 4 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
}

int gn_fused_delta(int pad, bool vec4) { return vec4 ? (4 - pad % 4) % 4 : 0; }

bool gn_fused_wino(int mg, int dil, const void* W) {
  return mg == GN_PRIVATE && (dil == 1 || dil == 2 || dil == 4) &&
         (reinterpret_cast<uintptr_t>(W) & 15) == 0;
}

bool gn_fused_fits(long long N, int C_in, int C_out, int T, int T_out, int pad, int dil, int cpg,
                   const void* x, const void* W) {
  const int delta = gn_fused_delta(pad, gn_fused_vec4(T, x));
  return T_out >= 1 && T_out <= 128 * GN_WAVES && dil <= 64 * GN_MG_MAX && C_in % GN_CI == 0 &&
         C_out % 16 == 0 && cpg >= 1 && 16 % cpg == 0 && gn_fused_groups(T_out, dil, delta) > 0 &&
         (reinterpret_cast<uintptr_t>(W) & 7) == 0 && N * (C_out / 16) <= 0x7fffffffLL;
}

template <int VW>
static void launch_mg(const GnFusedArgs& a, int mg, dim3 grid, dim3 block, hipStream_t stream) {
  switch (mg) {
    case GN_PRIVATE:
      if (a.wino)
        hipLaunchKernelGGL((conv_gn_fused_kernel<GN_PRIVATE, VW, true>), grid, block, 0, stream,
                           a);
      else
        hipLaunchKernelGGL((conv_gn_fused_kernel<GN_PRIVATE, VW, false>), grid, block, 0, stream,
                           a);
      break;
    case 4:
      hipLaunchKernelGGL((conv_gn_fused_kernel<4, VW, false>), grid, block, 0, stream, a);
      break;
    case 8:
      hipLaunchKernelGGL((conv_gn_fused_kernel<8, VW, false>), grid, block, 0, stream, a);
      break;
    case 12:
      hipLaunchKernelGGL((conv_gn_fused_kernel<12, VW, false>), grid, block, 0, stream, a);
      break;
    case 17:
      hipLaunchKernelGGL((conv_gn_fused_kernel<17, VW, false>), grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((conv_gn_fused_kernel<19, VW, false>), grid, block, 0, stream, a);
      break;
  }
}

hipError_t launch_conv_gn_fused(const GnFusedArgs& a, hipStream_t stream) {
  const long long nwg = (long long)a.N * a.n_cb;
  if (nwg <= 0) return hipSuccess;
  // the shape must be one the kernel's indexing covers (the host picks this path only then)
  const bool v4 = gn_fused_vec4(a.T, a.x);
  const int mg = gn_fused_groups(a.T_out, a.dil, a.delta);
  if (mg == 0 || a.mg != mg || a.vec4 != (int)v4 || a.delta != gn_fused_delta(a.pad, v4) ||
      a.T_out > 128 * GN_WAVES || a.C_in % GN_CI != 0 || a.n_cb * 16 != a.C_out || a.cpg < 1 ||
      16 % a.cpg != 0 || (a.wino && !gn_fused_wino(mg, a.dil, a.W)))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)nwg), block(64 * GN_WAVES);
  if (v4)
    launch_mg<4>(a, mg, grid, block, stream);
  else
    launch_mg<1>(a, mg, grid, block, stream);
  return hipGetLastError();
}

}  // namespace dconv1d
