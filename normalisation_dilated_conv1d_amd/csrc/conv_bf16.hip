// bfloat16 implicit-GEMM kernel for the pre-norm residual block with bfloat16 storage of
// x and out (POPCORNBENCH "Kimi-K2.6__l2_p12", first turn: block definition, eval-mode
// BN per channel, zero padding of the conv input, residual add).
//
// Same GEMM view as the float32 kernel (conv_f32.hip): one workgroup per (sample, output
// channel tile, 128 time steps), one wave per 64 channels x 128 steps, activations
// through LDS, weights straight from global memory into registers. The channel tile is
// 256 (4 waves) or, for wide layers, 512 (8 waves): every wave of a workgroup reads the
// same staged activations, so the wider tile stages each x chunk once for twice the
// MFMA work and halves the staging each wave does. What changes for bfloat16:
//
//   MFMA       = v_mfma_f32_16x16x32_bf16: 16x16 output block, K = 32 per instruction,
//                float32 accumulation. A lane feeds 8 consecutive K values of one row
//                (A) and of one column (B), so both operands must be K-contiguous.
//   K loop     = chunks of 64 input channels of one tap (two MFMA K-steps), ordered
//                (channel block, tap); C_in is padded to 128 so the chunk count is even.
//   B operand  = the chunk's activations z = ReLU(BN(x)) rounded to bfloat16, staged
//                transposed in LDS as [time column][64 channel rows], so the 8 rows a lane
//                needs are 16 contiguous bytes: one ds_read_b128 per MFMA. Each staging
//                lane holds 8 consecutive rows of a column in registers and writes them
//                with one ds_write_b128.
//   A operand  = weights rounded to bfloat16 by the repack kernel and stored in lane
//                order: one 16-byte load per (K-step, 16-channel block) per lane, loaded
//                two K-steps ahead through a 4-slot register ring.
//   x loads    = buffer loads (row offset in an SGPR). When every tap offset and L are
//                even (the paired path), each lane loads two adjacent time steps with one
//                aligned 4-byte load, and the loads go straight into LDS (buffer->LDS
//                loads) two chunks ahead of their use, so x latency has two chunks to
//                hide in and no staging registers are held across the MFMAs; otherwise
//                two 2-byte loads into registers, one chunk ahead.
//   schedule   = (paired path) a chunk's buffer->LDS loads are issued one row per
//                16-column block among the first K-step's MFMAs rather than in one burst
//                after the barrier, B operands run three blocks ahead through a 4-deep
//                register ring, and with 8 waves the waves sharing a SIMD (w and w+4)
//                run in opposite order: waves 0-3 do their MFMAs and then stage the next
//                chunk, waves 4-7 stage first, so each SIMD has MFMAs to run while one of
//                its waves stages.
//
// K-slot mapping: in K-step s of a chunk, quarter-wave q = lane/16 element e (0..7) is
// chunk row 32s + 8q + e, for A and B alike, so the sum over K is the plain sum over
// (channel, tap).

#include "internal.h"

namespace dconv1d {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace

template <int V>
struct Parity {
  static constexpr int value = V;
};

constexpr int KCB = 64;   // channel rows per chunk (two MFMA K-steps)
// buffer resource word 3 for raw (untyped, unswizzled) buffers on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;
constexpr int TTB = TILE_T_BF16;  // time steps per workgroup

// WV waves (4 or 8) per workgroup, two waves per SIMD (at most 256 registers each)
template <bool PAIR, int WV>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * WV, 64 * WV),
                               amdgpu_waves_per_eu(2, 2)))
conv_bf16_kernel(ConvF32Args a) {
  static_assert(WV == 4 || WV == 8, "4 or 8 waves");
  constexpr int NB = TTB / 16;              // 16-column MFMA blocks per wave (8)
  constexpr int RPW = KCB / WV;             // staged rows per wave (16 or 8)
  constexpr int CO_T = 64 * WV;             // output channels per workgroup
  constexpr int PITCH = KCB + 8;            // bf16 per LDS column (144 bytes)
  // Staged activations, double-buffered. Two separate arrays (not one 2-D one) and, for
  // the paired path, two raw-x arrays: every LDS access below names its array directly,
  // so the compiler can tell them apart and, before reading or writing one of them, waits
  // only for the buffer->LDS loads into that same array, leaving the prefetch of the
  // other one in flight.
  __shared__ __attribute__((aligned(16))) uint16_t zsA[TTB * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t zsB[TTB * PITCH];
  // Paired path: the raw x rows (64 channels x 128 steps) of the chunks one and two
  // ahead; every wave fills and reads only its own RPW rows. With 8 waves the two raw
  // arrays also hold epilogue tiles of waves 4..7 (two 16 x (128+4) float tiles each),
  // so they are at least that large on both paths.
  constexpr int EP_TILE = 16 * (TTB + 4) * 2;     // one wave's epilogue tile, in uint16
  constexpr int RAW_X = PAIR ? KCB * TTB : 2;
  constexpr int RAWN = WV > 4 && 2 * EP_TILE > RAW_X ? 2 * EP_TILE : RAW_X;
  __shared__ __attribute__((aligned(16))) uint16_t raw0[RAWN];
  __shared__ __attribute__((aligned(16))) uint16_t raw1[RAWN];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int lq = l >> 4;
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
  const int t0 = tt * TTB;

  const uint16_t* __restrict__ xn =
      reinterpret_cast<const uint16_t*>(a.x) + (size_t)n * a.C_in * a.L_in;
  const u32x4* __restrict__ Wp4 = reinterpret_cast<const u32x4*>(a.Wp);
  const int cb0 = (ct * CO_T) / 16 + 4 * w;

  f32x4 acc[4][NB];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][nb][r] = 0.f;

  // Staging: wave w stages rows [RPW*w, RPW*w + RPW) of the chunk. PAIR: lane l covers columns
  // 2l and 2l+1 with one 4-byte load per row; otherwise columns l and l + 64, 2 bytes each.
  uint32_t xr[RPW * (PAIR ? 1 : 2)];
  float sc[RPW], sh[RPW];

  // x is read with buffer loads: the wave-uniform row offset goes in an SGPR and the
  // per-lane time offset is one register per chunk, so a load costs no vector address
  // arithmetic (the weights stay plain global loads: that measured faster).
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xn), (short)0, (int)(2u * (uint32_t)a.C_in * (uint32_t)a.L_in),
      kBufferFlags);
  // Byte offsets within one sample's x: C_in*L_in < 2^31 (checked on the host), so
  // 2*C_in*L_in fits 32 unsigned bits; the buffer takes them as raw 32-bit words.
  auto row_bytes = [&](int ci) { return (int)(2u * (uint32_t)ci * (uint32_t)a.L_in); };
  auto load_bn = [&](int q) {
    const int c = q / 3;
    // wave-uniform addresses: read through the constant address space so the
    // compiler issues scalar loads into SGPRs
    const __attribute__((address_space(4))) float* scp =
        (const __attribute__((address_space(4))) float*)(a.scale + c * KCB + RPW * w);
    const __attribute__((address_space(4))) float* shp =
        (const __attribute__((address_space(4))) float*)(a.shift + c * KCB + RPW * w);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      sc[i] = scp[i];
      sh[i] = shp[i];
    }
  };
  auto load_x = [&](int q) {
    const int c = q / 3, k = q - 3 * c;
    const int off = k * a.dil - a.pad;
    if (PAIR) {
      // a padded tap may read any in-range pair: store_z masks it to zero (with even
      // offsets and even L an in-range pair start is at most L_in - 2)
      const uint32_t ts = tap_step(t0 + 2 * l, off);
      const int vo = 2 * (ts < (uint32_t)a.L_in ? (int)ts : 0);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int ci = min(c * KCB + RPW * w + i, a.C_in - 1);
        xr[i] = __builtin_amdgcn_raw_buffer_load_b32(xres, vo, row_bytes(ci), 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t ts = tap_step(t0 + l + 64 * j, off);
        const int vo = 2 * (ts < (uint32_t)a.L_in ? (int)ts : 0);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int ci = min(c * KCB + RPW * w + i, a.C_in - 1);
          xr[j * RPW + i] = __builtin_amdgcn_raw_buffer_load_b16(xres, vo, row_bytes(ci), 0);
        }
      }
    }
    load_bn(q);
  };
  // Paired path: rows [i0, i0 + cnt) of chunk q's raw x rows of this wave, one row of 128
  // steps per load (64 lanes x 4 bytes), straight into LDS.
  auto dma_x0 = [&](int q, int i0 = 0, int cnt = KCB / WV) {
    const int c = q / 3, k = q - 3 * c;
    const uint32_t ts = tap_step(t0 + 2 * l, k * a.dil - a.pad);
    const int vo = 2 * (ts < (uint32_t)a.L_in ? (int)ts : 0);
#pragma unroll
    for (int i = i0; i < i0 + cnt; ++i) {
      const int ci = min(c * KCB + RPW * w + i, a.C_in - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)&raw0[(RPW * w + i) * TTB], 4, vo,
          row_bytes(ci), 0, 0);
    }
  };
  auto dma_x1 = [&](int q, int i0 = 0, int cnt = KCB / WV) {
    const int c = q / 3, k = q - 3 * c;
    const uint32_t ts = tap_step(t0 + 2 * l, k * a.dil - a.pad);
    const int vo = 2 * (ts < (uint32_t)a.L_in ? (int)ts : 0);
#pragma unroll
    for (int i = i0; i < i0 + cnt; ++i) {
      const int ci = min(c * KCB + RPW * w + i, a.C_in - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)&raw1[(RPW * w + i) * TTB], 4, vo,
          row_bytes(ci), 0, 0);
    }
  };
  // (one copy of the buffer->LDS load and of the read per raw array, so each access
  // names its array)
  auto read_raw0 = [&] {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      xr[i] = *reinterpret_cast<const uint32_t*>(&raw0[(RPW * w + i) * TTB + 2 * l]);
  };
  auto read_raw1 = [&] {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      xr[i] = *reinterpret_cast<const uint32_t*>(&raw1[(RPW * w + i) * TTB + 2 * l]);
  };
  // z = ReLU(scale*x + shift) in float32, rounded to bf16 by the hardware pack (round to
  // nearest even), exactly 0 in the time padding; 8 consecutive rows of one column go to
  // LDS with one 16-byte write. `get(i)` returns row i of the column as float, converted
  // straight from the loaded bits. Channels past C_in need no mask: their folded scale
  // and shift are 0, so z = max(0*x + 0, 0) = 0 for the clamped load, also when it is
  // infinite or NaN (max drops a NaN operand).
  auto stage_column = [&](auto&& get, int col, uint32_t tkeep, uint16_t* dst) {
#pragma unroll
    for (int half = 0; half < RPW / 8; ++half) {
      uint32_t packed[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int i0 = 8 * half + e, i1 = i0 + 1;
        const f32x2 z = {fmaxf(fmaf(get(i0), sc[i0], sh[i0]), 0.f),
                         fmaxf(fmaf(get(i1), sc[i1], sh[i1]), 0.f)};
        packed[e >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(z, bf16x2)) & tkeep;
      }
      u32x4 pv = {packed[0], packed[1], packed[2], packed[3]};
      *reinterpret_cast<u32x4*>(dst + col * PITCH + RPW * w + 8 * half) = pv;
    }
  };
  auto store_z = [&](int q, uint16_t* dst) {
    const int c = q / 3, k = q - 3 * c;
    const int off = k * a.dil - a.pad;
    if (PAIR) {
      // with even offsets and even L both time steps of the pair are in or out together
      uint32_t tkeep = tap_step(t0 + 2 * l, off) < (uint32_t)a.L_in ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(tkeep));
      stage_column([&](int i) { return bf16_lo(xr[i]); }, 2 * l, tkeep, dst);
      stage_column([&](int i) { return bf16_hi(xr[i]); }, 2 * l + 1, tkeep, dst);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = l + 64 * j;
        uint32_t tkeep = tap_step(t0 + col, off) < (uint32_t)a.L_in ? 0xffffffffu : 0u;
        asm volatile("" : "+v"(tkeep));
        stage_column([&](int i) { return bf16_to_f32((uint16_t)xr[j * RPW + i]); }, col, tkeep,
                     dst);
      }
    }
  };
  // A operands of global K-step S (chunk S/2, step S%2): one 16-byte unit per
  // 16-channel block. Clamped to the last step so prefetches past the end stay in bounds.
  const int n_steps = 2 * a.Q;
  auto load_w = [&](int S, u32x4 (&dst)[4]) {
    S = min(S, n_steps - 1);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) dst[mb] = Wp4[(S * a.NCB + cb0 + mb) * 64 + l];
  };
  auto load_b = [&](const uint16_t* zb, int s, int nb) -> bf16x8 {
    const u32x4 v =
        *reinterpret_cast<const u32x4*>(zb + (16 * nb + l16) * PITCH + 32 * s + 8 * lq);
    return __builtin_bit_cast(bf16x8, v);
  };

  // Weights rotate through a ring of 4 K-step slots, loaded two K-steps ahead. The chunk
  // count is even (C_in is padded to 128), so the loop takes two chunks per trip and
  // every slot index (2*parity + s) % 4 is a compile-time constant.
  // (The 2-byte-load variant holds twice the staging registers, so it keeps a 2-slot
  // ring loaded one K-step ahead.)
  constexpr int RING = PAIR ? 4 : 2;
  constexpr int DIST = PAIR ? 2 : 1;
  u32x4 wr[RING][4];

  // One chunk (two K-steps) on LDS buffer zb. `next` stages the next chunk into the
  // other buffer after the chunk's MFMAs, the latest point before the barrier, which
  // gives its x loads the longest time to arrive; on the paired path with 8 waves,
  // waves 4-7 (`early`) stage before their MFMAs instead. `dma(nb)` issues this wave's
  // buffer->LDS rows of a later chunk among the MFMAs of the first K-step's block nb
  // (paired path; the other path loads x into registers before the chunk).
  const bool early = PAIR && WV == 8 && w >= 4;
  auto compute = [&](const uint16_t* zb, int q, auto P, auto&& next, auto&& dma) {
    constexpr int par = decltype(P)::value;
    if constexpr (PAIR) {
      if (early) next();
      constexpr int BR = 4, BP = 3;
      bf16x8 bv[BR];
#pragma unroll
      for (int i = 0; i < BP; ++i) bv[i] = load_b(zb, i / NB, i % NB);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int S = 2 * q + s;
        load_w(S + DIST, wr[(2 * par + s + DIST) % RING]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int it = s * NB + nb;
          if (s == 0) dma(nb);
          if (it + BP < 2 * NB) bv[(it + BP) % BR] = load_b(zb, (it + BP) / NB, (it + BP) % NB);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wr[(2 * par + s) % RING][mb]), bv[it % BR],
                acc[mb][nb], 0, 0, 0);
          // block by block in this order: left free, the scheduler moved each B read
          // down to just before its MFMAs and waited on it there (1-2% slower)
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!early) next();
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int S = 2 * q + s;
        load_w(S + DIST, wr[(2 * par + s + DIST) % RING]);
        bf16x8 bv[2];
        bv[0] = load_b(zb, s, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (nb + 1 < NB) bv[(nb + 1) & 1] = load_b(zb, s, nb + 1);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wr[(2 * par + s) % RING][mb]), bv[nb & 1],
                acc[mb][nb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      next();
    }
  };

  // Two chunks per trip. The staged chunk index is clamped to the last chunk, so the
  // body has no branches; the last trip stages that chunk a second time into the idle
  // buffer.
  const int Q = a.Q;
#pragma unroll
  for (int S = 0; S < DIST; ++S) load_w(S, wr[S]);
  if constexpr (PAIR) {
    // Chunk q: run chunk q's MFMAs, issuing among them the buffer->LDS loads of chunk q+2
    // (into the raw array chunk q was staged from), and stage chunk q+1 from the other
    // raw array (loaded during chunk q-1). The barrier carries no memory fence: the release fence
    // of __syncthreads would wait for the chunk q+2 loads still in flight. Nothing needs
    // it: raw rows are read only by the wave that loaded them (the compiler waits for its
    // own loads before the read), and the staged z writes are complete once lgkmcnt is 0.
    // The memory clobber keeps the compiler from moving LDS accesses across it.
    auto bar = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    dma_x0(0);
    dma_x1(min(1, Q - 1));
    load_bn(0);
    read_raw0();
    store_z(0, zsA);
    bar();
    constexpr int RPI = RPW / NB;   // raw rows loaded per 16-column block of K-step 0
    for (int q = 0; q < Q; q += 2) {
      load_bn(q + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(zsA, q, Parity<0>{}, [&] {
        read_raw1();
        store_z(q + 1, zsB);
      }, [&](int it) { dma_x0(min(q + 2, Q - 1), it * RPI, RPI); });
      bar();
      const int qn = min(q + 2, Q - 1);
      load_bn(qn);
      __builtin_amdgcn_sched_barrier(0);
      compute(zsB, q + 1, Parity<1>{}, [&] {
        read_raw0();
        store_z(qn, zsA);
      }, [&](int it) { dma_x1(min(q + 3, Q - 1), it * RPI, RPI); });
      bar();
    }
  } else {
    load_x(0);
    store_z(0, zsA);
    __syncthreads();
    for (int q = 0; q < Q; q += 2) {
      load_x(q + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(zsA, q, Parity<0>{}, [&] { store_z(q + 1, zsB); }, [](int) {});
      __syncthreads();
      const int qn = min(q + 2, Q - 1);
      load_x(qn);
      __builtin_amdgcn_sched_barrier(0);
      compute(zsB, q + 1, Parity<1>{}, [&] { store_z(qn, zsA); }, [](int) {});
      __syncthreads();
    }
  }

  // Epilogue: register r of block (mb, nb) is channel 16mb + 4*lq + r, time 16nb + l16.
  // not restrict: the residual may be out itself (in-place residual add)
  uint16_t* outn = reinterpret_cast<uint16_t*>(a.out) + (size_t)n * a.C_out * a.L_out;
  const uint16_t* resn =
      reinterpret_cast<const uint16_t*>(a.residual) + (size_t)n * a.C_out * a.L_out;
  const int co_base = ct * CO_T + 64 * w + 4 * lq;
  const bool vec_epi = ((a.L_out & 7) == 0) &&
                       (((reinterpret_cast<uintptr_t>(a.out) |
                          reinterpret_cast<uintptr_t>(a.residual)) & 15) == 0);
  if (vec_epi) {
    // Each 16-channel block of accumulators goes through the staging LDS so that a lane
    // then owns 8 consecutive time steps of one channel: one 16-byte residual load and
    // one 16-byte store per 8 outputs instead of eight 2-byte ones. The loop ends with a
    // barrier (the chunk count is even), so every wave is done with the B operands; the
    // explicit one keeps that true should the loop change. The last trip's buffer->LDS
    // load into raw1 is never read: the wait before the barrier lets it land before
    // waves 6 and 7 put their tiles there. Every wave uses its own 16 x (128+4) float
    // tile; the LDS accesses of a wave complete in order, so no further barrier is needed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    constexpr int EP = TTB + 4;
    // two 16 x (128+4) float tiles (16.9 KB) fit in each 18.4 KB staging buffer and in
    // each raw array
    uint16_t* eb = w < 2 ? &zsA[0] : w < 4 ? &zsB[0] : w < 6 ? &raw0[0] : &raw1[0];
    float* ep = reinterpret_cast<float*>(eb) + (w & 1) * (16 * EP);
    const int co_w = ct * CO_T + 64 * w;
    // after the transpose, lane (lq, l16) holds rows lq + 4i (i = 0..3) of each block,
    // time steps t0 + 8*l16 .. +7
    float bia[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int coc = min(co_w + 16 * mb + lq + 4 * i, a.C_out - 1);
        bia[mb][i] = a.bias ? a.bias[coc] : 0.f;
      }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ep[(4 * lq + r) * EP + 16 * nb + l16] = acc[mb][nb][r];
      // residual loads (clamped in-bounds; L_out is a multiple of 8, so a clamped start
      // is too) go out before any use
      u32x4 rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int coc = min(co_w + 16 * mb + lq + 4 * i, a.C_out - 1);
        const int tcl = min(t0 + 8 * l16, a.L_out - 8);
        rv[i] = *reinterpret_cast<const u32x4*>(resn + (size_t)coc * a.L_out + tcl);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = lq + 4 * i;
        const int co = co_w + 16 * mb + row;
        const int t = t0 + 8 * l16;
        const float* src = ep + row * EP + 8 * l16;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(src + 4);
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 o = {v[2 * e] + bia[mb][i] + bf16_lo(rv[i][e]),
                           v[2 * e + 1] + bia[mb][i] + bf16_hi(rv[i][e])};
          pk[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2));
        }
        const u32x4 ov = {pk[0], pk[1], pk[2], pk[3]};
        // t and L_out are multiples of 8: the 8 steps are all in range or all out.
        // Non-temporal: out is not read again here, and with one workgroup per CU each
        // round ends in a burst of output writes that nothing overlaps; stores that do
        // not allocate in the caches shorten it (about 5% of the kernel).
        if (co < a.C_out && t < a.L_out)
          __builtin_nontemporal_store(
              ov, reinterpret_cast<u32x4*>(outn + (size_t)co * a.L_out + t));
      }
    }
  } else {
    // Residual and bias loads use clamped (always in-bounds) addresses and are issued a
    // 16-channel block at a time before any use, so each block pays the memory latency
    // once; only the stores are predicated.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      uint16_t res[4][NB];
      float bco[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int coc = min(co_base + 16 * mb + r, a.C_out - 1);
        bco[r] = a.bias ? a.bias[coc] : 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int tc = min(t0 + 16 * nb + l16, a.L_out - 1);
          res[r][nb] = resn[(size_t)coc * a.L_out + tc];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co_base + 16 * mb + r;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int t = t0 + 16 * nb + l16;
          if (co < a.C_out && t < a.L_out) {
            const float o = acc[mb][nb][r] + bco[r] + bf16_to_f32(res[r][nb]);
            __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)o),
                                        &outn[(size_t)co * a.L_out + t]);
          }
        }
      }
    }
  }
}

// Per-call preparation for the bf16 kernel, one launch: the BN fold (as in prep.hip:
// scale = gamma/sqrt(var+eps), shift = beta - mean*scale, in double, rounded once;
// skipped when scale is null, as in training mode where the statistics pass folds) and
// the weight repack W[C_out][C_in][3] float32 -> bfloat16 (round to nearest even) in
// A-operand lane order. Unit (16 bytes) index (S*NCB + cb)*64 + lane, with S = 2*q + s
// the global K-step (chunk q = 3*c + k: channel block c of 64, tap k) and cb the
// 16-channel block; element e of the unit is
//   W[16*cb + lane%16][64*c + 32*s + 8*(lane/16) + e][k]   (0 outside C_out x C_in).
__global__ void __launch_bounds__(256)
prep_bf16_kernel(const float* __restrict__ W, int C_out, int C_in, int NCB, int total,
                 u32x4* __restrict__ Wp, const float* __restrict__ mean,
                 const float* __restrict__ var, const float* __restrict__ gamma,
                 const float* __restrict__ beta, float eps, float* __restrict__ scale,
                 float* __restrict__ shift, int Cin_pad) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < total) {
    const int lane = idx & 63;
    const int rest = idx >> 6;
    const int cb = rest % NCB;
    const int S = rest / NCB;
    const int q = S >> 1, s = S & 1;
    const int c = q / 3, k = q - 3 * c;
    const int co = 16 * cb + (lane & 15);
    const int ci0 = KCB * c + 32 * s + 8 * (lane >> 4);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ci = ci0 + e;
      const float v = (co < C_out && ci < C_in) ? W[((size_t)co * C_in + ci) * 3 + k] : 0.f;
      h[e] = f32_to_bf16(v);
    }
    u32x4 o = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
               h[6] | (h[7] << 16)};
    Wp[idx] = o;
  }
  if (scale != nullptr && idx < Cin_pad) {
    float sc = 0.f, sh = 0.f;
    if (idx < C_in && gamma == nullptr) {
      sc = 1.f;                          // no normalisation: the stage applies ReLU only
    } else if (idx < C_in) {
      const double sd = (double)gamma[idx] / sqrt((double)var[idx] + (double)eps);
      sc = (float)sd;
      sh = (float)((double)beta[idx] - (double)mean[idx] * sd);
    }
    scale[idx] = sc;
    shift[idx] = sh;
  }
}

hipError_t launch_prep_bf16(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                            void* Wp, const float* running_mean, const float* running_var,
                            const float* gamma, const float* beta, float eps, float* scale,
                            float* shift, hipStream_t stream) {
  const int NCB = Cout_pad / 16;
  const long long total = 3LL * Cin_pad * Cout_pad / 8;   // 16-byte units of 8 bf16
  const long long threads = total > Cin_pad ? total : Cin_pad;
  const int blocks = (int)((threads + 255) / 256);
  hipLaunchKernelGGL(prep_bf16_kernel, dim3(blocks), dim3(256), 0, stream, W, C_out, C_in, NCB,
                     (int)total, reinterpret_cast<u32x4*>(Wp), running_mean, running_var, gamma,
                     beta, eps, scale, shift, Cin_pad);
  return hipGetLastError();
}

int conv_bf16_co_tile(long long N, int L_out, int C_out) {
  // The 512-channel tile when it pads C_out no further than the 256-channel one and its
  // grid still fills every CU at least once (one 8-wave workgroup per CU).
  const long long tiles512 = (C_out + 511) / 512;
  const long long wgs = N * ((L_out + TTB - 1) / TTB) * tiles512;
  return (round_up(C_out, 512) == round_up(C_out, 256) && wgs >= 256) ? 512 : 256;
}

hipError_t launch_conv_bf16(const ConvF32Args& a, int co_tile, hipStream_t stream) {
  const long long nwg = (long long)a.N * a.n_tt * a.n_ct;
  if (nwg <= 0) return hipSuccess;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // the repacked weights and the folded scale/shift must cover every channel the grid's
  // tiles touch
  if ((co_tile != 256 && co_tile != 512) || a.NCB * 16 < a.n_ct * co_tile)
    return hipErrorInvalidValue;
  // every tap offset and tile start is even, L is even and x is 4-byte aligned: each
  // lane can load an aligned pair of time steps
  const bool pair = ((a.dil | a.pad | a.L_in) & 1) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.x) & 3) == 0;
  const dim3 grid((unsigned)nwg);
  if (co_tile == 512) {
    if (pair)
      hipLaunchKernelGGL((conv_bf16_kernel<true, 8>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((conv_bf16_kernel<false, 8>), grid, dim3(512), 0, stream, a);
  } else {
    if (pair)
      hipLaunchKernelGGL((conv_bf16_kernel<true, 4>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((conv_bf16_kernel<false, 4>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dconv1d
