// Internal declarations shared by the library's HIP translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dconv1d {

// K-chunk: 32 input channels of one tap. One chunk is one LDS stage.
constexpr int KC = 32;
// Output channels per workgroup of the largest float32 tile (4 waves x 64 channels),
// and the padding unit of the repacked output channels.
constexpr int CO_TILE_F32 = 256;
constexpr int NTHREADS = 256;

// Arguments of the float32 implicit-GEMM conv kernel. Sizes are int: the host checks
// that every per-sample index (C*L) fits in 31 bits; the sample offset is 64-bit.
struct ConvF32Args {
  const void* x;         // [N][C_in][L_in], float32 (bfloat16 bits for the bf16 kernel)
  const float* scale;    // [Cin_pad] folded BN scale (nullptr: no BN/ReLU on load)
  const float* shift;    // [Cin_pad] folded BN shift
  const float* Wp;       // repacked weights, see prep.hip
  const float* bias;     // [C_out] or nullptr
  void* out;             // [N][C_out][L_out], same storage type as x
  const void* residual;  // [N][C_out][L_out], same storage type as out; added by the
                         // residual epilogue (x for the block). May equal out exactly:
                         // each element is read by the thread that then writes it.
  float* partials;       // GroupNorm: [N][C_out][n_tt][3] (tile sum, centred sum of
                         // squares, count)
  int N, C_in, C_out, L_in, L_out;
  int pad, dil;          // tap k reads input t - pad + k*dil
  int NCB;               // 16-channel output blocks in the repacked weights (Cout_pad/16)
  int Q;                 // number of K-chunks = 3 * Cin_pad / KC
  int n_tt, n_ct;        // time tiles, output-channel tiles
};

enum ConvEpilogue { EPI_RESIDUAL = 0, EPI_GN_STATS = 1 };

inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

// Input step read by output step `s` (a tile start plus a column: below L_in + 2^10) at
// tap offset `off` = k*dil - pad (in [-L_in, L_in] for the block, whose padding is its
// dilation clamped to L_in). The sum is formed in unsigned arithmetic, whose wrap-around
// is defined, so it cannot overflow int when L_in is near 2^30; the result is below
// L_in exactly when the tap lies inside the input.
__device__ __forceinline__ uint32_t tap_step(int s, int off) {
  return (uint32_t)s + (uint32_t)off;
}

// prep.hip
hipError_t launch_prep_f32(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                           float* Wp, const float* running_mean, const float* running_var,
                           const float* gamma, const float* beta, float eps, float* scale,
                           float* shift, hipStream_t stream);

// conv_f32.hip
// Tile shape: tt time steps and 64*mb output channels per workgroup (float32 kernel:
// 4 waves of 16*mb channels; bf16 kernel: mb waves of 64 channels).
struct ConvTile {
  int tt, mb;
  int co_tile() const { return 64 * mb; }
};
hipError_t launch_conv_f32(const ConvF32Args& a, ConvTile tile, int epilogue, hipStream_t stream);

// prep.hip: BN fold + the Winograd weight transform, [Cin_pad/4 steps][Cout_pad/16][64] x 4
hipError_t launch_prep_wino(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                            float* Up, const float* running_mean, const float* running_var,
                            const float* gamma, const float* beta, float eps, float* scale,
                            float* shift, hipStream_t stream);
// conv_wino.hip: the float32 block by Winograd F(2,3) along the dilation lattice, for
// wino_supported(L) (L_in < 2^28; defined in api.hip with wino_pair_tiles and the choice
// of form and tiles); WINO_PAIRS output pairs and 64*wmb channels (wmb = 4, 2 or 1) per
// workgroup, a.n_tt = wino_pair_tiles(L, d), a.n_ct = ceil(C / (64*wmb)),
// a.Q = Cin_pad / KC, a.dil = a.pad = min(d, L)
constexpr int WINO_PAIRS = 32;
bool wino_supported(int L);
int wino_pair_tiles(int L, int dil);
// epilogue EPI_RESIDUAL (the block: BN in a.scale/a.shift, C_in == C_out) or EPI_GN_STATS
// (the conv of Conv1d + GroupNorm: a.scale null, partials [N][C_out][n_tt][3])
hipError_t launch_conv_wino(const ConvF32Args& a, int wmb, int epilogue, hipStream_t stream);

// conv_bf16.hip: 64-channel K-chunks, input channels padded to a multiple of 128 (an
// even chunk count), 128 time steps per tile
constexpr int KC_BF16 = 64;
constexpr int CIN_PAD_BF16 = 128;
constexpr int TILE_T_BF16 = 128;
hipError_t launch_prep_bf16(const float* W, int C_out, int C_in, int Cout_pad, int Cin_pad,
                            void* Wp, const float* running_mean, const float* running_var,
                            const float* gamma, const float* beta, float eps, float* scale,
                            float* shift, hipStream_t stream);
// Output channels per bf16 workgroup (256: 4 waves, or 512: 8 waves) for this shape;
// Cout_pad and n_ct follow from it, and launch_conv_bf16 takes the same value.
int conv_bf16_co_tile(long long N, int L_out, int C_out);
hipError_t launch_conv_bf16(const ConvF32Args& a, int co_tile, hipStream_t stream);

// bn_train.hip: training-mode BN statistics. Time steps of one (n, c) row per
// statistics workgroup; the partials hold one (sum, sum of squares) double pair per
// (channel, n, segment).
constexpr int STAT_SEG = 4096;
size_t bn_train_partials_bytes(int N, int C, int L);
// Writes scale/shift for channels [0, Cin_pad) (zero past C) from the batch statistics
// of x (float32, or bfloat16 bits when bf16), updates the running statistics when
// running_mean is non-null and stores the batch mean / inverse std when asked.
hipError_t launch_bn_train(const void* x, bool bf16, int N, int C, int L, int Cin_pad,
                           void* partials, const float* gamma, const float* beta, float eps,
                           float momentum, float* running_mean, float* running_var,
                           float* save_mean, float* save_invstd, float* scale, float* shift,
                           hipStream_t stream);

// gn.hip: partials [N][C_out][n_tt][3] (tile sum, centred sum of squares, count)
hipError_t launch_gn_normalize(float* out, const float* partials, const float* gamma,
                               const float* beta, float eps, int N, int C_out, int L_out,
                               int num_groups, int n_tt, hipStream_t stream);

}  // namespace dconv1d
