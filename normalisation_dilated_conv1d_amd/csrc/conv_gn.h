// Declarations of the single-launch Conv1d + GroupNorm kernel (conv_gn.hip), shared with
// the C ABI (api.hip). Not part of the ABI.
#pragma once

#include "internal.h"

namespace dconv1d {

// conv_gn.hip: Conv1d + GroupNorm in one launch when every group fits in a workgroup of
// 16 output channels x T_out <= 1024 steps. The staged window is 64*mg steps wide
// (gn_fused_groups; 0 when no instantiated width covers the shape) and starts at input
// step -pad - delta; x is staged with 16-byte loads when gn_fused_vec4, and then delta
// (gn_fused_delta) aligns the window start to a multiple of 4. gn_fused_groups returns
// GN_PRIVATE instead when 128 + 2*dil + delta <= GN_PW: then each wave stages its own
// GN_PW-step window, from step 128*wave - pad - delta on.
constexpr int GN_MG_MAX = 19;
constexpr int GN_PRIVATE = 1;   // mg value of the per-wave windows
constexpr int GN_PW = 136;      // their width in steps (and LDS row pitch: 8 mod 16)
struct GnFusedArgs {
  const float* x;       // [N][C_in][T]
  const float* W;       // [C_out][C_in][3], 8-byte aligned
  const float* bias;    // [C_out] or nullptr
  const float* gamma;   // [C_out] or nullptr (1)
  const float* beta;    // [C_out] or nullptr (0)
  float* out;           // [N][C_out][T_out]
  float eps;
  int N, C_in, C_out, T, T_out;
  int pad, dil;         // tap k reads input t - pad + k*dil
  int cpg;              // channels per group (divides 16)
  int mg;               // staged window width in 64-step groups, or GN_PRIVATE
                        // (gn_fused_groups(...))
  int vec4;             // 16-byte x loads, gn_fused_vec4(T, x)
  int delta;            // window start shift, gn_fused_delta(pad, vec4)
  int n_cb;             // C_out / 16
  int wino;             // Winograd F(2,3) conv (gn_fused_wino(...)), else the three taps
};
int gn_fused_groups(int T_out, int dil, int delta);
bool gn_fused_vec4(int T, const void* x);
int gn_fused_delta(int pad, bool vec4);
// The Winograd form runs with per-wave windows, dil 1, 2 or 4 (pairs of outputs dil apart
// tile a wave's 128 steps) and W 16-byte aligned.
bool gn_fused_wino(int mg, int dil, const void* W);
bool gn_fused_fits(long long N, int C_in, int C_out, int T, int T_out, int pad, int dil, int cpg,
                   const void* x, const void* W);
hipError_t launch_conv_gn_fused(const GnFusedArgs& a, hipStream_t stream);

}  // namespace dconv1d
