// C ABI of the library (declared in include/dconv1d.h): argument validation, the
// per-device workspace, kernel launches and the optional kernel timer.
//
// Validation follows the checks of the pages' host wrappers (POPCORNBENCH
// "Kimi-K2.6__l2_p12", first turn: device/contiguity checks, kernel size 3 with
// padding = dilation so the output keeps length L, 32-bit index limits; and
// "FW-GLM-5-1__l2_p35": output length T + 2p - d(k-1), channels divisible by groups),
// restated as status codes instead of exceptions.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "dconv1d.h"
#include "conv_gn.h"
#include "internal.h"

using namespace dconv1d;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DCONV1D_EHIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return abytes > 0 && bbytes > 0 && a0 < b0 + bbytes && b0 < a0 + abytes;
}

// ---------------------------------------------------------------- per-device workspace
// One workspace per device holds what a call's kernels share (folded BN vectors,
// repacked weights, partial statistics). Calls on different streams of one device would
// race on it, so every call that uses it holds the device's lock while it queues its
// kernels, waits (on the device, through an event, without blocking the host) for the
// last call that used it when that call ran on another stream, and records the event
// after its own last kernel.
constexpr int kMaxDevices = 64;
struct Workspace {
  std::mutex mu;
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;   // recorded after the last call's last kernel
  hipStream_t last = nullptr;  // the stream that call ran on
  bool pending = false;        // `done` has been recorded
};
Workspace g_ws[kMaxDevices];

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// Holds a device's workspace for the duration of one call.
class WorkspaceUse {
 public:
  // Locks the current device's workspace, grows it to at least `bytes` and orders
  // `stream` after the previous user of the workspace. On success *out is the
  // workspace. Under stream capture the event ordering is skipped (an event recorded or
  // waited on across the capture boundary is not allowed): captured calls are ordered
  // against other streams by the caller.
  int acquire(size_t bytes, hipStream_t stream, char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DCONV1D_EINVAL, "device %d out of range", dev);
    w_ = &g_ws[dev];
    lock_ = std::unique_lock<std::mutex>(w_->mu);
    stream_ = stream;
    captured_ = capturing(stream);
    if (w_->bytes < bytes) {
      if (w_->ptr) {
        // earlier calls may still be using the old buffer
        e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        (void)hipFree(w_->ptr);
        w_->ptr = nullptr;
        w_->bytes = 0;
      }
      const size_t sz = (bytes + (size_t(2) << 20) - 1) & ~((size_t(2) << 20) - 1);
      e = hipMalloc(&w_->ptr, sz);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        w_->ptr = nullptr;
        return fail(DCONV1D_ENOMEM, "workspace hipMalloc of %zu bytes failed: %s", sz,
                    hipGetErrorString(e));
      }
      w_->bytes = sz;
    }
    if (!captured_) {
      if (!w_->done) {
        e = hipEventCreateWithFlags(&w_->done, hipEventDisableTiming);
        if (e != hipSuccess) {
          w_->done = nullptr;
          return hip_fail(e, "hipEventCreateWithFlags");
        }
      }
      if (w_->pending && w_->last != stream) {
        e = hipStreamWaitEvent(stream, w_->done, 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
      }
    }
    held_ = true;
    *out = static_cast<char*>(w_->ptr);
    return DCONV1D_OK;
  }
  // Marks the end of this call's use (after its last kernel is queued, or after a failed
  // launch: whatever was queued still uses the workspace).
  ~WorkspaceUse() {
    if (!held_ || captured_) return;
    if (hipEventRecord(w_->done, stream_) == hipSuccess) {
      w_->last = stream_;
      w_->pending = true;
    } else {
      // without the event later calls cannot be ordered after this one: wait here
      (void)hipStreamSynchronize(stream_);
      w_->pending = false;
    }
  }

 private:
  Workspace* w_ = nullptr;
  std::unique_lock<std::mutex> lock_;
  hipStream_t stream_ = nullptr;
  bool captured_ = false;
  bool held_ = false;
};

// ---------------------------------------------------------------- fixed scratch array
// prenorm_dconv1d_fwd_noalloc keeps its folded BN vectors and repacked weights in this
// fixed device array instead of the workspace, so that it never allocates. It is sized
// for the float32 layout prenorm_common uses (scale, shift, repacked W, each 256-byte
// aligned) at C = kNoallocMaxC: 2 KiB + 2 KiB + 4 MiB (the four Winograd transforms;
// the direct kernel's three taps take 3 MiB). Every device the library runs on
// holds its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: the device address comes from hipGetSymbolAddress, looked
// up once per device (with that device current) and kept in g_scratch_ptr.
constexpr int64_t kNoallocMaxC = 512;
constexpr size_t kScratchBytes = 2 * (4 * kNoallocMaxC) + 4 * 4 * size_t(kNoallocMaxC) * kNoallocMaxC;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DCONV1D_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "hipGetSymbolAddress of the scratch array");
    }
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return DCONV1D_OK;
}

// ---------------------------------------------------------------- kernel timer
constexpr int kTimerSlots = 4096;
struct Timer {
  bool on = false;
  int device = -1;
  std::vector<hipEvent_t> ev;  // 2 per slot
  int used = 0;
};
std::mutex g_timer_mu;
Timer g_timer;

int timer_begin(hipStream_t s) {
  std::lock_guard<std::mutex> lock(g_timer_mu);
  if (!g_timer.on || g_timer.used >= kTimerSlots) return -1;
  const int slot = g_timer.used++;
  if (hipEventRecord(g_timer.ev[2 * slot], s) != hipSuccess) return -1;
  return slot;
}
void timer_end(int slot, hipStream_t s) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  (void)hipEventRecord(g_timer.ev[2 * slot + 1], s);
}

}  // namespace

// ---------------------------------------------------------------- algorithm choice
namespace dconv1d {

// The kernel runs any dilation; two rows' byte offsets must fit 32 bits.
bool wino_supported(int L) { return L >= 1 && L < (1 << 28); }

// Channel tiles. Both float32 kernels take 64*mb output channels per workgroup, mb = 4, 2
// or 1 (16-channel blocks per wave), and run their MFMAs at nearly one rate whatever the
// tile (the smaller ones with more workgroups per CU). So the fastest tile is the one with
// the least padded channel work, weighted by the tiles' relative rates; a tile's cost is
// its padded channel count divided by its rate (times 100).
namespace {

struct ChannelTile {
  int mb;
  long long cost;
};

ChannelTile best_channel_tile(int C, const int (&rate)[3]) {
  static const int mbs[3] = {4, 2, 1};
  ChannelTile best{4, -1};
  for (int i = 0; i < 3; ++i) {
    const long long cot = 64LL * mbs[i];
    const long long cost = (C + cot - 1) / cot * cot * 10000 / rate[i];
    if (best.cost < 0 || cost < best.cost) best = {mbs[i], cost};
  }
  return best;
}

// Relative rates of mb = 4, 2, 1. Direct kernel, measured on C = 256 and 512 (N = 32,
// L = 4096, d = 128): 1 : 0.98 : 0.95. On that shape with C = 64 the direct kernel took
// 38 us with mb = 1 against 119 us with mb = 4, C = 192 249 against 311 us, C = 320 661
// against 992 us (mb = 2: 764 us), while C = 256 stays at mb = 4 (407 against 430 us).
constexpr int kRateDirect[3] = {100, 98, 95};
// Winograd kernel, measured the same way (C = 256: 297, 309, 320 us; C = 512 at N = 16:
// 576, 602, 622 us): 1 : 0.96 : 0.93. With C = 64 it took 33 us with mb = 1 against 90 us
// with mb = 4, C = 128 88 us with mb = 2 (mb = 1: 90, mb = 4: 157), C = 192 187 us with
// mb = 1 against 229 us, C = 320 492 us with mb = 1 against 716 us.
constexpr int kRateWino[3] = {100, 96, 93};

// output pairs of the Winograd form: every pair of the super-blocks that cover [0, L)
long long wino_pairs(int L, int dil) {
  const long long d = dil < L ? dil : L;
  return ((long long)L + 2 * d - 1) / (2 * d) * d;
}

}  // namespace

// Channel tile of the Winograd kernel: the cheapest one by the cost above, halved while
// the grid has fewer than two workgroups per CU (512), as the direct kernel does: at
// N = 1 and 2 (C = 256, L = 4096, d = 128) 64-channel tiles took 21 and 28 us against 44
// and 44 us with 256-channel tiles (the direct kernel's best: 25 and 37 us).
int wino_channel_blocks(long long N, int C, int L, int dil) {
  const long long pair_tiles = wino_pair_tiles(L, dil < L ? dil : L);
  int mb = best_channel_tile(C, kRateWino).mb;
  while (mb > 1 && N * pair_tiles * ((C + 64LL * mb - 1) / (64LL * mb)) < 512) mb /= 2;
  return mb;
}

// Tile shape of the direct float32 kernel: the channel tile above with 128 time steps when
// that gives at least two workgroups per CU (512), else with 64; when even that leaves
// one wave per SIMD, half the channel tile (more, smaller workgroups, each x tile read
// once more), down to 64 channels.
ConvTile conv_f32_tile(int L_out, int N, int C_out) {
  auto wgs = [&](int tt, int cot) {
    return (long long)N * ((L_out + tt - 1) / tt) * ((C_out + cot - 1) / cot);
  };
  for (int mb = best_channel_tile(C_out, kRateDirect).mb;; mb /= 2) {
    if (wgs(128, 64 * mb) >= 512) return {128, mb};
    if (wgs(64, 64 * mb) >= 512 || mb == 1) return {64, mb};
  }
}

// A grid runs in rounds of (workgroups per CU) x 256 workgroups; a grid that overruns a
// whole number of rounds leaves most CUs idle in its last one. The factor by which that
// stretches the grid's time, with the workgroups per CU each tile fits in its registers
// (Winograd 242, 148, 108 VGPRs at mb = 4, 2, 1: 2, 3, 4 per CU; direct kernel at 128
// steps 239, 160, 124: 2, 3, 4; at 64 steps 144, 96, 72: 3, 5, 7). L = 1024, d = 97,
// N = 32, C = 256: 544 Winograd workgroups (two rounds, the second nearly empty) took
// 131.5 us against the direct kernel's 122.2 us in exactly one round of 512.
// A grid of less than one round is left at 1: its time is one workgroup's, which the
// channel-tile costs already compare.
static double round_factor(long long wgs, int per_cu) {
  const double rounds = (double)wgs / (256.0 * per_cu);
  return rounds >= 1.0 ? std::ceil(rounds) / rounds : 1.0;
}

static int wino_per_cu(int mb) { return mb == 4 ? 2 : mb == 2 ? 3 : 4; }
static int direct_per_cu(ConvTile t) {
  if (t.tt == 128) return t.mb == 4 ? 2 : t.mb == 2 ? 3 : 4;
  return t.mb == 4 ? 3 : t.mb == 2 ? 5 : 7;
}

// Whether the Winograd form is the faster one. It computes 4 products per output pair
// and input channel, over every pair of the super-blocks that cover [0, L); the direct
// form 3 per output step, and at equal channel tiles it runs its MFMAs at a higher rate
// (about 0.81 of the peak against 0.74). So the Winograd form needs at most 2L/3 pairs
// (every dilation up to L/2 that tiles L into whole super-blocks gives L/2; dilations
// close to L or above it give more, as most pairs' second output then lies past the
// end), scaled by the two forms' channel-tile costs. Measured on C=256 L=4096 against the
// direct kernel's 404 us at N=32: d = 3 to 300 348-373 us, d = 2500 (P = 0.61 L) 382 us,
// d = 1500 (P = 0.73 L) 453 us. Small grids take smaller channel tiles in both kernels
// (wino_channel_blocks, conv_f32_tile), and the Winograd form stays ahead there too:
// N = 1, 2 at d = 128 above; N = 1, C = 512, L = 4096, d = 8: 48 against 67 us; N = 4,
// C = 128, L = 1024, d = 16: 13 against 15 us; N = 2, C = 64, L = 2048, d = 4: 9.3
// against 10.1 us.
bool wino_faster(long long N, int C, int L, int dil) {
  if (!wino_supported(L) || dil < 1 || N < 1 || C < 1) return false;
  const ChannelTile w = best_channel_tile(C, kRateWino);
  const ChannelTile f = best_channel_tile(C, kRateDirect);
  // the grids each form launches, for the round factor
  const int d = dil < L ? dil : L;
  const int wmb = wino_channel_blocks(N, C, L, d);
  const long long wgs_w = N * wino_pair_tiles(L, d) * ((C + 64LL * wmb - 1) / (64LL * wmb));
  const ConvTile t = conv_f32_tile(L, (int)std::min<long long>(N, 0x7fffffffLL), C);
  const long long wgs_d = N * ((L + t.tt - 1) / t.tt) * ((C + t.co_tile() - 1) / t.co_tile());
  return 3.0 * wino_pairs(L, dil) * w.cost * round_factor(wgs_w, wino_per_cu(wmb)) <=
         2.0 * L * f.cost * round_factor(wgs_d, direct_per_cu(t));
}

// Pair tiles to launch. Pair p's first output step 2d*(p/d) + p%d grows with p, so the
// pairs with an output in range are a prefix, d*floor(L/2d) + min(d, L mod 2d) of them;
// tiles past it would compute nothing (L = 1024, d = 97: 17 tiles instead of the 19 that
// cover every super-block). The choice of form still counts every super-block's pairs.
int wino_pair_tiles(int L, int dil) {
  const long long d = dil;
  const long long pairs = d * (L / (2 * d)) + std::min<long long>(d, L % (2 * d));
  return (int)((pairs + WINO_PAIRS - 1) / WINO_PAIRS);
}

}  // namespace dconv1d

namespace {

// DCONV1D_WINOGRAD in the environment, read at every call: 0 or 1 when it is "0" or "1",
// else -1 (unset or anything else)
int winograd_override() {
  const char* v = std::getenv("DCONV1D_WINOGRAD");
  if (v != nullptr && (v[0] == '0' || v[0] == '1') && v[1] == '\0') return v[0] - '0';
  return -1;
}

// The float32 block's conv form: Winograd when the kernel can run the shape and is the
// faster one. DCONV1D_WINOGRAD overrides that: "0" the direct kernel always, "1" the
// Winograd kernel whenever it can run the shape (e.g. to compare the two, or to test the
// Winograd kernel on small shapes).
bool use_winograd(int64_t N, int C, int L, int d_eff) {
  const int o = winograd_override();
  if (o == 0) return false;
  if (o == 1) return wino_supported(L);
  return wino_faster((long long)N, C, L, d_eff);
}

// The conv form of the two-kernel Conv1d + GroupNorm path: the Winograd kernel needs the
// block's lattice, padding = dilation (so T_out = T), and is taken as for the block (the
// channel tiles follow C_out); DCONV1D_WINOGRAD overrides the same way. Sizes as
// validated by conv1d_groupnorm_fwd (T < 2^29).
bool gn_two_kernel_winograd(int64_t N, int64_t C_out, int64_t T, int64_t padding,
                            int64_t dilation) {
  if (padding != dilation) return false;
  return use_winograd(N, (int)C_out, (int)T, (int)std::min<int64_t>(dilation, T));
}

// ---------------------------------------------------------------- shared checks
constexpr int64_t kMaxChannels = 16384;
constexpr int64_t kMaxIndex = (int64_t(1) << 31) - 1;

int check_sizes_block(int64_t N, int64_t C, int64_t L, int64_t d, float eps) {
  if (N < 0) return fail(DCONV1D_EINVAL, "N must be >= 0 (got %lld)", (long long)N);
  if (C < 1 || C > kMaxChannels)
    return fail(DCONV1D_EINVAL, "C must be in [1, %lld] (got %lld)", (long long)kMaxChannels,
                (long long)C);
  if (L < 1 || L >= (int64_t(1) << 30))
    return fail(DCONV1D_EINVAL, "L must be in [1, 2^30) (got %lld)", (long long)L);
  if (d < 1) return fail(DCONV1D_EINVAL, "dilation d must be >= 1 (got %lld)", (long long)d);
  if (!(eps >= 0.f) || std::isinf(eps))
    return fail(DCONV1D_EINVAL, "eps must be finite and >= 0");
  if (C * L > kMaxIndex)
    return fail(DCONV1D_EINVAL, "C*L = %lld exceeds 2^31-1", (long long)(C * L));
  return DCONV1D_OK;
}

// Training-mode BN arguments (null for the eval-mode entry points).
struct TrainBn {
  float momentum;
  float* running_mean;  // nullable together with running_var: no running update
  float* running_var;
  float* save_mean;     // nullable
  float* save_invstd;   // nullable
};

// How the block's conv input is normalised.
enum class Norm { Eval, Train, External };

// The three block variants. x is the conv input and residual the tensor added to the
// conv output (x itself for Eval and Train; for External x is the caller's normalised
// activation, and gamma, beta and the running statistics are unused).
template <typename XT>
int prenorm_common(const XT* x, const XT* residual, const float* running_mean,
                   const float* running_var, const float* gamma, const float* beta, float eps,
                   const float* W, const float* b, XT* out, int64_t N, int64_t C, int64_t L,
                   int64_t d, hipStream_t stream, bool bf16, Norm norm, const TrainBn* train,
                   bool fixed_scratch = false) {
  // an empty batch has no data: x and out may then be NULL (torch gives empty tensors
  // a null data pointer)
  if (!x && N != 0) return fail(DCONV1D_EINVAL, "x is NULL");
  if (norm == Norm::External) {
    if (!residual && N != 0) return fail(DCONV1D_EINVAL, "residual is NULL");
  } else if (train) {
    if ((running_mean == nullptr) != (running_var == nullptr))
      return fail(DCONV1D_EINVAL, "running_mean and running_var must both be given or both NULL");
    if (!std::isfinite(train->momentum)) return fail(DCONV1D_EINVAL, "momentum must be finite");
  } else {
    if (!running_mean) return fail(DCONV1D_EINVAL, "running_mean is NULL");
    if (!running_var) return fail(DCONV1D_EINVAL, "running_var is NULL");
  }
  if (norm != Norm::External) {
    if (!gamma) return fail(DCONV1D_EINVAL, "gamma is NULL");
    if (!beta) return fail(DCONV1D_EINVAL, "beta is NULL");
  }
  if (!W) return fail(DCONV1D_EINVAL, "W is NULL");
  if (!out && N != 0) return fail(DCONV1D_EINVAL, "out is NULL");
  int st = check_sizes_block(N, C, L, d, eps);
  if (st != DCONV1D_OK) return st;
  if (fixed_scratch && C > kNoallocMaxC)
    return fail(DCONV1D_EINVAL, "C = %lld exceeds the %lld channels the no-allocation "
                "entry point's fixed scratch array holds", (long long)C,
                (long long)kNoallocMaxC);
  const int64_t per_sample = C * L;
  if (N > INT64_MAX / (per_sample * (int64_t)sizeof(XT)))
    return fail(DCONV1D_EINVAL, "N*C*L overflows");
  const uint64_t bytes = (uint64_t)N * per_sample * sizeof(XT);
  if (overlaps(x, bytes, out, bytes))
    return fail(DCONV1D_EALIAS, norm == Norm::External ? "out overlaps xn" : "out overlaps x");
  // out may be the residual itself (each element is read by the thread that writes
  // it), but not a shifted view of it
  if (norm == Norm::External && out != residual && overlaps(residual, bytes, out, bytes))
    return fail(DCONV1D_EALIAS, "out partially overlaps residual");
  if (train) {
    if (N != 0 && N * L < 2)
      return fail(DCONV1D_EINVAL, "training-mode BN needs more than one value per channel "
                                  "(N*L = %lld)", (long long)(N * L));
    // vectors written by the statistics pass must not overlap x, out or each other
    const void* outs[4] = {train->running_mean, train->running_var, train->save_mean,
                           train->save_invstd};
    const char* names[4] = {"running_mean", "running_var", "save_mean", "save_invstd"};
    const uint64_t vb = 4 * (uint64_t)C;
    for (int i = 0; i < 4; ++i) {
      if (!outs[i]) continue;
      if (overlaps(outs[i], vb, x, bytes) || overlaps(outs[i], vb, out, bytes))
        return fail(DCONV1D_EALIAS, "%s overlaps x or out", names[i]);
      for (int j = 0; j < i; ++j)
        if (outs[j] && overlaps(outs[i], vb, outs[j], vb))
          return fail(DCONV1D_EALIAS, "%s overlaps %s", names[i], names[j]);
    }
  }

  const int Ci = (int)C, Li = (int)L;
  // d >= L: both outer taps are always in the padding; d = L gives the same result and
  // keeps every tap offset inside int range.
  const int d_eff = (int)std::min<int64_t>(d, L);
  // float32 storage takes the Winograd kernel when use_winograd says so (32 output pairs
  // and the channel tile wino_channel_blocks picks), else the direct kernel with the tile
  // conv_f32_tile picks; bf16 storage runs the bf16-MFMA kernel: 64-channel K-chunks,
  // 128-step time tiles (a 256- or 512-channel tile). The repacked weights are padded to
  // whole 256-channel tiles (every smaller tile divides 256).
  const bool wino = !bf16 && use_winograd(N, Ci, Li, d_eff);
  const int Cin_pad = round_up(Ci, bf16 ? CIN_PAD_BF16 : KC);
  const int co_tile_bf16 = bf16 ? conv_bf16_co_tile(N, Li, Ci) : 0;
  const int Cout_pad = round_up(Ci, bf16 ? co_tile_bf16 : CO_TILE_F32);
  const ConvTile tile = bf16 ? ConvTile{TILE_T_BF16, co_tile_bf16 / 64}
                        : wino ? ConvTile{0, wino_channel_blocks(N, Ci, Li, d_eff)}
                               : conv_f32_tile(Li, (int)std::min<int64_t>(N, kMaxIndex), Ci);
  const int n_ct = (Ci + tile.co_tile() - 1) / tile.co_tile();
  const int n_tt = wino ? wino_pair_tiles(Li, d_eff) : (Li + tile.tt - 1) / tile.tt;
  if (N * n_tt * n_ct > kMaxIndex)
    return fail(DCONV1D_EINVAL, "grid of %lld workgroups is too large",
                (long long)(N * n_tt * n_ct));
  if (train && N * C * ((L + STAT_SEG - 1) / STAT_SEG) > kMaxIndex)
    return fail(DCONV1D_EINVAL, "statistics grid is too large");
  if (N == 0) return DCONV1D_OK;

  // repacked weights: three taps, or the four Winograd transforms
  const size_t wp_bytes = (bf16 ? 2 : 4) * (wino ? 4 : 3) * (size_t)Cin_pad * Cout_pad;
  const size_t off_scale = 0;
  const size_t off_shift = align256(off_scale + sizeof(float) * Cin_pad);
  const size_t off_wp = align256(off_shift + sizeof(float) * Cin_pad);
  const size_t off_part = align256(off_wp + wp_bytes);
  const size_t part_bytes = train ? bn_train_partials_bytes((int)N, Ci, Li) : 0;
  const size_t total = align256(off_part + part_bytes);
  char* ws = nullptr;
  WorkspaceUse use;
  if (fixed_scratch) {
    if (total > kScratchBytes)   // not reached: C <= kNoallocMaxC fits by construction
      return fail(DCONV1D_EINVAL, "scratch of %zu bytes needed, %zu available", total,
                  kScratchBytes);
    st = scratch_address(&ws);
  } else {
    st = use.acquire(total, stream, &ws);
  }
  if (st != DCONV1D_OK) return st;
  float* scale = reinterpret_cast<float*>(ws + off_scale);
  float* shift = reinterpret_cast<float*>(ws + off_shift);
  void* Wp = ws + off_wp;

  hipError_t e;
  if (train) {
    e = launch_bn_train(x, bf16, (int)N, Ci, Li, Cin_pad, ws + off_part, gamma, beta, eps,
                        train->momentum, train->running_mean, train->running_var,
                        train->save_mean, train->save_invstd, scale, shift, stream);
    if (e != hipSuccess) return hip_fail(e, "batch statistics kernel launch");
  }
  // Eval folds the running statistics here, External gets scale 1 / shift 0 (null
  // gamma), and Train only repacks W (the statistics pass folded already).
  float* fold_scale = train ? nullptr : scale;
  float* fold_shift = train ? nullptr : shift;
  const float* fold_gamma = norm == Norm::External ? nullptr : gamma;
  e = bf16 ? launch_prep_bf16(W, Ci, Ci, Cout_pad, Cin_pad, Wp, running_mean, running_var,
                              fold_gamma, beta, eps, fold_scale, fold_shift, stream)
      : wino ? launch_prep_wino(W, Ci, Ci, Cout_pad, Cin_pad, static_cast<float*>(Wp),
                                running_mean, running_var, fold_gamma, beta, eps, fold_scale,
                                fold_shift, stream)
             : launch_prep_f32(W, Ci, Ci, Cout_pad, Cin_pad, static_cast<float*>(Wp), running_mean,
                               running_var, fold_gamma, beta, eps, fold_scale, fold_shift, stream);
  if (e != hipSuccess) return hip_fail(e, "prep kernel launch");

  ConvF32Args a{};
  a.x = x;
  a.scale = scale;
  a.shift = shift;
  a.Wp = static_cast<const float*>(Wp);
  a.bias = b;
  a.out = out;
  a.residual = norm == Norm::External ? residual : x;
  a.partials = nullptr;
  a.N = (int)N;
  a.C_in = Ci;
  a.C_out = Ci;
  a.L_in = Li;
  a.L_out = Li;
  a.pad = d_eff;
  a.dil = d_eff;
  a.NCB = Cout_pad / 16;
  a.Q = wino ? Cin_pad / KC : 3 * Cin_pad / (bf16 ? KC_BF16 : KC);
  a.n_tt = n_tt;
  a.n_ct = n_ct;
  const int slot = timer_begin(stream);
  e = bf16 ? launch_conv_bf16(a, tile.co_tile(), stream)
      : wino ? launch_conv_wino(a, tile.mb, EPI_RESIDUAL, stream)
             : launch_conv_f32(a, tile, EPI_RESIDUAL, stream);
  timer_end(slot, stream);
  if (e != hipSuccess) return hip_fail(e, "conv kernel launch");
  return DCONV1D_OK;
}

}  // namespace

extern "C" {

int dconv1d_block_method(int64_t N, int64_t C, int64_t L, int64_t d) {
  if (N < 0 || C < 1 || C > kMaxChannels || L < 1 || d < 1) return DCONV1D_EINVAL;
  if (L >= (int64_t(1) << 30) || N == 0) return DCONV1D_METHOD_DIRECT;
  const int d_eff = (int)std::min<int64_t>(d, L);
  return use_winograd(N, (int)C, (int)L, d_eff) ? DCONV1D_METHOD_WINOGRAD
                                                : DCONV1D_METHOD_DIRECT;
}

int dconv1d_groupnorm_method(const float* x, const float* W, int64_t num_groups, int64_t N,
                             int64_t C_in, int64_t C_out, int64_t T, int64_t padding,
                             int64_t dilation) {
  if (N < 0 || C_in < 1 || C_in > kMaxChannels || C_out < 1 || C_out > kMaxChannels ||
      num_groups < 1 || C_out % num_groups != 0 || T < 1 || T >= (int64_t(1) << 29) ||
      padding < 0 || padding >= (int64_t(1) << 29) || dilation < 1)
    return DCONV1D_EINVAL;
  const int64_t T_out = T + 2 * padding - 2 * dilation;
  if (T_out < 1 || C_in * T > kMaxIndex || C_out * T_out > kMaxIndex) return DCONV1D_EINVAL;
  if (N == 0) return DCONV1D_METHOD_DIRECT;
  // T_out >= 1 bounds dilation by T/2 + padding < 2^30
  const int cpg = (int)(C_out / num_groups);
  if (!gn_fused_fits(N, (int)C_in, (int)C_out, (int)T, (int)T_out, (int)padding, (int)dilation,
                     cpg, x, W))
    return gn_two_kernel_winograd(N, C_out, T, padding, dilation) ? DCONV1D_METHOD_WINOGRAD
                                                                   : DCONV1D_METHOD_DIRECT;
  const int delta = gn_fused_delta((int)padding, gn_fused_vec4((int)T, x));
  const int mg = gn_fused_groups((int)T_out, (int)dilation, delta);
  return gn_fused_wino(mg, (int)dilation, W) && winograd_override() != 0
             ? DCONV1D_METHOD_WINOGRAD
             : DCONV1D_METHOD_DIRECT;
}

int prenorm_dconv1d_fwd(const float* x, const float* running_mean, const float* running_var,
                        const float* gamma, const float* beta, float eps, const float* W,
                        const float* b, float* out, int64_t N, int64_t C, int64_t L, int64_t d,
                        hipStream_t stream) {
  g_err.clear();
  return prenorm_common<float>(x, x, running_mean, running_var, gamma, beta, eps, W, b, out, N,
                               C, L, d, stream, false, Norm::Eval, nullptr);
}

int prenorm_dconv1d_fwd_noalloc(const float* x, const float* running_mean,
                                const float* running_var, const float* gamma, const float* beta,
                                float eps, const float* W, const float* b, float* out, int64_t N,
                                int64_t C, int64_t L, int64_t d, hipStream_t stream) {
  g_err.clear();
  return prenorm_common<float>(x, x, running_mean, running_var, gamma, beta, eps, W, b, out, N,
                               C, L, d, stream, false, Norm::Eval, nullptr, true);
}

int prenorm_dconv1d_fwd_bf16(const uint16_t* x, const float* running_mean,
                             const float* running_var, const float* gamma, const float* beta,
                             float eps, const float* W, const float* b, uint16_t* out,
                             int64_t N, int64_t C, int64_t L, int64_t d, hipStream_t stream) {
  g_err.clear();
  return prenorm_common<uint16_t>(x, x, running_mean, running_var, gamma, beta, eps, W, b, out,
                                  N, C, L, d, stream, true, Norm::Eval, nullptr);
}

int prenorm_dconv1d_fwd_train(const float* x, float* running_mean, float* running_var,
                              const float* gamma, const float* beta, float eps, float momentum,
                              const float* W, const float* b, float* out, float* save_mean,
                              float* save_invstd, int64_t N, int64_t C, int64_t L, int64_t d,
                              hipStream_t stream) {
  g_err.clear();
  const TrainBn t{momentum, running_mean, running_var, save_mean, save_invstd};
  return prenorm_common<float>(x, x, running_mean, running_var, gamma, beta, eps, W, b, out, N,
                               C, L, d, stream, false, Norm::Train, &t);
}

int prenorm_dconv1d_fwd_train_bf16(const uint16_t* x, float* running_mean, float* running_var,
                                   const float* gamma, const float* beta, float eps,
                                   float momentum, const float* W, const float* b, uint16_t* out,
                                   float* save_mean, float* save_invstd, int64_t N, int64_t C,
                                   int64_t L, int64_t d, hipStream_t stream) {
  g_err.clear();
  const TrainBn t{momentum, running_mean, running_var, save_mean, save_invstd};
  return prenorm_common<uint16_t>(x, x, running_mean, running_var, gamma, beta, eps, W, b, out,
                                  N, C, L, d, stream, true, Norm::Train, &t);
}

int relu_dconv1d_residual_fwd(const float* xn, const float* W, const float* b,
                              const float* residual, float* out, int64_t N, int64_t C, int64_t L,
                              int64_t d, hipStream_t stream) {
  g_err.clear();
  return prenorm_common<float>(xn, residual, nullptr, nullptr, nullptr, nullptr, 0.f, W, b, out,
                               N, C, L, d, stream, false, Norm::External, nullptr);
}

int relu_dconv1d_residual_fwd_bf16(const uint16_t* xn, const float* W, const float* b,
                                   const uint16_t* residual, uint16_t* out, int64_t N, int64_t C,
                                   int64_t L, int64_t d, hipStream_t stream) {
  g_err.clear();
  return prenorm_common<uint16_t>(xn, residual, nullptr, nullptr, nullptr, nullptr, 0.f, W, b,
                                  out, N, C, L, d, stream, true, Norm::External, nullptr);
}

int conv1d_groupnorm_fwd(const float* x, const float* W, const float* bias, const float* gamma,
                         const float* beta, float eps, int64_t num_groups, float* out, int64_t N,
                         int64_t C_in, int64_t C_out, int64_t T, int64_t padding,
                         int64_t dilation, hipStream_t stream) {
  g_err.clear();
  if (!x && N != 0) return fail(DCONV1D_EINVAL, "x is NULL");
  if (!W) return fail(DCONV1D_EINVAL, "W is NULL");
  if (!out && N != 0) return fail(DCONV1D_EINVAL, "out is NULL");
  if (N < 0) return fail(DCONV1D_EINVAL, "N must be >= 0 (got %lld)", (long long)N);
  if (C_in < 1 || C_in > kMaxChannels || C_out < 1 || C_out > kMaxChannels)
    return fail(DCONV1D_EINVAL, "C_in and C_out must be in [1, %lld]", (long long)kMaxChannels);
  if (num_groups < 1 || C_out % num_groups != 0)
    return fail(DCONV1D_EINVAL, "num_groups must be >= 1 and divide C_out (got %lld, C_out %lld)",
                (long long)num_groups, (long long)C_out);
  if (T < 1 || T >= (int64_t(1) << 29))
    return fail(DCONV1D_EINVAL, "T must be in [1, 2^29) (got %lld)", (long long)T);
  if (padding < 0 || padding >= (int64_t(1) << 29))
    return fail(DCONV1D_EINVAL, "padding must be in [0, 2^29)");
  if (dilation < 1) return fail(DCONV1D_EINVAL, "dilation must be >= 1");
  const int64_t T_out = T + 2 * padding - 2 * dilation;
  if (T_out < 1)
    return fail(DCONV1D_EINVAL, "output length T + 2*padding - 2*dilation = %lld < 1",
                (long long)T_out);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(DCONV1D_EINVAL, "eps must be finite and >= 0");
  if (C_in * T > kMaxIndex || C_out * T_out > kMaxIndex)
    return fail(DCONV1D_EINVAL, "C*T exceeds 2^31-1");
  if (N > INT64_MAX / (4 * std::max(C_in * T, C_out * T_out)))
    return fail(DCONV1D_EINVAL, "N*C*T overflows");
  if (overlaps(x, (uint64_t)N * C_in * T * 4, out, (uint64_t)N * C_out * T_out * 4))
    return fail(DCONV1D_EALIAS, "out overlaps x");

  const int Cin_pad = round_up((int)C_in, KC);
  const int Cout_pad = round_up((int)C_out, CO_TILE_F32);
  const int Lo = (int)T_out;
  const ConvTile tile = conv_f32_tile(Lo, (int)std::min<int64_t>(N, kMaxIndex), (int)C_out);
  const int n_ct = ((int)C_out + tile.co_tile() - 1) / tile.co_tile();
  const int n_tt = (Lo + tile.tt - 1) / tile.tt;
  if (N * n_tt * n_ct > kMaxIndex) return fail(DCONV1D_EINVAL, "grid too large");
  if (N == 0) return DCONV1D_OK;

  // Every group inside 16 output channels and T_out <= 1024: one launch, no workspace.
  const int cpg = (int)(C_out / num_groups);
  if (gn_fused_fits(N, (int)C_in, (int)C_out, (int)T, Lo, (int)padding, (int)dilation, cpg, x,
                    W)) {
    GnFusedArgs g{};
    g.x = x;
    g.W = W;
    g.bias = bias;
    g.gamma = gamma;
    g.beta = beta;
    g.out = out;
    g.eps = eps;
    g.N = (int)N;
    g.C_in = (int)C_in;
    g.C_out = (int)C_out;
    g.T = (int)T;
    g.T_out = Lo;
    g.pad = (int)padding;
    g.dil = (int)dilation;
    g.cpg = cpg;
    g.vec4 = gn_fused_vec4((int)T, x) ? 1 : 0;
    g.delta = gn_fused_delta((int)padding, g.vec4 != 0);
    g.mg = gn_fused_groups(Lo, (int)dilation, g.delta);
    g.n_cb = (int)C_out / 16;
    // the Winograd form whenever it runs the shape, unless DCONV1D_WINOGRAD is "0"
    g.wino = gn_fused_wino(g.mg, (int)dilation, W) && winograd_override() != 0 ? 1 : 0;
    const int slot = timer_begin(stream);
    hipError_t e = launch_conv_gn_fused(g, stream);
    timer_end(slot, stream);
    if (e != hipSuccess) return hip_fail(e, "conv+groupnorm kernel launch");
    return DCONV1D_OK;
  }

  // Two kernels: the conv (Winograd when gn_two_kernel_winograd says so, else the direct
  // kernel with the tile above) writes y into out and per-(channel, tile) statistics into
  // the workspace, then gn_normalize_kernel merges them per group and normalises out.
  const bool wino = gn_two_kernel_winograd(N, C_out, T, padding, dilation);
  const int d_w = (int)std::min<int64_t>(dilation, T);
  const int wmb = wino ? wino_channel_blocks(N, (int)C_out, (int)T, d_w) : 0;
  const int n_tt_c = wino ? wino_pair_tiles((int)T, d_w) : n_tt;
  const int n_ct_c = wino ? ((int)C_out + 64 * wmb - 1) / (64 * wmb) : n_ct;
  if (N * n_tt_c * n_ct_c > kMaxIndex) return fail(DCONV1D_EINVAL, "grid too large");
  const size_t off_wp = 0;
  const size_t off_part =
      align256(off_wp + sizeof(float) * (wino ? 4 : 3) * (size_t)Cin_pad * Cout_pad);
  const size_t total = align256(off_part + sizeof(float) * 3 * (size_t)N * C_out * n_tt_c);
  char* ws = nullptr;
  WorkspaceUse use;
  int st = use.acquire(total, stream, &ws);
  if (st != DCONV1D_OK) return st;
  float* Wp = reinterpret_cast<float*>(ws + off_wp);
  float* part = reinterpret_cast<float*>(ws + off_part);

  hipError_t e =
      wino ? launch_prep_wino(W, (int)C_out, (int)C_in, Cout_pad, Cin_pad, Wp, nullptr, nullptr,
                              nullptr, nullptr, 0.f, nullptr, nullptr, stream)
           : launch_prep_f32(W, (int)C_out, (int)C_in, Cout_pad, Cin_pad, Wp, nullptr, nullptr,
                             nullptr, nullptr, 0.f, nullptr, nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "prep kernel launch");

  // dilation > T + 2*padding would already make T_out < 1, so taps fit in int
  ConvF32Args a{};
  a.x = x;
  a.scale = nullptr;
  a.shift = nullptr;
  a.Wp = Wp;
  a.bias = bias;
  a.out = out;
  a.partials = part;
  a.N = (int)N;
  a.C_in = (int)C_in;
  a.C_out = (int)C_out;
  a.L_in = (int)T;
  a.L_out = Lo;
  // the Winograd form: padding = dilation, both taken as min(dilation, T) (dilations from
  // T on leave only the centre tap either way)
  a.pad = wino ? d_w : (int)padding;
  a.dil = wino ? d_w : (int)dilation;
  a.NCB = Cout_pad / 16;
  a.Q = (wino ? 1 : 3) * Cin_pad / KC;
  a.n_tt = n_tt_c;
  a.n_ct = n_ct_c;
  const int slot = timer_begin(stream);
  e = wino ? launch_conv_wino(a, wmb, EPI_GN_STATS, stream)
           : launch_conv_f32(a, tile, EPI_GN_STATS, stream);
  timer_end(slot, stream);
  if (e != hipSuccess) return hip_fail(e, "conv kernel launch");
  e = launch_gn_normalize(out, part, gamma, beta, eps, (int)N, (int)C_out, Lo, (int)num_groups,
                          n_tt_c, stream);
  if (e != hipSuccess) return hip_fail(e, "groupnorm kernel launch");
  return DCONV1D_OK;
}

const char* dconv1d_last_error(void) { return g_err.c_str(); }

void dconv1d_release(void) {
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    Workspace& w = g_ws[dev];
    std::lock_guard<std::mutex> lock(w.mu);
    if (!w.ptr && !w.done) continue;
    if (hipSetDevice(dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      if (w.ptr) (void)hipFree(w.ptr);
      if (w.done) (void)hipEventDestroy(w.done);
    }
    w.ptr = nullptr;
    w.bytes = 0;
    w.done = nullptr;
    w.last = nullptr;
    w.pending = false;
  }
  if (have_cur) (void)hipSetDevice(cur);
}

int dconv1d_timer_enable(int enable) {
  g_err.clear();
  std::lock_guard<std::mutex> lock(g_timer_mu);
  if (enable && g_timer.ev.empty()) {
    g_timer.ev.resize(2 * kTimerSlots);
    for (auto& ev : g_timer.ev) {
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) {
        g_timer.ev.clear();
        return hip_fail(e, "hipEventCreate");
      }
    }
  }
  g_timer.on = enable != 0;
  g_timer.used = 0;
  return DCONV1D_OK;
}

int dconv1d_timer_read(double* total_ms, int64_t* launches) {
  g_err.clear();
  std::lock_guard<std::mutex> lock(g_timer_mu);
  double sum = 0.0;
  for (int i = 0; i < g_timer.used; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = g_timer.used;
  g_timer.used = 0;
  return DCONV1D_OK;
}

}  // extern "C"
