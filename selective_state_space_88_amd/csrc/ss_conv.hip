// ss_conv.hip -- causal depthwise 1-D convolution in front of the scan (gfx950).
//
// Each Mamba block convolves its input along time, per channel and causally, before the
// selective SSM (bqwf.cn state-space survey, section 3.1); in decoding the block then keeps the
// last few inputs (the "Mamba -- selective state space model" study notes, pitfalls).  Per
// (b, d), with W taps and x before t = 0 taken from the carried state (or zero):
//   out_t = bias_d + sum_{j=0}^{W-1} w[d, j] x_{t - (W-1) + j},   optionally out_t * sigmoid(out_t).
//
// Mapping: a lane computes 8 consecutive outputs of a row (a piece) from that 8-step piece of x
// and the W - 1 inputs before it, the taps in registers.  A wave covers a few sweeps of 64
// consecutive pieces with all their loads issued first (more bytes in flight per wave); the
// inputs before a piece are those of the lane below, moved across with DPP (lane 0 takes lane 63
// of the sweep before), so x is read from HBM once: only lane 0 of a wave's first sweep loads its
// previous piece, and the first piece of a row takes them from the state.  The op is HBM-bound
// (x read and out written once); rows with 16-byte aligned pieces use vector accesses.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kCP = 8;        // outputs per thread and sweep
constexpr int kCMaxW = 8;     // taps
constexpr int kConvThreads = 256;
// consecutive 64-piece sweeps per wave, loads issued together (2 measured best: more bytes in
// flight per wave against fewer waves per SIMD)
constexpr int kSweeps = 2;

// pieces of 8 steps per row; an empty row still gets one (it writes the state)
inline int64_t conv_pieces(int64_t L) { return L > 0 ? (L + kCP - 1) / kCP : 1; }

__device__ __forceinline__ float wave_shr1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138 /* wave_shr:1 */, 0xf, 0xf, false));
}

// A wave owns pieces [64 SW w, 64 SW (w + 1)) of the row-major list of every row's pieces (fewer
// than 2^32 in all, so 32-bit indices); sweep k gives lane l the piece 64 SW w + 64 k + l.  Lanes
// past the end work on the last piece (in bounds) and store nothing.  FULL: every piece is whole
// and 16-byte aligned (L a multiple of 8, aligned rows), so loads and stores are unconditional.
template <typename TX, typename TO, bool SILU, bool FULL, int SW>
__global__ __launch_bounds__(kConvThreads) void conv1d_kernel(ConvArgs p) {
  const uint32_t pieces = (uint32_t)p.pieces, total = (uint32_t)p.total, channels = (uint32_t)p.channels;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t base = ((blockIdx.x * kConvThreads + threadIdx.x) >> 6) * (64u * SW);
  if (base >= total) return;   // whole waves only
  const int W = p.W;
  const int64_t L = FULL ? INT64_MAX : p.L;
  const bool vec = FULL ? true : p.vec;

  uint32_t piece[SW], bch[SW], dch[SW], rowk[SW];
  float cur[SW][kCP];
#pragma unroll
  for (int k = 0; k < SW; ++k) {
    const uint32_t idx = min(base + 64u * k + lane, total - 1);
    const uint32_t row = idx / pieces;
    rowk[k] = row;
    piece[k] = idx - row * pieces;
    bch[k] = row / channels;
    dch[k] = row - bch[k] * channels;
    const TX* xr = static_cast<const TX*>(p.x) + (int64_t)bch[k] * p.x_sb + (int64_t)dch[k] * p.x_sd;
    load_seg<kCP>(xr, (int64_t)piece[k] * kCP, L, vec, cur[k]);
  }

#pragma unroll
  for (int k = 0; k < SW; ++k) {
    const int64_t t0 = (int64_t)piece[k] * kCP;
    const uint32_t b = bch[k], d = dch[k];
    const TX* xr = static_cast<const TX*>(p.x) + (int64_t)b * p.x_sb + (int64_t)d * p.x_sd;
    // win[m] = x_{t0 - 8 + m}: the previous piece (the lane below, or lane 63 of the last sweep)
    float win[2 * kCP];
    win[0] = 0.f;   // x_{t0-8}: never a tap (W <= 8)
#pragma unroll
    for (int m = 1; m < kCP; ++m) {
      float v = wave_shr1(cur[k][m]);
      if (k > 0) {
        const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur[k - 1][m]), 63));
        v = lane == 0 ? top : v;
      }
      win[m] = v;
    }
    const float* sr = p.state_in ? p.state_in + (int64_t)b * p.si_sb + (int64_t)d * p.si_sd : nullptr;
    if (piece[k] == 0) {
      // before t = 0: the state holds x_{-(W-1)} .. x_{-1}
#pragma unroll
      for (int m = 1; m < kCP; ++m) {
        const int s = m - kCP;
        win[m] = (sr && s >= -(W - 1)) ? sr[(W - 1) + s] : 0.f;
      }
    } else if (k == 0 && lane == 0) {
      float prev[kCP];
      load_seg<kCP>(xr, t0 - kCP, L, vec, prev);
#pragma unroll
      for (int m = 1; m < kCP; ++m) win[m] = prev[m];
    }
#pragma unroll
    for (int m = 0; m < kCP; ++m) win[kCP + m] = cur[k][m];
    if (base + 64u * k + lane >= total) break;   // this lane is past the end in every later sweep too

    // taps newest first, wr[q] = w[W-1-q] on x_{t-q}, and bias: scalar loads when the sweep
    // lies in one row (rows only grow along it)
    float wr[kCMaxW], bias;
    if (__builtin_amdgcn_readfirstlane(rowk[k]) == __builtin_amdgcn_readlane(rowk[k], 63)) {
      const uint32_t du = __builtin_amdgcn_readfirstlane(d);
      cfloat* wc = to_constant(p.w) + (int64_t)du * p.w_sd;
#pragma unroll
      for (int q = 0; q < kCMaxW; ++q) wr[q] = q < W ? wc[W - 1 - q] : 0.f;
      bias = p.bias ? to_constant(p.bias)[du] : 0.f;
    } else {
      const float* wv = p.w + (int64_t)d * p.w_sd;
#pragma unroll
      for (int q = 0; q < kCMaxW; ++q) wr[q] = q < W ? wv[W - 1 - q] : 0.f;
      bias = p.bias ? p.bias[d] : 0.f;
    }
    float o[kCP];
#pragma unroll
    for (int m = 0; m < kCP; ++m) o[m] = bias;
#pragma unroll
    for (int q = 0; q < kCMaxW; ++q)
      if (q < W) {   // uniform
#pragma unroll
        for (int m = 0; m < kCP; ++m) o[m] = fmaf(wr[q], win[kCP + m - q], o[m]);
      }
    if constexpr (SILU) {
#pragma unroll
      for (int m = 0; m < kCP; ++m) o[m] *= __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-o[m] * kLog2e));
    }
    if (FULL || p.L > 0) {
      TO* orow = static_cast<TO*>(p.out) + (int64_t)b * p.o_sb + (int64_t)d * p.o_sd;
      store_seg<kCP>(orow, t0, L, vec, o);
    }
    // the last W - 1 inputs (reaching into the state when L < W - 1)
    if (p.state_out && piece[k] == pieces - 1) {
      float* so = p.state_out + (int64_t)b * p.so_sb + (int64_t)d * p.so_sd;
      for (int j = 0; j < W - 1; ++j) {
        const int64_t s = p.L - (W - 1) + j;
        so[j] = s >= 0 ? to_f32(xr[s]) : (sr ? sr[(W - 1) + s] : 0.f);
      }
    }
  }
}

template <typename TX, typename TO>
hipError_t launch_t(ConvArgs a, hipStream_t s) {
  a.pieces = conv_pieces(a.L);
  a.total = a.batch * a.channels * a.pieces;
  if (a.total == 0) return hipSuccess;
  const int64_t waves = (a.total + 64 * kSweeps - 1) / (64 * kSweeps);
  const dim3 grid((unsigned)((waves + kConvThreads / 64 - 1) / (kConvThreads / 64))), block(kConvThreads);
  const bool full = a.vec && a.L > 0 && a.L % kCP == 0;
#define SS_CONV(SL, FL) hipLaunchKernelGGL((conv1d_kernel<TX, TO, SL, FL, kSweeps>), grid, block, 0, s, a)
  if (a.silu) {
    if (full) SS_CONV(true, true); else SS_CONV(true, false);
  } else {
    if (full) SS_CONV(false, true); else SS_CONV(false, false);
  }
#undef SS_CONV
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv(const ConvArgs& a, hipStream_t s) {
  // the piece indices are 32-bit (the caller keeps the total below 2^32 - 256)
  if (a.x_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, s) : launch_t<float, float>(a, s);
}

}  // namespace ss
