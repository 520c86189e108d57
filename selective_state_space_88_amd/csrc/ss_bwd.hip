// ss_bwd.hip -- backward of the selective scan (gradients of every input), gfx950.
//
// The pages train the scan by recomputing its states instead of storing them (bqwf.cn
// state-space survey, section 2.2).  Here: a checkpoint pass stores each row's state at the
// start of every window of W steps (N floats per window), and the backward pass walks the
// windows in reverse, recomputing the states inside a window from its checkpoint and running
// the adjoint recurrence g_t = C_t dy0_t + a_{t+1} g_{t+1} (g = dLoss/dh) backwards through it.
// Per step and state it then accumulates, with dy0 = dy s(z) the gradient of the output before
// the gate s(z) = z sigmoid(z):
//   dC_t += dy0_t h_t,  dB_t += g_t dt_t u_t,  du_t += g_t dt_t B_t,
//   ddt_t += g_t (h_{t-1} a_t A + B_t u_t),  dA += g_t h_{t-1} a_t dt_t,
// and per step du_t += dy0_t D, dD += dy0_t u_t, ddelta_t = ddt_t sigmoid(x_t) (softplus'),
// dbias += ddelta_t.  The gate itself (dz_t = dy_t y0_t s'(z_t) and dy0) is a pass of its own
// between a forward recompute of y0 and this kernel (see launch_bwd).
//
// With heads (a step size, and optionally a scalar decay A_h, shared by a head's channels) the
// per-head gradients ddelta, dbias, dA (and dD when D is per head) are summed over the head's
// channels; with a scalar decay exp(dt A_h) is computed once per step for all N states.
//
// Mapping (as in the forward kernel): a wave owns one channel, lane j the K consecutive steps
// t0 + jK .. t0 + jK + K - 1 of a window; states go one at a time.  Inside a window both recurrences
// are scans of affine maps over the lanes: the states forward (x -> a x + b composed left to
// right), the adjoint backward (composed right to left); each lane runs its K steps from zero,
// the lanes' maps are combined by a shuffle scan, and each lane re-runs its steps from its true
// incoming value.  A block holds 8 channels of one (batch, B/C group): their dB and dC
// contributions are summed through LDS before one atomic add per (state, step).
//
// Few rows with long sequences (fewer 8-channel blocks than two per CU) cut each row's windows
// into sequence segments, one block per (8 channels, segment), so that the CUs fill without
// adding to the dB/dC atomics.  A segment starts from the adjoint the segments to its right
// hand it: a pre-pass (bwd_seg_kernel) computes each segment's own part of the adjoint entering
// it from the right and its total step size, and the backward block combines those of the
// segments to its right before its walk (bwd_kernel's prologue).
#include <algorithm>
#include <type_traits>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kBK = 8;               // steps per lane
constexpr int kBW = 64 * kBK;        // steps per window
constexpr int kBWaves = 4;           // channels (rows) per block of the checkpoint kernel
constexpr int kMWaves = 8;           // channels per block of the backward kernel (of one B/C group)
constexpr int kBMaxPairs = 64;       // N <= 128
constexpr int kBwdSP = 1;            // states per group of the backward kernel's state loop

// DPP move of v with control CTRL on the rows in ROWMASK; lanes with no source (or in masked
// rows) keep `old`
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWMASK, 0xf, false));
}

// (A, B) <- (A, B) o (Ao, Bo): this lane's map applied after the other one
__device__ __forceinline__ void compose(float& A, float& B, float Ao, float Bo) {
  B = fmaf(A, Bo, B);
  A = A * Ao;
}

// the next lane's map (lane 63: the identity)
__device__ __forceinline__ void shift_down(float& A, float& B) {
  A = dpp_or<0x130, 0xf>(1.f, A);   // wave_shl:1
  B = dpp_or<0x130, 0xf>(0.f, B);
}

// One scan step on both halves of the map with fused DPP instructions: B += B[src] A, then
// A *= A[src] (the source lane's map applied first).  A lane whose source is outside its row
// (row_shr/row_shl) or whose row is masked off is not written, i.e. composes with the identity.
// The trailing s_nop supplies the second wait state between a VALU write and the next DPP
// read of the same VGPR (the single chain leaves only one instruction between them).
#define SS_BSTEP(CTRL)                                  \
  "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n"               \
  "v_mul_f32_dpp %0, %0, %0 " CTRL "\n"                \
  "s_nop 0\n"

// Exclusive left-to-right scan of the lanes' maps over the 64 lanes: lane j ends with the maps
// of lanes 0..j-1 composed (lane 0: the identity).  Inclusive within rows of 16 by row_shr
// 1, 2, 4, 8, then rows 0 and 2 into rows 1 and 3 (row_bcast:15), lane 31 into rows 2 and 3
// (row_bcast:31), then a shift by one lane (wave_shr:1) onto the identity.
__device__ __forceinline__ void scan_up_exclusive(float& A, float& B) {
  float ea, eb;
  asm volatile("s_nop 1\n"
               SS_BSTEP("row_shr:1 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:2 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:4 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:8 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_bcast:15 row_mask:0xa bank_mask:0xf")
               SS_BSTEP("row_bcast:31 row_mask:0xc bank_mask:0xf")
               "v_mov_b32 %2, 1.0\n"
               "v_mov_b32 %3, 0\n"
               "v_mov_b32_dpp %2, %0 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
               "v_mov_b32_dpp %3, %1 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
               : "+v"(A), "+v"(B), "=&v"(ea), "=&v"(eb));
  A = ea;
  B = eb;
}

// Inclusive left-to-right scan over the 64 lanes (the steps of scan_up_exclusive without the
// final shift): lane j ends with the maps of lanes 0..j composed.
__device__ __forceinline__ void scan_up_inclusive(float& A, float& B) {
  asm volatile("s_nop 1\n"
               SS_BSTEP("row_shr:1 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:2 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:4 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shr:8 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_bcast:15 row_mask:0xa bank_mask:0xf")
               SS_BSTEP("row_bcast:31 row_mask:0xc bank_mask:0xf")
               : "+v"(A), "+v"(B));
}

// Inclusive right-to-left scan within each row of 16 lanes (row_shl 1, 2, 4, 8): lane j ends
// with the maps of lanes j..(end of its row), the highest lane's applied first.
__device__ __forceinline__ void scan_down_rows(float& A, float& B) {
  asm volatile("s_nop 1\n"
               SS_BSTEP("row_shl:1 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shl:2 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shl:4 row_mask:0xf bank_mask:0xf")
               SS_BSTEP("row_shl:8 row_mask:0xf bank_mask:0xf")
               : "+v"(A), "+v"(B));
}
#undef SS_BSTEP

// Inclusive right-to-left scan over the 64 lanes (lane j ends with the maps of lanes j..63, lane
// 63's applied first): within rows by fused DPP, then each row composed with the totals of the
// rows above it (read from their first lanes)
__device__ __forceinline__ void scan_down_fused(float& A, float& B, int lane) {
  scan_down_rows(A, B);
  const float a1 = readlane_f(A, 16), b1 = readlane_f(B, 16);
  const float a2 = readlane_f(A, 32), b2 = readlane_f(B, 32);
  const float a3 = readlane_f(A, 48), b3 = readlane_f(B, 48);
  // suffixes: rows 3.. (identity for row 3), 2: T3, 1: T2 o T3, 0: T1 o T2 o T3
  const float s2a = a3, s2b = b3;
  const float s1a = a2 * s2a, s1b = fmaf(a2, s2b, b2);
  const float s0a = a1 * s1a, s0b = fmaf(a1, s1b, b1);
  const int row = lane >> 4;
  const float Sa = row == 0 ? s0a : row == 1 ? s1a : row == 2 ? s2a : 1.f;
  const float Sb = row == 0 ? s0b : row == 1 ? s1b : row == 2 ? s2b : 0.f;
  compose(A, B, Sa, Sb);
}

__device__ __forceinline__ float wave_sum(float v) {
  // each row of 16 lanes summed by row_ror 8, 4, 2, 1 (every lane gets its row's total), then
  // the four row totals
  v += dpp_or<0x128, 0xf>(0.f, v);
  v += dpp_or<0x124, 0xf>(0.f, v);
  v += dpp_or<0x122, 0xf>(0.f, v);
  v += dpp_or<0x121, 0xf>(0.f, v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// Checkpoints: the state of every (row, window, state) at the window's start.
template <typename TIn, bool SCALAR>
__global__ __launch_bounds__(64 * kBWaves) void bwd_ckpt_kernel(BwdArgs p, int P, int64_t nwin, float* ckpt) {
  __shared__ float hst[kBWaves][kBMaxPairs][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kBWaves + wave;  // b * channels + d
  const bool live = row < p.batch * p.channels;
  const int64_t rr = live ? row : 0;
  const int64_t b = rr / p.channels, d = rr % p.channels;
  const int64_t g = d / p.chan_per_group, hd = d / p.chan_per_head;
  const int N = p.N;
  const TIn* ur = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* dr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  for (int pp = lane; pp < P; pp += 64) hst[wave][pp][0] = hst[wave][pp][1] = 0.f;
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    float dt[kBK], wv[kBK], dv[kBK], uv[kBK];
    load_seg<kBK>(dr, t0, p.L, p.vec, dv);
    load_seg<kBK>(ur, t0, p.L, p.vec, uv);
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const bool ok = t0 + k < p.L;
      const float x = dv[k] + bias;
      dt[k] = ok ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      wv[k] = dt[k] * uv[k];
    }
    // scalar decay: one exp per step for every state
    float ah[kBK];
    if constexpr (SCALAR) {
      const float A2 = p.A[hd] * kLog2e;
#pragma unroll
      for (int k = 0; k < kBK; ++k) ah[k] = __builtin_amdgcn_exp2f(dt[k] * A2);
    }
    for (int pp = 0; pp < P; ++pp) {
      float Af[2], Bf[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = 2 * pp + s;
        const bool nv = n < N;
        const float A2 = (nv && !SCALAR) ? p.A[d * p.A_sd + n] * kLog2e : 0.f;
        float bq[kBK];
        load_seg<kBK>(Bg + (nv ? n : 0) * p.B_sn, t0, nv ? p.L : 0, p.vec, bq);
        float a = 1.f, h = 0.f;
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          const float av = SCALAR ? ah[k] : __builtin_amdgcn_exp2f(dt[k] * A2);
          h = fmaf(av, h, wv[k] * bq[k]);
          a *= av;
        }
        Af[s] = a;
        Bf[s] = h;
        scan_up_inclusive(Af[s], Bf[s]);
      }
      // the window's start state is stored, and its end state (lane 63's map) carried on
      const float h0 = hst[wave][pp][0], h1 = hst[wave][pp][1];
      if (live && lane == 0) {
        float* c = ckpt + (row * nwin + w) * N;
        c[2 * pp] = h0;
        if (2 * pp + 1 < N) c[2 * pp + 1] = h1;
      }
      const float e0 = readlane_f(fmaf(Af[0], h0, Bf[0]), 63), e1 = readlane_f(fmaf(Af[1], h1, Bf[1]), 63);
      if (lane == 0) {
        hst[wave][pp][0] = e0;
        hst[wave][pp][1] = e1;
      }
    }
  }
}

// Sequence segments.  Segment j of a row covers windows [j wps, (j + 1) wps).  With the adjoint
// recurrence g_t = C_t dy0_t + a_{t+1} g_{t+1}, the value a block carries into a window from the
// right is a_t g_t at the first step t of the window after it.  Segment j's own part of that value
// at its start s_j (the dy0 of its steps only) is
//   Lj[n] = sum_{t in seg j} (prod_{s = s_j .. t} a_{s,n}) C_{t,n} dy0_t,
// its decay Dj[n] = prod_{s in seg j} a_{s,n} = 2^(A_n log2 e Sj) with Sj its total step size,
// and the value entering segment k from the right is R(k) = D_{k+1} R(k+1) + L_{k+1}, R(last) = 0.
constexpr int kSegMaxN = 32;          // the segmented path serves N <= 32 (states in registers)
constexpr int64_t kSegMinWin = 4;     // segments of at least 4 windows (2048 steps)
// states whose C rows the pre-pass loads together (measured on the 1M-step layer's backward:
// 4: 35.0, 8: 35.6, 16: 36.7 ms per call; 4 keeps three waves per SIMD)
constexpr int kSegG = 4;

struct BwdSegs {
  int64_t wps;   // windows per segment
  int32_t nseg;  // segments per row
};

// as many segments as give two 8-channel blocks per CU, none shorter than kSegMinWin windows
BwdSegs bwd_seg_plan(const BwdArgs& a) {
  const int64_t nwin = (a.L + kBW - 1) / kBW;
  const int64_t blocks = a.batch * a.groups * ((a.chan_per_group + kMWaves - 1) / kMWaves);
  int64_t S = 1;
  if (a.N <= kSegMaxN && blocks > 0)
    S = std::min<int64_t>((2 * (int64_t)cu_count() + blocks - 1) / blocks, nwin / kSegMinWin);
  S = std::max<int64_t>(S, 1);
  const int64_t wps = std::max<int64_t>((nwin + S - 1) / S, 1);
  return {wps, (int32_t)std::max<int64_t>((nwin + wps - 1) / wps, 1)};
}

// kBK steps of an aligned row lying wholly inside L, as the raw words of one or two 16-byte loads
// (issued by raw_load, widened by raw_widen: a group of loads can be issued before any waits)
template <typename T>
struct RawSteps;
template <>
struct RawSteps<bf16_t> {
  u32x4 v;
};
template <>
struct RawSteps<float> {
  f32x4 a, b;
};
__device__ __forceinline__ void raw_load(const bf16_t* p, RawSteps<bf16_t>& r) {
  r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load(const float* p, RawSteps<float>& r) {
  r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
}
__device__ __forceinline__ void raw_widen(const RawSteps<bf16_t>& r, float (&o)[kBK]) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = bf16_lo(w[e]);
    o[2 * e + 1] = bf16_hi(w[e]);
  }
}
__device__ __forceinline__ void raw_widen(const RawSteps<float>& r, float (&o)[kBK]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = r.a[e];
    o[4 + e] = r.b[e];
  }
}

// Per (row, segment j >= 1), one wave: Lj[0..N) and Sj into segw[(row nseg + j) (N + 1) + ..].
// Lane l takes the kBK steps t0 + l kBK .. of each window of the segment, walked left to right;
// the product of the decays from the segment's start to step t is 2^(A_n log2 e (S_w + s_t)),
// S_w the step sizes before the window (carried as the factor dp = 2^(A_n log2 e S_w), one exp
// per window) and s_t those of the window up to t (a prefix sum over the lanes), so that no
// exponent grows with the segment's length.
template <typename TIn, typename TDy, bool SCALAR, bool FGATE, int NS>
__global__ __launch_bounds__(256) void bwd_seg_kernel(BwdArgs p, int64_t wps, int nseg, float* __restrict__ segw) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rows = p.batch * p.channels;
  if (gw >= rows * (nseg - 1)) return;
  const int64_t row = gw / (nseg - 1);
  const int j = 1 + (int)(gw % (nseg - 1));
  const int64_t b = row / p.channels, d = row % p.channels;
  const int64_t g = d / p.chan_per_group, hd = d / p.chan_per_head;
  const int N = p.N;
  const int64_t L = p.L;
  const TIn* dr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TDy* dyr = static_cast<const TDy*>(p.dy) + b * p.dy_sb + d * p.dy_sd;
  const TIn* zr = FGATE ? static_cast<const TIn*>(p.gz) + b * p.z_sb + d * p.z_sd : nullptr;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  float A2[NS], acc[NS], dp[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    A2[n] = n < N ? (SCALAR ? p.A[hd] : p.A[d * p.A_sd + n]) * kLog2e : 0.f;
    acc[n] = 0.f;
    dp[n] = 1.f;
  }
  const int64_t nwin = (L + kBW - 1) / kBW;
  const int64_t wb = (int64_t)j * wps, we = std::min<int64_t>(nwin, wb + wps);
  float stot = 0.f;
  for (int64_t w = wb; w < we; ++w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    // a whole window of aligned rows takes its loads back to back (wave-uniform)
    const bool whole = p.vec && (w + 1) * kBW <= L;
    float dv[kBK], dy0[kBK], zz[kBK];
    if (whole) {
      RawSteps<TIn> rd, rz;
      RawSteps<TDy> ry;
      raw_load(dr + t0, rd);
      raw_load(dyr + t0, ry);
      if constexpr (FGATE) raw_load(zr + t0, rz);
      raw_widen(rd, dv);
      raw_widen(ry, dy0);
      if constexpr (FGATE) raw_widen(rz, zz);
    } else {
      load_seg<kBK>(dr, t0, L, p.vec, dv);
      load_seg<kBK>(dyr, t0, L, p.vec, dy0);
      if constexpr (FGATE) load_seg<kBK>(zr, t0, L, p.vec, zz);
    }
    if constexpr (FGATE) {
      // dy0 = dy s(z), s(z) = z sigmoid(z)
#pragma unroll
      for (int k = 0; k < kBK; ++k)
        dy0[k] *= zz[k] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-zz[k] * kLog2e));
    }
    // step sizes summed from the window's start: within the lane, then over the lanes before it
    float cs[kBK], run = 0.f;
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const float x = dv[k] + bias;
      run += t0 + k < L ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      cs[k] = run;
    }
    float inc = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    const float ex = inc - run;
    const float wtot = readlane_f(inc, 63);
#pragma unroll
    for (int k = 0; k < kBK; ++k) cs[k] += ex;
    // the C rows of kSegG states are loaded together (rows past N repeat the last one, unused),
    // so that a window waits for them once per group rather than once per state
#pragma unroll
    for (int n0 = 0; n0 < NS; n0 += kSegG) {
      if (n0 < N) {
        float cv[kSegG][kBK];
        if (whole) {
          RawSteps<TIn> raw[kSegG];
#pragma unroll
          for (int i = 0; i < kSegG; ++i) raw_load(Cg + (int64_t)(n0 + i < N ? n0 + i : N - 1) * p.C_sn + t0, raw[i]);
#pragma unroll
          for (int i = 0; i < kSegG; ++i) raw_widen(raw[i], cv[i]);
        } else {
#pragma unroll
          for (int i = 0; i < kSegG; ++i)
            load_seg<kBK>(Cg + (int64_t)(n0 + i < N ? n0 + i : N - 1) * p.C_sn, t0, L, p.vec, cv[i]);
        }
#pragma unroll
        for (int i = 0; i < kSegG; ++i) {
          const int n = n0 + i;
          if (n < N) {
            float sacc = 0.f;
#pragma unroll
            for (int k = 0; k < kBK; ++k)
              sacc = fmaf(__builtin_amdgcn_exp2f(A2[n] * cs[k]), cv[i][k] * dy0[k], sacc);
            acc[n] = fmaf(dp[n], sacc, acc[n]);
            dp[n] *= __builtin_amdgcn_exp2f(A2[n] * wtot);
          }
        }
      }
    }
    stot += wtot;
  }
  float* out = segw + (row * nseg + j) * (N + 1);
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (n < N) {
      const float v = wave_sum(acc[n]);
      if (lane == 0) out[n] = v;
    }
  }
  if (lane == 0) out[N] = stot;
}

// The backward of the ungated scan (a gated layer reaches it through launch_bwd with dy0 = dy
// s(z) as its upstream gradient).  SP: states per group (1 or 2), the unit of the state loop (P
// groups); one state at a time keeps the kernel within 128 VGPRs, i.e. two 8-wave blocks (four
// waves per SIMD) per CU.
// This lane's kBK consecutive per-step outputs v at row + t0 (steps past L not written): two
// 16-byte nontemporal stores when the row segment is 16-byte aligned and whole, else one store
// per step.
__device__ __forceinline__ void store_steps(float* row, int64_t t0, int64_t L, const float (&v)[kBK]) {
  float* q = row + t0;
  if (t0 + kBK <= L && (reinterpret_cast<uintptr_t>(q) & 15) == 0) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(q));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(q) + 1);
  } else {
#pragma unroll
    for (int k = 0; k < kBK; ++k)
      if (t0 + k < L) q[k] = v[k];
  }
}

template <typename TIn, typename TDy, bool SCALAR, int SP, bool FGATE>
__global__ __launch_bounds__(64 * kMWaves) __attribute__((amdgpu_waves_per_eu(SP == 1 ? 4 : 1))) void bwd_kernel(
    BwdArgs p, int P, int64_t nwin, const float* ckpt, int64_t wps, int nseg, const float* __restrict__ segw) {
  __shared__ float gcar[kMWaves][2 * kBMaxPairs];     // adjoint carried into the window from the right
  __shared__ float dAl[kMWaves][2 * kBMaxPairs];      // dA partial sums of the wave's channel
  // dB (SP states), dC (SP states) of the window's steps, step-major ([lane][k] = step lane K + k)
  // (two buffers, alternating by state, so that one barrier per state orders both the writes
  // before the sums and the sums before the next writes to the same buffer)
  __shared__ __attribute__((aligned(16))) float red[2][kMWaves][2 * SP][kBW];
  // B (SP states) and C (SP states) of a group's window, shared by the block's channels; two
  // buffers: the next group's rows are loaded while this group runs
  __shared__ __attribute__((aligned(16))) float bcs[2][2 * SP][kBW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // blocks of 8 channels of one group; when the group's channels are 4 mod 8, the last block's
  // last 4 waves work on a copy of a valid channel and contribute nothing
  // block = segment * (batch * groups * cblocks) + channel block; the segment's windows [wlo, whi)
  const int64_t cblocks = (p.chan_per_group + kMWaves - 1) / kMWaves;
  const int64_t nblk = p.batch * p.groups * cblocks;
  const int64_t kseg = blockIdx.x / nblk, bx = blockIdx.x % nblk;
  const int64_t wlo = kseg * wps, whi = std::min<int64_t>(nwin, wlo + wps);
  const int64_t bg = bx / cblocks, qd = bx % cblocks;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t ci = qd * kMWaves + wave;
  const bool valid = ci < p.chan_per_group;
  const int64_t d = g * p.chan_per_group + (valid ? ci : p.chan_per_group - 1);
  const int64_t row = b * p.channels + d;
  const int64_t hd = d / p.chan_per_head;
  const int N = p.N;
  const int64_t L = p.L;
  const TIn* ur = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* dr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TDy* dyr = static_cast<const TDy*>(p.dy) + b * p.dy_sb + d * p.dy_sd;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  float* dBg = p.dB + b * p.dB_sb + g * p.dB_sg;
  float* dCg = p.dC + b * p.dC_sb + g * p.dC_sg;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  const float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;
  for (int i = lane; i < 2 * kBMaxPairs; i += 64) {
    gcar[wave][i] = 0.f;
    dAl[wave][i] = 0.f;
  }
  if (kseg + 1 < nseg) {
    // the adjoint entering the segment from the right: R(k) = D_{k+1} R(k+1) + L_{k+1}
    for (int n = lane; n < N; n += 64) {
      const float A2n = (SCALAR ? p.A[hd] : p.A[d * p.A_sd + n]) * kLog2e;
      float R = 0.f;
      for (int64_t jj = nseg - 1; jj > kseg; --jj) {
        const float* sj = segw + (row * nseg + jj) * (N + 1);
        R = fmaf(__builtin_amdgcn_exp2f(A2n * sj[N]), R, sj[n]);
      }
      gcar[wave][n] = R;
    }
  }
  float dDacc = 0.f, dbacc = 0.f;
  // thread t stages row t / 64 (B of states SP pp .. SP pp + SP - 1, then C of the same), the
  // steps of lane t % 64; rows past N and steps past L are zero
  const int srow = threadIdx.x >> 6, sseg = threadIdx.x & 63;
  auto bc_load = [&](int64_t ww, int pq, float (&v)[kBK]) {
    const int n = SP * pq + (srow % SP);
    const bool nv = n < N && srow < 2 * SP;
    const TIn* src = srow < SP ? Bg + (nv ? n : 0) * p.B_sn : Cg + (nv ? n : 0) * p.C_sn;
    load_seg<kBK>(src, ww * kBW + (int64_t)kBK * sseg, nv ? L : 0, p.vec, v);
  };
  auto bc_store = [&](int bf, const float (&v)[kBK]) {
    if (srow >= 2 * SP) return;   // 2 SP rows, one per wave of the first 2 SP
    float* dst = &bcs[bf][srow][kBK * sseg];
    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
  };
  {
    float v[kBK];
    bc_load(whi - 1, 0, v);
    bc_store(0, v);
  }
  __syncthreads();
  int buf = 0;
  int rb = 0;   // the reduction buffer of the current state

  for (int64_t w = whi - 1; w >= wlo; --w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    // (u and delta are loaded again at the window's end rather than kept across the state loop)
    float dt[kBK], wv[kBK], dy0[kBK], du[kBK], ddt[kBK];
    float sdt = 0.f;   // the lane's steps' total step size
    {
      float dv[kBK], uu[kBK];
      load_seg<kBK>(dr, t0, L, p.vec, dv);
      load_seg<kBK>(ur, t0, L, p.vec, uu);
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        const float x = dv[k] + bias;
        dt[k] = t0 + k < L ? (p.softplus ? softplus_fast(x) : x) : 0.f;
        wv[k] = dt[k] * uu[k];
      }
    }
    load_seg<kBK>(dyr, t0, L, p.vec, dy0);
    if constexpr (FGATE) {
      // the gate: dz = dy y0 s'(z) written here, and the kernel runs on dy0 = dy s(z) (s(z) =
      // z sigmoid(z), s'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))))
      float zz[kBK], yy[kBK];
      load_seg<kBK>(static_cast<const TIn*>(p.gz) + b * p.z_sb + d * p.z_sd, t0, L, p.vec, zz);
      load_seg<kBK>(p.gy0 + row * L, t0, L, p.y0_vec, yy);
      float dzv[kBK];
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        const float sgz = 1.f / (1.f + __builtin_amdgcn_exp2f(-zz[k] * kLog2e));
        dzv[k] = dy0[k] * yy[k] * sgz * fmaf(zz[k], 1.f - sgz, 1.f);
        dy0[k] = dy0[k] * (zz[k] * sgz);
      }
      if (valid) store_steps(p.dz + b * p.dz_sb + d * p.dz_sd, t0, L, dzv);
    }
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      du[k] = 0.f;   // here: sum over the states of g_t B_t (du and ddt take it once per step below)
      ddt[k] = 0.f;
      sdt += dt[k];
    }
    // scalar decay: one exp per step for every state
    float ah[kBK];
    if constexpr (SCALAR) {
      const float A2 = p.A[hd] * kLog2e;
#pragma unroll
      for (int k = 0; k < kBK; ++k) ah[k] = __builtin_amdgcn_exp2f(dt[k] * A2);
    }
    for (int pp = 0; pp < P; ++pp) {
      // the next group's B and C rows (the first group of the window to the left after the last)
      // (only the first 2 SP waves stage rows: the others skip the load and its bounds checks)
      const bool more = pp + 1 < P || w > wlo;
      float nbc[kBK];
      if (more && srow < 2 * SP) bc_load(pp + 1 < P ? w : w - 1, pp + 1 < P ? pp + 1 : 0, nbc);
      float rB[SP][kBK], rC[SP][kBK];
      float dAp[SP];
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const int n = SP * pp + s;
        const bool nv = n < N;
        const float An = SCALAR ? p.A[hd] : (nv ? p.A[d * p.A_sd + n] : 0.f);
        const float A2 = An * kLog2e;
        float av[kBK], bv[kBK], cv[kBK];
        {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bcs[buf][s][kBK * lane]);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bcs[buf][s][kBK * lane + 4]);
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(&bcs[buf][SP + s][kBK * lane]);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(&bcs[buf][SP + s][kBK * lane + 4]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            bv[k] = b0[k];
            bv[4 + k] = b1[k];
            cv[k] = c0[k];
            cv[4 + k] = c1[k];
          }
        }
#pragma unroll
        for (int k = 0; k < kBK; ++k) av[k] = SCALAR ? ah[k] : __builtin_amdgcn_exp2f(dt[k] * A2);
        // states: the lane's steps from zero, the scan, then from the incoming state
        float Af = __builtin_amdgcn_exp2f(sdt * A2), Bf = 0.f;   // the decay over the lane's steps
#pragma unroll
        for (int k = 0; k < kBK; ++k) Bf = fmaf(av[k], Bf, wv[k] * bv[k]);
        const float Pl = Af;   // the lane's total decay (both directions)
        float Ae = Af, Be = Bf;
        scan_up_exclusive(Ae, Be);
        const float hw = nv ? ckpt[(row * nwin + w) * N + n] : 0.f;
        float hs[kBK + 1];
        hs[0] = fmaf(Ae, hw, Be);
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          hs[k + 1] = fmaf(av[k], hs[k], wv[k] * bv[k]);
        }
        // adjoint: the lane's steps from zero (right to left), the scan, then from the value
        // carried in from the right
        float c = 0.f;
#pragma unroll
        for (int k = kBK - 1; k >= 0; --k) c = av[k] * fmaf(cv[k], dy0[k], c);
        float Ar = Pl, Br2 = c;
        scan_down_fused(Ar, Br2, lane);
        float Ad = Ar, Bd = Br2;
        shift_down(Ad, Bd);
        const float Xw = gcar[wave][n];
        c = fmaf(Ad, Xw, Bd);
        float dAs = 0.f;
#pragma unroll
        for (int k = kBK - 1; k >= 0; --k) {
          const float gk = fmaf(cv[k], dy0[k], c);
          rC[s][k] = dy0[k] * hs[k + 1];
          rB[s][k] = gk * wv[k];
          du[k] = fmaf(gk, bv[k], du[k]);
          const float gha = gk * hs[k] * av[k];
          ddt[k] = fmaf(gha, An, ddt[k]);
          dAs = fmaf(gha, dt[k], dAs);
          c = av[k] * gk;
        }
        // the adjoint carried into the previous window: lane 0's value after its first step
        const float cl = readlane_f(c, 0);
        if (lane == 0) gcar[wave][n] = cl;
        dAp[s] = dAs;
      }
      // dA of the group's SP states: summed over the wave's lanes into the wave's partial sums
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        const float v = wave_sum(dAp[s]);
        if (lane == 0 && valid && SP * pp + s < N) dAl[wave][SCALAR ? 0 : SP * pp + s] += v;
      }
      // dB, dC of the group's states: summed over the block's 8 channels, then one atomic add per step;
      // consecutive lanes add to consecutive steps, so each wave's adds cover two cache lines
      if (!valid) {
#pragma unroll
        for (int s = 0; s < SP; ++s)
#pragma unroll
          for (int k = 0; k < kBK; ++k) rB[s][k] = rC[s][k] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < SP; ++s)
#pragma unroll
        for (int k = 0; k < kBK; k += 4) {
          *reinterpret_cast<f32x4*>(&red[rb][wave][s][lane * kBK + k]) = f32x4{rB[s][k], rB[s][k + 1], rB[s][k + 2], rB[s][k + 3]};
          *reinterpret_cast<f32x4*>(&red[rb][wave][SP + s][lane * kBK + k]) =
              f32x4{rC[s][k], rC[s][k + 1], rC[s][k + 2], rC[s][k + 3]};
        }
      if (more) bc_store(buf ^ 1, nbc);
      __syncthreads();
      // one step per thread (kBW = 64 kMWaves), one row of dB or dC per pass: the row's base is
      // uniform
      static_assert(kBW == 64 * kMWaves, "one step per thread");
      {
        const int64_t t = w * kBW + (int64_t)threadIdx.x;
#pragma unroll
        for (int which = 0; which < 2 * SP; ++which) {
          const int n = SP * pp + (which % SP);
          if (n < N && t < L) {
            float v = 0.f;
#pragma unroll
            for (int wv2 = 0; wv2 < kMWaves; ++wv2) v += red[rb][wv2][which][threadIdx.x];
            float* const base = which < SP ? dBg + n * p.dB_sn : dCg + n * p.dC_sn;
            atomicAdd(base + t, v);
          }
        }
      }
      // (no second barrier: the next state writes the other buffer, and this one again only
      // after the next state's barrier, which every thread reaches after these sums)
      buf ^= 1;
      rb ^= 1;
    }
    // per-step outputs of the window
    float* dur = p.du + b * p.du_sb + d * p.du_sd;
    float* ddr = p.ddelta + b * p.dd_sb + hd * p.dd_sh;
    float dxs[kBK], uu[kBK];
    {
      float dv[kBK];
      load_seg<kBK>(dr, t0, L, p.vec, dv);
      load_seg<kBK>(ur, t0, L, p.vec, uu);
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        // softplus'(x) = sigmoid(x)
        const float x = dv[k] + bias;
        const float sg = p.softplus ? 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)) : 1.f;
        // with gB = sum_n g B: du = dt gB + D dy0 and ddt += u gB
        const float gB = du[k];
        du[k] = fmaf(dt[k], gB, dy0[k] * Dd);
        ddt[k] = fmaf(uu[k], gB, ddt[k]);
        dxs[k] = (valid && t0 + k < L) ? ddt[k] * sg : 0.f;
      }
    }
    if (p.chan_per_head % kMWaves == 0 && p.chan_per_group % kMWaves == 0) {
      // the block's 8 channels share the head: summed through LDS, one atomic add per step
#pragma unroll
      for (int k = 0; k < kBK; k += 4)
        *reinterpret_cast<f32x4*>(&red[rb][wave][0][lane * kBK + k]) = f32x4{dxs[k], dxs[k + 1], dxs[k + 2], dxs[k + 3]};
      __syncthreads();
      for (int i = threadIdx.x; i < kBW; i += 64 * kMWaves) {
        const int64_t t = w * kBW + i;
        float v = 0.f;
#pragma unroll
        for (int wv2 = 0; wv2 < kMWaves; ++wv2) v += red[rb][wv2][0][i];
        if (t < L) atomicAdd(ddr + t, v);
      }
      __syncthreads();
    } else if (valid && p.chan_per_head == 1) {
      store_steps(ddr, t0, L, dxs);
    } else if (valid) {
#pragma unroll
      for (int k = 0; k < kBK; ++k)
        if (t0 + k < L) atomicAdd(ddr + t0 + k, dxs[k]);
    }
    if (valid) {
      store_steps(dur, t0, L, du);
#pragma unroll
      for (int k = 0; k < kBK; ++k) {
        if (t0 + k < L) {
          dbacc += dxs[k];
          dDacc = fmaf(dy0[k], uu[k], dDacc);
        }
      }
    }
  }
  // per-channel sums (over this batch row's steps): dA, dD, dbias, added across the batch
  const float dDs = wave_sum(dDacc), dbs = wave_sum(dbacc);
  if (!valid) return;
  if (lane == 0) {
    if (p.dD) atomicAdd(p.dD + (p.d_per_head ? hd : d), dDs);
    if (p.dbias) atomicAdd(p.dbias + hd, dbs);
    if (SCALAR) atomicAdd(p.dA + hd, dAl[wave][0]);
  }
  if (!SCALAR)
    for (int n = lane; n < N; n += 64) atomicAdd(p.dA + d * p.dA_sd + n, dAl[wave][n]);
}

// Up to kZeroJobs float regions set to zero by one launch: region k is p[i0 s0 + i1 s1 + i2 s2 +
// i3] over [n0, n1, n2, n3] (innermost stride 1).  The summed gradients start at zero; a kernel
// rather than a memset, so that a caller may capture the call in a graph.
constexpr int kZeroJobs = 6;
struct ZeroJobs {
  float* p[kZeroJobs];
  int64_t n[kZeroJobs][4];
  int64_t st[kZeroJobs][3];
  int count;
};

__global__ __launch_bounds__(256) void zero_kernel(ZeroJobs z) {
#pragma unroll
  for (int k = 0; k < kZeroJobs; ++k) {
    if (k >= z.count) break;
    const int64_t n1 = z.n[k][1], n2 = z.n[k][2], n3 = z.n[k][3];
    const int64_t total = z.n[k][0] * n1 * n2 * n3;
    float* const p = z.p[k];
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
      const int64_t i3 = i % n3, r = i / n3;
      const int64_t i2 = r % n2, r2 = r / n2;
      const int64_t i1 = r2 % n1, i0 = r2 / n1;
      p[i0 * z.st[k][0] + i1 * z.st[k][1] + i2 * z.st[k][2] + i3] = 0.f;
    }
  }
}

// The gate's backward: dz = dy y0 s'(z), and y0 (the output before the gate, recomputed by the
// forward into `y0`, [batch, channels, L] contiguous) replaced in place by dy0 = dy s(z), the
// gradient the ungated backward takes.
template <typename TIn, typename TDy>
__global__ __launch_bounds__(256) void gate_bwd_kernel(BwdArgs p, float* __restrict__ y0) {
  const int64_t total = p.batch * p.channels * p.L;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i % p.L, r = i / p.L;
    const int64_t d = r % p.channels, b = r / p.channels;
    const float zz = to_f32(static_cast<const TIn*>(p.z)[b * p.z_sb + d * p.z_sd + t]);
    const float g = to_f32(static_cast<const TDy*>(p.dy)[b * p.dy_sb + d * p.dy_sd + t]);
    // s(z) = z sigmoid(z), s'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
    const float sgz = 1.f / (1.f + __builtin_amdgcn_exp2f(-zz * kLog2e));
    p.dz[b * p.dz_sb + d * p.dz_sd + t] = g * y0[i] * sgz * fmaf(zz, 1.f - sgz, 1.f);
    y0[i] = g * (zz * sgz);
  }
}

template <typename TIn, typename TDy>
hipError_t launch_t(const BwdArgs& a, float* ws, hipStream_t s) {
  const int P = (a.N + 1) / 2;
  const int64_t nwin = (a.L + kBW - 1) / kBW;
  const int64_t rows = a.batch * a.channels;
  // the summed gradients start at zero (one kernel for all of them, not a memset: callers may
  // capture this)
  ZeroJobs zj{};
  int64_t zmax = 0;
  auto zero4 = [&](float* ptr, int64_t n0, int64_t n1, int64_t n2, int64_t n3, int64_t s0, int64_t s1, int64_t s2) {
    const int64_t total = n0 * n1 * n2 * n3;
    if (!ptr || total == 0) return;
    const int k = zj.count++;
    zj.p[k] = ptr;
    zj.n[k][0] = n0, zj.n[k][1] = n1, zj.n[k][2] = n2, zj.n[k][3] = n3;
    zj.st[k][0] = s0, zj.st[k][1] = s1, zj.st[k][2] = s2;
    zmax = std::max(zmax, total);
  };
  zero4(a.dD, 1, 1, 1, a.d_per_head ? a.heads : a.channels, 0, 0, 0);
  zero4(a.dbias, 1, 1, 1, a.heads, 0, 0, 0);
  if (a.scalar) zero4(a.dA, 1, 1, 1, a.heads, 0, 0, 0);
  else zero4(a.dA, 1, 1, a.channels, a.N, 0, 0, a.dA_sd);
  // a head's channels add into its step-size gradient
  if (a.chan_per_head > 1) zero4(a.ddelta, a.batch, 1, a.heads, a.L, a.dd_sb, 0, a.dd_sh);
  zero4(a.dB, a.batch, a.groups, a.N, a.L, a.dB_sb, a.dB_sg, a.dB_sn);
  zero4(a.dC, a.batch, a.groups, a.N, a.L, a.dC_sb, a.dC_sg, a.dC_sn);
  if (zj.count)
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<int64_t>((zmax + 255) / 256, 8192)), dim3(256), 0, s, zj);
  if (ssd_bwd_path(a)) return launch_ssd_bwd(a, ws, s);
  const dim3 cgrid((unsigned)((rows + kBWaves - 1) / kBWaves)), block(64 * kBWaves);
  if (!a.ckpt_ready) {
    if (a.scalar) hipLaunchKernelGGL((bwd_ckpt_kernel<TIn, true>), cgrid, block, 0, s, a, P, nwin, ws);
    else hipLaunchKernelGGL((bwd_ckpt_kernel<TIn, false>), cgrid, block, 0, s, a, P, nwin, ws);
  }
  // sequence segments: the pre-pass's results follow the checkpoints in the workspace
  const BwdSegs sp = bwd_seg_plan(a);
  float* segw = ws + rows * nwin * a.N;
  if (sp.nseg > 1) {
    const dim3 sgrid((unsigned)((rows * (sp.nseg - 1) + 3) / 4));
#define SS_SEG(SC, FG)                                                                                     \
  do {                                                                                                     \
    if (a.N <= 16) hipLaunchKernelGGL((bwd_seg_kernel<TIn, TDy, SC, FG, 16>), sgrid, dim3(256), 0, s, a, sp.wps, sp.nseg, segw); \
    else hipLaunchKernelGGL((bwd_seg_kernel<TIn, TDy, SC, FG, kSegMaxN>), sgrid, dim3(256), 0, s, a, sp.wps, sp.nseg, segw); \
  } while (0)
    if (a.gz) {
      if (a.scalar) SS_SEG(true, true); else SS_SEG(false, true);
    } else {
      if (a.scalar) SS_SEG(true, false); else SS_SEG(false, false);
    }
#undef SS_SEG
  }
  const dim3 grid((unsigned)(a.batch * a.groups * ((a.chan_per_group + kMWaves - 1) / kMWaves) * sp.nseg));
  const dim3 mblock(64 * kMWaves);
  const float* ck = ws;
#define SS_BWD(SC, FG)                                                                                   \
  hipLaunchKernelGGL((bwd_kernel<TIn, TDy, SC, kBwdSP, FG>), grid, mblock, 0, s, a, (a.N + kBwdSP - 1) / kBwdSP, \
                     nwin, ck, sp.wps, sp.nseg, segw)
  // (a gated call arrives here with z taken apart by launch_bwd: gz and gy0 set, the gate folded in)
  if (a.gz) {
    if (a.scalar) SS_BWD(true, true); else SS_BWD(false, true);
  } else {
    if (a.scalar) SS_BWD(true, false); else SS_BWD(false, false);
  }
#undef SS_BWD
  return hipGetLastError();
}

// A gated layer composes the ungated backward with the gate: the forward without the gate
// recomputes y0 = C h + D u (the output before the gate) into f32 rows; dz = dy y0 s'(z) and
// dy0 = dy s(z) follow elementwise, and the ungated backward runs on dy0.  The gate multiplies
// C h + D u as a whole, so dy0 is the ungated layer's whole upstream gradient.  The per-channel
// kernel computes dz and dy0 itself where it loads dy; the matrix form gets dy0 from an
// elementwise pass that overwrites y0.
bool gated_path(const BwdArgs& a) {
  return a.z != nullptr;
}

constexpr int64_t round64(int64_t n) { return (n + 63) / 64 * 64; }

// the forward without the gate, y0 into `y0` ([batch, channels, L] f32, contiguous)
ScanArgs ungated_forward(const BwdArgs& a, float* y0) {
  ScanArgs f{};
  f.u = a.u;
  f.delta = a.delta;
  f.B = a.B;
  f.C = a.C;
  f.z = nullptr;
  f.A = a.A;
  f.D = a.D;
  f.bias = a.bias;
  f.y = y0;
  f.batch = a.batch;
  f.channels = a.channels;
  f.L = a.L;
  f.N = a.N;
  f.heads = a.heads;
  f.groups = a.groups;
  f.chan_per_head = a.chan_per_head;
  f.chan_per_group = a.chan_per_group;
  f.d_per_head = a.d_per_head;
  f.softplus = a.softplus;
  f.in_bf16 = a.in_bf16;
  f.out_bf16 = 0;
  f.vec = a.vec && a.L % 4 == 0;   // y0's rows are L floats from a 256-byte aligned base
  f.u_sb = a.u_sb;
  f.u_sd = a.u_sd;
  f.dl_sb = a.dl_sb;
  f.dl_sh = a.dl_sh;
  f.B_sb = a.B_sb;
  f.B_sg = a.B_sg;
  f.B_sn = a.B_sn;
  f.C_sb = a.C_sb;
  f.C_sg = a.C_sg;
  f.C_sn = a.C_sn;
  f.y_sb = a.channels * a.L;
  f.y_sd = a.L;
  f.A_sd = a.scalar ? 0 : a.A_sd;
  return f;
}

// diagonal decay (A [channels, N]) takes no workspace
int64_t forward_ws_floats(const ScanArgs& f, bool scalar) {
  if (!scalar) return (diag_workspace_bytes(f) + 3) / 4;   // (sequence segments)
  return ssd_path(f) ? (ssd_workspace_bytes(f) + 3) / 4 : scalar_workspace_floats(f);
}

// An ungated diagonal layer on the window-slot path (few rows): the forward stores the
// checkpoints as it goes (on sequence segments where they apply) several times faster than the
// checkpoint pass, which walks each row's whole sequence on one wave; its output goes to a
// scratch row of L floats per (batch, channel)
bool fwd_checkpoints(const BwdArgs& a) {
  return !a.scalar && !a.z && !a.ckpt_ready && !ssd_bwd_path(a) && diag_slots_path(ungated_forward(a, nullptr));
}

// floats of the per-channel path's checkpoints and segment pre-pass
int64_t ckpt_seg_floats(const BwdArgs& a) {
  const BwdSegs sp = bwd_seg_plan(a);
  const int64_t rows = a.batch * a.channels;
  return rows * ((a.L + kBW - 1) / kBW) * a.N + (sp.nseg > 1 ? rows * sp.nseg * (a.N + 1) : 0);
}

}  // namespace

int64_t bwd_workspace_floats(const BwdArgs& a) {
  if (gated_path(a)) {
    BwdArgs b = a;
    b.z = nullptr;
    b.ckpt_ready = !a.scalar && !ssd_bwd_path(b) ? 1 : 0;   // as the launch sets it
    const int64_t ny = round64(a.batch * a.channels * a.L);
    return ny + round64(forward_ws_floats(ungated_forward(a, nullptr), a.scalar)) + bwd_workspace_floats(b);
  }
  if (ssd_bwd_path(a)) return ssd_bwd_workspace_floats(a);
  // the checkpoints, then (with sequence segments) the pre-pass's N + 1 floats per (row, segment),
  // then (checkpoints from the forward) its output and workspace
  if (!fwd_checkpoints(a)) return ckpt_seg_floats(a);
  return round64(ckpt_seg_floats(a)) + round64(a.batch * a.channels * a.L) +
         forward_ws_floats(ungated_forward(a, nullptr), false);
}

hipError_t launch_bwd(const BwdArgs& a, float* ws, hipStream_t s) {
  if (gated_path(a)) {
    float* y0 = ws;
    float* fws = y0 + round64(a.batch * a.channels * a.L);
    ScanArgs f = ungated_forward(a, y0);
    float* bws = fws + round64(forward_ws_floats(f, a.scalar));
    // a diagonal decay's forward also stores the per-channel backward's checkpoints (at the
    // start of its workspace), which then needs no checkpoint pass of its own
    BwdArgs b = a;
    b.z = nullptr;
    const bool fwd_ckpt = !a.scalar && !ssd_bwd_path(b);
    if (fwd_ckpt) {
      f.ckpt = bws;
      f.ckpt_nwin = (a.L + kBW - 1) / kBW;
    }
    hipError_t e = !a.scalar ? launch_diag(f, fws, s) : ssd_path(f) ? launch_ssd(f, fws, s) : launch_scalar(f, fws, s);
    if (e != hipSuccess) return e;
    b.ckpt_ready = fwd_ckpt ? 1 : 0;
    if (!ssd_bwd_path(b)) {
      // the per-channel kernel takes the gate itself (dz and dy0 where it loads dy): no pass of
      // its own, y0 read once
      b.gz = a.z;
      b.gy0 = y0;
      b.y0_vec = a.L % 4 == 0;
      return launch_bwd(b, bws, s);
    }
    const int64_t total = a.batch * a.channels * a.L;
    const dim3 grid((unsigned)std::min<int64_t>((total + 255) / 256, 16384));
#define SS_GATE(TI, TD) hipLaunchKernelGGL((gate_bwd_kernel<TI, TD>), grid, dim3(256), 0, s, a, y0)
    if (a.in_bf16) {
      if (a.dy_bf16) SS_GATE(bf16_t, bf16_t); else SS_GATE(bf16_t, float);
    } else {
      if (a.dy_bf16) SS_GATE(float, bf16_t); else SS_GATE(float, float);
    }
#undef SS_GATE
    b.dz = nullptr;
    b.dy = y0;
    b.dy_bf16 = 0;
    b.dy_sb = a.channels * a.L;
    b.dy_sd = a.L;
    b.vec = a.vec && a.L % 4 == 0;
    return launch_bwd(b, bws, s);
  }
  if (fwd_checkpoints(a)) {
    float* y0 = ws + round64(ckpt_seg_floats(a));
    ScanArgs f = ungated_forward(a, y0);
    f.ckpt = ws;
    f.ckpt_nwin = (a.L + kBW - 1) / kBW;
    const hipError_t e = launch_diag(f, y0 + round64(a.batch * a.channels * a.L), s);
    if (e != hipSuccess) return e;
    BwdArgs b = a;
    b.ckpt_ready = 1;
    return launch_bwd(b, ws, s);
  }
  if (a.in_bf16) return a.dy_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.dy_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
