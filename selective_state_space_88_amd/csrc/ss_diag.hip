// ss_diag.hip -- selective-scan forward with a diagonal decay A[d, n] (Mamba-1 S6), gfx950.
//
// Method (omica.com.cn Mamba explainer, sections 3 and 5; exponential-Euler per section 6.3):
//   h_t = exp(dt_t A_n) h_{t-1} + dt_t B_{t,n} u_t,   y_t = sum_n C_{t,n} h_t + D u_t
// The recurrence is linear in h, so consecutive steps compose with the associative operator
//   (a1, b1) then (a2, b2)  =  (a1 a2, a2 b1 + b2)
// which is what makes the parallel scan of the pages (Blelloch's work-efficient scan, named in
// the study notes' history and the bqwf.cn survey section 2.2) possible.
//
// Mapping on gfx950 (wave64):
//  - one wave per (b, d) row; its 64 lanes lie along time, lane j owning K consecutive steps,
//    so one window of the row covers 64*K steps; windows are walked in order and the state at
//    the end of each window is carried in registers to the next;
//  - the N states are processed one after another (n outer).  For state n each lane runs its
//    K steps once from zero (keeping the K decays a_t and inputs b_t in registers), the wave
//    combines the 64 lane aggregates with a DPP scan, and each lane re-runs its K steps from
//    the true incoming state to form h_t and accumulate y_t += C_{t,n} h_t.  Every exp is
//    evaluated once; the re-run costs one extra FMA per (t, n);
//  - softplus, D*u and the silu gate are fused; u, delta, z, y stream through HBM once, B and
//    C rows are shared by all channels of a group and come from L2.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kK = 16;              // steps per lane
constexpr int kWindow = 64 * kK;    // steps per wave window
constexpr int kWavesPerBlock = 4;

// Inclusive scan of (a, b) pairs over the 64 lanes, earliest lane first.
__device__ __forceinline__ void wave_scan_pairs(float& a, float& b, int lane) {
  const int lr = lane & 15;
#define SS_ROW_STEP(S)                                   \
  {                                                      \
    const float pa = dpp_f<0x110 + S>(a);                \
    const float pb = dpp_f<0x110 + S>(b);                \
    if (lr >= S) {                                       \
      b = fmaf(a, pb, b);                                \
      a = a * pa;                                        \
    }                                                    \
  }
  SS_ROW_STEP(1)
  SS_ROW_STEP(2)
  SS_ROW_STEP(4)
  SS_ROW_STEP(8)
#undef SS_ROW_STEP
  // rows of 16 are scanned; now prefix the row totals (lanes 15, 31, 47)
  const float a0 = readlane_f(a, 15), b0 = readlane_f(b, 15);
  const float a1 = readlane_f(a, 31), b1 = readlane_f(b, 31);
  const float a2 = readlane_f(a, 47), b2 = readlane_f(b, 47);
  const float p2a = a0 * a1, p2b = fmaf(a1, b0, b1);
  const float p3a = p2a * a2, p3b = fmaf(a2, p2b, b2);
  const int row = lane >> 4;
  float pa = 1.f, pb = 0.f;
  if (row == 1) { pa = a0; pb = b0; }
  if (row == 2) { pa = p2a; pb = p2b; }
  if (row == 3) { pa = p3a; pb = p3b; }
  b = fmaf(a, pb, b);
  a = a * pa;
}

template <typename TIn, typename TOut, bool GATE>
__global__ __launch_bounds__(64 * kWavesPerBlock) void diag_fwd_kernel(ScanArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= p.batch * p.channels) return;  // whole wave leaves; no block barriers below
  const int64_t b = row / p.channels, d = row % p.channels;
  const int64_t hd = d / p.chan_per_head, g = d / p.chan_per_group;
  const int64_t L = p.L;
  const int N = p.N;
  const bool vec = p.vec != 0;

  const TIn* __restrict__ u = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* __restrict__ dl = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TIn* __restrict__ zr = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  const TIn* __restrict__ Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* __restrict__ Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  TOut* __restrict__ y = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
  const float* __restrict__ Arow = p.A + d * p.A_sd;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  const float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;

  // carried state at the start of the current window: lane n holds state n (n < 64) in c0,
  // state 64 + n in c1.
  float c0 = 0.f, c1 = 0.f;

  for (int64_t w0 = 0; w0 < L; w0 += kWindow) {
    const int64_t t0 = w0 + (int64_t)lane * kK;
    float dt[kK], wv[kK], yv[kK];
    {
      float uv[kK];
      load_seg<kK>(u, t0, L, vec, uv);
      load_seg<kK>(dl, t0, L, vec, dt);
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        const float x = dt[j] + bias;
        float s = p.softplus ? softplus_f32(x) : x;
        if (t0 + j >= L) s = 0.f;  // steps past the end are the identity (a = 1, b = 0)
        dt[j] = s;
        wv[j] = s * uv[j];
        yv[j] = Dd * uv[j];
      }
    }
    float sdt = 0.f;
#pragma unroll
    for (int j = 0; j < kK; ++j) sdt += dt[j];

    for (int n = 0; n < N; ++n) {
      const float An = Arow[n] * kLog2e;
      float Bv[kK], Cv[kK];
      load_seg<kK>(Bg + n * p.B_sn, t0, L, vec, Bv);
      load_seg<kK>(Cg + n * p.C_sn, t0, L, vec, Cv);
      float av[kK], bv[kK];
      float h = 0.f;
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        av[j] = __builtin_amdgcn_exp2f(dt[j] * An);
        bv[j] = wv[j] * Bv[j];
        h = fmaf(av[j], h, bv[j]);
      }
      float sa = __builtin_amdgcn_exp2f(sdt * An);  // product of this lane's decays
      float sb = h;                                  // this lane's state from zero
      wave_scan_pairs(sa, sb, lane);
      // exclusive prefix: the lane before me
      float ea = __shfl_up(sa, 1, 64);
      float eb = __shfl_up(sb, 1, 64);
      if (lane == 0) {
        ea = 1.f;
        eb = 0.f;
      }
      const float cin = n < 64 ? readlane_f(c0, n) : readlane_f(c1, n - 64);
      h = fmaf(ea, cin, eb);
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        h = fmaf(av[j], h, bv[j]);
        yv[j] = fmaf(Cv[j], h, yv[j]);
      }
      const float hend = readlane_f(h, 63);
      if (n < 64) {
        if (lane == n) c0 = hend;
      } else {
        if (lane == n - 64) c1 = hend;
      }
    }

    if constexpr (GATE) {
      float zv[kK];
      load_seg<kK>(zr, t0, L, vec, zv);
#pragma unroll
      for (int j = 0; j < kK; ++j) yv[j] *= silu_f32(zv[j]);
    }
    store_seg<kK>(y, t0, L, vec, yv);
  }
}

template <typename TIn, typename TOut>
hipError_t launch_t(const ScanArgs& a, hipStream_t s) {
  const int64_t rows = a.batch * a.channels;
  const dim3 grid((unsigned)((rows + kWavesPerBlock - 1) / kWavesPerBlock));
  const dim3 block(64 * kWavesPerBlock);
  if (a.z)
    hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diag(const ScanArgs& a, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, s) : launch_t<float, float>(a, s);
}

}  // namespace ss
