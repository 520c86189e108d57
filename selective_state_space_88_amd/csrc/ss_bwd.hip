// ss_bwd.hip -- backward of the diagonal selective scan (gradients of every input), gfx950.
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
// and per step dz_t = dy_t y0_t s'(z_t), du_t += dy0_t D, dD += dy0_t u_t,
// ddelta_t = ddt_t sigmoid(x_t) (softplus'), dbias += ddelta_t.
//
// Mapping (as in the forward kernel): a wave owns one channel, lane j the K consecutive steps
// t0 + jK .. t0 + jK + K - 1 of a window; states go by pairs.  Inside a window both recurrences
// are scans of affine maps over the lanes: the states forward (x -> a x + b composed left to
// right), the adjoint backward (composed right to left); each lane runs its K steps from zero,
// the lanes' maps are combined by a shuffle scan, and each lane re-runs its steps from its true
// incoming value.  A block holds 4 channels of one (batch, B/C group): their dB and dC
// contributions are summed through LDS before one atomic add per (state, step).
#include <algorithm>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kBK = 8;               // steps per lane
constexpr int kBW = 64 * kBK;        // steps per window
constexpr int kBWaves = 4;           // channels per block
constexpr int kBMaxPairs = 64;       // N <= 128

// Inclusive scan of affine maps x -> A x + B over the 64 lanes, composed left to right (lane j
// ends with the map of lanes 0..j applied in order).
__device__ __forceinline__ void scan_up(float& A, float& B, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float Ao = __shfl_up(A, off), Bo = __shfl_up(B, off);
    if (lane >= off) {
      B = fmaf(A, Bo, B);
      A = A * Ao;
    }
  }
}

// Inclusive scan composed right to left (lane j ends with the map of lanes 63..j, lane 63's
// applied first).
__device__ __forceinline__ void scan_down(float& A, float& B, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float Ao = __shfl_down(A, off), Bo = __shfl_down(B, off);
    if (lane + off < 64) {
      B = fmaf(A, Bo, B);
      A = A * Ao;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename TIn>
__device__ __forceinline__ float ld(const TIn* p, int64_t i, bool ok) {
  return ok ? to_f32(p[i]) : 0.f;
}

// Checkpoints: the state of every (row, window, state) at the window's start.
template <typename TIn>
__global__ __launch_bounds__(64 * kBWaves) void bwd_ckpt_kernel(BwdArgs p, int P, int64_t nwin, float* ckpt) {
  __shared__ float hst[kBWaves][kBMaxPairs][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * kBWaves + wave;  // b * channels + d
  const bool live = row < p.batch * p.channels;
  const int64_t rr = live ? row : 0;
  const int64_t b = rr / p.channels, d = rr % p.channels;
  const int64_t g = d / p.chan_per_group;
  const int N = p.N;
  const TIn* ur = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* dr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + d * p.dl_sh;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const float bias = p.bias ? p.bias[d] : 0.f;
  for (int pp = lane; pp < P; pp += 64) hst[wave][pp][0] = hst[wave][pp][1] = 0.f;
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    float dt[kBK], wv[kBK];
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const bool ok = t0 + k < p.L;
      const float x = ld(dr, t0 + k, ok) + bias;
      dt[k] = ok ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      wv[k] = dt[k] * ld(ur, t0 + k, ok);
    }
    for (int pp = 0; pp < P; ++pp) {
      float Af[2], Bf[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = 2 * pp + s;
        const bool nv = n < N;
        const float A2 = nv ? p.A[d * p.A_sd + n] * kLog2e : 0.f;
        float a = 1.f, h = 0.f;
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          const float av = __builtin_amdgcn_exp2f(dt[k] * A2);
          h = fmaf(av, h, wv[k] * ld(Bg + (nv ? n : 0) * p.B_sn, t0 + k, nv && t0 + k < p.L));
          a *= av;
        }
        Af[s] = a;
        Bf[s] = h;
        scan_up(Af[s], Bf[s], lane);
      }
      // the window's start state is stored, and its end state (lane 63's map) carried on
      const float h0 = hst[wave][pp][0], h1 = hst[wave][pp][1];
      if (live && lane == 0) {
        float* c = ckpt + (row * nwin + w) * N;
        c[2 * pp] = h0;
        if (2 * pp + 1 < N) c[2 * pp + 1] = h1;
      }
      const float e0 = __shfl(fmaf(Af[0], h0, Bf[0]), 63), e1 = __shfl(fmaf(Af[1], h1, Bf[1]), 63);
      if (lane == 0) {
        hst[wave][pp][0] = e0;
        hst[wave][pp][1] = e1;
      }
    }
  }
}

template <typename TIn, typename TDy, bool GATE>
__global__ __launch_bounds__(64 * kBWaves) void bwd_kernel(BwdArgs p, int P, int64_t nwin, const float* ckpt) {
  __shared__ float gcar[kBWaves][kBMaxPairs][2];      // adjoint carried into the window from the right
  __shared__ float dAl[kBWaves][2 * kBMaxPairs];      // dA partial sums of the wave's channel
  // dB (2 states), dC (2 states) of the window's steps, step-major ([lane][k] = step lane K + k)
  __shared__ __attribute__((aligned(16))) float red[kBWaves][4][kBW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t quads = p.chan_per_group / kBWaves;
  const int64_t bg = blockIdx.x / quads, qd = blockIdx.x % quads;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t d = g * p.chan_per_group + qd * kBWaves + wave;
  const int64_t row = b * p.channels + d;
  const int N = p.N;
  const int64_t L = p.L;
  const TIn* ur = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* dr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + d * p.dl_sh;
  const TIn* zr = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  const TDy* dyr = static_cast<const TDy*>(p.dy) + b * p.dy_sb + d * p.dy_sd;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  float* dBg = p.dB + b * p.dB_sb + g * p.dB_sg;
  float* dCg = p.dC + b * p.dC_sb + g * p.dC_sg;
  const float bias = p.bias ? p.bias[d] : 0.f;
  const float Dd = p.D ? p.D[d] : 0.f;
  for (int i = lane; i < 2 * kBMaxPairs; i += 64) {
    gcar[wave][i / 2][i % 2] = 0.f;
    dAl[wave][i] = 0.f;
  }
  float dDacc = 0.f, dbacc = 0.f;

  for (int64_t w = nwin - 1; w >= 0; --w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    float dt[kBK], uu[kBK], wv[kBK], dy0[kBK], y0[kBK], du[kBK], ddt[kBK], sg[kBK], dyv[kBK], zv[kBK];
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const bool ok = t0 + k < L;
      const float x = ld(dr, t0 + k, ok) + bias;
      dt[k] = ok ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      // softplus'(x) = sigmoid(x)
      sg[k] = p.softplus ? 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)) : 1.f;
      uu[k] = ld(ur, t0 + k, ok);
      wv[k] = dt[k] * uu[k];
      dyv[k] = ok ? to_f32(dyr[t0 + k]) : 0.f;
      float gz = 1.f;
      if constexpr (GATE) {
        zv[k] = ld(zr, t0 + k, ok);
        gz = silu_fast(zv[k]);
      }
      dy0[k] = dyv[k] * gz;
      y0[k] = Dd * uu[k];
      du[k] = dy0[k] * Dd;
      ddt[k] = 0.f;
    }
    for (int pp = 0; pp < P; ++pp) {
      float rB[2][kBK], rC[2][kBK];
      float dAp[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = 2 * pp + s;
        const bool nv = n < N;
        const float An = nv ? p.A[d * p.A_sd + n] : 0.f;
        const float A2 = An * kLog2e;
        const TIn* Br = Bg + (nv ? n : 0) * p.B_sn;
        const TIn* Cr = Cg + (nv ? n : 0) * p.C_sn;
        float av[kBK], bv[kBK], cv[kBK];
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          const bool ok = nv && t0 + k < L;
          av[k] = __builtin_amdgcn_exp2f(dt[k] * A2);
          bv[k] = ld(Br, t0 + k, ok);
          cv[k] = ld(Cr, t0 + k, ok);
        }
        // states: the lane's steps from zero, the scan, then from the incoming state
        float Af = 1.f, Bf = 0.f;
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          Bf = fmaf(av[k], Bf, wv[k] * bv[k]);
          Af *= av[k];
        }
        const float Pl = Af;   // the lane's total decay (both directions)
        scan_up(Af, Bf, lane);
        float Ae = __shfl_up(Af, 1), Be = __shfl_up(Bf, 1);
        if (lane == 0) {
          Ae = 1.f;
          Be = 0.f;
        }
        const float hw = nv ? ckpt[(row * nwin + w) * N + n] : 0.f;
        float hs[kBK + 1];
        hs[0] = fmaf(Ae, hw, Be);
#pragma unroll
        for (int k = 0; k < kBK; ++k) {
          hs[k + 1] = fmaf(av[k], hs[k], wv[k] * bv[k]);
          y0[k] = fmaf(cv[k], hs[k + 1], y0[k]);
        }
        // adjoint: the lane's steps from zero (right to left), the scan, then from the value
        // carried in from the right
        float c = 0.f;
#pragma unroll
        for (int k = kBK - 1; k >= 0; --k) c = av[k] * fmaf(cv[k], dy0[k], c);
        float Ar = Pl, Br2 = c;
        scan_down(Ar, Br2, lane);
        float Ad = __shfl_down(Ar, 1), Bd = __shfl_down(Br2, 1);
        if (lane == 63) {
          Ad = 1.f;
          Bd = 0.f;
        }
        const float Xw = gcar[wave][pp][s];
        c = fmaf(Ad, Xw, Bd);
        float dAs = 0.f;
#pragma unroll
        for (int k = kBK - 1; k >= 0; --k) {
          const float gk = fmaf(cv[k], dy0[k], c);
          rC[s][k] = dy0[k] * hs[k + 1];
          rB[s][k] = gk * wv[k];
          du[k] = fmaf(gk * dt[k], bv[k], du[k]);
          const float gha = gk * hs[k] * av[k];
          ddt[k] = fmaf(gha, An, fmaf(gk * bv[k], uu[k], ddt[k]));
          dAs = fmaf(gha, dt[k], dAs);
          c = av[k] * gk;
        }
        // the adjoint carried into the previous window: lane 0's value after its first step
        const float cl = __shfl(c, 0);
        if (lane == 0) gcar[wave][pp][s] = cl;
        dAp[s] = dAs;
      }
      // dA of the pair: summed over the wave's lanes into the wave's partial sums
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float v = wave_sum(dAp[s]);
        if (lane == 0 && 2 * pp + s < N) dAl[wave][2 * pp + s] += v;
      }
      // dB, dC of the pair: summed over the block's 4 channels, then one atomic add per step;
      // consecutive lanes add to consecutive steps, so each wave's adds cover two cache lines
#pragma unroll
      for (int k = 0; k < kBK; k += 4) {
        *reinterpret_cast<f32x4*>(&red[wave][0][lane * kBK + k]) = f32x4{rB[0][k], rB[0][k + 1], rB[0][k + 2], rB[0][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][1][lane * kBK + k]) = f32x4{rB[1][k], rB[1][k + 1], rB[1][k + 2], rB[1][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][2][lane * kBK + k]) = f32x4{rC[0][k], rC[0][k + 1], rC[0][k + 2], rC[0][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][3][lane * kBK + k]) = f32x4{rC[1][k], rC[1][k + 1], rC[1][k + 2], rC[1][k + 3]};
      }
      __syncthreads();
      for (int i = threadIdx.x; i < 4 * kBW; i += 64 * kBWaves) {
        const int which = i / kBW, r = i % kBW;
        const int n = 2 * pp + (which & 1);
        const int64_t t = w * kBW + r;
        if (n < N && t < L) {
          const float v = red[0][which][r] + red[1][which][r] + red[2][which][r] + red[3][which][r];
          float* dst = (which < 2 ? dBg + n * p.dB_sn : dCg + n * p.dC_sn) + t;
          atomicAdd(dst, v);
        }
      }
      __syncthreads();
    }
    // per-step outputs of the window
    float* dur = p.du + b * p.du_sb + d * p.du_sd;
    float* ddr = p.ddelta + b * p.dd_sb + d * p.dd_sh;
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      if (t0 + k < L) {
        const float dx = ddt[k] * sg[k];
        dur[t0 + k] = du[k];
        ddr[t0 + k] = dx;
        dbacc += dx;
        dDacc = fmaf(dy0[k], uu[k], dDacc);
        if constexpr (GATE) {
          // s'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
          const float sgz = 1.f / (1.f + __builtin_amdgcn_exp2f(-zv[k] * kLog2e));
          p.dz[b * p.dz_sb + d * p.dz_sd + t0 + k] = dyv[k] * y0[k] * sgz * fmaf(zv[k], 1.f - sgz, 1.f);
        }
      }
    }
  }
  // per-channel sums (over this batch row's steps): dA, dD, dbias, added across the batch
  const float dDs = wave_sum(dDacc), dbs = wave_sum(dbacc);
  if (lane == 0) {
    if (p.dD) atomicAdd(p.dD + d, dDs);
    if (p.dbias) atomicAdd(p.dbias + d, dbs);
  }
  for (int n = lane; n < N; n += 64) atomicAdd(p.dA + d * p.dA_sd + n, dAl[wave][n]);
}

// p[i0 * s0 + i1 * s1 + i2 * s2 + i3] = 0 over [n0, n1, n2, n3] (innermost stride 1)
__global__ __launch_bounds__(256) void zero4_kernel(float* __restrict__ p, int64_t n0, int64_t n1, int64_t n2,
                                                    int64_t n3, int64_t s0, int64_t s1, int64_t s2) {
  const int64_t total = n0 * n1 * n2 * n3;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t i3 = i % n3, r = i / n3;
    const int64_t i2 = r % n2, r2 = r / n2;
    const int64_t i1 = r2 % n1, i0 = r2 / n1;
    p[i0 * s0 + i1 * s1 + i2 * s2 + i3] = 0.f;
  }
}

template <typename TIn, typename TDy>
hipError_t launch_t(const BwdArgs& a, float* ws, hipStream_t s) {
  const int P = (a.N + 1) / 2;
  const int64_t nwin = (a.L + kBW - 1) / kBW;
  const int64_t rows = a.batch * a.channels;
  // the summed gradients start at zero (a kernel, not a memset: callers may capture this)
  auto zero4 = [&](float* ptr, int64_t n0, int64_t n1, int64_t n2, int64_t n3, int64_t s0, int64_t s1, int64_t s2) {
    const int64_t total = n0 * n1 * n2 * n3;
    if (!ptr || total == 0) return;
    hipLaunchKernelGGL(zero4_kernel, dim3((unsigned)std::min<int64_t>((total + 255) / 256, 8192)), dim3(256), 0, s,
                       ptr, n0, n1, n2, n3, s0, s1, s2);
  };
  zero4(a.dD, 1, 1, 1, a.channels, 0, 0, 0);
  zero4(a.dbias, 1, 1, 1, a.channels, 0, 0, 0);
  zero4(a.dA, 1, 1, a.channels, a.N, 0, 0, a.dA_sd);
  zero4(a.dB, a.batch, a.groups, a.N, a.L, a.dB_sb, a.dB_sg, a.dB_sn);
  zero4(a.dC, a.batch, a.groups, a.N, a.L, a.dC_sb, a.dC_sg, a.dC_sn);
  hipLaunchKernelGGL((bwd_ckpt_kernel<TIn>), dim3((unsigned)((rows + kBWaves - 1) / kBWaves)), dim3(64 * kBWaves),
                     0, s, a, P, nwin, ws);
  const int64_t blocks = a.batch * a.groups * (a.chan_per_group / kBWaves);
  if (a.z)
    hipLaunchKernelGGL((bwd_kernel<TIn, TDy, true>), dim3((unsigned)blocks), dim3(64 * kBWaves), 0, s, a, P, nwin,
                       static_cast<const float*>(ws));
  else
    hipLaunchKernelGGL((bwd_kernel<TIn, TDy, false>), dim3((unsigned)blocks), dim3(64 * kBWaves), 0, s, a, P, nwin,
                       static_cast<const float*>(ws));
  return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_floats(const BwdArgs& a) {
  return a.batch * a.channels * ((a.L + kBW - 1) / kBW) * a.N;
}

hipError_t launch_bwd(const BwdArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.dy_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.dy_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
