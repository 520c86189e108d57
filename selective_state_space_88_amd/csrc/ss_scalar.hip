// ss_scalar.hip -- selective-scan forward with one scalar decay per head (Mamba-2 style), gfx950.
//
// Method: the same recurrence as the diagonal case with A_t = alpha_t I (bqwf.cn state-space
// survey, section 3.2; omica.com.cn Mamba explainer, section 6.2): for channel p of head h,
//   a_t = exp(dt_{h,t} A_h),  h_{t,n} = a_t h_{t-1,n} + dt_{h,t} u_{p,t} B_{t,n},
//   y_{p,t} = sum_n C_{t,n} h_{t,n} + D u_{p,t}
// The decay and the B/C rows are shared by every channel of a head, so on gfx950:
//  - lanes run along channels (64 per wave) and each wave owns 16 of the N states; the B/C
//    values of those 16 states at step t are wave-uniform and enter the FMAs as SGPR operands
//    (scalar loads from an fp32, state-innermost copy of B and C made by a small transpose);
//  - each lane walks time sequentially with its 16 states in VGPRs: per (t, n) one multiply
//    (dt u B), one FMA for the state and one FMA for the readout;
//  - the ceil(N/16) waves of a block hold the same channels and different states; their partial
//    readouts are summed through LDS every kT steps and written once, with D*u and the gate.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kNT = 16;   // states per wave
constexpr int kT = 32;    // steps per block of time between partial-sum reductions
constexpr int kMaxWaves = 8;

int npad_of(int N) { return (N + kNT - 1) / kNT * kNT; }

// B, C [batch, groups, N, L] (strided, bf16/f32)  ->  ws [batch, groups, L, Npad] f32,
// zero for n >= N.  One block transposes 64 steps x Npad states through LDS.
template <typename TIn>
__global__ __launch_bounds__(256) void transpose_bc_kernel(const TIn* __restrict__ src, int64_t s_b,
                                                           int64_t s_g, int64_t s_n, int groups,
                                                           int N, int Npad, int64_t L,
                                                           float* __restrict__ dst) {
  __shared__ float tile[64][129];
  const int64_t tiles_per_row = (L + 63) / 64;
  const int64_t bg = blockIdx.x / tiles_per_row;
  const int64_t t0 = (blockIdx.x % tiles_per_row) * 64;
  const int64_t b = bg / groups, g = bg % groups;
  const TIn* s = src + b * s_b + g * s_g;
  // read: consecutive threads along t
  for (int idx = threadIdx.x; idx < 64 * Npad; idx += blockDim.x) {
    const int n = idx / 64, tt = idx % 64;
    const int64_t t = t0 + tt;
    float v = 0.f;
    if (n < N && t < L) v = to_f32(s[n * s_n + t]);
    tile[tt][n] = v;
  }
  __syncthreads();
  float* o = dst + (bg * L + t0) * Npad;
  for (int idx = threadIdx.x; idx < 64 * Npad; idx += blockDim.x) {
    const int tt = idx / Npad, n = idx % Npad;
    if (t0 + tt < L) o[(int64_t)tt * Npad + n] = tile[tt][n];
  }
}

template <typename TIn, typename TOut, bool GATE>
__global__ __launch_bounds__(64 * kMaxWaves) void scalar_fwd_kernel(ScanArgs p,
                                                                    const float* __restrict__ wsB,
                                                                    const float* __restrict__ wsC,
                                                                    int Npad) {
  __shared__ float part[kMaxWaves][64][kT + 1];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int64_t cblocks = (p.channels + 63) / 64;
  const int64_t b = blockIdx.x / cblocks;
  const int64_t d0 = (blockIdx.x % cblocks) * 64;
  const int64_t L = p.L;
  const int64_t dl_ = d0 + lane < p.channels ? d0 + lane : p.channels - 1;  // clamp idle lanes
  const int64_t hd = dl_ / p.chan_per_head;
  const int64_t g = d0 / p.chan_per_group;  // uniform: checked on the host

  const TIn* __restrict__ u = static_cast<const TIn*>(p.u) + b * p.u_sb + dl_ * p.u_sd;
  const TIn* __restrict__ dlr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const float An = p.A[hd] * kLog2e;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  // B/C rows are read-only for the whole kernel: read them through the constant address
  // space so that the wave-uniform loads become scalar loads into SGPRs.
  const cfloat* Bs = to_constant(wsB + (b * p.groups + g) * L * Npad + wv * kNT);
  const cfloat* Cs = to_constant(wsC + (b * p.groups + g) * L * Npad + wv * kNT);

  float h[kNT];
#pragma unroll
  for (int i = 0; i < kNT; ++i) h[i] = 0.f;

  for (int64_t tb = 0; tb < L; tb += kT) {
    float av[kT], wv_[kT];
    {
      float uv[kT], dv[kT];
      // per-lane rows; the time rows of u are not required to be vector aligned here
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        const bool ok = tb + j < L;
        uv[j] = ok ? to_f32(u[tb + j]) : 0.f;
        dv[j] = ok ? to_f32(dlr[tb + j]) : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        const float x = dv[j] + bias;
        float s = p.softplus ? softplus_fast(x) : x;
        if (tb + j >= L) s = 0.f;
        av[j] = __builtin_amdgcn_exp2f(s * An);
        wv_[j] = s * uv[j];
      }
    }
    float yp[kT];
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const int64_t t = tb + j < L ? tb + j : L - 1;  // uniform
      const cfloat* bt = Bs + t * Npad;
      const cfloat* ct = Cs + t * Npad;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < kNT; ++i) {
        h[i] = fmaf(av[j], h[i], wv_[j] * bt[i]);
        acc = fmaf(ct[i], h[i], acc);
      }
      yp[j] = acc;
    }
#pragma unroll
    for (int j = 0; j < kT; ++j) part[wv][lane][j] = yp[j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * kT; idx += blockDim.x) {
      const int c = idx / kT, j = idx % kT;
      const int64_t d = d0 + c, t = tb + j;
      if (d < p.channels && t < L) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += part[w][c][j];
        const int64_t hdc = d / p.chan_per_head;
        const float uu = to_f32(static_cast<const TIn*>(p.u)[b * p.u_sb + d * p.u_sd + t]);
        if (p.D) s = fmaf(p.D[p.d_per_head ? hdc : d], uu, s);
        if constexpr (GATE) s *= silu_fast(to_f32(static_cast<const TIn*>(p.z)[b * p.z_sb + d * p.z_sd + t]));
        store_one(static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd + t, s);
      }
    }
    __syncthreads();
  }
}

template <typename TIn>
hipError_t transpose(const ScanArgs& a, const void* src, int64_t sb, int64_t sg, int64_t sn,
                     float* dst, hipStream_t s) {
  const int Npad = npad_of(a.N);
  const int64_t blocks = a.batch * a.groups * ((a.L + 63) / 64);
  hipLaunchKernelGGL((transpose_bc_kernel<TIn>), dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const TIn*>(src), sb, sg, sn, a.groups, a.N, Npad, a.L, dst);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const ScanArgs& a, float* ws, hipStream_t s) {
  const int Npad = npad_of(a.N);
  const int64_t plane = a.batch * a.groups * a.L * Npad;
  hipError_t e = transpose<TIn>(a, a.B, a.B_sb, a.B_sg, a.B_sn, ws, s);
  if (e != hipSuccess) return e;
  e = transpose<TIn>(a, a.C, a.C_sb, a.C_sg, a.C_sn, ws + plane, s);
  if (e != hipSuccess) return e;
  const int64_t blocks = a.batch * ((a.channels + 63) / 64);
  const dim3 block(64 * (Npad / kNT));
  if (a.z)
    hipLaunchKernelGGL((scalar_fwd_kernel<TIn, TOut, true>), dim3((unsigned)blocks), block, 0, s, a,
                       ws, ws + plane, Npad);
  else
    hipLaunchKernelGGL((scalar_fwd_kernel<TIn, TOut, false>), dim3((unsigned)blocks), block, 0, s, a,
                       ws, ws + plane, Npad);
  return hipGetLastError();
}

}  // namespace

int64_t scalar_workspace_floats(const ScanArgs& a) {
  return 2 * a.batch * a.groups * a.L * (int64_t)npad_of(a.N);
}

hipError_t launch_scalar(const ScanArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
