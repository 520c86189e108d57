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

// The head-uniform path: every head's channels fill whole 64-lane waves.
// (each block of 64 channels then lies in one head and one B/C group)
bool head_path(const ScanArgs& a) {
  return a.chan_per_head % 64 == 0 && a.chan_per_group % 64 == 0 && a.channels % 64 == 0;
}

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

// B and C [batch, groups, N, L] -> ws [batch, groups, L, Npad/8, 16] f32: for each step and
// each group of 8 states, the 8 B values then the 8 C values (zero for n >= N), so that a
// wave owning 8 states reads one step with a single 64-byte scalar load.
template <typename TIn>
__global__ __launch_bounds__(256) void interleave_bc_kernel(const TIn* __restrict__ Bsrc,
                                                            const TIn* __restrict__ Csrc,
                                                            int64_t b_sb, int64_t b_sg, int64_t b_sn,
                                                            int64_t c_sb, int64_t c_sg, int64_t c_sn,
                                                            int groups, int N, int Npad, int64_t L,
                                                            float* __restrict__ dst) {
  __shared__ float tile[2][64][129];
  const int64_t tiles_per_row = (L + 63) / 64;
  const int64_t bg = blockIdx.x / tiles_per_row;
  const int64_t t0 = (blockIdx.x % tiles_per_row) * 64;
  const int64_t b = bg / groups, g = bg % groups;
  const TIn* sb = Bsrc + b * b_sb + g * b_sg;
  const TIn* sc = Csrc + b * c_sb + g * c_sg;
  for (int idx = threadIdx.x; idx < 64 * Npad; idx += blockDim.x) {
    const int n = idx / 64, tt = idx % 64;
    const int64_t t = t0 + tt;
    float vb = 0.f, vc = 0.f;
    if (n < N && t < L) {
      vb = to_f32(sb[n * b_sn + t]);
      vc = to_f32(sc[n * c_sn + t]);
    }
    tile[0][tt][n] = vb;
    tile[1][tt][n] = vc;
  }
  __syncthreads();
  float* o = dst + (bg * L + t0) * (2 * Npad);
  for (int idx = threadIdx.x; idx < 64 * 2 * Npad; idx += blockDim.x) {
    const int tt = idx / (2 * Npad), r = idx % (2 * Npad);
    const int grp = r / 16, k = r % 16;
    const int n = grp * 8 + (k % 8);
    if (t0 + tt < L) o[(int64_t)tt * (2 * Npad) + r] = tile[k / 8][tt][n];
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
  // a block holds up to 64 channels of one (batch, B/C group)
  const int64_t cpg = p.chan_per_group;
  const int64_t cblocks = (cpg + 63) / 64;
  const int64_t bg = blockIdx.x / cblocks;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t d0 = g * cpg + (blockIdx.x % cblocks) * 64;
  const int64_t dend = (g + 1) * cpg;  // the group's last channel + 1
  const int64_t L = p.L;
  const int64_t dl_ = d0 + lane < dend ? d0 + lane : dend - 1;  // clamp idle lanes
  const int64_t hd = dl_ / p.chan_per_head;

  const TIn* __restrict__ u = static_cast<const TIn*>(p.u) + b * p.u_sb + dl_ * p.u_sd;
  const TIn* __restrict__ dlr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const float An = p.A[hd] * kLog2e;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  // B/C rows are read-only for the whole kernel: read them through the constant address
  // space so that the wave-uniform loads become scalar loads into SGPRs.
  const cfloat* Bs = to_constant(wsB + (b * p.groups + g) * L * Npad + wv * kNT);
  const cfloat* Cs = to_constant(wsC + (b * p.groups + g) * L * Npad + wv * kNT);

  // this wave's states wv * kNT + i of the lane's channel, from the caller's initial state or zero
  float h[kNT];
  {
    const float* hi = p.h_init ? p.h_init + b * p.hi_sb + dl_ * p.hi_sd : nullptr;
#pragma unroll
    for (int i = 0; i < kNT; ++i) h[i] = (hi && wv * kNT + i < p.N) ? hi[wv * kNT + i] : 0.f;
  }
  const float th = p.trap ? 0.5f : 0.f;

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
        float k = s;  // input coefficient: dt, or with zero-order hold (exp(dt A) - 1) / A
        if (p.zoh) {
          const float x = s * An * kLn2f;
          k = s * zoh_phi(x, av[j], __builtin_amdgcn_rcpf(x));
        }
        wv_[j] = k * uv[j];
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
        const float e = wv_[j] * bt[i];
        h[i] = fmaf(av[j], h[i], e);
        // trapezoidal rule: h carries k = h + e/2; y reads k - e/2
        acc = fmaf(ct[i], fmaf(-th, e, h[i]), acc);
      }
      yp[j] = acc;
    }
#pragma unroll
    for (int j = 0; j < kT; ++j) part[wv][lane][j] = yp[j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * kT; idx += blockDim.x) {
      const int c = idx / kT, j = idx % kT;
      const int64_t d = d0 + c, t = tb + j;
      if (d < dend && t < L) {
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
  // the state after the last step (steps past L are the identity)
  if (p.h_final && d0 + lane < dend) {
    float* hf = p.h_final + b * p.hf_sb + (d0 + lane) * p.hf_sd;
#pragma unroll
    for (int i = 0; i < kNT; ++i)
      if (wv * kNT + i < p.N) hf[wv * kNT + i] = h[i];
  }
}

// Fast path when every head covers whole waves (channels per head a multiple of 64): the
// head's step size and decay are computed once per step for the whole block, and the states
// are spread over NW (a power of two, at most 8) waves of kHS states each.  Per block of kHT
// steps:
//  (1) wave 0 computes dt and a = exp(dt A_h), one step per lane; the block copies the B/C
//      tile of these steps (f32, interleaved per 8 states, see interleave_bc_kernel) into LDS
//      and stores w = dt u transposed ([step][channel]);
//  (2) each wave advances its kHS states per step, reading B/C with wave-uniform (broadcast)
//      LDS reads, and keeps its partial readouts of the kHT steps in registers;
//  (3) the partial readouts are summed over the waves by a tree through LDS and the first
//      wave writes y = sum + D u (gated) for its 64 channels.
constexpr int kHS = 16;        // states per wave
constexpr int kHT = 32;        // steps per time block
constexpr int kHMaxWaves = 8;

int head_waves(int N) {
  int w = 1;
  while (w * kHS < N) w *= 2;
  return w;
}

template <typename TIn, typename TOut, bool GATE>
__global__ __launch_bounds__(64 * kHMaxWaves) void scalar_head_kernel(ScanArgs p,
                                                                      const float* __restrict__ wsBC,
                                                                      int Nh) {
  // bc[j][k]: step j of the tile; k = 16 * group + (0..7: B, 8..15: C) for 8-state groups
  __shared__ float bc[kHT][2 * kHS * kHMaxWaves];
  __shared__ float wbuf[kHT][65];
  __shared__ float red[kHMaxWaves / 2][kHT][64];
  __shared__ float abuf[kHT];
  __shared__ float dbuf[kHT];
  constexpr int E = 16 / (int)sizeof(TIn);  // elements per 16-byte chunk of a row
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nthreads = blockDim.x;
  const int nw = nthreads >> 6;
  const int64_t cblocks = p.channels / 64;
  const int64_t b = blockIdx.x / cblocks;
  const int64_t d0 = (blockIdx.x % cblocks) * 64;
  const int64_t L = p.L;
  const int64_t hd = d0 / p.chan_per_head;  // the block's 64 channels share one head
  const int64_t g = d0 / p.chan_per_group;
  const float An = p.A[hd] * kLog2e;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  const TIn* __restrict__ dlr = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const float* __restrict__ bcg = wsBC + (b * p.groups + g) * L * 2 * Nh;  // [t][2 * Nh]
  const bool vec = p.vec != 0;
  const int64_t d = d0 + lane;  // this lane's channel (wave 0 writes it)
  const TIn* __restrict__ ur = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;

  // this wave's states wv * kHS + i of the lane's channel, from the caller's initial state or zero
  float h[kHS];
  {
    const float* hi = p.h_init ? p.h_init + b * p.hi_sb + d * p.hi_sd : nullptr;
#pragma unroll
    for (int i = 0; i < kHS; ++i) h[i] = (hi && wv * kHS + i < p.N) ? hi[wv * kHS + i] : 0.f;
  }
  const float th = p.trap ? 0.5f : 0.f;

  for (int64_t tb = 0; tb < L; tb += kHT) {
    if (wv == 0 && lane < kHT) {
      const int64_t t = tb + lane;
      float dtv = 0.f, av = 1.f;  // steps past the end are the identity
      if (t < L) {
        const float x = to_f32(dlr[t]) + bias;
        dtv = p.softplus ? softplus_fast(x) : x;
        av = __builtin_amdgcn_exp2f(dtv * An);
        if (p.zoh) {
          // input coefficient (exp(dt A) - 1) / A instead of dt
          const float xz = dtv * An * kLn2f;
          dtv *= zoh_phi(xz, av, __builtin_amdgcn_rcpf(xz));
        }
      }
      dbuf[lane] = dtv;  // the input coefficient of the step
      abuf[lane] = av;
    }
    // the B/C tile: kHT rows of 2 * Nh floats, contiguous in the workspace
    {
      const int rowq = 2 * Nh / 4;  // 16-byte quads per step
      const f32x4* src = reinterpret_cast<const f32x4*>(bcg + tb * 2 * Nh);
      for (int q = threadIdx.x; q < kHT * rowq; q += nthreads) {
        const int j = q / rowq, k = q % rowq;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (tb + j < L) v = src[q];
        *reinterpret_cast<f32x4*>(&bc[j][4 * k]) = v;
      }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * (kHT / E); q += nthreads) {
      const int c = q / (kHT / E), k = q % (kHT / E);
      const int64_t t0 = tb + k * E;
      const TIn* __restrict__ uc = static_cast<const TIn*>(p.u) + b * p.u_sb + (d0 + c) * p.u_sd;
      float uv[E];
      if (vec && t0 + E <= L) {
        load_seg<E>(uc, t0, L, true, uv);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) uv[e] = (t0 + e < L) ? to_f32(uc[t0 + e]) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) wbuf[k * E + e][c] = dbuf[k * E + e] * uv[e];
    }
    __syncthreads();

    // the recurrence: this wave's kHS states, partial readouts of the tile kept in registers
    float acc[kHT];
#pragma unroll
    for (int j = 0; j < kHT; ++j) {
      const float a = abuf[j];
      const float w = wbuf[j][lane];
      const f32x4* q = reinterpret_cast<const f32x4*>(&bc[j][2 * kHS * wv]);
      float Bj[kHS], Cj[kHS];
#pragma unroll
      for (int grp = 0; grp < kHS / 8; ++grp) {
        const f32x4 b0 = q[4 * grp], b1 = q[4 * grp + 1], c0 = q[4 * grp + 2], c1 = q[4 * grp + 3];
        Bj[8 * grp + 0] = b0.x; Bj[8 * grp + 1] = b0.y; Bj[8 * grp + 2] = b0.z; Bj[8 * grp + 3] = b0.w;
        Bj[8 * grp + 4] = b1.x; Bj[8 * grp + 5] = b1.y; Bj[8 * grp + 6] = b1.z; Bj[8 * grp + 7] = b1.w;
        Cj[8 * grp + 0] = c0.x; Cj[8 * grp + 1] = c0.y; Cj[8 * grp + 2] = c0.z; Cj[8 * grp + 3] = c0.w;
        Cj[8 * grp + 4] = c1.x; Cj[8 * grp + 5] = c1.y; Cj[8 * grp + 6] = c1.z; Cj[8 * grp + 7] = c1.w;
      }
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kHS; ++i) {
        const float e = w * Bj[i];
        h[i] = fmaf(a, h[i], e);
        // trapezoidal rule: h carries k = h + e/2; y reads k - e/2
        sum = fmaf(Cj[i], fmaf(-th, e, h[i]), sum);
      }
      acc[j] = sum;
    }

    // tree reduction over the waves
    for (int half = nw / 2; half >= 1; half /= 2) {
      if (wv >= half && wv < 2 * half) {
#pragma unroll
        for (int j = 0; j < kHT; ++j) red[wv - half][j][lane] = acc[j];
      }
      __syncthreads();
      if (wv < half) {
#pragma unroll
        for (int j = 0; j < kHT; ++j) acc[j] += red[wv][j][lane];
      }
      __syncthreads();
    }

    if (wv == 0) {
      const int64_t t0 = tb;
      float uv[kHT], out[kHT];
      load_seg<kHT>(ur, t0, L, vec, uv);
      float zv[kHT];
      if constexpr (GATE) {
        const TIn* __restrict__ zr = static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd;
        load_seg<kHT>(zr, t0, L, vec, zv);
      }
#pragma unroll
      for (int j = 0; j < kHT; ++j) {
        float s = p.D ? fmaf(Dd, uv[j], acc[j]) : acc[j];
        if constexpr (GATE) s *= silu_fast(zv[j]);
        out[j] = s;
      }
      TOut* __restrict__ yr = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
      store_seg<kHT>(yr, t0, L, vec, out);
    }
  }
  // the state after the last step (steps past L are the identity)
  if (p.h_final) {
    float* hf = p.h_final + b * p.hf_sb + d * p.hf_sd;
#pragma unroll
    for (int i = 0; i < kHS; ++i)
      if (wv * kHS + i < p.N) hf[wv * kHS + i] = h[i];
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
  if (head_path(a)) {
    const int nw = head_waves(a.N);
    const int Nh = nw * kHS;
    const int64_t tblocks = a.batch * a.groups * ((a.L + 63) / 64);
    hipLaunchKernelGGL((interleave_bc_kernel<TIn>), dim3((unsigned)tblocks), dim3(256), 0, s,
                       static_cast<const TIn*>(a.B), static_cast<const TIn*>(a.C), a.B_sb, a.B_sg,
                       a.B_sn, a.C_sb, a.C_sg, a.C_sn, a.groups, a.N, Nh, a.L, ws);
    hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
    const int64_t blocks = a.batch * (a.channels / 64);
    const dim3 block(64 * nw);
    if (a.z)
      hipLaunchKernelGGL((scalar_head_kernel<TIn, TOut, true>), dim3((unsigned)blocks), block, 0, s, a, ws, Nh);
    else
      hipLaunchKernelGGL((scalar_head_kernel<TIn, TOut, false>), dim3((unsigned)blocks), block, 0, s, a, ws, Nh);
    return hipGetLastError();
  }
  hipError_t e = transpose<TIn>(a, a.B, a.B_sb, a.B_sg, a.B_sn, ws, s);
  if (e != hipSuccess) return e;
  e = transpose<TIn>(a, a.C, a.C_sb, a.C_sg, a.C_sn, ws + plane, s);
  if (e != hipSuccess) return e;
  const int64_t blocks = a.batch * a.groups * ((a.chan_per_group + 63) / 64);
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
  const int64_t n = head_path(a) ? (int64_t)head_waves(a.N) * kHS : (int64_t)npad_of(a.N);
  return 2 * a.batch * a.groups * a.L * n;
}

hipError_t launch_scalar(const ScanArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
