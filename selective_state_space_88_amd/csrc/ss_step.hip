// ss_step.hip -- one decoding step of the selective scan with a persistent state (gfx950).
//
// In recurrent (decode) mode the model reads one token at a time and updates a state of fixed
// size (the "Mamba -- selective state space model" study notes, core points and cases 1 and 3;
// the bqwf.cn state-space survey, section 1, on the recurrent mode's constant memory):
//   dt = softplus(delta + bias),  h = exp(dt A) h + dt B u,  y = C h + D u  (times silu(z)).
// It is the scan at L = 1 starting from the caller's state, and is computed here the same way
// as in the scan kernels (exp2 with log2 e folded into A, the same softplus and silu).
//
// Mapping: every (batch, channel) row gets G lanes (a power of two, at most 32, so that a row
// never leaves its wave), each lane four consecutive states; the row's readout is summed over
// its lanes with xor shuffles.  The state is read and written in place, coalesced along n
// (16-byte accesses per lane when the rows allow).  Blocks are one wave.
#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kStepThreads = 64;   // one wave per block: small decode problems still spread over the CUs
constexpr int kStatesPerLane = 4;

template <typename T>
struct Quad;
template <>
struct Quad<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ float get(const type& v, int i) { return v[i]; }
};
template <>
struct Quad<bf16_t> {
  typedef uint32_t type __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ float get(const type& v, int i) {
    return (i & 1) ? bf16_hi(v[i >> 1]) : bf16_lo(v[i >> 1]);
  }
};

// VEC: N a multiple of 4 and the state and B/C rows aligned for 16-byte (state, f32 B/C) or
// 8-byte (bf16 B/C) accesses: each lane moves its four states with single loads and stores.
template <typename TIn, typename TOut, bool GATE, bool VEC>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs p, int G) {
  const int tid = threadIdx.x;
  const int64_t rows = p.batch * p.channels;
  const int64_t row = (int64_t)blockIdx.x * (kStepThreads / G) + tid / G;
  const int j = tid % G;
  const bool live = row < rows;
  const int64_t rr = live ? row : 0;
  const int64_t b = rr / p.channels, d = rr % p.channels;
  const int64_t hd = d / p.chan_per_head, g = d / p.chan_per_group;

  const float x = to_f32(static_cast<const TIn*>(p.delta)[b * p.dl_sb + hd]) + (p.bias ? p.bias[hd] : 0.f);
  const float dt = p.softplus ? softplus_fast(x) : x;
  const float uu = to_f32(static_cast<const TIn*>(p.u)[b * p.u_sb + d]);
  const float w = dt * uu;
  const TIn* Br = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cr = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  float* hr = p.h + b * p.h_sb + d * p.h_sd;
  const float* Ar = p.scalar ? p.A + hd : p.A + d * p.A_sd;
  const int n0 = kStatesPerLane * j;

  float acc = 0.f;
  if constexpr (VEC) {
    if (live && n0 < p.N) {
      typedef typename Quad<TIn>::type QT;
      const f32x4 hv = *reinterpret_cast<const f32x4*>(hr + n0);
      const QT bv = *reinterpret_cast<const QT*>(Br + n0);
      const QT cv = *reinterpret_cast<const QT*>(Cr + n0);
      f32x4 av;
      if (p.scalar) {
        av = f32x4{Ar[0], Ar[0], Ar[0], Ar[0]};
      } else {
        av = *reinterpret_cast<const f32x4*>(Ar + n0);
      }
      f32x4 hn;
#pragma unroll
      for (int i = 0; i < kStatesPerLane; ++i) {
        const float a = __builtin_amdgcn_exp2f(dt * (av[i] * kLog2e));
        float wi = w;
        if (p.zoh) {
          const float x = dt * av[i];
          wi = w * zoh_phi(x, a, __builtin_amdgcn_rcpf(x));
        }
        const float e = wi * Quad<TIn>::get(bv, i);
        hn[i] = fmaf(a, hv[i], e);
        // trapezoidal rule: the state is k = h + e/2, y reads k - e/2
        acc = fmaf(Quad<TIn>::get(cv, i), p.trap ? fmaf(-0.5f, e, hn[i]) : hn[i], acc);
      }
      *reinterpret_cast<f32x4*>(hr + n0) = hn;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kStatesPerLane; ++i) {
      const int n = n0 + i;
      if (live && n < p.N) {
        const float An = p.scalar ? Ar[0] : Ar[n];
        const float a = __builtin_amdgcn_exp2f(dt * (An * kLog2e));
        float wi = w;
        if (p.zoh) {
          const float x = dt * An;
          wi = w * zoh_phi(x, a, __builtin_amdgcn_rcpf(x));
        }
        const float e = wi * to_f32(Br[n]);
        const float hn = fmaf(a, hr[n], e);
        hr[n] = hn;
        acc = fmaf(to_f32(Cr[n]), p.trap ? fmaf(-0.5f, e, hn) : hn, acc);
      }
    }
  }
  // the row's readout: its G lanes are an aligned group of the wave
  for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (live && j == 0) {
    float yy = acc;
    if (p.D) yy = fmaf(p.D[p.d_per_head ? hd : d], uu, yy);
    if constexpr (GATE) yy *= silu_fast(to_f32(static_cast<const TIn*>(p.z)[b * p.z_sb + d]));
    store_one(static_cast<TOut*>(p.y) + b * p.y_sb + d, yy);
  }
}

template <typename TIn, typename TOut>
hipError_t launch_t(const StepArgs& a, hipStream_t s) {
  int G = 1;
  while (G * kStatesPerLane < a.N) G *= 2;   // N <= 128: G <= 32
  const int64_t rows = a.batch * a.channels;
  const int64_t rpb = kStepThreads / G;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(kStepThreads);
  // 16-byte state rows and f32 A rows, 16- (f32) or 8-byte (bf16) B/C rows
  const int64_t qb = 4 * (int64_t)sizeof(TIn);
  auto al = [](const void* ptr, int64_t bytes) { return reinterpret_cast<uintptr_t>(ptr) % bytes == 0; };
  const bool vec = a.N % 4 == 0 && al(a.h, 16) && a.h_sb % 4 == 0 && a.h_sd % 4 == 0 && al(a.B, qb) &&
                   al(a.C, qb) && a.B_sb % 4 == 0 && a.B_sg % 4 == 0 && a.C_sb % 4 == 0 && a.C_sg % 4 == 0 &&
                   (a.scalar || (al(a.A, 16) && a.A_sd % 4 == 0));
#define SS_STEP(GT, V) hipLaunchKernelGGL((step_kernel<TIn, TOut, GT, V>), grid, block, 0, s, a, G)
  if (a.z) {
    if (vec) SS_STEP(true, true); else SS_STEP(true, false);
  } else {
    if (vec) SS_STEP(false, true); else SS_STEP(false, false);
  }
#undef SS_STEP
  return hipGetLastError();
}

__global__ __launch_bounds__(kStepThreads) void state_copy_kernel(const float* __restrict__ src, int64_t s_sb,
                                                                  int64_t s_sd, float* __restrict__ dst, int64_t d_sb,
                                                                  int64_t d_sd, int64_t channels, int64_t N,
                                                                  int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kStepThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i % N, bd = i / N, d = bd % channels, b = bd / channels;
  dst[b * d_sb + d * d_sd + n] = src ? src[b * s_sb + d * s_sd + n] : 0.f;
}

}  // namespace

hipError_t launch_state_copy(const float* src, int64_t s_sb, int64_t s_sd, float* dst, int64_t d_sb, int64_t d_sd,
                             int64_t batch, int64_t channels, int64_t N, hipStream_t s) {
  const int64_t total = batch * channels * N;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)((total + kStepThreads - 1) / kStepThreads)),
                     dim3(kStepThreads), 0, s, src, s_sb, s_sd, dst, d_sb, d_sd, channels, N, total);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, s) : launch_t<float, float>(a, s);
}

}  // namespace ss
