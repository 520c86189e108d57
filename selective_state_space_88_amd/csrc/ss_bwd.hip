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
// and per step dz_t = dy_t y0_t s'(z_t), du_t += dy0_t D, dD += dy0_t u_t,
// ddelta_t = ddt_t sigmoid(x_t) (softplus'), dbias += ddelta_t.
//
// With heads (a step size, and optionally a scalar decay A_h, shared by a head's channels) the
// per-head gradients ddelta, dbias, dA (and dD when D is per head) are summed over the head's
// channels; with a scalar decay exp(dt A_h) is computed once per step for all N states.
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
constexpr int kBWaves = 4;           // channels (rows) per block of the checkpoint kernel
constexpr int kMWaves = 8;           // channels per block of the backward kernel (of one B/C group)
constexpr int kBMaxPairs = 64;       // N <= 128

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

template <typename TIn, typename TDy, bool GATE, bool SCALAR>
__global__ __launch_bounds__(64 * kMWaves) void bwd_kernel(BwdArgs p, int P, int64_t nwin, const float* ckpt) {
  __shared__ float gcar[kMWaves][kBMaxPairs][2];      // adjoint carried into the window from the right
  __shared__ float dAl[kMWaves][2 * kBMaxPairs];      // dA partial sums of the wave's channel
  // dB (2 states), dC (2 states) of the window's steps, step-major ([lane][k] = step lane K + k)
  __shared__ __attribute__((aligned(16))) float red[kMWaves][4][kBW];
  // B (2 states) and C (2 states) of a pair's window, shared by the block's channels; two
  // buffers: the next pair's rows are loaded while this pair runs
  __shared__ __attribute__((aligned(16))) float bcs[2][4][kBW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // blocks of 8 channels of one group; when the group's channels are 4 mod 8, the last block's
  // last 4 waves work on a copy of a valid channel and contribute nothing
  const int64_t cblocks = (p.chan_per_group + kMWaves - 1) / kMWaves;
  const int64_t bg = blockIdx.x / cblocks, qd = blockIdx.x % cblocks;
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
  const TIn* zr = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  const TDy* dyr = static_cast<const TDy*>(p.dy) + b * p.dy_sb + d * p.dy_sd;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  float* dBg = p.dB + b * p.dB_sb + g * p.dB_sg;
  float* dCg = p.dC + b * p.dC_sb + g * p.dC_sg;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  const float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;
  for (int i = lane; i < 2 * kBMaxPairs; i += 64) {
    gcar[wave][i / 2][i % 2] = 0.f;
    dAl[wave][i] = 0.f;
  }
  float dDacc = 0.f, dbacc = 0.f;
  // thread t stages row t / 64 (B of state 2 pp, of 2 pp + 1, C of 2 pp, of 2 pp + 1), the steps
  // of lane t % 64; rows past N and steps past L are zero
  const int srow = threadIdx.x >> 6, sseg = threadIdx.x & 63;
  auto bc_load = [&](int64_t ww, int pq, float (&v)[kBK]) {
    const int n = 2 * pq + (srow & 1);
    const bool nv = n < N && srow < 4;
    const TIn* src = srow < 2 ? Bg + (nv ? n : 0) * p.B_sn : Cg + (nv ? n : 0) * p.C_sn;
    load_seg<kBK>(src, ww * kBW + (int64_t)kBK * sseg, nv ? L : 0, p.vec, v);
  };
  auto bc_store = [&](int bf, const float (&v)[kBK]) {
    if (srow >= 4) return;   // four rows, one per wave of the first four
    float* dst = &bcs[bf][srow][kBK * sseg];
    *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
  };
  {
    float v[kBK];
    bc_load(nwin - 1, 0, v);
    bc_store(0, v);
  }
  __syncthreads();
  int buf = 0;

  for (int64_t w = nwin - 1; w >= 0; --w) {
    const int64_t t0 = w * kBW + (int64_t)lane * kBK;
    float dt[kBK], uu[kBK], wv[kBK], dy0[kBK], y0[kBK], du[kBK], ddt[kBK], sg[kBK], dyv[kBK], zv[kBK], dv[kBK];
    float sdt = 0.f;   // the lane's steps' total step size
    load_seg<kBK>(dr, t0, L, p.vec, dv);
    load_seg<kBK>(ur, t0, L, p.vec, uu);
    load_seg<kBK>(dyr, t0, L, p.vec, dyv);
    if constexpr (GATE) load_seg<kBK>(zr, t0, L, p.vec, zv);
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const bool ok = t0 + k < L;
      const float x = dv[k] + bias;
      dt[k] = ok ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      // softplus'(x) = sigmoid(x)
      sg[k] = p.softplus ? 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)) : 1.f;
      wv[k] = dt[k] * uu[k];
      float gz = 1.f;
      if constexpr (GATE) gz = silu_fast(zv[k]);
      dy0[k] = dyv[k] * gz;
      y0[k] = Dd * uu[k];
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
      // the next pair's B and C rows (the first pair of the window to the left after the last)
      const bool more = pp + 1 < P || w > 0;
      float nbc[kBK];
      if (more) bc_load(pp + 1 < P ? w : w - 1, pp + 1 < P ? pp + 1 : 0, nbc);
      float rB[2][kBK], rC[2][kBK];
      float dAp[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int n = 2 * pp + s;
        const bool nv = n < N;
        const float An = SCALAR ? p.A[hd] : (nv ? p.A[d * p.A_sd + n] : 0.f);
        const float A2 = An * kLog2e;
        float av[kBK], bv[kBK], cv[kBK];
        {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(&bcs[buf][s][kBK * lane]);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(&bcs[buf][s][kBK * lane + 4]);
          const f32x4 c0 = *reinterpret_cast<const f32x4*>(&bcs[buf][2 + s][kBK * lane]);
          const f32x4 c1 = *reinterpret_cast<const f32x4*>(&bcs[buf][2 + s][kBK * lane + 4]);
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
          y0[k] = fmaf(cv[k], hs[k + 1], y0[k]);
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
        const float Xw = gcar[wave][pp][s];
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
        if (lane == 0) gcar[wave][pp][s] = cl;
        dAp[s] = dAs;
      }
      // dA of the pair: summed over the wave's lanes into the wave's partial sums
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const float v = wave_sum(dAp[s]);
        if (lane == 0 && valid && 2 * pp + s < N) dAl[wave][SCALAR ? 0 : 2 * pp + s] += v;
      }
      // dB, dC of the pair: summed over the block's 8 channels, then one atomic add per step;
      // consecutive lanes add to consecutive steps, so each wave's adds cover two cache lines
      if (!valid) {
#pragma unroll
        for (int k = 0; k < kBK; ++k) rB[0][k] = rB[1][k] = rC[0][k] = rC[1][k] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < kBK; k += 4) {
        *reinterpret_cast<f32x4*>(&red[wave][0][lane * kBK + k]) = f32x4{rB[0][k], rB[0][k + 1], rB[0][k + 2], rB[0][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][1][lane * kBK + k]) = f32x4{rB[1][k], rB[1][k + 1], rB[1][k + 2], rB[1][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][2][lane * kBK + k]) = f32x4{rC[0][k], rC[0][k + 1], rC[0][k + 2], rC[0][k + 3]};
        *reinterpret_cast<f32x4*>(&red[wave][3][lane * kBK + k]) = f32x4{rC[1][k], rC[1][k + 1], rC[1][k + 2], rC[1][k + 3]};
      }
      if (more) bc_store(buf ^ 1, nbc);
      __syncthreads();
      for (int i = threadIdx.x; i < 4 * kBW; i += 64 * kMWaves) {
        const int which = i / kBW, r = i % kBW;
        const int n = 2 * pp + (which & 1);
        const int64_t t = w * kBW + r;
        if (n < N && t < L) {
          float v = 0.f;
#pragma unroll
          for (int wv2 = 0; wv2 < kMWaves; ++wv2) v += red[wv2][which][r];
          float* dst = (which < 2 ? dBg + n * p.dB_sn : dCg + n * p.dC_sn) + t;
          atomicAdd(dst, v);
        }
      }
      __syncthreads();
      buf ^= 1;
    }
    // per-step outputs of the window
    float* dur = p.du + b * p.du_sb + d * p.du_sd;
    float* ddr = p.ddelta + b * p.dd_sb + hd * p.dd_sh;
    float dxs[kBK];
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      // with gB = sum_n g B: du = dt gB + D dy0 and ddt += u gB
      const float gB = du[k];
      du[k] = fmaf(dt[k], gB, dy0[k] * Dd);
      ddt[k] = fmaf(uu[k], gB, ddt[k]);
      dxs[k] = (valid && t0 + k < L) ? ddt[k] * sg[k] : 0.f;
    }
    if (p.chan_per_head % kMWaves == 0 && p.chan_per_group % kMWaves == 0) {
      // the block's 8 channels share the head: summed through LDS, one atomic add per step
#pragma unroll
      for (int k = 0; k < kBK; k += 4)
        *reinterpret_cast<f32x4*>(&red[wave][0][lane * kBK + k]) = f32x4{dxs[k], dxs[k + 1], dxs[k + 2], dxs[k + 3]};
      __syncthreads();
      for (int i = threadIdx.x; i < kBW; i += 64 * kMWaves) {
        const int64_t t = w * kBW + i;
        float v = 0.f;
#pragma unroll
        for (int wv2 = 0; wv2 < kMWaves; ++wv2) v += red[wv2][0][i];
        if (t < L) atomicAdd(ddr + t, v);
      }
      __syncthreads();
    } else if (valid && p.chan_per_head == 1) {
#pragma unroll
      for (int k = 0; k < kBK; ++k)
        if (t0 + k < L) ddr[t0 + k] = dxs[k];
    } else if (valid) {
#pragma unroll
      for (int k = 0; k < kBK; ++k)
        if (t0 + k < L) atomicAdd(ddr + t0 + k, dxs[k]);
    }
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      if (valid && t0 + k < L) {
        const float dx = dxs[k];
        dur[t0 + k] = du[k];
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
  if (!valid) return;
  if (lane == 0) {
    if (p.dD) atomicAdd(p.dD + (p.d_per_head ? hd : d), dDs);
    if (p.dbias) atomicAdd(p.dbias + hd, dbs);
    if (SCALAR) atomicAdd(p.dA + hd, dAl[wave][0]);
  }
  if (!SCALAR)
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
  zero4(a.dD, 1, 1, 1, a.d_per_head ? a.heads : a.channels, 0, 0, 0);
  zero4(a.dbias, 1, 1, 1, a.heads, 0, 0, 0);
  if (a.scalar) zero4(a.dA, 1, 1, 1, a.heads, 0, 0, 0);
  else zero4(a.dA, 1, 1, a.channels, a.N, 0, 0, a.dA_sd);
  // a head's channels add into its step-size gradient
  if (a.chan_per_head > 1) zero4(a.ddelta, a.batch, 1, a.heads, a.L, a.dd_sb, 0, a.dd_sh);
  zero4(a.dB, a.batch, a.groups, a.N, a.L, a.dB_sb, a.dB_sg, a.dB_sn);
  zero4(a.dC, a.batch, a.groups, a.N, a.L, a.dC_sb, a.dC_sg, a.dC_sn);
  if (ssd_bwd_path(a)) return launch_ssd_bwd(a, ws, s);
  const dim3 cgrid((unsigned)((rows + kBWaves - 1) / kBWaves)), block(64 * kBWaves);
  if (a.scalar) hipLaunchKernelGGL((bwd_ckpt_kernel<TIn, true>), cgrid, block, 0, s, a, P, nwin, ws);
  else hipLaunchKernelGGL((bwd_ckpt_kernel<TIn, false>), cgrid, block, 0, s, a, P, nwin, ws);
  const dim3 grid((unsigned)(a.batch * a.groups * ((a.chan_per_group + kMWaves - 1) / kMWaves)));
  const dim3 mblock(64 * kMWaves);
  const float* ck = ws;
#define SS_BWD(GT, SC) hipLaunchKernelGGL((bwd_kernel<TIn, TDy, GT, SC>), grid, mblock, 0, s, a, P, nwin, ck)
  if (a.z) {
    if (a.scalar) SS_BWD(true, true); else SS_BWD(true, false);
  } else {
    if (a.scalar) SS_BWD(false, true); else SS_BWD(false, false);
  }
#undef SS_BWD
  return hipGetLastError();
}

}  // namespace

int64_t bwd_workspace_floats(const BwdArgs& a) {
  if (ssd_bwd_path(a)) return ssd_bwd_workspace_floats(a);
  return a.batch * a.channels * ((a.L + kBW - 1) / kBW) * a.N;
}

hipError_t launch_bwd(const BwdArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.dy_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.dy_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
