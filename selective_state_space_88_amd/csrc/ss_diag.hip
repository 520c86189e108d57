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
//  - a block is 4 waves over 4 channels of one (batch, B/C group); each wave owns one channel
//    and its 64 lanes lie along time, lane j owning K consecutive steps, so one window of the
//    row covers 64*K steps.  Windows are walked in order; the state at the end of each window
//    is carried to the next in registers, so each exp is evaluated exactly once;
//  - the N states are processed two at a time (n outer).  For a state each lane runs its K steps
//    from zero (keeping the K decays a_t and inputs b_t in registers), the wave combines the 64
//    lane aggregates with a DPP scan (row_shr within rows of 16, row_bcast across rows, wave_shr
//    for the exclusive prefix), and each lane re-runs its K steps from the true incoming state
//    to form h_t and accumulate y_t += C_{t,n} h_t.  The two states of a pair are independent
//    chains, which the wave interleaves (and whose two scans fill each other's DPP wait states);
//  - the B and C rows of state n are shared by every channel of the block: they are read once
//    per block with coalesced 16-byte loads, widened to f32 and staged in LDS (double-buffered
//    over n, laid out [quad][lane] so each wave-wide 16-byte LDS read is one contiguous 1 KB);
//  - softplus, D*u and the silu gate are fused; u, delta, z and y stream through HBM once.
#include <type_traits>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kWaves = 4;

// Two independent exclusive scans over the 64 lanes (lane 0 earliest) of (a, b) pairs under
// (a1, b1) then (a2, b2) = (a1 a2, a2 b1 + b2).  Each step is one fused DPP multiply and one
// fused DPP FMA per scan: v_fmac_f32_dpp b, b[src], a  (b += b[src] * a) and
// v_mul_f32_dpp a, a[src], a.  A lane whose DPP source is outside its row (row_shr) or whose
// row is masked off (row_bcast with row_mask) is not written, i.e. it keeps its pair, which is
// the same as combining with the identity (1, 0).  Steps: row_shr:1,2,4,8 scan each row of 16
// lanes; row_bcast:15 (rows 1, 3) and row_bcast:31 (rows 2, 3) add the earlier rows; wave_shr:1
// turns the inclusive scan into the exclusive one (lane 0 gets the identity).  The two scans
// are interleaved so that every DPP read of a VGPR comes at least four instructions after the
// VALU write of it (the hardware needs two wait states there); the leading s_nop covers the
// compiler's last writes.
__device__ __forceinline__ void wave_exclusive_scan2(float& a0, float& b0, float& a1, float& b1) {
  float ea0, eb0, ea1, eb1;
#define SS_STEP(CTRL)                                   \
  "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n"                \
  "v_fmac_f32_dpp %3, %3, %2 " CTRL "\n"                \
  "v_mul_f32_dpp %0, %0, %0 " CTRL "\n"                 \
  "v_mul_f32_dpp %2, %2, %2 " CTRL "\n"
  asm volatile(
      "s_nop 1\n"
      SS_STEP("row_shr:1 row_mask:0xf bank_mask:0xf")
      SS_STEP("row_shr:2 row_mask:0xf bank_mask:0xf")
      SS_STEP("row_shr:4 row_mask:0xf bank_mask:0xf")
      SS_STEP("row_shr:8 row_mask:0xf bank_mask:0xf")
      SS_STEP("row_bcast:15 row_mask:0xa bank_mask:0xf")
      SS_STEP("row_bcast:31 row_mask:0xc bank_mask:0xf")
      "v_mov_b32 %4, 1.0\n"
      "v_mov_b32 %6, 1.0\n"
      "v_mov_b32 %5, 0\n"
      "v_mov_b32 %7, 0\n"
      "v_mov_b32_dpp %4, %0 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %6, %2 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %5, %1 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %7, %3 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "=&v"(ea0), "=&v"(eb0), "=&v"(ea1), "=&v"(eb1));
#undef SS_STEP
  a0 = ea0;
  b0 = eb0;
  a1 = ea1;
  b1 = eb1;
}

// Elements of TIn per 16-byte chunk.
template <typename TIn>
constexpr int chunk_elems() { return 16 / (int)sizeof(TIn); }

// A 16-byte chunk of a B/C row, held in registers between its global load and its LDS store.
template <typename TIn>
struct Chunk {
  u32x4 raw;
};

template <bool FULL, typename TIn>
__device__ __forceinline__ void load_chunk(const TIn* __restrict__ p, int64_t t, int64_t L, Chunk<TIn>& c) {
  constexpr int E = chunk_elems<TIn>();
  if constexpr (FULL) {
    // a plain (cached) load: B and C rows are shared by every channel and should stay in L2
    c.raw = *reinterpret_cast<const u32x4*>(p + t);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t bits = 0u;
      if (t + e < L) {
        if constexpr (sizeof(TIn) == 2) bits = reinterpret_cast<const uint16_t*>(p)[t + e];
        else bits = __float_as_uint(reinterpret_cast<const float*>(p)[t + e]);
      }
      if constexpr (sizeof(TIn) == 2) w[e / 2] |= bits << (16 * (e % 2));
      else w[e] = bits;
    }
    c.raw = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Widen a chunk to f32 and write it into an LDS row laid out as [quad][lane][4]: the chunk
// starts at quad i of lane j (a bf16 chunk spans quads i and i + 1).
template <typename TIn>
__device__ __forceinline__ void store_chunk(float* row, int i, int j, const Chunk<TIn>& c) {
  f32x4* q = reinterpret_cast<f32x4*>(row);
  if constexpr (sizeof(TIn) == 2) {
    q[i * 64 + j] = f32x4{bf16_lo(c.raw.x), bf16_hi(c.raw.x), bf16_lo(c.raw.y), bf16_hi(c.raw.y)};
    q[(i + 1) * 64 + j] = f32x4{bf16_lo(c.raw.z), bf16_hi(c.raw.z), bf16_lo(c.raw.w), bf16_hi(c.raw.w)};
  } else {
    q[i * 64 + j] =
        f32x4{__uint_as_float(c.raw.x), __uint_as_float(c.raw.y), __uint_as_float(c.raw.z), __uint_as_float(c.raw.w)};
  }
}

// K consecutive elements of one time row as raw 32-bit words (bf16 pairs or f32), so that a
// segment can be loaded one work item ahead and widened when it is used.
template <typename TIn, int K>
struct Seg {
  static constexpr int kWords = K * (int)sizeof(TIn) / 4;
  uint32_t w[kWords];
};

template <typename TIn, int K>
__device__ __forceinline__ void seg_load(const TIn* __restrict__ p, int64_t t0, int64_t L, bool full,
                                         Seg<TIn, K>& s) {
  constexpr int NW = Seg<TIn, K>::kWords;
  if (full) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p + t0);
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(q + i);
      s.w[4 * i] = v.x;
      s.w[4 * i + 1] = v.y;
      s.w[4 * i + 2] = v.z;
      s.w[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) s.w[i] = 0u;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (t0 + j < L) {
        if constexpr (sizeof(TIn) == 2)
          s.w[j / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(p)[t0 + j] << (16 * (j % 2));
        else
          s.w[j] = __float_as_uint(reinterpret_cast<const float*>(p)[t0 + j]);
      }
    }
  }
}

template <typename TIn, int K>
__device__ __forceinline__ float seg_get(const Seg<TIn, K>& s, int j) {
  if constexpr (sizeof(TIn) == 2) return (j & 1) ? bf16_hi(s.w[j / 2]) : bf16_lo(s.w[j / 2]);
  else return __uint_as_float(s.w[j]);
}

// Per-wave parameters of one channel.
struct Chan {
  int64_t b, g, d, hd;
  bool live;
};

template <typename TIn, typename TOut, bool GATE, int K>
#ifndef SS_DIAG_WAVES_PER_EU
#define SS_DIAG_WAVES_PER_EU 2
#endif
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(SS_DIAG_WAVES_PER_EU))) void diag_fwd_kernel(
    ScanArgs p, int64_t blocks_per_bg) {
  constexpr int W = 64 * K;                      // steps per window
  constexpr int Q = K / 4;                       // 16-byte quads per lane per row
  constexpr int E = chunk_elems<TIn>();          // elements per 16-byte chunk
  constexpr int CH = W / E;                      // chunks per row (of one tensor) per window
  constexpr int NCH = 4 * CH;                    // chunks per pair of states (B, C for each)
  constexpr int CPT = (NCH + 64 * kWaves - 1) / (64 * kWaves);  // chunks per thread
  static_assert(K % 8 == 0 && W % E == 0, "bad window");
  // stage[buf][r]: r = 0, 1 -> B, C of the pair's first state; 2, 3 -> B, C of the second.
  // Within a row, quad i (steps 4i..4i+3) of lane j sits at float offset (i * 64 + j) * 4, so
  // that one ds_read_b128 of the whole wave covers 1 KB of consecutive LDS (no bank conflicts).
  __shared__ float stage[2][4][Q * 64 * 4];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t L = p.L;
  const int N = p.N;
  const bool vec = p.vec != 0;
  const int64_t nwin = (L + W - 1) / W;
  const int64_t quads = p.batch * p.groups * blocks_per_bg;

  // Work item k of this block: quad blockIdx.x + (k / nwin) * gridDim.x, window k % nwin.  The
  // four waves of a block walk the same items (same batch, group and window; four channels).
  auto chan_of = [&](int64_t quad) {
    Chan c;
    const int64_t bg = quad / blocks_per_bg, blk = quad % blocks_per_bg;
    c.b = bg / p.groups;
    c.g = bg % p.groups;
    const int64_t local = blk * kWaves + wave;
    c.live = local < p.chan_per_group;
    c.d = c.g * p.chan_per_group + (c.live ? local : p.chan_per_group - 1);
    c.hd = c.d / p.chan_per_head;
    return c;
  };
  auto urow = [&](const Chan& c) { return static_cast<const TIn*>(p.u) + c.b * p.u_sb + c.d * p.u_sd; };
  auto drow = [&](const Chan& c) { return static_cast<const TIn*>(p.delta) + c.b * p.dl_sb + c.hd * p.dl_sh; };
  auto zrow = [&](const Chan& c) { return static_cast<const TIn*>(p.z) + c.b * p.z_sb + c.d * p.z_sd; };

  const int64_t my_items = blockIdx.x < quads ? ((quads - 1 - blockIdx.x) / gridDim.x + 1) * nwin : 0;
  if (my_items == 0) return;  // uniform over the block

  int64_t quad = blockIdx.x;
  Chan cc = chan_of(quad);
  Seg<TIn, K> su, sd, sz;
  float aq0 = 0.f, aq1 = 0.f;  // A row (times log2 e) across lanes: lane n holds state n (and 64 + n)
  auto lane_get = [&](float q0, float q1, int n) {
    return n < 64 ? readlane_f(q0, n) : readlane_f(q1, n - 64);
  };
  float cq0 = 0.f, cq1 = 0.f;  // carried state, lane n holds state n (and 64 + n)

  for (int64_t k = 0; k < my_items; ++k) {
    const int64_t win = k % nwin;
    const int64_t w0 = win * W;
    const bool full = vec && w0 + W <= L;
    const int64_t t0 = w0 + (int64_t)lane * K;
    if (win == 0) {
      if (k > 0) {
        quad += gridDim.x;
        cc = chan_of(quad);
      }
      const float* Arow = p.A + cc.d * p.A_sd;
      aq0 = lane < N ? Arow[lane] * kLog2e : 0.f;
      aq1 = lane + 64 < N ? Arow[lane + 64] * kLog2e : 0.f;
      cq0 = 0.f;
      cq1 = 0.f;
    }
    seg_load<TIn, K>(urow(cc), t0, L, full, su);
    seg_load<TIn, K>(drow(cc), t0, L, full, sd);
    const float bias = p.bias ? p.bias[cc.hd] : 0.f;
    const float Dd = p.D ? p.D[p.d_per_head ? cc.hd : cc.d] : 0.f;

    // prologue: step sizes from the prefetched u and delta
    float dt[K], wv[K], yv[K];
    float sdt = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float x = seg_get<TIn, K>(sd, j) + bias;
      float sp = p.softplus ? softplus_fast(x) : x;
      if (!full && t0 + j >= L) sp = 0.f;  // steps past the end are the identity (a = 1, b = 0)
      const float uu = seg_get<TIn, K>(su, j);
      dt[j] = sp;
      wv[j] = sp * uu;
      yv[j] = Dd * uu;
      sdt += sp;
    }

    // B/C rows of the states n0 and n0 + 1 (a state >= N reads as zeros): chunk q of the pair
    // is row r = q / CH (B n0, C n0, B n0+1, C n0+1) at window step (q % CH) * E.  Each thread
    // keeps a running source pointer per chunk (advanced by two states per pair) and the
    // chunk's LDS position.
    const TIn* __restrict__ Bg = static_cast<const TIn*>(p.B) + cc.b * p.B_sb + cc.g * p.B_sg;
    const TIn* __restrict__ Cg = static_cast<const TIn*>(p.C) + cc.b * p.C_sb + cc.g * p.C_sg;
    Chunk<TIn> st[CPT];
    const TIn* src[CPT];
    int64_t srcstep[CPT];
    int rrow[CPT], rq[CPT], rl[CPT];
#pragma unroll
    for (int kk = 0; kk < CPT; ++kk) {
      const int q = threadIdx.x + kk * 64 * kWaves;
      const int qc = (NCH % (64 * kWaves) == 0 || q < NCH) ? q : 0;
      const int r = qc / CH, qq = qc % CH, sw = qq * E;
      const int64_t stride = (r & 1) ? p.C_sn : p.B_sn;
      src[kk] = ((r & 1) ? Cg : Bg) + (r >> 1) * stride + w0 + sw;
      srcstep[kk] = 2 * stride;
      rrow[kk] = r;
      rq[kk] = (sw % K) / 4;
      rl[kk] = sw / K;
    }
    auto stage_load = [&](int n0) {
#pragma unroll
      for (int kk = 0; kk < CPT; ++kk) {
        const int q = threadIdx.x + kk * 64 * kWaves;
        if (NCH % (64 * kWaves) == 0 || q < NCH) {
          if (n0 + (rrow[kk] >> 1) >= N)
            st[kk].raw = u32x4{0u, 0u, 0u, 0u};
          else if (full)
            load_chunk<true>(src[kk], 0, 0, st[kk]);
          else
            load_chunk<false>(src[kk], 0, L - (w0 + (int64_t)(rl[kk] * K + rq[kk] * 4)), st[kk]);
          src[kk] += srcstep[kk];
        }
      }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int kk = 0; kk < CPT; ++kk) {
        const int q = threadIdx.x + kk * 64 * kWaves;
        if (NCH % (64 * kWaves) == 0 || q < NCH) store_chunk<TIn>(&stage[buf][rrow[kk]][0], rq[kk], rl[kk], st[kk]);
      }
    };

    stage_load(0);
    stage_store(0);
    __syncthreads();
    for (int n0 = 0; n0 < N; n0 += 2) {
      const int buf = (n0 >> 1) & 1;
      const bool more = n0 + 2 < N;
      if (more) stage_load(n0 + 2);
      const bool two = n0 + 1 < N;
      const float A0 = lane_get(aq0, aq1, n0);
      const float A1 = two ? lane_get(aq0, aq1, n0 + 1) : 0.f;  // a missing second state is inert
      // this lane's B values of both states, all LDS reads issued before any use
      f32x4 bq0[Q], bq1[Q];
      {
        const f32x4* B0 = reinterpret_cast<const f32x4*>(&stage[buf][0][0]) + lane;
        const f32x4* B1 = reinterpret_cast<const f32x4*>(&stage[buf][2][0]) + lane;
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          bq0[i] = B0[i * 64];
          bq1[i] = B1[i * 64];
        }
      }
      float av0[K], bv0[K], av1[K], bv1[K];
      float h0 = 0.f, h1 = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        av0[j] = __builtin_amdgcn_exp2f(dt[j] * A0);
        av1[j] = __builtin_amdgcn_exp2f(dt[j] * A1);
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        bv0[j] = wv[j] * bq0[j / 4][j % 4];
        bv1[j] = wv[j] * bq1[j / 4][j % 4];
        h0 = fmaf(av0[j], h0, bv0[j]);
        h1 = fmaf(av1[j], h1, bv1[j]);
      }
      // this lane's C values, read while the scan runs
      f32x4 cq0v[Q], cq1v[Q];
      {
        const f32x4* C0 = reinterpret_cast<const f32x4*>(&stage[buf][1][0]) + lane;
        const f32x4* C1 = reinterpret_cast<const f32x4*>(&stage[buf][3][0]) + lane;
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          cq0v[i] = C0[i * 64];
          cq1v[i] = C1[i * 64];
        }
      }
      // lane aggregates: decay over the lane's K steps and the lane's state from zero
      float sa0 = __builtin_amdgcn_exp2f(sdt * A0), sb0 = h0;
      float sa1 = __builtin_amdgcn_exp2f(sdt * A1), sb1 = h1;
      wave_exclusive_scan2(sa0, sb0, sa1, sb1);
      h0 = fmaf(sa0, lane_get(cq0, cq1, n0), sb0);
      h1 = fmaf(sa1, two ? lane_get(cq0, cq1, n0 + 1) : 0.f, sb1);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        h0 = fmaf(av0[j], h0, bv0[j]);
        h1 = fmaf(av1[j], h1, bv1[j]);
        yv[j] = fmaf(cq0v[j / 4][j % 4], h0, yv[j]);
        yv[j] = fmaf(cq1v[j / 4][j % 4], h1, yv[j]);
      }
      // the window's end state (lane 63) starts the next window of the row
      const float e0 = readlane_f(h0, 63), e1 = readlane_f(h1, 63);
      if (n0 < 64) cq0 = writelane_f(e0, n0, cq0); else cq1 = writelane_f(e0, n0 - 64, cq1);
      if (two) {
        if (n0 + 1 < 64) cq0 = writelane_f(e1, n0 + 1, cq0); else cq1 = writelane_f(e1, n0 - 63, cq1);
      }
      if (more) stage_store(buf ^ 1);
      __syncthreads();
    }

    if constexpr (GATE) {
      seg_load<TIn, K>(zrow(cc), t0, L, full, sz);
#pragma unroll
      for (int j = 0; j < K; ++j) yv[j] *= silu_fast(seg_get<TIn, K>(sz, j));
    }
    if (cc.live) {
      TOut* __restrict__ y = static_cast<TOut*>(p.y) + cc.b * p.y_sb + cc.d * p.y_sd;
      store_seg<K>(y, t0, L, full, yv);
    }

  }
}

template <typename TIn, typename TOut, int K>
hipError_t launch_k(const ScanArgs& a, hipStream_t s) {
  const int64_t blocks_per_bg = (a.chan_per_group + kWaves - 1) / kWaves;
  const int64_t quads = a.batch * a.groups * blocks_per_bg;
  // one block per channel quad; the block walks the quad's windows in order
  const int64_t blocks = quads;
  const dim3 grid((unsigned)blocks), block(64 * kWaves);
  if (a.z)
    hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, true, K>), grid, block, 0, s, a, blocks_per_bg);
  else
    hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, false, K>), grid, block, 0, s, a, blocks_per_bg);
  return hipGetLastError();
}

#ifndef SS_DIAG_K
#define SS_DIAG_K 16
#endif

template <typename TIn, typename TOut>
hipError_t launch_t(const ScanArgs& a, hipStream_t s) {
  return launch_k<TIn, TOut, SS_DIAG_K>(a, s);
}

}  // namespace

hipError_t launch_diag(const ScanArgs& a, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, s) : launch_t<float, float>(a, s);
}

}  // namespace ss
