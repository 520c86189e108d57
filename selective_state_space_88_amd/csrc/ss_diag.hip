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
//    is carried to the next through LDS, so each exp is evaluated exactly once;
//  - the N states are processed two at a time.  For a state each lane runs its K steps from
//    zero (keeping the K decays a_t and inputs b_t in registers), the wave combines the 64 lane
//    aggregates with a DPP scan (row_shr within rows of 16, row_bcast across rows, wave_shr for
//    the exclusive prefix), and each lane re-runs its K steps from the true incoming state to
//    form h_t and accumulate y_t += C_{t,n} h_t.  The two states of a pair are independent
//    chains, which the wave interleaves (and whose two scans fill each other's DPP wait states);
//  - B and C are shared by every channel of a (batch, group).  A small pre-pass widens them to
//    f32 and lays them out per window and state pair exactly as the scan reads them from LDS;
//    the scan then copies each pair's 16 KB into a three-slot LDS ring with direct-to-LDS
//    loads (global_load_lds_dwordx4), two pairs ahead of use, so the copy never passes through
//    registers and overlaps two pairs of arithmetic;
//  - u, delta and z of the next window are copied the same way into per-wave LDS slots while
//    the current window runs (u and delta right after they are read, z after the gate), so no
//    global load latency sits on the path.  The waits are explicit: before each ring barrier a
//    wave waits only for the pair the next iteration reads (vmcnt retires this wave's vector
//    memory operations, loads and stores alike, in issue order), never for what it issued after;
//  - softplus, D*u and the silu gate are fused; u, delta, z and y stream through HBM once, y
//    leaving through LDS so that every store instruction writes 1 KB of consecutive memory.
#include <algorithm>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kWaves = 4;                   // channels per block, one wave each
constexpr int kK = 16;                      // steps per lane
constexpr int kW = 64 * kK;                 // steps per window
constexpr int kQ = kK / 4;                  // 16-byte quads per lane of one row
constexpr int kSlotFloats = 4 * kW;         // one pair: B, C of state 2p, then of state 2p + 1
constexpr int kRing = 3;                    // pair slots in LDS
constexpr int kMaxPairs = 64;               // N <= 128

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

// One direct-to-LDS copy of 16 bytes per lane: lane i's 16 bytes from `src` land at
// lds_base + 16 i (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) then s_barrier: this wave's loads older than its last n have
// landed and its LDS reads are done.  vmcnt is an immediate, so n is dispatched over the
// values the kernel uses; anything larger waits for everything (always safe).
__device__ __forceinline__ void wait_vm_barrier(int n) {
  switch (n) {
#define SS_W(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    SS_W(1) SS_W(2) SS_W(3) SS_W(4) SS_W(5) SS_W(6) SS_W(7) SS_W(8) SS_W(9) SS_W(10)
    SS_W(11) SS_W(12) SS_W(13) SS_W(14) SS_W(15) SS_W(16) SS_W(17) SS_W(18) SS_W(19) SS_W(20)
#undef SS_W
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// K consecutive steps of one input row for one lane, as raw 32-bit words (bf16 pairs or f32).
// In a wave's LDS slot, 16-byte chunk c of lane j sits at word c * 256 + 4 j.
template <typename TIn>
struct Seg {
  static constexpr int kChunks = kK * (int)sizeof(TIn) / 16;
  static constexpr int kWords = 4 * kChunks;
  uint32_t w[kWords];
};

template <typename TIn>
__device__ __forceinline__ void seg_read(const uint32_t* slot, int lane, Seg<TIn>& s) {
#pragma unroll
  for (int c = 0; c < Seg<TIn>::kChunks; ++c) {
    const u32x4 v = reinterpret_cast<const u32x4*>(slot + c * 256)[lane];
    s.w[4 * c] = v.x;
    s.w[4 * c + 1] = v.y;
    s.w[4 * c + 2] = v.z;
    s.w[4 * c + 3] = v.w;
  }
}

template <typename TIn>
__device__ __forceinline__ float seg_get(const Seg<TIn>& s, int j) {
  if constexpr (sizeof(TIn) == 2) return (j & 1) ? bf16_hi(s.w[j / 2]) : bf16_lo(s.w[j / 2]);
  else return __uint_as_float(s.w[j]);
}

// Copy this lane's K steps of `row` starting at t0 into the wave's slot with direct-to-LDS
// loads.  Needs 16-byte aligned rows and L a multiple of 16 / sizeof(TIn), so that a chunk is
// either wholly inside the row or wholly past its end; chunks past the end copy the row's
// first chunk instead (in bounds; the scan masks those steps).
template <typename TIn>
__device__ __forceinline__ void seg_dma(const TIn* row, int64_t t0, int64_t L, uint32_t* slot) {
  constexpr int E = 16 / (int)sizeof(TIn);
#pragma unroll
  for (int c = 0; c < Seg<TIn>::kChunks; ++c) {
    const int64_t t = t0 + (int64_t)c * E;
    dma16(t < L ? row + t : row, slot + c * 256);
  }
}

// The same with ordinary element loads (any alignment; steps >= L read as 0), completed
// before returning.  Each wave reads only its own slot, so no barrier is needed after it.
template <typename TIn>
__device__ __forceinline__ void seg_fill(const TIn* row, int64_t t0, int64_t L, uint32_t* slot, int lane) {
  Seg<TIn> s;
#pragma unroll
  for (int i = 0; i < Seg<TIn>::kWords; ++i) s.w[i] = 0u;
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    if (t0 + j < L) {
      if constexpr (sizeof(TIn) == 2)
        s.w[j / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(row)[t0 + j] << (16 * (j % 2));
      else
        s.w[j] = __float_as_uint(reinterpret_cast<const float*>(row)[t0 + j]);
    }
  }
#pragma unroll
  for (int c = 0; c < Seg<TIn>::kChunks; ++c)
    reinterpret_cast<u32x4*>(slot + c * 256)[lane] =
        u32x4{s.w[4 * c], s.w[4 * c + 1], s.w[4 * c + 2], s.w[4 * c + 3]};
}

// Store this wave's window of y (lane j holds steps 16 j .. 16 j + 15) with each store
// instruction covering 1 KB of consecutive y: the lanes' 16-byte granules go to LDS, granule
// g at g ^ ((g >> 4) & (NC - 1)) so that neither the writes nor the reads conflict on banks,
// and instruction i then has lane j read and store granule 64 i + j.
template <typename TOut>
__device__ __forceinline__ void store_window_coalesced(uint32_t* stg, int lane, const float (&v)[kK],
                                                       TOut* __restrict__ y) {
  constexpr int NC = kK * (int)sizeof(TOut) / 16;
  u32x4 gr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if constexpr (sizeof(TOut) == 4) {
      gr[c] = u32x4{__float_as_uint(v[4 * c]), __float_as_uint(v[4 * c + 1]), __float_as_uint(v[4 * c + 2]),
                    __float_as_uint(v[4 * c + 3])};
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = f32_to_bf16_bits(v[8 * c + 2 * e]) | (f32_to_bf16_bits(v[8 * c + 2 * e + 1]) << 16);
      gr[c] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  u32x4* q = reinterpret_cast<u32x4*>(stg);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int g = NC * lane + c;
    q[g ^ ((g >> 4) & (NC - 1))] = gr[c];
  }
  u32x4* out = reinterpret_cast<u32x4*>(y);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int g = 64 * i + lane;
    __builtin_nontemporal_store(q[g ^ ((g >> 4) & (NC - 1))], out + g);
  }
}

// Pre-pass: B and C of every (batch, group) widened to f32, zero past L and past state N - 1,
// in the order the scan copies them: [batch, group][window][pair][row r][quad i][lane j][4],
// r = (B, C of state 2 pair, B, C of state 2 pair + 1), and element e of quad i of lane j is
// window step 16 j + 4 i + e.  One thread writes one 16-byte quad.
template <typename TIn>
__global__ __launch_bounds__(256) void bc_pack_kernel(ScanArgs p, f32x4* __restrict__ ws, int npairs,
                                                      int64_t nwin) {
  const int64_t total = p.batch * p.groups * nwin * npairs * 4 * kQ * 64;
  const int64_t L = p.L;
  for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
    const int j = (int)(o % 64);
    int64_t rest = o / 64;
    const int i = (int)(rest % kQ);
    rest /= kQ;
    const int r = (int)(rest % 4);
    rest /= 4;
    const int pair = (int)(rest % npairs);
    rest /= npairs;
    const int64_t win = rest % nwin;
    const int64_t bg = rest / nwin;
    const int64_t b = bg / p.groups, g = bg % p.groups;
    const int n = 2 * pair + (r >> 1);
    const int64_t t = win * kW + (int64_t)j * kK + 4 * i;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (n < p.N) {
      const TIn* row = (r & 1) ? static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg + n * p.C_sn
                               : static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg + n * p.B_sn;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < L) v[e] = to_f32(row[t + e]);
    }
    ws[o] = v;
  }
}

template <typename TIn, typename TOut, bool GATE, bool VEC>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void diag_fwd_kernel(
    ScanArgs p, const float* __restrict__ ws, int npairs, int64_t nwin, int64_t blocks_per_bg) {
  constexpr int NCI = Seg<TIn>::kChunks;             // 16-byte copies per lane per input row
  constexpr int kSegWords = NCI * 256;
  constexpr int NCO = kK * (int)sizeof(TOut) / 16;   // 16-byte stores per lane of y
  // ring[s]: one pair of B/C rows.  Row r of a slot holds quad i of lane j at float offset
  // (i * 64 + j) * 4, so one ds_read_b128 of the whole wave is 1 KB of consecutive LDS.
  __shared__ __attribute__((aligned(16))) float ring[kRing][kSlotFloats];
  // per wave: u, delta, z of one window
  __shared__ __attribute__((aligned(16))) uint32_t xin[3][kWaves][kSegWords];
  // per wave and pair: [0] = (A_2p, A_2p+1) * log2 e, [1] = the carried state of the pair
  __shared__ float2 par[kWaves][kMaxPairs][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t L = p.L;
  const int N = p.N;
  const int P = npairs;

  const int64_t quad = blockIdx.x;
  const int64_t bg = quad / blocks_per_bg, blk = quad % blocks_per_bg;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t local = blk * kWaves + wave;
  const bool live = local < p.chan_per_group;
  const int64_t d = g * p.chan_per_group + (live ? local : p.chan_per_group - 1);
  const int64_t hd = d / p.chan_per_head;
  const TIn* urow = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* drow = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TIn* zrow = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  const float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;
  const float* wsq = ws + bg * nwin * P * (int64_t)kSlotFloats;
  const int Qt = (int)(nwin * P);  // pair stages of this block, in order (window-major)

  {
    const float* Ar = p.A + d * p.A_sd;
    for (int pp = lane; pp < P; pp += 64) {
      const int n = 2 * pp;
      par[wave][pp][0] = make_float2(Ar[n] * kLog2e, n + 1 < N ? Ar[n + 1] * kLog2e : 0.f);
      par[wave][pp][1] = make_float2(0.f, 0.f);
    }
  }
  uint32_t* xu = xin[0][wave];
  uint32_t* xd = xin[1][wave];
  uint32_t* xz = xin[2][wave];

  // this wave's quarter (4 KB) of pair stage qs into ring slot s
  // Stage copies go through a buffer resource over this (batch, group)'s stages of one window,
  // so that the per-stage offset is a scalar and the lane offset a constant.
  const uint32_t lane_off = (uint32_t)lane * 16u + (uint32_t)wave * 4096u;
  auto stage_dma = [&](int qs, int s) {
    const int64_t wq = qs / P;
    const uint32_t off = (uint32_t)(qs - wq * P) * (uint32_t)(kSlotFloats * 4);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(wsq + wq * P * (int64_t)kSlotFloats), (short)0, P * kSlotFloats * 4, 0x00020000);
    float* dst = &ring[s][wave * 1024];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + i * 256), 16,
                                               lane_off + i * 1024, off, 0, 0);
  };
  auto x_copy = [&](const TIn* row, int64_t w, uint32_t* slot) {
    const int64_t t0 = w * kW + (int64_t)lane * kK;
    if constexpr (VEC) seg_dma<TIn>(row, t0, L, slot);
    else seg_fill<TIn>(row, t0, L, slot, lane);
  };

  if constexpr (VEC) {
    x_copy(urow, 0, xu);
    x_copy(drow, 0, xd);
    if constexpr (GATE) x_copy(zrow, 0, xz);
  }
  stage_dma(0, 0);
  if (Qt > 1) stage_dma(1, 1);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  int q = 0;       // current pair stage
  int slot = 0;    // its ring slot (q mod 3)
  int carry_ops = 0;  // memory ops issued in the last epilogue (counted by the first wait after it)
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t w0 = w * kW;
    const int64_t t0 = w0 + (int64_t)lane * kK;
    const bool full = w0 + kW <= L;

    // prologue: step sizes from this window's u and delta
    if constexpr (!VEC) {
      x_copy(urow, w, xu);
      x_copy(drow, w, xd);
    }
    float dt[kK], wv[kK], yv[kK];
    float sdt = 0.f;
    {
      Seg<TIn> su, sd;
      seg_read<TIn>(xu, lane, su);
      seg_read<TIn>(xd, lane, sd);
      if (full) {
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          const float x = seg_get<TIn>(sd, j) + bias;
          const float sp = p.softplus ? softplus_fast(x) : x;
          const float uu = seg_get<TIn>(su, j);
          dt[j] = sp;
          wv[j] = sp * uu;
          yv[j] = Dd * uu;
          sdt += sp;
        }
      } else {
        // steps past the end are the identity (a = 1, b = 0)
        const int rem = (int)(L - t0 < 0 ? 0 : (L - t0 > kK ? kK : L - t0));
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          const float x = seg_get<TIn>(sd, j) + bias;
          const float sp = j < rem ? (p.softplus ? softplus_fast(x) : x) : 0.f;
          const float uu = j < rem ? seg_get<TIn>(su, j) : 0.f;
          dt[j] = sp;
          wv[j] = sp * uu;
          yv[j] = Dd * uu;
          sdt += sp;
        }
      }
    }
    // the next window's u and delta into the slots just read
    int boundary_ops = carry_ops;
    if constexpr (VEC) {
      if (w + 1 < nwin) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        x_copy(urow, w + 1, xu);
        x_copy(drow, w + 1, xd);
        boundary_ops += 2 * NCI;
      }
    }

    for (int pp = 0; pp < P; ++pp) {
      int allow = pp == 0 ? boundary_ops : 0;
      if (q + 2 < Qt) {
        stage_dma(q + 2, slot == 0 ? 2 : slot - 1);
        allow += 4;
      }
      const float2 Ap = par[wave][pp][0];
      const float2 hin = par[wave][pp][1];
      const float* S = ring[slot];
      // this lane's B values of both states, all LDS reads issued before any use
      f32x4 bq0[kQ], bq1[kQ];
      {
        const f32x4* B0 = reinterpret_cast<const f32x4*>(S) + lane;
        const f32x4* B1 = reinterpret_cast<const f32x4*>(S + 2 * kW) + lane;
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
          bq0[i] = B0[i * 64];
          bq1[i] = B1[i * 64];
        }
      }
      float av0[kK], bv0[kK], av1[kK], bv1[kK];
      float h0 = 0.f, h1 = 0.f;
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        av0[j] = __builtin_amdgcn_exp2f(dt[j] * Ap.x);
        av1[j] = __builtin_amdgcn_exp2f(dt[j] * Ap.y);
      }
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        bv0[j] = wv[j] * bq0[j / 4][j % 4];
        bv1[j] = wv[j] * bq1[j / 4][j % 4];
        h0 = fmaf(av0[j], h0, bv0[j]);
        h1 = fmaf(av1[j], h1, bv1[j]);
      }
      // this lane's C values, read while the scan runs
      f32x4 cq0[kQ], cq1[kQ];
      {
        const f32x4* C0 = reinterpret_cast<const f32x4*>(S + kW) + lane;
        const f32x4* C1 = reinterpret_cast<const f32x4*>(S + 3 * kW) + lane;
#pragma unroll
        for (int i = 0; i < kQ; ++i) {
          cq0[i] = C0[i * 64];
          cq1[i] = C1[i * 64];
        }
      }
      // lane aggregates: decay over the lane's K steps and the lane's state from zero
      float sa0 = __builtin_amdgcn_exp2f(sdt * Ap.x), sb0 = h0;
      float sa1 = __builtin_amdgcn_exp2f(sdt * Ap.y), sb1 = h1;
      wave_exclusive_scan2(sa0, sb0, sa1, sb1);
      h0 = fmaf(sa0, hin.x, sb0);
      h1 = fmaf(sa1, hin.y, sb1);
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        h0 = fmaf(av0[j], h0, bv0[j]);
        h1 = fmaf(av1[j], h1, bv1[j]);
        yv[j] = fmaf(cq0[j / 4][j % 4], h0, yv[j]);
        yv[j] = fmaf(cq1[j / 4][j % 4], h1, yv[j]);
      }
      // the window's end state (lane 63) starts the same pair in the next window
      if (lane == 63) par[wave][pp][1] = make_float2(h0, h1);
      // the next stage's copies (this wave's and, after the barrier, everyone's) have landed
      if (q + 1 < Qt) wait_vm_barrier(allow);
      else asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // slot free for y
      ++q;
      slot = slot == 2 ? 0 : slot + 1;
    }

    // epilogue: gate, store, then this slot's z for the next window.  Only the stage copy
    // issued by the last pair may still be in flight here: everything before it (this
    // window's z and the next window's u and delta) has landed.
    if (q + 1 < Qt) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    carry_ops = 0;
    if constexpr (GATE) {
      if constexpr (!VEC) x_copy(zrow, w, xz);
      Seg<TIn> sz;
      seg_read<TIn>(xz, lane, sz);
#pragma unroll
      for (int j = 0; j < kK; ++j) yv[j] *= silu_fast(seg_get<TIn>(sz, j));
    }
    if (live) {
      TOut* __restrict__ y = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
      if (VEC && full) {
        // through this wave's quarter of the last pair's ring slot (free after that pair's
        // barrier; the next copy into it is issued by this wave after these reads), so that
        // each store instruction writes 1 KB of consecutive y
        uint32_t* stg = reinterpret_cast<uint32_t*>(&ring[slot == 0 ? 2 : slot - 1][wave * 1024]);
        store_window_coalesced<TOut>(stg, lane, yv, y + w0);
        carry_ops += NCO;
      } else {
        store_seg<kK>(y, t0, L, false, yv);
      }
    }
    if constexpr (VEC && GATE) {
      if (w + 1 < nwin) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        x_copy(zrow, w + 1, xz);
        carry_ops += NCI;
      }
    }
  }
}

int npairs_of(const ScanArgs& a) { return (a.N + 1) / 2; }
int64_t nwin_of(const ScanArgs& a) { return (a.L + kW - 1) / kW; }

template <typename TIn, typename TOut>
hipError_t launch_t(const ScanArgs& a, float* ws, hipStream_t s) {
  const int P = npairs_of(a);
  const int64_t nwin = nwin_of(a);
  {
    const int64_t quads = a.batch * a.groups * nwin * P * 4 * kQ * 64;
    const int64_t blocks = std::min<int64_t>((quads + 255) / 256, 16384);
    hipLaunchKernelGGL((bc_pack_kernel<TIn>), dim3((unsigned)blocks), dim3(256), 0, s, a,
                       reinterpret_cast<f32x4*>(ws), P, nwin);
  }
  const int64_t blocks_per_bg = (a.chan_per_group + kWaves - 1) / kWaves;
  const int64_t blocks = a.batch * a.groups * blocks_per_bg;  // one block per channel quad
  const bool dma = a.vec && a.L % (16 / (int64_t)sizeof(TIn)) == 0;
  const dim3 grid((unsigned)blocks), block(64 * kWaves);
#define SS_LAUNCH(G, V) \
  hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, G, V>), grid, block, 0, s, a, ws, P, nwin, blocks_per_bg)
  if (a.z) {
    if (dma) SS_LAUNCH(true, true); else SS_LAUNCH(true, false);
  } else {
    if (dma) SS_LAUNCH(false, true); else SS_LAUNCH(false, false);
  }
#undef SS_LAUNCH
  return hipGetLastError();
}

}  // namespace

int64_t diag_workspace_floats(const ScanArgs& a) {
  return a.batch * a.groups * nwin_of(a) * npairs_of(a) * (int64_t)kSlotFloats;
}

hipError_t launch_diag(const ScanArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
