// ss_ssd_bwd.hip -- backward of the scalar-decay scan in the chunked matrix form (gfx950, MFMA).
//
// With one decay per head (a_t = exp(dt_t A_h) shared by the head's channels and states; the
// Mamba-2 layout of the bqwf.cn survey, section 3.2, and the omica.com.cn explainer, section 6.2)
// the recurrence over a chunk of T steps is a handful of dense products, the state-space duality
// the pages describe.  With s_i the cumulative log decay inside the chunk (s_i includes step i),
// x_j = dt_j u_j (one value per channel p), H0 the state before the chunk and R the adjoint that
// reaches the chunk's last step from the right (R = a g of the next chunk's first step):
//   h_i = e^{s_i} H0 + sum_{j<=i} e^{s_i - s_j} x_j B_j^T
//   g_i = sum_{k>=i} e^{s_k - s_i} dy_k C_k^T + e^{s_{T-1} - s_i} R            (g = dLoss/dh)
// and the gradients of the chunk are, with DX = dY X^T, CB = C B^T, M1 = L o DX (L_kj =
// e^{s_k - s_j} for k >= j, else 0):
//   dC = diag(e^s) (dY H0) + M1 B                dB = M1^T C + diag(e^{s_{T-1} - s}) (X R)
//   dX = (L o CB)^T dY + diag(e^{s_{T-1} - s}) B R^T,   du = dt dX + D dy
//   R  <- e^{s_{T-1}} R + dY^T diag(e^s) C      (the adjoint handed to the previous chunk)
// The decay's gradient a_j dLoss/da_j = <g_j, a_j h_{j-1}> = <g_j, h_j> - x_j . dx_j, where
//   <g_j, h_j> = sum_{k>=j>=i} e^{s_k - s_i} DX_ki CB_ki + sum_{k>=j} e^{s_k} (dY H0)_k . C_k
//              + sum_{i<=j} e^{s_{T-1} - s_i} (X R)_i . B_i + e^{s_{T-1}} <R, H0>,
// gives ddt_j = u_j . dx_j + A a_j dLoss/da_j and dA = sum_j dt_j a_j dLoss/da_j.
//
// The first term is a sum over the rectangle k >= j >= i of W = M1 o CB; it equals the prefix sum of
// W's column sums minus the exclusive prefix sum of its row sums, so every per-step quantity is a
// scan over the chunk's 32 steps.  u is staged raw and dt folded into the products' epilogues.
//
// Two passes per (batch, head, 64-channel slab): the first walks the chunks forward and stores
// every chunk's starting state H0 (f32, [N][64]); the second walks them in reverse carrying R in
// MFMA accumulators.  The products read operands staged in LDS with the contracted index
// contiguous.  With bf16 inputs they run on v_mfma_f32_16x16x32_bf16, each f32 operand split into
// bf16 hi and lo parts (three products, two when the other operand is bf16 already: u, B, C);
// with f32 inputs on v_mfma_f32_16x16x4_f32 (each lane reads four consecutive k with one 16-byte
// read; the order of k inside a block of 16 is permuted the same way on both operands).  dB and
// dC are summed over the group's heads with atomic adds; per-head sums (ddelta over slabs, dA,
// dD, dbias) likewise.  A gated layer arrives here on dy s(z), with the gate composed around
// this backward by the caller.
#include <type_traits>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kCT = 32;            // steps per chunk
constexpr int kCP = 64;            // channels per block (a slab)
constexpr int kThr = 256;          // 4 waves
constexpr int kSP = kCP + 4;       // LDS row stride of [.][64] operands (floats)
constexpr int kST = kCT + 4;       // LDS row stride of [.][32] operands

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc[t] += A[i][0..K) . Bt_t[j][0..K) for NT 16x16 tiles sharing their 16 rows of A: lane l takes
// row i = l % 16 of A and row j = l % 16 of tile t's Bt = B + t * bstep.  Rows are k-contiguous
// and 16-byte aligned; lane l supplies k = 16 kb + 4 (l / 16) + m to MFMA m of block kb.  With
// SCALE, A's k-th column is multiplied by sc[k] on the way.  With TR the tiles come out transposed
// (acc[t] += Bt_t . A^T): lane l then holds column i = l % 16 and rows j = 4 (l / 16) + m.
template <int K, int NT, bool SCALE = false, bool TR = false>
__device__ __forceinline__ void mm(const float* A, int lda, const float* B, int ldb, int bstep, int lane,
                                   f32x4 (&acc)[NT], const float* sc = nullptr) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + 4 * q;
  const float* b = B + r * ldb + 4 * q;
#pragma unroll
  for (int kb = 0; kb < K / 16; ++kb) {
    f32x4 av = *reinterpret_cast<const f32x4*>(a + 16 * kb);
    if constexpr (SCALE) {
      const f32x4 s = *reinterpret_cast<const f32x4*>(sc + 16 * kb + 4 * q);
      av = av * s;
    }
    f32x4 bv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bv[t] = *reinterpret_cast<const f32x4*>(b + t * bstep + 16 * kb);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = TR ? mma4(bv[t][m], av[m], acc[t]) : mma4(av[m], bv[t][m], acc[t]);
  }
}

// As mm with K = 64, Bt a [rows][64] array swizzled as swz (rows 16 t + l % 16 of tile t).
template <int NT, bool TR = false>
__device__ __forceinline__ void mm_swz(const float* A, int lda, const float* Bsw, int lane, f32x4 (&acc)[NT]) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + 4 * q;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(a + 16 * kb);
    f32x4 bv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = 16 * t + r;
      bv[t] = *reinterpret_cast<const f32x4*>(Bsw + n * 64 + 4 * ((4 * kb + q) ^ r));
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = TR ? mma4(bv[t][m], av[m], acc[t]) : mma4(av[m], bv[t][m], acc[t]);
  }
}

// ---- the same products on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, bf16 inputs only).
// An f32 operand is split x = hi + lo (both bf16, round to nearest even; |x - hi - lo| <= 2^-18 |x|)
// and a product takes hi.hi + hi.lo + lo.hi (the dropped lo.lo is below 2^-16 of it); an operand
// that holds bf16 values exactly (u, B, C) is packed as it is and needs no lo.  Lane l supplies
// k = 32 kb + 8 (l / 16) + 0..7 of its rows (the f32 form above permutes k the same way on both
// operands, so the sums are the same products in another order); the accumulator layout is the
// f32 form's.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Split8 {
  bf16x8 hi, lo;
};

// eight values -> bf16 hi (and lo unless EXACT, where the values are bf16 already)
template <bool EXACT>
__device__ __forceinline__ Split8 split8(const float (&x)[8]) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (EXACT) {
      h[j] = (__float_as_uint(x[2 * j]) >> 16) | (__float_as_uint(x[2 * j + 1]) & 0xffff0000u);
      l[j] = 0u;
    } else {
      h[j] = pk_bf16(x[2 * j], x[2 * j + 1]);
      l[j] = pk_bf16(x[2 * j] - __uint_as_float(h[j] << 16), x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u));
    }
  }
  Split8 r;
  r.hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  r.lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
  return r;
}

// acc += a . b over 32 k of one lane's pair of operands (TR: acc += b . a)
template <bool AX, bool BX, bool TR>
__device__ __forceinline__ f32x4 mma3(const Split8& a, const Split8& b, f32x4 acc) {
  const bf16x8& ah = a.hi;
  const bf16x8& bh = b.hi;
  acc = TR ? mma32(bh, ah, acc) : mma32(ah, bh, acc);
  if constexpr (!BX) acc = TR ? mma32(b.lo, ah, acc) : mma32(ah, b.lo, acc);
  if constexpr (!AX) acc = TR ? mma32(bh, a.lo, acc) : mma32(a.lo, bh, acc);
  return acc;
}

__device__ __forceinline__ void read8(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

// mm on the bf16 matrix cores; AX / BX: A / B hold bf16 values exactly
template <int K, int NT, bool AX, bool BX, bool SCALE = false, bool TR = false>
__device__ __forceinline__ void mm3(const float* A, int lda, const float* B, int ldb, int bstep, int lane,
                                    f32x4 (&acc)[NT], const float* sc = nullptr) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + 8 * q;
  const float* b = B + r * ldb + 8 * q;
#pragma unroll
  for (int kb = 0; kb < K / 32; ++kb) {
    float av[8];
    read8(a + 32 * kb, av);
    if constexpr (SCALE) {
      float s8[8];
      read8(sc + 32 * kb + 8 * q, s8);
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] *= s8[i];
    }
    const Split8 as = split8<AX && !SCALE>(av);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float bv[8];
      read8(b + t * bstep + 32 * kb, bv);
      acc[t] = mma3<AX && !SCALE, BX, TR>(as, split8<BX>(bv), acc[t]);
    }
  }
}

// mm_swz on the bf16 matrix cores (K = 64, Bsw swizzled as swz; A and B both split)
template <int NT, bool TR = false>
__device__ __forceinline__ void mm3_swz(const float* A, int lda, const float* Bsw, int lane, f32x4 (&acc)[NT]) {
  const int r = lane & 15, q = lane >> 4;
  const float* a = A + r * lda + 8 * q;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    float av[8];
    read8(a + 32 * kb, av);
    const Split8 as = split8<false>(av);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = 16 * t + r;
      // granules 8 kb + 2 q and 8 kb + 2 q + 1 of row n
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(Bsw + n * 64 + 4 * ((8 * kb + 2 * q) ^ r));
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(Bsw + n * 64 + 4 * ((8 * kb + 2 * q + 1) ^ r));
      const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      acc[t] = mma3<false, false, TR>(as, split8<false>(bv), acc[t]);
    }
  }
}

// DPP move of v with control CTRL on the rows in ROWMASK; lanes with no source keep `old`
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWMASK, 0xf, false));
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// sum over each row of 16 lanes (lanes with the same l / 16), in every lane: row_ror 8, 4, 2, 1
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0x128>(0.f, v);
  v += dpp<0x124>(0.f, v);
  v += dpp<0x122>(0.f, v);
  v += dpp<0x121>(0.f, v);
  return v;
}

// sum over the wave (wave-uniform)
__device__ __forceinline__ float wave_total(float v) {
  v = row16_sum(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// inclusive prefix sum over lanes 0..31 (and, separately, over lanes 32..63): row_shr 1, 2, 4, 8
// within rows of 16, then row_bcast:15 adds the last lane of rows 0 and 2 to rows 1 and 3
__device__ __forceinline__ float scan32(float v) {
  v += dpp<0x111>(0.f, v);
  v += dpp<0x112>(0.f, v);
  v += dpp<0x114>(0.f, v);
  v += dpp<0x118>(0.f, v);
  v += dpp<0x142, 0xa>(0.f, v);
  return v;
}

struct Blk {
  int64_t b, h, g, d0;
};

__device__ __forceinline__ Blk block_of(const BwdArgs& p, int64_t blk) {
  const int slabs = p.chan_per_head / kCP;
  const int64_t bh = blk / slabs, slab = blk % slabs;
  Blk r;
  r.b = bh / p.heads;
  r.h = bh % p.heads;
  r.d0 = r.h * p.chan_per_head + slab * kCP;
  r.g = r.d0 / p.chan_per_group;
  return r;
}

// One direct-to-LDS copy of 16 bytes per lane: lane i's 16 bytes from `src` land at lds + 16 i
// (lds is wave-uniform).  Completion is observed with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const float* src, float* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Offset (floats) of granule g (4 floats) of row n in a [rows][64] array whose rows keep granule
// g at position g ^ (n % 16): sixteen lanes reading the same granule of sixteen rows hit
// different banks.
__device__ __forceinline__ int swz(int n, int g) { return n * kCP + 4 * (g ^ (n & 15)); }

// Pass 1: the state before every chunk, [blocks][chunks][NP][64] f32 (row n holds H0[0..63][n],
// swizzled as swz), and C B^T of every chunk, [batch][groups][chunks][4 tiles][64 lanes][4] in the
// lane order of the reverse pass's 16x16 tiles; a group's chunks are shared out over its blocks.
// The states evolve independently, so each (batch, head, slab) takes kStateSplit blocks, one per
// share of the states (more blocks than CUs on the multi-head layers, and with 128 states two or
// three blocks per CU to cover each other's waits).
template <int NT>
constexpr int kStateSplit = NT >= 8 ? 4 : 2;
template <typename TIn, int NT>
__global__ __launch_bounds__(kThr) void ssdb_state_kernel(BwdArgs p, int64_t nch, float* __restrict__ ws,
                                                          float* __restrict__ cbws) {
  constexpr int NP = 16 * NT;
  constexpr int SPL = kStateSplit<NT>;
  constexpr int NH = NT / SPL, NPH = NP / SPL;   // this block's state tiles and states
  constexpr int kSN = NP + 4;
  // bf16 inputs: the products on the bf16 matrix cores (mm3), else fp32 MFMA
  constexpr bool B3 = std::is_same<TIn, bf16_t>::value;
  __shared__ __attribute__((aligned(16))) float xt[kCP * kST];   // u^T [p][t]
  __shared__ __attribute__((aligned(16))) float wb[NPH * kST];   // e^{s_{T-1} - s_t} dt_t B [n][t], this share
  __shared__ __attribute__((aligned(16))) float ctn[kCT * kSN];  // C [t][n] (chunks whose C B^T this block forms)
  __shared__ __attribute__((aligned(16))) float btn[kCT * kSN];  // B [t][n]
  __shared__ float ss2[kCT], sdt[kCT];                           // cumulative log2 decay, dt
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int64_t bx = blockIdx.x / SPL;
  const int nh = blockIdx.x % SPL;           // share of the states: rows nh NPH ..
  const Blk k = block_of(p, bx);
  const int N = p.N;
  const int64_t L = p.L;
  const float A2 = p.A[k.h] * kLog2e;
  const float bias = p.bias ? p.bias[k.h] : 0.f;
  const TIn* dr = static_cast<const TIn*>(p.delta) + k.b * p.dl_sb + k.h * p.dl_sh;
  const TIn* ub = static_cast<const TIn*>(p.u) + k.b * p.u_sb + k.d0 * p.u_sd;
  const TIn* Bb = static_cast<const TIn*>(p.B) + k.b * p.B_sb + k.g * p.B_sg;
  const TIn* Cb = static_cast<const TIn*>(p.C) + k.b * p.C_sb + k.g * p.C_sg;
  float* wsb = ws + bx * nch * NP * kCP;
  float* cbg = cbws + (k.b * p.groups + k.g) * nch * 1024;
  const int ng = p.chan_per_group / kCP;                    // blocks sharing the group's B, C
  const int gi = (int)((k.d0 % p.chan_per_group) / kCP);
  // this thread's share of a chunk's loads: u (row pp, 8 steps from tt); B (row nh NPH + bn of
  // the share, 16 steps from bt)
  const int pp = tid >> 2, tt = 8 * (tid & 3);
  const int bn = tid >> 1, bt = 16 * (tid & 1), bnr = nh * NPH + bn;
  // two register sets, so that a chunk's loads are issued two chunks ahead of their use
  float pu[2][8], pbv[2][16], pdl[2] = {0.f, 0.f};
  auto fetch = [&](int64_t c, auto S) {
    constexpr int r = decltype(S)::value;
    const int64_t t0 = c * kCT;
    load_seg<8>(ub + pp * p.u_sd, t0 + tt, L, p.vec, pu[r]);
    if (bn < NPH && bnr < N) {
      load_seg<16>(Bb + bnr * p.B_sn, t0 + bt, L, p.vec, pbv[r]);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) pbv[r][e] = 0.f;
    }
    if (wave == 0) pdl[r] = (lane < kCT && t0 + lane < L) ? to_f32(dr[t0 + lane]) : 0.f;
  };
  const std::integral_constant<int, 0> set0{};
  const std::integral_constant<int, 1> set1{};
  fetch(0, set0);
  if (nch > 1) fetch(1, set1);
  f32x4 H[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) H[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // chunk c from register set S; false once the walk is over
  auto step = [&](int64_t c, auto S) -> bool {
    constexpr int r = decltype(S)::value;
    // the state before chunk c: lane holds H[p = 16 wave + 4 q + r'][n = NPH nh + 16 j + l16],
    // granule 4 wave + q
    float* hc = wsb + c * NP * kCP;
#pragma unroll
    for (int j = 0; j < NH; ++j)
      *reinterpret_cast<f32x4*>(hc + swz(nh * NPH + 16 * j + l16, 4 * wave + q)) = H[j];
    const bool cbjob = nh == 0 && c % ng == gi;
    if (c == nch - 1 && !cbjob) return false;
    const int64_t t0 = c * kCT;
    if (wave == 0) {
      const float x = pdl[r] + bias;
      const float dt = (lane < kCT && t0 + lane < L) ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      const float s = scan32(dt * A2);
      if (lane < kCT) {
        ss2[lane] = s;
        sdt[lane] = dt;
      }
    }
    *reinterpret_cast<f32x4*>(xt + pp * kST + tt) = f32x4{pu[r][0], pu[r][1], pu[r][2], pu[r][3]};
    *reinterpret_cast<f32x4*>(xt + pp * kST + tt + 4) = f32x4{pu[r][4], pu[r][5], pu[r][6], pu[r][7]};
    if (cbjob) {
      // this chunk's C and B with n contiguous, for C B^T
      for (int i = tid; i < NP * 4; i += kThr) {
        const int n = i >> 2, t8 = 8 * (i & 3);
        float v[8], w[8];
        if (n < N) {
          load_seg<8>(Cb + n * p.C_sn, t0 + t8, L, p.vec, v);
          load_seg<8>(Bb + n * p.B_sn, t0 + t8, L, p.vec, w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = w[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ctn[(t8 + e) * kSN + n] = v[e];
          btn[(t8 + e) * kSN + n] = w[e];
        }
      }
    }
    __syncthreads();   // ss2, sdt, xt, ctn, btn ready
    if (bn < NPH) {
      const float send = ss2[kCT - 1];
      float* v = pbv[r];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] *= sdt[bt + e] * __builtin_amdgcn_exp2f(send - ss2[bt + e]);
#pragma unroll
      for (int e = 0; e < 16; e += 4)
        *reinterpret_cast<f32x4*>(wb + bn * kST + bt + e) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    }
    if (c + 2 < nch) fetch(c + 2, S);   // this set's next chunk
    if (cbjob) {
      f32x4 cb[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (B3) mm3<NP, 1, true, true>(ctn + 16 * (wave >> 1) * kSN, kSN, btn + 16 * (wave & 1) * kSN, kSN, 0, lane, cb);
      else mm<NP, 1>(ctn + 16 * (wave >> 1) * kSN, kSN, btn + 16 * (wave & 1) * kSN, kSN, 0, lane, cb);
      *reinterpret_cast<f32x4*>(cbg + c * 1024 + (wave * 64 + lane) * 4) = cb[0];
    }
    __syncthreads();   // wb ready
    if (c == nch - 1) return false;
    const float dec = __builtin_amdgcn_exp2f(ss2[kCT - 1]);
#pragma unroll
    for (int j = 0; j < NH; ++j) H[j] = H[j] * dec;
    if constexpr (B3) mm3<kCT, NH, true, false>(xt + 16 * wave * kST, kST, wb, kST, 16 * kST, lane, H);
    else mm<kCT, NH>(xt + 16 * wave * kST, kST, wb, kST, 16 * kST, lane, H);
    __syncthreads();   // xt, wb, ss2, ctn, btn are rewritten by the next chunk
    return true;
  };
  for (int64_t c = 0; c < nch; c += 2) {
    if (!step(c, set0)) break;
    if (c + 1 >= nch || !step(c + 1, set1)) break;
  }
}

// Sequence segments of pass 2.  With fewer (batch, head, slab) rows than about five per CU, each
// row's chunks are cut into segments of cps chunks, one pass-2 block per (row, segment), so that
// every CU has blocks to run.  Walking chunk c leaves R <- D_c R + Q_c (D_c = 2^(A log2 e dt-sum
// of c), Q_c = dY^T diag(e^s) C), so segment j's own part of the R it hands to the segment on its
// left, and its decay, are
//   Lj = sum_{t in seg j} 2^(A log2 e S_t) dY_t^T C_t,   Dj = 2^(A log2 e S_end)
// with S_t the step sizes summed from the segment's first step to t; the R entering segment k
// from the right is R(k) = D_{k+1} R(k+1) + L_{k+1}, R(last) = 0.  The pre-pass below forms Lj
// (a [64 x N] product over the segment's steps, on the matrix cores like pass 2's R update) and
// log2 Dj; pass 2's prologue combines those of the segments to its right.
struct SegsB {
  int64_t cps;   // chunks per segment
  int32_t nseg;  // segments per row
};

SegsB ssdb_seg_plan(const BwdArgs& a) {
  const int64_t nch = (a.L + kCT - 1) / kCT;
  const int64_t rows = a.batch * a.heads * (a.chan_per_head / kCP);
  int64_t S = 1;
#ifndef SS_SSDB_SEG_ROUNDS
#define SS_SSDB_SEG_ROUNDS 5   // pass-2 blocks per CU the segments aim for (a tuning override)
#endif
  if (rows > 0) S = std::min<int64_t>((SS_SSDB_SEG_ROUNDS * (int64_t)cu_count() + rows - 1) / rows, nch / 8);
  S = std::max<int64_t>(S, 1);
  const int64_t cps = std::max<int64_t>((nch + S - 1) / S, 1);
  return {cps, (int32_t)std::max<int64_t>((nch + cps - 1) / cps, 1)};
}

// per (row, segment): Lj as [64][NP] f32, then log2 Dj
template <int NP>
constexpr int64_t seg_floats() { return (int64_t)kCP * NP + 1; }

// One block of 4 waves per (row, segment j >= 1); wave w forms rows p = 16 w .. of Lj.
template <typename TIn, typename TDy, int NT>
__global__ __launch_bounds__(kThr) void ssdb_seg_kernel(BwdArgs p, int64_t nch, SegsB sg, float* __restrict__ segw) {
  constexpr int NP = 16 * NT;
  constexpr bool B3 = std::is_same<TIn, bf16_t>::value;
  __shared__ __attribute__((aligned(16))) float dyt[kCP * kST];   // dy [p][t]
  __shared__ __attribute__((aligned(16))) float cnt[NP * kST];    // C [n][t]
  __shared__ __attribute__((aligned(16))) float wts[kCT];         // 2^(A log2 e S_t)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nrow = p.batch * p.heads * (p.chan_per_head / kCP);
  const int64_t rowi = blockIdx.x % nrow;
  const int j = 1 + (int)(blockIdx.x / nrow);
  const Blk k = block_of(p, rowi);
  const int N = p.N;
  const int64_t L = p.L;
  const float A2 = p.A[k.h] * kLog2e;
  const float bias = p.bias ? p.bias[k.h] : 0.f;
  const TIn* dr = static_cast<const TIn*>(p.delta) + k.b * p.dl_sb + k.h * p.dl_sh;
  const TDy* yb = static_cast<const TDy*>(p.dy) + k.b * p.dy_sb + k.d0 * p.dy_sd;
  const TIn* Cb = static_cast<const TIn*>(p.C) + k.b * p.C_sb + k.g * p.C_sg;
  const int64_t cb = (int64_t)j * sg.cps, ce = std::min<int64_t>(nch, cb + sg.cps);
  const int pp = tid >> 2, tt = 8 * (tid & 3);   // dy row and steps; C rows pp and pp + 64
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lg = 0.f;   // log2 decay from the segment's start to the chunk's (wave 0)
  float py[8], pc0[8], pc1[8], pdl = 0.f;
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * kCT;
    load_seg<8>(yb + pp * p.dy_sd, t0 + tt, L, p.vec, py);
    if (pp < N) load_seg<8>(Cb + pp * p.C_sn, t0 + tt, L, p.vec, pc0);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pc0[e] = 0.f;
    }
    if (NP > 64 && pp + 64 < N) load_seg<8>(Cb + (pp + 64) * p.C_sn, t0 + tt, L, p.vec, pc1);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pc1[e] = 0.f;
    }
    if (wave == 0) pdl = (lane < kCT && t0 + lane < L) ? to_f32(dr[t0 + lane]) : 0.f;
  };
  fetch(cb);
  for (int64_t c = cb; c < ce; ++c) {
    const int64_t t0 = c * kCT;
    if (wave == 0) {
      const bool live = lane < kCT && t0 + lane < L;
      const float x = pdl + bias;
      const float dt = live ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      const float sc = scan32(dt * A2);
      if (lane < kCT) wts[lane] = __builtin_amdgcn_exp2f(lg + sc);
      lg += lane_f(sc, kCT - 1);
    }
    *reinterpret_cast<f32x4*>(dyt + pp * kST + tt) = f32x4{py[0], py[1], py[2], py[3]};
    *reinterpret_cast<f32x4*>(dyt + pp * kST + tt + 4) = f32x4{py[4], py[5], py[6], py[7]};
    if (pp < NP) {
      *reinterpret_cast<f32x4*>(cnt + pp * kST + tt) = f32x4{pc0[0], pc0[1], pc0[2], pc0[3]};
      *reinterpret_cast<f32x4*>(cnt + pp * kST + tt + 4) = f32x4{pc0[4], pc0[5], pc0[6], pc0[7]};
    }
    if (NP > 64 && pp + 64 < NP) {
      *reinterpret_cast<f32x4*>(cnt + (pp + 64) * kST + tt) = f32x4{pc1[0], pc1[1], pc1[2], pc1[3]};
      *reinterpret_cast<f32x4*>(cnt + (pp + 64) * kST + tt + 4) = f32x4{pc1[4], pc1[5], pc1[6], pc1[7]};
    }
    __syncthreads();
    if (c + 1 < ce) fetch(c + 1);
    if constexpr (B3) mm3<kCT, NT, false, true, true>(dyt + 16 * wave * kST, kST, cnt, kST, 16 * kST, lane, acc, wts);
    else mm<kCT, NT, true>(dyt + 16 * wave * kST, kST, cnt, kST, 16 * kST, lane, acc, wts);
    __syncthreads();
  }
  float* out = segw + (rowi * sg.nseg + j) * seg_floats<NP>();
  const int q = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(16 * wave + 4 * q + r) * NP + 16 * t + l16] = acc[t][r];
  if (tid == 0) out[kCP * NP] = lg;
}

// Pass 2: the chunks in reverse, 8 waves (two per SIMD, so that one wave's LDS and MFMA waits
// are covered by the other's work).  Tiles per wave w: DX and C B^T (w < 4: rows 16 (w / 2),
// columns 16 (w % 2)); [T x N] products dY H0, X R, dC, dB (rows 16 (w % 2), state tiles
// from NB (w / 2)); dX (rows 16 (w % 2), channels 16 (w / 2)); R (channels 16 (w % 4), state
// tiles from NR (w / 4)).
constexpr int kThrB = 512;
template <typename TIn, typename TDy, int NT>
__global__ __launch_bounds__(kThrB) void ssdb_main_kernel(BwdArgs p, int64_t nch, const float* __restrict__ ws,
                                                          const float* __restrict__ cbws, SegsB sg,
                                                          const float* __restrict__ segw) {
  constexpr int NP = 16 * NT;
  constexpr int NB = NT >= 4 ? NT / 4 : 1;   // [T x N] state tiles per wave
  constexpr int NR = NT / 2;                 // R state tiles per wave
  // bf16 inputs: the products on the bf16 matrix cores (mm3: split f32 operands), else fp32 MFMA
  constexpr bool B3 = std::is_same<TIn, bf16_t>::value;
  __shared__ __attribute__((aligned(16))) float xn[kCT * kSP];    // u [t][p]
  __shared__ __attribute__((aligned(16))) float dyn[kCT * kSP];   // dy [t][p]
  __shared__ __attribute__((aligned(16))) float dyt[kCP * kST];   // dy [p][t]
  __shared__ __attribute__((aligned(16))) float bnt[NP * kST];    // B [n][t]
  __shared__ __attribute__((aligned(16))) float cnt[NP * kST];    // C [n][t]
  __shared__ __attribute__((aligned(16))) float rnp[NP * kSP];    // R [n][p]
  __shared__ __attribute__((aligned(16))) float hnp[NP * kCP];    // H0 [n][p], swizzled (copied straight from pass 1)
  __shared__ __attribute__((aligned(16))) float m1[kCT * kST];    // M1 [k][j]
  __shared__ __attribute__((aligned(16))) float m1t[kCT * kST];   // M1^T [j][k]
  __shared__ __attribute__((aligned(16))) float lcbt[kCT * kST];  // (L o CB)^T [j][k]
  __shared__ __attribute__((aligned(16))) float ses[kCT];         // e^{s_t}
  __shared__ __attribute__((aligned(16))) float sdt[kCT];
  __shared__ float ss2[kCT], ser[kCT], ssig[kCT];
  __shared__ float alp[4][kCT], bet[4][kCT], udp[4][kCT], rowp[2][kCT], colp[2][kCT], rh0[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  // block = segment * rows + (batch, head, slab) row; the segment's chunks [cbeg, cend)
  const int64_t nrow = p.batch * p.heads * (p.chan_per_head / kCP);
  const int64_t rowi = blockIdx.x % nrow, sgi = blockIdx.x / nrow;
  const int64_t cbeg = sgi * sg.cps, cend = std::min<int64_t>(nch, cbeg + sg.cps);
  const Blk k = block_of(p, rowi);
  const int N = p.N;
  const int64_t L = p.L;
  const float Ah = p.A[k.h], A2 = Ah * kLog2e;
  const float bias = p.bias ? p.bias[k.h] : 0.f;
  const int slabs = p.chan_per_head / kCP;
  const TIn* dr = static_cast<const TIn*>(p.delta) + k.b * p.dl_sb + k.h * p.dl_sh;
  const TIn* ub = static_cast<const TIn*>(p.u) + k.b * p.u_sb + k.d0 * p.u_sd;
  const TDy* yb = static_cast<const TDy*>(p.dy) + k.b * p.dy_sb + k.d0 * p.dy_sd;
  const TIn* Bb = static_cast<const TIn*>(p.B) + k.b * p.B_sb + k.g * p.B_sg;
  const TIn* Cb = static_cast<const TIn*>(p.C) + k.b * p.C_sb + k.g * p.C_sg;
  float* dBb = p.dB + k.b * p.dB_sb + k.g * p.dB_sg;
  float* dCb = p.dC + k.b * p.dC_sb + k.g * p.dC_sg;
  float* dub = p.du + k.b * p.du_sb + k.d0 * p.du_sd;
  float* ddb = p.ddelta + k.b * p.dd_sb + k.h * p.dd_sh;
  const float* wsb = ws + rowi * nch * NP * kCP;
  const float* cbg = cbws + (k.b * p.groups + k.g) * nch * 1024;
  const int w2 = wave & 1, wg = wave >> 1;      // row block of 16 steps, and a group of four
  const bool dxw = wave < 4;                    // the waves forming DX and C B^T
  const bool bcw = NT >= 4 || wave < 4;         // the waves with [T x N] tiles
  const int nb0 = wg * NB;                      // first [T x N] state tile
  const int rpi = wave & 3, nr0 = (wave >> 2) * NR;   // R: channel tile, first state tile
  // H0 of chunk c into hnp: NP / 4 copies of 1 KB, shared out over the waves
  auto h0_copy = [&](int64_t c) {
    const float* hc = wsb + c * NP * kCP;
    for (int i = wave; i < NP / 4; i += 8) dma16(hc + i * 256 + 4 * lane, hnp + i * 256);
  };
  h0_copy(cend - 1);
  // this thread's share of a chunk's loads, fetched one chunk ahead: u and dy (threads < 256: row
  // pp, 8 steps from tt), B and C (row bn, 8 steps from bt8), the raw step (wave 0)
  const int pp = (tid & 255) >> 2, tt = 8 * (tid & 3);
  const bool uth = tid < 256;
  const int bn = tid >> 2, bt8 = 8 * (tid & 3);
  const bool bth = bn < NP;
  float pu[8], py[8], pb[8], pc[8], pdl = 0.f;
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * kCT;
    if (uth) {
      load_seg<8>(ub + pp * p.u_sd, t0 + tt, L, p.vec, pu);
      load_seg<8>(yb + pp * p.dy_sd, t0 + tt, L, p.vec, py);
    }
    if (bth && bn < N) {
      load_seg<8>(Bb + bn * p.B_sn, t0 + bt8, L, p.vec, pb);
      load_seg<8>(Cb + bn * p.C_sn, t0 + bt8, L, p.vec, pc);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = pc[e] = 0.f;
    }
    if (wave == 0) pdl = (lane < kCT && t0 + lane < L) ? to_f32(dr[t0 + lane]) : 0.f;
  };
  fetch(cend - 1);
  // D of the channel this lane's dX tile covers
  const int pch = 16 * wg + l16;
  const float Dp = p.D ? p.D[p.d_per_head ? k.h : k.d0 + pch] : 0.f;
  f32x4 R[NR];   // R[p = 16 rpi + 4 q + r][n = 16 (nr0 + j) + l16]
#pragma unroll
  for (int j = 0; j < NR; ++j) R[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the R entering the segment from the right: R(k) = D_{k+1} R(k+1) + L_{k+1}
  for (int64_t jj = sg.nseg - 1; jj > sgi; --jj) {
    const float* sj = segw + (rowi * sg.nseg + jj) * seg_floats<NP>();
    const float dj = __builtin_amdgcn_exp2f(sj[kCP * NP]);
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        R[j][r] = fmaf(dj, R[j][r], sj[(16 * rpi + 4 * q + r) * NP + 16 * (nr0 + j) + l16]);
  }
  float dDl = 0.f;
  float dAacc = 0.f, dbacc = 0.f;

  for (int64_t c = cend - 1; c >= cbeg; --c) {
    const int64_t t0 = c * kCT;
    // ---- staging (from the registers fetched during the previous chunk)
    if (wave == 0) {
      const bool live = lane < kCT && t0 + lane < L;
      const float x = pdl + bias;
      const float dt = live ? (p.softplus ? softplus_fast(x) : x) : 0.f;
      const float sg = live ? (p.softplus ? __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e)) : 1.f) : 0.f;
      const float s = scan32(dt * A2);
      const float send = lane_f(s, kCT - 1);
      if (lane < kCT) {
        ss2[lane] = s;
        sdt[lane] = dt;
        ssig[lane] = sg;
        ses[lane] = __builtin_amdgcn_exp2f(s);
        ser[lane] = __builtin_amdgcn_exp2f(send - s);
      }
    }
    if (uth) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xn[(tt + e) * kSP + pp] = pu[e];
        dyn[(tt + e) * kSP + pp] = py[e];
      }
      *reinterpret_cast<f32x4*>(dyt + pp * kST + tt) = f32x4{py[0], py[1], py[2], py[3]};
      *reinterpret_cast<f32x4*>(dyt + pp * kST + tt + 4) = f32x4{py[4], py[5], py[6], py[7]};
    }
    if (bth) {
      *reinterpret_cast<f32x4*>(bnt + bn * kST + bt8) = f32x4{pb[0], pb[1], pb[2], pb[3]};
      *reinterpret_cast<f32x4*>(bnt + bn * kST + bt8 + 4) = f32x4{pb[4], pb[5], pb[6], pb[7]};
      *reinterpret_cast<f32x4*>(cnt + bn * kST + bt8) = f32x4{pc[0], pc[1], pc[2], pc[3]};
      *reinterpret_cast<f32x4*>(cnt + bn * kST + bt8 + 4) = f32x4{pc[4], pc[5], pc[6], pc[7]};
    }
    // R (the carry from the right) into LDS
#pragma unroll
    for (int j = 0; j < NR; ++j)
      *reinterpret_cast<f32x4*>(rnp + (16 * (nr0 + j) + l16) * kSP + 16 * rpi + 4 * q) = R[j];
    // this wave's tile of C B^T (formed by pass 1)
    f32x4 cb = f32x4{0.f, 0.f, 0.f, 0.f};
    if (dxw) cb = *reinterpret_cast<const f32x4*>(cbg + c * 1024 + (wave * 64 + lane) * 4);
    // the copies of H0 into hnp have landed (this wave's), then everyone's
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- DX = dY X^T and CB = C B^T (waves 0..3: rows 16 (w / 2), columns 16 (w % 2)), then the
    // masked matrices
    if (dxw) {
      const int ti = wave >> 1, half = wave & 1;
      f32x4 dx[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (B3) mm3<kCP, 1, false, true>(dyn + 16 * ti * kSP, kSP, xn + 16 * half * kSP, kSP, 0, lane, dx);
      else mm<kCP, 1>(dyn + 16 * ti * kSP, kSP, xn + 16 * half * kSP, kSP, 0, lane, dx);
      const int s = 16 * half + l16;   // column j = s of this lane; rows k = t below
      const float dts = sdt[s];
      float csum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * ti + 4 * q + r;
        const float e = t >= s ? __builtin_amdgcn_exp2f(ss2[t] - ss2[s]) : 0.f;
        const float mv = e * dx[0][r] * dts;   // X = diag(dt) U
        m1[t * kST + s] = mv;
        m1t[s * kST + t] = mv;
        lcbt[s * kST + t] = e * cb[r];
        // W = M1 o CB: this tile's part of row t's and column s's sums
        const float wv = mv * cb[r];
        csum += wv;
        const float rs = row16_sum(wv);
        if (l16 == 0) rowp[half][t] = rs;
      }
      csum += __shfl_xor(csum, 16);
      csum += __shfl_xor(csum, 32);
      if (q == 0) colp[ti][s] = csum;
    }
    // ---- dY H0 and X R, as transposed [N x T] tiles (state tiles nb0 .., steps 16 w2 ..): lane l
    // holds step 16 w2 + l % 16 and states 16 (nb0 + j) + 4 (l / 16) + r, so that the sums into dB
    // and dC below run along time (16 consecutive steps per row of lanes)
    f32x4 yh[NB], xr[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) yh[j] = xr[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tw = 16 * w2 + l16;   // this lane's step within the chunk
    if (bcw) {
      if constexpr (B3) {
        mm3_swz<NB, true>(dyn + 16 * w2 * kSP, kSP, hnp + 16 * nb0 * kCP, lane, yh);
        mm3<kCP, NB, true, false, false, true>(xn + 16 * w2 * kSP, kSP, rnp + 16 * nb0 * kSP, kSP, 16 * kSP, lane, xr);
      } else {
        mm_swz<NB, true>(dyn + 16 * w2 * kSP, kSP, hnp + 16 * nb0 * kCP, lane, yh);
        mm<kCP, NB, false, true>(xn + 16 * w2 * kSP, kSP, rnp + 16 * nb0 * kSP, kSP, 16 * kSP, lane, xr);
      }
      const float dtw = sdt[tw];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) xr[j][r] *= dtw;   // X R = diag(dt) U R
      // alpha_t = e^{s_t} (dY H0)_t . C_t and beta_t = e^{s_{T-1} - s_t} (X R)_t . B_t, partial over
      // this wave's state tiles: a lane's own states, then the four rows of lanes
      float a = 0.f, bsum = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * (nb0 + j) + 4 * q + r;
          a = fmaf(yh[j][r], cnt[n * kST + tw], a);
          bsum = fmaf(xr[j][r], bnt[n * kST + tw], bsum);
        }
      a += __shfl_xor(a, 16);
      bsum += __shfl_xor(bsum, 16);
      a += __shfl_xor(a, 32);
      bsum += __shfl_xor(bsum, 32);
      if (q == 0) {
        alp[wg][tw] = a * ses[tw];
        bet[wg][tw] = bsum * ser[tw];
      }
    } else {
      if (lane < kCT) alp[wg][lane] = bet[wg][lane] = 0.f;
    }
    {
      // <R, H0> over this wave's tiles of R
      float rh = 0.f;
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const f32x4 hv = *reinterpret_cast<const f32x4*>(hnp + swz(16 * (nr0 + j) + l16, 4 * rpi + q));
        rh = fmaf(R[j][0], hv[0], fmaf(R[j][1], hv[1], fmaf(R[j][2], hv[2], fmaf(R[j][3], hv[3], rh))));
      }
      rh = wave_total(rh);
      if (lane == 0) rh0[wave] = rh;
    }
    __syncthreads();   // m1, m1t, lcbt, row and column sums, alp, bet, rh0 ready; hnp no longer read
    if (c > cbeg) {
      h0_copy(c - 1);   // lands while this chunk's second half runs
      fetch(c - 1);
    }

    // ---- dC = diag(e^s) dY H0 + M1 B and dB = diag(e^{s_{T-1} - s}) X R + M1^T C, added to the group's
    if (bcw) {
      const float esw = ses[tw], erw = ser[tw];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          yh[j][r] *= esw;
          xr[j][r] *= erw;
        }
      if constexpr (B3) {
        mm3<kCT, NB, false, true, false, true>(m1 + 16 * w2 * kST, kST, bnt + 16 * nb0 * kST, kST, 16 * kST, lane, yh);
        mm3<kCT, NB, false, true, false, true>(m1t + 16 * w2 * kST, kST, cnt + 16 * nb0 * kST, kST, 16 * kST, lane, xr);
      } else {
        mm<kCT, NB, false, true>(m1 + 16 * w2 * kST, kST, bnt + 16 * nb0 * kST, kST, 16 * kST, lane, yh);
        mm<kCT, NB, false, true>(m1t + 16 * w2 * kST, kST, cnt + 16 * nb0 * kST, kST, 16 * kST, lane, xr);
      }
      const int64_t t = t0 + tw;
      if (t < L) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = 16 * (nb0 + j) + 4 * q + r;
            if (n < N) {
              atomicAdd(dCb + n * p.dC_sn + t, yh[j][r]);
              atomicAdd(dBb + n * p.dB_sn + t, xr[j][r]);
            }
          }
      }
    }

    // ---- dX = diag(e^{s_{T-1} - s}) B R^T + (L o CB)^T dY (rows 16 w2, channels 16 wg)
    {
      f32x4 dxa[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
      if constexpr (B3) {
        // B R^T over n, 32 states at a time (B exact in bf16, R split)
#pragma unroll
        for (int kb = 0; kb < NT / 2; ++kb) {
          float oa[8], ob[8];
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int n = 32 * kb + 8 * q + m;
            oa[m] = bnt[n * kST + 16 * w2 + l16];
            ob[m] = rnp[n * kSP + pch];
          }
          dxa[0] = mma3<true, false, false>(split8<true>(oa), split8<false>(ob), dxa[0]);
        }
      } else {
        // B R^T over n: the operands of block kb + 1 are read while block kb's products run
        float oa[2][4], ob[2][4];
        auto rd = [&](int kb, int s) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int n = 16 * kb + 4 * q + m;
            oa[s][m] = bnt[n * kST + 16 * w2 + l16];
            ob[s][m] = rnp[n * kSP + pch];
          }
        };
        rd(0, 0);
#pragma unroll
        for (int kb = 0; kb < NT; ++kb) {
          if (kb + 1 < NT) rd(kb + 1, (kb + 1) & 1);
#pragma unroll
          for (int m = 0; m < 4; ++m) dxa[0] = mma4(oa[kb & 1][m], ob[kb & 1][m], dxa[0]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) dxa[0][r] *= ser[16 * w2 + 4 * q + r];
      if constexpr (B3) mm3<kCT, 1, false, false>(lcbt + 16 * w2 * kST, kST, dyt + 16 * wg * kST, kST, 0, lane, dxa);
      else mm<kCT, 1>(lcbt + 16 * w2 * kST, kST, dyt + 16 * wg * kST, kST, 0, lane, dxa);
      // du = dt dX + D dy; u . dX per step; dD
      // (the lane's 4 steps of a channel are consecutive: one 16-byte store when whole and aligned)
      const int tl0 = 16 * w2 + 4 * q;
      const f32x4 dt4 = *reinterpret_cast<const f32x4*>(sdt + tl0);
      float* dst = dub + pch * p.du_sd + t0 + tl0;
      const f32x4 dy4 = *reinterpret_cast<const f32x4*>(dyt + pch * kST + tl0);
      f32x4 du4;
      float ud[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool live = t0 + tl0 + r < L;
        const float uv = live ? xn[(tl0 + r) * kSP + pch] : 0.f;
        du4[r] = fmaf(dt4[r], dxa[0][r], Dp * dy4[r]);
        ud[r] = uv * dxa[0][r];
        dDl = fmaf(dy4[r], uv, dDl);
      }
      if (t0 + tl0 + 4 <= L && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<f32x4*>(dst) = du4;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + tl0 + r < L) dst[r] = du4[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = row16_sum(ud[r]);
        if (l16 == 0) udp[wg][tl0 + r] = v;
      }
    }

    // ---- R <- e^{s_{T-1}} R + dY^T diag(e^s) C
    {
      const float dec = __builtin_amdgcn_exp2f(ss2[kCT - 1]);
#pragma unroll
      for (int j = 0; j < NR; ++j) R[j] = R[j] * dec;
      if constexpr (B3)
        mm3<kCT, NR, false, true, true>(dyt + 16 * rpi * kST, kST, cnt + 16 * nr0 * kST, kST, 16 * kST, lane, R, ses);
      else
        mm<kCT, NR, true>(dyt + 16 * rpi * kST, kST, cnt + 16 * nr0 * kST, kST, 16 * kST, lane, R, ses);
    }

    // ---- the decay's gradient per step (wave 0; lane j = step j; scans over the 32 steps)
    __syncthreads();   // udp ready
    if (wave == 0) {
      const int j = lane & (kCT - 1);
      const bool lo = lane < kCT;
      // inclusive prefix sums over lanes 0..31 (lanes 32..63 repeat them and are ignored)
      const float col = colp[0][j] + colp[1][j], row = rowp[0][j] + rowp[1][j];
      const float al = (alp[0][j] + alp[1][j]) + (alp[2][j] + alp[3][j]);
      const float be = (bet[0][j] + bet[1][j]) + (bet[2][j] + bet[3][j]);
      const float pcol = scan32(col), prow = scan32(row), pal = scan32(al), pbe = scan32(be);
      const float altot = lane_f(pal, kCT - 1);
      const float t1 = pcol - (prow - row);     // sum over k >= j >= i of W_ki
      const float t2 = altot - (pal - al);      // sum over k >= j of alpha_k
      const float t3 = pbe;                     // sum over i <= j of beta_i
      const float rhs = ((rh0[0] + rh0[1]) + (rh0[2] + rh0[3])) + ((rh0[4] + rh0[5]) + (rh0[6] + rh0[7]));
      const float t4 = __builtin_amdgcn_exp2f(ss2[kCT - 1]) * rhs;
      const float gh = t1 + t2 + t3 + t4;
      const float ud = (udp[0][j] + udp[1][j]) + (udp[2][j] + udp[3][j]);
      const float dt = sdt[j];
      const float qa = gh - dt * ud;                 // a_j dLoss/da_j
      const float ddt = fmaf(Ah, qa, ud);
      const float dx = ddt * ssig[j];
      if (lo && t0 + j < L) {
        if (slabs == 1) ddb[t0 + j] = dx;
        else atomicAdd(ddb + t0 + j, dx);
        dAacc = fmaf(dt, qa, dAacc);
        dbacc += dx;
      }
    }
    __syncthreads();   // every LDS buffer is restaged by the next chunk
  }

  // per-head and per-channel sums
  if (wave == 0) {
    const float dA = wave_total(dAacc), db = wave_total(dbacc);
    if (lane == 0) {
      atomicAdd(p.dA + k.h, dA);
      if (p.dbias) atomicAdd(p.dbias + k.h, db);
    }
  }
  if (p.dD) {
    float v = dDl;
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (p.d_per_head) {
      v = row16_sum(v);
      if (lane == 0) atomicAdd(p.dD + k.h, v);
    } else if (q == 0) {
      atomicAdd(p.dD + k.d0 + pch, v);
    }
  }
}

template <typename TIn, typename TDy, int NT>
hipError_t launch_nt(const BwdArgs& a, float* ws, hipStream_t s) {
  const int64_t nch = (a.L + kCT - 1) / kCT;
  const dim3 grid((unsigned)(a.batch * a.heads * (a.chan_per_head / kCP))), block(kThr);
  float* cbws = ws + a.batch * a.heads * (a.chan_per_head / kCP) * nch * (16 * NT) * kCP;
  hipLaunchKernelGGL((ssdb_state_kernel<TIn, NT>), dim3(kStateSplit<NT> * grid.x), block, 0, s, a, nch, ws, cbws);
  // sequence segments of pass 2: the pre-pass's results follow the C B^T records
  const SegsB sg = ssdb_seg_plan(a);
  float* segw = cbws + a.batch * a.groups * nch * 1024;
  if (sg.nseg > 1)
    hipLaunchKernelGGL((ssdb_seg_kernel<TIn, TDy, NT>), dim3((unsigned)(grid.x * (sg.nseg - 1))), block, 0, s, a, nch,
                       sg, segw);
  hipLaunchKernelGGL((ssdb_main_kernel<TIn, TDy, NT>), dim3((unsigned)(grid.x * sg.nseg)), dim3(kThrB), 0, s, a,
                     nch, static_cast<const float*>(ws), static_cast<const float*>(cbws), sg,
                     static_cast<const float*>(segw));
  return hipGetLastError();
}

template <typename TIn, typename TDy>
hipError_t launch_t(const BwdArgs& a, float* ws, hipStream_t s) {
  if (a.N <= 32) return launch_nt<TIn, TDy, 2>(a, ws, s);
  if (a.N <= 64) return launch_nt<TIn, TDy, 4>(a, ws, s);
  return launch_nt<TIn, TDy, 8>(a, ws, s);
}

}  // namespace

bool ssd_bwd_path(const BwdArgs& a) {
  return a.scalar && !a.z && a.chan_per_head % kCP == 0 && a.chan_per_group % kCP == 0 && a.N <= 128 && a.L > 0;
}

int64_t ssd_bwd_workspace_floats(const BwdArgs& a) {
  const int64_t np = a.N <= 32 ? 32 : a.N <= 64 ? 64 : 128;
  const int64_t nch = (a.L + kCT - 1) / kCT;
  // chunk states, then C B^T of every (batch, group, chunk), then (with sequence segments) the
  // pre-pass's [64][np] + 1 floats per (row, segment)
  const int64_t rows = a.batch * a.heads * (a.chan_per_head / kCP);
  const SegsB sg = ssdb_seg_plan(a);
  return rows * nch * np * kCP + a.batch * a.groups * nch * 1024 +
         (sg.nseg > 1 ? rows * sg.nseg * (kCP * np + 1) : 0);
}

hipError_t launch_ssd_bwd(const BwdArgs& a, float* ws, hipStream_t s) {
  if (a.in_bf16) return a.dy_bf16 ? launch_t<bf16_t, bf16_t>(a, ws, s) : launch_t<bf16_t, float>(a, ws, s);
  return a.dy_bf16 ? launch_t<float, bf16_t>(a, ws, s) : launch_t<float, float>(a, ws, s);
}

}  // namespace ss
