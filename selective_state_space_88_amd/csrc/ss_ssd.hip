// ss_ssd.hip -- scalar-decay selective scan in its chunked matrix form, on MFMA (gfx950).
//
// Method.  With one scalar decay per head, a_t = exp(dt_t A_h) (bqwf.cn state-space survey,
// section 3.2; omica.com.cn Mamba explainer, section 6.2), the recurrence over a chunk of T
// steps is a masked matrix product.  With S_t = sum_{r <= t} log2(a_r) inside the chunk and
// H the state entering it ([N, P] for the head's P channels):
//   y_t  = sum_{s <= t} 2^(S_t - S_s) (C_t . B_s) dt_s u_s  +  2^(S_t) C_t H  +  D u_t
//   H'   = 2^(S_{T-1}) H  +  sum_s 2^(S_{T-1} - S_s) B_s (dt_s u_s)
// (expanding h_t = a_t h_{t-1} + dt_t B_t u_t from the chunk's start: the mask matrix of the
// explainer's section 6.2 and the survey's block decomposition).  Per chunk that is
//   Y = (G o L) X  +  diag(2^S) C H,     H' = 2^(S_{T-1}) H + B^T Xd,
// G = C B^T [T, T], L the decay mask, X = dt u [T, P], Xd = X scaled by 2^(S_{T-1} - S_s):
// three dense contractions, done here with v_mfma_f32_16x16x32_bf16.
//
// Precision: B, C and u are bf16 inputs, exact as MFMA operands.  The f32 operands (G o L, X,
// Xd, H) are split as x = hi + lo with hi = bf16(x), lo = bf16(x - hi), and the products take
// hi*hi + hi*lo + lo*hi (or hi + lo against an exact operand): relative error ~2^-16 per
// product with f32 accumulation, and bf16's exponent range (nothing overflows that would not
// overflow in f32).
//
// Mapping.  A pre-pass computes, per (batch, group, chunk), G (causally masked) in f32 and
// copies of C and B (bf16, n padded to a multiple of 32 with zeros) into one record, each
// operand stored in the order the MFMA lanes consume it.
// The scan gives each block one (batch, head, 64-channel slab) and walks the chunks in order;
// wave w owns channels 16w..16w+15 of the slab and keeps their state H (N x 16) in MFMA
// accumulators across chunks.  MFMA 16x16x32 operand layout (checked on the device): lane l
// holds A[l % 16][8 (l / 16) + k], B[8 (l / 16) + k][l % 16] (k = 0..7), and
// D[4 (l / 16) + r][l % 16] (r = 0..3).  C H takes H straight from the accumulators: the
// contraction index n is permuted so that lane group g's eight K slots are the n it holds
// (4g..4g+3 of two consecutive 16-row tiles), and C is read in the same order.
#include <algorithm>
#include <atomic>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kT = 32;          // steps per chunk
constexpr int kSlab = 64;       // channels per block
constexpr int kWaves = 4;       // one per 16 channels

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

int npad32(int N) { return (N + 31) / 32 * 32; }
int64_t nchunks_of(const ScanArgs& a) { return (a.L + kT - 1) / kT; }
// bytes of one chunk record: G [T][T] f32, C [T][Np] bf16, B [Np][T] bf16
__host__ __device__ inline int64_t rec_bytes(int Np) { return (int64_t)kT * kT * 4 + 2LL * kT * Np * 2; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }


// x = hi + lo, both bf16 (round to nearest even), for eight values; the conversions go in
// pairs (converting the elements one by one takes one instruction each)
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = pk_bf16(x[2 * j], x[2 * j + 1]);
    l[j] = pk_bf16(x[2 * j] - __uint_as_float(h[j] << 16), x[2 * j + 1] - __uint_as_float(h[j] & 0xffff0000u));
  }
  hi = as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
  lo = as_bf16x8(u32x4{l[0], l[1], l[2], l[3]});
}

// DPP move of v with control CTRL on the rows in ROWMASK; lanes with no source, and lanes of
// masked rows, read 0
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, true));
}

__device__ __forceinline__ f32x4v mfma(bf16x8 a, bf16x8 b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pre-pass: one block per (batch, group, chunk).
template <typename TIn>
__global__ __launch_bounds__(256) void ssd_prep_kernel(ScanArgs p, uint8_t* __restrict__ ws, int Np,
                                                       int64_t nchunks) {
  __shared__ float sB[128][kT + 1], sC[128][kT + 1];
  const int64_t bgc = blockIdx.x;
  const int64_t c = bgc % nchunks, bg = bgc / nchunks;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t t0 = c * kT;
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  for (int i = threadIdx.x; i < Np * kT; i += 256) {
    const int n = i / kT, t = i % kT;
    const bool in = n < p.N && t0 + t < p.L;
    sB[n][t] = in ? to_f32(Bg[n * p.B_sn + t0 + t]) : 0.f;
    sC[n][t] = in ? to_f32(Cg[n * p.C_sn + t0 + t]) : 0.f;
  }
  __syncthreads();
  // G[t][s] = sum_n C[t][n] B[s][n] on the matrix cores (products of bf16 values are exact in
  // f32): wave w computes the 16 x 16 tile (t-tile w / 2, s-tile w % 2), its operands the staged
  // values' top 16 bits (each a bf16 held exactly in f32)
  __shared__ float sG[kT][kT + 1];
  {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int ti = w >> 1, si = w & 1, g = l >> 4, r16 = l & 15;
    f32x4v acc = f32x4v{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < Np / 32; ++ks) {
      uint32_t a[4], bb[4];
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int n0 = 32 * ks + 8 * g + 2 * k2;
        a[k2] = (__float_as_uint(sC[n0][16 * ti + r16]) >> 16) | (__float_as_uint(sC[n0 + 1][16 * ti + r16]) & 0xffff0000u);
        bb[k2] = (__float_as_uint(sB[n0][16 * si + r16]) >> 16) | (__float_as_uint(sB[n0 + 1][16 * si + r16]) & 0xffff0000u);
      }
      acc = mfma(as_bf16x8(u32x4{a[0], a[1], a[2], a[3]}), as_bf16x8(u32x4{bb[0], bb[1], bb[2], bb[3]}), acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sG[16 * ti + 4 * g + r][16 * si + r16] = acc[r];
  }
  __syncthreads();
  // the record holds every operand in the order the scan's MFMA lanes read it (lane l =
  // 16 g + q holds row q, K slots 8 g .. 8 g + 7), so that each wave reads it as contiguous
  // 16-byte pieces with no LDS bank conflicts
  uint8_t* rec = ws + bgc * rec_bytes(Np);
  // G [i][half][lane][4] f32: (G o causal)[t = 16 i + q][s = 8 g + 4 half + e]
  float* Gp = reinterpret_cast<float*>(rec);
  for (int i = threadIdx.x; i < kT * kT; i += 256) {
    const int e = i & 3, l = (i >> 2) & 63, half = (i >> 8) & 1, ti = i >> 9;
    const int t = 16 * ti + (l & 15), s = 8 * (l >> 4) + 4 * half + e;
    Gp[i] = s <= t ? sG[t][s] : 0.f;
  }
  // C [i][ks][lane][8] bf16: C[t = 16 i + q][n], with K slot e of lane group g holding
  // n = 32 ks + 4 g + (e % 4) + 16 (e / 4) (the order of the state accumulators' rows)
  uint16_t* Cp = reinterpret_cast<uint16_t*>(rec + kT * kT * 4);
  const int nks = Np / 32;
  for (int i = threadIdx.x; i < kT * Np; i += 256) {
    const int e = i & 7, l = (i >> 3) & 63, r = i >> 9;
    const int ks = r % nks, ti = r / nks;
    const int t = 16 * ti + (l & 15), n = 32 * ks + 4 * (l >> 4) + (e & 3) + 16 * (e >> 2);
    Cp[i] = (uint16_t)(__float_as_uint(sC[n][t]) >> 16);  // exact: the value is a bf16
  }
  // B [k][lane][8] bf16: B^T[n = 16 k + q][s = 8 g + e]
  uint16_t* Bp = Cp + kT * Np;
  for (int i = threadIdx.x; i < kT * Np; i += 256) {
    const int e = i & 7, l = (i >> 3) & 63, k = i >> 9;
    const int n = 16 * k + (l & 15), s = 8 * (l >> 4) + e;
    Bp[i] = (uint16_t)(__float_as_uint(sB[n][s]) >> 16);
  }
}

// Sequence segments: each (batch, head, slab) row is cut into nseg segments of cps chunks,
// one block each.  A state pass (STATE) runs the recurrence over every segment but the last
// from a zero state, with no output, and stores the segment's final state and its total
// log2 decay; the output pass starts segment k from the state the earlier segments hand
// over, H_in(k) = sum_{j<k} (product of the decays of segments j+1 .. k-1) H_end(j).
struct Segs {
  int64_t cps;          // chunks per segment
  int32_t nseg;         // segments per row
  float* hloc;          // per state-pass block: its wave-ordered final state (Np * 64 floats)
  float* dsum;          // per state-pass block: the log2 decay over its segment
};

// FULL: every chunk holds kT steps and every row is 16-byte aligned, so that the loop has no
// bounds checks (and the compiler can count the memory operations in flight exactly).
// STATE: the state pass (no y; only the B part of the record is staged).
//
// The loop is software-pipelined with one barrier per chunk.  While chunk c is computed from
// LDS buffer c % 2, chunk c + 1 (loaded into registers during chunk c - 1) is staged into the
// other buffer together with its step sizes and its masked matrix, and chunk c + 2 is loaded.
// What crosses waves (the C and B parts of the record, the masked matrix) is double-buffered;
// u, z, the G piece and the step sizes never leave the wave that loads them.
template <typename TOut, bool GATE, int NP, bool FULL, bool STATE>
__global__ __launch_bounds__(64 * kWaves) void ssd_scan_kernel(ScanArgs p, const uint8_t* __restrict__ ws,
                                                               int64_t nchunks, Segs sg) {
  using TIn = bf16_t;
  constexpr int Np = NP;    // states padded to a multiple of 32
  constexpr int nk = Np / 16;   // state tiles of 16
  constexpr int kGBytes = kT * kT * 4, kCBytes = kT * Np * 2, kBBytes = kT * Np * 2;
  // the record's part staged for all waves: C and B (output pass) or B (state pass)
  constexpr int kShOff = STATE ? kGBytes + kCBytes : kGBytes;
  constexpr int kShBytes = STATE ? kBBytes : kCBytes + kBBytes;
  constexpr int kShPieces = kShBytes / 16 / 256;   // 16-byte pieces per thread
  static_assert(kShBytes % (16 * 256) == 0, "record pieces");
  __shared__ __attribute__((aligned(16))) u32x4 sh[2][kShBytes / 16];
  // u (and z) of the slab's channels, in lane order: channel 16 w + q, steps 8 g .. 8 g + 7 at
  // [w][g][q][8], the B operand of wave w's lane 16 g + q (each wave reads only its own part)
  __shared__ __attribute__((aligned(16))) u32x4 su[64 * kWaves];
  __shared__ __attribute__((aligned(16))) u32x4 sz[GATE ? 64 * kWaves : 1];
  // per wave: the input coefficient k (dt, or (exp(dt A) - 1) / A with zero-order hold), S (log2
  // of the decay from the chunk's start), 2^S, k 2^(S_{T-1} - S)
  __shared__ __attribute__((aligned(16))) float sw[2][kWaves][4][kT];
  // the masked matrix of the chunk (the same for every channel of the head), split into bf16
  // hi and lo parts, as the A operand of t-tile i: [i][lane][8]; wave w computes the quarter
  // i = w / 2, K slots 4 (w % 2) .. 4 (w % 2) + 3
  __shared__ __attribute__((aligned(16))) u32x4 smh[2][STATE ? 1 : 2 * 64], sml[2][STATE ? 1 : 2 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g16 = lane >> 4, q = lane & 15;
  const int64_t L = p.L;
  const int64_t slabs = p.chan_per_head / kSlab;
  // block = ((segment * batch + b) * heads + h) * slabs + slab: neighbouring blocks share the
  // segment's chunk records
  const int64_t blk = blockIdx.x;
  const int64_t slab = blk % slabs;
  const int64_t h = (blk / slabs) % p.heads;
  const int64_t b = (blk / (slabs * p.heads)) % p.batch;
  const int64_t sgi = blk / (slabs * p.heads * p.batch);
  const int64_t row = (b * p.heads + h) * slabs + slab;   // (b, h, slab) index
  const int64_t rows = p.batch * p.heads * slabs;
  const int64_t cb = sgi * sg.cps, ce = (cb + sg.cps < nchunks) ? cb + sg.cps : nchunks;
  const int64_t c0 = h * p.chan_per_head + slab * kSlab;   // first channel of the slab
  const int64_t grp = c0 / p.chan_per_group;
  const float A2 = p.A[h] * kLog2e;
  const float bias = p.bias ? p.bias[h] : 0.f;
  const int64_t rb = rec_bytes(Np);
  const uint8_t* recs = ws + (b * p.groups + grp) * nchunks * rb;
  const TIn* drow = static_cast<const TIn*>(p.delta) + b * p.dl_sb + h * p.dl_sh;
  const int pch = 16 * wave + q;   // this lane's channel in the slab (B operand / D column)
  // with one D per head, D u_t is folded into the diagonal of the masked matrix (u is its
  // exact B operand); with one D per channel it is added to y.  (Read once here: inside the
  // loop the compiler would reload them after every y store.)
  const bool dfold = p.D && p.d_per_head;
  const float Dfold = dfold ? p.D[h] : 0.f;
  const float Dd = (p.D && !dfold) ? p.D[c0 + pch] : 0.f;
  TOut* const yr = static_cast<TOut*>(p.y) + b * p.y_sb + (c0 + pch) * p.y_sd;

  // this wave's state H[n][16w + q]: tile k holds rows 16k + 4 g16 + r
  f32x4v hacc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) hacc[k] = f32x4v{0.f, 0.f, 0.f, 0.f};
  // the first segment starts from the caller's state (later segments receive it through the
  // first segment's end state); the state pass adds it, decayed over the segment, at its end
  const float* const hinit = (sgi == 0 && p.h_init) ? p.h_init + b * p.hi_sb + (c0 + pch) * p.hi_sd : nullptr;
  if (!STATE && hinit) {
    const float* hi = hinit;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 16 * k + 4 * g16 + r;
        if (k < nk && n < p.N) hacc[k][r] = hi[n];
      }
  }
  if constexpr (!STATE) {
    // the state entering this segment, from the state pass's results (j = sgi - 1 first, whose
    // end state enters undecayed); segment j - 1's end state is loaded while segment j's is
    // added, so that the reads do not wait for each other one segment at a time
    auto hand = [&](int64_t j) {
      return reinterpret_cast<const f32x4v*>(sg.hloc) + ((j * rows + row) * kWaves + wave) * nk * 64 + lane;
    };
    f32x4v cur[8], nxt[8];
    if (sgi > 0) {
      const f32x4v* hl = hand(sgi - 1);
#pragma unroll
      for (int k = 0; k < 8; ++k) cur[k] = k < nk ? hl[k * 64] : f32x4v{0.f, 0.f, 0.f, 0.f};
    }
    float lg = 0.f;
    for (int64_t j = sgi - 1; j >= 0; --j) {
      if (j > 0) {
        const f32x4v* hl = hand(j - 1);
#pragma unroll
        for (int k = 0; k < 8; ++k) nxt[k] = k < nk ? hl[k * 64] : f32x4v{0.f, 0.f, 0.f, 0.f};
      }
      const float f = __builtin_amdgcn_exp2f(lg);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k < nk) hacc[k] += f * cur[k];
      lg += sg.dsum[j * rows + row];
#pragma unroll
      for (int k = 0; k < 8; ++k) cur[k] = nxt[k];
    }
  }
  // log2 decay over the chunks done so far.  The state pass walks its segment's chunks in
  // reverse, so that when a chunk is staged dlog is the decay from its end to the segment's
  // end: folded into the chunk's step weights (Xd), it makes the segment's end state the plain
  // sum of the chunks' B^T Xd, with no rescaling of the state per chunk.
  float dlog = 0.f;

  // registers holding the next chunk to stage
  // u / z piece of this thread: channel 16 (tid / 64) + tid % 16, steps 8 ((tid / 16) % 4) + 0..7
  const int pr = 16 * (tid >> 6) + (tid & 15), seg = 8 * ((tid >> 4) & 3);
  const TIn* ur = static_cast<const TIn*>(p.u) + b * p.u_sb + (c0 + pr) * p.u_sd;
  const TIn* zr = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + (c0 + pr) * p.z_sd : nullptr;
  u32x4 pf_sh[kShPieces], pf_g, pf_u, pf_z;
  uint32_t pf_d = 0u;   // raw bits of delta at step (lane % 32) of the chunk
  auto load_piece = [&](const TIn* rp, int64_t t) -> u32x4 {
    if (FULL || (p.vec && t + 8 <= L)) return *reinterpret_cast<const u32x4*>(rp + t);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (t + e < L) w[e / 2] |= (uint32_t)reinterpret_cast<const uint16_t*>(rp)[t + e] << (16 * (e % 2));
    return u32x4{w[0], w[1], w[2], w[3]};
  };
  auto prefetch = [&](int64_t c) {
    const uint8_t* rec = recs + c * rb;
    // the G piece this thread's quarter of the masked matrix needs is piece tid
    if constexpr (!STATE) pf_g = reinterpret_cast<const u32x4*>(rec)[tid];
#pragma unroll
    for (int m = 0; m < kShPieces; ++m) pf_sh[m] = reinterpret_cast<const u32x4*>(rec + kShOff)[tid + 256 * m];
    pf_u = load_piece(ur, c * kT + seg);
    if constexpr (GATE) pf_z = load_piece(zr, c * kT + seg);
    const int64_t t = c * kT + (lane & (kT - 1));
    pf_d = reinterpret_cast<const uint16_t*>(drow)[(FULL || t < L) ? t : 0];
  };

  // stage chunk c (from the registers) into buffer bf: the shared record part, this wave's
  // u / z, its step sizes and (output pass) its quarter of the masked matrix
  auto stage = [&](int64_t c, int bf) {
#pragma unroll
    for (int m = 0; m < kShPieces; ++m) sh[bf][tid + 256 * m] = pf_sh[m];
    su[tid] = pf_u;
    if constexpr (GATE) sz[tid] = pf_z;
    float* wdt = sw[bf][wave][0];
    float* wS = sw[bf][wave][1];
    // dt and S of the chunk, in lanes 0..31 of every wave (each wave keeps its own copy)
    {
      const int t = lane & (kT - 1);
      float dt = 0.f;
      if (lane < kT && (FULL || c * kT + t < L)) {
        const float x = __uint_as_float(pf_d << 16) + bias;
        dt = p.softplus ? softplus_fast(x) : x;
      }
      // inclusive prefix sum of dt * A * log2 e over lanes 0..31: DPP row_shr 1, 2, 4, 8
      // within rows of 16 (a source outside the row reads 0), then row 0's total added to
      // row 1 (row_bcast:15 on rows 1 and 3)
      float sc = dt * A2;
      sc += dpp_zero<0x111, 0xf>(sc);
      sc += dpp_zero<0x112, 0xf>(sc);
      sc += dpp_zero<0x114, 0xf>(sc);
      sc += dpp_zero<0x118, 0xf>(sc);
      sc += dpp_zero<0x142, 0xa>(sc);
      const float sEnd = readlane_f(sc, kT - 1);
      if (lane < kT) {
        // the input coefficient: dt, or with zero-order hold (exp(dt A) - 1) / A
        float kz = dt;
        if (p.zoh) {
          const float xz = dt * A2 * kLn2f;
          kz = dt * zoh_phi(xz, __builtin_amdgcn_exp2f(dt * A2), __builtin_amdgcn_rcpf(xz));
        }
        wdt[t] = kz;
        wS[t] = sc;
        sw[bf][wave][2][t] = __builtin_amdgcn_exp2f(sc);
        sw[bf][wave][3][t] = kz * __builtin_amdgcn_exp2f(sEnd - sc + (STATE ? dlog : 0.f));
      }
    }
    // this wave's quarter of the masked matrix (G o L)[t][s] dt_s (+ D on the diagonal), for
    // t = 16 iq + q, s = 8 g16 + 4 hq + e
    if constexpr (!STATE) {
      const int iq = wave >> 1, hq = wave & 1;
      const int t = 16 * iq + q;
      const float St = wS[t];
      const f32x4v Ssq = reinterpret_cast<const f32x4v*>(wS)[2 * g16 + hq];
      const f32x4v dtq = reinterpret_cast<const f32x4v*>(wdt)[2 * g16 + hq];
      const f32x4v gq = __builtin_bit_cast(f32x4v, pf_g);
      float m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 8 * g16 + 4 * hq + e;
        // (the record holds 0 above the diagonal; the exponent is masked there too, where it
        // may be large and positive)
        // (the trapezoidal rule reads y from h - e/2, i.e. halves the diagonal's input term)
        const float tw = (s == t && p.trap) ? 0.5f : 1.f;
        m[e] = tw * gq[e] * dtq[e] * __builtin_amdgcn_exp2f(s <= t ? St - Ssq[e] : -INFINITY) + (s == t ? Dfold : 0.f);
      }
      const uint32_t h0 = pk_bf16(m[0], m[1]), h1 = pk_bf16(m[2], m[3]);
      const uint32_t l0 = pk_bf16(m[0] - __uint_as_float(h0 << 16), m[1] - __uint_as_float(h0 & 0xffff0000u));
      const uint32_t l1 = pk_bf16(m[2] - __uint_as_float(h1 << 16), m[3] - __uint_as_float(h1 & 0xffff0000u));
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      reinterpret_cast<u32x2*>(smh[bf])[2 * (iq * 64 + lane) + hq] = u32x2{h0, h1};
      reinterpret_cast<u32x2*>(sml[bf])[2 * (iq * 64 + lane) + hq] = u32x2{l0, l1};
    }
  };

  // y of one chunk, t = 16 i + 4 g16 + r
  float yv[2][4];
  auto store_y = [&](int64_t tc) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t tg = tc + 16 * i + 4 * g16;
      const float* v = yv[i];
      if (FULL || (p.vec && tg + 4 <= L)) {
        if constexpr (sizeof(TOut) == 4) {
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(yr + tg));
        } else {
          typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
          __builtin_nontemporal_store(u32x2{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])},
                                      reinterpret_cast<u32x2*>(yr + tg));
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tg + r < L) store_one(yr + tg + r, v[r]);
      }
    }
  };

  // i-th chunk of the walk: in order (output pass), in reverse (state pass)
  const int64_t nc = ce - cb;
  auto chunk_at = [&](int64_t i) -> int64_t { return STATE ? ce - 1 - i : cb + i; };
  prefetch(chunk_at(0));
  stage(chunk_at(0), 0);
  prefetch(chunk_at(1 < nc ? 1 : 0));
  __syncthreads();
  for (int64_t i = 0; i < nc; ++i) {
    const int64_t c = chunk_at(i);
    const int bf = (int)(i & 1);
    const float* wS = sw[bf][wave][1];
    const float* weS = sw[bf][wave][2];
    const float* wXd = sw[bf][wave][3];
    const u32x4* Cp = sh[bf];                                // [i][ks][lane] (output pass)
    const u32x4* Bp = sh[bf] + (STATE ? 0 : kCBytes / 16);   // [k][lane]
    const float sEnd = wS[kT - 1];
    const float eT = __builtin_amdgcn_exp2f(sEnd);
    dlog += sEnd;

    // u[s = 8 g16 + k][pch]: the exact (bf16) B operand of the masked product; and
    // Xd[s][pch] = dt_s 2^(S_{T-1} - S_s) u_s, the B operand of the state update, split
    const u32x4 uw = su[tid];
    bf16x8 xdhi, xdlo;
    {
      const uint32_t uwv[4] = {uw.x, uw.y, uw.z, uw.w};
      const f32x4v xd0 = reinterpret_cast<const f32x4v*>(wXd)[2 * g16];
      const f32x4v xd1 = reinterpret_cast<const f32x4v*>(wXd)[2 * g16 + 1];
      float xd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        xd[k] = (k < 4 ? xd0[k] : xd1[k - 4]) * ((k & 1) ? bf16_hi(uwv[k / 2]) : bf16_lo(uwv[k / 2]));
      split8(xd, xdhi, xdlo);
    }

    if constexpr (!STATE) {
      // y tiles: t-tile i (rows 16 i + 4 g16 + r), this wave's 16 channels
      f32x4v yacc[2], iacc[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        yacc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
        iacc[i] = f32x4v{0.f, 0.f, 0.f, 0.f};
      }
      // within the chunk: the shared masked matrix (hi + lo) times u
      const bf16x8 ub = as_bf16x8(uw);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        yacc[i] = mfma(as_bf16x8(smh[bf][i * 64 + lane]), ub, yacc[i]);
        yacc[i] = mfma(as_bf16x8(sml[bf][i * 64 + lane]), ub, yacc[i]);
      }
      // from the carried state: C[t][n] H[n][pch], n in steps of 32 in the accumulators' order
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (2 * ks < nk) {
          float hv[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hv[r] = hacc[2 * ks][r];
            hv[4 + r] = hacc[2 * ks + 1][r];
          }
          bf16x8 hhi, hlo;
          split8(hv, hhi, hlo);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const bf16x8 ca = as_bf16x8(Cp[(i * (Np / 32) + ks) * 64 + lane]);
            iacc[i] = mfma(ca, hhi, iacc[i]);
            iacc[i] = mfma(ca, hlo, iacc[i]);
          }
        }
      }
      // y = within + 2^S_t (C H) + D u, gated; lane holds t = 16 i + 4 g16 + r of channel pch
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // u (and z) at steps 16 i + 4 g16 + 0..3 of channel pch: four bf16 of one lane-order piece
        const int uo = ((4 * wave + 2 * i + (g16 >> 1)) * 16 + q) * 8 + 4 * (g16 & 1);
        const uint2 uq = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(su) + uo);
        uint2 zq = uint2{0u, 0u};
        if constexpr (GATE) zq = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(sz) + uo);
        const uint32_t uwq[2] = {uq.x, uq.y}, zw[2] = {zq.x, zq.y};
        const f32x4v eS = reinterpret_cast<const f32x4v*>(weS)[4 * i + g16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float uu = (r & 1) ? bf16_hi(uwq[r / 2]) : bf16_lo(uwq[r / 2]);
          float yy = yacc[i][r] + eS[r] * iacc[i][r];
          if (!dfold) yy += Dd * uu;
          if constexpr (GATE) yy *= silu_fast((r & 1) ? bf16_hi(zw[r / 2]) : bf16_lo(zw[r / 2]));
          yv[i][r] = yy;
        }
      }
    }
    // carry the state over the chunk: H = 2^S_{T-1} H + B^T Xd (state pass: H += B^T Xd, Xd
    // already decayed to the segment's end)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < nk) {
        if constexpr (!STATE) hacc[k] = hacc[k] * eT;
        const bf16x8 ba = as_bf16x8(Bp[k * 64 + lane]);
        hacc[k] = mfma(ba, xdhi, hacc[k]);
        hacc[k] = mfma(ba, xdlo, hacc[k]);
      }
    }

    // stage the walk's next chunk (the last chunk stages itself again, unused), store y, load
    // the one after
    const int64_t i1 = i + 1 < nc ? i + 1 : i;
    stage(chunk_at(i1), bf ^ 1);
    if constexpr (!STATE) store_y(c * kT);
    prefetch(chunk_at(i + 2 < nc ? i + 2 : i1));
    __syncthreads();
  }

  if constexpr (STATE) {
    // this segment's end state (wave-ordered, as the output pass reads it) and decay
    // (with the caller's state decayed over the whole segment)
    f32x4v* hl = reinterpret_cast<f32x4v*>(sg.hloc) + (blk * kWaves + wave) * nk * 64 + lane;
    const float fin = __builtin_amdgcn_exp2f(dlog);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nk) {
        if (hinit) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int n = 16 * k + 4 * g16 + r;
            if (n < p.N) hacc[k][r] += fin * hinit[n];
          }
        }
        hl[k * 64] = hacc[k];
      }
    if (tid == 0) sg.dsum[blk] = dlog;
  } else {
    // the last segment ends with the state after the last step (steps past L are the identity)
    if (p.h_final && sgi == sg.nseg - 1) {
      float* hf = p.h_final + b * p.hf_sb + (c0 + pch) * p.hf_sd;
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = 16 * k + 4 * g16 + r;
          if (k < nk && n < p.N) hf[n] = hacc[k][r];
        }
    }
  }
}

}  // namespace

bool ssd_path(const ScanArgs& a) {
  return a.in_bf16 && a.chan_per_head % kSlab == 0 && a.chan_per_group % kSlab == 0;
}

// compute units of the current device (cached per device)
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

namespace {

// Blocks per CU the segments aim for.  Two output-pass blocks fit per CU (VGPRs and AGPRs
// share one register file: ~192 per lane, two waves per SIMD), and two rounds of them measured
// best: on workload 4 (160 rows of 256 chunks) 3 segments 0.321 ms, 4: 0.337, 6: 0.307,
// 8: 0.305, 12: 0.315, 16: 0.345 (shorter segments shorten the last round; more of them
// lengthen the state pass).
constexpr int kBlocksPerCU = 4;
constexpr int64_t kMinSegChunks = 16;

struct SegPlan {
  int64_t cps;
  int32_t nseg;
  int64_t rows;
};

// enough segments to give every CU about kBlocksPerCU blocks, none shorter than kMinSegChunks
// chunks (the state pass stages the B part in whole 16-byte pieces per thread: Np of 64, 128)
SegPlan seg_plan(const ScanArgs& a) {
  const int64_t nch = nchunks_of(a);
  const int64_t rows = a.batch * a.heads * (a.chan_per_head / kSlab);
  int64_t nseg = 1;
  if (npad32(a.N) % 64 == 0 && rows > 0)
    nseg = std::min<int64_t>((int64_t)kBlocksPerCU * cu_count() / rows, nch / kMinSegChunks);
#ifdef SS_SSD_SEGS
  if (npad32(a.N) % 64 == 0) nseg = std::min<int64_t>(SS_SSD_SEGS, nch);  // tuning override
#endif
  nseg = std::max<int64_t>(nseg, 1);
  const int64_t cps = (nch + nseg - 1) / nseg;
  nseg = (nch + cps - 1) / cps;
  return {cps, (int32_t)nseg, rows};
}

int64_t records_bytes(const ScanArgs& a) { return a.batch * a.groups * nchunks_of(a) * rec_bytes(npad32(a.N)); }

}  // namespace

int64_t ssd_workspace_bytes(const ScanArgs& a) {
  const SegPlan sp = seg_plan(a);
  const int64_t hand = (int64_t)(sp.nseg - 1) * sp.rows;   // state-pass blocks
  return records_bytes(a) + hand * (int64_t)npad32(a.N) * 64 * 4 + hand * 4;
}

hipError_t launch_ssd(const ScanArgs& a, void* ws, hipStream_t s) {
  const int Np = npad32(a.N);
  const int64_t nch = nchunks_of(a);
  hipLaunchKernelGGL((ssd_prep_kernel<bf16_t>), dim3((unsigned)(a.batch * a.groups * nch)), dim3(256), 0, s, a,
                     static_cast<uint8_t*>(ws), Np, nch);
  const SegPlan sp = seg_plan(a);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int64_t hand = (int64_t)(sp.nseg - 1) * sp.rows;
  Segs sg{sp.cps, sp.nseg, reinterpret_cast<float*>(w + records_bytes(a)), nullptr};
  sg.dsum = sg.hloc + hand * (int64_t)Np * 64;
  const dim3 block(64 * kWaves), sgrid((unsigned)hand), grid((unsigned)(sp.nseg * sp.rows));
  // whole chunks and 16-byte aligned rows: the variant without bounds checks
  const bool full = a.vec && a.L % kT == 0;
#define SS_STATE(TO, NPV)                                                                                  \
  if (hand > 0) {                                                                                          \
    if (full) hipLaunchKernelGGL((ssd_scan_kernel<TO, false, NPV, true, true>), sgrid, block, 0, s, a, w, nch, sg);  \
    else hipLaunchKernelGGL((ssd_scan_kernel<TO, false, NPV, false, true>), sgrid, block, 0, s, a, w, nch, sg);      \
  }
#define SS_LAUNCH(TO, GT, NPV)                                                                              \
  if (full) hipLaunchKernelGGL((ssd_scan_kernel<TO, GT, NPV, true, false>), grid, block, 0, s, a, w, nch, sg);     \
  else hipLaunchKernelGGL((ssd_scan_kernel<TO, GT, NPV, false, false>), grid, block, 0, s, a, w, nch, sg);
#define SS_OUT(NPV)                                                                                        \
  if (a.out_bf16) {                                                                                        \
    if (a.z) { SS_LAUNCH(bf16_t, true, NPV) } else { SS_LAUNCH(bf16_t, false, NPV) }                       \
  } else {                                                                                                 \
    if (a.z) { SS_LAUNCH(float, true, NPV) } else { SS_LAUNCH(float, false, NPV) }                         \
  }
  switch (Np) {
    case 32: SS_OUT(32) break;
    case 64: SS_STATE(float, 64) SS_OUT(64) break;
    case 96: SS_OUT(96) break;
    case 128: SS_STATE(float, 128) SS_OUT(128) break;
    default: return hipErrorInvalidValue;
  }
#undef SS_STATE
#undef SS_LAUNCH
#undef SS_OUT
  return hipGetLastError();
}

}  // namespace ss
