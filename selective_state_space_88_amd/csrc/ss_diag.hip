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
//  - a wave holds ROWS channels (1 or 2) of one (batch, B/C group), each on a row of
//    64 / ROWS lanes laid along time: lane j of a row owns K consecutive steps, so one window
//    of a channel covers (64 / ROWS) * K steps.  A block is 4 waves, i.e. 4 * ROWS channels
//    sharing B and C.  Windows are walked in order; the state at the end of each window is
//    carried to the next through LDS, so each exp is evaluated exactly once;
//  - the N states are processed two at a time.  For a state each lane runs its K steps from
//    zero (keeping the K decays a_t and inputs b_t in registers), the row combines its lane
//    aggregates with a DPP scan (row_shr within rows of 16 lanes, row_bcast across them, then
//    a shift for the exclusive prefix), and each lane re-runs its K steps from the true
//    incoming state to form h_t and accumulate y_t += C_{t,n} h_t.  The two states of a pair
//    are independent chains.  With one channel per wave (few rows, so few waves) the wave
//    interleaves them (their two scans fill each other's DPP wait states); with two channels
//    per wave (many rows) it runs them one after the other, which keeps the kernel within a
//    third of the register file and the block within a third of the LDS, i.e. three waves per
//    SIMD whose work covers each other's waits.  Two channels per wave also means a shorter scan
//    and half the B/C traffic per channel; one means more waves for short batches; the launch
//    picks;
//  - B and C are shared by every channel of a (batch, group).  Per state pair and window they
//    are copied into LDS with direct-to-LDS loads (buffer_load ... lds) several pairs ahead of
//    use, so the copies never pass through registers and overlap the arithmetic, and widened
//    to f32 in LDS by the whole block one pair ahead of use (see "B/C stages" below);
//  - u, delta and z of the next window are copied the same way into per-wave LDS slots while
//    the current window runs (u and delta right after they are read, z after the gate), so no
//    global load latency sits on the path.  The waits are explicit: before each ring barrier a
//    wave waits only for the pair the next iteration reads (vmcnt retires this wave's vector
//    memory operations, loads and stores alike, in issue order), never for what it issued after;
//  - softplus, D*u and the silu gate are fused; u, delta, z and y stream through HBM once, y
//    leaving through LDS so that every store instruction writes whole rows of consecutive y.
#include <stdlib.h>

#include <algorithm>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kWaves = 4;                   // waves per block
constexpr int kK = 16;                      // steps per lane

// Steps per window of one channel and floats of one f32 pair stage (B, C of state 2p, then of
// state 2p + 1).
template <int ROWS> constexpr int win_steps() { return (64 / ROWS) * kK; }
template <int ROWS> constexpr int slot_floats() { return 4 * win_steps<ROWS>(); }

// Two independent exclusive scans, within each row of 64 / ROWS lanes (lane 0 of the row
// earliest), of (a, b) pairs under (a1, b1) then (a2, b2) = (a1 a2, a2 b1 + b2).  Each step is
// one fused DPP multiply and one fused DPP FMA per scan: v_fmac_f32_dpp b, b[src], a
// (b += b[src] * a) and v_mul_f32_dpp a, a[src], a.  A lane whose DPP source is outside its
// 16-lane DPP row (row_shr) or whose DPP row is masked off (row_bcast with row_mask) is not
// written, i.e. it keeps its pair, which is the same as combining with the identity (1, 0).
// Steps: row_shr:1,2,4,8 scan each DPP row of 16 lanes; row_bcast:15 on DPP rows 1 and 3 adds
// rows 0 and 2 (a 32-lane channel row is complete here); for 64-lane rows row_bcast:31 on rows
// 2 and 3 then adds the first half.  The exclusive prefix shifts by one lane inside the row
// (lane 0 of the row gets the identity): wave_shr:1 for 64 lanes; for 32 lanes row_shr:1,
// with lane 16 of the row first given lane 15's value by row_bcast:15 on bank 0.  The two
// scans are interleaved so that every DPP read of a VGPR comes at least two instructions after
// the VALU write of it (the hardware needs two wait states there); the leading s_nop covers
// the compiler's last writes.
//
// The same statement also loads this lane's C values of the pair (eight 16-byte LDS reads at
// cbase + the given offsets, into c[0..7]) and waits for them at its end, so that the reads
// overlap the scan.  The slot they read is filled by direct-to-LDS copies whose completion the
// kernel establishes with its own vmcnt waits; read through plain C++, the compiler would
// put a wait for every copy in flight in front of them.
template <int ROWS, int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void row_exclusive_scan2(float& a0, float& b0, float& a1, float& b1, uint32_t cbase,
                                                    f32x4 (&c)[8]) {
  float ea0, eb0, ea1, eb1;
#define SS_STEP(CTRL)                                   \
  "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n"                \
  "v_fmac_f32_dpp %3, %3, %2 " CTRL "\n"                \
  "v_mul_f32_dpp %0, %0, %0 " CTRL "\n"                 \
  "v_mul_f32_dpp %2, %2, %2 " CTRL "\n"
#define SS_SCAN16                                       \
  "s_nop 1\n"                                           \
  SS_STEP("row_shr:1 row_mask:0xf bank_mask:0xf")       \
  SS_STEP("row_shr:2 row_mask:0xf bank_mask:0xf")       \
  SS_STEP("row_shr:4 row_mask:0xf bank_mask:0xf")       \
  SS_STEP("row_shr:8 row_mask:0xf bank_mask:0xf")
#define SS_IDENT                                        \
  "v_mov_b32 %4, 1.0\n"                                 \
  "v_mov_b32 %6, 1.0\n"                                 \
  "v_mov_b32 %5, 0\n"                                   \
  "v_mov_b32 %7, 0\n"
#define SS_SHIFT(CTRL)                                  \
  "v_mov_b32_dpp %4, %0 " CTRL "\n"                     \
  "v_mov_b32_dpp %6, %2 " CTRL "\n"                     \
  "v_mov_b32_dpp %5, %1 " CTRL "\n"                     \
  "v_mov_b32_dpp %7, %3 " CTRL "\n"
#define SS_LOADC                                        \
  "ds_read_b128 %8, %16 offset:%17\n"                   \
  "ds_read_b128 %9, %16 offset:%18\n"                   \
  "ds_read_b128 %10, %16 offset:%19\n"                  \
  "ds_read_b128 %11, %16 offset:%20\n"                  \
  "ds_read_b128 %12, %16 offset:%21\n"                  \
  "ds_read_b128 %13, %16 offset:%22\n"                  \
  "ds_read_b128 %14, %16 offset:%23\n"                  \
  "ds_read_b128 %15, %16 offset:%24\n"
#define SS_OPS                                                                                  \
  : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "=&v"(ea0), "=&v"(eb0), "=&v"(ea1), "=&v"(eb1),      \
    "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(c[4]), "=&v"(c[5]), "=&v"(c[6]),   \
    "=&v"(c[7])                                                                                 \
  : "v"(cbase), "n"(O0), "n"(O1), "n"(O2), "n"(O3), "n"(O4), "n"(O5), "n"(O6), "n"(O7)
  if constexpr (ROWS == 1) {
    asm volatile(SS_LOADC
                 SS_SCAN16
                 SS_STEP("row_bcast:15 row_mask:0xa bank_mask:0xf")
                 SS_STEP("row_bcast:31 row_mask:0xc bank_mask:0xf")
                 SS_IDENT
                 SS_SHIFT("wave_shr:1 row_mask:0xf bank_mask:0xf")
                 "s_waitcnt lgkmcnt(0)\n"
                 SS_OPS);
  } else if constexpr (ROWS == 2) {
    asm volatile(SS_LOADC
                 SS_SCAN16
                 SS_STEP("row_bcast:15 row_mask:0xa bank_mask:0xf")
                 SS_IDENT
                 SS_SHIFT("row_bcast:15 row_mask:0xa bank_mask:0x1")
                 SS_SHIFT("row_shr:1 row_mask:0xf bank_mask:0xf")
                 "s_waitcnt lgkmcnt(0)\n"
                 SS_OPS);
  } else {
    static_assert(ROWS == 1 || ROWS == 2, "1 or 2 channels per wave");
  }
#undef SS_OPS
#undef SS_LOADC
#undef SS_SHIFT
#undef SS_IDENT
#undef SS_SCAN16
#undef SS_STEP
  a0 = ea0;
  b0 = eb0;
  a1 = ea1;
  b1 = eb1;
}

// The same for one state, returning this lane's incoming state: an inclusive scan of (a, b)
// within each row of 64 / ROWS lanes gives every lane the map of its row's lanes up to itself,
// applied to the carried state (carry: the row's state before the window) that is the state
// at the end of the lane's steps, and a shift by one lane within the row (its first lane
// taking the carried state itself) makes it the state before them.  This lane's four C quads
// of the state (at cbase + the given offsets) are read while the scan runs.  A single chain
// leaves one instruction between a VALU write and the next DPP read of the same VGPR, so each
// step ends with an s_nop that supplies the second wait state.
template <int ROWS, int O0, int O1, int O2, int O3>
__device__ __forceinline__ float row_incoming_state1(float a, float bb, float carry, uint32_t cbase,
                                                     f32x4 (&c)[4]) {
  float he, hs;
#define SS_STEP1(CTRL)                                  \
  "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n"               \
  "v_mul_f32_dpp %0, %0, %0 " CTRL "\n"                \
  "s_nop 0\n"
#define SS_SCAN16_1                                     \
  "s_nop 1\n"                                          \
  SS_STEP1("row_shr:1 row_mask:0xf bank_mask:0xf")      \
  SS_STEP1("row_shr:2 row_mask:0xf bank_mask:0xf")      \
  SS_STEP1("row_shr:4 row_mask:0xf bank_mask:0xf")      \
  SS_STEP1("row_shr:8 row_mask:0xf bank_mask:0xf")
#define SS_END1                                         \
  "v_fma_f32 %2, %0, %8, %1\n"                         \
  "v_mov_b32 %3, %8\n"                                 \
  "s_nop 0\n"
#define SS_LOADC1                                       \
  "ds_read_b128 %4, %9 offset:%10\n"                   \
  "ds_read_b128 %5, %9 offset:%11\n"                   \
  "ds_read_b128 %6, %9 offset:%12\n"                   \
  "ds_read_b128 %7, %9 offset:%13\n"
#define SS_OPS1                                                                                 \
  : "+v"(a), "+v"(bb), "=&v"(he), "=&v"(hs), "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]) \
  : "v"(carry), "v"(cbase), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
  if constexpr (ROWS == 1) {
    asm volatile(SS_LOADC1
                 SS_SCAN16_1
                 SS_STEP1("row_bcast:15 row_mask:0xa bank_mask:0xf")
                 SS_STEP1("row_bcast:31 row_mask:0xc bank_mask:0xf")
                 SS_END1
                 "v_mov_b32_dpp %3, %2 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
                 "s_waitcnt lgkmcnt(0)\n"
                 SS_OPS1);
  } else if constexpr (ROWS == 2) {
    // the second half of a 32-lane row starts from lane 15 of the first (row_bcast:15 on the
    // first four lanes of DPP rows 1 and 3), the other lanes from the lane below (row_shr:1;
    // the first lane of each DPP row has no source there and keeps what it has)
    asm volatile(SS_LOADC1
                 SS_SCAN16_1
                 SS_STEP1("row_bcast:15 row_mask:0xa bank_mask:0xf")
                 SS_END1
                 "v_mov_b32_dpp %3, %2 row_bcast:15 row_mask:0xa bank_mask:0x1\n"
                 "v_mov_b32_dpp %3, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n"
                 "s_waitcnt lgkmcnt(0)\n"
                 SS_OPS1);
  } else {
    static_assert(ROWS == 1 || ROWS == 2, "1 or 2 channels per wave");
  }
#undef SS_OPS1
#undef SS_LOADC1
#undef SS_END1
#undef SS_SCAN16_1
#undef SS_STEP1
  return hs;
}

// The same for a 64-lane row with nothing read alongside: this lane's incoming state, from the
// lane aggregate (a, bb) and the row's carried state.
__device__ __forceinline__ float row_incoming_state(float a, float bb, float carry) {
  float he, hs;
#define SS_STEP1(CTRL)                                  \
  "v_fmac_f32_dpp %1, %1, %0 " CTRL "\n"               \
  "v_mul_f32_dpp %0, %0, %0 " CTRL "\n"                \
  "s_nop 0\n"
  asm volatile("s_nop 1\n"
               SS_STEP1("row_shr:1 row_mask:0xf bank_mask:0xf")
               SS_STEP1("row_shr:2 row_mask:0xf bank_mask:0xf")
               SS_STEP1("row_shr:4 row_mask:0xf bank_mask:0xf")
               SS_STEP1("row_shr:8 row_mask:0xf bank_mask:0xf")
               SS_STEP1("row_bcast:15 row_mask:0xa bank_mask:0xf")
               SS_STEP1("row_bcast:31 row_mask:0xc bank_mask:0xf")
               "v_fma_f32 %2, %0, %4, %1\n"
               "v_mov_b32 %3, %4\n"
               "s_nop 0\n"
               "v_mov_b32_dpp %3, %2 wave_shr:1 row_mask:0xf bank_mask:0xf\n"
               : "+v"(a), "+v"(bb), "=&v"(he), "=&v"(hs)
               : "v"(carry));
#undef SS_STEP1
  return hs;
}

// One direct-to-LDS copy of 16 bytes per lane: lane i's 16 bytes from `src` land at
// lds_base + 16 i (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) then s_barrier: this wave's memory operations older than its
// last n have completed and its LDS reads are done.  vmcnt is an immediate, so n is
// dispatched over the values the kernel uses; anything larger waits for everything (safe).
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

// lds_read8 plus CPT (1 or 2) 16-byte reads at rbase + 4 KB m and one at pbase (the pair's
// parameters), in the same statement.
template <int CPT, int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read8_plus(uint32_t base, f32x4 (&v)[8], uint32_t rbase, u32x4 (&raw)[CPT],
                                               uint32_t pbase, f32x4& pv) {
  if constexpr (CPT == 1) {
    asm volatile(
        "ds_read_b128 %9, %12\n\t"
        "ds_read_b128 %8, %11\n\t"
        "ds_read_b128 %0, %10 offset:%13\n\tds_read_b128 %1, %10 offset:%14\n\t"
        "ds_read_b128 %2, %10 offset:%15\n\tds_read_b128 %3, %10 offset:%16\n\t"
        "ds_read_b128 %4, %10 offset:%17\n\tds_read_b128 %5, %10 offset:%18\n\t"
        "ds_read_b128 %6, %10 offset:%19\n\tds_read_b128 %7, %10 offset:%20\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(raw[0]), "=&v"(pv)
        : "v"(base), "v"(rbase), "v"(pbase), "n"(O0), "n"(O1), "n"(O2), "n"(O3), "n"(O4), "n"(O5), "n"(O6),
          "n"(O7)
        : "memory");
  } else {
    static_assert(CPT == 2, "one or two chunks");
    asm volatile(
        "ds_read_b128 %10, %13\n\t"
        "ds_read_b128 %8, %12\n\tds_read_b128 %9, %12 offset:4096\n\t"
        "ds_read_b128 %0, %11 offset:%14\n\tds_read_b128 %1, %11 offset:%15\n\t"
        "ds_read_b128 %2, %11 offset:%16\n\tds_read_b128 %3, %11 offset:%17\n\t"
        "ds_read_b128 %4, %11 offset:%18\n\tds_read_b128 %5, %11 offset:%19\n\t"
        "ds_read_b128 %6, %11 offset:%20\n\tds_read_b128 %7, %11 offset:%21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(raw[0]), "=&v"(raw[1]), "=&v"(pv)
        : "v"(base), "v"(rbase), "v"(pbase), "n"(O0), "n"(O1), "n"(O2), "n"(O3), "n"(O4), "n"(O5), "n"(O6),
          "n"(O7)
        : "memory");
  }
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The zero-order-hold input coefficient (exp(dt A) - 1) / A of one (step, state), from
// x = dt A, the decay e = exp(x) already computed and rA = 1 / A (A = 0 gives x = 0).  Where
// |x| < 1/8, dt phi(x) with phi(x) = expm1(x) / x from its Taylor polynomial to degree 5
// (truncation below 1e-9 relative); elsewhere e rA - rA, whose relative error from e's
// rounding is at most 2^-23 / (1 - e^(-1/8)) ~ 1e-6.  (No per-step reciprocal: dt cancels.)
__device__ __forceinline__ float zoh_coef(float dt, float x, float e, float rA) {
  float q = 1.f / 720.f;
  q = fmaf(q, x, 1.f / 120.f);
  q = fmaf(q, x, 1.f / 24.f);
  q = fmaf(q, x, 1.f / 6.f);
  q = fmaf(q, x, 0.5f);
  q = fmaf(q, x, 1.f);
  return fabsf(x) < 0.125f ? dt * q : fmaf(e, rA, -rA);
}

// The carried state pair (.z, .w) of one pair's parameters, written through asm: a plain store
// would make the compiler wait for every copy in flight first.
__device__ __forceinline__ void par_state_write(float4* pp, float h0, float h1) {
  asm volatile("ds_write_b64 %0, %1 offset:8" ::"v"(lds_addr(pp)), "v"(f32x2v{h0, h1}) : "memory");
}

// Two 16-byte LDS reads, waited for in the same statement.  The slots they read are filled by
// direct-to-LDS copies whose completion the kernel establishes with its own vmcnt waits; read
// through plain C++ the compiler would put a wait for every copy in flight (stage copies and
// y stores included) in front of them.
__device__ __forceinline__ void lds_read2(const void* p0, const void* p1, u32x4& v0, u32x4& v1) {
  const uint32_t a0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p0;
  const uint32_t a1 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p1;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v0), "=&v"(v1)
               : "v"(a0), "v"(a1)
               : "memory");
}

__device__ __forceinline__ u32x4 lds_read1(const void* p0) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p0)) : "memory");
  return v;
}

// Eight 16-byte LDS reads at base + the given byte offsets and one at pbase (the pair's
// parameters), waited for in the same statement (for the same reason as lds_read2).
template <int O0, int O1, int O2, int O3, int O4, int O5, int O6, int O7>
__device__ __forceinline__ void lds_read8(uint32_t base, f32x4 (&v)[8], uint32_t pbase, f32x4& pv) {
  asm volatile(
      "ds_read_b128 %8, %10\n\t"
      "ds_read_b128 %0, %9 offset:%11\n\tds_read_b128 %1, %9 offset:%12\n\t"
      "ds_read_b128 %2, %9 offset:%13\n\tds_read_b128 %3, %9 offset:%14\n\t"
      "ds_read_b128 %4, %9 offset:%15\n\tds_read_b128 %5, %9 offset:%16\n\t"
      "ds_read_b128 %6, %9 offset:%17\n\tds_read_b128 %7, %9 offset:%18\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(pv)
      : "v"(base), "v"(pbase), "n"(O0), "n"(O1), "n"(O2), "n"(O3), "n"(O4), "n"(O5), "n"(O6), "n"(O7)
      : "memory");
}

template <typename TIn>
__device__ __forceinline__ void seg_read(const uint32_t* slot, int lane, Seg<TIn>& s) {
  static_assert(Seg<TIn>::kChunks % 2 == 0, "chunks are read in pairs");
#pragma unroll
  for (int c = 0; c < Seg<TIn>::kChunks; c += 2) {
    u32x4 v0, v1;
    lds_read2(reinterpret_cast<const u32x4*>(slot + c * 256) + lane,
              reinterpret_cast<const u32x4*>(slot + (c + 1) * 256) + lane, v0, v1);
    s.w[4 * c] = v0.x;
    s.w[4 * c + 1] = v0.y;
    s.w[4 * c + 2] = v0.z;
    s.w[4 * c + 3] = v0.w;
    s.w[4 * c + 4] = v1.x;
    s.w[4 * c + 5] = v1.y;
    s.w[4 * c + 6] = v1.z;
    s.w[4 * c + 7] = v1.w;
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

// ---------------------------------------------------------------------------------------
// B/C stages.  Pair p of window w is one stage: rows r = 0..3 are B, C of state 2p and B, C of
// state 2p + 1 over the window's W steps.  For odd N the last pair's second state reads as
// zeros (B = C = 0 leaves it at zero and out of y): its copies go through a buffer resource of
// zero size, and loads outside a buffer resource's range return zero.  In LDS the scan reads a stage
// as f32, row r's quad i (steps 4i..4i+3 of a lane) of lane j at float r W + (i LPC + j) 4, so
// that every ds_read_b128 of a wave reads consecutive LDS.  How a stage gets there:
//  - bf16 inputs, 16-byte rows: the four rows are copied raw (each wave one row, 16 bytes a
//    lane, direct-to-LDS buffer loads) into a raw ring of AHEAD slots AHEAD stages ahead of
//    use (3 with one channel per wave, 2 with two); one stage ahead of use the block widens
//    them into a 2-slot f32 ring (each thread 8 steps);
//  - f32 inputs, 16-byte rows: copied straight into the f32 layout, into a 3-slot f32 ring two
//    stages ahead of use;
//  - anything else: loaded element by element and widened into the 2-slot f32 ring one stage
//    ahead of use.
enum class StageMode { kWiden, kDirect, kElementwise };

template <typename TIn, bool VEC>
constexpr StageMode stage_mode() {
  return !VEC ? StageMode::kElementwise : (sizeof(TIn) == 2 ? StageMode::kWiden : StageMode::kDirect);
}

// One direct-to-LDS buffer load of 16 bytes per lane from a wave-uniform resource: lane i's
// 16 bytes at byte offset voff land at lds_base + 16 i.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}

// 16-byte LDS write through asm (the compiler would otherwise wait for every copy in flight
// before it, not knowing which LDS the copies write).
__device__ __forceinline__ void lds_write16(uint32_t addr, f32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// MODE bits (the plain forward, MODE 0, compiles without them):
//   kSIO   the call passes an initial and/or a final state;
//   kZOH   zero-order-hold input coefficient (exp(dt A) - 1) / A instead of dt;
//   kTRAP  exponential-trapezoidal rule: the scan runs the state k = h + e/2, which obeys the
//          Euler recurrence k_t = a_t k_{t-1} + e_t, and y reads C (k - e/2).
// kCKPT: also store the backward's checkpoints (ScanArgs::ckpt); only with none of the others
//        (the window-slot kernel: or with kSIO, a sequence segment's entering state)
// kPERT: (window-slot kernel, plain or with kCKPT) the timing stress of perturb_wait
constexpr int kSIO = 1, kZOH = 2, kTRAP = 4, kCKPT = 8, kPERT = 16;
template <typename TIn, typename TOut, bool GATE, bool VEC, int ROWS, int MODE>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(ROWS == 2 && sizeof(TIn) == 2 ? 3 : 2))) void diag_fwd_kernel(
    ScanArgs p, int npairs, int64_t nwin, int64_t blocks_per_bg) {
  constexpr bool SIO = (MODE & kSIO) != 0, ZOH = (MODE & kZOH) != 0, TRAP = (MODE & kTRAP) != 0;
  constexpr bool CKPT = (MODE & kCKPT) != 0;
  constexpr StageMode SMODE = stage_mode<TIn, VEC>();
  constexpr int LPC = 64 / ROWS;                     // lanes per channel row
  constexpr int W = win_steps<ROWS>();               // steps per window of a channel
  constexpr int SLOT = slot_floats<ROWS>();          // floats of one f32 stage
  // Two channels per wave (many rows) runs three waves per SIMD: the two states of a pair then
  // go one after the other (SPLIT), which keeps the registers within a third of the file, and
  // the raw ring has two slots, which keeps the block's LDS within a third of the CU's.  One
  // channel per wave (few rows, few waves) keeps both states in flight at once for the
  // instruction-level parallelism, and copies the raw stages three pairs ahead; so do f32
  // inputs, whose per-wave input slots are twice as large and allow only two blocks per CU.
  constexpr bool SPLIT = ROWS == 2 && sizeof(TIn) == 2;
  constexpr int NF = SMODE == StageMode::kDirect ? 3 : 2;       // f32 ring slots
  constexpr int AHEAD = SMODE == StageMode::kWiden ? (SPLIT ? 2 : 3) : 2;   // stages copied ahead of use
  // (the copy that the next pair's widening or reading needs was issued by this pair when
  // AHEAD is 2 in kWiden, by the pair before otherwise)
  constexpr bool NEED_LAST = SMODE == StageMode::kWiden && AHEAD == 2;
  constexpr int ROWB = W * (int)sizeof(TIn);                   // bytes of one stage row
  constexpr int NDMA = SMODE == StageMode::kWiden ? ROWB / 1024 : W / 256;  // copies per wave per stage
  constexpr int NCI = Seg<TIn>::kChunks;             // 16-byte copies per lane per input row
  constexpr int kSegWords = NCI * 256;
  constexpr int NCO = kK * (int)sizeof(TOut) / 16;   // 16-byte stores per lane of y
  constexpr int GPR = LPC * NCO;                     // 16-byte granules of y per channel row
  constexpr int CPT = W / 512;                       // 8-step chunks widened per thread per stage
  static_assert(ROWS == 1 || ROWS == 2, "1 or 2 channels per wave");
  __shared__ __attribute__((aligned(16))) float fring[NF][SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t rring[SMODE == StageMode::kWiden ? AHEAD : 1]
                                                       [SMODE == StageMode::kWiden ? ROWB : 4];
  // per wave: u, delta, z of one window (y leaves through the z slot once z has been read)
  __shared__ __attribute__((aligned(16))) uint32_t xin[kWaves][3][kSegWords];
  // per (wave, row, pair): (A_2p, A_2p+1) * log2 e and the carried state of the pair, sized
  // by the launch (kWaves * ROWS * pairs).  Read in the pair loop through asm with the B values:
  // the compiler cannot tell that the copies in flight do not write this array, and would wait
  // for all of them before a plain read.
  extern __shared__ float4 par[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPC;        // channel row of this lane
  const int jl = lane % LPC;       // lane within the row
  const int64_t L = p.L;
  const int N = p.N;
  const int P = npairs;

  const int64_t bg = blockIdx.x / blocks_per_bg, blk = blockIdx.x % blocks_per_bg;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t local0 = (blk * kWaves + wave) * ROWS;  // first channel (in the group) of the wave
  const int64_t cpg = p.chan_per_group;
  const int64_t local = local0 + r;
  const bool live = local < cpg;
  const bool wave_live = local0 + ROWS <= cpg;         // every row of the wave is a channel
  const int64_t d = g * cpg + (live ? local : cpg - 1);
  const int64_t hd = d / p.chan_per_head;
  const TIn* urow = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* drow = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TIn* zrow = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  float bias = p.bias ? p.bias[hd] : 0.f;
  float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;
  // complete these loads here, through a statement that redefines both values: otherwise the
  // compiler waits for them at their first use inside the window loop, i.e. for every copy in
  // flight there, once per window
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bias), "+v"(Dd));
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  const int Qt = (int)(nwin * P);  // pair stages of this block, in order (window-major)

  float4* mypar = par + (wave * ROWS + r) * P;
  {
    // the carried state starts at the caller's initial state, or at zero
    const float* Ar = p.A + d * p.A_sd;
    const float* hi = (SIO && p.h_init) ? p.h_init + b * p.hi_sb + d * p.hi_sd : nullptr;
    for (int pp = jl; pp < P; pp += LPC) {
      const int n = 2 * pp;
      mypar[pp] = make_float4(Ar[n] * kLog2e, n + 1 < N ? Ar[n + 1] * kLog2e : 0.f, hi ? hi[n] : 0.f,
                              (hi && n + 1 < N) ? hi[n + 1] : 0.f);
    }
  }
  uint32_t* xu = xin[wave][0];
  uint32_t* xd = xin[wave][1];
  uint32_t* xz = xin[wave][2];

  // row r (0..3) of stage qs: its global row (nullptr for a state >= N) and first step
  auto stage_row = [&](int qs, int rr, int64_t& t_first) -> const TIn* {
    const int wq = qs / P;
    const int pp = qs - wq * P;
    const int n = 2 * pp + (rr >> 1);
    t_first = (int64_t)wq * W;
    if (n >= N) return nullptr;
    return (rr & 1) ? Cg + n * p.C_sn : Bg + n * p.B_sn;
  };
  // Issue the copies of stage qs (kWiden: this wave's raw row; kDirect: this wave's row,
  // already in the f32 layout).  Chunks past L copy the row's first chunk (in bounds; the
  // scan masks those steps).
  auto stage_copy = [&](int qs) {
    int64_t t_first;
    const TIn* row = stage_row(qs, wave, t_first);
    const __amdgpu_buffer_rsrc_t rs =  // over the window, so offsets stay small; empty for no state
        __builtin_amdgcn_make_buffer_rsrc(const_cast<TIn*>(row ? row + t_first : Bg), (short)0,
                                          row ? 0x7fffffff : 0, 0x00020000);
    const int64_t lim = L - t_first;  // steps of this window inside the row
    if constexpr (SMODE == StageMode::kWiden) {
      uint32_t* dst = rring[qs % AHEAD] + wave * (ROWB / 4);
#pragma unroll
      for (int c = 0; c < NDMA; ++c) {
        const int64_t tl = (int64_t)(c * 64 + lane) * 8;  // 8 bf16 a lane
        dma16_buf(rs, (uint32_t)(tl < lim ? tl * 2 : 0), dst + c * 256);
      }
    } else {
      float* dst = &fring[qs % 3][wave * W];
#pragma unroll
      for (int c = 0; c < NDMA; ++c) {
        const int qd = c * 64 + lane;                  // quad (i, j) of the row in LDS order
        const int64_t tl = (int64_t)(qd % LPC) * kK + 4 * (qd / LPC);
        dma16_buf(rs, (uint32_t)(tl < lim ? tl * 4 : 0), dst + c * 256);
      }
    }
  };
  // Widen (kWiden: from the raw ring; kElementwise: from global memory) stage qs into f32 slot
  // fs: each thread does CPT chunks of 8 consecutive steps of one row.
  // (kWiden: raw[m] holds this thread's chunks of stage qs, read from the raw ring)
  auto stage_widen = [&](int qs, int fs, const u32x4* raw) {
    const uint32_t fbase = lds_addr(fring[fs]);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int k = (int)threadIdx.x + 256 * m;
      const int rr = k / (W / 8), cc = k % (W / 8);
      float v[8];
      if constexpr (SMODE == StageMode::kWiden) {
        const uint32_t wd[4] = {raw[m].x, raw[m].y, raw[m].z, raw[m].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16_lo(wd[e]);
          v[2 * e + 1] = bf16_hi(wd[e]);
        }
      } else {
        int64_t t_first;
        const TIn* row = stage_row(qs, rr, t_first);
        const int64_t t = t_first + 8 * cc;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = row && t + e < L ? to_f32(row[t + e]) : 0.f;
      }
      const int j = cc / 2, i0 = 2 * (cc % 2);
      lds_write16(fbase + 4u * (uint32_t)(rr * W + (i0 * LPC + j) * 4), f32x4{v[0], v[1], v[2], v[3]});
      lds_write16(fbase + 4u * (uint32_t)(rr * W + ((i0 + 1) * LPC + j) * 4), f32x4{v[4], v[5], v[6], v[7]});
    }
  };
  auto x_copy = [&](const TIn* row, int64_t w, uint32_t* slot) {
    const int64_t t0 = w * W + (int64_t)jl * kK;
    if constexpr (VEC) seg_dma<TIn>(row, t0, L, slot);
    else seg_fill<TIn>(row, t0, L, slot, lane);
  };

  // preamble: the first window's inputs and the first stages
  if constexpr (VEC) {
    x_copy(urow, 0, xu);
    x_copy(drow, 0, xd);
    if constexpr (GATE) x_copy(zrow, 0, xz);
  }
  if constexpr (SMODE == StageMode::kWiden) {
    for (int qs = 0; qs < AHEAD && qs < Qt; ++qs) stage_copy(qs);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    {
      u32x4 raw[CPT];
#pragma unroll
      for (int m = 0; m < CPT; ++m) raw[m] = lds_read1(rring[0] + ((int)threadIdx.x + 256 * m) * 4);
      stage_widen(0, 0, raw);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else if constexpr (SMODE == StageMode::kDirect) {
    for (int qs = 0; qs < 2 && qs < Qt; ++qs) stage_copy(qs);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    stage_widen(0, 0, nullptr);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  int q = 0;          // current pair stage
  int carry_ops = 0;  // memory ops issued in the last epilogue (counted by the first wait after it)
  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t w0 = w * W;
    const int64_t t0 = w0 + (int64_t)jl * kK;
    const bool full = w0 + W <= L;

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
          wv[j] = ZOH ? uu : sp * uu;   // (zero-order hold: u, its coefficient already holds dt)
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
          wv[j] = ZOH ? uu : sp * uu;   // (zero-order hold: u, its coefficient already holds dt)
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
      // copies of a later stage, and (kWiden, kElementwise) the next stage into f32
      // memory operations issued after the copy the next pair needs (NEED_LAST: none)
      int allow = (!NEED_LAST && pp == 0) ? boundary_ops : 0;
      if constexpr (SMODE != StageMode::kElementwise) {
        if (q + AHEAD < Qt) {
          stage_copy(q + AHEAD);
          if (!NEED_LAST) allow += NDMA;
        }
      }
      if constexpr (SMODE == StageMode::kElementwise)
        if (q + 1 < Qt) stage_widen(q + 1, (q + 1) & 1, nullptr);
      const int fs = SMODE == StageMode::kDirect ? q % 3 : (q & 1);
      // this lane's B values of both states: quad i of row r of the slot is at byte offset
      // 4 W r + 16 (i LPC + j) from the slot
      const uint32_t lbase = lds_addr(fring[fs]) + 16u * (uint32_t)jl;
      constexpr int QS = 16 * LPC;
      f32x4 bq[8];  // B of state 2p (quads 0-3), then of state 2p + 1
      f32x4 pq;     // (A pair, carried state pair) of this lane's channel
      if constexpr (SMODE == StageMode::kWiden) {
        // with this thread's raw chunks of the next stage, widened right after
        u32x4 raw[CPT];
        lds_read8_plus<CPT, 0, QS, 2 * QS, 3 * QS, 8 * W, 8 * W + QS, 8 * W + 2 * QS, 8 * W + 3 * QS>(
            lbase, bq, lds_addr(rring[(q + 1) % AHEAD]) + 16u * threadIdx.x, raw, lds_addr(mypar + pp), pq);
        if (q + 1 < Qt) stage_widen(q + 1, (q + 1) & 1, raw);
      } else {
        lds_read8<0, QS, 2 * QS, 3 * QS, 8 * W, 8 * W + QS, 8 * W + 2 * QS, 8 * W + 3 * QS>(lbase, bq,
                                                                                        lds_addr(mypar + pp), pq);
      }
      const float4 pv = make_float4(pq[0], pq[1], pq[2], pq[3]);
      // the backward's checkpoints: the carried states are the states at the window's start
      if (CKPT && live && jl == 0) {
        float* ck = p.ckpt + ((b * p.channels + d) * p.ckpt_nwin + w * (W / 512)) * N + 2 * pp;
        ck[0] = pv.z;
        if (2 * pp + 1 < N) ck[1] = pv.w;
      }
      if constexpr (SPLIT) {
        // the two states one after the other (the registers of one state's K decays and inputs
        // are reused by the next)
        float hend[2];
#pragma unroll
        for (int si = 0; si < 2; ++si) {
          const float An = si ? pv.y : pv.x;   // A_n log2 e
          float av[kK], bv[kK];
#pragma unroll
          for (int j = 0; j < kK; ++j) av[j] = __builtin_amdgcn_exp2f(dt[j] * An);
          if constexpr (ZOH) {
            // u B times (exp(dt A) - 1) / A, from the decays just computed
            const float Anl = An * kLn2f, rA = __builtin_amdgcn_rcpf(Anl);
#pragma unroll
            for (int j = 0; j < kK; ++j)
              bv[j] = zoh_coef(dt[j], dt[j] * Anl, av[j], rA) * wv[j] * bq[4 * si + j / 4][j % 4];
          } else {
#pragma unroll
            for (int j = 0; j < kK; ++j) bv[j] = wv[j] * bq[4 * si + j / 4][j % 4];
          }
          // the lane's steps from a zero state (the first step's decay multiplies zero)
          float h = bv[0];
#pragma unroll
          for (int j = 1; j < kK; ++j) h = fmaf(av[j], h, bv[j]);
          // lane aggregate: decay over the lane's K steps and the lane's state from zero; the
          // scan, with this lane's C values of the state read while it runs
          float sa = __builtin_amdgcn_exp2f(sdt * An), sb = h;
          f32x4 cq[4];
          const float carry = si ? pv.w : pv.z;
          if (si == 0)
            h = row_incoming_state1<ROWS, 4 * W, 4 * W + QS, 4 * W + 2 * QS, 4 * W + 3 * QS>(sa, sb, carry, lbase, cq);
          else
            h = row_incoming_state1<ROWS, 12 * W, 12 * W + QS, 12 * W + 2 * QS, 12 * W + 3 * QS>(sa, sb, carry, lbase,
                                                                                                cq);
#pragma unroll
          for (int j = 0; j < kK; ++j) {
            h = fmaf(av[j], h, bv[j]);
            if constexpr (TRAP) yv[j] = fmaf(cq[j / 4][j % 4], fmaf(-0.5f, bv[j], h), yv[j]);
            else yv[j] = fmaf(cq[j / 4][j % 4], h, yv[j]);
          }
          hend[si] = h;
        }
        // the window's end state (the row's last lane) starts the same pair in the next window
        if (jl == LPC - 1) par_state_write(mypar + pp, hend[0], hend[1]);
      } else {
        float av0[kK], bv0[kK], av1[kK], bv1[kK];
        float wz0[ZOH ? kK : 1], wz1[ZOH ? kK : 1];
        float h0, h1;
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          av0[j] = __builtin_amdgcn_exp2f(dt[j] * pv.x);
          av1[j] = __builtin_amdgcn_exp2f(dt[j] * pv.y);
        }
        if constexpr (ZOH) {
          // u times (exp(dt A) - 1) / A, from the decays just computed
          const float An0 = pv.x * kLn2f, An1 = pv.y * kLn2f;
          const float rA0 = __builtin_amdgcn_rcpf(An0), rA1 = __builtin_amdgcn_rcpf(An1);
#pragma unroll
          for (int j = 0; j < kK; ++j) {
            wz0[j] = zoh_coef(dt[j], dt[j] * An0, av0[j], rA0) * wv[j];
            wz1[j] = zoh_coef(dt[j], dt[j] * An1, av1[j], rA1) * wv[j];
          }
        }
        // the lane's steps from a zero state (the first step's decay multiplies zero)
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          bv0[j] = (ZOH ? wz0[j] : wv[j]) * bq[j / 4][j % 4];
          bv1[j] = (ZOH ? wz1[j] : wv[j]) * bq[4 + j / 4][j % 4];
          h0 = j ? fmaf(av0[j], h0, bv0[j]) : bv0[j];
          h1 = j ? fmaf(av1[j], h1, bv1[j]) : bv1[j];
        }
        // lane aggregates: decay over the lane's K steps and the lane's state from zero
        float sa0 = __builtin_amdgcn_exp2f(sdt * pv.x), sb0 = h0;
        float sa1 = __builtin_amdgcn_exp2f(sdt * pv.y), sb1 = h1;
        // the scan, with this lane's C values of both states read while it runs
        f32x4 cq[8];
        row_exclusive_scan2<ROWS, 4 * W, 4 * W + QS, 4 * W + 2 * QS, 4 * W + 3 * QS, 12 * W, 12 * W + QS,
                            12 * W + 2 * QS, 12 * W + 3 * QS>(sa0, sb0, sa1, sb1, lbase, cq);
        h0 = fmaf(sa0, pv.z, sb0);
        h1 = fmaf(sa1, pv.w, sb1);
        if constexpr (CKPT && W == 1024) {
          // (64-lane rows: lane 32's incoming states are the states 512 steps into the window)
          if (live && jl == 32 && 2 * w + 1 < p.ckpt_nwin) {
            float* ck = p.ckpt + ((b * p.channels + d) * p.ckpt_nwin + 2 * w + 1) * N + 2 * pp;
            ck[0] = h0;
            if (2 * pp + 1 < N) ck[1] = h1;
          }
        }
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          h0 = fmaf(av0[j], h0, bv0[j]);
          h1 = fmaf(av1[j], h1, bv1[j]);
          if constexpr (TRAP) {
            yv[j] = fmaf(cq[j / 4][j % 4], fmaf(-0.5f, bv0[j], h0), yv[j]);
            yv[j] = fmaf(cq[4 + j / 4][j % 4], fmaf(-0.5f, bv1[j], h1), yv[j]);
          } else {
            yv[j] = fmaf(cq[j / 4][j % 4], h0, yv[j]);
            yv[j] = fmaf(cq[4 + j / 4][j % 4], h1, yv[j]);
          }
        }
        // the window's end state (the row's last lane) starts the same pair in the next window
        if (jl == LPC - 1) par_state_write(mypar + pp, h0, h1);
      }
      // The copies the next iteration reads (kDirect: stage q + 1; kWiden: stage q + 2, which
      // it widens) have landed, this wave's and, after the barrier, everyone's; and every
      // wave is done with the slots the next iteration overwrites.
      if (q + 1 < Qt) wait_vm_barrier(allow);
      ++q;
    }

    // epilogue: gate, store, then this slot's z for the next window.  Only the stage copy
    // issued by the last pair may still be in flight here: everything before it (this
    // window's z and the next window's u and delta) has landed.
    if (SMODE != StageMode::kElementwise && q - 1 + AHEAD < Qt) {
      if constexpr (NDMA == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
      else if constexpr (NDMA == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    carry_ops = 0;
    if constexpr (GATE) {
      if constexpr (!VEC) x_copy(zrow, w, xz);
      Seg<TIn> sz;
      seg_read<TIn>(xz, lane, sz);
#pragma unroll
      for (int j = 0; j < kK; ++j) yv[j] *= silu_fast(seg_get<TIn>(sz, j));
    }
    if (VEC && full) {
      // Through LDS, so that each store instruction writes whole channel rows of consecutive
      // y.  Lane granule c (steps 4c.. of a f32 lane, 8c.. of a bf16 lane) is granule
      // g = NCO lane + c of the wave's window; it is kept at g ^ ((g >> 4) & (NCO - 1)) so that
      // neither the writes nor the reads conflict on banks, and store instruction i has lane
      // l take granule 64 i + l, i.e. granule (64 i + l) mod GPR of row (64 i + l) / GPR.  The
      // wave's z slot (read above) holds YP granules, so y goes through it in NPASS passes of
      // 64 / NPASS lanes' granules each.
      // (written and read through asm: plain C++ here would make the compiler wait for every
      // copy in flight)
      constexpr int YP = kSegWords / 4;                     // granules in the slot
      constexpr int NPASS = NCO * 64 > YP ? NCO * 64 / YP : 1;
      constexpr int IPP = NCO / NPASS;                       // store instructions per pass
      static_assert(NCO % NPASS == 0 && NCO * 64 <= NPASS * YP, "y fits the slot in whole passes");
      const uint32_t sbase = lds_addr(xz);
#pragma unroll
      for (int h = 0; h < NPASS; ++h) {
        if (lane / (64 / NPASS) == h) {
#pragma unroll
          for (int c = 0; c < NCO; ++c) {
            u32x4 gr;
            if constexpr (sizeof(TOut) == 4) {
              gr = u32x4{__float_as_uint(yv[4 * c]), __float_as_uint(yv[4 * c + 1]), __float_as_uint(yv[4 * c + 2]),
                         __float_as_uint(yv[4 * c + 3])};
            } else {
              uint32_t wd[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                wd[e] = f32_to_bf16_bits(yv[8 * c + 2 * e]) | (f32_to_bf16_bits(yv[8 * c + 2 * e + 1]) << 16);
              gr = u32x4{wd[0], wd[1], wd[2], wd[3]};
            }
            const int gi = NCO * lane + c - 64 * IPP * h;   // granule within the pass
            const uint32_t a = sbase + 16u * (uint32_t)(gi ^ ((gi >> 4) & (NCO - 1)));
            asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(gr) : "memory");
          }
        }
        // granule 64 i + l of the pass sits at 64 i + (l ^ ((l >> 4) & (NCO - 1))): one base,
        // offsets 1 KB i
        u32x4 yo[IPP];
        {
          const uint32_t a = sbase + 16u * (uint32_t)(lane ^ ((lane >> 4) & (NCO - 1)));
          if constexpr (IPP == 4)
            asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
                         "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
                         "s_waitcnt lgkmcnt(0)"
                         : "=&v"(yo[0]), "=&v"(yo[1]), "=&v"(yo[2]), "=&v"(yo[3])
                         : "v"(a)
                         : "memory");
          else if constexpr (IPP == 2)
            asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(yo[0]), "=&v"(yo[1])
                         : "v"(a)
                         : "memory");
          else
            asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(yo[0]) : "v"(a) : "memory");
        }
#pragma unroll
        for (int ii = 0; ii < IPP; ++ii) {
          const int gi = 64 * (IPP * h + ii) + lane;
          const int row = gi / GPR;
          const u32x4 v = yo[ii];
          if (local0 + row < cpg) {
            TOut* __restrict__ yr = static_cast<TOut*>(p.y) + b * p.y_sb + (g * cpg + local0 + row) * p.y_sd;
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(yr + w0) + gi % GPR);
          }
        }
      }
      if (wave_live) carry_ops += NCO;  // exactly NCO store instructions were issued
    } else if (live) {
      TOut* __restrict__ y = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
      store_seg<kK>(y, t0, L, false, yv);
    }
    if constexpr (VEC && GATE) {
      if (w + 1 < nwin) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        x_copy(zrow, w + 1, xz);
        carry_ops += NCI;
      }
    }
  }
  // the state after the last step (steps past L are the identity), carried by the row's last
  // lane into its pair slots
  if (SIO && p.h_final && live) {
    float* hf = p.h_final + b * p.hf_sb + d * p.hf_sd;
    for (int pp = jl; pp < P; pp += LPC) {
      const float4 pv = mypar[pp];
      hf[2 * pp] = pv.z;
      if (2 * pp + 1 < N) hf[2 * pp + 1] = pv.w;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Few rows, long sequences: several windows of a channel in flight ("window slots").
//
// When the (batch, channel) rows fit one round of one wave per SIMD (batch x channels <= 4 x CU
// count, e.g. the 1024 rows of a layer of a million steps), the kernel above gives each row one
// wave, which walks its windows in order: one wave per SIMD, and a wave on its own issues at
// best one instruction every few clocks.  Here each channel gets kSlots waves.  Slot k takes
// windows k, k + kSlots, k + 2 kSlots, ..., two states per step (Ns = ceil(N / 2) steps per
// window); the state at the end of window w (state n) is the carried state of window w + 1
// (state n), which belongs to the next slot.  The slots therefore run skewed: slot k handles
// pair np of its r-th window at step r Ns + np + k D (the skew D with 1 <= D <= (Ns - 1) / 2),
// so the carried states it reads were written D steps earlier by slot k - 1 (for slot 0:
// Ns - 2 D steps earlier, by the last slot in the round before).  One LDS word per (channel,
// state) holds them, and each wave publishes the steps it has completed: a wave waits only for
// the wave that writes the carried states it reads, which is normally D steps ahead.  Every
// write of a word is read by the next slot before the following write (each writer has itself
// waited, through the chain of slots, for the reader of the previous value).  No exp is
// evaluated twice; this is the associative scan's carry between chunks (study notes, history:
// the work-efficient parallel scan; bqwf.cn survey, section 2.2) with the chunks' order kept by
// the schedule instead of a look-back.
//
// Each wave fetches its own lanes' steps of B and C (bf16) for the step's two states and widens
// them itself, so the waves of a block share nothing but the carried states: no shared staging
// and no barrier in the loop.  Both are copied direct-to-LDS into per-wave areas, lane j's 16
// steps of a state as two 16-byte words 1 KB apart (conflict-free reads): B of the next step as
// soon as this step's B is in registers, C of this step at its start (needed at the readouts).
// u and delta go through two per-wave LDS slots: at a window's first step the wave reads u and
// delta and copies the window's z into u's slot and the next window's delta into delta's; at the
// window's last step it reads z and copies the next window's u into u's slot.  y leaves through
// the C area.  Every wait on the copies is
// explicit (vmcnt retires a wave's memory operations in issue order), and every read of copied
// LDS is inline asm that waits for itself.  A block is kSlotCh channels x kSlots slots = 12
// waves (3 per SIMD).  Needs bf16 inputs, 16-byte aligned rows, L a multiple of 8 (the
// direct-to-LDS copies) and N >= 5 (the skew).
constexpr int kSlots = 3;                  // windows in flight per channel
constexpr int kSlotCh = 4;                 // channels per block
constexpr int kSlotWaves = kSlots * kSlotCh;

__device__ __forceinline__ void lds_write_f32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Set (never cleared by a kernel) when a bounded wait between the waves of a block ran out of
// polls; read and cleared by the host (take_spin_error).  One per device.
__device__ int g_spin_error;

// s_waitcnt vmcnt(n) for the counts the window-slot kernel uses (anything else waits for all).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define SS_W(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    SS_W(4) SS_W(6) SS_W(8) SS_W(10) SS_W(12)
#undef SS_W
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// A wave's published progress word, read now (not cached in a register: the asm is volatile)
// and made wave-uniform.
__device__ __forceinline__ uint32_t progress_one(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

// Timing stress (race detection): with `perturb` set, a wave sleeps a pseudo-random number of
// ~64-clock rounds at each step, 0-7, and now and then 64 (a wave held up for a whole step), a
// different pattern for every (block, wave, step).  The results must not change: each wave reads
// another's data only behind the waits above, whatever the order the waves arrive in.
__device__ __forceinline__ void perturb_wait(uint32_t perturb, int s, int wave) {
  uint32_t h = (uint32_t)s * 0x9E3779B1u ^ ((uint32_t)wave * 0x85EBCA6Bu) ^ (blockIdx.x * 0xC2B2AE35u) ^ perturb;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint32_t n = (h & 0x3F0u) == 0 ? 64u : (h & 7u);
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
}

// Poll until ready() or `limit` polls have failed; in the latter case record the failure in
// g_spin_error and return (the kernel goes on and ends; its results are then wrong, which the
// host reports).  A wait can therefore never hang the GPU.
template <typename F>
__device__ __forceinline__ void spin_until(F ready, uint32_t limit) {
  for (uint32_t i = 0; !ready(); ++i) {
    if (i >= limit) {
      if ((threadIdx.x & 63) == 0) atomicOr(&g_spin_error, 1);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// This lane's B words of the step's two states (16-byte LDS reads at bb + 0, 1, 2, 3 KB), and
// the states' A log2 e and carried states (LDS words at pa0, pa1, pc0, pc1), read and waited for
// in one statement (read through plain C++, the compiler would wait for every copy in flight
// first).
__device__ __forceinline__ void slot_reads(uint32_t bb, u32x4 (&bq)[4], uint32_t pa0, uint32_t pa1, uint32_t pc0,
                                           uint32_t pc1, float (&An)[2], float (&carry)[2]) {
  asm volatile(
      "ds_read_b32 %4, %9\n\tds_read_b32 %5, %10\n\tds_read_b32 %6, %11\n\tds_read_b32 %7, %12\n\t"
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(bq[2]), "=&v"(bq[3]), "=&v"(An[0]), "=&v"(An[1]), "=&v"(carry[0]),
        "=&v"(carry[1])
      : "v"(bb), "v"(pa0), "v"(pa1), "v"(pc0), "v"(pc1)
      : "memory");
}

// This lane's C words of one state (16-byte LDS reads at cb, cb + 1 KB).
__device__ __forceinline__ void c_reads(uint32_t cb, u32x4& c0, u32x4& c1) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(c0), "=&v"(c1)
               : "v"(cb)
               : "memory");
}

// A slot's place in its schedule: q = s - k D counts its steps (q < 0: not started), np = q mod
// Ns the step's pair of states (2 np, 2 np + 1) and w = (q div Ns) kSlots + k the window; ob and
// oc are the element offsets of its first B and C row's window (2 np B_sn + w W, likewise),
// kept up to date with additions.
struct SlotPos {
  int q, np;
  int64_t w, ob, oc;
};

template <typename TOut, bool GATE, int MODE>
__global__ __launch_bounds__(64 * kSlotWaves) __attribute__((amdgpu_waves_per_eu(3))) void diag_slots_kernel(
    ScanArgs p, int64_t nwin, int64_t blocks_per_bg, int skew, int nsteps, uint32_t spin_limit,
    uint32_t perturb) {
  using TIn = bf16_t;
  constexpr bool SIO = (MODE & kSIO) != 0, ZOH = (MODE & kZOH) != 0, TRAP = (MODE & kTRAP) != 0;
  constexpr bool CKPT = (MODE & kCKPT) != 0;
  constexpr bool PERT = (MODE & kPERT) != 0;          // the timing stress (perturb_wait)
  constexpr int W = 64 * kK;                         // steps per window
  constexpr int NCI = Seg<TIn>::kChunks;             // 16-byte copies per lane per input row
  constexpr int kSegWords = NCI * 256;
  constexpr int NCO = kK * (int)sizeof(TOut) / 16;   // 16-byte stores per lane of y
  constexpr int GPR = 64 * NCO;                      // 16-byte granules of y per window
  // per wave: u (then z) and delta of its slot's window (see above)
  __shared__ __attribute__((aligned(16))) uint32_t xin[kSlotWaves][2][kSegWords];
  // per wave: B of the step's two states (words 0-511, 512-1023), then C of them (1024-2047);
  // lane j's 16 steps of a state at words 4 j (8 steps) and 256 + 4 j of its 512
  __shared__ __attribute__((aligned(16))) uint32_t bc[kSlotWaves][2048];
  // steps completed by each wave (wave k kSlotCh + c)
  __shared__ uint32_t prog[kSlotWaves];
  // [kSlotCh][N] A_n log2 e of the block's channels, then [kSlotCh][N] their carried states
  extern __shared__ float sp[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k = wave / kSlotCh;    // slot
  const int c = wave % kSlotCh;    // channel of the block
  const int64_t L = p.L;
  const int N = p.N;
  const int Ns = (N + 1) / 2;      // steps per window
  const int64_t bg = blockIdx.x / blocks_per_bg, blk = blockIdx.x % blocks_per_bg;
  const int64_t b = bg / p.groups, g = bg % p.groups;
  const int64_t cpg = p.chan_per_group;
  const int64_t local = blk * kSlotCh + c;
  const bool live = local < cpg;                      // (else a copy of a valid channel, not stored)
  const int64_t d = g * cpg + (live ? local : cpg - 1);
  const int64_t hd = d / p.chan_per_head;
  const TIn* urow = static_cast<const TIn*>(p.u) + b * p.u_sb + d * p.u_sd;
  const TIn* drow = static_cast<const TIn*>(p.delta) + b * p.dl_sb + hd * p.dl_sh;
  const TIn* zrow = GATE ? static_cast<const TIn*>(p.z) + b * p.z_sb + d * p.z_sd : nullptr;
  float bias = p.bias ? p.bias[hd] : 0.f;
  float Dd = p.D ? p.D[p.d_per_head ? hd : d] : 0.f;
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(bias), "+v"(Dd));
  const TIn* Bg = static_cast<const TIn*>(p.B) + b * p.B_sb + g * p.B_sg;
  const TIn* Cg = static_cast<const TIn*>(p.C) + b * p.C_sb + g * p.C_sg;
  if (k == 0) {
    // the carried state starts at the caller's initial state, or at zero
    const float* Ar = p.A + d * p.A_sd;
    const float* hi = (SIO && p.h_init) ? p.h_init + b * p.hi_sb + d * p.hi_sd : nullptr;
    for (int n = lane; n < N; n += 64) {
      sp[c * N + n] = Ar[n] * kLog2e;
      sp[(kSlotCh + c) * N + n] = hi ? hi[n] : 0.f;
    }
  }
  if (lane == 0) prog[wave] = 0;
  const uint32_t pa0 = lds_addr(sp + c * N);                // this channel's A log2 e
  const uint32_t pc0 = lds_addr(sp + (kSlotCh + c) * N);    // this channel's carried states
  // the wave that writes the carried states this wave reads (the previous slot's, same channel)
  const uint32_t prog_prev = lds_addr(&prog[((k + kSlots - 1) % kSlots) * kSlotCh + c]);
  const uint32_t prog_mine = lds_addr(&prog[wave]);
  uint32_t* xu = xin[wave][0];
  uint32_t* xd = xin[wave][1];
  const uint32_t bcb = lds_addr(&bc[wave][0]) + 16u * (uint32_t)lane;   // this lane's B words
  const uint32_t ccb = bcb + 4096u;                                      // and C words
  auto x_copy = [&](const TIn* row, int64_t w, uint32_t* slot) {
    seg_dma<TIn>(row, w * W + (int64_t)lane * kK, L, slot);
  };

  auto pos_at = [&](int s) {
    SlotPos ps;
    ps.q = s - k * skew;
    const int r = ps.q >= 0 ? ps.q / Ns : 0;
    ps.np = ps.q >= 0 ? ps.q - r * Ns : 0;
    ps.w = (int64_t)r * kSlots + k;
    ps.ob = 2 * ps.np * p.B_sn + ps.w * W;
    ps.oc = 2 * ps.np * p.C_sn + ps.w * W;
    return ps;
  };
  // from the last pair of a window to the next window's first
  const int64_t wrap_b = (int64_t)kSlots * W - 2 * (int64_t)Ns * p.B_sn;
  const int64_t wrap_c = (int64_t)kSlots * W - 2 * (int64_t)Ns * p.C_sn;
  auto advance = [&](SlotPos& ps) {
    if (++ps.q > 0) {
      ps.ob += 2 * p.B_sn;
      ps.oc += 2 * p.C_sn;
      if (++ps.np == Ns) {
        ps.np = 0;
        ps.w += kSlots;
        ps.ob += wrap_b;
        ps.oc += wrap_c;
      }
    }
  };
  // B (or C) of a position's two states into this wave's area at word `dst`: per state two
  // direct-to-LDS buffer copies through a resource over the window's part of the row, so that
  // lane j's offsets (32 j and 32 j + 16 bytes; an instruction offset would move the LDS
  // destination too) never change and the addressing is scalar; lane j's steps 16 j .. 16 j + 7
  // land at word 4 j of the state's 512, the next 8 at 256 + 4 j.  Steps past L lie outside the
  // resource and read as zero (L is a multiple of 8: no copy straddles the end); a state >= N,
  // or a slot without a window there, copies nothing (a resource of no bytes).
  const uint32_t lane_off = 32u * (uint32_t)lane, lane_off2 = lane_off + 16u;
  auto copy_pair = [&](const SlotPos& ps, const TIn* base, int64_t off, int64_t sn, int dst) {
    const bool act = ps.q >= 0 && ps.w < nwin;
    const int64_t rem = L - ps.w * W;
    const uint32_t bytes = act ? (uint32_t)(rem < W ? rem : W) * (uint32_t)sizeof(TIn) : 0u;
    const bool two = 2 * ps.np + 1 < N;
    const __amdgpu_buffer_rsrc_t r0 =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<TIn*>(act ? base + off : base), (short)0, (int)bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<TIn*>(act && two ? base + off + sn : base), (short)0, two ? (int)bytes : 0, 0x00020000);
    auto* l = (__attribute__((address_space(3))) uint32_t*)&bc[wave][dst];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, l, 16, lane_off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r0, l + 256, 16, lane_off2, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, l + 512, 16, lane_off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r1, l + 768, 16, lane_off2, 0, 0, 0);
  };

  // preamble: each slot's first window of u and delta, and its first step's B
  SlotPos cur = pos_at(0), nxt = pos_at(1);
  if (k < nwin) {
    x_copy(urow, k, xu);
    x_copy(drow, k, xd);
  }
  copy_pair(cur, Bg, cur.ob, p.B_sn, 0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  float dt[kK], wv[kK], yv[kK];
  float sdt = 0.f;
#pragma unroll
  for (int j = 0; j < kK; ++j) dt[j] = wv[j] = yv[j] = 0.f;
  // memory operations the previous step issued after its copy of this step's B (its y stores;
  // -1 for an unknown number)
  int after = 0;

  // one state of the step: lane pass from B words bw, the row's scan from the carried state, C
  // words from LDS (landed), the readout into yv; returns the window's end state (lane 63)
  // (ck: this state's checkpoint 512 steps into the window, or nullptr)
  auto one_state = [&](const uint32_t (&bw)[8], float An, float carry, uint32_t cwaddr, float* ck) {
    float av[kK], bv[kK];
#pragma unroll
    for (int j = 0; j < kK; ++j) av[j] = __builtin_amdgcn_exp2f(dt[j] * An);
    if constexpr (ZOH) {
      // u B times (exp(dt A) - 1) / A, from the decays just computed
      const float Anl = An * kLn2f, rA = __builtin_amdgcn_rcpf(Anl);
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        const float Bj = (j & 1) ? bf16_hi(bw[j / 2]) : bf16_lo(bw[j / 2]);
        bv[j] = zoh_coef(dt[j], dt[j] * Anl, av[j], rA) * wv[j] * Bj;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kK; ++j) bv[j] = wv[j] * ((j & 1) ? bf16_hi(bw[j / 2]) : bf16_lo(bw[j / 2]));
    }
    // the lane's steps from a zero state (the first step's decay multiplies zero)
    float h = bv[0];
#pragma unroll
    for (int j = 1; j < kK; ++j) h = fmaf(av[j], h, bv[j]);
    // lane aggregate (decay over the lane's steps, state from zero), then the row's scan from
    // the carried state
    h = row_incoming_state(__builtin_amdgcn_exp2f(sdt * An), h, carry);
    // (lane 32's incoming state is the state 512 steps into the window)
    if (CKPT && ck && lane == 32) *ck = h;
    u32x4 c0, c1;
    c_reads(cwaddr, c0, c1);
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int j = 0; j < kK; ++j) {
      const float Cj = (j & 1) ? bf16_hi(cw[j / 2]) : bf16_lo(cw[j / 2]);
      h = fmaf(av[j], h, bv[j]);
      if constexpr (TRAP) yv[j] = fmaf(Cj, fmaf(-0.5f, bv[j], h), yv[j]);
      else yv[j] = fmaf(Cj, h, yv[j]);
    }
    return h;
  };

  for (int s = 0; s < nsteps; ++s) {
    if constexpr (PERT) perturb_wait(perturb, s, wave);
    const bool act = cur.q >= 0 && cur.w < nwin;
    const int np = cur.np;
    const int64_t w = cur.w;
    const int64_t w0 = w * W;
    const int64_t t0 = w0 + (int64_t)lane * kK;
    const bool full = w0 + W <= L;
    const bool epi = act && np == Ns - 1;
    // this step's C; then everything issued before it has landed except what the previous step
    // issued after its copy of this step's B (its y stores and u copy) -- all of it at a window's
    // first step, whose u was copied at the previous step
    copy_pair(cur, Cg, cur.oc, p.C_sn, 1024);
    if (after == 0 || (act && np == 0)) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else wait_vmcnt(after < 0 ? 0 : after + 4);
    after = 0;
    int issued = 0;   // memory operations issued after this step's C copies, before its readouts
    u32x4 bq[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    float An[2] = {0.f, 0.f}, carry[2] = {0.f, 0.f};
    const int n0 = 2 * np;
    const bool two = n0 + 1 < N;
    if (act) {
      if (np == 0) {
        // the window's step sizes from u and delta (copied one window ago)
        Seg<TIn> su, sd;
        seg_read<TIn>(xu, lane, su);
        seg_read<TIn>(xd, lane, sd);
#pragma unroll
        for (int j = 0; j < kK; ++j) dt[j] = seg_get<TIn>(sd, j) + bias;
        if (p.softplus) {
#pragma unroll
          for (int j = 0; j < kK; ++j) dt[j] = softplus_fast(dt[j]);
        }
        if (!full) {
          // steps past the end are the identity (a = 1, b = 0); rem is 0, 8 or at least 16 (t0
          // and L are multiples of 8), so whole words of u are in or out
          const int rem = (int)(L - t0 < 0 ? 0 : (L - t0 > kK ? kK : L - t0));   // steps inside L
#pragma unroll
          for (int j = 0; j < kK; ++j) dt[j] = j < rem ? dt[j] : 0.f;
#pragma unroll
          for (int i = 0; i < kK / 2; ++i) su.w[i] = 2 * i < rem ? su.w[i] : 0u;
        }
        sdt = 0.f;
#pragma unroll
        for (int j = 0; j < kK; ++j) {
          const float uu = seg_get<TIn>(su, j);
          wv[j] = ZOH ? uu : dt[j] * uu;   // (zero-order hold: u, its coefficient already holds dt)
          yv[j] = Dd * uu;
          sdt += dt[j];
        }
        // the window's z into u's slot, the slot's next window's delta into delta's
        if constexpr (GATE) {
          x_copy(zrow, w, xu);
          issued += NCI;
        }
        if (w + kSlots < nwin) {
          x_copy(drow, w + kSlots, xd);
          issued += NCI;
        }
      }
      // the carried states of this step's pair were written (by the previous slot) D steps ago,
      // or Ns - 2 D steps ago for slot 0 (by the last slot, in the round before); the first
      // window starts from the initial state
      if (w > 0) {
        const int src = k ? s - skew : s - Ns + (kSlots - 1) * skew;
        spin_until([&] { return progress_one(prog_prev) >= (uint32_t)(src + 1); }, spin_limit);
      }
      const int n1 = two ? n0 + 1 : n0;
      slot_reads(bcb, bq, pa0 + 4u * (uint32_t)n0, pa0 + 4u * (uint32_t)n1, pc0 + 4u * (uint32_t)n0,
                 pc0 + 4u * (uint32_t)n1, An, carry);
    }
    // the next step's B into the area just read
    copy_pair(nxt, Bg, nxt.ob, p.B_sn, 0);
    issued += 4;
    if (act) {
      // this step's C has landed once at most what was issued after it (z, the u and delta
      // copies, the next step's B) is in flight
      wait_vmcnt(issued);
      // the backward's checkpoints: the window's start (the carried states) and 512 steps in
      float* ck0 = nullptr;
      if (CKPT && live) {
        float* ck = p.ckpt + b * p.ck_sb + d * p.ck_sd + (2 * w) * N + n0;
        if (lane == 0) {
          ck[0] = carry[0];
          if (two) ck[1] = carry[1];
        }
        if (2 * w + 1 < p.ckpt_nwin) ck0 = ck + N;
      }
      {
        const uint32_t bw[8] = {bq[0].x, bq[0].y, bq[0].z, bq[0].w, bq[1].x, bq[1].y, bq[1].z, bq[1].w};
        const float h = one_state(bw, An[0], carry[0], ccb, ck0);
        // the window's end state carries state n into the next window (the next slot)
        if (lane == 63) lds_write_f32(pc0 + 4u * (uint32_t)n0, h);
      }
      if (two) {
        const uint32_t bw[8] = {bq[2].x, bq[2].y, bq[2].z, bq[2].w, bq[3].x, bq[3].y, bq[3].z, bq[3].w};
        const float h = one_state(bw, An[1], carry[1], ccb + 2048u, ck0 ? ck0 + 1 : nullptr);
        if (lane == 63) lds_write_f32(pc0 + 4u * (uint32_t)(n0 + 1), h);
      }

      if (epi) {
        // epilogue: gate (z copied at the window's first step), then y through the C area (read
        // above), stored; then the slot's next window's u into u's slot
        if constexpr (GATE) {
          Seg<TIn> sz;
          seg_read<TIn>(xu, lane, sz);
#pragma unroll
          for (int j = 0; j < kK; ++j) yv[j] *= silu_fast(seg_get<TIn>(sz, j));
        }
        if (full) {
          // each store instruction writes whole runs of consecutive y: lane granule cc (steps
          // 4 cc.. of a f32 lane, 8 cc.. of a bf16 lane) is granule gi = NCO lane + cc of the
          // window, kept at gi ^ ((gi >> 4) & (NCO - 1)) so that neither the writes nor the reads
          // conflict on banks; store instruction ii has lane l take granule 64 ii + l
          const uint32_t sbase = lds_addr(&bc[wave][1024]);
          TOut* __restrict__ yr = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
#pragma unroll
          for (int cc = 0; cc < NCO; ++cc) {
            u32x4 gr;
            if constexpr (sizeof(TOut) == 4) {
              gr = u32x4{__float_as_uint(yv[4 * cc]), __float_as_uint(yv[4 * cc + 1]), __float_as_uint(yv[4 * cc + 2]),
                         __float_as_uint(yv[4 * cc + 3])};
            } else {
              uint32_t wd[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                wd[e] = f32_to_bf16_bits(yv[8 * cc + 2 * e]) | (f32_to_bf16_bits(yv[8 * cc + 2 * e + 1]) << 16);
              gr = u32x4{wd[0], wd[1], wd[2], wd[3]};
            }
            const int gi = NCO * lane + cc;
            const uint32_t a = sbase + 16u * (uint32_t)(gi ^ ((gi >> 4) & (NCO - 1)));
            asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(gr) : "memory");
          }
          u32x4 yo[NCO];
          {
            const uint32_t a = sbase + 16u * (uint32_t)(lane ^ ((lane >> 4) & (NCO - 1)));
            if constexpr (NCO == 4)
              asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
                           "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
                           "s_waitcnt lgkmcnt(0)"
                           : "=&v"(yo[0]), "=&v"(yo[1]), "=&v"(yo[2]), "=&v"(yo[3])
                           : "v"(a)
                           : "memory");
            else
              asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                           : "=&v"(yo[0]), "=&v"(yo[1])
                           : "v"(a)
                           : "memory");
          }
          if (live) {
#pragma unroll
            for (int ii = 0; ii < NCO; ++ii)
              __builtin_nontemporal_store(yo[ii], reinterpret_cast<u32x4*>(yr + w0) + (64 * ii + lane) % GPR);
            after = NCO;
          }
        } else if (live) {
          TOut* __restrict__ y = static_cast<TOut*>(p.y) + b * p.y_sb + d * p.y_sd;
          store_seg<kK>(y, t0, L, false, yv);
          after = -1;   // an unknown number of element stores
        }
        if (w + kSlots < nwin) {
          x_copy(urow, w + kSlots, xu);
          if (after >= 0) after += NCI;
        }
      }
    }
    // this wave's LDS writes (the carried states, the y staging) are done; then it says so
    asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(prog_mine), "v"((uint32_t)(s + 1)) : "memory");
    advance(cur);
    advance(nxt);
  }
  // the state after the last step (steps past L are the identity)
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (SIO && p.h_final && live && k == 0) {
    float* hf = p.h_final + b * p.hf_sb + d * p.hf_sd;
    for (int n = lane; n < N; n += 64) hf[n] = sp[(kSlotCh + c) * N + n];
  }
}

// The window-slot kernel serves few rows (at most one round of one wave per SIMD) with at least
// kSlots windows, bf16 inputs in 16-byte aligned rows and N >= 5.
bool slots_path(const ScanArgs& a) {
#ifdef SS_DIAG_NO_SLOTS
  return false;
#else
  return a.in_bf16 && a.vec && a.L % 8 == 0 && a.N >= 5 &&
         a.batch * a.channels <= (int64_t)kWaves * cu_count() && (a.L + 64 * kK - 1) / (64 * kK) >= kSlots;
#endif
}

template <typename TOut>
hipError_t launch_slots(const ScanArgs& a, hipStream_t s) {
  if (a.ckpt && a.ck_sd == 0) {
    // the dense checkpoint layout
    ScanArgs c = a;
    c.ck_sd = a.ckpt_nwin * a.N;
    c.ck_sb = a.channels * c.ck_sd;
    return launch_slots<TOut>(c, s);
  }
  constexpr int64_t W = 64 * kK;
  const int64_t nwin = (a.L + W - 1) / W;
  const int ns = (a.N + 1) / 2;            // steps per window (two states a step)
  const int skew = std::max(1, ns / 3);    // <= (ns - 1) / 2 for ns >= 3
  int64_t steps = 0;
  for (int k = 0; k < kSlots && k < nwin; ++k) {
    const int64_t windows = (nwin - k + kSlots - 1) / kSlots;
    steps = std::max(steps, windows * ns + (int64_t)k * skew);
  }
  const int64_t blocks_per_bg = (a.chan_per_group + kSlotCh - 1) / kSlotCh;
  const int64_t blocks = a.batch * a.groups * blocks_per_bg;
  const size_t dyn = sizeof(float) * 2 * kSlotCh * a.N;
  const dim3 grid((unsigned)blocks), block(64 * kSlotWaves);
  // polls of a wait between waves before it gives up (each poll sleeps ~64 clocks: ~0.5 s in
  // all, against ~1 us per step); SS_SPIN_LIMIT in the environment lowers it, so that tests can
  // force the failure path
  uint32_t spin_limit = 1u << 24;
  if (const char* e = getenv("SS_SPIN_LIMIT")) spin_limit = (uint32_t)strtoul(e, nullptr, 10);
  // SS_PERTURB=<nonzero seed> in the environment turns on the timing stress (perturb_wait), a
  // compile-time variant of the plain and the checkpointing kernels (other modes run without it)
  uint32_t perturb = 0;
  if (const char* e = getenv("SS_PERTURB")) perturb = (uint32_t)strtoul(e, nullptr, 10);
  int mode = ((a.h_init || a.h_final || a.zoh || a.trap) ? kSIO : 0) | (a.zoh ? kZOH : 0) | (a.trap ? kTRAP : 0) |
             (a.ckpt ? kCKPT : 0);
  if (perturb && (mode == 0 || mode == kCKPT)) mode |= kPERT;
#define SS_M(G, M)                                                                                          \
  case M:                                                                                                   \
    hipLaunchKernelGGL((diag_slots_kernel<TOut, G, M>), grid, block, dyn, s, a, nwin, blocks_per_bg, skew,  \
                       (int)steps, spin_limit, perturb);                                                    \
    break;
#define SS_LAUNCH(G)                                                                                        \
  switch (mode) {                                                                                           \
    SS_M(G, 0) SS_M(G, kSIO) SS_M(G, kSIO | kZOH) SS_M(G, kSIO | kTRAP) SS_M(G, kSIO | kZOH | kTRAP)        \
    SS_M(G, kPERT)                                                                                          \
    default: return hipErrorInvalidValue;                                                                   \
  }
  if (mode & kCKPT) {
    // (the backward's recompute: no gate, f32 y; an initial state only as a sequence segment)
    if (a.z || sizeof(TOut) != 4 || a.h_final || a.ck_sb <= 0 || a.ck_sd <= 0) return hipErrorInvalidValue;
    if (mode & kSIO)
      hipLaunchKernelGGL((diag_slots_kernel<TOut, false, kSIO | kCKPT>), grid, block, dyn, s, a, nwin, blocks_per_bg,
                         skew, (int)steps, spin_limit, perturb);
    else if (mode & kPERT)
      hipLaunchKernelGGL((diag_slots_kernel<TOut, false, kCKPT | kPERT>), grid, block, dyn, s, a, nwin, blocks_per_bg,
                         skew, (int)steps, spin_limit, perturb);
    else
      hipLaunchKernelGGL((diag_slots_kernel<TOut, false, kCKPT>), grid, block, dyn, s, a, nwin, blocks_per_bg, skew,
                         (int)steps, spin_limit, perturb);
  } else if (a.z) {
    SS_LAUNCH(true);
  } else {
    SS_LAUNCH(false);
  }
#undef SS_LAUNCH
#undef SS_M
  return hipGetLastError();
}


// ---- Sequence segments for few rows with long sequences (the window-slot path, one batch row).
// With fewer (batch, channel) rows than four per CU the window slots leave CUs idle.  The row's
// steps are then cut into S segments of equal length, each run by the window-slot kernel as a
// row of its own (segment j as batch index j: every time row is contiguous, so its offset is j
// times the segment length), started from the state the segments before it hand over.  A
// pre-pass gives, per (channel, segment j < S - 1), the segment's end state from a zero state,
//   E_j[n] = sum_{t in seg j} (prod_{s = t+1 .. end} a_{s,n}) dt_t u_t B_{t,n},
// and its total step size T_j (its decay is 2^(A_n log2 e T_j)); a combine pass forms the state
// entering each segment, H(0) = h_init (or 0), H(j + 1) = 2^(A_n log2 e T_j) H(j) + E_j.
constexpr int kFsK = 8;                 // steps per lane of the pre-pass
constexpr int kFsW = 64 * kFsK;         // steps per pre-pass iteration

struct FwdSegs {
  int64_t seg_len;   // steps per segment
  int32_t nseg;      // segments (1: none)
  int32_t sub;       // pre-pass pieces per segment (the pre-pass and the combine work on pieces)
};

bool slots_path(const ScanArgs& a);

// Segments apply to the plain exponential-Euler forward (no zero-order hold or trapezoid; the
// backward's checkpointing recompute too) of one batch row with N <= 32 on the window-slot path: S the largest power of two with S
// rows per channel fitting one round of the slots (4 per CU), L a multiple of S windows and at
// least kSlots windows per segment.
FwdSegs fwd_seg_plan(const ScanArgs& a) {
  constexpr int64_t W = 64 * kK;
  FwdSegs f{a.L, 1, 1};
#ifdef SS_NO_FWD_SEGS
  return f;   // (an ablation build: no segments)
#endif
  if (a.batch != 1 || a.zoh || a.trap || (a.ckpt && a.h_final) || a.N > 32 || !slots_path(a) || a.channels <= 0)
    return f;
  const int64_t cap = (int64_t)kWaves * cu_count() / a.channels;
  int64_t S = 1;
  while (2 * S <= cap && a.L % (2 * S * W) == 0 && a.L / (2 * S * W) >= kSlots) S *= 2;
  if (S == 1) return f;
  // pieces: enough pre-pass waves for about four per SIMD (one wave per channel and piece)
  const int64_t seg = a.L / S, want = 16 * (int64_t)cu_count();
  int64_t m = 1;
  while (a.channels * (S * m - 1) < want && seg % (2 * m * kFsW) == 0) m *= 2;
  return FwdSegs{seg, (int32_t)S, (int32_t)m};
}

// One wave per (channel d, piece j < P - 1) of the row's P equal pieces (a segment's pre-pass is
// cut into pieces so that it has enough waves; the combine composes them): E_j[0..N) and T_j into
// segw[(d (P - 1) + j) (N + 1) + ..].  The piece is walked from its end, kFsW steps at a time; the product of the decays
// after step t is 2^(A_n log2 e (T_after + s_t)), T_after the step sizes of the iterations walked
// so far (carried as the factor dp = 2^(A_n log2 e T_after)) and s_t those after t inside the
// iteration (its total minus the prefix up to t).
template <int NS>
__global__ __launch_bounds__(256) void fwd_seg_kernel(ScanArgs p, int64_t plen, int npieces, float* __restrict__ segw) {
  using TIn = bf16_t;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= p.channels * (npieces - 1)) return;
  const int64_t d = gw / (npieces - 1);
  const int j = (int)(gw % (npieces - 1));
  const int64_t g = d / p.chan_per_group, hd = d / p.chan_per_head;
  const int N = p.N;
  const TIn* ur = static_cast<const TIn*>(p.u) + d * p.u_sd;
  const TIn* dr = static_cast<const TIn*>(p.delta) + hd * p.dl_sh;
  const TIn* Bg = static_cast<const TIn*>(p.B) + g * p.B_sg;
  const float bias = p.bias ? p.bias[hd] : 0.f;
  float A2[NS], acc[NS], dp[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    A2[n] = n < N ? p.A[d * p.A_sd + n] * kLog2e : 0.f;
    acc[n] = 0.f;
    dp[n] = 1.f;
  }
  const int64_t tb = (int64_t)j * plen;
  float stot = 0.f;
  for (int64_t i = plen / kFsW - 1; i >= 0; --i) {
    const int64_t t0 = tb + i * kFsW + (int64_t)lane * kFsK;   // (whole, aligned: the plan's L)
    const u32x4 rd = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dr + t0));
    const u32x4 ru = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ur + t0));
    const uint32_t wd[4] = {rd.x, rd.y, rd.z, rd.w}, wu[4] = {ru.x, ru.y, ru.z, ru.w};
    float cs[kFsK], wv[kFsK], run = 0.f;
#pragma unroll
    for (int k = 0; k < kFsK; ++k) {
      const float x = ((k & 1) ? bf16_hi(wd[k / 2]) : bf16_lo(wd[k / 2])) + bias;
      const float dt = p.softplus ? softplus_fast(x) : x;
      run += dt;
      cs[k] = run;
      wv[k] = dt * ((k & 1) ? bf16_hi(wu[k / 2]) : bf16_lo(wu[k / 2]));
    }
    // step sizes after each step inside the iteration: its total minus the prefix up to the step
    float inc = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    const float wtot = readlane_f(inc, 63);
    const float ex = inc - run;
#pragma unroll
    for (int k = 0; k < kFsK; ++k) cs[k] = wtot - (ex + cs[k]);
#pragma unroll
    for (int n0 = 0; n0 < NS; n0 += 4) {
      if (n0 < N) {
        u32x4 rb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          rb[q] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(Bg + (int64_t)(n0 + q < N ? n0 + q : N - 1) * p.B_sn + t0));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + q;
          if (n < N) {
            const uint32_t wb[4] = {rb[q].x, rb[q].y, rb[q].z, rb[q].w};
            float sacc = 0.f;
#pragma unroll
            for (int k = 0; k < kFsK; ++k)
              sacc = fmaf(__builtin_amdgcn_exp2f(A2[n] * cs[k]),
                          wv[k] * ((k & 1) ? bf16_hi(wb[k / 2]) : bf16_lo(wb[k / 2])), sacc);
            acc[n] = fmaf(dp[n], sacc, acc[n]);
            dp[n] *= __builtin_amdgcn_exp2f(A2[n] * wtot);
          }
        }
      }
    }
    stot += wtot;
  }
  float* out = segw + (d * (npieces - 1) + j) * (N + 1);
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    if (n < N) {
      float v = acc[n];
      v += __shfl_xor(v, 32);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 1);
      if (lane == 0) out[n] = v;
    }
  }
  if (lane == 0) out[N] = stot;
}

// The state entering each piece, [P][channels][N] into hv: one thread per (channel, state).
__global__ __launch_bounds__(256) void fwd_seg_combine(ScanArgs p, int npieces, const float* __restrict__ segw,
                                                       float* __restrict__ hv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int N = p.N;
  if (i >= p.channels * N) return;
  const int64_t d = i / N;
  const int n = (int)(i % N);
  const float A2 = p.A[d * p.A_sd + n] * kLog2e;
  float h = p.h_init ? p.h_init[d * p.hi_sd + n] : 0.f;
  hv[d * N + n] = h;
  for (int j = 0; j + 1 < npieces; ++j) {
    const float* e = segw + (d * (npieces - 1) + j) * (N + 1);
    h = fmaf(__builtin_amdgcn_exp2f(A2 * e[N]), h, e[n]);
    hv[((int64_t)(j + 1) * p.channels + d) * N + n] = h;
  }
}

int npairs_of(const ScanArgs& a) { return (a.N + 1) / 2; }

// Channels per wave: one while every row still gets its own wave in a single round of one
// block of four waves per CU (one channel per wave fits one such block per CU in LDS); beyond
// that two, which run three waves per SIMD.  Measured on workload-1-shaped rows: 1024 rows 0.023
// ms with one channel per wave against 0.039 with two; 1280 rows 0.043 against 0.039; 6144 rows
// 0.131 against 0.069.
int rows_of(const ScanArgs& a) {
#ifdef SS_DIAG_ROWS
  return SS_DIAG_ROWS;
#else
  return a.batch * a.channels > (int64_t)kWaves * cu_count() ? 2 : 1;
#endif
}

int64_t nwin_of(const ScanArgs& a, int rows) {
  const int64_t W = (64 / rows) * kK;
  return (a.L + W - 1) / W;
}

template <typename TIn, typename TOut, int ROWS>
hipError_t launch_r(const ScanArgs& a, hipStream_t s) {
  const int P = npairs_of(a);
  const int64_t nwin = nwin_of(a, ROWS);
  const int64_t chans_per_block = kWaves * ROWS;
  const int64_t blocks_per_bg = (a.chan_per_group + chans_per_block - 1) / chans_per_block;
  const int64_t blocks = a.batch * a.groups * blocks_per_bg;
  // every time row 16-byte aligned and L a whole number of 16-byte chunks: copied with
  // direct-to-LDS loads
  const bool vec = a.vec && a.L % (16 / (int64_t)sizeof(TIn)) == 0;
  const dim3 grid((unsigned)blocks), block(64 * kWaves);
  const size_t par_bytes = sizeof(float4) * kWaves * ROWS * P;   // the per-pair parameters
  // the plain forward, or (state in/out checked at run time) with state in/out, zero-order hold
  // and/or the trapezoidal rule
  const int mode = ((a.h_init || a.h_final || a.zoh || a.trap) ? kSIO : 0) | (a.zoh ? kZOH : 0) | (a.trap ? kTRAP : 0) |
                   (a.ckpt ? kCKPT : 0);
#define SS_M(G, V, M)                                                                                        \
  case M:                                                                                                    \
    hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, G, V, ROWS, M>), grid, block, par_bytes, s, a, P, nwin, blocks_per_bg); \
    break;
#define SS_LAUNCH(G, V)                                                                                      \
  switch (mode) {                                                                                            \
    SS_M(G, V, 0) SS_M(G, V, kSIO) SS_M(G, V, kSIO | kZOH) SS_M(G, V, kSIO | kTRAP)                          \
    SS_M(G, V, kSIO | kZOH | kTRAP)                                                                          \
    default: return hipErrorInvalidValue;                                                                    \
  }
  if (mode == kCKPT) {
    // (the backward's recompute: no gate, f32 y)
    if (a.z || sizeof(TOut) != 4) return hipErrorInvalidValue;
    if (vec) hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, false, true, ROWS, kCKPT>), grid, block, par_bytes, s, a, P, nwin, blocks_per_bg);
    else hipLaunchKernelGGL((diag_fwd_kernel<TIn, TOut, false, false, ROWS, kCKPT>), grid, block, par_bytes, s, a, P, nwin, blocks_per_bg);
  } else if (a.z) {
    if (vec) { SS_LAUNCH(true, true); } else { SS_LAUNCH(true, false); }
  } else {
    if (vec) { SS_LAUNCH(false, true); } else { SS_LAUNCH(false, false); }
  }
#undef SS_LAUNCH
#undef SS_M
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const ScanArgs& a, hipStream_t s) {
  return rows_of(a) == 2 ? launch_r<TIn, TOut, 2>(a, s) : launch_r<TIn, TOut, 1>(a, s);
}

}  // namespace

hipError_t take_spin_error(int* failed) {
  int v = 0;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_spin_error), sizeof(int));
  if (e == hipSuccess && v) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_spin_error), &zero, sizeof(int));
  }
  *failed = v;
  return e;
}

bool diag_slots_path(const ScanArgs& a) { return slots_path(a); }

int64_t diag_workspace_bytes(const ScanArgs& a) {
  const FwdSegs f = fwd_seg_plan(a);
  if (f.nseg <= 1) return 0;
  // the pre-pass's (N + 1) floats per (channel, piece but the last), the states entering the
  // pieces, and (with h_final) the segments' final states
  const int64_t P = (int64_t)f.nseg * f.sub;
  const int64_t segf = a.channels * (P - 1) * (a.N + 1);
  const int64_t st = (int64_t)a.channels * a.N;
  return 4 * (segf + P * st + (a.h_final ? f.nseg * st : 0));
}

hipError_t launch_diag(const ScanArgs& a, void* ws, hipStream_t s) {
  const FwdSegs f = fwd_seg_plan(a);
  if (f.nseg <= 1) return launch_diag(a, s);
  if (!ws) return hipErrorInvalidValue;
  const int P = f.nseg * f.sub;              // pre-pass pieces
  const int64_t piece = f.seg_len / f.sub;
  float* segw = static_cast<float*>(ws);
  float* hv = segw + a.channels * (P - 1) * (a.N + 1);
  float* hf = hv + (int64_t)P * a.channels * a.N;
  const int64_t waves = a.channels * (P - 1);
  if (a.N <= 16)
    hipLaunchKernelGGL(fwd_seg_kernel<16>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a, piece, P, segw);
  else
    hipLaunchKernelGGL(fwd_seg_kernel<32>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a, piece, P, segw);
  hipLaunchKernelGGL(fwd_seg_combine, dim3((unsigned)((a.channels * a.N + 255) / 256)), dim3(256), 0, s, a, P, segw, hv);
  // the segments as rows of their own: batch index = segment, each time row offset by the
  // segment's start
  ScanArgs v = a;
  v.batch = f.nseg;
  v.L = f.seg_len;
  v.u_sb = v.dl_sb = v.B_sb = v.C_sb = v.y_sb = f.seg_len;
  v.z_sb = a.z ? f.seg_len : 0;
  v.h_init = hv;                                   // the state entering piece j sub
  v.hi_sb = (int64_t)f.sub * a.channels * a.N;
  v.hi_sd = a.N;
  v.h_final = a.h_final ? hf : nullptr;
  v.hf_sb = a.channels * a.N;
  v.hf_sd = a.N;
  if (a.ckpt) {
    // segment s's checkpoints are the sequence's from 512-step window s seg_len / 512 on
    v.ckpt_nwin = f.seg_len / 512;
    v.ck_sb = v.ckpt_nwin * a.N;
    v.ck_sd = a.ckpt_nwin * a.N;
  }
  const hipError_t e = a.out_bf16 ? launch_slots<bf16_t>(v, s) : launch_slots<float>(v, s);
  if (e != hipSuccess || !a.h_final) return e;
  // the last segment's final state is the caller's
  return launch_state_copy(hf + (int64_t)(f.nseg - 1) * a.channels * a.N, 0, a.N, a.h_final, 0, a.hf_sd, 1,
                           a.channels, a.N, s);
}

hipError_t launch_diag(const ScanArgs& a, hipStream_t s) {
  if (slots_path(a)) return a.out_bf16 ? launch_slots<bf16_t>(a, s) : launch_slots<float>(a, s);
  if (a.in_bf16) return a.out_bf16 ? launch_t<bf16_t, bf16_t>(a, s) : launch_t<bf16_t, float>(a, s);
  return a.out_bf16 ? launch_t<float, bf16_t>(a, s) : launch_t<float, float>(a, s);
}

}  // namespace ss
