// ss_probe.hip -- ceiling probes of the MI355X (gfx950) that bound the scan kernels: the issue
// cost of the VALU instructions the diagonal scan is made of (f32 multiply, FMA, exp, DPP FMA),
// whether an exp issued by one wave overlaps FMAs issued by another, and the HBM rates of a
// streaming copy and a streaming read.  A measurement library (libssprobe.so), used by
// bench.py --probe; it computes nothing of the scan itself.
//
// VALU probes: every wave runs `iters` rounds of 32 instructions, each writing one of 8 registers
// from two registers it never writes, so no instruction waits for another; the host divides the
// kernel's duration (in clocks) by the instructions each SIMD issued.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Kind { kMul = 0, kFma = 1, kExp = 2, kFmaDpp = 3, kExpFma = 4, kExp3Fma = 5 };

// 32 instructions per round, cycling over the 8 destination registers; sources %8, %9 only.
#define SS_R4(A, B, C, D) A("%0") B("%1") C("%2") D("%3") A("%4") B("%5") C("%6") D("%7")
#define SS_MUL(R) "v_mul_f32 " R ", %8, %9\n"
#define SS_FMA(R) "v_fma_f32 " R ", %8, %9, %8\n"
#define SS_EXP(R) "v_exp_f32 " R ", %8\n"
#define SS_DPP(R) "v_mul_f32_dpp " R ", %8, %9 row_shr:1 row_mask:0xf bank_mask:0xf\n"
#define SS_OUTS "+v"(r0), "+v"(r1), "+v"(r2), "+v"(r3), "+v"(r4), "+v"(r5), "+v"(r6), "+v"(r7)

template <int KIND>
__global__ __launch_bounds__(256) void valu_probe_kernel(int iters, float seed, float* out, uint64_t* clk) {
  const float a = seed + (float)threadIdx.x * 1e-7f, b = 0.999f;
  float r0 = a, r1 = a, r2 = a, r3 = a, r4 = a, r5 = a, r6 = a, r7 = a;
  // the shader clock (s_memtime) against the constant 100 MHz reference (s_memrealtime) over
  // the first wave's loop: the clock the probe ran at
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0t = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    if constexpr (KIND == kMul)
      asm volatile(SS_R4(SS_MUL, SS_MUL, SS_MUL, SS_MUL) SS_R4(SS_MUL, SS_MUL, SS_MUL, SS_MUL)
                   SS_R4(SS_MUL, SS_MUL, SS_MUL, SS_MUL) SS_R4(SS_MUL, SS_MUL, SS_MUL, SS_MUL)
                   : SS_OUTS : "v"(a), "v"(b));
    else if constexpr (KIND == kFma)
      asm volatile(SS_R4(SS_FMA, SS_FMA, SS_FMA, SS_FMA) SS_R4(SS_FMA, SS_FMA, SS_FMA, SS_FMA)
                   SS_R4(SS_FMA, SS_FMA, SS_FMA, SS_FMA) SS_R4(SS_FMA, SS_FMA, SS_FMA, SS_FMA)
                   : SS_OUTS : "v"(a), "v"(b));
    else if constexpr (KIND == kExp)
      asm volatile(SS_R4(SS_EXP, SS_EXP, SS_EXP, SS_EXP) SS_R4(SS_EXP, SS_EXP, SS_EXP, SS_EXP)
                   SS_R4(SS_EXP, SS_EXP, SS_EXP, SS_EXP) SS_R4(SS_EXP, SS_EXP, SS_EXP, SS_EXP)
                   : SS_OUTS : "v"(a), "v"(b));
    else if constexpr (KIND == kFmaDpp)
      asm volatile("s_nop 1\n" SS_R4(SS_DPP, SS_DPP, SS_DPP, SS_DPP) SS_R4(SS_DPP, SS_DPP, SS_DPP, SS_DPP)
                   SS_R4(SS_DPP, SS_DPP, SS_DPP, SS_DPP) SS_R4(SS_DPP, SS_DPP, SS_DPP, SS_DPP)
                   : SS_OUTS : "v"(a), "v"(b));
    else if constexpr (KIND == kExpFma)   // 16 exps and 16 FMAs, alternating
      asm volatile(SS_R4(SS_EXP, SS_FMA, SS_EXP, SS_FMA) SS_R4(SS_EXP, SS_FMA, SS_EXP, SS_FMA)
                   SS_R4(SS_EXP, SS_FMA, SS_EXP, SS_FMA) SS_R4(SS_EXP, SS_FMA, SS_EXP, SS_FMA)
                   : SS_OUTS : "v"(a), "v"(b));
    else                                  // 8 exps and 24 FMAs, one exp in four
      asm volatile(SS_R4(SS_EXP, SS_FMA, SS_FMA, SS_FMA) SS_R4(SS_EXP, SS_FMA, SS_FMA, SS_FMA)
                   SS_R4(SS_EXP, SS_FMA, SS_FMA, SS_FMA) SS_R4(SS_EXP, SS_FMA, SS_FMA, SS_FMA)
                   : SS_OUTS : "v"(a), "v"(b));
  }
  // keep the results live (one store per thread)
  out[blockIdx.x * blockDim.x + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1t = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1t - r0t;
  }
}
#undef SS_OUTS
#undef SS_DPP
#undef SS_EXP
#undef SS_FMA
#undef SS_MUL
#undef SS_R4

// Streaming copy: dst[i] = src[i], 16 bytes per thread per iteration, grid-stride.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Streaming read: each thread xors what it reads and writes one word at the end.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ out,
                                                         int64_t n) {
  uint32_t acc = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Launch the VALU probe of `kind` (0 multiply, 1 FMA, 2 exp, 3 DPP multiply, 4 exps and FMAs
// alternating, 5 one exp in four FMAs) with `blocks` blocks of 256 threads, each wave running
// `iters` rounds of 32 independent instructions; `out` holds blocks * 256 floats, `clk` two
// counts over the first wave's loop (shader clocks, then 100 MHz reference ticks).  Returns a
// hipError_t.
int ssp_valu(int kind, int blocks, int iters, float* out, uint64_t* clk, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (kind) {
#define SS_K(K) \
  case K: hipLaunchKernelGGL(valu_probe_kernel<K>, dim3(blocks), dim3(256), 0, s, iters, 0.5f, out, clk); break;
    SS_K(kMul) SS_K(kFma) SS_K(kExp) SS_K(kFmaDpp) SS_K(kExpFma) SS_K(kExp3Fma)
#undef SS_K
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Copy n16 16-byte words from src to dst (device pointers) with `blocks` blocks of 256 threads.
int ssp_copy(const void* src, void* dst, int64_t n16, int blocks, void* stream) {
  hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return (int)hipGetLastError();
}

// Read n16 16-byte words of src; `out` holds blocks * 256 words.
int ssp_read(const void* src, uint32_t* out, int64_t n16, int blocks, void* stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), out, n16);
  return (int)hipGetLastError();
}

}  // extern "C"
