// ss_api.hip -- C ABI of libssscan.so: validation, dispatch, workspace (pooled, or static scratch).  See include/ss_scan.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/ss_scan.h"
#include "ss_launch.h"

namespace {

// flag bits every scan entry point knows (SS_DETERMINISTIC is satisfied by construction on the
// forward paths and rejected by the backward)
constexpr uint32_t kScanFlags = SS_DELTA_SOFTPLUS | SS_Z_GATE_SILU | SS_DETERMINISTIC | SS_ZOH | SS_TRAPEZOID;

bool present(const ss_tensor* t) { return t != nullptr && t->data != nullptr; }

int64_t esize(int32_t dt) { return dt == SS_BF16 ? 2 : 4; }

// Byte extent [lo, hi) touched by a strided tensor (strides non-negative, checked first).
void extent(const ss_tensor* t, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = 0;
  for (int i = 0; i < t->ndim; ++i) last += (t->shape[i] - 1) * t->stride[i];
  *lo = reinterpret_cast<uintptr_t>(t->data);
  *hi = *lo + (uintptr_t)((last + 1) * esize(t->dtype));
}

int64_t numel(const ss_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// passed by the caller: a descriptor with data, or one of no elements (whose data may be NULL)
bool given(const ss_tensor* t) {
  if (t == nullptr) return false;
  if (t->data != nullptr) return true;
  if (t->ndim < 1 || t->ndim > 4) return false;
  for (int i = 0; i < t->ndim; ++i)
    if (t->shape[i] == 0) return true;
  return false;
}

int check_basic(const ss_tensor* t, int ndim) {
  if (t->ndim != ndim) return SS_ERR_SHAPE;
  if (t->dtype != SS_F32 && t->dtype != SS_BF16) return SS_ERR_DTYPE;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return SS_ERR_SHAPE;
    if (t->stride[i] < 0) return SS_ERR_STRIDE;
  }
  if (t->stride[ndim - 1] != 1 && t->shape[ndim - 1] > 1) return SS_ERR_STRIDE;
  return SS_OK;
}

bool aligned16(const ss_tensor* t) {
  if (reinterpret_cast<uintptr_t>(t->data) % 16) return false;
  const int64_t es = esize(t->dtype);
  for (int i = 0; i + 1 < t->ndim; ++i)
    if (t->shape[i] > 1 && (t->stride[i] * es) % 16) return false;
  return true;
}

// Stream-ordered workspace from a memory pool the library owns on each device.  The pool keeps
// freed blocks (its release threshold is "never"), so a call repeated on a stream reuses the
// same memory without a device allocation.  SS_FAULT=alloc in the environment makes the
// allocation fail, so that the failure path (SS_ERR_HIP, nothing enqueued, y untouched) can be
// exercised.
constexpr int kMaxDevices = 64;

hipError_t ws_pool(hipMemPool_t* pool) {
  static std::mutex mu;
  static hipMemPool_t pools[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    if ((e = hipMemPoolCreate(&p, &props)) != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    if ((e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
      (void)hipMemPoolDestroy(p);
      return e;
    }
    pools[dev] = p;
  }
  *pool = pools[dev];
  return hipSuccess;
}

hipError_t ws_alloc(void** ws, size_t bytes, hipStream_t s) {
  const char* fault = getenv("SS_FAULT");
  if (fault && strcmp(fault, "alloc") == 0) return hipErrorOutOfMemory;
  hipMemPool_t pool;
  hipError_t e = ws_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(ws, bytes, pool, s);
}

// Scratch of ss_scan_fwd_noalloc: one static array per device, which the code object reserves
// when it is loaded on that device.  In host code `scratch` names a host-side stand-in, not
// device memory: kernels get the device address, looked up once per device (with that device
// current) and kept.
static __device__ __align__(256) uint8_t scratch[SS_NOALLOC_SCRATCH_BYTES];

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addrs[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addrs[dev] = p;
  }
  *ptr = addrs[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int ss_version(void) { return SS_VERSION; }

const char* ss_strerror(int code) {
  switch (code) {
    case SS_OK: return "ok";
    case SS_ERR_NULL: return "a required tensor or data pointer is NULL";
    case SS_ERR_DTYPE: return "unsupported dtype or dtype mix";
    case SS_ERR_SHAPE: return "inconsistent tensor shapes";
    case SS_ERR_STRIDE: return "innermost stride must be 1 and strides non-negative";
    case SS_ERR_FLAGS: return "unknown flag bits, or SS_Z_GATE_SILU without z";
    case SS_ERR_UNSUPPORTED:
      return "unsupported size (N must be 1..128; at most 2^31 steps per row; conv width 1..8)";
    case SS_ERR_ALIAS: return "an output (y, a final state) overlaps an input or another output";
    case SS_ERR_HIP: return "HIP runtime error";
    case SS_ERR_DEADLOCK:
      return "a bounded wait between the waves of a kernel ran out: results since the last check are wrong";
    case SS_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown error code";
  }
}

int ss_check(void* stream) {
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SS_ERR_HIP;
  if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
  int failed = 0;
  if (ss::take_spin_error(&failed) != hipSuccess) return SS_ERR_HIP;
  return failed ? SS_ERR_DEADLOCK : SS_OK;
}

}  // extern "C"

namespace {

bool overlaps(const ss_tensor* a, const ss_tensor* b) {
  if (!present(a) || !present(b) || numel(a) == 0 || numel(b) == 0) return false;
  uintptr_t alo, ahi, blo, bhi;
  extent(a, &alo, &ahi);
  extent(b, &blo, &bhi);
  return alo < bhi && blo < ahi;
}

// a state tensor [batch, channels, N] f32 (state index innermost)
int check_state(const ss_tensor* h, int64_t Bt, int64_t Dc, int64_t N) {
  int rc;
  if ((rc = check_basic(h, 3))) return rc;
  if (h->dtype != SS_F32) return SS_ERR_DTYPE;
  if (h->shape[0] != Bt || h->shape[1] != Dc || h->shape[2] != N) return SS_ERR_SHAPE;
  return SS_OK;
}

int scan_common(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                const ss_tensor* C, const ss_tensor* D, const ss_tensor* z, const ss_tensor* delta_bias,
                uint32_t flags, const ss_tensor* h_init, ss_tensor* h_final, ss_tensor* y, void* stream,
                bool noalloc) {
  if (!u || !delta || !A || !B || !C || !y) return SS_ERR_NULL;
  if (flags & ~kScanFlags) return SS_ERR_FLAGS;
  const bool gate = (flags & SS_Z_GATE_SILU) != 0;
  if (gate != given(z)) return SS_ERR_FLAGS;
  int rc;
  if ((rc = check_basic(u, 3)) || (rc = check_basic(delta, 3)) || (rc = check_basic(B, 4)) ||
      (rc = check_basic(C, 4)) || (rc = check_basic(y, 3)))
    return rc;
  if (A->ndim != 1 && A->ndim != 2) return SS_ERR_SHAPE;
  if ((rc = check_basic(A, A->ndim))) return rc;
  if (gate && (rc = check_basic(z, 3))) return rc;
  if (present(D) && (rc = check_basic(D, 1))) return rc;
  if (present(delta_bias) && (rc = check_basic(delta_bias, 1))) return rc;

  // dtypes: u, delta, B, C, z agree; A, D, bias are f32; y is f32 or bf16
  const int32_t idt = u->dtype;
  if (delta->dtype != idt || B->dtype != idt || C->dtype != idt || (gate && z->dtype != idt))
    return SS_ERR_DTYPE;
  if (A->dtype != SS_F32 || (present(D) && D->dtype != SS_F32) ||
      (present(delta_bias) && delta_bias->dtype != SS_F32))
    return SS_ERR_DTYPE;

  const int64_t Bt = u->shape[0], Dc = u->shape[1], L = u->shape[2];
  const int64_t H = delta->shape[1], G = B->shape[1], N = B->shape[2];
  if (delta->shape[0] != Bt || delta->shape[2] != L) return SS_ERR_SHAPE;
  if (B->shape[0] != Bt || B->shape[3] != L) return SS_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (C->shape[i] != B->shape[i]) return SS_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (y->shape[i] != u->shape[i] || (gate && z->shape[i] != u->shape[i])) return SS_ERR_SHAPE;
  if (H <= 0 || G <= 0 || (Dc > 0 && (Dc % H || Dc % G))) return SS_ERR_SHAPE;
  const bool scalar = A->ndim == 1;
  if (scalar ? A->shape[0] != H : (A->shape[0] != Dc || A->shape[1] != N)) return SS_ERR_SHAPE;
  if (present(D) && D->shape[0] != Dc && D->shape[0] != H) return SS_ERR_SHAPE;
  if (present(delta_bias) && delta_bias->shape[0] != H) return SS_ERR_SHAPE;
  if (N < 1 || N > 128) return SS_ERR_UNSUPPORTED;
  if (L > ((int64_t)1 << 31)) return SS_ERR_UNSUPPORTED;
  if (present(h_init) && (rc = check_state(h_init, Bt, Dc, N))) return rc;
  if (present(h_final) && (rc = check_state(h_final, Bt, Dc, N))) return rc;
  if (present(h_final) && overlaps(h_final, h_init)) return SS_ERR_ALIAS;
  if (Bt * Dc == 0) return SS_OK;  // nothing to compute

  // y must not overlap any input
  uintptr_t ylo, yhi;
  extent(y, &ylo, &yhi);
  const ss_tensor* ins[] = {u, delta, A, B, C, D, z, delta_bias, h_init};
  for (const ss_tensor* t : ins) {
    if (!present(t) || numel(t) == 0) continue;
    uintptr_t lo, hi;
    extent(t, &lo, &hi);
    if (lo < yhi && ylo < hi) return SS_ERR_ALIAS;
    if (overlaps(h_final, t)) return SS_ERR_ALIAS;
  }
  if (overlaps(h_final, y)) return SS_ERR_ALIAS;

  if (L == 0) {
    // no steps: the final state is the initial one (zero without h_init)
    if (!present(h_final)) return SS_OK;
    const float* hi = present(h_init) ? static_cast<const float*>(h_init->data) : nullptr;
    return ss::launch_state_copy(hi, hi ? h_init->stride[0] : 0, hi ? h_init->stride[1] : 0,
                                 static_cast<float*>(h_final->data), h_final->stride[0], h_final->stride[1], Bt,
                                 Dc, N, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SS_OK
               : SS_ERR_HIP;
  }
  if (!u->data || !delta->data || !A->data || !B->data || !C->data || !y->data) return SS_ERR_NULL;
  ss::ScanArgs a{};
  a.u = u->data;
  a.delta = delta->data;
  a.B = B->data;
  a.C = C->data;
  a.z = gate ? z->data : nullptr;
  a.A = static_cast<const float*>(A->data);
  a.D = present(D) ? static_cast<const float*>(D->data) : nullptr;
  a.bias = present(delta_bias) ? static_cast<const float*>(delta_bias->data) : nullptr;
  a.y = y->data;
  a.batch = Bt;
  a.channels = Dc;
  a.L = L;
  a.N = (int32_t)N;
  a.heads = (int32_t)H;
  a.groups = (int32_t)G;
  a.chan_per_head = (int32_t)(Dc / H);
  a.chan_per_group = (int32_t)(Dc / G);
  a.d_per_head = present(D) && D->shape[0] != Dc ? 1 : 0;
  a.softplus = (flags & SS_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SS_ZOH) ? 1 : 0;
  a.trap = (flags & SS_TRAPEZOID) ? 1 : 0;
  a.in_bf16 = idt == SS_BF16;
  a.out_bf16 = y->dtype == SS_BF16;
  a.vec = aligned16(u) && aligned16(delta) && aligned16(B) && aligned16(C) && aligned16(y) &&
          (!gate || aligned16(z));
  a.u_sb = u->stride[0];
  a.u_sd = u->stride[1];
  a.dl_sb = delta->stride[0];
  a.dl_sh = delta->stride[1];
  a.z_sb = gate ? z->stride[0] : 0;
  a.z_sd = gate ? z->stride[1] : 0;
  a.B_sb = B->stride[0];
  a.B_sg = B->stride[1];
  a.B_sn = B->stride[2];
  a.C_sb = C->stride[0];
  a.C_sg = C->stride[1];
  a.C_sn = C->stride[2];
  a.y_sb = y->stride[0];
  a.y_sd = y->stride[1];
  a.A_sd = scalar ? 0 : A->stride[0];
  a.h_init = present(h_init) ? static_cast<const float*>(h_init->data) : nullptr;
  a.h_final = present(h_final) ? static_cast<float*>(h_final->data) : nullptr;
  a.hi_sb = a.h_init ? h_init->stride[0] : 0;
  a.hi_sd = a.h_init ? h_init->stride[1] : 0;
  a.hf_sb = a.h_final ? h_final->stride[0] : 0;
  a.hf_sd = a.h_final ? h_final->stride[1] : 0;
  if (present(D) && D->stride[0] != 1 && D->shape[0] > 1) return SS_ERR_STRIDE;
  if (present(delta_bias) && delta_bias->stride[0] != 1 && delta_bias->shape[0] > 1) return SS_ERR_STRIDE;
  if (scalar && A->stride[0] != 1 && A->shape[0] > 1) return SS_ERR_STRIDE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  // diagonal decay: a workspace only when few long rows are cut into sequence segments; scalar
  // decay: stream-ordered workspace for B/C (and, on the matrix path, C B^T per chunk) in the
  // order the kernel reads them
  const bool mfma = scalar && ss::ssd_path(a);
  const int64_t wsb = !scalar ? ss::diag_workspace_bytes(a)
                      : mfma  ? ss::ssd_workspace_bytes(a)
                              : ss::scalar_workspace_floats(a) * (int64_t)sizeof(float);
  if (!scalar && wsb == 0) return ss::launch_diag(a, s) == hipSuccess ? SS_OK : SS_ERR_HIP;
  auto run = [&](void* ws) -> hipError_t {
    if (!scalar) return ss::launch_diag(a, ws, s);
    return mfma ? ss::launch_ssd(a, ws, s) : ss::launch_scalar(a, static_cast<float*>(ws), s);
  };
  void* ws = nullptr;
  if (noalloc) {
    // the static scratch: every byte the kernels read they write first, so nothing is cleared
    if (wsb > (int64_t)SS_NOALLOC_SCRATCH_BYTES) return SS_ERR_SCRATCH;
    if (scratch_address(&ws) != hipSuccess) {
      (void)hipGetLastError();
      return SS_ERR_HIP;
    }
    return run(ws) == hipSuccess ? SS_OK : SS_ERR_HIP;
  }
  if (ws_alloc(&ws, (size_t)wsb, s) != hipSuccess) {
    (void)hipGetLastError();
    return SS_ERR_HIP;
  }
  const hipError_t e = run(ws);
  const hipError_t f = hipFreeAsync(ws, s);
  return (e == hipSuccess && f == hipSuccess) ? SS_OK : SS_ERR_HIP;
}

}  // namespace

extern "C" {

int ss_scan_fwd(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                const ss_tensor* delta_bias, uint32_t flags, ss_tensor* y, void* stream) {
  return scan_common(u, delta, A, B, C, D, z, delta_bias, flags, nullptr, nullptr, y, stream, false);
}

int ss_scan_fwd_state(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                      const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                      const ss_tensor* delta_bias, uint32_t flags, const ss_tensor* h_init,
                      ss_tensor* h_final, ss_tensor* y, void* stream) {
  return scan_common(u, delta, A, B, C, D, z, delta_bias, flags, h_init, h_final, y, stream, false);
}

int ss_scan_fwd_noalloc(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                        const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                        const ss_tensor* delta_bias, uint32_t flags, const ss_tensor* h_init,
                        ss_tensor* h_final, ss_tensor* y, void* stream) {
  return scan_common(u, delta, A, B, C, D, z, delta_bias, flags, h_init, h_final, y, stream, true);
}

int ss_scan_step(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                 const ss_tensor* C, const ss_tensor* D, const ss_tensor* z,
                 const ss_tensor* delta_bias, uint32_t flags, ss_tensor* h, ss_tensor* y, void* stream) {
  if (!u || !delta || !A || !B || !C || !h || !y) return SS_ERR_NULL;
  if (flags & ~kScanFlags) return SS_ERR_FLAGS;
  const bool gate = (flags & SS_Z_GATE_SILU) != 0;
  if (gate != given(z)) return SS_ERR_FLAGS;
  int rc;
  if ((rc = check_basic(u, 2)) || (rc = check_basic(delta, 2)) || (rc = check_basic(B, 3)) ||
      (rc = check_basic(C, 3)) || (rc = check_basic(y, 2)))
    return rc;
  if (A->ndim != 1 && A->ndim != 2) return SS_ERR_SHAPE;
  if ((rc = check_basic(A, A->ndim))) return rc;
  if (gate && (rc = check_basic(z, 2))) return rc;
  if (present(D) && (rc = check_basic(D, 1))) return rc;
  if (present(delta_bias) && (rc = check_basic(delta_bias, 1))) return rc;
  const int32_t idt = u->dtype;
  if (delta->dtype != idt || B->dtype != idt || C->dtype != idt || (gate && z->dtype != idt))
    return SS_ERR_DTYPE;
  if (A->dtype != SS_F32 || (present(D) && D->dtype != SS_F32) ||
      (present(delta_bias) && delta_bias->dtype != SS_F32))
    return SS_ERR_DTYPE;
  const int64_t Bt = u->shape[0], Dc = u->shape[1];
  const int64_t H = delta->shape[1], G = B->shape[1], N = B->shape[2];
  if (delta->shape[0] != Bt || B->shape[0] != Bt) return SS_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (C->shape[i] != B->shape[i]) return SS_ERR_SHAPE;
  for (int i = 0; i < 2; ++i)
    if (y->shape[i] != u->shape[i] || (gate && z->shape[i] != u->shape[i])) return SS_ERR_SHAPE;
  if (H <= 0 || G <= 0 || (Dc > 0 && (Dc % H || Dc % G))) return SS_ERR_SHAPE;
  const bool scalar = A->ndim == 1;
  if (scalar ? A->shape[0] != H : (A->shape[0] != Dc || A->shape[1] != N)) return SS_ERR_SHAPE;
  if (present(D) && D->shape[0] != Dc && D->shape[0] != H) return SS_ERR_SHAPE;
  if (present(delta_bias) && delta_bias->shape[0] != H) return SS_ERR_SHAPE;
  if (N < 1 || N > 128) return SS_ERR_UNSUPPORTED;
  if ((rc = check_state(h, Bt, Dc, N))) return rc;
  if (Bt * Dc == 0) return SS_OK;
  if (!u->data || !delta->data || !A->data || !B->data || !C->data || !y->data || !h->data) return SS_ERR_NULL;
  if (present(D) && D->stride[0] != 1 && D->shape[0] > 1) return SS_ERR_STRIDE;
  if (present(delta_bias) && delta_bias->stride[0] != 1 && delta_bias->shape[0] > 1) return SS_ERR_STRIDE;
  if (scalar && A->stride[0] != 1 && A->shape[0] > 1) return SS_ERR_STRIDE;
  // y and h are written: neither may overlap an input or the other
  const ss_tensor* ins[] = {u, delta, A, B, C, D, z, delta_bias};
  for (const ss_tensor* t : ins)
    if (overlaps(y, t) || overlaps(h, t)) return SS_ERR_ALIAS;
  if (overlaps(y, h)) return SS_ERR_ALIAS;

  ss::StepArgs a{};
  a.u = u->data;
  a.delta = delta->data;
  a.B = B->data;
  a.C = C->data;
  a.z = gate ? z->data : nullptr;
  a.A = static_cast<const float*>(A->data);
  a.D = present(D) ? static_cast<const float*>(D->data) : nullptr;
  a.bias = present(delta_bias) ? static_cast<const float*>(delta_bias->data) : nullptr;
  a.h = static_cast<float*>(h->data);
  a.y = y->data;
  a.batch = Bt;
  a.channels = Dc;
  a.N = (int32_t)N;
  a.heads = (int32_t)H;
  a.groups = (int32_t)G;
  a.chan_per_head = (int32_t)(Dc / H);
  a.chan_per_group = (int32_t)(Dc / G);
  a.scalar = scalar ? 1 : 0;
  a.zoh = (flags & SS_ZOH) ? 1 : 0;
  a.trap = (flags & SS_TRAPEZOID) ? 1 : 0;
  a.d_per_head = present(D) && D->shape[0] != Dc ? 1 : 0;
  a.softplus = (flags & SS_DELTA_SOFTPLUS) ? 1 : 0;
  a.in_bf16 = idt == SS_BF16;
  a.out_bf16 = y->dtype == SS_BF16;
  a.u_sb = u->stride[0];
  a.dl_sb = delta->stride[0];
  a.z_sb = gate ? z->stride[0] : 0;
  a.B_sb = B->stride[0];
  a.B_sg = B->stride[1];
  a.C_sb = C->stride[0];
  a.C_sg = C->stride[1];
  a.y_sb = y->stride[0];
  a.A_sd = scalar ? 0 : A->stride[0];
  a.h_sb = h->stride[0];
  a.h_sd = h->stride[1];
  return ss::launch_step(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SS_OK : SS_ERR_HIP;
}

// output gradient tensor: f32, the given shape, innermost stride 1
static int check_grad(const ss_tensor* t, int ndim, const int64_t* shape) {
  int rc;
  if ((rc = check_basic(t, ndim))) return rc;
  if (t->dtype != SS_F32) return SS_ERR_DTYPE;
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] != shape[i]) return SS_ERR_SHAPE;
  return SS_OK;
}

int ss_scan_bwd(const ss_tensor* u, const ss_tensor* delta, const ss_tensor* A, const ss_tensor* B,
                const ss_tensor* C, const ss_tensor* D, const ss_tensor* z, const ss_tensor* delta_bias,
                uint32_t flags, const ss_tensor* dy, ss_tensor* du, ss_tensor* ddelta, ss_tensor* dA,
                ss_tensor* dB, ss_tensor* dC, ss_tensor* dD, ss_tensor* dz, ss_tensor* ddelta_bias,
                void* stream) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return SS_ERR_NULL;
  if (flags & ~kScanFlags) return SS_ERR_FLAGS;
  const bool gate = (flags & SS_Z_GATE_SILU) != 0;
  if (gate != given(z)) return SS_ERR_FLAGS;
  int rc;
  if ((rc = check_basic(u, 3)) || (rc = check_basic(delta, 3)) || (rc = check_basic(B, 4)) ||
      (rc = check_basic(C, 4)) || (rc = check_basic(dy, 3)))
    return rc;
  if ((rc = check_basic(A, A->ndim == 2 ? 2 : 1))) return rc;
  if (gate && (rc = check_basic(z, 3))) return rc;
  if (present(D) && (rc = check_basic(D, 1))) return rc;
  if (present(delta_bias) && (rc = check_basic(delta_bias, 1))) return rc;
  const int32_t idt = u->dtype;
  if (delta->dtype != idt || B->dtype != idt || C->dtype != idt || (gate && z->dtype != idt)) return SS_ERR_DTYPE;
  if (A->dtype != SS_F32 || (present(D) && D->dtype != SS_F32) ||
      (present(delta_bias) && delta_bias->dtype != SS_F32))
    return SS_ERR_DTYPE;
  const int64_t Bt = u->shape[0], Dc = u->shape[1], L = u->shape[2];
  const int64_t H = delta->shape[1], G = B->shape[1], N = B->shape[2];
  if (delta->shape[0] != Bt || delta->shape[2] != L || B->shape[0] != Bt || B->shape[3] != L) return SS_ERR_SHAPE;
  for (int i = 0; i < 4; ++i)
    if (C->shape[i] != B->shape[i]) return SS_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if (dy->shape[i] != u->shape[i] || (gate && z->shape[i] != u->shape[i])) return SS_ERR_SHAPE;
  if (H <= 0 || G <= 0 || (Dc > 0 && (Dc % G || Dc % H))) return SS_ERR_SHAPE;
  const bool scalar = A->ndim == 1;
  if (scalar ? A->shape[0] != H : (A->shape[0] != Dc || A->shape[1] != N)) return SS_ERR_SHAPE;
  if (present(D) && D->shape[0] != Dc && D->shape[0] != H) return SS_ERR_SHAPE;
  if (present(delta_bias) && delta_bias->shape[0] != H) return SS_ERR_SHAPE;
  // the backward is written for the exponential-Euler rule, and its sums over channels and
  // batch are atomic adds (not reproducible to the last bit)
  if (flags & (SS_ZOH | SS_TRAPEZOID | SS_DETERMINISTIC)) return SS_ERR_UNSUPPORTED;
  if (N < 1 || N > 128) return SS_ERR_UNSUPPORTED;
  if (L > ((int64_t)1 << 31)) return SS_ERR_UNSUPPORTED;
  if (Dc > 0 && (Dc / G) % 4) return SS_ERR_UNSUPPORTED;
  if (dy->dtype != SS_F32 && dy->dtype != SS_BF16) return SS_ERR_DTYPE;
  const int64_t nD = present(D) ? D->shape[0] : Dc;
  const int64_t s_x[3] = {Bt, Dc, L}, s_dl[3] = {Bt, H, L}, s_bc[4] = {Bt, G, N, L}, s_a[2] = {Dc, N}, s_h[1] = {H},
                s_d[1] = {nD};
  if ((rc = check_grad(du, 3, s_x)) || (rc = check_grad(ddelta, 3, s_dl)) ||
      (rc = scalar ? check_grad(dA, 1, s_h) : check_grad(dA, 2, s_a)) || (rc = check_grad(dB, 4, s_bc)) ||
      (rc = check_grad(dC, 4, s_bc)))
    return rc;
  if (present(D) != given(dD)) return SS_ERR_NULL;   // dD exactly when D is given
  if (gate != given(dz)) return SS_ERR_NULL;         // dz exactly when the gate is on
  if (given(dD) && (rc = check_grad(dD, 1, s_d))) return rc;
  if (given(dz) && (rc = check_grad(dz, 3, s_x))) return rc;
  if (given(ddelta_bias) && (rc = check_grad(ddelta_bias, 1, s_h))) return rc;
  // outputs overlap neither the inputs nor each other
  const ss_tensor* ins[] = {u, delta, A, B, C, D, z, delta_bias, dy};
  ss_tensor* outs[] = {du, ddelta, dA, dB, dC, dD, dz, ddelta_bias};
  for (ss_tensor* o : outs) {
    for (const ss_tensor* t : ins)
      if (overlaps(o, t)) return SS_ERR_ALIAS;
    for (ss_tensor* o2 : outs)
      if (o2 != o && overlaps(o, o2)) return SS_ERR_ALIAS;
  }
  if (Bt * Dc == 0) return SS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0) {
    // no steps: the gradients of A, B, C, D and the bias are zero; du, ddelta, dz are empty
    float* zs[] = {static_cast<float*>(dA->data), present(D) ? static_cast<float*>(dD->data) : nullptr,
                   given(ddelta_bias) ? static_cast<float*>(ddelta_bias->data) : nullptr};
    const int64_t rws[] = {scalar ? 1 : Dc, 1, 1}, inn[] = {scalar ? H : N, nD, H},
                  st[] = {scalar ? 0 : dA->stride[0], 0, 0};
    for (int i = 0; i < 3; ++i)
      if (zs[i] && ss::launch_state_copy(nullptr, 0, 0, zs[i], 0, st[i], 1, rws[i], inn[i], s) != hipSuccess)
        return SS_ERR_HIP;
    return SS_OK;
  }
  if (!u->data || !delta->data || !A->data || !B->data || !C->data || !dy->data) return SS_ERR_NULL;
  if (present(D) && D->stride[0] != 1 && D->shape[0] > 1) return SS_ERR_STRIDE;
  if (present(delta_bias) && delta_bias->stride[0] != 1 && delta_bias->shape[0] > 1) return SS_ERR_STRIDE;

  ss::BwdArgs a{};
  a.u = u->data;
  a.delta = delta->data;
  a.B = B->data;
  a.C = C->data;
  a.z = gate ? z->data : nullptr;
  a.A = static_cast<const float*>(A->data);
  a.D = present(D) ? static_cast<const float*>(D->data) : nullptr;
  a.bias = present(delta_bias) ? static_cast<const float*>(delta_bias->data) : nullptr;
  a.dy = dy->data;
  a.du = static_cast<float*>(du->data);
  a.ddelta = static_cast<float*>(ddelta->data);
  a.dA = static_cast<float*>(dA->data);
  a.dB = static_cast<float*>(dB->data);
  a.dC = static_cast<float*>(dC->data);
  a.dD = given(dD) ? static_cast<float*>(dD->data) : nullptr;
  a.dz = gate ? static_cast<float*>(dz->data) : nullptr;
  a.dbias = given(ddelta_bias) ? static_cast<float*>(ddelta_bias->data) : nullptr;
  a.batch = Bt;
  a.channels = Dc;
  a.L = L;
  a.N = (int32_t)N;
  a.groups = (int32_t)G;
  a.chan_per_group = (int32_t)(Dc / G);
  a.heads = (int32_t)H;
  a.chan_per_head = (int32_t)(Dc / H);
  a.scalar = scalar ? 1 : 0;
  a.d_per_head = present(D) && nD != Dc ? 1 : 0;
  a.softplus = (flags & SS_DELTA_SOFTPLUS) ? 1 : 0;
  a.in_bf16 = idt == SS_BF16;
  a.dy_bf16 = dy->dtype == SS_BF16;
  a.vec = aligned16(u) && aligned16(delta) && aligned16(B) && aligned16(C) && aligned16(dy) &&
          (!gate || aligned16(z));
  a.u_sb = u->stride[0];
  a.u_sd = u->stride[1];
  a.dl_sb = delta->stride[0];
  a.dl_sh = delta->stride[1];
  a.z_sb = gate ? z->stride[0] : 0;
  a.z_sd = gate ? z->stride[1] : 0;
  a.B_sb = B->stride[0];
  a.B_sg = B->stride[1];
  a.B_sn = B->stride[2];
  a.C_sb = C->stride[0];
  a.C_sg = C->stride[1];
  a.C_sn = C->stride[2];
  a.A_sd = A->stride[0];
  a.dy_sb = dy->stride[0];
  a.dy_sd = dy->stride[1];
  a.du_sb = du->stride[0];
  a.du_sd = du->stride[1];
  a.dd_sb = ddelta->stride[0];
  a.dd_sh = ddelta->stride[1];
  a.dA_sd = dA->stride[0];
  a.dB_sb = dB->stride[0];
  a.dB_sg = dB->stride[1];
  a.dB_sn = dB->stride[2];
  a.dC_sb = dC->stride[0];
  a.dC_sg = dC->stride[1];
  a.dC_sn = dC->stride[2];
  a.dz_sb = gate ? dz->stride[0] : 0;
  a.dz_sd = gate ? dz->stride[1] : 0;

  void* ws = nullptr;
  const int64_t wsb = ss::bwd_workspace_floats(a) * (int64_t)sizeof(float);
  if (ws_alloc(&ws, (size_t)wsb, s) != hipSuccess) {
    (void)hipGetLastError();
    return SS_ERR_HIP;
  }
  const hipError_t e = ss::launch_bwd(a, static_cast<float*>(ws), s);
  const hipError_t f = hipFreeAsync(ws, s);
  return (e == hipSuccess && f == hipSuccess) ? SS_OK : SS_ERR_HIP;
}

int ss_conv1d(const ss_tensor* x, const ss_tensor* weight, const ss_tensor* bias, const ss_tensor* state_in,
              ss_tensor* state_out, uint32_t flags, ss_tensor* out, void* stream) {
  if (!x || !weight || !out) return SS_ERR_NULL;
  if (flags & ~(uint32_t)SS_CONV_SILU) return SS_ERR_FLAGS;
  int rc;
  if ((rc = check_basic(x, 3)) || (rc = check_basic(out, 3)) || (rc = check_basic(weight, 2))) return rc;
  if (present(bias) && (rc = check_basic(bias, 1))) return rc;
  if (weight->dtype != SS_F32 || (present(bias) && bias->dtype != SS_F32)) return SS_ERR_DTYPE;
  const int64_t Bt = x->shape[0], Dc = x->shape[1], L = x->shape[2], W = weight->shape[1];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != x->shape[i]) return SS_ERR_SHAPE;
  if (weight->shape[0] != Dc || W < 1) return SS_ERR_SHAPE;
  if (present(bias) && bias->shape[0] != Dc) return SS_ERR_SHAPE;
  if (W > 8) return SS_ERR_UNSUPPORTED;
  if (present(state_in) && (rc = check_state(state_in, Bt, Dc, W - 1))) return rc;
  if (present(state_out) && (rc = check_state(state_out, Bt, Dc, W - 1))) return rc;
  if (Bt * Dc == 0) return SS_OK;
  // one thread per 8 steps of a row, in a one-dimensional grid (below 2^32 threads)
  if ((L + 7) / 8 > (((int64_t)1 << 32) - 256) / (Bt * Dc)) return SS_ERR_UNSUPPORTED;
  if ((L > 0 && (!x->data || !out->data)) || (Dc > 0 && !weight->data)) return SS_ERR_NULL;
  if (present(bias) && bias->stride[0] != 1 && bias->shape[0] > 1) return SS_ERR_STRIDE;
  // out and state_out are written: neither may overlap an input or the other
  const ss_tensor* ins[] = {x, weight, bias, state_in};
  for (const ss_tensor* t : ins)
    if (overlaps(out, t) || overlaps(state_out, t)) return SS_ERR_ALIAS;
  if (overlaps(out, state_out)) return SS_ERR_ALIAS;
  const bool has_in = present(state_in) && W > 1, has_out = present(state_out) && W > 1;
  if (L == 0 && !has_out) return SS_OK;

  ss::ConvArgs a{};
  a.x = x->data;
  a.w = static_cast<const float*>(weight->data);
  a.bias = present(bias) ? static_cast<const float*>(bias->data) : nullptr;
  a.state_in = has_in ? static_cast<const float*>(state_in->data) : nullptr;
  a.state_out = has_out ? static_cast<float*>(state_out->data) : nullptr;
  a.out = out->data;
  a.batch = Bt;
  a.channels = Dc;
  a.L = L;
  a.W = (int32_t)W;
  a.silu = (flags & SS_CONV_SILU) ? 1 : 0;
  a.x_bf16 = x->dtype == SS_BF16;
  a.out_bf16 = out->dtype == SS_BF16;
  a.vec = L > 0 && aligned16(x) && aligned16(out);
  a.x_sb = x->stride[0];
  a.x_sd = x->stride[1];
  a.o_sb = out->stride[0];
  a.o_sd = out->stride[1];
  a.w_sd = weight->stride[0];
  a.si_sb = has_in ? state_in->stride[0] : 0;
  a.si_sd = has_in ? state_in->stride[1] : 0;
  a.so_sb = has_out ? state_out->stride[0] : 0;
  a.so_sd = has_out ? state_out->stride[1] : 0;
  return ss::launch_conv(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // extern "C"
