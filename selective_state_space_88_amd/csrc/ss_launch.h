// ss_launch.h -- internal interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

// Arguments of one scan, already validated.  Strides are in elements; the time stride is 1.
struct ScanArgs {
  const void* u;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;          // nullptr: no gate
  const float* A;         // [channels, N] (diagonal) or [heads] (scalar decay)
  const float* D;         // nullable
  const float* bias;      // nullable, [heads]
  void* y;
  int64_t batch, channels, L;
  int32_t N, heads, groups;
  int32_t chan_per_head, chan_per_group;
  int32_t d_per_head;     // D indexed by head
  int32_t softplus;
  int32_t in_bf16, out_bf16;
  int32_t vec;            // every time row is 16-byte aligned (vector loads / stores allowed)
  int64_t u_sb, u_sd, dl_sb, dl_sh, z_sb, z_sd;
  int64_t B_sb, B_sg, B_sn, C_sb, C_sg, C_sn;
  int64_t y_sb, y_sd, A_sd;
  // optional state in / out, [batch, channels, N] f32, state index innermost (stride 1)
  int32_t zoh;            // zero-order-hold input coefficient (exp(dt A) - 1) / A instead of dt
  int32_t trap;           // exponential-trapezoidal rule: y read from h - e/2 (the state is h + e/2)
  const float* h_init;    // nullptr: the state starts at zero
  float* h_final;         // nullptr: not written
  int64_t hi_sb, hi_sd, hf_sb, hf_sd;
  // diagonal decay only, for the backward: when set, the state at the start of every 512 steps
  // (checkpoint c of (b, d) at ckpt[((b channels + d) ckpt_nwin + c) N + n], ckpt_nwin =
  // ceil(L / 512)), as the backward's checkpoint pass would store it
  float* ckpt;
  int64_t ckpt_nwin;
  // the window-slot kernel's checkpoint strides of a batch row and of a channel, in floats (0:
  // the dense layout above); a sequence segment run as a row of its own writes its checkpoints
  // into the whole sequence's layout with them
  int64_t ck_sb, ck_sd;
};

// Arguments of one decoding step (L = 1), already validated.  Strides in elements.
struct StepArgs {
  const void* u;          // [batch, channels]
  const void* delta;      // [batch, heads]
  const void* B;          // [batch, groups, N]
  const void* C;
  const void* z;          // nullptr: no gate
  const float* A;         // [channels, N] or [heads]
  const float* D;         // nullable
  const float* bias;      // nullable
  float* h;               // [batch, channels, N], read and written in place
  void* y;                // [batch, channels]
  int64_t batch, channels;
  int32_t N, heads, groups;
  int32_t chan_per_head, chan_per_group;
  int32_t scalar;         // A per head
  int32_t zoh;            // zero-order-hold input coefficient
  int32_t trap;           // exponential-trapezoidal rule
  int32_t d_per_head;
  int32_t softplus;
  int32_t in_bf16, out_bf16;
  int64_t u_sb, dl_sb, z_sb, B_sb, B_sg, C_sb, C_sg, y_sb, A_sd, h_sb, h_sd;
};

// One step of the recurrence for every (batch, channel): h = exp(dt A) h + dt B u, y = C h + D u.
hipError_t launch_step(const StepArgs& a, hipStream_t stream);

// Arguments of the backward of a scan, already validated.  Inputs as in ScanArgs; dy [batch,
// channels, L]; every gradient f32 with the shape of its input, innermost stride 1.
struct BwdArgs {
  const void* u;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;          // nullptr: no gate
  const float* A;         // [channels, N]
  const float* D;         // nullable
  const float* bias;      // nullable, [channels]
  const void* dy;
  float *du, *ddelta, *dA, *dB, *dC;
  float *dD, *dz, *dbias; // nullable (absent input)
  int64_t batch, channels, L;
  int32_t N, groups, chan_per_group;
  int32_t heads, chan_per_head;
  int32_t scalar;         // A [heads]: one decay per head shared by its states
  int32_t d_per_head;     // D (and dD) indexed by head
  int32_t softplus, in_bf16, dy_bf16;
  int32_t vec;            // every input time row (and dy's) is 16-byte aligned
  int32_t ckpt_ready;     // the per-channel path's checkpoints are already in the workspace
  int32_t y0_vec;         // gy0's rows are 16-byte aligned
  // the gate folded into the per-channel kernel (set by launch_bwd for a gated call; z is then
  // nullptr): gz is the gate input (strides z_sb, z_sd), gy0 the output before the gate
  // ([batch, channels, L] f32, contiguous); the kernel writes dz and runs on dy0 = dy s(z)
  const void* gz;
  const float* gy0;
  int64_t u_sb, u_sd, dl_sb, dl_sh, z_sb, z_sd, B_sb, B_sg, B_sn, C_sb, C_sg, C_sn, A_sd, dy_sb, dy_sd;
  int64_t du_sb, du_sd, dd_sb, dd_sh, dA_sd, dB_sb, dB_sg, dB_sn, dC_sb, dC_sg, dC_sn, dz_sb, dz_sd;
};

// Gradients of sum(dy * y).  `ws` must hold bwd_workspace_floats(a) floats (the states at the
// start of every window, or of every chunk on the matrix path), ordered on `stream`.
int64_t bwd_workspace_floats(const BwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a, float* ws, hipStream_t stream);

// Scalar decay without a gate, heads and B/C groups in whole 64-channel slabs: the backward in the
// chunked matrix form on fp32 MFMA (launched by launch_bwd, after the summed gradients are zeroed).
bool ssd_bwd_path(const BwdArgs& a);
int64_t ssd_bwd_workspace_floats(const BwdArgs& a);
hipError_t launch_ssd_bwd(const BwdArgs& a, float* ws, hipStream_t stream);

// dst[b, d, n] = src[b, d, n] (src == nullptr: 0) for a [batch, channels, N] f32 state.
hipError_t launch_state_copy(const float* src, int64_t s_sb, int64_t s_sd, float* dst, int64_t d_sb,
                             int64_t d_sd, int64_t batch, int64_t channels, int64_t N, hipStream_t stream);

// Arguments of a causal depthwise convolution along time, already validated.  Strides in
// elements, time stride 1.
struct ConvArgs {
  const void* x;          // [batch, channels, L]
  const float* w;         // [channels, W]
  const float* bias;      // nullable, [channels]
  const float* state_in;  // nullable, [batch, channels, W - 1]: x_{-(W-1)} .. x_{-1}
  float* state_out;       // nullable, [batch, channels, W - 1]: the last W - 1 inputs
  void* out;              // [batch, channels, L]
  int64_t batch, channels, L;
  int32_t W;              // 1 .. 8
  int32_t silu, x_bf16, out_bf16;
  int32_t vec;            // x and out rows 16-byte aligned
  int64_t x_sb, x_sd, o_sb, o_sd, w_sd, si_sb, si_sd, so_sb, so_sd;
  int64_t pieces, total;  // set by launch_conv: 8-step pieces per row, and in all
};

// out_t = bias + sum_j w[j] x_{t-(W-1)+j} (optionally silu) for every (batch, channel) row.
hipError_t launch_conv(const ConvArgs& a, hipStream_t stream);

// Compute units of the current device (cached per device; 256 if the query fails).
int cu_count();

// Diagonal decay A [channels, N]: one or two (b, d) rows per wave, lanes along time; few rows
// take several windows of each row in flight.  One kernel, no workspace.
hipError_t launch_diag(const ScanArgs& a, hipStream_t stream);
// The same where a few rows with long sequences are cut into sequence segments, which takes a
// workspace: `ws` must hold diag_workspace_bytes(a) bytes (0: none, ws may be null) of device
// memory ordered on `stream`.
int64_t diag_workspace_bytes(const ScanArgs& a);
// whether a diagonal-decay forward runs on the window-slot kernel (few rows, at least three
// 1024-step windows, bf16 inputs in 16-byte aligned rows)
bool diag_slots_path(const ScanArgs& a);
hipError_t launch_diag(const ScanArgs& a, void* ws, hipStream_t stream);

// Whether a bounded wait between the waves of a block has run out since the last call (then
// the results of the calls in between are wrong); clears the record.  Synchronous.
hipError_t take_spin_error(int* failed);

// Scalar decay A [heads]: lanes along channels, 16 states per wave.  `ws` must hold
// scalar_workspace_floats(a) floats of device memory, ordered on `stream`.
int64_t scalar_workspace_floats(const ScanArgs& a);
hipError_t launch_scalar(const ScanArgs& a, float* ws, hipStream_t stream);

// Scalar decay in the chunked matrix form on MFMA (bf16 inputs, heads and B/C groups in whole
// 64-channel slabs).  `ws` must hold ssd_workspace_bytes(a) bytes (16-byte aligned) of device
// memory, ordered on `stream`.
bool ssd_path(const ScanArgs& a);
int64_t ssd_workspace_bytes(const ScanArgs& a);
hipError_t launch_ssd(const ScanArgs& a, void* ws, hipStream_t stream);

}  // namespace ss
