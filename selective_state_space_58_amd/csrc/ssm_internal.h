// Internal declarations shared by the host dispatch code and the HIP kernels
// of the MI355X selective-scan library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

namespace ssm {

// Set the calling thread's error detail and return `status`.
int fail(int status, const std::string& msg);

// ---------------------------------------------------------------- selective scan
// Kernel geometry: one wavefront (64 lanes) per workgroup.  The lanes form R
// rows of 64/R channels; row r owns states [r*S, r*S + S) of the wave's
// channels, so every (channel, state) pair lives in exactly one lane's VGPRs.
// R is 4 in general, 8 or 16 for layers with dstate <= 16 and too few
// (batch, channel) slices to give every SIMD several waves at R = 4.

// kModeSave: kModeFull that also stores the state at every 16-token tile start (for the backward)
enum ScanMode : int { kModeFull = 0, kModeState = 1, kModeSave = 2 };
constexpr int kSaveTile = 16;   // tokens between saved states

struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const float* h0;
  void* y;
  float* h_final;
  float* ws_state;   // (nchunks, batch, dim, dstate) chunk-local end states / carries
  float* ws_dsum;    // (nchunks, batch, dim) sum of dt over each chunk
  int64_t batch, seqlen, dim, dstate;
  int64_t chunk_len;  // tokens per time chunk (multiple of the time tile)
  int64_t nchunks;    // number of time chunks (1 = unsplit)
  int softplus;
  int act_bf16, delta_bf16;
  int vec_io;          // vector tile I/O allowed (16-byte aligned inputs)
  int reverse;         // scan the sequence from the last token to the first
  int euler;           // input discretization Bbar = dt * B instead of ZOH
  int delta_per_token; // delta is (batch, seqlen), one dt per token shared by all channels
  float* save_states;  // kModeSave: (ceil(seqlen/16), batch, dim, dstate) state entering every 16-token tile
};

struct ScanPlan {
  int R;              // rows of lanes per wave (4, 8 or 16); 64/R channels per wave
  int S;              // states per lane (power of two, R*S >= dstate)
  int T;              // time tile (tokens staged per LDS round)
  int64_t nchunks;
  int64_t chunk_len;
  size_t ws_bytes;
  bool long_path;     // one pass with time-split lanes (scan_long.hip) instead of chunks
};

ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus);

// Enqueue the whole selective scan (all phases).  Returns an ssm_status.
int launch_scan(const ScanArgs& a, const ScanPlan& p, bool final_only, void* stream);

// Long sequences on few slices in one pass, the lanes of a wave splitting the
// time axis (scan_long.hip).  scan_long_applies: the arguments fit that kernel
// (16 states, whole 8-channel groups, 16-byte aligned rows, no variant flags,
// enough channel groups for every CU); launch_scan_long returns an ssm_status.
bool scan_long_applies(const ScanArgs& a, int num_cus);
int launch_scan_long(const ScanArgs& a, void* stream);

// Workspace of the no-allocation scan entry point: a fixed device array of
// kNoAllocScratchBytes per GPU, shared by every such call on that GPU.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// Device address of the current GPU's array (looked up once per device).
// Fails with SSM_ERR_WORKSPACE when need exceeds the array, SSM_ERR_HIP on a
// runtime error.
int noalloc_scratch(size_t need, void** out);

// ---------------------------------------------------------------- selective scan backward
struct BwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  const float* h0;
  const void* dout;        // act dtype, like y
  const float* dh_final;   // or null
  void* dx;                // act dtype
  void* ddelta;            // delta dtype
  float* dA;               // (dim, dstate)
  float* dB;               // (batch, seqlen, dstate) fp32
  float* dC;
  float* dDskip;           // (dim) or null
  void* dz;                // act dtype; required when z is given
  float* ddelta_bias;      // (dim) or null
  float* dh0;              // (batch, dim, dstate) or null
  float* ws_ckpt;          // (ntiles, batch, dim, dstate) states at tile starts
  float* ws_part;          // 2 x (groups, batch, seqlen, 16) dB, dC partials of the channel groups
  int64_t ws_groups;       // channel groups (workgroups per batch row)
  float* acc;              // 3 x (batch, seqlen, dim) fp32: dx, ddelta, dz summed over state blocks (dstate > 16)
  int64_t n0;              // first state of the block of 16 this pass handles
  int first, last;         // first / last block of states
  int reverse;             // gradients of the reversed scan (tokens from the last to the first)
  int euler;               // gradients of the Euler discretization (gain dt)
  int tok_delta;           // delta (and ddelta) of shape (batch, seqlen), shared by every channel
  float* ddelta_tc;        // tok_delta: fp32 (batch, seqlen, dim) per-channel ddelta, summed after the passes
  const float* saved;      // states the forward stored at every 16-token tile start (no checkpoint pass), or null
  int64_t batch, seqlen, dim, dstate;
  int softplus;
  int act_bf16, delta_bf16;
};

size_t scan_bwd_ws_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool tok_delta, bool saved);
int launch_scan_bwd(const BwdArgs& a, void* stream);

// ---------------------------------------------------------------- SSD
struct SsdArgs {
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* dt_bias;
  const float* h0;
  void* y;
  float* h_final;
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate, chunk;
  int softplus;
  int dt_bf16;
  void* ws;
  // time chunks run in parallel (set by launch_ssd from the plan)
  int64_t tchunk, nchunks;
  float* ws_state;     // nchunks x (batch, nheads, headdim, dstate): chunk states, then carries
  float* ws_dsum;      // nchunks x (batch, nheads): a * sum of dt over the chunk
  float* ws_cb;        // (batch, 64-token block, group, causal 16x16 tile, lane) x 4: C_t . B_s per block
};

// Workspace plan of the SSD pass.  The C B^T products of every 64-token block
// (shared by all heads of a group) are formed once by a pre-pass.  When the
// (batch, head) pairs cannot fill the device, the sequence is also split into
// nchunks chunks of tchunk tokens (a multiple of 64) whose states are computed
// in parallel and combined by a carry pass.
struct SsdPlan {
  int64_t nchunks, tchunk;
  size_t ws_bytes;
  size_t dsum_off, cb_off;   // byte offsets of ws_dsum and ws_cb (ws_state at 0)
};
SsdPlan plan_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                 int num_cus);
size_t ssd_ws_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                    int64_t dstate, int64_t chunk);
int launch_ssd(const SsdArgs& a, void* stream);
// The blocked kernel (matrix cores) takes bf16 activations with headdim 64 or
// 128 and dstate 64 or 128; every other call runs the SSD as its recurrence
// (ssd_rec.hip: fp32 or bf16, any headdim, dstate up to kSsdRecMaxState, no
// workspace).
inline bool ssd_blocked_applies(bool act_bf16, int64_t headdim, int64_t dstate) {
  return act_bf16 && (headdim == 64 || headdim == 128) && (dstate == 64 || dstate == 128);
}
constexpr int64_t kSsdRecMaxState = 256;
int launch_ssd_rec(const SsdArgs& a, bool act_f32, void* stream);

// ---------------------------------------------------------------- single-token state update
// Channel d of batch b belongs to head d / headdim (headdim 1: every channel is
// its own head, the Mamba layout); dt, delta_bias and Dskip are indexed by head,
// A by (d, n) (a_per_head 0) or by head (a_per_head 1), B and C by
// (b, head / (nheads / ngroups), n).
struct StepArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  const float* delta_bias;
  float* state;       // (batch, dim, dstate) fp32, updated in place
  void* y;
  int64_t batch, dim, dstate, headdim, ngroups;
  int a_per_head;
  int softplus;
  int act_bf16, delta_bf16;
  int vec;            // 16-byte state/A and 8/16-byte B/C accesses allowed
};

int launch_state_update(const StepArgs& a, void* stream);

// ---------------------------------------------------------------- causal conv1d (+ SiLU)
struct ConvArgs {
  const void* x;          // (batch, seqlen, dim) act dtype
  const float* w;         // (dim, width)
  const float* bias;      // (dim) or null
  const void* state_in;   // (batch, dim, width-1) act dtype or null (zeros)
  void* out;              // (batch, seqlen, dim) act dtype
  void* state_out;        // (batch, dim, width-1) act dtype or null; may alias state_in
  int64_t batch, seqlen, dim, width;
  int silu;
  int act_bf16;
  int vec;                // 8 channels per thread with 16/32-byte accesses
};

int launch_conv(const ConvArgs& a, void* stream);

int device_cu_count();

}  // namespace ssm
