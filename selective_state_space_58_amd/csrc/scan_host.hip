// Selective scan: host-side planning and the phase sequence (chunk states,
// carry, output pass), plus the two small helper kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "ssm_internal.h"

// Workspace of ssm_scan_fwd_noalloc (time-split chunk states and step sums):
// one array per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel or a copy: on the host that name is only a stand-in
// for the symbol, so its device address is looked up per device with
// hipGetSymbolAddress (noalloc_scratch below) and that address is used.
static __device__ __align__(256) unsigned char scratch[ssm::kNoAllocScratchBytes];

namespace ssm {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(size_t need, void** out) {
  *out = nullptr;
  if (need > kNoAllocScratchBytes)
    return fail(5, "the no-allocation scan needs " + std::to_string(need) + " bytes of workspace for these shapes; "
                   "its fixed workspace holds " + std::to_string(kNoAllocScratchBytes));
  if (need == 0) return 0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(6, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(4, "device index beyond the no-allocation scan's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(6, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

#define SSM_DECL(R, XB, DB, S)                                                                         \
  hipError_t launch_scan_r##R##_x##XB##_d##DB##_s##S(int mode, const ScanArgs& a, dim3 grid, int64_t gpb, \
                                                     hipStream_t st);
#define SSM_DECL_ALL(XB, DB)                                                                             \
  SSM_DECL(4, XB, DB, 1) SSM_DECL(4, XB, DB, 2) SSM_DECL(4, XB, DB, 4) SSM_DECL(4, XB, DB, 8)            \
  SSM_DECL(4, XB, DB, 16) SSM_DECL(4, XB, DB, 32) SSM_DECL(8, XB, DB, 2) SSM_DECL(8, XB, DB, 32)          \
  SSM_DECL(16, XB, DB, 1)
SSM_DECL_ALL(0, 0)
SSM_DECL_ALL(0, 1)
SSM_DECL_ALL(1, 0)
SSM_DECL_ALL(1, 1)

namespace {

// Combine chunk aggregates in order ("SSM & Mamba": the recurrence composes,
// h_in(c+1) = exp(a * sum of dt over chunk c) * h_in(c) + h_loc(c)).
// Slot c of ws_state receives the state entering chunk c.
__global__ __launch_bounds__(256) void carry_kernel(ScanArgs a, int64_t nlocal, int write_final) {
  const int64_t total = a.batch * a.dim * a.dstate;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t n = i % a.dstate, bd = i / a.dstate, d = bd % a.dim;
  const float an = a.A[d * a.dstate + n];
  float h = a.h0 != nullptr ? a.h0[i] : 0.f;
  // the chunk values are loaded 8 at a time before they are combined, so the
  // loads overlap instead of each waiting behind the previous step
  constexpr int K = 8;
  for (int64_t c0 = 0; c0 < nlocal; c0 += K) {
    float loc[K], ds[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t c = c0 + j < nlocal ? c0 + j : nlocal - 1;
      loc[j] = a.ws_state[c * total + i];
      ds[j] = a.ws_dsum[c * a.batch * a.dim + bd];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (c0 + j < nlocal) {
        a.ws_state[(c0 + j) * total + i] = h;
        h = expf(an * ds[j]) * h + loc[j];
      }
    }
  }
  if (nlocal < a.nchunks) a.ws_state[nlocal * total + i] = h;
  if (write_final && a.h_final != nullptr) a.h_final[i] = h;
}

// seqlen == 0: the state passes through unchanged.
__global__ __launch_bounds__(256) void copy_state_kernel(const float* h0, float* out, int64_t total) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < total) out[i] = h0 != nullptr ? h0[i] : 0.f;
}

template <int XB, int DB>
hipError_t launch_s(int R, int S, int mode, const ScanArgs& a, dim3 grid, int64_t gpb, hipStream_t st);

#define SSM_LAUNCH_S(XB, DB)                                                                              \
  template <>                                                                                             \
  hipError_t launch_s<XB, DB>(int R, int S, int mode, const ScanArgs& a, dim3 grid, int64_t gpb,          \
                              hipStream_t st) {                                                           \
    if (R == 8 && S == 2) return launch_scan_r8_x##XB##_d##DB##_s2(mode, a, grid, gpb, st);               \
    if (R == 8 && S == 32) return launch_scan_r8_x##XB##_d##DB##_s32(mode, a, grid, gpb, st);             \
    if (R == 16 && S == 1) return launch_scan_r16_x##XB##_d##DB##_s1(mode, a, grid, gpb, st);             \
    if (R != 4) return hipErrorInvalidValue;                                                              \
    switch (S) {                                                                                          \
      case 1: return launch_scan_r4_x##XB##_d##DB##_s1(mode, a, grid, gpb, st);                           \
      case 2: return launch_scan_r4_x##XB##_d##DB##_s2(mode, a, grid, gpb, st);                           \
      case 4: return launch_scan_r4_x##XB##_d##DB##_s4(mode, a, grid, gpb, st);                           \
      case 8: return launch_scan_r4_x##XB##_d##DB##_s8(mode, a, grid, gpb, st);                           \
      case 16: return launch_scan_r4_x##XB##_d##DB##_s16(mode, a, grid, gpb, st);                         \
      case 32: return launch_scan_r4_x##XB##_d##DB##_s32(mode, a, grid, gpb, st);                         \
      default: return hipErrorInvalidValue;                                                               \
    }                                                                                                     \
  }
SSM_LAUNCH_S(0, 0)
SSM_LAUNCH_S(0, 1)
SSM_LAUNCH_S(1, 0)
SSM_LAUNCH_S(1, 1)

hipError_t launch_mode(const ScanPlan& p, int mode, const ScanArgs& a, dim3 grid, int64_t gpb, hipStream_t st) {
  if (a.act_bf16 && a.delta_bf16) return launch_s<1, 1>(p.R, p.S, mode, a, grid, gpb, st);
  if (a.act_bf16) return launch_s<1, 0>(p.R, p.S, mode, a, grid, gpb, st);
  if (a.delta_bf16) return launch_s<0, 1>(p.R, p.S, mode, a, grid, gpb, st);
  return launch_s<0, 0>(p.R, p.S, mode, a, grid, gpb, st);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }


}  // namespace

ScanPlan plan_scan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int num_cus) {
  ScanPlan p{};
  const int64_t simds = 4LL * (num_cus > 0 ? num_cus : 256);
  // Rows per wave.  Four rows of 16 channels run one wave per SIMD at best
  // and spend the fewest instructions per element; 16 rows of 4 channels
  // (one state per lane) or 8 rows of 8 give 4x or 2x the waves, so every
  // SIMD interleaves several, at more instructions per element.  With
  // w4 = 4-row waves per SIMD, the 4- and 8-row layouts both run in w4
  // rounds of workgroups, so a fractional w4 leaves their last round partly
  // empty; 16 rows run in (4/3) w4 finer rounds.  Measured at settled clocks
  // (16 states, bf16; ms for 16 / 8 / 4 rows): w4 0.75 (130M-like) 0.166 /
  // 0.194 / -; 1.0 0.205 / 0.193 / 0.247; 1.25 (2.8B-like) 0.516 / 0.582 /
  // 0.695; 1.5 0.303 / 0.296 / 0.352; 2.0 0.392 / 0.374 / 0.353; 2.5 0.471 /
  // 0.467 / 0.539; 3.0 0.579 / 0.545 / 0.540; 5.0 0.901 / 0.889 / 0.850.
  // Layers with so few (batch, channel) slices that even 16 rows cannot
  // fill the chip are split in time instead (below), where 4 rows measured
  // fastest.
  int S = 1;
  while (S * 4 < dstate) S *= 2;
  p.R = 4;
  const int64_t waves4 = batch * ceil_div(dim, 16);
  const bool time_split = waves4 > 0 && waves4 * 2 < simds && seqlen >= 16LL * 32;
  if (dstate <= 16 && !time_split) {
    const int64_t rem = waves4 % simds;   // 4-row waves of the last, partly filled round
    if (waves4 < simds) p.R = 16;
    else if (waves4 < 2 * simds) p.R = (rem > 0 && 2 * rem < simds) ? 16 : 8;
    else if (waves4 < 4 * simds) p.R = rem == 0 ? 4 : 8;
  }
  if (p.R != 4) S = 16 / p.R;
  if (dstate > 128) {
    // 129..256 states: 8 rows of 32 states (one wave per SIMD, 16-token tiles)
    p.R = 8;
    S = 32;
  }
  p.S = S;
  p.T = p.R == 4 ? 32 : (S >= 16 ? 16 : 64);   // the kernel's LDS tile
  const int64_t waves = batch * ceil_div(dim, 64 / p.R);
  int64_t nch = 1;
  // Split time only when fewer than half of the SIMDs would get a wave: the
  // split reruns the recurrence (pass 1), so it pays only when it fills the chip.
  // Then aim for chunks worth 8 waves per SIMD: the state pass costs the same
  // whatever the chunk count, and more waves hide more latency (b1 x 2048
  // channels x 131K tokens: 2.34 ms at 2 per SIMD, 2.22 at 4, 2.16 at 8 and 16,
  // 2.21 at 32).
  if (waves > 0 && waves * 2 < simds && seqlen > 0) {
    nch = ceil_div(8 * simds, waves);
    const int64_t min_len = 8LL * p.T;
    const int64_t max_ch = std::max<int64_t>(1, seqlen / min_len);
    nch = std::min(nch, max_ch);
  }
  const int64_t clen = ceil_div(ceil_div(std::max<int64_t>(seqlen, 1), nch), p.T) * p.T;
  nch = ceil_div(std::max<int64_t>(seqlen, 1), clen);
  p.nchunks = nch;
  p.chunk_len = clen;
  p.ws_bytes = 0;
  if (nch > 1) {
    const size_t st = (size_t)nch * (size_t)(batch * dim * dstate) * sizeof(float);
    const size_t ds = (size_t)nch * (size_t)(batch * dim) * sizeof(float);
    p.ws_bytes = ((st + 255) / 256) * 256 + ds;
  }
  return p;
}

int launch_scan(const ScanArgs& a0, const ScanPlan& p, bool final_only, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  ScanArgs a = a0;
  a.chunk_len = p.chunk_len;
  a.nchunks = p.nchunks;
  const int64_t total = a.batch * a.dim * a.dstate;
  if (a.seqlen == 0) {
    if (a.h_final != nullptr && total > 0) {
      copy_state_kernel<<<dim3((unsigned)ceil_div(total, 256)), 256, 0, st>>>(a.h0, a.h_final, total);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(6, std::string("copy_state_kernel launch: ") + hipGetErrorString(e));
    }
    return 0;
  }
  if (p.long_path) return launch_scan_long(a, stream);
  const int64_t gpb = ceil_div(a.dim, 64 / p.R);
  const int64_t nb = a.batch * gpb;
  if (nb > 0x7fffffffLL || p.nchunks > 65535) return fail(4, "grid too large");
  hipError_t e = hipSuccess;
  if (p.nchunks == 1) {
    const int full_mode = a.save_states != nullptr ? kModeSave : kModeFull;
    e = launch_mode(p, final_only ? kModeState : full_mode, a, dim3((unsigned)nb, 1), gpb, st);
    if (e != hipSuccess) return fail(6, std::string("scan kernel launch: ") + hipGetErrorString(e));
    return 0;
  }
  const int64_t nlocal = final_only ? p.nchunks : p.nchunks - 1;
  e = launch_mode(p, kModeState, a, dim3((unsigned)nb, (unsigned)nlocal), gpb, st);
  if (e != hipSuccess) return fail(6, std::string("chunk-state kernel launch: ") + hipGetErrorString(e));
  carry_kernel<<<dim3((unsigned)ceil_div(total, 256)), 256, 0, st>>>(a, nlocal, final_only ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(6, std::string("carry kernel launch: ") + hipGetErrorString(e));
  if (!final_only) {
    e = launch_mode(p, a.save_states != nullptr ? kModeSave : kModeFull, a, dim3((unsigned)nb, (unsigned)p.nchunks),
                    gpb, st);
    if (e != hipSuccess) return fail(6, std::string("scan kernel launch: ") + hipGetErrorString(e));
  }
  return 0;
}

}  // namespace ssm
