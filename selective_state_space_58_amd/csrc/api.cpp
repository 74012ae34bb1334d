// C ABI entry points of the MI355X selective-scan library: argument
// validation (host only, before any HIP call), planning, workspace handling
// and dispatch to the HIP kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <limits>
#include <string>

#include "../../include/ssm_mi355x.h"
#include "ssm_internal.h"

namespace ssm {

namespace {
thread_local std::string g_last_error;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / 4 / a) return false;  // keep byte offsets in range
  *out = a * b;
  return true;
}

bool elems_ok(std::initializer_list<int64_t> dims) {
  int64_t acc = 1;
  for (int64_t d : dims)
    if (!mul_ok(acc, d, &acc)) return false;
  return true;
}

bool aligned(const void* p, size_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

size_t dsize(int dt) { return dt == SSM_BF16 ? 2 : 4; }

// Stream-ordered scratch for calls that pass no workspace.
struct Scratch {
  void* ptr = nullptr;
  hipStream_t st = nullptr;
  ~Scratch() {
    if (ptr != nullptr) (void)hipFreeAsync(ptr, st);
  }
};

int get_workspace(void* user, size_t user_bytes, size_t need, hipStream_t st, Scratch* own, void** out) {
  *out = nullptr;
  if (need == 0) return SSM_OK;
  if (user != nullptr) {
    if (user_bytes < need)
      return fail(SSM_ERR_WORKSPACE, "workspace of " + std::to_string(user_bytes) + " bytes, need " +
                                         std::to_string(need));
    if (!aligned(user, 256)) return fail(SSM_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
    *out = user;
    return SSM_OK;
  }
  hipError_t e = hipMallocAsync(&own->ptr, need, st);
  if (e != hipSuccess) return fail(SSM_ERR_HIP, std::string("hipMallocAsync: ") + hipGetErrorString(e));
  own->st = st;
  *out = own->ptr;
  return SSM_OK;
}

int validate_scan(const void* x, const void* delta, const float* A, const void* B, const void* C,
                  const void* y_or_hf, bool final_only, const float* Dskip, const void* z, const float* bias,
                  const float* h0, const float* hf, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                  int act_dtype, int delta_dtype, int softplus) {
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 0) return fail(SSM_ERR_SHAPE, "negative size");
  // Tensors with no elements may be NULL (an empty framework tensor has no storage).
  const bool has_tok = batch > 0 && seqlen > 0 && dim > 0;
  const bool has_bc = batch > 0 && seqlen > 0;
  if ((has_tok && (x == nullptr || delta == nullptr)) || (dim > 0 && A == nullptr) ||
      (has_bc && (B == nullptr || (!final_only && C == nullptr))))
    return fail(SSM_ERR_NULL, "x, delta, A, B and C (forward) are required");
  if (final_only ? (batch > 0 && dim > 0 && y_or_hf == nullptr) : (has_tok && y_or_hf == nullptr))
    return fail(SSM_ERR_NULL, final_only ? "h_final is required" : "y is required");
  if (dstate == 0) return fail(SSM_ERR_SHAPE, "dstate must be >= 1");
  if (act_dtype != SSM_F32 && act_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "act_dtype must be SSM_F32 or SSM_BF16");
  if (delta_dtype != SSM_F32 && delta_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "delta_dtype must be SSM_F32 or SSM_BF16");
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_SHAPE, "delta_softplus must be 0 or 1");
  if (!elems_ok({batch, seqlen, dim}) || !elems_ok({batch, seqlen, dstate}) || !elems_ok({batch, dim, dstate}) ||
      !elems_ok({dim, dstate}))
    return fail(SSM_ERR_SHAPE, "sizes overflow 64-bit indexing");
  if (dstate > 256) return fail(SSM_ERR_UNSUPPORTED, "dstate > 256 is not supported");
  const size_t as = dsize(act_dtype), ds = dsize(delta_dtype);
  if (!aligned(x, as) || !aligned(B, as) || !aligned(C, as) || !aligned(z, as) || !aligned(y_or_hf, final_only ? 4 : as) ||
      !aligned(delta, ds) || !aligned(A, 4) || !aligned(Dskip, 4) || !aligned(bias, 4) || !aligned(h0, 4) ||
      !aligned(hf, 4))
    return fail(SSM_ERR_ALIGNMENT, "a pointer is not aligned to its element size");
  return SSM_OK;
}

int cached_cus = -1;

}  // namespace

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int device_cu_count() {
  if (cached_cus > 0) return cached_cus;
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
      prop.multiProcessorCount > 0) {
    cached_cus = prop.multiProcessorCount;
    return cached_cus;
  }
  (void)hipGetLastError();
  return 256;  // MI355X
}

}  // namespace ssm

using namespace ssm;

extern "C" {

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid or inconsistent size";
    case SSM_ERR_DTYPE: return "unknown dtype";
    case SSM_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSM_ERR_WORKSPACE: return "workspace too small";
    case SSM_ERR_HIP: return "HIP runtime error";
    case SSM_ERR_ALIGNMENT: return "misaligned pointer";
    default: return "unknown status";
  }
}

const char* ssm_last_error(void) { return g_last_error.c_str(); }

#ifndef SSM_SOURCE_DIGEST
#define SSM_SOURCE_DIGEST "0000000000000000000000000000000000000000000000000000000000000000"
#endif
// The marker lets a loader find the digest in the library file without loading it.
static const char kSourceDigest[] = "ssm-source-sha256:" SSM_SOURCE_DIGEST;
static_assert(sizeof(kSourceDigest) == 18 + 64 + 1, "the source digest is 64 hex digits");

const char* ssm_source_digest(void) { return kSourceDigest + 18; }

size_t ssm_scan_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > 256) return 0;
  return plan_scan(batch, seqlen, dim, dstate, device_cu_count()).ws_bytes;
}

static int scan_common(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                       const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                       int64_t dstate, int act_dtype, int delta_dtype, void* workspace, size_t workspace_bytes,
                       void* stream, bool final_only, int flags = 0, float* save_states = nullptr,
                       bool want_save = false, bool no_alloc = false) {
  g_last_error.clear();
  if ((flags & ~(SSM_SCAN_REVERSE | SSM_SCAN_EULER | SSM_SCAN_DELTA_PER_TOKEN)) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "unknown scan flag bits");
  int rc = validate_scan(x, delta, A, B, C, final_only ? (const void*)h_final : y, final_only, Dskip, z, delta_bias,
                         h0, h_final, batch, seqlen, dim, dstate, act_dtype, delta_dtype, delta_softplus);
  if (rc != SSM_OK) return rc;
  if (want_save && batch > 0 && seqlen > 0 && dim > 0 && save_states == nullptr)
    return fail(SSM_ERR_NULL, "states is required");
  if (!aligned(save_states, 4)) return fail(SSM_ERR_ALIGNMENT, "states must be 4-byte aligned");
  if (batch == 0 || dim == 0) return SSM_OK;
  const int cus = device_cu_count();
  ScanPlan p = plan_scan(batch, seqlen, dim, dstate, cus);
  hipStream_t st = (hipStream_t)stream;
  ScanArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = final_only ? nullptr : C;
  a.Dskip = final_only ? nullptr : Dskip;
  a.z = final_only ? nullptr : z;
  a.delta_bias = delta_bias; a.h0 = h0;
  a.y = final_only ? nullptr : y;
  a.h_final = h_final;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.dstate = dstate;
  a.softplus = delta_softplus;
  a.act_bf16 = act_dtype == SSM_BF16;
  a.delta_bf16 = delta_dtype == SSM_BF16;
  a.reverse = (flags & SSM_SCAN_REVERSE) != 0;
  a.euler = (flags & SSM_SCAN_EULER) != 0;
  a.delta_per_token = (flags & SSM_SCAN_DELTA_PER_TOKEN) != 0;
  a.save_states = want_save ? save_states : nullptr;
  // vector tile I/O: 16-byte aligned tensors (delta, when it is per channel, in either dtype)
  a.vec_io = aligned16(x) && (a.delta_per_token || aligned16(delta)) && aligned16(B) &&
             (final_only || aligned16(C)) && (final_only || aligned16(z));
  // A sequence the plan would split into time chunks runs in one pass with
  // time-split lanes instead when that kernel takes the arguments; it needs
  // no workspace.
  if (!final_only && p.nchunks > 1 && scan_long_applies(a, cus)) {
    p.long_path = true;
    p.ws_bytes = 0;
  }
  Scratch own;
  void* ws = nullptr;
  if (no_alloc) rc = noalloc_scratch(seqlen > 0 ? p.ws_bytes : 0, &ws);
  else rc = get_workspace(workspace, workspace_bytes, seqlen > 0 ? p.ws_bytes : 0, st, &own, &ws);
  if (rc != SSM_OK) return rc;
  if (ws != nullptr) {
    const size_t st_bytes = (size_t)p.nchunks * (size_t)(batch * dim * dstate) * sizeof(float);
    a.ws_state = (float*)ws;
    a.ws_dsum = (float*)((char*)ws + ((st_bytes + 255) / 256) * 256);
  }
  return launch_scan(a, p, final_only, stream);
}

int ssm_scan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                 const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                 const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                 int64_t dstate, int act_dtype, int delta_dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return scan_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                     dstate, act_dtype, delta_dtype, workspace, workspace_bytes, stream, false);
}

int ssm_scan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B, const void* C,
                         const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                         const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                         int64_t dstate, int act_dtype, int delta_dtype, void* stream) {
  return scan_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                     dstate, act_dtype, delta_dtype, nullptr, 0, stream, false, 0, nullptr, false, true);
}

size_t ssm_scan_fwd_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

int ssm_scan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                    const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                    int64_t dstate, int act_dtype, int delta_dtype, int flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return scan_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                     dstate, act_dtype, delta_dtype, workspace, workspace_bytes, stream, false, flags);
}

int ssm_scan_fwd_train(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                       const float* h0, void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t dim,
                       int64_t dstate, int act_dtype, int delta_dtype, int flags, float* states, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return scan_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                     dstate, act_dtype, delta_dtype, workspace, workspace_bytes, stream, false, flags, states, true);
}

size_t ssm_scan_train_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > 256) return 0;
  if (!elems_ok({batch, seqlen, dim, dstate})) return 0;
  return (size_t)((seqlen + kSaveTile - 1) / kSaveTile) * (size_t)(batch * dim * dstate) * sizeof(float);
}

int ssm_scan_final_state(const void* x, const void* delta, const float* A, const void* B, const float* delta_bias,
                         int delta_softplus, const float* h0, float* h_final, int64_t batch, int64_t seqlen,
                         int64_t dim, int64_t dstate, int act_dtype, int delta_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return scan_common(x, delta, A, B, nullptr, nullptr, nullptr, delta_bias, delta_softplus, h0, nullptr, h_final,
                     batch, seqlen, dim, dstate, act_dtype, delta_dtype, workspace, workspace_bytes, stream, true);
}

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                           int64_t dstate, int64_t chunk_size) {
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0 || chunk_size <= 0)
    return 0;
  // (the recurrent form needs none; bf16 activations on these shapes take the blocked kernel)
  if (!ssd_blocked_applies(true, headdim, dstate)) return 0;
  return ssd_ws_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size);
}

int ssd_chunk_scan_fwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* dt_bias, int dt_softplus, const float* h0,
                       void* y, float* h_final, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t ngroups, int64_t dstate, int64_t chunk_size, int act_dtype, int dt_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || ngroups < 0 || dstate < 0 || chunk_size < 0)
    return fail(SSM_ERR_SHAPE, "negative size");
  // Tensors with no elements may be NULL (an empty framework tensor has no storage).
  const bool has_tok = batch > 0 && seqlen > 0;
  if ((has_tok && (x == nullptr || dt == nullptr || B == nullptr || C == nullptr || y == nullptr)) ||
      (nheads > 0 && A == nullptr))
    return fail(SSM_ERR_NULL, "x, dt, A, B, C and y are required");
  if (nheads == 0 || headdim == 0 || ngroups == 0 || dstate == 0 || chunk_size == 0)
    return fail(SSM_ERR_SHAPE, "nheads, headdim, ngroups, dstate and chunk_size must be >= 1");
  if (nheads % ngroups != 0) return fail(SSM_ERR_SHAPE, "nheads must be a multiple of ngroups");
  if (act_dtype != SSM_F32 && act_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "act_dtype must be SSM_F32 or SSM_BF16");
  if (dt_dtype != SSM_F32 && dt_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "dt_dtype must be SSM_F32 or SSM_BF16");
  if (dt_softplus != 0 && dt_softplus != 1) return fail(SSM_ERR_SHAPE, "dt_softplus must be 0 or 1");
  if (!elems_ok({batch, seqlen, nheads, headdim}) || !elems_ok({batch, seqlen, ngroups, dstate}) ||
      !elems_ok({batch, nheads, headdim, dstate}))
    return fail(SSM_ERR_SHAPE, "sizes overflow 64-bit indexing");
  if (dstate > kSsdRecMaxState) return fail(SSM_ERR_UNSUPPORTED, "SSD supports dstate up to 256");
  if (chunk_size != 64 && chunk_size != 128 && chunk_size != 256)
    return fail(SSM_ERR_UNSUPPORTED, "SSD supports chunk_size 64, 128 or 256");
  const size_t ds = dsize(dt_dtype);
  if (!aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(z, 16) || !aligned(y, 16) ||
      !aligned(dt, ds) || !aligned(A, 4) || !aligned(Dskip, 4) || !aligned(dt_bias, 4) || !aligned(h0, 16) ||
      !aligned(h_final, 16))
    return fail(SSM_ERR_ALIGNMENT, "SSD needs 16-byte aligned x/B/C/z/y/h0/h_final and element-aligned dt");
  if (batch == 0) return SSM_OK;
  hipStream_t st = (hipStream_t)stream;
  const bool blocked = ssd_blocked_applies(act_dtype == SSM_BF16, headdim, dstate);
  Scratch own;
  void* ws = nullptr;
  const size_t need = blocked ? ssd_ws_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size) : 0;
  int rc = get_workspace(workspace, workspace_bytes, seqlen > 0 ? need : 0, st, &own, &ws);
  if (rc != SSM_OK) return rc;
  SsdArgs a{};
  a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z; a.dt_bias = dt_bias;
  a.h0 = h0; a.y = y; a.h_final = h_final;
  a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.headdim = headdim; a.ngroups = ngroups;
  a.dstate = dstate; a.chunk = chunk_size; a.softplus = dt_softplus; a.dt_bf16 = dt_dtype == SSM_BF16;
  a.ws = ws;
  return blocked ? launch_ssd(a, stream) : launch_ssd_rec(a, act_dtype == SSM_F32, stream);
}

static int step_common(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* bias, int softplus, float* state, void* y,
                       int64_t batch, int64_t dim, int64_t dstate, int64_t headdim, int64_t ngroups,
                       bool per_head, int act_dtype, int delta_dtype, void* stream) {
  g_last_error.clear();
  if (batch < 0 || dim < 0 || dstate < 0 || headdim < 0 || ngroups < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (dstate == 0 || headdim == 0 || ngroups == 0) return fail(SSM_ERR_SHAPE, "dstate, headdim and ngroups must be >= 1");
  if (dim % headdim != 0) return fail(SSM_ERR_SHAPE, "channels must be a whole number of heads");
  const int64_t nheads = dim / headdim;
  if (nheads % ngroups != 0) return fail(SSM_ERR_SHAPE, "nheads must be a multiple of ngroups");
  const bool has = batch > 0 && dim > 0;
  if ((has && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || state == nullptr ||
               y == nullptr)) ||
      (dim > 0 && A == nullptr))
    return fail(SSM_ERR_NULL, "x, delta/dt, A, B, C, state and y are required");
  if (act_dtype != SSM_F32 && act_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "act_dtype must be SSM_F32 or SSM_BF16");
  if (delta_dtype != SSM_F32 && delta_dtype != SSM_BF16)
    return fail(SSM_ERR_DTYPE, "delta dtype must be SSM_F32 or SSM_BF16");
  if (softplus != 0 && softplus != 1) return fail(SSM_ERR_SHAPE, "softplus flag must be 0 or 1");
  if (!elems_ok({batch, dim, dstate}) || !elems_ok({dim, dstate}) || !elems_ok({batch, ngroups, dstate}))
    return fail(SSM_ERR_SHAPE, "sizes overflow 64-bit indexing");
  if (dstate > 256) return fail(SSM_ERR_UNSUPPORTED, "dstate > 256 is not supported");
  const size_t as = dsize(act_dtype), ds = dsize(delta_dtype);
  if (!aligned(x, as) || !aligned(B, as) || !aligned(C, as) || !aligned(z, as) || !aligned(y, as) ||
      !aligned(delta, ds) || !aligned(A, 4) || !aligned(Dskip, 4) || !aligned(bias, 4) || !aligned(state, 4))
    return fail(SSM_ERR_ALIGNMENT, "a pointer is not aligned to its element size");
  if (!has) return SSM_OK;
  // the state is overwritten while y is written: they must not overlap
  const char* s0 = (const char*)state;
  const char* s1 = s0 + (size_t)(batch * dim * dstate) * sizeof(float);
  const char* y0 = (const char*)y;
  const char* y1 = y0 + (size_t)(batch * dim) * as;
  if (y0 < s1 && s0 < y1) return fail(SSM_ERR_SHAPE, "y must not overlap the state");
  StepArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z; a.delta_bias = bias;
  a.state = state; a.y = y;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.headdim = headdim; a.ngroups = ngroups;
  a.a_per_head = per_head ? 1 : 0;
  a.softplus = softplus;
  a.act_bf16 = act_dtype == SSM_BF16;
  a.delta_bf16 = delta_dtype == SSM_BF16;
  const size_t bc_align = act_dtype == SSM_BF16 ? 8 : 16;
  a.vec = dstate % 4 == 0 && aligned16(state) && (per_head || aligned16(A)) && aligned(B, bc_align) &&
          aligned(C, bc_align);
  return launch_state_update(a, stream);
}

int ssm_state_update(const void* x, const void* delta, const float* A, const void* B, const void* C,
                     const float* Dskip, const void* z, const float* delta_bias, int delta_softplus, float* state,
                     void* y, int64_t batch, int64_t dim, int64_t dstate, int act_dtype, int delta_dtype,
                     void* stream) {
  return step_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, state, y, batch, dim, dstate, 1, 1,
                     false, act_dtype, delta_dtype, stream);
}

int ssd_state_update(const void* x, const void* dt, const float* A, const void* B, const void* C,
                     const float* Dskip, const void* z, const float* dt_bias, int dt_softplus, float* state, void* y,
                     int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate, int act_dtype,
                     int dt_dtype, void* stream) {
  if (nheads < 0 || headdim < 0) {
    g_last_error.clear();
    return fail(SSM_ERR_SHAPE, "negative size");
  }
  int64_t dim = 0;
  if (!mul_ok(nheads, headdim, &dim)) return fail(SSM_ERR_SHAPE, "sizes overflow 64-bit indexing");
  return step_common(x, dt, A, B, C, Dskip, z, dt_bias, dt_softplus, state, y, batch, dim, dstate, headdim, ngroups,
                     true, act_dtype, dt_dtype, stream);
}

int ssm_causal_conv1d_fwd(const void* x, const float* weight, const float* bias, const void* state_in, int silu,
                          void* out, void* state_out, int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                          int act_dtype, void* stream) {
  g_last_error.clear();
  if (batch < 0 || seqlen < 0 || dim < 0 || width < 0) return fail(SSM_ERR_SHAPE, "negative size");
  if (width == 0) return fail(SSM_ERR_SHAPE, "width must be >= 1");
  if (silu != 0 && silu != 1) return fail(SSM_ERR_SHAPE, "silu must be 0 or 1");
  if (act_dtype != SSM_F32 && act_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "act_dtype must be SSM_F32 or SSM_BF16");
  const bool has_tok = batch > 0 && seqlen > 0 && dim > 0;
  if ((has_tok && (x == nullptr || out == nullptr)) || (dim > 0 && weight == nullptr))
    return fail(SSM_ERR_NULL, "x, weight and out are required");
  if (!elems_ok({batch, seqlen, dim}) || !elems_ok({dim, width}) || !elems_ok({batch, dim, width}))
    return fail(SSM_ERR_SHAPE, "sizes overflow 64-bit indexing");
  if (width > 8) return fail(SSM_ERR_UNSUPPORTED, "conv width > 8 is not supported");
  const size_t as = dsize(act_dtype);
  if (!aligned(x, as) || !aligned(out, as) || !aligned(state_in, as) || !aligned(state_out, as) ||
      !aligned(weight, 4) || !aligned(bias, 4))
    return fail(SSM_ERR_ALIGNMENT, "a pointer is not aligned to its element size");
  if (batch == 0 || dim == 0) return SSM_OK;
  if (has_tok) {
    const char* x0 = (const char*)x;
    const char* x1 = x0 + (size_t)(batch * seqlen * dim) * as;
    const char* o0 = (const char*)out;
    const char* o1 = o0 + (size_t)(batch * seqlen * dim) * as;
    if (o0 < x1 && x0 < o1) return fail(SSM_ERR_SHAPE, "out must not overlap x");
  }
  ConvArgs a{};
  a.x = x; a.w = weight; a.bias = bias; a.state_in = state_in; a.out = out; a.state_out = state_out;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.width = width; a.silu = silu;
  a.act_bf16 = act_dtype == SSM_BF16;
  a.vec = dim % 8 == 0 && aligned16(x) && aligned16(out);
  return launch_conv(a, stream);
}

size_t ssm_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > 256) return 0;
  if (!elems_ok({batch, seqlen, dim, dstate})) return 0;
  return scan_bwd_ws_bytes(batch, seqlen, dim, dstate, false, false);
}

size_t ssm_scan_bwd_ex_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int flags) {
  if ((flags & ~(SSM_SCAN_REVERSE | SSM_SCAN_EULER | SSM_SCAN_DELTA_PER_TOKEN)) != 0) return 0;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > 256) return 0;
  if (!elems_ok({batch, seqlen, dim, dstate})) return 0;
  return scan_bwd_ws_bytes(batch, seqlen, dim, dstate, (flags & SSM_SCAN_DELTA_PER_TOKEN) != 0, false);
}

size_t ssm_scan_bwd_train_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int flags) {
  if ((flags & ~(SSM_SCAN_REVERSE | SSM_SCAN_EULER | SSM_SCAN_DELTA_PER_TOKEN)) != 0) return 0;
  if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate <= 0 || dstate > 256) return 0;
  if (!elems_ok({batch, seqlen, dim, dstate})) return 0;
  return scan_bwd_ws_bytes(batch, seqlen, dim, dstate, (flags & SSM_SCAN_DELTA_PER_TOKEN) != 0, true);
}

static int bwd_common(const void* x, const void* delta, const float* A, const void* B, const void* C,
                      const float* Dskip, const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                      const void* dout, const float* dh_final, void* dx, void* ddelta, float* dA, float* dB,
                      float* dC, float* dDskip, void* dz, float* ddelta_bias, float* dh0, int64_t batch,
                      int64_t seqlen, int64_t dim, int64_t dstate, int act_dtype, int delta_dtype, int flags,
                      void* workspace, size_t workspace_bytes, void* stream, const float* saved = nullptr,
                      bool want_saved = false) {
  g_last_error.clear();
  if ((flags & ~(SSM_SCAN_REVERSE | SSM_SCAN_EULER | SSM_SCAN_DELTA_PER_TOKEN)) != 0)
    return fail(SSM_ERR_UNSUPPORTED, "unknown scan flag bits");
  int rc = validate_scan(x, delta, A, B, C, dx, false, Dskip, z, delta_bias, h0, dh0, batch, seqlen, dim, dstate,
                         act_dtype, delta_dtype, delta_softplus);
  if (rc != SSM_OK) return rc;
  const bool has_tok = batch > 0 && seqlen > 0 && dim > 0;
  if ((has_tok && (dout == nullptr || ddelta == nullptr || dB == nullptr || dC == nullptr)) ||
      (dim > 0 && dA == nullptr) || (has_tok && z != nullptr && dz == nullptr) ||
      (dim > 0 && Dskip != nullptr && dDskip == nullptr) || (dim > 0 && delta_bias != nullptr && ddelta_bias == nullptr))
    return fail(SSM_ERR_NULL, "dout, dx, ddelta, dA, dB, dC and the gradients of the optional inputs given are required");
  if (dstate > 256) return fail(SSM_ERR_UNSUPPORTED, "the backward pass supports dstate <= 256");
  if (want_saved && has_tok && saved == nullptr) return fail(SSM_ERR_NULL, "states is required");
  if (!aligned(saved, 4)) return fail(SSM_ERR_ALIGNMENT, "states must be 4-byte aligned");
  const size_t as = dsize(act_dtype), ds = dsize(delta_dtype);
  if (!aligned(dout, as) || !aligned(dx, as) || !aligned(dz, as) || !aligned(ddelta, ds) || !aligned(dA, 4) ||
      !aligned(dB, 4) || !aligned(dC, 4) || !aligned(dDskip, 4) || !aligned(ddelta_bias, 4) ||
      !aligned(dh_final, 4))
    return fail(SSM_ERR_ALIGNMENT, "a pointer is not aligned to its element size");
  if (batch == 0 || dim == 0) return SSM_OK;
  hipStream_t st = (hipStream_t)stream;
  Scratch own;
  void* ws = nullptr;
  const bool tok = (flags & SSM_SCAN_DELTA_PER_TOKEN) != 0;
  rc = get_workspace(workspace, workspace_bytes,
                     seqlen > 0 ? scan_bwd_ws_bytes(batch, seqlen, dim, dstate, tok, want_saved) : 0, st,
                     &own, &ws);
  if (rc != SSM_OK) return rc;
  BwdArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.z = z; a.delta_bias = delta_bias;
  a.h0 = h0; a.dout = dout; a.dh_final = dh_final;
  a.dx = dx; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC;
  a.dDskip = Dskip != nullptr ? dDskip : nullptr;
  a.dz = z != nullptr ? dz : nullptr;
  a.ddelta_bias = delta_bias != nullptr ? ddelta_bias : nullptr;
  a.dh0 = dh0; a.ws_ckpt = (float*)ws;
  a.batch = batch; a.seqlen = seqlen; a.dim = dim; a.dstate = dstate;
  a.softplus = delta_softplus; a.act_bf16 = act_dtype == SSM_BF16; a.delta_bf16 = delta_dtype == SSM_BF16;
  a.reverse = (flags & SSM_SCAN_REVERSE) != 0;
  a.euler = (flags & SSM_SCAN_EULER) != 0;
  a.tok_delta = tok;
  a.saved = want_saved ? saved : nullptr;
  return launch_scan_bwd(a, stream);
}

int ssm_scan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C, const float* Dskip,
                 const void* z, const float* delta_bias, int delta_softplus, const float* h0, const void* dout,
                 const float* dh_final, void* dx, void* ddelta, float* dA, float* dB, float* dC, float* dDskip,
                 void* dz, float* ddelta_bias, float* dh0, int64_t batch, int64_t seqlen, int64_t dim,
                 int64_t dstate, int act_dtype, int delta_dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return bwd_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, dout, dh_final, dx, ddelta, dA, dB,
                    dC, dDskip, dz, ddelta_bias, dh0, batch, seqlen, dim, dstate, act_dtype, delta_dtype, 0,
                    workspace, workspace_bytes, stream);
}

int ssm_scan_bwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                    const void* dout, const float* dh_final, void* dx, void* ddelta, float* dA, float* dB, float* dC,
                    float* dDskip, void* dz, float* ddelta_bias, float* dh0, int64_t batch, int64_t seqlen,
                    int64_t dim, int64_t dstate, int act_dtype, int delta_dtype, int flags, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return bwd_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, dout, dh_final, dx, ddelta, dA, dB,
                    dC, dDskip, dz, ddelta_bias, dh0, batch, seqlen, dim, dstate, act_dtype, delta_dtype, flags,
                    workspace, workspace_bytes, stream);
}

int ssm_scan_bwd_train(const void* x, const void* delta, const float* A, const void* B, const void* C,
                       const float* Dskip, const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                       const void* dout, const float* dh_final, void* dx, void* ddelta, float* dA, float* dB, float* dC,
                       float* dDskip, void* dz, float* ddelta_bias, float* dh0, int64_t batch, int64_t seqlen,
                       int64_t dim, int64_t dstate, int act_dtype, int delta_dtype, int flags, const float* states,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, dout, dh_final, dx, ddelta, dA, dB,
                    dC, dDskip, dz, ddelta_bias, dh0, batch, seqlen, dim, dstate, act_dtype, delta_dtype, flags,
                    workspace, workspace_bytes, stream, states, true);
}

}  // extern "C"
