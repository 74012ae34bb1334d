// Single-token state update (recurrent inference) for the selective SSM and
// its Mamba-2 form.
//
// Generation runs the recurrence one token at a time and keeps only the
// fixed-size state ("Mamba / SSM complete guide", sec. 2 recurrent view and
// sec. 4 inference; "Mamba-2 / Structured State Space Duality", inference:
// the past is compressed into the state, no growing cache).  One call advances
// every (batch, channel) state by one token:
//   dt     = softplus?(delta + bias)
//   h_n   <- exp(dt a_n) h_n + (exp(dt a_n) - 1)/a_n * B_n x
//   y      = (sum_n C_n h_n + Dskip x) * silu(z)
// with a_n = A[d, n] (Mamba, diagonal A per channel) or a_n = A[head] (Mamba-2,
// one scalar per head; dt, bias and Dskip per head, B and C per group).
//
// The step is bound by HBM: every state entry is read and written once
// (8 bytes) for ~8 flops.  A group of G lanes owns one channel's state; lane j
// of the group holds states [4j, 4j+4) and moves them with one 16-byte load
// and store when the layout allows, so a wave streams 1 KB of contiguous state
// per access; each lane group handles 2 or 4 channels a block apart and issues all
// their state loads first, to keep enough bytes in flight to cover HBM
// latency.  The state is touched once per call, so its loads and stores carry
// the nontemporal (streaming) hint: measured 165.7 -> 147.6 us on the b128 x
// 80-head Mamba-2 decode (4.57 TB/s) and 27.9 -> 26.7 us on the b128 x
// 5120-channel Mamba decode.  The readout sum is reduced over the G lanes of the group with
// cross-lane shuffles; lane 0 of the group applies skip and gate and stores y.
#include <hip/hip_runtime.h>

#include "scan_impl.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using scan_dev::hw_exp2;
using scan_dev::kLog2e;
using scan_dev::silu_f;
using scan_dev::softplus_f;

constexpr int kStepThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_act(const void* p, int64_t i, bool bf16) {
  if (bf16) return __builtin_bit_cast(float, (unsigned)(((const unsigned short*)p)[i]) << 16);
  return ((const float*)p)[i];
}

// 4 consecutive act values starting at element i (i is a multiple of 4 and
// the row is 8/16-byte aligned when vec is set).
__device__ __forceinline__ void load_act4(const void* p, int64_t i, bool bf16, bool vec, int valid, float (&v)[4]) {
  if (vec) {
    if (bf16) {
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 r = *reinterpret_cast<const u32x2*>((const unsigned short*)p + i);
      const unsigned r0 = r[0], r1 = r[1];
      v[0] = __builtin_bit_cast(float, r0 << 16);
      v[1] = __builtin_bit_cast(float, r0 & 0xffff0000u);
      v[2] = __builtin_bit_cast(float, r1 << 16);
      v[3] = __builtin_bit_cast(float, r1 & 0xffff0000u);
    } else {
      const float4 r = *reinterpret_cast<const float4*>((const float*)p + i);
      v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = k < valid ? load_act(p, i + k, bf16) : 0.f;
}

// ZOH gain (e^q - 1)/a, q = dt*a, accurate to ~5e-7 relative for every q:
// expm1(q)/q by its Taylor series (truncation < 8e-10) for |q| < 1/8, the
// direct form (cancellation < 6e-8/|q|) above.  a == 0 gives dt.
__device__ __forceinline__ float step_gain(float E, float dt, float a) {
  const float q = dt * a;
  const float phi = fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, 1.f / 720.f, 1.f / 120.f), 1.f / 24.f), 1.f / 6.f), 0.5f),
                         1.f);
  return fabsf(q) < 0.125f ? dt * phi : (E - 1.f) * scan_dev::hw_rcp(a);
}

// U channels per lane group, a block of lane groups apart: the state loads of
// all U channels are issued before any is used, so each wave keeps U x 1 KB of
// state in flight.  The grid is (channel blocks per batch row) x batch rows,
// linearised; PER_HEAD selects the Mamba-2 layout (one A, dt, bias, Dskip per
// head), where the decay and gain are the same for every state of a channel.
template <int G, bool VEC, bool PER_HEAD, int U>
__global__ __launch_bounds__(kStepThreads) void state_update_kernel(StepArgs a, unsigned blocks_per_row,
                                                                    int headdim_shift) {
  constexpr int CPB = kStepThreads / G;  // lane groups per block
  const unsigned b = blockIdx.x / blocks_per_row;
  const unsigned dblk = blockIdx.x - b * blocks_per_row;
  const unsigned dim = (unsigned)a.dim;
  const unsigned nheads = PER_HEAD ? dim / (unsigned)a.headdim : dim;
  const unsigned hpg = nheads / (unsigned)a.ngroups;
  const int N = (int)a.dstate;
  const int j = threadIdx.x % G;
  const int n0 = 4 * j;
  const int valid = N - n0 < 4 ? (N - n0 > 0 ? N - n0 : 0) : 4;
  const unsigned d0 = dblk * (unsigned)(CPB * U) + threadIdx.x / G;
  const size_t row = (size_t)b * dim;

  auto head_of = [&](unsigned d) -> unsigned {
    if (!PER_HEAD) return d;
    return headdim_shift >= 0 ? d >> headdim_shift : d / (unsigned)a.headdim;
  };

  float h[U][4], Av[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned d = d0 + u * CPB;
    if (d >= dim || valid == 0) continue;
    const float* st = a.state + (row + d) * N + n0;
    if (VEC) {
      const f32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st));
      h[u][0] = hv[0]; h[u][1] = hv[1]; h[u][2] = hv[2]; h[u][3] = hv[3];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) h[u][k] = k < valid ? st[k] : 0.f;
    }
    if (!PER_HEAD) {
      if (VEC) {
        const float4 av = *reinterpret_cast<const float4*>(a.A + (size_t)d * N + n0);
        Av[u][0] = av.x; Av[u][1] = av.y; Av[u][2] = av.z; Av[u][3] = av.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) Av[u][k] = k < valid ? a.A[(size_t)d * N + n0 + k] : 0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const unsigned d = d0 + u * CPB;
    if (d >= dim) break;  // a whole lane group leaves together; later u are past the end too
    const unsigned head = head_of(d);
    const unsigned grp = a.ngroups == 1 ? 0u : head / hpg;
    const float v = load_act(a.delta, (int64_t)b * nheads + head, a.delta_bf16) +
                    (a.delta_bias != nullptr ? a.delta_bias[head] : 0.f);
    const float dt = a.softplus ? softplus_f(v) : v;
    const float xv = load_act(a.x, row + d, a.act_bf16);
    float acc = 0.f;
    if (valid > 0) {
      const int64_t bc = ((int64_t)b * a.ngroups + grp) * N + n0;
      float Bv[4], Cv[4];
      load_act4(a.B, bc, a.act_bf16, VEC, valid, Bv);
      load_act4(a.C, bc, a.act_bf16, VEC, valid, Cv);
      if (PER_HEAD) {
        const float ah = a.A[head];
        const float E = hw_exp2(dt * ah * kLog2e);
        const float gx = step_gain(E, dt, ah) * xv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[u][k] = fmaf(E, h[u][k], gx * Bv[k]);
          acc = fmaf(Cv[k], h[u][k], acc);
        }
      } else {
        const float dtl = dt * kLog2e;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float an = Av[u][k];
          const float E = hw_exp2(dtl * an);
          h[u][k] = fmaf(E, h[u][k], step_gain(E, dt, an) * (Bv[k] * xv));
          acc = fmaf(Cv[k], h[u][k], acc);
        }
      }
      float* st = a.state + (row + d) * N + n0;
      if (VEC) {
        __builtin_nontemporal_store(f32x4{h[u][0], h[u][1], h[u][2], h[u][3]}, reinterpret_cast<f32x4*>(st));
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (k < valid) st[k] = h[u][k];
      }
    }
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, G);
    if (j == 0) {
      float yv = acc;
      if (a.Dskip != nullptr) yv = fmaf(a.Dskip[head], xv, yv);
      if (a.z != nullptr) yv *= silu_f(load_act(a.z, row + d, a.act_bf16));
      if (a.act_bf16) ((__bf16*)a.y)[row + d] = (__bf16)yv;
      else ((float*)a.y)[row + d] = yv;
    }
  }
}

// Channels per lane group: 4 for the per-head (Mamba-2) layout, 2 for the
// per-channel one (measured 166 vs 178 us and 29.6 vs 27.7 us on the
// serving-batch decode workloads).
constexpr int kStepUnroll = 4;
constexpr int kStepUnrollChannel = 2;

template <int G>
hipError_t launch_g(const StepArgs& a, hipStream_t st) {
  constexpr int CPB = kStepThreads / G;
  const int u = a.a_per_head ? kStepUnroll : kStepUnrollChannel;
  const unsigned bpr = (unsigned)((a.dim + CPB * u - 1) / (CPB * u));
  const dim3 grid((unsigned)(bpr * a.batch));
  int shift = -1;
  if (a.a_per_head && (a.headdim & (a.headdim - 1)) == 0) {
    shift = 0;
    while ((1LL << shift) < a.headdim) ++shift;
  }
  if (a.a_per_head) {
    if (a.vec) state_update_kernel<G, true, true, kStepUnroll><<<grid, kStepThreads, 0, st>>>(a, bpr, shift);
    else state_update_kernel<G, false, true, kStepUnroll><<<grid, kStepThreads, 0, st>>>(a, bpr, shift);
  } else {
    if (a.vec) state_update_kernel<G, true, false, kStepUnrollChannel><<<grid, kStepThreads, 0, st>>>(a, bpr, shift);
    else state_update_kernel<G, false, false, kStepUnrollChannel><<<grid, kStepThreads, 0, st>>>(a, bpr, shift);
  }
  return hipGetLastError();
}

}  // namespace

int launch_state_update(const StepArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.batch * a.dim == 0) return 0;
  int G = 1;
  while (4 * G < a.dstate) G *= 2;
  if (G > 64) return fail(4, "dstate > 256 is not supported by the state update");
  if (a.dim > 0x7fffffffLL - kStepThreads * kStepUnroll) return fail(4, "too many channels");
  const int64_t bpr = (a.dim + (kStepThreads / G) * kStepUnrollChannel - 1) / ((kStepThreads / G) * kStepUnrollChannel);
  if (bpr * a.batch > 0x7fffffffLL) return fail(4, "grid too large");
  hipError_t e;
  switch (G) {
    case 1: e = launch_g<1>(a, st); break;
    case 2: e = launch_g<2>(a, st); break;
    case 4: e = launch_g<4>(a, st); break;
    case 8: e = launch_g<8>(a, st); break;
    case 16: e = launch_g<16>(a, st); break;
    case 32: e = launch_g<32>(a, st); break;
    default: e = launch_g<64>(a, st); break;
  }
  if (e != hipSuccess) return fail(6, std::string("state update launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
