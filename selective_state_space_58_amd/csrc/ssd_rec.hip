// Mamba-2 SSD by its recurrence, for the calls the blocked matrix-core kernel
// (ssd_kernels.hip) does not take: fp32 activations, and head or state sizes
// other than 64 and 128.  With one scalar decay per head the SSD map is also a
// linear recurrence over tokens ("Mamba-2 / Structured State Space Duality":
// the SSM side of the duality; "Mamba / SSM complete guide" sec. 2, the
// recurrent view).  Per batch b, head h, head channel p and state n:
//   S[p][n] <- e^{dt a} S[p][n] + g(dt, a) B_t[n] x_t[p]
//   y_t[p]   = (C_t . S[p] + D x_t[p]) * silu(z_t[p])
// The decay and the ZOH gain g = (e^{dt a} - 1)/a are one per (token, head),
// so a state element costs one multiply and one FMA, and the readout one FMA.
//
// One workgroup of 4 waves per (batch, head, 32 head channels).  Wave w takes
// 8 channels; lane (c, q) = (lane / 8, lane % 8) holds channel c's states
// q NPL .. q NPL + NPL - 1 (dstate <= 8 NPL).  Tiles of 32 tokens
// are staged in LDS: the B and C rows (read by all 32 channels), x, silu(z),
// and the per-token decay and gain (one lane per token).  The readout's sum
// over a channel's states is three butterfly steps over the 8 lanes that hold
// them (DPP adds).  The workgroups walk their sequence independently, so a call with few
// (batch, head) pairs runs on few CUs.
#include "scan_impl.h"

namespace ssm {
namespace {

using namespace scan_dev;

constexpr int RT = 32;       // tokens per tile
constexpr int RW = 4;        // waves per workgroup
constexpr int RC = 8 * RW;   // head channels per workgroup

// Sum over the 8 lanes of an aligned group (lane bits 0-2), in every lane: quad swaps of 1 and 2
// lanes, then the half-row mirror (lane i with 7 - i) joins the two quads.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum8(float v) {
  v = dpp_add<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  return dpp_add<0x141>(v);   // row_half_mirror
}

__device__ __forceinline__ float ld_act(const void* p, int64_t i, bool f32) {
  if (f32) return reinterpret_cast<const float*>(p)[i];
  const unsigned u = (unsigned)reinterpret_cast<const unsigned short*>(p)[i] << 16;
  return __builtin_bit_cast(float, u);
}

template <bool XF, bool DTB, int NPL>
__global__ __launch_bounds__(64 * RW) void ssd_rec_kernel(SsdArgs a) {
  constexpr int NP = 8 * NPL;   // padded state count
  __shared__ float sB[RT * NP], sC[RT * NP];
  __shared__ float sX[RT * RC], sZ[RT * RC];
  __shared__ float sE[RT], sG[RT];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l >> 3, q = l & 7;
  const int64_t H = a.nheads, P = a.headdim, L = a.seqlen, G = a.ngroups, N = a.dstate;
  const int64_t ncg = (P + RC - 1) / RC;
  const int64_t cg = blockIdx.x % ncg;
  const int64_t h = (blockIdx.x / ncg) % H;
  const int64_t b = (blockIdx.x / ncg) / H;
  const int64_t grp = h / (H / G);
  const float av = a.A[h];
  const float bias = a.dt_bias != nullptr ? a.dt_bias[h] : 0.f;
  const float Dv = a.Dskip != nullptr ? a.Dskip[h] : 0.f;
  const int cw = 8 * w + c;                         // this lane's channel within the workgroup
  const int64_t p = cg * RC + cw;
  const bool p_ok = p < P;

  // state: lane (c, q) holds S[p][q NPL + k]
  const int64_t srow = ((b * H + h) * P + p) * N;
  float st[NPL];
#pragma unroll
  for (int k = 0; k < NPL; ++k) {
    const int64_t n = q * NPL + k;
    st[k] = (a.h0 != nullptr && p_ok && n < N) ? a.h0[srow + n] : 0.f;
  }

  for (int64_t t0 = 0; t0 < L; t0 += RT) {
    // ---- stage the tile
    for (int i = tid; i < RT * NP; i += 64 * RW) {
      const int t = i / NP, n = i % NP;
      const bool ok = t0 + t < L && n < N;
      const int64_t gi = ((b * L + t0 + t) * G + grp) * N + n;
      sB[i] = ok ? ld_act(a.B, gi, XF) : 0.f;
      sC[i] = ok ? ld_act(a.C, gi, XF) : 0.f;
    }
    for (int i = tid; i < RT * RC; i += 64 * RW) {
      const int t = i / RC, pc = i % RC;
      const int64_t pp = cg * RC + pc;
      const bool ok = t0 + t < L && pp < P;
      const int64_t gi = ((b * L + t0 + t) * H + h) * P + pp;
      sX[i] = ok ? ld_act(a.x, gi, XF) : 0.f;
      sZ[i] = (ok && a.z != nullptr) ? silu_f(ld_act(a.z, gi, XF)) : 1.f;
    }
    if (tid < RT) {
      const int64_t t = t0 + tid;
      float dt = 0.f;
      if (t < L) {
        const float v = ld_act(a.dt, (b * L + t) * H + h, !DTB) + bias;
        dt = a.softplus ? softplus_f(v) : v;
      }
      // past the end: no decay and no input
      const float e = hw_exp2(dt * av * kLog2e);
      sE[tid] = e;
      sG[tid] = zoh_gain_accurate(e, dt, av, 1.f / av);
    }
    lds_sync();

    // ---- the tile's tokens
    const int nt = (int)(L - t0 < RT ? L - t0 : RT);
    for (int t = 0; t < nt; ++t) {
      const float e = sE[t];
      const float xv = sX[t * RC + cw];
      const float gx = sG[t] * xv;
      const float* bt = sB + t * NP + q * NPL;
      const float* ct = sC + t * NP + q * NPL;
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < NPL; ++k) {
        st[k] = fmaf(e, st[k], gx * bt[k]);
        acc = fmaf(ct[k], st[k], acc);
      }
      acc = sum8(acc);   // over the channel's 8 lanes
      if (q == 0 && p_ok) {
        const float yv = fmaf(Dv, xv, acc) * sZ[t * RC + cw];
        const int64_t gi = ((b * L + t0 + t) * H + h) * P + p;
        if (XF) reinterpret_cast<float*>(a.y)[gi] = yv;
        else reinterpret_cast<unsigned short*>(a.y)[gi] = __builtin_bit_cast(unsigned short, (__bf16)yv);
      }
    }
    lds_sync();   // the tile's LDS is rewritten next
  }

  if (a.h_final != nullptr && p_ok) {
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const int64_t n = q * NPL + k;
      if (n < N) a.h_final[srow + n] = st[k];
    }
  }
}

template <bool XF, bool DTB>
hipError_t launch_rec_n(const SsdArgs& a, unsigned grid, hipStream_t st) {
  const int64_t N = a.dstate;
  const int npl = (int)((N + 7) / 8);
  if (npl <= 1) ssd_rec_kernel<XF, DTB, 1><<<grid, 64 * RW, 0, st>>>(a);
  else if (npl <= 2) ssd_rec_kernel<XF, DTB, 2><<<grid, 64 * RW, 0, st>>>(a);
  else if (npl <= 4) ssd_rec_kernel<XF, DTB, 4><<<grid, 64 * RW, 0, st>>>(a);
  else if (npl <= 8) ssd_rec_kernel<XF, DTB, 8><<<grid, 64 * RW, 0, st>>>(a);
  else if (npl <= 16) ssd_rec_kernel<XF, DTB, 16><<<grid, 64 * RW, 0, st>>>(a);
  else ssd_rec_kernel<XF, DTB, 32><<<grid, 64 * RW, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int launch_ssd_rec(const SsdArgs& a, bool act_f32, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.dstate < 1 || a.dstate > kSsdRecMaxState) return fail(4, "SSD recurrence supports dstate 1..256");
  const int64_t ncg = (a.headdim + RC - 1) / RC;
  const int64_t nwg = a.batch * a.nheads * ncg;
  if (nwg > 0x7fffffffLL) return fail(4, "grid too large");
  if (nwg == 0) return 0;
  hipError_t e;
  if (act_f32) e = a.dt_bf16 ? launch_rec_n<true, true>(a, (unsigned)nwg, st) : launch_rec_n<true, false>(a, (unsigned)nwg, st);
  else e = a.dt_bf16 ? launch_rec_n<false, true>(a, (unsigned)nwg, st) : launch_rec_n<false, false>(a, (unsigned)nwg, st);
  if (e != hipSuccess) return fail(6, std::string("SSD recurrence launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
