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
// One workgroup of 4 waves per (batch, head, 4 * 64 / LPC head channels).  A
// channel's states are spread over LPC lanes (8 to 64), NPL per lane (at most
// 4 from 33 states up): lane (c, q) = (lane / LPC, lane % LPC) holds channel
// c's states q NPL .. q NPL + NPL - 1.  Few states per lane give many waves:
// with 128 states, 32 lanes per channel make 4 waves per SIMD on the
// b2 x 64-head x 64-channel layer where 8 lanes of 16 states made one, whose
// per-token latency the other waves cannot hide.  Tiles of 32 tokens are staged
// in LDS: the B and C rows (read by all the workgroup's channels), x,
// silu(z), and the per-token decay and gain (one lane per token); each tile's
// inputs are loaded into registers while the previous tile is computed.  The
// readout's sum over a channel's LPC lanes is DPP adds: butterflies within
// groups of 8 and rows of 16 lanes, then row broadcasts (lane 15 of a row into
// the next row, lane 31 into rows 2 and 3) that leave the total in the
// channel's last lane.  The workgroups walk their sequence independently.
#include "scan_impl.h"

#include <type_traits>

namespace ssm {
namespace {

using namespace scan_dev;

constexpr int RT = 32;       // tokens per tile
constexpr int RW = 4;        // waves per workgroup

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
// v plus the DPP-moved v in the rows of ROWS (row mask); other rows keep v.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_rows(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false));
}
// Sum over the LPC lanes of an aligned group; the total ends in the group's last lane (in every lane
// of the group for 8 and 16).
template <int LPC>
__device__ __forceinline__ float sum_lanes(float v) {
  v = sum8(v);
  if constexpr (LPC >= 16) v = dpp_add<0x140>(v);                    // row_mirror: the two halves of a row
  if constexpr (LPC == 32) v = dpp_add_rows<0x142, 0xA>(v);          // row_bcast:15 into rows 1 and 3
  if constexpr (LPC == 64) {
    v = dpp_add_rows<0x142, 0xA>(v);                                 // rows 1 and 3: rows 0+1, 2+3
    v = dpp_add_rows<0x143, 0xC>(v);                                 // row_bcast:31 into rows 2 and 3
  }
  return v;
}

template <bool XF, bool DTB, int NPL, int LPC>
__global__ __launch_bounds__(64 * RW) void ssd_rec_kernel(SsdArgs a) {
  constexpr int NP = LPC * NPL;        // padded state count
  constexpr int CPW = 64 / LPC;        // channels per wave
  constexpr int RC = CPW * RW;         // head channels per workgroup
  __shared__ float sB[RT * NP], sC[RT * NP];
  __shared__ float sX[RT * RC], sZ[RT * RC];
  __shared__ float sE[RT], sG[RT];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l / LPC, q = l % LPC;
  const int64_t H = a.nheads, P = a.headdim, L = a.seqlen, G = a.ngroups, N = a.dstate;
  const int64_t ncg = (P + RC - 1) / RC;
  const int64_t cg = blockIdx.x % ncg;
  const int64_t h = (blockIdx.x / ncg) % H;
  const int64_t b = (blockIdx.x / ncg) / H;
  const int64_t grp = h / (H / G);
  const float av = a.A[h];
  const float bias = a.dt_bias != nullptr ? a.dt_bias[h] : 0.f;
  const float Dv = a.Dskip != nullptr ? a.Dskip[h] : 0.f;
  const int cw = CPW * w + c;                       // this lane's channel within the workgroup
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

  // ---- staging: each tile's inputs go into registers (raw bits) one tile ahead, then into LDS
  using RawA = typename std::conditional<XF, float, unsigned short>::type;   // B, C, x, z storage
  using RawD = typename std::conditional<DTB, unsigned short, float>::type;  // dt storage
  auto widen_a = [](RawA v) -> float {
    if constexpr (XF) return v;
    else return __builtin_bit_cast(float, (unsigned)v << 16);
  };
  auto widen_d = [](RawD v) -> float {
    if constexpr (DTB) return __builtin_bit_cast(float, (unsigned)v << 16);
    else return v;
  };
  constexpr int NT = 64 * RW;
  constexpr int KBC = (RT * NP + NT - 1) / NT;   // B (and C) items per thread per tile
  constexpr int KXZ = (RT * RC + NT - 1) / NT;   // x (and z) items per thread per tile
  const RawA* gB = reinterpret_cast<const RawA*>(a.B);
  const RawA* gC = reinterpret_cast<const RawA*>(a.C);
  const RawA* gX = reinterpret_cast<const RawA*>(a.x);
  const RawA* gZ = reinterpret_cast<const RawA*>(a.z);
  const RawD* gD = reinterpret_cast<const RawD*>(a.dt);
  RawA pb[KBC], pc[KBC], px[KXZ], pz[KXZ];
  RawD pdt = 0;
  // rows past the end load the last row (their values are not used)
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int j = 0; j < KBC; ++j) {
      const int i = tid + NT * j;
      if ((RT * NP) % NT != 0 && i >= RT * NP) break;
      const int t = i / NP, n = i % NP;
      const int64_t tt = t0 + t < L ? t0 + t : L - 1;
      const int64_t gi = ((b * L + tt) * G + grp) * N + (n < N ? n : 0);
      pb[j] = gB[gi];
      pc[j] = gC[gi];
    }
#pragma unroll
    for (int j = 0; j < KXZ; ++j) {
      const int i = tid + NT * j;
      if ((RT * RC) % NT != 0 && i >= RT * RC) break;
      const int t = i / RC, pcx = i % RC;
      const int64_t pp = cg * RC + pcx;
      const int64_t tt = t0 + t < L ? t0 + t : L - 1;
      const int64_t gi = ((b * L + tt) * H + h) * P + (pp < P ? pp : P - 1);
      px[j] = gX[gi];
      if (a.z != nullptr) pz[j] = gZ[gi];
    }
    if (tid < RT) {
      const int64_t tt = t0 + tid < L ? t0 + tid : L - 1;
      pdt = gD[(b * L + tt) * H + h];
    }
  };
  auto put = [&](int64_t t0) {
#pragma unroll
    for (int j = 0; j < KBC; ++j) {
      const int i = tid + NT * j;
      if ((RT * NP) % NT != 0 && i >= RT * NP) break;
      const int t = i / NP, n = i % NP;
      const bool ok = t0 + t < L && n < N;
      sB[i] = ok ? widen_a(pb[j]) : 0.f;
      sC[i] = ok ? widen_a(pc[j]) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < KXZ; ++j) {
      const int i = tid + NT * j;
      if ((RT * RC) % NT != 0 && i >= RT * RC) break;
      const int t = i / RC, pcx = i % RC;
      const bool ok = t0 + t < L && cg * RC + pcx < P;
      sX[i] = ok ? widen_a(px[j]) : 0.f;
      sZ[i] = (ok && a.z != nullptr) ? silu_f(widen_a(pz[j])) : 1.f;
    }
    if (tid < RT) {
      const int64_t t = t0 + tid;
      float dt = 0.f;
      if (t < L) {
        const float v = widen_d(pdt) + bias;
        dt = a.softplus ? softplus_f(v) : v;
      }
      // past the end: no decay and no input
      const float e = hw_exp2(dt * av * kLog2e);
      sE[tid] = e;
      sG[tid] = zoh_gain_accurate(e, dt, av, 1.f / av);
    }
  };

  if (L > 0) fetch(0);   // (an empty sequence has no row to read)
  for (int64_t t0 = 0; t0 < L; t0 += RT) {
    put(t0);
    lds_sync();
    if (t0 + RT < L) fetch(t0 + RT);

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
      acc = sum_lanes<LPC>(acc);   // over the channel's LPC lanes
      if (q == LPC - 1 && p_ok) {
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

// (lanes per channel, states per lane): the smallest that holds dstate, at most 4 states per lane
// from 33 states up
template <int LPC>
constexpr int rec_channels_per_wg() { return 64 / LPC * RW; }
template <bool XF, bool DTB, int NPL, int LPC>
hipError_t launch_rec_shape(const SsdArgs& a, hipStream_t st) {
  constexpr int RC = rec_channels_per_wg<LPC>();
  const int64_t nwg = a.batch * a.nheads * ((a.headdim + RC - 1) / RC);
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (nwg == 0) return hipSuccess;
  ssd_rec_kernel<XF, DTB, NPL, LPC><<<(unsigned)nwg, 64 * RW, 0, st>>>(a);
  return hipGetLastError();
}
template <bool XF, bool DTB>
hipError_t launch_rec_n(const SsdArgs& a, hipStream_t st) {
  const int64_t N = a.dstate;
  if (N <= 8) return launch_rec_shape<XF, DTB, 1, 8>(a, st);
  if (N <= 16) return launch_rec_shape<XF, DTB, 2, 8>(a, st);
  if (N <= 32) return launch_rec_shape<XF, DTB, 4, 8>(a, st);
  if (N <= 64) return launch_rec_shape<XF, DTB, 4, 16>(a, st);
  if (N <= 128) return launch_rec_shape<XF, DTB, 4, 32>(a, st);
  return launch_rec_shape<XF, DTB, 4, 64>(a, st);
}

}  // namespace

int launch_ssd_rec(const SsdArgs& a, bool act_f32, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.dstate < 1 || a.dstate > kSsdRecMaxState) return fail(4, "SSD recurrence supports dstate 1..256");
  if (a.batch * a.nheads * a.headdim == 0) return 0;
  // the most workgroups any shape makes: 8 channels per workgroup
  if (a.batch * a.nheads * ((a.headdim + 7) / 8) > 0x7fffffffLL) return fail(4, "grid too large");
  hipError_t e;
  if (act_f32) e = a.dt_bf16 ? launch_rec_n<true, true>(a, st) : launch_rec_n<true, false>(a, st);
  else e = a.dt_bf16 ? launch_rec_n<false, true>(a, st) : launch_rec_n<false, false>(a, st);
  if (e != hipSuccess) return fail(6, std::string("SSD recurrence launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
