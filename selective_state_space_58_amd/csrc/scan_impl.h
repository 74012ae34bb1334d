// Selective scan (Mamba S6) kernel template for MI355X / gfx950.
//
// Computes, per (batch b, channel d) slice and per state n, with exact ZOH for a
// diagonal A ("SSM & Mamba", Discretization/ZOH; "Paper explainer: Mamba",
// Technical details):
//   dt_t   = softplus(delta_t + bias_d)  (or delta_t + bias_d)
//   h_t,n  = exp(dt_t a_dn) h_{t-1,n} + (exp(dt_t a_dn) - 1)/a_dn * B_t,n x_t
//   y_t    = (sum_n C_t,n h_t,n + Dskip_d x_t) * silu(z_t)
// ("Mamba / SSM complete guide", sec. 5, selective_scan and the block's gate).
//
// Mapping to CDNA4.  The 64 lanes of a wave are R rows of 64/R columns (R = 4,
// 8 or 16): lane (row r, column c) holds states [r*S, r*S+S) of channel ch0+c
// in VGPRs for the whole sequence, so the state never touches memory.  (With
// 16 rows the four lanes of a quad are one channel's rows, see TileShape.)
// More rows give fewer channels per wave and so more waves for a given layer:
// the host picks R so that every SIMD gets waves to interleave.  The work per (t, d, n) element is 6 VALU ops plus one
// v_exp_f32; the per-(t, d) work (softplus, silu, skip, bf16 conversion,
// stores) is done once, not per state.
//   * Per time tile (T tokens) the wave stages (dt, x) and silu(z) per
//     (token, channel) and B_t, C_t (fp32) per (token, row) in LDS; the global
//     loads for the next tile are issued before the current tile is scanned.
//   * The readout sum over n is split over the R rows; every R tokens a
//     reduce-scatter over the rows (v_permlane32_swap / v_permlane16_swap for
//     lanes 32 and 16 apart, a DPP row rotation or a swizzle for 8 and 4, DPP
//     quad permutations for 2 and 1) leaves row r with the full sum for token
//     Rk + r, and that lane applies the skip and gate and stores y for that
//     token.
//   * Lanes whose channel is past `dim` load from a clamped (valid) address
//     and compute values that are never stored; a column never mixes with
//     another column, so nothing leaks.  Tokens past the end of the slice get
//     dt = 0, which leaves the state unchanged (exp(0) = 1, gain 0).
//
// ZOH gain accuracy: (exp(q) - 1)/a loses ~6e-8/|q| relative accuracy for small
// q = dt*a.  fp32 activations (and any wave that holds an |a| < 1e-2) take an
// accurate form dt * phi(q), phi(q) = expm1(q)/q by its Taylor series for
// |q| < 1/4; bf16 activations take the short form, whose error is far below
// bf16 resolution.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "device_common.h"
#include "ssm_internal.h"

namespace ssm {
namespace scan_dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }

template <bool BF16>
struct Act;
template <>
struct Act<true> {
  using T = __bf16;
};
template <>
struct Act<false> {
  using T = float;
};

// Raw storage bits held in the prefetch registers: bf16 stays 16-bit until it
// is staged, so the loads of the next tile are not waited on early.
template <bool BF16>
struct Raw;
template <>
struct Raw<true> {
  using T = unsigned short;
  __device__ static float f32(T v) { return __builtin_bit_cast(float, (unsigned)v << 16); }
};
template <>
struct Raw<false> {
  using T = float;
  __device__ static float f32(T v) { return v; }
};

// log(1 + e^v) without overflow.  Short form: log1p(e^-|v|) as log2(1 + e)*ln2,
// whose absolute error (< 6e-8) is far below bf16 resolution of the output.
// For v > 17, 1 + e rounds to 1 and the result is v itself; max(v, 0) is a median of three.
__device__ __forceinline__ float softplus_short(float v) {
  const float e = hw_exp2(-fabsf(v) * kLog2e);
  return __builtin_amdgcn_fmed3f(v, 0.f, __builtin_inff()) + hw_log2(1.f + e) * kLn2;
}

// Accurate form: log1p(e^-|v|) by its series when e^-|v| < 1/16.
__device__ __forceinline__ float softplus_f(float v) {
  const float e = hw_exp2(-fabsf(v) * kLog2e);
  const float ser = e * fmaf(e, fmaf(e, fmaf(e, fmaf(e, fmaf(e, -1.f / 6.f, 0.2f), -0.25f), 1.f / 3.f), -0.5f), 1.f);
  const float lg = hw_log2(1.f + e) * kLn2;
  const float r = fmaxf(v, 0.f) + (e < 0.0625f ? ser : lg);
  return v > 20.f ? v : r;
}

__device__ __forceinline__ float silu_f(float z) { return z * hw_rcp(1.f + hw_exp2(-z * kLog2e)); }

// ZOH gain (e^q - 1)/a with q = dt*a, accurate for small |q| (a == 0 gives dt).
__device__ __forceinline__ float zoh_gain_accurate(float E, float dt, float a, float ia) {
  const float q = dt * a;
  const float phi = fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, 1.f / 5040.f, 1.f / 720.f), 1.f / 120.f),
                                                 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
  const float g_long = fmaf(E, ia, -ia);
  return fabsf(q) < 0.25f ? dt * phi : g_long;
}

__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }

// One level of the row reduce-scatter: lanes whose bit `D` (a lane distance
// of 32, 16, 8, 4, 2 or 1) is clear end with a + a(lane ^ D), the others with
// b + b(lane ^ D).
template <int D>
__device__ __forceinline__ float pair_sum(float a, float b) {
  if constexpr (D == 32) {
    // permlane32_swap(a, b): a' = [a.lo | b.lo], b' = [a.hi | b.hi]  (halves of 32 lanes)
    const auto sw = __builtin_amdgcn_permlane32_swap(f_bits(a), f_bits(b), false, false);
    return bits_f(sw[0]) + bits_f(sw[1]);
  } else if constexpr (D == 16) {
    // permlane16_swap(a, b): odd 16-lane rows of a <-> even 16-lane rows of b
    const auto sw = __builtin_amdgcn_permlane16_swap(f_bits(a), f_bits(b), false, false);
    return bits_f(sw[0]) + bits_f(sw[1]);
  } else {
    const bool up = (__lane_id() & D) != 0;
    const float keep = up ? b : a, send = up ? a : b;
    int other;
    if constexpr (D == 8) {
      other = __builtin_amdgcn_update_dpp(0, (int)f_bits(send), 0x128, 0xf, 0xf, false);  // row_ror:8 = lane ^ 8
    } else if constexpr (D == 2) {
      other = __builtin_amdgcn_mov_dpp((int)f_bits(send), 0x4E, 0xf, 0xf, true);   // quad_perm [2,3,0,1]
    } else if constexpr (D == 1) {
      other = __builtin_amdgcn_mov_dpp((int)f_bits(send), 0xB1, 0xf, 0xf, true);   // quad_perm [1,0,3,2]
    } else {
      static_assert(D == 4, "row distance");
      other = __builtin_amdgcn_ds_swizzle((int)f_bits(send), 0x101f);  // bit mode: xor 4 within 32 lanes
    }
    return keep + bits_f((unsigned)other);
  }
}

// Value J of each quad of lanes in all four lanes of the quad (DPP quad_perm [J,J,J,J]).  As the
// operand of a VALU op the broadcast folds into the op itself.
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return bits_f((unsigned)__builtin_amdgcn_mov_dpp((int)f_bits(v), J * 0x55, 0xf, 0xf, true));
}

// Calls f(std::integral_constant<int, J>) for J = 0 .. N-1 (indices usable as template arguments).
template <int... J, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, J...>, F&& f) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// Lanes are R rows of 64/R (row = lane / (64/R)).  p[j] holds, in every lane,
// a partial sum for token j of a group of R.  Returns, in row r, the sum over
// the R rows of the same column of p[r]: each level pairs value i with value
// i + K/2 across the highest remaining lane bit, so the token index ends up
// equal to the row index.
template <int R>
__device__ __forceinline__ float reduce_scatter_rows(const float (&p)[R]) {
  float v[R];
#pragma unroll
  for (int j = 0; j < R; ++j) v[j] = p[j];
  // lane bits 5, 4, ... down to log2(64 / R)
#pragma unroll
  for (int K = R, D = 32; K > 1; K /= 2, D /= 2) {
#pragma unroll
    for (int i = 0; i < K / 2; ++i) {
      if (D == 32) v[i] = pair_sum<32>(v[i], v[i + K / 2]);
      else if (D == 16) v[i] = pair_sum<16>(v[i], v[i + K / 2]);
      else if (D == 8) v[i] = pair_sum<8>(v[i], v[i + K / 2]);
      else v[i] = pair_sum<4>(v[i], v[i + K / 2]);
    }
  }
  return v[0];
}

// The same for the 16-row quad layout (row = 4 * lane bits 4-5 + lane bits 0-1): the levels run over
// lane bits 5, 4, 1 and 0, which leaves row r with token r's sum as above.
__device__ __forceinline__ float reduce_scatter_quad16(const float (&p)[16]) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = pair_sum<32>(p[i], p[i + 8]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pair_sum<16>(v[i], v[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) v[i] = pair_sum<2>(v[i], v[i + 2]);
  return pair_sum<1>(v[0], v[1]);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int NW>
struct VecOf;
template <>
struct VecOf<4> {
  using T = u32x4;
};
template <>
struct VecOf<2> {
  using T = u32x2;
};
// (one word: a chunk of two bf16 delta values beside fp32 x, and the bf16 8-row wide-lane tiles, whose
// vector path is never taken)
typedef unsigned u32x1 __attribute__((ext_vector_type(1)));
template <>
struct VecOf<1> {
  using T = u32x1;
};

// V: the vector tile path (the one-wave tile paths of the 8- and 16-row layouts take 32-token tiles,
// whose prefetched items fit their registers; 64-token ones spilled)
template <int R_, int S, bool V = true>
struct TileShape {
  static constexpr int R = R_;
  static constexpr int CH = 64 / R;                // channels per wave
  static constexpr int NP = R * S;                 // padded state count of the wave
  static constexpr int T = R == 4 ? 32 : (S >= 16 ? 16 : (!V ? 32 : 64));   // tokens per LDS tile
  static constexpr int KX = T / R;                 // (token, channel) items per lane per tile
  static constexpr int KB = T * NP / 64;           // B (and C) items per lane per tile
  // lane -> (row, column).  4 and 8 rows: lane = row * CH + column.  16 rows (4 channels, one
  // state per lane): the column is lane bits 2-3 and the row 4 * (lane bits 4-5) + lane bits 0-1,
  // so that the four lanes of a quad belong to one channel.
  static __device__ __forceinline__ int row_of(int lane) { return R == 16 ? ((lane >> 4) << 2) | (lane & 3) : lane / CH; }
  static __device__ __forceinline__ int col_of(int lane) { return R == 16 ? (lane >> 2) & 3 : lane % CH; }
  // Row stride (in pairs) of the staged (dt, x) tile of a W-wave workgroup, and of the gate tile
  // unless GZ2.  The 16-row layout reads four token rows at once (one per quad lane): rows of 20
  // pairs put those reads on distinct LDS banks, where rows of 16 pairs would share them.
  template <int W>
  static constexpr int xs() { return CH * W + (R == 16 ? 4 : 0); }
  // The 16-row layout's gate tile holds (D x, silu z) pairs, read once per 16 tokens by the
  // readout (sixteen rows at once, on distinct banks with rows of 20 pairs as well).
  static constexpr bool GZ2 = R == 16;
  template <int W>
  static constexpr int gz_floats() { return (GZ2 ? 2 : 1) * T * xs<W>(); }
};

// GAIN: kGainShort (e^q - 1)/a, kGainAccurate (series near q = 0), kGainEuler dt.
enum GainMode : int { kGainShort = 0, kGainAccurate = 1, kGainEuler = 2 };

template <int RR, bool XB, bool DB, int S, int MODE, int GAIN, bool VEC, int W>
__device__ __forceinline__ void scan_body(const ScanArgs& a, int64_t b, int64_t ch0, int64_t chunk, int w,
                                          const float (&a2)[S], const float (&ia)[S], const float (&av)[S],
                                          float2* __restrict__ s_dx, float* __restrict__ s_gz,
                                          float* __restrict__ s_bc) {
  using TS = TileShape<RR, S, VEC>;
  using TX = typename Act<XB>::T;
  using TD = typename Act<DB>::T;
  constexpr int R = TS::R, CH = TS::CH, NP = TS::NP, T = TS::T, KX = TS::KX, KB = TS::KB;
  constexpr bool FULL = (MODE != kModeState);
  constexpr bool SAVE = (MODE == kModeSave);
  static_assert(!SAVE || T % kSaveTile == 0, "tiles hold whole save intervals");
  constexpr bool ACC = GAIN != kGainShort;   // accurate softplus as well
  // The state-only pass with the short ZOH gain carries a*h instead of h:
  // a*h' = E*(a*h) + (E - 1)*B*x, one instruction per element fewer than
  // h' = E*h + ((E - 1)/a)*B*x; the scale is undone when the state is stored.
  constexpr bool SCALED = !FULL && GAIN == kGainShort;
  static_assert(VEC || W == 1, "the scalar tile path runs one wave per workgroup");
  constexpr int WCH = W * CH;                 // channels per workgroup
  constexpr int XS = TS::template xs<W>();    // LDS row stride of s_dx (and s_gz, in pairs when GZ2)
  constexpr bool GZ2 = TS::GZ2;
  const int tid = threadIdx.x;                // thread in the workgroup
  const int lane = tid % 64;
  const int r = TS::row_of(lane), c = TS::col_of(lane);
  const int wc = w * CH + c;                  // this lane's channel within the workgroup
  const int64_t L = a.seqlen, dim = a.dim, N = a.dstate;
  const int64_t ch = ch0 + c;
  const bool ch_ok = ch < dim;
  const int cl = ch_ok ? c : (int)(dim - 1 - ch0);   // clamped column for loads
  const int64_t t_begin = chunk * a.chunk_len;
  const int64_t t_stop = (t_begin + a.chunk_len < L) ? t_begin + a.chunk_len : L;
  const int64_t slice_elems = a.batch * dim * N;
  const uint32_t dim32 = (uint32_t)dim;
  const uint32_t n32 = (uint32_t)N;

  using RX = typename Raw<XB>::T;
  using RD = typename Raw<DB>::T;
  const RX* __restrict__ gx = (const RX*)a.x;
  const RD* __restrict__ gd = (const RD*)a.delta;
  const RX* __restrict__ gz = (const RX*)a.z;
  const RX* __restrict__ gB = (const RX*)a.B;
  const RX* __restrict__ gC = (const RX*)a.C;
  TX* __restrict__ gy = (TX*)a.y;

  // ---- initial state
  const float* hin = nullptr;
  if (FULL) hin = (a.nchunks > 1) ? a.ws_state + chunk * slice_elems : a.h0;
  else hin = (a.nchunks == 1) ? a.h0 : nullptr;
  float h[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = r * S + s;
    h[s] = (hin != nullptr && ch_ok && n < N) ? hin[(b * dim + ch) * N + n] : 0.f;
    if constexpr (SCALED) h[s] *= av[s];
  }
  const float Dv = (FULL && a.Dskip != nullptr && ch_ok) ? a.Dskip[ch] : 0.f;
  const float bias = (a.delta_bias != nullptr && ch_ok) ? a.delta_bias[ch] : 0.f;
  const bool has_z = FULL && a.z != nullptr;
  const bool dense_bc = (N == NP);

  // Time direction.  Token t (processing order) of the tile starting at t0 is
  // global row grow0(t0) + u(t): u(t) = t forward; reversed, the tile covers
  // rows L - t0 - T .. L - 1 - t0 and u(t) = T - 1 - t, so row offsets stay
  // non-negative.
  const bool rev = a.reverse != 0;
  auto grow0 = [&](int64_t t0) -> int64_t { return rev ? L - t0 - T : t0; };
  auto urow = [&](int t) -> uint32_t { return (uint32_t)(rev ? T - 1 - t : t); };
  const bool tok_delta = a.delta_per_token != 0;

  // ---- register prefetch of one tile.  Row offsets are 32-bit, relative to a
  // wave-uniform 64-bit base, so loads use the scalar-base addressing form.
  RX px[KX], pz[KX], pb[KB], pc[KB];
  RD pd[KX];
  auto fetch_scalar = [&](int64_t t0) {
    const bool tail = t0 + T > t_stop;
    const int64_t row0 = (b * L + grow0(t0)) * dim + ch0;  // uniform
    const RX* xb = gx + row0;
    // delta shared by every channel of a token: one value per (batch, token)
    const RD* db = tok_delta ? gd + (b * L + grow0(t0)) : gd + row0;
    const RX* zb = gz + row0;
    const int64_t last = t_stop - 1 - t0;            // last valid local token (uniform)
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      int t = R * k + r;
      if (tail) t = t < last ? t : (int)last;
      const uint32_t off = urow(t) * dim32 + (uint32_t)cl;
      px[k] = xb[off];
      pd[k] = db[tok_delta ? urow(t) : off];
      if (has_z) pz[k] = zb[off];
    }
    const int64_t bc0 = (b * L + grow0(t0)) * N;     // uniform
    const RX* bb = gB + bc0;
    const RX* cb = gC + bc0;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int e = lane + 64 * j;
      int t = e / NP;
      const int n = e % NP;
      if (tail) t = t < last ? t : (int)last;
      // entries with n >= N load a valid element and are zeroed when staged
      const uint32_t off = (dense_bc && !tail && !rev) ? (uint32_t)e
                                                       : urow(t) * n32 + ((uint32_t)n < n32 ? (uint32_t)n : 0u);
      pb[j] = bb[off];
      if (FULL) pc[j] = cb[off];
    }
  };
  // ---- registers -> LDS: dt (softplus), x, silu(z); B and C as fp32
  auto stage_scalar = [&](int64_t t0) {
    const int64_t nvalid = t_stop - t0;             // uniform
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      const int t = R * k + r;
      const float v = Raw<DB>::f32(pd[k]) + bias;
      float dt = a.softplus ? (ACC ? softplus_f(v) : softplus_short(v)) : v;
      dt = (t < nvalid) ? dt : 0.f;
      const float xv = Raw<XB>::f32(px[k]);
      s_dx[t * XS + wc] = make_float2(dt, xv);
      if (FULL) {
        const float gv = has_z ? silu_f(Raw<XB>::f32(pz[k])) : 1.f;
        if constexpr (GZ2) reinterpret_cast<float2*>(s_gz)[t * XS + wc] = make_float2(Dv * xv, gv);
        else s_gz[t * XS + wc] = gv;
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int e = lane + 64 * j;
      const int t = e / NP, n = e % NP;
      const int base = ((t * R + n / S) * 2) * S + (n % S);
      const bool ok = (uint32_t)n < n32;
      s_bc[base] = ok ? Raw<XB>::f32(pb[j]) : 0.f;
      if (FULL) s_bc[base + S] = ok ? Raw<XB>::f32(pc[j]) : 0.f;
    }
  };


  // ---- vectorised tile I/O (every channel group full, pointers 16-byte
  // aligned, N == NP, delta stored like x).  The W waves of the workgroup
  // cover W*CH consecutive channels and load the tiles together: thread tid
  // moves whole chunks of VX bytes.  Chunk k of the x (delta, z) tile covers
  // token k / XROW, workgroup channels (k % XROW) * EX .. + EX, so each token
  // row of the workgroup is read as one contiguous run; B and C, shared by
  // every channel, are loaded once per workgroup in chunks of VBC bytes of the
  // (token, state)-contiguous tile.
  constexpr int NT = 64 * W;                                // threads per workgroup
  constexpr int XT = T * WCH * (int)sizeof(RX);             // bytes of one x tile
  constexpr int VX = XT / NT < 16 ? XT / NT : 16;           // bytes per x chunk
  using VTX = typename VecOf<VX / 4>::T;
  constexpr int EX = VX / (int)sizeof(RX);                  // channels per x chunk
  static_assert(!VEC || EX % 2 == 0, "x chunks hold whole (dt, x) float4 pairs");
  constexpr int XROW = WCH / EX;                            // chunks per token row
  constexpr int CXN = XT / (NT * VX);                       // x chunks per thread
  constexpr int BT = T * NP * (int)sizeof(RX);              // bytes of one B tile
  // bytes per B chunk: 8 when that gives every thread one, else 16 (with only
  // the first BT / 16 threads loading when the tile is smaller than that)
  constexpr int VBC = BT / NT == 8 ? 8 : 16;
  using VTB = typename VecOf<VBC / 4>::T;
  constexpr int EB = VBC / (int)sizeof(RX);                 // elements per B chunk
  constexpr int CBN = BT >= NT * VBC ? BT / (NT * VBC) : 1;  // B chunks per thread
  constexpr bool BPART = BT < NT * VBC;                     // some threads hold no B chunk
  constexpr int GW = S < EB ? S : EB;                       // floats per LDS write of B/C
  // delta moves in chunks of the same EX channels in its own dtype: VD bytes, as DV loads of at most 16
  // bytes (fp32 delta beside bf16 x can need two); one delta per token instead is loaded as a single
  // value per chunk and kept, already converted to fp32, in the chunk's first word
  constexpr int VD = EX * (int)sizeof(RD);
  constexpr int DV = VD > 16 ? VD / 16 : 1;
  using VTD = typename VecOf<VD / DV / 4>::T;
  constexpr int EPD = EX / DV;                              // delta elements per load
  VTX vx[CXN], vz[CXN];
  VTD vd[CXN][DV];
  VTB vb[CBN], vc[CBN];
  const int vc0 = (tid % XROW) * EX;                        // this thread's first workgroup channel
  const int64_t chw0 = ch0 - (int64_t)w * CH;               // first channel of the workgroup
  float vbias[EX], vDs[EX];
#pragma unroll
  for (int e = 0; e < EX; ++e) {
    vbias[e] = (VEC && a.delta_bias != nullptr) ? a.delta_bias[chw0 + vc0 + e] : 0.f;
    vDs[e] = (VEC && GZ2 && FULL && a.Dskip != nullptr) ? a.Dskip[chw0 + vc0 + e] : 0.f;
  }
  // (the element is copied to a scalar first: bit-casting a vector-element
  // lvalue directly reads element 0 with this compiler)
  auto raw_elem = [](const auto& v, int e) -> float {
    if constexpr (sizeof(RX) == 2) {
      const unsigned u = (v[e >> 1] >> (16 * (e & 1))) << 16;
      return __builtin_bit_cast(float, u);
    } else {
      const unsigned u = v[e];
      return __builtin_bit_cast(float, u);
    }
  };
  auto raw_delta = [](const VTD (&v)[DV], int e) -> float {
    const VTD w = v[e / EPD];
    const int k = e % EPD;
    if constexpr (sizeof(RD) == 2) {
      const unsigned u = (w[k >> 1] >> (16 * (k & 1))) << 16;
      return __builtin_bit_cast(float, u);
    } else {
      const unsigned u = w[k];
      return __builtin_bit_cast(float, u);
    }
  };
  auto fetch_vec = [&](int64_t t0) {
    const bool tail = t0 + T > t_stop;
    const int64_t last = t_stop - 1 - t0;
    const int64_t row0 = (b * L + grow0(t0)) * dim + chw0;  // uniform
    const char* xb = (const char*)(gx + row0);
    const char* db = (const char*)(gd + row0);
    const RD* dtok = gd + (b * L + grow0(t0));              // one delta per token
    const char* zb = (const char*)(gz + row0);
    const uint32_t rowb = dim32 * (uint32_t)sizeof(RX);
    const uint32_t rowd = dim32 * (uint32_t)sizeof(RD);
#pragma unroll
    for (int q = 0; q < CXN; ++q) {
      const int k = tid + NT * q;
      int tl = k / XROW;
      if (tail) tl = tl < last ? tl : (int)last;
      const uint32_t off = urow(tl) * rowb + (uint32_t)(k % XROW) * (uint32_t)VX;
      vx[q] = *reinterpret_cast<const VTX*>(xb + off);
      if (tok_delta) {
        vd[q][0][0] = __builtin_bit_cast(unsigned, Raw<DB>::f32(dtok[urow(tl)]));
      } else {
        const uint32_t offd = urow(tl) * rowd + (uint32_t)(k % XROW) * (uint32_t)VD;
#pragma unroll
        for (int i = 0; i < DV; ++i) vd[q][i] = *reinterpret_cast<const VTD*>(db + offd + 16 * i);
      }
      if (has_z) vz[q] = *reinterpret_cast<const VTX*>(zb + off);
    }
    const RX* bb = gB + (b * L + grow0(t0)) * N;            // uniform
    const RX* cb = gC + (b * L + grow0(t0)) * N;
#pragma unroll
    for (int q = 0; q < CBN; ++q) {
      const int e0 = (tid + NT * q) * EB;
      if (BPART && e0 >= T * NP) break;
      int t = e0 / NP;
      if (tail) t = t < last ? t : (int)last;
      const uint32_t off = urow(t) * (uint32_t)NP + (uint32_t)(e0 % NP);
      vb[q] = *reinterpret_cast<const VTB*>(bb + off);
      if (FULL) vc[q] = *reinterpret_cast<const VTB*>(cb + off);
    }
  };
  // (delta per token, gate, softplus) are uniform over the call: each combination stages through
  // code of its own, without per-item selects between the forms
  auto stage_vec_x = [&](int64_t nvalid, auto tokc, auto gatec, auto spc) {
    constexpr bool TOK = decltype(tokc)::value, GATE = decltype(gatec)::value, SP = decltype(spc)::value;
#pragma unroll
    for (int q = 0; q < CXN; ++q) {
      const int k = tid + NT * q;
      const int tl = k / XROW;
      float dxv[2 * EX];
      const unsigned dtok_bits = vd[q][0][0];
#pragma unroll
      for (int e = 0; e < EX; ++e) {
        const float v = (TOK ? __builtin_bit_cast(float, dtok_bits) : raw_delta(vd[q], e)) + vbias[e];
        dxv[2 * e] = SP ? (ACC ? softplus_f(v) : softplus_short(v)) : v;
        dxv[2 * e + 1] = raw_elem(vx[q], e);
      }
      float4* dst = reinterpret_cast<float4*>(s_dx + tl * XS + vc0);
#pragma unroll
      for (int e = 0; e < EX / 2; ++e) dst[e] = make_float4(dxv[4 * e], dxv[4 * e + 1], dxv[4 * e + 2], dxv[4 * e + 3]);
      // tokens past the end of the slice: dt = 0 (the same thread overwrites what it just wrote)
      if (nvalid < T && tl >= nvalid) {
#pragma unroll
        for (int e = 0; e < EX; ++e) s_dx[tl * XS + vc0 + e].x = 0.f;
      }
      if (FULL) {
        float gzv[EX];
#pragma unroll
        for (int e = 0; e < EX; ++e) gzv[e] = GATE ? silu_f(raw_elem(vz[q], e)) : 1.f;
        if constexpr (GZ2) {
          // (D x, silu z) pairs
          float4* gd4 = reinterpret_cast<float4*>(s_gz + 2 * (tl * XS + vc0));
#pragma unroll
          for (int e = 0; e < EX / 2; ++e)
            gd4[e] = make_float4(vDs[2 * e] * dxv[4 * e + 1], gzv[2 * e], vDs[2 * e + 1] * dxv[4 * e + 3], gzv[2 * e + 1]);
        } else if constexpr (EX % 4 == 0) {
          float4* gd4 = reinterpret_cast<float4*>(s_gz + tl * XS + vc0);
#pragma unroll
          for (int e = 0; e < EX / 4; ++e)
            gd4[e] = make_float4(gzv[4 * e], gzv[4 * e + 1], gzv[4 * e + 2], gzv[4 * e + 3]);
        } else {
          // two channels per chunk (fp32, 8 rows of 32 states): 8-byte writes
          float2* gd2 = reinterpret_cast<float2*>(s_gz + tl * XS + vc0);
#pragma unroll
          for (int e = 0; e < EX / 2; ++e) gd2[e] = make_float2(gzv[2 * e], gzv[2 * e + 1]);
        }
      }
    }
  };
  auto stage_vec = [&](int64_t t0) {
    const int64_t nvalid = t_stop - t0;
    const std::true_type Y;
    const std::false_type N;
    if (tok_delta) {
      if (has_z) {
        if (a.softplus) stage_vec_x(nvalid, Y, Y, Y);
        else stage_vec_x(nvalid, Y, Y, N);
      } else {
        if (a.softplus) stage_vec_x(nvalid, Y, N, Y);
        else stage_vec_x(nvalid, Y, N, N);
      }
    } else {
      if (has_z) {
        if (a.softplus) stage_vec_x(nvalid, N, Y, Y);
        else stage_vec_x(nvalid, N, Y, N);
      } else {
        if (a.softplus) stage_vec_x(nvalid, N, N, Y);
        else stage_vec_x(nvalid, N, N, N);
      }
    }
#pragma unroll
    for (int q = 0; q < CBN; ++q) {
      const int e0 = (tid + NT * q) * EB;
      if (BPART && e0 >= T * NP) break;
      const int t = e0 / NP, n0 = e0 % NP;
#pragma unroll
      for (int g = 0; g < EB / GW; ++g) {
        const int n = n0 + g * GW;
        const int base = ((t * R + n / S) * 2) * S + (n % S);
#pragma unroll
        for (int e = 0; e < GW; ++e) {
          s_bc[base + e] = raw_elem(vb[q], g * GW + e);
          if (FULL) s_bc[base + S + e] = raw_elem(vc[q], g * GW + e);
        }
      }
    }
  };
  auto fetch = [&](int64_t t0) {
    if constexpr (VEC) fetch_vec(t0);
    else fetch_scalar(t0);
  };
  auto stage = [&](int64_t t0) {
    if constexpr (VEC) stage_vec(t0);
    else stage_scalar(t0);
  };

  float dsum = 0.f;
  // kModeSave: the state entering token t (processing order, a multiple of 16) -> save_states[t / 16]
  auto save_state = [&](int64_t t) {
    if (!ch_ok || t >= L) return;
    float* o = a.save_states + ((t / kSaveTile) * a.batch + b) * dim * N + ch * N + r * S;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (r * S + s < N) o[s] = h[s];
  };
  fetch(t_begin);
  for (int64_t t0 = t_begin; t0 < t_stop; t0 += T) {
    lds_sync();
    stage(t0);
    if (t0 + T < t_stop) fetch(t0 + T);   // the staged registers are free again: next tile's loads before the barrier
    lds_sync();
    const int64_t nvalid = t_stop - t0;
    TX* yb = gy + (b * L + grow0(t0)) * dim + ch0;   // uniform
    const bool full_tile = ch_ok && nvalid >= T;       // uniform on the vector path
    const int nval32 = nvalid < T ? (int)nvalid : T;
    // Readout of the group of R tokens starting at tg: row r gets token tg + r.
    auto emit = [&](int tg, const float (&pr)[R]) {
      float tot;
      if constexpr (R == 16 && S == 1) tot = reduce_scatter_quad16(pr);
      else tot = reduce_scatter_rows<R>(pr);
      const int tl = tg + r;
      const float xv = s_dx[tl * XS + wc].y;
      const float yv = fmaf(Dv, xv, tot) * s_gz[tl * XS + wc];
      if (full_tile || (ch_ok && tl < nval32)) yb[urow(tl) * dim32 + (uint32_t)c] = (TX)yv;
    };
    if constexpr (R == 16 && S == 1) {
      // 16 rows of one state, quads of lanes on one channel.  Per step of U = 4 tokens a lane
      // reads the (dt, x) pair of one of them, token tb + lane % 4; the multiplies that use a
      // token's dt and x take it from that quad lane by a DPP broadcast folded into the
      // instruction, so the (dt, x) tile is read once per quad rather than once per lane.
      // Each lane reads its row's (B, C) pair per token.  Every 16 tokens end with the
      // reduce-scatter over the rows; the y values wait in registers for the tile's end.
      constexpr int U = 4;
      const int q4 = lane & 3;
      struct Step16 {
        float2 dx;
        float2 bc[U];
      };
      auto load16 = [&](int tb, Step16& g) {
        g.dx = s_dx[(tb + q4) * XS + wc];
#pragma unroll
        for (int j = 0; j < U; ++j) g.bc[j] = *reinterpret_cast<const float2*>(s_bc + ((tb + j) * R + r) * 2);
      };
      // exp(dt*a) one step ahead, as in the general path below
      auto exp16 = [&](const Step16& g, float (&E)[U]) {
        static_for<U>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          E[j] = hw_exp2(quad_bcast<j>(g.dx.x) * a2[0]);
        });
      };
      Step16 cur, nxt;
      float Ecur[U], Enxt[U];
      load16(0, cur);
      exp16(cur, Ecur);
      // readout products of the 16 tokens of a group, two groups' worth: on the vector path a group's
      // reduce-scatter runs after the first step of the next group, so that its exchange chain
      // overlaps that step's independent work
      constexpr bool DEFER_RS = VEC;
      float pr2[DEFER_RS ? 2 : 1][16];
      float yq[T / 16];   // y of token 16 g + r
      auto readout16 = [&](int gq) {
        const int tl = 16 * gq + r;
        const float2 e = reinterpret_cast<const float2*>(s_gz)[tl * XS + wc];   // (D x, silu z)
        yq[gq] = (reduce_scatter_quad16(pr2[DEFER_RS ? (gq & 1) : 0]) + e.x) * e.y;
        // the one-wave tile path stores at once: its prefetch registers leave no room for four
        // held y values
        if constexpr (!VEC) {
          if (ch_ok && tl < nval32) yb[urow(tl) * dim32 + (uint32_t)c] = (TX)yq[gq];
        }
      };
      constexpr int kStepUnroll = T / U;
#pragma unroll kStepUnroll
      for (int tb = 0; tb < T; tb += U) {
        if (tb + U < T) {
          load16(tb + U, nxt);
          exp16(nxt, Enxt);
        }
        // keep the next step's LDS reads and exponentials ahead of this step's work (the compiler
        // otherwise moves reads next to their use; 2.8B-like layer 0.495 -> 0.488 ms)
        __builtin_amdgcn_sched_barrier(0);
        if (SAVE && tb % kSaveTile == 0) save_state(t0 + tb);
        static_for<U>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          const float E = Ecur[j];
          const float u = quad_bcast<j>(cur.dx.y) * cur.bc[j].x;   // B x
          if constexpr (SCALED) {
            h[0] = fmaf(E, h[0], fmaf(E, u, -u));
          } else {
            float g;
            if constexpr (GAIN == kGainShort) {
              g = fmaf(E, ia[0], -ia[0]);
            } else {
              const float dt = quad_bcast<j>(cur.dx.x);
              g = GAIN == kGainEuler ? dt : zoh_gain_accurate(E, dt, av[0], ia[0]);
            }
            h[0] = fmaf(E, h[0], g * u);
          }
          if (FULL) pr2[DEFER_RS ? ((tb / 16) & 1) : 0][(tb + j) % 16] = cur.bc[j].y * h[0];
        });
        if (!FULL) dsum += cur.dx.x;   // this lane's token of the step (the quad adds up at the end)
        if (FULL) {
          if (DEFER_RS) {
            if (tb % 16 == 0 && tb >= 16) readout16(tb / 16 - 1);
          } else if ((tb + U) % 16 == 0) {
            readout16(tb / 16);
          }
        }
        if (tb + U < T) {
          cur = nxt;
#pragma unroll
          for (int j = 0; j < U; ++j) Ecur[j] = Enxt[j];
        }
      }
      if (FULL && DEFER_RS) readout16(T / 16 - 1);
      // the tile's stores after its loop, which then has no branches (vector path)
      if (FULL && VEC) {
        if (full_tile) {
#pragma unroll
          for (int g = 0; g < T / 16; ++g) yb[urow(16 * g + r) * dim32 + (uint32_t)c] = (TX)yq[g];
        } else {
#pragma unroll
          for (int g = 0; g < T / 16; ++g)
            if (ch_ok && 16 * g + r < nval32) yb[urow(16 * g + r) * dim32 + (uint32_t)c] = (TX)yq[g];
        }
      }
    } else if constexpr (S < 16) {
    // Operands of one step of U = 4 tokens: (dt, x) and this row's B/C
    // slices.  The next step's operands are read from LDS while the current
    // step is computed, so LDS latency overlaps the VALU work; a group of R
    // tokens (R / U steps) ends with the row reduce-scatter and the stores.
    constexpr int U = 4;
    struct Step {
      float2 dx[U];
      float b[U][S];
      float c[U][S];
    };
    auto load_step = [&](int tb, Step& g) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int tt = tb + j;
        g.dx[j] = s_dx[tt * XS + wc];
        const float* bc = s_bc + ((tt * R + r) * 2) * S;
        if constexpr (S >= 4) {
#pragma unroll
          for (int q = 0; q < S / 4; ++q) {
            const float4 vb = reinterpret_cast<const float4*>(bc)[q];
            g.b[j][4 * q] = vb.x; g.b[j][4 * q + 1] = vb.y; g.b[j][4 * q + 2] = vb.z; g.b[j][4 * q + 3] = vb.w;
            if (FULL) {
              const float4 vc = reinterpret_cast<const float4*>(bc + S)[q];
              g.c[j][4 * q] = vc.x; g.c[j][4 * q + 1] = vc.y; g.c[j][4 * q + 2] = vc.z; g.c[j][4 * q + 3] = vc.w;
            }
          }
        } else {
#pragma unroll
          for (int s = 0; s < S; ++s) { g.b[j][s] = bc[s]; g.c[j][s] = FULL ? bc[S + s] : 0.f; }
        }
      }
    };
    Step cur, nxt;
    load_step(0, cur);
    // exp(dt*a) of a step is computed one step ahead, so the transcendental
    // latency overlaps the previous step's state updates
    float Ecur[U][S], Enxt[U][S];
    auto step_exp = [&](const Step& g, float (&E)[U][S]) {
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int s = 0; s < S; ++s) E[j][s] = hw_exp2(g.dx[j].x * a2[s]);
    };
    step_exp(cur, Ecur);
    float pr[R];
    constexpr int kStepUnroll = T / U;   // full unroll: static register indices
#pragma unroll kStepUnroll
    for (int tb = 0; tb < T; tb += U) {
      if (tb + U < T) {
        load_step(tb + U, nxt);
        step_exp(nxt, Enxt);
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (SAVE && ((tb + j) % kSaveTile) == 0) save_state(t0 + tb + j);
        const float2 dx = cur.dx[j];
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const float E = Ecur[j][s];
          if constexpr (SCALED) {
            const float u = cur.b[j][s] * dx.y;
            h[s] = fmaf(E, h[s], fmaf(E, u, -u));
          } else {
            const float g = GAIN == kGainEuler      ? dx.x
                            : GAIN == kGainAccurate ? zoh_gain_accurate(E, dx.x, av[s], ia[s])
                                                    : fmaf(E, ia[s], -ia[s]);
            h[s] = fmaf(E, h[s], g * (cur.b[j][s] * dx.y));
          }
          if (FULL) acc = fmaf(cur.c[j][s], h[s], acc);
        }
        pr[R == U ? j : (tb + j) % R] = acc;   // static index: R == U, or the loop is fully unrolled
        if (!FULL) dsum += dx.x;
      }
      if (FULL && (R == U || (tb + U) % R == 0)) emit(tb + U - R, pr);
      if (tb + U < T) {
        cur = nxt;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
          for (int s = 0; s < S; ++s) Ecur[j][s] = Enxt[j][s];
      }
    }
    } else {
      // Wide lanes (16 or 32 states, 4 rows): one token at a time, operands
      // read and exponentials taken as they are used.  The S independent
      // state chains of a token cover the exp and LDS latencies; staging a
      // step ahead would hold 8S registers per lane and spill.
      static_assert(R == 4 || R == 8, "wide lanes use the 4- or 8-row layout");
#pragma unroll 1
      for (int tb = 0; tb < T; tb += R) {
        float pr[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int tt = tb + j;
          if (SAVE && (tt % kSaveTile) == 0) save_state(t0 + tt);
          const float2 dx = s_dx[tt * XS + wc];
          const float4* bc4 = reinterpret_cast<const float4*>(s_bc + ((tt * R + r) * 2) * S);
          float acc = 0.f;
#pragma unroll
          for (int q = 0; q < S / 4; ++q) {
            const float4 vb = bc4[q];
            const float4 vc = FULL ? bc4[S / 4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float bq[4] = {vb.x, vb.y, vb.z, vb.w};
            const float cq[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int st = 4 * q + e;
              const float E = hw_exp2(dx.x * a2[st]);
              if constexpr (SCALED) {
                const float u = bq[e] * dx.y;
                h[st] = fmaf(E, h[st], fmaf(E, u, -u));
              } else {
                const float g = GAIN == kGainEuler      ? dx.x
                                : GAIN == kGainAccurate ? zoh_gain_accurate(E, dx.x, av[st], ia[st])
                                                        : fmaf(E, ia[st], -ia[st]);
                h[st] = fmaf(E, h[st], g * (bq[e] * dx.y));
              }
              if (FULL) acc = fmaf(cq[e], h[st], acc);
            }
          }
          pr[j] = acc;
          if (!FULL) dsum += dx.x;
        }
        if (FULL) emit(tb, pr);
      }
    }
  }

  // ---- end state
  if constexpr (SCALED) {
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] *= ia[s];
  }
  float* hout = nullptr;
  if (FULL) hout = (chunk == a.nchunks - 1) ? a.h_final : nullptr;
  else hout = (a.nchunks == 1) ? a.h_final : a.ws_state + chunk * slice_elems;
  if (hout != nullptr && ch_ok) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t n = r * S + s;
      if (n < N) hout[(b * dim + ch) * N + n] = h[s];
    }
  }
  if constexpr (!FULL && R == 16 && S == 1) {
    // each lane summed the dt of the tokens it read (one in four): add up the quad
    dsum += bits_f((unsigned)__builtin_amdgcn_mov_dpp((int)f_bits(dsum), 0xB1, 0xf, 0xf, true));
    dsum += bits_f((unsigned)__builtin_amdgcn_mov_dpp((int)f_bits(dsum), 0x4E, 0xf, 0xf, true));
  }
  if (!FULL && a.nchunks > 1 && r == 0 && ch_ok) a.ws_dsum[chunk * a.batch * dim + b * dim + ch] = dsum;
}

// Waves per SIMD the register budget is sized for: the 4-row layout and wide
// lanes run one wave per SIMD on their target shapes, the 8- and 16-row
// layouts two and three.
template <int RR, int S>
constexpr int scan_waves_per_simd() {
  return (RR == 4 || S >= 16) ? 1 : RR == 8 ? 2 : 3;
}

// W waves per workgroup (1, or 4 on the vector path): the waves of a
// workgroup scan W consecutive channel groups of one batch row and share the
// staged tiles.
template <int RR, bool XB, bool DB, int S, int MODE, bool VEC, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(scan_waves_per_simd<RR, S>())))
void scan_kernel(ScanArgs a, int64_t groups_per_batch) {
  using TS = TileShape<RR, S, VEC>;
  constexpr int XS = TS::template xs<W>();
  __shared__ __attribute__((aligned(16))) float2 s_dx[TS::T * XS];
  __shared__ __attribute__((aligned(16))) float s_gz[TS::template gz_floats<W>()];
  __shared__ __attribute__((aligned(16))) float s_bc[TS::T * TS::R * 2 * S];

  // XCD-aware order: dispatch id i runs on XCD i % 8; give each XCD a contiguous
  // range of (batch, channel-group) tiles so neighbouring channel groups share L2.
  const int64_t nb = gridDim.x;
  int64_t lin = blockIdx.x;
  if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
  const int64_t wgs_per_batch = groups_per_batch / W;     // the host launches whole workgroups
  const int w = (int)(threadIdx.x / 64);
  const int64_t b = lin / wgs_per_batch;
  const int64_t ch0 = ((lin % wgs_per_batch) * W + w) * TS::CH;
  const int64_t chunk = blockIdx.y;

  const int lane = threadIdx.x % 64;
  const int r = TS::row_of(lane), c = TS::col_of(lane);
  const int64_t ch = ch0 + c;
  float a2[S], ia[S], av[S];
  bool tiny = false;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = r * S + s;
    const float an = (ch < a.dim && n < a.dstate) ? a.A[ch * a.dstate + n] : -1.f;
    av[s] = an;
    a2[s] = an * kLog2e;
    ia[s] = 1.f / an;
    tiny = tiny || !(fabsf(an) >= 1e-2f);
  }
  // the gain form is chosen once for the whole workgroup (its waves pass the
  // same barriers)
  const bool any_tiny = W == 1 ? __builtin_amdgcn_ballot_w64(tiny) != 0 : __syncthreads_or(tiny) != 0;
  if (a.euler)
    scan_body<RR, XB, DB, S, MODE, kGainEuler, VEC, W>(a, b, ch0, chunk, w, a2, ia, av, s_dx, s_gz, s_bc);
  else if (!XB || any_tiny)
    scan_body<RR, XB, DB, S, MODE, kGainAccurate, VEC, W>(a, b, ch0, chunk, w, a2, ia, av, s_dx, s_gz, s_bc);
  else
    scan_body<RR, XB, DB, S, MODE, kGainShort, VEC, W>(a, b, ch0, chunk, w, a2, ia, av, s_dx, s_gz, s_bc);
}

// The vectorised tile path needs whole chunks of the x and B/C tiles per thread.
template <int RR, bool XB, int S, int W>
constexpr bool vec_shape_ok() {
  using TS = TileShape<RR, S>;
  constexpr int sz = XB ? 2 : 4;
  constexpr int NT = 64 * W;
  constexpr int XT = TS::T * TS::CH * W * sz;
  constexpr int VX = XT / NT < 16 ? XT / NT : 16;
  constexpr int BT = TS::T * TS::NP * sz;
  return (VX == 8 || VX == 16) && XT % (NT * VX) == 0 && BT % 16 == 0 && (TS::CH * W) % (VX / sz) == 0;
}
template <int RR, bool XB, int S, int W>
bool vec_ok(const ScanArgs& a) {
  return vec_shape_ok<RR, XB, S, W>() && a.dstate == TileShape<RR, S>::NP && a.dim % (TileShape<RR, S>::CH * W) == 0;
}

// Launch the scan kernel for one (rows, act dtype, delta dtype, states-per-lane)
// combination.  `grid.x` counts channel groups; the vector path runs four of
// them per workgroup when the channels split into whole workgroups.
template <int RR, bool XB, bool DB, int SV>
hipError_t launch_scan_variant(int mode, const ScanArgs& a, dim3 grid, int64_t gpb, hipStream_t st) {
  constexpr int WV = 4;
  if constexpr (vec_shape_ok<RR, XB, SV, WV>()) {
    if (a.vec_io && vec_ok<RR, XB, SV, WV>(a) && gpb % WV == 0) {
      const dim3 g4(grid.x / WV, grid.y);
      if (mode == kModeFull) scan_kernel<RR, XB, DB, SV, kModeFull, true, WV><<<g4, 64 * WV, 0, st>>>(a, gpb);
      else if (mode == kModeSave) scan_kernel<RR, XB, DB, SV, kModeSave, true, WV><<<g4, 64 * WV, 0, st>>>(a, gpb);
      else scan_kernel<RR, XB, DB, SV, kModeState, true, WV><<<g4, 64 * WV, 0, st>>>(a, gpb);
      return hipGetLastError();
    }
  }
  if constexpr (vec_shape_ok<RR, XB, SV, 1>()) {
    if (a.vec_io && vec_ok<RR, XB, SV, 1>(a)) {
      if (mode == kModeFull) scan_kernel<RR, XB, DB, SV, kModeFull, true, 1><<<grid, 64, 0, st>>>(a, gpb);
      else if (mode == kModeSave) scan_kernel<RR, XB, DB, SV, kModeSave, true, 1><<<grid, 64, 0, st>>>(a, gpb);
      else scan_kernel<RR, XB, DB, SV, kModeState, true, 1><<<grid, 64, 0, st>>>(a, gpb);
      return hipGetLastError();
    }
  }
  if (mode == kModeFull) scan_kernel<RR, XB, DB, SV, kModeFull, false, 1><<<grid, 64, 0, st>>>(a, gpb);
  else if (mode == kModeSave) scan_kernel<RR, XB, DB, SV, kModeSave, false, 1><<<grid, 64, 0, st>>>(a, gpb);
  else scan_kernel<RR, XB, DB, SV, kModeState, false, 1><<<grid, 64, 0, st>>>(a, gpb);
  return hipGetLastError();
}

}  // namespace scan_dev
}  // namespace ssm
