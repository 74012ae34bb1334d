// Selective scan for long sequences on few (batch, channel) slices, in one
// pass: the lanes of a wave split the time axis.
//
// Same recurrence as scan_impl.h ("SSM & Mamba", Discretization/ZOH;
// "Mamba / SSM complete guide", sec. 5):
//   h_t = exp(dt_t a) h_{t-1} + (exp(dt_t a) - 1)/a * B_t x_t,  y_t = C_t . h_t + Dskip x_t (* silu(z_t)).
//
// A layer with few slices (the 131072-token layer has 2048 channels x 16
// states) cannot fill the chip if each lane walks its state through the whole
// sequence.  Here a wave owns ONE channel and a time tile of 256 tokens: lane
// (row r = lane / 16, group g = lane % 16) holds states 4r..4r+3 for tokens
// 16g .. 16g+15 of the tile.  Per tile:
//   1. every lane runs its 16 tokens from a zero state, keeping each token's
//      decay E = exp(dt a) and input term U = gain * B x in registers, and the
//      group's aggregate (P = prod E = exp(a * sum dt), h_loc);
//   2. an inclusive scan over the 16 groups of a row combines the aggregates
//      with the associative operator (P2, h2) o (P1, h1) = (P2 P1, P2 h1 + h2)
//      ("Paper explainer: Mamba", hardware-aware parallel scan; "Mamba / SSM
//      complete guide", sec. 5, with the corrected combine), by DPP row shifts
//      of 1, 2, 4 and 8 lanes; the tile's carried-in state then gives every
//      group its true starting state;
//   3. every lane replays its 16 tokens from that state (one fma per element
//      with the stored E and U) and forms the readout, which is summed over
//      the 4 rows by a reduce-scatter; row_newbcast hands the replayed state
//      of group 15, the tile's end state, to the whole row for the next tile.
// Per (t, d, n) element this costs one fma more than the serial scan, instead
// of the second pass over the sequence that a split into independently
// computed time chunks needs.  A workgroup holds 8 waves = 8 consecutive
// channels of one batch row (16-byte rows of bf16 x, delta and y) and stages
// their tiles, and the 16-state B/C tiles shared by all of them, in LDS.
#include <hip/hip_runtime.h>

#include <string>

#include "device_common.h"
#include "scan_impl.h"

namespace ssm {
namespace scan_long {

using namespace scan_dev;

constexpr int W = 8;          // waves (channels) per workgroup
constexpr int NT = 64 * W;    // threads per workgroup
constexpr int G = 16;         // time groups per wave (lane bits 0-3)
constexpr int TAU = 16;       // tokens per group
constexpr int T = G * TAU;    // tokens per tile
constexpr int NS = 16;        // states (4 rows x 4 per lane)

// LDS layouts, padded so that both access patterns of each array touch
// distinct banks (32 banks of 4 bytes): the staging threads write rows t,
// t+1, ... from consecutive lanes, and the compute reads one row per time
// group, t = 16 g + j, from the 16 lanes of a row.
// (dt, x) and silu(z) of (token t, channel w): rows of W + 1 slots plus one
// slot per 16 rows.  As 8-byte words: 18 t + 2 (t >> 4) + 2 w, so consecutive
// rows land 18 words apart (16 distinct bank pairs) and the 16 groups 2 words
// apart.
__device__ __forceinline__ int ix_dx(int t, int w) { return t * (W + 1) + (t >> 4) + w; }
// B and C of token t = 16 g + j, states 4 r .. 4 r + 3: 16-byte slot
// (4 j + r) * 16 + g.  The compute reads of token j of every group (lane
// (r, g) reads slot (4 j + r) 16 + g) are then one contiguous 1 KB block, and
// the staging threads, which take the tile's tokens in the transposed order
// t = 16 (k mod 16) + k / 16, write 16 consecutive slots per 16 lanes.  (Rows
// of 20 floats, read a token per group, cost twice the LDS cycles.)
__device__ __forceinline__ int ix_b4(int j, int r, int g) { return (j * 4 + r) * 16 + g; }
// y of (token t, channel w), fp32: rows of W + 1 floats plus one per 16 rows,
// so the 64 lanes writing tokens 16 g + 4 jq + r fall at most two to a bank,
// and so do the threads reading back consecutive rows.
__device__ __forceinline__ int ix_y(int t, int w) { return t * (W + 1) + (t >> 4) + w; }
constexpr int DX_SLOTS = T * (W + 1) + T / 16;
constexpr int BC_FLOATS = T * NS;
constexpr int Y_FLOATS = T * (W + 1) + T / 16;
static_assert(W == 8, "the padded layouts are laid out for 8 channels per workgroup");

template <int CTRL, bool ZERO_FILL>
__device__ __forceinline__ float dpp(float old, float v) {
  return bits_f((unsigned)__builtin_amdgcn_update_dpp((int)f_bits(old), (int)f_bits(v), CTRL, 0xf, 0xf, ZERO_FILL));
}
constexpr int kRowShr = 0x110;        // row_shr:k = kRowShr + k
constexpr int kRowBcast15 = 0x15F;    // row_newbcast:15

// One level of the inclusive scan along a 16-lane row: lanes g >= K take in
// the aggregate ending K groups earlier, h <- h + P * h[g - K] and
// P <- P * P[g - K] (the h updates read P before it changes).  The DPP source
// operand reads lane g - K of the row; with bound_ctrl off, lanes g < K have
// no source lane and are not written, so they keep their values.  The s_nop
// gives the two wait states a DPP read needs after a VALU write of its source.
template <int K>
__device__ __forceinline__ void hs_level(float (&h)[4], float (&P)[4]) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8, "row shift");
#define SSM_SHR(K) "row_shr:" #K " row_mask:0xf bank_mask:0xf"
#define SSM_HS_ASM(SH)                                                              \
  asm volatile("s_nop 1\n\t"                                                        \
               "v_fmac_f32_dpp %0, %0, %4 " SH "\n\t"                               \
               "v_fmac_f32_dpp %1, %1, %5 " SH "\n\t"                               \
               "v_fmac_f32_dpp %2, %2, %6 " SH "\n\t"                               \
               "v_fmac_f32_dpp %3, %3, %7 " SH "\n\t"                               \
               "v_mul_f32_dpp %4, %4, %4 " SH "\n\t"                                \
               "v_mul_f32_dpp %5, %5, %5 " SH "\n\t"                                \
               "v_mul_f32_dpp %6, %6, %6 " SH "\n\t"                                \
               "v_mul_f32_dpp %7, %7, %7 " SH                                        \
               : "+v"(h[0]), "+v"(h[1]), "+v"(h[2]), "+v"(h[3]), "+v"(P[0]), "+v"(P[1]), "+v"(P[2]), "+v"(P[3]))
  if constexpr (K == 1) SSM_HS_ASM(SSM_SHR(1));
  else if constexpr (K == 2) SSM_HS_ASM(SSM_SHR(2));
  else if constexpr (K == 4) SSM_HS_ASM(SSM_SHR(4));
  else SSM_HS_ASM(SSM_SHR(8));
#undef SSM_HS_ASM
#undef SSM_SHR
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// NW 32-bit words from global memory as 16-byte (or, for 8 bytes, one 8-byte)
// loads; the address is aligned to the access size.
template <int NW>
__device__ __forceinline__ void load_words(unsigned (&w)[NW], const char* p) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4 v = reinterpret_cast<const u32x4*>(p)[i];
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
  } else {
    static_assert(NW == 2, "rows of 8 or a multiple of 16 bytes");
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    w[0] = v[0]; w[1] = v[1];
  }
}
template <int NW>
__device__ __forceinline__ void store_words(char* p, const unsigned (&w)[NW]) {
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) reinterpret_cast<u32x4*>(p)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
  } else {
    static_assert(NW == 2, "rows of 8 or a multiple of 16 bytes");
    *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
  }
}

template <bool XB, bool DB, bool HASZ, bool SP, int GAIN>
__device__ __forceinline__ void long_body(const ScanArgs& a, int64_t b, int64_t chw0, const float (&a2)[4],
                                          const float (&ia)[4], const float (&av)[4], float2* __restrict__ s_dx,
                                          float* __restrict__ s_gz, float* __restrict__ s_b, float* __restrict__ s_c,
                                          float* __restrict__ s_y) {
  using TX = typename Act<XB>::T;
  using RX = typename Raw<XB>::T;
  using RD = typename Raw<DB>::T;
  constexpr bool ACC = GAIN != kGainShort;
  // the staged rows as 32-bit words: x (z) and delta rows of the W channels, B (C) rows of 16 states
  constexpr int XWD = (int)sizeof(RX) * W / 4;
  constexpr int DWD = (int)sizeof(RD) * W / 4;
  constexpr int BWD = (int)sizeof(RX) * NS / 4;
  const int tid = threadIdx.x;
  const int w = tid / 64, lane = tid % 64;
  const int r = lane / 16, g = lane % 16;
  const int64_t L = a.seqlen, dim = a.dim;
  const int64_t ch = chw0 + w;
  constexpr bool has_z = HASZ;
  const float Dv = a.Dskip != nullptr ? a.Dskip[ch] : 0.f;
  const char* gx = (const char*)a.x;
  const char* gd = (const char*)a.delta;
  const char* gz = (const char*)a.z;
  const char* gB = (const char*)a.B;
  const char* gC = (const char*)a.C;
  const size_t rowx = (size_t)dim * sizeof(RX), rowd = (size_t)dim * sizeof(RD);

  // thread roles in the staging: with 2T threads, threads 0..T-1 move row `tid`
  // of the x, delta (and z) tiles and threads T..2T-1 row `tid - T` of the B
  // and C tiles; with T threads every thread moves row `tid` of all of them
  static_assert(NT == T || NT == 2 * T, "one or two staging roles per tile row");
  const bool xrole = NT == T || tid < T;
  const bool bcrole = NT == T || tid >= T;
  const int trow = tid % T;
  const int brow = 16 * (trow & 15) + (trow >> 4);   // the B/C row this thread stages (see ix_b4)
  float bias[W];
#pragma unroll
  for (int e = 0; e < W; ++e) bias[e] = (xrole && a.delta_bias != nullptr) ? a.delta_bias[chw0 + e] : 0.f;
  unsigned px[XWD], pz[XWD], pd[DWD], pb[BWD], pc[BWD];
  auto fetch = [&](int64_t t0) {
    int64_t row = t0 + trow;
    row = row < L ? row : L - 1;   // the tail loads a valid row; its tokens get dt = 0
    int64_t rowb = t0 + brow;
    rowb = rowb < L ? rowb : L - 1;
    if (xrole) {
      const size_t ox = (size_t)(b * L + row) * rowx + (size_t)chw0 * sizeof(RX);
      const size_t od = (size_t)(b * L + row) * rowd + (size_t)chw0 * sizeof(RD);
      load_words<XWD>(px, gx + ox);
      load_words<DWD>(pd, gd + od);
      if (has_z) load_words<XWD>(pz, gz + ox);
    }
    if (bcrole) {
      const size_t ob = (size_t)(b * L + rowb) * NS * sizeof(RX);
      load_words<BWD>(pb, gB + ob);
      load_words<BWD>(pc, gC + ob);
    }
  };
  // element e of a staged row, widened to fp32
  auto elem = [](const unsigned* v, int e, auto tag) -> float {
    using R = decltype(tag);
    if constexpr (sizeof(R) == 2) {
      return __builtin_bit_cast(float, (v[e >> 1] >> (16 * (e & 1))) << 16);
    } else {
      return __builtin_bit_cast(float, v[e]);
    }
  };
  auto stage = [&](int64_t t0, int buf) {
    const bool ok = t0 + trow < L;
    if (xrole) {
      float2* sdx = s_dx + buf * DX_SLOTS;
      float* sgz = s_gz + (HASZ ? buf * DX_SLOTS : 0);
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const float v = elem(pd, e, RD{}) + bias[e];
        const float dt = SP ? (ACC ? softplus_f(v) : softplus_short(v)) : v;
        sdx[ix_dx(trow, e)] = make_float2(ok ? dt : 0.f, elem(px, e, RX{}));
        if (has_z) sgz[ix_dx(trow, e)] = silu_f(elem(pz, e, RX{}));
      }
    }
    if (bcrole) {
      float4* db = reinterpret_cast<float4*>(s_b + buf * BC_FLOATS);
      float4* dc = reinterpret_cast<float4*>(s_c + buf * BC_FLOATS);
#pragma unroll
      for (int q = 0; q < NS / 4; ++q) {
        const int o = ix_b4(brow & 15, q, brow >> 4);
        db[o] = make_float4(elem(pb, 4 * q, RX{}), elem(pb, 4 * q + 1, RX{}), elem(pb, 4 * q + 2, RX{}),
                            elem(pb, 4 * q + 3, RX{}));
        dc[o] = make_float4(elem(pc, 4 * q, RX{}), elem(pc, 4 * q + 1, RX{}), elem(pc, 4 * q + 2, RX{}),
                            elem(pc, 4 * q + 3, RX{}));
      }
    }
  };
  // y of the previous tile: LDS -> global, one row of the W channels per thread
  auto store_y = [&](int64_t t0, int buf) {
    for (int t = tid; t < T; t += NT) {
      if (t0 + t < L) {
        unsigned v[XWD];
        const float* yr = s_y + buf * Y_FLOATS + ix_y(t, 0);
#pragma unroll
        for (int i = 0; i < XWD; ++i) {
          if constexpr (sizeof(TX) == 2) {
            v[i] = (unsigned)__builtin_bit_cast(unsigned short, (TX)yr[2 * i]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, (TX)yr[2 * i + 1]) << 16);
          } else {
            v[i] = __builtin_bit_cast(unsigned, yr[i]);
          }
        }
        store_words<XWD>((char*)a.y + ((size_t)(b * L + t0 + t) * dim + chw0) * sizeof(TX), v);
      }
    }
  };

  // state entering the current tile, the same in all 16 groups of a row
  float carry[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int n = 4 * r + s;
    carry[s] = (a.h0 != nullptr && n < a.dstate) ? a.h0[(b * dim + ch) * a.dstate + n] : 0.f;
  }
  const int tg = g * TAU;   // this lane's first token within the tile

  // Tiles are double-buffered in LDS, one barrier per tile: while all waves
  // compute tile k from one buffer, the staging threads fill the other with
  // tile k+1 (loaded into registers one tile earlier), issue the loads of tile
  // k+2 and write tile k-1's y out.  The B/C staging waves do their part at
  // the start of the tile and the (dt, x) staging waves theirs, with the y
  // stores, at its end.  Each SIMD holds one wave of each kind, so the two
  // run their latency-bound stretches (the start of the scan, the aggregate
  // scan, the replay's end) out of step, and each covers the other's waits;
  // staging all at the start or all at the end measured 5-7% slower.  The
  // scan's LDS reads are issued two tokens ahead of their use; the scheduling
  // barriers keep the compiler from sinking them back next to their first
  // use, where each read's latency was exposed (bf16 rows; the fp32 variants
  // have no registers to spare for it).
  fetch(0);
  stage(0, 0);
  if (T < L) fetch(T);
  lds_sync();
  int cur = 0;
  for (int64_t t0 = 0; t0 < L; t0 += T, cur ^= 1) {
    const float2* sdx = s_dx + cur * DX_SLOTS;
    const float* sgz = s_gz + (HASZ ? cur * DX_SLOTS : 0);
    const float4* s_b4 = reinterpret_cast<const float4*>(s_b + cur * BC_FLOATS);
    const float4* s_c4 = reinterpret_cast<const float4*>(s_c + cur * BC_FLOATS);
    float* sy = s_y + cur * Y_FLOATS;
    if (!xrole && t0 + T < L) {   // B/C of the next tile into the other buffer, which no wave reads in this tile
      stage(t0 + T, cur ^ 1);
      if (t0 + 2 * T < L) fetch(t0 + 2 * T);
    }

    // 1. the group's tokens from a zero state
    float E[TAU][4], U[TAU][4], h[4];
    float dsum;
    constexpr int KD = XB ? 2 : 0;   // tokens of (dt, x) and B read ahead
    float2 dpre[2];
    float4 bpre[2];
    if (KD > 0) {
      dpre[0] = sdx[ix_dx(tg, w)];
      dpre[1] = sdx[ix_dx(tg + 1, w)];
      bpre[0] = s_b4[ix_b4(0, r, g)];
      bpre[1] = s_b4[ix_b4(1, r, g)];
    }
#pragma unroll
    for (int j = 0; j < TAU; ++j) {
      float2 dx;
      float4 bq;
      if (KD > 0) {
        dx = dpre[j & 1];
        bq = bpre[j & 1];
        if (j + 2 < TAU) {
          dpre[j & 1] = sdx[ix_dx(tg + j + 2, w)];
          bpre[j & 1] = s_b4[ix_b4(j + 2, r, g)];
        }
        if (j & 1) __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of these tokens' work
      } else {
        dx = sdx[ix_dx(tg + j, w)];
        bq = s_b4[ix_b4(j, r, g)];
      }
      const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float e = hw_exp2(dx.x * a2[s]);
        const float gn = GAIN == kGainEuler      ? dx.x
                         : GAIN == kGainAccurate ? zoh_gain_accurate(e, dx.x, av[s], ia[s])
                                                 : fmaf(e, ia[s], -ia[s]);
        const float u = gn * (bv[s] * dx.y);
        h[s] = j == 0 ? u : fmaf(e, h[s], u);   // from a zero state
        E[j][s] = e;
        U[j][s] = u;
      }
      dsum = j == 0 ? dx.x : dsum + dx.x;
    }

    // C of the replay's first two tokens, read ahead of the scan (the replay
    // reads each token's C two tokens ahead of its use)
    constexpr int KC = XB ? 2 : 0;
    float4 cpre[2];
    if (KC > 0) {
      cpre[0] = s_c4[ix_b4(0, r, g)];
      cpre[1] = s_c4[ix_b4(1, r, g)];
    }

    // 2. inclusive scan of the groups' (decay, state) aggregates along the row
    float P[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) P[s] = hw_exp2(a2[s] * dsum);
    hs_level<1>(h, P);
    hs_level<2>(h, P);
    hs_level<4>(h, P);
    hs_level<8>(h, P);
    float hin[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float end_true = fmaf(P[s], carry[s], h[s]);           // state after this lane's group
      hin[s] = dpp<kRowShr + 1, false>(carry[s], end_true);          // group 0 starts from the carry
    }

    // 3. replay from the true starting state; readout summed over the rows
#pragma unroll
    for (int s = 0; s < 4; ++s) h[s] = hin[s];
#pragma unroll
    for (int jq = 0; jq < TAU / 4; ++jq) {
      const int t = tg + 4 * jq + r;   // the token whose y this lane forms
      const float xv = sdx[ix_dx(t, w)].y;
      float pr[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * jq + jj;
        float4 cq;
        if (KC > 0) {
          cq = cpre[jj & 1];
          if (j + 2 < TAU) cpre[jj & 1] = s_c4[ix_b4(j + 2, r, g)];
          if (jj & 1) __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of these tokens' work
        } else {
          cq = s_c4[ix_b4(j, r, g)];
        }
        const float cv[4] = {cq.x, cq.y, cq.z, cq.w};
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          h[s] = fmaf(E[j][s], h[s], U[j][s]);
          acc = fmaf(cv[s], h[s], acc);
        }
        pr[jj] = acc;
      }
      const float tot = reduce_scatter_rows<4>(pr);   // row r: token tg + 4 jq + r
      float yv = fmaf(Dv, xv, tot);
      if (has_z) yv *= sgz[ix_dx(t, w)];
      sy[ix_y(t, w)] = yv;
    }
    // the state after the tile: the replayed state of group 15, in every lane of its row (each lane
    // has a source lane, so no old value is needed; carry, hin and the replayed state then share
    // registers, with no copies between tiles)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      carry[s] = bits_f((unsigned)__builtin_amdgcn_mov_dpp((int)f_bits(h[s]), kRowBcast15, 0xf, 0xf, false));

    if (xrole && t0 + T < L) {   // (dt, x) of the next tile
      stage(t0 + T, cur ^ 1);
      if (t0 + 2 * T < L) fetch(t0 + 2 * T);
    }
    if (t0 > 0) store_y(t0 - T, cur ^ 1);   // the previous tile's y (written before the last barrier)
    lds_sync();
  }
  store_y(((L - 1) / T) * T, cur ^ 1);

  if (a.h_final != nullptr && g == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int n = 4 * r + s;
      if (n < a.dstate) a.h_final[(b * dim + ch) * a.dstate + n] = carry[s];
    }
  }
}

template <bool XB, bool DB, bool HASZ, bool SP>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void scan_long_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) float2 s_dx[2 * DX_SLOTS];
  __shared__ __attribute__((aligned(16))) float s_gz[HASZ ? 2 * DX_SLOTS : 1];
  __shared__ __attribute__((aligned(16))) float s_b[2 * BC_FLOATS];
  __shared__ __attribute__((aligned(16))) float s_c[2 * BC_FLOATS];
  __shared__ __attribute__((aligned(16))) float s_y[2 * Y_FLOATS];

  // XCD-aware order: dispatch id i runs on XCD i % 8; each XCD takes a
  // contiguous range of channel groups, so the 8 workgroups that read one
  // 128-byte line of x, delta and y share that XCD's L2.
  const int64_t nb = gridDim.x;
  int64_t lin = blockIdx.x;
  if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
  const int64_t groups = a.dim / W;
  const int64_t b = lin / groups;
  const int64_t chw0 = (lin % groups) * W;
  const int r = (threadIdx.x % 64) / 16;
  const int64_t ch = chw0 + threadIdx.x / 64;
  float a2[4], ia[4], av[4];
  bool tiny = false;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int n = 4 * r + s;
    const float an = n < a.dstate ? a.A[ch * a.dstate + n] : -1.f;
    av[s] = an;
    a2[s] = an * kLog2e;
    ia[s] = 1.f / an;
    tiny = tiny || !(fabsf(an) >= 1e-2f);
  }
  // one gain form for the whole workgroup (its waves pass the same barriers)
  if (!XB || __syncthreads_or(tiny) != 0)
    long_body<XB, DB, HASZ, SP, kGainAccurate>(a, b, chw0, a2, ia, av, s_dx, s_gz, s_b, s_c, s_y);
  else
    long_body<XB, DB, HASZ, SP, kGainShort>(a, b, chw0, a2, ia, av, s_dx, s_gz, s_b, s_c, s_y);
}

}  // namespace scan_long

bool scan_long_applies(const ScanArgs& a, int num_cus) {
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  // one pass with time-split lanes: 16 states, whole 8-channel groups with
  // 16-byte rows, the plain forward, and enough channel groups to give every
  // CU a workgroup; shorter sequences than two tiles gain nothing
  if (a.dstate != scan_long::NS || a.dim % scan_long::W != 0 || a.seqlen < 2 * scan_long::T) return false;
  if (a.reverse || a.euler || a.delta_per_token || a.save_states != nullptr || !a.vec_io) return false;
  if (((uintptr_t)a.y & 15) != 0) return false;
  return a.batch * (a.dim / scan_long::W) >= cus;
}

int launch_scan_long(const ScanArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t blocks = a.batch * (a.dim / scan_long::W);
  if (blocks > 0x7fffffffLL) return fail(4, "grid too large");
  const dim3 grid((unsigned)blocks);
  using namespace scan_long;
  // one kernel per (act dtype, delta dtype, gate, softplus)
  using K = void (*)(ScanArgs);
  static const K table[16] = {
      scan_long_kernel<false, false, false, false>, scan_long_kernel<false, false, false, true>,
      scan_long_kernel<false, false, true, false>,  scan_long_kernel<false, false, true, true>,
      scan_long_kernel<false, true, false, false>,  scan_long_kernel<false, true, false, true>,
      scan_long_kernel<false, true, true, false>,   scan_long_kernel<false, true, true, true>,
      scan_long_kernel<true, false, false, false>,  scan_long_kernel<true, false, false, true>,
      scan_long_kernel<true, false, true, false>,   scan_long_kernel<true, false, true, true>,
      scan_long_kernel<true, true, false, false>,   scan_long_kernel<true, true, false, true>,
      scan_long_kernel<true, true, true, false>,    scan_long_kernel<true, true, true, true>};
  const int idx = (a.act_bf16 ? 8 : 0) | (a.delta_bf16 ? 4 : 0) | (a.z != nullptr ? 2 : 0) | (a.softplus ? 1 : 0);
  hipLaunchKernelGGL(table[idx], grid, dim3(NT), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(6, std::string("long-sequence scan kernel launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
