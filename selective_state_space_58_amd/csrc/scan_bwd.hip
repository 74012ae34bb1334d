// Backward pass of the selective scan (training): gradients of
//   loss = sum dout * out + sum dh_final * h_final
// with respect to x, delta (through bias and softplus), A, B, C, Dskip, z,
// delta_bias and h0, for the forward map of ssm_scan_fwd ("Mamba / SSM
// complete guide", sec. 5, and "SSM & Mamba", ZOH).  The pages give no
// backward pass; this is the adjoint of the recurrence, step by step:
//   lam_t  = dloss/dh_t = C_t dy_t + exp(dt_{t+1} a) lam_{t+1}
//   dx_t   = sum_n lam_n g_n B_n + Dskip dy_t,  ddt_t = sum_n lam_n (h_{t-1,n} E a + B_n x E)
//   dA_n   = sum_t lam_n (h_{t-1,n} E dt + B_n x dg/da),  dB, dC = sums over channels
// with E = exp(dt a), g = (E - 1)/a, dy = dout * silu(z).
//
// Mapping: the forward's 16-row lane layout (lane = state n x 4 channels, one
// state per lane, 16 states per pass) with four waves per workgroup covering 16
// consecutive channels of one batch row, which share the staged tiles.  A
// forward pass stores the state at the start of every 16-token tile in the
// workspace; the reverse pass then walks the tiles from the last, recomputes
// the tile's states and decays into LDS (with the readout, which the gate's
// gradient needs), and runs the adjoint backwards with lam in registers.
// Per-(token, channel) sums over the states (dx, ddt) use the forward's row
// reduce-scatter.  Per-(token, state) sums over channels (dB, dC) are summed
// over the 4 channels of a wave with DPP and over the 4 waves in LDS, then
// written as one partial per (workgroup, token, state) to the workspace; a
// second kernel adds the partials of the workgroups of a batch row (no
// atomics on the per-token gradients).  dA, Dskip and bias gradients are
// summed in registers and added once per wave.
//
// More than 16 states: given dy, the adjoint of each state is independent of
// the others, and the per-(token, channel) gradients (dx, ddt, dz) are sums
// over the states.  The pass therefore runs once per block of 16 states (in
// stream order), each adding its contribution to fp32 accumulators, and the
// last block writes the outputs; the skip terms enter with the first block.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "scan_impl.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using scan_dev::hw_exp2;
using scan_dev::hw_rcp;
using scan_dev::kLog2e;
using scan_dev::Raw;
using scan_dev::silu_f;
using scan_dev::softplus_f;
using scan_dev::zoh_gain_accurate;

constexpr int BT = 16;    // tokens per tile (states and decays of a tile are kept in LDS)
static_assert(BT == kSaveTile, "saved forward states are one per backward tile");
constexpr int BR = 16;    // lane rows: one state per lane
constexpr int BCH = 4;    // channels per wave
constexpr int BW = 4;     // waves per workgroup
constexpr int BWC = BW * BCH;   // channels per workgroup
constexpr int BG = 4;     // tokens per row reduction (token j of a group ends in rows 4j .. 4j+3)

__device__ __forceinline__ float sigmoid_f(float v) { return hw_rcp(1.f + hw_exp2(-v * kLog2e)); }

// d/da of the ZOH gain (e^{dt a} - 1)/a: (dt E - g)/a, or dt^2 psi(q) with
// psi(q) = sum_{k>=2} (k-1) q^{k-2}/k! for |q| < 1/8 (truncation < 1e-9).  The
// short form alone (bf16 inputs) loses ~2e-7/|q| relative accuracy, far below
// bf16 resolution.
template <bool ACC>
__device__ __forceinline__ float gain_da(float dt, float a, float ia, float E, float g) {
  const float dl = (dt * E - g) * ia;
  if (!ACC) return dl;
  const float q = dt * a;
  const float psi = fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, 1.f / 840.f, 1.f / 144.f), 1.f / 30.f), 1.f / 8.f),
                                 1.f / 3.f), 0.5f);
  return fabsf(q) < 0.125f ? dt * dt * psi : dl;
}

// ZOH gain from E = e^{dt a}: the accurate form (fp32 activations, or any
// |a| < 1e-2 in the workgroup) or the short form (E - 1)/a, as in the forward.
template <bool ACC>
__device__ __forceinline__ float bwd_gain(float E, float dt, float a, float ia) {
  return ACC ? zoh_gain_accurate(E, dt, a, ia) : fmaf(E, ia, -ia);
}

// p[j] holds, in every lane, a partial for token j of a group of 4.  Returns
// in lane (row r, column c) the sum of p[r / 4] over the 16 rows of column c:
// a reduce-scatter over lane bits 5 and 4 (row bits 3 and 2) leaves token r/4
// summed over four rows, and a butterfly over lane bits 3 and 2 adds the rest.
__device__ __forceinline__ float reduce4_rows(const float (&p)[4]) {
  const float u0 = scan_dev::pair_sum<32>(p[0], p[2]);
  const float u1 = scan_dev::pair_sum<32>(p[1], p[3]);
  float v = scan_dev::pair_sum<16>(u0, u1);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x101f));
  return v;
}

// Sum over the 4 lanes of a quad (the 4 channels of a row); every lane gets it.
// The empty asm statements hide where v came from, so the compiler cannot fuse
// the product that feeds v into the first add (an FMA cannot take a DPP
// source), and keep the second add out of a branch that only some lanes take
// (its DPP source must then be a separate move): each level stays one
// v_add_f32 with a DPP source.
__device__ __forceinline__ float quad_sum(float v) {
  asm("" : "+v"(v));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xf, 0xf, true));
  asm("" : "+v"(v));
  return v;
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* p, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dB, dC of states n0 .. n0+width-1 = sums of the per-workgroup partials of
// each batch row (partials laid out (group, batch * token, 16)).
__global__ __launch_bounds__(256) void bwd_sum_partials_kernel(const float* part_b, const float* part_c, float* dB,
                                                               float* dC, int64_t rows, int64_t groups, int64_t N,
                                                               int64_t n0, int width, int64_t L, int reverse) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * width) return;
  const int64_t bt = i / width;                  // (batch, token) in processing order
  const int nl = (int)(i - bt * width);
  const int64_t per_group = rows * BR;
  const int64_t o = bt * BR + nl;
  float sb = 0.f, sc = 0.f;
  // unrolled so that several groups' loads are in flight (52.8 -> 32.4 us on the 96-group headline layer);
  // each partial is read once (streaming hint)
#pragma unroll 8
  for (int64_t g = 0; g < groups; ++g) {
    sb += __builtin_nontemporal_load(part_b + g * per_group + o);
    sc += __builtin_nontemporal_load(part_c + g * per_group + o);
  }
  const int64_t t = bt % L;
  const int64_t row = reverse ? bt - t + (L - 1 - t) : bt;
  dB[row * N + n0 + nl] = sb;
  dC[row * N + n0 + nl] = sc;
}

struct BwdLds {
  float2 dx[BT * BWC];          // (dt, x) per (token, workgroup channel)
  float v[BT * BWC];            // delta + bias (before softplus)
  float dout[BT * BWC];
  float z[BT * BWC];
  float dy[BT * BWC];           // dout * silu(z)
  float bc[BT * BR * 2];        // (B, C) per (token, state)
  float h[BW * BT * 64];        // h_t per (wave, token, lane)
  float red[BW * BT * BR * 2];  // per-wave (dB, dC) partial per (token, state)
};

// MULTI: more than one block of 16 states (per-token gradients accumulated).
// GAIN: 0 short ZOH, 1 accurate ZOH, 2 Euler (gain dt).  REV: reversed scan.
template <bool XB, bool DB, int GAIN, bool MULTI, bool REV>
__device__ __forceinline__ void scan_bwd_body(const BwdArgs& a, int64_t b, int64_t chw0, int64_t grp, float av,
                                              float a2, float ia, bool nok, BwdLds& sm) {
  using RX = typename Raw<XB>::T;
  using RD = typename Raw<DB>::T;
  using TX = typename scan_dev::Act<XB>::T;
  using TD = typename scan_dev::Act<DB>::T;
  constexpr bool ACC = GAIN == 1;
  constexpr bool EULER = GAIN == 2;
  // ZOH gain (E - 1)/a, or dt for the Euler discretization
  auto gain = [&](float E, float dt) -> float { return EULER ? dt : bwd_gain<ACC>(E, dt, av, ia); };
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r = lane >> 2, c = lane & 3;
  const int wc = w * BCH + c;                // channel within the workgroup
  const int64_t L = a.seqlen, dim = a.dim, N = a.dstate;
  const int64_t ch = chw0 + wc;
  const bool ch_ok = ch < dim;
  const int ntile = (int)((L + BT - 1) / BT);
  const int64_t n0 = a.n0;                       // first state of this block of 16
  const int64_t hidx = (b * dim + ch) * N + n0 + r;   // this lane's state (valid when nok)
  const int64_t slice = a.batch * dim * BR;      // one checkpoint of the block's states
  const int64_t cidx = (b * dim + ch) * BR + r;
  const int64_t tcd = a.batch * L * dim;         // token-channel elements of one accumulator
  // processing-order token t sits at row L - 1 - t of the inputs when the scan runs in reverse
  auto grow = [&](int64_t t) -> int64_t { return REV ? L - 1 - t : t; };

  // the skip term and the Dskip gradient belong to the first block of states only
  const float Dv = (a.Dskip != nullptr && ch_ok && a.first) ? a.Dskip[ch] : 0.f;
  const RX* gx = (const RX*)a.x;
  const RD* gd = (const RD*)a.delta;
  const RX* gz = (const RX*)a.z;
  const RX* gdo = (const RX*)a.dout;
  const RX* gB = (const RX*)a.B;
  const RX* gC = (const RX*)a.C;

  // Staging of tile k: per (token, channel) one item per thread, per (token, state) one item per
  // thread.  fetch() loads a tile's items into registers one tile ahead of put_tile(), which converts
  // them and writes them to LDS, so the loads' latency overlaps the previous tile's work.
  const int s_tl = tid / BWC, s_cc = tid % BWC;             // (token, channel) item of this thread
  const int64_t s_chl = chw0 + s_cc < dim ? chw0 + s_cc : dim - 1;
  const float s_bias = a.delta_bias != nullptr ? a.delta_bias[s_chl] : 0.f;
  const int b_tl = tid / BR, b_n = tid % BR;                // (token, state) item of this thread
  RD pre_d;
  RX pre_x, pre_do, pre_z, pre_b, pre_c;
  auto fetch = [&](int k, bool full) {
    const int64_t t0 = (int64_t)k * BT;
    {
      const int64_t t = t0 + s_tl;
      const int64_t row = b * L + grow(t < L ? t : L - 1);
      const int64_t i = row * dim + s_chl;
      pre_d = gd[a.tok_delta ? row : i];
      pre_x = gx[i];
      if (full) {
        pre_do = gdo[i];
        if (a.z != nullptr) pre_z = gz[i];
      }
    }
    {
      const int64_t t = t0 + b_tl;
      const int64_t i = (b * L + grow(t < L ? t : L - 1)) * N + (n0 + b_n < N ? n0 + b_n : 0);
      pre_b = gB[i];
      if (full) pre_c = gC[i];
    }
  };
  auto put_tile = [&](int k, bool full) {
    const int64_t t0 = (int64_t)k * BT;
    {
      const bool ok = t0 + s_tl < L && chw0 + s_cc < dim;
      const float v = Raw<DB>::f32(pre_d) + s_bias;
      const float dt = ok ? (a.softplus ? softplus_f(v) : v) : 0.f;
      sm.dx[tid] = make_float2(dt, Raw<XB>::f32(pre_x));
      if (full) {
        sm.v[tid] = v;
        sm.dout[tid] = ok ? Raw<XB>::f32(pre_do) : 0.f;
        sm.z[tid] = (a.z != nullptr) ? Raw<XB>::f32(pre_z) : 0.f;
      }
    }
    {
      const bool ok = t0 + b_tl < L && n0 + b_n < N;
      sm.bc[(b_tl * BR + b_n) * 2] = ok ? Raw<XB>::f32(pre_b) : 0.f;
      if (full) sm.bc[(b_tl * BR + b_n) * 2 + 1] = ok ? Raw<XB>::f32(pre_c) : 0.f;
    }
  };
  // Per (token, channel) gradient k (0 dx, 1 ddelta, 2 dz) at element i: written
  // directly with one block of states; with several, summed in an fp32
  // accumulator (each element by the same lane in every block, blocks in
  // stream order) and converted after the last block.
  // With one delta per token, ddelta goes per channel to an fp32 buffer that a
  // second kernel sums over the channels.
  auto put = [&](int k, int64_t i, float v, auto* out) {
    using T = typename std::remove_pointer<decltype(out)>::type;
    auto store = [&](float s) {
      if (k == 1 && a.tok_delta) a.ddelta_tc[i] = s;
      else out[i] = (T)s;
    };
    if constexpr (!MULTI) {
      store(v);
      return;
    }
    float* p = a.acc + k * tcd + i;
    const float sum = a.first ? v : *p + v;
    if (a.last) store(sum);
    else *p = sum;
  };

  // ---- forward: the state at the start of every tile into the workspace (unless the forward pass
  // already stored the states at every tile start)
  float h = (a.h0 != nullptr && nok) ? a.h0[hidx] : 0.f;
  const int nck = a.saved != nullptr ? 0 : ntile;
  if (nck > 0) fetch(0, false);
  for (int k = 0; k < nck; ++k) {
    if (nok) a.ws_ckpt[(int64_t)k * slice + cidx] = h;
    lds_sync();
    put_tile(k, false);
    lds_sync();
    if (k + 1 < nck) fetch(k + 1, false);
#pragma unroll 4
    for (int tl = 0; tl < BT; ++tl) {
      const float2 dx = sm.dx[tl * BWC + wc];
      const float Bn = sm.bc[(tl * BR + r) * 2];
      const float E = hw_exp2(dx.x * a2);
      h = fmaf(E, h, gain(E, dx.x) * (Bn * dx.y));
    }
  }

  // ---- reverse
  float lam = (a.dh_final != nullptr && nok) ? a.dh_final[hidx] : 0.f;
  float dA = 0.f, dDacc = 0.f, dbacc = 0.f;
  // short ZOH gain: dg/da = (dt E - g) / a, so the gain part of dA is summed without the 1/a and
  // scaled once at the end
  float dAg = 0.f;
  float* hw = sm.h + w * BT * 64;
  float* rw = sm.red + w * BT * BR * 2;
  const int64_t per_group = a.batch * L * BR;
  if (ntile > 0) fetch(ntile - 1, true);
  // the state entering tile k (stored by the forward or by the pass above), also one tile ahead
  float pre_h = 0.f;
  auto fetch_h = [&](int k) {
    pre_h = !nok ? 0.f
                 : (a.saved != nullptr ? a.saved[((int64_t)k * a.batch + b) * dim * N + ch * N + n0 + r]
                                       : a.ws_ckpt[(int64_t)k * slice + cidx]);
  };
  if (ntile > 0) fetch_h(ntile - 1);
  // Barriers of a reverse tile: one after the staging (its items go to every wave) and one after
  // the adjoint (the dB/dC partials add the four waves' sums).  The recompute's states, dy and
  // readout, and the adjoint's partial sums, are per wave and need none; the barrier after the
  // adjoint also orders the next tile's staging after every wave's reads of this tile.
  lds_sync();
  for (int k = ntile - 1; k >= 0; --k) {
    const int64_t t0 = (int64_t)k * BT;
    put_tile(k, true);
    lds_sync();
    const float hstart = pre_h;
    if (k > 0) {
      fetch(k - 1, true);
      fetch_h(k - 1);
    }
    // recompute the tile's states and decays (into LDS) and its readout; y gives dz and dy
    float hs = hstart;
#pragma unroll
    for (int tb = 0; tb < BT; tb += BG) {
      float pr[BG];
#pragma unroll
      for (int j = 0; j < BG; ++j) {
        const int tl = tb + j;
        const float2 dx = sm.dx[tl * BWC + wc];
        const float Bn = sm.bc[(tl * BR + r) * 2], Cn = sm.bc[(tl * BR + r) * 2 + 1];
        const float E = hw_exp2(dx.x * a2);
        hs = fmaf(E, hs, gain(E, dx.x) * (Bn * dx.y));
        hw[tl * 64 + lane] = hs;
        pr[j] = Cn * hs;
      }
      const float tot = reduce4_rows(pr);   // rows 4j .. 4j+3: readout of token tb + j
      if ((r & 3) == 0) {
        const int tl = tb + (r >> 2);
        const int e = tl * BWC + wc;
        const float y = fmaf(Dv, sm.dx[e].y, tot);
        const float dout = sm.dout[e];
        float dy = dout;
        if (a.z != nullptr) {
          const float zz = sm.z[e];
          const float sg = sigmoid_f(zz);
          dy = dout * zz * sg;
          if (ch_ok && t0 + tl < L)
            put(2, (b * L + grow(t0 + tl)) * dim + ch, dout * y * (sg + zz * sg * (1.f - sg)), (TX*)a.dz);
        }
        sm.dy[e] = dy;
      }
    }
    // adjoint, tokens in reverse, in groups of 4 for the row reductions; the
    // state before token t is the state after token t-1, carried to the next
    // (earlier) token instead of read again
    float hcar = hw[(BT - 1) * 64 + lane];
#pragma unroll 2
    for (int tb = BT - BG; tb >= 0; tb -= BG) {
    float pdx[BG], pdt[BG];
#pragma unroll
    for (int j = BG - 1; j >= 0; --j) {
      const int tl = tb + j;
      const float2 dx = sm.dx[tl * BWC + wc];
      const float dy = sm.dy[tl * BWC + wc];
      const float Bn = sm.bc[(tl * BR + r) * 2], Cn = sm.bc[(tl * BR + r) * 2 + 1];
      const float E = hw_exp2(dx.x * a2);   // recomputed: cheaper than a store and a read of LDS
      const float ht = hcar;
      const float hp = tl > 0 ? hw[(tl - 1) * 64 + lane] : hstart;
      hcar = hp;
      const float g = gain(E, dx.x);
      lam = fmaf(Cn, dy, lam);
      // dC = sum over channels of h_t dy; dB = sum over channels of lam g x
      const float sc = quad_sum(ht * dy);
      const float sb = quad_sum(lam * g * dx.y);
      if (c == 0) {
        rw[(tl * BR + r) * 2] = sb;
        rw[(tl * BR + r) * 2 + 1] = sc;
      }
      const float dE = lam * hp;
      const float dg = lam * Bn * dx.y;
      pdx[j] = lam * g * Bn;
      // dg/ddt is E for ZOH and 1 for Euler; dg/da is zero for Euler
      pdt[j] = fmaf(dE * E, av, EULER ? dg : dg * E);
      if constexpr (EULER) {
        dA = fmaf(dE * E, dx.x, dA);
      } else if constexpr (ACC) {
        dA = fmaf(dE * E, dx.x, fmaf(dg, gain_da<ACC>(dx.x, av, ia, E, g), dA));
      } else {
        dA = fmaf(dE * E, dx.x, dA);
        dAg = fmaf(dg, fmaf(dx.x, E, -g), dAg);
      }
      lam *= E;
    }
    const float tdx = reduce4_rows(pdx);
    const float tdt = reduce4_rows(pdt);
    const int tl = tb + (r >> 2);
    if ((r & 3) == 0 && ch_ok && t0 + tl < L) {
      const int e = tl * BWC + wc;
      const float dy = sm.dy[e];
      const float dv = a.softplus ? tdt * sigmoid_f(sm.v[e]) : tdt;
      const int64_t i = (b * L + grow(t0 + tl)) * dim + ch;
      put(0, i, fmaf(Dv, dy, tdx), (TX*)a.dx);
      put(1, i, dv, (TD*)a.ddelta);
      if (a.first) dDacc = fmaf(dy, sm.dx[e].y, dDacc);
      dbacc += dv;
    }
    }
    lds_sync();
    // dB, dC partial of this workgroup: sum of the 4 waves
    {
      const int tl = tid / BR, n = tid % BR;
      if (t0 + tl < L && n0 + n < N) {
        float sb = 0.f, sc = 0.f;
#pragma unroll
        for (int q = 0; q < BW; ++q) {
          sb += sm.red[((q * BT + tl) * BR + n) * 2];
          sc += sm.red[((q * BT + tl) * BR + n) * 2 + 1];
        }
        const int64_t o = grp * per_group + (b * L + t0 + tl) * BR + n;
        a.ws_part[o] = sb;
        a.ws_part[(int64_t)a.ws_groups * per_group + o] = sc;
      }
    }
  }

  // ---- per-wave sums: dh0, dA per lane; Dskip and bias gradients summed over the 16 rows
  if (nok) {
    if (a.dh0 != nullptr) a.dh0[hidx] = lam;
    atomicAdd(a.dA + ch * N + n0 + r, (EULER || ACC) ? dA : fmaf(dAg, ia, dA));   // (1/a is infinite at a = 0)
  }
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
    dDacc += __shfl_xor(dDacc, o);
    dbacc += __shfl_xor(dbacc, o);
  }
  if (ch_ok && r == 0) {
    if (a.dDskip != nullptr) atomicAdd(a.dDskip + ch, dDacc);
    if (a.ddelta_bias != nullptr) atomicAdd(a.ddelta_bias + ch, dbacc);
  }
}

// One workgroup of four waves per 16 channels of a batch row.
template <bool XB, bool DB, bool MULTI, bool REV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void scan_bwd_kernel(BwdArgs a,
                                                                                              int64_t wgs_per_batch) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r = lane >> 2, c = lane & 3;
  const int64_t nb = gridDim.x;
  int64_t lin = blockIdx.x;
  if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);
  const int64_t b = lin / wgs_per_batch;
  const int64_t grp = lin % wgs_per_batch;
  const int64_t chw0 = grp * BWC;
  const int64_t ch = chw0 + w * BCH + c;
  const bool nok = ch < a.dim && a.n0 + r < a.dstate;
  const float av = nok ? a.A[ch * a.dstate + a.n0 + r] : -1.f;
  const float a2 = av * kLog2e, ia = 1.f / av;
  const bool tiny = !(fabsf(av) >= 1e-2f);
  __shared__ __attribute__((aligned(16))) BwdLds lds;
  if (a.euler) scan_bwd_body<XB, DB, 2, MULTI, REV>(a, b, chw0, grp, av, a2, ia, nok, lds);
  else if (!XB || __syncthreads_or(tiny)) scan_bwd_body<XB, DB, 1, MULTI, REV>(a, b, chw0, grp, av, a2, ia, nok, lds);
  else scan_bwd_body<XB, DB, 0, MULTI, REV>(a, b, chw0, grp, av, a2, ia, nok, lds);
}

template <bool XB, bool DB>
hipError_t launch_bwd_xd(const BwdArgs& a, dim3 grid, int64_t wgs, hipStream_t st) {
  if (a.reverse) {
    if (a.acc != nullptr) scan_bwd_kernel<XB, DB, true, true><<<grid, 256, 0, st>>>(a, wgs);
    else scan_bwd_kernel<XB, DB, false, true><<<grid, 256, 0, st>>>(a, wgs);
  } else {
    if (a.acc != nullptr) scan_bwd_kernel<XB, DB, true, false><<<grid, 256, 0, st>>>(a, wgs);
    else scan_bwd_kernel<XB, DB, false, false><<<grid, 256, 0, st>>>(a, wgs);
  }
  return hipGetLastError();
}

// One delta per token: ddelta[row] = sum over the channels of the per-channel
// ddelta, in a fixed order (lane-strided partial sums, then a wave tree), so
// it is deterministic.  One wave per (batch, token) row.
template <bool DB>
__global__ __launch_bounds__(256) void bwd_sum_channels_kernel(const float* __restrict__ tc, void* out, int64_t rows,
                                                               int64_t dim) {
  const int64_t row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = tc + row * dim;
  float s = 0.f;
  for (int64_t c = l; c < dim; c += 64) s += p[c];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (l == 0) {
    if (DB) ((__bf16*)out)[row] = (__bf16)s;
    else ((float*)out)[row] = s;
  }
}

// Workspace: the states of one block of 16 at every tile start, the dB/dC
// partials of one block, and (dstate > 16) the three fp32 accumulators.
size_t ckpt_bytes(int64_t batch, int64_t seqlen, int64_t dim) {
  const int64_t ntile = (seqlen + BT - 1) / BT;
  return ((size_t)(ntile * batch * dim * BR) * sizeof(float) + 255) / 256 * 256;
}
size_t part_bytes(int64_t batch, int64_t seqlen, int64_t dim) {
  const int64_t groups = (dim + BWC - 1) / BWC;
  return ((size_t)(2 * groups * batch * seqlen * BR) * sizeof(float) + 255) / 256 * 256;
}

}  // namespace

size_t acc_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  return dstate > BR ? ((size_t)(3 * batch * seqlen * dim) * sizeof(float) + 255) / 256 * 256 : 0;
}

size_t scan_bwd_ws_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, bool tok_delta, bool saved) {
  const size_t tc = tok_delta ? (size_t)(batch * seqlen * dim) * sizeof(float) : 0;
  return (saved ? 0 : ckpt_bytes(batch, seqlen, dim)) + part_bytes(batch, seqlen, dim) +
         acc_bytes(batch, seqlen, dim, dstate) + tc;
}

int launch_scan_bwd(const BwdArgs& a0, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  BwdArgs a = a0;
  // the gradients summed over batch and time are accumulated: clear them first
  auto zero = [&](float* p, int64_t n) -> hipError_t {
    if (p == nullptr || n == 0) return hipSuccess;
    bwd_zero_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(p, n);
    return hipGetLastError();
  };
  hipError_t e = zero(a.dA, a.dim * a.dstate);
  if (e == hipSuccess) e = zero(a.dDskip, a.dim);
  if (e == hipSuccess) e = zero(a.ddelta_bias, a.dim);
  if (e != hipSuccess) return fail(6, std::string("backward clear: ") + hipGetErrorString(e));
  const int64_t wgs = (a.dim + BWC - 1) / BWC;
  const int64_t nb = a.batch * wgs;
  if (nb > 0x7fffffffLL) return fail(4, "grid too large");
  a.ws_groups = wgs;
  a.ws_part = nullptr;
  a.acc = nullptr;
  a.ddelta_tc = nullptr;
  if (a.ws_ckpt != nullptr) {
    char* base = (char*)a.ws_ckpt;
    const size_t ck = a.saved != nullptr ? 0 : ckpt_bytes(a.batch, a.seqlen, a.dim);
    const size_t pb = part_bytes(a.batch, a.seqlen, a.dim);
    a.ws_part = (float*)(base + ck);
    if (a.dstate > BR) a.acc = (float*)(base + ck + pb);
    if (a.tok_delta) a.ddelta_tc = (float*)(base + ck + pb + acc_bytes(a.batch, a.seqlen, a.dim, a.dstate));
  }
  const dim3 grid((unsigned)nb);
  const int64_t rows = a.batch * a.seqlen;
  // the states are independent given dy: one pass per block of 16, in stream order
  for (int64_t n0 = 0; n0 < a.dstate; n0 += BR) {
    a.n0 = n0;
    a.first = n0 == 0;
    a.last = n0 + BR >= a.dstate;
    if (a.act_bf16 && a.delta_bf16) e = launch_bwd_xd<true, true>(a, grid, wgs, st);
    else if (a.act_bf16) e = launch_bwd_xd<true, false>(a, grid, wgs, st);
    else if (a.delta_bf16) e = launch_bwd_xd<false, true>(a, grid, wgs, st);
    else e = launch_bwd_xd<false, false>(a, grid, wgs, st);
    if (e != hipSuccess) return fail(6, std::string("backward launch: ") + hipGetErrorString(e));
    if (rows > 0) {
      const int width = (int)(a.dstate - n0 < BR ? a.dstate - n0 : BR);
      const int64_t items = rows * width;
      bwd_sum_partials_kernel<<<dim3((unsigned)((items + 255) / 256)), 256, 0, st>>>(
          a.ws_part, a.ws_part + wgs * rows * BR, a.dB, a.dC, rows, wgs, a.dstate, n0, width, a.seqlen, a.reverse);
      e = hipGetLastError();
      if (e != hipSuccess) return fail(6, std::string("backward partial sums: ") + hipGetErrorString(e));
    }
  }
  if (a.tok_delta && rows > 0) {
    const dim3 g((unsigned)((rows + 3) / 4));
    if (a.delta_bf16) bwd_sum_channels_kernel<true><<<g, 256, 0, st>>>(a.ddelta_tc, a.ddelta, rows, a.dim);
    else bwd_sum_channels_kernel<false><<<g, 256, 0, st>>>(a.ddelta_tc, a.ddelta, rows, a.dim);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(6, std::string("backward channel sum: ") + hipGetErrorString(e));
  }
  return 0;
}

}  // namespace ssm
