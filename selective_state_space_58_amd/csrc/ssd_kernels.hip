// Mamba-2 SSD (structured state space duality) forward for MI355X / gfx950.
//
// Per batch b and head h (scalar decay a = A[h], group g = h / (H/G)), with
// ZOH gain g_t = expm1(dt_t a)/a, the sequence map is
//   y_t[p] = sum_{s<=t} (C_t . B_s) exp(a sum_{r=s+1..t} dt_r) g_s x_s[p]
//            + C_t . exp(a sum_{r<=t} dt_r) h0[p]
// ("Mamba-2 / SSD": the SSM as a semiseparable matrix; linear and quadratic
// forms).  It is computed block by block ("Mamba / SSM complete guide",
// sec. 6: matrix products inside a chunk, a recurrence across chunks):
//   cum_t    = a * sum_{r in block, r<=t} dt_r          (inclusive, per block)
//   Y_diag   = M X,   M[t,s] = (C_t . B_s) exp(cum_t - cum_s) g_s for s <= t
//   Y_off    = diag(exp(cum_t)) C H^T                    (state entering the block)
//   S_blk    = (X o w)^T B,     w_s = exp(cum_end - cum_s) g_s
//   H       <- exp(cum_end) H + S_blk
//
// Mapping.  One workgroup of 8 waves per (batch, head, half of the 64 head
// channels): 256 workgroups for the 2-batch, 64-head workload, one per CU and
// two waves per SIMD.  The workgroup walks the sequence in 64-token blocks;
// the fp32 state H (32 x dstate) stays in MFMA accumulator registers for the
// whole sequence and is never written to HBM.  All products are
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  B, C and x are staged in
// LDS in their natural token-major layout; the products that contract over
// tokens (X for M X, X and B for (X o w)^T B) read their operands with the
// gfx950 LDS transpose load (ds_read_b64_tr_b16), so no transposed copies are
// made.  The fp32 operands (M, x*w and the state) enter as a bf16 high part
// plus a bf16 low part, keeping ~16 bits instead of 8: a single bf16 copy of
// the state loses accuracy where C.H cancels over the states.  The block's
// decay prefix sum is a DPP scan in one wave during staging; the next block's
// B, C, x and dt are loaded into registers while the current one computes.
//
// Block size.  Any chunk length that is a multiple of 64 gives the same map
// (the state entering a 64-token block is the decayed sum of everything
// before it, whether that part of the sum is formed as a matrix product or
// carried as state), so the kernel always passes state every 64 tokens: with
// the state on chip, a 64-token block needs fewer matrix FLOPs and a quarter
// of the decay exponentials of a 256-token block.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int QB = 64;    // tokens per block
constexpr int PS = 32;    // head channels per workgroup
constexpr int NWAVE = 8;  // waves per workgroup

__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }
__device__ __forceinline__ float exp_f(float v) { return hw_exp2(v * kLog2e); }

__device__ __forceinline__ float bf2f(u16 v) {
  const unsigned u = (unsigned)v << 16;
  return __builtin_bit_cast(float, u);
}
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ float softplus_f(float v) {
  const float e = hw_exp2(-fabsf(v) * kLog2e);
  const float ser = e * fmaf(e, fmaf(e, fmaf(e, fmaf(e, fmaf(e, -1.f / 6.f, 0.2f), -0.25f), 1.f / 3.f), -0.5f), 1.f);
  const float lg = hw_log2(1.f + e) * kLn2;
  const float r = fmaxf(v, 0.f) + (e < 0.0625f ? ser : lg);
  return v > 20.f ? v : r;
}

__device__ __forceinline__ float silu_f(float z) { return z * hw_rcp(1.f + hw_exp2(-z * kLog2e)); }

// ZOH gain (e^{dt a} - 1)/a, accurate for small |dt a| (gives dt when a == 0).
__device__ __forceinline__ float zoh_gain(float dt, float a) {
  const float q = dt * a;
  const float phi = fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, fmaf(q, 1.f / 5040.f, 1.f / 720.f), 1.f / 120.f),
                                                 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
  const float ia = 1.f / a;
  return fabsf(q) < 0.25f ? dt * phi : (exp_f(q) - 1.f) * ia;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x) {
  const int r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false);
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_f<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f<0x118, 0xf>(v);  // row_shr:8
  v += dpp_f<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Fragment with 8 consecutive bf16 of row `row` from column `col` (row-major LDS matrix).
__device__ __forceinline__ bf16x8 frag_rows(const u16* base, int row, int col, int stride) {
  return *reinterpret_cast<const bf16x8*>(base + row * stride + col);
}

// Transposed fragment: for lane i of each 16-lane group, rows k0 .. k0+7 of
// column c0 + i of a row-major bf16 LDS matrix.  Two ds_read_b64_tr_b16: lane
// j of the group loads row k0 + q + j/4, columns c0 + 4*(j%4) .. +3, and the
// hardware hands lane i element i%4 of the loads of lanes i/4, i/4+4, i/4+8,
// i/4+12, i.e. rows k0+q .. k0+q+3 of column c0 + i.
__device__ __forceinline__ u32x4 frag_cols_raw(const u16* base, int k0, int c0, int stride, int l16) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const u16* p0 = base + (k0 + (l16 >> 2)) * stride + c0 + 4 * (l16 & 3);
  const u16* p1 = p0 + 4 * stride;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

__device__ __forceinline__ u16 half_of(const u32x4& v, int q) {
  const unsigned w = v[q >> 1];
  return (u16)(w >> (16 * (q & 1)));
}

// FULL: outputs for one time chunk, starting from the state carried into it.
// !FULL: the chunk's own state contribution (from a zero state) and its total
// decay exponent a * sum(dt), for the carry pass; no outputs.  The state pass
// needs few registers and is held to 128 VGPRs (two workgroups per CU); the
// full pass keeps its 2 waves per SIMD (capping it at 128 VGPRs spills and
// measured 2.5x slower).
template <int N, bool DTB, bool FULL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(FULL ? 2 : 4))) void ssd_fused_kernel(SsdArgs a) {
  constexpr int SN = N + 8;        // row stride of [*][N] LDS arrays (bf16 elements)
  constexpr int SQ = QB + 8;       // row stride of [*][64] LDS arrays
  constexpr int SP = PS + 8;       // row stride of the x tile
  constexpr int KN = N / 32;       // k-steps over the state dimension
  constexpr int NTW = N / 64;      // 16-wide state tiles owned by each wave (4 waves per p-tile)
  constexpr int CPR = N / 8;       // 16-byte chunks per B/C row
  constexpr int BC_CHUNKS = QB * CPR / (NWAVE * 64);  // B (and C) chunks per thread per block
  static_assert(BC_CHUNKS >= 1 && (QB * CPR) % (NWAVE * 64) == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) u16 Cs[QB * SN];   // C block [t][n]
  __shared__ __attribute__((aligned(16))) u16 Bs[QB * SN];   // B block [s][n]
  __shared__ __attribute__((aligned(16))) u16 Xs[QB * SP];   // x block [s][p]
  __shared__ __attribute__((aligned(16))) u16 XWh[QB * SP];  // x_s[p] * w_s [s][p], high part
  __shared__ __attribute__((aligned(16))) u16 XWl[QB * SP];  // low part
  __shared__ __attribute__((aligned(16))) u16 Ms[QB * SQ];   // masked decayed C B^T [t][s], high part
  __shared__ __attribute__((aligned(16))) u16 Ml[QB * SQ];   // low part
  __shared__ __attribute__((aligned(16))) u16 Hs[PS * SN];   // state [p][n], high part
  __shared__ __attribute__((aligned(16))) u16 Hl[PS * SN];   // low part
  __shared__ float cumS[QB], gS[QB], eS[QB], wS[QB];
  __shared__ float decayS;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63, l16 = l & 15, g4 = l >> 4;
  const int tw = w & 3;        // this wave's 16-token tile of the block (outputs)
  const int pw = w >> 2;       // this wave's 16-channel tile of the 32 head channels
  const int64_t H = a.nheads, P = a.headdim, L = a.seqlen;
  const int64_t nb = gridDim.x;
  int64_t lin = blockIdx.x;
  if ((nb & 7) == 0) lin = (lin & 7) * (nb >> 3) + (lin >> 3);  // a contiguous range of heads per XCD
  const int ph = (int)(lin & 1);
  const int64_t h = (lin >> 1) % H;
  const int64_t b = (lin >> 1) / H;
  const int64_t grp = h / (H / a.ngroups);
  const float av = a.A[h];
  const float bias = a.dt_bias != nullptr ? a.dt_bias[h] : 0.f;
  const float Dv = a.Dskip != nullptr ? a.Dskip[h] : 0.f;
  const int64_t p0 = (int64_t)ph * PS;
  const int64_t chunk = blockIdx.y;
  const int64_t t_begin = chunk * a.tchunk;
  const int64_t t_end = t_begin + a.tchunk < L ? t_begin + a.tchunk : L;
  const int64_t slice = a.batch * H * P * N;     // one state per (batch, head)

  const u16* gX = (const u16*)a.x;
  const u16* gB = (const u16*)a.B;
  const u16* gC = (const u16*)a.C;
  const u16* gZ = (const u16*)a.z;
  u16* gY = (u16*)a.y;

  // strictly-upper 16x16 tiles of M are never written by the mask: zero them once
  for (int i = tid; i < QB * SQ; i += NWAVE * 64) {
    Ms[i] = 0;
    Ml[i] = 0;
  }

  // ---- state: wave w owns p-tile pw and n-tiles [NTW*tw, NTW*tw + NTW).  The products are
  // computed transposed (state^T = B^T (X o w), so each accumulator lane holds four consecutive
  // states of one channel: H[p = 16 pw + l16][n = 16 nt + 4 g4 + v], v = 0..3.
  // FULL: h0, or the carry into this chunk; !FULL: zero.
  const float* hin = !FULL ? nullptr : (a.nchunks > 1 ? a.ws_state + chunk * slice : a.h0);
  const int64_t hrow = ((b * H + h) * P + p0 + pw * 16 + l16) * N;   // this lane's channel row of a state
  f32x4 Hacc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int n = (NTW * tw + j) * 16 + 4 * g4;
    Hacc[j] = hin != nullptr ? *reinterpret_cast<const f32x4*>(hin + hrow + n) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto store_state_split = [&]() {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int idx = (pw * 16 + l16) * SN + (NTW * tw + j) * 16 + 4 * g4;
      u32x2 hi, lo;
#pragma unroll
      for (int v = 0; v < 4; v += 2) {
        const u16 h0b = f2bf(Hacc[j][v]), h1b = f2bf(Hacc[j][v + 1]);
        hi[v >> 1] = (unsigned)h0b | ((unsigned)h1b << 16);
        lo[v >> 1] = (unsigned)f2bf(Hacc[j][v] - bf2f(h0b)) | ((unsigned)f2bf(Hacc[j][v + 1] - bf2f(h1b)) << 16);
      }
      *reinterpret_cast<u32x2*>(Hs + idx) = hi;
      *reinterpret_cast<u32x2*>(Hl + idx) = lo;
    }
  };
  if (FULL) store_state_split();   // visible after the first barrier of the block loop

  // ---- register prefetch of one block
  u32x4 rc[BC_CHUNKS], rb[BC_CHUNKS], rx;
  float rdt = 0.f;
  const int64_t last = L - 1;
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int j = 0; j < BC_CHUNKS; ++j) {
      const int e = tid + NWAVE * 64 * j;
      const int row = e / CPR, c8 = e % CPR;
      int64_t t = t0 + row;
      t = t < last ? t : last;
      const int64_t off = ((b * L + t) * a.ngroups + grp) * N + c8 * 8;
      if (FULL) rc[j] = *reinterpret_cast<const u32x4*>(gC + off);
      rb[j] = *reinterpret_cast<const u32x4*>(gB + off);
    }
    if (tid < QB * PS / 8) {
      const int row = tid >> 2, c8 = tid & 3;
      int64_t t = t0 + row;
      t = t < last ? t : last;
      rx = *reinterpret_cast<const u32x4*>(gX + ((b * L + t) * H + h) * P + p0 + c8 * 8);
    }
    if (w == 0) {
      int64_t t = t0 + l;
      t = t < last ? t : last;
      const int64_t i = (b * L + t) * H + h;
      rdt = DTB ? bf2f(((const u16*)a.dt)[i]) : ((const float*)a.dt)[i];
    }
  };

  const int nblk = (int)((t_end - t_begin + QB - 1) / QB);
  float dsum = 0.f;                  // a * sum of dt over the chunk (wave 0)
  fetch(t_begin);
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = t_begin + (int64_t)blk * QB;
    // ---------------- stage the block (natural layouts) and the decay terms
#pragma unroll
    for (int j = 0; j < BC_CHUNKS; ++j) {
      const int e = tid + NWAVE * 64 * j;
      const int row = e / CPR, c8 = e % CPR;
      if (FULL) *reinterpret_cast<u32x4*>(Cs + row * SN + c8 * 8) = rc[j];
      *reinterpret_cast<u32x4*>(Bs + row * SN + c8 * 8) = rb[j];
    }
    if (tid < QB * PS / 8) {
      const int row = tid >> 2, c8 = tid & 3;
      *reinterpret_cast<u32x4*>(Xs + row * SP + c8 * 8) = rx;
    }
    if (w == 0) {
      // lane l = token t0 + l: dt, the inclusive scan of dt*a, gain and decays
      const float v = rdt + bias;
      float dtv = a.softplus ? softplus_f(v) : v;
      if (t0 + l >= L) dtv = 0.f;   // past the end: no input, no decay
      const float cum = wave_prefix_sum(dtv * av);
      const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), 63));
      const float gv = zoh_gain(dtv, av);
      cumS[l] = cum;
      gS[l] = gv;
      eS[l] = exp_f(cum);
      wS[l] = exp_f(cend - cum) * gv;
      if (l == 0) decayS = exp_f(cend);
      dsum += cend;
    }
    __syncthreads();
    if (tid < QB * PS / 8) {
      // x * w for the state product, once per workgroup, from the staged registers
      const int row = tid >> 2, c8 = tid & 3;
      const float ws = wS[row];
      u32x4 hi, lo;
#pragma unroll
      for (int q = 0; q < 8; q += 2) {
        const float f0 = bf2f(half_of(rx, q)) * ws, f1 = bf2f(half_of(rx, q + 1)) * ws;
        const u16 h0b = f2bf(f0), h1b = f2bf(f1);
        hi[q >> 1] = (unsigned)h0b | ((unsigned)h1b << 16);
        lo[q >> 1] = (unsigned)f2bf(f0 - bf2f(h0b)) | ((unsigned)f2bf(f1 - bf2f(h1b)) << 16);
      }
      *reinterpret_cast<u32x4*>(XWh + row * SP + c8 * 8) = hi;
      *reinterpret_cast<u32x4*>(XWl + row * SP + c8 * 8) = lo;
    }
    if (blk + 1 < nblk) fetch(t0 + QB);

    // ---------------- C B^T tiles -> mask -> M (bf16 high/low) in LDS
    if constexpr (FULL) {
      // (B C^T)[s][t]: lane (l16, g4) gets M's row t = 16 ti + l16 at s = 16 tj + 4 g4 .. +3
      auto cb_tile = [&](int ti, int tj) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk)
          acc = mfma(frag_rows(Bs, tj * 16 + l16, kk * 32 + g4 * 8, SN), frag_rows(Cs, ti * 16 + l16, kk * 32 + g4 * 8, SN),
                     acc);
        const int t = ti * 16 + l16;
        const int s0 = tj * 16 + 4 * g4;
        const float ct = cumS[t];
        u32x2 hi, lo;
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const int s = s0 + v;
          const float m0 = (t >= s) ? acc[v] * exp_f(ct - cumS[s]) * gS[s] : 0.f;
          const float m1 = (t >= s + 1) ? acc[v + 1] * exp_f(ct - cumS[s + 1]) * gS[s + 1] : 0.f;
          const u16 h0b = f2bf(m0), h1b = f2bf(m1);
          hi[v >> 1] = (unsigned)h0b | ((unsigned)h1b << 16);
          lo[v >> 1] = (unsigned)f2bf(m0 - bf2f(h0b)) | ((unsigned)f2bf(m1 - bf2f(h1b)) << 16);
        }
        *reinterpret_cast<u32x2*>(Ms + t * SQ + s0) = hi;
        *reinterpret_cast<u32x2*>(Ml + t * SQ + s0) = lo;
      };
      // 10 causal tiles: one per wave, a second for two of the waves that have no x * w to form
      switch (w) {
        case 0: cb_tile(0, 0); break;
        case 1: cb_tile(1, 0); break;
        case 2: cb_tile(1, 1); break;
        case 3: cb_tile(2, 0); break;
        case 4: cb_tile(2, 1); cb_tile(2, 2); break;
        case 5: cb_tile(3, 0); cb_tile(3, 1); break;
        case 6: cb_tile(3, 2); break;
        default: cb_tile(3, 3); break;
      }
    }

    // ---------------- Y_off^T = H C^T for (channel tile pw, token tile tw); H = state entering the block
    f32x4 yoff = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < (FULL ? KN : 0); ++kk) {
      const bf16x8 cb = frag_rows(Cs, tw * 16 + l16, kk * 32 + g4 * 8, SN);
      yoff = mfma(frag_rows(Hs, pw * 16 + l16, kk * 32 + g4 * 8, SN), cb, yoff);
      yoff = mfma(frag_rows(Hl, pw * 16 + l16, kk * 32 + g4 * 8, SN), cb, yoff);
    }

    __syncthreads();   // M and x*w complete; every wave has finished reading Hs/Hl

    // ---------------- S^T = B^T (X o w) for (state tiles of this wave, channel tile pw); H <- decay H + S
    {
      bf16x8 xh[2], xl[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // rows s = 32kk + 8g4 .. +7 of column p = 16pw + l16 of x*w
        xh[kk] = __builtin_bit_cast(bf16x8, frag_cols_raw(XWh, kk * 32 + g4 * 8, pw * 16, SP, l16));
        xl[kk] = __builtin_bit_cast(bf16x8, frag_cols_raw(XWl, kk * 32 + g4 * 8, pw * 16, SP, l16));
      }
      const float dec = decayS;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nt = NTW * tw + j;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 bt = __builtin_bit_cast(bf16x8, frag_cols_raw(Bs, kk * 32 + g4 * 8, nt * 16, SN, l16));
          s = mfma(bt, xh[kk], s);
          s = mfma(bt, xl[kk], s);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) Hacc[j][v] = fmaf(dec, Hacc[j][v], s[v]);
      }
    }


    // ---------------- Y_diag^T = X^T M^T for (channel tile pw, token tile tw), epilogue
    f32x4 ydiag = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FULL) {
      const int ksteps = (tw < 2) ? 1 : 2;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk < ksteps) {
          const bf16x8 xb = __builtin_bit_cast(bf16x8, frag_cols_raw(Xs, kk * 32 + g4 * 8, pw * 16, SP, l16));
          ydiag = mfma(xb, frag_rows(Ms, tw * 16 + l16, kk * 32 + g4 * 8, SQ), ydiag);
          ydiag = mfma(xb, frag_rows(Ml, tw * 16 + l16, kk * 32 + g4 * 8, SQ), ydiag);
        }
      }
    }
    if constexpr (FULL) {
      // lane (l16, g4): token t0 + 16 tw + l16, channels 16 pw + 4 g4 .. +3 (one 8-byte store)
      const int tl = tw * 16 + l16;
      const int p = pw * 16 + 4 * g4;
      const int64_t t = t0 + tl;
      if (t < L) {
        const float et = eS[tl];
        float yv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) yv[v] = fmaf(et, yoff[v], ydiag[v]);
        const int64_t gi = ((b * L + t) * H + h) * P + p0 + p;
        if (a.Dskip != nullptr) {
          const u32x2 xr = *reinterpret_cast<const u32x2*>(Xs + tl * SP + p);
#pragma unroll
          for (int v = 0; v < 4; ++v) yv[v] = fmaf(Dv, bf2f((u16)(xr[v >> 1] >> (16 * (v & 1)))), yv[v]);
        }
        if (a.z != nullptr) {
          const u32x2 zr = *reinterpret_cast<const u32x2*>(gZ + gi);
#pragma unroll
          for (int v = 0; v < 4; ++v) yv[v] *= silu_f(bf2f((u16)(zr[v >> 1] >> (16 * (v & 1)))));
        }
        u32x2 out;
        out[0] = (unsigned)f2bf(yv[0]) | ((unsigned)f2bf(yv[1]) << 16);
        out[1] = (unsigned)f2bf(yv[2]) | ((unsigned)f2bf(yv[3]) << 16);
        *reinterpret_cast<u32x2*>(gY + gi) = out;
      }
    }
    if (FULL) store_state_split();   // the state entering the next block
    __syncthreads();
  }

  float* hout = FULL ? (chunk == a.nchunks - 1 ? a.h_final : nullptr) : a.ws_state + chunk * slice;
  if (hout != nullptr) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) *reinterpret_cast<f32x4*>(hout + hrow + (NTW * tw + j) * 16 + 4 * g4) = Hacc[j];
  }
  if (!FULL && w == 0 && l == 0 && ph == 0) a.ws_dsum[chunk * a.batch * H + b * H + h] = dsum;
}

// Combine the chunk states in order: slot c of ws_state receives the state
// entering chunk c, h_in(c+1) = exp(dsum_c) h_in(c) + s(c), h_in(0) = h0.
__global__ __launch_bounds__(256) void ssd_carry_kernel(SsdArgs a) {
  const int64_t slice = a.batch * a.nheads * a.headdim * a.dstate;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= slice) return;
  const int64_t bh = i / (a.headdim * a.dstate);
  float hv = a.h0 != nullptr ? a.h0[i] : 0.f;
  for (int64_t c = 0; c + 1 < a.nchunks; ++c) {
    const float loc = a.ws_state[c * slice + i];
    a.ws_state[c * slice + i] = hv;
    hv = fmaf(exp_f(a.ws_dsum[c * a.batch * a.nheads + bh]), hv, loc);
  }
  a.ws_state[(a.nchunks - 1) * slice + i] = hv;
}

// seqlen == 0: the state passes through unchanged.
__global__ __launch_bounds__(256) void ssd_copy_state(const float* h0, float* out, int64_t total) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < total) out[i] = h0 != nullptr ? h0[i] : 0.f;
}

}  // namespace

SsdPlan plan_ssd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate, int num_cus) {
  // The full pass runs one workgroup per CU (its registers allow no second),
  // so time is split only when the (batch, head, half) workgroups cannot fill
  // the CUs: into enough chunks for one workgroup per CU, each of at least 8
  // blocks.  A split costs a state-only pass over its chunks and a carry of
  // one state per (batch, head); with the CUs already full it measured slower
  // (0.48 against 0.39 ms on the b2 x 64-head workload).
  SsdPlan p{1, 0, 0};
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t nwg = batch * nheads * (headdim / PS);
  if (nwg > 0 && nwg < cus && seqlen > 0) {
    int64_t nch = (cus + nwg - 1) / nwg;
    const int64_t max_ch = seqlen / (8 * QB);
    nch = nch < max_ch ? nch : max_ch;
    nch = nch > 1 ? nch : 1;
    const int64_t per = (seqlen + nch - 1) / nch;
    p.tchunk = (per + QB - 1) / QB * QB;
    p.nchunks = (seqlen + p.tchunk - 1) / p.tchunk;
  }
  p.tchunk = p.nchunks > 1 ? p.tchunk : (seqlen > 0 ? (seqlen + QB - 1) / QB * QB : QB);
  if (p.nchunks > 1) {
    const size_t st = (size_t)p.nchunks * (size_t)(batch * nheads * headdim * dstate) * sizeof(float);
    p.ws_bytes = (st + 255) / 256 * 256 + (size_t)p.nchunks * (size_t)(batch * nheads) * sizeof(float);
  }
  return p;
}

size_t ssd_ws_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t, int64_t dstate,
                    int64_t) {
  return plan_ssd(batch, seqlen, nheads, headdim, dstate, device_cu_count()).ws_bytes;
}

template <int N, bool DTB>
hipError_t launch_ssd_n(const SsdArgs& a, dim3 grid, hipStream_t st) {
  if (a.nchunks > 1) {
    ssd_fused_kernel<N, DTB, false><<<dim3(grid.x, (unsigned)(a.nchunks - 1)), NWAVE * 64, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t slice = a.batch * a.nheads * a.headdim * a.dstate;
    ssd_carry_kernel<<<dim3((unsigned)((slice + 255) / 256)), 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ssd_fused_kernel<N, DTB, true><<<dim3(grid.x, (unsigned)a.nchunks), NWAVE * 64, 0, st>>>(a);
  return hipGetLastError();
}

int launch_ssd(const SsdArgs& a0, void* stream) {
  SsdArgs a = a0;
  hipStream_t st = (hipStream_t)stream;
  if (a.seqlen == 0) {
    if (a.h_final != nullptr) {
      const int64_t total = a.batch * a.nheads * a.headdim * a.dstate;
      ssd_copy_state<<<dim3((unsigned)((total + 255) / 256)), 256, 0, st>>>(a.h0, a.h_final, total);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(6, std::string("SSD state copy: ") + hipGetErrorString(e));
    }
    return 0;
  }
  const int64_t nwg = a.batch * a.nheads * (a.headdim / PS);
  if (nwg > 0x7fffffffLL) return fail(4, "grid too large");
  const SsdPlan p = plan_ssd(a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, device_cu_count());
  if (p.nchunks > 65535) return fail(4, "grid too large");
  a.nchunks = p.nchunks;
  a.tchunk = p.tchunk;
  if (p.nchunks > 1) {
    if (a.ws == nullptr) return fail(5, "SSD time split needs its workspace");
    const size_t st_bytes = (size_t)p.nchunks * (size_t)(a.batch * a.nheads * a.headdim * a.dstate) * sizeof(float);
    a.ws_state = (float*)a.ws;
    a.ws_dsum = (float*)((char*)a.ws + (st_bytes + 255) / 256 * 256);
  }
  dim3 grid((unsigned)nwg);
  hipError_t e;
  if (a.dstate == 128) e = a.dt_bf16 ? launch_ssd_n<128, true>(a, grid, st) : launch_ssd_n<128, false>(a, grid, st);
  else e = a.dt_bf16 ? launch_ssd_n<64, true>(a, grid, st) : launch_ssd_n<64, false>(a, grid, st);
  if (e != hipSuccess) return fail(6, std::string("SSD kernel launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
