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
//   Y_diag   = (C B^T o M) X,   M[t,s] = exp(cum_t - cum_s) g_s for s <= t
//   Y_off    = diag(exp(cum_t)) C H^T                    (state entering the block)
//   S_blk    = (X o w)^T B,     w_s = exp(cum_end - cum_s) g_s
//   H       <- exp(cum_end) H + S_blk
//
// Mapping.  One workgroup of 4 waves per (batch, head, half of the 64 head
// channels): 2 x 64 x 2 = 256 workgroups for the 64-head, 2-batch workload,
// one per CU.  The workgroup walks the sequence in 64-token blocks; the fp32
// state H (32 x dstate) stays in the MFMA accumulator registers of the four
// waves for the whole sequence and is never written to HBM (only its bf16
// high/low copy for the next block's C H^T goes to LDS).  All products are
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the three fp32 operands
// (the masked C B^T, x*w and the state) enter as a bf16 high part plus a bf16
// low part, so they keep ~16 bits instead of 8.  The next block's B, C, x
// and dt are loaded into registers while the current block is computed.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int QB = 64;   // tokens per block
constexpr int PS = 32;   // head channels per workgroup

__device__ __forceinline__ float hw_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float hw_log2(float v) { return __builtin_amdgcn_logf(v); }
__device__ __forceinline__ float hw_rcp(float v) { return __builtin_amdgcn_rcpf(v); }
__device__ __forceinline__ float exp_f(float v) { return hw_exp2(v * kLog2e); }

__device__ __forceinline__ float bf2f(u16 v) { return __builtin_bit_cast(float, (unsigned)v << 16); }
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

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte fragment: 8 consecutive bf16 of row `row` starting at column `col`.
__device__ __forceinline__ bf16x8 frag(const u16* base, int row, int col, int stride) {
  return *reinterpret_cast<const bf16x8*>(base + row * stride + col);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 8 bf16, 16 bytes

__device__ __forceinline__ u16 half_of(u32x4 v, int q) { return (u16)(v[q >> 1] >> (16 * (q & 1))); }

template <int N, bool DTB>
__global__ __launch_bounds__(256) void ssd_fused_kernel(SsdArgs a) {
  constexpr int SN = N + 8;        // row stride of [*][N] LDS arrays (bf16 elements)
  constexpr int SQ = QB + 8;       // row stride of [*][64] LDS arrays
  constexpr int KN = N / 32;       // k-steps over the state dimension
  constexpr int NT = N / 16;       // 16-wide state tiles
  constexpr int NTW = NT / 4;      // state tiles owned by each wave
  constexpr int CPR = N / 8;       // 16-byte chunks per B/C row
  constexpr int BC_CHUNKS = QB * CPR / 256;  // B (and C) chunks loaded per thread per block
  static_assert(BC_CHUNKS >= 1 && (QB * CPR) % 256 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) u16 Cs[QB * SN];   // C block [t][n]
  __shared__ __attribute__((aligned(16))) u16 Bs[QB * SN];   // B block [s][n]
  __shared__ __attribute__((aligned(16))) u16 BsT[N * SQ];   // B block transposed [n][s]
  __shared__ __attribute__((aligned(16))) u16 XsT[PS * SQ];  // x block transposed [p][s]
  __shared__ __attribute__((aligned(16))) u16 Ms[QB * SQ];   // masked decayed C B^T [t][s], bf16 high part
  __shared__ __attribute__((aligned(16))) u16 Ml[QB * SQ];   // low part (M - high)
  __shared__ __attribute__((aligned(16))) u16 Hs[PS * SN];   // state [p][n], bf16 high part
  __shared__ __attribute__((aligned(16))) u16 Hl[PS * SN];   // state [p][n], bf16 low part (H - high)
  __shared__ float cumS[QB], gS[QB], eS[QB], wS[QB];
  __shared__ float decayS;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63, l16 = l & 15, g4 = l >> 4;
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

  const u16* gX = (const u16*)a.x;
  const u16* gB = (const u16*)a.B;
  const u16* gC = (const u16*)a.C;
  const u16* gZ = (const u16*)a.z;
  u16* gY = (u16*)a.y;

  // zero the strictly-upper 16x16 tiles of Ms once; the mask never writes them
  for (int i = tid; i < QB * SQ; i += 256) {
    Ms[i] = 0;
    Ml[i] = 0;
  }

  // ---- state: wave w owns n-tiles [w*NTW, w*NTW + NTW) x p-tiles {0, 1}
  f32x4 Hacc[2][NTW];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = (w * NTW + j) * 16 + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = pt * 16 + 4 * g4 + v;
        Hacc[pt][j][v] = a.h0 != nullptr ? a.h0[((b * H + h) * P + p0 + p) * N + n] : 0.f;
      }
    }

  // The state enters C H^T as two bf16 matrices, high = bf16(H) and
  // low = bf16(H - high), so the product keeps ~16 bits of the fp32 state (a
  // single bf16 copy loses too much where C.H cancels over the states).
  auto store_state_split = [&](const f32x4 (&Hr)[2][NTW], u16* hi, u16* lo) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int idx = (pt * 16 + 4 * g4 + v) * SN + (w * NTW + j) * 16 + l16;
          const u16 hb = f2bf(Hr[pt][j][v]);
          hi[idx] = hb;
          lo[idx] = f2bf(Hr[pt][j][v] - bf2f(hb));
        }
  };
  // bf16 copies of the initial state for the first block's C H^T (visible after
  // the first barrier of the block loop)
  store_state_split(Hacc, Hs, Hl);

  // ---- prefetch registers for one block
  u32x4 rc[BC_CHUNKS], rb[BC_CHUNKS], rx;
  float rdt = 0.f;
  auto fetch = [&](int64_t t0) {
    const int64_t last = L - 1;
#pragma unroll
    for (int j = 0; j < BC_CHUNKS; ++j) {
      const int e = tid + 256 * j;
      const int row = e / CPR, c8 = e % CPR;
      int64_t t = t0 + row;
      t = t < last ? t : last;
      const int64_t off = ((b * L + t) * a.ngroups + grp) * N + c8 * 8;
      rc[j] = *reinterpret_cast<const u32x4*>(gC + off);
      rb[j] = *reinterpret_cast<const u32x4*>(gB + off);
    }
    {
      const int row = tid >> 2, c8 = tid & 3;
      int64_t t = t0 + row;
      t = t < last ? t : last;
      rx = *reinterpret_cast<const u32x4*>(gX + ((b * L + t) * H + h) * P + p0 + c8 * 8);
    }
    if (tid < QB) {
      int64_t t = t0 + tid;
      t = t < last ? t : last;
      const int64_t i = (b * L + t) * H + h;
      rdt = DTB ? bf2f(((const u16*)a.dt)[i]) : ((const float*)a.dt)[i];
    }
  };

  // state readout of the block (Y_off) and diagonal part (Y_diag) of this wave's 16 rows
  const int nblk = (int)((L + QB - 1) / QB);
  fetch(0);
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = (int64_t)blk * QB;
    // ---------------- stage the block into LDS
#pragma unroll
    for (int j = 0; j < BC_CHUNKS; ++j) {
      const int e = tid + 256 * j;
      const int row = e / CPR, c8 = e % CPR;
      *reinterpret_cast<u32x4*>(Cs + row * SN + c8 * 8) = rc[j];
      *reinterpret_cast<u32x4*>(Bs + row * SN + c8 * 8) = rb[j];
#pragma unroll
      for (int q = 0; q < 8; ++q) BsT[(c8 * 8 + q) * SQ + row] = half_of(rb[j], q);
    }
    {
      const int row = tid >> 2, c8 = tid & 3;
#pragma unroll
      for (int q = 0; q < 8; ++q) XsT[(c8 * 8 + q) * SQ + row] = half_of(rx, q);
    }
    float dtv = 0.f;
    if (tid < QB) {
      const float v = rdt + bias;
      dtv = a.softplus ? softplus_f(v) : v;
      if (t0 + tid >= L) dtv = 0.f;   // past the end: no input, no decay
    }
    __syncthreads();
    if (blk + 1 < nblk) fetch(t0 + QB);

    // ---------------- per-token decay terms (wave 0): inclusive scan of dt*a over the block
    if (w == 0) {
      const float q = dtv * av;
      float cum = q;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(cum, d, 64);
        if (l >= d) cum += o;
      }
      const float cend = __shfl(cum, 63, 64);
      const float gv = zoh_gain(dtv, av);
      cumS[l] = cum;
      gS[l] = gv;
      eS[l] = exp_f(cum);
      wS[l] = exp_f(cend - cum) * gv;
      if (l == 0) decayS = exp_f(cend);
    }
    __syncthreads();

    // ---------------- C B^T tiles of this wave -> mask -> Ms (bf16)
    // causal 16x16 tiles (ti, tj), tj <= ti, split over the waves
    {
      auto cb_tile = [&](int ti, int tj) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk)
          acc = mfma(frag(Cs, ti * 16 + l16, kk * 32 + g4 * 8, SN), frag(Bs, tj * 16 + l16, kk * 32 + g4 * 8, SN), acc);
        const int s = tj * 16 + l16;
        const float cs = cumS[s], gs = gS[s];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = ti * 16 + 4 * g4 + v;
          const float m = (t >= s) ? acc[v] * exp_f(cumS[t] - cs) * gs : 0.f;
          const u16 mh = f2bf(m);
          Ms[t * SQ + s] = mh;
          Ml[t * SQ + s] = f2bf(m - bf2f(mh));
        }
      };
      if (w == 0) { cb_tile(0, 0); cb_tile(1, 0); cb_tile(1, 1); }
      else if (w == 1) { cb_tile(2, 0); cb_tile(2, 1); cb_tile(2, 2); }
      else if (w == 2) { cb_tile(3, 0); cb_tile(3, 1); }
      else { cb_tile(3, 2); cb_tile(3, 3); }
    }

    // ---------------- Y_off = C H^T for this wave's 16 rows (H = state entering the block)
    f32x4 yoff[2], ydiag[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      yoff[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      ydiag[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const bf16x8 ca = frag(Cs, w * 16 + l16, kk * 32 + g4 * 8, SN);
        yoff[pt] = mfma(ca, frag(Hs, pt * 16 + l16, kk * 32 + g4 * 8, SN), yoff[pt]);
        yoff[pt] = mfma(ca, frag(Hl, pt * 16 + l16, kk * 32 + g4 * 8, SN), yoff[pt]);
      }
    }

    // ---------------- S = (X o w)^T B for this wave's state tiles, then H <- decay H + S
    {
      // x*w enters as high + low bf16 parts (same reason as the state above)
      bf16x8 xa[2][2], xl[2][2];
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(XsT + (pt * 16 + l16) * SQ + kk * 32 + g4 * 8);
          bf16x8 fh, fl;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float f = bf2f(half_of(raw, q)) * wS[kk * 32 + g4 * 8 + q];
            fh[q] = (__bf16)f;
            fl[q] = (__bf16)(f - (float)fh[q]);
          }
          xa[pt][kk] = fh;
          xl[pt][kk] = fl;
        }
      const float dec = decayS;
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nt = w * NTW + j;
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 bt = frag(BsT, nt * 16 + l16, kk * 32 + g4 * 8, SQ);
            s = mfma(xa[pt][kk], bt, s);
            s = mfma(xl[pt][kk], bt, s);
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) Hacc[pt][j][v] = fmaf(dec, Hacc[pt][j][v], s[v]);
        }
      }
    }
    __syncthreads();   // Ms complete; every wave has finished reading Hs

    // ---------------- Y_diag = Ms X for this wave's rows
    {
      const int ksteps = (w < 2) ? 1 : 2;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          if (kk < ksteps) {
            const bf16x8 xb = frag(XsT, pt * 16 + l16, kk * 32 + g4 * 8, SQ);
            ydiag[pt] = mfma(frag(Ms, w * 16 + l16, kk * 32 + g4 * 8, SQ), xb, ydiag[pt]);
            ydiag[pt] = mfma(frag(Ml, w * 16 + l16, kk * 32 + g4 * 8, SQ), xb, ydiag[pt]);
          }
    }
    // ---------------- epilogue: y = Y_diag + exp(cum_t) Y_off (+ Dskip x) (* silu z)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tl = w * 16 + 4 * g4 + v;
        const int p = pt * 16 + l16;
        const int64_t t = t0 + tl;
        float yv = fmaf(eS[tl], yoff[pt][v], ydiag[pt][v]);
        if (t < L) {
          const int64_t gi = ((b * L + t) * H + h) * P + p0 + p;
          if (a.Dskip != nullptr) yv = fmaf(Dv, bf2f(XsT[p * SQ + tl]), yv);
          if (a.z != nullptr) yv *= silu_f(bf2f(gZ[gi]));
          gY[gi] = f2bf(yv);
        }
      }
    }
    // ---------------- bf16 high/low copy of the new state for the next block's C H^T
    store_state_split(Hacc, Hs, Hl);
    __syncthreads();
  }

  if (a.h_final != nullptr) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int n = (w * NTW + j) * 16 + l16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = pt * 16 + 4 * g4 + v;
          a.h_final[((b * H + h) * P + p0 + p) * N + n] = Hacc[pt][j][v];
        }
      }
  }
}

}  // namespace

size_t ssd_ws_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

int launch_ssd(const SsdArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.seqlen == 0) {
    // nothing to scan: the state passes through
    if (a.h_final != nullptr) {
      const size_t bytes = (size_t)(a.batch * a.nheads * a.headdim * a.dstate) * sizeof(float);
      hipError_t e = a.h0 != nullptr ? hipMemcpyAsync(a.h_final, a.h0, bytes, hipMemcpyDeviceToDevice, st)
                                     : hipMemsetAsync(a.h_final, 0, bytes, st);
      if (e != hipSuccess) return fail(6, std::string("SSD state copy: ") + hipGetErrorString(e));
    }
    return 0;
  }
  const int64_t nwg = a.batch * a.nheads * (a.headdim / PS);
  if (nwg > 0x7fffffffLL) return fail(4, "grid too large");
  dim3 grid((unsigned)nwg);
  if (a.dstate == 128) {
    if (a.dt_bf16) ssd_fused_kernel<128, true><<<grid, 256, 0, st>>>(a);
    else ssd_fused_kernel<128, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (a.dt_bf16) ssd_fused_kernel<64, true><<<grid, 256, 0, st>>>(a);
    else ssd_fused_kernel<64, false><<<grid, 256, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(6, std::string("SSD kernel launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
