// Causal depthwise 1-D convolution + SiLU: the step of the Mamba block that
// produces the scan's input x ("Mamba / SSM complete guide", sec. 5, the
// Mamba block: a Conv1d with one group per channel, padding width-1, output
// trimmed to the sequence length, then silu).  Per channel d:
//   out[t] = silu(bias_d + sum_k w[d][k] * x[t - (W-1) + k])
// where positions before the segment come from the carried-in state (the
// previous segment's last W-1 inputs; zeros when absent), and the segment's
// last W-1 inputs are written out as the new state.  With seqlen 1 and the
// state updated in place this is the decode-time convolution update.
//
// The pass is bound by HBM: x read once, out written once (the W-1 halo rows
// a chunk reads before its first token are the previous chunk's rows and come
// from L2).  A thread owns 8 consecutive channels (one 16-byte bf16 load per
// token) and a run of 16 tokens, keeps the W-tap window in registers and
// slides it one token at a time; neighbouring threads own neighbouring
// channel groups, so each token row is read as contiguous 1 KB wave accesses.
// out is stored with the nontemporal (streaming) hint (27.5 -> 26.9 us on the
// b8 x 2048 x 1536 pass); x is not, since its halo rows are read again.
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvTokens = 16;  // tokens per thread

template <bool BF16>
struct Vec8;
template <>
struct Vec8<true> {  // 8 bf16 in 16 bytes
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&v)[8]) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 r = *reinterpret_cast<const u32x4*>((const unsigned short*)p + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned u = r[q];
      v[2 * q] = __builtin_bit_cast(float, u << 16);
      v[2 * q + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&v)[8]) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const unsigned lo = __builtin_bit_cast(unsigned short, (__bf16)v[2 * q]);
      const unsigned hi = __builtin_bit_cast(unsigned short, (__bf16)v[2 * q + 1]);
      r[q] = lo | (hi << 16);
    }
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>((unsigned short*)p + i));
  }
};
template <>
struct Vec8<false> {  // 8 fp32 in 32 bytes
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>((const float*)p + i);
    const float4 b = *reinterpret_cast<const float4*>((const float*)p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&v)[8]) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>((float*)p + i));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>((float*)p + i + 4));
  }
};

template <bool BF16>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if (BF16) return __builtin_bit_cast(float, (unsigned)(((const unsigned short*)p)[i]) << 16);
  return ((const float*)p)[i];
}
template <bool BF16>
__device__ __forceinline__ void st1(void* p, int64_t i, float v) {
  if (BF16) ((__bf16*)p)[i] = (__bf16)v;
  else ((float*)p)[i] = v;
}

__device__ __forceinline__ float silu_conv(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f));
}

// V channels per thread (8 with 16/32-byte accesses, or 1).  Thread index
// order: channel group fastest, then token chunk, then batch.
template <int W, bool BF16, int V>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(ConvArgs a, unsigned cgroups, unsigned nchunk) {
  const unsigned lin = blockIdx.x * kConvThreads + threadIdx.x;
  const unsigned cg = lin % cgroups;
  const unsigned rest = lin / cgroups;
  const unsigned chunk = rest % nchunk;
  const unsigned b = rest / nchunk;
  if (b >= (unsigned)a.batch) return;
  const int64_t L = a.seqlen, dim = a.dim;
  const int64_t c0 = (int64_t)cg * V;
  const int64_t t0 = (int64_t)chunk * kConvTokens;
  const int64_t t1 = t0 + kConvTokens < L ? t0 + kConvTokens : L;
  const int64_t srow = ((int64_t)b * dim + c0) * (W - 1);  // state (b, c0, 0)

  auto load_row = [&](int64_t t, float (&v)[V]) {
    const int64_t i = ((int64_t)b * L + t) * dim + c0;
    if constexpr (V == 8) {
      Vec8<BF16>::load(a.x, i, v);
    } else {
      v[0] = ld1<BF16>(a.x, i);
    }
  };

  float wt[W][V], bs[V];
#pragma unroll
  for (int c = 0; c < V; ++c) {
#pragma unroll
    for (int k = 0; k < W; ++k) wt[k][c] = a.w[(c0 + c) * W + k];
    bs[c] = a.bias != nullptr ? a.bias[c0 + c] : 0.f;
  }
  // window: win[k] holds the input at position t - (W-1) + k
  float win[W][V];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t pos = t0 - (W - 1) + k;
    if (pos >= 0) {
      load_row(pos, win[k]);
    } else {
#pragma unroll
      for (int c = 0; c < V; ++c)
        win[k][c] = a.state_in != nullptr ? ld1<BF16>(a.state_in, srow + c * (W - 1) + (W - 1) + pos) : 0.f;
    }
  }
  // the chunk-0 thread writes the new state: it is the only reader of
  // state_in, and it has read what it needs, so state_out may alias state_in
  if (chunk == 0 && a.state_out != nullptr) {
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t pos = L - (W - 1) + j;
      float v[V];
      if (pos >= 0) {
        load_row(pos, v);
      } else {
        // position pos < 0 sits in the initial window at pos + W - 1 (selected with
        // static indices, so the window stays in registers)
#pragma unroll
        for (int c = 0; c < V; ++c) v[c] = 0.f;
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
          if (k == pos + (W - 1))
#pragma unroll
            for (int c = 0; c < V; ++c) v[c] = win[k][c];
      }
#pragma unroll
      for (int c = 0; c < V; ++c) st1<BF16>(a.state_out, srow + c * (W - 1) + j, v[c]);
    }
  }
#pragma unroll 4
  for (int64_t t = t0; t < t1; ++t) {
    load_row(t, win[W - 1]);
    float o[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
      float acc = bs[c];
#pragma unroll
      for (int k = 0; k < W; ++k) acc = fmaf(wt[k][c], win[k][c], acc);
      o[c] = a.silu ? silu_conv(acc) : acc;
    }
    const int64_t i = ((int64_t)b * L + t) * dim + c0;
    if constexpr (V == 8) {
      Vec8<BF16>::store(a.out, i, o);
    } else {
      st1<BF16>(a.out, i, o[0]);
    }
#pragma unroll
    for (int k = 0; k < W - 1; ++k)
#pragma unroll
      for (int c = 0; c < V; ++c) win[k][c] = win[k + 1][c];
  }
}

template <int W>
hipError_t launch_w(const ConvArgs& a, hipStream_t st) {
  const int V = a.vec ? 8 : 1;
  const int64_t cgroups = a.dim / V;
  const int64_t nchunk = a.seqlen > 0 ? (a.seqlen + kConvTokens - 1) / kConvTokens : 1;
  const int64_t threads = a.batch * nchunk * cgroups;
  const dim3 grid((unsigned)((threads + kConvThreads - 1) / kConvThreads));
  if (a.vec) {
    if (a.act_bf16) conv_kernel<W, true, 8><<<grid, kConvThreads, 0, st>>>(a, (unsigned)cgroups, (unsigned)nchunk);
    else conv_kernel<W, false, 8><<<grid, kConvThreads, 0, st>>>(a, (unsigned)cgroups, (unsigned)nchunk);
  } else {
    if (a.act_bf16) conv_kernel<W, true, 1><<<grid, kConvThreads, 0, st>>>(a, (unsigned)cgroups, (unsigned)nchunk);
    else conv_kernel<W, false, 1><<<grid, kConvThreads, 0, st>>>(a, (unsigned)cgroups, (unsigned)nchunk);
  }
  return hipGetLastError();
}

}  // namespace

int launch_conv(const ConvArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (a.batch == 0 || a.dim == 0) return 0;
  const int64_t V = a.vec ? 8 : 1;
  const int64_t nchunk = a.seqlen > 0 ? (a.seqlen + kConvTokens - 1) / kConvTokens : 1;
  if (a.batch * nchunk * (a.dim / V) + kConvThreads > 0xffffffffLL) return fail(4, "grid too large");
  hipError_t e;
  switch (a.width) {
    case 1: e = launch_w<1>(a, st); break;
    case 2: e = launch_w<2>(a, st); break;
    case 3: e = launch_w<3>(a, st); break;
    case 4: e = launch_w<4>(a, st); break;
    case 5: e = launch_w<5>(a, st); break;
    case 6: e = launch_w<6>(a, st); break;
    case 7: e = launch_w<7>(a, st); break;
    case 8: e = launch_w<8>(a, st); break;
    default: return fail(4, "conv width must be 1..8");
  }
  if (e != hipSuccess) return fail(6, std::string("conv1d launch: ") + hipGetErrorString(e));
  return 0;
}

}  // namespace ssm
