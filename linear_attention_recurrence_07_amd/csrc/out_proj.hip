// Output projection of the layer: out[r][n] = sum_j y[r][j] * W[n][j] on the CDNA4
// matrix cores (Kimi-K3 atlas, gate-project page: the gated-normed heads [B, 1, 12288]
// enter the output projection, 12,288 -> 7,168 features, no bias).
//
// At decode the rows are few (one per sequence) and the 176 MB weight is read once, so
// the kernel is bound by that stream.  A work-group owns 64 output features and one of S
// slices of K for up to 64 rows; its four waves each stream 16 weight rows straight from
// HBM into registers (loads for the next 256-wide K chunk are in flight while the current
// one is multiplied), and share the rows, which are staged through double-buffered LDS.
// Wave w computes features 16w..16w+15 for all 64 rows (MFMA 16x16x32 bf16, fp32
// accumulation).  With S > 1 each slice writes fp32 partial sums to a workspace and a
// second launch adds the S partials in a fixed order (deterministic results); S = 4 at
// the decode shape gives 448 work-groups, enough loads in flight for the weight stream.
#include <mutex>

#include "kda_chunk.h"
#include "kda_launch.h"

// Scratch of the allocation-free entry point (kda_gated_norm_proj_noalloc): the fp32
// partial sums of the split-K projection live in this file-scope device array instead of
// a caller workspace.  Every GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device address: the
// address is taken once per device with hipGetSymbolAddress (out_proj_static_scratch).
static __device__ __align__(256) uint8_t scratch[kda::kOutProjStaticScratchBytes];

namespace kda {
namespace {
using chunk::u32x4;

constexpr int BM = 64;          // rows per work-group
constexpr int BN = 64;          // output features per work-group (16 per wave)
constexpr int KC = 256;         // K per chunk
constexpr int NTH = 256;
constexpr int LDR = KC + 8;     // LDS row stride (bf16): 16 bytes of padding per row
constexpr int PA = BM * KC / 8 / NTH;   // 16-byte pieces of the row chunk per thread (8)
constexpr int KS = KC / 32;     // MFMA K steps per chunk (8)

__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

// Rows [m0, m0+64) x features [n0, n0+64) over K range [kb, kb + klen).  dst: out (S = 1,
// TOut) or this slice's fp32 partial tile.
template <typename TDst>
__global__ void __launch_bounds__(NTH)
out_proj_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, TDst *__restrict__ dst,
                int M, int N, int K, int klen, size_t slice_stride) {
  __shared__ uint16_t sa[2][BM * LDR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * BN;
  const int slice = blockIdx.y;
  const int m0 = blockIdx.z * BM;
  const int kb = slice * klen;
  const int nchunks = klen / KC;
  TDst *out = dst + slice * slice_stride;

  // this lane's weight row and K offset inside each 32-wide step
  const uint16_t *wrow = w + static_cast<size_t>(n0 + 16 * wave + l16) * K + kb + 8 * lg;
  u32x4 ra[PA], wb[KS];
  auto load = [&](int c) {
    const int k0 = kb + c * KC;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      ra[i] = (m0 + row < M) ? *reinterpret_cast<const u32x4 *>(x + static_cast<size_t>(m0 + row) * K + k0 + col)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) wb[s] = *reinterpret_cast<const u32x4 *>(wrow + c * KC + 32 * s);
    __asm__ volatile("" ::: "memory");
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&sa[buf][row * LDR + col]) = ra[i];
    }
  };

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  stage(0);
  u32x4 wc[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) wc[s] = wb[s];
  sync_lds();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load(c + 1);
    // lane (lg, r): row r of each 16-row tile and K elements 32s + 8lg .. +7, the same
    // K slots as its weight fragment
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&sa[buf][(16 * t + l16) * LDR + 32 * s + 8 * lg]);
        acc[t] = mma(a, wc[s], acc[t]);
      }
    if (c + 1 < nchunks) {
      stage(buf ^ 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) wc[s] = wb[s];
    }
    sync_lds();
  }
  // acc[t][i] = out[m0 + 16t + 4lg + i][n0 + 16 wave + l16]
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * t + 4 * lg + i;
      if (row < M) Elem<TDst>::store(out, static_cast<size_t>(row) * N + n0 + 16 * wave + l16, acc[t][i]);
    }
}

// out = sum over S slices of the fp32 partials, in slice order.
template <typename TOut>
__global__ void __launch_bounds__(NTH)
out_proj_reduce_kernel(const float *__restrict__ part, TOut *__restrict__ out, size_t count, int S) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * NTH + threadIdx.x) * 4;
  if (i >= count) return;
  float4 a = *reinterpret_cast<const float4 *>(part + i);
  for (int s = 1; s < S; ++s) {
    const float4 b = *reinterpret_cast<const float4 *>(part + static_cast<size_t>(s) * count + i);
    a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
  }
  Elem<TOut>::store4(out, i, a);
}

}  // namespace

bool out_proj_supports(int64_t M, int K, int N) {
  return K > 0 && K % KC == 0 && N > 0 && N % BN == 0 && M >= 0 && (M + BM - 1) / BM <= 65535;
}

// K slices: 4 (or 2) when the rows fit one tile and K divides evenly, else 1.
int out_proj_slices(int64_t M, int K) {
  if (M > BM) return 1;
  if (K % (4 * KC) == 0) return 4;
  if (K % (2 * KC) == 0) return 2;
  return 1;
}

size_t out_proj_workspace_bytes(int64_t M, int K, int N) {
  const int S = out_proj_slices(M, K);
  return S > 1 ? static_cast<size_t>(S) * static_cast<size_t>(M) * N * sizeof(float) : 0;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t out_proj_static_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_out_proj(const void *x, const void *w, void *out, int64_t M, int K, int N, int out_bf16,
                           void *ws, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int S = out_proj_slices(M, K);
  const dim3 grid(static_cast<unsigned>(N / BN), static_cast<unsigned>(S), static_cast<unsigned>((M + BM - 1) / BM));
  const uint16_t *xx = static_cast<const uint16_t *>(x), *ww = static_cast<const uint16_t *>(w);
  const int klen = K / S;
  if (S == 1) {
    if (out_bf16)
      hipLaunchKernelGGL((out_proj_kernel<uint16_t>), grid, dim3(NTH), 0, st, xx, ww, static_cast<uint16_t *>(out),
                         static_cast<int>(M), N, K, klen, size_t(0));
    else
      hipLaunchKernelGGL((out_proj_kernel<float>), grid, dim3(NTH), 0, st, xx, ww, static_cast<float *>(out),
                         static_cast<int>(M), N, K, klen, size_t(0));
    return hipGetLastError();
  }
  float *part = static_cast<float *>(ws);
  const size_t count = static_cast<size_t>(M) * N;
  hipLaunchKernelGGL((out_proj_kernel<float>), grid, dim3(NTH), 0, st, xx, ww, part, static_cast<int>(M), N, K,
                     klen, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rb = static_cast<unsigned>((count / 4 + NTH - 1) / NTH);
  if (out_bf16)
    hipLaunchKernelGGL((out_proj_reduce_kernel<uint16_t>), dim3(rb), dim3(NTH), 0, st, part,
                       static_cast<uint16_t *>(out), count, S);
  else
    hipLaunchKernelGGL((out_proj_reduce_kernel<float>), dim3(rb), dim3(NTH), 0, st, part, static_cast<float *>(out),
                       count, S);
  return hipGetLastError();
}

}  // namespace kda
