// Output projection of the layer: out[r][n] = sum_j y[r][j] * W[n][j] on the CDNA4
// matrix cores (Kimi-K3 atlas, gate-project page: the gated-normed heads [B, 1, 12288]
// enter the output projection, 12,288 -> 7,168 features, no bias).
//
// At decode the rows are few (one per sequence) and the 176 MB weight is read once, so
// the kernel is bound by that stream: a work-group owns 32 output features over the full
// K for up to 64 rows (224 work-groups at N = 7168), and stages the rows and its weight
// slice through double-buffered LDS in 256-wide K chunks while the matrix cores work on
// the previous chunk.  Wave w multiplies rows 16w..16w+15 against both 16-feature halves
// (MFMA 16x16x32 bf16, fp32 accumulation).  Larger row counts tile over a grid axis.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using chunk::u32x4;

constexpr int BM = 64;          // rows per work-group
constexpr int BN = 32;          // output features per work-group
constexpr int KC = 256;         // K per LDS chunk
constexpr int NTH = 256;
constexpr int LDR = KC + 8;     // LDS row stride (bf16): 16 bytes of padding per row
constexpr int PA = BM * KC / 8 / NTH;   // 16-byte pieces of the row chunk per thread (8)
constexpr int PB = BN * KC / 8 / NTH;   // pieces of the weight chunk per thread (4)

struct Smem {
  uint16_t a[2][BM * LDR];
  uint16_t b[2][BN * LDR];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS");

__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
}

template <typename TOut>
__global__ void __launch_bounds__(NTH)
out_proj_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, TOut *__restrict__ out,
                int M, int N, int K) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int nchunks = K / KC;

  u32x4 ra[PA], rb[PB];
  auto load = [&](int c) {
    const int k0 = c * KC;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      ra[i] = (m0 + row < M) ? *reinterpret_cast<const u32x4 *>(x + static_cast<size_t>(m0 + row) * K + k0 + col)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      rb[i] = *reinterpret_cast<const u32x4 *>(w + static_cast<size_t>(n0 + row) * K + k0 + col);
    }
    __asm__ volatile("" ::: "memory");
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&sm.a[buf][row * LDR + col]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tid + NTH * i, row = p / (KC / 8), col = (p % (KC / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&sm.b[buf][row * LDR + col]) = rb[i];
    }
  };

  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  load(0);
  stage(0);
  sync_lds();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load(c + 1);
    // lane (lg, r): row r of the tile, K elements 32s + 8lg .. +7 (the same K slots on
    // both operands)
    const uint16_t *pa = &sm.a[buf][(16 * wave + l16) * LDR + 8 * lg];
    const uint16_t *pb0 = &sm.b[buf][l16 * LDR + 8 * lg];
    const uint16_t *pb1 = &sm.b[buf][(16 + l16) * LDR + 8 * lg];
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      const u32x4 a = *reinterpret_cast<const u32x4 *>(pa + 32 * s);
      acc[0] = mma(a, *reinterpret_cast<const u32x4 *>(pb0 + 32 * s), acc[0]);
      acc[1] = mma(a, *reinterpret_cast<const u32x4 *>(pb1 + 32 * s), acc[1]);
    }
    if (c + 1 < nchunks) stage(buf ^ 1);
    sync_lds();
  }
  // acc[t][i] = out[m0 + 16 wave + 4 lg + i][n0 + 16 t + l16]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * wave + 4 * lg + i;
      if (row < M) Elem<TOut>::store(out, static_cast<size_t>(row) * N + n0 + 16 * t + l16, acc[t][i]);
    }
}

}  // namespace

bool out_proj_supports(int64_t M, int K, int N) {
  return K > 0 && K % KC == 0 && N > 0 && N % BN == 0 && M >= 0 && (M + BM - 1) / BM <= 65535;
}

hipError_t launch_out_proj(const void *x, const void *w, void *out, int64_t M, int K, int N, int out_bf16,
                           hipStream_t st) {
  if (M == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(N / BN), static_cast<unsigned>((M + BM - 1) / BM));
  const uint16_t *xx = static_cast<const uint16_t *>(x), *ww = static_cast<const uint16_t *>(w);
  if (out_bf16)
    hipLaunchKernelGGL((out_proj_kernel<uint16_t>), grid, dim3(NTH), 0, st, xx, ww, static_cast<uint16_t *>(out),
                       static_cast<int>(M), N, K);
  else
    hipLaunchKernelGGL((out_proj_kernel<float>), grid, dim3(NTH), 0, st, xx, ww, static_cast<float *>(out),
                       static_cast<int>(M), N, K);
  return hipGetLastError();
}

}  // namespace kda
