// Sigmoid-gated RMSNorm over one head's features:
//     y = w * x / sqrt(mean(x^2) + eps) * sigmoid(gate)
// (Kimi-K3 atlas, dense KDA layers / attention / gate-project page: o_norm is a fused
// gated RMSNorm with sigmoid activation over head_dim features, and its Parameters
// table gives it one head_dim weight).  Normalise first, then apply the weight and the
// gate.  HBM-bound: 3 x width elements move per row; each thread takes 8 consecutive
// features (one 16-byte bf16 load), a row is spread over width/8 lanes and reduced with
// cross-lane adds.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t *p, float (&x)[8]) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x); x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
    x[4] = lo_bf16(w.z); x[5] = hi_bf16(w.z); x[6] = lo_bf16(w.w); x[7] = hi_bf16(w.w);
  }
  __device__ __forceinline__ static void store(uint16_t *p, const float (&x)[8]) {
    uint4 w;
    w.x = pack_bf16x2(x[0], x[1]); w.y = pack_bf16x2(x[2], x[3]);
    w.z = pack_bf16x2(x[4], x[5]); w.w = pack_bf16x2(x[6], x[7]);
    store_nt(p, w);
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void store(float *p, const float (&x)[8]) {
    store_nt(p, make_float4(x[0], x[1], x[2], x[3]));
    store_nt(p + 4, make_float4(x[4], x[5], x[6], x[7]));
  }
};

constexpr int kThreads = 256;

template <int W, typename TX, typename TG, typename TOut>
__global__ void __launch_bounds__(kThreads)
gated_rmsnorm_kernel(const TX *x, const TG *__restrict__ gate,
                     const float *__restrict__ w, TOut *y, int64_t rows, float eps,
                     const int32_t *__restrict__ tok_end, int heads) {
  constexpr int LPR = W / 8;                 // lanes per row
  constexpr int RPB = kThreads / LPR;        // rows per block
  static_assert(LPR >= 1 && LPR <= 64, "width");
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / LPR;
  if (row >= rows) return;                   // whole rows drop out together
  // packed sequences: rows of tokens at or past the end of the last sequence are not touched
  if (tok_end != nullptr && row / heads >= static_cast<int64_t>(*tok_end)) return;
  const int c0 = (tid % LPR) * 8;
  const size_t base = static_cast<size_t>(row) * W + c0;
  float xv[8], gv[8];
  Vec8<TX>::load(x + base, xv);
  Vec8<TG>::load(gate + base, gv);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
  ss = lane_sum<LPR - 1>(ss);
  const float rn = rsqrtf(ss / W + eps);
  const float4 w0 = *reinterpret_cast<const float4 *>(w + c0);
  const float4 w1 = *reinterpret_cast<const float4 *>(w + c0 + 4);
  const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float yv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) yv[i] = wv[i] * (xv[i] * rn) * sigmoidf_(gv[i]);
  Vec8<TOut>::store(y + base, yv);
}

template <int W, typename TX, typename TG, typename TOut>
hipError_t launch_w(const void *x, const void *gate, const float *w, void *y, int64_t rows,
                    float eps, const int32_t *tok_end, int heads, hipStream_t st) {
  constexpr int RPB = kThreads / (W / 8);
  const int64_t blocks = (rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((gated_rmsnorm_kernel<W, TX, TG, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, st, static_cast<const TX *>(x),
                     static_cast<const TG *>(gate), w, static_cast<TOut *>(y), rows, eps, tok_end, heads);
  return hipGetLastError();
}

template <typename TX, typename TG, typename TOut>
hipError_t launch_t(const void *x, const void *gate, const float *w, void *y, int64_t rows,
                    int width, float eps, const int32_t *tok_end, int heads, hipStream_t st) {
  switch (width) {
    case 8: return launch_w<8, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 16: return launch_w<16, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 32: return launch_w<32, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 64: return launch_w<64, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 128: return launch_w<128, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 256: return launch_w<256, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    case 512: return launch_w<512, TX, TG, TOut>(x, gate, w, y, rows, eps, tok_end, heads, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gated_rmsnorm(const void *x, const void *gate, const float *w, void *y,
                                int64_t rows, int width, float eps, int x_bf16, int gate_bf16,
                                int out_bf16, hipStream_t st, const int32_t *tok_end, int heads) {
  using B = uint16_t;
  using F = float;
  const int code = (x_bf16 ? 4 : 0) | (gate_bf16 ? 2 : 0) | (out_bf16 ? 1 : 0);
  switch (code) {
    case 7: return launch_t<B, B, B>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 6: return launch_t<B, B, F>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 5: return launch_t<B, F, B>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 4: return launch_t<B, F, F>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 3: return launch_t<F, B, B>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 2: return launch_t<F, B, F>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    case 1: return launch_t<F, F, B>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
    default: return launch_t<F, F, F>(x, gate, w, y, rows, width, eps, tok_end, heads, st);
  }
}

}  // namespace kda
