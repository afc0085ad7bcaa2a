// Chunked KDA prefill on the vector ALUs (any head size up to 128, fp32 or bf16 inputs).
//
// The prompt kernel carries the state from chunk to chunk and never stores it per token
// (nnterp Kimi-Linear page, Notes, "Loading").  Within a chunk of C tokens, with S0 the
// incoming state, G_r = sum_{s<=r} g_s per key channel and k, q normalised:
//     A[s][j]  = beta_s sum_c k_sc k_jc exp(G_sc - G_jc)            (j < s)
//     (I + A) U = diag(beta) (V - (k * exp(G)) S0)                   forward substitution
//     Bqk[r][s] = sum_c q_rc k_sc exp(G_rc - G_sc)                   (s <= r)
//     O = (q * exp(G)) S0 + Bqk U
//     S = diag(exp(G_last)) S0 + (k * exp(G_last - G))^T U
// which equals the token-by-token recurrence up to rounding.  Every exponent above is
// <= 0, so this form accepts any g <= 0.  All arithmetic is fp32; the state lives in LDS.
// This kernel is the exact-precision path (fp32 inputs) and the fallback for head sizes
// the MFMA kernel does not cover; it is not tuned for speed.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kC = 16;     // tokens per chunk
constexpr int kNT = 256;   // threads per work-group

template <int D, typename TIn, typename TOut, bool NORM>
__global__ void __launch_bounds__(kNT)
prefill_valu_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                    const float *__restrict__ g, const float *__restrict__ beta,
                    const float *init, float *fin, const int32_t *__restrict__ cu,
                    const uint8_t *__restrict__ mask, TOut *__restrict__ o,
                    const TIn *__restrict__ gate, const float *__restrict__ norm_w,
                    TOut *__restrict__ y, int T, int H, float scale, int use_l2, float eps, int g_head) {
  constexpr int C = kC;
  __shared__ float sS[D][D];
  __shared__ float sK[C][D], sQ[C][D], sG[C][D], sV[C][D], sU[C][D];
  __shared__ float sKt[C][D], sQt[C][D], sKe[C][D];
  __shared__ float sA[C][C + 1], sB[C][C + 1];
  __shared__ float sBeta[C];

  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int n = unit / H, h = unit % H;
  int b, t_begin, t_end;
  if (cu) {
    b = 0;
    t_begin = cu[n];
    t_end = cu[n + 1];
  } else {
    b = n;
    t_begin = 0;
    t_end = T;
  }
  const size_t slab = (static_cast<size_t>(n) * H + h) * D * D;
  for (int e = tid; e < D * D; e += kNT) sS[e / D][e % D] = init ? init[slab + e] : 0.f;

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int L = min(C, t_end - c0);
    __syncthreads();
    // ---- load the chunk (padding and tokens past the sequence become zeros)
    for (int e = tid; e < C * D; e += kNT) {
      const int r = e / D, col = e % D;
      const int t = c0 + r;
      const bool valid = r < L && (mask == nullptr || mask[static_cast<size_t>(b) * T + t] != 0);
      const size_t idx = ((static_cast<size_t>(b) * T + t) * H + h) * D + col;
      sK[r][col] = valid ? Elem<TIn>::load(k, idx) : 0.f;
      sQ[r][col] = valid ? Elem<TIn>::load(q, idx) : 0.f;
      sG[r][col] = valid ? (g_head ? g[idx / D] : g[idx]) : 0.f;
      sV[r][col] = valid ? Elem<TIn>::load(v, idx) : 0.f;
    }
    if (tid < C) {
      const int t = c0 + tid;
      const bool valid = tid < L && (mask == nullptr || mask[static_cast<size_t>(b) * T + t] != 0);
      sBeta[tid] = valid ? beta[(static_cast<size_t>(b) * T + t) * H + h] : 0.f;
    }
    __syncthreads();
    // ---- L2 norms: 16 threads per token row
    {
      const int r = tid / 16, part = tid % 16;
      float sk = 0.f, sq = 0.f;
      for (int col = part; col < D; col += 16) {
        sk += sK[r][col] * sK[r][col];
        sq += sQ[r][col] * sQ[r][col];
      }
      sk = lane_sum<15>(sk);
      sq = lane_sum<15>(sq);
      const float kn = use_l2 ? rsqrtf(sk + kL2Eps) : 1.f;
      const float qn = (use_l2 ? rsqrtf(sq + kL2Eps) : 1.f) * scale;
      for (int col = part; col < D; col += 16) {
        sK[r][col] *= kn;
        sQ[r][col] *= qn;
      }
    }
    // ---- running decay sums per channel
    if (tid < D) {
      float acc = 0.f;
      for (int r = 0; r < C; ++r) {
        acc += sG[r][tid];
        sG[r][tid] = acc;
      }
    }
    __syncthreads();
    // ---- decayed operands
    for (int e = tid; e < C * D; e += kNT) {
      const int r = e / D, col = e % D;
      const float G = sG[r][col], Gl = sG[C - 1][col];
      sKt[r][col] = sK[r][col] * expf(G);
      sQt[r][col] = sQ[r][col] * expf(G);
      sKe[r][col] = sK[r][col] * expf(Gl - G);
    }
    // ---- intra-chunk products, one (s, j) pair per thread
    {
      const int s = tid / C, j = tid % C;
      float a = 0.f, bq = 0.f;
      if (j <= s) {
        for (int c = 0; c < D; ++c) {
          const float dec = expf(sG[s][c] - sG[j][c]);
          a += sK[s][c] * sK[j][c] * dec;
          bq += sQ[s][c] * sK[j][c] * dec;
        }
      }
      sA[s][j] = (j < s) ? sBeta[s] * a : 0.f;
      sB[s][j] = bq;
    }
    __syncthreads();
    // ---- X = beta (V - Kt S0), in sU
    for (int e = tid; e < C * D; e += kNT) {
      const int r = e / D, col = e % D;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc += sKt[r][i] * sS[i][col];
      sU[r][col] = sBeta[r] * (sV[r][col] - acc);
    }
    __syncthreads();
    // ---- (I + A) U = X by forward substitution; each thread owns value columns
    for (int col = tid; col < D; col += kNT) {
      for (int s = 1; s < C; ++s) {
        float acc = sU[s][col];
        for (int j = 0; j < s; ++j) acc -= sA[s][j] * sU[j][col];
        sU[s][col] = acc;
      }
    }
    __syncthreads();
    // ---- O = Qt S0 + Bqk U, staged in sV
    for (int e = tid; e < C * D; e += kNT) {
      const int r = e / D, col = e % D;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc += sQt[r][i] * sS[i][col];
      for (int s = 0; s <= r; ++s) acc += sB[r][s] * sU[s][col];
      sV[r][col] = acc;
    }
    __syncthreads();
    // ---- state carry
    for (int e = tid; e < D * D; e += kNT) {
      const int i = e / D, col = e % D;
      float acc = expf(sG[C - 1][i]) * sS[i][col];
      for (int s = 0; s < C; ++s) acc += sKe[s][i] * sU[s][col];
      sS[i][col] = acc;
    }
    // ---- outputs (and the gated norm over each token's row)
    {
      const int r = tid / 16, part = tid % 16;
      const int t = c0 + r;
      const size_t base = ((static_cast<size_t>(b) * T + t) * H + h) * D;
      float rn = 0.f;
      if constexpr (NORM) {
        float ss = 0.f;
        for (int col = part; col < D; col += 16) ss += sV[r][col] * sV[r][col];
        ss = lane_sum<15>(ss);
        rn = rsqrtf(ss / D + eps);
      }
      if (r < L) {
        for (int col = part; col < D; col += 16) {
          const float ov = sV[r][col];
          if (o != nullptr) Elem<TOut>::store(o, base + col, ov);   // null: y alone is wanted
          if constexpr (NORM) {
            const float gt = Elem<TIn>::load(gate, base + col);
            Elem<TOut>::store(y, base + col, norm_w[col] * (ov * rn) * sigmoidf_(gt));
          }
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += kNT) fin[slab + e] = sS[e / D][e % D];
}

template <int D, typename TIn, typename TOut>
hipError_t launch_typed(const Args &a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.N) * a.H), block(kNT);
  const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k),
            *v = static_cast<const TIn *>(a.v), *gate = static_cast<const TIn *>(a.gate);
  TOut *o = static_cast<TOut *>(a.o), *y = static_cast<TOut *>(a.y);
  if (a.y)
    hipLaunchKernelGGL((prefill_valu_kernel<D, TIn, TOut, true>), grid, block, 0, st, q, k, v, a.g,
                       a.beta, a.init, a.state, a.cu, a.mask, o, gate, a.norm_w, y, a.T, a.H,
                       a.scale, a.use_l2, a.eps, a.g_head);
  else
    hipLaunchKernelGGL((prefill_valu_kernel<D, TIn, TOut, false>), grid, block, 0, st, q, k, v, a.g,
                       a.beta, a.init, a.state, a.cu, a.mask, o, gate, a.norm_w, y, a.T, a.H,
                       a.scale, a.use_l2, a.eps, a.g_head);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Args &a, hipStream_t st) {
  if (a.in_bf16 && a.out_bf16) return launch_typed<D, uint16_t, uint16_t>(a, st);
  if (a.in_bf16) return launch_typed<D, uint16_t, float>(a, st);
  if (a.out_bf16) return launch_typed<D, float, uint16_t>(a, st);
  return launch_typed<D, float, float>(a, st);
}

}  // namespace

bool prefill_valu_supports(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_prefill_valu(const Args &a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_d<16>(a, st);
    case 32: return launch_d<32>(a, st);
    case 64: return launch_d<64>(a, st);
    case 128: return launch_d<128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
