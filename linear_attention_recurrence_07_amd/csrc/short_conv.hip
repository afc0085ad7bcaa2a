// Causal short convolution in front of the KDA kernel: one width-W filter per channel
// over the token axis, then SiLU (Kimi-K3 atlas, KDA layer page, kda-init code: a
// ShortConvolution with activation 'silu' on each of the projected queries, keys and
// values; nnterp Kimi-Linear page, module tree: Conv1d with groups = channels, kernel
// size 4, padding 3, no bias).  For channel c and a token t of a sequence
//     z = sum_j w[c][j] * x[t - (W-1) + j][c],     y = z * sigmoid(z)
// with the inputs before a sequence's first token taken from its carried state (the W-1
// inputs that preceded it, oldest first) or zero.  Padding tokens (mask 0) are skipped:
// their output is zero and they never enter the window.
//
// Memory-bound: every input is read once (plus a W-1 token halo per tile) and every
// output written once.  A thread owns 8 consecutive channels (one 16-byte bf16 vector)
// over a tile of 16 tokens of one batch row, so a wave reads 1 KB of one token row per
// load; it rebuilds the window at its tile start from the preceding tokens of the same
// sequence (or the carried state) and then slides it, loading 4 tokens ahead (small tiles
// give many work-groups, which measured faster than deeper loads per thread).  A tile of
// padding only writes zeros and skips the window.  When every row fits one tile (T <= 16,
// no packing: a decode step) the same thread writes the row's
// new carried state after its last token, having read the old one first.  Otherwise a
// second launch writes each sequence's new carried state with the same window rule at the
// sequence end; running after the first launch, it may overwrite the state the first one
// read.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int CPT = 8;          // channels per thread
constexpr int TT = 16;          // tokens per tile
constexpr int NTH = 256;        // threads per work-group
constexpr int PF = 4;           // tokens loaded ahead

typedef float f8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f8 load8(const uint16_t *p) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  return f8{lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y),
            lo_bf16(w.z), hi_bf16(w.z), lo_bf16(w.w), hi_bf16(w.w)};
}
__device__ __forceinline__ f8 load8(const float *p) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  return f8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}
// Inputs as loaded: 8 bf16 in one 16-byte vector (half the registers of fp32), or 8 fp32.
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
template <typename TIn>
struct Raw;
template <>
struct Raw<uint16_t> {
  typedef u4 type;
  __device__ __forceinline__ static type load(const uint16_t *p) { return *reinterpret_cast<const u4 *>(p); }
  __device__ __forceinline__ static f8 cvt(type w) {
    return f8{lo_bf16(w[0]), hi_bf16(w[0]), lo_bf16(w[1]), hi_bf16(w[1]),
              lo_bf16(w[2]), hi_bf16(w[2]), lo_bf16(w[3]), hi_bf16(w[3])};
  }
  __device__ __forceinline__ static type zero() { return u4{0u, 0u, 0u, 0u}; }
};
template <>
struct Raw<float> {
  typedef f8 type;
  __device__ __forceinline__ static type load(const float *p) { return load8(p); }
  __device__ __forceinline__ static f8 cvt(type v) { return v; }
  __device__ __forceinline__ static type zero() { return f8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }
};

__device__ __forceinline__ void store8(uint16_t *p, f8 v) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
  store_nt(p, w);
}
__device__ __forceinline__ void store8(float *p, f8 v) {
  store_nt(p, make_float4(v[0], v[1], v[2], v[3]));
  store_nt(p + 4, make_float4(v[4], v[5], v[6], v[7]));
}

// The sequence of batch row `row` that holds token t: [s, e) and its index n.
struct Seq {
  int n, s, e;
};
__device__ __forceinline__ Seq find_seq(const int32_t *cu, int N, int T, int row, int t) {
  if (!cu) return Seq{row, 0, T};
  int lo = 0, hi = N - 1;            // last n with start(n) <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(cu[mid], 0), T) <= t) lo = mid;
    else hi = mid - 1;
  }
  const int s = min(max(cu[lo], 0), T);
  return Seq{lo, s, max(s, min(cu[lo + 1], T))};
}

// The W-1 inputs that precede token t0 in sequence q (oldest first): the latest
// non-padding tokens in [q.s, t0), then the newest entries of the carried state.
template <typename TIn, int W, bool HAS_MASK>
__device__ __forceinline__ void window_before(typename Raw<TIn>::type (&h)[W - 1], const TIn *xrow, const TIn *init,
                                              const uint8_t *mrow, const Seq &q, int t0, int D, int c0) {
  int found[W - 1];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) found[j] = -1;
  int cnt = 0;
  for (int t = t0 - 1; t >= q.s && cnt < W - 1; --t) {
    if (HAS_MASK && mrow[t] == 0) continue;
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
      if (cnt == j) found[j] = t;      // found[0] is the newest
    ++cnt;
  }
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int slot = W - 2 - j;        // h[slot] takes the j-th newest input
    if (found[j] >= 0) {
      h[slot] = Raw<TIn>::load(xrow + static_cast<size_t>(found[j]) * D + c0);
    } else if (init) {
      // the (j - cnt)-th newest carried input: state slot W-2-(j-cnt)
      h[slot] = Raw<TIn>::load(init + (static_cast<size_t>(q.n) * (W - 1) + (W - 2 - (j - cnt))) * D + c0);
    } else {
      h[slot] = Raw<TIn>::zero();
    }
  }
}

__device__ __forceinline__ void store_state(uint16_t *p, u4 v) { *reinterpret_cast<u4 *>(p) = v; }
__device__ __forceinline__ void store_state(float *p, f8 v) { store8(p, v); }

// FUSED: one tile per row and no packing; the thread also writes the row's carried state
// (init and fin may then be the same buffer: each thread reads its channels' old state
// before writing them).
template <typename TIn, typename TOut, int W, bool HAS_MASK, bool FUSED>
__global__ void __launch_bounds__(NTH)
short_conv_kernel(const TIn *__restrict__ x, const float *__restrict__ w, const TIn *init,
                  const int32_t *__restrict__ cu, const uint8_t *__restrict__ mask, TOut *__restrict__ y,
                  TIn *fin, int T, int D, int N, int silu) {
  const int c0 = (blockIdx.x * NTH + threadIdx.x) * CPT;
  if (c0 >= D) return;
  const int row = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int t1 = min(t0 + TT, T);
  const TIn *xrow = x + static_cast<size_t>(row) * T * D;
  TOut *yrow = y + static_cast<size_t>(row) * T * D;
  const uint8_t *mrow = HAS_MASK ? mask + static_cast<size_t>(row) * T : nullptr;
  float tap[CPT][4];            // right-aligned taps per channel (conv_z)
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    tap[i][0] = tap[i][1] = tap[i][2] = 0.f;
#pragma unroll
    for (int j = 0; j < W; ++j) tap[i][4 - W + j] = w[(c0 + i) * W + j];
  }
  // filter output of the CPT channels for input x after the W-1 inputs hw[0..W-2] (oldest first)
  auto filt = [&](const f8 (&hw)[W - 1], f8 x) {
    f8 z;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float h4[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < W - 1; ++j) h4[4 - W + j] = hw[j][c];
      z[c] = conv_z(tap[c], h4[0], h4[1], h4[2], x[c], W);
      if (silu) z[c] = silu_act(z[c]);
    }
    return z;
  };

  Seq q = find_seq(cu, N, T, row, t0);
  if (t0 >= q.e) {                     // past the last packed sequence: nothing here
    if (!cu || q.n == N - 1) return;
  }
  using R = Raw<TIn>;
  if constexpr (HAS_MASK && !FUSED) {
    // a tile of padding only: zeros, and no window to rebuild (which would scan back
    // over the padded stretch before it)
    bool any = false;
    for (int t = t0; t < t1; ++t) any = any || mrow[t] != 0;
    if (!any) {
      for (int t = t0; t < t1; ++t)
        store8(yrow + static_cast<size_t>(t) * D + c0, f8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f});
      return;
    }
  }
  typename R::type h[W - 1];
  window_before<TIn, W, HAS_MASK>(h, xrow, init, mrow, q, t0, D, c0);

  for (int tb = t0; tb < t1; tb += PF) {
    typename R::type xin[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int t = min(tb + i, t1 - 1);
      xin[i] = R::load(xrow + static_cast<size_t>(t) * D + c0);
    }
    if (!HAS_MASK && tb + PF <= t1 && tb + PF <= q.e) {
      // whole batch inside one sequence, no padding: token i's window is win[i .. i+W-1]
      typename R::type win[W - 1 + PF];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) win[j] = h[j];
#pragma unroll
      for (int i = 0; i < PF; ++i) win[W - 1 + i] = xin[i];
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        f8 hw[W - 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) hw[j] = R::cvt(win[i + j]);
        store8(yrow + static_cast<size_t>(tb + i) * D + c0, filt(hw, R::cvt(win[i + W - 1])));
      }
#pragma unroll
      for (int j = 0; j < W - 1; ++j) h[j] = win[PF + j];
      continue;
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int t = tb + i;
      if (t >= t1) break;
      if (t >= q.e) {                  // next packed sequence (skipping empty ones)
        if (!cu || q.n == N - 1) return;   // tokens after the last sequence stay untouched
        int n = q.n + 1;
        while (n < N - 1 && min(max(cu[n + 1], 0), T) <= t) ++n;
        q = Seq{n, min(max(cu[n], 0), T), max(min(max(cu[n], 0), T), min(cu[n + 1], T))};
        if (t >= q.e) return;
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
          h[j] = init ? R::load(init + (static_cast<size_t>(q.n) * (W - 1) + j) * D + c0) : R::zero();
      }
      f8 out = f8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (!HAS_MASK || mrow[t] != 0) {
        f8 hw[W - 1];
#pragma unroll
        for (int j = 0; j < W - 1; ++j) hw[j] = R::cvt(h[j]);
        out = filt(hw, R::cvt(xin[i]));
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j) h[j] = h[j + 1];
        h[W - 2] = xin[i];
      }
      store8(yrow + static_cast<size_t>(t) * D + c0, out);
    }
  }
  if constexpr (FUSED) {
    if (fin) {
#pragma unroll
      for (int j = 0; j < W - 1; ++j) store_state(fin + (static_cast<size_t>(row) * (W - 1) + j) * D + c0, h[j]);
    }
  }
}

// New carried state of every sequence: the window before its end.
template <typename TIn, int W, bool HAS_MASK>
__global__ void __launch_bounds__(NTH)
short_conv_state_kernel(const TIn *__restrict__ x, const TIn *init, const int32_t *__restrict__ cu,
                        const uint8_t *__restrict__ mask, TIn *fin, int T, int D, int N) {
  const int c0 = (blockIdx.x * NTH + threadIdx.x) * CPT;
  if (c0 >= D) return;
  const int n = blockIdx.y;
  Seq q;
  int row;
  if (cu) {
    const int s = min(max(cu[n], 0), T);
    q = Seq{n, s, max(s, min(cu[n + 1], T))};
    row = 0;
  } else {
    q = Seq{n, 0, T};
    row = n;
  }
  const uint8_t *mrow = HAS_MASK ? mask + static_cast<size_t>(row) * T : nullptr;
  typename Raw<TIn>::type h[W - 1];
  window_before<TIn, W, HAS_MASK>(h, x + static_cast<size_t>(row) * T * D, init, mrow, q, q.e, D, c0);
#pragma unroll
  for (int j = 0; j < W - 1; ++j) store_state(fin + (static_cast<size_t>(n) * (W - 1) + j) * D + c0, h[j]);
}

template <typename TIn, typename TOut, int W>
hipError_t launch3(const ConvArgs &a, hipStream_t st) {
  const TIn *x = static_cast<const TIn *>(a.x);
  const TIn *init = static_cast<const TIn *>(a.init);
  const unsigned gx = static_cast<unsigned>((a.D / CPT + NTH - 1) / NTH);
  TIn *fin = static_cast<TIn *>(a.fin);
  const bool fused = a.T > 0 && a.T <= TT && !a.cu;
  if (a.T > 0) {
    const dim3 grid(gx, static_cast<unsigned>((a.T + TT - 1) / TT), static_cast<unsigned>(a.B));
    if (fused) {
      if (a.mask)
        hipLaunchKernelGGL((short_conv_kernel<TIn, TOut, W, true, true>), grid, dim3(NTH), 0, st, x, a.w, init,
                           a.cu, a.mask, static_cast<TOut *>(a.y), fin, a.T, a.D, a.N, a.silu);
      else
        hipLaunchKernelGGL((short_conv_kernel<TIn, TOut, W, false, true>), grid, dim3(NTH), 0, st, x, a.w, init,
                           a.cu, a.mask, static_cast<TOut *>(a.y), fin, a.T, a.D, a.N, a.silu);
    } else {
      if (a.mask)
        hipLaunchKernelGGL((short_conv_kernel<TIn, TOut, W, true, false>), grid, dim3(NTH), 0, st, x, a.w, init,
                           a.cu, a.mask, static_cast<TOut *>(a.y), fin, a.T, a.D, a.N, a.silu);
      else
        hipLaunchKernelGGL((short_conv_kernel<TIn, TOut, W, false, false>), grid, dim3(NTH), 0, st, x, a.w, init,
                           a.cu, a.mask, static_cast<TOut *>(a.y), fin, a.T, a.D, a.N, a.silu);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.fin && !fused) {
    const dim3 grid(gx, static_cast<unsigned>(a.N));
    if (a.mask)
      hipLaunchKernelGGL((short_conv_state_kernel<TIn, W, true>), grid, dim3(NTH), 0, st, x, init, a.cu, a.mask,
                         fin, a.T, a.D, a.N);
    else
      hipLaunchKernelGGL((short_conv_state_kernel<TIn, W, false>), grid, dim3(NTH), 0, st, x, init, a.cu, a.mask,
                         fin, a.T, a.D, a.N);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TIn, typename TOut>
hipError_t launch2(const ConvArgs &a, hipStream_t st) {
  switch (a.W) {
    case 2: return launch3<TIn, TOut, 2>(a, st);
    case 3: return launch3<TIn, TOut, 3>(a, st);
    default: return launch3<TIn, TOut, 4>(a, st);
  }
}

template <typename TIn, int W>
hipError_t carry3(const Args &a, hipStream_t st) {
  const int D = a.H * a.dk;            // channels of each projection (dk = dv)
  const unsigned gx = static_cast<unsigned>((D / CPT + NTH - 1) / NTH);
  const dim3 grid(gx, static_cast<unsigned>(a.N));
  const void *xs[3] = {a.q, a.k, a.v};
  for (int i = 0; i < 3; ++i) {
    if (a.conv.fin[i] == nullptr) continue;
    const TIn *x = static_cast<const TIn *>(xs[i]);
    const TIn *init = static_cast<const TIn *>(a.conv.init[i]);
    TIn *fin = static_cast<TIn *>(a.conv.fin[i]);
    if (a.mask)
      hipLaunchKernelGGL((short_conv_state_kernel<TIn, W, true>), grid, dim3(NTH), 0, st, x, init, a.cu, a.mask, fin,
                         a.T, D, a.N);
    else
      hipLaunchKernelGGL((short_conv_state_kernel<TIn, W, false>), grid, dim3(NTH), 0, st, x, init, a.cu, a.mask, fin,
                         a.T, D, a.N);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TIn>
hipError_t carry2(const Args &a, hipStream_t st) {
  switch (a.conv.W) {
    case 2: return carry3<TIn, 2>(a, st);
    case 3: return carry3<TIn, 3>(a, st);
    default: return carry3<TIn, 4>(a, st);
  }
}

}  // namespace

hipError_t launch_conv_carry(const Args &a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  return a.in_bf16 ? carry2<uint16_t>(a, st) : carry2<float>(a, st);
}

hipError_t launch_short_conv(const ConvArgs &a, hipStream_t st) {
  if (a.in_bf16)
    return a.out_bf16 ? launch2<uint16_t, uint16_t>(a, st) : launch2<uint16_t, float>(a, st);
  return a.out_bf16 ? launch2<float, uint16_t>(a, st) : launch2<float, float>(a, st);
}

}  // namespace kda
