// Per-token states of the bf16 chunked prefill (head size 128, 32-token chunks).
//
// The pages read the state after every token of a prompt (nnterp Kimi-Linear page,
// support() table, the 'states' row [batch, seq, heads, key_dim, value_dim]; Notes,
// "Loading").  Unrolled over one chunk, the recurrence is
//     S_t = diag(exp(g_t)) S_{t-1} + k^_t u_t^T,    u_t = beta_t (v_t - (diag(exp(g_t)) S_{t-1})^T k^_t)
// where the u_t of a chunk are exactly the rows of U that the state scan forms from the
// chunk's incoming state (U = W (V - (k^ exp(G)) S0)).  The scan therefore stores U of every
// chunk in the workspace and the state after the chunk's last position in the states
// tensor; this kernel then fills the chunk's other positions from the state before the
// chunk by the rank-one updates above.  Nothing in it is sequential across chunks: every
// (chunk, head, band of state rows) is an independent work-group, and the work is
// a plain stream of stores, 64 KB per token and head, so the kernel runs at the HBM write
// rate rather than at the token-by-token kernel's per-token latency.
//
// Work-group: NT threads own an RB x 128 band of the state (F4 float4 each, rows
// tid / 32 + RPS i, columns 4 (tid % 32) ..), so each token's band is one contiguous
// store of RB x 512 bytes.  Before the token loop the band's decays exp(g), the
// normalised keys (the L2 norm over all 128 channels, as the preparation forms it) and the
// chunk's U rows are staged in LDS; a padding token gets decay 1 and key 0 (its state is
// the carried one).
//
// Measured at T = 256 and 96 heads (the whole call): the whole state per work-group
// (RB = 128, 512 threads, 768 work-groups, all resident at once) 318 us; 32-row bands
// with 256 threads (3,072 work-groups) 339 us; 64- and 16-row bands slower; ordinary
// stores instead of non-temporal ones slower; splitting a chunk's positions over several
// work-groups that replay the earlier updates 329-386 us; one work-group per (sequence,
// head, 16-row band) walking every chunk in order, so that the stores sweep the tensor
// from start to end, 354 us.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int NT = 512;
constexpr int RB = 128;           // state rows (key channels) per work-group
constexpr int NRB = DK / RB;      // bands per (chunk, head)
constexpr int RPS = NT / 32;      // rows one store instruction of the work-group covers
constexpr int F4 = RB / RPS;      // float4 of the band per thread
static_assert(RB % RPS == 0 && (C * RB) % NT == 0 && (C * DV / 4) % NT == 0, "thread mappings");

template <bool HAS_INIT, bool HAS_MASK, bool G_HEAD>
__global__ void __launch_bounds__(NT)
chunk_states_kernel(const uint16_t *__restrict__ k, const float *__restrict__ g, const int32_t *__restrict__ cu,
                    const uint8_t *__restrict__ mask, const float *__restrict__ init, const float *__restrict__ uws,
                    float *states, int T, int H, int N, int use_l2) {
  __shared__ float4 s_u[C][DV / 4];    // u of the chunk's positions
  __shared__ float s_a[C][RB];         // exp(g) of the band's rows
  __shared__ float s_k[C][RB];         // k^ of the band's rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int band = static_cast<int>(blockIdx.x) % NRB;
  const int slot = static_cast<int>(blockIdx.x) / NRB;
  const int h = blockIdx.y;

  // ---------------------------------------------------------------- locate the chunk
  // (the slot numbering of the preparation and the scan)
  int b, t_begin, t_end, c, nseq;
  if (cu) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (mid + min(max(cu[mid], 0), T) / C <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = 0;
    t_end = min(cu[lo + 1], T);
    t_begin = max(0, min(cu[lo], t_end));
    c = slot - (lo + min(max(cu[lo], 0), T) / C);
    nseq = lo;
  } else {
    const int nch = (T + C - 1) / C;
    b = slot / nch;
    c = slot - b * nch;
    t_begin = 0;
    t_end = T;
    nseq = b;
  }
  if (c < 0 || c * C >= t_end - t_begin) return;   // no chunk in this slot
  const int t0 = t_begin + c * C;
  const int m = min(t0 + C, t_end) - 1 - t0;       // positions before the chunk's last (the scan writes that one)
  if (m <= 0) return;
  const size_t row0 = static_cast<size_t>(b) * T;
  const size_t st_tok = static_cast<size_t>(H) * DK * DV;   // floats between the states of two tokens
  const int r0 = band * RB;

  // ---------------------------------------------------------------- state before the chunk
  // c = 0: the initial state (or zeros); otherwise the state the scan stored at the previous
  // chunk's last position t0 - 1.
  const int col = 4 * (tid & 31);
  const int rr = tid >> 5;                          // rows rr + RPS i of the band
  float4 S[F4];
  {
    const float *src = nullptr;
    if (c > 0) src = states + (row0 + t0 - 1) * st_tok + static_cast<size_t>(h) * DK * DV;
    else if (HAS_INIT) src = init + (static_cast<size_t>(nseq) * H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < F4; ++i)
      S[i] = src ? *reinterpret_cast<const float4 *>(src + static_cast<size_t>(r0 + rr + RPS * i) * DV + col)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // ---------------------------------------------------------------- stage u, exp(g), k^
  {
    const float4 *up = reinterpret_cast<const float4 *>(uws + (static_cast<size_t>(slot) * H + h) * C * DV);
#pragma unroll
    for (int i = 0; i < C * DV / 4 / NT; ++i) {
      const int f = tid + NT * i, j = f >> 5;
      if (j < m) s_u[j][f & 31] = up[f];
    }
  }
#pragma unroll
  for (int i = 0; i < C * RB / NT; ++i) {
    const int f = tid + NT * i, j = f / RB, r = f % RB;
    if (j < m) {
      const size_t tok = row0 + t0 + j;
      const float gv = G_HEAD ? g[tok * H + h] : g[(tok * H + h) * DK + r0 + r];
      const bool real = !HAS_MASK || mask[tok] != 0;
      s_a[j][r] = real ? __expf(gv) : 1.f;
    }
  }
  // keys: wave w normalises positions w, w + 4, ...; lane l holds channels 2l, 2l + 1
  for (int j = wave; j < m; j += NT / 64) {
    const size_t tok = row0 + t0 + j;
    const uint32_t kw = reinterpret_cast<const uint32_t *>(k + (tok * H + h) * DK)[lane];
    const float k0 = lo_bf16(kw), k1 = hi_bf16(kw);
    float nk = 1.f;
    if (use_l2) nk = rsqrtf(wave_sum(k0 * k0 + k1 * k1) + kL2Eps);
    if (HAS_MASK && mask[tok] == 0) nk = 0.f;
    const int ch = 2 * lane - r0;
    if (ch >= 0 && ch < RB) {
      s_k[j][ch] = k0 * nk;
      s_k[j][ch + 1] = k1 * nk;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- the chunk's positions
  float *dst = states + (row0 + t0) * st_tok + static_cast<size_t>(h) * DK * DV + static_cast<size_t>(r0) * DV + col;
  for (int j = 0; j < m; ++j) {
    const float4 u = s_u[j][tid & 31];
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      const float a = s_a[j][rr + RPS * i], kk = s_k[j][rr + RPS * i];
      S[i].x = __builtin_fmaf(kk, u.x, a * S[i].x);
      S[i].y = __builtin_fmaf(kk, u.y, a * S[i].y);
      S[i].z = __builtin_fmaf(kk, u.z, a * S[i].z);
      S[i].w = __builtin_fmaf(kk, u.w, a * S[i].w);
      store_nt(dst + static_cast<size_t>(rr + RPS * i) * DV, S[i]);
    }
    dst += st_tok;
  }
}

}  // namespace

size_t chunk_states_u_bytes(long long B, long long T, long long H, long long N, bool packed) {
  return static_cast<size_t>(num_slots(B, T, N, packed) * H) * C * DV * sizeof(float);
}

float *chunk_states_u_area(const void *ws, long long B, long long T, long long H, long long N, bool packed) {
  return reinterpret_cast<float *>(static_cast<uint8_t *>(const_cast<void *>(ws)) +
                                   chunk_prep_workspace_bytes(B, T, H, N, packed));
}

hipError_t launch_chunk_states(const Args &a, const void *ws, hipStream_t st) {
  const bool packed = a.cu != nullptr;
  const long long slots = num_slots(a.B, a.T, a.N, packed);
  if (slots * a.H <= 0) return hipSuccess;
  const float *uws = chunk_states_u_area(ws, a.B, a.T, a.H, a.N, packed);
  const dim3 grid(static_cast<unsigned>(slots * NRB), static_cast<unsigned>(a.H));
  auto go = [&](auto init_t, auto mask_t, auto ghead_t) {
    hipLaunchKernelGGL((chunk_states_kernel<decltype(init_t)::value, decltype(mask_t)::value,
                                            decltype(ghead_t)::value>),
                       grid, dim3(NT), 0, st, static_cast<const uint16_t *>(a.k), a.g, a.cu, a.mask, a.init, uws,
                       a.states_out, a.T, a.H, a.N, a.use_l2);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto go2 = [&](auto init_t, auto mask_t) {
    if (a.g_head) go(init_t, mask_t, T_{});
    else go(init_t, mask_t, F_{});
  };
  auto go1 = [&](auto init_t) {
    if (a.mask) go2(init_t, T_{});
    else go2(init_t, F_{});
  };
  if (a.init) go1(T_{});
  else go1(F_{});
  return hipGetLastError();
}

}  // namespace kda
