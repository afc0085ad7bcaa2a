// State scan of the bf16 chunked prefill on the CDNA4 matrix cores (head size 128,
// 32-token chunks), with the sigmoid-gated RMSNorm fused into its output stage.
//
// The prompt kernel of the KDA recurrence carries the state from chunk to chunk (nnterp
// Kimi-Linear page, Notes, "Loading" and the KDA paragraph; section 04 docstring).  With
// S0 the incoming state, G the running sum of g over the chunk per key channel, and the
// chunk's record from the preparation kernel (kda_chunk.h):
//     U      = W (V - (k^ exp(G)) S0)
//     O      = (q^ exp(G)) S0 + Bqk U
//     S_next = diag(exp(G_last)) S0 + (k^ exp(G_last - G))^T U
// which is the token-by-token recurrence regrouped; it equals it up to rounding.  Then,
// per token and head (Kimi-K3 atlas, gate-project page, o_norm):
//     y = w * O / sqrt(mean(O^2) + eps) * sigmoid(gate)
//
// Work decomposition.  One work-group per (sequence, head) with eight waves, two per SIMD;
// wave w owns value columns 16w..16w+15 and keeps its 128 x 16 slice of the fp32 state in
// registers for the whole sequence.  Each step:
//   - stores the record and value tile of chunk c+1 (loaded two steps earlier into
//     registers) into the other half of a double-buffered LDS hand-over area, and issues
//     the loads of chunk c+3;
//   - runs chunk c's products on MFMA, the record's operands read straight from LDS in
//     fragment order (16-byte reads, no bank conflicts);
//   - writes chunk c's output tile to one of two LDS staging buffers and emits chunk c-1's
//     rows (norm, gate) from the other;
//   - ends with the one work-group barrier of the step.
//
// Precision: fp16 operands for the state, the decayed keys/queries and V - K S0; W and U
// as fp16 hi + lo parts; fp32 accumulation.  The fp16 state operand limits |S| to well
// inside fp16 range.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int NW = 8;             // waves per work-group; wave w owns columns 16w..16w+15
constexpr int NT = NW * 64;       // 512 threads
constexpr int LDV = DV + 8;       // value tile row stride (bf16)
constexpr int LDO = DV + 4;       // fp32 output staging row stride
constexpr int REC_PIECES = static_cast<int>(sizeof(Rec) / 16);
constexpr int PPT = (REC_PIECES + NT - 1) / NT;   // record pieces per thread (4)

struct alignas(16) Hand {
  Rec rec;
  uint16_t vt[C * LDV];        // bf16 value tile [token][column]
};
struct alignas(16) Smem {
  Hand hand[2];
  float ost[2][C * LDO];       // fp32 output tiles
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");
static_assert(sizeof(Hand) % 16 == 0 && (LDV * 2) % 16 == 0, "16-byte LDS stores");

__device__ __forceinline__ float sigmoid_fast(float x) {
  return __builtin_amdgcn_rcpf(1.f + fast_exp2(-x * kLog2e));
}

template <typename TOut, bool HAS_INIT, bool NORM>
__global__ void __launch_bounds__(NT, 1)
chunk_scan_kernel(const uint16_t *__restrict__ v, const Rec *__restrict__ ws, const float *init,
                  float *fin, const int32_t *__restrict__ cu, TOut *__restrict__ o,
                  const uint16_t *__restrict__ gate, const float *__restrict__ nw,
                  TOut *__restrict__ y, float eps, int T, int H, int units) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches stay scalar
  const int l16 = lane & 15, lg = lane >> 4;

  const int unit = blockIdx.x;
  if (unit >= units) return;
  const int n = unit / H, h = unit % H;
  int b, t_begin, t_end;
  long long slot0;
  if (cu) {
    b = 0;
    t_end = min(cu[n + 1], T);
    t_begin = max(0, min(cu[n], t_end));
    slot0 = packed_slot_base(n, t_begin);
  } else {
    b = n;
    t_begin = 0;
    t_end = T;
    slot0 = static_cast<long long>(n) * chunks_per_row(T);
  }
  const size_t slab = (static_cast<size_t>(n) * H + h) * DK * DV;
  const int nchunks = (t_end - t_begin + C - 1) / C;
  const size_t row0 = static_cast<size_t>(b) * T;              // first token row of this batch row
  const size_t tok_stride = static_cast<size_t>(H) * DV;       // elements between tokens (v, o, gate)
  // this thread's 8-column piece of a token row: token tid/16, columns (tid%16)*8
  const size_t piece = row0 * tok_stride + static_cast<size_t>(h) * DV + (tid & 15) * 8;
  const Rec *rp0 = ws + slot0 * H + h;                         // chunk c's record: rp0 + c * H
  const int wcol = 16 * wave + l16;                            // this lane's value column

  // ---------------------------------------------------------------- prefetch registers
  // Two sets, so a chunk's record and values are loaded two steps before they are staged.
  struct Pre {
    u32x4 r[PPT];
    u32x4 v;
  };
  Pre pre0, pre1;
  auto load = [&](Pre &pf, int cidx) {
    const u32x4 *rp = reinterpret_cast<const u32x4 *>(rp0 + static_cast<size_t>(cidx) * H);
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (i < PPT - 1 || tid + NT * i < REC_PIECES) pf.r[i] = rp[tid + NT * i];
    const int tv = min(t_begin + cidx * C + (tid >> 4), t_end - 1);
    pf.v = *reinterpret_cast<const u32x4 *>(v + piece + tv * tok_stride);
    __asm__ volatile("" ::: "memory");   // keep the loads here, ahead of their use
  };
  auto stage = [&](Hand &hd, const Pre &pf) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(&hd.rec);
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (i < PPT - 1 || tid + NT * i < REC_PIECES) dst[tid + NT * i] = pf.r[i];
    *reinterpret_cast<u32x4 *>(hd.vt + (tid >> 4) * LDV + (tid & 15) * 8) = pf.v;
  };
  auto load_gate = [&](int cidx) -> u32x4 {
    const int tv = min(t_begin + cidx * C + (tid >> 4), t_end - 1);
    const u32x4 gv = *reinterpret_cast<const u32x4 *>(gate + piece + tv * tok_stride);
    __asm__ volatile("" ::: "memory");
    return gv;
  };

  // ---------------------------------------------------------------- state
  f32x4 Sacc[DK / 16];                           // Sacc[t][i] = S[16t + 4lg + i][wcol]
#pragma unroll
  for (int t = 0; t < DK / 16; ++t) Sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (HAS_INIT) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[t][i] = init[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + wcol];
  }
  float wv[8];                                   // norm weight of this thread's 8 columns
  if (NORM) {
    const float4 w0 = *reinterpret_cast<const float4 *>(nw + (tid & 15) * 8);
    const float4 w1 = *reinterpret_cast<const float4 *>(nw + (tid & 15) * 8 + 4);
    wv[0] = w0.x; wv[1] = w0.y; wv[2] = w0.z; wv[3] = w0.w;
    wv[4] = w1.x; wv[5] = w1.y; wv[6] = w1.z; wv[7] = w1.w;
  }

  // ================================================================ products of one chunk
  auto products = [&](const Hand &hc, float *ost) {
    const u32x4 *KB = reinterpret_cast<const u32x4 *>(hc.rec.kb);
    const u32x4 *QT = reinterpret_cast<const u32x4 *>(hc.rec.qt);
    const u32x4 *KE = reinterpret_cast<const u32x4 *>(hc.rec.ket);
    const u32x4 *BQ = reinterpret_cast<const u32x4 *>(hc.rec.bq);
    const uint32_t valid = hc.rec.valid;
    // S0 as fp16 B operands; K step s covers channels {32s+4lg+0..3, 32s+16+4lg+0..3}
    uint4 Sh[DK / 32];
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const f32x4 a = Sacc[2 * s], bb = Sacc[2 * s + 1];
      Sh[s] = join(pack_f16x4(a[0], a[1], a[2], a[3]), pack_f16x4(bb[0], bb[1], bb[2], bb[3]));
    }
    // Y = V - (k^ exp(G)) S0 in fp16 (W carries the extra precision)
    uint2 yf[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s)
        acc = mfma_f16(__builtin_bit_cast(uint4, KB[(4 * m + s) * 64 + lane]), Sh[s], acc);
      f32x4 yy;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = SB * m + 4 * lg + i;
        // values of padding and of tokens past the end are zeroed (branch-free)
        const uint32_t keep = 0u - ((valid >> r) & 1u);
        yy[i] = __uint_as_float((static_cast<uint32_t>(hc.vt[r * LDV + wcol]) << 16) & keep) - acc[i];
      }
      yf[m] = pack_f16x4(yy[0], yy[1], yy[2], yy[3]);
    }
    // U0 = W00 Y0, U1 = W10 Y0 + W11 Y1, with W as hi + lo parts
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint2 w00 = __builtin_bit_cast(uint2, reinterpret_cast<const u32x2 *>(hc.rec.w00)[lane]);
    const uint2 w00l = __builtin_bit_cast(uint2, reinterpret_cast<const u32x2 *>(hc.rec.w00lo)[lane]);
    f32x4 U0 = mfma_f16k16(w00l, yf[0], zero);
    U0 = mfma_f16k16(w00, yf[0], U0);
    const uint4 w1 = __builtin_bit_cast(uint4, reinterpret_cast<const u32x4 *>(hc.rec.w1)[lane]);
    const uint4 w1l = __builtin_bit_cast(uint4, reinterpret_cast<const u32x4 *>(hc.rec.w1lo)[lane]);
    const uint4 y01 = join(yf[0], yf[1]);
    f32x4 U1 = mfma_f16(w1l, y01, zero);
    U1 = mfma_f16(w1, y01, U1);
    uint2 u0h, u0l, u1h, u1l;
    split_f16x4(U0, u0h, u0l);
    split_f16x4(U1, u1h, u1l);
    const uint4 Uh = join(u0h, u1h);   // tokens {4lg+0..3, 16+4lg+0..3} as K=32 B operands
    const uint4 Ul = join(u0l, u1l);
    // O = (q^ exp(G)) S0 + Bqk U
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s)
        acc = mfma_f16(__builtin_bit_cast(uint4, QT[(4 * m + s) * 64 + lane]), Sh[s], acc);
      const uint4 bqv = __builtin_bit_cast(uint4, BQ[m * 64 + lane]);
      acc = mfma_f16(bqv, Ul, acc);
      acc = mfma_f16(bqv, Uh, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) ost[(SB * m + 4 * lg + i) * LDO + wcol] = acc[i];
    }
    // S = diag(exp(G_last)) S0 + (k^ exp(G_last - G))^T U
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      const float4 e = *reinterpret_cast<const float4 *>(hc.rec.ec + 16 * t + 4 * lg);
      Sacc[t][0] *= e.x; Sacc[t][1] *= e.y; Sacc[t][2] *= e.z; Sacc[t][3] *= e.w;
      const uint4 kv = __builtin_bit_cast(uint4, KE[t * 64 + lane]);
      Sacc[t] = mfma_f16(kv, Ul, Sacc[t]);
      Sacc[t] = mfma_f16(kv, Uh, Sacc[t]);
    }
  };

  // ================================================================ output rows
  // Token tid/16 of chunk cidx, columns (tid%16)*8..+7: head output, and the gated norm
  // over the row (the 16 lanes of a row are one DPP row).
  auto emit = [&](int cidx, const float *ost, u32x4 gv) {
    const int r = tid >> 4, c8 = (tid & 15) * 8;
    const int t = t_begin + cidx * C + r;
    const float4 x0 = *reinterpret_cast<const float4 *>(ost + r * LDO + c8);
    const float4 x1 = *reinterpret_cast<const float4 *>(ost + r * LDO + c8 + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float yv[8];
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += xv[i] * xv[i];
      ss = row_sum16(ss);
      const float rn = rsqrtf(ss * (1.f / DV) + eps);
      const float gf[8] = {lo_bf16(gv[0]), hi_bf16(gv[0]), lo_bf16(gv[1]), hi_bf16(gv[1]),
                           lo_bf16(gv[2]), hi_bf16(gv[2]), lo_bf16(gv[3]), hi_bf16(gv[3])};
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[i] = wv[i] * (xv[i] * rn) * sigmoid_fast(gf[i]);
    }
    if (t < t_end) {
      const size_t off = piece + static_cast<size_t>(t) * tok_stride;
      if constexpr (sizeof(TOut) == 2) {
        uint4 w;
        w.x = pack_bf16x2(xv[0], xv[1]); w.y = pack_bf16x2(xv[2], xv[3]);
        w.z = pack_bf16x2(xv[4], xv[5]); w.w = pack_bf16x2(xv[6], xv[7]);
        *reinterpret_cast<uint4 *>(o + off) = w;
        if (NORM) {
          w.x = pack_bf16x2(yv[0], yv[1]); w.y = pack_bf16x2(yv[2], yv[3]);
          w.z = pack_bf16x2(yv[4], yv[5]); w.w = pack_bf16x2(yv[6], yv[7]);
          *reinterpret_cast<uint4 *>(y + off) = w;
        }
      } else {
        reinterpret_cast<float4 *>(o + off)[0] = x0;
        reinterpret_cast<float4 *>(o + off)[1] = x1;
        if (NORM) {
          reinterpret_cast<float4 *>(y + off)[0] = make_float4(yv[0], yv[1], yv[2], yv[3]);
          reinterpret_cast<float4 *>(y + off)[1] = make_float4(yv[4], yv[5], yv[6], yv[7]);
        }
      }
    }
  };

  if (nchunks > 0) {
    u32x4 gA = {0u, 0u, 0u, 0u}, gB = gA, gC = gA;   // gate tiles of chunks s-1, s, s+1
    const int last = nchunks - 1;
    load(pre0, 0);
    load(pre1, min(1, last));
    stage(sm.hand[0], pre0);
    load(pre0, min(2, last));
    if (NORM) gB = load_gate(0);
    sync_lds();
    // step s: stage chunk s+1 (loaded at step s-2), load chunk s+3 into the freed set,
    // products of chunk s, output rows of chunk s-1.  Chunks past the end repeat the last.
    auto step = [&](int s, Pre &stage_from) {
      stage(sm.hand[(s + 1) & 1], stage_from);
      load(stage_from, min(s + 3, last));
      if (NORM) gC = load_gate(min(s + 1, last));
      products(sm.hand[s & 1], sm.ost[s & 1]);
      if (s >= 1) emit(s - 1, sm.ost[(s + 1) & 1], gA);
      gA = gB;
      gB = gC;
      sync_lds();
    };
    int s = 0;
    for (; s + 1 < nchunks; s += 2) {
      step(s, pre1);                             // chunk s+1 is in pre1, s+2 in pre0
      step(s + 1, pre0);
    }
    if (s < nchunks) step(s, pre1);
    emit(last, sm.ost[(last + 2) & 1], gA);
  }

#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) fin[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + wcol] = Sacc[t][i];
}

template <typename TOut, bool HAS_INIT, bool NORM>
hipError_t launch3(const Args &a, const void *ws, hipStream_t st) {
  const int units = a.N * a.H;
  hipLaunchKernelGGL((chunk_scan_kernel<TOut, HAS_INIT, NORM>), dim3(static_cast<unsigned>(units)), dim3(NT), 0,
                     st, static_cast<const uint16_t *>(a.v), static_cast<const Rec *>(ws), a.init, a.state, a.cu,
                     static_cast<TOut *>(a.o), static_cast<const uint16_t *>(a.gate), a.norm_w,
                     static_cast<TOut *>(a.y), a.eps, a.T, a.H, units);
  return hipGetLastError();
}

template <typename TOut, bool HAS_INIT>
hipError_t launch2(const Args &a, const void *ws, hipStream_t st) {
  return a.y ? launch3<TOut, HAS_INIT, true>(a, ws, st) : launch3<TOut, HAS_INIT, false>(a, ws, st);
}

template <typename TOut>
hipError_t launch1(const Args &a, const void *ws, hipStream_t st) {
  return a.init ? launch2<TOut, true>(a, ws, st) : launch2<TOut, false>(a, ws, st);
}

}  // namespace

bool prefill_mfma_supports(int dk, int dv, int in_bf16) { return in_bf16 && dk == DK && dv == DV; }

// Offsets of tokens within one batch row are 32-bit: T * H * 128 must stay below 2^31.
bool prefill_mfma_fits(long long T, long long H) { return T * H * DK < (1LL << 31); }

hipError_t launch_chunk_scan(const Args &a, const void *ws, hipStream_t st) {
  if (a.N * static_cast<long long>(a.H) <= 0) return hipSuccess;
  return a.out_bf16 ? launch1<uint16_t>(a, ws, st) : launch1<float>(a, ws, st);
}

}  // namespace kda
