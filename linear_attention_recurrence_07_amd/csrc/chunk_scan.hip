// State scan of the bf16 chunked prefill on the CDNA4 matrix cores (head size 128,
// 32-token chunks).
//
// The prompt kernel of the KDA recurrence carries the state from chunk to chunk (nnterp
// Kimi-Linear page, Notes, "Loading" and the KDA paragraph; section 04 docstring).  With
// S0 the incoming state, G the running sum of g over the chunk per key channel, and the
// chunk's record from the preparation kernel (Bqk, W = (I + A)^-1 diag(beta), norms):
//     U      = W (V - (k^ exp(G)) S0)
//     O      = (q^ exp(G)) S0 + Bqk U
//     S_next = diag(exp(G_last)) S0 + (k^ exp(G_last - G))^T U
// which is the token-by-token recurrence regrouped; it equals it up to rounding.
//
// Work decomposition.  Value columns are independent, so a work-group owns one
// (sequence, head, 64-column tile) with eight waves, two per SIMD.  Every step handles
// two chunks, one apart, handed over through double-buffered LDS:
//   producer work on chunk c (all waves; 4 tokens x 2 channels per thread): unpack the
//     inputs loaded one chunk ahead, apply the norms, form exp(G) by per-group products
//     combined across waves, and write the decayed operands k^ exp(G), q^ exp(G),
//     (k^ exp(G_last - G))^T in fp16 plus the record's Bqk and W;
//   consumer work on chunk c-1 (waves 0-3): each wave owns 16 value columns and keeps its
//     128 x 16 slice of the fp32 state in registers for the whole sequence; every product
//     above runs on MFMA; the output tile goes out through LDS one step later.
// Two work-group barriers per step.
//
// Precision: fp16 operands for the state and decayed keys/queries (all bounded by the
// state and |k^|, |q^| <= 1 times decays <= 1), V - K S0 and U split into fp16 hi + lo
// parts; fp32 accumulation.  The fp16 state operand limits |S| to well inside fp16 range.
//
// MFMA operand trick.  A 16x16 fp32 accumulator tile holds rows 4*(lane/16)+i of column
// lane%16.  Two such tiles, converted, are the B operand of a 16x16x32 product whose K
// order is permuted the same way on the A side, so the state and U never leave registers.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int DVT = 64;           // value columns per work-group
constexpr int NTILE = DV / DVT;   // work-groups per (sequence, head)
constexpr int NCW = DVT / 16;     // consumer waves; each owns 16 value columns
constexpr int NW = 8;             // waves per work-group
constexpr int NT = NW * 64;       // 512 threads
constexpr int TPW = C / NW;       // tokens per producer wave (4)
static_assert(NCW == 4 && TPW == 4, "the thread mappings assume these sizes");

// LDS row strides in elements.
constexpr int LDS_ = DK + 4;      // fp16 [token][channel] state operands, 8-byte reads
constexpr int LDV = DVT + 8;      // value tile (bf16)
constexpr int LDB = C + 8;        // 32x32 Bqk and W (fp16)
constexpr int LDO = DVT + 4;      // fp32 output staging
// (k exp(G_last - G))^T: channel rows of 32 tokens, with 4 extra elements after every
// 2 rows so the transposed 8-byte writes spread over the banks.
__device__ __forceinline__ int ket_row(int ch) { return ch * C + (ch >> 1) * 4; }
constexpr int KET_SIZE = DK * C + (DK / 2) * 4;

// Data handed from the producer work on chunk c to the consumer work on it, one step later.
struct alignas(16) Hand {
  uint16_t kb[C * LDS_];       // fp16 k^ exp(G)
  uint16_t qt[C * LDS_];       // fp16 q^ exp(G)
  uint16_t ket[KET_SIZE];      // fp16 (k^ exp(G_last - G))^T
  uint16_t vt[C * LDV];        // bf16 value tile
  uint16_t bq[C * LDB];        // fp16 Bqk
  uint16_t w[C * LDB];         // fp16 (I + A)^-1 diag(beta)
  float ec[DK];                // decay over the whole chunk
};
struct alignas(16) Smem {
  Hand hand[2];
  float gtot[NW * DK];         // decay product over each 4-token group
  float ost[C * LDO];          // fp32 output staging
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget");

struct Raw {   // one chunk's inputs for one thread, as loaded
  uint32_t k[TPW], q[TPW];     // 2 bf16 channels per token
  f32x2 g[TPW];
  float nv;                    // lanes 0-3: kn, lanes 4-7: qn of the wave's tokens (0: no token)
  u32x2 v;                     // 4 bf16 values of the value tile
  float vk;                    // kn of the value tile's token (0: no token)
  u32x4 rec;                   // threads 0-255: one 16-byte piece of the record's Bqk, W
};

template <typename TOut, bool HAS_INIT>
__global__ void __launch_bounds__(NT, 1)
chunk_scan_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const uint16_t *__restrict__ v, const float *__restrict__ g,
                  const Rec *__restrict__ ws, const float *init, float *fin,
                  const int32_t *__restrict__ cu, TOut *__restrict__ o, int T, int H, int units) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches stay scalar
  const int l16 = lane & 15, lg = lane >> 4;

  // Work-groups are dealt to the 8 XCDs round-robin; give both column tiles of one
  // (sequence, head) ids 8 apart so they share an XCD's L2 for the common reads.
  const int id = blockIdx.x;
  const int unit = (id / (8 * NTILE)) * 8 + (id % 8);
  const int tile = (id / 8) % NTILE;
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
  const int col0 = tile * DVT;
  const size_t slab = (static_cast<size_t>(n) * H + h) * DK * DV;
  const int nchunks = (t_end - t_begin + C - 1) / C;
  const int tok_stride = H * DK;                               // elements between tokens (q, k, g)
  const size_t row0 = static_cast<size_t>(b) * T;              // first token row of this batch row
  const uint16_t *kp = k + row0 * tok_stride + h * DK + 2 * lane;
  const uint16_t *qp = q + row0 * tok_stride + h * DK + 2 * lane;
  const float *gp = g + row0 * tok_stride + h * DK + 2 * lane;
  const uint16_t *vp = v + row0 * H * DV + h * DV + col0 + (tid & 15) * 4;
  const Rec *rp0 = ws + slot0 * H + h;                         // chunk c's record: rp0 + c * H

  // ---------------------------------------------------------------- producer state
  const int blk = wave >> 2;                     // sub-block of this wave's tokens
  const int gi = wave & 3;                       // group within the sub-block
  Raw raw;
  // Loads are unconditional (clamped to the sequence's last token); padding and tokens
  // past the end are zeroed where the values are used, through their zero norm factors.
  auto load_raw = [&](int cidx) {
    const int c0 = t_begin + cidx * C;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tc = min(c0 + TPW * wave + j, t_end - 1);
      const int off = tc * tok_stride;
      raw.k[j] = *reinterpret_cast<const uint32_t *>(kp + off);
      raw.q[j] = *reinterpret_cast<const uint32_t *>(qp + off);
      raw.g[j] = *reinterpret_cast<const f32x2 *>(gp + off);
    }
    const Rec *rp = rp0 + static_cast<size_t>(cidx) * H;
    // lanes 0-3: kn of the wave's tokens, lanes 4-7: qn (per-lane loads, read out later)
    raw.nv = (lane & 4 ? rp->qn : rp->kn)[TPW * wave + (lane & 3)];
    if (wave < 4) raw.rec = reinterpret_cast<const u32x4 *>(rp)[tid];
    // value tile (32 tokens x 64 columns): token tid/16, 4 columns per thread
    const int tv = min(c0 + (tid >> 4), t_end - 1);
    raw.v = *reinterpret_cast<const u32x2 *>(vp + static_cast<size_t>(tv) * H * DV);
    raw.vk = rp->kn[tid >> 4];
    // keep these loads here, one step ahead of their use
    __asm__ volatile("" ::: "memory");
  };
  float kx[TPW][2], qx[TPW][2], fw[TPW][2], bw[TPW][2];

  // ---------------------------------------------------------------- consumer state (waves 0-3)
  const int wcol = 16 * (wave & 3) + l16;        // this lane's value column in the tile
  f32x4 Sacc[DK / 16];                           // Sacc[t][i] = S[16t + 4lg + i][col0 + wcol]
#pragma unroll
  for (int t = 0; t < DK / 16; ++t) Sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (HAS_INIT && wave < NCW) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[t][i] = init[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + col0 + wcol];
  }
  uint4 Sh[DK / 32];                             // S0 as fp16 B operands, shared by both sub-phases
  uint4 Uh = make_uint4(0, 0, 0, 0), Ul = Uh;

  // ================================================================ producer, sub-phase 1
  // Unpack the chunk's inputs, hand over the record and values, start loading the next
  // chunk, per-group decay products.
  auto prod1 = [&](Hand &hp, int c_next) {
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const float kn = readlane(raw.nv, j), qn = readlane(raw.nv, TPW + j);
      const bool valid = kn > 0.f;
      kx[j][0] = lo_bf16(raw.k[j]) * kn; kx[j][1] = hi_bf16(raw.k[j]) * kn;
      qx[j][0] = lo_bf16(raw.q[j]) * qn; qx[j][1] = hi_bf16(raw.q[j]) * qn;
      fw[j][0] = valid ? raw.g[j].x : 0.f; fw[j][1] = valid ? raw.g[j].y : 0.f;
    }
    *reinterpret_cast<u32x2 *>(hp.vt + (tid >> 4) * LDV + (tid & 15) * 4) =
        raw.vk > 0.f ? raw.v : u32x2{0u, 0u};
    if (wave < 4) {
      // pieces 0-127: Bqk rows, 128-255: W rows; 4 pieces of 8 elements per row
      const int p = tid & 127;
      uint16_t *dst = (tid < 128 ? hp.bq : hp.w) + (p >> 2) * LDB + (p & 3) * 8;
      *reinterpret_cast<u32x4 *>(dst) = raw.rec;
    }
    load_raw(c_next);
    // fw[j] = prod_{i<=j} e_i (inclusive), bw[j] = prod_{j<i<4} e_i (exclusive)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float e[TPW];
#pragma unroll
      for (int j = 0; j < TPW; ++j) e[j] = fast_exp2(fw[j][c] * kLog2e);
      float run = 1.f;
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        run *= e[j];
        fw[j][c] = run;
      }
      run = 1.f;
#pragma unroll
      for (int j = TPW - 1; j >= 0; --j) {
        bw[j][c] = run;
        run *= e[j];
      }
    }
    *reinterpret_cast<float2 *>(sm.gtot + wave * DK + 2 * lane) = make_float2(fw[TPW - 1][0], fw[TPW - 1][1]);
  };

  // ================================================================ producer, sub-phase 2
  // Combine the group decay products and write the decayed operands of the chunk.
  auto prod2 = [&](Hand &hp) {
    float gt[NW][2];
#pragma unroll
    for (int m = 0; m < NW; ++m) {
      const float2 x = *reinterpret_cast<const float2 *>(sm.gtot + m * DK + 2 * lane);
      gt[m][0] = x.x; gt[m][1] = x.y;
    }
    float pre[2], post[2], ec[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // this block's group products, selected with constant register indices
      const float b0 = blk ? gt[4][c] : gt[0][c], b1 = blk ? gt[5][c] : gt[1][c];
      const float b2 = blk ? gt[6][c] : gt[2][c], b3 = blk ? gt[7][c] : gt[3][c];
      const float p01 = b0 * b1, p23 = b2 * b3;
      const float e3m = gi == 0 ? 1.f : gi == 1 ? b0 : gi == 2 ? p01 : p01 * b2;   // block start -> group
      const float e4m = gi == 3 ? 1.f : gi == 2 ? b3 : gi == 1 ? p23 : b1 * p23;   // group -> block end
      const float d0 = (gt[0][c] * gt[1][c]) * (gt[2][c] * gt[3][c]);             // decay over block 0
      const float d1 = (gt[4][c] * gt[5][c]) * (gt[6][c] * gt[7][c]);             // decay over block 1
      pre[c] = blk ? d0 * e3m : e3m;             // chunk start -> group start
      post[c] = blk ? e4m : e4m * d1;            // group end -> chunk end
      ec[c] = d0 * d1;
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int r = TPW * wave + j;
      float kb[2], qt[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float e = pre[c] * fw[j][c];       // exp(G_r)
        kb[c] = kx[j][c] * e;
        qt[c] = qx[j][c] * e;
        kx[j][c] *= bw[j][c] * post[c];          // k^ exp(G_last - G_r), for the transpose
      }
      *reinterpret_cast<uint32_t *>(hp.kb + r * LDS_ + 2 * lane) = pack_f16x2(kb[0], kb[1]);
      *reinterpret_cast<uint32_t *>(hp.qt + r * LDS_ + 2 * lane) = pack_f16x2(qt[0], qt[1]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      *reinterpret_cast<uint2 *>(hp.ket + ket_row(2 * lane + c) + TPW * wave) =
          pack_f16x4(kx[0][c], kx[1][c], kx[2][c], kx[3][c]);
    if (wave == 0) *reinterpret_cast<float2 *>(hp.ec + 2 * lane) = make_float2(ec[0], ec[1]);
  };

  // ================================================================ consumer, sub-phase 1
  // Y = V - (k^ exp(G)) S0;  U0 = W00 Y0;  U1 = W10 Y0 + W11 Y1.
  auto cons1 = [&](const Hand &hc) {
    __asm__ volatile("" ::: "memory");   // not to be speculated onto producer-only waves
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {   // K step s covers channels {32s+4lg+0..3, 32s+16+4lg+0..3}
      const f32x4 a = Sacc[2 * s], bb = Sacc[2 * s + 1];
      Sh[s] = join(pack_f16x4(a[0], a[1], a[2], a[3]), pack_f16x4(bb[0], bb[1], bb[2], bb[3]));
    }
    uint2 yh[2], yl[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *ap = hc.kb + (SB * m + l16) * LDS_ + 4 * lg;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) acc = mfma_f16(join(lds_u2(ap + 32 * s), lds_u2(ap + 32 * s + 16)), Sh[s], acc);
      f32x4 y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = bf16_to_f32(hc.vt[(SB * m + 4 * lg + i) * LDV + wcol]) - acc[i];
      split_f16x4(y, yh[m], yl[m]);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const uint2 w00 = lds_u2(hc.w + l16 * LDB + 4 * lg);
    f32x4 U0 = mfma_f16k16(w00, yl[0], zero);
    U0 = mfma_f16k16(w00, yh[0], U0);
    const uint16_t *w1p = hc.w + (SB + l16) * LDB + 4 * lg;
    const uint4 w1 = join(lds_u2(w1p), lds_u2(w1p + 16));
    f32x4 U1 = mfma_f16(w1, join(yl[0], yl[1]), zero);
    U1 = mfma_f16(w1, join(yh[0], yh[1]), U1);
    uint2 u0h, u0l, u1h, u1l;
    split_f16x4(U0, u0h, u0l);
    split_f16x4(U1, u1h, u1l);
    Uh = join(u0h, u1h);   // tokens {4lg+0..3, 16+4lg+0..3} as K=32 B operands
    Ul = join(u0l, u1l);
  };

  // ================================================================ consumer, sub-phase 2
  // O = (q^ exp(G)) S0 + Bqk U into the staging buffer; then the state carry.
  auto cons2 = [&](const Hand &hc) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *ap = hc.qt + (SB * m + l16) * LDS_ + 4 * lg;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) acc = mfma_f16(join(lds_u2(ap + 32 * s), lds_u2(ap + 32 * s + 16)), Sh[s], acc);
      const uint16_t *bqp = hc.bq + (SB * m + l16) * LDB + 4 * lg;
      const uint4 bqv = join(lds_u2(bqp), lds_u2(bqp + 16));
      acc = mfma_f16(bqv, Ul, acc);
      acc = mfma_f16(bqv, Uh, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.ost[(SB * m + 4 * lg + i) * LDO + wcol] = acc[i];
    }
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      const float4 e = *reinterpret_cast<const float4 *>(hc.ec + 16 * t + 4 * lg);
      Sacc[t][0] *= e.x; Sacc[t][1] *= e.y; Sacc[t][2] *= e.z; Sacc[t][3] *= e.w;
      const uint16_t *ap = hc.ket + ket_row(16 * t + l16) + 4 * lg;
      const uint4 kv = join(lds_u2(ap), lds_u2(ap + 16));
      Sacc[t] = mfma_f16(kv, Ul, Sacc[t]);
      Sacc[t] = mfma_f16(kv, Uh, Sacc[t]);
    }
  };

  // ================================================================ consumer, output rows
  // Coalesced output rows of chunk cidx from the staging buffer (waves 0-3): token tid/8,
  // 8 columns per thread.
  auto cons3 = [&](int cidx) {
    const int r = tid >> 3, c8 = (tid & 7) * 8;
    const int t = t_begin + cidx * C + r;
    if (t < t_end) {
      TOut *op = o + ((row0 + t) * H + h) * DV + col0 + c8;
      const float *sp = sm.ost + r * LDO + c8;
      const float4 x0 = reinterpret_cast<const float4 *>(sp)[0];
      const float4 x1 = reinterpret_cast<const float4 *>(sp)[1];
      if constexpr (sizeof(TOut) == 2) {
        uint4 w;
        w.x = pack_bf16x2(x0.x, x0.y); w.y = pack_bf16x2(x0.z, x0.w);
        w.z = pack_bf16x2(x1.x, x1.y); w.w = pack_bf16x2(x1.z, x1.w);
        *reinterpret_cast<uint4 *>(op) = w;
      } else {
        reinterpret_cast<float4 *>(op)[0] = x0;
        reinterpret_cast<float4 *>(op)[1] = x1;
      }
    }
  };

  const bool consumer = wave < NCW;
  if (nchunks > 0) {
    load_raw(0);
    // step 0: producer work only
    prod1(sm.hand[0], min(1, nchunks - 1));
    sync_lds();
    prod2(sm.hand[0]);
    sync_lds();
    // steady state: producer work on chunk `step`, consumer work on chunk `step - 1`,
    // output rows of chunk `step - 2`
    for (int step = 1; step < nchunks; ++step) {
      Hand &hp = sm.hand[step & 1];
      const Hand &hc = sm.hand[(step + 1) & 1];
      prod1(hp, min(step + 1, nchunks - 1));
      if (consumer) {
        if (step >= 2) cons3(step - 2);
        cons1(hc);
      }
      sync_lds();
      prod2(hp);
      if (consumer) cons2(hc);
      sync_lds();
    }
    // last step: consumer work only
    const Hand &hc = sm.hand[(nchunks + 1) & 1];
    if (consumer) {
      if (nchunks >= 2) cons3(nchunks - 2);
      cons1(hc);
    }
    sync_lds();
    if (consumer) cons2(hc);
    sync_lds();
    if (consumer) cons3(nchunks - 1);
  }

  if (consumer) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fin[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + col0 + wcol] = Sacc[t][i];
  }
}

template <typename TOut, bool HAS_INIT>
hipError_t launch_init(const Args &a, const void *ws, hipStream_t st) {
  const int units = a.N * a.H;
  const unsigned grid = static_cast<unsigned>((units + 7) / 8) * 8 * NTILE;
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                 *v = static_cast<const uint16_t *>(a.v);
  const Rec *rec = static_cast<const Rec *>(ws);
  TOut *o = static_cast<TOut *>(a.o);
  hipLaunchKernelGGL((chunk_scan_kernel<TOut, HAS_INIT>), dim3(grid), dim3(NT), 0, st, q, k, v, a.g, rec,
                     a.init, a.state, a.cu, o, a.T, a.H, units);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_typed(const Args &a, const void *ws, hipStream_t st) {
  return a.init ? launch_init<TOut, true>(a, ws, st) : launch_init<TOut, false>(a, ws, st);
}

}  // namespace

bool prefill_mfma_supports(int dk, int dv, int in_bf16) { return in_bf16 && dk == DK && dv == DV; }

// Offsets of tokens within one batch row are 32-bit: T * H * 128 must stay below 2^31.
bool prefill_mfma_fits(long long T, long long H) { return T * H * DK < (1LL << 31); }

hipError_t launch_chunk_scan(const Args &a, const void *ws, hipStream_t st) {
  return a.out_bf16 ? launch_typed<uint16_t>(a, ws, st) : launch_typed<float>(a, ws, st);
}

}  // namespace kda
