// State scan of the bf16 chunked prefill on the CDNA4 matrix cores (head size 128,
// 32-token chunks).
//
// The prompt kernel of the KDA recurrence carries the state from chunk to chunk (nnterp
// Kimi-Linear page, Notes, "Loading" and the KDA paragraph; section 04 docstring).  With
// S0 the incoming state, G the running sum of g over the chunk per key channel, and the
// chunk's record from the preparation kernel (kda_chunk.h):
//     U      = W (V - (k^ exp(G)) S0)
//     O      = (q^ exp(G)) S0 + Bqk U
//     S_next = diag(exp(G_last)) S0 + (k^ exp(G_last - G))^T U
// which is the token-by-token recurrence regrouped; it equals it up to rounding.
//
// Work decomposition.  Value columns are independent in the recurrence, so a work-group
// owns one (sequence, head, 64-column tile); at 96 heads that is 192 work-groups, one per
// CU.  Eight waves, two per SIMD:
//   compute waves 0-3: wave w owns value columns 16w..16w+15 of the tile and keeps its
//     128 x 16 slice of the fp32 state in registers for the whole sequence.  Each chunk's
//     products run on MFMA with the record's operands read from LDS in fragment order
//     (16-byte reads, no bank conflicts).
//   helper waves 4-7: stage the record and value tile of chunk c+1 (loaded two or three
//     steps earlier into registers) into the other half of a double-buffered LDS
//     hand-over area, issue the loads of chunk c+3 (or c+4), and write chunk c-1's output
//     rows from a ring of output tiles, while the compute waves work on chunk c.
// One work-group barrier per step.  The two tiles of a head get work-group ids 8 apart,
// so they land on the same XCD and share its L2 for the record reads.
//
// Gated norm epilogue, when y is given (nnterp Kimi-Linear page and Kimi-K3 atlas,
// gate-project page: y = w * o / sqrt(mean(o^2) + eps) * sigmoid(gate) over the 128
// channels of a head).
// The mean needs both 64-column tiles of a head, which live in two work-groups.  When a
// helper writes chunk c's output rows (step c+1) it also publishes, per token, the sum of
// squares of its 64 columns as one 64-bit word (a flag in the high half, the float in
// the low half) in the workspace.  Compute wave 0 reads the partner tile's words for
// chunk c: it issues the device-coherent read (which bypasses the XCD's L2 and takes
// about a step) at step c+3, two steps after the partner published them, and at step
// c+4 passes the sums to the helpers through LDS; the helpers write y of chunk c at step
// c+5.  The compute waves issue no other global loads, so waiting for that read never
// waits for the helpers' prefetches.  The tiles therefore do not wait on each other in
// lockstep; the output tiles of the last six chunks stay in LDS.  The reader clears each
// word after use, and the preparation kernel clears them all, so no call sees another
// call's words.
// Forward progress: the two tiles of a head are consecutive work-groups of one XCD's
// dispatch order (work-groups are dealt to the XCDs round-robin and each XCD starts its
// own in id order), and a tile waits only for its partner.  So at most one work-group
// per XCD can wait for a partner that has not started, and the others finish and free
// their CUs; a wait can last long only while other work holds the CUs.  A wait is still
// bounded (about 2^22 polls, seconds): one that runs out gives NaN in y instead of a
// hang and sets the workspace's status word, which kda_chunk_prefill_status reports.
//
// Precision: fp16 operands for the state and the decayed keys/queries; W, U, Bqk and
// V - K S0 as fp16 hi + lo parts; fp32 accumulation.  The outputs can be far smaller than
// the terms they are the sum of (when the state already predicts the values well, as with
// filtered inputs that share a common direction), so the parts of those terms carry more
// than fp16's precision.  The fp16 state operand limits |S| to well inside fp16 range.
#include <type_traits>

#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int DVT = 64;           // value columns per work-group
constexpr int NTILE = DV / DVT;   // work-groups per (sequence, head)
constexpr int NW = 8;             // waves per work-group
constexpr int NT = NW * 64;       // 512 threads
constexpr int NCW = DVT / 16;     // compute waves, 16 columns each
constexpr int NHT = NT - NCW * 64;  // helper threads (256)
constexpr int LDV = DVT + 8;      // value tile row stride (bf16)
constexpr int LDO = DVT + 4;      // fp32 output tile row stride
constexpr int REC_PIECES = static_cast<int>(sizeof(Rec) / 16);
constexpr int kSpinLimit = 1 << 22;   // polls of a partner's word before giving up (several seconds)

constexpr int PPT = (REC_PIECES + NHT - 1) / NHT;   // record pieces per helper thread (8)
static_assert(NCW == 4 && NHT == 256, "thread mappings");

constexpr int LDVF = DVT + 4;     // fp32 value tile row stride
// F32V: the value tile holds fp32 values (the filtered values of the fused convolution)
template <bool F32V>
struct alignas(16) Hand {
  Rec rec;
  typename std::conditional<F32V, float, uint16_t>::type vt[C * (F32V ? LDVF : LDV)];   // [token][column]
};
template <int NOST, bool CONV>
struct alignas(16) Smem {
  Hand<CONV> hand[2];
  float ost[NOST][C * LDO];    // fp32 output tiles: chunk c in ost[c % NOST]
  float pss[2][C];             // NORM: the partner tile's sums of squares, chunk c in pss[c & 1]
  // CONV: raw value rows of chunk c in raw[c & 1][3 ..], after the three newest real
  // inputs before the chunk (rows 0..2, oldest first)
  uint16_t raw[CONV ? 2 : 1][CONV ? 3 + C : 1][LDV];
};
constexpr int kNormLag = 5;          // y of chunk c is written at step c + kNormLag
static_assert(sizeof(Smem<kNormLag + 1, true>) <= 160 * 1024, "LDS budget");
static_assert(sizeof(Hand<false>) % 16 == 0 && sizeof(Hand<true>) % 16 == 0 && (LDV * 2) % 16 == 0 &&
                  (LDVF * 4) % 16 == 0 && (LDO * 4) % 16 == 0, "16-byte LDS access");

// NORM: also write y (gated norm over the head's 128 channels); xs holds the exchanged
// partial sums of squares, 2 tiles x 32 tokens per (slot, head).  WRITE_O: store the head
// outputs o (only NORM may leave them out: the caller then wants y alone).  CONV: v is
// the raw projection; the helpers run its short convolution (cv).  STATES: for the
// per-token states, also store each chunk's U rows (fp32 [slot, head, token, column] in
// uws) and the state after the chunk's last position into states [.., T, H, DK, DV].
template <typename TOut, bool HAS_INIT, bool NORM, bool WRITE_O, bool CONV, bool STATES>
__global__ void __launch_bounds__(NT, 1)
chunk_scan_kernel(const uint16_t *__restrict__ v, const Rec *__restrict__ ws, const float *init,
                  float *fin, const int32_t *__restrict__ cu, TOut *__restrict__ o,
                  const uint16_t *__restrict__ gate, const float *__restrict__ norm_w, TOut *__restrict__ y,
                  uint64_t *xs, uint32_t *status, float eps, int T, int H, int units, ConvIn cv,
                  float *states, float *uws) {
  constexpr int NOST = NORM ? kNormLag + 1 : 2;
  __shared__ Smem<NOST, CONV> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: branches stay scalar
  const int l16 = lane & 15, lg = lane >> 4;
  const bool helper = wave >= NCW;
  const int ht = tid - NCW * 64;                               // helper thread index

  // Work-groups are dealt to the 8 XCDs round-robin; the tiles of one (sequence, head)
  // get ids 8 apart.
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
  const size_t row0 = static_cast<size_t>(b) * T;              // first token row of this batch row
  const size_t tok_stride = static_cast<size_t>(H) * DV;       // elements between tokens (v, o)
  // Addresses: a wave-uniform base plus a 32-bit per-lane byte offset.  Within one batch
  // row, token offsets stay below 2^32 bytes (T * H * 128 < 2^31).
  // A helper thread's row piece: token ht/8, columns (ht%8)*8 .. +7 of the tile.
  const int hr = ht >> 3, hc8 = (ht & 7) * 8;
  const uint32_t piece = static_cast<uint32_t>(h * DV + col0 + hc8) * 2u;   // bytes
  const uint32_t tok_bytes = static_cast<uint32_t>(H * DV) * 2u;
  const uint8_t *vrow = reinterpret_cast<const uint8_t *>(v + row0 * tok_stride);
  const Rec *rp0 = ws + slot0 * H + h;                         // chunk c's record: rp0 + c * H
  const int last = nchunks - 1;

  // ================================================================ helper side
  struct Pre {
    u32x4 r[PPT];
    u32x4 v;                   // the value piece of the chunk (CONV: of the next chunk)
    uint32_t valid;            // the chunk's token flags
  };
  const uint8_t *grow = reinterpret_cast<const uint8_t *>(gate + row0 * tok_stride);
  uint32_t vzero;              // 0 in a vector register: keeps the flag load a per-lane load
  __asm__ volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  auto load = [&](Pre &pre, int cidx) {
    const uint8_t *rp = reinterpret_cast<const uint8_t *>(rp0 + static_cast<size_t>(cidx) * H);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const uint8_t *rpi = rp + NHT * 16 * i;    // uniform base per piece row
      if (i < PPT - 1 || ht + NHT * i < REC_PIECES)
        pre.r[i] = *reinterpret_cast<const u32x4 *>(rpi + static_cast<uint32_t>(ht) * 16u);
    }
    pre.valid = *reinterpret_cast<const uint32_t *>(rp + offsetof(Rec, valid) + vzero);
    const int vidx = CONV ? min(cidx + 1, last) : cidx;
    const uint32_t tv = static_cast<uint32_t>(min(t_begin + vidx * C + hr, t_end - 1));
    pre.v = *reinterpret_cast<const u32x4 *>(vrow + (piece + tv * tok_bytes));
    __asm__ volatile("" ::: "memory");   // keep the loads here, ahead of their use
  };
  auto stage = [&](Hand<CONV> &hd, const Pre &pre) {
    u32x4 *dst = reinterpret_cast<u32x4 *>(&hd.rec);
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (i < PPT - 1 || ht + NHT * i < REC_PIECES) dst[ht + NHT * i] = pre.r[i];
    // values of padding and of tokens past the end are zeroed
    if constexpr (!CONV) {
      const bool keep = (pre.valid >> hr) & 1u;
      *reinterpret_cast<u32x4 *>(&hd.vt[hr * LDV + hc8]) = keep ? pre.v : u32x4{0u, 0u, 0u, 0u};
    }
  };

  // ================================================================ short convolution (helpers)
  // CONV (Kimi-K3 atlas, KDA layer page, kda-init code: a causal ShortConvolution with
  // SiLU on the value projection).  The value tile of a chunk is filtered from its raw rows
  // in LDS one step after they were written there, and handed to the compute waves in fp32.  A chunk's raw area starts with the
  // three newest real inputs before it, so a token's window is the newest real rows
  // before it in that area (its flags: the chunk's, with the three rows in front always
  // real); the next chunk's three rows are taken from the same area.  Padding therefore
  // never enters a window, and the window needs no look-back past one chunk.  At the
  // sequence start the three rows are its carried inputs (or zeros).
  float ctap[8][4];            // right-aligned taps of this thread's 8 value channels
  if constexpr (CONV) {
    if (helper) {
      const float *wp = cv.w[2] + (static_cast<size_t>(h) * DV + col0 + hc8) * cv.W;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ctap[i][jj] = jj >= 4 - cv.W ? wp[i * cv.W + jj - (4 - cv.W)] : 0.f;
    }
  }
  auto put_raw = [&](int buf, u32x4 w) { *reinterpret_cast<u32x4 *>(&sm.raw[buf][3 + hr][hc8]) = w; };
  // Filter chunk buf's tile into hd.vt (token hr, columns hc8..hc8+7), in fp32: the LDS
  // reads first (conv_read), the arithmetic and the stores later (conv_write), so that
  // other work covers the reads' latency.
  struct ConvRows {
    u32x4 x, r0, r1, r2;
  };
  auto conv_read = [&](int buf, uint32_t valid) -> ConvRows {
    // newest three real rows before token hr: bits 0..2 of ext (the rows before the chunk)
    // are always set, so three are always found
    const uint64_t ext = (static_cast<uint64_t>(valid) << 3) | 7u;
    const int e = hr + 3;
    uint64_t below = ext & ((uint64_t{1} << e) - 1u);
    const int p1 = 63 - __builtin_clzll(below);
    below &= ~(uint64_t{1} << p1);
    const int p2 = 63 - __builtin_clzll(below);
    below &= ~(uint64_t{1} << p2);
    const int p3 = 63 - __builtin_clzll(below);
    ConvRows cr;
    cr.x = *reinterpret_cast<const u32x4 *>(&sm.raw[buf][e][hc8]);
    cr.r2 = *reinterpret_cast<const u32x4 *>(&sm.raw[buf][p1][hc8]);
    cr.r1 = *reinterpret_cast<const u32x4 *>(&sm.raw[buf][p2][hc8]);
    cr.r0 = *reinterpret_cast<const u32x4 *>(&sm.raw[buf][p3][hc8]);
    return cr;
  };
  auto conv_write = [&](Hand<CONV> &hd, const ConvRows &cr, uint32_t valid) {
    float z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = i >> 1;
      auto el = [&](u32x4 x) { return (i & 1) ? hi_bf16(x[w]) : lo_bf16(x[w]); };
      // all four taps (a narrower filter's older taps are zero; its window rows are real
      // inputs, carried inputs or zeros, so finite): no per-element selects on the width
      z[i] = conv_z4(make_float4(ctap[i][0], ctap[i][1], ctap[i][2], ctap[i][3]), el(cr.r0), el(cr.r1), el(cr.r2),
                     el(cr.x));
      if (cv.silu) z[i] = silu_act(z[i]);
    }
    const bool keep = (valid >> hr) & 1u;
    if constexpr (CONV) {
      float *dst = hd.vt + hr * LDVF + hc8;
      reinterpret_cast<float4 *>(dst)[0] = keep ? make_float4(z[0], z[1], z[2], z[3]) : make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4 *>(dst)[1] = keep ? make_float4(z[4], z[5], z[6], z[7]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto conv_tile = [&](Hand<CONV> &hd, int buf, uint32_t valid) { conv_write(hd, conv_read(buf, valid), valid); };
  // The three newest real rows of chunk area `from` (flags `valid`) become rows 0..2 of
  // area `to` (threads 0..23: row ht/8); read and write apart, as for the filter.
  auto carry_read = [&](int from, uint32_t valid) -> u32x4 {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (ht < 24) {
      uint64_t ext = (static_cast<uint64_t>(valid) << 3) | 7u;
      const int q1 = 63 - __builtin_clzll(ext);
      ext &= ~(uint64_t{1} << q1);
      const int q2 = 63 - __builtin_clzll(ext);
      ext &= ~(uint64_t{1} << q2);
      const int q3 = 63 - __builtin_clzll(ext);
      const int src = hr == 2 ? q1 : (hr == 1 ? q2 : q3);
      w = *reinterpret_cast<const u32x4 *>(&sm.raw[from][src][hc8]);
    }
    return w;
  };
  auto carry_write = [&](int to, u32x4 w) {
    if (ht < 24) *reinterpret_cast<u32x4 *>(&sm.raw[to][hr][hc8]) = w;
  };
  auto carry = [&](int from, int to, uint32_t valid) { carry_write(to, carry_read(from, valid)); };
  // Token ht/8 of chunk cidx, columns (ht%8)*8..+7 of the tile.
  auto store_row = [&](TOut *dst, int t, float4 x0, float4 x1) {
    const size_t off = row0 * tok_stride + (piece + static_cast<uint32_t>(t) * tok_bytes) / 2u;
    if constexpr (sizeof(TOut) == 2) {
      uint4 w;
      w.x = pack_bf16x2(x0.x, x0.y); w.y = pack_bf16x2(x0.z, x0.w);
      w.z = pack_bf16x2(x1.x, x1.y); w.w = pack_bf16x2(x1.z, x1.w);
      *reinterpret_cast<uint4 *>(dst + off) = w;
    } else {
      reinterpret_cast<float4 *>(dst + off)[0] = x0;
      reinterpret_cast<float4 *>(dst + off)[1] = x1;
    }
  };
  // Writes the output rows of chunk cidx; returns the token's sum of squares over the
  // tile's 64 columns (NORM), the same in the 8 lanes of the token.
  auto emit = [&](int cidx, const float *ost) -> float {
    const int t = t_begin + cidx * C + hr;
    const float4 x0 = *reinterpret_cast<const float4 *>(ost + hr * LDO + hc8);
    const float4 x1 = *reinterpret_cast<const float4 *>(ost + hr * LDO + hc8 + 4);
    if constexpr (WRITE_O) {
      if (t < t_end) store_row(o, t, x0, x1);
    }
    if constexpr (NORM) {
      float ss = x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w;
      ss += x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
      return group_sum<8>(ss);                 // over the 8 lanes of the token
    }
    return 0.f;
  };

  // ================================================================ gated norm (helpers)
  // Exchange word of (chunk, tile, token).
  auto xword = [&](int cidx, int tl, int tok) {
    return xs + ((static_cast<size_t>(slot0 + cidx) * H + h) * NTILE + tl) * C + tok;
  };
  auto publish = [&](int cidx, float ss) {
    if ((ht & 7) == 0)
      __hip_atomic_store(xword(cidx, tile, hr), (uint64_t{1} << 32) | __float_as_uint(ss), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  auto fetch = [&](int cidx, int tok) -> uint64_t {
    return __hip_atomic_load(xword(cidx, tile ^ 1, tok), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // The partner's sum for (chunk, token), given a first read of its word; the caller
  // clears the word.  After one wait has run out, the later ones give up at once.
  bool lost = false;
  auto partner = [&](int cidx, int tok, uint64_t w) -> float {
    for (int n = 0; (w >> 32) != 1u; ++n) {
      if (lost || n == kSpinLimit) {
        if (!lost) __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lost = true;
        return __builtin_nanf("");
      }
      __builtin_amdgcn_s_sleep(2);
      w = fetch(cidx, tok);
    }
    return __uint_as_float(static_cast<uint32_t>(w));
  };
  auto clear = [&](int cidx, int tok) {
    __hip_atomic_store(xword(cidx, tile ^ 1, tok), uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // gate piece of token hr of chunk cidx and the chunk's token flags
  auto load_gate = [&](int cidx, u32x4 &gt, uint32_t &valid) {
    const uint32_t tv = static_cast<uint32_t>(min(t_begin + cidx * C + hr, t_end - 1));
    gt = *reinterpret_cast<const u32x4 *>(grow + (piece + tv * tok_bytes));
    valid = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(rp0 + static_cast<size_t>(cidx) * H) +
                                                offsetof(Rec, valid) + vzero);
  };
  float wn[8];                 // norm weights of this thread's 8 columns
  if constexpr (NORM) {
    if (helper) {
#pragma unroll
      for (int i = 0; i < 8; ++i) wn[i] = norm_w[col0 + hc8 + i];
    }
  }
  // y of token hr of chunk cidx from its output rows, the two tiles' sums of squares,
  // the gate piece and the chunk's token flags (padding gives 0).
  auto emit_y = [&](int cidx, const float *ost, float ss, u32x4 gt, uint32_t valid) {
    const int t = t_begin + cidx * C + hr;
    if (t >= t_end) return;
    const float rn = rsqrtf(ss * (1.f / DV) + eps);
    const bool keep = (valid >> hr) & 1u;
    float xv[8];
    *reinterpret_cast<float4 *>(xv) = *reinterpret_cast<const float4 *>(ost + hr * LDO + hc8);
    *reinterpret_cast<float4 *>(xv + 4) = *reinterpret_cast<const float4 *>(ost + hr * LDO + hc8 + 4);
    float yv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t gw = gt[i >> 1];
      const float gv = (i & 1) ? hi_bf16(gw) : lo_bf16(gw);
      // sigmoid from the hardware exp2 and reciprocal (each about 1 ulp)
      const float sg = __builtin_amdgcn_rcpf(1.f + fast_exp2(-kLog2e * gv));
      yv[i] = keep ? wn[i] * (xv[i] * rn) * sg : 0.f;
    }
    store_row(y, t, make_float4(yv[0], yv[1], yv[2], yv[3]), make_float4(yv[4], yv[5], yv[6], yv[7]));
  };

  // ================================================================ compute side
  f32x4 Sacc[DK / 16];                           // Sacc[t][i] = S[16t + 4lg + i][col0 + 16 wave + l16]
#pragma unroll
  for (int t = 0; t < DK / 16; ++t) Sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int wcol = 16 * wave + l16;              // this lane's column in the tile
  if (HAS_INIT && !helper) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[t][i] = init[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + col0 + wcol];
  }

  // S0 as fp16 B operands; K step s covers channels {32s+4lg+0..3, 32s+16+4lg+0..3}.
  // Formed at the end of the previous chunk, so the conversion overlaps its last products.
  uint4 Sh[DK / 32];
  auto to_f16 = [&]() {
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const f32x4 a = Sacc[2 * s], bb = Sacc[2 * s + 1];
      Sh[s] = join(pack_f16x4(a[0], a[1], a[2], a[3]), pack_f16x4(bb[0], bb[1], bb[2], bb[3]));
    }
  };
  to_f16();

  // One chunk's products.  The LDS reads of each phase are issued together ahead of their
  // first use (the empty asm statements keep them there), so their latency overlaps the
  // matrix-core work of the previous phase instead of stalling each product.
  auto products = [&](const Hand<CONV> &hc, float *ost, int cidx) {
    const u32x4 *KB = reinterpret_cast<const u32x4 *>(hc.rec.kb);
    const u32x4 *QT = reinterpret_cast<const u32x4 *>(hc.rec.qt);
    const u32x4 *KE = reinterpret_cast<const u32x4 *>(hc.rec.ket);
    const u32x4 *BQ = reinterpret_cast<const u32x4 *>(hc.rec.bq);
    const u32x4 *BQL = reinterpret_cast<const u32x4 *>(hc.rec.bqlo);
    // Every operand of the chunk is read at the start, in order of first use; each
    // phase then waits only for its own part.
    uint4 kbf[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) kbf[f] = __builtin_bit_cast(uint4, KB[f * 64 + lane]);
    const uint2 w00 = __builtin_bit_cast(uint2, reinterpret_cast<const u32x2 *>(hc.rec.w00)[lane]);
    const uint2 w00l = __builtin_bit_cast(uint2, reinterpret_cast<const u32x2 *>(hc.rec.w00lo)[lane]);
    const uint4 w1 = __builtin_bit_cast(uint4, reinterpret_cast<const u32x4 *>(hc.rec.w1)[lane]);
    const uint4 w1l = __builtin_bit_cast(uint4, reinterpret_cast<const u32x4 *>(hc.rec.w1lo)[lane]);
    float vv[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (CONV) vv[m][i] = hc.vt[(SB * m + 4 * lg + i) * LDVF + wcol];
        else vv[m][i] = bf16_to_f32(hc.vt[(SB * m + 4 * lg + i) * LDV + wcol]);
      }
    uint4 kef[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) kef[t] = __builtin_bit_cast(uint4, KE[t * 64 + lane]);
    float4 ecv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) ecv[t] = *reinterpret_cast<const float4 *>(hc.rec.ec + 16 * t + 4 * lg);
    uint4 qtf[8], bqf[2], bqlf[2];
#pragma unroll
    for (int f = 0; f < 8; ++f) qtf[f] = __builtin_bit_cast(uint4, QT[f * 64 + lane]);
#pragma unroll
    for (int m = 0; m < 2; ++m) bqf[m] = __builtin_bit_cast(uint4, BQ[m * 64 + lane]);
#pragma unroll
    for (int m = 0; m < 2; ++m) bqlf[m] = __builtin_bit_cast(uint4, BQL[m * 64 + lane]);
    __asm__ volatile("" ::: "memory");
    // Y = V - (k^ exp(G)) S0 in fp16 (W carries the extra precision)
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      acc0 = mfma_f16(kbf[s], Sh[s], acc0);
      acc1 = mfma_f16(kbf[4 + s], Sh[s], acc1);
    }
    // Y as hi + lo parts too: the delta rule's residual is often much smaller than V
    uint2 yf[2], yl[2];
    split_f16x4(f32x4{vv[0][0] - acc0[0], vv[0][1] - acc0[1], vv[0][2] - acc0[2], vv[0][3] - acc0[3]}, yf[0], yl[0]);
    split_f16x4(f32x4{vv[1][0] - acc1[0], vv[1][1] - acc1[1], vv[1][2] - acc1[2], vv[1][3] - acc1[3]}, yf[1], yl[1]);
    // U0 = W00 Y0, U1 = W10 Y0 + W11 Y1, with W and Y as hi + lo parts (lo x lo dropped)
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 U0 = mfma_f16k16(w00l, yf[0], zero);
    U0 = mfma_f16k16(w00, yl[0], U0);
    U0 = mfma_f16k16(w00, yf[0], U0);
    const uint4 y01 = join(yf[0], yf[1]), yl01 = join(yl[0], yl[1]);
    f32x4 U1 = mfma_f16(w1l, y01, zero);
    U1 = mfma_f16(w1, yl01, U1);
    U1 = mfma_f16(w1, y01, U1);
    // the decay over the chunk, applied while the products above run
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      Sacc[t][0] *= ecv[t].x; Sacc[t][1] *= ecv[t].y; Sacc[t][2] *= ecv[t].z; Sacc[t][3] *= ecv[t].w;
    }
    uint2 u0h, u0l, u1h, u1l;
    split_f16x4(U0, u0h, u0l);
    split_f16x4(U1, u1h, u1l);
    const uint4 Uh = join(u0h, u1h);   // tokens {4lg+0..3, 16+4lg+0..3} as K=32 B operands
    const uint4 Ul = join(u0l, u1l);
    // S = diag(exp(G_last)) S0 + (k^ exp(G_last - G))^T U
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      Sacc[t] = mfma_f16(kef[t], Ul, Sacc[t]);
      Sacc[t] = mfma_f16(kef[t], Uh, Sacc[t]);
    }
    if constexpr (STATES) {
      // A wave-uniform base plus this lane's byte offset, made opaque here so that the 40
      // store addresses are formed at the stores instead of being kept live across chunks.
      uint32_t lo = static_cast<uint32_t>(4 * lg * DV + col0 + wcol) * 4u;
      __asm__ volatile("" : "+v"(lo));
      uint8_t *up = reinterpret_cast<uint8_t *>(uws + (static_cast<size_t>(slot0 + cidx) * H + h) * C * DV) + lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<float *>(up + i * DV * 4) = U0[i];
        *reinterpret_cast<float *>(up + (SB + i) * DV * 4) = U1[i];
      }
      const int pl = min(t_begin + C * cidx + C - 1, t_end - 1);
      uint8_t *sp = reinterpret_cast<uint8_t *>(states + ((row0 + pl) * H + h) * DK * DV) + lo;
#pragma unroll
      for (int t = 0; t < DK / 16; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<float *>(sp + (16 * t + i) * DV * 4) = Sacc[t][i];
    }
    // O = (q^ exp(G)) S0 + Bqk U
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) acc = mfma_f16(qtf[4 * m + s], Sh[s], acc);
      acc = mfma_f16(bqf[m], Ul, acc);
      acc = mfma_f16(bqlf[m], Uh, acc);
      acc = mfma_f16(bqf[m], Uh, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) ost[(SB * m + 4 * lg + i) * LDO + wcol] = acc[i];
    }
    to_f16();                                    // S0 of the next chunk
  };

  // Step s: helpers stage chunk s+1 (loaded at step s-AHEAD+1), load chunk s+1+AHEAD into
  // the freed register set and write chunk s-1's rows; compute waves run chunk s.  Chunks past the
  // end repeat the last.  The two sides run separate loops with one work-group barrier
  // per step each (nchunks + 1 in all), so their loop-carried registers never overlap.
  // CONV: the value loads run one chunk ahead of the record loads; step s also filters
  // chunk s+1's tile (raw rows written at step s-1), carries its three newest real rows
  // to chunk s+2's area and writes chunk s+2's raw rows there.  One more barrier before
  // the loops puts chunk 0's raw rows in place.
  if (nchunks > 0) {
    if (helper) {
      // Register sets of loaded chunks: two (loads run two steps ahead), or three without the
      // convolution and the in-scan norm.  The helpers' streaming of records and values
      // bounds the scan (alone it takes 262-270 us at T = 8192 against about 225 us for the
      // compute waves alone), but mostly by the paired reads of each record, not by the
      // bytes in flight: three steps ahead gives at most a few per cent, four nothing more.
      constexpr bool DEEP = !CONV && !NORM;
      constexpr int AHEAD = DEEP ? 3 : 2;
      Pre pre0, pre1, pre2;
      load(pre0, 0);
      load(pre1, min(1, last));
      if constexpr (DEEP) load(pre2, min(2, last));
      if constexpr (CONV) {
        const uint32_t tv = static_cast<uint32_t>(min(t_begin + hr, t_end - 1));
        put_raw(0, *reinterpret_cast<const u32x4 *>(vrow + (piece + tv * tok_bytes)));
        if (ht < 24) {
          // row hr of the window before the sequence: its carried input W-4+hr (or zeros)
          const int e = cv.W - 4 + hr;
          u32x4 w = {0u, 0u, 0u, 0u};
          if (cv.init[2] != nullptr && e >= 0)
            w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(cv.init[2]) +
                                                 (static_cast<size_t>(n) * (cv.W - 1) + e) * tok_stride + h * DV +
                                                 col0 + hc8);
          *reinterpret_cast<u32x4 *>(&sm.raw[0][hr][hc8]) = w;
        }
        sync_lds();
        conv_tile(sm.hand[0], 0, pre0.valid);
        carry(0, 1, pre0.valid);
        put_raw(1, pre0.v);                      // chunk 1's raw rows
      }
      stage(sm.hand[0], pre0);
      load(pre0, min(AHEAD, last));
      // NORM: the gate pieces and flags of chunk s-5 in the set of step s's parity
      // (loaded at step s-2); at the start of step s, this tile's sums of squares of
      // chunks s-5 .. s-2
      u32x4 gA{}, gB{};
      uint32_t fA = 0, fB = 0;
      float ssr[kNormLag - 1] = {};
      sync_lds();
      auto hstep = [&](int s, Pre &from, u32x4 &gs, uint32_t &fs) {
        if constexpr (CONV) {
          // the filter's LDS reads go out first, then the record staging and the next loads
          // cover their latency; the filter arithmetic then overlaps the loads
          const uint32_t fvalid = from.valid;
          const ConvRows cr = conv_read((s + 1) & 1, fvalid);
          const u32x4 cw = carry_read((s + 1) & 1, fvalid);
          stage(sm.hand[(s + 1) & 1], from);
          const u32x4 fv = from.v;
          load(from, min(s + 3, last));
          conv_write(sm.hand[(s + 1) & 1], cr, fvalid);
          carry_write(s & 1, cw);
          put_raw(s & 1, fv);                    // chunk s+2's raw rows
        } else {
          stage(sm.hand[(s + 1) & 1], from);
          load(from, min(s + 1 + AHEAD, last));
        }
        float ss = 0.f;
        if (s >= 1) {
          ss = emit(s - 1, sm.ost[(s - 1) % NOST]);
          if constexpr (NORM) publish(s - 1, ss);
        }
        if constexpr (NORM) {
          if (s >= kNormLag) {
            const int c = s - kNormLag;
            emit_y(c, sm.ost[c % NOST], ssr[0] + sm.pss[c & 1][hr], gs, fs);
          }
          load_gate(max(s - (kNormLag - 2), 0), gs, fs);   // unconditional: the load is waited for by count
#pragma unroll
          for (int i = 0; i < kNormLag - 2; ++i) ssr[i] = ssr[i + 1];
          ssr[kNormLag - 2] = ss;
        }
        sync_lds();
      };
      int s = 0;
      if constexpr (DEEP) {
        for (; s + 2 < nchunks; s += 3) {
          hstep(s, pre1, gA, fA);                // chunk s+1 is in pre1, s+2 in pre2, s+3 in pre0
          hstep(s + 1, pre2, gA, fA);
          hstep(s + 2, pre0, gA, fA);
        }
        if (s < nchunks) hstep(s, pre1, gA, fA);
        if (s + 1 < nchunks) hstep(s + 1, pre2, gA, fA);
      } else {
        for (; s + 1 < nchunks; s += 2) {
          hstep(s, pre1, gA, fA);                // chunk s+1 is in pre1, s+2 in pre0
          hstep(s + 1, pre0, gB, fB);
        }
        if (s < nchunks) hstep(s, pre1, gA, fA);
      }
      const float ssl = emit(last, sm.ost[last % NOST]);
      if constexpr (NORM) {
        // y of chunks last-4 .. last.  The partner's sums of chunk last-4 are in LDS
        // (compute wave 0 read them at the last step); the later ones are read here.
        publish(last, ssl);
#pragma unroll
        for (int i = 0; i < kNormLag; ++i) {
          const int c = last - (kNormLag - 1) + i;
          if (c < 0) continue;
          const float own = (i < kNormLag - 1) ? ssr[i] : ssl;
          float other;
          if (i == 0) {
            other = sm.pss[c & 1][hr];
          } else {
            other = partner(c, hr, fetch(c, hr));
            if ((ht & 7) == 0) clear(c, hr);
          }
          u32x4 gt;
          uint32_t fl;
          load_gate(c, gt, fl);
          emit_y(c, sm.ost[c % NOST], own + other, gt, fl);
        }
      }
    } else {
      if constexpr (CONV) sync_lds();
      sync_lds();
      int oi = 0;
      uint64_t xw = 0;                           // NORM, wave 0: the partner's word of chunk s-4
      for (int s = 0; s < nchunks; ++s) {
        if constexpr (NORM) {
          if (wave == 0 && lane < C) {
            if (s >= kNormLag - 1) {
              const int c = s - (kNormLag - 1);
              sm.pss[c & 1][lane] = partner(c, lane, xw);
              clear(c, lane);
            }
            if (s >= kNormLag - 2) xw = fetch(s - (kNormLag - 2), lane);
          }
        }
        products(sm.hand[s & 1], sm.ost[oi], s);
        oi = (oi + 1 == NOST) ? 0 : oi + 1;
        sync_lds();
      }
    }
  }

  if (!helper) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) fin[slab + static_cast<size_t>(16 * t + 4 * lg + i) * DV + col0 + wcol] = Sacc[t][i];
  }
}

template <typename TOut, bool HAS_INIT, bool NORM, bool WRITE_O>
hipError_t launch3(const Args &a, const void *ws, uint64_t *xs, uint32_t *status, hipStream_t st) {
  static_assert(WRITE_O || NORM, "without the norm the head outputs are the only output");
  const int units = a.N * a.H;
  const unsigned grid = static_cast<unsigned>((units + 7) / 8) * 8 * NTILE;
  float *uws = nullptr;
  auto go = [&](auto conv_t, auto states_t) {
    hipLaunchKernelGGL((chunk_scan_kernel<TOut, HAS_INIT, NORM, WRITE_O, decltype(conv_t)::value,
                                          decltype(states_t)::value>),
                       dim3(grid), dim3(NT), 0, st, static_cast<const uint16_t *>(a.v), static_cast<const Rec *>(ws),
                       a.init, a.state, a.cu, static_cast<TOut *>(a.o), static_cast<const uint16_t *>(a.gate),
                       a.norm_w, static_cast<TOut *>(a.y), xs, status, a.eps, a.T, a.H, units, a.conv, a.states_out,
                       uws);
  };
  if constexpr (!NORM && WRITE_O) {
    if (a.states_out) {
      uws = chunk_states_u_area(ws, a.B, a.T, a.H, a.N, a.cu != nullptr);
      go(std::false_type{}, std::true_type{});
      return hipGetLastError();
    }
  }
  if (a.conv.W > 0) go(std::true_type{}, std::false_type{});
  else go(std::false_type{}, std::false_type{});
  return hipGetLastError();
}

template <typename TOut, bool HAS_INIT>
hipError_t launch2(const Args &a, const void *ws, uint64_t *xs, uint32_t *status, hipStream_t st) {
  if (a.states_out) return launch3<TOut, HAS_INIT, false, true>(a, ws, xs, status, st);
  if (!a.y) return launch3<TOut, HAS_INIT, false, true>(a, ws, xs, status, st);
  return a.o ? launch3<TOut, HAS_INIT, true, true>(a, ws, xs, status, st)
             : launch3<TOut, HAS_INIT, true, false>(a, ws, xs, status, st);
}

template <typename TOut>
hipError_t launch1(const Args &a, const void *ws, uint64_t *xs, uint32_t *status, hipStream_t st) {
  return a.init ? launch2<TOut, true>(a, ws, xs, status, st) : launch2<TOut, false>(a, ws, xs, status, st);
}

}  // namespace

bool prefill_mfma_supports(int dk, int dv, int in_bf16) { return in_bf16 && dk == DK && dv == DV; }

// Offsets of tokens within one batch row are 32-bit: T * H * 128 must stay below 2^31.
bool prefill_mfma_fits(long long T, long long H) { return T * H * DK < (1LL << 31); }

hipError_t launch_chunk_scan(const Args &a, const void *ws, hipStream_t st) {
  if (a.N * static_cast<long long>(a.H) <= 0) return hipSuccess;
  uint64_t *xs = chunk_exchange_words(ws, a.B, a.T, a.H, a.N, a.cu != nullptr);
  uint32_t *status = chunk_status_word(ws, a.B, a.T, a.H, a.N, a.cu != nullptr);
  return a.out_bf16 ? launch1<uint16_t>(a, ws, xs, status, st) : launch1<float>(a, ws, xs, status, st);
}

}  // namespace kda
