// Chunk preparation for the bf16 chunked prefill (head size 128, 32-token chunks).
//
// The chunked form of the KDA recurrence (nnterp Kimi-Linear page, Notes, "Loading" and
// the KDA paragraph; section 04 docstring) splits every chunk's work into a part that
// needs the incoming state and a part that does not.  This kernel does the second part
// for every (sequence, head, chunk) at once.  With G the running sum of g over the chunk
// (per key channel), k^ and q^ the normalised key and query (q^ also scaled):
//     A[s][j]   = beta_s sum_c k^_sc k^_jc exp(G_sc - G_jc)      (j < s)
//     Bqk[r][s] = sum_c q^_rc k^_sc exp(G_rc - G_sc)              (s <= r)
//     W         = (I + A)^-1 diag(beta)
// and the decayed operands k^ exp(G), q^ exp(G), k^ exp(G_last - G), exp(G_last).  All of
// it goes to the chunk's record (kda_chunk.h) in the scan kernel's MFMA operand order, so
// the scan only has to run U = W (V - (k^ exp(G)) S0), O = (q^ exp(G)) S0 + Bqk U and the
// state carry.
//
// Work-group: one (sequence, head, chunk), two waves; wave m owns the 16-token sub-block
// m.  Each lane holds its token's channels in MFMA operand order (lane 16 lg + r: token r
// of the sub-block, channels 32 s + kidx(lg, e) of K block s): g is loaded that way, q and
// k as 16 contiguous bytes per K block that one row swap puts in that order, so
//   * G is a prefix sum over the 16 lanes of a row (DPP row shifts), in log2 units, and
//     every decay factor is one exp2 of a difference of running sums;
//   * the decayed key and query fragments go from registers straight to the record;
//   * the intra-chunk products take both operands from registers (the off-diagonal block
//     reads sub-block 0's operand from LDS), with the operands swapped where the record
//     wants the transposed product;
//   * k^ exp(G_last - G) is transposed to its channel-major fragments by a matrix-core
//     product with a 0/1 selection operand (exact: one nonzero term per output).
// Decay factoring for the intra-chunk products: exp(G_s - G_j) is split into a row and a
// column factor around a reference token, the 8th token of the sub-block for a diagonal
// block (|exponent| <= 8 * 5 = 40 when g >= -5, bf16 operands; Bqk's diagonal blocks take
// bf16 hi + lo parts, three products), the sub-block boundary for the off-diagonal block
// (both factors <= 1, fp16).  The diagonal blocks of I + A are inverted by forward
// substitution; the off-diagonal block of W comes from two fp32 matrix-core products.
#include <type_traits>

#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int NT = 128;

struct Shared {
  float gx[2][2][DK];      // per sub-block: running sum of g (log2) at its 8th and its last token
  float sb[C];             // beta (0 for padding)
  u32x4 kof0[4][64];       // sub-block 0: fp16 k^ exp(G_15 - G) fragments, one per K block
  float at[2][SB][SB + 4]; // A's diagonal blocks, transposed: at[a][j][s] = A[16a+s][16a+j]
  float tm[2][SB][SB + 1]; // (I + A_aa)^-1
  float a10[SB][SB + 1];   // A(1,0)
  float pp[SB][SB + 1];    // A(1,0) (I + A_00)^-1
  u32x2 kx[2][4][64];      // k^ exp(G_last - G) fragment halves handed to the other wave
};
static_assert(sizeof(Shared) <= 20 * 1024, "LDS per work-group");

constexpr int kNoInput = -0x40000000;   // a window entry that reads zeros

// G_HEAD: g holds one decay per (token, head), shared by every key channel.
// CONV: q and k are the raw projections; the kernel runs their short convolution (cv).
template <bool HAS_MASK, bool G_HEAD, bool CONV>
__global__ void __launch_bounds__(NT)
chunk_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const float *__restrict__ g, const float *__restrict__ beta,
                  const int32_t *__restrict__ cu, const uint8_t *__restrict__ mask,
                  Rec *__restrict__ ws, uint64_t *__restrict__ xs, uint32_t *__restrict__ status, int T, int H,
                  int N, float scale, int use_l2, ConvIn cv) {
  // CONV: the filtered q (0) and k (1) of the chunk, fp32 [token][channel], in the space of
  // the shared arrays below (they are first written after the last read of these)
  union SmemU {
    Shared s;
    float cst[CONV ? 2 : 1][CONV ? C : 1][DK + 4];
  };
  __shared__ SmemU smu;
  Shared &sh = smu.s;
  auto &cst = smu.cst;
  const int tid = threadIdx.x, lane = tid & 63;
  if (blockIdx.x == 0 && tid == 0) *status = 0u;   // no wait of the coming scan has run out yet
  const int m = __builtin_amdgcn_readfirstlane(tid >> 6);   // sub-block of this wave
  const int r = lane & 15, lg = lane >> 4;

  // ---------------------------------------------------------------- locate the chunk
  const int h = static_cast<int>(blockIdx.x) % H;
  const int slot = static_cast<int>(blockIdx.x) / H;
  int b, t_begin, t_end, c, nseq;
  if (cu) {
    // largest n whose first slot is <= slot (first slots increase with n)
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
  if (c < 0 || c * C >= t_end - t_begin) return;   // no chunk in this slot (whole work-group)
  const int c0 = t_begin + c * C;
  Rec *rec = ws + static_cast<size_t>(slot) * H + h;
  // clear the chunk's words of the scan's norm exchange (2 tiles x 32 tokens)
  if (tid < 32) reinterpret_cast<u32x4 *>(xs + (static_cast<size_t>(slot) * H + h) * 64)[tid] = u32x4{0u, 0u, 0u, 0u};
  const size_t row0 = static_cast<size_t>(b) * T;
  // this lane's token (operand order, see below), its decays and its write strength (CONV:
  // loaded first, so that their latency overlaps the filter work)
  const int tok = c0 + SB * m + r;
  const int tcl = min(tok, t_end - 1);
  const int off = tcl * (H * DK) + h * DK + 4 * lg;
  const float *gp = G_HEAD ? g + (row0 + tcl) * H + h : g + row0 * H * DK + off;
  f32x4 G[4][2];
  float bt;
  auto load_g = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        if constexpr (G_HEAD) {
          const float gs = *gp;
          G[s][hh] = f32x4{gs, gs, gs, gs};
        } else {
          G[s][hh] = *reinterpret_cast<const f32x4 *>(gp + 32 * s + 16 * hh);
        }
      }
    bt = beta[(row0 + tcl) * H + h];
  };
  if constexpr (CONV) load_g();

  // ---------------------------------------------------------------- fused short convolution
  // CONV (Kimi-K3 atlas, KDA layer page, kda-init code: a causal ShortConvolution with SiLU
  // on each projection; nnterp Kimi-Linear page, Notes: the layer carries its last inputs
  // outside the state).  Wave 0 filters q and wave 1 k over the chunk; lane (tg, cg) takes
  // channels 8 cg .. 8 cg + 7 of tokens 8 tg .. 8 tg + 7.  Its window starts with the three
  // newest real tokens before its first one (padding never enters it), reaching back
  // before the chunk and then into the carried inputs of the sequence, and slides over its
  // real tokens.  The outputs go to LDS in fp32, where the loads below take them in
  // operand order instead of the inputs (no bf16 rounding: a filtered value lying at a
  // bf16 rounding midpoint would otherwise round either way depending on the last bits of
  // its fp32 computation, and the recurrence can be sensitive to one unit of a key).
  if constexpr (CONV) {
    const int cg = lane & 15, tg = lane >> 4;
    const int W = cv.W;
    const uint16_t *xin = m == 0 ? q : k;
    const uint16_t *xinit = static_cast<const uint16_t *>(m == 0 ? cv.init[0] : cv.init[1]);
    const size_t dstride = static_cast<size_t>(H) * DK;             // elements between tokens
    const size_t chan = static_cast<size_t>(h) * DK + 8 * cg;
    // the chunk's real tokens (bit i: token c0 + i)
    uint32_t vbits;
    {
      const int tt = c0 + (lane & 31);
      bool ok = tt < t_end;
      if constexpr (HAS_MASK) ok = ok && mask[row0 + min(tt, t_end - 1)] != 0;
      vbits = static_cast<uint32_t>(__ballot(ok));
    }
    // Sources of the three newest inputs before the chunk, newest first: a token of the
    // row (>= 0), carried input j (-1 - j), or zeros (kNoInput).
    int p0 = kNoInput, p1 = kNoInput, p2 = kNoInput, cnt = 0;
    auto push = [&](int src) {   // selects, not branches: kept in registers
      p0 = cnt == 0 ? src : p0;
      p1 = cnt == 1 ? src : p1;
      p2 = cnt == 2 ? src : p2;
      ++cnt;
    };
    if constexpr (HAS_MASK) {
      // 64 tokens at a time, back from the chunk start, until three real ones are found
      for (int base = c0 - 1; base >= t_begin && cnt < 3; base -= 64) {
        const int t = base - lane;
        const bool ok = t >= t_begin && mask[row0 + max(t, 0)] != 0;
        uint64_t bal = __ballot(ok);
        while (bal != 0 && cnt < 3) {
          push(base - __builtin_ctzll(bal));
          bal &= bal - 1;
        }
      }
    } else {
#pragma unroll
      for (int j = 1; j <= 3; ++j)
        if (c0 - j >= t_begin) push(c0 - j);
    }
    // the j-th newest carried input is entry W-1-j of the sequence's carried inputs
    for (int j = 1; j <= 3 && cnt < 3; ++j) push(xinit != nullptr && j <= W - 1 ? -1 - (W - 1 - j) : kNoInput);
    // this lane's window before token c0 + 8 tg: real tokens of the chunk before it, then p
    uint32_t below = vbits & ((1u << (8 * tg)) - 1u);
    auto pop_top = [&]() -> int {
      if (below == 0u) return -1;
      const int i = 31 - __builtin_clz(below);
      below &= ~(1u << i);
      return i;
    };
    const int i0 = pop_top(), i1 = pop_top(), i2 = pop_top();
    const int nin = (i0 >= 0) + (i1 >= 0) + (i2 >= 0);
    const int s0 = nin >= 1 ? c0 + i0 : p0;
    const int s1 = nin >= 2 ? c0 + i1 : (nin == 1 ? p0 : p1);
    const int s2 = nin >= 3 ? c0 + i2 : (nin == 2 ? p0 : (nin == 1 ? p1 : p2));
    auto load_src = [&](int src) -> u32x4 {
      if (src >= 0) return *reinterpret_cast<const u32x4 *>(xin + (row0 + src) * dstride + chan);
      if (src == kNoInput) return u32x4{0u, 0u, 0u, 0u};
      return *reinterpret_cast<const u32x4 *>(xinit + (static_cast<size_t>(nseq) * (W - 1) + (-1 - src)) * dstride + chan);
    };
    u32x4 rows[8];
    const int tt0 = c0 + 8 * tg;
#pragma unroll
    for (int i = 0; i < 8; ++i) rows[i] = load_src(min(tt0 + i, t_end - 1));
    const u32x4 w2 = load_src(s0), w1 = load_src(s1), w0 = load_src(s2);
    float tap[8][4];
    const float *wp = (m == 0 ? cv.w[0] : cv.w[1]) + chan * W;
    if (W == 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 t4 = *reinterpret_cast<const f32x4 *>(wp + 4 * i);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tap[i][jj] = t4[jj];
      }
    } else {
      // right-aligned: slot jj holds weight jj - (4 - W)
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) tap[i][jj] = jj >= 4 - W ? wp[i * W + jj - (4 - W)] : 0.f;
    }
    auto unpack = [](u32x4 w, float (&x)[8]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = lo_bf16(w[e]);
        x[2 * e + 1] = hi_bf16(w[e]);
      }
    };
    float h0[8], h1[8], h2[8];   // the window, oldest first
    unpack(w0, h0);
    unpack(w1, h1);
    unpack(w2, h2);
    auto filter = [&](auto all_real) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = decltype(all_real)::value || ((vbits >> (8 * tg + i)) & 1u);
        float x[8], z[8];
        unpack(rows[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // all four taps (a narrower filter's older taps are zero and its window rows
          // finite): no per-element selects on the width
          z[e] = conv_z4(make_float4(tap[e][0], tap[e][1], tap[e][2], tap[e][3]), h0[e], h1[e], h2[e], x[e]);
          if (cv.silu) z[e] = silu_act(z[e]);
          z[e] = ok ? z[e] : 0.f;
          h0[e] = ok ? h1[e] : h0[e];
          h1[e] = ok ? h2[e] : h1[e];
          h2[e] = ok ? x[e] : h2[e];
        }
        *reinterpret_cast<f32x4 *>(&cst[m][8 * tg + i][8 * cg]) = f32x4{z[0], z[1], z[2], z[3]};
        *reinterpret_cast<f32x4 *>(&cst[m][8 * tg + i][8 * cg + 4]) = f32x4{z[4], z[5], z[6], z[7]};
      }
    };
    // a wave whose lanes' tokens are all real (no padding, not past the end) skips the selects
    if (vbits == 0xffffffffu) filter(std::true_type{});
    else filter(std::false_type{});
    sync_lds();
  }

  // ---------------------------------------------------------------- load (operand order)
  bool valid = tok < t_end;
  if constexpr (HAS_MASK) valid = valid && mask[row0 + tcl] != 0;
  // q and k: one 16-byte load per K block, lane group lg reading channels 32 s + 8 L ..
  // 32 s + 8 L + 7 with L = (0, 2, 1, 3)[lg], then a row swap (operand_halves)
  const int off16 = tcl * (H * DK) + h * DK + 8 * (((lg & 1) << 1) | (lg >> 1));
  const uint16_t *kp = k + row0 * H * DK + off16;
  const uint16_t *qp = q + row0 * H * DK + off16;
  u32x2 kr[4][2], qr[4][2];
  u32x4 kw[4], qw[4];
  // CONV: the filtered k and q in operand order, fp32: slot e of K block s is channel
  // 32 s + kidx(lg, e) (read straight from LDS in that order)
  f32x4 kf[CONV ? 4 : 1][2], qf[CONV ? 4 : 1][2];
  if constexpr (CONV) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        kf[s][hh] = *reinterpret_cast<const f32x4 *>(&cst[1][SB * m + r][32 * s + 16 * hh + 4 * lg]);
        qf[s][hh] = *reinterpret_cast<const f32x4 *>(&cst[0][SB * m + r][32 * s + 16 * hh + 4 * lg]);
      }
    sync_lds();   // every read of the filtered values is done before the shared arrays are written
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kw[s] = *reinterpret_cast<const u32x4 *>(kp + 32 * s);
      qw[s] = *reinterpret_cast<const u32x4 *>(qp + 32 * s);
    }
    load_g();
  }
  if constexpr (!CONV) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      operand_halves(kw[s], kr[s][0], kr[s][1]);
      operand_halves(qw[s], qr[s][0], qr[s][1]);
    }
  }

  // ---------------------------------------------------------------- norms, running sums
  // Padding and tokens past the end act as no-ops: zero key, query, beta and decay.
  float nk, nq;
  {
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          float k0, k1, q0, q1;
          if constexpr (CONV) {
            k0 = kf[s][hh][2 * w]; k1 = kf[s][hh][2 * w + 1];
            q0 = qf[s][hh][2 * w]; q1 = qf[s][hh][2 * w + 1];
          } else {
            k0 = lo_bf16(kr[s][hh][w]); k1 = hi_bf16(kr[s][hh][w]);
            q0 = lo_bf16(qr[s][hh][w]); q1 = hi_bf16(qr[s][hh][w]);
          }
          ssk += k0 * k0 + k1 * k1;
          ssq += q0 * q0 + q1 * q1;
        }
    ssk = col_sum4(ssk);
    ssq = col_sum4(ssq);
    nk = valid ? (use_l2 ? rsqrtf(ssk + kL2Eps) : 1.f) : 0.f;
    nq = valid ? (use_l2 ? rsqrtf(ssq + kL2Eps) : 1.f) * scale : 0.f;
  }
  const float gsc = valid ? kLog2e : 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) G[s][hh][i] = row_prefix(G[s][hh][i] * gsc);
  if (r == 7 || r == 15) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<f32x4 *>(&sh.gx[m][r >> 3][32 * s + 16 * hh + 4 * lg]) = G[s][hh];
  }
  if (lg == 0) sh.sb[SB * m + r] = valid ? bt : 0.f;
  auto kval = [&](int s, int e) {
    if constexpr (CONV) {
      return kf[s][e >> 2][e & 3] * nk;
    } else {
      const uint32_t w = kr[s][e >> 2][(e >> 1) & 1];
      return (e & 1 ? hi_bf16(w) : lo_bf16(w)) * nk;
    }
  };
  auto qval = [&](int s, int e) {
    if constexpr (CONV) {
      return qf[s][e >> 2][e & 3] * nq;
    } else {
      const uint32_t w = qr[s][e >> 2][(e >> 1) & 1];
      return (e & 1 ? hi_bf16(w) : lo_bf16(w)) * nq;
    }
  };
  if (m == 0) {
    // sub-block 0's off-diagonal operand k^ exp(G_15 - G), needed by the other wave
    wave_sync_lds();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&sh.gx[0][1][32 * s + 16 * hh + 4 * lg]);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * hh + i] = kval(s, 4 * hh + i) * fast_exp2(t0[i] - G[s][hh][i]);
      }
      sh.kof0[s][lane] = u32x4{pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]),
                               pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7])};
    }
  }
  sync_lds();

  // ---------------------------------------------------------------- operands and products
  // Selection operands for the transpose of k^ exp(G_last - G): slot e of lane (lg, n) is 1
  // when kidx(lg, e) = n (first half of the K block) or 16 + n (second half).
  const uint32_t one = (lg == (r >> 2)) ? (0x3C00u << (16 * (r & 1))) : 0u;
  const bool wsel = (r & 2) != 0;
  const u32x4 id0 = {wsel ? 0u : one, wsel ? one : 0u, 0u, 0u};
  const u32x4 id1 = {0u, 0u, wsel ? 0u : one, wsel ? one : 0u};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 accA = zero, accB = zero, accA10 = zero, accB10 = zero;
  u32x2 kown[4];   // this wave's halves of its own four transposed fragments
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float rk[8], ck[8], rq[8], kb[8], qt[8], ke[8], k1[8], q1[8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ch = 32 * s + 16 * hh + 4 * lg;
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(&sh.gx[m][0][ch]);
      const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&sh.gx[0][1][ch]);
      const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&sh.gx[1][1][ch]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * hh + i;
        const float gl = G[s][hh][i];
        const float kk = kval(s, e), qq = qval(s, e);
        const float d1 = gl - gm[i];
        const float e1 = fast_exp2(d1), e1n = fast_exp2(-d1);
        // chunk-relative G and the distance to the chunk's last token
        const float gc = m ? gl + t0[i] : gl;
        const float tail = m ? t1[i] - gl : (t0[i] + t1[i]) - gl;
        const float eg = fast_exp2(gc), el = fast_exp2(tail);
        rk[e] = kk * e1;
        rq[e] = qq * e1;
        ck[e] = kk * e1n;
        kb[e] = kk * eg;
        qt[e] = qq * eg;
        ke[e] = kk * el;
        if (m) {
          const float e2 = fast_exp2(gl);   // exp(G - G_15) in sub-block 1
          k1[e] = kk * e2;
          q1[e] = qq * e2;
        }
      }
    }
    u32x4 rkb, ckh, ckl, rqh, rql, kbf, qtf, kef;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t h0, l0, h1, l1;
      rkb[w] = pack_bf16x2(rk[2 * w], rk[2 * w + 1]);
      split_bf16x2(ck[2 * w], ck[2 * w + 1], h0, l0);
      split_bf16x2(rq[2 * w], rq[2 * w + 1], h1, l1);
      ckh[w] = h0; ckl[w] = l0; rqh[w] = h1; rql[w] = l1;
      kbf[w] = pack_f16x2(kb[2 * w], kb[2 * w + 1]);
      qtf[w] = pack_f16x2(qt[2 * w], qt[2 * w + 1]);
      kef[w] = pack_f16x2(ke[2 * w], ke[2 * w + 1]);
    }
    reinterpret_cast<u32x4 *>(rec->kb[4 * m + s])[lane] = kbf;
    reinterpret_cast<u32x4 *>(rec->qt[4 * m + s])[lane] = qtf;
    // A_mm (rows s, cols j) and Bqk_mm transposed (rows key token, cols query token)
    accA = mma_bf16(rkb, ckh, accA);
    accB = mma_bf16(ckl, rqh, accB);
    accB = mma_bf16(ckh, rql, accB);
    accB = mma_bf16(ckh, rqh, accB);
    if (m) {
      const u32x4 ko = sh.kof0[s][lane];
      const u32x4 k14 = {pack_f16x2(k1[0], k1[1]), pack_f16x2(k1[2], k1[3]),
                         pack_f16x2(k1[4], k1[5]), pack_f16x2(k1[6], k1[7])};
      const u32x4 q14 = {pack_f16x2(q1[0], q1[1]), pack_f16x2(q1[2], q1[3]),
                         pack_f16x2(q1[4], q1[5]), pack_f16x2(q1[6], q1[7])};
      accA10 = mma_f16(k14, ko, accA10);    // A(1,0) without beta
      accB10 = mma_f16(ko, q14, accB10);    // Bqk(1,0) transposed
    }
    // transposed fragments 2s and 2s + 1: rows = channels, K = this wave's tokens
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 t = mma_f16(kef, j ? id1 : id0, zero);
      const u32x2 half = {pack_f16x2(t[0], t[1]), pack_f16x2(t[2], t[3])};
      const int tile = 2 * s + j;
      if ((tile >> 2) == m) kown[tile & 3] = half;
      else sh.kx[m][tile & 3][lane] = half;
    }
  }

  // ---------------------------------------------------------------- intra-chunk blocks
  const f32x4 bm = *reinterpret_cast<const f32x4 *>(&sh.sb[SB * m + 4 * lg]);   // beta of rows 4lg + i
  {
    // accA[i] = A'[4 lg + i][r]: A[s][j] = beta_s A'[s][j] for j < s, stored at[j][s]
    f32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (r < 4 * lg + i) ? bm[i] * accA[i] : 0.f;
    *reinterpret_cast<f32x4 *>(&sh.at[m][r][4 * lg]) = w;
    // accB[i] = Bqk[r][4 lg + i] of this sub-block (query row r, key column 4 lg + i)
    f32x4 bd;
#pragma unroll
    for (int i = 0; i < 4; ++i) bd[i] = (4 * lg + i <= r) ? accB[i] : 0.f;
    // hi + lo parts: the outputs are often much smaller than the two terms they are the
    // sum of (q^ exp(G) S0 and Bqk U), so Bqk's own rounding must stay far below fp16's
    u32x2 diag, diagl, left = {0u, 0u}, leftl = {0u, 0u};
    split4(bd, diag, diagl);
    if (m) split4(accB10, left, leftl);
    // row r of bq[m]: slots 0-3 = key tokens 4 lg + i, slots 4-7 = key tokens 16 + 4 lg + i
    reinterpret_cast<u32x4 *>(rec->bq[m])[lane] = m ? cat(left, diag) : cat(diag, u32x2{0u, 0u});
    reinterpret_cast<u32x4 *>(rec->bqlo[m])[lane] = m ? cat(leftl, diagl) : cat(diagl, u32x2{0u, 0u});
    if (m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.a10[4 * lg + i][r] = bm[i] * accA10[i];
    }
  }
  wave_sync_lds();
  {
    // column r of (I + A_mm)^-1 by forward substitution (lanes 16..63 repeat lanes 0..15)
    float tc[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) tc[i] = (i == r) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < SB - 1; ++j) {
      const float *col = sh.at[m][j];
#pragma unroll
      for (int i = j + 1; i < SB; ++i) tc[i] -= col[i] * tc[j];
    }
    if (lg == 0) {
#pragma unroll
      for (int i = 0; i < SB; ++i) sh.tm[m][i][r] = tc[i];
    }
  }
  sync_lds();

  // ---------------------------------------------------------------- W, the transposed keys, exp(G_last)
  // W = (I + A)^-1 diag(beta) = [[T0 B0, 0], [-T1 A10 T0 B0, T1 B1]], T_a = (I + A_aa)^-1.
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const u32x2 other = sh.kx[1 - m][tt][lane];
    reinterpret_cast<u32x4 *>(rec->ket[4 * m + tt])[lane] = m ? cat(other, kown[tt]) : cat(kown[tt], other);
  }
  // lane (lg, r) holds row r of W's block, key tokens 4 lg + i of the block
  const f32x4 bc = *reinterpret_cast<const f32x4 *>(&sh.sb[SB * m + 4 * lg]);
  f32x4 wd;
#pragma unroll
  for (int i = 0; i < 4; ++i) wd[i] = sh.tm[m][r][4 * lg + i] * bc[i];
  u32x2 wdh, wdl;
  split4(wd, wdh, wdl);
  if (m == 0) {
    reinterpret_cast<u32x2 *>(rec->w00)[lane] = wdh;
    reinterpret_cast<u32x2 *>(rec->w00lo)[lane] = wdl;
    if (r < 8) {   // exp(G_last) of channels 32 s + 16 hh + 4 lg + i, (s, hh) = (r / 2, r % 2)
      const int ch = 32 * (r >> 1) + 16 * (r & 1) + 4 * lg;
      const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&sh.gx[0][1][ch]);
      const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&sh.gx[1][1][ch]);
      f32x4 ec;
#pragma unroll
      for (int i = 0; i < 4; ++i) ec[i] = fast_exp2(t0[i] + t1[i]);
      *reinterpret_cast<f32x4 *>(&rec->ec[ch]) = ec;
    }
    const int tt = c0 + (lane & 31);
    bool v = tt < t_end;
    if constexpr (HAS_MASK) v = v && mask[row0 + min(tt, t_end - 1)] != 0;
    const uint64_t bal = __ballot(v);
    if (lane == 0) rec->valid = static_cast<uint32_t>(bal);
  } else {
    // P = A10 T0, then W10^T = -diag(beta0) P^T T1^T (rows = tokens of sub-block 0)
    f32x4 p = zero;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) p = mfma_f32k4(sh.a10[r][4 * kb4 + lg], sh.tm[0][4 * kb4 + lg][r], p);
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.pp[4 * lg + i][r] = p[i];
    wave_sync_lds();
    f32x4 wt = zero;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) wt = mfma_f32k4(sh.pp[4 * kb4 + lg][r], sh.tm[1][r][4 * kb4 + lg], wt);
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&sh.sb[4 * lg]);
    f32x4 w10;   // W10[r][4 lg + i]
#pragma unroll
    for (int i = 0; i < 4; ++i) w10[i] = -wt[i] * b0[i];
    u32x2 wlh, wll;
    split4(w10, wlh, wll);
    reinterpret_cast<u32x4 *>(rec->w1)[lane] = cat(wlh, wdh);
    reinterpret_cast<u32x4 *>(rec->w1lo)[lane] = cat(wll, wdl);
  }
}

}  // namespace

// Workspace of the bf16 chunked prefill: one record per (slot, head), then the scan's
// norm-exchange words, 64 per (slot, head).
size_t chunk_prep_workspace_bytes(long long B, long long T, long long H, long long N, bool packed) {
  return static_cast<size_t>(num_slots(B, T, N, packed) * H) * (kRecBytes + kExchangeBytes) + kStatusBytes;
}

uint64_t *chunk_exchange_words(const void *ws, long long B, long long T, long long H, long long N, bool packed) {
  const size_t rec_bytes = static_cast<size_t>(num_slots(B, T, N, packed) * H) * kRecBytes;
  return reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(const_cast<void *>(ws)) + rec_bytes);
}

uint32_t *chunk_status_word(const void *ws, long long B, long long T, long long H, long long N, bool packed) {
  const size_t bytes = static_cast<size_t>(num_slots(B, T, N, packed) * H) * (kRecBytes + kExchangeBytes);
  return reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(const_cast<void *>(ws)) + bytes);
}

hipError_t launch_chunk_prep(const Args &a, void *ws, hipStream_t st) {
  const long long slots = num_slots(a.B, a.T, a.N, a.cu != nullptr);
  const long long blocks = slots * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k);
  Rec *rec = static_cast<Rec *>(ws);
  uint64_t *xs = chunk_exchange_words(ws, a.B, a.T, a.H, a.N, a.cu != nullptr);
  uint32_t *status = chunk_status_word(ws, a.B, a.T, a.H, a.N, a.cu != nullptr);
  const dim3 grid(static_cast<unsigned>(blocks));
  auto go = [&](auto mask_t, auto ghead_t, auto conv_t) {
    hipLaunchKernelGGL((chunk_prep_kernel<decltype(mask_t)::value, decltype(ghead_t)::value, decltype(conv_t)::value>),
                       grid, dim3(NT), 0, st, q, k, a.g, a.beta, a.cu, a.mask, rec, xs, status, a.T, a.H, a.N,
                       a.scale, a.use_l2, a.conv);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto go2 = [&](auto mask_t, auto ghead_t) {
    if (a.conv.W > 0) go(mask_t, ghead_t, T_{});
    else go(mask_t, ghead_t, F_{});
  };
  if (a.g_head) {
    if (a.mask) go2(T_{}, T_{});
    else go2(F_{}, T_{});
  } else {
    if (a.mask) go2(T_{}, F_{});
    else go2(F_{}, F_{});
  }
  return hipGetLastError();
}

}  // namespace kda
