// Token-by-token KDA step (the decode kernel).
//
// Per head the state S[dk][dv] (fp32) is read once, advanced over the call's tokens
// and written back in place.  For each token (nnterp Kimi-Linear page, Notes, section
// on KDA decaying each key channel; section 04 docstring):
//     S' = diag(exp(g)) S                    decay every key channel first
//     r  = S'^T k,  u = beta (v - r)         delta-rule correction
//     S  = S' + k u^T
//     o  = S^T q = S'^T q + u (k . q)        one pass: both reductions read S'
// with k, q L2-normalised and q scaled by 1/sqrt(dk).
//
// Layout: one work-group per (batch row, head) slab, or, with few slabs and several
// tokens, per 16-column tile of one (value columns are independent in the recurrence:
// each column's update needs only k, q and its own column).  Thread (cg, rg) owns the
// four value columns 4cg..4cg+3 of the tile, key rows rg, rg+RG, rg+2RG, ... so a wave's
// float4 loads cover whole state row pieces (coalesced) and the slab lives in registers.
// The two column reductions (S'^T k, S'^T q) run over lanes with DPP moves, then over
// waves through LDS.  Column tiles load each token's inputs two tokens ahead.  This
// kernel is HBM-bound: at B=64, H=96, d=128 it moves 805 MB of state per step and does
// 0.86 flop per byte.
//
// With `states` set it also stores the state after every token ([B, T, H, dk, dv]; a
// padding token stores the carried state): the per-token states that the pages read by
// running a prompt through the token-by-token kernel (nnterp Kimi-Linear page, support()
// table, the 'states' row, and Notes, "Loading").
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// DVW: value columns per work-group (D: whole slab; the fused norm needs whole rows).
// STATES: also store the state after every token into `states`.
// CONV: q, k and v are the raw projections; the kernel runs their short convolution (cv)
// token by token from each row's carried inputs and, for whole slabs, writes the carried
// inputs after the call.
template <int D, int DVW, int RPT, typename TIn, typename TOut, bool NORM, bool STATES, bool CONV>
__global__ void __launch_bounds__((D / RPT) * (DVW / 4))
recurrent_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
                 const float *__restrict__ g, const float *__restrict__ beta,
                 float *__restrict__ state, const uint8_t *__restrict__ mask,
                 TOut *__restrict__ o, const TIn *__restrict__ gate,
                 const float *__restrict__ norm_w, TOut *__restrict__ y,
                 int T, int H, float scale, int use_l2, float eps, int g_head, float *__restrict__ states,
                 ConvIn cv) {
  constexpr int CG = DVW / 4;        // column groups (float4 each)
  constexpr int RG = D / RPT;        // row groups
  constexpr int NT = RG * CG;
  constexpr int NW = NT / 64;
  constexpr int NTILE = D / DVW;     // work-groups per slab
  static_assert(NT % 64 == 0 && 64 % CG == 0 && D % DVW == 0, "thread layout");
  static_assert(!NORM || DVW == D, "the fused norm needs whole rows");
  constexpr int RL = 64 / CG;        // consecutive lanes of a wave sharing a column group
  constexpr int EPL = (D + 63) / 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Lane l of wave w: column group l / RL, row group w * RL + l % RL, so a column's
  // partial sums over a wave's rows meet in RL consecutive lanes (DPP reach).
  const int cg = lane / RL, rg = wave * RL + lane % RL;
  const int slab = blockIdx.x / NTILE;
  const int col0 = (blockIdx.x % NTILE) * DVW;
  const int b = slab / H, h = slab % H;
  float *S = state + static_cast<size_t>(slab) * D * D + col0;

  // Token inputs (normalised k, q, decay factors; k.q, beta, the valid flag) and the
  // waves' partial column sums.  Column tiles keep three input sets and two sum sets in
  // flight (see the token loop below); whole slabs one of each.
  constexpr bool PF = DVW < D;
  constexpr int NB = PF ? 3 : 1, NR = PF ? 2 : 1;
  __shared__ float s_k[NB][D], s_q[NB][D], s_e[NB][D];
  __shared__ float s_red[NR][NW][2][DVW];
  __shared__ float s_scal[NB][4];

  // CONV: the filtered v of the tile's columns per input set; the filter windows (the
  // three newest real inputs, oldest first) of q, k (D channels) and v (the tile's DVW), raw
  // in the input dtype; the taps [channel][W] of the head's q, k and of the tile's v.  Only
  // wave 0 reads and writes the windows and taps.
  constexpr int NB_ = DVW < D ? 3 : 1;
  __shared__ float s_v[CONV ? NB_ : 1][CONV ? DVW : 1];
  __shared__ __attribute__((aligned(16))) TIn s_wq[CONV ? 3 : 1][CONV ? D : 1];
  __shared__ __attribute__((aligned(16))) TIn s_wk[CONV ? 3 : 1][CONV ? D : 1];
  __shared__ __attribute__((aligned(16))) TIn s_wv[CONV ? 3 : 1][CONV ? DVW : 1];
  __shared__ __attribute__((aligned(16))) float4 s_tq[CONV ? D : 1], s_tk[CONV ? D : 1], s_tv[CONV ? DVW : 1];
  const size_t ch_stride = static_cast<size_t>(H) * D;            // channels of a projection
  // element of window row jj (0..2, oldest first) of channel ch in a carried-input array
  auto carried = [&](int jj, size_t ch) {
    return (static_cast<size_t>(b) * (cv.W - 1) + (cv.W - 4 + jj)) * ch_stride + ch;
  };
  if constexpr (CONV) {
    // Wave 0 copies the taps and the carried inputs of row b into LDS with direct
    // global-to-LDS loads, issued just before its state loads: they hold no registers and
    // arrive with the state.  Data loaded this way is not covered by the compiler's own
    // waits, so wave 0 waits for all its loads (conv_ready) before it reads any of it.
    // Taps are kept four wide: a narrower filter's are right-aligned with zeros in front,
    // and the window rows they meet are zero, so the filter runs without width branches.
    if (wave == 0) {
      const int W = cv.W;
      // bytes: a multiple of 16; source and destination 16-byte aligned
      auto copy_lds = [&](const void *src, void *dst, int bytes) {
        // a wave-uniform base (scalar registers) plus one per-lane offset; the builtin
        // returns a signed int, so each half is taken back as unsigned before widening
        // (a sign-extended low half would set the address's upper bits)
        const uint64_t a = reinterpret_cast<uint64_t>(src);
        const uint32_t ahi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
        const uint32_t alo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu)));
        const char *base = reinterpret_cast<const char *>((static_cast<uint64_t>(ahi) << 32) | alo);
        for (int off = 0; off < bytes; off += 1024)
          if (lane * 16 < bytes - off)
            __builtin_amdgcn_global_load_lds(base + off + lane * 16,
                                             (__attribute__((address_space(3))) void *)(static_cast<char *>(dst) + off),
                                             16, 0, 0);
      };
      const float *wsrc[3] = {cv.w[0] + static_cast<size_t>(h) * D * W, cv.w[1] + static_cast<size_t>(h) * D * W,
                              cv.w[2] + (static_cast<size_t>(h) * D + col0) * W};
      float4 *tdst[3] = {s_tq, s_tk, s_tv};
      // the taps as stored ([channel][W]); a narrower filter's are spread to four wide in
      // place once they have arrived (conv_ready)
#pragma unroll
      for (int x = 0; x < 3; ++x) copy_lds(wsrc[x], tdst[x], (x == 2 ? DVW : D) * W * 4);
#pragma unroll
      for (int x = 0; x < 3; ++x) {
        const TIn *init = static_cast<const TIn *>(x == 0 ? cv.init[0] : (x == 1 ? cv.init[1] : cv.init[2]));
        const int nch = x == 2 ? DVW : D;
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) {
          TIn *row = x == 0 ? s_wq[jj] : (x == 1 ? s_wk[jj] : s_wv[jj]);
          if (init != nullptr && jj >= 4 - W) {
            copy_lds(init + carried(jj, static_cast<size_t>(h) * D + (x == 2 ? col0 : 0)), row,
                     nch * static_cast<int>(sizeof(TIn)));
          } else {
#pragma unroll
            for (int j = 0; j < EPL; ++j)
              if (lane + 64 * j < nch) row[lane + 64 * j] = TIn{};
          }
        }
      }
    }
  }
  float4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    s[m] = *reinterpret_cast<const float4 *>(S + static_cast<size_t>(rg + RG * m) * D + 4 * cg);

  auto conv_ready = [&]() {   // wave 0, before its first read of the taps or windows
    if constexpr (CONV) {
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const int W = cv.W;
      if (W != 4) {
        // [channel][W] -> [channel][4] right-aligned: every lane reads its channels' taps
        // before any lane writes (one wave, LDS operations in order)
        float4 *tdst[3] = {s_tq, s_tk, s_tv};
        float t[3][EPL][4];
#pragma unroll
        for (int x = 0; x < 3; ++x)
#pragma unroll
          for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            const float *src = reinterpret_cast<const float *>(tdst[x]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              t[x][j][jj] = (e < (x == 2 ? DVW : D) && jj >= 4 - W) ? src[e * W + jj - (4 - W)] : 0.f;
          }
        wave_sync_lds();
#pragma unroll
        for (int x = 0; x < 3; ++x)
#pragma unroll
          for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < (x == 2 ? DVW : D)) tdst[x][e] = make_float4(t[x][j][0], t[x][j][1], t[x][j][2], t[x][j][3]);
          }
        wave_sync_lds();
      }
    }
  };

  // Inputs of token t: wave 0 holds k, q, g, beta and the mask flag, every thread its
  // four columns of v.  Column tiles (few work-groups, each walking its tokens) load them
  // two tokens ahead; whole slabs (many work-groups per CU hide the latency, and the
  // extra registers would cost occupancy) at the start of token t.
  // Raw as loaded (bf16 stays 16-bit): converting right after a load would make the
  // compiler wait for it there instead of at the use a token or two later.
  typedef typename std::conditional<sizeof(TIn) == 2, uint2, float4>::type RawV;
  struct In {
    TIn k[EPL], q[EPL];
    float g[EPL], bt;
    uint32_t mk;
    RawV v;
    TIn vw[EPL];               // CONV, wave 0: raw v of the tile's columns lane + 64 j
  };
  auto f32_of = [](TIn x) -> float {
    if constexpr (sizeof(TIn) == 2) return bf16_to_f32(x);
    else return x;
  };
  auto f32x4_of = [](RawV x) -> float4 {
    if constexpr (sizeof(TIn) == 2) return make_float4(lo_bf16(x.x), hi_bf16(x.x), lo_bf16(x.y), hi_bf16(x.y));
    else return x;
  };
  auto fetch = [&](int t, In &in) {
    const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e < D) {
          in.k[j] = k[tok * D + e];
          in.q[j] = q[tok * D + e];
          in.g[j] = g_head ? g[tok] : g[tok * D + e];
        }
      }
      in.bt = beta[tok];
      in.mk = mask == nullptr ? 1u : mask[static_cast<size_t>(b) * T + t];
      if constexpr (CONV) {
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + 64 * j < DVW) in.vw[j] = v[tok * D + col0 + lane + 64 * j];
      }
    }
    if constexpr (!CONV) in.v = *reinterpret_cast<const RawV *>(v + tok * D + col0 + 4 * cg);
  };

  // CONV (Kimi-K3 atlas, KDA layer page, kda-init code: a causal ShortConvolution with SiLU
  // on each projection; nnterp Kimi-Linear page, Notes: the layer carries its last inputs
  // outside the state).  Wave 0 filters every channel of the token (q and k: lane + 64 j;
  // v: the tile's columns), reading the taps from memory and the windows from LDS; a
  // padding token leaves the windows as they are.  The filtered values stay in fp32.
  // One filter output of channel e of projection x (0 q, 1 k, 2 v) for raw input xr; the
  // window advances when `live`.
  auto filt = [&](int x, int e, float xr, bool live) -> float {
    const float4 tap = (x == 0 ? s_tq : (x == 1 ? s_tk : s_tv))[e];
    constexpr int J1 = CONV ? 1 : 0, J2 = CONV ? 2 : 0;   // (the windows exist only with CONV)
    TIn *w0 = x == 0 ? s_wq[0] : (x == 1 ? s_wk[0] : s_wv[0]);
    TIn *w1 = x == 0 ? s_wq[J1] : (x == 1 ? s_wk[J1] : s_wv[J1]);
    TIn *w2 = x == 0 ? s_wq[J2] : (x == 1 ? s_wk[J2] : s_wv[J2]);
    const TIn r0 = w0[e], r1 = w1[e], r2 = w2[e];
    float z = conv_z4(tap, f32_of(r0), f32_of(r1), f32_of(r2), xr);
    if (cv.silu) z = silu_act(z);
    if (live) {                // raw inputs, exact in the input dtype
      w0[e] = r1;
      w1[e] = r2;
      if constexpr (sizeof(TIn) == 2) w2[e] = f32_to_bf16(xr);
      else w2[e] = xr;
    }
    return z;                  // kept in fp32
  };

  // Wave 0: normalise token t's k and q, its decay factors, k.q, beta and the valid flag
  // into input set `nb` (from `in` for column tiles, else loaded here).
  auto prologue = [&](int t, const In &in, int nb) {
    const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
    float kk[EPL], qq[EPL], ee[EPL];
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      kk[j] = qq[j] = 0.f;
      ee[j] = 1.f;
      if (e < D) {
        if constexpr (PF) {
          kk[j] = f32_of(in.k[j]);
          qq[j] = f32_of(in.q[j]);
          ee[j] = fast_exp2(in.g[j] * kLog2e);
        } else {
          kk[j] = Elem<TIn>::load(k, tok * D + e);
          qq[j] = Elem<TIn>::load(q, tok * D + e);
          ee[j] = fast_exp2((g_head ? g[tok] : g[tok * D + e]) * kLog2e);
        }
        sk += kk[j] * kk[j];
        sq += qq[j] * qq[j];
      }
    }
    if constexpr (CONV) {
      // filter the raw inputs; the sums of squares are over the filtered values
      bool live;
      if constexpr (PF) live = in.mk != 0;
      else live = mask == nullptr || mask[static_cast<size_t>(b) * T + t] != 0;
      sk = sq = 0.f;
      float vr[EPL];
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        vr[j] = 0.f;
        if (e < DVW) {
          if constexpr (PF) vr[j] = f32_of(in.vw[j]);
          else vr[j] = Elem<TIn>::load(v, tok * D + col0 + e);
        }
      }
      // one filter at a time (the empty asm statements keep the compiler from hoisting the
      // next one's LDS reads): their operands would otherwise all be live at once, next to
      // the state, and cost occupancy
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e < D) {
          kk[j] = filt(1, e, kk[j], live);
          __asm__ volatile("" ::: "memory");
          qq[j] = filt(0, e, qq[j], live);
          __asm__ volatile("" ::: "memory");
          sk += kk[j] * kk[j];
          sq += qq[j] * qq[j];
        }
        if (e < DVW) {
          s_v[nb][e] = filt(2, e, vr[j], live);
          __asm__ volatile("" ::: "memory");
        }
      }
    }
    sk = wave_sum(sk);
    sq = wave_sum(sq);
    const float kn = use_l2 ? rsqrtf(sk + kL2Eps) : 1.f;
    const float qn = (use_l2 ? rsqrtf(sq + kL2Eps) : 1.f) * scale;
    float kq = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < D) {
        s_k[nb][e] = kk[j] * kn;
        s_q[nb][e] = qq[j] * qn;
        s_e[nb][e] = ee[j];
        kq += (kk[j] * kn) * (qq[j] * qn);
      }
    }
    kq = wave_sum(kq);
    if (lane == 0) {
      s_scal[nb][0] = kq;
      if constexpr (PF) {
        s_scal[nb][1] = in.bt;
        s_scal[nb][2] = in.mk != 0 ? 1.f : 0.f;
      } else {
        s_scal[nb][1] = beta[tok];
        s_scal[nb][2] = (mask == nullptr || mask[static_cast<size_t>(b) * T + t] != 0) ? 1.f : 0.f;
      }
    }
  };
  // Every wave: decay its rows with input set nb and put its partial S'^T k, S'^T q
  // column sums in sum set nr.
  auto partials = [&](int nb, int nr) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f), p = r;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = rg + RG * m;
      const float a = s_e[nb][i], kv = s_k[nb][i], qv = s_q[nb][i];
      s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
      r.x += kv * s[m].x; r.y += kv * s[m].y; r.z += kv * s[m].z; r.w += kv * s[m].w;
      p.x += qv * s[m].x; p.y += qv * s[m].y; p.z += qv * s[m].z; p.w += qv * s[m].w;
    }
    r.x = group_sum<RL>(r.x); r.y = group_sum<RL>(r.y);
    r.z = group_sum<RL>(r.z); r.w = group_sum<RL>(r.w);
    p.x = group_sum<RL>(p.x); p.y = group_sum<RL>(p.y);
    p.z = group_sum<RL>(p.z); p.w = group_sum<RL>(p.w);
    if (lane % RL == 0) {
      *reinterpret_cast<float4 *>(&s_red[nr][wave][0][4 * cg]) = r;
      *reinterpret_cast<float4 *>(&s_red[nr][wave][1][4 * cg]) = p;
    }
  };
  // Every thread: the delta-rule update of its rows and token t's output for its
  // columns, then the stores.  vv: token t's v of the thread's columns; graw: its gate
  // as loaded (read by wave 0 with the fused norm).
  auto finish = [&](int t, int nb, int nr, bool valid, float4 vv, RawV graw) {
    const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
    float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      float4 rr = *reinterpret_cast<const float4 *>(&s_red[nr][0][0][4 * cg]);
      float4 pp = *reinterpret_cast<const float4 *>(&s_red[nr][0][1][4 * cg]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float4 r2 = *reinterpret_cast<const float4 *>(&s_red[nr][w][0][4 * cg]);
        const float4 p2 = *reinterpret_cast<const float4 *>(&s_red[nr][w][1][4 * cg]);
        rr.x += r2.x; rr.y += r2.y; rr.z += r2.z; rr.w += r2.w;
        pp.x += p2.x; pp.y += p2.y; pp.z += p2.z; pp.w += p2.w;
      }
      const float bt = s_scal[nb][1], kq = s_scal[nb][0];
      float4 u;
      u.x = bt * (vv.x - rr.x); u.y = bt * (vv.y - rr.y);
      u.z = bt * (vv.z - rr.z); u.w = bt * (vv.w - rr.w);
      out.x = pp.x + u.x * kq; out.y = pp.y + u.y * kq;
      out.z = pp.z + u.z * kq; out.w = pp.w + u.w * kq;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const float kv = s_k[nb][rg + RG * m];
        s[m].x += kv * u.x; s[m].y += kv * u.y; s[m].z += kv * u.z; s[m].w += kv * u.w;
      }
    }
    if constexpr (STATES) {
      float *St = states + tok * D * D + col0;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        // store from a copy: the next token's decay may then rewrite s[m] without first
        // waiting for this store to complete
        float4 c;
        __asm__ volatile("v_mov_b32 %0, %1" : "=v"(c.x) : "v"(s[m].x));
        __asm__ volatile("v_mov_b32 %0, %1" : "=v"(c.y) : "v"(s[m].y));
        __asm__ volatile("v_mov_b32 %0, %1" : "=v"(c.z) : "v"(s[m].z));
        __asm__ volatile("v_mov_b32 %0, %1" : "=v"(c.w) : "v"(s[m].w));
        store_nt(St + static_cast<size_t>(rg + RG * m) * D + 4 * cg, c);
      }
    }
    if constexpr (PF) {
      // Every thread holds `out` of its columns; every wave stores the tile's row (the
      // same values to the same addresses), so each wave issues the same memory
      // operations every token and the wait for the prefetched inputs counts past the
      // stores instead of waiting for them.
      Elem<TOut>::store4(o, tok * D + col0 + 4 * cg, out);   // 0 for a padding token
    } else if (wave == 0) {
      // Every lane of wave 0 holds `out` of its column group, each group in RL lanes:
      // the row's sum of squares is the wave's sum over RL.
      float rn = 0.f;
      if constexpr (NORM) {
        const float ss = wave_sum(out.x * out.x + out.y * out.y + out.z * out.z + out.w * out.w) * (1.f / RL);
        rn = rsqrtf(ss / D + eps);
      }
      if (rg == 0) {   // one lane per column group stores the row
        Elem<TOut>::store4(o, tok * D + col0 + 4 * cg, out);
        if constexpr (NORM) {
          const float4 gt = f32x4_of(graw);
          const float4 w = *reinterpret_cast<const float4 *>(norm_w + 4 * cg);
          float4 yy;
          yy.x = w.x * out.x * rn * sigmoidf_(gt.x);
          yy.y = w.y * out.y * rn * sigmoidf_(gt.y);
          yy.z = w.z * out.z * rn * sigmoidf_(gt.z);
          yy.w = w.w * out.w * rn * sigmoidf_(gt.w);
          Elem<TOut>::store4(y, tok * D + 4 * cg, yy);
        }
      }
    }
  };

  In inA, inB;
  if constexpr (PF) {
    // Column tiles: one work-group barrier per token.  During token t's partial sums,
    // wave 0 already prepares token t+1's inputs in set (t+1) % 3; after the barrier every
    // thread finishes token t.  Set (t+1) % 3 was last read by token t-2, which every
    // thread finished before token t-1's barrier; token t-1's set is still being read
    // by threads finishing it, hence three sets.  Sum set t & 1 is next written at token
    // t+2, after token t+1's barrier.
    // The state's loads complete here, once (an empty asm that reads them), on every path
    // into the token loop: otherwise their waits sit at the first use inside the loop,
    // where every token would also wait for the previous one's memory operations.
#pragma unroll
    for (int m = 0; m < RPT; ++m) __asm__ volatile("" ::"v"(s[m].x), "v"(s[m].y), "v"(s[m].z), "v"(s[m].w));
    if (T > 0) {
      fetch(0, inA);
      if (T > 1) fetch(1, inB);
      if (wave == 0) {
        conv_ready();
        prologue(0, inA, 0);
      }
      sync_lds();
    }
    // token t: `cur` holds its inputs (v used here), `nxt` those of t+1 (prepared here);
    // `cur` is refilled with token t+2's.
    auto step = [&](int t, In &cur, In &nxt) {
      const int nb = t % 3, nr = t & 1;
      const bool valid = s_scal[nb][2] != 0.f;
      if (valid) partials(nb, nr);
      if (wave == 0 && t + 1 < T) prologue(t + 1, nxt, (t + 1) % 3);
      sync_lds();
      // refill `cur` with token t+2's inputs before this token's stores, so that waiting
      // for those loads later does not wait for the stores (one in-order counter)
      float4 vv;
      if constexpr (CONV) vv = *reinterpret_cast<const float4 *>(&s_v[nb][4 * cg]);
      else vv = f32x4_of(cur.v);
      fetch(min(t + 2, T - 1), cur);          // (the last token again near the end)
      finish(t, nb, nr, valid, vv, RawV{});   // column tiles: no fused norm, no gate
    };
    int t = 0;
    for (; t + 1 < T; t += 2) {
      step(t, inA, inB);
      step(t + 1, inB, inA);
    }
    if (t < T) step(t, inA, inB);
  } else {
    if (wave == 0) conv_ready();
    for (int t = 0; t < T; ++t) {
      // v of this thread's columns and the gate (wave 0, which writes y) are loaded
      // before the prologue: their latency overlaps the prologue and the partial sums
      // instead of following them.
      const size_t tok = (static_cast<size_t>(b) * T + t) * H + h;
      RawV vraw{};
      if constexpr (!CONV) vraw = *reinterpret_cast<const RawV *>(v + tok * D + col0 + 4 * cg);
      RawV graw{};
      if constexpr (NORM) {
        if (wave == 0) graw = *reinterpret_cast<const RawV *>(gate + tok * D + 4 * cg);
      }
      if (wave == 0) prologue(t, inA, 0);
      sync_lds();
      const bool valid = s_scal[0][2] != 0.f;
      if (valid) partials(0, 0);
      sync_lds();
      float4 vv;
      if constexpr (CONV) vv = *reinterpret_cast<const float4 *>(&s_v[0][4 * cg]);
      else vv = f32x4_of(vraw);
      finish(t, 0, 0, valid, vv, graw);
      sync_lds();   // the input and sum sets are rewritten by the next token
    }
  }

#pragma unroll
  for (int m = 0; m < RPT; ++m)
    store_nt(S + static_cast<size_t>(rg + RG * m) * D + 4 * cg, s[m]);

  if constexpr (CONV && !PF) {
    // The carried inputs after the call: window rows 4-W .. 2.  A whole slab is the only
    // reader of its head's channels, and they were read before any was written, so the
    // update may be in place.
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        if (e >= D) continue;
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          TIn *fin = static_cast<TIn *>(x == 0 ? cv.fin[0] : (x == 1 ? cv.fin[1] : cv.fin[2]));
          if (fin == nullptr) continue;
          const size_t ch = static_cast<size_t>(h) * D + e;
          const TIn *const wrow[3] = {x == 0 ? s_wq[0] : (x == 1 ? s_wk[0] : s_wv[0]),
                                      x == 0 ? s_wq[1] : (x == 1 ? s_wk[1] : s_wv[1]),
                                      x == 0 ? s_wq[2] : (x == 1 ? s_wk[2] : s_wv[2])};
#pragma unroll
          for (int jj = 0; jj < 3; ++jj)
            if (jj >= 4 - cv.W) fin[carried(jj, ch)] = wrow[jj][e];
        }
      }
    }
  }
}

template <int D, int DVW, int RPT, typename TIn, typename TOut>
hipError_t launch_typed(const Args &a, hipStream_t st) {
  constexpr int NT = (D / RPT) * (DVW / 4);
  const dim3 grid(static_cast<unsigned>(a.B) * a.H * (D / DVW)), block(NT);
  const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k),
            *v = static_cast<const TIn *>(a.v), *gate = static_cast<const TIn *>(a.gate);
  TOut *o = static_cast<TOut *>(a.o), *y = static_cast<TOut *>(a.y);
  auto go3 = [&](auto norm, auto with_states, auto conv) {
    hipLaunchKernelGGL((recurrent_kernel<D, DVW, RPT, TIn, TOut, decltype(norm)::value, decltype(with_states)::value,
                                         decltype(conv)::value>),
                       grid, block, 0, st, q, k, v, a.g, a.beta, a.state, a.mask, o, gate, a.norm_w, y, a.T, a.H,
                       a.scale, a.use_l2, a.eps, a.g_head, a.states_out, a.conv);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto go = [&](auto norm, auto with_states) { go3(norm, with_states, F_{}); };
  const bool norm = DVW == D && a.y != nullptr;
  if (a.conv.W > 0) {
    // the filtered path stores no per-token states
    if constexpr (DVW == D) {
      if (norm) go3(T_{}, F_{}, T_{});
      else go3(F_{}, F_{}, T_{});
    } else {
      go3(F_{}, F_{}, T_{});
    }
  } else if (a.states_out) {
    if constexpr (DVW == D) {
      if (norm) go(T_{}, T_{});
      else go(F_{}, T_{});
    } else {
      go(F_{}, T_{});
    }
  } else {
    if constexpr (DVW == D) {
      if (norm) go(T_{}, F_{});
      else go(F_{}, F_{});
    } else {
      go(F_{}, F_{});
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || DVW == D) return e;
  // column tiles: the carried inputs after the call (every tile of a head reads its q and
  // k windows) and the gated norm over whole rows run as passes of their own
  if (a.conv.W > 0) {
    e = launch_conv_carry(a, st);
    if (e != hipSuccess) return e;
  }
  if (a.y == nullptr) return hipSuccess;
  return launch_gated_rmsnorm(a.o, a.gate, a.norm_w, a.y, static_cast<int64_t>(a.B) * a.T * a.H, D, a.eps,
                              a.out_bf16, a.in_bf16, a.out_bf16, st);
}

template <int D, int DVW, int RPT>
hipError_t launch_d(const Args &a, hipStream_t st) {
  if (a.in_bf16 && a.out_bf16) return launch_typed<D, DVW, RPT, uint16_t, uint16_t>(a, st);
  if (a.in_bf16) return launch_typed<D, DVW, RPT, uint16_t, float>(a, st);
  if (a.out_bf16) return launch_typed<D, DVW, RPT, float, uint16_t>(a, st);
  return launch_typed<D, DVW, RPT, float, float>(a, st);
}

// Slabs below which a d = 128 slab is split into 8 work-groups of 16 columns when the
// call walks more than one token (a single token is one latency either way, and the
// split needs a separate norm pass).
constexpr long long kSplitSlabs = 512;

}  // namespace

bool recurrent_supports(int dk, int dv) {
  return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_recurrent(const Args &a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_d<16, 16, 1>(a, st);
    case 32: return launch_d<32, 32, 4>(a, st);
    case 64: return launch_d<64, 64, 8>(a, st);
    case 128:
      if (a.T > 1 && static_cast<long long>(a.B) * a.H < kSplitSlabs) return launch_d<128, 16, 4>(a, st);
      return launch_d<128, 128, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
