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
// Decay factoring for the intra-chunk products.  exp(G_s - G_j) is split into a row and a
// column factor around a reference point: the boundary between the two 16-token
// sub-blocks for the off-diagonal block (both factors <= 1, fp16), the 8th token of the
// sub-block for a diagonal block (|exponent| <= 8 * 5 = 40 when g >= -5, so bf16).  The
// diagonal Bqk blocks take bf16 hi + lo operands (three products), A's diagonal blocks
// single bf16.
//
// Work-group: one (sequence, head, chunk), 512 threads; thread (wave w, lane l) owns
// tokens 4w..4w+3 and channels 2l, 2l+1.  Two work-groups fit one CU.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {
namespace {
using namespace chunk;

constexpr int NW = 8;
constexpr int NT = NW * 64;
constexpr int TPW = C / NW;       // tokens per wave (4)
constexpr int LDK = DK + 8;       // [token][channel] operand rows, 16-byte reads
constexpr int LDA = SB * SB + 8;  // fp32 16x16 diagonal blocks of A, transposed

// LDS layout (bytes).  The operand arrays are dead once the intra-chunk products are
// formed; the record's fragments of k^ exp(G), q^ exp(G) and the transposed decayed keys
// are staged over their tail, in a padded layout (16 bytes after every 16 lanes) so the
// scattered 4- and 8-byte staging writes spread over the banks.  The rest of the record
// (Bqk, W, exp(G_last), flags) is staged after them, unpadded.
constexpr int OPB = C * LDK * 2;                // one [32][LDK] 16-bit operand array
constexpr int O_RKD = 0, O_RQH = OPB, O_RQL = 2 * OPB, O_CKH = 3 * OPB, O_CKL = 4 * OPB;
constexpr int O_KOF = 5 * OPB, O_RQ1 = 6 * OPB;
constexpr int OPS_END = 6 * OPB + SB * LDK * 2;
constexpr int LGB = 16 * 16 + 16;               // one padded group of 16 lanes
constexpr int TILEB = 4 * LGB;                  // one padded fragment (64 lanes)
constexpr int REGB = 8 * TILEB;                 // 8 fragments
constexpr int O_STG = OPS_END - 3 * REGB;       // kb, qt, ket staging (overlaps the operands)
constexpr int O_TAIL = OPS_END;                 // bq, w1, w00, ec, valid (as in the record)
constexpr int TAIL_BYTES = static_cast<int>(sizeof(Rec)) - 3 * 8 * 64 * 16;
constexpr int O_GTOT = O_TAIL + TAIL_BYTES;
constexpr int O_BETA = O_GTOT + NW * DK * 4;
constexpr int O_AT = O_BETA + C * 4;
constexpr int O_TM = O_AT + 2 * LDA * 4;
constexpr int O_A10 = O_TM + 2 * SB * (SB + 1) * 4;
constexpr int O_P = O_A10 + SB * (SB + 1) * 4;
constexpr int O_VB = O_P + SB * (SB + 1) * 4;
constexpr int LDS_BYTES = O_VB + C;
static_assert(O_STG >= 0 && O_STG % 16 == 0 && O_GTOT % 16 == 0 && O_AT % 16 == 0, "alignment");
static_assert(LDS_BYTES <= 80 * 1024, "two work-groups per CU");

// Key-side 16x16 blocks.  Result layout: acc[i] = block[4*lg + i][l16].
__device__ __forceinline__ f32x4 a_diag(const uint16_t *rkd, const uint16_t *ckh, int a, int l16, int lg) {
  const uint16_t *rp = rkd + (SB * a + l16) * LDK + 8 * lg;
  const uint16_t *cp = ckh + (SB * a + l16) * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(lds_u4(rp + 32 * s), lds_u4(cp + 32 * s), acc);
  return acc;
}
__device__ __forceinline__ f32x4 bqk_diag(const uint16_t *rqh, const uint16_t *rql, const uint16_t *ckh,
                                          const uint16_t *ckl, int a, int l16, int lg) {
  const int ro = (SB * a + l16) * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    const uint4 rh = lds_u4(rqh + ro + 32 * s), rl = lds_u4(rql + ro + 32 * s);
    const uint4 ch = lds_u4(ckh + ro + 32 * s), cl = lds_u4(ckl + ro + 32 * s);
    acc = mfma_bf16(rl, ch, acc);
    acc = mfma_bf16(rh, cl, acc);
    acc = mfma_bf16(rh, ch, acc);
  }
  return acc;
}
__device__ __forceinline__ f32x4 off_block(const uint16_t *rows, const uint16_t *kof, int l16, int lg) {
  const uint16_t *rp = rows + l16 * LDK + 8 * lg;
  const uint16_t *cp = kof + l16 * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) acc = mfma_f16(lds_u4(rp + 32 * s), lds_u4(cp + 32 * s), acc);
  return acc;
}
// Element (r, c) of a 32x32 token-by-token matrix in the bq fragments.
__device__ __forceinline__ int bq_elem(int r, int c) {
  return ((r >> 4) * 64 + 16 * kidx_lg(c) + (r & 15)) * 8 + kidx_e(c);
}
// The part of the record after the three channel-fragment arrays.
struct Tail {
  uint16_t bq[2][64][8];
  uint16_t w1[64][8];
  uint16_t w00[64][4];
  uint16_t w1lo[64][8];
  uint16_t w00lo[64][4];
  float ec[DK];
  uint32_t valid;
  uint32_t pad[3];
};
static_assert(sizeof(Tail) == TAIL_BYTES && offsetof(Rec, bq) == 3 * 8 * 64 * 16, "record tail");
// x = hi + lo with both parts fp16.
__device__ __forceinline__ void split_f16(float x, uint16_t &hi, uint16_t &lo) {
  const _Float16 h = static_cast<_Float16>(x);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = f16_bits(x - static_cast<float>(h));
}
// Byte offset of lane L of fragment `tile` in the padded staging layout.
__device__ __forceinline__ int stg_off(int tile, int L) { return tile * TILEB + (L >> 4) * LGB + (L & 15) * 16; }

template <bool HAS_MASK>
__global__ void __launch_bounds__(NT, 2)
chunk_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const float *__restrict__ g, const float *__restrict__ beta,
                  const int32_t *__restrict__ cu, const uint8_t *__restrict__ mask,
                  Rec *__restrict__ ws, int T, int H, int N, float scale, int use_l2) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint16_t *rkd = reinterpret_cast<uint16_t *>(lds + O_RKD);   // bf16 k exp(G - G_mid(block))
  uint16_t *rqh = reinterpret_cast<uint16_t *>(lds + O_RQH);   // bf16 q exp(G - G_mid(block)), hi
  uint16_t *rql = reinterpret_cast<uint16_t *>(lds + O_RQL);   //                                lo
  uint16_t *ckh = reinterpret_cast<uint16_t *>(lds + O_CKH);   // bf16 k exp(G_mid(block) - G), hi
  uint16_t *ckl = reinterpret_cast<uint16_t *>(lds + O_CKL);   //                                lo
  uint16_t *kof = reinterpret_cast<uint16_t *>(lds + O_KOF);   // fp16 k exp(G_15 - G) | k exp(G - G_15)
  uint16_t *rq1 = reinterpret_cast<uint16_t *>(lds + O_RQ1);   // fp16 q exp(G - G_15), block 1 rows
  uint8_t *stg = lds + O_STG;                                    // staged kb, qt, ket (padded)
  Tail &st = *reinterpret_cast<Tail *>(lds + O_TAIL);           // staged rest of the record
  float *gtot = reinterpret_cast<float *>(lds + O_GTOT);        // decay product of each 4-token group
  float *sbeta = reinterpret_cast<float *>(lds + O_BETA);
  float *at = reinterpret_cast<float *>(lds + O_AT);            // A_aa transposed: at[a][j][s]
  auto tm = reinterpret_cast<float (*)[SB][SB + 1]>(lds + O_TM);   // (I + A_aa)^-1
  auto a10 = reinterpret_cast<float (*)[SB + 1]>(lds + O_A10);     // A(1,0)
  auto pp = reinterpret_cast<float (*)[SB + 1]>(lds + O_P);        // A(1,0) (I + A_00)^-1
  uint8_t *vb = lds + O_VB;                                        // token flags

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  // ---------------------------------------------------------------- locate the chunk
  const int h = static_cast<int>(blockIdx.x) % H;
  const int slot = static_cast<int>(blockIdx.x) / H;
  int b, t_begin, t_end, c;
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
  } else {
    const int nch = (T + C - 1) / C;
    b = slot / nch;
    c = slot - b * nch;
    t_begin = 0;
    t_end = T;
  }
  if (c < 0 || c * C >= t_end - t_begin) return;   // no chunk in this slot (whole work-group)
  const int c0 = t_begin + c * C;
  Rec *rec = ws + static_cast<size_t>(slot) * H + h;

  const int tok_stride = H * DK;
  const size_t row0 = static_cast<size_t>(b) * T;
  const uint16_t *kp = k + row0 * tok_stride + h * DK + 2 * lane;
  const uint16_t *qp = q + row0 * tok_stride + h * DK + 2 * lane;
  const float *gp = g + row0 * tok_stride + h * DK + 2 * lane;
  const float *bp = beta + row0 * H + h;

  // ---------------------------------------------------------------- phase 1
  // Load, normalise q/k, per-group decay products.
  float kx[TPW][2], qx[TPW][2], fw[TPW][2], bw[TPW][2];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = c0 + TPW * wave + j;
    const int tc = min(t, t_end - 1);
    bool valid = t < t_end;
    if constexpr (HAS_MASK) valid = valid && mask[row0 + tc] != 0;
    const int off = tc * tok_stride;
    const uint32_t kk = *reinterpret_cast<const uint32_t *>(kp + off);
    const uint32_t qq = *reinterpret_cast<const uint32_t *>(qp + off);
    const float2 gg = *reinterpret_cast<const float2 *>(gp + off);
    const float bb = bp[tc * H];
    // padding and tokens past the sequence act as no-ops
    kx[j][0] = valid ? lo_bf16(kk) : 0.f; kx[j][1] = valid ? hi_bf16(kk) : 0.f;
    qx[j][0] = valid ? lo_bf16(qq) : 0.f; qx[j][1] = valid ? hi_bf16(qq) : 0.f;
    fw[j][0] = valid ? gg.x : 0.f; fw[j][1] = valid ? gg.y : 0.f;
    if (lane == 0) {
      sbeta[TPW * wave + j] = valid ? bb : 0.f;
      vb[TPW * wave + j] = valid;
    }
  }
  {
    float ss[2 * TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      ss[j] = kx[j][0] * kx[j][0] + kx[j][1] * kx[j][1];
      ss[TPW + j] = qx[j][0] * qx[j][0] + qx[j][1] * qx[j][1];
    }
    float x0, x1;
    wave_sum8(ss, x0, x1);
    // rows 0-1 of x0/x1 hold key sums, rows 2-3 query sums
    const float qs = lane >= 32 ? scale : 1.f;
    const float n0 = (use_l2 ? rsqrtf(x0 + kL2Eps) : 1.f) * qs;
    const float n1 = (use_l2 ? rsqrtf(x1 + kL2Eps) : 1.f) * qs;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const float kn = readlane(j & 1 ? n1 : n0, 16 * (j >> 1));
      const float qn = readlane(j & 1 ? n1 : n0, 32 + 16 * (j >> 1));
      kx[j][0] *= kn; kx[j][1] *= kn;
      qx[j][0] *= qn; qx[j][1] *= qn;
    }
  }
  // fw[j] = prod_{i<=j} e_i (inclusive), bw[j] = prod_{j<i<4} e_i (exclusive)
#pragma unroll
  for (int ch = 0; ch < 2; ++ch) {
    float e[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) e[j] = fast_exp2(fw[j][ch] * kLog2e);
    float run = 1.f;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      run *= e[j];
      fw[j][ch] = run;
    }
    run = 1.f;
#pragma unroll
    for (int j = TPW - 1; j >= 0; --j) {
      bw[j][ch] = run;
      run *= e[j];
    }
  }
  *reinterpret_cast<float2 *>(gtot + wave * DK + 2 * lane) = make_float2(fw[TPW - 1][0], fw[TPW - 1][1]);
  sync_lds();

  // ---------------------------------------------------------------- phase 2
  // Row and column factors of the intra-chunk products (to LDS) and the decayed operands
  // (kept in registers until the operand area is free).
  const int blk = wave >> 2;                     // sub-block of this wave's tokens
  const int gi = wave & 3;                       // group within the sub-block
  uint32_t okb[TPW], oqt[TPW];                   // fp16 pairs (channels 2l, 2l+1) per token
  uint2 oke[2];                                  // fp16 k^ exp(G_last - G) of the 4 tokens, per channel
  float ecv[2];
  {
    float e3m[2], e4m[2], ih1[2], ih2[2], pre[2], post[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float gt[NW];
#pragma unroll
      for (int m = 0; m < NW; ++m) gt[m] = gtot[m * DK + 2 * lane + ch];
      const float b0 = blk ? gt[4] : gt[0], b1 = blk ? gt[5] : gt[1];
      const float b2 = blk ? gt[6] : gt[2], b3 = blk ? gt[7] : gt[3];
      const float p01 = b0 * b1, p23 = b2 * b3;
      e3m[ch] = gi == 0 ? 1.f : gi == 1 ? b0 : gi == 2 ? p01 : p01 * b2;   // block start -> group
      e4m[ch] = gi == 3 ? 1.f : gi == 2 ? b3 : gi == 1 ? p23 : b1 * p23;   // group -> block end
      ih1[ch] = __builtin_amdgcn_rcpf(p01);      // block start -> 8th token
      ih2[ch] = __builtin_amdgcn_rcpf(p23);      // 8th token -> block end
      const float d0 = (gt[0] * gt[1]) * (gt[2] * gt[3]);     // decay over block 0
      const float d1 = (gt[4] * gt[5]) * (gt[6] * gt[7]);     // decay over block 1
      pre[ch] = blk ? d0 * e3m[ch] : e3m[ch];    // chunk start -> group start
      post[ch] = blk ? e4m[ch] : e4m[ch] * d1;   // group end -> chunk end
      ecv[ch] = d0 * d1;
    }
    float ke[TPW][2];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int r = TPW * wave + j;
      float k3[2], q3[2], k4[2], rk[2], rq[2], ck[2], kb[2], qt[2];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const float e3 = e3m[ch] * fw[j][ch];    // exp(G_r - G_block_start)
        const float e4 = bw[j][ch] * e4m[ch];    // exp(G_block_end - G_r)
        k3[ch] = kx[j][ch] * e3;
        q3[ch] = qx[j][ch] * e3;
        k4[ch] = kx[j][ch] * e4;
        rk[ch] = k3[ch] * ih1[ch];               // k exp(G_r - G_mid)
        rq[ch] = q3[ch] * ih1[ch];
        ck[ch] = k4[ch] * ih2[ch];               // k exp(G_mid - G_r)
        const float ef = pre[ch] * fw[j][ch];    // exp(G_r)
        kb[ch] = kx[j][ch] * ef;
        qt[ch] = qx[j][ch] * ef;
        ke[j][ch] = kx[j][ch] * (bw[j][ch] * post[ch]);   // k^ exp(G_last - G_r)
      }
      okb[j] = pack_f16x2(kb[0], kb[1]);
      oqt[j] = pack_f16x2(qt[0], qt[1]);
      const int o2 = r * LDK + 2 * lane;
      *reinterpret_cast<uint32_t *>(rkd + o2) = pack_bf16x2(rk[0], rk[1]);
      uint32_t hi, lo;
      split_bf16x2(rq[0], rq[1], hi, lo);
      *reinterpret_cast<uint32_t *>(rqh + o2) = hi;
      *reinterpret_cast<uint32_t *>(rql + o2) = lo;
      split_bf16x2(ck[0], ck[1], hi, lo);
      *reinterpret_cast<uint32_t *>(ckh + o2) = hi;
      *reinterpret_cast<uint32_t *>(ckl + o2) = lo;
      // off-diagonal factors around token 15
      *reinterpret_cast<uint32_t *>(kof + o2) =
          blk ? pack_f16x2(k3[0], k3[1]) : pack_f16x2(k4[0], k4[1]);
      if (blk) *reinterpret_cast<uint32_t *>(rq1 + o2 - SB * LDK) = pack_f16x2(q3[0], q3[1]);
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) oke[ch] = pack_f16x4(ke[0][ch], ke[1][ch], ke[2][ch], ke[3][ch]);
  }
  sync_lds();

  // ---------------------------------------------------------------- phase 3
  // A and Bqk blocks on the matrix cores, inverses of the diagonal blocks of I + A.
  if (wave == 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const f32x4 acc = a_diag(rkd, ckh, a, l16, lg);
      float4 w;   // A[s][j] = beta_s * acc for j < s, stored transposed at at[a][j][s]
      const float *bs = sbeta + SB * a + 4 * lg;
      w.x = (l16 < 4 * lg + 0) ? bs[0] * acc[0] : 0.f;
      w.y = (l16 < 4 * lg + 1) ? bs[1] * acc[1] : 0.f;
      w.z = (l16 < 4 * lg + 2) ? bs[2] * acc[2] : 0.f;
      w.w = (l16 < 4 * lg + 3) ? bs[3] * acc[3] : 0.f;
      *reinterpret_cast<float4 *>(at + a * LDA + l16 * SB + 4 * lg) = w;
    }
    wave_sync_lds();
    // (I + A_aa)^-1, column cc, by forward substitution; lanes 32-63 repeat 0-31
    const int a = (lane >> 4) & 1, cc = l16;
    float tc[SB];
#pragma unroll
    for (int r = 0; r < SB; ++r) tc[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < SB - 1; ++j) {
      const float *col = at + a * LDA + j * SB;   // A[.][j]
#pragma unroll
      for (int r = j + 1; r < SB; ++r) tc[r] -= col[r] * tc[j];
    }
    if (lane < 32) {
#pragma unroll
      for (int r = 0; r < SB; ++r) tm[a][r][cc] = tc[r];
    }
  } else if (wave == 1) {
    const f32x4 accA = off_block(kof + SB * LDK, kof, l16, lg);
    const f32x4 accB = off_block(rq1, kof, l16, lg);
    uint16_t *bq = &st.bq[0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = 4 * lg + i;
      a10[sl][l16] = sbeta[SB + sl] * accA[i];
      bq[bq_elem(SB + sl, l16)] = f16_bits(accB[i]);
      bq[bq_elem(sl, SB + l16)] = 0;             // above the diagonal blocks
    }
  } else if (wave < 4) {
    const int a = wave - 2;
    const f32x4 acc = bqk_diag(rqh, rql, ckh, ckl, a, l16, lg);
    uint16_t *bq = &st.bq[0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = 4 * lg + i;
      bq[bq_elem(SB * a + sl, SB * a + l16)] = f16_bits(l16 <= sl ? acc[i] : 0.f);
    }
  }
  sync_lds();

  // ---------------------------------------------------------------- phase 4
  // W = (I + A)^-1 diag(beta) = [[T0 B0, 0], [-T1 A10 T0 B0, T1 B1]], T_a = (I + A_aa)^-1;
  // the decayed operands into the staged record.
  {
    const int e = tid & 255, r = e >> 4, cc = e & 15;
    if (tid < 256) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < SB; ++m) s += a10[r][m] * tm[0][m][cc];
      pp[r][cc] = s;
    } else {
      const float w00 = tm[0][r][cc] * sbeta[cc];
      split_f16(w00, st.w00[16 * (cc >> 2) + r][cc & 3], st.w00lo[16 * (cc >> 2) + r][cc & 3]);
      const int c1 = SB + cc;                    // W(1,1) block of rows 16..31
      const float w11 = tm[1][r][cc] * sbeta[SB + cc];
      split_f16(w11, st.w1[16 * kidx_lg(c1) + r][kidx_e(c1)], st.w1lo[16 * kidx_lg(c1) + r][kidx_e(c1)]);
    }
    // k^ exp(G) and q^ exp(G): token r = 4w + j, channels 2l, 2l+1 -> tile (r/16, l/16),
    // lane 16 * lg(ch) + r % 16, slots e(ch) and e(ch) + 1.
    {
      const int ch = 2 * lane;
      const int tile = blk * 4 + (ch >> 5);
      const int ln = 16 * kidx_lg(ch & 31);
      const int el = kidx_e(ch & 31);
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int off = stg_off(tile, ln + ((TPW * wave + j) & 15)) + 2 * el;
        *reinterpret_cast<uint32_t *>(stg + off) = okb[j];
        *reinterpret_cast<uint32_t *>(stg + REGB + off) = oqt[j];
      }
      // transposed: channel ch + cc2 -> tile ch/16, lane 16 * lg(token) + ch % 16, slots of
      // tokens 4w..4w+3 (consecutive)
#pragma unroll
      for (int cc2 = 0; cc2 < 2; ++cc2) {
        const int chc = ch + cc2;
        const int off = stg_off(chc >> 4, 16 * kidx_lg(TPW * wave) + (chc & 15)) + 2 * kidx_e(TPW * wave);
        *reinterpret_cast<uint2 *>(stg + 2 * REGB + off) = oke[cc2];
      }
    }
    if (wave == 0) *reinterpret_cast<float2 *>(&st.ec[2 * lane]) = make_float2(ecv[0], ecv[1]);
    sync_lds();
    if (tid < 256) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < SB; ++m) s += tm[1][r][m] * pp[m][cc];
      split_f16(-s * sbeta[cc], st.w1[16 * kidx_lg(cc) + r][kidx_e(cc)], st.w1lo[16 * kidx_lg(cc) + r][kidx_e(cc)]);
    } else if (tid == 256) {
      uint32_t v = 0;
      for (int t = 0; t < C; ++t) v |= static_cast<uint32_t>(vb[t] != 0) << t;
      st.valid = v;
    }
    sync_lds();
  }
  // write the record out in 16-byte pieces
  constexpr int kPieces = static_cast<int>(sizeof(Rec) / 16);
  constexpr int kFragPieces = 3 * 8 * 64;
  for (int p = tid; p < kPieces; p += NT) {
    const int src = p < kFragPieces ? O_STG + (p >> 9) * REGB + stg_off((p >> 6) & 7, p & 63)
                                    : O_TAIL + (p - kFragPieces) * 16;
    reinterpret_cast<uint4 *>(rec)[p] = *reinterpret_cast<const uint4 *>(lds + src);
  }
}

}  // namespace

// Workspace records for the bf16 chunked prefill: one per (slot, head).
size_t chunk_prep_workspace_bytes(long long B, long long T, long long H, long long N, bool packed) {
  return static_cast<size_t>(num_slots(B, T, N, packed) * H) * kRecBytes;
}

hipError_t launch_chunk_prep(const Args &a, void *ws, hipStream_t st) {
  const long long slots = num_slots(a.B, a.T, a.N, a.cu != nullptr);
  const long long blocks = slots * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k);
  Rec *rec = static_cast<Rec *>(ws);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.mask)
    hipLaunchKernelGGL((chunk_prep_kernel<true>), grid, dim3(NT), 0, st, q, k, a.g, a.beta, a.cu, a.mask,
                       rec, a.T, a.H, a.N, a.scale, a.use_l2);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<false>), grid, dim3(NT), 0, st, q, k, a.g, a.beta, a.cu, a.mask,
                       rec, a.T, a.H, a.N, a.scale, a.use_l2);
  return hipGetLastError();
}

}  // namespace kda
