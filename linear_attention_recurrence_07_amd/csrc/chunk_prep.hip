// Chunk preparation for the bf16 chunked prefill (head size 128, 32-token chunks).
//
// The chunked form of the KDA recurrence (nnterp Kimi-Linear page, Notes, "Loading" and
// the KDA paragraph; section 04 docstring) splits every chunk's work into a part that
// needs the incoming state and a part that does not.  This kernel does the second part,
// for every (sequence, head, chunk) at once.  With G the running sum of g over the chunk
// (per key channel), k^ and q^ the normalised key and query (q^ also scaled):
//     A[s][j]   = beta_s sum_c k^_sc k^_jc exp(G_sc - G_jc)      (j < s)
//     Bqk[r][s] = sum_c q^_rc k^_sc exp(G_rc - G_sc)              (s <= r)
//     W         = (I + A)^-1 diag(beta)
// and stores Bqk, W and the per-token norm factors in the chunk's record (kda_chunk.h).
// The scan kernel then only needs U = W (V - (k^ exp(G)) S0) per chunk.
//
// Decay factoring.  exp(G_s - G_j) is split into a row and a column factor around a
// reference point: the boundary between the two 16-token sub-blocks for the off-diagonal
// block (both factors <= 1, fp16), the 8th token of the sub-block for a diagonal block
// (|exponent| <= 8 * 5 = 40 when g >= -5, so bf16).  Precision: the diagonal Bqk blocks
// take bf16 hi + lo operands (three products), A's diagonal blocks single bf16.
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

struct alignas(16) Smem {
  uint16_t rkd[C * LDK];       // bf16 k exp(G - G_mid(block))
  uint16_t rqd_hi[C * LDK];    // bf16 q exp(G - G_mid(block)), hi part
  uint16_t rqd_lo[C * LDK];    //                                  lo part
  uint16_t ckd_hi[C * LDK];    // bf16 k exp(G_mid(block) - G), hi part
  uint16_t ckd_lo[C * LDK];    //                                  lo part
  uint16_t kof[C * LDK];       // fp16 k exp(G_15 - G) on block 0 rows, k exp(G - G_15) on block 1 rows
  uint16_t rq1[SB * LDK];      // fp16 q exp(G - G_15) of block 1 rows
  float gtot[NW * DK];         // decay product over each 4-token group
  float beta[C];
  float at[2 * LDA];           // A_aa transposed: at[a][j][s] = A[16a+s][16a+j]
  float tm[2][SB][SB + 1];     // (I + A_aa)^-1
  float a10[SB][SB + 1];       // A(1,0)
  float p[SB][SB + 1];         // A(1,0) (I + A_00)^-1
  Rec rec;                     // staged record, written out in 16-byte pieces
};
static_assert(sizeof(Smem) <= 80 * 1024, "two work-groups per CU");

// Key-side 16x16 blocks.  Result layout: acc[i] = block[4*lg + i][l16].
__device__ __forceinline__ f32x4 a_diag(const Smem &sm, int a, int l16, int lg) {
  const uint16_t *rp = sm.rkd + (SB * a + l16) * LDK + 8 * lg;
  const uint16_t *cp = sm.ckd_hi + (SB * a + l16) * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) acc = mfma_bf16(lds_u4(rp + 32 * s), lds_u4(cp + 32 * s), acc);
  return acc;
}
__device__ __forceinline__ f32x4 bqk_diag(const Smem &sm, int a, int l16, int lg) {
  const int ro = (SB * a + l16) * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    const uint4 rh = lds_u4(sm.rqd_hi + ro + 32 * s), rl = lds_u4(sm.rqd_lo + ro + 32 * s);
    const uint4 ch = lds_u4(sm.ckd_hi + ro + 32 * s), cl = lds_u4(sm.ckd_lo + ro + 32 * s);
    acc = mfma_bf16(rl, ch, acc);
    acc = mfma_bf16(rh, cl, acc);
    acc = mfma_bf16(rh, ch, acc);
  }
  return acc;
}
__device__ __forceinline__ f32x4 off_block(const uint16_t *rows, const Smem &sm, int l16, int lg) {
  const uint16_t *rp = rows + l16 * LDK + 8 * lg;
  const uint16_t *cp = sm.kof + l16 * LDK + 8 * lg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) acc = mfma_f16(lds_u4(rp + 32 * s), lds_u4(cp + 32 * s), acc);
  return acc;
}

template <bool HAS_MASK>
__global__ void __launch_bounds__(NT, 2)
chunk_prep_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                  const float *__restrict__ g, const float *__restrict__ beta,
                  const int32_t *__restrict__ cu, const uint8_t *__restrict__ mask,
                  Rec *__restrict__ ws, int T, int H, int N, float scale, int use_l2) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;

  // ---------------------------------------------------------------- locate the chunk
  const int h = blockIdx.x % H;
  const long long slot = blockIdx.x / H;
  int b, t_begin, t_end;
  long long c;
  if (cu) {
    // largest n whose first slot is <= slot (first slots increase with n)
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (packed_slot_base(mid, min(max(cu[mid], 0), T)) <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = 0;
    t_end = min(cu[lo + 1], T);
    t_begin = max(0, min(cu[lo], t_end));
    c = slot - packed_slot_base(lo, min(max(cu[lo], 0), T));
  } else {
    const long long nch = chunks_per_row(T);
    b = static_cast<int>(slot / nch);
    c = slot % nch;
    t_begin = 0;
    t_end = T;
  }
  if (c < 0 || c * C >= t_end - t_begin) return;   // no chunk in this slot (whole work-group)
  const int c0 = t_begin + static_cast<int>(c) * C;
  Rec *rec = ws + slot * H + h;

  const int tok_stride = H * DK;
  const size_t row0 = static_cast<size_t>(b) * T;
  const uint16_t *kp = k + row0 * tok_stride + h * DK + 2 * lane;
  const uint16_t *qp = q + row0 * tok_stride + h * DK + 2 * lane;
  const float *gp = g + row0 * tok_stride + h * DK + 2 * lane;
  const float *bp = beta + row0 * H + h;

  // ---------------------------------------------------------------- phase 1
  // Load, normalise q/k, per-group decay products.
  float kx[TPW][2], qx[TPW][2], fw[TPW][2], bw[TPW][2];
  bool vld[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = c0 + TPW * wave + j;
    const int tc = min(t, t_end - 1);
    bool valid = t < t_end;
    if constexpr (HAS_MASK) valid = valid && mask[row0 + tc] != 0;
    vld[j] = valid;
    const int off = tc * tok_stride;
    const uint32_t kk = *reinterpret_cast<const uint32_t *>(kp + off);
    const uint32_t qq = *reinterpret_cast<const uint32_t *>(qp + off);
    const float2 gg = *reinterpret_cast<const float2 *>(gp + off);
    const float bb = bp[tc * H];
    // padding and tokens past the sequence act as no-ops
    kx[j][0] = valid ? lo_bf16(kk) : 0.f; kx[j][1] = valid ? hi_bf16(kk) : 0.f;
    qx[j][0] = valid ? lo_bf16(qq) : 0.f; qx[j][1] = valid ? hi_bf16(qq) : 0.f;
    fw[j][0] = valid ? gg.x : 0.f; fw[j][1] = valid ? gg.y : 0.f;
    if (lane == 0) sm.beta[TPW * wave + j] = valid ? bb : 0.f;
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
    float kn[TPW], qn[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      kn[j] = readlane(j & 1 ? n1 : n0, 16 * (j >> 1));
      qn[j] = readlane(j & 1 ? n1 : n0, 32 + 16 * (j >> 1));
      kx[j][0] *= kn[j]; kx[j][1] *= kn[j];
      qx[j][0] *= qn[j]; qx[j][1] *= qn[j];
    }
    // 0 marks padding and tokens past the end for the scan kernel
    if (lane < 2 * TPW) {
      const int j = lane & 3;
      const float kv = j == 0 ? (vld[0] ? kn[0] : 0.f) : j == 1 ? (vld[1] ? kn[1] : 0.f)
                     : j == 2 ? (vld[2] ? kn[2] : 0.f) : (vld[3] ? kn[3] : 0.f);
      const float qv = j == 0 ? (vld[0] ? qn[0] : 0.f) : j == 1 ? (vld[1] ? qn[1] : 0.f)
                     : j == 2 ? (vld[2] ? qn[2] : 0.f) : (vld[3] ? qn[3] : 0.f);
      if (lane < TPW) sm.rec.kn[TPW * wave + j] = kv;
      else sm.rec.qn[TPW * wave + j] = qv;
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
  *reinterpret_cast<float2 *>(sm.gtot + wave * DK + 2 * lane) = make_float2(fw[TPW - 1][0], fw[TPW - 1][1]);
  sync_lds();

  // ---------------------------------------------------------------- phase 2
  // Row and column factors of the intra-chunk products.
  {
    const int blk = wave >> 2;                   // sub-block of this wave's tokens
    const int gi = wave & 3;                     // group within the sub-block
    float e3m[2], e4m[2], ih1[2], ih2[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      float gt[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) gt[m] = sm.gtot[(4 * blk + m) * DK + 2 * lane + ch];
      const float p01 = gt[0] * gt[1], p23 = gt[2] * gt[3];
      e3m[ch] = gi == 0 ? 1.f : gi == 1 ? gt[0] : gi == 2 ? p01 : p01 * gt[2];   // block start -> group
      e4m[ch] = gi == 3 ? 1.f : gi == 2 ? gt[3] : gi == 1 ? p23 : gt[1] * p23;   // group -> block end
      ih1[ch] = __builtin_amdgcn_rcpf(p01);      // block start -> 8th token
      ih2[ch] = __builtin_amdgcn_rcpf(p23);      // 8th token -> block end
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int r = TPW * wave + j;
      float k3[2], q3[2], k4[2], rkd[2], rqd[2], ckd[2];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const float e3 = e3m[ch] * fw[j][ch];    // exp(G_r - G_block_start)
        const float e4 = bw[j][ch] * e4m[ch];    // exp(G_block_end - G_r)
        k3[ch] = kx[j][ch] * e3;
        q3[ch] = qx[j][ch] * e3;
        k4[ch] = kx[j][ch] * e4;
        rkd[ch] = k3[ch] * ih1[ch];              // k exp(G_r - G_mid)
        rqd[ch] = q3[ch] * ih1[ch];
        ckd[ch] = k4[ch] * ih2[ch];              // k exp(G_mid - G_r)
      }
      const int o2 = r * LDK + 2 * lane;
      *reinterpret_cast<uint32_t *>(sm.rkd + o2) = pack_bf16x2(rkd[0], rkd[1]);
      uint32_t hi, lo;
      split_bf16x2(rqd[0], rqd[1], hi, lo);
      *reinterpret_cast<uint32_t *>(sm.rqd_hi + o2) = hi;
      *reinterpret_cast<uint32_t *>(sm.rqd_lo + o2) = lo;
      split_bf16x2(ckd[0], ckd[1], hi, lo);
      *reinterpret_cast<uint32_t *>(sm.ckd_hi + o2) = hi;
      *reinterpret_cast<uint32_t *>(sm.ckd_lo + o2) = lo;
      // off-diagonal factors around token 15
      *reinterpret_cast<uint32_t *>(sm.kof + o2) =
          blk ? pack_f16x2(k3[0], k3[1]) : pack_f16x2(k4[0], k4[1]);
      if (blk) *reinterpret_cast<uint32_t *>(sm.rq1 + o2 - SB * LDK) = pack_f16x2(q3[0], q3[1]);
    }
  }
  sync_lds();

  // ---------------------------------------------------------------- phase 3
  // A and Bqk blocks on the matrix cores, inverses of the diagonal blocks of I + A.
  if (wave == 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const f32x4 acc = a_diag(sm, a, l16, lg);
      float4 w;   // A[s][j] = beta_s * acc for j < s, stored transposed at at[a][j][s]
      const float *bs = sm.beta + SB * a + 4 * lg;
      w.x = (l16 < 4 * lg + 0) ? bs[0] * acc[0] : 0.f;
      w.y = (l16 < 4 * lg + 1) ? bs[1] * acc[1] : 0.f;
      w.z = (l16 < 4 * lg + 2) ? bs[2] * acc[2] : 0.f;
      w.w = (l16 < 4 * lg + 3) ? bs[3] * acc[3] : 0.f;
      *reinterpret_cast<float4 *>(sm.at + a * LDA + l16 * SB + 4 * lg) = w;
    }
    wave_sync_lds();
    // (I + A_aa)^-1, column cc, by forward substitution; lanes 32-63 repeat 0-31
    const int a = (lane >> 4) & 1, cc = l16;
    float tc[SB];
#pragma unroll
    for (int r = 0; r < SB; ++r) tc[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < SB - 1; ++j) {
      const float *col = sm.at + a * LDA + j * SB;   // A[.][j]
#pragma unroll
      for (int r = j + 1; r < SB; ++r) tc[r] -= col[r] * tc[j];
    }
    if (lane < 32) {
#pragma unroll
      for (int r = 0; r < SB; ++r) sm.tm[a][r][cc] = tc[r];
    }
  } else if (wave == 1) {
    const f32x4 accA = off_block(sm.kof + SB * LDK, sm, l16, lg);
    const f32x4 accB = off_block(sm.rq1, sm, l16, lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = 4 * lg + i;
      sm.a10[sl][l16] = sm.beta[SB + sl] * accA[i];
      sm.rec.bqk[(SB + sl) * C + l16] = f16_bits(accB[i]);
      sm.rec.bqk[sl * C + SB + l16] = 0;           // above the diagonal blocks
    }
  } else if (wave < 4) {
    const int a = wave - 2;
    const f32x4 acc = bqk_diag(sm, a, l16, lg);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sl = 4 * lg + i;
      sm.rec.bqk[(SB * a + sl) * C + SB * a + l16] = f16_bits(l16 <= sl ? acc[i] : 0.f);
    }
  }
  sync_lds();

  // ---------------------------------------------------------------- phase 4
  // W = (I + A)^-1 diag(beta) = [[T0 B0, 0], [-T1 A10 T0 B0, T1 B1]], T_a = (I + A_aa)^-1.
  {
    const int e = tid & 255, r = e >> 4, cc = e & 15;
    if (tid < 256) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < SB; ++m) s += sm.a10[r][m] * sm.tm[0][m][cc];
      sm.p[r][cc] = s;
    } else {
      sm.rec.w[r * C + cc] = f16_bits(sm.tm[0][r][cc] * sm.beta[cc]);
      sm.rec.w[(SB + r) * C + SB + cc] = f16_bits(sm.tm[1][r][cc] * sm.beta[SB + cc]);
      sm.rec.w[r * C + SB + cc] = 0;
    }
    sync_lds();
    if (tid < 256) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < SB; ++m) s += sm.tm[1][r][m] * sm.p[m][cc];
      sm.rec.w[(SB + r) * C + cc] = f16_bits(-s * sm.beta[cc]);
    }
    sync_lds();
  }
  constexpr int kPieces = static_cast<int>(sizeof(Rec) / 16);
  if (tid < kPieces)
    reinterpret_cast<uint4 *>(rec)[tid] = reinterpret_cast<const uint4 *>(&sm.rec)[tid];
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
