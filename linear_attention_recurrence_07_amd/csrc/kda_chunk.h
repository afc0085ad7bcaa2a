// Shared pieces of the two-kernel chunked prefill (head size 128, 32-token chunks):
// operand packing, wave-wide sums, MFMA wrappers, and the per-chunk record that the
// preparation kernel writes and the scan kernel reads.
#pragma once

#include "kda_device.h"

namespace kda {
namespace chunk {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Native vectors for values held across loop iterations (HIP's uint2/uint4 are structs,
// which the optimiser may keep in memory instead of registers).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int C = 32;     // tokens per chunk
constexpr int SB = 16;    // tokens per sub-block

// Per (sequence, head, chunk) record in the workspace, written by the preparation kernel
// in the order the scan kernel's MFMA operands take.  A fragment is 64 lanes x 16 bytes:
// lane L = 16 * lg + r holds row r of a 16-row tile and the 8 K indices kidx(lg, e),
// e < 8, of a 32-wide K block (the same K permutation on both operands of a product).
//   kb[m*4+s]  fp16  k^ exp(G)      rows = tokens 16m.., K = channels 32s..
//   qt[m*4+s]  fp16  q^ exp(G)      same tiling (q^ includes the query scale)
//   ket[t]     fp16  k^ exp(G_last - G), transposed: rows = channels 16t.., K = tokens
//   bq[m], bqlo[m]  fp16  Bqk[r][s] = sum_c q^_rc k^_sc exp(G_rc - G_sc) (s <= r) as hi + lo
//              parts, rows 16m..
//   w1, w1lo   fp16  W = (I + A)^-1 diag(beta) as hi + lo parts, rows 16..31, K = 32 tokens
//   w00, w00lo fp16  W rows 0..15, K = tokens 0..15 (16x16x16 operand: e < 4 only)
//   ec[c]      fp32  exp(G_last) per key channel
//   valid      bit t set for a real token t of the chunk (not padding, not past the end)
// Padding and tokens past the end of a sequence have zero rows in kb, qt, ket, bq, and
// zero rows and columns in w.
struct alignas(16) Rec {
  uint16_t kb[8][64][8];
  uint16_t qt[8][64][8];
  uint16_t ket[8][64][8];
  uint16_t bq[2][64][8];
  uint16_t bqlo[2][64][8];
  uint16_t w1[64][8];
  uint16_t w00[64][4];
  uint16_t w1lo[64][8];
  uint16_t w00lo[64][4];
  float ec[DK];
  uint32_t valid;
  uint32_t pad[3];
};
static_assert(sizeof(Rec) == 32272, "record layout");
constexpr size_t kRecBytes = sizeof(Rec);
// Per (slot, head): the scan's gated-norm exchange, 2 tiles x 32 tokens of 64-bit words,
// stored after all records.
constexpr size_t kExchangeBytes = 2 * 32 * 8;
// After the exchange words: one 32-bit status word (in a 256-byte tail), set when a
// bounded wait between the two tiles of a head ran out; cleared by the preparation.
constexpr size_t kStatusBytes = 256;
// K index (0..31) of slot e (0..7) of lane group lg, and the inverse.
__host__ __device__ constexpr int kidx(int lg, int e) { return (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4); }
__host__ __device__ constexpr int kidx_lg(int x) { return (x & 15) >> 2; }
__host__ __device__ constexpr int kidx_e(int x) { return (x & 3) + 4 * (x >> 4); }

// Record slots.  Batched rows: slot = row * ceil(T / C) + chunk.  Packed sequences:
// slot = n + floor(start_n / C) + chunk with start_n = cu[n] clamped to [0, T], which is
// strictly increasing over (n, chunk) for valid offsets and stays below N + ceil(T / C)
// for any offsets (the scan's reads stay inside the workspace even for bad cu_seqlens).
__host__ __device__ inline long long chunks_per_row(long long T) { return (T + C - 1) / C; }
__host__ __device__ inline long long num_slots(long long B, long long T, long long N, bool packed) {
  return packed ? N + chunks_per_row(T) : B * chunks_per_row(T);
}
__device__ __forceinline__ long long packed_slot_base(int n, int start) { return n + start / C; }

// ------------------------------------------------------------------ operand packing
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ f16x8 as_f16x8(uint4 u) { return __builtin_bit_cast(f16x8, u); }
__device__ __forceinline__ f16x4 as_f16x4(uint2 u) { return __builtin_bit_cast(f16x4, u); }
__device__ __forceinline__ uint2 lds_u2(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ __forceinline__ uint4 lds_u4(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 join(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2 h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint2 pack_f16x4(float a, float b, float c, float d) {
  return make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
}
// x = hi + lo with both parts fp16 (about 22 significant bits together).
__device__ __forceinline__ void split_f16x4(f32x4 x, uint2 &hi, uint2 &lo) {
  hi = pack_f16x4(x[0], x[1], x[2], x[3]);
  const f16x4 h = as_f16x4(hi);
  lo = pack_f16x4(x[0] - static_cast<float>(h[0]), x[1] - static_cast<float>(h[1]),
                  x[2] - static_cast<float>(h[2]), x[3] - static_cast<float>(h[3]));
}
// (a, b) = hi + lo with both parts bf16 (about 16 significant bits together).
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - lo_bf16(hi), b - hi_bf16(hi));
}

// ------------------------------------------------------------------ wave-wide sums
// Sum over the 16 lanes of each row of a wave (DPP rotations and quad permutations).
__device__ __forceinline__ float row_sum16(float x) {
  const int r8 = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false);  // row_ror:8
  x += __builtin_bit_cast(float, r8);
  const int r4 = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false);  // row_ror:4
  x += __builtin_bit_cast(float, r4);
  const int q2 = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
  x += __builtin_bit_cast(float, q2);
  const int q1 = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
  return x + __builtin_bit_cast(float, q1);
}
// Sum of the two outputs of a lane swap.  The empty asm keeps the optimiser from folding
// the two outputs into one (it rewrites out0 + out1 as out0 + out0 otherwise).
__device__ __forceinline__ float swap_sum(uint32_t r0, uint32_t r1) {
  __asm__("" : "+v"(r1));
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
// a + b after swapping lanes 32-63 of a with lanes 0-31 of b: lanes 0-31 hold a folded
// over the two halves of the wave, lanes 32-63 hold b folded.
__device__ __forceinline__ float fold32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b),
                                                   false, false);
  return swap_sum(r[0], r[1]);
}
// The same with rows of 16: rows 0 and 2 hold a folded over row pairs, rows 1 and 3 b.
__device__ __forceinline__ float fold16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, a), __builtin_bit_cast(int, b),
                                                   false, false);
  return swap_sum(r[0], r[1]);
}
// Sums over the 64 lanes of eight values at once, by halving the lane range per value
// each swap.  On return the sum of v[m] is in every lane of row m >> 1 of x0 (m even)
// or x1 (m odd).
__device__ __forceinline__ void wave_sum8(const float (&v)[8], float &x0, float &x1) {
  const float w0 = fold32(v[0], v[4]), w1 = fold32(v[1], v[5]);
  const float w2 = fold32(v[2], v[6]), w3 = fold32(v[3], v[7]);
  x0 = row_sum16(fold16(w0, w2));
  x1 = row_sum16(fold16(w1, w3));
}
__device__ __forceinline__ float readlane(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// ------------------------------------------------------------------ matrix-core products
// 16x16 fp32 accumulator layout: acc[i] = C[4 * (lane / 16) + i][lane % 16].
__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16k16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(as_f16x4(a), as_f16x4(b), c, 0, 0, 0);
}

// ------------------------------------------------------------------ preparation helpers
// Value of lane r - N of the same 16-lane row (0 for r < N).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, true));
}
// Inclusive prefix sum over the 16 lanes of each row.
__device__ __forceinline__ float row_prefix(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}
// Sum over the four lanes r, r + 16, r + 32, r + 48.
__device__ __forceinline__ float col_sum4(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}
__device__ __forceinline__ f32x4 mfma_f32k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// x = hi + lo with both parts fp16, four values -> two fp16 pairs each.
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
  uint2 h, l;
  split_f16x4(x, h, l);
  hi = u32x2{h.x, h.y};
  lo = u32x2{l.x, l.y};
}
__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a[0], a[1], b[0], b[1]}; }
// w holds 8 channels 8L .. 8L+7 of a K block (L = (0, 2, 1, 3)[lg]); one row swap of its
// halves (odd rows of the first with even rows of the second) leaves channels 4lg .. 4lg+3
// in lo and 16 + 4lg .. 16 + 4lg + 3 in hi, the MFMA operand order.
__device__ __forceinline__ void operand_halves(u32x4 w, u32x2 &lo, u32x2 &hi) {
  const auto a = __builtin_amdgcn_permlane16_swap(w[0], w[2], false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(w[1], w[3], false, false);
  uint32_t a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
  __asm__("" : "+v"(a1), "+v"(b1));   // keep the optimiser from merging the swap's two outputs
  lo = u32x2{a0, b0};
  hi = u32x2{a1, b1};
}
__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Value of lane N of each 16-lane row, in every lane of that row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}

}  // namespace chunk
}  // namespace kda
