// Device helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;   // in-kernel q/k L2 norm: x / sqrt(sum x^2 + 1e-6)

// ------------------------------------------------------------------ bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// One packed conversion (v_cvt_pk_bf16_f32), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------------ typed element access
// Inputs are either fp32 or raw bf16 bits (uint16_t); outputs likewise.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
  // four consecutive elements (16-byte aligned)
  __device__ __forceinline__ static float4 load4(const float *p, size_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
  }
  __device__ __forceinline__ static void store4(float *p, size_t i, float4 v) {
    *reinterpret_cast<float4 *>(p + i) = v;
  }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  // four consecutive elements (8-byte aligned)
  __device__ __forceinline__ static float4 load4(const uint16_t *p, size_t i) {
    uint2 w = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y));
  }
  __device__ __forceinline__ static void store4(uint16_t *p, size_t i, float4 v) {
    *reinterpret_cast<uint2 *>(p + i) = pack_bf16x4(v.x, v.y, v.z, v.w);
  }
};

// ------------------------------------------------------------------ synchronisation
// Work-group barrier that orders LDS only.  A plain __syncthreads() also waits for
// every outstanding global load, which would stall register prefetches.
__device__ __forceinline__ void sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Make this wave's LDS writes visible to the rest of the same wave.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Sum over the lanes of a wave whose lane ids differ only in the bits of MASK
// (MASK = 31: over 32 consecutive lanes; MASK = 32: over the two half-waves).
template <int MASK>
__device__ __forceinline__ float lane_sum(float x) {
#pragma unroll
  for (int b = 1; b < 64; b <<= 1)
    if (MASK & b) x += __shfl_xor(x, b, 64);
  return x;
}

// Sums over lanes without LDS round trips, by DPP moves within 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over the N consecutive lanes of each aligned group (N = 2, 4, 8 or 16), in every
// lane of the group: quad swaps, then the half-row mirror (exact once the quads hold
// their sums), then a rotate by 8 within the row.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2, 4, 8 or 16 lanes");
  x += dpp_move<0xB1>(x);                              // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) x += dpp_move<0x4E>(x);        // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x += dpp_move<0x141>(x);       // row_half_mirror
  if constexpr (N >= 16) x += dpp_move<0x128>(x);      // row_ror:8
  return x;
}
// Sum over the 64 lanes of the wave (all active), wave-uniform.
__device__ __forceinline__ float wave_sum(float x) {
  const int r = __builtin_bit_cast(int, group_sum<16>(x));
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 48)));
}

// ------------------------------------------------------------------ streaming stores
// Non-temporal stores, for data that a kernel writes once and does not read back (the
// state after a step, per-token states, normalised and filtered outputs).  On MI355X
// they shorten the B = 64 decode step's state write-back by about a fifth and the
// per-token state stream by about 30% for the same bytes.  Loads stay ordinary: the
// same hint on the decode step's state loads made it slower.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(float *p, float4 v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store_nt(uint16_t *p, uint4 w) {
  __builtin_nontemporal_store(u32x4_nt{w.x, w.y, w.z, w.w}, reinterpret_cast<u32x4_nt *>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ------------------------------------------------------------------ short convolution
// One output of the causal width-W filter (W = 2..4) of a channel, before the activation:
//     z = tap[3] x + tap[4-W] h[4-W] + ... + tap[2] h[2]
// with x the current input and h[0..2] the three inputs before it (h[2] the newest).  The
// taps are right-aligned: tap[3] is the filter's last weight (the one that meets x) and
// tap[4-W .. 2] its first W-1, oldest first; window entries older than W-1 inputs are not
// read.  Every kernel that filters goes through these two functions in the same order of
// operations: at W = 4 they are the same operations, so the separate and the fused
// convolutions give the same bits; the fused kernels use conv_z4 for every width, and for
// a narrower filter its extra zero-tap products can only change the sign of a zero.
__device__ __forceinline__ float conv_z(const float (&tap)[4], float h0, float h1, float h2, float x, int W) {
  float z = tap[3] * x;
  if (W >= 4) z = __builtin_fmaf(tap[0], h0, z);
  if (W >= 3) z = __builtin_fmaf(tap[1], h1, z);
  return __builtin_fmaf(tap[2], h2, z);
}
// The same with all four taps applied (a narrower filter padded with zero taps on the left;
// its window entries there must be finite).
__device__ __forceinline__ float conv_z4(float4 tap, float h0, float h1, float h2, float x) {
  float z = tap.w * x;
  z = __builtin_fmaf(tap.x, h0, z);
  z = __builtin_fmaf(tap.y, h1, z);
  return __builtin_fmaf(tap.z, h2, z);
}
// z * sigmoid(z) from the hardware exp and reciprocal; 1 + e^-z = inf gives -0 for very
// negative z.
__device__ __forceinline__ float silu_act(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

}  // namespace kda
