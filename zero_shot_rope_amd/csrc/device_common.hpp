// device_common.hpp -- gfx950 device helpers shared by the bifocal attention kernels.
//
// Position arithmetic follows the Jet-Long pages (review page, Method; gist.science summary,
// Methodologie section 1): G = max(1, ceil(L / w_pretrained)), f(x) = floor(x / G), and the
// correction offset Delta_x = f(x) - x by which a base-position vector is rotated to reach
// its aliased position (gist.science summary, section 2: RoPE rotations compose additively).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bifocal {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A finite "minus infinity" for masked scores: exp2 of (this - any finite max) is exactly 0
// and (this - this) is 0, so no NaN can arise from fully masked rows or tiles.
constexpr float kNegBig = -1.0e30f;

// ---------------------------------------------------------------------------------------
// Position arithmetic (integers, bit-exact with the definition)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int aliased_position(int x, int G) { return x / G; }
__device__ __forceinline__ int correction_offset(int x, int G) { return x / G - x; }

// ---------------------------------------------------------------------------------------
// Correction rotation angles as fixed-point phases.
// For frequency omega_k the host passes W_k = round(2^32 * omega_k / (2 pi)) mod 2^32
// (turns per position step, 0.32 fixed point). The phase of offset Delta is
// (Delta * W_k) mod 2^32, an exact integer product, so the reduction of large angles
// (|Delta * omega| reaches ~1e5 rad at 128K) loses nothing; the only error is W_k's own
// rounding, |Delta| * pi * 2^-32 rad (7.2e-5 rad at |Delta| = 98303).
// The signed phase, times 2^-32, is the angle in turns in [-0.5, 0.5); the hardware sine
// and cosine (v_sin_f32 / v_cos_f32) take their argument in turns.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float phase_turns(int delta, uint32_t w) {
  const uint32_t ph = static_cast<uint32_t>(delta) * w;
  return static_cast<float>(static_cast<int32_t>(ph)) * 0x1p-32f;
}

__device__ __forceinline__ void turns_sincos(float t, float& s, float& c) {
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}

// ---------------------------------------------------------------------------------------
// bf16 <-> f32 (bf16 is the upper half of an f32; conversion to bf16 rounds to nearest even)
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Rotate 8 half-split pairs: lo[e] holds x_k, hi[e] holds x_{k + D/2} for k = k0 + e.
// Angles come from the phase W[e] * delta. Writes the rotated pairs back as bf16.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, int delta, const uint32_t* W) {
  u32x4 olo, ohi;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float x0 = bf16lo(lo[w]), x1 = bf16hi(lo[w]);
    float y0 = bf16lo(hi[w]), y1 = bf16hi(hi[w]);
    float s0, c0, s1, c1;
    turns_sincos(phase_turns(delta, W[2 * w]), s0, c0);
    turns_sincos(phase_turns(delta, W[2 * w + 1]), s1, c1);
    olo[w] = pack_bf16x2(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
    ohi[w] = pack_bf16x2(x0 * s0 + y0 * c0, x1 * s1 + y1 * c1);
  }
  lo = olo;
  hi = ohi;
}

// acc + lo(pk) + hi(pk) for a packed bf16 pair (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t pk, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

// True on every lane when `pred` holds on any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// ---------------------------------------------------------------------------------------
// MFMA 32x32x16 bf16 -> f32. Operand/result lane layout (wave64):
//   A[i][k]: lane i + 32*(k/8), element k%8      (k < 16)
//   B[k][j]: lane j + 32*(k/8), element k%8
//   C[i][j]: lane j + 32*((i/4)%2), register 4*(i/8) + i%4
// Only the (lane/32, element) -> k correspondence shared by A and B matters for the sum.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// MFMA 16x16x32 bf16 -> f32. Operand/result lane layout (wave64):
//   A[i][k]: lane i + 16*(k/8), element k%8      (k < 32)
//   B[k][j]: lane j + 16*(k/8), element k%8
//   C[i][j]: lane j + 16*(i/4), register i%4
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Value of lane l^32 (the other half of the wave) for every lane, via v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row index (within a 32-row MFMA block) held by register r of lane half h.
__device__ __forceinline__ constexpr int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------------------
// LDS tiles: swizzled layout, direct global->LDS loads, transposed reads
// ---------------------------------------------------------------------------------------
// Key/value tiles are row-major with 16-byte chunk c of row r stored at position c ^ swz(r).
// LDS has 64 four-byte banks, i.e. one 256-byte line. D = 128 (one row per line): swz(r) is a
// 4-bit permutation of r mod 16, so 16 consecutive rows read at one chunk (the K operand,
// ds_read_b128, 16 lanes per cycle) hit 16 distinct bank groups, and 4 consecutive rows read
// at chunks 0..3 (the transposed V operand, ds_read_b64_tr_b16, 32 lanes per cycle) hit
// disjoint groups. D = 64 (two rows per line): the same two properties per row parity.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

#define LDS_AS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void load_lds16(const void* g, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (LDS_AS void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposed read: within each 16-lane group, lane r names 4 consecutive bf16 of row r of a
// 16x4 block M; lane i receives M[4e + i/4][i%4] for e = 0..3.
__device__ __forceinline__ u32x2 read_tr(const uint16_t* lds) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(lds));
  return __builtin_bit_cast(u32x2, r);
}


}  // namespace bifocal
