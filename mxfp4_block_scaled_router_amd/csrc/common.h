// Internal definitions shared by the HIP kernels and the C-ABI host code of the
// MXFP4 routed-expert MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxmoe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// ---------------------------------------------------------------------------
// Preshuffled weight layout (per expert, per matrix of N rows x K columns).
//
// Rows are taken in groups of 16.  Within a row group the 16-byte MX blocks
// (32 E2M1 codes = one UE8M0 scale) are stored block-major:
//     codes[rg][b][r][16 bytes]      b = K-block (K/32 of them), r = row in group
// so the 64 lanes of a wave that load lane*16 bytes from (rg, kt) get
//     lane l -> row r = l % 16, block b = 4*kt + l / 16
// which is exactly the B operand of one 16x16x128 FP4 MFMA, or of four
// 16x16x32 bf16 MFMAs after unpacking (lane group g = l/16 supplies K
// elements 32*g .. 32*g+31 of the 128-element k-tile).
//
// Scales: one byte per (row, block), grouped per lane and per 4 k-tiles:
//     scales[rg][kt/4][lane][kt%4]   (K padded up to a multiple of 512)
// so one dword load per lane covers 4 k-tiles.
//
// w13 interleaves gate and up row groups: preshuffled row group 2i holds gate
// rows 16i..16i+15, row group 2i+1 holds up rows I+16i..I+16i+15.
// ---------------------------------------------------------------------------
constexpr int kRowsPerGroup = 16;
constexpr int kBlockK = 32;
constexpr int kTileK = 128;
constexpr int kScaleGroupK = 512;

__host__ __device__ inline int64_t codes_per_expert(int64_t N, int64_t K) { return N * (K / 2); }
__host__ __device__ inline int64_t scale_groups(int64_t K) {
  return (K + kScaleGroupK - 1) / kScaleGroupK;
}
__host__ __device__ inline int64_t scales_per_expert(int64_t N, int64_t K) {
  return (N / kRowsPerGroup) * scale_groups(K) * 256;
}
// byte offset of row group rg, k-tile kt inside one expert's codes
__host__ __device__ inline int64_t codes_tile_offset(int64_t rg, int64_t kt, int64_t K) {
  return rg * kRowsPerGroup * (K / 2) + kt * 1024;
}
// byte offset of the scale dword of (rg, k-tile group kt/4) for lane 0
__host__ __device__ inline int64_t scales_group_offset(int64_t rg, int64_t ktg, int64_t K) {
  return (rg * scale_groups(K) + ktg) * 256;
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
// UE8M0 byte -> the f32 scale operand of v_cvt_scalef32_*: the instruction uses
// only the exponent field (E8M0 semantics: 2^(S-127), 0xFF = NaN).  The 0x400000
// mantissa bit keeps S = 0 and S = 255 distinct from 0.0f and +inf.
__device__ __forceinline__ float e8m0_scale_operand(uint32_t s) {
  return __builtin_bit_cast(float, (s << 23) | 0x400000u);
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) -> 8 bf16 values
// E2M1 * 2^(S-127), exact.  The bf16x2 results are read as whole words.
__device__ __forceinline__ bf16x8_t unpack8_e2m1(uint32_t codes, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Clamped SwiGLU in fp32: gate clamped from above, up clamped both ways; the
// comparisons are false for NaN, so NaN passes through (no min/max instructions).
__device__ __forceinline__ float swiglu_clamped(float g, float u, float limit) {
  float gc = (g > limit) ? limit : g;
  float uc = (u > limit) ? limit : ((u < -limit) ? -limit : u);
  // v_rcp_f32 (1 ulp) instead of an IEEE division: the division's dozen
  // instructions per element were a large share of the epilogues
  float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gc));
  return (gc * sig) * uc;
}

// E2M1 magnitude code of a >= 0 (already divided by the block scale): nearest
// grid point, ties to the even code, saturating at 6.  The grid midpoints are
// 0.25 0.75 1.25 1.75 2.5 3.5 5; a tie rounds towards the even neighbour.
__device__ __forceinline__ uint32_t e2m1_magnitude_code(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// OCP MX scale byte for a block whose largest finite magnitude is amax (as fp32
// bits, sign cleared): floor(log2 amax) - 2 + 127 = exponent field - 2, clamped
// to [0, 254]; subnormal and zero amax give 0.
__device__ __forceinline__ uint32_t mx_scale_from_amax_bits(uint32_t amax_bits) {
  int ef = (int)(amax_bits >> 23);
  int s = ef - 2;
  s = s < 0 ? 0 : s;
  s = s > 254 ? 254 : s;
  return (uint32_t)s;
}

// 2^(127 - s) as fp32 for s in [0, 254]: the factor that divides by the block
// scale.  For s <= 253 it is a normal power of two; s = 254 needs 2^-127, which
// is applied in two exact steps by the caller's multiply chain.
__device__ __forceinline__ float mx_inv_scale(uint32_t s) {
  int e = 254 - (int)s;  // exponent field of 2^(127-s)
  if (e >= 1) return __builtin_bit_cast(float, (uint32_t)e << 23);
  return __builtin_bit_cast(float, 0x00400000u);  // 2^-127 (subnormal, exact)
}

// Quantise 32 fp32 values (one MX block) to 16 packed code bytes + a scale byte.
__device__ __forceinline__ void mx_quantize_block32(const float* v, uint32_t* packed4,
                                                    uint32_t* scale_out) {
  uint32_t amax_bits = 0;
  bool nonfinite = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t b = __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu;
    nonfinite |= (b >= 0x7F800000u);
    amax_bits = b > amax_bits ? b : amax_bits;
  }
  if (nonfinite) {
    packed4[0] = packed4[1] = packed4[2] = packed4[3] = 0;
    *scale_out = 255;
    return;
  }
  uint32_t s = mx_scale_from_amax_bits(amax_bits);
  float inv = mx_inv_scale(s);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = v[w * 8 + i];
      uint32_t sign = __builtin_bit_cast(uint32_t, x) >> 31;
      float a = __builtin_fabsf(x) * inv;
      word |= ((sign << 3) | e2m1_magnitude_code(a)) << (4 * i);
    }
    packed4[w] = word;
  }
  *scale_out = s;
}

// ---- MXFP8 (E4M3 elements: bias 7, 3 mantissa bits, largest 448, 0x7F NaN)

// E4M3 magnitude code of a >= 0 (already divided by the block scale): round to
// nearest, ties to the even code, saturating at 448 (code 0x7E).  Below 2^-6
// the grid step is 2^-9 (subnormals: code = a * 512 rounded); above, rounding
// the fp32 significand to 3 bits (nearest, ties to even, a carry moves into
// the exponent) and rebiasing the exponent from 127 to 7 gives the code.
__device__ __forceinline__ uint32_t e4m3_magnitude_code(float a) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;  // exponent field << 3 | 3 mantissa bits
  const uint32_t code = r - (120u << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// MXFP8 scale byte: floor(log2 amax) - 8 + 127 = exponent field - 8, clamped to
// [0, 254] (8 is the largest E4M3 exponent).
__device__ __forceinline__ uint32_t mx8_scale_from_amax_bits(uint32_t amax_bits) {
  int s = (int)(amax_bits >> 23) - 8;
  s = s < 0 ? 0 : s;
  s = s > 254 ? 254 : s;
  return (uint32_t)s;
}

// Quantise 32 fp32 values (one MX block) to 32 E4M3 code bytes + a scale byte.
__device__ __forceinline__ void mx8_quantize_block32(const float* v, uint32_t* codes8,
                                                     uint32_t* scale_out) {
  uint32_t amax_bits = 0;
  bool nonfinite = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t b = __builtin_bit_cast(uint32_t, v[i]) & 0x7FFFFFFFu;
    nonfinite |= (b >= 0x7F800000u);
    amax_bits = b > amax_bits ? b : amax_bits;
  }
  if (nonfinite) {
#pragma unroll
    for (int w = 0; w < 8; ++w) codes8[w] = 0;
    *scale_out = 255;
    return;
  }
  uint32_t s = mx8_scale_from_amax_bits(amax_bits);
  float inv = mx_inv_scale(s);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = v[w * 4 + i];
      uint32_t sign = __builtin_bit_cast(uint32_t, x) >> 31;
      float a = __builtin_fabsf(x) * inv;
      word |= ((sign << 7) | e4m3_magnitude_code(a)) << (8 * i);
    }
    codes8[w] = word;
  }
  *scale_out = s;
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Streaming loads of weight data, read once per step: the non-temporal hint
// keeps them from displacing reusable lines (activations, tables) in L2/MALL
// and measurably raises HBM read bandwidth on gfx950.
__device__ __forceinline__ u32x4_t ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t ld_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

}  // namespace mxmoe
