// OCP MX quantiser (bf16 / fp32 rows -> canonical MXFP4) and the one-time
// canonical -> gfx950-preshuffled weight layout change.
//
// Quantiser, per 32-element block along K (the block-scaled format of the XFP
// blog, section "路线二：硬件格式（NVFP4 / MXFP4）", with the OCP Microscaling
// scale rule): scale byte = clamp(floor(log2 amax) - 2 + 127, 0, 254), i.e. the
// exponent field of amax minus 2; each element is divided by 2^(scale-127)
// (exact: a power of two) and rounded to the nearest E2M1 value, ties to the
// even code, saturating at 6.  A block holding NaN or inf gets scale 0xFF and
// zero codes.  Codes are packed two per byte, element 2i in the low nibble
// (campaign page "glm53-mxfp4-mi355x", section "A fused tensor with two dtypes
// in it": a packed row is half the logical width).
//
// With fp8 set the elements are E4M3 instead (MXFP8, one byte each): scale byte
// = clamp(floor(log2 amax) - 8 + 127, 0, 254), nearest E4M3, ties to the even
// code, saturating at 448; NaN/inf blocks as above.
#include "common.h"
#include "launch.h"

namespace mxmoe {

// one thread per 32-element block
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  const int64_t nblk_row = a.K / 32;
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.rows * nblk_row) return;
  const int64_t row = b / nblk_row, blk = b % nblk_row;
  float v[32];
  if (a.in_dtype == 0) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(a.in) + row * a.in_row_stride + blk * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4_t w = *reinterpret_cast<const u32x4_t*>(p + q * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[q * 8 + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  } else {
    const float* p = reinterpret_cast<const float*>(a.in) + row * a.in_row_stride + blk * 32;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      f32x4_t w = *reinterpret_cast<const f32x4_t*>(p + q * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[q * 4 + i] = w[i];
    }
  }
  uint32_t s;
  if (a.fp8) {
    uint32_t c8[8];
    mx8_quantize_block32(v, c8, &s);
    u32x4_t* o = reinterpret_cast<u32x4_t*>(a.codes + row * a.K + blk * 32);
    o[0] = (u32x4_t){c8[0], c8[1], c8[2], c8[3]};
    o[1] = (u32x4_t){c8[4], c8[5], c8[6], c8[7]};
  } else {
    uint32_t packed[4];
    mx_quantize_block32(v, packed, &s);
    u32x4_t o = {packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4_t*>(a.codes + row * (a.K / 2) + blk * 16) = o;
  }
  a.scales[row * nblk_row + blk] = (uint8_t)s;
}

// codes: one thread per 16-byte output unit
__global__ __launch_bounds__(256) void preshuffle_codes_kernel(PreshuffleArgs a) {
  const int64_t units_per_expert = a.N * a.K / 32;  // 16-byte units
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= a.E * units_per_expert) return;
  const int64_t e = u / units_per_expert;
  int64_t rem = u % units_per_expert;
  const int64_t nblk = a.K / 32;
  const int64_t rg = rem / (nblk * 16);
  rem %= nblk * 16;
  const int64_t b = rem / 16, r = rem % 16;
  int64_t row;
  if (a.interleave_gate_up)
    row = ((rg & 1) ? a.N / 2 : 0) + (rg >> 1) * 16 + r;
  else
    row = rg * 16 + r;
  const uint8_t* src = a.canon_codes + e * a.N * (a.K / 2) + row * (a.K / 2) + b * 16;
  *reinterpret_cast<u32x4_t*>(a.codes + u * 16) = *reinterpret_cast<const u32x4_t*>(src);
}

// scales: one thread per output byte; [E][N/16][ceil(K/512)][64 lanes][4]
__global__ __launch_bounds__(256) void preshuffle_scales_kernel(PreshuffleArgs a) {
  const int64_t sg = scale_groups(a.K);
  const int64_t per_expert = (a.N / 16) * sg * 256;
  const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= a.E * per_expert) return;
  const int64_t e = o / per_expert;
  int64_t rem = o % per_expert;
  const int64_t rg = rem / (sg * 256);
  rem %= sg * 256;
  const int64_t ktg = rem / 256;
  rem %= 256;
  const int64_t lane = rem / 4, j = rem % 4;
  const int64_t kt = ktg * 4 + j;
  const int64_t g = lane / 16, r = lane % 16;
  const int64_t b = kt * 4 + g;  // K-block index
  int64_t row;
  if (a.interleave_gate_up)
    row = ((rg & 1) ? a.N / 2 : 0) + (rg >> 1) * 16 + r;
  else
    row = rg * 16 + r;
  uint8_t v = 0;
  if (b < a.K / 32) v = a.canon_scales[e * a.N * (a.K / 32) + row * (a.K / 32) + b];
  a.scales[o] = v;
}

// Load-time conversion in one pass: fp32 or bf16 expert weights [E][N][K]
// (canonical row order; w13: gate rows then up rows) -> preshuffled MXFP4.
// One thread per (expert, row group, K-block of the padded K, row in group):
// it quantises the 32 elements of that block (the OCP rule of
// quantize_kernel) and writes the 16 code bytes and the scale byte where
// preshuffle_codes_kernel / preshuffle_scales_kernel put them; a block past K
// (the scale groups' padding) only writes a zero scale byte.
__global__ __launch_bounds__(256) void quantize_preshuffle_kernel(QuantPreshuffleArgs a) {
  const int64_t nblk = a.K / 32;
  const int64_t sg = scale_groups(a.K);
  const int64_t pblk = sg * 16;                      // K-blocks incl. padding
  const int64_t per_rg = pblk * 16;                  // threads per row group
  const int64_t per_expert = (a.N / 16) * per_rg;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.E * per_expert) return;
  const int64_t e = t / per_expert;
  int64_t rem = t % per_expert;
  const int64_t rg = rem / per_rg;
  rem %= per_rg;
  const int64_t b = rem / 16, r = rem % 16;          // K-block, row in group
  const int64_t row = a.interleave_gate_up ? ((rg & 1) ? a.N / 2 : 0) + (rg >> 1) * 16 + r : rg * 16 + r;
  // preshuffled scale byte: [rg][kt/4][lane = 16 (b % 4) + r][kt % 4], kt = b / 4
  const int64_t kt = b / 4;
  uint8_t* sdst = a.scales + e * scales_per_expert(a.N, a.K) + scales_group_offset(rg, kt / 4, a.K) +
                  ((b % 4) * 16 + r) * 4 + kt % 4;
  if (b >= nblk) {
    *sdst = 0;
    return;
  }
  float v[32];
  if (a.in_dtype == 0) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(a.in) + (e * a.N + row) * a.K + b * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4_t w = *reinterpret_cast<const u32x4_t*>(p + q * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[q * 8 + 2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      }
    }
  } else {
    const float* p = reinterpret_cast<const float*>(a.in) + (e * a.N + row) * a.K + b * 32;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      f32x4_t w = *reinterpret_cast<const f32x4_t*>(p + q * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[q * 4 + i] = w[i];
    }
  }
  uint32_t packed[4], sc;
  mx_quantize_block32(v, packed, &sc);
  // preshuffled codes: [rg][b][r][16 bytes]
  *reinterpret_cast<u32x4_t*>(a.codes + e * codes_per_expert(a.N, a.K) + rg * 16 * (a.K / 2) + (b * 16 + r) * 16) =
      (u32x4_t){packed[0], packed[1], packed[2], packed[3]};
  *sdst = (uint8_t)sc;
}

hipError_t launch_quantize_preshuffle(const QuantPreshuffleArgs& a, hipStream_t s) {
  const int64_t n = a.E * (a.N / 16) * scale_groups(a.K) * 16 * 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_preshuffle_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t nb = a.rows * (a.K / 32);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_preshuffle(const PreshuffleArgs& a, hipStream_t s) {
  const int64_t units = a.E * a.N * a.K / 32;
  const int64_t sbytes = a.E * (a.N / 16) * scale_groups(a.K) * 256;
  if (units > 0)
    hipLaunchKernelGGL(preshuffle_codes_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, a);
  if (sbytes > 0)
    hipLaunchKernelGGL(preshuffle_scales_kernel, dim3((unsigned)((sbytes + 255) / 256)), dim3(256), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace mxmoe
