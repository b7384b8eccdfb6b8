// Experts kept in bf16 inside a fused expert buffer whose other experts are
// packed MXFP4 (campaign page "glm53-mxfp4-mi355x", section "A fused tensor
// with two dtypes in it": the exclusion set is per expert).  The routing gives
// such an expert its counts, offsets and sorted positions but no MXFP4 tiles;
// these two kernels compute its rows: gate_up + clamped SwiGLU into act, and
// down + the combine's contribution (fp32 atomics of w * y into out32, or y
// into the slot-ordered buffer), both on bf16 activations in every mode.
//
// Excluded experts are expected to be few, so the kernels are plain: a wave
// owns 16 rows of one expert x 16 output features and runs the whole K with
// v_mfma_f32_16x16x32_bf16, A rows and B rows read straight from global memory
// (lane group g takes K elements 8g..8g+7 of each 32-wide step); four waves per
// workgroup take adjacent feature blocks.  Rows beyond an expert's count are
// never loaded or stored.
#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

constexpr int kRowTilesMax = 4096;  // grid.y bound; larger row counts loop

struct Rows {
  int e = -1;       // table expert, -1: nothing to do
  int32_t cnt = 0;  // its rows
  int32_t off = 0;  // its first sorted position
};

// The expert of this workgroup's bf16 slot (blockIdx.x / feature blocks).
__device__ __forceinline__ Rows slot_rows(const XArgs& a, int fbw) {
  Rows r;
  const int j = (int)(blockIdx.x / fbw);
  const int e = a.xmap[a.E_local + j];
  if ((unsigned)e >= (unsigned)a.E_local) return r;
  r.e = e;
  r.cnt = a.counts[e];
  r.off = a.offsets[e];
  return r;
}

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// grid: (n * ceil(I / 64), min(ceil(T / 16), kRowTilesMax)); 256 threads
__global__ __launch_bounds__(256) void bf16x_gate_up_kernel(XArgs a) {
  const int64_t I = a.N / 2, K = a.K;
  const int fbw = (int)((I + 63) / 64);
  const Rows rr = slot_rows(a, fbw);
  if (rr.e < 0) return;
  const int j = (int)(blockIdx.x / fbw);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t fb = (int64_t)(blockIdx.x % fbw) * 4 + wave;  // 16-feature block of act
  if (fb * 16 >= I) return;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* wg = a.w + ((int64_t)j * a.N + fb * 16 + r) * K + 8 * g;  // gate row fb*16 + r
  const uint16_t* wu = wg + I * K;                                           // up row I + fb*16 + r
  for (int32_t r0 = (int32_t)blockIdx.y * 16; r0 < rr.cnt; r0 += (int32_t)gridDim.y * 16) {
    const int32_t p0 = rr.off + r0;
    const bool valid = r0 + r < rr.cnt;
    const uint16_t* xr = a.a + (int64_t)(valid ? a.pos_tok[p0 + r] : 0) * K + 8 * g;
    f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int64_t k0 = 0; k0 < K; k0 += 32) {
      const u32x4_t xv = valid ? load16(xr + k0) : (u32x4_t){0u, 0u, 0u, 0u};
      ag = mfma_bf16(xv, load16(wg + k0), ag);
      au = mfma_bf16(xv, load16(wu + k0), au);
    }
    // D: lane holds feature fb*16 + r of rows 4g .. 4g + 3
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 4 * g + q;
      if (r0 + row < rr.cnt)
        a.act[(int64_t)(p0 + row) * I + fb * 16 + r] =
            (uint16_t)f32_to_bf16_bits(swiglu_clamped(ag[q], au[q], a.clamp_limit));
    }
  }
}

// grid: (n * ceil(H / 64), min(ceil(T / 16), kRowTilesMax)); 256 threads
template <bool ORDERED>
__global__ __launch_bounds__(256) void bf16x_down_kernel(XArgs a) {
  const int64_t H = a.N, K = a.K;
  const int fbw = (int)((H + 63) / 64);
  const Rows rr = slot_rows(a, fbw);
  if (rr.e < 0) return;
  const int j = (int)(blockIdx.x / fbw);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t fb = (int64_t)(blockIdx.x % fbw) * 4 + wave;  // 16-feature block of y
  if (fb * 16 >= H) return;
  const int r = lane & 15, g = lane >> 4;
  const uint16_t* wr = a.w + ((int64_t)j * a.N + fb * 16 + r) * K + 8 * g;
  for (int32_t r0 = (int32_t)blockIdx.y * 16; r0 < rr.cnt; r0 += (int32_t)gridDim.y * 16) {
    const int32_t p0 = rr.off + r0;
    const bool valid = r0 + r < rr.cnt;
    const uint16_t* ar = a.a + (int64_t)(valid ? p0 + r : 0) * K + 8 * g;  // act row of position p0 + r
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int64_t k0 = 0; k0 < K; k0 += 32) {
      const u32x4_t av = valid ? load16(ar + k0) : (u32x4_t){0u, 0u, 0u, 0u};
      acc = mfma_bf16(av, load16(wr + k0), acc);
    }
    const int64_t n = fb * 16 + r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 4 * g + q;
      if (r0 + row < rr.cnt) {
        const int64_t p = p0 + row;
        if constexpr (ORDERED)
          a.ybuf[p * H + n] = acc[q];
        else
          unsafeAtomicAdd(a.out32 + (int64_t)a.pos_tok[p] * H + n, a.pos_w[p] * acc[q]);
      }
    }
  }
}

dim3 x_grid(const XArgs& a, int64_t features) {
  const int64_t fbw = (features + 63) / 64;
  int64_t rt = (a.T + 15) / 16;
  if (rt > kRowTilesMax) rt = kRowTilesMax;
  if (rt < 1) rt = 1;
  return dim3((unsigned)(fbw * a.n), (unsigned)rt);
}

__global__ __launch_bounds__(256) void expert_map_kernel(ExpertMapArgs m, int32_t* map) {
  for (int e = threadIdx.x; e < m.E; e += blockDim.x) {
    const bool x = (m.bits[e >> 5] >> (e & 31)) & 1u;
    int j = 0;
    for (int w = 0; w < (e >> 5); ++w) j += __builtin_popcount(m.bits[w]);
    j += __builtin_popcount(m.bits[e >> 5] & ((1u << (e & 31)) - 1u));
    map[e] = x ? j : -1;
    if (x) map[m.E + j] = e;
  }
}

}  // namespace

hipError_t launch_expert_map(const ExpertMapArgs& m, int32_t* map, hipStream_t s) {
  if (m.E <= 0 || m.E > kExpertMapMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_map_kernel, dim3(1), dim3(256), 0, s, m, map);
  return hipGetLastError();
}

hipError_t launch_bf16x_gate_up(const XArgs& a, hipStream_t s) {
  if (a.n <= 0 || a.T <= 0) return hipSuccess;
  if (a.K % 32 || a.N % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bf16x_gate_up_kernel, x_grid(a, a.N / 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bf16x_down(const XArgs& a, bool ordered, hipStream_t s) {
  if (a.n <= 0 || a.T <= 0) return hipSuccess;
  if (a.K % 32 || a.N % 16) return hipErrorInvalidValue;
  if (ordered)
    hipLaunchKernelGGL(bf16x_down_kernel<true>, x_grid(a, a.N), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(bf16x_down_kernel<false>, x_grid(a, a.N), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mxmoe
