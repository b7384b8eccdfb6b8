// Experts kept in bf16 inside a fused expert buffer whose other experts are
// packed MXFP4 (campaign page "glm53-mxfp4-mi355x", section "A fused tensor
// with two dtypes in it": the exclusion set is per expert).  The routing gives
// such an expert its counts, offsets and sorted positions but no MXFP4 tiles;
// these two kernels compute its rows: gate_up + clamped SwiGLU into act, and
// down + the combine's contribution (fp32 atomics of w * y into out32, or y
// into the slot-ordered buffer), both on bf16 activations in every mode.
//
// Excluded experts are expected to be few, so the kernels are plain: a
// workgroup owns RT x 16 rows of one expert and 16 output features, its NW
// waves split K evenly and each runs its part with v_mfma_f32_16x16x32_bf16
// (lane group g takes K elements 8g..8g+7 of each 32-wide step), the weight
// operand loaded once per step and reused for the RT row blocks; the partial
// sums meet in LDS and wave 0 writes the results.  A and B rows are read
// straight from global memory.  Rows beyond an expert's count are never
// loaded or stored.
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

// The expert of this workgroup's bf16 slot j.
__device__ __forceinline__ Rows slot_rows(const XArgs& a, int j) {
  Rows r;
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

// acc[m][rb] += A(row block rb) * B_m^T over this wave's K range [k_lo, k_lo + kw),
// for NB weight row blocks b[m] (16 rows each).  a_row[rb]: the lane's A row
// (null: a row past the count, zeros).
// KB steps of loads are issued before their MFMAs, so a wave has KB steps in
// flight instead of one.
template <int RT, int NB, int KB>
__device__ __forceinline__ void dot_steps(const uint16_t* const (&a_row)[RT], const uint16_t* const (&b)[NB],
                                          int64_t k0, f32x4_t (&acc)[NB][RT]) {
  u32x4_t bv[KB][NB], av[KB][RT];
#pragma unroll
  for (int t = 0; t < KB; ++t)
#pragma unroll
    for (int m = 0; m < NB; ++m) bv[t][m] = load16(b[m] + k0 + 32 * t);
#pragma unroll
  for (int t = 0; t < KB; ++t)
#pragma unroll
    for (int rb = 0; rb < RT; ++rb)
      av[t][rb] = a_row[rb] ? load16(a_row[rb] + k0 + 32 * t) : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < KB; ++t)
#pragma unroll
    for (int rb = 0; rb < RT; ++rb)
#pragma unroll
      for (int m = 0; m < NB; ++m) acc[m][rb] = mfma_bf16(av[t][rb], bv[t][m], acc[m][rb]);
}

template <int RT, int NB>
__device__ __forceinline__ void wave_dot(const uint16_t* const (&a_row)[RT], const uint16_t* const (&b)[NB],
                                         int64_t kw, f32x4_t (&acc)[NB][RT]) {
  constexpr int KB = 4;
  int64_t k0 = 0;
  for (; k0 + 32 * KB <= kw; k0 += 32 * KB) dot_steps<RT, NB, KB>(a_row, b, k0, acc);
  for (; k0 < kw; k0 += 32) dot_steps<RT, NB, 1>(a_row, b, k0, acc);
}

// Sum of the NW waves' partials into wave 0's acc (waves 1.. store to red).
template <int NW, int RT, int NB>
__device__ __forceinline__ bool reduce_waves(f32x4_t (&acc)[NB][RT], f32x4_t* red) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  if (wave > 0)
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int rb = 0; rb < RT; ++rb) red[(((wave - 1) * NB + m) * RT + rb) * 64 + lane] = acc[m][rb];
  __syncthreads();
  if (wave == 0)
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int rb = 0; rb < RT; ++rb) acc[m][rb] += red[(((w - 1) * NB + m) * RT + rb) * 64 + lane];
  return wave == 0;
}

// gate_up + SwiGLU.  grid: (n * I/16, row tiles); NW waves
template <int RT, int NW>
__global__ __launch_bounds__(64 * NW) void bf16x_gate_up_kernel(XArgs a) {
  __shared__ f32x4_t red[(NW - 1) * 2 * RT * 64];
  const int64_t I = a.N / 2, K = a.K, kw = K / NW;
  const int nfb = (int)(I / 16);
  const Rows rr = slot_rows(a, (int)(blockIdx.x / nfb));
  if (rr.e < 0) return;
  const int64_t j = blockIdx.x / nfb, fb = blockIdx.x % nfb;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int64_t k_lo = wave * kw + 8 * g;
  const uint16_t* const b[2] = {a.w + (j * a.N + fb * 16 + r) * K + k_lo,        // gate row fb*16 + r
                                a.w + (j * a.N + I + fb * 16 + r) * K + k_lo};   // up row I + fb*16 + r
  for (int32_t r0 = (int32_t)blockIdx.y * 16 * RT; r0 < rr.cnt; r0 += (int32_t)gridDim.y * 16 * RT) {
    const uint16_t* a_row[RT];
#pragma unroll
    for (int rb = 0; rb < RT; ++rb) {
      const int32_t row = r0 + rb * 16 + r;
      a_row[rb] = row < rr.cnt ? a.a + (int64_t)a.pos_tok[rr.off + row] * K + k_lo : nullptr;
    }
    f32x4_t acc[2][RT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rb = 0; rb < RT; ++rb) acc[m][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    wave_dot<RT, 2>(a_row, b, kw, acc);
    if (reduce_waves<NW, RT, 2>(acc, red)) {
      // D: lane holds feature fb*16 + r of rows 4g .. 4g + 3 of each row block
#pragma unroll
      for (int rb = 0; rb < RT; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t row = r0 + rb * 16 + 4 * g + q;
          if (row < rr.cnt)
            a.act[(int64_t)(rr.off + row) * I + fb * 16 + r] =
                (uint16_t)f32_to_bf16_bits(swiglu_clamped(acc[0][rb][q], acc[1][rb][q], a.clamp_limit));
        }
    }
    __syncthreads();
  }
}

// down + combine.  grid: (n * H/16, row tiles); NW waves
template <int RT, int NW, bool ORDERED>
__global__ __launch_bounds__(64 * NW) void bf16x_down_kernel(XArgs a) {
  __shared__ f32x4_t red[(NW - 1) * RT * 64];
  const int64_t H = a.N, K = a.K, kw = K / NW;
  const int nfb = (int)(H / 16);
  const Rows rr = slot_rows(a, (int)(blockIdx.x / nfb));
  if (rr.e < 0) return;
  const int64_t j = blockIdx.x / nfb, fb = blockIdx.x % nfb;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int64_t k_lo = wave * kw + 8 * g;
  const uint16_t* const b[1] = {a.w + (j * a.N + fb * 16 + r) * K + k_lo};
  for (int32_t r0 = (int32_t)blockIdx.y * 16 * RT; r0 < rr.cnt; r0 += (int32_t)gridDim.y * 16 * RT) {
    const uint16_t* a_row[RT];
#pragma unroll
    for (int rb = 0; rb < RT; ++rb) {
      const int32_t row = r0 + rb * 16 + r;
      a_row[rb] = row < rr.cnt ? a.a + (int64_t)(rr.off + row) * K + k_lo : nullptr;  // act row, sorted order
    }
    f32x4_t acc[1][RT];
#pragma unroll
    for (int rb = 0; rb < RT; ++rb) acc[0][rb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    wave_dot<RT, 1>(a_row, b, kw, acc);
    if (reduce_waves<NW, RT, 1>(acc, red)) {
      const int64_t n = fb * 16 + r;
#pragma unroll
      for (int rb = 0; rb < RT; ++rb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t row = r0 + rb * 16 + 4 * g + q;
          if (row < rr.cnt) {
            const int64_t p = rr.off + row;
            if constexpr (ORDERED)
              a.ybuf[p * H + n] = acc[0][rb][q];
            else
              unsafeAtomicAdd(a.out32 + (int64_t)a.pos_tok[p] * H + n, a.pos_w[p] * acc[0][rb][q]);
          }
        }
    }
    __syncthreads();
  }
}

// Row blocks per workgroup by the expected rows of an expert (as the MXFP4
// plans: T k / E_global), and waves by K.
struct XPlan {
  int rt, nw;
};
XPlan x_plan(const XArgs& a) {
  const int64_t rows = a.rows_per_expert;
  return {rows > 24 ? 4 : 1, (a.K / 32) % 8 == 0 ? 8 : 4};
}

dim3 x_grid(const XArgs& a, int64_t features, int rt) {
  int64_t tiles = (a.T + 16 * rt - 1) / (16 * rt);
  if (tiles > kRowTilesMax) tiles = kRowTilesMax;
  if (tiles < 1) tiles = 1;
  return dim3((unsigned)(features / 16 * a.n), (unsigned)tiles);
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

template <int RT, int NW>
void gate_up_rt_nw(const XArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((bf16x_gate_up_kernel<RT, NW>), grid, dim3(64 * NW), 0, s, a);
}
template <int RT, int NW>
void down_rt_nw(const XArgs& a, dim3 grid, bool ordered, hipStream_t s) {
  if (ordered)
    hipLaunchKernelGGL((bf16x_down_kernel<RT, NW, true>), grid, dim3(64 * NW), 0, s, a);
  else
    hipLaunchKernelGGL((bf16x_down_kernel<RT, NW, false>), grid, dim3(64 * NW), 0, s, a);
}

hipError_t launch_bf16x_gate_up(const XArgs& a, hipStream_t s) {
  if (a.n <= 0 || a.T <= 0) return hipSuccess;
  if (a.K % 128 || a.N % 32) return hipErrorInvalidValue;
  const XPlan p = x_plan(a);
  const dim3 grid = x_grid(a, a.N / 2, p.rt);
  if (p.rt == 4) {
    if (p.nw == 8) gate_up_rt_nw<4, 8>(a, grid, s); else gate_up_rt_nw<4, 4>(a, grid, s);
  } else {
    if (p.nw == 8) gate_up_rt_nw<1, 8>(a, grid, s); else gate_up_rt_nw<1, 4>(a, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_bf16x_down(const XArgs& a, bool ordered, hipStream_t s) {
  if (a.n <= 0 || a.T <= 0) return hipSuccess;
  if (a.K % 128 || a.N % 16) return hipErrorInvalidValue;
  const XPlan p = x_plan(a);
  const dim3 grid = x_grid(a, a.N, p.rt);
  if (p.rt == 4) {
    if (p.nw == 8) down_rt_nw<4, 8>(a, grid, ordered, s); else down_rt_nw<4, 4>(a, grid, ordered, s);
  } else {
    if (p.nw == 8) down_rt_nw<1, 8>(a, grid, ordered, s); else down_rt_nw<1, 4>(a, grid, ordered, s);
  }
  return hipGetLastError();
}

}  // namespace mxmoe
