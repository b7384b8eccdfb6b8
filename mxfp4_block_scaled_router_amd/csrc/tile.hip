// Grouped GEMMs for token tiles of up to 128 rows (prefill and the A4 path):
// the MFMA work is the cost, so a workgroup owns a 128-token x 256-weight-row
// output tile of one expert and streams K through LDS.
//
//   gate_up:  h = W13_e x_t, fused with the clamped SwiGLU -> act (bf16)
//   down:     y = W2_e a, fused with the weighted combine (fp32 atomics into
//             out32, or y rows for the ordered gather)
//
// Staging.  Each k-tile (128 of K) of the activation rows and of the 16
// preshuffled weight row groups (codes and the scale dwords that cover it)
// is copied straight from global memory into an LDS ring of STAGES slots by
// the gfx950 global->LDS load (a wave's instruction writes 64 x 16 bytes, lane
// i at slot + 16 i, from any per-lane address), so staging costs no registers.
// Every wave issues the same number of copies per k-tile; before using slot
// kt a wave waits until only the later stages' copies are outstanding, and one
// barrier per k-tile then publishes the slot to the whole workgroup and frees
// the slot the next copy writes (it was read in the previous iteration).
//
// Bank conflicts.  The activation rows are stored with their 16-byte chunks
// XOR-swizzled by the row (bf16: chunk c of row r at c ^ (r & 15); MXFP4:
// block c at c ^ ((r >> 2) & 3)), chosen through the per-lane source address
// of the copy, so the 16 lanes that read one MFMA operand hit 16 distinct
// 16-byte bank groups.  Weight codes and scales are read lane-contiguously.
//
// MFMA layout: as in the other GEMMs (lane l: row l%16, MX block l/16 of the
// k-tile; K element 8m+e of the block feeds bf16 MFMA m).  Eight waves form a
// 2 x 4 grid (two per SIMD, so one wave's unpacking overlaps the other's
// MFMAs); wave (wm, wn) owns rows 64 wm.. and weight row groups 4 wn..4 wn+3.
//
// Schedule.  Work items (row tile, 256-row weight block) are numbered
// tile-major; workgroup b runs on XCD b % 8 (round-robin dispatch), and each
// XCD takes a contiguous eighth of the items, so the workgroups resident on one
// XCD share activation tiles and weight blocks in that XCD's L2.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) int32_t const_i32;

constexpr int kMT = 128;        // token rows per tile
constexpr int kNT = 256;        // weight rows per tile
constexpr int kNRG = kNT / 16;  // weight row groups per tile
constexpr int kWaves = 8;       // 2 (rows) x 4 (weight row groups)
constexpr int kThreads = 64 * kWaves;

template <bool AFP4>
struct Cfg {
  static constexpr int A_BYTES = AFP4 ? kMT * 64 : kMT * 256;  // activation k-tile
  static constexpr int AS_BYTES = AFP4 ? kMT * 4 : 0;           // activation scale bytes
  static constexpr int B_BYTES = kNRG * 1024;                   // weight codes
  static constexpr int BS_BYTES = kNRG * 256;                   // weight scale dwords
  static constexpr int A_OFF = 0, AS_OFF = A_BYTES, B_OFF = A_BYTES + AS_BYTES, BS_OFF = B_OFF + B_BYTES;
  static constexpr int STAGE = BS_OFF + BS_BYTES;
  static constexpr int STAGES = AFP4 ? 4 : 3;
  static constexpr int A_CP = A_BYTES / 1024 / kWaves;  // copies per wave per k-tile
  static constexpr int AS_CP = AFP4 ? 1 : 0;  // 2 copies, made by the even and the odd waves alike
  static constexpr int B_CP = kNRG / kWaves;
  static constexpr int CP = A_CP + AS_CP + 2 * B_CP;
  static constexpr int ROWS_OFF = STAGES * STAGE;  // int32 [kMT]: A row index of each tile row
  static constexpr int LDS = ROWS_OFF + kMT * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((STAGES - 2) * CP < 64, "vmcnt range");
};

// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 encoding:
// vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void copy16(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void copy4(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

struct TileItem {
  int e, rows;
  int64_t p0;
  int n0;  // first weight row
};

// Item of this workgroup, or false.  XCD x = blockIdx % 8 takes items
// [x * per, x * per + per).
__device__ __forceinline__ bool tile_item(const GemmArgs& a, int ntl, TileItem* it) {
  const int n = ((const_i32*)a.tile_off)[a.E_local];
  const int items = n * ntl;
  const int per = (items + 7) / 8;
  const int b = blockIdx.x;
  const int j = b >> 3;
  const int item = (b & 7) * per + j;
  if (j >= per || item >= items) return false;
  const int t = item / ntl;
  const_i32* ti = (const_i32*)a.tiles + 4 * (int64_t)t;
  it->e = ti[0];
  it->rows = ti[1];
  it->p0 = ti[2];
  it->n0 = (item - t * ntl) * kNT;
  return true;
}

__device__ __forceinline__ void zero_duty(const GemmArgs& a) {
  if (!a.zero_buf) return;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = tid; i < a.zero_n / 4; i += nthreads) reinterpret_cast<f32x4_t*>(a.zero_buf)[i] = z;
}

// The k-loop: acc[rb][cb] += A(rows 64 wm + 16 rb ..) * W(row group 8 wn + cb)^T
// over all of K.  rowidx: LDS table of the A-matrix row of each tile row.
template <bool AFP4>
__device__ __forceinline__ void tile_mainloop(const GemmArgs& a, const TileItem& it, int64_t K, int64_t N,
                                              uint8_t* lds, f32x4_t (&acc)[4][4]) {
  using C = Cfg<AFP4>;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int KT = (int)(K / kTileK);
  const int32_t* rowidx = reinterpret_cast<const int32_t*>(lds + C::ROWS_OFF);

  // ---- per-lane copy sources (k-tile 0); k-tile kt adds kt * stride
  const uint8_t* a_src[C::A_CP];
  const uint8_t* as_src = nullptr;
  if constexpr (!AFP4) {
    const int64_t rb = K * 2;  // bytes per activation row
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;  // rows 4j .. 4j+3
      const int row = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      a_src[jj] = reinterpret_cast<const uint8_t*>(a.a_bf16) + (int64_t)rowidx[row] * rb + c * 16;
    }
  } else {
    const int64_t rb = K / 2;
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;  // rows 16j .. 16j+15
      const int row = 16 * j + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      a_src[jj] = a.a_codes + (int64_t)rowidx[row] * rb + c * 16;
    }
    const int row = 64 * (wave & 1) + lane;
    as_src = a.a_scales + (int64_t)rowidx[row] * (K / 32);  // waves 2.. repeat waves 0/1 (same bytes)
  }
  const int64_t cpe = codes_per_expert(N, K), spe = scales_per_expert(N, K);
  const uint8_t* ecodes = a.w_codes + (int64_t)it.e * cpe;
  const uint8_t* escales = a.w_scales + (int64_t)it.e * spe;
  const int nrg = (int)(N / 16);
  const uint8_t* b_src[C::B_CP];
  const uint8_t* bs_src[C::B_CP];
#pragma unroll
  for (int jj = 0; jj < C::B_CP; ++jj) {
    int rg = it.n0 / 16 + wave * C::B_CP + jj;
    rg = rg < nrg ? rg : nrg - 1;  // partial weight block: repeat the last group (not stored)
    b_src[jj] = ecodes + codes_tile_offset(rg, 0, K) + lane * 16;
    bs_src[jj] = escales + scales_group_offset(rg, 0, K) + lane * 4;
  }

  auto issue = [&](int kt, uint8_t* slot) {
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;
      copy16(a_src[jj] + (int64_t)kt * (AFP4 ? 64 : 256), slot + C::A_OFF + j * 1024);
    }
    if constexpr (AFP4) copy4(as_src + (int64_t)kt * 4, slot + C::AS_OFF + (wave & 1) * 256);
#pragma unroll
    for (int jj = 0; jj < C::B_CP; ++jj) {
      const int q = wave * C::B_CP + jj;
      copy16(b_src[jj] + (int64_t)kt * 1024, slot + C::B_OFF + q * 1024);
      copy4(bs_src[jj] + (int64_t)(kt >> 2) * 256, slot + C::BS_OFF + q * 256);
    }
  };

  auto compute = [&](int kt, const uint8_t* slot) {
    const int g = lane >> 4;
    u32x4_t bw[4];
    uint32_t sbyte[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int q = wn * 4 + cb;
      bw[cb] = *reinterpret_cast<const u32x4_t*>(slot + C::B_OFF + q * 1024 + lane * 16);
      const uint32_t sd = *reinterpret_cast<const uint32_t*>(slot + C::BS_OFF + q * 256 + lane * 4);
      sbyte[cb] = (sd >> (8 * (kt & 3))) & 0xFFu;
    }
    if constexpr (!AFP4) {
      float sc[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) sc[cb] = e8m0_scale_operand(sbyte[cb]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        bf16x8_t av[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const int row = wm * 64 + rb * 16 + (lane & 15);
          const int phys = (4 * g + m) ^ (lane & 15);
          av[rb] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(slot + C::A_OFF + row * 256 + phys * 16));
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const bf16x8_t bv = unpack8_e2m1(bw[cb][m], sc[cb]);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rb], bv, acc[rb][cb], 0, 0, 0);
        }
      }
    } else {
      i32x8_t A[4], B[4];
      uint32_t as[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int row = wm * 64 + rb * 16 + (lane & 15);
        const int phys = g ^ ((row >> 2) & 3);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slot + C::A_OFF + row * 64 + phys * 16);
        A[rb] = (i32x8_t){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        as[rb] = slot[C::AS_OFF + row * 4 + g];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        B[cb] = (i32x8_t){(int)bw[cb][0], (int)bw[cb][1], (int)bw[cb][2], (int)bw[cb][3], 0, 0, 0, 0};
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rb], B[cb], acc[rb][cb], 4, 4, 0,
                                                                         (int)as[rb], 0, (int)sbyte[cb]);
    }
  };

  // ---- pipeline: stages 0 .. STAGES-2 in flight before the loop
  constexpr int S = C::STAGES;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue(s, lds + s * C::STAGE);
  for (int kt0 = 0; kt0 < KT; kt0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int kt = kt0 + j;
      if (kt >= KT) break;
      // this wave's copies of k-tile kt are done once only the later stages'
      // copies (at most S-2 of them) are outstanding
      const int later = KT - 1 - kt < S - 2 ? KT - 1 - kt : S - 2;
      if (later >= S - 2) wait_vm<(S - 2) * C::CP>();
      else if (later == 2) wait_vm<2 * C::CP>();
      else if (later == 1) wait_vm<C::CP>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + S - 1 < KT) issue(kt + S - 1, lds + ((j + S - 1) % S) * C::STAGE);
      compute(kt, lds + j * C::STAGE);
    }
  }
}

}  // namespace

// gate_up + clamped SwiGLU.  grid: 8 * ceil(item bound / 8) workgroups of 256.
template <bool AFP4>
__global__ __launch_bounds__(kThreads) void tile_gate_up_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  using C = Cfg<AFP4>;
  zero_duty(a);
  const int64_t H = a.K, I = a.N / 2;
  const int ntl = (int)((a.N + kNT - 1) / kNT);
  TileItem it;
  if (!tile_item(a, ntl, &it)) return;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  for (int r = threadIdx.x; r < kMT; r += blockDim.x)
    rowidx[r] = a.sorted[it.p0 + (r < it.rows ? r : 0)] / a.top_k;  // token of the tile row
  __syncthreads();
  f32x4_t acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  tile_mainloop<AFP4>(a, it, H, a.N, lds, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nrg = (int)(a.N / 16);
  // row groups (2f, 2f+1) of the wave hold gate and up of feature group
  // (n0/16 + 4 wn + 2f) / 2
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int rg = it.n0 / 16 + wn * 4 + 2 * f;
    if (rg >= nrg) break;
    const int64_t n = (int64_t)(rg / 2) * 16 + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = wm * 64 + rb * 16 + 4 * (lane >> 4) + r;
        if (row < it.rows) {
          const float v = swiglu_clamped(acc[rb][2 * f][r], acc[rb][2 * f + 1][r], a.clamp_limit);
          a.act[(it.p0 + row) * I + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
  }
}

// down + combine.
template <bool AFP4, bool ORDERED>
__global__ __launch_bounds__(kThreads) void tile_down_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  using C = Cfg<AFP4>;
  const int64_t I = a.K, H = a.N;
  const int ntl = (int)((a.N + kNT - 1) / kNT);
  TileItem it;
  if (!tile_item(a, ntl, &it)) return;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  for (int r = threadIdx.x; r < kMT; r += blockDim.x)
    rowidx[r] = (int32_t)(it.p0 + (r < it.rows ? r : 0));  // sorted position of the tile row
  __syncthreads();
  f32x4_t acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  tile_mainloop<AFP4>(a, it, I, H, lds, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + rb * 16 + 4 * (lane >> 4) + r;
      if (row >= it.rows) continue;
      const int64_t p = it.p0 + row;
      int64_t tok = 0;
      float wgt = 0.f;
      if constexpr (!ORDERED) {
        tok = a.pos_tok[p];
        wgt = a.pos_w[p];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int64_t n = (int64_t)(it.n0 / 16 + wn * 4 + cb) * 16 + (lane & 15);
        if (n >= H) break;
        if constexpr (ORDERED) {
          a.ybuf[p * H + n] = acc[rb][cb][r];
        } else {
          unsafeAtomicAdd(a.out32 + tok * H + n, wgt * acc[rb][cb][r]);
        }
      }
    }
}

// ------------------------------------------------------------------ launchers
namespace {
int64_t tile_grid(int64_t max_tiles, int64_t N) {
  const int64_t items = max_tiles * ((N + kNT - 1) / kNT);
  return 8 * ((items + 7) / 8);
}

// Launch with `lds` bytes of dynamic LDS; the first launch of each kernel
// raises its dynamic-LDS limit to that size.
template <typename Kernel>
hipError_t launch_lds(Kernel kernel, int64_t grid, size_t lds, const GemmArgs& a, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr = hipSuccess;
  std::call_once(once, [&] {
    attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
  });
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gate_up_tile(const GemmArgs& a, int64_t max_tiles, bool a4, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = tile_grid(max_tiles, a.N);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  return a4 ? launch_lds(tile_gate_up_kernel<true>, grid, Cfg<true>::LDS, a, s)
            : launch_lds(tile_gate_up_kernel<false>, grid, Cfg<false>::LDS, a, s);
}

hipError_t launch_down_tile(const GemmArgs& a, int64_t max_tiles, bool a4, bool ordered, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const int64_t grid = tile_grid(max_tiles, a.N);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (a4)
    return ordered ? launch_lds(tile_down_kernel<true, true>, grid, Cfg<true>::LDS, a, s)
                   : launch_lds(tile_down_kernel<true, false>, grid, Cfg<true>::LDS, a, s);
  return ordered ? launch_lds(tile_down_kernel<false, true>, grid, Cfg<false>::LDS, a, s)
                 : launch_lds(tile_down_kernel<false, false>, grid, Cfg<false>::LDS, a, s);
}

}  // namespace mxmoe
