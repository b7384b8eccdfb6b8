// Grouped GEMMs for token tiles of up to 128 rows (prefill and the A4 path):
// the MFMA work is the cost, so a workgroup owns a 128-token x NT-weight-row
// output tile of one expert (NT = 16 NRG, NRG = 32 by default) and streams K
// through LDS.
//
//   gate_up:  h = W13_e x_t, fused with the clamped SwiGLU -> act (bf16)
//   down:     y = W2_e a, fused with the weighted combine (fp32 atomics into
//             out32, or y rows for the ordered gather)
//
// Staging.  Each k-tile (128 of K) of the activation rows and of the NRG
// preshuffled weight row groups is copied straight from global memory into
// an LDS ring of STAGES slots by the gfx950 global->LDS load (a wave's
// instruction writes 64 x 16 bytes, lane i at slot + 16 i, from any per-lane
// address), so staging costs no registers.  The weight scale dwords (one per
// lane and row group covers a group of 4 k-tiles) go the same way into one
// LDS buffer, a group at a time, and each wave reads its row groups' dwords
// into registers at the group's first k-tile.  Every wave issues the same
// copies in the same order per k-tile; before using slot kt a wave waits
// until only the loads issued after slot kt's are outstanding, and one
// barrier per k-tile then publishes the slot to the whole workgroup and frees
// the slot the next copy writes (it was read in the previous iteration).
// No per-lane global load feeds a register inside the loop: a register that
// a pending load writes makes the compiler wait for it, and vmcnt counts in
// issue order, so such a wait would also wait for every copy issued before.
//
// Bank conflicts.  The activation rows are stored with their 16-byte chunks
// XOR-swizzled by the row (bf16: chunk c of row r at c ^ (r & 15); MXFP4:
// block c at c ^ ((r >> 2) & 3)), chosen through the per-lane source address
// of the copy, so the 16 lanes that read one MFMA operand hit 16 distinct
// 16-byte bank groups.  Weight codes are read lane-contiguously.
//
// MFMA layout: as in the other GEMMs (lane l: row l%16, MX block l/16 of the
// k-tile; K element 8m+e of the block feeds bf16 MFMA m).  Eight waves form a
// 2 x 4 grid (two per SIMD, so one wave's unpacking overlaps the other's
// MFMAs); wave (wm, wn) owns rows 64 wm.. and weight row groups WN wn..
// (WN = NRG/4).  A wider tile moves fewer activation bytes and takes fewer
// barriers per MFMA.
//
// Schedule.  Work items (row tile, NT-row weight block) are numbered
// tile-major; workgroup b runs on XCD b % 8 (round-robin dispatch), and each
// XCD takes a contiguous eighth of the items, so the workgroups resident on one
// XCD share activation tiles and weight blocks in that XCD's L2.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) int32_t const_i32;

constexpr int kMT = 128;  // token rows per tile
constexpr int kWaves = 8;  // 2 (rows) x 4 (weight row groups)
constexpr int kThreads = 64 * kWaves;

// Activation formats: 0 bf16, 1 MXFP4 (A4), 2 MXFP8 with E4M3 elements (A8).
constexpr int kActBf16 = 0, kActFp4 = 1, kActFp8 = 2;
// bytes of one activation row per k-tile (128 elements)
constexpr int act_row_bytes(int af) { return af == kActFp4 ? 64 : af == kActFp8 ? 128 : 256; }

template <int AF, int NRG_>
struct Cfg {
  static constexpr int NRG = NRG_;                              // weight row groups per tile
  static constexpr int NT = 16 * NRG;
  static constexpr int WN = NRG / 4;                            // row groups per wave
  static constexpr int A_BYTES = kMT * act_row_bytes(AF);       // activation k-tile
  static constexpr int AS_BYTES = AF != kActBf16 ? kMT * 4 : 0; // activation scale bytes
  static constexpr int B_BYTES = NRG * 1024;                    // weight codes
  static constexpr int A_OFF = 0, AS_OFF = A_BYTES, B_OFF = A_BYTES + AS_BYTES;
  static constexpr int STAGE = B_OFF + B_BYTES;
  static constexpr int ROWS_BYTES = kMT * 4;  // int32 [kMT]: A row index of each tile row
  static constexpr int WS_BYTES = NRG * 256;   // weight scale dwords of one 4-k-tile group
  static constexpr int STAGES_FIT = (160 * 1024 - ROWS_BYTES - WS_BYTES) / STAGE;
  static constexpr int STAGES = STAGES_FIT > 4 ? 4 : STAGES_FIT;
  static constexpr int A_CP = A_BYTES / 1024 / kWaves;  // copies per wave per k-tile
  static constexpr int AS_CP = AF != kActBf16 ? 1 : 0;  // 2 copies, made by even and odd waves alike
  static constexpr int B_CP = NRG / kWaves;
  static constexpr int CP = A_CP + AS_CP + B_CP;

  static constexpr int WS_OFF = STAGES * STAGE;
  static constexpr int ROWS_OFF = WS_OFF + WS_BYTES;
  static constexpr int LDS = ROWS_OFF + ROWS_BYTES;
  static_assert(STAGES >= 2 && LDS <= 160 * 1024, "LDS budget");
  static_assert(WN % 4 == 0 && NRG % kWaves == 0, "tile shape");
  static constexpr int WSCP = NRG / kWaves;             // weight scale copies per wave per group
  static constexpr int MAXWAIT = (STAGES - 2) * (CP + WSCP);
  static_assert(MAXWAIT < 64, "vmcnt range");
};

// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 encoding:
// vmcnt[3:0] bits 3:0, expcnt bits 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// wait_vm<n>() for a wave-uniform n in [0, MAX] (larger n: wait for all)
template <int MAX, int N = 0>
__device__ __forceinline__ void wait_vm_dyn(int n) {
  if constexpr (N > MAX) {
    wait_vm<0>();
  } else {
    if (n == N) {
      wait_vm<N>();
      return;
    }
    wait_vm_dyn<MAX, N + 1>(n);
  }
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
__device__ __forceinline__ bool tile_item(const GemmArgs& a, int ntl, int nt, TileItem* it) {
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
  it->n0 = (item - t * ntl) * nt;
  return true;
}

__device__ __forceinline__ void zero_duty(const GemmArgs& a) {
  if (!a.zero_buf) return;
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = tid; i < a.zero_n / 4; i += nthreads) reinterpret_cast<f32x4_t*>(a.zero_buf)[i] = z;
}

// The k-loop: acc[rb][cb] += A(rows 64 wm + 16 rb ..) * W(row group WN wn + cb)^T
// over all of K.  rowidx (LDS): the A-matrix row of each tile row.
template <int AF, int NRG>
__device__ __forceinline__ void tile_mainloop(const GemmArgs& a, const TileItem& it, int64_t K, int64_t N,
                                              uint8_t* lds, f32x4_t (&acc)[4][NRG / 4]) {
  using C = Cfg<AF, NRG>;
  constexpr int WN = C::WN;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int KT = (int)(K / kTileK);
  const int32_t* rowidx = reinterpret_cast<const int32_t*>(lds + C::ROWS_OFF);

  // ---- per-lane copy sources (k-tile 0); k-tile kt adds kt * stride
  const uint8_t* a_src[C::A_CP];
  const uint8_t* as_src = nullptr;
  if constexpr (AF == kActBf16) {
    const int64_t rb = K * 2;  // bytes per activation row
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;  // rows 4j .. 4j+3
      const int row = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      a_src[jj] = reinterpret_cast<const uint8_t*>(a.a_bf16) + (int64_t)rowidx[row] * rb + c * 16;
    }
  } else if constexpr (AF == kActFp8) {
    // 128-byte rows: copy j fills rows 8j .. 8j+7, lane i row 8j + i/8 at chunk
    // i % 8, which holds the row's logical chunk (i % 8) ^ ((row >> 1) & 7)
    const int64_t rb = K;
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;
      const int row = 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      a_src[jj] = a.a_codes + (int64_t)rowidx[row] * rb + c * 16;
    }
    const int row = 64 * (wave & 1) + lane;
    as_src = a.a_scales + (int64_t)rowidx[row] * (K / 32);
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
    as_src = a.a_scales + (int64_t)rowidx[row] * (K / 32);
  }
  const int64_t cpe = codes_per_expert(N, K), spe = scales_per_expert(N, K);
  const uint8_t* ecodes = a.w_codes + (int64_t)it.e * cpe;
  const uint8_t* escales = a.w_scales + (int64_t)it.e * spe;
  const int nrg = (int)(N / 16);
  auto clamp_rg = [&](int rg) { return rg < nrg ? rg : nrg - 1; };  // partial block: repeat (not stored)
  // weight copies and scale loads: one per-lane pointer each plus wave-uniform
  // row-group offsets
  const uint8_t* b_lane = ecodes + lane * 16;
  const uint8_t* s_lane = escales + lane * 4;
  auto b_off = [&](int jj) -> int64_t {
    return codes_tile_offset(clamp_rg(it.n0 / 16 + wave * C::B_CP + jj), 0, K);
  };
  // scale dwords of 4-k-tile group q (clamped to the last group): wave w
  // copies row groups w WSCP .. w WSCP + WSCP - 1 of the tile, 256 bytes each
  const int NQ = (KT + 3) / 4;
  auto issue_scales = [&](int q) {
    q = q < NQ ? q : NQ - 1;
#pragma unroll
    for (int i = 0; i < C::WSCP; ++i) {
      const int rgl = wave * C::WSCP + i;
      copy4(s_lane + scales_group_offset(clamp_rg(it.n0 / 16 + rgl), q, K), lds + C::WS_OFF + rgl * 256);
    }
  };

  auto issue = [&](int kt, uint8_t* slot) {
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = wave * C::A_CP + jj;
      copy16(a_src[jj] + (int64_t)kt * act_row_bytes(AF), slot + C::A_OFF + j * 1024);
    }
    if constexpr (AF != kActBf16) copy4(as_src + (int64_t)kt * 4, slot + C::AS_OFF + (wave & 1) * 256);
#pragma unroll
    for (int jj = 0; jj < C::B_CP; ++jj) {
      const int q = wave * C::B_CP + jj;
      copy16(b_lane + b_off(jj) + (int64_t)kt * 1024, slot + C::B_OFF + q * 1024);
    }
  };

  // this wave's scale dwords of the current 4-k-tile group (row group
  // WN wn + cb), read from LDS at the group's first k-tile
  uint32_t scur[WN];

  auto compute = [&](int kt, const uint8_t* slot) {
    const int g = lane >> 4;
    u32x4_t bw[WN];
    uint32_t sbyte[WN];
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) {
      bw[cb] = *reinterpret_cast<const u32x4_t*>(slot + C::B_OFF + (wn * WN + cb) * 1024 + lane * 16);
      sbyte[cb] = (scur[cb] >> (8 * (kt & 3))) & 0xFFu;
    }
    if constexpr (AF == kActBf16) {
      float sc[WN];
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) sc[cb] = e8m0_scale_operand(sbyte[cb]);
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
        for (int cb = 0; cb < WN; ++cb) {
          const bf16x8_t bv = unpack8_e2m1(bw[cb][m], sc[cb]);
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rb], bv, acc[rb][cb], 0, 0, 0);
        }
      }
    } else {
      i32x8_t A[4];
      uint32_t as[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int row = wm * 64 + rb * 16 + (lane & 15);
        if constexpr (AF == kActFp8) {
          // 8-bit A elements: lane group g supplies K 16 g .. 16 g + 15 and
          // 64 + 16 g .. 64 + 16 g + 15 (logical chunks g and 4 + g), with the
          // scale of block g as for E2M1 (the MFMA reads block b's scale from
          // lane group b)
          const int sw = (row >> 1) & 7;
          const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(slot + C::A_OFF + row * 128 + (g ^ sw) * 16);
          const u32x4_t v1 =
              *reinterpret_cast<const u32x4_t*>(slot + C::A_OFF + row * 128 + ((4 + g) ^ sw) * 16);
          A[rb] = (i32x8_t){(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                            (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
        } else {
          const int phys = g ^ ((row >> 2) & 3);
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slot + C::A_OFF + row * 64 + phys * 16);
          A[rb] = (i32x8_t){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        }
        as[rb] = slot[C::AS_OFF + row * 4 + g];
      }
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) {
        const i32x8_t B = {(int)bw[cb][0], (int)bw[cb][1], (int)bw[cb][2], (int)bw[cb][3], 0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              A[rb], B, acc[rb][cb], AF == kActFp8 ? 0 : 4, 4, 0, (int)as[rb], 0, (int)sbyte[cb]);
      }
    }
  };

  // ---- pipeline: stages 0 .. STAGES-2 in flight before the loop.  Step kt:
  // wait for slot kt's copies, barrier, scale loads (steps 0 and 1 of a
  // group), the copies of k-tile kt + S - 1, compute k-tile kt.  Every step
  // issues its copies, past K those of the last k-tile again (into the slot
  // read in the previous step, free after the barrier): with the same
  // instructions on every path the compiler's own waits for the scale
  // registers count exactly and never fall back to waiting for everything.
  constexpr int S = C::STAGES;
  issue_scales(0);
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s < KT ? s : KT - 1, lds + s * C::STAGE);
  // vector-memory ops a step issues: the next group's scale copies (second
  // k-tile of a group: every wave has read the buffer at the first, before
  // this step's barrier), then the stage copies
  auto ops_of_step = [&](int st) -> int { return ((st & 3) == 1 ? C::WSCP : 0) + C::CP; };
  for (int kt0 = 0; kt0 < KT; kt0 += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kt = kt0 + j;
      if (kt >= KT) break;
      // ops issued after slot kt's copies (vmcnt counts in issue order): the
      // prologue's later stages (k-tile kt < S - 1) or the ops of the steps
      // between the one that issued slot kt and this one
      int after = 0;
      if (kt < S - 1) {
        after = (S - 2 - kt) * C::CP;
#pragma unroll
        for (int st = 0; st < S - 2; ++st)
          if (st < kt) after += ops_of_step(st);
      } else {
#pragma unroll
        for (int d = 1; d <= S - 2; ++d) after += ops_of_step(kt - d);
      }
      wait_vm_dyn<C::MAXWAIT>(after);
      __builtin_amdgcn_s_barrier();
      // a new 4-k-tile group starts: its scale dwords were copied at the
      // previous group's second k-tile (before the stage copies waited for
      // above), or in the prologue
      if (j == 0) {
#pragma unroll
        for (int cb = 0; cb < WN; ++cb)
          scur[cb] = *reinterpret_cast<const uint32_t*>(lds + C::WS_OFF + (wn * WN + cb) * 256 + lane * 4);
      }
      if (j == 1) issue_scales((kt >> 2) + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(kt + S - 1 < KT ? kt + S - 1 : KT - 1, lds + ((kt + S - 1) % S) * C::STAGE);
      compute(kt, lds + (kt % S) * C::STAGE);
    }
  }
}

// Tile width: NRG weight row groups (MXFP4_MOE_TILE_NRG, tests and benchmarks
// only, selects 16; default 32).
int tile_nrg() {
  static const int v = [] {
    const char* e = getenv("MXFP4_MOE_TILE_NRG");
    return e && !strcmp(e, "16") ? 16 : 32;
  }();
  return v;
}

}  // namespace

// gate_up + clamped SwiGLU.  grid: 8 * ceil(item bound / 8) workgroups of 512.
template <int AF, int NRG>
__global__ __launch_bounds__(kThreads) void tile_gate_up_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  using C = Cfg<AF, NRG>;
  constexpr int WN = C::WN;
  zero_duty(a);
  const int64_t H = a.K, I = a.N / 2;
  const int ntl = (int)((a.N + C::NT - 1) / C::NT);
  TileItem it;
  if (!tile_item(a, ntl, C::NT, &it)) return;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  for (int r = threadIdx.x; r < kMT; r += blockDim.x)
    rowidx[r] = a.sorted[it.p0 + (r < it.rows ? r : 0)] / a.top_k;  // token of the tile row
  __syncthreads();
  f32x4_t acc[4][WN];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  tile_mainloop<AF, NRG>(a, it, H, a.N, lds, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nrg = (int)(a.N / 16);
  // row groups (2f, 2f+1) of the wave hold gate and up of feature group
  // (n0/16 + WN wn + 2f) / 2
#pragma unroll
  for (int f = 0; f < WN / 2; ++f) {
    const int rg = it.n0 / 16 + wn * WN + 2 * f;
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
template <int AF, bool ORDERED, int NRG>
__global__ __launch_bounds__(kThreads) void tile_down_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  using C = Cfg<AF, NRG>;
  constexpr int WN = C::WN;
  const int64_t I = a.K, H = a.N;
  const int ntl = (int)((a.N + C::NT - 1) / C::NT);
  TileItem it;
  if (!tile_item(a, ntl, C::NT, &it)) return;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  for (int r = threadIdx.x; r < kMT; r += blockDim.x)
    rowidx[r] = (int32_t)(it.p0 + (r < it.rows ? r : 0));  // sorted position of the tile row
  __syncthreads();
  f32x4_t acc[4][WN];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  tile_mainloop<AF, NRG>(a, it, I, H, lds, acc);

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
      for (int cb = 0; cb < WN; ++cb) {
        const int64_t n = (int64_t)(it.n0 / 16 + wn * WN + cb) * 16 + (lane & 15);
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
int64_t tile_grid(int64_t max_tiles, int64_t N, int nt) {
  const int64_t items = max_tiles * ((N + nt - 1) / nt);
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
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int AF, int NRG>
hipError_t gate_up_af(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t grid = tile_grid(max_tiles, a.N, 16 * NRG);
  return launch_lds(tile_gate_up_kernel<AF, NRG>, grid, Cfg<AF, NRG>::LDS, a, s);
}
template <int AF, int NRG>
hipError_t down_af(const GemmArgs& a, int64_t max_tiles, bool ordered, hipStream_t s) {
  const int64_t grid = tile_grid(max_tiles, a.N, 16 * NRG);
  return ordered ? launch_lds(tile_down_kernel<AF, true, NRG>, grid, Cfg<AF, NRG>::LDS, a, s)
                 : launch_lds(tile_down_kernel<AF, false, NRG>, grid, Cfg<AF, NRG>::LDS, a, s);
}

template <int NRG>
hipError_t gate_up_nrg(const GemmArgs& a, int64_t max_tiles, int af, hipStream_t s) {
  if (af == kActFp8) return gate_up_af<kActFp8, NRG>(a, max_tiles, s);
  return af == kActFp4 ? gate_up_af<kActFp4, NRG>(a, max_tiles, s) : gate_up_af<kActBf16, NRG>(a, max_tiles, s);
}

template <int NRG>
hipError_t down_nrg(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, hipStream_t s) {
  if (af == kActFp8) return down_af<kActFp8, NRG>(a, max_tiles, ordered, s);
  return af == kActFp4 ? down_af<kActFp4, NRG>(a, max_tiles, ordered, s)
                       : down_af<kActBf16, NRG>(a, max_tiles, ordered, s);
}
}  // namespace

hipError_t launch_gate_up_tile(const GemmArgs& a, int64_t max_tiles, int af, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  return tile_nrg() == 16 ? gate_up_nrg<16>(a, max_tiles, af, s) : gate_up_nrg<32>(a, max_tiles, af, s);
}

hipError_t launch_down_tile(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  return tile_nrg() == 16 ? down_nrg<16>(a, max_tiles, af, ordered, s)
                          : down_nrg<32>(a, max_tiles, af, ordered, s);
}

}  // namespace mxmoe
