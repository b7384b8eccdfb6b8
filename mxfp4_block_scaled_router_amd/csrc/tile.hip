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
// XOR-swizzled by the row, chosen through the per-lane source address of the
// copy: bf16 (256-byte rows) chunk c of row r at c ^ bf16_swz(r), MXFP4
// (64-byte rows) block c at c ^ ((r >> 1) & 3), MXFP8 (128-byte rows) chunk c
// at c ^ ((r >> 1) & 7).  These are the patterns a probe of the operand reads
// (ds_read_b128, lane l reading row l % 16) measured free of LDS bank
// conflicts on gfx950 (an XOR by r & 15 for bf16, or by (r >> 2) & 3 for
// MXFP4, measures twice the LDS cycles).  Weight codes are read
// lane-contiguously.
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
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// bf16 activation rows: the physical 16-byte chunk of logical chunk c of row
// r is c ^ bf16_swz(r & 15) (for each row a permutation of its 16 chunks)
__device__ __forceinline__ int bf16_swz(int r) { return ((r & 3) << 2) ^ ((r >> 2) & 3); }

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr size_t kTileLdsMax = 160 * 1024;

// Activation formats: 0 bf16, 1 MXFP4 (A4), 2 MXFP8 with E4M3 elements (A8).
constexpr int kActBf16 = 0, kActFp4 = 1, kActFp8 = 2;
// bytes of one activation row per k-tile (128 elements)
constexpr int act_row_bytes(int af) { return af == kActFp4 ? 64 : af == kActFp8 ? 128 : 256; }

// Tile shape.  The eight waves form a WMW x (8 / WMW) grid; a wave owns RB
// 16-row blocks of the token tile and WN weight row groups.  IL: the row
// blocks of wave wm are wm, wm + WMW, wm + 2 WMW, ... (interleaved, so a
// partly filled tile spreads its rows over all waves); else the contiguous
// RB wm .. RB wm + RB - 1.
//   128-row tiles:  WMW 2, RB 4, WN NRG / 4 (128 x 512 with NRG 32)
//   320-row tiles:  WMW 4, RB 5, WN 4, interleaved (320 x 128): with MX
//                   activations one tile holds all rows of an expert of the
//                   A4 prefill workload, so its weights stream once (a wider
//                   weight block needs more accumulator registers than two
//                   waves per SIMD leave).
template <int AF, int WMW_, int RB_, int WN_, bool IL_, int SA_, int SB_, bool PF_ = false, bool RS_ = false>
struct Cfg {
  // RS (PF only): all activation scale bytes of the tile's rows are copied
  // into LDS once per tile ([MT][K/32], whole rows: full cache lines) instead
  // of a 4-byte-per-row gather per k-tile, which touches one cache line per
  // row for 4 useful bytes and dominated the copy path
  static constexpr bool RS = RS_;
  // PF: MX activations only, SA == SB: a step waits one k-tile ahead and
  // reads the next k-tile's operands from LDS into a second register set
  // while its MFMAs run on the current one (tile_mainloop_pf)
  static constexpr bool PF = PF_;
  static constexpr bool DW = false;
  static constexpr int WMW = WMW_, WNW = kWaves / WMW_, RB = RB_, WN = WN_;
  static constexpr bool IL = IL_;
  static constexpr int MT = 16 * RB * WMW;                      // token rows per tile
  static constexpr int NRG = WN * WNW;                          // weight row groups per tile
  static constexpr int NT = 16 * NRG;
  static constexpr int ARB = act_row_bytes(AF);
  static constexpr int A_BYTES = MT * ARB;                      // activation k-tile
  static constexpr int AS_BYTES = AF != kActBf16 && !RS ? MT * 4 : 0;  // activation scale bytes
  static constexpr int A_STAGE = A_BYTES + AS_BYTES;
  static constexpr int B_BYTES = NRG * 1024;                    // weight codes of one k-tile
  // two rings: SA activation slots (their copies hit L2: the rows are shared
  // by the tile's weight blocks) and SB weight slots (a stream from HBM,
  // which needs more bytes in flight)
  static constexpr int SA = SA_, SB = SB_;
  static constexpr int A_RING = 0, B_RING = SA * A_STAGE;
  static constexpr int ROWS_BYTES = MT * 4;  // int32 [MT]: A row index of each tile row
  static constexpr int WS_BYTES = 2 * NRG * 256;  // weight scale dwords of two 4-k-tile groups
  // activation copies of 1 KiB (a wave instruction: 64 lanes x 16 bytes) per
  // k-tile, spread over the waves; a wave whose share is short repeats the
  // last copy (same bytes to the same place), so every wave issues A_CP
  static constexpr int A_COPIES = A_BYTES / 1024;
  static constexpr int A_CP = (A_COPIES + kWaves - 1) / kWaves;
  // activation scale copies of 256 bytes (64 rows): one per wave, wave w
  // taking chunk w % AS_CHUNKS
  static constexpr int AS_CHUNKS = MT / 64;
  static constexpr int AS_CP = AF != kActBf16 && !RS ? 1 : 0;
  static constexpr int B_CP = NRG / kWaves;
  static constexpr int OPS_A = A_CP + AS_CP;  // vector-memory ops of one k-tile's activation copies

  static constexpr int WS_OFF = B_RING + SB * B_BYTES;
  static constexpr int ROWS_OFF = WS_OFF + WS_BYTES;
  static constexpr int RS_OFF = ROWS_OFF + ROWS_BYTES;  // RS: [MT][K/32] activation scale bytes
  static constexpr int LDS = RS_OFF;                     // without the row scales
  static constexpr int STAGE_MAX = WS_OFF;  // LDS free for the epilogue (the rings)
  static constexpr size_t lds_bytes(int64_t K) { return (size_t)LDS + (RS ? (size_t)MT * (size_t)(K / 32) : 0); }
  static_assert(SA >= 2 && SA <= 5 && SB >= SA && LDS <= 160 * 1024, "LDS budget");
  static_assert(!RS || PF, "row scales need the PF pipeline");
  static_assert(WN % 2 == 0 && NRG % kWaves == 0 && kWaves % WMW == 0, "tile shape");
  static_assert(A_BYTES % 1024 == 0 && MT % 64 == 0 && AS_CHUNKS <= kWaves, "copy shape");
  static constexpr int WSCP = NRG / kWaves;             // weight scale copies per wave per group
  // bound on the ops a wait lets stay outstanding (see tile_mainloop)
  static constexpr int MAXWAIT = (SB - 2) * B_CP + (SA - 1) * (WSCP + B_CP + 2 * OPS_A);
  static_assert(MAXWAIT < 64, "vmcnt range");
  // vector-memory ops of pipeline step st (the next group's scale copies at
  // a group's first k-tile, then the weight and activation copies)
  static constexpr int ops_of_step(int st) { return ((st & 3) == 0 ? WSCP : 0) + B_CP + OPS_A; }
  // ops issued after the activation copies of the k-tile a steady-state step
  // at position j of its group waits for: those of the SA - 2 steps before
  static constexpr int steady_after(int j) {
    int n = 0;
    for (int d = 1; d <= SA - 2; ++d) n += ops_of_step(j - d + 4);
    return n;
  }
  // PF pipeline: ops issued after the activation copies of k-tile kt + 1,
  // waited for at step kt (see tile_mainloop_pf)
  static constexpr int pf_after(int kt) {
    int n = 0;
    if (kt + 1 <= SA - 1) {
      n = (SA - 2 - kt) * (B_CP + OPS_A);
      for (int st = 0; st < kt; ++st) n += ops_of_step(st);
    } else {
      for (int d = 1; d <= SA - 2; ++d) n += ops_of_step(kt - d + 4);
    }
    return n;
  }
  static constexpr int pf_max_after() {
    int m = (SA - 1) * (B_CP + OPS_A);
    for (int kt = 0; kt < 8; ++kt) m = pf_after(kt) > m ? pf_after(kt) : m;
    return m;
  }
  static_assert(!PF || (AF != kActBf16 && SA == SB && pf_max_after() < 64), "PF pipeline");
  // 16-row block of the tile held as the wave's rb-th
  __device__ static constexpr int rowblock(int wm, int rb) { return IL ? wm + WMW * rb : RB * wm + rb; }
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
// weight streams are read once per step: non-temporal (cache policy nt), so
// they do not displace the activation rows that a tile's weight blocks share
// in L2
constexpr int kCpolNT = 2;
__device__ __forceinline__ void copy16_nt(const void* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, kCpolNT);
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

// The k-loop: acc[rb][cb] += A(row block C::rowblock(wm, rb)) * W(row group
// WN wn + cb)^T over all of K.  rowidx (LDS): the A-matrix row of each tile
// row.  Row blocks wholly past the tile's rows skip their MFMAs.
template <int AF, typename C>
__device__ __forceinline__ void tile_mainloop(const GemmArgs& a, const TileItem& it, int64_t K, int64_t N,
                                              uint8_t* lds, f32x4_t (&acc)[C::RB][C::WN]) {
  constexpr int WN = C::WN, RB = C::RB;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % C::WMW, wn = wave / C::WMW;
  const int KT = (int)(K / kTileK);
  const int32_t* rowidx = reinterpret_cast<const int32_t*>(lds + C::ROWS_OFF);

  // ---- per-lane copy sources (k-tile 0); k-tile kt adds kt * stride
  const uint8_t* a_src[C::A_CP];
  const uint8_t* as_src = nullptr;
  if constexpr (AF == kActBf16) {
    const int64_t rb = K * 2;  // bytes per activation row
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);  // rows 4j .. 4j+3
      const int row = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ bf16_swz(row & 15);
      a_src[jj] = reinterpret_cast<const uint8_t*>(a.a_bf16) + (int64_t)rowidx[row] * rb + c * 16;
    }
  } else if constexpr (AF == kActFp8) {
    // 128-byte rows: copy j fills rows 8j .. 8j+7, lane i row 8j + i/8 at chunk
    // i % 8, which holds the row's logical chunk (i % 8) ^ ((row >> 1) & 7)
    const int64_t rb = K;
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);
      const int row = 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      a_src[jj] = a.a_codes + (int64_t)rowidx[row] * rb + c * 16;
    }
    const int row = 64 * (wave % C::AS_CHUNKS) + lane;
    as_src = a.a_scales + (int64_t)rowidx[row] * (K / 32);
  } else {
    const int64_t rb = K / 2;
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);  // rows 16j .. 16j+15
      const int row = 16 * j + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 1) & 3);
      a_src[jj] = a.a_codes + (int64_t)rowidx[row] * rb + c * 16;
    }
    const int row = 64 * (wave % C::AS_CHUNKS) + lane;
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
      copy4(s_lane + scales_group_offset(clamp_rg(it.n0 / 16 + rgl), q, K),
            lds + C::WS_OFF + ((q & 1) * C::NRG + rgl) * 256);
    }
  };

  // activation copies of k-tile kt into slot (A rows, then their scale bytes)
  auto issue_a = [&](int kt, uint8_t* slot) {
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);
      copy16(a_src[jj] + (int64_t)kt * act_row_bytes(AF), slot + j * 1024);
    }
    if constexpr (AF != kActBf16)
      copy4(as_src + (int64_t)kt * 4, slot + C::A_BYTES + (wave % C::AS_CHUNKS) * 256);
  };
  // weight-code copies of k-tile kt into slot
  auto issue_b = [&](int kt, uint8_t* slot) {
#pragma unroll
    for (int jj = 0; jj < C::B_CP; ++jj) {
      const int q = wave * C::B_CP + jj;
      copy16(b_lane + b_off(jj) + (int64_t)kt * 1024, slot + q * 1024);
    }
  };

  // this wave's scale dwords of the current 4-k-tile group (row group
  // WN wn + cb), read from LDS at the group's first k-tile
  uint32_t scur[WN];

  auto compute = [&](int kt, const uint8_t* aslot, const uint8_t* bslot) {
    const int g = lane >> 4;
    u32x4_t bw[WN];
    uint32_t sbyte[WN];
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) {
      bw[cb] = *reinterpret_cast<const u32x4_t*>(bslot + (wn * WN + cb) * 1024 + lane * 16);
      sbyte[cb] = (scur[cb] >> (8 * (kt & 3))) & 0xFFu;
    }
    if constexpr (AF == kActBf16) {
      float sc[WN];
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) sc[cb] = e8m0_scale_operand(sbyte[cb]);
      // Sub-step m (K 32 m .. 32 m + 31).  Each weight row group's E2M1 codes
      // are unpacked while the previous row group's MFMAs issue (one unpack
      // between two MFMAs, into the other of two operand registers), and the
      // A operands of sub-step m + 1 are read after the first row group's
      // MFMAs, so their LDS latency hides behind the rest of the sub-step.
      // The scheduling-group barriers fix that interleave; 12 LDS reads at
      // most are in flight, within lgkmcnt's range.
      bf16x8_t av[2][RB];
      auto read_a = [&](int m, bf16x8_t (&dst)[RB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int row = C::rowblock(wm, rb) * 16 + (lane & 15);
          const int phys = (4 * g + m) ^ bf16_swz(lane & 15);
          dst[rb] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(aslot + row * 256 + phys * 16));
        }
      };
      read_a(0, av[0]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t bv[2];
        bv[0] = unpack8_e2m1(bw[0][m], sc[0]);
#pragma unroll
        for (int cb = 0; cb < WN; ++cb) {
          if (cb + 1 < WN) bv[(cb + 1) & 1] = unpack8_e2m1(bw[cb + 1][m], sc[cb + 1]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m & 1][rb], bv[cb & 1], acc[rb][cb], 0, 0, 0);
          if (cb == 0 && m < 3) read_a(m + 1, av[(m + 1) & 1]);
        }
        // schedule: the first row group's unpack, then MFMA / unpack pairs
        // (the A reads of the next sub-step after the first row group), then
        // the last row group's MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
#pragma unroll
        for (int i = 0; i < 4 * (WN - 1); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // VALU
          if (i == RB - 1 && m < 3) __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      i32x8_t A[RB];
      uint32_t as[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = C::rowblock(wm, rb) * 16 + (lane & 15);
        if constexpr (AF == kActFp8) {
          // 8-bit A elements: lane group g supplies K 16 g .. 16 g + 15 and
          // 64 + 16 g .. 64 + 16 g + 15 (logical chunks g and 4 + g), with the
          // scale of block g as for E2M1 (the MFMA reads block b's scale from
          // lane group b)
          const int sw = (row >> 1) & 7;
          const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(aslot + row * 128 + (g ^ sw) * 16);
          const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(aslot + row * 128 + ((4 + g) ^ sw) * 16);
          A[rb] = (i32x8_t){(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                            (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
        } else {
          const int phys = g ^ ((row >> 1) & 3);
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(aslot + row * 64 + phys * 16);
          A[rb] = (i32x8_t){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        }
        as[rb] = aslot[C::A_BYTES + row * 4 + g];
      }
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) {
        const i32x8_t B = {(int)bw[cb][0], (int)bw[cb][1], (int)bw[cb][2], (int)bw[cb][3], 0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                A[rb], B, acc[rb][cb], AF == kActFp8 ? 0 : 4, 4, 0, (int)as[rb], 0, (int)sbyte[cb]);
      }
    }
  };

  // ---- pipeline.  Prologue: the first scale group, then for p = 0, 1, ...
  // the weight copies of k-tile p (p <= SB - 2) and the activation copies of
  // k-tile p (p <= SA - 2).  Step kt: wait until k-tile kt's activation
  // copies -- issued after its weight copies -- have landed, barrier, scale
  // dwords (steps 0 and 1 of a group), the weight copies of k-tile kt + SB - 1
  // and the activation copies of k-tile kt + SA - 1, compute k-tile kt.
  // Every step issues its copies, past K those of the last k-tile again (into
  // the slot read in the previous step, free after the barrier): with the
  // same instructions on every path the compiler's own waits for the scale
  // registers count exactly and never fall back to waiting for everything.
  constexpr int SA = C::SA, SB = C::SB;
  constexpr int PM = SB - 2;  // last prologue index (SB >= SA)
  auto aslot = [&](int kt) { return lds + C::A_RING + (kt % SA) * C::A_STAGE; };
  auto bslot = [&](int kt) { return lds + C::B_RING + (kt % SB) * C::B_BYTES; };
  issue_scales(0);
#pragma unroll
  for (int p = 0; p <= PM; ++p) {
    issue_b(p < KT ? p : KT - 1, bslot(p));
    if (p <= SA - 2) issue_a(p < KT ? p : KT - 1, aslot(p));
  }
  // vector-memory ops a step issues: the next group's scale copies (first
  // k-tile of a group), then the weight and activation copies
  auto ops_of_step = [&](int st) -> int { return C::ops_of_step(st); };
  // one step; `after` = the vector-memory ops issued after k-tile kt's
  // activation copies (vmcnt counts in issue order)
  auto step = [&](int kt, int j, auto wait) {
    wait();
    __builtin_amdgcn_s_barrier();
    // a new 4-k-tile group starts: its scale dwords were copied at the
    // previous group's first k-tile (before, or with SA = 5 in the same step
    // just before, the activation copies waited for), or in the prologue
    if (j == 0) {
#pragma unroll
      for (int cb = 0; cb < WN; ++cb)
        scur[cb] = *reinterpret_cast<const uint32_t*>(
            lds + C::WS_OFF + (((kt >> 2) & 1) * C::NRG + wn * WN + cb) * 256 + lane * 4);
      // the next group's scale dwords, into the other buffer (last read at
      // the previous group's first k-tile, before this step's barrier)
      issue_scales((kt >> 2) + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_b(kt + SB - 1 < KT ? kt + SB - 1 : KT - 1, bslot(kt + SB - 1));
    issue_a(kt + SA - 1 < KT ? kt + SA - 1 : KT - 1, aslot(kt + SA - 1));
    compute(kt, aslot(kt), bslot(kt));
  };
  // waits: in the first group, the rest of the prologue and the steps before
  // this one (k-tile kt <= SA - 2, issued in the prologue), or the steps
  // between the one that issued its copies and this one; in later groups
  // (every k-tile issued in a step, SA <= 5) a constant for each position
  auto first_after = [&](int j) -> int {
    int after = 0;
    if (j <= SA - 2) {
#pragma unroll
      for (int p = 1; p <= PM; ++p)
        if (p > j) after += C::B_CP + (p <= SA - 2 ? C::OPS_A : 0);
#pragma unroll
      for (int st = 0; st < SA - 2; ++st)
        if (st < j) after += ops_of_step(st);
    } else {
#pragma unroll
      for (int d = 1; d <= SA - 2; ++d) after += ops_of_step(j - d);
    }
    return after;
  };
  for (int kt0 = 0; kt0 < KT; kt0 += 4) {
    const bool first = kt0 == 0;
    step(kt0, 0, [&] { if (first) wait_vm_dyn<C::MAXWAIT>(first_after(0)); else wait_vm<C::steady_after(0)>(); });
    if (kt0 + 1 < KT)
      step(kt0 + 1, 1, [&] { if (first) wait_vm_dyn<C::MAXWAIT>(first_after(1)); else wait_vm<C::steady_after(1)>(); });
    if (kt0 + 2 < KT)
      step(kt0 + 2, 2, [&] { if (first) wait_vm_dyn<C::MAXWAIT>(first_after(2)); else wait_vm<C::steady_after(2)>(); });
    if (kt0 + 3 < KT)
      step(kt0 + 3, 3, [&] { if (first) wait_vm_dyn<C::MAXWAIT>(first_after(3)); else wait_vm<C::steady_after(3)>(); });
  }
}

// The k-loop of the PF configurations (MX activations): step kt waits for
// k-tile kt + 1's copies, so that after the barrier the wave reads k-tile
// kt + 1's operands from LDS into one register set while its MFMAs consume
// k-tile kt's, read in the step before, from the other.  A slot's operands
// are in registers one step before the k-tile is used, so step kt refills
// slot kt with k-tile kt + S: S - 1 k-tiles stay in flight.  Before the
// barrier each wave waits for its own LDS reads (those of the slot the next
// copies overwrite have completed before any wave issues them).
template <int AF, typename C>
__device__ __forceinline__ void tile_mainloop_pf(const GemmArgs& a, const TileItem& it, int64_t K, int64_t N,
                                                 uint8_t* lds, f32x4_t (&acc)[C::RB][C::WN]) {
  constexpr int WN = C::WN, RB = C::RB, S = C::SA;
  const int lane = lane_id();
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % C::WMW, wn = wave / C::WMW;
  const int KT = (int)(K / kTileK);
  const int32_t* rowidx = reinterpret_cast<const int32_t*>(lds + C::ROWS_OFF);

  // ---- per-lane copy sources (k-tile 0); k-tile kt adds kt * row bytes
  const uint8_t* a_src[C::A_CP];
  const uint8_t* as_src;
  {
    const int64_t rb = K * act_row_bytes(AF) / kTileK;  // code bytes per activation row
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);
      int row, c;
      if constexpr (AF == kActFp8) {
        // copy j fills rows 8j .. 8j+7, lane i row 8j + i/8 at chunk i % 8,
        // which holds the row's logical chunk (i % 8) ^ ((row >> 1) & 7)
        row = 8 * j + (lane >> 3);
        c = (lane & 7) ^ ((row >> 1) & 7);
      } else {
        // copy j fills rows 16j .. 16j+15, lane i row 16j + i/4 at block i % 4,
        // which holds the row's logical block (i % 4) ^ ((row >> 1) & 3)
        row = 16 * j + (lane >> 2);
        c = (lane & 3) ^ ((row >> 1) & 3);
      }
      a_src[jj] = a.a_codes + (int64_t)rowidx[row] * rb + c * 16;
    }
    const int row = 64 * (wave % C::AS_CHUNKS) + lane;
    as_src = a.a_scales + (int64_t)rowidx[row] * (K / 32);
  }
  const int RSB = (int)(K / 32);  // activation scale bytes per row
  uint8_t* rs = lds + C::RS_OFF;
  // With rows of a multiple of 128 bytes the 16 rows of one MFMA operand
  // would fall into two LDS banks; their 16-byte chunks are then XOR-swizzled
  // by (row >> 1) & 7 (chosen through the copies' source addresses), which
  // puts the 16 rows' bytes of one k-tile into 16 distinct banks.
  const int rs_sw = RSB % 128 == 0 ? 7 : 0;
  if constexpr (C::RS) {
    // every scale byte of the tile's rows, row-major [MT][K/32]: a copy
    // instruction covers 1 KiB (or 256 bytes) of that array, whole rows apart
    // from its ends; issued before the prologue, so the first wait covers them
    if (RSB % 16 == 0) {
      const int n = C::MT * RSB / 1024;
      for (int i = wave; i < n; i += kWaves) {
        const int o = i * 1024 + lane * 16;
        const int row = o / RSB, chunk = (o % RSB) / 16;
        copy16(a.a_scales + (int64_t)rowidx[row] * RSB + (chunk ^ ((row >> 1) & rs_sw)) * 16, rs + i * 1024);
      }
    } else {
      const int n = C::MT * RSB / 256;
      for (int i = wave; i < n; i += kWaves) {
        const int o = i * 256 + lane * 4;
        copy4(a.a_scales + (int64_t)rowidx[o / RSB] * RSB + o % RSB, rs + i * 256);
      }
    }
  }
  const int64_t cpe = codes_per_expert(N, K), spe = scales_per_expert(N, K);
  const uint8_t* b_lane = a.w_codes + (int64_t)it.e * cpe + lane * 16;
  const uint8_t* s_lane = a.w_scales + (int64_t)it.e * spe + lane * 4;
  const int nrg = (int)(N / 16);
  auto clamp_rg = [&](int rg) { return rg < nrg ? rg : nrg - 1; };  // partial block: repeat (not stored)
  const int64_t b_off = codes_tile_offset(clamp_rg(it.n0 / 16 + wave * C::B_CP), 0, K);
  static_assert(C::B_CP == 1 && C::WSCP == 1, "one weight row group per wave");
  const int NQ = (KT + 3) / 4;
  auto issue_scales = [&](int q) {
    q = q < NQ ? q : NQ - 1;
    copy4(s_lane + scales_group_offset(clamp_rg(it.n0 / 16 + wave), q, K),
          lds + C::WS_OFF + ((q & 1) * C::NRG + wave) * 256);
  };
  auto slot = [&](int kt) { return lds + (kt % S) * C::A_STAGE; };
  auto bslot = [&](int kt) { return lds + C::B_RING + (kt % S) * C::B_BYTES; };
  auto issue = [&](int kt) {
    const int k = kt < KT ? kt : KT - 1;
    copy16_nt(b_lane + b_off + (int64_t)k * 1024, bslot(kt) + wave * 1024);
#pragma unroll
    for (int jj = 0; jj < C::A_CP; ++jj) {
      const int j = min(wave * C::A_CP + jj, C::A_COPIES - 1);
      copy16(a_src[jj] + (int64_t)k * act_row_bytes(AF), slot(kt) + j * 1024);
    }
    if constexpr (!C::RS) copy4(as_src + (int64_t)k * 4, slot(kt) + C::A_BYTES + (wave % C::AS_CHUNKS) * 256);
  };

  struct Frag {
    i32x8_t A[RB];
    uint32_t as[RB];
    u32x4_t B[WN];
  };
  auto load_frag = [&](Frag& f, int kt) {
    if constexpr (C::RS) kt = kt < KT ? kt : KT - 1;  // (operands past K are not used)
    const uint8_t* as_ = slot(kt);
    const uint8_t* bs_ = bslot(kt);
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) f.B[cb] = *reinterpret_cast<const u32x4_t*>(bs_ + (wn * WN + cb) * 1024 + lane * 16);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = C::rowblock(wm, rb) * 16 + (lane & 15);
      if constexpr (AF == kActFp8) {
        // 8-bit A elements: lane group g supplies K 16 g .. 16 g + 15 and
        // 64 + 16 g .. 64 + 16 g + 15 (logical chunks g and 4 + g), with the
        // scale of block g as for E2M1 (the MFMA reads block b's scale from
        // lane group b)
        const int sw = (row >> 1) & 7;
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(as_ + row * 128 + (g ^ sw) * 16);
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(as_ + row * 128 + ((4 + g) ^ sw) * 16);
        f.A[rb] = (i32x8_t){(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                            (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
      } else {
        const int phys = g ^ ((row >> 1) & 3);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(as_ + row * 64 + phys * 16);
        f.A[rb] = (i32x8_t){(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      }
      if constexpr (C::RS)
        f.as[rb] = rs[row * RSB + (((kt >> 2) ^ ((row >> 1) & rs_sw)) << 4) + 4 * (kt & 3) + g];
      else
        f.as[rb] = as_[C::A_BYTES + row * 4 + g];
    }
  };
  uint32_t scur[WN];  // this wave's scale dwords of the current 4-k-tile group
  auto mfma_frag = [&](const Frag& f, int kt) {
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) {
      const uint32_t sb = (scur[cb] >> (8 * (kt & 3))) & 0xFFu;
      const i32x8_t B = {(int)f.B[cb][0], (int)f.B[cb][1], (int)f.B[cb][2], (int)f.B[cb][3], 0, 0, 0, 0};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f.A[rb], B, acc[rb][cb], AF == kActFp8 ? 0 : 4, 4, 0, (int)f.as[rb], 0, (int)sb);
    }
  };
  // the wave's own LDS reads complete (lgkmcnt(0)), then the barrier; no
  // memory fence: an LDS release fence would also wait for every
  // global->LDS copy in flight (they write LDS), draining the ring each step
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: the first scale group, every slot's copies (k-tiles
  // 0 .. S-1), then k-tile 0's operands
  issue_scales(0);
#pragma unroll
  for (int p = 0; p < S; ++p) issue(p);
  wait_vm<(S - 1) * (C::B_CP + C::OPS_A)>();
  barrier();
  Frag F[2];
  load_frag(F[0], 0);
  // ---- step kt: wait for k-tile kt + 1's copies, barrier, (group start)
  // scale dwords and the next group's scale copies, refill slot kt with
  // k-tile kt + S, read k-tile kt + 1's operands, MFMAs of k-tile kt
  auto step = [&](int kt, int j, auto wait) {
    wait();
    barrier();
    if (j == 0) {
#pragma unroll
      for (int cb = 0; cb < WN; ++cb)
        scur[cb] = *reinterpret_cast<const uint32_t*>(
            lds + C::WS_OFF + (((kt >> 2) & 1) * C::NRG + wn * WN + cb) * 256 + lane * 4);
      issue_scales((kt >> 2) + 1);
    }
    issue(kt + S);
    load_frag(F[(j + 1) & 1], kt + 1);
    mfma_frag(F[j & 1], kt);
  };
  for (int kt0 = 0; kt0 < KT; kt0 += 4) {
    const bool first = kt0 == 0;
    step(kt0, 0, [&] { if (first) wait_vm_dyn<C::pf_max_after()>(C::pf_after(0)); else wait_vm<C::pf_after(4)>(); });
    if (kt0 + 1 < KT)
      step(kt0 + 1, 1, [&] { if (first) wait_vm_dyn<C::pf_max_after()>(C::pf_after(1)); else wait_vm<C::pf_after(5)>(); });
    if (kt0 + 2 < KT)
      step(kt0 + 2, 2, [&] { if (first) wait_vm_dyn<C::pf_max_after()>(C::pf_after(2)); else wait_vm<C::pf_after(6)>(); });
    if (kt0 + 3 < KT)
      step(kt0 + 3, 3, [&] { if (first) wait_vm_dyn<C::pf_max_after()>(C::pf_after(3)); else wait_vm<C::pf_after(7)>(); });
  }
  // the copies issued past K land before the workgroup ends
  wait_vm<0>();
}

// Direct-weight tiles (MXFP4 activations): a workgroup owns a 320-token x
// 256-weight-row tile of one expert.  Only the activation rows go through
// LDS; every wave loads its own four weight row groups' codes straight into
// registers (the preshuffled 1 KiB of a row group and k-tile is exactly one
// MFMA B operand), two k-tiles ahead.  With the weights in LDS every weight
// byte crossed LDS twice (the copy, then each of the four waves that read its
// row group) and the LDS traffic and per-k-tile waits set the pace; here LDS
// carries the activations only, and the two M halves of the workgroup read
// each weight slice from HBM and then L2.
//
// The activation rows of a k-tile are loaded into registers (8 bytes per lane
// and load, five loads per wave) one step before their k-tile and written to
// one of two LDS slots just before the step's barrier.  Every global load of
// the loop thus writes registers, so the compiler's own vmcnt waits count
// them exactly (loads that write LDS directly would make it wait for all).
// The tile's activation scale bytes (rows of kRsStride bytes: K/32 <= 128)
// and the weight scale dwords of its 16 row groups ([16][K/512][256 B]) are
// copied into LDS once, before the loop.
//   waves: 2 x 4 grid, wave (wm, wn) owns row blocks wm, wm + 2, ... (10) and
//   row groups 4 wn .. 4 wn + 3 (gate / up pairs); 160 accumulator VGPRs.
// Workgroup barrier for LDS hand-offs: LDS-only release / acquire fences
// (they wait for this wave's LDS operations, lgkmcnt, not for its global
// loads) keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

constexpr int kRsStride = 128;
template <int AF>
struct CfgDW {
  static constexpr bool DW = true, PF = false, RS = true, IL = true;
  static constexpr int WMW = 2, WNW = kWaves / WMW, RB = 10, WN = 4;
  static constexpr int MT = 16 * RB * WMW;  // 320 token rows
  static constexpr int NRG = WN * WNW;      // 16 weight row groups
  static constexpr int NT = 16 * NRG;       // 256 weight rows
  static constexpr int ARB = act_row_bytes(AF);
  static constexpr int A_BYTES = MT * ARB;
  // activation rows of a k-tile pair: 16-byte loads per lane (128 bytes of
  // each row), two LDS slots of two k-tiles each
  static constexpr int A_LD = 2 * A_BYTES / (kThreads * 16);
  static constexpr int ROWS_OFF = 4 * A_BYTES;
  static constexpr int RS_OFF = ROWS_OFF + MT * 4;
  static constexpr int WSC_OFF = RS_OFF + MT * kRsStride;
  static constexpr int STAGE_MAX = WSC_OFF;  // LDS free for the epilogue (slots, rows, row scales)
  static constexpr size_t lds_bytes(int64_t K) {
    return (size_t)WSC_OFF + (size_t)NRG * (size_t)(K / 512) * 256;
  }
  // K a multiple of 512 (whole scale groups, 16-byte scale chunks) and at
  // most kRsStride scale bytes per row
  static constexpr bool fits(int64_t K) {
    return K > 0 && K % 512 == 0 && K / 32 <= kRsStride && lds_bytes(K) <= kTileLdsMax;
  }
  static_assert(AF == kActFp4 && (2 * A_BYTES) % (kThreads * 16) == 0, "direct-weight tile");
  __device__ static constexpr int rowblock(int wm, int rb) { return wm + WMW * rb; }
};

// load_row(r): what row r of the tile is read from (a global load at most);
// row_value(v): its A-matrix row index.
template <int AF, typename C, typename LoadRow, typename RowValue>
__device__ __forceinline__ void tile_mainloop_dw(const GemmArgs& a, const TileItem& it, int64_t K, int64_t N,
                                                 uint8_t* lds, f32x4_t (&acc)[C::RB][C::WN], LoadRow load_row,
                                                 RowValue row_value) {
  constexpr int WN = C::WN, RB = C::RB;
  const int lane = lane_id();
  const int g = lane >> 4, l15 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % C::WMW, wn = wave / C::WMW;
  const int KT = (int)(K / kTileK);
  const int NQ = KT / 4;
  const int RSB = (int)(K / 32);  // activation scale bytes per row
  const int32_t* rowidx = reinterpret_cast<const int32_t*>(lds + C::ROWS_OFF);
  uint8_t* rs = lds + C::RS_OFF;
  uint8_t* wsc = lds + C::WSC_OFF;

  const int nrg = (int)(N / 16);
  const int rg0 = it.n0 / 16;
  const int nrgt = nrg - rg0 < C::NRG ? nrg - rg0 : C::NRG;  // row groups of this tile
  // weight codes: one buffer descriptor over the expert; the row group and
  // k-tile as the scalar offset, the lane's 16 bytes as the vector offset, a
  // k-tile past K an out-of-range vector offset (zeros, no memory traffic)
  const int64_t cpe = codes_per_expert(N, K);
  const __amdgpu_buffer_rsrc_t wrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.w_codes + (int64_t)it.e * cpe), (short)0, (int)cpe, 0x00020000);
  uint32_t brg[WN];    // byte offset of the row group (wave-uniform)
  uint32_t wsoff[WN];  // LDS offset of the row group's scale dwords (group 0)
#pragma unroll
  for (int cb = 0; cb < WN; ++cb) {
    const int rgl = min(wn * WN + cb, nrgt - 1);  // a partial tile repeats its last row group
    brg[cb] = __builtin_amdgcn_readfirstlane((uint32_t)codes_tile_offset(rg0 + rgl, 0, K));
    wsoff[cb] = (uint32_t)(rgl * NQ * 256 + lane * 4);
  }
  u32x4_t B[2][WN];
  auto load_b = [&](int kt, u32x4_t (&dst)[WN]) {
    const uint32_t vo = (uint32_t)lane * 16u + (kt < KT ? 0u : 0x80000000u);
    const uint32_t ko = (uint32_t)(kt < KT ? kt : 0) * 1024u;
#pragma unroll
    for (int cb = 0; cb < WN; ++cb)
      dst[cb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrc, vo, brg[cb] + ko, kCpolNT));
  };
  // prologue.  Each thread's tile row is looked up, the weights of k-tiles 0
  // and 1 (they depend on the item only) go out behind it, the rows go into
  // LDS (waiting for the lookups only) and a barrier that waits for LDS
  // traffic only publishes them; then the weight scale copies, the row scale
  // copies and the activations of k-tiles 0 and 1, and everything lands
  // before the loop, whose waits then count register loads only.
  static_assert(C::MT <= kThreads, "one tile row per thread");
  int32_t* rowidx_w = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  const bool has_row = (int)threadIdx.x < C::MT;
  int row_raw = 0;
  if (has_row) row_raw = load_row((int)threadIdx.x);
  __builtin_amdgcn_sched_barrier(0);
  load_b(0, B[0]);
  load_b(1, B[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (has_row) rowidx_w[threadIdx.x] = row_value(row_raw);
  lds_sync();
  // one-time copies.  Row scale bytes: row r at rs + r * kRsStride, its
  // 16-byte chunk c at c ^ ((r >> 1) & 7) (a copy covers 8 rows; lanes past
  // a row's K / 32 bytes copy its chunk 0 again into an unread chunk)
  // (every LDS read of the tile rows comes before the first copy into LDS: a
  // read behind such a copy makes the compiler wait for all loads)
  static_assert((C::MT / 8) % kWaves == 0, "row scale copies");
  constexpr int RS_CP = C::MT / 8 / kWaves;
  int rs_row[RS_CP];
#pragma unroll
  for (int ii = 0; ii < RS_CP; ++ii) rs_row[ii] = rowidx[8 * (wave + kWaves * ii) + (lane >> 3)];
  // activation loads of a k-tile pair: load j of thread t takes 16-byte piece
  // p = t % 8 of the pair's 128 bytes of tile row 64 j + t / 8 -- k-tile
  // p / 4 of the pair, logical chunk p % 4 -- stored at that k-tile's half of
  // the slot, chunk (p % 4) ^ ((row >> 1) & 3); that swizzle does not depend
  // on j, so load j lands an immediate 64 rows further
  uint32_t a_off[C::A_LD];
  uint32_t a_dst;
  {
    const int t = (int)threadIdx.x;
    const int p = t & 7;
#pragma unroll
    for (int j = 0; j < C::A_LD; ++j) {
      const int row = 64 * j + (t >> 3);
      a_off[j] = (uint32_t)rowidx[row] * (uint32_t)(K / 2) + (uint32_t)p * 16u;
    }
    const int row = t >> 3;
    a_dst = (uint32_t)((p >> 2) * C::A_BYTES + row * 64 + (((p & 3) ^ ((row >> 1) & 3)) << 4));
  }
  // buffer loads: the k-tile pair as the scalar offset, the row piece as a
  // 32-bit vector offset (no 64-bit address registers per load)
  const int64_t a_bytes = a.a_rows * (K / 2);
  const __amdgpu_buffer_rsrc_t arc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.a_codes), (short)0, (int)(a_bytes < INT32_MAX ? a_bytes : INT32_MAX), 0x00020000);
  u32x4_t areg[C::A_LD];
  auto load_a = [&](int kp) {  // k-tile pair kp (k-tiles 2 kp, 2 kp + 1)
    const uint32_t ko = (uint32_t)(2 * kp < KT ? kp : KT / 2 - 1) * 128u;
#pragma unroll
    for (int j = 0; j < C::A_LD; ++j)
      areg[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(arc, a_off[j], ko, 0));
  };
  auto store_a = [&](int kp) {
    uint8_t* dst = lds + (kp & 1) * 2 * C::A_BYTES + a_dst;
#pragma unroll
    for (int j = 0; j < C::A_LD; ++j) *reinterpret_cast<u32x4_t*>(dst + 64 * 64 * j) = areg[j];
  };
  __builtin_amdgcn_sched_barrier(0);
  {
    const int nch = RSB / 16;
#pragma unroll
    for (int ii = 0; ii < RS_CP; ++ii) {
      const int i = wave + kWaves * ii;
      const int row = 8 * i + (lane >> 3);
      const int cp = lane & 7;               // physical chunk
      const int cl = cp ^ ((row >> 1) & 7);  // logical chunk it holds
      copy16(a.a_scales + (int64_t)rs_row[ii] * RSB + (cl < nch ? cl : 0) * 16, rs + i * 1024);
    }
  }
  load_a(0);
  // weight scale dwords: the tile's row groups are contiguous; whole KiB by
  // every wave (NRG * K/512 / 4 <= 32 KiB: at most four each, a short share
  // repeating the last KiB), a last partial KiB (256-byte pieces) at the end
  const uint8_t* ws_src = a.w_scales + (int64_t)it.e * scales_per_expert(N, K) + scales_group_offset(rg0, 0, K);
  const int ws_kib = nrgt * NQ / 4, ws_rem = (nrgt * NQ) % 4;
  static_assert(C::NRG * (kRsStride * 32 / 512) / 4 <= 4 * kWaves, "weight scale copies");
  if (ws_kib > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = min(wave + kWaves * i, ws_kib - 1);
      copy16(ws_src + u * 1024 + lane * 16, wsc + u * 1024);
    }
  }
  if (ws_rem > 0) {
    const int u = min(wave, ws_rem - 1);
    copy4(ws_src + ws_kib * 1024 + u * 256 + lane * 4, wsc + ws_kib * 1024 + u * 256);
  }
  wait_vm<0>();
  __builtin_amdgcn_sched_barrier(0);
  // operand reads: row block rb of the wave is tile row 32 rb + 16 wm + l15;
  // the MXFP4 swizzle (row >> 1) & 3 and the scale swizzle (row >> 1) & 7
  // depend on l15 only, so every row block is an immediate offset from one
  // per-lane address
  const int row0 = 16 * wm + l15;
  const uint32_t a_lane = (uint32_t)(row0 * 64 + ((g ^ ((row0 >> 1) & 3)) * 16));
  const int ssw = (row0 >> 1) & 7;
  const uint32_t s_lane = (uint32_t)(row0 * kRsStride + g);

  uint32_t scur[WN];

  // Pair step kp (k-tiles kt = 2 kp and kt + 1; J0 = kt % 4): the pair's
  // activation rows (loaded in the previous pair step) are stored into slot
  // kp & 1 -- the compiler waits for those loads, and so for the earlier
  // weight loads -- and a barrier publishes the slot (every wave's reads of
  // that slot from pair kp - 2 ended before its barrier in pair kp - 1); the
  // next pair's rows are loaded; then k-tile kt's MFMAs and the weight loads
  // of k-tile kt + 2 into the registers they consumed, and the same for
  // k-tile kt + 1.  One barrier per two k-tiles.
  auto half = [&](int kt, auto Jc, u32x4_t (&bset)[WN], const uint8_t* slot) {
    constexpr int J = decltype(Jc)::value;
    const uint8_t* ab = slot + (kt & 1) * C::A_BYTES + a_lane;
    const uint8_t* sbp = rs + s_lane + (((kt >> 2) ^ ssw) << 4) + 4 * J;
    u32x4_t av[RB];
    uint32_t as[RB];
    auto read_a = [&](int rb) {
      av[rb] = *reinterpret_cast<const u32x4_t*>(ab + rb * 32 * 64);
      as[rb] = sbp[rb * 32 * kRsStride];
    };
    read_a(0);
    read_a(1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb + 2 < RB) read_a(rb + 2);
      const i32x8_t A = {(int)av[rb][0], (int)av[rb][1], (int)av[rb][2], (int)av[rb][3], 0, 0, 0, 0};
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) {
        const i32x8_t Bv = {(int)bset[cb][0], (int)bset[cb][1], (int)bset[cb][2], (int)bset[cb][3], 0, 0, 0, 0};
        acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bv, acc[rb][cb], 4, 4, 0, (int)as[rb], J,
                                                                       (int)scur[cb]);
      }
    }
    // two operand reads, then four MFMAs, per row block (reads two blocks ahead)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (rb + 2 < RB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, WN, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_b(kt + 2, bset);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pair = [&](int kp, auto J0) {
    constexpr int J = decltype(J0)::value;
    const int kt = 2 * kp;
    store_a(kp);
    lds_sync();  // this wave's stores and reads of the previous pair are done
    if constexpr (J == 0) {
#pragma unroll
      for (int cb = 0; cb < WN; ++cb)
        scur[cb] = *reinterpret_cast<const uint32_t*>(wsc + wsoff[cb] + (kt >> 2) * 256);
    }
    load_a(kp + 1);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* slot = lds + (kp & 1) * 2 * C::A_BYTES;
    half(kt, std::integral_constant<int, J>{}, B[0], slot);
    half(kt + 1, std::integral_constant<int, J + 1>{}, B[1], slot);
  };
  for (int kp0 = 0; kp0 < KT / 2; kp0 += 2) {
    pair(kp0, std::integral_constant<int, 0>{});
    pair(kp0 + 1, std::integral_constant<int, 2>{});
  }
}

}  // namespace

// One item of gate_up + clamped SwiGLU: the GEMM of the item's tile, then
// the SwiGLU of its gate / up pairs into act.
template <int AF, typename C>
__device__ __forceinline__ void tile_gate_up_item(const GemmArgs& a, const TileItem& it, uint8_t* lds) {
  constexpr int WN = C::WN, RB = C::RB;
  const int64_t H = a.K, I = a.N / 2;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  auto fill_rows = [&] {
    for (int r = threadIdx.x; r < C::MT; r += blockDim.x)
      rowidx[r] = a.sorted[it.p0 + (r < it.rows ? r : 0)] / a.top_k;  // token of the tile row
    __syncthreads();
  };
  if constexpr (!C::DW) fill_rows();
  f32x4_t acc[RB][WN];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  if constexpr (C::DW)
    tile_mainloop_dw<AF, C>(
        a, it, H, a.N, lds, acc, [&](int r) { return a.sorted[it.p0 + (r < it.rows ? r : 0)]; },
        [&](int v) { return v / a.top_k; });  // token of the tile row
  else if constexpr (C::PF)
    tile_mainloop_pf<AF, C>(a, it, H, a.N, lds, acc);
  else
    tile_mainloop<AF, C>(a, it, H, a.N, lds, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WMW, wn = wave / C::WMW;
  const int nrg = (int)(a.N / 16);
  // The tile's act (MT rows x NT/2 features, bf16) is assembled in LDS (the
  // rings are free once every wave is past the k-loop and the copies issued
  // past K have landed) and written out as 16-byte row pieces: one store per
  // 16 bytes instead of a 2-byte store per element.  LDS row r holds 16-byte
  // chunk c at c ^ (r & SW), so the four row quads of an MFMA block land in
  // different banks.  Lane (g, l15) of wave (wm, wn) holds rows
  // 16 rowblock(wm, rb) + 4 g + r and features 16 (WN wn / 2 + f) + l15.
  constexpr int FT = C::NT / 2;      // features of the tile
  constexpr int RBYTES = FT * 2;     // LDS row bytes
  constexpr int CH = RBYTES / 16;    // 16-byte chunks per row (a power of two)
  constexpr int SW = CH < 16 ? CH - 1 : 15;
  static_assert(C::MT * RBYTES <= C::STAGE_MAX && (CH & (CH - 1)) == 0, "act staging");
  static_assert((C::MT * RBYTES / 16) % kThreads == 0, "act pieces");
  wait_vm<0>();
  __syncthreads();
  (void)nrg;
  {
    const int g = lane >> 4, l15 = lane & 15;
#pragma unroll
    for (int f = 0; f < WN / 2; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int feat = 16 * (wn * WN / 2 + f) + l15;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int row = C::rowblock(wm, rb) * 16 + 4 * g + r;
          const float v = swiglu_clamped(acc[rb][2 * f][r], acc[rb][2 * f + 1][r], a.clamp_limit);
          *reinterpret_cast<__bf16*>(lds + row * RBYTES + (((feat >> 3) ^ (row & SW)) << 4) + (feat & 7) * 2) =
              (__bf16)v;
        }
      }
  }
  __syncthreads();
  // 16-byte pieces: piece q of the tile is row q / CH, chunk q % CH
  const int nfeat = (int)(I - it.n0 / 2) < FT ? (int)(I - it.n0 / 2) : FT;  // features of a partial tile
#pragma unroll
  for (int i = 0; i < C::MT * RBYTES / 16 / kThreads; ++i) {
    const int q = threadIdx.x + i * kThreads;
    const int row = q / CH, c = q % CH;
    if (row < it.rows && c * 8 < nfeat) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(lds + row * RBYTES + ((c ^ (row & SW)) << 4));
      *reinterpret_cast<u32x4_t*>(a.act + (it.p0 + row) * I + it.n0 / 2 + c * 8) = v;
    }
  }
}

// gate_up + clamped SwiGLU.  grid: 8 * ceil(item bound / 8) workgroups of 512.
template <int AF, typename C>
__global__ __launch_bounds__(kThreads) void tile_gate_up_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  zero_duty(a);
  const int ntl = (int)((a.N + C::NT - 1) / C::NT);
  TileItem it;
  if (!tile_item(a, ntl, C::NT, &it)) return;
  tile_gate_up_item<AF, C>(a, it, lds);
}

// One item of down + combine: the GEMM of the item's tile, then its rows
// into y (ordered combine) or w * y into out32 (fp32 atomics).
template <int AF, bool ORDERED, typename C>
__device__ __forceinline__ void tile_down_item(const GemmArgs& a, const TileItem& it, uint8_t* lds) {
  constexpr int WN = C::WN, RB = C::RB;
  const int64_t I = a.K, H = a.N;
  int32_t* rowidx = reinterpret_cast<int32_t*>(lds + C::ROWS_OFF);
  auto fill_rows = [&] {
    for (int r = threadIdx.x; r < C::MT; r += blockDim.x)
      rowidx[r] = (int32_t)(it.p0 + (r < it.rows ? r : 0));  // sorted position of the tile row
    __syncthreads();
  };
  if constexpr (!C::DW) fill_rows();
  f32x4_t acc[RB][WN];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < WN; ++cb) acc[rb][cb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  if constexpr (C::DW)
    tile_mainloop_dw<AF, C>(
        a, it, I, H, lds, acc, [&](int r) { return (int32_t)(it.p0 + (r < it.rows ? r : 0)); },
        [](int v) { return v; });  // sorted position of the tile row
  else if constexpr (C::PF)
    tile_mainloop_pf<AF, C>(a, it, I, H, lds, acc);
  else
    tile_mainloop<AF, C>(a, it, I, H, lds, acc);

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WMW, wn = wave / C::WMW;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = C::rowblock(wm, rb) * 16 + 4 * (lane >> 4) + r;
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

template <int AF, bool ORDERED, typename C>
__global__ __launch_bounds__(kThreads) void tile_down_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int ntl = (int)((a.N + C::NT - 1) / C::NT);
  TileItem it;
  if (!tile_item(a, ntl, C::NT, &it)) return;
  tile_down_item<AF, ORDERED, C>(a, it, lds);
}

// ------------------------------------------------------------------ launchers
namespace {
// 128 x 512 tiles (bf16 prefill and large MX calls) and 320 x 128 tiles (MX
// calls whose experts hold up to 320 rows)
template <int AF>
using Cfg128 = Cfg<AF, 2, 4, 8, false, AF == kActFp4 ? 3 : 2, AF == kActFp4 ? 3 : 2>;
template <int AF>
using Cfg320 = Cfg<AF, 4, 5, 4, true, AF == kActFp8 ? 3 : 4, AF == kActFp8 ? 3 : 4, true, AF == kActFp4>;

template <int AF>
using Cfg320DW = CfgDW<AF>;

int64_t tile_grid(int64_t max_tiles, int64_t N, int nt) {
  const int64_t items = max_tiles * ((N + nt - 1) / nt);
  return 8 * ((items + 7) / 8);
}

// The first use of each kernel on a device raises its dynamic-LDS limit there
// to kTileLdsMax.
template <typename Kernel>
hipError_t lds_limit(Kernel kernel) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static hipError_t attr[kMaxDevices];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    attr[dev] = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTileLdsMax);
  });
  return attr[dev];
}

// Launch with `lds` bytes of dynamic LDS.
template <typename Kernel>
hipError_t launch_lds(Kernel kernel, int64_t grid, size_t lds, const GemmArgs& a, hipStream_t s) {
  if (hipError_t e = lds_limit(kernel); e != hipSuccess) return e;
  if (lds > kTileLdsMax) return hipErrorInvalidValue;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int AF, typename C>
hipError_t gate_up_c(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t grid = tile_grid(max_tiles, a.N, C::NT);
  return launch_lds(tile_gate_up_kernel<AF, C>, grid, C::lds_bytes(a.K), a, s);
}
template <int AF, bool ORDERED, typename C>
hipError_t down_co(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  const int64_t grid = tile_grid(max_tiles, a.N, C::NT);
  return launch_lds(tile_down_kernel<AF, ORDERED, C>, grid, C::lds_bytes(a.K), a, s);
}
template <int AF, typename C>
hipError_t down_c(const GemmArgs& a, int64_t max_tiles, bool ordered, hipStream_t s) {
  return ordered ? down_co<AF, true, C>(a, max_tiles, s) : down_co<AF, false, C>(a, max_tiles, s);
}

template <int AF>
hipError_t gate_up_af(const GemmArgs& a, int64_t max_tiles, int mt, bool dw, hipStream_t s) {
  if constexpr (AF == kActFp4)
    if (dw && mt == Cfg320DW<AF>::MT) return gate_up_c<AF, Cfg320DW<AF>>(a, max_tiles, s);
  if (dw) return hipErrorInvalidValue;
  if constexpr (AF != kActBf16)
    if (mt == Cfg320<AF>::MT) return gate_up_c<AF, Cfg320<AF>>(a, max_tiles, s);
  if (mt != Cfg128<AF>::MT) return hipErrorInvalidValue;
  return gate_up_c<AF, Cfg128<AF>>(a, max_tiles, s);
}
template <int AF>
hipError_t down_af(const GemmArgs& a, int64_t max_tiles, int mt, bool dw, bool ordered, hipStream_t s) {
  if constexpr (AF == kActFp4)
    if (dw && mt == Cfg320DW<AF>::MT) return down_c<AF, Cfg320DW<AF>>(a, max_tiles, ordered, s);
  if (dw) return hipErrorInvalidValue;
  if constexpr (AF != kActBf16)
    if (mt == Cfg320<AF>::MT) return down_c<AF, Cfg320<AF>>(a, max_tiles, ordered, s);
  if (mt != Cfg128<AF>::MT) return hipErrorInvalidValue;
  return down_c<AF, Cfg128<AF>>(a, max_tiles, ordered, s);
}
}  // namespace

bool tile_fits(int af, int mt, int64_t K, bool dw) {
  if (dw) return af == kActFp4 && mt == 320 && Cfg320DW<kActFp4>::fits(K);
  if (mt == 128) return true;
  if (mt != 320 || af == kActBf16) return false;
  return af == kActFp4 ? Cfg320<kActFp4>::lds_bytes(K) <= kTileLdsMax : Cfg320<kActFp8>::lds_bytes(K) <= kTileLdsMax;
}

hipError_t launch_gate_up_tile(const GemmArgs& a, int64_t max_tiles, int af, int mt, bool dw, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (af == kActFp8) return gate_up_af<kActFp8>(a, max_tiles, mt, dw, s);
  return af == kActFp4 ? gate_up_af<kActFp4>(a, max_tiles, mt, dw, s)
                       : gate_up_af<kActBf16>(a, max_tiles, mt, dw, s);
}

hipError_t launch_down_tile(const GemmArgs& a, int64_t max_tiles, int af, int mt, bool dw, bool ordered,
                            hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (af == kActFp8) return down_af<kActFp8>(a, max_tiles, mt, dw, ordered, s);
  return af == kActFp4 ? down_af<kActFp4>(a, max_tiles, mt, dw, ordered, s)
                       : down_af<kActBf16>(a, max_tiles, mt, dw, ordered, s);
}

}  // namespace mxmoe
