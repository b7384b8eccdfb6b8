// Grouped GEMMs for token tiles of at most 16 rows (decode and small expert
// segments): the weight stream is the whole cost.  The work is a list of units
// (expert tile, 16-feature block), all of the same weight size; a persistent
// grid of resident workgroups takes equal contiguous shares of that list, so
// every workgroup streams from the start of the kernel to its end and none is
// left running alone in a tail.  Inside a workgroup K is split across the
// waves; each wave keeps a ring of D unit slices in flight (unit u+D-1 loads
// while unit u is computed) across unit and tile boundaries; partial sums meet
// in LDS and are added in a fixed wave order (deterministic).
//
// Weight unpack and the MX block scale are applied once per weight element
// per step, in registers (campaign page "glm53-mxfp4-mi355x", section "Serving
// throughput": that per-element cost is what MXFP4 adds).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "route_dev.h"

namespace mxmoe {

namespace {

__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Tile-table reads are wave-uniform and the table is constant while these
// kernels run, so they go through the constant address space (scalar loads,
// counted apart from the vector loads of the weight stream).
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int tile_count(const GemmArgs& a) {
  return ((const_i32*)a.tile_off)[a.E_local];
}
__device__ __forceinline__ int4 tile_entry(const GemmArgs& a, int t) {
  const_i32* p = (const_i32*)a.tiles + 4 * (int64_t)t;
  return make_int4(p[0], p[1], p[2], p[3]);
}

// A scale dword holds the scales of 4 k-tiles (one per byte).  A wave's
// k-tiles [w*KPW, w*KPW + KPW) cover at most kScaleWords<KPW> dwords: the
// largest span over the residues w*KPW mod 4 (KPW 8: 2, KPW 7: 3, KPW 4: 1).
constexpr int scale_words(int kpw) {
  int m = 1;
  for (int w = 0; w < 4; ++w) {
    const int n = ((w * kpw) % 4 + kpw - 1) / 4 + 1;
    m = n > m ? n : m;
  }
  return m;
}
template <int KPW>
constexpr int kScaleWords = scale_words(KPW);
static_assert(kScaleWords<4> == 1 && kScaleWords<5> == 2 && kScaleWords<6> == 2 && kScaleWords<7> == 3 &&
              kScaleWords<8> == 2);

// One wave's slice of one weight unit: NG row groups x KPW k-tiles (packed
// codes) plus the scale dwords covering those k-tiles.
template <int NG, int KPW>
struct WSlice {
  u32x4_t w[KPW][NG];
  uint32_t sd[NG][kScaleWords<KPW>];
};
// The dword holding k-tile kt's scale in a wave whose range starts at kt0
// (a select chain: no dynamic register indexing).
template <int NSW>
__device__ __forceinline__ uint32_t scale_word(const uint32_t (&sd)[NSW], int kt, int kt0) {
  const int idx = (kt >> 2) - (kt0 >> 2);
  uint32_t v = sd[0];
#pragma unroll
  for (int j = 1; j < NSW; ++j) v = idx == j ? sd[j] : v;
  return v;
}

// Activation formats: 0 bf16, 1 MXFP4 (A4), 2 MXFP8 with E4M3 elements (A8).
constexpr int kActBf16 = 0, kActFp4 = 1, kActFp8 = 2;

// Activation operands of one wave's K range: bf16 (4 MFMA operands per
// k-tile), or per lane and k-tile 32 MX elements -- 16 bytes of packed E2M1 or
// 32 bytes of E4M3 -- and one scale byte.
template <int KPW, int AF>
struct ASlice;
template <int KPW>
struct ASlice<KPW, kActBf16> {
  u32x4_t av[KPW][4];
};
template <int KPW>
struct ASlice<KPW, kActFp4> {
  u32x4_t av[KPW];
  uint32_t as[KPW];
};
template <int KPW>
struct ASlice<KPW, kActFp8> {
  u32x4_t av[KPW][2];
  uint32_t as[KPW];
};

// Weight slices are buffer loads against a descriptor that spans the unit's NG
// adjacent row groups; a unit past the workgroup's share gets an empty
// descriptor, whose loads return zeros without touching memory.  NT: the
// loads carry the non-temporal hint (each slice is read once per step);
// without it an expert spread over several tiles can find the slices in L2.
// k-tiles past KT are clamped to KT-1 and contribute zero in compute_refill.
template <bool NT>
constexpr int kWeightCpol = NT ? 2 : 0;
template <bool NT, int NG, int KPW>
__device__ __forceinline__ void load_wcodes(WSlice<NG, KPW>& t, __amdgpu_buffer_rsrc_t rc, uint32_t group_bytes,
                                            int c, int kt0, int KT) {
  const int kt = kt0 + c < KT ? kt0 + c : KT - 1;
  const uint32_t off = (uint32_t)kt * 1024u + (uint32_t)lane_id() * 16u;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
    t.w[c][gi] = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, gi * group_bytes + off, 0, kWeightCpol<NT>));
}
template <bool NT, int NG, int KPW>
__device__ __forceinline__ void load_wscales(WSlice<NG, KPW>& t, __amdgpu_buffer_rsrc_t rs, uint32_t group_sbytes,
                                             int kt0, int KT) {
  const int q0 = kt0 >> 2;
  const int qmax = (KT - 1) >> 2;
  const uint32_t lo = (uint32_t)lane_id() * 4u;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const uint32_t base = gi * group_sbytes + lo;
#pragma unroll
    for (int j = 0; j < kScaleWords<KPW>; ++j) {
      const int q = q0 + j < qmax ? q0 + j : qmax;
      t.sd[gi][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, base + (uint32_t)q * 256u, 0, kWeightCpol<NT>);
    }
  }
}
template <bool NT, int NG, int KPW>
__device__ __forceinline__ void load_wslice(WSlice<NG, KPW>& t, __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                            uint32_t group_bytes, uint32_t group_sbytes, int kt0, int KT) {
#pragma unroll
  for (int c = 0; c < KPW; ++c) load_wcodes<NT>(t, rc, group_bytes, c, kt0, KT);
  load_wscales<NT>(t, rs, group_sbytes, kt0, KT);
}

// Activation operands are buffer loads: a lane whose tile row is past the
// segment end, and every k-tile past K, uses an offset at or past the end of
// the buffer (oob, soob = its size), which the buffer range check turns into
// zeros without touching memory -- so the loads need no branch, their values
// need no select (a select would force a wait right after the load), and only
// valid rows generate traffic.
template <int KPW>
__device__ __forceinline__ void load_aslice(ASlice<KPW, kActBf16>& t, __amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            uint32_t oob, __amdgpu_buffer_rsrc_t, uint32_t, uint32_t, int kt0,
                                            int KT) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int c = 0; c < KPW; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t off = kt0 + c < KT ? off0 + (uint32_t)((kt0 + c) * kTileK + 32 * g + 8 * m) * 2u : oob;
      t.av[c][m] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
}
template <int KPW>
__device__ __forceinline__ void load_aslice(ASlice<KPW, kActFp4>& t, __amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            uint32_t oob, __amdgpu_buffer_rsrc_t rss, uint32_t soff0,
                                            uint32_t soob, int kt0, int KT) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = kt0 + c < KT;
    const uint32_t off = kin ? off0 + (uint32_t)(4 * (kt0 + c) + g) * 16u : oob;
    const uint32_t soff = kin ? soff0 + (uint32_t)(4 * (kt0 + c) + g) : soob;
    t.av[c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    t.as[c] = __builtin_amdgcn_raw_buffer_load_b8(rss, soff, 0, 0);
  }
}
// MXFP8 row: one byte per element.  With 8-bit A elements the scaled MFMA
// takes K elements 16 g .. 16 g + 15 of the k-tile from lane group g's first
// four registers and 64 + 16 g .. 64 + 16 g + 15 from its last four, while the
// scale byte of 32-element block b is still read from lane group b (layout
// measured on gfx950 with one-hot operands).  So lane group g loads the two
// 16-byte pieces at 128 kt + 16 g and 128 kt + 64 + 16 g, and block g's scale.
template <int KPW>
__device__ __forceinline__ void load_aslice(ASlice<KPW, kActFp8>& t, __amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            uint32_t oob, __amdgpu_buffer_rsrc_t rss, uint32_t soff0,
                                            uint32_t soob, int kt0, int KT) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = kt0 + c < KT;
    const uint32_t off = kin ? off0 + (uint32_t)(kt0 + c) * 128u + (uint32_t)g * 16u : oob;
    const uint32_t soff = kin ? soff0 + (uint32_t)(4 * (kt0 + c) + g) : soob;
    t.av[c][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    t.av[c][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64u, 0, 0));
    t.as[c] = __builtin_amdgcn_raw_buffer_load_b8(rss, soff, 0, 0);
  }
}

// acc[g] += A(16 rows x this wave's K range) * W(row group g)^T, k-tile by
// k-tile, and as each k-tile's registers are consumed, refill(c) loads the
// same k-tile of a later unit into them (refill(-1): the scale dwords, which
// are decoded into per-k-tile operands first).  The weight stream thus keeps
// a steady amount in flight without a second register copy of the slice.
// Slots past K contribute zero through both operands; FULL (every wave's
// k-tiles inside K) drops the zeroing selects.  MS 16-row blocks of the tile
// share each unpacked weight operand: acc[ms * NG + g].
template <bool FULL, int MS, int NG, int KPW, typename Refill>
__device__ __forceinline__ void compute_refill(WSlice<NG, KPW>& wt, const ASlice<KPW, kActBf16> (&at)[MS], int kt0,
                                               int KT, f32x4_t (&acc)[MS * NG], Refill&& refill) {
  float sc[KPW][NG];
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const int kt = FULL || kt0 + c < KT ? kt0 + c : KT - 1;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      sc[c][gi] = e8m0_scale_operand((scale_word(wt.sd[gi], kt, kt0) >> (8 * (kt & 3))) & 0xFFu);
  }
  refill(-1);
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = FULL || kt0 + c < KT;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4_t b = __builtin_bit_cast(u32x4_t, unpack8_e2m1(wt.w[c][gi][m], sc[c][gi]));
        if constexpr (!FULL) b = kin ? b : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
          acc[ms * NG + gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, at[ms].av[c][m]), __builtin_bit_cast(bf16x8_t, b), acc[ms * NG + gi], 0,
              0, 0);
      }
    }
    refill(c);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// MX activations (AF = A4 or A8): the scaled MFMA takes the raw blocks and
// both scale bytes; A's format code is FP4 (4) or FP8 E4M3 (0), W's FP4.
template <bool FULL, int MS, int NG, int KPW, int AF, typename Refill>
__device__ __forceinline__ void compute_refill(WSlice<NG, KPW>& wt, const ASlice<KPW, AF> (&at)[MS], int kt0, int KT,
                                               f32x4_t (&acc)[MS * NG], Refill&& refill) {
  uint32_t sbyte[KPW][NG];
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = FULL || kt0 + c < KT;
    const int kt = kin ? kt0 + c : KT - 1;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const uint32_t sb = (scale_word(wt.sd[gi], kt, kt0) >> (8 * (kt & 3))) & 0xFFu;
      sbyte[c][gi] = kin ? sb : 127u;
    }
  }
  refill(-1);
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = FULL || kt0 + c < KT;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      u32x4_t wb = wt.w[c][gi];
      if constexpr (!FULL) wb = kin ? wb : (u32x4_t){0u, 0u, 0u, 0u};
      const i32x8_t B = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3], 0, 0, 0, 0};
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const ASlice<KPW, AF>& t = at[ms];
        i32x8_t A;
        if constexpr (AF == kActFp8)
          A = (i32x8_t){(int)t.av[c][0][0], (int)t.av[c][0][1], (int)t.av[c][0][2], (int)t.av[c][0][3],
                        (int)t.av[c][1][0], (int)t.av[c][1][1], (int)t.av[c][1][2], (int)t.av[c][1][3]};
        else
          A = (i32x8_t){(int)t.av[c][0], (int)t.av[c][1], (int)t.av[c][2], (int)t.av[c][3], 0, 0, 0, 0};
        acc[ms * NG + gi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            A, B, acc[ms * NG + gi], AF == kActFp8 ? 0 : 4, 4, 0, (int)t.as[c], 0, (int)sbyte[c][gi]);
      }
    }
    refill(c);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Sum the NW waves' partials into wave 0 (fixed order).  red: LDS [NW][NG][64][4].
template <int NG>
__device__ __forceinline__ bool reduce_to_wave0(f32x4_t (&acc)[NG], float* red, int NW) {
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  if (wave > 0) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      *reinterpret_cast<f32x4_t*>(red + ((wave * NG + gi) * 64 + lane) * 4) = acc[gi];
  }
  __syncthreads();
  if (wave != 0) return false;
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(red + ((w * NG + gi) * 64 + lane) * 4);
      acc[gi] += v;
    }
  return true;
}

}  // namespace

// Units are numbered tile-major, u = tile * FB + feature block.  A share is
// cut at tile boundaries into segments; each segment loads its tile's
// activation operands once, then walks its units with a ring of D weight
// slices: unit i sits in slot i % D and, k-tile by k-tile as it is computed,
// unit i + D is loaded into the same slot.  Slots past the segment end load
// through an empty descriptor (no traffic).  Nothing loaded is
// carried from one segment to the next, so no loaded register has to be
// copied at a join (such a copy waits for every load in flight).
// Shares weighted by dispatch slot: of the workgroups resident on one CU the
// ones dispatched later stream more slowly, so workgroup b, the (b / cus)-th
// on its CU, gets a share in proportion to 1 / (1 + c * (b / cus)).  W(b) is
// the weight of the workgroups before b; every workgroup evaluates it the same
// way, so the shares tile [0, U) exactly.  cus == 0 or c == 0: equal shares.
__device__ __forceinline__ double slot_weight_before(unsigned b, unsigned G, unsigned cus, float c) {
  double w = 0.0;
  for (unsigned s = 0, b0 = 0; b0 < b; ++s, b0 += cus) {
    const unsigned n = (b - b0 < cus ? b - b0 : cus);
    w += (double)n / (1.0 + (double)c * s);
  }
  (void)G;
  return w;
}
__device__ __forceinline__ void share_bounds(int64_t U, unsigned b, unsigned G, int cus, float c, int64_t* ub,
                                             int64_t* ue) {
  if (cus <= 0 || c == 0.f) {
    *ub = U * b / G;
    *ue = U * (b + 1) / G;
    return;
  }
  const double tot = slot_weight_before(G, G, cus, c);
  *ub = b == 0 ? 0 : (int64_t)((double)U * (slot_weight_before(b, G, cus, c) / tot));
  *ue = b + 1 == G ? U : (int64_t)((double)U * (slot_weight_before(b + 1, G, cus, c) / tot));
}
__device__ __forceinline__ void share_of(int64_t U, int64_t* ub, int64_t* ue, int cus = 0, float c = 0.f) {
  share_bounds(U, blockIdx.x, gridDim.x, cus, c, ub, ue);
}

// Units sliced by XCD.  Workgroup b runs on XCD b % 8 (round-robin
// dispatch).  When the feature blocks per tile FB, the grid and the slot CU
// count divide by 8, XCD x owns the feature blocks fb = x, x + 8, x + 16, ...
// of every tile: its workgroups split the XCD's units v = tile * (FB / 8) +
// fb / 8 into shares as above (b / 8 among G / 8, on cus / 8 CUs), and unit
// v's feature block is 8 (v % (FB / 8)) + x.  An expert with several tiles
// then streams each of its weight slices into one XCD's L2 once, where its
// other tiles find it (with contiguous shares every XCD would stream the whole
// expert, too much for its L2).
constexpr int kXcds = 8;
struct UnitMap {
  int fbv;     // feature blocks per tile in this workgroup's numbering (FB or FB / 8)
  int step;    // feature block of virtual block j: step * j + first
  int first;
  __device__ int fb(int j) const { return step * j + first; }
};
__device__ __forceinline__ bool xcd_sliced(int FB, unsigned G, int cus) {
  return FB % kXcds == 0 && G % kXcds == 0 && (cus == 0 || cus % kXcds == 0);
}
// the share [ub, ue) of workgroup b (units in its numbering) and the numbering
__device__ __forceinline__ UnitMap unit_share(int64_t ntiles, int FB, unsigned b, unsigned G, int cus, float c,
                                              int64_t* ub, int64_t* ue) {
  if (xcd_sliced(FB, G, cus)) {
    share_bounds(ntiles * (FB / kXcds), b / kXcds, G / kXcds, cus / kXcds, c, ub, ue);
    return UnitMap{FB / kXcds, kXcds, (int)(b % kXcds)};
  }
  share_bounds(ntiles * FB, b, G, cus, c, ub, ue);
  return UnitMap{FB, 1, 0};
}

// Segments of a share [ub, ub + n) of tile-major units (FBV per tile), one per
// tile, in walk order.  Plain: in order.  Aligned (an expert may span several
// tiles, whose units are then processed by several workgroups of one XCD):
// the share's last tile first, then the others in order, and inside each
// segment the feature blocks rotated so that, where the segment holds it,
// block (k mod FBV) is walked at the workgroup's k-th unit.  Every workgroup
// then tends to read feature block j of an expert's tiles at the same time,
// so the slice is fetched once and found in L2 by the others.
struct Segment {
  int t;     // tile
  int fb0;   // first unit's feature block (in the workgroup's numbering)
  int nu;    // units
  int rot;   // unit i is feature block fb0 + (i + rot) mod nu
  __device__ int fb(int i) const {
    const int v = i + rot;
    return fb0 + (v < nu ? v : v - nu);
  }
};
__device__ __forceinline__ Segment share_segment(int64_t ub, int64_t ue, int FBV, int si, bool aligned, int k) {
  const int t_first = (int)(ub / FBV), t_last = (int)((ue - 1) / FBV);
  Segment g;
  g.t = aligned && t_last > t_first ? (si == 0 ? t_last : t_first + si - 1) : t_first + si;
  const int64_t tb = (int64_t)g.t * FBV;
  const int64_t sb = ub > tb ? ub : tb, se = ue < tb + FBV ? ue : tb + FBV;
  g.fb0 = (int)(sb - tb);
  g.nu = (int)(se - sb);
  g.rot = 0;
  if (aligned) {
    const int r = ((k - g.fb0) % FBV + FBV) % FBV;
    g.rot = r < g.nu ? r : 0;
  }
  return g;
}

// gate_up: unit = (tile, 16 gate + 16 up features); writes act = SwiGLU(gate,
// up) in bf16 at the tile's sorted positions.  Side duty: zero zero_buf.
// ROUTE: every workgroup first routes the tokens itself (route_block_masks, or
// route_block past 32 tokens or 64 local experts; tables in LDS after the
// partial buffers; workgroup 0 also writes the global tables that the down and
// combine kernels read, and with dn_desc the down shares), so no routing kernel
// runs before this one.  MS: 16-row blocks per tile (tiles of 16 MS rows),
// all multiplied by each weight slice.
template <int KPW, int D, int AF, bool FULL, bool ROUTE, int MS, bool NT>
__global__ __launch_bounds__(512) void gate_up_ksplit_kernel(GemmArgs a, RouteArgs ra) {
  static_assert(MS == 1 || !ROUTE, "the fused routing builds 16-row tiles");
  constexpr int NA = 2 * MS;      // accumulators: gate and up of each row block
  extern __shared__ float red[];  // [2][waves][NA][64][4], then (ROUTE) the routing tables
  // The routing runs at a raised wave priority: the workgroups dispatched
  // last onto a CU route while the first ones already stream, and at equal
  // priority the older waves' instructions go first and hold them back.
  if constexpr (ROUTE) __builtin_amdgcn_s_setprio(3);
  if (a.zero_buf) {
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = tid; i < a.zero_n / 4; i += nthreads) reinterpret_cast<f32x4_t*>(a.zero_buf)[i] = z;
  }
  const int lane = lane_id();
  const int r = lane & 15;
  const int wave = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int64_t H = a.K, I = a.N / 2;
  const int KT = (int)(H / kTileK);
  const int kt0 = wave * KPW;
  const int FB = (int)(I / 16);
  RouteLds rl;
  uint32_t* tmask = nullptr;  // with route_block_masks: each local expert's token mask
  int ntiles;
  if constexpr (ROUTE) {
    const int64_t S = ra.T * (int64_t)ra.top_k;
    const int64_t bound = (ra.E_local < S ? ra.E_local : S) + S / 16;
    rl = route_lds(reinterpret_cast<int32_t*>(red + 2 * NW * NA * 64 * 4), S, ra.E_local, bound);
    tmask = reinterpret_cast<uint32_t*>(rl.cnt);  // [E_local] (the chunk counts' space)
    if (masks_route_ok(ra))
      route_block_masks<kFusedRouteMaxVpl>(ra, rl, tmask, blockIdx.x == 0);
    else
      route_block<kFusedRouteMaxVpl>(ra, rl, blockIdx.x == 0);
    __builtin_amdgcn_s_setprio(0);
    ntiles = __builtin_amdgcn_readfirstlane(rl.t1[ra.E_local]);
    if (blockIdx.x == 0 && a.dn_desc) {
      // the down kernel's shares and first tiles (its tile table is this one)
      for (int b = threadIdx.x; b < a.dn_grid; b += blockDim.x) {
        int64_t dub, due;
        const UnitMap dm = unit_share(ntiles, a.dn_fb, (unsigned)b, (unsigned)a.dn_grid, a.dn_cus, a.dn_c, &dub, &due);
        int4 d0 = make_int4((int)dub, (int)due, 0, 0), d1 = make_int4(0, 0, 0, 0);
        if (dub < due) {
          const int t = (int)(dub / dm.fbv);
          const int4 ti = rl.tiles[t];
          d0.z = ti.x;
          d0.w = ti.y;
          d1.x = ti.z;
          d1.y = t;
        }
        a.dn_desc[2 * b] = d0;
        a.dn_desc[2 * b + 1] = d1;
      }
    }
  } else {
    ntiles = tile_count(a);
  }
  int64_t ub, ue;
  const UnitMap um = unit_share(ntiles, FB, blockIdx.x, gridDim.x, a.slot_cus, a.slot_c, &ub, &ue);
  const int FBV = um.fbv;
  const uint32_t gbytes = (uint32_t)(16 * (H / 2));
  const uint32_t gsbytes = (uint32_t)(scale_groups(H) * 256);
  const int64_t cpe = codes_per_expert(a.N, H), spe = scales_per_expert(a.N, H);
  // LDS partial buffers alternate strictly from unit to unit (padding slots
  // included), so a buffer is rewritten only after the barrier that follows
  // wave 0's reads of it
  int phase = 0;
  const int nseg = ue > ub ? (int)((ue - 1) / FBV - ub / FBV) + 1 : 0;
  const bool aligned = !ROUTE && a.wcache;
  for (int si = 0, k = 0; si < nseg; ++si) {
    const Segment sg = share_segment(ub, ue, FBV, si, aligned, k);
    const int t = sg.t;
    k += sg.nu;
    int4 ti;
    if constexpr (ROUTE) {
      const int4 v = rl.tiles[t];
      ti = make_int4(__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                     __builtin_amdgcn_readfirstlane(v.z), 0);
    } else {
      ti = tile_entry(a, t);
    }
    const int rows = ti.y;
    const int64_t p0 = ti.z;
    const uint8_t* ecodes = a.w_codes + (int64_t)ti.x * cpe;
    const uint8_t* escales = a.w_scales + (int64_t)ti.x * spe;
    const int nu = sg.nu;
    auto load_unit = [&](int i, WSlice<2, KPW>& w) {
      const int fb = um.fb(sg.fb(i));
      const bool ok = i < nu;
      load_wslice<NT>(w, make_rsrc(ecodes + codes_tile_offset(2 * fb, 0, H), ok ? 2 * gbytes : 0u),
                  make_rsrc(escales + scales_group_offset(2 * fb, 0, H), ok ? 2 * gsbytes : 0u), gbytes, gsbytes,
                  kt0, KT);
    };
    WSlice<2, KPW> wt[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_unit(j, wt[j]);
    // this lane's row of each row block and its token (garbage past the
    // tile's rows: unused)
    ASlice<KPW, AF> at[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int row = 16 * ms + r;
      const bool valid = row < rows;
      int32_t tok_raw;
      if constexpr (ROUTE) {
        if (masks_route_ok(ra)) {
          // row r of the tile: token bit (p0 - offs[e]) + r of the expert's mask
          const int e = ti.x;
          tok_raw = valid ? nth_set_bit32(tmask[e], (int)(p0 - rl.offs[e]) + r) : 0;
        } else {
          tok_raw = rl.ptok[p0 + (valid ? r : 0)];
        }
      } else
        tok_raw = a.tile_tok[(int64_t)t * (16 * MS) + row];
      const int64_t tok = valid ? tok_raw : 0;
      if constexpr (AF != kActBf16) {
        const int64_t rb = AF == kActFp8 ? H : H / 2;  // code bytes per row
        const uint32_t nb = (uint32_t)(a.a_rows * rb), ns = (uint32_t)(a.a_rows * (H / 32));
        load_aslice(at[ms], make_rsrc(a.a_codes, nb), valid ? (uint32_t)(tok * rb) : nb, nb,
                    make_rsrc(a.a_scales, ns), valid ? (uint32_t)(tok * (H / 32)) : ns, ns, kt0, KT);
      } else {
        const uint32_t nb = (uint32_t)(a.a_rows * H * 2);
        __amdgpu_buffer_rsrc_t rs = make_rsrc(a.a_bf16, nb);
        load_aslice(at[ms], rs, valid ? (uint32_t)(tok * H * 2) : nb, nb, rs, 0u, 0u, kt0, KT);
      }
    }
    // one rotation of the ring: units i0 .. i0+D-1.  The first rotation is
    // peeled so that the loop is entered with the same loads in flight as at
    // its back edge (a shared wait would otherwise drain the whole stream).
    auto rotation = [&](int i0) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int i = i0 + j;
        // unit i sits in slot j; unit i + D refills it as it is consumed
        const int fbn = um.fb(sg.fb(i + D));
        const bool okn = i + D < nu;
        const __amdgpu_buffer_rsrc_t rcn = make_rsrc(ecodes + codes_tile_offset(2 * fbn, 0, H), okn ? 2 * gbytes : 0u);
        const __amdgpu_buffer_rsrc_t rsn =
            make_rsrc(escales + scales_group_offset(2 * fbn, 0, H), okn ? 2 * gsbytes : 0u);
        f32x4_t acc[NA];
#pragma unroll
        for (int q = 0; q < NA; ++q) acc[q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        compute_refill<FULL, MS>(wt[j], at, kt0, KT, acc, [&](int part) {
          if (part < 0)
            load_wscales<NT>(wt[j], rsn, gsbytes, kt0, KT);
          else
            load_wcodes<NT>(wt[j], rcn, gbytes, part, kt0, KT);
        });
        float* rb = red + (phase++ & 1) * (NW * NA * 64 * 4);
        if (reduce_to_wave0<NA>(acc, rb, NW) && i < nu) {
          const int64_t nn = (int64_t)um.fb(sg.fb(i)) * 16 + r;
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = 16 * ms + 4 * (lane >> 4) + q;
              if (row < rows) {
                const float v = swiglu_clamped(acc[2 * ms][q], acc[2 * ms + 1][q], a.clamp_limit);
                a.act[(p0 + row) * I + nn] = (uint16_t)f32_to_bf16_bits(v);
              }
            }
        }
      }
    };
    rotation(0);
    for (int i0 = D; i0 < nu; i0 += D) rotation(i0);
  }
}

// down + combine: unit = (tile, 16*NG output features).  Atomic combine adds
// weight * y into out32[token]; ORDERED writes y per sorted position to ybuf.
template <int KPW, int NG, int D, int AF, bool ORDERED, bool FULL, int MS, bool NT>
__global__ __launch_bounds__(512) void down_ksplit_kernel(GemmArgs a) {
  constexpr int NA = NG * MS;     // accumulators: NG row groups of each row block
  extern __shared__ float red[];  // [2][waves][NA][64][4]
  const int lane = lane_id();
  const int r = lane & 15;
  const int wave = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int64_t I = a.K, H = a.N;
  const int KT = (int)(I / kTileK);
  const int kt0 = wave * KPW;
  const int FB = (int)(H / (16 * NG));
  int64_t ub, ue;
  int4 first = make_int4(0, 0, 0, 0);  // with descriptors: the first segment's tile entry
  const bool desc = a.dn_desc && (int)gridDim.x == a.dn_grid;
  UnitMap um;
  if (desc) {
    const_i32* dp = (const_i32*)a.dn_desc + 8 * (int64_t)blockIdx.x;
    ub = dp[0];
    ue = dp[1];
    first = make_int4(dp[2], dp[3], dp[4], 0);
    um = xcd_sliced(FB, gridDim.x, a.slot_cus) ? UnitMap{FB / kXcds, kXcds, (int)(blockIdx.x % kXcds)}
                                                : UnitMap{FB, 1, 0};
  } else {
    um = unit_share(tile_count(a), FB, blockIdx.x, gridDim.x, a.slot_cus, a.slot_c, &ub, &ue);
  }
  const int FBV = um.fbv;
  const uint32_t gbytes = (uint32_t)(16 * (I / 2));
  const uint32_t gsbytes = (uint32_t)(scale_groups(I) * 256);
  const int64_t cpe = codes_per_expert(H, I), spe = scales_per_expert(H, I);
  // LDS partial buffers alternate strictly from unit to unit (padding slots
  // included), so a buffer is rewritten only after the barrier that follows
  // wave 0's reads of it
  int phase = 0;
  const int nseg = ue > ub ? (int)((ue - 1) / FBV - ub / FBV) + 1 : 0;
  const bool aligned = !desc && a.wcache;
  for (int si = 0, k = 0; si < nseg; ++si) {
    const Segment sg = share_segment(ub, ue, FBV, si, aligned, k);
    const int t = sg.t;
    k += sg.nu;
    const int4 ti = desc && si == 0 ? first : tile_entry(a, t);
    const int rows = ti.y;
    const int64_t p0 = ti.z;
    const uint8_t* ecodes = a.w_codes + (int64_t)ti.x * cpe;
    const uint8_t* escales = a.w_scales + (int64_t)ti.x * spe;
    const int nu = sg.nu;
    auto load_unit = [&](int i, WSlice<NG, KPW>& w) {
      const int fb = um.fb(sg.fb(i));
      const bool ok = i < nu;
      load_wslice<NT>(w, make_rsrc(ecodes + codes_tile_offset(fb * NG, 0, I), ok ? NG * gbytes : 0u),
                  make_rsrc(escales + scales_group_offset(fb * NG, 0, I), ok ? NG * gsbytes : 0u), gbytes, gsbytes,
                  kt0, KT);
    };
    WSlice<NG, KPW> wt[D];
#pragma unroll
    for (int j = 0; j < D; ++j) load_unit(j, wt[j]);
    ASlice<KPW, AF> at[MS];
    // token and router weight of this lane's four output rows of each block
    int64_t tok[MS][4];
    float wgt[MS][4];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const bool valid = 16 * ms + r < rows;
      const int64_t pr = p0 + 16 * ms + r;
      if constexpr (AF != kActBf16) {
        const int64_t rb = AF == kActFp8 ? I : I / 2;  // code bytes per row
        const uint32_t nb = (uint32_t)(a.a_rows * rb), ns = (uint32_t)(a.a_rows * (I / 32));
        load_aslice(at[ms], make_rsrc(a.a_codes, nb), valid ? (uint32_t)(pr * rb) : nb, nb,
                    make_rsrc(a.a_scales, ns), valid ? (uint32_t)(pr * (I / 32)) : ns, ns, kt0, KT);
      } else {
        const uint32_t nb = (uint32_t)(a.a_rows * I * 2);
        __amdgpu_buffer_rsrc_t rs = make_rsrc(a.a_bf16, nb);
        load_aslice(at[ms], rs, valid ? (uint32_t)(pr * I * 2) : nb, nb, rs, 0u, 0u, kt0, KT);
      }
      if constexpr (!ORDERED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 16 * ms + 4 * (lane >> 4) + q;
          const int64_t pp = p0 + (row < rows ? row : 0);
          tok[ms][q] = a.pos_tok[pp];
          wgt[ms][q] = a.pos_w[pp];
        }
      }
    }
    auto rotation = [&](int i0) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int i = i0 + j;
        const int fbn = um.fb(sg.fb(i + D));
        const bool okn = i + D < nu;
        const __amdgpu_buffer_rsrc_t rcn =
            make_rsrc(ecodes + codes_tile_offset(fbn * NG, 0, I), okn ? NG * gbytes : 0u);
        const __amdgpu_buffer_rsrc_t rsn =
            make_rsrc(escales + scales_group_offset(fbn * NG, 0, I), okn ? NG * gsbytes : 0u);
        f32x4_t acc[NA];
#pragma unroll
        for (int q = 0; q < NA; ++q) acc[q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        compute_refill<FULL, MS>(wt[j], at, kt0, KT, acc, [&](int part) {
          if (part < 0)
            load_wscales<NT>(wt[j], rsn, gsbytes, kt0, KT);
          else
            load_wcodes<NT>(wt[j], rcn, gbytes, part, kt0, KT);
        });
        float* rb = red + (phase++ & 1) * (NW * NA * 64 * 4);
        if (reduce_to_wave0<NA>(acc, rb, NW) && i < nu) {
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = 16 * ms + 4 * (lane >> 4) + q;
              if (row < rows) {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                  const int64_t nn = ((int64_t)um.fb(sg.fb(i)) * NG + gi) * 16 + r;
                  if constexpr (ORDERED) {
                    a.ybuf[(p0 + row) * H + nn] = acc[ms * NG + gi][q];
                  } else {
                    unsafeAtomicAdd(a.out32 + tok[ms][q] * H + nn, wgt[ms][q] * acc[ms * NG + gi][q]);
                  }
                }
              }
            }
        }
      }
    };
    rotation(0);
    for (int i0 = D; i0 < nu; i0 += D) rotation(i0);
  }
}

// ------------------------------------------------------------------ launchers
//
// Variants: (KPW, D) = k-tiles per wave, ring slots (units ahead).  Default:
// KPW 4 (5 or 8 when K needs it to fit 8 waves), D 1.
// MXFP4_MOE_DECODE_VARIANT (tuning builds only) picks another,
// "k<KPW>d<D>" with KPW 2 or 4 and D 1 or 2.  MXFP4_MOE_DECODE_WGS_PER_CU
// caps the resident workgroups per CU.
namespace {
struct Variant {
  int kpw, d;
};

Variant pick(int64_t K, bool defaults_only = false) {
  const int64_t KT = K / kTileK;
  Variant v{KT <= 32 ? 4 : KT <= 40 ? 5 : KT <= 48 ? 6 : KT <= 56 ? 7 : 8, 1};
  if (defaults_only) return v;
  if (const char* env = tuning_env("MXFP4_MOE_DECODE_VARIANT")) {
    int kpw = 0, d = 0;
    if (sscanf(env, "k%dd%d", &kpw, &d) == 2 && (kpw == 2 || kpw == 4) && (d == 1 || d == 2) &&
        (KT + kpw - 1) / kpw <= 8)
      v = {kpw, d};
  }
  return v;
}

// Workgroups of this kernel that are resident at once on the current device
// (occupancy x CUs), cached per (device, kernel, block, LDS).
struct GridKey {
  int dev;
  const void* fn;
  int block;
  size_t lds;
  int cap;
  int grid;
};
std::mutex g_grid_mu;
GridKey g_grid_cache[128];
int g_grid_n = 0;

hipError_t resident_grid(const void* fn, int block, size_t lds, int* grid, int cap_per_cu = 0) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(g_grid_mu);
    for (int i = 0; i < g_grid_n; ++i) {
      const GridKey& k = g_grid_cache[i];
      if (k.dev == dev && k.fn == fn && k.block == block && k.lds == lds && k.cap == cap_per_cu) {
        *grid = k.grid;
        return hipSuccess;
      }
    }
  }
  int cus = 0, per_cu = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, lds)) != hipSuccess) return e;
  if (cap_per_cu > 0 && cap_per_cu < per_cu) per_cu = cap_per_cu;
  if (const char* env = tuning_env("MXFP4_MOE_DECODE_WGS_PER_CU")) {
    const int cap = atoi(env);
    if (cap > 0 && cap < per_cu) per_cu = cap;
  }
  if (per_cu < 1) per_cu = 1;
  *grid = cus * per_cu;
  std::lock_guard<std::mutex> lk(g_grid_mu);
  if (g_grid_n < 128) g_grid_cache[g_grid_n++] = GridKey{dev, fn, block, lds, cap_per_cu, *grid};
  return hipSuccess;
}

// Slot weights c of the shares (measured on MI355X: with 3 workgroups per CU
// the third streams ~1.35x slower than the first; c = 0.25 for gate_up and 0.1
// for down took the kernels' last workgroups in by ~1 us).
// MXFP4_MOE_SLOT_C_GU / MXFP4_MOE_SLOT_C_DN (tuning builds only) override them.
float slot_c(const char* name, float dflt) {
  const char* v = tuning_env(name);
  return v ? (float)atof(v) : dflt;
}
std::mutex g_cus_mu;
int g_cus[64];
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(g_cus_mu);
    if (g_cus[dev] > 0) return g_cus[dev];
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(g_cus_mu);
    g_cus[dev] = cus;
  }
  return cus;
}

template <typename Kernel, typename... Args>
hipError_t launch_persistent_capped(Kernel kernel, int nw, size_t lds, int64_t max_units, int cap_per_cu,
                                    hipStream_t s, const Args&... args) {
  int grid = 0;
  hipError_t e = resident_grid(reinterpret_cast<const void*>(kernel), nw * 64, lds, &grid, cap_per_cu);
  if (e != hipSuccess) return e;
  if ((int64_t)grid > max_units) grid = (int)max_units;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(nw * 64), lds, s, args...);
  return hipGetLastError();
}
template <typename Kernel, typename... Args>
hipError_t launch_persistent(Kernel kernel, int nw, size_t lds, int64_t max_units, hipStream_t s,
                             const Args&... args) {
  return launch_persistent_capped(kernel, nw, lds, max_units, 0, s, args...);
}

// The down kernel's occupancy allows 4 workgroups per CU, but at that size
// some of the grid was measured (MI355X, decode dims) to start only as others
// finished, up to 10 us late; a persistent grid must be resident, so down
// takes at most 3 per CU.
constexpr int kDownWgsPerCu = 3;

template <int KPW, int D, int AF>
hipError_t gate_up_v(const GemmArgs& a0, const RouteArgs* r, int64_t max_tiles, hipStream_t s) {
  GemmArgs a = a0;
  static const float c_gu = slot_c("MXFP4_MOE_SLOT_C_GU", 0.25f);
  a.slot_c = c_gu;
  a.slot_cus = a.slot_c != 0.f ? device_cus() : 0;
  const int KT = (int)(a.K / kTileK);
  const int nw = (KT + KPW - 1) / KPW;
  if (nw > 8) return hipErrorInvalidValue;
  const int64_t mu = max_tiles * (a.N / 2 / 16);
  const int ms = a.tile_ms == 2 ? 2 : 1;
  size_t lds = (size_t)2 * nw * 2 * ms * 64 * 4 * sizeof(float);
  if (r) {
    if (ms != 1) return hipErrorInvalidValue;
    const int64_t S = r->T * (int64_t)r->top_k;
    const int64_t bound = (r->E_local < S ? r->E_local : S) + S / 16;
    lds += (size_t)route_block_words(S, r->E_local, bound) * sizeof(int32_t);
    if (lds > kRouteFusedMaxLds) return hipErrorInvalidValue;
    return KT % KPW == 0
               ? launch_persistent(gate_up_ksplit_kernel<KPW, D, AF, true, true, 1, true>, nw, lds, mu, s, a, *r)
               : launch_persistent(gate_up_ksplit_kernel<KPW, D, AF, false, true, 1, true>, nw, lds, mu, s, a, *r);
  }
  const RouteArgs none{};
  auto go = [&](auto full, auto kms, auto nt) -> hipError_t {
    return launch_persistent(gate_up_ksplit_kernel<KPW, D, AF, decltype(full)::value, false, decltype(kms)::value,
                                                   decltype(nt)::value>,
                             nw, lds, mu, s, a, none);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  if (ms == 2 || a.wcache) {
    // 32-row tiles and cached weight loads come only in the default variants
    // (one unit ahead); cached loads only with 16-row tiles
    if constexpr (D == 1) {
      if (ms == 2) {
        if constexpr (KPW == 4) return KT % KPW == 0 ? go(T_{}, M2{}, T_{}) : go(F_{}, M2{}, T_{});
        return hipErrorInvalidValue;
      }
      return KT % KPW == 0 ? go(T_{}, M1{}, F_{}) : go(F_{}, M1{}, F_{});
    }
    return hipErrorInvalidValue;
  }
  return KT % KPW == 0 ? go(T_{}, M1{}, T_{}) : go(F_{}, M1{}, T_{});
}

// Share parameters of a down launch (down_ksplit_shares).
struct DownShares {
  int grid, fb, cus;
  float c;
};

template <int KPW, int D, int AF, bool ORDERED>
hipError_t down_v(const GemmArgs& a0, int64_t max_tiles, hipStream_t s, DownShares* q = nullptr) {
  GemmArgs a = a0;
  static const float c_dn = slot_c("MXFP4_MOE_SLOT_C_DN", 0.10f);
  a.slot_c = c_dn;
  a.slot_cus = a.slot_c != 0.f ? device_cus() : 0;
  constexpr int NG = 2;
  const int KT = (int)(a.K / kTileK);
  const int nw = (KT + KPW - 1) / KPW;
  if (nw > 8) return hipErrorInvalidValue;
  const int64_t mu = max_tiles * (a.N / 16 / NG);
  const int ms = a.tile_ms == 2 ? 2 : 1;
  const size_t lds = (size_t)2 * nw * NG * ms * 64 * 4 * sizeof(float);
  auto go = [&](auto kernel) -> hipError_t {
    if (!q) return launch_persistent_capped(kernel, nw, lds, mu, kDownWgsPerCu, s, a);
    // the grid launch_persistent_capped takes
    int grid = 0;
    const hipError_t e = resident_grid(reinterpret_cast<const void*>(kernel), nw * 64, lds, &grid, kDownWgsPerCu);
    if (e != hipSuccess) return e;
    q->grid = (int64_t)grid > mu ? (int)mu : grid;
    q->fb = (int)(a.N / 16 / NG);
    q->cus = a.slot_cus;
    q->c = a.slot_c;
    return hipSuccess;
  };
  if (ms == 2 || a.wcache) {
    if constexpr (D == 1) {
      if (ms == 2) {
        if constexpr (KPW == 4)
          return KT % KPW == 0 ? go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, true, 2, true>)
                               : go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, false, 2, true>);
        return hipErrorInvalidValue;
      }
      return KT % KPW == 0 ? go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, true, 1, false>)
                           : go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, false, 1, false>);
    }
    return hipErrorInvalidValue;
  }
  return KT % KPW == 0 ? go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, true, 1, true>)
                       : go(down_ksplit_kernel<KPW, NG, D, AF, ORDERED, false, 1, true>);
}

template <int KPW, int D>
hipError_t gate_up_kd(const GemmArgs& a, const RouteArgs* r, int64_t max_tiles, int af, hipStream_t s) {
  if (af == kActFp8) {
    if constexpr (KPW >= 4 && D == 1) return gate_up_v<KPW, D, kActFp8>(a, r, max_tiles, s);
    return hipErrorInvalidValue;
  }
  return af == kActFp4 ? gate_up_v<KPW, D, kActFp4>(a, r, max_tiles, s) : gate_up_v<KPW, D, kActBf16>(a, r, max_tiles, s);
}
template <int KPW, int D>
hipError_t down_kd(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, hipStream_t s,
                   DownShares* q = nullptr) {
  if (af == kActFp8) {
    // A8 comes only in the default variants (KPW 4, 5 or more with one unit ahead)
    if constexpr (KPW >= 4 && D == 1)
      return ordered ? down_v<KPW, D, kActFp8, true>(a, max_tiles, s, q)
                     : down_v<KPW, D, kActFp8, false>(a, max_tiles, s, q);
    return hipErrorInvalidValue;
  }
  if (af == kActFp4)
    return ordered ? down_v<KPW, D, kActFp4, true>(a, max_tiles, s, q)
                   : down_v<KPW, D, kActFp4, false>(a, max_tiles, s, q);
  return ordered ? down_v<KPW, D, kActBf16, true>(a, max_tiles, s, q)
                 : down_v<KPW, D, kActBf16, false>(a, max_tiles, s, q);
}
}  // namespace

#define MXMOE_DECODE_VARIANTS(F) F(2, 1) F(2, 2) F(4, 1) F(4, 2)

hipError_t launch_gate_up_ksplit(const GemmArgs& a, const RouteArgs* route, int64_t max_tiles, int af,
                                 hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const Variant v = pick(a.K, af == kActFp8);
#define F(KPW, D) \
  if (v.kpw == KPW && v.d == D) return gate_up_kd<KPW, D>(a, route, max_tiles, af, s);
  MXMOE_DECODE_VARIANTS(F)
#undef F
  if (v.kpw == 5) return gate_up_kd<5, 1>(a, route, max_tiles, af, s);
  if (v.kpw == 6) return gate_up_kd<6, 1>(a, route, max_tiles, af, s);
  if (v.kpw == 7) return gate_up_kd<7, 1>(a, route, max_tiles, af, s);
  return gate_up_kd<8, 1>(a, route, max_tiles, af, s);
}

namespace {
hipError_t down_dispatch(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, hipStream_t s,
                         DownShares* q) {
  const Variant v = pick(a.K, af == kActFp8);
#define F(KPW, D) \
  if (v.kpw == KPW && v.d == D) return down_kd<KPW, D>(a, max_tiles, af, ordered, s, q);
  MXMOE_DECODE_VARIANTS(F)
#undef F
  if (v.kpw == 5) return down_kd<5, 1>(a, max_tiles, af, ordered, s, q);
  if (v.kpw == 6) return down_kd<6, 1>(a, max_tiles, af, ordered, s, q);
  if (v.kpw == 7) return down_kd<7, 1>(a, max_tiles, af, ordered, s, q);
  return down_kd<8, 1>(a, max_tiles, af, ordered, s, q);
}
}  // namespace

bool ksplit_two_blocks_fit(int64_t K, int af) {
  // with 4 k-tiles per wave (K up to 4096) the second row block's activation
  // registers fit beside the first in every activation format (at most 256
  // VGPRs, two waves per SIMD); wider waves would spill
  (void)af;
  return pick(K, true).kpw <= 4;
}

hipError_t launch_down_ksplit(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  return down_dispatch(a, max_tiles, af, ordered, s, nullptr);
}

hipError_t down_ksplit_shares(const GemmArgs& a, int64_t max_tiles, int af, bool ordered, int* grid, int* fb,
                              int* cus, float* c) {
  DownShares q{0, 0, 0, 0.f};
  const hipError_t e = max_tiles > 0 ? down_dispatch(a, max_tiles, af, ordered, nullptr, &q) : hipSuccess;
  *grid = q.grid;
  *fb = q.fb;
  *cus = q.cus;
  *c = q.c;
  return e;
}

}  // namespace mxmoe
