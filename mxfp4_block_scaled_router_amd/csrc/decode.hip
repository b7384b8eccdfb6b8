// Grouped GEMMs for token tiles of at most 16 rows (decode and small expert
// segments): the weight stream is the whole cost, so each workgroup takes one
// (expert tile, 16-feature block) and splits K across its waves.  Every wave
// issues all of its loads -- the packed weight blocks of its K range and the
// matching activation operands -- before its first MFMA, so a resident
// workgroup keeps its whole weight tile in flight; partial sums meet in LDS
// and are added in a fixed wave order (deterministic).
//
// Weight unpack and the MX block scale are applied once per weight element
// per step, in registers (campaign page "glm53-mxfp4-mi355x", section "Serving
// throughput": that per-element cost is what MXFP4 adds).
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

__device__ __forceinline__ u32x4_t ldg16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ __forceinline__ bool tile_of(const GemmArgs& a, int tile, int* e, int* rows, int64_t* p0) {
  const int n = a.tile_off[a.E_local];
  const int4 ti = a.tiles[tile < n ? tile : 0];   // independent of n: both loads in flight together
  if (tile >= n) return false;
  *e = ti.x;
  *rows = ti.y;
  *p0 = ti.z;
  return true;
}

// One wave's slice of one weight unit: NG row groups x KPW k-tiles (packed
// codes) plus the scale dwords covering those k-tiles.
template <int NG, int KPW>
struct WSlice {
  u32x4_t w[KPW][NG];
  uint32_t sd[NG][2];
};

// Activation operands of one wave's K range: bf16 (4 MFMA operands per
// k-tile) or, A4, one packed block and its scale byte per k-tile.
template <int KPW, bool A4>
struct ASlice;
template <int KPW>
struct ASlice<KPW, false> {
  u32x4_t av[KPW][4];
};
template <int KPW>
struct ASlice<KPW, true> {
  u32x4_t av[KPW];
  uint32_t as[KPW];
};

// k-tiles past KT are clamped to KT-1 (a valid address: no branch around a
// load) and contribute zero in compute_slice.
template <int NG, int KPW>
__device__ __forceinline__ void load_wslice(WSlice<NG, KPW>& t, const uint8_t* const (&wc)[NG],
                                            const uint8_t* const (&wsb)[NG], int kt0, int KT) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < KPW; ++c)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      int kt = kt0 + c < KT ? kt0 + c : KT - 1;
      t.w[c][gi] = ld_stream16(wc[gi] + (int64_t)kt * 1024 + lane * 16);
    }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    int q0 = kt0 >> 2;
    int q1 = (kt0 + KPW - 1) >> 2;
    int qmax = (KT - 1) >> 2;
    q0 = q0 < qmax ? q0 : qmax;
    q1 = q1 < qmax ? q1 : qmax;
    t.sd[gi][0] = ld_stream4(wsb[gi] + (int64_t)q0 * 256 + lane * 4);
    t.sd[gi][1] = ld_stream4(wsb[gi] + (int64_t)q1 * 256 + lane * 4);
  }
}

// Activation operands are buffer loads: a lane whose tile row is past the
// segment end passes an offset at the end of the buffer, which the buffer
// range check turns into zeros without touching memory -- so the loads need no
// branch and only valid rows generate traffic.
template <int KPW>
__device__ __forceinline__ void load_aslice(ASlice<KPW, false>& t, __amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            __amdgpu_buffer_rsrc_t, uint32_t, int kt0, int KT) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int c = 0; c < KPW; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      int kt = kt0 + c < KT ? kt0 + c : KT - 1;
      uint32_t off = off0 + (uint32_t)(kt * kTileK + 32 * g + 8 * m) * 2u;
      u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      u32x4_t z = {0u, 0u, 0u, 0u};
      t.av[c][m] = (kt0 + c < KT) ? v : z;
    }
}
template <int KPW>
__device__ __forceinline__ void load_aslice(ASlice<KPW, true>& t, __amdgpu_buffer_rsrc_t rs, uint32_t off0,
                                            __amdgpu_buffer_rsrc_t rss, uint32_t soff0, int kt0, int KT) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    int kt = kt0 + c < KT ? kt0 + c : KT - 1;
    u32x4_t v = __builtin_bit_cast(
        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + (uint32_t)(4 * kt + g) * 16u, 0, 0));
    uint32_t sv = __builtin_amdgcn_raw_buffer_load_b8(rss, soff0 + (uint32_t)(4 * kt + g), 0, 0);
    u32x4_t z = {0u, 0u, 0u, 0u};
    t.av[c] = (kt0 + c < KT) ? v : z;
    t.as[c] = sv;
  }
}

// acc[g] += A(16 rows x this wave's K range) * W(row group g)^T.  Every k-tile
// slot runs (no branch); slots past K contribute zero through both operands.
template <int NG, int KPW>
__device__ __forceinline__ void compute_slice(const WSlice<NG, KPW>& wt, const ASlice<KPW, false>& at, int kt0,
                                              int KT, f32x4_t (&acc)[NG]) {
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = kt0 + c < KT;
    const int kt = kin ? kt0 + c : KT - 1;
    const int which = ((kt >> 2) == (kt0 >> 2)) ? 0 : 1;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float sc = e8m0_scale_operand((wt.sd[gi][which] >> (8 * (kt & 3))) & 0xFFu);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4_t b = __builtin_bit_cast(u32x4_t, unpack8_e2m1(wt.w[c][gi][m], sc));
        u32x4_t z = {0u, 0u, 0u, 0u};
        b = kin ? b : z;
        acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, at.av[c][m]),
                                                          __builtin_bit_cast(bf16x8_t, b), acc[gi], 0, 0, 0);
      }
    }
  }
}
template <int NG, int KPW>
__device__ __forceinline__ void compute_slice(const WSlice<NG, KPW>& wt, const ASlice<KPW, true>& at, int kt0,
                                              int KT, f32x4_t (&acc)[NG]) {
#pragma unroll
  for (int c = 0; c < KPW; ++c) {
    const bool kin = kt0 + c < KT;
    const int kt = kin ? kt0 + c : KT - 1;
    const int which = ((kt >> 2) == (kt0 >> 2)) ? 0 : 1;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      uint32_t sb = (wt.sd[gi][which] >> (8 * (kt & 3))) & 0xFFu;
      sb = kin ? sb : 127u;
      i32x8_t A = {(int)at.av[c][0], (int)at.av[c][1], (int)at.av[c][2], (int)at.av[c][3], 0, 0, 0, 0};
      u32x4_t wb = kin ? wt.w[c][gi] : (u32x4_t){0u, 0u, 0u, 0u};
      i32x8_t B = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3], 0, 0, 0, 0};
      acc[gi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[gi], 4, 4, 0, (int)at.as[c], 0,
                                                                 (int)sb);
    }
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

// gate_up for tiles of <= 16 rows.  grid: x = tile upper bound, y = I / (16*FPW).
// A workgroup keeps one token tile (its activation operands load once) and
// walks FPW blocks of 16 gate + 16 up features with a D-deep ring of weight
// slices: block f+D-1 is loading while block f is computed.  Wave w takes
// k-tiles [w*KPW, w*KPW + KPW).
template <int KPW, int FPW, int D, bool A4>
__global__ __launch_bounds__(512) void gate_up_ksplit_kernel(GemmArgs a) {
  extern __shared__ float red[];  // [2][waves][2][64][4]
  if (a.zero_buf) {
    const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    const int64_t tid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = tid; i < a.zero_n / 4; i += nthreads) reinterpret_cast<f32x4_t*>(a.zero_buf)[i] = z;
  }
  int e, rows;
  int64_t p0;
  if (!tile_of(a, blockIdx.x, &e, &rows, &p0)) return;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int64_t H = a.K, I = a.N / 2;
  const int KT = (int)(H / kTileK);
  const int kt0 = wave * KPW;
  const int64_t fb0 = (int64_t)blockIdx.y * FPW;
  const uint8_t* ebase = a.w_codes + (int64_t)e * codes_per_expert(a.N, H);
  const uint8_t* esb = a.w_scales + (int64_t)e * scales_per_expert(a.N, H);
  auto load_unit = [&](int f, WSlice<2, KPW>& w) {
    const int64_t fgi = fb0 + f;
    const uint8_t* wc[2] = {ebase + codes_tile_offset(2 * fgi, 0, H), ebase + codes_tile_offset(2 * fgi + 1, 0, H)};
    const uint8_t* wsb[2] = {esb + scales_group_offset(2 * fgi, 0, H), esb + scales_group_offset(2 * fgi + 1, 0, H)};
    load_wslice(w, wc, wsb, kt0, KT);
  };
  WSlice<2, KPW> wt[D];
#pragma unroll
  for (int f = 0; f < D - 1 && f < FPW; ++f) load_unit(f, wt[f]);
  const int r = lane & 15;
  const bool valid = r < rows;
  const int64_t tok = a.sorted[p0 + (valid ? r : 0)] / a.top_k;
  ASlice<KPW, A4> at;
  if constexpr (A4) {
    const uint32_t nb = (uint32_t)(a.a_rows * (H / 2)), ns = (uint32_t)(a.a_rows * (H / 32));
    load_aslice(at, make_rsrc(a.a_codes, nb), valid ? (uint32_t)(tok * (H / 2)) : nb, make_rsrc(a.a_scales, ns),
                valid ? (uint32_t)(tok * (H / 32)) : ns, kt0, KT);
  } else {
    const uint32_t nb = (uint32_t)(a.a_rows * H * 2);
    __amdgpu_buffer_rsrc_t rs = make_rsrc(a.a_bf16, nb);
    load_aslice(at, rs, valid ? (uint32_t)(tok * H * 2) : nb, rs, 0u, kt0, KT);
  }
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    if (f + D - 1 < FPW) load_unit(f + D - 1, wt[(f + D - 1) % D]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    compute_slice(wt[f % D], at, kt0, KT, acc);
    float* rb = red + (f & 1) * (NW * 2 * 64 * 4);
    if (reduce_to_wave0<2>(acc, rb, NW)) {
      const int64_t n = (fb0 + f) * 16 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int row = 4 * (lane >> 4) + q;
        if (row < rows) {
          float v = swiglu_clamped(acc[0][q], acc[1][q], a.clamp_limit);
          a.act[(p0 + row) * I + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// down + combine for tiles of <= 16 rows.  grid: x = tile upper bound,
// y = H / (16*NG*FPW); same walk over FPW blocks of 16*NG output features.
template <int KPW, int NG, int FPW, int D, bool A4, bool ORDERED>
__global__ __launch_bounds__(512) void down_ksplit_kernel(GemmArgs a) {
  extern __shared__ float red[];  // [2][waves][NG][64][4]
  int e, rows;
  int64_t p0;
  if (!tile_of(a, blockIdx.x, &e, &rows, &p0)) return;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int64_t I = a.K, H = a.N;
  const int KT = (int)(I / kTileK);
  const int kt0 = wave * KPW;
  const int64_t fb0 = (int64_t)blockIdx.y * FPW;
  const uint8_t* ebase = a.w_codes + (int64_t)e * codes_per_expert(H, I);
  const uint8_t* esb = a.w_scales + (int64_t)e * scales_per_expert(H, I);
  auto load_unit = [&](int f, WSlice<NG, KPW>& w) {
    const uint8_t* wc[NG];
    const uint8_t* wsb[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      wc[gi] = ebase + codes_tile_offset((fb0 + f) * NG + gi, 0, I);
      wsb[gi] = esb + scales_group_offset((fb0 + f) * NG + gi, 0, I);
    }
    load_wslice(w, wc, wsb, kt0, KT);
  };
  WSlice<NG, KPW> wt[D];
#pragma unroll
  for (int f = 0; f < D - 1 && f < FPW; ++f) load_unit(f, wt[f]);
  const int r = lane & 15;
  const bool valid = r < rows;
  const int64_t pr = p0 + r;
  ASlice<KPW, A4> at;
  if constexpr (A4) {
    const uint32_t nb = (uint32_t)(a.a_rows * (I / 2)), ns = (uint32_t)(a.a_rows * (I / 32));
    load_aslice(at, make_rsrc(a.a_codes, nb), valid ? (uint32_t)(pr * (I / 2)) : nb, make_rsrc(a.a_scales, ns),
                valid ? (uint32_t)(pr * (I / 32)) : ns, kt0, KT);
  } else {
    const uint32_t nb = (uint32_t)(a.a_rows * I * 2);
    __amdgpu_buffer_rsrc_t rs = make_rsrc(a.a_bf16, nb);
    load_aslice(at, rs, valid ? (uint32_t)(pr * I * 2) : nb, rs, 0u, kt0, KT);
  }
  // combine operands of this lane's four rows
  int64_t tok[4];
  float wgt[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * (lane >> 4) + q;
    const int32_t slot = a.sorted[p0 + (row < rows ? row : 0)];
    tok[q] = slot / a.top_k;
    wgt[q] = a.route_w[slot];
  }
#pragma unroll
  for (int f = 0; f < FPW; ++f) {
    if (f + D - 1 < FPW) load_unit(f + D - 1, wt[(f + D - 1) % D]);
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t acc[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) acc[gi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    compute_slice(wt[f % D], at, kt0, KT, acc);
    float* rb = red + (f & 1) * (NW * NG * 64 * 4);
    if (reduce_to_wave0<NG>(acc, rb, NW)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 4 * (lane >> 4) + q;
        if (row < rows) {
          const int64_t p = p0 + row;
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            const int64_t n = ((fb0 + f) * NG + gi) * 16 + r;
            if constexpr (ORDERED) {
              a.ybuf[p * H + n] = acc[gi][q];
            } else {
              float prod = wgt[q] * acc[gi][q];
              unsafeAtomicAdd(a.out32 + tok[q] * H + n, prod);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers
//
// Variants: (KPW, FPW, D) = k-tiles per wave, feature blocks per workgroup,
// weight ring depth.  Default: KPW 4 (5 or 8 when K needs it to fit 8 waves),
// FPW 4, D 2 -- the fastest of the measured set on the decode shape.
// MXFP4_MOE_DECODE_VARIANT (tests and benchmarks only) picks another, e.g.
// "k2d3f8" = KPW 2, FPW 8, D 3.
namespace {
struct Variant {
  int kpw, fpw, d;
};

Variant pick(int64_t K) {
  const int64_t KT = K / kTileK;
  Variant v{KT <= 32 ? 4 : KT <= 40 ? 5 : 8, 4, 2};
  if (const char* env = getenv("MXFP4_MOE_DECODE_VARIANT")) {
    if (!strcmp(env, "k4d2") && KT <= 32) v = {4, 4, 2};
    else if (!strcmp(env, "k4d3") && KT <= 32) v = {4, 4, 3};
    else if (!strcmp(env, "k2d2") && KT <= 16) v = {2, 4, 2};
    else if (!strcmp(env, "k2d3f8") && KT <= 16) v = {2, 8, 3};
  }
  return v;
}

template <int KPW, int FPW, int D>
hipError_t gate_up_v(const GemmArgs& a, int64_t max_tiles, bool a4, hipStream_t s) {
  const int nw = (int)((a.K / kTileK + KPW - 1) / KPW);
  const int64_t fb = a.N / 2 / 16;
  if (nw > 8 || fb % FPW) return hipErrorInvalidValue;
  dim3 grid((unsigned)max_tiles, (unsigned)(fb / FPW));
  size_t lds = (size_t)2 * nw * 2 * 64 * 4 * sizeof(float);
  if (a4) hipLaunchKernelGGL((gate_up_ksplit_kernel<KPW, FPW, D, true>), grid, dim3(nw * 64), lds, s, a);
  else hipLaunchKernelGGL((gate_up_ksplit_kernel<KPW, FPW, D, false>), grid, dim3(nw * 64), lds, s, a);
  return hipGetLastError();
}

template <int KPW, int FPW, int D>
hipError_t down_v(const GemmArgs& a, int64_t max_tiles, bool a4, bool ordered, hipStream_t s) {
  constexpr int NG = 2;
  const int nw = (int)((a.K / kTileK + KPW - 1) / KPW);
  const int64_t fb = a.N / 16 / NG;
  if (nw > 8 || fb % FPW) return hipErrorInvalidValue;
  dim3 grid((unsigned)max_tiles, (unsigned)(fb / FPW));
  size_t lds = (size_t)2 * nw * NG * 64 * 4 * sizeof(float);
  if (a4) {
    if (ordered) hipLaunchKernelGGL((down_ksplit_kernel<KPW, NG, FPW, D, true, true>), grid, dim3(nw * 64), lds, s, a);
    else hipLaunchKernelGGL((down_ksplit_kernel<KPW, NG, FPW, D, true, false>), grid, dim3(nw * 64), lds, s, a);
  } else {
    if (ordered) hipLaunchKernelGGL((down_ksplit_kernel<KPW, NG, FPW, D, false, true>), grid, dim3(nw * 64), lds, s, a);
    else hipLaunchKernelGGL((down_ksplit_kernel<KPW, NG, FPW, D, false, false>), grid, dim3(nw * 64), lds, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gate_up_ksplit(const GemmArgs& a, int64_t max_tiles, bool a4, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const Variant v = pick(a.K);
  if (v.kpw == 2 && v.fpw == 4 && v.d == 3) return gate_up_v<2, 4, 3>(a, max_tiles, a4, s);
  if (v.kpw == 2 && v.fpw == 4 && v.d == 2) return gate_up_v<2, 4, 2>(a, max_tiles, a4, s);
  if (v.kpw == 2 && v.fpw == 8) return gate_up_v<2, 8, 3>(a, max_tiles, a4, s);
  if (v.kpw == 4 && v.d == 2) return gate_up_v<4, 4, 2>(a, max_tiles, a4, s);
  if (v.kpw == 4) return gate_up_v<4, 4, 3>(a, max_tiles, a4, s);
  if (v.kpw == 5) return gate_up_v<5, 4, 2>(a, max_tiles, a4, s);
  return gate_up_v<8, 4, 2>(a, max_tiles, a4, s);
}

hipError_t launch_down_ksplit(const GemmArgs& a, int64_t max_tiles, bool a4, bool ordered, hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  const Variant v = pick(a.K);
  if (v.kpw == 2 && v.fpw == 4 && v.d == 3) return down_v<2, 4, 3>(a, max_tiles, a4, ordered, s);
  if (v.kpw == 2 && v.fpw == 4 && v.d == 2) return down_v<2, 4, 2>(a, max_tiles, a4, ordered, s);
  if (v.kpw == 2 && v.fpw == 8) return down_v<2, 8, 3>(a, max_tiles, a4, ordered, s);
  if (v.kpw == 4 && v.d == 2) return down_v<4, 4, 2>(a, max_tiles, a4, ordered, s);
  if (v.kpw == 4) return down_v<4, 4, 3>(a, max_tiles, a4, ordered, s);
  if (v.kpw == 5) return down_v<5, 4, 2>(a, max_tiles, a4, ordered, s);
  return down_v<8, 4, 2>(a, max_tiles, a4, ordered, s);
}

}  // namespace mxmoe
