// Grouped GEMMs of the routed experts over the permuted assignments.
//
//   gate_up:  h = W13_e x_t for the rows of one expert segment, fused with the
//             clamped SwiGLU; writes act (bf16) in sorted order.
//   down:     y = W2_e a for the same rows, fused with the weighted combine:
//             fp32 atomics into out32 (default) or y rows for an ordered gather.
//
// Weights stream from HBM in the preshuffled layout (common.h): each lane's
// 16-byte load is one MX block of one weight row, unpacked in registers by
// v_cvt_scalef32_pk_bf16_fp4 (exact: E2M1 * 2^(S-127) fits bf16) and fed to
// v_mfma_f32_16x16x32_bf16 as the B operand; in the A4 path the packed block
// and its scale byte go straight into v_mfma_scale_f32_16x16x128_f8f6f4.  The
// MXFP4 unpack plus block scale is paid once per weight element per workgroup
// (campaign page "glm53-mxfp4-mi355x", section "Serving throughput").
//
// MFMA operand layout (16x16x32 bf16, checked on gfx950): A lane l holds row
// l%16, K elements 8*(l/16)..+7; B lane l holds column l%16, the same K
// elements; D lane l holds column l%16, rows 4*(l/16)..+3.  Any permutation of
// K applied to both operands leaves the product unchanged, so K element
// 8*m + e of the lane's 32-element block feeds MFMA m (m = 0..3) of a k-tile.
//
// Tokens are the M dimension (A), weight rows the N dimension (B).
#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

struct Tile {
  int e;
  int rows;      // valid rows in this tile (<= MT)
  int64_t p0;    // first sorted position
};

__device__ __forceinline__ bool find_tile(const GemmArgs& a, int tile, int MT, Tile* out) {
  const int n = a.tile_off[a.E_local];
  const int4 ti = a.tiles[tile < n ? tile : 0];
  if (tile >= n) return false;
  out->e = ti.x;
  out->rows = ti.y;
  out->p0 = ti.z;
  return true;
}

__device__ __forceinline__ void zero_duty(const GemmArgs& a) {
  if (!a.zero_buf) return;
  const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * blockDim.x;
  const int64_t tid = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  f32x4_t* p = reinterpret_cast<f32x4_t*>(a.zero_buf);
  for (int64_t i = tid; i < a.zero_n / 4; i += nthreads) p[i] = z;
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_fp4(u32x4_t a, uint32_t sa, u32x4_t b, uint32_t sb, f32x4_t c) {
  i32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  i32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// ------------------------------------------------------------------------
// W4A16 main loop: acc[ms][g] += A(tile rows) x W(row group g)^T over all K.
//   NG weight row groups per wave, MS 16-row token subtiles per workgroup,
//   CH k-tiles (of 128) per pipeline stage.  The workgroup stages its A rows
//   in LDS per stage; row_off_lds[row] is the element offset of token-tile row
//   `row` from abase (-1: a zero row).
// ------------------------------------------------------------------------
template <int MS, int NG, int NW, int CH>
struct W4A16Loop {
  static constexpr int MT = 16 * MS;
  static constexpr int KC = CH * kTileK;          // K per stage
  static constexpr int LDS_STRIDE = KC + 8;       // bf16 elements per LDS row (16 B pad)
  static constexpr int NT = NW * 64;
  static constexpr int UNITS = MT * KC / 8;       // 16-byte units per stage
  static constexpr int UPT = (UNITS + NT - 1) / NT;

  static constexpr size_t lds_bytes() { return (size_t)MT * LDS_STRIDE * 2; }

  __device__ static void run(const int64_t* row_off_lds,            // LDS: row base offsets (elements), -1 = zero row
                             const uint16_t* abase, int64_t K,
                             const uint8_t* const* wc,              // [NG] codes base of row group
                             const uint8_t* const* wsb,             // [NG] scales base of row group
                             uint16_t* lds, f32x4_t (&acc)[MS][NG]) {
    const int lane = lane_id();
    const int g = lane >> 4;
    const int KT = (int)(K / kTileK);
    const int nstage = (KT + CH - 1) / CH;

    u32x4_t wcur[CH][NG], wnext[CH][NG];
    uint32_t scur[NG], snext[NG];
    u32x4_t stage_regs[UPT];

    auto load_w = [&](int st, u32x4_t (&wr)[CH][NG], uint32_t (&sr)[NG]) {
      const int kt0 = st * CH;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        sr[gi] = *reinterpret_cast<const uint32_t*>(wsb[gi] + (int64_t)(kt0 >> 2) * 256 + lane * 4);
#pragma unroll
        for (int c = 0; c < CH; ++c)
          if (kt0 + c < KT) wr[c][gi] = ld16(wc[gi] + (int64_t)(kt0 + c) * 1024 + lane * 16);
      }
    };
    auto load_stage_regs = [&](int st) {
      const int64_t k0 = (int64_t)st * KC;
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        int u = threadIdx.x + i * NT;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (u < UNITS) {
          int row = u / (KC / 8), col = (u % (KC / 8)) * 8;
          int64_t off = row_off_lds[row];
          if (off >= 0 && k0 + col < K) v = ld16(abase + off + k0 + col);
        }
        stage_regs[i] = v;
      }
    };
    auto store_stage_lds = [&]() {
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        int u = threadIdx.x + i * NT;
        if (u < UNITS) {
          int row = u / (KC / 8), col = (u % (KC / 8)) * 8;
          *reinterpret_cast<u32x4_t*>(lds + row * LDS_STRIDE + col) = stage_regs[i];
        }
      }
    };
    auto compute = [&](int st, const u32x4_t (&wr)[CH][NG], const uint32_t (&sr)[NG]) {
      const int kt0 = st * CH;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (kt0 + c >= KT) break;
        float sc[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          sc[gi] = e8m0_scale_operand((sr[gi] >> (8 * ((kt0 + c) & 3))) & 0xFFu);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          bf16x8_t av[MS];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) {
            const uint16_t* p = lds + (ms * 16 + (lane & 15)) * LDS_STRIDE + c * kTileK + 32 * g + 8 * m;
            av[ms] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
          }
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            bf16x8_t bv = unpack8_e2m1(wr[c][gi][m], sc[gi]);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) acc[ms][gi] = mfma_bf16(av[ms], bv, acc[ms][gi]);
          }
        }
      }
    };

    load_w(0, wcur, scur);
    load_stage_regs(0);
    for (int st = 0; st < nstage; ++st) {
      __syncthreads();
      store_stage_lds();
      __syncthreads();
      const bool more = st + 1 < nstage;
      if (more) {
        load_w(st + 1, wnext, snext);
        load_stage_regs(st + 1);
      }
      compute(st, wcur, scur);
      if (more) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) wcur[c][gi] = wnext[c][gi];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) scur[gi] = snext[gi];
      }
    }
  }
};

// ------------------------------------------------------------------------
// A4 main loop: both operands MXFP4, scaled FP4 MFMA, one MFMA per
// (token subtile, row group, k-tile).  A operands come straight from global
// memory: lane (row l%16, group l/16) loads block 4*kt + l/16 of its row.
// ------------------------------------------------------------------------
template <int MS, int NG>
__device__ __forceinline__ void a4_loop(const uint8_t* const (&arow)[MS], const uint8_t* const (&asrow)[MS],
                                        int64_t K, const uint8_t* const* wc, const uint8_t* const* wsb,
                                        f32x4_t (&acc)[MS][NG]) {
  const int lane = lane_id();
  const int g = lane >> 4;
  const int KT = (int)(K / kTileK);
  for (int kt = 0; kt < KT; ++kt) {
    u32x4_t av[MS];
    uint32_t sa[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      uint32_t s = 127;
      if (arow[ms]) {
        v = ld16(arow[ms] + (int64_t)(4 * kt + g) * 16);
        s = asrow[ms][4 * kt + g];
      }
      av[ms] = v;
      sa[ms] = s;
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      u32x4_t bv = ld16(wc[gi] + (int64_t)kt * 1024 + lane * 16);
      uint32_t sd = *reinterpret_cast<const uint32_t*>(wsb[gi] + (int64_t)(kt >> 2) * 256 + lane * 4);
      uint32_t sb = (sd >> (8 * (kt & 3))) & 0xFFu;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) acc[ms][gi] = mfma_fp4(av[ms], sa[ms], bv, sb, acc[ms][gi]);
    }
  }
}

}  // namespace

// ========================================================================
// gate_up + clamped SwiGLU
// grid: x = token tiles (upper bound), y = feature blocks of NW*FG*16 features
// ========================================================================
template <int MS, int FG, int NW, int CH, bool A4>
__global__ __launch_bounds__(NW * 64) void gate_up_kernel(GemmArgs a) {
  extern __shared__ uint16_t lds_dyn[];
  zero_duty(a);
  constexpr int MT = 16 * MS;
  constexpr int NG = 2 * FG;
  Tile tile;
  if (!find_tile(a, blockIdx.x, MT, &tile)) return;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t H = a.K, I = a.N / 2;
  const int64_t fgi0 = ((int64_t)blockIdx.y * NW + wave) * FG;

  const uint8_t* wc[NG];
  const uint8_t* wsb[NG];
  const uint8_t* ebase = a.w_codes + (int64_t)tile.e * codes_per_expert(a.N, H);
  const uint8_t* esb = a.w_scales + (int64_t)tile.e * scales_per_expert(a.N, H);
#pragma unroll
  for (int f = 0; f < FG; ++f)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu) {
      int64_t rg = 2 * (fgi0 + f) + gu;
      wc[2 * f + gu] = ebase + codes_tile_offset(rg, 0, H);
      wsb[2 * f + gu] = esb + scales_group_offset(rg, 0, H);
    }

  f32x4_t acc[MS][NG];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) acc[ms][gi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  if constexpr (A4) {
    const uint8_t* arow[MS];
    const uint8_t* asrow[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      int r = ms * 16 + (lane & 15);
      if (r < tile.rows) {
        int64_t tok = a.sorted[tile.p0 + r] / a.top_k;
        arow[ms] = a.a_codes + tok * (H / 2);
        asrow[ms] = a.a_scales + tok * (H / 32);
      } else {
        arow[ms] = nullptr;
        asrow[ms] = nullptr;
      }
    }
    a4_loop<MS, NG>(arow, asrow, H, wc, wsb, acc);
  } else {
    __shared__ int64_t row_off[MT];
    for (int r = threadIdx.x; r < MT; r += NW * 64)
      row_off[r] = r < tile.rows ? (int64_t)(a.sorted[tile.p0 + r] / a.top_k) * H : -1;
    __syncthreads();
    W4A16Loop<MS, NG, NW, CH>::run(row_off, a.a_bf16, H, wc, wsb, lds_dyn, acc);
  }

  // epilogue: act[p][n] = bf16(swiglu(g, u))
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int f = 0; f < FG; ++f) {
      const int64_t n = (fgi0 + f) * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int row = ms * 16 + 4 * (lane >> 4) + r;
        if (row < tile.rows) {
          float v = swiglu_clamped(acc[ms][2 * f][r], acc[ms][2 * f + 1][r], a.clamp_limit);
          a.act[(tile.p0 + row) * I + n] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
}

// ========================================================================
// down + combine
// grid: x = token tiles (upper bound), y = feature blocks of NW*FG*16 of H
// ========================================================================
template <int MS, int FG, int NW, int CH, bool A4, bool ORDERED>
__global__ __launch_bounds__(NW * 64) void down_kernel(GemmArgs a) {
  extern __shared__ uint16_t lds_dyn[];
  constexpr int MT = 16 * MS;
  constexpr int NG = FG;
  Tile tile;
  if (!find_tile(a, blockIdx.x, MT, &tile)) return;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t I = a.K, H = a.N;
  const int64_t rg0 = ((int64_t)blockIdx.y * NW + wave) * FG;

  const uint8_t* wc[NG];
  const uint8_t* wsb[NG];
  const uint8_t* ebase = a.w_codes + (int64_t)tile.e * codes_per_expert(H, I);
  const uint8_t* esb = a.w_scales + (int64_t)tile.e * scales_per_expert(H, I);
#pragma unroll
  for (int f = 0; f < FG; ++f) {
    wc[f] = ebase + codes_tile_offset(rg0 + f, 0, I);
    wsb[f] = esb + scales_group_offset(rg0 + f, 0, I);
  }
  f32x4_t acc[MS][NG];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) acc[ms][gi] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  if constexpr (A4) {
    const uint8_t* arow[MS];
    const uint8_t* asrow[MS];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      int r = ms * 16 + (lane & 15);
      if (r < tile.rows) {
        arow[ms] = a.a_codes + (tile.p0 + r) * (I / 2);
        asrow[ms] = a.a_scales + (tile.p0 + r) * (I / 32);
      } else {
        arow[ms] = nullptr;
        asrow[ms] = nullptr;
      }
    }
    a4_loop<MS, NG>(arow, asrow, I, wc, wsb, acc);
  } else {
    __shared__ int64_t row_off[MT];
    for (int r = threadIdx.x; r < MT; r += NW * 64)
      row_off[r] = r < tile.rows ? (tile.p0 + r) * I : -1;
    __syncthreads();
    W4A16Loop<MS, NG, NW, CH>::run(row_off, a.a_bf16, I, wc, wsb, lds_dyn, acc);
  }

  // epilogue
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int row = ms * 16 + 4 * (lane >> 4) + r;
      if (row < tile.rows) {
        const int64_t p = tile.p0 + row;
        if constexpr (ORDERED) {
#pragma unroll
          for (int f = 0; f < FG; ++f) {
            const int64_t n = (rg0 + f) * 16 + (lane & 15);
            a.ybuf[p * H + n] = acc[ms][f][r];
          }
        } else {
          const int32_t slot = a.sorted[p];
          const int64_t t = slot / a.top_k;
          const float wgt = a.route_w[slot];
#pragma unroll
          for (int f = 0; f < FG; ++f) {
            const int64_t n = (rg0 + f) * 16 + (lane & 15);
            float prod = wgt * acc[ms][f][r];
            unsafeAtomicAdd(a.out32 + t * H + n, prod);
          }
        }
      }
    }
}

// ========================================================================
// combine / cast
// ========================================================================
__global__ __launch_bounds__(256) void cast_out_kernel(CombineArgs a) {
  int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t n = a.T * a.H;
  if (i >= n) return;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.out32 + i);
  uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
  uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
  *reinterpret_cast<uint2*>(a.out + i) = make_uint2(lo, hi);
}

// out[t][n] = bf16( sum_j w[t,j] * y[inv[t,j]][n] ), slots in increasing j, fp32
__global__ __launch_bounds__(256) void combine_ordered_kernel(CombineArgs a) {
  int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int64_t n = a.T * a.H;
  if (i >= n) return;
  const int64_t t = i / a.H, c = i % a.H;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.top_k; ++j) {
    const int64_t s = t * a.top_k + j;
    const int32_t pos = a.inv[s];
    if (pos < 0) continue;
    const float wgt = a.route_w[s];
    f32x4_t y = *reinterpret_cast<const f32x4_t*>(a.ybuf + (int64_t)pos * a.H + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float prod = wgt * y[q];
      acc[q] = acc[q] + prod;
    }
  }
  uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
  uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
  *reinterpret_cast<uint2*>(a.out + i) = make_uint2(lo, hi);
  if (a.out32_copy) *reinterpret_cast<f32x4_t*>(a.out32_copy + i) = acc;
}

// Same sum, one workgroup per token: the token's slot positions and weights
// are scalar loads, and every thread issues the loads of all KMAX slot rows of
// its columns before adding them in increasing j (a slot past k or without a
// local expert loads row 0 and is skipped).
typedef const __attribute__((address_space(4))) int32_t c_i32;
typedef const __attribute__((address_space(4))) float c_f32;
template <int KMAX>
__global__ __launch_bounds__(256) void combine_gather_kernel(CombineArgs a) {
  const int64_t t = blockIdx.x;
  const int k = a.top_k;
  int32_t pos[KMAX];
  float w[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int64_t s = t * k + (j < k ? j : 0);
    pos[j] = j < k ? ((c_i32*)a.inv)[s] : -1;
    w[j] = ((c_f32*)a.route_w)[s];
  }
  const int64_t H = a.H;
  // two column chunks in flight per thread; the rows are read once
  // (non-temporal loads)
#pragma unroll 2
  for (int64_t c = threadIdx.x * 4; c < H; c += 4 * blockDim.x) {
    f32x4_t y[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      y[j] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(a.ybuf + (int64_t)(pos[j] >= 0 ? pos[j] : 0) * H + c));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (pos[j] < 0) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float prod = w[j] * y[j][q];
        acc[q] = acc[q] + prod;
      }
    }
    const int64_t i = t * H + c;
    uint32_t lo = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    uint32_t hi = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<uint2*>(a.out + i) = make_uint2(lo, hi);
    if (a.out32_copy) *reinterpret_cast<f32x4_t*>(a.out32_copy + i) = acc;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void copy_bytes_kernel(const uint8_t* src, uint8_t* dst, int64_t n16,
                                                         int64_t tail) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < n16; j += stride)
    reinterpret_cast<u32x4_t*>(dst)[j] = reinterpret_cast<const u32x4_t*>(src)[j];
  if (i < tail) dst[n16 * 16 + i] = src[n16 * 16 + i];
}

// ========================================================================
// launchers
// ========================================================================
namespace {

template <int MS, int FG, int NW, int CH, bool A4>
hipError_t gate_up_variant(const GemmArgs& a, int64_t max_tiles, hipStream_t s) {
  using L = W4A16Loop<MS, 2 * FG, NW, CH>;
  size_t lds = A4 ? 0 : L::lds_bytes();
  dim3 grid((unsigned)max_tiles, (unsigned)(a.N / 2 / 16 / (NW * FG)));
  hipLaunchKernelGGL((gate_up_kernel<MS, FG, NW, CH, A4>), grid, dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int MS, int FG, int NW, int CH, bool A4>
hipError_t down_variant(const GemmArgs& a, int64_t max_tiles, bool ordered, hipStream_t s) {
  using L = W4A16Loop<MS, FG, NW, CH>;
  size_t lds = A4 ? 0 : L::lds_bytes();
  dim3 grid((unsigned)max_tiles, (unsigned)(a.N / 16 / (NW * FG)));
  if (ordered)
    hipLaunchKernelGGL((down_kernel<MS, FG, NW, CH, A4, true>), grid, dim3(NW * 64), lds, s, a);
  else
    hipLaunchKernelGGL((down_kernel<MS, FG, NW, CH, A4, false>), grid, dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// The one plan of these kernels: (ms, fg, nw) = (4, 2, 4), 64-token tiles with
// the activation rows staged in LDS (16-row plans run the K-split kernels).
hipError_t launch_gate_up(const GemmArgs& a, const GemmPlan& p, int64_t max_tiles, bool a4,
                          hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (p.ms == 4 && p.fg == 2 && p.nw == 4)
    return a4 ? gate_up_variant<4, 2, 4, 2, true>(a, max_tiles, s)
              : gate_up_variant<4, 2, 4, 2, false>(a, max_tiles, s);
  return hipErrorInvalidValue;
}

hipError_t launch_down(const GemmArgs& a, const GemmPlan& p, int64_t max_tiles, bool a4, bool ordered,
                       hipStream_t s) {
  if (max_tiles <= 0) return hipSuccess;
  if (p.ms == 4 && p.fg == 2 && p.nw == 4)
    return a4 ? down_variant<4, 2, 4, 2, true>(a, max_tiles, ordered, s)
              : down_variant<4, 2, 4, 2, false>(a, max_tiles, ordered, s);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, bool ordered, hipStream_t s) {
  const int64_t n4 = a.T * a.H / 4;
  if (n4 == 0) return hipSuccess;
  dim3 grid((unsigned)((n4 + 255) / 256));
  if (ordered && a.top_k <= 8 && a.T <= INT32_MAX)
    hipLaunchKernelGGL(combine_gather_kernel<8>, dim3((unsigned)a.T), dim3(256), 0, s, a);
  else if (ordered && a.top_k == 9 && a.T <= INT32_MAX)  // top-8 + the shared expert
    hipLaunchKernelGGL(combine_gather_kernel<9>, dim3((unsigned)a.T), dim3(256), 0, s, a);
  else if (ordered && a.top_k <= 16 && a.T <= INT32_MAX)
    hipLaunchKernelGGL(combine_gather_kernel<16>, dim3((unsigned)a.T), dim3(256), 0, s, a);
  else if (ordered)
    hipLaunchKernelGGL(combine_ordered_kernel, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(cast_out_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  int64_t n16 = bytes / 16, tail = bytes % 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_bytes_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint8_t*)src, (uint8_t*)dst, n16, tail);
  return hipGetLastError();
}

}  // namespace mxmoe
