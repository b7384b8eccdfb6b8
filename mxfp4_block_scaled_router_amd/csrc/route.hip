// Router (softmax -> top-k -> renormalise) and the token permutation
// (local filter, per-expert histogram, prefix sum, stable scatter).
//
// Routing picks the experts "the router picked" for each token and reads only
// those (campaign page "glm53-mxfp4-mi355x", section "A file is a census; a
// decode step is a sample").  Selection is done on the logits, which softmax
// maps monotonically: ties go to the lower expert id.  The weights of the k
// picks are exp(l_j - l_max) / sum_i exp(l_i - l_max), computed in fp64 and
// rounded once to fp32 -- the softmax normaliser cancels in the renormalisation.
//
// Top-k: 16 lanes (one DPP row) per token, each holding every 16th logit; k
// rounds of a 16-lane argmax on (orderable logit, inverted id) keys.
//
// Permutation: slot s = t*k + j.  Slots are cut into 64-slot chunks; one wave
// per chunk finds each slot's rank among the chunk's earlier slots with the same
// expert (ballot over matching lanes) and the chunk's per-expert counts.  A
// scan over chunks gives each (chunk, expert) its base, an exclusive scan over
// experts the offsets, and the scatter puts slot s at
// offsets[e] + base[chunk][e] + rank[s] -- the stable counting sort.
#include "common.h"
#include "launch.h"

namespace mxmoe {

namespace {

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}

// DPP row (16-lane) butterflies: quad [1,0,3,2], quad [2,3,0,1], half mirror,
// mirror.  Each pairs every lane with a distinct partner, so after the four
// steps every lane of the row holds the row's reduction.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void max_step(uint32_t& hi, uint32_t& lo) {
  uint32_t oh = dpp<CTRL>(hi), ol = dpp<CTRL>(lo);
  bool take = (oh > hi) || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}
__device__ __forceinline__ void row16_max_u64(uint32_t& hi, uint32_t& lo) {
  max_step<kDppXor1>(hi, lo);
  max_step<kDppXor2>(hi, lo);
  max_step<kDppHalfMirror>(hi, lo);
  max_step<kDppMirror>(hi, lo);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t lo = dpp<CTRL>((uint32_t)u), hi = dpp<CTRL>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double row16_sum_f64(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return v;
}

// Top-k of token t by the 16-lane row of this lane.  lexp_out[s - slot_base]
// receives the local expert (or -1) of each of the token's k slots s.
template <int VPL>
__device__ void topk_row(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base) {
  const int r = lane_id() & 15;
  const int E = a.E_global, k = a.top_k;
  const float* row = a.logits + t * (int64_t)E;
  uint32_t khi[VPL], klo[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = r + 16 * i;
    bool in = e < E;
    float v = in ? row[e] : 0.0f;
    khi[i] = in ? orderable(v) : 0u;
    klo[i] = in ? 0xFFFFFFFFu - (uint32_t)e : 0u;
  }
  uint32_t p0hi = 0, p0lo = 0, p1hi = 0, p1lo = 0;  // picks r and r + 16
  uint32_t maxhi = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bh = 0, bl = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      bool take = (khi[i] > bh) || (khi[i] == bh && klo[i] > bl);
      bh = take ? khi[i] : bh;
      bl = take ? klo[i] : bl;
    }
    row16_max_u64(bh, bl);
    const uint32_t id = 0xFFFFFFFFu - bl;
    if ((int)(id & 15) == r) {
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if ((uint32_t)i == (id >> 4)) khi[i] = klo[i] = 0u;
    }
    if (j == 0) maxhi = bh;
    if (j == r) { p0hi = bh; p0lo = bl; }
    if (j == r + 16) { p1hi = bh; p1lo = bl; }
  }
  const double m = (double)from_orderable(maxhi);
  const bool has0 = r < k, has1 = r + 16 < k;
  const double e0 = has0 ? exp((double)from_orderable(p0hi) - m) : 0.0;
  const double e1 = has1 ? exp((double)from_orderable(p1hi) - m) : 0.0;
  const double sum = row16_sum_f64(e0 + e1);
  const int64_t s0 = t * k;
  if (has0) {
    int id = (int)(0xFFFFFFFFu - p0lo);
    a.ids[s0 + r] = id;
    const float w = (float)(e0 / sum);
    a.w[s0 + r] = w;
    if (w_out) w_out[s0 + r - slot_base] = w;
    int le = id - a.first_local;
    lexp_out[s0 + r - slot_base] = (le >= 0 && le < a.E_local) ? le : -1;
  }
  if (has1) {
    int id = (int)(0xFFFFFFFFu - p1lo);
    a.ids[s0 + r + 16] = id;
    const float w = (float)(e1 / sum);
    a.w[s0 + r + 16] = w;
    if (w_out) w_out[s0 + r + 16 - slot_base] = w;
    int le = id - a.first_local;
    lexp_out[s0 + r + 16 - slot_base] = (le >= 0 && le < a.E_local) ? le : -1;
  }
}

__device__ void topk_any(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base) {
  const int vpl = (a.E_global + 15) / 16;
  if (vpl <= 1) topk_row<1>(a, t, lexp_out, w_out, slot_base);
  else if (vpl <= 2) topk_row<2>(a, t, lexp_out, w_out, slot_base);
  else if (vpl <= 4) topk_row<4>(a, t, lexp_out, w_out, slot_base);
  else if (vpl <= 8) topk_row<8>(a, t, lexp_out, w_out, slot_base);
  else if (vpl <= 16) topk_row<16>(a, t, lexp_out, w_out, slot_base);
  else topk_row<32>(a, t, lexp_out, w_out, slot_base);
}

// Rank of each slot of chunk c among the chunk's slots with the same local
// expert, and the chunk's per-expert counts cnt[e * stride] (zeroed
// beforehand; only experts present in the chunk are written).  One wave.
// The lanes holding the same expert are found bit by bit: one ballot per bit
// of the expert id (nbits = bits of E_local - 1), each lane keeping the lanes
// that agree with its own bit -- a fixed number of ballots, however many
// distinct experts the chunk holds.
__device__ void chunk_ranks(int64_t S, int64_t c, const int32_t* lexp, int32_t* cnt, int64_t stride,
                            int32_t* rank, int nbits) {
  const int lane = lane_id();
  const int64_t s = c * 64 + lane;
  const int e = s < S ? lexp[s] : -1;
  uint64_t same = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  if (e >= 0) {
    const uint64_t below = same & ((1ull << lane) - 1ull);
    if (below == 0) cnt[e * stride] = __popcll(same);
    if (s < S) rank[s] = __popcll(below);
  } else if (s < S) {
    rank[s] = 0;
  }
}

// Exclusive scan of the per-expert counts v[0..n) by one wave: expert offsets
// and, for the two token-tile heights mt1/mt2, tile offsets (prefix of
// ceil(v/mt)) into offs_lds[0..n] and t1_lds[0..n] (entry n = total).  With
// write_global it also writes a.offsets, a.tile_off1/2 and the flat tile
// tables tiles1/tiles2: tile i -> {expert, rows, first sorted position, 0}.
__device__ void wave_scan_experts(const int32_t* v, int n, const RouteArgs& a, bool write_global,
                                  int32_t* offs_lds, int32_t* t1_lds) {
  const int lane = lane_id();
  const int mt1 = a.mt1, mt2 = a.mt2;
  const int per = (n + 63) / 64;
  const int b = lane * per;
  int32_t s0 = 0, s1 = 0, s2 = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      int32_t c = v[b + i];
      s0 += c;
      s1 += (c + mt1 - 1) / mt1;
      s2 += (c + mt2 - 1) / mt2;
    }
  // inclusive wave prefix of the lane totals
  int32_t i0 = s0, i1 = s1, i2 = s2;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t a0 = __shfl_up(i0, off, 64), a1 = __shfl_up(i1, off, 64), a2 = __shfl_up(i2, off, 64);
    if (lane >= off) { i0 += a0; i1 += a1; i2 += a2; }
  }
  int32_t r0 = i0 - s0, r1 = i1 - s1, r2 = i2 - s2;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int e = b + i;
      const int32_t c = v[e];
      offs_lds[e] = r0;
      t1_lds[e] = r1;
      if (write_global) {
        a.offsets[e] = r0;
        a.tile_off1[e] = r1;
        a.tile_off2[e] = r2;
        for (int32_t m0 = 0, j = 0; m0 < c; m0 += mt1, ++j)
          a.tiles1[r1 + j] = make_int4(e, c - m0 < mt1 ? c - m0 : mt1, r0 + m0, 0);
        for (int32_t m0 = 0, j = 0; m0 < c; m0 += mt2, ++j)
          a.tiles2[r2 + j] = make_int4(e, c - m0 < mt2 ? c - m0 : mt2, r0 + m0, 0);
      }
      r0 += c;
      r1 += (c + mt1 - 1) / mt1;
      r2 += (c + mt2 - 1) / mt2;
    }
  if (lane == 63) {
    offs_lds[n] = i0;
    t1_lds[n] = i1;
    if (write_global) {
      a.offsets[n] = i0;
      a.tile_off1[n] = i1;
      a.tile_off2[n] = i2;
    }
  }
}

// Sorted position pos of slot s: the permutation both ways, the side tables
// (token and router weight w of pos) and -- for 16-row tiles -- the token of
// that tile row.  off_e, tile_e: offset and first 16-row tile of the slot's
// expert.
__device__ __forceinline__ void place_slot(const RouteArgs& a, int64_t s, int32_t pos, float w, int32_t off_e,
                                           int32_t tile_e) {
  const int32_t t = (int32_t)(s / a.top_k);
  a.sorted[pos] = (int32_t)s;
  a.inv[s] = pos;
  a.pos_tok[pos] = t;
  a.pos_w[pos] = w;
  if (a.tile_tok) {
    const int32_t rel = pos - off_e;
    a.tile_tok[(int64_t)(tile_e + rel / 16) * 16 + rel % 16] = t;
  }
}

}  // namespace

// ---------------------------------------------------------------- kernels

// Whole routing in one workgroup of 512 threads, for small T*k*E (decode).
// Everything read after the logits comes from LDS: slot experts, weights and
// ranks, chunk counts, counts, expert and tile offsets.
__global__ __launch_bounds__(512) void route_small_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int nwaves = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = lane_id();
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  const int E = a.E_local;
  int32_t* lexp = lds;                                  // [S]
  int32_t* rank = lexp + S;                             // [S]
  float* wl = reinterpret_cast<float*>(rank + S);       // [S]
  int32_t* cnt = reinterpret_cast<int32_t*>(wl + S);    // [nchunk][E]
  int32_t* counts = cnt + nchunk * E;                   // [E]
  int32_t* offs = counts + E;                           // [E + 1]
  int32_t* t1 = offs + E + 1;                           // [E + 1]
  for (int64_t i = threadIdx.x; i < nchunk * E; i += blockDim.x) cnt[i] = 0;
  for (int64_t t = wave * 4 + (lane >> 4); t < a.T; t += nwaves * 4) topk_any(a, t, lexp, wl, 0);
  __syncthreads();
  const int nbits = 32 - __builtin_clz((unsigned)(E > 1 ? E - 1 : 1));
  for (int64_t c = wave; c < nchunk; c += nwaves) chunk_ranks(S, c, lexp, cnt + c * E, 1, rank, nbits);
  __syncthreads();
  // per expert: running sum over chunks -> chunk bases; totals -> counts
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int64_t c = 0; c < nchunk; ++c) {
      int32_t v = cnt[c * E + e];
      cnt[c * E + e] = run;
      run += v;
    }
    counts[e] = run;
    a.counts[e] = run;
  }
  __syncthreads();
  if (wave == 0) wave_scan_experts(counts, E, a, true, offs, t1);
  __syncthreads();
  for (int64_t s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = lexp[s];
    if (e >= 0)
      place_slot(a, s, offs[e] + cnt[(s / 64) * E + e] + rank[s], wl[s], offs[e], t1[e]);
    else
      a.inv[s] = -1;
  }
}

// ---- routing for larger T*k*E, in three kernels
// (1) top-k and chunk ranks: a workgroup of 256 threads (16 rows of 16 lanes)
// takes `tpb` tokens, tpb*k a multiple of 64, so its slots are whole chunks.
// Chunk counts are stored expert-major, chunk_cnt[e][chunk].
__global__ __launch_bounds__(256) void route_topk_chunk_kernel(RouteArgs a, int tpb) {
  extern __shared__ int32_t lds[];
  const int wave = threadIdx.x / 64;
  const int E = a.E_local, k = a.top_k;
  const int64_t S = a.T * (int64_t)k;
  const int64_t nchunk = (S + 63) / 64;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  const int64_t s0 = t0 * k;
  const int nslot = tpb * k;
  const int nch = nslot / 64;
  int32_t* lexp = lds;  // [nslot], indexed by slot - s0
  for (int i = threadIdx.x; i < nslot; i += blockDim.x) lexp[i] = -1;
  for (int64_t i = threadIdx.x; i < (int64_t)nch * E; i += blockDim.x) {
    const int64_t c = s0 / 64 + i % nch;
    if (c < nchunk) a.chunk_cnt[(i / nch) * nchunk + c] = 0;
  }
  __syncthreads();
  for (int64_t t = t0 + threadIdx.x / 16; t < t0 + tpb && t < a.T; t += blockDim.x / 16)
    topk_any(a, t, lexp, nullptr, s0);
  __syncthreads();
  const int nbits = 32 - __builtin_clz((unsigned)(E > 1 ? E - 1 : 1));
  for (int c = wave; c < nch; c += blockDim.x / 64) {
    const int64_t gc = s0 / 64 + c;
    if (gc >= nchunk) break;
    chunk_ranks(S - s0, c, lexp, a.chunk_cnt + gc, nchunk, a.rank + s0, nbits);
  }
  for (int i = threadIdx.x; i < nslot; i += blockDim.x)
    if (s0 + i < S) a.lexp[s0 + i] = lexp[i];
}

// (2) one wave per expert: exclusive scan of its chunk counts (in place, the
// chunk bases) and its total count.
__global__ __launch_bounds__(256) void route_chunk_scan_kernel(RouteArgs a) {
  const int lane = lane_id();
  const int e = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (e >= a.E_local) return;
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  int32_t* row = a.chunk_cnt + (int64_t)e * nchunk;
  int32_t carry = 0;
  for (int64_t c0 = 0; c0 < nchunk; c0 += 64) {
    const int64_t c = c0 + lane;
    const int32_t v = c < nchunk ? row[c] : 0;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (c < nchunk) row[c] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) a.counts[e] = carry;
}

// (3) scatter, many workgroups: each scans the counts into LDS offsets (the
// first also writes the offset and tile tables), then places its slots.
__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int E = a.E_local;
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  int32_t* counts = lds;             // [E]
  int32_t* offs = counts + E;        // [E + 1]
  int32_t* t1 = offs + E + 1;        // [E + 1]
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[e] = a.counts[e];
  __syncthreads();
  if (threadIdx.x < 64) wave_scan_experts(counts, E, a, blockIdx.x == 0, offs, t1);
  __syncthreads();
  for (int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; s < S; s += (int64_t)gridDim.x * blockDim.x) {
    const int e = a.lexp[s];
    if (e >= 0)
      place_slot(a, s, offs[e] + a.chunk_cnt[(int64_t)e * nchunk + s / 64] + a.rank[s], a.w[s], offs[e], t1[e]);
    else
      a.inv[s] = -1;
  }
}

namespace {
size_t small_lds_bytes(int64_t S, int64_t E) {
  const int64_t nchunk = (S + 63) / 64;
  return (size_t)(3 * S + nchunk * E + 3 * E + 2) * sizeof(int32_t);
}
int64_t gcd64(int64_t x, int64_t y) { return y ? gcd64(y, x % y) : x; }
}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int64_t S = a.T * (int64_t)a.top_k;
  if (S == 0) return hipSuccess;
  const int64_t work = a.T * ((a.E_global + 15) / 16) * a.top_k;  // per-lane compare rounds
  const size_t lds = small_lds_bytes(S, a.E_local);
  if (lds <= kRouteFusedMaxLds && work <= 8192) {
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(512), lds, stream, a);
    return hipGetLastError();
  }
  // tokens per workgroup: a multiple of 64/gcd(64,k) (whole chunks), at least 16
  int64_t unit = 64 / gcd64(64, a.top_k);
  int64_t tpb = unit;
  while (tpb < 16) tpb += unit;
  const int64_t nblk = (a.T + tpb - 1) / tpb;
  hipLaunchKernelGGL(route_topk_chunk_kernel, dim3((unsigned)nblk), dim3(256),
                     (size_t)(tpb * a.top_k) * sizeof(int32_t), stream, a, (int)tpb);
  hipLaunchKernelGGL(route_chunk_scan_kernel, dim3((unsigned)((a.E_local + 3) / 4)), dim3(256), 0, stream, a);
  const int64_t nscatter = (S + 255) / 256 < 1024 ? (S + 255) / 256 : 1024;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)nscatter), dim3(256),
                     (size_t)(3 * a.E_local + 2) * sizeof(int32_t), stream, a);
  return hipGetLastError();
}

}  // namespace mxmoe
