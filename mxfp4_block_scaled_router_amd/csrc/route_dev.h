// Device side of the router and the token permutation, shared by the routing
// kernels and by the decode gate_up kernel, which routes a few tokens itself
// at its start.  Helpers have internal linkage (one copy per source file).
#pragma once

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

// Keys: orderable logit in the high word, inverted expert id in the low word,
// so a larger key is a larger logit or, on a tie, the lower id; every real key
// is nonzero and no two are equal.  Sorted descending within the lane
// (bitonic network over the lane's N keys).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&k)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ stride;
        if (l > i) {
          const bool desc = (i & size) == 0;
          const uint64_t x = k[i], y = k[l];
          const bool sw = desc ? (x < y) : (x > y);
          k[i] = sw ? y : x;
          k[l] = sw ? x : y;
        }
      }
}

// (0, the identity of an unsigned maximum, as the DPP source of lanes out of
// the row -- none here -- lets the compiler fold each step into one v_max_u32
// with a DPP operand)
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max_dpp_u32<kDppXor1>(v);
  v = max_dpp_u32<kDppXor2>(v);
  v = max_dpp_u32<kDppHalfMirror>(v);
  return max_dpp_u32<kDppMirror>(v);
}
// The row's largest 64-bit key from 32-bit maxima: the largest high word,
// then the largest low word among the lanes holding it (the same key as a
// 64-bit maximum, in single-instruction DPP steps).
__device__ __forceinline__ uint64_t row16_max_key32(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t bh = row16_max_u32(hi);
  const uint32_t bl = row16_max_u32(hi == bh ? lo : 0u);
  return ((uint64_t)bh << 32) | bl;
}

// Top-k of token t by the 16-lane row of this lane.  lexp_out[s - slot_base]
// receives the local expert (or -1) of each of the token's k slots s; with
// write_global the ids and weights also go to a.ids and a.w; tmask (LDS, may
// be null) gets bit t set in the entry of each local expert picked.
// Each lane holds logits r, r + 16, ... as sorted keys; a round takes the
// row's largest head (16-lane butterfly) and the one lane that holds it pops.
template <int VPL>
__device__ void topk_row(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base,
                         bool write_global, uint32_t* tmask = nullptr) {
  const int r = lane_id() & 15;
  const int E = a.E_global, k = a.picks;
  const float* row = a.logits + t * (int64_t)E;
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = r + 16 * i;
    const bool in = e < E;
    const float v = in ? row[e] : 0.0f;
    key[i] = in ? ((uint64_t)orderable(v) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  sort_desc<VPL>(key);
  uint64_t p0 = 0, p1 = 0, mx = 0;  // picks r and r + 16, first pick
  for (int j = 0; j < k; ++j) {
    const uint64_t best = row16_max_key32(key[0]);
    const bool pop = key[0] == best;
#pragma unroll
    for (int i = 0; i + 1 < VPL; ++i) key[i] = pop ? key[i + 1] : key[i];
    key[VPL - 1] = pop ? 0ull : key[VPL - 1];
    if (j == 0) mx = best;
    if (j == r) p0 = best;
    if (j == r + 16) p1 = best;
  }
  const uint32_t maxhi = (uint32_t)(mx >> 32);
  const uint32_t p0hi = (uint32_t)(p0 >> 32), p0lo = (uint32_t)p0;
  const uint32_t p1hi = (uint32_t)(p1 >> 32), p1lo = (uint32_t)p1;
  const double m = (double)from_orderable(maxhi);
  const bool has0 = r < k, has1 = r + 16 < k;
  const double e0 = has0 ? exp((double)from_orderable(p0hi) - m) : 0.0;
  const double e1 = has1 ? exp((double)from_orderable(p1hi) - m) : 0.0;
  const double sum = row16_sum_f64(e0 + e1);
  const int64_t s0 = t * a.top_k;  // slots per token (picks + shared)
  if (has0) {
    int id = (int)(0xFFFFFFFFu - p0lo);
    const float w = (float)(e0 / sum);
    if (write_global) {
      a.ids[s0 + r] = id;
      a.w[s0 + r] = w;
    }
    if (w_out) w_out[s0 + r - slot_base] = w;
    int le = id - a.first_local;
    lexp_out[s0 + r - slot_base] = (le >= 0 && le < a.E_route) ? le : -1;
    if (tmask && le >= 0 && le < a.E_route) atomicOr(&tmask[le], 1u << (uint32_t)t);
  }
  if (has1) {
    int id = (int)(0xFFFFFFFFu - p1lo);
    const float w = (float)(e1 / sum);
    if (write_global) {
      a.ids[s0 + r + 16] = id;
      a.w[s0 + r + 16] = w;
    }
    if (w_out) w_out[s0 + r + 16 - slot_base] = w;
    int le = id - a.first_local;
    lexp_out[s0 + r + 16 - slot_base] = (le >= 0 && le < a.E_route) ? le : -1;
    if (tmask && le >= 0 && le < a.E_route) atomicOr(&tmask[le], 1u << (uint32_t)t);
  }
  // shared expert: the slot after the picks, table expert E_route, weight 1
  if (a.top_k > k && r == 0) {
    if (write_global) {
      a.ids[s0 + k] = E;
      a.w[s0 + k] = 1.0f;
    }
    if (w_out) w_out[s0 + k - slot_base] = 1.0f;
    lexp_out[s0 + k - slot_base] = a.E_route;
    if (tmask) atomicOr(&tmask[a.E_route], 1u << (uint32_t)t);
  }
}

// Whole-wave reductions: the 16-lane row reduction, then the four row results
// combined in scalar registers (wave-uniform results).  Every lane active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint64_t wave_max_key32(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t bh = wave_max_u32(hi);
  const uint32_t bl = wave_max_u32(hi == bh ? lo : 0u);
  return ((uint64_t)bh << 32) | bl;
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l), hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row16_sum_f64(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Top-k of token t by a whole wave, lane l holding logits l, l + 64, ...: with
// many experts the per-lane sort and the per-round shifts are four times
// shorter than with one 16-lane row per token.  Same keys, same picks and the
// same fp64 weights as topk_row (the fp64 sum is taken in another order).
// Every lane of the wave must call it for the same t.
template <int VPL>
__device__ void topk_wave(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base,
                          bool write_global) {
  const int l = lane_id();
  const int E = a.E_global, k = a.picks;
  const float* row = a.logits + t * (int64_t)E;
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = l + 64 * i;
    const bool in = e < E;
    const float v = in ? row[e] : 0.0f;
    key[i] = in ? ((uint64_t)orderable(v) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  sort_desc<VPL>(key);
  uint64_t p = 0, mx = 0;  // pick l, first pick
  for (int j = 0; j < k; ++j) {
    const uint64_t best = wave_max_key32(key[0]);
    const bool pop = key[0] == best;
#pragma unroll
    for (int i = 0; i + 1 < VPL; ++i) key[i] = pop ? key[i + 1] : key[i];
    key[VPL - 1] = pop ? 0ull : key[VPL - 1];
    if (j == 0) mx = best;
    if (j == l) p = best;
  }
  const double m = (double)from_orderable((uint32_t)(mx >> 32));
  const bool has = l < k;
  const double e0 = has ? exp((double)from_orderable((uint32_t)(p >> 32)) - m) : 0.0;
  const double sum = wave_sum_f64(e0);
  const int64_t s0 = t * a.top_k;  // slots per token (picks + shared)
  if (has) {
    const int id = (int)(0xFFFFFFFFu - (uint32_t)p);
    const float w = (float)(e0 / sum);
    if (write_global) {
      a.ids[s0 + l] = id;
      a.w[s0 + l] = w;
    }
    if (w_out) w_out[s0 + l - slot_base] = w;
    const int le = id - a.first_local;
    lexp_out[s0 + l - slot_base] = (le >= 0 && le < a.E_route) ? le : -1;
  }
  // shared expert: the slot after the picks, table expert E_route, weight 1
  if (a.top_k > k && l == 0) {
    if (write_global) {
      a.ids[s0 + k] = E;
      a.w[s0 + k] = 1.0f;
    }
    if (w_out) w_out[s0 + k - slot_base] = 1.0f;
    lexp_out[s0 + k - slot_base] = a.E_route;
  }
}
__device__ void topk_wave_any(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base,
                              bool write_global = true) {
  const int vpl = (a.E_global + 63) / 64;
  if (vpl <= 1) topk_wave<1>(a, t, lexp_out, w_out, slot_base, write_global);
  else if (vpl <= 2) topk_wave<2>(a, t, lexp_out, w_out, slot_base, write_global);
  else if (vpl <= 4) topk_wave<4>(a, t, lexp_out, w_out, slot_base, write_global);
  else topk_wave<8>(a, t, lexp_out, w_out, slot_base, write_global);
}

// MAXVPL: largest logits-per-lane variant compiled in (E_global <= 16 MAXVPL)
template <int MAXVPL = 32>
__device__ void topk_any(const RouteArgs& a, int64_t t, int32_t* lexp_out, float* w_out, int64_t slot_base,
                         bool write_global = true, uint32_t* tmask = nullptr) {
  const int vpl = (a.E_global + 15) / 16;
  if (vpl <= 1) topk_row<1>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
  else if (vpl <= 2) topk_row<2>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
  else if (MAXVPL <= 4 || vpl <= 4) topk_row<4>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
  else if (MAXVPL <= 8 || vpl <= 8) topk_row<8>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
  else if (MAXVPL <= 16 || vpl <= 16) topk_row<16>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
  else topk_row<32>(a, t, lexp_out, w_out, slot_base, write_global, tmask);
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

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each 16-lane
// row (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read 0), then
// lane 15 of rows 0 and 2 added into rows 1 and 3 (row_bcast:15) and lane 31
// into rows 2 and 3 (row_bcast:31); rows masked off keep adding 0.
__device__ __forceinline__ int32_t wave_incl_sum(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}

// Whether table expert e is kept in bf16 (its rows get no MXFP4 tiles).
__device__ __forceinline__ bool bf16_expert(const RouteArgs& a, int e) { return a.xmap && a.xmap[e] >= 0; }

// Exclusive scan of the per-expert counts v[0..n) by one wave: expert offsets
// and, for the two token-tile heights mt1/mt2, tile offsets (prefix of
// ceil(v/mt), 0 for an expert kept in bf16) into offs_lds[0..n] and
// t1_lds[0..n] (entry n = total).  With write_global it also writes a.offsets,
// a.tile_off1/2 and the flat tile tables tiles1/tiles2: tile i -> {expert,
// rows, first sorted position, 0}.  tiles_lds (may be null) receives the mt1
// tile table.
__device__ void wave_scan_experts(const int32_t* v, int n, const RouteArgs& a, bool write_global,
                                  int32_t* offs_lds, int32_t* t1_lds, int4* tiles_lds = nullptr) {
  const int lane = lane_id();
  const int mt1 = a.mt1, mt2 = a.mt2;
  if (n <= 64 && ((mt1 & (mt1 - 1)) | (mt2 & (mt2 - 1))) == 0) {
    // one expert per lane, tile counts by shifts (power-of-two tile heights)
    const int sh1 = __builtin_ctz((unsigned)mt1), sh2 = __builtin_ctz((unsigned)mt2);
    const bool in = lane < n;
    const int32_t c = in ? v[lane] : 0;
    const int32_t ct = in && !bf16_expert(a, lane) ? c : 0;  // rows that get tiles
    const int32_t n1 = (ct + mt1 - 1) >> sh1, n2 = (ct + mt2 - 1) >> sh2;
    const int32_t i0 = wave_incl_sum(c), i1 = wave_incl_sum(n1);
    const int32_t i2 = mt2 == mt1 ? i1 : wave_incl_sum(n2);
    const int32_t r0 = i0 - c, r1 = i1 - n1, r2 = i2 - n2;
    if (in) {
      offs_lds[lane] = r0;
      t1_lds[lane] = r1;
      if (tiles_lds)
        for (int32_t j = 0; j < n1; ++j)
          tiles_lds[r1 + j] = make_int4(lane, min(ct - (j << sh1), mt1), r0 + (j << sh1), 0);
      if (write_global) {
        a.offsets[lane] = r0;
        a.tile_off1[lane] = r1;
        a.tile_off2[lane] = r2;
        for (int32_t j = 0; j < n1; ++j)
          a.tiles1[r1 + j] = make_int4(lane, min(ct - (j << sh1), mt1), r0 + (j << sh1), 0);
        for (int32_t j = 0; j < n2; ++j)
          a.tiles2[r2 + j] = make_int4(lane, min(ct - (j << sh2), mt2), r0 + (j << sh2), 0);
      }
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
    return;
  }
  const int per = (n + 63) / 64;
  const int b = lane * per;
  int32_t s0 = 0, s1 = 0, s2 = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      int32_t c = v[b + i];
      const int32_t ct = bf16_expert(a, b + i) ? 0 : c;  // rows that get tiles
      s0 += c;
      s1 += (ct + mt1 - 1) / mt1;
      s2 += (ct + mt2 - 1) / mt2;
    }
  // inclusive wave prefix of the lane totals
  const int32_t i0 = wave_incl_sum(s0), i1 = wave_incl_sum(s1), i2 = wave_incl_sum(s2);
  int32_t r0 = i0 - s0, r1 = i1 - s1, r2 = i2 - s2;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int e = b + i;
      const int32_t c = v[e];
      const int32_t ct = bf16_expert(a, e) ? 0 : c;
      offs_lds[e] = r0;
      t1_lds[e] = r1;
      if (tiles_lds)
        for (int32_t m0 = 0, j = 0; m0 < ct; m0 += mt1, ++j)
          tiles_lds[r1 + j] = make_int4(e, ct - m0 < mt1 ? ct - m0 : mt1, r0 + m0, 0);
      if (write_global) {
        a.offsets[e] = r0;
        a.tile_off1[e] = r1;
        a.tile_off2[e] = r2;
        for (int32_t m0 = 0, j = 0; m0 < ct; m0 += mt1, ++j)
          a.tiles1[r1 + j] = make_int4(e, ct - m0 < mt1 ? ct - m0 : mt1, r0 + m0, 0);
        for (int32_t m0 = 0, j = 0; m0 < ct; m0 += mt2, ++j)
          a.tiles2[r2 + j] = make_int4(e, ct - m0 < mt2 ? ct - m0 : mt2, r0 + m0, 0);
      }
      r0 += c;
      r1 += (ct + mt1 - 1) / mt1;
      r2 += (ct + mt2 - 1) / mt2;
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
// (token and router weight w of pos) and -- for the K-split kernels' tiles
// of mt1 (16 or 32) rows -- the token of that tile row.  e, off_e, tile_e:
// the slot's expert, its offset and first mt1-row tile (an expert kept in
// bf16 has no tiles).
__device__ __forceinline__ void place_slot(const RouteArgs& a, int64_t s, int32_t pos, float w, int e,
                                           int32_t off_e, int32_t tile_e) {
  const int32_t t = (int32_t)(s / a.top_k);
  a.sorted[pos] = (int32_t)s;
  a.inv[s] = pos;
  a.pos_tok[pos] = t;
  a.pos_w[pos] = w;
  if (a.tile_tok && !bf16_expert(a, e)) {
    const int32_t rel = pos - off_e;
    a.tile_tok[(int64_t)(tile_e + rel / a.mt1) * a.mt1 + rel % a.mt1] = t;
  }
}

// LDS of route_block in 32-bit words: the mt1 tile table (int4 entries, first,
// so it stays 16-byte aligned), then per slot expert / rank / weight, the
// per-position token, chunk counts, counts and the two offset arrays.
__host__ __device__ constexpr int64_t route_block_words(int64_t S, int64_t E, int64_t tile_bound) {
  return 4 * tile_bound + 4 * S + ((S + 63) / 64) * E + 3 * E + 2;
}

struct RouteLds {
  int4* tiles;     // [tile bound]  mt1 tiles {expert, rows, first sorted position, 0}
  int32_t* lexp;   // [S]
  int32_t* rank;   // [S]
  float* wl;       // [S]
  int32_t* ptok;   // [S]  token of each sorted position
  int32_t* cnt;    // [nchunk][E]
  int32_t* counts; // [E]
  int32_t* offs;   // [E + 1]
  int32_t* t1;     // [E + 1]  mt1 tile offsets; t1[E] = number of tiles
};

// tile_bound 0: no LDS tile table (tiles is null and nothing is written there)
__device__ __forceinline__ RouteLds route_lds(int32_t* base, int64_t S, int64_t E, int64_t tile_bound) {
  RouteLds L;
  L.tiles = tile_bound > 0 ? reinterpret_cast<int4*>(base) : nullptr;
  L.lexp = base + 4 * tile_bound;
  L.rank = L.lexp + S;
  L.wl = reinterpret_cast<float*>(L.rank + S);
  L.ptok = reinterpret_cast<int32_t*>(L.wl + S);
  L.cnt = L.ptok + S;
  L.counts = L.cnt + ((S + 63) / 64) * E;
  L.offs = L.counts + E;
  L.t1 = L.offs + E + 1;
  return L;
}

// Workgroup barrier for LDS traffic only: a release fence before and an
// acquire fence after the barrier, both limited to workgroup scope and the
// LDS address space, so the compiler keeps LDS accesses on their side of it
// and the hardware waits for this wave's LDS operations (lgkmcnt(0)) but not
// for its vector-memory loads, which may stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The whole routing of a.T tokens by one workgroup (any number of waves),
// everything after the logits kept in LDS: slot experts, weights and ranks,
// chunk counts, counts, expert and tile offsets, the mt1 tile table and the
// token of every sorted position.  With write_global the workgroup also writes
// every global routing table (ids, w, counts, offsets, tile tables, sorted,
// inv, pos_tok, pos_w, tile_tok).  Ends with the LDS results visible to the
// whole workgroup.  MAXVPL: as in topk_any.  The barriers after the top-k
// wait only for LDS traffic (nothing here reads global memory written inside
// the routing), so the global table stores stay in flight across them.
// Position of the n-th set bit of m (n < popcount(m)): a five-step binary
// search on popcounts, the same instructions on every lane.
__device__ __forceinline__ int nth_set_bit32(uint32_t m, int n) {
  int pos = 0;
#pragma unroll
  for (int sh = 16; sh >= 1; sh >>= 1) {
    const uint32_t lo = m & ((1u << sh) - 1u);
    const int c = __builtin_popcount(lo);
    const bool up = n >= c;
    n = up ? n - c : n;
    m = up ? m >> sh : lo;
    pos = up ? pos + sh : pos;
  }
  return pos;
}

// Whether route_block_masks applies: at most 32 tokens (a token mask per
// expert fits 32 bits), at most 64 local experts (one lane each), no experts
// kept in bf16.
__device__ __forceinline__ bool masks_route_ok(const RouteArgs& a) {
  return a.T <= 32 && a.E_local <= 64 && !a.xmap && ((a.mt1 & (a.mt1 - 1)) | (a.mt2 & (a.mt2 - 1))) == 0;
}

// The routing of route_block for few tokens, from a token mask per local
// expert instead of chunk ranks: a token picks an expert at most once, so the
// expert's rows in slot order are its tokens in increasing order, a slot's rank
// is the popcount of the mask below its token, and counts, offsets and tile
// offsets follow from one wave's popcounts and prefix sums (power-of-two tile
// heights).  Fills L.offs,
// L.t1, L.counts, L.tiles and tmask[E_local] (LDS; the token of row r of an
// expert's tile j is bit 16 j + r of its mask, nth_set_bit32); no L.ptok.  With
// write_global the workgroup also writes every global routing table, as
// route_block does.  Ends with the LDS results visible to the workgroup.
template <int MAXVPL = 32>
__device__ void route_block_masks(const RouteArgs& a, const RouteLds& L, uint32_t* tmask, bool write_global) {
  const int nwaves = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = lane_id();
  const int64_t S = a.T * (int64_t)a.top_k;
  const int E = a.E_local, k = a.top_k;
  // the masks are zero before any pick is ORed into them
  for (int e = threadIdx.x; e < E; e += blockDim.x) tmask[e] = 0u;
  lds_barrier();
  for (int64_t t = wave * 4 + (lane >> 4); t < a.T; t += nwaves * 4)
    topk_any<MAXVPL>(a, t, L.lexp, L.wl, 0, write_global, tmask);
  lds_barrier();
  if (wave == 0) {
    const int mt1 = a.mt1, mt2 = a.mt2;
    const int sh1 = __builtin_ctz((unsigned)mt1), sh2 = __builtin_ctz((unsigned)mt2);
    const bool in = lane < E;
    const uint32_t m = in ? tmask[lane] : 0u;
    const int32_t c = __builtin_popcount(m);
    const int32_t n1 = (c + mt1 - 1) >> sh1, n2 = (c + mt2 - 1) >> sh2;
    const int32_t i0 = wave_incl_sum(c), i1 = wave_incl_sum(n1);
    const int32_t i2 = mt2 == mt1 ? i1 : wave_incl_sum(n2);
    const int32_t p0 = i0 - c, r1 = i1 - n1, r2 = i2 - n2;
    if (in) {
      L.counts[lane] = c;
      L.offs[lane] = p0;
      L.t1[lane] = r1;
      for (int32_t j = 0; j < n1; ++j)
        L.tiles[r1 + j] = make_int4(lane, min(c - (j << sh1), mt1), p0 + (j << sh1), 0);
      if (write_global) {
        a.counts[lane] = c;
        a.offsets[lane] = p0;
        a.tile_off1[lane] = r1;
        a.tile_off2[lane] = r2;
        for (int32_t j = 0; j < n1; ++j)
          a.tiles1[r1 + j] = make_int4(lane, min(c - (j << sh1), mt1), p0 + (j << sh1), 0);
        for (int32_t j = 0; j < n2; ++j)
          a.tiles2[r2 + j] = make_int4(lane, min(c - (j << sh2), mt2), p0 + (j << sh2), 0);
      }
    }
    if (lane == 63) {
      L.offs[E] = i0;
      L.t1[E] = i1;
      if (write_global) {
        a.offsets[E] = i0;
        a.tile_off1[E] = i1;
        a.tile_off2[E] = i2;
      }
    }
  }
  lds_barrier();
  if (write_global) {
    // the permutation and the per-position tables: slot s of token t on
    // expert e sits at offs[e] + popcount(mask_e below t)
    for (int64_t s = threadIdx.x; s < S; s += blockDim.x) {
      const int e = L.lexp[s];
      if (e >= 0) {
        const int t = (int)(s / k);
        const int32_t pos = L.offs[e] + __builtin_popcount(tmask[e] & ((1u << t) - 1u));
        place_slot(a, s, pos, L.wl[s], e, L.offs[e], L.t1[e]);
      } else {
        a.inv[s] = -1;
      }
    }
  }
}

template <int MAXVPL = 32>
__device__ void route_block(const RouteArgs& a, const RouteLds& L, bool write_global) {
  const int nwaves = blockDim.x / 64;
  const int wave = threadIdx.x / 64, lane = lane_id();
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  const int E = a.E_local;
  for (int64_t i = threadIdx.x; i < nchunk * E; i += blockDim.x) L.cnt[i] = 0;
  for (int64_t t = wave * 4 + (lane >> 4); t < a.T; t += nwaves * 4)
    topk_any<MAXVPL>(a, t, L.lexp, L.wl, 0, write_global);
  __syncthreads();
  const int nbits = 32 - __builtin_clz((unsigned)(E > 1 ? E - 1 : 1));
  for (int64_t c = wave; c < nchunk; c += nwaves) chunk_ranks(S, c, L.lexp, L.cnt + c * E, 1, L.rank, nbits);
  lds_barrier();
  // per expert: running sum over chunks -> chunk bases; totals -> counts
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int64_t c = 0; c < nchunk; ++c) {
      int32_t v = L.cnt[c * E + e];
      L.cnt[c * E + e] = run;
      run += v;
    }
    L.counts[e] = run;
    if (write_global) a.counts[e] = run;
  }
  lds_barrier();
  if (wave == 0) wave_scan_experts(L.counts, E, a, write_global, L.offs, L.t1, L.tiles);
  lds_barrier();
  for (int64_t s = threadIdx.x; s < S; s += blockDim.x) {
    const int e = L.lexp[s];
    if (e >= 0) {
      const int32_t pos = L.offs[e] + L.cnt[(s / 64) * E + e] + L.rank[s];
      L.ptok[pos] = (int32_t)(s / a.top_k);
      if (write_global) place_slot(a, s, pos, L.wl[s], e, L.offs[e], L.t1[e]);
    } else if (write_global) {
      a.inv[s] = -1;
    }
  }
  lds_barrier();
}

}  // namespace


}  // namespace mxmoe
