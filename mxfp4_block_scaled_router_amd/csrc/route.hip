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
#include <stdlib.h>

#include "route_dev.h"

namespace mxmoe {

// ---------------------------------------------------------------- kernels

// Whole routing in one workgroup of 512 threads, for small T*k*E (decode).
__global__ __launch_bounds__(512) void route_small_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int64_t S = a.T * (int64_t)a.top_k;
  route_block(a, route_lds(lds, S, a.E_local, 0), true);
}

// ---- routing for larger T*k*E, in three kernels
// (1) top-k and chunk ranks: a workgroup takes `tpb` tokens, tpb*k a multiple
// of 64, so its slots are whole chunks; 256 threads (16 rows of 16 lanes, one
// token per row) or (wave_tok) one wave per token (topk_wave).  Chunk counts
// are stored expert-major, chunk_cnt[e][chunk].
__global__ __launch_bounds__(1024) void route_topk_chunk_kernel(RouteArgs a, int tpb, int wave_tok) {
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
  if (wave_tok) {
    for (int64_t t = t0 + wave; t < t0 + tpb && t < a.T; t += blockDim.x / 64)
      topk_wave_any(a, t, lexp, nullptr, s0);
  } else {
    for (int64_t t = t0 + threadIdx.x / 16; t < t0 + tpb && t < a.T; t += blockDim.x / 16)
      topk_any(a, t, lexp, nullptr, s0);
  }
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
      place_slot(a, s, offs[e] + a.chunk_cnt[(int64_t)e * nchunk + s / 64] + a.rank[s], a.w[s], e, offs[e],
                 t1[e]);
    else
      a.inv[s] = -1;
  }
}

// (2 + 3) in one launch when the chunk table is small: every workgroup scans
// the expert-major chunk counts into chunk bases in its own LDS (one wave per
// expert), the first also writes counts, offsets and the tile tables, then
// each places its slots.  The slot loads go out before the scan.
__global__ __launch_bounds__(1024) void route_scan_scatter_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int E = a.E_local;
  const int64_t S = a.T * (int64_t)a.top_k;
  const int nchunk = (int)((S + 63) / 64);
  int32_t* cnt = lds;                           // [E][nchunk]: counts, then bases
  int32_t* counts = cnt + (int64_t)E * nchunk;  // [E]
  int32_t* offs = counts + E;                   // [E + 1]
  int32_t* t1 = offs + E + 1;                   // [E + 1]
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one slot per thread
  const bool live = s < S;
  const int e_s = live ? a.lexp[s] : -1;
  const int32_t r_s = live ? a.rank[s] : 0;
  const float w_s = live ? a.w[s] : 0.f;
  for (int i = threadIdx.x; i < E * nchunk; i += blockDim.x) cnt[i] = a.chunk_cnt[i];
  __syncthreads();
  const int lane = lane_id(), nw = blockDim.x / 64;
  for (int e = threadIdx.x / 64; e < E; e += nw) {
    int32_t* row = cnt + (int64_t)e * nchunk;
    int32_t carry = 0;
    for (int c0 = 0; c0 < nchunk; c0 += 64) {
      const int c = c0 + lane;
      const int32_t v = c < nchunk ? row[c] : 0;
      const int32_t incl = wave_incl_sum(v);
      if (c < nchunk) row[c] = carry + incl - v;
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) {
      counts[e] = carry;
      if (blockIdx.x == 0) a.counts[e] = carry;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) wave_scan_experts(counts, E, a, blockIdx.x == 0, offs, t1);
  __syncthreads();
  if (live) {
    if (e_s >= 0)
      place_slot(a, s, offs[e_s] + cnt[(int64_t)e_s * nchunk + s / 64] + r_s, w_s, e_s, offs[e_s], t1[e_s]);
    else
      a.inv[s] = -1;
  }
}

namespace {
// chunk tables up to this many entries take route_scan_scatter_kernel
constexpr int64_t kScanScatterMaxEntries = 8192;
constexpr int64_t kScanScatterMaxSlots = 16 * 1024;
size_t small_lds_bytes(int64_t S, int64_t E) { return (size_t)route_block_words(S, E, 0) * sizeof(int32_t); }
int64_t gcd64(int64_t x, int64_t y) { return y ? gcd64(y, x % y) : x; }
}  // namespace

bool route_fusable(const RouteArgs& a) {
  const int64_t S = a.T * (int64_t)a.top_k;
  if (S <= 0 || a.T > 32 || a.mt1 != 16 || a.E_local < 1 || a.E_global > 16 * kFusedRouteMaxVpl) return false;
  const int64_t bound = (a.E_local < S ? a.E_local : S) + S / 16;
  return (size_t)route_block_words(S, a.E_local, bound) * sizeof(int32_t) <= 16 * 1024;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int64_t S = a.T * (int64_t)a.top_k;
  if (S == 0) return hipSuccess;
  const int64_t work = a.T * ((a.E_global + 15) / 16) * a.picks;  // per-lane compare rounds
  const size_t lds = small_lds_bytes(S, a.E_local);
  // one workgroup wins up to ~48 tokens of 64 experts, top-8 (measured)
  int64_t small_work = 2048;
  if (const char* env = tuning_env("MXFP4_MOE_ROUTE_SMALL_WORK")) small_work = atoll(env);  // tuning builds only
  if (lds <= kRouteFusedMaxLds && work <= small_work) {
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(512), lds, stream, a);
    return hipGetLastError();
  }
  // more than 64 experts and few tokens: one wave per token (up to 16 waves), a
  // shorter chain per token; with many tokens (the launch fills the GPU) the
  // 16-lane rows, which take fewer instructions per token (measured: prefill
  // routing 31 us with rows, 35 us with waves; ep_share 20.4 -> 17.6 us)
  const int wave_tok = a.E_global > 64 && a.T <= 2048 ? 1 : 0;
  // tokens per workgroup: a multiple of 64/gcd(64,k) (whole chunks), at least
  // 16 for the 16-lane rows (one workgroup of 16 rows) and 8 with a wave per token
  int64_t unit = 64 / gcd64(64, a.top_k);
  int64_t tpb = unit;
  while (tpb < (wave_tok ? 8 : 16)) tpb += unit;
  const int64_t nblk = (a.T + tpb - 1) / tpb;
  const int64_t threads = wave_tok ? (tpb < 16 ? tpb : 16) * 64 : 256;
  hipLaunchKernelGGL(route_topk_chunk_kernel, dim3((unsigned)nblk), dim3((unsigned)(threads < 256 ? 256 : threads)),
                     (size_t)(tpb * a.top_k) * sizeof(int32_t), stream, a, (int)tpb, wave_tok);
  const int64_t entries = ((S + 63) / 64) * a.E_local;
  if (entries <= kScanScatterMaxEntries && S <= kScanScatterMaxSlots) {
    hipLaunchKernelGGL(route_scan_scatter_kernel, dim3((unsigned)((S + 1023) / 1024)), dim3(1024),
                       (size_t)(entries + 3 * a.E_local + 2) * sizeof(int32_t), stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_chunk_scan_kernel, dim3((unsigned)((a.E_local + 3) / 4)), dim3(256), 0, stream, a);
  const int64_t nscatter = (S + 255) / 256 < 1024 ? (S + 255) / 256 : 1024;
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)nscatter), dim3(256),
                     (size_t)(3 * a.E_local + 2) * sizeof(int32_t), stream, a);
  return hipGetLastError();
}

}  // namespace mxmoe
