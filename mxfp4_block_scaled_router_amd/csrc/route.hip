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

constexpr int kMaxEPL = 16;  // logits per lane: E_global <= 1024

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Top-k of one token's logits by one wave.  Writes ids/w and the local expert
// of each slot (or -1) to lexp.
template <int EPL>
__device__ void topk_token(const float* __restrict__ logits, int64_t t, int E, int k, int first_local,
                           int E_local, int32_t* __restrict__ ids, float* __restrict__ w,
                           int32_t* __restrict__ lexp) {
  const int lane = lane_id();
  uint64_t key[EPL];
  float val[EPL];
  const float* row = logits + t * (int64_t)E;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = i * 64 + lane;
    float v = e < E ? row[e] : 0.0f;
    val[i] = v;
    key[i] = e < E ? (((uint64_t)orderable(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e)) : 0;
  }
  int my_id = -1;      // pick j held by lane j
  float my_logit = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    int id = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (i * 64 + lane == id) key[i] = 0;
    if (lane == j) my_id = id;
  }
  // gather the picked logits to lanes 0..k-1 (owner lane of id = id % 64, slot id / 64)
  {
    int src_lane = my_id >= 0 ? (my_id & 63) : 0;
    int src_slot = my_id >= 0 ? (my_id >> 6) : 0;
    float cand = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float v = __shfl(val[i], src_lane, 64);
      if (i == src_slot) cand = v;
    }
    my_logit = cand;
  }
  double m = __shfl((double)my_logit, 0, 64);  // pick 0 holds the largest logit
  double ex = (lane < k) ? exp((double)my_logit - m) : 0.0;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) sum += __shfl(ex, j, 64);
  if (lane < k) {
    int64_t s = t * k + lane;
    ids[s] = my_id;
    w[s] = (float)(ex / sum);
    int le = my_id - first_local;
    lexp[s] = (le >= 0 && le < E_local) ? le : -1;
  }
}

template <int EPL>
__device__ void topk_dispatch_body(const RouteArgs& a, int64_t t) {
  topk_token<EPL>(a.logits, t, a.E_global, a.top_k, a.first_local, a.E_local, a.ids, a.w, a.lexp);
}

__device__ void topk_any(const RouteArgs& a, int64_t t) {
  int epl = (a.E_global + 63) / 64;
  if (epl <= 1) topk_dispatch_body<1>(a, t);
  else if (epl <= 2) topk_dispatch_body<2>(a, t);
  else if (epl <= 4) topk_dispatch_body<4>(a, t);
  else if (epl <= 8) topk_dispatch_body<8>(a, t);
  else topk_dispatch_body<kMaxEPL>(a, t);
}

// Rank of each slot of chunk c among the chunk's slots with the same local
// expert, and the chunk's per-expert counts (cnt_row has E_local entries, zeroed
// beforehand; only experts present in the chunk are written).  One wave.
__device__ void chunk_ranks(const RouteArgs& a, int64_t c, int32_t* cnt_row, int32_t* __restrict__ rank) {
  const int lane = lane_id();
  const int64_t S = a.T * (int64_t)a.top_k;
  int64_t s = c * 64 + lane;
  int e = s < S ? a.lexp[s] : -1;
  uint64_t remaining = __ballot(e >= 0);
  int my_rank = 0;
  while (remaining) {
    int leader = __ffsll((unsigned long long)remaining) - 1;
    int le = __shfl(e, leader, 64);
    uint64_t mask = __ballot(e == le);
    if (e == le) my_rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == leader) cnt_row[le] = __popcll(mask);
    remaining &= ~mask;
  }
  if (s < S) rank[s] = my_rank;
}

// Exclusive scan over experts of v (one value per expert, E_local <= 1024) in a
// workgroup; returns through out[] (E_local + 1 entries, out[E_local] = total).
// Must be called by all threads of the workgroup.
__device__ void wg_exclusive_scan(const int32_t* v, int32_t* out, int n, int32_t* lds_tmp) {
  // simple: thread 0..n-1 copy, then a Hillis-Steele scan in LDS
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < n; i += nt) lds_tmp[i] = v[i];
  __syncthreads();
  for (int off = 1; off < n; off <<= 1) {
    int32_t add[4];
    int q = 0;
    for (int i = tid; i < n; i += nt) add[q++] = (i >= off) ? lds_tmp[i - off] : 0;
    __syncthreads();
    q = 0;
    for (int i = tid; i < n; i += nt) lds_tmp[i] += add[q++];
    __syncthreads();
  }
  for (int i = tid; i < n; i += nt) out[i + 1] = lds_tmp[i];
  if (tid == 0) out[0] = 0;
  __syncthreads();
}

// Per (chunk, expert) bases, counts, offsets and tile offsets.  One workgroup
// of 1024 threads (16 waves).  cnt[c][e] (global or LDS) holds chunk counts and
// is overwritten with the chunk's base within the expert.
__device__ void scan_chunks(const RouteArgs& a, int32_t* cnt, int64_t nchunk, int32_t* lds_wave_sum,
                            int32_t* lds_tmp, int32_t* lds_counts) {
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int nwaves = blockDim.x / 64;
  const int E = a.E_local;
  int64_t per = (nchunk + nwaves - 1) / nwaves;
  int64_t c0 = wave * per, c1 = c0 + per < nchunk ? c0 + per : nchunk;
  // pass 1: per-wave sums per expert (lane = expert, in strides of 64)
  for (int e0 = 0; e0 < E; e0 += 64) {
    int e = e0 + lane;
    int32_t sum = 0;
    if (e < E)
      for (int64_t c = c0; c < c1; ++c) sum += cnt[c * E + e];
    if (e < E) lds_wave_sum[wave * E + e] = sum;
  }
  __syncthreads();
  // exclusive scan over waves per expert; totals = counts
  for (int e = tid; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int w = 0; w < nwaves; ++w) {
      int32_t v = lds_wave_sum[w * E + e];
      lds_wave_sum[w * E + e] = run;
      run += v;
    }
    lds_counts[e] = run;
    a.counts[e] = run;
  }
  __syncthreads();
  // pass 2: chunk bases
  for (int e0 = 0; e0 < E; e0 += 64) {
    int e = e0 + lane;
    if (e < E) {
      int32_t run = lds_wave_sum[wave * E + e];
      for (int64_t c = c0; c < c1; ++c) {
        int32_t v = cnt[c * E + e];
        cnt[c * E + e] = run;
        run += v;
      }
    }
  }
  // offsets and tile offsets
  wg_exclusive_scan(lds_counts, a.offsets, E, lds_tmp);
  for (int t = 0; t < 2; ++t) {
    int mt = t == 0 ? a.mt1 : a.mt2;
    int32_t* dst = t == 0 ? a.tile_off1 : a.tile_off2;
    for (int e = tid; e < E; e += blockDim.x) lds_tmp[e + 1024] = (lds_counts[e] + mt - 1) / mt;
    __syncthreads();
    wg_exclusive_scan(lds_tmp + 1024, dst, E, lds_tmp);
  }
}

__device__ void scatter_slot(const RouteArgs& a, int64_t s, const int32_t* cnt, const int32_t* offsets) {
  int e = a.lexp[s];
  if (e >= 0) {
    int32_t pos = offsets[e] + cnt[(s / 64) * a.E_local + e] + a.rank[s];
    a.sorted[pos] = (int32_t)s;
    a.inv[s] = pos;
  } else {
    a.inv[s] = -1;
  }
}

}  // namespace

// ---------------------------------------------------------------- kernels

// Whole routing in one workgroup (small T*k): LDS holds the chunk counts.
__global__ __launch_bounds__(1024) void route_fused_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int nwaves = blockDim.x / 64;
  const int wave = threadIdx.x / 64;
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  int32_t* cnt = lds;                                  // [nchunk][E_local]
  int32_t* wave_sum = cnt + nchunk * a.E_local;        // [16][E_local]
  int32_t* counts = wave_sum + 16 * a.E_local;         // [E_local]
  int32_t* tmp = counts + a.E_local;                   // [2048]
  for (int64_t i = threadIdx.x; i < nchunk * a.E_local; i += blockDim.x) cnt[i] = 0;
  for (int64_t t = wave; t < a.T; t += nwaves) topk_any(a, t);
  __threadfence_block();
  __syncthreads();
  for (int64_t c = wave; c < nchunk; c += nwaves) chunk_ranks(a, c, cnt + c * a.E_local, a.rank);
  __threadfence_block();
  __syncthreads();
  scan_chunks(a, cnt, nchunk, wave_sum, tmp, counts);
  __syncthreads();
  for (int64_t s = threadIdx.x; s < S; s += blockDim.x) scatter_slot(a, s, cnt, a.offsets);
}

// Multi-kernel routing for large T*k.
__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a) {
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t n_cnt = ((S + 63) / 64) * a.E_local;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_cnt;
       i += (int64_t)gridDim.x * blockDim.x)
    a.chunk_cnt[i] = 0;
  int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (t < a.T) topk_any(a, t);
}

__global__ __launch_bounds__(256) void route_chunk_kernel(RouteArgs a) {
  const int64_t S = a.T * (int64_t)a.top_k;
  int64_t c = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (c * 64 < S) chunk_ranks(a, c, a.chunk_cnt + c * a.E_local, a.rank);
}

__global__ __launch_bounds__(1024) void route_scan_kernel(RouteArgs a) {
  extern __shared__ int32_t lds[];
  const int64_t S = a.T * (int64_t)a.top_k;
  const int64_t nchunk = (S + 63) / 64;
  int32_t* wave_sum = lds;                        // [16][E_local]
  int32_t* counts = wave_sum + 16 * a.E_local;    // [E_local]
  int32_t* tmp = counts + a.E_local;              // [2048]
  scan_chunks(a, a.chunk_cnt, nchunk, wave_sum, tmp, counts);
}

__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
  const int64_t S = a.T * (int64_t)a.top_k;
  int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) scatter_slot(a, s, a.chunk_cnt, a.offsets);
}

size_t route_fused_lds_bytes(int64_t S, int64_t E_local) {
  int64_t nchunk = (S + 63) / 64;
  return (size_t)(nchunk * E_local + 16 * E_local + E_local + 2048) * sizeof(int32_t);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const int64_t S = a.T * (int64_t)a.top_k;
  if (S == 0) return hipSuccess;
  size_t fused_lds = route_fused_lds_bytes(S, a.E_local);
  if (fused_lds <= kRouteFusedMaxLds) {
    hipLaunchKernelGGL(route_fused_kernel, dim3(1), dim3(1024), fused_lds, stream, a);
    return hipGetLastError();
  }
  const int64_t nchunk = (S + 63) / 64;
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(route_chunk_kernel, dim3((unsigned)((nchunk + 3) / 4)), dim3(256), 0, stream, a);
  size_t scan_lds = (size_t)(16 * a.E_local + a.E_local + 2048) * sizeof(int32_t);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), scan_lds, stream, a);
  hipLaunchKernelGGL(route_scatter_kernel, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxmoe
