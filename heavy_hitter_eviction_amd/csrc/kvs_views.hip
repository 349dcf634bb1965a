// Side-car views over the per-block table (Context views at marginal cost,
// section 3, "Pure side-car vs. materialized": a view filters the score table,
// and one threshold serves both to answer queries and to decide which
// fine-grained history is worth storing; section 7, SOTA grounding,
// per-system reductions: Scissorhands counts the turns a token's attention
// passes a threshold).
//
// kvs_counters: per block, the Scissorhands count of turns whose Attended
// exceeded hot_theta, and the number of consecutive turns the EMA has stayed
// below cold_theta; once that reaches cold_limit the block's trajectory ring
// is cleared (its fine-grained history dropped, Cumulative kept).
//
// kvs_filter: per sequence, the ascending ids of the existing, alive blocks
// whose score exceeds theta -- the set of spans a threshold view answers with.

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

__global__ __launch_bounds__(256) void kvs_counters(CounterArgs a) {
  const size_t n = (size_t)a.B * a.nbmax;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
    if (a.hot_count) a.hot_count[x] += a.attended[x] > a.hot_theta ? 1 : 0;
    if (a.cold_turns) {
      const int c = a.ema[x] < a.cold_theta ? a.cold_turns[x] + 1 : 0;
      a.cold_turns[x] = c;
      if (a.traj && a.cold_limit > 0 && c >= a.cold_limit) {
        const size_t b = x / a.nbmax, blk = x - b * a.nbmax;
        for (int s = 0; s < a.traj_cap; ++s) a.traj[(b * a.traj_cap + s) * a.nbmax + blk] = 0.0f;
      }
    }
  }
}

hipError_t launch_counters(const CounterArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.B * a.nbmax;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(kvs_counters, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

constexpr int kFilterThreads = 1024;

// One workgroup per sequence; chunks of 1024 blocks are compacted in order
// with wave ballots and a prefix over the 16 wave counts.
__global__ __launch_bounds__(kFilterThreads) void kvs_filter(FilterArgs a) {
  __shared__ int wcount[kFilterThreads / 64];
  __shared__ int s_base;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = a.cur_pos[b];
  const int nexist = i < 0 ? 0 : min(i / kTile + 1, a.nbmax);
  const float* score = a.score + (size_t)b * a.nbmax;
  const uint32_t* alive = a.alive ? a.alive + (size_t)b * a.kwords : nullptr;
  int32_t* ids = a.ids + (size_t)b * a.ids_stride;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < nexist; c0 += kFilterThreads) {
    const int blk = c0 + tid;
    bool take = false;
    if (blk < nexist) {
      take = score[blk] > a.theta;
      if (take && alive) take = (alive[blk >> 5] >> (blk & 31)) & 1u;
    }
    const uint64_t m = __ballot(take);
    if (lane == 0) wcount[wave] = __popcll(m);
    __syncthreads();
    int before = s_base;
    for (int w = 0; w < wave; ++w) before += wcount[w];
    const int pos = before + __popcll(m & ((1ull << lane) - 1ull));
    if (take && pos < a.ids_stride) ids[pos] = blk;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < kFilterThreads / 64; ++w) tot += wcount[w];
      s_base += tot;
    }
    __syncthreads();
  }
  if (tid == 0) a.n_ids[b] = s_base;
}

hipError_t launch_filter(const FilterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(kvs_filter, dim3(a.B), dim3(kFilterThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
