// Block side-car update and heavy-hitter block selection.
//
// Side-car (Context views at marginal cost, section 2 Tier 1): per block,
// Attended (this turn), EMA, Cumulative and a bounded trajectory ring, O(1)
// per block per turn.
//
// Selection (Context Optimization, "H2O KV Cache Eviction"): sinks and recent
// tokens kept unconditionally; among the remaining alive blocks the
// highest-scoring ones survive, here at 16-token block granularity (Per-Head
// Attention as a Scoring Signal: the block is the unit that is kept). The
// top-k is an exact radix select on 64-bit keys (order-preserving score bits,
// then the complemented block index), so equal scores go to the lower index
// and every key is distinct.

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

__global__ __launch_bounds__(256) void kvs_sidecar(float* mass, float* att, float* ema, float* cum,
                                                    float* traj, int B, int nbmax, int traj_cap,
                                                    int slot, float alpha) {
  const size_t n = (size_t)B * nbmax;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
    const size_t b = x / nbmax, blk = x - b * nbmax;
    sidecar_block(mass, att, ema, cum, traj, x, (int)b, (int)blk, nbmax, traj_cap, slot, alpha, mass[x]);
  }
}

hipError_t launch_sidecar(float* mass, float* att, float* ema, float* cum, float* traj, int B,
                          int nbmax, int traj_cap, int64_t step, float alpha, hipStream_t st) {
  const size_t n = (size_t)B * nbmax;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kvs_sidecar, dim3((unsigned)blocks), dim3(256), 0, st, mass, att, ema, cum, traj,
                     B, nbmax, traj_cap, (int)(step % traj_cap), alpha);
  return hipGetLastError();
}

// Order-preserving map of a float to uint32 (-0 and +0 map alike).
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = f32_bits(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t select_key(float score, int blk) {
  return ((uint64_t)float_order(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)blk);
}

constexpr int kSelThreads = 1024;

// One workgroup per sequence.
__global__ __launch_bounds__(kSelThreads) void kvs_select(SelectArgs a) {
  extern __shared__ uint32_t alive_lds[];  // [kwords]: alive bits, staged so keep may alias alive
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint64_t s_prefix;
  __shared__ int s_remaining, s_ncand, s_base, s_done;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = a.cur_pos[b];
  const int nexist = min(i / kTile + 1, a.nbmax);
  const int rlo = max(0, i - a.recent + 1) / kTile;
  const int rhi = i / kTile;
  const int shi = a.sinks > 0 ? (min(a.sinks, i + 1) - 1) / kTile : -1;
  const float* score = a.score + (size_t)b * a.nbmax;
  const bool have_alive = a.alive != nullptr;
  if (have_alive)
    for (int w = tid; w < a.kwords; w += kSelThreads) alive_lds[w] = a.alive[(size_t)b * a.kwords + w];

  auto is_prot = [&](int blk) { return (blk >= rlo && blk <= rhi) || blk <= shi; };
  auto is_cand = [&](int blk) {
    if (blk >= nexist || is_prot(blk)) return false;
    return !have_alive || ((alive_lds[blk >> 5] >> (blk & 31)) & 1u);
  };

  // candidate count
  if (tid == 0) {
    s_ncand = 0;
    s_prefix = 0;
    s_done = 0;
  }
  __syncthreads();
  int cnt = 0;
  for (int blk = tid; blk < nexist; blk += kSelThreads) cnt += is_cand(blk) ? 1 : 0;
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (lane == 0) atomicAdd(&s_ncand, cnt);
  __syncthreads();
  const int ncand = s_ncand;
  const int k = min(a.budget, ncand);
  if (tid == 0) s_remaining = k;
  __syncthreads();

  // Radix select of the k-th largest key, 8 bits at a time from the top. When
  // every key of the chosen digit bin is taken, the lower bits do not matter
  // and the search stops (threshold = prefix with zero low bits).
  const bool take_all = (k == ncand);
  if (k > 0 && !take_all) {
    uint64_t mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int x = tid; x < 256; x += kSelThreads) hist[x] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix;
      for (int blk = tid; blk < nexist; blk += kSelThreads) {
        if (!is_cand(blk)) continue;
        const uint64_t key = select_key(score[blk], blk);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // suffix sums over bins (lane L owns bins 4L..4L+3), then locate the bin
        // holding the remaining-th largest key
        const int rem = s_remaining;
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        uint32_t suf = h0 + h1 + h2 + h3;  // inclusive suffix over lanes >= L after the scan
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_down(suf, off, 64);
          if (lane + off < 64) suf += o;
        }
        const uint32_t above = suf - (h0 + h1 + h2 + h3);  // keys in bins of higher lanes
        const bool here = above < (uint32_t)rem && suf >= (uint32_t)rem;
        if (here) {
          uint32_t acc = above;
          int d = 4 * lane + 3;
          const uint32_t hv[4] = {h0, h1, h2, h3};
          for (int q = 3; q >= 0; --q) {
            d = 4 * lane + q;
            if (acc + hv[q] >= (uint32_t)rem) break;
            acc += hv[q];
          }
          const int new_rem = rem - (int)acc;
          s_remaining = new_rem;
          s_prefix = prefix | ((uint64_t)d << shift);
          s_done = (hist[d] == (uint32_t)new_rem) ? 1 : 0;
        }
      }
      __syncthreads();
      mask |= (uint64_t)0xFF << shift;
      if (s_done) break;
    }
  }
  const uint64_t thresh = s_prefix;

  auto kept = [&](int blk) -> bool {
    if (blk >= nexist) return true;  // not written yet: never evicted
    if (is_prot(blk)) return true;
    if (!is_cand(blk) || k == 0) return false;
    if (take_all) return true;
    return select_key(score[blk], blk) >= thresh;
  };

  // keep mask words and ascending ids of kept existing blocks, 1024 blocks at a time
  if (tid == 0) s_base = 0;
  __syncthreads();
  int32_t* ids = a.sel_ids + (size_t)b * a.nbmax;
  uint32_t* keep = a.keep + (size_t)b * a.kwords;
  for (int c0 = 0; c0 < a.kwords * 32; c0 += kSelThreads) {
    const int blk = c0 + tid;
    const bool f = blk < a.nbmax && kept(blk);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
    const int w = blk >> 5;
    if ((lane & 31) == 0 && w < a.kwords) keep[w] = (uint32_t)(bal >> (lane & 32));
    const bool fe = f && blk < nexist;
    const uint64_t bale = __builtin_amdgcn_ballot_w64(fe);
    const int before = __builtin_popcountll(bale & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = (uint32_t)__builtin_popcountll(bale);
    __syncthreads();
    int off = s_base;
    for (int ww = 0; ww < wave; ++ww) off += (int)wsum[ww];
    if (fe) ids[off + before] = blk;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int ww = 0; ww < kSelThreads / 64; ++ww) t += (int)wsum[ww];
      s_base += t;
    }
    __syncthreads();
  }
  if (tid == 0) a.n_sel[b] = s_base;
}

// ---------------------------------------------------------------------------
// The same selection with a sequence's keys in registers: thread t holds the
// order bits of blocks t, t + 1024, ... (KPT of them, nbmax <= 1024 KPT), so
// the radix passes read no memory. In the first pass a wave's increments for
// its first lane's digit are added at once (the top digit is the score's
// sign and exponent bits, shared by most blocks, whose LDS atomics would
// otherwise serialise on one address); later digits are spread, and plain
// atomics are cheapest there. The kept ids are placed with one scan over
// (thread slice, wave) counts. With SC the side-car update of the sequence's
// blocks comes first, in the same arithmetic as kvs_sidecar, and the
// selection scores the updated array. Same keys, threshold and outputs as
// kvs_select.
// ---------------------------------------------------------------------------
constexpr int kSelRegMax = 16;  // keys per thread: sequences of up to 16384 blocks

template <int KPT, bool SC>
__global__ __launch_bounds__(kSelThreads) void kvs_select_reg(SelectArgs a) {
  extern __shared__ uint32_t alive_lds[];  // [kwords]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t offs[KPT * (kSelThreads / 64)];  // kept counts, then offsets, per (slice, wave)
  __shared__ uint64_t s_prefix;
  __shared__ int s_remaining, s_ncand, s_done, s_total;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = a.cur_pos[b];  // used after the first barrier: its wait comes with the scores'
  const bool have_alive = a.alive != nullptr;
  // alive words to LDS, once the scores' loads are issued (so neither waits
  // for the other)
  auto stage_alive = [&]() {
    if (have_alive)
      for (int w = tid; w < a.kwords; w += kSelThreads) alive_lds[w] = a.alive[(size_t)b * a.kwords + w];
  };
  if (tid == 0) {
    s_ncand = 0;
    s_prefix = 0;
    s_done = 0;
  }

  // order bits of this thread's blocks (after the side-car update with SC).
  // Every load is issued before any store: the compiler must assume the
  // arrays may overlap, so a store would hold back every later load.
  const size_t row = (size_t)b * a.nbmax;
  uint32_t ord[KPT];
  if constexpr (SC) {
    float A[KPT], E[KPT], C[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (kSelThreads * j >= a.nbmax) break;  // slices past the last block
      const size_t x = row + min(tid + kSelThreads * j, a.nbmax - 1);  // clamped: loads are unconditional
      A[j] = a.mass[x];
      E[j] = a.ema[x];
      C[j] = a.cum[x];
    }
    stage_alive();
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (kSelThreads * j >= a.nbmax) {
        ord[j] = 0;
        continue;
      }
      E[j] = a.alpha * A[j] + (1.0f - a.alpha) * E[j];
      C[j] = C[j] + A[j];
      ord[j] = float_order(a.score_src == 0 ? C[j] : (a.score_src == 1 ? E[j] : A[j]));
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int blk = tid + kSelThreads * j;
      if (kSelThreads * j >= a.nbmax) break;
      if (blk < a.nbmax) {
        const size_t x = row + blk;
        a.att[x] = A[j];
        a.ema[x] = E[j];
        a.cum[x] = C[j];
        if (a.traj) a.traj[((size_t)b * a.traj_cap + a.slot) * a.nbmax + blk] = A[j];
        a.mass[x] = 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      ord[j] = kSelThreads * j < a.nbmax ? float_order(a.score[row + min(tid + kSelThreads * j, a.nbmax - 1)]) : 0u;
    stage_alive();
  }
  __syncthreads();
  const int nexist = min(i / kTile + 1, a.nbmax);
  const int rlo = max(0, i - a.recent + 1) / kTile;
  const int rhi = i / kTile;
  const int shi = a.sinks > 0 ? (min(a.sinks, i + 1) - 1) / kTile : -1;

  auto is_prot = [&](int blk) { return (blk >= rlo && blk <= rhi) || blk <= shi; };
  auto is_cand = [&](int blk) {
    if (blk >= nexist || is_prot(blk)) return false;
    return !have_alive || ((alive_lds[blk >> 5] >> (blk & 31)) & 1u);
  };
  uint32_t cm = 0;  // candidate bit per slice
#pragma unroll
  for (int j = 0; j < KPT; ++j) cm |= is_cand(tid + kSelThreads * j) ? (1u << j) : 0u;
  int cnt = __builtin_popcount(cm);
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if (lane == 0) atomicAdd(&s_ncand, cnt);
  __syncthreads();
  const int ncand = s_ncand;
  const int k = min(a.budget, ncand);
  if (tid == 0) s_remaining = k;
  __syncthreads();
  auto key_of = [&](int j) -> uint64_t {
    return ((uint64_t)ord[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(tid + kSelThreads * j));
  };

  const bool take_all = (k == ncand);
  if (k > 0 && !take_all) {
    uint64_t mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (kSelThreads * j >= nexist) break;  // no candidates past the existing blocks
        const uint64_t key = key_of(j);
        bool v = ((cm >> j) & 1u) && (key & mask) == prefix;
        const uint32_t d = (uint32_t)(key >> shift) & 0xFFu;
        if (shift == 56) {
          // the top digit (sign and exponent bits) is shared by most keys:
          // the wave's first lane counts everyone holding its digit at once
          const uint64_t act = __builtin_amdgcn_ballot_w64(v);
          if (act != 0) {
            const int lead = __builtin_ctzll(act);
            const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, lead);
            const uint64_t m = __builtin_amdgcn_ballot_w64(v && d == d0);
            if (lane == lead) atomicAdd(&hist[d0], (uint32_t)__builtin_popcountll(m));
            if (d == d0) v = false;
          }
        }
        if (v) atomicAdd(&hist[d], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // suffix sums over bins (lane L owns bins 4L..4L+3), then the bin
        // holding the remaining-th largest key
        const int rem = s_remaining;
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
        uint32_t suf = h0 + h1 + h2 + h3;
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_down(suf, off, 64);
          if (lane + off < 64) suf += o;
        }
        const uint32_t above = suf - (h0 + h1 + h2 + h3);
        if (above < (uint32_t)rem && suf >= (uint32_t)rem) {
          uint32_t acc = above;
          int d = 4 * lane + 3;
          const uint32_t hv[4] = {h0, h1, h2, h3};
          for (int q = 3; q >= 0; --q) {
            d = 4 * lane + q;
            if (acc + hv[q] >= (uint32_t)rem) break;
            acc += hv[q];
          }
          const int new_rem = rem - (int)acc;
          s_remaining = new_rem;
          s_prefix = prefix | ((uint64_t)d << shift);
          s_done = (hist[d] == (uint32_t)new_rem) ? 1 : 0;
        }
      }
      __syncthreads();
      mask |= (uint64_t)0xFF << shift;
      if (s_done) break;
    }
  }
  const uint64_t thresh = s_prefix;
  auto kept = [&](int j) -> bool {
    const int blk = tid + kSelThreads * j;
    if (blk >= a.nbmax) return false;
    if (blk >= nexist || is_prot(blk)) return true;  // not written yet, or protected
    if (!((cm >> j) & 1u) || k == 0) return false;
    return take_all || key_of(j) >= thresh;
  };

  // keep words, and per (slice, wave) counts of kept existing blocks
  uint32_t* keep = a.keep + (size_t)b * a.kwords;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int blk = tid + kSelThreads * j;
    if (kSelThreads * j >= a.nbmax) {  // a slice past the last block: no words, no ids
      if (lane == 0) offs[j * (kSelThreads / 64) + wave] = 0;
      continue;
    }
    const bool f = kept(j);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
    const int w = blk >> 5;
    if ((lane & 31) == 0 && w < a.kwords) keep[w] = (uint32_t)(bal >> (lane & 32));
    const uint64_t bale = __builtin_amdgcn_ballot_w64(f && blk < nexist);
    if (lane == 0) offs[j * (kSelThreads / 64) + wave] = (uint32_t)__builtin_popcountll(bale);
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan over the (slice, wave) counts in ascending block order
    constexpr int N = KPT * (kSelThreads / 64);
    constexpr int PER = (N + 63) / 64;
    uint32_t v[PER];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int x = lane * PER + q;
      v[q] = x < N ? offs[x] : 0u;
      sum += v[q];
    }
    uint32_t inc = sum;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(inc, off, 64);
      if (lane >= off) inc += o;
    }
    uint32_t run = inc - sum;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int x = lane * PER + q;
      if (x < N) offs[x] = run;
      run += v[q];
    }
    if (lane == 63) s_total = (int)inc;
  }
  __syncthreads();
  int32_t* ids = a.sel_ids + (size_t)b * a.nbmax;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int blk = tid + kSelThreads * j;
    if (kSelThreads * j >= nexist) break;
    const bool fe = kept(j) && blk < nexist;
    const uint64_t bale = __builtin_amdgcn_ballot_w64(fe);
    if (fe) ids[offs[j * (kSelThreads / 64) + wave] + __builtin_popcountll(bale & below)] = blk;
  }
  if (tid == 0) a.n_sel[b] = s_total;
}

template <bool SC>
hipError_t launch_select_reg(const SelectArgs& a, int kpt, size_t lds, hipStream_t st) {
  switch (kpt) {
    case 1: hipLaunchKernelGGL((kvs_select_reg<1, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL((kvs_select_reg<2, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL((kvs_select_reg<4, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 8: hipLaunchKernelGGL((kvs_select_reg<8, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    default: hipLaunchKernelGGL((kvs_select_reg<16, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const size_t lds = a.alive ? (size_t)a.kwords * 4 : 0;
  int kpt = 1;
  while (kpt < kSelRegMax && (size_t)kpt * kSelThreads < (size_t)a.nbmax) kpt *= 2;
  if ((size_t)kpt * kSelThreads >= (size_t)a.nbmax)
    return a.mass ? launch_select_reg<true>(a, kpt, lds, st) : launch_select_reg<false>(a, kpt, lds, st);
  // wider sequences: the side-car as its own launch, then the memory-reading select
  SelectArgs s = a;
  if (a.mass) {
    const hipError_t e = launch_sidecar(a.mass, a.att, a.ema, a.cum, a.traj, a.B, a.nbmax, a.traj_cap,
                                        a.slot, a.alpha, st);
    if (e != hipSuccess) return e;
    s.score = a.score_src == 0 ? a.cum : (a.score_src == 1 ? a.ema : a.att);
  }
  hipLaunchKernelGGL(kvs_select, dim3(a.B), dim3(kSelThreads), lds, st, s);
  return hipGetLastError();
}

}  // namespace kvs
