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
// the radix passes read no memory. The rows are addressed through buffer
// resources of the row's size: blocks past nbmax read as zero and their
// stores are dropped, so the slices need no bounds branches. The radix runs
// over the 32 order bits of the score, 8-bit digits from the highest; when
// keys are still tied after the last digit, the tied ones are ranked by block
// index with one scan and the lowest indices kept, which is the order of the
// 64-bit keys of kvs_select. The digits start at the highest bit where the
// existing blocks' keys differ (one min/max reduction finds it). Every wave
// scans the 256-bin histogram itself, so a pass needs one barrier; three
// histogram buffers take turns, so that clearing one never meets the reads
// or increments of another. In the first pass a wave's increments for its
// first lane's digit are added at once (that digit is often shared by most
// blocks, whose LDS atomics would otherwise serialise on one address). The
// kept ids
// are placed with one scan over (thread slice, wave) counts. With SC the
// side-car update of the sequence's blocks comes first, in the same
// arithmetic as kvs_sidecar, and the selection scores the updated array.
// Same keys, threshold and outputs as kvs_select.
// ---------------------------------------------------------------------------
constexpr int kSelRegMax = 16;  // keys per thread: sequences of up to 16384 blocks
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sel_row(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float sel_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void sel_store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
}

// Counts c[j][w] (slice j, wave w) in LDS, ranked in ascending (j, w) order,
// which is ascending block order. Lane j < KPT of the calling wave gets the
// exclusive prefix at (j, wave); *total is the sum of all. No barrier: every
// wave computes what it needs.
template <int KPT>
__device__ __forceinline__ uint32_t slice_prefix(const uint32_t* c, int wave, int lane, uint32_t* total) {
  uint32_t mine = 0, before = 0;
  if (lane < KPT) {
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t x = c[lane * kSelWaves + w];
      mine += x;
      before += w < wave ? x : 0u;
    }
  }
  uint32_t inc = mine;
#pragma unroll
  for (int off = 1; off < KPT; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)inc, off, 64);
    if (lane >= off) inc += o;
  }
  *total = (uint32_t)__builtin_amdgcn_readlane((int)inc, KPT - 1);
  return inc - mine + before;
}

template <int KPT, bool SC>
__global__ __launch_bounds__(kSelThreads) void kvs_select_reg(SelectArgs a) {
  extern __shared__ uint32_t alive_lds[];  // [kwords]
  __shared__ __attribute__((aligned(16))) uint32_t hist[3][256];
  __shared__ uint32_t wcand[kSelWaves];           // candidates per wave
  __shared__ uint32_t wlo[kSelWaves], whi[kSelWaves];  // range of the existing blocks' order bits, per wave
  __shared__ uint32_t tcnt[KPT * kSelWaves];      // tied keys per (slice, wave)
  __shared__ uint32_t kcnt[KPT * kSelWaves];      // kept existing blocks per (slice, wave)
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = a.nbmax;
  const uint32_t rb = (uint32_t)nb * 4u;
  const size_t row = (size_t)b * nb;
  const bool have_alive = a.alive != nullptr;
  auto voff = [&](int j) { return (uint32_t)(tid + kSelThreads * j) * 4u; };

  // every load is issued before any store (the rows may overlap as far as
  // the compiler knows): the alive word first (one per thread: a row of at
  // most 16384 blocks has at most 512 words), so that staging it waits for
  // nothing else, then the rows, then the position
  static_assert(kSelRegMax * kSelThreads / 32 <= kSelThreads, "one alive word per thread");
  const bool stage = have_alive && tid < a.kwords;
  uint32_t aw = 0u;
  if (stage) aw = a.alive[(size_t)b * a.kwords + tid];
  uint32_t ord[KPT];
  float A[KPT], E[KPT], C[KPT];
  if constexpr (SC) {
    const auto rm = sel_row(a.mass + row, rb), re = sel_row(a.ema + row, rb), rc = sel_row(a.cum + row, rb);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      A[j] = sel_load(rm, voff(j));
      E[j] = sel_load(re, voff(j));
      C[j] = sel_load(rc, voff(j));
    }
  } else {
    const auto rs = sel_row(a.score + row, rb);
#pragma unroll
    for (int j = 0; j < KPT; ++j) A[j] = sel_load(rs, voff(j));
  }
  const int i = a.cur_pos[b];
  if (stage) alive_lds[tid] = aw;
  if (tid < 512) (&hist[0][0])[tid] = 0u;  // the first two passes' buffers
  if constexpr (SC) {
    const auto ra = sel_row(a.att + row, rb), re = sel_row(a.ema + row, rb), rc = sel_row(a.cum + row, rb),
               rm = sel_row(a.mass + row, rb);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      E[j] = a.alpha * A[j] + (1.0f - a.alpha) * E[j];
      C[j] = C[j] + A[j];
      ord[j] = float_order(a.score_src == 0 ? C[j] : (a.score_src == 1 ? E[j] : A[j]));
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      sel_store(ra, voff(j), A[j]);
      sel_store(re, voff(j), E[j]);
      sel_store(rc, voff(j), C[j]);
      sel_store(rm, voff(j), 0.0f);
    }
    if (a.traj) {
      const auto rt = sel_row(a.traj + ((size_t)b * a.traj_cap + a.slot) * nb, rb);
#pragma unroll
      for (int j = 0; j < KPT; ++j) sel_store(rt, voff(j), A[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) ord[j] = float_order(A[j]);
  }
  const int nexist = min(i / kTile + 1, nb);
  const int rlo = max(0, i - a.recent + 1) / kTile;
  const int rhi = i / kTile;
  const int shi = a.sinks > 0 ? (min(a.sinks, i + 1) - 1) / kTile : -1;
  {
    // the range of the existing blocks' order bits (the candidates are among
    // them): the radix starts at the highest bit where they differ
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool e = tid + kSelThreads * j < nexist;
      lo = e ? min(lo, ord[j]) : lo;
      hi = e ? max(hi, ord[j]) : hi;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    }
    if (lane == 0) {
      wlo[wave] = lo;
      whi[wave] = hi;
    }
  }
  __syncthreads();
  auto is_prot = [&](int blk) { return ((blk >= rlo) & (blk <= rhi)) | (blk <= shi); };
  uint32_t cm = 0;  // candidate bit per slice
  {
    uint32_t wc = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int blk = tid + kSelThreads * j;
      // bitwise, not short-circuit: no branches per slice
      bool alive = true;
      if (have_alive) alive = (alive_lds[min(blk >> 5, a.kwords - 1)] >> (blk & 31)) & 1u;
      const bool c = (blk < nexist) & !is_prot(blk) & alive;
      cm |= c ? (1u << j) : 0u;
      wc += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(c));
    }
    if (lane == 0) wcand[wave] = wc;
  }

  // radix passes over the order bits, 8-bit digits from the highest bit
  // where the existing keys differ (the bits above it are common to all):
  // prefix holds the bits chosen so far, rem how many keys under it are
  // still to keep. The first barrier also brings the candidate counts.
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    lo = min(lo, wlo[w]);
    hi = max(hi, whi[w]);
  }
  int pos = lo == hi ? -1 : 31 - __builtin_clz(lo ^ hi);
  // bits above pos (all of them when every existing key is the same)
  uint32_t mask = pos < 0 ? ~0u : (pos >= 31 ? 0u : ~((2u << pos) - 1u));
  uint32_t prefix = hi & mask;
  int ncand = 0, k = 0, rem = 0;
  bool select = false, resolved = false, first = true;
  int hb = 0;
  do {
    const int shift = max(pos - 7, 0);
    const uint32_t dmask = pos >= 0 ? (2u << (pos - shift)) - 1u : 0u;
    uint32_t* h = hist[hb];
    if (pos >= 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        bool v = (((cm >> j) & 1u) != 0) & ((ord[j] & mask) == prefix);
        const uint32_t d = (ord[j] >> shift) & dmask;
        if (first) {
          // the first digit is often shared by most blocks (scores of few
          // binades): a wave's increments for its first lane's digit go in
          // as one atomic, so its lanes do not serialise on one address
          const uint64_t act = __builtin_amdgcn_ballot_w64(v);
          if (act != 0) {
            const int lead = __builtin_ctzll(act);
            const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, lead);
            const uint64_t m = __builtin_amdgcn_ballot_w64(v & (d == d0));
            if (lane == lead) atomicAdd(&h[d0], (uint32_t)__builtin_popcountll(m));
            v = v & (d != d0);
          }
        }
        if (v) atomicAdd(&h[d], 1u);
      }
    }
    __syncthreads();
    if (first) {
      first = false;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) ncand += (int)wcand[w];
      k = min(a.budget, ncand);
      rem = k;
      select = k > 0 && k < ncand;
      if (!select) break;
    }
    if (pos < 0) break;  // every candidate has the same key: the ties decide
    // the bin holding the rem-th largest key under the prefix (lane L owns
    // bins 4L .. 4L + 3; suffix sums over lanes)
    const u32x4 hv = *(const u32x4*)&h[4 * lane];
    const uint32_t own = hv[0] + hv[1] + hv[2] + hv[3];
    uint32_t suf = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_down((int)suf, off, 64);
      if (lane + off < 64) suf += o;
    }
    const uint32_t above = suf - own;
    const bool here = above < (uint32_t)rem && suf >= (uint32_t)rem;
    uint32_t acc = above, dl = 4u * lane, cl = hv[0];
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      dl = 4u * lane + q;
      cl = hv[q];
      if (acc + hv[q] >= (uint32_t)rem) break;
      acc += hv[q];
    }
    const uint64_t hm = __builtin_amdgcn_ballot_w64(here);
    const int src = hm != 0 ? __builtin_ctzll(hm) : 0;
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)dl, src);
    const uint32_t above_d = (uint32_t)__builtin_amdgcn_readlane((int)acc, src);
    const uint32_t cnt_d = (uint32_t)__builtin_amdgcn_readlane((int)cl, src);
    // the buffer two passes ahead was last read in the previous pass
    const int hn = hb == 2 ? 0 : hb + 1;
    const int hc = hn == 2 ? 0 : hn + 1;
    if (tid < 256) hist[hc][tid] = 0u;
    prefix |= d << shift;
    mask |= dmask << shift;
    rem -= (int)above_d;
    hb = hn;
    if (cnt_d == (uint32_t)rem) {
      resolved = true;
      break;
    }
    pos = shift - 1;
  } while (pos >= 0);

  // keys tied at the threshold after every digit: keep the rem lowest blocks
  uint32_t tk = 0;  // tied keys kept, per slice
  if (select && !resolved) {
    uint64_t tb[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      tb[j] = __builtin_amdgcn_ballot_w64(((cm >> j) & 1u) && ord[j] == prefix);
      if (lane == 0) tcnt[j * kSelWaves + wave] = (uint32_t)__builtin_popcountll(tb[j]);
    }
    __syncthreads();
    uint32_t tot;
    const uint32_t pre = slice_prefix<KPT>(tcnt, wave, lane, &tot);
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t rank = (uint32_t)__builtin_amdgcn_readlane((int)pre, j) + (uint32_t)__builtin_popcountll(tb[j] & below);
      if (((tb[j] >> lane) & 1ull) && rank < (uint32_t)rem) tk |= 1u << j;
    }
  }
  // kept: inside the row, and not written yet or protected, or a candidate
  // that the budget takes (all of them when they fit); bitwise, no branches
  const bool any = k != 0, all = !select;
  auto kept = [&](int j) -> bool {
    const int blk = tid + kSelThreads * j;
    const bool score_ok = resolved ? ord[j] >= prefix : (ord[j] > prefix) | (((tk >> j) & 1u) != 0);
    const bool cand = ((cm >> j) & 1u) != 0;
    return (blk < nb) & ((blk >= nexist) | is_prot(blk) | (cand & any & (all | score_ok)));
  };

  // keep words, and per (slice, wave) counts of kept existing blocks
  uint32_t* keep = a.keep + (size_t)b * a.kwords;
  uint64_t kb[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int blk = tid + kSelThreads * j;
    const bool f = kept(j);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
    const int w = blk >> 5;
    if ((lane & 31) == 0 && w < a.kwords) keep[w] = (uint32_t)(bal >> (lane & 32));
    kb[j] = __builtin_amdgcn_ballot_w64(f && blk < nexist);
    if (lane == 0) kcnt[j * kSelWaves + wave] = (uint32_t)__builtin_popcountll(kb[j]);
  }
  __syncthreads();
  uint32_t total;
  const uint32_t pre = slice_prefix<KPT>(kcnt, wave, lane, &total);
  int32_t* ids = a.sel_ids + (size_t)b * a.nbmax;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)pre, j);
    if ((kb[j] >> lane) & 1ull) ids[base + __builtin_popcountll(kb[j] & below)] = tid + kSelThreads * j;
  }
  if (tid == 0) a.n_sel[b] = (int)total;
}

template <bool SC>
hipError_t launch_select_reg(const SelectArgs& a, int kpt, size_t lds, hipStream_t st) {
  switch (kpt) {
    case 1: hipLaunchKernelGGL((kvs_select_reg<1, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL((kvs_select_reg<2, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 3: hipLaunchKernelGGL((kvs_select_reg<3, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL((kvs_select_reg<4, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 6: hipLaunchKernelGGL((kvs_select_reg<6, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 9: hipLaunchKernelGGL((kvs_select_reg<9, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    case 12: hipLaunchKernelGGL((kvs_select_reg<12, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
    default: hipLaunchKernelGGL((kvs_select_reg<16, SC>), dim3(a.B), dim3(kSelThreads), lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const size_t lds = a.alive ? (size_t)a.kwords * 4 : 0;
  // slices per thread: the smallest instantiated count that covers the row
  // (each slice costs its loads and ALU work whether its blocks exist or not)
  const int need = (int)(((size_t)a.nbmax + kSelThreads - 1) / kSelThreads);
  const int kpt = need <= 4 ? max(need, 1) : need <= 6 ? 6 : need <= 9 ? 9 : need <= 12 ? 12 : kSelRegMax;
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
