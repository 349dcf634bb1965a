// Block compaction of a linear cache (Context Optimization, "H2O KV Cache
// Eviction / How It Works in Flash-MoE", step 4: surviving entries move to
// contiguous positions, and later passes read one shorter run of positions),
// here at 16-slot block granularity: kept block ids[k] becomes block k.
//
// In place. Ids outside the cache move nothing. With ids ascending, the destination k of a move can only coincide
// with the source ids[j] of an earlier move j < k (ids[j] >= j), never with a
// later one. Moves are therefore done in chunks: a workgroup loads a whole
// chunk's sources into registers, waits at a barrier, then stores; later
// chunks read sources above every destination already written.

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

constexpr int kCompactThreads = 512;
constexpr int kPiecesPerThread = 8;  // 16-byte pieces held per thread per chunk (two chunks in flight)

// With ids ascending and distinct, ids[k] == k holds exactly on a prefix (once
// ids[k] > k it stays so). Returns its length: moves start there. One pass,
// each thread checking a strided share, reduced with an LDS minimum.
__device__ int in_place_prefix(const int32_t* ids, int n, int* s_first) {
  if (threadIdx.x == 0) *s_first = n;
  __syncthreads();
  int first = n;
  for (int k = threadIdx.x; k < n; k += kCompactThreads)
    if (ids[k] != k) {
      first = k;
      break;
    }
  if (first < n) atomicMin(s_first, first);
  __syncthreads();
  return *s_first;
}

// K/V tiles of one (KV head, sequence), plus the sequence's K/V scales (KV
// head 0's workgroup). grid (Hkv, B). Chunks are software-pipelined: the
// next chunk's sources (never a destination of this or an earlier chunk) are
// loaded while this chunk is stored; a barrier separates each chunk's loads
// from its own stores.
__global__ __launch_bounds__(kCompactThreads) void kvs_compact_kv(CompactArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = min(max(a.n_keep[b], 0), min(a.ids_stride, a.NT));
  const int32_t* ids = a.ids + (size_t)b * a.ids_stride;
  const size_t tb = (size_t)a.tile_bytes;               // one tile of K (or V)
  const size_t region = (size_t)a.NT * tb;
  char* kreg = (char*)a.k + ((size_t)b * a.Hkv + g) * region;
  char* vreg = (char*)a.v + ((size_t)b * a.Hkv + g) * region;
  const bool scales = g == 0 && a.ks != nullptr;
  float* ksb = scales ? a.ks + (size_t)b * a.C : nullptr;
  float* vsb = scales ? a.vs + (size_t)b * a.C : nullptr;
  // pieces per tile: K and V codes, then (head 0) 4 + 4 pieces of scales
  const int code_pieces = (int)(tb / 16);
  const int pieces_per_tile = 2 * code_pieces + (scales ? 8 : 0);
  const int chunk = max(1, kCompactThreads * kPiecesPerThread / pieces_per_tile);  // tiles per round
  __shared__ int s_first;
  const int m = in_place_prefix(ids, n, &s_first);
  // address of piece pc of block blk
  auto addr = [&](int blk, int pc) -> char* {
    if (pc < code_pieces) return kreg + (size_t)blk * tb + 16 * pc;
    if (pc < 2 * code_pieces) return vreg + (size_t)blk * tb + 16 * (pc - code_pieces);
    if (pc < 2 * code_pieces + 4) return (char*)(ksb + (size_t)blk * kTile + 4 * (pc - 2 * code_pieces));
    return (char*)(vsb + (size_t)blk * kTile + 4 * (pc - 2 * code_pieces - 4));
  };
  auto load = [&](u32x4* buf, int k0) {
    const int total = min(chunk, n - k0) * pieces_per_tile;
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int x = tid + r * kCompactThreads;
      if (x < total) {
        const int k = k0 + x / pieces_per_tile;
        const int src = ids[k];
        if (src >= 0 && src < a.NT && src != k) buf[r] = *(const u32x4*)addr(src, x % pieces_per_tile);
      }
    }
  };
  auto store = [&](const u32x4* buf, int k0) {
    const int total = min(chunk, n - k0) * pieces_per_tile;
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int x = tid + r * kCompactThreads;
      if (x < total) {
        const int k = k0 + x / pieces_per_tile;
        const int src = ids[k];
        if (src >= 0 && src < a.NT && src != k) *(u32x4*)addr(k, x % pieces_per_tile) = buf[r];
      }
    }
  };
  if (m >= n) return;
  u32x4 bufa[kPiecesPerThread], bufb[kPiecesPerThread];
  load(bufa, m);
  for (int k0 = m; k0 < n; k0 += 2 * chunk) {
    __syncthreads();  // chunk k0 read everywhere before any of its stores
    if (k0 + chunk < n) load(bufb, k0 + chunk);
    store(bufa, k0);
    if (k0 + chunk >= n) break;
    __syncthreads();
    if (k0 + 2 * chunk < n) load(bufa, k0 + 2 * chunk);
    store(bufb, k0 + chunk);
  }
}

// One row of one per-block table (4-byte entries, [B][rows][nbmax]): entry
// ids[k] moves to k, entries n .. nbmax-1 become zero. grid (total rows, B).
__global__ __launch_bounds__(kCompactThreads) void kvs_compact_rows(CompactArgs a) {
  const int b = blockIdx.y;
  int row = blockIdx.x, t = 0;
  while (t < a.n_tables && row >= a.table_rows[t]) row -= a.table_rows[t++];
  if (t >= a.n_tables) return;
  uint32_t* base = (uint32_t*)a.tables[t] + ((size_t)b * a.table_rows[t] + row) * a.nbmax;
  const int n = min(max(a.n_keep[b], 0), min(a.ids_stride, a.nbmax));
  const int32_t* ids = a.ids + (size_t)b * a.ids_stride;
  const int tid = threadIdx.x;
  __shared__ int s_first;
  const int m = in_place_prefix(ids, n, &s_first);
  for (int k0 = m; k0 < n; k0 += kCompactThreads * kPiecesPerThread) {
    uint32_t v[kPiecesPerThread];
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int k = k0 + tid + r * kCompactThreads;
      if (k < n && ids[k] >= 0 && ids[k] < a.nbmax && ids[k] != k) v[r] = base[ids[k]];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int k = k0 + tid + r * kCompactThreads;
      if (k < n && ids[k] >= 0 && ids[k] < a.nbmax && ids[k] != k) base[k] = v[r];
    }
    __syncthreads();
  }
  for (int k = n + tid; k < a.nbmax; k += kCompactThreads) base[k] = 0u;
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(kvs_compact_kv, dim3(a.Hkv, a.B), dim3(kCompactThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_tables == 0) return e;
  int rows = 0;
  for (int t = 0; t < a.n_tables; ++t) rows += a.table_rows[t];
  hipLaunchKernelGGL(kvs_compact_rows, dim3(rows, a.B), dim3(kCompactThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
