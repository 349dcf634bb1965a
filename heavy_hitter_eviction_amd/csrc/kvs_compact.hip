// Block compaction of a linear cache (Context Optimization, "H2O KV Cache
// Eviction / How It Works in Flash-MoE", step 4: surviving entries move to
// contiguous positions so later kernels see a shorter, contiguous sequence),
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
constexpr int kPiecesPerThread = 8;  // 16-byte pieces held per thread per chunk

// K/V tiles of one (KV head, sequence), plus the sequence's K/V scales (KV
// head 0's workgroup). grid (Hkv, B).
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
  for (int k0 = 0; k0 < n; k0 += chunk) {
    const int nk = min(chunk, n - k0);
    const int total = nk * pieces_per_tile;
    u32x4 buf[kPiecesPerThread];
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int x = tid + r * kCompactThreads;
      if (x < total) {
        const int k = k0 + x / pieces_per_tile, pc = x % pieces_per_tile;
        const int src = ids[k];
        if (src < 0 || src >= a.NT) continue;  // not a block of this cache: no move
        if (pc < code_pieces) buf[r] = *(const u32x4*)(kreg + (size_t)src * tb + 16 * pc);
        else if (pc < 2 * code_pieces) buf[r] = *(const u32x4*)(vreg + (size_t)src * tb + 16 * (pc - code_pieces));
        else if (pc < 2 * code_pieces + 4) buf[r] = *(const u32x4*)(ksb + (size_t)src * kTile + 4 * (pc - 2 * code_pieces));
        else buf[r] = *(const u32x4*)(vsb + (size_t)src * kTile + 4 * (pc - 2 * code_pieces - 4));
      }
    }
    __syncthreads();  // every source of this chunk is read before any store
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int x = tid + r * kCompactThreads;
      if (x < total) {
        const int k = k0 + x / pieces_per_tile, pc = x % pieces_per_tile;
        if (ids[k] < 0 || ids[k] >= a.NT) continue;
        if (pc < code_pieces) *(u32x4*)(kreg + (size_t)k * tb + 16 * pc) = buf[r];
        else if (pc < 2 * code_pieces) *(u32x4*)(vreg + (size_t)k * tb + 16 * (pc - code_pieces)) = buf[r];
        else if (pc < 2 * code_pieces + 4) *(u32x4*)(ksb + (size_t)k * kTile + 4 * (pc - 2 * code_pieces)) = buf[r];
        else *(u32x4*)(vsb + (size_t)k * kTile + 4 * (pc - 2 * code_pieces - 4)) = buf[r];
      }
    }
    __syncthreads();
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
  for (int k0 = 0; k0 < n; k0 += kCompactThreads * kPiecesPerThread) {
    uint32_t v[kPiecesPerThread];
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int k = k0 + tid + r * kCompactThreads;
      if (k < n && ids[k] >= 0 && ids[k] < a.nbmax) v[r] = base[ids[k]];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int k = k0 + tid + r * kCompactThreads;
      if (k < n && ids[k] >= 0 && ids[k] < a.nbmax) base[k] = v[r];
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
