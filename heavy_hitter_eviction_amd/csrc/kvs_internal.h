// Internal launch interfaces of libkvs (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

enum : int { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// Waves per decode (partial) workgroup; one such workgroup per compute unit.
constexpr int kPartialWaves = 8;
// LDS floats the decode kernel keeps for the appended row of its KV head:
// K and V values as the cache holds them (at most 2 x 128 x 4 bytes), then
// the two FP8 scales in the last two floats.
constexpr int kAppRowFloats = 260;

struct PartialArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  const int32_t* pos_of_slot;
  const int32_t* cur_pos;
  const uint32_t* keep;
  const int32_t* ids;    // [B][ids_stride] block ids to read (re-attend), or NULL
  const int32_t* n_ids;  // [B] entries of ids used per sequence
  // one partial per partition (workgroup)
  float* ws_m;     // [B][Hq][P] max (log2 units)
  float* ws_l;     // [B][Hq][P] sum of 2^(logit - max)
  float* ws_o;     // [B][Hq][P][D] unnormalised output
  float* ws_e;     // [B][Hkv][NT][NSUB][G] per-tile block sums, relative to the
                   // max of the partition's workgroup (its waves' ws_m)
  int* ws_pid;     // [B][Hkv][NT] partition map of a linear range: the index of
                   // the partition that read each tile of the range
  float* ws_w;     // [B][P][Hq] merge weights 2^(m_p - M) / L per partition and
                   // head, written by the workgroup that merges the outputs
  float* ws_time;  // [workgroups][kPartialWaves][2] tiles processed, clock ticks
  const float* rates;  // [8] relative streaming rate per dispatch class, or NULL
  int B, Hq, Hkv, G, C, NT, window, nbmax, kwords, tpp, nparts;
  int ids_stride;
  int dyn;     // 1: waves claim tiles dynamically; 0: fixed round-robin order
  int tl_cap;  // LDS capacity of the kept-tile list (>= any partition's tiles)
  int adapt;   // 1: partitions may be weighted by the measured rates (tl_cap allows it)
  float scale_log2;
  // Fused append: row b of app_k / app_v ([B][Hkv*D], bf16 if app_bf16, else
  // f32) is written at position cur_pos[b] of the cache (k, v, ks, vs and
  // pos_of_slot are then written too) before the tile holding it is read.
  // NULL app_k: no append.
  const void* app_k;
  const void* app_v;
  int app_bf16;
  // Output merge in the kernel: every partition of a (sequence, KV head) adds
  // 1 to the pair's counter (pair_flag[(b * Hkv + g) * P], zero at entry;
  // the region holds B * Hkv * P words) once its partial is in memory; the
  // one that reads back P - 1 merges the group's partials into out and puts
  // the counter back to zero.
  uint32_t* pair_flag;
  void* out;
};

// Most layers one kvs_combine launch sums (kvs_tap_masses).
constexpr int kMaxTapLayers = 128;

// Block masses of n_layers calls' records, added in call order. Layer l's
// workspace starts at lws[l]; every layer has the same plan (offsets).
struct CombineArgs {
  const char* lws[kMaxTapLayers];
  size_t off_w, off_e, off_pid, off_time, off_rates;
  int n_layers;
  int layers_per_chunk;  // layers whose tables fit the LDS at once
  int n_wg;       // partial workgroups per layer that wrote clock records
  const int32_t* cur_pos;
  float* mass;
  float* head_mass;  // [B][Hq][nbmax] per-head block masses (+=), or NULL
  float* mass_max;   // [B][nbmax] running max over heads (and calls), or NULL
  int B, Hq, Hkv, C, NT, nbmax, tpp, nparts, n_mass_chunks, window;
  // the turn's side-car update in the same launch (kvs_combine_layers only;
  // sc_att NULL: none): the arrays of kvs_update_sidecar, the trajectory
  // slot and the EMA weight
  float *sc_att, *sc_ema, *sc_cum, *sc_traj;
  int sc_traj_cap, sc_slot;
  float sc_alpha;
};

// Side-car columns of the layer combine (sweeping the blocks its tiles do
// not reach), per sequence.
constexpr int kCmbSidecarCols = 4;

// One block's side-car update, the arithmetic of kvs_update_sidecar: with A
// the turn's mass of block blk of sequence b (x = b * nbmax + blk),
// attended = A, ema = alpha A + (1 - alpha) ema, cum += A, the trajectory
// slot = A, and the mass back to zero.
__device__ __forceinline__ void sidecar_block(float* mass, float* att, float* ema, float* cum, float* traj,
                                              size_t x, int b, int blk, int nbmax, int traj_cap, int slot,
                                              float alpha, float A) {
  att[x] = A;
  ema[x] = alpha * A + (1.0f - alpha) * ema[x];
  cum[x] = cum[x] + A;
  if (traj) traj[((size_t)b * traj_cap + slot) * nbmax + blk] = A;
  mass[x] = 0.0f;
}

// LDS floats one layer's combine tables take: the per (partition, head)
// record weights. A combine workgroup also needs 16 floats for rates.
__host__ __device__ inline size_t combine_layer_floats(int Hq, int Hkv, int P) {
  (void)Hkv;
  return (size_t)Hq * P;
}
constexpr size_t kCombineLdsBytes = 49152;

hipError_t launch_partial(int kv, int d, const PartialArgs& a, bool scored, bool ring,
                          size_t lds_bytes, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, bool ring, hipStream_t st);
// The layer-parallel form (no per-head masses); its LDS must fit kCombineLdsBytes.
size_t combine_layers_lds_bytes(int Hq, int Hkv, int P, int L, bool ring);
hipError_t launch_combine_layers(const CombineArgs& a, bool ring, hipStream_t st);

// Fills n_words 32-bit words at dst (16-byte aligned) with value, on the
// stream (a kernel, not a memset node).
hipError_t launch_fill_u32(uint32_t* dst, size_t n_words, uint32_t value, hipStream_t st);

hipError_t launch_encode_fp8(const void* src, int src_bf16, int64_t n_rows, int row_len,
                             uint8_t* codes, float* scales, hipStream_t st);

struct AppendArgs {
  const void* k_rows;
  const void* v_rows;
  const int32_t* row_seq;
  const int32_t* row_pos;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  int32_t* pos_of_slot;
  int n_rows, B, Hkv, D, C, ring, kv, src_bf16;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

hipError_t launch_sidecar(float* mass, float* att, float* ema, float* cum, float* traj, int B,
                          int nbmax, int traj_cap, int64_t step, float alpha, hipStream_t st);

struct SelectArgs {
  const float* score;
  const uint32_t* alive;
  const int32_t* cur_pos;
  uint32_t* keep;
  int32_t* sel_ids;
  int32_t* n_sel;
  int B, nbmax, kwords, budget, recent, sinks;
  // Side-car update in the same launch (kvs_update_sidecar_select), applied
  // to every block before the selection, which then scores with the updated
  // array score_src names (0 cumulative, 1 EMA, 2 attended). NULL mass: none.
  float* mass;
  float* att;
  float* ema;
  float* cum;
  float* traj;
  int traj_cap, slot, score_src;
  float alpha;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t st);

struct CounterArgs {
  const float* attended;
  const float* ema;
  int32_t* hot_count;   // [B][nbmax] or NULL
  int32_t* cold_turns;  // [B][nbmax] or NULL
  float* traj;          // [B][traj_cap][nbmax] or NULL (no trajectory GC)
  int B, nbmax, traj_cap, cold_limit;
  float hot_theta, cold_theta;
};
hipError_t launch_counters(const CounterArgs& a, hipStream_t st);

struct FilterArgs {
  const float* score;
  const uint32_t* alive;
  const int32_t* cur_pos;
  int32_t* ids;
  int32_t* n_ids;
  int B, nbmax, kwords, ids_stride;
  float theta;
};
hipError_t launch_filter(const FilterArgs& a, hipStream_t st);

constexpr int kMaxCompactTables = 8;
struct CompactArgs {
  void* k;
  void* v;
  float* ks;
  float* vs;
  const int32_t* ids;     // [B][ids_stride] kept block ids, ascending
  const int32_t* n_keep;  // [B]
  void* tables[kMaxCompactTables];  // per-block tables of 4-byte entries [B][rows][nbmax]
  int table_rows[kMaxCompactTables];
  int n_tables;
  int B, Hkv, C, NT, nbmax, ids_stride, tile_bytes;
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t st);

struct SnapArgs {
  const void* q;             // [B][W][Hq][D] bf16 window queries
  const void* k;
  const float* ks;
  const int32_t* n_prompt;   // [B]
  float* part_ml;            // [B][Hkv][W*G][nparts][2] workspace
  float* col_m;              // [B][Hkv][W*G] workspace
  float* col_l;              // [B][Hkv][W*G] workspace
  float* token_score;        // [B][Hq][C]
  float* block_score;        // [B][nbmax] (+=) or NULL
  int B, Hq, Hkv, G, C, NT, nbmax, W, tpp, nparts, pool;
  int nparts0;               // the first pass's partitions (what the second pass merges)
  float scale_log2;
};
hipError_t launch_snap(int kv, int d, const SnapArgs& a, hipStream_t st);

// Streaming-read probe: bytes (a multiple of 1024) read once by `workgroups`
// 8-wave workgroups, each storing one sum to sums[workgroup].
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sums, int workgroups, hipStream_t st);

}  // namespace kvs
