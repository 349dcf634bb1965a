// libkvs C ABI: argument checking, partition planning and launches.
// Declarations and the full contract of every entry point are in include/kvs.h.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kvs.h"
#include "kvs_internal.h"

namespace {

constexpr int kTileSlots = 16;
// One decode workgroup (kPartialWaves waves) per compute unit of MI355X (256
// CUs). With several workgroups per CU the younger ones were served last by
// the memory pipeline and finished up to a third later; inside one workgroup
// the waves share the partition's tiles dynamically instead.
constexpr int kTargetWorkgroups = 256;
constexpr int kLdsBudgetFloats = 16384;  // 64 KiB per decode workgroup for the partition's records
// the whole workgroup, output slots included (the MI355X gives a workgroup
// up to 160 KiB)
constexpr size_t kLdsMaxBytes = 163840;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dt) { return dt == KVS_F32 ? 4 : dt == KVS_BF16 ? 2 : 1; }

int check_geom(const kvs_geom* g) {
  if (!g) return KVS_EINVAL;
  if (g->batch < 1 || g->n_kv_heads < 1 || g->n_q_heads < 1) return KVS_EINVAL;
  if (g->n_q_heads % g->n_kv_heads) return KVS_EINVAL;
  if (g->n_q_heads / g->n_kv_heads > 16) return KVS_ENOTIMPL;
  if (g->capacity < kTileSlots || g->capacity % kTileSlots) return KVS_EINVAL;
  if (g->window < 0) return KVS_EINVAL;
  if (g->ring != 0 && g->ring != 1) return KVS_EINVAL;
  if (g->n_blocks_max < 1) return KVS_EINVAL;
  if (!g->ring && g->n_blocks_max < g->capacity / kTileSlots) return KVS_EINVAL;
  if (!(g->softmax_scale > 0.0f) || !isfinite(g->softmax_scale)) return KVS_EINVAL;
  if (g->deterministic != 0 && g->deterministic != 1) return KVS_EINVAL;
  const int kv = g->kv_dtype, q = g->q_dtype, d = g->head_dim;
  if (kv != KVS_F32 && kv != KVS_BF16 && kv != KVS_FP8_E4M3) return KVS_EDTYPE;
  if (kv == KVS_F32) {
    if (q != KVS_F32) return KVS_EDTYPE;
    if (d != 16 && d != 64 && d != 128) return KVS_EDTYPE;
  } else {
    if (q != KVS_BF16) return KVS_EDTYPE;
    if (d != 64 && d != 128) return KVS_EDTYPE;
  }
  // sizes that must fit the kernels' 32-bit indexing of per-sequence slots;
  // one (sequence, KV head) region is addressed with 32-bit buffer offsets
  if ((int64_t)g->capacity * g->n_kv_heads * d > (int64_t)1 << 40) return KVS_EINVAL;
  if ((int64_t)g->capacity * d * elem_bytes(kv) > (int64_t)0xFFFF0000) return KVS_EINVAL;
  return KVS_OK;
}

struct Plan {
  int NT, tpp, nparts, nsub, G, S, tl_cap, n_wg, adapt;
  size_t off_m, off_l, off_o, off_e, off_pid, off_w, off_time, off_rates, off_cnt, total;
  size_t lds_partial;
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(const kvs_geom* g) {
  Plan p{};
  p.G = g->n_q_heads / g->n_kv_heads;
  p.NT = g->capacity / kTileSlots;
  p.nsub = g->ring ? 2 : 1;
  const int pairs = g->batch * g->n_kv_heads;
  int ptarget = (kTargetWorkgroups + pairs - 1) / pairs;
  if (ptarget < 1) ptarget = 1;
  int tpp = (p.NT + ptarget - 1) / ptarget;
  if (tpp < 4) tpp = 4;
  // the partial kernel keeps per-wave side data and, per tile of its
  // partition, the block-sum records and the kept-tile list in LDS: bound the
  // partition so that part stays <= 64 KiB
  const int nw = kvs::kPartialWaves;
  const int lds_fixed = nw * 256 + kvs::kAppRowFloats + 8 + 2 * nw * 16 + p.NT / 32 + 1;  // + the keep bitmap
  const int per_tile = p.G * (p.nsub + 1) + 1;
  const int tpp_lds = (kLdsBudgetFloats - lds_fixed) / per_tile;
  if (tpp > tpp_lds) tpp = tpp_lds < 4 ? 4 : tpp_lds;
  // the mass combine keeps a layer's record weights
  // in LDS: bound them to 48 KiB
  while (true) {
    const int np = (p.NT + tpp - 1) / tpp;
    if (kvs::combine_layer_floats(g->n_q_heads, g->n_kv_heads, np) * 4 <= kvs::kCombineLdsBytes) break;
    tpp *= 2;
  }
  p.tpp = tpp;
  p.nparts = (p.NT + tpp - 1) / tpp;
  p.S = p.nparts;
  p.n_wg = p.nparts * pairs;
  // a linear range's partitions may be weighted by the measured rates, each
  // weight within 1/1.2 .. 1.2 of the others' mean: the list must then hold a
  // share of up to 1.44 / (1.44 + nparts - 1) of the tiles; without the LDS
  // for that the split stays even
  p.tl_cap = tpp;
  p.adapt = 0;
  if (!g->ring) {
    const int need = (int)(1.44 * p.NT / (1.44 + p.nparts - 1)) + 2;
    if (need <= tpp_lds) {
      p.adapt = 1;
      if (need > p.tl_cap) p.tl_cap = need;
    }
  }
  const size_t bh = (size_t)g->batch * g->n_q_heads;
  p.off_m = 0;
  p.off_l = round256(p.off_m + bh * p.S * 4);
  p.off_o = round256(p.off_l + bh * p.S * 4);
  p.off_e = round256(p.off_o + bh * p.S * g->head_dim * 4);
  p.off_pid = round256(p.off_e + (size_t)g->batch * p.NT * p.nsub * g->n_q_heads * 4);
  p.off_w = round256(p.off_pid + (size_t)pairs * p.NT * 4);
  p.off_time = round256(p.off_w + bh * p.nparts * 4);
  p.off_rates = round256(p.off_time + (size_t)p.n_wg * nw * 2 * 4);
  p.off_cnt = round256(p.off_rates + 8 * 4);
  p.total = round256(p.off_cnt + (size_t)pairs * p.nparts * 4);
  // LDS: the fixed part and the records, then (16-byte aligned) one output
  // slot per wave, rows padded by 4 floats; at the end the output merge of a
  // (sequence, KV head) stages 3 G nparts floats from the output slots on
  const size_t rec_end = (size_t)lds_fixed + (size_t)p.tl_cap * per_tile;
  const size_t o_start = (rec_end + 3) & ~(size_t)3;
  const size_t o_end = o_start + (size_t)nw * p.G * (g->head_dim + 4);
  const size_t merge_end = o_start + 3 * (size_t)p.G * p.nparts;
  p.lds_partial = 4 * (o_end > merge_end ? o_end : merge_end);
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVS_OK : KVS_EHIP; }

}  // namespace

extern "C" {

const char* kvs_version(void) { return "libkvs 0.1 (gfx950)"; }

const char* kvs_status_str(int s) {
  switch (s) {
    case KVS_OK: return "ok";
    case KVS_EINVAL: return "invalid argument or geometry";
    case KVS_EDTYPE: return "unsupported dtype or head-dim combination";
    case KVS_EALIGN: return "pointer not 16-byte aligned";
    case KVS_EWS: return "workspace too small";
    case KVS_EHIP: return "HIP launch failure";
    case KVS_ENOTIMPL: return "not implemented for this combination";
    case KVS_ESCRATCH: return "geometry needs more than the static scratch maximum (KVS_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kvs_cache_bytes(const kvs_geom* g, size_t* kv_bytes, size_t* scale_bytes, size_t* pos_bytes) {
  int st = check_geom(g);
  if (st) return st;
  const size_t slots = (size_t)g->batch * g->capacity;
  if (kv_bytes) *kv_bytes = slots * g->n_kv_heads * g->head_dim * elem_bytes(g->kv_dtype);
  if (scale_bytes) *scale_bytes = g->kv_dtype == KVS_FP8_E4M3 ? slots * 4 : 0;
  if (pos_bytes) *pos_bytes = g->ring ? slots * 4 : 0;
  return KVS_OK;
}

int kvs_encode_fp8(const void* src, int32_t src_dtype, int64_t n_rows, int32_t row_len,
                   uint8_t* codes, float* scales, void* stream) {
  if (src_dtype != KVS_F32 && src_dtype != KVS_BF16) return KVS_EDTYPE;
  if (n_rows < 0 || row_len < 1 || row_len > 65536) return KVS_EINVAL;
  if (n_rows == 0) return KVS_OK;
  if (!src || !codes || !scales) return KVS_EINVAL;
  if (!aligned16(src) || !aligned16(codes) || !aligned16(scales)) return KVS_EALIGN;
  return hip_status(kvs::launch_encode_fp8(src, src_dtype == KVS_BF16, n_rows, row_len, codes,
                                           scales, (hipStream_t)stream));
}

int kvs_append_kv(const kvs_geom* g, const void* k_rows, const void* v_rows, int32_t src_dtype,
                  int32_t n_rows, const int32_t* row_seq, const int32_t* row_pos, void* k_cache,
                  void* v_cache, float* k_scale, float* v_scale, int32_t* pos_of_slot,
                  void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (n_rows < 0) return KVS_EINVAL;
  if (src_dtype != KVS_F32 && src_dtype != KVS_BF16) return KVS_EDTYPE;
  const bool fp8 = g->kv_dtype == KVS_FP8_E4M3;
  if (!fp8 && src_dtype != g->kv_dtype) return KVS_EDTYPE;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return KVS_EINVAL;
  if ((g->ring != 0) != (pos_of_slot != nullptr)) return KVS_EINVAL;
  if (n_rows == 0) return KVS_OK;
  if (!k_rows || !v_rows || !row_seq || !row_pos || !k_cache || !v_cache) return KVS_EINVAL;
  const void* ptrs[] = {k_rows, v_rows, row_seq, row_pos, k_cache, v_cache, k_scale, v_scale, pos_of_slot};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  kvs::AppendArgs a{};
  a.k_rows = k_rows; a.v_rows = v_rows; a.row_seq = row_seq; a.row_pos = row_pos;
  a.k_cache = k_cache; a.v_cache = v_cache; a.k_scale = k_scale; a.v_scale = v_scale;
  a.pos_of_slot = pos_of_slot;
  a.n_rows = n_rows; a.B = g->batch; a.Hkv = g->n_kv_heads; a.D = g->head_dim; a.C = g->capacity;
  a.ring = g->ring; a.kv = g->kv_dtype == KVS_FP8_E4M3 ? kvs::KV_FP8 : g->kv_dtype == KVS_BF16 ? kvs::KV_BF16 : kvs::KV_F32;
  a.src_bf16 = src_dtype == KVS_BF16;
  return hip_status(kvs::launch_append(a, (hipStream_t)stream));
}

int kvs_decode_workspace_bytes(const kvs_geom* g, size_t* bytes) {
  int st = check_geom(g);
  if (st) return st;
  if (!bytes) return KVS_EINVAL;
  *bytes = make_plan(g).total;
  return KVS_OK;
}

int kvs_decode_workspace_init(const kvs_geom* g, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (!workspace) return KVS_EINVAL;
  if (!aligned16(workspace)) return KVS_EALIGN;
  const Plan p = make_plan(g);
  if (workspace_bytes < p.total) return KVS_EWS;
  return hip_status(kvs::launch_fill_u32((uint32_t*)workspace, p.total / 4, 0u, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Points the decode arguments at the plan's regions of the workspace ws; the
// completion counters go to flags, or to the plan's own region when flags is
// NULL.
void bind_workspace(const Plan& p, char* ws, uint32_t* flags, kvs::PartialArgs* a, kvs::CombineArgs* c) {
  a->ws_m = (float*)(ws + p.off_m); a->ws_l = (float*)(ws + p.off_l);
  a->ws_o = (float*)(ws + p.off_o); a->ws_e = (float*)(ws + p.off_e);
  a->ws_pid = (int*)(ws + p.off_pid); a->ws_time = (float*)(ws + p.off_time);
  a->ws_w = (float*)(ws + p.off_w);
  a->pair_flag = flags ? flags : (uint32_t*)(ws + p.off_cnt);
  a->rates = (const float*)(ws + p.off_rates);
  c->lws[0] = ws;
}

// Shared argument checks and setup of the two decode phases.
int decode_setup(const kvs_geom* g, const void* q, const void* k_cache, const void* v_cache,
                 const float* k_scale, const float* v_scale, const int32_t* pos_of_slot,
                 const int32_t* cur_pos, const uint32_t* keep_mask, void* out, float* mass_accum,
                 void* workspace, size_t workspace_bytes, Plan* plan, kvs::PartialArgs* a,
                 kvs::CombineArgs* c, int* kv) {
  int st = check_geom(g);
  if (st) return st;
  const bool fp8 = g->kv_dtype == KVS_FP8_E4M3;
  if (!q || !k_cache || !v_cache || !cur_pos || !out || !workspace) return KVS_EINVAL;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return KVS_EINVAL;
  if ((g->ring != 0) != (pos_of_slot != nullptr)) return KVS_EINVAL;
  if (keep_mask && g->window > 0) return KVS_EINVAL;
  const void* ptrs[] = {q, k_cache, v_cache, k_scale, v_scale, pos_of_slot, cur_pos, keep_mask, out, mass_accum, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  const Plan p = make_plan(g);
  if (p.lds_partial > kLdsMaxBytes) return KVS_ENOTIMPL;  // partition bookkeeping beyond LDS
  if (workspace_bytes < p.total) return KVS_EWS;
  *plan = p;
  *a = kvs::PartialArgs{};
  *c = kvs::CombineArgs{};
  a->q = q; a->k = k_cache; a->v = v_cache; a->ks = k_scale; a->vs = v_scale;
  a->pos_of_slot = pos_of_slot; a->cur_pos = cur_pos; a->keep = keep_mask;
  bind_workspace(p, (char*)workspace, nullptr, a, c);
  a->out = out;
  a->B = g->batch; a->Hq = g->n_q_heads; a->Hkv = g->n_kv_heads; a->G = p.G; a->C = g->capacity;
  a->NT = p.NT; a->window = g->window; a->nbmax = g->n_blocks_max;
  a->kwords = (g->n_blocks_max + 31) / 32; a->tpp = p.tpp; a->nparts = p.nparts;
  a->dyn = g->deterministic ? 0 : 1; a->tl_cap = p.tl_cap; a->adapt = p.adapt;
  a->scale_log2 = g->softmax_scale * 1.4426950408889634f;
  c->n_layers = 1; c->layers_per_chunk = 1;
  c->off_w = p.off_w; c->off_e = p.off_e; c->off_pid = p.off_pid;
  c->off_time = p.off_time; c->off_rates = p.off_rates;
  c->cur_pos = cur_pos; c->n_wg = p.n_wg;
  c->mass = mass_accum;
  c->B = g->batch; c->Hq = g->n_q_heads; c->Hkv = g->n_kv_heads; c->C = g->capacity; c->NT = p.NT;
  c->nbmax = g->n_blocks_max; c->tpp = p.tpp; c->nparts = p.nparts; c->window = g->window;
  c->n_mass_chunks = (p.NT + 255) / 256;
  *kv = fp8 ? kvs::KV_FP8 : g->kv_dtype == KVS_BF16 ? kvs::KV_BF16 : kvs::KV_F32;
  return KVS_OK;
}

}  // namespace

extern "C" {

#define KVS_DECODE_ARGS                                                                          \
  const kvs_geom *g, const void *q, const void *k_cache, const void *v_cache,                     \
      const float *k_scale, const float *v_scale, const int32_t *pos_of_slot,                     \
      const int32_t *cur_pos, const uint32_t *keep_mask, void *out, float *mass_accum,            \
      void *workspace, size_t workspace_bytes, void *stream
#define KVS_DECODE_SETUP                                                                         \
  Plan p;                                                                                        \
  kvs::PartialArgs a;                                                                            \
  kvs::CombineArgs c;                                                                            \
  int kv;                                                                                        \
  int st = decode_setup(g, q, k_cache, v_cache, k_scale, v_scale, pos_of_slot, cur_pos,           \
                        keep_mask, out, mass_accum, workspace, workspace_bytes, &p, &a, &c, &kv); \
  if (st) return st;                                                                             \
  hipStream_t s = (hipStream_t)stream;

int kvs_decode_partial(KVS_DECODE_ARGS) {
  KVS_DECODE_SETUP
  return hip_status(kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, g->ring != 0,
                                        p.lds_partial, s));
}

int kvs_decode_combine(KVS_DECODE_ARGS) {
  KVS_DECODE_SETUP
  (void)kv;
  return hip_status(kvs::launch_combine(c, g->ring != 0, s));
}

int kvs_decode_attn_scored(KVS_DECODE_ARGS) {
  KVS_DECODE_SETUP
  hipError_t e = kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, g->ring != 0,
                                     p.lds_partial, s);
  if (e != hipSuccess) return KVS_EHIP;
  return hip_status(kvs::launch_combine(c, g->ring != 0, s));
}

int kvs_decode_attn_profiled(const kvs_geom* g, const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* pos_of_slot,
                             const int32_t* cur_pos, const uint32_t* keep_mask, void* out,
                             float* mass_accum, float* head_mass, float* mass_max, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if ((head_mass && !aligned16(head_mass)) || (mass_max && !aligned16(mass_max))) return KVS_EALIGN;
  Plan p;
  kvs::PartialArgs a;
  kvs::CombineArgs c;
  int kv;
  int st = decode_setup(g, q, k_cache, v_cache, k_scale, v_scale, pos_of_slot, cur_pos, keep_mask, out,
                        mass_accum, workspace, workspace_bytes, &p, &a, &c, &kv);
  if (st) return st;
  c.head_mass = head_mass;
  c.mass_max = mass_max;
  const bool scored = mass_accum || head_mass || mass_max;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvs::launch_partial(kv, g->head_dim, a, scored, g->ring != 0, p.lds_partial, s);
  if (e != hipSuccess) return KVS_EHIP;
  return hip_status(kvs::launch_combine(c, g->ring != 0, s));
}

}  // extern "C"

namespace {

// The fused-append arguments (after decode_setup has checked the rest).
int append_args(const kvs_geom* g, const void* k_new, const void* v_new, int32_t src_dtype,
                kvs::PartialArgs* a) {
  if (src_dtype != KVS_F32 && src_dtype != KVS_BF16) return KVS_EDTYPE;
  if (g->kv_dtype != KVS_FP8_E4M3 && src_dtype != g->kv_dtype) return KVS_EDTYPE;
  if (!k_new || !v_new) return KVS_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new)) return KVS_EALIGN;
  a->app_k = k_new;
  a->app_v = v_new;
  a->app_bf16 = src_dtype == KVS_BF16;
  return KVS_OK;
}

}  // namespace

extern "C" {

#define KVS_APPEND_DECODE_ARGS                                                                   \
  const kvs_geom *g, const void *k_new, const void *v_new, int32_t src_dtype, const void *q,     \
      void *k_cache, void *v_cache, float *k_scale, float *v_scale, int32_t *pos_of_slot,         \
      const int32_t *cur_pos, const uint32_t *keep_mask, void *out, float *mass_accum,            \
      void *workspace, size_t workspace_bytes, void *stream
#define KVS_APPEND_DECODE_SETUP                                                                  \
  KVS_DECODE_SETUP                                                                               \
  st = append_args(g, k_new, v_new, src_dtype, &a);                                              \
  if (st) return st;

int kvs_append_decode_partial(KVS_APPEND_DECODE_ARGS) {
  KVS_APPEND_DECODE_SETUP
  return hip_status(kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, g->ring != 0,
                                        p.lds_partial, s));
}

int kvs_append_decode_attn(KVS_APPEND_DECODE_ARGS) {
  KVS_APPEND_DECODE_SETUP
  hipError_t e = kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, g->ring != 0,
                                     p.lds_partial, s);
  if (e != hipSuccess) return KVS_EHIP;
  return hip_status(kvs::launch_combine(c, g->ring != 0, s));
}

int kvs_decode_attn_tap(const kvs_geom* g, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* pos_of_slot,
                        const int32_t* cur_pos, const uint32_t* keep_mask, void* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  float* mass_accum = nullptr;
  KVS_DECODE_SETUP
  (void)c;
  return hip_status(kvs::launch_partial(kv, g->head_dim, a, true, g->ring != 0, p.lds_partial, s));
}

int kvs_append_decode_attn_tap(const kvs_geom* g, const void* k_new, const void* v_new, int32_t src_dtype,
                               const void* q, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                               int32_t* pos_of_slot, const int32_t* cur_pos, const uint32_t* keep_mask,
                               void* out, void* workspace, size_t workspace_bytes, void* stream) {
  float* mass_accum = nullptr;
  KVS_APPEND_DECODE_SETUP
  (void)c;
  return hip_status(kvs::launch_partial(kv, g->head_dim, a, true, g->ring != 0, p.lds_partial, s));
}

}  // extern "C"

namespace {

// Checks and arguments of kvs_tap_masses; *parallel: the layer-parallel
// combine applies.
int tap_setup(const kvs_geom* g, void* const* workspaces, int32_t n_layers, size_t workspace_bytes,
              const int32_t* cur_pos, float* mass_accum, float* head_mass, float* mass_max,
              kvs::CombineArgs* cp, bool* parallel) {
  int st = check_geom(g);
  if (st) return st;
  if (n_layers < 1 || n_layers > kvs::kMaxTapLayers || !workspaces || !cur_pos) return KVS_EINVAL;
  const void* ptrs[] = {cur_pos, mass_accum, head_mass, mass_max};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return KVS_EALIGN;
  const Plan p = make_plan(g);
  if (workspace_bytes < p.total) return KVS_EWS;
  kvs::CombineArgs& c = *cp;
  c = kvs::CombineArgs{};
  for (int l = 0; l < n_layers; ++l) {
    if (!workspaces[l]) return KVS_EINVAL;
    if (!aligned16(workspaces[l])) return KVS_EALIGN;
    c.lws[l] = (const char*)workspaces[l];
  }
  c.n_layers = n_layers;
  const size_t per_layer = kvs::combine_layer_floats(g->n_q_heads, g->n_kv_heads, p.nparts) * 4;
  const int fit = (int)(kvs::kCombineLdsBytes / per_layer);
  c.layers_per_chunk = fit < 1 ? 1 : (fit < n_layers ? fit : n_layers);
  c.off_w = p.off_w; c.off_e = p.off_e; c.off_pid = p.off_pid;
  c.off_time = p.off_time; c.off_rates = p.off_rates;
  c.n_wg = p.n_wg; c.cur_pos = cur_pos;
  c.mass = mass_accum; c.head_mass = head_mass; c.mass_max = mass_max;
  c.B = g->batch; c.Hq = g->n_q_heads; c.Hkv = g->n_kv_heads; c.C = g->capacity; c.NT = p.NT;
  c.nbmax = g->n_blocks_max; c.tpp = p.tpp; c.nparts = p.nparts; c.window = g->window;
  c.n_mass_chunks = (p.NT + 255) / 256;
  // without per-head masses, and when every layer's tables fit the LDS at
  // once, the layers are summed in parallel (same values, bit for bit)
  *parallel = !head_mass && kvs::combine_layers_lds_bytes(g->n_q_heads, g->n_kv_heads, p.nparts, n_layers,
                                                          g->ring != 0) <= kvs::kCombineLdsBytes;
  return KVS_OK;
}

hipError_t launch_tap(const kvs::CombineArgs& c, bool parallel, bool ring, hipStream_t s) {
  return parallel ? kvs::launch_combine_layers(c, ring, s) : kvs::launch_combine(c, ring, s);
}


}  // namespace

extern "C" {

int kvs_tap_masses(const kvs_geom* g, void* const* workspaces, int32_t n_layers, size_t workspace_bytes,
                   const int32_t* cur_pos, float* mass_accum, float* head_mass, float* mass_max, void* stream) {
  kvs::CombineArgs c;
  bool parallel = false;
  const int st = tap_setup(g, workspaces, n_layers, workspace_bytes, cur_pos, mass_accum, head_mass, mass_max, &c,
                           &parallel);
  if (st) return st;
  return hip_status(launch_tap(c, parallel, g->ring != 0, (hipStream_t)stream));
}

int kvs_reattend_blocks(const kvs_geom* g, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* cur_pos,
                        const int32_t* block_ids, const int32_t* n_ids, int32_t ids_stride, void* out,
                        float* mass_accum, void* workspace, size_t workspace_bytes, void* stream) {
  if (!g) return KVS_EINVAL;
  if (g->ring != 0 || g->window != 0) return KVS_EINVAL;  // the list replaces masks and windows
  if (!block_ids || !n_ids || ids_stride < 1) return KVS_EINVAL;
  if (!aligned16(block_ids) || !aligned16(n_ids)) return KVS_EALIGN;
  Plan p;
  kvs::PartialArgs a;
  kvs::CombineArgs c;
  int kv;
  int st = decode_setup(g, q, k_cache, v_cache, k_scale, v_scale, nullptr, cur_pos, nullptr, out,
                        mass_accum, workspace, workspace_bytes, &p, &a, &c, &kv);
  if (st) return st;
  a.ids = block_ids;
  a.n_ids = n_ids;
  a.ids_stride = ids_stride;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, false, p.lds_partial, s);
  if (e != hipSuccess) return KVS_EHIP;
  return hip_status(kvs::launch_combine(c, false, s));
}

}  // extern "C"

namespace {

int sidecar_check(const float* mass_accum, const float* attended, const float* ema, const float* cum,
                  const float* traj, int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step,
                  float alpha) {
  if (batch < 1 || n_blocks_max < 1 || traj_cap < 1 || step < 0) return KVS_EINVAL;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return KVS_EINVAL;
  if (!mass_accum || !attended || !ema || !cum) return KVS_EINVAL;
  const void* ptrs[] = {mass_accum, attended, ema, cum, traj};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  return KVS_OK;
}

}  // namespace

extern "C" {

int kvs_update_sidecar(float* mass_accum, float* attended, float* ema, float* cum, float* traj,
                       int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step,
                       float alpha, void* stream) {
  const int st = sidecar_check(mass_accum, attended, ema, cum, traj, batch, n_blocks_max, traj_cap, step, alpha);
  if (st) return st;
  return hip_status(kvs::launch_sidecar(mass_accum, attended, ema, cum, traj, batch, n_blocks_max,
                                        traj_cap, step, alpha, (hipStream_t)stream));
}

namespace {
struct SnapPlan {
  int tpp, nparts;
  size_t off_part, off_m, off_l, total;
};
// Partitions of the prefill scoring passes: one round of workgroups of 4
// waves, about 1024 for bf16 keys (four per CU at up to 128 VGPRs) and 512 for
// FP8 keys (two per CU at up to 256 VGPRs).
SnapPlan snap_plan(const kvs_geom* g, int window) {
  SnapPlan p{};
  const int NT = g->capacity / kTileSlots;
  const int pairs = g->batch * g->n_kv_heads;
  const int target = g->kv_dtype == KVS_FP8_E4M3 ? 512 : 1024;
  int pt = (target + pairs - 1) / pairs;
  if (pt < 1) pt = 1;
  p.tpp = (NT + pt - 1) / pt;
  if (p.tpp < 1) p.tpp = 1;
  p.nparts = (NT + p.tpp - 1) / p.tpp;
  const size_t cols = (size_t)g->batch * g->n_kv_heads * window * (g->n_q_heads / g->n_kv_heads);
  p.off_part = 0;
  p.off_m = round256(cols * p.nparts * 2 * 4);
  p.off_l = round256(p.off_m + cols * 4);
  p.total = round256(p.off_l + cols * 4);
  return p;
}
}  // namespace

int kvs_snapkv_workspace_bytes(const kvs_geom* g, int32_t window, size_t* bytes) {
  int st = check_geom(g);
  if (st) return st;
  if (!bytes || window < 1) return KVS_EINVAL;
  *bytes = snap_plan(g, window).total;
  return KVS_OK;
}

int kvs_snapkv_scores(const kvs_geom* g, const void* q_window, int32_t window, const void* k_cache,
                      const float* k_scale, const int32_t* n_prompt, float* token_score, float* block_score,
                      int32_t pool_kernel, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (g->ring != 0) return KVS_EINVAL;
  if (g->kv_dtype == KVS_F32) return KVS_ENOTIMPL;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (window < 1 || pool_kernel < 1 || pool_kernel % 2 == 0 || pool_kernel > 33) return KVS_EINVAL;
  // a lane's 16 columns hold whole heads only when G divides 16
  if (window * G > 128 || 16 % G != 0) return KVS_ENOTIMPL;
  const bool fp8 = g->kv_dtype == KVS_FP8_E4M3;
  if (!q_window || !k_cache || !n_prompt || !token_score || !workspace) return KVS_EINVAL;
  if (fp8 != (k_scale != nullptr)) return KVS_EINVAL;
  const void* ptrs[] = {q_window, k_cache, k_scale, n_prompt, token_score, block_score, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  const SnapPlan p = snap_plan(g, window);
  if (workspace_bytes < p.total) return KVS_EWS;
  char* ws = (char*)workspace;
  kvs::SnapArgs a{};
  a.q = q_window; a.k = k_cache; a.ks = k_scale; a.n_prompt = n_prompt;
  a.part_ml = (float*)(ws + p.off_part); a.col_m = (float*)(ws + p.off_m); a.col_l = (float*)(ws + p.off_l);
  a.token_score = token_score; a.block_score = block_score;
  a.B = g->batch; a.Hq = g->n_q_heads; a.Hkv = g->n_kv_heads; a.G = G; a.C = g->capacity;
  a.NT = g->capacity / kTileSlots; a.nbmax = g->n_blocks_max; a.W = window; a.tpp = p.tpp;
  a.nparts = p.nparts; a.pool = pool_kernel;
  a.scale_log2 = g->softmax_scale * 1.4426950408889634f;
  return hip_status(kvs::launch_snap(fp8 ? kvs::KV_FP8 : kvs::KV_BF16, g->head_dim, a, (hipStream_t)stream));
}

int kvs_compact_blocks(const kvs_geom* g, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const int32_t* keep_ids, const int32_t* n_keep, int32_t ids_stride,
                       const kvs_block_table* tables, int32_t n_tables, void* stream) {
  int st = check_geom(g);
  if (st) return st;
  if (g->ring != 0) return KVS_EINVAL;
  const bool fp8 = g->kv_dtype == KVS_FP8_E4M3;
  if (!k_cache || !v_cache || !keep_ids || !n_keep || ids_stride < 1) return KVS_EINVAL;
  if (fp8 != (k_scale != nullptr) || fp8 != (v_scale != nullptr)) return KVS_EINVAL;
  if (n_tables < 0 || n_tables > kvs::kMaxCompactTables || (n_tables > 0 && !tables)) return KVS_EINVAL;
  const void* ptrs[] = {k_cache, v_cache, k_scale, v_scale, keep_ids, n_keep};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  kvs::CompactArgs a{};
  for (int t = 0; t < n_tables; ++t) {
    if (!tables[t].data || tables[t].rows < 1) return KVS_EINVAL;
    if (!aligned16(tables[t].data)) return KVS_EALIGN;
    a.tables[t] = tables[t].data;
    a.table_rows[t] = tables[t].rows;
  }
  a.n_tables = n_tables;
  a.k = k_cache; a.v = v_cache; a.ks = k_scale; a.vs = v_scale; a.ids = keep_ids; a.n_keep = n_keep;
  a.B = g->batch; a.Hkv = g->n_kv_heads; a.C = g->capacity; a.NT = g->capacity / kTileSlots;
  a.nbmax = g->n_blocks_max; a.ids_stride = ids_stride;
  a.tile_bytes = kTileSlots * g->head_dim * elem_bytes(g->kv_dtype);
  return hip_status(kvs::launch_compact(a, (hipStream_t)stream));
}

int kvs_update_counters(const float* attended, const float* ema, int32_t* hot_count, int32_t* cold_turns,
                        float* traj, int32_t batch, int32_t n_blocks_max, int32_t traj_cap, float hot_theta,
                        float cold_theta, int32_t cold_limit, void* stream) {
  if (batch < 1 || n_blocks_max < 1 || cold_limit < 0) return KVS_EINVAL;
  if (!isfinite(hot_theta) || !isfinite(cold_theta)) return KVS_EINVAL;
  if (hot_count && !attended) return KVS_EINVAL;
  if (cold_turns && !ema) return KVS_EINVAL;
  if (traj && (!cold_turns || traj_cap < 1)) return KVS_EINVAL;
  const void* ptrs[] = {attended, ema, hot_count, cold_turns, traj};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  if (!hot_count && !cold_turns) return KVS_OK;
  kvs::CounterArgs a{};
  a.attended = attended; a.ema = ema; a.hot_count = hot_count; a.cold_turns = cold_turns; a.traj = traj;
  a.B = batch; a.nbmax = n_blocks_max; a.traj_cap = traj_cap; a.cold_limit = cold_limit;
  a.hot_theta = hot_theta; a.cold_theta = cold_theta;
  return hip_status(kvs::launch_counters(a, (hipStream_t)stream));
}

int kvs_filter_blocks(const float* score, const uint32_t* alive, const int32_t* cur_pos, int32_t batch,
                      int32_t n_blocks_max, float theta, int32_t* ids, int32_t* n_ids, int32_t ids_stride,
                      void* stream) {
  if (batch < 1 || n_blocks_max < 1 || ids_stride < 1 || isnan(theta)) return KVS_EINVAL;
  if (!score || !cur_pos || !ids || !n_ids) return KVS_EINVAL;
  const void* ptrs[] = {score, alive, cur_pos, ids, n_ids};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  kvs::FilterArgs a{};
  a.score = score; a.alive = alive; a.cur_pos = cur_pos; a.ids = ids; a.n_ids = n_ids;
  a.B = batch; a.nbmax = n_blocks_max; a.kwords = (n_blocks_max + 31) / 32; a.ids_stride = ids_stride;
  a.theta = theta;
  return hip_status(kvs::launch_filter(a, (hipStream_t)stream));
}

int kvs_select_blocks(const float* score, const uint32_t* alive, const int32_t* cur_pos,
                      int32_t batch, int32_t n_blocks_max, int32_t budget_blocks,
                      int32_t recent_tokens, int32_t sink_tokens, uint32_t* keep_mask,
                      int32_t* sel_ids, int32_t* n_sel, void* stream) {
  if (batch < 1 || n_blocks_max < 1) return KVS_EINVAL;
  if (budget_blocks < 0 || recent_tokens < 1 || sink_tokens < 0) return KVS_EINVAL;
  if (!score || !cur_pos || !keep_mask || !sel_ids || !n_sel) return KVS_EINVAL;
  const void* ptrs[] = {score, alive, cur_pos, keep_mask, sel_ids, n_sel};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  kvs::SelectArgs a{};
  a.score = score; a.alive = alive; a.cur_pos = cur_pos; a.keep = keep_mask; a.sel_ids = sel_ids;
  a.n_sel = n_sel; a.B = batch; a.nbmax = n_blocks_max; a.kwords = (n_blocks_max + 31) / 32;
  a.budget = budget_blocks; a.recent = recent_tokens; a.sinks = sink_tokens;
  return hip_status(kvs::launch_select(a, (hipStream_t)stream));
}

int kvs_stream_read(const void* buf, size_t bytes, uint32_t* sums, int32_t workgroups, void* stream) {
  if (!buf || !sums || workgroups < 1 || workgroups > 65536) return KVS_EINVAL;
  if (bytes == 0 || bytes % 1024 != 0 || (size_t)workgroups > bytes / 1024) return KVS_EINVAL;
  if (!aligned16(buf) || !aligned16(sums)) return KVS_EALIGN;
  return hip_status(kvs::launch_stream_read(buf, bytes, sums, workgroups, (hipStream_t)stream));
}

}  // extern "C"

namespace {

int sidecar_select_setup(float* mass_accum, float* attended, float* ema, float* cum, float* traj,
                         int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step, float alpha,
                         int32_t score_source, const uint32_t* alive, const int32_t* cur_pos,
                         int32_t budget_blocks, int32_t recent_tokens, int32_t sink_tokens, uint32_t* keep_mask,
                         int32_t* sel_ids, int32_t* n_sel, kvs::SelectArgs* out) {
  if (batch < 1 || n_blocks_max < 1 || traj_cap < 1 || step < 0) return KVS_EINVAL;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return KVS_EINVAL;
  if (score_source < KVS_SCORE_CUMULATIVE || score_source > KVS_SCORE_ATTENDED) return KVS_EINVAL;
  if (budget_blocks < 0 || recent_tokens < 1 || sink_tokens < 0) return KVS_EINVAL;
  if (!mass_accum || !attended || !ema || !cum || !cur_pos || !keep_mask || !sel_ids || !n_sel)
    return KVS_EINVAL;
  const void* ptrs[] = {mass_accum, attended, ema, cum, traj, alive, cur_pos, keep_mask, sel_ids, n_sel};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KVS_EALIGN;
  kvs::SelectArgs a{};
  a.alive = alive; a.cur_pos = cur_pos; a.keep = keep_mask; a.sel_ids = sel_ids; a.n_sel = n_sel;
  a.B = batch; a.nbmax = n_blocks_max; a.kwords = (n_blocks_max + 31) / 32;
  a.budget = budget_blocks; a.recent = recent_tokens; a.sinks = sink_tokens;
  a.mass = mass_accum; a.att = attended; a.ema = ema; a.cum = cum; a.traj = traj;
  a.traj_cap = traj_cap; a.slot = (int)(step % traj_cap); a.alpha = alpha; a.score_src = score_source;
  *out = a;
  return KVS_OK;
}

}  // namespace

extern "C" {

int kvs_update_sidecar_select(float* mass_accum, float* attended, float* ema, float* cum, float* traj,
                              int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step,
                              float alpha, int32_t score_source, const uint32_t* alive,
                              const int32_t* cur_pos, int32_t budget_blocks, int32_t recent_tokens,
                              int32_t sink_tokens, uint32_t* keep_mask, int32_t* sel_ids, int32_t* n_sel,
                              void* stream) {
  kvs::SelectArgs a;
  const int st = sidecar_select_setup(mass_accum, attended, ema, cum, traj, batch, n_blocks_max, traj_cap, step,
                                      alpha, score_source, alive, cur_pos, budget_blocks, recent_tokens,
                                      sink_tokens, keep_mask, sel_ids, n_sel, &a);
  if (st) return st;
  return hip_status(kvs::launch_select(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The arguments of layer l's partial launch in kvs_decode_step.
int step_layer_setup(const kvs_geom* g, const kvs_layer_bufs& L, int32_t src_dtype, const int32_t* cur_pos,
                     const uint32_t* keep_mask, size_t workspace_bytes, Plan* p, kvs::PartialArgs* a, int* kv) {
  kvs::CombineArgs unused;
  int st = decode_setup(g, L.q, L.k_cache, L.v_cache, L.k_scale, L.v_scale, L.pos_of_slot, cur_pos, keep_mask, L.out,
                        nullptr, L.workspace, workspace_bytes, p, a, &unused, kv);
  if (st) return st;
  if ((L.k_new == nullptr) != (L.v_new == nullptr)) return KVS_EINVAL;
  return L.k_new ? append_args(g, L.k_new, L.v_new, src_dtype, a) : KVS_OK;
}


// The end of a step: the layers' masses added into mass_accum, then the turn
// (if any) closed. Without selection, and when the layer-parallel combine
// applies, the side-car update runs in the combine's launch (the same
// arithmetic on the same masses: bit for bit the two calls).
struct CloseStep {
  kvs::CombineArgs c;
  bool parallel = false;
  kvs::SelectArgs sa{};
};

int close_setup(const kvs_geom* g, void* const* workspaces, int32_t n_layers, size_t workspace_bytes,
                const int32_t* cur_pos, float* mass_accum, const kvs_turn_args* turn, CloseStep* cs) {
  int st = tap_setup(g, workspaces, n_layers, workspace_bytes, cur_pos, mass_accum, nullptr, nullptr, &cs->c,
                     &cs->parallel);
  if (st) return st;
  if (!turn) return KVS_OK;
  if (turn->select != 0 && turn->select != 1) return KVS_EINVAL;
  if (turn->select)
    return sidecar_select_setup(mass_accum, turn->attended, turn->ema, turn->cum, turn->traj, g->batch,
                                g->n_blocks_max, turn->traj_cap, turn->step, turn->alpha, turn->score_source,
                                turn->alive, cur_pos, turn->budget_blocks, turn->recent_tokens, turn->sink_tokens,
                                turn->keep_out, turn->sel_ids, turn->n_sel, &cs->sa);
  st = sidecar_check(mass_accum, turn->attended, turn->ema, turn->cum, turn->traj, g->batch, g->n_blocks_max,
                     turn->traj_cap, turn->step, turn->alpha);
  if (st) return st;
  if (cs->parallel) {
    kvs::CombineArgs& c = cs->c;
    c.sc_att = turn->attended;
    c.sc_ema = turn->ema;
    c.sc_cum = turn->cum;
    c.sc_traj = turn->traj;
    c.sc_traj_cap = turn->traj_cap;
    c.sc_slot = (int)(turn->step % turn->traj_cap);
    c.sc_alpha = turn->alpha;
  }
  return KVS_OK;
}

int close_launch(const kvs_geom* g, const CloseStep& cs, const kvs_turn_args* turn, hipStream_t s) {
  if (launch_tap(cs.c, cs.parallel, g->ring != 0, s) != hipSuccess) return KVS_EHIP;
  if (!turn || cs.c.sc_att) return hip_status(hipGetLastError());
  if (turn->select) return hip_status(kvs::launch_select(cs.sa, s));
  return hip_status(kvs::launch_sidecar(cs.c.mass, turn->attended, turn->ema, turn->cum, turn->traj, g->batch,
                                        g->n_blocks_max, turn->traj_cap, turn->step, turn->alpha, s));
}

}  // namespace

extern "C" {

// One whole decode step: every check first (layer by layer), then the
// launches, each layer's arguments set up again (a few integer operations)
// rather than kept, so the call needs no storage.
int kvs_decode_step(const kvs_geom* g, int32_t n_layers, const kvs_layer_bufs* layers, int32_t src_dtype,
                    const int32_t* cur_pos, const uint32_t* keep_mask, size_t workspace_bytes,
                    float* mass_accum, const kvs_turn_args* turn, void* stream) {
  if (!g || !layers || n_layers < 1 || n_layers > kvs::kMaxTapLayers) return KVS_EINVAL;
  void* ws[kvs::kMaxTapLayers];
  for (int l = 0; l < n_layers; ++l) {
    Plan p;
    kvs::PartialArgs a;
    int kv;
    const int st = step_layer_setup(g, layers[l], src_dtype, cur_pos, keep_mask, workspace_bytes, &p, &a, &kv);
    if (st) return st;
    ws[l] = layers[l].workspace;
  }
  // without mass_accum the block sums stay in the workspaces (for a later
  // kvs_tap_masses) and there is no turn to close
  if (!mass_accum && turn) return KVS_EINVAL;
  CloseStep cs;
  if (mass_accum) {
    const int st = close_setup(g, ws, n_layers, workspace_bytes, cur_pos, mass_accum, turn, &cs);
    if (st) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  for (int l = 0; l < n_layers; ++l) {
    Plan p;
    kvs::PartialArgs a;
    int kv;
    step_layer_setup(g, layers[l], src_dtype, cur_pos, keep_mask, workspace_bytes, &p, &a, &kv);
    if (kvs::launch_partial(kv, g->head_dim, a, true, g->ring != 0, p.lds_partial, s) != hipSuccess) return KVS_EHIP;
  }
  if (!mass_accum) return KVS_OK;
  return close_launch(g, cs, turn, s);
}

int kvs_close_step(const kvs_geom* g, void* const* workspaces, int32_t n_layers, size_t workspace_bytes,
                   const int32_t* cur_pos, float* mass_accum, const kvs_turn_args* turn, void* stream) {
  if (!mass_accum || !turn) return KVS_EINVAL;
  CloseStep cs;
  const int st = close_setup(g, workspaces, n_layers, workspace_bytes, cur_pos, mass_accum, turn, &cs);
  if (st) return st;
  return close_launch(g, cs, turn, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kvs_decode_attn_scored_noalloc: the decode workspace in a static device
// array instead of a caller buffer.
// ---------------------------------------------------------------------------
namespace {

// The array's first part holds the completion counters, at the same place for
// every geometry: each call leaves the counters it used at zero (its merging
// workgroups reset them), so they are zero at the start of every call,
// whatever geometry the previous call had. The rest holds one call's
// workspace regions (partials, block records, partition map, merge weights,
// clock records and the per-class rates, which are sanitised on read).
constexpr size_t kNoallocFlagBytes = 64 * 1024;  // counter region: B * Hkv * partitions words
constexpr size_t kNoallocWsBytes = (size_t)KVS_NOALLOC_SCRATCH_BYTES - kNoallocFlagBytes;
constexpr int kMaxDevices = 64;

// One copy per GPU, zero when the code object is loaded; held until the
// process ends. Host code never uses its name as an address: the device
// address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) __attribute__((used)) unsigned char scratch[KVS_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];  // device address of scratch, per device (nullptr: not set up)

// The current device's scratch address. At its first use on a device (that
// device current) the address is looked up and the flag region is cleared
// once more on the caller's stream (a fill kernel, no memset node).
int scratch_of_current_device(hipStream_t s, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVS_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return KVS_EHIP;
    if (kvs::launch_fill_u32((uint32_t*)ptr, kNoallocFlagBytes / 4, 0u, s) != hipSuccess) return KVS_EHIP;
    g_scratch[dev] = (char*)ptr;
  }
  *out = g_scratch[dev];
  return KVS_OK;
}

}  // namespace

extern "C" {

int kvs_decode_attn_scored_noalloc(const kvs_geom* g, const void* q, const void* k_cache, const void* v_cache,
                                   const float* k_scale, const float* v_scale, const int32_t* pos_of_slot,
                                   const int32_t* cur_pos, const uint32_t* keep_mask, void* out,
                                   float* mass_accum, void* stream) {
  Plan p;
  kvs::PartialArgs a;
  kvs::CombineArgs c;
  int kv;
  // every argument check first, against a stand-in workspace address of the
  // largest size (nothing is launched or dereferenced before the rebinding)
  void* const stand_in = (void*)(uintptr_t)256;
  int st = decode_setup(g, q, k_cache, v_cache, k_scale, v_scale, pos_of_slot, cur_pos, keep_mask, out,
                        mass_accum, stand_in, kNoallocWsBytes, &p, &a, &c, &kv);
  if (st == KVS_EWS) return KVS_ESCRATCH;
  if (st) return st;
  if ((size_t)g->batch * g->n_kv_heads * p.nparts * 4 > kNoallocFlagBytes) return KVS_ESCRATCH;
  hipStream_t s = (hipStream_t)stream;
  char* base = nullptr;
  st = scratch_of_current_device(s, &base);
  if (st) return st;
  bind_workspace(p, base + kNoallocFlagBytes, (uint32_t*)base, &a, &c);
  hipError_t e = kvs::launch_partial(kv, g->head_dim, a, mass_accum != nullptr, g->ring != 0, p.lds_partial, s);
  if (e != hipSuccess) return KVS_EHIP;
  return hip_status(kvs::launch_combine(c, g->ring != 0, s));
}

}  // extern "C"
