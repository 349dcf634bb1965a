/*
 * kvs.h -- C ABI of libkvs: scored decode attention over a KV cache, with the
 * per-(sequence, 16-token block) attention-mass tap, the block side-car and
 * heavy-hitter block selection, for AMD Instinct MI355X (gfx950).
 *
 * Every call is asynchronous on the HIP stream it is given (``stream`` is a
 * hipStream_t; NULL means the null stream). The library never allocates,
 * frees or synchronises: the caller owns every buffer. Unless stated
 * otherwise a pointer argument is a DEVICE pointer and must be 16-byte
 * aligned. Calls return KVS_OK (0) or a negative kvs_status; when a call
 * returns an error nothing has been launched. Calls are re-entrant and may be
 * made from several host threads. The only process-wide state is that of
 * kvs_decode_attn_scored_noalloc: a static device scratch array per GPU and
 * the host table of its per-device addresses (guarded by a mutex); every
 * other call works on caller-owned buffers only.
 *
 * Terms. B sequences; Hq query heads and Hkv KV heads with G = Hq / Hkv
 * query heads reading each KV head (query head h reads KV head h / G); head
 * dimension d; C slots per sequence; a block is 16 consecutive absolute
 * positions (block b = position / 16); NBmax = n_blocks_max block entries per
 * sequence in every per-block array; W = ceil(NBmax / 32) mask words.
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef KVS_API
#define KVS_API __attribute__((visibility("default")))
#endif

/* Status codes. */
typedef enum {
  KVS_OK = 0,
  KVS_EINVAL = -1,   /* bad geometry or argument, or a forbidden combination  */
  KVS_EDTYPE = -2,   /* unsupported dtype or dtype/head-dim combination        */
  KVS_EALIGN = -3,   /* a pointer is not 16-byte aligned                       */
  KVS_EWS = -4,      /* workspace smaller than kvs_decode_workspace_bytes      */
  KVS_EHIP = -5,     /* the HIP runtime refused a launch                       */
  KVS_ENOTIMPL = -6, /* a combination the library does not provide             */
  KVS_ESCRATCH = -7  /* geometry needs more than KVS_NOALLOC_SCRATCH_BYTES     */
} kvs_status;

typedef enum {
  KVS_F32 = 0,
  KVS_BF16 = 1,
  KVS_FP8_E4M3 = 2   /* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits */
} kvs_dtype;

/*
 * Cache geometry. It is fixed when the cache is allocated and must be passed
 * unchanged to every call on that cache: element size, layout and scale
 * arrays all follow from it (Context Optimization, "FP8 KV Cache / Flag
 * Ordering": the FP8 and window choices have to be made before the buffers
 * exist, or float-sized buffers end up holding FP8 data).
 *
 *   batch          B >= 1
 *   n_q_heads      Hq >= 1, a multiple of n_kv_heads, Hq / Hkv <= 16
 *   n_kv_heads     Hkv >= 1
 *   head_dim       d: 16, 64 or 128 for KVS_F32; 64 or 128 for BF16 and FP8
 *   capacity       C slots per sequence, a positive multiple of 16
 *   window         0 = unlimited; w >= 1 lets position i read only positions
 *                  i-w+1 .. i (LLM mechanics III, "1. Define the window")
 *   ring           0: slot = position (requires position < C);
 *                  1: circular cache, slot = position mod C, and the absolute
 *                  position held by each slot is kept in pos_of_slot
 *                  (Context Optimization, "Sliding Window Attention / Design";
 *                  LLM mechanics III, "5. Keep three indices separate")
 *   n_blocks_max   NBmax: entries per sequence of mass/score/side-car arrays.
 *                  Linear caches need NBmax >= C / 16; ring caches need
 *                  NBmax > (largest position ever written) / 16.
 *   kv_dtype       element type of the cache
 *   q_dtype        KVS_F32 with a KVS_F32 cache, KVS_BF16 otherwise; the
 *                  attention output has the same type
 *   softmax_scale  logit multiplier, finite and > 0 (usually 1/sqrt(d))
 *   deterministic  0: the decode kernel's waves share each partition's
 *                  tiles dynamically (fastest; the rounding of out and of
 *                  the block masses can differ in the last bits between
 *                  runs); 1: fixed tile order, results bit-identical between
 *                  runs and between scored and unscored calls
 */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t window;
  int32_t ring;
  int32_t n_blocks_max;
  int32_t kv_dtype;  /* kvs_dtype */
  int32_t q_dtype;   /* kvs_dtype */
  float softmax_scale;
  int32_t deterministic;  /* 0 or 1 */
} kvs_geom;

/*
 * Cache layout (one layer; K and V are separate buffers of the same size):
 *   K, V   [B][Hkv][C/16] tiles of 16 slots x d elements, each tile stored
 *          fragment-major so the decode kernel reads it in whole KiB runs.
 *          With element size s (4, 2 or 1 bytes), slot t (0..15) and head
 *          dimension x inside a tile live at byte
 *            K: 16*(16*(4*(x*s/64) + (x*s%64)/16) + t) + x*s%16
 *            V: with a = t/4, e = t%4, j = x/(d/16), n = x%(d/16), u = (4n+e)*s:
 *               16*(16*(4*(u/16) + a) + j) + u%16
 *          Caches are meant to be written through kvs_append_kv.
 *   k_scale, v_scale  [B][C] float     FP8 caches only: one scale per
 *                                      (sequence, slot) covering all Hkv*d
 *                                      values of that position
 *   pos_of_slot [B][C] int32           ring caches only; -1 marks an empty slot
 * kvs_cache_bytes() gives the byte sizes.
 */
KVS_API int kvs_cache_bytes(const kvs_geom* geom, size_t* kv_bytes, size_t* scale_bytes,
                    size_t* pos_bytes);

/*
 * kvs_encode_fp8 -- per-row FP8 E4M3 encoding (Context Optimization,
 * "FP8 KV Cache / How It Works": per position, scale = absmax / 240, each
 * value divided by it, clipped to +-448 and rounded to an 8-bit code, the
 * scale kept apart from the codes).
 *
 * For each row r of ``src`` ([n_rows][row_len], KVS_F32 or KVS_BF16, bf16
 * widened exactly): a = max |x|; s = a / 240 rounded once to float32;
 * code = E4M3(x / s), the quotient rounded once to float32, then rounded to
 * the nearest E4M3 value with ties to even after clipping to +-448; the sign
 * is kept (-0 encodes as 0x80). A row with a == 0 gets s = 0 and all codes 0.
 * Outputs: codes [n_rows][row_len] uint8, scales [n_rows] float. Non-finite
 * inputs are outside the contract (the result is unspecified, no fault).
 * n_rows >= 0 (0 launches nothing), 1 <= row_len <= 65536.
 */
KVS_API int kvs_encode_fp8(const void* src, int32_t src_dtype, int64_t n_rows, int32_t row_len,
                   uint8_t* codes, float* scales, void* stream);

/*
 * kvs_append_kv -- write n_rows new positions into one layer's cache.
 * Row r holds the K (and V) values of every KV head for position
 * row_pos[r] of sequence row_seq[r]: k_rows, v_rows are [n_rows][Hkv*d] of
 * src_dtype (KVS_F32 or KVS_BF16). The slot is the position (linear) or
 * position mod C (ring). For an FP8 cache each row is encoded exactly as
 * kvs_encode_fp8 does and its scales go to k_scale / v_scale at that slot;
 * for a BF16 or F32 cache src_dtype must equal the cache type and the values
 * are copied. For a ring cache pos_of_slot[seq][slot] receives the position.
 * Two rows may not target the same (sequence, slot). Row indices outside
 * [0, B) or positions outside the cache (negative, or >= C when linear) are
 * skipped by the kernel. k_scale, v_scale: non-NULL iff the cache is FP8;
 * pos_of_slot: non-NULL iff ring.
 */
KVS_API int kvs_append_kv(const kvs_geom* geom, const void* k_rows, const void* v_rows, int32_t src_dtype,
                  int32_t n_rows, const int32_t* row_seq, const int32_t* row_pos,
                  void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                  int32_t* pos_of_slot, void* stream);

/* Workspace bytes kvs_decode_attn_scored needs; depends on geometry only. */
KVS_API int kvs_decode_workspace_bytes(const kvs_geom* geom, size_t* bytes);

/*
 * kvs_decode_workspace_init -- make a decode workspace ready: fills its first
 * kvs_decode_workspace_bytes() bytes with zeros, on the stream, with a fill
 * kernel (no memset node, so it may be captured in a HIP graph). The decode
 * calls need the workspace's completion counters (one per sequence and KV
 * head) to be zero when they start and leave them zero when they end, so this
 * is needed once after allocation (a zero-filled buffer is equally valid) and
 * again before the workspace is used with another geometry (the counters then
 * sit elsewhere).
 * Errors: KVS_EINVAL (bad geometry or NULL), KVS_EALIGN, KVS_EWS.
 */
KVS_API int kvs_decode_workspace_init(const kvs_geom* geom, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * kvs_decode_attn_scored -- one layer of the scored decode step.
 *
 * For every sequence b the current token's K/V are already in the cache
 * (write, then attend: a position is inside its own window) and
 * i = cur_pos[b] is its absolute position. Key slot t is read when its
 * absolute position p (t if linear, pos_of_slot[b][t] if ring) satisfies
 * p >= 0, p <= i, p >= i - w + 1 when window w > 0, and, when keep_mask is
 * given, bit (p / 16) of keep_mask[b] is set. For every query head h:
 *   logits  s_j = softmax_scale * (q_h . k_j)    (FP8: k_j = code_j * k_scale)
 *   weights p_j = exp(s_j - max) / sum exp(s - max)
 *   out_h   = sum_j p_j v_j                      (FP8: v_j = code_j * v_scale)
 * (Context views at marginal cost, section 0 and Tier 0: the post-softmax
 * weights the pass computes anyway.) When mass_accum is not NULL the weights
 * are also reduced per (sequence, block) and summed over all query heads
 * (Context Optimization, "H2O / How It Works": scores accumulated across all
 * query heads; Per-Head Attention as a Scoring Signal: score per head, place
 * per 16-token block):
 *   mass_accum[b][p/16] += sum_h sum_{read j in block} p_j
 * Heads are added in ascending order and layers in call order. With
 * geom.deterministic = 1 results are bit-reproducible, and with
 * mass_accum == NULL no mass work runs while ``out`` stays bit-identical to
 * the scored call (the tap never changes the math; Context views at marginal
 * cost, Tier 0 invariant). With geom.deterministic = 0 both hold up to
 * floating-point rounding.
 *
 *   q           [B][Hq][d] q_dtype
 *   k_cache, v_cache, k_scale, v_scale, pos_of_slot: as in kvs_append_kv
 *   cur_pos     [B] int32
 *   keep_mask   [B][W] uint32 or NULL (all blocks kept); only with window 0
 *               (Context Optimization, "H2O vs Sliding Window": eviction
 *               replaces the window, so the two are never combined)
 *   out         [B][Hq][d] q_dtype
 *   mass_accum  [B][NBmax] float or NULL
 *   workspace   device scratch of at least kvs_decode_workspace_bytes(),
 *               owned by the caller and initialised for this geometry with
 *               kvs_decode_workspace_init (or zero-filled); calls that share
 *               one must not overlap. Its completion counters are zero when a
 *               call starts and zero again when it ends. Besides
 *               per-call partials it keeps, from call to call, the streaming
 *               rate measured for each of the GPU's dispatch classes
 *               (workgroup id mod 8); in dynamic mode the next call splits
 *               each sequence's tiles over its workgroups by those rates
 *               (unreadable rates count as equal); the rates never change a
 *               result beyond rounding.
 *
 * Preconditions the library cannot check (unspecified results, never a
 * fault): the current token is readable (so no row is all-masked); a ring
 * cache only holds position p in slot p mod C; inputs are finite.
 */
KVS_API int kvs_decode_attn_scored(const kvs_geom* geom, const void* q, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale,
                           const int32_t* pos_of_slot, const int32_t* cur_pos,
                           const uint32_t* keep_mask, void* out, float* mass_accum,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_decode_attn_scored_noalloc -- kvs_decode_attn_scored without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * call allocates nothing: its workspace is a static device array of
 * KVS_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends. Results are those of kvs_decode_attn_scored (bit for bit with
 * geom.deterministic = 1). The caller still passes inputs and outputs, as
 * there; the stream must belong to the current device.
 *
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several host threads without ordering) race
 * and give unspecified results. Each call leaves the array's completion
 * counters zero, so consecutive calls of any geometries need nothing in
 * between. The first call on each device looks up the array's address (with
 * that device current) and clears its counter region on the call's stream.
 *
 * Errors: as kvs_decode_attn_scored; KVS_ESCRATCH when the geometry's
 * workspace (kvs_decode_workspace_bytes) does not fit the array beside its
 * 64 KiB counter region, or its counters (B * Hkv * partitions words) do not
 * fit that region; KVS_EHIP when the array's address cannot be found.
 */
#define KVS_NOALLOC_SCRATCH_BYTES (16u << 20)
KVS_API int kvs_decode_attn_scored_noalloc(const kvs_geom* geom, const void* q, const void* k_cache,
                                           const void* v_cache, const float* k_scale, const float* v_scale,
                                           const int32_t* pos_of_slot, const int32_t* cur_pos,
                                           const uint32_t* keep_mask, void* out, float* mass_accum,
                                           void* stream);

/*
 * kvs_decode_attn_tap, kvs_append_decode_attn_tap, kvs_tap_masses -- the
 * scored decode step with the block masses added once per step instead of
 * once per layer (Context views at marginal cost, Tier 0: the tap leaves
 * per-block sums that are reduced later; section 2: the side-car consumes
 * them once per turn).
 *
 * The two per-layer calls take the arguments of kvs_decode_attn_scored and
 * kvs_append_decode_attn without mass_accum: they compute ``out`` in the same
 * way and leave the layer's per-block sums in ``workspace``, which must then
 * stay untouched until kvs_tap_masses has read it (one workspace per layer).
 * kvs_tap_masses then adds the masses of all n_layers calls, in order, exactly
 * as one scored call per layer would have: mass_accum (and head_mass /
 * mass_max as in kvs_decode_attn_profiled) get the same values, bit for bit
 * in deterministic mode.
 *
 *   workspaces  host array of n_layers device workspace pointers, the ones
 *               the per-layer calls used, in call order (1 <= n_layers <= 128)
 *   cur_pos     the [B] positions the per-layer calls used
 *   mass_accum, head_mass, mass_max: as in kvs_decode_attn_profiled, each
 *               may be NULL (all NULL: nothing to do)
 * Errors: KVS_EINVAL for a bad geometry, layer count or NULL pointer,
 * KVS_EALIGN, KVS_EWS if workspace_bytes is below kvs_decode_workspace_bytes().
 */
KVS_API int kvs_decode_attn_tap(const kvs_geom* geom, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* pos_of_slot, const int32_t* cur_pos,
                                const uint32_t* keep_mask, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);
KVS_API int kvs_append_decode_attn_tap(const kvs_geom* geom, const void* k_new, const void* v_new,
                                       int32_t src_dtype, const void* q, void* k_cache, void* v_cache,
                                       float* k_scale, float* v_scale, int32_t* pos_of_slot,
                                       const int32_t* cur_pos, const uint32_t* keep_mask, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream);
KVS_API int kvs_tap_masses(const kvs_geom* geom, void* const* workspaces, int32_t n_layers,
                           size_t workspace_bytes, const int32_t* cur_pos, float* mass_accum,
                           float* head_mass, float* mass_max, void* stream);

/*
 * kvs_decode_partial, kvs_decode_combine -- the two phases of
 * kvs_decode_attn_scored, with the same arguments and checks. The partial
 * phase reads the cache and leaves, per (sequence, query head, partition of
 * slots), the partition's running max, sum of exponentials and unnormalised
 * output, plus per-block sums of the post-softmax weights, in ``workspace``;
 * the combine phase turns them into ``out`` and adds the normalised block
 * masses into ``mass_accum``. Calling partial then combine on one stream, with
 * the same arguments and workspace, is exactly kvs_decode_attn_scored; the
 * split lets a caller time or overlap the phases. The combine phase does not
 * read the cache buffers but validates them like the partial phase.
 */
KVS_API int kvs_decode_partial(const kvs_geom* geom, const void* q, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* pos_of_slot, const int32_t* cur_pos,
                               const uint32_t* keep_mask, void* out, float* mass_accum,
                               void* workspace, size_t workspace_bytes, void* stream);
KVS_API int kvs_decode_combine(const kvs_geom* geom, const void* q, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* pos_of_slot, const int32_t* cur_pos,
                               const uint32_t* keep_mask, void* out, float* mass_accum,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvs_append_decode_attn -- kvs_append_kv of the step's new rows followed by
 * kvs_decode_attn_scored, in one pass over the cache (the write-then-attend
 * order of a decode step: Context Optimization, "FP8 KV Cache / How It Works"
 * for the encoding, "Context views at marginal cost" for the scored read).
 *
 * Row b of k_new / v_new ([B][Hkv*d] of src_dtype, KVS_F32 or KVS_BF16; for a
 * BF16 or F32 cache src_dtype must equal the cache type) goes to position
 * cur_pos[b] of sequence b exactly as kvs_append_kv with row_seq[b] = b and
 * row_pos[b] = cur_pos[b] writes it (same codes, scales and pos_of_slot
 * entry; skipped when cur_pos[b] < 0, or >= C for a linear cache), and the
 * attention then reads it: the results equal those two calls on one stream
 * (bit for bit in deterministic mode). The workgroup holding the new slot
 * writes it before reading that tile, so the separate append launch and its
 * pass over the row go away. The cache buffers are written, hence not const.
 * Other arguments, checks and errors as kvs_decode_attn_scored; null or
 * misaligned k_new / v_new give KVS_EINVAL / KVS_EALIGN, a bad src_dtype
 * KVS_EDTYPE.
 *
 * kvs_append_decode_partial is its partial phase (append + partial); follow it
 * with kvs_decode_combine, with the same arguments, on the same stream.
 */
KVS_API int kvs_append_decode_attn(const kvs_geom* geom, const void* k_new, const void* v_new,
                                   int32_t src_dtype, const void* q, void* k_cache, void* v_cache,
                                   float* k_scale, float* v_scale, int32_t* pos_of_slot,
                                   const int32_t* cur_pos, const uint32_t* keep_mask, void* out,
                                   float* mass_accum, void* workspace, size_t workspace_bytes,
                                   void* stream);
KVS_API int kvs_append_decode_partial(const kvs_geom* geom, const void* k_new, const void* v_new,
                                      int32_t src_dtype, const void* q, void* k_cache, void* v_cache,
                                      float* k_scale, float* v_scale, int32_t* pos_of_slot,
                                      const int32_t* cur_pos, const uint32_t* keep_mask, void* out,
                                      float* mass_accum, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * kvs_decode_attn_profiled -- kvs_decode_attn_scored with the per-axis views
 * of the block masses (Context views at marginal cost, section 4: the
 * observer's layer and head axes kept as a reduced per-span profile, not the
 * matrix; the per-layer and per-head rows of its views table; Per-Head
 * Attention as a Scoring Signal, "Fix: score per head, place per block": a
 * block is kept while at least one head gives it weight).
 *
 * Same arguments and checks as kvs_decode_attn_scored, plus two optional
 * outputs (NULL skips each; all three mass outputs may be NULL):
 *   head_mass  [B][Hq][NBmax] float: head_mass[b][h][blk] += the block mass of
 *              query head h alone (sum over its read keys of p_j)
 *   mass_max   [B][NBmax] float: mass_max[b][blk] = max(mass_max[b][blk],
 *              max over heads h of head h's block mass)
 * mass_accum, if given, gets the same head-summed masses as the scored call.
 * Passing one mass_accum per layer gives the per-layer profile; passing the
 * same mass_max to every layer gives the max over layers and heads.
 */
KVS_API int kvs_decode_attn_profiled(const kvs_geom* geom, const void* q, const void* k_cache,
                                     const void* v_cache, const float* k_scale, const float* v_scale,
                                     const int32_t* pos_of_slot, const int32_t* cur_pos,
                                     const uint32_t* keep_mask, void* out, float* mass_accum,
                                     float* head_mass, float* mass_max, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * kvs_reattend_blocks -- one layer of attention for a new query over a chosen
 * set of cached blocks only (Context views at marginal cost, "Tier 2 —
 * RE-ATTEND" and "Fact 3": to ask how relevant stored spans are to a new
 * query, that query attends over the cached keys of those spans only and the
 * distribution it produces is read; cached keys and values are reused as
 * they are, and the cost grows with the number of selected tokens).
 *
 * Exactly kvs_decode_attn_scored on a linear cache (ring == 0, window == 0,
 * else KVS_EINVAL) with the keep mask replaced by a list: key slot t is read
 * when t <= cur_pos[b] and block t / 16 appears among the first n_ids[b]
 * entries of block_ids[b]. Entries may repeat and come in any order; entries
 * outside 0 .. C/16-1 are ignored (the selection's sel_ids / n_sel can be
 * passed as they are). ``out`` is the attention over those keys; when
 * mass_accum is not NULL the per-block masses of the new query (its
 * distribution over the chosen spans, summed over query heads) are added to
 * mass_accum[b][block]. A sequence with no readable key gets a zero output
 * and no mass.
 *
 *   block_ids   [B][ids_stride] int32, device, 16-byte aligned
 *   n_ids       [B] int32, device, 16-byte aligned; values are clamped to
 *               0 .. ids_stride
 *   ids_stride  >= 1
 *   other arguments as in kvs_decode_attn_scored (pos_of_slot and keep_mask
 *   do not apply)
 */
KVS_API int kvs_reattend_blocks(const kvs_geom* geom, const void* q, const void* k_cache,
                                const void* v_cache, const float* k_scale, const float* v_scale,
                                const int32_t* cur_pos, const int32_t* block_ids, const int32_t* n_ids,
                                int32_t ids_stride, void* out, float* mass_accum, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kvs_update_sidecar -- close one turn (Context views at marginal cost,
 * section 2 Tier 1 and section 3: {Attended, EMA, Cumulative, traj}, O(1) per
 * block per turn). With A = mass_accum (this step's mass):
 *   attended = A;  ema = alpha*A + (1-alpha)*ema;  cum += A;
 *   traj[b][step mod traj_cap][:] = A;  mass_accum = 0.
 * mass_accum, attended, ema, cum: [B][NBmax] float; traj: [B][traj_cap][NBmax]
 * float or NULL. step >= 0 counts turns from 0; 1 <= traj_cap; 0 <= alpha <= 1.
 */
KVS_API int kvs_update_sidecar(float* mass_accum, float* attended, float* ema, float* cum, float* traj,
                       int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step,
                       float alpha, void* stream);

/*
 * kvs_snapkv_scores -- prefill scoring from an observation window (Context
 * views at marginal cost, section 7, SOTA grounding, per-system reductions,
 * SnapKV: once, when the prompt is done, the weights the last W prompt
 * queries give each prompt token are added up per head, and each token's
 * score becomes the maximum over an odd neighbourhood -- 7 tokens on the page
 * -- so the neighbours of a high-scoring key score high too), placed per
 * 16-token block (Per-Head Attention as a Scoring Signal, "Fix: score per
 * head, place per block").
 *
 * For sequence b with n = n_prompt[b] prompt tokens in a linear cache and
 * window query w (0 <= w < W) of head h at position n - W + w, reading keys
 * j <= its position with softmax weights p_{w,h,j} (logits as in
 * kvs_decode_attn_scored):
 *   token_score[b][h][j] = sum_w p_{w,h,j}                       (j < n)
 *   block_score[b][k]   += sum_h sum_{j in block k, j < n} max_{|i-j| <= R, 0 <= i < n} token_score[b][h][i]
 * with R = (pool_kernel - 1) / 2, summed in a fixed order. Queries at
 * negative positions (n < W) read nothing. token_score entries j >= n are not
 * written; block_score may be NULL.
 *
 *   q_window     [B][W][Hq][d] bf16
 *   k_cache, k_scale  as in kvs_append_kv (bf16 or FP8 caches; F32 gives
 *                KVS_ENOTIMPL; a ring cache gives KVS_EINVAL)
 *   n_prompt     [B] int32, 0 <= n <= C
 *   token_score  [B][Hq][C] float
 *   block_score  [B][NBmax] float or NULL
 *   workspace    at least kvs_snapkv_workspace_bytes(geom, W)
 * W * (Hq / Hkv) <= 128 and Hq / Hkv dividing 16 (1, 2, 4, 8 or 16), else
 * KVS_ENOTIMPL; pool_kernel must be odd, at most 33.
 */
KVS_API int kvs_snapkv_workspace_bytes(const kvs_geom* geom, int32_t window, size_t* bytes);
KVS_API int kvs_snapkv_scores(const kvs_geom* geom, const void* q_window, int32_t window,
                              const void* k_cache, const float* k_scale, const int32_t* n_prompt,
                              float* token_score, float* block_score, int32_t pool_kernel,
                              void* workspace, size_t workspace_bytes, void* stream);

/* One per-block table to compact alongside the cache: 4-byte entries (float
 * or int32) laid out [B][rows][NBmax] (rows = 1 for Attended, EMA,
 * Cumulative or a counter; rows = traj_cap for the trajectory ring). */
typedef struct {
  void* data;
  int32_t rows;
} kvs_block_table;

/*
 * kvs_compact_blocks -- move the kept blocks of a linear cache to the front,
 * in order (Context Optimization, "H2O KV Cache Eviction / How It Works in
 * Flash-MoE", step 4: survivors are moved to contiguous positions so later
 * passes read one shorter run of positions), at 16-slot block granularity
 * (Per-Head Attention as a Scoring Signal: the block is the unit kept).
 *
 * For each sequence b and k < n_keep[b] (clamped to ids_stride and C/16),
 * block keep_ids[b][k] becomes block k: its K and V codes of every KV head,
 * its K/V scales (FP8), and its entry in every row of every table. Table
 * entries from n_keep[b] on are set to zero; cache slots from block n_keep[b]
 * on are left as they were (never read: decode reads slots <= cur_pos). Ids
 * outside 0 .. C/16-1 move nothing. In place, on the stream; a ring cache
 * gives KVS_EINVAL.
 *
 * After compaction the sequence continues at position (n_keep[b]-1)*16 +
 * (i mod 16) + 1 when the current block (that of position i) is the last one
 * kept, as kvs_select_blocks always keeps it; positions are then positions in
 * the compacted sequence.
 *
 *   keep_ids  [B][ids_stride] int32, ascending and distinct (kvs_select_blocks'
 *             sel_ids); other orders give unspecified contents, never a fault
 *   n_keep    [B] int32
 *   tables    n_tables (0..8) entries, each 16-byte aligned
 */
KVS_API int kvs_compact_blocks(const kvs_geom* geom, void* k_cache, void* v_cache, float* k_scale,
                               float* v_scale, const int32_t* keep_ids, const int32_t* n_keep,
                               int32_t ids_stride, const kvs_block_table* tables, int32_t n_tables,
                               void* stream);

/*
 * kvs_update_counters -- side-car counters for threshold views, once per turn
 * after kvs_update_sidecar (Context views at marginal cost, section 3: a view
 * filters the score table, and the same threshold decides which history is
 * kept: a span whose EMA has been under it for K turns loses its per-turn
 * trajectory and keeps only its Cumulative value; section 7, SOTA grounding,
 * per-system reductions: Scissorhands counts the turns a token's attention
 * passes a threshold). Per block x of
 * every sequence (all n_blocks_max entries):
 *   hot_count[x]  += (attended[x] > hot_theta)                (NULL: skipped)
 *   cold_turns[x]  = ema[x] < cold_theta ? cold_turns[x] + 1 : 0  (NULL: skipped)
 *   if traj != NULL, cold_limit > 0 and cold_turns[x] >= cold_limit:
 *       traj[b][s][blk] = 0 for every slot s of the ring
 *
 *   attended, ema  [B][NBmax] float (as kept by kvs_update_sidecar)
 *   hot_count, cold_turns  [B][NBmax] int32, start at zero
 *   traj   [B][traj_cap][NBmax] float; needs cold_turns
 * Errors: KVS_EINVAL for sizes < 1, cold_limit < 0, non-finite thresholds, a
 * counter without its input, traj without cold_turns; KVS_EALIGN.
 */
KVS_API int kvs_update_counters(const float* attended, const float* ema, int32_t* hot_count,
                                int32_t* cold_turns, float* traj, int32_t batch, int32_t n_blocks_max,
                                int32_t traj_cap, float hot_theta, float cold_theta, int32_t cold_limit,
                                void* stream);

/*
 * kvs_filter_blocks -- a threshold view (Context views at marginal cost,
 * section 3: the spans whose score is above a threshold, worked out when the
 * query comes, returned as a set of spans). For each sequence b with
 * i = cur_pos[b], the ascending
 * ids of the existing blocks (0 .. i/16, below NBmax) that are alive (bit set
 * in alive[b], or every block when alive is NULL) and whose score exceeds
 * theta. n_ids[b] is the number of such blocks; ids[b] holds the first
 * min(n_ids[b], ids_stride) of them. The result can be passed to
 * kvs_reattend_blocks (the Tier 1 to Tier 2 handoff).
 *
 *   score  [B][NBmax] float (Attended, EMA, Cumulative, or any per-block scalar)
 *   alive  [B][ceil(NBmax/32)] uint32 or NULL
 *   ids    [B][ids_stride] int32; n_ids [B] int32
 * Errors: KVS_EINVAL (sizes, NaN theta, NULL required pointers), KVS_EALIGN.
 */
KVS_API int kvs_filter_blocks(const float* score, const uint32_t* alive, const int32_t* cur_pos,
                              int32_t batch, int32_t n_blocks_max, float theta, int32_t* ids,
                              int32_t* n_ids, int32_t ids_stride, void* stream);

/*
 * kvs_select_blocks -- heavy-hitter block selection (Context Optimization,
 * "H2O KV Cache Eviction": sinks and recent tokens are always kept; among the
 * rest the top scorers survive), at 16-token block granularity.
 * For sequence b with i = cur_pos[b], the existing blocks are 0 .. i/16.
 * Protected: every block meeting positions [max(0, i-recent+1), i], and, when
 * sink_tokens > 0, every block meeting positions [0, sink_tokens-1].
 * Candidates: existing, alive (bit set in alive[b], or all when alive is
 * NULL), not protected. Kept: protected blocks plus the budget_blocks
 * candidates with the largest (score, -block index): equal scores go to the
 * lower block index.
 *   score     [B][NBmax] float (e.g. the Cumulative array), finite
 *   alive     [B][W] uint32 or NULL
 *   keep_mask [B][W] uint32 out: bit b set for kept blocks and for every
 *             block b > i/16 (not yet written, so never evicted)
 *   sel_ids   [B][NBmax] int32 out: kept blocks (b <= i/16) in ascending order
 *   n_sel     [B] int32 out: number of entries of sel_ids
 * budget_blocks >= 0, recent_tokens >= 1, sink_tokens >= 0. Sequences with
 * i / 16 >= NBmax have their blocks clipped to NBmax.
 */
KVS_API int kvs_select_blocks(const float* score, const uint32_t* alive, const int32_t* cur_pos,
                      int32_t batch, int32_t n_blocks_max, int32_t budget_blocks,
                      int32_t recent_tokens, int32_t sink_tokens, uint32_t* keep_mask,
                      int32_t* sel_ids, int32_t* n_sel, void* stream);

/*
 * kvs_update_sidecar_select -- kvs_update_sidecar followed by
 * kvs_select_blocks in one launch (Context views at marginal cost, section 2
 * Tier 1, closing the turn; Context Optimization, "H2O KV Cache Eviction",
 * selecting on the score it just updated). The selection scores the updated
 * array score_source names: KVS_SCORE_CUMULATIVE (H2O's accumulated
 * attention), KVS_SCORE_EMA or KVS_SCORE_ATTENDED (TOVA: this turn's mass).
 * Every output equals that of the two calls with the same arguments, bit for
 * bit. Arguments, layouts and errors as in the two calls; alive may be the
 * same buffer as keep_mask (the feedback of evict mode).
 */
#define KVS_SCORE_CUMULATIVE 0
#define KVS_SCORE_EMA 1
#define KVS_SCORE_ATTENDED 2
KVS_API int kvs_update_sidecar_select(float* mass_accum, float* attended, float* ema, float* cum, float* traj,
                                      int32_t batch, int32_t n_blocks_max, int32_t traj_cap, int64_t step,
                                      float alpha, int32_t score_source, const uint32_t* alive,
                                      const int32_t* cur_pos, int32_t budget_blocks, int32_t recent_tokens,
                                      int32_t sink_tokens, uint32_t* keep_mask, int32_t* sel_ids,
                                      int32_t* n_sel, void* stream);

/*
 * kvs_decode_step -- one whole scored decode step in one call: for every
 * layer the append of the new position and the scored attention, then the
 * block masses of all layers added once, then the turn's side-car update (and
 * the heavy-hitter selection). It is the per-turn loop of Context views at
 * marginal cost (Tier 0: the tap during the forward pass; section 2: the
 * side-car updated once per turn from the summed masses) with the selection
 * of Context Optimization, "H2O KV Cache Eviction" (steps 2 and 3), made by
 * the library instead of by one host call per layer: the launches and every
 * result are exactly those of
 *   for l in 0 .. n_layers - 1:
 *     kvs_append_decode_attn_tap(geom, layers[l].k_new, layers[l].v_new,
 *         src_dtype, layers[l].q, layers[l].k_cache, ..., cur_pos, keep_mask,
 *         layers[l].out, layers[l].workspace, workspace_bytes, stream)
 *     (kvs_decode_attn_tap when layers[l].k_new is NULL: nothing appended)
 *   if mass_accum: kvs_tap_masses(geom, {layers[l].workspace}, n_layers,
 *                  workspace_bytes, cur_pos, mass_accum, NULL, NULL, stream)
 *   if turn: kvs_update_sidecar_select(mass_accum, turn->attended, ...,
 *            geom->batch, geom->n_blocks_max, ...) when turn->select is 1,
 *            else kvs_update_sidecar(mass_accum, turn->attended, ...).
 *
 *   layers      HOST array of n_layers kvs_layer_bufs (1 <= n_layers <= 128);
 *               the pointers in it are device pointers, as in the calls above;
 *               every layer has its own workspace (workspace_bytes each)
 *   src_dtype   KVS_F32 or KVS_BF16: the new rows' dtype (as in
 *               kvs_append_decode_attn_tap)
 *   cur_pos, keep_mask: shared by all layers, as in the per-layer calls
 *   mass_accum  [B][NBmax] float32 the masses are added into (read by the
 *               side-car), or NULL: the layers only, their block sums left
 *               in the workspaces for a later kvs_tap_masses (turn must then
 *               be NULL)
 *   turn        HOST pointer to the turn's arguments, or NULL: no side-car
 *               update. turn->alive may be turn->keep_out (evict mode feeds
 *               the mask back); the trajectory slot is turn->step mod traj_cap.
 * The library keeps no pointer after the call returns. Errors: those of the
 * calls above; every argument of every layer is checked before the first
 * launch, so an error launches nothing.
 */
typedef struct kvs_layer_bufs {
  const void* q;          /* [B][Hq][d], the geometry's q dtype */
  const void* k_new;      /* [B][Hkv*d] new K row of each sequence, src_dtype; NULL: no append */
  const void* v_new;      /* [B][Hkv*d] new V row; NULL exactly when k_new is */
  void* k_cache;
  void* v_cache;
  float* k_scale;         /* FP8 caches only, else NULL */
  float* v_scale;
  int32_t* pos_of_slot;   /* ring caches only, else NULL */
  void* out;              /* [B][Hq][d] */
  void* workspace;        /* this layer's decode workspace */
} kvs_layer_bufs;

typedef struct kvs_turn_args {
  float* attended;        /* [B][NBmax] side-car arrays, as in kvs_update_sidecar */
  float* ema;
  float* cum;
  float* traj;            /* [B][traj_cap][NBmax], or NULL */
  int32_t traj_cap;
  int32_t select;         /* 1: update and select in one launch; 0: update only */
  int64_t step;           /* the turn index */
  float alpha;            /* EMA weight in [0, 1] */
  int32_t score_source;   /* KVS_SCORE_*, with select */
  const uint32_t* alive;  /* [B][W] or NULL, with select */
  int32_t budget_blocks;  /* with select, as in kvs_select_blocks */
  int32_t recent_tokens;
  int32_t sink_tokens;
  uint32_t* keep_out;     /* [B][W] keep mask written by the selection */
  int32_t* sel_ids;       /* [B][NBmax] */
  int32_t* n_sel;         /* [B] */
} kvs_turn_args;

KVS_API int kvs_decode_step(const kvs_geom* geom, int32_t n_layers, const kvs_layer_bufs* layers,
                            int32_t src_dtype, const int32_t* cur_pos, const uint32_t* keep_mask,
                            size_t workspace_bytes, float* mass_accum, const kvs_turn_args* turn,
                            void* stream);

/*
 * kvs_close_step -- the end of a step whose layers ran without mass_accum
 * (kvs_decode_step with mass_accum NULL, or the per-layer _tap calls): the
 * layers' block masses added into mass_accum, then the turn closed, with
 * every result exactly that of
 *   kvs_tap_masses(geom, workspaces, n_layers, workspace_bytes, cur_pos,
 *                  mass_accum, NULL, NULL, stream)
 *   kvs_update_sidecar_select(...) when turn->select is 1, else
 *   kvs_update_sidecar(mass_accum, turn->attended, ...)
 * (Context views at marginal cost, section 2: the side-car is updated once
 * per turn from the summed masses). Without selection the side-car update
 * runs in the mass combine's launch when the combine sums the layers in
 * parallel (every layer's merge tables fit its LDS), else in a launch of its
 * own. Arguments as in the calls above; turn is a HOST pointer, not NULL.
 * Errors: those of the calls above, checked before the first launch.
 */
KVS_API int kvs_close_step(const kvs_geom* geom, void* const* workspaces, int32_t n_layers,
                           size_t workspace_bytes, const int32_t* cur_pos, float* mass_accum,
                           const kvs_turn_args* turn, void* stream);

/*
 * kvs_stream_read -- a measurement helper, not part of the decode step: the
 * streaming-read ceiling that the decode kernel's KV scan is compared with
 * (Context views at marginal cost, section 7, Fact 3: the read of the cached
 * keys by the query is the cost that cannot be avoided). Reads every byte of
 * buf once with the decode kernel's kind of load (non-temporal 16-byte buffer
 * loads, 1 KiB of consecutive bytes per wave instruction), split into
 * `workgroups` equal slices of whole KiB, one 8-wave workgroup each, and
 * stores the 32-bit wrapping sum of each slice's dwords in sums[workgroup]
 * (so no load can be skipped). Time it with events on the stream.
 *   buf   device, 16-byte aligned, bytes > 0 and a multiple of 1024
 *   sums  device uint32 [workgroups], 16-byte aligned
 *   1 <= workgroups <= min(65536, bytes / 1024)
 * Errors: KVS_EINVAL, KVS_EALIGN, KVS_EHIP.
 */
KVS_API int kvs_stream_read(const void* buf, size_t bytes, uint32_t* sums, int32_t workgroups, void* stream);

/* Static text for a status code. */
KVS_API const char* kvs_status_str(int status);

/* Library version string. */
KVS_API const char* kvs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */
