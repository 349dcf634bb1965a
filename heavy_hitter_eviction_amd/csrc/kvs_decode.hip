// Scored split-K decode attention for gfx950.
//
// kvs_partial: one workgroup of 8 waves per (partition of slots, KV head,
// sequence), one workgroup per compute unit. The waves take batches of
// 16-slot tiles of the partition from a shared LDS counter and run an online
// softmax over them for all G query heads of the KV head at once:
//
//   QK:  S^T[token][head] = K[token][:] . Q[head][:]   MFMA, A = K tile, B = Q^T
//   PV:  O^T[dim][head]  += V^T[dim][token] . P^T[token][head]   MFMA
//
// With S^T and O^T the MFMA result layout puts one query head per lane column
// (lane l holds head l%16 and rows 4*(l/16)+r), so the running max, the sum and
// the rescale of O stay inside the lane; the only cross-lane work is a
// two-step reduction over the four 16-lane rows per tile. Heads G..15 are zero
// padding of the 16-wide MFMA. bf16 and FP8 caches use bf16 MFMAs (FP8 codes
// are widened exactly; the per-position K scale multiplies the logit and the V
// scale is folded into P); F32 caches use the f32 MFMA.
//
// The tap (Context views at marginal cost, Tier 0): for every tile the wave
// also sums its post-softmax weights per head relative to its running max and
// keeps that record in LDS; at the end of the partition the records are
// rescaled to the workgroup max and stored with the partition's (max, sum,
// unnormalised O). kvs_combine then turns them into exact normalised masses.
//
// kvs_combine: per sequence, M_h = max_p m_p, L_h = sum_p l_p 2^(m_p - M_h);
// O_h = sum_p o_p 2^(m_p - M_h) / L_h; block mass = sum_h E_h,b 2^(m_p(b) - M_h)
// / L_h, heads in ascending order, added to mass_accum[b].

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

template <int KV>
struct KvT;
template <>
struct KvT<KV_F32> {
  static constexpr int eb = 4;
};
template <>
struct KvT<KV_BF16> {
  static constexpr int eb = 2;
};
template <>
struct KvT<KV_FP8> {
  static constexpr int eb = 1;
};

// Per-lane register image of one 16-slot tile.
template <int KV, int D>
struct TileRegs {
  static constexpr int NCH = D * KvT<KV>::eb / 64;  // 16-byte chunks per lane, K and V each
  u32x4 k[NCH];
  u32x4 v[NCH];
};

// Buffer resources (base in scalar registers, bounds-checked: reads past
// num_records return 0) over one (sequence, KV head)'s K and V regions and one
// sequence's scale and position arrays, plus the lane's constant byte offsets.
// A tile then costs one scalar offset per load.
struct TileAddr {
  __amdgpu_buffer_rsrc_t k, v;
  uint32_t koff, voff;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw untyped 32-bit dword access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// AUX = 2 sets the non-temporal (streaming) cache policy, for bytes read once.
template <int AUX>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}

template <int KV, int D, bool RING>
__device__ __forceinline__ void load_tile(TileRegs<KV, D>& t, const TileAddr& ad, uint32_t so) {
  constexpr int NCH = TileRegs<KV, D>::NCH;
  // K and V tiles are stored fragment-major: chunk i of every lane is one
  // contiguous 1 KiB run (lane-major), so each load instruction reads whole
  // cache lines, streamed past the caches (non-temporal). so is the tile's
  // byte offset in the (sequence, KV head) region.
#pragma unroll
  for (int i = 0; i < NCH; ++i) t.k[i] = bload16<2>(ad.k, ad.koff + 1024 * i, so);
#pragma unroll
  for (int i = 0; i < NCH; ++i) t.v[i] = bload16<2>(ad.v, ad.voff + 1024 * i, so);
}

// Lane's t-th contraction element of the QK product lives at head dimension
// dim(t, kg): the K load above gives element t of chunk t/EPC at row offset
// 64 (t/EPC) + 16 kg bytes.
template <int KV>
__device__ __forceinline__ int qk_dim(int t, int kg) {
  constexpr int EPC = 16 / KvT<KV>::eb;
  return (t / EPC) * 4 * EPC + kg * EPC + t % EPC;
}

// ---- merging partitions (the partial kernel's own merge of a (sequence,
// KV head)'s outputs) ----
// Partition p's merge weight for one head from the partitions' maxima m[q]
// and sums l[q] (in LDS): M = max_q m_q, L = sum_q l_q 2^(m_q - M) in
// ascending q, w_p = 2^(m_p - M) / L (0 for an empty partition). Every
// lane of a head computes the same M and L. Up to eight partitions come in
// one batch of LDS reads (indices clamped, terms past P are +0); more take a
// batch per eight partitions for the maximum and again for the sum.
__device__ __forceinline__ float merge_weight(const float* m, const float* l, int P, int p) {
  const float mp = m[p];
  float M = -__builtin_inff();
  float L = 0.0f;
  if (P <= 8) {
    float mv[8], lv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mv[i] = m[min(i, P - 1)];
      lv[i] = l[min(i, P - 1)];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) M = fmaxf(M, mv[i]);
    const bool none = M == -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i)
      L += (i >= P || none || mv[i] == -__builtin_inff()) ? 0.0f : lv[i] * fast_exp2(mv[i] - M);
  } else {
    for (int q0 = 0; q0 < P; q0 += 8) {
      float mv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) mv[i] = m[min(q0 + i, P - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) M = fmaxf(M, mv[i]);
    }
    const bool none = M == -__builtin_inff();
    for (int q0 = 0; q0 < P; q0 += 8) {
      float mv[8], lv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mv[i] = m[min(q0 + i, P - 1)];
        lv[i] = l[min(q0 + i, P - 1)];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
        L += (q0 + i >= P || none || mv[i] == -__builtin_inff()) ? 0.0f : lv[i] * fast_exp2(mv[i] - M);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  return (mp == -__builtin_inff() || inv == 0.0f) ? 0.0f : fast_exp2(mp - M) * inv;
}

// Largest log2 of an exponential term of the partial kernel's online
// softmax (see the reference rule in its tile step).
constexpr float kLazyLog2 = 8.0f;

template <int KV>
struct Pipe {
  // tile buffers per wave (depth - 1 tiles in flight); also the tiles a wave
  // claims at a time
  static constexpr int depth = KV == KV_F32 ? 2 : 4;
};

template <int KV, int D, bool SCORED, bool RING>
__global__ __launch_bounds__(64 * kPartialWaves, 1) void kvs_partial(PartialArgs a) {
  constexpr int NW = kPartialWaves;      // waves per workgroup
  constexpr int NTH = 64 * NW;           // threads per workgroup
  constexpr int NSUB = RING ? 2 : 1;
  constexpr int NC = D / 16;  // PV output chunks of 16 dims
  constexpr int NBUF = Pipe<KV>::depth;
  constexpr int BATCH = NBUF;            // tiles per claim
  constexpr int QPT = 64 / BATCH;        // side-data quads (16 bytes) per tile
  constexpr int eb = KvT<KV>::eb;
  extern __shared__ float lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int G = a.G;
  const int h = j;                       // query head within the group (this lane's column)
  const bool hreal = h < G;
  const uint64_t clk0 = __builtin_amdgcn_s_memrealtime();
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wg_id = part + a.nparts * (g + a.Hkv * b);  // dispatch order: XCD = id mod 8
  // fused append: the appending wave fetches the new K and V rows right away
  // (their address needs no cur_pos), before any tile load, so the append
  // never waits behind its own tile loads (vector loads complete in order);
  // it is decided further down whether this workgroup appends at all. FP8
  // takes the scale from the whole row: values 8 lane .. 8 lane + 7 (and, for
  // bf16 rows, 512 + 8 lane ..) come here, the rest in the append itself.
  // This KV head's values (dims lane, lane + 64) come separately.
  const int app_n = a.Hkv * D;
  const size_t app_rb = (size_t)b * app_n;
  constexpr int XPL = D > 64 ? D / 64 : 1;  // appended dims per lane
  u32x4 app_k0[2], app_v0[2];  // bf16 rows: [r] holds values 512 r + 8 lane ..; f32 rows: [0..1] values 8 lane ..
  uint32_t app_hk[XPL], app_hv[XPL];  // this head's values as stored in the row (bf16 or f32 bits)
  const bool app_wave = a.app_k != nullptr && wave == NW - 1;
  // a ring's position: requested first (a vector load, so waiting for it
  // waits for nothing issued later), used once the first tile loads are out
  int ring_pos = 0;
  if constexpr (RING) ring_pos = a.cur_pos[b];
  if (app_wave) {
    if constexpr (KV == KV_FP8) {
      if (a.app_bf16) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (512 * r + 8 * lane < app_n) {
            app_k0[r] = *(const u32x4*)((const uint16_t*)a.app_k + app_rb + 512 * r + 8 * lane);
            app_v0[r] = *(const u32x4*)((const uint16_t*)a.app_v + app_rb + 512 * r + 8 * lane);
          }
        }
      } else if (8 * lane < app_n) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          app_k0[c] = *(const u32x4*)((const float*)a.app_k + app_rb + 8 * lane + 4 * c);
          app_v0[c] = *(const u32x4*)((const float*)a.app_v + app_rb + 8 * lane + 4 * c);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < XPL; ++c) {
      const int x = lane + 64 * c;
      if (x >= D) continue;
      const size_t i = app_rb + (size_t)g * D + x;
      if (KV == KV_F32 || !a.app_bf16) {
        app_hk[c] = ((const uint32_t*)a.app_k)[i];
        app_hv[c] = ((const uint32_t*)a.app_v)[i];
      } else {
        app_hk[c] = ((const uint16_t*)a.app_k)[i];
        app_hv[c] = ((const uint16_t*)a.app_v)[i];
      }
    }
  }
  // Query operand (B of the QK MFMA): lane holds Q[h][dim(t, kg)], zeros for
  // padding heads. Runs of EPC consecutive dims are read with 16-byte loads
  // at entry (they need no cur_pos) and converted once the first tile loads
  // are in flight.
  const int hq = g * G + min(h, G - 1);
  constexpr int QN = D / 4;
  constexpr int EPC = 16 / eb;                  // dims per run
  constexpr int QE = KV == KV_F32 ? 4 : 2;      // query element bytes
  constexpr int QRUN = EPC * QE / 16;           // 16-byte words per run
  u32x4 qraw[QN / EPC][QRUN];
  {
    const char* qrow = (const char*)a.q + ((size_t)b * a.Hq + hq) * D * QE;
#pragma unroll
    for (int r = 0; r < QN / EPC; ++r)
#pragma unroll
      for (int c = 0; c < QRUN; ++c)
        qraw[r][c] = *(const u32x4*)(qrow + (size_t)qk_dim<KV>(r * EPC, kg) * QE + 16 * c);
  }
  // Partition weights: the measured streaming rate of each dispatch class,
  // one per lane in a single load, with the position's, after the loads
  // above (eight guarded scalar-indexed loads would each wait for the one
  // before)
  const bool use_rates = !RING && a.dyn && a.adapt && a.rates != nullptr;
  const float r_lane = use_rates && lane < 8 ? a.rates[lane] : 1.0f;
  // The current position. A linear cache's partition range depends on it: a
  // vector load, waited for together with the rates. A ring's does not: its
  // position was requested at entry and is read once the first tile loads
  // are out.
  int i_cur = RING ? 0 : __builtin_amdgcn_readfirstlane(a.cur_pos[b]);
  float wcls[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_lane), c));
    wcls[c] = (r >= 0.5f && r <= 2.0f) ? fminf(fmaxf(r, 1.0f / 1.2f), 1.2f) : 1.0f;  // NaN -> 1
  }
  // from the position: the first readable one (window) and the slot this
  // call appends (the workgroup whose tiles hold it writes this KV head's
  // part of the row there before anyone reads that tile)
  int lo = 0, app_cand = -1, app_cand_tile = -1;
  auto set_position = [&]() {
    lo = a.window > 0 ? i_cur - a.window + 1 : (int)0x80000000;
    app_cand = (a.app_k != nullptr && i_cur >= 0 && (RING || i_cur < a.C)) ? (RING ? i_cur % a.C : i_cur) : -1;
    app_cand_tile = app_cand >= 0 ? app_cand / kTile : -1;
  };
  if constexpr (!RING) set_position();
  const int cls0 = (a.nparts * (g + a.Hkv * b)) & 7;  // class of partition 0
  // weight of partitions [0, k): partition q belongs to class (cls0 + q) mod 8
  auto wprefix = [&](int k) -> float {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = (c - cls0) & 7;  // first partition of class c
      const int cnt = k > d ? (k - 1 - d) / 8 + 1 : 0;
      acc += wcls[c] * (float)cnt;
    }
    return acc;
  };
  const float wtot = wprefix(a.nparts);
  // boundary q of n items split by weight (boundary 0 is 0, boundary nparts is n)
  auto split_at = [&](int q, int n) -> int {
    if (q >= a.nparts) return n;
    return min(n, (int)((float)n * (wprefix(q) / wtot) + 0.5f));
  };

  // This workgroup's tiles [t0, t1). A ring reads every tile; a linear cache
  // splits its readable range [gtb, gte) (window start .. current position)
  // over the partitions, so a partly filled or compacted cache keeps every
  // workgroup busy. Workgroups are placed on the chip's XCDs in dispatch
  // order (id mod 8), and XCDs stream at measurably different rates; with
  // dynamic claiming the split follows the rates the previous launches
  // measured per dispatch class (clamped to +-20 % of the mean), so the
  // partitions of a range finish together; otherwise it is even. With a keep
  // list the split divides the kept tiles (worked out below), otherwise the
  // tile range.
  int gtb = 0, gte = a.NT;
  int t0, t1;
  if constexpr (RING) {
    t0 = part * a.tpp;
    t1 = min(t0 + a.tpp, a.NT);
  } else {
    gte = max(0, min(a.NT, i_cur / kTile + 1));
    gtb = a.window > 0 ? min(gte, max(lo, 0) / kTile) : 0;
    t0 = __builtin_amdgcn_readfirstlane(gtb + split_at(part, gte - gtb));
    t1 = __builtin_amdgcn_readfirstlane(gtb + split_at(part + 1, gte - gtb));
  }

  // LDS carve-up (16-byte aligned parts first): per-wave side data (FP8
  // scales, ring positions of the claimed tiles), the appended row of this KV
  // head as the cache holds it (K and V values, then the FP8 scales), then
  // the kept-tile count, the claim counter, the appended row's flag and the
  // list split point, each wave's final max and sum per head, the block-sum
  // records of every list entry (sums per sub-block and head, and the running
  // max they are relative to), the list of kept tiles and the keep bitmap.
  // The waves' final outputs go to an area of their own after the bitmap.
  float* side_area = lds;                               // [NW][64 quads][4]
  uint8_t* app_lds = (uint8_t*)(side_area + NW * 256);  // [2][D * eb] bytes; the scales in its last 2 floats
  int* misc = (int*)(side_area + NW * 256 + kAppRowFloats);  // [8]
  float* mw = (float*)(misc + 8);                       // [NW][16]
  float* lw = mw + NW * 16;                             // [NW][16]
  float* e_rec = lw + NW * 16;                          // [tl_cap][NSUB][G]
  float* m_rec = e_rec + (size_t)a.tl_cap * NSUB * G;   // [tl_cap][G]
  int* tlist = (int*)(m_rec + (size_t)a.tl_cap * G);    // [tl_cap]
  uint32_t* kb = (uint32_t*)(tlist + a.tl_cap);         // [NT / 32 + 1]
  // the waves' outputs at the end: one slot per wave, 16-byte aligned after
  // the bitmap
  float* ow = lds + ((((float*)(kb + a.NT / 32 + 1) - lds) + 3) & ~(ptrdiff_t)3);
  if (threadIdx.x == 0) {
    misc[1] = NW;  // claim counter: batches 0 .. NW - 1 are the waves' first
    misc[2] = 0;
    misc[6] = -1;  // the partition count, once wave 0 has it
  }

  // With a keep mask, or a list of block ids to re-attend, on a linear cache
  // (tile = block), the kept tiles of the range [r_lo, r_hi) (the pair's
  // range with two partitions, else this workgroup's) become a bitmap, and
  // wave 0 compacts this workgroup's kept tiles into tlist, so other tiles
  // are never read. Without either, the list is implicit: entry i is tile
  // t0 + i.
  const uint32_t* keep_b = a.keep ? a.keep + (size_t)b * a.kwords : nullptr;
  const bool use_ids = !RING && a.ids != nullptr;
  const bool use_list = !RING && (keep_b != nullptr || use_ids);
  const int r_lo = gtb, r_hi = gte;
  const int nwords = (r_hi - r_lo + 31) >> 5;
  if (use_list) {
    if (use_ids) {
      // ids may repeat and come in any order
      for (int w = threadIdx.x; w < nwords; w += NTH) kb[w] = 0u;
      __syncthreads();
      const int nid = min(max(a.n_ids[b], 0), a.ids_stride);
      const int32_t* idb = a.ids + (size_t)b * a.ids_stride;
      for (int k = threadIdx.x; k < nid; k += NTH) {
        const int id = idb[k];
        if (id >= r_lo && id < r_hi) atomicOr(&kb[(id - r_lo) >> 5], 1u << ((id - r_lo) & 31));
      }
    } else {
      // the keep words, shifted to start at tile r_lo (tiles >= NBmax are kept)
      for (int w = threadIdx.x; w < nwords; w += NTH) {
        const int t = r_lo + 32 * w;
        const int wa = t >> 5, sh = t & 31;
        auto word = [&](int x) -> uint32_t {
          if (x >= a.kwords) return ~0u;
          uint32_t v = keep_b[x];
          const int past = 32 * x + 32 - a.nbmax;   // bits at or past NBmax
          if (past > 0) v |= past >= 32 ? ~0u : ~0u << (32 - past);
          return v;
        };
        uint32_t v = word(wa) >> sh;
        if (sh) v |= word(wa + 1) << (32 - sh);
        const int nvalid = r_hi - t;
        if (nvalid < 32) v &= (1u << nvalid) - 1u;
        kb[w] = v;
      }
    }
    __syncthreads();
  }

  // Block-sum records of this (sequence, KV head): tile t, sub-block sb,
  // query head hh of the group, laid out [NT][NSUB][G], so one workgroup's
  // records are one contiguous run; stored relative to the workgroup's max
  // per head. Every tile of the readable range gets them each launch
  // (skipped tiles zeros).
  const size_t rec_row = ((size_t)b * a.Hkv + g) * a.NT;
  const size_t hq0 = (size_t)g * G;
  auto e_index = [&](int t, int sb, int hh) -> size_t { return ((rec_row + t) * NSUB + sb) * G + hh; };
  if (use_list && wave == 0) {
    // the partitions divide the kept tiles by weight: this one takes entries
    // [e0, e1); its tiles run from the tile of entry e0 (the range start for
    // entry 0) to the tile of entry e1 (the range end past the last entry)
    int n_kept = 0;
    for (int c = 0; c < nwords; c += 64) {
      int cnt = c + lane < nwords ? __popc(kb[c + lane]) : 0;
      for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
      n_kept += cnt;
    }
    auto tile_of_entry = [&](int e) -> int {
      if (e <= 0) return r_lo;
      if (e >= n_kept) return r_hi;
      int found = r_hi, run = 0;
      for (int c = 0; c < nwords && found == r_hi; c += 64) {
        const uint32_t wv = c + lane < nwords ? kb[c + lane] : 0u;
        const int cnt = __popc(wv);
        int incl = cnt;  // inclusive prefix over the lanes
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        const uint64_t hit = __ballot(run + incl > e && cnt > 0);
        if (hit) {
          const int ln = __builtin_ctzll(hit);
          const uint32_t wsel = __shfl(wv, ln, 64);
          int rank = e - (run + __shfl(incl, ln, 64) - __popc(wsel));  // set bits to skip
          uint32_t x = wsel;
          for (int it = 0; it < 32 && rank > 0; ++it, --rank) x &= x - 1u;  // drop the skipped bits
          found = r_lo + 32 * (c + ln) + (x ? __builtin_ctz(x) : 31);
        }
        run += __shfl(incl, 63, 64);
      }
      return found;
    };
    t0 = part == 0 ? r_lo : tile_of_entry(split_at(part, n_kept));
    t1 = part == a.nparts - 1 ? r_hi : tile_of_entry(split_at(part + 1, n_kept));
    if (lane == 0) {
      misc[4] = t0;
      misc[5] = t1;
    }
    int n = 0;
    for (int c = t0; c < t1; c += 64) {
      const int t = c + lane;
      const int rb = t - r_lo;
      const bool kept = t < t1 && ((kb[rb >> 5] >> (rb & 31)) & 1u);
      const uint64_t m = __ballot(kept);
      if (kept) {
        const int e = n + __popcll(m & ((1ull << lane) - 1ull));
        tlist[e] = t;
      }
      n += __popcll(m);
    }
    if (lane == 0) misc[0] = n;
  }
  // (without a list the workgroup's first barrier comes after the first
  // tile loads are issued, below)
  if (use_list) {
    __syncthreads();
    t0 = __builtin_amdgcn_readfirstlane(misc[4]);
    t1 = __builtin_amdgcn_readfirstlane(misc[5]);
  }
  // Tiles that can hold a readable key.
  const int tb = t0, te = t1;
  // the appended slot if this workgroup's tiles hold it (set once the
  // position is known)
  int app_slot = -1, app_tile = -1;
  // uniform (readfirstlane): the tile offsets derived from these are scalar
  // operands of the buffer loads, which the compiler would otherwise wrap in
  // a per-lane loop
  const int n_items = __builtin_amdgcn_readfirstlane(use_list ? misc[0] : te - tb);
  const int n_batches = (n_items + BATCH - 1) / BATCH;
  auto tile_of = [&](int e) -> int {  // tile of list entry e < n_items (wave-uniform e)
    if (use_list) return __builtin_amdgcn_readfirstlane(tlist[e]);
    return tb + e;
  };
  // Wave w reads batch w first (its loads go out before the workgroup's
  // first barrier); then the waves take batches of BATCH consecutive list
  // entries from a shared counter, so a wave that is served faster by the
  // memory system reads more tiles and all waves of the workgroup finish
  // within about one batch. In deterministic mode wave w takes batches w,
  // w + NW, ... instead.
  int n_claimed = 0;
  auto claim = [&]() -> int {
    int v = 0;
    if (a.dyn) {
      if (lane == 0) v = __hip_atomic_fetch_add(&misc[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      v = __builtin_amdgcn_readfirstlane(v);
    } else {
      v = wave + NW * n_claimed;
    }
    ++n_claimed;
    return v;
  };

  float qf[QN];
  bf16x8 qb[D / 32 > 0 ? D / 32 : 1];
  auto convert_q = [&]() {
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int r = 0; r < QN / EPC; ++r) {
#pragma unroll
        for (int c = 0; c < QRUN; ++c) {
          const u32x4 w = qraw[r][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[r * EPC + 4 * c + e] = hreal ? bits_to_f32(w[e]) : 0.0f;
        }
      }
    } else {
      // the B operand of MFMA c is the lane's bf16 values 8 c .. 8 c + 7,
      // which are one 16-byte run as loaded (zeros for padding heads)
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 w = qraw[(8 * c) / EPC][((8 * c) % EPC) / 8];
        u32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = hreal ? w[e] : 0u;
        qb[c] = __builtin_bit_cast(bf16x8, m);
      }
    }
  };

  f32x4 oacc[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // Ring laps: positions read at step i lie in [i - C + 1, i], so at most two
  // laps (i / C and i / C - 1) share a tile; their parity names the sub-block.
  int lap_i = 0, lap_base = 0;  // (set with the position)

  TileAddr ad;
  {
    const size_t bg = (size_t)b * a.Hkv + g;
    const uint32_t region = (uint32_t)((size_t)a.C * D * eb);
    ad.k = make_rsrc((const char*)a.k + bg * region, region);
    ad.v = make_rsrc((const char*)a.v + bg * region, region);
    ad.koff = (uint32_t)(16 * lane);
    ad.voff = (uint32_t)(16 * lane);
  }

  // ---- per-slot side data (FP8 scales, ring positions) of a claimed batch ----
  // One gathered 16-byte-per-lane load brings all of it: lane l serves tile
  // l / QPT of the batch and quad q = l % QPT of that tile: K scales 4q..4q+3
  // for q < 4, V scales 4(q-4).. for q < 8, ring positions 4(q-8).. for
  // q < 12. The quads are staged in the wave's LDS area and read back per
  // tile, so a tile costs its KiB-wide K/V loads and nothing else on the
  // vector memory path. The next batch's quads are fetched while the current
  // batch is in use.
  const float* ks_b = a.ks ? a.ks + (size_t)b * a.C : nullptr;
  const float* vs_b = a.vs ? a.vs + (size_t)b * a.C : nullptr;
  const int32_t* pos_b = a.pos_of_slot ? a.pos_of_slot + (size_t)b * a.C : nullptr;
  constexpr bool SIDE = KV == KV_FP8 || RING;
  u32x4 pf = {0u, 0u, 0u, 0u};
  auto gather = [&](int bi) {
    if constexpr (SIDE) {
      // clamped to a real slot, also for a batch past the list (the first
      // batch is requested unconditionally)
      const int e = max(0, min(BATCH * bi + lane / QPT, n_items - 1));
      const int t = min(max(use_list ? tlist[e] : tb + e, 0), a.NT - 1);
      const int q = lane % QPT;
      const size_t base = (size_t)t * kTile;
      const void* src;
      if constexpr (KV == KV_FP8 && RING) {
        src = q < 4 ? (const void*)(ks_b + base + 4 * q)
            : q < 8 ? (const void*)(vs_b + base + 4 * (q - 4))
                    : (const void*)(pos_b + base + 4 * ((q - 8) & 3));
      } else if constexpr (KV == KV_FP8) {
        src = q < 4 ? (const void*)(ks_b + base + 4 * q) : (const void*)(vs_b + base + 4 * ((q - 4) & 3));
      } else {
        src = (const void*)(pos_b + base + 4 * ((q - 8) & 3));
      }
      pf = *(const u32x4*)src;
    }
  };
  float* side_w = side_area + wave * 256;
  auto commit = [&]() {
    if constexpr (SIDE) *(u32x4*)(side_w + 4 * lane) = pf;
  };

  // ---- the slot appended in this call ----
  // The appending wave publishes the values the cache will hold for it (this
  // KV head's K and V, the FP8 scales) in LDS and raises misc[2] before it
  // writes the cache, so a wave that reads the tile takes the slot from LDS
  // and never waits for those writes (what its tile load brought for the
  // slot, old or new, is replaced). K of slot t sits in the lanes with
  // lane % 16 == t (16 bytes per chunk); V of slot t in the 16 lanes of group
  // t / 4, interleaved with the three other slots of the group (element n of
  // dim group j at byte (4 n + t % 4) eb of its chunk).
  int app_ts = 0;
  auto patch_appended = [&](TileRegs<KV, D>& t, f32x4& ks, f32x4& vs, int4& cpos) {
    while (__hip_atomic_load(&misc[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    constexpr int NCH = TileRegs<KV, D>::NCH;
    if ((lane & 15) == app_ts) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) t.k[i] = *(const u32x4*)(app_lds + 64 * i + 16 * kg);
    }
    if (kg == (app_ts >> 2)) {
      const int e = app_ts & 3;
      const uint8_t* vrow = app_lds + D * eb;
      const int x0 = (lane & 15) * (D / 16);
      constexpr int EPV = 4 / eb;  // values of one slot per 16-byte chunk
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
#pragma unroll
        for (int w = 0; w < EPV; ++w) {
          const int x = x0 + EPV * i + w;
          const int bo = (4 * w + e) * eb;       // byte of the chunk
          const int dw = bo >> 2;                 // its dword (e is uniform)
          const uint32_t sh = 8u * (uint32_t)(bo & 3);
          uint32_t val, keep_mask;
          if constexpr (eb == 1) {
            val = (uint32_t)vrow[x] << sh;
            keep_mask = ~(0xFFu << sh);
          } else if constexpr (eb == 2) {
            val = (uint32_t)((const uint16_t*)vrow)[x] << sh;
            keep_mask = ~(0xFFFFu << sh);
          } else {
            val = ((const uint32_t*)vrow)[x];
            keep_mask = 0u;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q == dw) t.v[i][q] = (t.v[i][q] & keep_mask) | val;
        }
      }
      const int r = e;  // the slot's row among this lane's four
      if constexpr (KV == KV_FP8) {
        const float sk = ((const float*)app_lds)[kAppRowFloats - 2];
        const float sv = ((const float*)app_lds)[kAppRowFloats - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q == r) ks[q] = sk;
          if (q == r) vs[q] = sv;
        }
      }
      if constexpr (RING) {
        if (r == 0) cpos.x = i_cur;
        if (r == 1) cpos.y = i_cur;
        if (r == 2) cpos.z = i_cur;
        if (r == 3) cpos.w = i_cur;
      }
    }
  };

  // ---- one tile: online softmax, block sums, PV ----
  auto process = [&](TileRegs<KV, D>& cur, const int tile, const int tau, const int ent) {
    f32x4 ks = {0.f, 0.f, 0.f, 0.f}, vs = {0.f, 0.f, 0.f, 0.f};
    int4 cpos = make_int4(0, 0, 0, 0);
    if constexpr (KV == KV_FP8) {
      ks = *(const f32x4*)(side_w + (tau * QPT + kg) * 4);
      vs = *(const f32x4*)(side_w + (tau * QPT + 4 + kg) * 4);
    }
    if constexpr (RING) cpos = *(const int4*)(side_w + (tau * QPT + 8 + kg) * 4);
    if (tile == app_tile) patch_appended(cur, ks, vs, cpos);
    bool valid[4];
    int sub[4];
    bool all_valid, any_valid;
    // a ring tile whose slots are all readable and of one lap (the usual
    // case) skips the per-slot masks and sub-block split; its sub-block sums
    // come out bit for bit as the general path's
    int one_lap = -1;  // that lap's sub-block, or -1
    if constexpr (RING) {
      const int pmin = min(min(cpos.x, cpos.y), min(cpos.z, cpos.w));
      const int pmax = max(max(cpos.x, cpos.y), max(cpos.z, cpos.w));
      if (keep_b == nullptr && wave_all(pmin >= max(lo, 0) && pmax <= i_cur)) {
        if (wave_all(pmin >= lap_base)) one_lap = lap_i & 1;
        else if (wave_all(pmax < lap_base)) one_lap = (lap_i - 1) & 1;
      }
    }
    if (RING && one_lap >= 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        valid[r] = true;
        sub[r] = one_lap;
      }
      all_valid = any_valid = true;
    } else if constexpr (RING) {
      const int pr[4] = {cpos.x, cpos.y, cpos.z, cpos.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pr[r];
        bool v = p >= 0 && p <= i_cur && p >= lo;
        if (v && keep_b != nullptr) {
          const int blk = p >> 4;
          v = blk >= a.nbmax || ((keep_b[blk >> 5] >> (blk & 31)) & 1u);
        }
        valid[r] = v;
        sub[r] = ((p >= lap_base) ? lap_i : lap_i - 1) & 1;
      }
      all_valid = wave_all(valid[0] && valid[1] && valid[2] && valid[3]);
      any_valid = wave_any(valid[0] || valid[1] || valid[2] || valid[3]);
    } else {
      const int p0 = tile * kTile;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = p0 + 4 * kg + r;
        valid[r] = p <= i_cur && p >= lo;
        sub[r] = 0;
      }
      all_valid = p0 >= lo && p0 + kTile - 1 <= i_cur;  // uniform
      any_valid = true;                                  // tb..te only holds readable tiles
    }
    if (!any_valid) {
      if constexpr (SCORED) {
        if (kg == 0 && hreal) {
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb) e_rec[(ent * NSUB + sb) * G + h] = 0.0f;
          m_rec[ent * G + h] = -__builtin_inff();
        }
      }
      return;
    }

    // Codes of keys that are not read are zeroed before use: the cache may hold
    // anything there, and 0 * NaN would poison the PV product.
    if (!all_valid) {
      if constexpr (KV == KV_FP8) {
        // lane's V bytes: dim-group n, token e at byte 4 n + e
        const uint32_t m = (valid[0] ? 0x000000FFu : 0u) | (valid[1] ? 0x0000FF00u : 0u) |
                           (valid[2] ? 0x00FF0000u : 0u) | (valid[3] ? 0xFF000000u : 0u);
#pragma unroll
        for (int i = 0; i < TileRegs<KV, D>::NCH; ++i) cur.v[i] &= m;
      } else if constexpr (KV == KV_BF16) {
        const uint32_t m0 = (valid[0] ? 0x0000FFFFu : 0u) | (valid[1] ? 0xFFFF0000u : 0u);
        const uint32_t m1 = (valid[2] ? 0x0000FFFFu : 0u) | (valid[3] ? 0xFFFF0000u : 0u);
        const u32x4 m = {m0, m1, m0, m1};
#pragma unroll
        for (int i = 0; i < TileRegs<KV, D>::NCH; ++i) cur.v[i] &= m;
      } else {
        const u32x4 m = {valid[0] ? ~0u : 0u, valid[1] ? ~0u : 0u, valid[2] ? ~0u : 0u, valid[3] ? ~0u : 0u};
#pragma unroll
        for (int i = 0; i < TileRegs<KV, D>::NCH; ++i) cur.v[i] &= m;
      }
    }

    // ---- S^T = K Q^T ----
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int t = 0; t < QN; ++t)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_f32(cur.k[t / 4][t % 4]), qf[t], s, 0, 0, 0);
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[c]), qb[c], s, 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 w = cur.k[c >> 1];
        const u32x2 lo2 = fp8x4_to_bf16x4(w[2 * (c & 1)]);
        const u32x2 hi2 = fp8x4_to_bf16x4(w[2 * (c & 1) + 1]);
        const u32x4 kk = {lo2[0], lo2[1], hi2[0], hi2[1]};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kk), qb[c], s, 0, 0, 0);
      }
    }

    // ---- logits in log2 units, masked ----
    float tl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x;
      if constexpr (KV == KV_FP8) x = s[r] * (ks[r] * a.scale_log2);
      else x = s[r] * a.scale_log2;
      tl[r] = (all_valid || valid[r]) ? x : -__builtin_inff();
    }
    float mx = fmaxf(fmaxf(tl[0], tl[1]), fmaxf(tl[2], tl[3]));
    mx = rows_max(mx);
    // The reference the exponentials are taken against moves only when the
    // tile's max passes it by more than kLazyLog2 (or there is none yet): the
    // terms stay at most 2^kLazyLog2, and the output and sum are rescaled
    // rarely rather than at nearly every tile of a short range. Any
    // reference gives the same softmax up to rounding.
    const float m_new = mx > m_run + kLazyLog2 ? mx : m_run;
    const float alpha = fast_exp2(m_run - m_new);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(tl[r] - m_new);

    float esub0 = 0.f, esub1 = 0.f;
    if constexpr (NSUB == 2) {
      if (one_lap >= 0) {
        // the same sums as below with every slot in sub-block one_lap
        float e = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) e += p[r];
        e = rows_sum(e);
        esub0 = one_lap ? 0.0f : e;
        esub1 = one_lap ? e : 0.0f;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          esub0 += sub[r] ? 0.0f : p[r];
          esub1 += sub[r] ? p[r] : 0.0f;
        }
        esub0 = rows_sum(esub0);
        esub1 = rows_sum(esub1);
      }
    } else {
      esub0 = rows_sum((p[0] + p[1]) + (p[2] + p[3]));
    }
    l_run = l_run * alpha + (esub0 + esub1);

    if constexpr (SCORED) {
      // the tile's block sums and the running max they are relative to
      if (kg == 0 && hreal) {
        e_rec[(ent * NSUB) * G + h] = esub0;
        if constexpr (NSUB == 2) e_rec[(ent * NSUB + 1) * G + h] = esub1;
        m_rec[ent * G + h] = m_new;
      }
    }

    if (wave_any(alpha != 1.0f)) {
#pragma unroll
      for (int n = 0; n < NC; ++n) oacc[n] *= alpha;
    }
    m_run = m_new;

    // ---- O^T += V^T P^T ----
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = 4 * n + r;  // lane's V element: dim (D/16) j + n, token 4 kg + r
          oacc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_f32(cur.v[u / 4][u % 4]), p[r], oacc[n], 0, 0, 0);
        }
      }
    } else {
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (KV == KV_FP8) pw[r] = p[r] * vs[r];
        else pw[r] = p[r];
      }
      bf16x4 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] = (__bf16)pw[r];
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        u32x2 vv;
        if constexpr (KV == KV_BF16) {
          // 4 bf16 per n: chunk n/2, dwords 2 (n%2), 2 (n%2) + 1
          vv[0] = cur.v[n >> 1][2 * (n & 1)];
          vv[1] = cur.v[n >> 1][2 * (n & 1) + 1];
        } else {
          // 4 codes per n: chunk n/4, dword n%4
          vv = fp8x4_to_bf16x4(cur.v[n >> 2][n & 3]);
        }
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv),
                                                            __builtin_bit_cast(s16x4, pb), oacc[n], 0, 0, 0);
      }
    }
  };

  // ---- software pipeline: NBUF - 1 tiles of this wave in flight ----
  // Every vector-memory load in the loop is unconditional, so the compiler's
  // wait counts keep all of them in flight; loads past the last list entry
  // use an offset beyond the buffer's range, which returns zeros without a
  // memory access. Tile i of the current batch sits in buf[i]; step s loads
  // the tile NBUF - 1 entries ahead (the last of this batch, then the first
  // ones of the next claimed batch) and processes tile s.
  const uint32_t oob = (uint32_t)((size_t)a.C * D * eb);  // first offset past the region
  constexpr uint32_t tile_bytes = (uint32_t)kTile * D * eb;
  auto soff_of = [&](int bi, int i) -> uint32_t {
    const int e = BATCH * bi + i;
    // a scalar operand of the loads: uniform, and marked so
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(e < n_items ? (uint32_t)tile_of(e) * tile_bytes : oob));
  };
  // ---- fused append (last wave, before its first claim; a ring's row
  // before the first barrier) ----
  // Same encoding as kvs_append_rows: the FP8 scale covers every KV head of
  // the position, so each workgroup of the sequence derives it from the whole
  // row (identical values); this workgroup writes its own head's codes.
  uint32_t kbits[XPL], vbits[XPL];
  float sk = 0.0f, sv = 0.0f;
  auto encode_row = [&]() {
    const int n = app_n;
    const size_t rb = app_rb;
    const int sbf = a.app_bf16;
    if constexpr (KV == KV_FP8) {
      float mk = 0.0f, mv = 0.0f;
      for (int i = 8 * lane; i < n; i += 8 * 64) {  // 8 values per lane and load (n % 8 == 0)
        float xk[8], xv[8];
        const bool pre = i < (sbf ? 1024 : 512);  // fetched at kernel entry
        if (sbf) {
          const u32x4 wk = pre ? app_k0[i >= 512] : *(const u32x4*)((const uint16_t*)a.app_k + rb + i);
          const u32x4 wv = pre ? app_v0[i >= 512] : *(const u32x4*)((const uint16_t*)a.app_v + rb + i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xk[2 * e] = bf16_lo(wk[e]);
            xk[2 * e + 1] = bf16_hi(wk[e]);
            xv[2 * e] = bf16_lo(wv[e]);
            xv[2 * e + 1] = bf16_hi(wv[e]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const f32x4 fk = pre ? __builtin_bit_cast(f32x4, app_k0[c]) : *(const f32x4*)((const float*)a.app_k + rb + i + 4 * c);
            const f32x4 fv = pre ? __builtin_bit_cast(f32x4, app_v0[c]) : *(const f32x4*)((const float*)a.app_v + rb + i + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              xk[4 * c + e] = fk[e];
              xv[4 * c + e] = fv[e];
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mk = fmaxf(mk, fabsf(xk[e]));
          mv = fmaxf(mv, fabsf(xv[e]));
        }
      }
      mk = wave_max(mk);
      mv = wave_max(mv);
      sk = fp8_scale_of(mk);
      sv = fp8_scale_of(mv);
    }
    // this KV head's values as the cache holds them (codes, bf16 or f32
    // bits), dims lane and lane + 64, from the values fetched at entry: first
    // into LDS for the waves that read the tile in this call (they patch the
    // slot from there), then the flag, then the cache writes, which no wave
    // of this call waits for
#pragma unroll
    for (int c = 0; c < XPL; ++c) {
      const int x = lane + 64 * c;
      if (x >= D) continue;
      if constexpr (KV == KV_FP8) {
        const float xk = sbf ? bf16_lo(app_hk[c]) : bits_to_f32(app_hk[c]);
        const float xv = sbf ? bf16_lo(app_hv[c]) : bits_to_f32(app_hv[c]);
        kbits[c] = encode_with_scale(xk, sk);
        vbits[c] = encode_with_scale(xv, sv);
        app_lds[x] = (uint8_t)kbits[c];
        app_lds[D + x] = (uint8_t)vbits[c];
      } else if constexpr (KV == KV_BF16) {
        kbits[c] = app_hk[c];
        vbits[c] = app_hv[c];
        ((uint16_t*)app_lds)[x] = (uint16_t)kbits[c];
        ((uint16_t*)app_lds)[D + x] = (uint16_t)vbits[c];
      } else {
        kbits[c] = app_hk[c];
        vbits[c] = app_hv[c];
        ((uint32_t*)app_lds)[x] = kbits[c];
        ((uint32_t*)app_lds)[D + x] = vbits[c];
      }
    }
    if (lane == 0) {
      ((float*)app_lds)[kAppRowFloats - 2] = sk;
      ((float*)app_lds)[kAppRowFloats - 1] = sv;
    }
  };
  auto publish_row = [&]() {
    // the wave's LDS writes are done (lgkmcnt 0, no wait on memory) before
    // the flag is raised
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(&misc[2], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int t = app_slot & (kTile - 1);
    const size_t base = (((size_t)b * a.Hkv + g) * (size_t)(a.C / kTile) + app_tile) * tile_bytes;
    char* kc = (char*)const_cast<void*>(a.k) + base;
    char* vc = (char*)const_cast<void*>(a.v) + base;
#pragma unroll
    for (int c = 0; c < XPL; ++c) {
      const int x = lane + 64 * c;
      if (x >= D) continue;
      char* kp = kc + k_tile_offset(t, x, eb);
      char* vp = vc + v_tile_offset(t, x, D, eb);
      if constexpr (KV == KV_FP8) {
        *(uint8_t*)kp = (uint8_t)kbits[c];
        *(uint8_t*)vp = (uint8_t)vbits[c];
      } else if constexpr (KV == KV_BF16) {
        *(uint16_t*)kp = (uint16_t)kbits[c];
        *(uint16_t*)vp = (uint16_t)vbits[c];
      } else {
        *(uint32_t*)kp = kbits[c];
        *(uint32_t*)vp = vbits[c];
      }
    }
    if (lane == 0) {
      if constexpr (KV == KV_FP8) {
        const_cast<float*>(a.ks)[(size_t)b * a.C + app_slot] = sk;
        const_cast<float*>(a.vs)[(size_t)b * a.C + app_slot] = sv;
      }
      if constexpr (RING) const_cast<int32_t*>(a.pos_of_slot)[(size_t)b * a.C + app_slot] = i_cur;
    }
  };
  // First batch of this wave: its own index, its side data and first tiles
  // requested before the workgroup's first barrier (without a keep list),
  // the batch holding the appended slot too (the slot is patched from LDS).
  // They are requested even when the wave has no batch (side data of a real
  // slot, tile loads past the buffer's range: zeros without a memory
  // access): a conditional request would make the compiler's wait counts
  // assume the shorter queue, so the append below would wait for these
  // tiles instead of only for the row fetched at entry.
  TileRegs<KV, D> buf[NBUF];
  int cur = wave;
  ++n_claimed;
  gather(cur);
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) load_tile<KV, D, RING>(buf[i], ad, soff_of(cur, i));
  if constexpr (RING) {
    i_cur = __builtin_amdgcn_readfirstlane(ring_pos);
    set_position();
    lap_i = i_cur / a.C;
    lap_base = lap_i * a.C;
  }
  app_slot = (app_cand_tile >= tb && app_cand_tile < te) ? app_cand : -1;
  app_tile = app_slot >= 0 ? app_cand_tile : -1;
  app_ts = app_slot & (kTile - 1);
  // A ring's appending wave encodes the new row into LDS now, while the
  // first tiles are on their way; it publishes it after the barrier.
  if (RING && app_slot >= 0 && wave == NW - 1) encode_row();
  // the claim counter and the append flag are initialised (with a keep list
  // the list's barrier has seen to that)
  if (!use_list) __syncthreads();
  if (app_slot >= 0 && wave == NW - 1) {
    if constexpr (!RING) encode_row();
    publish_row();
  }

  int n_done = 0;  // tiles this wave processed
  if (cur < n_batches) {
    convert_q();
    while (true) {
      commit();
      const int nxt = claim();
      gather(nxt);
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        load_tile<KV, D, RING>(buf[(s + NBUF - 1) % NBUF], ad,
                               s == 0 ? soff_of(cur, NBUF - 1) : soff_of(nxt, s - 1));
        const int e = BATCH * cur + s;
        if (e < n_items) process(buf[s], tile_of(e), s, e);
      }
      n_done += min(BATCH, n_items - BATCH * cur);
      if (nxt >= n_batches) break;
      cur = nxt;
    }
  }

  // ---- end of the partition: records, then the workgroup's partial ----
  // This wave's running max, sum and output (unscaled) per head go to LDS
  // for the workgroup's merge; the outputs in an area of their own that no
  // wave uses while streaming, [NW][G][DP] with rows padded by 4 floats
  // against bank conflicts.
  constexpr int DP = D + 4;
  if (hreal) {
    if (kg == 0) {
      mw[wave * 16 + h] = m_run;
      lw[wave * 16 + h] = l_run;
    }
    float* dst = ow + (wave * G + h) * DP;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d0 = NC * (4 * kg + r);  // lane's dims d0 .. d0 + NC - 1
      if constexpr (NC % 4 == 0) {
#pragma unroll
        for (int n0 = 0; n0 < NC; n0 += 4)
          *(f32x4*)(dst + d0 + n0) = f32x4{oacc[n0][r], oacc[n0 + 1][r], oacc[n0 + 2][r], oacc[n0 + 3][r]};
      } else {
#pragma unroll
        for (int n = 0; n < NC; ++n) dst[d0 + n] = oacc[n][r];
      }
    }
  }
  // this wave's streaming time (clock ticks, 100 MHz), stored with its tile
  // count after the handshake below, for the split of later launches
  const float wave_ticks = (float)(__builtin_amdgcn_s_memrealtime() - clk0);
  // Stores that nothing in this launch reads (clock records, block records
  // and a linear range's partition map) go out after the partial's
  // handshake: vector-memory completions count in issue order, so a store
  // issued before the partial would be waited for with it.
  auto store_side = [&]() {
    if (a.ws_time != nullptr && lane == 0) {
      float* tm = a.ws_time + ((size_t)wg_id * NW + wave) * 2;
      tm[0] = (float)n_done;
      tm[1] = wave_ticks;
    }
  };
  __syncthreads();
  auto wg_max = [&](int hh) -> float {
    float M = -__builtin_inff();
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * 16 + hh]);
    return M;
  };

  // The block-sum records, rescaled from the running max at the time to the
  // workgroup max per head, are stored as contiguous runs once every wave is
  // done: global stores inside the streaming loop would hold up the in-order
  // completion count the tile loads are waited on with. Threads th0 .. th0 +
  // nth - 1 of the workgroup store them (all of them, or the waves other than
  // wave 0 while it runs the output-merge handshake below).
  auto store_records = [&](int th0, int nth) {
    const int per_e = NSUB * G;
    const int tid = threadIdx.x - th0;
    if (G % 4 == 0 && nth % (per_e / 4) == 0) {
      // four heads of one sub-block per 16-byte piece (an entry's records
      // and maxima are contiguous per head): a thread keeps piece c of every
      // (nth / pieces)-th entry, with its four heads' workgroup maxima
      const int cpe = per_e / 4;
      const int r0 = 4 * (tid % cpe), h0 = r0 % G;
      float M[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) M[i] = wg_max(h0 + i);
      const int estep = nth / cpe;
      for (int e = tid / cpe; e < n_items; e += estep) {
        const f32x4 ev = *(const f32x4*)(e_rec + e * per_e + r0);
        const f32x4 mr = *(const f32x4*)(m_rec + e * G + h0);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = (M[i] == -__builtin_inff() || mr[i] == -__builtin_inff()) ? 0.0f : ev[i] * fast_exp2(mr[i] - M[i]);
        const int t = use_list ? tlist[e] : tb + e;
        *(f32x4*)(a.ws_e + e_index(t, 0, 0) + r0) = v;
      }
    } else if (nth % per_e == 0) {
      // the usual case: a thread keeps one (sub-block, head) r of every
      // (nth / per_e)-th entry, so its head's workgroup max is taken once
      const int r = tid % per_e, hh = r % G;
      const float M = wg_max(hh);
      const int estep = nth / per_e;
      for (int e = tid / per_e; e < n_items; e += estep) {
        const float mr = m_rec[e * G + hh];
        const float v =
            (M == -__builtin_inff() || mr == -__builtin_inff()) ? 0.0f : e_rec[e * per_e + r] * fast_exp2(mr - M);
        const int t = use_list ? tlist[e] : tb + e;
        a.ws_e[e_index(t, 0, 0) + r] = v;
      }
    } else {
      for (int x = tid; x < n_items * per_e; x += nth) {
        const int e = x / per_e;
        const int hh = x % G;
        const float M = wg_max(hh);
        const float mr = m_rec[e * G + hh];
        const float v = (M == -__builtin_inff() || mr == -__builtin_inff()) ? 0.0f : e_rec[x] * fast_exp2(mr - M);
        const int t = use_list ? tlist[e] : tb + e;
        a.ws_e[e_index(t, 0, 0) + (x - e * per_e)] = v;
      }
    }
    if (use_list && G % 4 == 0) {
      // tiles of the range that were not kept: zero records (16-byte pieces)
      const int cpe = per_e / 4;
      for (int x = tid; x < (te - tb) * cpe; x += nth) {
        const int tl = x / cpe;
        const int rb = tb + tl - r_lo;
        if (!((kb[rb >> 5] >> (rb & 31)) & 1u))
          *(f32x4*)(a.ws_e + e_index(tb + tl, 0, 0) + 4 * (x - tl * cpe)) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else if (use_list) {
      // tiles of the range that were not kept: zero records
      for (int x = tid; x < (te - tb) * per_e; x += nth) {
        const int tl = x / per_e;
        const int rb = tb + tl - r_lo;
        if (!((kb[rb >> 5] >> (rb & 31)) & 1u)) a.ws_e[e_index(tb + tl, 0, 0) + (x - tl * per_e)] = 0.0f;
      }
    }
    // a linear range's partition map: this partition's index at each of its
    // tiles, for the mass combine to find the tile's merge weights (a ring's
    // partitions are fixed ranges of tpp tiles)
    if constexpr (!RING)
      for (int x = tid; x < te - tb; x += nth) a.ws_pid[rec_row + tb + x] = part;
  };

  // The waves' outputs merge into one partial per workgroup, after the one
  // barrier above: the thread of output (head hh, dim dd) scales each wave's
  // output by 2^(m_wave - M), M the workgroup max of the head (0 for a wave
  // that read nothing: its output and sum are zero), and adds the terms in
  // wave order; the thread of dim 0 does the same for the sums and stores
  // M and the sum. One batch of LDS reads per output, no further barrier.
  const size_t pbase = (size_t)b * a.Hq + hq0;  // first head of the group
  auto store_partial = [&]() {
    for (int x = threadIdx.x; x < G * D; x += NTH) {
      const int hh = x / D, dd = x % D;
      float mv[NW], t[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mv[w] = mw[w * 16 + hh];
        t[w] = ow[(w * G + hh) * DP + dd];
      }
      float M = -__builtin_inff();
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mv[w]);
      float f[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) f[w] = mv[w] == -__builtin_inff() ? 0.0f : fast_exp2(mv[w] - M);
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) o += t[w] * f[w];
      // the partials go to memory past the (per-XCD, non-coherent) L2, for
      // the merge below: relaxed system-scope stores are written through
      __hip_atomic_store(&a.ws_o[((pbase + hh) * a.nparts + part) * D + dd], o, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      if (dd == 0) {
        float lt[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) lt[w] = lw[w * 16 + hh];
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) l += lt[w] * f[w];
        __hip_atomic_store(&a.ws_m[(pbase + hh) * a.nparts + part], M, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&a.ws_l[(pbase + hh) * a.nparts + part], l, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  };
  store_partial();

  // Head hh's output merge by one wave, for at most eight partitions: lane p
  // takes partition p's maximum and sum (past P: -inf and 0), M and L come
  // from reductions over lanes 0 .. 7, lane p's weight w_p = 2^(m_p - M) / L
  // (0 for an empty partition) is stored for the mass combines and read into
  // a scalar register, and each lane sums sum_p w_p o_p for its DPL
  // consecutive dims with four accumulators (p mod 4) in ascending p. All
  // loads are system coherent (the partials were written through) and go out
  // together.
  auto merge_head = [&](int hh) {
    const int P = a.nparts;
    constexpr int DPL = D >= 64 ? D / 64 : 1;  // dims per lane
    const size_t row = (pbase + hh) * P;        // this head's partitions
    constexpr int kSysCoherent = 1 | 16;        // sc0 sc1
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(a.ws_o + row * D, (uint32_t)((size_t)P * D * 4));
    const int d0 = min(lane * DPL, D - DPL);
    float ov[8][DPL];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= P) continue;  // (wave-uniform: every load is waited for at once below)
      const int off = (k * D + d0) * 4;
      if constexpr (DPL == 2) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(orsrc, off, 0, kSysCoherent));
        ov[k][0] = bits_to_f32(v[0]);
        ov[k][1] = bits_to_f32(v[1]);
      } else {
        ov[k][0] = bits_to_f32(__builtin_amdgcn_raw_buffer_load_b32(orsrc, off, 0, kSysCoherent));
      }
    }
    const int pl = min(lane & 7, P - 1);
    const float m_raw = __hip_atomic_load(a.ws_m + row + pl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const float l_raw = __hip_atomic_load(a.ws_l + row + pl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const bool mine = (lane & 7) < P;
    const float mp = mine ? m_raw : -__builtin_inff();
    const float M = oct_max(mp);
    const float ep = (M == -__builtin_inff() || mp == -__builtin_inff()) ? 0.0f : fast_exp2(mp - M);
    const float L = oct_sum(mine ? l_raw * ep : 0.0f);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const float w = (mp == -__builtin_inff() || inv == 0.0f) ? 0.0f : ep * inv;
    if (lane < P) a.ws_w[((size_t)b * P + lane) * a.Hq + hq0 + hh] = w;
    float acc[4][DPL];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[k][e] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k >= P) continue;
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[k & 3][e] += ov[k][e] * wk;
    }
    if (lane * DPL < D) {
      float o[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = (acc[0][e] + acc[1][e]) + (acc[2][e] + acc[3][e]);
      const size_t oi = (pbase + hh) * D + lane * DPL;
      if constexpr (KV != KV_F32) {
        if constexpr (DPL == 2) {
          *(uint32_t*)((uint16_t*)a.out + oi) =
              (uint32_t)f32_to_bf16_rne(o[0]) | ((uint32_t)f32_to_bf16_rne(o[1]) << 16);
        } else {
          ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(o[0]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) ((float*)a.out)[oi + e] = o[e];
      }
    }
  };

  // ---- the last partition of this (sequence, KV head) to finish merges the
  // group's outputs, so the output needs no further launch. Each partition,
  // once its partial is in memory, adds 1 to the pair's completion counter
  // (zero at entry: the workspace contract) with one system-scope atomic,
  // performed at memory past every XCD's L2; the partition that reads back
  // nparts - 1 is the last and merges, then puts the counter back to zero, so
  // each call ends with it zero again (the next call, or a graph replay,
  // starts clean). One round trip to memory per partition and no retries
  // (a compare-and-swap took one retry per partition finishing at the same
  // time; a flag per partition took a store and then a load). ----
  // The partials are write-through stores; once every wave has them
  // acknowledged (vmcnt 0) they are in memory, so the flag needs no cache
  // writeback, and the merging workgroup reads them past its caches.
  // (Device-scope fences here write back the whole L2 per workgroup and
  // cost tens of microseconds per launch.)
  // With at most eight partitions and no more heads than waves, wave 0
  // counts, waves 1 .. G - 1 wait for the count in LDS, and in the last
  // partition wave h merges head h, while waves G .. NW - 1 store the block
  // records (with G = NW every wave stores its share after the merge: the
  // completion count is per wave, so records stored first would be waited
  // for with the merge's loads). Otherwise wave 0 counts and merges alone
  // while the other waves store the records.
  if (a.pair_flag == nullptr) {
    store_side();
    if constexpr (SCORED) store_records(0, NTH);
    return;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores acknowledged
  __syncthreads();
  if (a.nparts <= 8 && G <= NW) {
    const int P = a.nparts;
    if (wave >= G) {
      store_side();
      if constexpr (SCORED) store_records(64 * G, NTH - 64 * G);
      return;
    }
    uint32_t* fl = a.pair_flag + ((size_t)b * a.Hkv + g) * P;  // word 0: the pair's counter
    int cnt;
    if (wave == 0) {
      uint32_t old = 0u;
      // system scope: performed at memory, past every XCD's L2
      if (lane == 0) old = __hip_atomic_fetch_add(fl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      // (non-negative even for a counter that did not start at zero)
      cnt = __builtin_amdgcn_readfirstlane((int)min(old, 0x7FFFFFFFu));
      if (lane == 0) __hip_atomic_store(&misc[6], cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      // misc[6] is -1 from entry until wave 0 has the count (a round trip)
      while ((cnt = __hip_atomic_load(&misc[6], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < 0)
        __builtin_amdgcn_s_sleep(1);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
    }
    const bool last = cnt == P - 1;
    if (last) merge_head(wave);
    // every partition has counted: back to zero for the next call (after the
    // merge's loads, which would otherwise wait for this store)
    if (last && wave == 0 && lane == 0) __hip_atomic_store(fl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    store_side();
    if constexpr (SCORED)
      if (G == NW) store_records(0, NTH);
    return;
  }
  if (wave != 0) {
    store_side();
    if constexpr (SCORED) store_records(64, NTH - 64);
    return;
  }
  // Wave 0 alone from here: it counts the partition and, if last, merges
  // (it stores no records, so its loads wait for nothing else; no barrier
  // follows, and the merge tables sit in the waves' output area, which the
  // other waves no longer use).
  uint32_t* fl = a.pair_flag + ((size_t)b * a.Hkv + g) * a.nparts;  // word 0: the pair's counter
  uint32_t old = 0u;
  // system scope: performed at memory, past every XCD's L2
  if (lane == 0) old = __hip_atomic_fetch_add(fl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  old = (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
  if (old == (uint32_t)(a.nparts - 1)) {
    const int P = a.nparts;
    auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM); };
    float* mT = ow;             // [G][P] partition maxima
    float* lT = mT + G * P;     // [G][P] partition sums
    float* wT = lT + G * P;     // [P][G] weights
    // The outputs in groups of 4 dims: group q is head 4q / D, dims 4q % D
    // .. + 3; lane takes groups lane, lane + 64, ... The partials of the
    // lane's first two groups (first 8 partitions) are requested with the
    // maxima and sums, 16-byte loads past the caches (system coherent, as
    // the partials were written through), so all arrive in one round trip.
    const int n_grp = G * D / 4;
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(a.ws_o + pbase * P * D, (uint32_t)((size_t)G * P * D * 4));
    constexpr int kSysCoherent = 1 | 16;  // sc0 sc1
    auto ld4 = [&](int grp, int p) -> f32x4 {
      const int hh = 4 * grp / D, d0 = 4 * grp % D;
      return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           orsrc, (int)((((size_t)hh * P + p) * D + d0) * 4), 0, kSysCoherent));
    };
    f32x4 pre[2][8];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int k = 0; k < 8; ++k) pre[gi][k] = ld4(min(lane + 64 * gi, n_grp - 1), min(k, P - 1));
    for (int x0 = 0; x0 < G * P; x0 += 64) {
      const int x = x0 + lane;
      const float mv = x < G * P ? ld(a.ws_m + pbase * P + x) : 0.0f;
      const float lv = x < G * P ? ld(a.ws_l + pbase * P + x) : 0.0f;
      if (x < G * P) {
        mT[x] = mv;
        lT[x] = lv;
      }
    }
    // the tables are read by other lanes of this wave: LDS operations of a
    // wave complete in order; the fence keeps the compiler from reordering
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // one lane per (head, partition); the same weights scale the block
    // records in the mass combine
    for (int x = lane; x < G * P; x += 64) {
      const int hh = x / P, p = x % P;
      const float w = merge_weight(mT + hh * P, lT + hh * P, P, p);
      wT[p * G + hh] = w;
      a.ws_w[((size_t)b * P + p) * a.Hq + hq0 + hh] = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // sum_p o_p w_p with four accumulators (p mod 4) in ascending p; first:
    // the group's partials of partitions 0 .. 7
    // (eight weights read in one batch and terms past P selected away, not
    // branched over: a read under a branch is waited for on its own)
    auto out_group = [&](int grp, const f32x4 (&first)[8]) {
      const int hh = 4 * grp / D;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      f32x4 acc[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = zero;
      float wk[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) wk[k] = wT[min(k, P - 1) * G + hh];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const f32x4 t = first[k] * wk[k];
        acc[k & 3] += k < P ? t : zero;
      }
      for (int p0 = 8; p0 < P; p0 += 8) {
        f32x4 ov[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          ov[k] = ld4(grp, min(p0 + k, P - 1));
          wk[k] = wT[min(p0 + k, P - 1) * G + hh];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const f32x4 t = ov[k] * wk[k];
          acc[k & 3] += p0 + k < P ? t : zero;
        }
      }
      const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      const size_t oi = (pbase + hh) * D + 4 * grp % D;
      if constexpr (KV != KV_F32) {
        uint32_t* dst = (uint32_t*)((uint16_t*)a.out + oi);
        dst[0] = (uint32_t)f32_to_bf16_rne(sum[0]) | ((uint32_t)f32_to_bf16_rne(sum[1]) << 16);
        dst[1] = (uint32_t)f32_to_bf16_rne(sum[2]) | ((uint32_t)f32_to_bf16_rne(sum[3]) << 16);
      } else {
        *(f32x4*)((float*)a.out + oi) = sum;
      }
    };
    if (lane < n_grp) out_group(lane, pre[0]);
    if (lane + 64 < n_grp) out_group(lane + 64, pre[1]);
    for (int grp = lane + 128; grp < n_grp; grp += 64) {
      f32x4 fr[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) fr[k] = ld4(grp, min(k, P - 1));
      out_group(grp, fr);
    }
    if (lane == 0) __hip_atomic_store(fl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  store_side();
}

// ---- block records for the mass combines ----
// Records of heads hc .. hc + HC - 1 (clamped to Hq - 1; the caller masks the
// heads past Hq) of one tile, one layer and one sequence: rec covers the
// sequence's [Hkv][NT][NSUB][G] records, vo is the tile's byte offset
// (tc NSUB G 4). Head h sits at row h / G, entry h % G: the per-head part of
// the address is the same for the whole wave (a scalar offset), so the loads
// need one address register between them. With V4 (G % 4 == 0) four heads of
// a group come in one 16-byte load, consecutive lanes (tiles) reading
// consecutive 16-byte pieces.
template <int NSUB, int HC, bool V4>
__device__ __forceinline__ void load_rec(float (&ev)[NSUB][HC], __amdgpu_buffer_rsrc_t rec, uint32_t vo, int hc,
                                         int Hq, int G, int NT) {
  if constexpr (V4) {
#pragma unroll
    for (int q = 0; q < HC / 4; ++q) {
      const int hh = min(hc + 4 * q, Hq - 4);
      const int gg = hh / G;
      const uint32_t so = ((uint32_t)gg * NT * NSUB * G + (hh - gg * G)) * 4;
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        const f32x4 e4 =
            __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rec, (int)vo, (int)(so + sb * G * 4), 0));
#pragma unroll
        for (int k = 0; k < 4; ++k) ev[sb][4 * q + k] = e4[k];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < HC; ++k) {
      const int hh = min(hc + k, Hq - 1);
      const int gg = hh / G;
      const uint32_t so = ((uint32_t)gg * NT * NSUB * G + (hh - gg * G)) * 4;
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb)
        ev[sb][k] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rec, (int)vo, (int)(so + sb * G * 4), 0));
    }
  }
}

// Partition that produced tile tc's records for the KV heads of a record
// chunk (heads hc .. hc + HC - 1, one entry per 4-head group with V4, else
// per head): a ring's partitions are fixed ranges of tpp tiles; a linear
// range's come from the partition map the partial kernel stored
// ([B][Hkv][NT] ints, map = this sequence's rows), loaded with the chunk's
// records (clamped to 0 .. P - 1 where used).
template <int HC, bool V4, bool RING>
__device__ __forceinline__ void load_pid(int (&pv)[V4 ? HC / 4 : HC], __amdgpu_buffer_rsrc_t map, int tc, int hc,
                                         int Hq, int G, int NT, int P, int tpp) {
  constexpr int PG = V4 ? 4 : 1;
#pragma unroll
  for (int i = 0; i < HC / PG; ++i) {
    if constexpr (RING) {
      pv[i] = min(tc / tpp, P - 1);
    } else {
      const int gg = min(hc + PG * i, Hq - PG) / G;
      pv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(map, tc * 4, (int)((uint32_t)gg * NT * 4), 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: grid (n_mass_chunks + n_layers, B), 256 threads: the block masses
// of n_layers calls (one for kvs_decode_combine, a whole step's layers for
// kvs_tap_masses), added in call order.
// Each thread adds, for its tile and sub-block, sum_h E w_p(tile),h over the
// heads in ascending order, layer after layer, into mass_accum: E is the
// tile's record relative to its partition's max, and w_p,h = 2^(m_p - M_h) /
// L_h (M_h = max_p m_p, L_h = sum_p l_p 2^(m_p - M_h)) the weight the partial
// kernel's output merge computed and stored for partition p and head h. The
// extra columns (sequence 0 only) refresh each layer's per-class streaming
// rates from its clock records.
// ---------------------------------------------------------------------------
template <bool RING, bool V4>
__global__ __launch_bounds__(256) void kvs_combine(CombineArgs a) {
  extern __shared__ float lds[];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int P = a.nparts, L = a.n_layers;
  auto ws_f = [&](int l, size_t off) { return (const float*)(a.lws[l] + off); };

  if ((int)blockIdx.x >= a.n_mass_chunks) {
    // ---- rates of one layer: per dispatch class (workgroup id mod 8),
    // tiles per tick of its workgroups (a workgroup's time is its slowest
    // wave's), relative to the mean over classes, blended half-and-half into
    // the stored value ----
    const int l = blockIdx.x - a.n_mass_chunks;
    if (b != 0 || l >= L) return;
    const float* ws_time = ws_f(l, a.off_time);
    float* rates = (float*)(a.lws[l] + a.off_rates);
    float* ct = lds;       // [8] tiles
    float* cs = lds + 8;   // [8] ticks
    if (tid < 16) lds[tid] = 0.0f;
    __syncthreads();
    for (int w = tid; w < a.n_wg; w += 256) {
      float tiles = 0.0f, ticks = 0.0f;
      for (int k = 0; k < kPartialWaves; ++k) {
        const float* tm = ws_time + ((size_t)w * kPartialWaves + k) * 2;
        tiles += tm[0];
        ticks = fmaxf(ticks, tm[1]);
      }
      if (tiles > 0.0f && ticks > 0.0f && tiles < 1e9f && ticks < 1e9f) {
        atomicAdd(&ct[w & 7], tiles);
        atomicAdd(&cs[w & 7], ticks);
      }
    }
    __syncthreads();
    if (tid < 8) {
      // every thread derives the mean itself, then blends its own class
      float mean = 0.0f;
      int nv = 0;
      for (int c = 0; c < 8; ++c) {
        const float r = cs[c] > 0.0f ? ct[c] / cs[c] : 0.0f;
        if (r > 0.0f) {
          mean += r;
          ++nv;
        }
      }
      const float r = cs[tid] > 0.0f ? ct[tid] / cs[tid] : 0.0f;
      const float old = rates[tid];
      if (nv > 0 && r > 0.0f) {
        const float rel = fminf(fmaxf(r / (mean / (float)nv), 0.5f), 2.0f);
        const bool ok = old >= 0.5f && old <= 2.0f;  // NaN fails too
        rates[tid] = ok ? 0.5f * old + 0.5f * rel : rel;
      }
    }
    return;
  }

  // Each workgroup first issues the global loads that need nothing from the
  // shared tables (the first layer's records of its tile, the current
  // masses, the first layers' record weights), then
  // builds the tables and finishes, the next layer's records loading while
  // one layer is summed. Loads are unconditional (indices clamped into
  // range, unused values masked later): conditional loads make the compiler
  // wait for each one.
  constexpr int NSUB = RING ? 2 : 1;
  constexpr int HC = RING ? 16 : 32;   // heads per record chunk
  const int G = a.Hq / a.Hkv;
  const int n_ml = a.Hq * P;                 // record weights per layer
  const int lc0 = min(L, a.layers_per_chunk);
  // layer-table block of layer slot s in LDS
  const int per_layer = (int)combine_layer_floats(a.Hq, a.Hkv, P);
  auto t_wp = [&](int s_) { return lds + (size_t)s_ * per_layer; };          // [P][Hq]
  // the first chunk's weights: two per thread prefetched
  const int n_stage = lc0 * n_ml;
  auto stage_src = [&](int l0, int x) -> float {
    // value x of the staged weights of layers [l0, l0 + lc)
    const int l = l0 + x / n_ml, r = x % n_ml;
    return ws_f(l, a.off_w)[(size_t)b * n_ml + r];
  };
  auto stage_dst = [&](int x) -> float* { return t_wp(x / n_ml) + x % n_ml; };
  const float pre0 = stage_src(0, min(tid, n_stage - 1));
  const float pre1 = stage_src(0, min(tid + 256, n_stage - 1));

  // tile t of this thread (tiles with records: every tile of a ring; a
  // linear cache's readable range). Without a window the range starts at
  // tile 0, so the record loads need not wait for cur_pos; the range end
  // and the blocks come after them.
  int tlo = 0;
  if constexpr (!RING) {
    if (a.window > 0) {
      const int ic = a.cur_pos[b];
      const int thi0 = max(0, min(a.NT, ic / kTile + 1));
      tlo = min(thi0, max(ic - a.window + 1, 0) / kTile);
    }
  }
  const int t = tlo + (int)blockIdx.x * 256 + tid;
  // records of heads past Hq (clamped duplicates) get weight 0; a dead
  // thread's values are never used
  const int tc = min(max(t, 0), a.NT - 1);
  // this sequence's records of layer l; the tile's byte offset
  const uint32_t rec_bytes = (uint32_t)a.Hkv * a.NT * NSUB * G * 4;
  const uint32_t rec_vo = (uint32_t)tc * NSUB * G * 4;
  constexpr int PV = V4 ? HC / 4 : HC;
  const uint32_t map_bytes = (uint32_t)a.Hkv * a.NT * 4;
  auto load_records = [&](int l, int hc, float (&ev)[NSUB][HC], int (&pv)[PV]) {
    const char* base = a.lws[l] + a.off_e + (size_t)b * rec_bytes;
    load_rec<NSUB, HC, V4>(ev, make_rsrc(base, rec_bytes), rec_vo, hc, a.Hq, G, a.NT);
    load_pid<HC, V4, RING>(pv, make_rsrc(a.lws[l] + a.off_pid + (size_t)b * map_bytes, map_bytes), tc, hc, a.Hq, G,
                           a.NT, P, a.tpp);
  };
  float ev[NSUB][HC], ev_next[NSUB][HC];
  int pv[PV], pv_next[PV];
  load_records(0, 0, ev, pv);
  float mass_run[NSUB], max_run[NSUB];
  if constexpr (!RING) {
    // a linear cache's block is the tile: its index needs no cur_pos
    const size_t mi = (size_t)b * a.nbmax + min(tc, a.nbmax - 1);
    mass_run[0] = a.mass != nullptr ? a.mass[mi] : 0.0f;
    max_run[0] = a.mass_max != nullptr ? a.mass_max[mi] : 0.0f;
  }
  const int i_cur = a.cur_pos[b];
  int thi = a.NT;
  if constexpr (!RING) thi = max(0, min(a.NT, i_cur / kTile + 1));
  const bool m_live = t < thi;
  const int lap_i = RING ? i_cur / a.C : 0;
  int blk[NSUB];
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    blk[sb] = t;
    if constexpr (RING) {
      const int lap = ((lap_i & 1) == sb) ? lap_i : lap_i - 1;
      blk[sb] = lap < 0 ? -1 : lap * (a.C / kTile) + t;
    }
    if (!m_live || blk[sb] >= a.nbmax) blk[sb] = -1;
  }
  if constexpr (RING) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const size_t mi = (size_t)b * a.nbmax + max(blk[sb], 0);
      mass_run[sb] = a.mass != nullptr ? a.mass[mi] : 0.0f;
      max_run[sb] = a.mass_max != nullptr ? a.mass_max[mi] : 0.0f;
    }
  }

  // Per-head masses: the sequence's [Hq][nbmax] rows as one buffer, the
  // block as the lane's offset and the head as a scalar one. With every head
  // in one chunk a thread keeps its heads' masses in registers over the
  // layers: read once, each layer's values added in order, written once (the
  // same additions as a read-modify-write per layer).
  const bool hm_reg = a.head_mass != nullptr && a.Hq <= HC;
  const __amdgpu_buffer_rsrc_t hr =
      make_rsrc(a.head_mass != nullptr ? a.head_mass + (size_t)b * a.Hq * a.nbmax : nullptr,
                a.head_mass != nullptr ? (uint32_t)a.Hq * a.nbmax * 4 : 0u);
  float hacc[NSUB][HC];
  if (hm_reg && m_live) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const uint32_t hvo = (uint32_t)max(blk[sb], 0) * 4;
#pragma unroll
      for (int k = 0; k < HC; ++k)
        hacc[sb][k] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(hr, (int)hvo, (int)((uint32_t)min(k, a.Hq - 1) * a.nbmax * 4), 0));
    }
  }

  for (int l0 = 0; l0 < L; l0 += lc0) {
    const int lc = min(lc0, L - l0);
    // ---- tables of layers [l0, l0 + lc) ----
    if (l0 > 0) __syncthreads();  // the previous chunk's tables are done with
    const int n_st = lc * n_ml;
    // four values per thread in flight per round (one round trip each)
    auto stage_rest = [&](int la, int x_first) {
      for (int x0 = x_first; x0 < n_st; x0 += 4 * 256) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = stage_src(la, min(x0 + tid + 256 * k, n_st - 1));
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (x0 + tid + 256 * k < n_st) *stage_dst(x0 + tid + 256 * k) = v[k];
      }
    };
    if (l0 == 0) {
      if (tid < n_st) *stage_dst(tid) = pre0;
      if (tid + 256 < n_st) *stage_dst(tid + 256) = pre1;
      stage_rest(0, 512);
    } else {
      stage_rest(l0, 0);
    }
    __syncthreads();
    if (!m_live) continue;

    for (int s_ = 0; s_ < lc; ++s_) {
      const int l = l0 + s_;
      const float* wp = t_wp(s_);
      float acc[NSUB], mx[NSUB];
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        acc[sb] = 0.0f;
        mx[sb] = 0.0f;
      }
      // heads in ascending order, HC at a time (head h sits at row (b, h / G)
      // of the records, entry h % G); per-head masses read-modify-written
      // alongside when asked for. Every tile of the range has records from
      // this layer's call, relative to its partition's max.
      for (int hc = 0; hc < a.Hq; hc += HC) {
        if (hc > 0) load_records(l, hc, ev, pv);
        // the next layer's first records load while this chunk is summed
        const bool prefetch = hc + HC >= a.Hq && l + 1 < L;
        if (prefetch) load_records(l + 1, 0, ev_next, pv_next);
        // the chunk's products E w, in place of its records: a group's four
        // weights read from LDS (unconditional, clamped) as they are used,
        // heads in ascending order per sub-block; heads past Hq add +0 (sums
        // and maxima are >= 0: no change)
        if constexpr (V4) {
#pragma unroll
          for (int q = 0; q < HC / 4; ++q) {
            const int hh = min(hc + 4 * q, a.Hq - 4);
            const f32x4 w4 = *(const f32x4*)(wp + min(max(pv[q], 0), P - 1) * a.Hq + hh);
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const float v = hc + 4 * q + k < a.Hq ? ev[sb][4 * q + k] * w4[k] : 0.0f;
                ev[sb][4 * q + k] = v;
                acc[sb] += v;
                mx[sb] = fmaxf(mx[sb], v);
              }
          }
        } else {
#pragma unroll
          for (int k = 0; k < HC; ++k) {
            const int hh = min(hc + k, a.Hq - 1);
            const float w = wp[min(max(pv[k], 0), P - 1) * a.Hq + hh];
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb) {
              const float v = hc + k < a.Hq ? ev[sb][k] * w : 0.0f;
              ev[sb][k] = v;
              acc[sb] += v;
              mx[sb] = fmaxf(mx[sb], v);
            }
          }
        }
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
          if (hm_reg) {
            // heads past Hq add +0
#pragma unroll
            for (int k = 0; k < HC; ++k) hacc[sb][k] = hacc[sb][k] + ev[sb][k];
          } else if (a.head_mass != nullptr && blk[sb] >= 0) {
            // per-head masses, eight read-modify-writes in flight at a time
            const uint32_t hvo = (uint32_t)blk[sb] * 4;
#pragma unroll
            for (int k0 = 0; k0 < HC; k0 += 8) {
              if (hc + k0 >= a.Hq) break;
              float hv[8];
#pragma unroll
              for (int k = 0; k < 8; ++k) {
                const uint32_t so = (uint32_t)min(hc + k0 + k, a.Hq - 1) * a.nbmax * 4;
                hv[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(hr, (int)hvo, (int)so, 0));
              }
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if (hc + k0 + k < a.Hq)
                  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hv[k] + ev[sb][k0 + k]), hr, (int)hvo,
                                                        (int)((uint32_t)(hc + k0 + k) * a.nbmax * 4), 0);
            }
          }
        }
        if (prefetch) {
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
            for (int k = 0; k < HC; ++k) ev[sb][k] = ev_next[sb][k];
#pragma unroll
          for (int i = 0; i < PV; ++i) pv[i] = pv_next[i];
        }
      }
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        mass_run[sb] = mass_run[sb] + acc[sb];
        max_run[sb] = fmaxf(max_run[sb], mx[sb]);
      }
    }
  }
  if (!m_live) return;
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    if (blk[sb] < 0) continue;
    const size_t mi = (size_t)b * a.nbmax + blk[sb];
    if (a.mass != nullptr) a.mass[mi] = mass_run[sb];
    if (a.mass_max != nullptr) a.mass_max[mi] = max_run[sb];
    if (hm_reg) {
#pragma unroll
      for (int k = 0; k < HC; ++k)
        if (k < a.Hq)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hacc[sb][k]), hr, (int)((uint32_t)blk[sb] * 4),
                                                (int)((uint32_t)k * a.nbmax * 4), 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Layer-parallel combine (kvs_tap_masses without per-head masses): grid
// (ceil(NT / (64 TG)), B) plus n_layers rate columns, 512 threads. Wave w of
// a workgroup takes tile group w % TG (64 consecutive tiles, one per lane)
// and layers w / TG, w / TG + 8 / TG, ... (TG = 1 from 8 layers up), keeping
// each (tile, layer)'s sum over heads, computed exactly as kvs_combine does,
// in LDS; then one lane per tile adds them in layer order to the current
// mass, so the result equals the layer-by-layer sum bit for bit. A wave stages only its own layers' weights, loaded
// together with its records, so the one barrier is before the final sums.
// ---------------------------------------------------------------------------
constexpr int kCmbTiles = 64;
constexpr int kCmbWaves = 8;

// Tile groups of a layer-parallel workgroup: with fewer than 8 layers the
// waves split the tiles too (TG groups of 64 tiles, TG L <= 8, TG a power
// of two), so no wave idles.
__host__ __device__ inline int cmb_groups(int L) {
  int g = 1;
  while (g * 2 * L <= kCmbWaves) g *= 2;
  return g;
}

// Two workgroups per compute unit (<= 128 VGPRs): the mass workgroups of the
// 397B-like step (16 sequences x 32 chunks) are then all resident at once.
template <bool RING, bool V4>
__global__ __launch_bounds__(64 * kCmbWaves) __attribute__((amdgpu_waves_per_eu(4)))
void kvs_combine_layers(CombineArgs a) {
  constexpr int NTH = 64 * kCmbWaves;
  extern __shared__ float lds[];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-layer pointers load as scalars
  const int P = a.nparts, L = a.n_layers;
  constexpr int NSUB = RING ? 2 : 1;
  constexpr int HC = RING ? 16 : 32;
  auto ws_f = [&](int l, size_t off) { return (const float*)(a.lws[l] + off); };
  const int TG = cmb_groups(L);
  const int tpw = kCmbTiles * TG;  // tiles per workgroup
  const int n_chunks = (a.NT + tpw - 1) / tpw;
  // The blocks [c_lo, c_hi) of sequence b that the mass workgroups reach:
  // a linear cache's readable tiles, a ring's two laps (i / C and
  // i / C - 1) of every tile.
  auto reached = [&](int& c_lo, int& c_hi) {
    const int ic = a.cur_pos[b];
    if constexpr (RING) {
      const int lap_i = ic / a.C;
      c_lo = max(lap_i - 1, 0) * a.NT;
      c_hi = (lap_i + 1) * a.NT;
    } else {
      c_hi = max(0, min(a.NT, ic / kTile + 1));
      c_lo = a.window > 0 ? min(c_hi, max(ic - a.window + 1, 0) / kTile) : 0;
    }
    c_hi = min(c_hi, a.nbmax);
    c_lo = min(c_lo, c_hi);
  };
  if ((int)blockIdx.x >= n_chunks + L) {
    // ---- side-car columns: the turn's update of the blocks the mass
    // workgroups do not reach (their masses are this turn's as they stand)
    if (a.sc_att == nullptr) return;
    int c_lo, c_hi;
    reached(c_lo, c_hi);
    const int col = blockIdx.x - n_chunks - L;
    for (int blk = col * NTH + tid; blk < a.nbmax; blk += kCmbSidecarCols * NTH) {
      if (blk >= c_lo && blk < c_hi) continue;
      const size_t x = (size_t)b * a.nbmax + blk;
      sidecar_block(a.mass, a.sc_att, a.sc_ema, a.sc_cum, a.sc_traj, x, b, blk, a.nbmax, a.sc_traj_cap,
                    a.sc_slot, a.sc_alpha, a.mass[x]);
    }
    return;
  }
  if ((int)blockIdx.x >= n_chunks) {
    // rates: the same per-layer refresh as in kvs_combine
    const int l = blockIdx.x - n_chunks;
    if (b != 0 || l >= L) return;
    const float* ws_time = ws_f(l, a.off_time);
    float* rates = (float*)(a.lws[l] + a.off_rates);
    float* ct = lds;
    float* cs = lds + 8;
    if (tid < 16) lds[tid] = 0.0f;
    __syncthreads();
    for (int w = tid; w < a.n_wg; w += NTH) {
      float tiles = 0.0f, ticks = 0.0f;
      for (int k = 0; k < kPartialWaves; ++k) {
        const float* tm = ws_time + ((size_t)w * kPartialWaves + k) * 2;
        tiles += tm[0];
        ticks = fmaxf(ticks, tm[1]);
      }
      if (tiles > 0.0f && ticks > 0.0f && tiles < 1e9f && ticks < 1e9f) {
        atomicAdd(&ct[w & 7], tiles);
        atomicAdd(&cs[w & 7], ticks);
      }
    }
    __syncthreads();
    if (tid < 8) {
      float mean = 0.0f;
      int nv = 0;
      for (int c = 0; c < 8; ++c) {
        const float r = cs[c] > 0.0f ? ct[c] / cs[c] : 0.0f;
        if (r > 0.0f) {
          mean += r;
          ++nv;
        }
      }
      const float r = cs[tid] > 0.0f ? ct[tid] / cs[tid] : 0.0f;
      const float old = rates[tid];
      if (nv > 0 && r > 0.0f) {
        const float rel = fminf(fmaxf(r / (mean / (float)nv), 0.5f), 2.0f);
        const bool ok = old >= 0.5f && old <= 2.0f;
        rates[tid] = ok ? 0.5f * old + 0.5f * rel : rel;
      }
    }
    return;
  }

  const int G = a.Hq / a.Hkv;
  const int per = a.Hq * P;  // one layer's table: the record weights [P][Hq]
  auto t_wp = [&](int l) { return lds + (size_t)l * per; };
  float* cl = lds + (size_t)L * per;  // [tpw][L][NSUB][2]: sum and max over heads
  // this wave: tile group tg, layers l0, l0 + ls, ...
  const int tg = wv % TG, l0 = wv / TG, ls = kCmbWaves / TG;
  const int tl = tg * 64 + lane;  // tile of this lane within the workgroup

  // tile of this lane; without a window the range starts at tile 0, so the
  // loads below need not wait for cur_pos
  int tlo = 0;
  if constexpr (!RING) {
    if (a.window > 0) {
      const int ic = a.cur_pos[b];
      const int thi0 = max(0, min(a.NT, ic / kTile + 1));
      tlo = min(thi0, max(ic - a.window + 1, 0) / kTile);
    }
  }
  const int t = tlo + (int)blockIdx.x * tpw + tl;
  const int tc = min(max(t, 0), a.NT - 1);
  const uint32_t rec_bytes = (uint32_t)a.Hkv * a.NT * NSUB * G * 4;
  const uint32_t rec_vo = (uint32_t)tc * NSUB * G * 4;
  constexpr int PV = V4 ? HC / 4 : HC;
  const uint32_t map_bytes = (uint32_t)a.Hkv * a.NT * 4;
  auto load_records = [&](int l, int hc, float (&ev)[NSUB][HC], int (&pv)[PV]) {
    const char* lw = a.lws[min(l, L - 1)];
    load_rec<NSUB, HC, V4>(ev, make_rsrc(lw + a.off_e + (size_t)b * rec_bytes, rec_bytes), rec_vo, hc, a.Hq, G, a.NT);
    load_pid<HC, V4, RING>(pv, make_rsrc(lw + a.off_pid + (size_t)b * map_bytes, map_bytes), tc, hc, a.Hq, G, a.NT,
                           P, a.tpp);
  };
  // Tables of up to 128 values per layer (the usual case): each wave stages
  // those of its own layers and reads only those (waves of a layer's tile
  // groups write the same values), so no workgroup barrier comes before the
  // sums. The first two layers' tables
  // (two values per lane each) are issued ahead of the records, so storing
  // them waits for nothing else. Larger tables (many partitions) are staged
  // by the whole workgroup, four values per thread in flight, then a barrier.
  auto tab_val = [&](int l, int r) -> float {
    return ((const float*)(a.lws[min(l, L - 1)] + a.off_w))[(size_t)b * per + min(r, per - 1)];
  };
  const bool coop = per > 128;
  float tv[2][2];
  if (!coop) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) tv[j][k] = tab_val(l0 + j * ls, lane + 64 * k);
  }
  asm volatile("" ::: "memory");
  float ev[NSUB][HC], ev_next[NSUB][HC];
  int pv[PV], pv_next[PV];
  load_records(l0, 0, ev, pv);
  load_records(l0 + ls, 0, ev_next, pv_next);
  // a linear cache's block is the tile: the first wave of each tile group
  // fetches the current masses it adds to now (a ring's blocks depend on
  // cur_pos, read at the end)
  float mass0 = 0.0f, max0 = 0.0f;
  if constexpr (!RING) {
    if (l0 == 0) {
      const size_t mi = (size_t)b * a.nbmax + min(tc, a.nbmax - 1);
      mass0 = a.mass != nullptr ? a.mass[mi] : 0.0f;
      max0 = a.mass_max != nullptr ? a.mass_max[mi] : 0.0f;
    }
  }
  asm volatile("" ::: "memory");
  if (!coop) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int l = l0 + j * ls;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (l < L && lane + 64 * k < per) t_wp(l)[lane + 64 * k] = tv[j][k];
    }
    // layers past a wave's second
    for (int l = l0 + 2 * ls; l < L; l += ls)
      for (int r = lane; r < per; r += 64) t_wp(l)[r] = tab_val(l, r);
  } else {
    // every layer's tables in one flat index (layer-major, as in LDS), four
    // values per thread in flight: one memory round trip for up to 2048
    // values, not one per layer
    const int n_tab = L * per;
    for (int x0 = 0; x0 < n_tab; x0 += 4 * NTH) {
      float v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int x = min(x0 + tid + k * NTH, n_tab - 1);
        v[k] = tab_val(x / per, x % per);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (x0 + tid + k * NTH < n_tab) lds[x0 + tid + k * NTH] = v[k];
    }
    __syncthreads();
  }

  // ---- this wave's layers: per (tile, layer) sums over heads ----
  // Layer l's sum and max over heads for this lane's tile into cl, its first
  // head chunk given in ev (further chunks, when Hq > HC, loaded into ev here).
  // Heads in ascending order per sub-block; each group's four weights are read
  // from LDS as they are used.
  auto sum_layer = [&](int l, float (&ev)[NSUB][HC], int (&pv)[PV]) {
    const float* wp = t_wp(l);
    float acc[NSUB], mx[NSUB];
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      acc[sb] = 0.0f;
      mx[sb] = 0.0f;
    }
    for (int hc = 0; hc < a.Hq; hc += HC) {
      if (hc > 0) load_records(l, hc, ev, pv);
      // heads past Hq add +0 (sums and maxima are >= 0: no change)
      if constexpr (V4) {
#pragma unroll
        for (int q = 0; q < HC / 4; ++q) {
          const int hh = min(hc + 4 * q, a.Hq - 4);
          const f32x4 w4 = *(const f32x4*)(wp + min(max(pv[q], 0), P - 1) * a.Hq + hh);
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float v = hc + 4 * q + k < a.Hq ? ev[sb][4 * q + k] * w4[k] : 0.0f;
              acc[sb] += v;
              mx[sb] = fmaxf(mx[sb], v);
            }
        }
      } else {
#pragma unroll
        for (int k = 0; k < HC; ++k) {
          const int hh = min(hc + k, a.Hq - 1);
          const float w = wp[min(max(pv[k], 0), P - 1) * a.Hq + hh];
#pragma unroll
          for (int sb = 0; sb < NSUB; ++sb) {
            const float v = hc + k < a.Hq ? ev[sb][k] * w : 0.0f;
            acc[sb] += v;
            mx[sb] = fmaxf(mx[sb], v);
          }
        }
      }
    }
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      cl[((tl * L + l) * NSUB + sb) * 2] = acc[sb];
      cl[((tl * L + l) * NSUB + sb) * 2 + 1] = mx[sb];
    }
  };
  // the first two layers' first chunks are in flight since the start
  if (l0 < L) sum_layer(l0, ev, pv);
  if (l0 + ls < L) sum_layer(l0 + ls, ev_next, pv_next);
  for (int l = l0 + 2 * ls; l < L; l += ls) {
    load_records(l, 0, ev, pv);
    sum_layer(l, ev, pv);
  }
  __syncthreads();

  // ---- one lane per tile: the layers in call order ----
  if (l0 != 0) return;  // the first wave of each tile group
  const int i_cur = a.cur_pos[b];
  int thi = a.NT;
  if constexpr (!RING) thi = max(0, min(a.NT, i_cur / kTile + 1));
  if (t >= thi) return;
  const int lap_i = RING ? i_cur / a.C : 0;
#pragma unroll
  for (int sb = 0; sb < NSUB; ++sb) {
    int blk = t;
    if constexpr (RING) {
      const int lap = ((lap_i & 1) == sb) ? lap_i : lap_i - 1;
      blk = lap < 0 ? -1 : lap * (a.C / kTile) + t;
    }
    if (blk < 0 || blk >= a.nbmax) continue;
    const size_t mi = (size_t)b * a.nbmax + blk;
    float mass_run = mass0, max_run = max0;
    if constexpr (RING) {
      mass_run = a.mass != nullptr ? a.mass[mi] : 0.0f;
      max_run = a.mass_max != nullptr ? a.mass_max[mi] : 0.0f;
    }
    for (int l = 0; l < L; ++l) {
      mass_run = mass_run + cl[((tl * L + l) * NSUB + sb) * 2];
      max_run = fmaxf(max_run, cl[((tl * L + l) * NSUB + sb) * 2 + 1]);
    }
    if (a.sc_att != nullptr)  // the turn's side-car update with this mass
      sidecar_block(a.mass, a.sc_att, a.sc_ema, a.sc_cum, a.sc_traj, mi, b, blk, a.nbmax, a.sc_traj_cap,
                    a.sc_slot, a.sc_alpha, mass_run);
    else if (a.mass != nullptr)
      a.mass[mi] = mass_run;
    if (a.mass_max != nullptr) a.mass_max[mi] = max_run;
  }
}

size_t combine_layers_lds_bytes(int Hq, int Hkv, int P, int L, bool ring) {
  return ((size_t)L * combine_layer_floats(Hq, Hkv, P) + (size_t)kCmbTiles * cmb_groups(L) * L * (ring ? 2 : 1) * 2) *
         sizeof(float);
}

hipError_t launch_combine_layers(const CombineArgs& a, bool ring, hipStream_t st) {
  if (!(a.mass || a.mass_max)) return hipSuccess;
  const int tpw = kCmbTiles * cmb_groups(a.n_layers);
  const int n_chunks = (a.NT + tpw - 1) / tpw;
  dim3 grid(n_chunks + a.n_layers + (a.sc_att ? kCmbSidecarCols : 0), a.B), block(64 * kCmbWaves);
  size_t lds = combine_layers_lds_bytes(a.Hq, a.Hkv, a.nparts, a.n_layers, ring);
  if (lds < 16 * sizeof(float)) lds = 16 * sizeof(float);
  // four heads of a group per 16-byte record load when the group size allows
  const bool v4 = (a.Hq / a.Hkv) % 4 == 0;
  if (ring) {
    if (v4) hipLaunchKernelGGL((kvs_combine_layers<true, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine_layers<true, false>), grid, block, lds, st, a);
  } else {
    if (v4) hipLaunchKernelGGL((kvs_combine_layers<false, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine_layers<false, false>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
template <int KV, int D>
static hipError_t launch_partial_t(const PartialArgs& a, bool scored, bool ring, size_t lds_bytes,
                                   hipStream_t st) {
  dim3 grid(a.nparts, a.Hkv, a.B), block(64 * kPartialWaves);
  if (scored) {
    if (ring) hipLaunchKernelGGL((kvs_partial<KV, D, true, true>), grid, block, lds_bytes, st, a);
    else hipLaunchKernelGGL((kvs_partial<KV, D, true, false>), grid, block, lds_bytes, st, a);
  } else {
    if (ring) hipLaunchKernelGGL((kvs_partial<KV, D, false, true>), grid, block, lds_bytes, st, a);
    else hipLaunchKernelGGL((kvs_partial<KV, D, false, false>), grid, block, lds_bytes, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_partial(int kv, int d, const PartialArgs& a, bool scored, bool ring,
                          size_t lds_bytes, hipStream_t st) {
  if (kv == KV_F32) {
    if (d == 16) return launch_partial_t<KV_F32, 16>(a, scored, ring, lds_bytes, st);
    if (d == 64) return launch_partial_t<KV_F32, 64>(a, scored, ring, lds_bytes, st);
    if (d == 128) return launch_partial_t<KV_F32, 128>(a, scored, ring, lds_bytes, st);
  } else if (kv == KV_BF16) {
    if (d == 64) return launch_partial_t<KV_BF16, 64>(a, scored, ring, lds_bytes, st);
    if (d == 128) return launch_partial_t<KV_BF16, 128>(a, scored, ring, lds_bytes, st);
  } else if (kv == KV_FP8) {
    if (d == 64) return launch_partial_t<KV_FP8, 64>(a, scored, ring, lds_bytes, st);
    if (d == 128) return launch_partial_t<KV_FP8, 128>(a, scored, ring, lds_bytes, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, bool ring, hipStream_t st) {
  // outputs are merged by the partial kernel: without mass work there is
  // nothing to do (the partition rates then keep their last values)
  if (!(a.mass || a.head_mass || a.mass_max)) return hipSuccess;
  dim3 grid(a.n_mass_chunks + a.n_layers, a.B), block(256);
  size_t lds = (size_t)a.layers_per_chunk * combine_layer_floats(a.Hq, a.Hkv, a.nparts) * sizeof(float);
  if (lds < 16 * sizeof(float)) lds = 16 * sizeof(float);
  const bool v4 = (a.Hq / a.Hkv) % 4 == 0;
  if (ring) {
    if (v4) hipLaunchKernelGGL((kvs_combine<true, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine<true, false>), grid, block, lds, st, a);
  } else {
    if (v4) hipLaunchKernelGGL((kvs_combine<false, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine<false, false>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace kvs
