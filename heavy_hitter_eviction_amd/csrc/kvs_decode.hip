// Scored split-K decode attention for gfx950.
//
// kvs_partial: one workgroup (4 waves) per (partition of slots, KV head,
// sequence). Each wave walks 16-slot tiles of its partition (tiles w, w+4, ...)
// with an online softmax, for all G query heads of the KV head at once:
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
// also sums its post-softmax weights per head relative to its running max; at
// the end of the partition those block sums are rescaled to the partition max
// and stored with the partition's (max, sum, unnormalised O). kvs_combine then
// turns them into exact normalised masses.
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
  f32x4 ks, vs;    // FP8 scales of the lane's 4 tokens
  int32_t pos[4];  // ring: absolute positions of the lane's 4 tokens
};

template <int KV, int D, bool RING>
__device__ __forceinline__ void load_tile(TileRegs<KV, D>& t, const PartialArgs& a, int b, int g,
                                          int tile, int lane) {
  constexpr int eb = KvT<KV>::eb;
  constexpr int NCH = TileRegs<KV, D>::NCH;
  const int j = lane & 15, kg = lane >> 4;
  const size_t bg = (size_t)b * a.Hkv + g;
  // K: this lane's token is row j of the tile; chunk i covers row bytes [64 i + 16 kg, +16).
  const char* krow = (const char*)a.k + ((bg * a.C + (size_t)tile * kTile + j) * D) * eb;
#pragma unroll
  for (int i = 0; i < NCH; ++i)
    t.k[i] = __builtin_nontemporal_load((const u32x4*)(krow + 64 * i + 16 * kg));
  // V: tile layout [4][D][4]; this lane reads [kg][(D/16) j .. +D/16][0..3], contiguous.
  const char* vt = (const char*)a.v + ((bg * (a.C / kTile) + tile) * (size_t)(kTile * D)) * eb;
  const char* vl = vt + ((size_t)kg * D + (D / 16) * j) * 4 * eb;
#pragma unroll
  for (int i = 0; i < NCH; ++i) t.v[i] = __builtin_nontemporal_load((const u32x4*)(vl + 16 * i));
  const size_t slot0 = (size_t)b * a.C + (size_t)tile * kTile + 4 * kg;
  if constexpr (KV == KV_FP8) {
    t.ks = *(const f32x4*)(a.ks + slot0);
    t.vs = *(const f32x4*)(a.vs + slot0);
  }
  if constexpr (RING) {
    const int4 p = *(const int4*)(a.pos_of_slot + slot0);
    t.pos[0] = p.x; t.pos[1] = p.y; t.pos[2] = p.z; t.pos[3] = p.w;
  }
}

// Lane's t-th contraction element of the QK product lives at head dimension
// dim(t, kg): the K load above gives element t of chunk t/EPC at row offset
// 64 (t/EPC) + 16 kg bytes.
template <int KV>
__device__ __forceinline__ int qk_dim(int t, int kg) {
  constexpr int EPC = 16 / KvT<KV>::eb;
  return (t / EPC) * 4 * EPC + kg * EPC + t % EPC;
}

template <int KV, int D, bool SCORED, bool RING>
__global__ __launch_bounds__(256, 2) void kvs_partial(PartialArgs a) {
  constexpr int NCH = TileRegs<KV, D>::NCH;
  constexpr int NSUB = RING ? 2 : 1;
  constexpr int NC = D / 16;  // PV output chunks of 16 dims
  extern __shared__ float lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kg = lane >> 4;
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const int h = j;                       // query head within the group (this lane's column)
  const bool hreal = h < G;
  const int i_cur = a.cur_pos[b];
  const int lo = a.window > 0 ? i_cur - a.window + 1 : (int)0x80000000;

  const int t0 = part * a.tpp;
  const int t1 = min(t0 + a.tpp, a.NT);
  const int ntl = t1 - t0;

  // LDS carve-up: per-tile block sums and running maxima, then the wave merge area.
  float* e_rec = lds;                                   // [ntl][NSUB][G]
  float* m_rec = e_rec + a.tpp * NSUB * G;              // [ntl][G]
  float* mw = m_rec + a.tpp * G;                        // [4][G]
  float* lw = mw + 4 * G;                               // [4][G]
  float* ow = lw + 4 * G;                               // [4][G][D]
  if constexpr (SCORED) {
    for (int x = threadIdx.x; x < ntl * NSUB * G; x += 256) e_rec[x] = 0.0f;
    for (int x = threadIdx.x; x < ntl * G; x += 256) m_rec[x] = -__builtin_inff();
  }
  __syncthreads();

  // Tiles that can hold a readable key.
  int tb = t0, te = t1;
  if constexpr (!RING) {
    te = min(te, i_cur / kTile + 1);
    if (a.window > 0) tb = max(tb, max(lo, 0) / kTile);
  }

  // Query operand (B of the QK MFMA): lane holds Q[h][dim(t, kg)], zeros for padding heads.
  const int hq = g * G + h;
  constexpr int QN = D / 4;
  float qf[QN];
#pragma unroll
  for (int t = 0; t < QN; ++t) {
    float x = 0.0f;
    if (hreal) {
      const size_t qi = ((size_t)b * a.Hq + hq) * D + qk_dim<KV>(t, kg);
      if constexpr (KV == KV_F32)
        x = ((const float*)a.q)[qi];
      else
        x = bits_to_f32((uint32_t)((const uint16_t*)a.q)[qi] << 16);
    }
    qf[t] = x;
  }
  bf16x8 qb[D / 32 > 0 ? D / 32 : 1];
  if constexpr (KV != KV_F32) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[c][e] = (__bf16)qf[8 * c + e];  // exact: Q is bf16
  }

  f32x4 oacc[NC];
#pragma unroll
  for (int n = 0; n < NC; ++n) oacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // Ring laps: positions read at step i lie in [i - C + 1, i], so at most two
  // laps (i / C and i / C - 1) share a tile; their parity names the sub-block.
  const int lap_i = RING ? i_cur / a.C : 0;
  const int lap_base = lap_i * a.C;

  auto tile_kept = [&](int tile) -> bool {
    if constexpr (RING) {
      return true;
    } else {
      if (a.keep == nullptr) return true;
      if (tile >= a.nbmax) return true;
      return (a.keep[(size_t)b * a.kwords + (tile >> 5)] >> (tile & 31)) & 1u;
    }
  };

  TileRegs<KV, D> cur, nxt;
  int tile = tb + wave;
  while (tile < te && !tile_kept(tile)) tile += 4;
  if (tile < te) load_tile<KV, D, RING>(cur, a, b, g, tile, lane);

  while (tile < te) {
    int ntile = tile + 4;
    while (ntile < te && !tile_kept(ntile)) ntile += 4;
    if (ntile < te) load_tile<KV, D, RING>(nxt, a, b, g, ntile, lane);

    // ---- validity of the lane's 4 tokens (rows 4 kg + r of the tile) ----
    bool valid[4];
    int sub[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (RING) {
        const int p = cur.pos[r];
        bool v = p >= 0 && p <= i_cur && p >= lo;
        if (v && a.keep != nullptr) {
          const int blk = p >> 4;
          v = blk >= a.nbmax || ((a.keep[(size_t)b * a.kwords + (blk >> 5)] >> (blk & 31)) & 1u);
        }
        valid[r] = v;
        sub[r] = ((p >= lap_base) ? lap_i : lap_i - 1) & 1;
      } else {
        const int p = tile * kTile + 4 * kg + r;
        valid[r] = p <= i_cur && p >= lo;
        sub[r] = 0;
      }
    }
    const bool lane_all = valid[0] && valid[1] && valid[2] && valid[3];
    const bool lane_any = valid[0] || valid[1] || valid[2] || valid[3];
    if (wave_any(lane_any)) {
      const bool all_valid = wave_all(lane_all);

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
        float x = s[r] * a.scale_log2;
        if constexpr (KV == KV_FP8) x = s[r] * (cur.ks[r] * a.scale_log2);
        tl[r] = valid[r] ? x : -__builtin_inff();
      }
      float mx = fmaxf(fmaxf(tl[0], tl[1]), fmaxf(tl[2], tl[3]));
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(tl[r] - m_new);

      float esub0 = 0.f, esub1 = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (NSUB == 2 && sub[r]) esub1 += p[r];
        else esub0 += p[r];
      }
      esub0 = rows_sum(esub0);
      if constexpr (NSUB == 2) esub1 = rows_sum(esub1);
      l_run = l_run * alpha + (esub0 + esub1);

      if constexpr (SCORED) {
        if (kg == 0 && hreal) {
          const int tlc = tile - t0;
          e_rec[(tlc * NSUB) * G + h] = esub0;
          if constexpr (NSUB == 2) e_rec[(tlc * NSUB + 1) * G + h] = esub1;
          m_rec[tlc * G + h] = m_new;
        }
      }

      if (wave_any(alpha != 1.0f)) {
#pragma unroll
        for (int n = 0; n < NC; ++n) oacc[n] *= alpha;
      }
      m_run = m_new;

      // ---- O^T += V^T P^T ----
      if constexpr (KV == KV_F32) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = p[r];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int u = 4 * n + r;  // lane's V element: dim (D/16) j + n, token 4 kg + r
            float vv = bits_to_f32(cur.v[u / 4][u % 4]);
            if (!all_valid) vv = valid[r] ? vv : 0.0f;
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, pv[r], oacc[n], 0, 0, 0);
          }
        }
      } else {
        float pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[r] = p[r];
          if constexpr (KV == KV_FP8) pw[r] = p[r] * cur.vs[r];
        }
        const u32x2 pb = {pack_bf16x2(pw[0], pw[1]), pack_bf16x2(pw[2], pw[3])};
        u32x2 vmask = {0xFFFFFFFFu, 0xFFFFFFFFu};
        if (!all_valid) {
          vmask[0] = (valid[0] ? 0x0000FFFFu : 0u) | (valid[1] ? 0xFFFF0000u : 0u);
          vmask[1] = (valid[2] ? 0x0000FFFFu : 0u) | (valid[3] ? 0xFFFF0000u : 0u);
        }
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
          vv[0] &= vmask[0];
          vv[1] &= vmask[1];
          oacc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv),
                                                              __builtin_bit_cast(s16x4, pb), oacc[n], 0, 0, 0);
        }
      }
    }
    cur = nxt;
    tile = ntile;
  }

  // ---- merge the four waves of the partition ----
  if (hreal) {
    if (kg == 0) {
      mw[wave * G + h] = m_run;
      lw[wave * G + h] = l_run;
    }
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) ow[(wave * G + h) * D + (D / 16) * (4 * kg + r) + n] = oacc[n][r];
  }
  __syncthreads();

  const size_t pbase = ((size_t)b * a.Hq + (size_t)g * G);  // first head of the group
  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int hh = x / D, dd = x % D;
    float M = fmaxf(fmaxf(mw[hh], mw[G + hh]), fmaxf(mw[2 * G + hh], mw[3 * G + hh]));
    float o = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o += ow[(w * G + hh) * D + dd] * fast_exp2(mw[w * G + hh] - M);
    }
    a.ws_o[((pbase + hh) * a.nparts + part) * D + dd] = o;
  }
  for (int hh = threadIdx.x; hh < G; hh += 256) {
    float M = fmaxf(fmaxf(mw[hh], mw[G + hh]), fmaxf(mw[2 * G + hh], mw[3 * G + hh]));
    float l = 0.0f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < 4; ++w) l += lw[w * G + hh] * fast_exp2(mw[w * G + hh] - M);
    }
    a.ws_m[(pbase + hh) * a.nparts + part] = M;
    a.ws_l[(pbase + hh) * a.nparts + part] = l;
  }
  if constexpr (SCORED) {
    // Block sums rescaled from the running max at the time to the partition max.
    for (int x = threadIdx.x; x < G * ntl * NSUB; x += 256) {
      const int hh = x / (ntl * NSUB);
      const int rem = x % (ntl * NSUB);
      const int tlc = rem / NSUB, sb = rem % NSUB;
      const float M = fmaxf(fmaxf(mw[hh], mw[G + hh]), fmaxf(mw[2 * G + hh], mw[3 * G + hh]));
      float e = e_rec[(tlc * NSUB + sb) * G + hh];
      const float mr = m_rec[tlc * G + hh];
      e = (M == -__builtin_inff() || mr == -__builtin_inff()) ? 0.0f : e * fast_exp2(mr - M);
      a.ws_e[((pbase + hh) * a.NT + t0 + tlc) * NSUB + sb] = e;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: grid (n_o_chunks + n_mass_chunks, B), 256 threads.
// ---------------------------------------------------------------------------
template <bool RING, bool Q_BF16>
__global__ __launch_bounds__(256) void kvs_combine(CombineArgs a) {
  extern __shared__ float lds[];
  const int b = blockIdx.y;
  const int P = a.nparts;
  float* wgt = lds;                    // [Hq][P]: 2^(m_p - M_h) / L_h
  // per-head max and normaliser
  for (int h = threadIdx.x; h < a.Hq; h += 256) {
    const float* m = a.ws_m + ((size_t)b * a.Hq + h) * P;
    const float* l = a.ws_l + ((size_t)b * a.Hq + h) * P;
    float M = -__builtin_inff();
    for (int p = 0; p < P; ++p) M = fmaxf(M, m[p]);
    float L = 0.0f;
    if (M != -__builtin_inff())
      for (int p = 0; p < P; ++p) L += l[p] * fast_exp2(m[p] - M);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    for (int p = 0; p < P; ++p)
      wgt[h * P + p] = (M == -__builtin_inff()) ? 0.0f : fast_exp2(m[p] - M) * inv;
  }
  __syncthreads();

  if ((int)blockIdx.x < a.n_o_chunks) {
    const int total = a.Hq * a.D;
    for (int x = blockIdx.x * 256 + threadIdx.x; x < total; x += a.n_o_chunks * 256) {
      const int h = x / a.D, d = x % a.D;
      const float* o = a.ws_o + (((size_t)b * a.Hq + h) * P) * a.D + d;
      float acc = 0.0f;
      for (int p = 0; p < P; ++p) acc += o[(size_t)p * a.D] * wgt[h * P + p];
      const size_t oi = ((size_t)b * a.Hq + h) * a.D + d;
      if constexpr (Q_BF16)
        ((uint16_t*)a.out)[oi] = f32_to_bf16_rne(acc);
      else
        ((float*)a.out)[oi] = acc;
    }
    return;
  }
  if (a.mass == nullptr) return;
  constexpr int NSUB = RING ? 2 : 1;
  const int chunk = blockIdx.x - a.n_o_chunks;
  const int i_cur = a.cur_pos[b];
  const int lap_i = RING ? i_cur / a.C : 0;
  for (int t = chunk * 256 + threadIdx.x; t < a.NT; t += a.n_mass_chunks * 256) {
    const int p = t / a.tpp;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      float acc = 0.0f;
      for (int h = 0; h < a.Hq; ++h)
        acc += a.ws_e[(((size_t)b * a.Hq + h) * a.NT + t) * NSUB + sb] * wgt[h * P + p];
      int blk = t;
      if constexpr (RING) {
        const int lap = ((lap_i & 1) == sb) ? lap_i : lap_i - 1;
        if (lap < 0) continue;
        blk = lap * (a.C / kTile) + t;
      }
      if (blk < a.nbmax) a.mass[(size_t)b * a.nbmax + blk] += acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
template <int KV, int D>
static hipError_t launch_partial_t(const PartialArgs& a, bool scored, bool ring, size_t lds_bytes,
                                   hipStream_t st) {
  dim3 grid(a.nparts, a.Hkv, a.B), block(256);
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

hipError_t launch_combine(const CombineArgs& a, bool ring, bool q_bf16, hipStream_t st) {
  dim3 grid(a.n_o_chunks + (a.mass ? a.n_mass_chunks : 0), a.B), block(256);
  const size_t lds = (size_t)a.Hq * a.nparts * sizeof(float);
  if (ring) {
    if (q_bf16) hipLaunchKernelGGL((kvs_combine<true, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine<true, false>), grid, block, lds, st, a);
  } else {
    if (q_bf16) hipLaunchKernelGGL((kvs_combine<false, true>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((kvs_combine<false, false>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace kvs
