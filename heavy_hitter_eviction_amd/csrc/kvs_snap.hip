// SnapKV-style prefill scoring (Context views at marginal cost, section 7,
// SOTA grounding, per-system reductions: once, when the prompt is done, the
// weights the last N prompt queries -- the observation window -- give each
// prompt token are added up per head, and that per-token score is replaced by
// its maximum over a 7-token neighbourhood, so the neighbours of a
// high-scoring key score high too), placed per 16-token block (Per-Head
// Attention as a Scoring Signal, "Fix: score per head, place per block").
//
// Column n of a (KV head, sequence) is (window query w, head h of the group),
// n = w*G + h; query w sits at position n_prompt - W + w and reads keys at or
// before it. Two passes over K (V is not needed):
//   pass 0 (kvs_snap_pass<.., 0>; for FP8 keys kvs_snap_pass0_f8): per
//     partition of tiles, each column's reference M and sum of 2^(s - M)
//     (S^T = K Q^T on MFMA);
//   kvs_snap_merge: per-column M and L over the partitions (with at most
//     8 partitions, the second pass merges them itself);
//   kvs_snap_pass<.., 1>: p = 2^(s - M) / L, summed over the window's queries
//     per (token, head): token_score[b][h][token];
//   kvs_snap_pool: per head, max over tokens j-R .. j+R (R = kernel/2) inside
//     the prompt, summed over the block's tokens and over heads, added to
//     block_score[b][block].
// M is not the exact column max: a lane moves its reference only when its new
// exponentials would add up past 2^32, so the rescale is rare; any reference
// gives the same p up to rounding. Tiles that end before the first window
// query need no mask (every column reads all their keys); only the last few
// tiles of a prompt take the masked path.

#include <type_traits>

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

template <int KV>
__device__ __forceinline__ int snap_dim(int t, int kg) {  // as the decode kernel's K fragment order
  constexpr int EPC = KV == KV_FP8 ? 16 : 8;
  return (t / EPC) * 4 * EPC + kg * EPC + t % EPC;
}

constexpr int kSnapMaxCB = 8;  // column blocks of 16 (W*G <= 128)
// Up to this many first-pass partitions the second pass merges their column
// statistics itself; past it kvs_snap_merge does, once per column.
constexpr int kSnapFoldParts = 8;

// Sum of 16 values as a balanced tree (independent adds, short dependency chains).
__device__ __forceinline__ float tree_sum16(const float* x) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// A lane's reference for its exponentials only moves when its new terms add
// up past this: each stays below 2^32, and a lane's sum over a whole prompt
// stays far inside the float range.
constexpr float kSnapLazyCap = 4294967296.0f;

}  // namespace

template <int KV, int D, int PASS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void kvs_snap_pass(SnapArgs a) {
  constexpr bool F8 = KV == KV_FP8;
  constexpr int eb = F8 ? 1 : 2;
  constexpr int NCH = D * eb / 64;   // 16-byte K chunks per lane per tile
  constexpr int NPL = D / 32;        // 16-byte query planes per column block
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, W = a.W, NCOL = W * G, NCB = (NCOL + 15) / 16;
  const int NCBe = (NCB + 1) & ~1;  // column blocks go two at a time
  u32x4* qpl = (u32x4*)lds;                                  // [NCBe][NPL][64] query planes
  f32x2* colML = (f32x2*)(qpl + NCBe * NPL * 64);           // [128] (column max, 1 / L); (+inf, 0): reads nothing
  float* wm = (float*)(colML + kSnapMaxCB * 16);             // [4 waves][128]
  float* wl = wm + 4 * kSnapMaxCB * 16;                      // [4 waves][128]
  const uint16_t* qg = (const uint16_t*)a.q;
  auto qrow = [&](int n) { return qg + (((size_t)b * W + n / G) * a.Hq + (size_t)g * G + n % G) * D; };

  // Query planes. bf16 keys: B fragments of the 16x16x32 bf16 MFMA in the K
  // fragment's dimension order (zeros for padding columns).
  // FP8 keys: the 16x16x128 FP8 MFMA takes keys as stored. The window's
  // queries are scaled by one power of two 2^sq (largest |q| into [128, 256))
  // and each scaled value v is split into hi = E4M3(v) and lo = E4M3(v - hi):
  // a bf16 value has 8 significant bits, hi keeps the top 4 and the remainder
  // fits the 4 bits of lo, so hi + lo = v exactly (only elements below 2^-10
  // of the largest lose low bits to the subnormal range). The 32 bytes of a
  // lane's B operand are two planes: for D = 128, (hi | lo) x (dims 0-63 |
  // 64-127 part of the lane); for D = 64, (hi, lo) paired with the key chunk
  // repeated, so one MFMA adds both products.
  // Every global load of the staging is issued before the first use, so the
  // prologue waits out one memory latency, not one per loop trip.
  float sl2 = a.scale_log2;  // multiplies raw scores into log2 units
  f32x2 ml_in = {__builtin_inff(), 0.0f};
  if constexpr (PASS == 1) {
    if (tid < NCOL) {
      const size_t ci = ((size_t)b * a.Hkv + g) * NCOL + tid;
      float M, L;
      if (a.nparts0 <= kSnapFoldParts) {
        // few first-pass partitions: their (reference, sum) pairs are merged
        // here, in kvs_snap_merge's arithmetic and order, instead of by a
        // launch of their own
        const float* pm = a.part_ml + ci * a.nparts0 * 2;
        float pmv[2 * kSnapFoldParts];
#pragma unroll
        for (int q = 0; q < kSnapFoldParts; ++q)
          if (q < a.nparts0) {
            pmv[2 * q] = pm[2 * q];
            pmv[2 * q + 1] = pm[2 * q + 1];
          }
        M = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < kSnapFoldParts; ++q)
          if (q < a.nparts0) M = fmaxf(M, pmv[2 * q]);
        L = 0.0f;
        if (M != -__builtin_inff()) {
#pragma unroll
          for (int q = 0; q < kSnapFoldParts; ++q)
            if (q < a.nparts0) L += pmv[2 * q + 1] * fast_exp2(pmv[2 * q] - M);
        }
      } else {
        M = a.col_m[ci];
        L = a.col_l[ci];
      }
      if (L > 0.0f) ml_in = f32x2{M, 1.0f / L};
    }
  }
  if constexpr (F8) {
    // source entries (block cb, 16-dim chunk, lane): 16 query values that
    // give one hi and one lo plane entry
    constexpr int NSC = D / 64;
    constexpr int kPer = kSnapMaxCB * NSC * 64 / 256;
    u32x4 src[kPer][2];
    uint32_t mx = 0;  // largest |q| as bf16 magnitude bits (monotone in |q|)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = tid + 256 * i, cb = x / (NSC * 64), chunk = (x / 64) % NSC, l = x % 64;
      const int n = cb * 16 + (l & 15);
      src[i][0] = src[i][1] = u32x4{0u, 0u, 0u, 0u};
      if (n < NCOL) {
        const u32x4* q = (const u32x4*)(qrow(n) + 64 * chunk + 16 * (l >> 4));
        src[i][0] = q[0];
        src[i][1] = q[1];
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(src[i][h][e] & 0x7FFFu, (src[i][h][e] >> 16) & 0x7FFFu));
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    uint32_t* red = (uint32_t*)wm;  // free until pass 0's end
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const int ex = (int)(mx >> 7);  // biased exponent of the largest |q|
    const int sq = mx == 0 ? 0 : ex == 0 ? 100 : min(100, 134 - ex);
    const float up = bits_to_f32((uint32_t)(127 + sq) << 23);
    sl2 *= bits_to_f32((uint32_t)(127 - sq) << 23);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = tid + 256 * i, cb = x / (NSC * 64), chunk = (x / 64) % NSC, l = x % 64;
      if (cb >= NCBe) continue;
      u32x4 hi, lo;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w0 = src[i][d >> 1][2 * (d & 1)], w1 = src[i][d >> 1][2 * (d & 1) + 1];
        const float f0 = bf16_lo(w0) * up, f1 = bf16_hi(w0) * up, f2 = bf16_lo(w1) * up, f3 = bf16_hi(w1) * up;
        s16x2 c = {0, 0};
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, f0, f1, 1.0f, false);
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, f2, f3, 1.0f, true);
        hi[d] = __builtin_bit_cast(uint32_t, c);
        const f32x2 v01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[d], 1.0f, false);
        const f32x2 v23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[d], 1.0f, true);
        c = s16x2{0, 0};
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, f0 - v01[0], f1 - v01[1], 1.0f, false);
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c, f2 - v23[0], f3 - v23[1], 1.0f, true);
        lo[d] = __builtin_bit_cast(uint32_t, c);
      }
      qpl[(cb * NPL + chunk) * 64 + l] = hi;
      qpl[(cb * NPL + NSC + chunk) * 64 + l] = lo;
    }
  } else {
    constexpr int kPer = kSnapMaxCB * NPL * 64 / 256;
    u32x4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = tid + 256 * i, cb = x / (NPL * 64), c = (x / 64) % NPL, l = x % 64;
      const int n = cb * 16 + (l & 15);
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (n < NCOL) v[i] = *(const u32x4*)(qrow(n) + snap_dim<KV>(8 * c, l >> 4));
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (tid + 256 * i < NCBe * NPL * 64) qpl[tid + 256 * i] = v[i];
  }
  if constexpr (PASS == 1) {
    if (tid < kSnapMaxCB * 16) colML[tid] = ml_in;
  }
  __syncthreads();

  const int npr = __builtin_amdgcn_readfirstlane(min(max(a.n_prompt[b], 0), a.C));
  const int te = max(0, min(a.NT, (npr + kTile - 1) / kTile));
  const int t0 = min(te, part * a.tpp), t1 = min(te, t0 + a.tpp);
  // tiles before tf end before the first window query's position, so every
  // column reads all their keys: [t0, tm) needs no mask, [tm, t1) does
  const int tf = npr >= W ? (npr - W) / kTile : 0;
  const int tm = max(t0, min(t1, tf));
  const size_t region = (size_t)a.C * D * eb;
  const char* kbase = (const char*)a.k + ((size_t)b * a.Hkv + g) * region;
  const float* ksb = a.ks ? a.ks + (size_t)b * a.C : nullptr;

  // pass 0: per lane and column block, a reference and the sum of 2^(x - ref)
  // over the lane's keys; pass 1 reads its column's max and 1 / L from LDS
  float m_run[kSnapMaxCB], l_run[kSnapMaxCB];
#pragma unroll
  for (int cb = 0; cb < kSnapMaxCB; ++cb) {
    m_run[cb] = -__builtin_inff();
    l_run[cb] = 0.0f;
  }
  auto col_ml = [&](int cb) { return colML[cb * 16 + j]; };

  // a tile's K as MFMA A operands, loaded straight into them: FP8, the lane's
  // 32 bytes (D = 128) or its chunk twice (D = 64); bf16, NPL 16-byte chunks
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  struct KOp {
    i32x8 f8;
    bf16x8 bf[F8 ? 1 : NPL];
    f32x4 ks;  // FP8 per-token scales of the lane's 4 rows
  };
  // buffer loads: the tile offset is one scalar, the lane's offset constant
  // (bases and offsets pinned to scalar registers: the compiler cannot see
  // that they are wave-uniform and would otherwise loop over lanes)
  auto uniform_ptr = [](const void* p) {
    const uint64_t u = (uint64_t)p;
    return (void*)(((uint64_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
  };
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(kbase), (short)0, (int)region, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(ksb ? ksb : (const float*)a.n_prompt), (short)0, F8 ? a.C * 4 : 0, 0x00020000);
  auto kld = [&](uint32_t vo, uint32_t so) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)vo, (int)so, 2));
  };
  auto load_k = [&](KOp& o, int t) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(t * (kTile * D * eb));
    if constexpr (F8) {
      const u32x4 c0 = kld(16 * lane, so);
      const u32x4 c1 = NCH > 1 ? kld(16 * lane + 1024, so) : c0;
      o.f8 = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      o.ks = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, 16 * kg, __builtin_amdgcn_readfirstlane(t * kTile * 4), 0));
    } else {
#pragma unroll
      for (int c = 0; c < NPL; ++c) o.bf[c] = __builtin_bit_cast(bf16x8, kld(16 * lane + 1024 * c, so));
      o.ks = f32x4{1.f, 1.f, 1.f, 1.f};
    }
  };
  // S^T block for one tile and column block cb (rows: the tile's tokens)
  auto bplane = [&](int cb, int pl) { return qpl[(cb * NPL + pl) * 64 + lane]; };
  auto b8 = [&](int cb, int f) {
    const u32x4 x0 = bplane(cb, 2 * f), x1 = bplane(cb, 2 * f + 1);
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  auto mma = [&](const KOp& k, int cb) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (F8) {
#pragma unroll
      for (int f = 0; f < NPL / 2; ++f)
        s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k.f8, b8(cb, f), s, 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < NPL; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.bf[c], __builtin_bit_cast(bf16x8, bplane(cb, c)), s, 0, 0, 0);
    }
    return s;
  };
  // In the FP8 loop the next block's MFMAs and query reads are spread over
  // this block's VALU work (one MFMA, one LDS read, then a few VALU ops).
  auto interleave = [&]() __attribute__((always_inline)) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
  };
  // unmasked tiles, pass 0: exponentials of one block's terms over a tile
  // pair against the lane's reference; the reference moves only when the new
  // terms add up past 2^32 (or the lane has none yet: the sum is +inf), so the
  // rescale is rare. Without a second tile its terms are dropped.
  auto soft0 = [&](int cb, const f32x4& s0, const f32x4& s1, const float (*kss)[4], bool two) {
    const float m = m_run[cb];
    const float e0 = (fast_exp2(fmaf(s0[0], kss[0][0], -m)) + fast_exp2(fmaf(s0[1], kss[0][1], -m))) +
                     (fast_exp2(fmaf(s0[2], kss[0][2], -m)) + fast_exp2(fmaf(s0[3], kss[0][3], -m)));
    const float e1 = (fast_exp2(fmaf(s1[0], kss[1][0], -m)) + fast_exp2(fmaf(s1[1], kss[1][1], -m))) +
                     (fast_exp2(fmaf(s1[2], kss[1][2], -m)) + fast_exp2(fmaf(s1[3], kss[1][3], -m)));
    float e = e0 + (two ? e1 : 0.0f);
    interleave();
    if (wave_any(!(e <= kSnapLazyCap))) {
      float x0[4], x1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x0[r] = s0[r] * kss[0][r];
        x1[r] = two ? s1[r] * kss[1][r] : -__builtin_inff();
      }
      const float m_new = fmaxf(fmaxf(m, fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3]))),
                                fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3])));
      l_run[cb] *= fast_exp2(m - m_new);
      m_run[cb] = m_new;
      e = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) e += fast_exp2(x0[r] - m_new) + fast_exp2(x1[r] - m_new);
    }
    l_run[cb] += e;
  };
  // unmasked tile, pass 1: acc += 2^(x - M) / L (padding columns: M = +inf, 1/L = 0)
  auto soft1 = [&](int cb, const f32x4& s0, const f32x4& s1, const float (*kss)[4], float (*acc)[4]) {
    const f32x2 ml = col_ml(cb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      acc[0][r] = fmaf(fast_exp2(fmaf(s0[r], kss[0][r], -ml[0])), ml[1], acc[0][r]);
      acc[1][r] = fmaf(fast_exp2(fmaf(s1[r], kss[1][r], -ml[0])), ml[1], acc[1][r]);
    }
    interleave();
  };
  // sum over the window's queries: the columns of one head are the lanes
  // j, j + G, j + 2G, ... of each 16-lane row, in every column block
  auto head_sum = [&](float* acc) {
    for (int off = G; off < 16; off <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], off, 64);
    }
  };

  // unmasked tiles, two per step sharing each query fragment read: wave w
  // takes t0 + w and t0 + w + 4, then 8 tiles on. Two register sets take
  // turns: the next pair loads into one while the other is consumed, so no
  // loaded register is copied and no wait sits on the loop's back edge.
  {
    KOp kb[2][2];
    auto issue = [&](auto P, int t) __attribute__((always_inline)) {
      load_k(kb[decltype(P)::value][0], t);
      load_k(kb[decltype(P)::value][1], t + 4);
    };
    auto step = [&](auto P, int t) __attribute__((always_inline)) {
      const KOp& k0 = kb[decltype(P)::value][0];
      const KOp& k1 = kb[decltype(P)::value][1];
      const bool two = t + 4 < tm;
      float kss[2][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kss[0][r] = k0.ks[r] * sl2;
        kss[1][r] = k1.ks[r] * sl2;
      }
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      auto soft = [&](int cb, const f32x4& x0, const f32x4& x1) __attribute__((always_inline)) {
        if constexpr (PASS == 0)
          soft0(cb, x0, x1, kss, two);
        else
          soft1(cb, x0, x1, kss, acc);  // a second tile past the end is summed but never stored
      };
      if constexpr (F8) {
        // one column block at a time, software-pipelined: the MFMAs of block
        // cb + 1 (query fragments read one block earlier) are issued before
        // the exponentials of block cb, so the matrix pipe and the VALU work
        // at once; the fragments of block cb + 2 load meanwhile
        i32x8 qf[NPL / 2];
        f32x4 sc[2][2];
        auto frag = [&](int cb) __attribute__((always_inline)) {
#pragma unroll
          for (int f = 0; f < NPL / 2; ++f) qf[f] = b8(cb, f);
        };
        auto mm = [&](int bi) __attribute__((always_inline)) {
          sc[bi][0] = sc[bi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NPL / 2; ++f) {
            sc[bi][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k0.f8, qf[f], sc[bi][0], 0, 0, 0, 0, 0, 0);
            sc[bi][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k1.f8, qf[f], sc[bi][1], 0, 0, 0, 0, 0, 0);
          }
        };
        frag(0);
        mm(0);
        if (NCB > 1) frag(1);
#pragma unroll
        for (int cb = 0; cb < kSnapMaxCB; ++cb) {
          if (cb >= NCB) break;
          if (cb + 1 < NCB) mm((cb + 1) & 1);
          if (cb + 2 < NCB) frag(cb + 2);
          soft(cb, sc[cb & 1][0], sc[cb & 1][1]);
        }
      } else {
        // bf16: two column blocks at a time, four accumulations
#pragma unroll
        for (int cb = 0; cb < kSnapMaxCB; cb += 2) {
          if (cb >= NCB) break;
          f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
#pragma unroll
          for (int c = 0; c < NPL; ++c) {
            const bf16x8 qa = __builtin_bit_cast(bf16x8, bplane(cb, c));
            const bf16x8 qb = __builtin_bit_cast(bf16x8, bplane(cb + 1, c));
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0.bf[c], qa, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1.bf[c], qa, s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0.bf[c], qb, s2, 0, 0, 0);
            s3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1.bf[c], qb, s3, 0, 0, 0);
          }
          soft(cb, s0, s1);
          soft(cb + 1, s2, s3);
        }
      }
      if constexpr (PASS == 1) {
        head_sum(acc[0]);
        head_sum(acc[1]);
        if (j < G) {
          float* dst = a.token_score + ((size_t)b * a.Hq + (size_t)g * G + j) * a.C + (size_t)t * kTile + 4 * kg;
          *(f32x4*)dst = f32x4{acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
          if (two) *(f32x4*)(dst + 4 * kTile) = f32x4{acc[1][0], acc[1][1], acc[1][2], acc[1][3]};
        }
      }
    };
    constexpr std::integral_constant<int, 0> P0{};
    constexpr std::integral_constant<int, 1> P1{};
    // The loads are issued unconditionally (a tile past the end reads
    // whatever is there, or zeros past the region's end, and is never used):
    // a conditional issue would make every wait assume the shorter queue.
    int t = t0 + wave;
    if (t < tm) issue(P0, t);
    while (t < tm) {
      issue(P1, t + 8);
      step(P0, t);
      t += 8;
      if (t >= tm) break;
      issue(P0, t + 8);
      step(P1, t);
      t += 8;
    }
  }

  // masked tiles (the last few before the window's end), one at a time
  for (int t = tm + wave; t < t1; t += 4) {
    KOp k;
    load_k(k, t);
    const f32x4 ks = k.ks;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < kSnapMaxCB; ++cb) {
      if (cb >= NCB) break;
      const f32x4 s = mma(k, cb);
      const int n = cb * 16 + j;
      const int qpos = npr - W + (n < NCOL ? n / G : 0);
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = t * kTile + 4 * kg + r;
        valid[r] = n < NCOL && p <= qpos && p < npr;
      }
      if constexpr (PASS == 0) {
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = valid[r] ? s[r] * (ks[r] * sl2) : -__builtin_inff();
        const float m_new = fmaxf(m_run[cb], fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        if (m_new != -__builtin_inff()) {
          float e = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) e += fast_exp2(x[r] - m_new);
          l_run[cb] = l_run[cb] * fast_exp2(m_run[cb] - m_new) + e;
          m_run[cb] = m_new;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (valid[r]) acc[r] = fmaf(fast_exp2(fmaf(s[r], ks[r] * sl2, -col_ml(cb)[0])), col_ml(cb)[1], acc[r]);
      }
    }
    if constexpr (PASS == 1) {
      head_sum(acc);
      if (j < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = t * kTile + 4 * kg + r;
          if (p < npr) a.token_score[((size_t)b * a.Hq + (size_t)g * G + j) * a.C + p] = acc[r];
        }
      }
    }
  }

  if constexpr (PASS == 0) {
    // the four lanes of a column, then the four waves: one (max, sum) per
    // column for this partition
#pragma unroll
    for (int cb = 0; cb < kSnapMaxCB; ++cb) {
      if (cb >= NCB) break;
      const float M = rows_max(m_run[cb]);
      const float ls = M == -__builtin_inff() ? 0.0f : l_run[cb] * fast_exp2(m_run[cb] - M);
      const float L = rows_sum(ls);
      const int n = cb * 16 + j;
      if (kg == 0 && n < NCOL) {
        wm[wave * kSnapMaxCB * 16 + n] = M;
        wl[wave * kSnapMaxCB * 16 + n] = L;
      }
    }
    __syncthreads();
    for (int n = tid; n < NCOL; n += 256) {
      float M = -__builtin_inff();
      for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w * kSnapMaxCB * 16 + n]);
      float L = 0.0f;
      if (M != -__builtin_inff())
        for (int w = 0; w < 4; ++w) L += wl[w * kSnapMaxCB * 16 + n] * fast_exp2(wm[w * kSnapMaxCB * 16 + n] - M);
      const size_t si = ((((size_t)b * a.Hkv + g) * NCOL + n) * a.nparts + part) * 2;
      a.part_ml[si] = M;
      a.part_ml[si + 1] = L;
    }
  }
}

// Pass 0 for FP8 keys on the 32x32x64 FP8 MFMA. A step takes the tile pair
// (t, t + 4) as the 32 rows of A (keys as stored, 32 bytes a lane: lane l
// holds token l % 16 of tile t + 4 * ((l >> 4) & 1), dims 32 (l >> 5) +
// [0, 32) of each 64-dim slice) and a 32-column block of the window as B
// (query planes as below), so one LDS read of the query serves 32 tokens, and
// the MFMAs of the next column block are issued between this block's
// exponentials: with this shape the VALU keeps working while the matrix pipe
// runs, which the 16x16x128 shape does not allow (measured on gfx950). The
// accumulator's lane l holds column l % 32 and rows 8 q + 4 (l >> 5) + r
// (register 4 q + r). Two waves per SIMD: a workgroup's four waves each keep
// two tile pairs of K and scales in registers (one in use, one loading).
// Pass 1 stays on the 16x16 kernel, where it measured faster.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void kvs_snap_pass0_f8(SnapArgs a) {
  constexpr int NSL = D / 64;          // 64-dim slices: MFMAs per (block, part)
  constexpr int NPL = NSL * 4;         // 16-byte query planes per 32-column block: slice x (hi, lo) x half
  constexpr int TB = kTile * D;        // bytes per K tile
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, W = a.W, NCOL = W * G;
  constexpr int NB = 4;                // 32-column blocks (W*G <= 128; padding columns have zero queries)
  u32x4* qpl = (u32x4*)lds;                                    // [NB][NPL][64]
  float* wm = (float*)(qpl + NB * NPL * 64);                   // [4 waves][128]
  float* wl = wm + 4 * kSnapMaxCB * 16;                        // [4 waves][128]
  const uint16_t* qg = (const uint16_t*)a.q;
  auto qrow = [&](int n) { return qg + (((size_t)b * W + n / G) * a.Hq + (size_t)g * G + n % G) * D; };

  // Query planes: the window's queries scaled by one power of two 2^sq
  // (largest |q| into [128, 256)), each scaled value v split into hi =
  // E4M3(v) and lo = E4M3(v - hi); a bf16 value has 8 significant bits, hi
  // keeps the top 4 and lo the rest, so hi + lo = v exactly (only elements
  // below 2^-10 of the largest lose low bits to the subnormal range). Plane
  // (slice s, part p, half u) of block cb holds, for lane l, the codes of
  // column 32 cb + l % 32, dims 64 s + 32 (l >> 5) + 16 u + [0, 16). All
  // global loads are issued before the first use.
  float sl2 = a.scale_log2;
  {
    constexpr int kPer = 4 * NSL * 64 / 256;  // source entries (block, slice, lane) per thread
    u32x4 src[kPer][4];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = tid + 256 * i, cb = x / (NSL * 64), sl = (x / 64) % NSL, l = x % 64;
      const int n = cb * 32 + (l & 31);
#pragma unroll
      for (int u = 0; u < 4; ++u) src[i][u] = u32x4{0u, 0u, 0u, 0u};
      if (n < NCOL) {
        const u32x4* q = (const u32x4*)(qrow(n) + 64 * sl + 32 * (l >> 5));
#pragma unroll
        for (int u = 0; u < 4; ++u) src[i][u] = q[u];
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = max(mx, max(src[i][u][e] & 0x7FFFu, (src[i][u][e] >> 16) & 0x7FFFu));
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    uint32_t* red = (uint32_t*)wm;  // free until pass 0's end
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const int ex = (int)(mx >> 7);  // biased exponent of the largest |q|
    const int sq = mx == 0 ? 0 : ex == 0 ? 100 : min(100, 134 - ex);
    const float up = bits_to_f32((uint32_t)(127 + sq) << 23);
    sl2 *= bits_to_f32((uint32_t)(127 - sq) << 23);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int x = tid + 256 * i, cb = x / (NSL * 64), sl = (x / 64) % NSL, l = x % 64;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 hi, lo;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t w0 = src[i][2 * u + (d >> 1)][2 * (d & 1)], w1 = src[i][2 * u + (d >> 1)][2 * (d & 1) + 1];
          const float f0 = bf16_lo(w0) * up, f1 = bf16_hi(w0) * up, f2 = bf16_lo(w1) * up, f3 = bf16_hi(w1) * up;
          s16x2 cv = {0, 0};
          cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv, f0, f1, 1.0f, false);
          cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv, f2, f3, 1.0f, true);
          hi[d] = __builtin_bit_cast(uint32_t, cv);
          const f32x2 v01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[d], 1.0f, false);
          const f32x2 v23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[d], 1.0f, true);
          cv = s16x2{0, 0};
          cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv, f0 - v01[0], f1 - v01[1], 1.0f, false);
          cv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv, f2 - v23[0], f3 - v23[1], 1.0f, true);
          lo[d] = __builtin_bit_cast(uint32_t, cv);
        }
        qpl[(cb * NPL + (sl * 2 + 0) * 2 + u) * 64 + l] = hi;
        qpl[(cb * NPL + (sl * 2 + 1) * 2 + u) * 64 + l] = lo;
      }
    }
  }
  __syncthreads();

  const int npr = __builtin_amdgcn_readfirstlane(min(max(a.n_prompt[b], 0), a.C));
  const int te = max(0, min(a.NT, (npr + kTile - 1) / kTile));
  const int t0 = min(te, part * a.tpp), t1 = min(te, t0 + a.tpp);
  // tiles before tf end before the first window query's position, so every
  // column reads all their keys: pairs inside [t0, tm) need no mask
  const int tf = npr >= W ? (npr - W) / kTile : 0;
  const int tm = max(t0, min(t1, tf));
  const size_t region = (size_t)a.C * D;
  auto uniform_ptr = [](const void* p) {
    const uint64_t u = (uint64_t)p;
    return (void*)(((uint64_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
  };
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr((const char*)a.k + ((size_t)b * a.Hkv + g) * region), (short)0, (int)region, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.ks + (size_t)b * a.C), (short)0, a.C * 4, 0x00020000);
  // lane's byte offsets: K (token l % 16 of tile t or t + 4, key groups
  // 2 (l >> 5) and 2 (l >> 5) + 1 of a slice), scales (rows 8 q + 4 h + r)
  const uint32_t kvo = ((lane >> 4) & 1) * 4 * TB + 16 * (32 * h + (lane & 15));

  // A tile pair: K as MFMA operands and the per-token scales of the
  // accumulator rows 8 q + 4 h + [0, 4), q = 0..3
  struct Pair {
    i32x8 k[NSL];
    f32x4 ks[4];
  };
  auto load_pair = [&](Pair& o, int t) __attribute__((always_inline)) {
    const int so = __builtin_amdgcn_readfirstlane(t * TB);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const u32x4 x0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(kvo + 1024 * sl), so, 2));
      const u32x4 x1 =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(kvo + 1024 * sl + 256), so, 2));
      o.k[sl] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
    const int ss = __builtin_amdgcn_readfirstlane(t * kTile * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o.ks[q] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, (q >> 1) * 4 * kTile * 4 + (8 * (q & 1) + 4 * h) * 4, ss, 0));
  };
  auto bop = [&](int cb, int sl, int pt) {
    const u32x4 x0 = qpl[(cb * NPL + (sl * 2 + pt) * 2) * 64 + lane];
    const u32x4 x1 = qpl[(cb * NPL + (sl * 2 + pt) * 2 + 1) * 64 + lane];
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  // rows = the pair's 32 tokens, columns = the block's 32 columns
  auto scores = [&](const Pair& p, int cb) __attribute__((always_inline)) {
    f32x16 s = {};
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(p.k[sl], bop(cb, sl, pt), s, 0, 0, 0, 0, 0, 0);
    return s;
  };
  // issue order inside a block: the next block's query reads, then its MFMAs
  // one at a time between runs of this block's VALU work, so the wave keeps
  // issuing VALU while each MFMA runs
  auto interleave = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * NSL, 0);
#pragma unroll
    for (int i = 0; i < 2 * NSL; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  float m_run[NB], l_run[NB];  // the lane's column of each block
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    m_run[cb] = -__builtin_inff();
    l_run[cb] = 0.0f;
  }

  // One step over a tile pair. MASKED: rows past the prompt or after a
  // column's query are left out and tile t + 4 only counts when two is set.
  auto step = [&](const Pair& p, int t, bool two, auto MASKED) __attribute__((always_inline)) {
    constexpr bool MK = decltype(MASKED)::value;
    float kss[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) kss[k] = p.ks[k >> 2][k & 3] * sl2;
    f32x16 sc[2];
    sc[0] = scores(p, 0);
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      if (cb + 1 < NB) sc[(cb + 1) & 1] = scores(p, cb + 1);
      const f32x16& S = sc[cb & 1];
      const int n = cb * 32 + c;
      if constexpr (!MK) {
        // the reference moves only when the new terms add up past 2^32 (or
        // the lane has none yet: the sum is +inf), so the rescale is rare
        const float m = m_run[cb];
        float ex[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) ex[k] = fast_exp2(fmaf(S[k], kss[k], -m));
        float e = tree_sum16(ex);
        interleave();
        if (wave_any(!(e <= kSnapLazyCap))) {
          float mx = m;
#pragma unroll
          for (int k = 0; k < 16; ++k) mx = fmaxf(mx, S[k] * kss[k]);
          l_run[cb] *= fast_exp2(m - mx);
          m_run[cb] = mx;
#pragma unroll
          for (int k = 0; k < 16; ++k) ex[k] = fast_exp2(S[k] * kss[k] - mx);
          e = tree_sum16(ex);
        }
        l_run[cb] += e;
      } else {
        const int qpos = npr - W + (n < NCOL ? n / G : 0);
        float x[16], mx = m_run[cb];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int q = k >> 2, pos = (t + 4 * (q >> 1)) * kTile + 8 * (q & 1) + 4 * h + (k & 3);
          const bool valid = n < NCOL && pos <= qpos && pos < npr && (two || q < 2);
          x[k] = valid ? S[k] * kss[k] : -__builtin_inff();
          mx = fmaxf(mx, x[k]);
        }
        if (mx != -__builtin_inff()) {
#pragma unroll
          for (int k = 0; k < 16; ++k) x[k] = fast_exp2(x[k] - mx);
          l_run[cb] = l_run[cb] * fast_exp2(m_run[cb] - mx) + tree_sum16(x);
          m_run[cb] = mx;
        }
      }
    }
  };

  // Wave w takes the pairs (t, t + 4), t = t0 + w, t0 + w + 8, ...: every
  // tile of [t0, t1) once. Two register sets take turns (one in use, one
  // loading); loads are issued unconditionally (past the end they read
  // whatever is there, or zeros past the region, and are not used), since a
  // conditional issue would make every wait assume the shorter queue.
  {
    Pair pr[2];
    constexpr std::integral_constant<bool, false> UNMASKED{};
    constexpr std::integral_constant<bool, true> MASKED{};
    int t = t0 + wave;
    if (t + 4 < tm) load_pair(pr[0], t);
    while (t + 4 < tm) {
      load_pair(pr[1], t + 8);
      step(pr[0], t, true, UNMASKED);
      t += 8;
      if (!(t + 4 < tm)) break;
      load_pair(pr[0], t + 8);
      step(pr[1], t, true, UNMASKED);
      t += 8;
    }
    for (; t < t1; t += 8) {
      load_pair(pr[0], t);
      step(pr[0], t, t + 4 < t1, MASKED);
    }
  }

  {
    // the two halves of a column, then the four waves: one (max, sum) per
    // column for this partition
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      auto sw = __builtin_amdgcn_permlane32_swap(f32_bits(m_run[cb]), f32_bits(m_run[cb]), false, false);
      const float M = fmaxf(bits_to_f32(sw[0]), bits_to_f32(sw[1]));
      const float ls = M == -__builtin_inff() ? 0.0f : l_run[cb] * fast_exp2(m_run[cb] - M);
      auto sw2 = __builtin_amdgcn_permlane32_swap(f32_bits(ls), f32_bits(ls), false, false);
      const float L = bits_to_f32(sw2[0]) + bits_to_f32(sw2[1]);
      const int n = cb * 32 + c;
      if (h == 0 && n < NCOL) {
        wm[wave * kSnapMaxCB * 16 + n] = M;
        wl[wave * kSnapMaxCB * 16 + n] = L;
      }
    }
    __syncthreads();
    for (int n = tid; n < NCOL; n += 256) {
      float M = -__builtin_inff();
      for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w * kSnapMaxCB * 16 + n]);
      float L = 0.0f;
      if (M != -__builtin_inff())
        for (int w = 0; w < 4; ++w) L += wl[w * kSnapMaxCB * 16 + n] * fast_exp2(wm[w * kSnapMaxCB * 16 + n] - M);
      const size_t si = ((((size_t)b * a.Hkv + g) * NCOL + n) * a.nparts + part) * 2;
      a.part_ml[si] = M;
      a.part_ml[si + 1] = L;
    }
  }
}

// grid (ceil(NCOL*Hkv/256), B): exact per-column max and sum over partitions
__global__ __launch_bounds__(256) void kvs_snap_merge(SnapArgs a) {
  const int b = blockIdx.y;
  const int NCOL = a.W * a.G;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= a.Hkv * NCOL) return;
  const size_t ci = (size_t)b * a.Hkv * NCOL + x;
  const float* pm = a.part_ml + ci * a.nparts * 2;
  float M = -__builtin_inff();
  for (int p = 0; p < a.nparts; ++p) M = fmaxf(M, pm[2 * p]);
  float L = 0.0f;
  if (M != -__builtin_inff())
    for (int p = 0; p < a.nparts; ++p) L += pm[2 * p + 1] * fast_exp2(pm[2 * p] - M);
  a.col_m[ci] = M;
  a.col_l[ci] = L;
}

// grid (ceil(C / 256), B): a workgroup pools 256 tokens (16 blocks) of one
// sequence; wave w takes heads w, w + 4, ... in ascending order. A lane owns 4
// consecutive tokens and reads the NQ float4s centred on them (ceil(R / 4) on
// either side), takes each token's max over the R on either side inside the
// prompt, and the 4 lanes of a block add their sums. The block's four wave
// sums are added in wave order.
constexpr int kPoolTokens = 256;
constexpr int kPoolMaxR = 16;
template <int NQ>
__global__ __launch_bounds__(256) void kvs_snap_pool(SnapArgs a) {
  constexpr int HQ = NQ / 2;
  __shared__ float wsum[4][kPoolTokens / kTile];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int npr = __builtin_amdgcn_readfirstlane(min(max(a.n_prompt[b], 0), a.C));
  const int lo = blockIdx.x * kPoolTokens;
  if (lo >= npr) return;
  const int R = a.pool / 2;
  const int p0 = lo + 4 * lane;
  float bsum = 0.0f;
  for (int h = wave; h < a.Hq; h += 4) {
    const float* sc = a.token_score + ((size_t)b * a.Hq + h) * a.C;
    float v[4 * NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int ps = p0 + 4 * (q - HQ);   // a multiple of 4: ps < npr <= C keeps ps + 3 inside the row
      f32x4 x = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
      if (ps >= 0 && ps < npr) x = *(const f32x4*)(sc + ps);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = ps + e < npr ? x[e] : -__builtin_inff();
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float m = v[4 * HQ + u];
#pragma unroll
      for (int k = 1; k <= 4 * HQ; ++k)
        if (k <= R) m = fmaxf(m, fmaxf(v[4 * HQ + u - k], v[4 * HQ + u + k]));
      if (p0 + u < npr) s += m;
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    bsum += s;
  }
  if ((lane & 3) == 0) wsum[wave][lane >> 2] = bsum;
  __syncthreads();
  if (tid < kPoolTokens / kTile) {
    const int blk = blockIdx.x * (kPoolTokens / kTile) + tid;
    if (blk < a.nbmax && blk * kTile < npr)
      a.block_score[(size_t)b * a.nbmax + blk] += (wsum[0][tid] + wsum[1][tid]) + (wsum[2][tid] + wsum[3][tid]);
  }
}

template <int KV, int D>
static hipError_t launch_snap_t(const SnapArgs& a, hipStream_t st) {
  const int ncol = a.W * a.G;
  const size_t tail = (2 + 8) * kSnapMaxCB * 16 * sizeof(float);
  const size_t lds16 = (size_t)((((ncol + 15) / 16) + 1) & ~1) * (D / 32) * 64 * 16 + tail;
  hipError_t e;
  if constexpr (KV == KV_FP8) {
    hipLaunchKernelGGL((kvs_snap_pass0_f8<D>), dim3(a.nparts, a.Hkv, a.B), dim3(256), (size_t)4 * (D / 16) * 64 * 16 + tail,
                       st, a);
  } else {
    hipLaunchKernelGGL((kvs_snap_pass<KV, D, 0>), dim3(a.nparts, a.Hkv, a.B), dim3(256), lds16, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.nparts > kSnapFoldParts) {
    hipLaunchKernelGGL(kvs_snap_merge, dim3((a.Hkv * ncol + 255) / 256, a.B), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // pass 1 (16x16 kernel, four waves per SIMD) takes its own partition of the
  // tiles: about 1024 workgroups
  SnapArgs a1 = a;
  a1.nparts0 = a.nparts;
  const int pairs = a.B * a.Hkv;
  const int pt = max(1, (1024 + pairs - 1) / pairs);
  a1.tpp = max(1, (a.NT + pt - 1) / pt);
  a1.nparts = (a.NT + a1.tpp - 1) / a1.tpp;
  hipLaunchKernelGGL((kvs_snap_pass<KV, D, 1>), dim3(a1.nparts, a.Hkv, a.B), dim3(256), lds16, st, a1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.block_score) {
    const int R = a.pool / 2;
    if (R > kPoolMaxR) return hipErrorInvalidValue;
    const dim3 pg((a.C + kPoolTokens - 1) / kPoolTokens, a.B);
    if (R <= 4)
      hipLaunchKernelGGL(kvs_snap_pool<3>, pg, dim3(256), 0, st, a);
    else if (R <= 8)
      hipLaunchKernelGGL(kvs_snap_pool<5>, pg, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(kvs_snap_pool<9>, pg, dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_snap(int kv, int d, const SnapArgs& a, hipStream_t st) {
  if (kv == KV_BF16) {
    if (d == 64) return launch_snap_t<KV_BF16, 64>(a, st);
    if (d == 128) return launch_snap_t<KV_BF16, 128>(a, st);
  } else if (kv == KV_FP8) {
    if (d == 64) return launch_snap_t<KV_FP8, 64>(a, st);
    if (d == 128) return launch_snap_t<KV_FP8, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvs
