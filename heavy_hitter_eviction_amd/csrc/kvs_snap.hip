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
//   kvs_snap_pass<.., 0>: per partition of tiles, each column's reference M
//     and sum of 2^(s - M) (S^T = K Q^T on MFMA, 16 columns per block);
//   kvs_snap_merge: per-column M and L over the partitions;
//   kvs_snap_pass<.., 1>: p = 2^(s - M) / L, summed over the window's queries
//     per (token, head): token_score[b][h][token];
//   kvs_snap_pool: per head, max over tokens j-R .. j+R (R = kernel/2) inside
//     the prompt, summed over the block's tokens and over heads, added to
//     block_score[b][block].
// M is not the exact column max: a lane moves its reference only when a logit
// passes it by more than 8 (log2 units), so no exponential exceeds 2^8 and the
// rescale is rare; any reference gives the same p up to rounding. Tiles that
// end before the first window query need no mask (every column reads all
// their keys); only the last few tiles of a prompt take the masked path.

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
// A lane's reference for its exponentials only moves when a new logit passes
// it by more than this (log2 units): every exponential stays below 2^8 and
// most tiles skip the rescale.
constexpr float kSnapLazy = 8.0f;

}  // namespace

template <int KV, int D, int PASS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void kvs_snap_pass(SnapArgs a) {
  constexpr int eb = KV == KV_FP8 ? 1 : 2;
  constexpr int NCH = D * eb / 64;   // 16-byte K chunks per lane per tile
  constexpr int NC32 = D / 32;       // MFMA contraction chunks
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, W = a.W, NCOL = W * G, NCB = (NCOL + 15) / 16;
  const int NCBe = (NCB + 1) & ~1;  // column blocks go two at a time
  bf16x8* qfrag = (bf16x8*)lds;                              // [NCBe][NC32][64]
  float* colM = (float*)(qfrag + NCBe * NC32 * 64);          // [128] column max (+inf: reads nothing)
  float* colIL = colM + kSnapMaxCB * 16;                     // [128] 1 / L (0: reads nothing)
  float* wm = colIL + kSnapMaxCB * 16;                       // [4 waves][128]
  float* wl = wm + 4 * kSnapMaxCB * 16;                      // [4 waves][128]

  // window queries as B fragments (zeros for padding columns)
  for (int x = tid; x < NCBe * NC32 * 64; x += 256) {
    const int cb = x / (NC32 * 64), c = (x / 64) % NC32, l = x % 64;
    const int n = cb * 16 + (l & 15), lk = l >> 4;
    bf16x8 f;
    if (n < NCOL) {
      const int w = n / G, h = n % G;
      const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)b * W + w) * a.Hq + (size_t)g * G + h) * D;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = __builtin_bit_cast(__bf16, qrow[snap_dim<KV>(8 * c + e, lk)]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (__bf16)0.0f;
    }
    qfrag[x] = f;
  }
  if constexpr (PASS == 1) {
    for (int n = tid; n < kSnapMaxCB * 16; n += 256) {
      float M = __builtin_inff(), IL = 0.0f;
      if (n < NCOL) {
        const size_t ci = ((size_t)b * a.Hkv + g) * NCOL + n;
        const float L = a.col_l[ci];
        if (L > 0.0f) {
          M = a.col_m[ci];
          IL = 1.0f / L;
        }
      }
      colM[n] = M;
      colIL[n] = IL;
    }
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
  // over the lane's keys; pass 1: the lane's column max and 1 / L
  float m_run[kSnapMaxCB], l_run[kSnapMaxCB];
#pragma unroll
  for (int cb = 0; cb < kSnapMaxCB; ++cb) {
    if constexpr (PASS == 0) {
      m_run[cb] = -__builtin_inff();
      l_run[cb] = 0.0f;
    } else {
      m_run[cb] = colM[cb * 16 + j];
      l_run[cb] = colIL[cb * 16 + j];
    }
  }

  auto load_k = [&](u32x4* kc, f32x4& ks, int t) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) kc[i] = *(const u32x4*)(kbase + (size_t)t * kTile * D * eb + 1024 * i + 16 * lane);
    if constexpr (KV == KV_FP8) ks = *(const f32x4*)(ksb + (size_t)t * kTile + 4 * kg);
  };
  auto to_bf16 = [&](const u32x4* kc, bf16x8* kk) {
#pragma unroll
    for (int c = 0; c < NC32; ++c) {
      if constexpr (KV == KV_FP8) {
        const u32x4 w = kc[c >> 1];
        const u32x2 lo2 = fp8x4_to_bf16x4(w[2 * (c & 1)]);
        const u32x2 hi2 = fp8x4_to_bf16x4(w[2 * (c & 1) + 1]);
        const u32x4 k4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
        kk[c] = __builtin_bit_cast(bf16x8, k4);
      } else {
        kk[c] = __builtin_bit_cast(bf16x8, kc[c]);
      }
    }
  };
  // unmasked tile, pass 0: lane-private running sums, rescaled only when some
  // lane's logit passes its reference by more than kSnapLazy
  auto soft0 = [&](int cb, const f32x4& s, const float* kss) {
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = s[r] * kss[r];
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (wave_any(mx > m_run[cb] + kSnapLazy)) {
      const float m_new = fmaxf(m_run[cb], mx);
      l_run[cb] *= fast_exp2(m_run[cb] - m_new);
      m_run[cb] = m_new;
    }
    l_run[cb] += (fast_exp2(x[0] - m_run[cb]) + fast_exp2(x[1] - m_run[cb])) +
                 (fast_exp2(x[2] - m_run[cb]) + fast_exp2(x[3] - m_run[cb]));
  };
  // unmasked tile, pass 1: acc += 2^(x - M) / L (padding columns: M = +inf, 1/L = 0)
  auto soft1 = [&](int cb, const f32x4& s, const float* kss, float* acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(fast_exp2(fmaf(s[r], kss[r], -m_run[cb])), l_run[cb], acc[r]);
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
  // takes t0 + w and t0 + w + 4, then 8 tiles on; the next pair is in flight
  {
    u32x4 kn[2][NCH];
    f32x4 ksn[2] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};
    int t = t0 + wave;
    if (t < tm) {
      load_k(kn[0], ksn[0], t);
      load_k(kn[1], ksn[1], t + 4 < tm ? t + 4 : t);
    }
    for (; t < tm; t += 8) {
      const bool two = t + 4 < tm;
      bf16x8 kk[2][NC32];
      to_bf16(kn[0], kk[0]);
      to_bf16(kn[1], kk[1]);
      float kss[2][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kss[0][r] = ksn[0][r] * a.scale_log2;
        kss[1][r] = ksn[1][r] * a.scale_log2;
      }
      if (t + 8 < tm) {
        load_k(kn[0], ksn[0], t + 8);
        load_k(kn[1], ksn[1], t + 12 < tm ? t + 12 : t + 8);
      }
      float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int cb = 0; cb < kSnapMaxCB; cb += 2) {
        if (cb >= NCB) break;
        // four independent accumulations: (block cb, cb + 1) x (tile t, t + 4)
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
#pragma unroll
        for (int c = 0; c < NC32; ++c) {
          const bf16x8 qa = qfrag[(cb * NC32 + c) * 64 + lane];
          const bf16x8 qb = qfrag[((cb + 1) * NC32 + c) * 64 + lane];
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[0][c], qa, s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[1][c], qa, s1, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[0][c], qb, s2, 0, 0, 0);
          s3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[1][c], qb, s3, 0, 0, 0);
        }
        if constexpr (PASS == 0) {
          soft0(cb, s0, kss[0]);
          soft0(cb + 1, s2, kss[0]);
          if (two) {
            soft0(cb, s1, kss[1]);
            soft0(cb + 1, s3, kss[1]);
          }
        } else {
          // a repeated second tile is summed but never stored
          soft1(cb, s0, kss[0], acc[0]);
          soft1(cb + 1, s2, kss[0], acc[0]);
          soft1(cb, s1, kss[1], acc[1]);
          soft1(cb + 1, s3, kss[1], acc[1]);
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
    }
  }

  // masked tiles (the last few before the window's end), one at a time
  for (int t = tm + wave; t < t1; t += 4) {
    u32x4 kc[NCH];
    f32x4 ks = {1.f, 1.f, 1.f, 1.f};
    load_k(kc, ks, t);
    bf16x8 kk[NC32];
    to_bf16(kc, kk);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < kSnapMaxCB; ++cb) {
      if (cb >= NCB) break;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC32; ++c)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], qfrag[(cb * NC32 + c) * 64 + lane], s, 0, 0, 0);
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
        for (int r = 0; r < 4; ++r) x[r] = valid[r] ? s[r] * (ks[r] * a.scale_log2) : -__builtin_inff();
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
          if (valid[r]) acc[r] = fmaf(fast_exp2(fmaf(s[r], ks[r] * a.scale_log2, -m_run[cb])), l_run[cb], acc[r]);
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
static hipError_t launch_snap_t(const SnapArgs& a, size_t lds, hipStream_t st) {
  dim3 grid(a.nparts, a.Hkv, a.B), block(256);
  hipLaunchKernelGGL((kvs_snap_pass<KV, D, 0>), grid, block, lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ncol = a.W * a.G;
  hipLaunchKernelGGL(kvs_snap_merge, dim3((a.Hkv * ncol + 255) / 256, a.B), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((kvs_snap_pass<KV, D, 1>), grid, block, lds, st, a);
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
  const int ncb = ((a.W * a.G + 15) / 16 + 1) & ~1;
  const size_t lds = (size_t)ncb * (d / 32) * 64 * 16 + (2 + 8) * kSnapMaxCB * 16 * sizeof(float);
  if (kv == KV_BF16) {
    if (d == 64) return launch_snap_t<KV_BF16, 64>(a, lds, st);
    if (d == 128) return launch_snap_t<KV_BF16, 128>(a, lds, st);
  } else if (kv == KV_FP8) {
    if (d == 64) return launch_snap_t<KV_FP8, 64>(a, lds, st);
    if (d == 128) return launch_snap_t<KV_FP8, 128>(a, lds, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvs
