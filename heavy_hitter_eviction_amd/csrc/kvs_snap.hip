// SnapKV-style prefill scoring (Context views at marginal cost, section 3,
// Fact 1: one-shot at the end of prefill, the attention of the last N prompt
// queries -- the observation window -- is pooled into one score per prompt
// token per head, then max-pooled with kernel 7 so that a kept key drags its
// neighbours), placed per 16-token block (Per-Head Attention as a Scoring
// Signal: score per head, place per block).
//
// Column n of a (KV head, sequence) is (window query w, head h of the group),
// n = w*G + h; query w sits at position n_prompt - W + w and reads keys at or
// before it. Two passes over K (V is not needed):
//   kvs_snap_pass<.., 0>: per partition of tiles, each column's running max and
//     sum of exponentials (S^T = K Q^T on MFMA, 16 columns per block);
//   kvs_snap_merge: exact per-column max M and sum L over the partitions;
//   kvs_snap_pass<.., 1>: p = 2^(s - M) / L, summed over the window's queries
//     per (token, head): token_score[b][h][token];
//   kvs_snap_pool: per head, max over tokens j-R .. j+R (R = kernel/2) inside
//     the prompt, summed over the block's tokens and over heads in ascending
//     order, added to block_score[b][block].

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

}  // namespace

template <int KV, int D, int PASS>
__global__ __launch_bounds__(256) void kvs_snap_pass(SnapArgs a) {
  constexpr int eb = KV == KV_FP8 ? 1 : 2;
  constexpr int NCH = D * eb / 64;   // 16-byte K chunks per lane per tile
  constexpr int NC32 = D / 32;       // MFMA contraction chunks
  extern __shared__ float lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kg = lane >> 4;
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G, W = a.W, NCOL = W * G, NCB = (NCOL + 15) / 16;
  bf16x8* qfrag = (bf16x8*)lds;                              // [NCB][NC32][64]
  float* colM = (float*)(qfrag + NCB * NC32 * 64);           // [NCOL]
  float* colIL = colM + kSnapMaxCB * 16;                     // [NCOL] 1 / L
  float* wm = colIL + kSnapMaxCB * 16;                       // [4 waves][NCOL]
  float* wl = wm + 4 * kSnapMaxCB * 16;                      // [4 waves][NCOL]

  // window queries as B fragments (zeros for padding columns)
  for (int x = tid; x < NCB * NC32 * 64; x += 256) {
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
    for (int n = tid; n < NCOL; n += 256) {
      const size_t ci = ((size_t)b * a.Hkv + g) * NCOL + n;
      colM[n] = a.col_m[ci];
      const float L = a.col_l[ci];
      colIL[n] = L > 0.0f ? 1.0f / L : 0.0f;
    }
  }
  __syncthreads();

  const int npr = min(max(a.n_prompt[b], 0), a.C);
  const int te = max(0, min(a.NT, (npr + kTile - 1) / kTile));
  const int t0 = min(te, part * a.tpp), t1 = min(te, t0 + a.tpp);
  const size_t region = (size_t)a.C * D * eb;
  const char* kbase = (const char*)a.k + ((size_t)b * a.Hkv + g) * region;
  const float* ksb = a.ks ? a.ks + (size_t)b * a.C : nullptr;

  float m_run[kSnapMaxCB], l_run[kSnapMaxCB];
#pragma unroll
  for (int cb = 0; cb < kSnapMaxCB; ++cb) {
    m_run[cb] = -__builtin_inff();
    l_run[cb] = 0.0f;
  }
  // one tile of prefetch: the next tile's K (and FP8 scales) load while this
  // one is processed; past the end the load reads the current tile again
  auto load_k = [&](u32x4* kc, f32x4& ks, int t) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) kc[i] = *(const u32x4*)(kbase + (size_t)t * kTile * D * eb + 1024 * i + 16 * lane);
    if constexpr (KV == KV_FP8) ks = *(const f32x4*)(ksb + (size_t)t * kTile + 4 * kg);
  };
  u32x4 kn[NCH];
  f32x4 ksn = {1.f, 1.f, 1.f, 1.f};
  if (t0 + wave < t1) load_k(kn, ksn, t0 + wave);
  for (int t = t0 + wave; t < t1; t += 4) {
    u32x4 kc[NCH];
    f32x4 ks = ksn;
#pragma unroll
    for (int i = 0; i < NCH; ++i) kc[i] = kn[i];
    load_k(kn, ksn, t + 4 < t1 ? t + 4 : t);
    // a tile before the first window query's position is read by every column
    const bool all_read = t * kTile + kTile - 1 < npr - W && NCOL % 16 == 0;
    bf16x8 kk[NC32];
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
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = t * kTile + 4 * kg + r;
        const bool valid = all_read || (n < NCOL && p <= qpos && p < npr);
        x[r] = valid ? s[r] * (ks[r] * a.scale_log2) : -__builtin_inff();
      }
      if constexpr (PASS == 0) {
        const float mx = rows_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float m_new = fmaxf(m_run[cb], mx);
        if (m_new != -__builtin_inff()) {
          float e = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) e += fast_exp2(x[r] - m_new);
          l_run[cb] = l_run[cb] * fast_exp2(m_run[cb] - m_new) + rows_sum(e);
          m_run[cb] = m_new;
        }
      } else {
        float pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pw[r] = x[r] == -__builtin_inff() ? 0.0f : fast_exp2(x[r] - colM[min(n, NCOL - 1)]) * colIL[min(n, NCOL - 1)];
        // sum over the window's queries: columns of one head are the lanes
        // j, j + G, j + 2G, ... of each 16-lane row
        for (int off = G; off < 16; off <<= 1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) pw[r] += __shfl_xor(pw[r], off, 64);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += pw[r];
      }
    }
    if constexpr (PASS == 1) {
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
    // merge the four waves, then one (max, sum) per column for this partition
    if (kg == 0) {
#pragma unroll
      for (int cb = 0; cb < kSnapMaxCB; ++cb) {
        if (cb >= NCB) break;
        const int n = cb * 16 + j;
        if (n < NCOL) {
          wm[wave * kSnapMaxCB * 16 + n] = m_run[cb];
          wl[wave * kSnapMaxCB * 16 + n] = l_run[cb];
        }
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

// grid (ceil(C / 1024), B): a workgroup pools 1024 tokens (64 blocks) of one
// sequence. For each head in ascending order it stages the tokens and the R on
// either side in LDS, takes each token's windowed max, and adds the block's
// 16 pooled values into its running sum.
constexpr int kPoolTokens = 1024;
constexpr int kPoolMaxR = 16;
__global__ __launch_bounds__(256) void kvs_snap_pool(SnapArgs a) {
  __shared__ float row[kPoolTokens + 2 * kPoolMaxR];
  __shared__ float part[kPoolTokens / kTile][kTile / 4];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int npr = min(max(a.n_prompt[b], 0), a.C);
  const int lo = blockIdx.x * kPoolTokens;
  if (lo >= npr) return;
  const int R = a.pool / 2;
  const int blk_local = tid >> 2, q = tid & 3;   // 64 blocks x 4 quarters of 4 tokens
  float sum = 0.0f;
  for (int h = 0; h < a.Hq; ++h) {
    const float* sc = a.token_score + ((size_t)b * a.Hq + h) * a.C;
    __syncthreads();
    for (int x = tid; x < kPoolTokens + 2 * R; x += 256) {
      const int tok = lo - R + x;
      row[x] = (tok >= 0 && tok < npr) ? sc[tok] : -__builtin_inff();
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tl = blk_local * kTile + q * 4 + u;          // token within the chunk
      if (lo + tl < npr) {
        float m = -__builtin_inff();
        for (int k = 0; k <= 2 * R; ++k) m = fmaxf(m, row[tl + k]);
        sum += m;
      }
    }
  }
  part[blk_local][q] = sum;
  __syncthreads();
  if (q == 0) {
    const int blk = blockIdx.x * (kPoolTokens / kTile) + blk_local;
    if (blk < a.nbmax && blk * kTile < npr)
      a.block_score[(size_t)b * a.nbmax + blk] +=
          (part[blk_local][0] + part[blk_local][1]) + (part[blk_local][2] + part[blk_local][3]);
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
    hipLaunchKernelGGL(kvs_snap_pool, dim3((a.C + kPoolTokens - 1) / kPoolTokens, a.B), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_snap(int kv, int d, const SnapArgs& a, hipStream_t st) {
  const int ncb = (a.W * a.G + 15) / 16;
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
