// FP8 encoding and cache writes.
//
// Encoding follows Context Optimization, "FP8 KV Cache / How It Works": one
// scale per position, scale = absmax / 240 (headroom below the E4M3 maximum of
// 448), every value divided by the scale, clipped and quantised to E4M3 with
// round-to-nearest-even, the scale stored beside the codes.

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

// Workgroup max of non-negative values (256 threads).
__device__ __forceinline__ float block_max256(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Word fill: each thread stores 16 bytes, the tail word by word.
__global__ __launch_bounds__(256) void kvs_fill_u32(uint32_t* dst, size_t n_words, uint32_t value) {
  const size_t n4 = n_words / 4;
  const size_t stride = (size_t)gridDim.x * 256;
  const u32x4 v = {value, value, value, value};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) ((u32x4*)dst)[i] = v;
  const size_t t = 4 * n4 + (size_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n_words) dst[t] = value;
}

hipError_t launch_fill_u32(uint32_t* dst, size_t n_words, uint32_t value, hipStream_t st) {
  if (n_words == 0) return hipSuccess;
  const size_t n4 = (n_words + 3) / 4;
  const int blocks = (int)(n4 < (size_t)1024 * 256 ? (n4 + 255) / 256 : 1024);
  hipLaunchKernelGGL(kvs_fill_u32, dim3(blocks), dim3(256), 0, st, dst, n_words, value);
  return hipGetLastError();
}

// One workgroup per row.
__global__ __launch_bounds__(256) void kvs_encode_rows(const void* src, int src_bf16, int row_len,
                                                        uint8_t* codes, float* scales) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  const size_t base = row * (size_t)row_len;
  float m = 0.0f;
  for (int i = threadIdx.x; i < row_len; i += 256) m = fmaxf(m, fabsf(load_src(src, base + i, src_bf16)));
  m = block_max256(m, red);
  const float s = fp8_scale_of(m);
  if (threadIdx.x == 0) scales[row] = s;
  for (int i = threadIdx.x; i < row_len; i += 256)
    codes[base + i] = (uint8_t)encode_with_scale(load_src(src, base + i, src_bf16), s);
}

hipError_t launch_encode_fp8(const void* src, int src_bf16, int64_t n_rows, int row_len,
                             uint8_t* codes, float* scales, hipStream_t st) {
  const int64_t kMaxGrid = 1 << 30;
  for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxGrid) {
    const int64_t n = n_rows - r0 < kMaxGrid ? n_rows - r0 : kMaxGrid;
    const size_t off = (size_t)r0 * row_len;
    const void* s = (const char*)src + off * (src_bf16 ? 2 : 4);
    hipLaunchKernelGGL(kvs_encode_rows, dim3((unsigned)n), dim3(256), 0, st, s, src_bf16, row_len,
                       codes + off, scales + r0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One workgroup per appended row: K and V of every KV head of one position,
// written into the fragment-major tile layout (k_tile_offset / v_tile_offset).
template <int KV>
__global__ __launch_bounds__(256) void kvs_append_rows(AppendArgs a) {
  __shared__ float red[4];
  constexpr int eb = KV == KV_F32 ? 4 : KV == KV_BF16 ? 2 : 1;
  const int r = blockIdx.x;
  const int seq = a.row_seq[r];
  const int pos = a.row_pos[r];
  if (seq < 0 || seq >= a.B || pos < 0 || (!a.ring && pos >= a.C)) return;
  const int slot = a.ring ? pos % a.C : pos;
  const int n = a.Hkv * a.D;
  const size_t rb = (size_t)r * n;
  float sk = 0.0f, sv = 0.0f;
  if constexpr (KV == KV_FP8) {
    float mk = 0.0f, mv = 0.0f;
    for (int i = threadIdx.x; i < n; i += 256) {
      mk = fmaxf(mk, fabsf(load_src(a.k_rows, rb + i, a.src_bf16)));
      mv = fmaxf(mv, fabsf(load_src(a.v_rows, rb + i, a.src_bf16)));
    }
    sk = fp8_scale_of(block_max256(mk, red));
    sv = fp8_scale_of(block_max256(mv, red));
    if (threadIdx.x == 0) {
      a.k_scale[(size_t)seq * a.C + slot] = sk;
      a.v_scale[(size_t)seq * a.C + slot] = sv;
    }
  }
  if (a.ring && threadIdx.x == 0) a.pos_of_slot[(size_t)seq * a.C + slot] = pos;
  const int tile = slot >> 4, t = slot & 15;
  const size_t tile_bytes = (size_t)kTile * a.D * eb;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int g = i / a.D, dim = i - g * a.D;
    const size_t base = (((size_t)seq * a.Hkv + g) * (a.C >> 4) + tile) * tile_bytes;
    char* kp = (char*)a.k_cache + base + k_tile_offset(t, dim, eb);
    char* vp = (char*)a.v_cache + base + v_tile_offset(t, dim, a.D, eb);
    if constexpr (KV == KV_FP8) {
      *(uint8_t*)kp = (uint8_t)encode_with_scale(load_src(a.k_rows, rb + i, a.src_bf16), sk);
      *(uint8_t*)vp = (uint8_t)encode_with_scale(load_src(a.v_rows, rb + i, a.src_bf16), sv);
    } else if constexpr (KV == KV_BF16) {
      *(uint16_t*)kp = ((const uint16_t*)a.k_rows)[rb + i];
      *(uint16_t*)vp = ((const uint16_t*)a.v_rows)[rb + i];
    } else {
      *(float*)kp = ((const float*)a.k_rows)[rb + i];
      *(float*)vp = ((const float*)a.v_rows)[rb + i];
    }
  }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.n_rows <= 0) return hipSuccess;
  dim3 grid(a.n_rows), block(256);
  if (a.kv == KV_FP8) hipLaunchKernelGGL(kvs_append_rows<KV_FP8>, grid, block, 0, st, a);
  else if (a.kv == KV_BF16) hipLaunchKernelGGL(kvs_append_rows<KV_BF16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(kvs_append_rows<KV_F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kvs
