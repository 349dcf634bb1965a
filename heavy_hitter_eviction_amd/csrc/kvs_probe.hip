// Streaming-read ceiling of the GPU, measured with the decode kernel's own
// kind of load: every 16-byte piece of a buffer is read once with a
// non-temporal raw buffer load, one instruction covering 1 KiB of
// consecutive bytes across a wave's 64 lanes, eight waves per workgroup.
// Every loaded dword is added into a per-thread sum and each workgroup stores
// the sum of its threads, so no load can be dropped by the compiler (an
// exclusive-or fold of repeated loads can be).
//
// Workgroup w reads the w-th of `workgroups` equal slices (whole KiB runs;
// the last takes the remainder); inside a slice, wave v reads runs v, v + 8,
// ..., eight runs in flight per wave.

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

constexpr int kProbeWaves = 8;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(64 * kProbeWaves, 1) void kvs_stream_read(const uint8_t* buf, uint64_t runs,
                                                                        uint32_t* sums) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t per = runs / gridDim.x;
  const uint64_t r0 = per * blockIdx.x;
  const uint64_t n = blockIdx.x == gridDim.x - 1 ? runs - r0 : per;
  uint32_t acc = 0;
  // one buffer resource per 1 GiB window of the slice: 32-bit offsets
  for (uint64_t w0 = 0; w0 < n; w0 += (1u << 20)) {
    const uint32_t wn = (uint32_t)((n - w0) < (1u << 20) ? (n - w0) : (1u << 20));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf + (r0 + w0) * 1024), (short)0, (int)(wn * 1024u),
                                          0x00020000);
    uint32_t k = (uint32_t)wave;
    for (; k + (kProbeUnroll - 1) * kProbeWaves < wn; k += kProbeUnroll * kProbeWaves) {
      u32x4 v[kProbeUnroll];
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u)
        v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, (int)(16 * lane), (int)((k + u * kProbeWaves) * 1024u), 2));
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u) acc += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
    }
    for (; k < wn; k += kProbeWaves) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(16 * lane),
                                                                                    (int)(k * 1024u), 2));
      acc += (v[0] + v[1]) + (v[2] + v[3]);
    }
  }
  for (int off = 32; off > 0; off >>= 1) acc += (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t part[kProbeWaves];
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kProbeWaves; ++w) s += part[w];
    sums[blockIdx.x] = s;
  }
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sums, int workgroups, hipStream_t st) {
  hipLaunchKernelGGL(kvs_stream_read, dim3(workgroups), dim3(64 * kProbeWaves), 0, st, (const uint8_t*)buf,
                     (uint64_t)(bytes / 1024), sums);
  return hipGetLastError();
}

}  // namespace kvs
