// Read-bandwidth probe (measurement only, built into libl3probe.so apart
// from the library): streams a device buffer and reports nothing but time,
// so that the gather's rate can be set against what plain reads of the same
// kind reach on the device it runs on.
//
//   int l3probe_read(const void* buf, int64_t bytes, int pattern, int grid,
//                    void* sink, hipStream_t stream)
//
// buf: device buffer of `bytes` bytes, a multiple of 65536 (64 KiB blocks);
// sink: one device float, written only if an impossible checksum turns up
// (it keeps the loads alive). Patterns:
//   0: 1 KiB contiguous per wave instruction, ordinary loads;
//   1: the gather's score-operand pattern: each 64 KiB block taken as 16
//      rows of 4 KiB, every wave instruction reading 64 bytes from each of
//      the 16 rows (lane l: row l % 16, 16-byte piece l / 16), the rows
//      walked in 64-byte steps, ordinary loads;
//   2: as 0 with non-temporal (streaming) loads;
//   3: as 1 with non-temporal loads (the two 64-byte halves of a row's
//      128-byte line read by consecutive instructions);
//   4: as 3 with the halves four instructions apart (of each eight loads
//      in flight, the first halves of four lines, then their second halves).
// Returns 0, or -1 for a bad pattern or size, or the HIP error code of the
// launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 65536;
constexpr int kDepth = 8;  // loads in flight per lane

template <int PATTERN>
__global__ __launch_bounds__(256) void read_probe_kernel(
    const uint8_t* __restrict__ buf, int64_t nblocks, float* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
  // lane's first byte within a block and the stride of its successive loads
  constexpr bool rows16 = PATTERN == 1 || PATTERN >= 3;
  constexpr bool nt = PATTERN >= 2;
  const int first = rows16 ? (lane & 15) * 4096 + (lane >> 4) * 16 : lane * 16;
  const int step = rows16 ? 64 : 1024;
  unsigned mix = 0;
  for (int64_t b = wave; b < nblocks; b += waves) {
    const uint8_t* p = buf + b * kBlock + first;
    for (int i = 0; i < 64; i += kDepth) {
      u32x4 v[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        // pattern 4: steps 0, 2, 4, 6, 1, 3, 5, 7 of the eight
        const int su = PATTERN == 4 ? (u & 3) * 2 + (u >> 2) : u;
        const u32x4* q = reinterpret_cast<const u32x4*>(p + (i + su) * step);
        v[u] = nt ? __builtin_nontemporal_load(q) : *q;
      }
#pragma unroll
      for (int u = 0; u < kDepth; ++u) mix += v[u].x ^ v[u].w;
    }
  }
  if (mix == 0x9e3779b9u) sink[0] = 1.0f;
}

}  // namespace

extern "C" int l3probe_read(const void* buf, int64_t bytes, int pattern,
                            int grid, void* sink, hipStream_t stream) {
  if (bytes <= 0 || bytes % kBlock != 0 || grid <= 0) return -1;
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  float* s = static_cast<float*>(sink);
  const int64_t nb = bytes / kBlock;
  switch (pattern) {
    case 0: read_probe_kernel<0><<<grid, 256, 0, stream>>>(p, nb, s); break;
    case 1: read_probe_kernel<1><<<grid, 256, 0, stream>>>(p, nb, s); break;
    case 2: read_probe_kernel<2><<<grid, 256, 0, stream>>>(p, nb, s); break;
    case 3: read_probe_kernel<3><<<grid, 256, 0, stream>>>(p, nb, s); break;
    case 4: read_probe_kernel<4><<<grid, 256, 0, stream>>>(p, nb, s); break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}
