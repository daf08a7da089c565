// Token re-ordering between the original frame-major order t = f*S + s and a
// head's kernel layout. Temporal heads use the spatial-major order
// p = s*F + f so that a narrow spatial band is one contiguous run of rows
// (the head kinds need different token orders, Newsbite "Interesting
// facts"); other heads keep p = t. HBM-bound: every 16-byte chunk is read
// once and written once, consecutive threads touch consecutive chunks of a
// destination row.
#include "svg_internal.hpp"

namespace svg {
namespace {

// Heads [h0, h0 + gridDim.y) of one mode. Destination rows in [0, N) of a
// head, chunks of 16 bytes, grid-stride over the head. A head is under
// 2 GiB, so chunk indices fit in 32 bits.
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst, int32_t F,
                                                      int32_t S, int32_t chunks, int32_t mode) {
  const int32_t total = F * S * chunks;
  const size_t head = (size_t)blockIdx.y * (size_t)total;
  const uint4* s_h = src + head;
  uint4* d_h = dst + head;
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += gridDim.x * blockDim.x) {
    const int32_t r = i / chunks;  // destination row
    const int32_t c = i - r * chunks;
    int32_t sr = r;
    if (mode == 1) {  // to spatial-major: destination p = s*F + f
      const int32_t s = r / F;
      sr = (r - s * F) * S + s;
    } else if (mode == 2) {  // back to frame-major: destination t = f*S + s
      const int32_t f = r / S;
      sr = (r - f * S) * F + f;
    }
    d_h[i] = s_h[sr * chunks + c];
  }
}

}  // namespace

hipError_t launch_permute_tokens(const void* src, void* dst, int32_t F, int32_t S,
                                 int32_t H, int32_t D, const int32_t* kinds,
                                 int32_t direction, hipStream_t stream) {
  const int32_t chunks = D / 8;
  const int64_t per_head = (int64_t)F * S * chunks;
  auto mode_of = [&](int32_t h) {
    return kinds[h] == SVG_HEAD_TEMPORAL ? (direction == SVG_TO_KERNEL_LAYOUT ? 1 : 2) : 0;
  };
  // one launch per run of consecutive heads with the same mode
  for (int32_t h0 = 0; h0 < H;) {
    const int32_t mode = mode_of(h0);
    int32_t h1 = h0 + 1;
    while (h1 < H && mode_of(h1) == mode && h1 - h0 < 65535) ++h1;
    // about 16,384 blocks per launch (64 per CU on a 256-CU part), at most
    // one per 256 chunks: fewer blocks left HBM bandwidth unused (5.26 TB/s
    // with 4,096 against 5.50 with 16,384 on the main workload)
    const int64_t want = (16384 + (h1 - h0) - 1) / (h1 - h0);  // blocks per head
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((per_head + 255) / 256, want));
    const uint4* s = (const uint4*)src + (int64_t)h0 * per_head;
    uint4* d = (uint4*)dst + (int64_t)h0 * per_head;
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks, (unsigned)(h1 - h0)), dim3(256), 0,
                       stream, s, d, F, S, chunks, mode);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    h0 = h1;
  }
  return hipSuccess;
}

}  // namespace svg
