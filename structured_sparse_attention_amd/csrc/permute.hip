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

// One head: dst rows r in [0, N), chunks of 16 bytes, grid-stride.
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst,
                                                      int32_t F, int32_t S,
                                                      int32_t chunks, int32_t mode) {
  const int64_t N = (int64_t)F * S;
  const int64_t total = N * chunks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i % chunks;
    const int64_t r = i / chunks;  // destination row
    int64_t sr = r;
    if (mode == 1) {               // to spatial-major: destination p = s*F + f
      const int64_t s = r / F, f = r % F;
      sr = f * S + s;
    } else if (mode == 2) {        // back to frame-major: destination t = f*S + s
      const int64_t f = r / S, s = r % S;
      sr = s * F + f;
    }
    dst[r * chunks + c] = src[sr * chunks + c];
  }
}

}  // namespace

hipError_t launch_permute_tokens(const void* src, void* dst, int32_t F, int32_t S,
                                 int32_t H, int32_t D, const int32_t* kinds,
                                 int32_t direction, hipStream_t stream) {
  const int32_t chunks = D / 8;
  const int64_t per_head = (int64_t)F * S * chunks;
  const int64_t blocks = std::min<int64_t>((per_head + 255) / 256, 32768);
  for (int32_t h = 0; h < H; ++h) {
    int32_t mode = 0;
    if (kinds[h] == SVG_HEAD_TEMPORAL) mode = direction == SVG_TO_KERNEL_LAYOUT ? 1 : 2;
    const uint4* s = (const uint4*)src + (int64_t)h * per_head;
    uint4* d = (uint4*)dst + (int64_t)h * per_head;
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       s, d, F, S, chunks, mode);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace svg
