// Streaming-read probe: reads a device buffer once with 16-byte loads and
// folds it into one word per wave, so that the benchmark can measure the
// HBM read rate this GPU sustains for a plain, well-formed read stream (the
// ceiling the decode kernels' cache reads are compared against besides the
// nominal peak).  Built into its own library, libmla_probe.so; it is not part
// of the libmla ABI.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each thread keeps four 16-byte loads in flight (grid-stride over the
// buffer); the XOR of everything read leaves as one word per wave, so no
// load can be dropped.
__global__ void __launch_bounds__(256) k_stream_read(const u32x4* __restrict__ src, size_t n16,
                                                      uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = v;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from `src` with `blocks` work-groups of 256
// threads; sink receives blocks * 4 words.  Returns 0, or -1 on a bad
// argument or a failed launch.
int mla_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  if (!src || !sink || blocks < 1 || bytes % 16 != 0) return -1;
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, stream, (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
