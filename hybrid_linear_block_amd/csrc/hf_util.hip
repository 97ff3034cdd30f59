// hf_util.hip -- small device utilities of libhf.
#include "hf_device.h"
#include "hf_launch.h"

namespace hf {

namespace {

// Zero `words` 32-bit words (a plain store kernel rather than a memset node, so
// the clear behaves the same inside captured graphs).
__global__ void fill_zero_words(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ void fill_zero_bytes(uint8_t* p, size_t bytes) {
  const size_t i = threadIdx.x;
  if (i < bytes) p[i] = 0u;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const size_t words = bytes / 4;
  if (words) {
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    fill_zero_words<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<uint32_t*>(p), words);
  }
  if (bytes % 4)
    fill_zero_bytes<<<1, 4, 0, stream>>>(static_cast<uint8_t*>(p) + words * 4, bytes % 4);
  return hipGetLastError();
}

}  // namespace hf
