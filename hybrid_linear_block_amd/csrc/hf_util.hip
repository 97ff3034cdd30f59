// hf_util.hip -- small device utilities of libhf.
#include <math.h>

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

// Per head (blockIdx.y) and tensor (blockIdx.z: 0 = K, 1 = V), copy n16 16-byte
// words from src + head * hs16 to dst + head * hs16; source and destination do not
// overlap.
__global__ void __launch_bounds__(256)
    copy_rows_kv(const uint4* __restrict__ k_src, const uint4* __restrict__ v_src,
                 uint4* __restrict__ k_dst, uint4* __restrict__ v_dst, int64_t n16, int64_t hs16) {
  const int64_t off = (int64_t)blockIdx.y * hs16;
  const uint4* src = (blockIdx.z ? v_src : k_src) + off;
  uint4* dst = (blockIdx.z ? v_dst : k_dst) + off;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

// Angle table of the relative temporal rotation: entry (p, i) = cos and sin of
// p * base^(-i / half), computed in double precision and rounded once to fp32.
__global__ void rope_table(float2* cs, int npos, int half, double ln_base) {
  const int64_t n = (int64_t)npos * half;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int pos = (int)(x / half), i = (int)(x % half);
    const double ang = (double)pos * exp(-ln_base * (double)i / (double)half);
    cs[x] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

}  // namespace

hipError_t launch_rope_table(float2* cs, int npos, int half, double theta_base,
                             hipStream_t stream) {
  const int64_t n = (int64_t)npos * half;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  rope_table<<<(unsigned)blocks, 256, 0, stream>>>(cs, npos, half, log(theta_base));
  return hipGetLastError();
}

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

hipError_t launch_copy_rows_kv(const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                               int heads, size_t bytes_per_head, size_t head_stride_bytes,
                               hipStream_t stream) {
  if (bytes_per_head == 0 || heads < 1) return hipSuccess;
  const int64_t n16 = (int64_t)(bytes_per_head / 16);
  int64_t bx = (n16 + 255) / 256;
  const int64_t cap = 4096 / (2 * heads) > 0 ? 4096 / (2 * heads) : 1;  // ~4096 workgroups
  if (bx > cap) bx = cap;
  copy_rows_kv<<<dim3((unsigned)bx, (unsigned)heads, 2), 256, 0, stream>>>(
      static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
      static_cast<uint4*>(k_dst), static_cast<uint4*>(v_dst), n16,
      (int64_t)(head_stride_bytes / 16));
  return hipGetLastError();
}

}  // namespace hf
