// hf_reduce.h -- second pass of the absorb: S[h] += sum_s partial[h][s] (and z),
// splits added in order, and the bf16 hi/lo split of the new S (gfx950).
//
// Shared by the absorb_reduce kernel and by the kernel that runs it next to the
// top-K selection in one launch (the two read and write different buffers).
// The sums are those of the absorb of evicted tokens into the linear state (the
// gist.science English summary "Long-Horizon Streaming Video Generation via
// Hybrid Attention with Decoupled Distillation", 2.A.1).
#pragma once

#include "hf_device.h"

namespace hf {

constexpr int RED_THREADS = 256;

// Floats per partial: the head's full state (D x D, value-major) and z (D).
template <int D>
constexpr int part_floats() { return D * D + D; }

// Groups of RED_THREADS threads per head of the reduce.
template <int D>
constexpr int red_groups() { return (part_floats<D>() / 4 + RED_THREADS - 1) / RED_THREADS; }

// hi = bf16(x), lo = bf16(x - hi) for 4 values, packed little-endian.
__device__ __forceinline__ void split4(const float4 x, uint2& hi, uint2& lo) {
  const float v[4] = {x.x, x.y, x.z, x.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = f32_to_bf16_bits(v[e]);
    l[e] = f32_to_bf16_bits(v[e] - bf16_to_f32(h[e]));
  }
  hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

template <int D>
__device__ __forceinline__ void store_split(uint16_t* s_split, int h, int e4, float4 x) {
  uint2 hi, lo;
  split4(x, hi, lo);
  uint16_t* dst = s_split + (size_t)h * 2 * D * D + e4;
  *reinterpret_cast<uint2*>(dst) = hi;
  *reinterpret_cast<uint2*>(dst + D * D) = lo;
}

// Group `grp` of head h (RED_THREADS threads, thread tid): each thread owns 4 consecutive
// floats of the partial layout; the loads of a group of 4 splits are issued
// together, then added in split order.
template <int D>
__device__ __forceinline__ void absorb_reduce_group(int grp, int h,
                                                    const float* __restrict__ partials,
                                                    int n_split, float* __restrict__ S,
                                                    float* __restrict__ z,
                                                    uint16_t* __restrict__ s_split,
                                                    int tid) {
  constexpr int P = part_floats<D>();
  const int e4 = (grp * RED_THREADS + tid) * 4;
  if (e4 >= P) return;
  const float* p = partials + (size_t)h * n_split * P + e4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = 0;
  for (; s + 4 <= n_split; s += 4) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(p + (size_t)(s + u) * P);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc.x += x[u].x;
      acc.y += x[u].y;
      acc.z += x[u].z;
      acc.w += x[u].w;
    }
  }
  for (; s < n_split; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(p + (size_t)s * P);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  float* dst = e4 < D * D ? S + (size_t)h * D * D + e4 : z + (size_t)h * D + (e4 - D * D);
  float4 o = *reinterpret_cast<float4*>(dst);
  o.x += acc.x;
  o.y += acc.y;
  o.z += acc.z;
  o.w += acc.w;
  *reinterpret_cast<float4*>(dst) = o;
  if (s_split && e4 < D * D) store_split<D>(s_split, h, e4, o);
}

}  // namespace hf
