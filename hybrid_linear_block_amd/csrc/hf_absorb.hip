// hf_absorb.hip -- fold evicted tokens into the linear state (gfx950).
//
// Per head: S[j][i] += sum_n V[n][j] phi(K[n][i]) and z[i] += sum_n phi(K[n][i]),
// the incremental absorption of evicted tokens into a compact key-value state
// described in the authors' abstract (fugumt.com listing of arXiv 2604.10103v1)
// and in the gist.science English summary "Long-Horizon Streaming Video
// Generation via Hybrid Attention with Decoupled Distillation", 2.A.1.
//
// Work split: one workgroup per (head, token split) forms the partial state of
// its tokens for the whole head and writes it to the workspace; a second kernel
// adds the partials to S and z in split order. No atomics or device-wide fences
// are involved (on a chip whose XCDs have separate L2 caches those would have to
// write the L2 back), and the order of every sum is fixed, so the result is
// bitwise reproducible.
//
// The workgroup bodies are in hf_absorb_parts.h.
#include <atomic>

#include "hf_absorb_parts.h"
#include "hf_device.h"
#include "hf_launch.h"
#include "hf_reduce.h"

namespace hf {

namespace {

// Second pass (absorb_reduce_group, shared with the selection launch).
template <int D>
__global__ __launch_bounds__(RED_THREADS) void absorb_reduce(const float* __restrict__ partials,
                                                             int n_split, float* __restrict__ S,
                                                             float* __restrict__ z,
                                                             uint16_t* __restrict__ s_split) {
  absorb_reduce_group<D>(blockIdx.x, blockIdx.y, partials, n_split, S, z, s_split, threadIdx.x);
}

template <int D>
__global__ __launch_bounds__(RED_THREADS) void split_state(const float* __restrict__ S,
                                                           uint16_t* __restrict__ s_split) {
  const int e4 = (blockIdx.x * RED_THREADS + threadIdx.x) * 4, h = blockIdx.y;
  if (e4 >= D * D) return;
  store_split<D>(s_split, h, e4, *reinterpret_cast<const float4*>(S + (size_t)h * D * D + e4));
}

template <typename T, int D>
__global__ __launch_bounds__((absorb::threads<T, D>())) void absorb_parts(
    const T* __restrict__ kev, const T* __restrict__ vev, int64_t n_ev, int64_t hs, int tps,
    int n_split, float* __restrict__ partials) {
  absorb::item<T, D>(blockIdx.x, n_split, kev, vev, n_ev, hs, tps, partials);
}

}  // namespace

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

AbsorbPlan absorb_plan(int dtype, int heads, int d, int64_t n_ev) {
  AbsorbPlan p;
  int64_t per;
  if (dtype == 0) {
    // bf16: as many splits as fill every compute unit once (the kernel's LDS ring
    // admits one workgroup per unit at d = 128, three at d = 64), at most the maximum,
    // in whole 32-token tiles.
    const int per_cu = d == 128 ? 1 : 3;
    int target = per_cu * device_cu_count() / (heads > 0 ? heads : 1);
    if (target > kAbsorbMaxSplits) target = kAbsorbMaxSplits;
    if (target < 1) target = 1;
    per = (n_ev + target - 1) / target;
    if (per < 128) per = 128;
    per = (per + absorb::BT - 1) / absorb::BT * absorb::BT;
  } else {
    per = (n_ev + kAbsorbMaxSplits - 1) / kAbsorbMaxSplits;
    if (per < 128) per = 128;
    per = (per + absorb::TS - 1) / absorb::TS * absorb::TS;  // whole fp32 token tiles
  }
  p.tokens_per_split = (int)per;
  p.n_split = (int)((n_ev + per - 1) / per);
  if (p.n_split < 1) p.n_split = 1;
  return p;
}

size_t absorb_partial_floats(int heads, int d) {
  return (size_t)heads * kAbsorbMaxSplits * (size_t)(d * d + d);
}

int absorb_items(int dtype, int heads, int d, const AbsorbPlan& p) {
  const int per = dtype == 0 ? 1 : (d / absorb::AT) * (d / absorb::AT);
  return p.n_split * per * heads;
}

hipError_t launch_absorb_parts(int dtype, int heads, int d, const void* k, const void* v,
                               int64_t n_ev, int64_t head_stride, float* partials,
                               hipStream_t stream) {
  const AbsorbPlan p = absorb_plan(dtype, heads, d, n_ev);
  const int items = absorb_items(dtype, heads, d, p);
#define HF_ABS(T, D)                                                                        \
  absorb_parts<T, D><<<items, absorb::threads<T, D>(), 0, stream>>>(                        \
      static_cast<const T*>(k), static_cast<const T*>(v), n_ev, head_stride,                \
      p.tokens_per_split, p.n_split, partials)
  if (dtype == 0) {
    if (d == 128) HF_ABS(bf16_t, 128); else HF_ABS(bf16_t, 64);
  } else {
    if (d == 128) HF_ABS(float, 128); else HF_ABS(float, 64);
  }
#undef HF_ABS
  return hipGetLastError();
}

hipError_t launch_absorb_reduce(int dtype, int heads, int d, int64_t n_ev, const float* partials,
                                float* S, float* z, uint16_t* s_split, hipStream_t stream) {
  const AbsorbPlan p = absorb_plan(dtype, heads, d, n_ev);
#define HF_RED(D)                                                                   \
  absorb_reduce<D><<<dim3((part_floats<D>() / 4 + RED_THREADS - 1) / RED_THREADS, heads), \
                     RED_THREADS, 0, stream>>>(partials, p.n_split, S, z, s_split)
  if (d == 128) HF_RED(128); else HF_RED(64);
#undef HF_RED
  return hipGetLastError();
}

hipError_t launch_absorb(int dtype, int heads, int d, const void* k, const void* v, int64_t n_ev,
                         int64_t head_stride, float* S, float* z, float* partials,
                         uint16_t* s_split, hipStream_t stream) {
  hipError_t e = launch_absorb_parts(dtype, heads, d, k, v, n_ev, head_stride, partials, stream);
  if (e != hipSuccess) return e;
  return launch_absorb_reduce(dtype, heads, d, n_ev, partials, S, z, s_split, stream);
}

hipError_t launch_split_state(int heads, int d, const float* S, uint16_t* s_split,
                              hipStream_t stream) {
  const int blocks = (d * d / 4 + RED_THREADS - 1) / RED_THREADS;
  if (d == 128)
    split_state<128><<<dim3(blocks, heads), RED_THREADS, 0, stream>>>(S, s_split);
  else
    split_state<64><<<dim3(blocks, heads), RED_THREADS, 0, stream>>>(S, s_split);
  return hipGetLastError();
}

}  // namespace hf
