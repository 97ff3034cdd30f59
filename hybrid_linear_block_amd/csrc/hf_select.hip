// hf_select.hip -- block importance scores and top-K key-block selection (gfx950).
//
// The sparse path keeps, for every query block, only the key blocks with the
// highest block importance score (gist.science English summary "Long-Horizon
// Streaming Video Generation via Hybrid Attention with Decoupled Distillation",
// 2.A.2 "Block-Sparse Sliding Window Attention"). The importance of key block j
// for query block i is tau * mean(Q rows of i) . mean(K rows of j), in fp32.
//
// block_pool  (HBM-bound): one workgroup per (block, head) streams the block's
//             rows once with 16-byte coalesced loads and writes the fp32 row mean.
// score_select (latency-bound): one workgroup per (query block, head) forms the
//             block's scores against all key blocks, then selects the top_k by
//             exact rank counting on a unique order-preserving key (score bits,
//             then lower index first) and compacts the kept indices in ascending
//             order with wave ballots. Ties therefore go to the lower index, and
//             -0.0 counts as +0.0.
#include "hf_device.h"
#include "hf_launch.h"

namespace hf {

namespace {

constexpr int POOL_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(POOL_THREADS) void block_pool(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ k, int64_t n_kv,
    int64_t kv_hs, int block, int nqb, float* __restrict__ pooled_q,
    float* __restrict__ pooled_k, int nqb_cap, int nkb_cap) {
  constexpr int VEC = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int CPR = D / VEC;           // chunks per row
  constexpr int RPP = POOL_THREADS / CPR;  // rows per pass
  __shared__ float red[RPP][D];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const bool is_q = b < nqb;
  const int blk = is_q ? b : b - nqb;
  const int64_t n = is_q ? n_q : n_kv;
  const T* base = (is_q ? q + (size_t)h * q_hs : k + (size_t)h * kv_hs);
  const int64_t r0 = (int64_t)blk * block;
  const int64_t r1 = r0 + block < n ? r0 + block : n;
  const int cc = tid % CPR, rg = tid / CPR;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int64_t r = r0 + rg; r < r1; r += RPP) {
    const uint4 x = *reinterpret_cast<const uint4*>(base + r * D + cc * VEC);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += bf16_to_f32(half16(x, e));
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += __uint_as_float(word(x, e));
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rg][cc * VEC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int p = 0; p < RPP; ++p) s += red[p][tid];
    const float mean = s / (float)(r1 - r0);
    float* dst = is_q ? pooled_q + ((size_t)h * nqb_cap + blk) * D
                      : pooled_k + ((size_t)h * nkb_cap + blk) * D;
    dst[tid] = mean;
  }
}

constexpr int SEL_THREADS = 256;

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D>
__global__ __launch_bounds__(SEL_THREADS) void score_select(
    const float* __restrict__ pooled_q, const float* __restrict__ pooled_k, int nqb, int nkb,
    int nqb_cap, int nkb_cap, float scale, int top_k, int32_t* __restrict__ sel,
    float* __restrict__ scores_out) {
  __shared__ uint32_t key[kMaxKeyBlocks];
  __shared__ int wave_cnt[SEL_THREADS / 64];
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  // 16 lanes per key block, D/16 consecutive features per lane.
  constexpr int PER = D / 16;
  const int sub = lane & 15, slot = tid >> 4;  // 16 key blocks per pass
  const float* qm = pooled_q + ((size_t)h * nqb_cap + i) * D + sub * PER;
  float qv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) qv[e] = qm[e];
  for (int j0 = 0; j0 < nkb; j0 += SEL_THREADS / 16) {
    const int j = j0 + slot;
    float s = 0.f;
    if (j < nkb) {
      const float* km = pooled_k + ((size_t)h * nkb_cap + j) * D + sub * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) s += qv[e] * km[e];
    }
    // Fixed-order butterfly over the 16 lanes of this key block.
    s += __shfl_xor(s, 8, 16);
    s += __shfl_xor(s, 4, 16);
    s += __shfl_xor(s, 2, 16);
    s += __shfl_xor(s, 1, 16);
    if (j < nkb && sub == 0) {
      const float sc = s * scale;
      key[j] = score_key(sc);
      if (scores_out) scores_out[((size_t)h * nqb + i) * nkb + j] = sc;
    }
  }
  __syncthreads();
  if (!sel) return;
  int32_t* out = sel + ((size_t)h * nqb + i) * top_k;
  int base = 0;  // kept blocks with a lower index than this pass
  for (int j0 = 0; j0 < nkb; j0 += SEL_THREADS) {
    const int j = j0 + tid;
    bool keep = false;
    if (j < nkb) {
      const uint32_t kj = key[j];
      int rank = 0;  // blocks ranked strictly before j
      for (int m = 0; m < nkb; ++m) {
        const uint32_t km = key[m];
        rank += (km > kj) | ((km == kj) & (m < j));
      }
      keep = rank < top_k;
    }
    const uint64_t bal = __ballot(keep);
    if (lane == 0) wave_cnt[w] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int q = 0; q < w; ++q) off += wave_cnt[q];
    if (keep) out[off + __popcll(bal & ((1ull << lane) - 1ull))] = j;
    for (int q = 0; q < SEL_THREADS / 64; ++q) base += wave_cnt[q];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_block_pool(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, int64_t n_kv, int64_t kv_hs,
                             float* pooled_q, float* pooled_k, int nqb_cap, int nkb_cap,
                             hipStream_t stream) {
  const int nqb = (int)((n_q + block - 1) / block);
  const int nkb = (int)((n_kv + block - 1) / block);
  dim3 grid(nqb + nkb, heads);
#define HF_POOL(T, D)                                                                        \
  block_pool<T, D><<<grid, POOL_THREADS, 0, stream>>>(                                       \
      static_cast<const T*>(q), n_q, q_hs, static_cast<const T*>(k), n_kv, kv_hs, block, nqb, \
      pooled_q, pooled_k, nqb_cap, nkb_cap)
  if (dtype == 0) {
    if (d == 128) HF_POOL(bf16_t, 128); else HF_POOL(bf16_t, 64);
  } else {
    if (d == 128) HF_POOL(float, 128); else HF_POOL(float, 64);
  }
#undef HF_POOL
  return hipGetLastError();
}

hipError_t launch_score_select(int heads, int d, int nqb, int nkb, int nqb_cap, int nkb_cap,
                               const float* pooled_q, const float* pooled_k, float scale,
                               int top_k, int32_t* sel, float* scores_out, hipStream_t stream) {
  dim3 grid(nqb, heads);
  if (d == 128)
    score_select<128><<<grid, SEL_THREADS, 0, stream>>>(pooled_q, pooled_k, nqb, nkb, nqb_cap,
                                                        nkb_cap, scale, top_k, sel, scores_out);
  else
    score_select<64><<<grid, SEL_THREADS, 0, stream>>>(pooled_q, pooled_k, nqb, nkb, nqb_cap,
                                                       nkb_cap, scale, top_k, sel, scores_out);
  return hipGetLastError();
}

}  // namespace hf
