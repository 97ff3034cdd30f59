// hf_select.hip -- block importance scores and top-K key-block selection (gfx950).
//
// The sparse path keeps, for every query block, only the key blocks with the
// highest block importance score (gist.science English summary "Long-Horizon
// Streaming Video Generation via Hybrid Attention with Decoupled Distillation",
// 2.A.2 "Block-Sparse Sliding Window Attention"). The importance of key block j
// for query block i is tau * mean(Q rows of i) . mean(K rows of j), in fp32.
//
// block_pool  (HBM-bound): one wave per (head, block) streams the block's rows
//             once with 16-byte coalesced loads (all in flight together) and
//             writes the fp32 row mean.
// score_select (latency-bound): one workgroup per (5 query blocks, head) forms
//             their scores against all key blocks (four lanes per key block),
//             then one wave per query block selects the top_k exactly on an
//             order-preserving uint32 key of the fp32 score (-0.0 counts as
//             +0.0), ties going to the lower index, and writes the kept indices
//             in ascending order.
// absorb_and_pool / select_and_reduce: the same pooling and selection with the
//             absorb's partial states (first) and its reduce (second) as extra
//             workgroups of the launch, for the one-stream combined call.
#include <atomic>

#include "hf_absorb_parts.h"
#include "hf_device.h"
#include "hf_launch.h"
#include "hf_reduce.h"

namespace hf {

namespace {

constexpr int POOL_THREADS = 256;  // 4 waves, one (head, block) per wave

// The angles of one 8-row group's chunk (pairs p0 .. p0 + VEC/2 - 1) for the temporal
// rotation: with at least 8 tokens per frame a group spans at most two frames, so the
// (cos, sin) of both are loaded once (t0 for rows in the group's first frame, t1 for
// the next) and row r of the group is in the first frame iff r < split.
template <int VEC>
struct GroupAngles {
  float2 t0[VEC / 2], t1[VEC / 2];
  int split;
};
template <int VEC>
__device__ __forceinline__ GroupAngles<VEC> group_angles(const Rope& rope, int p0,
                                                         int64_t wrow0) {
  GroupAngles<VEC> a;
  const uint32_t tpf = (uint32_t)rope.tpf, f0 = (uint32_t)wrow0 / tpf;
  a.split = (int)(tpf - ((uint32_t)wrow0 - f0 * tpf));  // rows left in the first frame
  const uint32_t cap = (uint32_t)rope.cap;
  const float2* c0 = rope.cs + (size_t)(f0 < cap ? f0 : cap) * rope.half;
  const float2* c1 = rope.cs + (size_t)(f0 + 1 < cap ? f0 + 1 : cap) * rope.half;
#pragma unroll
  for (int e = 0; e < VEC / 2; ++e) {
    const bool on = p0 + e < rope.half;
    a.t0[e] = on ? c0[p0 + e] : make_float2(1.f, 0.f);
    a.t1[e] = on ? c1[p0 + e] : make_float2(1.f, 0.f);
  }
  return a;
}

// Rotate the VEC features of row r of the group (pairs below rope.half turn by the
// row's position; the others keep cos 1, sin 0, which leaves them exactly as they are).
template <int VEC>
__device__ __forceinline__ void rope_row(float* v, const GroupAngles<VEC>& a, int r) {
#pragma unroll
  for (int e = 0; e < VEC; e += 2) {
    const float2 t = r < a.split ? a.t0[e / 2] : a.t1[e / 2];
    const float x = v[e], y = v[e + 1];
    v[e] = x * t.x - y * t.y;
    v[e + 1] = x * t.y + y * t.x;
  }
}

// VEC fp32 values as one 16-byte chunk of T (bf16: rounded to nearest even).
template <typename T>
__device__ __forceinline__ uint4 narrow16(const float* v) {
  if constexpr (sizeof(T) == 2)
    return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                      pack_bf16x2(v[6], v[7]));
  else
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
}

// Row mean of one block per wave, summed by 8-row groups: lane (rg, cc) owns the
// 16-byte column chunk cc of the groups rg, rg + RPI, ... of the block (all row
// loads in flight together), adds each group's 8 rows in row order, adds its groups
// in order, and the lanes' totals are combined with lane exchanges in a fixed tree
// (every lane ends with the same sum). A key block's group sums can come from, and
// go to, a cache of 8-row sums (KeyCache), which gives the same sums bit for bit.
template <typename T, int D, bool ROPE>
__device__ __forceinline__ void pool_wave(
    int wid, const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ k,
    int64_t n_kv, int64_t kv_hs, int block, int nqb, int nkb, int heads,
    float* __restrict__ pooled_q, float* __restrict__ pooled_k, int nqb_cap, int nkb_cap,
    const KeyCache& kc, const Rope& rope, const Ragged& rag) {
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / VEC;         // chunks per row
  constexpr int RPI = 64 / CPR;        // lane groups (rows per wave-wide load)
  constexpr int GPL = 8 / RPI;         // 8-row groups per lane (blocks have at most 64 rows)
  static_assert(RPI >= 1 && RPI <= 8 && 8 % RPI == 0, "lane groups per 8-row group");
  const int lane = threadIdx.x & 63;
  int h, blk;
  bool is_q;
  int64_t n;
  const T* base;
  if (rag.on) {  // query blocks of every head, then each head's own key blocks
    if (wid >= heads * nqb + rag.kb0[heads]) return;
    is_q = wid < heads * nqb;
    if (is_q) {
      h = wid / nqb;
      blk = wid % nqb;
    } else {
      const int kw = wid - heads * nqb;
      h = 0;
      while (rag.kb0[h + 1] <= kw) ++h;
      blk = kw - rag.kb0[h];
    }
    n = is_q ? n_q : (int64_t)(rag.off[h + 1] - rag.off[h]);
    base = is_q ? q + (size_t)h * q_hs : k + (size_t)rag.off[h] * D;
  } else {
    if (wid >= heads * (nqb + nkb)) return;
    h = wid / (nqb + nkb);
    const int b = wid % (nqb + nkb);
    is_q = b < nqb;
    blk = is_q ? b : b - nqb;
    n = is_q ? n_q : n_kv;
    base = is_q ? q + (size_t)h * q_hs : k + (size_t)h * kv_hs;
  }
  const int64_t r0 = (int64_t)blk * block;
  const int64_t r1 = r0 + block < n ? r0 + block : n;
  const int cc = lane % CPR, rg = lane / CPR;
  // Group i of this lane: rows r0 + 8 (rg + RPI i) + 0..7; cached iff it is a key
  // group whose absolute index is in the cache's range.
  const bool use_cache = !is_q && kc.ring != nullptr;  // wave-uniform
  bool cached[GPL];
  int64_t gabs[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int64_t row0 = r0 + 8 * (rg + RPI * i);
    gabs[i] = kc.g0 + row0 / 8;
    cached[i] = use_cache && row0 < r1 && gabs[i] >= kc.lo && gabs[i] < kc.hi;
  }
  uint4 x[GPL][8];
#pragma unroll
  for (int i = 0; i < GPL; ++i)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = r0 + 8 * (rg + RPI * i) + r;
      x[i][r] = ld16(base + row * D + cc * VEC, row < r1 && !cached[i]);  // past the block: 0
    }
  float tot[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) tot[e] = 0.f;
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    float g8[VEC];
    float* slot = nullptr;
    if (use_cache)
      slot = kc.ring + ((size_t)h * kc.cap + (size_t)(gabs[i] & (kc.cap - 1))) * D + cc * VEC;
    if (cached[i]) {
#pragma unroll
      for (int e = 0; e < VEC; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(slot + e);
        g8[e] = v.x, g8[e + 1] = v.y, g8[e + 2] = v.z, g8[e + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) g8[e] = 0.f;
      const int64_t grow0 = r0 + 8 * (rg + RPI * i);  // the group's first row
      const bool rot = ROPE && cc * VEC < 2 * rope.half && grow0 < r1;
      GroupAngles<VEC> ang;
      if constexpr (ROPE)
        if (rot) ang = group_angles<VEC>(rope, cc * VEC / 2, is_q ? rope.q_row0 + grow0 : grow0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float v[VEC];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = bf16_to_f32(half16(x[i][r], e));
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = __uint_as_float(word(x[i][r], e));
        }
        if constexpr (ROPE) {
          const int64_t row = grow0 + r;
          if (row < r1) {
            if (rot) rope_row<VEC>(v, ang, r);
            if (!is_q)  // the window's rotated keys for the attention kernel
              *reinterpret_cast<uint4*>(static_cast<T*>(rope.k_out) + (size_t)h * rope.k_out_hs +
                                        row * D + cc * VEC) = narrow16<T>(v);
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) g8[e] += v[e];
      }
      if (use_cache && r0 + 8 * (rg + RPI * i) < r1) {  // a key group of the window
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *reinterpret_cast<float4*>(slot + e) = make_float4(g8[e], g8[e + 1], g8[e + 2], g8[e + 3]);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) tot[e] += g8[e];
  }
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) tot[e] += __shfl_xor(tot[e], off);
  if (rg == 0) {
    const float inv = 1.f / (float)(r1 - r0);
    float* dst = is_q ? pooled_q + ((size_t)h * nqb_cap + blk) * D
                      : pooled_k + ((size_t)h * nkb_cap + blk) * D;
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<float4*>(dst + cc * VEC + e) =
          make_float4(tot[e] * inv, tot[e + 1] * inv, tot[e + 2] * inv, tot[e + 3] * inv);
  }
}

template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(POOL_THREADS) void block_pool(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ k, int64_t n_kv,
    int64_t kv_hs, int block, int nqb, int nkb, int heads, float* __restrict__ pooled_q,
    float* __restrict__ pooled_k, int nqb_cap, int nkb_cap, KeyCache kc, Rope rope, Ragged rg) {
  pool_wave<T, D, ROPE>(blockIdx.x * (POOL_THREADS / 64) + (threadIdx.x >> 6), q, n_q, q_hs, k, n_kv,
                  kv_hs, block, nqb, nkb, heads, pooled_q, pooled_k, nqb_cap, nkb_cap, kc, rope,
                  rg);
}

// The absorb's partial states and the block pooling in one launch: workgroups
// below n_abs are absorb workgroups (absorb::item), the others pool one (head,
// block) per wave. The two read and write different buffers and both are bound by
// memory, so they share the launch (and its ramp) instead of running one after
// the other. The absorb workgroups come first, so that they are spread over the
// compute units before the pooling fills the rest.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__((absorb::threads<T, D>())) void absorb_and_pool(
    const T* __restrict__ kev, const T* __restrict__ vev, int64_t n_ev, int64_t ev_hs, int tps,
    int n_split, float* __restrict__ partials, int n_abs, const T* __restrict__ q, int64_t n_q,
    int64_t q_hs, const T* __restrict__ k, int64_t n_kv, int64_t kv_hs, int block, int nqb,
    int nkb, int heads, float* __restrict__ pooled_q, float* __restrict__ pooled_k, int nqb_cap,
    int nkb_cap, KeyCache kc, Rope rope, Ragged rg) {
  if ((int)blockIdx.x < n_abs) {
    absorb::item<T, D>(blockIdx.x, n_split, kev, vev, n_ev, ev_hs, tps, partials);
  } else {
    // The pooling workgroups are as many as fit next to the absorb's (the launcher
    // sizes them), and each wave pools every n_waves-th block, so that all of the
    // pooling streams from the start instead of waiting for free slots.
    constexpr int WPG = absorb::threads<T, D>() / 64;  // pooling waves per workgroup
    const int n_waves = ((int)gridDim.x - n_abs) * WPG;
    const int total = rg.on ? heads * nqb + rg.kb0[heads] : heads * (nqb + nkb);
    for (int wid = ((int)blockIdx.x - n_abs) * WPG + (int)(threadIdx.x >> 6); wid < total;
         wid += n_waves)
      pool_wave<T, D, ROPE>(wid, q, n_q, q_hs, k, n_kv, kv_hs, block, nqb, nkb, heads, pooled_q,
                      pooled_k, nqb_cap, nkb_cap, kc, rope, rg);
  }
}

constexpr int SEL_THREADS = 1024;  // 16 waves: the score phase, then 4 of them select

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int SEL_QB = 5;  // query blocks per workgroup, one selecting wave each

// Scores of SEL_QB query blocks against all key blocks (four lanes per key block,
// fixed-order dot products), then one wave per query block selects exactly:
// T = the top_k-th largest key is found bit by bit (count of keys >= candidate by
// ballots), every key above T is kept, and keys equal to T are kept in ascending
// index order until top_k are kept; the kept indices are written in ascending
// order. Keys are unique up to exact score ties, which therefore go to the lower
// index.
template <int D, int NE>
__device__ __forceinline__ void select_group(
    int qg, int h, const float* __restrict__ pooled_q, const float* __restrict__ pooled_k,
    int nqb, int nkb, int nqb_cap, int nkb_cap, float scale, int top_k,
    int32_t* __restrict__ sel, float* __restrict__ scores_out, const Ragged& rg) {
  // Ragged windows: this head's own block count and top_k; rows of sel keep the stride
  // top_k (the largest of the heads') passed in.
  const int sel_stride = top_k;
  if (rg.on) {
    nkb = rg.kb0[h + 1] - rg.kb0[h];
    top_k = rg.top_k[h];
  }
  // Four adjacent lanes per key block, each over a quarter of the features (the
  // block's row is read as four contiguous segments); the quarters are added with
  // two lane exchanges, which give every lane of the four the same sum. One pass
  // covers SEL_THREADS / 4 key blocks (256), so the pooled key rows' load latency is
  // paid once.
  constexpr int PARTS = 4, EV = D / 4 / PARTS;  // float4s per quarter
  __shared__ uint32_t key[SEL_QB][kMaxKeyBlocks];
  // The pooled query rows by quarter, each quarter padded by one float4: the four
  // quarters a wave reads at once then start 4 banks apart instead of on the same bank.
  __shared__ float4 qs[SEL_QB][PARTS][EV + 1];
  const int i0 = qg * SEL_QB, tid = threadIdx.x;
  const int nq = nqb - i0 < SEL_QB ? nqb - i0 : SEL_QB;
  static_assert(SEL_THREADS % PARTS == 0, "a key block's lanes stay in one pass");
  // The first pass's key rows are requested before the query rows are staged, so that
  // the two loads' latencies overlap instead of following one another.
  auto key_part = [&](int x) {
    return reinterpret_cast<const float4*>(pooled_k + ((size_t)h * nkb_cap + x / PARTS) * D) +
           (x % PARTS) * EV;
  };
  float4 kv[EV];
  if (tid < nkb * PARTS) {
    const float4* km = key_part(tid);
#pragma unroll
    for (int e = 0; e < EV; ++e) kv[e] = km[e];
  }
  for (int x = tid; x < SEL_QB * (D / 4); x += SEL_THREADS) {
    const int r = x / (D / 4), e = x % (D / 4);
    qs[r][e / EV][e % EV] = r < nq ? reinterpret_cast<const float4*>(
                                         pooled_q + ((size_t)h * nqb_cap + i0 + r) * D)[e]
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  for (int x = tid; x < nkb * PARTS; x += SEL_THREADS) {
    const int j = x / PARTS, part = x % PARTS;
    if (x != tid) {  // later passes (more than SEL_THREADS / PARTS key blocks)
      const float4* km = key_part(x);
#pragma unroll
      for (int e = 0; e < EV; ++e) kv[e] = km[e];
    }
    float sq[SEL_QB];
#pragma unroll
    for (int r = 0; r < SEL_QB; ++r) {
      // Query row r's reads stay here (all rows hoisted at once would not fit the
      // registers of a 1024-thread workgroup and would serialise the loads above).
      asm volatile("" ::: "memory");
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        const float4 qv = qs[r][part][e];
        s += qv.x * kv[e].x;
        s += qv.y * kv[e].y;
        s += qv.z * kv[e].z;
        s += qv.w * kv[e].w;
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      sq[r] = s * scale;
    }
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < SEL_QB; ++r) {
        key[r][j] = score_key(sq[r]);
        if (scores_out && r < nq) scores_out[((size_t)h * nqb + i0 + r) * nkb + j] = sq[r];
      }
    }
  }
  __syncthreads();
  const int r = tid >> 6, lane = tid & 63;
  if (!sel || r >= nq) return;
  // Keys of this query block in registers, key j = 64e + lane; past the window the
  // key is 0, which never counts (every candidate below is >= 1, and a finite
  // score's key is >= 1).
  uint32_t kr[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int j = e * 64 + lane;
    kr[e] = j < nkb ? key[r][j] : 0u;
  }
  auto count_at_least = [&](uint32_t cand) {
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < NE; ++e) cnt += __popcll(__ballot(kr[e] >= cand));
    return cnt;
  };
  uint32_t T = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    if (count_at_least(cand) >= top_k) T = cand;
  }
  const int need = top_k - count_at_least(T + 1u);  // keys equal to T to keep
  const uint64_t lt = (1ull << lane) - 1ull;
  int32_t* out = sel + ((size_t)h * nqb + i0 + r) * sel_stride;
  int pos = 0, eq_before = 0;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const bool eq = kr[e] == T;  // T >= 1, so padding never matches
    const uint64_t beq = __ballot(eq);
    const bool keep = kr[e] > T || (eq && eq_before + __popcll(beq & lt) < need);
    eq_before += __popcll(beq);
    const uint64_t bk = __ballot(keep);
    if (keep) out[pos + __popcll(bk & lt)] = e * 64 + lane;
    pos += __popcll(bk);
  }
}

template <int D, int NE>
__global__ __launch_bounds__(SEL_THREADS) void score_select(
    const float* __restrict__ pooled_q, const float* __restrict__ pooled_k, int nqb, int nkb,
    int nqb_cap, int nkb_cap, float scale, int top_k, int32_t* __restrict__ sel,
    float* __restrict__ scores_out, Ragged rg) {
  select_group<D, NE>(blockIdx.x, blockIdx.y, pooled_q, pooled_k, nqb, nkb, nqb_cap, nkb_cap,
                      scale, top_k, sel, scores_out, rg);
}

// The selection and the absorb's reduce in one launch: workgroups below n_sel
// select (n_qg groups of query blocks per head), the others reduce (red_wgs per
// head, RED_PER_WG reduce groups each). They read and write different buffers.
// The reduce is bound by what each of its compute units pulls from memory, so a
// reduce workgroup runs one group fewer than it could hold (at 12 heads and 74 query
// blocks: 72 reduce workgroups beside the 180 selecting ones, one per compute unit),
// and its fourth group of threads idles.
constexpr int RED_PER_WG = SEL_THREADS / RED_THREADS - 1;
static_assert(SEL_THREADS % RED_THREADS == 0, "whole reduce groups per workgroup");
template <int D>
constexpr int red_wgs() { return (red_groups<D>() + RED_PER_WG - 1) / RED_PER_WG; }
template <int D, int NE>
__global__ __launch_bounds__(SEL_THREADS) void select_and_reduce(
    const float* __restrict__ pooled_q, const float* __restrict__ pooled_k, int nqb, int nkb,
    int nqb_cap, int nkb_cap, float scale, int top_k, int32_t* __restrict__ sel, int n_qg,
    int n_sel, const float* __restrict__ partials, int n_split, float* __restrict__ S,
    float* __restrict__ z, uint16_t* __restrict__ s_split) {
  if ((int)blockIdx.x < n_sel) {
    select_group<D, NE>((int)blockIdx.x % n_qg, (int)blockIdx.x / n_qg, pooled_q, pooled_k, nqb,
                        nkb, nqb_cap, nkb_cap, scale, top_k, sel, nullptr, Ragged());
  } else {
    const int r = (int)blockIdx.x - n_sel;
    const int grp = (r % red_wgs<D>()) * RED_PER_WG + (int)threadIdx.x / RED_THREADS;
    if ((int)threadIdx.x / RED_THREADS < RED_PER_WG && grp < red_groups<D>())
      absorb_reduce_group<D>(grp, r / red_wgs<D>(), partials, n_split, S, z, s_split,
                             (int)threadIdx.x % RED_THREADS);
  }
}

}  // namespace

hipError_t launch_block_pool(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, int64_t n_kv, int64_t kv_hs,
                             float* pooled_q, float* pooled_k, int nqb_cap, int nkb_cap,
                             hipStream_t stream, const KeyCache& kc, const Rope& rope,
                             const Ragged& rg) {
  const int nqb = (int)((n_q + block - 1) / block);
  const int nkb = (int)((n_kv + block - 1) / block);
  const int waves = rg.on ? heads * nqb + rg.kb0[heads] : heads * (nqb + nkb);
  const int grid = (waves + POOL_THREADS / 64 - 1) / (POOL_THREADS / 64);
#define HF_POOL_R(T, D, R)                                                                    \
  block_pool<T, D, R><<<grid, POOL_THREADS, 0, stream>>>(                                    \
      static_cast<const T*>(q), n_q, q_hs, static_cast<const T*>(k), n_kv, kv_hs, block, nqb, \
      nkb, heads, pooled_q, pooled_k, nqb_cap, nkb_cap, kc, rope, rg)
#define HF_POOL(T, D) \
  do { if (rope.cs) HF_POOL_R(T, D, true); else HF_POOL_R(T, D, false); } while (0)
  if (dtype == 0) {
    if (d == 128) HF_POOL(bf16_t, 128); else HF_POOL(bf16_t, 64);
  } else {
    if (d == 128) HF_POOL(float, 128); else HF_POOL(float, 64);
  }
#undef HF_POOL
#undef HF_POOL_R
  return hipGetLastError();
}

// Pooling workgroups of an absorb_and_pool launch: the resident slots the absorb's
// n_abs workgroups leave free (at least one per compute unit), at most `needed`.
// `occ_cache` (one per kernel instance) keeps the occupancy per device.
template <typename K>
int pool_workgroups(K kernel, int threads, int n_abs, int needed,
                    std::atomic<int> (&occ_cache)[64]) {
  int dev = 0, occ = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64)
    occ = occ_cache[dev].load(std::memory_order_relaxed);
  if (occ < 1) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess ||
        occ < 1)
      occ = 1;
    if (dev >= 0 && dev < 64) occ_cache[dev].store(occ, std::memory_order_relaxed);
  }
  const int n_cu = device_cu_count();
  int n = occ * n_cu - n_abs;
  if (n < n_cu) n = n_cu;
  return n < needed ? n : needed;
}

hipError_t launch_absorb_and_pool(int dtype, int heads, int d, int block, const void* k_ev,
                                  const void* v_ev, int64_t n_ev, int64_t ev_hs, float* partials,
                                  const void* q, int64_t n_q, int64_t q_hs, const void* k,
                                  int64_t n_kv, int64_t kv_hs, float* pooled_q, float* pooled_k,
                                  int nqb_cap, int nkb_cap, hipStream_t stream,
                                  const KeyCache& kc, const Rope& rope) {
  const int nqb = (int)((n_q + block - 1) / block);
  const int nkb = (int)((n_kv + block - 1) / block);
  const AbsorbPlan p = absorb_plan(dtype, heads, d, n_ev);
  const int n_abs = absorb_items(dtype, heads, d, p);
#define HF_ABSPOOL_R(T, D, R)                                                                  \
  {                                                                                            \
    constexpr int wpg = absorb::threads<T, D>() / 64;                                          \
    static std::atomic<int> occ_cache[64];                                                     \
    const int n_pool = pool_workgroups(absorb_and_pool<T, D, R>, absorb::threads<T, D>(), n_abs, \
                                       (heads * (nqb + nkb) + wpg - 1) / wpg, occ_cache);      \
    absorb_and_pool<T, D, R><<<n_abs + n_pool, absorb::threads<T, D>(), 0, stream>>>(          \
        static_cast<const T*>(k_ev), static_cast<const T*>(v_ev), n_ev, ev_hs,                 \
        p.tokens_per_split, p.n_split, partials, n_abs, static_cast<const T*>(q), n_q, q_hs,   \
        static_cast<const T*>(k), n_kv, kv_hs, block, nqb, nkb, heads, pooled_q, pooled_k,     \
        nqb_cap, nkb_cap, kc, rope, Ragged());                                                 \
  }
#define HF_ABSPOOL(T, D) \
  { if (rope.cs) HF_ABSPOOL_R(T, D, true) else HF_ABSPOOL_R(T, D, false) }
  if (dtype == 0) {
    if (d == 128) HF_ABSPOOL(bf16_t, 128) else HF_ABSPOOL(bf16_t, 64)
  } else {
    if (d == 128) HF_ABSPOOL(float, 128) else HF_ABSPOOL(float, 64)
  }
#undef HF_ABSPOOL
#undef HF_ABSPOOL_R
  return hipGetLastError();
}

hipError_t launch_score_select(int heads, int d, int nqb, int nkb, int nqb_cap, int nkb_cap,
                               const float* pooled_q, const float* pooled_k, float scale,
                               int top_k, int32_t* sel, float* scores_out, hipStream_t stream,
                               const Ragged& rg) {
  dim3 grid((nqb + SEL_QB - 1) / SEL_QB, heads);
#define HF_SEL(D, NE)                                                                      \
  score_select<D, NE><<<grid, SEL_THREADS, 0, stream>>>(pooled_q, pooled_k, nqb, nkb, nqb_cap, \
                                                         nkb_cap, scale, top_k, sel, scores_out, \
                                                         rg)
  // NE = 64-key chunks held per lane in the selection (the smallest that covers nkb).
  if (d == 128) {
    if (nkb <= 256) HF_SEL(128, 4); else if (nkb <= 512) HF_SEL(128, 8); else HF_SEL(128, 32);
  } else {
    if (nkb <= 256) HF_SEL(64, 4); else if (nkb <= 512) HF_SEL(64, 8); else HF_SEL(64, 32);
  }
#undef HF_SEL
  return hipGetLastError();
}

hipError_t launch_select_and_reduce(int dtype, int heads, int d, int nqb, int nkb, int nqb_cap,
                                    int nkb_cap, const float* pooled_q, const float* pooled_k,
                                    float scale, int top_k, int32_t* sel, const float* partials,
                                    int64_t n_ev, float* S, float* z, uint16_t* s_split,
                                    hipStream_t stream) {
  const int n_qg = (nqb + SEL_QB - 1) / SEL_QB;
  const int n_sel = n_qg * heads;
  const int n_split = absorb_plan(dtype, heads, d, n_ev).n_split;
#define HF_SELRED(D, NE)                                                                    \
  select_and_reduce<D, NE><<<n_sel + red_wgs<D>() * heads, SEL_THREADS, 0, stream>>>(        \
      pooled_q, pooled_k, nqb, nkb, nqb_cap, nkb_cap, scale, top_k, sel, n_qg, n_sel,       \
      partials, n_split, S, z, s_split)
  if (d == 128) {
    if (nkb <= 256) HF_SELRED(128, 4); else if (nkb <= 512) HF_SELRED(128, 8); else HF_SELRED(128, 32);
  } else {
    if (nkb <= 256) HF_SELRED(64, 4); else if (nkb <= 512) HF_SELRED(64, 8); else HF_SELRED(64, 32);
  }
#undef HF_SELRED
  return hipGetLastError();
}

}  // namespace hf
