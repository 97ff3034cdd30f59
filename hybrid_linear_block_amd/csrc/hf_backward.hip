// hf_backward.hip -- backward pass of the per-chunk hybrid attention (gfx950).
//
// Hybrid Forcing trains through this path ([EN] 2.B-C, decoupled distillation; the
// state is learnable, [EN] 2.A.1). With the key-block selection of the forward call
// held fixed and L = sum(dout * out), per head (tau = scale, phi = elu + 1):
//   softmax path  dv_t += p_rt dout_r, dl_rt = p_rt (dout_r . v_t - D_r),
//                 D_r = dout_r . o_swa_r, dq_r += tau sum_t dl_rt k_t,
//                 dk_t += tau dl_rt q_r;
//   linear read   f = phi(q_r), den = z . f + eps, g = dout_r / den,
//                 c = -(dout_r . S f) / den^2, dS += g f^T, dz += c f,
//                 dq_r += phi'(q_r) * (S^T g + c z);
//   absorb        dv_n = dS phi(k_n), dk_n = phi'(k_n) * (dS^T v_n + dz).
//
// No atomics: every sum runs in a fixed order, so the results are bitwise
// reproducible. Kernels:
//   bwd_inv_sel        per (head, 64 key blocks): the query blocks that selected each,
//                      ascending.
// fp32 states (fp32 arithmetic on the vector units; a row's dot products are split
// over TPR adjacent lanes and reduced with xor shuffles, tiles staged in LDS as fp32):
//   bwd_rows           per (head, query block): pass 1 recomputes each row's softmax
//                      (log-sum-exp and o_swa, hence D_r) over its selected blocks, then
//                      the linear read's terms; pass 2 accumulates dq; stores per-row
//                      (lse, D, den, c) for the other kernels;
//   bwd_kv             per (head, key block): dk and dv over the query blocks that
//                      selected it;
//   bwd_state          per (head, 4 rows of dS, or z): dS and dz over all query rows;
//   absorb_bwd         per (head, 64 evicted tokens): dk_ev and dv_ev.
// bf16 states (v_mfma_f32_16x16x32_bf16; fp32 operands split into bf16 hi + lo, so the
// products keep ~fp32 accuracy, fp32 accumulation):
//   bwd_dq2            the softmax part of dq, lse and D (tiles staged like the forward);
//   bwd_rows_lin_mfma  the linear read's part of dq, den and c;
//   bwd_kv2            dk and dv (tiles staged like the forward);
//   bwd_state_mfma     partial dS and dz per 256 query rows, bwd_state_reduce sums them
//                      in order;
//   absorb_bwd_mfma    dk_ev and dv_ev.
#include <type_traits>

#include "hf_device.h"
#include "hf_launch.h"

namespace hf {

namespace {

constexpr int BT = 256;  // threads per workgroup
constexpr float kL2e = 1.4426950408889634f;

__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const bf16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float phi_prime(float x) { return x > 0.f ? 1.f : __expf(x); }

// 2^x on the transcendental unit (one v_exp_f32). Results below 2^-126 may flush to
// zero; the weights and rescale factors this serves are then negligible next to the
// row's largest term, which is at least 1/n.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the TPR adjacent lanes of a row; every lane gets the same bits (xor
// butterfly, commutative adds). Within a quad the exchanges are DPP quad
// permutations (no LDS round trip); wider rows use ds_bpermute for the rest.
__device__ __forceinline__ float dpp_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float dpp_half_mirror(float x) {  // lane i <- 7 - i in each 8
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror(float x) {  // lane i <- 15 - i in each 16
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
}
// After the quad steps every lane holds its quad's sum; the mirrors pair each lane
// with one in the other quad (then the other half of 16), so the adds stay
// commutative pairs and all TPR lanes end with the same bits.
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(TPR >= 1 && TPR <= 16, "rows of up to 16 lanes");
  if (TPR >= 2) x += dpp_xor1(x);
  if (TPR >= 4) x += dpp_xor2(x);
  if (TPR >= 8) x += dpp_half_mirror(x);
  if (TPR >= 16) x += dpp_mirror(x);
  return x;
}

__device__ __forceinline__ int clamp_block(int j, int n) { return j < 0 ? 0 : (j >= n ? n - 1 : j); }

__device__ __forceinline__ void widen_store(float* o, uint4 w, const bf16_t*, bool ph) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float lo = __uint_as_float(x[k] << 16), hi = __uint_as_float(x[k] & 0xffff0000u);
    if (ph) {
      lo = phi(lo);
      hi = phi(hi);
    }
    o[2 * k] = lo;
    o[2 * k + 1] = hi;
  }
}
__device__ __forceinline__ void widen_store(float* o, uint4 w, const float*, bool ph) {
  float4 f = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                         __uint_as_float(w.w));
  if (ph) f = make_float4(phi(f.x), phi(f.y), phi(f.z), phi(f.w));
  *reinterpret_cast<float4*>(o) = f;
}

// Rows [row0, row0 + R) of a [N][D] head into an fp32 tile (phi applied if PHI);
// rows >= n read as 0. Every 16-byte load of the workgroup's share is issued before
// the first LDS store, so the memory latency is paid once per tile.
template <typename T, int D, int R, bool PHI = false>
__device__ __forceinline__ void load_tile(const T* __restrict__ base, int64_t row0, int64_t n,
                                          float* tile) {
  constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte load
  constexpr int NV = R * D / EPV;
  constexpr int PER = (NV + BT - 1) / BT;
  uint4 buf[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int v = threadIdx.x + k * BT;
    const int64_t r = row0 + (v * EPV) / D;
    buf[k] = (v < NV && r < n)
                 ? *reinterpret_cast<const uint4*>(base + r * D + (v * EPV) % D)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int v = threadIdx.x + k * BT;
    if (v < NV) {
      const int64_t r = row0 + (v * EPV) / D;
      if (PHI && r >= n) {
#pragma unroll
        for (int x = 0; x < EPV; ++x) tile[v * EPV + x] = 0.f;
      } else {
        widen_store(tile + v * EPV, buf[k], base, PHI);
      }
    }
  }
}

// One workgroup per (head, 64 key blocks j0 .. j0 + 63). The head's selection rows are
// read once, flat and coalesced, a chunk of up to kInvChunk query blocks at a time; each
// entry in the workgroup's range sets bit (j, i) of a bitmap in LDS; then thread j - j0
// appends the query blocks of its row of bits in ascending order. Entries outside
// [0, nkb) set no bit and a repeated entry sets its bit once (the rows are strictly
// ascending and in range by the backward's contract).
constexpr int kInvKeys = 64;                // key blocks per workgroup
constexpr int kInvWords = 32;               // bitmap words per key block and chunk
constexpr int kInvChunk = 32 * kInvWords;   // query blocks per chunk
__global__ __launch_bounds__(256) void bwd_inv_sel(const int32_t* __restrict__ sel, int nqb,
                                                   int nkb, int top_k, int32_t* __restrict__ cnt,
                                                   int32_t* __restrict__ list, int nqb_cap) {
  __shared__ uint32_t bits[kInvKeys][kInvWords];
  const int groups = (nkb + kInvKeys - 1) / kInvKeys;
  const int h = (int)blockIdx.x / groups, j0 = ((int)blockIdx.x % groups) * kInvKeys;
  const int tid = (int)threadIdx.x;
  const int32_t* sh = sel + (int64_t)h * nqb * top_k;
  const int jl = tid;  // threads 0 .. 63 own key block j0 + jl
  int n = 0;
  for (int i0 = 0; i0 < nqb; i0 += kInvChunk) {
    const int rows = nqb - i0 < kInvChunk ? nqb - i0 : kInvChunk;
    for (int e = tid; e < kInvKeys * kInvWords; e += 256) (&bits[0][0])[e] = 0u;
    __syncthreads();
    const int n_ent = rows * top_k;  // <= kInvChunk * kMaxKeyBlocks
    const int32_t* base = sh + (int64_t)i0 * top_k;
    constexpr int U = 8;  // loads in flight per thread
    for (int f0 = 0; f0 < n_ent; f0 += U * 256) {
      int32_t jv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * 256 + tid;
        jv[u] = f < n_ent ? base[f] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int f = f0 + u * 256 + tid;
        const int jj = jv[u] - j0;
        if (jj >= 0 && jj < kInvKeys && jv[u] < nkb) {
          const int i = f / top_k;
          atomicOr(&bits[jj][i >> 5], 1u << (i & 31));
        }
      }
    }
    __syncthreads();
    if (jl < kInvKeys && j0 + jl < nkb) {
      int32_t* out = list + ((int64_t)h * nkb + j0 + jl) * nqb_cap;
      for (int w = 0; w * 32 < rows; ++w) {
        uint32_t m = bits[jl][w];
        while (m) {
          out[n++] = i0 + 32 * w + __builtin_ctz(m);
          m &= m - 1u;
        }
      }
    }
    __syncthreads();
  }
  if (jl < kInvKeys && j0 + jl < nkb) cnt[(int64_t)h * nkb + j0 + jl] = n;
}

// Query rows per workgroup of bwd_rows and key rows per workgroup of bwd_kv, and
// the rows of their staged tiles: 32 (16 for 16-row blocks), so that two 32-row
// fp32 tiles (32 KB at d = 128) and a 16-feature slice per lane leave room for
// several workgroups per compute unit.
template <int BLK>
constexpr int kRows = BLK > 32 ? 32 : BLK;

// Body of the fp32 row kernel.
template <typename T, int D, int BLK>
__device__ __forceinline__ void rows_body(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ kg,
    const T* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int nkb, const float* __restrict__ S, const float* __restrict__ z,
    float eps, float scale, const T* __restrict__ dout, int64_t do_hs, float* __restrict__ dq,
    int64_t dq_hs, float* __restrict__ rs, int64_t nq_cap) {
  // A query block is split into 32-row parts.
  constexpr int RPW = kRows<BLK>, KT = RPW, SPLIT = BLK / RPW;
  constexpr int TPR = BT / RPW, DS = D / TPR;
  static_assert(DS % 4 == 0, "float4 slices");
  __shared__ __align__(16) float tk[KT * D];
  __shared__ __align__(16) float tv[KT * D];
  const int h = blockIdx.x / (nqb * SPLIT), i = (blockIdx.x / SPLIT) % nqb;
  const int part = blockIdx.x % SPLIT;
  const int rl = threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * DS;
  const int64_t r = (int64_t)i * BLK + part * RPW + rl;
  const bool live = r < n_q;
  const int64_t rr = live ? r : n_q - 1;
  const T* kh = kg + (int64_t)h * kv_hs;
  const T* vh = vg + (int64_t)h * kv_hs;
  const float* zh = z + (int64_t)h * D;
  const int32_t* my_sel = sel + ((int64_t)h * nqb + i) * top_k;
  float qv[DS], dov[DS], acc[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    qv[e] = ldf(q + (int64_t)h * q_hs + rr * D + d0 + e);
    dov[e] = ldf(dout + (int64_t)h * do_hs + rr * D + d0 + e);
    acc[e] = 0.f;
  }
  const float sl2 = scale * kL2e;

  // ---- pass 1: softmax statistics and o_swa (online, base 2) ----
  float m2 = -INFINITY, l = 0.f;
  for (int tt = 0; tt < top_k * SPLIT; ++tt) {
    const int64_t k0 = (int64_t)clamp_block(my_sel[tt / SPLIT], nkb) * BLK + (tt % SPLIT) * KT;
    if (k0 >= n_kv) continue;  // the ragged last block has no second half
    __syncthreads();
    load_tile<T, D, KT>(kh, k0, n_kv, tk);
    load_tile<T, D, KT>(vh, k0, n_kv, tv);
    __syncthreads();
    const int nvalid = (int)min((int64_t)KT, n_kv - k0);
    // Keys in groups of 4 (independent dot products, one max update per group),
    // then the remainder one by one.
    int u = 0;
    for (; u + 4 <= nvalid; u += 4) {
      float x[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* kr = tk + (u + w) * D + d0;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DS; ++e) s += qv[e] * kr[e];
        x[w] = s;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) x[w] = row_sum<TPR>(x[w]) * sl2;
      const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (mx > m2) {
        const float a = exp2_hw(m2 - mx);
        l *= a;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] *= a;
        m2 = mx;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p = exp2_hw(x[w] - m2);
        l += p;
        const float* vr = tv + (u + w) * D + d0;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] += p * vr[e];
      }
    }
    for (; u < nvalid; ++u) {
      const float* kr = tk + u * D + d0;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) s += qv[e] * kr[e];
      const float x = row_sum<TPR>(s) * sl2;
      if (x > m2) {
        const float a = exp2_hw(m2 - x);
        l *= a;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] *= a;
        m2 = x;
      }
      const float p = exp2_hw(x - m2);
      l += p;
      const float* vr = tv + u * D + d0;
#pragma unroll
      for (int e = 0; e < DS; ++e) acc[e] += p * vr[e];
    }
  }
  const float inv_l = 1.f / l;
  float dpart = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) dpart += dov[e] * (acc[e] * inv_l);
  const float Dr = row_sum<TPR>(dpart);
  const float lse2 = m2 + log2f(l);

  // ---- linear read: den, c = -(dout . S f) / den^2, dq_lin ----
  float fz = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) fz += phi(qv[e]) * zh[d0 + e];
  const float den = row_sum<TPR>(fz) + eps;
  const float inv_den = 1.f / den;
  __syncthreads();  // every wave is done with the last tiles
  const float* Sh = S + (int64_t)h * D * D;
  float* frow = tk + rl * D;
  float* grow = tv + rl * D;
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    frow[d0 + e] = phi(qv[e]);
    grow[d0 + e] = dov[e] * inv_den;
  }
  __syncthreads();
  // (S f)_j for the slice's rows j, column chunk by column chunk
  float sf[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) sf[e] = 0.f;
#pragma unroll 2
  for (int c4 = 0; c4 < D; c4 += 4) {
    const float4 f4 = *reinterpret_cast<const float4*>(frow + c4);
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const float4 s4 = *reinterpret_cast<const float4*>(Sh + (int64_t)(d0 + e) * D + c4);
      sf[e] += s4.x * f4.x + s4.y * f4.y + s4.z * f4.z + s4.w * f4.w;
    }
  }
  float cpart = 0.f;
#pragma unroll
  for (int e = 0; e < DS; ++e) cpart += dov[e] * sf[e];
  const float c = -row_sum<TPR>(cpart) * inv_den * inv_den;
  float dql[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) dql[e] = 0.f;
#pragma unroll 2
  for (int j = 0; j < D; ++j) {
    const float gj = grow[j];
    const float* srow = Sh + (int64_t)j * D + d0;
#pragma unroll
    for (int e = 0; e < DS; e += 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(srow + e);
      dql[e] += gj * s4.x;
      dql[e + 1] += gj * s4.y;
      dql[e + 2] += gj * s4.z;
      dql[e + 3] += gj * s4.w;
    }
  }
#pragma unroll
  for (int e = 0; e < DS; ++e) acc[e] = phi_prime(qv[e]) * (dql[e] + c * zh[d0 + e]);

  // ---- pass 2: dq of the softmax path ----
  for (int tt = 0; tt < top_k * SPLIT; ++tt) {
    const int64_t k0 = (int64_t)clamp_block(my_sel[tt / SPLIT], nkb) * BLK + (tt % SPLIT) * KT;
    if (k0 >= n_kv) continue;
    __syncthreads();
    load_tile<T, D, KT>(kh, k0, n_kv, tk);
    load_tile<T, D, KT>(vh, k0, n_kv, tv);
    __syncthreads();
    const int nvalid = (int)min((int64_t)KT, n_kv - k0);
    for (int u = 0; u < nvalid; ++u) {
      const float* kr = tk + u * D + d0;
      const float* vr = tv + u * D + d0;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        s += qv[e] * kr[e];
        dp += dov[e] * vr[e];
      }
      s = row_sum<TPR>(s);
      dp = row_sum<TPR>(dp);
      const float p = exp2_hw(s * sl2 - lse2);
      const float dl = scale * p * (dp - Dr);
#pragma unroll
      for (int e = 0; e < DS; ++e) acc[e] += dl * kr[e];
    }
  }
  if (live) {
    float* o = dq + (int64_t)h * dq_hs + r * D + d0;
#pragma unroll
    for (int e = 0; e < DS; ++e) o[e] = acc[e];
    if (d0 == 0) {
      float* st = rs + ((int64_t)h * nq_cap + r) * 4;
      st[0] = lse2;
      st[1] = Dr;
      st[2] = den;
      st[3] = c;
    }
  }
}

#define HF_ROWS_ARGS                                                                       \
  const T *__restrict__ q, int64_t n_q, int64_t q_hs, const T *__restrict__ kg,            \
      const T *__restrict__ vg, int64_t n_kv, int64_t kv_hs,                                \
      const int32_t *__restrict__ sel, int top_k, int nqb, int nkb,                         \
      const float *__restrict__ S, const float *__restrict__ z, float eps, float scale,     \
      const T *__restrict__ dout, int64_t do_hs, float *__restrict__ dq, int64_t dq_hs,     \
      float *__restrict__ rs, int64_t nq_cap
#define HF_ROWS_PASS \
  q, n_q, q_hs, kg, vg, n_kv, kv_hs, sel, top_k, nqb, nkb, S, z, eps, scale, dout, do_hs, dq, dq_hs, rs, nq_cap

// Both passes and the linear read (fp32 states), at four waves per SIMD.
template <typename T, int D, int BLK>
__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(4))) void bwd_rows(
    HF_ROWS_ARGS) {
  rows_body<T, D, BLK>(HF_ROWS_PASS);
}

#undef HF_ROWS_ARGS
#undef HF_ROWS_PASS

template <typename T, int D, int BLK>
__global__ __launch_bounds__(BT) void bwd_kv(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ kg,
    const T* __restrict__ vg, int64_t n_kv, int64_t kv_hs, int nkb, float scale,
    const T* __restrict__ dout, int64_t do_hs, const float* __restrict__ rs, int64_t nq_cap,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ list, int nqb_cap,
    float* __restrict__ dk, float* __restrict__ dv, int64_t dkv_hs) {
  constexpr int RPW = kRows<BLK>, QT = RPW, SPLIT = BLK / RPW;
  constexpr int TPR = BT / RPW, DS = D / TPR;
  __shared__ __align__(16) float tq[QT * D];
  __shared__ __align__(16) float tdo[QT * D];
  __shared__ float tst[QT * 2];
  const int h = blockIdx.x / (nkb * SPLIT), jb = (blockIdx.x / SPLIT) % nkb;
  const int part = blockIdx.x % SPLIT;
  const int kl = threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * DS;
  const int64_t t = (int64_t)jb * BLK + part * RPW + kl;
  const bool live = t < n_kv;
  const int64_t tt = live ? t : n_kv - 1;
  const T* qh = q + (int64_t)h * q_hs;
  const T* doh = dout + (int64_t)h * do_hs;
  float kv[DS], vv[DS], gk[DS], gv[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    kv[e] = ldf(kg + (int64_t)h * kv_hs + tt * D + d0 + e);
    vv[e] = ldf(vg + (int64_t)h * kv_hs + tt * D + d0 + e);
    gk[e] = gv[e] = 0.f;
  }
  const float sl2 = scale * kL2e;
  const int64_t slot = (int64_t)h * nkb + jb;
  const int n_sel = cnt[slot];
  for (int x = 0; x < n_sel * SPLIT; ++x) {
    const int64_t q0 = (int64_t)list[slot * nqb_cap + x / SPLIT] * BLK + (x % SPLIT) * QT;
    if (q0 >= n_q) continue;  // the ragged last query block has no second half
    __syncthreads();
    load_tile<T, D, QT>(qh, q0, n_q, tq);
    load_tile<T, D, QT>(doh, q0, n_q, tdo);
    for (int e = threadIdx.x; e < QT; e += BT) {
      const int64_t r = q0 + e;
      const float* st = rs + ((int64_t)h * nq_cap + (r < n_q ? r : n_q - 1)) * 4;
      tst[2 * e] = st[0];
      tst[2 * e + 1] = st[1];
    }
    __syncthreads();
    const int nvalid = (int)min((int64_t)QT, n_q - q0);
    for (int u = 0; u < nvalid; ++u) {
      const float* qr = tq + u * D + d0;
      const float* dr = tdo + u * D + d0;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        s += kv[e] * qr[e];
        dp += vv[e] * dr[e];
      }
      s = row_sum<TPR>(s);
      dp = row_sum<TPR>(dp);
      const float p = exp2_hw(s * sl2 - tst[2 * u]);
      const float dl = scale * p * (dp - tst[2 * u + 1]);
#pragma unroll
      for (int e = 0; e < DS; ++e) {
        gv[e] += p * dr[e];
        gk[e] += dl * qr[e];
      }
    }
  }
  if (live) {
    float* ok = dk + (int64_t)h * dkv_hs + t * D + d0;
    float* ov = dv + (int64_t)h * dkv_hs + t * D + d0;
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      ok[e] = gk[e];
      ov[e] = gv[e];
    }
  }
}

// bf16 dq of the softmax path, staged as the forward attention kernel stages its tiles:
// one workgroup per (head, 64-row query block), 2 waves x 32 query rows, the selected
// blocks' K and V tiles loaded straight from global memory into LDS (16-byte global->LDS
// loads, swizzled rows), XCD-remapped like the forward launch. The Q and dO rows of a
// wave stay in registers as B operands. Two passes over the selected blocks:
//   1. S^T = K Q^T and dP^T = V dO^T (K and V rows by ds_read_b128), then, online per
//      query with a lazily moved reference max, l = sum exp2(s - m) and
//      D' = sum exp2(s - m) dP: lse = m + log2 l and D = D' / l (= dO . o_swa);
//   2. dP^T first (V rows; V(t+1) is then requested while K(t) is read), S^T, P =
//      exp2(s tau log2e - lse), dL^T = tau P^T (dP^T - D) split into bf16 hi + lo as B
//      operands in the key order of the S^T result layout, and dQ^T += K^T dL^T with K^T
//      by the transposing LDS read (the forward's V^T addressing on the K tile).
// Writes the softmax part of dq and (lse, D) per row; the linear read's part is added by
// bwd_rows_lin_mfma.
template <int D, bool SHORT>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq2(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const bf16_t* __restrict__ kg,
    const bf16_t* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int nkb, int n_logical, float scale, const bf16_t* __restrict__ dout,
    int64_t do_hs, float* __restrict__ dq, int64_t dq_hs, float* __restrict__ rs,
    int64_t nq_cap) {
  constexpr int BLK = 64, NW = 2, NQT = 2, NMT = 4, NET = D / 16, NKS = D / 32;
  constexpr int CPR = D / 8, TCH = BLK * CPR, LPT = TCH / (NW * 64);
  constexpr float kSlack = 8.f;  // the reference max moves when a score exceeds it by more
  typedef Mfma<bf16_t> M;
  __shared__ uint4 lds_k[TCH];
  __shared__ uint4 lds_v[TCH];
  const int logical = xcd_remap(blockIdx.x, gridDim.x, n_logical);
  if (logical < 0) return;
  const int h = logical / nqb, i = logical % nqb;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const bf16_t* qh = q + (int64_t)h * q_hs;
  const bf16_t* kh = kg + (int64_t)h * kv_hs;
  const bf16_t* vh = vg + (int64_t)h * kv_hs;
  const bf16_t* doh = dout + (int64_t)h * do_hs;
  const int32_t* my_sel = sel + ((int64_t)h * nqb + i) * top_k;
  const int64_t qrow0 = (int64_t)i * BLK + w * 32;
  const float sl2 = scale * kL2e;

  // ---- tile staging (as the forward kernel) ----
  constexpr int RPU = NW * 64 / CPR;
  constexpr int NPAT = RPU % 16 == 0 ? 1 : 2;
  uint32_t lpat[NPAT];
#pragma unroll
  for (int u = 0; u < NPAT; ++u) {
    const int P = (u * NW + w) * 64 + lane;
    const int row = P / CPR, cc = (P % CPR) ^ swz<CPR>(row);
    lpat[u] = (uint32_t)((row - u * RPU) * D + cc * 8) * 2u;
  }
  auto tile_row0 = [&](int jb) {
    const int64_t r0 = (int64_t)jb * BLK;
    return (!SHORT && r0 + BLK > n_kv) ? n_kv - BLK : r0;
  };
  auto issue_tile = [&](const bf16_t* src, int jb, const uint4* tile) {
    const bf16_t* tb = src + (size_t)tile_row0(jb) * D;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(tile) + w * 64 * 16);
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const uint32_t off = lpat[u % NPAT];
      if constexpr (!SHORT) {
        lds_dma16(tb + u * RPU * D, off, base + u * NW * 64 * 16);
      } else {
        const uint32_t row_bytes = D * 2, row = u * RPU + off / row_bytes;
        const uint32_t last = (uint32_t)(n_kv - 1 - tile_row0(jb));
        lds_dma16(tb, (row <= last ? row : last) * row_bytes + off % row_bytes,
                  base + u * NW * 64 * 16);
      }
    }
  };
  // keys of the tile that lie outside block jb (ragged last block): -inf
  auto mask = [&](int jb, f32x4 (&st)[NMT][NQT]) {
    const int64_t key0 = (int64_t)jb * BLK;
    if (key0 + BLK > n_kv) {
      const int valid = (int)(n_kv - key0);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = mt * 16 + g * 4 + r;
          const bool out = SHORT ? tr >= valid : tr < BLK - valid;
#pragma unroll
          for (int n = 0; n < NQT; ++n) st[mt][n][r] = out ? -INFINITY : st[mt][n][r];
        }
    }
  };

  int jb = clamp_block(my_sel[0], nkb);
  issue_tile(vh, jb, lds_v);
  issue_tile(kh, jb, lds_k);

  // Q and dO operands: lane holds row 16n + c, features 32s + 8g .. + 8
  bf16x8 qop[NQT][NKS], dop[NQT][NKS];
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int64_t r = qrow0 + n * 16 + c;
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      qop[n][s2] = as_bf16x8(ld16(qh + r * D + s2 * 32 + g * 8, r < n_q));
      dop[n][s2] = as_bf16x8(ld16(doh + r * D + s2 * 32 + g * 8, r < n_q));
    }
  }
  // LDS byte addresses: K / V rows (key tile mt adds mt * kRow16), K^T (chunk c2 adds
  // 2 c2 kRow16, its second half one more kRow16)
  constexpr uint32_t kRow16 = 16 * CPR * 16;
  uint32_t kaddr[NKS], vaddr[NKS], taddr[NET];
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2) {
    const uint32_t o = (uint32_t)(c * CPR + ((s2 * 4 + g) ^ swz<CPR>(c))) * 16u;
    kaddr[s2] = lds_offset(lds_k) + o;
    vaddr[s2] = lds_offset(lds_v) + o;
  }
  {
    const int rv = 4 * g + ((lane & 15) >> 2), pp = lane & 3;
#pragma unroll
    for (int et = 0; et < NET; ++et)
      taddr[et] = lds_offset(lds_k) +
                  (uint32_t)(rv * CPR + ((2 * et + (pp >> 1)) ^ swz<CPR>(rv))) * 16u + (pp & 1) * 8u;
  }
  // products of one tile: st (K rows x Q) or dp (V rows x dO)
  auto rows_x = [&](const uint32_t (&addr)[NKS], const bf16x8 (&op)[NQT][NKS],
                    f32x4 (&out)[NMT][NQT]) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int n = 0; n < NQT; ++n) out[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      bf16x8 a[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) a[mt] = as_bf16x8(lds_ld16(addr[s2] + mt * kRow16));
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int n = 0; n < NQT; ++n) out[mt][n] = M::mma(a[mt], op[n][s2], out[mt][n]);
    }
  };

  // ---- pass 1: lse and D ----
  float m_run[NQT], l_part[NQT], d_part[NQT];
#pragma unroll
  for (int n = 0; n < NQT; ++n) m_run[n] = l_part[n] = d_part[n] = 0.f;
  for (int t = 0; t < top_k; ++t) {
    const bool more = t + 1 < top_k;
    // the next block, or pass 2's first block after the last one
    const int jb_next = clamp_block(my_sel[more ? t + 1 : 0], nkb);
    wait_vmem<0>();
    lds_barrier();
    // products and tile requests at a raised issue priority, the VALU work at the
    // normal one (as in the forward kernel: the SIMD's waves drift into different phases)
    __builtin_amdgcn_s_setprio(2);
    f32x4 st[NMT][NQT], dp[NMT][NQT];
    rows_x(kaddr, qop, st);
    rows_x(vaddr, dop, dp);
    lds_barrier();  // every wave has read both tiles
    issue_tile(vh, jb_next, lds_v);
    issue_tile(kh, jb_next, lds_k);
    __builtin_amdgcn_s_setprio(0);
    mask(jb, st);
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      float mxr = -INFINITY;  // on the unscaled scores (sl2 > 0 keeps the order)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mxr = fmaxf(mxr, st[mt][n][r]);
      const float mx = mxr * sl2;
      if (t == 0) m_run[n] = max_over_groups(mx);  // finite: a block holds a window key
      if (__builtin_amdgcn_ballot_w64(mx - m_run[n] > kSlack)) {  // wave-uniform
        const float d_blk = max_over_groups(mx) - m_run[n];
        const float shift = d_blk > kSlack ? d_blk : 0.f;
        const float a = exp2_hw(-shift);
        m_run[n] += shift;
        l_part[n] *= a;
        d_part[n] *= a;
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2_hw(__builtin_fmaf(st[mt][n][r], sl2, -m_run[n]));
          l_part[n] += e;
          d_part[n] += e * dp[mt][n][r];
        }
    }
    jb = jb_next;
  }
  float lse2[NQT], Dr[NQT];
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const float l = sum_over_groups(l_part[n]);
    lse2[n] = m_run[n] + log2f(l);
    Dr[n] = sum_over_groups(d_part[n]) / l;
  }

  // ---- pass 2: dQ^T += K^T dL^T ----
  f32x4 gT[NET][NQT];
#pragma unroll
  for (int e = 0; e < NET; ++e)
#pragma unroll
    for (int n = 0; n < NQT; ++n) gT[e][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < top_k; ++t) {
    const bool more = t + 1 < top_k;
    const int jb_next = more ? clamp_block(my_sel[t + 1], nkb) : 0;
    wait_vmem<LPT>();  // V(t) has landed (K(t) may be in flight)
    lds_barrier();
    __builtin_amdgcn_s_setprio(2);  // dP and S products, tile requests (dQ products: normal)
    f32x4 dp[NMT][NQT];
    rows_x(vaddr, dop, dp);
    lds_barrier();  // every wave has read V(t)
    if (more) {
      issue_tile(vh, jb_next, lds_v);
      wait_vmem<LPT>();  // K(t) has landed (V(t+1) may be in flight)
    } else {
      wait_vmem<0>();
    }
    lds_barrier();
    f32x4 st[NMT][NQT];
    rows_x(kaddr, qop, st);
    __builtin_amdgcn_s_setprio(0);
    mask(jb, st);
    // dL in the key order of the result layout, split into bf16 hi + lo
    bf16x8 lh[2][NQT], ll[2][NQT];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        float lv[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          lv[r] = exp2_hw(st[2 * c2][n][r] * sl2 - lse2[n]) * (dp[2 * c2][n][r] - Dr[n]);
          lv[4 + r] = exp2_hw(st[2 * c2 + 1][n][r] * sl2 - lse2[n]) * (dp[2 * c2 + 1][n][r] - Dr[n]);
        }
        split_bf16x8(lv, lh[c2][n], ll[c2][n]);
      }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      bf16x8 kt[NET];
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const v4i16 lo = lds_tr8(taddr[et] + 2 * c2 * kRow16);
        const v4i16 hi = lds_tr8(taddr[et] + (2 * c2 + 1) * kRow16);
        kt[et] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int n = 0; n < NQT; ++n) {
          gT[et][n] = M::mma(kt[et], lh[c2][n], gT[et][n]);
          gT[et][n] = M::mma(kt[et], ll[c2][n], gT[et][n]);
        }
    }
    lds_barrier();  // every wave has read K(t)
    __builtin_amdgcn_s_setprio(2);
    if (more) issue_tile(kh, jb_next, lds_k);
    __builtin_amdgcn_s_setprio(0);
    jb = jb_next;
  }
  // lane holds dq[row 16n + c][16 et + 4g .. + 3] / tau (dL went in without tau)
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int64_t r = qrow0 + n * 16 + c;
    if (r >= n_q) continue;
    float* o = dq + (int64_t)h * dq_hs + r * D;
#pragma unroll
    for (int et = 0; et < NET; ++et)
      *reinterpret_cast<float4*>(o + 16 * et + 4 * g) =
          make_float4(scale * gT[et][n][0], scale * gT[et][n][1], scale * gT[et][n][2],
                      scale * gT[et][n][3]);
    if (g == 0) {
      float* st = rs + ((int64_t)h * nq_cap + r) * 4;
      st[0] = lse2[n];
      st[1] = Dr[n];
    }
  }
}

// bf16 dk and dv with the forward kernel's tile staging: one workgroup per (head, 64-key
// block), 4 waves x 16 keys (K and V of the wave's keys stay in registers as B
// operands), over the query blocks that selected the block. Per query block its Q and
// dO tiles are loaded straight from global memory into LDS (16-byte global->LDS loads,
// swizzled rows; rows past the chunk repeat its last row and get weight 0). dP = dO V^T
// (dO rows by ds_read_b128) comes first, then S = Q K^T (Q rows), P = exp2(s tau log2e
// - lse), dL = tau P (dP - D); P and dL become B operands (bf16 hi + lo) in the query
// order of the result layout; dV^T += dO^T P and dK^T += Q^T dL with dO^T and Q^T by the
// transposing LDS read. The dO tile is released (and the next one requested) before the
// dK products, the Q tile after them.
template <int D>
__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_kv2(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const bf16_t* __restrict__ kg,
    const bf16_t* __restrict__ vg, int64_t n_kv, int64_t kv_hs, int nkb, float scale,
    const bf16_t* __restrict__ dout, int64_t do_hs, const float* __restrict__ rs, int64_t nq_cap,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ list, int nqb_cap,
    float* __restrict__ dk, float* __restrict__ dv, int64_t dkv_hs) {
  constexpr int BLK = 64, NW = 4, NMQ = 4, NET = D / 16, NKS = D / 32;
  constexpr int CPR = D / 8, TCH = BLK * CPR, LPT = TCH / (NW * 64);
  typedef Mfma<bf16_t> M;
  __shared__ uint4 lds_q[TCH];
  __shared__ uint4 lds_o[TCH];
  __shared__ uint4 lds_st[NW][BLK];  // per wave: the block's rows of the statistics
  const int h = blockIdx.x / nkb, jb = blockIdx.x % nkb;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const float sl2 = scale * kL2e;
  const int64_t key = (int64_t)jb * BLK + w * 16 + c;
  const bool kvalid = key < n_kv;
  bf16x8 kop[NKS], vop[NKS];
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2) {
    const int64_t off = (int64_t)h * kv_hs + key * D + 32 * s2 + 8 * g;
    kop[s2] = as_bf16x8(ld16(kg + off, kvalid));
    vop[s2] = as_bf16x8(ld16(vg + off, kvalid));
  }
  const bf16_t* qh = q + (int64_t)h * q_hs;
  const bf16_t* doh = dout + (int64_t)h * do_hs;
  const int64_t slot = (int64_t)h * nkb + jb;
  const int n_sel = cnt[slot];
  const int32_t* my_list = list + slot * nqb_cap;

  // tile loads: load u of this wave fills LDS chunks (u NW + w) 64 + lane with chunk
  // (row, slot ^ swz(row)); rows past the chunk read its last row
  constexpr int RPU = NW * 64 / CPR;
  uint32_t lrow[LPT], lcol[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int P = (u * NW + w) * 64 + lane;
    const int row = P / CPR, cc = (P % CPR) ^ swz<CPR>(row);
    lrow[u] = (uint32_t)row;
    lcol[u] = (uint32_t)cc * 16u;
  }
  static_assert(RPU >= 1, "rows per load");
  auto issue = [&](const bf16_t* src, int64_t q0, const uint4* tile) {
    const uint32_t last = (uint32_t)(n_q - 1 - q0);
    const bf16_t* tb = src + (size_t)q0 * D;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(tile) + w * 64 * 16);
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const uint32_t row = lrow[u] <= last ? lrow[u] : last;
      lds_dma16(tb, row * (uint32_t)(D * 2) + lcol[u], base + u * NW * 64 * 16);
    }
  };
  constexpr uint32_t kRow16 = 16 * CPR * 16;
  uint32_t qaddr[NKS], oaddr[NKS], tq[NET], to[NET];
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2) {
    const uint32_t o = (uint32_t)(c * CPR + ((s2 * 4 + g) ^ swz<CPR>(c))) * 16u;
    qaddr[s2] = lds_offset(lds_q) + o;
    oaddr[s2] = lds_offset(lds_o) + o;
  }
  {
    const int rv = 4 * g + ((lane & 15) >> 2), pp = lane & 3;
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      const uint32_t o = (uint32_t)(rv * CPR + ((2 * et + (pp >> 1)) ^ swz<CPR>(rv))) * 16u +
                         (pp & 1) * 8u;
      tq[et] = lds_offset(lds_q) + o;
      to[et] = lds_offset(lds_o) + o;
    }
  }
  auto rows_x = [&](const uint32_t (&addr)[NKS], const bf16x8 (&op)[NKS], f32x4 (&out)[NMQ]) {
#pragma unroll
    for (int m = 0; m < NMQ; ++m) out[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      bf16x8 a[NMQ];
#pragma unroll
      for (int m = 0; m < NMQ; ++m) a[m] = as_bf16x8(lds_ld16(addr[s2] + m * kRow16));
#pragma unroll
      for (int m = 0; m < NMQ; ++m) out[m] = M::mma(a[m], op[s2], out[m]);
    }
  };
  // statistics rows (16 bytes each) of query rows q0 .. q0 + 63 into this wave's copy
  const float* rsh = rs + (int64_t)h * nq_cap * 4;
  const uint32_t st_base = __builtin_amdgcn_readfirstlane(lds_offset(&lds_st[w][0]));
  auto issue_st = [&](int64_t q0) {
    const uint32_t last = (uint32_t)(n_q - 1 - q0);
    const uint32_t row = (uint32_t)lane <= last ? (uint32_t)lane : last;
    lds_dma16(rsh + q0 * 4, row * 16u, st_base);
  };
  auto tr_ops = [&](const uint32_t (&addr)[NET], int c2, bf16x8 (&out)[NET]) {
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      const v4i16 lo = lds_tr8(addr[et] + 2 * c2 * kRow16);
      const v4i16 hi = lds_tr8(addr[et] + (2 * c2 + 1) * kRow16);
      out[et] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };

  f32x4 dvT[NET], dkT[NET];
#pragma unroll
  for (int e = 0; e < NET; ++e) dvT[e] = dkT[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (n_sel > 0) {
    int64_t q0 = (int64_t)my_list[0] * BLK;
    issue(doh, q0, lds_o);
    issue_st(q0);
    issue(qh, q0, lds_q);
    for (int x = 0; x < n_sel; ++x) {
      const bool more = x + 1 < n_sel;
      const int64_t q0n = more ? (int64_t)my_list[x + 1] * BLK : 0;
      const int n_valid = n_q - q0 < BLK ? (int)(n_q - q0) : BLK;  // rows past: weight 0
      wait_vmem<LPT>();  // dO(x) and the statistics have landed (Q(x) may be in flight)
      lds_barrier();
      f32x4 dp[NMQ];
      rows_x(oaddr, vop, dp);
      wait_vmem<0>();  // Q(x)
      lds_barrier();
      f32x4 sc[NMQ];
      rows_x(qaddr, kop, sc);
      // P and dL in the query order of the result layout (lane: queries 4g .. 4g + 3 of
      // tiles 2c2 and 2c2 + 1, key c), split into bf16 hi + lo
      // (dL without tau, which the result takes once; rows past the chunk, in its last
      // query block only, get weight 0)
      bf16x8 ph[2], pl[2], lh[2], ll[2];
      auto weights = [&](auto masked) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          float pv[8], lv[8];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int m = 2 * c2 + hf, ql = 16 * m + 4 * g + r;
              const float2 st = lds_ld8f(st_base + ql * 16u);
              float p = exp2_hw(sc[m][r] * sl2 - st.x);
              if constexpr (decltype(masked)::value) p = ql < n_valid ? p : 0.f;
              pv[4 * hf + r] = p;
              lv[4 * hf + r] = p * (dp[m][r] - st.y);
            }
          split_bf16x8(pv, ph[c2], pl[c2]);
          split_bf16x8(lv, lh[c2], ll[c2]);
        }
      };
      if (n_valid < BLK) weights(std::true_type{});
      else weights(std::false_type{});
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 a[NET];
        tr_ops(to, c2, a);
#pragma unroll
        for (int et = 0; et < NET; ++et) {
          dvT[et] = M::mma(a[et], ph[c2], dvT[et]);
          dvT[et] = M::mma(a[et], pl[c2], dvT[et]);
        }
      }
      lds_barrier();  // every wave has read dO(x)
      if (more) {
        issue(doh, q0n, lds_o);
        issue_st(q0n);
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 a[NET];
        tr_ops(tq, c2, a);
#pragma unroll
        for (int et = 0; et < NET; ++et) {
          dkT[et] = M::mma(a[et], lh[c2], dkT[et]);
          dkT[et] = M::mma(a[et], ll[c2], dkT[et]);
        }
      }
      lds_barrier();  // every wave has read Q(x)
      if (more) issue(qh, q0n, lds_q);
      q0 = q0n;
    }
  }
  if (kvalid) {
    float* pk = dk + (int64_t)h * dkv_hs + key * D;
    float* pv = dv + (int64_t)h * dkv_hs + key * D;
#pragma unroll
    for (int e = 0; e < NET; ++e) {
      *reinterpret_cast<float4*>(pk + 16 * e + 4 * g) =  // dL went in without tau
          make_float4(scale * dkT[e][0], scale * dkT[e][1], scale * dkT[e][2], scale * dkT[e][3]);
      *reinterpret_cast<float4*>(pv + 16 * e + 4 * g) =
          make_float4(dvT[e][0], dvT[e][1], dvT[e][2], dvT[e][3]);
    }
  }
}

// Workgroup (h, jt): jt < D / NJ forms dS rows NJ jt .. NJ jt + NJ - 1, jt == D / NJ forms
// dz. Four rows per workgroup: 33 workgroups per head at d = 128, so that the grid
// covers the compute units.
constexpr int kStateRows = 4;
template <typename T, int D>
__global__ __launch_bounds__(BT) void bwd_state(const T* __restrict__ q, int64_t n_q,
                                                int64_t q_hs, const T* __restrict__ dout,
                                                int64_t do_hs, const float* __restrict__ rs,
                                                int64_t nq_cap, float* __restrict__ dS,
                                                float* __restrict__ dz) {
  constexpr int RC = 32, NJ = kStateRows, JPT = NJ * D / BT;  // rows/chunk, dS rows, outs/thread
  __shared__ __align__(16) float tf[RC * D];
  __shared__ float tg[RC * NJ];
  constexpr int NT = D / NJ + 1;
  const int h = blockIdx.x / NT, jt = blockIdx.x % NT;
  const bool is_z = jt == D / NJ;
  const int col = threadIdx.x % D, j0 = threadIdx.x / D;  // rows j0, j0 + BT/D, ...
  const T* qh = q + (int64_t)h * q_hs;
  const T* doh = dout + (int64_t)h * do_hs;
  const float* rsh = rs + (int64_t)h * nq_cap * 4;
  float a[JPT];
#pragma unroll
  for (int e = 0; e < JPT; ++e) a[e] = 0.f;
  for (int64_t r0 = 0; r0 < n_q; r0 += RC) {
    __syncthreads();
    load_tile<T, D, RC, true>(qh, r0, n_q, tf);
    for (int e = threadIdx.x; e < RC * NJ; e += BT) {
      const int64_t r = r0 + e / NJ;
      float g = 0.f;
      if (r < n_q) {
        const float* st = rsh + r * 4;
        g = is_z ? (e % NJ == 0 ? st[3] : 0.f)
                 : ldf(doh + r * D + jt * NJ + (e % NJ)) / st[2];
      }
      tg[e] = g;
    }
    __syncthreads();
    const int nr = (int)min((int64_t)RC, n_q - r0);
    for (int u = 0; u < nr; ++u) {
      const float f = tf[u * D + col];
#pragma unroll
      for (int e = 0; e < JPT; ++e) a[e] += tg[u * NJ + j0 + e * (BT / D)] * f;
    }
  }
  if (is_z) {
    if (j0 == 0) dz[(int64_t)h * D + col] = a[0];
  } else {
#pragma unroll
    for (int e = 0; e < JPT; ++e)
      dS[((int64_t)h * D + jt * NJ + j0 + e * (BT / D)) * D + col] = a[e];
  }
}

template <typename T, int D>
__global__ __launch_bounds__(BT) void absorb_bwd(const T* __restrict__ k, const T* __restrict__ v,
                                                 int64_t n_ev, int64_t ev_hs,
                                                 const float* __restrict__ dS,
                                                 const float* __restrict__ dz,
                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                 int64_t dev_hs, int ntile) {
  constexpr int BLK = 64, TPR = BT / BLK, DS = D / TPR;
  __shared__ __align__(16) float tf[BLK * D];
  __shared__ __align__(16) float tv[BLK * D];
  __shared__ __align__(16) float tS[D * D];  // dS of the head, read by every token
  const int h = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int nl = threadIdx.x / TPR, d0 = (threadIdx.x % TPR) * DS;
  const int64_t n = (int64_t)tile * BLK + nl;
  const bool live = n < n_ev;
  const int64_t nn = live ? n : n_ev - 1;
  const float* zh = dz + (int64_t)h * D;
  for (int e = threadIdx.x; e < D * D / 4; e += BT)
    reinterpret_cast<float4*>(tS)[e] =
        reinterpret_cast<const float4*>(dS + (int64_t)h * D * D)[e];
  const float* Sh = tS;
  float kx[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    kx[e] = ldf(k + (int64_t)h * ev_hs + nn * D + d0 + e);
    tf[nl * D + d0 + e] = phi(kx[e]);
    tv[nl * D + d0 + e] = ldf(v + (int64_t)h * ev_hs + nn * D + d0 + e);
  }
  __syncthreads();
  const float* frow = tf + nl * D;
  const float* vrow = tv + nl * D;
  float ov[DS], ok[DS];
#pragma unroll
  for (int e = 0; e < DS; ++e) ov[e] = ok[e] = 0.f;
#pragma unroll 2
  for (int c4 = 0; c4 < D; c4 += 4) {  // dv[j] = dS[j] . phi(k), column chunk by chunk
    const float4 f4 = *reinterpret_cast<const float4*>(frow + c4);
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      const float4 s4 = *reinterpret_cast<const float4*>(Sh + (int64_t)(d0 + e) * D + c4);
      ov[e] += s4.x * f4.x + s4.y * f4.y + s4.z * f4.z + s4.w * f4.w;
    }
  }
#pragma unroll 2
  for (int j = 0; j < D; ++j) {  // dk[i] = phi'(k_i) (sum_j v_j dS[j][i] + dz[i])
    const float vj = vrow[j];
    const float* srow = Sh + (int64_t)j * D + d0;
#pragma unroll
    for (int e = 0; e < DS; e += 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(srow + e);
      ok[e] += vj * s4.x;
      ok[e + 1] += vj * s4.y;
      ok[e + 2] += vj * s4.z;
      ok[e + 3] += vj * s4.w;
    }
  }
  if (live) {
    float* pk = dk + (int64_t)h * dev_hs + n * D + d0;
    float* pv = dv + (int64_t)h * dev_hs + n * D + d0;
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      pk[e] = phi_prime(kx[e]) * (ok[e] + zh[d0 + e]);
      pv[e] = ov[e];
    }
  }
}

// bf16 absorb backward on MFMA (v_mfma_f32_16x16x32_bf16), one workgroup per (head,
// 64 evicted tokens), wave w owning the output feature tiles 2w, 2w + 1 of both
// gradients for all 64 tokens:
//   dv^T = dS Phi^T        (A = rows of dS, B = phi(k) of the tokens)
//   dk^T = dS^T V^T        (A = columns of dS, B = v of the tokens), then
//   dk   = phi'(k) (dk + dz).
// The fp32 operands (dS, phi(k)) are split into bf16 hi + lo and multiplied in three
// products (hi hi, lo hi, hi lo); v is exact bf16, so dk takes two. A lane's B
// operand is 8 consecutive features of one token (one 16-byte load of its row); its
// A operand is 8 consecutive entries of a row (dv) or a column (dk) of dS, read from
// global memory (dS is 64 KB per head and stays in cache). Results leave straight
// from the MFMA layout: 4 consecutive features of one token per lane.
template <int D>
__global__ __launch_bounds__(BT) void absorb_bwd_mfma(const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, int64_t n_ev,
                                                      int64_t ev_hs, const float* __restrict__ dS,
                                                      const float* __restrict__ dz,
                                                      float* __restrict__ dk, float* __restrict__ dv,
                                                      int64_t dev_hs, int ntile) {
  constexpr int NKS = D / 32, NT = 4, FT = D / 16 / 4;  // k-steps, token tiles, tiles per wave
  typedef Mfma<bf16_t> M;
  const int h = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const bf16_t* kh = k + (int64_t)h * ev_hs;
  const bf16_t* vh = v + (int64_t)h * ev_hs;
  const float* Sh = dS + (int64_t)h * D * D;
  const int64_t n0 = (int64_t)tile * 64;
  f32x4 av[FT][NT], ak[FT][NT];
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int t = 0; t < NT; ++t) av[f][t] = ak[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    // B operands of the 4 token tiles: phi(k) split, v exact
    bf16x8 fh[NT], fl[NT], vb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t n = n0 + 16 * t + c;
      const bool ok = n < n_ev;
      const uint4 kr = ok ? *reinterpret_cast<const uint4*>(kh + n * D + 32 * s + 8 * g) : zero4();
      const uint4 vr = ok ? *reinterpret_cast<const uint4*>(vh + n * D + 32 * s + 8 * g) : zero4();
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = ok ? phi(bf16_to_f32(half16(kr, e))) : 0.f;
      split_bf16x8(f, fh[t], fl[t]);
      vb[t] = as_bf16x8(vr);
    }
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const int ft = FT * w + f;  // output feature tile
      // A for dv: dS[16 ft + c][32 s + 8 g .. + 8]; for dk: dS[32 s + 8 g + e][16 ft + c]
      float ra[8], rc[8];
      const float4 r0 = *reinterpret_cast<const float4*>(Sh + (16 * ft + c) * D + 32 * s + 8 * g);
      const float4 r1 = *reinterpret_cast<const float4*>(Sh + (16 * ft + c) * D + 32 * s + 8 * g + 4);
      ra[0] = r0.x, ra[1] = r0.y, ra[2] = r0.z, ra[3] = r0.w;
      ra[4] = r1.x, ra[5] = r1.y, ra[6] = r1.z, ra[7] = r1.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) rc[e] = Sh[(32 * s + 8 * g + e) * D + 16 * ft + c];
      bf16x8 rh, rl, ch, cl;
      split_bf16x8(ra, rh, rl);
      split_bf16x8(rc, ch, cl);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        av[f][t] = M::mma(rh, fh[t], av[f][t]);
        av[f][t] = M::mma(rl, fh[t], av[f][t]);
        av[f][t] = M::mma(rh, fl[t], av[f][t]);
        ak[f][t] = M::mma(ch, vb[t], ak[f][t]);
        ak[f][t] = M::mma(cl, vb[t], ak[f][t]);
      }
    }
  }
  // lane holds features 16 ft + 4 g .. + 3 of token 16 t + c
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t n = n0 + 16 * t + c;
    if (n >= n_ev) continue;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      const int i0 = 16 * (FT * w + f) + 4 * g;
      *reinterpret_cast<float4*>(dv + (int64_t)h * dev_hs + n * D + i0) =
          make_float4(av[f][t][0], av[f][t][1], av[f][t][2], av[f][t][3]);
      const uint2 kq = *reinterpret_cast<const uint2*>(kh + n * D + i0);
      const float4 z4 = *reinterpret_cast<const float4*>(dz + (int64_t)h * D + i0);
      const float kx[4] = {bf16_to_f32(kq.x & 0xFFFFu), bf16_to_f32(kq.x >> 16),
                           bf16_to_f32(kq.y & 0xFFFFu), bf16_to_f32(kq.y >> 16)};
      *reinterpret_cast<float4*>(dk + (int64_t)h * dev_hs + n * D + i0) =
          make_float4(phi_prime(kx[0]) * (ak[f][t][0] + z4.x), phi_prime(kx[1]) * (ak[f][t][1] + z4.y),
                      phi_prime(kx[2]) * (ak[f][t][2] + z4.z), phi_prime(kx[3]) * (ak[f][t][3] + z4.w));
    }
  }
}

// bf16 linear-read part of dq on MFMA, one workgroup per (head, 64-row query block),
// wave w owning rows 16w .. 16w + 15 (one per lane c). With f = phi(q_r), den = z . f
// + eps and g = dout_r / den:
//   (S f)^T = S F^T           A = rows of S, B = f of the wave's rows,
//   c_r     = -(dout_r . S f) / den^2,
//   (S^T g)^T = S^T G^T       A = columns of S, B = g of the wave's rows,
//   dq_r   += phi'(q_r) (S^T g + c_r z),
// and den, c go to the per-row statistics for the dS / dz kernel. The bf16 hi/lo split
// of S (kept by the state for the forward epilogue) is staged in LDS; its rows are read
// with ds_read_b128, its columns with the transposing read (rows 4g .. 4g + 3 and
// 4g + 16 .. 4g + 19 of a 32-row step for lane group g, so g takes that order of the
// contracted index); f and g are split into hi + lo in registers; three products each.
template <int D>
__global__ __launch_bounds__(BT) void bwd_rows_lin_mfma(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const uint16_t* __restrict__ s_split,
    const float* __restrict__ z, float eps, const bf16_t* __restrict__ dout, int64_t do_hs,
    float* __restrict__ dq, int64_t dq_hs, float* __restrict__ rs, int64_t nq_cap, int nqb) {
  constexpr int NKS = D / 32, NT = D / 16, RSB = D + 16;
  typedef Mfma<bf16_t> M;
  __shared__ __align__(16) bf16_t sS[2 * D * RSB];  // hi rows, then lo rows
  const int h = blockIdx.x / nqb, i = blockIdx.x % nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t r = (int64_t)i * 64 + 16 * w + c;
  const bool live = r < n_q;
  const int64_t rr = live ? r : n_q - 1;
  const bf16_t* qr = q + (int64_t)h * q_hs + rr * D;
  const bf16_t* dr = dout + (int64_t)h * do_hs + rr * D;
  const float* zh = z + (int64_t)h * D;
  // stage the split of S
  const uint16_t* Ssp = s_split + (int64_t)h * 2 * D * D;
  for (int x = threadIdx.x; x < 2 * D * (D / 8); x += BT) {
    const int row = x / (D / 8), ch = x % (D / 8);  // row of [hi; lo]
    *reinterpret_cast<uint4*>(sS + row * RSB + ch * 8) =
        *reinterpret_cast<const uint4*>(Ssp + (int64_t)row * D + ch * 8);
  }
  // f of this lane's row in k-step order (B operand of S F^T) and den
  bf16x8 fhi[NKS], flo[NKS];
  float qv[NKS][8];
  float den = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2) {
    const uint4 qb = *reinterpret_cast<const uint4*>(qr + 32 * s2 + 8 * g);
    const float4 z0 = *reinterpret_cast<const float4*>(zh + 32 * s2 + 8 * g);
    const float4 z1 = *reinterpret_cast<const float4*>(zh + 32 * s2 + 8 * g + 4);
    const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[s2][e] = bf16_to_f32(half16(qb, e));
      f[e] = phi(qv[s2][e]);
      den += zz[e] * f[e];
    }
    split_bf16x8(f, fhi[s2], flo[s2]);
  }
  den = sum_over_groups(den) + eps;
  const float inv_den = 1.f / den;
  // g of this lane's row in the transposing read's order of the contracted index
  bf16x8 ghi[NKS], glo[NKS];
#pragma unroll
  for (int s2 = 0; s2 < NKS; ++s2) {
    const uint2 a = *reinterpret_cast<const uint2*>(dr + 32 * s2 + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2*>(dr + 32 * s2 + 4 * g + 16);
    const uint32_t wv[4] = {a.x, a.y, b.x, b.y};
    float gv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = bf16_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) * inv_den;
    split_bf16x8(gv, ghi[s2], glo[s2]);
  }
  __syncthreads();
  const uint32_t sb = lds_offset(sS);
  // (S f)^T tiles and c_r
  float cpart = 0.f;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) {
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      const uint32_t o = (uint32_t)((16 * jt + c) * RSB + 32 * s2 + 8 * g) * 2u;
      const bf16x8 sh = as_bf16x8(lds_ld16(sb + o));
      const bf16x8 sl = as_bf16x8(lds_ld16(sb + o + (uint32_t)D * RSB * 2u));
      a = M::mma(sh, fhi[s2], a);
      a = M::mma(sl, fhi[s2], a);
      a = M::mma(sh, flo[s2], a);
    }
    // lane holds (S f)[16 jt + 4 g + 0..3] of its row
    const uint2 dv2 = *reinterpret_cast<const uint2*>(dr + 16 * jt + 4 * g);
    cpart += bf16_to_f32(dv2.x & 0xFFFFu) * a[0] + bf16_to_f32(dv2.x >> 16) * a[1] +
             bf16_to_f32(dv2.y & 0xFFFFu) * a[2] + bf16_to_f32(dv2.y >> 16) * a[3];
  }
  const float cr = -sum_over_groups(cpart) * inv_den * inv_den;
  // (S^T g)^T tiles and the update of dq
  const int jj = (lane & 15) >> 2, pp = lane & 3;
  const uint32_t row_lo = (uint32_t)(4 * g + jj) * RSB * 2u + pp * 8u;
  const uint32_t row_hi = row_lo + 16u * RSB * 2u;
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      const uint32_t b = sb + (uint32_t)(32 * s2 * RSB) * 2u + it * 32u;
      const v4i16 h0 = lds_tr8(b + row_lo), h1 = lds_tr8(b + row_hi);
      const v4i16 l0 = lds_tr8(b + row_lo + (uint32_t)D * RSB * 2u);
      const v4i16 l1 = lds_tr8(b + row_hi + (uint32_t)D * RSB * 2u);
      const bf16x8 th = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
      const bf16x8 tl = __builtin_bit_cast(bf16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
      a = M::mma(th, ghi[s2], a);
      a = M::mma(tl, ghi[s2], a);
      a = M::mma(th, glo[s2], a);
    }
    if (live) {  // lane holds (S^T g)[16 it + 4 g + 0..3] of its row
      const int i0 = 16 * it + 4 * g;
      const uint2 qq = *reinterpret_cast<const uint2*>(qr + i0);
      const float4 z4 = *reinterpret_cast<const float4*>(zh + i0);
      float* o = dq + (int64_t)h * dq_hs + r * D + i0;
      const float4 prev = *reinterpret_cast<const float4*>(o);
      *reinterpret_cast<float4*>(o) = make_float4(
          prev.x + phi_prime(bf16_to_f32(qq.x & 0xFFFFu)) * (a[0] + cr * z4.x),
          prev.y + phi_prime(bf16_to_f32(qq.x >> 16)) * (a[1] + cr * z4.y),
          prev.z + phi_prime(bf16_to_f32(qq.y & 0xFFFFu)) * (a[2] + cr * z4.z),
          prev.w + phi_prime(bf16_to_f32(qq.y >> 16)) * (a[3] + cr * z4.w));
    }
  }
  if (live && g == 0) {
    float* st = rs + ((int64_t)h * nq_cap + r) * 4;
    st[2] = den;
    st[3] = cr;
  }
}

// bf16 dS and dz on MFMA: dS = G^T F and dz = F^T c over the query rows, where
// g_r = dout_r / den_r, f_r = phi(q_r) and c_r come from the per-row statistics of
// the linear read. One workgroup per (head, chunk of kStateChunk rows) writes the
// chunk's partial dS and dz; bwd_state_reduce adds the chunks in order (no atomics).
// Per 32-row k-step the workgroup forms g and f once (fp32, split into bf16 hi + lo)
// into LDS row-major; both MFMA operands are then 8 rows of one column, read with the
// transposing LDS read (rows 4g .. 4g + 3 and 4g + 16 .. 4g + 19 of the step for lane
// group g, the same row order for both operands), and each dS tile takes three
// products (hi hi, lo hi, hi lo). Wave w owns dS rows 32w .. 32w + 31 (two 16-row
// tiles at d = 128) against all columns.
constexpr int kStateChunk = kBwdStateChunk;
template <int D>
__global__ __launch_bounds__(BT) void bwd_state_mfma(const bf16_t* __restrict__ q, int64_t n_q,
                                                     int64_t q_hs, const bf16_t* __restrict__ dout,
                                                     int64_t do_hs, const float* __restrict__ rs,
                                                     int64_t nq_cap, float* __restrict__ part,
                                                     int n_chunk) {
  constexpr int NT = D / 16, JT = NT / 4;  // column tiles; row tiles per wave
  constexpr int RSB = D + 16;               // LDS row stride (bf16): conflict-free transposing reads
  constexpr int CPT = 32 * (D / 8) / BT;    // 16-byte chunks per thread per step
  typedef Mfma<bf16_t> M;
  __shared__ __align__(16) bf16_t gh[32 * RSB], gl[32 * RSB], fh[32 * RSB], fl[32 * RSB];
  __shared__ float zred[BT / (D / 8)][D];
  const int h = blockIdx.x / n_chunk, p = blockIdx.x % n_chunk;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const bf16_t* qh = q + (int64_t)h * q_hs;
  const bf16_t* doh = dout + (int64_t)h * do_hs;
  const float* rsh = rs + (int64_t)h * nq_cap * 4;
  // staging: thread's chunk ch (8 features) of rows rr, rr + BT / (D / 8), ...
  const int ch = threadIdx.x % (D / 8), rr = threadIdx.x / (D / 8);
  float zacc[8] = {};
  f32x4 acc[JT][NT];
#pragma unroll
  for (int j = 0; j < JT; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // transposing-read addresses: lane (4jj + pp) of group g -> row 4g + jj, columns 4pp ..
  const int jj = (lane & 15) >> 2, pp = lane & 3;
  const uint32_t row_lo = (uint32_t)(4 * g + jj) * RSB * 2u + pp * 8u;
  const uint32_t row_hi = row_lo + 16u * RSB * 2u;
  auto tr_op = [&](const bf16_t* base, int col_tile) {
    const uint32_t b = lds_offset(base) + col_tile * 32u;
    const v4i16 lo = lds_tr8(b + row_lo), hi = lds_tr8(b + row_hi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  const int64_t r_begin = (int64_t)p * kStateChunk;
  const int64_t r_end = r_begin + kStateChunk < n_q ? r_begin + kStateChunk : n_q;
  for (int64_t r0 = r_begin; r0 < r_end; r0 += 32) {
    __syncthreads();  // every wave is done with the previous step's operands
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int row = rr + u * (BT / (D / 8));
      const int64_t r = r0 + row;
      float f[8], gv[8];
      if (r < r_end) {
        const uint4 qb = *reinterpret_cast<const uint4*>(qh + r * D + ch * 8);
        const uint4 db = *reinterpret_cast<const uint4*>(doh + r * D + ch * 8);
        const float inv_den = 1.f / rsh[r * 4 + 2], cr = rsh[r * 4 + 3];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = phi(bf16_to_f32(half16(qb, e)));
          gv[e] = bf16_to_f32(half16(db, e)) * inv_den;
          zacc[e] += cr * f[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = gv[e] = 0.f;
      }
      bf16x8 a, b, x, y;
      split_bf16x8(gv, a, b);
      split_bf16x8(f, x, y);
      *reinterpret_cast<bf16x8*>(gh + row * RSB + ch * 8) = a;
      *reinterpret_cast<bf16x8*>(gl + row * RSB + ch * 8) = b;
      *reinterpret_cast<bf16x8*>(fh + row * RSB + ch * 8) = x;
      *reinterpret_cast<bf16x8*>(fl + row * RSB + ch * 8) = y;
    }
    __syncthreads();
    bf16x8 ah[JT], al[JT];
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      ah[j] = tr_op(gh, JT * w + j);
      al[j] = tr_op(gl, JT * w + j);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 bh = tr_op(fh, t), bl = tr_op(fl, t);
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        acc[j][t] = M::mma(ah[j], bh, acc[j][t]);
        acc[j][t] = M::mma(al[j], bh, acc[j][t]);
        acc[j][t] = M::mma(ah[j], bl, acc[j][t]);
      }
    }
  }
  // partial dS of the chunk in MFMA order: [tile (row tile, column tile)][lane][4]
  float* ph = part + ((int64_t)h * n_chunk + p) * (D * D + D);
#pragma unroll
  for (int j = 0; j < JT; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      *reinterpret_cast<float4*>(ph + ((JT * w + j) * NT + t) * 256 + lane * 4) =
          make_float4(acc[j][t][0], acc[j][t][1], acc[j][t][2], acc[j][t][3]);
  // partial dz: the staging threads' column sums, added in thread order
#pragma unroll
  for (int e = 0; e < 8; ++e) zred[rr][ch * 8 + e] = zacc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float z = 0.f;
    for (int k = 0; k < BT / (D / 8); ++k) z += zred[k][threadIdx.x];
    ph[D * D + threadIdx.x] = z;
  }
}

// dS and dz from the chunks' partials, added in chunk order.
template <int D>
__global__ __launch_bounds__(BT) void bwd_state_reduce(const float* __restrict__ part,
                                                       int n_chunk, float* __restrict__ dS,
                                                       float* __restrict__ dz) {
  constexpr int NT = D / 16, PER = D * D + D;
  const int h = blockIdx.y;
  const int x = blockIdx.x * BT + threadIdx.x;  // element of a partial
  if (x >= PER) return;
  const float* ph = part + (int64_t)h * n_chunk * PER + x;
  float a = 0.f;
  for (int p = 0; p < n_chunk; ++p) a += ph[(int64_t)p * PER];
  if (x >= D * D) {
    dz[(int64_t)h * D + (x - D * D)] = a;
  } else {  // MFMA order -> dS[16 jt + 4 g + r][16 t + c]
    const int tile = x / 256, l = (x % 256) / 4, r = x % 4;
    const int jt = tile / NT, t = tile % NT;
    dS[(int64_t)h * D * D + (16 * jt + 4 * (l >> 4) + r) * D + 16 * t + (l & 15)] = a;
  }
}

template <typename T, int D, int BLK>
hipError_t run_attend_bwd(const BwdArgs& a, int stage, hipStream_t s) {
  const int nqb = (int)((a.n_q + BLK - 1) / BLK), nkb = (int)((a.n_kv + BLK - 1) / BLK);
  const int64_t inv_n = (int64_t)a.heads * ((nkb + kInvKeys - 1) / kInvKeys);
  if (stage == 0)
    bwd_inv_sel<<<(unsigned)inv_n, 256, 0, s>>>(a.sel, nqb, nkb, a.top_k, a.inv_cnt,
                                                 a.inv_list, a.nqb_cap);
  if (stage == 1 && std::is_same<T, bf16_t>::value && BLK == 64) {
    const int n_logical = a.heads * nqb;
#define HF_DQ2(SHORT)                                                                          \
  bwd_dq2<D, SHORT><<<(unsigned)((n_logical + 7) / 8 * 8), 128, 0, s>>>(                       \
      static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, static_cast<const bf16_t*>(a.k),         \
      static_cast<const bf16_t*>(a.v), a.n_kv, a.kv_hs, a.sel, a.top_k, nqb, nkb, n_logical,     \
      a.scale, static_cast<const bf16_t*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap)
    if (a.n_kv < 64) HF_DQ2(true); else HF_DQ2(false);
#undef HF_DQ2
    bwd_rows_lin_mfma<D><<<(unsigned)(a.heads * nqb), BT, 0, s>>>(
        static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, a.s_split, a.z, a.eps,
        static_cast<const bf16_t*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap, nqb);
  } else if (stage == 1)
    bwd_rows<T, D, BLK><<<(unsigned)(a.heads * nqb * (BLK / kRows<BLK>)), BT, 0, s>>>(
        static_cast<const T*>(a.q), a.n_q, a.q_hs, static_cast<const T*>(a.k),
        static_cast<const T*>(a.v), a.n_kv, a.kv_hs, a.sel, a.top_k, nqb, nkb, a.S, a.z, a.eps,
        a.scale, static_cast<const T*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap);
  if (stage == 2 && std::is_same<T, bf16_t>::value && BLK == 64)
    bwd_kv2<D><<<(unsigned)(a.heads * nkb), BT, 0, s>>>(
        static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, static_cast<const bf16_t*>(a.k),
        static_cast<const bf16_t*>(a.v), a.n_kv, a.kv_hs, nkb, a.scale,
        static_cast<const bf16_t*>(a.dout), a.do_hs, a.rowstats, a.nq_cap, a.inv_cnt, a.inv_list,
        a.nqb_cap, a.dk, a.dv, a.dkv_hs);
  else if (stage == 2)
    bwd_kv<T, D, BLK><<<(unsigned)(a.heads * nkb * (BLK / kRows<BLK>)), BT, 0, s>>>(
        static_cast<const T*>(a.q), a.n_q, a.q_hs, static_cast<const T*>(a.k),
        static_cast<const T*>(a.v), a.n_kv, a.kv_hs, nkb, a.scale, static_cast<const T*>(a.dout),
        a.do_hs, a.rowstats, a.nq_cap, a.inv_cnt, a.inv_list, a.nqb_cap, a.dk, a.dv, a.dkv_hs);
  if (stage == 3 && std::is_same<T, bf16_t>::value) {
    const int n_chunk = (int)((a.n_q + kStateChunk - 1) / kStateChunk);
    bwd_state_mfma<D><<<(unsigned)(a.heads * n_chunk), BT, 0, s>>>(
        static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, static_cast<const bf16_t*>(a.dout),
        a.do_hs, a.rowstats, a.nq_cap, a.state_part, n_chunk);
    bwd_state_reduce<D><<<dim3((D * D + D + BT - 1) / BT, a.heads), BT, 0, s>>>(
        a.state_part, n_chunk, a.dS, a.dz);
  } else if (stage == 3)
    bwd_state<T, D><<<(unsigned)(a.heads * (D / kStateRows + 1)), BT, 0, s>>>(
        static_cast<const T*>(a.q), a.n_q, a.q_hs, static_cast<const T*>(a.dout), a.do_hs,
        a.rowstats, a.nq_cap, a.dS, a.dz);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_absorb_bwd(int heads, const void* k, const void* v, int64_t n_ev, int64_t ev_hs,
                          const float* dS, const float* dz, float* dk, float* dv, int64_t dev_hs,
                          hipStream_t s) {
  const int ntile = (int)((n_ev + 63) / 64);
  if constexpr (std::is_same<T, bf16_t>::value)
    absorb_bwd_mfma<D><<<(unsigned)(heads * ntile), BT, 0, s>>>(
        static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), n_ev, ev_hs, dS, dz, dk, dv,
        dev_hs, ntile);
  else
    absorb_bwd<T, D><<<(unsigned)(heads * ntile), BT, 0, s>>>(
        static_cast<const T*>(k), static_cast<const T*>(v), n_ev, ev_hs, dS, dz, dk, dv, dev_hs,
        ntile);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_backward(int dtype, int d, int block, const BwdArgs& a, int stage,
                                  hipStream_t s) {
  if (dtype == 0) {
    if (block == 64 && d == 128) return run_attend_bwd<bf16_t, 128, 64>(a, stage, s);
    if (block == 64 && d == 64) return run_attend_bwd<bf16_t, 64, 64>(a, stage, s);
  } else {
    if (block == 16 && d == 64) return run_attend_bwd<float, 64, 16>(a, stage, s);
    if (block == 16 && d == 128) return run_attend_bwd<float, 128, 16>(a, stage, s);
    if (block == 64 && d == 64) return run_attend_bwd<float, 64, 64>(a, stage, s);
    if (block == 64 && d == 128) return run_attend_bwd<float, 128, 64>(a, stage, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_absorb_backward(int dtype, int heads, int d, const void* k, const void* v,
                                  int64_t n_ev, int64_t ev_hs, const float* dS, const float* dz,
                                  float* dk, float* dv, int64_t dev_hs, hipStream_t s) {
  if (n_ev <= 0) return hipSuccess;
  if (dtype == 0) {
    if (d == 128) return run_absorb_bwd<bf16_t, 128>(heads, k, v, n_ev, ev_hs, dS, dz, dk, dv, dev_hs, s);
    if (d == 64) return run_absorb_bwd<bf16_t, 64>(heads, k, v, n_ev, ev_hs, dS, dz, dk, dv, dev_hs, s);
  } else {
    if (d == 128) return run_absorb_bwd<float, 128>(heads, k, v, n_ev, ev_hs, dS, dz, dk, dv, dev_hs, s);
    if (d == 64) return run_absorb_bwd<float, 64>(heads, k, v, n_ev, ev_hs, dS, dz, dk, dv, dev_hs, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace hf
