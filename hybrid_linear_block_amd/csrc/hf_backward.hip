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
// Kernels (fp32 arithmetic throughout, no atomics: every sum runs in a fixed order,
// so the results are bitwise reproducible):
//   bwd_inv_sel  per (head, key block): the query blocks that selected it, ascending;
//   bwd_rows     per (head, query block): pass 1 recomputes each row's softmax
//                (log-sum-exp and o_swa, hence D_r) over its selected blocks, then
//                the linear read's terms; pass 2 accumulates dq; stores per-row
//                (lse, D, den, c) for the other kernels;
//   bwd_kv       per (head, key block): dk and dv over the query blocks that
//                selected it;
//   bwd_state    per (head, 8 rows of dS, or z): dS and dz over all query rows;
//   absorb_bwd   per (head, 64 evicted tokens): dk_ev and dv_ev.
// A row's dot products are split over TPR adjacent lanes (DS features each) and
// reduced with xor shuffles; K/V or Q/dout tiles are staged in LDS as fp32.
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

// One workgroup per (head, key block): each thread looks for the key block in one
// query block's ascending selection row (binary search); thread 0 then appends the
// hits in query-block order.
__global__ __launch_bounds__(256) void bwd_inv_sel(const int32_t* __restrict__ sel, int nqb,
                                                   int nkb, int top_k, int32_t* __restrict__ cnt,
                                                   int32_t* __restrict__ list, int nqb_cap) {
  __shared__ int hit[256];
  const int64_t x = blockIdx.x;
  const int h = (int)(x / nkb), j = (int)(x % nkb);
  int n = 0;  // thread 0's running count
  for (int base = 0; base < nqb; base += 256) {
    const int i = base + (int)threadIdx.x;
    bool f = false;
    if (i < nqb) {
      const int32_t* row = sel + ((int64_t)h * nqb + i) * top_k;
      int lo = 0, hi = top_k;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (row[mid] < j) lo = mid + 1;
        else hi = mid;
      }
      f = lo < top_k && row[lo] == j;
    }
    hit[threadIdx.x] = f;
    __syncthreads();
    if (threadIdx.x == 0)
      for (int t = 0; t < 256 && base + t < nqb; ++t)
        if (hit[t]) list[x * nqb_cap + n++] = base + t;
    __syncthreads();
  }
  if (threadIdx.x == 0) cnt[x] = n;
}

// Query rows per workgroup of bwd_rows and key rows per workgroup of bwd_kv, and
// the rows of their staged tiles: 32 (16 for 16-row blocks), so that two 32-row
// fp32 tiles (32 KB at d = 128) and a 16-feature slice per lane leave room for
// several workgroups per compute unit.
template <int BLK>
constexpr int kRows = BLK > 32 ? 32 : BLK;

// Body of the row kernels. LIN: only the linear read's terms, added to dq (which holds
// the softmax path's part, written by bwd_dq_mfma together with lse and D); stores den
// and c only.
template <typename T, int D, int BLK, bool LIN>
__device__ __forceinline__ void rows_body(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ kg,
    const T* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int nkb, const float* __restrict__ S, const float* __restrict__ z,
    float eps, float scale, const T* __restrict__ dout, int64_t do_hs, float* __restrict__ dq,
    int64_t dq_hs, float* __restrict__ rs, int64_t nq_cap) {
  // The linear-only form takes a whole query block per workgroup (one staging of S
  // per 64 rows); the full form splits it into 32-row halves.
  constexpr int RPW = LIN ? BLK : kRows<BLK>, KT = RPW, SPLIT = BLK / RPW;
  constexpr int TPR = BT / RPW, DS = D / TPR;
  static_assert(DS % 4 == 0, "float4 slices");
  __shared__ __align__(16) float tk[KT * D];
  __shared__ __align__(16) float tv[KT * D];
  // S of the head for the linear read, staged in the linear-only form (whose
  // workgroups do little else); the full form reads it from the cache.
  __shared__ __align__(16) float tS[LIN ? D * D : 4];
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
  if constexpr (!LIN)
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
        const float a = exp2f(m2 - mx);
        l *= a;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] *= a;
        m2 = mx;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p = exp2f(x[w] - m2);
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
        const float a = exp2f(m2 - x);
        l *= a;
#pragma unroll
        for (int e = 0; e < DS; ++e) acc[e] *= a;
        m2 = x;
      }
      const float p = exp2f(x - m2);
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
  if (LIN)
    for (int e = threadIdx.x; e < D * D / 4; e += BT)
      reinterpret_cast<float4*>(tS)[e] =
          reinterpret_cast<const float4*>(S + (int64_t)h * D * D)[e];
  const float* Sh = LIN ? tS : S + (int64_t)h * D * D;
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
  if constexpr (!LIN)
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
      const float p = exp2f(s * sl2 - lse2);
      const float dl = scale * p * (dp - Dr);
#pragma unroll
      for (int e = 0; e < DS; ++e) acc[e] += dl * kr[e];
    }
  }
  if (live) {
    float* o = dq + (int64_t)h * dq_hs + r * D + d0;
#pragma unroll
    for (int e = 0; e < DS; ++e) o[e] = LIN ? o[e] + acc[e] : acc[e];
    if (d0 == 0) {
      float* st = rs + ((int64_t)h * nq_cap + r) * 4;
      if (!LIN) {
        st[0] = lse2;
        st[1] = Dr;
      }
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
  rows_body<T, D, BLK, false>(HF_ROWS_PASS);
}

// The linear read's terms only (after bwd_dq_mfma); its LDS copy of S sets the occupancy.
template <typename T, int D, int BLK>
__global__ __launch_bounds__(BT) void bwd_rows_lin(HF_ROWS_ARGS) {
  rows_body<T, D, BLK, true>(HF_ROWS_PASS);
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
      const float p = exp2f(s * sl2 - tst[2 * u]);
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

// bf16 dq of the softmax path on MFMA (v_mfma_f32_16x16x32_bf16), one workgroup per
// (head, 64-row query block), wave w owning queries 16w .. 16w + 15, whose Q and dO
// rows stay in registers as B operands. Three passes over the selected key blocks:
// A the row max of the scores S^T = K Q^T; B the sum l of exp2(S tau log2e - m) and
// O^T += V^T P^T, giving lse and D = dO . O / l; C dP^T = V dO^T, dL^T = tau P^T (dP^T
// - D) and dQ^T += K^T dL^T. The key order of the last two products comes from the
// result layout of S^T (a lane holds keys 4g .. 4g + 3 of two 16-key tiles), so P^T
// and dL^T are B operands in registers, split into bf16 hi and lo parts, and V^T and
// K^T are read as A operands from transposed copies staged in LDS. Writes the softmax
// part of dq and (lse, D) per row; the linear read's part is added by bwd_rows<LIN>.
template <int D>
__global__ __launch_bounds__(BT) void bwd_dq_mfma(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const bf16_t* __restrict__ kg,
    const bf16_t* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int nkb, float scale, const bf16_t* __restrict__ dout, int64_t do_hs,
    float* __restrict__ dq, int64_t dq_hs, float* __restrict__ rs, int64_t nq_cap) {
  constexpr int BLK = 64, NKS = D / 32, NE = D / 16;
  constexpr int RS = D + 8, TS = BLK + 8;
  typedef Mfma<bf16_t> M;
  __shared__ __align__(16) bf16_t ks[BLK * RS];
  __shared__ __align__(16) bf16_t vs[BLK * RS];
  __shared__ __align__(16) bf16_t kt[D * TS];
  __shared__ __align__(16) bf16_t vt[D * TS];
  const int h = blockIdx.x / nqb, i = blockIdx.x % nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const float sl2 = scale * kL2e;
  const int64_t qrow = (int64_t)i * BLK + w * 16 + c;
  const bool qvalid = qrow < n_q;
  bf16x8 qop[NKS], dop[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    qop[s] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(q + (int64_t)h * q_hs + qrow * D +
                                                                 32 * s + 8 * g)
                              : zero4());
    dop[s] = as_bf16x8(qvalid ? *reinterpret_cast<const uint4*>(dout + (int64_t)h * do_hs +
                                                                 qrow * D + 32 * s + 8 * g)
                              : zero4());
  }
  const bf16_t* kh = kg + (int64_t)h * kv_hs;
  const bf16_t* vh = vg + (int64_t)h * kv_hs;
  const int32_t* my_sel = sel + ((int64_t)h * nqb + i) * top_k;

  // Stage key block jb: K row-major (always), V row-major, K^T, V^T as asked.
  auto stage = [&](int jb, bool v_rows, bool k_t, bool v_t) {
    __syncthreads();  // every wave is done with the previous block's copies
    for (int v = threadIdx.x; v < BLK * (D / 8); v += BT) {
      const int r = v % BLK, ch = v / BLK;
      const int64_t row = (int64_t)jb * BLK + r;
      const bool ok = row < n_kv;
      const uint4 a = ok ? *reinterpret_cast<const uint4*>(kh + row * D + ch * 8) : zero4();
      *reinterpret_cast<uint4*>(ks + r * RS + ch * 8) = a;
      if (k_t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) kt[(ch * 8 + e) * TS + r] = (bf16_t)half16(a, e);
      }
      if (v_rows || v_t) {
        const uint4 b = ok ? *reinterpret_cast<const uint4*>(vh + row * D + ch * 8) : zero4();
        if (v_rows) *reinterpret_cast<uint4*>(vs + r * RS + ch * 8) = b;
        if (v_t) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vt[(ch * 8 + e) * TS + r] = (bf16_t)half16(b, e);
        }
      }
    }
    __syncthreads();
  };
  // S^T tiles of the staged block (keys past the window: -inf), in log2 units.
  auto scores = [&](int jb, f32x4 (&st)[4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        a = M::mma(as_bf16x8(*reinterpret_cast<const uint4*>(ks + (16 * mt + c) * RS + 32 * s +
                                                             8 * g)),
                   qop[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = (int64_t)jb * BLK + 16 * mt + 4 * g + r;
        st[mt][r] = key < n_kv ? a[r] * sl2 : -INFINITY;
      }
    }
  };
  // A operand of a transposed copy: row 16e + c, keys 32c2 + 4g + 0..3 and + 16.
  auto tr_op = [&](const bf16_t* t, int e, int c2) {
    const int o = (16 * e + c) * TS + 32 * c2 + 4 * g;
    const uint2 a0 = *reinterpret_cast<const uint2*>(t + o);
    const uint2 a1 = *reinterpret_cast<const uint2*>(t + o + 16);
    return as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
  };

  // ---- pass A: row max ----
  float m = -INFINITY;
  for (int t = 0; t < top_k; ++t) {
    const int jb = clamp_block(my_sel[t], nkb);
    stage(jb, false, false, false);
    f32x4 st[4];
    scores(jb, st);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      m = fmaxf(m, fmaxf(fmaxf(st[mt][0], st[mt][1]), fmaxf(st[mt][2], st[mt][3])));
  }
  m = max_over_groups(m);  // finite: every block holds a key of the window

  // ---- pass B: l and O^T = V^T P^T at the fixed max ----
  float lsum = 0.f;
  f32x4 oT[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) oT[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < top_k; ++t) {
    const int jb = clamp_block(my_sel[t], nkb);
    stage(jb, false, false, true);
    f32x4 st[4];
    scores(jb, st);
    float p[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mt][r] = exp2f(st[mt][r] - m);
        lsum += p[mt][r];
      }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float pv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = p[2 * c2][r];
        pv[4 + r] = p[2 * c2 + 1][r];
      }
      bf16x8 ph, pl;
      split_bf16x8(pv, ph, pl);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const bf16x8 a = tr_op(vt, e, c2);
        oT[e] = M::mma(a, ph, oT[e]);
        oT[e] = M::mma(a, pl, oT[e]);
      }
    }
  }
  const float l = sum_over_groups(lsum);
  const float lse2 = m + log2f(l);
  float dpart = 0.f;
  if (qvalid) {
    const bf16_t* dr = dout + (int64_t)h * do_hs + qrow * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const uint2 u = *reinterpret_cast<const uint2*>(dr + 16 * e + 4 * g);
      dpart += bf16_to_f32(u.x & 0xffffu) * oT[e][0] + bf16_to_f32(u.x >> 16) * oT[e][1] +
               bf16_to_f32(u.y & 0xffffu) * oT[e][2] + bf16_to_f32(u.y >> 16) * oT[e][3];
    }
  }
  const float Dr = sum_over_groups(dpart) / l;

  // ---- pass C: dQ^T += K^T dL^T ----
  f32x4 gT[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) gT[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < top_k; ++t) {
    const int jb = clamp_block(my_sel[t], nkb);
    stage(jb, true, true, false);
    f32x4 st[4];
    scores(jb, st);
    float dl[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        a = M::mma(as_bf16x8(*reinterpret_cast<const uint4*>(vs + (16 * mt + c) * RS + 32 * s +
                                                             8 * g)),
                   dop[s], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) dl[mt][r] = scale * exp2f(st[mt][r] - lse2) * (a[r] - Dr);
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float lv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lv[r] = dl[2 * c2][r];
        lv[4 + r] = dl[2 * c2 + 1][r];
      }
      bf16x8 lh, ll;
      split_bf16x8(lv, lh, ll);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const bf16x8 a = tr_op(kt, e, c2);
        gT[e] = M::mma(a, lh, gT[e]);
        gT[e] = M::mma(a, ll, gT[e]);
      }
    }
  }
  if (qvalid) {
    float* o = dq + (int64_t)h * dq_hs + qrow * D;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      *reinterpret_cast<float4*>(o + 16 * e + 4 * g) = make_float4(gT[e][0], gT[e][1], gT[e][2],
                                                                    gT[e][3]);
    if (g == 0) {
      float* st = rs + ((int64_t)h * nq_cap + qrow) * 4;
      st[0] = lse2;
      st[1] = Dr;
    }
  }
}

// bf16 dk and dv on MFMA (v_mfma_f32_16x16x32_bf16), one workgroup per (head, 64-key
// block), wave w owning keys 16w .. 16w + 15, over the query blocks that selected the
// block. Per 64-row query block: S = Q K^T and dP = dO V^T (K and V of the wave's keys
// stay in registers as the B operands), P = exp2(S tau log2e - lse), dL = tau P (dP -
// D); then dV^T += dO^T P and dK^T += Q^T dL. The contraction over queries takes its
// k order from the result layout of S (a lane holds queries 4g .. 4g + 3 of two
// 16-query tiles), so P and dL become B operands in registers, split into bf16 hi and
// lo parts (Q and dO are exact bf16, so the products keep ~fp32 accuracy), while dO^T
// and Q^T are read as A operands from transposed copies staged in LDS.
template <int D>
__global__ __launch_bounds__(BT) void bwd_kv_mfma(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const bf16_t* __restrict__ kg,
    const bf16_t* __restrict__ vg, int64_t n_kv, int64_t kv_hs, int nkb, float scale,
    const bf16_t* __restrict__ dout, int64_t do_hs, const float* __restrict__ rs, int64_t nq_cap,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ list, int nqb_cap,
    float* __restrict__ dk, float* __restrict__ dv, int64_t dkv_hs) {
  constexpr int BLK = 64, NKS = D / 32, NE = D / 16;
  constexpr int RS = D + 8;    // row stride of the row-major copies (bf16)
  constexpr int TS = BLK + 8;  // row stride of the transposed copies (bf16)
  typedef Mfma<bf16_t> M;
  __shared__ __align__(16) bf16_t qs[BLK * RS];
  __shared__ __align__(16) bf16_t dos[BLK * RS];
  __shared__ __align__(16) bf16_t qt[D * TS];
  __shared__ __align__(16) bf16_t dot_[D * TS];
  __shared__ float tst[BLK * 2];
  const int h = blockIdx.x / nkb, jb = blockIdx.x % nkb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const float sl2 = scale * kL2e;
  const int64_t key = (int64_t)jb * BLK + w * 16 + c;
  const bool kvalid = key < n_kv;
  bf16x8 kop[NKS], vop[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int64_t off = (int64_t)h * kv_hs + key * D + 32 * s + 8 * g;
    kop[s] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(kg + off) : zero4());
    vop[s] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(vg + off) : zero4());
  }
  f32x4 dvT[NE], dkT[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) dvT[e] = dkT[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16_t* qh = q + (int64_t)h * q_hs;
  const bf16_t* doh = dout + (int64_t)h * do_hs;
  const int64_t slot = (int64_t)h * nkb + jb;
  const int n_sel = cnt[slot];
  for (int x = 0; x < n_sel; ++x) {
    const int64_t q0 = (int64_t)list[slot * nqb_cap + x] * BLK;
    __syncthreads();  // every wave is done with the previous query block
    for (int v = threadIdx.x; v < BLK * (D / 8); v += BT) {
      const int r = v % BLK, ch = v / BLK;  // consecutive lanes take consecutive rows
      const int64_t row = q0 + r;
      const uint4 a = row < n_q ? *reinterpret_cast<const uint4*>(qh + row * D + ch * 8) : zero4();
      const uint4 b =
          row < n_q ? *reinterpret_cast<const uint4*>(doh + row * D + ch * 8) : zero4();
      *reinterpret_cast<uint4*>(qs + r * RS + ch * 8) = a;
      *reinterpret_cast<uint4*>(dos + r * RS + ch * 8) = b;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qt[(ch * 8 + i) * TS + r] = (bf16_t)half16(a, i);
        dot_[(ch * 8 + i) * TS + r] = (bf16_t)half16(b, i);
      }
    }
    for (int e = threadIdx.x; e < BLK; e += BT) {
      const int64_t row = q0 + e;
      const float* st = rs + ((int64_t)h * nq_cap + (row < n_q ? row : 0)) * 4;
      tst[2 * e] = row < n_q ? st[0] : INFINITY;  // rows past the chunk: weight 0
      tst[2 * e + 1] = row < n_q ? st[1] : 0.f;
    }
    __syncthreads();
    float P[4][4], L[4][4];
#pragma unroll
    for (int nq = 0; nq < 4; ++nq) {
      f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, pa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int o = (16 * nq + c) * RS + 32 * s + 8 * g;
        sa = M::mma(as_bf16x8(*reinterpret_cast<const uint4*>(qs + o)), kop[s], sa);
        pa = M::mma(as_bf16x8(*reinterpret_cast<const uint4*>(dos + o)), vop[s], pa);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = 16 * nq + 4 * g + r;
        const float p = exp2f(sa[r] * sl2 - tst[2 * ql]);
        P[nq][r] = p;
        L[nq][r] = scale * p * (pa[r] - tst[2 * ql + 1]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float pv[8], lv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = P[2 * kk][i];
        pv[4 + i] = P[2 * kk + 1][i];
        lv[i] = L[2 * kk][i];
        lv[4 + i] = L[2 * kk + 1][i];
      }
      bf16x8 ph, pl, lh, ll;
      split_bf16x8(pv, ph, pl);
      split_bf16x8(lv, lh, ll);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int o = (16 * e + c) * TS + 32 * kk + 4 * g;
        const uint2 d0 = *reinterpret_cast<const uint2*>(dot_ + o);
        const uint2 d1 = *reinterpret_cast<const uint2*>(dot_ + o + 16);
        const uint2 q0v = *reinterpret_cast<const uint2*>(qt + o);
        const uint2 q1v = *reinterpret_cast<const uint2*>(qt + o + 16);
        const bf16x8 ado = as_bf16x8(make_uint4(d0.x, d0.y, d1.x, d1.y));
        const bf16x8 aq = as_bf16x8(make_uint4(q0v.x, q0v.y, q1v.x, q1v.y));
        dvT[e] = M::mma(ado, ph, dvT[e]);
        dvT[e] = M::mma(ado, pl, dvT[e]);
        dkT[e] = M::mma(aq, lh, dkT[e]);
        dkT[e] = M::mma(aq, ll, dkT[e]);
      }
    }
  }
  if (kvalid) {
    float* pk = dk + (int64_t)h * dkv_hs + key * D;
    float* pv = dv + (int64_t)h * dkv_hs + key * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      *reinterpret_cast<float4*>(pk + 16 * e + 4 * g) =
          make_float4(dkT[e][0], dkT[e][1], dkT[e][2], dkT[e][3]);
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
  const int64_t inv_n = (int64_t)a.heads * nkb;
  if (stage == 0)
    bwd_inv_sel<<<(unsigned)inv_n, 256, 0, s>>>(a.sel, nqb, nkb, a.top_k, a.inv_cnt,
                                                 a.inv_list, a.nqb_cap);
  if (stage == 1 && std::is_same<T, bf16_t>::value && BLK == 64) {
    bwd_dq_mfma<D><<<(unsigned)(a.heads * nqb), BT, 0, s>>>(
        static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, static_cast<const bf16_t*>(a.k),
        static_cast<const bf16_t*>(a.v), a.n_kv, a.kv_hs, a.sel, a.top_k, nqb, nkb, a.scale,
        static_cast<const bf16_t*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap);
    bwd_rows_lin_mfma<D><<<(unsigned)(a.heads * nqb), BT, 0, s>>>(
        static_cast<const bf16_t*>(a.q), a.n_q, a.q_hs, a.s_split, a.z, a.eps,
        static_cast<const bf16_t*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap, nqb);
  } else if (stage == 1)
    bwd_rows<T, D, BLK><<<(unsigned)(a.heads * nqb * (BLK / kRows<BLK>)), BT, 0, s>>>(
        static_cast<const T*>(a.q), a.n_q, a.q_hs, static_cast<const T*>(a.k),
        static_cast<const T*>(a.v), a.n_kv, a.kv_hs, a.sel, a.top_k, nqb, nkb, a.S, a.z, a.eps,
        a.scale, static_cast<const T*>(a.dout), a.do_hs, a.dq, a.dq_hs, a.rowstats, a.nq_cap);
  if (stage == 2 && std::is_same<T, bf16_t>::value && BLK == 64)
    bwd_kv_mfma<D><<<(unsigned)(a.heads * nkb), BT, 0, s>>>(
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
