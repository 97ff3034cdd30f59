// hf_sparse_swa.hip -- block-sparse sliding-window attention with the fused
// linear-state read (gfx950).
//
// For every query row r of query block i of head h:
//   o_swa[r] = sum over the rows t of the selected key blocks of
//              softmax_t(tau q_r . k_t) v_t                  (online softmax)
//   out[r]   = o_swa[r] + S phi(q_r) / (z . phi(q_r) + eps)
// The sparse path is the block-sparse attention inside the sliding window of the
// gist.science English summary "Long-Horizon Streaming Video Generation via
// Hybrid Attention with Decoupled Distillation", 2.A.2; the read of the linear
// state is its 2.A.1; the sum of the two is stated in "Resumen Tecnico: Hybrid
// Forcing", 2.A.2.
//
// One workgroup per (query block, head); BLK/QW waves, each owning QW query rows.
// The loop runs over the workgroup's selected key blocks in ascending order: the
// block's K rows (row-major) and V rows (bf16: transposed and key-permuted so
// that each MFMA lane's 8 keys are contiguous) are staged in LDS while the next
// block's rows are already in flight into registers. S^T = K Q^T is formed on
// MFMA so that a lane holds 4 keys of one query; the row max and sum then need
// only two cross-lane steps, and the probabilities are already in the layout of
// the B operand of O^T += V^T P^T. The epilogue reads S and z of the head,
// computes S phi(Q)^T on MFMA (bf16: S and phi(q) split into hi + lo bf16 parts,
// three products) and the normaliser in fp32, and writes the sum.
//
// Workgroups are remapped so that each XCD walks one contiguous range of
// (head, query block) pairs: the co-resident workgroups of an XCD share a head's
// window and sweep it in the same ascending order, which keeps the gathered K/V
// blocks in that XCD's L2.
#include "hf_device.h"
#include "hf_launch.h"

namespace hf {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int BLK>
struct SwaSmem;

template <int D, int BLK>
struct SwaSmem<bf16_t, D, BLK> {
  bf16_t k[BLK][D + 8];   // row-major K block (+16 B pad per row)
  bf16_t vt[D][BLK + 8];  // V^T, keys permuted per 32-key chunk
};

template <int D, int BLK>
struct SwaSmem<float, D, BLK> {
  float k[BLK][D + 4];
  float v[BLK][D + 4];
};

// Position of key `k` in a transposed V row: key = 32c + 16hh + 4gg + r is stored
// at 32c + 8gg + 4hh + r, so that lane group gg finds its 8 keys (4 from each of
// the two 16-key score tiles of the 32-key chunk) in one 16-byte read.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~31) + ((key & 15) >> 2) * 8 + ((key >> 4) & 1) * 4 + (key & 3);
}

template <typename T, int D, int BLK, int QW>
struct SwaCfg {
  static constexpr int NW = BLK / QW;      // waves per workgroup
  static constexpr int NT = NW * 64;       // threads
  static constexpr int NQT = QW / 16;      // query tiles per wave
  static constexpr int NMT = BLK / 16;     // key tiles per block
  static constexpr int NET = D / 16;       // output feature tiles
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = D / VEC;      // 16-byte chunks per row
  static constexpr int KCH = BLK * CPR / NT;  // K chunks per thread
  // V chunks per thread: bf16 stages groups of 4 keys x 8 features (4 chunks).
  static constexpr int VCH = sizeof(T) == 2 ? (BLK / 4) * CPR / NT * 4 : BLK * CPR / NT;
  static_assert(BLK * CPR % NT == 0, "staging split");
};

template <typename T, int D, int BLK, int QW>
__global__ __launch_bounds__((BLK / QW) * 64) void sparse_swa(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ kg,
    const T* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int n_logical, const float* __restrict__ S,
    const float* __restrict__ z, float eps, float scale, T* __restrict__ out, int64_t out_hs) {
  using C = SwaCfg<T, D, BLK, QW>;
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KSTEP = M::KSTEP, KP = M::KP;
  constexpr int NKS = D / KSTEP;  // k-steps over features
  __shared__ SwaSmem<T, D, BLK> sm;

  const int logical = xcd_remap(blockIdx.x, gridDim.x, n_logical);
  if (logical < 0) return;
  const int h = logical / nqb, i = logical % nqb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  const T* qh = q + (size_t)h * q_hs;
  const T* kh = kg + (size_t)h * kv_hs;
  const T* vh = vg + (size_t)h * kv_hs;
  const int32_t* my_sel = sel + ((size_t)h * nqb + i) * top_k;
  const int64_t qrow0 = (int64_t)i * BLK + w * QW;

  // ---- Q operands (B of S^T = K Q^T): lane holds Q[16n + c][s*KSTEP + g*KP ..] ----
  op_t qop[C::NQT][NKS];
#pragma unroll
  for (int n = 0; n < C::NQT; ++n) {
    const int64_t r = qrow0 + n * 16 + c;
    const bool ok = r < n_q;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if constexpr (KP == 8) {
        qop[n][s] = as_bf16x8(ld16(qh + r * D + s * KSTEP + g * KP, ok));
      } else {
        qop[n][s] = ok ? qh[r * D + s * KSTEP + g] : 0.f;
      }
    }
  }

  // ---- staging helpers ----
  uint4 kreg[C::KCH], vreg[C::VCH];
  auto load_block = [&](int jb) {
    const int64_t base = (int64_t)jb * BLK;
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int ch = tid + u * C::NT;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      kreg[u] = ld16(kh + (base + row) * D + cc * C::VEC, base + row < n_kv);
    }
    if constexpr (KP == 8) {
#pragma unroll
      for (int u = 0; u < C::VCH / 4; ++u) {
        const int gq = tid + u * C::NT;
        const int kgp = gq / C::CPR, cc = gq % C::CPR;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = base + kgp * 4 + r;
          vreg[u * 4 + r] = ld16(vh + row * D + cc * C::VEC, row < n_kv);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < C::VCH; ++u) {
        const int ch = tid + u * C::NT;
        const int row = ch / C::CPR, cc = ch % C::CPR;
        vreg[u] = ld16(vh + (base + row) * D + cc * C::VEC, base + row < n_kv);
      }
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int ch = tid + u * C::NT;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      *reinterpret_cast<uint4*>(&sm.k[row][cc * C::VEC]) = kreg[u];
    }
    if constexpr (KP == 8) {
#pragma unroll
      for (int u = 0; u < C::VCH / 4; ++u) {
        const int gq = tid + u * C::NT;
        const int kgp = gq / C::CPR, cc = gq % C::CPR;
        const int pos = vt_pos(kgp * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = half16(vreg[u * 4 + 0], e), b = half16(vreg[u * 4 + 1], e);
          const uint32_t cc2 = half16(vreg[u * 4 + 2], e), d2 = half16(vreg[u * 4 + 3], e);
          *reinterpret_cast<uint2*>(&sm.vt[cc * 8 + e][pos]) =
              make_uint2(a | (b << 16), cc2 | (d2 << 16));
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < C::VCH; ++u) {
        const int ch = tid + u * C::NT;
        const int row = ch / C::CPR, cc = ch % C::CPR;
        *reinterpret_cast<uint4*>(&sm.v[row][cc * C::VEC]) = vreg[u];
      }
    }
  };

  f32x4 acc[C::NET][C::NQT];
#pragma unroll
  for (int e = 0; e < C::NET; ++e)
#pragma unroll
    for (int n = 0; n < C::NQT; ++n) acc[e][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[C::NQT], l_run[C::NQT];
#pragma unroll
  for (int n = 0; n < C::NQT; ++n) {
    m_run[n] = -INFINITY;
    l_run[n] = 0.f;
  }
  const float sl2 = scale * kLog2e;

  int jb_next = my_sel[0];
  load_block(jb_next);
  for (int t = 0; t < top_k; ++t) {
    const int jb = jb_next;
    __syncthreads();  // every wave is done with the previous block's tiles
    store_block();
    __syncthreads();
    if (t + 1 < top_k) {
      jb_next = my_sel[t + 1];
      load_block(jb_next);  // in flight while this block is computed
    }

    // ---- S^T = K Q^T: st[mt][n][r] = score(key 16mt + 4g + r, query 16n + c) ----
    f32x4 st[C::NMT][C::NQT];
#pragma unroll
    for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
      for (int n = 0; n < C::NQT; ++n) st[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int mt = 0; mt < C::NMT; ++mt) {
        op_t kop;
        if constexpr (KP == 8) {
          kop = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.k[mt * 16 + c][s * KSTEP + g * 8]));
        } else {
          kop = sm.k[mt * 16 + c][s * KSTEP + g];
        }
#pragma unroll
        for (int n = 0; n < C::NQT; ++n) st[mt][n] = M::mma(kop, qop[n][s], st[mt][n]);
      }
    }

    // ---- online softmax (base 2) ----
    const int64_t key0 = (int64_t)jb * BLK;
    const bool tail = key0 + BLK > n_kv;
    float p[C::NMT][C::NQT][4];
#pragma unroll
    for (int n = 0; n < C::NQT; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = st[mt][n][r] * sl2;
          if (tail && key0 + mt * 16 + g * 4 + r >= n_kv) x = -INFINITY;
          p[mt][n][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[n], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[n] - m_new);
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = __builtin_amdgcn_exp2f(p[mt][n][r] - m_new);
          if constexpr (KP == 8) e = bf16_to_f32(f32_to_bf16_bits(e));  // the weight PV uses
          p[mt][n][r] = e;
          rs += e;
        }
      rs += __shfl_xor(rs, 16);
      rs += __shfl_xor(rs, 32);
      l_run[n] = l_run[n] * alpha + rs;
      m_run[n] = m_new;
#pragma unroll
      for (int e = 0; e < C::NET; ++e) acc[e][n] *= alpha;
    }

    // ---- O^T += V^T P^T ----
    if constexpr (KP == 8) {
#pragma unroll
      for (int c2 = 0; c2 < BLK / 32; ++c2) {
        op_t pop[C::NQT];
#pragma unroll
        for (int n = 0; n < C::NQT; ++n) {
          uint32_t b[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            b[r] = f32_to_bf16_bits(p[2 * c2][n][r]);
            b[4 + r] = f32_to_bf16_bits(p[2 * c2 + 1][n][r]);
          }
          pop[n] = as_bf16x8(make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                        b[4] | (b[5] << 16), b[6] | (b[7] << 16)));
        }
#pragma unroll
        for (int et = 0; et < C::NET; ++et) {
          const op_t vop =
              as_bf16x8(*reinterpret_cast<const uint4*>(&sm.vt[et * 16 + c][c2 * 32 + g * 8]));
#pragma unroll
          for (int n = 0; n < C::NQT; ++n) acc[et][n] = M::mma(vop, pop[n], acc[et][n]);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < C::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int et = 0; et < C::NET; ++et) {
            const float vop = sm.v[mt * 16 + g * 4 + r][et * 16 + c];
#pragma unroll
            for (int n = 0; n < C::NQT; ++n) acc[et][n] = M::mma(vop, p[mt][n][r], acc[et][n]);
          }
    }
  }

  // ---- epilogue: linear read of the state + sum of the paths ----
  const float* Sh = S + (size_t)h * D * D;
  const float* zh = z + (size_t)h * D;
  f32x4 num[C::NET][C::NQT];
#pragma unroll
  for (int e = 0; e < C::NET; ++e)
#pragma unroll
    for (int n = 0; n < C::NQT; ++n) num[e][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den[C::NQT];
#pragma unroll
  for (int n = 0; n < C::NQT; ++n) den[n] = 0.f;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int i0 = s * KSTEP + g * KP;  // this lane's features i0 .. i0+KP-1
    if constexpr (KP == 8) {
      const float4 z0 = *reinterpret_cast<const float4*>(zh + i0);
      const float4 z1 = *reinterpret_cast<const float4*>(zh + i0 + 4);
      const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      bf16x8 fhi[C::NQT], flo[C::NQT];
#pragma unroll
      for (int n = 0; n < C::NQT; ++n) {
        const uint4 qb = __builtin_bit_cast(uint4, qop[n][s]);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = phi(bf16_to_f32(half16(qb, e)));
          den[n] += zz[e] * f[e];
        }
        split_bf16x8(f, fhi[n], flo[n]);
      }
#pragma unroll
      for (int et = 0; et < C::NET; ++et) {
        const float* sp = Sh + (size_t)(et * 16 + c) * D + i0;
        const float4 a0 = *reinterpret_cast<const float4*>(sp);
        const float4 a1 = *reinterpret_cast<const float4*>(sp + 4);
        const float sv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bf16x8 shi, slo;
        split_bf16x8(sv, shi, slo);
#pragma unroll
        for (int n = 0; n < C::NQT; ++n) {
          num[et][n] = M::mma(shi, fhi[n], num[et][n]);
          num[et][n] = M::mma(slo, fhi[n], num[et][n]);
          num[et][n] = M::mma(shi, flo[n], num[et][n]);
        }
      }
    } else {
      const float zz = zh[i0];
      float f[C::NQT];
#pragma unroll
      for (int n = 0; n < C::NQT; ++n) {
        f[n] = phi(qop[n][s]);
        den[n] += zz * f[n];
      }
#pragma unroll
      for (int et = 0; et < C::NET; ++et) {
        const float sv = Sh[(size_t)(et * 16 + c) * D + i0];
#pragma unroll
        for (int n = 0; n < C::NQT; ++n) num[et][n] = M::mma(sv, f[n], num[et][n]);
      }
    }
  }
  T* oh = out + (size_t)h * out_hs;
#pragma unroll
  for (int n = 0; n < C::NQT; ++n) {
    float dn = den[n];
    dn += __shfl_xor(dn, 16);
    dn += __shfl_xor(dn, 32);
    const float inv_den = 1.f / (dn + eps);
    const float inv_l = 1.f / l_run[n];
    const int64_t r = qrow0 + n * 16 + c;
    if (r >= n_q) continue;
#pragma unroll
    for (int et = 0; et < C::NET; ++et) {
      float o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = acc[et][n][k] * inv_l + num[et][n][k] * inv_den;
      T* dst = oh + r * D + et * 16 + g * 4;
      if constexpr (KP == 8) {
        const uint2 pk = make_uint2(f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                                    f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16));
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <typename T, int D, int BLK, int QW>
hipError_t launch(const void* q, int64_t n_q, int64_t q_hs, const void* k, const void* v,
                  int64_t n_kv, int64_t kv_hs, const int32_t* sel, int top_k, int heads,
                  const float* S, const float* z, float eps, float scale, void* out,
                  int64_t out_hs, hipStream_t stream) {
  using Cf = SwaCfg<T, D, BLK, QW>;
  const int nqb = (int)((n_q + BLK - 1) / BLK);
  const int n_logical = nqb * heads;
  const int n_wg = (n_logical + 7) / 8 * 8;
  sparse_swa<T, D, BLK, QW><<<n_wg, Cf::NT, 0, stream>>>(
      static_cast<const T*>(q), n_q, q_hs, static_cast<const T*>(k), static_cast<const T*>(v),
      n_kv, kv_hs, sel, top_k, nqb, n_logical, S, z, eps, scale, static_cast<T*>(out), out_hs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_swa(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, const void* v, int64_t n_kv,
                             int64_t kv_hs, const int32_t* sel, int top_k, const float* S,
                             const float* z, float eps, float scale, void* out, int64_t out_hs,
                             hipStream_t stream) {
#define HF_SWA(T, D, BLK, QW)                                                                 \
  return launch<T, D, BLK, QW>(q, n_q, q_hs, k, v, n_kv, kv_hs, sel, top_k, heads, S, z, eps, \
                               scale, out, out_hs, stream)
  if (dtype == 0) {
    if (block == 64 && d == 128) HF_SWA(bf16_t, 128, 64, 32);
    if (block == 64 && d == 64) HF_SWA(bf16_t, 64, 64, 32);
  } else {
    if (block == 16 && d == 64) HF_SWA(float, 64, 16, 16);
    if (block == 16 && d == 128) HF_SWA(float, 128, 16, 16);
    if (block == 64 && d == 64) HF_SWA(float, 64, 64, 32);
    if (block == 64 && d == 128) HF_SWA(float, 128, 64, 32);
  }
#undef HF_SWA
  return hipErrorInvalidValue;
}

}  // namespace hf
