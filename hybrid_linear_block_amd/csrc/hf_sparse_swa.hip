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
#include "hf_absorb_parts.h"
#include "hf_launch.h"

namespace hf {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Item of workgroup wg in a ragged launch: the hardware hands consecutive workgroups to
// the 8 XCDs in turn; XCD wg % 8 takes the (wg / 8)-th item of its range (-1: none).
__device__ __forceinline__ int ragged_item(const Ragged& rg, int wg) {
  const int x = wg & 7, k = wg >> 3;
  return rg.xcd0[x] + k < rg.xcd0[x + 1] ? rg.xcd0[x] + k : -1;
}

// The angle table row (cos, sin of every rotated pair) of window row wrow's position.
__device__ __forceinline__ const float2* rope_cs(const Rope& rope, int64_t wrow) {
  const uint32_t f = (uint32_t)wrow / (uint32_t)rope.tpf;
  return rope.cs + (size_t)(f < (uint32_t)rope.cap ? f : (uint32_t)rope.cap) * rope.half;
}

template <typename T, int D, int BLK>
struct SwaSmem;

// bf16: K and V blocks row-major in 16-byte chunks; chunk cc of row r is stored
// in slot cc ^ swz(r). Two reads use the tiles: the K operand (ds_read_b128; lane
// (g, c) reads chunk 4s + g of row c) and the transposing V read
// (ds_read_b64_tr_b16; 8 rows x one aligned chunk pair per half-wave). gfx950 LDS
// has 64 four-byte banks; the transposing read serves each half-wave in one pass,
// so 8 consecutive rows need distinct slot pairs, but ds_read_b128 does not serve
// the 16 lanes of one lane group together, and a swizzle that only keeps those 16
// slots distinct (e.g. 2 (r mod 8) + bit 3 of r) still conflicts 2-way. The linear
// (over GF(2)) swizzles below were chosen so that both reads are conflict-free, as
// measured with the LDS bank-conflict counter on patterns of exactly these reads.
// With 128-byte rows (CPR = 8) two rows share the 64 banks, so swz has 3 bits.
// (swz<CPR>, in hf_device.h, is that swizzle.)
template <int D, int BLK>
struct SwaSmem<bf16_t, D, BLK> {
  uint4 k[BLK * D / 8];
  uint4 v[BLK * D / 8];
};

template <int D, int BLK>
struct SwaSmem<float, D, BLK> {
  float k[BLK][D + 4];
  float v[BLK][D + 4];
};

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
  static constexpr int VCH = BLK * CPR / NT;  // V chunks per thread
  static_assert(BLK * CPR % NT == 0, "staging split");
};

template <typename T, int D, int BLK, int QW, bool ROPE>
__global__ __launch_bounds__((BLK / QW) * 64) void sparse_swa(
    const T* __restrict__ q, int64_t n_q, int64_t q_hs, const T* __restrict__ kg,
    const T* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int n_logical, const float* __restrict__ S,
    const float* __restrict__ z, float eps, float scale, T* __restrict__ out, int64_t out_hs,
    Rope rope, Ragged rg) {
  using C = SwaCfg<T, D, BLK, QW>;
  using M = Mfma<T>;
  using op_t = typename M::op_t;
  constexpr int KSTEP = M::KSTEP, KP = M::KP;
  constexpr int NKS = D / KSTEP;  // k-steps over features
  __shared__ SwaSmem<T, D, BLK> sm;

  // Ragged windows: XCD x takes its work-balanced range of the head-major items.
  const int logical = rg.on ? ragged_item(rg, blockIdx.x) : xcd_remap(blockIdx.x, gridDim.x, n_logical);
  if (logical < 0) return;
  const int h = logical / nqb, i = logical % nqb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  const T* qh = q + (size_t)h * q_hs;
  const T* kh = ROPE ? static_cast<const T*>(rope.k_out) + (size_t)h * rope.k_out_hs
                     : kg + (size_t)h * kv_hs;
  const T* vh = vg + (size_t)h * kv_hs;
  const int32_t* my_sel = sel + ((size_t)h * nqb + i) * top_k;
  if (rg.on) {  // this head's own window and top_k (sel rows keep the stride top_k)
    kh = kg + (size_t)rg.off[h] * D;
    vh = vg + (size_t)rg.off[h] * D;
    n_kv = rg.off[h + 1] - rg.off[h];
    top_k = rg.top_k[h];
  }
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
        const int f = s * KSTEP + g;
        qop[n][s] = ok ? qh[r * D + f] : 0.f;
        if constexpr (ROPE) {  // pair (f & ~1, f | 1) turns by the row's position
          if (ok && (f >> 1) < rope.half) {
            const float x = qop[n][s], y = qh[r * D + (f ^ 1)];
            const float2 t = rope_cs(rope, rope.q_row0 + r)[f >> 1];
            qop[n][s] = (f & 1) ? y * t.y + x * t.x : x * t.x - y * t.y;
          }
        }
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
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int ch = tid + u * C::NT;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      vreg[u] = ld16(vh + (base + row) * D + cc * C::VEC, base + row < n_kv);
    }
  };
  auto store_block = [&]() {
    if constexpr (KP == 8) {
#pragma unroll
      for (int u = 0; u < C::KCH; ++u) {
        const int ch = tid + u * C::NT;
        const int row = ch / C::CPR, cc = ch % C::CPR;
        sm.k[row * C::CPR + (cc ^ (row & (C::CPR - 1)))] = kreg[u];
      }
#pragma unroll
      for (int u = 0; u < C::VCH; ++u) {
        const int ch = tid + u * C::NT;
        const int row = ch / C::CPR, cc = ch % C::CPR;
        sm.v[row * C::CPR + (cc ^ (row & (C::CPR - 1)))] = vreg[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < C::KCH; ++u) {
        const int ch = tid + u * C::NT;
        const int row = ch / C::CPR, cc = ch % C::CPR;
        *reinterpret_cast<uint4*>(&sm.k[row][cc * C::VEC]) = kreg[u];
      }
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
          const int row = mt * 16 + c;
          kop = as_bf16x8(sm.k[row * C::CPR + ((s * 4 + g) ^ (row & (C::CPR - 1)))]);
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
        // A = V^T of this 32-key chunk, keys in the order of pop: lane group g takes
        // keys 32c2 + 4g + 0..3 (score tile 2c2) then 32c2 + 16 + 4g + 0..3 (tile
        // 2c2 + 1); source lane 4j + p of the group points at V[row j][16et + 4p ..].
        const int jr = (lane & 15) >> 2, pp = lane & 3;
#pragma unroll
        for (int et = 0; et < C::NET; ++et) {
          const int chunk = 2 * et + (pp >> 1);
          const int r0 = c2 * 32 + 4 * g + jr, r1 = r0 + 16;
          const char* vb = reinterpret_cast<const char*>(sm.v);
          const v4i16 lo = lds_read_tr(vb + (r0 * C::CPR + (chunk ^ (r0 & (C::CPR - 1)))) * 16 +
                                       (pp & 1) * 8);
          const v4i16 hi = lds_read_tr(vb + (r1 * C::CPR + (chunk ^ (r1 & (C::CPR - 1)))) * 16 +
                                       (pp & 1) * 8);
          const op_t vop = __builtin_bit_cast(op_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3,
                                                                            4, 5, 6, 7));
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
        float qv = qop[n][s];
        if constexpr (ROPE) {  // the linear read takes the unrotated query
          const int64_t r = qrow0 + n * 16 + c;
          qv = r < n_q ? qh[r * D + i0] : 0.f;
        }
        f[n] = phi(qv);
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

// ---------------------------------------------------------------------------
// bf16, 64-row blocks: 2 waves x 32 query rows per workgroup.
//
// K and V blocks go from global memory straight into LDS (16-byte
// global_load_lds, no staging registers) in the swizzled row-major layout above.
// The two tiles are single-buffered and their loads are staggered so each one
// overlaps compute: K(t+1) streams in during the softmax and O^T += V^T P^T of
// block t, V(t) during S^T = K Q^T and the softmax of block t. Three barriers per
// block: K(t) has landed (which also frees the V tile of block t - 1, so V(t) is
// requested from then on, in pieces between the k-steps of S^T), every wave is done
// with K(t), V(t) has landed. The V operand
// is read with the transposing LDS read, so V needs no transposed copy. The
// epilogue normalises the accumulators in place, adds the linear read on MFMA
// into them and stores the rows from registers.

// The running reference max of a query moves only when a block's max exceeds it by
// more than this (log2 units), so weights stay <= 2^8 and the output rescale is
// skipped whenever no query of the wave moved (softmax is shift-invariant).
constexpr float kLazyMaxSlack = 8.f;

template <int D, bool SHORT, bool ROPE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void sparse_swa_bf16(
    const bf16_t* __restrict__ q, int64_t n_q, int64_t q_hs, const bf16_t* __restrict__ kg,
    const bf16_t* __restrict__ vg, int64_t n_kv, int64_t kv_hs, const int32_t* __restrict__ sel,
    int top_k, int nqb, int n_logical, const uint16_t* __restrict__ s_split,
    const float* __restrict__ z, float eps, float scale, bf16_t* __restrict__ out,
    int64_t out_hs, Rope rope, Ragged rg, AbsorbAhead ab) {
  constexpr int BLK = 64, NW = 2, NQT = 2, NMT = 4, NET = D / 16, NKS = D / 32;
  constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  constexpr int TCH = BLK * CPR;        // chunks per tile
  constexpr int LPT = TCH / (NW * 64);  // global->LDS loads per lane per tile
  static_assert(LPT % NKS == 0, "the V tile's loads spread evenly over the k-steps");
  // Separate objects, so that the compiler can tell an in-flight load into one
  // tile from reads of the other; after the loop they stage the slices of S.
  __shared__ uint4 lds_k[TCH];
  __shared__ uint4 lds_v[TCH];

  // Workgroups past the attention part form the partial states of an absorb in the
  // same LDS (the two tile buffers are its two stages).
  if (ab.n_split > 0 && (int)blockIdx.x >= ab.n_attn_wg) {
    const int it = (int)blockIdx.x - ab.n_attn_wg;
    absorb::absorb_part_bf16_w2<D>(it % ab.n_split, it / ab.n_split,
                                   static_cast<const bf16_t*>(ab.k),
                                   static_cast<const bf16_t*>(ab.v), ab.n_ev, ab.hs, ab.tps,
                                   ab.n_split, ab.partials, lds_k, lds_v);
    return;
  }
  // Ragged windows: XCD x takes its work-balanced range of the head-major items.
  const int logical =
      rg.on ? ragged_item(rg, blockIdx.x) : xcd_remap(blockIdx.x, ab.n_attn_wg, n_logical);
  if (logical < 0) return;
  const int h = logical / nqb, i = logical % nqb;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const bf16_t* qh = q + (size_t)h * q_hs;
  const bf16_t* kh = ROPE ? static_cast<const bf16_t*>(rope.k_out) + (size_t)h * rope.k_out_hs
                          : kg + (size_t)h * kv_hs;
  const bf16_t* vh = vg + (size_t)h * kv_hs;
  const int32_t* my_sel = sel + ((size_t)h * nqb + i) * top_k;
  if (rg.on) {  // this head's own window and top_k (sel rows keep the stride top_k)
    kh = kg + (size_t)rg.off[h] * D;
    vh = vg + (size_t)rg.off[h] * D;
    n_kv = rg.off[h + 1] - rg.off[h];
    top_k = rg.top_k[h];
  }
  const int64_t qrow0 = (int64_t)i * BLK + w * 32;

  // Load u of this wave fills LDS chunks (u*NW + w)*64 + lane of a tile with global
  // chunk (row, slot ^ swz(row)) of the block: rows RPU u + (w*64 + lane) / CPR. The
  // swizzle reads row bits 0..3 only, so the lane's offset inside its row group
  // repeats every 2 loads (RPU = 8) or every load (RPU a multiple of 16); the row
  // group goes into the wave-uniform base. Rows past the window (ragged last block
  // only) repeat the last row: their scores are masked, so the values only need to
  // be finite.
  constexpr int RPU = NW * 64 / CPR;  // tile rows per load of the workgroup
  constexpr int NPAT = RPU % 16 == 0 ? 1 : 2;
  static_assert(RPU % 8 == 0, "offset period");
  uint32_t lpat[NPAT];  // byte offsets inside the row group
#pragma unroll
  for (int u = 0; u < NPAT; ++u) {
    const int P = (u * NW + w) * 64 + lane;
    const int row = P / CPR, cc = (P % CPR) ^ swz<CPR>(row);
    lpat[u] = (uint32_t)((row - u * RPU) * D + cc * 8) * 2u;
  }
  // The ragged last block of the window is loaded as the window's last BLK rows
  // (all in bounds; its valid keys are then the tile's last rows and the rows
  // before them are masked), so every load of every tile takes the same address
  // path. The short form (a window shorter than one block, or ragged windows where some
  // head's is) keeps every tile at its block's first row and repeats the window's last
  // row past its end instead.
  auto tile_row0 = [&](int jb) {
    const int64_t r0 = (int64_t)jb * BLK;
    return (!SHORT && r0 + BLK > n_kv) ? n_kv - BLK : r0;
  };
  auto issue_part = [&](const bf16_t* src, int jb, const uint4* tile, int u) {  // load u
    const bf16_t* tb = src + (size_t)tile_row0(jb) * D;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(tile) + w * 64 * 16);
    const uint32_t off = lpat[u % NPAT];
    if constexpr (!SHORT) {
      lds_dma16(tb + u * RPU * D, off, base + u * NW * 64 * 16);
    } else {  // rows of the tile past the window read the window's last row
      const uint32_t row_bytes = D * 2, row = u * RPU + off / row_bytes;
      const uint32_t last = (uint32_t)(n_kv - 1 - tile_row0(jb));  // tile-relative
      lds_dma16(tb, (row <= last ? row : last) * row_bytes + off % row_bytes,
                base + u * NW * 64 * 16);
    }
  };
  auto issue_tile = [&](const bf16_t* src, int jb, const uint4* tile) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) issue_part(src, jb, tile, u);
  };

  // The linear read's S operands are staged through the same two buffers, one k-step
  // at a time: slice s holds, for each output feature tile et and each part (hi,
  // lo) of the split S, the 64 lanes' A operands (S[16et + c][32s + 8g .. +8]) as
  // 1 KB in lane order, so that both waves read them back linearly. A slice is
  // NET * 2 KB = one tile, LPT loads per lane, to the same LDS offsets as a tile.
  const uint16_t* Ssh = s_split + (size_t)h * 2 * D * D;
  const uint32_t soff = (uint32_t)(c * D + g * 8) * 2u;  // lane part of the S address
  auto issue_s = [&](int ks, const uint4* tile) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(tile) + w * 64 * 16);
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int pr = u * NW + w, et = pr >> 1, part = pr & 1;  // operand (et, part)
      lds_dma16(Ssh + (size_t)part * D * D + et * 16 * D + ks * 32, soff, base + u * NW * 64 * 16);
    }
  };
  static_assert(NET * 2 == LPT * NW, "an S slice is one tile");

  // The first key block's K tile is requested before the Q operands, so that its
  // latency overlaps the Q loads and the normaliser below (the vector memory counter
  // completes in order: the waits for Q cover this older load too).
  int jb = my_sel[0];
  issue_tile(kh, jb, lds_k);

  // Q operands (B of S^T = K Q^T): lane holds Q[16n + c][32s + 8g .. +8].
  bf16x8 qop[NQT][NKS];
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int64_t r = qrow0 + n * 16 + c;
#pragma unroll
    for (int s = 0; s < NKS; ++s) qop[n][s] = as_bf16x8(ld16(qh + r * D + s * 32 + g * 8, r < n_q));
  }

  // Normaliser of the linear read, 1 / (z . phi(q) + eps), formed here (fp32) so that
  // it is ready when the epilogue folds the linear read into the accumulators.
  float inv_den[NQT];
  {
    const float* zh = z + (size_t)h * D;
    float den[NQT] = {};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int i0 = s * 32 + g * 8;
      const float4 z0 = *reinterpret_cast<const float4*>(zh + i0);
      const float4 z1 = *reinterpret_cast<const float4*>(zh + i0 + 4);
      const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        const uint4 qb = __builtin_bit_cast(uint4, qop[n][s]);
#pragma unroll
        for (int e = 0; e < 8; ++e) den[n] += zz[e] * phi(bf16_to_f32(half16(qb, e)));
      }
    }
#pragma unroll
    for (int n = 0; n < NQT; ++n) inv_den[n] = 1.f / (sum_over_groups(den[n]) + eps);
  }
  if constexpr (ROPE) {  // the QK operands turn by the row's position (rounded to bf16)
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      const int64_t r = qrow0 + n * 16 + c;
      const float2* cs = rope_cs(rope, rope.q_row0 + (r < n_q ? r : n_q - 1));
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int p0 = 16 * s + 4 * g;  // this lane's pairs p0 .. p0 + 3
        if (p0 < rope.half) {
          const uint4 qb = __builtin_bit_cast(uint4, qop[n][s]);
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float a = bf16_to_f32(half16(qb, 2 * e)), b = bf16_to_f32(half16(qb, 2 * e + 1));
            if (p0 + e < rope.half) {
              const float2 t = cs[p0 + e];
              const float a2 = a * t.x - b * t.y;
              b = a * t.y + b * t.x;
              a = a2;
            }
            w[e] = pack_bf16x2(a, b);
          }
          qop[n][s] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
    }
  }

  f32x4 acc[NET][NQT];
#pragma unroll
  for (int e = 0; e < NET; ++e)
#pragma unroll
    for (int n = 0; n < NQT; ++n) acc[e][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of the weights on the MFMA (P times a ones operand; every row of the
  // result holds the sum of the query's column), so the sums are those of exactly
  // the bf16 weights that go into O.
  f32x4 acc_l[NQT];
  float m_run[NQT];  // reference max of each query (log2 units), set by the first block
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    m_run[n] = 0.f;
    acc_l[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = as_bf16x8(make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const float sl2 = scale * kLog2e;
  // LDS byte addresses of this lane's operand reads. The swizzle reads row bits 0..3
  // only, so the key tile (16 rows), the 32-key chunk and the second half of a chunk
  // (16 rows) are constant offsets from these.
  //   K operand (k-step s, key tile mt): row 16mt + c, chunk 4s + g.
  //   V^T operand (feature tile et, chunk c2): source lane 4j + p of group g points at
  //   features 16et + 4p .. +3 of row 32c2 + 4g + j (and of that row + 16).
  uint32_t kaddr[NKS], vaddr[NET];
#pragma unroll
  for (int s = 0; s < NKS; ++s)
    kaddr[s] = lds_offset(lds_k) + (uint32_t)(c * CPR + ((s * 4 + g) ^ swz<CPR>(c))) * 16u;
  {
    const int rv = 4 * g + ((lane & 15) >> 2), pp = lane & 3;
#pragma unroll
    for (int et = 0; et < NET; ++et)
      vaddr[et] = lds_offset(lds_v) +
                  (uint32_t)(rv * CPR + ((2 * et + (pp >> 1)) ^ swz<CPR>(rv))) * 16u + (pp & 1) * 8u;
  }
  constexpr uint32_t kRow16 = 16 * CPR * 16;  // bytes of 16 tile rows

#pragma clang loop unroll(disable)  // no peeled first step (register pressure)
  for (int t = 0; t < top_k; ++t) {
    const bool more = t + 1 < top_k;
    const int jb_next = more ? my_sel[t + 1] : 0;
    wait_vmem<0>();  // K(t) has landed
    lds_barrier();  // ... for every wave; every wave is also done with V(t-1)
    // The next block index is taken here, where the barrier has already waited for
    // the scalar load, so no scalar load is pending once the operand reads start
    // (it would make every wait for them a full wait).
    asm volatile("" ::"s"(jb_next));

    // ---- S^T = K Q^T: st[mt][n][r] = score(key 16mt + 4g + r, query 16n + c) ----
    f32x4 st[NMT][NQT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int n = 0; n < NQT; ++n) st[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The operands of k-step 0 are read up front, those of step s + 1 while the
    // products of step s run (two steps ahead measured the same and held 16 more VGPRs).
    bf16x8 kop[NKS][NMT];
    auto read_k = [&](int s) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) kop[s][mt] = as_bf16x8(lds_ld16(kaddr[s] + mt * kRow16));
    };
    read_k(0);
    // The S products and the tile requests run at a raised issue priority, the PV
    // products at the normal one: a SIMD's two resident waves (of different
    // workgroups) then tend to be in different phases, one wave's softmax or PV work
    // filling the gaps of the other's S products (measured: 3% faster than raising
    // both product phases, which is 2% faster than raising none).
    __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (s + 1 < NKS) read_k(s + 1);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int n = 0; n < NQT; ++n)
          st[mt][n] = Mfma<bf16_t>::mma(kop[s][mt], qop[n][s], st[mt][n]);
      if (s + 1 < NKS) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {  // one read of step s + 1 after every 2 products
          __builtin_amdgcn_sched_group_barrier(0x008, NQT, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // V(t) is requested in pieces between the k-steps, behind queued products.
#pragma unroll
      for (int u = s * (LPT / NKS); u < (s + 1) * (LPT / NKS); ++u) issue_part(vh, jb, lds_v, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();  // every wave is done with K(t)
    __builtin_amdgcn_s_setprio(2);
    if (more) issue_tile(kh, jb_next, lds_k);
    else issue_s(0, lds_k);  // last block: the first S slice takes the K buffer
    __builtin_amdgcn_s_setprio(0);

    // ---- online softmax (base 2) with a lazily moved reference max ----
    const int64_t key0 = (int64_t)jb * BLK;
    if (key0 + BLK > n_kv) {  // ragged last block: tile rows outside the block get -inf
      const int valid = (int)(n_kv - key0);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = mt * 16 + g * 4 + r;  // tile row of this key
          const bool out = SHORT ? tr >= valid : tr < BLK - valid;
#pragma unroll
          for (int n = 0; n < NQT; ++n) st[mt][n][r] = out ? -INFINITY : st[mt][n][r];
        }
    }
    // Exponent of every weight relative to the query's reference max, t = s tau log2 e
    // - m (the FMA output needs no canonicalisation for the max below). The
    // reference moves only when some key of the block exceeds it by more than the
    // slack: each lane checks its own 16 keys of the query, and only if any lane of
    // the wave sees that (rare after the first block) is the block max formed
    // across the lane groups, t shifted and the output rescaled.
    if (t == 0) {  // the reference starts at the first block's max (finite: every
                   // block has a key in the window)
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        float m4[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          m4[mt] = fmaxf(fmaxf(st[mt][n][0], st[mt][n][1]), fmaxf(st[mt][n][2], st[mt][n][3]));
        m_run[n] = max_over_groups(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * sl2;
      }
    }
    f32x4 tx[NMT][NQT];
    float mx[NQT];
    bool move_any = false;
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tx[mt][n][r] = __builtin_fmaf(st[mt][n][r], sl2, -m_run[n]);
      // a running max taking two new values per step (v_max3_f32)
      float m = fmaxf(tx[0][n][0], tx[0][n][1]);
#pragma unroll
      for (int k = 2; k < 4 * NMT; k += 2)
        m = fmaxf(fmaxf(m, tx[k / 4][n][k % 4]), tx[(k + 1) / 4][n][(k + 1) % 4]);
      mx[n] = m;
      move_any |= mx[n] > kLazyMaxSlack;
    }
    if (__builtin_amdgcn_ballot_w64(move_any)) {  // wave-uniform
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        const float d_blk = max_over_groups(mx[n]);  // block max - reference
        const float shift = d_blk > kLazyMaxSlack ? d_blk : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        m_run[n] += shift;
        acc_l[n] *= alpha;
#pragma unroll
        for (int e = 0; e < NET; ++e) acc[e][n] *= alpha;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) tx[mt][n] -= shift;
      }
    }
    uint32_t pk[NMT][NQT][2];  // bf16 weights, packed in pairs (the B operand of PV)
#pragma unroll
    for (int n = 0; n < NQT; ++n)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        float e4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) e4[r] = __builtin_amdgcn_exp2f(tx[mt][n][r]);
        pk[mt][n][0] = pack_bf16x2(e4[0], e4[1]);
        pk[mt][n][1] = pack_bf16x2(e4[2], e4[3]);
      }

    wait_vmem<LPT>();  // V(t) has landed (K(t+1) or S slice 0 may be in flight)
    lds_barrier();

    // ---- O^T += V^T P^T ----
    // Lane group g takes keys 32c2 + 4g + 0..3 then 32c2 + 16 + 4g + 0..3 (the key
    // order of the weights in pop). The V^T operands of the first 32-key chunk are
    // read up front, those of the second while the first chunk's products run.
    bf16x8 vop[2][NET];
    auto read_v = [&](int c2) {
#pragma unroll
      for (int et = 0; et < NET; ++et) {
        const v4i16 lo = lds_tr8(vaddr[et] + 2 * c2 * kRow16);
        const v4i16 hi = lds_tr8(vaddr[et] + (2 * c2 + 1) * kRow16);
        vop[c2][et] =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto mma_v = [&](int c2) {
      bf16x8 pop[NQT];
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        pop[n] = as_bf16x8(make_uint4(pk[2 * c2][n][0], pk[2 * c2][n][1], pk[2 * c2 + 1][n][0],
                                      pk[2 * c2 + 1][n][1]));
        acc_l[n] = Mfma<bf16_t>::mma(ones, pop[n], acc_l[n]);
      }
#pragma unroll
      for (int et = 0; et < NET; ++et)
#pragma unroll
        for (int n = 0; n < NQT; ++n)
          acc[et][n] = Mfma<bf16_t>::mma(vop[c2][et], pop[n], acc[et][n]);
    };
    read_v(0);
    __builtin_amdgcn_sched_barrier(0);
    read_v(1);
    mma_v(0);
#pragma unroll
    for (int k = 0; k < 2 * NET; ++k) {  // one read of chunk 1 after each product of chunk 0
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_v(1);
    if (!more && NKS > 1) {  // last block: the second S slice takes the V buffer
      lds_barrier();         // every wave is done with V(t)
      issue_s(1, lds_v);
    }
    jb = jb_next;
  }

  // ---- epilogue ----
  if constexpr (ROPE) {  // the linear read takes the unrotated queries
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      const int64_t r = qrow0 + n * 16 + c;
#pragma unroll
      for (int s = 0; s < NKS; ++s) qop[n][s] = as_bf16x8(ld16(qh + r * D + s * 32 + g * 8, r < n_q));
    }
  }
  // out = O / l + S phi(q) / (z . phi(q) + eps): the accumulators are normalised in
  // place, then the linear read accumulates S (phi(q) / den) into them on MFMA, with
  // S and the scaled phi(q) split into bf16 hi + lo (three products; the split of S
  // is kept up to date with S by the absorb). Slice s of S is in buffer s % 2; slice
  // s + 2 is loaded into it once both waves have read slice s.
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const float inv_l = 1.f / acc_l[n][0];
#pragma unroll
    for (int et = 0; et < NET; ++et) acc[et][n] *= inv_l;
  }
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    bf16x8 fhi[NQT], flo[NQT];
#pragma unroll
    for (int n = 0; n < NQT; ++n) {
      const uint4 qb = __builtin_bit_cast(uint4, qop[n][s]);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = phi(bf16_to_f32(half16(qb, e))) * inv_den[n];
      split_bf16x8(f, fhi[n], flo[n]);
    }
    if (s + 1 < NKS) wait_vmem<LPT>(); else wait_vmem<0>();  // slice s has landed
    lds_barrier();
    const uint32_t sb = lds_offset(s % 2 == 0 ? lds_k : lds_v) + lane * 16u;
    bf16x8 shi[NET], slo[NET];
#pragma unroll
    for (int et = 0; et < NET; ++et) {
      shi[et] = as_bf16x8(lds_ld16(sb + (2 * et) * 1024u));
      slo[et] = as_bf16x8(lds_ld16(sb + (2 * et + 1) * 1024u));
    }
    if (s + 2 < NKS) {
      lds_barrier();  // every wave has read slice s
      issue_s(s + 2, s % 2 == 0 ? lds_k : lds_v);
    }
#pragma unroll
    for (int et = 0; et < NET; ++et)
#pragma unroll
      for (int n = 0; n < NQT; ++n) {
        acc[et][n] = Mfma<bf16_t>::mma(shi[et], fhi[n], acc[et][n]);
        acc[et][n] = Mfma<bf16_t>::mma(slo[et], fhi[n], acc[et][n]);
        acc[et][n] = Mfma<bf16_t>::mma(shi[et], flo[n], acc[et][n]);
      }
  }
  // Stores straight from the MFMA layout: lane (c, g) holds features 16et + 4g .. +3
  // of query row 16n + c (8 bytes); a wave's 8 stores per row complete it in L2.
  bf16_t* oh = out + (size_t)h * out_hs;
  const bool full = qrow0 + 32 <= n_q;  // wave-uniform
#pragma unroll
  for (int n = 0; n < NQT; ++n) {
    const int64_t r = qrow0 + n * 16 + c;
    if (full || r < n_q) {
#pragma unroll
      for (int et = 0; et < NET; ++et)
        *reinterpret_cast<uint2*>(oh + r * D + et * 16 + g * 4) =
            make_uint2(pack_bf16x2(acc[et][n][0], acc[et][n][1]),
                       pack_bf16x2(acc[et][n][2], acc[et][n][3]));
    }
  }
}

// Workgroups per XCD of a ragged launch: the longest XCD range.
int ragged_width(const Ragged& rg) {
  int w = 0;
  for (int x = 0; x < 8; ++x) w = rg.xcd0[x + 1] - rg.xcd0[x] > w ? rg.xcd0[x + 1] - rg.xcd0[x] : w;
  return w > 0 ? w : 1;
}

template <int D>
hipError_t launch_bf16(const void* q, int64_t n_q, int64_t q_hs, const void* k, const void* v,
                       int64_t n_kv, int64_t kv_hs, const int32_t* sel, int top_k, int heads,
                       const uint16_t* s_split, const float* z, float eps, float scale,
                       void* out, int64_t out_hs, hipStream_t stream, const Rope& rope,
                       const Ragged& rg, const AbsorbAhead& ab_in) {
  const int nqb = (int)((n_q + 63) / 64);
  const int n_logical = nqb * heads;
  const int n_wg = rg.on ? 8 * ragged_width(rg) : (n_logical + 7) / 8 * 8;
  // The absorb's workgroups come after the attention's: the dispatcher hands them the
  // slots the attention leaves free, and they never delay an attention workgroup.
  AbsorbAhead ab = ab_in;
  ab.n_attn_wg = n_wg;
  if (ab.n_ev <= 0) ab.n_split = 0;
  const int grid = n_wg + heads * ab.n_split;
#define HF_SWA_BF16(SHORT, ROPE)                                                             \
  sparse_swa_bf16<D, SHORT, ROPE><<<grid, 128, 0, stream>>>(                                 \
      static_cast<const bf16_t*>(q), n_q, q_hs, static_cast<const bf16_t*>(k),                \
      static_cast<const bf16_t*>(v), n_kv, kv_hs, sel, top_k, nqb, n_logical, s_split, z, eps,  \
      scale,                                                                                  \
      static_cast<bf16_t*>(out), out_hs, rope, rg, ab)
  // A window shorter than one block takes the short form (for ragged windows: the
  // shortest head's window, n_kv the call passes).
  if (rope.cs) {
    if (n_kv < 64) HF_SWA_BF16(true, true); else HF_SWA_BF16(false, true);
  } else {
    if (n_kv < 64) HF_SWA_BF16(true, false); else HF_SWA_BF16(false, false);
  }
#undef HF_SWA_BF16
  return hipGetLastError();
}

template <typename T, int D, int BLK, int QW>
hipError_t launch(const void* q, int64_t n_q, int64_t q_hs, const void* k, const void* v,
                  int64_t n_kv, int64_t kv_hs, const int32_t* sel, int top_k, int heads,
                  const float* S, const float* z, float eps, float scale, void* out,
                  int64_t out_hs, hipStream_t stream, const Rope& rope, const Ragged& rg) {
  using Cf = SwaCfg<T, D, BLK, QW>;
  const int nqb = (int)((n_q + BLK - 1) / BLK);
  const int n_logical = nqb * heads;
  const int n_wg = rg.on ? 8 * ragged_width(rg) : (n_logical + 7) / 8 * 8;
#define HF_SWA_GEN(ROPE)                                                                      \
  sparse_swa<T, D, BLK, QW, ROPE><<<n_wg, Cf::NT, 0, stream>>>(                               \
      static_cast<const T*>(q), n_q, q_hs, static_cast<const T*>(k), static_cast<const T*>(v), \
      n_kv, kv_hs, sel, top_k, nqb, n_logical, S, z, eps, scale, static_cast<T*>(out), out_hs, \
      rope, rg)
  if (rope.cs) HF_SWA_GEN(true); else HF_SWA_GEN(false);
#undef HF_SWA_GEN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_swa(int dtype, int heads, int d, int block, const void* q, int64_t n_q,
                             int64_t q_hs, const void* k, const void* v, int64_t n_kv,
                             int64_t kv_hs, const int32_t* sel, int top_k, const float* S,
                             const uint16_t* s_split, const float* z, float eps, float scale,
                             void* out, int64_t out_hs, hipStream_t stream, const Rope& rope,
                             const Ragged& rg, const AbsorbAhead& ab) {
#define HF_SWA(T, D, BLK, QW)                                                                 \
  return launch<T, D, BLK, QW>(q, n_q, q_hs, k, v, n_kv, kv_hs, sel, top_k, heads, S, z, eps, \
                               scale, out, out_hs, stream, rope, rg)
  if (dtype == 0) {
    if (block == 64 && d == 128)
      return launch_bf16<128>(q, n_q, q_hs, k, v, n_kv, kv_hs, sel, top_k, heads, s_split, z,
                              eps, scale, out, out_hs, stream, rope, rg, ab);
    if (block == 64 && d == 64)
      return launch_bf16<64>(q, n_q, q_hs, k, v, n_kv, kv_hs, sel, top_k, heads, s_split, z,
                             eps, scale, out, out_hs, stream, rope, rg, ab);
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
