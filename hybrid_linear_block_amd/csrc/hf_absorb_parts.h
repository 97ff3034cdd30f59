// hf_absorb_parts.h -- the workgroup bodies of the absorb (gfx950): the partial
// state of one token split, written to the workspace for the in-order reduce.
//
// Per head: S[j][i] += sum_n V[n][j] phi(K[n][i]) and z[i] += sum_n phi(K[n][i]),
// the incremental absorption of evicted tokens into a compact key-value state
// (the gist.science English summary "Long-Horizon Streaming Video Generation via
// Hybrid Attention with Decoupled Distillation", 2.A.1). Shared by the absorb
// kernel and by the launch that runs the absorb next to the block pooling.
#pragma once

#include "hf_device.h"
#include "hf_reduce.h"

namespace hf {
namespace absorb {


constexpr float kLog2eAbs = 1.4426950408889634f;

// fp32 path: grid (token split, 64x64 state tile, head).
constexpr int AT = 64;       // state tile edge
constexpr int TS = 64;       // tokens staged per iteration
constexpr int NTHR = 256;    // 4 waves, each owns a 32x32 quarter of the tile

// fp32: row-major tiles [TS tokens][64 features (+4 pad)] of V and phi.
constexpr int FPITCH = AT + 4;

struct AbsorbSmemF32 {
  float vs[TS][FPITCH];
  float fs[TS][FPITCH];
  float zred[8][AT];
};

// bf16: K and V token tiles (BT tokens x D features, rows of D*2 bytes) go straight
// from global memory into an NST-stage LDS ring (16-byte global->LDS loads, one per
// thread per tile). Both MFMA operands come from the transposing LDS read (tokens,
// the contraction index, end up contiguous per lane); phi, the tail mask and the
// hi/lo split are applied to the K operand in registers. A transposing read covers
// 32 bytes of rows 8g + e (+4), g, e = 0..3; chunk cc of row r sits in slot
// cc ^ 2 swz(r), which gives the rows that one half-wave reads (g = 0, 1 or 2, 3)
// distinct 32-byte bank groups.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (r & 3) | ((r >> 1) & 4);  // rows of 256 B: 8 groups
  else return ((r >> 1) & 1) | ((r >> 2) & 2);            // rows of 128 B: 2 rows per 256 B
}
constexpr int BT = 32;   // tokens per stage
constexpr int BNST = 4;  // stages in the ring (BNST - 1 in flight ahead of the one in use)

template <int D>
struct AbsorbStage {  // one ring stage: the K tile, then the V tile
  uint4 k[BT * D / 8];
  uint4 v[BT * D / 8];
};

// Workgroup (token split `split`, head h) of the bf16 absorb: D * 4 threads.
template <int D>
__device__ __forceinline__ void absorb_part_bf16(int split, int h, const bf16_t* __restrict__ kev,
                                                 const bf16_t* __restrict__ vev, int64_t n_ev,
                                                 int64_t hs, int tps, int n_split,
                                                 float* __restrict__ partials) {
  constexpr int NW = D / 16;       // waves: one per 16 key features
  constexpr int NTH = NW * 64;
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int TCH = BT * CPR;    // chunks per tile (== NTH: one load per thread)
  constexpr int NJT = D / 16;      // value-feature tiles
  static_assert(TCH == NTH, "one 16-byte load per thread and tile");
  // The whole ring spans less than 64 KB, so a stage's tile base is an immediate
  // offset of the LDS reads once the stage index is a compile-time constant.
  static_assert(sizeof(AbsorbStage<D>) * BNST <= 65536, "ring offsets fit the immediate");
  __shared__ AbsorbStage<D> ring[BNST];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (int64_t)split * tps;
  const int64_t n1 = n0 + tps < n_ev ? n0 + tps : n_ev;
  const int niter = (int)((n1 - n0 + BT - 1) / BT);
  const bf16_t* kb = kev + (size_t)h * hs;
  const bf16_t* vb = vev + (size_t)h * hs;

  // Thread tid fills LDS chunk tid of a tile (row tid / CPR, slot tid % CPR) with
  // global chunk slot ^ 2 swz(row) of that row.
  const int lrow = tid / CPR;
  const uint32_t loff = (uint32_t)(lrow * D + (((tid % CPR) ^ (2 * swz<D>(lrow))) * 8)) * 2u;
  auto issue = [&](int t, int st) {
    const int64_t r0 = n0 + (int64_t)t * BT;
    const bf16_t* kt = kb + (size_t)r0 * D;
    const bf16_t* vt = vb + (size_t)r0 * D;
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds_offset(&ring[st].k[0]) + w * 1024);
    const uint32_t vbase = __builtin_amdgcn_readfirstlane(lds_offset(&ring[st].v[0]) + w * 1024);
    const int64_t left = n1 - r0;
    uint32_t off = loff;
    if (left < BT) {  // partial last tile: rows past the end repeat the last row (masked)
      const uint32_t last = (uint32_t)left - 1;
      if ((uint32_t)lrow > last) off = last * (D * 2) + loff % (D * 2);
    }
    lds_dma16(kt, off, kbase);
    lds_dma16(vt, off, vbase);
  };

  // Transposing-read source role: lane 4e + q of group g points at row 8g + e (+4),
  // columns col0 + 4q .. +3 (chunk col0/8 + q/2, half q & 1).
  const int e_row = (lane & 15) >> 2, q = lane & 3;
  auto tr_off = [&](int row, int col0) {  // byte offset inside a tile
    const int cc = (col0 >> 3) + (q >> 1);
    return (uint32_t)((row * CPR + (cc ^ (2 * swz<D>(row)))) * 16 + (q & 1) * 8);
  };
  const int ra = 8 * g + e_row, rb = ra + 4;
  // Per-lane read addresses in stage 0; stage st adds st * sizeof(stage) as an immediate.
  const uint32_t ring0 = lds_offset(&ring[0]);
  const uint32_t koff_a = ring0 + tr_off(ra, w * 16), koff_b = ring0 + tr_off(rb, w * 16);
  uint32_t voff_a[NJT], voff_b[NJT];
#pragma unroll
  for (int j = 0; j < NJT; ++j) {
    voff_a[j] = ring0 + (uint32_t)sizeof(ring[0].k) + tr_off(ra, j * 16);
    voff_b[j] = ring0 + (uint32_t)sizeof(ring[0].k) + tr_off(rb, j * 16);
  }

  f32x4 acc[NJT];
#pragma unroll
  for (int j = 0; j < NJT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;

  for (int t = 0; t < BNST - 1 && t < niter; ++t) issue(t, t);
  for (int t0 = 0; t0 < niter; t0 += BNST) {
#pragma unroll
    for (int st = 0; st < BNST; ++st) {  // stage st of the ring holds tile t0 + st
      const int t = t0 + st;
      if (t >= niter) break;
      // Tile t has landed once at most (#later tiles issued) * 2 loads remain.
      const int later = niter - 1 - t < BNST - 2 ? niter - 1 - t : BNST - 2;
      static_assert(BNST - 2 == 2, "wait cases");
      if (later >= 2) wait_vmem<4>();
      else if (later == 1) wait_vmem<2>();
      else wait_vmem<0>();
      lds_barrier();  // ... for every wave; every wave is also done with tile t-1
      if (t + BNST - 1 < niter) issue(t + BNST - 1, (st + BNST - 1) % BNST);  // stage of t-1
      const int valid = (int)(n1 - (n0 + (int64_t)t * BT));  // tokens of this tile in range
      constexpr uint32_t kStage = sizeof(AbsorbStage<D>);
      // A: V^T for every value-feature tile, tokens in the same order as B. The reads
      // are issued before the phi work so that their latency is hidden behind it; the
      // hi products of all tiles go before the lo products, so no MFMA waits for the
      // one just before it.
      bf16x8 a[NJT];
#pragma unroll
      for (int j = 0; j < NJT; ++j) {
        const v4i16 v0 = lds_tr8(voff_a[j] + st * kStage), v1 = lds_tr8(voff_b[j] + st * kStage);
        a[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the phi work
      // B: phi(K) for this wave's 16 key features, tokens 8g + 0..7, split hi + lo.
      // phi(x) = exp(min(x, 0)) + max(x, 0): x + 1 for x > 0 (exp(0) = 1 exactly), e^x
      // otherwise (plus zero).
      const v4i16 k0 = lds_tr8(koff_a + st * kStage), k1 = lds_tr8(koff_b + st * kStage);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32((uint32_t)(uint16_t)(e < 4 ? k0[e] : k1[e - 4]));
        f[e] = __builtin_amdgcn_exp2f(fminf(x * kLog2eAbs, 0.f)) + fmaxf(x, 0.f);
      }
      if (valid < BT) {  // partial last tile (wave-uniform): tokens past the end weigh 0
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 8 * g + e < valid ? f[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) zacc += f[e];
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
        lw[e] = pack_bf16x2(f[2 * e] - __uint_as_float(hw[e] << 16),
                            f[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
      }
      const bf16x8 bh = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 bl = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
      for (int j = 0; j < NJT; ++j) acc[j] = Mfma<bf16_t>::mma(a[j], bh, acc[j]);
#pragma unroll
      for (int j = 0; j < NJT; ++j) acc[j] = Mfma<bf16_t>::mma(a[j], bl, acc[j]);
    }
  }

  // Partial state: acc[j][r] = S[16j + 4g + r][16w + c].
  float* part = partials + ((size_t)h * n_split + split) * part_floats<D>();
#pragma unroll
  for (int j = 0; j < NJT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[(j * 16 + g * 4 + r) * D + w * 16 + c] = acc[j][r];
  const float zs = sum_over_groups(zacc);
  if (g == 0) part[D * D + w * 16 + c] = zs;
}

// The partial state of absorb_part_bf16, bit for bit, formed by a workgroup of two
// waves (128 threads) inside the LDS of another kernel: wave w owns the key-feature
// tiles w * NIT .. w * NIT + NIT - 1 against every value-feature tile, and the token
// tiles pass through two stages, st0 and st1 (each a K tile followed by a V tile,
// BT * D * 4 bytes), one tile ahead. Every accumulator takes the products of
// absorb_part_bf16 in the same order (per token tile the hi product, then the lo
// product) and every z the same additions, so the partials are identical.
template <int D>
__device__ __forceinline__ void absorb_part_bf16_w2(int split, int h,
                                                    const bf16_t* __restrict__ kev,
                                                    const bf16_t* __restrict__ vev, int64_t n_ev,
                                                    int64_t hs, int tps, int n_split,
                                                    float* __restrict__ partials,
                                                    const void* st0, const void* st1) {
  constexpr int NTH = 128;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int LPT = BT * CPR / NTH;   // loads per thread per tile
  constexpr int NJT = D / 16;           // value-feature tiles
  constexpr int NIT = D / 32;           // key-feature tiles per wave
  constexpr uint32_t kTile = BT * D * 2;  // bytes of one token tile
  static_assert(LPT * NTH == BT * CPR, "whole loads per tile");
  // Workgroup-uniform by construction; said so for the compiler, since the tile
  // addresses must be scalar operands of the loads.
  split = __builtin_amdgcn_readfirstlane(split);
  h = __builtin_amdgcn_readfirstlane(h);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (int64_t)split * tps;
  const int64_t n1 = n0 + tps < n_ev ? n0 + tps : n_ev;
  const int niter = (int)((n1 - n0 + BT - 1) / BT);
  const bf16_t* kb = kev + (size_t)h * hs;
  const bf16_t* vb = vev + (size_t)h * hs;

  // Load u of thread tid fills LDS chunk u * NTH + tid of a tile (row P / CPR, slot
  // P % CPR) with global chunk slot ^ 2 swz(row) of that row, as in absorb_part_bf16.
  int lrow[LPT];
  uint32_t loff[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int P = u * NTH + tid;
    lrow[u] = P / CPR;
    loff[u] = (uint32_t)(lrow[u] * D + (((P % CPR) ^ (2 * swz<D>(lrow[u]))) * 8)) * 2u;
  }
  auto issue = [&](int t, uint32_t sbase) {
    const int64_t r0 = n0 + (int64_t)t * BT;
    const bf16_t* kt = kb + (size_t)r0 * D;
    const bf16_t* vt = vb + (size_t)r0 * D;
    const int64_t left = n1 - r0;
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      uint32_t off = loff[u];
      if (left < BT) {  // partial last tile: rows past the end repeat the last row (masked)
        const uint32_t last = (uint32_t)left - 1;
        if ((uint32_t)lrow[u] > last) off = last * (D * 2) + loff[u] % (D * 2);
      }
      const uint32_t base = __builtin_amdgcn_readfirstlane(sbase + u * NTH * 16 + w * 1024);
      lds_dma16(kt, off, base);
      lds_dma16(vt, off, base + kTile);
    }
  };

  // Transposing-read source role, as in absorb_part_bf16.
  const int e_row = (lane & 15) >> 2, q = lane & 3;
  auto tr_off = [&](int row, int col0) {
    const int cc = (col0 >> 3) + (q >> 1);
    return (uint32_t)((row * CPR + (cc ^ (2 * swz<D>(row)))) * 16 + (q & 1) * 8);
  };
  const int ra = 8 * g + e_row, rb = ra + 4;
  uint32_t koff_a[NIT], koff_b[NIT], voff_a[NJT], voff_b[NJT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    koff_a[i] = tr_off(ra, (w * NIT + i) * 16);
    koff_b[i] = tr_off(rb, (w * NIT + i) * 16);
  }
#pragma unroll
  for (int j = 0; j < NJT; ++j) {
    voff_a[j] = kTile + tr_off(ra, j * 16);
    voff_b[j] = kTile + tr_off(rb, j * 16);
  }

  f32x4 acc[NJT][NIT];
#pragma unroll
  for (int j = 0; j < NJT; ++j)
#pragma unroll
    for (int i = 0; i < NIT; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc[NIT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) zacc[i] = 0.f;

  const uint32_t sb0 = lds_offset(st0), sb1 = lds_offset(st1);
  if (niter > 0) issue(0, sb0);
  for (int t = 0; t < niter; ++t) {
    const uint32_t sb = (t & 1) ? sb1 : sb0;
    wait_vmem<0>();  // tile t has landed
    lds_barrier();   // ... for both waves, which are also done with tile t - 1
    if (t + 1 < niter) issue(t + 1, (t & 1) ? sb0 : sb1);
    const int valid = (int)(n1 - (n0 + (int64_t)t * BT));
    bf16x8 a[NJT];
#pragma unroll
    for (int j = 0; j < NJT; ++j) {
      const v4i16 v0 = lds_tr8(sb + voff_a[j]), v1 = lds_tr8(sb + voff_b[j]);
      a[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const v4i16 k0 = lds_tr8(sb + koff_a[i]), k1 = lds_tr8(sb + koff_b[i]);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_to_f32((uint32_t)(uint16_t)(e < 4 ? k0[e] : k1[e - 4]));
        f[e] = __builtin_amdgcn_exp2f(fminf(x * kLog2eAbs, 0.f)) + fmaxf(x, 0.f);
      }
      if (valid < BT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 8 * g + e < valid ? f[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) zacc[i] += f[e];
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
        lw[e] = pack_bf16x2(f[2 * e] - __uint_as_float(hw[e] << 16),
                            f[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
      }
      const bf16x8 bh = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 bl = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
      for (int j = 0; j < NJT; ++j) acc[j][i] = Mfma<bf16_t>::mma(a[j], bh, acc[j][i]);
#pragma unroll
      for (int j = 0; j < NJT; ++j) acc[j][i] = Mfma<bf16_t>::mma(a[j], bl, acc[j][i]);
    }
  }

  float* part = partials + ((size_t)h * n_split + split) * part_floats<D>();
#pragma unroll
  for (int j = 0; j < NJT; ++j)
#pragma unroll
    for (int i = 0; i < NIT; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[(j * 16 + g * 4 + r) * D + (w * NIT + i) * 16 + c] = acc[j][i][r];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const float zs = sum_over_groups(zacc[i]);
    if (g == 0) part[D * D + (w * NIT + i) * 16 + c] = zs;
  }
}

// Workgroup (token split, 64x64 state tile, head h) of the fp32 absorb: NTHR threads.
template <int D>
__device__ __forceinline__ void absorb_part_f32(int split, int tile, int h,
                                                const float* __restrict__ kev,
                                                const float* __restrict__ vev, int64_t n_ev,
                                                int64_t hs, int tps, int n_split,
                                                float* __restrict__ partials) {
  constexpr int NT = D / AT;
  __shared__ AbsorbSmemF32 sm;
  const int jt = tile / NT, it = tile % NT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wj = w >> 1, wi = w & 1;
  const int64_t n0 = (int64_t)split * tps;
  const int64_t n1 = n0 + tps < n_ev ? n0 + tps : n_ev;

  // Threads 0..127 stage V (columns jt*64..), 128..255 stage phi(K) (columns it*64..):
  // chunk u of a thread covers token row sid/16 + 8u, features 4*(sid%16)..+3.
  const bool is_v = tid < 128;
  const int sid = tid & 127;
  const int col4 = sid & 15, row0 = sid >> 4;
  const float* src = (is_v ? vev + (size_t)jt * AT : kev + (size_t)it * AT) + (size_t)h * hs +
                     col4 * 4;
  float zsum[4] = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = n0; t0 < n1; t0 += TS) {
    uint4 rows[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t n = t0 + row0 + 8 * u;
      rows[u] = ld16(src + n * D, n < n1);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = row0 + 8 * u;
      float4 x = __builtin_bit_cast(float4, rows[u]);
      if (!is_v) {
        const bool ok = t0 + r < n1;
        x.x = ok ? phi(x.x) : 0.f;
        x.y = ok ? phi(x.y) : 0.f;
        x.z = ok ? phi(x.z) : 0.f;
        x.w = ok ? phi(x.w) : 0.f;
        zsum[0] += x.x;
        zsum[1] += x.y;
        zsum[2] += x.z;
        zsum[3] += x.w;
        *reinterpret_cast<float4*>(&sm.fs[r][col4 * 4]) = x;
      } else {
        *reinterpret_cast<float4*>(&sm.vs[r][col4 * 4]) = x;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TS / 4; ++ks) {
      float a[2], b[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        a[q] = sm.vs[ks * 4 + g][wj * 32 + q * 16 + c];
        b[q] = sm.fs[ks * 4 + g][wi * 32 + q * 16 + c];
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) acc[jj][ii] = Mfma<float>::mma(a[jj], b[ii], acc[jj][ii]);
    }
  }

  // This workgroup's 64x64 tile of the head's partial state (z from the jt == 0 tiles).
  float* part = partials + ((size_t)h * n_split + split) * part_floats<D>();
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[(size_t)(jt * AT + wj * 32 + jj * 16 + g * 4 + r) * D + it * AT + wi * 32 + ii * 16 +
             c] = acc[jj][ii][r];
  if (!is_v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.zred[row0][col4 * 4 + e] = zsum[e];
  }
  __syncthreads();
  if (tid < AT && jt == 0) {
    float s = 0.f;
    for (int q = 0; q < 8; ++q) s += sm.zred[q][tid];
    part[D * D + it * AT + tid] = s;
  }
}

// Threads per workgroup and workgroups per absorb of n_split token splits.
template <typename T, int D>
constexpr int threads() { return sizeof(T) == 2 ? D * 4 : NTHR; }
template <typename T, int D>
constexpr int items_per_split_head() { return sizeof(T) == 2 ? 1 : (D / AT) * (D / AT); }

// Absorb workgroup `item` of a 1-D enumeration: the split varies fastest, then the
// state tile (fp32), then the head.
template <typename T, int D>
__device__ __forceinline__ void item(int it, int n_split, const T* __restrict__ kev,
                                     const T* __restrict__ vev, int64_t n_ev, int64_t hs, int tps,
                                     float* __restrict__ partials) {
  const int split = it % n_split, rest = it / n_split;
  if constexpr (sizeof(T) == 2) {
    absorb_part_bf16<D>(split, rest, kev, vev, n_ev, hs, tps, n_split, partials);
  } else {
    constexpr int NTT = items_per_split_head<T, D>();
    absorb_part_f32<D>(split, rest % NTT, rest / NTT, kev, vev, n_ev, hs, tps, n_split, partials);
  }
}

}  // namespace absorb
}  // namespace hf
