// hf_absorb.hip -- fold evicted tokens into the linear state (gfx950).
//
// Per head: S[j][i] += sum_n V[n][j] phi(K[n][i]) and z[i] += sum_n phi(K[n][i]),
// the incremental absorption of evicted tokens into a compact key-value state
// described in the authors' abstract (fugumt.com listing of arXiv 2604.10103v1)
// and in the gist.science English summary "Long-Horizon Streaming Video
// Generation via Hybrid Attention with Decoupled Distillation", 2.A.1.
//
// Work split: grid (token split, 64x64 output tile, head). A workgroup stages 64
// evicted tokens at a time in LDS (transposed so that tokens, the contraction
// index, are contiguous per MFMA lane), forms phi(K) in fp32 and, for bf16
// inputs, splits it into bf16 hi + lo so that the bf16 MFMA keeps ~fp32
// accuracy (V is exact in bf16). Each workgroup writes a partial 64x64 tile (and
// a partial z) to the workspace; a second kernel adds the partials in split
// order to S and z. No atomics or device-wide fences are involved (on a chip
// whose XCDs have separate L2 caches those would have to write the L2 back),
// and the order of every sum is fixed, so the result is bitwise reproducible.
#include "hf_device.h"
#include "hf_launch.h"

namespace hf {

namespace {

constexpr int AT = 64;       // output tile edge
constexpr int TS = 64;       // tokens staged per iteration
constexpr int NTHR = 256;    // 4 waves, each owns a 32x32 quarter of the tile
constexpr int PART = AT * AT + AT;  // floats per partial: tile + z slice

// bf16: transposed tiles [64 features][TS tokens (+8 pad)] of V, phi_hi, phi_lo.
constexpr int BPITCH = TS + 8;
// fp32: row-major tiles [TS tokens][64 features (+4 pad)] of V and phi.
constexpr int FPITCH = AT + 4;

template <typename T>
struct AbsorbSmem;

template <>
struct AbsorbSmem<bf16_t> {
  bf16_t vt[AT][BPITCH];
  bf16_t fhi[AT][BPITCH];
  bf16_t flo[AT][BPITCH];
  float zred[16][AT];
};

template <>
struct AbsorbSmem<float> {
  float vs[TS][FPITCH];
  float fs[TS][FPITCH];
  float zred[8][AT];
};

// Second pass: S[h][tile] += sum_s partial[s] (and z), splits added in order.
template <int D>
__global__ __launch_bounds__(NTHR) void absorb_reduce(const float* __restrict__ partials,
                                                      int n_split, float* __restrict__ S,
                                                      float* __restrict__ z) {
  constexpr int NT = D / AT;
  const int e = blockIdx.x * NTHR + threadIdx.x;
  const int tile = blockIdx.y, h = blockIdx.z;
  const int jt = tile / NT, it = tile % NT;
  if (e >= PART || (e >= AT * AT && jt != 0)) return;
  const float* p = partials + ((size_t)h * NT * NT + tile) * n_split * PART + e;
  float acc = 0.f;
  for (int s = 0; s < n_split; ++s) acc += p[(size_t)s * PART];
  if (e < AT * AT) {
    float* dst = S + (size_t)h * D * D + (size_t)(jt * AT + e / AT) * D + it * AT + e % AT;
    *dst += acc;
  } else {
    z[(size_t)h * D + it * AT + (e - AT * AT)] += acc;
  }
}

// bf16: K and V token tiles (64 tokens x 64 features, 128-byte rows) go straight
// from global memory into a 4-stage LDS ring (16-byte global->LDS loads); chunk
// cc of row r sits in slot cc ^ (r mod 8) ^ 4((r / 8) mod 2), so the transposing
// reads of the four lane groups (rows 8 apart) fall on different banks. Both MFMA
// operands are read with the transposing LDS read (tokens, the contraction index,
// end up contiguous per lane); phi, the tail mask and the hi/lo split are applied
// to the K operand in registers.
__device__ __forceinline__ int abs_slot(int row, int cc) {
  return cc ^ (row & 7) ^ (((row >> 3) & 1) << 2);
}

template <int D>
__global__ __launch_bounds__(NTHR) void absorb_bf16(const bf16_t* __restrict__ kev,
                                                    const bf16_t* __restrict__ vev,
                                                    int64_t n_ev, int64_t hs, int tps,
                                                    int n_split,
                                                    float* __restrict__ partials) {
  constexpr int NT = D / AT;       // tiles per edge
  constexpr int NST = 4;           // pipeline stages
  constexpr int TCH = TS * AT / 8; // 16-byte chunks per tile (512)
  constexpr int LPT = TCH / NTHR;  // loads per lane per tile (2)
  __shared__ uint4 lds_k[NST][TCH];
  __shared__ uint4 lds_v[NST][TCH];
  const int split = blockIdx.x, tile = blockIdx.y, h = blockIdx.z;
  const int jt = tile / NT, it = tile % NT;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (int64_t)split * tps;
  const int64_t n1 = n0 + tps < n_ev ? n0 + tps : n_ev;
  const int niter = (int)((n1 - n0 + TS - 1) / TS);
  const bf16_t* kb = kev + (size_t)h * hs + it * AT;
  const bf16_t* vb = vev + (size_t)h * hs + jt * AT;

  // Load u of wave w fills chunks (u*4 + w)*64 + lane of a tile.
  uint32_t loff[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    const int P = (u * 4 + w) * 64 + lane;
    const int row = P / 8, slot = P % 8;
    const int cc = slot ^ (row & 7) ^ (((row >> 3) & 1) << 2);  // inverse of abs_slot
    loff[u] = (uint32_t)(row * D + cc * 8) * 2u;
  }
  auto issue = [&](int t) {
    const int st = t % NST;
    const bf16_t* kt = kb + (size_t)(n0 + (int64_t)t * TS) * D;
    const bf16_t* vt = vb + (size_t)(n0 + (int64_t)t * TS) * D;
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds_offset(&lds_k[st][0]) + w * 1024);
    const uint32_t vbase = __builtin_amdgcn_readfirstlane(lds_offset(&lds_v[st][0]) + w * 1024);
    const int64_t left = n1 - (n0 + (int64_t)t * TS);
    if (left >= TS) {
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        lds_dma16(kt, loff[u], kbase + u * 4096);
        lds_dma16(vt, loff[u], vbase + u * 4096);
      }
    } else {  // partial last tile: rows past the end repeat the last row (masked below)
      const uint32_t rb = D * 2, last = (uint32_t)left - 1;
#pragma unroll
      for (int u = 0; u < LPT; ++u) {
        const uint32_t row = loff[u] / rb;
        const uint32_t off = row <= last ? loff[u] : last * rb + loff[u] % rb;
        lds_dma16(kt, off, kbase + u * 4096);
        lds_dma16(vt, off, vbase + u * 4096);
      }
    }
  };

  // Wave w owns key-feature columns 16w .. 16w+15 of the tile and all 64 value
  // rows, so phi of every K element is formed exactly once.
  f32x4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  const int jr = (lane & 15) >> 2, pp = lane & 3;  // transposing-read source role

  // Byte address of the 8 bytes (row, 4 features at col) of a tile.
  auto tr_addr = [&](const uint4* base, int row, int col) {
    return reinterpret_cast<const char*>(base) + (row * 8 + abs_slot(row, col >> 3)) * 16 +
           ((col >> 2) & 1) * 8;
  };

  for (int t = 0; t < NST - 1 && t < niter; ++t) issue(t);
  for (int t = 0; t < niter; ++t) {
    // Stage t has landed once at most (#later stages issued) * 2 * LPT loads remain.
    const int later = (niter - 1 - t) < (NST - 2) ? (niter - 1 - t) : (NST - 2);
    if (later >= 2) wait_vmem<2 * 2 * LPT>();
    else if (later == 1) wait_vmem<2 * LPT>();
    else wait_vmem<0>();
    lds_barrier();
    if (t + NST - 1 < niter) issue(t + NST - 1);  // its stage was consumed at t - 1
    const int st = t % NST;
    const int valid = (int)(n1 - (n0 + (int64_t)t * TS));  // tokens of this tile in range
#pragma unroll
    for (int ks = 0; ks < TS / 32; ++ks) {
      const int r0 = ks * 32 + g * 8 + jr;  // rows of the first transposing read
      // B: phi(K) for this wave's 16 columns, tokens ks*32 + 8g + 0..7, split hi + lo.
      const int ck = w * 16 + pp * 4;
      const v4i16 k0 = lds_read_tr(tr_addr(lds_k[st], r0, ck));
      const v4i16 k1 = lds_read_tr(tr_addr(lds_k[st], r0 + 4, ck));
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (uint32_t)(uint16_t)(e < 4 ? k0[e] : k1[e - 4]);
        const int tok = ks * 32 + g * 8 + e;  // token of element e in this lane
        f[e] = tok < valid ? phi(bf16_to_f32(bits)) : 0.f;
        zacc += f[e];
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
        lw[e] = pack_bf16x2(f[2 * e] - __uint_as_float(hw[e] << 16),
                            f[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
      }
      const bf16x8 bh = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8 bl = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
      // A: V^T for the 4 value-row tiles.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cv = q * 16 + pp * 4;
        const v4i16 v0 = lds_read_tr(tr_addr(lds_v[st], r0, cv));
        const v4i16 v1 = lds_read_tr(tr_addr(lds_v[st], r0 + 4, cv));
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[q] = Mfma<bf16_t>::mma(a, bh, acc[q]);
        acc[q] = Mfma<bf16_t>::mma(a, bl, acc[q]);
      }
    }
  }

  // Partial tile and partial z.
  float* part = partials + (((size_t)h * NT * NT + tile) * n_split + split) * PART;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[(q * 16 + g * 4 + r) * AT + w * 16 + c] = acc[q][r];
  const float zs = sum_over_groups(zacc);
  if (g == 0) part[AT * AT + w * 16 + c] = zs;
}

template <int D>
__global__ __launch_bounds__(NTHR) void absorb_f32(const float* __restrict__ kev,
                                                   const float* __restrict__ vev, int64_t n_ev,
                                                   int64_t hs, int tps, int n_split,
                                                   float* __restrict__ partials) {
  constexpr int NT = D / AT;
  __shared__ AbsorbSmem<float> sm;
  const int split = blockIdx.x, tile = blockIdx.y, h = blockIdx.z;
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

  float* part = partials + (((size_t)h * NT * NT + tile) * n_split + split) * PART;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[(wj * 32 + jj * 16 + g * 4 + r) * AT + wi * 32 + ii * 16 + c] = acc[jj][ii][r];
  if (!is_v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.zred[row0][col4 * 4 + e] = zsum[e];
  }
  __syncthreads();
  if (tid < AT) {
    float s = 0.f;
    for (int q = 0; q < 8; ++q) s += sm.zred[q][tid];
    part[AT * AT + tid] = s;
  }
}

}  // namespace

AbsorbPlan absorb_plan(int64_t n_ev) {
  AbsorbPlan p;
  int64_t per = (n_ev + kAbsorbMaxSplits - 1) / kAbsorbMaxSplits;
  if (per < 256) per = 256;
  per = (per + TS - 1) / TS * TS;
  p.tokens_per_split = (int)per;
  p.n_split = (int)((n_ev + per - 1) / per);
  if (p.n_split < 1) p.n_split = 1;
  return p;
}

size_t absorb_partial_floats(int heads, int d) {
  const int nt = d / AT;
  return (size_t)heads * nt * nt * kAbsorbMaxSplits * PART;
}

hipError_t launch_absorb(int dtype, int heads, int d, const void* k, const void* v, int64_t n_ev,
                         int64_t head_stride, float* S, float* z, float* partials,
                         hipStream_t stream) {
  const AbsorbPlan p = absorb_plan(n_ev);
  const int nt = d / AT;
  dim3 grid(p.n_split, nt * nt, heads);
#define HF_ABS(KER, T, D)                                                                     \
  KER<D><<<grid, NTHR, 0, stream>>>(static_cast<const T*>(k), static_cast<const T*>(v), n_ev, \
                                    head_stride, p.tokens_per_split, p.n_split, partials)
  if (dtype == 0) {
    if (d == 128) HF_ABS(absorb_bf16, bf16_t, 128); else HF_ABS(absorb_bf16, bf16_t, 64);
  } else {
    if (d == 128) HF_ABS(absorb_f32, float, 128); else HF_ABS(absorb_f32, float, 64);
  }
#undef HF_ABS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 rgrid((PART + NTHR - 1) / NTHR, nt * nt, heads);
  if (d == 128)
    absorb_reduce<128><<<rgrid, NTHR, 0, stream>>>(partials, p.n_split, S, z);
  else
    absorb_reduce<64><<<rgrid, NTHR, 0, stream>>>(partials, p.n_split, S, z);
  return hipGetLastError();
}

}  // namespace hf
