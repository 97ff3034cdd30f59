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

template <int D>
__global__ __launch_bounds__(NTHR) void absorb_bf16(const bf16_t* __restrict__ kev,
                                                    const bf16_t* __restrict__ vev,
                                                    int64_t n_ev, int64_t hs, int tps,
                                                    int n_split,
                                                    float* __restrict__ partials) {
  constexpr int NT = D / AT;  // tiles per edge
  __shared__ AbsorbSmem<bf16_t> sm;
  const int split = blockIdx.x, tile = blockIdx.y, h = blockIdx.z;
  const int jt = tile / NT, it = tile % NT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wj = w >> 1, wi = w & 1;
  const int64_t n0 = (int64_t)split * tps;
  const int64_t n1 = n0 + tps < n_ev ? n0 + tps : n_ev;

  // Staging role: threads 0..127 stage V columns jt*64.., threads 128..255 stage
  // K columns it*64..; each handles 4 consecutive tokens x 8 features.
  const bool is_v = tid < 128;
  const int sid = tid & 127;
  const int tg = sid >> 3, cg = sid & 7;
  const bf16_t* src = (is_v ? vev + (size_t)jt * AT : kev + (size_t)it * AT) + (size_t)h * hs +
                      cg * 8;
  float zsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) zsum[e] = 0.f;

  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = n0; t0 < n1; t0 += TS) {
    uint4 rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = t0 + tg * 4 + r;
      rows[r] = ld16(src + n * D, n < n1);
    }
    __syncthreads();  // previous iteration's MFMAs are done with the tiles
    if (is_v) {
      // Transpose 4 tokens x 8 features into 8 rows of 4 tokens.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = half16(rows[r], e);
        uint2 pk = make_uint2(v4[0] | (v4[1] << 16), v4[2] | (v4[3] << 16));
        *reinterpret_cast<uint2*>(&sm.vt[cg * 8 + e][tg * 4]) = pk;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t hi4[4], lo4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = t0 + tg * 4 + r < n1;
          const float x = bf16_to_f32(half16(rows[r], e));
          const float f = ok ? phi(x) : 0.f;
          zsum[e] += f;
          hi4[r] = f32_to_bf16_bits(f);
          lo4[r] = f32_to_bf16_bits(f - bf16_to_f32(hi4[r]));
        }
        *reinterpret_cast<uint2*>(&sm.fhi[cg * 8 + e][tg * 4]) =
            make_uint2(hi4[0] | (hi4[1] << 16), hi4[2] | (hi4[3] << 16));
        *reinterpret_cast<uint2*>(&sm.flo[cg * 8 + e][tg * 4]) =
            make_uint2(lo4[0] | (lo4[1] << 16), lo4[2] | (lo4[3] << 16));
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TS / 32; ++ks) {
      bf16x8 a[2], bh[2], bl[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        a[q] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.vt[wj * 32 + q * 16 + c][ks * 32 + g * 8]));
        bh[q] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.fhi[wi * 32 + q * 16 + c][ks * 32 + g * 8]));
        bl[q] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.flo[wi * 32 + q * 16 + c][ks * 32 + g * 8]));
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          acc[jj][ii] = Mfma<bf16_t>::mma(a[jj], bh[ii], acc[jj][ii]);
          acc[jj][ii] = Mfma<bf16_t>::mma(a[jj], bl[ii], acc[jj][ii]);
        }
    }
  }

  // Partial tile -> workspace.
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
    for (int e = 0; e < 8; ++e) sm.zred[tg][cg * 8 + e] = zsum[e];
  }
  __syncthreads();
  if (tid < AT) {
    float s = 0.f;
    for (int q = 0; q < 16; ++q) s += sm.zred[q][tid];
    part[AT * AT + tid] = s;
  }
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
