// hf_device.h -- device helpers shared by the gfx950 kernels of libhf.
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32, wave64): with lane l, g = l / 16 and c = l % 16,
//   A operand (16 x KSTEP, row-major M x K): lane holds A[c][g*KP .. g*KP+KP)
//   B operand (KSTEP x 16, K x N):          lane holds B[g*KP .. g*KP+KP)[c]
//   C/D (16 x 16 fp32):                     lane holds D[4g + r][c], r = 0..3
// with KSTEP = 32, KP = 8 for bf16 and KSTEP = 4, KP = 1 for fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bf16 is carried as its 16-bit pattern

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// phi(x) = elu(x) + 1
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KSTEP = 32;
  static constexpr int KP = 8;
  typedef bf16x8 op_t;
  __device__ __forceinline__ static f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 4;
  static constexpr int KP = 1;
  typedef float op_t;
  __device__ __forceinline__ static f32x4 mma(op_t a, op_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Pack 8 bf16 patterns (as 4 uint32 words, low half first) into an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// Split 8 fp32 values into bf16 hi + lo operands (x ~= hi + lo to ~2^-17 relative):
// hi = bf16(x), lo = bf16(x - hi), both rounded to nearest even by the hardware pack.
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    l[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h[e] << 16),
                       x[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
  }
  hi = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
  lo = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
}

// Word k / 16-bit half e of a 16-byte register value (indices are compile-time
// constants after unrolling, so these fold to register selects).
__device__ __forceinline__ uint32_t word(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}
__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  return (word(v, e >> 1) >> ((e & 1) * 16)) & 0xFFFFu;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 16-byte global load with an in-bounds predicate (out of bounds reads nothing and
// yields zeros).
__device__ __forceinline__ uint4 ld16(const void* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : zero4();
}

// Map a launch-order workgroup id to a logical work index so that each XCD (the
// hardware hands consecutive workgroups to the 8 XCDs in turn) processes one
// contiguous range of the logical order. Returns -1 for padding workgroups.
__device__ __forceinline__ int xcd_remap(int wg, int n_wg_padded, int n_logical) {
  const int per = n_wg_padded >> 3;
  const int logical = (wg & 7) * per + (wg >> 3);
  return logical < n_logical ? logical : -1;
}


// ---------------------------------------------------------------------------
// LDS staging helpers shared by the MFMA kernels.

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, if lane
// 4j + p supplies the address of 4 consecutive elements M[j][4p .. 4p+3], lane i
// receives M[0..3][i].
__device__ __forceinline__ v4i16 lds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}


typedef __attribute__((address_space(3))) void lds_void;

// This wave's LDS reads are complete, then a plain s_barrier (no memory fence, so
// in-flight global->LDS loads are not waited for).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte global -> LDS load of every lane: lane l's 16 bytes land at LDS byte
// offset lds_off + 16 l (lds_off wave-uniform). Issued from inline asm so that the
// compiler does not track it: the kernel orders these loads itself (wait_vmem and
// the barriers), and the compiler's own tracking would make every LDS read wait
// for all of them. Vector-memory operations complete in issue order, so loads the
// compiler does not know about can only make its own waits stricter. m0 is used
// by nothing else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Address = wave-uniform base (SGPR pair) + per-lane 32-bit byte offset. The
// compiler cannot see hazards inside the asm, so two wait states separate the m0
// write (and any VALU write of the offset register) from the load, as the
// compiler itself does for this instruction.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_off), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p);
}

// LDS accesses by byte offset: a lane-varying offset plus a compile-time constant
// lets the constant go into the instruction's offset field.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(uint32_t byte_off) {
  const u32x4_t v =
      *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((size_t)byte_off);
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float2 lds_ld8f(uint32_t byte_off) {
  const f32x2_t v =
      *reinterpret_cast<const __attribute__((address_space(3))) f32x2_t*>((size_t)byte_off);
  return make_float2(v.x, v.y);
}
__device__ __forceinline__ v4i16 lds_tr8(uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((size_t)byte_off));
}


// Swizzle of the 16-byte chunks of a tile row in LDS (64-row K/V tiles, rows of
// CPR chunks): chunk cc of row r lives in slot cc ^ swz(r). Chosen (as a linear map
// over GF(2) of row bits 0..3) so that both ds_read_b128 operand reads (lane (g, c)
// reads chunk 4s + g of row c) and the transposing reads (8 rows x one aligned chunk
// pair per half-wave) are free of bank conflicts; with 128-byte rows (CPR = 8) two
// rows share the 64 banks, so swz has 3 bits.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) return ((r & 1) << 3) ^ (r & 6) ^ (((r >> 3) & 1) * 5);
  else return (r & 6) ^ (((r >> 3) & 1) * 5);
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt field");  // 6 bits: [3:0] and [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Cross-lane reductions over the 4 lane groups (l, l^16, l^32, l^48) that hold the
// same MFMA column: the gfx950 permlane swaps exchange lane halves / 16-lane rows.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  // Both partners form the same two-term sums, so every lane ends with the same total.
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace hf
