// pkv_common.h - device types and small helpers shared by the gfx950 kernels.
//
// Internal to libpagedkv.so.  Wave64 throughout: one wavefront = 64 lanes;
// the 16x16 matrix-core ops see a lane as (group g = lane / 16, row/column
// r = lane % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pkv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum KvType { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_E4M3 = 3 };

constexpr int kBlockSize = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int T> struct ElemBytes;
template <> struct ElemBytes<KV_F32> { static constexpr int value = 4; };
template <> struct ElemBytes<KV_F16> { static constexpr int value = 2; };
template <> struct ElemBytes<KV_BF16> { static constexpr int value = 2; };
template <> struct ElemBytes<KV_E4M3> { static constexpr int value = 1; };

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// Element offset of (token slot t, dim d) inside a V tile, n = 4 / elem bytes.
__device__ __forceinline__ int v_tile_elem(int t, int d, int n) {
  return (((((d / (16 * n)) * 4 + t / 4) * 16 + d % 16) * n + (d / 16) % n) * 4 + t % 4);
}

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Raw buffer access: a 128-bit descriptor (base, byte size, gfx9 dword3 with
// a 32-bit data format) in scalar registers; reads past `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_tile_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Cache-policy operand marking a load non-temporal (the `nt` bit): the lines
// are streamed through L2 and the memory-side cache with early eviction.  On
// gfx950 a plain read stream reaches ~6.3 TB/s and an `nt` one ~7.1 TB/s.
constexpr int kStreamLoad = 2;
template <int POLICY>
__device__ __forceinline__ u32x4 buffer_ld16_policy(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

// Cache-policy operand of buffer loads/stores selecting device (agent)
// scope on gfx950: the access is coherent across the XCDs' L2 caches.
constexpr int kDeviceScope = 16;
// s_waitcnt immediate for vmcnt(0) with the other counters left alone.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum over the four lanes that share lane % 16 (lanes r, r+16, r+32,
// r+48), with gfx950's lane swaps (VALU, no LDS round trip): with both
// operands x, v_permlane16_swap returns (rows 0,0,2,2 ; rows 1,1,3,3) of x
// and v_permlane32_swap (lanes 0-31 twice ; lanes 32-63 twice), so the two
// results hold every lane's partner across 16 (then 32).  The partner sums
// pair the same values as x + shuffle-xor would, so the bits match.
// The second operand goes through an opaque copy: given one value for both,
// the compiler takes the two results as equal and drops the combine.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t x) {
  uint32_t y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}
template <bool ROWS16>
__device__ __forceinline__ void lane_swap(float x, float& lo_half, float& hi_half) {
  const uint32_t u = __float_as_uint(x);
  const auto r = ROWS16 ? __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false)
                        : __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
  lo_half = __uint_as_float(r[0]);   // the lower of the two partner lanes' values
  hi_half = __uint_as_float(r[1]);   // the upper one's
}
__device__ __forceinline__ float max_over_groups(float x) {
  float a, b;
  lane_swap<true>(x, a, b);
  x = fmaxf(a, b);
  lane_swap<false>(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_over_groups(float x) {
  // (x_l + x_(l^16)) + (x_(l^32) + x_(l^48)), as the shuffle form; IEEE
  // addition is commutative, so which operand is the lane's own is moot
  float a, b;
  lane_swap<true>(x, a, b);
  x = a + b;
  lane_swap<false>(x, a, b);
  return a + b;
}

// ------------------------------------------------------------ matrix cores
// D(16x16, f32) += A(16xK) * B(Kx16).  Lane l supplies row l%16 of A and
// column l%16 of B, each with its k-slots (l/16)*k_per_lane + j; it receives
// D[4*(l/16) + j][l%16] for j = 0..3.  Since A and B share the k-slot
// assignment, which hardware k a slot is does not change the sum.
__device__ __forceinline__ f32x4 mma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------- E4M3
// OCP E4M3FN codes -> f16, exactly, with the gfx950 packed conversion
// (one instruction per two codes; every E4M3 value is an f16 value).  The
// conversion reads bytes 0-1 (first call) and 2-3 (second) of x, low byte
// to the low half, so four codes come out in byte order.
__device__ __forceinline__ f16x4 e4m3x4_to_f16x4(uint32_t x) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
  return bitcast<f16x4>(u32x2{a, b});
}
// Sixteen codes (the bytes of c in order) -> two groups of eight f16.
__device__ __forceinline__ void e4m3x16_to_f16x8x2(u32x4 c, f16x8& lo, f16x8& hi) {
  const u32x2 c0 = bitcast<u32x2>(e4m3x4_to_f16x4(c.x)), c1 = bitcast<u32x2>(e4m3x4_to_f16x4(c.y));
  const u32x2 c2 = bitcast<u32x2>(e4m3x4_to_f16x4(c.z)), c3 = bitcast<u32x2>(e4m3x4_to_f16x4(c.w));
  lo = bitcast<f16x8>(u32x4{c0.x, c0.y, c1.x, c1.y});
  hi = bitcast<f16x8>(u32x4{c2.x, c2.y, c3.x, c3.y});
}

// fp32 in [-448, 448] -> nearest OCP E4M3 code, ties to even.  Below the
// smallest normal 2^-6 the code's mantissa is the value in units of 2^-9,
// rounded to nearest even; above, the fp32 exponent is re-biased from 127 to
// 7 and the 23-bit mantissa rounded to 3 bits (a carry rolls into the
// exponent).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t u = __float_as_uint(a) - (120u << 23);
    mag = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
  }
  return sign | mag;
}

}  // namespace pkv
