// decode.hip - paged grouped-query decode attention for gfx950.
//
// What it computes: for sequence b and query head i (KV head h = i / G),
// softmax(q . K^T * scale) V over the first L_b tokens of the sequence,
// gathered from the block pool through its block table, with online softmax
// ("rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
// row "PagedAttention V2"; "LLM Serving Kernels", section "Projects", row 04:
// page tables, GQA/MQA, online softmax).  In split mode each partition of
// the context yields a normalised partial output and its log-sum-exp; the
// reduce kernel merges them (flash-decoding).  Also here: the same with a
// sliding window (only the last W positions), a balanced schedule (equal
// 16-token tile shares per wave, split at any point, merged by log-sum-exp),
// and the multi-token step (several new tokens per sequence, causal).
//
// Kernels: paged_decode_kernel / paged_decode_persistent (one pass, split
// partials, or split with an in-kernel merge), paged_decode_stream +
// stream_merge_kernel (balanced schedule), paged_prefill_persistent +
// prefill_merge_kernel (multi-token step), lse_merge_kernel (partition
// merge of the split pair).
//
// How, on CDNA4:
//  * One workgroup = NW wave64s = one (partition, kv head, sequence).  The
//    waves take the partition's 16-token blocks round-robin, each keeping its
//    own running max / sum / accumulator, and merge through LDS at the end.
//  * GQA packing: all G (<= 16) query heads of a KV head are the 16 columns
//    of one matrix-core tile, so each K/V tile fetched from HBM serves the
//    whole group.  S^T[16 tokens x 16 heads] = K_tile[16 x D] * Q^T[D x 16]
//    and O^T[D x 16 heads] += V^T[D x 16 tokens] * P^T[16 tokens x 16 heads]
//    run on MFMA 16x16 ops; unused head columns carry q = 0.
//  * The tile layouts (see pagedkv.h) make every lane's operand a 16-byte
//    load and every wave load one contiguous 1 KiB, straight into registers.
//  * S^T lands with each lane holding 4 tokens of one head, exactly the
//    B-operand layout P^T needs for the PV product: the softmax needs only a
//    lane-local max over 4 values plus two cross-group shuffles per block.
//  * P stays fp32-accurate: 16-bit PV uses P = hi + lo (two 16-bit parts,
//    two MFMAs), so only V's own rounding is in the product.  The
//    multi-token step, when it has many rows per sequence, takes tiles in
//    pairs and runs PV on the K = 32 form (twice the rate of K = 16).
//  * E4M3 codes decode to fp16 exactly with the packed hardware conversion;
//    the block's K scale folds into its logit factor, its V scale into P
//    (times a running power of two that keeps P inside f16's range).
//  * Softmax runs in base 2 (log2 e folded into the scale).
#include "pkv_common.h"
#include "pkv_launch.h"
#include "pkv_sched.h"

#include <algorithm>
#include <atomic>

namespace pkv {

// ------------------------------------------------------------ tile traits
// Per KV element type: NLOAD 16-byte loads per lane for a K tile and as many
// for a V tile; NQ 16-byte q-operand registers; NT = D/16 output d-tiles.

template <int KVT, int D> struct TileOps;

// f16 / bf16 KV: QK^T on 16x16x32 MFMA, PV on 16x16x16 MFMA.
template <int KVT, int D> struct Tile16 {
  static constexpr bool kBf16 = (KVT == KV_BF16);
  typedef typename std::conditional<kBf16, bf16x8, f16x8>::type V8;
  typedef typename std::conditional<kBf16, bf16x4, f16x4>::type V4;
  typedef typename std::conditional<kBf16, __bf16, _Float16>::type S;
  static constexpr int NLOAD = D * 2 / 64;
  static constexpr int NQ = NLOAD;
  static constexpr int NT = D / 16;
  typedef uint16_t QElem;

  // Lane (g, r): K load m holds token r, dims [8c, 8c+8) with c = 4m + g;
  // the q operand holds the same dims of query head r (qoff: head r's row).
  __device__ static void load_q(u32x4 (&qop)[NQ], __amdgpu_buffer_rsrc_t qr, uint32_t qoff, int g) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = buffer_ld16(qr, qoff + (8 * (4 * m + g)) * 2);
  }
  __device__ static f32x4 qk(const u32x4 (&kt)[NLOAD], const u32x4 (&qop)[NQ]) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) s = mma_k32(bitcast<V8>(kt[m]), bitcast<V8>(qop[m]), s);
    return s;
  }
  // Zero V of tokens 4g + j with j >= nv (V load m: dwords x,y = d-tile 2m,
  // tokens (0,1),(2,3); z,w = d-tile 2m+1).
  __device__ static void mask_v(u32x4 (&vt)[NLOAD], int nv) {
    const uint32_t m01 = (nv > 0 ? 0x0000FFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
    const uint32_t m23 = (nv > 2 ? 0x0000FFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      vt[m].x &= m01; vt[m].y &= m23; vt[m].z &= m01; vt[m].w &= m23;
    }
  }
  // P as hi + lo 16-bit parts: hi = p rounded to the 16-bit type, lo =
  // (p - hi) rounded.  For bf16 the float value of hi is its bits moved to
  // the top half, read off the packed pair, not a second conversion.
  template <typename VN, int N>
  __device__ static void split_p(const float (&p)[N], VN& hi, VN& lo) {
    if constexpr (kBf16) {
      typedef float F2 __attribute__((ext_vector_type(2)));
      typedef __bf16 B2 __attribute__((ext_vector_type(2)));
      typedef uint32_t UW __attribute__((ext_vector_type(N / 2)));
      UW hw, lw;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        const uint32_t w = bitcast<uint32_t>(__builtin_convertvector(F2{p[2 * i], p[2 * i + 1]}, B2));
        hw[i] = w;
        const F2 r = {p[2 * i] - __uint_as_float(w << 16), p[2 * i + 1] - __uint_as_float(w & 0xFFFF0000u)};
        lw[i] = bitcast<uint32_t>(__builtin_convertvector(r, B2));
      }
      hi = bitcast<VN>(hw);
      lo = bitcast<VN>(lw);
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const S h = static_cast<S>(p[j]);
        hi[j] = h;
        lo[j] = static_cast<S>(p[j] - static_cast<float>(h));
      }
    }
  }
  __device__ static void pv(f32x4 (&o)[NT], const u32x4 (&vt)[NLOAD], const float (&p)[4], float) {
    V4 hi, lo;
    split_p(p, hi, lo);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x2 a = (n & 1) ? u32x2{vt[n >> 1].z, vt[n >> 1].w} : u32x2{vt[n >> 1].x, vt[n >> 1].y};
      o[n] = mma_k16(bitcast<V4>(a), hi, o[n]);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x2 a = (n & 1) ? u32x2{vt[n >> 1].z, vt[n >> 1].w} : u32x2{vt[n >> 1].x, vt[n >> 1].y};
      o[n] = mma_k16(bitcast<V4>(a), lo, o[n]);
    }
  }
  // PV over two tiles (a, b) at once on the K = 32 form, at twice the
  // K = 16 form's rate.  The sum over k takes any order of the 32 tokens as
  // long as both operands use it: k-slots 8g..8g+3 are tile a's tokens
  // 4g..4g+3 and 8g+4..8g+7 tile b's, which is what lane (g, r) already
  // holds of P (p[0..3] for a, p[4..7] for b) and of V (8 bytes per d-tile
  // and tile), so the operands form without lane exchanges.
  __device__ static void pv2(f32x4 (&o)[NT], const u32x4 (&va)[NLOAD], const u32x4 (&vb)[NLOAD],
                             const float (&p)[8]) {
    V8 hi, lo;
    split_p(p, hi, lo);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x4 a = (n & 1) ? u32x4{va[n >> 1].z, va[n >> 1].w, vb[n >> 1].z, vb[n >> 1].w}
                              : u32x4{va[n >> 1].x, va[n >> 1].y, vb[n >> 1].x, vb[n >> 1].y};
      o[n] = mma_k32(bitcast<V8>(a), hi, o[n]);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x4 a = (n & 1) ? u32x4{va[n >> 1].z, va[n >> 1].w, vb[n >> 1].z, vb[n >> 1].w}
                              : u32x4{va[n >> 1].x, va[n >> 1].y, vb[n >> 1].x, vb[n >> 1].y};
      o[n] = mma_k32(bitcast<V8>(a), lo, o[n]);
    }
  }
};
template <int D> struct TileOps<KV_F16, D> : Tile16<KV_F16, D> {};
template <int D> struct TileOps<KV_BF16, D> : Tile16<KV_BF16, D> {};

// f32 KV: 16x16x4 f32 MFMA for both products.
template <int D> struct TileOps<KV_F32, D> {
  static constexpr int NLOAD = D / 16;
  static constexpr int NQ = NLOAD;
  static constexpr int NT = D / 16;
  __device__ static void load_q(u32x4 (&qop)[NQ], __amdgpu_buffer_rsrc_t qr, uint32_t qoff, int g) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = buffer_ld16(qr, qoff + (4 * (4 * m + g)) * 4);
  }
  // K load m: token r, dims [4c, 4c+4), c = 4m + g; one MFMA per dim.
  __device__ static f32x4 qk(const u32x4 (&kt)[NLOAD], const u32x4 (&qop)[NQ]) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      const f32x4 k = bitcast<f32x4>(kt[m]);
      const f32x4 q = bitcast<f32x4>(qop[m]);
#pragma unroll
      for (int i = 0; i < 4; ++i) s = mma_k4(k[i], q[i], s);
    }
    return s;
  }
  __device__ static void mask_v(u32x4 (&vt)[NLOAD], int nv) {
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      if (nv <= 0) vt[m].x = 0u;
      if (nv <= 1) vt[m].y = 0u;
      if (nv <= 2) vt[m].z = 0u;
      if (nv <= 3) vt[m].w = 0u;
    }
  }
  // V load n: d-tile n, row 16n + r, tokens 4g..4g+3; one MFMA per token.
  __device__ static void pv(f32x4 (&o)[NT], const u32x4 (&vt)[NLOAD], const float (&p)[4], float) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const f32x4 v = bitcast<f32x4>(vt[n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[n] = mma_k4(v[j], p[j], o[n]);
    }
  }
};

// E4M3 KV with f16 queries: codes decode to f16 (exact) for f16 MFMA.
template <int D> struct TileOps<KV_E4M3, D> {
  static constexpr int NLOAD = D / 64;
  static constexpr int NQ = 2 * NLOAD;
  static constexpr int NT = D / 16;
  // K load m: token r, dims [16c, 16c+16), c = 4m + g, as two halves of 8.
  __device__ static void load_q(u32x4 (&qop)[NQ], __amdgpu_buffer_rsrc_t qr, uint32_t qoff, int g) {
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      qop[2 * m] = buffer_ld16(qr, qoff + (16 * (4 * m + g)) * 2);
      qop[2 * m + 1] = buffer_ld16(qr, qoff + (16 * (4 * m + g)) * 2 + 16);
    }
  }
  __device__ static f32x4 qk(const u32x4 (&kt)[NLOAD], const u32x4 (&qop)[NQ]) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      f16x8 lo, hi;
      e4m3x16_to_f16x8x2(kt[m], lo, hi);
      s = mma_k32(lo, bitcast<f16x8>(qop[2 * m]), s);
      s = mma_k32(hi, bitcast<f16x8>(qop[2 * m + 1]), s);
    }
    return s;
  }
  // V load m: dword qd = d-tile 4m + qd, bytes = tokens 4g..4g+3.
  __device__ static void mask_v(u32x4 (&vt)[NLOAD], int nv) {
    const uint32_t mk = (nv > 0 ? 0x000000FFu : 0u) | (nv > 1 ? 0x0000FF00u : 0u) |
                        (nv > 2 ? 0x00FF0000u : 0u) | (nv > 3 ? 0xFF000000u : 0u);
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      vt[m].x &= mk; vt[m].y &= mk; vt[m].z &= mk; vt[m].w &= mk;
    }
  }
  // pscale = the block's V scale times a power of two chosen by the caller
  // (attend_packs) so that P * pscale stays inside f16's range for the hi/lo
  // split whatever the scale; the caller removes the power of two at the end.
  __device__ static void pv(f32x4 (&o)[NT], const u32x4 (&vt)[NLOAD], const float (&p)[4], float pscale) {
    // hi + lo must split one fp32 value ps exactly.  Left to itself the
    // compiler derives the hi that lo is taken against straight from the
    // unrounded product p * pscale (a mixed-precision multiply with one f16
    // rounding) while the hi fed to the matrix cores rounds the fp32
    // product; where those two differ the pair is off by one f16 ulp of ps
    // (2^-11 relative).  Passing the product through an opaque copy makes
    // both come from the same fp32 register.
#pragma clang fp contract(off)
    f16x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ps = __uint_as_float(opaque_copy(__float_as_uint(p[j] * pscale)));
      const _Float16 h = static_cast<_Float16>(ps);
      hi[j] = h;
      lo[j] = static_cast<_Float16>(ps - static_cast<float>(h));
    }
    f16x4 v[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) v[n] = e4m3x4_to_f16x4(vt[n >> 2][n & 3]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mma_k16(v[n], hi, o[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mma_k16(v[n], lo, o[n]);
  }
};

// ------------------------------------------------------------------ store
// Four consecutive dims of one head in the requested output type.
__device__ __forceinline__ void store4(void* base, size_t idx, int out_dtype, f32x4 v) {
  if (out_dtype == KV_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = v;
  } else if (out_dtype == KV_F16) {
    f16x4 h = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]),
               static_cast<_Float16>(v[2]), static_cast<_Float16>(v[3])};
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(base) + idx) = h;
  } else {
    bf16x4 h = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]),
                static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(base) + idx) = h;
  }
}

// ----------------------------------------------------------------- merge
// One wave merges n partial rows of one (sequence, query head): row s has
// a normalised output o_s (D floats at o_row0 + s*D) and a log-sum-exp
// lse_s; out = sum_s w_s o_s / sum_s w_s with w_s = exp(lse_s - max lse).
// The rows go in batches of eight with an online (running-max) merge, so
// each batch's lse and o loads issue together and n <= 8 costs one round
// trip.  Loads are bounded buffer loads (past row n they read 0 and get
// weight 0), so none is conditional.  The order of summation is fixed:
// s = 0, 1, ...  Returns this lane's D/64 output dims (lane * D/64 + k).
// Adds n rows to a running merge (max M in log2 units, weight sum wsum,
// unnormalised sum acc).
template <int D, bool COH>
__device__ __forceinline__ void merge_rows(const float* lse, const float* o_row0, int n, int lane, float& M,
                                           float& wsum, float (&acc)[D / 64]) {
  // Every rounding step is spelled out (explicit FMAs, no contraction), so
  // the in-kernel merge and the reduce kernel give the same bits.
#pragma clang fp contract(off)
  constexpr int PER = D / 64;
  constexpr int BATCH = 8;
  // COH: the partials were written by other workgroups in this launch, so
  // they are read with device-scope (sc1) loads, which do not hit stale L2
  // lines of this XCD.
  constexpr int aux = COH ? kDeviceScope : 0;
  const auto lse_r = make_tile_rsrc(lse, n * 4);
  const auto o_r = make_tile_rsrc(o_row0, n * D * 4);
  for (int c = 0; c < n; c += BATCH) {
    float l[BATCH], v[BATCH][PER];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      l[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lse_r, (c + u) * 4, 0, aux));
#pragma unroll
      for (int k = 0; k < PER; ++k)
        v[u][k] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(o_r, ((c + u) * D + lane * PER + k) * 4, 0, aux));
    }
    float mc = M;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      l[u] = (c + u < n) ? l[u] * kLog2e : -INFINITY;
      mc = fmaxf(mc, l[u]);
    }
    const float alpha = fast_exp2(M - mc);   // M = -inf on the first batch: alpha = 0
    M = mc;
    wsum *= alpha;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= alpha;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float w = fast_exp2(l[u] - M);
      wsum += w;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = __builtin_fmaf(w, v[u][k], acc[k]);
    }
  }
}

template <int D, bool COH>
__device__ __forceinline__ void merge_partitions(const float* lse, const float* o_row0, int n, int lane,
                                                 float (&acc)[D / 64]) {
  constexpr int PER = D / 64;
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float M = -INFINITY;
  float wsum = 0.f;
  merge_rows<D, COH>(lse, o_row0, n, lane, M, wsum, acc);
  const float inv = 1.f / wsum;
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] *= inv;
}

// As merge_partitions over the rows of two arrays, n1 rows at (lse1, o1)
// and n2 at (lse2, o2); each batch loads eight rows of both arrays in one
// round trip.
template <int D>
__device__ __forceinline__ void merge_partitions2(const float* lse1, const float* o1, int n1, const float* lse2,
                                                  const float* o2, int n2, int lane, float (&acc)[D / 64]) {
#pragma clang fp contract(off)
  constexpr int PER = D / 64;
  constexpr int BATCH = 8;
  const auto lse1_r = make_tile_rsrc(lse1, n1 * 4);
  const auto o1_r = make_tile_rsrc(o1, n1 * D * 4);
  const auto lse2_r = make_tile_rsrc(lse2, n2 * 4);
  const auto o2_r = make_tile_rsrc(o2, n2 * D * 4);
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float M = -INFINITY;
  float wsum = 0.f;
  const int n = max(n1, n2);
  for (int c = 0; c < n; c += BATCH) {
    float l[2 * BATCH], v[2 * BATCH][PER];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      l[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lse1_r, (c + u) * 4, 0, 0));
      l[BATCH + u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lse2_r, (c + u) * 4, 0, 0));
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const uint32_t off = ((c + u) * D + lane * PER + k) * 4;
        v[u][k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(o1_r, off, 0, 0));
        v[BATCH + u][k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(o2_r, off, 0, 0));
      }
    }
    float mc = M;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      l[u] = (c + u < n1) ? l[u] * kLog2e : -INFINITY;
      l[BATCH + u] = (c + u < n2) ? l[BATCH + u] * kLog2e : -INFINITY;
      mc = fmaxf(mc, fmaxf(l[u], l[BATCH + u]));
    }
    const float alpha = fast_exp2(M - mc);
    M = mc;
    wsum *= alpha;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= alpha;
#pragma unroll
    for (int u = 0; u < 2 * BATCH; ++u) {
      const float w = fast_exp2(l[u] - M);
      wsum += w;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = __builtin_fmaf(w, v[u][k], acc[k]);
    }
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] *= inv;
}

template <int D>
__device__ __forceinline__ void store_row_part(void* out, size_t row, int lane, int out_dtype,
                                               const float (&acc)[D / 64]) {
  constexpr int PER = D / 64;
  const size_t idx = row * D + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (out_dtype == KV_F32) static_cast<float*>(out)[idx + k] = acc[k];
    else if (out_dtype == KV_F16) static_cast<_Float16*>(out)[idx + k] = static_cast<_Float16>(acc[k]);
    else static_cast<__bf16*>(out)[idx + k] = static_cast<__bf16>(acc[k]);
  }
}

// ----------------------------------------------------------------- kernel
// MODE_FINAL: one partition covers the whole context; write out.
// MODE_PARTIAL: write each partition's (o, lse) to the workspace.
// MODE_SPLIT: as PARTIAL, but a sequence with a single partition writes out
// directly, and for the others the last partition to finish (counted with a
// device-scope atomic per (sequence, kv head)) merges them into out and
// resets the counter to zero.
enum { MODE_FINAL = 0, MODE_PARTIAL = 1, MODE_SPLIT = 2 };

// Largest amount (log2 units) a logit may exceed the running reference max
// before the accumulators are rescaled; keeps every p = exp2(x - m) <= 2^8.
constexpr float kSlack = 8.0f;

// Sliding window: the first attended position of a context of L tokens
// (max(0, L - W) for a window W > 0, else 0) and the block holding it, where
// the sequence's partitions (or its run of tiles) begin.
__device__ __forceinline__ int window_lo(int L, int window) { return window > 0 ? max(0, L - window) : 0; }
__device__ __forceinline__ int window_block(int L, int window) { return window_lo(L, window) / kBlockSize; }

// Workgroup-shared state of one work item: the NW waves' softmax states for
// the cross-wave merge, and the merge ticket of the split mode.
// The cross-wave merge stages the waves' accumulators through LDS in two
// passes of half the d-tiles: 16 KiB instead of 32 KiB at D = 128, so three
// decode workgroups fit on a CU (their registers allow three) instead of two.
constexpr int kMergePasses = 2;
template <int NW, int NT>
struct ItemShared {
  float m[NW][16];
  float l[NW][16];
  f32x4 o[NW][NT / kMergePasses][64];
  int ticket;
};

// The loads of one work item that do not depend on its math: this wave's
// first 64 physical block ids (lane j: logical block blk0 + wid + NW*j,
// bounded by the table row) and the query operand of the lane's head column
// (zero for columns >= G).  Issued ahead of the item, so their latency hides
// behind the previous item's streaming.
template <int KVT, int D>
struct ItemPrefetch {
  int ids;
  u32x4 qop[TileOps<KVT, D>::NQ];
};

// Ids of blocks first + stride*j (lane j) of sequence b's table row, and
// the q operand of kv head h's query group.
template <int KVT, int D>
__device__ __forceinline__ void meta_prefetch(const DecodeParams& p, int b, int h, int first, int stride,
                                              ItemPrefetch<KVT, D>& pf) {
  // Buffer loads bounded by the table row / the group's q rows: lanes past
  // the end read 0 without a branch, so no load here is conditional (a
  // conditional load would make the compiler drain every outstanding load
  // at the next wait).
  constexpr int QB = (KVT == KV_F32) ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const auto tr = make_tile_rsrc(p.block_tables + static_cast<size_t>(b) * p.mbps, p.mbps * 4);
  const int id0 = first + stride * lane;
  pf.ids = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(tr, static_cast<uint32_t>(id0) * 4u, 0, 0));
  const auto qr = make_tile_rsrc(static_cast<const char*>(p.q) +
                                     (static_cast<size_t>(b) * p.num_q_heads + h * p.group) * D * QB,
                                 p.group * D * QB);
  TileOps<KVT, D>::load_q(pf.qop, qr, static_cast<uint32_t>(r * D * QB), lane >> 4);
}

template <int KVT, int D, int NW>
__device__ __forceinline__ void item_prefetch(const DecodeParams& p, int b, int h, int part, int L,
                                              ItemPrefetch<KVT, D>& pf) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  meta_prefetch<KVT, D>(p, b, h, window_block(L, p.window) + part * p.partition_blocks + wid, NW, pf);
}

// One wave's running softmax state for the G heads of a KV head: lane
// (g, r) holds head column r's reference max, its share of the sum over
// the tokens 4g..4g+3 of every block, and O^T d-tiles (rows 4g..4g+3).
template <int NT>
struct WaveState {
  float m;
  float l;
  f32x4 o[NT];
  __device__ void reset(float m0 = -INFINITY) {
    m = m0;
    l = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Streams the blocks first + stride*i (i < count) of sequence b (context
// length L, kv head h, positions before lo masked off; with CAUSAL, each
// lane's head column also masks positions after its own limit lim) through
// one wave's softmax state.  `ids` holds the
// physical ids of the first 64 of them (lane j: block first + stride*j).
//
// NPK > 1 (the multi-token step): NPK packs of query columns share every
// tile, each with its own q operand, softmax state and causal limits, so a
// tile fetched once serves NPK x 16 columns.
//
// PAIRS (f16 / bf16 only): tiles go two at a time, PV on the K = 32 form
// (TileOps::pv2); the ring holds the pair, and the next pair's K loads go
// out after the QK^T products, its V loads after the PV products.
template <int KVT, int D, int PF, bool CAUSAL, int POLICY, int NPK, bool PAIRS = false>
__device__ __forceinline__ void attend_packs(const DecodeParams& p, int b, int h, int L, int lo, int first,
                                             int stride, int count, int ids,
                                             const u32x4 (&qop)[NPK][TileOps<KVT, D>::NQ],
                                             WaveState<D / 16> (&st)[NPK], const int (&lim)[NPK]) {
  typedef TileOps<KVT, D> T;
  constexpr int E = ElemBytes<KVT>::value;
  constexpr int TILE = kBlockSize * D * E;  // bytes of one (block, kv head) tile
  constexpr int NL = T::NLOAD;
  constexpr int NT = T::NT;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a block
  const int32_t* table = p.block_tables + static_cast<size_t>(b) * p.mbps;

  // Tile loads are buffer loads: each tile's descriptor (base = the tile,
  // size = TILE bytes) lives in scalar registers and every lane adds one
  // 32-bit offset, so no per-tile 64-bit vector addresses are needed.
  uint32_t lane_off[NL];
#pragma unroll
  for (int m = 0; m < NL; ++m) lane_off[m] = static_cast<uint32_t>(lane) * 16u + m * 1024u;
  const char* kcache = static_cast<const char*>(p.k_cache);
  const char* vcache = static_cast<const char*>(p.v_cache);
  // A load past the last block still issues, through a zero-size
  // descriptor (reads 0, no memory traffic), so the loop has no
  // conditional loads and each wait covers exactly the tile it needs.
  // POLICY: cache policy of the tile loads, kStreamLoad (non-temporal) for
  // tiles one step reads once, 0 (ordinary) for tiles other work reads
  // again soon (the multi-token step's, read by every pack of query rows).
  // E4M3: the block's K and V scales ride in the ring with its tile, loaded
  // just before the tile's codes, so the wait for a tile covers its scales
  // and never the tiles prefetched after it.
  const auto scale_r = make_tile_rsrc(p.kv_scales, KVT == KV_E4M3 ? 2 * p.num_blocks * p.num_kv_heads * 4 : 0);
  auto load_tile = [&](u32x4 (&kt)[NL], u32x4 (&vt)[NL], float& ksc, float& vsc, int blk, bool valid) {
    const size_t tile = (static_cast<size_t>(blk) * p.num_kv_heads + h) * TILE;
    if constexpr (KVT == KV_E4M3) {
      const uint32_t so = static_cast<uint32_t>(blk * p.num_kv_heads + h) * 4u;
      ksc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scale_r, so, 0, 0));
      vsc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          scale_r, so + static_cast<uint32_t>(p.num_blocks * p.num_kv_heads) * 4u, 0, 0));
    }
    const auto kr = make_tile_rsrc(kcache + tile, valid ? TILE : 0);
    const auto vr = make_tile_rsrc(vcache + tile, valid ? TILE : 0);
#pragma unroll
    for (int m = 0; m < NL; ++m) kt[m] = buffer_ld16_policy<POLICY>(kr, lane_off[m]);
#pragma unroll
    for (int m = 0; m < NL; ++m) vt[m] = buffer_ld16_policy<POLICY>(vr, lane_off[m]);
  };

  // E4M3 V scales: P goes to the matrix cores as p * vsc * 2^(7 - vexp),
  // where 2^vexp bounds every V scale seen so far (vexp is wave-uniform: a
  // scale belongs to one (block, kv head), the same for every lane).  With
  // p <= 2^kSlack = 2^8 the product stays below 2^15, inside f16's range,
  // for any scale; a block whose scale needs a larger vexp shrinks the
  // accumulators by the (exact) power of two first, and the end of the run
  // multiplies them by 2^(vexp - 7).
  int vexp = -126;

  // Lowest causal limit of each pack (wave-uniform: lane 0 holds the pack's
  // first token, the smallest limit); blocks that end at or before it need
  // no causal mask.
  int lim_lo[NPK];
#pragma unroll
  for (int k = 0; k < NPK; ++k) lim_lo[k] = CAUSAL ? __builtin_amdgcn_readfirstlane(lim[k]) : 0;
  int lim_min = lim_lo[0];
#pragma unroll
  for (int k = 1; k < NPK; ++k) lim_min = min(lim_min, lim_lo[k]);

  auto process = [&](const u32x4 (&kt)[NL], u32x4 (&vt)[NL], float ksc, float vsc, int i) {
    const int tok0 = (first + stride * i) * kBlockSize;
    float f = p.qk_scale_log2;
    float pscale = 1.f;
    if constexpr (KVT == KV_E4M3) {
      f *= ksc;
      const uint32_t vbits = __builtin_amdgcn_readfirstlane(__float_as_uint(vsc));
      const int e_blk = static_cast<int>((vbits >> 23) & 0xFFu) - 126;   // vsc < 2^e_blk
      if (e_blk > vexp) {
        const float shrink = __builtin_amdgcn_ldexpf(1.f, vexp - e_blk);
#pragma unroll
        for (int k = 0; k < NPK; ++k)
#pragma unroll
          for (int n = 0; n < NT; ++n) st[k].o[n] *= shrink;
        vexp = e_blk;
      }
      pscale = __builtin_amdgcn_ldexpf(__uint_as_float(vbits), 7 - vexp);
    }
    const bool tail = tok0 + kBlockSize > L;   // the sequence's last, partly filled block
    if (tail) T::mask_v(vt, L - tok0 - 4 * g);
#pragma unroll
    for (int k = 0; k < NPK; ++k) {
      const f32x4 s = T::qk(kt, qop[k]);
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = s[j] * f;
      if (tail) {
        const int nv = L - tok0 - 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (j < nv) ? x[j] : -INFINITY;
      }
      if (tok0 < lo) {              // the window's first block: positions before lo
        const int nlo = lo - tok0 - 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (j < nlo) ? -INFINITY : x[j];
      }
      if constexpr (CAUSAL) {       // this lane's column sees positions <= lim only
        if (tok0 + kBlockSize - 1 > lim_lo[k]) {
          const int nc = lim[k] - tok0 - 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = (j <= nc) ? x[j] : -INFINITY;
        }
      }
      // Lazy rescaling: the reference max only moves when some head's block
      // max exceeds it by more than kSlack (log2 units), so exp2(x - m)
      // stays below 2^kSlack and the accumulators are rescaled about once
      // per run of blocks instead of every block.  The first block always
      // moves it.
      WaveState<NT>& sk = st[k];
      const float bm = max_over_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      if (__any(bm > sk.m + kSlack)) {
        const float m_new = fmaxf(sk.m, bm);
        const float alpha = fast_exp2(sk.m - m_new);
        sk.m = m_new;
        sk.l *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) sk.o[n] *= alpha;
      }
      float pr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - sk.m);
      sk.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      T::pv(sk.o, vt, pr, pscale);
    }
  };

  // Blocks go in chunks of up to 64: the chunk's physical ids arrive in one
  // vector load (lane j: the chunk's j-th block) and are read out with
  // readlane.  Tiles stream through a ring of PF register buffers: before
  // block j is processed, the loads of block j + PF - 1 are issued, so PF - 1
  // tiles are in flight while the matrix cores work on one.
  if constexpr (PAIRS) {
    const auto tile_r = [&](const char* cache, int blk, bool valid) {
      return make_tile_rsrc(cache + (static_cast<size_t>(blk) * p.num_kv_heads + h) * TILE, valid ? TILE : 0);
    };
    auto load_half = [&](u32x4 (&t)[NL], const char* cache, int blk, bool valid) {
      const auto r = tile_r(cache, blk, valid);
#pragma unroll
      for (int m = 0; m < NL; ++m) t[m] = buffer_ld16_policy<POLICY>(r, lane_off[m]);
    };
    // Scale and mask one tile's four logits of pack k (tile starting at
    // position tok0).
    auto logits = [&](const f32x4& sv, float* x, int tok0, int k) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = sv[j] * p.qk_scale_log2;
      if (tok0 + kBlockSize > L) {
        const int nv = L - tok0 - 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (j < nv) ? x[j] : -INFINITY;
      }
      if (tok0 < lo) {
        const int nlo = lo - tok0 - 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (j < nlo) ? -INFINITY : x[j];
      }
      if constexpr (CAUSAL) {
        if (tok0 + kBlockSize - 1 > lim_lo[k]) {
          const int nc = lim[k] - tok0 - 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = (j <= nc) ? x[j] : -INFINITY;
        }
      }
    };
    u32x4 kb[2][NL], vb[2][NL];
    for (int base = 0; base < count; base += 64) {
      const int cnt = min(64, count - base);
      if (base > 0) ids = (lane < cnt) ? table[first + stride * (base + lane)] : 0;
      {
        const int i0 = __builtin_amdgcn_readlane(ids, 0);
        const int i1 = __builtin_amdgcn_readlane(ids, min(1, cnt - 1));
        // K before V, as the loop issues them (the next pair's K after
        // the scores, its V after PV): the memory counter drains in
        // issue order, so with the same order on entry the wait before
        // the scores covers only the K loads.  Left to the scheduler, the
        // first pair's V went first, and the wait merged at the loop head
        // drained everything, the V just issued included, every pair.
        load_half(kb[0], kcache, i0, true);
        load_half(kb[1], kcache, i1, 1 < cnt);
        __builtin_amdgcn_sched_barrier(0);
        load_half(vb[0], vcache, i0, true);
        load_half(vb[1], vcache, i1, 1 < cnt);
      }
      // One pair.  MASKED: the general form; otherwise the pair is known
      // to need no mask (both tiles whole, inside the window and at or
      // below every column's causal limit), and the body carries none of
      // the per-lane compares, which the compiler would issue ahead of the
      // (rarely taken) masking branches.
      auto pair = [&](int i, auto masked) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        const bool two = i + 1 < cnt;   // else tile b is a zero-size load: V = 0, its logits masked
        const int tok0 = (first + stride * (base + i)) * kBlockSize;
        const int tok1 = tok0 + stride * kBlockSize;
        f32x4 sa[NPK], sb[NPK];
#pragma unroll
        for (int k = 0; k < NPK; ++k) {
          sa[k] = T::qk(kb[0], qop[k]);
          sb[k] = T::qk(kb[1], qop[k]);
        }
        const int n2 = __builtin_amdgcn_readlane(ids, min(i + 2, cnt - 1));
        const int n3 = __builtin_amdgcn_readlane(ids, min(i + 3, cnt - 1));
        load_half(kb[0], kcache, n2, i + 2 < cnt);
        load_half(kb[1], kcache, n3, i + 3 < cnt);
        if constexpr (MASKED) {
          if (tok0 + kBlockSize > L) T::mask_v(vb[0], L - tok0 - 4 * g);
          if (two && tok1 + kBlockSize > L) T::mask_v(vb[1], L - tok1 - 4 * g);
        }
#pragma unroll
        for (int k = 0; k < NPK; ++k) {
          float x[8];
          if constexpr (MASKED) {
            logits(sa[k], x, tok0, k);
            logits(sb[k], x + 4, tok1, k);
            if (!two) {
#pragma unroll
              for (int j = 4; j < 8; ++j) x[j] = -INFINITY;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[j] = sa[k][j] * p.qk_scale_log2;
              x[4 + j] = sb[k][j] * p.qk_scale_log2;
            }
          }
          WaveState<NT>& sk = st[k];
          const float bm = max_over_groups(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))));
          if (__any(bm > sk.m + kSlack)) {   // lazy rescaling, as in the one-tile step
            const float m_new = fmaxf(sk.m, bm);
            const float alpha = fast_exp2(sk.m - m_new);
            sk.m = m_new;
            sk.l *= alpha;
#pragma unroll
            for (int n = 0; n < NT; ++n) sk.o[n] *= alpha;
          }
          float pr[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pr[j] = fast_exp2(x[j] - sk.m);
          sk.l += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
          T::pv2(sk.o, vb[0], vb[1], pr);
        }
        load_half(vb[0], vcache, n2, i + 2 < cnt);
        load_half(vb[1], vcache, n3, i + 3 < cnt);
      };
      // The pairs that need no mask form one run (positions only grow with
      // i): masked pairs before it (the window's first block), the run,
      // masked pairs after it (the causal diagonal, the context's tail).
      auto clean = [&](int i) __attribute__((always_inline)) {
        const int tok0 = (first + stride * (base + i)) * kBlockSize;
        const int tok1 = tok0 + stride * kBlockSize;
        return i + 1 < cnt && tok1 + kBlockSize <= L && tok0 >= lo &&
               (!CAUSAL || tok1 + kBlockSize - 1 <= lim_min);
      };
      int i = 0;
      for (; i < cnt && !clean(i); i += 2) pair(i, std::true_type{});
      for (; i < cnt && clean(i); i += 2) pair(i, std::false_type{});
      for (; i < cnt; i += 2) pair(i, std::true_type{});
    }
    return;
  }
  u32x4 kb[PF][NL], vb[PF][NL];
  float ks[PF], vs[PF];
  for (int base = 0; base < count; base += 64) {
    const int cnt = min(64, count - base);
    if (base > 0) ids = (lane < cnt) ? table[first + stride * (base + lane)] : 0;
#pragma unroll
    for (int s = 0; s < PF - 1; ++s)
      load_tile(kb[s], vb[s], ks[s], vs[s], __builtin_amdgcn_readlane(ids, min(s, cnt - 1)), s < cnt);
    for (int i = 0; i < cnt; i += PF) {
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        const int j = i + s;
        const int nxt = j + PF - 1;
        const int slot = (s + PF - 1) % PF;
        load_tile(kb[slot], vb[slot], ks[slot], vs[slot], __builtin_amdgcn_readlane(ids, min(nxt, cnt - 1)),
                  nxt < cnt);
        if (j < cnt) process(kb[s], vb[s], ks[s], vs[s], base + j);
      }
    }
  }
  if constexpr (KVT == KV_E4M3) {
    const float grow = __builtin_amdgcn_ldexpf(1.f, vexp - 7);
#pragma unroll
    for (int k = 0; k < NPK; ++k)
#pragma unroll
      for (int n = 0; n < NT; ++n) st[k].o[n] *= grow;
  }
}

// One pack of query columns (decode: the GQA group of one token).
template <int KVT, int D, int PF, bool CAUSAL = false, int POLICY = CAUSAL ? 0 : kStreamLoad>
__device__ __forceinline__ void attend_blocks(const DecodeParams& p, int b, int h, int L, int lo, int first,
                                              int stride, int count, int ids,
                                              const u32x4 (&qop)[TileOps<KVT, D>::NQ],
                                              WaveState<D / 16>& st, int lim = 0) {
  WaveState<D / 16> sa[1] = {st};
  const int la[1] = {lim};
  attend_packs<KVT, D, PF, CAUSAL, POLICY, 1>(
      p, b, h, L, lo, first, stride, count, ids,
      *reinterpret_cast<const u32x4(*)[1][TileOps<KVT, D>::NQ]>(&qop), sa, la);
  st = sa[0];
}

// Merges the NW waves' softmax states of one item through LDS: M and Lsum
// get the combined max and sum of this lane's head column, and emit(n, acc)
// receives the normalised output d-tiles n = wid, wid + NW, ...
template <int NW, int NT, typename Emit>
__device__ __forceinline__ void merge_waves(float m_run, float l_run, const f32x4 (&o)[NT],
                                            ItemShared<NW, NT>& sm, int wid, int lane, float& M,
                                            float& Lsum, Emit emit) {
  const int g = lane >> 4;
  const int r = lane & 15;
  if constexpr (NW > 1) {
    constexpr int NTH = NT / kMergePasses;   // d-tiles staged per pass
    if (g == 0) {
      sm.m[wid][r] = m_run;
      sm.l[wid][r] = l_run;
    }
    float fw[NW];
    float inv = 0.f;
#pragma unroll
    for (int pass = 0; pass < kMergePasses; ++pass) {
      if (pass > 0) __syncthreads();   // the previous pass's reads are done
#pragma unroll
      for (int n = 0; n < NTH; ++n) sm.o[wid][n][lane] = o[pass * NTH + n];
      __syncthreads();
      if (pass == 0) {
        M = sm.m[0][r];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][r]);
        Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          fw[w] = fast_exp2(sm.m[w][r] - M);
          Lsum += fw[w] * sm.l[w][r];
        }
        inv = 1.f / Lsum;
      }
      for (int n = wid; n < NTH; n += NW) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += fw[w] * sm.o[w][n][lane];
        emit(pass * NTH + n, acc * inv);
      }
    }
  } else {
    M = m_run;
    Lsum = l_run;
    const float inv = 1.f / Lsum;
#pragma unroll
    for (int n = 0; n < NT; ++n) emit(n, o[n] * inv);
  }
}

// The fused step's new token of sequence b into slot `off` of its block
// `last` (the physical block its table names, skipped when out of range):
// kv head h's K and V rows of k_new / v_new, laid out as the tiles are (one
// wave; lane c moves 16-byte chunk c of the rows).
template <int KVT, int D>
__device__ __forceinline__ void write_new_token(const DecodeParams& p, int b, int h, int last, int off) {
  if constexpr (KVT != KV_E4M3) {   // E4M3 pools take their tokens through kv_cache_append_e4m3
    constexpr int E = ElemBytes<KVT>::value;
    typedef typename std::conditional<E == 4, uint32_t, uint16_t>::type Elem;
    constexpr int X = 16 / E;   // elements per chunk
    constexpr int CH = D / X;   // chunks per row
    const int lane = threadIdx.x & 63;
    if (lane < CH) {
      // The block id and the new K and V rows load together (none depends
      // on another): one round trip before the stores, not two.
      const int blk = p.block_tables[static_cast<size_t>(b) * p.mbps + last];
      const size_t row = (static_cast<size_t>(b) * p.num_kv_heads + h) * D * E + lane * 16;
      const u32x4 kv = ld16(static_cast<const char*>(p.k_new) + row);
      const u32x4 vv = ld16(static_cast<const char*>(p.v_new) + row);
      if (blk < 0 || blk >= p.num_blocks) return;
      const size_t tile = (static_cast<size_t>(blk) * p.num_kv_heads + h) * kBlockSize * D * E;
      char* kc = static_cast<char*>(const_cast<void*>(p.k_cache));
      char* vc = static_cast<char*>(const_cast<void*>(p.v_cache));
      st16(kc + tile + (static_cast<size_t>(lane) * kBlockSize + off) * 16, kv);
      Elem vals[X];
      __builtin_memcpy(vals, &vv, 16);
      Elem* vt = reinterpret_cast<Elem*>(vc + tile);
#pragma unroll
      for (int i = 0; i < X; ++i) vt[v_tile_elem(off, lane * X + i, 4 / E)] = vals[i];
    }
  }
}

// One work item: sequence b (context length L), kv head h, partition `part`.
template <int KVT, int D, int NW, int MODE, int PF>
__device__ __forceinline__ void decode_item(const DecodeParams& p, int b, int h, int part, int L,
                                            const ItemPrefetch<KVT, D>& pf,
                                            ItemShared<NW, D / 16>& sm) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = p.group;
  const int Hq = p.num_q_heads;
  const int lo = window_lo(L, p.window);
  const int base_blk = lo / kBlockSize;     // partition 0 starts at the window's first block
  const int blk0 = base_blk + part * p.partition_blocks;
  const int first = blk0 + wid;
  const int qhead = h * G + r;
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblk - base_blk + p.partition_blocks - 1) / p.partition_blocks;

  if (MODE != MODE_PARTIAL && L == 0) {  // empty context: zero output
    if (part == 0 && r < G) {
      const size_t row = (static_cast<size_t>(b) * Hq + h * G + r) * D;
      for (int n = wid; n < NT; n += NW) store4(p.out, row + 16 * n + 4 * g, p.out_dtype, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    return;
  }
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + p.partition_blocks);
  const bool direct = (MODE == MODE_FINAL) || (MODE == MODE_SPLIT && nparts == 1);

  // Fused decode step: the item that holds position L - 1 writes the new
  // token there first; the barrier makes the stores visible to every wave
  // of the workgroup before any of them loads the block.  Only the split
  // mode carries new tokens (paged_decode_step); compiled out of the
  // others, the single-pass kernel fits three workgroups per CU.
  if (MODE == MODE_SPLIT && p.k_new != nullptr) {
    const int last = (L - 1) / kBlockSize;
    if (last >= blk0 && last < blk1) {   // workgroup-uniform
      if (wid == 0) write_new_token<KVT, D>(p, b, h, last, (L - 1) % kBlockSize);
      __syncthreads();
    }
  }

  // Blocks of this wave: first + NW * i, i < nmine.
  const int nmine = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;
  WaveState<NT> st;
  st.reset();
  // Tile loads stream (non-temporal) except in a split sequence's first
  // partition: prompts shared between sequences (parallel samples, beams, a
  // common system prompt) sit at the start, and the sequences sharing them
  // read those tiles close in time, so there they stay cacheable.
  if (MODE != MODE_FINAL && part == 0)
    attend_blocks<KVT, D, PF, false, 0>(p, b, h, L, lo, first, NW, nmine, pf.ids, pf.qop, st);
  else
    attend_blocks<KVT, D, PF, false, kStreamLoad>(p, b, h, L, lo, first, NW, nmine, pf.ids, pf.qop, st);
  float m_run = st.m;
  float l_run = st.l;
  f32x4 (&o)[NT] = st.o;
  l_run = sum_over_groups(l_run);

  // ---- merge the NW waves' (max, sum, accumulator) and write
  const size_t out_row = (static_cast<size_t>(b) * Hq + qhead) * D;
  const size_t part_row = (static_cast<size_t>(b) * Hq + qhead) * p.num_partitions + part;
  // Split mode: partials go out with device-scope (sc1) stores, complete at
  // the device coherence point once the wave's store counter drains.
  const auto part_r = make_tile_rsrc(p.tmp_out + part_row * D, D * 4);
  auto emit = [&](int n, f32x4 acc) {
    if (r < G) {
      if (direct) store4(p.out, out_row + 16 * n + 4 * g, p.out_dtype, acc);
      else if (MODE == MODE_SPLIT)
        __builtin_amdgcn_raw_buffer_store_b128(bitcast<u32x4>(acc), part_r, (16 * n + 4 * g) * 4, 0, kDeviceScope);
      else *reinterpret_cast<f32x4*>(p.tmp_out + part_row * D + 16 * n + 4 * g) = acc;
    }
  };
  float M, Lsum;
  merge_waves<NW, NT>(m_run, l_run, o, sm, wid, lane, M, Lsum, emit);
  if (direct) return;
  const float lse = (M + fast_log2(Lsum)) * kLn2;
  if constexpr (MODE == MODE_SPLIT) {
    if (wid == 0 && g == 0 && r < G)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), make_tile_rsrc(p.tmp_lse + part_row, 4), 0, 0,
                                            kDeviceScope);
    // Count this partition once all its waves' partial stores are complete
    // at device scope; the workgroup that takes the last ticket merges.
    // The ordering rests on the ISA's scope bits, not on a language-level
    // release: the partials are stored and loaded with device scope (written
    // through to, and read from, the device coherence point, past the XCD
    // L2's own copies), every wave waits for its stores to complete before
    // the barrier, and only then is the ticket (a device atomic) taken.  An
    // acquire-release ticket would add an L2 write-back and invalidate per
    // partition; measured, the B = 32 step went 23 -> 28 us and the fused
    // headline layer 66 -> 124 us.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    int* counter = p.counters + static_cast<size_t>(b) * p.num_kv_heads + h;
    if (threadIdx.x == 0) sm.ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sm.ticket != nparts - 1) return;
    for (int gg = wid; gg < G; gg += NW) {
      const size_t row = static_cast<size_t>(b) * Hq + h * G + gg;
      float acc[D / 64];
      merge_partitions<D, true>(p.tmp_lse + row * p.num_partitions,
                                p.tmp_out + row * p.num_partitions * D, nparts, lane, acc);
      store_row_part<D>(p.out, row, lane, p.out_dtype, acc);
    }
    if (threadIdx.x == 0) *counter = 0;   // ready for the next call
  } else {
    if (wid == 0 && g == 0 && r < G) p.tmp_lse[part_row] = lse;
  }
}

// One workgroup per work item (sequence, kv head, partition), partition
// fastest: the partitions of one sequence are dispatched together, and
// sequences in order, so sequences sharing prefix blocks read them close in
// time.  Items past a sequence's context exit at once.
template <int KVT, int D, int NW, int MODE, int PF>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(const DecodeParams p) {
  __shared__ ItemShared<NW, D / 16> sm;
  const int item = static_cast<int>(blockIdx.x);
  const int part = item % p.num_partitions;
  const int h = (item / p.num_partitions) % p.num_kv_heads;
  const int b = item / (p.num_partitions * p.num_kv_heads);
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  ItemPrefetch<KVT, D> pf;
  item_prefetch<KVT, D, NW>(p, b, h, part, L, pf);
  decode_item<KVT, D, NW, MODE, PF>(p, b, h, part, L, pf, sm);
}

// Persistent form: as many workgroups as fit on the GPU at once.  Each one
// first counts the non-empty work items of every sequence (an exclusive
// prefix sum in LDS), then walks its share of the items, mapping each back
// to (sequence, kv head, partition).  No workgroup is launched for an empty
// partition.
constexpr int kXcds = 8;       // accelerator complex dies of an MI355X
// Neighbouring sequences whose first partitions run together.  The split
// mode keeps one: there the last partition of a (sequence, kv head) merges
// them all, so a sequence's partitions are best finished close together
// (measured ~4% faster on a 32-sequence layer without shared prefixes).
template <int MODE>
constexpr int seq_block() { return MODE == MODE_SPLIT ? 1 : 8; }

template <int KVT, int D, int NW, int MODE, int PF>
__global__ __launch_bounds__(NW * 64) void paged_decode_persistent(const DecodeParams p) {
  __shared__ ItemShared<NW, D / 16> sm;
  __shared__ int s_cum[kMaxSeqsPersistent + 1];   // items before sequence b
  __shared__ int s_np[kMaxSeqsPersistent];        // partitions of sequence b
  __shared__ int s_len[kMaxSeqsPersistent];       // context length of sequence b
  __shared__ int s_wsum[NW];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;

  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += NW * 64) {
    const int i = c0 + static_cast<int>(threadIdx.x);
    int items = 0;
    if (i < B) {
      const int L = max(0, min(p.context_lens[i], p.mbps * kBlockSize));
      const int nb = (L + kBlockSize - 1) / kBlockSize - window_block(L, p.window);
      int np = (nb + p.partition_blocks - 1) / p.partition_blocks;
      if (MODE != MODE_PARTIAL) np = max(np, 1);   // an empty context still writes zeros
      s_np[i] = np;
      s_len[i] = L;
      items = np * Hkv;
    }
    // inclusive scan within the wave, then across the NW waves
    int x = items;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wid] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wid; ++w) before += s_wsum[w];
    int total = 0;
    for (int w = 0; w < NW; ++w) total += s_wsum[w];
    if (i < B) s_cum[i + 1] = before + x;
    if (i == 0) s_cum[0] = 0;
    carry += total;
    __syncthreads();
  }
  // Items are split into 8 contiguous ranges, one per XCD (workgroup w runs
  // on XCD w % 8), and each XCD's workgroups stride through their range.
  // Neighbouring sequences, which are the ones likely to share prefix
  // blocks, are then read through one L2, and each XCD gets 1/8 of the
  // items.  The grid is a multiple of 8.
  const int N = carry;
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = gridDim.x / kXcds;
  const int lo = static_cast<int>(static_cast<int64_t>(N) * xcd / kXcds);
  const int hi = static_cast<int>(static_cast<int64_t>(N) * (xcd + 1) / kXcds);
  // Item n -> (sequence, kv head, partition).  Sequences go in blocks of
  // kSeqBlock neighbours; inside a block the first partitions of all its
  // sequences (every kv head) come first, then each sequence's remaining
  // partitions.  Neighbouring sequences that share a prompt (parallel
  // samples, beams) then read their shared leading blocks at the same time,
  // through one XCD's L2, instead of one sequence at a time after the L2 has
  // moved on.
  constexpr int kSeqBlock = seq_block<MODE>();
  auto locate = [&](int n, int& b, int& h, int& part) {
    int lo_m = 0, hi_m = (B + kSeqBlock - 1) / kSeqBlock;
    while (hi_m - lo_m > 1) {
      const int mid = (lo_m + hi_m) >> 1;
      if (s_cum[mid * kSeqBlock] <= n) lo_m = mid;
      else hi_m = mid;
    }
    const int b0 = lo_m * kSeqBlock;
    const int b1 = min(B, b0 + kSeqBlock);
    int local = n - s_cum[b0];
    int firsts = 0;   // items of the block's first partitions
    for (int bb = b0; bb < b1; ++bb) firsts += (s_np[bb] > 0) ? Hkv : 0;
    b = b1 - 1;
    h = 0;
    part = 0;
    if (local < firsts) {
      int k = local / Hkv;
      for (int bb = b0; bb < b1; ++bb) {
        if (s_np[bb] > 0 && k-- == 0) {
          b = bb;
          break;
        }
      }
      h = local % Hkv;
      return;
    }
    local -= firsts;
    for (int bb = b0; bb < b1; ++bb) {
      const int rest = (s_np[bb] > 0) ? (s_np[bb] - 1) * Hkv : 0;
      if (local < rest) {
        b = bb;
        h = local / (s_np[bb] - 1);
        part = 1 + local % (s_np[bb] - 1);
        return;
      }
      local -= rest;
    }
  };
  ItemPrefetch<KVT, D> cur, nxt;
  int b, h, part, b2, h2, part2;

  int n = lo + static_cast<int>(blockIdx.x) / kXcds;
  if (n >= hi) return;
  locate(n, b, h, part);
  item_prefetch<KVT, D, NW>(p, b, h, part, s_len[b], cur);
  while (true) {
    // The next item's ids and q load while this item streams (the last item
    // prefetches itself again, so the load is never conditional).
    const int n2 = n + per_xcd;
    locate(min(n2, hi - 1), b2, h2, part2);
    item_prefetch<KVT, D, NW>(p, b2, h2, part2, s_len[b2], nxt);
    decode_item<KVT, D, NW, MODE, PF>(p, b, h, part, s_len[b], cur, sm);
    __syncthreads();   // the next item reuses the merge state
    if (n2 >= hi) break;
    n = n2;
    b = b2;
    h = h2;
    part = part2;
    cur = nxt;
  }
}

// ------------------------------------------------------ multi-token step
// Several new tokens per sequence (chunked prefill, speculative
// verification): sequence b's query rows query_start[b] .. query_start[b+1]-1
// are its n_b newest tokens, at positions L - n_b .. L - 1, and the row of
// token j attends causally to positions 0 .. L - n_b + j ("rvLLM:
// High-performance LLM inference in Rust", section "CUDA Kernels", row
// "FlashAttention-2": prefill and decode with causal masking).  A pack of
// TP = 16 / G tokens x G heads fills the 16 matrix-core columns, and each
// column masks the positions after its own token.  A wave carries
// kPacksPerWave packs at once, so each K/V tile it fetches serves
// kPacksPerWave x TP tokens of the whole group.  Work items are (sequence,
// kv head, group of packs, partition); a group's partitions cover the
// blocks up to its last token.
constexpr int kPacksPerWave = 2;
struct QueryRows {
  int q0;   // first query row of the sequence
  int n;    // its number of query rows (<= its context length)
};

// A work item's loads that do not depend on its math, for NPK packs: the
// wave's first 64 block ids and each pack's q operand, issued at the
// item's start.
template <int KVT, int D, int NPK>
struct PackPrefetch {
  int ids;
  u32x4 qop[NPK][TileOps<KVT, D>::NQ];
};

template <int KVT, int D, int NW, int NPK>
__device__ __forceinline__ void prefill_prefetch(const DecodeParams& p, int b, int h, int grp, int part,
                                                 QueryRows qrow, PackPrefetch<KVT, D, NPK>& pf) {
  constexpr int QB = (KVT == KV_F32) ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int G = p.group;
  const auto tr = make_tile_rsrc(p.block_tables + static_cast<size_t>(b) * p.mbps, p.mbps * 4);
  const int id0 = part * p.partition_blocks + wid + NW * lane;
  pf.ids = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(tr, static_cast<uint32_t>(id0) * 4u, 0, 0));
  const uint32_t row_bytes = static_cast<uint32_t>(p.num_q_heads * D * QB);
  const auto qr = make_tile_rsrc(static_cast<const char*>(p.q) + static_cast<size_t>(qrow.q0) * row_bytes,
                                 qrow.n * row_bytes);
#pragma unroll
  for (int k = 0; k < NPK; ++k) {
    // Column r of pack k: token j0 + r / G, head h * G + r % G; unused
    // columns (and packs past the sequence's rows) read past the
    // descriptor's end, i.e. zeros.
    const int j0 = (grp * NPK + k) * p.tokens_per_pack;
    const int ncols = max(0, min(p.tokens_per_pack, qrow.n - j0)) * G;
    const uint32_t qoff = r < ncols ? static_cast<uint32_t>(((j0 + r / G) * p.num_q_heads + h * G + r % G) * D * QB)
                                    : static_cast<uint32_t>(qrow.n) * row_bytes;
    TileOps<KVT, D>::load_q(pf.qop[k], qr, qoff, lane >> 4);
  }
}

// One work item: sequence b, kv head h, packs grp*NPK .. grp*NPK + NPK - 1
// (TP = tokens_per_pack tokens each), partition `part` of the blocks up to
// the group's last token.
template <int KVT, int D, int NW, int MODE, int PF, int NPK, bool PAIRS>
__device__ __forceinline__ void prefill_item(const DecodeParams& p, int b, int h, int grp, int part, int L,
                                             QueryRows qrow, const PackPrefetch<KVT, D, NPK>& pf,
                                             ItemShared<NW, D / 16>& sm) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = p.group;
  const int TP = p.tokens_per_pack;
  const int base = L - qrow.n;                      // position of the sequence's first query row
  int pos[NPK];                                     // last position each column sees (-1: none)
  int jj[NPK];
  bool valid[NPK];
#pragma unroll
  for (int k = 0; k < NPK; ++k) {
    const int j0 = (grp * NPK + k) * TP;
    const int ntok = max(0, min(TP, qrow.n - j0));
    valid[k] = r < ntok * G;
    jj[k] = valid[k] ? r / G : 0;
    pos[k] = valid[k] ? base + j0 + jj[k] : -1;
  }
  const int l_item = base + min(qrow.n, (grp + 1) * NPK * TP);   // positions the group reads
  const int nblk = (l_item + kBlockSize - 1) / kBlockSize;
  const int blk0 = part * p.partition_blocks;
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + p.partition_blocks);
  const int first = blk0 + wid;
  const int nmine = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;
  WaveState<NT> st[NPK];
#pragma unroll
  for (int k = 0; k < NPK; ++k) st[k].reset(-1e30f);   // finite: a column may see no position in a wave's blocks
  attend_packs<KVT, D, PF, true, 0, NPK, PAIRS>(p, b, h, l_item, 0, first, NW, nmine, pf.ids, pf.qop, st, pos);

#pragma unroll
  for (int k = 0; k < NPK; ++k) {
    const float l_run = sum_over_groups(st[k].l);
    const int j0 = (grp * NPK + k) * TP;
    const size_t row = static_cast<size_t>(qrow.q0 + j0 + jj[k]) * p.num_q_heads + h * G + r % G;
    const bool col_ok = valid[k] && blk0 * kBlockSize <= pos[k];   // the partition holds a position of it
    auto emit = [&](int n, f32x4 acc) {
      if (!col_ok) return;
      if (MODE == MODE_FINAL) store4(p.out, row * D + 16 * n + 4 * g, p.out_dtype, acc);
      else *reinterpret_cast<f32x4*>(p.tmp_out + (row * p.num_partitions + part) * D + 16 * n + 4 * g) = acc;
    };
    if (k > 0) __syncthreads();   // the previous pack's merge has read the shared state
    float M, Lsum;
    merge_waves<NW, NT>(st[k].m, l_run, st[k].o, sm, wid, lane, M, Lsum, emit);
    if (MODE == MODE_PARTIAL && wid == 0 && g == 0 && col_ok)
      p.tmp_lse[row * p.num_partitions + part] = (M + fast_log2(Lsum)) * kLn2;
  }
}

// Persistent form of the multi-token step, laid out like
// paged_decode_persistent: LDS prefix sums of each sequence's items, XCD
// ranges.  16-bit caches are held to 256 registers, two waves per SIMD (the
// pair loop's three runs of pairs otherwise drift a few registers past it
// and halve the waves); f32 tiles need more than that.
template <int KVT, int D, int NW, int MODE, int PF, int NPK, bool PAIRS>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KVT == KV_F32 ? 1 : 2)))
void paged_prefill_persistent(const DecodeParams p) {
  __shared__ ItemShared<NW, D / 16> sm;
  __shared__ int s_cum[kMaxSeqsPersistent + 1];   // items before sequence b
  __shared__ int s_len[kMaxSeqsPersistent];       // context length
  __shared__ int s_q0[kMaxSeqsPersistent];        // first query row
  __shared__ int s_nq[kMaxSeqsPersistent];        // query rows
  __shared__ int s_ccum[kMaxSeqsPersistent + 1];  // tiles of the items before sequence b
  __shared__ int s_span[kMaxSeqsPersistent];      // tiles of one kv head's groups
  __shared__ int s_wsum[2][NW];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int TPG = p.tokens_per_pack * NPK;   // tokens of a group of packs
  auto parts_of = [&](int L, int n) {   // partitions of each group of a sequence
    return n > 0 ? ((L + kBlockSize - 1) / kBlockSize + p.partition_blocks - 1) / p.partition_blocks : 0;
  };

  // Exclusive prefix sums over sequences of the items and of their tiles
  // (Hkv x the blocks every group reads: group_prefix).
  int carry = 0, ccarry = 0;
  for (int c0 = 0; c0 < B; c0 += NW * 64) {
    const int i = c0 + static_cast<int>(threadIdx.x);
    int items = 0, cost = 0;
    if (i < B) {
      const int L = max(0, min(p.context_lens[i], p.mbps * kBlockSize));
      const int q0 = max(0, min(p.query_start[i], p.num_query_tokens));
      const int q1 = max(q0, min(p.query_start[i + 1], p.num_query_tokens));
      const int n = min(q1 - q0, L);
      const int span = static_cast<int>(group_prefix(L, n, TPG, num_groups(n, TPG)));
      s_len[i] = L;
      s_q0[i] = q0;
      s_nq[i] = n;
      s_span[i] = span;
      items = Hkv * num_groups(n, TPG) * parts_of(L, n);
      cost = Hkv * span;
    }
    int x = items, y = cost;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int xs = __shfl_up(x, off);
      const int ys = __shfl_up(y, off);
      if (lane >= off) {
        x += xs;
        y += ys;
      }
    }
    if (lane == 63) {
      s_wsum[0][wid] = x;
      s_wsum[1][wid] = y;
    }
    __syncthreads();
    int before = carry, cbefore = ccarry;
    for (int w = 0; w < wid; ++w) {
      before += s_wsum[0][w];
      cbefore += s_wsum[1][w];
    }
    int total = 0, ctotal = 0;
    for (int w = 0; w < NW; ++w) {
      total += s_wsum[0][w];
      ctotal += s_wsum[1][w];
    }
    if (i < B) {
      s_cum[i + 1] = before + x;
      s_ccum[i + 1] = cbefore + y;
    }
    if (i == 0) s_cum[0] = s_ccum[0] = 0;
    carry += total;
    ccarry += ctotal;
    __syncthreads();
  }
  const int N = carry;
  const int C = ccarry;
  // In one pass with more items than workgroups, XCD ranges are cut by
  // tiles, not by items: items (sequence, kv head, group) differ in length
  // with their sequence's context, and ranges of equal item counts left
  // the most loaded wave 1.92x the mean (chunked prefill; 1.33x by tiles,
  // host count; measured 214 -> 184 us).  With at most one item per
  // workgroup the step is bound by its longest item whatever the ranges,
  // and equal counts keep every workgroup at one item (speculative
  // verification: 71 us, 76 by tiles).  Partitioned items are capped at a
  // partition's blocks, so counts already track tiles (by tiles: 1.42x ->
  // 1.55x on the host count, P = 1024 242 -> 285 us).  First item at or
  // after tile c of the item order.
  auto item_at = [&](int64_t c) {
    if (c >= C) return N;
    int lo_b = 0, hi_b = B;
    while (hi_b - lo_b > 1) {
      const int mid = (lo_b + hi_b) >> 1;
      if (s_ccum[mid] <= c) lo_b = mid;
      else hi_b = mid;
    }
    const int b = lo_b;
    const int L = s_len[b], n = s_nq[b];
    const int ng = num_groups(n, TPG);
    const int parts = parts_of(L, n);
    const int rem = static_cast<int>(c - s_ccum[b]);
    const int h = rem / s_span[b];
    const int rem2 = rem - h * s_span[b];
    int lo_g = 0, hi_g = ng;
    while (hi_g - lo_g > 1) {
      const int mid = (lo_g + hi_g) >> 1;
      if (group_prefix(L, n, TPG, mid) <= rem2) lo_g = mid;
      else hi_g = mid;
    }
    const int part = (rem2 - static_cast<int>(group_prefix(L, n, TPG, lo_g))) / p.partition_blocks;
    return s_cum[b] + (h * ng + lo_g) * parts + min(part, parts - 1);
  };
  const int xcd = blockIdx.x % kXcds;
  const int per_xcd = gridDim.x / kXcds;
  const bool by_tiles = MODE == MODE_FINAL && N > static_cast<int>(gridDim.x);
  const int lo = by_tiles ? item_at(static_cast<int64_t>(C) * xcd / kXcds)
                          : static_cast<int>(static_cast<int64_t>(N) * xcd / kXcds);
  const int hi = by_tiles ? item_at(static_cast<int64_t>(C) * (xcd + 1) / kXcds)
                          : static_cast<int>(static_cast<int64_t>(N) * (xcd + 1) / kXcds);
  // Item n -> (sequence, kv head, group of packs, partition), partition fastest.
  auto locate = [&](int n, int& b, int& h, int& pack, int& part) {
    int lo_b = 0, hi_b = B;
    while (hi_b - lo_b > 1) {
      const int mid = (lo_b + hi_b) >> 1;
      if (s_cum[mid] <= n) lo_b = mid;
      else hi_b = mid;
    }
    b = lo_b;
    const int parts = parts_of(s_len[b], s_nq[b]);
    const int per_head = ((s_nq[b] + TPG - 1) / TPG) * parts;
    const int local = n - s_cum[b];
    h = local / per_head;
    const int rem = local % per_head;
    pack = rem / parts;
    part = rem % parts;
  };
  int n = lo + static_cast<int>(blockIdx.x) / kXcds;
  if (n >= hi) return;
  // An item's ids and q load at its start: items here are long (many
  // tiles per wave), so the one exposed latency costs little, and holding
  // the next item's q operands through the current one would take 32
  // registers (measured: no faster with them).
  while (true) {
    int b, h, pack, part;
    locate(n, b, h, pack, part);
    PackPrefetch<KVT, D, NPK> cur;
    prefill_prefetch<KVT, D, NW, NPK>(p, b, h, pack, part, QueryRows{s_q0[b], s_nq[b]}, cur);
    prefill_item<KVT, D, NW, MODE, PF, NPK, PAIRS>(p, b, h, pack, part, s_len[b], QueryRows{s_q0[b], s_nq[b]}, cur,
                                                   sm);
    __syncthreads();   // the next item reuses the merge state
    n += per_xcd;
    if (n >= hi) break;
  }
}

// One wave per (query row, head): merges the row's partitions 0 ..
// ceil((position + 1) / P) - 1.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // wave-uniform
  if (pair >= p.num_query_tokens * p.num_q_heads) return;
  const int t = pair / p.num_q_heads;
  // Sequence of row t: last b with query_start[b] <= t.
  int lo_b = 0, hi_b = p.num_seqs;
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (p.query_start[mid] <= t) lo_b = mid;
    else hi_b = mid;
  }
  const int b = lo_b;
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  const int q0 = max(0, min(p.query_start[b], p.num_query_tokens));
  const int q1 = max(q0, min(p.query_start[b + 1], p.num_query_tokens));
  const int nq = min(q1 - q0, L);
  float acc[D / 64];
  if (t - q0 >= nq || t < q0) {   // no such row in a consistent batch: zeros
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
  } else {
    const int pos = L - nq + (t - q0);
    const int n = min((pos + p.partition_size) / p.partition_size, p.num_partitions);
    merge_partitions<D, false>(p.tmp_lse + static_cast<size_t>(pair) * p.num_partitions,
                               p.tmp_out + static_cast<size_t>(pair) * p.num_partitions * D, n, lane, acc);
  }
  store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
}

// ------------------------------------------------------ balanced schedule
// Per-wave form (E4M3 caches; the others take the per-compute-unit form
// below).  Every wave of a resident grid is a worker with an equal share of
// the batch's 16-token tiles, whatever the mix of context lengths.  The tiles
// of all (sequence, kv head) items form one stream -- sequence-major, then
// kv head, then block -- and worker w of R takes tiles [T*w/R, T*(w+1)/R).
// A share may begin or end inside an item: each piece of an item that a
// worker covers is a segment with its own normalised partial output and
// log-sum-exp (flash-decoding's split, at tile granularity), and the merge
// kernel combines an item's segments.  A segment that is a whole item
// writes the output directly.
//
// Segment (item i, worker w) keeps its partial in slot i + w: along the
// stream both i and w are non-decreasing and one of them grows at every new
// segment, so slots never collide, and item i's segments are the slots
// i + w0 .. i + w1 (w0, w1 the workers of its first and last tile).
constexpr int kMinTilesPerWorker = 8;

__device__ __forceinline__ int stream_workers(int T, int max_workers) {
  return min(max_workers, (T + kMinTilesPerWorker - 1) / kMinTilesPerWorker);
}
// Worker holding tile t: the largest w with floor(T*w/R) <= t.
__device__ __forceinline__ int stream_worker_of(int64_t t, int T, int R) {
  return static_cast<int>(((t + 1) * R + T - 1) / T - 1);
}

template <int KVT, int D, int NW, int PF>
__global__ __launch_bounds__(NW * 64) void paged_decode_stream(const DecodeParams p) {
  constexpr int NT = D / 16;
  __shared__ int s_cum[kMaxSeqsPersistent + 1];   // tiles before sequence b
  __shared__ int s_len[kMaxSeqsPersistent];       // context length of sequence b
  __shared__ int s_wsum[NW];
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = p.group;

  // Exclusive prefix sum over sequences of Hkv * blocks (LDS).
  int carry = 0;
  for (int c = 0; c < B; c += NW * 64) {
    const int i = c + static_cast<int>(threadIdx.x);
    int tiles = 0;
    if (i < B) {
      const int L = max(0, min(p.context_lens[i], p.mbps * kBlockSize));
      s_len[i] = L;
      tiles = Hkv * ((L + kBlockSize - 1) / kBlockSize - window_block(L, p.window));
    }
    int x = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wid] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wid; ++w) before += s_wsum[w];
    int total = 0;
    for (int w = 0; w < NW; ++w) total += s_wsum[w];
    if (i < B) s_cum[i + 1] = before + x;
    if (i == 0) s_cum[0] = 0;
    carry += total;
    __syncthreads();
  }
  const int T = carry;
  // The merge kernel reads the same prefix sums.
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= B; i += NW * 64) p.seq_tiles[i] = s_cum[i];
  if (T == 0) return;

  // Workers fill 8 contiguous ranges, one per XCD (workgroup k runs on XCD
  // k % 8), so neighbouring sequences -- the ones likely to share prefix
  // blocks -- go through one L2; inside a range, workers spread over the
  // workgroups first.  From here on the waves are independent.
  const int R = stream_workers(T, p.num_workers);
  const int xcd = blockIdx.x % kXcds;
  const int wg_per_xcd = gridDim.x / kXcds;
  const int r_lo = R * xcd / kXcds;
  const int r_hi = R * (xcd + 1) / kXcds;
  const int w = r_lo + wid * wg_per_xcd + static_cast<int>(blockIdx.x) / kXcds;
  if (w >= r_hi) return;
  const int t_begin = static_cast<int>(static_cast<int64_t>(T) * w / R);
  const int t_end = static_cast<int>(static_cast<int64_t>(T) * (w + 1) / R);

  // An item's tiles are its blocks from the window's first block on:
  // tile j of sequence b is block window_block(L_b) + j.
  auto item_tiles = [&](int b) {
    return (s_len[b] + kBlockSize - 1) / kBlockSize - window_block(s_len[b], p.window);
  };
  // Tile t -> (sequence, kv head, tile of the item): last b with s_cum[b] <= t.
  auto locate = [&](int t, int& b, int& h, int& j) {
    int lo_b = 0, hi_b = B;
    while (hi_b - lo_b > 1) {
      const int mid = (lo_b + hi_b) >> 1;
      if (s_cum[mid] <= t) lo_b = mid;
      else hi_b = mid;
    }
    b = lo_b;
    const int nt = item_tiles(b);
    const int local = t - s_cum[b];
    h = local / nt;
    j = local % nt;
  };

  int t = t_begin;
  int b, h, j0, b2, h2, j2;
  locate(t, b, h, j0);
  ItemPrefetch<KVT, D> cur, nxt;
  meta_prefetch<KVT, D>(p, b, h, window_block(s_len[b], p.window) + j0, 1, cur);
  WaveState<NT> st;
  while (true) {
    const int L = s_len[b];
    const int lo = window_lo(L, p.window);
    const int base = lo / kBlockSize;
    const int nt = item_tiles(b);
    const int j1 = min(nt, j0 + (t_end - t));
    const int t2 = t + (j1 - j0);
    // The next segment's ids and q load while this one streams (the last
    // segment prefetches its own last tile again: never a conditional load).
    locate(min(t2, t_end - 1), b2, h2, j2);
    meta_prefetch<KVT, D>(p, b2, h2, window_block(s_len[b2], p.window) + j2, 1, nxt);
    st.reset();
    attend_blocks<KVT, D, PF>(p, b, h, L, lo, base + j0, 1, j1 - j0, cur.ids, cur.qop, st);
    const float l_sum = sum_over_groups(st.l);
    const float inv = 1.f / l_sum;
    if (r < G) {
      if (j0 == 0 && j1 == nt) {   // the whole item: final output
        const size_t row = (static_cast<size_t>(b) * p.num_q_heads + h * G + r) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) store4(p.out, row + 16 * n + 4 * g, p.out_dtype, st.o[n] * inv);
      } else {
        const size_t slot = static_cast<size_t>(r) * p.num_slots + b * Hkv + h + w;
#pragma unroll
        for (int n = 0; n < NT; ++n)
          *reinterpret_cast<f32x4*>(p.tmp_out + slot * D + 16 * n + 4 * g) = st.o[n] * inv;
        if (g == 0) p.tmp_lse[slot] = (st.m + fast_log2(l_sum)) * kLn2;
      }
    }
    if (t2 >= t_end) break;
    t = t2;
    b = b2;
    h = h2;
    j0 = j2;
    cur = nxt;
  }
}

// One wave per (sequence, query head): merges the item's segments when its
// tiles were split between workers, writes zeros for an empty context.
template <int D>
__global__ __launch_bounds__(256) void stream_merge_kernel(const ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // wave-uniform
  if (pair >= p.num_seqs * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int qh = pair % p.num_q_heads;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int h = qh / G;
  const int gg = qh % G;
  // Sequence b's blocks follow from the tile offsets the stream kernel
  // left: (seq_tiles[b + 1] - seq_tiles[b]) / Hkv.
  const int s0 = p.seq_tiles[b];
  const int nb = (p.seq_tiles[b + 1] - s0) / p.num_kv_heads;
  const int T = p.seq_tiles[p.num_seqs];
  float acc[D / 64];
  if (nb == 0) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
    store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
    return;
  }
  const int R = stream_workers(T, p.num_workers);
  const int64_t s = s0 + static_cast<int64_t>(h) * nb;
  const int w0 = stream_worker_of(s, T, R);
  const int w1 = stream_worker_of(s + nb - 1, T, R);
  if (w0 == w1) return;   // one segment: its worker wrote the output
  const size_t slot0 = static_cast<size_t>(gg) * p.num_slots + b * p.num_kv_heads + h + w0;
  merge_partitions<D, false>(p.tmp_lse + slot0, p.tmp_out + slot0 * D, w1 - w0 + 1, lane, acc);
  store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
}

// ------------------------------------------------- CU-balanced schedule
// One workgroup per compute unit, and every unit gets an equal, tile-exact
// share of the batch's 16-token tiles (the sequence-major stream of the
// per-wave schedule above, with shares in the place of its workers): the
// time of a memory-bound step is set by the unit that streams the most.
// Inside a unit the waves take their tiles at run time.  Waves of one unit
// do not stream at one rate (measured with equal fixed shares: the wave
// placed first on a SIMD finished a third earlier than the second), so a
// fixed split leaves a unit partly idle at its end.
//
// Parts and units.  A piece is the part of one (sequence, kv head) item
// that falls in the share.  Its tiles among the item's first kCuCachedTiles
// form the piece's first part, loaded with the ordinary cache policy
// (prompts shared between sequences sit at the start, and the caches keep
// them for the other sequences); the rest form its second part, streamed
// (non-temporal).  Each part is cut into units of up to RD consecutive
// tiles.  Units are numbered over the first parts of all the share's pieces,
// then over the second parts, and a wave takes the next unit with one LDS
// atomic add, finding it by walking a cursor of its own forward (the
// numbers a wave takes only grow).  A unit has one item, so one query
// operand and one softmax state; and a wave meets all first-part units
// before any second-part unit, so each phase runs in a loop of its own with
// a single load policy.
//
// A wave keeps a running state for the part it is on.  When its next unit
// belongs to another part it disposes of the state: a state covering the
// whole part is written out at once; any other is merged into the part's
// LDS accumulator (a slot found or taken under an allocation lock, merged
// under the slot's own lock), and the wave whose merge completes the part's
// tile count writes the result and frees the slot.  A result is the output
// when the part is the whole item, else a partial (normalised output and
// natural-log LSE) in slot item + share of the phase's array, merged across
// parts and shares by cu_merge_kernel.  No lock is held while waiting for
// anything else, and a slot is never short: each slot in use belongs to a
// part that still has tiles in some wave (in its state or in one of the
// three units it has taken), a wave covers at most four parts, and there
// are 4 x NW slots.  So no wave ever waits for another wave's tiles.
//
// Which wave takes which unit varies from call to call, and so does the
// order in which a part's tiles are summed: two calls may differ in the
// last bits of fp32.
constexpr int kSlotFree = -1;
constexpr int kSpinLimit = 1 << 22;
// Tiles of an item's first part (cached loads).  Measured on the ragged
// 128-sequence layer with 32-block shared prompts: 32 / 36 / 40 / 44 / 48 /
// 56 / 64; 40 was fastest, ~0.4 us ahead of 48 over seven paired runs.
constexpr int kCuCachedTiles = 40;

template <int NT>
struct CuAcc {
  f32x4 o[NT][64];   // lane layout of WaveState::o
  float m[16];       // per head column: reference max (log2 units)
  float l[16];       // per head column: sum of exp2(x - m)
};

template <int NT, int NS>
struct CuShared {
  CuAcc<NT> acc[NS];
  int tag[NS];      // ordinal of the part the slot holds, or kSlotFree
  int tiles[NS];    // tiles merged into the slot so far
  int lock[NS];     // guards the slot's accumulator and tile count
  int alloc_lock;   // guards finding or taking a slot for a part
  int next_unit;    // first unit no wave has taken
};

// One tile's step of the online softmax for the G heads of a KV head (one
// wave): logits, lazy max, P, PV.  vexp as in attend_packs (E4M3 only).
template <int KVT, int D>
__device__ __forceinline__ void cu_tile(WaveState<D / 16>& st, int& vexp, const u32x4 (&kt)[TileOps<KVT, D>::NLOAD],
                                        u32x4 (&vt)[TileOps<KVT, D>::NLOAD], float ksc, float vsc,
                                        const u32x4 (&qop)[TileOps<KVT, D>::NQ], float qk_scale_log2, int tok0,
                                        int L, int lo, int g) {
  typedef TileOps<KVT, D> T;
  constexpr int NT = T::NT;
  float f = qk_scale_log2;
  float pscale = 1.f;
  if constexpr (KVT == KV_E4M3) {
    f *= ksc;
    const uint32_t vbits = __builtin_amdgcn_readfirstlane(__float_as_uint(vsc));
    const int e_blk = static_cast<int>((vbits >> 23) & 0xFFu) - 126;
    if (e_blk > vexp) {
      const float shrink = __builtin_amdgcn_ldexpf(1.f, vexp - e_blk);
#pragma unroll
      for (int n = 0; n < NT; ++n) st.o[n] *= shrink;
      vexp = e_blk;
    }
    pscale = __builtin_amdgcn_ldexpf(__uint_as_float(vbits), 7 - vexp);
  }
  const bool tail = tok0 + kBlockSize > L;
  if (tail) T::mask_v(vt, L - tok0 - 4 * g);
  const f32x4 s = T::qk(kt, qop);
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = s[j] * f;
  if (tail) {
    const int nv = L - tok0 - 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (j < nv) ? x[j] : -INFINITY;
  }
  if (tok0 < lo) {
    const int nlo = lo - tok0 - 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (j < nlo) ? -INFINITY : x[j];
  }
  const float bm = max_over_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if (__any(bm > st.m + kSlack)) {
    const float m_new = fmaxf(st.m, bm);
    const float alpha = fast_exp2(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.o[n] *= alpha;
  }
  float pr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - st.m);
  st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  T::pv(st.o, vt, pr, pscale);
}

// Writes a finished part: out (normalised) for a whole item, else the
// partial pair (normalised output, natural-log LSE) in slot item + share of
// the phase's array (0: first parts, 1: second parts).
// Column r of lane (g, r) is query head h*G + r; acc is O^T d-tiles.
template <int D>
__device__ __forceinline__ void cu_emit(const DecodeParams& p, int b, int h, int item, int share, int phase,
                                        bool whole, float M, float Lsum, const f32x4 (&acc)[D / 16], int g, int r) {
  constexpr int NT = D / 16;
  const int G = p.group;
  if (r >= G) return;
  const float inv = 1.f / Lsum;
  if (whole) {
    const size_t row = (static_cast<size_t>(b) * p.num_q_heads + h * G + r) * D;
#pragma unroll
    for (int n = 0; n < NT; ++n) store4(p.out, row + 16 * n + 4 * g, p.out_dtype, acc[n] * inv);
  } else {
    const size_t slot = static_cast<size_t>(phase * G + r) * p.num_slots + item + share;
#pragma unroll
    for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4*>(p.tmp_out + slot * D + 16 * n + 4 * g) = acc[n] * inv;
    if (g == 0) p.tmp_lse[slot] = (M + fast_log2(Lsum)) * kLn2;
  }
}

template <int KVT, int D, int NW, int RD>
__global__ __launch_bounds__(NW * 64) void paged_decode_cu_stream(const DecodeParams p) {
  typedef TileOps<KVT, D> T;
  constexpr int NT = T::NT;
  constexpr int NL = T::NLOAD;
  constexpr int NQ = T::NQ;
  constexpr int E = ElemBytes<KVT>::value;
  constexpr int TILE = kBlockSize * D * E;
  constexpr int QB = (KVT == KV_F32) ? 4 : 2;
  // Accumulator slots: a slot is taken by the first wave that parks a
  // part and freed by the merge that completes it, so every part holding a
  // slot still has tiles in some wave (in its state or in one of the three
  // units it has taken), and a wave covers at most four parts: 4 * NW slots
  // never run out.
  constexpr int NS = 4 * NW;
  static_assert(sizeof(CuShared<NT, NS>) + sizeof(int) * (2 * kMaxSeqsPersistent + 1 + NW) > 80 * 1024,
                "the LDS must keep a second workgroup off the compute unit");
  __shared__ CuShared<NT, NS> sh;
  __shared__ int s_cum[kMaxSeqsPersistent + 1];   // tiles before sequence b
  __shared__ int s_len[kMaxSeqsPersistent];       // context length of sequence b
  __shared__ int s_wsum[NW];
  const int B = p.num_seqs;
  const int Hkv = p.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = p.group;

  if (threadIdx.x < NS) {
    sh.tag[threadIdx.x] = kSlotFree;
    sh.tiles[threadIdx.x] = 0;
    sh.lock[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    sh.next_unit = 2 * NW;   // units w and NW + w are wave w's first two, taken without the counter
    sh.alloc_lock = 0;
  }
  // Exclusive prefix sum over sequences of Hkv * (tiles from the window's
  // first block to the end).
  int carry = 0;
  for (int c = 0; c < B; c += NW * 64) {
    const int i = c + static_cast<int>(threadIdx.x);
    int tiles = 0;
    if (i < B) {
      const int L = max(0, min(p.context_lens[i], p.mbps * kBlockSize));
      s_len[i] = L;
      tiles = Hkv * ((L + kBlockSize - 1) / kBlockSize - window_block(L, p.window));
    }
    int x = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wid] = x;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wid; ++w) before += s_wsum[w];
    int total = 0;
    for (int w = 0; w < NW; ++w) total += s_wsum[w];
    if (i < B) s_cum[i + 1] = before + x;
    if (i == 0) s_cum[0] = 0;
    carry += total;
    __syncthreads();
  }
  const int Tt = carry;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= B; i += NW * 64) p.seq_tiles[i] = s_cum[i];
  // Share of this workgroup: consecutive shares sit on one XCD (workgroup k
  // runs on XCD k % 8), so neighbouring sequences, the ones likely to share
  // prompt blocks, go through one L2.  A small batch uses fewer shares, at
  // least kMinTilesPerWorker tiles each, so no share is empty (the merge
  // takes every share an item spans).
  const int nwg = gridDim.x;
  const int R = stream_workers(Tt, nwg);
  const int share = (nwg % kXcds == 0)
                        ? static_cast<int>(blockIdx.x % kXcds) * (nwg / kXcds) + static_cast<int>(blockIdx.x) / kXcds
                        : static_cast<int>(blockIdx.x);
  if (share >= R) return;
  const int t0 = static_cast<int>(static_cast<int64_t>(Tt) * share / R);
  const int t1 = static_cast<int>(static_cast<int64_t>(Tt) * (share + 1) / R);
  if (t1 <= t0) return;

  // Parts.  Every piece has a first part, its tiles among the first
  // kCuCachedTiles of the item (loaded with the ordinary cache policy), and
  // a second part, the rest (streamed); either may be empty.  Units are
  // numbered over the first parts of all the share's pieces, then over the
  // second parts, so a wave's units run through the first phase and then
  // the second, and each phase has a loop of its own with one load policy
  // (a branch between policies around the loads would make the compiler
  // wait for every load in flight).  Parts are numbered the same way (part
  // ordinal pk: piece index in the first phase, pieces + piece index in the
  // second), the order in which their units are taken.
  //
  // The wave's cursor: the piece (item (b, h), whose nb tiles are stream
  // tiles s_i .. s_i + nb - 1; the piece is stream tiles [ps, pe)), the
  // phase, the first unit of the current part (ubase) and its ordinal.
  struct Cursor {
    int b, h, nb, s_i, ps, pe, ubase, pk, phase;
  };
  auto item_tiles = [&](int b) __attribute__((always_inline)) {
    const int L = s_len[b];
    return __builtin_amdgcn_readfirstlane((L + kBlockSize - 1) / kBlockSize - window_block(L, p.window));
  };
  auto set_piece = [&](Cursor& c) __attribute__((always_inline)) {
    c.s_i = __builtin_amdgcn_readfirstlane(s_cum[c.b]) + c.h * c.nb;
    c.ps = max(c.s_i, t0);
    c.pe = min(c.s_i + c.nb, t1);
  };
  // Stream tiles [qa, qb) of the cursor's part (qb <= qa: empty).
  auto part_of = [&](const Cursor& c, int& qa, int& qb) __attribute__((always_inline)) {
    const int cut = c.s_i + kCuCachedTiles;
    qa = c.phase == 0 ? c.ps : max(c.ps, cut);
    qb = c.phase == 0 ? min(c.pe, cut) : c.pe;
  };
  auto part_units = [&](const Cursor& c) __attribute__((always_inline)) {
    int qa, qb;
    part_of(c, qa, qb);
    return qb > qa ? (qb - qa + RD - 1) / RD : 0;
  };
  Cursor first;
  {
    // Sequence of tile t0: the last b with s_cum[b] <= t0, by a two-level
    // 64-way search (each level one LDS read per lane and a ballot; B <=
    // 4096, and s_cum[0] = 0 <= t0 sets the first bit of each ballot).
    const int stride = (B + 63) / 64;
    const int i1 = lane * stride;
    const uint64_t m1 = __ballot(i1 < B && s_cum[min(i1, B - 1)] <= t0);
    const int base = (63 - __builtin_clzll(m1)) * stride;
    const int i2 = base + lane;
    const uint64_t m2 = __ballot(lane < stride && i2 < B && s_cum[min(i2, B - 1)] <= t0);
    const int lo_b = __builtin_amdgcn_readfirstlane(base + 63 - __builtin_clzll(m2));
    first.b = lo_b;
    first.nb = item_tiles(lo_b);
    first.h = (t0 - __builtin_amdgcn_readfirstlane(s_cum[lo_b])) / first.nb;
    set_piece(first);
    first.ubase = 0;
    first.pk = 0;
    first.phase = 0;
  }
  Cursor cur = first;   // (the slot tags, locks and counter set above are visible: the prefix loop synchronised)

  const char* kcache = static_cast<const char*>(p.k_cache);
  const char* vcache = static_cast<const char*>(p.v_cache);
  uint32_t lane_off[NL];
#pragma unroll
  for (int m = 0; m < NL; ++m) lane_off[m] = static_cast<uint32_t>(lane) * 16u + m * 1024u;
  const auto scale_r = make_tile_rsrc(p.kv_scales, KVT == KV_E4M3 ? 2 * p.num_blocks * Hkv * 4 : 0);

  // A unit taken by this wave.
  struct Claim {
    int b, h, j0, n;   // item (sequence b, kv head h), first block index, tiles (0: no unit left)
    int pk, len;       // part ordinal and its tile count
    int phase;         // 0: first part (cached), 1: second part (streamed)
    int whole;         // the part is the whole item
    int id;            // lane k < n: physical block of tile k
  };
  // Unit u (u < 0: the next one from the counter).
  auto claim = [&](Claim& C, int u = -1) __attribute__((always_inline)) {
    if (u < 0) {
      if (lane == 0) u = __hip_atomic_fetch_add(&sh.next_unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      u = __builtin_amdgcn_readfirstlane(u);
    }
    while (true) {
      if (cur.ps >= t1) {   // past the share's last piece
        if (cur.phase == 1) break;
        const int ub = cur.ubase, pk = cur.pk;
        cur = first;        // second phase: the pieces again, from the first
        cur.phase = 1;
        cur.ubase = ub;
        cur.pk = pk;
        continue;
      }
      const int units = part_units(cur);
      if (u < cur.ubase + units) break;
      cur.ubase += units;
      ++cur.pk;
      if (++cur.h == Hkv) {
        cur.h = 0;
        ++cur.b;
      }
      if (cur.b < B) {
        if (cur.h == 0) cur.nb = item_tiles(cur.b);
        set_piece(cur);
      } else {
        cur.ps = cur.pe = t1;
      }
    }
    if (cur.ps < t1) {
      int qa, qb;
      part_of(cur, qa, qb);
      const int ts = qa + (u - cur.ubase) * RD;   // the unit's first stream tile
      C.b = cur.b;
      C.h = cur.h;
      C.n = min(RD, qb - ts);
      C.j0 = window_block(__builtin_amdgcn_readfirstlane(s_len[cur.b]), p.window) + (ts - cur.s_i);
      C.pk = cur.pk;
      C.len = qb - qa;
      C.phase = cur.phase;
      C.whole = qa == cur.s_i && qb == cur.s_i + cur.nb;
    } else {
      C.b = C.h = C.j0 = C.n = 0;
      C.pk = -1;
      C.len = C.phase = C.whole = 0;
    }
    // Unconditional load (lanes without a tile read the unit's first entry).
    C.id = p.block_tables[static_cast<size_t>(C.b) * p.mbps + C.j0 + (lane < C.n ? lane : 0)];
  };

  // Ring of RD tile buffers: buffer k holds tile k of the unit being processed.
  u32x4 kb[RD][NL], vb[RD][NL];
  float ks[RD], vs[RD];
#pragma unroll
  for (int k = 0; k < RD; ++k) ks[k] = vs[k] = 1.f;
  auto load_tile = [&](int k, const Claim& C, auto policy) __attribute__((always_inline)) {
    constexpr int POL = decltype(policy)::value;
    const bool valid = k < C.n;
    const int blk = __builtin_amdgcn_readlane(C.id, k);
    const size_t tile = (static_cast<size_t>(valid ? blk : 0) * Hkv + C.h) * TILE;
    if constexpr (KVT == KV_E4M3) {
      const uint32_t so = static_cast<uint32_t>((valid ? blk : 0) * Hkv + C.h) * 4u;
      ks[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scale_r, so, 0, 0));
      vs[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            scale_r, so + static_cast<uint32_t>(p.num_blocks * Hkv) * 4u, 0, 0));
    }
    const auto kr = make_tile_rsrc(kcache + tile, valid ? TILE : 0);
    const auto vr = make_tile_rsrc(vcache + tile, valid ? TILE : 0);
#pragma unroll
    for (int m = 0; m < NL; ++m) kb[k][m] = buffer_ld16_policy<POL>(kr, lane_off[m]);
#pragma unroll
    for (int m = 0; m < NL; ++m) vb[k][m] = buffer_ld16_policy<POL>(vr, lane_off[m]);
  };
  // Query operand of a unit's item: head column r of the group (a zero-size
  // descriptor when there is no unit: every load still issues).
  auto load_q = [&](u32x4 (&qop)[NQ], const Claim& C) __attribute__((always_inline)) {
    const auto qr = make_tile_rsrc(
        static_cast<const char*>(p.q) + (static_cast<size_t>(C.b) * p.num_q_heads + C.h * G) * D * QB,
        C.n > 0 ? G * D * QB : 0);
    T::load_q(qop, qr, static_cast<uint32_t>(r * D * QB), g);
  };

  // The wave's running state and its part.
  WaveState<NT> st;
  int vexp = -126;
  int cpk = -1, cb = 0, chh = 0, clen = 0, cphase = 0, cwhole = 0, ccount = 0;

  // Dispose of the state of the current part (ccount of its clen tiles).
  auto finish_state = [&]() __attribute__((always_inline)) {
    const int item = cb * Hkv + chh;
    if constexpr (KVT == KV_E4M3) {
      const float grow = __builtin_amdgcn_ldexpf(1.f, vexp - 7);
#pragma unroll
      for (int n = 0; n < NT; ++n) st.o[n] *= grow;
    }
    float l_col = sum_over_groups(st.l);
    if (ccount == clen) {   // the whole part is in this state
      cu_emit<D>(p, cb, chh, item, share, cphase, cwhole, st.m, l_col, st.o, g, r);
      return;
    }
    // Find the part's slot, or take a free one (the first wave to park the
    // part), under the allocation lock; then merge under the slot's lock.
    // Neither lock is held while waiting for anything else.
    auto spin_lock = [&](int* l) __attribute__((always_inline)) {
      for (int it = 0; it < kSpinLimit; ++it) {
        int got = 0;
        if (lane == 0) {
          int expected = 0;
          got = __hip_atomic_compare_exchange_strong(l, &expected, 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (__builtin_amdgcn_readfirstlane(got)) break;
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    auto unlock = [&](int* l) __attribute__((always_inline)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) __hip_atomic_store(l, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int slot = 0;
    for (int it = 0; it < kSpinLimit; ++it) {   // one pass: a free slot exists (see NS)
      spin_lock(&sh.alloc_lock);
      const int t_lane = lane < NS ? sh.tag[lane] : 0;
      const uint64_t hit = __ballot(lane < NS && t_lane == cpk);
      const uint64_t free_slots = __ballot(lane < NS && t_lane == kSlotFree);
      if (hit || free_slots) {
        slot = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(hit ? hit : free_slots)));
        if (!hit && lane == 0) {
          sh.tag[slot] = cpk;
          sh.tiles[slot] = 0;
        }
        unlock(&sh.alloc_lock);
        break;
      }
      unlock(&sh.alloc_lock);
      __builtin_amdgcn_s_sleep(1);
    }
    CuAcc<NT>& a = sh.acc[slot];
    spin_lock(&sh.lock[slot]);
    const int before = __builtin_amdgcn_readfirstlane(sh.tiles[slot]);
    bool done = false;
    if (before == 0) {   // the first share of the part to arrive
#pragma unroll
      for (int n = 0; n < NT; ++n) a.o[n][lane] = st.o[n];
      if (g == 0) {
        a.m[r] = st.m;
        a.l[r] = l_col;
      }
      if (lane == 0) sh.tiles[slot] = ccount;
    } else {             // merge with what is there
      const float ms = a.m[r];
      const float mn = fmaxf(ms, st.m);
      const float fs = fast_exp2(ms - mn);
      const float fw = fast_exp2(st.m - mn);
#pragma unroll
      for (int n = 0; n < NT; ++n) st.o[n] = a.o[n][lane] * fs + st.o[n] * fw;
      l_col = a.l[r] * fs + l_col * fw;
      st.m = mn;
      const int total = before + ccount;
      done = total == clen;
      if (done) {
        if (lane == 0) sh.tag[slot] = kSlotFree;
      } else {
#pragma unroll
        for (int n = 0; n < NT; ++n) a.o[n][lane] = st.o[n];
        if (g == 0) {
          a.m[r] = mn;
          a.l[r] = l_col;
        }
        if (lane == 0) sh.tiles[slot] = total;
      }
    }
    unlock(&sh.lock[slot]);
    if (done) cu_emit<D>(p, cb, chh, item, share, cphase, cwhole, st.m, l_col, st.o, g, r);
  };

  constexpr std::integral_constant<int, 0> kCached{};
  constexpr std::integral_constant<int, kStreamLoad> kStream{};
  // P: the unit being processed (tiles in the ring, q in qop); N: the next
  // unit (ids loaded, q loading into qn, tiles loading as P's buffers free
  // up); Z: taken at the top of each round (ids loading).
  Claim P, N, Z;
  u32x4 qop[NQ], qn[NQ];
  // One round: P's tiles through the state; tile k of N goes into buffer k
  // as soon as it is free (a zero-size load past N's end), with the given
  // cache policy.
  auto round = [&](auto policy) __attribute__((always_inline)) {
    claim(Z);
    load_q(qn, N);
    if (P.pk != cpk) {   // a unit has one part: switch between units only
      if (cpk >= 0) finish_state();
      st.reset();
      vexp = -126;
      cpk = P.pk;
      cb = P.b;
      chh = P.h;
      clen = P.len;
      cphase = P.phase;
      cwhole = P.whole;
      ccount = 0;
    }
    const int L = __builtin_amdgcn_readfirstlane(s_len[P.b]);
    const int lo = window_lo(L, p.window);
#pragma unroll
    for (int k = 0; k < RD; ++k) {
      if (k < P.n) {
        cu_tile<KVT, D>(st, vexp, kb[k], vb[k], ks[k], vs[k], qop, p.qk_scale_log2, (P.j0 + k) * kBlockSize, L,
                        lo, g);
        ++ccount;
      }
      load_tile(k, N, policy);
    }
  };
  auto rotate = [&]() __attribute__((always_inline)) {
    P = N;
    N = Z;
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = qn[m];
  };
  claim(P, wid);
  if (P.n == 0) return;
  load_q(qop, P);
  claim(N, NW + wid);
#pragma unroll
  for (int k = 0; k < RD; ++k) load_tile(k, P, kCached);   // (a second-part first unit is cached too)
  // First phase: N's tiles cached.
  while (N.n > 0 && N.phase == 0) {
    round(kCached);
    rotate();
  }
  // Second phase: N's tiles streamed (or none).
  while (true) {
    round(kStream);
    if (N.n == 0) break;
    rotate();
  }
  finish_state();
}

// Merges, per (sequence, query head), the parts of items that were not
// written whole: item i's first parts sit in slots i + w of the first
// array for the shares w0 .. wa holding its first kCuCachedTiles tiles, its
// second parts in slots i + w of the second array for the shares wb .. w1
// holding the rest; an empty context gets zeros.
template <int D>
__global__ __launch_bounds__(256) void cu_merge_kernel(const ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // wave-uniform
  if (pair >= p.num_seqs * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int qh = pair % p.num_q_heads;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int h = qh / G;
  const int gg = qh % G;
  const int s0 = p.seq_tiles[b];
  const int nb = (p.seq_tiles[b + 1] - s0) / p.num_kv_heads;
  const int T = p.seq_tiles[p.num_seqs];
  float acc[D / 64];
  if (nb == 0) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
    store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
    return;
  }
  const int R = stream_workers(T, p.num_workers);
  const int64_t s = s0 + static_cast<int64_t>(h) * nb;
  const int na = min(nb, kCuCachedTiles);   // tiles of the first parts
  const int w0 = stream_worker_of(s, T, R);
  const int wa = stream_worker_of(s + na - 1, T, R);
  if (na == nb && w0 == wa) return;        // one part, the whole item: written directly
  const int item = b * p.num_kv_heads + h;
  const size_t first = (static_cast<size_t>(gg) * p.num_slots + item + w0);
  int wb = 0, nparts_b = 0;
  if (nb > na) {
    wb = stream_worker_of(s + na, T, R);
    nparts_b = stream_worker_of(s + nb - 1, T, R) - wb + 1;
  }
  const size_t second = (static_cast<size_t>(G + gg) * p.num_slots + item + wb);
  merge_partitions2<D>(p.tmp_lse + first, p.tmp_out + first * D, wa - w0 + 1, p.tmp_lse + second,
                       p.tmp_out + second * D, nparts_b, lane, acc);
  store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
}

// ----------------------------------------------------------------- reduce
// One wave per (sequence, query head) merges its non-empty partitions.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));  // wave-uniform
  if (pair >= p.num_seqs * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  const int origin = window_block(L, p.window) * kBlockSize;   // partition 0's first position
  const int n = min((L - origin + p.partition_size - 1) / p.partition_size, p.num_partitions);
  float acc[D / 64];
  if (n > 0) {
    merge_partitions<D, false>(p.tmp_lse + static_cast<size_t>(pair) * p.num_partitions,
                        p.tmp_out + static_cast<size_t>(pair) * p.num_partitions * D, n, lane, acc);
  } else {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
  }
  store_row_part<D>(p.out, pair, lane, p.out_dtype, acc);
}

// --------------------------------------------------------------- launchers
constexpr int kWaves = 4;
#ifndef PKV_PREFETCH
#define PKV_PREFETCH 2
#endif
constexpr int kPrefetch = PKV_PREFETCH;  // tile buffers per wave

// Ring depth (tile buffers per wave).  Two: one tile streams in while the
// matrix cores work on the other.  Deeper rings (3-4, for the smaller e4m3
// and D = 64 tiles too) measured no faster: with two waves per SIMD the
// loads in flight already cover the memory latency.
template <int KVT, int D>
constexpr int ring_depth() {
  return kPrefetch;
}

// Workgroups of kernel KERNEL that fit on the current device at once
// (compute units x resident workgroups per unit); queried once per kernel
// and device.  The kernel is a template argument so that every kernel has a
// cache of its own (they share one function type).
template <auto KERNEL, int MAX_PER_CU = 0>
static int resident_workgroups(int block) {
  static std::atomic<int> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 16) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERNEL, block, 0) != hipSuccess || per_cu <= 0) per_cu = 1;
  if (MAX_PER_CU > 0) per_cu = std::min(per_cu, MAX_PER_CU);
  const int n = cus * per_cu;
  if (dev < 16) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int KVT, int D, int MODE, int PF>
static hipError_t launch_mode(const DecodeParams& p, hipStream_t stream) {
  const int block = kWaves * 64;
  const int64_t items = static_cast<int64_t>(p.num_partitions) * p.num_kv_heads * p.num_seqs;
  if (items == 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (p.num_seqs <= kMaxSeqsPersistent) {
    auto kernel = paged_decode_persistent<KVT, D, kWaves, MODE, PF>;
    int64_t grid = std::min<int64_t>(items, resident_workgroups<paged_decode_persistent<KVT, D, kWaves, MODE, PF>>(block));
    grid = std::max<int64_t>(kXcds, grid / kXcds * kXcds);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(block), 0, stream, p);
  } else {
    hipLaunchKernelGGL((paged_decode_kernel<KVT, D, kWaves, MODE, PF>), dim3(static_cast<unsigned>(items)),
                       dim3(block), 0, stream, p);
  }
  return hipGetLastError();
}

template <int KVT, int D>
static hipError_t launch_decode_t(DecodeParams p, int mode, hipStream_t stream) {
  constexpr int kPf = ring_depth<KVT, D>();
  if (mode == MODE_FINAL) p.num_partitions = 1;
  if (mode == MODE_PARTIAL) return launch_mode<KVT, D, MODE_PARTIAL, kPf>(p, stream);
  if (mode == MODE_SPLIT) return launch_mode<KVT, D, MODE_SPLIT, kPf>(p, stream);
  return launch_mode<KVT, D, MODE_FINAL, kPf>(p, stream);
}

// Balanced schedule: the grid of the stream kernel for the current device.
template <int KVT, int D>
static int stream_grid() {
  constexpr int kPf = ring_depth<KVT, D>();
  // At most two workgroups per CU: where registers allow three (the 16-bit
  // and E4M3 kernels), the third made the FP8 layer 6% and the ragged B=128
  // layer 4% slower (smaller shares, more segments to merge).
  const int res = resident_workgroups<paged_decode_stream<KVT, D, kWaves, kPf>, 2>(kWaves * 64);
  return std::max(kXcds, res / kXcds * kXcds);
}

template <int KVT, int D>
static hipError_t launch_stream_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int kPf = ring_depth<KVT, D>();
  const int grid = stream_grid<KVT, D>();
  if (p.num_workers != grid * kWaves) return hipErrorInvalidValue;
  hipLaunchKernelGGL((paged_decode_stream<KVT, D, kWaves, kPf>), dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int KVT>
static hipError_t launch_decode_d(const DecodeParams& p, int head_dim, int mode, hipStream_t s) {
  return head_dim == 64 ? launch_decode_t<KVT, 64>(p, mode, s) : launch_decode_t<KVT, 128>(p, mode, s);
}

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, int mode,
                         hipStream_t stream) {
  switch (kv_dtype) {
    case KV_F32: return launch_decode_d<KV_F32>(p, head_dim, mode, stream);
    case KV_F16: return launch_decode_d<KV_F16>(p, head_dim, mode, stream);
    case KV_BF16: return launch_decode_d<KV_BF16>(p, head_dim, mode, stream);
    case KV_E4M3: return launch_decode_d<KV_E4M3>(p, head_dim, mode, stream);
  }
  return hipErrorInvalidValue;
}

// The per-wave balanced schedule serves E4M3 caches (their tiles carry
// twice the arithmetic per byte, which two waves per SIMD hide and the
// per-compute-unit schedule's one wave per SIMD does not).
int stream_max_workers(int kv_dtype, int head_dim) {
  if (kv_dtype != KV_E4M3) return 0;
  const int grid = head_dim == 64 ? stream_grid<KV_E4M3, 64>() : stream_grid<KV_E4M3, 128>();
  return grid * kWaves;
}

hipError_t launch_stream(const DecodeParams& p, int kv_dtype, int head_dim, hipStream_t stream) {
  if (kv_dtype != KV_E4M3) return hipErrorInvalidValue;
  return head_dim == 64 ? launch_stream_t<KV_E4M3, 64>(p, stream) : launch_stream_t<KV_E4M3, 128>(p, stream);
}

// CU-balanced schedule: waves per workgroup (one workgroup per compute
// unit) and tiles per unit.  The accumulator slots take 4 x waves x
// (16 x D x 4 + 128) bytes of LDS: at D = 128 four waves (one per SIMD,
// up to 512 registers each) fill 133 KiB, at D = 64 eight waves 135 KiB.
// A unit's tiles are also the wave's ring (tiles in flight): six at D = 128
// (16-bit) measured ~1 us faster than four or eight on the ragged B = 128
// layer, level with five and ~0.5 us ahead of seven; f32 tiles are twice
// the size.
template <int KVT, int D>
constexpr int cu_waves() {
  return D == 128 ? 4 : 8;
}
template <int KVT, int D>
constexpr int cu_ring() {
  return KVT == KV_F32 ? (D == 64 ? 2 : 4) : (D == 128 ? 6 : 4);
}

int cu_stream_workers() {
  static std::atomic<int> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 16) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 16) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The grid is one workgroup per compute unit (the kernel's LDS, over half
// of a unit's 160 KiB, keeps a second one off every unit).
template <int KVT, int D>
static hipError_t launch_cu_stream_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int NW = cu_waves<KVT, D>();
  if (p.num_workers <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((paged_decode_cu_stream<KVT, D, NW, cu_ring<KVT, D>()>), dim3(static_cast<unsigned>(p.num_workers)),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_cu_stream(const DecodeParams& p, int kv_dtype, int head_dim, hipStream_t stream) {
  switch (kv_dtype) {
    case KV_F32: return head_dim == 64 ? launch_cu_stream_t<KV_F32, 64>(p, stream) : launch_cu_stream_t<KV_F32, 128>(p, stream);
    case KV_F16: return head_dim == 64 ? launch_cu_stream_t<KV_F16, 64>(p, stream) : launch_cu_stream_t<KV_F16, 128>(p, stream);
    case KV_BF16: return head_dim == 64 ? launch_cu_stream_t<KV_BF16, 64>(p, stream) : launch_cu_stream_t<KV_BF16, 128>(p, stream);
  }
  return hipErrorInvalidValue;   // E4M3 caches take the per-wave schedule
}

hipError_t launch_cu_merge(const ReduceParams& p, hipStream_t stream) {
  const int pairs = p.num_seqs * p.num_q_heads;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((pairs + 3) / 4), block(256);
  if (p.head_dim == 64) hipLaunchKernelGGL(cu_merge_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(cu_merge_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_stream_merge(const ReduceParams& p, hipStream_t stream) {
  const int pairs = p.num_seqs * p.num_q_heads;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((pairs + 3) / 4), block(256);
  if (p.head_dim == 64) hipLaunchKernelGGL(stream_merge_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(stream_merge_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

template <auto KERNEL>
static hipError_t launch_prefill_kernel(const DecodeParams& p, hipStream_t stream) {
  const int grid = std::max(kXcds, resident_workgroups<KERNEL>(kWaves * 64) / kXcds * kXcds);
  hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int KVT, int D, int MODE>
static hipError_t launch_prefill_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int kPf = ring_depth<KVT, D>();
  // Tiles in pairs (PV on the K = 32 form) for 16-bit caches when the
  // sequences average 16 or more query rows, where the step is bound by
  // the matrix cores and the softmax (chunked prefill, 137 rows per
  // sequence: 223 -> 202 us).  With a few rows per sequence it is bound by
  // memory, and the one-tile path keeps more loads in flight (speculative
  // verification, 4 rows: 71 us, 74 with pairs); with one row per sequence
  // it also rounds exactly as the decode kernels do.
  if constexpr (KVT == KV_F16 || KVT == KV_BF16) {
    if (static_cast<int64_t>(p.num_query_tokens) >= 16LL * p.num_seqs)
      return launch_prefill_kernel<paged_prefill_persistent<KVT, D, kWaves, MODE, kPf, kPacksPerWave, true>>(p,
                                                                                                           stream);
  }
  return launch_prefill_kernel<paged_prefill_persistent<KVT, D, kWaves, MODE, kPf, kPacksPerWave, false>>(p, stream);
}

template <int KVT>
static hipError_t launch_prefill_d(const DecodeParams& p, int head_dim, int mode, hipStream_t s) {
  if (head_dim == 64)
    return mode == MODE_FINAL ? launch_prefill_t<KVT, 64, MODE_FINAL>(p, s) : launch_prefill_t<KVT, 64, MODE_PARTIAL>(p, s);
  return mode == MODE_FINAL ? launch_prefill_t<KVT, 128, MODE_FINAL>(p, s) : launch_prefill_t<KVT, 128, MODE_PARTIAL>(p, s);
}

hipError_t launch_prefill(const DecodeParams& p, int kv_dtype, int head_dim, int mode, hipStream_t stream) {
  switch (kv_dtype) {
    case KV_F32: return launch_prefill_d<KV_F32>(p, head_dim, mode, stream);
    case KV_F16: return launch_prefill_d<KV_F16>(p, head_dim, mode, stream);
    case KV_BF16: return launch_prefill_d<KV_BF16>(p, head_dim, mode, stream);
    case KV_E4M3: return launch_prefill_d<KV_E4M3>(p, head_dim, mode, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_merge(const ReduceParams& p, hipStream_t stream) {
  const int64_t pairs = static_cast<int64_t>(p.num_query_tokens) * p.num_q_heads;
  if (pairs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4)), block(256);
  if (p.head_dim == 64) hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  const int pairs = p.num_seqs * p.num_q_heads;
  const dim3 grid((pairs + 3) / 4), block(256);
  if (p.head_dim == 64) hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
