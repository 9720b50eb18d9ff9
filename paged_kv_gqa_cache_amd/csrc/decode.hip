// decode.hip - paged grouped-query decode attention for gfx950.
//
// What it computes: for sequence b and query head i (KV head h = i / G),
// softmax(q . K^T * scale) V over the first L_b tokens of the sequence,
// gathered from the block pool through its block table, with online softmax
// ("rvLLM: High-performance LLM inference in Rust", section "CUDA Kernels",
// row "PagedAttention V2"; "LLM Serving Kernels", section "Projects", row 04:
// page tables, GQA/MQA, online softmax).  In split mode each partition of
// the context yields a normalised partial output and its log-sum-exp; the
// reduce kernel merges them (flash-decoding).
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
//    two MFMAs), so only V's own rounding is in the product.
//  * E4M3 codes decode to fp16 with shifts/masks (value * 2^-8); the K scale
//    and 2^8 fold into the block's logit factor, the V scale into P.
//  * Softmax runs in base 2 (log2 e folded into the scale).
#include "pkv_common.h"
#include "pkv_launch.h"

#include <algorithm>

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
  __device__ static void pv(f32x4 (&o)[NT], const u32x4 (&vt)[NLOAD], const float (&p)[4], float) {
    V4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const S h = static_cast<S>(p[j]);
      hi[j] = h;
      lo[j] = static_cast<S>(p[j] - static_cast<float>(h));
    }
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

// E4M3 KV with f16 queries: codes decode to f16 (value * 2^-8) for f16 MFMA.
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
      e4m3x16_to_f16x8x2_scaled(kt[m], lo, hi);
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
  // pscale = V scale * 2^8 folds the block's V scale into P.
  __device__ static void pv(f32x4 (&o)[NT], const u32x4 (&vt)[NLOAD], const float (&p)[4], float pscale) {
    f16x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ps = p[j] * pscale;
      const _Float16 h = static_cast<_Float16>(ps);
      hi[j] = h;
      lo[j] = static_cast<_Float16>(ps - static_cast<float>(h));
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mma_k16(e4m3x4_to_f16x4_scaled(vt[n >> 2][n & 3]), hi, o[n]);
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] = mma_k16(e4m3x4_to_f16x4_scaled(vt[n >> 2][n & 3]), lo, o[n]);
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
// One wave merges one (sequence, query head)'s n partitions:
// out = sum_p w_p o_p / sum_p w_p with w_p = exp(lse_p - max lse).  Lane s
// holds partition s's weight (64 partitions per pass); partial rows are
// fetched eight at a time so their loads overlap.  Returns this lane's D/64
// output dims (lane * D/64 + k).
template <int D, bool COH>
__device__ __forceinline__ void merge_partitions(const float* lse, const float* o_row0, int n, int lane,
                                                 float (&acc)[D / 64]) {
  constexpr int PER = D / 64;
  constexpr int BATCH = 8;
  // COH: the partials were written by other workgroups in this launch, so
  // they are read with device-scope (sc1) loads, which do not hit stale L2
  // lines of this XCD.
  const auto lse_r = make_tile_rsrc(lse, n * 4);
  const auto o_r = make_tile_rsrc(o_row0, n * D * 4);
  auto ld_lse = [&](int s) -> float {
    if constexpr (COH) return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lse_r, s * 4, 0, kDeviceScope));
    else return lse[s];
  };
  auto ld_o = [&](int s, int k) -> float {
    if constexpr (COH)
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(o_r, (s * D + lane * PER + k) * 4, 0, kDeviceScope));
    else return o_row0[static_cast<size_t>(s) * D + lane * PER + k];
  };
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float M = -INFINITY;
  for (int c = 0; c < n; c += 64) M = fmaxf(M, (c + lane < n) ? ld_lse(c + lane) : -INFINITY);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float wsum = 0.f;
  for (int c = 0; c < n; c += 64) {
    const float w = (c + lane < n) ? fast_exp2((ld_lse(c + lane) - M) * kLog2e) : 0.f;
    wsum += w;
    const int cnt = min(64, n - c);
    for (int j = 0; j < cnt; j += BATCH) {
      float v[BATCH][PER];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (j + u < cnt) {
#pragma unroll
          for (int k = 0; k < PER; ++k) v[u][k] = ld_o(c + j + u, k);
        }
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (j + u < cnt) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
#pragma unroll
          for (int k = 0; k < PER; ++k) acc[k] += wu * v[u][k];
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off);
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

// Workgroup-shared state of one work item: the NW waves' softmax states for
// the cross-wave merge, and the merge ticket of the split mode.
template <int NW, int NT>
struct ItemShared {
  float m[NW][16];
  float l[NW][16];
  f32x4 o[NW][NT][64];
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

template <int KVT, int D, int NW>
__device__ __forceinline__ void item_prefetch(const DecodeParams& p, int b, int h, int part,
                                              ItemPrefetch<KVT, D>& pf) {
  // Buffer loads bounded by the table row / the group's q rows: lanes past
  // the end read 0 without a branch, so no load here is conditional (a
  // conditional load would make the compiler drain every outstanding load
  // at the next wait).
  constexpr int QB = (KVT == KV_F32) ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const auto tr = make_tile_rsrc(p.block_tables + static_cast<size_t>(b) * p.mbps, p.mbps * 4);
  const int id0 = part * p.partition_blocks + wid + NW * lane;
  pf.ids = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(tr, static_cast<uint32_t>(id0) * 4u, 0, 0));
  const auto qr = make_tile_rsrc(static_cast<const char*>(p.q) +
                                     (static_cast<size_t>(b) * p.num_q_heads + h * p.group) * D * QB,
                                 p.group * D * QB);
  TileOps<KVT, D>::load_q(pf.qop, qr, static_cast<uint32_t>(r * D * QB), lane >> 4);
}

// One work item: sequence b (context length L), kv head h, partition `part`.
template <int KVT, int D, int NW, int MODE, int PF>
__device__ __forceinline__ void decode_item(const DecodeParams& p, int b, int h, int part, int L,
                                            const ItemPrefetch<KVT, D>& pf,
                                            ItemShared<NW, D / 16>& sm) {
  typedef TileOps<KVT, D> T;
  constexpr int E = ElemBytes<KVT>::value;
  constexpr int TILE = kBlockSize * D * E;  // bytes of one (block, kv head) tile
  constexpr int NL = T::NLOAD;
  constexpr int NT = T::NT;

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a block
  const int r = lane & 15;   // head column (outputs) / token or dim row (loads)
  const int G = p.group;
  const int Hq = p.num_q_heads;

  const int32_t* table = p.block_tables + static_cast<size_t>(b) * p.mbps;
  const int blk0 = part * p.partition_blocks;
  const int first = blk0 + wid;
  int ids = pf.ids;
  const int qhead = h * G + r;
#define qop pf.qop
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int nparts = (nblk + p.partition_blocks - 1) / p.partition_blocks;

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

  // Blocks of this wave: first + NW * i, i < nmine.
  const int nmine = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;

  // Tile loads are buffer loads: each tile's descriptor (base = the tile,
  // size = TILE bytes) lives in scalar registers and every lane adds one
  // 32-bit offset, so no per-tile 64-bit vector addresses are needed.
  uint32_t lane_off[NL];
#pragma unroll
  for (int m = 0; m < NL; ++m) lane_off[m] = static_cast<uint32_t>(lane) * 16u + m * 1024u;
  const char* kcache = static_cast<const char*>(p.k_cache);
  const char* vcache = static_cast<const char*>(p.v_cache);
  // A load past the wave's last block still issues, through a zero-size
  // descriptor (reads 0, no memory traffic), so the loop has no
  // conditional loads and each wait covers exactly the tile it needs.
  auto load_tile = [&](u32x4 (&kt)[NL], u32x4 (&vt)[NL], int blk, bool valid) {
    const size_t tile = (static_cast<size_t>(blk) * p.num_kv_heads + h) * TILE;
    const auto kr = make_tile_rsrc(kcache + tile, valid ? TILE : 0);
    const auto vr = make_tile_rsrc(vcache + tile, valid ? TILE : 0);
#pragma unroll
    for (int m = 0; m < NL; ++m) kt[m] = buffer_ld16(kr, lane_off[m]);
#pragma unroll
    for (int m = 0; m < NL; ++m) vt[m] = buffer_ld16(vr, lane_off[m]);
  };

  float m_run = -INFINITY;  // running max (base-2 logits) of head r
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const u32x4 (&kt)[NL], u32x4 (&vt)[NL], int i, int blk) {
    const int tok0 = (first + NW * i) * kBlockSize;
    const f32x4 s = T::qk(kt, qop);
    float f = p.qk_scale_log2;
    float pscale = 1.f;
    if constexpr (KVT == KV_E4M3) {
      f *= 256.f * p.kv_scales[static_cast<size_t>(blk) * p.num_kv_heads + h];
      pscale = 256.f * p.kv_scales[(static_cast<size_t>(p.num_blocks) + blk) * p.num_kv_heads + h];
    }
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = s[j] * f;
    if (tok0 + kBlockSize > L) {  // the sequence's last, partly filled block
      const int nv = L - tok0 - 4 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = (j < nv) ? x[j] : -INFINITY;
      T::mask_v(vt, nv);
    }
    // Lazy rescaling: the reference max m_run only moves when some head's
    // block max exceeds it by more than kSlack (log2 units), so exp2(x - m_run)
    // stays below 2^kSlack and the accumulators are rescaled about once per
    // partition instead of every block.  The first block always moves it.
    const float bm = max_over_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    if (__any(bm > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, bm);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    T::pv(o, vt, pr, pscale);
  };

  // Blocks go in chunks of up to 64: the chunk's physical ids arrive in one
  // vector load (lane j: the chunk's j-th block) and are read out with
  // readlane.  Tiles stream through a ring of PF register buffers: before
  // block j is processed, the loads of block j + PF - 1 are issued, so PF - 1
  // tiles are in flight while the matrix cores work on one.
  u32x4 kb[PF][NL], vb[PF][NL];
  int bid[PF];
  for (int base = 0; base < nmine; base += 64) {
    const int cnt = min(64, nmine - base);
    if (base > 0) ids = (lane < cnt) ? table[first + NW * (base + lane)] : 0;
#pragma unroll
    for (int s = 0; s < PF - 1; ++s) {
      bid[s] = __builtin_amdgcn_readlane(ids, min(s, cnt - 1));
      load_tile(kb[s], vb[s], bid[s], s < cnt);
    }
    for (int i = 0; i < cnt; i += PF) {
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        const int j = i + s;
        const int nxt = j + PF - 1;
        const int slot = (s + PF - 1) % PF;
        bid[slot] = __builtin_amdgcn_readlane(ids, min(nxt, cnt - 1));
        load_tile(kb[slot], vb[slot], bid[slot], nxt < cnt);
        if (j < cnt) process(kb[s], vb[s], base + j, bid[s]);
      }
    }
  }

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
  if constexpr (NW > 1) {
    if (g == 0) {
      sm.m[wid][r] = m_run;
      sm.l[wid][r] = l_run;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) sm.o[wid][n][lane] = o[n];
    __syncthreads();
    float fw[NW];
    M = sm.m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm.m[w][r]);
    Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      fw[w] = fast_exp2(sm.m[w][r] - M);
      Lsum += fw[w] * sm.l[w][r];
    }
    const float inv = 1.f / Lsum;
    for (int n = wid; n < NT; n += NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += fw[w] * sm.o[w][n][lane];
      emit(n, acc * inv);
    }
  } else {
    M = m_run;
    Lsum = l_run;
    const float inv = 1.f / Lsum;
#pragma unroll
    for (int n = 0; n < NT; ++n) emit(n, o[n] * inv);
  }
  if (direct) return;
  const float lse = (M + fast_log2(Lsum)) * kLn2;
  if constexpr (MODE == MODE_SPLIT) {
    if (wid == 0 && g == 0 && r < G)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), make_tile_rsrc(p.tmp_lse + part_row, 4), 0, 0,
                                            kDeviceScope);
    // Count this partition once all its waves' partial stores are complete
    // at device scope; the workgroup that takes the last ticket merges.
    // No cache maintenance is needed: the partials are written and read
    // with device-scope accesses, and the counter is a device atomic.
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

#undef qop

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
  ItemPrefetch<KVT, D> pf;
  item_prefetch<KVT, D, NW>(p, b, h, part, pf);
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  decode_item<KVT, D, NW, MODE, PF>(p, b, h, part, L, pf, sm);
}

// Persistent form: as many workgroups as fit on the GPU at once.  Each one
// first counts the non-empty work items of every sequence (an exclusive
// prefix sum in LDS), then walks item n = blockIdx.x, + gridDim.x, ... in
// sequence-major order, mapping n back to (sequence, kv head, partition) by
// binary search.  No workgroup is launched for an empty partition.
constexpr int kMaxSeqsPersistent = 2048;
constexpr int kXcds = 8;   // accelerator complex dies of an MI355X

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
      const int nb = (L + kBlockSize - 1) / kBlockSize;
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
  // Item n -> (sequence, kv head, partition): last b with s_cum[b] <= n.
  auto locate = [&](int n, int& b, int& h, int& part) {
    int lo_b = 0, hi_b = B;
    while (hi_b - lo_b > 1) {
      const int mid = (lo_b + hi_b) >> 1;
      if (s_cum[mid] <= n) lo_b = mid;
      else hi_b = mid;
    }
    b = lo_b;
    const int local = n - s_cum[b];
    h = local / s_np[b];
    part = local % s_np[b];
  };
  ItemPrefetch<KVT, D> cur, nxt;
  int b, h, part, b2, h2, part2;

  int n = lo + static_cast<int>(blockIdx.x) / kXcds;
  if (n >= hi) return;
  locate(n, b, h, part);
  item_prefetch<KVT, D, NW>(p, b, h, part, cur);
  while (true) {
    // The next item's ids and q load while this item streams (the last item
    // prefetches itself again, so the load is never conditional).
    const int n2 = n + per_xcd;
    locate(min(n2, hi - 1), b2, h2, part2);
    item_prefetch<KVT, D, NW>(p, b2, h2, part2, nxt);
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

// ----------------------------------------------------------------- reduce
// One wave per (sequence, query head) merges its non-empty partitions.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= p.num_seqs * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  const int n = min((L + p.partition_size - 1) / p.partition_size, p.num_partitions);
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

// Workgroups of `kernel` that fit on the current device at once (compute
// units x resident workgroups per unit); queried once per kernel and device.
template <typename K>
static int resident_workgroups(K kernel, int block) {
  static int cached[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 16 && cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu <= 0) per_cu = 1;
  const int n = cus * per_cu;
  if (dev < 16) cached[dev] = n;
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
    int64_t grid = std::min<int64_t>(items, resident_workgroups(kernel, block));
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
  // Register budget: a K+V tile pair takes D*e/8 VGPRs per lane; keep the
  // ring within what two waves per SIMD allow (f32 with D = 128: two tiles).
  constexpr int kPf = (ElemBytes<KVT>::value * D >= 512) ? 2 : kPrefetch;
  if (mode == MODE_FINAL) p.num_partitions = 1;
  if (mode == MODE_PARTIAL) return launch_mode<KVT, D, MODE_PARTIAL, kPf>(p, stream);
  if (mode == MODE_SPLIT) return launch_mode<KVT, D, MODE_SPLIT, kPf>(p, stream);
  return launch_mode<KVT, D, MODE_FINAL, kPf>(p, stream);
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

hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream) {
  const int pairs = p.num_seqs * p.num_q_heads;
  const dim3 grid((pairs + 3) / 4), block(256);
  if (p.head_dim == 64) hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
