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
  // the q operand holds the same dims of query head r.
  __device__ static void load_q(u32x4 (&qop)[NQ], const void* qrow, int g) {
    const uint16_t* q = static_cast<const uint16_t*>(qrow);
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = q ? ld16(q + 8 * (4 * m + g)) : u32x4{0, 0, 0, 0};
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
  __device__ static void load_q(u32x4 (&qop)[NQ], const void* qrow, int g) {
    const float* q = static_cast<const float*>(qrow);
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = q ? ld16(q + 4 * (4 * m + g)) : u32x4{0, 0, 0, 0};
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
  __device__ static void load_q(u32x4 (&qop)[NQ], const void* qrow, int g) {
    const uint16_t* q = static_cast<const uint16_t*>(qrow);
#pragma unroll
    for (int m = 0; m < NLOAD; ++m) {
      qop[2 * m] = q ? ld16(q + 16 * (4 * m + g)) : u32x4{0, 0, 0, 0};
      qop[2 * m + 1] = q ? ld16(q + 16 * (4 * m + g) + 8) : u32x4{0, 0, 0, 0};
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

// ----------------------------------------------------------------- kernel
template <int KVT, int D, int NW, bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(const DecodeParams p) {
  typedef TileOps<KVT, D> T;
  constexpr int E = ElemBytes<KVT>::value;
  constexpr int TILE = kBlockSize * D * E;  // bytes of one (block, kv head) tile
  constexpr int NL = T::NLOAD;
  constexpr int NT = T::NT;

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;   // lane group: tokens 4g..4g+3 of a block
  const int r = lane & 15;   // head column (outputs) / token or dim row (loads)
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = p.group;
  const int Hq = p.num_q_heads;

  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int blk0 = part * p.partition_blocks;

  if (!PARTIAL && L == 0) {  // empty context: zero output
    if (r < G) {
      const size_t row = (static_cast<size_t>(b) * Hq + h * G + r) * D;
      for (int n = wid; n < NT; n += NW) store4(p.out, row + 16 * n + 4 * g, p.out_dtype, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    return;
  }
  if (blk0 >= nblk) return;
  const int blk1 = min(nblk, blk0 + p.partition_blocks);

  // Query operand of this lane's head column (zero for columns >= G).
  const int qhead = h * G + r;
  const char* qrow = (r < G) ? static_cast<const char*>(p.q) +
                                   (static_cast<size_t>(b) * Hq + qhead) * D * (KVT == KV_F32 ? 4 : 2)
                             : nullptr;
  u32x4 qop[T::NQ];
  T::load_q(qop, qrow, g);

  // Blocks of this wave: blk0 + wid + NW * i, i < nmine.
  const int first = blk0 + wid;
  const int nmine = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;
  const int32_t* table = p.block_tables + static_cast<size_t>(b) * p.mbps;

  const size_t blk_stride = static_cast<size_t>(p.num_kv_heads) * TILE;
  const char* kbase = static_cast<const char*>(p.k_cache) + static_cast<size_t>(h) * TILE + lane * 16;
  const char* vbase = static_cast<const char*>(p.v_cache) + static_cast<size_t>(h) * TILE + lane * 16;
  auto load_tile = [&](u32x4 (&kt)[NL], u32x4 (&vt)[NL], int blk) {
    const char* kp = kbase + static_cast<size_t>(blk) * blk_stride;
    const char* vp = vbase + static_cast<size_t>(blk) * blk_stride;
#pragma unroll
    for (int m = 0; m < NL; ++m) kt[m] = ld16(kp + m * 1024);
#pragma unroll
    for (int m = 0; m < NL; ++m) vt[m] = ld16(vp + m * 1024);
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
    const float bm = max_over_groups(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pr[j] = fast_exp2(x[j] - m_new);
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
    for (int n = 0; n < NT; ++n) o[n] *= alpha;
    T::pv(o, vt, pr, pscale);
  };

  // Blocks go in chunks of up to 64: the chunk's physical ids are fetched
  // with one vector load (lane j: the chunk's j-th block) and read out with
  // readlane; inside a chunk the tile loads run one block ahead of the math.
  u32x4 kA[NL], vA[NL], kB[NL], vB[NL];
  for (int base = 0; base < nmine; base += 64) {
    const int cnt = min(64, nmine - base);
    const int ids = (lane < cnt) ? table[first + NW * (base + lane)] : 0;
    int bA = __builtin_amdgcn_readlane(ids, 0), bB = 0;
    load_tile(kA, vA, bA);
    int i = 0;
    for (; i + 1 < cnt; i += 2) {
      bB = __builtin_amdgcn_readlane(ids, i + 1);
      load_tile(kB, vB, bB);
      process(kA, vA, base + i, bA);
      if (i + 2 < cnt) {
        bA = __builtin_amdgcn_readlane(ids, i + 2);
        load_tile(kA, vA, bA);
      }
      process(kB, vB, base + i + 1, bB);
    }
    if (i < cnt) process(kA, vA, base + i, bA);
  }

  l_run = sum_over_groups(l_run);

  // ---- merge the NW waves' (max, sum, accumulator) and write
  float M, Lsum;
  float fw[NW];
  if constexpr (NW > 1) {
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    __shared__ f32x4 sm_o[NW][NT][64];
    if (g == 0) {
      sm_m[wid][r] = m_run;
      sm_l[wid][r] = l_run;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) sm_o[wid][n][lane] = o[n];
    __syncthreads();
    M = sm_m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
    Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      fw[w] = fast_exp2(sm_m[w][r] - M);
      Lsum += fw[w] * sm_l[w][r];
    }
    const float inv = 1.f / Lsum;
    for (int n = wid; n < NT; n += NW) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += fw[w] * sm_o[w][n][lane];
      acc *= inv;
      if (r < G) {
        if constexpr (PARTIAL) {
          const size_t row = ((static_cast<size_t>(b) * Hq + qhead) * p.num_partitions + part) * D;
          *reinterpret_cast<f32x4*>(p.tmp_out + row + 16 * n + 4 * g) = acc;
        } else {
          const size_t row = (static_cast<size_t>(b) * Hq + qhead) * D;
          store4(p.out, row + 16 * n + 4 * g, p.out_dtype, acc);
        }
      }
    }
  } else {
    M = m_run;
    Lsum = l_run;
    const float inv = 1.f / Lsum;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const f32x4 acc = o[n] * inv;
      if (r < G) {
        if constexpr (PARTIAL) {
          const size_t row = ((static_cast<size_t>(b) * Hq + qhead) * p.num_partitions + part) * D;
          *reinterpret_cast<f32x4*>(p.tmp_out + row + 16 * n + 4 * g) = acc;
        } else {
          const size_t row = (static_cast<size_t>(b) * Hq + qhead) * D;
          store4(p.out, row + 16 * n + 4 * g, p.out_dtype, acc);
        }
      }
    }
  }
  if constexpr (PARTIAL) {
    if (wid == 0 && g == 0 && r < G)
      p.tmp_lse[(static_cast<size_t>(b) * Hq + qhead) * p.num_partitions + part] =
          (M + fast_log2(Lsum)) * kLn2;
  }
}

// ----------------------------------------------------------------- reduce
// One wave per (sequence, query head): out = sum_p w_p o_p / sum_p w_p with
// w_p = exp(lse_p - max lse) over the sequence's non-empty partitions.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(const ReduceParams p) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= p.num_seqs * p.num_q_heads) return;
  const int b = pair / p.num_q_heads;
  const int L = max(0, min(p.context_lens[b], p.mbps * kBlockSize));
  const int n = min((L + p.partition_size - 1) / p.partition_size, p.num_partitions);
  const float* lse = p.tmp_lse + static_cast<size_t>(pair) * p.num_partitions;
  const float* o = p.tmp_out + static_cast<size_t>(pair) * p.num_partitions * D + lane * PER;

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  if (n > 0) {
    float M = -INFINITY;
    for (int s = lane; s < n; s += 64) M = fmaxf(M, lse[s]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float wsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float w = fast_exp2((lse[s] - M) * kLog2e);
      wsum += w;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += w * o[static_cast<size_t>(s) * D + k];
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= inv;
  }
  const size_t idx = static_cast<size_t>(pair) * D + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (p.out_dtype == KV_F32) static_cast<float*>(p.out)[idx + k] = acc[k];
    else if (p.out_dtype == KV_F16) static_cast<_Float16*>(p.out)[idx + k] = static_cast<_Float16>(acc[k]);
    else static_cast<__bf16*>(p.out)[idx + k] = static_cast<__bf16>(acc[k]);
  }
}

// --------------------------------------------------------------- launchers
constexpr int kWaves = 4;

template <int KVT, int D>
static hipError_t launch_decode_t(const DecodeParams& p, bool partial, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (partial) {
    const dim3 grid(p.num_partitions, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<KVT, D, kWaves, true>), grid, block, 0, stream, p);
  } else {
    const dim3 grid(1, p.num_kv_heads, p.num_seqs);
    hipLaunchKernelGGL((paged_decode_kernel<KVT, D, kWaves, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

template <int KVT>
static hipError_t launch_decode_d(const DecodeParams& p, int head_dim, bool partial, hipStream_t s) {
  return head_dim == 64 ? launch_decode_t<KVT, 64>(p, partial, s) : launch_decode_t<KVT, 128>(p, partial, s);
}

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, bool partial,
                         hipStream_t stream) {
  switch (kv_dtype) {
    case KV_F32: return launch_decode_d<KV_F32>(p, head_dim, partial, stream);
    case KV_F16: return launch_decode_d<KV_F16>(p, head_dim, partial, stream);
    case KV_BF16: return launch_decode_d<KV_BF16>(p, head_dim, partial, stream);
    case KV_E4M3: return launch_decode_d<KV_E4M3>(p, head_dim, partial, stream);
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
