// kv_write.hip - moving new K/V into the paged pool (gfx950).
//
//  * kv_write_kernel: the step's new tokens, bit-exact, into their slots
//    ("rvLLM: High-performance LLM inference in Rust", section "CUDA
//    Kernels", row "Reshape and Cache"; "rvllm - A Small LLM Inference Engine
//    in Rust", section "How it's put together": explicit write positions).
//  * quantize_e4m3_kernel: whole blocks of fp32 K/V into E4M3 codes with one
//    fp32 scale per (block, kv head) ("LLM Serving Kernels", section
//    "Projects", row 05: E4M3 storage, page scales; "rvLLM: ...", "CUDA
//    Kernels", row "FP8 KV Cache": per-head scaling).
//
//  * append_e4m3_kernel: new tokens quantised into an E4M3 pool one at a
//    time, growing the block's scale (and re-encoding its earlier codes)
//    when a token exceeds it, so the scale stays fp32(amax / 448) over the
//    block's tokens.
//  * copy_blocks_kernel: whole blocks copied inside the pool, for
//    copy-on-write forks ("rvLLM: ...", "CUDA Kernels", row "Block Copy":
//    KV cache block copy for beam search; section "Architecture": the block
//    manager's copy-on-write).
//
// All are pure data movement plus index arithmetic; the tile layouts are
// the ones documented in pagedkv.h.
#include "pkv_common.h"
#include "pkv_launch.h"

namespace pkv {

// One thread per (token, kv head, 16-byte chunk of that head's D elements).
// K: the chunk is also a contiguous 16 bytes of the K tile (chunk c of token
// `off` sits at byte (c*16 + off)*16).  V: its elements scatter to their
// V-tile positions.
template <int E>
__global__ __launch_bounds__(256) void kv_write_kernel(const WriteParams p) {
  typedef typename std::conditional<E == 4, uint32_t, uint16_t>::type Elem;
  constexpr int X = 16 / E;   // elements per chunk
  constexpr int N = 4 / E;
  const int chunks = p.head_dim / X;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = p.num_tokens * p.num_kv_heads * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;
  const int h = static_cast<int>(th % p.num_kv_heads);
  const int64_t t = th / p.num_kv_heads;
  // The token's K and V do not depend on its slot: their loads go out
  // together with the slot's, so the launch waits for one round trip.
  const size_t row_bytes = static_cast<size_t>(p.head_dim) * E;
  const size_t src = (static_cast<size_t>(t) * p.num_kv_heads + h) * row_bytes + c * 16;
  const u32x4 kv = ld16(static_cast<const char*>(p.k) + src);
  const u32x4 vv = ld16(static_cast<const char*>(p.v) + src);
  asm volatile("" ::: "memory");   // keeps the loads above the slot test (no wait is implied)
  const int64_t slot = p.slots[t];
  if (slot < 0 || slot >= static_cast<int64_t>(p.num_blocks) * kBlockSize) return;
  const int64_t blk = slot / kBlockSize;
  const int off = static_cast<int>(slot % kBlockSize);
  const size_t tile = (static_cast<size_t>(blk) * p.num_kv_heads + h) * kBlockSize * row_bytes;

  st16(static_cast<char*>(p.k_cache) + tile + (static_cast<size_t>(c) * kBlockSize + off) * 16, kv);

  Elem vals[X];
  __builtin_memcpy(vals, &vv, 16);
  Elem* vt = reinterpret_cast<Elem*>(static_cast<char*>(p.v_cache) + tile);
#pragma unroll
  for (int i = 0; i < X; ++i) vt[v_tile_elem(off, c * X + i, N)] = vals[i];
}

// One wave per (block, kv head, K or V) tile; a workgroup takes four
// consecutive tiles, ordered (block, K or V, kv head), so the kv heads of a
// block sit side by side and the workgroup's loads cover whole source rows.
// Each lane loads 16 bytes (4 consecutive dims of one token) at a time, the
// wave takes the tile's amax, and the codes go into an LDS image of the tile
// in its cache layout, which the wave then stores with 16-byte writes.
// scale = fp32(amax / 448) over the block's valid slots (1 if amax is 0);
// code = nearest-even E4M3 of clamp(fp32(x / scale), -448, 448); slots at or
// past valid_tokens get code 0.
//
// The quotient is formed as fp32((double)x * (1 / (double)scale)), which
// equals the correctly rounded fp32 x / scale wherever that is a normal
// number: the double product is within 2^-52 (relative) of x / scale, while
// a quotient of two 24-bit numbers lies either on an fp32 value or at least
// ~2^-49 (relative) away from the nearest rounding midpoint (it is never on
// one: x = scale * midpoint would need the midpoint's 25-bit odd
// significand).  Below 2^-126 the two may differ, but every such value
// encodes as a zero code of the same sign either way.  gfx950's
// v_cvt_pk_fp8_f32 then rounds two clamped quotients to OCP E4M3 codes,
// ties to even.  Source reads and code writes stream (non-temporal): each
// byte is touched once.
template <int D>
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const QuantParams p) {
  constexpr int TB = kBlockSize * D;         // bytes of codes in one tile
  constexpr int NJ = kBlockSize * D / 256;   // 16-byte loads per lane
  constexpr int C4 = D / 4;                  // 16-byte pieces per source row
  __shared__ __align__(16) unsigned char img[4][TB];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // tile indices stay scalar
  const uint32_t Hkv = static_cast<uint32_t>(p.num_kv_heads);
  const uint64_t ntiles = static_cast<uint64_t>(p.num_src_blocks) * Hkv * 2;
  const uint64_t tile = static_cast<uint64_t>(blockIdx.x) * 4 + wid;
  if (tile >= ntiles) return;   // wave-uniform; no workgroup barrier follows
  uint32_t pair;                // block * 2 + (V ? 1 : 0)
  if (ntiles <= 0xFFFFFFFFull) pair = static_cast<uint32_t>(tile) / Hkv;
  else pair = static_cast<uint32_t>(tile / Hkv);
  pair = __builtin_amdgcn_readfirstlane(pair);   // the division runs on the VALU
  const int h = static_cast<int>(tile - static_cast<uint64_t>(pair) * Hkv);
  const bool is_v = (pair & 1u) != 0;
  const int i = static_cast<int>(pair >> 1);
  const int valid = __builtin_amdgcn_readfirstlane(max(0, min(p.valid_tokens[i], kBlockSize)));
  // Head h's rows of the block: row t at t * Hkv * D floats.  The descriptor
  // ends after row valid - 1, so the rows past it read as zeros.
  const float* src = (is_v ? p.v_src : p.k_src) + (static_cast<size_t>(i) * kBlockSize * Hkv + h) * D;
  const auto rsrc = make_tile_rsrc(src, valid > 0 ? ((valid - 1) * static_cast<int>(Hkv) + 1) * D * 4 : 0);
  u32x4 x[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 64 + lane;
    x[j] = buffer_ld16_policy<kStreamLoad>(rsrc, static_cast<uint32_t>((e / C4) * static_cast<int>(Hkv) * D * 4 + (e % C4) * 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) amax = fmaxf(amax, fabsf(__uint_as_float(x[j][k])));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  const double inv = 1.0 / static_cast<double>(scale);
  unsigned char* im = img[wid];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 64 + lane;
    const int t = e / C4;
    const int d = 4 * (e % C4);
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      y[k] = fminf(fmaxf(static_cast<float>(static_cast<double>(__uint_as_float(x[j][k])) * inv), -448.0f), 448.0f);
    // Slots past valid_tokens loaded as +0 and so encode as code 0.
    uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false));
    w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], static_cast<int>(w), true));
    if (!is_v) {   // K: dims d..d+3 of token t are 4 consecutive bytes of one 16-byte chunk
      *reinterpret_cast<uint32_t*>(&im[((d / 16) * kBlockSize + t) * 16 + d % 16]) = w;
    } else {       // V: each dim lands in its own chunk (tokens are the fast index there)
#pragma unroll
      for (int k = 0; k < 4; ++k) im[v_tile_elem(t, d + k, 4)] = static_cast<unsigned char>(w >> (8 * k));
    }
  }
  // The wave reads back only the image it wrote: LDS operations of one wave
  // complete in order, so a wave-level scheduling barrier is enough.
  __builtin_amdgcn_wave_barrier();
  const int blk = p.block_ids[i];
  char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + (static_cast<size_t>(blk) * Hkv + h) * TB;
#pragma unroll
  for (int off = lane * 16; off < TB; off += 1024)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&im[off]), reinterpret_cast<u32x4*>(dst + off));
  if (lane == 0) p.kv_scales[((is_v ? static_cast<size_t>(p.num_blocks) : 0) + blk) * Hkv + h] = scale;
}

// One workgroup (D threads) per (token, kv head, K-or-V); thread d owns dim
// d of every slot of the block.  Each rounding step is fp32: token scale
// s = amax / 448.  When every earlier code of the block is a zero (always so
// for its first token), the token sets the scale (1 if s is 0): the block's
// tokens so far have amax 0, and the scale follows the bulk quantiser's
// rule.  Otherwise a token with s above the stored scale re-encodes the
// earlier slots as code(clamp(decode(c) * old / s)) and stores s.  The
// token's own code is code(clamp(x / scale)).  At most one token per block
// per launch.
__global__ __launch_bounds__(128) void append_e4m3_kernel(const AppendParams p) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int d = threadIdx.x;
  const int D = p.head_dim;
  const float x = (is_v ? p.v : p.k)[(static_cast<size_t>(t) * p.num_kv_heads + h) * D + d];   // before the slot: one round trip
  const int64_t slot = p.slots[t];
  if (slot < 0 || slot >= static_cast<int64_t>(p.num_blocks) * kBlockSize) return;   // whole workgroup
  const int64_t blk = slot / kBlockSize;
  const int off = static_cast<int>(slot % kBlockSize);

  float amax = fabsf(x);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float sm[2];
  if ((d & 63) == 0) sm[d >> 6] = amax;
  __syncthreads();
  amax = sm[0];
  if (D > 64) amax = fmaxf(amax, sm[1]);
  const float s_tok = amax / 448.0f;

  uint8_t* tile = static_cast<uint8_t*>(is_v ? p.v_cache : p.k_cache) +
                  (static_cast<size_t>(blk) * p.num_kv_heads + h) * kBlockSize * D;
  auto pos = [&](int tt) -> int {   // byte of (slot tt, dim d) in the tile
    return is_v ? v_tile_elem(tt, d, 4) : ((d / 16) * kBlockSize + tt) * 16 + d % 16;
  };
  float* sc = p.kv_scales + (is_v ? static_cast<size_t>(p.num_blocks) * p.num_kv_heads : 0) +
              static_cast<size_t>(blk) * p.num_kv_heads + h;
  // Any non-zero code (magnitude bits) among this dim's earlier slots.
  uint32_t nz = 0;
  for (int o = 0; o < off; ++o) nz |= tile[pos(o)] & 0x7Fu;
  const bool earlier_zero = __syncthreads_or(static_cast<int>(nz)) == 0;
  float s;
  if (earlier_zero) {
    s = s_tok > 0.f ? s_tok : 1.0f;
  } else {
    const float s_old = *sc;
    s = s_old;
    if (s_tok > s_old) {
      for (int o = 0; o < off; ++o) {
        const uint8_t c = tile[pos(o)];
        const float v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false)[0] * s_old;
        tile[pos(o)] = static_cast<uint8_t>(f32_to_e4m3(fminf(fmaxf(v / s_tok, -448.0f), 448.0f)));
      }
      s = s_tok;
    }
  }
  tile[pos(off)] = static_cast<uint8_t>(f32_to_e4m3(fminf(fmaxf(x / s, -448.0f), 448.0f)));
  __syncthreads();   // every thread has read the old scale
  if (d == 0) *sc = s;
}

hipError_t launch_append_e4m3(const AppendParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.num_tokens), p.num_kv_heads, 2), block(p.head_dim);
  hipLaunchKernelGGL(append_e4m3_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

// A block's Hkv tiles are one contiguous run of 16-byte chunks; grid
// (chunks / 1024, pairs, K-or-V), four chunks per thread.  Pairs naming a block
// outside the pool are skipped.  The first threads of each (pair, K-or-V)
// (blockIdx.x = 0) also copy that block's Hkv scales of an E4M3 pool.
__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyParams p) {
  const int pair = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int src = p.block_mapping[2 * pair];
  const int dst = p.block_mapping[2 * pair + 1];
  if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) return;
  char* cache = static_cast<char*>(is_v ? p.v_cache : p.k_cache);
  const u32x4* from = reinterpret_cast<const u32x4*>(cache + static_cast<size_t>(src) * p.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(cache + static_cast<size_t>(dst) * p.block_bytes);
  // Each thread moves chunks c0, c0 + 256, c0 + 512, c0 + 768 of this
  // workgroup's 1024-chunk span: all four loads issue before the stores.
  // Both sides stream (non-temporal): the copy touches each byte once.
  const int64_t nchunks = p.block_bytes / 16;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x;
  u32x4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (c0 + 256 * u < nchunks) x[u] = __builtin_nontemporal_load(from + c0 + 256 * u);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (c0 + 256 * u < nchunks) __builtin_nontemporal_store(x[u], to + c0 + 256 * u);
  if (p.kv_scales != nullptr && blockIdx.x == 0) {
    float* sc = p.kv_scales + (is_v ? static_cast<size_t>(p.num_blocks) * p.num_kv_heads : 0);
    for (int h = threadIdx.x; h < p.num_kv_heads; h += 256)
      sc[static_cast<size_t>(dst) * p.num_kv_heads + h] = sc[static_cast<size_t>(src) * p.num_kv_heads + h];
  }
}

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const int64_t chunks = p.block_bytes / 16;
  const dim3 grid(static_cast<unsigned>((chunks + 1023) / 1024), static_cast<unsigned>(p.num_pairs), 2), block(256);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_write(const WriteParams& p, hipStream_t stream) {
  const int64_t chunks = p.head_dim * p.elem_bytes / 16;
  const int64_t total = p.num_tokens * p.num_kv_heads * chunks;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256)), block(256);
  if (p.elem_bytes == 4) hipLaunchKernelGGL(kv_write_kernel<4>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(kv_write_kernel<2>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const QuantParams& p, hipStream_t stream) {
  if (p.num_src_blocks == 0) return hipSuccess;
  const int64_t tiles = static_cast<int64_t>(p.num_src_blocks) * p.num_kv_heads * 2;
  const dim3 grid(static_cast<unsigned>((tiles + 3) / 4)), block(256);
  if (p.head_dim == 128) hipLaunchKernelGGL(quantize_e4m3_kernel<128>, grid, block, 0, stream, p);
  else if (p.head_dim == 64) hipLaunchKernelGGL(quantize_e4m3_kernel<64>, grid, block, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
