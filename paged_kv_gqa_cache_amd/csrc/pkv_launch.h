// pkv_launch.h - kernel parameter blocks and launchers (internal to libpagedkv.so).
//
// The launchers assume arguments already validated by the C ABI layer
// (abi.hip): sizes positive, supported dtypes, head_dim / group size in
// range, partition size a multiple of 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Sequences whose per-sequence tables fit in a persistent workgroup's LDS.
// The decode kernels fall back to one workgroup per item above it; the
// balanced schedule and the multi-token step reject larger batches.
constexpr int kMaxSeqsPersistent = 2048;

struct DecodeParams {
  const void* q;               // [B][Hq][D]
  const void* k_cache;         // [NB][Hkv][tile]
  const void* v_cache;
  const int32_t* block_tables; // [B][MBPS]
  const int32_t* context_lens; // [B]
  const float* kv_scales;      // [2][NB][Hkv] (e4m3 only)
  void* out;                   // [B][Hq][D] (final mode)
  float* tmp_out;              // [B][Hq][S][D] (partial mode)
  float* tmp_lse;              // [B][Hq][S]
  float qk_scale_log2;         // scale * log2(e)
  int32_t num_seqs, num_q_heads, num_kv_heads, group, num_blocks, mbps;
  int32_t partition_blocks;    // blocks per partition (final mode: covers MBPS)
  int32_t num_partitions;      // S
  int32_t out_dtype;
  int32_t* counters;           // [B][Hkv] split mode: partitions finished (zero between calls)
  // Balanced schedule: tmp_out is [G][num_slots][D], tmp_lse [G][num_slots].
  int32_t* seq_tiles;          // [B + 1] tiles before each sequence (written by the kernel)
  int32_t num_workers;         // waves of the resident grid
  int32_t num_slots;           // B * Hkv + num_workers
  int32_t window;              // sliding window in tokens (0: whole context)
  // Multi-token step: q and out are [num_query_tokens][Hq][D], partials
  // [num_query_tokens][Hq][S][D]; sequence b owns rows query_start[b] ..
  const int32_t* query_start;  // [B + 1]
  int32_t num_query_tokens;
  int32_t tokens_per_pack;     // 16 / G
  // Fused decode step (null: none): sequence b's new token, K and V rows
  // [B][Hkv][D] in the cache dtype, written at position L_b - 1 by the work
  // item that reads that block, before it reads it.
  const void* k_new;
  const void* v_new;
};

struct ReduceParams {
  const float* tmp_out;
  const float* tmp_lse;
  const int32_t* context_lens;
  void* out;
  int32_t num_seqs, num_q_heads, head_dim, mbps, partition_size, num_partitions, out_dtype;
  // Balanced schedule only.
  const int32_t* seq_tiles;
  int32_t num_kv_heads, num_workers, num_slots;
  int32_t window;              // sliding window in tokens (0: whole context)
  // Multi-token step only.
  const int32_t* query_start;
  int32_t num_query_tokens;
};

struct WriteParams {
  const void* k;
  const void* v;
  const int64_t* slots;
  void* k_cache;
  void* v_cache;
  int64_t num_tokens;
  int32_t num_kv_heads, head_dim, num_blocks, elem_bytes;
};

struct QuantParams {
  const float* k_src;           // [n][16][Hkv][D]
  const float* v_src;
  const int32_t* block_ids;     // [n]
  const int32_t* valid_tokens;  // [n]
  void* k_cache;
  void* v_cache;
  float* kv_scales;             // [2][NB][Hkv]
  int32_t num_src_blocks, num_kv_heads, head_dim, num_blocks;
};

struct AppendParams {
  const float* k;               // [num_tokens][Hkv][D]
  const float* v;
  const int64_t* slots;         // [num_tokens]; negative skips
  void* k_cache;                // e4m3 pool
  void* v_cache;
  float* kv_scales;             // [2][NB][Hkv]
  int64_t num_tokens;
  int32_t num_kv_heads, head_dim, num_blocks;
};

struct CopyParams {
  const int32_t* block_mapping;  // [num_pairs][2]: (src, dst)
  void* k_cache;
  void* v_cache;
  float* kv_scales;              // [2][NB][Hkv] for an e4m3 pool, else null
  int64_t block_bytes;           // Hkv * 16 * D * elem bytes (a multiple of 16)
  int32_t num_pairs, num_blocks, num_kv_heads;
};

// Each returns hipSuccess or the launch error.
// mode: 0 one pass to out, 1 partials to the workspace, 2 partials merged
// in-kernel by the last partition of each (sequence, kv head).
hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, int mode,
                         hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t stream);
// Balanced schedule: worker count of the resident grid on the current
// device, the tile-stream kernel, and the merge of split items.
int stream_max_workers(int kv_dtype, int head_dim);
hipError_t launch_stream(const DecodeParams& p, int kv_dtype, int head_dim, hipStream_t stream);
hipError_t launch_stream_merge(const ReduceParams& p, hipStream_t stream);
// CU-balanced schedule: one workgroup per compute unit (cu_stream_workers()
// of them on the current device), equal tile shares per unit; items split
// between units are merged by launch_stream_merge.
int cu_stream_workers();
hipError_t launch_cu_stream(const DecodeParams& p, int kv_dtype, int head_dim, hipStream_t stream);
hipError_t launch_cu_merge(const ReduceParams& p, hipStream_t stream);
// Multi-token step: mode 0 one pass to out, 1 partials; then the merge.
hipError_t launch_prefill(const DecodeParams& p, int kv_dtype, int head_dim, int mode, hipStream_t stream);
hipError_t launch_prefill_merge(const ReduceParams& p, hipStream_t stream);
hipError_t launch_kv_write(const WriteParams& p, hipStream_t stream);
hipError_t launch_quantize_e4m3(const QuantParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t stream);
hipError_t launch_append_e4m3(const AppendParams& p, hipStream_t stream);
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int32_t out_words, hipStream_t stream);

}  // namespace pkv
