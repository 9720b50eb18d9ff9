// abi.hip - the C ABI of libpagedkv.so (declared in include/pagedkv.h).
//
// Host side only: argument validation, parameter blocks, dispatch to the
// gfx950 kernels on the caller's stream.  No allocation, no synchronisation,
// no device reads.  Errors return a status and leave a thread-local message.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/pagedkv.h"
#include "pkv_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int elem_bytes(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_E4M3: return 1;
  }
  return 0;
}

// Checks shared by every entry point that reads the pool.
int check_desc(const pkv_desc* d, bool need_seqs) {
  if (!d) return fail(PKV_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs < 0");
  if (need_seqs && d->num_seqs > 65535) return fail(PKV_ERR_INVALID_ARG, "num_seqs > 65535");
  if (d->num_kv_heads < 1 || d->num_q_heads < 1)
    return fail(PKV_ERR_INVALID_ARG, "head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_kv_heads > 65535) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads > 65535");
  if (d->block_size != 16) return fail(PKV_ERR_INVALID_ARG, "block_size must be 16 (got %d)", d->block_size);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", d->head_dim);
  if (d->num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks < 1");
  if (d->max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq < 1");
  if (static_cast<int64_t>(d->max_blocks_per_seq) * 16 > (int64_t(1) << 30))
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  if (d->sliding_window < 0) return fail(PKV_ERR_INVALID_ARG, "sliding_window < 0");
  return PKV_OK;
}

int check_attn_types(const pkv_desc* d, const float* kv_scales) {
  const int q = d->q_dtype, kv = d->kv_dtype, o = d->out_dtype;
  bool okc = false;
  if (q == PKV_F32 && kv == PKV_F32) okc = (o == PKV_F32);
  else if (q == PKV_F16 && kv == PKV_F16) okc = (o == PKV_F32 || o == PKV_F16);
  else if (q == PKV_BF16 && kv == PKV_BF16) okc = (o == PKV_F32 || o == PKV_BF16);
  else if (q == PKV_F16 && kv == PKV_E4M3) okc = (o == PKV_F32 || o == PKV_F16);
  if (!okc) return fail(PKV_ERR_UNSUPPORTED, "unsupported dtypes q=%d kv=%d out=%d", q, kv, o);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G > 16) return fail(PKV_ERR_UNSUPPORTED, "query heads per KV head %d > 16", G);
  if (kv == PKV_E4M3 && !kv_scales) return fail(PKV_ERR_INVALID_ARG, "e4m3 cache needs kv_scales");
  if (kv != PKV_E4M3 && kv_scales) return fail(PKV_ERR_INVALID_ARG, "kv_scales given for a non-e4m3 cache");
  return PKV_OK;
}

int64_t partitions(const pkv_desc* d, int32_t psize) {
  return (static_cast<int64_t>(d->max_blocks_per_seq) * 16 + psize - 1) / psize;
}

// Split workspace: [counters int32 B*Hkv | pad to 256][tmp_lse f32 B*Hq*S | pad][tmp_out f32 B*Hq*S*D]
struct SplitLayout {
  int64_t lse_off, out_off, total;
};
int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
SplitLayout split_layout(const pkv_desc* d, int64_t s) {
  SplitLayout l;
  const int64_t rows = static_cast<int64_t>(d->num_seqs) * d->num_q_heads * s;
  l.lse_off = align256(static_cast<int64_t>(d->num_seqs) * d->num_kv_heads * 4);
  l.out_off = l.lse_off + align256(rows * 4);
  l.total = l.out_off + rows * d->head_dim * 4;
  return l;
}

// Balanced workspace: [seq_tiles int32 B+1 | pad to 256][tmp_lse f32 A*G*slots | pad]
// [tmp_out f32 A*G*slots*D].  f32 / f16 / bf16 caches run the per-compute-unit
// schedule: slots = B*Hkv + the compute units, A = 2 arrays of partials (the
// items' first parts and the rest).  E4M3 caches run the per-wave schedule:
// slots = B*Hkv + the resident grid's wave count, A = 1.
struct BalancedLayout {
  int64_t slots, lse_off, out_off, total;
  int32_t workers;
  bool per_cu;
};
int check_balanced(const pkv_desc* d) {
  if (d->num_seqs > pkv::kMaxSeqsPersistent)
    return fail(PKV_ERR_UNSUPPORTED, "balanced schedule takes at most %d sequences (got %d)",
                pkv::kMaxSeqsPersistent, d->num_seqs);
  if (static_cast<int64_t>(d->num_seqs) * d->num_kv_heads * d->max_blocks_per_seq > 0x7FFFFFFFLL)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs * num_kv_heads * max_blocks_per_seq exceeds 2^31 - 1");
  return PKV_OK;
}
BalancedLayout balanced_layout(const pkv_desc* d) {
  BalancedLayout l;
  l.per_cu = d->kv_dtype != PKV_E4M3;
  l.workers = l.per_cu ? pkv::cu_stream_workers() : pkv::stream_max_workers(d->kv_dtype, d->head_dim);
  const int64_t G = d->num_q_heads / d->num_kv_heads;
  const int64_t arrays = l.per_cu ? 2 : 1;
  l.slots = static_cast<int64_t>(d->num_seqs) * d->num_kv_heads + l.workers;
  l.lse_off = align256((static_cast<int64_t>(d->num_seqs) + 1) * 4);
  l.out_off = l.lse_off + align256(arrays * G * l.slots * 4);
  l.total = l.out_off + arrays * G * l.slots * d->head_dim * 4;
  return l;
}

int check_partition(int32_t psize) {
  if (psize <= 0 || psize % 16) return fail(PKV_ERR_INVALID_ARG, "partition_size %d is not a positive multiple of 16", psize);
  return PKV_OK;
}

pkv::DecodeParams decode_params(const void* q, const void* kc, const void* vc, const int32_t* bt,
                                const int32_t* cl, float scale, const float* kvs, const pkv_desc* d) {
  pkv::DecodeParams p{};
  p.q = q;
  p.k_cache = kc;
  p.v_cache = vc;
  p.block_tables = bt;
  p.context_lens = cl;
  p.kv_scales = kvs;
  p.qk_scale_log2 = scale * 1.4426950408889634f;
  p.num_seqs = d->num_seqs;
  p.num_q_heads = d->num_q_heads;
  p.num_kv_heads = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.num_blocks = d->num_blocks;
  p.mbps = d->max_blocks_per_seq;
  p.out_dtype = d->out_dtype;
  p.window = d->sliding_window;
  return p;
}

// Scratch of paged_decode_attention_balanced_static: a file-scope device
// array (one copy on every GPU the library runs on, held until the process
// ends).  In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to a kernel.
constexpr int64_t kStaticScratchBytes = int64_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on its first use on
// that device (the device is current for the lookup).
int static_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d past the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err; }

const char* pkv_version(void) { return "pagedkv 0.2.0 gfx950"; }

const char* pagedkv_last_error(void) { return g_err; }

const char* pagedkv_version(void) { return pkv_version(); }

int pkv_read_bandwidth_probe(const void* src, int64_t bytes, uint32_t* out, int32_t out_words, void* stream) {
  if (!src || !out) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (bytes <= 0 || bytes % 16 != 0) return fail(PKV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(PKV_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (out_words <= 0) return fail(PKV_ERR_INVALID_ARG, "out_words must be positive");
  return hip_status(pkv::launch_read_probe(src, bytes, out, out_words, static_cast<hipStream_t>(stream)),
                    "pkv_read_bandwidth_probe launch");
}

int64_t paged_decode_num_partitions(const pkv_desc* desc, int32_t partition_size) {
  if (check_desc(desc, false) || check_partition(partition_size)) return -1;
  return partitions(desc, partition_size);
}

int64_t paged_decode_workspace_bytes(const pkv_desc* desc, int32_t partition_size) {
  if (check_desc(desc, false) || check_partition(partition_size)) return -1;
  const int64_t s = partitions(desc, partition_size);
  const int64_t rows = static_cast<int64_t>(desc->num_seqs) * desc->num_q_heads * s;
  return rows * desc->head_dim * 4 + rows * 4;
}

int64_t paged_decode_split_workspace_bytes(const pkv_desc* desc, int32_t partition_size) {
  if (check_desc(desc, false) || check_partition(partition_size)) return -1;
  return split_layout(desc, partitions(desc, partition_size)).total;
}

int64_t paged_decode_balanced_workspace_bytes(const pkv_desc* desc) {
  if (check_desc(desc, false) || check_balanced(desc)) return -1;
  const BalancedLayout lay = balanced_layout(desc);
  if (lay.workers <= 0) return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d", desc->kv_dtype), -1;
  return lay.total;
}

int kv_cache_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, false)) return e;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens < 0");
  if (desc->kv_dtype == PKV_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write into an e4m3 cache: use kv_cache_quantize_e4m3");
  if (desc->kv_dtype != PKV_F32 && desc->kv_dtype != PKV_F16 && desc->kv_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d", desc->kv_dtype);
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_tokens * desc->num_kv_heads * (desc->head_dim / 4) > (int64_t(1) << 36))
    return fail(PKV_ERR_INVALID_ARG, "num_tokens too large");
  pkv::WriteParams p{};
  p.k = k;
  p.v = v;
  p.slots = slot_mapping;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.num_tokens = num_tokens;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.num_blocks = desc->num_blocks;
  p.elem_bytes = elem_bytes(desc->kv_dtype);
  return hip_status(pkv::launch_kv_write(p, static_cast<hipStream_t>(stream)), "kv_cache_write launch");
}

int kv_cache_quantize_e4m3(const float* k_src, const float* v_src, const int32_t* block_ids,
                           const int32_t* valid_tokens, int32_t num_src_blocks, void* k_cache,
                           void* v_cache, float* kv_scales, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, false)) return e;
  if (desc->kv_dtype != PKV_E4M3) return fail(PKV_ERR_INVALID_ARG, "kv_dtype must be e4m3");
  if (num_src_blocks < 0 || num_src_blocks > 0x7FFFFFFF / 2)
    return fail(PKV_ERR_INVALID_ARG, "num_src_blocks out of range");
  if (num_src_blocks == 0) return ok();
  if (!k_src || !v_src || !block_ids || !valid_tokens || !k_cache || !v_cache || !kv_scales)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::QuantParams p{};
  p.k_src = k_src;
  p.v_src = v_src;
  p.block_ids = block_ids;
  p.valid_tokens = valid_tokens;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.kv_scales = kv_scales;
  p.num_src_blocks = num_src_blocks;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.num_blocks = desc->num_blocks;
  return hip_status(pkv::launch_quantize_e4m3(p, static_cast<hipStream_t>(stream)),
                    "kv_cache_quantize_e4m3 launch");
}

int kv_cache_append_e4m3(const float* k, const float* v, const int64_t* slot_mapping, int64_t num_tokens,
                         void* k_cache, void* v_cache, float* kv_scales, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, false)) return e;
  if (desc->kv_dtype != PKV_E4M3) return fail(PKV_ERR_INVALID_ARG, "kv_dtype must be e4m3");
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF) return fail(PKV_ERR_INVALID_ARG, "num_tokens out of range");
  if (desc->num_kv_heads > 65535) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads > 65535");
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !kv_scales)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::AppendParams p{};
  p.k = k;
  p.v = v;
  p.slots = slot_mapping;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.kv_scales = kv_scales;
  p.num_tokens = num_tokens;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.num_blocks = desc->num_blocks;
  return hip_status(pkv::launch_append_e4m3(p, static_cast<hipStream_t>(stream)), "kv_cache_append_e4m3 launch");
}

int kv_cache_copy_blocks(const int32_t* block_mapping, int32_t num_pairs, void* k_cache, void* v_cache,
                         float* kv_scales, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, false)) return e;
  const int e_bytes = elem_bytes(desc->kv_dtype);
  if (e_bytes == 0) return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d", desc->kv_dtype);
  if (num_pairs < 0 || num_pairs > 65535) return fail(PKV_ERR_INVALID_ARG, "num_pairs must be in [0, 65535]");
  if (desc->kv_dtype == PKV_E4M3 && !kv_scales) return fail(PKV_ERR_INVALID_ARG, "e4m3 cache needs kv_scales");
  if (desc->kv_dtype != PKV_E4M3 && kv_scales)
    return fail(PKV_ERR_INVALID_ARG, "kv_scales given for a non-e4m3 cache");
  if (num_pairs == 0) return ok();
  if (!block_mapping || !k_cache || !v_cache) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::CopyParams p{};
  p.block_mapping = block_mapping;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.kv_scales = kv_scales;
  p.block_bytes = static_cast<int64_t>(desc->num_kv_heads) * 16 * desc->head_dim * e_bytes;
  p.num_pairs = num_pairs;
  p.num_blocks = desc->num_blocks;
  p.num_kv_heads = desc->num_kv_heads;
  return hip_status(pkv::launch_copy_blocks(p, static_cast<hipStream_t>(stream)), "kv_cache_copy_blocks launch");
}

int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                           const float* kv_scales, void* out, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_attn_types(desc, kv_scales)) return e;
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (desc->num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::DecodeParams p = decode_params(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, desc);
  p.out = out;
  p.partition_blocks = desc->max_blocks_per_seq;
  p.num_partitions = 1;
  return hip_status(pkv::launch_decode(p, desc->kv_dtype, desc->head_dim, 0,
                                       static_cast<hipStream_t>(stream)),
                    "paged_decode_attention launch");
}

int paged_decode_attention_partial(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   float scale, const float* kv_scales, int32_t partition_size,
                                   float* tmp_out, float* tmp_lse, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_attn_types(desc, kv_scales)) return e;
  if (int e = check_partition(partition_size)) return e;
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (desc->num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !tmp_out || !tmp_lse)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  const int64_t s = partitions(desc, partition_size);
  if (s > 0x7FFFFFFF) return fail(PKV_ERR_INVALID_ARG, "too many partitions");
  pkv::DecodeParams p = decode_params(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, desc);
  p.tmp_out = tmp_out;
  p.tmp_lse = tmp_lse;
  p.partition_blocks = partition_size / 16;
  p.num_partitions = static_cast<int32_t>(s);
  return hip_status(pkv::launch_decode(p, desc->kv_dtype, desc->head_dim, 1,
                                       static_cast<hipStream_t>(stream)),
                    "paged_decode_attention_partial launch");
}

static int split_common(const void* q, const void* k_new, const void* v_new, const void* k_cache,
                        const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                        float scale, const float* kv_scales, int32_t partition_size, void* workspace,
                        int64_t workspace_bytes, void* out, const pkv_desc* desc, void* stream,
                        const char* what) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_attn_types(desc, kv_scales)) return e;
  if (int e = check_partition(partition_size)) return e;
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (desc->num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !workspace || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(PKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int64_t s = partitions(desc, partition_size);
  if (s > 0x7FFFFFFF) return fail(PKV_ERR_INVALID_ARG, "too many partitions");
  const SplitLayout lay = split_layout(desc, s);
  if (workspace_bytes < lay.total)
    return fail(PKV_ERR_INVALID_ARG, "workspace of %lld bytes is smaller than the %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(lay.total));
  char* ws = static_cast<char*>(workspace);
  pkv::DecodeParams p = decode_params(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, desc);
  p.out = out;
  p.counters = reinterpret_cast<int32_t*>(ws);
  p.tmp_lse = reinterpret_cast<float*>(ws + lay.lse_off);
  p.tmp_out = reinterpret_cast<float*>(ws + lay.out_off);
  p.partition_blocks = partition_size / 16;
  p.num_partitions = static_cast<int32_t>(s);
  p.k_new = k_new;
  p.v_new = v_new;
  return hip_status(pkv::launch_decode(p, desc->kv_dtype, desc->head_dim, 2,
                                       static_cast<hipStream_t>(stream)),
                    what);
}

int paged_decode_attention_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float scale, const float* kv_scales, int32_t partition_size,
                                 void* workspace, int64_t workspace_bytes, void* out,
                                 const pkv_desc* desc, void* stream) {
  return split_common(q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                      partition_size, workspace, workspace_bytes, out, desc, stream,
                      "paged_decode_attention_split launch");
}

int paged_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t partition_size, void* workspace, int64_t workspace_bytes, void* out,
                      const pkv_desc* desc, void* stream) {
  if (desc && desc->kv_dtype == PKV_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "paged_decode_step into an e4m3 cache: use kv_cache_append_e4m3");
  if (desc && desc->num_seqs > 0 && (!k_new || !v_new))
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  return split_common(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, nullptr,
                      partition_size, workspace, workspace_bytes, out, desc, stream, "paged_decode_step launch");
}

// Checks shared by the two balanced entry points (everything but the workspace).
static int balanced_checks(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, float scale, const float* kv_scales, const void* out,
                           const pkv_desc* desc) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_attn_types(desc, kv_scales)) return e;
  if (int e = check_balanced(desc)) return e;
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (desc->num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  return PKV_OK;
}

// The balanced schedule's two launches on a workspace already checked
// against lay: the tile stream, then the merge of the partials.
static int balanced_main(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, const float* kv_scales, char* ws,
                         const BalancedLayout& lay, void* out, const pkv_desc* desc, void* stream,
                         const char* what) {
  pkv::DecodeParams p = decode_params(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, desc);
  p.out = out;
  p.seq_tiles = reinterpret_cast<int32_t*>(ws);
  p.tmp_lse = reinterpret_cast<float*>(ws + lay.lse_off);
  p.tmp_out = reinterpret_cast<float*>(ws + lay.out_off);
  p.num_workers = lay.workers;
  p.num_slots = static_cast<int32_t>(lay.slots);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(lay.per_cu ? pkv::launch_cu_stream(p, desc->kv_dtype, desc->head_dim, st)
                               : pkv::launch_stream(p, desc->kv_dtype, desc->head_dim, st),
                    what);
}

static int balanced_merge(char* ws, const BalancedLayout& lay, void* out, const pkv_desc* desc, void* stream,
                          const char* what) {
  pkv::ReduceParams r{};
  r.tmp_out = reinterpret_cast<float*>(ws + lay.out_off);
  r.tmp_lse = reinterpret_cast<float*>(ws + lay.lse_off);
  r.out = out;
  r.num_seqs = desc->num_seqs;
  r.num_q_heads = desc->num_q_heads;
  r.head_dim = desc->head_dim;
  r.mbps = desc->max_blocks_per_seq;
  r.out_dtype = desc->out_dtype;
  r.seq_tiles = reinterpret_cast<int32_t*>(ws);
  r.num_kv_heads = desc->num_kv_heads;
  r.num_workers = lay.workers;
  r.num_slots = static_cast<int32_t>(lay.slots);
  r.window = desc->sliding_window;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(lay.per_cu ? pkv::launch_cu_merge(r, st) : pkv::launch_stream_merge(r, st), what);
}

static int balanced_run(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        const int32_t* context_lens, float scale, const float* kv_scales, char* ws,
                        const BalancedLayout& lay, void* out, const pkv_desc* desc, void* stream, const char* what) {
  if (int e = balanced_main(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, ws, lay, out, desc,
                            stream, what))
    return e;
  return balanced_merge(ws, lay, out, desc, stream, what);
}

// Checks a caller workspace for the balanced schedule.
static int balanced_workspace_check(const void* workspace, int64_t workspace_bytes, const BalancedLayout& lay) {
  if (!workspace) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(PKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < lay.total)
    return fail(PKV_ERR_INVALID_ARG, "workspace of %lld bytes is smaller than the %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(lay.total));
  if (lay.slots > 0x7FFFFFFF / 16) return fail(PKV_ERR_INVALID_ARG, "too many partial slots");
  return PKV_OK;
}

int paged_decode_attention_balanced(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                                    const float* kv_scales, void* workspace, int64_t workspace_bytes,
                                    void* out, const pkv_desc* desc, void* stream) {
  if (int e = balanced_checks(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, out, desc)) return e;
  if (desc->num_seqs == 0) return ok();
  const BalancedLayout lay = balanced_layout(desc);
  if (int e = balanced_workspace_check(workspace, workspace_bytes, lay)) return e;
  return balanced_run(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                      static_cast<char*>(workspace), lay, out, desc, stream, "paged_decode_attention_balanced launch");
}

int paged_decode_attention_balanced_partial(const void* q, const void* k_cache, const void* v_cache,
                                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                                            const float* kv_scales, void* workspace, int64_t workspace_bytes,
                                            void* out, const pkv_desc* desc, void* stream) {
  if (int e = balanced_checks(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, out, desc)) return e;
  if (desc->num_seqs == 0) return ok();
  const BalancedLayout lay = balanced_layout(desc);
  if (int e = balanced_workspace_check(workspace, workspace_bytes, lay)) return e;
  return balanced_main(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales,
                       static_cast<char*>(workspace), lay, out, desc, stream,
                       "paged_decode_attention_balanced_partial launch");
}

int paged_decode_attention_balanced_reduce(void* workspace, int64_t workspace_bytes, void* out, const pkv_desc* desc,
                                           void* stream) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_balanced(desc)) return e;
  if (desc->num_seqs == 0) return ok();
  if (!out) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  const BalancedLayout lay = balanced_layout(desc);
  if (lay.workers <= 0) return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d", desc->kv_dtype);
  if (int e = balanced_workspace_check(workspace, workspace_bytes, lay)) return e;
  return balanced_merge(static_cast<char*>(workspace), lay, out, desc, stream,
                        "paged_decode_attention_balanced_reduce launch");
}

int paged_decode_attention_balanced_static(const void* q, const void* k_cache, const void* v_cache,
                                           const int32_t* block_tables, const int32_t* context_lens, float scale,
                                           const float* kv_scales, void* out, const pkv_desc* desc, void* stream) {
  if (int e = balanced_checks(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, out, desc)) return e;
  if (desc->num_seqs == 0) return ok();
  const BalancedLayout lay = balanced_layout(desc);
  if (lay.total > kStaticScratchBytes)
    return fail(PKV_ERR_INVALID_ARG,
                "paged_decode_attention_balanced_static needs %lld bytes of scratch; the static buffer holds %lld "
                "(use paged_decode_attention_balanced with a workspace)",
                static_cast<long long>(lay.total), static_cast<long long>(kStaticScratchBytes));
  char* ws = nullptr;
  if (int e = static_scratch(&ws)) return e;
  return balanced_run(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, ws, lay, out, desc, stream,
                      "paged_decode_attention_balanced_static launch");
}

int64_t paged_prefill_workspace_bytes(const pkv_desc* desc, int32_t num_query_tokens, int32_t partition_size) {
  if (check_desc(desc, false)) return -1;
  if (num_query_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_query_tokens < 0"), -1;
  if (partition_size == 0) return 0;
  if (check_partition(partition_size)) return -1;
  const int64_t rows = static_cast<int64_t>(num_query_tokens) * desc->num_q_heads * partitions(desc, partition_size);
  return align256(rows * 4) + rows * desc->head_dim * 4;
}

int paged_prefill_attention(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start, int32_t num_query_tokens,
                            float scale, const float* kv_scales, int32_t partition_size, void* workspace,
                            int64_t workspace_bytes, void* out, const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, true)) return e;
  if (int e = check_attn_types(desc, kv_scales)) return e;
  if (desc->num_seqs > pkv::kMaxSeqsPersistent)
    return fail(PKV_ERR_UNSUPPORTED, "multi-token step takes at most %d sequences (got %d)",
                pkv::kMaxSeqsPersistent, desc->num_seqs);
  if (desc->sliding_window != 0) return fail(PKV_ERR_UNSUPPORTED, "multi-token step has no sliding window");
  if (partition_size != 0)
    if (int e = check_partition(partition_size)) return e;
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  if (num_query_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_query_tokens < 0");
  if (static_cast<int64_t>(num_query_tokens) * desc->num_q_heads > 0x7FFFFFFF / 2)
    return fail(PKV_ERR_INVALID_ARG, "num_query_tokens * num_q_heads too large");
  if (desc->num_seqs == 0 || num_query_tokens == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::DecodeParams p = decode_params(q, k_cache, v_cache, block_tables, context_lens, scale, kv_scales, desc);
  p.query_start = query_start;
  p.num_query_tokens = num_query_tokens;
  p.tokens_per_pack = 16 / p.group;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (partition_size == 0) {
    p.out = out;
    p.partition_blocks = desc->max_blocks_per_seq;
    p.num_partitions = 1;
    return hip_status(pkv::launch_prefill(p, desc->kv_dtype, desc->head_dim, 0, st), "paged_prefill_attention launch");
  }
  const int64_t s_parts = partitions(desc, partition_size);
  const int64_t rows = static_cast<int64_t>(num_query_tokens) * desc->num_q_heads * s_parts;
  const int64_t need = align256(rows * 4) + rows * desc->head_dim * 4;
  if (!workspace) return fail(PKV_ERR_INVALID_ARG, "null workspace");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(PKV_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(PKV_ERR_INVALID_ARG, "workspace of %lld bytes is smaller than the %lld needed",
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
  char* ws = static_cast<char*>(workspace);
  p.tmp_lse = reinterpret_cast<float*>(ws);
  p.tmp_out = reinterpret_cast<float*>(ws + align256(rows * 4));
  p.partition_blocks = partition_size / 16;
  p.num_partitions = static_cast<int32_t>(s_parts);
  if (int e = hip_status(pkv::launch_prefill(p, desc->kv_dtype, desc->head_dim, 1, st), "paged_prefill_attention launch"))
    return e;
  pkv::ReduceParams r{};
  r.tmp_out = p.tmp_out;
  r.tmp_lse = p.tmp_lse;
  r.context_lens = context_lens;
  r.out = out;
  r.num_seqs = desc->num_seqs;
  r.num_q_heads = desc->num_q_heads;
  r.head_dim = desc->head_dim;
  r.mbps = desc->max_blocks_per_seq;
  r.partition_size = partition_size;
  r.num_partitions = p.num_partitions;
  r.out_dtype = desc->out_dtype;
  r.query_start = query_start;
  r.num_query_tokens = num_query_tokens;
  return hip_status(pkv::launch_prefill_merge(r, st), "paged_prefill_attention merge launch");
}

int paged_decode_attention_reduce(const float* tmp_out, const float* tmp_lse,
                                  const int32_t* context_lens, int32_t partition_size, void* out,
                                  const pkv_desc* desc, void* stream) {
  if (int e = check_desc(desc, false)) return e;
  if (int e = check_partition(partition_size)) return e;
  const int o = desc->out_dtype;
  if (o != PKV_F32 && o != PKV_F16 && o != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "out_dtype %d", o);
  if (desc->num_seqs == 0) return ok();
  if (!tmp_out || !tmp_lse || !context_lens || !out) return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (static_cast<int64_t>(desc->num_seqs) * desc->num_q_heads > 0x7FFFFFFF / 2)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs * num_q_heads too large");
  pkv::ReduceParams p{};
  p.tmp_out = tmp_out;
  p.tmp_lse = tmp_lse;
  p.context_lens = context_lens;
  p.out = out;
  p.num_seqs = desc->num_seqs;
  p.num_q_heads = desc->num_q_heads;
  p.head_dim = desc->head_dim;
  p.mbps = desc->max_blocks_per_seq;
  p.partition_size = partition_size;
  p.num_partitions = static_cast<int32_t>(partitions(desc, partition_size));
  p.out_dtype = o;
  p.window = desc->sliding_window;
  return hip_status(pkv::launch_reduce(p, static_cast<hipStream_t>(stream)),
                    "paged_decode_attention_reduce launch");
}

}  // extern "C"
