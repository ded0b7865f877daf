// C-ABI host layer: argument validation, split planning, workspace carving and
// kernel launch.  Validation runs before any HIP call, so every error status is
// reachable (and tested) on a machine without a GPU.
#include "attn_mi355x.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "attn_internal.h"

static_assert(attn::kNoallocScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "scratch size of the header");

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

attn_status ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kAlign = 256;
constexpr int kMaxGridYZ = 65535;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(attn_dtype d) { return d == ATTN_F32 || d == ATTN_BF16; }

// Largest power of two <= x (x >= 1).
int pow2_floor(long long x) {
  int p = 1;
  while ((long long)p * 2 <= x && p < (1 << 30)) p *= 2;
  return p;
}

// Positions per decode block (the work unit of the fixed schedule; the queue
// hands out single blocks, or for large batches units of four blocks first)
// when the caller leaves it to the library: about B*Hkv*T_max / 4096 rounded
// down to a multiple of 64, so that every one of the ~256 queue workgroups
// takes several units even when the lengths are ragged and the last units are
// short (512 at B 32, Hkv 8, T_max 8192: measured best), at most 1024, and long
// enough that the fp32 partial of a unit (n_rep * D * 4 bytes written and read
// back) stays small next to its cache bytes (chunk * D * 4); with 16 or more
// query heads per KV head the per-unit costs dominate a short chunk (measured),
// hence the higher floors.  At 32 query heads per KV head (B 16, one KV head,
// 8192 positions) the 1024 floor leaves 128 units for 256 compute units, yet
// 512 (256 units) measures no faster: 21.3-21.7 against 21.0-21.1 us; the
// kernel's time there is its fixed start and end, not the streaming.
int choose_chunk(int B, int Hkv, int n_rep, int T_max) {
  int lo = 64;
  if (n_rep >= 8) lo = 128;
  if (n_rep >= 16) lo = 512;
  if (n_rep >= 32) lo = 1024;
  const long long want = (long long)B * Hkv * T_max / 4096 / 64 * 64;
  return (int)(want < lo ? lo : (want > 1024 ? 1024 : want));
}

// Below this many blocks the decode runs one workgroup per unit (see gqa_layout).
constexpr long long kQueueMinBlocks = 256;

// FP8 caches: a chunk a quarter longer than choose_chunk's (at least 64 more
// positions, a multiple of 64).  It never makes more blocks, so a workspace
// sized for choose_chunk suffices.  Measured on the Llama-3-8B decode shape
// (512 -> 640 positions), both lengths in interleaved rounds in each process:
// 512 took 58.8-59.6 us in six of ten processes and 53.7-54.8 us in the other
// four (which one depends on the process's allocations), 640 took 54.2-55.3 us
// in all eight that ran it.
// Like choose_chunk it stays at most 1024 (a paged unit holds at most 128
// page numbers: four blocks of 1024 positions at 32 per page).
int choose_chunk_fp8(int B, int Hkv, int n_rep, int T_max) {
  const int c = choose_chunk(B, Hkv, n_rep, T_max);
  const int more = c / 4 / 64 * 64;
  const int f = c + (more > 64 ? more : 64);
  return f < 1024 ? f : 1024;
}

bool valid_split(int split) { return split == 0 || (split >= 64 && split <= 65536 && split % 64 == 0); }

// Decode schedule and workspace layout.  Work units are chunks of `chunk`
// positions of one (sequence, KV head): split_tokens, or chosen by the library
// when 0.  Workspace: [queue counter, 256 bytes][lse slots*n_rep][o_part
// slots*n_rep*D] with slots = B*Hkv*n_chunks (none when every sequence is one
// chunk), each piece 256-byte aligned.  The queue schedule is used when the
// batch has more blocks than the 256 compute units of an MI355X: with fewer,
// every workgroup would take at most one unit, and one workgroup per unit
// starts its loads without the queue's plan (a prefix sum over all cache
// lengths before the first unit is known).  Measured on the MQA sweep setting
// (B 16, one KV head, 8192 positions: 128 blocks of 1024): 22.3 -> 21.0 us.
struct GqaLayout {
  int chunk, n_chunks;
  bool queue;  // units taken from the device-wide queue (else one workgroup per unit)
  long long slots;
  size_t lse_off, o_off, total;
};

GqaLayout gqa_layout(int B, int Hq, int Hkv, int D, int T_max, int split_tokens, bool all_partials = false,
                     bool kv_fp8 = false) {
  GqaLayout l;
  const int n_rep = Hq / (Hkv > 0 ? Hkv : 1);
  l.chunk = split_tokens ? split_tokens
                         : (kv_fp8 ? choose_chunk_fp8 : choose_chunk)(B, Hkv, n_rep, T_max);
  l.n_chunks = (int)(((long long)T_max + l.chunk - 1) / l.chunk);
  l.queue = B <= attn::kQueueMaxB && l.n_chunks >= 2 && (long long)B * Hkv * l.n_chunks > kQueueMinBlocks;
  l.slots = (l.n_chunks >= 2 || all_partials) ? (long long)B * Hkv * l.n_chunks : 0;
  l.lse_off = 256;
  l.o_off = l.lse_off + align_up((size_t)l.slots * n_rep * sizeof(float));
  l.total = l.o_off + align_up((size_t)l.slots * n_rep * D * sizeof(float));
  return l;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Compute units the default MLA chunk length is planned for (MI355X).  A fixed
// number rather than the current device's, so that the workspace size of a
// call does not depend on which device is current; on a device with another
// count the plan stays valid, only less balanced.
constexpr int kPlanCUs = 256;

// MLA decode workspace: [per-sequence done counters, B x 4 bytes][lse B x
// n_splits x H][o_part B x n_splits x H x r] fp32, each piece 256-byte aligned.
struct MlaLayout {
  int split, n_splits;
  size_t lse_off, o_part_off, total;
};

MlaLayout mla_layout(int B, int H, int r, int T_max, int split_tokens) {
  MlaLayout l;
  // One (chunk, sequence) workgroup serves all heads; aim for about one
  // workgroup per compute unit over the whole batch, with chunks of at least
  // 256 positions so that each wave's copy ring runs several steps.
  if (split_tokens) {
    l.split = split_tokens;
  } else {
    const long long want = ((long long)B * T_max + kPlanCUs - 1) / kPlanCUs;
    long long s = 256;
    while (s < want && s < 65536) s <<= 1;
    l.split = (int)s;
  }
  l.n_splits = (T_max + l.split - 1) / l.split;
  const size_t rows = (size_t)B * H * l.n_splits;
  l.lse_off = align_up((size_t)B * sizeof(unsigned));
  l.o_part_off = l.lse_off + align_up(rows * sizeof(float));
  l.total = l.o_part_off + align_up(rows * r * sizeof(float));
  return l;
}

attn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid size argument";
    case ATTN_ERR_GROUPS: return "KV head count does not divide query head count";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head size, dtype or layout";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

size_t attn_decode_gqa_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int T_max,
                                       int split_tokens) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 || T_max <= 0 || !valid_split(split_tokens))
    return 0;
  return gqa_layout(B, Hq, Hkv, head_dim, T_max, split_tokens).total;
}

namespace {

// Shared checks and launch of the two decode entry points.  k_new != null: a
// decode step that also takes the new token's K/V (see attn_decode_gqa_append).
// kv_scales != null: caches of FP8 E4M3 codes with scales {k_scale, v_scale}.
attn_status gqa_decode_common(const char* fn, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                              const void* v_cache, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                              int head_dim, int T_max, float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype,
                              int split_tokens, void* workspace, size_t workspace_bytes, void* stream,
                              const float* kv_scales = nullptr, bool noalloc = false,
                              const int32_t* block_table = nullptr, int page_size = 0, int n_pages = 0,
                              const float* k_row_scales = nullptr, const float* v_row_scales = nullptr) {
  const bool append = k_new != nullptr;
  const bool kv_fp8 = kv_scales != nullptr;
  if (!q || !k_cache || !v_cache || !cache_lens || !out)
    return fail(ATTN_ERR_NULL, "%s: q, k_cache, v_cache, cache_lens and out must be non-NULL", fn);
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 || T_max <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d Hq=%d Hkv=%d head_dim=%d T_max=%d)", fn,
                B, Hq, Hkv, head_dim, T_max);
  if (B > kMaxGridYZ || Hkv > kMaxGridYZ)
    return fail(ATTN_ERR_SHAPE, "%s: B and Hkv must be <= %d", fn, kMaxGridYZ);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_GROUPS, "%s: Hkv=%d does not divide Hq=%d (remainder %d); not rounded", fn,
                Hkv, Hq, Hq % Hkv);
  if (!valid_split(split_tokens))
    return fail(ATTN_ERR_SHAPE, "%s: split_tokens=%d must be 0 or a multiple of 64 in [64, 65536]", fn,
                split_tokens);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  const int n_rep = Hq / Hkv;
  const int in_bf16 = in_dtype == ATTN_BF16;
  if (!attn::gqa_decode_supported(head_dim, n_rep, in_bf16))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: head_dim=%d with Hq/Hkv=%d and %s inputs is not built", fn,
                head_dim, n_rep, in_bf16 ? "bf16" : "fp32");
  if (kv_fp8 && head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: fp8 caches are built for head_dim 128 only (got %d)", fn, head_dim);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: q, caches and out must be 16-byte aligned", fn);
  const GqaLayout lay = gqa_layout(B, Hq, Hkv, head_dim, T_max, split_tokens, append, kv_fp8);
  if (!lay.queue && lay.n_chunks > kMaxGridYZ)
    return fail(ATTN_ERR_SHAPE, "%s: ceil(T_max/split_tokens)=%d chunks exceed %d", fn, lay.n_chunks,
                kMaxGridYZ);
  if (lay.slots >= (1ll << 31) / (n_rep > 0 ? n_rep : 1))
    return fail(ATTN_ERR_SHAPE, "%s: too many chunks (B*Hkv*ceil(T_max/split_tokens) too large)", fn);
  if (noalloc) {
    if (lay.total > attn::kNoallocScratchBytes)
      return fail(ATTN_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch; the built-in scratch holds %zu",
                  fn, lay.total, attn::kNoallocScratchBytes);
  } else {
    if (!workspace || workspace_bytes < lay.total)
      return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, lay.total,
                  workspace_bytes, workspace ? "" : " (NULL)");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(ATTN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }

  if (noalloc) {
    // every call on a device shares its scratch; the queue counter is zeroed first
    const attn_status st = hip_status(attn::noalloc_scratch(&workspace), fn);
    if (st != ATTN_OK) return st;
    const attn_status sc =
        hip_status(attn::launch_clear_queue(static_cast<unsigned*>(workspace), static_cast<hipStream_t>(stream)), fn);
    if (sc != ATTN_OK) return sc;
  }
  attn::GqaDecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.lens = cache_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.queue = reinterpret_cast<unsigned*>(ws);
  a.lse = reinterpret_cast<float*>(ws + lay.lse_off);
  a.o_part = reinterpret_cast<float*>(ws + lay.o_off);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = head_dim;
  a.T_max = T_max;
  a.n_rep = n_rep;
  a.chunk = lay.chunk;
  a.n_chunks = lay.n_chunks;
  a.use_queue = lay.queue;
  a.big_units = 0;
  a.grid_wgs = 0;
  a.cus = 0;
  if (lay.queue) {
    // at most four decode workgroups fit on a compute unit; the launcher trims
    // the grid to what is actually resident
    const int cus = device_cus();
    if (cus <= 0) return fail(ATTN_ERR_HIP, "%s: cannot query the current device", fn);
    a.cus = cus;
    a.grid_wgs = cus * 4;
    // big units only where every workgroup still gets many units when the
    // cache is full (B*Hkv*n_chunks blocks at most)
    a.big_units = (long long)B * Hkv * lay.n_chunks >= 16LL * cus;
  }
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.scale_log2e = scale * kLog2e * (kv_fp8 ? kv_scales[0] : 1.f);
  a.in_bf16 = in_bf16;
  a.out_bf16 = out_dtype == ATTN_BF16;
  a.kv_fp8 = kv_fp8;
  a.v_scale = kv_fp8 ? kv_scales[1] : 1.f;
  a.append = append;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = const_cast<void*>(k_cache);
  a.v_cache = const_cast<void*>(v_cache);
  a.kv_int4 = k_row_scales != nullptr;
  a.k_scales = k_row_scales;
  a.v_scales = v_row_scales;
  a.block_table = block_table;
  a.page_size = page_size;
  a.table_stride = block_table ? T_max / page_size : 0;
  a.n_pages = n_pages;
  return hip_status(attn::launch_gqa_decode(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

attn_status attn_decode_gqa(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                            int head_dim, int T_max, float softmax_scale, attn_dtype in_dtype,
                            attn_dtype out_dtype, int split_tokens, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return gqa_decode_common("attn_decode_gqa", q, nullptr, nullptr, k_cache, v_cache, cache_lens, out, B, Hq, Hkv,
                           head_dim, T_max, softmax_scale, in_dtype, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream);
}

namespace {

// Checks shared by the paged GQA decode entry points.
attn_status gqa_paged_checks(const char* fn, const int32_t* block_table, int page_size, int n_pages,
                             int max_pages_per_seq, attn_dtype in_dtype, int split_tokens) {
  if (!block_table) return fail(ATTN_ERR_NULL, "%s: block_table must be non-NULL", fn);
  if (page_size <= 0 || n_pages <= 0 || max_pages_per_seq <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: page_size, n_pages and max_pages_per_seq must be positive (%d, %d, %d)", fn,
                page_size, n_pages, max_pages_per_seq);
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "%s: page_size * max_pages_per_seq too large", fn);
  if (page_size % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size=%d must be a multiple of 32", fn, page_size);
  if (in_dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: paged caches are built for bf16 inputs only", fn);
  if (split_tokens > 1024)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: split_tokens=%d: at most 1024 with paged caches", fn, split_tokens);
  return ATTN_OK;
}

}  // namespace

attn_status attn_decode_gqa_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                  const int32_t* cache_lens, void* out, int B, int Hq, int Hkv, int head_dim,
                                  int page_size, int n_pages, int max_pages_per_seq, float softmax_scale,
                                  attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_gqa_paged";
  const attn_status st = gqa_paged_checks(fn, block_table, page_size, n_pages, max_pages_per_seq, in_dtype,
                                          split_tokens);
  if (st != ATTN_OK) return st;
  return gqa_decode_common(fn, q, nullptr, nullptr, k_pages, v_pages, cache_lens, out, B, Hq, Hkv, head_dim,
                           page_size * max_pages_per_seq, softmax_scale, in_dtype, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream, nullptr, false, block_table, page_size, n_pages);
}

attn_status attn_decode_gqa_paged_append(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                         void* v_pages, const int32_t* block_table, const int32_t* cache_lens,
                                         void* out, int B, int Hq, int Hkv, int head_dim, int page_size, int n_pages,
                                         int max_pages_per_seq, float softmax_scale, attn_dtype in_dtype,
                                         attn_dtype out_dtype, int split_tokens, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_gqa_paged_append";
  if (!k_new || !v_new) return fail(ATTN_ERR_NULL, "%s: k_new and v_new must be non-NULL", fn);
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: k_new and v_new must be 16-byte aligned", fn);
  const attn_status st = gqa_paged_checks(fn, block_table, page_size, n_pages, max_pages_per_seq, in_dtype,
                                          split_tokens);
  if (st != ATTN_OK) return st;
  return gqa_decode_common(fn, q, k_new, v_new, k_pages, v_pages, cache_lens, out, B, Hq, Hkv, head_dim,
                           page_size * max_pages_per_seq, softmax_scale, in_dtype, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream, nullptr, false, block_table, page_size, n_pages);
}

attn_status attn_decode_gqa_paged_fp8kv(const void* q, const void* k_pages, const void* v_pages, float k_scale,
                                        float v_scale, const int32_t* block_table, const int32_t* cache_lens,
                                        void* out, int B, int Hq, int Hkv, int head_dim, int page_size, int n_pages,
                                        int max_pages_per_seq, float softmax_scale, attn_dtype out_dtype,
                                        int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_gqa_paged_fp8kv";
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(ATTN_ERR_SHAPE, "%s: k_scale and v_scale must be positive and finite (got %g, %g)", fn,
                (double)k_scale, (double)v_scale);
  const attn_status st = gqa_paged_checks(fn, block_table, page_size, n_pages, max_pages_per_seq, ATTN_BF16,
                                          split_tokens);
  if (st != ATTN_OK) return st;
  const float scales[2] = {k_scale, v_scale};
  return gqa_decode_common(fn, q, nullptr, nullptr, k_pages, v_pages, cache_lens, out, B, Hq, Hkv, head_dim,
                           page_size * max_pages_per_seq, softmax_scale, ATTN_BF16, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream, scales, false, block_table, page_size, n_pages);
}

attn_status attn_decode_gqa_int4kv(const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
                                   const float* v_scales, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                   int head_dim, int T_max, float softmax_scale, attn_dtype out_dtype,
                                   int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_gqa_int4kv";
  if (!k_scales || !v_scales) return fail(ATTN_ERR_NULL, "%s: k_scales and v_scales must be non-NULL", fn);
  if (head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: int4 caches are built for head_dim 128 only (got %d)", fn, head_dim);
  if ((reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: the scales must be 4-byte aligned", fn);
  return gqa_decode_common(fn, q, nullptr, nullptr, k_codes, v_codes, cache_lens, out, B, Hq, Hkv, head_dim, T_max,
                           softmax_scale, ATTN_BF16, out_dtype, split_tokens, workspace, workspace_bytes, stream,
                           nullptr, false, nullptr, 0, 0, k_scales, v_scales);
}

attn_status attn_decode_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_lens, void* out, int B, int Hq, int Hkv, int head_dim,
                                    int T_max, float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                    int split_tokens, void* stream) {
  return gqa_decode_common("attn_decode_gqa_noalloc", q, nullptr, nullptr, k_cache, v_cache, cache_lens, out, B, Hq,
                           Hkv, head_dim, T_max, softmax_scale, in_dtype, out_dtype, split_tokens, nullptr, 0, stream,
                           nullptr, true);
}

attn_status attn_decode_gqa_fp8kv(const void* q, const void* k_cache, const void* v_cache, float k_scale,
                                  float v_scale, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                  int head_dim, int T_max, float softmax_scale, attn_dtype out_dtype, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return fail(ATTN_ERR_SHAPE, "attn_decode_gqa_fp8kv: k_scale and v_scale must be positive and finite");
  const float scales[2] = {k_scale, v_scale};
  return gqa_decode_common("attn_decode_gqa_fp8kv", q, nullptr, nullptr, k_cache, v_cache, cache_lens, out, B, Hq, Hkv,
                           head_dim, T_max, softmax_scale, ATTN_BF16, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream, scales);
}

size_t attn_decode_gqa_append_workspace_bytes(int B, int Hq, int Hkv, int head_dim, int T_max, int split_tokens) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 || T_max <= 0 || !valid_split(split_tokens))
    return 0;
  return gqa_layout(B, Hq, Hkv, head_dim, T_max, split_tokens, true).total;
}

attn_status attn_decode_gqa_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, const int32_t* cache_lens, void* out, int B, int Hq, int Hkv,
                                   int head_dim, int T_max, float softmax_scale, attn_dtype in_dtype,
                                   attn_dtype out_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!k_new || !v_new)
    return fail(ATTN_ERR_NULL, "attn_decode_gqa_append: k_new and v_new must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_gqa_append: k_new and v_new must be 16-byte aligned");
  return gqa_decode_common("attn_decode_gqa_append", q, k_new, v_new, k_cache, v_cache, cache_lens, out, B, Hq,
                           Hkv, head_dim, T_max, softmax_scale, in_dtype, out_dtype, split_tokens, workspace,
                           workspace_bytes, stream);
}

namespace {

// Shared checks and launch of the prefill entry points.  start_pos == null
// means no cached prefix (k and v then hold exactly S rows per sequence);
// k_new != null that the new rows come in k_new / v_new and are written into
// k and v by the same launch.
attn_status prefill_common(const char* fn, const void* q, const void* k, const void* v,
                           const int32_t* start_pos, const int32_t* q_lens, void* out, int B, int S, int Hq,
                           int Hkv, int head_dim, int T_kv, float softmax_scale, attn_dtype in_dtype,
                           attn_dtype out_dtype, void* stream, const void* k_new = nullptr,
                           const void* v_new = nullptr, const int32_t* block_table = nullptr, int page_size = 0,
                           int n_pages = 0, int table_stride = 0) {
  if (!q || !k || !v || !out)
    return fail(ATTN_ERR_NULL, "%s: q, k, v and out must be non-NULL", fn);
  if ((k_new != nullptr) != (v_new != nullptr))
    return fail(ATTN_ERR_NULL, "%s: k_new and v_new must be non-NULL", fn);
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || head_dim <= 0 || T_kv <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d S=%d Hq=%d Hkv=%d head_dim=%d T=%d)", fn, B, S,
                Hq, Hkv, head_dim, T_kv);
  if (B > kMaxGridYZ || Hq > kMaxGridYZ)
    return fail(ATTN_ERR_SHAPE, "%s: B and Hq must be <= %d", fn, kMaxGridYZ);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_GROUPS, "%s: Hkv=%d does not divide Hq=%d (remainder %d); not rounded", fn, Hkv, Hq,
                Hq % Hkv);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (in_dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: only bf16 inputs are built (MFMA path)", fn);
  if (!attn::prefill_supported(head_dim))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: head_dim=%d is not built", fn, head_dim);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(k_new) ||
      !aligned16(v_new))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: q, k, v, out and the new rows must be 16-byte aligned", fn);
  attn::PrefillArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.page_size = page_size;
  a.n_pages = n_pages;
  a.table_stride = table_stride;
  a.q = q;
  a.k = k;
  a.v = v;
  a.start_pos = start_pos;
  a.q_lens = q_lens;
  a.out = out;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = head_dim;
  a.n_rep = Hq / Hkv;
  a.T_kv = T_kv;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.scale_log2e = scale * kLog2e;
  a.out_bf16 = out_dtype == ATTN_BF16;
  return hip_status(attn::launch_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

attn_status attn_prefill_gqa_causal(const void* q, const void* k, const void* v, void* out, int B,
                                    int S, int Hq, int Hkv, int head_dim, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream) {
  return prefill_common("attn_prefill_gqa_causal", q, k, v, nullptr, nullptr, out, B, S, Hq, Hkv, head_dim, S,
                        softmax_scale, in_dtype, out_dtype, stream);
}

attn_status attn_prefill_gqa_cached(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* start_pos, const int32_t* q_lens, void* out, int B, int S,
                                    int Hq, int Hkv, int head_dim, int T_max, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream) {
  if (!start_pos)
    return fail(ATTN_ERR_NULL, "attn_prefill_gqa_cached: start_pos must be non-NULL");
  return prefill_common("attn_prefill_gqa_cached", q, k_cache, v_cache, start_pos, q_lens, out, B, S, Hq, Hkv,
                        head_dim, T_max, softmax_scale, in_dtype, out_dtype, stream);
}

attn_status attn_prefill_gqa_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                                   const int32_t* start_pos, const int32_t* q_lens, void* out, int B, int S, int Hq,
                                   int Hkv, int head_dim, int page_size, int n_pages, int max_pages_per_seq,
                                   float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype, void* stream) {
  static const char* fn = "attn_prefill_gqa_paged";
  if (!start_pos) return fail(ATTN_ERR_NULL, "%s: start_pos must be non-NULL", fn);
  if (!block_table) return fail(ATTN_ERR_NULL, "%s: block_table must be non-NULL", fn);
  if (page_size <= 0 || n_pages <= 0 || max_pages_per_seq <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: page_size, n_pages and max_pages_per_seq must be positive (%d, %d, %d)", fn,
                page_size, n_pages, max_pages_per_seq);
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "%s: page_size * max_pages_per_seq too large", fn);
  if (page_size % 64 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size=%d must be a multiple of 64", fn, page_size);
  return prefill_common(fn, q, k_pages, v_pages, start_pos, q_lens, out, B, S, Hq, Hkv, head_dim,
                        page_size * max_pages_per_seq, softmax_scale, in_dtype, out_dtype, stream, nullptr, nullptr,
                        block_table, page_size, n_pages, max_pages_per_seq);
}

attn_status attn_prefill_gqa_cached_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                           void* v_cache, const int32_t* start_pos, const int32_t* q_lens, void* out,
                                           int B, int S, int Hq, int Hkv, int head_dim, int T_max,
                                           float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype,
                                           void* stream) {
  static const char* fn = "attn_prefill_gqa_cached_append";
  if (!start_pos) return fail(ATTN_ERR_NULL, "%s: start_pos must be non-NULL", fn);
  if (!k_new || !v_new) return fail(ATTN_ERR_NULL, "%s: k_new and v_new must be non-NULL", fn);
  return prefill_common(fn, q, k_cache, v_cache, start_pos, q_lens, out, B, S, Hq, Hkv, head_dim, T_max,
                        softmax_scale, in_dtype, out_dtype, stream, k_new, v_new);
}

attn_status attn_prefill_mla_causal(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                    const void* c_kv, const void* k_rope, const int32_t* start_pos,
                                    const int32_t* q_lens, void* out, int B, int S, int H, int nope_head_dim,
                                    int rope_dim, int v_head_dim, int kv_lora_rank, int T_max, float softmax_scale,
                                    attn_dtype in_dtype, attn_dtype out_dtype, void* stream) {
  static const char* fn = "attn_prefill_mla_causal";
  if (!q_nope || !q_rope || !w_uk || !w_uv || !c_kv || !k_rope || !out)
    return fail(ATTN_ERR_NULL, "%s: q_nope, q_rope, w_uk, w_uv, c_kv, k_rope and out must be non-NULL", fn);
  if (B <= 0 || S <= 0 || H <= 0 || nope_head_dim <= 0 || rope_dim <= 0 || v_head_dim <= 0 || kv_lora_rank <= 0 ||
      T_max <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d S=%d H=%d T_max=%d)", fn, B, S, H, T_max);
  if (B > kMaxGridYZ || H > kMaxGridYZ) return fail(ATTN_ERR_SHAPE, "%s: B and H must be <= %d", fn, kMaxGridYZ);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (in_dtype != ATTN_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: only bf16 inputs are built (MFMA path)", fn);
  if (!attn::mla_prefill_supported(nope_head_dim, rope_dim, v_head_dim, kv_lora_rank))
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s: widths nope=%d rope=%d v=%d kv_lora_rank=%d are not built (built: 96, 48, 96, 128)", fn,
                nope_head_dim, rope_dim, v_head_dim, kv_lora_rank);
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(c_kv) ||
      !aligned16(k_rope) || !aligned16(out))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: every tensor must be 16-byte aligned", fn);
  attn::MlaPrefillArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.start_pos = start_pos;
  a.q_lens = q_lens;
  a.out = out;
  a.B = B;
  a.S = S;
  a.H = H;
  a.dn = nope_head_dim;
  a.dR = rope_dim;
  a.dv = v_head_dim;
  a.r = kv_lora_rank;
  a.T_kv = T_max;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)(nope_head_dim + rope_dim));
  a.scale_log2e = scale * kLog2e;
  a.out_bf16 = out_dtype == ATTN_BF16;
  return hip_status(attn::launch_mla_prefill(a, static_cast<hipStream_t>(stream)), fn);
}

attn_status attn_rope_append(void* q, void* k_new, void* k_cache, const void* x_new, void* x_cache,
                             const int32_t* start_pos, const int32_t* n_new, int B, int S, int Hq, int Hk,
                             int rope_dim, int x_row_bytes, int T_max, float rope_base, attn_dtype dtype,
                             void* stream) {
  static const char* fn = "attn_rope_append";
  if (!k_new) return fail(ATTN_ERR_NULL, "%s: k_new must be non-NULL", fn);
  if (B <= 0 || S <= 0 || Hk <= 0 || rope_dim <= 0 || x_row_bytes < 0 || (q && Hq <= 0))
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d S=%d Hq=%d Hk=%d rope_dim=%d x_row_bytes=%d)", fn,
                B, S, Hq, Hk, rope_dim, x_row_bytes);
  if ((k_cache || x_row_bytes > 0) && T_max <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: T_max must be positive when a cache is written (T_max=%d)", fn, T_max);
  if (x_row_bytes > 0 && (!x_new || !x_cache))
    return fail(ATTN_ERR_NULL, "%s: x_new and x_cache must be non-NULL when x_row_bytes > 0", fn);
  if (x_row_bytes > 0 && !k_cache)
    return fail(ATTN_ERR_NULL, "%s: x is written only together with k_cache", fn);
  if (!valid_dtype(dtype)) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (rope_dim % 8 != 0 || rope_dim > attn::rope_max_dim())
    return fail(ATTN_ERR_UNSUPPORTED, "%s: rope_dim=%d must be a multiple of 8 in [8, %d]", fn, rope_dim,
                attn::rope_max_dim());
  if (x_row_bytes % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: x_row_bytes=%d must be a multiple of 16", fn, x_row_bytes);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(k_cache) || !aligned16(x_new) || !aligned16(x_cache))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: buffers must be 16-byte aligned", fn);
  if (!(rope_base > 0.f) || !std::isfinite(rope_base))
    return fail(ATTN_ERR_SHAPE, "%s: rope_base must be positive and finite (got %g)", fn, (double)rope_base);
  attn::RopeAppendArgs a;
  a.q = q;
  a.k_new = k_new;
  a.k_cache = k_cache;
  a.x_new = x_row_bytes > 0 ? x_new : nullptr;
  a.x_cache = x_row_bytes > 0 ? x_cache : nullptr;
  a.start_pos = start_pos;
  a.n_new = n_new;
  a.B = B;
  a.S = S;
  a.Hq = q ? Hq : 0;
  a.Hk = Hk;
  a.d = rope_dim;
  a.x_row_bytes = x_row_bytes;
  a.T_max = T_max;
  a.log2_base = std::log2((double)rope_base);
  a.bf16 = dtype == ATTN_BF16;
  return hip_status(attn::launch_rope_append(a, static_cast<hipStream_t>(stream)), fn);
}

attn_status attn_cache_append(const void* new_a, void* cache_a, int row_bytes_a, const void* new_b, void* cache_b,
                              int row_bytes_b, const int32_t* start_pos, const int32_t* n_new, int B, int S,
                              int T_max, void* stream) {
  static const char* fn = "attn_cache_append";
  if (!new_a || !cache_a) return fail(ATTN_ERR_NULL, "%s: new_a and cache_a must be non-NULL", fn);
  if (B <= 0 || S <= 0 || T_max <= 0 || row_bytes_a <= 0 || row_bytes_b < 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d S=%d T_max=%d row_bytes_a=%d row_bytes_b=%d)", fn, B,
                S, T_max, row_bytes_a, row_bytes_b);
  if (B > kMaxGridYZ) return fail(ATTN_ERR_SHAPE, "%s: B must be <= %d", fn, kMaxGridYZ);
  if (row_bytes_a % 16 != 0 || row_bytes_b % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: row sizes must be multiples of 16 bytes (%d, %d)", fn, row_bytes_a,
                row_bytes_b);
  if (row_bytes_b > 0 && (!new_b || !cache_b))
    return fail(ATTN_ERR_NULL, "%s: new_b and cache_b must be non-NULL when row_bytes_b > 0", fn);
  if ((long long)(row_bytes_a + (long long)row_bytes_b) / 16 * S > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "%s: S * row bytes too large", fn);
  if (!aligned16(new_a) || !aligned16(cache_a) || (row_bytes_b > 0 && (!aligned16(new_b) || !aligned16(cache_b))))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: buffers must be 16-byte aligned", fn);
  attn::CacheAppendArgs a;
  a.new_a = new_a;
  a.cache_a = cache_a;
  a.new_b = row_bytes_b > 0 ? new_b : nullptr;
  a.cache_b = row_bytes_b > 0 ? cache_b : nullptr;
  a.start_pos = start_pos;
  a.n_new = n_new;
  a.row_bytes_a = row_bytes_a;
  a.row_bytes_b = row_bytes_b;
  a.B = B;
  a.S = S;
  a.T_max = T_max;
  return hip_status(attn::launch_cache_append(a, static_cast<hipStream_t>(stream)), fn);
}

size_t attn_decode_mla_workspace_bytes(int B, int H, int kv_lora_rank, int rope_dim, int T_max,
                                       int split_tokens) {
  if (B <= 0 || H <= 0 || kv_lora_rank <= 0 || rope_dim < 0 || T_max <= 0 || !valid_split(split_tokens))
    return 0;
  return mla_layout(B, H, kv_lora_rank, T_max, split_tokens).total;
}

int attn_decode_mla_supported(int H, int kv_lora_rank, int rope_dim, attn_dtype in_dtype) {
  return in_dtype == ATTN_BF16 && attn::mla_decode_supported(H, kv_lora_rank, rope_dim) ? 1 : 0;
}

namespace {

// Shared checks and launch of the MLA decode entry points.  c_new != null: a
// decode step that also takes the new token's latent row (attn_decode_mla_append);
// block_table != null: paged caches (attn_decode_mla_paged; c_kv and k_rope are
// page pools, T_max = page_size * table_stride).
attn_status mla_decode_common(const char* fn, const void* q_nope, const void* q_rope, const void* c_new,
                              const void* kr_new, const void* w_uk, const void* w_uv, const void* c_kv,
                              const void* k_rope, const int32_t* cache_lens, void* out, int B, int H,
                              int nope_head_dim, int rope_dim, int v_head_dim, int kv_lora_rank, int T_max,
                              float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const int32_t* block_table = nullptr, int page_size = 0, int n_pages = 0,
                              int table_stride = 0, bool c_fp8 = false, float c_scale = 1.f) {
  const bool append = c_new != nullptr;
  if (!q_nope || !q_rope || !w_uk || !w_uv || !c_kv || !k_rope || !cache_lens || !out)
    return fail(ATTN_ERR_NULL, "%s: all tensor pointers must be non-NULL", fn);
  if (B <= 0 || H <= 0 || nope_head_dim <= 0 || rope_dim <= 0 || v_head_dim <= 0 || kv_lora_rank <= 0 ||
      T_max <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: sizes must be positive (B=%d H=%d nope=%d rope=%d v=%d rank=%d T_max=%d)", fn,
                B, H, nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, T_max);
  if (B > kMaxGridYZ) return fail(ATTN_ERR_SHAPE, "%s: B must be <= %d", fn, kMaxGridYZ);
  if (nope_head_dim > 256 || nope_head_dim % 8 != 0 || v_head_dim > 256 || v_head_dim % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s: nope_head_dim must be a multiple of 8 and v_head_dim a multiple of 16, both up to 256 "
                "(got %d, %d)", fn, nope_head_dim, v_head_dim);
  if (!valid_split(split_tokens))
    return fail(ATTN_ERR_SHAPE, "%s: split_tokens=%d must be 0 or a multiple of 64 in [64, 65536]", fn,
                split_tokens);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(ATTN_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  if (!attn_decode_mla_supported(H, kv_lora_rank, rope_dim, in_dtype))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: H=%d kv_lora_rank=%d rope_dim=%d %s is not built", fn, H, kv_lora_rank,
                rope_dim, in_dtype == ATTN_BF16 ? "bf16" : "fp32");
  if (!aligned16(c_kv) || !aligned16(k_rope) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(out) ||
      (append && (!aligned16(c_new) || !aligned16(kr_new))))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: c_kv, k_rope, w_uk, w_uv, out (and the new rows) must be 16-byte aligned",
                fn);
  const MlaLayout lay = mla_layout(B, H, kv_lora_rank, T_max, split_tokens);
  if (block_table && lay.split / page_size + 2 > 128)
    return fail(ATTN_ERR_UNSUPPORTED,
                "%s: a chunk of %d positions spans more than 128 pages of %d; pass split_tokens of at most %d", fn,
                lay.split, page_size, 126 * page_size / 64 * 64);
  if (!workspace || workspace_bytes < lay.total)
    return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, lay.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(ATTN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  attn::MlaDecodeArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.lens = cache_lens;
  a.out = out;
  char* ws = static_cast<char*>(workspace);
  a.done = reinterpret_cast<unsigned*>(ws);
  a.o_part = reinterpret_cast<float*>(ws + lay.o_part_off);
  a.lse = reinterpret_cast<float*>(ws + lay.lse_off);
  a.B = B;
  a.H = H;
  a.dn = nope_head_dim;
  a.dR = rope_dim;
  a.dv = v_head_dim;
  a.r = kv_lora_rank;
  a.T_max = T_max;
  a.split = lay.split;
  a.n_splits = lay.n_splits;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)(nope_head_dim + rope_dim));
  a.scale_log2e = scale * kLog2e;
  a.out_bf16 = out_dtype == ATTN_BF16;
  a.append = append;
  a.c_new = c_new;
  a.kr_new = kr_new;
  a.c_cache = const_cast<void*>(c_kv);
  a.kr_cache = const_cast<void*>(k_rope);
  a.block_table = block_table;
  a.page_size = page_size;
  a.n_pages = n_pages;
  a.table_stride = table_stride;
  a.c_fp8 = c_fp8;
  a.c_scale = c_scale;
  return hip_status(attn::launch_mla_decode(a, static_cast<hipStream_t>(stream)), fn);
}

}  // namespace

attn_status attn_decode_mla_absorbed(const void* q_nope, const void* q_rope, const void* w_uk,
                                     const void* w_uv, const void* c_kv, const void* k_rope,
                                     const int32_t* cache_lens, void* out, int B, int H,
                                     int nope_head_dim, int rope_dim, int v_head_dim,
                                     int kv_lora_rank, int T_max, float softmax_scale,
                                     attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_common("attn_decode_mla_absorbed", q_nope, q_rope, nullptr, nullptr, w_uk, w_uv, c_kv, k_rope,
                           cache_lens, out, B, H, nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, T_max,
                           softmax_scale, in_dtype, out_dtype, split_tokens, workspace, workspace_bytes, stream);
}

attn_status attn_decode_mla_paged(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                  const void* c_pages, const void* k_rope_pages, const int32_t* block_table,
                                  const int32_t* cache_lens, void* out, int B, int H, int nope_head_dim, int rope_dim,
                                  int v_head_dim, int kv_lora_rank, int page_size, int n_pages, int max_pages_per_seq,
                                  float softmax_scale, attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_mla_paged";
  if (!block_table) return fail(ATTN_ERR_NULL, "%s: block_table must be non-NULL", fn);
  if (page_size <= 0 || n_pages <= 0 || max_pages_per_seq <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: page_size, n_pages and max_pages_per_seq must be positive (%d, %d, %d)", fn,
                page_size, n_pages, max_pages_per_seq);
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "%s: page_size * max_pages_per_seq too large", fn);
  if (page_size % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size=%d must be a multiple of 16", fn, page_size);
  return mla_decode_common(fn, q_nope, q_rope, nullptr, nullptr, w_uk, w_uv, c_pages, k_rope_pages, cache_lens, out, B,
                           H, nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, page_size * max_pages_per_seq,
                           softmax_scale, in_dtype, out_dtype, split_tokens, workspace, workspace_bytes, stream,
                           block_table, page_size, n_pages, max_pages_per_seq);
}

attn_status attn_decode_mla_fp8kv(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                  const void* c_kv, float c_scale, const void* k_rope, const int32_t* cache_lens,
                                  void* out, int B, int H, int nope_head_dim, int rope_dim, int v_head_dim,
                                  int kv_lora_rank, int T_max, float softmax_scale, attn_dtype out_dtype,
                                  int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_mla_fp8kv";
  if (!(c_scale > 0.f) || !std::isfinite(c_scale))
    return fail(ATTN_ERR_SHAPE, "%s: c_scale must be positive and finite (got %g)", fn, (double)c_scale);
  return mla_decode_common(fn, q_nope, q_rope, nullptr, nullptr, w_uk, w_uv, c_kv, k_rope, cache_lens, out, B, H,
                           nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, T_max, softmax_scale, ATTN_BF16,
                           out_dtype, split_tokens, workspace, workspace_bytes, stream, nullptr, 0, 0, 0, true,
                           c_scale);
}

attn_status attn_decode_mla_paged_fp8kv(const void* q_nope, const void* q_rope, const void* w_uk, const void* w_uv,
                                        const void* c_pages, float c_scale, const void* k_rope_pages,
                                        const int32_t* block_table, const int32_t* cache_lens, void* out, int B, int H,
                                        int nope_head_dim, int rope_dim, int v_head_dim, int kv_lora_rank,
                                        int page_size, int n_pages, int max_pages_per_seq, float softmax_scale,
                                        attn_dtype out_dtype, int split_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  static const char* fn = "attn_decode_mla_paged_fp8kv";
  if (!block_table) return fail(ATTN_ERR_NULL, "%s: block_table must be non-NULL", fn);
  if (!(c_scale > 0.f) || !std::isfinite(c_scale))
    return fail(ATTN_ERR_SHAPE, "%s: c_scale must be positive and finite (got %g)", fn, (double)c_scale);
  if (page_size <= 0 || n_pages <= 0 || max_pages_per_seq <= 0)
    return fail(ATTN_ERR_SHAPE, "%s: page_size, n_pages and max_pages_per_seq must be positive (%d, %d, %d)", fn,
                page_size, n_pages, max_pages_per_seq);
  if ((long long)page_size * max_pages_per_seq > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "%s: page_size * max_pages_per_seq too large", fn);
  if (page_size % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size=%d must be a multiple of 16", fn, page_size);
  return mla_decode_common(fn, q_nope, q_rope, nullptr, nullptr, w_uk, w_uv, c_pages, k_rope_pages, cache_lens, out, B,
                           H, nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, page_size * max_pages_per_seq,
                           softmax_scale, ATTN_BF16, out_dtype, split_tokens, workspace, workspace_bytes, stream,
                           block_table, page_size, n_pages, max_pages_per_seq, true, c_scale);
}

attn_status attn_decode_mla_append(const void* q_nope, const void* q_rope, const void* c_new, const void* k_rope_new,
                                   const void* w_uk, const void* w_uv, void* c_kv, void* k_rope,
                                   const int32_t* cache_lens, void* out, int B, int H, int nope_head_dim,
                                   int rope_dim, int v_head_dim, int kv_lora_rank, int T_max, float softmax_scale,
                                   attn_dtype in_dtype, attn_dtype out_dtype, int split_tokens, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!c_new || !k_rope_new)
    return fail(ATTN_ERR_NULL, "attn_decode_mla_append: c_new and k_rope_new must be non-NULL");
  return mla_decode_common("attn_decode_mla_append", q_nope, q_rope, c_new, k_rope_new, w_uk, w_uv, c_kv, k_rope,
                           cache_lens, out, B, H, nope_head_dim, rope_dim, v_head_dim, kv_lora_rank, T_max,
                           softmax_scale, in_dtype, out_dtype, split_tokens, workspace, workspace_bytes, stream);
}

}  // extern "C"
