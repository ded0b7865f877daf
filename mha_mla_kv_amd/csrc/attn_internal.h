// Internal interface between the C-ABI host layer (attn_api.cpp) and the HIP
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

// Tokens per MFMA tile processed by one wave in the decode kernels.
constexpr int kDecodeTileTokens = 32;
// Waves per decode workgroup.
constexpr int kDecodeWaves = 4;

// Largest batch the queue schedule of the decode kernels plans for (its
// per-sequence prefix of chunk counts lives in LDS); larger batches launch one
// workgroup per unit.
constexpr int kQueueMaxB = 1024;

struct GqaDecodeArgs {
  const void* q;          // [B, Hq, D]
  const void* k;          // [B, T_max, Hkv, D]
  const void* v;          // [B, T_max, Hkv, D]
  const int32_t* lens;    // [B]
  void* out;              // [B, Hq, D]
  unsigned* queue;        // work-queue counter, zero between calls (workspace)
  float* lse;             // [B, Hkv, n_chunks, n_rep] log2-sum-exp of each unit    (workspace)
  float* o_part;          // [B, Hkv, n_chunks, n_rep, D] normalised unit outputs  (workspace)
  int B, Hq, Hkv, D, T_max, n_rep;
  int chunk;              // positions per work unit (multiple of 64)
  int n_chunks;           // ceil(T_max / chunk)
  int use_queue;          // 1: resident workgroups take units from the queue; 0: one workgroup per unit
  int big_units;          // queue: 1 to hand out most of each sequence in units of four blocks
  int grid_wgs;           // queue: most workgroups to launch
  int cus;                // queue: compute units of the device
  float scale_log2e;      // softmax scale * log2(e)
  int in_bf16;            // 1: bf16 inputs, 0: fp32 inputs
  int out_bf16;           // 1: bf16 output, 0: fp32 output
  // decode step with the new token's K/V (append != 0): every unit writes a
  // partial, and the merge adds the new token and writes it to the cache at
  // position lens[b] (when lens[b] < T_max)
  int append;
  const void* k_new;      // [B, Hkv, D]
  const void* v_new;      // [B, Hkv, D]
  void* k_cache;          // the k array, written at the new position
  void* v_cache;          // the v array
  // caches of OCP FP8 E4M3 values (kv_fp8 != 0): value = v_scale * code for V;
  // the K scale is folded into scale_log2e
  int kv_fp8;
  float v_scale;
  // paged caches (block_table != null): k and v are pools of n_pages pages of
  // page_size positions ([n_pages, page_size, Hkv, D]); position t of sequence
  // b sits in page block_table[b * table_stride + t / page_size] (clamped to
  // [0, n_pages)), at row t % page_size.  page_size is a multiple of 32 and a
  // unit spans at most 128 pages.
  const int32_t* block_table = nullptr;
  int page_size = 0;
  int table_stride = 0;
  int n_pages = 0;
  // caches of signed 4-bit codes (kv_int4 != 0), head-major: [B, Hkv, T_max, D/2]
  // bytes, code 2i in the low nibble of byte i; value = scale of the row * code
  int kv_int4 = 0;
  const float* k_scales = nullptr;  // [B, Hkv, T_max]
  const float* v_scales = nullptr;  // [B, Hkv, T_max]
};

struct PrefillArgs {
  const void* q;                // [B, S, Hq, D] bf16 (the new tokens)
  const void* k;                // [B, T_kv, Hkv, D] bf16
  const void* v;                // [B, T_kv, Hkv, D] bf16
  const int32_t* start_pos;     // [B] cached prefix length, or null: 0
  const int32_t* q_lens;        // [B] new tokens per sequence, or null: S
  void* out;                    // [B, S, Hq, D]
  int B, S, Hq, Hkv, D, n_rep;
  int T_kv;                     // key rows per sequence in k and v (S without a prefix)
  float scale_log2e;
  int out_bf16;
  // new rows in their own arrays (k_new != null, start_pos required): keys at
  // positions P.. are read from them, and they are written into k and v at P..
  const void* k_new = nullptr;  // [B, S, Hkv, D] bf16
  const void* v_new = nullptr;  // [B, S, Hkv, D] bf16
  // paged cache (block_table != null, start_pos required, no k_new): k and v are
  // pools [n_pages, page_size, Hkv, D]; position t of sequence b is row
  // t % page_size of page block_table[b * table_stride + t / page_size]
  // (clamped to [0, n_pages)); page_size a multiple of 64; T_kv = page_size * table_stride
  const int32_t* block_table = nullptr;
  int page_size = 0;
  int table_stride = 0;
  int n_pages = 0;
};

struct MlaPrefillArgs {
  const void* q_nope;           // [B, S, H, dn] bf16 (the new tokens)
  const void* q_rope;           // [B, S, H, dR] bf16
  const void* w_uk;             // [H, dn, r] bf16
  const void* w_uv;             // [H, dv, r] bf16
  const void* c_kv;             // [B, T_kv, r] bf16
  const void* k_rope;           // [B, T_kv, dR] bf16
  const int32_t* start_pos;     // [B] cached prefix length, or null: 0
  const int32_t* q_lens;        // [B] new tokens per sequence, or null: S
  void* out;                    // [B, S, H, dv]
  int B, S, H, dn, dR, dv, r, T_kv;
  float scale_log2e;
  int out_bf16;
};

struct CacheAppendArgs {
  const void* new_a;            // [B, S, row_bytes_a]
  void* cache_a;                // [B, T_max, row_bytes_a]
  const void* new_b;            // [B, S, row_bytes_b] (row_bytes_b 0: no second pair)
  void* cache_b;                // [B, T_max, row_bytes_b]
  const int32_t* start_pos;     // [B], or null: 0
  const int32_t* n_new;         // [B], or null: S
  int row_bytes_a, row_bytes_b; // multiples of 16
  int B, S, T_max;
};

struct MlaDecodeArgs {
  const void* q_nope;   // [B, H, dn]
  const void* q_rope;   // [B, H, dR]
  const void* w_uk;     // [H, dn, r]
  const void* w_uv;     // [H, dv, r]
  const void* c_kv;     // [B, T_max, r]
  const void* k_rope;   // [B, T_max, dR]
  const int32_t* lens;  // [B]
  void* out;            // [B, H, dv]
  unsigned* done;       // [B] chunks of the sequence finished so far, zero between calls (workspace)
  float* o_part;        // [B, n_splits, H, r]  normalised chunk outputs in the latent space (workspace)
  float* lse;           // [B, n_splits, H]     their log2-sum-exps (workspace)
  int B, H, dn, dR, dv, r, T_max;
  int split, n_splits;
  float scale_log2e;
  int out_bf16;
  // decode step with the new token (append != 0): its latent row and rotated
  // key part are merged as one more partial by the workgroup that finishes the
  // sequence, which then writes them into the caches at row lens[b] (when
  // lens[b] < T_max); the cache pass reads only rows below lens[b]
  int append;
  const void* c_new;    // [B, r]
  const void* kr_new;   // [B, dR]
  void* c_cache;        // the c_kv array, written at the new position
  void* kr_cache;       // the k_rope array
  // paged caches (block_table != null, no append): c_kv and k_rope are pools of
  // n_pages pages of page_size positions ([n_pages, page_size, r] and
  // [n_pages, page_size, dR]); position t of sequence b sits in page
  // block_table[b * table_stride + t / page_size] (clamped to [0, n_pages)), at
  // row t % page_size.  page_size is a multiple of 16 and a chunk spans at most
  // 128 pages.
  const int32_t* block_table = nullptr;
  int page_size = 0;
  int table_stride = 0;
  int n_pages = 0;
  // latent cache of OCP FP8 E4M3 codes (c_fp8 != 0; not paged, no append):
  // c_kv holds [B, T_max, r] bytes, value = c_scale * code; k_rope stays bf16
  int c_fp8 = 0;
  float c_scale = 1.f;
};

struct RopeAppendArgs {
  void* q;                      // [B, S, Hq, d] rotated in place, or null
  const void* k_new;            // [B, S, Hk, d]
  void* k_cache;                // [B, T_max, Hk, d] written at the positions, or null: k_new rotated in place
  const void* x_new;            // [B, S, x_row_bytes] copied as is (x_row_bytes 0: none)
  void* x_cache;                // [B, T_max, x_row_bytes]
  const int32_t* start_pos;     // [B], or null: 0
  const int32_t* n_new;         // [B], or null: S
  int B, S, Hq, Hk, d, x_row_bytes, T_max;
  double log2_base;             // log2 of the rope base
  int bf16;                     // 1: bf16 q and k, 0: fp32
};

// Each launcher validates nothing (the host layer has done it) and returns the
// HIP status of its launches.  Returns hipErrorInvalidValue for an
// unsupported template combination (the host layer checks *_supported first).
bool gqa_decode_supported(int D, int n_rep, int in_bf16);
hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t stream);

bool prefill_supported(int D);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

bool mla_prefill_supported(int dn, int dR, int dv, int r);
hipError_t launch_mla_prefill(const MlaPrefillArgs& a, hipStream_t stream);

hipError_t launch_cache_append(const CacheAppendArgs& a, hipStream_t stream);

int rope_max_dim();
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t stream);

bool mla_decode_supported(int H, int r, int dR);
hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t stream);

// The device-resident scratch of the allocation-free decode (decode_gqa.hip):
// its address on the current device (looked up once per device, then cached),
// and a launch that zeroes its work-queue counter (the first 4 bytes).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_clear_queue(unsigned* queue, hipStream_t stream);

}  // namespace attn
