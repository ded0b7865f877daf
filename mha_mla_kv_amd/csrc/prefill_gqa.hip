// Causal GQA prefill on bf16 MFMA for gfx950.
//
// What is computed: out[b,i,h] = sum_{j<=i} softmax_j(scale q[b,i,h].k[b,j,g]) v[b,j,g]
// with g = floor(h / n_rep) -- Attention.forward of the "模型架构｜MQA & GQA 调研"
// page (code section) with start_pos = 0 and its additive causal mask, i.e. the
// scaled_dot_product_attention(is_causal=True) call in the MultiHeadLatentAttention
// listing of the qqstock DeepSeek MLA article.  P is rounded to bf16 before the
// PV product, as the page's softmax(...).type_as(xq) does.
//
// How (not from the pages; designed for CDNA4):
//  * One workgroup = 4 waves = a tile of 128 query rows of one (head, sequence);
//    each wave owns 32 rows.  The linear workgroup id is mapped so that all heads
//    of one KV group of one sequence run on the same XCD (one L2), heaviest
//    q-tiles (most keys) first.
//  * K/V tiles of 64 keys go HBM -> LDS with global_load_lds_dwordx4 (no staging
//    registers, no LDS write instructions), double-buffered, one barrier per
//    tile.  Key rows are stored unpadded with their 16-byte chunks XOR-swizzled
//    by key, which keeps the 16-byte K operand reads and the transposed V reads
//    free of bank conflicts.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a 32-key K block is the A operand,
//    the wave's Q^T is the B operand, held in registers for the whole kernel.  The
//    accumulator gives each lane one query row (lane % 32) and 16 keys.
//  * O^T += V^T P^T: P stays in the accumulator layout and is the B operand after
//    a key permutation shared with the A operand; V^T comes from the row-major V
//    tile through ds_read_b64_tr_b16.
//  * Online softmax in base 2, scale and max folded into one FMA per score.  The
//    reference max only moves (and O, l are rescaled) when a tile's max exceeds
//    it by more than 2^8: probabilities then stay below 256, far inside bf16 and
//    fp32 range, and most tiles skip the O rescale.
//  * A wave skips tiles entirely above its diagonal; only diagonal tiles mask.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kBM = 128;              // query rows per workgroup
constexpr int kBN = 64;               // keys per tile
constexpr int kWaves = 4;             // 32 rows each
constexpr float kRescaleSlack = 8.f;  // log2 units the reference max may trail the true max

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap_b32 a, b exchanges the upper half of a with the lower half of
// b (gfx950): with a and b both holding x, lane l ends up with x_l and x_(l^32).
// Inline asm (both operands read and written) because the compiler builtin for
// this instruction loses its second result; the s_nop pairs cover the
// VALU-write -> permlane-read hazard.
__device__ __forceinline__ float2 pair_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float max_xor32(float x) { const float2 p = pair_xor32(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor32(float x) { const float2 p = pair_xor32(x); return p.x + p.y; }

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: lane i of a 16-lane group points at row T0 + i/4, columns
// 4(i%4).. of a row-major [key][dim] block; lane j receives keys T0..T0+3 of
// column j.
__device__ __forceinline__ u16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}

// 16-byte chunk c of key row r sits at chunk position c ^ swz(r).  Over 8
// consecutive keys swz takes 8 distinct values (K operand reads: 8 lanes of one
// chunk index per LDS cycle), and over 4 consecutive keys an even-aligned chunk
// pair lands on 4 distinct pairs (transposed V reads: 4 keys x 2 chunks per cycle).
__device__ __forceinline__ int swz(int r) { return ((r << 1) + (r >> 2)) & 7; }

// HBM -> LDS copy of one 64-key tile of K or V (D/8 chunks per key); every lane
// of an instruction writes its 16 bytes at LDS base + 16 * lane, so the lane
// fetches the chunk that belongs at that position.  Keys past the end repeat
// the last key (masked by causality).
template <int D>
__device__ __forceinline__ void load_tile_lds(u16* lds_tile, const u16* src, size_t row_stride, int key0, int S,
                                              int wave, int lane) {
  constexpr int kChunks = D / 8;
  constexpr int kRowsPerInst = 64 / kChunks;
  constexpr int kInstPerWave = kBN / kRowsPerInst / kWaves;
#pragma unroll
  for (int i = 0; i < kInstPerWave; ++i) {
    const int r0 = (wave * kInstPerWave + i) * kRowsPerInst;
    const int r = r0 + lane / kChunks;
    const int p = lane % kChunks;
    const int key = min(key0 + r, S - 1);
    const u16* g = src + (size_t)key * row_stride + 8 * (p ^ swz(r));
    __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)(lds_tile + r0 * D),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Workgroup id -> (q-tile, head, sequence).  Workgroups are dealt to the 8 XCDs
// round-robin by id.  When the (sequence, KV group) pairs split evenly over the
// XCDs, each XCD gets whole groups, so a group's K/V is read through one L2;
// within an XCD the heaviest q-tiles go first.  Otherwise: heaviest q-tile
// first, heads fastest.
struct Tile {
  int qt, h, b;
};
__device__ __forceinline__ Tile map_tile(const PrefillArgs& a, int id) {
  const int n_qt = (a.S + kBM - 1) / kBM;
  const int groups = a.B * a.Hkv;
  Tile t;
  if (groups % 8 == 0) {
    const int xcd = id & 7, slot = id >> 3;
    const int gpx = groups / 8;
    const int per_rank = gpx * a.n_rep;
    const int rank = slot / per_rank, rem = slot - rank * per_rank;
    const int grp = xcd * gpx + rem / a.n_rep;
    t.qt = n_qt - 1 - rank;
    t.b = grp / a.Hkv;
    t.h = (grp - t.b * a.Hkv) * a.n_rep + rem % a.n_rep;
  } else {
    const int per_rank = a.B * a.Hq;
    const int rank = id / per_rank, rem = id - rank * per_rank;
    t.qt = n_qt - 1 - rank;
    t.b = rem / a.Hq;
    t.h = rem - t.b * a.Hq;
  }
  return t;
}

// Running state of one wave: O^T accumulators, reference max, partial row sum.
template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m, lsum;
};

// One 64-key tile: issue the copies of tile kt+1 into (kn, vn) if there is one,
// consume tile kt from (kc, vc) if some row of the wave sees it, then wait for
// the copies and meet at the barrier.  The four buffers are distinct LDS
// variables addressed directly, so the compiler can tell the copies in flight
// from the reads of the current tile and does not wait for them before reading.
template <int D>
__device__ __forceinline__ void tile_step(RowState<D>& st, const u16* kc, const u16* vc, u16* kn, u16* vn,
                                          const bf16x8 (&qop)[D / 16], int kt, int n_kt, int last_kt, int row0,
                                          int my_row, const u16* kp, const u16* vp, size_t kv_row, int S,
                                          float c_log2, int wave, int lane) {
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  const int ln = lane & 31, h2 = lane >> 5;
  if (kt + 1 < n_kt) {  // (kn, vn) were released by the last barrier
    load_tile_lds<D>(kn, kp, kv_row, (kt + 1) * kBN, S, wave, lane);
    load_tile_lds<D>(vn, vp, kv_row, (kt + 1) * kBN, S, wave, lane);
  }
  if (kt <= last_kt) {
    const int kv0 = kt * kBN;
    // S^T blocks: lane holds S^T[key kv0 + 32j + 8(i/4) + 4h2 + i%4][row ln]
    f32x16 sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      const int key = 32 * j + ln;
      const u16* kr = kc + key * D;
      const int sw = swz(key);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr + 8 * ((2 * c + h2) ^ sw)));
        acc = mfma_32x32x16(kop, qop[c], acc);
      }
      sc[j] = acc;
    }
    if (kv0 + kBN - 1 > row0) {  // the tile reaches above the diagonal of some row
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + 32 * j + 8 * (i >> 2) + 4 * h2 + (i & 3);
          sc[j][i] = key <= my_row ? sc[j][i] : kNegInf;
        }
    }
    float mr = kNegInf;  // raw row max; the scale is positive
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) mr = fmaxf(mr, sc[j][i]);
    const float mt = max_xor32(mr) * c_log2;
    // key 0 is visible to every row, so tile 0 always sets a finite reference
    if (__builtin_amdgcn_ballot_w64(mt > st.m + kRescaleSlack) != 0) {
      const float mn = fmaxf(st.m, mt);
      const float alpha = exp2_fast(st.m - mn);
      st.m = mn;
      st.lsum *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d) st.o[d] *= alpha;
    }
    // P^T operand of PV step v: S^T block v/2, values 8(v%2)..+8
    bf16x8 pop[4];
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p = exp2_fast(fmaf(sc[v >> 1][8 * (v & 1) + jj], c_log2, -st.m));
        ps += p;
        pop[v][jj] = (__bf16)p;
      }
    st.lsum += ps;
    // O^T[dims 32d..][rows] += V^T P^T.  Step v covers keys 16v + 4h2 + (0..3) and
    // 16v + 8 + 4h2 + (0..3) of the tile; 16-lane group (g16, h2) of a transposed
    // read points at key 16v + 4h2 + (i16 >> 2) (+8), dims 32d + 16g16 + 4(i16 & 3).
    const int g16 = (lane >> 4) & 1, i16 = lane & 15;
    const int v_chunk = 2 * g16 + ((i16 & 3) >> 1);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int klo = 16 * v + 4 * h2 + (i16 >> 2), khi = klo + 8;
      const u16* plo = vc + klo * D + 4 * (i16 & 1);
      const u16* phi = vc + khi * D + 4 * (i16 & 1);
      const int swlo = swz(klo), swhi = swz(khi);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        const u16x4 lo = lds_read_tr16(plo + 8 * ((4 * d + v_chunk) ^ swlo));
        const u16x4 hi = lds_read_tr16(phi + 8 * ((4 * d + v_chunk) ^ swhi));
        const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        st.o[d] = mfma_32x32x16(__builtin_bit_cast(bf16x8, av), pop[v], st.o[d]);
      }
    }
  }
  wait_vmem();      // this thread's copies of tile kt+1 have landed
  __syncthreads();  // ... and everyone's; nobody reads tile kt any more
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_causal(PrefillArgs a) {
  static_assert(D % 32 == 0 && D <= 128, "head_dim");
  static_assert(kBM == 32 * kWaves, "one 32-row slice per wave");
  constexpr int KC = D / 16;
  constexpr int DB = D / 32;
  constexpr int kTile = kBN * D;
  __shared__ __attribute__((aligned(1024))) u16 k0[kTile];
  __shared__ __attribute__((aligned(1024))) u16 k1[kTile];
  __shared__ __attribute__((aligned(1024))) u16 v0[kTile];
  __shared__ __attribute__((aligned(1024))) u16 v1[kTile];

  const Tile tl = map_tile(a, blockIdx.x);
  const int h = tl.h, b = tl.b;
  const int g = h / a.n_rep;
  const int q0 = tl.qt * kBM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, h2 = lane >> 5;

  const size_t q_row = (size_t)a.Hq * D;
  const size_t kv_row = (size_t)a.Hkv * D;
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)b * a.S * a.Hq + h) * D;
  const u16* kp = static_cast<const u16*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * D;
  const u16* vp = static_cast<const u16*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * D;

  // keys needed by the workgroup: [0, min(S, q0 + BM)); tiles 0..last_kt are
  // visible to some row of this wave
  const int kv_end = min(a.S, q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;
  const int row0 = q0 + wave * 32;
  const int last_kt = min(n_kt - 1, (row0 + 31) / kBN);
  const int my_row = row0 + ln;

  load_tile_lds<D>(k0, kp, kv_row, 0, a.S, wave, lane);
  load_tile_lds<D>(v0, vp, kv_row, 0, a.S, wave, lane);

  // Q^T as the B operand: lane holds Q[row ln][16c + 8h2 ..+8]
  bf16x8 qop[KC];
  {
    const u16* qr = qp + (size_t)min(my_row, a.S - 1) * q_row + 8 * h2;
#pragma unroll
    for (int c = 0; c < KC; ++c) qop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qr + 16 * c));
  }

  RowState<D> st;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[d][i] = 0.f;
  st.m = kNegInf;
  st.lsum = 0.f;
  const float c_log2 = a.scale_log2e;

  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile_step<D>(st, k0, v0, k1, v1, qop, kt, n_kt, last_kt, row0, my_row, kp, vp, kv_row, a.S, c_log2, wave, lane);
    if (kt + 1 < n_kt)
      tile_step<D>(st, k1, v1, k0, v0, qop, kt + 1, n_kt, last_kt, row0, my_row, kp, vp, kv_row, a.S, c_log2, wave,
                   lane);
  }

  // normalise and store: lane holds O^T[dims 32d + 8(i/4) + 4h2 + (i%4)][row ln]
  const float lsum = sum_xor32(st.lsum);
  if (my_row < a.S) {
    const float inv = 1.f / lsum;
    const size_t orow = ((size_t)b * a.S + my_row) * a.Hq + h;
    if (a.out_bf16) {
      u16* op = static_cast<u16*>(a.out) + orow * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(u16, (__bf16)(st.o[d][4 * q4 + e] * inv));
          *reinterpret_cast<u16x4*>(op + 32 * d + 8 * q4 + 4 * h2) = w;
        }
    } else {
      float* op = static_cast<float*>(a.out) + orow * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(op + 32 * d + 8 * q4 + 4 * h2) =
              make_float4(st.o[d][4 * q4] * inv, st.o[d][4 * q4 + 1] * inv, st.o[d][4 * q4 + 2] * inv,
                          st.o[d][4 * q4 + 3] * inv);
    }
  }
}

}  // namespace

bool prefill_supported(int D) { return D == 64 || D == 128; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (!prefill_supported(a.D)) return hipErrorInvalidValue;
  const long long wgs = (long long)((a.S + kBM - 1) / kBM) * a.Hq * a.B;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  if (a.D == 128) hipLaunchKernelGGL(prefill_causal<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(prefill_causal<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
