// Split-K ("flash-decode") GQA / MQA / MHA decode for gfx950.
//
// What is computed: for every sequence b and query head h of KV group
// g = floor(h / n_rep), out[b,h] = softmax_t(scale q[b,h].K[b,t,g]) V[b,t,g]
// over the cached positions t < L_b.  This is the score / fp32 softmax /
// weighted-sum core of Attention.forward in the code section of the
// "模型架构｜MQA & GQA 调研" page for a single new query token, with the
// contiguous query-head grouping its repeat_kv expansion defines.
//
// How (not from the pages; designed for CDNA4):
//  * Work is cut into "pieces": a range of cached positions of one (sequence,
//    KV head).  A workgroup streams a piece's K and V rows from HBM exactly once
//    and applies them to all n_rep query heads of the group -- the repeat_kv
//    copies are never made.  Its four waves take interleaved 32-token tiles.
//  * Two schedules.  Fixed: chunks of `split` positions, grid (Hkv, chunks, B).
//    Balanced (default): every workgroup derives the same plan from cache_lens
//    on the device and takes an equal share of all cached (position, KV head)
//    rows, so ragged lengths leave no tail of idle compute units.
//  * bf16 path: scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the
//    tile's tokens as M and (padded) query heads as N, so the K tile is the A
//    operand and is loaded straight from HBM with one 16-byte load per lane per
//    32 dims.  P stays in the accumulator layout and becomes the B operand of
//    O^T += V^T P^T after a token permutation that both operands share.  V is
//    staged row-major in LDS (one private region per wave, 16-byte writes) and
//    read back transposed with ds_read_b64_tr_b16.
//  * fp32 path (VALU): 16 lanes cover one token's row (head_dim/16 elements
//    each); dot products are reduced inside the 16-lane DPP row.
//  * Online softmax in base 2 (scale * log2 e folded in, v_exp_f32).  A piece
//    that covers its whole sequence writes the output directly.  Otherwise it
//    writes a normalised partial and its log2-sum-exp (cache-bypassing stores),
//    then bumps the segment's completion counter; the workgroup that completes
//    the segment merges all its pieces and resets the counter to 0.
//  * Positions at or beyond L_b are never read: a tile's row index is clamped
//    to the piece end - 1 and scores past the piece end are masked to -inf.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the four 16-lane rows of a wave without LDS traffic.
// v_permlane16_swap_b32 a, b exchanges rows 1 and 3 of a with rows 0 and 2 of b;
// v_permlane32_swap_b32 a, b the upper half of a with the lower half of b
// (gfx950).  With a and b both holding x, lane l ends up with x_l and x_(l^16)
// (resp. x_(l^32)) in a and b.  Written as inline asm (both operands read and
// written) because the compiler builtin for these instructions loses its second
// result; the s_nop pairs cover the VALU-write -> permlane-read hazard.
__device__ __forceinline__ float2 pair_xor16(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float2 pair_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float max_xor16(float x) { const float2 p = pair_xor16(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max_xor32(float x) { const float2 p = pair_xor32(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor16(float x) { const float2 p = pair_xor16(x); return p.x + p.y; }
__device__ __forceinline__ float sum_xor32(float x) { const float2 p = pair_xor32(x); return p.x + p.y; }

// exp2(m - M) that is 0 (not NaN) when m is -inf.
__device__ __forceinline__ float rescale(float m, float M) { return m == kNegInf ? 0.f : exp2_fast(m - M); }

__device__ __forceinline__ bf16x8 load_bf16x8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (gfx950): within each 16-lane group, lane i supplies the
// address of 4 consecutive 16-bit elements M[i][0..3]; lane j receives
// M[j/4 + 4k][j%4] for k = 0..3.  With lane i pointing at row (T0 + i/4),
// columns 4(i%4)..4(i%4)+3 of a row-major [token][dim] tile, lane j receives
// the 4 tokens T0..T0+3 of column j: a transposed read.
__device__ __forceinline__ u16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}

// Orders this wave's LDS writes before its later LDS reads (and vice versa):
// waits for outstanding LDS operations and stops the compiler moving LDS
// accesses across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));  // quad xor 1
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));  // quad xor 2
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, true)); // row_ror 4
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true)); // row_ror 8
  return x;
}

__device__ __forceinline__ int clamp_len(int L, int T_max) { return L < 0 ? 0 : (L > T_max ? T_max : L); }

// Values that are the same in every lane (read from LDS or computed from such
// values), moved to scalar registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned long long uniform(unsigned long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// ---------------------------------------------------------------------------
// Schedule

struct Piece {
  int b, g;         // sequence and KV head
  int t0, t1;       // positions [t0, t1) of the sequence
  int slot;         // partial-result slot of this piece
  int first_slot;   // slots of the segment's pieces: first_slot .. first_slot + count - 1
  int count;        // number of pieces of the segment (b, g)
};

// Per-workgroup shared state of the schedule and of the piece epilogue.
struct SchedShared {
  int b0;                     // balanced: first sequence of this workgroup's range
  int last;                   // this workgroup completed the current segment
  float m[64], inv[64];       // merge: per-head max and 1/sum of chunk weights
};

// Balanced schedule.  Rows of (position, KV head) are numbered sequence-major,
// then KV head, then position: segment (b, g) covers [Hkv*P_b + g*N_b, .. + N_b)
// where P_b = sum_{b'<b} N_b'.  Workgroup w of G takes [w*N/G, (w+1)*N/G) of the
// N = Hkv*P_B rows.  The piece of workgroup w in segment s gets slot w + s
// (unique: moving to the next piece increments w or s), so the pieces of segment
// s use the consecutive slots w_first + s .. w_last + s.
struct Balanced {
  unsigned N;  // total rows (< 2^31: checked on the host)
  int G;       // workgroups that take work
  __device__ unsigned start(int w) const { return (unsigned)(((unsigned long long)w * N) / (unsigned)G); }
  // largest w with start(w) <= x  (x < N)
  __device__ int owner(unsigned x) const {
    return (int)((((unsigned long long)x + 1) * (unsigned)G - 1) / N);
  }
};

// Block-wide exclusive prefix sum of clamped lengths into pre[0..B] (B <= 1024,
// four sequences per thread).  pre and wsum live in LDS scratch; returns pre[B].
__device__ unsigned long long length_prefix(const GqaDecodeArgs& a, unsigned long long* pre, unsigned long long* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long v[4], tsum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    v[i] = b < a.B ? (unsigned long long)clamp_len(a.lens[b], a.T_max) : 0ull;
    tsum += v[i];
  }
  unsigned long long inc = tsum;  // inclusive scan over the wave
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  unsigned long long run = inc - tsum;
  for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    if (b < a.B) pre[b] = run;
    run += v[i];
  }
  if (tid == 0) pre[a.B] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return pre[a.B];
}

// ---------------------------------------------------------------------------
// Cross-workgroup exchange of partial results.  An agent-scope __threadfence()
// on gfx950 writes back and invalidates the whole L2 of the XCD, which is far too
// slow to issue once per workgroup.  Instead the partials are written and read
// with agent-scope atomic stores/loads, which bypass the non-coherent L2 copies
// (sc1), and ordering is enforced by waiting for the stores' completion before
// the completion counter is bumped.
__device__ __forceinline__ void store_coherent(float* p, float x, float y) {
  const unsigned long long v = ((unsigned long long)__builtin_bit_cast(unsigned, y) << 32) | __builtin_bit_cast(unsigned, x);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float x) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __builtin_bit_cast(unsigned, x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__builtin_bit_cast(float, (unsigned)v), __builtin_bit_cast(float, (unsigned)(v >> 32)));
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
// Wait until this thread's memory operations have completed (vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Piece epilogue: ob[n_rep][D] (normalised output of the piece) and lse[n_rep]
// (log2-sum-exp) are in LDS.  Writes the output directly when the piece is the
// whole segment; otherwise publishes the partial and, if this workgroup
// completes the segment, merges the segment's partials into the output.
template <int D>
__device__ void finish_piece(const GqaDecodeArgs& a, const Piece& pc, const float* ob, const float* lse,
                             SchedShared& sh) {
  const int tid = threadIdx.x;
  const int n_rep = a.n_rep;
  const size_t out_row0 = (size_t)pc.b * a.Hq + (size_t)pc.g * n_rep;
  auto store_out = [&](int hd, int d2, float2 v) {
    const size_t off = (out_row0 + hd) * D + 2 * d2;
    if (a.out_bf16) {
      const unsigned w = (unsigned)__builtin_bit_cast(u16, (__bf16)v.x) |
                         ((unsigned)__builtin_bit_cast(u16, (__bf16)v.y) << 16);
      *reinterpret_cast<unsigned*>(static_cast<u16*>(a.out) + off) = w;
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + off) = v;
    }
  };
  constexpr int D2 = D / 2;
  if (pc.count == 1) {
    for (int e = tid; e < n_rep * D2; e += 256) {
      const int hd = e / D2, d2 = e - hd * D2;
      store_out(hd, d2, *reinterpret_cast<const float2*>(ob + hd * D + 2 * d2));
    }
    __syncthreads();
    return;
  }
  float* o_ws = a.o_part + (size_t)pc.slot * n_rep * D;
  for (int e = tid; e < n_rep * D2; e += 256) store_coherent(o_ws + 2 * e, ob[2 * e], ob[2 * e + 1]);
  for (int hd = tid; hd < n_rep; hd += 256) store_coherent(a.lse + (size_t)pc.slot * n_rep + hd, lse[hd]);
  wait_vmem();      // this thread's partial stores have completed
  __syncthreads();  // ... and every thread's
  int* cnt = a.counters + (size_t)pc.b * a.Hkv + pc.g;
  if (tid == 0) sh.last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == pc.count - 1;
  __syncthreads();
  if (!sh.last) return;
  // this workgroup completed the segment: merge its pieces (coherent loads)
  for (int hd = tid; hd < n_rep; hd += 256) {
    float M = kNegInf;
    for (int k = 0; k < pc.count; ++k) M = fmaxf(M, load_coherent(a.lse + (size_t)(pc.first_slot + k) * n_rep + hd));
    float S = 0.f;
    for (int k = 0; k < pc.count; ++k)
      S += exp2_fast(load_coherent(a.lse + (size_t)(pc.first_slot + k) * n_rep + hd) - M);
    sh.m[hd] = M;
    sh.inv[hd] = 1.f / S;
  }
  __syncthreads();
  for (int e = tid; e < n_rep * D2; e += 256) {
    const int hd = e / D2, d2 = e - hd * D2;
    const float M = sh.m[hd];
    float2 acc = {0.f, 0.f};
    for (int k = 0; k < pc.count; ++k) {
      const size_t sl = (size_t)(pc.first_slot + k);
      const float w = exp2_fast(load_coherent(a.lse + sl * n_rep + hd) - M);
      const float2 v = load_coherent2(a.o_part + (sl * n_rep + hd) * D + 2 * d2);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
    }
    const float sc = sh.inv[hd];
    store_out(hd, d2, make_float2(acc.x * sc, acc.y * sc));
  }
  // leave the counter zero for the next call
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
}

// Zero output rows of a (sequence, KV head) with an empty cache (it has no piece).
template <int D>
__device__ void zero_rows(const GqaDecodeArgs& a, int b, int g) {
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * a.n_rep;
  for (int e = threadIdx.x; e < a.n_rep * D; e += 256) {
    if (a.out_bf16) static_cast<u16*>(a.out)[row0 * D + e] = 0;
    else static_cast<float*>(a.out)[row0 * D + e] = 0.f;
  }
}

// Drives the schedule: calls process(piece) for every piece of this workgroup,
// in order, each followed by the epilogue.  process leaves ob/lse in LDS.
// `scratch` (>= 8 * (B + 5) bytes of LDS) holds the balanced plan until the
// first piece starts.
template <int D, bool BALANCED, typename Process>
__device__ void run_schedule(const GqaDecodeArgs& a, SchedShared& sh, void* scratch, float* ob, float* lse,
                             Process&& process) {
  if constexpr (!BALANCED) {
    const int g = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
    const int L = clamp_len(a.lens[b], a.T_max);
    if (L == 0) {
      if (s == 0) zero_rows<D>(a, b, g);
      return;
    }
    const int c0 = s * a.split;
    if (c0 >= L) return;
    Piece pc;
    pc.b = b;
    pc.g = g;
    pc.t0 = c0;
    pc.t1 = min(c0 + a.split, L);
    pc.count = (L + a.split - 1) / a.split;
    pc.first_slot = (b * a.Hkv + g) * a.n_splits;
    pc.slot = pc.first_slot + s;
    process(pc);
    finish_piece<D>(a, pc, ob, lse, sh);
  } else {
    unsigned long long* pre = static_cast<unsigned long long*>(scratch);  // [B + 1]
    unsigned long long* wsum = pre + (a.B + 1);                             // [4]
    const unsigned long long P_B = uniform(length_prefix(a, pre, wsum));
    const int w = blockIdx.x;
    // empty sequences: workgroups take them round-robin
    for (int b = w; b < a.B; b += gridDim.x)
      if (pre[b + 1] == pre[b])
        for (int g = 0; g < a.Hkv; ++g) zero_rows<D>(a, b, g);
    Balanced bl;
    bl.N = (unsigned)(P_B * (unsigned)a.Hkv);
    if (bl.N == 0) return;
    bl.G = (int)min((unsigned)gridDim.x, (bl.N + a.min_rows_per_wg - 1) / a.min_rows_per_wg);
    if (w >= bl.G) return;
    const unsigned x0 = bl.start(w), x1 = bl.start(w + 1);
    if (x0 >= x1) return;
    // sequence holding row x0: Hkv*pre[b] <= x0 < Hkv*pre[b+1]
    for (int b = threadIdx.x; b < a.B; b += 256)
      if (pre[b] * a.Hkv <= x0 && x0 < pre[b + 1] * a.Hkv) sh.b0 = b;
    __syncthreads();
    int b = uniform(sh.b0);
    const unsigned seq_start = (unsigned)uniform(pre[b]) * a.Hkv;
    int L = uniform((int)(pre[b + 1] - pre[b]));
    int g = (int)((x0 - seq_start) / (unsigned)L);
    unsigned seg_start = seq_start + (unsigned)g * L;
    __syncthreads();  // pre[] (in the tile scratch) is dead from here on
    unsigned x = x0;
    while (x < x1) {
      const unsigned seg_end = seg_start + L;
      const unsigned e = seg_end < x1 ? seg_end : x1;
      Piece pc;
      pc.b = b;
      pc.g = g;
      pc.t0 = (int)(x - seg_start);
      pc.t1 = (int)(e - seg_start);
      const int s = b * a.Hkv + g;
      const int wf = bl.owner(seg_start), wl = bl.owner(seg_end - 1);
      pc.count = wl - wf + 1;
      pc.first_slot = wf + s;
      pc.slot = w + s;
      process(pc);
      finish_piece<D>(a, pc, ob, lse, sh);
      x = e;
      if (x >= x1) break;
      // next non-empty segment (one exists: x < x1 <= N)
      seg_start = seg_end;
      if (++g == a.Hkv) {
        g = 0;
        do {
          ++b;
          L = uniform(clamp_len(a.lens[b], a.T_max));
        } while (L == 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA.  HB blocks of 16 query heads (n_rep <= 16 * HB).
// Waves per SIMD the register allocation targets: four fit head_dim <= 96 with
// the next tile in flight; head_dim 128 needs up to 168 registers (three waves).
#ifndef ATTN_DECODE_WAVES_PER_EU_D128
#define ATTN_DECODE_WAVES_PER_EU_D128 3
#endif
template <int D, int HB, bool BALANCED>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(HB > 1 ? 1 : (D == 128 ? ATTN_DECODE_WAVES_PER_EU_D128 : 4))))
void gqa_decode_bf16(GqaDecodeArgs a) {
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
  constexpr int KC = D / 32;           // 32-wide dim chunks (QK contraction)
  constexpr int DW = D / 16;           // 16-wide dim blocks (PV output rows)
  constexpr int VP = D + 16;           // V tile row pitch in elements ([token][dim], padded)
  constexpr int kVtElems = kDecodeWaves * kDecodeTileTokens * VP;
  // epilogue scratch (floats): m and l per wave and head, [HB*16][D] outputs, lse
  static_assert(2 * kDecodeWaves * HB * 16 * 4 + HB * 16 * D * 4 + HB * 16 * 4 <= kVtElems * 2, "scratch");
  static_assert((kBalancedMaxB + 5) * 8 <= kVtElems * 2, "balanced plan scratch");
  __shared__ __attribute__((aligned(16))) u16 smem[kVtElems];
  __shared__ SchedShared sh;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, grp = lane >> 4;
  const int n_rep = a.n_rep;
  float* mw = reinterpret_cast<float*>(smem);   // [waves][HB*16]
  float* lw = mw + kDecodeWaves * HB * 16;      // [waves][HB*16]
  float* ob = lw + kDecodeWaves * HB * 16;      // [HB*16][D]
  float* lse_s = ob + HB * 16 * D;              // [HB*16]
  u16* vt = smem + wave * kDecodeTileTokens * VP;
  const size_t tok_stride = (size_t)a.Hkv * D;

  auto process = [&](const Piece& pc_) {
    const int pb = uniform(pc_.b), pg = uniform(pc_.g), pt0 = uniform(pc_.t0);
    const u16* qp = static_cast<const u16*>(a.q) + ((size_t)pb * a.Hq + (size_t)pg * n_rep) * D;
    const u16* kp = static_cast<const u16*>(a.k) + ((size_t)pb * a.T_max * a.Hkv + pg) * D;
    const u16* vp = static_cast<const u16*>(a.v) + ((size_t)pb * a.T_max * a.Hkv + pg) * D;
    const int c1 = uniform(pc_.t1);
    // Q^T as the B operand: lane holds Q[head = 16hb + row][dims 32c + 8grp .. +8]
    bf16x8 qop[HB][KC];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = hb * 16 + row;
#pragma unroll
      for (int c = 0; c < KC; ++c)
        qop[hb][c] = head < n_rep ? load_bf16x8(qp + (size_t)head * D + 32 * c + 8 * grp)
                                  : __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
    float m[HB], lsum[HB];
    f32x4 o[HB][DW];  // O^T: lane holds dims 16w + 4grp + i of head 16hb + row
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m[hb] = kNegInf;
      lsum[hb] = 0.f;
#pragma unroll
      for (int w = 0; w < DW; ++w) o[hb][w] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // K as the A operand (row = token), V in the same layout.  Rows past the
    // piece end re-read its last row (their scores are masked), which also makes
    // the one-tile-ahead loads below safe to issue unconditionally.
    auto load_k = [&](bf16x8 (&kr)[2][KC], int t0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = min(t0 + 16 * u + row, c1 - 1);
        const u16* krow = kp + (size_t)tok * tok_stride + 8 * grp;
#pragma unroll
        for (int c = 0; c < KC; ++c) kr[u][c] = load_bf16x8(krow + 32 * c);
      }
    };
    auto load_v = [&](bf16x8 (&vr)[2][KC], int t0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tok = min(t0 + 16 * u + row, c1 - 1);
        const u16* vrow = vp + (size_t)tok * tok_stride + 8 * grp;
#pragma unroll
        for (int c = 0; c < KC; ++c) vr[u][c] = load_bf16x8(vrow + 32 * c);
      }
    };
    constexpr int kStep = kDecodeWaves * kDecodeTileTokens;
    int t0 = pt0 + wave * kDecodeTileTokens;
    bf16x8 kr[2][KC], vr[2][KC];
    if (t0 < c1) {
      load_k(kr, t0);
      load_v(vr, t0);
    }
    // Per tile: V(t) -> LDS, then V(t+1) is requested; scores on K(t), then
    // K(t+1) is requested; PV from LDS.  About one tile stays in flight per wave
    // with no extra registers.
    for (; t0 < c1; t0 += kStep) {
      // V tile into this wave's LDS region, row-major [token][dim]
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < KC; ++c)
          *reinterpret_cast<u16x8*>(vt + (16 * u + row) * VP + 32 * c + 8 * grp) = __builtin_bit_cast(u16x8, vr[u][c]);
      load_v(vr, t0 + kStep);
      // Scores: lane holds S^T[token 16u + 4grp + i][head 16hb + row]
      float sc[HB][2][4];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < KC; ++c) acc = mfma_16x16x32(kr[u][c], qop[hb][c], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = t0 + 16 * u + 4 * grp + i;
            sc[hb][u][i] = tok < c1 ? acc[i] * a.scale_log2e : kNegInf;
          }
        }
      }
      load_k(kr, t0 + kStep);
      // Online softmax per head; P^T as the B operand of the PV product.
      bf16x8 pop[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float mt = kNegInf;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[hb][u][i]);
        mt = max_xor16(mt);
        mt = max_xor32(mt);
        const float mn = fmaxf(m[hb], mt);  // finite: the tile's first token is valid
        const float alpha = exp2_fast(m[hb] - mn);
        m[hb] = mn;
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_fast(sc[hb][u][i] - mn);
            ps += p;
            pop[hb][4 * u + i] = (__bf16)p;
          }
        lsum[hb] = lsum[hb] * alpha + ps;
#pragma unroll
        for (int w = 0; w < DW; ++w) o[hb][w] *= alpha;
      }
      wave_lds_sync();
      // O^T[dims 16w..][heads] += V^T[16 dims][32 tokens (permuted)] P^T; the A operand
      // (tokens 4grp..4grp+3 and 16+4grp..16+4grp+3 of dim 16w+row) comes from two
      // transposed LDS reads.
      const u16* trbase = vt + (4 * grp + (row >> 2)) * VP + 4 * (row & 3);
#pragma unroll
      for (int w = 0; w < DW; ++w) {
        const u16x4 lo = lds_read_tr16(trbase + 16 * w);
        const u16x4 hi = lds_read_tr16(trbase + 16 * VP + 16 * w);
        const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[hb][w] = mfma_16x16x32(__builtin_bit_cast(bf16x8, av), pop[hb], o[hb][w]);
        // at most half of the transposed operands in flight (register pressure)
        if (w == DW / 2 - 1) __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
    }
    // ---- merge the four waves into ob / lse_s ----
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      lsum[hb] = sum_xor16(lsum[hb]);
      lsum[hb] = sum_xor32(lsum[hb]);
    }
    __syncthreads();  // every wave is done with its V region
    if (grp == 0) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        mw[wave * HB * 16 + hb * 16 + row] = m[hb];
        lw[wave * HB * 16 + hb * 16 + row] = lsum[hb];
      }
    }
    __syncthreads();
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int hd = hb * 16 + row;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w * HB * 16 + hd]);
      float Lt = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w * HB * 16 + hd], M) * lw[w * HB * 16 + hd];
      const float f = rescale(m[hb], M) / Lt;
#pragma unroll
      for (int w = 0; w < DW; ++w) o[hb][w] *= f;
      if (wave == 0 && grp == 0) lse_s[hd] = M + __log2f(Lt);
    }
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int dw = 0; dw < DW; ++dw) {
            float4* dst = reinterpret_cast<float4*>(ob + (hb * 16 + row) * D + 16 * dw + 4 * grp);
            const float4 cur = w == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : *dst;
            *dst = make_float4(cur.x + o[hb][dw][0], cur.y + o[hb][dw][1], cur.z + o[hb][dw][2],
                               cur.w + o[hb][dw][3]);
          }
      }
      __syncthreads();
    }
  };
  run_schedule<D, BALANCED>(a, sh, smem, ob, lse_s, process);
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU.  16 rows of 16 lanes; row r takes positions t0 + r + 16k.
template <int D, int NR, bool BALANCED>
__global__ __launch_bounds__(256) void gqa_decode_f32(GqaDecodeArgs a) {
  static_assert(D % 16 == 0, "head_dim must be a multiple of 16");
  constexpr int E = D / 16;
  __shared__ float mw[kDecodeWaves][NR], lw[kDecodeWaves][NR];
  __shared__ __attribute__((aligned(16))) float ob[NR * D];
  __shared__ float lse_s[NR];
  __shared__ unsigned long long plan[kBalancedMaxB + 5];
  __shared__ SchedShared sh;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rid = threadIdx.x >> 4, col = threadIdx.x & 15;
  const int n_rep = a.n_rep;
  const size_t tok_stride = (size_t)a.Hkv * D;

  auto process = [&](const Piece& pc) {
    const float* qp = static_cast<const float*>(a.q) + ((size_t)pc.b * a.Hq + (size_t)pc.g * n_rep) * D + col * E;
    const float* kp = static_cast<const float*>(a.k) + ((size_t)pc.b * a.T_max * a.Hkv + pc.g) * D + col * E;
    const float* vp = static_cast<const float*>(a.v) + ((size_t)pc.b * a.T_max * a.Hkv + pc.g) * D + col * E;
    float qv[NR][E], acc[NR][E], m[NR], l[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        qv[h][e] = h < n_rep ? qp[(size_t)h * D + e] * a.scale_log2e : 0.f;
        acc[h][e] = 0.f;
      }
    }
    for (int t = pc.t0 + rid; t < pc.t1; t += 16) {
      float kr[E], vr[E];
#pragma unroll
      for (int e = 0; e < E; ++e) kr[e] = kp[(size_t)t * tok_stride + e];
#pragma unroll
      for (int e = 0; e < E; ++e) vr[e] = vp[(size_t)t * tok_stride + e];
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        if (h < n_rep) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) d = fmaf(qv[h][e], kr[e], d);
          d = row16_sum(d);
          const float mn = fmaxf(m[h], d);
          const float alpha = exp2_fast(m[h] - mn);
          const float p = exp2_fast(d - mn);
          m[h] = mn;
          l[h] = l[h] * alpha + p;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vr[e], acc[h][e] * alpha);
        }
      }
    }
    // merge the four rows of each wave (lanes 16 and 32 apart)
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      if (h < n_rep) {
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
          const float mo = __shfl_xor(m[h], off);
          const float lo = __shfl_xor(l[h], off);
          const float M = fmaxf(m[h], mo);
          const float fa = rescale(m[h], M), fb = rescale(mo, M);
          l[h] = l[h] * fa + lo * fb;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] = acc[h][e] * fa + __shfl_xor(acc[h][e], off) * fb;
          m[h] = M;
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        mw[wave][h] = m[h];
        lw[wave][h] = l[h];
      }
    }
    __syncthreads();
    float Mh[NR], Lh[NR];
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w][h]);
      float Lt = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w][h], M) * lw[w][h];
      Mh[h] = M;
      Lh[h] = Lt;
    }
    if (threadIdx.x == 0) {
#pragma unroll
      for (int h = 0; h < NR; ++h)
        if (h < n_rep) lse_s[h] = Mh[h] + __log2f(Lh[h]);
    }
    for (int w = 0; w < kDecodeWaves; ++w) {
      if (wave == w && lane < 16) {
#pragma unroll
        for (int h = 0; h < NR; ++h) {
          if (h < n_rep) {
            const float f = rescale(m[h], Mh[h]) / Lh[h];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              float* dst = &ob[h * D + col * E + e];
              *dst = (w == 0 ? 0.f : *dst) + acc[h][e] * f;
            }
          }
        }
      }
      __syncthreads();
    }
  };
  run_schedule<D, BALANCED>(a, sh, plan, ob, lse_s, process);
}

template <int D, bool BAL>
hipError_t launch_bf16(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int hb = (a.n_rep + 15) / 16;
  if (hb == 1) hipLaunchKernelGGL((gqa_decode_bf16<D, 1, BAL>), grid, dim3(256), 0, st, a);
  else if (hb == 2) hipLaunchKernelGGL((gqa_decode_bf16<D, 2, BAL>), grid, dim3(256), 0, st, a);
  else if (hb <= 4) hipLaunchKernelGGL((gqa_decode_bf16<D, 4, BAL>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D, bool BAL>
hipError_t launch_f32(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int n = a.n_rep;
  if (n == 1) hipLaunchKernelGGL((gqa_decode_f32<D, 1, BAL>), grid, dim3(256), 0, st, a);
  else if (n == 2) hipLaunchKernelGGL((gqa_decode_f32<D, 2, BAL>), grid, dim3(256), 0, st, a);
  else if (n <= 4) hipLaunchKernelGGL((gqa_decode_f32<D, 4, BAL>), grid, dim3(256), 0, st, a);
  else if (n <= 8) hipLaunchKernelGGL((gqa_decode_f32<D, 8, BAL>), grid, dim3(256), 0, st, a);
  else if (n <= 16) hipLaunchKernelGGL((gqa_decode_f32<D, 16, BAL>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <bool BAL>
hipError_t launch_mode(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  if (a.in_bf16)
    return a.D == 64 ? launch_bf16<64, BAL>(a, grid, st) : a.D == 96 ? launch_bf16<96, BAL>(a, grid, st)
                                                                      : launch_bf16<128, BAL>(a, grid, st);
  return a.D == 64 ? launch_f32<64, BAL>(a, grid, st) : a.D == 96 ? launch_f32<96, BAL>(a, grid, st)
                                                                   : launch_f32<128, BAL>(a, grid, st);
}

}  // namespace

bool gqa_decode_supported(int D, int n_rep, int in_bf16) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (n_rep < 1) return false;
  return in_bf16 ? n_rep <= 64 : n_rep <= 16;
}

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t st) {
  if (!gqa_decode_supported(a.D, a.n_rep, a.in_bf16)) return hipErrorInvalidValue;
  if (a.balanced) {
    if (a.B > kBalancedMaxB || a.grid_wgs < 1 || a.min_rows_per_wg < 1) return hipErrorInvalidValue;
    return launch_mode<true>(a, dim3(a.grid_wgs), st);
  }
  // KV heads vary fastest so the workgroups of one chunk's heads (interleaved in
  // memory, one row of Hkv*D per token) are dispatched together.
  return launch_mode<false>(a, dim3(a.Hkv, a.n_splits, a.B), st);
}

}  // namespace attn
