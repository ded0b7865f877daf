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
//  * Work is cut into units: a chunk of cached positions of one (sequence, KV
//    head).  A workgroup streams a unit's K and V rows from HBM exactly once and
//    applies them to all n_rep query heads of the group -- the repeat_kv copies
//    are never made.  Its four waves take interleaved 32-token tiles.
//  * Schedule: the resident workgroups take units from a device-wide queue
//    (an atomic counter), planned on the device from cache_lens.  Under full
//    load the compute units stream at different rates, so a static equal split
//    ends with most of them idle; the queue keeps all of them busy until the
//    last units.  Batches larger than the LDS plan launch one workgroup per unit.
//  * Loads: K and V rows are read in row order with non-temporal buffer loads
//    (whole 64-byte segments per load, bounded by the buffer size so rows past
//    the unit end read as zeros without traffic), then staged per wave in LDS.
//  * bf16 path: scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the
//    tile's tokens as M and (padded) query heads as N; the K operand is read
//    from LDS.  P stays in the accumulator layout and becomes the B operand of
//    O^T += V^T P^T after a token permutation that both operands share; V is
//    read back transposed with ds_read_b64_tr_b16.
//  * fp32 path (VALU): 16 lanes cover one token's row (head_dim/16 elements
//    each); dot products are reduced inside the 16-lane DPP row.
//  * Online softmax in base 2 (scale * log2 e folded in, v_exp_f32).  A unit
//    that covers its whole sequence writes the output directly; otherwise it
//    writes a normalised partial and its log2-sum-exp, and a second kernel
//    combines the partials of each (sequence, KV head).
//  * Scores of positions at or beyond the unit end are masked to -inf; no
//    cache row at or beyond L_b is read.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ float bf16_to_f32(u16 x) { return __builtin_bit_cast(float, (unsigned)x << 16); }

// Cache policy of the K/V loads: non-temporal (streaming).  The cache is read
// once per call; these loads neither displace reusable lines nor wait on them.
constexpr int kStreamPolicy = 2;

// The decode's running max moves only when a tile's max exceeds it by more than
// this (log2 units): probabilities stay below 2^8, and most tiles skip the
// rescale of the accumulators.
constexpr float kLazyMax = 8.f;

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// int4 cache words: the 8 codes of a word (two per byte, low nibble first) as
// eight bf16 of value 136 + c.  Byte t times 0x1001 puts its high nibble at
// bits 16..19 beside the low one at bits 0..3; (x & 0x000F000F) ^ 0x43084308
// keeps the two nibbles, flips their sign bits (c + 8) and sets the exponent
// (0x4300), one v_bitop3 (truth table 0x6a: (s0 & s1) ^ s2).
__device__ __forceinline__ u32x4 int4_word(unsigned w) {
  u32x4 h;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    h[k] = __builtin_amdgcn_bitop3_b32(((w >> (8 * k)) & 0xFFu) * 0x1001u, 0x000F000Fu, 0x43084308u, 0x6a);
  return h;
}

// fp8 cache words: the 8 E4M3 codes of two words as eight bf16 (exact).  Each
// conversion widens the codes of one 16-bit half into a pair of bf16; the pairs
// are moved as whole words (extracting the two bf16 of a pair separately was
// miscompiled into a copy of the first one).
__device__ __forceinline__ u32x4 fp8_words(unsigned w0, unsigned w1) {
  u32x4 h;
  h[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false));
  h[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true));
  h[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false));
  h[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true));
  return h;
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

// ---------------------------------------------------------------------------
// Work units and their schedule
//
// A unit is chunk j of one (sequence b, KV head g): positions
// [j*chunk, min((j+1)*chunk, L_b)).  Sequence b has n_b = ceil(L_b / chunk)
// chunks per KV head.  A unit of a one-chunk sequence writes the output rows of
// its group directly; otherwise it writes a normalised partial output and its
// log2-sum-exp to slot (b*Hkv + g)*n_chunks + j, and gqa_decode_merge combines
// the partials of each (b, g) afterwards.
//
// Queue schedule: a grid of the workgroups that are resident at once; each takes
// the next unit from a device-wide counter until none is left, so units go to
// whichever workgroup is free (compute units do not stream at equal rates under
// full load, and a static equal split leaves the fast ones idle at the end).
// Units are numbered sequence-major, then chunk, then KV head: units taken at
// about the same time read the same cache rows (all KV heads of a position are
// adjacent in memory).  Fixed schedule (batches too large for the queue's plan
// in LDS): grid (Hkv, n_chunks, B), one workgroup per unit, empty ones exit.

struct Unit {
  int b, g;    // sequence and KV head
  int t0, t1;  // positions [t0, t1)
  int j, n;    // chunk index and chunks of the sequence
};

// Queue: ticket of the workgroup's next unit, taken ahead of time by thread 0
// while the current unit finishes (valid = 0: not taken yet).
struct NextUnit {
  unsigned v;
  int valid;
};

// Units 0 .. gridDim.x - 1 go to the workgroups of the same index; the queue
// hands out the rest: unit = gridDim.x + the counter before the increment.
// (An increment, atomic_inc with no wrap bound, rather than an add: the add's
// wave-level combining would wait for the result right where it is issued.)
__device__ __forceinline__ unsigned take_ticket(const GqaDecodeArgs& a) {
  return __builtin_amdgcn_atomic_inc32(a.queue, 0xffffffffu, __ATOMIC_RELAXED, "agent");
}

// Per-workgroup shared state of the schedule.
struct UnitShared {
  unsigned unit;     // queue: unit taken by this workgroup
  int b;             // queue: its sequence
  unsigned wsum[8];  // per-wave sums of the plan's prefix scans
};

// Blocks of `chunk` positions of one (sequence, KV head): nb = ceil(L / chunk).
// In the queue schedule (when the batch has blocks enough for it) the first
// kBigBlocks * nbig blocks form big units of kBigBlocks blocks, nbig =
// 3 nb / (4 kBigBlocks); the rest are single-block units, handed out after
// every big unit of the batch.  The end of the queue
// is thus made of small units, so the workgroups run out of work at about the
// same time.  Partials are stored at the slot of their first block.
constexpr int kBigBlocks = 4;

struct Split {
  int nb;    // blocks
  int nbig;  // big units (0 in the fixed schedule)
  __device__ int parts() const { return nb - (kBigBlocks - 1) * nbig; }
  // block index (= slot) of partial p
  __device__ int slot(int p) const { return p < nbig ? kBigBlocks * p : p + (kBigBlocks - 1) * nbig; }
};

__device__ __forceinline__ Split split_of(const GqaDecodeArgs& a, int L) {
  Split sp;
  sp.nb = (L + a.chunk - 1) / a.chunk;
  sp.nbig = a.use_queue && a.big_units ? 3 * sp.nb / (4 * kBigBlocks) : 0;
  return sp;
}

// Block-wide exclusive prefix sums over the batch (B <= kQueueMaxB, four
// sequences per thread) of the big-unit counts into preB[0..B] and of the
// single-block unit counts into preS[0..B]; the clamped lengths into len[0..B).
__device__ void unit_prefix(const GqaDecodeArgs& a, unsigned* preB, unsigned* preS, int* len, unsigned* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned vb[4], vs[4], tb = 0, ts = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    const int L = b < a.B ? clamp_len(a.lens[b], a.T_max) : 0;
    if (b < a.B) len[b] = L;
    const Split sp = split_of(a, L);
    vb[i] = (unsigned)sp.nbig;
    vs[i] = (unsigned)(sp.nb - kBigBlocks * sp.nbig);
    tb += vb[i];
    ts += vs[i];
  }
  unsigned ib = tb, is = ts;  // inclusive scans over the wave
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned yb = __shfl_up(ib, off), ys = __shfl_up(is, off);
    if (lane >= off) {
      ib += yb;
      is += ys;
    }
  }
  if (lane == 63) {
    wsum[wave] = ib;
    wsum[4 + wave] = is;
  }
  __syncthreads();
  unsigned rb = ib - tb, rs = is - ts;
  for (int w = 0; w < wave; ++w) {
    rb += wsum[w];
    rs += wsum[4 + w];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * tid + i;
    if (b < a.B) {
      preB[b] = rb;
      preS[b] = rs;
    }
    rb += vb[i];
    rs += vs[i];
  }
  if (tid == 0) {
    preB[a.B] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    preS[a.B] = wsum[4] + wsum[5] + wsum[6] + wsum[7];
  }
  __syncthreads();
}

// Writes one output element pair (out_dtype) of row `row` (= b*Hq + h).
__device__ __forceinline__ void store_out2(const GqaDecodeArgs& a, size_t row, int d, float x, float y) {
  const size_t off = row * a.D + d;
  if (a.out_bf16) {
    const unsigned w = (unsigned)__builtin_bit_cast(u16, (__bf16)x) | ((unsigned)__builtin_bit_cast(u16, (__bf16)y) << 16);
    *reinterpret_cast<unsigned*>(static_cast<u16*>(a.out) + off) = w;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + off) = make_float2(x, y);
  }
}

// Unit epilogue: the normalised output of the unit is the sum of NS slices
// ob[s * slice + head * OP + dim] in LDS (row pitch OP floats), its
// log2-sum-exp lse[n_rep].  Ends with a barrier (ob is reused).
template <int D, int NS = 1, int OP = D>
__device__ void store_unit(const GqaDecodeArgs& a, const Unit& u, const float* ob, const float* lse, int slice = 0) {
  const int tid = threadIdx.x, n_rep = a.n_rep;
  constexpr int D2 = D / 2;
  auto value = [&](int hd, int d2) {
    float2 v = *reinterpret_cast<const float2*>(ob + hd * OP + 2 * d2);
#pragma unroll
    for (int sl = 1; sl < NS; ++sl) {
      const float2 w = *reinterpret_cast<const float2*>(ob + sl * slice + hd * OP + 2 * d2);
      v.x += w.x;
      v.y += w.y;
    }
    return v;
  };
  if (u.n == 1 && !a.append) {
    const size_t row0 = (size_t)u.b * a.Hq + (size_t)u.g * n_rep;
    for (int e = tid; e < n_rep * D2; e += 256) {
      const int hd = e / D2, d2 = e - hd * D2;
      const float2 v = value(hd, d2);
      store_out2(a, row0 + hd, 2 * d2, v.x, v.y);
    }
  } else {
    const size_t slot = ((size_t)u.b * a.Hkv + u.g) * a.n_chunks + u.j;
    float2* o_ws = reinterpret_cast<float2*>(a.o_part + slot * n_rep * D);
    for (int e = tid; e < n_rep * D2; e += 256) {
      const int hd = e / D2, d2 = e - hd * D2;
      o_ws[e] = value(hd, d2);
    }
    for (int hd = tid; hd < n_rep; hd += 256) a.lse[slot * n_rep + hd] = lse[hd];
  }
  __syncthreads();
}

// Zero output rows of a (sequence, KV head) with an empty cache (it has no unit).
template <int D>
__device__ void zero_rows(const GqaDecodeArgs& a, int b, int g) {
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * a.n_rep;
  for (int e = threadIdx.x; e < a.n_rep * D; e += 256) {
    if (a.out_bf16) static_cast<u16*>(a.out)[row0 * D + e] = 0;
    else static_cast<float*>(a.out)[row0 * D + e] = 0.f;
  }
}

// Fixed schedule: the unit of this workgroup, grid (Hkv, n_chunks, B).  Returns
// false (after zeroing the group's output rows for an empty sequence) when the
// workgroup has no unit.
template <int D>
__device__ bool fixed_unit(const GqaDecodeArgs& a, Unit& u) {
  const int g = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(a.lens[b], a.T_max);
  if (L == 0) {
    if (j == 0) zero_rows<D>(a, b, g);
    return false;
  }
  u.b = b;
  u.g = g;
  u.j = j;
  u.t0 = j * a.chunk;
  if (u.t0 >= L) return false;
  u.t1 = min(u.t0 + a.chunk, L);
  u.n = split_of(a, L).parts();
  return true;
}

// Queue schedule: unit counts of the batch (big units come first) and the
// plan's LDS arrays.
struct QueuePlan {
  unsigned n_big, n_units;
  const unsigned* preB;  // [B + 1] big units before sequence b (per KV head)
  const unsigned* preS;  // [B + 1] single-block units before sequence b
  const int* len;        // [B] clamped cache lengths
};

// LDS of the queue plan, in unsigned: preB, preS, len.
constexpr int kQueuePlanWords = 3 * (kQueueMaxB + 1);

// Plans the queue (prefix sums in LDS) and zeroes the output rows of empty
// sequences (workgroups take them round-robin).
template <int D>
__device__ QueuePlan queue_plan(const GqaDecodeArgs& a, unsigned* lds, UnitShared& sh) {
  unsigned* preB = lds;
  unsigned* preS = lds + kQueueMaxB + 1;
  int* len = reinterpret_cast<int*>(lds + 2 * (kQueueMaxB + 1));
  unit_prefix(a, preB, preS, len, sh.wsum);
  for (int b = blockIdx.x; b < a.B; b += gridDim.x)
    if (len[b] == 0)
      for (int g = 0; g < a.Hkv; ++g) zero_rows<D>(a, b, g);
  QueuePlan pl;
  pl.n_big = (unsigned)uniform((int)preB[a.B]) * (unsigned)a.Hkv;
  pl.n_units = pl.n_big + (unsigned)uniform((int)preS[a.B]) * (unsigned)a.Hkv;
  pl.preB = preB;
  pl.preS = preS;
  pl.len = len;
  return pl;
}

// Units are numbered sequence-major, then block, then KV head: big units first,
// then the single-block ones.  The thread that finds the sequence b of unit x
// (Hkv*pre[b] <= x' < Hkv*pre[b+1]) writes it to sh.b; a barrier must follow.
__device__ __forceinline__ void find_sequence(const GqaDecodeArgs& a, const QueuePlan& pl, unsigned x,
                                              UnitShared& sh) {
  const bool big = x < pl.n_big;
  const unsigned* pr = big ? pl.preB : pl.preS;
  const unsigned xr = big ? x : x - pl.n_big;
  const unsigned Hkv = (unsigned)a.Hkv;
  for (int b = threadIdx.x; b < a.B; b += 256)
    if (pr[b] * Hkv <= xr && xr < pr[b + 1] * Hkv) sh.b = b;
}

// Unit x of sequence b (uniform values).
__device__ __forceinline__ Unit queue_unit(const GqaDecodeArgs& a, const QueuePlan& pl, unsigned x, int b) {
  const bool big = x < pl.n_big;
  const unsigned* pr = big ? pl.preB : pl.preS;
  const unsigned xr = big ? x : x - pl.n_big;
  const unsigned Hkv = (unsigned)a.Hkv;
  Unit u;
  u.b = b;
  const int L = uniform(pl.len[b]);
  const Split sp = split_of(a, L);
  const unsigned r = xr - (unsigned)uniform((int)pr[b]) * Hkv;
  const int k = (int)(r / Hkv);
  u.g = (int)(r - (unsigned)k * Hkv);
  u.j = big ? kBigBlocks * k : kBigBlocks * sp.nbig + k;
  u.n = sp.parts();
  u.t0 = u.j * a.chunk;
  u.t1 = min(u.t0 + (big ? kBigBlocks : 1) * a.chunk, L);
  return u;
}

// Drives the schedule for a kernel without cross-unit prefetch: for every unit
// of this workgroup, process(unit, next) leaves the unit's normalised output in
// ob and its log2-sum-exp in lse (LDS), and store_unit publishes it.  `pre`
// (queue only) holds kQueuePlanWords unsigned of LDS for the whole kernel.
template <int D, bool QUEUE, typename Process>
__device__ void run_units(const GqaDecodeArgs& a, UnitShared& sh, unsigned* pre, float* ob, float* lse,
                          Process&& process) {
  if constexpr (!QUEUE) {
    Unit u;
    if (!fixed_unit<D>(a, u)) return;
    NextUnit nx = {0u, 0};
    process(u, nx);
    store_unit<D>(a, u, ob, lse);
  } else {
    const QueuePlan plan = queue_plan<D>(a, pre, sh);
    unsigned x = blockIdx.x;
    while (x < plan.n_units) {
      find_sequence(a, plan, x, sh);
      __syncthreads();
      const Unit u = queue_unit(a, plan, x, uniform(sh.b));
      NextUnit nx = {0u, 0};
      process(u, nx);
      store_unit<D>(a, u, ob, lse);  // ends with a barrier: every thread has read sh.b and sh.unit
      if (threadIdx.x == 0) sh.unit = gridDim.x + (nx.valid ? nx.v : take_ticket(a));
      __syncthreads();
      x = (unsigned)uniform((int)sh.unit);
    }
  }
}

// Element pairs of one (sequence, KV head) output block that a merge
// workgroup combines.
constexpr int kMergePairs = 256;

// Cache row (in [Hkv, D] rows) that holds position t of sequence b: t of the
// contiguous cache, or row t mod page_size of the page the block table names
// (clamped to the pool) for paged caches.
__device__ __forceinline__ size_t cache_row(const GqaDecodeArgs& a, int b, int t) {
  if (!a.block_table) return (size_t)b * a.T_max + t;
  const int e = a.block_table[(size_t)b * a.table_stride + t / a.page_size];
  const int page = min(max(e, 0), a.n_pages - 1);
  return (size_t)page * a.page_size + (t - (t / a.page_size) * a.page_size);
}

// Combines the partials of every (sequence, KV head) with more than one chunk:
// out = sum_j 2^(lse_j - M) o_j / sum_j 2^(lse_j - M), M = max_j lse_j.  Grid
// (Hkv * ceil(n_rep * D / 2 / kMergePairs), B): each thread merges one pair
// of output elements.  Also returns the queue counter to zero for the next
// call (the decode kernel has finished: same stream).
// In a decode step with the new token (a.append), every (sequence, KV head) is
// merged: the new token is one more partial, with log2 score
// scale_log2e * q . k_new and output v_new, and the thread of query head 0 of
// the group writes its element pair of k_new and v_new to the cache row of
// position lens[b] (the decode kernel read only rows below it; for paged
// caches the row of that position's page).
__global__ __launch_bounds__(256) void gqa_decode_merge(GqaDecodeArgs a) {
  const int tid = threadIdx.x, b = blockIdx.y;
  if (a.use_queue && blockIdx.x == 0 && b == 0 && tid == 0) *a.queue = 0u;
  const int n_rep = a.n_rep, D2 = a.D / 2;
  const int n_eb = (n_rep * D2 + kMergePairs - 1) / kMergePairs;
  const int g = blockIdx.x / n_eb, e = (blockIdx.x - g * n_eb) * kMergePairs + tid;
  if (e >= n_rep * D2) return;
  const int L = clamp_len(a.lens[b], a.T_max);
  const Split sp = split_of(a, L);
  const int n = sp.parts();
  if (n <= 1 && !a.append) return;  // written by the decode kernel
  const size_t s0 = ((size_t)b * a.Hkv + g) * a.n_chunks;
  const float* lse = a.lse + s0 * n_rep;
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * n_rep;
  const float2* op = reinterpret_cast<const float2*>(a.o_part + s0 * n_rep * a.D);
  const size_t jstride = (size_t)n_rep * D2;  // float2 per slot
  {
    const int hd = e / D2, d2 = e - hd * D2;
    // one pass with a running max; eight partials per batch, loaded before use
    // (indices clamped, the extra ones weigh 2^-inf = 0)
    float M = kNegInf, S = 0.f;
    float2 acc = {0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += 8) {
      float w[8];
      float2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = sp.slot(min(j0 + k, n - 1));
        w[k] = lse[(size_t)j * n_rep + hd];
        v[k] = op[(size_t)j * jstride + e];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (j0 + k >= n) w[k] = kNegInf;
        const float Mn = fmaxf(M, w[k]);  // finite from the first partial on
        const float f = rescale(M, Mn), wk = exp2_fast(w[k] - Mn);
        S = S * f + wk;
        acc.x = acc.x * f + wk * v[k].x;
        acc.y = acc.y * f + wk * v[k].y;
        M = Mn;
      }
    }
    if (a.append) {
      const size_t kv = ((size_t)b * a.Hkv + g) * a.D;
      const size_t qr = (row0 + hd) * a.D;
      // head_dim 64 and 128: the D/2 threads of a head are consecutive lanes of
      // one wave (blocks of 256 threads start at a head), so each multiplies its
      // own pair and the wave sums them; other widths loop over the whole row
      const bool lanes_sum = D2 == 32 || D2 == 64;
      float dot = 0.f, vx, vy;
      if (a.in_bf16) {
        const u16* qp = static_cast<const u16*>(a.q) + qr;
        const u16* kp = static_cast<const u16*>(a.k_new) + kv;
        if (lanes_sum) {
          const unsigned qw = *reinterpret_cast<const unsigned*>(qp + 2 * d2);
          const unsigned kw = *reinterpret_cast<const unsigned*>(kp + 2 * d2);
          dot = fmaf(bf16_to_f32((u16)(qw & 0xffffu)), bf16_to_f32((u16)(kw & 0xffffu)),
                     bf16_to_f32((u16)(qw >> 16)) * bf16_to_f32((u16)(kw >> 16)));
          for (int off = D2 / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
        } else {
          for (int d = 0; d < a.D; d += 8) {
            const u16x8 qa = *reinterpret_cast<const u16x8*>(qp + d);
            const u16x8 ka = *reinterpret_cast<const u16x8*>(kp + d);
#pragma unroll
            for (int i = 0; i < 8; ++i) dot = fmaf(bf16_to_f32(qa[i]), bf16_to_f32(ka[i]), dot);
          }
        }
        const unsigned vw = *reinterpret_cast<const unsigned*>(static_cast<const u16*>(a.v_new) + kv + 2 * d2);
        vx = bf16_to_f32((u16)(vw & 0xffffu));
        vy = bf16_to_f32((u16)(vw >> 16));
        if (hd == 0 && L < a.T_max) {
          const size_t dst = cache_row(a, b, L) * a.Hkv * a.D + (size_t)g * a.D + 2 * d2;
          *reinterpret_cast<unsigned*>(static_cast<u16*>(a.k_cache) + dst) =
              *reinterpret_cast<const unsigned*>(kp + 2 * d2);
          *reinterpret_cast<unsigned*>(static_cast<u16*>(a.v_cache) + dst) = vw;
        }
      } else {
        const float* qp = static_cast<const float*>(a.q) + qr;
        const float* kp = static_cast<const float*>(a.k_new) + kv;
        if (lanes_sum) {
          const float2 qa = *reinterpret_cast<const float2*>(qp + 2 * d2);
          const float2 ka = *reinterpret_cast<const float2*>(kp + 2 * d2);
          dot = fmaf(qa.x, ka.x, qa.y * ka.y);
          for (int off = D2 / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
        } else {
          for (int d = 0; d < a.D; d += 4) {
            const float4 qa = *reinterpret_cast<const float4*>(qp + d);
            const float4 ka = *reinterpret_cast<const float4*>(kp + d);
            dot = fmaf(qa.x, ka.x, dot);
            dot = fmaf(qa.y, ka.y, dot);
            dot = fmaf(qa.z, ka.z, dot);
            dot = fmaf(qa.w, ka.w, dot);
          }
        }
        const float2 vv = *reinterpret_cast<const float2*>(static_cast<const float*>(a.v_new) + kv + 2 * d2);
        vx = vv.x;
        vy = vv.y;
        if (hd == 0 && L < a.T_max) {
          const size_t dst = cache_row(a, b, L) * a.Hkv * a.D + (size_t)g * a.D + 2 * d2;
          *reinterpret_cast<float2*>(static_cast<float*>(a.k_cache) + dst) =
              *reinterpret_cast<const float2*>(kp + 2 * d2);
          *reinterpret_cast<float2*>(static_cast<float*>(a.v_cache) + dst) = vv;
        }
      }
      const float s = dot * a.scale_log2e;
      const float Mn = fmaxf(M, s);
      const float f = rescale(M, Mn), wk = exp2_fast(s - Mn);
      S = S * f + wk;
      acc.x = acc.x * f + wk * vx;
      acc.y = acc.y * f + wk * vy;
    }
    const float sc = 1.f / S;
    store_out2(a, row0 + hd, 2 * d2, acc.x * sc, acc.y * sc);
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA.  HB blocks of 16 query heads (n_rep <= 16 * HB).
// Waves per SIMD the register allocation targets (the fixed schedule runs
// several workgroups per compute unit): four fit head_dim 64, head_dim 96 and
// 128 need up to 168 registers (three waves) with the next tile in flight.  Two
// head blocks fit 256 registers without spilling (two waves); allowed more, the
// compiler kept the accumulators in AGPRs and the MQA sweep setting (n_rep 32)
// ran 6% slower (22.3 vs 21.0 us).  Four head blocks need more (one wave).
// KV8: the caches hold OCP FP8 E4M3 values (one byte each), converted to bf16
// (exactly) on their way into LDS; the K scale is folded into the softmax
// scale by the host, the V scale is applied to each unit's output.
// PAGED: the caches are page pools and a block table maps positions to pages;
// a unit's page numbers are read once (two per lane) when the unit begins, and
// every 32-position tile, which lies within one page, reads its page number
// from those registers.
// KV4: the caches hold signed 4-bit codes (two per byte, low nibble first) with
// one fp32 scale per cached row.  Each code c goes into the LDS tile as the
// bf16 value 136 + c, whose bits are 0x4300 | (c + 8): a bit operation, no
// arithmetic.  The offset is removed after the products, exactly in fp32: the
// scores subtract 136 * sum(q) (q as the MFMA sees it), the outputs 136 *
// sum(p') with p' = bf16(p * v_scale) the PV operand; the row's K scale
// multiplies its score, its V scale its probability.  The wave's 32 K and 32 V
// scales of a tile are read with the tile (one per lane) and staged in LDS.
template <int D, int HB, bool QUEUE, bool KV8 = false, bool PAGED = false, bool KV4 = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(HB > 2 || (HB > 1 && KV4) ? 1 : (HB > 1 ? 2 : (D >= 96 ? (QUEUE ? 2 : 3) : 4)))))
void gqa_decode_bf16(GqaDecodeArgs a) {
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
  static_assert(!KV8 || D == 128, "fp8 caches: head_dim 128");
  static_assert(!KV4 || (D == 128 && !KV8 && !PAGED), "int4 caches: head_dim 128, contiguous");
  constexpr int EB = KV8 ? 1 : 2;      // bytes per cached element (bf16, fp8)
  constexpr int RB = KV4 ? D / 2 : D * EB;  // bytes of one KV head's row
  constexpr int kEPU = 16 * D / RB;    // elements per 16-byte unit
  constexpr int KC = D / 32;           // 32-wide dim chunks (QK contraction)
  constexpr int DW = D / 16;           // 16-wide dim blocks (PV output rows)
  constexpr int VP = D + 16;           // V tile row pitch in elements ([token][dim], padded)
  constexpr int kUnits = RB / 16;                             // 16-byte units per K/V row
  constexpr int kLanesPerRow = kUnits <= 4 ? 4 : kUnits <= 8 ? 8 : 16;  // lanes that load one row
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  constexpr int kLoads = kDecodeTileTokens / kRowsPerLoad;   // 16-byte V loads per lane per tile
  // int4 K tiles go straight from memory into the MFMA operands; bf16 and
  // fp8 K tiles go through LDS like V (a lane's operand is 64 bytes of a row
  // in 16-byte pieces: read directly, each load instruction would take half
  // of every line of 16 rows, and the bf16 decode ran 4% slower)
  constexpr bool KD = KV4;
  constexpr int KP = D + 8;            // K tile row pitch (16 rows of one column: distinct LDS banks)
  constexpr int kStep = kDecodeWaves * kDecodeTileTokens;    // positions per round of the four waves
  constexpr int kVtElems = kDecodeWaves * kDecodeTileTokens * VP;
  // epilogue scratch (floats), overlaying the tiles: m and l per wave and head,
  // one [HB*16][OP] output slice per wave (the waves write their scaled outputs
  // at once and the store sums the slices), lse.  The row pitch OP = D + 4
  // puts the 16 head rows of one 16-byte-per-lane write on distinct LDS banks
  // (with pitch D they all hit the same four).  With more than one head block
  // the slices outgrow the tiles and the LDS array grows to hold them (up to
  // 134 KB at HB 4: one workgroup per compute unit in any case).
  constexpr int OP = D + 4;
  constexpr int kSliceFloats = HB * 16 * OP;
  constexpr int kScratchElems = (2 * kDecodeWaves * HB * 16 + kDecodeWaves * kSliceFloats + HB * 16) * 2;
  constexpr int kSmemElems = kScratchElems > kVtElems ? kScratchElems : kVtElems;
  static_assert(HB == 1 || kSmemElems * 2 + kQueuePlanWords * 4 <= 160 * 1024, "LDS");
  static_assert(HB > 1 || kSmemElems == kVtElems, "one head block: the scratch fits the tiles");
  __shared__ __attribute__((aligned(16))) u16 smem[kSmemElems];
  __shared__ __attribute__((aligned(16))) float scl[KV4 ? kDecodeWaves * 64 : 4];  // int4: K, V scales per wave
  __shared__ unsigned pre[QUEUE ? kQueuePlanWords : 1];
  __shared__ UnitShared sh;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int row = lane & 15, grp = lane >> 4;
  const int n_rep = a.n_rep;
  float* mw = reinterpret_cast<float*>(smem);   // [waves][HB*16]
  float* lw = mw + kDecodeWaves * HB * 16;      // [waves][HB*16]
  float* ob = lw + kDecodeWaves * HB * 16;      // [waves][HB*16][OP]
  float* lse_s = ob + kDecodeWaves * kSliceFloats;  // [HB*16]
  u16* vt = smem + wave * kDecodeTileTokens * VP;
  // bytes between consecutive positions of one head: int4 caches are head-major
  const int row_bytes = KV4 ? RB : uniform(a.Hkv * RB);
  // this lane's row within a load and its 16-byte unit in the row
  const int lrow = lane / kLanesPerRow, lunit = min(lane % kLanesPerRow, kUnits - 1);
  const unsigned row_off = (unsigned)(lrow * row_bytes + 16 * lunit);

  // base of this (sequence, KV head)'s rows (paged: of the head's rows in the pool)
  auto k_head = [&](const Unit& u) {
    if constexpr (PAGED) return static_cast<const char*>(a.k) + (size_t)u.g * RB;
    if constexpr (KV4) return static_cast<const char*>(a.k) + ((size_t)u.b * a.Hkv + u.g) * a.T_max * RB;
    return static_cast<const char*>(a.k) + ((size_t)u.b * a.T_max * a.Hkv + u.g) * RB;
  };
  auto v_head = [&](const Unit& u) {
    if constexpr (PAGED) return static_cast<const char*>(a.v) + (size_t)u.g * RB;
    if constexpr (KV4) return static_cast<const char*>(a.v) + ((size_t)u.b * a.Hkv + u.g) * a.T_max * RB;
    return static_cast<const char*>(a.v) + ((size_t)u.b * a.T_max * a.Hkv + u.g) * RB;
  };
  // paged: the current unit's first page slot and its page numbers (slot
  // unit_p0 + i in lane i % 64 of pg[i / 64])
  int unit_p0 = 0;
  int pg[2] = {0, 0};
  // address of position t0's row (t0 a multiple of 32)
  auto tile_base = [&](const char* head0, int t0) -> const char* {
    if constexpr (PAGED) {
      const int rel = min(max(t0 / a.page_size - unit_p0, 0), 127);
      const int e = rel < 64 ? __builtin_amdgcn_readlane(pg[0], rel) : __builtin_amdgcn_readlane(pg[1], rel - 64);
      const int page = min(max(e, 0), a.n_pages - 1);
      return head0 + ((size_t)page * a.page_size + (size_t)(t0 - (t0 / a.page_size) * a.page_size)) * row_bytes;
    }
    return head0 + (size_t)t0 * row_bytes;
  };

  // V tiles of 32 positions are read in row order with streaming
  // (non-temporal) buffer loads: lane group lane / kLanesPerRow of load i
  // fetches row kRowsPerLoad * i + lane / kLanesPerRow, each lane one 16-byte
  // unit (head_dim 96: lanes past the 12th unit repeat it), so a load covers
  // whole rows.  The tile's buffer resource starts at its first row and ends
  // with this head's part of row c1 - 1: rows at or past the unit end read as
  // zeros and cost no memory traffic, so loads ahead can be issued
  // unconditionally.  One resource per tile keeps the scalar work per load to
  // an offset.
  // 16-byte chunk j of a tile row (dims 8j .. 8j+7) is stored at chunk
  // swz(j) = j ^ ((j >> 3) & 1): with the widened fp8 and int4 rows, the
  // eight lanes of one 128-byte LDS pass then write eight distinct bank groups
  // (unswizzled, chunks j and j + 8 of a row share theirs).
  auto swz = [](int j) { return j ^ ((j >> 3) & 1); };
  auto tile_rsrc = [&](const char* head0, int t0, int c1) {
    // rows of the tile before c1, 0..32; bytes up to the end of the last
    // (row_bytes >= RB, so no rows gives a non-positive count)
    const int rows = min(max(c1 - t0, 0), kDecodeTileTokens);
    const int n = max(rows * row_bytes - row_bytes + RB, 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile_base(head0, t0)), (short)0, n, 0x00020000);
  };
  auto load_rows = [&](bf16x8 (&r)[kLoads], const char* head0, int t0, int c1) {
    const auto rs = tile_rsrc(head0, t0, c1);
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      r[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (int)(row_off + (unsigned)(kRowsPerLoad * i * row_bytes)), 0, kStreamPolicy));
  };
  // int4 K tiles go straight into the scores' MFMA operands (no LDS): lane
  // (row, grp) reads the 16 bytes of its 32 contiguous dims 32grp .. 32grp+31
  // of the rows of tokens 16s + row (s = 0, 1), a whole 64-byte row per four
  // lanes; operand slot c holds dims 32grp + 8c .. +8, and so does the query
  // operand.  Rows at or past c1 read as zeros.
  auto load_k = [&](bf16x8 (&r)[kLoads], const char* head0, int t0, int c1) {
    const auto rs = tile_rsrc(head0, t0, c1);
#pragma unroll
    for (int s = 0; s < 2; ++s)
      r[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (16 * s + row) * row_bytes + 16 * grp, 0, kStreamPolicy));
  };
  static_assert(!KD || kLoads == 2, "int4: two 16-byte loads per lane and tile, as the V tile");
  // int4: the tile's scales, lane l < 32 the K scale of row t0 + l, lane l >= 32
  // the V scale of row t0 + l - 32 (rows at or past c1 read as zeros)
  auto load_scales = [&](float& sr, const Unit& u, int t0, int c1) {
    if constexpr (KV4) {
      const int rows = min(max(c1 - t0, 0), kDecodeTileTokens);
      const size_t r0 = ((size_t)u.b * a.Hkv + u.g) * a.T_max + t0;  // head-major: the 32 scales are contiguous
      const float* base = (lane < 32 ? a.k_scales : a.v_scales) + r0;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, rows * 4, 0x00020000);
      sr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (lane & 31) * 4, 0, 0));
    }
  };
  // Tile registers written to this wave's LDS tile ([token][dim], row pitch
  // `pitch`, chunks swizzled).
  // fp8 rows: each 16-byte unit holds 16 values, widened to two 16-byte bf16 writes.
  // int4 rows: each 16-byte unit holds 32 codes, widened to four 16-byte writes.
  auto store_rows = [&](const bf16x8 (&r)[kLoads], int pitch) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      u16* dst = vt + (kRowsPerLoad * i + lrow) * pitch;
      constexpr int kChunks = kEPU / 8;  // 16-byte bf16 chunks per loaded unit
#pragma unroll
      for (int w = 0; w < kChunks; ++w) {
        const int j = kChunks * lunit + w;
        u16* p = dst + 8 * swz(j);
        if constexpr (KV4) {
          *reinterpret_cast<u32x4*>(p) = int4_word(__builtin_bit_cast(u32x4, r[i])[w]);
        } else if constexpr (KV8) {
          const u32x4 wd = __builtin_bit_cast(u32x4, r[i]);
          *reinterpret_cast<u32x4*>(p) = fp8_words(wd[2 * w], wd[2 * w + 1]);
        } else {
          *reinterpret_cast<u16x8*>(p) = __builtin_bit_cast(u16x8, r[i]);
        }
      }
    }
  };

  // Registers that carry a unit's inputs: Q^T as the B operand (lane holds
  // Q[head = 16hb + row][the dims of slot c]) and this wave's next K/V tile.
  bf16x8 qop[HB][KC];
  bf16x8 kr[kLoads], vr[kLoads];
  float sr = 0.f;  // int4: the next tile's scale (see load_scales)
  // Requests the query block of unit u and this wave's first tile of it.
  // The query block is read through a buffer resource that ends with head
  // n_rep - 1: the padding heads read as zeros, with no branch.
  auto begin_unit = [&](const Unit& u) {
    if constexpr (PAGED) {
      // the unit's page numbers, before the query block (the first tile waits for them)
      unit_p0 = u.t0 / a.page_size;
      const int np = (u.t1 - 1) / a.page_size - unit_p0 + 1;
      const int32_t* tb = a.block_table + (size_t)u.b * a.table_stride + unit_p0;
      pg[0] = lane < np ? tb[lane] : 0;
      pg[1] = lane + 64 < np ? tb[lane + 64] : 0;
    }
    const u16* qp = static_cast<const u16*>(a.q) + ((size_t)u.b * a.Hq + (size_t)u.g * n_rep) * D;
    const auto qs = __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(qp), (short)0, n_rep * D * 2, 0x00020000);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = hb * 16 + row;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int dim = KD ? 32 * grp + 8 * c : 32 * c + 8 * grp;
        qop[hb][c] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qs, (head * D + dim) * 2, 0, 0));
      }
    }
    if constexpr (KD) load_k(kr, k_head(u), u.t0 + wave * kDecodeTileTokens, u.t1);
    else load_rows(kr, k_head(u), u.t0 + wave * kDecodeTileTokens, u.t1);
    load_rows(vr, v_head(u), u.t0 + wave * kDecodeTileTokens, u.t1);
    load_scales(sr, u, u.t0 + wave * kDecodeTileTokens, u.t1);
  };

  // Streams unit u (begin_unit(u) issued): this wave's online-softmax state.
  float m[HB], lsum[HB];
  float q136[HB];     // int4: 136 * sum of q (this lane's head row)
  f32x4 psum[HB];     // int4: sum of the PV operand p' per head (every element), by MFMA
  f32x4 o[HB][DW];  // O^T: lane holds dims 16w + 4grp + i of head 16hb + row
  // the transposed V reads: lane's 4-dim group of row 4grp + row / 4, for
  // dim blocks w < 4 and (chunk parity flipped by the swizzle) w >= 4
  const u16* trbase = vt + (4 * grp + (row >> 2)) * VP + 4 * (row & 3);
  const u16* trbase_hi = vt + (4 * grp + (row >> 2)) * VP + 8 * (((row >> 1) & 1) ^ 1) + 4 * (row & 1);
  auto stream_unit = [&](const Unit& u, NextUnit& nx) {
    const char* kp = k_head(u);
    const char* vp = v_head(u);
    const int c1 = u.t1;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m[hb] = kNegInf;
      lsum[hb] = 0.f;
      psum[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < DW; ++w) o[hb][w] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KV4) {
        float qs = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) qs += (float)qop[hb][c][e];
        q136[hb] = 136.f * sum_xor32(sum_xor16(qs));
      }
    }
    // Per tile: K(t) -> LDS (int4: the K registers are the operands); scores;
    // K(t + kStep) requested; V(t) -> LDS (same region); V(t + kStep)
    // requested; softmax; PV from LDS.  Only a unit's last
    // tile can hold positions at or past its end (the others end before
    // t0 + kStep < c1), so only it masks the scores.  The wave's last tile
    // requests nothing further: a load past the unit end would read nothing,
    // but it still makes a round trip, and the next unit's loads into the same
    // registers would wait for it.
    auto tile = [&](const int t0, auto next) {
      constexpr bool NEXT = decltype(next)::value;
      constexpr bool MASK = !NEXT;
      if constexpr (QUEUE) {
        // second-to-last tile of wave 0 (or its only one): take the workgroup's
        // next unit, so the queue's round trip overlaps the end of this one
        if (wave == 0 && t0 + 2 * kStep >= c1 && lane == 0 && !nx.valid) {
          nx.v = take_ticket(a);
          nx.valid = 1;
        }
      }
      // Raw scores: lane holds S^T[token 16s + 4grp + i][head 16hb + row]; the
      // A operand (token 16s + row, the dims of slot c) from the K registers
      // (int4) or from LDS (dims 32c + 8grp .. +8).
      f32x4 acc[HB][2];
      {
        bf16x8 ka[2][KC];
        if constexpr (KD) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const u32x4 wd = __builtin_bit_cast(u32x4, kr[s]);
#pragma unroll
            for (int c = 0; c < KC; ++c) ka[s][c] = __builtin_bit_cast(bf16x8, int4_word(wd[c]));
          }
        } else {
          store_rows(kr, KP);
          wave_lds_sync();
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int c = 0; c < KC; ++c)
              ka[s][c] = __builtin_bit_cast(
                  bf16x8, *reinterpret_cast<const u16x8*>(vt + (16 * s + row) * KP + 8 * swz(4 * c + grp)));
        }
        // the accumulation chains of the two token blocks (and head blocks)
        // alternate, so no MFMA waits for the one issued just before it
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int s = 0; s < 2; ++s) acc[hb][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int s = 0; s < 2; ++s) acc[hb][s] = mfma_16x16x32(ka[s][c], qop[hb][c], acc[hb][s]);
      }
      // the next K tile once this one's operands are consumed; V overwrites the
      // K tile after its operand reads are done
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NEXT) {
        if constexpr (KD) load_k(kr, kp, t0 + kStep, c1);
        else load_rows(kr, kp, t0 + kStep, c1);
      }
      if constexpr (!KD) wave_lds_sync();
      if constexpr (KV4) scl[wave * 64 + lane] = lane < 32 ? sr * a.scale_log2e : sr;  // K scales: times the softmax scale
      store_rows(vr, VP);
      if constexpr (NEXT) load_scales(sr, u, t0 + kStep, c1);
      wave_lds_sync();
      if constexpr (NEXT) load_rows(vr, vp, t0 + kStep, c1);
      f32x4 ks[2] = {}, vs[2] = {};
      if constexpr (KV4) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          ks[s] = *reinterpret_cast<const f32x4*>(&scl[wave * 64 + 16 * s + 4 * grp]);
          vs[s] = *reinterpret_cast<const f32x4*>(&scl[wave * 64 + 32 + 16 * s + 4 * grp]);
        }
      }
      float sc[HB][2][4];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x;
            if constexpr (KV4) x = (acc[hb][s][i] - q136[hb]) * ks[s][i];
            else x = acc[hb][s][i] * a.scale_log2e;
            if constexpr (MASK) x = t0 + 16 * s + 4 * grp + i < c1 ? x : kNegInf;
            sc[hb][s][i] = x;
          }
      // Online softmax per head; P^T as the B operand of the PV product.  The
      // running max moves only when a tile's max exceeds it by more than
      // kLazyMax (log2 units), so the probabilities stay below 2^kLazyMax and
      // the accumulators are rescaled only on such tiles (rare once the first
      // tiles have set the max).
      bf16x8 pop[HB];
      float alpha[HB];
      bool up_any = false;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float mt = kNegInf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[hb][s][i]);
        mt = max_xor16(mt);
        mt = max_xor32(mt);
        const bool up = mt > m[hb] + kLazyMax;  // the tile's first token is valid: mt is finite
        const float mn = up ? mt : m[hb];
        alpha[hb] = exp2_fast(m[hb] - mn);  // 1 unless up (0 on the first tile)
        up_any |= up;
        m[hb] = mn;
        float ps = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_fast(sc[hb][s][i] - mn);
            if constexpr (KV4) {
              // the PV operand is p times the row's V scale
              ps += p;
              pop[hb][4 * s + i] = (__bf16)(p * vs[s][i]);
            } else {
              // the row sum adds the bf16-rounded probability the PV product uses
              const __bf16 pb = (__bf16)p;
              ps += (float)pb;
              pop[hb][4 * s + i] = pb;
            }
          }
        lsum[hb] = lsum[hb] * alpha[hb] + ps;
      }
      if (__builtin_amdgcn_ballot_w64(up_any) != 0) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
          for (int w = 0; w < DW; ++w) o[hb][w] *= alpha[hb];
          if constexpr (KV4) psum[hb] *= alpha[hb];
        }
      }
      // int4: sum p' over the tile's tokens with the PV product's own operands
      // (an A operand of ones), for the offset removal
      if constexpr (KV4) {
        const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                             (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) psum[hb] = mfma_16x16x32(ones, pop[hb], psum[hb]);
      }
      // O^T[dims 16w..][heads] += V^T[16 dims][32 tokens (permuted)] P^T; the A operand
      // (tokens 4grp..4grp+3 and 16+4grp..16+4grp+3 of dim 16w+row) comes from two
      // transposed LDS reads.
#pragma unroll
      for (int w = 0; w < DW; ++w) {
        const u16* tb = (w < 4 ? trbase : trbase_hi) + 16 * w;
        const u16x4 lo = lds_read_tr16(tb);
        const u16x4 hi = lds_read_tr16(tb + 16 * VP);
        const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) o[hb][w] = mfma_16x16x32(__builtin_bit_cast(bf16x8, av), pop[hb], o[hb][w]);
        // at most half of the transposed operands in flight (register pressure)
        if (w == DW / 2 - 1) __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
    };
    int t0 = u.t0 + wave * kDecodeTileTokens;
    for (; t0 + kStep < c1; t0 += kStep) tile(t0, std::true_type{});
    if (t0 < c1) tile(t0, std::false_type{});
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      lsum[hb] = sum_xor16(lsum[hb]);
      lsum[hb] = sum_xor32(lsum[hb]);
      if constexpr (KV4) {
        // remove the codes' offset: O^T holds sum p' (136 + c); every element
        // of psum holds this lane's head's sum p'
        const float off = 136.f * psum[hb][0];
#pragma unroll
        for (int w = 0; w < DW; ++w) o[hb][w] -= off;
      }
    }
  };

  // Merges the four waves' states of unit u into ob / lse_s and stores it.
  // Entered after a barrier that follows the waves' mw / lw writes.
  auto finish_unit = [&](const Unit& u) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int hd = hb * 16 + row;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w * HB * 16 + hd]);
      float Lt = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w * HB * 16 + hd], M) * lw[w * HB * 16 + hd];
      const float f = rescale(m[hb], M) / Lt * (KV8 ? a.v_scale : 1.f);
#pragma unroll
      for (int w = 0; w < DW; ++w) o[hb][w] *= f;
      if (wave == 0 && grp == 0) lse_s[hd] = M + __log2f(Lt);
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int dw = 0; dw < DW; ++dw)
        *reinterpret_cast<float4*>(ob + wave * kSliceFloats + (hb * 16 + row) * OP + 16 * dw + 4 * grp) =
            make_float4(o[hb][dw][0], o[hb][dw][1], o[hb][dw][2], o[hb][dw][3]);
    __syncthreads();
    store_unit<D, kDecodeWaves, OP>(a, u, ob, lse_s, kSliceFloats);  // ends with a barrier (ob is reused)
  };
  auto publish_state = [&]() {
    if (grp == 0) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        mw[wave * HB * 16 + hb * 16 + row] = m[hb];
        lw[wave * HB * 16 + hb * 16 + row] = lsum[hb];
      }
    }
  };

  if constexpr (!QUEUE) {
    Unit u;
    if (!fixed_unit<D>(a, u)) return;
    begin_unit(u);
    NextUnit nx = {0u, 0};
    stream_unit(u, nx);
    __syncthreads();  // every wave is done with its LDS tile
    publish_state();
    __syncthreads();
    finish_unit(u);
  } else {
    const QueuePlan plan = queue_plan<D>(a, pre, sh);
    unsigned x = blockIdx.x;
    if (x >= plan.n_units) return;
    find_sequence(a, plan, x, sh);
    __syncthreads();
    Unit u = queue_unit(a, plan, x, uniform(sh.b));
    begin_unit(u);
    for (;;) {
      NextUnit nx = {0u, 0};
      stream_unit(u, nx);
      if (tid == 0) sh.unit = gridDim.x + (nx.valid ? nx.v : take_ticket(a));
      __syncthreads();  // every wave is done with its LDS tile; the next ticket is visible
      x = (unsigned)uniform((int)sh.unit);
      const bool more = x < plan.n_units;
      if (more) find_sequence(a, plan, x, sh);
      publish_state();
      __syncthreads();
      // request the next unit's inputs before this one is merged and stored
      Unit un = u;
      if (more) {
        un = queue_unit(a, plan, x, uniform(sh.b));
        begin_unit(un);
      }
      finish_unit(u);
      if (!more) break;
      u = un;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU.  16 rows of 16 lanes; row r takes positions t0 + r + 16k.
template <int D, int NR, bool QUEUE>
__global__ __launch_bounds__(256) void gqa_decode_f32(GqaDecodeArgs a) {
  static_assert(D % 16 == 0, "head_dim must be a multiple of 16");
  constexpr int E = D / 16;
  __shared__ float mw[kDecodeWaves][NR], lw[kDecodeWaves][NR];
  __shared__ __attribute__((aligned(16))) float ob[NR * D];
  __shared__ float lse_s[NR];
  __shared__ unsigned pre[QUEUE ? kQueuePlanWords : 1];
  __shared__ UnitShared sh;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rid = threadIdx.x >> 4, col = threadIdx.x & 15;
  const int n_rep = a.n_rep;
  const size_t tok_stride = (size_t)a.Hkv * D;

  auto process = [&](const Unit& pc, NextUnit&) {
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
  run_units<D, QUEUE>(a, sh, pre, ob, lse_s, process);
}

// Workgroups of 256 threads of `kernel` that are resident on one compute unit of
// the current device (0 if the query fails); asked once per kernel and device.
int resident_per_cu(const void* kernel) {
  struct Entry { const void* k; int dev, n; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.k == kernel && e.dev == dev) return e.n;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess) n = 0;
  cache.push_back({kernel, dev, n});
  return n;
}

// Launches kernel(a).  A queue grid is trimmed to the workgroups that are
// resident at once (more would only wait for the first ones to drain the queue),
// and to at most max_per_cu of them per compute unit.
template <typename Kernel>
hipError_t launch_one(Kernel kernel, const GqaDecodeArgs& a, dim3 grid, hipStream_t st, int max_per_cu) {
  if (a.use_queue) {
    int per_cu = resident_per_cu(reinterpret_cast<const void*>(kernel));
    if (per_cu > max_per_cu) per_cu = max_per_cu;
    if (per_cu > 0 && a.cus > 0 && per_cu * a.cus < (int)grid.x) grid.x = per_cu * a.cus;
  }
  hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Queue workgroups per compute unit of the MFMA kernel.  One: each keeps one
// 32-position tile per wave in flight and the next unit's first tile requested
// while it finishes a unit, which is enough to keep HBM busy, and with a single
// workgroup per compute unit none of them is starved by the others (the
// hardware favours older waves, so extra workgroups stream far slower and hold
// their units longest).  FP8 caches: two.  A tile then carries half the bytes
// for the same LDS, MFMA and softmax work, and a lone wave per SIMD leaves the
// chains of dependent steps bare; a second workgroup fills them (Llama-3-8B
// shaped decode, B 32: 60.0 -> 55.4 us; three: 59.0 us, and again 59.5 against
// 65.8 us once the LDS tiles were swizzled).  int4 caches: three (a quarter of
// the bytes per tile and more VALU work to widen them; 49.3 -> 42.9 us).
constexpr int kMfmaWgsPerCu = 1;
constexpr int kMfmaWgsPerCuFp8 = 2;
constexpr int kMfmaWgsPerCuInt4 = 3;

template <int D, bool QUEUE, bool KV8 = false, bool PAGED = false, bool KV4 = false>
hipError_t launch_bf16(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int hb = (a.n_rep + 15) / 16;
  constexpr int kNarrow = KV4 ? kMfmaWgsPerCuInt4 : (KV8 ? kMfmaWgsPerCuFp8 : kMfmaWgsPerCu);  // workgroups per CU, one head block
  if (hb == 1) return launch_one(gqa_decode_bf16<D, 1, QUEUE, KV8, PAGED, KV4>, a, grid, st, kNarrow);
  if (hb == 2) return launch_one(gqa_decode_bf16<D, 2, QUEUE, KV8, PAGED, KV4>, a, grid, st, kMfmaWgsPerCu);
  if (hb <= 4) return launch_one(gqa_decode_bf16<D, 4, QUEUE, KV8, PAGED, KV4>, a, grid, st, kMfmaWgsPerCu);
  return hipErrorInvalidValue;
}

template <int D, bool QUEUE>
hipError_t launch_f32(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int n = a.n_rep;
  if (n == 1) return launch_one(gqa_decode_f32<D, 1, QUEUE>, a, grid, st, 8);
  if (n == 2) return launch_one(gqa_decode_f32<D, 2, QUEUE>, a, grid, st, 8);
  if (n <= 4) return launch_one(gqa_decode_f32<D, 4, QUEUE>, a, grid, st, 8);
  if (n <= 8) return launch_one(gqa_decode_f32<D, 8, QUEUE>, a, grid, st, 8);
  if (n <= 16) return launch_one(gqa_decode_f32<D, 16, QUEUE>, a, grid, st, 8);
  return hipErrorInvalidValue;
}

template <bool QUEUE>
hipError_t launch_mode(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  if (a.kv_fp8) {
    if (a.D != 128) return hipErrorInvalidValue;
    return a.block_table ? launch_bf16<128, QUEUE, true, true>(a, grid, st) : launch_bf16<128, QUEUE, true>(a, grid, st);
  }
  if (a.kv_int4) return a.D == 128 ? launch_bf16<128, QUEUE, false, false, true>(a, grid, st) : hipErrorInvalidValue;
  if (a.block_table) {
    if (!a.in_bf16) return hipErrorInvalidValue;
    return a.D == 64 ? launch_bf16<64, QUEUE, false, true>(a, grid, st)
           : a.D == 96 ? launch_bf16<96, QUEUE, false, true>(a, grid, st)
                       : launch_bf16<128, QUEUE, false, true>(a, grid, st);
  }
  if (a.in_bf16)
    return a.D == 64 ? launch_bf16<64, QUEUE>(a, grid, st) : a.D == 96 ? launch_bf16<96, QUEUE>(a, grid, st)
                                                                        : launch_bf16<128, QUEUE>(a, grid, st);
  return a.D == 64 ? launch_f32<64, QUEUE>(a, grid, st) : a.D == 96 ? launch_f32<96, QUEUE>(a, grid, st)
                                                                     : launch_f32<128, QUEUE>(a, grid, st);
}

// Zeroes the work-queue counter of a scratch buffer (a kernel rather than a
// memset, so that the call can be captured in a graph).
__global__ void clear_queue(unsigned* queue) { *queue = 0u; }

// Scratch of the allocation-free decode: the workspace of attn_decode_gqa
// (queue counter, log2-sum-exps, partial outputs) in device memory that the
// code object holds, one copy per device, for callers that cannot allocate.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  // in host code `scratch` names a host-side stand-in; the device address of
  // each device's copy comes from the runtime, once per device
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_clear_queue(unsigned* queue, hipStream_t st) {
  hipLaunchKernelGGL(clear_queue, dim3(1), dim3(1), 0, st, queue);
  return hipGetLastError();
}

bool gqa_decode_supported(int D, int n_rep, int in_bf16) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (n_rep < 1) return false;
  return in_bf16 ? n_rep <= 64 : n_rep <= 16;
}

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t st) {
  if (!gqa_decode_supported(a.D, a.n_rep, a.in_bf16)) return hipErrorInvalidValue;
  if (a.chunk < 1 || a.n_chunks < 1) return hipErrorInvalidValue;
  hipError_t e;
  if (a.use_queue) {
    if (a.B > kQueueMaxB || a.n_chunks < 2 || a.grid_wgs < 1 || !a.queue) return hipErrorInvalidValue;
    e = launch_mode<true>(a, dim3(a.grid_wgs), st);
  } else {
    // KV heads vary fastest so the workgroups of one chunk's heads (interleaved
    // in memory, one row of Hkv*D per position) are dispatched together.
    e = launch_mode<false>(a, dim3(a.Hkv, a.n_chunks, a.B), st);
  }
  if (e != hipSuccess || (a.n_chunks < 2 && !a.append)) return e;
  const int n_eb = (a.n_rep * (a.D / 2) + kMergePairs - 1) / kMergePairs;
  hipLaunchKernelGGL(gqa_decode_merge, dim3(a.Hkv * n_eb, a.B), dim3(kMergePairs), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
