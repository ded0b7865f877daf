// MLA decode in absorbed form for gfx950.
//
// What is computed (qqstock DeepSeek MLA article, sections 1-4 and 6, and its
// MultiHeadLatentAttention listing): keys are [W_UK[h] c , k_rope] and values
// W_UV[h] c, where only the latent c (kv_lora_rank wide) and the rotated key
// part k_rope (shared by all heads) are cached.  Folding W_UK into the query and
// applying W_UV after the weighted sum gives the same numbers while reading only
// the cached rows:
//   q_lat  = [W_UK[h]^T q_nope , q_rope],  s_t = scale q_lat . [c_t , k_rope_t],
//   o_lat  = sum_t softmax(s)_t c_t,       out = W_UV[h] o_lat.
//
// Three kernels (not from the pages; designed for CDNA4), each a single memory
// round trip where it can be:
//  1. mla_absorb, one workgroup per (head, sequence): q_lat in fp32, kept as a
//     bf16 hi/lo pair (the MFMA score then sees ~16 mantissa bits of q_lat).
//  2. mla_decode_fused, grid (chunk, sequence), 4 waves, every workgroup serving
//     all heads (padded to 16) of one chunk of one sequence, so each cache row is
//     read from HBM once.  Wave w owns the 16-token slices c0 + 64k + 16w of the
//     chunk and runs its own 3-stage ring of buffer_load_dwordx4 ... lds copies
//     of the c_kv and k_rope slices.  S^T = [c k_rope] q_lat^T on 16x16x32 MFMA
//     (a trailing 16-wide rope chunk is zero-padded to 32) with the latent read
//     from LDS; P^T is the accumulator as it stands; O^T += V^T P^T on 16x16x16
//     MFMA with V^T read transposed (ds_read_b64_tr_b16) from the same latent
//     slice, since values share the latent with the un-rotated key.  A wave only
//     reads rows it copied itself, so the loop has no workgroup barrier.  The
//     four waves merge through LDS and the chunk's normalised o_lat and
//     log2-sum-exp go to the workspace.
//  3. mla_merge_wuv, one workgroup per (head, sequence): log2-sum-exp merge of
//     the chunks, then out = W_UV[h] o_lat with the W_UV rows already in flight.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kHeadsPad = 16;
constexpr int kWaves = kDecodeWaves;     // 4
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = 16;               // tokens per wave slice
constexpr int kStep = kSlice * kWaves;   // tokens per workgroup step
constexpr int kStages = 3;
constexpr float kRescaleSlack = 8.f;     // log2 units the reference max may trail the true max

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane16_swap_b32 a, b exchanges rows 1 and 3 of a with rows 0 and 2 of b;
// v_permlane32_swap_b32 a, b the upper half of a with the lower half of b
// (gfx950).  With a and b both holding x, lane l ends up with x_l and x_(l^16)
// (resp. x_(l^32)).  Inline asm (both operands read and written) because the
// compiler builtin for these instructions loses its second result; the s_nop
// pairs cover the VALU-write -> permlane-read hazard.  No memory is touched.
__device__ __forceinline__ float2 pair_xor16(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float2 pair_xor32(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float max_xor16(float x) { const float2 p = pair_xor16(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float max_xor32(float x) { const float2 p = pair_xor32(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor16(float x) { const float2 p = pair_xor16(x); return p.x + p.y; }
__device__ __forceinline__ float sum_xor32(float x) { const float2 p = pair_xor32(x); return p.x + p.y; }
__device__ __forceinline__ float rescale(float m, float M) { return m == kNegInf ? 0.f : exp2_fast(m - M); }
__device__ __forceinline__ int clamp_len(int L, int T_max) { return L < 0 ? 0 : (L > T_max ? T_max : L); }
__device__ __forceinline__ float bf16_to_f32(u16 x) { return __builtin_bit_cast(float, (unsigned)x << 16); }

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// ds_read_b64_tr_b16: lane i of a 16-lane group points at row T0 + i/4,
// columns 4(i%4).. of a row-major [token][dim] block; lane j receives tokens
// T0..T0+3 of column j.
__device__ __forceinline__ s16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Latent slice layout in LDS: 16 rows of R bf16, 16-byte chunk c of row r at
// chunk position c ^ swz<R>(r).  gfx950's LDS serves 256 bytes per clock (16
// lanes of a 16-byte read, 32 lanes of an 8-byte read).  The QK operand read
// takes one chunk index from 16 consecutive rows, so swz is a bijection on them
// modulo the 256-byte bank period; the transposed read takes a chunk pair from
// 8 consecutive rows, so swz / 2 is a bijection on those (modulo the period).
template <int R>
__device__ __forceinline__ int swz(int r) {
  if constexpr (R >= 128) return 2 * (r & 7) + ((r >> 3) & 1);
  else return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

template <int R, int DR>
struct Cfg {
  static constexpr int RW = R + DR;
  static constexpr int KC = R / 32;           // 32-wide latent chunks of the score
  static constexpr int RC = DR / 32;          // 32-wide rope chunks
  static constexpr bool R16 = (DR % 32) != 0; // one trailing 16-wide rope chunk
  static constexpr int DW = R / 16;           // 16-wide latent blocks of O^T
  static constexpr int kC = kSlice * R;       // latent slice (u16)
  static constexpr int kCInst = kC * 2 / 1024;  // copy instructions per latent slice
  static constexpr int kRInst = (kSlice * DR * 2 + 1023) / 1024;
  static constexpr int kR = kRInst * 512;     // rope slice (u16), padded to whole copies
  static constexpr int kInstPerSlice = kCInst + kRInst;
};

// Per-lane constants of the slice copies and reads.
template <int R, int DR>
struct Lanes {
  int lane, row, grp;
  int c_voff[Cfg<R, DR>::kCInst];  // byte offset in the global latent slice of this lane's copy
  int k_off;                       // QK operand read: element offset, XOR 32c per chunk
  int v_off;                       // transposed V read: element offset, XOR 16w per block
  __device__ __forceinline__ Lanes(int lane_) : lane(lane_), row(lane_ & 15), grp(lane_ >> 4) {
    constexpr int CPR = R / 8;  // chunks per row
#pragma unroll
    for (int q = 0; q < Cfg<R, DR>::kCInst; ++q) {
      const int s = 64 * q + lane, r = s / CPR, p = s % CPR;
      c_voff[q] = r * 2 * R + 16 * (p ^ swz<R>(r));
    }
    k_off = row * R + 8 * (grp ^ swz<R>(row));
    const int i = lane & 15, r = 4 * grp + (i >> 2);
    v_off = r * R + 8 * (((i & 3) >> 1) ^ swz<R>(r)) + 4 * (i & 1);
  }
};

// Buffer resource over rows [t0, lim) of a [T_max, width] bf16 cache of sequence
// b: rows at or past lim read as zeros and cost no memory traffic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int b, int T_max, int width, int t0,
                                                           int lim) {
  const int rows = lim - t0;
  const char* p = static_cast<const char*>(base) + ((size_t)b * T_max + (rows > 0 ? t0 : 0)) * width * 2;
  const unsigned long long n = rows > 0 ? (unsigned long long)rows * width * 2 : 0ull;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, (int)(n < 0xffffffffull ? n : 0xffffffffull),
                                           0x00020000);
}

template <int R, int DR>
__device__ __forceinline__ void issue_slice(u16* cdst, u16* rdst, const MlaDecodeArgs& a, int b, int t0, int lim,
                                            const Lanes<R, DR>& ln) {
  using C = Cfg<R, DR>;
  const auto rc = rows_rsrc(a.c_kv, b, a.T_max, R, t0, lim);
  const auto rr = rows_rsrc(a.k_rope, b, a.T_max, DR, t0, lim);
#pragma unroll
  for (int q = 0; q < C::kCInst; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(cdst + 512 * q), 16,
                                             ln.c_voff[q], 0, 0, 0);
#pragma unroll
  for (int q = 0; q < C::kRInst; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)(rdst + 512 * q), 16,
                                             16 * (64 * q + ln.lane), 0, 0, 0);
}

// vmcnt(n): wait until at most n of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

template <int R, int DR>
struct WaveState {
  f32x4 o[R / 16];  // O^T[16w + 4grp + i][head row]
  float m, lsum;    // reference max (scaled, log2) and this lane's part of the row sum
};

// ---------------------------------------------------------------------------
// q_lat[b][hl][h][0:R] = hi / lo bf16 parts of W_UK[h]^T q_nope[b,h] (fp32 sum);
// q_lat[b][0][h][R:R+DR] = q_rope[b,h], q_lat[b][1][h][R:] = 0; padded heads
// h in [H, 16) are zero.  Grid (16, B), 256 threads, one workgroup per (head,
// sequence): thread t owns latent columns 8(t % (R/8)) .. +8 (16-byte loads of
// W_UK rows, which stay in L2 across the sequences) and every P-th row (P =
// 2048 / R); a thread's loads are issued together before the first use, and
// the P partial sums meet in LDS.
// Rows [i0, i0 + U*P) of this thread's part: U loads of 16 bytes (row-clamped,
// so there is no branch between them) issued before any use.
template <int R, int U, int P>
__device__ __forceinline__ void absorb_rows(float (&acc)[8], const u16* wk, const u16* qn, int i0, int dn) {
  u16x8 wv[U];
  u16 qv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = min(i0 + u * P, dn - 1);
    wv[u] = *reinterpret_cast<const u16x8*>(wk + (size_t)i * R);
    qv[u] = qn[i];
  }
  asm volatile("" ::: "memory");  // issue the whole batch before the first use
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float q = i0 + u * P < dn ? bf16_to_f32(qv[u]) : 0.f;  // clamped rows count 0
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(bf16_to_f32(wv[u][e]), q, acc[e]);
  }
}

template <int R, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void mla_absorb(MlaDecodeArgs a) {
  constexpr int RW = R + DR;
  constexpr int OCT = R / 8;    // column octets
  constexpr int P = 256 / OCT;  // row parts
  __shared__ float red[P][R];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int oct = tid % OCT, part = tid / OCT;
  u16* ql = static_cast<u16*>(a.q_lat) + ((size_t)b * 2 * kHeadsPad + h) * RW;
  if (h >= a.H) {
    for (int e = tid; e < RW; e += 256) ql[e] = ql[kHeadsPad * RW + e] = 0;
    return;
  }
  const u16* wk = static_cast<const u16*>(a.w_uk) + (size_t)h * a.dn * R + 8 * oct;
  const u16* qn = static_cast<const u16*>(a.q_nope) + ((size_t)b * a.H + h) * a.dn;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int rows_per_part = (a.dn + P - 1) / P;  // uniform: pick the batch that covers it
  if (rows_per_part <= 2) absorb_rows<R, 2, P>(acc, wk, qn, part, a.dn);
  else if (rows_per_part <= 4) absorb_rows<R, 4, P>(acc, wk, qn, part, a.dn);
  else if (rows_per_part <= 8) absorb_rows<R, 8, P>(acc, wk, qn, part, a.dn);
  else
    for (int i0 = part; i0 < a.dn; i0 += 16 * P) absorb_rows<R, 16, P>(acc, wk, qn, i0, a.dn);
#pragma unroll
  for (int e = 0; e < 8; ++e) red[part][8 * oct + e] = acc[e];
  __syncthreads();
  for (int j = tid; j < R; j += 256) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < P; ++q) v += red[q][j];
    const __bf16 hi = (__bf16)v;
    ql[j] = __builtin_bit_cast(u16, hi);
    ql[kHeadsPad * RW + j] = __builtin_bit_cast(u16, (__bf16)(v - (float)hi));
  }
  const u16* qr = static_cast<const u16*>(a.q_rope) + ((size_t)b * a.H + h) * DR;
  for (int e = tid; e < DR; e += 256) {
    ql[R + e] = qr[e];
    ql[kHeadsPad * RW + R + e] = 0;
  }
}

// One 16-token slice from (cs, rs): scores, online softmax, O^T update.
template <int R, int DR>
__device__ __forceinline__ void slice_step(WaveState<R, DR>& st, const u16* cs, const u16* rs, const bf16x8 (&qhi)[R / 32],
                                           const bf16x8 (&qlo)[R / 32], const bf16x8* qr32, bf16x8 qr16, int t0, int c1,
                                           float c, const Lanes<R, DR>& ln) {
  using C = Cfg<R, DR>;
  // S^T[token 4grp + i][head row]: A = slice rows (token = row), B = q_lat^T.
  // Two accumulation chains (the hi and lo parts of q_lat) alternate, so no
  // MFMA waits for the one issued just before it; they meet at the end.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < C::KC; ++k) {
    const bf16x8 cr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(cs + (ln.k_off ^ (32 * k))));
    acc = mfma_16x16x32(cr, qhi[k], acc);
    acc2 = mfma_16x16x32(cr, qlo[k], acc2);
  }
#pragma unroll
  for (int k = 0; k < C::RC; ++k) {
    const bf16x8 kr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(rs + ln.row * DR + 32 * k + 8 * ln.grp));
    acc = mfma_16x16x32(kr, qr32[k], acc);
  }
  if constexpr (C::R16) {
    // trailing 16 rope dims as a 16x16x32 product whose upper 16 contraction
    // lanes (grp >= 2) are zero in both operands: the score chain then uses one
    // MFMA shape only (a dependent chain that switches shape needs more wait
    // states than the compiler provides on gfx950)
    const bf16x8 kr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(rs + ln.row * DR + 32 * C::RC + 8 * ln.grp));
    const bf16x8 z = {};
    acc2 = mfma_16x16x32(ln.grp < 2 ? kr : z, qr16, acc2);
  }
  acc += acc2;
  float s[4], mt = kNegInf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = t0 + 4 * ln.grp + i < c1 ? acc[i] * c : kNegInf;
    mt = fmaxf(mt, s[i]);
  }
  mt = max_xor32(max_xor16(mt));
  // The reference max only moves (and O, l are rescaled) when the slice's max
  // exceeds it by more than 2^8: probabilities stay below 256, well inside bf16
  // and fp32, and most slices skip the rescale.
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kRescaleSlack) != 0) {
    const float mn = fmaxf(st.m, mt);
    const float alpha = rescale(st.m, mn);
    st.m = mn;
    st.lsum *= alpha;
#pragma unroll
    for (int w = 0; w < C::DW; ++w) st.o[w] *= alpha;
  }
  const float ms = st.m == kNegInf ? 0.f : st.m;  // nothing visible yet: p = 2^-inf = 0
  s16x4 pop;
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 pb = (__bf16)exp2_fast(s[i] - ms);
    pop[i] = __builtin_bit_cast(short, pb);
    ps += (float)pb;  // the rounded probabilities the product uses
  }
  st.lsum += ps;
  // O^T[16w..16w+15][heads] += V^T[dims][16 tokens] P^T[tokens][heads]
#pragma unroll
  for (int w = 0; w < C::DW; ++w) st.o[w] = mfma_16x16x16(lds_read_tr16(cs + (ln.v_off ^ (16 * w))), pop, st.o[w]);
}

template <int R, int DR>
__global__ __launch_bounds__(kThreads) void mla_decode_fused(MlaDecodeArgs a) {
  using C = Cfg<R, DR>;
  constexpr int RW = C::RW;
  // three ring stages per wave, each a distinct LDS variable so the compiler can
  // tell the copies in flight from the reads of the resident stage
  // per wave and stage: the latent slice and the rope slice
  __shared__ __attribute__((aligned(1024))) u16 stg0[kWaves][C::kC];
  __shared__ __attribute__((aligned(1024))) u16 stg1[kWaves][C::kC];
  __shared__ __attribute__((aligned(1024))) u16 stg2[kWaves][C::kC];
  __shared__ __attribute__((aligned(1024))) u16 rop0[kWaves][C::kR];
  __shared__ __attribute__((aligned(1024))) u16 rop1[kWaves][C::kR];
  __shared__ __attribute__((aligned(1024))) u16 rop2[kWaves][C::kR];
  // epilogue scratch: one [16 heads][R] fp32 output slice per wave, two in each
  // of stages 0 and 1; m and l per wave and head in stage 2
  static_assert(2 * kHeadsPad * R * 4 == (int)sizeof(stg0), "two output slices per stage");
  static_assert(2 * kWaves * kHeadsPad * 4 <= (int)sizeof(stg2), "m, l scratch");

  const int s = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int n_chunks = (L + a.split - 1) / a.split;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Lanes<R, DR> ln(tid & 63);

  // The stages start zeroed: rows past the chunk end are read (with P = 0) by
  // the transposed V product, and uninitialised LDS could hold NaN patterns.
  // (Done while the length is in flight.)
  {
    const u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    u16* const bufs[6] = {&stg0[0][0], &stg1[0][0], &stg2[0][0], &rop0[0][0], &rop1[0][0], &rop2[0][0]};
#pragma unroll
    for (int k = 0; k < 6; ++k)
      for (int e = 8 * tid; e < kWaves * (k < 3 ? C::kC : C::kR); e += 8 * kThreads)
        *reinterpret_cast<u16x8*>(bufs[k] + e) = z;
  }
  if (s >= n_chunks) return;  // past the sequence (an empty one is zeroed by the merge)
  const int c0 = s * a.split, c1 = min(c0 + a.split, L);
  const int n_steps = (c1 - c0 + kStep - 1) / kStep;
  const int tw0 = c0 + kSlice * wave;  // first token of this wave's first slice
  __syncthreads();
  // q_lat^T as the B operand: lane holds q_lat[head row][32k + 8grp ..+8] (hi and lo);
  // requested after the first two slices (their copies are then already in flight)
  const u16* qlat = static_cast<const u16*>(a.q_lat) + (size_t)b * 2 * kHeadsPad * RW;
  bf16x8 qhi[C::KC], qlo[C::KC], qr32[C::RC > 0 ? C::RC : 1], qr16 = {};
  auto load_q = [&]() {
#pragma unroll
    for (int k = 0; k < C::KC; ++k) {
      qhi[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qlat + ln.row * RW + 32 * k + 8 * ln.grp));
      qlo[k] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u16x8*>(qlat + (kHeadsPad + ln.row) * RW + 32 * k + 8 * ln.grp));
    }
#pragma unroll
    for (int k = 0; k < C::RC; ++k)
      qr32[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qlat + ln.row * RW + R + 32 * k + 8 * ln.grp));
    if constexpr (C::R16) {  // the last 16 rope dims in contraction lanes 0..15, zero above
      const bf16x8 v =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qlat + ln.row * RW + R + 32 * C::RC + 8 * ln.grp));
      if (ln.grp < 2) qr16 = v;
    }
    // wait here (this also covers the first two slices' copies, issued earlier):
    // the operands are then known to be in registers everywhere in the loop
    wait_vmem();
  };

  // ---- stream the wave's slices through the ring
  WaveState<R, DR> st;
#pragma unroll
  for (int w = 0; w < C::DW; ++w) st.o[w] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.lsum = 0.f;
  const float c = a.scale_log2e;
  // Step k: copy slice k+2 into stage (k+2) % 3, wait for slice k, consume stage
  // k % 3.  The loop starts at k = -2 (copies only), so every copy comes from
  // the same three places in the loop body: the compiler then tracks which
  // stage each copy in flight belongs to across the back edge and adds no
  // waits beyond this one.  Copies of slices past the chunk read nothing.
  auto step = [&](int k, const u16* cs, const u16* rs, u16* cn, u16* rn) {
    issue_slice<R, DR>(cn, rn, a, b, tw0 + (k + 2) * kStep, c1, ln);
    if (k >= 0 && k < n_steps) {
      wait_vmcnt<2 * C::kInstPerSlice>();
      slice_step<R, DR>(st, cs, rs, qhi, qlo, qr32, qr16, tw0 + k * kStep, c1, c, ln);
    }
  };
  // the iteration that loads q_lat, as a value the compiler does not fold (a
  // first iteration peeled off the loop would end with a wait for every copy)
  const int k_q = __builtin_amdgcn_readfirstlane(n_steps > 0 ? -2 : -1);
  for (int k = -2; k < n_steps; k += kStages) {  // k = -2, 1, 4, ... : stage (k+2) % 3 = 0
    step(k, stg1[wave], rop1[wave], stg0[wave], rop0[wave]);
    step(k + 1, stg2[wave], rop2[wave], stg1[wave], rop1[wave]);
    if (k == k_q) load_q();
    step(k + 2, stg0[wave], rop0[wave], stg2[wave], rop2[wave]);
  }
  wait_vmem();  // the copies past the end (zeros) land before the stages are reused
  st.lsum = sum_xor32(sum_xor16(st.lsum));

  // ---- merge the four waves (LDS, reusing the stages)
  // Each wave writes its scaled O^T into its own [16][R] slice; 16-byte unit u
  // of head row h sits at unit position u ^ (h & 15), so the 16 rows of one
  // write land on distinct banks.
  __syncthreads();
  float* mw = reinterpret_cast<float*>(&stg2[0][0]);  // [waves][16]
  float* lw = mw + kWaves * kHeadsPad;                // [waves][16]
  auto slice = [&](int w) {
    return reinterpret_cast<float*>(w < 2 ? &stg0[0][0] : &stg1[0][0]) + (w & 1) * kHeadsPad * R;
  };
  if (ln.grp == 0) {
    mw[wave * kHeadsPad + ln.row] = st.m;
    lw[wave * kHeadsPad + ln.row] = st.lsum;
  }
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w * kHeadsPad + ln.row]);
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Lt += rescale(mw[w * kHeadsPad + ln.row], M) * lw[w * kHeadsPad + ln.row];
    const float f = rescale(st.m, M) / Lt;
#pragma unroll
    for (int w = 0; w < C::DW; ++w) st.o[w] *= f;
  }
  {
    float* ob = slice(wave) + ln.row * R;
#pragma unroll
    for (int dw = 0; dw < C::DW; ++dw)
      *reinterpret_cast<f32x4*>(ob + 4 * ((4 * dw + ln.grp) ^ ln.row)) = st.o[dw];
  }
  __syncthreads();

  // publish this chunk's normalised o_lat (the sum of the four slices) and
  // log2-sum-exp (ordered for the merge kernel by the kernel boundary)
  const size_t row0 = (size_t)b * a.H;
  for (int e = tid; e < a.H * (R / 4); e += kThreads) {
    const int h = e / (R / 4), d4 = e - h * (R / 4);
    const int off = h * R + 4 * (d4 ^ (h & 15));
    f32x4 v = *reinterpret_cast<const f32x4*>(slice(0) + off);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += *reinterpret_cast<const f32x4*>(slice(w) + off);
    *reinterpret_cast<f32x4*>(a.o_part + ((row0 + h) * a.n_splits + s) * R + 4 * d4) = v;
  }
  for (int h = tid; h < a.H; h += kThreads) {
    float M = kNegInf;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w * kHeadsPad + h]);
    float Lt = 0.f;
    for (int w = 0; w < kWaves; ++w) Lt += rescale(mw[w * kHeadsPad + h], M) * lw[w * kHeadsPad + h];
    a.lse[(row0 + h) * a.n_splits + s] = M + __log2f(Lt);
  }
}

// ---------------------------------------------------------------------------
// out[b,h] = W_UV[h] o_lat[b,h], with o_lat the log2-sum-exp merge of the
// sequence's chunk partials.  Grid (H, B), 256 threads.  Thread i < v_head_dim
// owns output row i: its W_UV row (R/8 loads of 16 bytes) is requested first,
// so it is in flight while threads j < R merge latent column j; the dot product
// then reads o_lat from LDS (the same address in every lane).  A sequence with
// an empty cache gets zeros.
template <int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void mla_merge_wuv(MlaDecodeArgs a) {
  constexpr int OCT = R / 8;
  constexpr int U = OCT < 16 ? OCT : 16;  // row loads in flight per batch
  __shared__ __attribute__((aligned(16))) float olat[R];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int n = (L + a.split - 1) / a.split;
  const size_t oi0 = ((size_t)b * a.H + h) * a.dv;
  if (n == 0) {
    for (int i = tid; i < a.dv; i += 256) {
      if (a.out_bf16) static_cast<u16*>(a.out)[oi0 + i] = 0;
      else static_cast<float*>(a.out)[oi0 + i] = 0.f;
    }
    return;
  }
  const u16* wrow = static_cast<const u16*>(a.w_uv) + ((size_t)h * a.dv + min(tid, a.dv - 1)) * R;
  u16x8 w8[U];
#pragma unroll
  for (int c = 0; c < U; ++c) w8[c] = *reinterpret_cast<const u16x8*>(wrow + 8 * c);
  // merge: thread j < R owns column j; eight chunks in flight, running max
  const size_t row = (size_t)b * a.H + h;
  for (int j = tid; j < R; j += 256) {
    const float* lse = a.lse + row * a.n_splits;
    const float* op = a.o_part + row * a.n_splits * R + j;
    float M = kNegInf, S = 0.f, acc = 0.f;
    for (int k0 = 0; k0 < n; k0 += 8) {
      float lv[8], ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = min(k0 + u, n - 1);
        lv[u] = lse[k];
        ov[u] = op[(size_t)k * R];
      }
      // chunks past the end (loaded clamped) get weight 2^-inf = 0; entry u = 0
      // is always a real chunk, so M is finite before any of them
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u >= n) lv[u] = kNegInf;
        const float Mn = fmaxf(M, lv[u]);
        const float f = rescale(M, Mn), w = exp2_fast(lv[u] - Mn);
        S = S * f + w;
        acc = acc * f + w * ov[u];
        M = Mn;
      }
    }
    olat[j] = acc / S;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < U; ++c) {
    const float4 o0 = *reinterpret_cast<const float4*>(olat + 8 * c);
    const float4 o1 = *reinterpret_cast<const float4*>(olat + 8 * c + 4);
    acc = fmaf(bf16_to_f32(w8[c][0]), o0.x, acc);
    acc = fmaf(bf16_to_f32(w8[c][1]), o0.y, acc);
    acc = fmaf(bf16_to_f32(w8[c][2]), o0.z, acc);
    acc = fmaf(bf16_to_f32(w8[c][3]), o0.w, acc);
    acc = fmaf(bf16_to_f32(w8[c][4]), o1.x, acc);
    acc = fmaf(bf16_to_f32(w8[c][5]), o1.y, acc);
    acc = fmaf(bf16_to_f32(w8[c][6]), o1.z, acc);
    acc = fmaf(bf16_to_f32(w8[c][7]), o1.w, acc);
  }
  for (int c0 = U; c0 < OCT; c0 += U) {  // R = 256: the rest of the row
#pragma unroll
    for (int c = 0; c < U; ++c) w8[c] = *reinterpret_cast<const u16x8*>(wrow + 8 * (c0 + c));
#pragma unroll
    for (int c = 0; c < U; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(bf16_to_f32(w8[c][e]), olat[8 * (c0 + c) + e], acc);
  }
  if (tid < a.dv) {
    if (a.out_bf16) static_cast<__bf16*>(a.out)[oi0 + tid] = (__bf16)acc;
    else static_cast<float*>(a.out)[oi0 + tid] = acc;
  }
}

template <int R, int DR>
hipError_t launch_rd(const MlaDecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((mla_absorb<R, DR>), dim3(kHeadsPad, a.B), dim3(256), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mla_decode_fused<R, DR>), dim3(a.n_splits, a.B), dim3(kThreads), 0, st, a);
  const hipError_t e2 = hipGetLastError();
  if (e2 != hipSuccess) return e2;
  hipLaunchKernelGGL((mla_merge_wuv<R>), dim3(a.H, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int R>
hipError_t launch_r(const MlaDecodeArgs& a, hipStream_t st) {
  switch (a.dR) {
    case 16: return launch_rd<R, 16>(a, st);
    case 32: return launch_rd<R, 32>(a, st);
    case 48: return launch_rd<R, 48>(a, st);
    case 64: return launch_rd<R, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mla_decode_supported(int H, int r, int dR) {
  return H >= 1 && H <= kHeadsPad && (r == 64 || r == 128 || r == 256) &&
         (dR == 16 || dR == 32 || dR == 48 || dR == 64);
}

hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t st) {
  if (!mla_decode_supported(a.H, a.r, a.dR)) return hipErrorInvalidValue;
  if (a.split % kStep != 0) return hipErrorInvalidValue;
  return a.r == 64 ? launch_r<64>(a, st) : a.r == 128 ? launch_r<128>(a, st) : launch_r<256>(a, st);
}

}  // namespace attn
