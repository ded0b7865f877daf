// MLA decode in absorbed form for gfx950, one kernel launch per call.
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
// How (not from the pages; designed for CDNA4).  One workgroup per (chunk of
// cached positions, sequence) serves all heads (padded to 16), so each cache
// row is read from HBM once.  Eight waves with two roles:
//  * waves 0-3 stream the chunk: wave w owns the 16-token slices c0 + 64k + 16w
//    and runs its own ring of kStages buffer_load_dwordx4 ... lds copies
//    (non-temporal) of the c_kv and k_rope slices, so a compute unit keeps about
//    four slices per wave in flight.  S^T = [c k_rope] q_lat^T on 16x16x32 MFMA
//    (a trailing 16-wide rope chunk zero-padded to 32) with the latent read from
//    LDS; P^T is the accumulator as it stands; O^T += V^T P^T on 16x16x16 MFMA
//    with V^T read transposed (ds_read_b64_tr_b16) from the same latent slice,
//    since values share the latent with the un-rotated key.  A wave only reads
//    rows it copied itself, so the loop has no workgroup barrier.
//  * waves 4-7 ("helpers") absorb the query while the first copies are in
//    flight, two heads each: their first W_UK and q_nope loads go out before
//    the cache length is known and before the streaming waves' copies (rows
//    read as they are stored, fp32 sums of bf16 pairs, the result kept as a
//    bf16 hi/lo pair so that the MFMA score sees ~16 mantissa bits); then they
//    request the W_UV rows of their first head and wait; after the stream each
//    applies out^T = W_UV o_lat^T on MFMA for its heads (o_lat as a bf16 hi/lo
//    pair), one head per product with the other heads' columns of the o_lat
//    operand zero.
// A sequence of several chunks is merged inside the same launch: every chunk
// stores its normalised o_lat and log2-sum-exp with device-coherent stores,
// waits for them to complete and counts itself done on the sequence's counter;
// the workgroup that finishes last (the counter's old value is n - 1) reads the
// partials back with device-coherent loads, merges them by their
// log2-sum-exps, applies W_UV and returns the counter to zero.  Nothing waits
// on another workgroup, so no schedule can deadlock.
// A decode step with the new token (attn_decode_mla_append) adds the new
// token as one more partial in that merge (its log2 score from q_lat and the
// new rows, its value the new latent row) and writes the new rows into the
// caches at row L, which the cache pass never reads.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kHeadsPad = 16;
constexpr int kWaves = kDecodeWaves;     // 4 streaming waves
constexpr int kHelpers = 4;              // helper waves
constexpr int kThreads = 64 * (kWaves + kHelpers);
constexpr int kSlice = 16;               // tokens per wave slice
constexpr int kStep = kSlice * kWaves;   // tokens per workgroup step
constexpr float kRescaleSlack = 8.f;     // log2 units the reference max may trail the true max
// Cache policy of the ring copies: non-temporal (the cache is read once per call).
constexpr int kStreamPolicy = 2;

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
__device__ __forceinline__ u16 f32_to_bf16(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

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

// Device-coherent 32-bit accesses of the cross-workgroup merge: relaxed atomics
// at agent scope, which gfx950 performs at the device's coherence point (they
// bypass the per-XCD L2 for reads and write through it), so a workgroup on
// another XCD sees them once they have completed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __builtin_bit_cast(unsigned, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}

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

template <int R, int DR, bool F8 = false>
struct Cfg {
  static constexpr int RW = R + DR;
  static constexpr int KC = R / 32;           // 32-wide latent chunks of the score
  static constexpr int RC = DR / 32;          // 32-wide rope chunks
  static constexpr bool R16 = (DR % 32) != 0; // one trailing 16-wide rope chunk
  static constexpr int DW = R / 16;           // 16-wide latent blocks of O^T
  static constexpr int kC = kSlice * R;       // latent slice (u16)
  // copy instructions per latent slice (fp8 latent: R bytes per row, copied raw)
  static constexpr int kCInst = F8 ? kSlice * R / 1024 : kC * 2 / 1024;
  static constexpr int kRInst = (kSlice * DR * 2 + 1023) / 1024;
  static constexpr int kR = kRInst * 512;     // rope slice (u16), padded to whole copies
  static constexpr int kInstPerSlice = kCInst + kRInst;
  // ring depth: as many stages as fit next to the absorbed query and the merge
  // buffers in about 158 KB of LDS, at most 5
  static constexpr int kStageBytes = kWaves * (kC + kR) * 2;
  static constexpr int kQlatBytes = 2 * kHeadsPad * RW * 2;
  static constexpr int kOlatBytes = 2 * kHeadsPad * R * 2;
  static constexpr int kFit = (158 * 1024 - kQlatBytes - kOlatBytes) / kStageBytes;
  static constexpr int kStages = kFit > 5 ? 5 : kFit;
  static_assert(kStages >= 3, "ring depth");
};

// Per-lane constants of the slice copies and reads.
template <int R, int DR, bool F8 = false>
struct Lanes {
  int lane, row, grp;
  int c_voff[Cfg<R, DR, F8>::kCInst];  // byte offset in the global latent slice of this lane's copy
  int k_off;                       // QK operand read: element offset, XOR 32c per chunk
  int v_off;                       // transposed V read: element offset, XOR 16w per block
  __device__ __forceinline__ Lanes(int lane_) : lane(lane_), row(lane_ & 15), grp(lane_ >> 4) {
    constexpr int CPR = R / 8;  // chunks per row
#pragma unroll
    for (int q = 0; q < Cfg<R, DR, F8>::kCInst; ++q) {
      const int s = 64 * q + lane;
      if constexpr (F8) {
        // raw fp8 rows, 16-byte slot s = row s / (R / 16), bytes 16 (s mod R / 16) of it
        c_voff[q] = (s / (R / 16)) * R + 16 * (s % (R / 16));
      } else {
        const int r = s / CPR, p = s % CPR;
        c_voff[q] = r * 2 * R + 16 * (p ^ swz<R>(r));
      }
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

// Paged caches: the chunk's page numbers, read once when it starts (slot
// p0 + i of the sequence's block-table row in lane i % 64 of pg[i / 64]).
struct ChunkPages {
  int p0;
  int pg[2];
};

// Buffer resource over the 16-row slice at t0 of a paged [n_pages, page_size,
// width] bf16 cache (page_size a multiple of 16, so the slice lies in one
// page): its page number comes from the chunk's registers by v_readlane
// (t0 is wave-uniform), clamped to the pool; rows at or past lim read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, const MlaDecodeArgs& a,
                                                            const ChunkPages& cp, int width, int t0, int lim) {
  const int rows = min(lim - t0, 16);
  const int rel = min(max(t0 / a.page_size - cp.p0, 0), 127);
  const int e = rel < 64 ? __builtin_amdgcn_readlane(cp.pg[0], rel) : __builtin_amdgcn_readlane(cp.pg[1], rel - 64);
  const int page = min(max(e, 0), a.n_pages - 1);
  const size_t row0 = (size_t)page * a.page_size + (size_t)(t0 - (t0 / a.page_size) * a.page_size);
  const char* p = static_cast<const char*>(base) + row0 * width * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, rows > 0 ? rows * width * 2 : 0,
                                           0x00020000);
}

// Copies the 16-row slice at t0 (rows past lim read as zeros) into (cdst, rdst).
template <int R, int DR, bool PAGED, bool F8 = false>
__device__ __forceinline__ void issue_slice(u16* cdst, u16* rdst, const MlaDecodeArgs& a, int b, int t0, int lim,
                                            const Lanes<R, DR, F8>& ln, const ChunkPages& cp) {
  using C = Cfg<R, DR, F8>;
  __amdgpu_buffer_rsrc_t rc, rr;
  if constexpr (F8 && PAGED) {  // pages of rows of R one-byte codes
    rc = page_rsrc(a.c_kv, a, cp, R / 2, t0, lim);
    rr = page_rsrc(a.k_rope, a, cp, DR, t0, lim);
  } else if constexpr (F8) {  // rows of R one-byte codes
    rc = rows_rsrc(a.c_kv, b, a.T_max, R / 2, t0, lim);
    rr = rows_rsrc(a.k_rope, b, a.T_max, DR, t0, lim);
  } else if constexpr (PAGED) {
    rc = page_rsrc(a.c_kv, a, cp, R, t0, lim);
    rr = page_rsrc(a.k_rope, a, cp, DR, t0, lim);
  } else {
    rc = rows_rsrc(a.c_kv, b, a.T_max, R, t0, lim);
    rr = rows_rsrc(a.k_rope, b, a.T_max, DR, t0, lim);
  }
#pragma unroll
  for (int q = 0; q < C::kCInst; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(cdst + 512 * q), 16,
                                             ln.c_voff[q], 0, 0, kStreamPolicy);
#pragma unroll
  for (int q = 0; q < C::kRInst; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)(rdst + 512 * q), 16,
                                             16 * (64 * q + ln.lane), 0, 0, kStreamPolicy);
}

// vmcnt(n): wait until at most n of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Orders this wave's LDS accesses before its later ones: waits for its
// outstanding LDS operations and keeps the compiler from moving LDS accesses
// across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// fp8 latent: a ring stage holds the slice's raw rows (R one-byte E4M3 codes
// each, 16-byte slot s = row s / (R / 16), bytes 16 (s mod R / 16)); each lane
// widens the slots it copied, exactly (E4M3 values fit bf16), into the bf16
// slice layout in place (16-byte chunk c of row r at chunk position c ^ swz(r)).
// Every lane's raw reads complete before any lane writes.
template <int R>
__device__ __forceinline__ void widen_slice(u16* cs, int lane) {
  constexpr int NS = kSlice * R / 1024;  // raw slots per lane
  u32x4 raw[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) raw[u] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(cs) + 16 * (64 * u + lane));
  wave_lds_sync();
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int t = 64 * u + lane, r = t / (R / 16), j = t % (R / 16);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {  // chunk 2j + hh: codes 8hh .. 8hh+7 of the slot
      u32x4 w;
      w[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[u][2 * hh], 1.f, false));
      w[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[u][2 * hh], 1.f, true));
      w[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[u][2 * hh + 1], 1.f, false));
      w[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[u][2 * hh + 1], 1.f, true));
      *reinterpret_cast<u32x4*>(cs + r * R + 8 * ((2 * j + hh) ^ swz<R>(r))) = w;
    }
  }
  wave_lds_sync();
}

template <int R, int DR>
struct WaveState {
  f32x4 o[R / 16];  // O^T[16w + 4grp + i][head row]
  float m, lsum;    // reference max (scaled, log2) and this lane's part of the row sum
};

// One 16-token slice from (cs, rs): scores, online softmax, O^T update.
template <int R, int DR, bool F8 = false>
__device__ __forceinline__ void slice_step(WaveState<R, DR>& st, const u16* cs, const u16* rs, const bf16x8 (&qhi)[R / 32],
                                           const bf16x8 (&qlo)[R / 32], const bf16x8* qr32, bf16x8 qr16, int t0, int c1,
                                           float c, const Lanes<R, DR, F8>& ln) {
  using C = Cfg<R, DR, F8>;
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

// ---------------------------------------------------------------------------
// Helper work.
//
// Absorb: q_lat[hl][h][0:R] = hi / lo bf16 parts of W_UK[h]^T q_nope[b,h]
// (fp32 sums), q_lat[0][h][R:R+DR] = q_rope[b,h], q_lat[1][h][R:] = 0; padding
// heads h in [H, 16) are zero.  The four helper waves do it, helper j the heads
// j + 4i two at a time (j and j + 4, then j + 8 and j + 12); lane (o, p) owns
// latent octet o (columns 8o .. 8o+7, R/8 octets) and the kAbsorbRows
// consecutive W_UK rows from p * kAbsorbRows of a round (P = 64 / (R/8) phases
// per round).  All loads of a round -- the W_UK rows and the matching q_nope
// elements of both heads -- are requested before the first is used, through
// buffer resources that end with the head's rows, so rows past nope_head_dim
// read as zeros.  Two rows at a time meet the q_nope pair in one
// v_dot2_f32_bf16 per column; the P phases meet by lane exchanges.
constexpr int kAbsorbRows = 12;

template <int R>
struct AbsorbLoads {
  u16x8 w[2][kAbsorbRows];            // W_UK rows of the two heads (8 latent columns each)
  u16x8 q[2][(kAbsorbRows + 7) / 8];  // q_nope elements of those rows (and a few past them)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}

// Requests the loads of round k0 (rows k0 + p * kAbsorbRows ..) of heads h0, h1.
template <int R>
__device__ __forceinline__ void absorb_issue(AbsorbLoads<R>& ld, const MlaDecodeArgs& a, int b, int h0, int h1, int k0,
                                             int lane) {
  constexpr int OCT = R / 8;
  const int o = lane % OCT, p = lane / OCT;
  const int r0 = k0 + p * kAbsorbRows;
  // one per-lane offset per operand kind; the row step is the (uniform) scalar offset
  const int wv = (r0 * R + 8 * o) * 2, qv = r0 * 2;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int h = hh ? h1 : h0;
    const auto wr = bytes_rsrc(static_cast<const u16*>(a.w_uk) + (size_t)h * a.dn * R, a.dn * R * 2);
    const auto qr = bytes_rsrc(static_cast<const u16*>(a.q_nope) + ((size_t)b * a.H + h) * a.dn, a.dn * 2);
#pragma unroll
    for (int t = 0; t < kAbsorbRows; ++t)
      ld.w[hh][t] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(wr, wv, t * R * 2, 0));
#pragma unroll
    for (int t = 0; t < (kAbsorbRows + 7) / 8; ++t)
      ld.q[hh][t] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, qv, 16 * t, 0));
  }
}

template <int R>
__device__ __forceinline__ void absorb_dot(float (&acc)[2][8], const AbsorbLoads<R>& ld) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int t = 0; t < kAbsorbRows; t += 2) {
      const bf16x2 q2 = __builtin_bit_cast(bf16x2, (unsigned)ld.q[hh][t / 8][t % 8] |
                                                       ((unsigned)ld.q[hh][t / 8][t % 8 + 1] << 16));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16x2 w2 = __builtin_bit_cast(bf16x2, (unsigned)ld.w[hh][t][e] | ((unsigned)ld.w[hh][t + 1][e] << 16));
        acc[hh][e] = __builtin_amdgcn_fdot2_f32_bf16(w2, q2, acc[hh][e], false);
      }
    }
}

// Writes the padding heads and the rope part of q_lat for helper j's heads
// (j + 4i); rope[i] holds element `lane` of head j + 4i's q_rope (loaded with
// the absorb's other operands, so that nothing here waits on memory).
template <int R, int DR>
__device__ void absorb_fixed_parts(const MlaDecodeArgs& a, int j, int lane, const u16 (&rope)[4], u16* qlat) {
  constexpr int RW = R + DR;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = j + i * kHelpers;
    u16* hi = qlat + h * RW;
    u16* lo = qlat + (kHeadsPad + h) * RW;
    if (h >= a.H) {
      for (int e = lane; e < RW; e += 64) hi[e] = lo[e] = 0;
    } else if (lane < DR) {
      hi[R + lane] = rope[i];
      lo[R + lane] = 0;
    }
  }
}

// Sums the phases of the two heads' accumulators and writes their q_lat rows.
template <int R, int DR>
__device__ __forceinline__ void absorb_store(float (&acc)[2][8], int h0, int h1, bool two, int lane, u16* qlat,
                                             float cs) {
  constexpr int RW = R + DR;
  constexpr int OCT = R / 8;
  const int o = lane % OCT, p = lane / OCT;
#pragma unroll
  for (int off = OCT; off < 64; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off);
  if (p == 0) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1 && !two) break;
      const int h = hh ? h1 : h0;
      u16x8 vh, vl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = acc[hh][e] * cs;  // the latent cache's scale (1 for bf16 caches)
        const __bf16 x = (__bf16)y;
        vh[e] = __builtin_bit_cast(u16, x);
        vl[e] = f32_to_bf16(y - (float)x);
      }
      *reinterpret_cast<u16x8*>(qlat + h * RW + 8 * o) = vh;
      *reinterpret_cast<u16x8*>(qlat + (kHeadsPad + h) * RW + 8 * o) = vl;
    }
  }
}

// W_UV: out[b,h,i] = sum_j W_UV[h][i][j] o_lat[h][j] on 16x16x32 MFMA,
// out^T[16ib + 4grp + r][col] = sum_k A[i][k] B[k][col] with A = the W_UV[h] rows
// (as stored: 8 consecutive j per lane) and B = o_lat^T (its bf16 hi and lo
// parts, two products) with every column but h zeroed, so that column h of the
// product is head h's output.  Helper j takes heads j, j + 4, ...; the A
// operands of a batch of 16-row blocks of one head are requested together (the
// first batch while the stream runs).
template <int R>
struct UvBatch {
  static constexpr int kBlocks = R >= 256 ? 3 : 6;  // 96 registers of operands
  bf16x8 a[kBlocks][R / 32];
};

template <int R>
__device__ __forceinline__ void load_uv(UvBatch<R>& u, const MlaDecodeArgs& a, int h, int ib0, int lane) {
  const int row = lane & 15, grp = lane >> 4;
  const u16* base = static_cast<const u16*>(a.w_uv) + (size_t)h * a.dv * R;
#pragma unroll
  for (int ib = 0; ib < UvBatch<R>::kBlocks; ++ib) {
    const int i = min(16 * (ib0 + ib) + row, a.dv - 1);  // rows past dv: clamped, never stored
#pragma unroll
    for (int k = 0; k < R / 32; ++k)
      u.a[ib][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(base + (size_t)i * R + 32 * k + 8 * grp));
  }
}

// Applies a loaded batch (head h, blocks ib0..) to o_lat (olat: [2][16][R] bf16
// hi and lo parts in LDS) and writes the head's output rows.
template <int R>
__device__ __forceinline__ void apply_uv(const UvBatch<R>& u, const MlaDecodeArgs& a, const u16* olat, int b, int h,
                                         int ib0, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const bool mine = col == h;
  constexpr int NB = UvBatch<R>::kBlocks;
  const bf16x8 z = {};
  f32x4 acc[NB];
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) acc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < R / 32; ++k) {
    const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(olat + col * R + 32 * k + 8 * grp));
    const bf16x8 bl =
        __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(olat + (kHeadsPad + col) * R + 32 * k + 8 * grp));
    const bf16x8 oh = mine ? bh : z, ol = mine ? bl : z;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      acc[ib] = mfma_16x16x32(u.a[ib][k], oh, acc[ib]);
      acc[ib] = mfma_16x16x32(u.a[ib][k], ol, acc[ib]);
    }
  }
  if (mine) {
    const size_t o0 = ((size_t)b * a.H + h) * a.dv;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      acc[ib] *= a.c_scale;  // o_lat was summed over the latent cache's codes (scale 1 for bf16 caches)
      const int i = 16 * (ib0 + ib) + 4 * grp;
      if (i < a.dv) {  // dv is a multiple of 16: a block is valid as a whole
        if (a.out_bf16) {
          u16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = f32_to_bf16(acc[ib][r]);
          *reinterpret_cast<u16x4*>(static_cast<u16*>(a.out) + o0 + i) = v;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o0 + i) = acc[ib];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int R, int DR, bool PAGED, bool F8 = false>
__global__ __launch_bounds__(kThreads) void mla_decode(MlaDecodeArgs a) {
  using C = Cfg<R, DR, F8>;
  constexpr int RW = C::RW;
  constexpr int S = C::kStages;
  // ring stages, each a distinct LDS variable so that the compiler can tell the
  // copies in flight from the reads of the resident stage
  __shared__ __attribute__((aligned(1024))) u16 stg0[kWaves][C::kC];
  __shared__ __attribute__((aligned(1024))) u16 stg1[kWaves][C::kC];
  __shared__ __attribute__((aligned(1024))) u16 stg2[kWaves][C::kC];
  __shared__ alignas(S > 3 ? 1024 : 16) u16 stg3[S > 3 ? kWaves : 1][S > 3 ? C::kC : 8];
  __shared__ alignas(S > 4 ? 1024 : 16) u16 stg4[S > 4 ? kWaves : 1][S > 4 ? C::kC : 8];
  __shared__ __attribute__((aligned(1024))) u16 rop0[kWaves][C::kR];
  __shared__ __attribute__((aligned(1024))) u16 rop1[kWaves][C::kR];
  __shared__ __attribute__((aligned(1024))) u16 rop2[kWaves][C::kR];
  __shared__ alignas(S > 3 ? 1024 : 16) u16 rop3[S > 3 ? kWaves : 1][S > 3 ? C::kR : 8];
  __shared__ alignas(S > 4 ? 1024 : 16) u16 rop4[S > 4 ? kWaves : 1][S > 4 ? C::kR : 8];
  __shared__ __attribute__((aligned(16))) u16 qlat[2 * kHeadsPad * RW];  // [hi, lo][16][RW]
  __shared__ __attribute__((aligned(16))) u16 olat[2 * kHeadsPad * R];   // [hi, lo][16][R]
  __shared__ float lse_s[kHeadsPad];
  __shared__ float snew_s[kHeadsPad];  // decode step: the new token's log2 score per head
  __shared__ int last_s;
  // after the stream: one [16 heads][R] fp32 output slice per streaming wave,
  // two in each of stages 0 and 1; m and l per wave and head in stage 2
  static_assert(2 * kHeadsPad * R * 4 == (int)sizeof(stg0), "two output slices per stage");
  static_assert(2 * kWaves * kHeadsPad * 4 <= (int)sizeof(stg2), "m, l scratch");

  const int s = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const bool streamer = wave < kWaves;
  const int j = wave - kWaves;  // helper index
  // a helper's first round of absorb loads does not depend on the cache length:
  // it goes out while the length is read
  AbsorbLoads<R> ld;
  if (!streamer && j < a.H) absorb_issue<R>(ld, a, b, j, j + kHelpers < a.H ? j + kHelpers : j, 0, lane);
  const int L = clamp_len(a.lens[b], a.T_max);
  // a decode step with the new token has at least one (possibly empty) chunk,
  // whose workgroup adds the new token
  const int n_chunks = max((L + a.split - 1) / a.split, a.append ? 1 : 0);
  if (s >= n_chunks) {  // past the sequence; an empty sequence gets zeros from chunk 0
    wait_vmem();
    if (n_chunks == 0 && s == 0)
      for (int e = tid; e < a.H * a.dv; e += kThreads) {
        if (a.out_bf16) static_cast<u16*>(a.out)[(size_t)b * a.H * a.dv + e] = 0;
        else static_cast<float*>(a.out)[(size_t)b * a.H * a.dv + e] = 0.f;
      }
    return;
  }
  const int c0 = s * a.split, c1 = min(c0 + a.split, L);
  float* mw = reinterpret_cast<float*>(&stg2[0][0]);  // [waves][16]
  float* lw = mw + kWaves * kHeadsPad;                // [waves][16]
  auto slice = [&](int w) {
    return reinterpret_cast<float*>(w < 2 ? &stg0[0][0] : &stg1[0][0]) + (w & 1) * kHeadsPad * R;
  };

  WaveState<R, DR> st;
  // W_UV operands of the wave's first head: requested by a helper while the
  // stream runs, by a streaming wave once its ring has drained
  UvBatch<R> uv;
  // a streaming wave's ring stages and lane constants (made where they are used,
  // so that they take no registers in the helpers' code)
  auto stage_c = [&](int i) -> u16* {
    u16* const c[5] = {stg0[wave], stg1[wave], stg2[wave], stg3[S > 3 ? wave : 0], stg4[S > 4 ? wave : 0]};
    return c[i];
  };
  auto stage_r = [&](int i) -> u16* {
    u16* const r[5] = {rop0[wave], rop1[wave], rop2[wave], rop3[S > 3 ? wave : 0], rop4[S > 4 ? wave : 0]};
    return r[i];
  };
  const int tw0 = c0 + kSlice * wave;  // streaming wave: first token of its first slice

  // ---- the helpers absorb the query while the streaming waves start their
  // cache copies.  The copies go out once the helpers' first two rounds of
  // weight reads have (a bare barrier, no wait for the loads): issued after a
  // burst of cache copies, the weight reads waited behind the whole device's
  // burst in the memory queues.
  // paged: the chunk's page numbers (a chunk spans at most 128 pages), read by
  // the streaming waves before their first copies
  ChunkPages cpg = {0, {0, 0}};
  if (PAGED && streamer) {
    cpg.p0 = c0 / a.page_size;
    const int np = (c1 - 1) / a.page_size - cpg.p0 + 1;
    const int32_t* tb = a.block_table + (size_t)b * a.table_stride + cpg.p0;
    cpg.pg[0] = lane < np ? tb[lane] : 0;
    cpg.pg[1] = lane + 64 < np ? tb[lane + 64] : 0;
  }
  if (streamer) {
    const Lanes<R, DR, F8> ln(lane);
    __builtin_amdgcn_s_barrier();  // (0)
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      issue_slice<R, DR, PAGED, F8>(stage_c(i), stage_r(i), a, b, tw0 + i * kStep, c1, ln, cpg);
  } else {
    constexpr int P = 64 / (R / 8);
    constexpr int kRound = P * kAbsorbRows;  // W_UK rows per round
    u16 rope[4] = {0, 0, 0, 0};
    const u16* qr = static_cast<const u16*>(a.q_rope) + (size_t)b * a.H * DR + lane;
    if (lane < DR) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (j + i * kHelpers < a.H) rope[i] = qr[(j + i * kHelpers) * DR];
    }
    // the first pair (j, j + 4): its first round is in flight; barrier (0) after
    // the second round's loads are issued (or after the first round)
    {
      const int h0 = j, h1 = j + kHelpers;
      const bool have = h0 < a.H, two = h1 < a.H;
      float acc[2][8] = {};
      int k0 = 0;
      if (have) {
        absorb_dot<R>(acc, ld);
        k0 = kRound;
        if (k0 < a.dn) absorb_issue<R>(ld, a, b, h0, two ? h1 : h0, k0, lane);
      }
      __builtin_amdgcn_s_barrier();  // (0)
      absorb_fixed_parts<R, DR>(a, j, lane, rope, qlat);
      if (have) {
        for (; k0 < a.dn; k0 += kRound) {
          absorb_dot<R>(acc, ld);
          if (k0 + kRound < a.dn) absorb_issue<R>(ld, a, b, h0, two ? h1 : h0, k0 + kRound, lane);
        }
        absorb_store<R, DR>(acc, h0, h1, two, lane, qlat, a.c_scale);
      }
    }
    // further pairs (more than 8 heads)
    for (int h0 = j + 2 * kHelpers; h0 < a.H; h0 += 2 * kHelpers) {
      const int h1 = h0 + kHelpers;
      const bool two = h1 < a.H;
      float acc[2][8] = {};
      absorb_issue<R>(ld, a, b, h0, two ? h1 : h0, 0, lane);
      for (int k0 = 0; k0 < a.dn; k0 += kRound) {
        absorb_dot<R>(acc, ld);
        if (k0 + kRound < a.dn) absorb_issue<R>(ld, a, b, h0, two ? h1 : h0, k0 + kRound, lane);
      }
      absorb_store<R, DR>(acc, h0, h1, two, lane, qlat, a.c_scale);
    }
  }
  __syncthreads();  // (1) q_lat is complete
  if (streamer) {
    // ---- stream the wave's slices through the ring
    const Lanes<R, DR, F8> ln(lane);
    const int n_steps = (c1 - c0 + kStep - 1) / kStep;
    // q_lat^T as the B operand: lane holds q_lat[head row][32k + 8grp ..+8] (hi and lo)
    bf16x8 qhi[C::KC], qlo[C::KC], qr32[C::RC > 0 ? C::RC : 1], qr16 = {};
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
#pragma unroll
    for (int w = 0; w < C::DW; ++w) st.o[w] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.lsum = 0.f;
    const float c = a.scale_log2e;
    // Step k: copy slice k + S - 1 into stage (k + S - 1) % S, wait for slice
    // k, consume stage k % S.  The body is unrolled over the S stages, so every
    // copy comes from the same S places in the loop: the compiler then tracks
    // which stage each copy in flight belongs to across the back edge and adds
    // no waits beyond this one.  Copies of slices past the chunk read nothing.
    for (int k = 0; k < n_steps; k += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const int kk = k + i;
        issue_slice<R, DR, PAGED, F8>(stage_c((i + S - 1) % S), stage_r((i + S - 1) % S), a, b,
                                      tw0 + (kk + S - 1) * kStep, c1, ln, cpg);
        if (kk < n_steps) {
          wait_vmcnt<(S - 1) * C::kInstPerSlice>();
          if constexpr (F8) widen_slice<R>(stage_c(i), lane);
          slice_step<R, DR, F8>(st, stage_c(i), stage_r(i), qhi, qlo, qr32, qr16, tw0 + kk * kStep, c1, c, ln);
        }
      }
    }
    wait_vmem();  // the copies past the end (zeros) land before the stages are reused
    st.lsum = sum_xor32(sum_xor16(st.lsum));
    // the W_UV operands of this wave's head (wave + 4): requested now, in
    // registers by the time o_lat is merged
    if (wave + kHelpers < a.H) load_uv<R>(uv, a, wave + kHelpers, 0, lane);
  }
  if (!streamer) {
    if (j < a.H) load_uv<R>(uv, a, j, 0, lane);
    // decode step: the new token's score, scale * q_lat . [c_new, k_rope_new], per head
    if (a.append) {
      const u16* cn = static_cast<const u16*>(a.c_new) + (size_t)b * R;
      const u16* kn = static_cast<const u16*>(a.kr_new) + (size_t)b * DR;
      for (int h = j; h < a.H; h += kHelpers) {
        float acc = 0.f;
        for (int e = lane; e < RW; e += 64) {
          const float x = bf16_to_f32(e < R ? cn[e] : kn[e - R]);
          acc = fmaf(bf16_to_f32(qlat[h * RW + e]) + bf16_to_f32(qlat[(kHeadsPad + h) * RW + e]), x, acc);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) snew_s[h] = acc * a.scale_log2e;
      }
    }
  }

  // ---- merge the four streaming waves (LDS, reusing the stages)
  // Each wave writes its scaled O^T into its own [16][R] slice; 16-byte unit u
  // of head row h sits at unit position u ^ (h & 15), so the 16 rows of one
  // write land on distinct banks.
  __syncthreads();  // (2) every streaming wave is done with its ring
  const int row = lane & 15, grp = lane >> 4;
  if (streamer && grp == 0) {
    mw[wave * kHeadsPad + row] = st.m;
    lw[wave * kHeadsPad + row] = st.lsum;
  }
  __syncthreads();  // (3)
  if (streamer) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w * kHeadsPad + row]);
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Lt += rescale(mw[w * kHeadsPad + row], M) * lw[w * kHeadsPad + row];
    const float f = Lt > 0.f ? rescale(st.m, M) / Lt : 0.f;  // an empty chunk (decode step, L = 0)
    float* ob = slice(wave) + row * R;
#pragma unroll
    for (int dw = 0; dw < C::DW; ++dw)
      *reinterpret_cast<f32x4*>(ob + 4 * ((4 * dw + grp) ^ row)) = st.o[dw] * f;
    if (wave == 0 && grp == 0) lse_s[row] = M + __log2f(Lt);
  }
  __syncthreads();  // (4)

  // this chunk's normalised o_lat (the sum of the four slices): as the hi / lo
  // operand of W_UV when it is the sequence's only chunk, else to the workspace
  const bool single = n_chunks == 1;
  const size_t prow = ((size_t)b * a.n_splits + s) * a.H;  // partial rows of this chunk
  for (int e = tid; e < a.H * (R / 4); e += kThreads) {
    const int h = e / (R / 4), d4 = e - h * (R / 4);
    const int off = h * R + 4 * (d4 ^ (h & 15));
    f32x4 v = *reinterpret_cast<const f32x4*>(slice(0) + off);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += *reinterpret_cast<const f32x4*>(slice(w) + off);
    if (single) {
      if (a.append) {  // the new token as one more partial
        const float lo = lse_s[h], sn = snew_s[h];
        const float M = fmaxf(lo, sn);
        const float wo = rescale(lo, M), wn = exp2_fast(sn - M), inv = 1.f / (wo + wn);
        const u16* cn = static_cast<const u16*>(a.c_new) + (size_t)b * R + 4 * d4;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (wo * v[r] + wn * bf16_to_f32(cn[r])) * inv;
      }
      u16x4 vh, vl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 x = (__bf16)v[r];
        vh[r] = __builtin_bit_cast(u16, x);
        vl[r] = f32_to_bf16(v[r] - (float)x);
      }
      *reinterpret_cast<u16x4*>(olat + h * R + 4 * d4) = vh;
      *reinterpret_cast<u16x4*>(olat + (kHeadsPad + h) * R + 4 * d4) = vl;
    } else {
      float* dst = a.o_part + (prow + h) * R + 4 * d4;
#pragma unroll
      for (int r = 0; r < 4; ++r) store_coherent(dst + r, v[r]);
    }
  }
  if (!single) {
    for (int h = tid; h < a.H; h += kThreads) store_coherent(a.lse + prow + h, lse_s[h]);
    wait_vmem();      // this thread's partial stores have completed
    __syncthreads();  // (5) ... and every thread's
    if (tid == 0) {
      const unsigned before = __hip_atomic_fetch_add(a.done + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_s = before == (unsigned)(n_chunks - 1);
    }
    __syncthreads();  // (6)
    if (!last_s) return;
    // the last chunk to finish: merge every chunk's partial by its log2-sum-exp
    if (tid == 0) __hip_atomic_store(a.done + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const size_t row0 = (size_t)b * a.n_splits * a.H;
    for (int e = tid; e < a.H * R; e += kThreads) {
      const int h = e / R, d = e - h * R;
      float M = kNegInf, Ssum = 0.f, acc = 0.f;
      for (int k0 = 0; k0 < n_chunks; k0 += 8) {
        float lv[8], ov[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = min(k0 + u, n_chunks - 1);
          lv[u] = load_coherent(a.lse + row0 + (size_t)k * a.H + h);
          ov[u] = load_coherent(a.o_part + (row0 + (size_t)k * a.H + h) * R + d);
        }
        // chunks past the end (loaded clamped) weigh 2^-inf = 0; entry 0 of the
        // first batch is a real chunk, so M is finite before any of them
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k0 + u >= n_chunks) lv[u] = kNegInf;
          const float Mn = fmaxf(M, lv[u]);
          const float f = rescale(M, Mn), w = exp2_fast(lv[u] - Mn);
          Ssum = Ssum * f + w;
          acc = acc * f + w * ov[u];
          M = Mn;
        }
      }
      if (a.append) {  // the new token as one more partial
        const float sn = snew_s[h];
        const float Mn = fmaxf(M, sn);
        const float f = rescale(M, Mn), w = exp2_fast(sn - Mn);
        Ssum = Ssum * f + w;
        acc = acc * f + w * bf16_to_f32(static_cast<const u16*>(a.c_new)[(size_t)b * R + d]);
      }
      const float v = acc / Ssum;
      const __bf16 x = (__bf16)v;
      olat[h * R + d] = __builtin_bit_cast(u16, x);
      olat[(kHeadsPad + h) * R + d] = f32_to_bf16(v - (float)x);
    }
  }
  __syncthreads();  // (7) o_lat is in LDS

  // decode step: the new token's rows go into the caches (every chunk of the
  // sequence has finished reading them, and none reads row L)
  if (a.append && L < a.T_max) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if (tid < R / 8)
      reinterpret_cast<u32x4*>(static_cast<u16*>(a.c_cache) + ((size_t)b * a.T_max + L) * R)[tid] =
          reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.c_new) + (size_t)b * R)[tid];
    else if (tid >= 64 && tid < 64 + DR / 8)
      reinterpret_cast<u32x4*>(static_cast<u16*>(a.kr_cache) + ((size_t)b * a.T_max + L) * DR)[tid - 64] =
          reinterpret_cast<const u32x4*>(static_cast<const u16*>(a.kr_new) + (size_t)b * DR)[tid - 64];
  }

  // ---- out = W_UV o_lat, all eight waves: helper j takes heads j, j + 8, ...,
  // streaming wave w heads w + 4, w + 12, ... (each wave's first batch already
  // in registers)
  {
    const int h0 = streamer ? wave + kHelpers : j;
    const int nb = a.dv / 16;
    for (int h = h0; h < a.H; h += kWaves + kHelpers) {
      for (int ib0 = 0; ib0 < nb; ib0 += UvBatch<R>::kBlocks) {
        if (h != h0 || ib0 != 0) load_uv<R>(uv, a, h, ib0, lane);
        apply_uv<R>(uv, a, olat, b, h, ib0, lane);
      }
    }
  }
}

template <int R, int DR>
hipError_t launch_rd(const MlaDecodeArgs& a, hipStream_t st) {
  if (a.c_fp8 && a.block_table)
    hipLaunchKernelGGL((mla_decode<R, DR, true, true>), dim3(a.n_splits, a.B), dim3(kThreads), 0, st, a);
  else if (a.c_fp8) hipLaunchKernelGGL((mla_decode<R, DR, false, true>), dim3(a.n_splits, a.B), dim3(kThreads), 0, st, a);
  else if (a.block_table) hipLaunchKernelGGL((mla_decode<R, DR, true>), dim3(a.n_splits, a.B), dim3(kThreads), 0, st, a);
  else hipLaunchKernelGGL((mla_decode<R, DR, false>), dim3(a.n_splits, a.B), dim3(kThreads), 0, st, a);
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
  if (a.split % kStep != 0 || a.dv % 16 != 0 || a.dv > 256 || a.dn > 256 || !a.done) return hipErrorInvalidValue;
  if (a.block_table && (a.page_size <= 0 || a.page_size % kSlice != 0 || a.n_pages <= 0 || a.append ||
                        a.split / a.page_size + 2 > 128))
    return hipErrorInvalidValue;
  if (a.c_fp8 && (a.append || !(a.c_scale > 0.f))) return hipErrorInvalidValue;
  return a.r == 64 ? launch_r<64>(a, st) : a.r == 128 ? launch_r<128>(a, st) : launch_r<256>(a, st);
}

}  // namespace attn
