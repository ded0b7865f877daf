// Causal GQA prefill on bf16 MFMA for gfx950, with or without a cached prefix.
//
// What is computed: out[b,i,h] = sum_{j<=P+i} softmax_j(scale q[b,i,h].k[b,j,g]) v[b,j,g]
// with g = floor(h / n_rep) and P = start_pos[b] the number of cached positions
// before the new tokens -- Attention.forward of the "模型架构｜MQA & GQA 调研"
// page (code section): the new K/V rows sit in the cache at start_pos.., the keys
// are the first start_pos + seqlen cache rows, and the additive causal mask is
// aligned to the bottom right, so new token i (position P + i) sees every cached
// position up to its own.  P = 0 is the scaled_dot_product_attention(is_causal=True)
// call in the MultiHeadLatentAttention listing of the qqstock DeepSeek MLA
// article.  Rows i >= q_lens[b] are written as zeros.  P is rounded to bf16
// before the PV product, as the page's softmax(...).type_as(xq) does.
//
// How (not from the pages; designed for CDNA4):
//  * One workgroup = 4 waves = a tile of 128 query rows of one (head, sequence);
//    each wave owns 32 rows.  The linear workgroup id is mapped so that all heads
//    of one KV group of one sequence run on the same XCD (one L2), heaviest
//    q-tiles (most keys) first.
//  * K/V tiles of 64 keys go HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    staging registers, no LDS write instructions), double-buffered, one barrier
//    per tile.  The buffer resource ends at the sequence's last key, so keys past
//    it read as zeros without address clamping.  Key rows are stored unpadded
//    with their 16-byte chunks XOR-swizzled by key, which keeps the 16-byte K
//    operand reads and the transposed V reads free of bank conflicts on the
//    256-byte-per-clock LDS.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a 32-key K block is the A operand,
//    the wave's Q^T is the B operand, held in registers for the whole kernel.  The
//    accumulator gives each lane one query row (lane % 32) and 16 keys.
//  * O^T += V^T P^T: P stays in the accumulator layout and is the B operand after
//    a key permutation shared with the A operand; V^T comes from the row-major V
//    tile through ds_read_b64_tr_b16.
//  * Online softmax in base 2.  The query operand is scaled by scale * log2(e)
//    once (rounded to bf16, as the query itself is), and each tile's score
//    products accumulate onto -m, the row's reference max, held in a register
//    block that is the first MFMA's C operand: a probability is then one
//    v_exp_f32 of the accumulator.  The row sum adds the bf16-rounded
//    probabilities the PV product uses.  The reference max only moves (and O, l
//    and the tile's scores are shifted) when a tile's max exceeds it by more
//    than 2^8: probabilities then stay below 256, far inside bf16 and fp32
//    range, and most tiles skip the rescale.
//  * A wave skips tiles entirely above its diagonal; only diagonal tiles mask.
//    With a prefix the diagonal is shifted right by P; a q-tile with no new
//    token left writes zeros and reads nothing.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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
// VALU-write -> permlane-read hazard.  Not volatile: it touches no memory, so
// the scheduler may move loads and other arithmetic across it.
__device__ __forceinline__ float2 pair_xor32(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float max_xor32(float x) { const float2 p = pair_xor32(x); return fmaxf(p.x, p.y); }
__device__ __forceinline__ float sum_xor32(float x) { const float2 p = pair_xor32(x); return p.x + p.y; }

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight bf16 query elements times f, rounded back to bf16 (the query operand of
// the score products).
__device__ __forceinline__ bf16x8 scaled_operand(u16x8 x, float f) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)(__builtin_bit_cast(float, (unsigned)x[e] << 16) * f);
  return r;
}

// ds_read_b64_tr_b16: lane i of a 16-lane group points at row T0 + i/4, columns
// 4(i%4).. of a row-major [key][dim] block; lane j receives keys T0..T0+3 of
// column j.
__device__ __forceinline__ u16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}

// 16-byte chunk c of key row r sits at chunk position c ^ swz<D>(r).  gfx950's
// LDS serves 256 bytes per clock: 16 lanes of a 16-byte read, 32 lanes of an
// 8-byte read.  K operand reads take one chunk index from 16 consecutive keys,
// so swz must be a bijection on 16 consecutive keys modulo the 256-byte bank
// period; transposed V reads take an aligned block of 4 chunks from 4
// consecutive keys, so those keys must land the block on 4 different blocks.
// D = 128 (256-byte rows): swz = 4 (r % 4) + (r / 4) % 4.
// D = 64 (128-byte rows, two per bank period): swz = 4 ((r / 2) % 2) + (r / 4) % 4.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// HBM -> LDS copies of 64-key tiles of K or V (D/8 16-byte chunks per key) with
// buffer_load_dwordx4 ... lds.  Each lane of an instruction writes its 16 bytes at
// LDS base + 16 * lane, so the lane fetches the chunk that belongs at that
// position.  The buffer resource of a tile starts at the tile's first key and
// ends after the sequence's last key (nothing for a tile outside 0..n_kt-1):
// reads past it return zeros, so keys beyond the sequence and pipeline fill or
// drain tiles cost no memory traffic and need no clamping.
template <int D>
struct TileCopy {
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerInst = 64 / kChunks;
  static constexpr int kInst = kBN / kRowsPerInst / kWaves;  // instructions per wave and tile
  int voff[kInst];  // per-lane byte offset within the tile
  int wave;

  __device__ __forceinline__ TileCopy(int wave_, int lane, int row_bytes) : wave(wave_) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int r = (wave * kInst + i) * kRowsPerInst + lane / kChunks;
      voff[i] = r * row_bytes + 16 * ((lane % kChunks) ^ swz<D>(r));
    }
  }

  // payload: bytes of one key's row that belong to this head (2 * D unless the
  // source rows are narrower than the LDS rows)
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const u16* p, int kt, int n_kt, int kv_len,
                                                                int row_bytes, int payload = 2 * D) {
    const bool ok = kt >= 0 && kt < n_kt;
    const int key0 = ok ? kt * kBN : 0;
    const char* base = reinterpret_cast<const char*>(p) + (size_t)key0 * row_bytes;
    const unsigned long long end = (unsigned long long)(kv_len - 1 - key0) * row_bytes + payload;
    const unsigned num = ok ? (unsigned)(end < 0xffffffffull ? end : 0xffffffffull) : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)num, 0x00020000);
  }

  __device__ __forceinline__ void issue(u16* lds_tile, __amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int i = 0; i < kInst; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(lds_tile + (wave * kInst + i) * kRowsPerInst * D), 16,
          voff[i], 0, 0, 0);
  }
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Workgroup id -> (q-tile, head, sequence).  Workgroups are dealt to the 8 XCDs
// round-robin by id.  When the (sequence, KV group) pairs split evenly over the
// XCDs, each XCD gets whole groups, so a group's K/V is read through one L2;
// within an XCD the heaviest q-tiles go first.  Otherwise: heaviest q-tile
// first, heads fastest.
struct Tile {
  int qt, h, b;
};
__device__ __forceinline__ Tile map_tile(int S, int B, int Hq, int Hkv, int n_rep, int id) {
  const int n_qt = (S + kBM - 1) / kBM;
  const int groups = B * Hkv;
  Tile t;
  if (groups % 8 == 0) {
    const int xcd = id & 7, slot = id >> 3;
    const int gpx = groups / 8;
    const int per_rank = gpx * n_rep;
    const int rank = slot / per_rank, rem = slot - rank * per_rank;
    const int grp = xcd * gpx + rem / n_rep;
    t.qt = n_qt - 1 - rank;
    t.b = grp / Hkv;
    t.h = (grp - t.b * Hkv) * n_rep + rem % n_rep;
  } else {
    const int per_rank = B * Hq;
    const int rank = id / per_rank, rem = id - rank * per_rank;
    t.qt = n_qt - 1 - rank;
    t.b = rem / Hq;
    t.h = rem - t.b * Hq;
  }
  return t;
}

// Per-lane constants of a wave.  row0 / my_row index the new tokens; pos0 /
// my_pos are their positions in the sequence (P added), which the causal cut uses.
struct Lane {
  int lane, ln, h2, row0, my_row, pos0, my_pos;
  float c;  // softmax scale * log2(e)
};

// LDS element offsets.  swz<D>(key) depends on key only through key % 16 in a way
// that is the same for keys 32j + ln (j = 0, 1) and for keys 16v + x (v = 0..3),
// and row r starts at r * D, whose low bits are clear.  So chunk c of key row
// `key` sits at (key * D + 8 * (h ^ swz)) ^ (16 * c') for c = 2c' + h, and the
// block of 4 chunks 4d + (0..3) of a transposed read at (...) ^ (32 * d): one
// per-lane base, XORed with a constant, plus an immediate for the key block.
struct LdsOffsets {
  int k;      // K operand read of chunk h2 of key ln
  int v_lo;   // transposed V read, lower key quad of step 0, dim block 0
  int v_hi;   // ... upper key quad
};

template <int D>
__device__ __forceinline__ LdsOffsets lds_offsets(const Lane& w) {
  LdsOffsets o;
  o.k = w.ln * D + 8 * (w.h2 ^ swz<D>(w.ln));
  const int g16 = (w.lane >> 4) & 1, i16 = w.lane & 15;
  const int vc = 2 * g16 + ((i16 & 3) >> 1);  // chunk within the dim block
  const int klo = 4 * w.h2 + (i16 >> 2), khi = klo + 8;
  o.v_lo = klo * D + 4 * (i16 & 1) + 8 * (vc ^ swz<D>(klo));
  o.v_hi = khi * D + 4 * (i16 & 1) + 8 * (vc ^ swz<D>(khi));
  return o;
}

// S^T of one tile from the K tile kc: lane holds S^T[key 32j + 8(i/4) + 4h2 + i%4][row ln]
// (keys relative to the tile) plus init (the row's -m).  A = 32-key K block, B =
// the wave's scaled Q^T.  D is the head size, DL the LDS row pitch of the tile
// (>= D).
template <int D, int DL = D>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const u16* kc, const bf16x8 (&qop)[D / 16], int off,
                                        const f32x16& init) {
  s[0] = init;
  s[1] = init;
  // the two 32-key blocks' chains alternate, so no MFMA waits for the one before it
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u16* kr = kc + 32 * j * DL + (off ^ (16 * c));
      s[j] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr)), qop[c], s[j]);
    }
  // issue order: operand reads four MFMAs ahead of their use
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int u = 0; u < 2 * (D / 16); ++u) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// O^T[dims 32d..][rows] += V^T P^T over one tile from the V tile vc.  Step v of the
// contraction covers keys 16v + 4h2 + (0..3) and 16v + 8 + 4h2 + (0..3); 16-lane
// group (g16, h2) of a transposed read points at key 16v + 4h2 + (i16 >> 2) (+8),
// dims 32d + 16g16 + 4(i16 & 3).
template <int D, int DL = D>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[D / 32], const u16* vc, const bf16x8 (&p)[4], int off_lo,
                                        int off_hi) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
      const u16x4 lo = lds_read_tr16(vc + 16 * v * DL + (off_lo ^ (32 * d)));
      const u16x4 hi = lds_read_tr16(vc + 16 * v * DL + (off_hi ^ (32 * d)));
      const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[d] = mfma_32x32x16(__builtin_bit_cast(bf16x8, av), p[v], o[d]);
    }
  }
}

// Running state of one wave: O^T accumulators, reference max m (log2 units of
// the scaled scores), -m in all 16 elements (the score products' initial
// accumulator), partial row sum.
template <int D>
struct RowState {
  f32x16 o[D / 32];
  f32x16 negm;
  float m, lsum;
};

template <int D>
__device__ __forceinline__ void init_rows(RowState<D>& st) {
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[d][i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) st.negm[i] = 0.f;
  st.m = 0.f;  // replaced by the first tile's max
  st.lsum = 0.f;
}

// Online softmax of one tile's scores sc (S^T layout of qk_tile, already scaled
// and relative to the reference max): masks the keys at positions past each
// row's cut (its own position, or the last cached position for a tile of cached
// keys), moves the reference max when needed (shifting the tile's scores and
// rescaling O and the row sum), and returns the probabilities as the four bf16
// P^T operands of PV.  kv0: position of the tile's first key; cut0: the lowest
// cut of the wave's rows (wave-uniform), cut: this lane's row's cut; first: the
// wave's first tile, which sets the reference (key 0 is visible to every row, so
// its max is finite).
template <int D>
__device__ __forceinline__ void softmax_tile(RowState<D>& st, f32x16 (&sc)[2], bf16x8 (&pop)[4], int kv0, int cut0,
                                             int cut, bool first, const Lane& w) {
  if (kv0 + kBN - 1 > cut0) {  // the tile reaches past the cut of some row
    const int t = cut - kv0 - 4 * w.h2;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[j][i] = 32 * j + 8 * (i >> 2) + (i & 3) <= t ? sc[j][i] : kNegInf;
  }
  float mr = kNegInf;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) mr = fmaxf(mr, sc[j][i]);
  const float mt = max_xor32(mr);  // the row's max above the reference
  if (first || __builtin_amdgcn_ballot_w64(mt > kRescaleSlack) != 0) {
    const float mn = st.m + (first ? mt : fmaxf(mt, 0.f));
    const float shift = mn - st.m;
    const float alpha = first ? 0.f : exp2_fast(st.m - mn);  // O and l are still zero on the first tile
    st.m = mn;
    st.lsum *= alpha;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) st.o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[j][i] -= shift;
#pragma unroll
    for (int i = 0; i < 16; ++i) st.negm[i] = -mn;
  }
  // P^T operand of PV step v: S^T block v/2, values 8(v%2)..+8
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) pop[v][jj] = (__bf16)exp2_fast(sc[v >> 1][8 * (v & 1) + jj]);
  // row sum of the bf16-rounded probabilities (the ones the PV product uses),
  // two per v_dot2_f32_bf16 against (1, 1), in four independent chains
  const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
  float ps4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < 4; ++v)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x2 pair = {pop[v][2 * q], pop[v][2 * q + 1]};
      ps4[q] = __builtin_amdgcn_fdot2_f32_bf16(pair, one, ps4[q], false);
    }
  st.lsum += (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
}

// Where the keys of a sequence come from.  Tiles 0 .. n1-1 hold positions
// 0 .. P-1 from the cache (k, v); tiles n1 .. n_kt-1 hold positions P .. from
// the new rows (kn, vn), one 64-key tile after another.  Without separate new
// rows n1 = n_kt and every tile comes from the cache.  PAGED: the cache is a
// pool of pages (k and v point at the KV head's columns of the pool's first
// row), and tile kt, which lies in one page (page_size a multiple of 64), starts
// at row page * page_size + (64 kt mod page_size) of the pool, its page number
// read from the sequence's block-table row trow (a scalar load per tile).
template <int D, int DL, bool PAGED = false>
struct KeySource {
  const u16 *k, *v, *kn, *vn;
  int row_bytes;
  int P, n1, n_kt;
  int len1, len2;  // keys in the first and in the second source
  const int32_t* trow = nullptr;
  int page_size = 0, n_pages = 0;

  __device__ __forceinline__ int kv0(int kt) const { return kt < n1 ? kt * kBN : P + (kt - n1) * kBN; }
  __device__ __forceinline__ void issue(const TileCopy<DL>& cp, u16* kl, u16* vl, int kt) const {
    if constexpr (PAGED) {
      const bool ok = kt >= 0 && kt < n_kt;
      const int key0 = ok ? kt * kBN : 0;
      const int e = ok ? __builtin_amdgcn_readfirstlane(trow[key0 / page_size]) : 0;
      const int page = min(max(e, 0), n_pages - 1);
      const size_t row0 = (size_t)page * page_size + (size_t)(key0 - (key0 / page_size) * page_size);
      const int rows = min(len1 - key0, kBN);
      const int num = ok && rows > 0 ? (rows - 1) * row_bytes + 2 * D : 0;
      const char* kb = reinterpret_cast<const char*>(k) + row0 * row_bytes;
      const char* vb = reinterpret_cast<const char*>(v) + row0 * row_bytes;
      cp.issue(kl, __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), (short)0, num, 0x00020000));
      cp.issue(vl, __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), (short)0, num, 0x00020000));
      return;
    }
    if (kt < n1) {
      cp.issue(kl, TileCopy<DL>::rsrc(k, kt, n1, len1, row_bytes, 2 * D));
      cp.issue(vl, TileCopy<DL>::rsrc(v, kt, n1, len1, row_bytes, 2 * D));
    } else {
      cp.issue(kl, TileCopy<DL>::rsrc(kn, kt - n1, n_kt - n1, len2, row_bytes, 2 * D));
      cp.issue(vl, TileCopy<DL>::rsrc(vn, kt - n1, n_kt - n1, len2, row_bytes, 2 * D));
    }
  }
};

// One 64-key tile: issue the copies of tile kt+1 into (kn, vn), consume tile kt
// from (kc, vc) if some row of the wave sees it, then wait for the copies and
// meet at the barrier.  The four buffers are distinct LDS variables addressed
// directly, so the compiler can tell the copies in flight from the reads of the
// current tile and does not wait for them before reading.  Tiles of the cache
// (kt < n1) when the new rows come separately are cut at the last cached
// position P - 1 (their tail reads as zeros); the others at each row's own
// position.
template <int D, int DL, bool PAGED>
__device__ __forceinline__ void tile_step(RowState<D>& st, const u16* kc, const u16* vc, u16* kn, u16* vn,
                                          const bf16x8 (&qop)[D / 16], int kt, int last_kt,
                                          const KeySource<D, DL, PAGED>& src, const TileCopy<DL>& cp,
                                          const LdsOffsets& off, const Lane& w) {
  if (kt + 1 < src.n_kt) src.issue(cp, kn, vn, kt + 1);  // (kn, vn) were released by the last barrier
  if (kt <= last_kt) {
    f32x16 sc[2];
    qk_tile<D, DL>(sc, kc, qop, off.k, st.negm);
    bf16x8 pop[4];
    const bool cached_tile = kt < src.n1 && src.n1 < src.n_kt;
    softmax_tile<D>(st, sc, pop, src.kv0(kt), cached_tile ? src.P - 1 : w.pos0, cached_tile ? src.P - 1 : w.my_pos,
                    kt == 0, w);
    pv_tile<D, DL>(st.o, vc, pop, off.v_lo, off.v_hi);
  }
  wait_vmem();      // this thread's copies of tile kt+1 have landed
  __syncthreads();  // ... and everyone's; nobody reads tile kt any more
}

// Stores one output row from the O^T accumulators (lane holds O^T[dims
// 32d + 8(i/4) + 4h2 + (i%4)][row ln]) times inv, or zeros when !valid.
template <int D>
__device__ __forceinline__ void store_rows(void* out, size_t orow, int out_bf16, const f32x16 (&o)[D / 32], bool valid,
                                           float inv, int h2) {
  constexpr int DB = D / 32;
  if (out_bf16) {
    u16* op = static_cast<u16*>(out) + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = __builtin_bit_cast(u16, (__bf16)(valid ? o[d][4 * q4 + e] * inv : 0.f));
        *reinterpret_cast<u16x4*>(op + 32 * d + 8 * q4 + 4 * h2) = o4;
      }
  } else {
    float* op = static_cast<float*>(out) + orow * D;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) f = make_float4(o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv, o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
        *reinterpret_cast<float4*>(op + 32 * d + 8 * q4 + 4 * h2) = f;
      }
  }
}

// MODE 0: no prefix (start_pos null); 1: a cached prefix, the new rows already
// in the cache; 2: a cached prefix, the new rows in their own arrays (k_new,
// v_new), read from there and written into the cache at P.. by the workgroups
// of the first head of each KV group; 3: mode 1 over a paged cache (k and v are
// page pools, block_table maps each sequence's positions to pages).  Modes 0
// and 1 run the same code; the separate symbols keep them apart in kernel
// profiles.
template <int D, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_causal(PrefillArgs a) {
  static_assert(D % 32 == 0 && D <= 128, "head_dim");
  static_assert(kBM == 32 * kWaves, "one 32-row slice per wave");
  constexpr int KC = D / 16;
  // LDS row pitch: head_dim 96 rows (192 bytes, which no 16-byte XOR swizzle
  // covers) sit in the head_dim-128 layout; the copies' lanes that fall past the
  // row's 12 chunks read the next bytes or zeros, and QK and PV never read those
  // columns
  constexpr int DL = D == 96 ? 128 : D;
  constexpr int kTile = kBN * DL;
  __shared__ __attribute__((aligned(1024))) u16 k0[kTile];
  __shared__ __attribute__((aligned(1024))) u16 k1[kTile];
  __shared__ __attribute__((aligned(1024))) u16 v0[kTile];
  __shared__ __attribute__((aligned(1024))) u16 v1[kTile];

  const Tile tl = map_tile(a.S, a.B, a.Hq, a.Hkv, a.n_rep, blockIdx.x);
  const int h = tl.h, b = tl.b;
  const int g = h / a.n_rep;
  const int q0 = tl.qt * kBM;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // cached prefix P (clamped to the cache) and new tokens n_q (clamped to S and
  // to the room left in the cache)
  const int P = a.start_pos ? min(max(a.start_pos[b], 0), a.T_kv) : 0;
  const int n_q = min(a.q_lens ? min(max(a.q_lens[b], 0), a.S) : a.S, a.T_kv - P);
  Lane w;
  w.lane = tid & 63;
  w.ln = w.lane & 31;
  w.h2 = w.lane >> 5;
  w.row0 = q0 + wave * 32;
  w.my_row = w.row0 + w.ln;
  w.pos0 = P + w.row0;
  w.my_pos = P + w.my_row;
  w.c = a.scale_log2e;

  const size_t q_row = (size_t)a.Hq * D;
  const int row_bytes = a.Hkv * D * 2;
  const size_t orow = ((size_t)b * a.S + w.my_row) * a.Hq + h;
  if (q0 >= n_q) {  // no new token in this q-tile: zero rows, nothing to read
    const f32x16 none[D / 32] = {};
    if (w.my_row < a.S) store_rows<D>(a.out, orow, a.out_bf16, none, false, 0.f, w.h2);
    return;
  }
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)b * a.S * a.Hq + h) * D;
  // (paged: the KV head's columns of the pool's first row; the tiles add their page's rows)
  const u16* kp = static_cast<const u16*>(a.k) + ((MODE == 3 ? 0 : (size_t)b * a.T_kv * a.Hkv) + g) * D;
  const u16* vp = static_cast<const u16*>(a.v) + ((MODE == 3 ? 0 : (size_t)b * a.T_kv * a.Hkv) + g) * D;

  // keys of the sequence: [0, kv_len); keys needed by the workgroup:
  // [0, min(kv_len, P + q0 + BM)); tiles 0..last_kt are visible to some row of
  // this wave
  const int kv_len = P + n_q;
  const int kv_end = min(kv_len, P + q0 + kBM);
  KeySource<D, DL, MODE == 3> src;
  if constexpr (MODE == 3) {
    src.trow = a.block_table + (size_t)b * a.table_stride;
    src.page_size = a.page_size;
    src.n_pages = a.n_pages;
  }
  src.k = kp;
  src.v = vp;
  src.row_bytes = row_bytes;
  src.P = P;
  int last_kt;
  if constexpr (MODE == 2) {  // the new rows have the same layout as the cache's, S rows per sequence
    src.kn = static_cast<const u16*>(a.k_new) + ((size_t)b * a.S * a.Hkv + g) * D;
    src.vn = static_cast<const u16*>(a.v_new) + ((size_t)b * a.S * a.Hkv + g) * D;
    src.n1 = (P + kBN - 1) / kBN;
    src.n_kt = src.n1 + (kv_end - P + kBN - 1) / kBN;
    src.len1 = P;
    src.len2 = n_q;
    last_kt = min(src.n_kt - 1, src.n1 + (w.row0 + 31) / kBN);
  } else {
    src.kn = kp;
    src.vn = vp;
    src.n_kt = src.n1 = (kv_end + kBN - 1) / kBN;
    src.len1 = src.len2 = kv_len;
    last_kt = min(src.n_kt - 1, (w.pos0 + 31) / kBN);
  }
  const int n_kt = src.n_kt;

  const TileCopy<DL> cp(wave, w.lane, row_bytes);
  src.issue(cp, k0, v0, 0);
  const LdsOffsets off = lds_offsets<DL>(w);

  // (scale * log2 e) Q^T as the B operand: lane holds Q[row ln][16c + 8h2 ..+8]
  bf16x8 qop[KC];
  {
    const u16* qr = qp + (size_t)min(w.my_row, a.S - 1) * q_row + 8 * w.h2;
#pragma unroll
    for (int c = 0; c < KC; ++c) qop[c] = scaled_operand(*reinterpret_cast<const u16x8*>(qr + 16 * c), w.c);
  }

  RowState<D> st;
  init_rows(st);

  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile_step<D, DL, MODE == 3>(st, k0, v0, k1, v1, qop, kt, last_kt, src, cp, off, w);
    if (kt + 1 < n_kt) tile_step<D, DL, MODE == 3>(st, k1, v1, k0, v0, qop, kt + 1, last_kt, src, cp, off, w);
  }

  // normalise and store; rows past the new tokens are zeros
  const float lsum = sum_xor32(st.lsum);
  if (w.my_row < a.S) store_rows<D>(a.out, orow, a.out_bf16, st.o, w.my_row < n_q, 1.f / lsum, w.h2);

  if constexpr (MODE == 2) {
    // the cache write of this q-tile's new rows (first head of the KV group
    // only): rows q0 .. min(q0 + BM, n_q) - 1 to cache rows P + q0 ..  No
    // workgroup of this launch reads cache rows at or past P.
    if (h % a.n_rep == 0) {
      constexpr int kChunks = D / 8;  // 16-byte chunks of a row of one KV head
      const int rows = min(kBM, n_q - q0);
      const size_t ld = (size_t)a.Hkv * D;  // elements between rows, both sides
      u16* kc = const_cast<u16*>(kp) + (size_t)(P + q0) * ld;
      u16* vc = const_cast<u16*>(vp) + (size_t)(P + q0) * ld;
      const u16* kn = src.kn + (size_t)q0 * ld;
      const u16* vn = src.vn + (size_t)q0 * ld;
      for (int i = tid; i < rows * kChunks; i += 256) {
        const size_t e = (size_t)(i / kChunks) * ld + 8 * (i % kChunks);
        const u16x8 kx = *reinterpret_cast<const u16x8*>(kn + e);
        const u16x8 vx = *reinterpret_cast<const u16x8*>(vn + e);
        *reinterpret_cast<u16x8*>(kc + e) = kx;
        *reinterpret_cast<u16x8*>(vc + e) = vx;
      }
    }
  }
}


// ---------------------------------------------------------------------------
// MLA causal prefill, absorbed form.
//
// What is computed: out[b,i,h] = W_UV[h] sum_{j<=P+i} softmax_j(scale (q_c . c_j +
// q_rope[b,i,h] . k_rope_j)) c_j with q_c = W_UK[h]^T q_nope[b,i,h] -- the
// scaled_dot_product_attention(is_causal=True) call of the MultiHeadLatentAttention
// listing on the qqstock DeepSeek MLA article, whose keys [W_UK c, k_rope] and
// values W_UV c are rebuilt from the latent: folding W_UK into the query and
// applying W_UV after the weighted sum (sections 2 and 4 of the article) gives
// the same numbers, and k_rope is shared by all heads (section 3).  With a cached
// prefix of P positions new token i sits at position P + i (bottom-right causal
// cut), as in the GQA prefill above.
//
// How (not from the pages): the GQA prefill's tiles and online softmax with one
// KV stream shared by all H heads.  The latent tile c [64 keys x 128] is the K
// operand of the first 128 score dimensions and also the V operand of PV, so one
// copy serves both; a second tile holds k_rope [64 x dR] (LDS rows of 64
// elements, XOR-swizzled as the head_dim-64 tiles) for the last dR dimensions.
// Prologue: each wave's 32 absorbed query rows q_c^T = W_UK[h]^T q_nope^T on
// MFMA, with W_UK[h] staged transposed in LDS; the accumulator layout is moved
// into the B-operand layout by exchanging half of each lane's values with lane ^ 32.
// Epilogue: out^T = W_UV[h] O^T on MFMA from the normalised O^T, moved the same
// way.  q_c and o_lat enter those MFMAs as bf16, like P.

// A 32x32 MFMA accumulator block X^T[k][row] (lane holds k = 8q + 4h2 + e for
// i = 4q + e, row = lane % 32), times f, as the B operands of two 16-wide
// k-steps: op[s] holds X[row][16s + 8h2 + 0..7] in bf16.  For k-step s the lane
// half h2 = 0 needs its own k = 16s + 0..3 and the other half's 16s + 4..7, the
// half h2 = 1 the first half's 16s + 8..11 and its own 16s + 12..15: each lane
// sends one of its two groups to lane ^ 32 (ds_bpermute, which the compiler
// orders after the MFMA that wrote the accumulator).
__device__ __forceinline__ void acc_to_operands(const f32x16& acc, float f, bf16x8* op, int h2) {
#pragma unroll
  for (int sblk = 0; sblk < 2; ++sblk) {
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = acc[8 * sblk + e] * f;
      hi[e] = acc[8 * sblk + 4 + e] * f;
      const float got = __shfl_xor(h2 ? lo[e] : hi[e], 32);
      if (h2) lo[e] = got;
      else hi[e] = got;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      op[sblk][e] = (__bf16)lo[e];
      op[sblk][4 + e] = (__bf16)hi[e];
    }
  }
}

// S^T of one tile: 128 latent dimensions from the c tile, DR rope dimensions
// from the rope tile (rows of 64 elements).
template <int DR>
__device__ __forceinline__ void qk_tile_mla(f32x16 (&s)[2], const u16* cc, const u16* rc, const bf16x8 (&qop)[8],
                                            const bf16x8 (&qrop)[DR / 16], int off, int off_r, const f32x16& init) {
  s[0] = init;
  s[1] = init;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u16* kr = cc + 32 * j * 128 + (off ^ (16 * c));
      s[j] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr)), qop[c], s[j]);
    }
#pragma unroll
  for (int c = 0; c < DR / 16; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u16* kr = rc + 32 * j * 64 + (off_r ^ (16 * c));
      s[j] = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr)), qrop[c], s[j]);
    }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int u = 0; u < 2 * (8 + DR / 16); ++u) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <int DR>
__device__ __forceinline__ void tile_step_mla(RowState<128>& st, const u16* cc, const u16* rc, u16* cn, u16* rn,
                                              const bf16x8 (&qop)[8], const bf16x8 (&qrop)[DR / 16], int kt,
                                              int n_kt, int last_kt, const u16* cp, const u16* rp, int kv_len,
                                              const TileCopy<128>& cpc, const TileCopy<64>& cpr,
                                              const LdsOffsets& off, int off_r, const Lane& w) {
  if (kt + 1 < n_kt) {  // (cn, rn) were released by the last barrier
    cpc.issue(cn, TileCopy<128>::rsrc(cp, kt + 1, n_kt, kv_len, 256));
    cpr.issue(rn, TileCopy<64>::rsrc(rp, kt + 1, n_kt, kv_len, 2 * DR, 2 * DR));
  }
  if (kt <= last_kt) {
    f32x16 sc[2];
    qk_tile_mla<DR>(sc, cc, rc, qop, qrop, off.k, off_r, st.negm);
    bf16x8 pop[4];
    softmax_tile<128>(st, sc, pop, kt * kBN, w.pos0, w.my_pos, kt == 0, w);
    pv_tile<128>(st.o, cc, pop, off.v_lo, off.v_hi);  // V = the latent tile
  }
  wait_vmem();
  __syncthreads();
}

// Stores out^T blocks (lane holds out^T[32eb + 8q + 4h2 + e][row ln]) of one row,
// or zeros when !valid.
template <int DV>
__device__ __forceinline__ void store_mla_row(void* out, size_t orow, int out_bf16, const f32x16 (&o)[DV / 32],
                                              bool valid, int h2) {
  if (out_bf16) {
    u16* op = static_cast<u16*>(out) + orow * DV;
#pragma unroll
    for (int eb = 0; eb < DV / 32; ++eb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = __builtin_bit_cast(u16, (__bf16)(valid ? o[eb][4 * q4 + e] : 0.f));
        *reinterpret_cast<u16x4*>(op + 32 * eb + 8 * q4 + 4 * h2) = o4;
      }
  } else {
    float* op = static_cast<float*>(out) + orow * DV;
#pragma unroll
    for (int eb = 0; eb < DV / 32; ++eb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) f = make_float4(o[eb][4 * q4], o[eb][4 * q4 + 1], o[eb][4 * q4 + 2], o[eb][4 * q4 + 3]);
        *reinterpret_cast<float4*>(op + 32 * eb + 8 * q4 + 4 * h2) = f;
      }
  }
}

template <int DN, int DR, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mla(MlaPrefillArgs a) {
  static_assert(DN % 16 == 0 && DN <= 128 && DR % 16 == 0 && DR <= 64 && DV % 32 == 0 && DV <= 128, "widths");
  constexpr int R = 128;         // kv_lora_rank
  constexpr int WP = DN + 8;     // row pitch of W_UK^T in LDS: 16-byte reads of 16 rows hit distinct banks
  __shared__ __attribute__((aligned(1024))) u16 c0[kBN * R];
  __shared__ __attribute__((aligned(1024))) u16 c1[kBN * R];
  __shared__ __attribute__((aligned(1024))) u16 r0[kBN * 64];
  __shared__ __attribute__((aligned(1024))) u16 r1[kBN * 64];
  __shared__ __attribute__((aligned(16))) u16 wukT[R * WP];

  const Tile tl = map_tile(a.S, a.B, a.H, 1, a.H, blockIdx.x);
  const int h = tl.h, b = tl.b;
  const int q0 = tl.qt * kBM;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.start_pos ? min(max(a.start_pos[b], 0), a.T_kv) : 0;
  const int n_q = min(a.q_lens ? min(max(a.q_lens[b], 0), a.S) : a.S, a.T_kv - P);
  Lane w;
  w.lane = tid & 63;
  w.ln = w.lane & 31;
  w.h2 = w.lane >> 5;
  w.row0 = q0 + wave * 32;
  w.my_row = w.row0 + w.ln;
  w.pos0 = P + w.row0;
  w.my_pos = P + w.my_row;
  w.c = a.scale_log2e;
  const size_t orow = ((size_t)b * a.S + w.my_row) * a.H + h;
  if (q0 >= n_q) {  // no new token in this q-tile: zero rows, nothing to read
    const f32x16 none[DV / 32] = {};
    if (w.my_row < a.S) store_mla_row<DV>(a.out, orow, a.out_bf16, none, false, w.h2);
    return;
  }
  const u16* cp = static_cast<const u16*>(a.c_kv) + (size_t)b * a.T_kv * R;
  const u16* rp = static_cast<const u16*>(a.k_rope) + (size_t)b * a.T_kv * DR;
  const int kv_len = P + n_q;
  const int kv_end = min(kv_len, P + q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;
  const int last_kt = min(n_kt - 1, (w.pos0 + 31) / kBN);

  const TileCopy<128> cpc(wave, w.lane, 2 * R);
  const TileCopy<64> cpr(wave, w.lane, 2 * DR);
  cpc.issue(c0, TileCopy<128>::rsrc(cp, 0, n_kt, kv_len, 2 * R));
  cpr.issue(r0, TileCopy<64>::rsrc(rp, 0, n_kt, kv_len, 2 * DR, 2 * DR));

  // W_UK[h] [DN][R] -> LDS transposed [R][WP]: thread-consecutive rows i, so the
  // 2-byte writes of a wave are consecutive
  const u16* wk = static_cast<const u16*>(a.w_uk) + (size_t)h * DN * R;
#pragma unroll
  for (int k = 0; k < DN / 16; ++k) {
    const int id = tid + 256 * k;
    const int i = id % DN, jc = id / DN;
    const u16x8 v = *reinterpret_cast<const u16x8*>(wk + (size_t)i * R + 8 * jc);
#pragma unroll
    for (int e = 0; e < 8; ++e) wukT[(8 * jc + e) * WP + i] = v[e];
  }
  // q_nope^T and q_rope^T B operands: lane holds row ln's dims 16c + 8h2 .. +8
  const int qrow = min(w.my_row, a.S - 1);
  const u16* qn = static_cast<const u16*>(a.q_nope) + (((size_t)b * a.S + qrow) * a.H + h) * DN + 8 * w.h2;
  const u16* qr = static_cast<const u16*>(a.q_rope) + (((size_t)b * a.S + qrow) * a.H + h) * DR + 8 * w.h2;
  bf16x8 qnop[DN / 16];
#pragma unroll
  for (int c = 0; c < DN / 16; ++c) qnop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qn + 16 * c));
  bf16x8 qrop[DR / 16];
#pragma unroll
  for (int c = 0; c < DR / 16; ++c) qrop[c] = scaled_operand(*reinterpret_cast<const u16x8*>(qr + 16 * c), w.c);
  __syncthreads();  // W_UK^T staged

  // q_c^T[j][row] = sum_i W_UK^T[j][i] q_nope^T[i][row], 32 j at a time, times scale * log2 e
  bf16x8 qop[8];
#pragma unroll
  for (int jb = 0; jb < R / 32; ++jb) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const u16* ar = wukT + (32 * jb + w.ln) * WP + 8 * w.h2;
#pragma unroll
    for (int c = 0; c < DN / 16; ++c)
      acc = mfma_32x32x16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(ar + 16 * c)), qnop[c], acc);
    acc_to_operands(acc, w.c, &qop[2 * jb], w.h2);
  }

  const LdsOffsets off = lds_offsets<128>(w);
  const int off_r = lds_offsets<64>(w).k;
  RowState<128> st;
  init_rows(st);

  wait_vmem();
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    tile_step_mla<DR>(st, c0, r0, c1, r1, qop, qrop, kt, n_kt, last_kt, cp, rp, kv_len, cpc, cpr, off, off_r, w);
    if (kt + 1 < n_kt)
      tile_step_mla<DR>(st, c1, r1, c0, r0, qop, qrop, kt + 1, n_kt, last_kt, cp, rp, kv_len, cpc, cpr, off, off_r,
                        w);
  }

  // o_lat = O / l as the B operand, then out^T = W_UV[h] o_lat^T, 32 output dims at a time
  const float inv = 1.f / sum_xor32(st.lsum);
  bf16x8 oop[8];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc_to_operands(st.o[d], inv, &oop[2 * d], w.h2);
  const u16* wv = static_cast<const u16*>(a.w_uv) + ((size_t)h * DV + w.ln) * R + 8 * w.h2;
  f32x16 ov[DV / 32];
#pragma unroll
  for (int eb = 0; eb < DV / 32; ++eb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) ov[eb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      ov[eb] = mfma_32x32x16(
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(wv + (size_t)32 * eb * R + 16 * c)), oop[c],
          ov[eb]);
  }
  if (w.my_row < a.S) store_mla_row<DV>(a.out, orow, a.out_bf16, ov, w.my_row < n_q, w.h2);
}

// Explicit instantiations: without them the host stubs of only some of the
// kernel templates launched below were emitted.
template __global__ void prefill_causal<128, 0>(PrefillArgs);
template __global__ void prefill_causal<96, 0>(PrefillArgs);
template __global__ void prefill_causal<64, 0>(PrefillArgs);
template __global__ void prefill_causal<128, 1>(PrefillArgs);
template __global__ void prefill_causal<96, 1>(PrefillArgs);
template __global__ void prefill_causal<64, 1>(PrefillArgs);
template __global__ void prefill_causal<128, 2>(PrefillArgs);
template __global__ void prefill_causal<96, 2>(PrefillArgs);
template __global__ void prefill_causal<64, 2>(PrefillArgs);
template __global__ void prefill_causal<128, 3>(PrefillArgs);
template __global__ void prefill_causal<96, 3>(PrefillArgs);
template __global__ void prefill_causal<64, 3>(PrefillArgs);
template __global__ void prefill_mla<96, 48, 96>(MlaPrefillArgs);

}  // namespace

bool prefill_supported(int D) { return D == 64 || D == 96 || D == 128; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (!prefill_supported(a.D)) return hipErrorInvalidValue;
  const long long wgs = (long long)((a.S + kBM - 1) / kBM) * a.Hq * a.B;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  const int mode = a.block_table ? 3 : a.k_new ? 2 : a.start_pos ? 1 : 0;
  if ((mode == 2 || mode == 3) && !a.start_pos) return hipErrorInvalidValue;
  if (mode == 3 && (a.k_new || a.page_size <= 0 || a.page_size % kBN != 0 || a.n_pages <= 0)) return hipErrorInvalidValue;
#define ATTN_PREFILL_LAUNCH(DD)                                                                                  \
  do {                                                                                                             \
    if (mode == 3) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_causal<DD, 3>), grid, dim3(256), 0, st, a);         \
    else if (mode == 2) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_causal<DD, 2>), grid, dim3(256), 0, st, a);    \
    else if (mode == 1) hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_causal<DD, 1>), grid, dim3(256), 0, st, a);    \
    else hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_causal<DD, 0>), grid, dim3(256), 0, st, a);                   \
  } while (0)
  if (a.D == 128) ATTN_PREFILL_LAUNCH(128);
  else if (a.D == 96) ATTN_PREFILL_LAUNCH(96);
  else ATTN_PREFILL_LAUNCH(64);
#undef ATTN_PREFILL_LAUNCH
  return hipGetLastError();
}

bool mla_prefill_supported(int dn, int dR, int dv, int r) { return r == 128 && dn == 96 && dR == 48 && dv == 96; }

hipError_t launch_mla_prefill(const MlaPrefillArgs& a, hipStream_t st) {
  if (!mla_prefill_supported(a.dn, a.dR, a.dv, a.r)) return hipErrorInvalidValue;
  const long long wgs = (long long)((a.S + kBM - 1) / kBM) * a.H * a.B;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  hipLaunchKernelGGL(HIP_KERNEL_NAME(prefill_mla<96, 48, 96>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
