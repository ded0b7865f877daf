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
//  * One workgroup per (chunk of `split` cached positions, KV head, sequence).
//    It streams the chunk's K and V rows from HBM exactly once and applies them
//    to all n_rep query heads of the group -- the repeat_kv copies are never
//    made.  Four waves take interleaved 32-token tiles of the chunk.
//  * bf16 path: scores are S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the
//    tile's tokens as M and (padded) query heads as N, so the K tile is the A
//    operand and is loaded straight from HBM with one 16-byte load per lane per
//    32 dims.  P stays in the accumulator layout and becomes the B operand of
//    O^T += V^T P^T after a token permutation that both operands share.  V is
//    staged row-major in LDS (one private region per wave, 16-byte writes) and
//    read back transposed with ds_read_b64_tr_b16.
//  * fp32 path (VALU): 16 lanes cover one token's row (head_dim/16 elements
//    each); dot products are reduced inside the 16-lane DPP row.
//  * Online softmax in base 2 (scale * log2 e folded in, v_exp_f32), running
//    max / sum per head; each workgroup writes its chunk's normalised partial
//    output and log2-sum-exp, and a second kernel merges the chunks.
//  * Positions at or beyond L_b are never read: the last tile clamps its row
//    index to L_b - 1 and masks those scores to -inf.
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

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ int clamp_len(int L, int T_max) { return L < 0 ? 0 : (L > T_max ? T_max : L); }

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA.  HB blocks of 16 query heads (n_rep <= 16 * HB).
template <int D, int HB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HB == 1 ? 4 : 1))) void gqa_decode_bf16_partial(GqaDecodeArgs a) {
  static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
  constexpr int KC = D / 32;           // 32-wide dim chunks (QK contraction)
  constexpr int DW = D / 16;           // 16-wide dim blocks (PV output rows)
  constexpr int VP = D + 16;           // V tile row pitch in elements ([token][dim], padded)
  constexpr int kVtElems = kDecodeWaves * kDecodeTileTokens * VP;
  // merge scratch (floats): m and l per wave and head, then [HB*16][D] outputs
  static_assert(2 * kDecodeWaves * HB * 16 * 4 + HB * 16 * D * 4 <= kVtElems * 2, "merge scratch must fit");
  __shared__ __attribute__((aligned(16))) u16 smem[kVtElems];

  const int g = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int c0 = s * a.split;
  if (c0 >= L) return;  // uniform: the whole chunk is past the cache length
  const int c1 = min(c0 + a.split, L);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, grp = lane >> 4;
  const int n_rep = a.n_rep;

  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)b * a.Hq + (size_t)g * n_rep) * D;
  const size_t tok_stride = (size_t)a.Hkv * D;
  const u16* kp = static_cast<const u16*>(a.k) + ((size_t)b * a.T_max * a.Hkv + g) * D;
  const u16* vp = static_cast<const u16*>(a.v) + ((size_t)b * a.T_max * a.Hkv + g) * D;

  // Q^T as the B operand: lane holds Q[head = 16hb + row][dims 32c + 8grp .. +8]
  bf16x8 qop[HB][KC];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = hb * 16 + row;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (head < n_rep) {
        qop[hb][c] = load_bf16x8(qp + (size_t)head * D + 32 * c + 8 * grp);
      } else {
        qop[hb][c] = __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
      }
    }
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
  u16* vt = smem + wave * kDecodeTileTokens * VP;

  // K as the A operand (row = token), V in the same layout.  Row indices are
  // clamped to L - 1: rows past the chunk end re-read a valid row and their
  // scores are masked.
  auto load_tile = [&](bf16x8 (&kr)[2][KC], bf16x8 (&vr)[2][KC], int t0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = min(t0 + 16 * u + row, L - 1);
      const u16* krow = kp + (size_t)tok * tok_stride + 8 * grp;
#pragma unroll
      for (int c = 0; c < KC; ++c) kr[u][c] = load_bf16x8(krow + 32 * c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = min(t0 + 16 * u + row, L - 1);
      const u16* vrow = vp + (size_t)tok * tok_stride + 8 * grp;
#pragma unroll
      for (int c = 0; c < KC; ++c) vr[u][c] = load_bf16x8(vrow + 32 * c);
    }
  };
  auto process_tile = [&](const bf16x8 (&kr)[2][KC], const bf16x8 (&vr)[2][KC], int t0) {
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
    // Online softmax per head; P^T as the B operand of the PV product.
    bf16x8 pop[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float mt = kNegInf;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[hb][u][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
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
    // V tile into this wave's LDS region, row-major [token][dim]
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        *reinterpret_cast<u16x8*>(vt + (16 * u + row) * VP + 32 * c + 8 * grp) = __builtin_bit_cast(u16x8, vr[u][c]);
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
    }
    wave_lds_sync();
  };

  // Tiles of this wave: t0 = c0 + 32*wave + 128*i, one at a time.  (Keeping a
  // second tile in flight was measured slower: it halves the waves per SIMD.)
  for (int t0 = c0 + wave * kDecodeTileTokens; t0 < c1; t0 += kDecodeWaves * kDecodeTileTokens) {
    bf16x8 kA[2][KC], vA[2][KC];
    load_tile(kA, vA, t0);
    process_tile(kA, vA, t0);
  }

  // ---- merge the four waves of the workgroup ----
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    lsum[hb] += __shfl_xor(lsum[hb], 16);
    lsum[hb] += __shfl_xor(lsum[hb], 32);
  }
  __syncthreads();  // every wave is done with its V^T region
  float* mw = reinterpret_cast<float*>(smem);   // [waves][HB*16]
  float* lw = mw + kDecodeWaves * HB * 16;      // [waves][HB*16]
  float* ob = lw + kDecodeWaves * HB * 16;      // [HB*16][D]
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
  }
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int dw = 0; dw < DW; ++dw)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* dst = ob + (hb * 16 + row) * D + 16 * dw + 4 * grp + i;
            *dst = (w == 0 ? 0.f : *dst) + o[hb][dw][i];
          }
    }
    __syncthreads();
  }
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * n_rep;
  for (int e = threadIdx.x; e < n_rep * D; e += 256) {
    const int hd = e / D, d = e - hd * D;
    a.o_part[((row0 + hd) * a.n_splits + s) * D + d] = ob[hd * D + d];
  }
  for (int hd = threadIdx.x; hd < n_rep; hd += 256) {
    float M = kNegInf;
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w * HB * 16 + hd]);
    float Lt = 0.f;
    for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w * HB * 16 + hd], M) * lw[w * HB * 16 + hd];
    a.lse[(row0 + hd) * a.n_splits + s] = M + __log2f(Lt);
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU.  16 rows of 16 lanes; row r takes positions c0 + r + 16k.
template <int D, int NR>
__global__ __launch_bounds__(256) void gqa_decode_f32_partial(GqaDecodeArgs a) {
  static_assert(D % 16 == 0, "head_dim must be a multiple of 16");
  constexpr int E = D / 16;
  __shared__ float mw[kDecodeWaves][NR], lw[kDecodeWaves][NR];
  __shared__ float ob[NR][D];

  const int g = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int c0 = s * a.split;
  if (c0 >= L) return;
  const int c1 = min(c0 + a.split, L);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rid = threadIdx.x >> 4, col = threadIdx.x & 15;
  const int n_rep = a.n_rep;

  const float* qp = static_cast<const float*>(a.q) + ((size_t)b * a.Hq + (size_t)g * n_rep) * D + col * E;
  const size_t tok_stride = (size_t)a.Hkv * D;
  const float* kp = static_cast<const float*>(a.k) + ((size_t)b * a.T_max * a.Hkv + g) * D + col * E;
  const float* vp = static_cast<const float*>(a.v) + ((size_t)b * a.T_max * a.Hkv + g) * D + col * E;

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
  for (int t = c0 + rid; t < c1; t += 16) {
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
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (wave == w && lane < 16) {
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        if (h < n_rep) {
          const float f = rescale(m[h], Mh[h]) / Lh[h];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float* dst = &ob[h][col * E + e];
            *dst = (w == 0 ? 0.f : *dst) + acc[h][e] * f;
          }
        }
      }
    }
    __syncthreads();
  }
  const size_t row0 = (size_t)b * a.Hq + (size_t)g * n_rep;
  for (int e = threadIdx.x; e < n_rep * D; e += 256) {
    const int hd = e / D, d = e - hd * D;
    a.o_part[((row0 + hd) * a.n_splits + s) * D + d] = ob[hd][d];
  }
  if (threadIdx.x < n_rep) {
#pragma unroll
    for (int h = 0; h < NR; ++h)
      if (h == (int)threadIdx.x) a.lse[(row0 + h) * a.n_splits + s] = Mh[h] + __log2f(Lh[h]);
  }
}

// ---------------------------------------------------------------------------
// Merge the chunks of every (sequence, query head) by their log2-sum-exp.
// One wave per row.  Lane l covers dims 4*(l % (D/4)) .. +4 of the chunks
// s = l / (D/4) + k * (64 / (D/4)), so all of a row's partial loads are issued
// together; the lane groups are then summed with cross-lane shuffles.
template <int D>
__global__ __launch_bounds__(256) void gqa_decode_merge(GqaDecodeArgs a) {
  static_assert(D == 64 || D == 128 || D == 96, "head_dim");
  constexpr int LPR = D / 4;                       // lanes per chunk row (16, 24 or 32)
  constexpr int G = 64 / LPR;                      // chunk rows per pass (4, 2 or 2)
  const int rowid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rowid >= a.B * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int b = rowid / a.Hq;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int n = (L + a.split - 1) / a.split;
  const float* lse = a.lse + (size_t)rowid * a.n_splits;
  const float* op = a.o_part + (size_t)rowid * a.n_splits * D;
  float M = kNegInf;
  for (int s = lane; s < n; s += 64) M = fmaxf(M, lse[s]);
  M = wave_max(M);
  const int gi = lane / LPR, li = lane - gi * LPR;
  const bool active = gi < G;  // D = 96: lanes 48..63 idle
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (active) {
    for (int s = gi; s < n; s += G) {
      const float w = exp2_fast(lse[s] - M);
      const float4 v = *reinterpret_cast<const float4*>(op + (size_t)s * D + 4 * li);
      wsum += w;
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
  }
  // add the G chunk groups into group 0 (lanes LPR apart)
#pragma unroll
  for (int k = 1; k < G; k <<= 1) {
    const int src = (lane + k * LPR) & 63;
    wsum += __shfl(wsum, src);
    acc.x += __shfl(acc.x, src);
    acc.y += __shfl(acc.y, src);
    acc.z += __shfl(acc.z, src);
    acc.w += __shfl(acc.w, src);
  }
  if (gi != 0) return;
  const float inv = n > 0 ? 1.f / wsum : 0.f;
  if (a.out_bf16) {
    __bf16* out = static_cast<__bf16*>(a.out) + (size_t)rowid * D + 4 * li;
    out[0] = (__bf16)(acc.x * inv);
    out[1] = (__bf16)(acc.y * inv);
    out[2] = (__bf16)(acc.z * inv);
    out[3] = (__bf16)(acc.w * inv);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)rowid * D + 4 * li) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

template <int D>
hipError_t launch_bf16(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int hb = (a.n_rep + 15) / 16;
  if (hb == 1) hipLaunchKernelGGL((gqa_decode_bf16_partial<D, 1>), grid, dim3(256), 0, st, a);
  else if (hb == 2) hipLaunchKernelGGL((gqa_decode_bf16_partial<D, 2>), grid, dim3(256), 0, st, a);
  else if (hb <= 4) hipLaunchKernelGGL((gqa_decode_bf16_partial<D, 4>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const GqaDecodeArgs& a, dim3 grid, hipStream_t st) {
  const int n = a.n_rep;
  if (n == 1) hipLaunchKernelGGL((gqa_decode_f32_partial<D, 1>), grid, dim3(256), 0, st, a);
  else if (n == 2) hipLaunchKernelGGL((gqa_decode_f32_partial<D, 2>), grid, dim3(256), 0, st, a);
  else if (n <= 4) hipLaunchKernelGGL((gqa_decode_f32_partial<D, 4>), grid, dim3(256), 0, st, a);
  else if (n <= 8) hipLaunchKernelGGL((gqa_decode_f32_partial<D, 8>), grid, dim3(256), 0, st, a);
  else if (n <= 16) hipLaunchKernelGGL((gqa_decode_f32_partial<D, 16>), grid, dim3(256), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool gqa_decode_supported(int D, int n_rep, int in_bf16) {
  if (D != 64 && D != 96 && D != 128) return false;
  if (n_rep < 1) return false;
  return in_bf16 ? n_rep <= 64 : n_rep <= 16;
}

hipError_t launch_gqa_decode(const GqaDecodeArgs& a, hipStream_t st) {
  if (!gqa_decode_supported(a.D, a.n_rep, a.in_bf16)) return hipErrorInvalidValue;
  // KV heads vary fastest so the workgroups of one chunk's heads (interleaved in
  // memory, one row of Hkv*D per token) are dispatched together.
  const dim3 grid(a.Hkv, a.n_splits, a.B);
  hipError_t e;
  if (a.in_bf16) {
    e = a.D == 64 ? launch_bf16<64>(a, grid, st) : a.D == 96 ? launch_bf16<96>(a, grid, st) : launch_bf16<128>(a, grid, st);
  } else {
    e = a.D == 64 ? launch_f32<64>(a, grid, st) : a.D == 96 ? launch_f32<96>(a, grid, st) : launch_f32<128>(a, grid, st);
  }
  if (e != hipSuccess) return e;
  const dim3 mgrid((a.B * a.Hq + 3) / 4);
  if (a.D == 64) hipLaunchKernelGGL(gqa_decode_merge<64>, mgrid, dim3(256), 0, st, a);
  else if (a.D == 96) hipLaunchKernelGGL(gqa_decode_merge<96>, mgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(gqa_decode_merge<128>, mgrid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
