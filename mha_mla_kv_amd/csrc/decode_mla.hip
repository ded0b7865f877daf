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
// Kernels (not from the pages; designed for CDNA4):
//  1. mla_absorb: q_lat per (sequence, head) in fp32, stored as a bf16 hi/lo
//     pair so the MFMA score keeps ~16 mantissa bits of q_lat.
//  2. mla_decode_partial: one workgroup per (chunk, sequence) serves all heads
//     (padded to 16), so every [c_kv , k_rope] row is read from HBM once per
//     sequence.  S^T = [c k_rope] q_lat^T on v_mfma_f32_16x16x32_bf16 (plus one
//     16x16x16 step when rope_dim is an odd multiple of 16); the latent tile is
//     reused as V (values share it with the un-rotated key): it is staged
//     row-major in LDS and read back transposed with ds_read_b64_tr_b16.  Online base-2 softmax as in the GQA decode.
//  3. mla_merge_wuv: log2-sum-exp merge of the chunks into o_lat, then
//     out = W_UV[h] o_lat in fp32.
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
__device__ __forceinline__ float rescale(float m, float M) { return m == kNegInf ? 0.f : exp2_fast(m - M); }
__device__ __forceinline__ int clamp_len(int L, int T_max) { return L < 0 ? 0 : (L > T_max ? T_max : L); }

__device__ __forceinline__ bf16x8 load_bf16x8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}
__device__ __forceinline__ s16x4 load_s16x4(const u16* p) {
  return __builtin_bit_cast(s16x4, *reinterpret_cast<const u16x4*>(p));
}
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// ds_read_b64_tr_b16: lane i of a 16-lane group points at row T0 + i/4,
// columns 4(i%4).. of a row-major [token][dim] tile; lane j receives tokens
// T0..T0+3 of column j.
__device__ __forceinline__ u16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ float bf16_to_f32(u16 x) { return __builtin_bit_cast(float, (unsigned)x << 16); }

// ---------------------------------------------------------------------------
// q_lat[b][hl][h][0:r]     = hi / lo bf16 parts of W_UK[h]^T q_nope[b,h]
// q_lat[b][0][h][r:r+dR]   = q_rope[b,h];  q_lat[b][1][h][r:r+dR] = 0
// heads h in [H, 16) are zero.
// Grid (16, B), block 256: one workgroup per (padded head, sequence); thread j
// owns latent column j (coalesced reads of W_UK rows), q_nope comes from LDS.
__global__ __launch_bounds__(256) void mla_absorb(MlaDecodeArgs a) {
  __shared__ float qs[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const int RW = a.r + a.dR;
  u16* ql_hi = static_cast<u16*>(a.q_lat) + ((size_t)b * 2 * kHeadsPad + h) * RW;
  u16* ql_lo = ql_hi + (size_t)kHeadsPad * RW;
  if (h >= a.H) {
    for (int j = threadIdx.x; j < RW; j += 256) {
      ql_hi[j] = 0;
      ql_lo[j] = 0;
    }
    return;
  }
  const u16* qn = static_cast<const u16*>(a.q_nope) + ((size_t)b * a.H + h) * a.dn;
  for (int i = threadIdx.x; i < a.dn; i += 256) qs[i] = bf16_to_f32(qn[i]);
  __syncthreads();
  const u16* wk = static_cast<const u16*>(a.w_uk) + (size_t)h * a.dn * a.r;
  for (int j = threadIdx.x; j < a.r; j += 256) {
    float acc = 0.f;
    for (int i = 0; i < a.dn; ++i) acc = fmaf(bf16_to_f32(wk[(size_t)i * a.r + j]), qs[i], acc);
    const __bf16 h16 = (__bf16)acc;
    ql_hi[j] = __builtin_bit_cast(u16, h16);
    ql_lo[j] = __builtin_bit_cast(u16, (__bf16)(acc - (float)h16));
  }
  const u16* qr = static_cast<const u16*>(a.q_rope) + ((size_t)b * a.H + h) * a.dR;
  for (int e = threadIdx.x; e < a.dR; e += 256) {
    ql_hi[a.r + e] = qr[e];
    ql_lo[a.r + e] = 0;
  }
}

// ---------------------------------------------------------------------------
template <int R, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R <= 128 ? 4 : 1))) void mla_decode_partial(MlaDecodeArgs a) {
  static_assert(R % 32 == 0 && DR % 16 == 0 && DR >= 16 && DR <= 64, "unsupported latent/rope widths");
  constexpr int KC = R / 32;         // 32-wide latent chunks
  constexpr int RC = DR / 32;        // 32-wide rope chunks
  constexpr bool R16 = (DR % 32) != 0;  // one trailing 16-wide rope chunk
  constexpr int RW = R + DR;
  constexpr int DW = R / 16;         // 16-wide latent blocks of the PV output
  constexpr int VP = R + 16;  // latent tile row pitch ([token][dim], padded)
  constexpr int kVtElems = kDecodeWaves * kDecodeTileTokens * VP;
  static_assert(2 * kDecodeWaves * kHeadsPad * 4 + kHeadsPad * R * 4 <= kVtElems * 2, "merge scratch must fit");
  __shared__ __attribute__((aligned(16))) u16 smem[kVtElems];

  const int s = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int c0 = s * a.split;
  if (c0 >= L) return;
  const int c1 = min(c0 + a.split, L);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane & 15, grp = lane >> 4;

  const u16* ql = static_cast<const u16*>(a.q_lat) + (size_t)b * 2 * kHeadsPad * RW;
  bf16x8 qhi[KC], qlo[KC], qr32[RC > 0 ? RC : 1];
  s16x4 qr16 = {0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qhi[c] = load_bf16x8(ql + (size_t)row * RW + 32 * c + 8 * grp);
    qlo[c] = load_bf16x8(ql + (size_t)(kHeadsPad + row) * RW + 32 * c + 8 * grp);
  }
#pragma unroll
  for (int c = 0; c < RC; ++c) qr32[c] = load_bf16x8(ql + (size_t)row * RW + R + 32 * c + 8 * grp);
  if constexpr (R16) qr16 = load_s16x4(ql + (size_t)row * RW + R + 32 * RC + 4 * grp);

  const u16* cp = static_cast<const u16*>(a.c_kv) + (size_t)b * a.T_max * R;
  const u16* rp = static_cast<const u16*>(a.k_rope) + (size_t)b * a.T_max * DR;

  float m = kNegInf, lsum = 0.f;
  f32x4 o[DW];
#pragma unroll
  for (int w = 0; w < DW; ++w) o[w] = f32x4{0.f, 0.f, 0.f, 0.f};
  u16* vt = smem + wave * kDecodeTileTokens * VP;

  constexpr int RCA = RC > 0 ? RC : 1;
  // Latent rows as the A operand (row = token); indices clamped to L - 1 (rows
  // past the chunk end re-read a valid row and are masked).
  auto load_tile = [&](bf16x8 (&cr)[2][KC], bf16x8 (&kr32)[2][RCA], s16x4 (&kr16)[2], int t0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = min(t0 + 16 * u + row, L - 1);
      const u16* crow = cp + (size_t)tok * R + 8 * grp;
      const u16* rrow = rp + (size_t)tok * DR;
#pragma unroll
      for (int c = 0; c < KC; ++c) cr[u][c] = load_bf16x8(crow + 32 * c);
#pragma unroll
      for (int c = 0; c < RC; ++c) kr32[u][c] = load_bf16x8(rrow + 32 * c + 8 * grp);
      if constexpr (R16) kr16[u] = load_s16x4(rrow + 32 * RC + 4 * grp);
    }
  };
  auto process_tile = [&](const bf16x8 (&cr)[2][KC], const bf16x8 (&kr32)[2][RCA], const s16x4 (&kr16)[2],
                          int t0) {
    float sc[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        acc = mfma_16x16x32(cr[u][c], qhi[c], acc);
        acc = mfma_16x16x32(cr[u][c], qlo[c], acc);
      }
#pragma unroll
      for (int c = 0; c < RC; ++c) acc = mfma_16x16x32(kr32[u][c], qr32[c], acc);
      if constexpr (R16) acc = mfma_16x16x16(kr16[u], qr16, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * u + 4 * grp + i;
        sc[u][i] = tok < c1 ? acc[i] * a.scale_log2e : kNegInf;
      }
    }
    float mt = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sc[u][i]);
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    const float mn = fmaxf(m, mt);
    const float alpha = exp2_fast(m - mn);
    m = mn;
    bf16x8 pop;
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_fast(sc[u][i] - mn);
        ps += p;
        pop[4 * u + i] = (__bf16)p;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int w = 0; w < DW; ++w) o[w] *= alpha;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        *reinterpret_cast<u16x8*>(vt + (16 * u + row) * VP + 32 * c + 8 * grp) = __builtin_bit_cast(u16x8, cr[u][c]);
    wave_lds_sync();
    const u16* trbase = vt + (4 * grp + (row >> 2)) * VP + 4 * (row & 3);
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      const u16x4 lo = lds_read_tr16(trbase + 16 * w);
      const u16x4 hi = lds_read_tr16(trbase + 16 * VP + 16 * w);
      const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[w] = mfma_16x16x32(__builtin_bit_cast(bf16x8, av), pop, o[w]);
    }
    wave_lds_sync();
  };

  for (int t0 = c0 + wave * kDecodeTileTokens; t0 < c1; t0 += kDecodeWaves * kDecodeTileTokens) {
    bf16x8 cA[2][KC], rA[2][RCA];
    s16x4 sA[2];
    load_tile(cA, rA, sA, t0);
    process_tile(cA, rA, sA, t0);
  }

  lsum = sum_xor16(lsum);
  lsum = sum_xor32(lsum);
  __syncthreads();
  float* mw = reinterpret_cast<float*>(smem);  // [waves][16]
  float* lw = mw + kDecodeWaves * kHeadsPad;   // [waves][16]
  float* ob = lw + kDecodeWaves * kHeadsPad;   // [16][R]
  if (grp == 0) {
    mw[wave * kHeadsPad + row] = m;
    lw[wave * kHeadsPad + row] = lsum;
  }
  __syncthreads();
  {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w * kHeadsPad + row]);
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w * kHeadsPad + row], M) * lw[w * kHeadsPad + row];
    const float f = rescale(m, M) / Lt;
#pragma unroll
    for (int w = 0; w < DW; ++w) o[w] *= f;
  }
  for (int w = 0; w < kDecodeWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int dw = 0; dw < DW; ++dw)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = ob + row * R + 16 * dw + 4 * grp + i;
          *dst = (w == 0 ? 0.f : *dst) + o[dw][i];
        }
    }
    __syncthreads();
  }
  const size_t row0 = (size_t)b * a.H;
  for (int e = threadIdx.x; e < a.H * R; e += 256) {
    const int hd = e / R, d = e - hd * R;
    a.o_part[((row0 + hd) * a.n_splits + s) * R + d] = ob[hd * R + d];
  }
  for (int hd = threadIdx.x; hd < a.H; hd += 256) {
    float M = kNegInf;
    for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, mw[w * kHeadsPad + hd]);
    float Lt = 0.f;
    for (int w = 0; w < kDecodeWaves; ++w) Lt += rescale(mw[w * kHeadsPad + hd], M) * lw[w * kHeadsPad + hd];
    a.lse[(row0 + hd) * a.n_splits + s] = M + __log2f(Lt);
  }
}

// ---------------------------------------------------------------------------
// One workgroup per (head, sequence): merge the chunks into o_lat[r] (LDS),
// then out[b,h,i] = sum_j W_UV[h][i][j] o_lat[j].  The W_UV product runs one
// output row per wave step: lanes split the r-long dot product (16-byte loads of
// the row) and a wave reduction finishes it.
__global__ __launch_bounds__(256) void mla_merge_wuv(MlaDecodeArgs a) {
  __shared__ float olat[256];
  __shared__ float wts[64];
  __shared__ float wsum_s;
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(a.lens[b], a.T_max);
  const int n = (L + a.split - 1) / a.split;
  const int R = a.r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = (size_t)b * a.H + h;
  const float* lse = a.lse + row * a.n_splits;
  const float* op = a.o_part + row * a.n_splits * R;
  if (wave == 0) {
    // chunk weights 2^(lse_s - max); n <= n_splits, read 64 at a time
    float M = kNegInf;
    for (int s = lane; s < n; s += 64) M = fmaxf(M, lse[s]);
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float ws = 0.f;
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int s = s0 + lane;
      const float w = s < n ? exp2_fast(lse[s] - M) : 0.f;
      ws += w;
      if (s0 == 0) wts[lane] = w;
    }
    for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
    if (lane == 0) wsum_s = ws;
  }
  __syncthreads();
  const float inv = n > 0 ? 1.f / wsum_s : 0.f;
  for (int j = tid; j < R; j += 256) {
    float acc = 0.f;
    for (int s = 0; s < n; ++s) {
      // weights of chunks >= 64 are recomputed (only for very long caches)
      const float w = s < 64 ? wts[s] : 0.f;
      acc = fmaf(w, op[(size_t)s * R + j], acc);
    }
    olat[j] = acc * inv;
  }
  if (n > 64) {
    // rare: more than 64 chunks; add the rest with recomputed weights
    __syncthreads();
    float M = kNegInf;
    for (int s = 0; s < n; ++s) M = fmaxf(M, lse[s]);
    for (int j = tid; j < R; j += 256) {
      float acc = 0.f;
      for (int s = 64; s < n; ++s) acc = fmaf(exp2_fast(lse[s] - M), op[(size_t)s * R + j], acc);
      olat[j] += acc * inv;
    }
  }
  __syncthreads();
  const u16* wv = static_cast<const u16*>(a.w_uv) + (size_t)h * a.dv * R;
  for (int i = wave; i < a.dv; i += 4) {
    const u16* wrow = wv + (size_t)i * R;
    float acc = 0.f;
    for (int j = 8 * lane; j < R; j += 512) {
      const u16x8 w8 = *reinterpret_cast<const u16x8*>(wrow + j);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(bf16_to_f32(w8[k]), olat[j + k], acc);
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) {
      const size_t oi = row * a.dv + i;
      if (a.out_bf16) static_cast<__bf16*>(a.out)[oi] = (__bf16)acc;
      else static_cast<float*>(a.out)[oi] = acc;
    }
  }
}

template <int R>
hipError_t launch_partial(const MlaDecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (a.dR) {
    case 16: hipLaunchKernelGGL((mla_decode_partial<R, 16>), grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL((mla_decode_partial<R, 32>), grid, dim3(256), 0, st, a); break;
    case 48: hipLaunchKernelGGL((mla_decode_partial<R, 48>), grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((mla_decode_partial<R, 64>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool mla_decode_supported(int H, int r, int dR) {
  return H >= 1 && H <= kHeadsPad && (r == 64 || r == 128 || r == 256) &&
         (dR == 16 || dR == 32 || dR == 48 || dR == 64);
}

hipError_t launch_mla_decode(const MlaDecodeArgs& a, hipStream_t st) {
  if (!mla_decode_supported(a.H, a.r, a.dR)) return hipErrorInvalidValue;
  // w_uv rows are read 16 bytes at a time
  if (a.r % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mla_absorb, dim3(kHeadsPad, a.B), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.n_splits, a.B);
  e = a.r == 64 ? launch_partial<64>(a, grid, st) : a.r == 128 ? launch_partial<128>(a, grid, st)
                                                               : launch_partial<256>(a, grid, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_merge_wuv, dim3(a.H, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
