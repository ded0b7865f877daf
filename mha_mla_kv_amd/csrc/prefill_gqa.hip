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
//    each wave owns 32 rows.  Workgroups are issued heaviest (last) q-tile first.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: a 32-token K block is the A operand
//    (read from LDS, 16 bytes per lane), the wave's Q^T is the B operand, held in
//    registers for the whole kernel.  The accumulator gives each lane one query
//    row (lane % 32) and 16 tokens, so the row max needs one cross-half shuffle.
//  * O^T += V^T P^T: P stays in the accumulator layout and is the B operand after
//    a token permutation shared with the A operand; V^T comes from a row-major V
//    tile in LDS through ds_read_b64_tr_b16.
//  * K/V tiles of 64 tokens are double-buffered: the next tile is fetched into
//    registers with coalesced 16-byte loads while the current one is consumed.
//  * Online softmax in base 2; a wave skips tiles entirely above its diagonal.
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
constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kWaves = 4;     // 32 rows each

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

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: lane i of a 16-lane group points at row T0 + i/4, columns
// 4(i%4).. of a row-major [token][dim] tile; lane j receives tokens T0..T0+3 of
// column j.
__device__ __forceinline__ u16x4 lds_read_tr16(const u16* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_bit_cast(u16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p)));
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_causal(PrefillArgs a) {
  static_assert(D % 32 == 0 && D <= 128, "head_dim");
  static_assert(kBM == 32 * kWaves, "one 32-row slice per wave");
  constexpr int KP = D + 8;    // K tile pitch (elements): conflict-free 16-byte reads
  constexpr int VP = D + 16;   // V tile pitch: conflict-free transposed reads
  constexpr int KC = D / 16;   // 16-wide k chunks of the QK contraction
  constexpr int DB = D / 32;   // 32-wide dim blocks of O^T
  constexpr int kKElems = kBN * KP, kVElems = kBN * VP;
  constexpr int kLoads = kBN * D / 8 / 256;  // 16-byte loads per thread per tensor and tile
  __shared__ __attribute__((aligned(16))) u16 smem[2 * (kKElems + kVElems)];

  // heaviest q-tile first: blockIdx.x = 0 takes the last q-tile
  const int n_qt = (a.S + kBM - 1) / kBM;
  const int qt = n_qt - 1 - (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / a.n_rep;
  const int q0 = qt * kBM;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 31, h2 = lane >> 5;

  const size_t q_row = (size_t)a.Hq * D;
  const size_t kv_row = (size_t)a.Hkv * D;
  const u16* qp = static_cast<const u16*>(a.q) + ((size_t)b * a.S * a.Hq + h) * D;
  const u16* kp = static_cast<const u16*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * D;
  const u16* vp = static_cast<const u16*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * D;

  // This wave's query rows; Q^T as the B operand: lane holds Q[row ln][16c + 8h2 ..+8]
  const int row0 = q0 + wave * 32;
  const int my_row = row0 + ln;
  bf16x8 qop[KC];
  {
    const u16* qr = qp + (size_t)min(my_row, a.S - 1) * q_row + 8 * h2;
#pragma unroll
    for (int c = 0; c < KC; ++c) qop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qr + 16 * c));
  }

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = kNegInf, lsum = 0.f;

  // keys needed by this workgroup: [0, min(S, q0 + BM))
  const int kv_end = min(a.S, q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;

  // global -> register staging: thread covers token tid/16 + 16*i, dims 8*(tid%16)..
  u16x8 stk[kLoads], stv[kLoads];
  const int st_tok = tid / (D / 8), st_col = 8 * (tid % (D / 8));
  constexpr int kTokStep = 256 / (D / 8);
  auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int tok = min(kt * kBN + st_tok + kTokStep * i, a.S - 1);
      stk[i] = *reinterpret_cast<const u16x8*>(kp + (size_t)tok * kv_row + st_col);
      stv[i] = *reinterpret_cast<const u16x8*>(vp + (size_t)tok * kv_row + st_col);
    }
  };
  auto stash = [&](int buf) {
    u16* ks = smem + buf * (kKElems + kVElems);
    u16* vs = ks + kKElems;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int t = st_tok + kTokStep * i;
      *reinterpret_cast<u16x8*>(ks + t * KP + st_col) = stk[i];
      *reinterpret_cast<u16x8*>(vs + t * VP + st_col) = stv[i];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) fetch(kt + 1);
    const int kv0 = kt * kBN;
    if (kv0 <= row0 + 31) {  // some key of the tile is visible to some row of the wave
      const u16* ks = smem + buf * (kKElems + kVElems);
      const u16* vs = ks + kKElems;
      // S^T blocks: lane holds S^T[key kv0 + 32j + 8(i/4) + 4h2 + i%4][row ln]
      f32x16 sc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
        const u16* kr = ks + (32 * j + ln) * KP + 8 * h2;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr + 16 * c));
          acc = mfma_32x32x16(kop, qop[c], acc);
        }
        sc[j] = acc;
      }
      const bool diag = kv0 + kBN - 1 > row0;  // some key may lie above some row's diagonal
      float mt = kNegInf;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sc[j][i] * a.scale_log2e;
          if (diag) {
            const int key = kv0 + 32 * j + 8 * (i >> 2) + 4 * h2 + (i & 3);
            s = key <= my_row ? s : kNegInf;
          }
          sc[j][i] = s;
          mt = fmaxf(mt, s);
        }
      mt = max_xor32(mt);
      const float mn = fmaxf(m, mt);  // finite: key 0 is visible to every row, in tile 0
      const float alpha = exp2_fast(m - mn);
      m = mn;
      // P^T operands of the four 16-key PV steps: step v uses S^T block v/2, values 8(v%2)..+8
      bf16x8 pop[4];
      float ps = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = exp2_fast(sc[v >> 1][8 * (v & 1) + jj] - mn);
          ps += p;
          pop[v][jj] = (__bf16)p;
        }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int d = 0; d < DB; ++d) o[d] *= alpha;
      // O^T[dims 32d..][rows] += V^T P^T; step v covers keys 16v + 4h2 + (0..3) and
      // 16v + 8 + 4h2 + (0..3) of the tile (two transposed reads per operand)
      const int g16 = (lane >> 4) & 1;  // which 16-dim half of the 32-dim block
      const int i16 = lane & 15;
      const u16* vbase = vs + (4 * h2 + (i16 >> 2)) * VP + 16 * g16 + 4 * (i16 & 3);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const u16x4 lo = lds_read_tr16(vbase + (16 * v) * VP + 32 * d);
          const u16x4 hi = lds_read_tr16(vbase + (16 * v + 8) * VP + 32 * d);
          const u16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[d] = mfma_32x32x16(__builtin_bit_cast(bf16x8, av), pop[v], o[d]);
        }
      }
    }
    if (kt + 1 < n_kt) {
      stash(buf ^ 1);
    }
    __syncthreads();
  }

  // normalise and store: lane holds O^T[dims 32d + 8(i/4) + 4h2 + (i%4)][row ln]
  lsum = sum_xor32(lsum);
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
          for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(u16, (__bf16)(o[d][4 * q4 + e] * inv));
          *reinterpret_cast<u16x4*>(op + 32 * d + 8 * q4 + 4 * h2) = w;
        }
    } else {
      float* op = static_cast<float*>(a.out) + orow * D;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(op + 32 * d + 8 * q4 + 4 * h2) =
              make_float4(o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv, o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
    }
  }
}

}  // namespace

bool prefill_supported(int D) { return D == 64 || D == 128; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (!prefill_supported(a.D)) return hipErrorInvalidValue;
  const dim3 grid((a.S + kBM - 1) / kBM, a.Hq, a.B);
  if (a.D == 128) hipLaunchKernelGGL(prefill_causal<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(prefill_causal<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
