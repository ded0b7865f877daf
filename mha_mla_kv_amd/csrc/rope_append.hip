// Rotary position embedding of the new tokens' queries and keys, fused with the
// cache write of the keys (and of a second, unrotated stream).
//
// What is computed, for token i < n_b of sequence b at position m = P_b + i
// (P_b = max(start_pos[b], 0), n_b = n_new[b] clamped to [0, S]):
//   every head vector x of q and of k_new (width d) is rotated pair by pair,
//   (x[2j], x[2j+1]) turned by the angle m * base^(-2j/d);
//   the rotated key row goes to k_cache[b, m] and the x_new row to
//   x_cache[b, m] when m < T_max (or the key is rotated in place when there is
//   no k_cache); q is rotated in place.
// This is the step of Attention.forward on the "模型架构｜MQA & GQA 调研" page
// (code section) before the cache is read: apply_rotary_emb on the queries and
// keys, then the cache_k / cache_v writes at start_pos.  The pages call the
// rotation without printing it; the rotation of consecutive pairs with
// frequencies base^(-2j/d) is LLaMA-2's, whose Attention class that page prints.
// With MLA the rotated parts are q_rope and the shared k_rope, and x is the
// latent c_kv (qqstock DeepSeek MLA article, sections 1 and 3).
//
// How (not from the pages): one wave per token.  The wave first builds the
// token's table of (cos, sin) for the d/2 frequencies in LDS -- the angle and
// its reduction modulo 2 pi in fp64, the sine and cosine of the reduced angle in
// fp32 -- so every head of the token shares one table.  Then its lanes stream
// the q, k and x rows in 16-byte units (consecutive lanes on consecutive units,
// coalesced), four units in flight per lane, rotating in fp32 and rounding once
// to the element type.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kWaves = 4;          // tokens per workgroup
constexpr int kMaxPairs = 512;     // rope widths up to 1024
constexpr int kInFlight = 4;       // 16-byte units per lane and round

// 2 pi as a double and the remainder of 2 pi beyond it (for the two-step reduction)
constexpr double kTwoPiHi = 6.283185307179586232;
constexpr double kTwoPiLo = 2.449293598294706414e-16;
constexpr double kInvTwoPi = 0.15915494309189533577;

__device__ __forceinline__ float bf16_to_f32(u16 h) { return __uint_as_float((unsigned)h << 16); }
__device__ __forceinline__ u16 f32_to_bf16(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

// Rotates one 16-byte unit of a head vector starting at element e0 (a multiple
// of the unit's element count, so pairs never straddle units) with the table tab.
template <bool BF16>
__device__ __forceinline__ u32x4 rotate_unit(u32x4 u, int e0, const float2* tab) {
  if constexpr (BF16) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {  // one pair per 32-bit word: low half x[2j], high half x[2j+1]
      const float2 cs = tab[e0 / 2 + p];
      const float re = bf16_to_f32((u16)(u[p] & 0xffffu)), im = bf16_to_f32((u16)(u[p] >> 16));
      const float o0 = re * cs.x - im * cs.y;
      const float o1 = re * cs.y + im * cs.x;
      r[p] = (unsigned)f32_to_bf16(o0) | ((unsigned)f32_to_bf16(o1) << 16);
    }
    return r;
  } else {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float2 cs = tab[e0 / 2 + p];
      const float re = __uint_as_float(u[2 * p]), im = __uint_as_float(u[2 * p + 1]);
      r[2 * p] = __float_as_uint(re * cs.x - im * cs.y);
      r[2 * p + 1] = __float_as_uint(re * cs.y + im * cs.x);
    }
    return r;
  }
}

// Rotates `heads` head vectors of width d from src into dst (16-byte units;
// src may equal dst), lanes of one wave.
template <bool BF16>
__device__ __forceinline__ void rotate_rows(const u32x4* src, u32x4* dst, int heads, int d, const float2* tab,
                                            int lane) {
  constexpr int kElems = BF16 ? 8 : 4;  // elements per unit
  const int per_head = d / kElems;
  const int units = heads * per_head;
  for (int c0 = lane; c0 < units; c0 += 64 * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) {
      const int c = c0 + 64 * t;
      if (c < units) v[t] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) {
      const int c = c0 + 64 * t;
      if (c < units) dst[c] = rotate_unit<BF16>(v[t], (c % per_head) * kElems, tab);
    }
  }
}

__device__ __forceinline__ void copy_row(const u32x4* src, u32x4* dst, int units, int lane) {
  for (int c0 = lane; c0 < units; c0 += 64 * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) {
      const int c = c0 + 64 * t;
      if (c < units) v[t] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) {
      const int c = c0 + 64 * t;
      if (c < units) dst[c] = v[t];
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kWaves) void rope_append(RopeAppendArgs a) {
  __shared__ float2 tab_all[kWaves][kMaxPairs];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long long tok = (long long)blockIdx.x * kWaves + wave;  // b * S + i
  const bool have = tok < (long long)a.B * a.S;
  const int b = have ? (int)(tok / a.S) : 0;
  const int i = have ? (int)(tok - (long long)b * a.S) : 0;
  const int P = a.start_pos ? max(a.start_pos[b], 0) : 0;
  const int n = a.n_new ? min(max(a.n_new[b], 0), a.S) : a.S;
  const bool live = have && i < n;
  const long long m = (long long)P + i;  // the token's position
  float2* tab = tab_all[wave];
  if (live) {
    const int pairs = a.d / 2;
    for (int j = lane; j < pairs; j += 64) {
      const double theta = exp2(-(2.0 * j / a.d) * a.log2_base);
      const double ang = (double)m * theta;
      const double k = rint(ang * kInvTwoPi);
      const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));  // in [-pi, pi] up to rounding
      float s, c;
      sincosf((float)r, &s, &c);
      tab[j] = make_float2(c, s);
    }
  }
  __syncthreads();  // each wave reads only its own table; every wave reaches this barrier
  if (!live) return;

  constexpr int kElemBytes = BF16 ? 2 : 4;
  const size_t row_q = (size_t)a.Hq * a.d * kElemBytes / 16;  // 16-byte units per token row
  const size_t row_k = (size_t)a.Hk * a.d * kElemBytes / 16;
  if (a.q) {
    u32x4* q = static_cast<u32x4*>(a.q) + (size_t)tok * row_q;
    rotate_rows<BF16>(q, q, a.Hq, a.d, tab, lane);
  }
  const u32x4* ks = static_cast<const u32x4*>(a.k_new) + (size_t)tok * row_k;
  if (a.k_cache == nullptr) {  // rotate the new keys in place
    rotate_rows<BF16>(ks, const_cast<u32x4*>(ks), a.Hk, a.d, tab, lane);
  } else if (m < a.T_max) {
    u32x4* kd = static_cast<u32x4*>(a.k_cache) + ((size_t)b * a.T_max + (size_t)m) * row_k;
    rotate_rows<BF16>(ks, kd, a.Hk, a.d, tab, lane);
  }
  if (a.x_row_bytes > 0 && m < a.T_max) {
    const int ux = a.x_row_bytes / 16;
    const u32x4* xs = static_cast<const u32x4*>(a.x_new) + (size_t)tok * ux;
    u32x4* xd = static_cast<u32x4*>(a.x_cache) + ((size_t)b * a.T_max + (size_t)m) * ux;
    copy_row(xs, xd, ux, lane);
  }
}

template __global__ void rope_append<true>(RopeAppendArgs);
template __global__ void rope_append<false>(RopeAppendArgs);

}  // namespace

int rope_max_dim() { return 2 * kMaxPairs; }

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t st) {
  const long long tokens = (long long)a.B * a.S;
  const long long wgs = (tokens + kWaves - 1) / kWaves;
  if (wgs < 1 || wgs > 0x7fffffffLL || a.d > 2 * kMaxPairs) return hipErrorInvalidValue;
  if (a.bf16) hipLaunchKernelGGL(HIP_KERNEL_NAME(rope_append<true>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, st, a);
  else hipLaunchKernelGGL(HIP_KERNEL_NAME(rope_append<false>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
