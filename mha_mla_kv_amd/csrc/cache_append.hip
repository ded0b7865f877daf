// Cache append: the new tokens' rows written into a KV cache at their positions.
//
// What is computed: cache[b, P_b + i, :] = new[b, i, :] for i < n_b, for one or
// two (new, cache) pairs in one launch -- the cache_k / cache_v writes at
// start_pos .. start_pos + seqlen of Attention.forward on the "模型架构｜MQA &
// GQA 调研" page (code section), made before the cache is read; with the MLA
// latent cache the pair is (c_kv, k_rope), the two things the qqstock DeepSeek
// MLA article's section 1 and 3 say are cached.  P_b is clamped to [0, T_max],
// n_b to [0, min(S, T_max - P_b)]; rows outside [P_b, P_b + n_b) are untouched.
//
// How: a plain copy in 16-byte units, consecutive threads on consecutive units
// of a row, so both sides are coalesced; one grid row per sequence.  The bytes
// are moved, not converted, so any element type works.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void cache_append(CacheAppendArgs a) {
  const int b = blockIdx.y;
  const int P = a.start_pos ? min(max(a.start_pos[b], 0), a.T_max) : 0;
  const int n = min(a.n_new ? min(max(a.n_new[b], 0), a.S) : a.S, a.T_max - P);
  const int ua = a.row_bytes_a / 16, ub = a.row_bytes_b / 16, u = ua + ub;
  const long long total = (long long)n * u;
  for (long long id = (long long)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (long long)gridDim.x * blockDim.x) {
    const int i = (int)(id / u), c = (int)(id - (long long)i * u);
    if (c < ua) {
      const u32x4* src = static_cast<const u32x4*>(a.new_a) + ((size_t)b * a.S + i) * ua + c;
      u32x4* dst = static_cast<u32x4*>(a.cache_a) + ((size_t)b * a.T_max + P + i) * ua + c;
      *dst = *src;
    } else {
      const u32x4* src = static_cast<const u32x4*>(a.new_b) + ((size_t)b * a.S + i) * ub + (c - ua);
      u32x4* dst = static_cast<u32x4*>(a.cache_b) + ((size_t)b * a.T_max + P + i) * ub + (c - ua);
      *dst = *src;
    }
  }
}

}  // namespace

hipError_t launch_cache_append(const CacheAppendArgs& a, hipStream_t st) {
  const long long units = (long long)a.S * ((a.row_bytes_a + a.row_bytes_b) / 16);
  const long long blocks = (units + 255) / 256;
  const unsigned gx = (unsigned)(blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks));
  hipLaunchKernelGGL(cache_append, dim3(gx, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace attn
