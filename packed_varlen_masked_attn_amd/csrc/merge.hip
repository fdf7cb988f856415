// Merge of partial attention results computed over disjoint key sets, through
// their log-sum-exp: the combining step of Ring attention ("[RFC]:
// HunyuanImage 3.0 deployment", Proposed Change P2; the Parallelism
// Acceleration Guide's Ring-Attention), where each rank attends to one chunk
// of the keys and values. For every (query, head) row r:
//   lse(r) = log sum_c exp(lse_c(r)),   O(r) = sum_c exp(lse_c(r) - lse(r)) O_c(r)
// A row whose parts all have lse = -inf (no key anywhere) gives O = 0 and
// lse = -inf.
//
// Memory-bound: each row reads n_parts x (4 D + 4) bytes and writes 2 D (+4).
// One row is handled by D/4 lanes, each owning four consecutive fp32 of every
// part (16-byte loads, coalesced across the row), so a 256-thread workgroup
// covers 1024 / D rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pva_internal.h"

namespace pva {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts, int n_parts,
                                                    int64_t rows, __bf16* __restrict__ out,
                                                    float* __restrict__ lse_out) {
  constexpr int TPR = D / 4;  // lanes per row
  const int64_t row = int64_t(blockIdx.x) * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int col = 4 * (threadIdx.x % TPR);
  // every part's lse and O slice is loaded before any is used, four parts
  // at a time, so that each lane keeps several 16-byte loads in flight (the
  // partial results are read once: non-temporal loads)
  constexpr int U = 4;
  float top = -INFINITY;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  for (int p0 = 0; p0 < n_parts; p0 += U) {
    float lp[U];
    f32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u;
      lp[u] = p < n_parts ? __builtin_nontemporal_load(lse_parts + int64_t(p) * rows + row) : -INFINITY;
      o[u] = p < n_parts ? __builtin_nontemporal_load(
                               reinterpret_cast<const f32x4*>(o_parts + (int64_t(p) * rows + row) * D + col))
                         : f32x4{};
    }
    // running max over the parts seen so far; earlier sums are rescaled when it moves
    float t = top;
#pragma unroll
    for (int u = 0; u < U; ++u) t = fmaxf(t, lp[u]);
    if (t != -INFINITY) {
      const float r = top == -INFINITY ? 0.0f : __expf(top - t);
      acc *= r;
      den *= r;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = lp[u] == -INFINITY ? 0.0f : __expf(lp[u] - t);
        acc += w * o[u];
        den += w;
      }
      top = t;
    }
  }
  bf16x4 res;
  float lse = -INFINITY;
  if (top == -INFINITY) {
    res = bf16x4{};
  } else {
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = (__bf16)(acc[e] * inv);
    lse = top + __logf(den);
  }
  *reinterpret_cast<bf16x4*>(out + row * D + col) = res;
  if (lse_out && col == 0) lse_out[row] = lse;
}

}  // namespace

int launch_merge(const float* o_parts, const float* lse_parts, int n_parts, int64_t rows, int head_dim, void* out,
                 float* lse_out, hipStream_t stream) {
  if (rows == 0) return PVA_OK;
  const int rpb = 256 / (head_dim / 4);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > int64_t(INT32_MAX)) return PVA_ERR_UNSUPPORTED;
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(unsigned(blocks)), dim3(256), 0, stream, o_parts, lse_parts, n_parts,
                       rows, static_cast<__bf16*>(out), lse_out);
  else if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(unsigned(blocks)), dim3(256), 0, stream, o_parts, lse_parts, n_parts,
                       rows, static_cast<__bf16*>(out), lse_out);
  else
    return PVA_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PVA_OK : PVA_ERR_HIP;
}

}  // namespace pva
