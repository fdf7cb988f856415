// C-ABI of the packed mixed-mask attention library: argument validation,
// descriptor lifetime, error reporting and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pva_internal.h"

namespace pva {
int launch_fwd_bf16(const void* q, const void* k, const void* v, const int32_t* cu, const pva_seg_desc* d,
                    float scale, const OutSpec& out, const PagedKV* paged, hipStream_t stream);
int launch_merge(const float* o_parts, const float* lse_parts, int n_parts, int64_t rows, int head_dim, void* out,
                 float* lse_out, hipStream_t stream);
int launch_fwd_fp8(const void* q, const void* k, const void* v, const float* qs, const float* ks,
                   const float* vs, const int32_t* cu, const pva_seg_desc* d, float scale, const OutSpec& out,
                   hipStream_t stream);
}  // namespace pva

namespace {

thread_local std::string g_last_error;

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int ok() {
  g_last_error.clear();
  return PVA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_error(hipError_t e, const char* what) {
  return set_error(PVA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int check_one_cu(const int32_t* cu, const std::vector<int32_t>& want, const char* name, hipStream_t stream) {
  std::vector<int32_t> host(want.size());
  hipError_t e = hipMemcpyAsync(host.data(), cu, host.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_error(e, (std::string("PVA_CHECK: reading ") + name).c_str());
  if (host != want)
    return set_error(PVA_ERR_INVALID_ARG, std::string("PVA_CHECK: device ") + name + " differs from the descriptor's");
  return PVA_OK;
}

int check_cu(const int32_t* cu_q, const int32_t* cu_k, const pva_seg_desc* d, hipStream_t stream) {
  const char* env = std::getenv("PVA_CHECK");
  if (!env || std::strcmp(env, "1") != 0) return PVA_OK;
  int st = check_one_cu(cu_k, d->plan.cu_seqlens, "cu_seqlens_k", stream);
  if (st == PVA_OK && cu_q != cu_k) st = check_one_cu(cu_q, d->plan.cu_seqlens_q, "cu_seqlens_q", stream);
  return st;
}

int validate_fwd(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                 const pva_seg_desc* d, float scale, void* out, pva_dtype want) {
  // every check here is host-only and runs before anything touches the device
  if (!d) return set_error(PVA_ERR_INVALID_ARG, "seg_desc is NULL");
  // a tensor of zero rows may come without an address (q and out when no row
  // is queried, k and v when the key chunks hold no rows)
  const bool no_queries = d->plan.total_q == 0, no_keys = d->plan.total_tokens == 0;
  if (((!q || !out) && !no_queries) || ((!k || !v) && !no_keys) || !cu_q || !cu_k)
    return set_error(PVA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return set_error(PVA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (!(std::isfinite(scale) && scale > 0.0f)) return set_error(PVA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d->plan.dtype != want)
    return set_error(PVA_ERR_INVALID_ARG, "seg_desc was built for another dtype");
  if (!d->d_items) return set_error(PVA_ERR_INVALID_ARG, "seg_desc was built host-only and cannot be launched");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e, "hipGetDevice");
  if (dev != d->device)
    return set_error(PVA_ERR_INVALID_ARG, "seg_desc was built on device " + std::to_string(d->device) +
                                              " but the current device is " + std::to_string(dev));
  if (d->scratch_generation != 0 && !pva::scratch_is_current(d->device, d->scratch_generation))
    return set_error(PVA_ERR_INVALID_ARG,
                     "a later pva_seg_desc_build_noalloc on this device replaced this descriptor's work list: "
                     "build it again");
  return PVA_OK;
}

// Where a descriptor's device work list goes.
enum class Placement {
  kHostOnly,       // nowhere: inspection only
  kOwnAllocation,  // one hipMalloc per descriptor, freed with it
  kScratch,        // the device's fixed no-alloc buffer (no allocation)
};

// Builds a plan with `plan_fn` and, unless host-only, uploads the work list
// and the key limits to the current device (one buffer: items, then limits).
template <typename PlanFn>
int build_common(PlanFn plan_fn, Placement placement, void* stream, pva_seg_desc** out) {
  if (!out) return set_error(PVA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pva_seg_desc* d = new (std::nothrow) pva_seg_desc();
  if (!d) return set_error(PVA_ERR_NO_MEMORY, "host allocation failed");
  std::string err;
  int st;
  try {
    st = plan_fn(&d->plan, &err);
  } catch (const std::bad_alloc&) {
    st = PVA_ERR_NO_MEMORY;
    err = "host allocation failed";
  }
  if (st != PVA_OK) {
    delete d;
    return set_error(st, err);
  }
  if (placement != Placement::kHostOnly) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      delete d;
      return hip_error(e, "hipGetDevice");
    }
    d->device = dev;
    const size_t item_bytes = (d->plan.items.size() * sizeof(pva::WorkItem) + 255) / 256 * 256;
    const size_t lim_bytes = d->plan.key_lim.size() * sizeof(int32_t);
    // never empty: a device descriptor always has a work-list address, also
    // when it queries no row (then it has no items and no limits)
    const size_t bytes = std::max<size_t>(item_bytes + lim_bytes, 256);
    void* base = nullptr;
    if (placement == Placement::kScratch) {
      // the fixed buffer is never allocated or freed here
      st = pva::scratch_acquire(dev, bytes, &base, &d->scratch_generation, &err);
      if (st != PVA_OK) {
        delete d;
        return set_error(st, err);
      }
    } else {
      e = hipMalloc(&base, bytes);
      if (e != hipSuccess) {
        delete d;
        return set_error(PVA_ERR_NO_MEMORY, std::string("hipMalloc of the work list: ") + hipGetErrorString(e));
      }
    }
    d->d_items = base;
    d->d_lims = reinterpret_cast<int32_t*>(static_cast<char*>(base) + item_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!d->plan.items.empty())
      e = hipMemcpyAsync(d->d_items, d->plan.items.data(), d->plan.items.size() * sizeof(pva::WorkItem),
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess && lim_bytes > 0)
      e = hipMemcpyAsync(d->d_lims, d->plan.key_lim.data(), lim_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      if (placement == Placement::kOwnAllocation) (void)hipFree(base);
      delete d;
      return hip_error(e, "uploading the work list");
    }
  }
  *out = d;
  return ok();
}

int build_two(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads, int32_t head_dim,
              pva_dtype dtype, Placement placement, void* stream, pva_seg_desc** out) {
  return build_common(
      [&](pva::Plan* p, std::string* err) {
        return pva::build_plan(text_len, image_len, nseq, num_heads, head_dim, dtype, p, err);
      },
      placement, stream, out);
}

int build_segs(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count, const int32_t* q_start,
               const int32_t* k_lo, const int32_t* k_hi, int32_t nseq, int32_t num_heads, int32_t head_dim,
               pva_dtype dtype, bool upload, void* stream, pva_seg_desc** out) {
  return build_common(
      [&](pva::Plan* p, std::string* err) {
        return pva::build_plan_segments(seg_len, seg_kind, seg_count, q_start, k_lo, k_hi, nseq, num_heads, head_dim,
                                        dtype, p, err);
      },
      upload ? Placement::kOwnAllocation : Placement::kHostOnly, stream, out);
}

int fwd_bf16(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
             const pva_seg_desc* d, float scale, const pva::OutSpec& out, void* stream) {
  int st = validate_fwd(q, k, v, cu_q, cu_k, d, scale, out.o, PVA_BF16);
  if (st != PVA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = check_cu(cu_q, cu_k, d, s)) != PVA_OK) return st;
  // no key rows: every tile range is empty and nothing is read, but the
  // kernels still form addresses from a base
  if (!k) k = d->d_items;
  if (!v) v = d->d_items;
  st = pva::launch_fwd_bf16(q, k, v, cu_k, d, scale, out, nullptr, s);
  if (st != PVA_OK) return set_error(st, "bf16 kernel launch failed");
  return ok();
}

int fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale, const float* k_scale,
            const float* v_scale, const int32_t* cu_q, const int32_t* cu_k, const pva_seg_desc* d, float scale,
            const pva::OutSpec& out, void* stream) {
  int st = validate_fwd(q, k, v, cu_q, cu_k, d, scale, out.o, PVA_FP8_E4M3);
  if (st != PVA_OK) return st;
  if (!q_scale || !k_scale || !v_scale) return set_error(PVA_ERR_INVALID_ARG, "a scale pointer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = check_cu(cu_q, cu_k, d, s)) != PVA_OK) return st;
  // no key rows: every tile range is empty and nothing is read, but the
  // kernels still form addresses from a base
  if (!k) k = d->d_items;
  if (!v) v = d->d_items;
  st = pva::launch_fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_k, d, scale, out, s);
  if (st == PVA_ERR_UNSUPPORTED) return set_error(st, "the fp8 kernel takes head_dim 128 and its own tile shape only");
  if (st != PVA_OK) return set_error(st, "fp8 kernel launch failed");
  return ok();
}

// Output of a launch that writes a plain bf16 result.
pva::OutSpec plain_out(void* out) { return pva::OutSpec{out, 0, nullptr, nullptr, nullptr}; }

// Output of an accumulating key-chunk launch: the running result is read from
// (o_acc, lse_acc) and the merged one written back to them, or, with `out`,
// O goes to out in bf16 (lse_acc is updated either way).
int accumulate_out(const pva_seg_desc* d, float* o_acc, float* lse_acc, void* out, pva::OutSpec* spec) {
  if (!d) return set_error(PVA_ERR_INVALID_ARG, "seg_desc is NULL");
  if ((!o_acc || !lse_acc) && d->plan.total_q > 0) return set_error(PVA_ERR_INVALID_ARG, "o_acc or lse_acc is NULL");
  if (!aligned16(o_acc)) return set_error(PVA_ERR_INVALID_ARG, "o_acc must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse_acc) & 3u) != 0)
    return set_error(PVA_ERR_INVALID_ARG, "lse_acc must be 4-byte aligned");
  // other rows' running values must not be overwritten before they are read
  const uintptr_t elems = uintptr_t(d->plan.total_q) * uintptr_t(d->plan.num_heads) * uintptr_t(d->plan.head_dim);
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(o_acc), b1 = b0 + 4 * elems;
  const uintptr_t l0 = reinterpret_cast<uintptr_t>(lse_acc),
                  l1 = l0 + 4 * uintptr_t(d->plan.total_q) * uintptr_t(d->plan.num_heads);
  if (b0 < l1 && l0 < b1) return set_error(PVA_ERR_INVALID_ARG, "o_acc overlaps lse_acc");
  if (out) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(out), a1 = a0 + 2 * elems;
    if ((a0 < b1 && b0 < a1) || (a0 < l1 && l0 < a1))
      return set_error(PVA_ERR_INVALID_ARG, "out overlaps o_acc or lse_acc");
    *spec = pva::OutSpec{out, 0, lse_acc, o_acc, lse_acc};
  } else {
    *spec = pva::OutSpec{o_acc, 1, lse_acc, o_acc, lse_acc};
  }
  return PVA_OK;
}

int need_full_queries(const pva_seg_desc* d) {
  if (d && d->plan.queries_suffix())
    return set_error(PVA_ERR_INVALID_ARG, "seg_desc queries only a suffix of its sequences: use packed_attn_fwd_varlen");
  return PVA_OK;
}

}  // namespace

extern "C" {

int pva_seg_desc_build(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
                       int32_t head_dim, pva_dtype dtype, void* stream, pva_seg_desc** out) {
  return build_two(text_len, image_len, nseq, num_heads, head_dim, dtype, Placement::kOwnAllocation, stream, out);
}

int pva_seg_desc_build_noalloc(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
                               int32_t head_dim, pva_dtype dtype, void* stream, pva_seg_desc** out) {
  return build_two(text_len, image_len, nseq, num_heads, head_dim, dtype, Placement::kScratch, stream, out);
}

int pva_seg_desc_build_host(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
                            int32_t head_dim, pva_dtype dtype, pva_seg_desc** out) {
  return build_two(text_len, image_len, nseq, num_heads, head_dim, dtype, Placement::kHostOnly, nullptr, out);
}

int pva_seg_desc_build_segments(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                const int32_t* q_start, int32_t nseq, int32_t num_heads, int32_t head_dim,
                                pva_dtype dtype, void* stream, pva_seg_desc** out) {
  return build_segs(seg_len, seg_kind, seg_count, q_start, nullptr, nullptr, nseq, num_heads, head_dim, dtype, true,
                    stream, out);
}

int pva_seg_desc_build_segments_host(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                     const int32_t* q_start, int32_t nseq, int32_t num_heads, int32_t head_dim,
                                     pva_dtype dtype, pva_seg_desc** out) {
  return build_segs(seg_len, seg_kind, seg_count, q_start, nullptr, nullptr, nseq, num_heads, head_dim, dtype, false,
                    nullptr, out);
}

int pva_seg_desc_build_kv_chunk(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi, int32_t nseq,
                                int32_t num_heads, int32_t head_dim, pva_dtype dtype, void* stream,
                                pva_seg_desc** out) {
  if (!k_lo || !k_hi) return set_error(PVA_ERR_INVALID_ARG, "k_lo / k_hi is NULL");
  return build_segs(seg_len, seg_kind, seg_count, q_start, k_lo, k_hi, nseq, num_heads, head_dim, dtype, true, stream,
                    out);
}

int pva_seg_desc_build_kv_chunk_host(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                     const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi, int32_t nseq,
                                     int32_t num_heads, int32_t head_dim, pva_dtype dtype, pva_seg_desc** out) {
  if (!k_lo || !k_hi) return set_error(PVA_ERR_INVALID_ARG, "k_lo / k_hi is NULL");
  return build_segs(seg_len, seg_kind, seg_count, q_start, k_lo, k_hi, nseq, num_heads, head_dim, dtype, false,
                    nullptr, out);
}

int pva_seg_desc_cu_seqlens(const pva_seg_desc* d, const int32_t** host_cu, int32_t* len) {
  if (!d || !host_cu || !len) return set_error(PVA_ERR_INVALID_ARG, "NULL argument");
  *host_cu = d->plan.cu_seqlens.data();
  *len = static_cast<int32_t>(d->plan.cu_seqlens.size());
  return ok();
}

int pva_seg_desc_cu_seqlens_q(const pva_seg_desc* d, const int32_t** host_cu_q, int32_t* len) {
  if (!d || !host_cu_q || !len) return set_error(PVA_ERR_INVALID_ARG, "NULL argument");
  *host_cu_q = d->plan.cu_seqlens_q.data();
  *len = static_cast<int32_t>(d->plan.cu_seqlens_q.size());
  return ok();
}

int pva_seg_desc_key_limits(const pva_seg_desc* d, const int32_t** key_limits, int32_t* len) {
  if (!d || !key_limits || !len) return set_error(PVA_ERR_INVALID_ARG, "NULL argument");
  *key_limits = d->plan.key_lim.data();
  *len = static_cast<int32_t>(d->plan.key_lim.size());
  return ok();
}

int64_t pva_seg_desc_useful_flops(const pva_seg_desc* d) { return d ? d->plan.useful_flops : -1; }

int pva_seg_desc_tile(const pva_seg_desc* d, int32_t* block_m, int32_t* block_n) {
  if (!d || !block_m || !block_n) return set_error(PVA_ERR_INVALID_ARG, "NULL argument");
  *block_m = d->plan.tile.bm;
  *block_n = d->plan.tile.bn;
  return ok();
}

int pva_seg_desc_work_items(const pva_seg_desc* d, const int32_t** items, int32_t* n_items) {
  if (!d || !items || !n_items) return set_error(PVA_ERR_INVALID_ARG, "NULL argument");
  *items = reinterpret_cast<const int32_t*>(d->plan.items.data());
  *n_items = static_cast<int32_t>(d->plan.items.size());
  return ok();
}

void pva_seg_desc_free(pva_seg_desc* d) {
  if (!d) return;
  if (d->d_items && d->scratch_generation == 0) {  // the no-alloc buffer is never freed
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != d->device && d->device >= 0) (void)hipSetDevice(d->device);
    (void)hipFree(d->d_items);
    if (cur >= 0 && cur != d->device) (void)hipSetDevice(cur);
  }
  delete d;
}

int packed_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    const pva_seg_desc* seg_desc, float scale, void* out, void* stream) {
  int st = need_full_queries(seg_desc);
  if (st != PVA_OK) return st;
  return fwd_bf16(q, k, v, cu_seqlens, cu_seqlens, seg_desc, scale, plain_out(out), stream);
}

int packed_attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale, void* out,
                           void* stream) {
  return fwd_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc, scale, plain_out(out), stream);
}

int packed_attn_fwd_partial(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale, float* out_f32,
                            float* lse, void* stream) {
  if (!lse && !(seg_desc && seg_desc->plan.total_q == 0)) return set_error(PVA_ERR_INVALID_ARG, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return set_error(PVA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return fwd_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc, scale, pva::OutSpec{out_f32, 1, lse, nullptr, nullptr},
                  stream);
}

int packed_attn_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          int32_t table_stride, int32_t block_size, int32_t num_blocks, const int32_t* cu_seqlens_q,
                          const pva_seg_desc* seg_desc, float scale, void* out, void* stream) {
  // host checks first (the K/V pointers stand in for cu_seqlens_k, which paged K/V does not use)
  int st = validate_fwd(q, k_pool, v_pool, cu_seqlens_q, cu_seqlens_q, seg_desc, scale, out, PVA_BF16);
  if (st != PVA_OK) return st;
  if (!block_table) return set_error(PVA_ERR_INVALID_ARG, "block_table is NULL");
  if (seg_desc->plan.chunked()) return set_error(PVA_ERR_INVALID_ARG, "paged K/V takes whole-sequence descriptors");
  if (block_size < pva::kBf16BlockN || (block_size & (block_size - 1)) != 0 || block_size > (1 << 20))
    return set_error(PVA_ERR_INVALID_ARG, "block_size must be a power of two, >= 32 and <= 2^20");
  if (num_blocks < 1) return set_error(PVA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (int64_t(num_blocks) * block_size * seg_desc->plan.num_heads * seg_desc->plan.head_dim > (int64_t(1) << 62))
    return set_error(PVA_ERR_INVALID_ARG, "pool too large");
  int64_t need = 0;
  for (int32_t L : seg_desc->plan.seq_len) need = std::max<int64_t>(need, (int64_t(L) + block_size - 1) / block_size);
  if (table_stride < need)
    return set_error(PVA_ERR_INVALID_ARG, "table_stride is smaller than the blocks the longest sequence needs");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* env = std::getenv("PVA_CHECK");
  if (env && std::strcmp(env, "1") == 0) {
    if ((st = check_one_cu(cu_seqlens_q, seg_desc->plan.cu_seqlens_q, "cu_seqlens_q", s)) != PVA_OK) return st;
    std::vector<int32_t> tbl(size_t(seg_desc->plan.nseq) * table_stride);
    hipError_t e = hipMemcpyAsync(tbl.data(), block_table, tbl.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_error(e, "PVA_CHECK: reading block_table");
    for (int32_t q = 0; q < seg_desc->plan.nseq; ++q) {
      const int64_t nb = (int64_t(seg_desc->plan.seq_len[q]) + block_size - 1) / block_size;
      for (int64_t b = 0; b < nb; ++b) {
        const int32_t x = tbl[size_t(q) * table_stride + b];
        if (x < 0 || x >= num_blocks) return set_error(PVA_ERR_INVALID_ARG, "PVA_CHECK: block_table entry out of range");
      }
    }
  }
  const pva::PagedKV pg{block_table, table_stride, block_size, num_blocks};
  st = pva::launch_fwd_bf16(q, k_pool, v_pool, cu_seqlens_q, seg_desc, scale, plain_out(out), &pg, s);
  if (st != PVA_OK) return set_error(st, "bf16 kernel launch failed");
  return ok();
}

int pva_merge_partials(const float* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows, int32_t head_dim,
                       void* out, float* lse_out, void* stream) {
  if (n_parts < 1) return set_error(PVA_ERR_INVALID_ARG, "n_parts must be >= 1");
  if (rows < 0) return set_error(PVA_ERR_INVALID_ARG, "rows must be >= 0");
  // zero rows may come without addresses
  if ((!o_parts || !lse_parts || !out) && rows > 0) return set_error(PVA_ERR_INVALID_ARG, "a tensor pointer is NULL");
  if (head_dim != 64 && head_dim != 128) return set_error(PVA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (!aligned16(o_parts) || !aligned16(out)) return set_error(PVA_ERR_INVALID_ARG, "o_parts and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse_parts) & 3u) != 0 || (reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0)
    return set_error(PVA_ERR_INVALID_ARG, "lse_parts and lse_out must be 4-byte aligned");
  if (rows > (int64_t(1) << 40) / head_dim / n_parts) return set_error(PVA_ERR_INVALID_ARG, "tensor too large");
  int st = pva::launch_merge(o_parts, lse_parts, n_parts, rows, head_dim, out, lse_out, static_cast<hipStream_t>(stream));
  if (st != PVA_OK) return set_error(st, "merge kernel launch failed");
  return ok();
}

int packed_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale, const float* k_scale,
                        const float* v_scale, const int32_t* cu_seqlens, const pva_seg_desc* seg_desc, float scale,
                        void* out, void* stream) {
  int st = need_full_queries(seg_desc);
  if (st != PVA_OK) return st;
  return fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens, cu_seqlens, seg_desc, scale, plain_out(out), stream);
}

int packed_attn_fwd_varlen_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                               const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale, void* out,
                               void* stream) {
  return fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, seg_desc, scale, plain_out(out),
                 stream);
}

int packed_attn_fwd_partial_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                float* out_f32, float* lse, void* stream) {
  if (!lse && !(seg_desc && seg_desc->plan.total_q == 0)) return set_error(PVA_ERR_INVALID_ARG, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return set_error(PVA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, seg_desc, scale,
                 pva::OutSpec{out_f32, 1, lse, nullptr, nullptr}, stream);
}

int packed_attn_fwd_partial_accumulate(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                       float* o_acc, float* lse_acc, void* out, void* stream) {
  pva::OutSpec spec{};
  int st = accumulate_out(seg_desc, o_acc, lse_acc, out, &spec);
  if (st != PVA_OK) return st;
  return fwd_bf16(q, k, v, cu_seqlens_q, cu_seqlens_k, seg_desc, scale, spec, stream);
}

int packed_attn_fwd_partial_accumulate_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                           const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                           float* o_acc, float* lse_acc, void* out, void* stream) {
  pva::OutSpec spec{};
  int st = accumulate_out(seg_desc, o_acc, lse_acc, out, &spec);
  if (st != PVA_OK) return st;
  return fwd_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, seg_desc, scale, spec, stream);
}

int pva_timeline_clear(pva_dtype kernel) {
  if (kernel != PVA_BF16 && kernel != PVA_FP8_E4M3) return set_error(PVA_ERR_INVALID_ARG, "unknown kernel dtype");
  void* p = nullptr;
  const int st = kernel == PVA_BF16 ? pva::timeline_records_bf16(&p) : pva::timeline_records_fp8(&p);
  if (st == PVA_ERR_UNSUPPORTED)
    return set_error(st, "this library records no workgroup timeline (libpva_timeline.so does)");
  if (st != PVA_OK) return set_error(st, "locating the timeline records failed");
  const size_t bytes = size_t(PVA_TIMELINE_MAX_ITEMS) * PVA_TIMELINE_FIELDS * sizeof(uint64_t);
  hipError_t e = hipMemset(p, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_error(e, "clearing the timeline records");
  return ok();
}

int pva_timeline_read(pva_dtype kernel, uint64_t* host_records, int64_t n_records) {
  if (kernel != PVA_BF16 && kernel != PVA_FP8_E4M3) return set_error(PVA_ERR_INVALID_ARG, "unknown kernel dtype");
  if (!host_records) return set_error(PVA_ERR_INVALID_ARG, "host_records is NULL");
  if (n_records < 0 || n_records > PVA_TIMELINE_MAX_ITEMS)
    return set_error(PVA_ERR_INVALID_ARG, "n_records must lie in [0, PVA_TIMELINE_MAX_ITEMS]");
  void* p = nullptr;
  const int st = kernel == PVA_BF16 ? pva::timeline_records_bf16(&p) : pva::timeline_records_fp8(&p);
  if (st == PVA_ERR_UNSUPPORTED)
    return set_error(st, "this library records no workgroup timeline (libpva_timeline.so does)");
  if (st != PVA_OK) return set_error(st, "locating the timeline records failed");
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess && n_records > 0)
    e = hipMemcpy(host_records, p, size_t(n_records) * PVA_TIMELINE_FIELDS * sizeof(uint64_t),
                  hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_error(e, "reading the timeline records");
  return ok();
}

const char* pva_last_error(void) { return g_last_error.c_str(); }

const char* pva_version(void) {
#ifdef PVA_WG_TIMELINE
  return "pva 0.3 gfx950 (workgroup timeline)";
#else
  return "pva 0.3 gfx950";
#endif
}

}  // extern "C"
