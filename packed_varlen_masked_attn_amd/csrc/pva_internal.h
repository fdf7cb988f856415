// Internal declarations shared by the planner, the C-ABI layer and the kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pva.h"

#if defined(__HIPCC__)
#define PVA_HOST_DEVICE __host__ __device__
#else
#define PVA_HOST_DEVICE
#endif

namespace pva {

// One record of the device work list: a (sequence, head, query tile).
// k_full_end / k_end are key-tile indices: tiles [0, k_full_end) need no mask,
// [k_full_end, k_end) are masked element-wise, tiles >= k_end are never read.
struct WorkItem {
  int32_t seq;     // -1: empty slot (keeps the XCD alignment of the list)
  int32_t head;
  int32_t q0;      // first query row of the tile, relative to the sequence start
  int32_t q_rows;  // valid rows in the tile (<= BM)
  int32_t k_full_end;
  int32_t k_end;
  int32_t qo_row;  // row of Q and O holding query row q0 (packed queried rows)
  int32_t seq_len; // K/V rows held for this sequence (its length unless chunked)
};
static_assert(sizeof(WorkItem) == 32, "work item is 8 int32");

// Tile shape of the bf16 kernel, shared with the planner (the work list's
// key-tile indices are in units of kBf16BlockN keys).
#ifndef PVA_BF16_BN
#define PVA_BF16_BN 32
#endif
#ifndef PVA_BF16_BM
#define PVA_BF16_BM 128
#endif
constexpr int32_t kBf16BlockM = PVA_BF16_BM;
constexpr int32_t kBf16BlockN = PVA_BF16_BN;

// LDS ring depth of each kernel: a work item with k_end key tiles loads the K
// rows of tiles [0, k_end + stages) and the V rows of tiles
// [0, k_end + stages - 1) (the loads run ahead of the arithmetic on every
// path; tiles past the sequence end have an empty range, below).
constexpr int32_t kBf16Stages = 3;
constexpr int32_t kFp8Stages = 4;

// Byte ranges of the K/V tile loads. One head's rows of a sequence (or of
// its key chunk) are `rows` rows, `row_stride` bytes apart and `row_bytes`
// long; its span runs from the first byte of the first row to the last byte
// of the last row, and is empty when the sequence holds no key rows.
PVA_HOST_DEVICE constexpr uint32_t head_span_bytes(int32_t rows, uint32_t row_stride, uint32_t row_bytes) {
  return rows > 0 ? uint32_t(rows - 1) * row_stride + row_bytes : 0u;
}
// A tile's loads go through a buffer resource that starts `tile_offset`
// bytes into the span and ends with it, so loads at or past the range read
// zeros without touching memory; a tile past the end gets an empty range.
PVA_HOST_DEVICE constexpr uint32_t tile_range_bytes(uint32_t span, uint32_t tile_offset) {
  return span - (tile_offset < span ? tile_offset : span);
}

// Tile shape used by the kernels for a given element type and head size.
struct TileShape {
  int32_t bm;  // query rows per work item
  int32_t bn;  // keys per streamed tile
};
TileShape tile_shape(pva_dtype dtype, int32_t head_dim);

// Number of XCDs whose L2 caches the scheduler groups work for.
constexpr int kNumXcd = 8;

struct Plan {
  pva_dtype dtype = PVA_BF16;
  int32_t nseq = 0, num_heads = 0, head_dim = 0;
  TileShape tile{0, 0};
  std::vector<int32_t> text_len, image_len;  // two-segment builds only (for inspection)
  std::vector<int32_t> seq_len, q_start;     // per sequence: length, first queried row
  std::vector<int32_t> k_lo, kv_len;         // per sequence: first key row held by K/V, rows held
  std::vector<int32_t> cu_seqlens;           // K/V row offsets [nseq + 1]
  std::vector<int32_t> cu_seqlens_q;         // Q/O row offsets [nseq + 1] (equal when q_start == 0)
  std::vector<int32_t> key_lim;              // per queried row: allowed K/V rows are [0, lim) of its sequence
  std::vector<WorkItem> items;               // launch order, XCD-interleaved, padded with empty slots
  int64_t useful_flops = 0;
  int64_t total_tokens = 0;  // K/V rows
  int64_t total_q = 0;       // Q/O rows
  bool queries_suffix() const { return total_q != total_tokens || chunked(); }
  bool chunked() const {
    for (size_t s = 0; s < kv_len.size(); ++s)
      if (k_lo[s] != 0 || kv_len[s] != seq_len[s]) return true;
    return false;
  }
};

// Where a forward launch writes its result (device pointers). Rows are the
// queried rows in packed order; lse is indexed row * H + head.
//   o        bf16 [rows, H, D], or fp32 when o_f32
//   lse      fp32 log-sum-exp of each row's scaled scores, or null
//   acc_o,   a running fp32 result [rows, H, D] and its log-sum-exp over other
//   acc_lse  keys of the same rows, folded into this launch's result before it
//            is written (log-sum-exp weights; a row whose acc_lse is -inf
//            takes nothing from acc_o), or both null. o and lse may be acc_o
//            and acc_lse: each lane reads its elements before writing them.
struct OutSpec {
  void* o;
  int o_f32;
  float* lse;
  const float* acc_o;
  const float* acc_lse;
};

// K / V held in a paged pool [num_blocks, block_size, H, D] (device table).
struct PagedKV {
  const int32_t* table;  // device int32 [nseq * stride]: pool block of each block of keys
  int32_t stride;        // table entries per sequence
  int32_t block_size;    // keys per block: a power of two, a multiple of the key tile
  int32_t num_blocks;    // blocks in each pool
};

// Fixed device buffer of the allocation-free descriptor builder (one per
// device). scratch_acquire hands out its address on the current device
// (taken once per device) for `bytes` bytes and starts a new generation,
// which retires the previous no-alloc descriptor of that device;
// scratch_is_current tells whether a descriptor's generation still owns it.
constexpr size_t kNoAllocScratchBytes = PVA_NOALLOC_SCRATCH_BYTES;
int scratch_acquire(int device, size_t bytes, void** ptr, uint64_t* generation, std::string* err);
bool scratch_is_current(int device, uint64_t generation);

// Device address of a forward kernel's workgroup-timeline records on the
// current device (the timing build only; PVA_ERR_UNSUPPORTED otherwise).
int timeline_records_bf16(void** ptr);
int timeline_records_fp8(void** ptr);

// Validates and plans; on failure returns a status and fills `err`.
// Two segments per sequence: text (causal) then one image block (full).
int build_plan(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
               int32_t head_dim, pva_dtype dtype, Plan* plan, std::string* err);
// Any number of segments per sequence, an optional first queried row and an
// optional key chunk [k_lo, k_hi) held by K/V (both NULL: whole sequences).
int build_plan_segments(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                        const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi, int32_t nseq,
                        int32_t num_heads, int32_t head_dim, pva_dtype dtype, Plan* plan, std::string* err);

}  // namespace pva

// The descriptor handed across the C-ABI.
struct pva_seg_desc {
  pva::Plan plan;
  void* d_items = nullptr;    // device copy of plan.items (nullptr for host-only descriptors)
  int32_t* d_lims = nullptr;  // device copy of plan.key_lim (same allocation as d_items)
  int32_t device = -1;        // HIP device the work list lives on
  uint64_t scratch_generation = 0;  // > 0: the work list lives in that device's no-alloc buffer
};
