// Host-only checks of the segment-descriptor builder, the tile scheduler and
// the C-ABI's argument validation, meant to be built with AddressSanitizer
// and UndefinedBehaviorSanitizer (g++, no device code) and run without a GPU.
//
// Besides the planner's own invariants it replays, for every work item, the
// byte ranges of the K/V tile loads the kernels issue (the same range
// functions the kernels call, over the same tiles) and checks that each one
// lies inside the item's own rows of the K/V tensor. The key-chunk case with
// an empty chunk on the last sequence is among the inputs: a tile range
// formed from a row count of zero must be empty, not wrap around.
//
// Exit status 0 when every check holds; the first failures are printed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "pva.h"
#include "pva_internal.h"

// This test program holds no kernels: the C-ABI layer's launchers are stand-ins
// that must never be reached (every call here fails validation on the host).
namespace pva {
int launch_fwd_bf16(const void*, const void*, const void*, const int32_t*, const pva_seg_desc*, float, const OutSpec&,
                    const PagedKV*, hipStream_t) {
  std::fprintf(stderr, "FAIL: a bf16 launch was reached\n");
  std::abort();
}
int launch_merge(const float*, const float*, int, int64_t, int, void*, float*, hipStream_t) {
  std::fprintf(stderr, "FAIL: a merge launch was reached\n");
  std::abort();
}
int launch_fwd_fp8(const void*, const void*, const void*, const float*, const float*, const float*, const int32_t*,
                   const pva_seg_desc*, float, const OutSpec&, hipStream_t) {
  std::fprintf(stderr, "FAIL: an fp8 launch was reached\n");
  std::abort();
}
int scratch_acquire(int, size_t, void**, uint64_t*, std::string*) {
  std::fprintf(stderr, "FAIL: the no-alloc buffer was reached\n");
  std::abort();
}
bool scratch_is_current(int, uint64_t) { return false; }
// as in the library's own build, which records no workgroup timeline
int timeline_records_bf16(void**) { return PVA_ERR_UNSUPPORTED; }
int timeline_records_fp8(void**) { return PVA_ERR_UNSUPPORTED; }
}  // namespace pva

namespace {

int g_failures = 0;
long g_checks = 0;

void fail(const std::string& what) {
  if (g_failures < 20) std::fprintf(stderr, "FAIL: %s\n", what.c_str());
  ++g_failures;
}

// the message is only formed when the check fails
#define expect(cond, what)      \
  do {                          \
    ++g_checks;                 \
    if (!(cond)) fail(what);    \
  } while (0)

// ---- the range functions at their edges
void check_range_functions() {
  using pva::head_span_bytes;
  using pva::tile_range_bytes;
  for (uint32_t e : {1u, 2u}) {
    for (uint32_t D : {64u, 128u}) {
      const uint32_t row = D * e;
      for (uint32_t H : {1u, 2u, 8u, 32u, 128u}) {
        const uint32_t stride = H * row;
        expect(head_span_bytes(0, stride, row) == 0, "no rows -> empty span");
        expect(head_span_bytes(-5, stride, row) == 0, "negative rows -> empty span");
        expect(head_span_bytes(1, stride, row) == row, "one row -> one row's bytes");
        for (int32_t rows : {31, 32, 33, 63, 64, 65}) {
          const uint64_t want = uint64_t(rows - 1) * stride + row;
          expect(head_span_bytes(rows, stride, row) == want, "tile-edge span");
        }
        // the largest row count the planner accepts: rows * stride < 2^31
        const int32_t rmax = int32_t(((uint64_t(1) << 31) - 1) / stride);
        const uint64_t span = uint64_t(rmax - 1) * stride + row;
        expect(span < (uint64_t(1) << 31), "largest span below 2^31");
        expect(head_span_bytes(rmax, stride, row) == span, "largest span exact");
        const uint32_t s = uint32_t(span);
        expect(tile_range_bytes(s, 0) == s, "first tile sees the whole span");
        expect(tile_range_bytes(s, s - 1) == 1, "last byte");
        expect(tile_range_bytes(s, s) == 0, "offset at the end -> empty");
        expect(tile_range_bytes(s, s + 1) == 0, "offset past the end -> empty");
        expect(tile_range_bytes(s, 0x80000000u) == 0, "offset 2^31 -> empty");
        expect(tile_range_bytes(s, 0xFFFFFFFFu) == 0, "largest offset -> empty");
        expect(tile_range_bytes(0, 0) == 0 && tile_range_bytes(0, 12345) == 0, "empty span -> empty ranges");
      }
    }
  }
}

struct Desc {
  pva_seg_desc* d = nullptr;
  ~Desc() { pva_seg_desc_free(d); }
};

struct Case {
  std::vector<int32_t> seg_len, seg_kind, seg_count, q_start, k_lo, k_hi;
  int32_t nseq = 0, H = 1, D = 128;
  pva_dtype dtype = PVA_BF16;
  bool chunked = false;
};

// Full-sequence key limits of the multi-segment mask (text: i + 1, image
// block [a, b): b), written out from the mask's definition.
std::vector<int32_t> seq_limits(const int32_t* len, const int32_t* kind, int32_t n) {
  std::vector<int32_t> lim;
  int32_t a = 0;
  for (int32_t g = 0; g < n; ++g) {
    for (int32_t i = a; i < a + len[g]; ++i) lim.push_back(kind[g] == PVA_SEG_CAUSAL ? i + 1 : a + len[g]);
    a += len[g];
  }
  return lim;
}

// Checks one planned descriptor: shapes, key limits, tile classes, row
// coverage and every K/V tile load range of every work item.
void check_plan(const Case& c, const pva_seg_desc* d, const std::string& tag) {
  const int32_t *cu, *cuq, *lims, *items;
  int32_t ncu, ncuq, nlim, nitems, bm, bn;
  expect(pva_seg_desc_cu_seqlens(d, &cu, &ncu) == PVA_OK, tag + " cu accessor");
  expect(pva_seg_desc_cu_seqlens_q(d, &cuq, &ncuq) == PVA_OK, tag + " cu_q accessor");
  expect(pva_seg_desc_key_limits(d, &lims, &nlim) == PVA_OK, tag + " limits accessor");
  expect(pva_seg_desc_work_items(d, &items, &nitems) == PVA_OK, tag + " items accessor");
  expect(pva_seg_desc_tile(d, &bm, &bn) == PVA_OK, tag + " tile accessor");
  if (g_failures) return;
  expect(ncu == c.nseq + 1 && ncuq == c.nseq + 1 && cu[0] == 0 && cuq[0] == 0, tag + " offsets shape");
  expect(nlim == cuq[c.nseq], tag + " one key limit per queried row");
  const int64_t esize = c.dtype == PVA_FP8_E4M3 ? 1 : 2;
  const int32_t stages = c.dtype == PVA_FP8_E4M3 ? pva::kFp8Stages : pva::kBf16Stages;
  const int64_t nk = cu[c.nseq], nq = cuq[c.nseq];
  const int64_t hd = int64_t(c.H) * c.D;
  const int64_t k_bytes = nk * hd * esize;  // bytes of the K (and of the V) tensor

  // expected key limits per queried row, from the mask definition
  int64_t g0 = 0, pairs = 0;
  std::vector<int32_t> seq_of_q(size_t(nq), -1);
  for (int32_t s = 0; s < c.nseq; ++s) {
    const int32_t n = c.seg_count[s];
    const std::vector<int32_t> full = seq_limits(&c.seg_len[g0], &c.seg_kind[g0], n);
    g0 += n;
    const int32_t L = int32_t(full.size());
    const int32_t qs = c.q_start.empty() ? 0 : c.q_start[s];
    const int32_t lo = c.chunked ? c.k_lo[s] : 0, hi = c.chunked ? c.k_hi[s] : L;
    expect(cu[s + 1] - cu[s] == hi - lo, tag + " cu_seqlens counts the key rows held");
    expect(cuq[s + 1] - cuq[s] == L - qs, tag + " cu_seqlens_q counts the queried rows");
    for (int32_t i = qs; i < L; ++i) {
      const int32_t want = std::min(std::max(full[i] - lo, 0), hi - lo);
      const int64_t r = cuq[s] + (i - qs);
      expect(lims[r] == want, tag + " key limit of row " + std::to_string(i) + " of sequence " + std::to_string(s));
      if (i > qs) expect(lims[r] >= lims[r - 1], tag + " limits never decrease");
      seq_of_q[size_t(r)] = s;
      pairs += want;
    }
  }
  expect(pva_seg_desc_useful_flops(d) == 4 * int64_t(c.D) * c.H * pairs, tag + " useful flops");

  // work items: coverage, tile classes, every memory range the kernels touch
  std::vector<uint8_t> covered(size_t(nq * c.H), 0);
  const uint32_t rs_bytes = uint32_t(hd * esize);
  for (int32_t n = 0; n < nitems; ++n) {
    const pva::WorkItem w = reinterpret_cast<const pva::WorkItem*>(items)[n];
    if (w.seq < 0) continue;
    const std::string it = tag + " item " + std::to_string(n);
    expect(w.seq < c.nseq && w.head >= 0 && w.head < c.H, it + " seq/head in range");
    if (w.seq >= c.nseq || w.head < 0 || w.head >= c.H) continue;
    const int32_t qs = c.q_start.empty() ? 0 : c.q_start[w.seq];
    const int32_t Lk = cu[w.seq + 1] - cu[w.seq];
    expect(w.seq_len == Lk, it + " holds the sequence's key rows");
    expect(w.q_rows >= 1 && w.q_rows <= bm, it + " rows per item");
    expect(w.qo_row == cuq[w.seq] + (w.q0 - qs), it + " Q/O row of the first query");
    expect(w.qo_row >= cuq[w.seq] && int64_t(w.qo_row) + w.q_rows <= cuq[w.seq + 1], it + " rows inside the sequence");
    if (w.qo_row < 0 || int64_t(w.qo_row) + w.q_rows > nq) continue;
    for (int32_t r = 0; r < w.q_rows; ++r) {
      uint8_t& cov = covered[size_t((int64_t(w.qo_row) + r) * c.H + w.head)];
      expect(cov == 0, it + " row covered once");
      cov = 1;
    }
    const int32_t lim_first = lims[w.qo_row], lim_last = lims[w.qo_row + w.q_rows - 1];
    expect(0 <= w.k_full_end && w.k_full_end <= w.k_end, it + " tile classes ordered");
    expect(int64_t(w.k_full_end) * bn <= lim_first, it + " FULL tiles need no mask");
    expect(int64_t(w.k_end) * bn >= lim_last && int64_t(w.k_end - 1) * bn < std::max(lim_last, 1),
           it + " SKIP starts at the last row's limit");
    // K/V tile loads: K tiles [0, k_end + stages), V tiles [0, k_end + stages - 1),
    // each from byte t * BN * row stride of the head's span, as the kernels form it
    const int64_t base = (int64_t(cu[w.seq]) * hd + int64_t(w.head) * c.D) * esize;
    const uint32_t span = pva::head_span_bytes(w.seq_len, rs_bytes, uint32_t(c.D * esize));
    expect(Lk > 0 || span == 0, it + " an empty chunk has an empty span");
    if (span > 0) expect(base >= 0 && base + int64_t(span) <= k_bytes, it + " span inside the K/V tensor");
    for (int32_t t = 0; t < w.k_end + stages; ++t) {
      const uint32_t o = uint32_t(t * bn) * rs_bytes;
      const uint32_t range = pva::tile_range_bytes(span, o);
      if (range == 0) continue;
      expect(int64_t(o) + range <= int64_t(span), it + " tile range inside the span");
      expect(base + int64_t(o) >= 0 && base + int64_t(o) + range <= k_bytes,
             it + " tile " + std::to_string(t) + " load inside the K/V tensor");
    }
  }
  for (size_t i = 0; i < covered.size(); ++i)
    if (!covered[i]) {
      expect(false, tag + " queried (row, head) " + std::to_string(i) + " not covered");
      break;
    }
}

void random_cases(uint64_t seed, int n_cases) {
  std::mt19937_64 rng(seed);
  auto uni = [&](int64_t a, int64_t b) { return int64_t(std::uniform_int_distribution<int64_t>(a, b)(rng)); };
  for (int k = 0; k < n_cases; ++k) {
    Case c;
    c.nseq = int32_t(uni(1, 6));
    c.dtype = uni(0, 2) == 0 ? PVA_FP8_E4M3 : PVA_BF16;
    c.D = c.dtype == PVA_FP8_E4M3 ? 128 : (uni(0, 1) ? 64 : 128);
    c.H = int32_t(uni(1, 5));
    c.chunked = uni(0, 1) == 1;
    const bool suffix = uni(0, 2) == 0;
    for (int32_t s = 0; s < c.nseq; ++s) {
      const int32_t n = int32_t(uni(1, 4));
      int32_t L = 0;
      for (int32_t g = 0; g < n; ++g) {
        const int32_t len = uni(0, 3) == 0 ? 0 : int32_t(uni(1, uni(0, 1) ? 70 : 400));
        c.seg_len.push_back(len);
        c.seg_kind.push_back(int32_t(uni(0, 1)));
        L += len;
      }
      if (L == 0) {
        c.seg_len.back() = 1;
        L = 1;
      }
      c.seg_count.push_back(n);
      c.q_start.push_back(suffix ? int32_t(uni(0, L)) : 0);
      int32_t lo = int32_t(uni(0, L)), hi = int32_t(uni(0, L));
      if (lo > hi) std::swap(lo, hi);
      if (uni(0, 3) == 0) hi = lo;                      // empty chunk
      if (s == c.nseq - 1 && uni(0, 1)) lo = hi = L;    // empty chunk at the very end of K/V
      c.k_lo.push_back(lo);
      c.k_hi.push_back(hi);
    }
    Desc d;
    int st;
    if (c.chunked)
      st = pva_seg_desc_build_kv_chunk_host(c.seg_len.data(), c.seg_kind.data(), c.seg_count.data(), c.q_start.data(),
                                            c.k_lo.data(), c.k_hi.data(), c.nseq, c.H, c.D, c.dtype, &d.d);
    else
      st = pva_seg_desc_build_segments_host(c.seg_len.data(), c.seg_kind.data(), c.seg_count.data(),
                                            c.q_start.data(), c.nseq, c.H, c.D, c.dtype, &d.d);
    const std::string tag = "case " + std::to_string(seed) + "/" + std::to_string(k);
    expect(st == PVA_OK, tag + " builds: " + pva_last_error());
    if (st == PVA_OK) check_plan(c, d.d, tag);
  }
}

// Two-segment builder at the pages' shapes and at the 2^31 head-span limit.
void two_segment_cases() {
  struct TS { std::vector<int32_t> t, i; int32_t H, D; pva_dtype dt; };
  const std::vector<TS> cases = {
      {{16, 16}, {48, 48}, 2, 64, PVA_BF16},
      {{128, 128}, {4096, 4096}, 32, 128, PVA_BF16},
      {{445, 445, 349, 349, 293, 293, 185, 185}, {1024, 1024, 2304, 2304, 4096, 4096, 3840, 3840}, 32, 128, PVA_BF16},
      {{445, 445, 349, 349, 293, 293, 185, 185}, {1024, 1024, 2304, 2304, 4096, 4096, 3840, 3840}, 32, 128,
       PVA_FP8_E4M3},
      {{256, 256}, {16384, 16384}, 8, 128, PVA_BF16},
      {{0, 1, 5}, {1, 0, 0}, 3, 64, PVA_BF16},
      {{1000}, {65535 - 1000}, 128, 128, PVA_BF16},     // largest bf16 head slice at H = D = 128
      {{1000}, {131071 - 1000}, 128, 128, PVA_FP8_E4M3},  // largest fp8 head slice
  };
  int n = 0;
  for (const TS& c : cases) {
    Desc d;
    const int32_t nseq = int32_t(c.t.size());
    const int st = pva_seg_desc_build_host(c.t.data(), c.i.data(), nseq, c.H, c.D, c.dt, &d.d);
    expect(st == PVA_OK, "two-segment case " + std::to_string(n) + " builds");
    if (st == PVA_OK) {
      Case cc;
      cc.nseq = nseq;
      cc.H = c.H;
      cc.D = c.D;
      cc.dtype = c.dt;
      for (int32_t s = 0; s < nseq; ++s) {
        cc.seg_len.push_back(c.t[s]);
        cc.seg_len.push_back(c.i[s]);
        cc.seg_kind.push_back(PVA_SEG_CAUSAL);
        cc.seg_kind.push_back(PVA_SEG_FULL);
        cc.seg_count.push_back(2);
      }
      check_plan(cc, d.d, "two-segment case " + std::to_string(n));
    }
    ++n;
  }
  // one token past the largest slice is refused, not wrapped
  const int32_t t = 1000, i = 65536 - 1000;
  pva_seg_desc* d = nullptr;
  expect(pva_seg_desc_build_host(&t, &i, 1, 128, 128, PVA_BF16, &d) == PVA_ERR_UNSUPPORTED && d == nullptr,
         "L * H * D * 2 = 2^31 refused");
  const int32_t i8 = 131072 - 1000;
  expect(pva_seg_desc_build_host(&t, &i8, 1, 128, 128, PVA_FP8_E4M3, &d) == PVA_ERR_UNSUPPORTED && d == nullptr,
         "L * H * D = 2^31 (fp8) refused");
}

// Invalid arguments come back as status codes; nothing is read out of bounds.
void reject_cases() {
  pva_seg_desc* d = nullptr;
  const int32_t t1[] = {4}, i1[] = {8}, neg[] = {-1}, big[] = {INT32_MAX}, one[] = {1};
  expect(pva_seg_desc_build_host(t1, i1, 0, 2, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "nseq 0");
  expect(pva_seg_desc_build_host(neg, i1, 1, 2, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "negative text");
  expect(pva_seg_desc_build_host(big, one, 1, 1, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "T + I > int32");
  expect(pva_seg_desc_build_host(t1, i1, 1, 0, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "no heads");
  expect(pva_seg_desc_build_host(t1, i1, 1, 2, 96, PVA_BF16, &d) == PVA_ERR_UNSUPPORTED, "D 96");
  expect(pva_seg_desc_build_host(t1, i1, 1, 2, 64, PVA_FP8_E4M3, &d) == PVA_ERR_UNSUPPORTED, "fp8 D 64");
  expect(pva_seg_desc_build_host(nullptr, i1, 1, 2, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "NULL text_len");
  expect(pva_seg_desc_build_host(t1, i1, 1, 2, 64, PVA_BF16, nullptr) == PVA_ERR_INVALID_ARG, "NULL out");
  const int32_t zero[] = {0};
  expect(pva_seg_desc_build_host(zero, zero, 1, 2, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG, "empty sequence");
  // two sequences whose total overflows int32
  const int32_t tt[] = {INT32_MAX / 2 + 1, INT32_MAX / 2 + 1}, ii[] = {0, 0};
  expect(pva_seg_desc_build_host(tt, ii, 2, 1, 64, PVA_BF16, &d) != PVA_OK, "packed total > int32");
  // segment builder
  const int32_t sl[] = {5, 7}, sk[] = {PVA_SEG_CAUSAL, PVA_SEG_FULL}, sc[] = {2}, badk[] = {0, 2};
  const int32_t qs_bad[] = {13}, lo_bad[] = {6}, hi_bad[] = {5}, hi_over[] = {13}, lo_neg[] = {-1};
  expect(pva_seg_desc_build_segments_host(sl, badk, sc, nullptr, 1, 1, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG,
         "segment kind 2");
  const int32_t sc0[] = {0};
  expect(pva_seg_desc_build_segments_host(sl, sk, sc0, nullptr, 1, 1, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG,
         "no segments");
  expect(pva_seg_desc_build_segments_host(sl, sk, sc, qs_bad, 1, 1, 64, PVA_BF16, &d) == PVA_ERR_INVALID_ARG,
         "q_start past L");
  expect(pva_seg_desc_build_kv_chunk_host(sl, sk, sc, nullptr, lo_bad, hi_bad, 1, 1, 64, PVA_BF16, &d) ==
             PVA_ERR_INVALID_ARG, "k_lo > k_hi");
  expect(pva_seg_desc_build_kv_chunk_host(sl, sk, sc, nullptr, one, hi_over, 1, 1, 64, PVA_BF16, &d) ==
             PVA_ERR_INVALID_ARG, "k_hi past L");
  expect(pva_seg_desc_build_kv_chunk_host(sl, sk, sc, nullptr, lo_neg, one, 1, 1, 64, PVA_BF16, &d) ==
             PVA_ERR_INVALID_ARG, "negative k_lo");
  expect(pva_seg_desc_build_kv_chunk_host(sl, sk, sc, nullptr, nullptr, one, 1, 1, 64, PVA_BF16, &d) ==
             PVA_ERR_INVALID_ARG, "k_lo NULL");
  expect(d == nullptr, "no descriptor on failure");

  // forward and merge entry points refuse on the host, before any device work
  Desc h;
  expect(pva_seg_desc_build_host(t1, i1, 1, 2, 64, PVA_BF16, &h.d) == PVA_OK, "host descriptor");
  alignas(16) static char buf[256];
  const int32_t* cu = reinterpret_cast<const int32_t*>(buf);
  expect(packed_attn_fwd(buf, buf, buf, cu, h.d, 0.125f, buf, nullptr) == PVA_ERR_INVALID_ARG,
         "host-only descriptor cannot be launched");
  expect(packed_attn_fwd(buf, buf, buf, cu, nullptr, 0.125f, buf, nullptr) == PVA_ERR_INVALID_ARG, "NULL desc");
  expect(packed_attn_fwd(buf + 2, buf, buf, cu, h.d, 0.125f, buf, nullptr) == PVA_ERR_INVALID_ARG, "misaligned q");
  expect(packed_attn_fwd(buf, buf, buf, cu, h.d, -1.0f, buf, nullptr) == PVA_ERR_INVALID_ARG, "negative scale");
  expect(packed_attn_fwd_fp8(buf, buf, buf, nullptr, nullptr, nullptr, cu, h.d, 0.1f, buf, nullptr) ==
             PVA_ERR_INVALID_ARG, "fp8 on a bf16 descriptor");
  expect(packed_attn_fwd_partial(buf, buf, buf, cu, cu, h.d, 0.1f, reinterpret_cast<float*>(buf), nullptr,
                                 nullptr) == PVA_ERR_INVALID_ARG, "partial without lse");
  float* fb = reinterpret_cast<float*>(buf);
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, nullptr, fb, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "accumulate without o_acc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, fb, nullptr, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "accumulate without lse_acc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, fb + 1, fb, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "misaligned o_acc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, fb, fb + 4, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "o_acc overlapping lse_acc");
  alignas(16) static float o_run[4096], l_run[64];  // one row set: 12 rows x 2 heads x 64
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, o_run, l_run, o_run + 8, nullptr) ==
             PVA_ERR_INVALID_ARG, "bf16 output overlapping o_acc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, o_run, l_run, l_run, nullptr) ==
             PVA_ERR_INVALID_ARG, "bf16 output overlapping lse_acc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, nullptr, 0.1f, fb, fb, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "accumulate NULL desc");
  expect(packed_attn_fwd_partial_accumulate(buf, buf, buf, cu, cu, h.d, 0.1f, o_run, l_run, nullptr, nullptr) ==
             PVA_ERR_INVALID_ARG, "accumulate on a host-only descriptor");
  expect(packed_attn_fwd_partial_accumulate_fp8(buf, buf, buf, fb, fb, fb, cu, cu, h.d, 0.1f, o_run, l_run, nullptr,
                                                nullptr) == PVA_ERR_INVALID_ARG, "fp8 accumulate on a bf16 descriptor");
  expect(pva_merge_partials(nullptr, nullptr, 1, 4, 64, buf, nullptr, nullptr) == PVA_ERR_INVALID_ARG, "merge NULL");
  expect(pva_merge_partials(reinterpret_cast<float*>(buf), reinterpret_cast<float*>(buf), 0, 4, 64, buf, nullptr,
                            nullptr) == PVA_ERR_INVALID_ARG, "merge no parts");
  expect(pva_merge_partials(reinterpret_cast<float*>(buf), reinterpret_cast<float*>(buf), 2, 4, 96, buf, nullptr,
                            nullptr) == PVA_ERR_UNSUPPORTED, "merge D 96");
  expect(pva_merge_partials(reinterpret_cast<float*>(buf), reinterpret_cast<float*>(buf), 2, int64_t(1) << 40, 64,
                            buf, nullptr, nullptr) == PVA_ERR_INVALID_ARG, "merge too large");
  expect(std::string(pva_last_error()).size() > 0, "an error message is set");
}

}  // namespace

// The workgroup-timeline calls validate their arguments before touching a
// device, and the library's own build refuses them.
void timeline_cases() {
  uint64_t buf[PVA_TIMELINE_FIELDS * 2] = {};
  expect(pva_timeline_clear(static_cast<pva_dtype>(7)) == PVA_ERR_INVALID_ARG, "timeline: unknown kernel");
  expect(pva_timeline_read(PVA_BF16, nullptr, 2) == PVA_ERR_INVALID_ARG, "timeline: NULL records");
  expect(pva_timeline_read(PVA_BF16, buf, -1) == PVA_ERR_INVALID_ARG, "timeline: negative count");
  expect(pva_timeline_read(PVA_FP8_E4M3, buf, int64_t(PVA_TIMELINE_MAX_ITEMS) + 1) == PVA_ERR_INVALID_ARG,
         "timeline: count past the buffer");
  expect(pva_timeline_clear(PVA_BF16) == PVA_ERR_UNSUPPORTED, "timeline: library build refuses clear");
  expect(pva_timeline_read(PVA_FP8_E4M3, buf, 2) == PVA_ERR_UNSUPPORTED, "timeline: library build refuses read");
}

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? std::atoi(argv[1]) : 400;
  check_range_functions();
  two_segment_cases();
  reject_cases();
  timeline_cases();
  for (uint64_t seed = 1; seed <= 4; ++seed) random_cases(seed, n_cases / 4);
  std::printf("host checks: %ld checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
