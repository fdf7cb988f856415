// Segment-descriptor builder and varlen tile scheduler (host C++).
//
// The mask is the Generalized Causal Attention of "[RFC]: HunyuanImage 3.0
// deployment" (Proposed Change P0, attention mask challenge; Model structure,
// item 1): text rows causal over the text prefix, image rows see their whole
// sequence. Its key limit lim(i) never decreases along i, so every row's
// allowed keys are a prefix [0, lim(i)) and a query tile [qa, qb) needs:
//   key tiles below floor(lim(qa) / BN)        : FULL (no mask at all)
//   key tiles from ceil(lim(qb - 1) / BN) on    : SKIP (never loaded)
//   key tiles in between                        : PARTIAL (element mask)
// which is the block-sparse form the RFC names, and also its split into
// causal and full segments, with no partial-result merge needed.

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <numeric>

#include "pva_internal.h"

namespace pva {

TileShape tile_shape(pva_dtype dtype, int32_t head_dim) {
  (void)head_dim;
  if (dtype == PVA_FP8_E4M3) return TileShape{128, 64};
  return TileShape{kBf16BlockM, kBf16BlockN};
}

namespace {

int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}

struct Group {  // all query tiles of one (sequence, head)
  int32_t seq, head;
  int64_t cost;
  std::vector<WorkItem> items;
};

}  // namespace

int build_plan(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
               int32_t head_dim, pva_dtype dtype, Plan* plan, std::string* err) {
  if (!plan) return fail(err, PVA_ERR_INVALID_ARG, "plan output is NULL");
  if (!text_len || !image_len) return fail(err, PVA_ERR_INVALID_ARG, "text_len/image_len is NULL");
  if (nseq < 1) return fail(err, PVA_ERR_INVALID_ARG, "nseq must be >= 1");
  if (num_heads < 1) return fail(err, PVA_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (dtype != PVA_BF16 && dtype != PVA_FP8_E4M3) return fail(err, PVA_ERR_INVALID_ARG, "unknown dtype");
  if (head_dim != 64 && head_dim != 128) return fail(err, PVA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype == PVA_FP8_E4M3 && head_dim != 128)
    return fail(err, PVA_ERR_UNSUPPORTED, "the fp8 path supports head_dim 128 only");

  Plan p;
  p.dtype = dtype;
  p.nseq = nseq;
  p.num_heads = num_heads;
  p.head_dim = head_dim;
  p.tile = tile_shape(dtype, head_dim);
  p.text_len.assign(text_len, text_len + nseq);
  p.image_len.assign(image_len, image_len + nseq);
  p.seq_len.resize(nseq);
  p.cu_seqlens.resize(nseq + 1);
  int64_t total = 0, pairs = 0;
  p.cu_seqlens[0] = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t T = text_len[s], I = image_len[s];
    if (T < 0 || I < 0) return fail(err, PVA_ERR_INVALID_ARG, "text_len and image_len must be >= 0");
    if (T + I < 1) return fail(err, PVA_ERR_INVALID_ARG, "every sequence needs at least one token");
    if (T + I > INT32_MAX) return fail(err, PVA_ERR_INVALID_ARG, "sequence too long");
    // the kernels address one head's rows of a sequence with 32-bit byte
    // offsets below 2^31 (row stride H * D elements of at most 2 bytes)
    if ((T + I) * int64_t(num_heads) * head_dim * 2 >= (int64_t(1) << 31))
      return fail(err, PVA_ERR_UNSUPPORTED, "sequence too long for 32-bit head addressing (L * H * D * 2 >= 2^31)");
    total += T + I;
    if (total > INT32_MAX) return fail(err, PVA_ERR_INVALID_ARG, "packed token count exceeds int32");
    p.seq_len[s] = static_cast<int32_t>(T + I);
    p.cu_seqlens[s + 1] = static_cast<int32_t>(total);
    pairs += T * (T + 1) / 2 + I * (T + I);
  }
  // element offsets are formed as (token * H + h) * D in int64 on the device
  if (total * int64_t(num_heads) * head_dim > (int64_t(1) << 62))
    return fail(err, PVA_ERR_INVALID_ARG, "tensor too large");
  p.total_tokens = total;
  p.useful_flops = 4 * int64_t(head_dim) * num_heads * pairs;

  // ---- segment descriptors: per (sequence, query tile) tile classes
  const int32_t BM = p.tile.bm, BN = p.tile.bn;
  std::vector<std::vector<WorkItem>> seq_tiles(nseq);
  for (int32_t s = 0; s < nseq; ++s) {
    const int32_t T = p.text_len[s], L = p.seq_len[s];
    for (int32_t qa = 0; qa < L; qa += BM) {
      const int32_t qb = std::min(qa + BM, L);
      const int32_t lim_a = key_limit(qa, T, L), lim_b = key_limit(qb - 1, T, L);
      WorkItem w;
      w.seq = s;
      w.head = 0;
      w.q0 = qa;
      w.q_rows = qb - qa;
      w.k_full_end = lim_a / BN;
      w.k_end = (lim_b + BN - 1) / BN;
      w.text_len = T;
      w.seq_len = L;
      seq_tiles[s].push_back(w);
    }
  }

  // ---- varlen tile scheduler
  // Cost of an item ~ key tiles it streams, plus a fixed per-item overhead.
  auto item_cost = [](const WorkItem& w) { return int64_t(w.k_end) * 4 + 3; };
  std::vector<Group> groups;
  groups.reserve(size_t(nseq) * num_heads);
  for (int32_t s = 0; s < nseq; ++s) {
    for (int32_t h = 0; h < num_heads; ++h) {
      Group g{s, h, 0, seq_tiles[s]};
      for (auto& w : g.items) {
        w.head = h;
        g.cost += item_cost(w);
      }
      // within a group: most expensive tiles first (LPT)
      std::stable_sort(g.items.begin(), g.items.end(),
                       [&](const WorkItem& a, const WorkItem& b) { return item_cost(a) > item_cost(b); });
      groups.push_back(std::move(g));
    }
  }
  // Groups of one (sequence, head) share K/V, so all their tiles go to one XCD
  // (one L2). Groups are placed on XCDs longest-first onto the least-loaded XCD.
  std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& b) { return a.cost > b.cost; });
  std::vector<int64_t> load(kNumXcd, 0);
  std::vector<std::vector<WorkItem>> bins(kNumXcd);
  for (auto& g : groups) {
    int x = int(std::min_element(load.begin(), load.end()) - load.begin());
    load[x] += g.cost;
    bins[x].insert(bins[x].end(), g.items.begin(), g.items.end());
  }
  // Workgroups are dispatched to XCDs round-robin by workgroup index, so slot
  // j of XCD x sits at list position j * kNumXcd + x; shorter bins are padded
  // with empty slots to keep that alignment.
  size_t longest = 0;
  for (auto& b : bins) longest = std::max(longest, b.size());
  p.items.clear();
  p.items.reserve(longest * kNumXcd);
  WorkItem empty{-1, 0, 0, 0, 0, 0, 0, 0};
  for (size_t j = 0; j < longest; ++j)
    for (int x = 0; x < kNumXcd; ++x) p.items.push_back(j < bins[x].size() ? bins[x][j] : empty);
  // trailing empty slots carry no alignment information
  while (!p.items.empty() && p.items.back().seq < 0) p.items.pop_back();

  *plan = std::move(p);
  return PVA_OK;
}

}  // namespace pva
