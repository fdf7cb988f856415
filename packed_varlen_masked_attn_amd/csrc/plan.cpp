// Segment-descriptor builder and varlen tile scheduler (host C++).
//
// The mask is the Generalized Causal Attention of "[RFC]: HunyuanImage 3.0
// deployment" (Proposed Change P0, attention mask challenge; Model structure,
// item 1): a sequence is a list of segments; a token of a text (causal)
// segment sees every key up to itself, a token of an image (full) block sees
// every key up to the end of its block. Its key limit lim(i) never decreases
// along i, so every row's allowed keys are a prefix [0, lim(i)) and a query
// tile [qa, qb) needs:
//   key tiles below floor(lim(qa) / BN)        : FULL (no mask at all)
//   key tiles from ceil(lim(qb - 1) / BN) on    : SKIP (never loaded)
//   key tiles in between                        : PARTIAL (element mask)
// which is the block-sparse form the RFC names, and also its split into
// causal and full segments, with no partial-result merge needed. The
// two-segment case (text prefix, one image block) is the RFC's packed batch.
//
// Queries may cover only a suffix [q_start, L) of a sequence (the prefix's
// keys and values are reused; Model structure item 1, the single Prefix KV):
// query tiles then start at q_start and Q / O hold only the queried rows.
//
// K / V may hold only a chunk [k_lo, k_hi) of each sequence's keys (one
// rank's share in Ring attention, Proposed Change P2): each queried row's
// key limit is then taken relative to the chunk and clamped to [0, chunk
// length]; a row whose limit is 0 has no key in the chunk.

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

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

struct Group {  // all query tiles of one (sequence, head)
  int32_t seq, head;
  int64_t cost;
  std::vector<WorkItem> items;
};

struct SeqSpec {
  std::vector<int32_t> seg_len, seg_kind;
  int32_t q_start = 0;
  int32_t k_lo = 0, k_hi = -1;  // key rows held by K/V; k_hi < 0: to the end
};

int check_shape(int32_t nseq, int32_t num_heads, int32_t head_dim, pva_dtype dtype, std::string* err) {
  if (nseq < 1) return fail(err, PVA_ERR_INVALID_ARG, "nseq must be >= 1");
  if (num_heads < 1) return fail(err, PVA_ERR_INVALID_ARG, "num_heads must be >= 1");
  if (dtype != PVA_BF16 && dtype != PVA_FP8_E4M3) return fail(err, PVA_ERR_INVALID_ARG, "unknown dtype");
  if (head_dim != 64 && head_dim != 128) return fail(err, PVA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dtype == PVA_FP8_E4M3 && head_dim != 128)
    return fail(err, PVA_ERR_UNSUPPORTED, "the fp8 path supports head_dim 128 only");
  return PVA_OK;
}

// Plans validated sequence specs (segment kinds and lengths checked by the callers).
int plan_sequences(const std::vector<SeqSpec>& seqs, int32_t num_heads, int32_t head_dim, pva_dtype dtype,
                   Plan* plan, std::string* err) {
  const int32_t nseq = static_cast<int32_t>(seqs.size());
  Plan p;
  p.dtype = dtype;
  p.nseq = nseq;
  p.num_heads = num_heads;
  p.head_dim = head_dim;
  p.tile = tile_shape(dtype, head_dim);
  const int64_t esize = dtype == PVA_FP8_E4M3 ? 1 : 2;  // bytes per Q/K/V element
  p.seq_len.resize(nseq);
  p.q_start.resize(nseq);
  p.k_lo.resize(nseq);
  p.kv_len.resize(nseq);
  p.cu_seqlens.assign(nseq + 1, 0);
  p.cu_seqlens_q.assign(nseq + 1, 0);
  int64_t total = 0, total_q = 0, pairs = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    int64_t L = 0;
    for (int32_t n : seqs[s].seg_len) L += n;
    if (L < 1) return fail(err, PVA_ERR_INVALID_ARG, "every sequence needs at least one token");
    if (L > INT32_MAX) return fail(err, PVA_ERR_INVALID_ARG, "sequence too long");
    const int32_t qs = seqs[s].q_start;
    if (qs < 0 || qs > L) return fail(err, PVA_ERR_INVALID_ARG, "q_start must lie in [0, L]");
    const int64_t lo = seqs[s].k_lo, hi = seqs[s].k_hi < 0 ? L : seqs[s].k_hi;
    if (lo < 0 || lo > hi || hi > L) return fail(err, PVA_ERR_INVALID_ARG, "key chunk must satisfy 0 <= k_lo <= k_hi <= L");
    const int64_t Lk = hi - lo;
    // the kernels address one head's rows of a sequence with 32-bit byte
    // offsets below 2^31 (row stride H * D elements of `esize` bytes)
    if (Lk * int64_t(num_heads) * head_dim * esize >= (int64_t(1) << 31))
      return fail(err, PVA_ERR_UNSUPPORTED,
                  "sequence too long for 32-bit head addressing (L * H * D * element bytes >= 2^31)");
    total += Lk;
    total_q += L - qs;
    if (total > INT32_MAX || total_q > INT32_MAX)
      return fail(err, PVA_ERR_INVALID_ARG, "packed token count exceeds int32");
    p.seq_len[s] = static_cast<int32_t>(L);
    p.q_start[s] = qs;
    p.k_lo[s] = static_cast<int32_t>(lo);
    p.kv_len[s] = static_cast<int32_t>(Lk);
    p.cu_seqlens[s + 1] = static_cast<int32_t>(total);
    p.cu_seqlens_q[s + 1] = static_cast<int32_t>(total_q);
  }
  // element offsets are formed as (token * H + h) * D in int64 on the device
  if (std::max(total, total_q) * int64_t(num_heads) * head_dim > (int64_t(1) << 62))
    return fail(err, PVA_ERR_INVALID_ARG, "tensor too large");
  p.total_tokens = total;
  p.total_q = total_q;

  // ---- key limits of the queried rows, in the coordinates of the K/V rows
  // held: lim(i) = i + 1 in a text segment, the block's end in an image
  // block, then shifted by k_lo and clamped to [0, kv_len]
  p.key_lim.resize(static_cast<size_t>(total_q));
  std::vector<int32_t> lim;
  for (int32_t s = 0; s < nseq; ++s) {
    lim.assign(p.seq_len[s], 0);
    int32_t a = 0;
    for (size_t g = 0; g < seqs[s].seg_len.size(); ++g) {
      const int32_t b = a + seqs[s].seg_len[g];
      for (int32_t i = a; i < b; ++i) lim[i] = seqs[s].seg_kind[g] == PVA_SEG_CAUSAL ? i + 1 : b;
      a = b;
    }
    int32_t* out = p.key_lim.data() + p.cu_seqlens_q[s];
    for (int32_t i = p.q_start[s]; i < p.seq_len[s]; ++i) {
      const int32_t c = std::min(std::max(lim[i] - p.k_lo[s], 0), p.kv_len[s]);
      out[i - p.q_start[s]] = c;
      pairs += c;
    }
  }
  p.useful_flops = 4 * int64_t(head_dim) * num_heads * pairs;

  // ---- segment descriptors: per (sequence, query tile) tile classes
  const int32_t BM = p.tile.bm, BN = p.tile.bn;
  std::vector<std::vector<WorkItem>> seq_tiles(nseq);
  for (int32_t s = 0; s < nseq; ++s) {
    const int32_t L = p.seq_len[s], qs = p.q_start[s];
    // key limit of row `row` of the sequence (a queried row, row >= qs)
    auto qlim = [&](int32_t row) { return p.key_lim[size_t(p.cu_seqlens_q[s]) + size_t(row - qs)]; };
    for (int32_t qa = qs; qa < L; qa += BM) {
      const int32_t qb = std::min(qa + BM, L);
      WorkItem w;
      w.seq = s;
      w.head = 0;
      w.q0 = qa;
      w.q_rows = qb - qa;
      w.k_full_end = qlim(qa) / BN;
      w.k_end = (qlim(qb - 1) + BN - 1) / BN;
      w.qo_row = p.cu_seqlens_q[s] + (qa - qs);
      w.seq_len = p.kv_len[s];
      seq_tiles[s].push_back(w);
    }
  }

  // ---- varlen tile scheduler
  // Cost of an item ~ key tiles it streams, plus a fixed per-item overhead.
  auto item_cost = [](const WorkItem& w) { return int64_t(w.k_end) * 4 + 3; };
  std::vector<Group> groups;
  groups.reserve(size_t(nseq) * num_heads);
  for (int32_t s = 0; s < nseq; ++s) {
    if (seq_tiles[s].empty()) continue;
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
  // Each XCD's queue runs longest item first. The dispatcher hands out
  // workgroups in index order, round-robin over the XCDs, and waits when the
  // next one's XCD has no free slot; with the queues in cost order the items
  // at one position finish at about the same time on every XCD, which keeps
  // those waits short (stable: a group's items stay together).
  for (auto& b : bins)
    std::stable_sort(b.begin(), b.end(), [&](const WorkItem& u, const WorkItem& v) { return item_cost(u) > item_cost(v); });
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

}  // namespace

int build_plan(const int32_t* text_len, const int32_t* image_len, int32_t nseq, int32_t num_heads,
               int32_t head_dim, pva_dtype dtype, Plan* plan, std::string* err) {
  if (!plan) return fail(err, PVA_ERR_INVALID_ARG, "plan output is NULL");
  if (!text_len || !image_len) return fail(err, PVA_ERR_INVALID_ARG, "text_len/image_len is NULL");
  int st = check_shape(nseq, num_heads, head_dim, dtype, err);
  if (st != PVA_OK) return st;
  std::vector<SeqSpec> seqs(nseq);
  for (int32_t s = 0; s < nseq; ++s) {
    if (text_len[s] < 0 || image_len[s] < 0)
      return fail(err, PVA_ERR_INVALID_ARG, "text_len and image_len must be >= 0");
    if (int64_t(text_len[s]) + image_len[s] > INT32_MAX) return fail(err, PVA_ERR_INVALID_ARG, "sequence too long");
    seqs[s].seg_len = {text_len[s], image_len[s]};
    seqs[s].seg_kind = {PVA_SEG_CAUSAL, PVA_SEG_FULL};
  }
  st = plan_sequences(seqs, num_heads, head_dim, dtype, plan, err);
  if (st != PVA_OK) return st;
  plan->text_len.assign(text_len, text_len + nseq);
  plan->image_len.assign(image_len, image_len + nseq);
  return PVA_OK;
}

int build_plan_segments(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                        const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi, int32_t nseq,
                        int32_t num_heads, int32_t head_dim, pva_dtype dtype, Plan* plan, std::string* err) {
  if (!plan) return fail(err, PVA_ERR_INVALID_ARG, "plan output is NULL");
  if (!seg_len || !seg_kind || !seg_count) return fail(err, PVA_ERR_INVALID_ARG, "a segment array is NULL");
  int st = check_shape(nseq, num_heads, head_dim, dtype, err);
  if (st != PVA_OK) return st;
  std::vector<SeqSpec> seqs(nseq);
  int64_t g = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    if (seg_count[s] < 1) return fail(err, PVA_ERR_INVALID_ARG, "every sequence needs at least one segment");
    int64_t L = 0;
    for (int32_t k = 0; k < seg_count[s]; ++k, ++g) {
      if (seg_len[g] < 0) return fail(err, PVA_ERR_INVALID_ARG, "segment lengths must be >= 0");
      if (seg_kind[g] != PVA_SEG_CAUSAL && seg_kind[g] != PVA_SEG_FULL)
        return fail(err, PVA_ERR_INVALID_ARG, "segment kind must be PVA_SEG_CAUSAL or PVA_SEG_FULL");
      L += seg_len[g];
      if (L > INT32_MAX) return fail(err, PVA_ERR_INVALID_ARG, "sequence too long");
      seqs[s].seg_len.push_back(seg_len[g]);
      seqs[s].seg_kind.push_back(seg_kind[g]);
    }
    seqs[s].q_start = q_start ? q_start[s] : 0;
    if ((k_lo == nullptr) != (k_hi == nullptr))
      return fail(err, PVA_ERR_INVALID_ARG, "k_lo and k_hi must both be given or both be NULL");
    if (k_lo) {
      if (k_hi[s] < 0) return fail(err, PVA_ERR_INVALID_ARG, "key chunk must satisfy 0 <= k_lo <= k_hi <= L");
      seqs[s].k_lo = k_lo[s];
      seqs[s].k_hi = k_hi[s];
    }
  }
  return plan_sequences(seqs, num_heads, head_dim, dtype, plan, err);
}

}  // namespace pva
