// FP8 (OCP E4M3FN) packed mixed-mask attention forward for gfx950; bf16 out.
//
// Same operation and mask as the bf16 kernel ("[RFC]: HunyuanImage 3.0
// deployment", Proposed Change P0 and Model structure item 1). Q, K and V are
// E4M3 codes with one fp32 dequantisation scale per (sequence, head) and
// tensor; QK^T and PV run on the fp8 MFMA (v_mfma_f32_32x32x64_f8f6f4, twice
// the bf16 rate), with fp32 accumulation.
//
// One workgroup = 4 waves = one work item (sequence, head, 128 query rows);
// each wave owns 32 query rows. Keys are streamed in tiles of 64, so that one
// lane's 32 probabilities of a tile form exactly one K=64 MFMA operand.
//
// Per wave and key tile j:
//   S^T[key, q] = K Q^T     two 32-key blocks x two 64-wide steps over d;
//                           A = K from LDS (two 16-byte reads per lane),
//                           B = Q^T in registers for the whole item.
//   softmax in fp32, log2 domain, with the score scale q_s * k_s * scale
//   folded into the exponent; lazy rescaling as in the bf16 kernel, with a
//   lower threshold and the probabilities shifted up by a power of two
//   (kP8Shift below) so that they use E4M3's normal range.
//   P is quantised to E4M3 (round to nearest even) straight from the S^T
//   accumulators into the B operand of PV; probabilities stay <= 2^8.75,
//   inside the format's range.
//   O^T[d, q] += V^T P^T    A = V^T read with ds_read_b64_tr_b8 (8 keys of
//                           one column per read); one 16x16x128 MFMA on the
//                           same P operand (rowsum_fp8 below) accumulates
//                           l = sum of the quantised probabilities, i.e.
//                           exactly the weights PV applied, so every output
//                           row is a convex combination of V rows.
//   a tile in which some row's largest probability may carry a sizeable
//   share of that row's weight (kResidualFactor below) gets a second PV pass
//   with the probabilities' E4M3 residuals.
//   O = O^T * v_s / l at the end.
// The software pipeline (LDS DMA rings, S(j+1) MFMAs beside the exponentials
// of tile j, PV(j) MFMAs beside the row max of tile j+1) is the bf16
// kernel's.
#include <type_traits>

#include "kernel_common.h"

namespace pva {

namespace {

#ifdef PVA_WG_TIMELINE
__device__ unsigned long long g_timeline[uint64_t(PVA_TIMELINE_MAX_ITEMS) * PVA_TIMELINE_FIELDS];
__device__ __forceinline__ unsigned long long* timeline_records() { return g_timeline; }
#else
__device__ __forceinline__ unsigned long long* timeline_records() { return nullptr; }
#endif

typedef int i32x2 __attribute__((ext_vector_type(2)));

// Probabilities are quantised to E4M3 as p = 2^(score - m + kP8Shift), m the
// row's reference max (log2 units), which is raised whenever a tile's max
// exceeds it by more than kP8Lazy. So p stays at or below 2^8.75 < 448
// (E4M3's largest finite value), and a row's largest p is at least
// 2^kP8Shift: keys up to 11 log2 units below the row max keep E4M3's normal
// range (2^-6 and up, 2^-4 relative rounding) instead of 6 with p_max = 1;
// below it the spacing is a fixed 2^-9, a large relative error on
// probabilities that still carry mass when the scores spread widely (the
// bulk of a long row's weight sits there at softmax scales around 0.2). The
// shift cancels in O / l.
constexpr float kP8Shift = 5.0f;
constexpr float kP8Lazy = 3.75f;
static_assert(kP8Shift + kP8Lazy < 8.807f, "largest probability below 448");

// A tile gets a second PV pass with the E4M3 residuals of its probabilities
// (lo = q(p - q(p)), which carries each weight to about 2^-8 relative
// instead of 2^-4) when, for some row of the wave, the tile's largest
// probability exceeds 1/kResidualFactor of the row's sum of weights so far,
// this tile included. That sum never exceeds the row's final sum, so every
// key whose final weight reaches 1/kResidualFactor is carried at the finer
// precision; a key left at E4M3 precision moves its row's output by less
// than 2^-4 / kResidualFactor times its |v - o|, and such keys' rounding
// errors are independent. Rows whose weight sits on a few keys (peaked
// softmax, early causal text rows) are the ones that trigger it.
constexpr float kResidualFactor = 8.0f;

struct Fp8Cfg {
  static constexpr int D = 128;
  static constexpr int BM = 128, BN = 64, NW = 4, NT = 256;
  static constexpr int NB = BN / 32;   // 32-key blocks per tile
  static constexpr int C = D / 16;     // 16-byte chunks per K/V row
  static constexpr int NKS = D / 64;   // 64-wide MFMA steps over d for S^T
  static constexpr int NDB = D / 32;   // 32-row blocks of O^T (plus one block for l)
  static constexpr int NS = kFp8Stages;  // LDS stages per tensor
  // K and V rows unpadded (C 16-byte chunks each). K's chunks are
  // XOR-permuted per row: the 16-byte operand reads of 16 consecutive rows
  // at one logical chunk then touch 16 different 16-byte bank groups (rows
  // of one parity share 8 groups, which the permutation (r / 2) mod 8
  // spreads). V's 32-byte column pairs are XOR-swizzled for the transpose
  // reads (vswz below).
  static constexpr int KROW = C, KSLOTS = BN * KROW, KTILE = KSLOTS * 16;
  static constexpr int VROW = C, VSLOTS = BN * VROW, VTILE = VSLOTS * 16;
  static_assert(C == 8, "the K permutation is written for 8 chunks per row");
  static __device__ __forceinline__ int kswz(int r) { return (r >> 1) & (C - 1); }
  // every wave issues exactly this many DMA instructions per tile
  static constexpr int DMA_MIN = KSLOTS / NT + VSLOTS / NT;
  static_assert(KSLOTS % NT == 0 && VSLOTS % NT == 0, "uniform DMA rounds");
};

struct KSwizzledChunks {
  static __device__ __forceinline__ int chunk(int row, int pos) { return pos ^ Fp8Cfg::kswz(row); }
};

// Position of a V row's 32-byte column pairs: pair p of row k sits at pair
// p ^ vswz(k). A transpose read touches, for one half-wave, the rows
// {0,1,2,3,8,9,10,11} + 16 r + 4 g of the tile at one pair; with this
// swizzle the same-parity rows among them land on four different pairs, so
// the eight rows fill the 256-byte bank window once.
__device__ __forceinline__ int vswz(int k) { return ((k >> 1) + ((k >> 3) << 1)) & 3; }

struct VSwizzledPairs {
  static __device__ __forceinline__ int chunk(int row, int pos) {
    return 2 * ((pos >> 1) ^ vswz(row)) + (pos & 1);
  }
};

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // E4M3 x E4M3 (format code 0 for both operands), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Row sums of a probability operand on one 16x16x128 E4M3 MFMA (half the
// cycles of a 32x32x64 block). As a 16x16x128 B operand, lane l's 32 bytes
// form column l % 16 for the l / 16-th quarter of the contraction; they are
// the probabilities of query l % 32, so columns c and c + 16 each collect two
// queries' halves. The selector A holds E4M3 1.0 where row r and quarter
// l / 16 agree in parity (bit 2 of r against bit 0 of the quarter), else 0:
// output rows 4 (l / 16) .. +3 of column l % 16, which lane l receives, then
// hold the full sum of query l % 32 in all four of its registers.
__device__ __forceinline__ f32x4 rowsum_fp8(const i32x8& sel, const i32x8& p, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, p, c, 0, 0, 0, 0, 0, 0);
}

struct Fp8Kernel {
  using Cfg = Fp8Cfg;
  static constexpr int BN = Cfg::BN, NB = Cfg::NB, C = Cfg::C, NKS = Cfg::NKS, NDB = Cfg::NDB;
  using KLoader = BufLoader<Cfg::NT, Cfg::KROW, Cfg::KSLOTS, KSwizzledChunks>;
  using VLoader = BufLoader<Cfg::NT, Cfg::VROW, Cfg::VSLOTS, VSwizzledPairs>;

  // K operand of 64-wide step c for key block b: row 32 b + l32, bytes
  // 64 c + 32 g .. +31, i.e. logical chunks 4 c + 2 g and 4 c + 2 g + 1 (any
  // d assignment works as long as Q uses the same). The permutation depends
  // on the row only through (l32 / 2) mod 8, so block b adds an immediate.
  struct KAddr {
    uint32_t o[NKS][2];
    __device__ __forceinline__ void init(int l32, int g) {
      const int sw = Cfg::kswz(l32);
#pragma unroll
      for (int c = 0; c < NKS; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) o[c][h] = uint32_t(16 * C * l32 + 16 * ((4 * c + 2 * g + h) ^ sw));
    }
  };
  static __device__ __forceinline__ i32x8 read_k(const uint8_t* kst, int b, int c, const KAddr& ka) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(kst + 16 * C * 32 * b + ka.o[c][0]);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(kst + 16 * C * 32 * b + ka.o[c][1]);
    return i32x8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // V^T operand of column block db: byte 8 r + e of lane l is
  // V[16 r + 8 (e / 4) + 4 g + e % 4][32 db + l % 32], the same key order as
  // the probability operand: its byte j = 16 b + i holds element (b, i) of
  // the S^T accumulators, key 32 b + 8 (i / 4) + 4 g + i % 4.
  static __device__ __forceinline__ i32x8 read_v(const uint8_t* vst, int db, const int (&vrow0)[1], int vsw,
                                                 int half, int p8) {
    i32x8 a;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint8_t* src = vst + 16 * Cfg::VROW * (16 * r + vrow0[0]) + 32 * (db ^ vsw) + 16 * half + p8;
      const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PVA_LDS i32x2*)(src));
      a[2 * r] = t[0];
      a[2 * r + 1] = t[1];
    }
    return a;
  }

  static __device__ __forceinline__ void mask(f32x16 (&s)[NB], int k0, int g, int mylim) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * b + 8 * (i / 4) + 4 * g + (i % 4);
        if (key >= mylim) s[b][i] = -INFINITY;
      }
  }

  // (IEEE maximum: no canonicalisation of the MFMA results it reads)
  static __device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
  }
  // the row's largest raw score in a tile (shared by both half-waves)
  static __device__ __forceinline__ float tile_max(const f32x16 (&s)[NB]) {
    float mx = max3(s[0][0], s[0][1], s[0][2]);
#pragma unroll
    for (int idx = 3; idx + 1 < NB * 16; idx += 2) mx = max3(mx, s[idx / 16][idx % 16], s[(idx + 1) / 16][(idx + 1) % 16]);
    mx = __builtin_elementwise_maximum(mx, s[NB - 1][15]);
    return half_swap_max(mx);
  }

  // E4M3 probabilities of one element pair -> two bytes of a packed dword
  // (HI selects the upper 16 bits; the other half of `old` is kept)
  template <bool HI>
  static __device__ __forceinline__ int pack2(float a, float b, int old) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  }

  // S(j+1) MFMAs, one K operand read ahead, each followed by a quarter of
  // the probabilities of tile j (program-order interleave, bounded registers)
  static __device__ __forceinline__ void s_with_probs(f32x16 (&snext)[NB], const uint8_t* kst,
                                                      const i32x8 (&qf)[NKS], const f32x16 (&scur)[NB],
                                                      float scale_log2, float m, i32x8& pb, float (&pf)[NB * 16],
                                                      const KAddr& kad) {
    constexpr int NSTEP = NB * NKS;  // (b, c) pairs
    constexpr int WPS = 8 / NSTEP;   // packed probability dwords per MFMA step
    i32x8 ka = read_k(kst, 0, 0, kad);
#pragma unroll
    for (int b = 0; b < NB; ++b) snext[b] = f32x16{};
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int c = st / NB, b = st % NB;
      i32x8 kn;
      if (st + 1 < NSTEP) kn = read_k(kst, (st + 1) % NB, (st + 1) / NB, kad);
      snext[b] = mfma_fp8(ka, qf[c], snext[b]);
#pragma unroll
      for (int ww = 0; ww < WPS; ++ww) {
        const int w = st * WPS + ww, pbb = w / 4, i0 = 4 * (w % 4);
        float* p = pf + 4 * w;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(scur[pbb][i0 + e], scale_log2, -m));
        // (both halves of the dword are written: no zero-initialised target)
        pb[w] = pack2<true>(p[2], p[3], pack2<false>(p[0], p[1], pb[w]));
      }
      if (st + 1 < NSTEP) ka = kn;
    }
    pin(pb);
  }

  // PV(j) MFMAs (the row sum first, so that it is complete early, then the
  // NDB column blocks), one V^T operand read ahead, each followed by
  // a slice of the row max of tile j+1 (raw scores)
  static __device__ __forceinline__ float pv_with_max(f32x16 (&o)[NDB], f32x4& l, const uint8_t* vst,
                                                      const i32x8& pb, const i32x8& sel, const f32x16 (&snext)[NB],
                                                      const int (&vrow0)[1], int vsw, int half, int p8) {
    constexpr int NMAX = (NB * 16 - 2) / 2;  // max3 operations over the tile's 32 scores (after the first)
    constexpr int PER = (NMAX + NDB - 1) / NDB;
    float mx = max3(snext[0][0], snext[0][1], snext[0][2]);
    i32x8 va = read_v(vst, 0, vrow0, vsw, half, p8);
    l = rowsum_fp8(sel, pb, l);
    // keeps the scheduler from sinking the row-sum MFMA to the end of the
    // phase, where the residual test would wait for its result
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x8 vn;
      if (db + 1 < NDB) vn = read_v(vst, db + 1, vrow0, vsw, half, p8);
      o[db] = mfma_fp8(va, pb, o[db]);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int t = db * PER + e;  // scores 3 + 2 t and 4 + 2 t
        if (t < NMAX) {
          const int a = 3 + 2 * t, b = a + 1;
          mx = b < NB * 16 ? max3(mx, snext[a / 16][a % 16], snext[b / 16][b % 16])
                           : __builtin_elementwise_maximum(mx, snext[a / 16][a % 16]);
        }
      }
      if (db + 1 < NDB) va = vn;
    }
    return half_swap_max(mx);
  }

  // second PV pass with the E4M3 residuals of a tile's probabilities (the
  // fp32 probabilities pf, minus their E4M3 values pb)
  static __device__ __forceinline__ void pv_residual(f32x16 (&o)[NDB], f32x4& l, const uint8_t* vst,
                                                     const float (&pf)[NB * 16], const i32x8& pb, const i32x8& sel,
                                                     const int (&vrow0)[1], int vsw, int half, int p8) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    i32x8 pl;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(pb[w], false);
      const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(pb[w], true);
      const float* p = pf + 4 * w;
      pl[w] = pack2<true>(p[2] - h23[0], p[3] - h23[1], pack2<false>(p[0] - h01[0], p[1] - h01[1], 0));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = mfma_fp8(read_v(vst, db, vrow0, vsw, half, p8), pl, o[db]);
    l = rowsum_fp8(sel, pl, l);
  }

  static __device__ __forceinline__ void pin(i32x8& pb) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int v = pb[w];
      asm volatile("" : "+v"(v));
      pb[w] = v;
    }
  }
};

__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                         const uint8_t* __restrict__ V,
                                                         const float* __restrict__ q_scale,
                                                         const float* __restrict__ k_scale,
                                                         const float* __restrict__ v_scale,
                                                         const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ lims,
                                                         const WorkItem* __restrict__ items, int H,
                                                         float scale_log2e, OutSpec out) {
  using Kn = Fp8Kernel;
  using Cfg = Fp8Cfg;
  constexpr int D = Cfg::D, BN = Cfg::BN, NB = Cfg::NB, NKS = Cfg::NKS, NDB = Cfg::NDB, NS = Cfg::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[Cfg::KTILE], k1s[Cfg::KTILE], k2s[Cfg::KTILE], k3s[Cfg::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[Cfg::VTILE], v1s[Cfg::VTILE], v2s[Cfg::VTILE], v3s[Cfg::VTILE];
  uint8_t* const kst[NS] = {k0s, k1s, k2s, k3s};
  uint8_t* const vst[NS] = {v0s, v1s, v2s, v3s};

  WgTimeline tl;
  tl.start();
  const WorkItem it = items[blockIdx.x];
  if (it.seq < 0) return;  // empty slot; uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int L = it.seq_len;
  const int64_t rs = int64_t(H) * D;  // bytes (one byte per element) between tokens of one head
  const uint32_t rs32 = uint32_t(rs);  // the planner keeps L * rs below 2^31
  // bytes from a head's first row of the sequence to the end of its last row
  // (none for a key chunk that holds no rows of this sequence)
  const uint32_t head_bytes = head_span_bytes(L, rs32, uint32_t(D));
  const int32_t kseq = cu[it.seq];  // first K/V token of the sequence
  const int64_t base = int64_t(kseq) * rs + int64_t(it.head) * D;
  // Q and O hold the queried rows only: row r of the sequence is row qo_row + r - q0
  const int64_t qbase = int64_t(it.qo_row - it.q0) * rs + int64_t(it.head) * D;
  const uint8_t* Qh = Q + qbase;
  const uint8_t* Kb = K + base;
  const uint8_t* Vb = V + base;
  const int sh = it.seq * H + it.head;
  // log2 units per raw score, kept at least the smallest normal float: a
  // zero q or k scale (all scores equal) must still turn a masked score
  // (-inf) into a zero probability, which -inf * 0 would not
  const float scale_log2 = __builtin_fmaxf(q_scale[sh] * k_scale[sh] * scale_log2e, 1.17549435e-38f);
  const float vs = v_scale[sh];

  // this lane's query row and its key limit (rows past the tile: L, the K/V
  // rows held); the limits never decrease along the rows, so the wave's
  // first row has the smallest. The limits are stored per queried row.
  const int qend = it.q0 + it.q_rows;
  // key limit of query row r of the sequence (r in [q0, qend)): stored at
  // queried-row index qo_row + r - q0
  auto row_lim = [&](int r) { return lims[it.qo_row + (r - it.q0)]; };
  const int qrow = it.q0 + 32 * wave + l32;
  const int mylim = qrow < qend ? row_lim(qrow) : L;
  const int wrow0 = it.q0 + 32 * wave;
  const bool wave_active = wrow0 < qend;
  const int wlim_min = wave_active ? row_lim(wrow0) : L;
  const int kend = it.k_end;
  // the wave's own last key tile (past its last row's key limit every tile is
  // fully masked for all its rows); 0 for a wave whose rows all lie past the
  // tile. From there on the wave only moves its share of the K/V tiles and
  // meets the barriers.
  const int wkend =
      wave_active ? min(kend, __builtin_amdgcn_readfirstlane((row_lim(min(wrow0 + 31, qend - 1)) + BN - 1) / BN)) : 0;

  typename Kn::KLoader kld;
  typename Kn::VLoader vld;
  // tile t's buffer resource starts at key row t * BN and ends with the
  // sequence: rows past the end read as zeros
  kld.init(rs32, lane, wave);
  vld.init(rs32, lane, wave);
  // (a tile past the sequence end gets an empty range: it reads as zeros and
  // touches no memory; the scalar read keeps the range in scalar registers)
  auto tile_bytes = [&](uint32_t o) { return tile_range_bytes_uniform(head_bytes, o); };
  auto ld_k = [&](int t, uint8_t* stage) {
    const uint32_t o = uint32_t(t * BN) * rs32;
    kld.load(make_rsrc(Kb + o, tile_bytes(o)), stage, wave);
  };
  auto ld_v = [&](int t, uint8_t* stage) {
    const uint32_t o = uint32_t(t * BN) * rs32;
    vld.load(make_rsrc(Vb + o, tile_bytes(o)), stage, wave);
  };
  // Every tile load is issued whatever kend is: each wave then has the same
  // loads in flight on every path, and the partial vmcnt waits below are
  // exact also for the compiler, which otherwise guards LDS reads with full
  // waits.
  ld_k(0, kst[0]);
  ld_k(1, kst[1]);
  ld_v(0, vst[0]);
  ld_k(2, kst[2]);
  ld_v(1, vst[1]);
  ld_k(3, kst[3]);
  ld_v(2, vst[2]);

  // Q^T operands: step c holds d = 64 c + 32 g .. +31 of this lane's query row
  i32x8 qf[NKS];
#pragma unroll
  for (int c = 0; c < NKS; ++c) {
    if (qrow < qend)
      qf[c] = *reinterpret_cast<const i32x8*>(Qh + int64_t(qrow) * rs + 64 * c + 32 * g);
    else
      qf[c] = i32x8{};
  }

  // O^T accumulators and the row sums l of the weights PV applied
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  f32x4 lacc = {};
  i32x8 sel;
  {
    const int sel4 = ((lane >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;  // E4M3 1.0 per byte, or 0
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      // opaque copies: as a known value the compiler would rebuild the
      // 8-register operand every tile
      int t = sel4;
      asm volatile("" : "+v"(t));
      sel[w] = t;
    }
  }
  // The row's reference max m (log2 units) is kept as the derived values the
  // tile loop uses: the exponent bias mb = m - kP8Shift of the probabilities
  // p = 2^(score * scale_log2 - mb), the bias of the residual test and the
  // raw-score threshold past which a tile moves the reference (they change
  // only when it moves).
  float m_run = 0.0f, mb = -kP8Shift, mres = 0.0f, thr = 0.0f;
  auto set_reference = [&](float m) {
    m_run = m;
    mb = m - kP8Shift;
    mres = mb - __builtin_log2f(kResidualFactor);
    thr = (m + kP8Lazy) / scale_log2;
  };

  // per-lane constant parts of the V^T transpose-read addresses: this lane
  // feeds key row 16 r + vrow0 (r = 0..3), columns 32 db + 16 half + 8 p8
  const int e = (lane & 15) >> 1;
  const int vrow0[1] = {8 * (e >> 2) + 4 * g + (e & 3)};
  const int vsw = vswz(vrow0[0]);
  const int half = (lane >> 4) & 1, p8 = 8 * (lane & 1);
  typename Kn::KAddr kad;
  kad.init(l32, g);

  wait_vmcnt<2 * Cfg::DMA_MIN>();
  lds_barrier();
  tl.prologue_done();

  auto s_mfma = [&](f32x16(&s)[NB], const uint8_t* kt) {
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
    for (int c = 0; c < NKS; ++c)
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = mfma_fp8(Kn::read_k(kt, b, c, kad), qf[c], s[b]);
  };

  f32x16 sa[NB], sb[NB];
  float tmax = -INFINITY;  // the current tile's largest raw score of the row
  if (wkend > 0) {
    s_mfma(sa, kst[0]);
    if (BN > wlim_min) Kn::mask(sa, 0, g, mylim);
    tmax = Kn::tile_max(sa);
    // a row with no key in range keeps a finite reference (its p are all 0)
    set_reference(tmax == -INFINITY ? 0.0f : tmax * scale_log2);
  }

  auto iteration = [&](auto sj_tag, int j, f32x16(&scur)[NB], f32x16(&snext)[NB]) {
    constexpr int SJ = decltype(sj_tag)::value;
    lds_barrier();
    ld_k(j + NS, kst[SJ]);
    ld_v(j + NS - 1, vst[(SJ + NS - 1) % NS]);
    const int k1 = (j + 1) * BN;
    // S(j+1) MFMAs beside the exponentials of tile j
    i32x8 pb;
    float pf[NB * 16];
    // (this VALU-heavy phase at raised wave priority: measured slightly
    // faster than equal priorities, and than raising it around PV instead)
    __builtin_amdgcn_s_setprio(1);
    Kn::s_with_probs(snext, kst[(SJ + 1) % NS], qf, scur, scale_log2, mb, pb, pf, kad);
    __builtin_amdgcn_s_setprio(0);
    if (__builtin_expect(k1 + BN > wlim_min, 0)) Kn::mask(snext, k1, g, mylim);
    // PV(j) MFMAs beside the row max of tile j+1
    const float mt = Kn::pv_with_max(oacc, lacc, vst[SJ], pb, sel, snext, vrow0, vsw, half, p8);
    // residual pass when a key of this tile may carry 1/kResidualFactor of
    // its row's weight: kResidualFactor times the tile's largest probability
    // against the row's sum so far, this tile included (a row without keys
    // has 0 against 0 and never asks for it)
    if (__builtin_expect(wave_any(fast_exp2(fmaf(tmax, scale_log2, -mres)) > lacc[0]), 0))
      Kn::pv_residual(oacc, lacc, vst[SJ], pf, pb, sel, vrow0, vsw, half, p8);
    tmax = mt;
    const bool need = mt > thr;
    if (__builtin_expect(wave_any(need), 0)) {
      const float mtl = mt * scale_log2;
      const float alpha = need ? fast_exp2(m_run - mtl) : 1.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) lacc[i] *= alpha;
      if (need) set_reference(mtl);
    }
    wait_vmcnt<2 * Cfg::DMA_MIN>();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Four unrolled iterations per trip, each guarded; the last tile's
  // iteration also computes S of the tile after it on a stale stage, which
  // the mask turns entirely into -inf (no effect on the result).
  for (int j = 0; j < wkend; j += 4) {
    iteration(I0{}, j, sa, sb);
    if (j + 1 >= wkend) break;
    iteration(I1{}, j + 1, sb, sa);
    if (j + 2 >= wkend) break;
    iteration(I2{}, j + 2, sa, sb);
    if (j + 3 >= wkend) break;
    iteration(I3{}, j + 3, sb, sa);
  }
  tl.loop_done();
  // the rest of the item's tiles: the same barriers and DMA as an iteration
  // above, none of its arithmetic
  for (int j = wkend; j < kend; ++j) {
    lds_barrier();
    const int sk = j % NS, sv = (j + NS - 1) % NS;
    ld_k(j + NS, sk == 0 ? kst[0] : sk == 1 ? kst[1] : sk == 2 ? kst[2] : kst[3]);
    ld_v(j + NS - 1, sv == 0 ? vst[0] : sv == 1 ? vst[1] : sv == 2 ? vst[2] : vst[3]);
    wait_vmcnt<2 * Cfg::DMA_MIN>();
  }

  // the loads of the last iterations (tiles past kend) must land before the
  // workgroup ends and its LDS is handed to another
  wait_vmcnt<0>();

  // ---- epilogue: O = O^T * v_s / l (l from the row-sum MFMA), bf16, or fp32
  // for partial results, folded into a running result when one is given;
  // optionally the row's log-sum-exp of the scaled scores,
  // ln 2 * (m + log2 l - kP8Shift) with l the sum of the weights PV applied
  // (-inf for a row with no key in range)
  if (wave_active && qrow < qend) {
    const float lt = lacc[0];
    write_row<NDB>(out, qbase + int64_t(qrow) * rs, int64_t(it.qo_row - it.q0 + qrow) * H + it.head, g, oacc,
                   lt > 0.0f ? vs / lt : 0.0f, lt > 0.0f ? 0.6931471805599453f * (mb + __log2f(lt)) : -INFINITY);
  }
  tl.finish(timeline_records(), wkend, kend);
}

}  // namespace

int timeline_records_fp8(void** ptr) {
#ifdef PVA_WG_TIMELINE
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(g_timeline)) == hipSuccess ? PVA_OK : PVA_ERR_HIP;
#else
  (void)ptr;
  return PVA_ERR_UNSUPPORTED;
#endif
}

int launch_fwd_fp8(const void* q, const void* k, const void* v, const float* qs, const float* ks, const float* vs,
                   const int32_t* cu, const pva_seg_desc* d, float scale, const OutSpec& out, hipStream_t stream) {
  if (d->plan.head_dim != Fp8Cfg::D) return PVA_ERR_UNSUPPORTED;
  if (d->plan.tile.bm != Fp8Cfg::BM || d->plan.tile.bn != Fp8Cfg::BN) return PVA_ERR_UNSUPPORTED;
  const int n = static_cast<int>(d->plan.items.size());
  if (n == 0) return PVA_OK;
  const float scale_log2e = static_cast<float>(double(scale) * 1.4426950408889634);
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3(n), dim3(Fp8Cfg::NT), 0, stream, static_cast<const uint8_t*>(q),
                     static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), qs, ks, vs, cu, d->d_lims,
                     static_cast<const WorkItem*>(d->d_items), d->plan.num_heads, scale_log2e, out);
  return hipGetLastError() == hipSuccess ? PVA_OK : PVA_ERR_HIP;
}

}  // namespace pva
