// Packed mixed-mask attention forward for gfx950: bf16 in, fp32 accumulate,
// bf16 out.
//
// Operation: "[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0 (packed
// cu_seqlens attention over requests of mixed resolution; its attention mask
// challenge) and Model structure item 1 (Generalized Causal Attention: causal
// text prefix, bidirectional image block that sees the whole prefix).
//
// One workgroup = 4 waves = one work item (sequence, head, 128 query rows);
// each wave owns 32 query rows, three workgroups share a CU (three waves
// per SIMD, at most 168 registers each). Keys are streamed in tiles of 32.
//
// Per wave and key tile j, on 32x32x16 bf16 MFMA:
//   S^T[key, q] = K Q^T    A = K from LDS (16-byte reads), B = Q^T held in
//                          registers for the whole item. Each lane then owns
//                          one query column, so row max and row sum are
//                          in-lane plus one exchange between the two 32-lane
//                          halves.
//   online softmax in fp32, log2 domain, lazy rescaling of O and l.
//   O^T[d, q] += V^T P^T   B = P^T straight from the S^T accumulators (cast to
//                          bf16, no shuffle: the contraction order of the keys
//                          is permuted instead), A = V^T read from the
//                          row-major V tile with ds_read_b64_tr_b16.
//
// Software pipeline (iteration j, one barrier each):
//   issue global->LDS loads of K(j+NS) and V(j+NS-1) (buffer loads straight
//   into LDS; rows past the sequence end read as zeros)
//   phase 1: [S(j+1) MFMAs] next to [exp / bf16 packing of tile j]
//   (partial tiles only) element mask of tile j+1
//   phase 2: [PV(j) MFMAs] next to [row sums of tile j, row max of tile j+1];
//            the V^T operands are read from LDS two MFMAs ahead
//   rare branch: rescale O and l when a row's reference max moved
//   wait for the loads of K(j+2) and V(j+1) only; later ones stay in flight
// K and V each have a ring of NS = 3 LDS stages (48 KB per workgroup): a
// load issued at iteration j is waited for at the end of iteration j + 1.
// Tiles the mask fully hides are never loaded; tiles it fully allows skip
// the element mask. A wave whose rows all lie past the tile only moves its
// share of the tiles and meets the barriers.
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

template <int D>
struct Bf16Cfg {
  static constexpr int BM = kBf16BlockM, BN = kBf16BlockN, NW = BM / 32, NT = 64 * NW;
  static_assert(BM % 32 == 0 && BN == 32, "one 32-row query block per wave; 32-key tiles");
  static constexpr int C = D / 8;          // 16-byte chunks per K/V row
  static constexpr int NKC = D / 16;       // MFMA k-steps over the head dimension for S^T
  static constexpr int NDB = D / 32;       // 32-row blocks of O^T
  static constexpr int NS = kBf16Stages;   // LDS stages per tensor
  // K and V tiles are stored unpadded (C 16-byte chunks per row), with the
  // chunks of each row XOR-permuted so that the MFMA operand reads are free of
  // LDS bank conflicts:
  //  * K is read 16 bytes per lane, 16 consecutive rows per LDS cycle at one
  //    logical chunk: swz_k spreads those 16 reads over 16 bank groups;
  //  * V is read with ds_read_b64_tr_b16, 4 consecutive rows x 64 bytes per
  //    half-wave: swz_v (whole 64-byte quarters) puts the 4 rows in 4
  //    different quarters of the 256-byte bank window.
  // Both depend on the row only through bits that the per-step row offsets
  // (16 kc, +8) keep, so each lane needs one address per K chunk and one per
  // 32-column V block, and the step offsets are immediates.
  static constexpr int KSLOTS = BN * C;
  static constexpr int KTILE = KSLOTS * 16;
  static constexpr int VSLOTS = BN * C;
  static constexpr int VTILE = VSLOTS * 16;
  static __device__ __forceinline__ int swz_k(int r) { return ((r * C) / 16) % C; }
  static __device__ __forceinline__ int swz_v(int r) { return 4 * (((r * C) / 16) % (C / 4)); }
  struct KMap {
    static __device__ __forceinline__ int chunk(int r, int pos) { return pos ^ swz_k(r); }
  };
  struct VMap {
    static __device__ __forceinline__ int chunk(int r, int pos) { return pos ^ swz_v(r); }
  };
  // DMA instructions every wave issues per tile (some waves issue one more);
  // the partial vmcnt waits count only these, so waves with more loads in
  // flight simply wait a little longer
  static constexpr int DMA_MIN = KSLOTS / NT + VSLOTS / NT;
  static_assert(3 * (KTILE + VTILE) * NS <= 160 * 1024, "three workgroups per CU");
};

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

template <int D>
struct Kernel {
  using Cfg = Bf16Cfg<D>;
  static constexpr int BN = Cfg::BN, C = Cfg::C, NKC = Cfg::NKC, NDB = Cfg::NDB;
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

  // ---- K and V tiles: unpadded rows, XOR-permuted chunks
  using KLoader = BufLoader<Cfg::NT, C, Cfg::KSLOTS, typename Cfg::KMap>;
  using VLoader = BufLoader<Cfg::NT, C, Cfg::VSLOTS, typename Cfg::VMap>;

  // Per-lane byte offsets (within a stage) of the operand reads: K chunk c of
  // row l32; V^T block db of rows v_row0 (steps add 16 kc rows, +8 rows).
  struct ReadAddr {
    uint32_t k[NKC];
    uint32_t v[NDB];
    __device__ __forceinline__ void init(int l32, int g, int v_row0, int v_col) {
#pragma unroll
      for (int c = 0; c < NKC; ++c) k[c] = uint32_t(16 * (C * l32 + ((2 * c + g) ^ Cfg::swz_k(l32))));
      const int hv = Cfg::swz_v(v_row0) / 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) v[db] = uint32_t(16 * C * v_row0 + 64 * (db ^ hv) + 2 * v_col);
    }
  };

  // ---- K operand of d-chunk c
  static __device__ __forceinline__ bf16x8 read_k(const uint8_t* kst, int c, const ReadAddr& ra) {
    return *reinterpret_cast<const bf16x8*>(kst + ra.k[c]);
  }

  // ---- V^T operand of PV step `step` (16-key step kc, 32-column block db)
  static __device__ __forceinline__ s16x8 read_v_step(const uint8_t* vst, int step, const ReadAddr& ra) {
    const int kc = step / NDB, db = step % NDB;
    const uint8_t* p0 = vst + ra.v[db] + 16 * C * 16 * kc;
    const uint8_t* p1 = p0 + 16 * C * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p1));
    return s16x8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // ---- S^T = K Q^T of one tile (prologue only; the loop interleaves it)
  static __device__ __forceinline__ f32x16 s_tile(const uint8_t* kst, const bf16x8 (&qf)[NKC], const ReadAddr& ra) {
    f32x16 s = {};
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(kst, c, ra), qf[c], s, 0, 0, 0);
    return s;
  }

  // Probabilities of a tile: p_i = 2^(s_i * scale_log2 - m) in bf16, packed
  // two per dword (pair k = elements 2k, 2k+1). Pair k's element i sits at
  // key 8 (i / 4) + 4 g + i % 4 of the tile, which is the B-operand order of
  // PV's 16-key step i / 8 with the keys' contraction order permuted.
  static constexpr int EPC = 16 / NKC;  // exponentials per S MFMA
  static_assert(EPC % 2 == 0, "whole pairs per MFMA");

  // ---- phase 1: S(j+1) = K Q^T (NKC dependent MFMAs), each listed with EPC
  // exponentials of tile j and the bf16 packing of the previous group's
  // (the compiler's scheduler places them).
  // The K operands are read two chunks ahead.
  static constexpr int NSTEP = 2 * NDB;
  static __device__ __forceinline__ void s_phase(f32x16& snext, const uint8_t* kst, const bf16x8 (&qf)[NKC],
                                                 const f32x16& scur, float scale_log2, float m, float (&e)[16],
                                                 uint32_t (&pk)[8], const ReadAddr& ra) {
    bf16x8 ka[3];
    ka[0] = read_k(kst, 0, ra);
    if (NKC > 1) ka[1] = read_k(kst, 1, ra);
    snext = f32x16{};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if (c + 2 < NKC) ka[(c + 2) % 3] = read_k(kst, c + 2, ra);
      snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c % 3], qf[c], snext, 0, 0, 0);
#pragma unroll
      for (int i = c * EPC; i < (c + 1) * EPC; ++i) e[i] = fast_exp2(fmaf(scur[i], scale_log2, -m));
      if (c > 0) {
#pragma unroll
        for (int k = (c - 1) * EPC / 2; k < c * EPC / 2; ++k) pk[k] = pack_bf16(e[2 * k], e[2 * k + 1]);
      }
      }
    // consume the results in an empty asm: the compiler must compute them
    // here, not sink them past the mask branch that follows into phase 2
#pragma unroll
    for (int k = 0; k < (NKC - 1) * EPC / 2; ++k) asm volatile("" : "+v"(pk[k]));
#pragma unroll
    for (int i = (NKC - 1) * EPC; i < 16; ++i) asm volatile("" : "+v"(e[i]));
  }

  static __device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }

  // ---- phase 2: O^T += V^T P^T (2 NDB MFMAs), each listed with the row-sum
  // dot products of the probabilities and, from the third on, part of the
  // row max of S(j+1). The V^T operands are read two steps ahead (holding all
  // of them from phase 1 on would not fit three waves per SIMD).
  static __device__ __forceinline__ void pv_phase(f32x16 (&o)[NDB], s16x8 (&va)[NSTEP], const float (&e)[16],
                                                  uint32_t (&pk)[8], const f32x16& snext, float& mx, float& psum,
                                                  const uint8_t* vst, const ReadAddr& ra) {
    va[0] = read_v_step(vst, 0, ra);
    va[1] = read_v_step(vst, 1, ra);
    constexpr int PPS = 8 / NSTEP;  // row-sum pairs per step
    constexpr int MAX_FROM = NSTEP > 2 ? 2 : 0;  // S(j+1) is complete two MFMAs in
    float part[2] = {0.0f, 0.0f};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // the 8 max3 operations of the tile's 16 scores, spread over steps MAX_FROM..
    int nmax = 0;
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      if (step == 0) {
        // the last group's pairs (not packed in phase 1)
#pragma unroll
        for (int k = (NKC - 1) * EPC / 2; k < 8; ++k) pk[k] = pack_bf16(e[2 * k], e[2 * k + 1]);
      }
      if (step + 2 < NSTEP) va[step + 2] = read_v_step(vst, step + 2, ra);
      const int kc = step / NDB, db = step % NDB;
      const i32x4 b = {int(pk[4 * kc]), int(pk[4 * kc + 1]), int(pk[4 * kc + 2]), int(pk[4 * kc + 3])};
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[step]),
                                                      __builtin_bit_cast(bf16x8, b), o[db], 0, 0, 0);
#pragma unroll
      for (int k = step * PPS; k < (step + 1) * PPS; ++k) {
        part[k % 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[k]), ones, part[k % 2], false);
        asm volatile("" : "+v"(part[k % 2]));  // keep it next to this step's MFMA
      }
      if (step >= MAX_FROM) {
        const int upto = 8 * (step + 1 - MAX_FROM) / (NSTEP - MAX_FROM);
#pragma unroll
        for (; nmax < upto; ++nmax) {
          if (nmax == 0)
            mx = max3(snext[0], snext[1], snext[2]);
          else if (nmax < 7)
            mx = max3(mx, snext[2 * nmax + 1], snext[2 * nmax + 2]);
          else
            mx = __builtin_elementwise_maximum(mx, snext[15]);
        }
      }
      }
    psum = part[0] + part[1];
  }

  // ---- element mask: keys at or past the lane's limit get -inf
  static __device__ __forceinline__ void mask(f32x16& s, int k0, int g, int mylim) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = k0 + 8 * (i / 4) + 4 * g + (i % 4);
      if (key >= mylim) s[i] = -INFINITY;
    }
  }

  // ---- tile max in log2 units, shared by both half-waves
  static __device__ __forceinline__ float tile_max(const f32x16& s, float scale_log2) {
    float mx = max3(s[0], s[1], s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = max3(mx, s[i], s[i + 1]);
    mx = __builtin_elementwise_maximum(mx, s[15]);
    return half_swap_max(mx) * scale_log2;
  }
};

// K / V in a paged pool [num_blocks, block_size, H, D]: key row r of
// sequence s sits in pool block table[s * stride + r / block_size], row
// r % block_size. block_size is a power of two and a multiple of the key
// tile, so every tile lies inside one block.
struct Paging {
  const int32_t* table;
  int32_t stride;       // table entries per sequence
  int32_t block_shift;  // log2(block_size)
  int32_t num_blocks;
};

template <int D, bool PAGED>
__device__ __forceinline__ void fwd_bf16_body(const __bf16* __restrict__ Q,
                                                                    const __bf16* __restrict__ K,
                                                                    const __bf16* __restrict__ V,
                                                                    const int32_t* __restrict__ cu,
                                                                    const int32_t* __restrict__ lims,
                                                                    const WorkItem* __restrict__ items, int H,
                                                                    float scale_log2, const OutSpec& out,
                                                                    Paging pg) {
  using Kn = Kernel<D>;
  using Cfg = typename Kn::Cfg;
  using s16x8 = typename Kn::s16x8;
  constexpr int BN = Cfg::BN, NKC = Cfg::NKC, NDB = Cfg::NDB, NS = Cfg::NS;
  static_assert(NS == 3, "the loop below is unrolled for a ring of three stages");
  // separate arrays per stage: the compiler sees that an LDS DMA into one
  // stage and reads of another do not alias
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[Cfg::KTILE], k1s[Cfg::KTILE], k2s[Cfg::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[Cfg::VTILE], v1s[Cfg::VTILE], v2s[Cfg::VTILE];
  uint8_t* const kst[NS] = {k0s, k1s, k2s};
  uint8_t* const vst[NS] = {v0s, v1s, v2s};

  WgTimeline tl;
  tl.start();
  const WorkItem it = items[blockIdx.x];
  if (it.seq < 0) return;  // empty slot; uniform over the workgroup

  // the wave index is uniform per wave; reading it through a scalar register
  // makes every per-wave condition below a scalar branch
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int L = it.seq_len;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive tokens of one head
  const uint32_t rs2 = uint32_t(rs) * 2u;  // bytes (the planner keeps L * rs2 below 2^31)
  // bytes from a head's first row of the sequence to the end of its last row
  // (none for a key chunk that holds no rows of this sequence)
  const uint32_t head_bytes = head_span_bytes(L, rs2, 2u * D);
  constexpr bool paged = PAGED;
  const int32_t kseq = paged ? 0 : cu[it.seq];  // first K/V token of the sequence (contiguous K/V)
  const int64_t base = int64_t(kseq) * rs + int64_t(it.head) * D;
  // Q and O hold the queried rows only: row r of the sequence is row qo_row + r - q0
  const int64_t qbase = int64_t(it.qo_row - it.q0) * rs + int64_t(it.head) * D;
  const __bf16* Qh = Q + qbase;

  // this lane's query row and its key limit; rows past the tile see all L
  // keys held (their outputs are never stored). The limits are stored per
  // queried row and never decrease along the rows, so the wave's first row
  // has the smallest.
  const int qend = it.q0 + it.q_rows;
  // key limit of query row r of the sequence (r in [q0, qend)): stored at
  // queried-row index qo_row + r - q0
  auto row_lim = [&](int r) { return lims[it.qo_row + (r - it.q0)]; };
  const int wrow0 = it.q0 + 32 * wave;
  const int qrow = wrow0 + l32;
  const int mylim = qrow < qend ? row_lim(qrow) : L;
  const bool wave_active = wrow0 < qend;  // uniform per wave: a scalar branch
  const int wlim_min = wave_active ? row_lim(wrow0) : L;
  const int kend = it.k_end;
  // The wave's own last key tile: past the key limit of its last row every
  // tile is fully masked for all its rows (limits never decrease along the
  // rows). From there on, and for a wave whose rows all lie past the tile
  // (in the last tile of a sequence), the wave only moves its share of the
  // K/V tiles and meets the barriers (the loop after the tile loop below).
  const int wkend =
      wave_active ? min(kend, __builtin_amdgcn_readfirstlane((row_lim(min(wrow0 + 31, qend - 1)) + BN - 1) / BN)) : 0;

  // prologue DMA in the order the tiles are needed: K0 K1 V0 | K2 V1
  // (tile t's resource starts at key row t * BN and ends with the sequence)
  typename Kn::KLoader kld;
  typename Kn::VLoader vld;
  kld.init(rs2, lane, wave);
  vld.init(rs2, lane, wave);
  // paged K/V: a tile's pool block comes from the table (a scalar load). The
  // loop reads the blocks of the next iteration's tiles one iteration ahead,
  // so the load has landed by the barrier that starts that iteration. An
  // entry outside [0, num_blocks) is clamped so that no load leaves the pool.
  // (read through the constant address space: a scalar load, whose wait does
  // not also wait for the K/V DMA the way a vector load's would)
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  const const_i32p tbl = paged ? (const_i32p)(pg.table + int64_t(it.seq) * pg.stride) : nullptr;
  // raw table entry of tile t's block; clamped where it is used, so that the
  // scalar load is only waited for there
  auto block_of = [&](int t) -> int {
    if (!paged || t >= kend) return 0;
    return tbl[(t * BN) >> pg.block_shift];
  };
  auto tile_src = [&](const __bf16* contiguous, int t, int blk, uint32_t& bytes) -> const uint8_t* {
    const int k0 = t * BN;
    if (paged) {
      blk = min(max(blk, 0), pg.num_blocks - 1);
      const int row = k0 & ((1 << pg.block_shift) - 1);
      // the rows of the sequence in this tile; none for a tile past its end
      // (the scalar read keeps the range in scalar registers)
      bytes = uint32_t(__builtin_amdgcn_readfirstlane(head_span_bytes(min(BN, L - k0), rs2, 2u * D)));
      return reinterpret_cast<const uint8_t*>(contiguous + ((int64_t(blk) << pg.block_shift) + row) * rs +
                                              int64_t(it.head) * D);
    } else {
      const uint32_t o = uint32_t(k0) * rs2;
      // nothing for a tile past the sequence end
      bytes = tile_range_bytes_uniform(head_bytes, o);
      return reinterpret_cast<const uint8_t*>(contiguous + base) + o;
    }
  };
  auto ld_k = [&](int t, uint8_t* stage, int blk) {
    uint32_t bytes;
    const uint8_t* src = tile_src(K, t, blk, bytes);
    kld.load(make_rsrc(src, bytes), stage, wave);
  };
  auto ld_v = [&](int t, uint8_t* stage, int blk) {
    uint32_t bytes;
    const uint8_t* src = tile_src(V, t, blk, bytes);
    vld.load(make_rsrc(src, bytes), stage, wave);
  };
  // Every tile load is issued whatever kend is (a tile past the sequence end
  // reads as zeros and touches no memory): each wave then has the same loads
  // in flight on every path, and the partial vmcnt waits below are exact
  // also for the compiler, which otherwise guards LDS reads with full waits.
  ld_k(0, kst[0], block_of(0));
  ld_k(1, kst[1], block_of(1));
  ld_v(0, vst[0], block_of(0));
  ld_k(2, kst[2], block_of(2));
  ld_v(1, vst[1], block_of(1));
  // pool blocks of the tiles the first loop iteration loads
  int kblk = block_of(NS), vblk = block_of(NS - 1);

  // Q^T operands: chunk c holds d = 16c + 8g .. +7 of this lane's query row
  bf16x8 qf[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    if (qrow < qend)
      qf[c] = *reinterpret_cast<const bf16x8*>(Qh + int64_t(qrow) * rs + 16 * c + 8 * g);
    else
      qf[c] = bf16x8{};
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  RowState st{-INFINITY, 0.0f};

  // per-lane LDS offsets of the K and V^T (transpose-read) operands
  typename Kn::ReadAddr ra;
  ra.init(l32, g, 4 * g + (lane & 15) / 4, 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  // K0, K1, V0 must have landed; K2 V1 may still be in flight
  wait_vmcnt<Cfg::DMA_MIN>();
  lds_barrier();
  tl.prologue_done();

  f32x16 sa, sb;
  // S(0) and its reference max. Rows past the sequence end, and tiles past a
  // row's key limit, are computed masked: their probabilities are exactly
  // zero. That keeps every branch in the loop scalar and rare.
  if (wkend > 0) {
    sa = Kn::s_tile(kst[0], qf, ra);
    if (BN > wlim_min) Kn::mask(sa, 0, g, mylim);
    st.m = Kn::tile_max(sa, scale_log2);  // first tile: O and l are still zero
    // a row with no key in range keeps a finite reference (its p are all 0)
    if (st.m == -INFINITY) st.m = 0.0f;
  }

  // Iteration j; `scur` holds S(j), `snext` receives S(j+1). SJ = j % NS
  // (compile-time in each unrolled copy). The rare branches (element mask,
  // rescale) are marked unlikely so that the common path falls through.
  auto iteration = [&](auto sj_tag, int j, f32x16& scur, f32x16& snext) {
    constexpr int SJ = decltype(sj_tag)::value;
    lds_barrier();  // every wave is done with S(j) (K stage SJ) and PV(j-1) (V stage SJ-1)
    ld_k(j + NS, kst[SJ], kblk);
    ld_v(j + NS - 1, vst[(SJ + NS - 1) % NS], vblk);
    if constexpr (PAGED) {  // the next iteration's blocks, read ahead
      kblk = block_of(j + NS + 1);
      vblk = block_of(j + NS);
    }
    const int k1 = (j + 1) * BN;
    s16x8 va[Kn::NSTEP];  // V^T operands of PV(j), read during phase 2
    float e[16];
    uint32_t pk[8];
    Kn::s_phase(snext, kst[(SJ + 1) % NS], qf, scur, scale_log2, st.m, e, pk, ra);
    if (__builtin_expect(k1 + BN > wlim_min, 0)) Kn::mask(snext, k1, g, mylim);
    float mx, psum;
    Kn::pv_phase(oacc, va, e, pk, snext, mx, psum, vst[SJ], ra);
    st.l += psum;
    const float mt = half_swap_max(mx) * scale_log2;
    const bool need = mt > st.m + kLazyRescale;
    if (__builtin_expect(wave_any(need), 0)) {
      // per-lane decision: a lane that does not need it keeps its max (alpha = 1
      // exactly), so each row's arithmetic depends on its own scores only
      const float alpha = need ? fast_exp2(st.m - mt) : 1.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      st.l *= alpha;
      st.m = need ? mt : st.m;
    }
    // K(j+2) and V(j+1) are needed next; the loads of iteration j may stay
    // in flight
    wait_vmcnt<Cfg::DMA_MIN>();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  // Six unrolled iterations per trip (two rounds of the three-stage ring, so
  // that the S buffers alternate), each guarded; the last tile's
  // iteration also computes S of the tile after it on a stale stage, which
  // the mask turns entirely into -inf (no effect on the result).
  for (int j = 0; j < wkend; j += 6) {
    iteration(I0{}, j, sa, sb);
    if (j + 1 >= wkend) break;
    iteration(I1{}, j + 1, sb, sa);
    if (j + 2 >= wkend) break;
    iteration(I2{}, j + 2, sa, sb);
    if (j + 3 >= wkend) break;
    iteration(I0{}, j + 3, sb, sa);
    if (j + 4 >= wkend) break;
    iteration(I1{}, j + 4, sa, sb);
    if (j + 5 >= wkend) break;
    iteration(I2{}, j + 5, sb, sa);
  }
  tl.loop_done();
  // the rest of the item's tiles: the same barriers and DMA as an iteration
  // above, none of its arithmetic
  for (int j = wkend; j < kend; ++j) {
    lds_barrier();
    // stage of tile j + 3 (K) and j + 2 (V), picked without indexing the
    // stage tables at run time
    const int sk = j % NS, sv = (j + NS - 1) % NS;
    ld_k(j + NS, sk == 0 ? kst[0] : sk == 1 ? kst[1] : kst[2], kblk);
    ld_v(j + NS - 1, sv == 0 ? vst[0] : sv == 1 ? vst[1] : vst[2], vblk);
    if constexpr (PAGED) {
      kblk = block_of(j + NS + 1);
      vblk = block_of(j + NS);
    }
    wait_vmcnt<Cfg::DMA_MIN>();
  }

  // the loads of the last iterations (tiles past kend) must land before the
  // workgroup ends and its LDS is handed to another
  wait_vmcnt<0>();

  // ---- epilogue: O = O^T / l (bf16, or fp32 for partial results), rows of
  // this tile only, folded into a running result when one is given;
  // optionally the row's log-sum-exp of the scaled scores, ln 2 * (m + log2 l)
  // (-inf for a row with no key in range)
  const float lt = half_swap_sum(st.l);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (qrow < qend)
    write_row<NDB>(out, qbase + int64_t(qrow) * rs, int64_t(it.qo_row - it.q0 + qrow) * H + it.head, g, oacc, inv,
                   lt > 0.0f ? 0.6931471805599453f * (st.m + __log2f(lt)) : -INFINITY);
  tl.finish(timeline_records(), wkend, kend);
}

// Two kernels over the same body: K/V contiguous in [N, H, D], or paged.
template <int D>
__global__ __launch_bounds__(Bf16Cfg<D>::NT, 3) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lims, const WorkItem* __restrict__ items, int H,
    float scale_log2, OutSpec out) {
  fwd_bf16_body<D, false>(Q, K, V, cu, lims, items, H, scale_log2, out, Paging{nullptr, 0, 0, 0});
}

template <int D>
__global__ __launch_bounds__(Bf16Cfg<D>::NT, 3) void fwd_bf16_paged_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ lims, const WorkItem* __restrict__ items, int H,
    float scale_log2, OutSpec out, Paging pg) {
  fwd_bf16_body<D, true>(Q, K, V, cu, lims, items, H, scale_log2, out, pg);
}

template <int D>
int launch(const void* q, const void* k, const void* v, const int32_t* cu, const pva_seg_desc* d, float scale,
           const OutSpec& out, const PagedKV* paged, hipStream_t stream) {
  using Cfg = Bf16Cfg<D>;
  const int n = static_cast<int>(d->plan.items.size());
  if (n == 0) return PVA_OK;
  const float scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634);
  const auto* qp = static_cast<const __bf16*>(q);
  const auto* kp = static_cast<const __bf16*>(k);
  const auto* vp = static_cast<const __bf16*>(v);
  const auto* items = static_cast<const WorkItem*>(d->d_items);
  if (paged) {
    int shift = 0;
    while ((1 << shift) < paged->block_size) ++shift;
    const Paging pg{paged->table, paged->stride, shift, paged->num_blocks};
    hipLaunchKernelGGL(fwd_bf16_paged_kernel<D>, dim3(n), dim3(Cfg::NT), 0, stream, qp, kp, vp, cu, d->d_lims, items,
                       d->plan.num_heads, scale_log2, out, pg);
  } else {
    hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(n), dim3(Cfg::NT), 0, stream, qp, kp, vp, cu, d->d_lims, items,
                       d->plan.num_heads, scale_log2, out);
  }
  return hipGetLastError() == hipSuccess ? PVA_OK : PVA_ERR_HIP;
}

}  // namespace

int timeline_records_bf16(void** ptr) {
#ifdef PVA_WG_TIMELINE
  return hipGetSymbolAddress(ptr, HIP_SYMBOL(g_timeline)) == hipSuccess ? PVA_OK : PVA_ERR_HIP;
#else
  (void)ptr;
  return PVA_ERR_UNSUPPORTED;
#endif
}

int launch_fwd_bf16(const void* q, const void* k, const void* v, const int32_t* cu, const pva_seg_desc* d,
                    float scale, const OutSpec& out, const PagedKV* paged, hipStream_t stream) {
  switch (d->plan.head_dim) {
    case 64: return launch<64>(q, k, v, cu, d, scale, out, paged, stream);
    case 128: return launch<128>(q, k, v, cu, d, scale, out, paged, stream);
    default: return PVA_ERR_UNSUPPORTED;
  }
}

}  // namespace pva
