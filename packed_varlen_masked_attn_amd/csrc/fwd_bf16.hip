// Packed mixed-mask attention forward for gfx950: bf16 in, fp32 accumulate,
// bf16 out.
//
// Operation: "[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0 (packed
// cu_seqlens attention over requests of mixed resolution; its attention mask
// challenge) and Model structure item 1 (Generalized Causal Attention: causal
// text prefix, bidirectional image block that sees the whole prefix).
//
// One workgroup = 4 waves = one work item (sequence, head, 256 query rows);
// one wave per SIMD, each owning 64 query rows as two 32-row blocks that share
// every K and V operand read. Keys are streamed in tiles of 32.
//
// Per wave and key tile j, on 32x32x16 bf16 MFMA:
//   S^T[key, q] = K Q^T    A = K from LDS (16-byte reads), B = Q^T held in
//                          registers for the whole item. Each lane then owns
//                          one query column of each block, so row max and
//                          row sum are in-lane plus one exchange between the
//                          two 32-lane halves.
//   online softmax in fp32, log2 domain, lazy rescaling of O and l.
//   O^T[d, q] += V^T P^T   B = P^T straight from the S^T accumulators (cast to
//                          bf16, no shuffle: the contraction order of the keys
//                          is permuted instead), A = V^T read from the
//                          row-major V tile with ds_read_b64_tr_b16.
//
// Software pipeline (iteration j, one barrier each):
//   issue global->LDS loads of K(j+NS) and V(j+NS-1) (direct LDS DMA)
//   [S(j+1) MFMAs]  interleaved with  [exp / row sums / bf16 cast of tile j]
//   (partial tiles only) element mask of tile j+1
//   [PV(j) MFMAs]   interleaved with  [row max of tile j+1]
//   rare branch: rescale O and l when a row's reference max moved
//   wait for the loads of K(j+2) and V(j+1) only; later ones stay in flight
// K and V each have a ring of NS LDS stages, so every load has NS-1
// iterations to land. Tiles the mask fully hides are never loaded; tiles it
// fully allows skip the element mask.
#include <type_traits>

#include "kernel_common.h"

#ifndef PVA_BF16_QB
#define PVA_BF16_QB 1  // 32-row query blocks per wave: 1 (2 waves/SIMD) or 2 (1 wave/SIMD)
#endif

namespace pva {

namespace {

template <int D>
struct Bf16Cfg {
  static constexpr int QB = PVA_BF16_QB;   // 32-row query blocks per wave
  static constexpr int BM = kBf16BlockM, BN = kBf16BlockN, NW = BM / (32 * QB), NT = 64 * NW;
  static_assert(BM == NW * QB * 32 && BN == 32, "waves x 32-row query blocks; 32-key tiles");
  static constexpr int C = D / 8;          // 16-byte chunks per K/V row
  static constexpr int NKC = D / 16;       // MFMA k-steps over the head dimension for S^T
  static constexpr int NDB = D / 32;       // 32-row blocks of O^T
  static constexpr int NS = 4;             // LDS stages per tensor
  // K rows are padded by one 16-byte chunk: the 16 consecutive rows a K
  // operand read touches at one chunk then fall on 16 different bank groups,
  // and the address stays affine in the chunk (one base register).
  static constexpr int KROW = C + 1;                        // chunks per padded K row
  // 16-byte slots of a K / V stage, rounded up to whole 64-lane DMA rounds
  static constexpr int KSLOTS = (BN * KROW + 63) / 64 * 64;
  static constexpr int KTILE = KSLOTS * 16;
  // V rows are padded by 64 bytes: the four consecutive rows a transpose read
  // touches then sit in four different 64-byte quarters of the bank window,
  // and the address stays affine in the column block (one base register).
  static constexpr int VROW = C + 4;                        // chunks per padded V row
  static constexpr int VSLOTS = (BN * VROW + 63) / 64 * 64;
  static constexpr int VTILE = VSLOTS * 16;
  // DMA instructions every wave issues per tile (some waves issue one more);
  // the partial vmcnt waits count only these, so waves with more loads in
  // flight simply wait a little longer
  static constexpr int DMA_MIN = KSLOTS / NT + VSLOTS / NT;
  static_assert(QB == 2 || 2 * (KTILE + VTILE) * NS <= 160 * 1024, "two workgroups per CU");
};

template <int D>
struct Kernel {
  using Cfg = Bf16Cfg<D>;
  static constexpr int BN = Cfg::BN, QB = Cfg::QB, C = Cfg::C, NKC = Cfg::NKC, NDB = Cfg::NDB;
  typedef short s16x8 __attribute__((ext_vector_type(8)));

  // ---- K and V tiles: rows padded to KROW / VROW 16-byte slots
  using KLoader = BufLoader<Cfg::NT, Cfg::KROW, Cfg::KSLOTS, PaddedRows<C>>;
  using VLoader = BufLoader<Cfg::NT, Cfg::VROW, Cfg::VSLOTS, PaddedRows<C>>;

  // ---- K operands of one tile: row l32, chunk 2c + g
  static __device__ __forceinline__ void read_k(bf16x8 (&a)[NKC], const uint8_t* kst, int l32, int g) {
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      a[c] = *reinterpret_cast<const bf16x8*>(kst + 16 * (l32 * Cfg::KROW + 2 * c + g));
  }

  // ---- V^T operands of one tile: for 16-key step kc and 32-column block db
  static __device__ __forceinline__ void read_v(s16x8 (&a)[2][NDB], const uint8_t* vst, int v_row0, int v_col) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db) a[kc][db] = read_v_step(vst, kc * NDB + db, v_row0, v_col);
  }

  // ---- S^T = K Q^T for both query blocks (two independent MFMA chains)
  static __device__ __forceinline__ void s_mfma(f32x16 (&s)[QB], const bf16x8 (&a)[NKC],
                                                const bf16x8 (&qf)[QB][NKC]) {
#pragma unroll
    for (int h = 0; h < QB; ++h) s[h] = f32x16{};
#pragma unroll
    for (int c = 0; c < NKC; ++c)
#pragma unroll
      for (int h = 0; h < QB; ++h) s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], qf[h][c], s[h], 0, 0, 0);
  }

  // ---- O^T += V^T P^T for both query blocks
  static __device__ __forceinline__ void pv_mfma(f32x16 (&o)[QB][NDB], const s16x8 (&a)[2][NDB],
                                                 const bf16x8 (&pb)[QB][2]) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < QB; ++h)
          o[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kc][db]), pb[h][kc],
                                                             o[h][db], 0, 0, 0);
  }

  // ---- instruction interleaving hints for the scheduler (same basic block)
  // masks: 0x008 MFMA, 0x002 VALU, 0x080 any LDS, 0x100 LDS read
  static __device__ __forceinline__ void schedule_s_with_exp() {
    __builtin_amdgcn_sched_group_barrier(0x100, NKC, 0);
#pragma unroll
    for (int i = 0; i < QB * NKC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
  }
  static __device__ __forceinline__ void schedule_pv_with_max() {
    __builtin_amdgcn_sched_group_barrier(0x080, 4 * NDB, 0);
#pragma unroll
    for (int i = 0; i < 2 * QB * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
  }

  // ---- an empty asm that consumes the probabilities: the compiler must have
  // them in registers at this point, so it cannot sink their computation past
  // the following branch into the PV block
  static __device__ __forceinline__ void pin(bf16x8 (&pb)[QB][2], float (&psum)[QB]) {
#pragma unroll
    for (int h = 0; h < QB; ++h) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        i32x4 v = __builtin_bit_cast(i32x4, pb[h][k]);
        asm volatile("" : "+v"(v));
        pb[h][k] = __builtin_bit_cast(bf16x8, v);
      }
      asm volatile("" : "+v"(psum[h]));
    }
  }

  // ---- S(j+1) = K Q^T for both query blocks, interleaved in program order
  // with the probabilities of tile j: per d-chunk c, one K read two chunks
  // ahead, two MFMAs (one per query block), then four exponentials.
  static __device__ __forceinline__ void s_with_probs(f32x16 (&snext)[QB], const uint8_t* kst,
                                                      const bf16x8 (&qf)[QB][NKC], const f32x16 (&scur)[QB],
                                                      float scale_log2, const RowState (&st)[QB],
                                                      bf16x8 (&pb)[QB][2], float (&psum)[QB], int l32, int g) {
    constexpr int PER_C = (QB * 16 + NKC - 1) / NKC;  // exponentials per d-chunk
    const uint8_t* krow = kst + 16 * (l32 * Cfg::KROW + g);
    auto rd = [&](int c) { return *reinterpret_cast<const bf16x8*>(krow + 32 * c); };
    bf16x8 ka[3];
    ka[0] = rd(0);
    if (NKC > 1) ka[1] = rd(1);
#pragma unroll
    for (int h = 0; h < QB; ++h) snext[h] = f32x16{};
    float part[QB][2];
#pragma unroll
    for (int h = 0; h < QB; ++h) part[h][0] = part[h][1] = 0.0f;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if (c + 2 < NKC) ka[(c + 2) % 3] = rd(c + 2);
#pragma unroll
      for (int h = 0; h < QB; ++h)
        snext[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c % 3], qf[h][c], snext[h], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < PER_C; ++e) {
        const int idx = c * PER_C + e;  // element of the (QB x 16) probability tile
        if (idx < QB * 16) {
          const int h = idx / 16, i = idx % 16;
          pb[h][i / 8][i % 8] = (__bf16)fast_exp2(fmaf(scur[h][i], scale_log2, -st[h].m));
          if (i % 2 == 1) {
            // row sum of the bf16 probabilities PV actually uses, two at a time
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 pair = {pb[h][i / 8][i % 8 - 1], pb[h][i / 8][i % 8]};
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            part[h][(i / 2) % 2] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, part[h][(i / 2) % 2], false);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < QB; ++h) psum[h] = part[h][0] + part[h][1];
    pin(pb, psum);
  }

  // ---- O^T += V^T P^T for both query blocks, interleaved in program order
  // with the row max of tile j+1: per (kc, db) step, one V^T operand read two
  // steps ahead, two MFMAs, then a few max operations.
  static __device__ __forceinline__ s16x8 read_v_step(const uint8_t* vst, int step, int v_row0, int v_col) {
    const int kc = step / NDB, db = step % NDB;
    // rows 16 kc + v_row0 (+8), columns 32 db + v_col .. +3 of the padded tile
    const uint8_t* p0 = vst + 16 * Cfg::VROW * (16 * kc + v_row0) + 2 * (32 * db + v_col);
    const uint8_t* p1 = p0 + 16 * Cfg::VROW * 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p0));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p1));
    return s16x8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // `va0`, `va1`: the operands of steps 0 and 1, read early by the caller.
  static __device__ __forceinline__ void pv_with_max(f32x16 (&o)[QB][NDB], const uint8_t* vst,
                                                     const bf16x8 (&pb)[QB][2], const f32x16 (&snext)[QB],
                                                     float scale_log2, float (&mt)[QB], int v_row0, int v_col,
                                                     s16x8 va0, s16x8 va1) {
    constexpr int NSTEP = 2 * NDB;
    auto rd = [&](int step) { return read_v_step(vst, step, v_row0, v_col); };
    s16x8 va[3];
    va[0] = va0;
    va[1] = va1;
    float mx[QB];
#pragma unroll
    for (int h = 0; h < QB; ++h) mx[h] = snext[h][0];
    constexpr int PER_STEP = (QB * 15 + NSTEP - 1) / NSTEP;
#pragma unroll
    for (int step = 0; step < NSTEP; ++step) {
      if (step + 2 < NSTEP) va[(step + 2) % 3] = rd(step + 2);
      const int kc = step / NDB, db = step % NDB;
#pragma unroll
      for (int h = 0; h < QB; ++h)
        o[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[step % 3]), pb[h][kc],
                                                           o[h][db], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < PER_STEP; ++e) {
        const int idx = step * PER_STEP + e;  // element 1..15 of each block's max
        if (idx < QB * 15) {
          const int h = idx / 15, i = 1 + idx % 15;
          mx[h] = fmaxf(mx[h], snext[h][i]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < QB; ++h) mt[h] = half_swap_max(mx[h]) * scale_log2;
  }

  // ---- element mask: keys at or past a lane's limit get -inf
  static __device__ __forceinline__ void mask(f32x16 (&s)[QB], int k0, int g, const int (&mylim)[QB]) {
#pragma unroll
    for (int h = 0; h < QB; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i / 4) + 4 * g + (i % 4);
        if (key >= mylim[h]) s[h][i] = -INFINITY;
      }
  }

  // ---- tile max in log2 units per block, shared by both half-waves
  static __device__ __forceinline__ void tile_max(const f32x16 (&s)[QB], float scale_log2, float (&mt)[QB]) {
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      float mx = s[h][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[h][i]);
      mt[h] = half_swap_max(mx) * scale_log2;
    }
  }

  // ---- probabilities of a tile (bf16 B operands of PV) and their fp32 sums
  static __device__ __forceinline__ void probs(const f32x16 (&s)[QB], float scale_log2, const RowState (&st)[QB],
                                               bf16x8 (&pb)[QB][2], float (&psum)[QB]) {
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      float part[2] = {0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 16; ++i) pb[h][i / 8][i % 8] = (__bf16)fast_exp2(fmaf(s[h][i], scale_log2, -st[h].m));
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 pair = {pb[h][i / 8][i % 8], pb[h][i / 8][i % 8 + 1]};
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        part[(i / 2) % 2] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, part[(i / 2) % 2], false);
      }
      psum[h] = part[0] + part[1];
    }
  }
};

template <int D>
__global__ __launch_bounds__(kBf16BlockM * 2 / PVA_BF16_QB, 3 - PVA_BF16_QB) void fwd_bf16_kernel(const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          const int32_t* __restrict__ cu,
                                                          const WorkItem* __restrict__ items, int H,
                                                          float scale_log2, __bf16* __restrict__ O) {
  using Kn = Kernel<D>;
  using Cfg = typename Kn::Cfg;
  using s16x8 = typename Kn::s16x8;
  constexpr int BN = Cfg::BN, QB = Cfg::QB, NKC = Cfg::NKC, NDB = Cfg::NDB, NS = Cfg::NS;
  static_assert(NS == 4, "the loop below is unrolled for a ring of four stages");
  // separate arrays per stage: the compiler sees that an LDS DMA into one
  // stage and reads of another do not alias
  __shared__ __attribute__((aligned(1024))) uint8_t k0s[Cfg::KTILE], k1s[Cfg::KTILE], k2s[Cfg::KTILE], k3s[Cfg::KTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t v0s[Cfg::VTILE], v1s[Cfg::VTILE], v2s[Cfg::VTILE], v3s[Cfg::VTILE];
  uint8_t* const kst[NS] = {k0s, k1s, k2s, k3s};
  uint8_t* const vst[NS] = {v0s, v1s, v2s, v3s};

  const WorkItem it = items[blockIdx.x];
  if (it.seq < 0) return;  // empty slot; uniform over the workgroup

  // the wave index is uniform per wave; reading it through a scalar register
  // makes every per-wave condition below a scalar branch
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int T = it.text_len, L = it.seq_len;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive tokens of one head
  const uint32_t rs2 = uint32_t(rs) * 2u;  // bytes (the planner keeps L * rs2 below 2^31)
  // bytes from a head's first row of the sequence to the end of its last row
  const uint32_t head_bytes = uint32_t(L - 1) * rs2 + 2u * D;
  const int64_t base = int64_t(cu[it.seq]) * rs + int64_t(it.head) * D;
  const __bf16* Qh = Q + base;
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(K + base);
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(V + base);

  // this lane's query rows (one per block) and their key limits; rows past
  // the sequence end act as image rows (their outputs are never stored)
  const int wrow0 = it.q0 + 32 * QB * wave;
  int qrow[QB], mylim[QB];
#pragma unroll
  for (int h = 0; h < QB; ++h) {
    qrow[h] = wrow0 + 32 * h + l32;
    mylim[h] = key_limit(qrow[h], T, L);
  }
  const int wlim_min = key_limit(wrow0, T, L);  // smallest key limit of the wave's rows
  const int kend = it.k_end;

  // prologue DMA in the order the tiles are needed: K0 K1 V0 | K2 V1 | K3 V2
  // (tile t's resource starts at key row t * BN and ends with the sequence)
  typename Kn::KLoader kld;
  typename Kn::VLoader vld;
  // V's extra DMA rounds go to the waves that issue none for K
  const int vwave = (wave + Cfg::NW / 2) % Cfg::NW;
  kld.init(rs2, lane, wave);
  vld.init(rs2, lane, vwave);
  auto ld_k = [&](int t, uint8_t* stage) {
    const uint32_t o = uint32_t(t * BN) * rs2;
    kld.load(make_rsrc(Kb + o, head_bytes - o), stage, wave);
  };
  auto ld_v = [&](int t, uint8_t* stage) {
    const uint32_t o = uint32_t(t * BN) * rs2;
    vld.load(make_rsrc(Vb + o, head_bytes - o), stage, vwave);
  };
  if (kend > 0) ld_k(0, kst[0]);
  if (kend > 1) ld_k(1, kst[1]);
  if (kend > 0) ld_v(0, vst[0]);
  if (kend > 2) ld_k(2, kst[2]);
  if (kend > 1) ld_v(1, vst[1]);
  if (kend > 3) ld_k(3, kst[3]);
  if (kend > 2) ld_v(2, vst[2]);

  // Q^T operands: chunk c holds d = 16c + 8g .. +7 of this lane's query rows
  bf16x8 qf[QB][NKC];
#pragma unroll
  for (int h = 0; h < QB; ++h)
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      if (qrow[h] < L)
        qf[h][c] = *reinterpret_cast<const bf16x8*>(Qh + int64_t(qrow[h]) * rs + 16 * c + 8 * g);
      else
        qf[h][c] = bf16x8{};
    }

  f32x16 oacc[QB][NDB];
#pragma unroll
  for (int h = 0; h < QB; ++h)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[h][db] = f32x16{};
  RowState st[QB];
#pragma unroll
  for (int h = 0; h < QB; ++h) st[h] = RowState{-INFINITY, 0.0f};

  // per-lane constant parts of the V^T (transpose-read) addresses
  const int v_row0 = 4 * g + (lane & 15) / 4;
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // K0, K1, V0 must have landed; K2 V1 K3 V2 may still be in flight
  if (kend > 3)
    wait_vmcnt<2 * Cfg::DMA_MIN>();
  else
    wait_vmcnt<0>();
  lds_barrier();

  f32x16 sa[QB], sb[QB];
  // S(0) and its reference max. Rows past the sequence end, and tiles past a
  // row's key limit, are computed masked: their probabilities are exactly
  // zero. That keeps every branch in the loop scalar and rare.
  if (kend > 0) {
    bf16x8 ka[NKC];
    Kn::read_k(ka, kst[0], l32, g);
    Kn::s_mfma(sa, ka, qf);
    if (BN > wlim_min) Kn::mask(sa, 0, g, mylim);
    float mt[QB];
    Kn::tile_max(sa, scale_log2, mt);
#pragma unroll
    for (int h = 0; h < QB; ++h) st[h].m = mt[h];  // first tile: O and l are still zero
  }

  // Iteration j; `scur` holds S(j), `snext`
  // receives S(j+1). SJ = j % NS (compile-time in each unrolled copy). The
  // rare branches (element mask, rescale) are marked unlikely so that the
  // common path falls through without a taken branch.
  auto iteration = [&](auto sj_tag, int j, f32x16(&scur)[QB], f32x16(&snext)[QB]) {
    constexpr int SJ = decltype(sj_tag)::value;
    lds_barrier();  // every wave is done with S(j) (K stage SJ) and PV(j-1) (V stage SJ-1)
    const bool steady = j + NS < kend;
    if (steady) ld_k(j + NS, kst[SJ]);
    if (j + NS - 1 < kend) ld_v(j + NS - 1, vst[(SJ + NS - 1) % NS]);
    const int k1 = (j + 1) * BN;
    // the first two V^T operands of PV(j): their LDS latency hides behind block A
    const s16x8 va0 = Kn::read_v_step(vst[SJ], 0, v_row0, v_col);
    const s16x8 va1 = Kn::read_v_step(vst[SJ], 1, v_row0, v_col);
    // S(j+1) MFMAs interleaved with the exponentials of tile j
    bf16x8 pb[QB][2];
    float psum[QB];
    Kn::s_with_probs(snext, kst[(SJ + 1) % NS], qf, scur, scale_log2, st, pb, psum, l32, g);
#pragma unroll
    for (int h = 0; h < QB; ++h) st[h].l += psum[h];
    if (__builtin_expect(k1 + BN > wlim_min, 0)) Kn::mask(snext, k1, g, mylim);
    // PV(j) MFMAs interleaved with the row max of tile j+1
    float mt[QB];
    Kn::pv_with_max(oacc, vst[SJ], pb, snext, scale_log2, mt, v_row0, v_col, va0, va1);
#pragma unroll
    for (int h = 0; h < QB; ++h) {
      const bool need = mt[h] > st[h].m + kLazyRescale;
      if (__builtin_expect(wave_any(need), 0)) {
        // per-lane decision: a lane that does not need it keeps its max (alpha = 1
        // exactly), so each row's arithmetic depends on its own scores only
        const float alpha = need ? fast_exp2(st[h].m - mt[h]) : 1.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[h][db][i] *= alpha;
        st[h].l *= alpha;
        st[h].m = need ? mt[h] : st[h].m;
      }
    }
    // K(j+2) and V(j+1) are needed next; the loads of iterations j-1 and j
    // may stay in flight in steady state
    if (steady)
      wait_vmcnt<2 * Cfg::DMA_MIN>();
    else
      wait_vmcnt<0>();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // Four unrolled iterations per trip, each guarded; the last tile's
  // iteration also computes S of the tile after it on a stale stage, which
  // the mask turns entirely into -inf (no effect on the result).
  for (int j = 0; j < kend; j += 4) {
    iteration(I0{}, j, sa, sb);
    if (j + 1 >= kend) break;
    iteration(I1{}, j + 1, sb, sa);
    if (j + 2 >= kend) break;
    iteration(I2{}, j + 2, sa, sb);
    if (j + 3 >= kend) break;
    iteration(I3{}, j + 3, sb, sa);
  }

  // ---- epilogue: O = O^T / l, bf16, rows of this sequence only
#pragma unroll
  for (int h = 0; h < QB; ++h) {
    const float lt = half_swap_sum(st[h].l);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qrow[h] < L) {
      __bf16* orow = O + base + int64_t(qrow[h]) * rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[h][db][4 * i4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * i4 + 4 * g) = w;
        }
    }
  }
}

template <int D>
int launch(const void* q, const void* k, const void* v, const int32_t* cu, const pva_seg_desc* d, float scale,
           void* out, hipStream_t stream) {
  using Cfg = Bf16Cfg<D>;
  const int n = static_cast<int>(d->plan.items.size());
  if (n == 0) return PVA_OK;
  const float scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634);
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(n), dim3(Cfg::NT), 0, stream, static_cast<const __bf16*>(q),
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), cu,
                     static_cast<const WorkItem*>(d->d_items), d->plan.num_heads, scale_log2,
                     static_cast<__bf16*>(out));
  return hipGetLastError() == hipSuccess ? PVA_OK : PVA_ERR_HIP;
}

}  // namespace

int launch_fwd_bf16(const void* q, const void* k, const void* v, const int32_t* cu, const pva_seg_desc* d,
                    float scale, void* out, hipStream_t stream) {
  switch (d->plan.head_dim) {
    case 64: return launch<64>(q, k, v, cu, d, scale, out, stream);
    case 128: return launch<128>(q, k, v, cu, d, scale, out, stream);
    default: return PVA_ERR_UNSUPPORTED;
  }
}

}  // namespace pva
