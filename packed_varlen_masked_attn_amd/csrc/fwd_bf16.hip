// Packed mixed-mask attention forward for gfx950: bf16 in, fp32 accumulate,
// bf16 out.
//
// Operation: "[RFC]: HunyuanImage 3.0 deployment", Proposed Change P0 (packed
// cu_seqlens attention over requests of mixed resolution; its attention mask
// challenge) and Model structure item 1 (Generalized Causal Attention: causal
// text prefix, bidirectional image block that sees the whole prefix).
//
// One workgroup = 4 waves = one work item (sequence, head, 128 query rows);
// each wave owns 32 query rows. Key/value tiles of 64 keys are streamed
// through double-buffered LDS, the next tile's global loads in flight while
// the current one is consumed.
//
// Per wave and key tile, on 32x32x16 bf16 MFMA:
//   S^T[key, q] = K Q^T    A = K from LDS (16-byte reads), B = Q^T held in
//                          registers for the whole item. Each lane then owns
//                          one query column and 16 keys per 32-key block, so
//                          row max / row sum are in-lane plus one exchange
//                          between the two 32-lane halves.
//   online softmax in fp32, log2 domain, lazy rescaling of O and l.
//   O^T[d, q] += V^T P^T   B = P^T straight from the S^T accumulators (cast to
//                          bf16, no shuffle: the contraction order of the keys
//                          is permuted instead), A = V^T read from the
//                          row-major V tile with ds_read_b64_tr_b16.
// Tiles the mask fully hides are never loaded; tiles it fully allows skip the
// element mask.
#include "kernel_common.h"

namespace pva {

namespace {

template <int D>
struct Bf16Cfg {
  static constexpr int BM = 128, BN = 64, NW = 4, NT = 256;
  static constexpr int C = D / 8;     // 16-byte chunks per K/V row
  static constexpr int NKC = D / 16;  // MFMA k-steps over the head dimension for S^T
  static constexpr int NDB = D / 32;  // 32-row blocks of O^T
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int NLD = BN * C / NT;  // 16-byte loads per thread per tensor per tile
  static constexpr int SMEM = 2 * 2 * TILE_BYTES;  // double-buffered K and V
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          const int32_t* __restrict__ cu,
                                                          const WorkItem* __restrict__ items, int H,
                                                          float scale_log2, __bf16* __restrict__ O) {
  using Cfg = Bf16Cfg<D>;
  constexpr int BN = Cfg::BN, C = Cfg::C, NKC = Cfg::NKC, NDB = Cfg::NDB, NLD = Cfg::NLD;
  constexpr int TB = Cfg::TILE_BYTES;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const WorkItem it = items[blockIdx.x];
  if (it.seq < 0) return;  // empty slot; uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int T = it.text_len, L = it.seq_len;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive tokens of one head
  const int64_t base = int64_t(cu[it.seq]) * rs + int64_t(it.head) * D;
  const __bf16* Qh = Q + base;
  const __bf16* Kh = K + base;
  const __bf16* Vh = V + base;

  // this lane's query row and its key limit; rows past the sequence end act
  // as image rows (their outputs are never stored)
  const int qrow = it.q0 + 32 * wave + l32;
  const int mylim = key_limit(qrow, T, L);
  const int wrow0 = it.q0 + 32 * wave;
  const bool wave_active = wrow0 < L;
  const int wlim_min = key_limit(wrow0, T, L);
  const int wlim_max = wave_active ? key_limit(min(wrow0 + 31, L - 1), T, L) : 0;

  // Q^T operand: chunk c holds d = 16c + 8g .. +7 of this lane's query row
  bf16x8 qf[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) {
    if (qrow < L)
      qf[c] = *reinterpret_cast<const bf16x8*>(Qh + int64_t(qrow) * rs + 16 * c + 8 * g);
    else
      qf[c] = bf16x8{};
  }

  uint4 kst[NLD], vst[NLD];
  auto gload = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int u = tid + Cfg::NT * i, r = u / C, c = u % C, key = k0 + r;
      if (key < L) {
        kst[i] = *reinterpret_cast<const uint4*>(Kh + int64_t(key) * rs + 8 * c);
        vst[i] = *reinterpret_cast<const uint4*>(Vh + int64_t(key) * rs + 8 * c);
      } else {
        kst[i] = uint4{0, 0, 0, 0};
        vst[i] = uint4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* kb = smem + buf * 2 * TB;
    uint8_t* vb = kb + TB;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int u = tid + Cfg::NT * i, r = u / C, c = u % C;
      *reinterpret_cast<uint4*>(kb + 16 * (r * C + (c ^ swz_k<C>(r)))) = kst[i];
      *reinterpret_cast<uint4*>(vb + 16 * (r * C + (c ^ swz_v<C>(r)))) = vst[i];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  // per-lane constant parts of the V^T (transpose-read) addresses
  const int v_row0 = 4 * g + (lane & 15) / 4;
  const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  const int kend = it.k_end;
  if (kend > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < kend; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kend) gload(kt + 1);
    const int k0 = kt * BN;
    if (k0 < wlim_max) {
      const uint8_t* kb = smem + buf * 2 * TB;
      const uint8_t* vb = kb + TB;
      // ---- S^T = K Q^T for keys k0 .. k0+63 (two 32-key blocks)
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int r = 32 * b + l32;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + 16 * (r * C + ((2 * c + g) ^ swz_k<C>(r))));
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sacc[b], 0, 0, 0);
        }
      }
      // ---- element mask on tiles the mask does not fully allow for this wave
      if (k0 + BN > wlim_min) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * b + 8 * (i / 4) + 4 * g + (i % 4);
            if (key >= mylim) sacc[b][i] = -INFINITY;
          }
      }
      // ---- online softmax (log2 domain)
      float mx = sacc[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[b][i]);
      mx = half_swap_max(mx);
      const float mt = mx * scale_log2;
      const bool need = mt > m_run + kLazyRescale;
      if (wave_any(need)) {
        // per-lane decision: a lane that does not need it keeps its max (alpha = 1
        // exactly), so each row's arithmetic depends on its own scores only
        const float mnew = need ? mt : m_run;
        const float alpha = need ? fast_exp2(m_run - mnew) : 1.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        l_run *= alpha;
        m_run = mnew;
      }
      bf16x8 pb[4];
      float psum = 0.0f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[b][i], scale_log2, -m_run));
          psum += p;
          pb[2 * b + i / 8][i % 8] = (__bf16)p;
        }
      l_run += psum;
      // ---- O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + v_col;
          const int chunk = col >> 3, boff = 2 * (col & 7);
          const int r0 = 16 * kc + v_row0, r1 = r0 + 8;
          const uint8_t* p0 = vb + 16 * (r0 * C + (chunk ^ swz_v<C>(r0))) + boff;
          const uint8_t* p1 = vb + 16 * (r1 * C + (chunk ^ swz_v<C>(r1))) + boff;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PVA_LDS s16x4*)(p1));
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 a16 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 a = __builtin_bit_cast(bf16x8, a16);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], oacc[db], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < kend) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, bf16, rows of this sequence only
  if (wave_active) {
    const float lt = half_swap_sum(l_run);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    if (qrow < L) {
      __bf16* orow = O + base + int64_t(qrow) * rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[db][4 * i4 + e] * inv);
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
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_bf16_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::SMEM) != hipSuccess)
      return PVA_ERR_HIP;
    attr_set = true;
  }
  const float scale_log2 = static_cast<float>(double(scale) * 1.4426950408889634);
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3(n), dim3(Cfg::NT), Cfg::SMEM, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), cu,
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
