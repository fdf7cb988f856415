// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pva_internal.h"

namespace pva {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define PVA_LDS __attribute__((address_space(3)))

// Softmax scores are kept in log2 units; the running max is only raised when
// a tile's max exceeds it by more than this many units, so probabilities stay
// below 2^kLazyRescale and O/l are rescaled rarely. Exact up to rounding: O
// and l always share the same reference max.
constexpr float kLazyRescale = 8.0f;

// Maximum over the two 32-lane halves of a wave: permlane32_swap(x, x) hands
// each lane its own value and its partner's (lane ^ 32) in some order.
// (IEEE maximum: no canonicalisation of the MFMA results it reads)
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with vmcnt = N and the other counters untouched (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 7, lgkmcnt 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup timeline of the timing build (the library compiled with
// PVA_WG_TIMELINE, libpva_timeline.so). Thread 0 of each work item's
// workgroup keeps the real-time counter (100 MHz) at the workgroup's start,
// after its prologue, after its tile loop and at its end, the shader-clock
// counter after the prologue and after the loop, and stores them with the
// hardware ids of its CU and XCD into record blockIdx.x of its kernel's
// buffer (layout in include/pva.h, pva_timeline_read). In the library's own
// build the struct is empty and every call compiles to nothing.
struct WgTimeline {
#ifdef PVA_WG_TIMELINE
  uint64_t t0 = 0, t1 = 0, t2 = 0, c1 = 0, c2 = 0;
  __device__ __forceinline__ void start() { t0 = __builtin_amdgcn_s_memrealtime(); }
  __device__ __forceinline__ void prologue_done() {
    t1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void loop_done() {
    t2 = __builtin_amdgcn_s_memrealtime();
    c2 = __builtin_amdgcn_s_memtime();
  }
  // `buf`: the kernel's record array; `tiles`: the first wave's key tiles;
  // `kend`: the item's key tiles
  __device__ __forceinline__ void finish(unsigned long long* buf, int tiles, int kend) const {
    const uint64_t t3 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x != 0 || blockIdx.x >= PVA_TIMELINE_MAX_ITEMS) return;
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    unsigned long long* r = buf + uint64_t(PVA_TIMELINE_FIELDS) * blockIdx.x;
    r[0] = t0;
    r[1] = t1;
    r[2] = t2;
    r[3] = t3;
    r[4] = c1;
    r[5] = c2;
    r[6] = hw;
    r[7] = xcc;
    r[8] = uint64_t(tiles);
    r[9] = uint64_t(kend);
    r[10] = blockIdx.x;
    r[11] = 1;  // record written
  }
#else
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void prologue_done() {}
  __device__ __forceinline__ void loop_done() {}
  __device__ __forceinline__ void finish(unsigned long long*, int, int) const {}
#endif
};

// Workgroup barrier without the global-memory fence __syncthreads() implies
// (that fence would also wait for every DMA still in flight). LDS reads issued
// before it have been consumed by then; the memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// tile_range_bytes(span, offset) = span - min(offset, span) for wave-uniform
// values, on the scalar unit (the compiler forms that saturating subtract on
// the vector unit and reads it back with v_readfirstlane; here: s_min_u32
// then s_sub_u32, the same two operations)
__device__ __forceinline__ uint32_t tile_range_bytes_uniform(uint32_t span, uint32_t offset) {
  uint32_t r;
  asm("s_min_u32 %0, %1, %2\n\ts_sub_u32 %0, %2, %0" : "=&s"(r) : "s"(offset), "s"(span) : "scc");
  return r;
}

// Per-lane state of the online softmax for one query column.
struct RowState {
  float m;  // reference max (log2 units); O and l are relative to it
  float l;  // this lane's partial row sum (the other half-wave holds the rest)
};

// Buffer resource over the bytes [base, base + bytes) (raw, no stride):
// loads at offsets at or past `bytes` return zeros instead of touching
// memory. gfx9 resource word 3 (data format 32, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// An offset that is out of range of every resource built by make_rsrc for
// fewer than 2^31 bytes: its loads write zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Global -> LDS DMA of one key tile through a buffer resource whose range
// ends at the last byte of the sequence's rows of this head: rows past the
// sequence end read as zeros, so the tile needs neither clamping nor a slow
// path. The tile occupies SLOTS 16-byte slots (ROW per key row, SLOTS a
// multiple of 64); lane `lane` of wave-round (i, wave) fills slot
// NT * i + 64 * wave + lane. Slot s holds chunk Map::chunk(r, s % ROW) of tile
// row r = s / ROW; pad slots (chunk -1) get an out-of-range offset and are
// written with zeros. A wave whose round starts past the tile skips it (a
// scalar branch). Per lane, only a constant 32-bit offset per round is kept.
template <int NT, int ROW, int SLOTS, typename Map>
struct BufLoader {
  static_assert(SLOTS % 64 == 0, "whole-wave rounds");
  static constexpr int ROUNDS = (SLOTS + NT - 1) / NT;
  uint32_t off[ROUNDS];
  __device__ __forceinline__ void init(uint32_t rs2, int lane, int wave) {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int s = NT * i + 64 * wave + lane;
      const int r = s / ROW, c = Map::chunk(r, s % ROW);
      off[i] = (s < SLOTS && c >= 0) ? uint32_t(r) * rs2 + 16u * uint32_t(c) : kOutOfRange;
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, uint8_t* stage, int wave) const {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i) {
      const int s0 = NT * i + 64 * wave;
      if (NT * (i + 1) > SLOTS && s0 >= SLOTS) continue;  // only the last round can be partial
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (PVA_LDS void*)(stage + 16 * s0), 16, off[i], 0, 0, 0);
    }
  }
};

// Epilogue of one query row: the lane holds elements 32 db + 8 i4 + 4 g + e
// (db < NDB, i4 < 4, e < 4) of the row's unnormalised O^T; inv = scale / l
// (0 for a row with no key), lse_c the row's log-sum-exp (natural log, -inf
// for no key). With a running result (out.acc_o), the two combine as two key
// sets of one softmax ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change
// P2, Ring-Attention Integration): lse = log(e^lse_acc + e^lse_c),
// O = e^(lse_acc - lse) O_acc + e^(lse_c - lse) O_c. Rows of o and lse are
// orow (element offset of the row's first element) and lrow (row * H + head).
template <int NDB>
__device__ __forceinline__ void write_row(const OutSpec& out, int64_t orow, int64_t lrow, int g,
                                          const f32x16 (&oacc)[NDB], float inv, float lse_c) {
  // value(group, O elements) of the lane's 4-element groups (group
  // 4 db + i4 holds columns 32 db + 8 i4 + 4 g .. +3), stored as fp32 or bf16
  auto store = [&](auto value) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = 32 * db + 8 * i4 + 4 * g;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = oacc[db][4 * i4 + e];
        w = value(4 * db + i4, w);
        if (out.o_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out.o) + orow + col) = w;
        } else {
          bf16x4 b;
#pragma unroll
          for (int e = 0; e < 4; ++e) b[e] = (__bf16)w[e];
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out.o) + orow + col) = b;
        }
      }
  };
  if (!out.acc_o) {
    store([&](int, f32x4 w) { return w * inv; });
    if (out.lse && g == 0) out.lse[lrow] = lse_c;
    return;
  }
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  // the running row and its log-sum-exp are read together (one memory round
  // trip); the row is used only where the log-sum-exp says it holds a result
  const float lp = out.acc_lse[lrow];
  f32x4 prev[NDB * 4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      prev[4 * db + i4] = *reinterpret_cast<const f32x4*>(out.acc_o + orow + 32 * db + 8 * i4 + 4 * g);
  const float mx = __builtin_elementwise_maximum(lp, lse_c);
  float wc = 0.0f, wp = 0.0f, lse_out = -INFINITY;
  if (mx > -INFINITY) {
    const float ep = fast_exp2((lp - mx) * kLog2e), ec = fast_exp2((lse_c - mx) * kLog2e);
    const float sum = ep + ec, rs = 1.0f / sum;
    wp = ep * rs;
    wc = inv * (ec * rs);
    lse_out = mx + kLn2 * __log2f(sum);
  }
  // (a row the running result has not reached takes nothing from acc_o,
  // whatever it holds: NaN there must not reach the result)
  const bool use_prev = wp > 0.0f;
  store([&](int grp, f32x4 w) { return w * wc + (use_prev ? prev[grp] * wp : f32x4{}); });
  if (out.lse && g == 0) out.lse[lrow] = lse_out;
}

}  // namespace pva
