// A C++ program that uses the library through include/pva.h and the HIP
// runtime only (no Python): it builds a descriptor, runs the bf16 forward on
// device buffers it allocates itself, and checks the result against closed
// forms of the masked softmax ("[RFC]: HunyuanImage 3.0 deployment",
// Proposed Change P0 and Model structure item 1: causal text rows, image
// rows that see the whole text prefix and their image block):
//   * with every key row zero all allowed scores are equal, so a text row i
//     returns the mean of V rows 0..i and an image row the mean of all L
//     rows of its sequence;
//   * text row 0 sees key 0 only, so its output is v_0 bitwise.
// It also checks the useful-FLOP count against 4 D H sum(T(T+1)/2 + I L)
// and that invalid arguments come back as status codes with a message.
// Exit status 0 when every check passes.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "pva.h"

namespace {

int failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

// float -> bf16 bits, round to nearest even (finite inputs)
uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

float from_bf16(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

bool hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::fprintf(stderr, "FAIL: %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  int ndev = 0;
  if (!hip_ok(hipGetDeviceCount(&ndev), "hipGetDeviceCount") || ndev < 1) return 2;

  // three sequences: text + image, text only, image only
  const int32_t text_len[] = {37, 70, 0};
  const int32_t image_len[] = {150, 0, 90};
  const int32_t nseq = 3, H = 3, D = 128;
  std::vector<int32_t> off(nseq + 1, 0);
  for (int s = 0; s < nseq; ++s) off[s + 1] = off[s] + text_len[s] + image_len[s];
  const int64_t N = off[nseq];
  const size_t elems = size_t(N) * H * D;

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 2;
  pva_seg_desc* desc = nullptr;
  check(pva_seg_desc_build(text_len, image_len, nseq, H, D, PVA_BF16, stream, &desc) == PVA_OK, "descriptor");
  if (!desc) return 1;

  int64_t want = 0;
  for (int s = 0; s < nseq; ++s) {
    const int64_t T = text_len[s], I = image_len[s];
    want += T * (T + 1) / 2 + I * (T + I);
  }
  check(pva_seg_desc_useful_flops(desc) == 4 * int64_t(D) * H * want, "useful FLOPs");
  const int32_t* host_cu = nullptr;
  int32_t cu_len = 0;
  check(pva_seg_desc_cu_seqlens(desc, &host_cu, &cu_len) == PVA_OK && cu_len == nseq + 1, "cu_seqlens");
  for (int s = 0; host_cu && s <= nseq; ++s) check(host_cu[s] == off[s], "cu_seqlens values");

  // Q random, K zero, V random (bf16)
  std::mt19937 gen(1234);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  std::vector<uint16_t> hq(elems), hk(elems, 0), hv(elems), ho(elems, 0);
  for (auto& x : hq) x = to_bf16(nd(gen));
  for (auto& x : hv) x = to_bf16(nd(gen));

  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dout = nullptr, *dcu = nullptr;
  const size_t bytes = elems * sizeof(uint16_t);
  bool ok = hip_ok(hipMalloc(&dq, bytes), "hipMalloc q") && hip_ok(hipMalloc(&dk, bytes), "hipMalloc k") &&
            hip_ok(hipMalloc(&dv, bytes), "hipMalloc v") && hip_ok(hipMalloc(&dout, bytes), "hipMalloc out") &&
            hip_ok(hipMalloc(&dcu, sizeof(int32_t) * (nseq + 1)), "hipMalloc cu");
  ok = ok && hip_ok(hipMemcpy(dq, hq.data(), bytes, hipMemcpyHostToDevice), "copy q") &&
       hip_ok(hipMemcpy(dk, hk.data(), bytes, hipMemcpyHostToDevice), "copy k") &&
       hip_ok(hipMemcpy(dv, hv.data(), bytes, hipMemcpyHostToDevice), "copy v") &&
       hip_ok(hipMemcpy(dcu, off.data(), sizeof(int32_t) * (nseq + 1), hipMemcpyHostToDevice), "copy cu");
  if (!ok) return 2;

  const float scale = 1.0f / std::sqrt(float(D));
  check(packed_attn_fwd(dq, dk, dv, static_cast<const int32_t*>(dcu), desc, scale, dout, stream) == PVA_OK,
        "packed_attn_fwd");
  if (!hip_ok(hipStreamSynchronize(stream), "synchronize") ||
      !hip_ok(hipMemcpy(ho.data(), dout, bytes, hipMemcpyDeviceToHost), "copy out"))
    return 2;

  // closed forms: the mean of the V rows each query row may see
  double worst = 0.0;
  std::vector<double> sum(size_t(H) * D);
  for (int s = 0; s < nseq; ++s) {
    const int T = text_len[s], L = off[s + 1] - off[s];
    std::fill(sum.begin(), sum.end(), 0.0);
    std::vector<std::vector<double>> prefix_mean(L);
    for (int r = 0; r < L; ++r) {  // running sums over key rows 0..r
      for (size_t e = 0; e < sum.size(); ++e) sum[e] += from_bf16(hv[(size_t(off[s]) + r) * H * D + e]);
      if (r < T || r == L - 1) {
        prefix_mean[r].resize(sum.size());
        for (size_t e = 0; e < sum.size(); ++e) prefix_mean[r][e] = sum[e] / (r + 1);
      }
    }
    for (int r = 0; r < L; ++r) {
      const std::vector<double>& ref = r < T ? prefix_mean[r] : prefix_mean[L - 1];
      for (size_t e = 0; e < ref.size(); ++e) {
        const double got = from_bf16(ho[(size_t(off[s]) + r) * H * D + e]);
        const double err = std::fabs(got - ref[e]);
        // bf16 output rounding (2^-9 relative) plus fp32 accumulation
        if (err > std::ldexp(std::fabs(ref[e]), -8) + 1e-4) {
          if (failures < 5) std::fprintf(stderr, "seq %d row %d elem %zu: %g vs %g\n", s, r, e, got, ref[e]);
          check(false, "mean of the visible V rows");
        }
        worst = std::fmax(worst, err);
      }
    }
    if (T > 0)  // text row 0 sees key 0 only
      check(std::memcmp(&ho[size_t(off[s]) * H * D], &hv[size_t(off[s]) * H * D], sizeof(uint16_t) * H * D) == 0,
            "text row 0 is v_0 bitwise");
  }

  // invalid arguments: status codes and a message, nothing launched
  check(packed_attn_fwd(nullptr, dk, dv, static_cast<const int32_t*>(dcu), desc, scale, dout, stream) ==
            PVA_ERR_INVALID_ARG, "NULL q refused");
  check(std::strlen(pva_last_error()) > 0, "error message set");
  check(packed_attn_fwd(dq, dk, dv, static_cast<const int32_t*>(dcu), desc, -1.0f, dout, stream) ==
            PVA_ERR_INVALID_ARG, "negative scale refused");
  check(packed_attn_fwd(dq, dk, dv, static_cast<const int32_t*>(dcu), nullptr, scale, dout, stream) ==
            PVA_ERR_INVALID_ARG, "NULL descriptor refused");

  pva_seg_desc_free(desc);
  (void)hipFree(dq);
  (void)hipFree(dk);
  (void)hipFree(dv);
  (void)hipFree(dout);
  (void)hipFree(dcu);
  (void)hipStreamDestroy(stream);
  std::printf("abi_consumer: %s (%lld rows, max |O - closed form| %.3e, %s)\n", failures ? "FAILED" : "ok",
              static_cast<long long>(N), worst, pva_version());
  return failures ? 1 : 0;
}
