// Log-sum-exp merge of partial attention results.
//
// Combines the per-chunk pieces of a row into the full-context result, the
// step that the ring of the CP section accumulates into ("Scaling LLM
// Inference", soumitrasaha.com reader notes, "The communication bottleneck
// across all three axes"): with M = max_c lse_c and w_c = exp(lse_c - M),
// out = sum_c w_c O_c / sum_c w_c and lse = M + ln(sum_c w_c).
//
// Bandwidth bound: D/4 threads per row, each streaming 16 bytes of every
// partial; sums run in partial order (deterministic).
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeLaunch a) {
  constexpr int TPR = D / 4;          // threads per row
  constexpr int RPB = 256 / TPR;      // rows per workgroup
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int64_t rows = (int64_t)a.B * a.S * a.H;
  if (row >= rows) return;
  const int h = (int)(row % a.H);
  const int64_t bs = row / a.H;
  const int s = (int)(bs % a.S);
  const int b = (int)(bs / a.S);

  const int64_t loff = b * a.pl_sb + s * a.pl_ss + h * a.pl_sh;
  const int64_t ooff = b * a.p_sb + s * a.p_ss + h * a.p_sh + 4 * part;
  float M = kNegInf;
  for (int c = 0; c < a.n; ++c) M = fmaxf(M, a.lse[c][loff]);

  f32x4 acc = (f32x4){};
  float den = 0.f;
  if (M != kNegInf) {
    for (int c = 0; c < a.n; ++c) {
      const float w = fast_exp2((a.lse[c][loff] - M) * kLog2e);
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.o[c] + ooff);
      den += w;
      acc[0] = fmaf(w, v[0], acc[0]);
      acc[1] = fmaf(w, v[1], acc[1]);
      acc[2] = fmaf(w, v[2], acc[2]);
      acc[3] = fmaf(w, v[3], acc[3]);
    }
  }
  const float inv = (den > 0.f) ? 1.f / den : 0.f;
  const f32x4 r = acc * inv;
  const int64_t out_off = b * a.o_sb + s * a.o_ss + h * a.o_sh + 4 * part;
  if (a.out_bf16) {
    const u32x2 pk = {pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(a.out) + out_off) = pk;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + out_off) = r;
  }
  if (a.out_lse != nullptr && part == 0)
    a.out_lse[b * a.ol_sb + s * a.ol_ss + h * a.ol_sh] = (den > 0.f) ? M + fast_log2(den) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_merge(const MergeLaunch& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.S * a.H;
  if (rows <= 0) return hipSuccess;
  const int tpr = a.D / 4;
  const long long blocks = (rows * tpr + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.D == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
