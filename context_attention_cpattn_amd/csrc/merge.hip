// Log-sum-exp merge of partial attention results.
//
// Combines the per-chunk pieces of a row into the full-context result, the
// step that the ring of the CP section accumulates into ("Scaling LLM
// Inference", soumitrasaha.com reader notes, "The communication bottleneck
// across all three axes"): with M = max_c lse_c and w_c = exp(lse_c - M),
// out = sum_c w_c O_c / sum_c w_c and lse = M + ln(sum_c w_c).
//
// Bandwidth bound: D/4 threads per row, each streaming 16 bytes of every
// partial, eight partials' loads in flight at a time; sums run in partial
// order (deterministic).
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

// One row's merge, shared by both kernels (and built from the same pieces as
// the chunk walk's merge tail) so they round identically.  The partials'
// LSEs give M first; then the O pieces are read in batches of 8 (all loads
// of a batch issued before any is used, for memory-level parallelism) and
// accumulated in partial order.  o_at(c) / l_at(c) give the c-th partial's
// 16 bytes of this thread and its LSE.
template <class OAt, class LAt>
__device__ __forceinline__ void merge_row(int n, OAt o_at, LAt l_at, f32x4& res, float& M, float& den) {
  M = kNegInf;
  for (int c = 0; c < n; ++c) M = fmaxf(M, l_at(c));
  f32x4 acc = (f32x4){};
  den = 0.f;
  if (M != kNegInf) {
    for (int c0 = 0; c0 < n; c0 += 8) {
      f32x4 v[8];
      float lw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < n) {
          v[u] = o_at(c0 + u);
          lw[u] = l_at(c0 + u);
        }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u < n) {
          const float w = merge_weight(lw[u], M);
          den += w;
          merge_acc(acc, w, v[u]);
        }
    }
  }
  res = acc * merge_inv(den);
}

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
  f32x4 r;
  float M, den;
  merge_row(
      a.n, [&](int c) { return *reinterpret_cast<const f32x4*>(a.o[c] + ooff); }, [&](int c) { return a.lse[c][loff]; },
      r, M, den);
  store_row(a.out, a.out_bf16, b * a.o_sb + s * a.o_ss + h * a.o_sh + 4 * part, r);
  if (a.out_lse != nullptr && part == 0)
    a.out_lse[b * a.ol_sb + s * a.ol_ss + h * a.ol_sh] = merged_lse(M, den);
}

template <int D>
__global__ __launch_bounds__(256) void ring_merge_kernel(const RingMergeLaunch a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int part = tid % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int64_t per_owner = (int64_t)a.B * a.C * a.H;
  if (row >= per_owner * a.P) return;
  const int i = (int)(row / per_owner);
  const int64_t r = row - i * per_owner;  // row of owner i's slots, [B][C][H] order
  const int h = (int)(r % a.H);
  const int64_t bs = r / a.H;
  const int s = (int)(bs % a.C);
  const int b = (int)(bs / a.C);
  const int n = a.n_vis[i];
  const int64_t s0 = a.slot0[i];
  auto slot = [&](int c) -> int64_t { return s0 + arrival_kv(a.pass_q != 0, i, n, c); };
  f32x4 res;
  float M, den;
  merge_row(
      n, [&](int c) { return *reinterpret_cast<const f32x4*>(a.ws_o + slot(c) * a.slot_o + r * D + 4 * part); },
      [&](int c) { return a.ws_l[slot(c) * a.slot_l + r]; }, res, M, den);
  const int64_t sg = (int64_t)i * a.C + s;  // row of the full sequence
  store_row(a.out, a.out_bf16, b * a.o_sb + sg * a.o_ss + h * a.o_sh + 4 * part, res);
  if (a.out_lse != nullptr && part == 0)
    a.out_lse[b * a.ol_sb + sg * a.ol_ss + h * a.ol_sh] = merged_lse(M, den);
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

hipError_t launch_ring_merge(const RingMergeLaunch& a, hipStream_t s) {
  const long long rows = (long long)a.P * a.B * a.C * a.H;
  if (rows <= 0) return hipSuccess;
  const long long blocks = (rows * (a.D / 4) + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.D == 128)
    hipLaunchKernelGGL(ring_merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(ring_merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
