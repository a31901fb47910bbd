// Partial attention for fp32 Q/K/V on the vector ALUs (fp32 throughout).
//
// Same operation as the bf16 MFMA kernel (a rank's queries against one K/V
// chunk; "Scaling LLM Inference", techreport.ngo rewrite, "Context
// Parallelism for Million-Token Contexts"), for inputs that must not be
// rounded to bf16.  T = D/32 adjacent lanes share one query row, each holding
// 32 of its D components of q and of the output; a score is a 32-term partial
// dot product per lane reduced across the T lanes.  K/V tiles of 32 keys are
// staged in LDS and read as broadcasts.  The online softmax is updated key by
// key in base 2 (scale folded into the exponent), so this path has no
// lazy-rescale approximation of the reference max.
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

template <int D>
__global__ __launch_bounds__(256) void partial_f32_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int T = D / 32;       // lanes per query row
  constexpr int ROWS = 256 / T;   // query rows per workgroup
  constexpr int BN = 32;          // keys per tile
  constexpr float SCALE_LOG2 = (D == 64) ? 0.18033688011112042f : 0.12751743082459868f;
  __shared__ __attribute__((aligned(16))) float ks[BN * D];
  __shared__ __attribute__((aligned(16))) float vs[BN * D];

  const int tid = threadIdx.x;
  const int part = tid % T;
  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = (a.xcd_order ? xcd_logical_block(blockIdx.x, per_item * a.n_items) : (int)blockIdx.x);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];
  const int Sk = it.sk > 0 ? it.sk : a.Sk;  // keys of this item's K/V block

  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh +
                    (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const float* kp = static_cast<const float*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                    (int64_t)it.kv_chunk * a.kv_chunk_len * a.k_ss;
  const float* vp = static_cast<const float*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                    (int64_t)it.kv_chunk * a.kv_chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse != nullptr ? a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh : nullptr;  // LSE optional
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.kv_chunk_len;

  const int m0 = qt * ROWS;
  const int row = m0 + tid / T;
  const bool row_ok = row < a.Sq;
  const int64_t qpos = qpos0 + row;

  int n_end = Sk;
  if (a.causal) {
    const int64_t last_row = (int64_t)min(m0 + ROWS, a.Sq) - 1;
    n_end = (int)max<int64_t>(0, min<int64_t>(Sk, qpos0 + last_row - kvpos0 + 1));
  }

  float q[32], o[32];
  {
    const float* qr = qp + (int64_t)row * a.q_ss + 32 * part;
#pragma unroll
    for (int x = 0; x < 32; x += 4) {
      const f32x4 v4 = row_ok ? *reinterpret_cast<const f32x4*>(qr + x) : (f32x4){};
      q[x] = v4[0]; q[x + 1] = v4[1]; q[x + 2] = v4[2]; q[x + 3] = v4[3];
    }
  }
#pragma unroll
  for (int x = 0; x < 32; ++x) o[x] = 0.f;
  float m = kNegInf, l = 0.f;

  for (int n0 = 0; n0 < n_end; n0 += BN) {
    // cooperative tile load: BN*D floats of K and of V, 16 bytes per thread per pass
    for (int idx = tid; idx < BN * D / 4; idx += 256) {
      const int key = (idx * 4) / D, d = (idx * 4) % D;
      const bool ok = n0 + key < Sk;
      *reinterpret_cast<f32x4*>(ks + key * D + d) =
          ok ? *reinterpret_cast<const f32x4*>(kp + (int64_t)(n0 + key) * a.k_ss + d) : (f32x4){};
      *reinterpret_cast<f32x4*>(vs + key * D + d) =
          ok ? *reinterpret_cast<const f32x4*>(vp + (int64_t)(n0 + key) * a.v_ss + d) : (f32x4){};
    }
    __syncthreads();
    const int kmax = min(BN, n_end - n0);
    for (int j = 0; j < kmax; ++j) {
      const float* kr = ks + j * D + 32 * part;
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < 32; ++x) dot = fmaf(q[x], kr[x], dot);
#pragma unroll
      for (int off = 1; off < T; off <<= 1) dot += __shfl_xor(dot, off);
      const int key = n0 + j;
      const bool vis = !a.causal || kvpos0 + key <= qpos;
      const float s = vis ? dot * SCALE_LOG2 : kNegInf;
      const float m_new = fmaxf(m, s);
      if (m_new != kNegInf) {
        const float alpha = fast_exp2(m - m_new);
        const float p = fast_exp2(s - m_new);
        l = l * alpha + p;
        const float* vr = vs + j * D + 32 * part;
#pragma unroll
        for (int x = 0; x < 32; ++x) o[x] = fmaf(p, vr[x], o[x] * alpha);
        m = m_new;
      }
    }
    __syncthreads();
  }

  if (row_ok) {
    const bool acc = a.accumulate != 0;
    const RowOut ro = row_out(m, l, acc, acc ? lp[(int64_t)row * a.l_ss] : 0.f);
    float* orow = op + (int64_t)row * a.o_ss + 32 * part;
#pragma unroll
    for (int x = 0; x < 32; x += 4) {
      f32x4 v4 = {o[x] * ro.s_new, o[x + 1] * ro.s_new, o[x + 2] * ro.s_new, o[x + 3] * ro.s_new};
      if (acc) {
        const f32x4 old = *reinterpret_cast<const f32x4*>(orow + x);
        v4 = (f32x4){fmaf(old[0], ro.s_old, v4[0]), fmaf(old[1], ro.s_old, v4[1]), fmaf(old[2], ro.s_old, v4[2]),
                     fmaf(old[3], ro.s_old, v4[3])};
      }
      *reinterpret_cast<f32x4*>(orow + x) = v4;
    }
    if (part == 0 && lp != nullptr) lp[(int64_t)row * a.l_ss] = ro.lse;
  }
}

}  // namespace

int partial_f32_rows_per_block(int D) { return 256 / (D / 32); }

hipError_t launch_partial_f32(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s) {
  const long long blocks = (long long)a.n_items * a.B * a.Hq * n_qtiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128)
    hipLaunchKernelGGL(partial_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL(partial_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
