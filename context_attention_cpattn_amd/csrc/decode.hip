// Split-KV decode: one new query token per sequence against a cached K/V.
//
// Decode streams the KV cache and is memory-bandwidth bound ("Scaling LLM
// Inference", techreport.ngo rewrite, "Why Parallelism Defines LLM Serving
// Cost"); the cache grows linearly with context ("Context Parallelism for
// Million-Token Contexts").  Every byte of K and V is read exactly once from
// HBM, so the kernel is organised for memory-level parallelism: one wave
// per work unit (batch, KV head, block of up to 16 query heads sharing it,
// chunk, sub-split), four independent units per workgroup, and the next
// 32-key tile's loads in flight while the current tile is used.
//
// The 16 query heads of a KV head form the 16 columns of a 16x16x32 bf16
// MFMA: S^T = K Q^T puts keys on rows, so a lane holds 4 keys of one head and
// the row max / sum are reduced across the 4 lane groups.  K goes straight
// from global memory into the A-operand layout; V is transposed through a
// wave-private LDS tile so the A operand of O^T = V^T P^T is two 8-byte
// reads.  Each unit writes a partial (O normalised, LSE) to the workspace;
// the partials are merged afterwards.
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

constexpr float kTau = 8.0f;

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int dv_swz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

template <int D>
__global__ __launch_bounds__(256) void decode_bf16_kernel(const DecodeLaunch a) {
  constexpr int TK = 32;              // keys per tile
  constexpr int NS = D / 32;          // k-steps of S^T (32 d each)
  constexpr int NDB = D / 16;         // 16-wide column blocks of O^T
  constexpr int CPL = D / 64;         // V chunks per lane per key (1 or 2)
  constexpr int VROW = TK * 2;        // bytes per V^T row
  constexpr float SCALE_LOG2 = (D == 64) ? 0.18033688011112042f : 0.12751743082459868f;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * D * VROW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wave;
  const int total = a.B * a.Hkv * a.head_blocks * a.n_chunks * a.n_split;
  if (unit >= total) return;  // whole wave leaves; the kernel has no workgroup barrier

  int u = unit;
  const int sp = u % a.n_split; u /= a.n_split;
  const int c = u % a.n_chunks; u /= a.n_chunks;
  const int hb = u % a.head_blocks; u /= a.head_blocks;
  const int kvh = u % a.Hkv;
  const int b = u / a.Hkv;

  const int chunk_len = a.Skv / a.n_chunks;
  const int k_lo = c * chunk_len + sp * a.split_len;
  const int k_hi = min(k_lo + a.split_len, (c + 1) * chunk_len);

  const int x = lane & 15;   // head within the block (MFMA column)
  const int g4 = lane >> 4;  // lane group
  const int head = hb * 16 + x;
  const bool head_ok = head < a.G;
  const int h = kvh * a.G + head;

  // Q^T fragments (B operand): column = head, k-slots = d chunk 4 s + g4
  bf16x8 qf[NS];
  {
    const __bf16* qr = static_cast<const __bf16*>(a.q) + b * a.q_sb + (int64_t)h * a.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = head_ok ? as_bf16x8(ld_global16(qr + (4 * s + g4) * 8)) : (bf16x8){};
  }

  const __bf16* kb = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const __bf16* vb = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  uint8_t* vs = smem + wave * (D * VROW);

  const int vkg = lane >> 3;  // 4-key group of the V tile (0..7)
  const int vcl = lane & 7;   // d chunk(s): vcl + 8 cc

  u32x4 kf[2][NS], vf[4][CPL];
  u32x4 kn[2][NS], vn[4][CPL];
  auto load = [&](int k0, u32x4 (&kk)[2][NS], u32x4 (&vv)[4][CPL]) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int key = k0 + 16 * blk + x;
      const bool ok = key < k_hi;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        kk[blk][s] = ok ? ld_global16(kb + (int64_t)key * a.k_ss + (4 * s + g4) * 8) : (u32x4){};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * vkg + j;
      const bool ok = key < k_hi;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc)
        vv[j][cc] = ok ? ld_global16(vb + (int64_t)key * a.v_ss + (vcl + 8 * cc) * 8) : (u32x4){};
    }
  };

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x4){};
  float m_run = kNegInf, l_run = 0.f;

  if (k_lo < k_hi) load(k_lo, kf, vf);
  for (int k0 = k_lo; k0 < k_hi; k0 += TK) {
    const bool has_next = k0 + TK < k_hi;
    if (has_next) load(k0 + TK, kn, vn);

    // ---- S^T = K Q^T: two 16-key blocks
    f32x4 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f32x4 acc = (f32x4){};
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = mfma16(as_bf16x8(kf[blk][s]), qf[s], acc);
      sacc[blk] = acc;
    }
    if (k0 + TK > k_hi) {
      const int lim = k_hi - k0;  // tile-local keys [0, lim) exist
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[blk][i] = (16 * blk + 4 * g4 + i < lim) ? sacc[blk][i] : kNegInf;
    }

    // ---- online softmax over the 4 lane groups of a head
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * SCALE_LOG2;
    if (__any(mt > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float mref = (m_run == kNegInf) ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(fmaf(sacc[0][i], SCALE_LOG2, -mref));
      p[4 + i] = fast_exp2(fmaf(sacc[1][i], SCALE_LOG2, -mref));
    }
    l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    // B operand of O^T = V^T P^T: slot j < 4 <-> key 4 g4 + j, slot j >= 4 <-> key 16 + 4 g4 + j - 4
    const u32x4 pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7])};

    // ---- V^T into the wave's LDS tile: row d holds the 32 keys of this tile
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const int dch = vcl + 8 * cc;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int de = dch * 8 + 2 * w;
        const int dodd = de + 1;
        const u32x2 ev = {pack_lo16(vf[0][cc][w], vf[1][cc][w]), pack_lo16(vf[2][cc][w], vf[3][cc][w])};
        const u32x2 od = {pack_hi16(vf[0][cc][w], vf[1][cc][w]), pack_hi16(vf[2][cc][w], vf[3][cc][w])};
        st_lds8(vs + de * VROW + ((vkg ^ dv_swz(de)) << 3), ev);
        st_lds8(vs + dodd * VROW + ((vkg ^ dv_swz(dodd)) << 3), od);
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + x;
      const uint8_t* vrow = vs + d * VROW;
      const int sw = dv_swz(d);
      const u32x2 lo = ld_lds8(vrow + ((g4 ^ sw) << 3));
      const u32x2 hi = ld_lds8(vrow + (((4 + g4) ^ sw) << 3));
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
      oacc[db] = mfma16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
    }
    wave_lds_sync();

    if (has_next) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int s = 0; s < NS; ++s) kf[blk][s] = kn[blk][s];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) vf[j][cc] = vn[j][cc];
    }
  }

  // ---- partial out: normalised O and natural-log LSE
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (head_ok) {
    const int p_idx = c * a.n_split + sp;
    const int64_t rowi = (int64_t)p_idx * a.B * a.Hq + (int64_t)b * a.Hq + h;
    float* orow = a.o + rowi * D;
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g4) = oacc[db] * inv;
    if (g4 == 0) a.lse[rowi] = (l_tot > 0.f) ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeLaunch& a, int D, hipStream_t s) {
  const long long units = (long long)a.B * a.Hkv * a.head_blocks * a.n_chunks * a.n_split;
  if (units <= 0) return hipSuccess;
  const long long blocks = (units + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128)
    hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (D == 64)
    hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
