// Split-KV decode: one new query token per sequence against a cached K/V.
//
// Decode streams the KV cache and is memory-bandwidth bound ("Scaling LLM
// Inference", techreport.ngo rewrite, "Why Parallelism Defines LLM Serving
// Cost"); the cache grows linearly with context ("Context Parallelism for
// Million-Token Contexts").  Every byte of K and V is read exactly once from
// HBM, so the kernel is organised to keep enough bytes in flight per CU.  A
// work unit is (batch, KV head, block of up to 16 query heads sharing it,
// chunk, sub-split); each unit writes a partial (O normalised, LSE) to the
// workspace, and the partials are merged afterwards.  Every chunk has a base
// pointer and a length of its own, so the chunks may be the equal pieces of
// one cache or the shards of a cache cut across CP ranks; a unit that finds no
// key in its range writes the empty partial (O = 0, LSE = -inf).
//
// The 16 query heads of a KV head form the 16 columns of a 16x16x32 bf16
// MFMA: S^T = K Q^T puts keys on rows, so a lane holds 4 keys of one head and
// the row max / sum are reduced across the 4 lane groups.
#include <algorithm>
#include <atomic>

#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

constexpr float kTau = 8.0f;

// ---------------------------------------------------------------------------
// Workgroups are persistent (one per CU, looping over work units) and move
// K/V through LDS with global_load_lds_dwordx4, four stages
// of 64-key tiles deep, so about three tiles per CU are in flight at all
// times -- also across the boundary between one unit and the next.  The
// four waves of a workgroup all compute the (cheap) scores S^T = K Q^T of
// the whole tile, so they hold identical softmax state, and each wave
// accumulates its own quarter of the D columns of O^T = V^T P^T: no
// cross-wave combine is needed.  V^T operands come from the row-major V tile
// through ds_read_b64_tr_b16 (within a 16-lane group, lane 4a+b receives
// element b of the 8-byte rows addressed by lanes a, a+4, a+8, a+12).  The
// unit's 16 query heads travel with its first tile through the same kind of
// load, so the kernel issues no other global load that s_waitcnt vmcnt
// would have to account for.
// ---------------------------------------------------------------------------
// global_load_lds_dwordx4 with the non-temporal hint: every K/V byte of the
// cache is read exactly once, so the stream is marked as not worth keeping in
// the caches (measured: 5.9 -> 6.5 TB/s on the 128 x 32K-key cache).
__device__ __forceinline__ void gload_lds16_stream(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u32x2 ld_lds8_tr(const uint8_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(__attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

template <int D>
struct StreamCfg {
  static constexpr int TK = 64;                    // keys per tile
  static constexpr int ROWB = D * 2;               // bytes per K/V row
  static constexpr int CH = D / 8;                 // 16-byte chunks per row
  static constexpr int TB = TK * ROWB;             // bytes of a K (or V) tile
  static constexpr int QB = 16 * ROWB;             // bytes of the unit's query block
  static constexpr int STAGE = 2 * TB + QB;        // K, V, Q
  static constexpr int NST = 4;                    // stages (three tiles in flight)
  static constexpr int KP = TK * CH / 256;         // K (and V) pieces per thread per tile
  static constexpr int LPT = 2 * KP;               // K/V loads per thread per tile (a unit's first
                                                   // tile adds one more, for the query block)
  // chunk swizzles: K rows are read 16 at a time at one chunk, V rows 8 at a
  // time as 32-byte pairs; both keep those reads on distinct banks
  __device__ static int kswz(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
  __device__ static int vswz(int key) { return D == 128 ? 2 * (key & 7) : 2 * ((key >> 1) & 3); }
};

template <int D>
__global__ __launch_bounds__(256) void decode_stream_kernel(const DecodeLaunch a, const int total) {
  using C = StreamCfg<D>;
  constexpr int TK = C::TK, ROWB = C::ROWB, TB = C::TB, STAGE = C::STAGE, NST = C::NST, KP = C::KP, LPT = C::LPT;
  constexpr int NS = D / 32;    // QK k-steps (32 d each)
  constexpr int NDB = D / 64;   // 16-column blocks of O^T per wave (a wave owns D/4 columns)
  constexpr float SCALE_LOG2 = (D == 64) ? 0.18033688011112042f : 0.12751743082459868f;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int x = lane & 15;   // head within the block (MFMA column) / row within a 16-row block
  const int g4 = lane >> 4;  // lane group
  const int s16 = x;

  struct Unit {
    int b, kvh, hb, c, sp, k_lo, nt, lim_last, rot;
  };
  auto decode_unit = [&](int u) {
    const int u0 = u;
    Unit r;
    r.sp = u % a.n_split; u /= a.n_split;
    r.c = u % a.n_chunks; u /= a.n_chunks;
    r.hb = u % a.head_blocks; u /= a.head_blocks;
    r.kvh = u % a.Hkv;
    r.b = u / a.Hkv;
    r.k_lo = r.sp * a.split_len;  // rows of block c
    const int k_hi = min(r.k_lo + a.split_len, a.len[r.c]);
    const int n = max(0, k_hi - r.k_lo);
    r.nt = (n + TK - 1) / TK;
    r.lim_last = n - (r.nt - 1) * TK;  // keys in the last tile
    // The unit's tiles are visited starting at tile rot and wrapping around.
    // Units start at power-of-two-aligned addresses; without the rotation the
    // workgroups running side by side would all stream from the same offset
    // of their regions and crowd the same HBM channels (measured: a plain
    // streaming read of that pattern loses ~8% against a contiguous one).
    // The softmax is order-independent, so only rounding changes.
    r.rot = r.nt > 0 ? (int)(((unsigned)u0 * 37u) % (unsigned)r.nt) : 0;
    return r;
  };

  // ---- fetch cursor: the next tile of this workgroup's unit sequence ----
  int fu = blockIdx.x;
  int ft = 0;
  Unit fU = decode_unit(min(fu, total - 1));
  auto fetch_skip_empty = [&]() {
    while (fu < total && ft >= fU.nt) {
      fu += gridDim.x;
      ft = 0;
      if (fu < total) fU = decode_unit(fu);
    }
  };
  fetch_skip_empty();
  const uint32_t lbase = lds_addr(smem) + wave * 64 * 16;
  // returns whether a tile was fetched into `stage`
  auto fetch = [&](int stage) -> bool {
    if (fu >= total) return false;
    int tt = ft + fU.rot;  // tile of the unit in visiting order ft
    if (tt >= fU.nt) tt -= fU.nt;
    const int n_keys = (tt == fU.nt - 1) ? fU.lim_last : TK;
    const int k0 = fU.k_lo + tt * TK;
    const __bf16* kb = static_cast<const __bf16*>(a.kc[fU.c]) + fU.b * a.k_sb + fU.kvh * a.k_sh;
    const __bf16* vb = static_cast<const __bf16*>(a.vc[fU.c]) + fU.b * a.v_sb + fU.kvh * a.v_sh;
    const uint32_t dst = lbase + stage * STAGE;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = i * 256 + tid;        // piece: key pc / CH, physical chunk pc % CH
      const int key = pc / C::CH;
      const int ch = pc % C::CH;
      const int64_t row = k0 + min(key, n_keys - 1);  // rows past the end re-read the last one (masked)
      gload_lds16_stream(kb + row * a.k_ss + ((ch ^ C::kswz(key)) << 3), dst + i * 256 * 16);
      gload_lds16_stream(vb + row * a.v_ss + ((ch ^ C::vswz(key)) << 3), dst + TB + i * 256 * 16);
    }
    if (ft == 0) {
      // query block: 16 heads x D (piece tid mod (16 CH); with D = 64 two threads load each piece)
      const int pc = tid % (16 * C::CH);
      const int hx = pc / C::CH;
      const int head = fU.hb * 16 + hx;
      const int h = fU.kvh * a.G + min(head, a.G - 1);
      const __bf16* qr = static_cast<const __bf16*>(a.q) + fU.b * a.q_sb + (int64_t)h * a.q_sh;
      gload_lds16(qr + (pc % C::CH) * 8, lds_addr(smem) + stage * STAGE + 2 * TB + (pc - lane) * 16);
    }
    ++ft;
    fetch_skip_empty();
    return true;
  };

  // ---- per-lane LDS offsets ----
  int koff[NS];  // K operand, k-step s: row x of a 16-key block, chunk 4s + g4
#pragma unroll
  for (int s = 0; s < NS; ++s) koff[s] = x * ROWB + (((4 * s + g4) ^ C::kswz(x)) << 4);
  int voff[NDB];  // V^T operand, column block db of this wave: rows 4 g4 + s16/4 (+32kk, +16)
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = wave * (D / 4) + 16 * db;
    const int r = 4 * g4 + (s16 >> 2);
    voff[db] = TB + r * ROWB + (((d0 / 8 + ((s16 & 3) >> 1)) ^ C::vswz(r)) << 4) + (s16 & 1) * 8;
  }

  // prologue: NST-1 tiles in flight
  int n_inflight = 0;  // tiles fetched but not yet consumed
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) n_inflight += fetch(i) ? 1 : 0;
  int cs = 0;  // stage of the next tile to consume

  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const Unit U = decode_unit(u);
    const int head = U.hb * 16 + x;
    const bool head_ok = head < a.G;
    const int h = U.kvh * a.G + head;

    f32x4 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = (f32x4){};
    float m_run = kNegInf, l_run = 0.f;
    bf16x8 qf[NS];

    for (int t = 0; t < U.nt; ++t) {
      // this tile must have landed (later tiles' loads stay in flight), and
      // every wave must be done with the stage the next fetch refills.  The
      // count covers the K/V loads of the later tiles only; any other
      // memory operation issued after this tile's loads (a query block, the
      // stores of a finished unit) only makes the wait stricter.
      const int after = n_inflight - 1;
      if (after >= 2)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LPT) : "memory");
      else if (after == 1)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LPT) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      n_inflight += fetch((cs + NST - 1) % NST) ? 1 : 0;
      const uint8_t* st = smem + cs * STAGE;
      if (t == 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(ld_lds16(st + 2 * TB + x * ROWB + (4 * s + g4) * 16));
      }

      // ---- S^T = K Q^T: four 16-key blocks.  All operand reads go out first
      // (one wave per SIMD: nothing else hides their latency), then the
      // MFMAs alternate over the four independent accumulators.
      u32x4 kop[4][NS];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int s = 0; s < NS; ++s) kop[kb][s] = ld_lds16(st + kb * 16 * ROWB + koff[s]);
      u32x2 vlo[2][NDB], vhi[2][NDB];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          vlo[kk][db] = ld_lds8_tr(st + voff[db] + (32 * kk) * ROWB);
          vhi[kk][db] = ld_lds8_tr(st + voff[db] + (32 * kk + 16) * ROWB);
        }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 sacc[4] = {(f32x4){}, (f32x4){}, (f32x4){}, (f32x4){}};
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sacc[kb] = mfma16(as_bf16x8(kop[kb][s]), qf[s], sacc[kb]);
      int tt = t + U.rot;  // this tile's place in the unit
      if (tt >= U.nt) tt -= U.nt;
      if (tt == U.nt - 1 && U.lim_last < TK) {
        const int lim = U.lim_last - 4 * g4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[kb][i] = (16 * kb + i < lim) ? sacc[kb][i] : kNegInf;
      }

      // ---- online softmax of each head over the 4 lane groups
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
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
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = fast_exp2(fmaf(sacc[kb][i], SCALE_LOG2, -mref));
          l_run += p[kb][i];
        }

      // ---- O^T += V^T P^T over two 32-key k-steps; slot j < 4 <-> key 32kk + 4 g4 + j,
      //      slot j >= 4 <-> key 32kk + 16 + 4 g4 + j - 4
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const u32x4 pb = {pack_bf16(p[2 * kk][0], p[2 * kk][1]), pack_bf16(p[2 * kk][2], p[2 * kk][3]),
                          pack_bf16(p[2 * kk + 1][0], p[2 * kk + 1][1]), pack_bf16(p[2 * kk + 1][2], p[2 * kk + 1][3])};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 av = {vlo[kk][db][0], vlo[kk][db][1], vhi[kk][db][0], vhi[kk][db][1]};
          oacc[db] = mfma16(as_bf16x8(av), as_bf16x8(pb), oacc[db]);
        }
      }
      cs = (cs + 1) % NST;
      --n_inflight;
    }

    // ---- partial out: normalised O (this wave's columns) and natural-log LSE
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (head_ok) {
      const int p_idx = U.c * a.n_split + U.sp;
      float* orow = a.o + p_idx * a.o_slot + U.b * a.o_sb + h * a.o_sh + wave * (D / 4);
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g4) = oacc[db] * inv;
      if (wave == 0 && g4 == 0)
        a.lse[p_idx * a.l_slot + U.b * a.l_sb + h * a.l_sh] = (l_tot > 0.f) ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

// Compute units of the current device, cached per device.  Several host
// threads may make their first call at once: each entry is an atomic that
// they may all fill with the same value.
hipError_t cu_count(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    n = n > 0 ? n : 1;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeLaunch& a, int D, hipStream_t s) {
  const long long units = (long long)a.B * a.Hkv * a.head_blocks * a.n_chunks * a.n_split;
  if (units <= 0) return hipSuccess;
  if (units > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // one persistent workgroup per CU (the LDS stages take most of a CU's LDS)
  int n_cu = 0;
  const hipError_t e = cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const int grid = (int)std::min<long long>(units, n_cu);
  if (D == 128)
    hipLaunchKernelGGL(decode_stream_kernel<128>, dim3(grid), dim3(256), 0, s, a, (int)units);
  else if (D == 64)
    hipLaunchKernelGGL(decode_stream_kernel<64>, dim3(grid), dim3(256), 0, s, a, (int)units);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
