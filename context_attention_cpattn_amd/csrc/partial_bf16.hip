// Partial attention of Q blocks against K/V blocks, bf16 inputs on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// This is the per-step work of a context-parallel ring: a rank's local
// queries against the K/V chunk it holds at that step ("Scaling LLM
// Inference", techreport.ngo rewrite, "Context Parallelism for Million-Token
// Contexts").  Prefill of this kind is compute bound ("Why Parallelism
// Defines LLM Serving Cost"), so the two contractions run on MFMA and the
// softmax bookkeeping is kept per lane.
//
// Workgroup = 4 waves = 128 query rows of one head; each wave owns 32 rows.
// K/V tiles of BN keys are staged through LDS (double buffered: the next
// tile's global loads are in flight while the current one is used).
//
// Orientation: each wave computes S^T = K Q^T (keys on the MFMA rows, its 32
// queries on the columns), so a lane holds scores of ONE query.  The row max
// and row sum are then in-lane reductions plus one exchange with the lane 32
// away.  The probabilities are already in the B-operand layout of the second
// product O^T = V^T P^T, so P never leaves registers.  V^T is written to LDS
// transposed (4 keys x 8 d per thread, repacked with v_perm) so the A operand
// of that product is two 8-byte LDS reads per lane.
//
// Softmax runs in base 2 with the 1/sqrt(D) scale folded into one FMA.  The
// running max is only raised when a tile's max exceeds it by more than
// kTau (2^8), so most tiles skip the O rescale; the probabilities stay
// <= 2^8, well inside bf16/fp32 range, and the result is exact in real
// arithmetic because the final normalisation uses the same reference max.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {
#ifdef CPATTN_TIMING
__device__ unsigned long long g_cpattn_stamps[8 * 160 * 4];
#define STAMP(w, p, k, blk) do { if ((blk) == CPATTN_TIMING && (p) < 160 && (threadIdx.x & 63) == 0) g_cpattn_stamps[((w) * 160 + (p)) * 4 + (k)] = __builtin_readcyclecounter(); } while (0)
#else
#define STAMP(w, p, k, blk) do {} while (0)
#endif

constexpr float kTau = 8.0f;

template <int D>
struct Cfg {
  static constexpr int BM = 128;             // query rows per workgroup
  static constexpr int BN = 8192 / D;        // keys per tile (64 for D=128, 128 for D=64)
  static constexpr int DCH = D / 8;          // 16-byte chunks per K/V row
  static constexpr int NKB = BN / 32;        // 32-key blocks per tile
  static constexpr int NDS = D / 16;         // k-steps of S^T = K Q^T
  static constexpr int NDB = D / 32;         // 32-wide column blocks of O
  static constexpr int KBYTES = BN * D * 2;  // one K tile (= one V^T tile)
  static constexpr int STAGE = 2 * KBYTES;
  static constexpr int KPT = BN * DCH / 256; // K chunks loaded per thread
  static constexpr int VROW = BN * 2;        // bytes of one V^T row (one d)
  static constexpr float SCALE_LOG2 = (D == 64) ? 0.18033688011112042f : 0.12751743082459868f;
};
static_assert(Cfg<128>::KPT == 4 && Cfg<64>::KPT == 4, "tile shape");
static_assert(Cfg<128>::BN / 4 * Cfg<128>::DCH == 256 && Cfg<64>::BN / 4 * Cfg<64>::DCH == 256, "V split");

// XOR swizzles keeping both the tile stores and the MFMA operand reads free
// of LDS bank conflicts.
template <int D>
__device__ __forceinline__ int k_swz(int key, int ch) { return ch ^ (key & (Cfg<D>::DCH - 1)); }
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 15; }

template <int D>
__global__ __launch_bounds__(256) void partial_bf16_kernel(const PartialLaunch a, const int n_qtiles) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // ---- which (item, query tile, batch, head) this workgroup computes
  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;  // later (heavier under the mask) tiles first
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  const int m0 = qt * C::BM;
  const int r0 = m0 + wave * 32;  // first row of this wave
  const int row = r0 + l32;       // this lane's query row

  // keys [0, n_end) can be visible to some row of this workgroup
  int n_end = a.Sk;
  if (a.causal) {
    const int64_t last_row = (int64_t)min(m0 + C::BM, a.Sq) - 1;
    const int64_t lim = qpos0 + last_row - kvpos0 + 1;
    n_end = (int)max<int64_t>(0, min<int64_t>(a.Sk, lim));
  }
  const int n_tiles = (n_end + C::BN - 1) / C::BN;

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = (f32x16){};
  float m_run = kNegInf;
  float l_run = 0.f;

  if (n_tiles > 0) {
    // Q fragments, B operand of S^T = K Q^T: column = this lane's row,
    // k-slots = d in [16 s + 8 g, 16 s + 8 g + 8).
    bf16x8 qf[C::NDS];
    {
      const bool ok = row < a.Sq;
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
#pragma unroll
      for (int s = 0; s < C::NDS; ++s) qf[s] = ok ? as_bf16x8(ld_global16(qr + 16 * s)) : (bf16x8){};
    }

    u32x4 kreg[C::KPT];
    u32x4 vreg[4];
    const int vkg = tid / C::DCH;  // this thread's 4-key group of the V tile
    const int vch = tid % C::DCH;  // and its 16-byte d chunk

    auto load_tile = [&](int t) {
      const int n0 = t * C::BN;
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        const int idx = tid + 256 * i;
        const int key = idx / C::DCH, ch = idx % C::DCH;
        kreg[i] = (n0 + key < a.Sk) ? ld_global16(kp + (int64_t)(n0 + key) * a.k_ss + ch * 8) : (u32x4){};
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = n0 + 4 * vkg + kk;
        vreg[kk] = (key < a.Sk) ? ld_global16(vp + (int64_t)key * a.v_ss + vch * 8) : (u32x4){};
      }
    };
    auto store_tile = [&](int stage) {
      uint8_t* ks = smem + stage * C::STAGE;
      uint8_t* vs = ks + C::KBYTES;
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        const int idx = tid + 256 * i;
        const int key = idx / C::DCH, ch = idx % C::DCH;
        st_lds16(ks + key * (D * 2) + (k_swz<D>(key, ch) << 4), kreg[i]);
      }
      // 4 keys x 8 d -> for each d, the 4 keys' values side by side
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int de = vch * 8 + 2 * w;
        const int dodd = de + 1;
        const u32x2 ev = {pack_lo16(vreg[0][w], vreg[1][w]), pack_lo16(vreg[2][w], vreg[3][w])};
        const u32x2 od = {pack_hi16(vreg[0][w], vreg[1][w]), pack_hi16(vreg[2][w], vreg[3][w])};
        st_lds8(vs + de * C::VROW + ((vkg ^ v_swz(de)) << 3), ev);
        st_lds8(vs + dodd * C::VROW + ((vkg ^ v_swz(dodd)) << 3), od);
      }
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
      const bool has_next = (t + 1) < n_tiles;
      if (has_next) load_tile(t + 1);

      const uint8_t* ks = smem + (t & 1) * C::STAGE;
      const uint8_t* vs = ks + C::KBYTES;
      const int n0 = t * C::BN;
      const bool wave_active = (r0 < a.Sq) && (!a.causal || kvpos0 + n0 <= qpos0 + r0 + 31);

      if (wave_active) {
        // ---- S^T = K Q^T for this tile: NKB blocks of 32 keys x 32 queries
        f32x16 sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          const int key = kb * 32 + l32;
          const uint8_t* krow = ks + key * (D * 2);
          f32x16 acc = (f32x16){};
#pragma unroll
          for (int s = 0; s < C::NDS; ++s) {
            const u32x4 kv = ld_lds16(krow + (k_swz<D>(key, 2 * s + g) << 4));
            acc = mfma32(as_bf16x8(kv), qf[s], acc);
          }
          sacc[kb] = acc;
        }

        // ---- mask (only tiles that straddle the diagonal or the block end)
        const bool full = (n0 + C::BN <= a.Sk) && (!a.causal || kvpos0 + n0 + C::BN - 1 <= qpos0 + r0);
        if (!full) {
          // visibility is monotone in the key, so this row sees exactly the
          // tile-local keys [0, lim)
          int64_t lim64 = (int64_t)a.Sk - n0;
          if (a.causal) lim64 = min<int64_t>(lim64, qpos0 + row - kvpos0 - n0 + 1);
          const int lim = (int)max<int64_t>(0, min<int64_t>(lim64, C::BN));
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kl = kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
              sacc[kb][i] = (kl < lim) ? sacc[kb][i] : kNegInf;
            }
          }
        }

        // ---- online softmax (base 2), lazily rescaled
        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = fmaxf(mx, xor32(mx));
        const float mt = mx * C::SCALE_LOG2;
        if (__any(mt > m_run + kTau)) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha;
          m_run = m_new;
        }
        const float mref = (m_run == kNegInf) ? 0.f : m_run;

        u32x4 pk[C::NKB][2];
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[i] = fast_exp2(fmaf(sacc[kb][i], C::SCALE_LOG2, -mref));
            lsum += p[i];
          }
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
            pk[kb][t2] = (u32x4){pack_bf16(p[8 * t2 + 0], p[8 * t2 + 1]), pack_bf16(p[8 * t2 + 2], p[8 * t2 + 3]),
                                 pack_bf16(p[8 * t2 + 4], p[8 * t2 + 5]), pack_bf16(p[8 * t2 + 6], p[8 * t2 + 7])};
        }
        l_run += lsum;

        // ---- O^T += V^T P^T; k-slot j of lane group g <-> key
        //      32 kb + 16 t2 + 8 (j / 4) + 4 g + (j % 4), matching the S^T layout
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int d = db * 32 + l32;
          const uint8_t* vrow = vs + d * C::VROW;
          const int sw = v_swz(d);
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int c8 = 8 * kb + 4 * t2 + g;
              const u32x2 lo = ld_lds8(vrow + ((c8 ^ sw) << 3));
              const u32x2 hi = ld_lds8(vrow + (((c8 + 2) ^ sw) << 3));
              const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
              oacc[db] = mfma32(as_bf16x8(av), as_bf16x8(pk[kb][t2]), oacc[db]);
            }
          }
        }
      }

      if (has_next) store_tile((t + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue: combine the two half-rows' sums, normalise, store
  const float l_tot = l_run + xor32(l_run);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv, oacc[db][4 * i4 + 2] * inv,
                          oacc[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (m_run + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// D = 128 kernel: 64 query rows per wave.
//
// Each wave owns two 32-row blocks (A and B).  Every K operand read from LDS
// feeds one MFMA of each block and every V^T operand read feeds one PV MFMA
// of each block, halving LDS operand traffic per FLOP compared with 32 rows
// per wave (at full MFMA rate 32 rows/wave would need the whole LDS read
// bandwidth).  The K tile goes straight from global memory into the swizzled
// LDS layout (global_load_lds_dwordx4: lane i of an instruction fills the
// i-th 16-byte slot, so each lane fetches the chunk that belongs in its
// slot); V still passes through registers for the 4x8 transpose.
// ---------------------------------------------------------------------------
#ifndef CPATTN_D128_NW
#define CPATTN_D128_NW 8   // waves per workgroup
#endif
#ifndef CPATTN_D128_PRIO
#define CPATTN_D128_PRIO 1  // raise wave priority during the MFMA phases
#endif
#ifndef CPATTN_D128_SCHED
#define CPATTN_D128_SCHED 0  // issue order of the K operand reads (see the QK phase)
#endif
#ifndef CPATTN_D128_STAGES
#define CPATTN_D128_STAGES 3  // LDS stages of the plain D = 128 kernel
#endif
#ifndef CPATTN_D128_PIPE
#define CPATTN_D128_PIPE 4   // 0: plain, 1: software-pipelined, 2: ping-pong, 3: direct-to-LDS K and V, 3 stages,
                             // 4: as 3 with MFMA / VALU interleaved inside each wave
#endif
#ifndef CPATTN_V4_KLA
#define CPATTN_V4_KLA 4
#endif
#ifndef CPATTN_V4_VLA
#define CPATTN_V4_VLA 4
#endif
#ifndef CPATTN_D128_V4_STAGES
#define CPATTN_D128_V4_STAGES 3
#endif
#ifndef CPATTN_PIPE_VALU
#define CPATTN_PIPE_VALU 7   // softmax VALU instructions issued after each MFMA of the next tile
#endif
#ifndef CPATTN_D128_VPRE
#define CPATTN_D128_VPRE 0   // read the V operands before the softmax
#endif
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

struct Blk {
  f32x16 o[4];   // O^T accumulators, 4 column blocks of 32 d
  float m, l;    // running reference max (log2 domain) and partial sum
};

template <int NKB>
__device__ __forceinline__ void softmax_block(f32x16 (&s)[NKB], Blk& bk, u32x4 (&pk)[NKB][2], float scale_log2) {
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  mx = pair32_max(mx);
  const float mt = mx * scale_log2;
  if (__any(mt > bk.m + kTau)) {
    const float m_new = fmaxf(bk.m, mt);
    const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(bk.m - m_new);
    bk.l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) bk.o[db] *= alpha;
    bk.m = m_new;
  }
  const float mref = (bk.m == kNegInf) ? 0.f : bk.m;
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(fmaf(s[kb][i], scale_log2, -mref));
      lsum += p[i];
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      pk[kb][t2] = (u32x4){pack_bf16(p[8 * t2 + 0], p[8 * t2 + 1]), pack_bf16(p[8 * t2 + 2], p[8 * t2 + 3]),
                           pack_bf16(p[8 * t2 + 4], p[8 * t2 + 5]), pack_bf16(p[8 * t2 + 6], p[8 * t2 + 7])};
  }
  bk.l += lsum;
}

// Keep tile-local keys [0, lim) of this lane's row.  The lane's keys are
// kb*32 + 8*(i/4) + 4g + i%4, so comparing the constant part against lim - 4g
// keeps every index an inline immediate.
template <int NKB>
__device__ __forceinline__ void mask_block(f32x16 (&s)[NKB], int lim, int g) {
  const int limg = lim - 4 * g;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = (kb * 32 + 8 * (i >> 2) + (i & 3) < limg) ? s[kb][i] : kNegInf;
}

// V^T tile of the D = 128 kernel: row d holds the 64 keys of the tile.  Inside
// each 16-key group the 4-key groups are stored in the order 0, 2, 1, 3, so
// the 8 keys that lane group g feeds to one PV k-step (keys 4g..4g+3 and
// 8+4g..8+4g+3) are 16 contiguous bytes.  16-byte units are XOR-swizzled by
// (d mod 32) so that 16 consecutive rows hit distinct banks and the swizzle
// of row d and row d + 32 agree (a lane's read offsets do not depend on which
// 32-row block of O it is accumulating).
__device__ __forceinline__ int vt_swz(int d) { return (((d & 31) >> 1) ^ ((d & 31) >> 4)) & 7; }
__device__ __forceinline__ int vt_offset(int d, int kg) {
  const int kp = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);  // swap the two low bits of the group index
  return d * 128 + (((kp >> 1) ^ vt_swz(d)) << 4) + ((kp & 1) << 3);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void partial_bf16_d128_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NKB = 2, NDS = 8;
  constexpr int NT = NW * 64;                 // threads
  constexpr int BM = NW * 32;                 // query rows per workgroup (32 per wave)
  constexpr int KBYTES = BN * D * 2;          // one K (or V^T) tile
  constexpr int STAGE = 2 * KBYTES;
  constexpr int KCH = BN * 16 / NT;           // 16-byte K chunks per thread (direct to LDS)
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  static_assert(NT == 512 && KCH == 2, "the V staging below assumes 8 waves (2 keys per thread)");
  constexpr int NST = CPATTN_D128_STAGES;    // LDS stages (2: one tile ahead, 3: two tiles ahead)
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  // kv position minus q position of the blocks' first rows, clamped: sizes are
  // below 2^30, so a clamped distance still decides every row the same way
  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;  // first row of this wave
  const int row = r0 + l32;       // this lane's query row

  int n_end = a.Sk;
  if (a.causal) n_end = max(0, min(a.Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;

  Blk bk;
#pragma unroll
  for (int db = 0; db < 4; ++db) bk.o[db] = (f32x16){};
  bk.m = kNegInf;
  bk.l = 0.f;

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
      const bool ok = row < a.Sq;
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[s] = ok ? as_bf16x8(ld_global16(qr + 16 * s)) : (bf16x8){};
    }

    // Loop-invariant per-lane offsets (bytes within a stage).
    int koff[NDS];  // K operand of k-step s: row l32, 16-byte chunk 2s+g (swizzled); block kb adds 32 rows
#pragma unroll
    for (int s = 0; s < NDS; ++s) koff[s] = l32 * (D * 2) + (((2 * s + g) ^ (l32 & 15)) << 4);
    int voff[4];    // V^T operand of k-step u = 2kb+t2: row l32, unit 2u+g (swizzled); block db adds 32 rows
#pragma unroll
    for (int u = 0; u < 4; ++u) voff[u] = KBYTES + l32 * 128 + (((2 * u + g) ^ vt_swz(l32)) << 4);

    // K: instruction i of wave w fills the 16-byte LDS slots i*NT + w*64 + lane,
    // so each lane fetches the global chunk that belongs in its slot.
    const __bf16* ksrc[KCH];
    int kkey[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int slot = i * NT + wave * 64 + lane;
      kkey[i] = slot >> 4;
      ksrc[i] = kp + (int64_t)kkey[i] * a.k_ss + (((slot & 15) ^ (kkey[i] & 15)) * 8);
    }
    // V: thread owns keys 2*vkg, 2*vkg+1 of one 16-byte d chunk vch, written
    // transposed (two keys = 4 bytes) into rows 8*vch .. 8*vch+7 of V^T.
    const int vkg = tid >> 4, vch = tid & 15;
    const __bf16* vsrc = vp + (int64_t)(2 * vkg) * a.v_ss + vch * 8;
    int vwoff[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) vwoff[w] = KBYTES + vt_offset(vch * 8 + 2 * w, vkg >> 1) + (vkg & 1) * 4;

    // V staging: with three stages a set per stage (a fetch and the store of
    // the previous fetch overlap), with two stages a single set
    constexpr int NVS = (NST == 2) ? 1 : NST;
    u32x4 vregs[NVS][2];
    auto load_tile = [&](int t, int stage, u32x4 (&vreg)[2]) {
      const int n0 = t * BN;
      const bool tail = n0 + BN > a.Sk;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        // rows past the block end are clamped to the last row and masked later
        const __bf16* src = tail ? kp + (int64_t)min(n0 + kkey[i], a.Sk - 1) * a.k_ss +
                                       (((i * NT + wave * 64 + lane) & 15) ^ (kkey[i] & 15)) * 8
                                 : ksrc[i] + (int64_t)n0 * a.k_ss;
        gload_lds16(src, lds_addr(smem) + stage * STAGE + (i * NT + wave * 64) * 16);
      }
      const __bf16* vs0 = vsrc + (int64_t)n0 * a.v_ss;
      vreg[0] = (!tail || n0 + 2 * vkg < a.Sk) ? ld_global16(vs0) : (u32x4){};
      vreg[1] = (!tail || n0 + 2 * vkg + 1 < a.Sk) ? ld_global16(vs0 + a.v_ss) : (u32x4){};
    };
    auto store_v = [&](int stage, const u32x4 (&vreg)[2]) {
      uint8_t* vs = smem + stage * STAGE;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint32_t*>(vs + vwoff[w]) = pack_lo16(vreg[0][w], vreg[1][w]);        // d = 8 vch + 2w
        *reinterpret_cast<uint32_t*>(vs + vwoff[w] + 128) = pack_hi16(vreg[0][w], vreg[1][w]);  // d + 1
      }
    };

    // One 64-key tile from LDS stage ST (a compile-time constant, so every LDS
    // address is a per-lane offset plus an immediate).
    auto tile = [&](int t, auto stage_tag) {
      constexpr int ST = decltype(stage_tag)::value;
      constexpr int LD = (ST + NST - 1) % NST;  // stage of the tile being fetched (t + NST - 1)
      constexpr int SV = (ST + 1) % NST;        // stage whose V is stored at the end of this tile (t + 1)
      STAMP(wave, t, 0, L);
      const bool do_load = (t + NST - 1) < n_tiles;
      if (do_load) load_tile(t + NST - 1, LD, vregs[LD % NVS]);
      const uint8_t* base = smem + ST * STAGE;
      const int n0 = t * BN;
      const bool wave_active = (r0 < a.Sq) && (!a.causal || dpos + n0 <= r0 + 31);

      if (wave_active) {
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
        f32x16 sc[NKB];
#if CPATTN_D128_SCHED == 2
        {
          // all 16 K operands in flight before the first MFMA
          u32x4 kop[NKB][NDS];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int s = 0; s < NDS; ++s) kop[kb][s] = ld_lds16(base + koff[s] + kb * 32 * (D * 2));
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            f32x16 x = (f32x16){};
#pragma unroll
            for (int s = 0; s < NDS; ++s) x = mfma32(as_bf16x8(kop[kb][s]), qf[s], x);
            sc[kb] = x;
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        }
#else
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          u32x4 kop[NDS];
#pragma unroll
          for (int s = 0; s < NDS; ++s) kop[s] = ld_lds16(base + koff[s] + kb * 32 * (D * 2));
          f32x16 x = (f32x16){};
#pragma unroll
          for (int s = 0; s < NDS; ++s) x = mfma32(as_bf16x8(kop[s]), qf[s], x);
          sc[kb] = x;
#if CPATTN_D128_SCHED == 1
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#endif
        }
#endif
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
        if (n0 + BN > a.Sk || (a.causal && dpos + n0 + BN - 1 > r0)) {
          int lim = a.Sk - n0;
          if (a.causal) lim = min(lim, row - dpos - n0 + 1);
          mask_block<NKB>(sc, max(0, min(lim, BN)), g);
        }
        u32x4 pk[NKB][2];
#if CPATTN_D128_VPRE
        // V operands requested before the softmax so their latency hides under it
        u32x4 vop[4][4];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int u = 0; u < 4; ++u) vop[db][u] = ld_lds16(base + voff[u] + db * 32 * 128);
        softmax_block<NKB>(sc, bk, pk, SCALE_LOG2);
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int u = 0; u < 4; ++u) bk.o[db] = mfma32(as_bf16x8(vop[db][u]), as_bf16x8(pk[u >> 1][u & 1]), bk.o[db]);
#else
        softmax_block<NKB>(sc, bk, pk, SCALE_LOG2);
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4 av = ld_lds16(base + voff[u] + db * 32 * 128);
            bk.o[db] = mfma32(as_bf16x8(av), as_bf16x8(pk[u >> 1][u & 1]), bk.o[db]);
          }
        }
#endif
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
      }

      STAMP(wave, t, 1, L);
      // V of tile t+1 (fetched NST-2 tiles ago) goes to LDS now; with two stages
      // that is the fetch issued at the top of this tile
      if ((t + 1) < n_tiles && (NST == 2 || t >= 1)) store_v(SV, vregs[SV % NVS]);
      // K of tile t+1 must have landed and every LDS write be done before the
      // barrier; with three stages the fetch of tile t+2 (4 loads per thread)
      // stays in flight, so the barrier is issued without __syncthreads'
      // wait-for-everything
      STAMP(wave, t, 2, L);
      if (NST == 3 && do_load)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      STAMP(wave, t, 3, L);
    };

    load_tile(0, 0, vregs[0]);
    if (NST == 3 && n_tiles > 1) load_tile(1, 1, vregs[1 % NVS]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_v(0, vregs[0]);
    if (NST == 3 && n_tiles > 1) store_v(1, vregs[1 % NVS]);
    __syncthreads();
    if constexpr (NST == 2) {
      for (int t = 0; t < n_tiles; t += 2) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
      }
    } else {
      for (int t = 0; t < n_tiles; t += 3) {
        tile(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
        if (t + 2 < n_tiles) tile(t + 2, std::integral_constant<int, 2>{});
      }
    }
  }

  const float l_tot = pair32_sum(bk.l);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {bk.o[db][4 * i4 + 0] * inv, bk.o[db][4 * i4 + 1] * inv, bk.o[db][4 * i4 + 2] * inv,
                          bk.o[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (bk.m + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// Software-pipelined D = 128 kernel.  Same tiles, layouts and arithmetic as
// partial_bf16_d128_kernel, but each wave overlaps the QK^T MFMAs of tile t+1
// with the softmax of tile t inside one branch-free block whose issue order
// interleaves MFMA and VALU instructions, then runs the P.V MFMAs of tile t.
// LDS holds three K/V stages: tile t+1 is resident while V of tile t is still
// being read and tile t+2 is being filled.
// ---------------------------------------------------------------------------
template <int NW>
__global__ __launch_bounds__(NW * 64) void partial_bf16_d128_pipe_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NKB = 2, NDS = 8;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KBYTES = BN * D * 2;
  constexpr int STAGE = 2 * KBYTES;
  constexpr int KCH = BN * 16 / NT;
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  static_assert(NT == 512 && KCH == 2, "the V staging below assumes 8 waves (2 keys per thread)");
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;
  const int row = r0 + l32;

  int n_end = a.Sk;
  if (a.causal) n_end = max(0, min(a.Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;
  // tiles [0, w_tiles) hold a key some row of this wave can see (visibility is monotone)
  int w_tiles = 0;
  if (r0 < a.Sq) {
    const int w_end = a.causal ? max(0, min(n_end, min(r0 + 32, a.Sq) - dpos)) : n_end;
    w_tiles = (w_end + BN - 1) / BN;
  }

  Blk bk;
#pragma unroll
  for (int db = 0; db < 4; ++db) bk.o[db] = (f32x16){};
  bk.m = kNegInf;
  bk.l = 0.f;

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
      const bool ok = row < a.Sq;
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[s] = ok ? as_bf16x8(ld_global16(qr + 16 * s)) : (bf16x8){};
    }
    int koff[NDS];
#pragma unroll
    for (int s = 0; s < NDS; ++s) koff[s] = l32 * (D * 2) + (((2 * s + g) ^ (l32 & 15)) << 4);
    int voff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) voff[u] = KBYTES + l32 * 128 + (((2 * u + g) ^ vt_swz(l32)) << 4);

    const __bf16* ksrc[KCH];
    int kkey[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int slot = i * NT + wave * 64 + lane;
      kkey[i] = slot >> 4;
      ksrc[i] = kp + (int64_t)kkey[i] * a.k_ss + (((slot & 15) ^ (kkey[i] & 15)) * 8);
    }
    const int vkg = tid >> 4, vch = tid & 15;
    const __bf16* vsrc = vp + (int64_t)(2 * vkg) * a.v_ss + vch * 8;
    int vwoff[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) vwoff[w] = KBYTES + vt_offset(vch * 8 + 2 * w, vkg >> 1) + (vkg & 1) * 4;

    u32x4 vreg[2];
    auto load_tile = [&](int t, int stage) {
      const int n0 = t * BN;
      const bool tail = n0 + BN > a.Sk;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const __bf16* src = tail ? kp + (int64_t)min(n0 + kkey[i], a.Sk - 1) * a.k_ss +
                                       (((i * NT + wave * 64 + lane) & 15) ^ (kkey[i] & 15)) * 8
                                 : ksrc[i] + (int64_t)n0 * a.k_ss;
        uint8_t* dst = smem + stage * STAGE + (i * NT + wave * 64) * 16;
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
      }
      const __bf16* vs0 = vsrc + (int64_t)n0 * a.v_ss;
      vreg[0] = (!tail || n0 + 2 * vkg < a.Sk) ? ld_global16(vs0) : (u32x4){};
      vreg[1] = (!tail || n0 + 2 * vkg + 1 < a.Sk) ? ld_global16(vs0 + a.v_ss) : (u32x4){};
    };
    auto store_v = [&](int stage) {
      uint8_t* vs = smem + stage * STAGE;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint32_t*>(vs + vwoff[w]) = pack_lo16(vreg[0][w], vreg[1][w]);
        *reinterpret_cast<uint32_t*>(vs + vwoff[w] + 128) = pack_hi16(vreg[0][w], vreg[1][w]);
      }
    };
    auto qk = [&](const uint8_t* base, f32x16 (&sc)[NKB]) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x16 x = (f32x16){};
#pragma unroll
        for (int s = 0; s < NDS; ++s) x = mfma32(as_bf16x8(ld_lds16(base + koff[s] + kb * 32 * (D * 2))), qf[s], x);
        sc[kb] = x;
      }
    };
    auto mask_tile = [&](int t, f32x16 (&sc)[NKB]) {
      const int n0 = t * BN;
      if (n0 + BN > a.Sk || (a.causal && dpos + n0 + BN - 1 > r0)) {
        int lim = a.Sk - n0;
        if (a.causal) lim = min(lim, row - dpos - n0 + 1);
        mask_block<NKB>(sc, max(0, min(lim, BN)), g);
      }
    };

    f32x16 sc[NKB], sn[NKB];
    // prologue: tiles 0 and 1 in flight, S(0) computed
    load_tile(0, 0);
    store_v(0);
    if (n_tiles > 1) load_tile(1, 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (n_tiles > 1) store_v(1);
    __syncthreads();
    if (w_tiles > 0) qk(smem, sc);

    auto tile = [&](int t, auto cur_tag) {
      constexpr int CUR = decltype(cur_tag)::value;
      constexpr int NXT = (CUR + 1) % 3, NN = (CUR + 2) % 3;
      const bool load2 = (t + 2) < n_tiles;
      if (load2) load_tile(t + 2, NN);
      if (t < w_tiles) {
        mask_tile(t, sc);
        // ---- branch-free block: S(t+1) MFMAs interleaved with the softmax of S(t)
        float mx = sc[0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
        mx = pair32_max(mx);
        const float mt = mx * SCALE_LOG2;
        const bool raise = __any(mt > bk.m + kTau);
        const float m_new = raise ? fmaxf(bk.m, mt) : bk.m;
        const float mref = (m_new == kNegInf) ? 0.f : m_new;
        // rare: raise the reference max of O and l (before the interleaved
        // block, so nothing separates the exps from the MFMAs they hide under)
        if (raise) {
          const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(bk.m - m_new);
          bk.l *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) bk.o[db] *= alpha;
        }
        bk.m = m_new;
        // the interleaved block below holds only MFMA work of tile t+1 and
        // the exp / sum / convert work of tile t, which depend on nothing else
        __builtin_amdgcn_sched_barrier(0);
        u32x4 pk[NKB][2];
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            p[i] = fast_exp2(fmaf(sc[kb][i], SCALE_LOG2, -mref));
            lsum += p[i];
          }
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
            pk[kb][t2] = (u32x4){pack_bf16(p[8 * t2 + 0], p[8 * t2 + 1]), pack_bf16(p[8 * t2 + 2], p[8 * t2 + 3]),
                                 pack_bf16(p[8 * t2 + 4], p[8 * t2 + 5]), pack_bf16(p[8 * t2 + 6], p[8 * t2 + 7])};
        }
        // unconditional, so this stays one basic block; after the wave's last
        // visible tile the result is simply not used
        qk(smem + NXT * STAGE, sn);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // K operand reads run four ahead
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                 // next K operand read
          __builtin_amdgcn_sched_group_barrier(0x402, CPATTN_PIPE_VALU, 0);  // exp / sum / convert (VALU | TRANS)
        }
        __builtin_amdgcn_sched_barrier(0);
        bk.l += lsum;
        // ---- O^T += V^T P^T for tile t
        const uint8_t* base = smem + CUR * STAGE;
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            bk.o[db] = mfma32(as_bf16x8(ld_lds16(base + voff[u] + db * 32 * 128)), as_bf16x8(pk[u >> 1][u & 1]), bk.o[db]);
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sc[kb] = sn[kb];
      }
      if (load2) store_v(NN);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 3) {
      tile(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 < n_tiles) tile(t + 2, std::integral_constant<int, 2>{});
    }
  }

  const float l_tot = pair32_sum(bk.l);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {bk.o[db][4 * i4 + 0] * inv, bk.o[db][4 * i4 + 1] * inv, bk.o[db][4 * i4 + 2] * inv,
                          bk.o[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (bk.m + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// Ping-pong D = 128 kernel.  The 8 waves form two groups (waves 0-3 and 4-7;
// one wave of each group per SIMD).  Time is cut into phases separated by
// workgroup barriers; in every phase one group runs its MFMA work (P.V of
// tile t-1 and Q.K^T of tile t) while the other runs its softmax (of the tile
// whose scores it produced in its previous phase).  So each SIMD always has
// one wave feeding the matrix core and one wave on the vector ALUs.
//
// Tile t's K is read in phases 2t (group 0) and 2t+1 (group 1); its V in
// phases 2t+2 and 2t+3.  K and V therefore sit in separate double buffers:
// K(t+1) and V(t) are fetched during phases 2t and 2t+1 (K straight into LDS,
// V through registers and stored transposed at the end of phase 2t+1).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void partial_bf16_d128_pp_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NKB = 2, NDS = 8, NW = 8, NT = 512;
  constexpr int BM = NW * 32;
  constexpr int KBYTES = BN * D * 2;   // one K tile == one V^T tile
  constexpr int KCH = BN * 16 / NT;    // 2
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  // layout: K buffer 0 | K buffer 1 | V^T buffer 0 | V^T buffer 1
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * KBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int group = wave >> 2;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;
  const int row = r0 + l32;

  int n_end = a.Sk;
  if (a.causal) n_end = max(0, min(a.Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;
  int w_tiles = 0;  // tiles [0, w_tiles) hold a key some row of this wave can see
  if (r0 < a.Sq) {
    const int w_end = a.causal ? max(0, min(n_end, min(r0 + 32, a.Sq) - dpos)) : n_end;
    w_tiles = (w_end + BN - 1) / BN;
  }

  Blk bk;
#pragma unroll
  for (int db = 0; db < 4; ++db) bk.o[db] = (f32x16){};
  bk.m = kNegInf;
  bk.l = 0.f;

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
      const bool ok = row < a.Sq;
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[s] = ok ? as_bf16x8(ld_global16(qr + 16 * s)) : (bf16x8){};
    }
    int koff[NDS];
#pragma unroll
    for (int s = 0; s < NDS; ++s) koff[s] = l32 * (D * 2) + (((2 * s + g) ^ (l32 & 15)) << 4);
    int voff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) voff[u] = l32 * 128 + (((2 * u + g) ^ vt_swz(l32)) << 4);

    const __bf16* ksrc[KCH];
    int kkey[KCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int slot = i * NT + wave * 64 + lane;
      kkey[i] = slot >> 4;
      ksrc[i] = kp + (int64_t)kkey[i] * a.k_ss + (((slot & 15) ^ (kkey[i] & 15)) * 8);
    }
    const int vkg = tid >> 4, vch = tid & 15;
    const __bf16* vsrc = vp + (int64_t)(2 * vkg) * a.v_ss + vch * 8;
    int vwoff[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) vwoff[w] = vt_offset(vch * 8 + 2 * w, vkg >> 1) + (vkg & 1) * 4;

    auto load_k = [&](int t) {
      const int n0 = t * BN;
      const bool tail = n0 + BN > a.Sk;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const __bf16* src = tail ? kp + (int64_t)min(n0 + kkey[i], a.Sk - 1) * a.k_ss +
                                       (((i * NT + wave * 64 + lane) & 15) ^ (kkey[i] & 15)) * 8
                                 : ksrc[i] + (int64_t)n0 * a.k_ss;
        uint8_t* dst = smem + (t & 1) * KBYTES + (i * NT + wave * 64) * 16;
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
      }
    };
    u32x4 vreg[2];
    auto load_v = [&](int t) {
      const int n0 = t * BN;
      const bool tail = n0 + BN > a.Sk;
      const __bf16* vs0 = vsrc + (int64_t)n0 * a.v_ss;
      vreg[0] = (!tail || n0 + 2 * vkg < a.Sk) ? ld_global16(vs0) : (u32x4){};
      vreg[1] = (!tail || n0 + 2 * vkg + 1 < a.Sk) ? ld_global16(vs0 + a.v_ss) : (u32x4){};
    };
    auto store_v = [&](int t) {
      uint8_t* vs = smem + (2 + (t & 1)) * KBYTES;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint32_t*>(vs + vwoff[w]) = pack_lo16(vreg[0][w], vreg[1][w]);
        *reinterpret_cast<uint32_t*>(vs + vwoff[w] + 128) = pack_hi16(vreg[0][w], vreg[1][w]);
      }
    };

    f32x16 sc[NKB];
    u32x4 pk[NKB][2];

    load_k(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const int n_phases = 2 * n_tiles + 2;
    for (int p = 0; p < n_phases; ++p) {
      const bool even = (p & 1) == 0;
      const int tl = p >> 1;
      if (even) {
        if (tl + 1 < n_tiles) load_k(tl + 1);
        if (tl < n_tiles) load_v(tl);
      }
      STAMP(wave, p, 0, L);
      const int lp_ = p - group;  // this wave's own phase
      if (lp_ >= 0) {
        const int t = lp_ >> 1;
        if ((lp_ & 1) == 0) {
          // ---- MFMA phase: O += P(t-1) V(t-1), then S(t) = K(t) Q^T
          if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
          if (t >= 1 && t - 1 < w_tiles) {
            const uint8_t* vb = smem + (2 + ((t - 1) & 1)) * KBYTES;
            u32x4 vop[4][4];
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int u = 0; u < 4; ++u) vop[db][u] = ld_lds16(vb + voff[u] + db * 32 * 128);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int u = 0; u < 4; ++u)
                bk.o[db] = mfma32(as_bf16x8(vop[db][u]), as_bf16x8(pk[u >> 1][u & 1]), bk.o[db]);
          }
          if (t < w_tiles) {
            const uint8_t* kb_ = smem + (t & 1) * KBYTES;
            u32x4 kop[NKB][NDS];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int s2 = 0; s2 < NDS; ++s2) kop[kb][s2] = ld_lds16(kb_ + koff[s2] + kb * 32 * (D * 2));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              f32x16 x = (f32x16){};
#pragma unroll
              for (int s2 = 0; s2 < NDS; ++s2) x = mfma32(as_bf16x8(kop[kb][s2]), qf[s2], x);
              sc[kb] = x;
            }
          }
          if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
        } else if (t < w_tiles) {
          // ---- softmax phase for tile t
          const int n0 = t * BN;
          if (n0 + BN > a.Sk || (a.causal && dpos + n0 + BN - 1 > r0)) {
            int lim = a.Sk - n0;
            if (a.causal) lim = min(lim, row - dpos - n0 + 1);
            mask_block<NKB>(sc, max(0, min(lim, BN)), g);
          }
          softmax_block<NKB>(sc, bk, pk, SCALE_LOG2);
        }
      }
      STAMP(wave, p, 1, L);
      if (!even) {
        if (tl < n_tiles) store_v(tl);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      STAMP(wave, p, 2, L);
      __syncthreads();
      STAMP(wave, p, 3, L);
    }
  }

  const float l_tot = pair32_sum(bk.l);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {bk.o[db][4 * i4 + 0] * inv, bk.o[db][4 * i4 + 1] * inv, bk.o[db][4 * i4 + 2] * inv,
                          bk.o[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (bk.m + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// D = 128 kernel, third form: both K and V tiles go straight from global
// memory into LDS (global_load_lds_dwordx4), three LDS stages deep (the tile
// two ahead is in flight while the current one is used), and the V^T operand
// of O^T = V^T P^T is read from the row-major V tile with the gfx950
// transposing LDS read ds_read_b64_tr_b16.  Within a 16-lane group that read
// hands lane 4a+b element b of the 8-byte rows addressed by lanes a, a+4, a+8
// and a+12; so when lane s addresses row key0 + s/4 at columns D0 + 4(s%4),
// lane i receives V[key0 .. key0+3][D0 + i] -- four keys of one column.
//
// LDS stage = K tile (64 keys x 256 B, 16-byte chunks XOR-swizzled by
// key & 15) + V tile (64 keys x 256 B, chunks XOR-swizzled by 4 (key & 3)).
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u32x2 ld_lds8_tr(const uint8_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(__attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

__global__ __launch_bounds__(512) void partial_bf16_d128_v3_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NKB = 2, NDS = 8, NT = 512, BM = 256;
  constexpr int TBYTES = BN * D * 2;  // one K or V tile
  constexpr int STAGE = 2 * TBYTES;   // K then V
  constexpr int NST = 3;
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;
  const int row = r0 + l32;

  int n_end = a.Sk;
  if (a.causal) n_end = max(0, min(a.Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;

  Blk bk;
#pragma unroll
  for (int db = 0; db < 4; ++db) bk.o[db] = (f32x16){};
  bk.m = kNegInf;
  bk.l = 0.f;

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
      const bool ok = row < a.Sq;
#pragma unroll
      for (int s2 = 0; s2 < NDS; ++s2) qf[s2] = ok ? as_bf16x8(ld_global16(qr + 16 * s2)) : (bf16x8){};
    }
    // K operand of k-step s: row l32 (+32 per key block), chunk 2s+g swizzled by the row
    int koff[NDS];
#pragma unroll
    for (int s2 = 0; s2 < NDS; ++s2) koff[s2] = l32 * 256 + (((2 * s2 + g) ^ (l32 & 15)) << 4);
    // V^T operand, column block db: this lane addresses key 4g + ks (+16u + 8 half) at
    // columns 32 db + 16 c16 + 4 (s & 3), chunk swizzled by 4 ks
    int voff[4];
    {
      const int s16 = lane & 15, ks = s16 >> 2, c16 = l32 >> 4, c8 = (s16 & 3) >> 1, bo = (s16 & 1) * 8;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        voff[db] = TBYTES + (4 * g + ks) * 256 + ((4 * (db ^ ks) + 2 * c16 + c8) << 4) + bo;
    }
    // fetch slots: 16-byte slot i*NT + wave*64 + lane of a tile holds key slot>>4,
    // physical chunk slot&15 (logical chunk for K: ^ (key & 15), for V: ^ 4 (key & 3))
    int fkey[2], fkch[2], fvch[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = i * NT + wave * 64 + lane;
      fkey[i] = slot >> 4;
      fkch[i] = (slot & 15) ^ (fkey[i] & 15);
      fvch[i] = (slot & 15) ^ (4 * (fkey[i] & 3));
    }
    const uint32_t lbase = lds_addr(smem);
    auto load_tile = [&](int t, int stage) {
      const int n0 = t * BN;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // rows past the block end are clamped to the last row: their scores are
        // masked to -inf and their p is exactly 0
        const int64_t key = min(n0 + fkey[i], a.Sk - 1);
        const uint32_t dst = lbase + stage * STAGE + (i * NT + wave * 64) * 16;
        gload_lds16(kp + key * a.k_ss + fkch[i] * 8, dst);
        gload_lds16(vp + key * a.v_ss + fvch[i] * 8, dst + TBYTES);
      }
    };

    auto tile = [&](int t, auto stage_tag) {
      constexpr int ST = decltype(stage_tag)::value;
      constexpr int LD = (ST + 2) % NST;
      const bool do_load = (t + 2) < n_tiles;
      if (do_load) load_tile(t + 2, LD);
      const uint8_t* base = smem + ST * STAGE;
      const int n0 = t * BN;
      const bool wave_active = (r0 < a.Sq) && (!a.causal || dpos + n0 <= r0 + 31);
      if (wave_active) {
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
        f32x16 sc[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          u32x4 kop[NDS];
#pragma unroll
          for (int s2 = 0; s2 < NDS; ++s2) kop[s2] = ld_lds16(base + koff[s2] + kb * 32 * 256);
          f32x16 x = (f32x16){};
#pragma unroll
          for (int s2 = 0; s2 < NDS; ++s2) x = mfma32(as_bf16x8(kop[s2]), qf[s2], x);
          sc[kb] = x;
        }
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
        if (n0 + BN > a.Sk || (a.causal && dpos + n0 + BN - 1 > r0)) {
          int lim = a.Sk - n0;
          if (a.causal) lim = min(lim, row - dpos - n0 + 1);
          mask_block<NKB>(sc, max(0, min(lim, BN)), g);
        }
        u32x4 pk[NKB][2];
        softmax_block<NKB>(sc, bk, pk, SCALE_LOG2);
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x2 lo = ld_lds8_tr(base + voff[db] + (16 * u) * 256);
            const u32x2 hi = ld_lds8_tr(base + voff[db] + (16 * u + 8) * 256);
            const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
            bk.o[db] = mfma32(as_bf16x8(av), as_bf16x8(pk[u >> 1][u & 1]), bk.o[db]);
          }
        }
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
      }
      // tile t+1's K and V (fetched two tiles ago) must have landed; the fetch
      // of tile t+2 (4 transfers per thread) stays in flight
      if (do_load)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    load_tile(0, 0);
    if (n_tiles > 1) load_tile(1, 1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int t = 0; t < n_tiles; t += 3) {
      tile(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) tile(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 < n_tiles) tile(t + 2, std::integral_constant<int, 2>{});
    }
  }

  const float l_tot = pair32_sum(bk.l);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {bk.o[db][4 * i4 + 0] * inv, bk.o[db][4 * i4 + 1] * inv, bk.o[db][4 * i4 + 2] * inv,
                          bk.o[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (bk.m + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}


// ---------------------------------------------------------------------------
// D = 128 kernel, fourth form: the third form's data movement (K and V
// direct to LDS, V^T through the transposing read), with each wave's work
// software-pipelined so that its matrix and vector work overlap.  Iteration t
// runs two phases:
//   A: S(t+1) = K(t+1) Q^T on the matrix cores, while the vector unit packs
//      P(t) to bf16 and adds it to the row sums;
//   B: O^T += V(t)^T P(t)^T on the matrix cores, while the vector unit takes
//      the row maxima of S(t+1), moves the running reference and evaluates
//      the exponentials P(t+1).
// Each MFMA is followed by its slice of the vector work, and a scheduling
// fence after every slice keeps the compiler from regrouping them.  The O
// rescale a moved reference needs (rare, see kTau) runs after phase B, once
// P(t) has been accumulated against the old reference.
// ---------------------------------------------------------------------------
// Empty asm that claims to rewrite x: the value must be computed before this
// point (passes that sink or hoist code cannot move it past), which keeps the
// vector work of the pipelined loop in the slot it was written in.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

template <int NST>
__global__ __launch_bounds__(512) void partial_bf16_d128_v4_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NDS = 8, NT = 512, BM = 256;
  constexpr int TBYTES = BN * D * 2;  // one K or V tile
  constexpr int STAGE = 2 * TBYTES;   // K then V
  constexpr int KLA = CPATTN_V4_KLA;            // K operand reads issued this many MFMAs ahead
  constexpr int VLA = CPATTN_V4_VLA;            // V operand reads issued this many MFMAs ahead
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  static_assert(NST == 3 || NST == 4, "3 or 4 LDS stages");
  __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int bh = a.B * a.Hq;
  const int per_item = bh * n_qtiles;
  const int L = xcd_logical_block(blockIdx.x, per_item * a.n_items);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh;
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;
  const int row = r0 + l32;

  int n_end = a.Sk;
  if (a.causal) n_end = max(0, min(a.Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  float m = kNegInf;  // running reference (log2 domain) of this lane's row
  float l = 0.f;      // this lane's share of the row sum, relative to m

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      const __bf16* qr = qp + (int64_t)row * a.q_ss + 8 * g;
      const bool ok = row < a.Sq;
#pragma unroll
      for (int s2 = 0; s2 < NDS; ++s2) qf[s2] = ok ? as_bf16x8(ld_global16(qr + 16 * s2)) : (bf16x8){};
    }
    int koff[NDS];
#pragma unroll
    for (int s2 = 0; s2 < NDS; ++s2) koff[s2] = l32 * 256 + (((2 * s2 + g) ^ (l32 & 15)) << 4);
    int voff[4];
    {
      const int s16 = lane & 15, ks = s16 >> 2, c16 = l32 >> 4, c8 = (s16 & 3) >> 1, bo = (s16 & 1) * 8;
#pragma unroll
      for (int db = 0; db < 4; ++db)
        voff[db] = TBYTES + (4 * g + ks) * 256 + ((4 * (db ^ ks) + 2 * c16 + c8) << 4) + bo;
    }
    // Fetch: 16-byte slot i*NT + wave*64 + lane of a tile holds key slot>>4 at
    // physical chunk slot&15.  The source pointers advance one tile per fetch.
    int fkey[2];
    const __bf16* kf[2];
    const __bf16* vf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int slot = i * NT + wave * 64 + lane;
      fkey[i] = slot >> 4;
      kf[i] = kp + fkey[i] * a.k_ss + (((slot & 15) ^ (fkey[i] & 15)) << 3);
      vf[i] = vp + fkey[i] * a.v_ss + (((slot & 15) ^ (4 * (fkey[i] & 3))) << 3);
    }
    const int64_t kstep = (int64_t)BN * a.k_ss, vstep = (int64_t)BN * a.v_ss;
    const uint32_t lbase = lds_addr(smem) + wave * 64 * 16;
    int n_fetched = 0;
    auto fetch = [&](int stage) {
      const uint32_t dst = lbase + stage * STAGE;
      if ((n_fetched + 1) * BN <= a.Sk) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          gload_lds16(kf[i], dst + i * NT * 16);
          gload_lds16(vf[i], dst + i * NT * 16 + TBYTES);
        }
      } else {
        // rows past the block end re-read the last row: their scores are masked
        // to -inf, so their p is exactly 0
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int over = max(0, n_fetched * BN + fkey[i] - (a.Sk - 1));
          gload_lds16(kf[i] - over * a.k_ss, dst + i * NT * 16);
          gload_lds16(vf[i] - over * a.v_ss, dst + i * NT * 16 + TBYTES);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        kf[i] += kstep;
        vf[i] += vstep;
      }
      ++n_fetched;
    };

    auto mask_tile = [&](f32x16 (&sc)[2], int t) -> bool {
      const int n0 = t * BN;
      if (n0 + BN > a.Sk || (a.causal && dpos + n0 + BN - 1 > r0)) {
        int lim = a.Sk - n0;
        if (a.causal) lim = min(lim, row - dpos - n0 + 1);
        mask_block<2>(sc, max(0, min(lim, BN)), g);
        return true;
      }
      return false;
    };

    // Scores of the newest tile (sn), the packed probabilities of the tile
    // being accumulated (pw: word w holds p[2w], p[2w+1] of this lane's 32
    // keys, words 0..7 from key block 0, 8..15 from key block 1), and the
    // state of the reference move made for the newest tile.
    f32x16 sn[2];
    uint32_t pw[16];
    bool need = false;
    float alpha = 1.f;
    float mref = 0.f;
    // max over scores f0 .. f1-1 of key block kb (mx must already hold a value
    // unless this starts at score 0 of key block 0)
    auto part_max = [&](float& mx, int kb, int f0, int f1) {
#pragma unroll
      for (int f = f0; f < f1; ++f) mx = (kb == 0 && f == 0) ? sn[0][0] : fmaxf(mx, sn[kb][f]);
    };
    // reference move for the newest tile: the row sum is rescaled at once, O
    // before the next PV phase (the current one still adds old-reference terms)
    auto move_ref = [&](float mx) {
      mx = pair32_max(mx);
      const float mt = mx * SCALE_LOG2;
      need = __any(mt > m + kTau);
      const float m_new = need ? fmaxf(m, mt) : m;
      alpha = (m_new == m) ? 1.f : fast_exp2(m - m_new);
      l *= alpha;
      m = m_new;
      mref = (m == kNegInf) ? 0.f : m;
    };
    // probabilities of scores 2w, 2w+1 of key block kb -> packed word, row sum
    auto prob_pair = [&](const f32x16& x, int w) -> uint32_t {
      const float p0 = fast_exp2(fmaf(x[2 * w], SCALE_LOG2, -mref));
      const float p1 = fast_exp2(fmaf(x[2 * w + 1], SCALE_LOG2, -mref));
      l += p0 + p1;
      return pack_bf16(p0, p1);
    };

    // prologue: tiles 0 .. NST-2 in flight, wait for tiles 0 and 1
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
      if (i < n_tiles) fetch(i);
    if (NST == 4 && n_tiles > 2)
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    {
      sn[0] = (f32x16){};
      sn[1] = (f32x16){};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        sn[j >> 3] = mfma32(as_bf16x8(ld_lds16(smem + koff[j & 7] + (j >> 3) * 8192)), qf[j & 7], sn[j >> 3]);
      mask_tile(sn, 0);
      float mx;
      part_max(mx, 0, 0, 16);
      part_max(mx, 1, 0, 16);
      move_ref(mx);
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[w] = prob_pair(sn[0], w);
    }

    // Iteration t.  The last one also computes scores for the tile after the
    // last: every one of them is masked (that tile starts at or past the
    // block's last visible key), so its max is -inf, the reference stays and
    // its probabilities are 0; its K operands come from a stale stage.
    auto iteration = [&](int t, auto st_tag) {
      constexpr int ST = decltype(st_tag)::value;
      constexpr int SN = (ST + 1) % NST;
      constexpr int SL = (ST + NST - 1) % NST;
      const uint8_t* cur = smem + ST * STAGE;
      const uint8_t* nxt = smem + SN * STAGE;
      const bool do_fetch = t + NST - 1 < n_tiles;
      if (do_fetch) fetch(SL);

      u32x4 kop[16];
      u32x2 vlo[16], vhi[16];
      auto read_v = [&](int jj) {  // operands of PV MFMA jj: u = jj >> 2, db = jj & 3
        const int u = jj >> 2, db = jj & 3;
        vlo[jj] = ld_lds8_tr(cur + voff[db] + (16 * u) * 256);
        vhi[jj] = ld_lds8_tr(cur + voff[db] + (16 * u + 8) * 256);
      };
      // ---- phase A: S(t+1) = K(t+1) Q^T; key block 1 of P(t) ----
      const f32x16 s1 = sn[1];  // scores of tile t, key block 1
      f32x16 x[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int j = 0; j < KLA; ++j) kop[j] = ld_lds16(nxt + koff[j & 7] + (j >> 3) * 8192);
      __builtin_amdgcn_sched_barrier(0);
      float mx0 = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + KLA < 16) kop[j + KLA] = ld_lds16(nxt + koff[(j + KLA) & 7] + ((j + KLA) >> 3) * 8192);
        if (j >= 16 - VLA) read_v(j - (16 - VLA));
        x[j >> 3] = mfma32(as_bf16x8(kop[j]), qf[j & 7], x[j >> 3]);
        if (j < 8) {
          pw[8 + j] = prob_pair(s1, j);
          pin(pw[8 + j]);
          pin(l);
        }
        if (j >= 9) {
          // running max over key block 0 of tile t+1 (done by the 8th MFMA)
#pragma unroll
          for (int f = (j == 9) ? 0 : 2 * j - 16; f < 2 * j - 14; ++f) mx0 = (f == 0) ? x[0][0] : fmaxf(mx0, x[0][f]);
          pin(mx0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      sn[0] = x[0];
      sn[1] = x[1];
      if (mask_tile(sn, t + 1)) part_max(mx0, 0, 0, 16);
      __builtin_amdgcn_sched_barrier(0);

      // ---- phase B: O^T += V(t)^T P(t)^T; row max, reference, key block 0 of P(t+1) ----
      uint32_t pn[8];
      float mx = mx0;
      // O still holds terms against the reference before the last move
      if (need) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        if (jj + VLA < 16) read_v(jj + VLA);
        const int u = jj >> 2, db = jj & 3;
        const u32x4 av = {vlo[jj][0], vlo[jj][1], vhi[jj][0], vhi[jj][1]};
        const u32x4 bp = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
        o[db] = mfma32(as_bf16x8(av), as_bf16x8(bp), o[db]);
        if (jj <= 1) {
          part_max(mx, 1, 8 * jj, 8 * jj + 8);
          pin(mx);
        } else if (jj == 2) {
          move_ref(mx);
          pin(l);
          pin(alpha);
          pin(mref);
        } else if (jj <= 10) {
          pn[jj - 3] = prob_pair(sn[0], jj - 3);
          pin(pn[jj - 3]);
          pin(l);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) pw[w] = pn[w];
      // tile t+2 must have landed; fetches of later tiles stay in flight
      if (NST == 4 && do_fetch)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    for (int t = 0; t < n_tiles; t += NST) {
      iteration(t, std::integral_constant<int, 0>{});
      if (t + 1 < n_tiles) iteration(t + 1, std::integral_constant<int, 1>{});
      if (t + 2 < n_tiles) iteration(t + 2, std::integral_constant<int, 2>{});
      if constexpr (NST == 4)
        if (t + 3 < n_tiles) iteration(t + 3, std::integral_constant<int, 3 % NST>{});
    }
  }

  const float l_tot = pair32_sum(l);
  if (row < a.Sq) {
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 v4 = {o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv, o[db][4 * i4 + 2] * inv,
                          o[db][4 * i4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
      }
    if (g == 0) lp[(int64_t)row * a.l_ss] = (l_tot > 0.f) ? (m + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

int partial_bf16_rows_per_block(int D) { return D == 128 ? CPATTN_D128_NW * 32 : 128; }

hipError_t launch_partial_bf16(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s) {
  const long long blocks = (long long)a.n_items * a.B * a.Hq * n_qtiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128)
    if (CPATTN_D128_PIPE == 4)
      hipLaunchKernelGGL(partial_bf16_d128_v4_kernel<CPATTN_D128_V4_STAGES>, dim3((unsigned)blocks), dim3(512), 0, s, a,
                         n_qtiles);
    else if (CPATTN_D128_PIPE == 3)
      hipLaunchKernelGGL(partial_bf16_d128_v3_kernel, dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
    else if (CPATTN_D128_PIPE == 2)
      hipLaunchKernelGGL(partial_bf16_d128_pp_kernel, dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
    else if (CPATTN_D128_PIPE == 1)
      hipLaunchKernelGGL((partial_bf16_d128_pipe_kernel<CPATTN_D128_NW>), dim3((unsigned)blocks),
                         dim3(CPATTN_D128_NW * 64), 0, s, a, n_qtiles);
    else
      hipLaunchKernelGGL((partial_bf16_d128_kernel<CPATTN_D128_NW>), dim3((unsigned)blocks),
                         dim3(CPATTN_D128_NW * 64), 0, s, a, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL(partial_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn

#ifdef CPATTN_TIMING
extern "C" int cpattn_debug_stamps(unsigned long long* host, int n) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(cpattn::g_cpattn_stamps), sizeof(unsigned long long) * n, 0,
                                  hipMemcpyDeviceToHost);
}
#endif
