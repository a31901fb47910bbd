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
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

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
#ifndef CPATTN_D128_BN
#define CPATTN_D128_BN 64  // keys per K/V tile
#endif
#ifndef CPATTN_D128_RB
#define CPATTN_D128_RB 1   // 32-row query blocks per wave
#endif
#ifndef CPATTN_D128_NW
#define CPATTN_D128_NW 8   // waves per workgroup
#endif
#ifndef CPATTN_D128_PRIO
#define CPATTN_D128_PRIO 1  // raise wave priority during the MFMA phases
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

template <int NKB>
__device__ __forceinline__ void mask_block(f32x16 (&s)[NKB], int lim, int g) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
      s[kb][i] = (kl < lim) ? s[kb][i] : kNegInf;
    }
}

// V^T tile of the D = 128 kernel: row d holds the BN keys of the tile.  Inside
// each 16-key group the 4-key groups are stored in the order 0, 2, 1, 3, so
// the 8 keys that lane group g feeds to one PV k-step (keys 4g..4g+3 and
// 8+4g..8+4g+3) are 16 contiguous bytes.  16-byte units are XOR-swizzled by
// row so 16 consecutive rows hit distinct banks.
template <int BN>
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 4)) & (BN / 8 - 1); }
template <int BN>
__device__ __forceinline__ int vt_offset(int d, int kg) {
  const int kp = (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);  // swap the two low bits of the group index
  return d * (BN * 2) + ((((kp >> 1) ^ vt_swz<BN>(d))) << 4) + ((kp & 1) << 3);
}

template <int BN, int RB, int NW>
__global__ __launch_bounds__(NW * 64) void partial_bf16_d128_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, DCH = 16, NKB = BN / 32, NDS = 8;
  constexpr int NT = NW * 64;                 // threads
  constexpr int BM = NW * 32 * RB;            // query rows per workgroup
  constexpr int KBYTES = BN * D * 2, STAGE = 2 * KBYTES, VROW = BN * 2;
  constexpr int KCH = BN * DCH / NT;          // 16-byte K chunks per thread (direct to LDS)
  constexpr int KPV = BN * DCH / NT;          // V keys per thread (one 16-byte chunk each)
  constexpr float SCALE_LOG2 = 0.12751743082459868f;
  static_assert(KCH >= 1 && (KPV == 2 || KPV == 4), "tile split");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

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

  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32 * RB;  // first row of this wave; block r covers r0 + 32 r ..
  int row[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) row[r] = r0 + 32 * r + l32;

  int n_end = a.Sk;
  if (a.causal) {
    const int64_t last_row = (int64_t)min(m0 + BM, a.Sq) - 1;
    n_end = (int)max<int64_t>(0, min<int64_t>(a.Sk, qpos0 + last_row - kvpos0 + 1));
  }
  const int n_tiles = (n_end + BN - 1) / BN;

  Blk blk[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
#pragma unroll
    for (int db = 0; db < 4; ++db) blk[r].o[db] = (f32x16){};
    blk[r].m = kNegInf;
    blk[r].l = 0.f;
  }

  if (n_tiles > 0) {
    bf16x8 qf[RB][NDS];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const __bf16* qr = qp + (int64_t)row[r] * a.q_ss + 8 * g;
      const bool ok = row[r] < a.Sq;
#pragma unroll
      for (int s = 0; s < NDS; ++s) qf[r][s] = ok ? as_bf16x8(ld_global16(qr + 16 * s)) : (bf16x8){};
    }

    // K: instruction i of wave w fills the 16-byte LDS slots i*NT + w*64 + lane
    auto load_k = [&](int t, int stage) {
      const int n0 = t * BN;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int slot = i * NT + wave * 64 + lane;
        const int key = slot >> 4;
        const int ch = (slot & 15) ^ (key & 15);
        const int gkey = min(n0 + key, a.Sk - 1);  // rows past the block end are masked later
        const __bf16* src = kp + (int64_t)gkey * a.k_ss + ch * 8;
        uint8_t* dst = smem + stage * STAGE + (i * NT + wave * 64) * 16;
        __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)dst, 16, 0, 0);
      }
    };
    // V: thread owns KPV consecutive keys of one 16-byte d chunk
    u32x4 vreg[KPV];
    const int vkg = tid >> 4, vch = tid & 15;
    auto load_v = [&](int t) {
      const int n0 = t * BN;
#pragma unroll
      for (int kk = 0; kk < KPV; ++kk) {
        const int key = n0 + KPV * vkg + kk;
        vreg[kk] = (key < a.Sk) ? ld_global16(vp + (int64_t)key * a.v_ss + vch * 8) : (u32x4){};
      }
    };
    auto store_v = [&](int stage) {
      uint8_t* vs = smem + stage * STAGE + KBYTES;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int de = vch * 8 + 2 * w;
        const int dodd = de + 1;
        if constexpr (KPV == 4) {
          const int kg = vkg;  // 4-key group
          const u32x2 ev = {pack_lo16(vreg[0][w], vreg[1][w]), pack_lo16(vreg[2][w], vreg[3][w])};
          const u32x2 od = {pack_hi16(vreg[0][w], vreg[1][w]), pack_hi16(vreg[2][w], vreg[3][w])};
          st_lds8(vs + vt_offset<BN>(de, kg), ev);
          st_lds8(vs + vt_offset<BN>(dodd, kg), od);
        } else {
          const int kg = vkg >> 1, half = (vkg & 1) * 4;  // two keys: 4 bytes of a 4-key group
          *reinterpret_cast<uint32_t*>(vs + vt_offset<BN>(de, kg) + half) = pack_lo16(vreg[0][w], vreg[1][w]);
          *reinterpret_cast<uint32_t*>(vs + vt_offset<BN>(dodd, kg) + half) = pack_hi16(vreg[0][w], vreg[1][w]);
        }
      }
    };

    load_k(0, 0);
    load_v(0);
    store_v(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
      const bool has_next = (t + 1) < n_tiles;
      if (has_next) {
        load_k(t + 1, (t + 1) & 1);
        load_v(t + 1);
      }
      const uint8_t* ks = smem + (t & 1) * STAGE;
      const uint8_t* vs = ks + KBYTES;
      const int n0 = t * BN;
      const bool wave_active = (r0 < a.Sq) && (!a.causal || kvpos0 + n0 <= qpos0 + r0 + 32 * RB - 1);

      if (wave_active) {
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);
        f32x16 sc[RB][NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int key = kb * 32 + l32;
          const uint8_t* krow = ks + key * (D * 2);
          u32x4 kop[NDS];
#pragma unroll
          for (int s = 0; s < NDS; ++s) kop[s] = ld_lds16(krow + ((((2 * s + g) ^ (key & 15))) << 4));
          f32x16 x[RB];
#pragma unroll
          for (int r = 0; r < RB; ++r) x[r] = (f32x16){};
#pragma unroll
          for (int s = 0; s < NDS; ++s)
#pragma unroll
            for (int r = 0; r < RB; ++r) x[r] = mfma32(as_bf16x8(kop[s]), qf[r][s], x[r]);
#pragma unroll
          for (int r = 0; r < RB; ++r) sc[r][kb] = x[r];
        }
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
        if (n0 + BN > a.Sk || (a.causal && kvpos0 + n0 + BN - 1 > qpos0 + r0)) {
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            int64_t lim = (int64_t)a.Sk - n0;
            if (a.causal) lim = min<int64_t>(lim, qpos0 + row[r] - kvpos0 - n0 + 1);
            mask_block<NKB>(sc[r], (int)max<int64_t>(0, min<int64_t>(lim, BN)), g);
          }
        }
        u32x4 pk[RB][NKB][2];
#pragma unroll
        for (int r = 0; r < RB; ++r) softmax_block<NKB>(sc[r], blk[r], pk[r], SCALE_LOG2);
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(1);

#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + l32;
          const uint8_t* vrow = vs + d * VROW;
          const int sw = vt_swz<BN>(d);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              // 16-byte unit 2 * (16-key group) + g holds keys 4g..4g+3 and 8+4g..8+4g+3 of the group
              const u32x4 av = ld_lds16(vrow + (((2 * (2 * kb + t2) + g) ^ sw) << 4));
#pragma unroll
              for (int r = 0; r < RB; ++r) blk[r].o[db] = mfma32(as_bf16x8(av), as_bf16x8(pk[r][kb][t2]), blk[r].o[db]);
            }
          }
        }
        if (CPATTN_D128_PRIO) __builtin_amdgcn_s_setprio(0);
      }

      if (has_next) store_v((t + 1) & 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const Blk& bk = blk[r];
    const float l_tot = bk.l + xor32(bk.l);
    if (row[r] < a.Sq) {
      const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
      float* orow = op + (int64_t)row[r] * a.o_ss;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 v4 = {bk.o[db][4 * i4 + 0] * inv, bk.o[db][4 * i4 + 1] * inv, bk.o[db][4 * i4 + 2] * inv,
                            bk.o[db][4 * i4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4 + 4 * g) = v4;
        }
      if (g == 0) lp[(int64_t)row[r] * a.l_ss] = (l_tot > 0.f) ? (bk.m + fast_log2(l_tot)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

int partial_bf16_rows_per_block(int D) { return D == 128 ? CPATTN_D128_NW * 32 * CPATTN_D128_RB : 128; }

hipError_t launch_partial_bf16(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s) {
  const long long blocks = (long long)a.n_items * a.B * a.Hq * n_qtiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128)
    hipLaunchKernelGGL((partial_bf16_d128_kernel<CPATTN_D128_BN, CPATTN_D128_RB, CPATTN_D128_NW>), dim3((unsigned)blocks),
                       dim3(CPATTN_D128_NW * 64), 0, s, a, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL(partial_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn
