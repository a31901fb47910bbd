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
// Orientation (both kernels): each wave computes S^T = K Q^T (keys on the
// MFMA rows, its 32 queries on the columns), so a lane holds scores of ONE
// query.  Row reductions are in-lane plus one exchange with the lane 32
// away, and the probabilities come out in the B-operand layout of the second
// product O^T = V^T P^T, so P never leaves registers.
//
// Softmax runs in base 2 with the 1/sqrt(D) scale folded into one FMA.  The
// running reference is only raised when scores exceed it by more than kTau
// (2^8 in probability), so most tiles skip the O rescale; probabilities stay
// <= 2^8, well inside bf16/fp32 range, and the result is exact in real
// arithmetic because the final normalisation uses the same reference.
//
// D = 64: 4 waves = 128 query rows per workgroup, K/V staged through LDS by
// registers (V transposed on the way in).  D = 128: the kernel further down.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

constexpr float kTau = 8.0f;
constexpr float kTwoTau = 256.0f;  // 2^kTau

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
  const int L = (a.xcd_order ? xcd_logical_block(blockIdx.x, per_item * a.n_items) : (int)blockIdx.x);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;  // later (heavier under the mask) tiles first
  rem = rem % bh;
  const int b = rem / a.Hq;
  const int h = rem - b * a.Hq;
  const int kvh = h / a.G;
  const Item it = a.items[item];
  const int Sk = it.sk > 0 ? it.sk : a.Sk;  // keys of this item's K/V block

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse != nullptr ? a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh : nullptr;  // LSE optional
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.kv_chunk_len;

  const int m0 = qt * C::BM;
  const int r0 = m0 + wave * 32;  // first row of this wave
  const int row = r0 + l32;       // this lane's query row

  // keys [0, n_end) can be visible to some row of this workgroup
  int n_end = Sk;
  if (a.causal) {
    const int64_t last_row = (int64_t)min(m0 + C::BM, a.Sq) - 1;
    const int64_t lim = qpos0 + last_row - kvpos0 + 1;
    n_end = (int)max<int64_t>(0, min<int64_t>(Sk, lim));
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
        kreg[i] = (n0 + key < Sk) ? ld_global16(kp + (int64_t)(n0 + key) * a.k_ss + ch * 8) : (u32x4){};
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = n0 + 4 * vkg + kk;
        vreg[kk] = (key < Sk) ? ld_global16(vp + (int64_t)key * a.v_ss + vch * 8) : (u32x4){};
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
        const bool full = (n0 + C::BN <= Sk) && (!a.causal || kvpos0 + n0 + C::BN - 1 <= qpos0 + r0);
        if (!full) {
          // visibility is monotone in the key, so this row sees exactly the
          // tile-local keys [0, lim)
          int64_t lim64 = (int64_t)Sk - n0;
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
    const bool acc = a.accumulate != 0;
    const RowOut ro = row_out(m_run, l_tot, acc, acc ? lp[(int64_t)row * a.l_ss] : 0.f);
    float* orow = op + (int64_t)row * a.o_ss;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float* dst = orow + db * 32 + 8 * i4 + 4 * g;
        f32x4 v4 = {oacc[db][4 * i4 + 0] * ro.s_new, oacc[db][4 * i4 + 1] * ro.s_new, oacc[db][4 * i4 + 2] * ro.s_new,
                    oacc[db][4 * i4 + 3] * ro.s_new};
        if (acc) {
          const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
          v4 = (f32x4){fmaf(old[0], ro.s_old, v4[0]), fmaf(old[1], ro.s_old, v4[1]), fmaf(old[2], ro.s_old, v4[2]),
                       fmaf(old[3], ro.s_old, v4[3])};
        }
        *reinterpret_cast<f32x4*>(dst) = v4;
      }
    }
    if (g == 0 && lp != nullptr) lp[(int64_t)row * a.l_ss] = ro.lse;
  }
}


// ---------------------------------------------------------------------------
// D = 128 kernel.
//
// Workgroup = 8 waves = 256 query rows of one head, 32 rows per wave (two
// waves per SIMD).  K and V tiles of 64 keys go straight from global memory
// into LDS (global_load_lds_dwordx4), three stages deep; waves 0-3 do the
// fetching, so the queue on the CU's memory unit stalls only the older wave
// of each SIMD pair, which the pipeline below otherwise favours.  The V^T
// operand of O^T = V^T P^T is read from the row-major V tile with the gfx950
// transposing read ds_read_b64_tr_b16: within a 16-lane group it hands lane
// 4a+b element b of the 8-byte rows addressed by lanes a, a+4, a+8 and a+12,
// so when lane s addresses row key0 + s/4 at columns D0 + 4(s%4), lane i
// receives V[key0 .. key0+3][D0 + i] -- four keys of one column.
//
// LDS: the K tiles of the three stages (64 keys x 256 B each, 16-byte chunks
// XOR-swizzled by key & 15), then their V tiles (chunks XOR-swizzled by
// 4 (key & 3)); with K and V apart, every operand read reaches its data
// through the 16-bit offset of ds_read from one per-lane base.  The query
// tile (256 rows x 256 B) has a 64 KB region of its own, filled once per
// workgroup, for 160 KB in all.
//
// Each wave's work is software-pipelined so that its matrix and vector work
// overlap.  Iteration t runs two phases:
//   A: S(t+1) = K(t+1) Q^T on the matrix cores, while the vector unit
//      evaluates, packs and sums key block 1 of P(t);
//   B: O^T += V(t)^T P(t)^T on the matrix cores, while the vector unit does
//      key block 0 of P(t+1).
// Each MFMA is followed by its slice of the vector work (one probability),
// skewed over three slots: slot j takes the exponential of score j, the
// exponent argument of score j+1 and the row-sum add and bf16 pack of score
// j-1, so no instruction of a slot waits on another of the same slot.  A
// scheduling fence after every slice and empty asm "uses" of its results
// keep the compiler from regrouping them.  Waves in phase A outrank waves in
// phase B, so the wave of a SIMD pair that falls behind catches up.
//
// The probabilities of a tile are evaluated against the running reference m
// without first taking the tile's row max.  Once a tile's probabilities are
// all in, a wave whose lanes all have a reference and partial sums of at
// most 2^kTau (so every p <= 2^kTau) keeps them; any other wave recomputes
// that tile's scores (its K is still in LDS), moves the reference to the row
// max and evaluates the probabilities again.  The move rescales the row sum
// at once and O before the tile's PV.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ u32x2 ld_lds8_tr(const uint8_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(__attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Keep tile-local keys [0, lim) of this lane's row.  The lane's keys are
// kb*32 + 8*(i/4) + 4g + i%4, so comparing the constant part against lim - 4g
// keeps every index an inline immediate.
__device__ __forceinline__ void mask_block(f32x16 (&s)[2], int lim, int g) {
  const int limg = lim - 4 * g;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = (kb * 32 + 8 * (i >> 2) + (i & 3) < limg) ? s[kb][i] : kNegInf;
}

// Empty asm that claims to rewrite x: the value must be computed before this
// point (passes that sink or hoist code cannot move it past), which keeps the
// vector work of the pipelined loop in the slot it was written in.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// SEG: an item's key range is a run of chunks of seg_tiles tiles each, and
// every chunk's partial goes to its own slot (item.slot + chunk): at each
// boundary the finished partial is written and the softmax restarts exactly as
// a launch of that chunk alone would.  Without SEG an item writes one result.
template <bool SEG>
__global__ __launch_bounds__(512) void partial_bf16_d128_kernel(const PartialLaunch a, const int n_qtiles) {
  constexpr int D = 128, BN = 64, NDS = 8, BM = 256;
  constexpr int TBYTES = BN * D * 2;  // one K or V tile
  constexpr int NST = 3;              // LDS stages: tile t+2 is fetched while t and t+1 are read
  // LDS: the K tiles of all stages, then the V tiles, so every operand read's
  // offset from its per-lane base fits the 16-bit immediate of ds_read
  constexpr int VBASE = NST * TBYTES;
  constexpr int KLA = 4;              // K operand reads issued this many MFMAs ahead
  constexpr int VLA = 4;              // V operand reads issued this many MFMAs ahead
  constexpr int FW = 4;               // fetching waves
  constexpr int FL = 1024 / (FW * 64);  // 16-byte pieces of K (and of V) per fetching lane
  constexpr float SCALE_LOG2 = 0.12751743082459868f;  // log2(e) / sqrt(128)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * NST * TBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t qsm[BM * D * 2];  // the query tile, rows of 256 B

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: fetch bases and LDS targets stay scalar
  const int l32 = lane & 31;
  const int g = lane >> 5;

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

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh +
                     (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse != nullptr ? a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh : nullptr;  // LSE optional
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.kv_chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * BM;
  const int r0 = m0 + wave * 32;
  const int row = r0 + l32;

  int n_end = Sk;
  if (a.causal) n_end = max(0, min(Sk, min(m0 + BM, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  float m = kNegInf;  // running reference (log2 domain) of this lane's row
  float l = 0.f;      // this lane's share of the row sum, relative to m

  // With segments and a merge tail, the LSE of each segment's partial for this
  // wave's rows is kept in LDS: 32 rows x 64 segments per wave, in the wave's
  // own rows of the query tile area, which only this wave reads (once, in the
  // prologue).
  float* const seg_lse = reinterpret_cast<float*>(qsm) + wave * 32 * 64;

  // normalise and store this lane's row of segment `seg` (slot item.slot + seg)
  // from the running reference m_ and row share l_
  auto write_out = [&](int seg, float m_, float l_) {
    const float l_tot = pair32_sum(l_);
    if (row < a.Sq) {
      const bool acc = a.accumulate != 0;
      float* const lps = lp != nullptr ? lp + seg * a.l_slot : nullptr;
      const RowOut ro = row_out(m_, l_tot, acc, acc ? lps[(int64_t)row * a.l_ss] : 0.f);
      float* orow = op + seg * a.o_slot + (int64_t)row * a.o_ss;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float* dst = orow + db * 32 + 8 * i4 + 4 * g;
          f32x4 v4 = {o[db][4 * i4 + 0] * ro.s_new, o[db][4 * i4 + 1] * ro.s_new, o[db][4 * i4 + 2] * ro.s_new,
                      o[db][4 * i4 + 3] * ro.s_new};
          if (acc) {
            const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
            v4 = (f32x4){fmaf(old[0], ro.s_old, v4[0]), fmaf(old[1], ro.s_old, v4[1]), fmaf(old[2], ro.s_old, v4[2]),
                         fmaf(old[3], ro.s_old, v4[3])};
          }
          *reinterpret_cast<f32x4*>(dst) = v4;
        }
      if (g == 0 && lps != nullptr) lps[(int64_t)row * a.l_ss] = ro.lse;
      if constexpr (SEG)
        if (g == 0 && a.final_out != nullptr) seg_lse[seg * 32 + l32] = ro.lse;
    }
  };

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      // The query tile reaches LDS by whole rows (16 lanes per 256-byte row, 16-byte
      // chunks XOR-swizzled by the row), so each load moves four contiguous row
      // pieces instead of 32 scattered ones; rows past the block end re-read its
      // last row and are zeroed when read back.
      const uint32_t qdst = lds_addr(qsm) + wave * 64 * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int slot = i * 512 + wave * 64 + lane;
        const int rr = slot >> 4;
        const int c = (slot & 15) ^ (rr & 15);
        const int grow = min(m0 + rr, a.Sq - 1);
        gload_lds16(qp + (int64_t)grow * a.q_ss + c * 8, qdst + i * 512 * 16);
      }
    }
    // K operand of k-step s: row l32 (+32 for key block 1), chunk 2s+g swizzled by the row
    int koff[NDS];
#pragma unroll
    for (int s2 = 0; s2 < NDS; ++s2) koff[s2] = l32 * 256 + (((2 * s2 + g) ^ (l32 & 15)) << 4);
    // V^T operand, column block db: this lane addresses key 4g + ks (+16u + 8 half) at
    // columns 32 db + 16 c16 + 4 (s & 3), chunk swizzled by 4 ks
    int voff[4];
    {
      const int s16 = lane & 15, ks = s16 >> 2, c16 = l32 >> 4, c8 = (s16 & 3) >> 1, bo = (s16 & 1) * 8;
#pragma unroll
      for (int db = 0; db < 4; ++db) voff[db] = VBASE + (4 * g + ks) * 256 + ((4 * (db ^ ks) + 2 * c16 + c8) << 4) + bo;
    }
    // Fetch: piece i of fetching wave fw, lane l is tile slot i*FW*64 + fw*64 + l,
    // which holds key slot>>4 at physical chunk slot&15 (logical chunk for K:
    // ^ (key & 15), for V: ^ 4 (key & 3)).  Each lane keeps its pieces' byte
    // offsets from the tile start; the tile starts are scalar and advance one
    // tile per fetch.
    const bool fetcher = wave < FW;
    int fkey[FL];
    uint32_t kof[FL], vof[FL];
#pragma unroll
    for (int i = 0; i < FL; ++i) {
      const int slot = i * FW * 64 + (wave % FW) * 64 + lane;
      fkey[i] = slot >> 4;
      kof[i] = (uint32_t)(2 * (fkey[i] * a.k_ss + (((slot & 15) ^ (fkey[i] & 15)) << 3)));
      vof[i] = (uint32_t)(2 * (fkey[i] * a.v_ss + (((slot & 15) ^ (4 * (fkey[i] & 3))) << 3)));
    }
    const uint8_t* kt = reinterpret_cast<const uint8_t*>(kp);
    const uint8_t* vt = reinterpret_cast<const uint8_t*>(vp);
    const int64_t kstep = 2 * BN * a.k_ss, vstep = 2 * BN * a.v_ss;
    const uint32_t lbase = lds_addr(smem) + (wave % FW) * 64 * 16;
    int n_fetched = 0;
    auto fetch = [&](int stage) {
      const uint32_t dst = lbase + stage * TBYTES;
      if (fetcher) {
        if ((n_fetched + 1) * BN <= Sk) {
#pragma unroll
          for (int i = 0; i < FL; ++i) {
            gload_lds16(kt, kof[i], dst + i * FW * 64 * 16);
            gload_lds16(vt, vof[i], dst + i * FW * 64 * 16 + VBASE);
          }
        } else {
          // rows past the block end re-read the last row: their scores are
          // masked to -inf, so their p is exactly 0
#pragma unroll
          for (int i = 0; i < FL; ++i) {
            const int over = max(0, n_fetched * BN + fkey[i] - (Sk - 1));
            gload_lds16(kt, kof[i] - (uint32_t)(2 * over * a.k_ss), dst + i * FW * 64 * 16);
            gload_lds16(vt, vof[i] - (uint32_t)(2 * over * a.v_ss), dst + i * FW * 64 * 16 + VBASE);
          }
        }
        kt += kstep;
        vt += vstep;
      }
      ++n_fetched;
    };

    // The masked tiles (diagonal and block end), the slow path of the lazy
    // reference and the rescale after it are rare: marked unlikely, their code
    // is laid out after the loop, so the six unrolled iterations' common path
    // stays compact (~450 instructions each instead of ~830; +0.5-1%).
    auto mask_tile = [&](f32x16 (&sc)[2], int t) {
      const int n0 = t * BN;
      if (__builtin_expect(n0 + BN > Sk || (a.causal && dpos + n0 + BN - 1 > r0), 0)) {
        int lim = Sk - n0;
        if (a.causal) lim = min(lim, row - dpos - n0 + 1);
        mask_block(sc, max(0, min(lim, BN)), g);
      }
    };

    // Two sets of tile state, used alternately by even and odd iterations so
    // that no iteration copies registers into the next: scores of the newest
    // tile, and packed P of the tile being accumulated (word w: p[2w], p[2w+1];
    // words 0..7 from key block 0, 8..15 from key block 1).
    f32x16 snA[2], snB[2];
    uint32_t pwA[16], pwB[16];
    float lt = 0.f;     // this lane's partial sum of that tile
    // A finished segment whose stores wait for the next iteration's fetch to be
    // issued first, so the per-tile wait for that fetch does not also wait for
    // them: its reference, row share and index (O stays in o until then).
    bool pend = false;
    float m_pend = 0.f, l_pend = 0.f;
    int seg_pend = 0;
    int seg_left = a.seg_tiles, seg_idx = 0;  // tiles left in the current segment, its index
    bool need = false;  // O must be rescaled by alpha before the next PV
    float alpha = 1.f;
    float mref = 0.f;
    auto prob = [&](float x) -> float {
      const float pv = fast_exp2(fmaf(x, SCALE_LOG2, -mref));
      lt += pv;
      return pv;
    };
    // QK MFMA j of a tile: key block j & 1, k-step j >> 1 (consecutive MFMAs
    // accumulate into different blocks)
    auto scores = [&](const uint8_t* kbase, f32x16 (&sc)[2]) {
      sc[0] = (f32x16){};
      sc[1] = (f32x16){};
#pragma unroll
      for (int j = 0; j < 16; ++j)
        sc[j & 1] = mfma32(as_bf16x8(ld_lds16(kbase + koff[j >> 1] + (j & 1) * 8192)), qf[j >> 1], sc[j & 1]);
    };
    // move the reference to the row max of sc (never down)
    auto move_to_max = [&](const f32x16 (&sc)[2]) {
      float mx = sc[0][0];
#pragma unroll
      for (int f = 1; f < 32; ++f) mx = fmaxf(mx, sc[f >> 4][f & 15]);
      mx = pair32_max(mx);
      const float m_new = fmaxf(m, mx * SCALE_LOG2);
      alpha = (m_new == m) ? 1.f : fast_exp2(m - m_new);
      l *= alpha;
      m = m_new;
      mref = (m == kNegInf) ? 0.f : m;
      need = true;
    };
    // the slow path for tile t (its K and mask), recomputing all of pw and lt
    auto redo_tile = [&](const uint8_t* kbase, int t, uint32_t (&pw)[16]) {
      f32x16 sc[2];
      scores(kbase, sc);
      mask_tile(sc, t);
      move_to_max(sc);
      lt = 0.f;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const float p0 = prob(sc[w >> 3][2 * (w & 7)]);
        const float p1 = prob(sc[w >> 3][2 * (w & 7) + 1]);
        pw[w] = pack_bf16(p0, p1);
      }
    };

    // prologue: tiles 0 and 1 fetched and landed; S(0), its reference, and key block 0 of P(0)
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
      if (i < n_tiles) fetch(i);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (r0 >= a.Sq) {
      // No row of this wave is a query (a block shorter than the workgroup's
      // 256 rows): keep the others' fetch and barrier schedule, skip the math,
      // so the SIMD's matrix core serves the other wave alone.
      for (int t = 0; t < n_tiles; ++t) {
        if (t + NST - 1 < n_tiles) fetch((t + NST - 1) % NST);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    } else {
      {
        // Q fragments, B operand of S^T = K Q^T: column = this lane's row,
        // k-slots = d in [16 s + 8 g, 16 s + 8 g + 8)
        const int rr = wave * 32 + l32;
        const bool ok = row < a.Sq;
#pragma unroll
        for (int s2 = 0; s2 < NDS; ++s2)
          qf[s2] = ok ? as_bf16x8(ld_lds16(qsm + rr * 256 + (((2 * s2 + g) ^ (rr & 15)) << 4))) : (bf16x8){};
      }
      {
        scores(smem, snA);
        mask_tile(snA, 0);
        move_to_max(snA);
        need = false;  // O is still zero
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float p0 = prob(snA[0][2 * w]);
          const float p1 = prob(snA[0][2 * w + 1]);
          pwA[w] = pack_bf16(p0, p1);
        }
      }

      // Iteration t.  The last one also computes scores for the tile after the
      // last: every one of them is masked (that tile starts at or past the
      // block's last visible key), so its probabilities are 0; its K operands
      // come from a stale stage that no fetch is writing.
      auto iteration = [&](int t, auto st_tag, f32x16 (&sn)[2], f32x16 (&x)[2], uint32_t (&pw)[16],
                           uint32_t (&pn)[16]) {
        constexpr int ST = decltype(st_tag)::value;
        constexpr int SN = (ST + 1) % NST;
        constexpr int SL = (ST + NST - 1) % NST;
        const uint8_t* cur = smem + ST * TBYTES;  // K of tile t at cur, V at cur + VBASE (voff)
        const uint8_t* nxt = smem + SN * TBYTES;
        // tile t+2 goes into the stage tile t-1 used
        const bool do_fetch = t + NST - 1 < n_tiles;
        if (do_fetch) fetch(SL);
        if constexpr (SEG) {
          if (pend) {
            write_out(seg_pend, m_pend, l_pend);
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
            pend = false;
          }
        }

        u32x4 kop[16];
        u32x2 vlo[16], vhi[16];
        auto read_v = [&](int jj) {  // operands of PV MFMA jj: u = jj >> 2, db = jj & 3
          const int u = jj >> 2, db = jj & 3;
          vlo[jj] = ld_lds8_tr(cur + voff[db] + (16 * u) * 256);
          vhi[jj] = ld_lds8_tr(cur + voff[db] + (16 * u + 8) * 256);
        };
        // ---- phase A: S(t+1) = K(t+1) Q^T; key block 1 of P(t) ----
        __builtin_amdgcn_s_setprio(1);
        const f32x16& s1 = sn[1];
        x[0] = (f32x16){};
        x[1] = (f32x16){};
#pragma unroll
        for (int j = 0; j < KLA; ++j) kop[j] = ld_lds16(nxt + koff[j >> 1] + (j & 1) * 8192);
        float pe = 0.f, pp = 0.f;
        float xa = fmaf(s1[0], SCALE_LOG2, -mref);
        pin(xa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j + KLA < 16) kop[j + KLA] = ld_lds16(nxt + koff[(j + KLA) >> 1] + ((j + KLA) & 1) * 8192);
          if (j >= 16 - VLA) read_v(j - (16 - VLA));
          x[j & 1] = mfma32(as_bf16x8(kop[j]), qf[j >> 1], x[j & 1]);
          // slot j: exponent of score j, argument of score j+1, sum and pack of score j-1
          const float pv = fast_exp2(xa);
          if (j < 15) xa = fmaf(s1[j + 1], SCALE_LOG2, -mref);
          if (j > 0) {
            lt += pp;
            if ((j - 1) & 1) {
              pw[8 + ((j - 1) >> 1)] = pack_bf16(pe, pp);
              pin(pw[8 + ((j - 1) >> 1)]);
            } else {
              pe = pp;
              pin(pe);
            }
          }
          pp = pv;
          pin(pp);
          pin(xa);
          pin(lt);
          __builtin_amdgcn_sched_barrier(0);
        }
        lt += pp;
        pw[15] = pack_bf16(pe, pp);
        mask_tile(x, t + 1);
        // tile t is complete: keep it, or take the slow path
        if (__builtin_expect(__any(!(lt <= kTwoTau) || m == kNegInf), 0)) redo_tile(cur, t, pw);
        l += lt;
        lt = 0.f;
        __builtin_amdgcn_sched_barrier(0);

        // ---- phase B: O^T += V(t)^T P(t)^T; key block 0 of P(t+1) ----
        __builtin_amdgcn_s_setprio(0);
        if (__builtin_expect(need, 0)) {
#pragma unroll
          for (int db = 0; db < 4; ++db) o[db] *= alpha;
          need = false;
        }
        xa = fmaf(x[0][0], SCALE_LOG2, -mref);
        pin(xa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (jj + VLA < 16) read_v(jj + VLA);
          const int u = jj >> 2, db = jj & 3;
          const u32x4 av = {vlo[jj][0], vlo[jj][1], vhi[jj][0], vhi[jj][1]};
          const u32x4 bp = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
          o[db] = mfma32(as_bf16x8(av), as_bf16x8(bp), o[db]);
          const float pv = fast_exp2(xa);
          if (jj < 15) xa = fmaf(x[0][jj + 1], SCALE_LOG2, -mref);
          if (jj > 0) {
            lt += pp;
            if ((jj - 1) & 1) {
              pn[(jj - 1) >> 1] = pack_bf16(pe, pp);
              pin(pn[(jj - 1) >> 1]);
            } else {
              pe = pp;
              pin(pe);
            }
          }
          pp = pv;
          pin(pp);
          pin(xa);
          pin(lt);
          __builtin_amdgcn_sched_barrier(0);
        }
        lt += pp;
        pn[7] = pack_bf16(pe, pp);
        if constexpr (SEG) {
          if (--seg_left == 0) {
            seg_left = a.seg_tiles;
            seg_pend = seg_idx++;
          }
          if (seg_left == a.seg_tiles && t + 1 < n_tiles) {
            // A chunk boundary: this pair's partial is complete (written at the
            // start of the next iteration, O zeroed there before its first PV),
            // and the next pair starts exactly as a launch of its own would:
            // zero state, the reference at the row max of its first tile (whose
            // scores x already holds, masked), then key block 0 of that tile's P.
            pend = true;
            m_pend = m;
            l_pend = l;
            m = kNegInf;
            l = 0.f;
            lt = 0.f;
            move_to_max(x);
            need = false;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const float p0 = prob(x[0][2 * w]);
              const float p1 = prob(x[0][2 * w + 1]);
              pn[w] = pack_bf16(p0, p1);
            }
          }
        }
        // tile t+2 (fetched above) must have landed before any wave reads it
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      };
      // six iterations per trip: three LDS stages times two register sets
      static_assert(NST == 3, "the loop below is unrolled over three stages");
      for (int t = 0; t < n_tiles; t += 2 * NST) {
        iteration(t, std::integral_constant<int, 0>{}, snA, snB, pwA, pwB);
        if (t + 1 < n_tiles) iteration(t + 1, std::integral_constant<int, 1>{}, snB, snA, pwB, pwA);
        if (t + 2 < n_tiles) iteration(t + 2, std::integral_constant<int, 2>{}, snA, snB, pwA, pwB);
        if (t + 3 < n_tiles) iteration(t + 3, std::integral_constant<int, 0>{}, snB, snA, pwB, pwA);
        if (t + 4 < n_tiles) iteration(t + 4, std::integral_constant<int, 1>{}, snA, snB, pwA, pwB);
        if (t + 5 < n_tiles) iteration(t + 5, std::integral_constant<int, 2>{}, snB, snA, pwB, pwA);
      }
    }
  }

  const int last_seg = SEG && n_tiles > 0 ? (n_tiles - 1) / a.seg_tiles : 0;
  write_out(last_seg, m, l);
  if constexpr (SEG) {
    // Segments past this query tile's last visible key hold pairs its rows see
    // nothing of (queries shorter than K/V put the last chunk's first keys after
    // the early rows): each gets the empty partial, O = 0 and LSE = -inf.
    const int n_seg = (Sk + a.seg_tiles * BN - 1) / (a.seg_tiles * BN);
    if (last_seg + 1 < n_seg) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
      m = kNegInf;
      l = 0.f;
      for (int seg = last_seg + 1; seg < n_seg; ++seg) write_out(seg, m, l);
    }
    if (a.final_out != nullptr && row < a.Sq) {
      // Merge tail: this lane's pieces of the n_seg partials it has just
      // written, in the ring order's arrival order, with the arithmetic of the
      // ring merge kernel (the same pieces in the same order: bit-identical).
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      const int i = it.q_chunk;
      const bool pq = a.pass_q != 0;
      float M = kNegInf;
      for (int c = 0; c < n_seg; ++c) M = fmaxf(M, seg_lse[c * 32 + l32]);
      f32x4 acc[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] = (f32x4){};
      float den = 0.f;
      const float* const orow = op + (int64_t)row * a.o_ss + 4 * g;
      auto load_seg = [&](int j, f32x4 (&v)[16]) {
        const float* src = orow + j * a.o_slot;
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = *reinterpret_cast<const f32x4*>(src + (k >> 2) * 32 + 8 * (k & 3));
      };
      if (M != kNegInf) {
        f32x4 cur[16], nxt[16];
        int j = arrival_kv(pq, i, n_seg, 0);
        load_seg(j, cur);
        for (int c = 0; c < n_seg; ++c) {
          const int jn = c + 1 < n_seg ? arrival_kv(pq, i, n_seg, c + 1) : j;
          if (c + 1 < n_seg) load_seg(jn, nxt);
          const float w = merge_weight(seg_lse[j * 32 + l32], M);
          den += w;
#pragma unroll
          for (int k = 0; k < 16; ++k) merge_acc(acc[k], w, cur[k]);
#pragma unroll
          for (int k = 0; k < 16; ++k) cur[k] = nxt[k];
          j = jn;
        }
      }
      const float inv = merge_inv(den);
      const int64_t grow = (int64_t)i * a.chunk_len + row;
      const int64_t fo = b * a.f_sb + grow * a.f_ss + h * a.f_sh + 4 * g;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        store_row(a.final_out, a.final_bf16 != 0, fo + (k >> 2) * 32 + 8 * (k & 3), acc[k] * inv);
      if (g == 0 && a.final_lse != nullptr) a.final_lse[b * a.fl_sb + grow * a.fl_ss + h * a.fl_sh] = merged_lse(M, den);
    }
  }
}

}  // namespace

int partial_bf16_rows_per_block(int D) { return D == 128 ? 256 : 128; }

hipError_t launch_partial_bf16(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s) {
  const long long blocks = (long long)a.n_items * a.B * a.Hq * n_qtiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128 && a.seg_tiles > 0)
    hipLaunchKernelGGL(partial_bf16_d128_kernel<true>, dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else if (D == 128)
    hipLaunchKernelGGL(partial_bf16_d128_kernel<false>, dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL(partial_bf16_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, a, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn

