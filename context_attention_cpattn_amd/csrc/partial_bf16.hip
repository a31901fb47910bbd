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
// Orientation: each wave computes S^T = K Q^T (keys on the
// MFMA rows, its 32 queries on the columns), so a lane holds scores of ONE
// query.  Row reductions are in-lane plus one exchange with the lane 32
// away, and the probabilities come out in the B-operand layout of the second
// product O^T = V^T P^T, so P never leaves registers.
//
// Softmax runs in base 2 with the 1/sqrt(D) scale folded into one FMA.  The
// running reference is only raised when scores exceed it by more than 8
// (2^8 in probability), so most tiles skip the O rescale; probabilities stay
// <= 2^8, well inside bf16/fp32 range, and the result is exact in real
// arithmetic because the final normalisation uses the same reference.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

constexpr float kTwoTau = 256.0f;  // 2^8: the reference moves when a probability would exceed it

// ---------------------------------------------------------------------------
// The kernel, for head dimensions D = 128 and D = 64.
//
// Workgroup = 8 waves = 256 query rows of one head (or of 2, 4 or 8 heads of
// one K/V head when query blocks are short), 32 rows per wave (two waves per
// SIMD).  K and V tiles of 64 keys go straight from global memory
// into LDS (global_load_lds_dwordx4), three stages deep; waves 0-3 do the
// fetching, so the queue on the CU's memory unit stalls only the older wave
// of each SIMD pair, which the pipeline below otherwise favours.  The V^T
// operand of O^T = V^T P^T is read from the row-major V tile with the gfx950
// transposing read ds_read_b64_tr_b16: within a 16-lane group it hands lane
// 4a+b element b of the 8-byte rows addressed by lanes a, a+4, a+8 and a+12,
// so when lane s addresses row key0 + s/4 at columns D0 + 4(s%4), lane i
// receives V[key0 .. key0+3][D0 + i] -- four keys of one column.
//
// LDS: the K tiles of the three stages (64 keys x 2D bytes each, 16-byte
// chunks XOR-swizzled by key & 15 for D = 128, by (key >> 1) & 7 for the
// 128-byte rows of D = 64), then their V tiles (chunks XOR-swizzled by
// 4 (key & 3), or 2 (key & 3)); with K and V apart, every operand read
// reaches its data through the 16-bit offset of ds_read from one per-lane
// base.  The query tile has a region of its own (64 KB), filled once per
// workgroup: 160 KB in all for D = 128, 112 KB for D = 64.
//
// Each wave's work is software-pipelined so that its matrix and vector work
// overlap.  Iteration t runs two phases:
//   A: S(t+1) = K(t+1) Q^T on the matrix cores, while the vector unit
//      evaluates, packs and sums key block 1 of P(t);
//   B: O^T += V(t)^T P(t)^T on the matrix cores, while the vector unit does
//      key block 0 of P(t+1).
// Each MFMA is followed by its slice of the vector work (one probability;
// two with D = 64, whose phases have 8 MFMAs for the 16 probabilities),
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
// most 2^8 (so every p <= 2^8) keeps them; any other wave recomputes
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
template <int D, bool SEG>
__global__ __launch_bounds__(512) void partial_bf16_fast_kernel(const PartialLaunch a, const int n_qtiles) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  constexpr int BN = 64, BM = 256;
  constexpr int ROWB = D * 2;          // bytes of a Q, K or V row
  constexpr int CH = D / 8;            // 16-byte chunks of a row
  constexpr int NDS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;          // 32-column blocks of O^T
  constexpr int NQK = 2 * NDS;         // QK MFMAs of a tile (two key blocks)
  constexpr int NPV = 4 * NDB;         // PV MFMAs of a tile (four 16-key groups)
  // Each phase evaluates 16 probabilities per lane; with D = 64 a phase has 8
  // MFMAs, so two probability slots follow each of them.
  constexpr int RA = 16 / NQK, RB = 16 / NPV;
  static_assert(16 % NQK == 0 && 16 % NPV == 0, "probability slots per MFMA");
  constexpr int TBYTES = BN * ROWB;   // one K or V tile
  constexpr int KB1 = 32 * ROWB;      // key block 1 of a K tile
  constexpr int NST = 3;              // LDS stages: tile t+2 is fetched while t and t+1 are read
  // LDS: the K tiles of all stages, then the V tiles, so every operand read's
  // offset from its per-lane base fits the 16-bit immediate of ds_read
  constexpr int VBASE = NST * TBYTES;
  constexpr int KLA = 4;              // K operand reads issued this many MFMAs ahead
  constexpr int VLA = 4;              // V operand reads issued this many MFMAs ahead
  constexpr int FW = 4;               // fetching waves
  constexpr int FL = BN * CH / (FW * 64);  // 16-byte pieces of K (and of V) per fetching lane
  constexpr float SCALE_LOG2 = D == 64 ? 0.18033688011112042f : 0.12751743082459868f;  // log2(e) / sqrt(D)
  // the query tile (rows of ROWB bytes); at least 64 KB, for the LSE copies of the merge tail
  constexpr int QSM = BM * ROWB > 32 * 64 * 4 * 8 ? BM * ROWB : 32 * 64 * 4 * 8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * NST * TBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t qsm[QSM];
  // Row swizzles of the 16-byte chunks in LDS: K (and Q) rows by the row (D = 128) or its
  // half (D = 64, 128-byte rows), V rows by the row mod 4, so the operand reads of a
  // 16-lane group spread over the banks.
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vswz = [](int r) { return D == 128 ? 4 * (r & 3) : 2 * (r & 3); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: fetch bases and LDS targets stay scalar
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // Head packing: the workgroup's 256 query rows are 2^hpl heads of the same K/V
  // head, RPH = 256 >> hpl rows of each, so that query blocks of 128 rows or fewer
  // still give every wave rows.  Wave w takes head h0 + w / WPH and rows
  // (w % WPH) * 32 of that head's RPH.
  const int hpl = a.head_pack_log2;
  const int WPH = 8 >> hpl;   // waves per head
  const int RPH = BM >> hpl;  // query rows per head
  const int hb_n = a.Hq >> hpl;
  const int bh = a.B * hb_n;
  const int per_item = bh * n_qtiles;
  const int L = (a.xcd_order ? xcd_logical_block(blockIdx.x, per_item * a.n_items) : (int)blockIdx.x);
  const int item = L / per_item;
  int rem = L - item * per_item;
  const int qt = n_qtiles - 1 - rem / bh;
  rem = rem % bh;
  const int b = rem / hb_n;
  const int h0 = (rem - b * hb_n) << hpl;
  const int h = h0 + wave / WPH;  // this wave's head
  const int kvh = h0 / a.G;
  const Item it = a.items[item];
  const int Sk = it.sk > 0 ? it.sk : a.Sk;  // keys of this item's K/V block

  // the Q block without its head offset (the query tile's rows span 2^hpl heads)
  const __bf16* qb = static_cast<const __bf16*>(a.q) + b * a.q_sb + (int64_t)it.q_chunk * a.chunk_len * a.q_ss;
  const __bf16* kp = static_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.k_ss;
  const __bf16* vp = static_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh +
                     (int64_t)it.kv_chunk * a.kv_chunk_len * a.v_ss;
  float* op = a.o + it.slot * a.o_slot + b * a.o_sb + h * a.o_sh;
  float* lp = a.lse != nullptr ? a.lse + it.slot * a.l_slot + b * a.l_sb + h * a.l_sh : nullptr;  // LSE optional
  const int64_t qpos0 = a.q_pos0 + (int64_t)it.q_chunk * a.chunk_len;
  const int64_t kvpos0 = a.kv_pos0 + (int64_t)it.kv_chunk * a.kv_chunk_len;

  const int dpos = (int)max<int64_t>(-(1 << 30), min<int64_t>(1 << 30, kvpos0 - qpos0));
  const int m0 = qt * RPH;
  const int r0 = m0 + (wave % WPH) * 32;
  const int row = r0 + l32;

  int n_end = Sk;
  if (a.causal) n_end = max(0, min(Sk, min(m0 + RPH, a.Sq) - dpos));
  const int n_tiles = (n_end + BN - 1) / BN;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = (f32x16){};
  float m = kNegInf;  // running reference (log2 domain) of this lane's row
  float l = 0.f;      // this lane's share of the row sum, relative to m

  // With segments and a merge tail, the LSE of each segment's partial for this
  // wave's rows is kept in LDS: 32 rows x 64 segments per wave in the query tile
  // area.  Every wave reads its query fragments in the prologue, before the
  // first tile's barrier, and the first LSE copy is written after it.
  float* const seg_lse = reinterpret_cast<float*>(qsm) + wave * 32 * 64;

  // normalise and store this lane's row of segment `seg` (slot item.slot + seg)
  // from the running reference m_ and row share l_; with `keep` the row is not
  // stored but left in o, its factor in keep_s, for the merge tail to take
  float keep_s = 0.f;
  auto write_out = [&](int seg, float m_, float l_, bool keep) {
    const float l_tot = pair32_sum(l_);
    if (row < a.Sq) {
      const bool acc = !SEG && a.accumulate != 0;  // chunk walks never accumulate
      float* const lps = lp != nullptr ? lp + seg * a.l_slot : nullptr;
      float* const orow = op + seg * a.o_slot + (int64_t)row * a.o_ss + 4 * g;
      constexpr int NP = 4 * NDB;  // 16-byte pieces of this lane's half of the row
      // An accumulating write reads the running row first, all of it before
      // the first wait: one memory round trip instead of one per piece.
      f32x4 old[NP];
      float lse_old = 0.f;
      if (acc) {
        lse_old = lps[(int64_t)row * a.l_ss];
#pragma unroll
        for (int k = 0; k < NP; ++k) old[k] = *reinterpret_cast<const f32x4*>(orow + (k >> 2) * 32 + 8 * (k & 3));
      }
      const RowOut ro = row_out(m_, l_tot, acc, lse_old);
      keep_s = ro.s_new;
      if (!keep) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int db = k >> 2, i4 = k & 3;
          f32x4 v4 = {o[db][4 * i4 + 0] * ro.s_new, o[db][4 * i4 + 1] * ro.s_new, o[db][4 * i4 + 2] * ro.s_new,
                      o[db][4 * i4 + 3] * ro.s_new};
          if (acc)
            v4 = (f32x4){fmaf(old[k][0], ro.s_old, v4[0]), fmaf(old[k][1], ro.s_old, v4[1]),
                         fmaf(old[k][2], ro.s_old, v4[2]), fmaf(old[k][3], ro.s_old, v4[3])};
          *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i4) = v4;
        }
        if (g == 0 && lps != nullptr) lps[(int64_t)row * a.l_ss] = ro.lse;
      }
      if constexpr (SEG)
        if (g == 0 && a.final_out != nullptr) seg_lse[seg * 32 + l32] = ro.lse;
    }
  };

  if (n_tiles > 0) {
    bf16x8 qf[NDS];
    {
      // The query tile reaches LDS by whole rows (CH lanes per row, 16-byte chunks
      // XOR-swizzled by the row), so each load moves contiguous row pieces
      // instead of 32 scattered ones; rows past the block end re-read its last
      // row and are zeroed when read back.  Tile row rr is row m0 + rr % RPH of
      // head h0 + rr / RPH.
      const uint32_t qdst = lds_addr(qsm) + wave * 64 * 16;
#pragma unroll
      for (int i = 0; i < BM * CH / 512; ++i) {
        const int slot = i * 512 + wave * 64 + lane;
        const int rr = slot / CH;
        const int c = (slot % CH) ^ kswz(rr);
        const int grow = min(m0 + (rr & (RPH - 1)), a.Sq - 1);
        gload_lds16(qb + (h0 + (rr >> (8 - hpl))) * a.q_sh + (int64_t)grow * a.q_ss + c * 8, qdst + i * 512 * 16);
      }
    }
    // K operand of k-step s: row l32 (+32 for key block 1), chunk 2s+g swizzled by the row
    int koff[NDS];
#pragma unroll
    for (int s2 = 0; s2 < NDS; ++s2) koff[s2] = l32 * ROWB + (((2 * s2 + g) ^ kswz(l32)) << 4);
    // V^T operand, column block db: this lane addresses key 4g + ks (+16u + 8 half) at
    // columns 32 db + 16 c16 + 4 (s & 3), its chunk swizzled by the key mod 4
    int voff[NDB];
    {
      const int s16 = lane & 15, ks = s16 >> 2, c16 = l32 >> 4, c8 = (s16 & 3) >> 1, bo = (s16 & 1) * 8;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        voff[db] = VBASE + (4 * g + ks) * ROWB + (((4 * db + 2 * c16 + c8) ^ vswz(ks)) << 4) + bo;
    }
    // Fetch: piece i of fetching wave fw, lane l is tile slot i*FW*64 + fw*64 + l,
    // which holds key slot/CH at physical chunk slot%CH (logical chunk: ^ kswz(key)
    // for K, ^ vswz(key) for V).  Each lane keeps its pieces' byte offsets from
    // the tile start; the tile starts are scalar and advance one tile per fetch.
    const bool fetcher = wave < FW;
    int fkey[FL];
    uint32_t kof[FL], vof[FL];
#pragma unroll
    for (int i = 0; i < FL; ++i) {
      const int slot = i * FW * 64 + (wave % FW) * 64 + lane;
      fkey[i] = slot / CH;
      kof[i] = (uint32_t)(2 * (fkey[i] * a.k_ss + (((slot % CH) ^ kswz(fkey[i])) << 3)));
      vof[i] = (uint32_t)(2 * (fkey[i] * a.v_ss + (((slot % CH) ^ vswz(fkey[i])) << 3)));
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
      for (int j = 0; j < NQK; ++j)
        sc[j & 1] = mfma32(as_bf16x8(ld_lds16(kbase + koff[j >> 1] + (j & 1) * KB1)), qf[j >> 1], sc[j & 1]);
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
          qf[s2] = ok ? as_bf16x8(ld_lds16(qsm + rr * ROWB + (((2 * s2 + g) ^ kswz(rr)) << 4))) : (bf16x8){};
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
            write_out(seg_pend, m_pend, l_pend, false);
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] = (f32x16){};
            pend = false;
          }
        }

        u32x4 kop[NQK];
        u32x2 vlo[NPV], vhi[NPV];
        auto read_v = [&](int jj) {  // operands of PV MFMA jj: key group u = jj / NDB, column block jj % NDB
          const int u = jj / NDB, db = jj % NDB;
          vlo[jj] = ld_lds8_tr(cur + voff[db] + (16 * u) * ROWB);
          vhi[jj] = ld_lds8_tr(cur + voff[db] + (16 * u + 8) * ROWB);
        };
        // ---- phase A: S(t+1) = K(t+1) Q^T; key block 1 of P(t) ----
        __builtin_amdgcn_s_setprio(1);
        const f32x16& s1 = sn[1];
        x[0] = (f32x16){};
        x[1] = (f32x16){};
#pragma unroll
        for (int j = 0; j < KLA; ++j) kop[j] = ld_lds16(nxt + koff[j >> 1] + (j & 1) * KB1);
        float pe = 0.f, pp = 0.f;
        float xa = fmaf(s1[0], SCALE_LOG2, -mref);
        pin(xa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j % RA == 0) {
            const int jm = j / RA;  // QK MFMA jm: key block jm & 1, k-step jm >> 1
            if (jm + KLA < NQK) kop[jm + KLA] = ld_lds16(nxt + koff[(jm + KLA) >> 1] + ((jm + KLA) & 1) * KB1);
            if (jm >= NQK - VLA) read_v(jm - (NQK - VLA));
            x[jm & 1] = mfma32(as_bf16x8(kop[jm]), qf[jm >> 1], x[jm & 1]);
          }
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
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
          need = false;
        }
        xa = fmaf(x[0][0], SCALE_LOG2, -mref);
        pin(xa);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (jj % RB == 0) {
            const int jm = jj / RB;  // PV MFMA jm: key group u, column block db
            if (jm + VLA < NPV) read_v(jm + VLA);
            const int u = jm / NDB, db = jm % NDB;
            const u32x4 av = {vlo[jm][0], vlo[jm][1], vhi[jm][0], vhi[jm][1]};
            const u32x4 bp = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
            o[db] = mfma32(as_bf16x8(av), as_bf16x8(bp), o[db]);
          }
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
  // Both ring orders merge the owner's own chunk first.  When that chunk is also
  // the last one this walk computed (every query tile of a causal prefill at
  // equal lengths), its partial is still in o: the merge tail takes it from
  // there instead of storing it and reading it back.
  const bool keep_first = SEG && a.final_out != nullptr && last_seg == it.q_chunk;
  write_out(last_seg, m, l, keep_first);
  if constexpr (SEG) {
    // Segments past this query tile's last visible key hold pairs its rows see
    // nothing of (queries shorter than K/V put the last chunk's first keys after
    // the early rows): each gets the empty partial, O = 0 and LSE = -inf.
    const int n_seg = (Sk + a.seg_tiles * BN - 1) / (a.seg_tiles * BN);
    if (last_seg + 1 < n_seg) {
      if (keep_first) {
        // o still holds the kept partial: store the empty ones directly (the
        // bits write_out stores for a zeroed o and no key: +0 and -inf)
        if (row < a.Sq) {
          constexpr int NP = 4 * NDB;
          for (int seg = last_seg + 1; seg < n_seg; ++seg) {
            float* const orow = op + seg * a.o_slot + (int64_t)row * a.o_ss + 4 * g;
#pragma unroll
            for (int k = 0; k < NP; ++k) *reinterpret_cast<f32x4*>(orow + (k >> 2) * 32 + 8 * (k & 3)) = (f32x4){};
            if (g == 0 && lp != nullptr) lp[seg * a.l_slot + (int64_t)row * a.l_ss] = kNegInf;
            if (g == 0) seg_lse[seg * 32 + l32] = kNegInf;
          }
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = (f32x16){};
        m = kNegInf;
        l = 0.f;
        for (int seg = last_seg + 1; seg < n_seg; ++seg) write_out(seg, m, l, false);
      }
    }
    if (a.final_out != nullptr && row < a.Sq) {
      // Merge tail: this lane's pieces of the n_seg partials it has just
      // written (the first in arrival order, the own chunk's, taken from o when
      // kept), in the ring order's arrival order, with the arithmetic of the
      // ring merge kernel (the same pieces in the same order: bit-identical).
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      const int i = it.q_chunk;
      const bool pq = a.pass_q != 0;
      float M = kNegInf;
      for (int c = 0; c < n_seg; ++c) M = fmaxf(M, seg_lse[c * 32 + l32]);
      constexpr int NP = 4 * NDB;  // 16-byte pieces of this lane's row
      f32x4 acc[NP];
#pragma unroll
      for (int k = 0; k < NP; ++k) acc[k] = (f32x4){};
      float den = 0.f;
      const float* const orow = op + (int64_t)row * a.o_ss + 4 * g;
      auto load_seg = [&](int j, f32x4 (&v)[NP]) {
        const float* src = orow + j * a.o_slot;
#pragma unroll
        for (int k = 0; k < NP; ++k) v[k] = *reinterpret_cast<const f32x4*>(src + (k >> 2) * 32 + 8 * (k & 3));
      };
      if (M != kNegInf) {
        f32x4 cur[NP], nxt[NP];
        int j = arrival_kv(pq, i, n_seg, 0);
        if (keep_first) {
          // the partial write_out would have stored: the same products of o and s_new
#pragma unroll
          for (int k = 0; k < NP; ++k)
            cur[k] = (f32x4){o[k >> 2][4 * (k & 3) + 0] * keep_s, o[k >> 2][4 * (k & 3) + 1] * keep_s,
                             o[k >> 2][4 * (k & 3) + 2] * keep_s, o[k >> 2][4 * (k & 3) + 3] * keep_s};
        } else {
          load_seg(j, cur);
        }
        for (int c = 0; c < n_seg; ++c) {
          const int jn = c + 1 < n_seg ? arrival_kv(pq, i, n_seg, c + 1) : j;
          if (c + 1 < n_seg) load_seg(jn, nxt);
          const float w = merge_weight(seg_lse[j * 32 + l32], M);
          den += w;
#pragma unroll
          for (int k = 0; k < NP; ++k) merge_acc(acc[k], w, cur[k]);
#pragma unroll
          for (int k = 0; k < NP; ++k) cur[k] = nxt[k];
          j = jn;
        }
      }
      const float inv = merge_inv(den);
      const int64_t grow = (int64_t)i * a.chunk_len + row;
      const int64_t fo = b * a.f_sb + grow * a.f_ss + h * a.f_sh + 4 * g;
#pragma unroll
      for (int k = 0; k < NP; ++k)
        store_row(a.final_out, a.final_bf16 != 0, fo + (k >> 2) * 32 + 8 * (k & 3), acc[k] * inv);
      if (g == 0 && a.final_lse != nullptr) a.final_lse[b * a.fl_sb + grow * a.fl_ss + h * a.fl_sh] = merged_lse(M, den);
    }
  }
}

}  // namespace

int partial_bf16_rows_per_block(int D) { return (D == 64 || D == 128) ? 256 : 128; }

int partial_bf16_head_pack_log2(int Sq, int G) {
  int hpl = 0;
  while (hpl < 3 && Sq <= (256 >> (hpl + 1)) && G % (2 << hpl) == 0) ++hpl;
  return hpl;
}

hipError_t launch_partial_bf16(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s) {
  const long long blocks = (long long)a.n_items * a.B * (a.Hq >> a.head_pack_log2) * n_qtiles;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (D == 128 && a.seg_tiles > 0)
    hipLaunchKernelGGL((partial_bf16_fast_kernel<128, true>), dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else if (D == 128)
    hipLaunchKernelGGL((partial_bf16_fast_kernel<128, false>), dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else if (D == 64 && a.seg_tiles > 0)
    hipLaunchKernelGGL((partial_bf16_fast_kernel<64, true>), dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else if (D == 64)
    hipLaunchKernelGGL((partial_bf16_fast_kernel<64, false>), dim3((unsigned)blocks), dim3(512), 0, s, a, n_qtiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace cpattn

