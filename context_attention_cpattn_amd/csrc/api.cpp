// C ABI of the context-parallel attention library: argument checks, the
// simulated CP ring driver, the split-KV decode driver and error reporting.
// Every check runs before the first HIP call; see include/cpattn.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/cpattn.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

cpattn_status fail(cpattn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

cpattn_status ok() {
  g_err.clear();
  return CPATTN_OK;
}

cpattn_status hip_fail(hipError_t e, const char* what) {
  return fail(CPATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxKvTokenStride = int64_t(1) << 24;

int64_t elem_bytes(int32_t dt) { return dt == CPATTN_BF16 ? 2 : (dt == CPATTN_F32 ? 4 : 0); }

int64_t numel(const cpattn_tensor& t) { return t.B * t.S * t.H * t.D; }

// Shape/stride/alignment checks of one descriptor.  `lse` tensors have D == 1
// and only need 4-byte alignment; others need 16-byte rows.
cpattn_status check_tensor(const cpattn_tensor* t, const char* name, bool lse) {
  if (t == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "%s: descriptor is NULL", name);
  if (t->reserved != 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: reserved field must be 0", name);
  const int64_t eb = elem_bytes(t->dtype);
  if (eb == 0) return fail(CPATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)t->dtype);
  if (t->B < 0 || t->S < 0 || t->H < 0 || t->D < 0)
    return fail(CPATTN_ERR_INVALID_ARG, "%s: negative size", name);
  if (t->stride_b < 0 || t->stride_s < 0 || t->stride_h < 0)
    return fail(CPATTN_ERR_INVALID_ARG, "%s: negative stride", name);
  if (lse && t->D != 1) return fail(CPATTN_ERR_INVALID_ARG, "%s: an LSE tensor must have D == 1", name);
  if (t->B > INT32_MAX || t->S >= (int64_t(1) << 30) || t->H > INT32_MAX)
    return fail(CPATTN_ERR_UNSUPPORTED, "%s: sequence lengths of 2^30 or more (or B, H beyond 2^31-1) are not supported", name);
  if (numel(*t) == 0) return ok();
  if (t->data == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "%s: data is NULL", name);
  const uintptr_t p = reinterpret_cast<uintptr_t>(t->data);
  if (lse) {
    if (p % 4) return fail(CPATTN_ERR_INVALID_ARG, "%s: data must be 4-byte aligned", name);
  } else {
    const int64_t q = 16 / eb;
    if (p % 16) return fail(CPATTN_ERR_INVALID_ARG, "%s: data must be 16-byte aligned", name);
    if (t->stride_b % q || t->stride_s % q || t->stride_h % q)
      return fail(CPATTN_ERR_INVALID_ARG, "%s: strides must be multiples of %lld elements", name, (long long)q);
    if (t->D > 1 && t->stride_h < t->D && t->H > 1)
      return fail(CPATTN_ERR_INVALID_ARG, "%s: stride_h smaller than D overlaps rows", name);
  }
  return ok();
}

bool same_bshd(const cpattn_tensor& a, const cpattn_tensor& b) {
  return a.B == b.B && a.S == b.S && a.H == b.H && a.D == b.D;
}
bool same_bsh(const cpattn_tensor& a, const cpattn_tensor& b) { return a.B == b.B && a.S == b.S && a.H == b.H; }
bool same_strides(const cpattn_tensor& a, const cpattn_tensor& b) {
  return a.stride_b == b.stride_b && a.stride_s == b.stride_s && a.stride_h == b.stride_h;
}

// Common checks for attention inputs q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D].
cpattn_status check_qkv(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v) {
  cpattn_status s;
  if ((s = check_tensor(q, "q", false)) != CPATTN_OK) return s;
  if ((s = check_tensor(k, "k", false)) != CPATTN_OK) return s;
  if ((s = check_tensor(v, "v", false)) != CPATTN_OK) return s;
  if (q->dtype != k->dtype || q->dtype != v->dtype)
    return fail(CPATTN_ERR_INVALID_ARG, "q, k and v must share one dtype");
  if (q->B != k->B || q->B != v->B) return fail(CPATTN_ERR_INVALID_ARG, "batch sizes of q, k, v differ");
  if (k->S != v->S || k->H != v->H) return fail(CPATTN_ERR_INVALID_ARG, "k and v shapes differ");
  if (q->D != k->D || q->D != v->D) return fail(CPATTN_ERR_INVALID_ARG, "head_dim of q, k, v differ");
  if (k->H < 1 || q->H < 1) return fail(CPATTN_ERR_INVALID_ARG, "head counts must be >= 1");
  if (q->H % k->H != 0) return fail(CPATTN_ERR_INVALID_ARG, "Hq (%lld) is not a multiple of Hkv (%lld)",
                                    (long long)q->H, (long long)k->H);
  if (q->D != 64 && q->D != 128)
    return fail(CPATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)q->D);
  if ((int64_t)q->B * q->H > INT32_MAX / 4) return fail(CPATTN_ERR_UNSUPPORTED, "B*Hq too large");
  // the prefill kernel addresses a K/V tile by 32-bit byte offsets from its start
  if (k->stride_s > kMaxKvTokenStride || v->stride_s > kMaxKvTokenStride)
    return fail(CPATTN_ERR_UNSUPPORTED, "k/v token strides above 2^24 elements are not supported");
  return ok();
}

cpattn::PartialLaunch base_partial(const cpattn_tensor& q, const cpattn_tensor& k, const cpattn_tensor& v) {
  cpattn::PartialLaunch a;
  std::memset(&a, 0, sizeof a);
  a.q = q.data;
  a.k = k.data;
  a.v = v.data;
  a.q_sb = q.stride_b; a.q_ss = q.stride_s; a.q_sh = q.stride_h;
  a.k_sb = k.stride_b; a.k_ss = k.stride_s; a.k_sh = k.stride_h;
  a.v_sb = v.stride_b; a.v_ss = v.stride_s; a.v_sh = v.stride_h;
  a.B = (int32_t)q.B;
  a.Hq = (int32_t)q.H;
  a.G = (int32_t)(q.H / k.H);
  a.xcd_order = 1;
  return a;
}

hipError_t launch_partial(cpattn::PartialLaunch& a, int dtype, int D, int Sq, hipStream_t st) {
  if (dtype == CPATTN_BF16) {
    // Packing heads trades workgroups for busy waves.  Estimated time: rounds of
    // workgroups over the compute units, times 1.64 when a SIMD holds two busy
    // waves instead of one (two waves per SIMD reach ~0.50 of peak against ~0.41
    // for one, so a workgroup with twice the rows takes ~1.64 times as long).
    int n_cu = 0;
    if (cpattn::cu_count(&n_cu) != hipSuccess) n_cu = 1;
    const int rpb0 = cpattn::partial_bf16_rows_per_block(D);
    const int hp_max = cpattn::partial_bf16_head_pack_log2(Sq, a.G);
    int hpl = 0;
    long long best = -1;
    for (int l = 0; l <= hp_max; ++l) {
      const int rpb = rpb0 >> l;
      const long long wgs = (long long)a.n_items * a.B * (a.Hq >> l) * ((Sq + rpb - 1) / rpb);
      const int busy = std::min(8, (1 << l) * ((std::min(Sq, rpb) + 31) / 32));  // waves with rows
      const long long est = (wgs + n_cu - 1) / n_cu * (busy > 4 ? 164 : 100);
      if (best < 0 || est < best) {
        best = est;
        hpl = l;
      }
    }
    a.head_pack_log2 = hpl;
    const int rpb = rpb0 >> hpl;
    return cpattn::launch_partial_bf16(a, D, (Sq + rpb - 1) / rpb, st);
  }
  const int rpb = cpattn::partial_f32_rows_per_block(D);
  return cpattn::launch_partial_f32(a, D, (Sq + rpb - 1) / rpb, st);
}

// ---- ring layout (host side; one GPU runs every rank)
//
// Q [B, Sq, Hq, D] and K/V [B, Skv, Hkv, D] are cut into P equal chunks: Q
// chunk i has Cq = Sq / P rows at global positions q0 + i Cq + [0, Cq) with
// q0 = Skv - Sq (the queries are the last Sq positions of the sequence, which
// makes Sq = Skv the full prefill); K/V chunk j has Ckv = Skv / P rows at
// j Ckv + [0, Ckv).  Under the causal mask Q chunk i sees the K/V chunks
// [0, n_vis[i]): those whose first key is not after its last query.  The
// workspace holds one slot per visible pair, slot0[i] + j.
struct RingLayout {
  int P;
  int64_t Cq, Ckv, q0;
  int64_t n_items, slot_o, slot_l;  // slots; elements per O slot / LSE slot
  int32_t n_vis[cpattn::kMaxMerge], slot0[cpattn::kMaxMerge];
  size_t o_bytes, bytes;
};

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

RingLayout ring_layout(const cpattn_tensor& q, int64_t Skv, int P, bool causal) {
  RingLayout L;
  std::memset(&L, 0, sizeof L);
  L.P = P;
  L.Cq = q.S / P;
  L.Ckv = Skv / P;
  L.q0 = Skv - q.S;
  for (int i = 0; i < P; ++i) {
    int64_t n = P;
    if (L.Cq == 0) n = 0;
    else if (causal) n = std::min<int64_t>(P, (L.q0 + (i + 1) * L.Cq - 1) / L.Ckv + 1);
    L.n_vis[i] = (int32_t)n;
    L.slot0[i] = (int32_t)L.n_items;
    L.n_items += n;
  }
  L.slot_o = q.B * L.Cq * q.H * q.D;
  L.slot_l = q.B * L.Cq * q.H;
  L.o_bytes = align_up((size_t)(L.n_items * L.slot_o) * 4);
  L.bytes = L.o_bytes + align_up((size_t)(L.n_items * L.slot_l) * 4);
  return L;
}

struct Pair {
  int q, kv;
};

// Work items of ring step s: rank r holds (Q_r, KV_{(r-s) mod P}) under
// Pass-KV and (Q_{(r-s) mod P}, KV_r) under Pass-Q; pairs whose K/V chunk the
// Q chunk sees nothing of are dropped.
std::vector<Pair> ring_step(const RingLayout& L, int s, int order) {
  std::vector<Pair> items;
  const int P = L.P;
  for (int r = 0; r < P; ++r) {
    const int other = ((r - s) % P + P) % P;
    const Pair p = (order == CPATTN_PASS_KV) ? Pair{r, other} : Pair{other, r};
    if (p.kv >= L.n_vis[p.q]) continue;
    items.push_back(p);
  }
  return items;
}

// Bytes a P-rank ring would move between ranks.  At every step after the
// first each rank receives its neighbour's chunk: K and V of one chunk under
// Pass-KV, one Q chunk under Pass-Q.  Under Pass-Q every pair computed away
// from its Q chunk's owner (all visible pairs but the P diagonal ones) also
// sends its partial back: fp32 O and fp32 LSE per query row and head.
struct RingBytes {
  uint64_t pass_kv, pass_q;
};

RingBytes ring_bytes(const cpattn_tensor& q, const cpattn_tensor& k, const RingLayout& L) {
  const uint64_t e = (uint64_t)elem_bytes(q.dtype);
  const uint64_t hops = (uint64_t)L.P * (uint64_t)(L.P - 1);
  const uint64_t kv_chunk = 2 * (uint64_t)q.B * L.Ckv * k.H * q.D * e;
  const uint64_t q_chunk = (uint64_t)q.B * L.Cq * q.H * q.D * e;
  const uint64_t partial = (uint64_t)q.B * L.Cq * q.H * (q.D + 1) * 4;
  const uint64_t remote = L.n_items > L.P ? (uint64_t)(L.n_items - L.P) : 0;
  return RingBytes{hops * kv_chunk, hops * q_chunk + remote * partial};
}

// CPATTN_ORDER_AUTO: the order that moves fewer bytes, Pass-KV on a tie.
int resolve_order(int order, const cpattn_tensor& q, const cpattn_tensor& k, const RingLayout& L) {
  if (order != CPATTN_ORDER_AUTO) return order;
  const RingBytes rb = ring_bytes(q, k, L);
  return rb.pass_q < rb.pass_kv ? CPATTN_PASS_Q : CPATTN_PASS_KV;
}

bool valid_order(int order) { return order == CPATTN_PASS_KV || order == CPATTN_PASS_Q || order == CPATTN_ORDER_AUTO; }

cpattn_status check_ring(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int n_chunks,
                         int order, int causal) {
  cpattn_status s;
  if ((s = check_qkv(q, k, v)) != CPATTN_OK) return s;
  if (k->S < q->S)
    return fail(CPATTN_ERR_INVALID_ARG, "k/v (%lld rows) must be at least as long as q (%lld rows): the queries are "
                "the last positions of the sequence", (long long)k->S, (long long)q->S);
  if (n_chunks < 1) return fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be >= 1");
  if (n_chunks > cpattn::kMaxMerge)
    return fail(CPATTN_ERR_UNSUPPORTED, "n_chunks above %d not supported", cpattn::kMaxMerge);
  if (q->S % n_chunks != 0 || k->S % n_chunks != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "sequence lengths %lld (q) and %lld (k/v) must both be divisible by n_chunks %d",
                (long long)q->S, (long long)k->S, n_chunks);
  if (!valid_order(order)) return fail(CPATTN_ERR_INVALID_ARG, "unknown ring order");
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  return ok();
}

// ---- split-KV decode layout
//
// n_chunks K/V blocks of at most `cap` rows each.  The decode kernel runs one
// persistent workgroup per CU that streams its units back to back; about four
// units per CU of a 256-CU device balance the load without cutting the stream
// into many short units, so blocks are cut into sub-splits (of at least 256
// keys) until there are about 1024 units.
struct DecodeLayout {
  int n_split, split_len, head_blocks, n_part;
  size_t o_bytes, bytes;
};

DecodeLayout decode_layout(const cpattn_tensor& q, int64_t Hkv, int64_t cap, int n_chunks) {
  DecodeLayout L;
  const int64_t G = q.H / Hkv;
  L.head_blocks = (int)((G + 15) / 16);
  const int64_t base_units = q.B * Hkv * L.head_blocks * n_chunks;
  int ns = 1;
  while (base_units * ns < 1024 && cap / (2 * ns) >= 256 && (int64_t)n_chunks * ns * 2 <= cpattn::kMaxMerge) ns *= 2;
  L.n_split = ns;
  const int64_t per = (cap + ns - 1) / ns;
  L.split_len = (int)((per + 31) / 32 * 32);
  if (L.split_len == 0) L.split_len = 32;
  L.n_part = n_chunks * ns;
  L.o_bytes = align_up((size_t)(L.n_part * q.B * q.H * q.D) * 4);
  L.bytes = L.o_bytes + align_up((size_t)(L.n_part * q.B * q.H) * 4);
  return L;
}

cpattn_status check_decode(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v, int n_chunks) {
  cpattn_status s;
  if ((s = check_qkv(q, k, v)) != CPATTN_OK) return s;
  if (q->dtype != CPATTN_BF16) return fail(CPATTN_ERR_UNSUPPORTED, "split-KV decode takes BF16 inputs");
  if (q->S != 1) return fail(CPATTN_ERR_INVALID_ARG, "split-KV decode takes one query token (q.S == 1)");
  if (n_chunks < 1) return fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be >= 1");
  if (n_chunks > cpattn::kMaxMerge)
    return fail(CPATTN_ERR_UNSUPPORTED, "n_chunks above %d not supported", cpattn::kMaxMerge);
  if (k->S % n_chunks != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "KV length %lld not divisible by n_chunks %d", (long long)k->S, n_chunks);
  if (q->H / k->H > 64) return fail(CPATTN_ERR_UNSUPPORTED, "more than 64 query heads per KV head");
  return ok();
}

cpattn_status check_out(const cpattn_tensor* out, const cpattn_tensor* lse, const cpattn_tensor& q,
                        bool out_bf16_ok, bool lse_required) {
  cpattn_status s;
  if ((s = check_tensor(out, "out", false)) != CPATTN_OK) return s;
  if (!(out->dtype == CPATTN_F32 || (out_bf16_ok && out->dtype == CPATTN_BF16)))
    return fail(CPATTN_ERR_INVALID_ARG, "out has an unsupported dtype");
  if (!same_bshd(*out, q)) return fail(CPATTN_ERR_INVALID_ARG, "out shape differs from q");
  if (lse == nullptr) {
    if (lse_required) return fail(CPATTN_ERR_INVALID_ARG, "lse descriptor is NULL");
    return ok();
  }
  if ((s = check_tensor(lse, "lse", true)) != CPATTN_OK) return s;
  if (lse->dtype != CPATTN_F32) return fail(CPATTN_ERR_INVALID_ARG, "lse must be F32");
  if (!same_bsh(*lse, q)) return fail(CPATTN_ERR_INVALID_ARG, "lse shape differs from q's [B, S, H]");
  return ok();
}

cpattn_status check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return ok();
  if (ws == nullptr) return fail(CPATTN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 16) return fail(CPATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if (have < need) return fail(CPATTN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return ok();
}

// K/V cache shards: n descriptors of one shape, dtype and strides (only the
// data pointers differ), with the K and V shards alike.
cpattn_status check_shards(const cpattn_tensor* ks, const cpattn_tensor* vs, int n) {
  if (ks == nullptr || vs == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "shard arrays are NULL");
  if (n < 1) return fail(CPATTN_ERR_INVALID_ARG, "the number of shards must be >= 1");
  if (n > cpattn::kMaxMerge) return fail(CPATTN_ERR_UNSUPPORTED, "more than %d shards", cpattn::kMaxMerge);
  cpattn_status s;
  for (int r = 0; r < n; ++r) {
    if ((s = check_tensor(&ks[r], "k shard", false)) != CPATTN_OK) return s;
    if ((s = check_tensor(&vs[r], "v shard", false)) != CPATTN_OK) return s;
    if (ks[r].dtype != ks[0].dtype || vs[r].dtype != ks[0].dtype)
      return fail(CPATTN_ERR_INVALID_ARG, "shards must share one dtype");
    if (!same_bshd(ks[r], ks[0]) || !same_strides(ks[r], ks[0]))
      return fail(CPATTN_ERR_INVALID_ARG, "k shard %d differs in shape or strides from k shard 0", r);
    if (!same_bshd(vs[r], ks[0]) || !same_strides(vs[r], vs[0]))
      return fail(CPATTN_ERR_INVALID_ARG, "v shard %d differs in shape or strides", r);
  }
  if (ks[0].D != 64 && ks[0].D != 128)
    return fail(CPATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)ks[0].D);
  return ok();
}

// Split-KV decode of q against K/V blocks kc[c], vc[c] of len[c] rows (the
// blocks share strides), then the merge of the partials in block order.
cpattn_status run_decode(const cpattn_tensor& q, const cpattn_tensor& k, const cpattn_tensor& v, int n_blocks,
                         const void* const* kc, const void* const* vc, const int64_t* len, const DecodeLayout& L,
                         cpattn_tensor* out, cpattn_tensor* lse, void* workspace, hipStream_t st) {
  float* ws_o = static_cast<float*>(workspace);
  float* ws_l = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.o_bytes);
  cpattn::DecodeLaunch d;
  std::memset(&d, 0, sizeof d);
  d.q = q.data;
  d.o = ws_o; d.lse = ws_l;
  d.o_slot = q.B * q.H * q.D; d.o_sb = q.H * q.D; d.o_sh = q.D;
  d.l_slot = q.B * q.H; d.l_sb = q.H; d.l_sh = 1;
  d.q_sb = q.stride_b; d.q_sh = q.stride_h;
  d.k_sb = k.stride_b; d.k_ss = k.stride_s; d.k_sh = k.stride_h;
  d.v_sb = v.stride_b; d.v_ss = v.stride_s; d.v_sh = v.stride_h;
  d.B = (int32_t)q.B; d.Hq = (int32_t)q.H; d.Hkv = (int32_t)k.H; d.G = (int32_t)(q.H / k.H);
  d.n_chunks = n_blocks;
  d.n_split = L.n_split;
  d.split_len = L.split_len;
  d.head_blocks = L.head_blocks;
  for (int c = 0; c < n_blocks; ++c) {
    d.kc[c] = kc[c];
    d.vc[c] = vc[c];
    d.len[c] = (int32_t)len[c];
  }
  hipError_t e = cpattn::launch_decode_bf16(d, (int)q.D, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");

  cpattn::MergeLaunch m;
  std::memset(&m, 0, sizeof m);
  m.n = L.n_part;
  const int64_t part_o = q.B * q.H * q.D, part_l = q.B * q.H;
  for (int c = 0; c < m.n; ++c) {
    m.o[c] = ws_o + c * part_o;
    m.lse[c] = ws_l + c * part_l;
  }
  m.out_bf16 = out->dtype == CPATTN_BF16;
  m.B = (int32_t)q.B; m.S = 1; m.H = (int32_t)q.H; m.D = (int32_t)q.D;
  m.p_sb = q.H * q.D; m.p_ss = q.H * q.D; m.p_sh = q.D;
  m.pl_sb = q.H; m.pl_ss = q.H; m.pl_sh = 1;
  m.out = out->data;
  m.o_sb = out->stride_b; m.o_ss = out->stride_s; m.o_sh = out->stride_h;
  if (lse != nullptr) {
    m.out_lse = static_cast<float*>(lse->data);
    m.ol_sb = lse->stride_b; m.ol_ss = lse->stride_s; m.ol_sh = lse->stride_h;
  }
  e = cpattn::launch_merge(m, st);
  if (e != hipSuccess) return hip_fail(e, "decode merge launch");
  return ok();
}

// Partial attention of the given (q-chunk, kv-chunk) pairs into their
// workspace slots, in launches of at most kMaxItems pairs.
cpattn_status launch_ring_items(const cpattn_tensor& q, const cpattn_tensor& k, const cpattn_tensor& v,
                                const RingLayout& L, bool causal, const std::vector<Pair>& pairs, void* workspace,
                                void* stream, const char* what) {
  cpattn::PartialLaunch a = base_partial(q, k, v);
  a.o = static_cast<float*>(workspace);
  a.lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.o_bytes);
  a.o_sh = q.D; a.o_ss = q.H * q.D; a.o_sb = L.Cq * q.H * q.D;
  a.l_sh = 1; a.l_ss = q.H; a.l_sb = L.Cq * q.H;
  a.o_slot = L.slot_o;
  a.l_slot = L.slot_l;
  a.q_pos0 = L.q0;
  a.chunk_len = L.Cq;
  a.kv_chunk_len = L.Ckv;
  a.Sq = (int32_t)L.Cq;
  a.Sk = (int32_t)L.Ckv;
  a.causal = causal ? 1 : 0;
  size_t i = 0;
  while (i < pairs.size()) {
    a.n_items = 0;
    for (; i < pairs.size() && a.n_items < cpattn::kMaxItems; ++i)
      a.items[a.n_items++] = cpattn::Item{pairs[i].q, pairs[i].kv, L.slot0[pairs[i].q] + pairs[i].kv, 0};
    const hipError_t e = launch_partial(a, q.dtype, (int)q.D, (int)L.Cq, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return ok();
}

// Keys [0, sk) of the K/V sequence that some query of Q chunk i can see.
int64_t owner_keys(const RingLayout& L, int i, bool causal) {
  const int64_t Skv = L.Ckv * L.P;
  return causal ? std::min<int64_t>(Skv, L.q0 + (i + 1) * L.Cq) : Skv;
}

cpattn_status ring_merge_impl(const RingLayout& L, int order, const void* workspace, cpattn_tensor* out,
                              cpattn_tensor* lse, void* stream) {
  cpattn::RingMergeLaunch m;
  std::memset(&m, 0, sizeof m);
  m.ws_o = static_cast<const float*>(workspace);
  m.ws_l = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + L.o_bytes);
  m.slot_o = L.slot_o;
  m.slot_l = L.slot_l;
  m.P = L.P;
  m.C = (int32_t)L.Cq; m.B = (int32_t)out->B; m.H = (int32_t)out->H; m.D = (int32_t)out->D;
  m.pass_q = order == CPATTN_PASS_Q ? 1 : 0;
  m.out_bf16 = out->dtype == CPATTN_BF16;
  m.out = out->data;
  m.o_sb = out->stride_b; m.o_ss = out->stride_s; m.o_sh = out->stride_h;
  if (lse != nullptr) {
    m.out_lse = static_cast<float*>(lse->data);
    m.ol_sb = lse->stride_b; m.ol_ss = lse->stride_s; m.ol_sh = lse->stride_h;
  }
  for (int i = 0; i < L.P; ++i) {
    m.n_vis[i] = L.n_vis[i];
    m.slot0[i] = L.slot0[i];
  }
  const hipError_t e = cpattn::launch_ring_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ring merge launch");
  return ok();
}

}  // namespace

extern "C" {

const char* cpattn_last_error(void) { return g_err.c_str(); }

const char* cpattn_version(void) { return "cpattn 0.2.0 gfx950"; }

cpattn_status cpattn_partial(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                             int64_t q_offset, int64_t kv_offset, int causal, cpattn_tensor* out,
                             cpattn_tensor* lse, void* stream) {
  cpattn_status s;
  if ((s = check_qkv(q, k, v)) != CPATTN_OK) return s;
  if ((s = check_out(out, lse, *q, false, true)) != CPATTN_OK) return s;
  if (q_offset < 0 || kv_offset < 0) return fail(CPATTN_ERR_INVALID_ARG, "offsets must be >= 0");
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (q->S == 0 || q->B == 0) return ok();

  // One query row per sequence (a decode-shaped call) with at most 64 query
  // heads per KV head goes to the split-KV decode kernel as a single partial:
  // its query heads share each K/V read, where the prefill kernel would give
  // every head a 256-row workgroup of its own.  The row sees the key prefix
  // [0, visible).
  const int64_t G = q->H / k->H;
  if (q->S == 1 && q->dtype == CPATTN_BF16 && (q->D == 64 || q->D == 128) && G <= 64) {
    int64_t visible = k->S;
    if (causal) visible = std::max<int64_t>(0, std::min<int64_t>(k->S, q_offset - kv_offset + 1));
    cpattn::DecodeLaunch d;
    std::memset(&d, 0, sizeof d);
    d.q = q->data;
    d.kc[0] = k->data; d.vc[0] = v->data; d.len[0] = (int32_t)visible;
    d.o = static_cast<float*>(out->data);
    d.lse = static_cast<float*>(lse->data);
    d.o_slot = 0; d.o_sb = out->stride_b; d.o_sh = out->stride_h;
    d.l_slot = 0; d.l_sb = lse->stride_b; d.l_sh = lse->stride_h;
    d.q_sb = q->stride_b; d.q_sh = q->stride_h;
    d.k_sb = k->stride_b; d.k_ss = k->stride_s; d.k_sh = k->stride_h;
    d.v_sb = v->stride_b; d.v_ss = v->stride_s; d.v_sh = v->stride_h;
    d.B = (int32_t)q->B; d.Hq = (int32_t)q->H; d.Hkv = (int32_t)k->H; d.G = (int32_t)G;
    d.n_chunks = 1;
    d.n_split = 1;
    d.split_len = (int32_t)((std::max<int64_t>(visible, 1) + 63) / 64 * 64);
    d.head_blocks = (int32_t)((G + 15) / 16);
    const hipError_t e = cpattn::launch_decode_bf16(d, (int)q->D, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "partial attention (one query row) launch");
    return ok();
  }

  cpattn::PartialLaunch a = base_partial(*q, *k, *v);
  a.o = static_cast<float*>(out->data);
  a.lse = static_cast<float*>(lse->data);
  a.o_sb = out->stride_b; a.o_ss = out->stride_s; a.o_sh = out->stride_h;
  a.l_sb = lse->stride_b; a.l_ss = lse->stride_s; a.l_sh = lse->stride_h;
  a.q_pos0 = q_offset;
  a.kv_pos0 = kv_offset;
  a.Sq = (int32_t)q->S;
  a.Sk = (int32_t)k->S;
  a.causal = causal;
  a.n_items = 1;
  a.items[0] = cpattn::Item{0, 0, 0, 0};
  const hipError_t e = launch_partial(a, q->dtype, (int)q->D, (int)q->S, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "partial attention launch");
  return ok();
}

cpattn_status cpattn_merge(const cpattn_tensor* partials, const cpattn_tensor* lses, int n, cpattn_tensor* out,
                           cpattn_tensor* out_lse, void* stream) {
  if (partials == nullptr || lses == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "partials/lses array is NULL");
  if (n < 1 || n > cpattn::kMaxMerge) return fail(CPATTN_ERR_INVALID_ARG, "n must be in [1, %d]", cpattn::kMaxMerge);
  cpattn_status s;
  const cpattn_tensor& p0 = partials[0];
  const cpattn_tensor& l0 = lses[0];
  for (int c = 0; c < n; ++c) {
    if ((s = check_tensor(&partials[c], "partial", false)) != CPATTN_OK) return s;
    if ((s = check_tensor(&lses[c], "partial lse", true)) != CPATTN_OK) return s;
    if (partials[c].dtype != CPATTN_F32 || lses[c].dtype != CPATTN_F32)
      return fail(CPATTN_ERR_INVALID_ARG, "partials and their LSE must be F32");
    if (!same_bshd(partials[c], p0) || !same_strides(partials[c], p0))
      return fail(CPATTN_ERR_INVALID_ARG, "partial %d differs in shape or strides from partial 0", c);
    if (!same_bsh(lses[c], p0) || !same_strides(lses[c], l0))
      return fail(CPATTN_ERR_INVALID_ARG, "lse %d differs in shape or strides", c);
  }
  if (p0.D != 64 && p0.D != 128)
    return fail(CPATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)p0.D);
  if ((s = check_out(out, out_lse, p0, true, false)) != CPATTN_OK) return s;
  if (numel(p0) == 0) return ok();

  cpattn::MergeLaunch m;
  std::memset(&m, 0, sizeof m);
  for (int c = 0; c < n; ++c) {
    m.o[c] = static_cast<const float*>(partials[c].data);
    m.lse[c] = static_cast<const float*>(lses[c].data);
  }
  m.n = n;
  m.out_bf16 = out->dtype == CPATTN_BF16;
  m.B = (int32_t)p0.B; m.S = (int32_t)p0.S; m.H = (int32_t)p0.H; m.D = (int32_t)p0.D;
  m.p_sb = p0.stride_b; m.p_ss = p0.stride_s; m.p_sh = p0.stride_h;
  m.pl_sb = l0.stride_b; m.pl_ss = l0.stride_s; m.pl_sh = l0.stride_h;
  m.out = out->data;
  m.o_sb = out->stride_b; m.o_ss = out->stride_s; m.o_sh = out->stride_h;
  if (out_lse != nullptr) {
    m.out_lse = static_cast<float*>(out_lse->data);
    m.ol_sb = out_lse->stride_b; m.ol_ss = out_lse->stride_s; m.ol_sh = out_lse->stride_h;
  }
  const hipError_t e = cpattn::launch_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

size_t cpattn_ring_prefill_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks, int causal) {
  if (check_tensor(q, "q", false) != CPATTN_OK) return 0;
  int64_t Skv = q->S;
  if (k != nullptr) {
    if (check_tensor(k, "k", false) != CPATTN_OK) return 0;
    Skv = k->S;
  }
  if (Skv < q->S) {
    fail(CPATTN_ERR_INVALID_ARG, "k/v must be at least as long as q");
    return 0;
  }
  if (n_chunks < 1 || n_chunks > cpattn::kMaxMerge || q->S % n_chunks != 0 || Skv % n_chunks != 0) {
    fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be in [1, %d] and divide both sequence lengths", cpattn::kMaxMerge);
    return 0;
  }
  if (causal != 0 && causal != 1) {
    fail(CPATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
    return 0;
  }
  ok();
  return ring_layout(*q, Skv, n_chunks, causal != 0).bytes;
}

cpattn_status cpattn_ring_select_order(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks, int causal,
                                       int* order, uint64_t* bytes_pass_kv, uint64_t* bytes_pass_q) {
  cpattn_status s;
  if ((s = check_tensor(q, "q", false)) != CPATTN_OK) return s;
  if ((s = check_tensor(k, "k", false)) != CPATTN_OK) return s;
  if (order == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "order is NULL");
  if (q->B != k->B || q->D != k->D || k->H < 1 || q->H % k->H != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "q and k shapes do not match");
  if (q->dtype != k->dtype) return fail(CPATTN_ERR_INVALID_ARG, "q and k must share one dtype");
  if (k->S < q->S) return fail(CPATTN_ERR_INVALID_ARG, "k/v must be at least as long as q");
  if (n_chunks < 1 || n_chunks > cpattn::kMaxMerge || q->S % n_chunks != 0 || k->S % n_chunks != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be in [1, %d] and divide both sequence lengths",
                cpattn::kMaxMerge);
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  const RingLayout L = ring_layout(*q, k->S, n_chunks, causal != 0);
  const RingBytes rb = ring_bytes(*q, *k, L);
  *order = rb.pass_q < rb.pass_kv ? CPATTN_PASS_Q : CPATTN_PASS_KV;
  if (bytes_pass_kv != nullptr) *bytes_pass_kv = rb.pass_kv;
  if (bytes_pass_q != nullptr) *bytes_pass_q = rb.pass_q;
  return ok();
}

cpattn_status cpattn_ring_step(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                               int n_chunks, int order /* cpattn_order */, int causal, int step, void* workspace,
                               size_t workspace_bytes, void* stream) {
  cpattn_status s;
  if ((s = check_ring(q, k, v, n_chunks, order, causal)) != CPATTN_OK) return s;
  if (step < 0 || step >= n_chunks) return fail(CPATTN_ERR_INVALID_ARG, "step %d outside [0, %d)", step, n_chunks);
  if (q->S == 0 || q->B == 0) return ok();
  const bool cz = causal != 0;
  const RingLayout L = ring_layout(*q, k->S, n_chunks, cz);
  if ((s = check_workspace(workspace, workspace_bytes, L.bytes)) != CPATTN_OK) return s;
  const int ord = resolve_order(order, *q, *k, L);
  return launch_ring_items(*q, *k, *v, L, cz, ring_step(L, step, ord), workspace, stream, "ring step launch");
}

cpattn_status cpattn_ring_step_accumulate(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                          int n_chunks, int order /* cpattn_order */, int causal, int step,
                                          cpattn_tensor* out, cpattn_tensor* lse, void* stream) {
  cpattn_status s;
  if ((s = check_ring(q, k, v, n_chunks, order, causal)) != CPATTN_OK) return s;
  if (step < 0 || step >= n_chunks) return fail(CPATTN_ERR_INVALID_ARG, "step %d outside [0, %d)", step, n_chunks);
  if ((s = check_out(out, lse, *q, false, true)) != CPATTN_OK) return s;
  if (q->S == 0 || q->B == 0) return ok();
  const bool cz = causal != 0;
  const RingLayout L = ring_layout(*q, k->S, n_chunks, cz);
  const int ord = resolve_order(order, *q, *k, L);
  cpattn::PartialLaunch a = base_partial(*q, *k, *v);
  a.o = static_cast<float*>(out->data);
  a.o_sb = out->stride_b; a.o_ss = out->stride_s; a.o_sh = out->stride_h;
  a.o_slot = L.Cq * out->stride_s;  // owner i's rows start at row i Cq
  a.lse = static_cast<float*>(lse->data);
  a.l_sb = lse->stride_b; a.l_ss = lse->stride_s; a.l_sh = lse->stride_h;
  a.l_slot = L.Cq * lse->stride_s;
  a.q_pos0 = L.q0;
  a.chunk_len = L.Cq;
  a.kv_chunk_len = L.Ckv;
  a.Sq = (int32_t)L.Cq;
  a.Sk = (int32_t)L.Ckv;
  a.causal = cz ? 1 : 0;
  // step 0 is every owner's first arrival (its own chunk): it writes; later steps merge
  a.accumulate = step > 0 ? 1 : 0;
  a.n_items = 0;
  for (const Pair& p : ring_step(L, step, ord)) a.items[a.n_items++] = cpattn::Item{p.q, p.kv, p.q, 0};
  if (a.n_items == 0) return ok();
  const hipError_t e = launch_partial(a, q->dtype, (int)q->D, (int)L.Cq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "accumulating ring step launch");
  return ok();
}

cpattn_status cpattn_ring_merge(int n_chunks, int order /* cpattn_order */, int causal, int64_t kv_len, const void* workspace,
                                size_t workspace_bytes, cpattn_tensor* out, cpattn_tensor* lse, void* stream) {
  cpattn_status s;
  if (n_chunks < 1) return fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be >= 1");
  if (n_chunks > cpattn::kMaxMerge)
    return fail(CPATTN_ERR_UNSUPPORTED, "n_chunks above %d not supported", cpattn::kMaxMerge);
  if (order != CPATTN_PASS_KV && order != CPATTN_PASS_Q)
    return fail(CPATTN_ERR_INVALID_ARG, "ring merge needs the order the steps ran in (Pass-KV or Pass-Q)");
  if (causal != 0 && causal != 1) return fail(CPATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if ((s = check_tensor(out, "out", false)) != CPATTN_OK) return s;
  if (out->D != 64 && out->D != 128)
    return fail(CPATTN_ERR_UNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)out->D);
  if ((s = check_out(out, lse, *out, true, false)) != CPATTN_OK) return s;
  if (kv_len < out->S) return fail(CPATTN_ERR_INVALID_ARG, "kv_len %lld shorter than the output's %lld rows",
                                   (long long)kv_len, (long long)out->S);
  if (out->S % n_chunks != 0 || kv_len % n_chunks != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "sequence lengths %lld (q) and %lld (k/v) must both be divisible by n_chunks %d",
                (long long)out->S, (long long)kv_len, n_chunks);
  if (out->S == 0 || out->B == 0) return ok();
  const RingLayout L = ring_layout(*out, kv_len, n_chunks, causal != 0);
  if ((s = check_workspace(const_cast<void*>(workspace), workspace_bytes, L.bytes)) != CPATTN_OK) return s;
  return ring_merge_impl(L, order, workspace, out, lse, stream);
}

cpattn_status cpattn_ring_prefill(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                  int n_chunks, int order /* cpattn_order */, int causal, cpattn_tensor* out,
                                  cpattn_tensor* lse, void* workspace, size_t workspace_bytes, void* stream) {
  cpattn_status s;
  if ((s = check_ring(q, k, v, n_chunks, order, causal)) != CPATTN_OK) return s;
  if ((s = check_out(out, lse, *q, true, false)) != CPATTN_OK) return s;
  if (q->S == 0 || q->B == 0) return ok();
  const bool cz = causal != 0;
  const RingLayout L = ring_layout(*q, k->S, n_chunks, cz);
  if ((s = check_workspace(workspace, workspace_bytes, L.bytes)) != CPATTN_OK) return s;
  const int ord = resolve_order(order, *q, *k, L);
  // On one device the pairs of all ring steps are independent, so they go
  // out together; each lands in its own slot, and the merge reads the slots
  // in the ring order's arrival order.
  int n_cu = 0;
  if (cpattn::cu_count(&n_cu) != hipSuccess) n_cu = 1;
  const long long walk_wgs = (long long)n_chunks * q->B * q->H * ((L.Cq + 255) / 256);
  if (q->dtype == CPATTN_BF16 && (q->D == 128 || q->D == 64) && L.Ckv % 64 == 0 && L.Ckv <= 16384 &&
      walk_wgs >= 2LL * n_cu) {
    // K/V chunks of a multiple of 64 tokens: one work item per owner whose
    // query tile walks every key it sees in one pass (as in the fused
    // prefill), writing each K/V chunk's partial to that pair's slot at the
    // chunk boundary and restarting the softmax there exactly as a launch of
    // the pair alone would -- the same partials, bit for bit, without a
    // workgroup prologue per pair -- and merging them at the end of the walk.
    // 8K tokens in 1024-token chunks: 0.357 -> 0.326 ms against per-pair
    // launches and a merge pass; 128K in 8192-token chunks: 60.1 -> 57.7 ms.
    // Longer chunks amortise a pair's prologue over more tiles than the
    // walk's boundary code costs (1M in 131072-token chunks: per-pair 0.8%
    // faster), so they launch per pair.  So do walks of fewer than two
    // workgroups per compute unit, whose per-pair workgroups fill the chip
    // (and can pack heads): 2048 new tokens on 131072 cached ones, 16 ranks
    // (256 walking workgroups): 2.29 -> 1.79 ms.
    cpattn::PartialLaunch a = base_partial(*q, *k, *v);
    a.o = static_cast<float*>(workspace);
    a.lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.o_bytes);
    a.o_sh = q->D; a.o_ss = q->H * q->D; a.o_sb = L.Cq * q->H * q->D;
    a.l_sh = 1; a.l_ss = q->H; a.l_sb = L.Cq * q->H;
    a.o_slot = L.slot_o;
    a.l_slot = L.slot_l;
    a.q_pos0 = L.q0;
    a.chunk_len = L.Cq;
    a.kv_chunk_len = L.Ckv;
    a.Sq = (int32_t)L.Cq;
    a.Sk = (int32_t)k->S;
    a.causal = cz ? 1 : 0;
    a.seg_tiles = (int32_t)(L.Ckv / 64);
    a.xcd_order = 0;  // launch order, heaviest owner first
    // Each query tile merges its own partials when its walk is done (arrival
    // order, the ring merge kernel's arithmetic), so no merge pass follows.
    a.final_out = out->data;
    a.final_bf16 = out->dtype == CPATTN_BF16;
    a.pass_q = ord == CPATTN_PASS_Q ? 1 : 0;
    a.f_sb = out->stride_b; a.f_ss = out->stride_s; a.f_sh = out->stride_h;
    if (lse != nullptr) {
      a.final_lse = static_cast<float*>(lse->data);
      a.fl_sb = lse->stride_b; a.fl_ss = lse->stride_s; a.fl_sh = lse->stride_h;
    }
    a.n_items = 0;
    for (int i = n_chunks - 1; i >= 0; --i)
      a.items[a.n_items++] = cpattn::Item{i, 0, L.slot0[i], (int32_t)owner_keys(L, i, cz)};
    const hipError_t e = launch_partial(a, q->dtype, (int)q->D, (int)L.Cq, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "ring prefill launch");
    return ok();
  }
  // The workgroups of a launch are dealt to the XCDs in contiguous eighths of
  // the grid, so the diagonal pairs (half the work of a full pair under the
  // causal mask at equal lengths) are spread evenly through the list: every
  // eighth gets its share of them.
  std::vector<Pair> full, diag;
  for (int step = 0; step < n_chunks; ++step)
    for (const Pair& p : ring_step(L, step, ord)) (cz && p.q == p.kv ? diag : full).push_back(p);
  std::vector<Pair> pairs;
  pairs.reserve(full.size() + diag.size());
  const size_t n = full.size() + diag.size();
  size_t fi = 0, di = 0;
  for (size_t i = 0; i < n; ++i) {
    // diagonal pair number d goes to position floor((d + 0.5) * n / n_diag)
    const bool take_diag = di < diag.size() && (fi == full.size() || (2 * di + 1) * n <= 2 * i * diag.size() + diag.size());
    pairs.push_back(take_diag ? diag[di++] : full[fi++]);
  }
  if ((s = launch_ring_items(*q, *k, *v, L, cz, pairs, workspace, stream, "ring prefill launch")) != CPATTN_OK)
    return s;
  return ring_merge_impl(L, ord, workspace, out, lse, stream);
}

cpattn_status cpattn_ring_prefill_fused(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                        int n_chunks, int causal, cpattn_tensor* out, cpattn_tensor* lse,
                                        void* stream) {
  cpattn_status s;
  if ((s = check_ring(q, k, v, n_chunks, CPATTN_PASS_KV, causal)) != CPATTN_OK) return s;
  if ((s = check_out(out, lse, *q, false, false)) != CPATTN_OK) return s;
  if (q->S == 0 || q->B == 0) return ok();
  const int P = n_chunks;
  const bool cz = causal != 0;
  const RingLayout L = ring_layout(*q, k->S, P, cz);
  cpattn::PartialLaunch a = base_partial(*q, *k, *v);
  a.o = static_cast<float*>(out->data);
  a.o_sb = out->stride_b; a.o_ss = out->stride_s; a.o_sh = out->stride_h;
  a.o_slot = L.Cq * out->stride_s;  // owner i's rows start at row i Cq of the output
  if (lse != nullptr) {
    a.lse = static_cast<float*>(lse->data);
    a.l_sb = lse->stride_b; a.l_ss = lse->stride_s; a.l_sh = lse->stride_h;
    a.l_slot = L.Cq * lse->stride_s;
  }
  a.q_pos0 = L.q0;
  a.chunk_len = L.Cq;
  a.kv_chunk_len = L.Ckv;
  a.Sq = (int32_t)L.Cq;
  a.Sk = (int32_t)k->S;
  a.causal = causal;
  // One item per owner: Q chunk i against the keys it sees, accumulated in
  // one pass.  The owners' costs differ up to P-fold, so the grid keeps its
  // launch order (consecutive workgroups go to different XCDs) with the
  // heaviest owner first.
  a.xcd_order = 0;
  a.n_items = 0;
  for (int i = P - 1; i >= 0; --i) a.items[a.n_items++] = cpattn::Item{i, 0, i, (int32_t)owner_keys(L, i, cz)};
  const hipError_t e = launch_partial(a, q->dtype, (int)q->D, (int)L.Cq, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fused ring prefill launch");
  return ok();
}

size_t cpattn_splitkv_decode_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k, int n_chunks) {
  if (check_tensor(q, "q", false) != CPATTN_OK || check_tensor(k, "k", false) != CPATTN_OK) return 0;
  if (k->H < 1 || q->H % k->H != 0) {
    fail(CPATTN_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
    return 0;
  }
  if (n_chunks < 1 || n_chunks > cpattn::kMaxMerge || k->S % n_chunks != 0) {
    fail(CPATTN_ERR_INVALID_ARG, "n_chunks must be in [1, %d] and divide the KV length", cpattn::kMaxMerge);
    return 0;
  }
  ok();
  return decode_layout(*q, k->H, k->S / n_chunks, n_chunks).bytes;
}

cpattn_status cpattn_splitkv_decode(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                    int n_chunks, cpattn_tensor* out, cpattn_tensor* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  cpattn_status s;
  if ((s = check_decode(q, k, v, n_chunks)) != CPATTN_OK) return s;
  if ((s = check_out(out, lse, *q, true, false)) != CPATTN_OK) return s;
  if (q->B == 0) return ok();
  const int64_t C = k->S / n_chunks;
  const DecodeLayout L = decode_layout(*q, k->H, C, n_chunks);
  if ((s = check_workspace(workspace, workspace_bytes, L.bytes)) != CPATTN_OK) return s;
  const void* kc[cpattn::kMaxMerge];
  const void* vc[cpattn::kMaxMerge];
  int64_t len[cpattn::kMaxMerge];
  for (int c = 0; c < n_chunks; ++c) {
    kc[c] = static_cast<const __bf16*>(k->data) + c * C * k->stride_s;
    vc[c] = static_cast<const __bf16*>(v->data) + c * C * v->stride_s;
    len[c] = C;
  }
  return run_decode(*q, *k, *v, n_chunks, kc, vc, len, L, out, lse, workspace, static_cast<hipStream_t>(stream));
}

cpattn_status cpattn_splitkv_decode_noalloc(const cpattn_tensor* q, const cpattn_tensor* k, const cpattn_tensor* v,
                                            int n_chunks, cpattn_tensor* out, cpattn_tensor* lse, void* stream) {
  cpattn_status s;
  if ((s = check_decode(q, k, v, n_chunks)) != CPATTN_OK) return s;
  if ((s = check_out(out, lse, *q, true, false)) != CPATTN_OK) return s;
  const int64_t C = k->S / n_chunks;
  const DecodeLayout L = decode_layout(*q, k->H, C, n_chunks);
  if (L.bytes > cpattn::kScratchBytes)
    return fail(CPATTN_ERR_WORKSPACE, "this decode needs %zu bytes of scratch; the fixed scratch holds %zu "
                "(use cpattn_splitkv_decode with a workspace)", L.bytes, cpattn::kScratchBytes);
  if (q->B == 0) return ok();
  void* scratch = nullptr;
  const hipError_t e = cpattn::scratch_address(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
  const void* kc[cpattn::kMaxMerge];
  const void* vc[cpattn::kMaxMerge];
  int64_t len[cpattn::kMaxMerge];
  for (int c = 0; c < n_chunks; ++c) {
    kc[c] = static_cast<const __bf16*>(k->data) + c * C * k->stride_s;
    vc[c] = static_cast<const __bf16*>(v->data) + c * C * v->stride_s;
    len[c] = C;
  }
  return run_decode(*q, *k, *v, n_chunks, kc, vc, len, L, out, lse, scratch, static_cast<hipStream_t>(stream));
}

cpattn_status cpattn_kv_cache_write(const cpattn_tensor* k, const cpattn_tensor* v, int n_chunks,
                                    const cpattn_tensor* k_shards, const cpattn_tensor* v_shards, void* stream) {
  cpattn_status s;
  if ((s = check_tensor(k, "k", false)) != CPATTN_OK) return s;
  if ((s = check_tensor(v, "v", false)) != CPATTN_OK) return s;
  if (!same_bshd(*k, *v) || k->dtype != v->dtype) return fail(CPATTN_ERR_INVALID_ARG, "k and v differ in shape or dtype");
  if ((s = check_shards(k_shards, v_shards, n_chunks)) != CPATTN_OK) return s;
  if (k->S % n_chunks != 0)
    return fail(CPATTN_ERR_INVALID_ARG, "sequence length %lld not divisible by n_chunks %d", (long long)k->S, n_chunks);
  const cpattn_tensor& sh = k_shards[0];
  if (sh.dtype != k->dtype || sh.B != k->B || sh.H != k->H || sh.D != k->D)
    return fail(CPATTN_ERR_INVALID_ARG, "shards must match k/v in dtype, batch, heads and head_dim");
  const int64_t C = k->S / n_chunks;
  if (sh.S < C) return fail(CPATTN_ERR_INVALID_ARG, "shards hold %lld rows, a chunk has %lld", (long long)sh.S, (long long)C);
  if (C == 0 || k->B == 0 || k->H == 0) return ok();
  const int64_t eb = elem_bytes(k->dtype);
  // K and V in one launch when they share strides (as tensors of one shape
  // usually do) and their jobs fit; otherwise one launch each.
  const bool together = 2 * n_chunks <= cpattn::kMaxMerge && k->stride_b == v->stride_b &&
                        k->stride_s == v->stride_s && k->stride_h == v->stride_h &&
                        k_shards[0].stride_b == v_shards[0].stride_b && k_shards[0].stride_s == v_shards[0].stride_s &&
                        k_shards[0].stride_h == v_shards[0].stride_h;
  cpattn::CopyLaunch c;
  for (int t = 0; t < 2; ++t) {
    const cpattn_tensor& src = t == 0 ? *k : *v;
    const cpattn_tensor* dst = t == 0 ? k_shards : v_shards;
    if (t == 0 || !together) {
      std::memset(&c, 0, sizeof c);
      c.elem_bytes = (int32_t)eb;
      c.B = (int32_t)src.B; c.rows = (int32_t)C; c.H = (int32_t)src.H; c.D = (int32_t)src.D;
      c.s_sb = src.stride_b; c.s_ss = src.stride_s; c.s_sh = src.stride_h;
      c.d_sb = dst[0].stride_b; c.d_ss = dst[0].stride_s; c.d_sh = dst[0].stride_h;
    }
    for (int r = 0; r < n_chunks; ++r) {
      c.src[c.n_jobs] = static_cast<const char*>(src.data) + r * C * src.stride_s * eb;
      c.dst[c.n_jobs] = dst[r].data;
      ++c.n_jobs;
    }
    if (t == 1 || !together) {
      const hipError_t e = cpattn::launch_copy(c, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, "cache write launch");
    }
  }
  return ok();
}

cpattn_status cpattn_kv_cache_append(const cpattn_tensor* k_new, const cpattn_tensor* v_new,
                                     const cpattn_tensor* k_shard, const cpattn_tensor* v_shard, int64_t row,
                                     void* stream) {
  cpattn_status s;
  if ((s = check_tensor(k_new, "k_new", false)) != CPATTN_OK) return s;
  if ((s = check_tensor(v_new, "v_new", false)) != CPATTN_OK) return s;
  if (!same_bshd(*k_new, *v_new) || k_new->dtype != v_new->dtype)
    return fail(CPATTN_ERR_INVALID_ARG, "k_new and v_new differ in shape or dtype");
  if ((s = check_shards(k_shard, v_shard, 1)) != CPATTN_OK) return s;
  if (k_shard->dtype != k_new->dtype || k_shard->B != k_new->B || k_shard->H != k_new->H || k_shard->D != k_new->D)
    return fail(CPATTN_ERR_INVALID_ARG, "the shard must match the new rows in dtype, batch, heads and head_dim");
  if (row < 0 || row + k_new->S > k_shard->S)
    return fail(CPATTN_ERR_INVALID_ARG, "rows [%lld, %lld) do not fit a shard of %lld rows", (long long)row,
                (long long)(row + k_new->S), (long long)k_shard->S);
  if (k_new->S == 0 || k_new->B == 0 || k_new->H == 0) return ok();
  const int64_t eb = elem_bytes(k_new->dtype);
  for (int t = 0; t < 2; ++t) {
    const cpattn_tensor& src = t == 0 ? *k_new : *v_new;
    const cpattn_tensor& dst = t == 0 ? *k_shard : *v_shard;
    cpattn::CopyLaunch c;
    std::memset(&c, 0, sizeof c);
    c.n_jobs = 1;
    c.elem_bytes = (int32_t)eb;
    c.B = (int32_t)src.B; c.rows = (int32_t)src.S; c.H = (int32_t)src.H; c.D = (int32_t)src.D;
    c.s_sb = src.stride_b; c.s_ss = src.stride_s; c.s_sh = src.stride_h;
    c.d_sb = dst.stride_b; c.d_ss = dst.stride_s; c.d_sh = dst.stride_h;
    c.src[0] = src.data;
    c.dst[0] = static_cast<char*>(dst.data) + row * dst.stride_s * eb;
    const hipError_t e = cpattn::launch_copy(c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "cache append launch");
  }
  return ok();
}

size_t cpattn_cp_decode_workspace_size(const cpattn_tensor* q, const cpattn_tensor* k_shards, int n_shards) {
  if (check_tensor(q, "q", false) != CPATTN_OK) return 0;
  if (k_shards == nullptr || n_shards < 1 || n_shards > cpattn::kMaxMerge) {
    fail(CPATTN_ERR_INVALID_ARG, "need 1 to %d shard descriptors", cpattn::kMaxMerge);
    return 0;
  }
  if (check_tensor(&k_shards[0], "k shard", false) != CPATTN_OK) return 0;
  if (k_shards[0].H < 1 || q->H % k_shards[0].H != 0) {
    fail(CPATTN_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
    return 0;
  }
  ok();
  return decode_layout(*q, k_shards[0].H, k_shards[0].S, n_shards).bytes;
}

cpattn_status cpattn_cp_decode(const cpattn_tensor* q, const cpattn_tensor* k_shards, const cpattn_tensor* v_shards,
                               const int64_t* shard_len, int n_shards, cpattn_tensor* out, cpattn_tensor* lse,
                               void* workspace, size_t workspace_bytes, void* stream) {
  cpattn_status s;
  if ((s = check_shards(k_shards, v_shards, n_shards)) != CPATTN_OK) return s;
  if ((s = check_decode(q, &k_shards[0], &v_shards[0], 1)) != CPATTN_OK) return s;
  if (shard_len == nullptr) return fail(CPATTN_ERR_INVALID_ARG, "shard_len is NULL");
  for (int r = 0; r < n_shards; ++r)
    if (shard_len[r] < 0 || shard_len[r] > k_shards[0].S)
      return fail(CPATTN_ERR_INVALID_ARG, "shard %d: length %lld outside [0, %lld]", r, (long long)shard_len[r],
                  (long long)k_shards[0].S);
  if ((s = check_out(out, lse, *q, true, false)) != CPATTN_OK) return s;
  if (q->B == 0) return ok();
  const DecodeLayout L = decode_layout(*q, k_shards[0].H, k_shards[0].S, n_shards);
  if ((s = check_workspace(workspace, workspace_bytes, L.bytes)) != CPATTN_OK) return s;
  const void* kc[cpattn::kMaxMerge];
  const void* vc[cpattn::kMaxMerge];
  for (int r = 0; r < n_shards; ++r) {
    kc[r] = k_shards[r].data;
    vc[r] = v_shards[r].data;
  }
  return run_decode(*q, k_shards[0], v_shards[0], n_shards, kc, vc, shard_len, L, out, lse, workspace,
                    static_cast<hipStream_t>(stream));
}

}  // extern "C"
