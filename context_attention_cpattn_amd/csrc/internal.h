// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/cpattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

constexpr int kMaxItems = 160;  // partial-attention work items per launch (kernel argument ~2.8 KB)
constexpr int kMaxMerge = 64;   // partials per merge launch (CPATTN_MAX_MERGE)
static_assert(kMaxMerge <= kMaxItems, "the pairs of one ring step (at most kMaxMerge) fit one launch");

// One (Q block, K/V block) pair of a launch.  Pointers are derived from the
// launch's base pointers: Q rows start at q_chunk * chunk_len, K/V rows at
// kv_chunk * kv_chunk_len, and the outputs go to slot `slot` of the output base.
struct Item {
  int32_t q_chunk;
  int32_t kv_chunk;
  int32_t slot;
  int32_t sk;  // keys of this item's K/V block; 0 = the launch's Sk
};

struct PartialLaunch {
  const void* q;  // element type: bf16 or float, per the launcher
  const void* k;
  const void* v;
  float* o;
  float* lse;     // may be null (no LSE wanted)
  int64_t q_sb, q_ss, q_sh;  // element strides
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int64_t l_sb, l_ss, l_sh;
  int64_t o_slot, l_slot;    // element distance between output slots
  int64_t q_pos0, kv_pos0;   // global position of row 0 of chunk 0
  int64_t chunk_len;         // Q rows per chunk (used only to derive item pointers)
  int64_t kv_chunk_len;      // K/V rows per chunk
  int32_t B, Sq, Sk, Hq, G;  // Sq/Sk: rows of one Q/K/V block; G = Hq / Hkv
  int32_t causal;
  int32_t n_items;
  int32_t xcd_order;  // 1: each XCD takes a contiguous share of the grid; 0: launch order
  int32_t accumulate; // 1: merge into the (O, LSE) already at the destination (lse not null; no segments)
  int32_t head_pack_log2;  // bf16 kernel: a workgroup takes 2^this heads of one K/V head (launcher sets it)
  int32_t seg_tiles;  // > 0: an item's keys form segments of this many 64-key tiles, each one
                      // written as its own partial to slot item.slot + segment (D = 128 BF16)
  // With segments and final_out set, each query tile also merges its segments'
  // partials once its walk is done, in the ring order's arrival order (pass_q),
  // into row item.q_chunk * chunk_len + row of final_out (and final_lse).
  void* final_out;
  int32_t final_bf16, pass_q;
  int64_t f_sb, f_ss, f_sh;
  float* final_lse;           // may be null
  int64_t fl_sb, fl_ss, fl_sh;
  Item items[kMaxItems];
};

struct MergeLaunch {
  const float* o[kMaxMerge];
  const float* lse[kMaxMerge];
  int32_t n;
  int32_t out_bf16;
  int32_t B, S, H, D;
  int64_t p_sb, p_ss, p_sh;   // partial O strides (shared)
  int64_t pl_sb, pl_ss, pl_sh;  // partial LSE strides (shared)
  void* out;
  int64_t o_sb, o_ss, o_sh;
  float* out_lse;             // may be null
  int64_t ol_sb, ol_ss, ol_sh;
};

// Merge of a ring's workspace slots into the final output: every owner i
// merges its partials in the ring order's arrival order (computed in the
// kernel), all owners in one launch.  Owner i sees K/V chunks [0, n_vis[i])
// and its pair with K/V chunk j sits in slot slot0[i] + j.
struct RingMergeLaunch {
  const float* ws_o;          // slot t: O [B][C][H][D] at ws_o + t * slot_o
  const float* ws_l;          // slot t: LSE [B][C][H] at ws_l + t * slot_l
  int64_t slot_o, slot_l;
  int32_t P, C, B, H, D;      // C: query rows per chunk
  int32_t pass_q;             // ring order: 0 = Pass-KV, 1 = Pass-Q
  int32_t out_bf16;
  void* out;                  // [B][P*C][H][D]
  int64_t o_sb, o_ss, o_sh;
  float* out_lse;             // may be null
  int64_t ol_sb, ol_ss, ol_sh;
  int32_t n_vis[kMaxMerge];
  int32_t slot0[kMaxMerge];
};

// Split-KV decode over n_chunks K/V blocks, each at its own base pointer (the
// chunks of one cache, or the shards of a cache cut across CP ranks); every
// block shares the element strides below.
struct DecodeLaunch {
  const void* q;  // bf16 [B, 1, Hq, D]
  float* o;       // partial p, batch b, head h at o + p*o_slot + b*o_sb + h*o_sh (D contiguous)
  float* lse;     // partial LSE at lse + p*l_slot + b*l_sb + h*l_sh
  int64_t o_slot, o_sb, o_sh;
  int64_t l_slot, l_sb, l_sh;
  int64_t q_sb, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int32_t B, Hq, Hkv, G;
  int32_t n_chunks, n_split;  // partial p = chunk * n_split + split
  int32_t split_len;          // keys per split (multiple of 32, last split may be shorter)
  int32_t head_blocks;        // ceil(G / 16)
  const void* kc[kMaxMerge];  // bf16 block c: [B, len[c], Hkv, D] at kc[c] / vc[c]
  const void* vc[kMaxMerge];
  int32_t len[kMaxMerge];
};

// Row copies between [B, S, H, D] views of one dtype: job j copies rows
// [0, rows) of src[j] to dst[j]; all jobs share the strides.
struct CopyLaunch {
  const void* src[kMaxMerge];
  void* dst[kMaxMerge];
  int32_t n_jobs;
  int32_t elem_bytes;
  int32_t B, rows, H, D;
  int64_t s_sb, s_ss, s_sh;  // element strides
  int64_t d_sb, d_ss, d_sh;
};

// Launchers return hipSuccess or the launch error.
hipError_t launch_partial_bf16(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s);
hipError_t launch_partial_f32(const PartialLaunch& a, int D, int n_qtiles, hipStream_t s);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t s);
hipError_t launch_ring_merge(const RingMergeLaunch& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeLaunch& a, int D, hipStream_t s);
hipError_t launch_copy(const CopyLaunch& a, hipStream_t s);

hipError_t cu_count(int* out);  // compute units of the current device (cached, thread-safe)

// The fixed scratch of cpattn_splitkv_decode_noalloc: kScratchBytes of device
// memory per GPU, its device address looked up once per device (thread-safe).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void** out);

int partial_bf16_rows_per_block(int D);  // query rows per workgroup of the bf16 kernel
// log2 of the query heads a bf16 workgroup takes: 1, 2 or 3 when query blocks of
// at most 128, 64 or 32 rows leave room and the heads of a K/V group allow it
int partial_bf16_head_pack_log2(int Sq, int G);
int partial_f32_rows_per_block(int D);

}  // namespace cpattn
