// Row copies into KV-cache shards.
//
// The prefill constructs the KV cache of every layer and decode reads (and
// extends) it ("Scaling LLM Inference", techreport.ngo rewrite, "Why
// Parallelism Defines LLM Serving Cost"); with the sequence cut across CP
// ranks, each rank's shard of the cache holds its own chunk's K/V.  These
// copies put a prefill's chunks into their shards and append new tokens.
//
// Bandwidth bound.  When every batch row's [rows, H, D] block is contiguous
// on both sides (the usual layout), each (job, batch row) is one flat run of
// 16-byte pieces, four per thread with every load issued before any store;
// otherwise one thread per 16-byte piece, consecutive threads on consecutive
// pieces of a [H, D] token row.  Every byte is read once and written once, so
// both sides carry the non-temporal hint (the decode workload's 2 GiB of K/V
// into 8 shards: 0.91 -> 0.80 ms).
#include "device.h"
#include "internal.h"

namespace cpattn {
namespace {

__global__ __launch_bounds__(256) void copy_rows_kernel(const CopyLaunch a, const int64_t pieces_per_job) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = pieces_per_job * a.n_jobs;
  if (t >= total) return;
  const int job = (int)(t / pieces_per_job);
  int64_t r = t - job * pieces_per_job;
  const int ppr = a.D * a.elem_bytes / 16;  // pieces per (token, head) row
  const int pc = (int)(r % ppr);
  r /= ppr;
  const int h = (int)(r % a.H);
  r /= a.H;
  const int64_t s = r % a.rows;
  const int64_t b = r / a.rows;
  const int64_t e_per_piece = 16 / a.elem_bytes;
  const int64_t so = b * a.s_sb + s * a.s_ss + h * a.s_sh + pc * e_per_piece;
  const int64_t dof = b * a.d_sb + s * a.d_ss + h * a.d_sh + pc * e_per_piece;
  const uint8_t* src = static_cast<const uint8_t*>(a.src[job]) + so * a.elem_bytes;
  uint8_t* dst = static_cast<uint8_t*>(a.dst[job]) + dof * a.elem_bytes;
  __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src)),
                              reinterpret_cast<u32x4*>(dst));
}

// Flat runs: blockIdx.y = job * B + batch row, n16 pieces per run, 1024 per
// workgroup.
__global__ __launch_bounds__(256) void copy_flat_kernel(const CopyLaunch a, const uint32_t n16) {
  const int job = (int)blockIdx.y / a.B;
  const int b = (int)blockIdx.y - job * a.B;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.src[job]) +
                                                    (int64_t)b * a.s_sb * a.elem_bytes);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.dst[job]) + (int64_t)b * a.d_sb * a.elem_bytes);
  const uint32_t i0 = blockIdx.x * 1024u + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + 256u * u < n16) v[u] = __builtin_nontemporal_load(src + i0 + 256u * u);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (i0 + 256u * u < n16) __builtin_nontemporal_store(v[u], dst + i0 + 256u * u);
}

}  // namespace

hipError_t launch_copy(const CopyLaunch& a, hipStream_t s) {
  const long long per_job = (long long)a.B * a.rows * a.H * (a.D * a.elem_bytes / 16);
  const long long total = per_job * a.n_jobs;
  if (total <= 0) return hipSuccess;
  const long long run = (long long)a.rows * a.H * (a.D * a.elem_bytes / 16);  // pieces per (job, batch row)
  const bool flat = a.s_sh == a.D && a.s_ss == (int64_t)a.H * a.D && a.d_sh == a.D && a.d_ss == (int64_t)a.H * a.D;
  if (flat && run < 0xffffffffLL - 1024 && (long long)a.n_jobs * a.B <= 65535) {
    hipLaunchKernelGGL(copy_flat_kernel, dim3((unsigned)((run + 1023) / 1024), (unsigned)(a.n_jobs * a.B)), dim3(256), 0,
                       s, a, (uint32_t)run);
    return hipGetLastError();
  }
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, (int64_t)per_job);
  return hipGetLastError();
}

}  // namespace cpattn
