// gfx950 kernel for the KV-cache commit after a verification.
//
// Lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com), section
// "KV 캐시 처리(KV cache dance)": the verifier's pass over N drafts writes their
// KV entries into a scratch area; once n of them are accepted, entries
// 0..n-1 are committed to the sequence's cache at its current length and the
// rest are dropped, so the next pass reads the prefix and the accepted drafts
// only (the lesson's exercise 4 checks exactly that).
//
// One workgroup per (plane, sequence): its threads copy that sequence's n
// accepted entries of that plane, 16 bytes per thread per step, from scratch
// to cache. Bandwidth-bound: 2 * n * entry_bytes per (plane, sequence).

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "specv.h"

namespace {

constexpr int kThreads = 256;

struct KvParams {
  uint8_t* cache;
  const uint8_t* scratch;
  const int32_t* n_accepted;
  const int32_t* cache_len;
  int32_t* out_len;
  int64_t cache_plane_stride, cache_seq_stride;
  int64_t scratch_plane_stride, scratch_seq_stride;
  int64_t words;  // 16-byte words per entry
  int n_planes, batch, n_draft, max_len;
};

// n accepted entries of sequence b if they can be committed, else -1.
__device__ __forceinline__ int committed(const KvParams& P, int b, int& start) {
  const int n = P.n_accepted[b];
  start = P.cache_len[b];
  if (n < 0 || n > P.n_draft || start < 0 || int64_t(start) + n > P.max_len) return -1;
  return n;
}

__global__ __launch_bounds__(kThreads) void kv_commit_kernel(KvParams P) {
  const int b = int(blockIdx.x % unsigned(P.batch));
  const int p = int(blockIdx.x / unsigned(P.batch));
  int start = 0;
  const int n = committed(P, b, start);
  if (p == 0 && threadIdx.x == 0) P.out_len[b] = n < 0 ? -1 : start + n;
  if (n <= 0 || p >= P.n_planes) return;
  const uint4* __restrict__ src =
      reinterpret_cast<const uint4*>(P.scratch + p * P.scratch_plane_stride + b * P.scratch_seq_stride);
  uint4* __restrict__ dst = reinterpret_cast<uint4*>(P.cache + p * P.cache_plane_stride + b * P.cache_seq_stride) +
                            int64_t(start) * P.words;
  // The n entries are contiguous in both areas: one run of n * words words.
  const int64_t total = int64_t(n) * P.words;
  for (int64_t i = threadIdx.x; i < total; i += kThreads) dst[i] = src[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" SPECV_API int specv_kv_commit(int n_planes, int batch, int n_draft, int max_len, int64_t entry_bytes,
                                         void* cache, int64_t cache_plane_stride, int64_t cache_seq_stride,
                                         const void* scratch, int64_t scratch_plane_stride,
                                         int64_t scratch_seq_stride, const int32_t* n_accepted,
                                         const int32_t* cache_len, int32_t* out_cache_len, void* stream) {
  if (n_planes < 0 || batch < 0 || n_draft < 1 || max_len < 0 || entry_bytes < 16) return SPECV_EINVAL;
  if (batch == 0) return SPECV_OK;
  if (!n_accepted || !cache_len || !out_cache_len) return SPECV_EINVAL;
  if (n_planes > 0 && (!cache || !scratch)) return SPECV_EINVAL;
  if (entry_bytes % 16 || cache_plane_stride % 16 || cache_seq_stride % 16 || scratch_plane_stride % 16 ||
      scratch_seq_stride % 16)
    return SPECV_EALIGN;
  if ((n_planes > 0 && (!aligned16(cache) || !aligned16(scratch))) ||
      (reinterpret_cast<uintptr_t>(n_accepted) & 3u) || (reinterpret_cast<uintptr_t>(cache_len) & 3u) ||
      (reinterpret_cast<uintptr_t>(out_cache_len) & 3u))
    return SPECV_EALIGN;
  const int64_t blocks = int64_t(batch) * (n_planes > 0 ? n_planes : 1);
  if (blocks >= (int64_t(1) << 31)) return SPECV_EINVAL;
  KvParams P;
  P.cache = static_cast<uint8_t*>(cache);
  P.scratch = static_cast<const uint8_t*>(scratch);
  P.n_accepted = n_accepted;
  P.cache_len = cache_len;
  P.out_len = out_cache_len;
  P.cache_plane_stride = cache_plane_stride;
  P.cache_seq_stride = cache_seq_stride;
  P.scratch_plane_stride = scratch_plane_stride;
  P.scratch_seq_stride = scratch_seq_stride;
  P.words = entry_bytes / 16;
  P.n_planes = n_planes;
  P.batch = batch;
  P.n_draft = n_draft;
  P.max_len = max_len;
  hipLaunchKernelGGL(kv_commit_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, static_cast<hipStream_t>(stream), P);
  return hipGetLastError() == hipSuccess ? SPECV_OK : SPECV_EHIP;
}
