// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;            // threads per workgroup (4 wave64s)
constexpr int kStatsChunkBytes = 65536;  // row-statistics item: 64 KB of logits of either dtype
constexpr int kSampChunk = 2048;         // logits per draw-chunk item
constexpr int kUncMax = 4;               // uncertain-sign tokens one draw chunk records

// Largest vocabulary a handle accepts, so a sequence's draw chunks fit in LDS.
constexpr int kMaxVocab = 1 << 19;
constexpr int kMaxSampChunks = kMaxVocab / kSampChunk;

// Smallest positive temperature accepted: keeps log2(e)/T and max|z|*log2(e)/T
// finite in fp32 for logits up to 2^64 in magnitude.
constexpr float kMinTemperature = 0x1p-60f;

inline int stats_chunk_elems(int dtype) { return kStatsChunkBytes / (dtype == 0 ? 4 : 2); }

enum SeqMode : int { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Records passed between workgroups, in 64-bit words whose high half holds
// the call's sequence number (see specv_kernels.hip).
constexpr int kPartWords = 4;                        // one (row, chunk) partial
constexpr int kSeqWords = 8;                         // one sequence's decision
constexpr int kNormWords = 32;                       // one draw chunk's sums (256 bytes)

struct Workspace {
  uint64_t* partials;  // [max_batch * (2*max_draft+1)][n_stats_chunks][kPartWords]
  uint64_t* seq;       // [max_batch][kSeqWords]
  uint64_t* norm;      // [max_batch][n_samp_chunks][kNormWords]
  double* exp_table;   // [64]: 2^(j/64)
  float* row_lse;      // [batch][2N+1] of the last call
  int* row_argmax;     // [batch][2N+1] of the last call
  int n_stats_chunks;
  int n_samp_chunks;
  int stats_chunk;  // logits per row-statistics item
};

struct VerifyArgs {
  int batch;
  int n_draft;
  int vocab;
  int dtype;  // specv_dtype
  const void* draft;
  const void* target;
  const int* tokens;
  const float* accept_u;
  const float* sample_u;
  const float* temperature;
  int* out_tokens;
  int* out_n;
  uint32_t epoch;       // nonzero, different from the previous call's
  uint64_t wait_ticks;  // bound on in-kernel waits (100 MHz ticks)
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kMaxStages = 8;

// Names of the kernel stages launch_verify enqueues, in order.
const char* stage_name(int stage);

// Enqueue the whole verification on `stream`. If `events` is non-null it holds
// kMaxStages + 1 events: events[k] is recorded before stage k and
// events[*n_stages] after the last stage.
hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* events,
                         int* n_stages);

// Workgroups one launch uses (the grid must stay below 2^31).
int64_t grid_blocks(int batch, int n_draft, int n_stats_chunks, int n_samp_chunks);

// Zero `bytes` (a multiple of 16) of device memory on `stream` with a kernel.
hipError_t clear_records(void* mem, size_t bytes, hipStream_t stream);

}  // namespace specv
