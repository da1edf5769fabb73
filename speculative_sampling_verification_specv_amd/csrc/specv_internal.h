// Internal interface between the C-ABI host code and the gfx950 kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;      // threads per workgroup (4 wave64s)
constexpr int kStatsChunk = 8192;  // logits per row-statistics work item
constexpr int kSampChunk = 4096;   // logits per draw (NORM) work item

// Largest vocabulary a handle accepts, so a sequence's draw chunks fit in LDS.
constexpr int kMaxVocab = 1 << 22;
constexpr int kMaxSampChunks = kMaxVocab / kSampChunk;

// Smallest positive temperature accepted: keeps log2(e)/T and max|z|*log2(e)/T
// finite in fp32 for logits up to 2^64 in magnitude.
constexpr float kMinTemperature = 0x1p-60f;

// Largest call epoch before the tagged words are cleared and numbering restarts.
constexpr unsigned kMaxEpoch = 0xffffu;

enum SeqMode : int { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Scratch device memory owned by a handle. Every word is 64 bits: a 48-bit
// payload and the 16-bit epoch of the call that wrote it.
struct Workspace {
  uint64_t* stat_words;  // [max_batch * (2*max_draft+1)][n_stats_chunks][2]
  uint64_t* seq_words;   // [max_batch][seq_words_per_sequence()]
  uint64_t* norm_words;  // [max_batch][n_samp_chunks][norm_words_per_chunk()]
  long long n_words;     // total words, all three arrays (contiguous from stat_words)
  double* exp_table;     // [64]: 2^(j/64)
  float* row_lse;        // [batch][2N+1] of the last call
  int* row_argmax;       // [batch][2N+1] of the last call
  int n_stats_chunks;
  int n_samp_chunks;
#ifdef SPECV_TRACE
  unsigned long long* trace;  // per-slot item records (diagnostic builds only)
  long long trace_slots;
#endif
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
};

// Per-call launch parameters chosen by the host.
struct LaunchConfig {
  long long max_blocks;              // persistent grid cap
  int lag_decide;                    // item groups (sequences) between STAT(b) and DECIDE(b)
  int lag_norm;                      // ... and NORM(b, *)
  int lag_draw;                      // ... and DRAW(b)
  unsigned epoch;                    // 1..kMaxEpoch
  unsigned long long timeout_ticks;  // wall-clock ticks a wait lasts before it computes the item itself
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kMaxStages = 8;

// Names of the kernel stages launch_verify enqueues, in order.
const char* stage_name(int stage);

// Workgroups of the verify kernel one CU can hold.
int max_blocks_per_cu(int dtype);

// Tagged words per draw chunk and per sequence.
int norm_words_per_chunk();
int seq_words_per_sequence();

// Zero n words (epoch 0 is never used, so cleared words read as stale).
hipError_t clear_words(uint64_t* p, long long n, hipStream_t stream);

// Enqueue the whole verification on `stream`. If `events` is non-null it holds
// kMaxStages + 1 events: events[k] is recorded before stage k and
// events[*n_stages] after the last stage.
hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, const LaunchConfig& cfg, hipStream_t stream,
                         hipEvent_t* events, int* n_stages);

}  // namespace specv
