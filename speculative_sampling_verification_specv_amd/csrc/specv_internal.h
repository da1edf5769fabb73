// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;            // threads per workgroup (4 wave64s)
constexpr int kStatsChunkBytes = 32768;  // row-statistics item: 32 KB of logits of either dtype
constexpr int kSampChunk = 4096;         // logits per draw-chunk item
constexpr int kUncMax = 16;              // uncertain-sign tokens one draw chunk records

// Largest vocabulary a handle accepts, so a sequence's draw chunks fit in LDS.
constexpr int kMaxVocab = 1 << 22;
constexpr int kMaxSampChunks = kMaxVocab / kSampChunk;

// Smallest positive temperature accepted: keeps log2(e)/T and max|z|*log2(e)/T
// finite in fp32 for logits up to 2^64 in magnitude.
constexpr float kMinTemperature = 0x1p-60f;

inline int stats_chunk_elems(int dtype) { return kStatsChunkBytes / (dtype == 0 ? 4 : 2); }

enum SeqMode : int { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Row statistics of one (row, chunk): m = largest logit, s = sum of
// 2^(z*c - fl(m*c)) with c = log2(e)/T, idx = first index attaining m.
struct RowPartial {
  float m;
  float s;
  int idx;
  int pad;
};

// What the decision leaves for the draw of one sequence.
struct SeqRecord {
  int mode;  // SeqMode
  int j;     // first rejected position, or N when all were accepted
  float m_target;
  float m_draft;
  double log_rho;  // log(Zt/Zd) of row j from the fp32 row sums (residual only)
  double pad;
};

// fp64 sums of one draw chunk. After a rejection: zt, zd = sums of
// exp((z - max)/T) over target and draft row j; a, b = the same over the tokens
// whose residual weight is certainly positive; n_unc tokens of uncertain sign
// (listed in idx when n_unc <= kUncMax). For the bonus only zt is used.
struct NormRecord {
  double zt, zd, a, b;
  int n_unc;
  int idx[kUncMax];
  int pad;
};

struct Workspace {
  RowPartial* partials;  // [max_batch * (2*max_draft+1)][n_stats_chunks]
  SeqRecord* seq;        // [max_batch]
  NormRecord* norm;      // [max_batch][n_samp_chunks]
  double* exp_table;     // [64]: 2^(j/64)
  float* row_lse;        // [batch][2N+1] of the last call
  int* row_argmax;       // [batch][2N+1] of the last call
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

}  // namespace specv
