// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;       // threads per workgroup (4 wave64s)
constexpr int kStatsChunk = 8192;   // logits per row-statistics work item
constexpr int kSampChunk = 4096;    // logits per sampler work item
constexpr int kDecideThreads = 64;  // one wave64 per sequence decides

// Partial statistics of one (row, chunk): m = largest raw logit, s = sum of
// 2^((z - m) * c) with c = log2(e) / T, idx = first index attaining m.
struct RowPartial {
  float m;
  float s;
  int idx;
  int pad;
};

enum SeqMode : int { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// What the decision left for the sampler of one sequence.
struct SeqState {
  int mode;        // SeqMode
  int j;           // first rejected position, or N when all were accepted
  float m_target;  // largest raw logit of the target row drawn from
  float m_draft;   // largest raw logit of draft row j (residual only)
  double inv_t;    // 1 / T in fp64
};

struct Workspace {
  RowPartial* partials;  // [max_batch * (2*max_draft+1)][n_stats_chunks]
  float* row_lse;        // [batch][2N+1] of the last call
  int* row_argmax;       // [batch][2N+1] of the last call
  SeqState* seq;         // [max_batch]
  double2* norm_part;    // [max_batch][n_samp_chunks]: fp64 sums of exp((z - m)/T), target and draft
  double* wsum_part;     // [max_batch][n_samp_chunks]: fp64 sums of the draw's weights
  int n_stats_chunks;
  int n_samp_chunks;
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
