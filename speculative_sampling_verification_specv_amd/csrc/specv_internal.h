// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;      // threads per workgroup (4 wave64s)
constexpr int kStatBytes = 65536;  // row-statistics item: 64 KB of one row, either dtype

// A draw member covers 4096 logits of each row it reads (16 per thread),
// split into kSubs sub-chunks of 32 consecutive threads.
constexpr int kMemberElems = 4096;
inline int member_elems(int) { return kMemberElems; }
constexpr int kSubs = 8;
constexpr int kUncMax = 8;  // uncertain-sign tokens a member record lists

// Largest vocabulary a handle accepts, so a sequence's members fit one per
// lane of a wave in the finisher.
constexpr int kMaxVocab = 1 << 18;
constexpr int kMaxMembers = kMaxVocab / kMemberElems;

// Smallest positive temperature accepted: keeps log2(e)/T and max|z|*log2(e)/T
// finite in fp32 for logits up to 2^64 in magnitude.
constexpr float kMinTemperature = 0x1p-60f;

inline int stat_chunk_elems(int dtype) { return kStatBytes / (dtype == 0 ? 4 : 2); }

// Acceptance-rate item: 32 KB of a draft row and the same span of its target
// row (both in flight at once: 16 16-byte loads per thread).
constexpr int kRateBytes = 32768;
inline int rate_chunk_elems(int dtype) { return kRateBytes / (dtype == 0 ? 4 : 2); }

constexpr int kCounterStride = 64;

// A lazy call verifies positions in stages [0,2), [2,2g), [2g,2g^2), ...
// (each stage's decision ends the sequences it rejects or completes, so
// later stages read the rows of fewer sequences; each stage also adds a
// decision to the chain). Growth g = 4 unless one position of the batch (its
// draft and target rows) is at least 96 MB, where the rows a finer stage
// saves outweigh the chain: then g = 2. (Measured: g = 4 best at B = 64,
// V = 128256 bf16 and level at B = 32, N = 16 fp32; g = 2 about 10 us faster
// at B = 256, V = 151936 bf16.) Writes bounds[0..k] and returns the number of
// stages k (at most kMaxLazyStages for n_draft <= 64).
constexpr int kMaxLazyStages = 6;
inline int lazy_growth(int batch, int vocab, int dtype) {
  return int64_t(batch) * vocab * (dtype == 0 ? 4 : 2) * 2 >= int64_t(96000000) ? 2 : 4;
}
inline int lazy_stage_bounds(int n_draft, int growth, int* bounds) {
  int k = 0, lo = 0;
  bounds[0] = 0;
  while (lo < n_draft && k < kMaxLazyStages) {
    const int hi = lo == 0 ? (n_draft < 2 ? n_draft : 2) : (n_draft < growth * lo ? n_draft : growth * lo);
    bounds[++k] = hi;
    lo = hi;
  }
  return k;
}

// What a sampled sequence's draw does: a residual or bonus draw, nothing because an
// input is invalid (-1 outputs), or nothing because a wait gave up (-2 outputs).
enum SeqMode : int {
  kModeNone = 0,
  kModeResidual = 1,
  kModeBonus = 2,
  kModeInvalid = 3,
  kModeFailed = 4
};

// Device workspace: records one launch writes and the next reads.
struct Workspace {
  void* partials;    // [max_batch][2*max_draft+1][n_stat_chunks] row-statistics partials
  void* seq;         // [max_batch] decisions
  void* records;     // [max_batch][n_members] draw-member records
  double* row_lse;   // [batch][2N+1] of the last call (fp64; NaN for rows not read)
  int* row_argmax;   // [batch][2N+1] of the last call
  // Per sequence, how many draw members of a launch are done with it; the
  // last one resets its count to zero. Zero between calls. One counter per
  // kCounterStride ints (its own 256-byte line), so that atomics on different
  // sequences' counters never contend for a line.
  int* draw_done;    // [max_batch * kCounterStride]
  double* rate_parts;  // [max_batch][max_draft][n_rate_chunks] acceptance-rate partial sums (handles only)
  uint64_t* alive;     // [max_batch][(2*max_draft+1)*n_stat_chunks + kMaxLazyStages] lazy calls' go-on words (handles only)
  int n_stat_chunks;
  int n_rate_chunks;
  int resident_blocks;  // workgroups of the verification kernel the device holds at once
  int n_members;     // draw members per sequence
  int stat_chunk;    // logits per row-statistics item
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
  uint32_t tag;         // the call's number (never 0), carried by every hand-off word
  uint32_t debug;       // also check that the uniforms lie in [0, 1)
  uint64_t wait_ticks;  // bound of every wait between workgroups, in wall-clock ticks
  // Nonzero: the lazy verification (stages of positions, one launch).
  int lazy = 0;
  // Nonzero: a sampling call (n_draft = 0; draw members only, see Params).
  int sample = 0;
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

constexpr int kMaxStages = 8;


// Workgroups of the verification kernel for `dtype` the current device holds
// at once (-1 on a HIP error).
int max_resident_blocks(int dtype);

// Names of the kernel stages launch_verify enqueues, in order.
const char* stage_name(int stage);

// Record sizes (bytes) the workspace must hold per unit: per row-statistics
// item, per sequence, per draw member.
size_t partial_bytes();
size_t seq_bytes();
size_t member_bytes();

struct RatesArgs {
  int batch;
  int n_draft;
  int vocab;
  int dtype;  // specv_dtype
  const void* draft;
  const void* target;
  const int* tokens;
  const float* temperature;
  float* out_alpha;  // [batch][n_draft]
  float* out_tau;    // [batch]
};

// Enqueue the acceptance-rate passes on `stream`; they read the row
// log-normalisers and argmaxes the last verification left in `w`.
hipError_t launch_rates(const RatesArgs& a, const Workspace& w, hipStream_t stream);

// Enqueue the whole verification on `stream`. If `events` is non-null it holds
// kMaxStages + 1 events: events[k] is recorded before stage k and
// events[*n_stages] after the last stage.
hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* events,
                         int* n_stages);

}  // namespace specv
