// C-ABI host side of libspecv: handle, workspace, argument checks, launches.
// The public contract (layouts, ownership, errors) is in include/specv.h.

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>
#include <vector>

#include "specv.h"
#include "specv_internal.h"
#include "specv_math.h"

struct specv_ctx {
  int device;
  int max_batch;
  int max_draft;
  int vocab;
  int dtype;
  void* mem;  // one device allocation holding the whole workspace
  size_t mem_bytes;
  specv::Workspace ws;
  int last_batch;        // -1 until a verify succeeds
  int last_n_draft;
  uint32_t next_tag;     // number of the next call (1, 2, ...; 0 is skipped)
  uint32_t debug;        // SPECV_DEBUG was set at create: check the uniforms on the device
  uint64_t wait_ticks;   // bound of every wait between workgroups, in wall-clock ticks
  int clock_khz;         // the device's wall-clock rate
  bool timing;                               // record stage events on every verify
  bool timed_call;                           // the last verify recorded them
  int timed_stages;                          // stages the last timed verify launched
  hipEvent_t events[specv::kMaxStages + 1];  // created on first enable
  bool events_created;
};

namespace {

// Makes `device` current for the lifetime of the guard and restores the caller's.
class DeviceGuard {
 public:
  explicit DeviceGuard(int device) {
    ok_ = hipGetDevice(&prev_) == hipSuccess;
    if (ok_ && prev_ != device) ok_ = hipSetDevice(device) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
  }
  bool ok() const { return ok_; }

 private:
  int prev_ = 0;
  bool ok_ = false;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Default bound of a wait between the workgroups of one launch (a normal
// wait lasts microseconds; the bound only matters if the device fails to run
// a workgroup that another waits for).
constexpr int64_t kDefaultWaitUs = 100000;

// Number of the call after `tag`: never one whose low 17 bits are all zero
// (0 included), which the kernels' row-statistics records could not tell
// from a zeroed word.
uint32_t next_call_tag(uint32_t tag) {
  do {
    ++tag;
  } while ((tag & 0x1ffffu) == 0u);
  return tag;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// out[i] = float(in[i]) for the row diagnostics.
__global__ void narrow_to_float(const double* in, float* out, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    out[i] = float(in[i]);
}

// Lays out a workspace for calls up to (max_batch, max_draft) at `vocab` and
// `dtype` from `base` (which may be null to only size it); returns its size
// in bytes. The regions are 256-byte aligned if `base` is. `handle`: also
// the acceptance-rate partials and the lazy calls' go-on words (handles
// only).
size_t layout_workspace(int max_batch, int max_draft, int vocab, int dtype, char* base, specv::Workspace* ws,
                        bool handle) {
  const int chunk = specv::stat_chunk_elems(dtype);
  const int nch = specv::ceil_div(vocab, chunk);
  const int nm = specv::ceil_div(vocab, specv::member_elems(dtype));
  const size_t rows = size_t(max_batch) * size_t(2 * max_draft + 1);
  size_t off = 0;
  const size_t off_partials = off;
  off = align_up(off + rows * nch * specv::partial_bytes(), 256);
  const size_t off_seq = off;
  off = align_up(off + size_t(max_batch) * specv::seq_bytes(), 256);
  const size_t off_records = off;
  off = align_up(off + size_t(max_batch) * nm * specv::member_bytes(), 256);
  const size_t off_lse = off;
  off = align_up(off + rows * sizeof(double), 256);
  const size_t off_argmax = off;
  off = align_up(off + rows * sizeof(int), 256);
  const size_t off_counters = off;
  off = align_up(off + size_t(max_batch) * specv::kCounterStride * sizeof(int), 256);
  const size_t off_alive = off;
  if (handle)
    off = align_up(off + size_t(max_batch) * (size_t(2 * max_draft + 1) * nch + specv::kMaxLazyStages) * sizeof(uint64_t),
                   256);
  const size_t off_rates = off;
  const int nrc = specv::ceil_div(vocab, specv::rate_chunk_elems(dtype));
  if (handle) off = align_up(off + size_t(max_batch) * size_t(max_draft) * nrc * sizeof(double), 256);
  if (ws != nullptr) {
    ws->partials = base + off_partials;
    ws->seq = base + off_seq;
    ws->records = base + off_records;
    ws->row_lse = reinterpret_cast<double*>(base + off_lse);
    ws->row_argmax = reinterpret_cast<int*>(base + off_argmax);
    ws->draw_done = reinterpret_cast<int*>(base + off_counters);
    ws->rate_parts = handle ? reinterpret_cast<double*>(base + off_rates) : nullptr;
    ws->alive = handle ? reinterpret_cast<uint64_t*>(base + off_alive) : nullptr;
    ws->n_stat_chunks = nch;
    ws->n_rate_chunks = nrc;
    ws->n_members = nm;
    ws->stat_chunk = chunk;
  }
  return off;
}

// Whether a launch of (batch, n_draft) at `vocab` and `dtype` has a grid the
// runtime takes (one workgroup per row-statistics item, decision and draw
// member, below 2^31; a lazy call has a decision per stage).
bool grid_fits(int batch, int n_draft, int vocab, int dtype) {
  const int64_t nch = specv::ceil_div(vocab, specv::stat_chunk_elems(dtype));
  const int64_t nm = specv::ceil_div(vocab, specv::member_elems(dtype));
  return int64_t(batch) * (2 * n_draft + 1) * nch + int64_t(batch) * (nm + specv::kMaxLazyStages) < (int64_t(1) << 31);
}

}  // namespace

extern "C" {

const char* specv_strerror(int code) {
  switch (code) {
    case SPECV_OK: return "success";
    case SPECV_EINVAL: return "invalid argument";
    case SPECV_ENOMEM: return "device memory allocation failed";
    case SPECV_EHIP: return "HIP runtime error or kernel launch failure";
    case SPECV_EALIGN: return "device pointer misaligned";
    case SPECV_ESTATE: return "no successful specv_verify on this handle yet";
    case SPECV_ERANGE: return "size beyond the static workspace of specv_verify_static (batch <= 256, n_draft <= 16)";
    default: return "unknown specv status code";
  }
}

int specv_create(specv_handle* out, int max_batch, int max_draft, int vocab, specv_dtype dtype, int device) {
  if (out == nullptr) return SPECV_EINVAL;
  *out = nullptr;
  if (max_batch < 1 || max_draft < 1 || max_draft > SPECV_MAX_DRAFT) return SPECV_EINVAL;
  if (vocab < 1 || vocab > specv::kMaxVocab) return SPECV_EINVAL;
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_EINVAL;
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess) return SPECV_EHIP;
  if (device < 0 || device >= n_dev) return SPECV_EINVAL;
  if (!grid_fits(max_batch, max_draft, vocab, dtype)) return SPECV_EINVAL;
  const size_t off = layout_workspace(max_batch, max_draft, vocab, dtype, nullptr, nullptr, true);

  DeviceGuard guard(device);
  if (!guard.ok()) return SPECV_EHIP;
  specv_ctx* h = new (std::nothrow) specv_ctx();
  if (h == nullptr) return SPECV_ENOMEM;
  if (hipMalloc(&h->mem, off) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return SPECV_ENOMEM;
  }
  h->device = device;
  h->max_batch = max_batch;
  h->max_draft = max_draft;
  h->vocab = vocab;
  h->dtype = dtype;
  h->mem_bytes = off;
  layout_workspace(max_batch, max_draft, vocab, dtype, static_cast<char*>(h->mem), &h->ws, true);
  h->ws.resident_blocks = specv::max_resident_blocks(dtype);
  if (h->ws.resident_blocks < 1 || hipMemset(h->mem, 0, off) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(h->mem);
    delete h;
    return SPECV_EHIP;
  }
  h->last_batch = -1;
  h->last_n_draft = 0;
  h->next_tag = 1;
  {
    const char* dbg = getenv("SPECV_DEBUG");
    h->debug = (dbg != nullptr && dbg[0] != '\0' && strcmp(dbg, "0") != 0) ? 1u : 0u;
  }
  if (hipDeviceGetAttribute(&h->clock_khz, hipDeviceAttributeWallClockRate, device) != hipSuccess ||
      h->clock_khz <= 0) {
    (void)hipFree(h->mem);
    delete h;
    return SPECV_EHIP;
  }
  h->wait_ticks = uint64_t(kDefaultWaitUs) * uint64_t(h->clock_khz) / 1000u;
  h->timing = false;
  h->timed_call = false;
  h->timed_stages = 0;
  h->events_created = false;
  *out = h;
  return SPECV_OK;
}

int specv_verify(specv_handle h, int batch, int n_draft, const void* draft_logits, const void* target_logits,
                 const int32_t* draft_tokens, const float* accept_uniforms, const float* sample_uniforms,
                 const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted, void* stream) {
  if (h == nullptr) return SPECV_EINVAL;
  if (batch < 0 || batch > h->max_batch) return SPECV_EINVAL;
  if (n_draft < 1 || n_draft > h->max_draft) return SPECV_EINVAL;
  if (batch == 0) return SPECV_OK;
  if (!draft_logits || !target_logits || !draft_tokens || !accept_uniforms || !sample_uniforms || !temperature ||
      !out_tokens || !out_n_accepted)
    return SPECV_EINVAL;
  if (!aligned(draft_logits, 16) || !aligned(target_logits, 16)) return SPECV_EALIGN;
  if (!aligned(draft_tokens, 4) || !aligned(accept_uniforms, 4) || !aligned(sample_uniforms, 4) ||
      !aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(out_n_accepted, 4))
    return SPECV_EALIGN;

  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  specv::VerifyArgs a;
  a.batch = batch;
  a.n_draft = n_draft;
  a.vocab = h->vocab;
  a.dtype = h->dtype;
  a.draft = draft_logits;
  a.target = target_logits;
  a.tokens = draft_tokens;
  a.accept_u = accept_uniforms;
  a.sample_u = sample_uniforms;
  a.temperature = temperature;
  a.out_tokens = out_tokens;
  a.out_n = out_n_accepted;
  a.tag = h->next_tag;
  a.debug = h->debug;
  a.wait_ticks = h->wait_ticks;
  int stages = 0;
  if (specv::launch_verify(a, h->ws, s, h->timing ? h->events : nullptr, &stages) != hipSuccess) return SPECV_EHIP;
  h->next_tag = next_call_tag(h->next_tag);
  h->last_batch = batch;
  h->last_n_draft = n_draft;
  h->timed_call = h->timing;
  h->timed_stages = stages;
  return SPECV_OK;
}

int specv_verify_lazy(specv_handle h, int batch, int n_draft, const void* draft_logits, const void* target_logits,
                      const int32_t* draft_tokens, const float* accept_uniforms, const float* sample_uniforms,
                      const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted, void* stream) {
  if (h == nullptr) return SPECV_EINVAL;
  if (batch < 0 || batch > h->max_batch) return SPECV_EINVAL;
  if (n_draft < 1 || n_draft > h->max_draft) return SPECV_EINVAL;
  if (batch == 0) return SPECV_OK;
  if (!draft_logits || !target_logits || !draft_tokens || !accept_uniforms || !sample_uniforms || !temperature ||
      !out_tokens || !out_n_accepted)
    return SPECV_EINVAL;
  if (!aligned(draft_logits, 16) || !aligned(target_logits, 16)) return SPECV_EALIGN;
  if (!aligned(draft_tokens, 4) || !aligned(accept_uniforms, 4) || !aligned(sample_uniforms, 4) ||
      !aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(out_n_accepted, 4))
    return SPECV_EALIGN;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  specv::VerifyArgs a;
  a.batch = batch;
  a.n_draft = n_draft;
  a.vocab = h->vocab;
  a.dtype = h->dtype;
  a.draft = draft_logits;
  a.target = target_logits;
  a.tokens = draft_tokens;
  a.accept_u = accept_uniforms;
  a.sample_u = sample_uniforms;
  a.temperature = temperature;
  a.out_tokens = out_tokens;
  a.out_n = out_n_accepted;
  a.debug = h->debug;
  a.wait_ticks = h->wait_ticks;
  a.lazy = 1;
  a.tag = h->next_tag;
  // One launch: the stages (lazy_stage_bounds) one after the other in the
  // launch order, each over the sequences still going on at its first
  // position, then the draws.
  int stages = 0;
  if (specv::launch_verify(a, h->ws, s, nullptr, &stages) != hipSuccess) return SPECV_EHIP;
  h->next_tag = next_call_tag(h->next_tag);
  h->last_batch = batch;
  h->last_n_draft = n_draft;
  h->timed_call = false;
  return SPECV_OK;
}

int specv_sample(specv_handle h, int n_rows, const void* logits, const float* temperature, const float* uniforms,
                 int32_t* out_tokens, void* stream) {
  if (h == nullptr) return SPECV_EINVAL;
  if (n_rows < 0 || n_rows > h->max_batch) return SPECV_EINVAL;
  if (n_rows == 0) return SPECV_OK;
  if (!logits || !temperature || !uniforms || !out_tokens) return SPECV_EINVAL;
  if (!aligned(logits, 16)) return SPECV_EALIGN;
  if (!aligned(temperature, 4) || !aligned(uniforms, 4) || !aligned(out_tokens, 4)) return SPECV_EALIGN;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  // The verification with no drafts: each row is a sequence's only verifier
  // row, so its draw is the bonus draw from softmax(row / T) (the argmax at
  // T = 0); nothing reads drafts, draft tokens or accept uniforms. One pass
  // over each row: draw members only (the kernel's sampling mode).
  specv::VerifyArgs a;
  a.sample = 1;
  a.batch = n_rows;
  a.n_draft = 0;
  a.vocab = h->vocab;
  a.dtype = h->dtype;
  a.draft = logits;
  a.target = logits;
  a.tokens = nullptr;
  a.accept_u = nullptr;
  a.sample_u = uniforms;
  a.temperature = temperature;
  a.out_tokens = out_tokens;
  a.out_n = nullptr;
  a.tag = h->next_tag;
  a.debug = h->debug;
  a.wait_ticks = h->wait_ticks;
  int stages = 0;
  if (specv::launch_verify(a, h->ws, static_cast<hipStream_t>(stream), h->timing ? h->events : nullptr, &stages) !=
      hipSuccess)
    return SPECV_EHIP;
  h->next_tag = next_call_tag(h->next_tag);
  h->last_batch = n_rows;
  h->last_n_draft = 0;
  h->timed_call = h->timing;
  h->timed_stages = stages;
  return SPECV_OK;
}

int specv_acceptance_rates(specv_handle h, int batch, int n_draft, const void* draft_logits, const void* target_logits,
                           const int32_t* draft_tokens, const float* temperature, float* out_alpha, float* out_tau,
                           void* stream) {
  if (h == nullptr) return SPECV_EINVAL;
  if (batch < 0 || batch > h->max_batch || n_draft < 1 || n_draft > h->max_draft) return SPECV_EINVAL;
  if (batch == 0) return SPECV_OK;
  if (!draft_logits || !target_logits || !draft_tokens || !temperature || !out_alpha || !out_tau) return SPECV_EINVAL;
  if (!aligned(draft_logits, 16) || !aligned(target_logits, 16)) return SPECV_EALIGN;
  if (!aligned(draft_tokens, 4) || !aligned(temperature, 4) || !aligned(out_alpha, 4) || !aligned(out_tau, 4))
    return SPECV_EALIGN;
  if (h->last_batch != batch || h->last_n_draft != n_draft) return SPECV_ESTATE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  specv::RatesArgs a;
  a.batch = batch;
  a.n_draft = n_draft;
  a.vocab = h->vocab;
  a.dtype = h->dtype;
  a.draft = draft_logits;
  a.target = target_logits;
  a.tokens = draft_tokens;
  a.temperature = temperature;
  a.out_alpha = out_alpha;
  a.out_tau = out_tau;
  return specv::launch_rates(a, h->ws, static_cast<hipStream_t>(stream)) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}

int specv_row_stats(specv_handle h, float* out_lse, int32_t* out_argmax, void* stream) {
  if (h == nullptr || out_lse == nullptr || out_argmax == nullptr) return SPECV_EINVAL;
  if (!aligned(out_lse, 4) || !aligned(out_argmax, 4)) return SPECV_EALIGN;
  if (h->last_batch < 0) return SPECV_ESTATE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  const size_t n = size_t(h->last_batch) * size_t(2 * h->last_n_draft + 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(narrow_to_float, dim3(unsigned(std::min<size_t>((n + 255) / 256, 4096))), dim3(256), 0, s,
                     h->ws.row_lse, out_lse, n);
  if (hipGetLastError() != hipSuccess) return SPECV_EHIP;
  if (hipMemcpyAsync(out_argmax, h->ws.row_argmax, n * sizeof(int), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SPECV_EHIP;
  return SPECV_OK;
}

int specv_set_wait_limit(specv_handle h, int64_t microseconds) {
  if (h == nullptr || microseconds < 0 || microseconds > int64_t(3600) * 1000000) return SPECV_EINVAL;
  h->wait_ticks = uint64_t(microseconds) * uint64_t(h->clock_khz) / 1000u;
  return SPECV_OK;
}

int specv_set_timing(specv_handle h, int enable) {
  if (h == nullptr) return SPECV_EINVAL;
  if (enable && !h->events_created) {
    DeviceGuard guard(h->device);
    if (!guard.ok()) return SPECV_EHIP;
    for (int i = 0; i <= specv::kMaxStages; ++i) {
      if (hipEventCreate(&h->events[i]) != hipSuccess) {
        for (int k = 0; k < i; ++k) (void)hipEventDestroy(h->events[k]);
        return SPECV_EHIP;
      }
    }
    h->events_created = true;
  }
  h->timing = enable != 0;
  return SPECV_OK;
}

int specv_last_timings(specv_handle h, float* ms, int capacity, int* count) {
  if (h == nullptr || ms == nullptr || count == nullptr || capacity < 1) return SPECV_EINVAL;
  if (!h->timed_call) return SPECV_ESTATE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  const int n = h->timed_stages;
  if (hipEventSynchronize(h->events[n]) != hipSuccess) return SPECV_EHIP;
  for (int i = 0; i < n && i < capacity; ++i) {
    if (hipEventElapsedTime(&ms[i], h->events[i], h->events[i + 1]) != hipSuccess) return SPECV_EHIP;
  }
  *count = n;
  return SPECV_OK;
}

const char* specv_stage_name(int stage) { return specv::stage_name(stage); }



void specv_destroy(specv_handle h) {
  if (h == nullptr) return;
  {
    DeviceGuard guard(h->device);
    if (guard.ok()) {
      (void)hipDeviceSynchronize();
      (void)hipFree(h->mem);
      if (h->events_created)
        for (int i = 0; i <= specv::kMaxStages; ++i) (void)hipEventDestroy(h->events[i]);
    }
  }
  delete h;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// specv_verify_static: the same verification with no handle and no
// allocation. Its workspace is `scratch`, a device array of this file (one
// copy per GPU, held until the process ends), laid out once for the largest
// call it takes; the kernels receive its device address as they receive a
// handle's workspace.

namespace {

constexpr int kStaticMaxBatch = 256;
constexpr int kStaticMaxDraft = 16;
// layout_workspace(256, 16, 2^18, float32) = 8367104 bytes; checked at set-up.
constexpr size_t kStaticBytes = size_t(8) << 20;
constexpr int kStaticMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticBytes];

namespace {

// Fills n 16-byte words with zeros (once per device, before the first call).
__global__ void zero_words(uint4* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct StaticDevice {
  std::atomic<int> ready{0};
  char* ptr = nullptr;  // device address of `scratch` on this device
  int resident[2] = {0, 0};
  uint64_t wait_ticks = 0;
  uint32_t debug = 0;
  std::atomic<uint32_t> tag{1};
};
StaticDevice g_static[kStaticMaxDevices];
std::mutex g_static_mu;

uint32_t take_tag(std::atomic<uint32_t>& t) {
  uint32_t cur = t.load(std::memory_order_relaxed);
  while (!t.compare_exchange_weak(cur, next_call_tag(cur), std::memory_order_relaxed)) {
  }
  return cur;
}

// Once per device, with that device current: the array's device address, the
// launch parameters, and the array cleared on `stream` (ahead of the call
// that set it up).
int static_setup(int dev, hipStream_t stream) {
  StaticDevice& sd = g_static[dev];
  if (sd.ready.load(std::memory_order_acquire)) return SPECV_OK;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (sd.ready.load(std::memory_order_relaxed)) return SPECV_OK;
  if (layout_workspace(kStaticMaxBatch, kStaticMaxDraft, specv::kMaxVocab, SPECV_F32, nullptr, nullptr, false) >
      kStaticBytes)
    return SPECV_EHIP;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return SPECV_EHIP;
  }
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return SPECV_EHIP;
  const int r0 = specv::max_resident_blocks(SPECV_F32), r1 = specv::max_resident_blocks(SPECV_BF16);
  if (r0 < 1 || r1 < 1) return SPECV_EHIP;
  hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(ptr), kStaticBytes / 16);
  if (hipGetLastError() != hipSuccess) return SPECV_EHIP;
  sd.ptr = static_cast<char*>(ptr);
  sd.resident[SPECV_F32] = r0;
  sd.resident[SPECV_BF16] = r1;
  sd.wait_ticks = uint64_t(kDefaultWaitUs) * uint64_t(khz) / 1000u;
  const char* dbg = getenv("SPECV_DEBUG");
  sd.debug = (dbg != nullptr && dbg[0] != '\0' && strcmp(dbg, "0") != 0) ? 1u : 0u;
  sd.ready.store(1, std::memory_order_release);
  return SPECV_OK;
}

}  // namespace

extern "C" int specv_verify_static(int batch, int n_draft, int vocab, specv_dtype dtype, const void* draft_logits,
                                   const void* target_logits, const int32_t* draft_tokens,
                                   const float* accept_uniforms, const float* sample_uniforms,
                                   const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted,
                                   void* stream) {
  if (batch < 0 || n_draft < 1 || vocab < 1) return SPECV_EINVAL;
  if (dtype != SPECV_F32 && dtype != SPECV_BF16) return SPECV_EINVAL;
  if (batch > kStaticMaxBatch || n_draft > kStaticMaxDraft || vocab > specv::kMaxVocab) return SPECV_ERANGE;
  if (batch == 0) return SPECV_OK;
  if (!draft_logits || !target_logits || !draft_tokens || !accept_uniforms || !sample_uniforms || !temperature ||
      !out_tokens || !out_n_accepted)
    return SPECV_EINVAL;
  if (!aligned(draft_logits, 16) || !aligned(target_logits, 16)) return SPECV_EALIGN;
  if (!aligned(draft_tokens, 4) || !aligned(accept_uniforms, 4) || !aligned(sample_uniforms, 4) ||
      !aligned(temperature, 4) || !aligned(out_tokens, 4) || !aligned(out_n_accepted, 4))
    return SPECV_EALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kStaticMaxDevices) return SPECV_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rc = static_setup(dev, s);
  if (rc != SPECV_OK) return rc;
  StaticDevice& sd = g_static[dev];
  // Every region at the offset of the largest layout, whatever this call's
  // vocabulary, so the counters always sit where the last call left them at 0.
  specv::Workspace ws;
  layout_workspace(kStaticMaxBatch, kStaticMaxDraft, specv::kMaxVocab, SPECV_F32, sd.ptr, &ws, false);
  ws.stat_chunk = specv::stat_chunk_elems(dtype);
  ws.n_stat_chunks = specv::ceil_div(vocab, ws.stat_chunk);
  ws.n_members = specv::ceil_div(vocab, specv::member_elems(dtype));
  ws.resident_blocks = sd.resident[dtype];
  specv::VerifyArgs a;
  a.batch = batch;
  a.n_draft = n_draft;
  a.vocab = vocab;
  a.dtype = dtype;
  a.draft = draft_logits;
  a.target = target_logits;
  a.tokens = draft_tokens;
  a.accept_u = accept_uniforms;
  a.sample_u = sample_uniforms;
  a.temperature = temperature;
  a.out_tokens = out_tokens;
  a.out_n = out_n_accepted;
  a.tag = take_tag(sd.tag);
  a.debug = sd.debug;
  a.wait_ticks = sd.wait_ticks;
  int stages = 0;
  return specv::launch_verify(a, ws, s, nullptr, &stages) == hipSuccess ? SPECV_OK : SPECV_EHIP;
}
