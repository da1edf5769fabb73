// C-ABI host side of libspecv: handle, workspace, argument checks, launches.
// The public contract (layouts, ownership, errors) is in include/specv.h.

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
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

  const int chunk = specv::stat_chunk_elems(dtype);
  const int nch = specv::ceil_div(vocab, chunk);
  const int nm = specv::ceil_div(vocab, specv::member_elems(dtype));
  const size_t rows = size_t(max_batch) * size_t(2 * max_draft + 1);
  // Grid: one workgroup per row-statistics item, per decision and per draw member.
  if (int64_t(rows) * nch + int64_t(max_batch) * (nm + 1) >= (int64_t(1) << 31)) return SPECV_EINVAL;

  size_t off = 0;
  const size_t off_partials = off;
  off = align_up(off + rows * nch * specv::partial_bytes(), 256);
  const size_t off_seq = off;
  off = align_up(off + size_t(max_batch) * specv::seq_bytes(), 256);
  const size_t off_records = off;
  off = align_up(off + size_t(max_batch) * nm * specv::member_bytes(), 256);
  const size_t off_lse = off;
  off = align_up(off + rows * sizeof(float), 256);
  const size_t off_argmax = off;
  off = align_up(off + rows * sizeof(int), 256);
  const size_t off_counters = off;
  off = align_up(off + size_t(max_batch) * specv::kCounterStride * sizeof(int), 256);

  DeviceGuard guard(device);
  if (!guard.ok()) return SPECV_EHIP;
  specv_ctx* h = new (std::nothrow) specv_ctx();
  if (h == nullptr) return SPECV_ENOMEM;
  if (hipMalloc(&h->mem, off) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return SPECV_ENOMEM;
  }
  char* base = static_cast<char*>(h->mem);
  h->device = device;
  h->max_batch = max_batch;
  h->max_draft = max_draft;
  h->vocab = vocab;
  h->dtype = dtype;
  h->mem_bytes = off;
  h->ws.partials = base + off_partials;
  h->ws.seq = base + off_seq;
  h->ws.records = base + off_records;
  h->ws.row_lse = reinterpret_cast<float*>(base + off_lse);
  h->ws.row_argmax = reinterpret_cast<int*>(base + off_argmax);
  h->ws.draw_done = reinterpret_cast<int*>(base + off_counters);
  h->ws.n_stat_chunks = nch;
  h->ws.n_members = nm;
  h->ws.stat_chunk = chunk;
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

int specv_row_stats(specv_handle h, float* out_lse, int32_t* out_argmax, void* stream) {
  if (h == nullptr || out_lse == nullptr || out_argmax == nullptr) return SPECV_EINVAL;
  if (!aligned(out_lse, 4) || !aligned(out_argmax, 4)) return SPECV_EALIGN;
  if (h->last_batch < 0) return SPECV_ESTATE;
  DeviceGuard guard(h->device);
  if (!guard.ok()) return SPECV_EHIP;
  const size_t n = size_t(h->last_batch) * size_t(2 * h->last_n_draft + 1);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(out_lse, h->ws.row_lse, n * sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess)
    return SPECV_EHIP;
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
