// gfx950 kernels for batched speculative-sampling verification.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with "Step 1: 거절 단계" (the
// accept test) and "Step 2: 잔차 분포" (the residual); blog "…투기적 디코딩
// (Speculative Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// One launch per call. B sequences, N drafts, 2N+1 rows of V logits each; the
// grid is B*(2N+1)*nch row-statistics workgroups followed by B*nsch draw-chunk
// workgroups, both in sequence order:
//   row statistics  one workgroup per (row, 32 KB chunk): fp32 max, sum of
//                   2^(z*c - fl(max*c)) with c = log2(e)/T, first argmax, and
//                   the logit at the row's draft token if the chunk holds it.
//                   Streaming and HBM-bound; greedy sequences skip draft rows.
//                   The sequence's last workgroup (its last chunk of target
//                   row N) then collects the sequence's row partials, merges
//                   them into log-normalisers, runs the N accept tests in fp64
//                   and writes the accepted prefix and a sequence record.
//   draw chunks     one workgroup per (sequence, 4096-logit chunk): waits for
//                   the sequence record, sums fp64 exps over its chunk of the
//                   row(s) the draw needs; the sequence's last chunk
//                   workgroup then collects the chunk sums, finds the chunk
//                   where the inverse CDF crosses u*S and rescans it in fp64.
// Draw-chunk workgroups come after every row-statistics workgroup in the
// grid, so those of early sequences run while the stream is still going.
//
// The residual weight of token x is w_x = max(0, et_x/Zt - ed_x/Zd)
// = max(0, et_x - rho*ed_x)/Zt with rho = Zt/Zd, so its sign only depends on
// whether log(et_x/ed_x) exceeds log(rho). The decision knows log(rho) from the
// fp32 row sums to ~1e-6; a draw chunk treats tokens more than 1e-4 away from it
// as certain and sums their exps into A and B, so the chunk's weight is
// (A - rho*B)/Zt plus the exact terms of its few uncertain tokens, whose exps
// the chunk records. One pass over the rows gives the normalisers and every
// chunk weight.
//
// Records passed between workgroups are 64-bit words written and read with
// device-coherent (agent-scope relaxed atomic) stores and loads; each word
// carries the call's sequence number in its high half, so a reader knows a
// word is current without fences, counters or cache write-backs. A workgroup
// waiting for records polls them for a bounded time; past that bound it
// computes the missing records itself. Records are deterministic, so a
// duplicate computes and writes the very same bits, and no wait depends on
// the order in which the hardware dispatches workgroups.
//
// Every reduction has a fixed order, so results are bitwise reproducible.

#include <float.h>
#include <limits.h>
#include <math.h>

#include "specv_internal.h"
#include "specv_math.h"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;
constexpr float kFltMax = 3.402823466e38f;
constexpr int kWaves = kThreads / 64;
constexpr int kRun = kSampChunk / kThreads;            // consecutive logits a thread owns in a draw chunk
static_assert(kMaxSampChunks <= kThreads, "the draw gives each thread at most one chunk");
constexpr int kMaxRows = 2 * 64 + 1;
constexpr double kSignBand = 1e-4;  // |log(et/ed) - log(rho)| at or below this is uncertain
constexpr int kMaxRecomputeRounds = 3;  // a waiter's own recomputation always completes in one

__device__ __forceinline__ bool temperature_valid(float t) {
  return t == 0.0f || (t >= kMinTemperature && t <= kFltMax);
}

// c in 2^(z*c) == exp(z/T); finite for T >= kMinTemperature.
__device__ __forceinline__ float exp2_coef(float t) { return kLog2e / t; }

// K = fl(m * c), never contracted into a neighbouring add.
__device__ __forceinline__ float scaled_max(float m, float c) { return __fmul_rn(m, c); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Diagnostic builds (-DSPECV_TRACE) stamp the wall clock (100 MHz) at fixed
// points of each workgroup.
#if defined(SPECV_TRACE)
constexpr int kTraceBlocks = 1 << 17;
constexpr int kTraceWords = 8;
__device__ uint64_t g_trace[kTraceBlocks * kTraceWords];
__device__ __forceinline__ void trace(int slot) {
  if (threadIdx.x == 0 && blockIdx.x < kTraceBlocks)
    g_trace[int64_t(blockIdx.x) * kTraceWords + slot] = wall_clock64();
}
#else
__device__ __forceinline__ void trace(int) {}
#endif

// ---------------------------------------------------------------------------
// Tagged device-coherent words: payload in the low half, the call's sequence
// number in the high half.

__device__ __forceinline__ void put_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_word(uint64_t* p, uint32_t v, uint32_t ep) {
  put_u64(p, (uint64_t(ep) << 32) | v);
}
__device__ __forceinline__ void put_word_f(uint64_t* p, float v, uint32_t ep) { put_word(p, __float_as_uint(v), ep); }
__device__ __forceinline__ void put_word_d(uint64_t* p, double v, uint32_t ep) {
  const uint64_t u = double_to_bits(v);
  put_word(p, uint32_t(u), ep);
  put_word(p + 1, uint32_t(u >> 32), ep);
}
// Reads clear `ok` when the word is not from this call.
__device__ __forceinline__ uint32_t get_word(const uint64_t* p, uint32_t ep, bool& ok) {
  const uint64_t w = get_u64(p);
  ok = ok && uint32_t(w >> 32) == ep;
  return uint32_t(w);
}
__device__ __forceinline__ float get_word_f(const uint64_t* p, uint32_t ep, bool& ok) {
  return __uint_as_float(get_word(p, ep, ok));
}
__device__ __forceinline__ double get_word_d(const uint64_t* p, uint32_t ep, bool& ok) {
  const uint32_t lo = get_word(p, ep, ok);
  const uint32_t hi = get_word(p + 1, ep, ok);
  return bits_to_double((uint64_t(hi) << 32) | lo);
}
// This thread's earlier stores are complete (visible to every workgroup).
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Logit access.

template <typename T>
struct Logit;

template <>
struct Logit<float> {
  static constexpr int kVec = 4;  // logits per 16-byte load
  __device__ static float at(const float* p, int64_t i) { return p[i]; }
  __device__ static void unpack(const uint4& x, float (&v)[kVec]) {
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z);
    v[3] = __uint_as_float(x.w);
  }
};

template <>
struct Logit<uint16_t> {  // bfloat16 bits
  static constexpr int kVec = 8;
  __device__ static float at(const uint16_t* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
  __device__ static void unpack(const uint4& x, float (&v)[kVec]) {
    v[0] = __uint_as_float(x.x << 16);
    v[1] = __uint_as_float(x.x & 0xffff0000u);
    v[2] = __uint_as_float(x.y << 16);
    v[3] = __uint_as_float(x.y & 0xffff0000u);
    v[4] = __uint_as_float(x.z << 16);
    v[5] = __uint_as_float(x.z & 0xffff0000u);
    v[6] = __uint_as_float(x.w << 16);
    v[7] = __uint_as_float(x.w & 0xffff0000u);
  }
};

// kRun consecutive logits of a row starting at element e, as fp32; -inf at
// and past `vocab`. 16-byte loads when the row start is 16-byte aligned and
// the run lies inside the row.
template <typename T>
__device__ __forceinline__ void load_run(const T* __restrict__ row, int e, int vocab, bool vec_ok,
                                         float (&z)[kRun]) {
  constexpr int kVec = Logit<T>::kVec;
  if (vec_ok && e + kRun <= vocab) {
    const uint4* __restrict__ p = reinterpret_cast<const uint4*>(row + e);
    uint4 x[kRun / kVec];
#pragma unroll
    for (int u = 0; u < kRun / kVec; ++u) x[u] = p[u];
#pragma unroll
    for (int u = 0; u < kRun / kVec; ++u) {
      float v[kVec];
      Logit<T>::unpack(x[u], v);
#pragma unroll
      for (int k = 0; k < kVec; ++k) z[u * kVec + k] = v[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < kRun; ++k) z[k] = (e + k < vocab) ? Logit<T>::at(row, e + k) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Block reductions (fixed order).

__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double total = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) total += red[w];
  return total;
}

// Block-wide inclusive scan of one double per thread; returns the thread's
// inclusive prefix and sets total.
__device__ __forceinline__ double block_scan(double v, double& total, double* red) {
  const int lane = threadIdx.x & 63;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  __syncthreads();
  if (lane == 63) red[threadIdx.x >> 6] = incl;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < (int(threadIdx.x) >> 6)) before += red[w];
    total += red[w];
  }
  return before + incl;
}

// ---------------------------------------------------------------------------
// Row statistics.

// Running state: m = largest logit seen, idx = its first index, s = sum of
// 2^(z*c - k) with k = fl(m*c) once a finite logit was seen (0 before, while
// s is 0 too). The exact product m*c differs from k by r = fma(m, c, -k); the
// decision removes it.
struct StatAcc {
  float m;
  float k;
  float s;
  int idx;
};

__device__ __forceinline__ void acc_init(StatAcc& a) {
  a.m = -INFINITY;
  a.k = 0.0f;
  a.s = 0.0f;
  a.idx = INT_MAX;
}

// Fold n logits with consecutive indices base..base+n-1. A thread visits its
// indices in increasing order, so a strict '>' keeps a repeated maximum's
// first index.
template <bool kSampled, int n>
__device__ __forceinline__ void acc_values(StatAcc& a, const float (&v)[n], int base, float c) {
  float vmax = v[0];
#pragma unroll
  for (int k = 1; k < n; ++k) vmax = fmaxf(vmax, v[k]);
  if (vmax > a.m) {
    int first = n - 1;
#pragma unroll
    for (int k = n - 1; k >= 0; --k) first = (v[k] == vmax) ? k : first;
    if (kSampled) {
      const float k_new = scaled_max(vmax, c);
      a.s = (a.s == 0.0f) ? 0.0f : a.s * fast_exp2(a.k - k_new);
      a.k = k_new;
    }
    a.m = vmax;
    a.idx = base + first;
  }
  if (kSampled) {
    float e[n];
#pragma unroll
    for (int k = 0; k < n; ++k) e[k] = fast_exp2(fmaf(v[k], c, -a.k));
#pragma unroll
    for (int w = 1; w < n; w *= 2)
#pragma unroll
      for (int k = 0; k + w < n; k += 2 * w) e[k] += e[k + w];
    a.s += e[0];
  }
}

// Merge partial (m2, s2, i2) into (m, s, idx).
template <bool kSampled>
__device__ __forceinline__ void acc_merge(float& m, float& s, int& idx, float m2, float s2, int i2, float c) {
  const float mm = fmaxf(m, m2);
  if (kSampled) {
    const float km = scaled_max(mm, c);
    const float a = (m == mm) ? s : s * fast_exp2(scaled_max(m, c) - km);
    const float b = (m2 == mm) ? s2 : s2 * fast_exp2(scaled_max(m2, c) - km);
    s = a + b;
  }
  idx = (m > m2) ? idx : ((m2 > m) ? i2 : min(idx, i2));
  m = mm;
}

// Statistics of elements [e0, e1) of a row. The vectors a thread owns are
// folded in the same order whatever kGroup (how many 16-byte loads are in
// flight at once), so every kGroup gives bitwise the same result.
template <typename T, bool kSampled, int kGroup>
__device__ __forceinline__ void stats_chunk(const T* __restrict__ row, int64_t row_flat, int e0, int e1, float c,
                                            StatAcc& a) {
  constexpr int kVec = Logit<T>::kVec;
  const int tid = threadIdx.x;
  // Element g of the flat buffer is 16-byte aligned iff g % kVec == 0 (the
  // buffer base is 16-byte aligned); a misaligned row start peels a head.
  const int mis = int((row_flat + e0) % kVec);
  int ea = e0 + (kVec - mis) % kVec;
  if (ea > e1) ea = e1;
  const int nv = (e1 - ea) / kVec;
  const int et = ea + nv * kVec;
  if (tid < ea - e0) {
    const float v[1] = {Logit<T>::at(row, e0 + tid)};
    acc_values<kSampled>(a, v, e0 + tid, c);
  }
  // A chunk holds at most kMaxVec 16-byte vectors per thread; a group's loads
  // are all issued before any of them is used.
  constexpr int kMaxVec = kStatsChunkBytes / 16 / kThreads;
  static_assert(kMaxVec % kGroup == 0, "groups tile the chunk");
  const uint4* __restrict__ vrow = reinterpret_cast<const uint4*>(row + ea);
#pragma unroll
  for (int g0 = 0; g0 < kMaxVec; g0 += kGroup) {
    uint4 x[kGroup];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int k = tid + (g0 + u) * kThreads;
      if (k < nv) x[u] = vrow[k];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int k = tid + (g0 + u) * kThreads;
      if (k < nv) {
        float v[kVec];
        Logit<T>::unpack(x[u], v);
        acc_values<kSampled>(a, v, ea + k * kVec, c);
      }
    }
  }
  if (tid < e1 - et) {
    const float v[1] = {Logit<T>::at(row, et + tid)};
    acc_values<kSampled>(a, v, et + tid, c);
  }
}

struct StatShared {
  float m[kWaves], s[kWaves];
  int idx[kWaves];
};

template <bool kSampled>
__device__ __forceinline__ void block_merge(StatAcc& a, float c, StatShared& sh) {
  float m = a.m, s = a.s;
  int idx = a.idx;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    const int i2 = __shfl_xor(idx, off);
    acc_merge<kSampled>(m, s, idx, m2, s2, i2, c);
  }
  if ((threadIdx.x & 63) == 0) {
    sh.m[threadIdx.x >> 6] = m;
    sh.s[threadIdx.x >> 6] = s;
    sh.idx[threadIdx.x >> 6] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sh.m[0];
    s = sh.s[0];
    idx = sh.idx[0];
    for (int w = 1; w < kWaves; ++w) acc_merge<kSampled>(m, s, idx, sh.m[w], sh.s[w], sh.idx[w], c);
    a.m = m;
    a.s = s;
    a.idx = idx;
  }
}

// Everything the launch needs; passed by value.
struct Params {
  const void* draft;
  const void* target;
  const int* tokens;
  const float* accept_u;
  const float* sample_u;
  const float* temperature;
  int* out_tokens;
  int* out_n;
  float* row_lse;
  int* row_argmax;
  uint64_t* partials;  // [rows][nch][kPartWords]
  uint64_t* seq;       // [batch][kSeqWords]
  uint64_t* norm;      // [batch][nsch][kNormWords]
  const double* exp_table;
  uint64_t wait_ticks;  // bound on a wait, in 100 MHz wall-clock ticks
  uint32_t epoch;       // this call's sequence number, never 0
  int n_draft;
  int vocab;
  int nch;     // row-statistics chunks per row
  int chunk;   // logits per row-statistics chunk
  int nsch;    // draw chunks per row
  int vec_ok;  // rows start 16-byte aligned
  int n_stat_items;
};

// Record layouts (64-bit tagged words).
//   row partial:  m, s, idx, logit at the row's draft token (when in the chunk)
//   sequence:     mode | j << 8, m_target, m_draft, log_rho (2 words)
//   draw chunk:   zt, zd, a, b (2 words each), n_unc, then per uncertain token et, ed (2 words each)
constexpr int kNormHead = 9;

__device__ __forceinline__ uint64_t* partial_at(const Params P, int b, int r, int c) {
  return P.partials + ((int64_t(b) * (2 * P.n_draft + 1) + r) * P.nch + c) * kPartWords;
}
__device__ __forceinline__ uint64_t* norm_at(const Params P, int b, int c) {
  return P.norm + (int64_t(b) * P.nsch + c) * kNormWords;
}

// Did the wait that started at t0 run out? Uniform over the workgroup.
__device__ __forceinline__ bool wait_expired(const Params P, uint64_t t0) {
  return __syncthreads_or(wall_clock64() - t0 > P.wait_ticks);
}

struct DecideShared {
  float row_m[kMaxRows];
  double row_logz[kMaxRows];
  int row_idx[kMaxRows];
  float row_zg[kMaxRows];
  int row_done[kMaxRows];
  int bad_part;
  unsigned long long rej_mask;
};

constexpr int kUncPerThread = 2;  // uncertain tokens a thread stages; more overflow the chunk

struct DrawShared {
  double red[kWaves];
  int unc_base[kWaves];
  double unc_et[kUncPerThread][kThreads];
  double unc_ed[kUncPerThread][kThreads];
  double w[kMaxSampChunks];
  int flag[kMaxSampChunks];  // while collecting: chunk still missing; then: its uncertain-token count
  int pick[2];
};

struct Shared {
  double exp_table[kExpTableSize];
  StatShared st;
  union {
    DecideShared dec;
    DrawShared drw;
  } u;
};

// ---------------------------------------------------------------------------
// Row statistics.

// The draft token of row r (draft row i or target row i: d_i), or -1 for target row N.
__device__ __forceinline__ int row_token(const Params P, int b, int r) {
  const int N = P.n_draft;
  const int pos = r < N ? r : r - N;
  return pos < N ? P.tokens[int64_t(b) * N + pos] : -1;
}

// Statistics of chunk c of row r of sequence b (whole workgroup); thread 0
// writes the tagged partial. kGroup: 16-byte loads in flight per thread (the
// result does not depend on it).
template <typename T, int kGroup>
__device__ __forceinline__ void stat_item(const Params P, Shared& sh, int b, int r, int c, float t) {
  const int N = P.n_draft;
  const bool greedy = (t == 0.0f);
  const int64_t row_flat = (r < N) ? (int64_t(b) * N + r) * P.vocab : (int64_t(b) * (N + 1) + (r - N)) * P.vocab;
  const T* rowp = static_cast<const T*>(r < N ? P.draft : P.target) + row_flat;
  const int e0 = c * P.chunk;
  const int e1 = min(P.vocab, e0 + P.chunk);
  const int d = row_token(P, b, r);
  StatAcc a;
  acc_init(a);
  if (greedy) {
    stats_chunk<T, false, kGroup>(rowp, row_flat, e0, e1, 0.0f, a);
    block_merge<false>(a, 0.0f, sh.st);
  } else {
    const float c2 = exp2_coef(t);
    stats_chunk<T, true, kGroup>(rowp, row_flat, e0, e1, c2, a);
    block_merge<true>(a, c2, sh.st);
  }
  if (threadIdx.x == 0) {
    const float zg = (d >= e0 && d < e1) ? Logit<T>::at(rowp, d) : 0.0f;
    uint64_t* out = partial_at(P, b, r, c);
    put_word_f(out, a.m, P.epoch);
    put_word_f(out + 1, a.s, P.epoch);
    put_word(out + 2, uint32_t(a.idx), P.epoch);
    put_word_f(out + 3, zg, P.epoch);
  }
}

// ---------------------------------------------------------------------------
// Decision.

struct SeqInfo {
  int mode;
  int j;
  float m_target;
  float m_draft;
  double log_rho;
};

__device__ __forceinline__ void write_seq(const Params P, int b, const SeqInfo& s) {
  uint64_t* w = P.seq + int64_t(b) * kSeqWords;
  put_word(w, uint32_t(s.mode) | (uint32_t(s.j) << 8), P.epoch);
  put_word_f(w + 1, s.m_target, P.epoch);
  put_word_f(w + 2, s.m_draft, P.epoch);
  put_word_d(w + 3, s.log_rho, P.epoch);
}

// The decision for sequence b: per-row log-normalisers and argmaxes from the
// row partials, the N accept tests, the first rejection; writes the accepted
// prefix (and the token itself when greedy), the row diagnostics and the
// sequence record. Every workgroup that runs it for a call computes and
// writes the same values.
template <typename T>
__device__ __forceinline__ SeqInfo decide_seq(const Params P, Shared& sh, int b) {
  DecideShared& ds = sh.u.dec;
  const int N = P.n_draft;
  const int R = 2 * N + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int* tok = P.tokens + int64_t(b) * N;
  int* otok = P.out_tokens + int64_t(b) * (N + 1);
  float* lse = P.row_lse + int64_t(b) * R;
  int* amax = P.row_argmax + int64_t(b) * R;
  const float t = P.temperature[b];
  SeqInfo rec{kModeNone, 0, 0.0f, 0.0f, 0.0};

  int d = 0;
  float ua = 0.0f;
  bool bad = !temperature_valid(t);
  if (tid < N) {
    d = tok[tid];
    bad = bad || d < 0 || d >= P.vocab;
    ua = P.accept_u[int64_t(b) * N + tid];
  }
  if (__syncthreads_or(bad)) {
    for (int i = tid; i <= N; i += kThreads) otok[i] = -1;
    for (int r = tid; r < R; r += kThreads) {
      lse[r] = NAN;
      amax[r] = -1;
    }
    if (tid == 0) {
      P.out_n[b] = -1;
      write_seq(P, b, rec);
    }
    return rec;
  }
  const bool greedy = (t == 0.0f);
  const float c = greedy ? 0.0f : exp2_coef(t);
  const double inv_t = greedy ? 0.0 : 1.0 / double(t);
  const int r_first = greedy ? N : 0;
  for (int r = tid; r < R; r += kThreads) ds.row_done[r] = (r < r_first);
  __syncthreads();

  // Merge each row's chunk partials once they are all current: waves take
  // rows wave, wave+4, ...; lanes take chunks lane, lane+64, ..., then a
  // fixed butterfly. Past the wait bound the workgroup computes the missing
  // partials itself.
  const uint64_t t0 = wall_clock64();
  int rounds = 0;
  while (true) {
    for (int r = r_first + wave; r < R; r += kWaves) {
      if (ds.row_done[r]) continue;
      const int gchunk = (r < 2 * N) ? tok[r < N ? r : r - N] / P.chunk : -1;
      float m = -INFINITY, s = 0.0f, zg = 0.0f;
      int idx = INT_MAX;
      bool ok = true;
      for (int k = lane; k < P.nch; k += 64) {
        const uint64_t* w = partial_at(P, b, r, k);
        const float m2 = get_word_f(w, P.epoch, ok);
        const float s2 = get_word_f(w + 1, P.epoch, ok);
        const int i2 = int(get_word(w + 2, P.epoch, ok));
        const float z2 = get_word_f(w + 3, P.epoch, ok);
        if (greedy)
          acc_merge<false>(m, s, idx, m2, s2, i2, c);
        else
          acc_merge<true>(m, s, idx, m2, s2, i2, c);
        if (k == gchunk) zg = z2;
      }
      if (__ballot(!ok) != 0) continue;  // wave-uniform
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float s2 = __shfl_xor(s, off);
        const int i2 = __shfl_xor(idx, off);
        zg += __shfl_xor(zg, off);  // one lane holds the token's logit, the others 0: exact
        if (greedy)
          acc_merge<false>(m, s, idx, m2, s2, i2, c);
        else
          acc_merge<true>(m, s, idx, m2, s2, i2, c);
      }
      if (lane == 0) {
        if (idx == INT_MAX) idx = 0;  // an all -inf row: every index ties, the first wins
        // log sum_x exp((z_x - m)/T) = ln2 * (log2 s - r), r = m*c - fl(m*c) exactly.
        const double logz = greedy ? 0.0 : kLn2 * (log2(double(s)) - double(fmaf(m, c, -scaled_max(m, c))));
        ds.row_m[r] = m;
        ds.row_logz[r] = logz;
        ds.row_idx[r] = idx;
        ds.row_zg[r] = zg;
        ds.row_done[r] = 1;
        lse[r] = greedy ? NAN : float(double(m) * inv_t + logz);
        amax[r] = idx;
      }
    }
    if (__syncthreads_and(tid >= R || ds.row_done[tid] != 0)) break;
    if (wait_expired(P, t0)) {
      if (++rounds > kMaxRecomputeRounds) {
        // Unreachable unless the records are broken: fail the sequence
        // rather than wait forever.
        for (int i = tid; i <= N; i += kThreads) otok[i] = -1;
        if (tid == 0) {
          P.out_n[b] = -1;
          write_seq(P, b, rec);
        }
        __syncthreads();
        return rec;
      }
      for (int r = r_first; r < R; ++r) {
        if (ds.row_done[r]) continue;
        for (int k = 0; k < P.nch; ++k) {
          if (tid == 0) {
            bool ok = true;
            const uint64_t* w = partial_at(P, b, r, k);
            for (int q = 0; q < kPartWords; ++q) (void)get_word(w + q, P.epoch, ok);
            ds.bad_part = ok ? 0 : 1;
          }
          __syncthreads();
          const bool missing = ds.bad_part != 0;
          __syncthreads();
          if (missing) stat_item<T, 2>(P, sh, b, r, k, t);
        }
      }
      stores_done();
      __syncthreads();
    } else {
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (greedy) {
    for (int r = tid; r < N; r += kThreads) {
      lse[r] = NAN;
      amax[r] = -1;
    }
  }

  bool accept = true;
  if (tid < N) {
    const float zt = ds.row_zg[N + tid];
    const float zd = ds.row_zg[tid];
    if (greedy) {
      accept = (d == ds.row_idx[N + tid]);
    } else if (zd == -INFINITY) {
      accept = true;  // p(d) == 0: the ratio is infinite
    } else {
      const double log_q = (double(zt) - double(ds.row_m[N + tid])) * inv_t - ds.row_logz[N + tid];
      const double log_p = (double(zd) - double(ds.row_m[tid])) * inv_t - ds.row_logz[tid];
      accept = double(ua) < exp(log_q - log_p);
    }
  }
  // N <= 64: every decision lives in wave 0.
  if (wave == 0) {
    const unsigned long long rej = __ballot(tid < N && !accept);
    if (lane == 0) ds.rej_mask = rej;
  }
  __syncthreads();
  const unsigned long long rej = ds.rej_mask;
  const int j = rej ? (__ffsll(rej) - 1) : N;
  rec.mode = greedy ? kModeNone : (j < N ? kModeResidual : kModeBonus);
  rec.j = j;
  rec.m_target = ds.row_m[N + j];
  rec.m_draft = (j < N && !greedy) ? ds.row_m[j] : 0.0f;
  rec.log_rho = (j < N && !greedy) ? ds.row_logz[N + j] - ds.row_logz[j] : 0.0;
  for (int i = tid; i <= N; i += kThreads) {
    if (i < j)
      otok[i] = tok[i];
    else if (i > j)
      otok[i] = -1;
    else if (greedy)
      otok[i] = ds.row_idx[N + j];
  }
  if (tid == 0) {
    P.out_n[b] = j;
    write_seq(P, b, rec);
  }
  __syncthreads();
  return rec;
}

// The record of sequence b once current; past the wait bound the workgroup
// makes the decision itself.
template <typename T>
__device__ __forceinline__ SeqInfo wait_seq(const Params P, Shared& sh, int b) {
  const uint64_t* w = P.seq + int64_t(b) * kSeqWords;
  const uint64_t t0 = wall_clock64();
  do {
    bool ok = true;
    SeqInfo s;
    const uint32_t mj = get_word(w, P.epoch, ok);
    s.m_target = get_word_f(w + 1, P.epoch, ok);
    s.m_draft = get_word_f(w + 2, P.epoch, ok);
    s.log_rho = get_word_d(w + 3, P.epoch, ok);
    s.mode = int(mj & 0xffu);
    s.j = int(mj >> 8);
    if (__syncthreads_and(ok)) return s;
    __builtin_amdgcn_s_sleep(2);
  } while (!wait_expired(P, t0));
  return decide_seq<T>(P, sh, b);
}

// ---------------------------------------------------------------------------
// Draw chunks and the draw.

template <typename T>
struct DrawRows {
  const T* trow;
  const T* drow;
  double mt, md, inv_t;
  bool residual;
};

template <typename T>
__device__ __forceinline__ DrawRows<T> draw_rows(const Params P, int b, const SeqInfo& s) {
  const int N = P.n_draft;
  DrawRows<T> d;
  d.trow = static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + s.j) * P.vocab;
  d.drow = static_cast<const T*>(P.draft) + (int64_t(b) * N + min(s.j, N - 1)) * P.vocab;
  d.mt = s.m_target;
  d.md = s.m_draft;
  d.inv_t = 1.0 / double(P.temperature[b]);
  d.residual = (s.mode == kModeResidual);
  return d;
}

// Argument (z - max)/T of a token's exp; every step forms it the same way.
__device__ __forceinline__ double exp_arg(float z, double m, double inv_t) { return (double(z) - m) * inv_t; }

// Keeps the scheduler from interleaving the fp64 work of many tokens, which
// would hold their temporaries live at once and cost occupancy.
__device__ __forceinline__ void fp64_step_fence() { __builtin_amdgcn_sched_barrier(0); }

// Residual weight of a token from its exps and the reciprocal normalisers.
__device__ __forceinline__ double resid_weight(double et, double ed, double rt, double rd) {
  return fmax(0.0, et * rt - ed * rd);
}

// fp64 sums of draw chunk c of sequence b, written as a tagged record.
template <typename T>
__device__ __forceinline__ void norm_item(const Params P, Shared& sh, int b, int c, const DrawRows<T>& d, double log_rho) {
  DrawShared& ws = sh.u.drw;
  const int tid = threadIdx.x;
  const int e0 = c * kSampChunk + tid * kRun;
  float zt[kRun], zd[kRun];
  load_run(d.trow, e0, P.vocab, P.vec_ok != 0, zt);
  if (d.residual) load_run(d.drow, e0, P.vocab, P.vec_ok != 0, zd);
  double st = 0.0, sd = 0.0, sa = 0.0, sb = 0.0;
  int n_unc = 0;  // uncertain-sign tokens of this thread; the first kUncPerThread are staged
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    const double at = exp_arg(zt[k], d.mt, d.inv_t);
    const double et = exp_nonpos(at, sh.exp_table);
    st += et;
    if (d.residual) {
      const double ad = exp_arg(zd[k], d.md, d.inv_t);
      const double ed = exp_nonpos(ad, sh.exp_table);
      sd += ed;
      // at - ad is +inf when the draft gives the token zero mass.
      const double lr = at - ad;
      const bool pos = et > 0.0 && (ed == 0.0 || lr > log_rho + kSignBand);
      const bool band = et > 0.0 && !pos && lr >= log_rho - kSignBand;
      sa += pos ? et : 0.0;
      sb += pos ? ed : 0.0;
      if (band && n_unc < kUncPerThread) {
        ws.unc_et[n_unc][tid] = et;
        ws.unc_ed[n_unc][tid] = ed;
      }
      n_unc += band ? 1 : 0;
    }
    fp64_step_fence();
  }
  uint64_t* out = norm_at(P, b, c);
  st = block_sum(st, ws.red);
  int total = 0;
  if (d.residual) {
    sd = block_sum(sd, ws.red);
    sa = block_sum(sa, ws.red);
    sb = block_sum(sb, ws.red);
    // Uncertain tokens in ascending token order (threads own ascending runs),
    // with their exps; a thread past its staging capacity overflows the chunk.
    const int cnt = (n_unc <= kUncPerThread) ? n_unc : kUncMax + 1;
    int incl = cnt;
    const int lane = tid & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int up = __shfl_up(incl, off);
      if (lane >= off) incl += up;
    }
    if (lane == 63) ws.unc_base[tid >> 6] = incl;
    __syncthreads();
    int slot = incl - cnt;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      if (wv < (tid >> 6)) slot += ws.unc_base[wv];
      total += ws.unc_base[wv];
    }
    __syncthreads();
    if (total <= kUncMax) {
      for (int i = 0; i < cnt; ++i) {
        uint64_t* e = out + kNormHead + 4 * (slot + i);
        put_word_d(e, ws.unc_et[i][tid], P.epoch);
        put_word_d(e + 2, ws.unc_ed[i][tid], P.epoch);
      }
    }
  }
  if (tid == 0) {
    put_word_d(out, st, P.epoch);
    put_word_d(out + 2, sd, P.epoch);
    put_word_d(out + 4, sa, P.epoch);
    put_word_d(out + 6, sb, P.epoch);
    put_word(out + 8, uint32_t(total), P.epoch);
  }
}

// Weight sum of one chunk from its logits (after a rejection): used for
// chunks whose uncertain tokens overflowed their record.
template <typename T>
__device__ __forceinline__ double chunk_weight(const Params P, Shared& sh, int c, const DrawRows<T>& d, double rt, double rd) {
  const int e0 = c * kSampChunk + threadIdx.x * kRun;
  float zt[kRun], zd[kRun];
  load_run(d.trow, e0, P.vocab, P.vec_ok != 0, zt);
  load_run(d.drow, e0, P.vocab, P.vec_ok != 0, zd);
  double w = 0.0;
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    w += resid_weight(exp_nonpos(exp_arg(zt[k], d.mt, d.inv_t), sh.exp_table),
                      exp_nonpos(exp_arg(zd[k], d.md, d.inv_t), sh.exp_table), rt, rd);
    fp64_step_fence();
  }
  return block_sum(w, sh.u.drw.red);
}

// Sum of the chunk weights over all chunks, as a scan in groups of kThreads
// chunks (the order the crossing search uses).
__device__ __forceinline__ double weight_total(DrawShared& ws, int nsch) {
  double S = 0.0;
  for (int g = 0; g < nsch; g += kThreads) {
    const int cc = g + threadIdx.x;
    double tot;
    block_scan(cc < nsch ? ws.w[cc] : 0.0, tot, ws.red);
    S += tot;
  }
  return S;
}

// The draw for sequence b, by the workgroup of its last draw chunk.
template <typename T>
__device__ __forceinline__ void draw_seq(const Params P, Shared& sh, int b, const SeqInfo& s, const DrawRows<T>& d) {
  DrawShared& ws = sh.u.drw;
  const int tid = threadIdx.x;
  const int nsch = P.nsch;

  // Collect the chunk records: thread tid owns chunk tid. Every pass reads
  // them all afresh; past the wait bound the missing ones are computed here.
  double rz, rzd, ra, rb;
  int rn;
  const uint64_t t0 = wall_clock64();
  int rounds = 0;
  while (true) {
    bool ok = true;
    rz = rzd = ra = rb = 0.0;
    rn = 0;
    if (tid < nsch) {
      const uint64_t* w = norm_at(P, b, tid);
      rz = get_word_d(w, P.epoch, ok);
      rzd = get_word_d(w + 2, P.epoch, ok);
      ra = get_word_d(w + 4, P.epoch, ok);
      rb = get_word_d(w + 6, P.epoch, ok);
      rn = int(get_word(w + 8, P.epoch, ok));
      ws.flag[tid] = ok ? 0 : 1;
    }
    if (__syncthreads_and(ok)) break;
    if (!wait_expired(P, t0)) {
      __builtin_amdgcn_s_sleep(2);
      continue;
    }
    if (++rounds > kMaxRecomputeRounds) {
      // Unreachable unless the records are broken: fail the draw.
      if (tid == 0) P.out_tokens[int64_t(b) * (P.n_draft + 1) + s.j] = -1;
      return;
    }
    for (int cc = 0; cc < nsch; ++cc)
      if (ws.flag[cc]) norm_item<T>(P, sh, b, cc, d, s.log_rho);
    stores_done();
    __syncthreads();
  }
  double rt = 0.0, rd = 0.0;
  if (d.residual) {
    const double zt = block_sum(rz, ws.red);
    const double zd = block_sum(rzd, ws.red);
    rt = 1.0 / zt;
    rd = 1.0 / zd;
    const double rho = zt * rd;
    if (tid < nsch) {
      ws.w[tid] = rt * (ra - rho * rb);
      ws.flag[tid] = rn;
    }
    __syncthreads();
    // Exact terms of the uncertain tokens from their recorded exps: lane
    // group g of 16 takes chunk c0 + g, lane k its k-th token; a fixed
    // butterfly sums the group. A chunk whose entries are not all current
    // yet is retried, and past the wait bound recomputed from its logits.
    const int g = tid >> 4, k = tid & 15;
    const uint64_t t1 = wall_clock64();
    bool pending = true;
    while (pending) {
      bool stale = false;
      for (int c0 = 0; c0 < nsch; c0 += kThreads / 16) {
        const int cc = c0 + g;
        const int n = (cc < nsch) ? ws.flag[cc] : 0;
        double x = 0.0;
        bool ok = true;
        if (k < n && n <= kUncMax) {
          const uint64_t* e = norm_at(P, b, cc) + kNormHead + 4 * k;
          const double et = get_word_d(e, P.epoch, ok);
          const double ed = get_word_d(e + 2, P.epoch, ok);
          x = resid_weight(et, ed, rt, rd);
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
          x += __shfl_xor(x, off, 16);
          ok = ok && __shfl_xor(int(ok), off, 16);
        }
        stale = stale || !ok;
        if (k == 0 && n > 0 && n <= kUncMax && ok) {
          ws.w[cc] += x;
          ws.flag[cc] = 0;  // done
        }
      }
      pending = __syncthreads_or(stale);
      if (pending && wait_expired(P, t1)) {
        for (int cc = tid; cc < nsch; cc += kThreads)
          if (ws.flag[cc] > 0 && ws.flag[cc] <= kUncMax) ws.flag[cc] = kUncMax + 1;
        __syncthreads();
        pending = false;
      } else if (pending) {
        __builtin_amdgcn_s_sleep(2);
      }
    }
    // Chunks whose uncertain tokens overflowed their record: recompute.
    for (int cc = 0; cc < nsch; ++cc) {
      if (ws.flag[cc] > kUncMax) {
        const double wc = chunk_weight<T>(P, sh, cc, d, rt, rd);
        if (tid == 0) ws.w[cc] = wc;
      }
    }
  } else if (tid < nsch) {
    ws.w[tid] = rz;
  }
  __syncthreads();
  double S = weight_total(ws, nsch);
  bool fallback = false;
  if (d.residual && !(S > 0.0)) {
    // Every residual weight rounded to zero: draw from q_j itself, whose
    // chunk weights are the chunks' Zt scaled by 1/Zt.
    fallback = true;
    __syncthreads();
    if (tid < nsch) ws.w[tid] = rt * rz;
    __syncthreads();
    S = weight_total(ws, nsch);
  }
  const double target_mass = double(P.sample_u[b]) * S;
  // First chunk with positive weight whose inclusive prefix exceeds target_mass.
  double before = 0.0;
  int chunk = -1, last_pos = -1;
  for (int g = 0; g < nsch && chunk < 0; g += kThreads) {
    const int cc = g + tid;
    const double w = cc < nsch ? ws.w[cc] : 0.0;
    double tot;
    const double incl = before + block_scan(w, tot, ws.red);
    if (tid == 0) {
      ws.pick[0] = INT_MAX;
      ws.pick[1] = -1;
    }
    __syncthreads();
    if (cc < nsch && incl > target_mass && w > 0.0) atomicMin(&ws.pick[0], cc);
    if (cc < nsch && w > 0.0) atomicMax(&ws.pick[1], cc);
    __syncthreads();
    if (ws.pick[1] >= 0) last_pos = ws.pick[1];
    if (ws.pick[0] != INT_MAX) chunk = ws.pick[0];
    before += tot;
    __syncthreads();
  }
  if (chunk < 0) chunk = max(last_pos, 0);  // rounding left u*S at or past the total
  // Exclusive prefix of the chosen chunk, in the same group-scan order.
  before = 0.0;
  for (int g = 0; g < chunk; g += kThreads) {
    const int cc = g + tid;
    double tot;
    block_scan(cc < chunk ? ws.w[cc] : 0.0, tot, ws.red);
    before += tot;
  }
  // Rescan the chunk: thread tid owns kRun consecutive tokens; their weights
  // are formed twice (for the thread's sum, then for the walk) rather than kept.
  const int e_base = chunk * kSampChunk + tid * kRun;
  float zt[kRun], zd[kRun];
  load_run(d.trow, e_base, P.vocab, P.vec_ok != 0, zt);
  if (d.residual) load_run(d.drow, e_base, P.vocab, P.vec_ok != 0, zd);
  auto weight = [&](int k) {
    const double et = exp_nonpos(exp_arg(zt[k], d.mt, d.inv_t), sh.exp_table);
    if (!d.residual) return et;
    if (fallback) return et * rt;
    return resid_weight(et, exp_nonpos(exp_arg(zd[k], d.md, d.inv_t), sh.exp_table), rt, rd);
  };
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    run += weight(k);
    fp64_step_fence();
  }
  // Hide the logits' values from the optimiser so the walk recomputes the
  // weights instead of keeping all of them live from the first pass.
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    asm volatile("" : "+v"(zt[k]));
    if (d.residual) asm volatile("" : "+v"(zd[k]));
  }
  double tot;
  const double incl = block_scan(run, tot, ws.red);
  double cum = before + (incl - run);
  if (tid == 0) {
    ws.pick[0] = INT_MAX;
    ws.pick[1] = -1;
  }
  __syncthreads();
  int first = INT_MAX, last = -1;
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    const double wk = weight(k);
    cum += wk;
    if (first == INT_MAX && cum > target_mass && wk > 0.0) first = k;
    if (wk > 0.0) last = k;
    fp64_step_fence();
  }
  if (first != INT_MAX) atomicMin(&ws.pick[0], e_base + first);
  if (last >= 0) atomicMax(&ws.pick[1], e_base + last);
  __syncthreads();
  if (tid == 0) {
    int token = (ws.pick[0] != INT_MAX) ? ws.pick[0] : ws.pick[1];
    if (token < 0) token = 0;
    P.out_tokens[int64_t(b) * (P.n_draft + 1) + s.j] = token;
  }
}

// ---------------------------------------------------------------------------
// The launch.

template <typename T>
// At most 128 VGPRs (four waves per SIMD): the row-statistics workgroups
// stream with 32 KB each in flight, enough to keep HBM busy at this occupancy.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_kernel(Params P) {
  __shared__ Shared sh;
  trace(0);
  if (int(blockIdx.x) < P.n_stat_items) {
    const int R = 2 * P.n_draft + 1;
    const int item = blockIdx.x;
    const int row = item / P.nch;
    const int chunk = item - row * P.nch;
    const int b = row / R;
    const int r = row - b * R;
    const float t = P.temperature[b];
    if (temperature_valid(t) && !(t == 0.0f && r < P.n_draft))
      stat_item<T, kStatsChunkBytes / 16 / kThreads>(P, sh, b, r, chunk, t);
    trace(1);
    if (r == R - 1 && chunk == P.nch - 1) {
      __syncthreads();
      decide_seq<T>(P, sh, b);
      trace(2);
    }
    return;
  }
  const int k = int(blockIdx.x) - P.n_stat_items;
  const int b = k / P.nsch;
  const int c = k - b * P.nsch;
  if (threadIdx.x < kExpTableSize) sh.exp_table[threadIdx.x] = P.exp_table[threadIdx.x];
  const SeqInfo s = wait_seq<T>(P, sh, b);
  trace(1);
  if (s.mode == kModeNone) return;
  const DrawRows<T> d = draw_rows<T>(P, b, s);
  norm_item<T>(P, sh, b, c, d, s.log_rho);
  trace(2);
  if (c != P.nsch - 1) return;
  __syncthreads();
  draw_seq<T>(P, sh, b, s, d);
  trace(3);
}

const char* const kStageNames[] = {"verify"};
constexpr int kNumStages = 1;

template <typename T>
hipError_t launch_typed(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* ev) {
  const int R = 2 * a.n_draft + 1;
  Params p;
  p.draft = a.draft;
  p.target = a.target;
  p.tokens = a.tokens;
  p.accept_u = a.accept_u;
  p.sample_u = a.sample_u;
  p.temperature = a.temperature;
  p.out_tokens = a.out_tokens;
  p.out_n = a.out_n;
  p.row_lse = w.row_lse;
  p.row_argmax = w.row_argmax;
  p.partials = w.partials;
  p.seq = w.seq;
  p.norm = w.norm;
  p.exp_table = w.exp_table;
  p.wait_ticks = a.wait_ticks;
  p.epoch = a.epoch;
  p.n_draft = a.n_draft;
  p.vocab = a.vocab;
  p.nch = w.n_stats_chunks;
  p.chunk = w.stats_chunk;
  p.nsch = w.n_samp_chunks;
  p.vec_ok = (int64_t(a.vocab) * int64_t(sizeof(T))) % 16 == 0;
  p.n_stat_items = a.batch * R * p.nch;
  const int64_t blocks = int64_t(p.n_stat_items) + int64_t(a.batch) * p.nsch;
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  hipLaunchKernelGGL(verify_kernel<T>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p);
  if (ev != nullptr) (void)hipEventRecord(ev[1], stream);
  return hipGetLastError();
}

// Zeroes n 16-byte words (used when the call sequence number wraps).
__global__ void clear_kernel(uint4* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

const char* stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

hipError_t clear_records(void* mem, size_t bytes, hipStream_t stream) {
  const int64_t n = int64_t(bytes / 16);
  hipLaunchKernelGGL(clear_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(mem), n);
  return hipGetLastError();
}

#if defined(SPECV_TRACE)
// Copies the stamps of the last launches into out (kTraceBlocks * 8 words) and clears them.
extern "C" __attribute__((visibility("default"))) int specv_debug_trace(uint64_t* out, int64_t cap_words) {
  const size_t bytes = sizeof(g_trace);
  if (out == nullptr || cap_words * int64_t(sizeof(uint64_t)) < int64_t(bytes)) return -1;
  if (hipDeviceSynchronize() != hipSuccess) return -3;
  if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_trace), bytes, 0, hipMemcpyDeviceToHost) != hipSuccess) return -3;
  void* dev = nullptr;
  if (hipGetSymbolAddress(&dev, HIP_SYMBOL(g_trace)) != hipSuccess) return -3;
  if (hipMemset(dev, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) return -3;
  return 0;
}
#endif

hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* events,
                         int* n_stages) {
  if (n_stages != nullptr) *n_stages = kNumStages;
  if (a.dtype == 0) return launch_typed<float>(a, w, stream, events);
  return launch_typed<uint16_t>(a, w, stream, events);
}

}  // namespace specv
