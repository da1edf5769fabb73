// gfx950 kernels for batched speculative-sampling verification.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with "Step 1: 거절 단계" (the
// accept test) and "Step 2: 잔차 분포" (the residual); blog "…투기적 디코딩
// (Speculative Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// One launch per call. B sequences, N drafts, 2N+1 rows of V logits each.
// Two kinds of workgroups share the grid:
//   row statistics  one per (row, 64 KB chunk): fp32 max, sum of
//                   2^(z*c - fl(max*c)) with c = log2(e)/T, first argmax, and
//                   the logit at the row's draft token if the chunk holds it.
//                   Streaming and HBM-bound; greedy sequences skip draft rows.
//                   The sequence's last one (last chunk of target row N) then
//                   collects the sequence's row partials, merges them into
//                   log-normalisers, runs the N accept tests and writes the
//                   accepted prefix and a sequence record.
//   draw chunks     one per (sequence, 2048-logit chunk): waits for the
//                   sequence record, sums fp64 exps over its chunk of the
//                   row(s) the draw needs; the sequence's last one then
//                   collects the chunk sums, finds the chunk where the inverse
//                   CDF crosses u*S and rescans it in fp64.
// The grid holds every row-statistics workgroup first, then every draw-chunk
// workgroup; draw chunks of sequences decided early run while the last rows
// still stream.
//
// The residual weight of token x is w_x = max(0, et_x/Zt - ed_x/Zd)
// = max(0, et_x - rho*ed_x)/Zt with rho = Zt/Zd, so its sign only depends on
// whether log(et_x/ed_x) exceeds log(rho). The decision knows log(rho) from the
// fp32 row sums to a few 1e-6; a draw chunk treats tokens more than 1e-4 away from it
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
constexpr int kMaxRows = 2 * 64 + 1;
constexpr double kSignBand = 1e-4;      // |log(et/ed) - log(rho)| at or below this is uncertain
constexpr int kUncPerThread = 2;        // uncertain tokens a thread stages; more overflow the chunk
constexpr int kMaxRecomputeRounds = 3;  // a waiter's own recomputation always completes in one
static_assert(kMaxSampChunks <= kThreads, "the draw gives each thread at most one chunk");

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
  int batch;
  int n_draft;
  int vocab;
  int nch;     // row-statistics chunks per row
  int chunk;   // logits per row-statistics chunk
  int nsch;    // draw chunks per row
  int vec_ok;  // rows start 16-byte aligned
};

// Record layouts (64-bit tagged words).
//   row partial:  m, s, idx, logit at the row's draft token (when in the chunk)
//   sequence:     mode | j << 8, m_target, m_draft, log_rho (2 words)
//   draw chunk:   zt, zd, a, b (2 words each), n_unc, then per uncertain token et, ed (2 words each)
constexpr int kNormHead = 9;
static_assert(kNormHead + 4 * kUncMax <= kNormWords, "draw-chunk record layout");

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

constexpr int kStageParts = 1024;  // row partials the decision holds in LDS at once

struct DecideShared {
  float row_m[kMaxRows];
  double row_logz[kMaxRows];
  int row_idx[kMaxRows];
  float row_zg[kMaxRows];
  float part_m[kStageParts];
  float part_s[kStageParts];
  int part_idx[kStageParts];  // -1: the partial is not current yet
  float part_zg[kStageParts];
  unsigned long long rej_mask;
};

struct DrawShared {
  double red[4 * kWaves];
  int unc_base[kWaves];
  double unc_et[kUncPerThread][kThreads];
  double unc_ed[kUncPerThread][kThreads];
  int flag[kMaxSampChunks];  // chunk record still missing (collecting), or overflowed (recompute)
  double w[kThreads];        // chunk weights, then the rescanned chunk's per-thread sums
  int pick;
  double before;
};

struct Shared {
  double exp_table[kExpTableSize];
  StatShared st;
  union {
    DecideShared dec;
    DrawShared drw;
  } u;
};

// Sums four doubles over the workgroup in a fixed order.
__device__ __forceinline__ void block_sum4(double& a, double& b, double& c, double& d, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off);
    b += __shfl_xor(b, off);
    c += __shfl_xor(c, off);
    d += __shfl_xor(d, off);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    const int w = threadIdx.x >> 6;
    red[w] = a;
    red[kWaves + w] = b;
    red[2 * kWaves + w] = c;
    red[3 * kWaves + w] = d;
  }
  __syncthreads();
  a = red[0];
  b = red[kWaves];
  c = red[2 * kWaves];
  d = red[3 * kWaves];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    a += red[w];
    b += red[kWaves + w];
    c += red[2 * kWaves + w];
    d += red[3 * kWaves + w];
  }
}

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
//
// The normalisers come from fp32 row sums (relative error ~1e-6); logs and
// the ratio are taken in fp64, so log(rho) is good to a few 1e-6 (well inside
// the draw's sign band) and a decision can only differ from exact arithmetic
// when u is within a few 1e-6 of the ratio.
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
  // The row partials, a group of rows at a time: every thread loads partials
  // tid, tid + kThreads, ... of the group (one round trip per pass) until all
  // are current; past the wait bound the workgroup computes the missing ones
  // itself. Then waves merge rows wave, wave+4, ... of the group: lanes take
  // chunks lane, lane+64, ..., then a fixed butterfly.
  const int rows_per_group = max(1, kStageParts / P.nch);
  for (int rg = r_first; rg < R; rg += rows_per_group) {
    const int nr = min(rows_per_group, R - rg);
    const int np = nr * P.nch;
    const uint64_t t0 = wall_clock64();
    int rounds = 0;
    while (true) {
      bool ok = true;
      for (int i = tid; i < np; i += kThreads) {
        const int rr = i / P.nch;
        const uint64_t* w = partial_at(P, b, rg + rr, i - rr * P.nch);
        bool okp = true;
        ds.part_m[i] = get_word_f(w, P.epoch, okp);
        ds.part_s[i] = get_word_f(w + 1, P.epoch, okp);
        const int idx = int(get_word(w + 2, P.epoch, okp));
        ds.part_zg[i] = get_word_f(w + 3, P.epoch, okp);
        ds.part_idx[i] = okp ? idx : -1;
        ok = ok && okp;
      }
      if (__syncthreads_and(ok)) break;
      trace(5);
      if (!wait_expired(P, t0)) {
        __builtin_amdgcn_s_sleep(2);
        continue;
      }
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
      for (int i = 0; i < np; ++i) {
        if (ds.part_idx[i] < 0) {
          const int rr = i / P.nch;
          stat_item<T, 2>(P, sh, b, rg + rr, i - rr * P.nch, t);
        }
      }
      stores_done();
      __syncthreads();
    }
    for (int rr = wave; rr < nr; rr += kWaves) {
      const int r = rg + rr;
      float m = -INFINITY, s = 0.0f;
      int idx = INT_MAX;
      for (int k = lane; k < P.nch; k += 64) {
        const int i = rr * P.nch + k;
        if (greedy)
          acc_merge<false>(m, s, idx, ds.part_m[i], ds.part_s[i], ds.part_idx[i], c);
        else
          acc_merge<true>(m, s, idx, ds.part_m[i], ds.part_s[i], ds.part_idx[i], c);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const float s2 = __shfl_xor(s, off);
        const int i2 = __shfl_xor(idx, off);
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
        ds.row_zg[r] = (r < 2 * N) ? ds.part_zg[rr * P.nch + tok[r < N ? r : r - N] / P.chunk] : 0.0f;
        lse[r] = greedy ? NAN : float(double(m) * inv_t + logz);
        amax[r] = idx;
      }
    }
    __syncthreads();
  }
  trace(3);
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
      // log(q(d)/p(d)); the test is u < exp of it.
      const double lr = ((double(zt) - double(ds.row_m[N + tid])) - (double(zd) - double(ds.row_m[tid]))) * inv_t -
                        (ds.row_logz[N + tid] - ds.row_logz[tid]);
      accept = double(ua) < exp(lr);
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
  double nmt, nmd;  // -max/T of the target and draft rows
  double inv_t;
  bool residual;
};

template <typename T>
__device__ __forceinline__ DrawRows<T> draw_rows(const Params P, int b, const SeqInfo& s) {
  const int N = P.n_draft;
  DrawRows<T> d;
  d.trow = static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + s.j) * P.vocab;
  d.drow = static_cast<const T*>(P.draft) + (int64_t(b) * N + min(s.j, N - 1)) * P.vocab;
  d.inv_t = 1.0 / double(P.temperature[b]);
  d.nmt = -double(s.m_target) * d.inv_t;
  d.nmd = -double(s.m_draft) * d.inv_t;
  d.residual = (s.mode == kModeResidual);
  return d;
}

// Argument z/T - max/T of a token's exp; every step forms it the same way.
__device__ __forceinline__ double exp_arg(float z, double nm, double inv_t) { return fma(double(z), inv_t, nm); }

// Keeps the scheduler from interleaving the fp64 work of many tokens, which
// would hold their temporaries live at once and cost occupancy.
__device__ __forceinline__ void fp64_step_fence() { __builtin_amdgcn_sched_barrier(0); }

// Residual weight of a token from its exps and the reciprocal normalisers.
__device__ __forceinline__ double resid_weight(double et, double ed, double rt, double rd) {
  return fmax(0.0, et * rt - ed * rd);
}

// fp64 sums of draw chunk c of sequence b, written as a tagged record.
template <typename T>
__device__ __forceinline__ void norm_item(const Params P, Shared& sh, int b, int c, const DrawRows<T>& d,
                                          double log_rho) {
  DrawShared& ws = sh.u.drw;
  const int tid = threadIdx.x;
  const int e0 = c * kSampChunk + tid * kRun;
  float zt[kRun], zd[kRun];
  load_run(d.trow, e0, P.vocab, P.vec_ok != 0, zt);
  if (d.residual) load_run(d.drow, e0, P.vocab, P.vec_ok != 0, zd);
  // The sign of w_x follows (zt - zd)/T - (mt - md)/T against log(rho); fp32
  // gets it to ~1e-6 here, well inside the band.
  const float inv_tf = float(d.inv_t);
  const float dmf = float(d.nmt - d.nmd);  // -(mt - md)/T
  const float hi = float(log_rho + kSignBand), lo = float(log_rho - kSignBand);
  double st = 0.0, sd = 0.0, sa = 0.0, sb = 0.0;
  int n_unc = 0;  // uncertain-sign tokens of this thread; the first kUncPerThread are staged
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    const double et = exp_nonpos(exp_arg(zt[k], d.nmt, d.inv_t), sh.exp_table);
    st += et;
    if (d.residual) {
      const double ed = exp_nonpos(exp_arg(zd[k], d.nmd, d.inv_t), sh.exp_table);
      sd += ed;
      // +inf when the draft gives the token zero mass, NaN (neither side)
      // when both rows do: such a token adds nothing wherever it goes.
      const float lr = fmaf(zt[k] - zd[k], inv_tf, dmf);
      const bool pos = lr > hi;
      const bool band = !pos && lr >= lo;
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
  block_sum4(st, sd, sa, sb, ws.red);
  int total = 0;
  if (d.residual) {
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
__device__ __forceinline__ double chunk_weight(const Params P, Shared& sh, int c, const DrawRows<T>& d, double rt,
                                               double rd) {
  const int e0 = c * kSampChunk + threadIdx.x * kRun;
  float zt[kRun], zd[kRun];
  load_run(d.trow, e0, P.vocab, P.vec_ok != 0, zt);
  load_run(d.drow, e0, P.vocab, P.vec_ok != 0, zd);
  double w = 0.0;
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    w += resid_weight(exp_nonpos(exp_arg(zt[k], d.nmt, d.inv_t), sh.exp_table),
                      exp_nonpos(exp_arg(zd[k], d.nmd, d.inv_t), sh.exp_table), rt, rd);
    fp64_step_fence();
  }
  return block_sum(w, sh.u.drw.red);
}

// Crossing searches run by wave 0 over kThreads values v[0..kThreads): lane l
// owns v[4l..4l+3]. Lane sums (in order), a wave inclusive scan, then each
// lane walks its four values from its exclusive prefix.

// Inclusive wave scan of one double per lane (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(x, off);
    if (lane >= off) x += up;
  }
  return x;
}

// First index i with positive v[i] whose inclusive prefix exceeds target,
// else the last index with positive v[i], else 0; returns target - prefix
// before i through `rem` and the total through S. Uniform over wave 0.
__device__ __forceinline__ int find_crossing_abs(const double* v, int lane, double target, double& S, double& rem) {
  constexpr int kPer = kThreads / 64;
  double own = 0.0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) own += v[kPer * lane + q];
  const double incl = wave_scan(own, lane);
  S = __shfl(incl, 63);
  double pre = incl - own;  // exclusive prefix of this lane's values
  int cross = INT_MAX, lastpos = -1;
  double cross_pre = 0.0, last_pre = 0.0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = kPer * lane + q;
    const double x = v[i];
    if (x > 0.0) {
      if (cross == INT_MAX && pre + x > target) {
        cross = i;
        cross_pre = pre;
      }
      lastpos = i;
      last_pre = pre;
    }
    pre += x;
  }
  const unsigned long long has = __ballot(cross != INT_MAX);
  if (has) {
    const int src = __ffsll(has) - 1;
    const int i = __shfl(cross, src);
    rem = target - __shfl(cross_pre, src);
    return i;
  }
  const unsigned long long pos = __ballot(lastpos >= 0);
  if (pos) {
    const int src = 63 - __clzll(pos);
    const int i = __shfl(lastpos, src);
    rem = target - __shfl(last_pre, src);
    return i;
  }
  rem = target;
  return 0;
}

// The chunk search: target = u * S over the chunk weights.
__device__ __forceinline__ int find_crossing(const double* v, int lane, double u, double& S, double& rem) {
  constexpr int kPer = kThreads / 64;
  double own = 0.0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) own += v[kPer * lane + q];
  S = __shfl(wave_scan(own, lane), 63);
  double r;
  const int i = find_crossing_abs(v, lane, u * S, S, r);
  if (lane == 0) rem = r;
  return i;
}

// The draw for sequence b, by the workgroup of its last draw chunk.
template <typename T>
__device__ __forceinline__ void draw_seq(const Params P, Shared& sh, int b, const SeqInfo& s, const DrawRows<T>& d) {
  DrawShared& ws = sh.u.drw;
  const int tid = threadIdx.x;
  const int nsch = P.nsch;

  // Collect the chunk records with their uncertain-token entries: thread tid
  // owns chunk tid. Every pass reads them afresh; past the wait bound the
  // missing ones are computed here.
  const bool mine = tid < nsch;
  double rz, rzd, ra, rb;
  double uet[kUncMax], ued[kUncMax];
  int rn;
  const uint64_t t0 = wall_clock64();
  int rounds = 0;
  while (true) {
    bool ok = true;
    rz = rzd = ra = rb = 0.0;
    rn = 0;
    if (mine) {
      const uint64_t* w = norm_at(P, b, tid);
      rz = get_word_d(w, P.epoch, ok);
      rzd = get_word_d(w + 2, P.epoch, ok);
      ra = get_word_d(w + 4, P.epoch, ok);
      rb = get_word_d(w + 6, P.epoch, ok);
      rn = int(get_word(w + 8, P.epoch, ok));
#pragma unroll
      for (int k = 0; k < kUncMax; ++k) {
        bool okk = true;
        uet[k] = get_word_d(w + kNormHead + 4 * k, P.epoch, okk);
        ued[k] = get_word_d(w + kNormHead + 4 * k + 2, P.epoch, okk);
        // Only entries the record holds must be current (none when it overflowed).
        ok = ok && (okk || k >= rn || rn > kUncMax);
      }
      ws.flag[tid] = ok ? 0 : 1;
    }
    if (__syncthreads_and(ok)) break;
    trace(7);
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
  trace(4);
  double rt = 0.0, rd = 0.0;
  double wc = rz;  // bonus: the chunk's sum of exps
  if (d.residual) {
    double zt = rz, zd = rzd, unused0 = 0.0, unused1 = 0.0;
    block_sum4(zt, zd, unused0, unused1, ws.red);
    rt = 1.0 / zt;
    rd = 1.0 / zd;
    const double rho = zt * rd;
    wc = rt * (ra - rho * rb);
#pragma unroll
    for (int k = 0; k < kUncMax; ++k)
      if (k < rn) wc += resid_weight(uet[k], ued[k], rt, rd);
    // Chunks whose uncertain tokens overflowed their record: recompute.
    if (__syncthreads_or(mine && rn > kUncMax)) {
      if (mine) ws.flag[tid] = rn > kUncMax ? 1 : 0;
      __syncthreads();
      for (int cc = 0; cc < nsch; ++cc) {
        if (ws.flag[cc]) {
          const double w2 = chunk_weight<T>(P, sh, cc, d, rt, rd);
          if (tid == cc) wc = w2;
        }
      }
    }
  }
  if (!mine) wc = 0.0;
  trace(5);
  // Chunk search by wave 0: lane l sums chunks 4l..4l+3 in order, a wave scan
  // gives S and each lane's prefix, and the first chunk with positive weight
  // whose inclusive prefix exceeds u*S is the crossing.
  ws.w[tid] = wc;
  __syncthreads();
  bool fallback = false;
  if (tid < 64) {
    double S;
    int chunk = find_crossing(ws.w, tid, double(P.sample_u[b]), S, ws.before);
    // Every residual weight rounded to zero (S <= 0): flag the fallback.
    if (d.residual && !(S > 0.0)) chunk = -1;
    if (tid == 0) ws.pick = chunk;
  }
  __syncthreads();
  if (ws.pick < 0) {
    // Draw from q_j itself, whose chunk weights are the chunks' Zt scaled by 1/Zt.
    fallback = true;
    ws.w[tid] = mine ? rt * rz : 0.0;
    __syncthreads();
    if (tid < 64) {
      double S;
      const int chunk = find_crossing(ws.w, tid, double(P.sample_u[b]), S, ws.before);
      if (tid == 0) ws.pick = chunk;
    }
    __syncthreads();
  }
  const int chunk = ws.pick;
  const double target_mass = ws.before;  // mass still to cover inside the chunk
  __syncthreads();
  trace(6);
  // Rescan the chunk: thread tid owns kRun consecutive tokens; wave 0 finds
  // the thread whose run crosses, that thread the token.
  const int e_base = chunk * kSampChunk + tid * kRun;
  double w[kRun];
  double run = 0.0;
  {
    float zt[kRun], zd[kRun];
    load_run(d.trow, e_base, P.vocab, P.vec_ok != 0, zt);
    if (d.residual) load_run(d.drow, e_base, P.vocab, P.vec_ok != 0, zd);
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const double et = exp_nonpos(exp_arg(zt[k], d.nmt, d.inv_t), sh.exp_table);
      if (!d.residual)
        w[k] = et;
      else if (fallback)
        w[k] = et * rt;
      else
        w[k] = resid_weight(et, exp_nonpos(exp_arg(zd[k], d.nmd, d.inv_t), sh.exp_table), rt, rd);
      run += w[k];
      fp64_step_fence();
    }
  }
  ws.w[tid] = run;
  __syncthreads();
  if (tid < 64) {
    double S, rem;
    const int thr = find_crossing_abs(ws.w, tid, target_mass, S, rem);
    if (tid == 0) {
      ws.pick = thr;
      ws.before = rem;
    }
  }
  __syncthreads();
  if (tid == ws.pick) {
    // Walk this thread's run: first token with positive weight whose running
    // sum exceeds the remaining mass, else (rounding) the last positive one.
    const double rem = ws.before;
    double cum = 0.0;
    int token = -1, last = -1;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      cum += w[k];
      if (token < 0 && cum > rem && w[k] > 0.0) token = k;
      if (w[k] > 0.0) last = k;
    }
    const int k = token >= 0 ? token : last;
    P.out_tokens[int64_t(b) * (P.n_draft + 1) + s.j] = k >= 0 ? e_base + k : 0;
  }
}

// ---------------------------------------------------------------------------
// The launch.

// What workgroup x does: the row statistics of every sequence come first in
// the grid, then the draw chunks of every sequence, both in sequence order.
// (Draw chunks dispatched while rows still stream would take issue slots from
// the stream, whose ALU is already close to busy.)
struct Work {
  bool stat;
  int b;
  int idx;  // row-statistics item within the sequence (r * nch + chunk), or draw chunk
};

__device__ __forceinline__ Work work_of(const Params P, int x) {
  const int A = (2 * P.n_draft + 1) * P.nch;
  Work w;
  w.stat = x < P.batch * A;
  if (w.stat) {
    w.b = x / A;
    w.idx = x - w.b * A;
  } else {
    x -= P.batch * A;
    w.b = x / P.nsch;
    w.idx = x - w.b * P.nsch;
  }
  return w;
}

// Decisions and draws sit on the critical path of the sequences that finish
// last, while the CU is busy with other workgroups' streaming and fp64
// sums: their waves take issue priority.
__device__ __forceinline__ void critical_path() { __builtin_amdgcn_s_setprio(3); }

// At most 128 VGPRs (four waves per SIMD): row-statistics workgroups keep
// 64 KB each in flight, enough to keep HBM busy at this occupancy.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_kernel(Params P) {
  __shared__ Shared sh;
  trace(0);
  const Work wk = work_of(P, int(blockIdx.x));
  const int b = wk.b;
  if (wk.stat) {
    const int R = 2 * P.n_draft + 1;
    const int r = wk.idx / P.nch;
    const int chunk = wk.idx - r * P.nch;
    const float t = P.temperature[b];
    if (temperature_valid(t) && !(t == 0.0f && r < P.n_draft))
      stat_item<T, kStatsChunkBytes / 16 / kThreads>(P, sh, b, r, chunk, t);
    trace(1);
    if (r == R - 1 && chunk == P.nch - 1) {
      critical_path();
      __syncthreads();
      decide_seq<T>(P, sh, b);
      trace(2);
    }
    return;
  }
  const int c = wk.idx;
  for (int i = threadIdx.x; i < kExpTableSize; i += kThreads) sh.exp_table[i] = P.exp_table[i];
  const SeqInfo s = wait_seq<T>(P, sh, b);
  trace(1);
  if (s.mode == kModeNone) return;
  const DrawRows<T> d = draw_rows<T>(P, b, s);
  norm_item<T>(P, sh, b, c, d, s.log_rho);
  trace(2);
  if (c != P.nsch - 1) return;
  critical_path();
  __syncthreads();
  draw_seq<T>(P, sh, b, s, d);
  trace(3);
}

const char* const kStageNames[] = {"verify"};
constexpr int kNumStages = 1;

template <typename T>
hipError_t launch_typed(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* ev) {
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
  p.batch = a.batch;
  p.n_draft = a.n_draft;
  p.vocab = a.vocab;
  p.nch = w.n_stats_chunks;
  p.chunk = w.stats_chunk;
  p.nsch = w.n_samp_chunks;
  p.vec_ok = (int64_t(a.vocab) * int64_t(sizeof(T))) % 16 == 0;
  const int64_t blocks = grid_blocks(a.batch, a.n_draft, p.nch, p.nsch);
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

int64_t grid_blocks(int batch, int n_draft, int n_stats_chunks, int n_samp_chunks) {
  return int64_t(batch) * (int64_t(2 * n_draft + 1) * n_stats_chunks + n_samp_chunks);
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
