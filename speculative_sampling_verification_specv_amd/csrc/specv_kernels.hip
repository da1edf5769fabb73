// gfx950 kernel for batched speculative-sampling verification: one persistent launch.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with "Step 1: 거절 단계" (the
// accept test) and "Step 2: 잔차 분포" (the residual); blog "…투기적 디코딩
// (Speculative Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// Work items, per sequence b (B sequences, N drafts, 2N+1 rows of V logits):
//   STAT(b, r, c)  fp32 (max, sum 2^(z*c - K), first argmax) of 8192 logits of row r.
//   DECIDE(b)      merge STAT partials into per-row log-normalisers, run the N
//                  accept tests in fp64, find the first rejection j.
//   NORM(b, c)     fp64 exp of 4096 logits of the row(s) the draw needs. After a
//                  rejection: fp64 sums Zt, Zd of exp((z - max)/T) over target and
//                  draft row j, and the sums A, B of the same over the tokens whose
//                  residual weight is certainly positive, plus the indices of the
//                  few tokens whose sign is uncertain (see below). For the bonus:
//                  the sum of exp((z - max)/T) over target row N.
//   DRAW(b)        chunk weights, inverse CDF over them, an fp64 rescan of the
//                  crossing chunk, the token.
// Items are laid out in slots, sequence-major, with DECIDE, NORM and DRAW of
// sequence b placed a few sequences after STAT(b, ...); slot s belongs to
// workgroup s mod G, so the draw's fp64 work overlaps later sequences' HBM
// streaming.
//
// The residual weight of token x is w_x = max(0, et_x/Zt - ed_x/Zd)
// = max(0, et_x - rho*ed_x)/Zt with rho = Zt/Zd, so its sign only depends on
// whether log(et_x/ed_x) exceeds log(rho). DECIDE knows log(rho) from the fp32
// row sums to ~1e-6; NORM treats tokens more than 1e-4 away from it as certain
// and sums their exps into A and B, so that a chunk's weight is (A - rho*B)/Zt
// plus the exact terms of its uncertain tokens. No chunk has to wait for the
// global normalisers.
//
// Communication between workgroups uses no fences and no read-modify-write
// atomics (both are very slow across this GPU's per-XCD L2 caches). Each result
// travels in 64-bit words written and read with relaxed agent-scope atomics
// (single-copy atomic, coherent across XCDs); every word carries the call's
// 16-bit epoch, so a reader knows a word is from this call without any reset.
// A reader polls until all the words it needs carry the epoch. If that takes
// longer than a timeout (the producer's workgroup may not be resident), it
// computes the missing items itself: every item is a deterministic function of
// the inputs, so a duplicate write stores identical bits. Progress therefore
// never depends on workgroups being co-resident.
//
// Every reduction has a fixed order, so results are bitwise reproducible.

#include <float.h>
#include <limits.h>
#include <math.h>

#include <numeric>

#include "specv_internal.h"
#include "specv_math.h"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;
constexpr float kFltMax = 3.402823466e38f;
constexpr int kWaves = kThreads / 64;
constexpr int kSampPer = kSampChunk / kThreads;  // logits per thread in a NORM item
constexpr int kMaxRows = 2 * 64 + 1;
constexpr int kUncMax = 16;                      // uncertain tokens a NORM item records
constexpr int kNormWords = 9 + kUncMax;          // Zt, Zd, A, B (2 words each), count, indices
constexpr int kSeqWords = 4;
constexpr double kSignBand = 1e-4;               // |log(et/ed) - log(rho)| below this is uncertain
constexpr int kStageCap = 1024;                  // STAT partials DECIDE stages in LDS

__device__ __forceinline__ bool temperature_valid(float t) {
  return t == 0.0f || (t >= kMinTemperature && t <= kFltMax);
}

// c in 2^(z*c) == exp(z/T); finite for T >= kMinTemperature.
__device__ __forceinline__ float exp2_coef(float t) { return kLog2e / t; }

// K = fl(m * c), never contracted into a neighbouring add.
__device__ __forceinline__ float scaled_max(float m, float c) { return __fmul_rn(m, c); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---------------------------------------------------------------------------
// Epoch-tagged words.

__device__ __forceinline__ void publish(uint64_t* p, uint64_t payload48, unsigned epoch) {
  __hip_atomic_store(p, (payload48 << 16) | (epoch & 0xffffu), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(uint64_t w, unsigned epoch) { return (w & 0xffffu) == (epoch & 0xffffu); }
__device__ __forceinline__ uint64_t payload(uint64_t w) { return w >> 16; }

// STAT partial: (m, s, idx) in two words.
__device__ __forceinline__ void publish_partial(uint64_t* w, float m, float s, int idx, unsigned epoch) {
  const uint32_t mb = __float_as_uint(m), sb = __float_as_uint(s);
  publish(w, (uint64_t(mb) << 16) | (sb >> 16), epoch);
  publish(w + 1, (uint64_t(sb & 0xffffu) << 32) | uint32_t(idx), epoch);
}
__device__ __forceinline__ void unpack_partial(uint64_t w0, uint64_t w1, float& m, float& s, int& idx) {
  const uint64_t p0 = payload(w0), p1 = payload(w1);
  m = __uint_as_float(uint32_t(p0 >> 16));
  s = __uint_as_float((uint32_t(p0 & 0xffffu) << 16) | uint32_t(p1 >> 32));
  idx = int(uint32_t(p1 & 0xffffffffu));
}

// fp64 value in two words.
__device__ __forceinline__ void publish_f64(uint64_t* w, double v, unsigned epoch) {
  const uint64_t b = double_to_bits(v);
  publish(w, b >> 32, epoch);
  publish(w + 1, b & 0xffffffffu, epoch);
}
__device__ __forceinline__ double unpack_f64(uint64_t w0, uint64_t w1) {
  return bits_to_double((payload(w0) << 32) | (payload(w1) & 0xffffffffu));
}

// What DECIDE leaves for the draw of one sequence.
struct SeqInfo {
  int mode;  // SeqMode
  int j;
  float m_target;  // largest logit of target row j
  float m_draft;   // largest logit of draft row j (residual only)
  double log_rho;  // log(Zt/Zd) from the fp32 row sums (residual only)
};
__device__ __forceinline__ void publish_seq(uint64_t* w, const SeqInfo& s, unsigned epoch) {
  publish(w, (uint64_t(__float_as_uint(s.m_target)) << 16) | (uint64_t(s.j & 0xff) << 8) | uint64_t(s.mode & 0xff),
          epoch);
  publish(w + 1, uint64_t(__float_as_uint(s.m_draft)) << 16, epoch);
  publish_f64(w + 2, s.log_rho, epoch);
}
__device__ __forceinline__ SeqInfo unpack_seq(uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3) {
  SeqInfo s;
  const uint64_t p0 = payload(w0);
  s.m_target = __uint_as_float(uint32_t(p0 >> 16));
  s.j = int((p0 >> 8) & 0xff);
  s.mode = int(p0 & 0xff);
  s.m_draft = __uint_as_float(uint32_t(payload(w1) >> 16));
  s.log_rho = unpack_f64(w2, w3);
  return s;
}

// ---------------------------------------------------------------------------
// Kernel parameters and shared memory.

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
  uint64_t* stat_words;  // [B*R][nch][2]
  uint64_t* seq_words;   // [B][kSeqWords]
  uint64_t* norm_words;  // [B][nsch][kNormWords]
  const double* exp_table;
  int batch;
  int n_draft;
  int vocab;
  int nch;
  int nsch;
  int spg;  // slots per group
  long long total_slots;
  int lag_decide;
  int lag_norm;
  int lag_draw;
  unsigned epoch;
  unsigned long long timeout_ticks;
#ifdef SPECV_TRACE
  unsigned long long* trace;  // [total_slots][4]: kind|block<<8, start, end, wait ticks|timeouts<<48
  long long trace_slots;
#endif
};

struct Shared {
  double exp_table[kExpTableSize];
  double red[kWaves * 2];
  float row_m[kMaxRows];
  double row_logz[kMaxRows];
  int row_idx[kMaxRows];
  int flag;
  int pick[2];
  int unc_base[kWaves];
  // DECIDE stages STAT partials here; DRAW keeps chunk weights and flags here.
  union {
    struct {
      float m[kStageCap];
      float s[kStageCap];
      int idx[kStageCap];
    } part;
    struct {
      double w[kMaxSampChunks];
      int dirty[kMaxSampChunks];
    } draw;
  } u;
#ifdef SPECV_TRACE
  unsigned long long wait_ticks;
  unsigned long long timeouts;
#endif
};

__device__ __forceinline__ double block_sum(double v, Shared& sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  double total = sh.red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) total += sh.red[w];
  return total;
}

// Block-wide inclusive scan of one double per thread (fixed order); returns
// the thread's inclusive prefix and sets total.
__device__ __forceinline__ double block_scan(double v, double& total, Shared& sh) {
  const int lane = threadIdx.x & 63;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  __syncthreads();
  if (lane == 63) sh.red[threadIdx.x >> 6] = incl;
  __syncthreads();
  double before = 0.0;
  total = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < (int(threadIdx.x) >> 6)) before += sh.red[w];
    total += sh.red[w];
  }
  return before + incl;
}

__device__ __forceinline__ void note_wait(Shared& sh, unsigned long long t0, bool timed_out) {
#ifdef SPECV_TRACE
  if (threadIdx.x == 0) {
    sh.wait_ticks += wall_clock64() - t0;
    sh.timeouts += timed_out ? 1 : 0;
  }
#endif
}

// True (in every thread) once all n words carry the epoch; false on timeout.
__device__ bool block_wait(uint64_t* words, int n, const Params P, Shared& sh) {
  const unsigned long long t0 = wall_clock64();
  while (true) {
    bool ok = true;
    for (int i = threadIdx.x; i < n; i += kThreads) ok = ok && tagged(fetch(words + i), P.epoch);
    if (__syncthreads_and(ok)) {
      note_wait(sh, t0, false);
      return true;
    }
    const bool expired = (wall_clock64() - t0) > P.timeout_ticks;
    if (__syncthreads_or(expired)) {
      note_wait(sh, t0, true);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// True (in every thread) if the k words at p all carry the epoch.
__device__ bool block_has(uint64_t* p, int k, const Params P, Shared& sh) {
  __syncthreads();
  if (threadIdx.x == 0) {
    bool ok = true;
    for (int i = 0; i < k; ++i) ok = ok && tagged(fetch(p + i), P.epoch);
    sh.flag = ok;
  }
  __syncthreads();
  return sh.flag != 0;
}

// ---------------------------------------------------------------------------
// STAT: fp32 row statistics of one chunk.

// Running state: m = largest logit seen, idx = its first index, s = sum of
// 2^(z*c - k) with k = fl(m*c) once a finite logit was seen (0 before, while
// s is 0 too). The exact product m*c differs from k by r = fma(m, c, -k); the
// decision step removes it.
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

template <typename T, bool kSampled>
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
  // A chunk holds at most kMaxVec 16-byte vectors per thread: issue all loads
  // before any use so they are in flight together.
  constexpr int kMaxVec = kStatsChunk / kVec / kThreads;
  const uint4* __restrict__ vrow = reinterpret_cast<const uint4*>(row + ea);
  uint4 x[kMaxVec];
#pragma unroll
  for (int u = 0; u < kMaxVec; ++u) {
    const int k = tid + u * kThreads;
    if (k < nv) x[u] = vrow[k];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < kMaxVec; ++u) {
    const int k = tid + u * kThreads;
    if (k < nv) {
      float v[kVec];
      Logit<T>::unpack(x[u], v);
      acc_values<kSampled>(a, v, ea + k * kVec, c);
    }
  }
  if (tid < e1 - et) {
    const float v[1] = {Logit<T>::at(row, et + tid)};
    acc_values<kSampled>(a, v, et + tid, c);
  }
}

template <bool kSampled>
__device__ __forceinline__ void block_merge(StatAcc& a, float c, Shared& sh) {
  float m = a.m, s = a.s;
  int idx = a.idx;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    const int i2 = __shfl_xor(idx, off);
    acc_merge<kSampled>(m, s, idx, m2, s2, i2, c);
  }
  float* sm = reinterpret_cast<float*>(sh.red);  // 4 floats m, 4 floats s, 4 ints idx fit in red[8]
  float* ss = sm + kWaves;
  int* si = reinterpret_cast<int*>(ss + kWaves);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sm[threadIdx.x >> 6] = m;
    ss[threadIdx.x >> 6] = s;
    si[threadIdx.x >> 6] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0];
    s = ss[0];
    idx = si[0];
    for (int w = 1; w < kWaves; ++w) acc_merge<kSampled>(m, s, idx, sm[w], ss[w], si[w], c);
    a.m = m;
    a.s = s;
    a.idx = idx;
  }
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const Params P, int b, int r, int64_t& row_flat) {
  const int N = P.n_draft;
  if (r < N) {
    row_flat = (int64_t(b) * N + r) * P.vocab;
    return static_cast<const T*>(P.draft) + row_flat;
  }
  row_flat = (int64_t(b) * (N + 1) + (r - N)) * P.vocab;
  return static_cast<const T*>(P.target) + row_flat;
}

// Computes and publishes STAT(b, r, chunk); t is sequence b's temperature.
// Skips rows the sequence never needs.
template <typename T>
__device__ void stat_item(const Params P, Shared& sh, int b, int r, int chunk, float t) {
  if (!temperature_valid(t)) return;
  const bool greedy = (t == 0.0f);
  if (greedy && r < P.n_draft) return;
  int64_t row_flat;
  const T* rowp = row_ptr<T>(P, b, r, row_flat);
  const int e0 = chunk * kStatsChunk;
  const int e1 = min(P.vocab, e0 + kStatsChunk);
  StatAcc a;
  acc_init(a);
  if (greedy) {
    stats_chunk<T, false>(rowp, row_flat, e0, e1, 0.0f, a);
    block_merge<false>(a, 0.0f, sh);
  } else {
    const float c = exp2_coef(t);
    stats_chunk<T, true>(rowp, row_flat, e0, e1, c, a);
    block_merge<true>(a, c, sh);
  }
  if (threadIdx.x == 0) {
    const int R = 2 * P.n_draft + 1;
    publish_partial(P.stat_words + ((int64_t(b) * R + r) * P.nch + chunk) * 2, a.m, a.s, a.idx, P.epoch);
  }
}

// ---------------------------------------------------------------------------
// DECIDE: log-normalisers, accept tests, first rejection, outputs.

// Waits for (or computes) the STAT partials of rows [r0, R); when they fit,
// leaves them unpacked in shared memory (returns true).
template <typename T>
__device__ bool gather_stats(const Params P, Shared& sh, int b, int r0, float t) {
  const int R = 2 * P.n_draft + 1;
  const int n_part = (R - r0) * P.nch;
  uint64_t* base = P.stat_words + (int64_t(b) * R + r0) * P.nch * 2;
  const bool staged = n_part <= kStageCap;
  const unsigned long long t0 = wall_clock64();
  bool waited_out = false;
  while (true) {
    bool ok = true;
    for (int i = threadIdx.x; i < n_part; i += kThreads) {
      const uint64_t w0 = fetch(base + 2 * i), w1 = fetch(base + 2 * i + 1);
      ok = ok && tagged(w0, P.epoch) && tagged(w1, P.epoch);
      if (staged) unpack_partial(w0, w1, sh.u.part.m[i], sh.u.part.s[i], sh.u.part.idx[i]);
    }
    if (__syncthreads_and(ok)) break;
    const bool expired = (wall_clock64() - t0) > P.timeout_ticks;
    if (__syncthreads_or(expired)) {
      waited_out = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  note_wait(sh, t0, waited_out);
  if (waited_out) {
    for (int r = r0; r < R; ++r)
      for (int c = 0; c < P.nch; ++c)
        if (!block_has(P.stat_words + ((int64_t(b) * R + r) * P.nch + c) * 2, 2, P, sh)) stat_item<T>(P, sh, b, r, c, t);
    __syncthreads();
    if (staged) {
      for (int i = threadIdx.x; i < n_part; i += kThreads)
        unpack_partial(fetch(base + 2 * i), fetch(base + 2 * i + 1), sh.u.part.m[i], sh.u.part.s[i],
                       sh.u.part.idx[i]);
    }
  }
  __syncthreads();
  return staged;
}

template <typename T>
__device__ void decide_item(const Params P, Shared& sh, int b) {
  const int N = P.n_draft;
  const int R = 2 * N + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int* tok = P.tokens + int64_t(b) * N;
  int* otok = P.out_tokens + int64_t(b) * (N + 1);
  float* lse = P.row_lse + int64_t(b) * R;
  int* amax = P.row_argmax + int64_t(b) * R;
  uint64_t* seqw = P.seq_words + int64_t(b) * kSeqWords;

  // Issue the inputs of the accept tests before waiting for the row sums.
  const float t = P.temperature[b];
  int d = 0;
  float zt = 0.0f, zd = 0.0f, ua = 0.0f;
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
      SeqInfo s{kModeNone, 0, 0.0f, 0.0f, 0.0};
      publish_seq(seqw, s, P.epoch);
    }
    return;
  }
  const bool greedy = (t == 0.0f);
  if (tid < N && !greedy) {
    zt = Logit<T>::at(static_cast<const T*>(P.target), (int64_t(b) * (N + 1) + tid) * P.vocab + d);
    zd = Logit<T>::at(static_cast<const T*>(P.draft), (int64_t(b) * N + tid) * P.vocab + d);
  }
  const int r_first = greedy ? N : 0;
  const bool staged = gather_stats<T>(P, sh, b, r_first, t);
  const float c = greedy ? 0.0f : exp2_coef(t);
  const double inv_t = greedy ? 0.0 : 1.0 / double(t);

  // Merge each row's chunk partials: lanes take chunks lane, lane+64, ...,
  // then a butterfly; waves take rows wave, wave+4, ...
  for (int r = wave; r < R; r += kWaves) {
    if (r < r_first) {
      if (lane == 0) {
        lse[r] = NAN;
        amax[r] = -1;
      }
      continue;
    }
    uint64_t* rw = P.stat_words + (int64_t(b) * R + r) * P.nch * 2;
    const int pbase = (r - r_first) * P.nch;
    float m = -INFINITY, s = 0.0f;
    int idx = INT_MAX;
    for (int k = lane; k < P.nch; k += 64) {
      float m2, s2;
      int i2;
      if (staged) {
        m2 = sh.u.part.m[pbase + k];
        s2 = sh.u.part.s[pbase + k];
        i2 = sh.u.part.idx[pbase + k];
      } else {
        unpack_partial(fetch(rw + 2 * k), fetch(rw + 2 * k + 1), m2, s2, i2);
      }
      if (greedy)
        acc_merge<false>(m, s, idx, m2, s2, i2, c);
      else
        acc_merge<true>(m, s, idx, m2, s2, i2, c);
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
      sh.row_m[r] = m;
      sh.row_logz[r] = logz;
      sh.row_idx[r] = idx;
      lse[r] = greedy ? NAN : float(double(m) * inv_t + logz);
      amax[r] = idx;
    }
  }
  __syncthreads();

  if (wave == 0) {
    bool accept = true;
    if (lane < N) {
      if (greedy) {
        accept = (d == sh.row_idx[N + lane]);
      } else if (zd == -INFINITY) {
        accept = true;  // p(d) == 0: the ratio is infinite
      } else {
        const double log_q = (double(zt) - double(sh.row_m[N + lane])) * inv_t - sh.row_logz[N + lane];
        const double log_p = (double(zd) - double(sh.row_m[lane])) * inv_t - sh.row_logz[lane];
        accept = double(ua) < exp(log_q - log_p);
      }
    }
    const unsigned long long rej = __ballot(lane < N && !accept);
    const int j = rej ? (__ffsll(rej) - 1) : N;
    // Position j of a sampled sequence is left to DRAW: a duplicate DECIDE
    // running after it must not overwrite the drawn token.
    for (int i = lane; i <= N; i += 64) {
      if (i < j)
        otok[i] = tok[i];
      else if (i > j)
        otok[i] = -1;
      else if (greedy)
        otok[i] = sh.row_idx[N + j];
    }
    if (lane == 0) {
      P.out_n[b] = j;
      SeqInfo s;
      s.mode = greedy ? kModeNone : (j < N ? kModeResidual : kModeBonus);
      s.j = j;
      s.m_target = sh.row_m[N + j];
      s.m_draft = (j < N && !greedy) ? sh.row_m[j] : 0.0f;
      s.log_rho = (j < N && !greedy) ? sh.row_logz[N + j] - sh.row_logz[j] : 0.0;
      publish_seq(seqw, s, P.epoch);
    }
  }
  __syncthreads();
}

template <typename T>
__device__ SeqInfo ensure_decided(const Params P, Shared& sh, int b) {
  uint64_t* w = P.seq_words + int64_t(b) * kSeqWords;
  if (!block_wait(w, kSeqWords, P, sh)) decide_item<T>(P, sh, b);
  return unpack_seq(fetch(w), fetch(w + 1), fetch(w + 2), fetch(w + 3));
}

// ---------------------------------------------------------------------------
// Draw: fp64 exps, chunk sums, inverse CDF.

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

// Arguments (z - max)/T of token e's exps; -inf past the row end.
template <typename T>
__device__ __forceinline__ void draw_args(const DrawRows<T>& d, int e, int vocab, double& at, double& ad) {
  at = -INFINITY;
  ad = -INFINITY;
  if (e < vocab) {
    at = (double(Logit<T>::at(d.trow, e)) - d.mt) * d.inv_t;
    if (d.residual) ad = (double(Logit<T>::at(d.drow, e)) - d.md) * d.inv_t;
  }
}

// Residual weight of a token from its exps and the reciprocal normalisers.
__device__ __forceinline__ double resid_weight(double et, double ed, double rt, double rd) {
  return fmax(0.0, et * rt - ed * rd);
}

// NORM(b, c): publishes Zt, Zd, A, B and the uncertain tokens of one chunk
// (bonus: only Zt, the chunk's weight).
template <typename T>
__device__ void norm_compute(const Params P, Shared& sh, int b, int c, const DrawRows<T>& d, double log_rho) {
  const int tid = threadIdx.x;
  double zt = 0.0, zd = 0.0, sa = 0.0, sb = 0.0;
  uint32_t unc = 0;  // bit k: token c*kSampChunk + tid + k*kThreads is uncertain
#pragma unroll
  for (int k = 0; k < kSampPer; ++k) {
    double at, ad;
    draw_args(d, c * kSampChunk + tid + k * kThreads, P.vocab, at, ad);
    const double et = exp_nonpos(at, sh.exp_table);
    zt += et;
    if (d.residual) {
      const double ed = exp_nonpos(ad, sh.exp_table);
      zd += ed;
      if (et > 0.0) {
        const double lr = at - ad;  // +inf when the draft gives the token zero mass
        if (ed == 0.0 || lr > log_rho + kSignBand) {
          sa += et;
          sb += ed;
        } else if (lr >= log_rho - kSignBand) {
          unc |= 1u << k;
        }
      }
    }
  }
  zt = block_sum(zt, sh);
  uint64_t* w = P.norm_words + (int64_t(b) * P.nsch + c) * kNormWords;
  if (!d.residual) {
    if (tid == 0) publish_f64(w, zt, P.epoch);
    __syncthreads();
    return;
  }
  zd = block_sum(zd, sh);
  sa = block_sum(sa, sh);
  sb = block_sum(sb, sh);
  // Uncertain tokens, listed in (thread, k) order.
  const int cnt = __popc(unc);
  int incl = cnt;
  const int lane = tid & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  __syncthreads();
  if (lane == 63) sh.unc_base[tid >> 6] = incl;
  __syncthreads();
  int slot = incl - cnt, total = 0;
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wv < (tid >> 6)) slot += sh.unc_base[wv];
    total += sh.unc_base[wv];
  }
  if (total <= kUncMax) {
#pragma unroll
    for (int k = 0; k < kSampPer; ++k)
      if (unc & (1u << k)) publish(w + 9 + slot++, uint64_t(c * kSampChunk + tid + k * kThreads), P.epoch);
  }
  if (tid == 0) {
    publish_f64(w, zt, P.epoch);
    publish_f64(w + 2, zd, P.epoch);
    publish_f64(w + 4, sa, P.epoch);
    publish_f64(w + 6, sb, P.epoch);
    publish(w + 8, uint64_t(total), P.epoch);
    // Unused index words still need the epoch: a reader waits on all of them.
    for (int k = min(total, kUncMax); k < kUncMax; ++k) publish(w + 9 + k, 0, P.epoch);
  }
  __syncthreads();
}

template <typename T>
__device__ void norm_item(const Params P, Shared& sh, int b, int c) {
  const SeqInfo s = ensure_decided<T>(P, sh, b);
  if (s.mode == kModeNone) return;
  norm_compute<T>(P, sh, b, c, draw_rows<T>(P, b, s), s.log_rho);
}

// Weight sum of one chunk from its logits (after a rejection): used for
// chunks with too many uncertain tokens.
template <typename T>
__device__ double chunk_weight(const Params P, Shared& sh, int c, const DrawRows<T>& d, double rt, double rd) {
  double w = 0.0;
#pragma unroll
  for (int k = 0; k < kSampPer; ++k) {
    double at, ad;
    draw_args(d, c * kSampChunk + threadIdx.x + k * kThreads, P.vocab, at, ad);
    w += resid_weight(exp_nonpos(at, sh.exp_table), exp_nonpos(ad, sh.exp_table), rt, rd);
  }
  return block_sum(w, sh);
}

// DRAW(b): chunk weights, the crossing chunk, an fp64 scan of it.
template <typename T>
__device__ void draw_item(const Params P, Shared& sh, int b) {
  const SeqInfo s = ensure_decided<T>(P, sh, b);
  if (s.mode == kModeNone) return;
  DrawRows<T> d = draw_rows<T>(P, b, s);
  const int tid = threadIdx.x;
  const int nsch = P.nsch;
  uint64_t* nw = P.norm_words + int64_t(b) * nsch * kNormWords;
  const int words_per_chunk = d.residual ? kNormWords : 2;
  // Wait for every chunk's NORM words (bonus: the first two of each chunk).
  {
    const unsigned long long t0 = wall_clock64();
    bool waited_out = false;
    while (true) {
      bool ok = true;
      for (int i = tid; i < nsch * words_per_chunk; i += kThreads) {
        const int cc = i / words_per_chunk, k = i - cc * words_per_chunk;
        ok = ok && tagged(fetch(nw + cc * kNormWords + k), P.epoch);
      }
      if (__syncthreads_and(ok)) break;
      const bool expired = (wall_clock64() - t0) > P.timeout_ticks;
      if (__syncthreads_or(expired)) {
        waited_out = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    note_wait(sh, t0, waited_out);
    if (waited_out) {
      for (int cc = 0; cc < nsch; ++cc)
        if (!block_has(nw + cc * kNormWords, words_per_chunk, P, sh)) norm_compute<T>(P, sh, b, cc, d, s.log_rho);
      __syncthreads();
    }
  }
  // Normalisers (fixed order) and the chunk weights.
  double rt = 0.0, rd = 0.0, rho = 0.0;
  if (d.residual) {
    double zt = 0.0, zd = 0.0;
    for (int cc = tid; cc < nsch; cc += kThreads) {
      zt += unpack_f64(fetch(nw + cc * kNormWords), fetch(nw + cc * kNormWords + 1));
      zd += unpack_f64(fetch(nw + cc * kNormWords + 2), fetch(nw + cc * kNormWords + 3));
    }
    zt = block_sum(zt, sh);
    zd = block_sum(zd, sh);
    rt = 1.0 / zt;
    rd = 1.0 / zd;
    rho = zt * rd;
  }
  for (int cc = tid; cc < nsch; cc += kThreads) {
    uint64_t* w = nw + cc * kNormWords;
    double wc = unpack_f64(fetch(w), fetch(w + 1));
    int dirty = 0;
    if (d.residual) {
      const double sa = unpack_f64(fetch(w + 4), fetch(w + 5));
      const double sb = unpack_f64(fetch(w + 6), fetch(w + 7));
      const int nu = int(payload(fetch(w + 8)));
      wc = rt * (sa - rho * sb);
      if (nu > kUncMax) {
        dirty = 1;
      } else {
        for (int k = 0; k < nu; ++k) {
          const int e = int(payload(fetch(w + 9 + k)));
          double at, ad;
          draw_args(d, e, P.vocab, at, ad);
          wc += resid_weight(exp_nonpos(at, sh.exp_table), exp_nonpos(ad, sh.exp_table), rt, rd);
        }
      }
    }
    sh.u.draw.w[cc] = wc;
    sh.u.draw.dirty[cc] = dirty;
  }
  __syncthreads();
  for (int cc = 0; cc < nsch; ++cc) {
    if (sh.u.draw.dirty[cc]) {
      const double wc = chunk_weight<T>(P, sh, cc, d, rt, rd);
      if (tid == 0) sh.u.draw.w[cc] = wc;
      __syncthreads();
    }
  }
  // Total S, as a scan over the chunk weights in groups of 256 chunks.
  double S = 0.0;
  for (int g = 0; g < nsch; g += kThreads) {
    const int cc = g + tid;
    double tot;
    block_scan(cc < nsch ? sh.u.draw.w[cc] : 0.0, tot, sh);
    S += tot;
  }
  bool fallback = false;
  if (d.residual && !(S > 0.0)) {
    // Every residual weight rounded to zero: draw from q_j itself, whose
    // chunk weights are the chunks' Zt scaled by 1/Zt.
    fallback = true;
    __syncthreads();
    for (int cc = tid; cc < nsch; cc += kThreads)
      sh.u.draw.w[cc] = rt * unpack_f64(fetch(nw + cc * kNormWords), fetch(nw + cc * kNormWords + 1));
    __syncthreads();
    S = 0.0;
    for (int g = 0; g < nsch; g += kThreads) {
      const int cc = g + tid;
      double tot;
      block_scan(cc < nsch ? sh.u.draw.w[cc] : 0.0, tot, sh);
      S += tot;
    }
  }
  const double target_mass = double(P.sample_u[b]) * S;
  // First chunk whose inclusive prefix exceeds target_mass.
  double before = 0.0;
  int chunk = -1, last_pos = -1;
  for (int g = 0; g < nsch && chunk < 0; g += kThreads) {
    const int cc = g + tid;
    const double w = cc < nsch ? sh.u.draw.w[cc] : 0.0;
    double tot;
    const double incl = before + block_scan(w, tot, sh);
    if (tid == 0) {
      sh.pick[0] = INT_MAX;
      sh.pick[1] = -1;
    }
    __syncthreads();
    if (cc < nsch && incl > target_mass && w > 0.0) atomicMin(&sh.pick[0], cc);
    if (cc < nsch && w > 0.0) atomicMax(&sh.pick[1], cc);
    __syncthreads();
    if (sh.pick[1] >= 0) last_pos = sh.pick[1];
    if (sh.pick[0] != INT_MAX) chunk = sh.pick[0];
    before += tot;
    __syncthreads();
  }
  if (chunk < 0) chunk = max(last_pos, 0);  // rounding left u*S at or past the total
  // Exclusive prefix of the chosen chunk, in the same group-scan order.
  before = 0.0;
  for (int g = 0; g < chunk; g += kThreads) {
    const int cc = g + tid;
    double tot;
    block_scan(cc < chunk ? sh.u.draw.w[cc] : 0.0, tot, sh);
    before += tot;
  }
  // Scan the chunk: thread t owns kSampPer consecutive tokens.
  const int e_base = chunk * kSampChunk + tid * kSampPer;
  double w[kSampPer];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < kSampPer; ++k) {
    double at, ad;
    draw_args(d, e_base + k, P.vocab, at, ad);
    const double et = exp_nonpos(at, sh.exp_table);
    if (!d.residual)
      w[k] = et;
    else if (fallback)
      w[k] = et * rt;
    else
      w[k] = resid_weight(et, exp_nonpos(ad, sh.exp_table), rt, rd);
    run += w[k];
  }
  double tot;
  const double incl = block_scan(run, tot, sh);
  double cum = before + (incl - run);
  if (tid == 0) {
    sh.pick[0] = INT_MAX;
    sh.pick[1] = -1;
  }
  __syncthreads();
  int first = INT_MAX, last = -1;
#pragma unroll
  for (int k = 0; k < kSampPer; ++k) {
    cum += w[k];
    if (first == INT_MAX && cum > target_mass && w[k] > 0.0) first = k;
    if (w[k] > 0.0) last = k;
  }
  if (first != INT_MAX) atomicMin(&sh.pick[0], e_base + first);
  if (last >= 0) atomicMax(&sh.pick[1], e_base + last);
  __syncthreads();
  if (tid == 0) {
    int token = (sh.pick[0] != INT_MAX) ? sh.pick[0] : sh.pick[1];
    if (token < 0) token = 0;
    P.out_tokens[int64_t(b) * (P.n_draft + 1) + s.j] = token;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The persistent kernel.

enum ItemKind : int { kNoItem = 0, kStat = 1, kDecide = 2, kNorm = 3, kDraw = 4 };

struct Slot {
  int kind;
  int b;
  int r;  // STAT row
  int c;  // STAT or NORM chunk
};

__device__ __forceinline__ Slot slot_item(const Params P, long long s) {
  Slot it{kNoItem, 0, 0, 0};
  const int n_stat = (2 * P.n_draft + 1) * P.nch;
  const int g = int(s / P.spg);
  const int o = int(s - (long long)g * P.spg);
  if (o < n_stat) {
    if (g < P.batch) it = Slot{kStat, g, o / P.nch, o % P.nch};
  } else if (o == n_stat) {
    const int b = g - P.lag_decide;
    if (b >= 0 && b < P.batch) it = Slot{kDecide, b, 0, 0};
  } else if (o < n_stat + 1 + P.nsch) {
    const int b = g - P.lag_norm;
    if (b >= 0 && b < P.batch) it = Slot{kNorm, b, 0, o - n_stat - 1};
  } else {
    const int b = g - P.lag_draw;
    if (b >= 0 && b < P.batch) it = Slot{kDraw, b, 0, 0};
  }
  return it;
}

template <typename T>
__global__ __launch_bounds__(kThreads, 4) void verify_kernel(Params P) {
  __shared__ Shared sh;
  if (threadIdx.x < kExpTableSize) sh.exp_table[threadIdx.x] = P.exp_table[threadIdx.x];
  __syncthreads();
  long long s = blockIdx.x;
  Slot it = slot_item(P, s);
  // The temperature of the next STAT item is loaded one item ahead.
  float t_next = (it.kind == kStat) ? P.temperature[it.b] : 0.0f;
  for (; s < P.total_slots; s += gridDim.x) {
    const Slot cur = it;
    const float t_cur = t_next;
    it = slot_item(P, s + gridDim.x);
    if (s + gridDim.x < P.total_slots && it.kind == kStat) t_next = P.temperature[it.b];
#ifdef SPECV_TRACE
    const unsigned long long t_start = wall_clock64();
    if (threadIdx.x == 0) {
      sh.wait_ticks = 0;
      sh.timeouts = 0;
    }
#endif
    switch (cur.kind) {
      case kStat:
        stat_item<T>(P, sh, cur.b, cur.r, cur.c, t_cur);
        break;
      case kDecide:
        decide_item<T>(P, sh, cur.b);
        break;
      case kNorm:
        norm_item<T>(P, sh, cur.b, cur.c);
        break;
      case kDraw:
        draw_item<T>(P, sh, cur.b);
        break;
      default:
        break;
    }
#ifdef SPECV_TRACE
    __syncthreads();
    if (threadIdx.x == 0 && cur.kind != kNoItem && s < P.trace_slots) {
      unsigned long long* rec = P.trace + s * 4;
      rec[0] = (unsigned long long)cur.kind | ((unsigned long long)blockIdx.x << 8);
      rec[1] = t_start;
      rec[2] = wall_clock64();
      rec[3] = sh.wait_ticks | (sh.timeouts << 48);
    }
#endif
  }
}

__global__ void clear_words_kernel(uint64_t* p, long long n) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    p[i] = 0;
}

const char* const kStageNames[] = {"verify"};
constexpr int kNumStages = 1;

template <typename T>
hipError_t launch_typed(const VerifyArgs& a, const Workspace& w, const LaunchConfig& cfg, hipStream_t stream,
                        hipEvent_t* ev) {
  Params P;
  P.draft = a.draft;
  P.target = a.target;
  P.tokens = a.tokens;
  P.accept_u = a.accept_u;
  P.sample_u = a.sample_u;
  P.temperature = a.temperature;
  P.out_tokens = a.out_tokens;
  P.out_n = a.out_n;
  P.row_lse = w.row_lse;
  P.row_argmax = w.row_argmax;
  P.stat_words = w.stat_words;
  P.seq_words = w.seq_words;
  P.norm_words = w.norm_words;
  P.exp_table = w.exp_table;
  P.batch = a.batch;
  P.n_draft = a.n_draft;
  P.vocab = a.vocab;
  P.nch = w.n_stats_chunks;
  P.nsch = w.n_samp_chunks;
  const int R = 2 * a.n_draft + 1;
  P.spg = R * P.nch + 1 + P.nsch + 1;
  P.lag_decide = cfg.lag_decide;
  P.lag_norm = cfg.lag_norm;
  P.lag_draw = cfg.lag_draw;
  P.total_slots = (long long)(a.batch + cfg.lag_draw) * P.spg;
  P.epoch = cfg.epoch;
  P.timeout_ticks = cfg.timeout_ticks;
#ifdef SPECV_TRACE
  P.trace = w.trace;
  P.trace_slots = w.trace_slots;
#endif
  // A grid size sharing a factor with the group size would give every
  // workgroup the same item types (e.g. only DRAW items); keep them coprime.
  long long grid = std::min<long long>(P.total_slots, cfg.max_blocks);
  while (grid > 1 && std::gcd(grid, (long long)P.spg) != 1) --grid;
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  hipLaunchKernelGGL(verify_kernel<T>, dim3(unsigned(grid)), dim3(kThreads), 0, stream, P);
  if (ev != nullptr) (void)hipEventRecord(ev[1], stream);
  return hipGetLastError();
}

}  // namespace

const char* stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

int max_blocks_per_cu(int dtype) {
  int occ = 0;
  if (dtype == 0)
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, verify_kernel<float>, kThreads, 0);
  else
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, verify_kernel<uint16_t>, kThreads, 0);
  return occ;
}

int norm_words_per_chunk() { return kNormWords; }
int seq_words_per_sequence() { return kSeqWords; }

hipError_t clear_words(uint64_t* p, long long n, hipStream_t stream) {
  hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, const LaunchConfig& cfg, hipStream_t stream,
                         hipEvent_t* events, int* n_stages) {
  if (n_stages != nullptr) *n_stages = kNumStages;
  if (a.dtype == 0) return launch_typed<float>(a, w, cfg, stream, events);
  return launch_typed<uint16_t>(a, w, cfg, stream, events);
}

}  // namespace specv
