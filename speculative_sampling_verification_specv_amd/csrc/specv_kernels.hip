// gfx950 kernels for batched speculative-sampling verification.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with "Step 1: 거절 단계" (the
// accept test) and "Step 2: 잔차 분포" (the residual); blog "…투기적 디코딩
// (Speculative Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// Three launches per call, B sequences, N drafts, 2N+1 rows of V logits each:
//   stat_kernel     one workgroup per (row, 32 KB chunk): fp32 max, sum of
//                   2^(z*c - fl(max*c)) with c = log2(e)/T, first argmax.
//                   Streaming and HBM-bound; greedy sequences skip draft rows.
//   decide_norm     one workgroup per (sequence, 4096-logit draw chunk). Each
//                   merges its sequence's row partials into log-normalisers and
//                   runs the N accept tests in fp64 (the same deterministic
//                   computation in every workgroup of the sequence; chunk 0
//                   writes the outputs), then sums the fp64 exps of its chunk of
//                   the row(s) the draw needs.
//   draw_kernel     one workgroup per sequence: chunk weights, inverse CDF over
//                   them, an fp64 rescan of the crossing chunk, the token.
//
// The residual weight of token x is w_x = max(0, et_x/Zt - ed_x/Zd)
// = max(0, et_x - rho*ed_x)/Zt with rho = Zt/Zd, so its sign only depends on
// whether log(et_x/ed_x) exceeds log(rho). The decision knows log(rho) from the
// fp32 row sums to ~1e-6; a draw chunk treats tokens more than 1e-4 away from it
// as certain and sums their exps into A and B, so the chunk's weight is
// (A - rho*B)/Zt plus the exact terms of its few uncertain tokens. One pass over
// the rows gives the normalisers and every chunk weight.
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
constexpr int kSampPer = kSampChunk / kThreads;  // logits per thread in a draw chunk
constexpr int kMaxRows = 2 * 64 + 1;
constexpr double kSignBand = 1e-4;  // |log(et/ed) - log(rho)| at or below this is uncertain
constexpr int kStageCap = 1024;     // row partials the decision stages in LDS

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

// Block-wide inclusive scan of one double per thread (fixed order); returns
// the thread's inclusive prefix and sets total.
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
  constexpr int kMaxVec = kStatsChunkBytes / 16 / kThreads;
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
__device__ __forceinline__ void block_merge(StatAcc& a, float c) {
  __shared__ float sm[kWaves], ss[kWaves];
  __shared__ int si[kWaves];
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

struct StatParams {
  const void* draft;
  const void* target;
  const float* temperature;
  RowPartial* partials;
  int n_draft;
  int vocab;
  int nch;
  int chunk;
};

// One workgroup per (row, chunk) item: item = (b*(2N+1) + r)*nch + c. Rows a
// sequence never needs (draft rows at T = 0, every row of an invalid
// temperature) are skipped; their partials are never read.
template <typename T>
__global__ __launch_bounds__(kThreads) void stat_kernel(StatParams P) {
  const int R = 2 * P.n_draft + 1;
  const int item = blockIdx.x;
  const int row = item / P.nch;
  const int chunk = item - row * P.nch;
  const int b = row / R;
  const int r = row - b * R;
  const float t = P.temperature[b];
  if (!temperature_valid(t)) return;
  const bool greedy = (t == 0.0f);
  if (greedy && r < P.n_draft) return;
  const int N = P.n_draft;
  const int64_t row_flat = (r < N) ? (int64_t(b) * N + r) * P.vocab : (int64_t(b) * (N + 1) + (r - N)) * P.vocab;
  const T* rowp = static_cast<const T*>(r < N ? P.draft : P.target) + row_flat;
  const int e0 = chunk * P.chunk;
  const int e1 = min(P.vocab, e0 + P.chunk);
  StatAcc a;
  acc_init(a);
  if (greedy) {
    stats_chunk<T, false>(rowp, row_flat, e0, e1, 0.0f, a);
    block_merge<false>(a, 0.0f);
  } else {
    const float c = exp2_coef(t);
    stats_chunk<T, true>(rowp, row_flat, e0, e1, c, a);
    block_merge<true>(a, c);
  }
  if (threadIdx.x == 0) {
    RowPartial p;
    p.m = a.m;
    p.s = a.s;
    p.idx = a.idx;
    p.pad = 0;
    P.partials[item] = p;
  }
}

// ---------------------------------------------------------------------------
// Decision and draw chunks.

struct DrawParams {
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
  const RowPartial* partials;
  SeqRecord* seq;
  NormRecord* norm;
  const double* exp_table;
  int n_draft;
  int vocab;
  int nch;
  int nsch;
};

template <typename T>
struct DrawRows {
  const T* trow;
  const T* drow;
  double mt, md, inv_t;
  bool residual;
};

template <typename T>
__device__ __forceinline__ DrawRows<T> draw_rows(const DrawParams& P, int b, const SeqRecord& s, float t) {
  const int N = P.n_draft;
  DrawRows<T> d;
  d.trow = static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + s.j) * P.vocab;
  d.drow = static_cast<const T*>(P.draft) + (int64_t(b) * N + min(s.j, N - 1)) * P.vocab;
  d.mt = s.m_target;
  d.md = s.m_draft;
  d.inv_t = 1.0 / double(t);
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

struct DecideShared {
  double exp_table[kExpTableSize];
  double red[kWaves];
  float row_m[kMaxRows];
  double row_logz[kMaxRows];
  int row_idx[kMaxRows];
  int unc_base[kWaves];
  float part_m[kStageCap];
  float part_s[kStageCap];
  int part_idx[kStageCap];
};

// The decision for sequence b, computed identically by every workgroup that
// asks: per-row log-normalisers and argmaxes from the row partials, the N
// accept tests, the first rejection. The workgroup with `write` set also
// writes the outputs, the row diagnostics and the sequence record.
template <typename T>
__device__ SeqRecord decide(const DrawParams& P, DecideShared& sh, int b, float t, bool write) {
  const int N = P.n_draft;
  const int R = 2 * N + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int* tok = P.tokens + int64_t(b) * N;
  int* otok = P.out_tokens + int64_t(b) * (N + 1);
  float* lse = P.row_lse + int64_t(b) * R;
  int* amax = P.row_argmax + int64_t(b) * R;
  SeqRecord rec{kModeNone, 0, 0.0f, 0.0f, 0.0, 0.0};

  int d = 0;
  float ua = 0.0f;
  bool bad = !temperature_valid(t);
  if (tid < N) {
    d = tok[tid];
    bad = bad || d < 0 || d >= P.vocab;
    ua = P.accept_u[int64_t(b) * N + tid];
  }
  if (__syncthreads_or(bad)) {
    if (write) {
      for (int i = tid; i <= N; i += kThreads) otok[i] = -1;
      for (int r = tid; r < R; r += kThreads) {
        lse[r] = NAN;
        amax[r] = -1;
      }
      if (tid == 0) {
        P.out_n[b] = -1;
        P.seq[b] = rec;
      }
    }
    return rec;
  }
  const bool greedy = (t == 0.0f);
  float zt = 0.0f, zd = 0.0f;
  if (tid < N && !greedy) {
    zt = Logit<T>::at(static_cast<const T*>(P.target), (int64_t(b) * (N + 1) + tid) * P.vocab + d);
    zd = Logit<T>::at(static_cast<const T*>(P.draft), (int64_t(b) * N + tid) * P.vocab + d);
  }
  const int r_first = greedy ? N : 0;
  const int n_part = (R - r_first) * P.nch;
  const RowPartial* parts = P.partials + (int64_t(b) * R + r_first) * P.nch;
  const bool staged = n_part <= kStageCap;
  if (staged) {
    for (int i = tid; i < n_part; i += kThreads) {
      const RowPartial p = parts[i];
      sh.part_m[i] = p.m;
      sh.part_s[i] = p.s;
      sh.part_idx[i] = p.idx;
    }
    __syncthreads();
  }
  const float c = greedy ? 0.0f : exp2_coef(t);
  const double inv_t = greedy ? 0.0 : 1.0 / double(t);

  // Merge each row's chunk partials: lanes take chunks lane, lane+64, ...,
  // then a butterfly; waves take rows wave, wave+4, ...
  for (int r = r_first + wave; r < R; r += kWaves) {
    const int pbase = (r - r_first) * P.nch;
    float m = -INFINITY, s = 0.0f;
    int idx = INT_MAX;
    for (int k = lane; k < P.nch; k += 64) {
      float m2, s2;
      int i2;
      if (staged) {
        m2 = sh.part_m[pbase + k];
        s2 = sh.part_s[pbase + k];
        i2 = sh.part_idx[pbase + k];
      } else {
        const RowPartial p = parts[pbase + k];
        m2 = p.m;
        s2 = p.s;
        i2 = p.idx;
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
      if (write) {
        lse[r] = greedy ? NAN : float(double(m) * inv_t + logz);
        amax[r] = idx;
      }
    }
  }
  if (write && greedy) {
    for (int r = tid; r < N; r += kThreads) {
      lse[r] = NAN;
      amax[r] = -1;
    }
  }
  __syncthreads();

  bool accept = true;
  if (tid < N) {
    if (greedy) {
      accept = (d == sh.row_idx[N + tid]);
    } else if (zd == -INFINITY) {
      accept = true;  // p(d) == 0: the ratio is infinite
    } else {
      const double log_q = (double(zt) - double(sh.row_m[N + tid])) * inv_t - sh.row_logz[N + tid];
      const double log_p = (double(zd) - double(sh.row_m[tid])) * inv_t - sh.row_logz[tid];
      accept = double(ua) < exp(log_q - log_p);
    }
  }
  // N <= 64: every decision lives in wave 0.
  __shared__ unsigned long long rej_mask;
  if (wave == 0) {
    const unsigned long long rej = __ballot(tid < N && !accept);
    if (lane == 0) rej_mask = rej;
  }
  __syncthreads();
  const unsigned long long rej = rej_mask;
  const int j = rej ? (__ffsll(rej) - 1) : N;
  rec.mode = greedy ? kModeNone : (j < N ? kModeResidual : kModeBonus);
  rec.j = j;
  rec.m_target = sh.row_m[N + j];
  rec.m_draft = (j < N && !greedy) ? sh.row_m[j] : 0.0f;
  rec.log_rho = (j < N && !greedy) ? sh.row_logz[N + j] - sh.row_logz[j] : 0.0;
  if (write) {
    for (int i = tid; i <= N; i += kThreads) {
      if (i < j)
        otok[i] = tok[i];
      else if (i > j)
        otok[i] = -1;
      else if (greedy)
        otok[i] = sh.row_idx[N + j];
    }
    if (tid == 0) {
      P.out_n[b] = j;
      P.seq[b] = rec;
    }
  }
  __syncthreads();
  return rec;
}

// fp64 sums of one draw chunk (see NormRecord).
template <typename T>
__device__ void norm_chunk(const DrawParams& P, DecideShared& sh, int b, int c, const DrawRows<T>& d,
                           double log_rho) {
  const int tid = threadIdx.x;
  double zt = 0.0, zd = 0.0, sa = 0.0, sb = 0.0;
  uint32_t unc = 0;  // bit k: token c*kSampChunk + tid + k*kThreads has an uncertain sign
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
  NormRecord* out = P.norm + int64_t(b) * P.nsch + c;
  zt = block_sum(zt, sh.red);
  if (!d.residual) {
    if (tid == 0) out->zt = zt;
    return;
  }
  zd = block_sum(zd, sh.red);
  sa = block_sum(sa, sh.red);
  sb = block_sum(sb, sh.red);
  // Uncertain tokens, listed in (thread, k) order.
  const int cnt = __popc(unc);
  int incl = cnt;
  const int lane = tid & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
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
      if (unc & (1u << k)) out->idx[slot++] = c * kSampChunk + tid + k * kThreads;
  }
  if (tid == 0) {
    out->zt = zt;
    out->zd = zd;
    out->a = sa;
    out->b = sb;
    out->n_unc = total;
  }
}

// One workgroup per (sequence, draw chunk): the decision, then the chunk sums.
template <typename T>
__global__ __launch_bounds__(kThreads) void decide_norm_kernel(DrawParams P) {
  __shared__ DecideShared sh;
  const int b = blockIdx.x / P.nsch;
  const int c = blockIdx.x - b * P.nsch;
  if (threadIdx.x < kExpTableSize) sh.exp_table[threadIdx.x] = P.exp_table[threadIdx.x];
  const float t = P.temperature[b];
  const SeqRecord s = decide<T>(P, sh, b, t, c == 0);
  if (s.mode == kModeNone) return;
  norm_chunk<T>(P, sh, b, c, draw_rows<T>(P, b, s, t), s.log_rho);
}

struct DrawShared {
  double exp_table[kExpTableSize];
  double red[kWaves];
  double w[kMaxSampChunks];
  int dirty[kMaxSampChunks];
  int pick[2];
};

// Weight sum of one chunk from its logits (after a rejection): used for
// chunks with more uncertain tokens than their record holds.
template <typename T>
__device__ double chunk_weight(const DrawParams& P, DrawShared& sh, int c, const DrawRows<T>& d, double rt,
                               double rd) {
  double w = 0.0;
#pragma unroll
  for (int k = 0; k < kSampPer; ++k) {
    double at, ad;
    draw_args(d, c * kSampChunk + threadIdx.x + k * kThreads, P.vocab, at, ad);
    w += resid_weight(exp_nonpos(at, sh.exp_table), exp_nonpos(ad, sh.exp_table), rt, rd);
  }
  return block_sum(w, sh.red);
}

// One workgroup per sequence: chunk weights, the crossing chunk, an fp64 scan of it.
template <typename T>
__global__ __launch_bounds__(kThreads) void draw_kernel(DrawParams P) {
  __shared__ DrawShared sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nsch = P.nsch;
  if (tid < kExpTableSize) sh.exp_table[tid] = P.exp_table[tid];
  const SeqRecord s = P.seq[b];
  if (s.mode == kModeNone) return;
  const float t = P.temperature[b];
  const DrawRows<T> d = draw_rows<T>(P, b, s, t);
  const NormRecord* nr = P.norm + int64_t(b) * nsch;
  __syncthreads();

  // Normalisers (fixed order) and the chunk weights.
  double rt = 0.0, rd = 0.0, rho = 0.0;
  if (d.residual) {
    double zt = 0.0, zd = 0.0;
    for (int cc = tid; cc < nsch; cc += kThreads) {
      zt += nr[cc].zt;
      zd += nr[cc].zd;
    }
    zt = block_sum(zt, sh.red);
    zd = block_sum(zd, sh.red);
    rt = 1.0 / zt;
    rd = 1.0 / zd;
    rho = zt * rd;
  }
  for (int cc = tid; cc < nsch; cc += kThreads) {
    double wc;
    int dirty = 0;
    if (!d.residual) {
      wc = nr[cc].zt;
    } else {
      wc = rt * (nr[cc].a - rho * nr[cc].b);
      const int nu = nr[cc].n_unc;
      if (nu > kUncMax) {
        dirty = 1;
      } else {
        double extra[kUncMax];
#pragma unroll
        for (int k = 0; k < kUncMax; ++k) {
          extra[k] = 0.0;
          if (k < nu) {
            double at, ad;
            draw_args(d, nr[cc].idx[k], P.vocab, at, ad);
            extra[k] = resid_weight(exp_nonpos(at, sh.exp_table), exp_nonpos(ad, sh.exp_table), rt, rd);
          }
        }
#pragma unroll
        for (int k = 0; k < kUncMax; ++k) wc += extra[k];
      }
    }
    sh.w[cc] = wc;
    sh.dirty[cc] = dirty;
  }
  __syncthreads();
  for (int cc = 0; cc < nsch; ++cc) {
    if (sh.dirty[cc]) {
      const double wc = chunk_weight<T>(P, sh, cc, d, rt, rd);
      if (tid == 0) sh.w[cc] = wc;
      __syncthreads();
    }
  }
  // Total S, as a scan over the chunk weights in groups of 256 chunks.
  double S = 0.0;
  for (int g = 0; g < nsch; g += kThreads) {
    const int cc = g + tid;
    double tot;
    block_scan(cc < nsch ? sh.w[cc] : 0.0, tot, sh.red);
    S += tot;
  }
  bool fallback = false;
  if (d.residual && !(S > 0.0)) {
    // Every residual weight rounded to zero: draw from q_j itself, whose
    // chunk weights are the chunks' Zt scaled by 1/Zt.
    fallback = true;
    __syncthreads();
    for (int cc = tid; cc < nsch; cc += kThreads) sh.w[cc] = rt * nr[cc].zt;
    __syncthreads();
    S = 0.0;
    for (int g = 0; g < nsch; g += kThreads) {
      const int cc = g + tid;
      double tot;
      block_scan(cc < nsch ? sh.w[cc] : 0.0, tot, sh.red);
      S += tot;
    }
  }
  const double target_mass = double(P.sample_u[b]) * S;
  // First chunk whose inclusive prefix exceeds target_mass.
  double before = 0.0;
  int chunk = -1, last_pos = -1;
  for (int g = 0; g < nsch && chunk < 0; g += kThreads) {
    const int cc = g + tid;
    const double w = cc < nsch ? sh.w[cc] : 0.0;
    double tot;
    const double incl = before + block_scan(w, tot, sh.red);
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
    block_scan(cc < chunk ? sh.w[cc] : 0.0, tot, sh.red);
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
  const double incl = block_scan(run, tot, sh.red);
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
}

const char* const kStageNames[] = {"row_stats", "decide_norm", "draw"};
constexpr int kNumStages = 3;

template <typename T>
hipError_t launch_typed(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* ev) {
  const int R = 2 * a.n_draft + 1;
  StatParams sp;
  sp.draft = a.draft;
  sp.target = a.target;
  sp.temperature = a.temperature;
  sp.partials = w.partials;
  sp.n_draft = a.n_draft;
  sp.vocab = a.vocab;
  sp.nch = w.n_stats_chunks;
  sp.chunk = w.stats_chunk;
  DrawParams dp;
  dp.draft = a.draft;
  dp.target = a.target;
  dp.tokens = a.tokens;
  dp.accept_u = a.accept_u;
  dp.sample_u = a.sample_u;
  dp.temperature = a.temperature;
  dp.out_tokens = a.out_tokens;
  dp.out_n = a.out_n;
  dp.row_lse = w.row_lse;
  dp.row_argmax = w.row_argmax;
  dp.partials = w.partials;
  dp.seq = w.seq;
  dp.norm = w.norm;
  dp.exp_table = w.exp_table;
  dp.n_draft = a.n_draft;
  dp.vocab = a.vocab;
  dp.nch = w.n_stats_chunks;
  dp.nsch = w.n_samp_chunks;
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  hipLaunchKernelGGL(stat_kernel<T>, dim3(unsigned(int64_t(a.batch) * R * sp.nch)), dim3(kThreads), 0, stream, sp);
  if (ev != nullptr) (void)hipEventRecord(ev[1], stream);
  hipLaunchKernelGGL(decide_norm_kernel<T>, dim3(unsigned(int64_t(a.batch) * dp.nsch)), dim3(kThreads), 0, stream,
                     dp);
  if (ev != nullptr) (void)hipEventRecord(ev[2], stream);
  hipLaunchKernelGGL(draw_kernel<T>, dim3(unsigned(a.batch)), dim3(kThreads), 0, stream, dp);
  if (ev != nullptr) (void)hipEventRecord(ev[3], stream);
  return hipGetLastError();
}

}  // namespace

const char* stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* events,
                         int* n_stages) {
  if (n_stages != nullptr) *n_stages = kNumStages;
  if (a.dtype == 0) return launch_typed<float>(a, w, stream, events);
  return launch_typed<uint16_t>(a, w, stream, events);
}

}  // namespace specv
