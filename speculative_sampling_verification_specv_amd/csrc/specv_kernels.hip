// gfx950 kernels for batched speculative-sampling verification.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with its "Step 1" (accept
// test) and "Step 2" (residual distribution); blog "…투기적 디코딩(Speculative
// Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// Pipeline for one call (B sequences, N drafts, vocabulary V):
//   1. row_stats: every (row, 8192-logit chunk) reduces to (max, sum 2^((z-max)c),
//      first argmax) in fp32; streaming, HBM-bound. Greedy sequences skip
//      their draft rows.
//   2. decide: one wave per sequence merges the chunk partials into per-row
//      log-normalisers, runs the N accept tests in fp64 and finds the first
//      rejection with a ballot.
//   3. resid_norm: for sequences that rejected, fp64 normalisers of target and
//      draft row j, recomputed from the logits (fp32 normalisers are not
//      accurate enough for the residual draw).
//   4. weights: fp64 per-chunk sums of the draw weights, (q_j - p_j)_+ after a
//      rejection or exp((z - max)/T) of target row N for the bonus.
//   5. draw: one workgroup per sequence finds the chunk where the cumulative
//      weight crosses u * S and scans it in fp64 to find the token.
// Every reduction has a fixed order, so results are bitwise reproducible.

#include <float.h>
#include <limits.h>
#include <math.h>

#include "specv_internal.h"

namespace specv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFltMax = 3.402823466e38f;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ bool temperature_valid(float t) { return t >= 0.0f && t <= kFltMax; }

// c in 2^((z - m) * c) == exp((z - m) / T); clamped so a denormal T yields a
// huge finite factor rather than inf (0 * inf would give NaN at z == m).
__device__ __forceinline__ float exp2_coef(float t) { return fminf(kLog2e / t, kFltMax); }

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
// Row statistics (max, tempered sum-exp, first argmax), fp32.

// Running state of one thread: m = largest logit seen, idx = its first index,
// s = sum of 2^((z - shift) * c) where shift == m once a finite logit was seen
// (0 before, when s is 0 too).
struct StatAcc {
  float m;
  float s;
  float shift;
  int idx;
};

__device__ __forceinline__ void acc_init(StatAcc& a) {
  a.m = -INFINITY;
  a.s = 0.0f;
  a.shift = 0.0f;
  a.idx = INT_MAX;
}

// Fold n logits with consecutive indices base..base+n-1 into the state. Each
// thread visits its indices in increasing order, so a strict '>' keeps the
// first index of a repeated maximum.
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
      a.s = (a.s == 0.0f) ? 0.0f : a.s * fast_exp2((a.shift - vmax) * c);
      a.shift = vmax;
    }
    a.m = vmax;
    a.idx = base + first;
  }
  if (kSampled) {
    float e[n];
#pragma unroll
    for (int k = 0; k < n; ++k) e[k] = fast_exp2((v[k] - a.shift) * c);
#pragma unroll
    for (int w = 1; w < n; w *= 2)
#pragma unroll
      for (int k = 0; k + w < n; k += 2 * w) e[k] += e[k + w];
    a.s += e[0];
  }
}

// Merge partial (m2, s2, i2) into (m, s, i): larger max wins, sums are
// rescaled to the common max, ties in the max keep the lower index.
template <bool kSampled>
__device__ __forceinline__ void acc_merge(float& m, float& s, int& idx, float m2, float s2, int i2, float c) {
  const float mm = fmaxf(m, m2);
  if (kSampled) {
    const float a = (m == mm) ? s : s * fast_exp2((m - mm) * c);
    const float b = (m2 == mm) ? s2 : s2 * fast_exp2((m2 - mm) * c);
    s = a + b;
  }
  idx = (m > m2) ? idx : ((m2 > m) ? i2 : min(idx, i2));
  m = mm;
}

template <typename T, bool kSampled>
__device__ __forceinline__ void stats_chunk(const T* __restrict__ row, int64_t row_flat, int e0, int e1,
                                            float c, StatAcc& a) {
  constexpr int kVec = Logit<T>::kVec;
  const int tid = threadIdx.x;
  // Element g of the flat buffer is 16-byte aligned iff g % kVec == 0 (the
  // base pointer is 16-byte aligned).
  const int mis = int((row_flat + e0) % kVec);
  int ea = e0 + (kVec - mis) % kVec;
  if (ea > e1) ea = e1;
  const int nv = (e1 - ea) / kVec;
  const int et = ea + nv * kVec;
  if (tid < ea - e0) {
    const float v[1] = {Logit<T>::at(row, e0 + tid)};
    acc_values<kSampled>(a, v, e0 + tid, c);
  }
  const uint4* __restrict__ vrow = reinterpret_cast<const uint4*>(row + ea);
  int k = tid;
  for (; k + 3 * kThreads < nv; k += 4 * kThreads) {
    const uint4 x0 = vrow[k];
    const uint4 x1 = vrow[k + kThreads];
    const uint4 x2 = vrow[k + 2 * kThreads];
    const uint4 x3 = vrow[k + 3 * kThreads];
    float v[kVec];
    Logit<T>::unpack(x0, v);
    acc_values<kSampled>(a, v, ea + k * kVec, c);
    Logit<T>::unpack(x1, v);
    acc_values<kSampled>(a, v, ea + (k + kThreads) * kVec, c);
    Logit<T>::unpack(x2, v);
    acc_values<kSampled>(a, v, ea + (k + 2 * kThreads) * kVec, c);
    Logit<T>::unpack(x3, v);
    acc_values<kSampled>(a, v, ea + (k + 3 * kThreads) * kVec, c);
  }
  for (; k < nv; k += kThreads) {
    float v[kVec];
    Logit<T>::unpack(vrow[k], v);
    acc_values<kSampled>(a, v, ea + k * kVec, c);
  }
  if (tid < e1 - et) {
    const float v[1] = {Logit<T>::at(row, et + tid)};
    acc_values<kSampled>(a, v, et + tid, c);
  }
}

template <bool kSampled>
__device__ __forceinline__ void block_merge(StatAcc& a, float c) {
  __shared__ float sm_m[kWaves], sm_s[kWaves];
  __shared__ int sm_i[kWaves];
  float m = a.m, s = a.s;
  int idx = a.idx;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off);
    const float s2 = __shfl_xor(s, off);
    const int i2 = __shfl_xor(idx, off);
    acc_merge<kSampled>(m, s, idx, m2, s2, i2, c);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm_m[wave] = m;
    sm_s[wave] = s;
    sm_i[wave] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm_m[0];
    s = sm_s[0];
    idx = sm_i[0];
    for (int w = 1; w < kWaves; ++w) acc_merge<kSampled>(m, s, idx, sm_m[w], sm_s[w], sm_i[w], c);
    a.m = m;
    a.s = s;
    a.idx = idx;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(const T* __restrict__ draft,
                                                             const T* __restrict__ target,
                                                             const float* __restrict__ temperature, int n_draft,
                                                             int vocab, int nch, RowPartial* __restrict__ partials) {
  const int R = 2 * n_draft + 1;
  const int item = blockIdx.x;
  const int row = item / nch;
  const int chunk = item - row * nch;
  const int b = row / R;
  const int lr = row - b * R;
  const float t = temperature[b];
  if (!temperature_valid(t)) return;
  const bool greedy = (t == 0.0f);
  if (greedy && lr < n_draft) return;  // greedy verification never needs the draft rows
  const bool is_draft = lr < n_draft;
  const int64_t row_flat = is_draft ? (int64_t(b) * n_draft + lr) * vocab
                                    : (int64_t(b) * (n_draft + 1) + (lr - n_draft)) * vocab;
  const T* rowp = (is_draft ? draft : target) + row_flat;
  const int e0 = chunk * kStatsChunk;
  const int e1 = min(vocab, e0 + kStatsChunk);
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
    partials[item] = p;
  }
}

// ---------------------------------------------------------------------------
// Decision: per-row log-normalisers, N accept tests, first rejection.

template <typename T>
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(
    const T* __restrict__ draft, const T* __restrict__ target, const int* __restrict__ tokens,
    const float* __restrict__ accept_u, const float* __restrict__ temperature, int n_draft, int vocab, int nch,
    const RowPartial* __restrict__ partials, float* __restrict__ row_lse, int* __restrict__ row_argmax,
    SeqState* __restrict__ seq, int* __restrict__ out_tokens, int* __restrict__ out_n) {
  constexpr int kMaxRows = 2 * 64 + 1;
  __shared__ float sm_m[kMaxRows];
  __shared__ double sm_logs[kMaxRows];
  __shared__ int sm_idx[kMaxRows];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = n_draft;
  const int R = 2 * N + 1;
  const int* tok = tokens + int64_t(b) * N;
  int* otok = out_tokens + int64_t(b) * (N + 1);
  float* lse = row_lse + int64_t(b) * R;
  int* amax = row_argmax + int64_t(b) * R;

  const float t = temperature[b];
  bool bad = !temperature_valid(t);
  for (int i = lane; i < N; i += kDecideThreads) {
    const int d = tok[i];
    bad = bad || d < 0 || d >= vocab;
  }
  if (__ballot(bad) != 0) {
    for (int i = lane; i <= N; i += kDecideThreads) otok[i] = -1;
    for (int r = lane; r < R; r += kDecideThreads) {
      lse[r] = NAN;
      amax[r] = -1;
    }
    if (lane == 0) {
      out_n[b] = -1;
      seq[b].mode = kModeNone;
    }
    return;
  }

  const bool greedy = (t == 0.0f);
  const float c = greedy ? 0.0f : exp2_coef(t);
  const double inv_t = greedy ? 0.0 : 1.0 / double(t);
  for (int r = lane; r < R; r += kDecideThreads) {
    if (greedy && r < N) {
      lse[r] = NAN;
      amax[r] = -1;
      continue;
    }
    const RowPartial* rp = partials + (int64_t(b) * R + r) * nch;
    float m = rp[0].m, s = rp[0].s;
    int idx = rp[0].idx;
    for (int k = 1; k < nch; ++k) {
      if (greedy)
        acc_merge<false>(m, s, idx, rp[k].m, rp[k].s, rp[k].idx, c);
      else
        acc_merge<true>(m, s, idx, rp[k].m, rp[k].s, rp[k].idx, c);
    }
    if (idx == INT_MAX) idx = 0;  // an all -inf row: every index ties, the first wins
    const double logs = greedy ? 0.0 : log(double(s));
    sm_m[r] = m;
    sm_logs[r] = logs;
    sm_idx[r] = idx;
    lse[r] = greedy ? NAN : float(double(m) * inv_t + logs);
    amax[r] = idx;
  }
  __syncthreads();

  // Lane i < N makes decision i.
  bool accept = true;
  if (lane < N) {
    const int d = tok[lane];
    if (greedy) {
      accept = (d == sm_idx[N + lane]);
    } else {
      const float zt = Logit<T>::at(target, (int64_t(b) * (N + 1) + lane) * vocab + d);
      const float zd = Logit<T>::at(draft, (int64_t(b) * N + lane) * vocab + d);
      if (zd == -INFINITY) {
        accept = true;  // p(d) == 0: the ratio is infinite
      } else {
        const double log_q = (double(zt) - double(sm_m[N + lane])) * inv_t - sm_logs[N + lane];
        const double log_p = (double(zd) - double(sm_m[lane])) * inv_t - sm_logs[lane];
        accept = double(accept_u[int64_t(b) * N + lane]) < exp(log_q - log_p);
      }
    }
  }
  const unsigned long long rej = __ballot(lane < N && !accept);
  const int j = rej ? (__ffsll(rej) - 1) : N;
  for (int i = lane; i <= N; i += kDecideThreads) {
    int v = -1;
    if (i < j)
      v = tok[i];
    else if (i == j && greedy)
      v = sm_idx[N + j];
    otok[i] = v;
  }
  if (lane == 0) {
    out_n[b] = j;
    SeqState st;
    st.mode = greedy ? kModeNone : (j < N ? kModeResidual : kModeBonus);
    st.j = j;
    st.m_target = sm_m[N + j];
    st.m_draft = (j < N) ? sm_m[j] : 0.0f;
    st.inv_t = inv_t;
    seq[b] = st;
  }
}

// ---------------------------------------------------------------------------
// Residual / bonus draw, fp64.

__device__ __forceinline__ double block_sum(double v) {
  __shared__ double sm[kWaves];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[wave] = v;
  __syncthreads();
  double total = sm[0];
  for (int w = 1; w < kWaves; ++w) total += sm[w];
  return total;
}

template <typename T>
struct DrawRow {
  const T* trow;
  const T* drow;
  double mt, md, inv_t;
  double rt, rd;  // 1 / normalisers (residual only)
  bool residual;

  // Weight of token e: (q - p)_+ after a rejection, exp((z - m)/T) of the
  // target row otherwise (the bonus, self-normalised by its own sum).
  __device__ __forceinline__ double weight(int e) const {
    const double et = exp((double(Logit<T>::at(trow, e)) - mt) * inv_t);
    if (!residual) return et;
    const double ed = exp((double(Logit<T>::at(drow, e)) - md) * inv_t);
    return fmax(0.0, et * rt - ed * rd);
  }
};

template <typename T>
__device__ __forceinline__ DrawRow<T> make_draw_row(const T* draft, const T* target, int b, int N, int vocab,
                                                    const SeqState& st, const double2* norm, int nsch) {
  DrawRow<T> p;
  p.trow = target + (int64_t(b) * (N + 1) + st.j) * vocab;
  p.drow = (st.j < N) ? draft + (int64_t(b) * N + st.j) * vocab : nullptr;
  p.mt = st.m_target;
  p.md = st.m_draft;
  p.inv_t = st.inv_t;
  p.residual = (st.mode == kModeResidual);
  p.rt = p.rd = 0.0;
  if (p.residual) {
    double zt = 0.0, zd = 0.0;
    for (int c = 0; c < nsch; ++c) {
      zt += norm[c].x;
      zd += norm[c].y;
    }
    p.rt = 1.0 / zt;
    p.rd = 1.0 / zd;
  }
  return p;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void resid_norm_kernel(const T* __restrict__ draft,
                                                              const T* __restrict__ target, int n_draft,
                                                              int vocab, int nsch, const SeqState* __restrict__ seq,
                                                              double2* __restrict__ norm_part) {
  const int b = blockIdx.x / nsch;
  const int c = blockIdx.x - b * nsch;
  const SeqState st = seq[b];
  if (st.mode != kModeResidual) return;
  const T* trow = target + (int64_t(b) * (n_draft + 1) + st.j) * vocab;
  const T* drow = draft + (int64_t(b) * n_draft + st.j) * vocab;
  const int e0 = c * kSampChunk;
  const int e1 = min(vocab, e0 + kSampChunk);
  const double mt = st.m_target, md = st.m_draft;
  double zt = 0.0, zd = 0.0;
  for (int e = e0 + threadIdx.x; e < e1; e += kThreads) {
    zt += exp((double(Logit<T>::at(trow, e)) - mt) * st.inv_t);
    zd += exp((double(Logit<T>::at(drow, e)) - md) * st.inv_t);
  }
  zt = block_sum(zt);
  zd = block_sum(zd);
  if (threadIdx.x == 0) norm_part[int64_t(b) * nsch + c] = make_double2(zt, zd);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void weights_kernel(const T* __restrict__ draft, const T* __restrict__ target,
                                                           int n_draft, int vocab, int nsch,
                                                           const SeqState* __restrict__ seq,
                                                           const double2* __restrict__ norm_part,
                                                           double* __restrict__ wsum_part) {
  const int b = blockIdx.x / nsch;
  const int c = blockIdx.x - b * nsch;
  const SeqState st = seq[b];
  if (st.mode == kModeNone) return;
  const DrawRow<T> p = make_draw_row(draft, target, b, n_draft, vocab, st, norm_part + int64_t(b) * nsch, nsch);
  const int e0 = c * kSampChunk;
  const int e1 = min(vocab, e0 + kSampChunk);
  double w = 0.0;
  for (int e = e0 + threadIdx.x; e < e1; e += kThreads) w += p.weight(e);
  w = block_sum(w);
  if (threadIdx.x == 0) wsum_part[int64_t(b) * nsch + c] = w;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void draw_kernel(const T* __restrict__ draft, const T* __restrict__ target,
                                                        const float* __restrict__ sample_u, int n_draft, int vocab,
                                                        int nsch, const SeqState* __restrict__ seq,
                                                        const double2* __restrict__ norm_part,
                                                        double* __restrict__ wsum_part, int* __restrict__ out_tokens) {
  constexpr int kPer = kSampChunk / kThreads;  // consecutive weights per thread in the scan
  __shared__ double w_lds[kSampChunk];
  __shared__ double wave_tot[kWaves];
  __shared__ double sh_before, sh_target;
  __shared__ int sh_chunk, sh_first, sh_last;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const SeqState st = seq[b];
  if (st.mode == kModeNone) return;
  DrawRow<T> p = make_draw_row(draft, target, b, n_draft, vocab, st, norm_part + int64_t(b) * nsch, nsch);
  double* wsum = wsum_part + int64_t(b) * nsch;
  const double u = double(sample_u[b]);

  // A residual whose weights all rounded to zero falls back to q_j itself.
  if (p.residual) {
    double S = 0.0;
    for (int c = 0; c < nsch; ++c) S += wsum[c];
    if (!(S > 0.0)) {
      p.residual = false;
      for (int c = 0; c < nsch; ++c) {
        const int e1 = min(vocab, (c + 1) * kSampChunk);
        double w = 0.0;
        for (int e = c * kSampChunk + tid; e < e1; e += kThreads) w += p.weight(e);
        w = block_sum(w);
        __syncthreads();
        if (tid == 0) wsum[c] = w;
      }
      __syncthreads();
    }
  }

  if (tid == 0) {
    double S = 0.0;
    for (int c = 0; c < nsch; ++c) S += wsum[c];
    const double target_mass = u * S;
    double before = 0.0;
    int chunk = -1;
    for (int c = 0; c < nsch; ++c) {
      const double next = before + wsum[c];
      if (next > target_mass) {
        chunk = c;
        break;
      }
      before = next;
    }
    if (chunk < 0) {  // rounding left u*S at or past the total: last chunk with weight
      chunk = nsch - 1;
      while (chunk > 0 && !(wsum[chunk] > 0.0)) --chunk;
      before = 0.0;
      for (int c = 0; c < chunk; ++c) before += wsum[c];
    }
    sh_chunk = chunk;
    sh_before = before;
    sh_target = target_mass;
    sh_first = INT_MAX;
    sh_last = -1;
  }
  __syncthreads();
  const int chunk = sh_chunk;
  const int e0 = chunk * kSampChunk;
  for (int i = tid; i < kSampChunk; i += kThreads) {
    const int e = e0 + i;
    w_lds[i] = (e < vocab) ? p.weight(e) : 0.0;
  }
  __syncthreads();

  // Inclusive scan: each thread owns kPer consecutive weights.
  double local[kPer];
  double run = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    run += w_lds[tid * kPer + k];
    local[k] = run;
  }
  // Exclusive scan of the per-thread totals across the block.
  double incl = run;
  const int lane = tid & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  const int wave = tid >> 6;
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  double base = sh_before;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  base += incl - run;
  const double target_mass = sh_target;
  int first = INT_MAX, last = -1;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = tid * kPer + k;
    if (first == INT_MAX && base + local[k] > target_mass) first = i;
    if (w_lds[i] > 0.0) last = i;
  }
  if (first != INT_MAX) atomicMin(&sh_first, first);
  if (last >= 0) atomicMax(&sh_last, last);
  __syncthreads();
  if (tid == 0) {
    const int k = (sh_first != INT_MAX) ? sh_first : sh_last;
    out_tokens[int64_t(b) * (n_draft + 1) + st.j] = e0 + k;
  }
}

const char* const kStageNames[] = {"row_stats", "decide", "resid_norm", "weights", "draw"};
constexpr int kNumStages = 5;

template <typename T>
hipError_t launch_typed(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* ev) {
  const T* draft = static_cast<const T*>(a.draft);
  const T* target = static_cast<const T*>(a.target);
  const int R = 2 * a.n_draft + 1;
  const int nch = w.n_stats_chunks;
  const int nsch = w.n_samp_chunks;
  const int64_t stat_items = int64_t(a.batch) * R * nch;
  const unsigned samp_items = unsigned(int64_t(a.batch) * nsch);
  int stage = 0;
  auto mark = [&]() {
    if (ev != nullptr) (void)hipEventRecord(ev[stage], stream);
    ++stage;
  };
  mark();
  hipLaunchKernelGGL(row_stats_kernel<T>, dim3(unsigned(stat_items)), dim3(kThreads), 0, stream, draft, target,
                     a.temperature, a.n_draft, a.vocab, nch, w.partials);
  mark();
  hipLaunchKernelGGL(decide_kernel<T>, dim3(a.batch), dim3(kDecideThreads), 0, stream, draft, target, a.tokens,
                     a.accept_u, a.temperature, a.n_draft, a.vocab, nch, w.partials, w.row_lse, w.row_argmax, w.seq,
                     a.out_tokens, a.out_n);
  mark();
  hipLaunchKernelGGL(resid_norm_kernel<T>, dim3(samp_items), dim3(kThreads), 0, stream, draft, target, a.n_draft,
                     a.vocab, nsch, w.seq, w.norm_part);
  mark();
  hipLaunchKernelGGL(weights_kernel<T>, dim3(samp_items), dim3(kThreads), 0, stream, draft, target, a.n_draft,
                     a.vocab, nsch, w.seq, w.norm_part, w.wsum_part);
  mark();
  hipLaunchKernelGGL(draw_kernel<T>, dim3(a.batch), dim3(kThreads), 0, stream, draft, target, a.sample_u,
                     a.n_draft, a.vocab, nsch, w.seq, w.norm_part, w.wsum_part, a.out_tokens);
  if (ev != nullptr) (void)hipEventRecord(ev[stage], stream);
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
