// gfx950 kernels for batched speculative-sampling verification.
//
// Pages: lesson "추측 디코딩 — 초안 작성, 검증, 반복" (factory.pai-world.com),
// section "핵심 알고리즘(Core algorithm)" steps 4-6 with "Step 1: 거절 단계" (the
// accept test) and "Step 2: 잔차 분포" (the residual); blog "…투기적 디코딩
// (Speculative Decoding)과 검증 샘플링 아키텍처" (tech.blogsailing.com), section 3's
// verification loop.
//
// One launch per call, on the caller's stream. Each workgroup takes a role
// from its index (role_of); a workgroup only ever waits for workgroups that
// precede it in the launch order, and every wait is bounded.
//
//   row statistics  one workgroup per item (kStatBytes of one row): fp32
//                   max, sum of 2^(z*c - fl(max*c)) with c = log2(e)/T and
//                   first argmax, stored as the item's partial. Pure
//                   streaming, HBM-bound; greedy sequences skip their draft
//                   rows.
//   decision        one workgroup per sequence (and stage, in a lazy call),
//                   after its items: merges the row partials into
//                   log-normalisers, takes the accept decisions, writes them
//                   out (the token itself when greedy) and publishes the
//                   draw's record, or in a lazy call lets the sequence's next
//                   stage go on.
//   draw member     one workgroup per (sampled sequence, kMemberElems logits of
//                   each of the draw's row(s)), after the decision: fp64 exps
//                   of its logits summed into a member record. The last member
//                   of a sequence to report is its finisher: the fp64
//                   normalisers and member weights from the records, the
//                   member and then its sub-chunk where the inverse CDF
//                   crosses u*S, an exact rescan of that sub-chunk's tokens
//                   (loaded while the sub-chunk is picked), the token.
//
// A sampling call (no drafts) is a launch of its own kernel (sample_kernel)
// of draw members only, each taking its own largest logit as the reference of
// its exps; the finisher rescales them.
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
constexpr int kMaxRows = 2 * 64 + 1;
constexpr int kStatVecs = kStatBytes / 16 / kThreads;  // 16-byte vectors per thread per item
static_assert(kMaxMembers <= 64, "one member per lane of each of the finisher's waves");


__device__ __forceinline__ bool temperature_valid(float t) {
  return t == 0.0f || (t >= kMinTemperature && t <= kFltMax);
}

// c in 2^(z*c) == exp(z/T); finite for T >= kMinTemperature.
__device__ __forceinline__ float exp2_coef(float t) { return kLog2e / t; }

// K = fl(m * c), never contracted into a neighbouring add.
__device__ __forceinline__ float scaled_max(float m, float c) { return __fmul_rn(m, c); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Diagnostic builds (-DSPECV_TRACE) stamp the wall clock (100 MHz) at fixed
// points of each workgroup's work: kernel 0 the draw members (sequence * nm +
// member), 1 the finishers (sequence), 2 the row-statistics items (sequence *
// items per sequence + item).
#if defined(SPECV_TRACE)
constexpr int kTraceSlots = 8;
constexpr int kTraceBlocks = 1 << 16;
__device__ uint64_t g_trace[3][kTraceBlocks * kTraceSlots];
__shared__ unsigned g_trace_idx;
__device__ __forceinline__ void trace_at(int kernel, unsigned idx, int slot) {
  if (threadIdx.x == 0 && idx < kTraceBlocks) g_trace[kernel][idx * kTraceSlots + slot] = wall_clock64();
}
__device__ __forceinline__ void trace_set(unsigned idx) {
  if (threadIdx.x == 0) g_trace_idx = idx;
}
__device__ __forceinline__ void trace(int kernel, int slot) {
  if (threadIdx.x == 0) trace_at(kernel, g_trace_idx, slot);
}
#else
__device__ __forceinline__ void trace_at(int, unsigned, int) {}
__device__ __forceinline__ void trace_set(unsigned) {}
__device__ __forceinline__ void trace(int, int) {}
#endif

// ---------------------------------------------------------------------------
// Workgroup barriers. Workgroups exchange data through LDS only at barriers,
// so a barrier waits for LDS traffic alone: HIP's __syncthreads also waits for
// every global load and store in flight (a release fence), which would stall
// loads a workgroup keeps in flight across a barrier.

__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Uniform ORs of two per-thread flags over the workgroup (bit 0: a, bit 1: b).
__shared__ int g_vote2[kThreads / 64];
__device__ __forceinline__ int block_any2(bool a, bool b) {
  const unsigned long long ma = __ballot(a), mb = __ballot(b);
  if ((threadIdx.x & 63) == 0) g_vote2[threadIdx.x >> 6] = (ma != 0ull ? 1 : 0) | (mb != 0ull ? 2 : 0);
  barrier();
  int r = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) r |= g_vote2[w];
  barrier();
  return r;
}


// ---------------------------------------------------------------------------
// Cross-lane steps within a wave through DPP (data-parallel primitives: an
// operand read from another lane of the same row of 16, or broadcast from the
// last lane of a row), which cost about as much as an ordinary VALU op, where
// a shuffle through the LDS crossbar waits on a memory round trip.
//
// Lane patterns: kXor1 and kXor2 exchange within quads; kHalfMirror pairs
// lane i with 7 - i and kMirror lane i with 15 - i, so after kXor1, kXor2,
// kHalfMirror and kMirror every lane holds its row's combination (the
// combining operation must be commutative and associative up to the fixed
// order this gives). kRowShr(k) reads lane i - k of the row; kBcast15 and
// kBcast31 read lane 15 (31) into the rows that row_mask enables; kWaveShr1
// reads lane i - 1 of the wave. Lanes with no source, or outside row_mask,
// get `old`.
constexpr int kXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kBcast15 = 0x142;
constexpr int kBcast31 = 0x143;
constexpr int kWaveShr1 = 0x138;
constexpr int kRowShr(int k) { return 0x110 + k; }

template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old = 0u) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(v), kCtrl, kRowMask, 0xf, false));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp_f32(float v, float old = 0.0f) {
  return __uint_as_float(dpp_u32<kCtrl, kRowMask>(__float_as_uint(v), __float_as_uint(old)));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ int dpp_i32(int v, int old = 0) {
  return int(dpp_u32<kCtrl, kRowMask>(uint32_t(v), uint32_t(old)));
}
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {  // `old` is 0.0
  const uint64_t b = double_to_bits(v);
  const uint32_t lo = dpp_u32<kCtrl, kRowMask>(uint32_t(b)), hi = dpp_u32<kCtrl, kRowMask>(uint32_t(b >> 32));
  return bits_to_double((uint64_t(hi) << 32) | lo);
}

// Lane `lane` (uniform) of v.
__device__ __forceinline__ double read_lane(double v, int lane) {
  const uint64_t b = double_to_bits(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b)), lane));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(b >> 32)), lane));
  return bits_to_double((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ double row_sum(double v) {
  v += dpp_f64<kXor1>(v);
  v += dpp_f64<kXor2>(v);
  v += dpp_f64<kHalfMirror>(v);
  v += dpp_f64<kMirror>(v);
  return v;
}

// Sum over the wave, the same in every lane (rows added in a fixed order).
__device__ __forceinline__ double wave_sum(double v) {
  v = row_sum(v);
  return (read_lane(v, 0) + read_lane(v, 16)) + (read_lane(v, 32) + read_lane(v, 48));
}

// Inclusive prefix sums over the wave, in lane order.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_f64<kRowShr(1)>(v);
  v += dpp_f64<kRowShr(2)>(v);
  v += dpp_f64<kRowShr(4)>(v);
  v += dpp_f64<kRowShr(8)>(v);
  v += dpp_f64<kBcast15, 0xa>(v);
  v += dpp_f64<kBcast31, 0xc>(v);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i32<kRowShr(1)>(v);
  v += dpp_i32<kRowShr(2)>(v);
  v += dpp_i32<kRowShr(4)>(v);
  v += dpp_i32<kRowShr(8)>(v);
  v += dpp_i32<kBcast15, 0xa>(v);
  v += dpp_i32<kBcast31, 0xc>(v);
  return v;
}

// A read-only value at a uniform address, through the constant address space
// (a scalar load: counted apart from the vector loads in flight, so using it
// does not wait for them). Only for inputs the kernel never writes.
template <typename V>
__device__ __forceinline__ V load_uniform(const V* p) {
  typedef const __attribute__((address_space(4))) V ConstV;
  return *(ConstV*)(p);
}

// ---------------------------------------------------------------------------
// Logit access.

template <typename T>
struct Logit;

template <>
struct Logit<float> {
  static constexpr int kVec = 4;   // logits per 16-byte load
  static constexpr int kPer = 16;  // logits of one row per draw-member thread
  __device__ static float at(const float* p, int64_t i) { return p[i]; }
  __device__ static uint32_t bits(const float* p, int64_t i) { return __float_as_uint(p[i]); }
  __device__ static float from_bits(uint32_t b) { return __uint_as_float(b); }
  static constexpr uint32_t kNegInf = 0xff800000u;
  // Element k of logits packed four per uint4 (k a compile-time constant).
  template <int n>
  __device__ static float element(const uint4 (&x)[n], int k) {
    const uint4& v = x[k / 4];
    const uint32_t w = (k % 4 == 0) ? v.x : (k % 4 == 1) ? v.y : (k % 4 == 2) ? v.z : v.w;
    return __uint_as_float(w);
  }
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
  static constexpr int kPer = 16;
  __device__ static float at(const uint16_t* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
  __device__ static uint32_t bits(const uint16_t* p, int64_t i) { return p[i]; }
  __device__ static float from_bits(uint32_t b) { return __uint_as_float(b << 16); }
  static constexpr uint32_t kNegInf = 0xff80u;
  // Element k of logits packed eight per uint4 (k a compile-time constant).
  template <int n>
  __device__ static float element(const uint4 (&x)[n], int k) {
    const uint4& v = x[k / 8];
    const int h = k % 8;
    const uint32_t w = (h < 2) ? v.x : (h < 4) ? v.y : (h < 6) ? v.z : v.w;
    return __uint_as_float((h & 1) ? (w & 0xffff0000u) : (w << 16));
  }
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

// kPer consecutive logits of a row from element e, packed as stored (16-byte
// loads when aligned and inside the row; elements past `vocab` read as -inf).
template <typename T, int n>
__device__ __forceinline__ void load_packed(const T* __restrict__ row, int e, int vocab, bool vec_ok, uint4 (&x)[n]) {
  constexpr int kVec = Logit<T>::kVec;
  if (vec_ok && e + n * kVec <= vocab) {
    const uint4* __restrict__ p = reinterpret_cast<const uint4*>(row + e);
#pragma unroll
    for (int u = 0; u < n; ++u) x[u] = p[u];
  } else {
    uint32_t w[4 * n];
#pragma unroll
    for (int i = 0; i < 4 * n; ++i) w[i] = 0u;
#pragma unroll
    for (int k = 0; k < n * kVec; ++k) {
      const uint32_t v = (e + k < vocab) ? Logit<T>::bits(row, e + k) : Logit<T>::kNegInf;
      if (kVec == 4)
        w[k] = v;
      else
        w[k / 2] |= (k & 1) ? (v << 16) : v;
    }
#pragma unroll
    for (int u = 0; u < n; ++u) x[u] = make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]);
  }
}

// Element k (a run-time index) of logits packed as stored, by selection:
// registers cannot be indexed at run time.
template <typename T, int n>
__device__ __forceinline__ float element_at(const uint4 (&x)[n], int k) {
  float r = 0.0f;
#pragma unroll
  for (int kk = 0; kk < n * Logit<T>::kVec; ++kk) r = (k == kk) ? Logit<T>::element(x, kk) : r;
  return r;
}

// ---------------------------------------------------------------------------
// Block reductions (fixed order). `red` holds 2 * kWaves doubles.

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  barrier();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  barrier();
  double total = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) total += red[w];
  return total;
}

// ---------------------------------------------------------------------------
// Row statistics.

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

// One merge step with the state DPP pattern kCtrl brings from another lane
// (lanes outside kRowMask merge the empty state: no change).
template <bool kSampled, int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ void merge_step(float& m, float& s, int& idx, float c) {
  const float m2 = dpp_f32<kCtrl, kRowMask>(m, -INFINITY);
  const float s2 = dpp_f32<kCtrl, kRowMask>(s, 0.0f);
  const int i2 = dpp_i32<kCtrl, kRowMask>(idx, INT_MAX);
  acc_merge<kSampled>(m, s, idx, m2, s2, i2, c);
}


// ---------------------------------------------------------------------------
// Device-coherent words. Records that one workgroup hands to another within a
// launch are written and read only as agent-scope relaxed atomics: these
// bypass the per-XCD L2s' stale or dirty copies, so no L2 write-back or
// invalidation (what an agent-scope release or acquire fence costs) is ever
// needed.

__device__ __forceinline__ void put_u64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_u64(const void* p) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_d(double* p, double v) { put_u64(p, double_to_bits(v)); }
__device__ __forceinline__ void put_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Records written by one workgroup and read by another within a launch. Every
// word is a 32-bit payload in its low half and the call's tag in its high half
// (the host numbers its calls 1, 2, ...; never 0), so a reader takes each word
// on its own once its tag is the current call's, needs no order between the
// words of a record, and never takes a word that an earlier call left behind.
// Readers also zero what they take (so words read zero at every call's start,
// also when a captured launch is replayed).
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t payload) { return (uint64_t(tag) << 32) | payload; }
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t tag) { return uint32_t(w >> 32) == tag; }

// Row statistics of one item in two words: the largest logit m with the
// call's tag, and sx = s | v << 31 | (tag & kTag17) << 47, where
// s = sum of 2^(z*c - fl(m*c)) (>= 1/2 when m is finite; 1 for a greedy,
// skipped or all -inf item, where no merge uses it; positive, so its sign bit
// is left out) and v = 1 + the first index of m within the item (0: none).
// The host never numbers a call with tag & kTag17 == 0, so a zeroed sx never
// looks current. (Fewer words per item matter: each is a device-coherent
// store, and with 3 words a B = 256 call took 5 us longer.)
struct PartialRec {
  uint64_t m, sx;
};
constexpr uint32_t kTag17 = 0x1ffffu;
__device__ __forceinline__ uint64_t pack_sx(float s, uint32_t v, uint32_t tag) {
  return uint64_t(__float_as_uint(s) & 0x7fffffffu) | (uint64_t(v) << 31) | (uint64_t(tag & kTag17) << 47);
}
__device__ __forceinline__ bool sx_current(uint64_t w, uint32_t tag) { return uint32_t(w >> 47) == (tag & kTag17); }
// One sequence's decision, published for its draw members.
struct SeqRec {
  uint64_t jm;      // j | mode << 8
  uint64_t mt;      // largest logit of target row j
  uint64_t md;      // largest logit of draft row j (residual draws)
  uint64_t logrho;  // log(Zt/Zd) of row j from the fp32 row sums, as fp32 (residual draws)
};
// One draw member's fp64 sums as 64-bit words (written once each, read by
// the finisher after the member has reported):
struct MemberRec {
  static constexpr int kStatus = 0;       // the call's tag << 32 | 1 if the member saw the decision
  static constexpr int kZt = 1, kZd = 2;  // sums of the target and draft exps
  static constexpr int kA = 3;            // + k: sub-chunk k's sum of et over certainly positive tokens
  static constexpr int kB = kA + kSubs;   // + k: the same sum of ed
  static constexpr int kNUnc = kB + kSubs;  // uncertain-sign tokens (kUncMax + 1: more than listed)
  static constexpr int kPos = kNUnc + 1;    // + i: their positions, ascending
  static constexpr int kEt = kPos + kUncMax;  // + i: their exps in the target row
  static constexpr int kEd = kEt + kUncMax;   // + i: and in the draft row
  static constexpr int kAt = kEd + kUncMax;   // the member's sums of et and ed over certainly positive tokens
  static constexpr int kBt = kAt + 1;
  static constexpr int kWords = kBt + 1;
  // A sampling call's members have no draft row and no uncertain tokens; those
  // slots hold the member's largest logit (the reference of its exps) and
  // the first index where it occurs.
  static constexpr int kMax = kZd;
  static constexpr int kArg = kNUnc;
  uint64_t w[kWords];
};

__device__ __forceinline__ void put_d_word(MemberRec* r, int word, double v) { put_d(reinterpret_cast<double*>(&r->w[word]), v); }

// Everything the launches need; passed by value.
struct Params {
  const void* draft;
  const void* target;
  const int* tokens;
  const float* accept_u;
  const float* sample_u;
  const float* temperature;
  int* out_tokens;
  int* out_n;
  double* row_lse;
  int* row_argmax;
  PartialRec* partials;  // [batch][2N+1][nch], one per item
  SeqRec* seq;           // [batch]
  MemberRec* records;    // [batch][nm]
  int* draw_done;        // [batch * kCounterStride] draw members done (zero between launches)
  int items_per_seq;     // whole call: row-statistics items per sequence, (2N+1) * nch
  int lag;               // whole call: draw members of sequence b follow the row statistics of sequence b + lag
  int batch;
  int n_draft;
  int vocab;
  int nch;    // row-statistics chunks per row
  int chunk;  // logits per row-statistics chunk
  int nm;     // draw members per sequence
  uint32_t flags;       // kVecOk: rows start 16-byte aligned; kDebug: check that the uniforms lie in [0, 1)
  uint32_t tag;         // this call's number (never 0): the high half of every hand-off word
  uint32_t wait_ticks;  // bound of every wait, in ticks of the 100 MHz wall clock
  // A whole call verifies positions [0, N) in one stage. A lazy call runs
  // stages s = 0 .. n_stages-1 over positions [st_bound[s], st_bound[s+1])
  // in the same launch: the statistics groups of every sequence for stage 0,
  // then for stage 1, ..., then every sequence's draw members. The decision
  // of stage s leaves each workgroup of the sequence's stage s+1 a go-on word
  // (see alive_item): 1 if its drafts so far are all accepted, else 0.
  int lazy;
  int n_stages;
  int st_bound[kMaxLazyStages + 1];
  int st_base[kMaxLazyStages + 1];  // lazy: first workgroup of stage s; st_base[n_stages]: the draw members
  uint64_t* alive;                  // lazy: the go-on words, [batch][(2N+1) * nch + kMaxLazyStages]
};
constexpr uint32_t kVecOk = 1, kDebug = 2;

// Partial of item (row r, chunk c) of sequence b.
__device__ __forceinline__ PartialRec* partial_at(const Params& P, int b, int r, int c) {
  return P.partials + (int64_t(b) * (2 * P.n_draft + 1) + r) * P.nch + c;
}

// Stage s: positions [lo, hi).
struct Stage {
  int s, lo, hi;
};
__device__ __forceinline__ Stage stage_at(const Params& P, int s) { return Stage{s, P.st_bound[s], P.st_bound[s + 1]}; }
// Rows a sequence reads in a stage: draft and target rows lo..hi-1, and
// target row N if hi = N.
__device__ __forceinline__ int stage_rows(const Params& P, const Stage& st) {
  return 2 * (st.hi - st.lo) + (st.hi == P.n_draft ? 1 : 0);
}
// Row lr of a stage's rows as a row of the sequence (draft rows 0..N-1,
// then target rows 0..N).
__device__ __forceinline__ int global_row(const Params& P, const Stage& st, int lr) {
  const int n = st.hi - st.lo;
  return lr < n ? st.lo + lr : (lr < 2 * n ? P.n_draft + st.lo + (lr - n) : 2 * P.n_draft);
}
// The go-on words of a lazy call: one per row-statistics item (row r, chunk
// c) and one per decision of stage s of sequence b, each written by the
// sequence's decision of the stage before and taken (and zeroed) by the
// workgroup it is for.
__device__ __forceinline__ int64_t alive_per_seq(const Params& P) {
  return int64_t(2 * P.n_draft + 1) * P.nch + kMaxLazyStages;
}
__device__ __forceinline__ uint64_t* alive_item(const Params& P, int b, int r, int c) {
  return P.alive + int64_t(b) * alive_per_seq(P) + int64_t(r) * P.nch + c;
}
__device__ __forceinline__ uint64_t* alive_dec(const Params& P, int b, int s) {
  return P.alive + int64_t(b) * alive_per_seq(P) + int64_t(2 * P.n_draft + 1) * P.nch + s;
}

// One row-statistics item: chunk c of row r of sequence b.
struct Item {
  int b, r, c;
  bool live;  // in range and read (greedy sequences skip draft rows; invalid ones skip everything)
  bool sampled;
  float coef;  // log2(e)/T when sampled
  int64_t row_flat;
  int e0, e1;  // chunk [e0, e1) of the row
  int ea, nv;  // first 16-byte aligned element, whole vectors from there
  int et;      // first element after the vectors
};

template <typename T>
__device__ __forceinline__ Item item_at(const Params& P, const Stage& st, int b, int idx) {
  constexpr int kVec = Logit<T>::kVec;
  Item it;
  it.live = false;
  const int N = P.n_draft;
  it.c = idx % P.nch;
  it.b = b;
  it.r = global_row(P, st, idx / P.nch);
  const float temp = load_uniform(P.temperature + it.b);
  if (!temperature_valid(temp) || (temp == 0.0f && it.r < N)) return it;
  it.live = true;
  it.sampled = temp != 0.0f;
  it.coef = it.sampled ? exp2_coef(temp) : 0.0f;
  it.row_flat = it.r < N ? (int64_t(it.b) * N + it.r) * P.vocab : (int64_t(it.b) * (N + 1) + (it.r - N)) * P.vocab;
  it.e0 = it.c * P.chunk;
  it.e1 = min(P.vocab, it.e0 + P.chunk);
  // Element g of a logits buffer is 16-byte aligned iff g % kVec == 0 (the
  // buffer base is 16-byte aligned); a misaligned chunk start peels a head.
  const int mis = int((it.row_flat + it.e0) % kVec);
  it.ea = min(it.e1, it.e0 + (kVec - mis) % kVec);
  it.nv = (it.e1 - it.ea) / kVec;
  it.et = it.ea + it.nv * kVec;
  return it;
}

template <typename T>
__device__ __forceinline__ const T* item_row(const Params& P, const Item& it) {
  return static_cast<const T*>(it.r < P.n_draft ? P.draft : P.target) + it.row_flat;
}

// An item's logits in flight: this thread's 16-byte vectors tid + u*kThreads
// and its head and tail element (raw bits). Every
// load is issued unconditionally at a clamped, valid address (the fold
// ignores what lies outside the item): loads under per-thread branches make
// the compiler wait for every load in flight where the branches join.
struct ItemRegs {
  uint4 x[kStatVecs];
  uint32_t head, tail;
};

// A 16-byte load marked non-temporal (streamed through the caches). The
// statistics pass reads each logit once; with the hint the stream of 16-byte
// loads runs at 6.5 TB/s where plain loads reach 5.7 on this part.
typedef unsigned StreamV4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const StreamV4 t = __builtin_nontemporal_load(reinterpret_cast<const StreamV4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <typename T>
__device__ __forceinline__ void item_load(const Params& P, const Item& it, ItemRegs& g) {
  if (!it.live) return;
  const int tid = threadIdx.x;
  const T* row = item_row<T>(P, it);
  // The bulk first, so that nothing waits before it is in flight.
  if (it.nv > 0) {
    const uint4* __restrict__ v = reinterpret_cast<const uint4*>(row + it.ea);
#pragma unroll
    for (int u = 0; u < kStatVecs; ++u) g.x[u] = load_stream(v + min(tid + u * kThreads, it.nv - 1));
  }
  // Head and tail elements exist only for chunks that are not 16-byte aligned
  // (a uniform test).
  if (it.ea > it.e0 || it.et < it.e1) {
    g.head = Logit<T>::bits(row, min(it.e0 + tid, it.e1 - 1));
    g.tail = Logit<T>::bits(row, max(it.e0, min(it.et + tid, it.e1 - 1)));
  } else {
    g.head = 0u;
    g.tail = 0u;
  }
}

// Largest of three floats in one instruction. The logits are finite or
// -inf, so the quieting of signalling NaNs that fmaxf implies (an extra
// instruction per operand) is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}


// Over the wave, the same in every lane (rows combined in a fixed order).
__device__ __forceinline__ float lane_f(float v, int lane) { return __int_as_float(read_lane(__float_as_int(v), lane)); }
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kXor1>(v));
  v = fmaxf(v, dpp_f32<kXor2>(v));
  v = fmaxf(v, dpp_f32<kHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ int wave_min(int v) {
  v = min(v, dpp_i32<kXor1>(v));
  v = min(v, dpp_i32<kXor2>(v));
  v = min(v, dpp_i32<kHalfMirror>(v));
  v = min(v, dpp_i32<kMirror>(v));
  return min(min(read_lane(v, 0), read_lane(v, 16)), min(read_lane(v, 32), read_lane(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kXor1>(v);
  v += dpp_f32<kXor2>(v);
  v += dpp_f32<kHalfMirror>(v);
  v += dpp_f32<kMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// A folded item: thread 0 holds the merged state.
struct Partial {
  float m, s;
  int idx;
};

template <int n>
__device__ __forceinline__ float max_of(const float (&v)[n]) {
  static_assert(n == 4 || n == 8, "a 16-byte group of logits");
  float a = max3(v[0], v[1], v[2]);
  a = max3(a, v[3], v[n == 4 ? 3 : 4]);
  if (n == 8) {
    a = max3(a, v[5], v[6]);
    a = max3(a, v[7], v[7]);
  }
  return a;
}

// Sum of 2^(z*c - k) over a group (a fixed tree).
template <int n>
__device__ __forceinline__ float group_exp_sum(const float (&v)[n], float c, float k) {
  float e[n];
#pragma unroll
  for (int q = 0; q < n; ++q) e[q] = fast_exp2(fmaf(v[q], c, -k));
#pragma unroll
  for (int w = 1; w < n; w *= 2)
#pragma unroll
    for (int q = 0; q + w < n; q += 2 * w) e[q] += e[q + w];
  return e[0];
}

// One wave's share of a loaded item, folded group by group as the loads
// arrive: each thread tracks its largest logit and where it first occurs
// (its head element, one of its 16-byte groups, or its tail element); for a
// sampled row it sums 2^(z*c - k) against one wave-wide reference k, set from
// the first group with a finite logit and raised (rescaling the sums) only
// when a group's logit would exceed it by 2^64, so the common path has no
// per-group rescaling. At the end the sums are brought to k = fl(M*c) with M
// the wave's largest logit. The first index of M is looked for only by the
// lanes that hold it, in the group where they first saw it, read again (from
// the cache). kFull: every group of every thread lies inside the item
// (nothing to mask). Returns the wave's partial, the same in every lane.
template <typename T, bool kSampled, bool kFull>
__device__ __forceinline__ Partial wave_fold(const Params& P, const Item& it, ItemRegs& g) {
  constexpr int kVec = Logit<T>::kVec;
  const int tid = threadIdx.x;
  const float c = it.coef;
  const float hv = tid < it.ea - it.e0 ? Logit<T>::from_bits(g.head) : -INFINITY;
  const float tv = tid < it.e1 - it.et ? Logit<T>::from_bits(g.tail) : -INFINITY;
  // `where` is -1 for the head, u for group u, kStatVecs for the tail; a
  // strict '>' keeps the first place (the thread's indices increase in that
  // order).
  float tmax = hv;
  int where = -1;
  // The wave's reference (uniform). It starts finite and below every scaled
  // logit, so the first finite logit raises it, -inf logits add exactly 0
  // before that, and neither check needs a test of its own.
  float k = -FLT_MAX;
  float s = 0.0f;
  // Folds one group (values v, maximum gm) into the state.
  auto fold = [&](const auto& v, float gm, int place, bool in) {
    const bool up = gm > tmax;
    where = up ? place : where;
    tmax = up ? gm : tmax;
    if (kSampled) {
      if (__ballot(fmaf(gm, c, -k) > 64.0f)) {
        // Rare: raise the reference to the wave's largest logit so far.
        const float k2 = scaled_max(wave_max(tmax), c);
        s = s * fast_exp2(k - k2);  // s is 0 until the first raise
        k = k2;
      }
      const float e = group_exp_sum(v, c, k);
      s += in ? e : 0.0f;
    }
  };
  {
    const float v[1] = {hv};
    fold(v, hv, -1, true);
  }
#pragma unroll
  for (int u = 0; u < kStatVecs; ++u) {
    float v[kVec];
    Logit<T>::unpack(g.x[u], v);
    const bool in = kFull || tid + u * kThreads < it.nv;
    fold(v, in ? max_of(v) : -INFINITY, u, in);
  }
  {
    const float v[1] = {tv};
    fold(v, tv, kStatVecs, true);
  }
  const float mw = wave_max(tmax);
  if (kSampled) s = (mw == -INFINITY) ? 0.0f : wave_sum(s * fast_exp2(k - scaled_max(mw, c)));
  // First index of M.
  const bool hold = mw != -INFINITY && tmax == mw;
  int idx = INT_MAX;
  if (hold && where < 0) idx = it.e0 + tid;
  if (hold && where == kStatVecs) idx = it.et + tid;
  if (hold && where >= 0 && where < kStatVecs) {
    const uint4 again = reinterpret_cast<const uint4*>(item_row<T>(P, it) + it.ea)[tid + where * kThreads];
    float v[kVec];
    Logit<T>::unpack(again, v);
    int first = kVec - 1;
#pragma unroll
    for (int q = kVec - 1; q >= 0; --q) first = (v[q] == mw) ? q : first;
    idx = it.ea + (tid + where * kThreads) * kVec + first;
  }
  if (mw != -INFINITY) idx = wave_min(idx);
  return Partial{mw, s, idx};
}

template <typename T>
__device__ __forceinline__ Partial item_reduce(const Params& P, const Item& it, ItemRegs& g) {
  const bool full = it.ea == it.e0 && it.et == it.e1 && it.nv == kStatVecs * kThreads;
  if (it.sampled) return full ? wave_fold<T, true, true>(P, it, g) : wave_fold<T, true, false>(P, it, g);
  return full ? wave_fold<T, false, true>(P, it, g) : wave_fold<T, false, false>(P, it, g);
}

__shared__ Partial g_wave_part[kWaves];

// The item's partial: the waves' partials (lane 63 of each) merged in wave
// order through LDS, stored by thread 0 (see PartialRec).
__device__ __forceinline__ void partial_write(const Params& P, const Item& it, const Partial& q) {
  if ((threadIdx.x & 63) == 63) g_wave_part[threadIdx.x >> 6] = q;
  barrier();
  if (threadIdx.x == 0) {
    Partial a = g_wave_part[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const Partial& o = g_wave_part[w];
      if (it.live && it.sampled)
        acc_merge<true>(a.m, a.s, a.idx, o.m, o.s, o.idx, it.coef);
      else
        acc_merge<false>(a.m, a.s, a.idx, o.m, o.s, o.idx, 0.0f);
    }
    PartialRec* p = partial_at(P, it.b, it.r, it.c);
    const uint32_t v = (it.live && a.idx >= it.e0 && a.idx < it.e1) ? uint32_t(a.idx - it.e0 + 1) : 0u;
    put_u64(&p->m, tagged(P.tag, __float_as_uint(a.m)));
    put_u64(&p->sx, pack_sx(a.s != 0.0f ? a.s : 1.0f, v, P.tag));
  }
}

// ---------------------------------------------------------------------------
// Hand-over between the workgroups of one launch.

__shared__ int g_last;

// Counts this workgroup as done with a unit that `total` workgroups of the
// launch each report once. Returns true, in every thread, in the workgroup that
// reports last, which resets the count to zero for the next launch. Each
// thread's record stores (device-coherent words) have completed before the
// workgroup reports, so the last one reads every record complete. No
// workgroup ever waits for another.
__device__ __forceinline__ bool last_arrival(int* count, int total) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_last = (prev == total - 1);
    if (prev == total - 1) put_i(count, 0);
  }
  __syncthreads();
  return g_last != 0;
}

// ---------------------------------------------------------------------------
// Decision.

// Publishes sequence b's decision for its draw members. Only sampled
// sequences (T > 0) have draw members waiting; the last of them zeroes the
// record again.
__device__ __forceinline__ void publish(const Params& P, int b, int mode, int j, float mt, float md, double log_rho) {
  SeqRec* q = P.seq + b;
  put_u64(&q->jm, tagged(P.tag, uint32_t(j) | (uint32_t(mode) << 8)));
  put_u64(&q->mt, tagged(P.tag, __float_as_uint(mt)));
  put_u64(&q->md, tagged(P.tag, __float_as_uint(md)));
  put_u64(&q->logrho, tagged(P.tag, __float_as_uint(float(log_rho))));
}

// Whether sequence b's draw members wait for its decision: a positive valid
// temperature (invalid tokens still give it a decision, with no draw).
__device__ __forceinline__ bool has_draw_members(float t) { return t > 0.0f && temperature_valid(t); }

constexpr int kStageParts = 256;  // row partials the decision holds in LDS at once

// Wall-clock deadline of a wait that starts now (s_memrealtime: 100 MHz).
__device__ __forceinline__ uint64_t deadline_after(uint64_t ticks) { return wall_clock64() + ticks; }
__device__ __forceinline__ bool before(uint64_t deadline) { return wall_clock64() < deadline; }

__shared__ int g_go;

// A lazy call's go-on word for this workgroup (stage >= 1): waits for it
// (until the call's wait bound), takes and zeroes it. Returns 1 (the
// sequence goes on in this stage), 0 (it ended in an earlier stage) or -1
// (the wait gave up), the same in every thread.
__device__ __forceinline__ int take_go(const Params& P, uint64_t* w) {
  if (threadIdx.x == 0) {
    uint64_t v = get_u64(w);
    if (!has_tag(v, P.tag)) {
      const uint64_t deadline = deadline_after(P.wait_ticks);
      while (!has_tag(v, P.tag) && before(deadline)) {
        __builtin_amdgcn_s_sleep(8);
        v = get_u64(w);
      }
    }
    const bool ok = P.wait_ticks != 0 && has_tag(v, P.tag);
    put_u64(w, 0);
    g_go = ok ? int(uint32_t(v) & 1u) : -1;
  }
  barrier();
  return g_go;
}

// The decision of stage st of sequence b leaves the go-on words of the
// sequence's next stage (whole workgroup; nothing after a lazy call's last
// stage or in a whole call).
__device__ __forceinline__ void signal_go(const Params& P, const Stage& st, int b, bool go) {
  if (!P.lazy || st.s + 1 >= P.n_stages) return;
  const Stage nx = stage_at(P, st.s + 1);
  const int n = stage_rows(P, nx) * P.nch;
  const uint64_t v = tagged(P.tag, go ? 1u : 0u);
  for (int k = int(threadIdx.x); k <= n; k += kThreads)
    put_u64(k < n ? alive_item(P, b, global_row(P, nx, k / P.nch), k % P.nch) : alive_dec(P, b, nx.s), v);
}

struct DecideShared {
  float row_m[kMaxRows];
  double row_logz[kMaxRows];
  int row_idx[kMaxRows];
  Partial part[kStageParts];
  int tok[kMaxRows / 2];
  unsigned long long rej_mask;
};
static_assert(kStageParts == kThreads, "one staged row partial per thread");
static_assert(int64_t(kMaxVocab) * 4 / kStatBytes <= kStageParts, "a row's partials fit one group");

static_assert(sizeof(kExp2Table) == kThreads * sizeof(double), "the exp table is filled one entry per thread");

// A draw workgroup's LDS. The sampling kernel stages only the first words of
// each member record (it has no draft row and no uncertain tokens), which
// keeps its LDS small enough for eight workgroups per CU.
template <bool kSample>
struct DrawShared {
  static constexpr int kStageWords = kSample ? MemberRec::kNUnc + 1 : MemberRec::kWords;
  double red[4 * kWaves];
  double exp2_tab[kThreads];  // kExp2Table, for exp_nonpos_tab (members and the finisher)
  union {
    struct {
      double unc_et[2][kThreads];  // member: staged uncertain tokens (two per thread)
      double unc_ed[2][kThreads];
    } mem;
    uint64_t stage[kMaxMembers * kStageWords];  // finisher: the sequence's member records
  };
  double tw[32 * 16];  // finisher: the crossing sub-chunk's token weights
  float wave_m[kWaves];            // sampling member: each wave's largest logit and its first index
  int wave_i[kWaves];
  int unc_base[kWaves];
};

struct Shared {
  union {
    DecideShared dec;
    DrawShared<false> drw;
  } u;
};

__shared__ Shared g_shared;
__shared__ DrawShared<true> g_sample_shared;

struct SeqInfo {
  float temp;
  int mode;
  int j;
  float m_target;
  float m_draft;
  double log_rho;  // log(Zt/Zd) of row j from the fp32 row sums (residual only)
};

// A SeqInfo the workgroup holds in common (read from LDS), as wave-uniform
// values: scalar address arithmetic and branches.
__device__ __forceinline__ SeqInfo uniform(const SeqInfo& s) {
  auto f = [](float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); };
  const uint64_t lr = double_to_bits(s.log_rho);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(lr))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(lr >> 32))));
  return SeqInfo{f(s.temp), __builtin_amdgcn_readfirstlane(s.mode), __builtin_amdgcn_readfirstlane(s.j), f(s.m_target),
                 f(s.m_draft), bits_to_double((uint64_t(hi) << 32) | lo)};
}

// Whether a whole call reads each sequence's target row N late in the launch
// (after the accept tests; see decide and role_of). Row N only matters to a
// sequence's draw when every draft is accepted, which long drafts rarely
// are; there it takes about 1.7 us off B = 32, N = 16 fp32, while for
// shorter drafts it moves nothing or costs (B = 64, N = 5 level, B = 256,
// N = 7 2 us slower).
constexpr int kLateRowNDrafts = 8;
__device__ __forceinline__ bool late_row_n(const Params& P) { return !P.lazy && P.n_draft >= kLateRowNDrafts; }

// Waits (until `deadline`) for partial q of this call (its item starts at
// element e0 of the row), then takes it and zeroes its words. Returns false
// if the wait gave up (always, when the wait bound is 0: the host's way to
// exercise this path).
__device__ __forceinline__ bool take_partial(const Params& P, PartialRec* q, int e0, uint64_t deadline,
                                             Partial& out) {
  const uint32_t tag = P.tag;
  uint64_t m = get_u64(&q->m), x = get_u64(&q->sx);
  auto ready = [&] { return has_tag(m, tag) && sx_current(x, tag); };
  while (!ready() && before(deadline)) {
    __builtin_amdgcn_s_sleep(4);
    if (!has_tag(m, tag)) m = get_u64(&q->m);
    if (!sx_current(x, tag)) x = get_u64(&q->sx);
  }
  const bool ok = P.wait_ticks != 0 && ready();
  put_u64(&q->m, 0);
  put_u64(&q->sx, 0);
  const uint32_t v = uint32_t(x >> 31) & 0xffffu;
  out = Partial{__uint_as_float(uint32_t(m)), __uint_as_float(uint32_t(x) & 0x7fffffffu), v ? e0 + int(v) - 1 : INT_MAX};
  return ok;
}

// Row diagnostics lse = NaN, argmax = -1 for sequence b's rows at positions
// >= from (target row N counting as the last position), all of them rows
// that no other workgroup writes: those of later stages when the sequence
// ends in stage st, or its own and later ones when the stage fails.
__device__ __forceinline__ void mark_unread(const Params& P, int b, const Stage& st, int from) {
  const int N = P.n_draft, R = 2 * N + 1;
  double* lse = P.row_lse + int64_t(b) * R;
  int* amax = P.row_argmax + int64_t(b) * R;
  for (int r = int(threadIdx.x); r < R; r += kThreads) {
    const bool mark = r < N ? r >= from : (r < 2 * N ? r - N >= from : (from < N || st.hi == N));
    if (mark) {
      lse[r] = NAN;
      amax[r] = -1;
    }
  }
}

// The decision of stage st for sequence b (whole workgroup, once per
// sequence and stage): per-row log-normalisers and argmaxes from the row
// partials of the stage's rows, the accept tests of its positions [lo, hi),
// the first rejection. Writes the row diagnostics and the accepted prefix; a
// greedy sequence's emitted token and n_accepted too, while a sampled
// sequence's are written by its draw's finisher, from the record published
// here. In a lazy call a sequence whose drafts lo..hi-1 are all accepted
// (hi < N) goes on to the next stage: its drafts so far are written, nothing
// is drawn, and the next stage's workgroups are told to go on. `go` is the
// stage's go-on word (1 for stage 0): 0 means the sequence ended in an
// earlier stage (its items read nothing, so nothing is taken), -1 that the
// wait for the word gave up.
//
// The normalisers come from fp32 row sums (relative error ~1e-6); logs and
// the ratio are taken in fp64, so a decision can only differ from exact
// arithmetic when u is within a few 1e-6 of the ratio.
template <typename T>
__device__ __forceinline__ void decide(const Params& P, Shared& sh, const Stage& st, int b, int go) {
  if (go == 0) {
    signal_go(P, st, b, false);
    return;
  }
  DecideShared& ds = sh.u.dec;
  const int N = P.n_draft;
  const int R = 2 * N + 1;
  const int lo = st.lo, hi = st.hi, ns = hi - lo;
  const bool last = hi == N;
  const int Rs = go > 0 ? stage_rows(P, st) : 0;  // no partials are taken after a failed wait
  // A long draft's target row N is read by items placed later in the launch
  // (just before the sequence's draw members; see role_of): the accept tests
  // do not need it, so its partials are taken after them, and only a
  // sequence that accepts every draft waits for them before its draw is
  // published.
  const bool split = late_row_n(P) && last && Rs > 0;
  const int Rs_main = split ? Rs - 1 : Rs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int* tok = P.tokens + int64_t(b) * N;
  int* otok = P.out_tokens + int64_t(b) * (N + 1);
  double* lse = P.row_lse + int64_t(b) * R;
  int* amax = P.row_argmax + int64_t(b) * R;
  // Every row partial of the launch's rows is taken (and zeroed) whatever the
  // outcome, a group of rows at a time (thread i takes partial i of the
  // group).
  const int pr = P.nch;  // partials per row
  const int rows_per_group = max(1, kStageParts / pr);
  PartialRec* part_b = P.partials + int64_t(b) * R * pr;
  // The inputs are checked where a sequence starts (lo = 0), all N positions
  // at once; thread i < ns tests position lo + i. (n_draft = 0 is the plain
  // draw from one row: no draft tokens, no uniforms to test.)
  const int tv = min(tid, max(N - 1, 0));
  const int dv = N > 0 ? tok[tv] : 0;
  const float uv = N > 0 ? P.accept_u[int64_t(b) * N + tv] : 0.0f;
  const int pos = lo + min(tid, max(ns - 1, 0));
  const int d = ns > 0 ? tok[pos] : 0;
  const float ua = ns > 0 ? P.accept_u[int64_t(b) * N + pos] : 0.0f;
  const float t = load_uniform(P.temperature + b);
  const float us = load_uniform(P.sample_u + b);
  if (tid < ns) ds.tok[lo + tid] = d;
  bool bad = false;
  if (lo == 0) {
    bad = !temperature_valid(t) || (tid < N && (dv < 0 || dv >= P.vocab));
    if (P.flags & kDebug)
      bad = bad || (tid < N && !(uv >= 0.0f && uv < 1.0f)) || (t > 0.0f && !(us >= 0.0f && us < 1.0f));
  }
  const bool greedy = (t == 0.0f);
  // Thread i < ns: the logits of draft token d at position lo + i in its draft
  // and target rows (requested now; used by the accept test).
  float zt = 0.0f, zd = 0.0f;
  if (tid < ns && go > 0 && !greedy && d >= 0 && d < P.vocab) {
    zt = Logit<T>::at(static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + pos) * P.vocab, d);
    zd = Logit<T>::at(static_cast<const T*>(P.draft) + (int64_t(b) * N + pos) * P.vocab, d);
  }
  const bool draws = has_draw_members(t);  // draw members wait for this decision
  const float c = greedy ? 0.0f : exp2_coef(t);
  const double inv_t = greedy ? 0.0 : 1.0 / double(t);
  const int r_first = greedy ? N : 0;
  // Quads of lanes each merge one row: lane k of a quad folds partials k,
  // k + 4, ... of the row in order, then two exchange steps within the quad.
  constexpr int cs = 4;
  const int rows_per_wave = 64 / cs;
  const int seg = lane / cs, k_in_seg = lane - seg * cs;
  bool timed_out = go < 0, any_bad = false;
  // Takes the partials of the stage's rows [first, end) a group at a time
  // and merges them (unless the sequence has failed); returns whether a
  // partial of these rows came too late.
  auto take_rows = [&](int first, int end) -> bool {
    const uint64_t deadline = deadline_after(P.wait_ticks);
    bool rows_late = false;
    for (int rg = first; rg < end; rg += rows_per_group) {
      const int nr = min(rows_per_group, end - rg);
      const int np = nr * pr;
      bool late = false;
      if (tid < np) {
        Partial q;
        const int kc = tid % pr;
        late = !take_partial(P, part_b + int64_t(global_row(P, st, rg + tid / pr)) * pr + kc, kc * P.chunk, deadline, q);
        ds.part[tid] = q;
      }
      // (also the barrier that makes the group's partials visible); the input
      // checks join the first group's vote, so the partials are requested
      // before anything waits for the draft tokens.
      const int vote = block_any2(rg == 0 && bad, late);
      any_bad = any_bad || (vote & 1);
      rows_late = rows_late || (vote & 2);
      if (any_bad || timed_out || rows_late) continue;
      if (rg == 0) trace(2, 4);
      for (int r0 = wave * rows_per_wave; r0 < nr; r0 += kWaves * rows_per_wave) {
        const int rr = r0 + seg;
        const int r = global_row(P, st, rg + min(rr, nr - 1));
        const bool row_ok = rr < nr && r >= r_first;
        float m = -INFINITY, s = 0.0f;
        int idx = INT_MAX;
        if (row_ok) {
          for (int k = k_in_seg; k < pr; k += cs) {
            const Partial& q = ds.part[rr * pr + k];
            if (greedy)
              acc_merge<false>(m, s, idx, q.m, q.s, q.idx, c);
            else
              acc_merge<true>(m, s, idx, q.m, q.s, q.idx, c);
          }
        }
        if (greedy) {
          merge_step<false, kXor1>(m, s, idx, c);
          merge_step<false, kXor2>(m, s, idx, c);
        } else {
          merge_step<true, kXor1>(m, s, idx, c);
          merge_step<true, kXor2>(m, s, idx, c);
        }
        if (row_ok && k_in_seg == 0) {
          if (idx == INT_MAX) idx = 0;  // an all -inf row: every index ties, the first wins
          // log sum_x exp((z_x - m)/T) = ln2 * (log2 s - r), r = m*c - fl(m*c)
          // exactly; log2 s in fp32 (within 1e-7 of |log2 s|: s carries fp32
          // rounding already).
          const double logz =
              greedy ? 0.0 : kLn2 * (double(__builtin_amdgcn_logf(s)) - double(fmaf(m, c, -scaled_max(m, c))));
          ds.row_m[r] = m;
          ds.row_logz[r] = logz;
          ds.row_idx[r] = idx;
          lse[r] = greedy ? double(NAN) : double(m) * inv_t + logz;
          amax[r] = idx;
        }
      }
      barrier();
    }
    return rows_late;
  };
  timed_out = take_rows(0, Rs_main) || timed_out;
  if (split && (any_bad || timed_out)) take_rows(Rs_main, Rs);  // taken (and zeroed) all the same
  if (any_bad || timed_out) {
    // Invalid inputs give -1 everywhere; a partial that never came (not
    // expected: a workgroup that was not dispatched in time) gives -2.
    const int code = any_bad ? -1 : -2;
    mark_unread(P, b, st, lo);
    signal_go(P, st, b, false);
    if (draws) {
      // The finisher writes the sentinels.
      if (tid == 0) publish(P, b, any_bad ? kModeInvalid : kModeFailed, 0, 0.0f, 0.0f, 0.0);
    } else {
      for (int i = tid; i <= N; i += kThreads) otok[i] = code;
      if (tid == 0 && P.out_n != nullptr) P.out_n[b] = code;
    }
    return;
  }
  trace(2, 5);
  if (greedy) {
    for (int r = lo + tid; r < hi; r += kThreads) {
      lse[r] = NAN;
      amax[r] = -1;
    }
  }

  bool accept = true;
  if (tid < ns) {
    const int i = lo + tid;
    if (greedy) {
      accept = (d == ds.row_idx[N + i]);
    } else if (zd == -INFINITY) {
      accept = true;  // p(d) == 0: the ratio is infinite
    } else {
      // log(q(d)/p(d)); the test is u < exp of it.
      const double lr = ((double(zt) - double(ds.row_m[N + i])) - (double(zd) - double(ds.row_m[i]))) * inv_t -
                        (ds.row_logz[N + i] - ds.row_logz[i]);
      // u < 1 <= exp(lr) when lr >= 0; the library exp only where the local one underflows.
      accept = lr >= 0.0 || double(ua) < (lr >= -708.0 ? exp_nonpos(lr) : exp(lr));
    }
  }
  // N <= 64: every decision lives in wave 0.
  if (wave == 0) {
    const unsigned long long rej = __ballot(tid < ns && !accept);
    if (lane == 0) ds.rej_mask = rej;
  }
  barrier();
  trace(2, 6);
  const unsigned long long rej = ds.rej_mask;
  const int j = rej ? lo + (__ffsll(rej) - 1) : hi;
  const bool go_on = j == hi && !last;  // a lazy call's sequence that goes on to the next stage
  const bool needs_row_n = split && j == N;  // the bonus (greedy: the argmax of row N) waits for row N
  // The draw's record first (the draw members wait for it), or the next
  // stage's go-on words.
  if (tid == 0 && !greedy && !go_on && !needs_row_n) {
    const float md = j < N ? ds.row_m[j] : 0.0f;
    const double log_rho = j < N ? ds.row_logz[N + j] - ds.row_logz[j] : 0.0;
    publish(P, b, j < N ? kModeResidual : kModeBonus, j, ds.row_m[N + j], md, log_rho);
  }
  // Rows of the stages after this one are never read when the sequence ends
  // here.
  if (!go_on && !last) mark_unread(P, b, st, hi);
  signal_go(P, st, b, go_on);
  for (int i = lo + tid; i <= N; i += kThreads) {
    if (i < j)
      otok[i] = ds.tok[i];
    else if (go_on)
      break;
    else if (i > j)
      otok[i] = -1;
    else if (greedy && !needs_row_n)
      otok[i] = ds.row_idx[N + j];
  }
  if (tid == 0 && greedy && !go_on && !needs_row_n && P.out_n != nullptr) P.out_n[b] = j;
  if (!split) return;
  // Target row N: its diagnostics, and the draw or the greedy token of a
  // sequence that accepted every draft.
  if (take_rows(Rs_main, Rs)) {
    if (tid == 0) {
      lse[2 * N] = NAN;
      amax[2 * N] = -1;
    }
    if (needs_row_n) {
      if (draws) {
        if (tid == 0) publish(P, b, kModeFailed, 0, 0.0f, 0.0f, 0.0);
      } else {
        for (int i = tid; i <= N; i += kThreads) otok[i] = -2;
        if (tid == 0 && P.out_n != nullptr) P.out_n[b] = -2;
      }
    }
    return;
  }
  if (needs_row_n && tid == 0) {
    if (greedy) {
      otok[N] = ds.row_idx[2 * N];
      if (P.out_n != nullptr) P.out_n[b] = N;
    } else {
      publish(P, b, kModeBonus, N, ds.row_m[2 * N], 0.0f, 0.0);
    }
  }
}

// ---------------------------------------------------------------------------
// The draw.

template <typename T>
struct DrawRows {
  const T* trow;
  const T* drow;
  double nmt, nmd;  // -max/T of the target and draft rows
  double inv_t;
};

template <typename T>
__device__ __forceinline__ DrawRows<T> draw_rows(const Params& P, int b, const SeqInfo& s) {
  const int N = P.n_draft;
  DrawRows<T> d;
  d.trow = static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + s.j) * P.vocab;
  d.drow = N > 0 ? static_cast<const T*>(P.draft) + (int64_t(b) * N + min(s.j, N - 1)) * P.vocab : d.trow;
  d.inv_t = 1.0 / double(s.temp);
  d.nmt = -double(s.m_target) * d.inv_t;
  d.nmd = -double(s.m_draft) * d.inv_t;
  return d;
}

// Argument z/T - max/T of a token's exp; every step forms it the same way.
__device__ __forceinline__ double exp_arg(float z, double nm, double inv_t) { return fma(double(z), inv_t, nm); }

// The residual weight max(0, et/Zt - ed/Zd) scaled by Zt*Zd: max(0, et*rt -
// ed*rd) with rt = Zd, rd = Zt (the draw only compares weights with each
// other and with u times their sum, so a common scale changes nothing, and
// it spares two divisions on the finisher's path). The rounding is spelled
// out so every place that forms a weight gets the same bits.
__device__ __forceinline__ double resid_weight(double et, double ed, double rt, double rd) {
  return fmax(0.0, fma(et, rt, -__dmul_rn(ed, rd)));
}

// ---------------------------------------------------------------------------
// Draw members.
//
// After a rejection the residual weight of token x is
//   w_x = max(0, et_x/Zt - ed_x/Zd) = max(0, et_x - rho*ed_x)/Zt,  rho = Zt/Zd,
// (et, ed: exps relative to the row maxima), so its sign only depends on
// whether log(et_x/ed_x) exceeds log(rho). The decision knows log(rho) from
// the fp32 row sums to a few 1e-6, and log(et_x/ed_x) is the difference of
// the two exps' fp64 arguments; a member treats tokens more than
// kSignBand away from it as certain and sums their exps into A and B per
// sub-chunk, so a sub-chunk's weight is A/Zt - B/Zd plus the exact terms of
// its few uncertain tokens, which the record lists. One pass over the rows
// gives the normalisers and every sub-chunk weight.

constexpr double kSignBand = 1e-4;

// Member c of sequence b: fp64 exps of its kPer logits per thread of the
// draw's row(s) (target row j and draft row j after a rejection, target row N
// for the bonus), summed and classified; writes the member's record.
template <typename T>
struct MemberRows {
  static constexpr int kG = Logit<T>::kPer / Logit<T>::kVec;  // 16-byte groups per row
  double tab_v;  // this thread's entry of kExp2Table
  uint4 xt[kG], xd[kG];
  // The exp table entry first (a cached read that arrives before the rows),
  // then member c's logits of the target row (and the draft row after a
  // rejection).
  __device__ __forceinline__ void load(const Params& P, const DrawRows<T>& d, int c, bool residual) {
    const int e = (c * kThreads + int(threadIdx.x)) * Logit<T>::kPer;
    tab_v = kExp2Table[threadIdx.x];
    load_packed(d.trow, e, P.vocab, (P.flags & kVecOk) != 0, xt);
    if (residual) load_packed(d.drow, e, P.vocab, (P.flags & kVecOk) != 0, xd);
  }
};

template <typename T, bool kSample>
__device__ __forceinline__ void member_record(const Params& P, DrawShared<kSample>& ws, int b, int c,
                                              const SeqInfo& s, MemberRows<T>& rows) {
  const bool residual = !kSample && s.mode == kModeResidual;
  const bool draw = residual || s.mode == kModeBonus;  // (a sampling call's greedy row: the maximum only)
  constexpr int kPer = Logit<T>::kPer;
  constexpr int kG = MemberRows<T>::kG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  DrawRows<T> d = draw_rows<T>(P, b, s);
  const int e = (c * kThreads + tid) * kPer;
  uint4 (&xt)[kG] = rows.xt;
  uint4 (&xd)[kG] = rows.xd;
  trace(0, 1);
  ws.exp2_tab[tid] = rows.tab_v;
  float mc = -INFINITY;  // sampling call: this member's largest logit and its first index
  int ic = INT_MAX;
  if (kSample) {
    float tm = -INFINITY;
    int ti = INT_MAX;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float v = Logit<T>::element(xt, k);
      ti = v > tm ? e + k : ti;  // strict: the first place (a thread's tokens ascend)
      tm = fmaxf(v, tm);
    }
    const float wm = wave_max(tm);
    const int wi = wave_min(tm == wm ? ti : INT_MAX);
    if (lane == 0) {
      ws.wave_m[tid >> 6] = wm;
      ws.wave_i[tid >> 6] = wi;
    }
  }
  barrier();
  if (kSample) {
    mc = ws.wave_m[0];
    ic = ws.wave_i[0];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) {
      ic = ws.wave_m[wv] > mc ? ws.wave_i[wv] : ic;  // waves hold ascending runs: an equal one comes later
      mc = fmaxf(ws.wave_m[wv], mc);
    }
    // (a chunk of -inf logits only: any finite reference gives exps of 0)
    d.nmt = mc == -INFINITY ? 0.0 : -double(mc) * d.inv_t;
  }
  const double* tab = ws.exp2_tab;
  double st = 0.0, sd = 0.0, sa = 0.0, sb = 0.0;
  uint32_t unc = 0;  // bit k: token k of this thread has an uncertain sign
  if (!draw) {
    // nothing to sum
  } else if (residual) {
    // The sign of w_x follows log(et/ed) = at - ad (the exps' fp64 arguments,
    // exact to about 1e-16 of their size) against log(rho).
    const double hi = s.log_rho + kSignBand, lo = s.log_rho - kSignBand;
    bool any_band = false;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const double at = exp_arg(Logit<T>::element(xt, k), d.nmt, d.inv_t);
      const double ad = exp_arg(Logit<T>::element(xd, k), d.nmd, d.inv_t);
      const double et = exp_nonpos_tab(at, tab);
      const double ed = exp_nonpos_tab(ad, tab);
      st += et;
      sd += ed;
      // +inf when the draft gives the token zero mass, NaN (neither class)
      // when both rows do: such a token adds nothing wherever it goes.
      const double lr = at - ad;
      const bool pos = lr > hi;
      const bool band = !pos && lr >= lo;
      const double pos_d = pos ? 1.0 : 0.0;  // adds et and ed exactly, or nothing
      sa = fma(pos_d, et, sa);
      sb = fma(pos_d, ed, sb);
      any_band = any_band || band;
    }
    // Uncertain tokens are rare (a wave in tens holds one): their bits are
    // taken in a second pass, with the same arithmetic, only where needed.
    if (__ballot(any_band)) {
      // The logits pass through an empty asm the compiler cannot see
      // through: otherwise it keeps the first pass's kPer fp64 differences
      // live until here instead of recomputing them.
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        asm volatile("" : "+v"(xt[u].x), "+v"(xt[u].y), "+v"(xt[u].z), "+v"(xt[u].w));
        asm volatile("" : "+v"(xd[u].x), "+v"(xd[u].y), "+v"(xd[u].z), "+v"(xd[u].w));
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const double lr = exp_arg(Logit<T>::element(xt, k), d.nmt, d.inv_t) -
                          exp_arg(Logit<T>::element(xd, k), d.nmd, d.inv_t);
        unc |= (!(lr > hi) && lr >= lo) ? (1u << k) : 0u;
      }
    }
  } else {
    // A copy the compiler cannot see through: otherwise it computes the
    // target row's kPer fp64 exp arguments once above both branches and
    // keeps them all live (spills in the fp32 build).
    uint4 yt[kG];
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      yt[u] = xt[u];
      asm volatile("" : "+v"(yt[u].x), "+v"(yt[u].y), "+v"(yt[u].z), "+v"(yt[u].w));
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) st += exp_nonpos_tab(exp_arg(Logit<T>::element(yt, k), d.nmt, d.inv_t), tab);
    sa = st;
  }
  trace(0, 2);
  // The first two uncertain tokens of this thread: their exps again (the same
  // bits, from the logits still in registers), staged in LDS; more overflow
  // the record.
  const int n_unc = __popc(unc);
  int unc_k0 = 0, unc_k1 = 0;
  if (n_unc > 0) {
    unc_k0 = __ffs(int(unc)) - 1;
    unc_k1 = n_unc > 1 ? __ffs(int(unc & (unc - 1))) - 1 : 0;
    for (int i = 0; i < min(n_unc, 2); ++i) {
      const int k = i == 0 ? unc_k0 : unc_k1;
      ws.mem.unc_et[i][tid] = exp_nonpos_tab(exp_arg(element_at<T>(xt, k), d.nmt, d.inv_t), tab);
      ws.mem.unc_ed[i][tid] = exp_nonpos_tab(exp_arg(element_at<T>(xd, k), d.nmd, d.inv_t), tab);
    }
  }
  MemberRec* rec = P.records + int64_t(b) * P.nm + c;
  // Sub-chunk sums: 32 consecutive threads per sub-chunk (lanes 0..31 and
  // 32..63 of each wave): row sums, then row 0's added into row 1 and row
  // 2's into row 3, so lanes 31 and 63 hold them.
  sa = row_sum(sa);
  sb = row_sum(sb);
  sa += dpp_f64<kBcast15, 0xa>(sa);
  sb += dpp_f64<kBcast15, 0xa>(sb);
  if ((lane & 31) == 31) {
    put_d_word(rec, MemberRec::kA + (tid >> 5), sa);
    put_d_word(rec, MemberRec::kB + (tid >> 5), sb);
  }
  // One exchange through LDS for the wave totals of st, sd, sa and sb and the wave
  // counts of uncertain tokens (in ascending token order: threads own
  // ascending runs; a thread past its staging capacity overflows the record).
  const int cnt = !residual ? 0 : (n_unc <= 2) ? n_unc : kUncMax + 1;
  const int incl = wave_incl_scan(cnt);
  st = row_sum(st);
  sd = row_sum(sd);
  st += dpp_f64<kBcast15, 0xa>(st);
  sd += dpp_f64<kBcast15, 0xa>(sd);
  st += dpp_f64<kBcast31, 0xc>(st);  // lane 63: the wave's totals
  sd += dpp_f64<kBcast31, 0xc>(sd);
  sa += dpp_f64<kBcast31, 0xc>(sa);
  sb += dpp_f64<kBcast31, 0xc>(sb);
  const int wave = tid >> 6;
  if (lane == 63) {
    ws.red[wave] = st;
    ws.red[kWaves + wave] = sd;
    ws.red[2 * kWaves + wave] = sa;
    ws.red[3 * kWaves + wave] = sb;
    ws.unc_base[wave] = incl;
  }
  barrier();
  int slot = incl - cnt, total = 0;
#pragma unroll
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wv < wave) slot += ws.unc_base[wv];
    total += ws.unc_base[wv];
  }
  if (total <= kUncMax) {
    for (int i = 0; i < cnt; ++i) {
      put_u64(&rec->w[MemberRec::kPos + slot + i], uint64_t(uint32_t(e + (i == 0 ? unc_k0 : unc_k1))));
      put_d_word(rec, MemberRec::kEt + slot + i, ws.mem.unc_et[i][tid]);
      put_d_word(rec, MemberRec::kEd + slot + i, ws.mem.unc_ed[i][tid]);
    }
  }
  if (tid == 0) {
    double zt = ws.red[0], zd = ws.red[kWaves];
#pragma unroll
    for (int wv = 1; wv < kWaves; ++wv) {
      zt += ws.red[wv];
      zd += ws.red[kWaves + wv];
    }
    put_d_word(rec, MemberRec::kZt, zt);
    if (kSample) {
      put_d_word(rec, MemberRec::kMax, double(mc));
      put_u64(&rec->w[MemberRec::kArg], uint64_t(uint32_t(ic)));
    } else {
      put_d_word(rec, MemberRec::kZd, zd);
      put_u64(&rec->w[MemberRec::kNUnc], uint64_t(min(total, kUncMax + 1)));
      if (residual) {
        double at = ws.red[2 * kWaves], bt = ws.red[3 * kWaves];
#pragma unroll
        for (int wv = 1; wv < kWaves; ++wv) {
          at += ws.red[2 * kWaves + wv];
          bt += ws.red[3 * kWaves + wv];
        }
        put_d_word(rec, MemberRec::kAt, at);
        put_d_word(rec, MemberRec::kBt, bt);
      }
    }
  }
}

// Exact weights of sub-chunk `sub` of member c (whole workgroup): each thread
// takes kPer/8 consecutive tokens; returns this thread's weights' sum and its
// weights through w. rd = 0 after a rejection gives et*rt (q, scaled)
// instead of the residual. The exps are the members' (the same function and table), bit
// for bit.
template <typename T>
__device__ __forceinline__ double sub_weights(const Params& P, const DrawRows<T>& d, const double* tab, int c, int sub,
                                              bool residual, double rt, double rd, double (&w)[Logit<T>::kPer / 8],
                                              int& e0) {
  constexpr int kQ = Logit<T>::kPer / 8;  // a sub-chunk holds 32*kPer tokens: kQ per thread
  e0 = c * kThreads * Logit<T>::kPer + sub * 32 * Logit<T>::kPer + int(threadIdx.x) * kQ;
  double sum = 0.0;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int x = e0 + q;
    const float zt = x < P.vocab ? Logit<T>::at(d.trow, x) : -INFINITY;
    const double et = exp_nonpos_tab(exp_arg(zt, d.nmt, d.inv_t), tab);
    if (residual) {
      const float zd = x < P.vocab ? Logit<T>::at(d.drow, x) : -INFINITY;
      const double ed = exp_nonpos_tab(exp_arg(zd, d.nmd, d.inv_t), tab);
      w[q] = rd > 0.0 ? resid_weight(et, ed, rt, rd) : et * rt;
    } else {
      w[q] = et * rt;  // (rt = 1 for a verification's bonus draw: exact)
    }
    sum += w[q];
  }
  return sum;
}

// Exact weights of the kSubs sub-chunks of member c (whole workgroup, a rare
// path): they replace the member's staged A words, which the finisher then
// takes as the sub-chunk weights themselves. The caller makes them visible
// with a barrier.
template <typename T>
__device__ __forceinline__ void exact_member_weights(const Params& P, DrawShared<false>& ws, const DrawRows<T>& d, int c,
                                                     double rt, double rd) {
#pragma unroll 1
  for (int sub = 0; sub < kSubs; ++sub) {
    double wq[Logit<T>::kPer / 8];
    int e0;
    const double v = block_sum(sub_weights<T>(P, d, ws.exp2_tab, c, sub, true, rt, rd, wq, e0), ws.red);
    if (threadIdx.x == 0) ws.stage[c * MemberRec::kWords + MemberRec::kA + sub] = double_to_bits(v);
  }
}

// Token pairs (x_k, x_k + 1), x_k = x0 + k*32*kPer (x0 even), k < kSubs, of
// one row as stored, kept in registers until one k is chosen: each load is
// issued at a clamped index with no branch, and tokens at and past `vocab`
// become -inf when the pair is taken. Rows 16-byte aligned: one aligned load
// per pair (the vocabulary is then even); else one load per token.
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
static_assert(kSubs == 8, "one vector lane per sub-chunk");

template <typename T>
struct PairRow {
  u32x8 a, b;  // aligned bfloat16: a holds both tokens, b is unused; else a: token x_k, b: token x_k + 1
  __device__ __forceinline__ void load(const T* __restrict__ row, int x0, int vocab, bool vec_ok) {
    if (vec_ok) {
#pragma unroll
      for (int k = 0; k < kSubs; ++k) {
        const int xc = min(x0 + k * 32 * Logit<T>::kPer, vocab - 2);
        if constexpr (sizeof(T) == 2) {
          a[k] = *reinterpret_cast<const uint32_t*>(row + xc);
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(row + xc);
          a[k] = v.x;
          b[k] = v.y;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kSubs; ++k) {
        const int x = x0 + k * 32 * Logit<T>::kPer;
        a[k] = Logit<T>::bits(row, min(x, vocab - 1));
        b[k] = Logit<T>::bits(row, min(x + 1, vocab - 1));
      }
    }
  }
  // Pair k (wave-uniform) as fp32 logits.
  __device__ __forceinline__ void take(int k, int x0, int vocab, bool vec_ok, float& z0, float& z1) const {
    const uint32_t wa = a[k];
    if (sizeof(T) == 2 && vec_ok) {
      z0 = Logit<T>::from_bits(wa & 0xffffu);
      z1 = Logit<T>::from_bits(wa >> 16);
    } else {
      z0 = Logit<T>::from_bits(wa);
      z1 = Logit<T>::from_bits(b[k]);
    }
    const int x = x0 + k * 32 * Logit<T>::kPer;
    if (x >= vocab) z0 = -INFINITY;
    if (x + 1 >= vocab) z1 = -INFINITY;
  }
};

// ---------------------------------------------------------------------------
// The finisher (the last member of a sequence to report). The member records
// are staged in LDS. Then every wave, on its own (lane l reading record l),
// forms the normalisers and each member's weight, picks the member where the
// inverse CDF crosses u*S, issues the loads of that member's tokens (two of
// each sub-chunk per thread) and, while they are in flight, forms the
// member's sub-chunk weights and picks the crossing sub-chunk. The workgroup
// then forms the exact weights of that sub-chunk's tokens and wave 0 finds
// the token. A member's weight comes from its certain-sign totals and its
// uncertain tokens, a sub-chunk's from its own sums: they agree up to
// rounding, and each search falls back to its last positive value when
// rounding leaves no crossing.

// Inverse CDF within one wave over n values per lane, in lane order then value
// order, against `target`: the first value with positive weight whose
// inclusive prefix exceeds it, else the last positive one; returns lane*n +
// index (-1 if none is positive) and rem = target minus the prefix before it.
// `total` gets the sum of all values. Uniform over the wave.
template <int n>
__device__ __forceinline__ int wave_inverse_cdf(const double (&w)[n], double u, bool scale_by_total, double& rem,
                                                double& total) {
    double own = 0.0;
#pragma unroll
  for (int k = 0; k < n; ++k) own += w[k];
  const double incl = wave_incl_scan(own);
  total = read_lane(incl, 63);
  const double target = scale_by_total ? u * total : u;
  double cum = dpp_f64<kWaveShr1>(incl);  // lane 0: 0
  double hit_pre = 0.0, last_pre = 0.0;
  int hit = -1, lastp = -1;
#pragma unroll
  for (int k = 0; k < n; ++k) {
    const double x = w[k];
    if (x > 0.0) {
      if (hit < 0 && cum + x > target) {
        hit = k;
        hit_pre = cum;
      }
      lastp = k;
      last_pre = cum;
    }
    cum += x;
  }
  const unsigned long long hm = __ballot(hit >= 0);
  if (hm) {
    const int src = __ffsll(hm) - 1;
    rem = target - read_lane(hit_pre, src);
    return src * n + read_lane(hit, src);
  }
  const unsigned long long pm = __ballot(lastp >= 0);
  if (pm) {
    const int src = 63 - __clzll(pm);
    rem = target - read_lane(last_pre, src);
    return src * n + read_lane(lastp, src);
  }
  rem = target;
  return -1;
}

template <typename T, bool kSample>
__device__ __forceinline__ void finish(const Params& P, DrawShared<kSample>& ws, int b, const SeqInfo& s_lds) {
  const SeqInfo s = uniform(s_lds);
  const bool residual = !kSample && s.mode == kModeResidual;
  constexpr int kPer = Logit<T>::kPer;
  static_assert(kPer / 8 == 2, "a sub-chunk holds two tokens per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int nm = P.nm;  // <= 64
  const bool mine = lane < nm;
  const double us = double(load_uniform(P.sample_u + b));  // in flight from the start
  // The sequence's member records (their first kW words each), in one
  // coalesced round trip: every load is issued (at a clamped index) before
  // any is stored.
  constexpr int kW = DrawShared<kSample>::kStageWords;
  constexpr int kStageIters = (kMaxMembers * kW + kThreads - 1) / kThreads;
  const uint64_t* src = P.records[0].w + (int64_t(b) * nm) * MemberRec::kWords;
  const int n_words = nm * kW;
  uint64_t words[kStageIters];
#pragma unroll
  for (int u = 0; u < kStageIters; ++u) {
    const int i = min(tid + u * kThreads, n_words - 1);
    words[u] = get_u64(src + (kW == MemberRec::kWords ? i : (i / kW) * MemberRec::kWords + i % kW));
  }
#pragma unroll
  for (int u = 0; u < kStageIters; ++u)
    if (tid + u * kThreads < n_words) ws.stage[tid + u * kThreads] = words[u];
  barrier();
  trace_at(1, b, 1);
  const uint64_t* r = ws.stage + (mine ? lane : 0) * kW;
  // Every member must have seen this call's decision, and the decision must
  // call for a draw; otherwise the sequence gets its sentinels here.
  const bool failed = __ballot(mine && r[MemberRec::kStatus] != tagged(P.tag, 1u)) != 0ull;
  const DrawRows<T> d = draw_rows<T>(P, b, s);
  float m_l = 0.0f, M = 0.0f;  // sampling call: member lane's largest logit, the row's
  int idx = 0;
  double scale = 0.0;  // sampling call: member lane's exps times this are relative to the row's maximum
  if (kSample) {
    // A sampling call: the row's largest logit M and its first index from
    // the members' own; each member's exps rescaled by exp((m_c - M)/T).
    // Its row diagnostics are written here (there is no decision).
    m_l = mine ? float(bits_to_double(r[MemberRec::kMax])) : -INFINITY;
    M = wave_max(m_l);
    idx = wave_min(mine && m_l == M ? int(uint32_t(r[MemberRec::kArg])) : INT_MAX);
    if (idx == INT_MAX) idx = 0;  // every logit -inf: every index ties
    const bool valid = s.mode != kModeInvalid && !failed;
    const bool sampled = valid && s.mode == kModeBonus;
    scale = sampled && mine ? exp_nonpos((double(m_l) - double(M)) * d.inv_t) : 0.0;
    if (!sampled) {
      if (tid == 0) {
        P.row_lse[b] = double(NAN);
        P.row_argmax[b] = valid ? idx : -1;
        if (valid) P.out_tokens[b] = idx;  // greedy: the first argmax
      }
      if (valid) return;
    }
  }
  if (failed || !(residual || s.mode == kModeBonus)) {
    const int code = s.mode == kModeInvalid ? -1 : -2;
    int* otok = P.out_tokens + int64_t(b) * (P.n_draft + 1);
    for (int i = tid; i <= P.n_draft; i += kThreads) otok[i] = code;
    if (tid == 0 && P.out_n != nullptr) P.out_n[b] = code;
    return;
  }
  // Normalisers (fixed-order DPP sums over the members). The draw's weights
  // are scaled by Zt*Zd: et*Zd - ed*Zt after a rejection; the bonus: et
  // (sampling call: et times the member's scale).
  double rt = 1.0, rd = 0.0;
  if (residual) {
    rd = wave_sum(mine ? bits_to_double(r[MemberRec::kZt]) : 0.0);
    rt = wave_sum(mine ? bits_to_double(r[MemberRec::kZd]) : 0.0);
  }
  const int nunc = residual && mine ? int(r[MemberRec::kNUnc]) : 0;
  // Members whose uncertain tokens overflowed their record: exact sub-chunk
  // weights (whole workgroup).
  const unsigned long long over = __ballot(nunc > kUncMax);
  if constexpr (!kSample) {
    for (unsigned long long o = over; o != 0ull; o &= o - 1ull) exact_member_weights<T>(P, ws, d, __ffsll(o) - 1, rt, rd);
    if (over != 0ull) barrier();
  }
  bool from_q = false;
  // Member lane's weight: the sum of its exact sub-chunk weights where the
  // staged A words hold them; else A*Zd - B*Zt plus its uncertain tokens' in
  // token order (the bonus: the member's sum of et, scaled when sampling).
  auto member_weight = [&]() -> double {
    if (!mine) return 0.0;
    if (from_q || ((over >> lane) & 1ull)) {
      double w = 0.0;
#pragma unroll
      for (int k = 0; k < kSubs; ++k) w += bits_to_double(r[MemberRec::kA + k]);
      return w;
    }
    if (!residual) return kSample ? scale * bits_to_double(r[MemberRec::kZt]) : bits_to_double(r[MemberRec::kZt]);
    double w = fma(bits_to_double(r[MemberRec::kAt]), rt, -__dmul_rn(bits_to_double(r[MemberRec::kBt]), rd));
    for (int i = 0; i < nunc; ++i)
      w += resid_weight(bits_to_double(r[MemberRec::kEt + i]), bits_to_double(r[MemberRec::kEd + i]), rt, rd);
    return w;
  };
  double wl[1] = {member_weight()};
  double rem, total;
  int c = wave_inverse_cdf<1>(wl, us, true, rem, total);
  if (residual && !(total > 0.0)) {
    // Every residual weight rounded to zero: draw from q_j itself, sub-chunk
    // by sub-chunk exactly.
    from_q = true;
    if constexpr (!kSample) {
      for (int cc = 0; cc < nm; ++cc) exact_member_weights<T>(P, ws, d, cc, rt, 0.0);
      barrier();
    }
    wl[0] = member_weight();
    c = wave_inverse_cdf<1>(wl, us, true, rem, total);
  }
  c = max(c, 0);
  // Member c's tokens, two of each sub-chunk per thread (the crossing
  // sub-chunk's are the ones used), requested before its sub-chunk weights
  // are formed.
  const bool two_rows = residual && !from_q;
  const bool vec_ok = (P.flags & kVecOk) != 0;
  const int x0 = c * kThreads * kPer + 2 * tid;
  PairRow<T> pt, pd;
  pt.load(d.trow, x0, P.vocab, vec_ok);
  if (two_rows) pd.load(d.drow, x0, P.vocab, vec_ok);
  // A sampling call's row log-normaliser, while the loads are in flight.
  const double lse = kSample ? double(M) * d.inv_t + log(wave_sum(wl[0])) : 0.0;
  // Member c's sub-chunk weights (lane k < kSubs holds sub-chunk k's) and
  // the crossing sub-chunk, against what remains of u*S past the members
  // before c.
  const uint64_t* rc = ws.stage + c * kW;
  const double scale_c = kSample ? read_lane(scale, c) : 1.0;
  double wk = 0.0;
  if (lane < kSubs) {
    wk = bits_to_double(rc[MemberRec::kA + lane]);
    if (!(from_q || ((over >> c) & 1ull))) {
      if (residual) {
        wk = fma(wk, rt, -__dmul_rn(bits_to_double(rc[MemberRec::kB + lane]), rd));
        const int nu = int(rc[MemberRec::kNUnc]);  // <= kUncMax: the member's list is whole
        for (int i = 0; i < nu; ++i) {
          const int sub = (int(rc[MemberRec::kPos + i]) - c * kThreads * kPer) / (32 * kPer);
          if (sub == lane)
            wk += resid_weight(bits_to_double(rc[MemberRec::kEt + i]), bits_to_double(rc[MemberRec::kEd + i]), rt, rd);
        }
      } else if (kSample) {
        wk *= scale_c;
      }
    }
  }
  double wv[1] = {wk};
  double rem2, total2;
  const int sub = max(wave_inverse_cdf<1>(wv, rem, false, rem2, total2), 0);
  trace_at(1, b, 2);
  // The crossing sub-chunk's exact token weights (two per thread, in token
  // order), then wave 0 finds the token: lane l takes weights 8l .. 8l+7. (A
  // sampling call's member exps are relative to its own maximum, scaled.)
  float zt[2], zd[2] = {0.0f, 0.0f};
  pt.take(sub, x0, P.vocab, vec_ok, zt[0], zt[1]);
  if (two_rows) pd.take(sub, x0, P.vocab, vec_ok, zd[0], zd[1]);
  double nmt = d.nmt;
  if (kSample) {
    const float m_c = __int_as_float(read_lane(__float_as_int(m_l), c));
    nmt = m_c == -INFINITY ? 0.0 : -double(m_c) * d.inv_t;
  }
  const double rts = kSample ? scale_c : rt;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const double et = exp_nonpos_tab(exp_arg(zt[q], nmt, d.inv_t), ws.exp2_tab);
    double wq;
    if (two_rows) {
      const double ed = exp_nonpos_tab(exp_arg(zd[q], d.nmd, d.inv_t), ws.exp2_tab);
      wq = rd > 0.0 ? resid_weight(et, ed, rts, rd) : et * rts;
    } else {
      wq = et * rts;  // (rt = 1 for a verification's bonus draw: exact)
    }
    ws.tw[tid * 2 + q] = wq;
  }
  trace_at(1, b, 3);
  barrier();
  if (tid < 64) {
    constexpr int kL = 32 * kPer / 64;  // token weights per lane
    double v[kL];
#pragma unroll
    for (int k = 0; k < kL; ++k) v[k] = ws.tw[lane * kL + k];
    double rem3, total3;
    const int k = wave_inverse_cdf<kL>(v, rem2, false, rem3, total3);
    if (lane == 0) {
      const int first = c * kThreads * kPer + sub * 32 * kPer;
      P.out_tokens[int64_t(b) * (P.n_draft + 1) + s.j] = k >= 0 ? first + k : 0;
      if (P.out_n != nullptr) P.out_n[b] = s.j;
      if (kSample) {
        P.row_lse[b] = lse;
        P.row_argmax[b] = idx;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels.

// A sequence's decision and its finisher lie on the path of the sequences
// that end last, while their CU is busy with other workgroups' streaming or
// fp64 sums: their waves take issue priority.
__device__ __forceinline__ void critical_path() { __builtin_amdgcn_s_setprio(3); }

// Row-statistics item `idx` of sequence b in stage st: stores the item's
// partial (a placeholder when the item is not read) and is done. In a lazy
// call's later stages it first takes its go-on word, and stores nothing for a
// sequence that ended earlier (its decision takes nothing either).
template <typename T>
__device__ __forceinline__ void stat_role(const Params& P, const Stage& st, int b, int idx) {
  trace_set(unsigned(b) * unsigned(P.items_per_seq + 1) + unsigned(idx));
  trace(2, 0);
  if (st.s > 0 && take_go(P, alive_item(P, b, global_row(P, st, idx / P.nch), idx % P.nch)) != 1) return;
  const Item it = item_at<T>(P, st, b, idx);
  Partial q{-INFINITY, 0.0f, INT_MAX - 1};
  if (it.live) {
    ItemRegs g;
    item_load<T>(P, it, g);
    // Loads in flight: folding them takes issue priority over the draw
    // members' fp64 work on the same CU, so items free their slots sooner.
    __builtin_amdgcn_s_setprio(2);
    q = item_reduce<T>(P, it, g);
  }
  trace(2, 1);
  partial_write(P, it, q);
}

// The decision of sequence b, in a workgroup of its own that follows the
// sequence's row-statistics items in the launch order.
template <typename T>
__device__ __forceinline__ void decision_role(const Params& P, Shared& sh, const Stage& st, int b) {
  trace_set(unsigned(b) * unsigned(P.items_per_seq + 1) + unsigned(P.items_per_seq));
  trace(2, 0);
  critical_path();
  decide<T>(P, sh, st, b, st.s > 0 ? take_go(P, alive_dec(P, b, st.s)) : 1);
  trace(2, 3);
}

// Waits (until the call's wait bound) for sequence b's decision. A draw
// member only waits for the decision workgroup, which precedes it in the
// launch order and waits only for row-statistics workgroups that precede it
// and never wait. Returns false if the wait gave up (s.mode is then
// kModeFailed).

__shared__ SeqInfo g_seq;
__shared__ int g_seq_ok;

__device__ __forceinline__ bool wait_decision(const Params& P, int b, float temp, SeqInfo& s) {
  if (threadIdx.x == 0) {
    const SeqRec* q = P.seq + b;
    const uint32_t tag = P.tag;
    uint64_t jm = get_u64(&q->jm), mt = get_u64(&q->mt), md = get_u64(&q->md), lr = get_u64(&q->logrho);
    auto ready = [&] { return has_tag(jm, tag) && has_tag(mt, tag) && has_tag(md, tag) && has_tag(lr, tag); };
    if (!ready()) {
      const uint64_t deadline = deadline_after(P.wait_ticks);
      while (!ready() && before(deadline)) {
        __builtin_amdgcn_s_sleep(8);
        if (!has_tag(jm, tag)) jm = get_u64(&q->jm);
        if (!has_tag(mt, tag)) mt = get_u64(&q->mt);
        if (!has_tag(md, tag)) md = get_u64(&q->md);
        if (!has_tag(lr, tag)) lr = get_u64(&q->logrho);
      }
    }
    const bool ok = P.wait_ticks != 0 && ready();
    g_seq_ok = ok;
    g_seq = ok ? SeqInfo{temp, int((jm >> 8) & 0xff), int(jm & 0xff), __uint_as_float(uint32_t(mt)),
                         __uint_as_float(uint32_t(md)), double(__uint_as_float(uint32_t(lr)))}
               : SeqInfo{temp, kModeFailed, 0, 0.0f, 0.0f, 0.0};
  }
  barrier();
  s = g_seq;
  return g_seq_ok != 0;
}

// Draw member c of sequence b. Every member of a sampled sequence reports
// (with whether it saw this call's decision) when done; the last one clears
// the decision's record and finishes the sequence: its token and n_accepted,
// or its sentinels.
template <typename T, bool kSample>
__device__ __forceinline__ void draw_role(const Params& P, DrawShared<kSample>& ws, int b, int c) {
  // A sampling call's row is known from the start: its logits are requested
  // before anything waits for the temperature.
  MemberRows<T> rows;
  if (kSample) rows.load(P, DrawRows<T>{static_cast<const T*>(P.target) + int64_t(b) * P.vocab, nullptr, 0.0, 0.0, 0.0}, c, false);
  const float temp = load_uniform(P.temperature + b);
  if (!kSample && !has_draw_members(temp)) return;
  trace_set(unsigned(b) * unsigned(P.nm) + unsigned(c));
  trace(0, 0);
  SeqInfo s;
  bool saw = true;
  if (kSample) {
    // No decision: the row's own draw (the first argmax when greedy).
    bool bad = !temperature_valid(temp);
    if (P.flags & kDebug) {
      const float us = load_uniform(P.sample_u + b);
      bad = bad || (temp > 0.0f && !(us >= 0.0f && us < 1.0f));
    }
    s = SeqInfo{temp, bad ? kModeInvalid : (temp == 0.0f ? kModeNone : kModeBonus), 0, 0.0f, 0.0f, 0.0};
    if (threadIdx.x == 0) g_seq = s;
  } else {
    saw = wait_decision(P, b, temp, s);
  }
  trace(0, 5);
  if (s.mode == kModeResidual || s.mode == kModeBonus || (kSample && s.mode == kModeNone)) {
    if (!kSample) rows.load(P, draw_rows<T>(P, b, s), c, s.mode == kModeResidual);
    member_record<T, kSample>(P, ws, b, c, s, rows);
  }
  if (threadIdx.x == 0) put_u64(&P.records[int64_t(b) * P.nm + c].w[MemberRec::kStatus], tagged(P.tag, saw ? 1u : 0u));
  trace(0, 3);
  const bool last = last_arrival(P.draw_done + b * kCounterStride, P.nm);
  trace(0, 4);
  if (last) {
    if (threadIdx.x == 0) {
      put_u64(&P.seq[b].jm, 0);
      put_u64(&P.seq[b].mt, 0);
      put_u64(&P.seq[b].md, 0);
      put_u64(&P.seq[b].logrho, 0);
    }
    critical_path();
    trace_at(1, b, 0);
    // The decision read again from LDS rather than kept in registers across
    // the member's work (where it made the fp32 build spill).
    asm volatile("" ::: "memory");
    const SeqInfo s_again = g_seq;
    finish<T, kSample>(P, ws, b, s_again);
    trace_at(1, b, 4);
  }
}

// What workgroup x of the launch does. A sequence's statistics group (for a
// stage) is its row-statistics items followed by its decision workgroup.
// Whole call: the statistics groups of sequences 0..lag-1, then for each
// sequence p the statistics group of sequence p + lag (while there is one)
// followed by the draw members of sequence p. Lazy call: every sequence's
// statistics group of stage 0, then of stage 1, ..., then every sequence's
// draw members (each waits for the decision of whichever stage ends its
// sequence, which precedes it).
struct Role {
  int kind;  // 0 row statistics, 1 decision, 2 draw member
  int s;     // stage
  int b;
  int idx;   // row-statistics item within the sequence's stage, or draw member
};

__device__ __forceinline__ Role role_of(const Params& P, int x) {
  Role w;
  if (P.lazy) {
    int s = 0;
    while (s < P.n_stages && x >= P.st_base[s + 1]) ++s;
    if (s == P.n_stages) {
      x -= P.st_base[s];
      w.kind = 2;
      w.s = s - 1;
      w.b = x / P.nm;
      w.idx = x - w.b * P.nm;
      return w;
    }
    const int A = stage_rows(P, stage_at(P, s)) * P.nch + 1;
    x -= P.st_base[s];
    w.s = s;
    w.b = x / A;
    w.idx = x - w.b * A;
    w.kind = w.idx < A - 1 ? 0 : 1;
    return w;
  }
  // With a late row N (long drafts), a sequence's statistics group holds only
  // the items of its draft rows and target rows 0..N-1 and its decision; the
  // K items of its target row N come just before its draw members.
  const int K = late_row_n(P) ? P.nch : 0;
  const int A = P.items_per_seq - K + 1, M = P.nm, L = P.lag, D = K + M;
  w.s = 0;
  if (x < L * A) {
    w.b = x / A;
    const int z = x - w.b * A;
    w.kind = z < A - 1 ? 0 : 1;
    w.idx = z;
    return w;
  }
  x -= L * A;
  const int n1 = P.batch - L;  // pairs (statistics group of p + L, row N and draw of p)
  int p, z;
  if (x < n1 * (A + D)) {
    p = x / (A + D);
    z = x - p * (A + D);
    if (z < A) {
      w.b = p + L;
      w.kind = z < A - 1 ? 0 : 1;
      w.idx = z;
      return w;
    }
    z -= A;
  } else {
    x -= n1 * (A + D);
    p = n1 + x / D;
    z = x - (p - n1) * D;
  }
  w.b = p;
  if (z < K) {
    w.kind = 0;
    w.idx = A - 1 + z;  // the items of target row N follow the sequence's other items
  } else {
    w.kind = 2;
    w.idx = z - K;
  }
  return w;
}

// Five waves per SIMD: the most the draw members' registers allow without spills.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5, 8))) void verify_kernel(Params P) {
  Shared& sh = g_shared;
  const Role w = role_of(P, int(blockIdx.x));
  if (w.kind == 0)
    stat_role<T>(P, stage_at(P, w.s), w.b, w.idx);
  else if (w.kind == 1)
    decision_role<T>(P, sh, stage_at(P, w.s), w.b);
  else
    draw_role<T, false>(P, sh.u.drw, w.b, w.idx);
}

// The draft-side draw: draw members only, member c of row b being workgroup
// b * nm + c; each row's draw is a bonus draw from the row alone. Eight
// waves per SIMD (its registers and LDS allow eight workgroups per CU).
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void sample_kernel(Params P) {
  const int x = int(blockIdx.x);
  const int b = x / P.nm;
  draw_role<T, true>(P, g_sample_shared, b, x - b * P.nm);
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
  p.partials = static_cast<PartialRec*>(w.partials);
  p.seq = static_cast<SeqRec*>(w.seq);
  p.records = static_cast<MemberRec*>(w.records);
  p.draw_done = w.draw_done;
  p.batch = a.batch;
  p.n_draft = a.n_draft;
  p.vocab = a.vocab;
  p.nch = w.n_stat_chunks;
  p.chunk = w.stat_chunk;
  p.nm = w.n_members;
  p.lazy = a.lazy ? 1 : 0;
  p.alive = w.alive;
  p.items_per_seq = (2 * a.n_draft + 1) * w.n_stat_chunks;
  int64_t blocks;
  if (a.sample) {
    p.n_stages = 1;
    p.st_bound[0] = 0;
    p.st_bound[1] = 0;
    p.lag = 0;
    blocks = int64_t(a.batch) * p.nm;
  } else if (p.lazy) {
    p.n_stages = lazy_stage_bounds(a.n_draft, lazy_growth(a.batch, a.vocab, a.dtype), p.st_bound);
    int64_t base = 0;
    for (int s = 0; s < p.n_stages; ++s) {
      p.st_base[s] = int(base);
      const int hi = p.st_bound[s + 1], lo = p.st_bound[s];
      base += int64_t(a.batch) * ((2 * (hi - lo) + (hi == a.n_draft ? 1 : 0)) * w.n_stat_chunks + 1);
    }
    p.st_base[p.n_stages] = int(base);
    p.lag = 0;
    blocks = base + int64_t(a.batch) * p.nm;
  } else {
    p.n_stages = 1;
    p.st_bound[0] = 0;
    p.st_bound[1] = a.n_draft;
    // The lag: about three chip-fulls of resident workgroups of (row
    // statistics, draw) pairs, so a sequence's decision is normally out before
    // its draw members start.
    p.lag = max(1, min(a.batch, ceil_div(3 * w.resident_blocks, p.items_per_seq + 1 + p.nm)));
    blocks = int64_t(a.batch) * (p.items_per_seq + 1 + p.nm);
  }
  p.flags = ((int64_t(a.vocab) * int64_t(sizeof(T))) % 16 == 0 ? kVecOk : 0u) | (a.debug ? kDebug : 0u);
  p.tag = a.tag;
  // (not min(): on the host it takes ints)
  p.wait_ticks = a.wait_ticks > uint64_t(UINT32_MAX) ? UINT32_MAX : uint32_t(a.wait_ticks);
  if (ev != nullptr) (void)hipEventRecord(ev[0], stream);
  if (a.sample)
    hipLaunchKernelGGL(sample_kernel<T>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(verify_kernel<T>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, p);
  if (ev != nullptr) (void)hipEventRecord(ev[1], stream);
  return hipGetLastError();
}

int resident_blocks(int dtype) {
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const hipError_t e = dtype == 0 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<float>, kThreads, 0)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<uint16_t>, kThreads, 0);
  if (e != hipSuccess) return -1;
  return max(1, per_cu) * max(1, cus);
}

}  // namespace

int max_resident_blocks(int dtype) { return resident_blocks(dtype); }

const char* stage_name(int stage) {
  return (stage >= 0 && stage < kNumStages) ? kStageNames[stage] : nullptr;
}

#if defined(SPECV_TRACE)
// Copies the stamps of the last launches (draw members, finishers, row-statistics items) into out and clears them.
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

size_t partial_bytes() { return sizeof(PartialRec); }
size_t seq_bytes() { return sizeof(SeqRec); }
size_t member_bytes() { return sizeof(MemberRec); }

hipError_t launch_verify(const VerifyArgs& a, const Workspace& w, hipStream_t stream, hipEvent_t* events,
                         int* n_stages) {
  if (n_stages != nullptr) *n_stages = kNumStages;
  if (a.dtype == 0) return launch_typed<float>(a, w, stream, events);
  return launch_typed<uint16_t>(a, w, stream, events);
}

}  // namespace specv
