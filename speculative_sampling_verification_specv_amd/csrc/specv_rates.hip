// gfx950 kernels for per-position acceptance telemetry.
//
// For a verified batch, alpha_i = sum_x min(p_i(x), q_i(x)) is the
// probability that draft i is accepted once position i is reached (lesson
// "추측 디코딩 — 초안 작성, 검증, 반복", section "속도 향상을 결정하는 것";
// guide "친구가 먼저 쓰고 선생님이 채점합니다", section "몇 글자를 미리 쓰게
// 할까요"), and tau = sum_{k=0..N} prod_{i<k} alpha_i is the expected number
// of tokens one verifier pass emits. p and q come from the row
// log-normalisers the verification left in the workspace (fp64), so the
// rates take one more pass over the 2N draft and target rows:
//
//   rate_parts_kernel    one workgroup per (sequence, position, 32 KB span of
//                        the draft row and the same span of the target row):
//                        sum of min(p, q) over the span, stored as one fp64
//                        partial. Bandwidth-bound.
//   rate_finish_kernel   one wave per sequence: the partials summed in item
//                        order, tau from the alphas. At T = 0 both
//                        distributions are point masses (the draft token, the
//                        verifier's first argmax): alpha_i = [d_i == argmax].

#include <float.h>
#include <math.h>

#include "specv_internal.h"

namespace specv {
namespace {

constexpr double kLog2eD = 1.4426950408889634;

struct RateParams {
  const void* draft;
  const void* target;
  const int* tokens;
  const float* temperature;
  const double* row_lse;
  const int* row_argmax;
  double* parts;
  float* out_alpha;
  float* out_tau;
  int batch, n_draft, vocab, nch, chunk, vec_ok;
};

__device__ __forceinline__ bool sampled_temperature(float t) { return t >= kMinTemperature && t <= FLT_MAX; }

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float at(const float* p, int64_t i) { return p[i]; }
  __device__ static float get(const uint4& v, int k) {
    return __uint_as_float(k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w);
  }
};
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int kVec = 8;
  __device__ static float at(const uint16_t* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
  __device__ static float get(const uint4& v, int k) {
    const uint32_t w = (k < 2) ? v.x : (k < 4) ? v.y : (k < 6) ? v.z : v.w;
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// min(p, q) of one token: p = 2^(zd*c - Ld*log2e), q likewise, each argument
// formed in fp64 (exact to about 1e-16 of its size). exp2 is increasing, so
// min(p, q) is 2^ of the smaller argument: one fp32 exp per token.
__device__ __forceinline__ float min_pq(float zd, float zt, double c, double ld, double lt) {
  return __builtin_amdgcn_exp2f(float(fmin(fma(double(zd), c, ld), fma(double(zt), c, lt))));
}

// A 16-byte load marked non-temporal: each logit is read once.
typedef unsigned RateV4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const RateV4 t = __builtin_nontemporal_load(reinterpret_cast<const RateV4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 8))) void rate_parts_kernel(RateParams P) {
  __shared__ double red[4];
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLoads = kRateBytes / 16 / 256;  // 16-byte loads per thread and row
  const int N = P.n_draft, R = 2 * N + 1;
  const int c = int(blockIdx.x % unsigned(P.nch));
  const int bi = int(blockIdx.x / unsigned(P.nch));
  const int i = bi % N, b = bi / N;
  const int tid = int(threadIdx.x);
  double* out = P.parts + (int64_t(b) * N + i) * P.nch + c;
  const T* drow = static_cast<const T*>(P.draft) + (int64_t(b) * N + i) * P.vocab;
  const T* trow = static_cast<const T*>(P.target) + (int64_t(b) * (N + 1) + i) * P.vocab;
  const int e0 = c * P.chunk, e1 = min(P.vocab, e0 + P.chunk);
  // Every 16-byte load of both rows is issued (at a clamped, valid index)
  // before any arithmetic, and before the row's temperature and
  // log-normalisers are waited for, so the item's 64 KB are in flight at once.
  const int nv = P.vec_ok ? (e1 - e0) / kVec : 0;
  uint4 xd[kLoads], xt[kLoads];
  if (nv > 0) {
    const uint4* dv = reinterpret_cast<const uint4*>(drow + e0);
    const uint4* tv = reinterpret_cast<const uint4*>(trow + e0);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int v = min(tid + u * 256, nv - 1);
      xd[u] = load_stream(dv + v);
      xt[u] = load_stream(tv + v);
    }
  }
  const float t = P.temperature[b];
  const double ld = P.row_lse[int64_t(b) * R + i], lt = P.row_lse[int64_t(b) * R + N + i];
  if (!sampled_temperature(t) || isnan(ld) || isnan(lt)) {
    if (tid == 0) *out = NAN;
    return;
  }
  const double cf = kLog2eD / double(t);
  const double nld = -ld * kLog2eD, nlt = -lt * kLog2eD;
  float acc = 0.0f;
  if (nv > 0) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      // Each group taken as it arrives: the empty asm keeps the compiler from
      // widening every logit of the item to fp64 ahead of time (which needs
      // far more registers than the loads themselves).
      asm volatile("" : "+v"(xd[u].x), "+v"(xd[u].y), "+v"(xd[u].z), "+v"(xd[u].w));
      asm volatile("" : "+v"(xt[u].x), "+v"(xt[u].y), "+v"(xt[u].z), "+v"(xt[u].w));
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < kVec; ++k) part += min_pq(Elem<T>::get(xd[u], k), Elem<T>::get(xt[u], k), cf, nld, nlt);
      acc += tid + u * 256 < nv ? part : 0.0f;
    }
  }
  for (int e = e0 + nv * kVec + tid; e < e1; e += 256) acc += min_pq(Elem<T>::at(drow, e), Elem<T>::at(trow, e), cf, nld, nlt);
  // Fixed-order block sum in fp64.
  double s = acc;
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) *out = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(64) void rate_finish_kernel(RateParams P) {
  __shared__ double alpha[64];
  const int N = P.n_draft, R = 2 * N + 1;
  const int b = blockIdx.x, lane = threadIdx.x;
  const float t = P.temperature[b];
  const bool greedy = t == 0.0f;
  bool bad = !(greedy || sampled_temperature(t));
  double a = NAN;
  if (lane < N) {
    const int d = P.tokens[int64_t(b) * N + lane];
    bad = bad || d < 0 || d >= P.vocab;
    if (greedy) {
      const int g = P.row_argmax[int64_t(b) * R + N + lane];
      a = g < 0 ? NAN : (d == g ? 1.0 : 0.0);
    } else {
      const double* parts = P.parts + (int64_t(b) * N + lane) * P.nch;
      a = 0.0;
      for (int c = 0; c < P.nch; ++c) a += parts[c];
    }
  }
  bad = __ballot(bad) != 0ull;
  if (lane < N) {
    alpha[lane] = bad ? NAN : a;
    P.out_alpha[int64_t(b) * N + lane] = float(alpha[lane]);
  }
  __syncthreads();
  if (lane == 0) {
    double tau = 0.0, reach = 1.0;
    for (int k = 0; k <= N; ++k) {
      tau += reach;
      if (k < N) reach *= alpha[k];
    }
    P.out_tau[b] = float(tau);
  }
}

}  // namespace

hipError_t launch_rates(const RatesArgs& a, const Workspace& w, hipStream_t stream) {
  RateParams p;
  p.draft = a.draft;
  p.target = a.target;
  p.tokens = a.tokens;
  p.temperature = a.temperature;
  p.row_lse = w.row_lse;
  p.row_argmax = w.row_argmax;
  p.parts = w.rate_parts;
  p.out_alpha = a.out_alpha;
  p.out_tau = a.out_tau;
  p.batch = a.batch;
  p.n_draft = a.n_draft;
  p.vocab = a.vocab;
  p.chunk = rate_chunk_elems(a.dtype);
  p.nch = ceil_div(a.vocab, p.chunk);
  const int esz = a.dtype == 0 ? 4 : 2;
  p.vec_ok = (int64_t(a.vocab) * esz) % 16 == 0;
  const int64_t blocks = int64_t(a.batch) * a.n_draft * p.nch;
  if (a.dtype == 0)
    hipLaunchKernelGGL(rate_parts_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(rate_parts_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(rate_finish_kernel, dim3(unsigned(a.batch)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace specv
