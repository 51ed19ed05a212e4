// Temperature / top-p (nucleus) draws from rows of fp32 logits, one workgroup
// per row. The serving recommendation is temperature 1.0 and top-p 0.95
// (lucasainews article "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로
// 공개", section "실행 방법"); the pages fix nothing else, and the rule used is:
//   * mass of token i: q_i = round(exp((l_i - max l) / T) * 2^40), an integer,
//     so every sum below is exact and independent of the reduction order;
//   * nucleus: tokens whose logit is at least the largest logit value tau such
//     that the tokens at or above tau hold at least top_p of the total mass
//     (all ties at tau kept); top_p >= 1 keeps every token;
//   * draw: with the caller's uniform u in [0, 1), r = floor(u * nucleus mass),
//     and the token is the first nucleus token in id order whose running mass
//     exceeds r;
//   * T <= 0: greedy (the lowest id among the largest logits).
// tau is found by a radix select on the order-preserving 32-bit key of the
// logit (four 8-bit digits, most significant first), with histograms of mass
// rather than counts; the draw scans 16 contiguous id spans (one per wave),
// then walks the span that holds r 64 ids at a time. Every pass reads the row
// from L2 (a 131072-token row is 512 KB), eight loads per thread in flight; the
// passes are then bound by the ~30 VALU operations per element of the integer mass
// on the row's one CU (about 26 us per pass at 131072 logits).
#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int SAMPLE_THREADS = 1024;
constexpr int SAMPLE_WAVES = SAMPLE_THREADS / 64;
constexpr double kMassScale = 1099511627776.0;  // 2^40

DORY_DEV uint32_t logit_key(float v) {
  const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);  // -0 and +0 are one logit
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

DORY_DEV unsigned long long token_mass(float v, float mx, float inv_t) {
  return (unsigned long long)rint((double)expf((v - mx) * inv_t) * kMassScale);
}

DORY_DEV unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Calls f(i, l[i]) for the indices i = tid + SAMPLE_THREADS k of a row, loading SAMPLE_UNROLL
// values per thread before using them, so that each thread keeps that many L2 loads in flight
// (one load at a time left every pass waiting on L2 latency).
constexpr int SAMPLE_UNROLL = 8;
template <typename F>
DORY_DEV void for_each_logit(const float* __restrict__ l, int V, int tid, F&& f) {
  for (int base = tid; base < V; base += SAMPLE_THREADS * SAMPLE_UNROLL) {
    float v[SAMPLE_UNROLL];
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const int i = base + u * SAMPLE_THREADS;
      v[u] = i < V ? l[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const int i = base + u * SAMPLE_THREADS;
      if (i < V) f(i, v[u]);
    }
  }
}

__global__ void __launch_bounds__(SAMPLE_THREADS) k_sample(const float* __restrict__ logits, int V, float inv_t,
                                                           float top_p, const float* __restrict__ uniforms,
                                                           int32_t* __restrict__ ids) {
  __shared__ unsigned long long hist[256];
  __shared__ unsigned long long wred[SAMPLE_WAVES];
  __shared__ float fred[SAMPLE_WAVES];
  __shared__ int ired[SAMPLE_WAVES];
  __shared__ unsigned long long s_above, s_rem;
  __shared__ uint32_t s_prefix;
  __shared__ int s_wave;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* l = logits + (size_t)blockIdx.x * V;

  // row maximum (and, for greedy, the lowest id holding it)
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  for_each_logit(l, V, tid, [&](int i, float v) __attribute__((always_inline)) {
    if (v > mx) { mx = v; mi = i; }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (ov > mx || (ov == mx && oi < mi)) { mx = ov; mi = oi; }
  }
  if (lane == 0) { fred[w] = mx; ired[w] = mi; }
  __syncthreads();
  mx = fred[0];
  mi = ired[0];
  for (int i = 1; i < SAMPLE_WAVES; ++i)
    if (fred[i] > mx || (fred[i] == mx && ired[i] < mi)) { mx = fred[i]; mi = ired[i]; }
  if (!(inv_t > 0.f)) {
    if (tid == 0) ids[blockIdx.x] = mi == 0x7fffffff ? 0 : mi;
    return;
  }

  // total mass
  unsigned long long part = 0;
  for_each_logit(l, V, tid, [&](int, float v) __attribute__((always_inline)) { part += token_mass(v, mx, inv_t); });
  part = wave_sum_u64(part);
  if (lane == 0) wred[w] = part;
  __syncthreads();
  unsigned long long total = 0;
  for (int i = 0; i < SAMPLE_WAVES; ++i) total += wred[i];
  __syncthreads();  // wred is reused below

  // threshold key: largest key K with mass(key >= K) >= target (radix select on mass)
  uint32_t kstar = 0;
  unsigned long long mass_s = total;
  if (top_p < 1.f) {
    // at least one unit, so top_p <= 0 keeps the top logit and its ties
    const unsigned long long target = max(1ull, (unsigned long long)ceil((double)fmaxf(top_p, 0.f) * (double)total));
    if (tid == 0) { s_prefix = 0; s_above = 0; }
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      for_each_logit(l, V, tid, [&](int, float v) __attribute__((always_inline)) {
        const uint32_t k = logit_key(v);
        if (pass == 0 || (k >> (shift + 8)) == (prefix >> (shift + 8)))
          atomicAdd(&hist[(k >> shift) & 255u], token_mass(v, mx, inv_t));
      });
      __syncthreads();
      if (tid == 0) {
        unsigned long long cum = s_above;
        int d = 255;
        for (; d > 0; --d) {
          if (cum + hist[d] >= target) break;
          cum += hist[d];
        }
        // digit d: keys above this digit hold cum; keys equal to it complete the target
        s_above = cum;
        s_prefix = prefix | ((uint32_t)d << shift);
        if (pass == 3) s_rem = cum + hist[d];
      }
      __syncthreads();  // the scan is done before the next pass clears hist; publishes s_prefix
    }
    kstar = s_prefix;
    mass_s = s_rem;
  }

  // draw: r = floor(u * mass_s); first nucleus token in id order whose running mass exceeds r
  const double u = (double)uniforms[blockIdx.x];
  unsigned long long r = (unsigned long long)floor(u * (double)mass_s);
  if (r >= mass_s) r = mass_s - 1;
  const int span = ((V + SAMPLE_WAVES - 1) / SAMPLE_WAVES + 63) & ~63;
  const int s0 = w * span, s1 = min(V, s0 + span);
  unsigned long long wm = 0;
  for (int b = s0 + lane; b < s1; b += 64 * SAMPLE_UNROLL) {
    float v[SAMPLE_UNROLL];
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) v[u] = b + 64 * u < s1 ? l[b + 64 * u] : 0.f;
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u)
      if (b + 64 * u < s1 && logit_key(v[u]) >= kstar) wm += token_mass(v[u], mx, inv_t);
  }
  wm = wave_sum_u64(wm);
  if (lane == 0) wred[w] = wm;
  __syncthreads();
  if (tid == 0) {
    unsigned long long base = 0;
    int sel = SAMPLE_WAVES - 1;
    for (int i = 0; i < SAMPLE_WAVES; ++i) {
      if (r < base + wred[i]) { sel = i; break; }
      base += wred[i];
    }
    s_wave = sel;
    s_rem = r - base;
  }
  __syncthreads();
  if (w != s_wave) return;
  unsigned long long rem = s_rem;
  int last = -1;  // last nucleus id seen: the answer if rounding leaves r unreached
  // groups of 64 ids in id order; SAMPLE_UNROLL groups' logits are loaded before they are walked
  for (int gb = s0; gb < s1; gb += 64 * SAMPLE_UNROLL) {
    float v[SAMPLE_UNROLL];
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const int i = gb + 64 * u + lane;
      v[u] = i < s1 ? l[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const int g = gb + 64 * u;
      if (g >= s1) break;
      const int i = g + lane;
      const unsigned long long q = i < s1 && logit_key(v[u]) >= kstar ? token_mass(v[u], mx, inv_t) : 0ull;
      // inclusive scan of q over the 64 lanes
      unsigned long long incl = q;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
      }
      const unsigned long long gtot = __shfl(incl, 63, 64);
      if (rem < gtot) {
        const unsigned long long hit = __ballot(incl > rem && q > 0);
        if (lane == 0) ids[blockIdx.x] = g + (int)__builtin_ctzll(hit);
        return;
      }
      rem -= gtot;
      const unsigned long long seen = __ballot(q > 0);
      if (seen) last = g + 63 - (int)__builtin_clzll(seen);
    }
  }
  if (lane == 0) ids[blockIdx.x] = last >= 0 ? last : 0;
}

hipError_t launch_sample(const float* logits, int rows, int V, float temperature, float top_p, const float* uniforms,
                         int32_t* ids, hipStream_t st) {
  if (rows < 0 || V < 1 || V > (1 << 23)) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const float inv_t = temperature > 0.f ? 1.f / temperature : 0.f;
  DORY_LAUNCH(k_sample, dim3(rows), dim3(SAMPLE_THREADS), 0, st, logits, V, inv_t, top_p, uniforms, ids);
  return hipGetLastError();
}

}  // namespace dory
