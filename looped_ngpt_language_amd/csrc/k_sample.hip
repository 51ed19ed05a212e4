// Temperature / top-p (nucleus) draws from rows of fp32 logits, each row spread over P
// workgroups. The serving recommendation is temperature 1.0 and top-p 0.95 (lucasainews article
// "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로 공개", section "실행 방법"); the pages fix
// nothing else, and the rule used is:
//   * mass of token i: q_i = round(exp((l_i - max l) / T) * 2^40), an integer, so every sum
//     below is exact and independent of the reduction order;
//   * nucleus: tokens whose logit is at least the largest logit value tau such that the tokens
//     at or above tau hold at least top_p of the total mass (all ties at tau kept); top_p >= 1
//     keeps every token;
//   * draw: with the caller's uniform u in [0, 1), r = floor(u * nucleus mass), and the token is
//     the first nucleus token in id order whose running mass exceeds r;
//   * T <= 0: greedy (the lowest id among the largest logits).
// tau is found by a radix select on the order-preserving 32-bit key of the logit (four 8-bit
// digits, most significant first) with histograms of mass rather than counts.
//
// A row is cut into P contiguous chunks of C ids, one workgroup each (grid P x rows), so that a
// single row (batch-1 decode) spreads over the chip instead of one CU. The steps hand their
// results to the next through a scratch buffer, one launch each (a kernel boundary is the only
// cross-workgroup ordering used):
//   1. chunk maxima (with the lowest id holding each), and the row's histograms zeroed;
//   2. row maximum; greedy rows end here. Chunk masses: the chunk's total, the row total and the
//      histogram of the first digit (global 64-bit atomics, one per bin and workgroup);
//   3-5. digits 2..4: every workgroup re-derives the digits chosen so far from the histograms
//      (a block scan over 256 bins each), then adds its chunk's histogram of the next digit for
//      the keys that share that prefix;
//   6. the threshold key and the nucleus mass from the four histograms; each chunk's nucleus mass;
//   7. one workgroup per row: the chunk that holds r (scan over the chunk masses), then the
//      256-id sub-block inside it that holds r (block scan), then the id (one lane's walk).
// top_p >= 1 skips 3-6 (the nucleus is the whole row, the chunk masses are step 2's totals).
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int SMP_T = 256;  // threads per workgroup
constexpr int SMP_W = SMP_T / 64;
constexpr int SMP_UNROLL = 8;
constexpr int SMP_HROW = 4 * 256 + 8;  // u64 per row: four 256-bin histograms, the row total, padding
constexpr int SMP_TOTAL = 4 * 256;     // index of the row total
constexpr int SMP_MAX_CHUNKS = 256;
constexpr double kMassScale = 1099511627776.0;  // 2^40
typedef unsigned long long u64;

DORY_DEV uint32_t logit_key(float v) {
  const uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);  // -0 and +0 are one logit
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

DORY_DEV u64 token_mass(float v, float mx, float inv_t) {
  return (u64)rint((double)expf((v - mx) * inv_t) * kMassScale);
}

DORY_DEV u64 wave_sum_u64(u64 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DORY_DEV u64 wave_incl_scan_u64(u64 v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Inclusive scan of one u64 per thread over the workgroup (thread order).
DORY_DEV u64 block_incl_scan_u64(u64 v, u64* s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_incl_scan_u64(v, lane);
  if (lane == 63) s_w[w] = v;
  __syncthreads();
  u64 off = 0;
  for (int i = 0; i < w; ++i) off += s_w[i];
  __syncthreads();
  return v + off;
}

DORY_DEV u64 block_sum_u64(u64 v, u64* s_w) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum_u64(v);
  if (lane == 0) s_w[w] = v;
  __syncthreads();
  u64 s = 0;
  for (int i = 0; i < SMP_W; ++i) s += s_w[i];
  __syncthreads();
  return s;
}

// f(i, l[i]) for the ids i of [c0, c1) this thread owns, SMP_UNROLL loads in flight per thread.
template <typename F>
DORY_DEV void for_chunk(const float* __restrict__ l, int c0, int c1, F&& f) {
  for (int base = c0 + (int)threadIdx.x; base < c1; base += SMP_T * SMP_UNROLL) {
    float v[SMP_UNROLL];
#pragma unroll
    for (int u = 0; u < SMP_UNROLL; ++u) {
      const int i = base + u * SMP_T;
      v[u] = i < c1 ? l[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < SMP_UNROLL; ++u) {
      const int i = base + u * SMP_T;
      if (i < c1) f(i, v[u]);
    }
  }
}

DORY_DEV bool better(float v, int i, float m, int mi) { return v > m || (v == m && i < mi); }

// Row maximum and the lowest id holding it, from the P chunk maxima (every thread gets them).
DORY_DEV void row_max(const int2* __restrict__ pm, int P, float* s_m, int* s_i, float& mx, int& mi) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  mx = -INFINITY;
  mi = 0x7fffffff;
  for (int p = threadIdx.x; p < P; p += SMP_T) {
    const int2 e = pm[p];
    const float v = __int_as_float(e.x);
    if (better(v, e.y, mx, mi)) { mx = v; mi = e.y; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (better(ov, oi, mx, mi)) { mx = ov; mi = oi; }
  }
  if (lane == 0) { s_m[w] = mx; s_i[w] = mi; }
  __syncthreads();
  mx = s_m[0];
  mi = s_i[0];
  for (int i = 1; i < SMP_W; ++i)
    if (better(s_m[i], s_i[i], mx, mi)) { mx = s_m[i]; mi = s_i[i]; }
  __syncthreads();
}

// One digit of the radix select: given the digit histogram h[256] (mass of the keys sharing the
// prefix chosen so far, by the next digit) and the mass `above` of keys above that prefix, the
// digit d is the largest with above + mass(digits >= d) >= target; `above` becomes the mass of
// the keys above the prefix extended by d. Thread t looks at digit 255 - t.
DORY_DEV uint32_t select_digit(const u64* __restrict__ h, u64 target, u64& above, u64* s_w, u64* s_v) {
  const int t = threadIdx.x;
  const u64 hv = h[255 - t];
  const u64 incl = block_incl_scan_u64(hv, s_w);   // mass of digits >= 255 - t
  const int below = __syncthreads_count(above + incl < target);
  const int ts = below < 255 ? below : 255;        // the first thread whose running mass reaches target
  if (t == ts) *s_v = incl - hv;
  __syncthreads();
  above += *s_v;
  __syncthreads();
  return 255u - (uint32_t)ts;
}

// Nucleus target of a row: at least one unit, so top_p <= 0 keeps the top logit and its ties.
DORY_DEV u64 nucleus_target(u64 total, float top_p) {
  const u64 t = (u64)ceil((double)fmaxf(top_p, 0.f) * (double)total);
  return t > 0 ? t : 1ull;
}

struct SmpArgs {
  const float* logits;
  const float* uniforms;
  int32_t* ids;
  int V, P, C;
  float inv_t, top_p;
  int2* pmax;   // [rows][P] chunk max (float bits), lowest id holding it
  u64* hist;    // [rows][SMP_HROW]
  u64* cmass;   // [rows][P]
  u64* sel;     // [rows][2] threshold key, nucleus mass
};

__global__ void __launch_bounds__(SMP_T) k_smp_max(SmpArgs a) {
  __shared__ float s_m[SMP_W];
  __shared__ int s_i[SMP_W];
  const int p = blockIdx.x, r = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* l = a.logits + (size_t)r * a.V;
  const int c0 = p * a.C, c1 = min(a.V, c0 + a.C);
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  for_chunk(l, c0, c1, [&](int i, float v) __attribute__((always_inline)) {
    if (v > mx) { mx = v; mi = i; }   // ids in increasing order per thread: the first one stays
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(mx, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (better(ov, oi, mx, mi)) { mx = ov; mi = oi; }
  }
  if (lane == 0) { s_m[w] = mx; s_i[w] = mi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < SMP_W; ++i)
      if (better(s_m[i], s_i[i], mx, mi)) { mx = s_m[i]; mi = s_i[i]; }
    a.pmax[(size_t)r * a.P + p] = make_int2(__float_as_int(mx), mi);
  }
  // the row's histograms and total start at zero for this call
  u64* h = a.hist + (size_t)r * SMP_HROW;
  for (int i = p * SMP_T + threadIdx.x; i < SMP_HROW; i += a.P * SMP_T) h[i] = 0ull;
}

// greedy != 0: write the row's argmax and stop. Else chunk masses (total, first-digit histogram
// when hist != 0).
__global__ void __launch_bounds__(SMP_T) k_smp_mass(SmpArgs a, int greedy, int with_hist) {
  __shared__ float s_m[SMP_W];
  __shared__ int s_i[SMP_W];
  __shared__ u64 s_w[SMP_W];
  __shared__ u64 hl[256];
  const int p = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  float mx;
  int mi;
  row_max(a.pmax + (size_t)r * a.P, a.P, s_m, s_i, mx, mi);
  if (greedy) {
    if (p == 0 && t == 0) a.ids[r] = mi == 0x7fffffff ? 0 : mi;
    return;
  }
  hl[t] = 0ull;
  __syncthreads();
  const float* l = a.logits + (size_t)r * a.V;
  const int c0 = p * a.C, c1 = min(a.V, c0 + a.C);
  u64 part = 0;
  for_chunk(l, c0, c1, [&](int, float v) __attribute__((always_inline)) {
    const u64 q = token_mass(v, mx, a.inv_t);
    part += q;
    if (with_hist && q) atomicAdd(&hl[logit_key(v) >> 24], q);
  });
  const u64 tot = block_sum_u64(part, s_w);   // its barriers also order the LDS histogram
  u64* h = a.hist + (size_t)r * SMP_HROW;
  if (t == 0) {
    a.cmass[(size_t)r * a.P + p] = tot;
    if (tot) atomicAdd(&h[SMP_TOTAL], tot);
  }
  if (with_hist && hl[t]) atomicAdd(&h[t], hl[t]);
}

// Digit `pass` (1..3) of the radix select.
__global__ void __launch_bounds__(SMP_T) k_smp_digit(SmpArgs a, int pass) {
  __shared__ float s_m[SMP_W];
  __shared__ int s_i[SMP_W];
  __shared__ u64 s_w[SMP_W];
  __shared__ u64 s_v;
  __shared__ u64 hl[256];
  const int p = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  float mx;
  int mi;
  row_max(a.pmax + (size_t)r * a.P, a.P, s_m, s_i, mx, mi);
  const u64* h = a.hist + (size_t)r * SMP_HROW;
  const u64 target = nucleus_target(h[SMP_TOTAL], a.top_p);
  u64 above = 0;
  uint32_t prefix = 0;
  for (int j = 0; j < pass; ++j) prefix |= select_digit(h + 256 * j, target, above, s_w, &s_v) << (24 - 8 * j);
  hl[t] = 0ull;
  __syncthreads();
  const int shift = 24 - 8 * pass;
  const float* l = a.logits + (size_t)r * a.V;
  const int c0 = p * a.C, c1 = min(a.V, c0 + a.C);
  for_chunk(l, c0, c1, [&](int, float v) __attribute__((always_inline)) {
    const uint32_t k = logit_key(v);
    if ((k >> (shift + 8)) == (prefix >> (shift + 8))) {
      const u64 q = token_mass(v, mx, a.inv_t);
      if (q) atomicAdd(&hl[(k >> shift) & 255u], q);
    }
  });
  __syncthreads();
  if (hl[t]) atomicAdd(const_cast<u64*>(h) + 256 * pass + t, hl[t]);
}

// Threshold key and nucleus mass; each chunk's nucleus mass.
__global__ void __launch_bounds__(SMP_T) k_smp_nucleus(SmpArgs a) {
  __shared__ float s_m[SMP_W];
  __shared__ int s_i[SMP_W];
  __shared__ u64 s_w[SMP_W];
  __shared__ u64 s_v;
  const int p = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  float mx;
  int mi;
  row_max(a.pmax + (size_t)r * a.P, a.P, s_m, s_i, mx, mi);
  const u64* h = a.hist + (size_t)r * SMP_HROW;
  const u64 target = nucleus_target(h[SMP_TOTAL], a.top_p);
  u64 above = 0;
  uint32_t kstar = 0, d = 0;
  for (int j = 0; j < 4; ++j) {
    d = select_digit(h + 256 * j, target, above, s_w, &s_v);
    kstar |= d << (24 - 8 * j);
  }
  const u64 mass_s = above + h[256 * 3 + d];
  const float* l = a.logits + (size_t)r * a.V;
  const int c0 = p * a.C, c1 = min(a.V, c0 + a.C);
  u64 part = 0;
  for_chunk(l, c0, c1, [&](int, float v) __attribute__((always_inline)) {
    if (logit_key(v) >= kstar) part += token_mass(v, mx, a.inv_t);
  });
  const u64 tot = block_sum_u64(part, s_w);
  if (t == 0) {
    a.cmass[(size_t)r * a.P + p] = tot;
    if (p == 0) { a.sel[2 * r] = kstar; a.sel[2 * r + 1] = mass_s; }
  }
}

// The draw: one workgroup per row.
__global__ void __launch_bounds__(SMP_T) k_smp_draw(SmpArgs a, int with_sel) {
  __shared__ float s_m[SMP_W];
  __shared__ int s_i[SMP_W];
  __shared__ u64 s_w[SMP_W];
  __shared__ u64 s_rem;
  __shared__ int s_sel;
  const int r = blockIdx.x, t = threadIdx.x;
  float mx;
  int mi;
  row_max(a.pmax + (size_t)r * a.P, a.P, s_m, s_i, mx, mi);
  const uint32_t kstar = with_sel ? (uint32_t)a.sel[2 * r] : 0u;
  const u64 mass_s = with_sel ? a.sel[2 * r + 1] : a.hist[(size_t)r * SMP_HROW + SMP_TOTAL];
  u64 rr = (u64)floor((double)a.uniforms[r] * (double)mass_s);
  if (rr >= mass_s) rr = mass_s - 1;
  // the chunk holding rr (P <= SMP_T: one chunk per thread)
  const u64 cm = t < a.P ? a.cmass[(size_t)r * a.P + t] : 0ull;
  const u64 ci = block_incl_scan_u64(cm, s_w);
  const int j = min(__syncthreads_count(ci <= rr), a.P - 1);
  if (t == j) s_rem = rr - (ci - cm);
  __syncthreads();
  u64 rem = s_rem;
  // the sub-block of the chunk holding rem: thread s owns ids [c0 + s * sub, +sub)
  const float* l = a.logits + (size_t)r * a.V;
  const int c0 = j * a.C, c1 = min(a.V, c0 + a.C);
  const int sub = (a.C + SMP_T - 1) / SMP_T;
  const int s0 = min(c1, c0 + t * sub), s1 = min(c1, s0 + sub);
  u64 my = 0;
  for (int i = s0; i < s1; ++i) {
    const float v = l[i];
    if (logit_key(v) >= kstar) my += token_mass(v, mx, a.inv_t);
  }
  const u64 si = block_incl_scan_u64(my, s_w);
  const int s = __syncthreads_count(si <= rem);
  if (t == 0) s_sel = -1;
  __syncthreads();
  if (t == s) {
    u64 run = si - my;   // mass before this thread's sub-block
    for (int i = s0; i < s1; ++i) {
      const float v = l[i];
      if (logit_key(v) < kstar) continue;
      run += token_mass(v, mx, a.inv_t);
      if (run > rem) { s_sel = i; break; }
    }
  }
  __syncthreads();
  if (t == 0) a.ids[r] = s_sel >= 0 ? s_sel : (mi == 0x7fffffff ? 0 : mi);  // the fallback is unreachable
}

// ------------------------------------------------------------------ launch and scratch

// Chunks per row: enough workgroups to spread a few rows over the chip, at most SMP_MAX_CHUNKS,
// at least 512 ids per chunk.
static int sample_chunks(int rows, int V) {
  const int by_rows = (2048 + rows - 1) / rows;
  const int by_len = (V + 511) / 512;
  return std::max(1, std::min(std::min(by_rows, by_len), SMP_MAX_CHUNKS));
}

static size_t al256(size_t v) { return (v + 255) / 256 * 256; }

size_t sample_scratch_bytes(int rows, int V) {
  if (rows <= 0) return 0;
  const size_t P = (size_t)sample_chunks(rows, V), R = (size_t)rows;
  return al256(R * P * 8) + al256(R * SMP_HROW * 8) + al256(R * P * 8) + al256(R * 16);
}

hipError_t launch_sample(const float* logits, int rows, int V, float temperature, float top_p, const float* uniforms,
                         int32_t* ids, void* scratch, size_t scratch_bytes, hipStream_t st) {
  if (rows < 0 || V < 1 || V > (1 << 23) || !(temperature == temperature) || !(top_p == top_p))
    return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  if (!scratch || scratch_bytes < sample_scratch_bytes(rows, V)) return hipErrorInvalidValue;
  const int P = sample_chunks(rows, V);
  const int C = ((V + P - 1) / P + 63) & ~63;
  const bool greedy = !(temperature > 0.f);
  // 1/T above the largest float (a subnormal T) is clamped: every logit below the maximum then
  // has mass 0, as in the exact rule
  const float inv_t = greedy ? 0.f : (float)std::min(1.0 / (double)temperature, (double)3.4028234663852886e38);
  char* s = static_cast<char*>(scratch);
  SmpArgs a{logits, uniforms, ids, V, P, C, inv_t, top_p, nullptr, nullptr, nullptr, nullptr};
  a.pmax = reinterpret_cast<int2*>(s);
  s += al256((size_t)rows * P * 8);
  a.hist = reinterpret_cast<u64*>(s);
  s += al256((size_t)rows * SMP_HROW * 8);
  a.cmass = reinterpret_cast<u64*>(s);
  s += al256((size_t)rows * P * 8);
  a.sel = reinterpret_cast<u64*>(s);
  const dim3 grid(P, rows);
  const bool full = top_p >= 1.f;
  DORY_LAUNCH(k_smp_max, grid, dim3(SMP_T), 0, st, a);
  DORY_LAUNCH(k_smp_mass, grid, dim3(SMP_T), 0, st, a, greedy ? 1 : 0, full ? 0 : 1);
  if (greedy) return hipGetLastError();
  if (!full) {
    for (int pass = 1; pass < 4; ++pass) DORY_LAUNCH(k_smp_digit, grid, dim3(SMP_T), 0, st, a, pass);
    DORY_LAUNCH(k_smp_nucleus, grid, dim3(SMP_T), 0, st, a);
  }
  DORY_LAUNCH(k_smp_draw, dim3(rows), dim3(SMP_T), 0, st, a, full ? 0 : 1);
  return hipGetLastError();
}

// Scratch of dory_sample: one buffer per device, allocated on first use and grown when a call
// needs more; kept until the process ends.
namespace {
std::mutex g_lib_mu;
constexpr int kMaxDevices = 64;
void* g_lib_ptr[kMaxDevices] = {};
size_t g_lib_bytes[kMaxDevices] = {};
}  // namespace

hipError_t sample_library_scratch(int rows, int V, void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const size_t need = sample_scratch_bytes(rows, V);
  std::lock_guard<std::mutex> lk(g_lib_mu);
  if (g_lib_bytes[dev] < need) {
    if (g_lib_ptr[dev]) {
      e = hipFree(g_lib_ptr[dev]);   // waits for work already queued on the device
      g_lib_ptr[dev] = nullptr;
      g_lib_bytes[dev] = 0;
      if (e != hipSuccess) return e;
    }
    e = hipMalloc(&g_lib_ptr[dev], need);
    if (e != hipSuccess) { g_lib_ptr[dev] = nullptr; return e; }
    g_lib_bytes[dev] = need;
  }
  *ptr = g_lib_ptr[dev];
  *bytes = g_lib_bytes[dev];
  return hipSuccess;
}

// Scratch of dory_sample_static: a fixed device array, one copy per GPU. In host code its name
// stands for no device address; the address of the current device's copy comes from
// hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kSampleStaticScratchBytes];
namespace {
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
}  // namespace

hipError_t sample_static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_static_ptr[dev] = p;
  }
  *ptr = g_static_ptr[dev];
  return hipSuccess;
}

}  // namespace dory
