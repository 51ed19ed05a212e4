// Row-wise kernels of the looped nGPT forward pass: embedding gather, the
// normalised residual step, the loop injection and state normalisation, the
// greedy argmax, page-table updates and the rotary table.
//
// Normalised residual step of every sublayer (nGPT backbone; onedev.kr summary
// "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를 조절한다", section "어떻게 동작하나"):
//   h <- N(h + alpha * (N(y) - h)),  N(v) = v / ||v||_2.
// Loop update (same section): u_t = N(s_{t-1} + x), s_t = N(F(u_t)).
#include "common.h"
#include "kernels.h"

namespace dory {

constexpr int ROW_THREADS = 256;
constexpr int ROW_EPT = 16;  // elements per thread: d <= 4096

// h[m] = E[tok[m]] (fp32), hb[m] = E[tok[m]] (storage type).
template <typename T>
__global__ void __launch_bounds__(ROW_THREADS) k_embed(const int32_t* __restrict__ tokens,
                                                       const T* __restrict__ E, int vocab, int d,
                                                       float* __restrict__ h, T* __restrict__ hb,
                                                       int32_t* __restrict__ err) {
  const int m = blockIdx.x;
  int tok = tokens[m];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    tok = tok < 0 ? 0 : vocab - 1;
  }
  const T* e = E + (size_t)tok * d;
  for (int i = threadIdx.x; i < d; i += ROW_THREADS) {
    const float v = St<T>::ld(e, i);
    h[(size_t)m * d + i] = v;
    hb[(size_t)m * d + i] = e[i];
  }
}

// h <- N(h + alpha (N(y) - h)); hb <- storage copy of h.
template <typename T>
__global__ void __launch_bounds__(ROW_THREADS) k_residual(float* __restrict__ h, const float* __restrict__ y,
                                                          const float* __restrict__ alpha,
                                                          T* __restrict__ hb, int d) {
  __shared__ float red[ROW_THREADS / 64];
  const size_t base = (size_t)blockIdx.x * d;
  float yv[ROW_EPT], hv[ROW_EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    yv[e] = i < d ? y[base + i] : 0.f;
    hv[e] = i < d ? h[base + i] : 0.f;
    ss += yv[e] * yv[e];
  }
  const float ry = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
  float st = 0.f;
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    const float a = i < d ? alpha[i] : 0.f;
    hv[e] = hv[e] + a * (yv[e] * ry - hv[e]);
    st += hv[e] * hv[e];
  }
  const float rh = rsqrtf(fmaxf(block_sum(st, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    if (i < d) {
      const float v = hv[e] * rh;
      h[base + i] = v;
      St<T>::st(hb, base + i, v);
    }
  }
}

// The same step with y the sum of S split-K partial slices y[s][M][d] (slice = M * d floats), summed
// in slice order from zero exactly as the split-K reduce kernel sums them, so the result equals
// reduce-then-residual bit for bit while skipping that kernel and its y round trip. U slices are
// loaded per trip (every load unconditional: indices past the last slice or the row re-read it).
template <typename T, int U>
__global__ void __launch_bounds__(ROW_THREADS) k_residual_parts(float* __restrict__ h, const float* __restrict__ y,
                                                                int S, size_t slice, const float* __restrict__ alpha,
                                                                T* __restrict__ hb, int d) {
  __shared__ float red[ROW_THREADS / 64];
  const size_t base = (size_t)blockIdx.x * d;
  float yv[ROW_EPT], hv[ROW_EPT];
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    yv[e] = 0.f;
    hv[e] = h[base + min((int)threadIdx.x + e * ROW_THREADS, d - 1)];
  }
  for (int s0 = 0; s0 < S; s0 += U) {
    float t[U][ROW_EPT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < ROW_EPT; ++e)
        t[u][e] = y[(size_t)min(s0 + u, S - 1) * slice + base + min((int)threadIdx.x + e * ROW_THREADS, d - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < ROW_EPT; ++e)
        if (s0 + u < S) yv[e] += t[u][e];
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    if ((int)threadIdx.x + e * ROW_THREADS >= d) yv[e] = hv[e] = 0.f;
    ss += yv[e] * yv[e];
  }
  const float ry = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
  float st = 0.f;
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    const float a = i < d ? alpha[i] : 0.f;
    hv[e] = hv[e] + a * (yv[e] * ry - hv[e]);
    st += hv[e] * hv[e];
  }
  const float rh = rsqrtf(fmaxf(block_sum(st, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    if (i < d) {
      const float v = hv[e] * rh;
      h[base + i] = v;
      St<T>::st(hb, base + i, v);
    }
  }
}

// out = N(a + b) written to h (fp32) and hb (storage); a and b may alias.
// With b == nullptr: out = N(a), also written to s when s != nullptr.
template <typename T>
__global__ void __launch_bounds__(ROW_THREADS) k_norm_sum(const float* a, const float* b, float* h, float* s,
                                                          T* __restrict__ hb, int d) {
  __shared__ float red[ROW_THREADS / 64];
  const size_t base = (size_t)blockIdx.x * d;
  float v[ROW_EPT];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    v[e] = i < d ? a[base + i] + (b ? b[base + i] : 0.f) : 0.f;
    ss += v[e] * v[e];
  }
  const float r = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    if (i < d) {
      const float o = v[e] * r;
      h[base + i] = o;
      if (s) s[base + i] = o;
      St<T>::st(hb, base + i, o);
    }
  }
}

// Loop boundary of the recurrent core in one pass over each row (onedev.kr summary
// "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를 조절한다", section "어떻게 동작하나":
// s_0 = x, u_t = N(s_{t-1} + x), s_t = N(F(u_t))). v is the row of h, first advanced by the
// pending sublayer step N(v + alpha (N(y) - v)) when y != nullptr (that result is written back
// to h). Then, by mode:
//   LOOP_START (end of the input stack, h = x): u_1 = N(v + v) -> hout, hb;
//   LOOP_NEXT  (end of loop t < k): s_t = N(v) -> s; u_{t+1} = N(s_t + x) -> hout, hb;
//   LOOP_LAST  (end of loop k): s_k = N(v) -> s, hout, hb.
// Each step is computed exactly as the separate residual and norm kernels compute it (same
// reductions, same order), so results are bit-identical to launching them one after another.
// hout may alias h (the row is read whole before anything is written).
enum { LOOP_START = 0, LOOP_NEXT = 1, LOOP_LAST = 2 };
template <typename T>
__global__ void __launch_bounds__(ROW_THREADS) k_loop_step(float* h, const float* __restrict__ y,
                                                           const float* __restrict__ alpha,
                                                           const float* __restrict__ x, float* __restrict__ s,
                                                           float* hout, T* __restrict__ hb, int d, int mode) {
  __shared__ float red[ROW_THREADS / 64];
  const size_t base = (size_t)blockIdx.x * d;
  float hv[ROW_EPT];
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    hv[e] = i < d ? h[base + i] : 0.f;
  }
  if (y) {  // the pending sublayer step, as k_residual
    float yv[ROW_EPT];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) {
      const int i = threadIdx.x + e * ROW_THREADS;
      yv[e] = i < d ? y[base + i] : 0.f;
      ss += yv[e] * yv[e];
    }
    const float ry = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
    float st = 0.f;
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) {
      const int i = threadIdx.x + e * ROW_THREADS;
      const float a = i < d ? alpha[i] : 0.f;
      hv[e] = hv[e] + a * (yv[e] * ry - hv[e]);
      st += hv[e] * hv[e];
    }
    const float rh = rsqrtf(fmaxf(block_sum(st, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) hv[e] *= rh;
    if (mode == LOOP_START) {
#pragma unroll
      for (int e = 0; e < ROW_EPT; ++e) {
        const int i = threadIdx.x + e * ROW_THREADS;
        if (i < d) h[base + i] = hv[e];
      }
    }
  }
  if (mode != LOOP_START) {  // s_t = N(v), as k_norm_sum with one operand
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) ss += hv[e] * hv[e];
    const float r = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) {
      const int i = threadIdx.x + e * ROW_THREADS;
      hv[e] *= r;
      if (i < d) s[base + i] = hv[e];
    }
  }
  if (mode != LOOP_LAST) {  // u = N(a + b), as k_norm_sum with two operands
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) {
      const int i = threadIdx.x + e * ROW_THREADS;
      const float b = mode == LOOP_START ? hv[e] : (i < d ? x[base + i] : 0.f);
      hv[e] = i < d ? hv[e] + b : 0.f;
      ss += hv[e] * hv[e];
    }
    const float r = rsqrtf(fmaxf(block_sum(ss, red, ROW_THREADS / 64), DORY_TINY_SS));
#pragma unroll
    for (int e = 0; e < ROW_EPT; ++e) hv[e] *= r;
  }
#pragma unroll
  for (int e = 0; e < ROW_EPT; ++e) {
    const int i = threadIdx.x + e * ROW_THREADS;
    if (i < d) {
      hout[base + i] = hv[e];
      St<T>::st(hb, base + i, hv[e]);
    }
  }
}

// ids[r] = argmax_j logits[r, j], lowest j on ties. Two passes: grid (rows,
// ARGMAX_PARTS) workgroups each reduce a contiguous slice to (max, index), then
// one workgroup per row reduces the slices. Ties keep the lower index.
constexpr int ARGMAX_THREADS = 256;
constexpr int ARGMAX_PARTS = kArgmaxParts;

DORY_DEV void argmax_combine(float& best, int& bi, float ov, int oi) {
  if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
}

DORY_DEV void block_argmax(float& best, int& bi) {
  __shared__ float sv[ARGMAX_THREADS / 64];
  __shared__ int si[ARGMAX_THREADS / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) argmax_combine(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) { sv[w] = best; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int i = 1; i < ARGMAX_THREADS / 64; ++i) argmax_combine(best, bi, sv[i], si[i]);
}

__global__ void __launch_bounds__(ARGMAX_THREADS) k_argmax_part(const float* __restrict__ logits, int V,
                                                                float* __restrict__ pv, int* __restrict__ pi) {
  const int row = blockIdx.x, part = blockIdx.y;
  const int chunk = (V + ARGMAX_PARTS - 1) / ARGMAX_PARTS;
  const int j0 = part * chunk, j1 = min(V, j0 + chunk);
  const float* r = logits + (size_t)row * V;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int j = j0 + threadIdx.x; j < j1; j += ARGMAX_THREADS) {
    const float v = r[j];
    if (v > best) { best = v; bi = j; }  // j increases: first maximum kept
  }
  block_argmax(best, bi);
  if (threadIdx.x == 0) {
    pv[row * ARGMAX_PARTS + part] = best;
    pi[row * ARGMAX_PARTS + part] = bi;
  }
}

__global__ void __launch_bounds__(64) k_argmax_final(const float* __restrict__ pv, const int* __restrict__ pi,
                                                     int32_t* __restrict__ ids) {
  const int row = blockIdx.x, t = threadIdx.x;
  float best = pv[row * ARGMAX_PARTS + t];
  int bi = pi[row * ARGMAX_PARTS + t];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) argmax_combine(best, bi, __shfl_xor(best, o, 64), __shfl_xor(bi, o, 64));
  if (t == 0) ids[row] = bi == 0x7fffffff ? 0 : bi;
}

// Page-table scatter: table[upd[2i]] = upd[2i+1]. The checked build skips (and flags) an entry
// index outside the table's `entries`.
__global__ void k_apply_updates(int32_t* __restrict__ table, const int32_t* __restrict__ upd, int n, int entries,
                                int32_t* __restrict__ flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = upd[2 * i];
#if DORY_CHECKED
  if ((uint32_t)e >= (uint32_t)entries) {
    atomicOr(flags, kDevFlagPageIndex);
    return;
  }
#endif
  table[e] = upd[2 * i + 1];
}

// Rotary table: tab[p][i] = (cos, sin)(p * theta^(-2i/dh)), angle and cos/sin in fp64.
__global__ void k_rope_table(float2* __restrict__ tab, int max_len, int half, int dh, double theta) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)max_len * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)dh);
  const double ang = (double)p * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ void k_copy_f32(float* __restrict__ dst, const float* __restrict__ src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------- launchers

template <typename T>
static hipError_t embed_t(const int32_t* tokens, const void* E, int V, int d, int M, float* h, void* hb,
                          int32_t* err, hipStream_t st) {
  DORY_LAUNCH(k_embed<T>, dim3(M), dim3(ROW_THREADS), 0, st, tokens, (const T*)E, V, d, h, (T*)hb, err);
  return hipGetLastError();
}
hipError_t launch_embed(int dtype, const int32_t* tokens, const void* E, int V, int d, int M, float* h, void* hb,
                        int32_t* err, hipStream_t st) {
  return dtype == 0 ? embed_t<float>(tokens, E, V, d, M, h, hb, err, st)
                    : embed_t<bf16_t>(tokens, E, V, d, M, h, hb, err, st);
}

hipError_t launch_residual(int dtype, float* h, const float* y, const float* alpha, void* hb, int M, int d,
                           hipStream_t st, int parts) {
  if (parts > 1) {
    if (dtype != 1 || parts > 64) return hipErrorInvalidValue;
    const size_t slice = (size_t)M * d;
    if (parts >= 8)
      DORY_LAUNCH((k_residual_parts<bf16_t, 8>), dim3(M), dim3(ROW_THREADS), 0, st, h, y, parts, slice, alpha,
                  (bf16_t*)hb, d);
    else if (parts >= 4)
      DORY_LAUNCH((k_residual_parts<bf16_t, 4>), dim3(M), dim3(ROW_THREADS), 0, st, h, y, parts, slice, alpha,
                  (bf16_t*)hb, d);
    else
      DORY_LAUNCH((k_residual_parts<bf16_t, 2>), dim3(M), dim3(ROW_THREADS), 0, st, h, y, parts, slice, alpha,
                  (bf16_t*)hb, d);
    return hipGetLastError();
  }
  if (dtype == 0)
    DORY_LAUNCH(k_residual<float>, dim3(M), dim3(ROW_THREADS), 0, st, h, y, alpha, (float*)hb, d);
  else
    DORY_LAUNCH(k_residual<bf16_t>, dim3(M), dim3(ROW_THREADS), 0, st, h, y, alpha, (bf16_t*)hb, d);
  return hipGetLastError();
}

hipError_t launch_loop_step(int dtype, float* h, const float* y, const float* alpha, const float* x, float* s,
                            float* hout, void* hb, int M, int d, int mode, hipStream_t st) {
  if (dtype == 0)
    DORY_LAUNCH(k_loop_step<float>, dim3(M), dim3(ROW_THREADS), 0, st, h, y, alpha, x, s, hout, (float*)hb, d, mode);
  else
    DORY_LAUNCH(k_loop_step<bf16_t>, dim3(M), dim3(ROW_THREADS), 0, st, h, y, alpha, x, s, hout, (bf16_t*)hb, d,
                mode);
  return hipGetLastError();
}

hipError_t launch_norm_sum(int dtype, const float* a, const float* b, float* h, float* s, void* hb, int M, int d,
                           hipStream_t st) {
  if (dtype == 0)
    DORY_LAUNCH(k_norm_sum<float>, dim3(M), dim3(ROW_THREADS), 0, st, a, b, h, s, (float*)hb, d);
  else
    DORY_LAUNCH(k_norm_sum<bf16_t>, dim3(M), dim3(ROW_THREADS), 0, st, a, b, h, s, (bf16_t*)hb, d);
  return hipGetLastError();
}

// scratch: rows * ARGMAX_PARTS floats + as many ints
hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* ids, void* scratch, hipStream_t st) {
  float* pv = static_cast<float*>(scratch);
  int* pi = reinterpret_cast<int*>(pv + (size_t)rows * ARGMAX_PARTS);
  DORY_LAUNCH(k_argmax_part, dim3(rows, ARGMAX_PARTS), dim3(ARGMAX_THREADS), 0, st, logits, V, pv, pi);
  DORY_LAUNCH(k_argmax_final, dim3(rows), dim3(64), 0, st, (const float*)pv, (const int*)pi, ids);
  return hipGetLastError();
}

hipError_t launch_apply_updates(int32_t* table, const int32_t* upd, int n, int entries, int32_t* flags,
                                hipStream_t st) {
  if (n <= 0) return hipSuccess;
  DORY_LAUNCH(k_apply_updates, dim3((n + 255) / 256), dim3(256), 0, st, table, upd, n, entries, flags);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* tab, int max_len, int dh, double theta, hipStream_t st) {
  const size_t n = (size_t)max_len * (dh / 2);
  DORY_LAUNCH(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, tab, max_len, dh / 2, dh,
                     theta);
  return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  DORY_LAUNCH(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, dst, src, n);
  return hipGetLastError();
}

}  // namespace dory
