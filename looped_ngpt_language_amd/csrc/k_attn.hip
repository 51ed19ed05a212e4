// Attention sublayer kernels: rotary embedding + per-head L2 norm of q and k with
// the paged KV write, row attention (split over keys for decode) and the merge
// of split partials.
//
// Attention of a row at position p, query head h, KV head g = h / (H/H_kv):
//   o = sum_j softmax_j(scale * q^.k^_j) v_j over keys p-W < j <= p (sliding
//   window) or 0 <= j <= p (full); every 4th physical block is full, the rest
//   sliding-window (onedev.kr summary "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를
//   조절한다", section "어떻게 동작하나": 3:1 interleave).
// The chunk's keys/values are written to the block's cache slot before any
// query reads it; in last-loop mode every loop writes the recurrent block's
// single slot (onedev.kr, section "전제와 한계").
//
// KV pool layout: slot-major; a page slot holds 16 tokens of one layer slot:
//   [K|V][H_kv][16 tokens][d_h] in the storage type.
#include "common.h"
#include "kernels.h"

namespace dory {

// One wave per (row, head). Heads 0..H-1 are queries: q^ = N(RoPE(q)) -> q_out.
// Heads H..H+H_kv-1 are keys: k^ = N(RoPE(k)) and v go to the cache page of the
// row's position.
template <typename T>
__global__ void __launch_bounds__(64) k_rope_qk_kv(const float* __restrict__ qkv, const int32_t* __restrict__ rows,
                                                   const int32_t* __restrict__ ptab, int max_pages,
                                                   const float2* __restrict__ rope, T* __restrict__ q_out,
                                                   T* __restrict__ kv_slot, int H, int Hkv, int dh,
                                                   size_t page_elems) {
  const int m = blockIdx.x, hd = blockIdx.y, lane = threadIdx.x;
  const int seq = rows[2 * m], pos = rows[2 * m + 1];
  const int half = dh >> 1;
  const int nq = (H + 2 * Hkv) * dh;
  const float* src = qkv + (size_t)m * nq + (size_t)hd * dh;
  float a0 = 0.f, a1 = 0.f;  // pair (i, i + dh/2) with i = lane (dh <= 128)
  const bool act = lane < half;
  if (act) {
    const float x1 = src[lane], x2 = src[lane + half];
    const float2 cs = rope[(size_t)pos * half + lane];
    a0 = x1 * cs.x - x2 * cs.y;
    a1 = x1 * cs.y + x2 * cs.x;
  }
  const float r = rsqrtf(fmaxf(wave_sum(a0 * a0 + a1 * a1), DORY_TINY_SS));
  if (hd < H) {
    if (act) {
      T* q = q_out + (size_t)m * H * dh + (size_t)hd * dh;
      St<T>::st(q, lane, a0 * r);
      St<T>::st(q, lane + half, a1 * r);
    }
    return;
  }
  const int g = hd - H;
  const int page = ptab[(size_t)seq * max_pages + (pos >> 4)];
  T* kp = kv_slot + (size_t)page * page_elems + ((size_t)g * 16 + (pos & 15)) * dh;
  T* vp = kp + (size_t)Hkv * 16 * dh;
  const float* vsrc = src + (size_t)Hkv * dh;
  if (act) {
    St<T>::st(kp, lane, a0 * r);
    St<T>::st(kp, lane + half, a1 * r);
    St<T>::st(vp, lane, vsrc[lane]);
    St<T>::st(vp, lane + half, vsrc[lane + half]);
  }
}

constexpr int ATT_THREADS = 256;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int GMAX = 8;  // query heads per KV head

DORY_DEV float safe_scale(float m_old, float m_new) { return m_old == -INFINITY ? 0.f : __expf(m_old - m_new); }

// Row attention: grid (rows, H_kv, splits). Each workgroup handles the query
// heads of one KV head for one row over one contiguous share of its key range.
// A lane holds 8 consecutive dims; LPK = DH/8 lanes share one key.
template <typename T, int DH>
__global__ void __launch_bounds__(ATT_THREADS) k_attn_rows(
    const T* __restrict__ q, const int32_t* __restrict__ rows, const int32_t* __restrict__ ptab, int max_pages,
    const T* __restrict__ kv_slot, size_t page_elems, int H, int Hkv, int window, float scale, int splits,
    T* __restrict__ out, float* __restrict__ part_ml, float* __restrict__ part_o) {
  constexpr int LPK = DH / 8;
  constexpr int KPW = 64 / LPK;
  __shared__ float sm[ATT_WAVES][GMAX], sl[ATT_WAVES][GMAX];
  __shared__ float so[ATT_WAVES][GMAX][DH];

  const int m = blockIdx.x, g = blockIdx.y, sp = blockIdx.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int G = H / Hkv;
  const int seq = rows[2 * m], pos = rows[2 * m + 1];
  const int lo = window > 0 ? max(0, pos - window + 1) : 0;
  const int nkeys = pos - lo + 1;
  const int chunk = (nkeys + splits - 1) / splits;
  const int kbeg = lo + sp * chunk;
  const int kend = min(pos + 1, kbeg + chunk);
  const int e0 = (lane % LPK) * 8;

  float qf[GMAX][8];
#pragma unroll
  for (int gi = 0; gi < GMAX; ++gi) {
    if (gi < G) {
      load8(q + ((size_t)m * H + (size_t)g * G + gi) * DH + e0, qf[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[gi][e] *= scale;
    }
  }
  float mx[GMAX], ls[GMAX], acc[GMAX][8];
#pragma unroll
  for (int gi = 0; gi < GMAX; ++gi) {
    mx[gi] = -INFINITY;
    ls[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
  }
  const size_t vofs = (size_t)Hkv * 16 * DH;
  for (int j = kbeg + wv * KPW + lane / LPK; j < kend; j += ATT_WAVES * KPW) {
    const int page = ptab[(size_t)seq * max_pages + (j >> 4)];
    const T* kp = kv_slot + (size_t)page * page_elems + ((size_t)g * 16 + (j & 15)) * DH + e0;
    float kf[8], vf[8];
    load8(kp, kf);
    load8(kp + vofs, vf);
#pragma unroll
    for (int gi = 0; gi < GMAX; ++gi) {
      if (gi < G) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += qf[gi][e] * kf[e];
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) s += __shfl_xor(s, o, 64);
        const float mn = fmaxf(mx[gi], s);
        const float c = safe_scale(mx[gi], mn);
        const float p = __expf(s - mn);
        ls[gi] = ls[gi] * c + p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = acc[gi][e] * c + p * vf[e];
        mx[gi] = mn;
      }
    }
  }
  // Merge the key groups of the wave (lanes differing in lane / LPK).
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
#pragma unroll
    for (int gi = 0; gi < GMAX; ++gi) {
      if (gi < G) {
        const float m2 = __shfl_xor(mx[gi], o, 64);
        const float l2 = __shfl_xor(ls[gi], o, 64);
        const float mn = fmaxf(mx[gi], m2);
        const float c1 = safe_scale(mx[gi], mn), c2 = safe_scale(m2, mn);
        ls[gi] = ls[gi] * c1 + l2 * c2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a2 = __shfl_xor(acc[gi][e], o, 64);
          acc[gi][e] = acc[gi][e] * c1 + a2 * c2;
        }
        mx[gi] = mn;
      }
    }
  }
  if (lane < LPK) {
    for (int gi = 0; gi < G; ++gi) {
      if (lane == 0) { sm[wv][gi] = mx[gi]; sl[wv][gi] = ls[gi]; }
#pragma unroll
      for (int e = 0; e < 8; ++e) so[wv][gi][e0 + e] = acc[gi][e];
    }
  }
  __syncthreads();
  // Merge the waves: thread t handles (head gi, dim e) pairs.
  for (int idx = threadIdx.x; idx < G * DH; idx += ATT_THREADS) {
    const int gi = idx / DH, e = idx % DH;
    float M = -INFINITY;
    for (int w = 0; w < ATT_WAVES; ++w) M = fmaxf(M, sm[w][gi]);
    float L = 0.f, A = 0.f;
    for (int w = 0; w < ATT_WAVES; ++w) {
      const float c = safe_scale(sm[w][gi], M);
      L += sl[w][gi] * c;
      A += so[w][gi][e] * c;
    }
    const int hq = g * G + gi;
    if (splits == 1) {
      St<T>::st(out, ((size_t)m * H + hq) * DH + e, L > 0.f ? A / L : 0.f);
    } else {
      const size_t pi = ((size_t)m * H + hq) * splits + sp;
      part_o[pi * DH + e] = A;
      if (e == 0) { part_ml[2 * pi] = M; part_ml[2 * pi + 1] = L; }
    }
  }
}

// Merge split partials: grid rows*H, block DH threads.
template <typename T>
__global__ void k_attn_merge(const float* __restrict__ part_ml, const float* __restrict__ part_o, int splits,
                             int dh, T* __restrict__ out) {
  const size_t rh = blockIdx.x;
  const int e = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[2 * (rh * splits + s)]);
  float L = 0.f, A = 0.f;
  for (int s = 0; s < splits; ++s) {
    const size_t pi = rh * splits + s;
    const float c = safe_scale(part_ml[2 * pi], M);
    L += part_ml[2 * pi + 1] * c;
    A += part_o[pi * dh + e] * c;
  }
  if (e < dh) St<T>::st(out, rh * dh + e, L > 0.f ? A / L : 0.f);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_rope_qk_kv(int dtype, const float* qkv, const int32_t* rows, const int32_t* ptab, int max_pages,
                             const float2* rope, void* q_out, void* kv_slot, int M, int H, int Hkv, int dh,
                             size_t page_elems, hipStream_t st) {
  dim3 grid(M, H + Hkv);
  if (dtype == 0)
    hipLaunchKernelGGL(k_rope_qk_kv<float>, grid, dim3(64), 0, st, qkv, rows, ptab, max_pages, rope,
                       (float*)q_out, (float*)kv_slot, H, Hkv, dh, page_elems);
  else
    hipLaunchKernelGGL(k_rope_qk_kv<bf16_t>, grid, dim3(64), 0, st, qkv, rows, ptab, max_pages, rope,
                       (bf16_t*)q_out, (bf16_t*)kv_slot, H, Hkv, dh, page_elems);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_t(const void* q, const int32_t* rows, const int32_t* ptab, int max_pages, const void* kv,
                         size_t page_elems, int M, int H, int Hkv, int dh, int window, float scale, int splits,
                         void* out, float* part_ml, float* part_o, hipStream_t st) {
  dim3 grid(M, Hkv, splits);
#define DORY_ATT(DHV)                                                                                         \
  hipLaunchKernelGGL((k_attn_rows<T, DHV>), grid, dim3(ATT_THREADS), 0, st, (const T*)q, rows, ptab, max_pages, \
                     (const T*)kv, page_elems, H, Hkv, window, scale, splits, (T*)out, part_ml, part_o)
  switch (dh) {
    case 32: DORY_ATT(32); break;
    case 64: DORY_ATT(64); break;
    case 128: DORY_ATT(128); break;
    default: return hipErrorInvalidValue;
  }
#undef DORY_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(k_attn_merge<T>, dim3(M * H), dim3(dh), 0, st, part_ml, part_o, splits, dh, (T*)out);
  return hipGetLastError();
}

hipError_t launch_attn_rows(int dtype, const void* q, const int32_t* rows, const int32_t* ptab, int max_pages,
                            const void* kv, size_t page_elems, int M, int H, int Hkv, int dh, int window,
                            float scale, int splits, void* out, float* part_ml, float* part_o, hipStream_t st) {
  if (H / Hkv > GMAX) return hipErrorInvalidValue;
  return dtype == 0 ? attn_t<float>(q, rows, ptab, max_pages, kv, page_elems, M, H, Hkv, dh, window, scale, splits,
                                    out, part_ml, part_o, st)
                    : attn_t<bf16_t>(q, rows, ptab, max_pages, kv, page_elems, M, H, Hkv, dh, window, scale, splits,
                                     out, part_ml, part_o, st);
}

}  // namespace dory
