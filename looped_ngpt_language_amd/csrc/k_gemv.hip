// Weight-streaming GEMV for decode (M <= 2 rows): C[M,N] = X[M,K] . W[N,K]^T
// with every weight byte read once. Epilogues as in the GEMM: fp32 store, or
// the SwiGLU of the fused gate/up weight (z = silu(X.Wg^T) * (X.Wu^T), Wg = rows
// 0..F-1 and Wu = rows F..2F-1 of W) stored as bf16.
//
// The input rows are either bf16 rows X [M, K] or (RES) the pending
// normalised residual step of the previous sublayer,
//   x = N(h + alpha * (N(y) - h))     (h, y fp32 [M, K], alpha [K]; nGPT backbone,
// onedev.kr summary "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를 조절한다", section
// "어떻게 동작하나"): the workgroup builds bf16(x) in LDS while its weight loads
// are in flight, and workgroup 0 writes the fp32 x to hout for the next
// residual step.
#include "common.h"
#include "kernels.h"

namespace dory {

// One wave per group of R output rows; lane l reads 16-byte chunks l, l+64, ...
// of each weight row (KCH chunks per lane, K = 512*KCH). The weight loads are
// issued first.
template <int KCH, int R, int MR, bool DUAL, bool RES>
__global__ void __launch_bounds__(256) k_gemv_bf16(const bf16_t* __restrict__ X, const bf16_t* __restrict__ W,
                                                   void* __restrict__ Y, int M, int N, int F,
                                                   const float* __restrict__ rh, const float* __restrict__ ry,
                                                   const float* __restrict__ ralpha, float* __restrict__ hout) {
  constexpr int K = KCH * 512;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = blockIdx.x * 4 + (tid >> 6);
  const int nrows_out = DUAL ? F : N;
  const int r0 = wave * R;
  const bool active = r0 < nrows_out;
  constexpr int NB = DUAL ? 2 : 1;
  u32x4_t wr[NB][R][KCH];
  if (active) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(r0 + r, nrows_out - 1) + b * F;
        const bf16_t* wp = W + (size_t)n * K + (size_t)lane * 8;
#pragma unroll
        for (int c = 0; c < KCH; ++c) wr[b][r][c] = *reinterpret_cast<const u32x4_t*>(wp + c * 512);
      }
  }
  uint4 xr[MR][KCH];
  if constexpr (RES) {
    constexpr int EPT = K / 256;
    __shared__ __attribute__((aligned(16))) bf16_t xs[MR][K];
    __shared__ float red[4];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      if (m >= M) break;
      float hv[EPT], yv[EPT];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + 256 * e;
        hv[e] = rh[(size_t)m * K + i];
        yv[e] = ry[(size_t)m * K + i];
        ss += yv[e] * yv[e];
      }
      const float iy = rsqrtf(fmaxf(block_sum(ss, red, 4), DORY_TINY_SS));
      float st = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + 256 * e;
        hv[e] += ralpha[i] * (yv[e] * iy - hv[e]);
        st += hv[e] * hv[e];
      }
      const float ih = rsqrtf(fmaxf(block_sum(st, red, 4), DORY_TINY_SS));
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + 256 * e;
        const float v = hv[e] * ih;
        xs[m][i] = f32_to_bf16(v);
        if (blockIdx.x == 0) hout[(size_t)m * K + i] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        xr[m][c] = m < M ? *reinterpret_cast<const uint4*>(&xs[m][(c * 64 + lane) * 8]) : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        xr[m][c] = m < M ? *reinterpret_cast<const uint4*>(X + (size_t)m * K + (size_t)(c * 64 + lane) * 8)
                         : make_uint4(0, 0, 0, 0);
  }
  if (!active) return;
  float acc[NB][R][MR];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const u32x4_t w = wr[b][r][c];
          const uint4 x = xr[m][c];
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), s, false);
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), s, false);
        }
        acc[b][r][m] = wave_sum(s);
      }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = r0 + r;
      if (n >= nrows_out) continue;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if (m >= M) continue;
        if (DUAL)
          reinterpret_cast<bf16_t*>(Y)[(size_t)m * F + n] = f32_to_bf16(silu(acc[0][r][m]) * acc[NB - 1][r][m]);
        else
          reinterpret_cast<float*>(Y)[(size_t)m * N + n] = acc[0][r][m];
      }
    }
  }
}

struct ResArgs {
  const float *h, *y, *alpha;
  float* hout;
};

template <int KCH, bool DUAL, bool RES>
static hipError_t gemv_k(const bf16_t* X, const bf16_t* W, void* Y, int M, int N, int F, const ResArgs& ra,
                         hipStream_t st) {
  const int rows_out = DUAL ? F : N;
  constexpr int R = KCH >= 16 ? 1 : 2;  // keeps the weight registers of a wave near 128 VGPRs
  const int waves = (rows_out + R - 1) / R;
  const dim3 grid((waves + 3) / 4);
  if (M == 1)
    DORY_LAUNCH((k_gemv_bf16<KCH, R, 1, DUAL, RES>), grid, dim3(256), 0, st, X, W, Y, M, N, F, ra.h, ra.y, ra.alpha,
                ra.hout);
  else
    DORY_LAUNCH((k_gemv_bf16<KCH, R, 2, DUAL, RES>), grid, dim3(256), 0, st, X, W, Y, M, N, F, ra.h, ra.y, ra.alpha,
                ra.hout);
  return hipGetLastError();
}

template <bool DUAL, bool RES>
static hipError_t gemv_dispatch(const bf16_t* X, const bf16_t* W, void* Y, int M, int N, int K, int F,
                                const ResArgs& ra, hipStream_t st) {
  switch (K) {
    case 1024: return gemv_k<2, DUAL, RES>(X, W, Y, M, N, F, ra, st);
    case 3072: return gemv_k<6, DUAL, RES>(X, W, Y, M, N, F, ra, st);
    case 4096: return gemv_k<8, DUAL, RES>(X, W, Y, M, N, F, ra, st);
    case 8192:
      if constexpr (!RES) return gemv_k<16, DUAL, false>(X, W, Y, M, N, F, ra, st);
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

bool gemv_supported(int K) { return K == 1024 || K == 3072 || K == 4096 || K == 8192; }
bool gemv_residual_supported(int K) { return K == 1024 || K == 3072 || K == 4096; }

hipError_t launch_gemv(bool dual, const void* X, const void* W, void* out, int M, int N, int K, hipStream_t st) {
  if (M < 1 || M > 2 || !gemv_supported(K)) return hipErrorNotSupported;
  const int F = dual ? N / 2 : 0;
  const ResArgs none{nullptr, nullptr, nullptr, nullptr};
  return dual ? gemv_dispatch<true, false>((const bf16_t*)X, (const bf16_t*)W, out, M, N, K, F, none, st)
              : gemv_dispatch<false, false>((const bf16_t*)X, (const bf16_t*)W, out, M, N, K, F, none, st);
}

hipError_t launch_gemv_residual(bool dual, const void* W, void* out, int M, int N, int K, const float* h,
                                const float* y, const float* alpha, float* hout, hipStream_t st) {
  if (M < 1 || M > 2 || !gemv_residual_supported(K)) return hipErrorNotSupported;
  const int F = dual ? N / 2 : 0;
  const ResArgs ra{h, y, alpha, hout};
  return dual ? gemv_dispatch<true, true>(nullptr, (const bf16_t*)W, out, M, N, K, F, ra, st)
              : gemv_dispatch<false, true>(nullptr, (const bf16_t*)W, out, M, N, K, F, ra, st);
}

}  // namespace dory
