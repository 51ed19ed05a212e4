// Dense projections of the block and the LM head: C[M,N] = A[M,K] . B[N,K]^T
// with A the activations (row-major, K contiguous) and B a weight matrix stored
// [out, in]. Accumulation is fp32. Epilogues: fp32 store, or the SwiGLU of the
// fused gate/up weight (z = silu(A.Bg^T) * (A.Bu^T), Bg = rows 0..F-1 and
// Bu = rows F..2F-1 of B) stored in the model's storage type.
//
//  - k_gemm_mfma: bf16 MFMA (v_mfma_f32_32x32x16_bf16), 128x128x64 tiles,
//    4 waves of 64x64, LDS double-buffered; for the bf16 model at M > 2.
//  - k_gemv_bf16: weight-streaming kernel for M <= 2 rows (decode); the x rows
//    stay in registers, every weight byte is read once, dot2 bf16 FMA.
//  - k_gemm_f32: plain FMA tiles for the fp32 model.
#include "common.h"
#include "kernels.h"

namespace dory {

DORY_DEV float silu(float z) { return z / (1.f + __expf(-z)); }

// ------------------------------------------------------------------ fp32 tiles

constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <bool DUAL>
__global__ void __launch_bounds__(256) k_gemm_f32(const float* __restrict__ A, const float* __restrict__ B,
                                                  float* __restrict__ C, int M, int N, int K, int F) {
  __shared__ float As[F_BK][F_BM + 4];
  __shared__ float Bs[DUAL ? 2 : 1][F_BK][F_BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * F_BM, n0 = blockIdx.x * F_BN;
  float acc[DUAL ? 2 : 1][4][4] = {};
  for (int k0 = 0; k0 < K; k0 += F_BK) {
    for (int i = tid; i < F_BM * F_BK; i += 256) {
      const int r = i / F_BK, c = i % F_BK;
      const int gm = min(m0 + r, M - 1), gk = k0 + c;
      As[c][r] = gk < K ? A[(size_t)gm * K + gk] : 0.f;
    }
    for (int b = 0; b < (DUAL ? 2 : 1); ++b) {
      for (int i = tid; i < F_BN * F_BK; i += 256) {
        const int r = i / F_BK, c = i % F_BK;
        const int gn = min(n0 + r, N - 1) + b * F, gk = k0 + c;
        Bs[b][c][r] = gk < K ? B[(size_t)gn * K + gk] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < (DUAL ? 2 : 1); ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float bv = Bs[b][kk][tx * 4 + j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[b][i][j] += a[i] * bv;
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty * 4 + i, gn = n0 + tx * 4 + j;
      if (gm < M && gn < N) {
        if (DUAL)
          C[(size_t)gm * N + gn] = silu(acc[0][i][j]) * acc[DUAL ? 1 : 0][i][j];
        else
          C[(size_t)gm * N + gn] = acc[0][i][j];
      }
    }
}

// ------------------------------------------------------------------ bf16 MFMA

constexpr int MF_BM = 128, MF_BN = 128, MF_BK = 64;
constexpr int MF_LDA = MF_BK + 8;  // padded LDS row (elements): 144 B rows keep ds_read_b128 conflict-free

// 32x32x16 bf16 MFMA operand layouts (checked on gfx950):
//  A: lane l holds A[l%32][8*(l/32) .. +8);  B: lane l holds B^T[l%32][8*(l/32) .. +8)
//  D: element v of lane l is D[8*(v/4) + 4*(l/32) + v%4][l%32].
template <bool DUAL>
__global__ void __launch_bounds__(256) k_gemm_mfma(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                   void* __restrict__ Cv, int M, int N, int K, int F) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][MF_BM * MF_LDA];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][MF_BN * MF_LDA];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = blockIdx.y * MF_BM;
  // Plain: tile columns n0..n0+127 of C. Dual: z columns c0..c0+63, B rows
  // c0.. (gate) in tile rows 0..63 and F+c0.. (up) in tile rows 64..127.
  const int n0 = DUAL ? blockIdx.x * (MF_BN / 2) : blockIdx.x * MF_BN;

  // global -> register staging: 4 chunks of 16 B per thread for A and for B
  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      const int gm = min(m0 + r, M - 1);
      ra[i] = *reinterpret_cast<const uint4*>(A + (size_t)gm * K + k0 + kc);
      int gn;
      if (DUAL) gn = (r < 64) ? min(n0 + r, F - 1) : F + min(n0 + r - 64, F - 1);
      else gn = min(n0 + r, N - 1);
      rb[i] = *reinterpret_cast<const uint4*>(B + (size_t)gn * K + k0 + kc);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int r = c >> 3, kc = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[buf][r * MF_LDA + kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][r * MF_LDA + kc]) = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int arow = wm * 64 + (lane & 31);
  const int bcol0 = DUAL ? wn * 32 : wn * 64;
  const int bcol1 = DUAL ? 64 + wn * 32 : wn * 64 + 32;
  const int kl = (lane >> 5) * 8;

  const int nk = K / MF_BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * MF_BK);
#pragma unroll
    for (int ks = 0; ks < MF_BK / 16; ++ks) {
      const int kk = ks * 16 + kl;
      bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&As[cur][arow * MF_LDA + kk]);
      bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&As[cur][(arow + 32) * MF_LDA + kk]);
      bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&Bs[cur][(bcol0 + (lane & 31)) * MF_LDA + kk]);
      bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&Bs[cur][(bcol1 + (lane & 31)) * MF_LDA + kk]);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      sstore(cur ^ 1);
    }
    __syncthreads();
  }

  const int col = lane & 31;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int gm = m0 + wm * 64 + rt * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (gm >= M) continue;
      if (DUAL) {
        const int gc = n0 + wn * 32 + col;
        if (gc < F) {
          const float z = silu(acc[rt][0][v]) * acc[rt][1][v];
          reinterpret_cast<bf16_t*>(Cv)[(size_t)gm * F + gc] = f32_to_bf16(z);
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const int gn = n0 + wn * 64 + ct * 32 + col;
          if (gn < N) reinterpret_cast<float*>(Cv)[(size_t)gm * N + gn] = acc[rt][ct][v];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 GEMV (M <= 2)

// One wave per group of R output rows; lane l reads 16-byte chunks l, l+64, ...
// of each weight row (KCH chunks per lane, K = 512*KCH).
template <int KCH, int R, int MR, bool DUAL>
__global__ void __launch_bounds__(256) k_gemv_bf16(const bf16_t* __restrict__ X, const bf16_t* __restrict__ W,
                                                   void* __restrict__ Y, int M, int N, int F) {
  constexpr int K = KCH * 512;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nrows_out = DUAL ? F : N;
  const int r0 = wave * R;
  if (r0 >= nrows_out) return;
  uint4 xr[MR][KCH];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < KCH; ++c)
      xr[m][c] = m < M ? *reinterpret_cast<const uint4*>(X + (size_t)m * K + (size_t)(c * 64 + lane) * 8)
                       : make_uint4(0, 0, 0, 0);
  constexpr int NB = DUAL ? 2 : 1;
  float acc[NB][R][MR];
  u32x4_t wr[NB][R][KCH];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = min(r0 + r, nrows_out - 1) + b * F;
      const bf16_t* wp = W + (size_t)n * K + (size_t)lane * 8;
#pragma unroll
      for (int c = 0; c < KCH; ++c) wr[b][r][c] = *reinterpret_cast<const u32x4_t*>(wp + c * 512);
    }
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

// ------------------------------------------------------------------ launchers

template <int KCH, bool DUAL>
static hipError_t gemv_k(const bf16_t* X, const bf16_t* W, void* Y, int M, int N, int F, hipStream_t st) {
  const int rows_out = DUAL ? F : N;
  constexpr int R = KCH >= 16 ? 1 : 2;  // keeps the weight registers of a wave near 128 VGPRs
  const int waves = (rows_out + R - 1) / R;
  const dim3 grid((waves + 3) / 4);
  if (M == 1)
    hipLaunchKernelGGL((k_gemv_bf16<KCH, R, 1, DUAL>), grid, dim3(256), 0, st, X, W, Y, M, N, F);
  else
    hipLaunchKernelGGL((k_gemv_bf16<KCH, R, 2, DUAL>), grid, dim3(256), 0, st, X, W, Y, M, N, F);
  return hipGetLastError();
}

template <bool DUAL>
static hipError_t gemv_dispatch(const bf16_t* X, const bf16_t* W, void* Y, int M, int N, int K, int F,
                                hipStream_t st) {
  switch (K) {
    case 1024: return gemv_k<2, DUAL>(X, W, Y, M, N, F, st);
    case 3072: return gemv_k<6, DUAL>(X, W, Y, M, N, F, st);
    case 4096: return gemv_k<8, DUAL>(X, W, Y, M, N, F, st);
    case 8192: return gemv_k<16, DUAL>(X, W, Y, M, N, F, st);
    default: return hipErrorNotSupported;
  }
}

bool gemv_supported(int K) { return K == 1024 || K == 3072 || K == 4096 || K == 8192; }

// out: fp32 [M,N] (plain) or storage-type z [M,F] (dual, N = 2F).
hipError_t launch_gemm(int dtype, bool dual, const void* A, const void* B, void* out, int M, int N, int K,
                       hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int F = dual ? N / 2 : 0;
  if (dtype == 0) {
    const int ncols = dual ? F : N;
    dim3 grid((ncols + F_BN - 1) / F_BN, (M + F_BM - 1) / F_BM);
    if (dual)
      hipLaunchKernelGGL(k_gemm_f32<true>, grid, dim3(256), 0, st, (const float*)A, (const float*)B, (float*)out,
                         M, F, K, F);
    else
      hipLaunchKernelGGL(k_gemm_f32<false>, grid, dim3(256), 0, st, (const float*)A, (const float*)B, (float*)out,
                         M, N, K, 0);
    return hipGetLastError();
  }
  if (K % MF_BK != 0) return hipErrorNotSupported;
  if (M <= 2 && gemv_supported(K)) {
    return dual ? gemv_dispatch<true>((const bf16_t*)A, (const bf16_t*)B, out, M, N, K, F, st)
                : gemv_dispatch<false>((const bf16_t*)A, (const bf16_t*)B, out, M, N, K, F, st);
  }
  const int ncols = dual ? F : N;
  dim3 grid((ncols + (dual ? MF_BN / 2 : MF_BN) - 1) / (dual ? MF_BN / 2 : MF_BN), (M + MF_BM - 1) / MF_BM);
  if (dual)
    hipLaunchKernelGGL(k_gemm_mfma<true>, grid, dim3(256), 0, st, (const bf16_t*)A, (const bf16_t*)B, out, M, N, K, F);
  else
    hipLaunchKernelGGL(k_gemm_mfma<false>, grid, dim3(256), 0, st, (const bf16_t*)A, (const bf16_t*)B, out, M, N, K, 0);
  return hipGetLastError();
}

}  // namespace dory
