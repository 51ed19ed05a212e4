// Dense projections of the block and the LM head: C[M,N] = A[M,K] . B[N,K]^T
// with A the activations (row-major, K contiguous) and B a weight matrix stored
// [out, in]. Accumulation is fp32. Epilogues: fp32 store, or the SwiGLU of the
// fused gate/up weight (z = silu(A.Bg^T) * (A.Bu^T), Bg = rows 0..F-1 and
// Bu = rows F..2F-1 of B) stored in the model's storage type.
//
//  - k_gemm_tile: bf16 MFMA (v_mfma_f32_16x16x32_bf16) tiles of 128..256 rows
//    and columns, LDS double-buffered, optional split-K; for the bf16 model at
//    M > 2 (M <= 2 goes to the weight-streaming GEMV of k_gemv.hip).
//  - k_gemm_f32: plain FMA tiles for the fp32 model.
#include "common.h"
#include "kernels.h"

namespace dory {

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

constexpr int MF_BK = 64;

// 16x16x32 bf16 MFMA operand layouts (gfx950):
//  A: lane l holds A[l%16][8*(l/16) .. +8);  B: lane l holds B^T[l%16][8*(l/16) .. +8)
//  D: element v of lane l is D[4*(l/16) + v][l%16].
// (The 32x32x16 form gives bit-identical results here but sustains a lower
// MFMA rate under the chip's power management on these shapes: measured
// 5-10% slower per projection.)
//
// Tile BM x BN x 64, WM x WN waves of (BM/WM) x (BN/WN), TM x TN MFMA tiles of
// 16x16 per wave. LDS is double-buffered; the operand tiles of k-tile kt+1 are
// loaded into registers (16 bytes per lane per load: lane l of a wave load
// covers bytes 16l..16l+15 of a 1 KB block = 8 tile rows of 64 bf16) while
// k-tile kt is multiplied, and written to the idle LDS buffer afterwards, so the
// global-load latency overlaps a whole k-tile of MFMA work. (Direct
// global->LDS loads would save the register round trip, but the compiler then
// waits for every outstanding load before each LDS read, since it cannot tell
// the two buffers apart.) With PF2 two register sets alternate and each k-tile
// is requested two k-tiles ahead (more latency cover, more registers).
// LDS banks: gfx950 serves a 16-byte-per-lane read to 64 banks of 4 bytes, so
// the 16 rows a pass touches (128 bytes each) must land on 16 distinct
// (row parity, chunk) pairs: the eight 16-byte chunks of row r are XOR-swizzled
// by (r >> 1) & 7 (rows r, r + 1 share the swizzle but sit in opposite bank
// halves), which the LDS conflict counter reads as zero.
// The grid is 1-D; workgroup b runs on XCD b % 8, and tiles are dealt so each
// XCD walks a contiguous run of weight-column tiles over all row tiles, which
// keeps every weight tile's re-reads inside one XCD's L2.
// Dual: the tile's B rows are BN/2 gate rows then the BN/2 matching up rows;
// gate tile j pairs with up tile j + TN/2 in the same lanes for the epilogue.
// Split-K: blockIdx.y selects the K range [y * k_len, (y+1) * k_len); with
// gridDim.y > 1 (plain only) the fp32 tile goes to partial slice y of Cv,
// [gridDim.y][M][N], summed afterwards by k_splitk_reduce.
DORY_DEV int lds_swz(int r) { return (r >> 1) & 7; }

template <int BM, int BN, int WM, int WN, bool DUAL, bool PF2>
__global__ void __launch_bounds__(64 * WM * WN) k_gemm_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                            void* __restrict__ Cv, int M, int N, int K, int F,
                                                            int m_tiles, int n_tiles, int k_len) {
  constexpr int WAVES = WM * WN;
  constexpr int MS = 16;                                     // MFMA tile edge
  constexpr int TM = BM / (MS * WM), TN = BN / (MS * WN);
  constexpr int IA = BM / (8 * WAVES), IB = BN / (8 * WAVES);  // 1 KB load instructions per wave per k-tile
  static_assert(TM >= 1 && TN >= 1 && IA * 8 * WAVES == BM && IB * 8 * WAVES == BN && (!DUAL || TN % 2 == 0),
                "tile shape");
  __shared__ __attribute__((aligned(1024))) bf16_t As[2][BM * MF_BK];
  __shared__ __attribute__((aligned(1024))) bf16_t Bs[2][BN * MF_BK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;

  const int ntiles = m_tiles * n_tiles;
  const int b = blockIdx.x;
  int t = b;
  if ((ntiles & 7) == 0) t = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int tm = t % m_tiles, tn = t / m_tiles;
  const int m0 = tm * BM;
  const int n0 = DUAL ? tn * (BN / 2) : tn * BN;  // first C column (plain) or z column (dual)

  // this lane's global source row and chunk for each load instruction: lane l
  // fills physical slot l & 7 of tile row 8i + l/8, i.e. logical chunk (l & 7) ^ swz
  const int lrow = lane >> 3;                  // row within the 8-row block
  const int kbase = blockIdx.y * k_len;
  const bf16_t* asrc[IA];
  const bf16_t* bsrc[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r = (wid * IA + i) * 8 + lrow;
    asrc[i] = A + (size_t)min(m0 + r, M - 1) * K + kbase + ((lane & 7) ^ lds_swz(r)) * 8;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int r = (wid * IB + i) * 8 + lrow;
    int gn;
    if (DUAL) gn = (r < BN / 2) ? min(n0 + r, F - 1) : F + min(n0 + r - BN / 2, F - 1);
    else gn = min(n0 + r, N - 1);
    bsrc[i] = B + (size_t)gn * K + kbase + ((lane & 7) ^ lds_swz(r)) * 8;
  }

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  // B-tile row of this wave's column tile j
  int brow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (DUAL) brow[j] = j < TN / 2 ? wn * (BN / (2 * WN)) + j * MS : BN / 2 + wn * (BN / (2 * WN)) + (j - TN / 2) * MS;
    else brow[j] = wn * (BN / WN) + j * MS;
  }
  const int arow0 = wm * (BM / WM) + (lane & 15);
  const int kgrp = lane >> 4;  // 8-element k group of this lane within an MFMA's 32 k

  const int nk = k_len / MF_BK;
  float* const Cf = reinterpret_cast<float*>(Cv) + (size_t)blockIdx.y * M * N;
#define DORY_GLOAD(RA, RB, K1)                                                                                   \
  do {                                                                                                           \
    _Pragma("unroll") for (int i = 0; i < IA; ++i) RA[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + (K1));    \
    _Pragma("unroll") for (int i = 0; i < IB; ++i) RB[i] = *reinterpret_cast<const u32x4_t*>(bsrc[i] + (K1));    \
  } while (0)
#define DORY_SWRITE(RA, RB, S)                                                                                   \
  do {                                                                                                           \
    _Pragma("unroll") for (int i = 0; i < IA; ++i)                                                               \
      *reinterpret_cast<u32x4_t*>(&As[S][(wid * IA + i) * 512 + lane * 8]) = RA[i];                              \
    _Pragma("unroll") for (int i = 0; i < IB; ++i)                                                               \
      *reinterpret_cast<u32x4_t*>(&Bs[S][(wid * IB + i) * 512 + lane * 8]) = RB[i];                              \
  } while (0)
#define DORY_COMPUTE(S)                                                                                          \
  do {                                                                                                           \
    const bf16_t* as = As[S];                                                                                    \
    const bf16_t* bs = Bs[S];                                                                                    \
    _Pragma("unroll") for (int ks = 0; ks < MF_BK / 32; ++ks) {                                                  \
      const int ch = 4 * ks + kgrp; /* logical 16-byte chunk of this lane's 8 k values */                        \
      bf16x8_t af[TM], bfr[TN];                                                                                  \
      _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                                           \
        const int r = arow0 + i * MS;                                                                            \
        af[i] = *reinterpret_cast<const bf16x8_t*>(&as[r * 64 + ((ch ^ lds_swz(r)) << 3)]);                      \
      }                                                                                                          \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                                           \
        const int r = brow[j] + (lane & 15);                                                                     \
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&bs[r * 64 + ((ch ^ lds_swz(r)) << 3)]);                     \
      }                                                                                                          \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                                             \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                                           \
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);                \
    }                                                                                                            \
  } while (0)
  u32x4_t ra[IA], rb[IB];
  if constexpr (!PF2) {
    DORY_GLOAD(ra, rb, 0);
    DORY_SWRITE(ra, rb, 0);
    if (nk > 1) DORY_GLOAD(ra, rb, MF_BK);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      DORY_COMPUTE(cur);
      if (kt + 1 < nk) {
        DORY_SWRITE(ra, rb, cur ^ 1);  // every wave finished reading buffer cur^1 before the last barrier
        if (kt + 2 < nk) DORY_GLOAD(ra, rb, (kt + 2) * MF_BK);
      }
      __syncthreads();
    }
  } else {
    // register set 0 carries the odd k-tiles, set 1 the even ones (from tile 2)
    u32x4_t ra1[IA], rb1[IB];
    DORY_GLOAD(ra, rb, 0);
    DORY_SWRITE(ra, rb, 0);
    if (nk > 1) DORY_GLOAD(ra, rb, MF_BK);
    if (nk > 2) DORY_GLOAD(ra1, rb1, 2 * MF_BK);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      DORY_COMPUTE(0);
      if (kt + 1 >= nk) break;
      DORY_SWRITE(ra, rb, 1);
      if (kt + 3 < nk) DORY_GLOAD(ra, rb, (kt + 3) * MF_BK);
      __syncthreads();
      DORY_COMPUTE(1);
      if (kt + 2 < nk) {
        DORY_SWRITE(ra1, rb1, 0);
        if (kt + 4 < nk) DORY_GLOAD(ra1, rb1, (kt + 4) * MF_BK);
      }
      __syncthreads();
    }
  }
#undef DORY_COMPUTE
#undef DORY_GLOAD
#undef DORY_SWRITE

  const int col = lane & 15;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int gm = m0 + wm * (BM / WM) + i * MS + 4 * (lane >> 4) + v;
      if (gm >= M) continue;
      if (DUAL) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int gc = n0 + wn * (BN / (2 * WN)) + j * MS + col;
          if (gc < F) {
            const float z = silu(acc[i][j][v]) * acc[i][j + TN / 2][v];
            reinterpret_cast<bf16_t*>(Cv)[(size_t)gm * F + gc] = f32_to_bf16(z);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int gn = n0 + wn * (BN / WN) + j * MS + col;
          if (gn < N) Cf[(size_t)gm * N + gn] = acc[i][j][v];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

// Sum of split-K partials [S][M][N]: plain -> fp32 [M][N]; dual (N = 2F) ->
// bf16 z[m][c] = silu(gate) * up with gate = column c, up = column F + c.
template <bool DUAL>
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* __restrict__ part, int S, int M, int N,
                                                       void* __restrict__ out) {
  const int cols = DUAL ? N / 2 : N;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)M * cols) return;
  const size_t m = idx / cols, c = idx % cols;
  const size_t slice = (size_t)M * N;
  float a = 0.f, u = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    a += part[sp * slice + m * N + c];
    if (DUAL) u += part[sp * slice + m * N + cols + c];
  }
  if (DUAL) reinterpret_cast<bf16_t*>(out)[idx] = f32_to_bf16(silu(a) * u);
  else reinterpret_cast<float*>(out)[idx] = a;
}

template <int BM, int BN, int WM, int WN, bool PF2 = false>
static hipError_t tile_launch(const bf16_t* A, const bf16_t* B, void* out, int M, int N, int K, int F, bool dual,
                              hipStream_t st) {
  const int ncols = dual ? F : N;
  const int cols_per_tile = dual ? BN / 2 : BN;
  const int mt = (M + BM - 1) / BM, nt = (ncols + cols_per_tile - 1) / cols_per_tile;
  const dim3 grid(mt * nt), block(64 * WM * WN);
  if (dual) {
    if constexpr ((BN / (16 * WN)) % 2 == 0)
      DORY_LAUNCH((k_gemm_tile<BM, BN, WM, WN, true, PF2>), grid, block, 0, st, A, B, out, M, N, K, F, mt, nt, K);
    else
      return hipErrorNotSupported;
  } else {
    DORY_LAUNCH((k_gemm_tile<BM, BN, WM, WN, false, PF2>), grid, block, 0, st, A, B, out, M, N, K, F, mt, nt, K);
  }
  return hipGetLastError();
}

// Tile shape: the candidate with the least estimated time, taken as the tiles
// of the busiest CU (tiles dealt evenly over 256 CUs) times the tile's area over
// its measured per-CU rate (area per unit time at equal K on the ~4B prefill
// projections: 256x256 on gate/up, 256x192 on qkv, 128x192 on o and down,
// 256x128 and 128x128 on the same shapes). Shapes that split N into about 256
// tiles (one per CU) avoid the half-empty last round a larger tile leaves.
static hipError_t launch_tile_gemm(const bf16_t* A, const bf16_t* B, void* out, int M, int N, int K, int F, bool dual,
                                   hipStream_t st) {
  const int ncols = dual ? F : N;
  struct Cand { int bm, bn, tn; double rate; };  // tn: MFMA column tiles per wave (dual needs an even count)
  static const Cand cands[] = {{256, 256, 8, 4.0}, {256, 192, 6, 3.69}, {128, 192, 6, 3.15},
                               {256, 128, 4, 3.34}, {128, 128, 4, 2.87}};
  int best = 0;
  double best_t = 1e300;
  for (int i = 0; i < (int)(sizeof(cands) / sizeof(cands[0])); ++i) {
    const Cand& c = cands[i];
    if (dual && c.tn % 2) continue;
    const int cpt = dual ? c.bn / 2 : c.bn;
    const long tiles = (long)((M + c.bm - 1) / c.bm) * ((ncols + cpt - 1) / cpt);
    const double t = (double)((tiles + 255) / 256) * c.bm * c.bn / c.rate;
    if (t < best_t * 0.999) { best_t = t; best = i; }
  }
  switch (best) {
    case 0: return tile_launch<256, 256, 4, 2>(A, B, out, M, N, K, F, dual, st);
    case 1: return tile_launch<256, 192, 4, 2>(A, B, out, M, N, K, F, dual, st);
    case 2: return tile_launch<128, 192, 4, 2, true>(A, B, out, M, N, K, F, dual, st);
    case 3: return tile_launch<256, 128, 4, 2>(A, B, out, M, N, K, F, dual, st);
    default: return tile_launch<128, 128, 2, 2>(A, B, out, M, N, K, F, dual, st);
  }
}

// out: fp32 [M,N] (plain) or storage-type z [M,F] (dual, N = 2F).
// Few rows (3..256): 128x128 tiles leave most CUs idle, so K is split until the
// grid has >= 256 workgroups (partials in `split_ws`, then a reduce kernel).
static int choose_split(int M, int N, int K, size_t split_ws_bytes) {
  const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  int S = 1;
  while (tiles * S < 256 && S < 16 && (K / MF_BK) % (2 * S) == 0 &&
         (size_t)(2 * S) * M * N * sizeof(float) <= split_ws_bytes)
    S *= 2;
  return S;
}

hipError_t launch_gemm(int dtype, bool dual, const void* A, const void* B, void* out, int M, int N, int K,
                       float* split_ws, size_t split_ws_bytes, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  const int F = dual ? N / 2 : 0;
  if (dtype == 0) {
    const int ncols = dual ? F : N;
    dim3 grid((ncols + F_BN - 1) / F_BN, (M + F_BM - 1) / F_BM);
    if (dual)
      DORY_LAUNCH(k_gemm_f32<true>, grid, dim3(256), 0, st, (const float*)A, (const float*)B, (float*)out,
                         M, F, K, F);
    else
      DORY_LAUNCH(k_gemm_f32<false>, grid, dim3(256), 0, st, (const float*)A, (const float*)B, (float*)out,
                         M, N, K, 0);
    return hipGetLastError();
  }
  if (K % MF_BK != 0) return hipErrorNotSupported;
  if (M <= 2 && gemv_supported(K)) return launch_gemv(dual, A, B, nullptr, out, M, N, K, st);
  if (M <= 256 && split_ws) {
    const int S = choose_split(M, N, K, split_ws_bytes);
    if (S > 1) {
      const int mt = (M + 127) / 128, nt = (N + 127) / 128;
      DORY_LAUNCH((k_gemm_tile<128, 128, 2, 4, false, false>), dim3(mt * nt, S), dim3(512), 0, st, (const bf16_t*)A,
                  (const bf16_t*)B, (void*)split_ws, M, N, K, 0, mt, nt, K / S);
      const size_t outs = (size_t)M * (dual ? F : N);
      if (dual)
        DORY_LAUNCH(k_splitk_reduce<true>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st,
                    (const float*)split_ws, S, M, N, out);
      else
        DORY_LAUNCH(k_splitk_reduce<false>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st,
                    (const float*)split_ws, S, M, N, out);
      return hipGetLastError();
    }
  }
  return launch_tile_gemm((const bf16_t*)A, (const bf16_t*)B, out, M, N, K, F, dual, st);
}

}  // namespace dory
