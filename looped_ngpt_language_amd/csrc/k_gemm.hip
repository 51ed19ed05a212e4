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
#include <algorithm>

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
// 16x16 per wave, S-stage LDS ring (S = 2 or 3).
// Operand tiles go global -> LDS directly (global_load_lds_dwordx4: 16 bytes
// per lane, lane l of a wave instruction filling bytes 16l..16l+15 of a 1 KB
// block = 8 tile rows of 64 bf16), with no register staging and no LDS store
// instructions: k-tile kt+S-1 is requested right after the barrier that frees
// its stage, so its load overlaps S-1 k-tiles of MFMA work. The load is issued
// from inline assembly and its completion awaited explicitly (s_waitcnt vmcnt
// before each barrier): issued through the compiler's builtin, the load makes
// the compiler wait for every outstanding load before every LDS read, since it
// cannot tell the stages apart. Measured against register staging on the ~4B
// prefill projections: 5-20% faster, bit-identical.
// LDS banks: gfx950 serves a 16-byte-per-lane read to 64 banks of 4 bytes, so
// the 16 rows a pass touches (128 bytes each) must land on 16 distinct
// (row parity, chunk) pairs: the eight 16-byte chunks of row r are XOR-swizzled
// by (r >> 1) & 7 (rows r, r + 1 share the swizzle but sit in opposite bank
// halves), which the LDS conflict counter reads as zero. A lane's load source
// is the logical chunk that lands in its fixed LDS slot.
// The grid is 1-D; workgroup b runs on XCD b % 8, and tiles are dealt so each
// XCD walks a contiguous run of weight-column tiles over all row tiles, which
// keeps every weight tile's re-reads inside one XCD's L2.
// Dual: the tile's B rows are BN/2 gate rows then the BN/2 matching up rows;
// gate tile j pairs with up tile j + TN/2 in the same lanes for the epilogue.
// Split-K: blockIdx.y selects the K range [y * k_len, (y+1) * k_len); with
// gridDim.y > 1 (plain only) the fp32 tile goes to partial slice y of Cv,
// [gridDim.y][M][N], summed afterwards by k_splitk_reduce.
// Byte offsets are 32-bit: the host refuses operands of 4 GiB or more.
DORY_DEV int lds_swz(int r) { return (r >> 1) & 7; }


template <int BM, int BN, int WM, int WN, bool DUAL, int S>
__global__ void __launch_bounds__(64 * WM * WN) k_gemm_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                            void* __restrict__ Cv, int M, int N, int K, int F,
                                                            int m_tiles, int n_tiles, int k_len) {
  constexpr int WAVES = WM * WN, MS = 16;
  constexpr int TM = BM / (MS * WM), TN = BN / (MS * WN);
  constexpr int IA = BM / (8 * WAVES), IB = BN / (8 * WAVES);  // 1 KB loads per wave per k-tile
  // EVEN: every wave loads IA blocks of A and IB of B. Otherwise the (BM + BN) / 8 blocks of a
  // k-tile are dealt round-robin over the waves (NL per wave at most, the last round partial);
  // the per-wave load counts then differ, so only two stages (whose waits are for zero) are allowed.
  constexpr bool EVEN = IA * 8 * WAVES == BM && IB * 8 * WAVES == BN;
  constexpr int NB = (BM + BN) / 8, NL = (NB + WAVES - 1) / WAVES;
  constexpr int PER_TILE = EVEN ? IA + IB : NL;
  static_assert(TM >= 1 && TN >= 1 && BM % 8 == 0 && BN % 8 == 0 && (!DUAL || TN % 2 == 0), "tile shape");
  static_assert(S >= 2 && (S - 2) * PER_TILE <= 63 && (EVEN || S == 2), "stages");
  __shared__ __attribute__((aligned(1024))) bf16_t As[S][BM * MF_BK];
  __shared__ __attribute__((aligned(1024))) bf16_t Bs[S][BN * MF_BK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;

  const int ntiles = m_tiles * n_tiles;
  const int b = blockIdx.x;
  int t = b;
  if ((ntiles & 7) == 0) t = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int tm = t % m_tiles, tn = t / m_tiles;
  const int m0 = tm * BM;
  const int n0 = DUAL ? tn * (BN / 2) : tn * BN;  // first C column (plain) or z column (dual)

  // byte offset of this lane's source (row, logical chunk) for each load: lane l
  // fills physical slot l & 7 of tile row 8i + l/8, i.e. logical chunk (l & 7) ^ swz
  const int lrow = lane >> 3;
  auto a_off = [&](int r) __attribute__((always_inline)) {
    return ((uint32_t)min(m0 + r, M - 1) * (uint32_t)K + ((lane & 7) ^ lds_swz(r)) * 8) * 2;
  };
  auto b_off = [&](int r) __attribute__((always_inline)) {
    int gn;
    if (DUAL) gn = (r < BN / 2) ? min(n0 + r, F - 1) : F + min(n0 + r - BN / 2, F - 1);
    else gn = min(n0 + r, N - 1);
    return ((uint32_t)gn * (uint32_t)K + ((lane & 7) ^ lds_swz(r)) * 8) * 2;
  };
  constexpr int IAE = EVEN ? IA : 1, IBE = EVEN ? IB : 1, NLE = EVEN ? 1 : NL;
  uint32_t offa[IAE], offb[IBE], offl[NLE];
  if constexpr (EVEN) {
#pragma unroll
    for (int i = 0; i < IA; ++i) offa[i] = a_off((wid * IA + i) * 8 + lrow);
#pragma unroll
    for (int i = 0; i < IB; ++i) offb[i] = b_off((wid * IB + i) * 8 + lrow);
  } else {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int blk = min(wid + WAVES * i, NB - 1);  // blocks past NB are never issued
      offl[i] = blk < BM / 8 ? a_off(blk * 8 + lrow) : b_off((blk - BM / 8) * 8 + lrow);
    }
  }
  const bf16_t* const Ak = A + (size_t)blockIdx.y * k_len;
  const bf16_t* const Bk = B + (size_t)blockIdx.y * k_len;
  const uint32_t lds_a = (uint32_t)(size_t)&As[0][0], lds_b = (uint32_t)(size_t)&Bs[0][0];
  auto issue = [&](int kt, int st) __attribute__((always_inline)) {
    const bf16_t* a = Ak + kt * MF_BK;
    const bf16_t* bb = Bk + kt * MF_BK;
    if constexpr (EVEN) {
#pragma unroll
      for (int i = 0; i < IA; ++i) lds_dma16(a, offa[i], lds_a + st * (BM * MF_BK * 2) + (wid * IA + i) * 1024);
#pragma unroll
      for (int i = 0; i < IB; ++i) lds_dma16(bb, offb[i], lds_b + st * (BN * MF_BK * 2) + (wid * IB + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int blk = wid + WAVES * i;  // wave-uniform
        if (blk < BM / 8) lds_dma16(a, offl[i], lds_a + st * (BM * MF_BK * 2) + blk * 1024);
        else if (blk < NB) lds_dma16(bb, offl[i], lds_b + st * (BN * MF_BK * 2) + (blk - BM / 8) * 1024);
      }
    }
  };

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
  // prologue: k-tiles 0 .. S-2 into stages 0 .. S-2; k-tile 0 must land before the barrier
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < nk) issue(p, p);
  if (nk >= S - 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * PER_TILE));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    // stage (st + S - 1) % S was last read in k-tile kt - 1, which every wave has finished
    const bool more = kt + S - 1 < nk;
    if (more) issue(kt + S - 1, st == 0 ? S - 1 : st - 1);
    const bf16_t* as = As[st];
    const bf16_t* bs = Bs[st];
#pragma unroll
    for (int ks = 0; ks < MF_BK / 32; ++ks) {
      const int ch = 4 * ks + kgrp;  // logical 16-byte chunk of this lane's 8 k values
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = arow0 + i * MS;
        af[i] = *reinterpret_cast<const bf16x8_t*>(&as[r * 64 + ((ch ^ lds_swz(r)) << 3)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = brow[j] + (lane & 15);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&bs[r * 64 + ((ch ^ lds_swz(r)) << 3)]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // k-tile kt+1 must have landed before the barrier: only loads issued after it may remain
    if (more) __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * PER_TILE));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    st = st + 1 == S ? 0 : st + 1;
  }

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

template <int BM, int BN, int WM, int WN, int S = 2>
static hipError_t tile_launch(const bf16_t* A, const bf16_t* B, void* out, int M, int N, int K, int F, bool dual,
                              hipStream_t st) {
  const int ncols = dual ? F : N;
  const int cols_per_tile = dual ? BN / 2 : BN;
  const int mt = (M + BM - 1) / BM, nt = (ncols + cols_per_tile - 1) / cols_per_tile;
  const dim3 grid(mt * nt), block(64 * WM * WN);
  if (dual) {
    if constexpr ((BN / (16 * WN)) % 2 == 0)
      DORY_LAUNCH((k_gemm_tile<BM, BN, WM, WN, true, S>), grid, block, 0, st, A, B, out, M, N, K, F, mt, nt, K);
    else
      return hipErrorNotSupported;
  } else {
    DORY_LAUNCH((k_gemm_tile<BM, BN, WM, WN, false, S>), grid, block, 0, st, A, B, out, M, N, K, F, mt, nt, K);
  }
  return hipGetLastError();
}

// Tile shape: the candidate with the least estimated time, taken as the tiles
// of the busiest CU (tiles dealt evenly over 256 CUs) times the tile's area over
// its measured per-CU rate (area per unit time at equal K on the ~4B prefill
// projections: 256x256 on gate/up, 256x192 and 256x160 on qkv, 128x192 on o and
// down, 256x128 and 128x128 on the same shapes; 256x128 over several rounds, where
// its activation re-reads cost most: 2560-token gate/up fetched 1.46 GB per
// launch from beyond L2 against 0.30 GB for 256x256). Shapes that split N into about 256
// tiles (one per CU) avoid the half-empty last round a larger tile leaves.
static hipError_t launch_tile_gemm(const bf16_t* A, const bf16_t* B, void* out, int M, int N, int K, int F, bool dual,
                                   hipStream_t st) {
  const int ncols = dual ? F : N;
  struct Cand { int bm, bn, tn; double rate; };  // tn: MFMA column tiles per wave (dual needs an even count)
  static const Cand cands[] = {{256, 256, 8, 4.0}, {256, 192, 6, 3.69}, {128, 192, 6, 3.15},
                               {256, 128, 4, 3.0}, {128, 128, 4, 2.87}, {256, 160, 5, 3.4}};
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
    case 2: return tile_launch<128, 192, 4, 2, 3>(A, B, out, M, N, K, F, dual, st);
    case 3: return tile_launch<256, 128, 4, 2>(A, B, out, M, N, K, F, dual, st);
    case 5: return tile_launch<256, 160, 4, 2>(A, B, out, M, N, K, F, dual, st);
    default: return tile_launch<128, 128, 2, 2>(A, B, out, M, N, K, F, dual, st);
  }
}

// out: fp32 [M,N] (plain) or storage-type z [M,F] (dual, N = 2F).
// Few rows (3..256): 128x128 tiles leave most CUs idle, so K is split (partials in
// `split_ws`, then a reduce kernel) until the grid has enough workgroups: 256, or from 64
// rows on 128 (at least two splits while the tiles alone are fewer than 256). Each split
// writes and the reduce re-reads an M x N fp32 slice, which at 128 rows of the ~4B
// projections costs more than the wider grid gains: 128 workgroups (with the 4-stage ring
// below) beat 256 on o / qkv / down (14.5 / 18.5 / 21.4 vs 17.5 / 21.6 / 25.9 us), while
// gate/up (128 tiles) needs its 2 splits (31 vs 49 us unsplit). At a few rows the slices are
// small and the wider grid streams the weights faster (5-row speculative verify).
static bool wide_rows(int M) { return M >= 64; }
static int choose_split(int M, int N, int K, size_t split_ws_bytes) {
  const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  const long target = wide_rows(M) ? 128 : 256;
  int S = 1;
  while ((tiles * S < target || (S == 1 && tiles < 256)) && S < 16 && (K / MF_BK) % (2 * S) == 0 &&
         (size_t)(2 * S) * M * N * sizeof(float) <= split_ws_bytes)
    S *= 2;
  return S;
}

hipError_t launch_gemm(int dtype, bool dual, const void* A, const void* B, void* out, int M, int N, int K,
                       float* split_ws, size_t split_ws_bytes, hipStream_t st, int* parts) {
  if (parts) *parts = 0;
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
  // 32-bit byte offsets inside the tile kernels: a weight matrix must stay below 4 GiB; an
  // activation operand that does not (a 262144-token chunk at K = 8192) goes in row blocks
  if ((size_t)N * K * 2 > 0xFFFFFFFFull) return hipErrorNotSupported;
  if ((size_t)M * K * 2 > 0xFFFFFFFFull) {
    const int cap = (int)((0xFFFFFFFFull / ((size_t)K * 2)) / 256 * 256);
    const int nblk = (M + cap - 1) / cap;
    const int mb = ((M + nblk - 1) / nblk + 255) / 256 * 256;  // balanced row blocks
    const size_t ocols = dual ? (size_t)F : (size_t)N;
    const size_t oes = dual ? 2 : 4;  // bf16 z or fp32 out
    for (int m0 = 0; m0 < M; m0 += mb) {
      hipError_t e = launch_gemm(dtype, dual, static_cast<const bf16_t*>(A) + (size_t)m0 * K, B,
                                 static_cast<char*>(out) + (size_t)m0 * ocols * oes, std::min(mb, M - m0), N, K,
                                 split_ws, split_ws_bytes, st, nullptr);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (M <= kGemvMaxRows && gemv_supported(K)) return launch_gemv(dual, A, B, nullptr, out, M, N, K, st);
  if (M >= 64 && M <= 128 && split_ws && (dual || (N <= 4096 && K <= 4096))) {
    // One row tile of 64..128 rows (batched decode): 128 x 64 tiles on 8 waves (two per SIMD, 32 x 32
    // each), a 3-stage ring. gate/up runs unsplit with the SwiGLU epilogue in the tile (no partials,
    // no reduce launch); the smaller plain products split K until the grid would pass 256
    // workgroups. At 128 rows of the ~4B projections, timed after a 1 GB read that empties the
    // memory-side cache, against the 128 x 128 four-wave split-K tiles: gate/up 33.2 vs 34.1 us
    // (with its reduce), o 16.0 vs 17.5 (4 partial slices instead of 8); qkv (22.4 vs 21.2), down
    // (26.2 vs 23.7) and the LM head (228 vs 185) stay on the other tiles.
    if (dual) {
      const int nt = (F + 31) / 32;
      DORY_LAUNCH((k_gemm_tile<128, 64, 4, 2, true, 3>), dim3(nt), dim3(512), 0, st, (const bf16_t*)A,
                  (const bf16_t*)B, out, M, N, K, F, 1, nt, K);
      return hipGetLastError();
    }
    const int nt = (N + 63) / 64;
    int S = 1;
    while (nt * 2 * S <= 256 && (K / MF_BK) % (2 * S) == 0 && (size_t)(2 * S) * M * N * sizeof(float) <= split_ws_bytes)
      S *= 2;
    if (S == 1) {
      DORY_LAUNCH((k_gemm_tile<128, 64, 4, 2, false, 3>), dim3(nt), dim3(512), 0, st, (const bf16_t*)A,
                  (const bf16_t*)B, out, M, N, K, 0, 1, nt, K);
      return hipGetLastError();
    }
    DORY_LAUNCH((k_gemm_tile<128, 64, 4, 2, false, 3>), dim3(nt, S), dim3(512), 0, st, (const bf16_t*)A,
                (const bf16_t*)B, (void*)split_ws, M, N, K, 0, 1, nt, K / S);
    if (parts) {
      *parts = S;
      return hipGetLastError();
    }
    const size_t outs = (size_t)M * N;
    DORY_LAUNCH(k_splitk_reduce<false>, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, st,
                (const float*)split_ws, S, M, N, out);
    return hipGetLastError();
  }
  if (M <= 256 && split_ws) {
    const int S = choose_split(M, N, K, split_ws_bytes);
    if (S > 1) {
      const int mt = (M + 127) / 128, nt = (N + 127) / 128;
      // a long K range (16 k-tiles, or 6 from 64 rows on) streams its weights through a 4-stage
      // ring (3 k-tiles in flight, one workgroup per CU); shorter ranges keep 2 stages, so two
      // workgroups share a CU
      if (K / S / MF_BK >= (wide_rows(M) ? 6 : 16))
        DORY_LAUNCH((k_gemm_tile<128, 128, 2, 4, false, 4>), dim3(mt * nt, S), dim3(512), 0, st, (const bf16_t*)A,
                    (const bf16_t*)B, (void*)split_ws, M, N, K, 0, mt, nt, K / S);
      else
        DORY_LAUNCH((k_gemm_tile<128, 128, 2, 4, false, 2>), dim3(mt * nt, S), dim3(512), 0, st, (const bf16_t*)A,
                    (const bf16_t*)B, (void*)split_ws, M, N, K, 0, mt, nt, K / S);
      if (parts && !dual) {
        *parts = S;
        return hipGetLastError();
      }
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
