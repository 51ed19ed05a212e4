// Weight-streaming GEMV for decode (M <= 8 rows): C[M,N] = X[M,K] . W[N,K]^T
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

// Weights either bf16 [N, K] (MX = 0), MXFP8 [N, K] (MX = 1: OCP Microscaling
// Formats v1.0, FP8 E4M3 element codes, one E8M0 scale 2^(code - 127) per 32
// consecutive elements of a row) or MXFP4 [N, K / 2] (MX = 2: FP4 E2M1 element
// codes, two per byte, element 2i in the low nibble, the same scales); an MX
// element pair is turned into the exact bf16 pair value * scale by
// v_cvt_scalef32_pk_bf16_fp8 / _fp4 and fed to the same v_dot2_f32_bf16 as the
// bf16 path, so MXFP8 halves and MXFP4 quarters the weight bytes.
// A lane chunk holds EPC = 8 (bf16, 16 bytes) or 16 (MXFP8: 16 bytes; MXFP4: 8
// bytes) elements of a row.
//
// MX scales are stored lane-major: lane l's chunk c of a row covers scale block
// j = 32 c + l / 2, and the row's scale bytes are laid out as [32][KCHP] (byte
// p * KCHP + c holds block 32 c + p; KCHP = KCH rounded up to a power of two,
// padding bytes unused), so one load of KCHP bytes brings a lane all the scales
// of its chunks of a row.

DORY_DEV float e8m0_to_f32(uint32_t code) { return __uint_as_float(code ? code << 23 : 0x00400000u); }

template <int KCH> struct MxScaleRow {
  static constexpr int P = KCH <= 1 ? 1 : KCH <= 2 ? 2 : KCH <= 4 ? 4 : 8;  // bytes per lane pair
  static constexpr int WORDS = (P + 3) / 4;
  static constexpr int BYTES = 32 * P;                                         // scale bytes per row
};

int mx_scale_row_bytes(int K) {
  switch (K) {
    case 1024: return MxScaleRow<1>::BYTES;
    case 3072: return MxScaleRow<3>::BYTES;
    case 4096: return MxScaleRow<4>::BYTES;
    case 8192: return MxScaleRow<8>::BYTES;
    default: return 0;
  }
}

// One wave per group of R output rows; lane l reads 16-byte chunks l, l+64, ...
// of each weight row (KCH chunks per lane, K = 64 * EPC * KCH). The small loads
// of the residual prologue (h, y, alpha) are issued before the weight stream, so
// that the prologue's arithmetic and reductions run while the weights arrive
// (loads complete in issue order). Up to 2 input rows live in registers; with
// MR > 2 (3..8 rows: a speculative verify chunk, a few decode rows) the M input
// rows go global -> LDS directly (global_load_lds_dwordx4, no registers), in
// flight together with the weight stream; each 16-byte input chunk read from LDS
// then serves the wave's R rows.
template <int KCH, int R, int MR, bool DUAL, bool RES, int MX>
__global__ void __launch_bounds__(256) k_gemv(const bf16_t* __restrict__ X, const void* __restrict__ Wv,
                                              const uint8_t* __restrict__ Sc, void* __restrict__ Y, int M, int N,
                                              int F, const float* __restrict__ rh, const float* __restrict__ ry,
                                              const float* __restrict__ ralpha, float* __restrict__ hout) {
  constexpr int EPC = MX ? 16 : 8;
  constexpr int K = KCH * 64 * EPC;
  constexpr bool XL = MR > 2;                // input rows staged in LDS (bf16, no residual prologue)
  static_assert(!XL || (!RES && !MX), "3..8 input rows: bf16 weights, no prologue");
  constexpr int RB = MX == 2 ? K / 2 : MX ? K : 2 * K;   // bytes per weight row
  constexpr int CB = MX == 2 ? 8 : 16;                     // bytes per lane chunk
  constexpr int XU = EPC / 8;                // 16-byte x pieces per chunk
  constexpr int EPT = RES ? K / 256 : 1;     // prologue elements per thread
  using SR = MxScaleRow<KCH>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = blockIdx.x * 4 + (tid >> 6);
  const int nrows_out = DUAL ? F : N;
  const int r0 = wave * R;
  const bool active = r0 < nrows_out;
  constexpr int NB = DUAL ? 2 : 1;
  const char* W = static_cast<const char*>(Wv);
  float hv[MR][EPT], yv[MR][EPT], av[EPT];
  if constexpr (RES) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) av[e] = ralpha[tid + 256 * e];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + 256 * e, mm = min(m, M - 1);
        hv[m][e] = rh[(size_t)mm * K + i];
        yv[m][e] = ry[(size_t)mm * K + i];
      }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight stream
  }
  __shared__ __attribute__((aligned(16))) bf16_t xl[XL ? MR * K : 8];
  // Unconditional (the row index is clamped, so idle tail waves re-read the last
  // row): a branch here would make the in-order load counter wait for the weight
  // stream before the prologue.
  u32x4_t wr[NB][R][MX == 2 ? 1 : KCH];
  uint2 wr4[NB][R][MX == 2 ? KCH : 1];
  uint32_t sw[NB][R][SR::WORDS];
  {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = min(r0 + r, nrows_out - 1) + b * F;
        const char* wp = W + (size_t)n * RB + (size_t)lane * CB;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          if constexpr (MX == 2) wr4[b][r][c] = *reinterpret_cast<const uint2*>(wp + c * 64 * CB);
          else wr[b][r][c] = *reinterpret_cast<const u32x4_t*>(wp + c * 64 * CB);
        }
        if constexpr (MX) {
          const uint8_t* sp = Sc + (size_t)n * SR::BYTES + (lane >> 1) * SR::P;
          if constexpr (SR::P == 8) {
            const uint2 v = *reinterpret_cast<const uint2*>(sp);
            sw[b][r][0] = v.x;
            sw[b][r][SR::WORDS - 1] = v.y;
          } else if constexpr (SR::P == 4) {
            sw[b][r][0] = *reinterpret_cast<const uint32_t*>(sp);
          } else if constexpr (SR::P == 2) {
            sw[b][r][0] = *reinterpret_cast<const uint16_t*>(sp);
          } else {
            sw[b][r][0] = *sp;
          }
        }
      }
  }
  if constexpr (XL) {
    // The M input rows, 1 KB per wave instruction, dealt over the 4 waves. Issued from inline
    // assembly with a memory clobber, after the weight loads: the compiler keeps those loads
    // ahead of it, so both streams are in flight together. The wait is for every load the wave
    // issued; the barrier then publishes every wave's share of the rows.
    const int nblk = M * K * 2 / 1024;
    const uint32_t lds0 = (uint32_t)(size_t)&xl[0];
    for (int blk = tid >> 6; blk < nblk; blk += 4) lds_dma16(X, (uint32_t)blk * 1024 + lane * 16, lds0 + blk * 1024);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (!active) return;
    float acc[NB][R][MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float sacc[NB][R];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < R; ++r) sacc[b][r] = 0.f;
      if (m < M) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const uint4 x = *reinterpret_cast<const uint4*>(&xl[m * K + (c * 64 + lane) * 8]);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const u32x4_t w = wr[b][r][c];
              float t = sacc[b][r];
              t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), t, false);
              t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), t, false);
              t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), t, false);
              t = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), t, false);
              sacc[b][r] = t;
            }
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[b][r][m] = wave_sum(sacc[b][r]);
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
    return;
  }
  uint4 xr[XL ? 1 : MR][KCH][XU];
  if constexpr (RES) {
    __shared__ __attribute__((aligned(16))) bf16_t xs[MR][K];
    __shared__ float red[4];
    // rows m >= M (never launched: MR = M) would repeat row M - 1 and store nothing to hout;
    // no branch here, so the loads above stay where they are
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) ss += yv[m][e] * yv[m][e];
      const float iy = rsqrtf(fmaxf(block_sum(ss, red, 4), DORY_TINY_SS));
      float st = 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        hv[m][e] += av[e] * (yv[m][e] * iy - hv[m][e]);
        st += hv[m][e] * hv[m][e];
      }
      const float ih = rsqrtf(fmaxf(block_sum(st, red, 4), DORY_TINY_SS));
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = tid + 256 * e;
        const float v = hv[m][e] * ih;
        xs[m][i] = f32_to_bf16(v);
        if (blockIdx.x == 0 && m < M) hout[(size_t)m * K + i] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int u = 0; u < XU; ++u)
          xr[m][c][u] = m < M ? *reinterpret_cast<const uint4*>(&xs[m][(c * 64 + lane) * EPC + 8 * u])
                              : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int c = 0; c < KCH; ++c)
#pragma unroll
        for (int u = 0; u < XU; ++u)
          xr[m][c][u] = m < M ? *reinterpret_cast<const uint4*>(X + (size_t)m * K + (size_t)(c * 64 + lane) * EPC +
                                                               8 * u)
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
          const u32x4_t w = wr[b][r][MX == 2 ? 0 : c];
          if constexpr (MX == 2) {
            // byte i of the chunk holds elements 2i (low nibble) and 2i + 1; x word k holds
            // elements 2k, 2k + 1
            const float scale = e8m0_to_f32((sw[b][r][c >> 2] >> (8 * (c & 3))) & 0xFFu);
            const uint2 w4 = wr4[b][r][c];
            const uint4 x0 = xr[m][c][0], x1 = xr[m][c][1];
            const uint32_t xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.x, scale, 0);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.x, scale, 1);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.x, scale, 2);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.x, scale, 3);
            const bf16x2_t p4 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.y, scale, 0);
            const bf16x2_t p5 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.y, scale, 1);
            const bf16x2_t p6 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.y, scale, 2);
            const bf16x2_t p7 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w4.y, scale, 3);
            s = __builtin_amdgcn_fdot2_f32_bf16(p0, as_bf16x2(xx[0]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p1, as_bf16x2(xx[1]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p2, as_bf16x2(xx[2]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p3, as_bf16x2(xx[3]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p4, as_bf16x2(xx[4]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p5, as_bf16x2(xx[5]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p6, as_bf16x2(xx[6]), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(p7, as_bf16x2(xx[7]), s, false);
          } else if constexpr (MX) {
            // word j holds elements 4j .. 4j+3; x piece u holds elements 8u .. 8u+7
            const float scale = e8m0_to_f32((sw[b][r][c >> 2] >> (8 * (c & 3))) & 0xFFu);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            const uint4 x0 = xr[m][c][0], x1 = xr[m][c][1];
            const uint32_t xx[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[j], scale, false);
              const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ww[j], scale, true);
              s = __builtin_amdgcn_fdot2_f32_bf16(lo, as_bf16x2(xx[2 * j]), s, false);
              s = __builtin_amdgcn_fdot2_f32_bf16(hi, as_bf16x2(xx[2 * j + 1]), s, false);
            }
          } else {
            const uint4 x = xr[m][c][0];
            s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.x), as_bf16x2(x.x), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.y), as_bf16x2(x.y), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.z), as_bf16x2(x.z), s, false);
            s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.w), as_bf16x2(x.w), s, false);
          }
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

// MXFP8 quantisation (the spec's conversion rule): one thread per 32-element
// block of a bf16 row; X = 2^e, e = floor(log2 max|v|) - 8 clamped to [-127, 127]
// (an all-zero block gets e = -127); each v / X is rounded to E4M3 (round to
// nearest even on its 3-bit mantissa or, below 2^-6, on the 2^-9 subnormal
// step), magnitudes of 448 and above saturate to 448; the sign bit is kept.
// With srb > 0 the scales are written lane-major (row stride srb bytes, see
// above); srb = 0 gives the plain [rows, cols / 32] layout.
// FMT = 2 (MXFP4): e = floor(log2 max|v|) - 2, each v / X rounded to FP4 E2M1 (0, 0.5, 1, 1.5,
// 2, 3, 4, 6; nearest, ties to the even code, above 6 saturating to 6), two codes per byte
// (element 2i in the low nibble), 16 bytes per block.
template <int FMT>
__global__ void __launch_bounds__(256) k_mx_quantize(const bf16_t* __restrict__ src, long long blocks, int nblk,
                                                     int srb, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= blocks) return;
  const uint4* p = reinterpret_cast<const uint4*>(src + b * 32);
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p[i];
    u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
  }
  uint32_t amax_bits = 0;  // |v| of bf16 values compare as integers
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_bits = max(amax_bits, max((u[i] << 16) & 0x7FFFFFFFu, u[i] & 0x7FFF0000u));
  const int ebits = (int)(amax_bits >> 23);
  const int e = max(-127, min(127, (ebits ? ebits - 127 : -200) - (FMT == 2 ? 2 : 8)));
  long long si = b;
  if (srb > 0) {
    const long long n = b / nblk;
    const int j = (int)(b - n * nblk), p = srb / 32;
    si = n * srb + (j & 31) * p + (j >> 5);
  }
  scales[si] = (uint8_t)(e + 127);
  if constexpr (FMT == 2) {
    uint32_t o4[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t bits = (i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16);
      const float q = ldexpf(__uint_as_float(bits & 0x7FFFFFFFu), -e);  // exact: power-of-two scaling
      // midpoints between neighbours: a tie goes to the even code (mantissa bit 0)
      const uint32_t mag = q <= 0.25f ? 0u : q < 0.75f ? 1u : q <= 1.25f ? 2u : q < 1.75f ? 3u
                         : q <= 2.5f ? 4u : q < 3.5f ? 5u : q <= 5.f ? 6u : 7u;
      o4[i >> 3] |= ((bits >> 31) << 3 | mag) << (4 * (i & 7));
    }
    *reinterpret_cast<uint4*>(codes + b * 16) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
    return;
  }
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t bits = (i & 1) ? (u[i >> 1] & 0xFFFF0000u) : (u[i >> 1] << 16);
    const float q = ldexpf(__uint_as_float(bits & 0x7FFFFFFFu), -e);  // exact: power-of-two scaling
    uint32_t mag;
    if (q >= 448.f) {
      mag = 126;
    } else if (q < 0.015625f) {  // below 2^-6: subnormal step 2^-9
      mag = (uint32_t)rintf(q * 512.f);
    } else {
      const int qe = (int)((__float_as_uint(q) >> 23) & 0xFF) - 127;   // -6 .. 8
      const float t = rintf((ldexpf(q, -qe) - 1.f) * 8.f);               // 0 .. 8
      mag = t >= 8.f ? (uint32_t)((qe + 8) << 3) : (uint32_t)((qe + 7) << 3) + (uint32_t)t;
    }
    out[i >> 2] |= ((bits >> 31) << 7 | mag) << (8 * (i & 3));
  }
  uint4* o = reinterpret_cast<uint4*>(codes + b * 32);
  o[0] = make_uint4(out[0], out[1], out[2], out[3]);
  o[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

struct ResArgs {
  const float *h, *y, *alpha;
  float* hout;
};

template <int KCH, bool DUAL, bool RES, int MX>
static hipError_t gemv_k(const bf16_t* X, const void* W, const uint8_t* Sc, void* Y, int M, int N, int F,
                         const ResArgs& ra, hipStream_t st) {
  const int rows_out = DUAL ? F : N;
  // rows per wave: 16-byte weight chunks per lane near 12-16 (registers near 128 VGPRs)
  constexpr int R = MX ? (KCH >= 8 ? 2 : 4) : (KCH >= 16 ? 1 : 2);
  const int waves = (rows_out + R - 1) / R;
  const dim3 grid((waves + 3) / 4);
  if (M == 1)
    DORY_LAUNCH((k_gemv<KCH, R, 1, DUAL, RES, MX>), grid, dim3(256), 0, st, X, W, Sc, Y, M, N, F, ra.h, ra.y,
                ra.alpha, ra.hout);
  else if (M == 2)
    DORY_LAUNCH((k_gemv<KCH, R, 2, DUAL, RES, MX>), grid, dim3(256), 0, st, X, W, Sc, Y, M, N, F, ra.h, ra.y,
                ra.alpha, ra.hout);
  else if constexpr (!RES && !MX) {
    // 3..8 rows, staged in LDS (M rows of K bf16: at most 128 KB); two weight rows per wave, so
    // each staged input chunk serves both
    constexpr int R2 = 2;
    const dim3 grid2((rows_out + 4 * R2 - 1) / (4 * R2));
    if (M <= 4)
      DORY_LAUNCH((k_gemv<KCH, R2, 4, DUAL, false, false>), grid2, dim3(256), 0, st, X, W, Sc, Y, M, N, F, ra.h,
                  ra.y, ra.alpha, ra.hout);
    else if (M == 5)
      DORY_LAUNCH((k_gemv<KCH, R2, 5, DUAL, false, false>), grid2, dim3(256), 0, st, X, W, Sc, Y, M, N, F, ra.h,
                  ra.y, ra.alpha, ra.hout);
    else
      DORY_LAUNCH((k_gemv<KCH, R2, 8, DUAL, false, false>), grid2, dim3(256), 0, st, X, W, Sc, Y, M, N, F, ra.h,
                  ra.y, ra.alpha, ra.hout);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <bool DUAL, bool RES, int MX>
static hipError_t gemv_dispatch(const bf16_t* X, const void* W, const uint8_t* Sc, void* Y, int M, int N, int K,
                                int F, const ResArgs& ra, hipStream_t st) {
  constexpr int D = MX ? 1024 : 512;  // elements per lane chunk column (64 lanes x EPC)
  switch (K) {
    case 1024: return gemv_k<1024 / D, DUAL, RES, MX>(X, W, Sc, Y, M, N, F, ra, st);
    case 3072: return gemv_k<3072 / D, DUAL, RES, MX>(X, W, Sc, Y, M, N, F, ra, st);
    case 4096: return gemv_k<4096 / D, DUAL, RES, MX>(X, W, Sc, Y, M, N, F, ra, st);
    case 8192:
      if constexpr (!RES) return gemv_k<8192 / D, DUAL, false, MX>(X, W, Sc, Y, M, N, F, ra, st);
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

bool gemv_supported(int K) { return K == 1024 || K == 3072 || K == 4096 || K == 8192; }
bool gemv_residual_supported(int K) { return K == 1024 || K == 3072 || K == 4096; }

hipError_t launch_gemv(bool dual, const void* X, const void* W, const uint8_t* scales, void* out, int M, int N, int K,
                       hipStream_t st, int mx_fmt) {
  if (M < 1 || M > (scales ? 2 : kGemvMaxRows) || !gemv_supported(K)) return hipErrorNotSupported;
  const int F = dual ? N / 2 : 0;
  const ResArgs none{nullptr, nullptr, nullptr, nullptr};
  const bf16_t* x = (const bf16_t*)X;
  if (scales && mx_fmt == 2)
    return dual ? gemv_dispatch<true, false, 2>(x, W, scales, out, M, N, K, F, none, st)
                : gemv_dispatch<false, false, 2>(x, W, scales, out, M, N, K, F, none, st);
  if (scales)
    return dual ? gemv_dispatch<true, false, 1>(x, W, scales, out, M, N, K, F, none, st)
                : gemv_dispatch<false, false, 1>(x, W, scales, out, M, N, K, F, none, st);
  return dual ? gemv_dispatch<true, false, 0>(x, W, nullptr, out, M, N, K, F, none, st)
              : gemv_dispatch<false, false, 0>(x, W, nullptr, out, M, N, K, F, none, st);
}

hipError_t launch_gemv_residual(bool dual, const void* W, const uint8_t* scales, void* out, int M, int N, int K,
                                const float* h, const float* y, const float* alpha, float* hout, hipStream_t st,
                                int mx_fmt) {
  if (M < 1 || M > 2 || !gemv_residual_supported(K)) return hipErrorNotSupported;
  const int F = dual ? N / 2 : 0;
  const ResArgs ra{h, y, alpha, hout};
  if (scales && mx_fmt == 2)
    return dual ? gemv_dispatch<true, true, 2>(nullptr, W, scales, out, M, N, K, F, ra, st)
                : gemv_dispatch<false, true, 2>(nullptr, W, scales, out, M, N, K, F, ra, st);
  if (scales)
    return dual ? gemv_dispatch<true, true, 1>(nullptr, W, scales, out, M, N, K, F, ra, st)
                : gemv_dispatch<false, true, 1>(nullptr, W, scales, out, M, N, K, F, ra, st);
  return dual ? gemv_dispatch<true, true, 0>(nullptr, W, nullptr, out, M, N, K, F, ra, st)
              : gemv_dispatch<false, true, 0>(nullptr, W, nullptr, out, M, N, K, F, ra, st);
}

hipError_t launch_mx_quantize(const void* src, long long rows, int cols, void* codes, void* scales, bool lane_major,
                              hipStream_t st, int fmt) {
  if (rows < 0 || cols <= 0 || cols % 32 || (fmt != 1 && fmt != 2)) return hipErrorInvalidValue;
  const int srb = lane_major ? mx_scale_row_bytes(cols) : 0;
  if (lane_major && srb == 0) return hipErrorNotSupported;
  const long long blocks = rows * (cols / 32);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)((blocks + 255) / 256));
  if (fmt == 2)
    DORY_LAUNCH(k_mx_quantize<2>, grid, dim3(256), 0, st, (const bf16_t*)src, blocks, cols / 32, srb, (uint8_t*)codes,
                (uint8_t*)scales);
  else
    DORY_LAUNCH(k_mx_quantize<1>, grid, dim3(256), 0, st, (const bf16_t*)src, blocks, cols / 32, srb, (uint8_t*)codes,
                (uint8_t*)scales);
  return hipGetLastError();
}

}  // namespace dory
