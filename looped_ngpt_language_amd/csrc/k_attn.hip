// Attention sublayer kernels: rotary embedding + per-head L2 norm of q and k with
// the paged KV write, the split-key decode attention (with the rotary/norm/KV
// write of the new token fused in and the split merge done by the last
// workgroup), an MFMA flash-attention kernel for prefill chunks, and a generic
// row kernel for the fp32 model.
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
// KV pool layout: slot-major; a page slot holds 16 tokens of one layer slot,
// keys row-major and values transposed so both attention products load
// contiguous 16-byte operands:
//   K: [H_kv][16 tokens][d_h]     V^T: [H_kv][d_h][16 tokens, order vperm]
// Within a value row, token t sits at vperm(t) = t with bits 2 and 3 swapped
// (0-3, 8-11, 4-7, 12-15): the 8 tokens {4h..4h+3, 8+4h..8+4h+3} that one
// lane's share of a 32x32 score tile covers are then 16 contiguous bytes.
#include "common.h"
#include "kernels.h"

namespace dory {

// Page-table and RoPE-row reads through the index guard (PageGuard, kernels.h): plain reads in
// the default build; bounds-checked, flagged and clamped to index 0 in the DORY_CHECKED build.
DORY_DEV int32_t page_at(const int32_t* __restrict__ tab, int max_pages, int seq, int pi, const PageGuard& gd) {
#if DORY_CHECKED
  if ((uint32_t)seq >= (uint32_t)gd.max_seqs || (uint32_t)pi >= (uint32_t)max_pages) {
    atomicOr(gd.flags, kDevFlagPageIndex);
    return 0;
  }
  const int32_t p = tab[(size_t)seq * max_pages + pi];
  if ((uint32_t)p >= (uint32_t)gd.pool_pages) {
    atomicOr(gd.flags, kDevFlagPageId);
    return 0;
  }
  return p;
#else
  return tab[(size_t)seq * max_pages + pi];
#endif
}
DORY_DEV int rope_row(int pos, const PageGuard& gd) {
#if DORY_CHECKED
  if ((uint32_t)pos >= (uint32_t)gd.max_pos) {
    atomicOr(gd.flags, kDevFlagPosition);
    return 0;
  }
#endif
  return pos;
}

// RoPE of the dimension pair (x1, x2) = (x[i], x[i + dh/2]) with cs = (cos, sin) of the
// position's angle, and the reciprocal L2 norm of the rotated head (summed over the wave). The
// operations are fused in one fixed order, so every kernel that writes a position's k^ (prefill,
// chunk, decode) rounds it to the same bits.
DORY_DEV void rope_pair(float x1, float x2, float2 cs, float& a0, float& a1) {
  a0 = __builtin_fmaf(x1, cs.x, -(x2 * cs.y));
  a1 = __builtin_fmaf(x1, cs.y, x2 * cs.x);
}
DORY_DEV float rope_rnorm(float a0, float a1) {
  return rsqrtf(fmaxf(wave_sum(__builtin_fmaf(a0, a0, a1 * a1)), DORY_TINY_SS));
}

// ---------------------------------------------------------------- rotary + norm + KV write

// One wave per (row, head). Heads 0..H-1 are queries: q^ = N(RoPE(q)) -> q_out.
// Heads H..H+H_kv-1 are keys: k^ = N(RoPE(k)) and v go to the cache page of the
// row's position.
template <typename T>
__global__ void __launch_bounds__(64) k_rope_qk_kv(const float* __restrict__ qkv, const int32_t* __restrict__ rows,
                                                   const int32_t* __restrict__ ptab, int max_pages,
                                                   const float2* __restrict__ rope, T* __restrict__ q_out,
                                                   T* __restrict__ kv_slot, int H, int Hkv, int dh,
                                                   size_t page_elems, const PageGuard gd) {
  const int m = blockIdx.x, hd = blockIdx.y, lane = threadIdx.x;
  const int seq = rows[2 * m], pos = rows[2 * m + 1];
  const int half = dh >> 1;
  const int nq = (H + 2 * Hkv) * dh;
  const float* src = qkv + (size_t)m * nq + (size_t)hd * dh;
  float a0 = 0.f, a1 = 0.f;  // pair (i, i + dh/2) with i = lane (dh <= 128)
  const bool act = lane < half;
  if (act) {
    const float x1 = src[lane], x2 = src[lane + half];
    const float2 cs = rope[(size_t)rope_row(pos, gd) * half + lane];
    rope_pair(x1, x2, cs, a0, a1);
  }
  const float r = rope_rnorm(a0, a1);
  if (hd < H) {
    if (act) {
      T* q = q_out + (size_t)m * H * dh + (size_t)hd * dh;
      St<T>::st(q, lane, a0 * r);
      St<T>::st(q, lane + half, a1 * r);
    }
    return;
  }
  const int g = hd - H, tok = pos & 15;
  const int page = page_at(ptab, max_pages, seq, pos >> 4, gd);
  T* kp = kv_slot + (size_t)page * page_elems + ((size_t)g * 16 + tok) * dh;
  T* vt = kv_slot + (size_t)page * page_elems + (size_t)Hkv * 16 * dh + (size_t)g * dh * 16 + vperm(tok);
  const float* vsrc = src + (size_t)Hkv * dh;
  if (act) {
    St<T>::st(kp, lane, a0 * r);
    St<T>::st(kp, lane + half, a1 * r);
    St<T>::st(vt, (size_t)lane * 16, vsrc[lane]);
    St<T>::st(vt, (size_t)(lane + half) * 16, vsrc[lane + half]);
  }
}

// RoPE + per-head L2 norm + KV write for a chunk of consecutive positions pos0 .. pos0+M-1 of
// one sequence (bf16, d_h = 128), one workgroup per (16-token page, KV head): the G query heads,
// the key head and the value head of the group's rows are processed one wave per (row, head), 16
// waves, so that each wave has few dependent load round trips;
// the page's key block [16][128] and value block V^T [128][16] (token t at column vperm(t)) are
// assembled in LDS and written as whole 4 KB blocks (only the chunk's own rows / columns on the
// partial pages at either end of the chunk, whose other tokens belong to earlier calls).
__global__ void __launch_bounds__(1024) k_rope_page(const float* __restrict__ qkv, int seq, int pos0, int M,
                                                   const int32_t* __restrict__ ptab, int max_pages,
                                                   const float2* __restrict__ rope, bf16_t* __restrict__ q_out,
                                                   bf16_t* __restrict__ kv_slot, int H, int Hkv,
                                                   size_t page_elems, const PageGuard gd) {
  constexpr int DH = 128;
  __shared__ __attribute__((aligned(16))) bf16_t kt[16][DH];
  __shared__ __attribute__((aligned(16))) bf16_t vt[DH][16];
  const int g = blockIdx.y, G = H / Hkv;
  const int pg = pos0 / 16 + blockIdx.x;            // page of the sequence
  const int r0 = pg * 16 - pos0;                     // chunk row of the page's token 0 (may be < 0)
  const int i_lo = max(0, -r0), i_hi = min(16, M - r0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nq = (H + 2 * Hkv) * DH;
  const int units = 16 * (G + 2);
  for (int u = w; u < units; u += 16) {
    const int i = u / (G + 2), hu = u % (G + 2);
    if (i < i_lo || i >= i_hi) continue;
    const int r = r0 + i, pos = pos0 + r;
    const float* src = qkv + (size_t)r * nq;
    if (hu == G + 1) {                               // value: no rotation, no norm
      const float* v = src + (size_t)(H + Hkv + g) * DH;
      vt[lane][vperm(i)] = f32_to_bf16(v[lane]);
      vt[lane + 64][vperm(i)] = f32_to_bf16(v[lane + 64]);
      continue;
    }
    const int head = hu < G ? g * G + hu : H + g;    // query head, or the key head
    const float* x = src + (size_t)head * DH;
    const float x1 = x[lane], x2 = x[lane + 64];
    const float2 cs = rope[(size_t)rope_row(pos, gd) * 64 + lane];
    float a0, a1;
    rope_pair(x1, x2, cs, a0, a1);
    const float rn = rope_rnorm(a0, a1);
    if (hu < G) {
      bf16_t* q = q_out + ((size_t)r * H + head) * DH;
      q[lane] = f32_to_bf16(a0 * rn);
      q[lane + 64] = f32_to_bf16(a1 * rn);
    } else {
      kt[i][lane] = f32_to_bf16(a0 * rn);
      kt[i][lane + 64] = f32_to_bf16(a1 * rn);
    }
  }
  __syncthreads();
  const int page = page_at(ptab, max_pages, seq, pg, gd);
  bf16_t* kp = kv_slot + (size_t)page * page_elems + (size_t)g * 16 * DH;
  bf16_t* vp = kv_slot + (size_t)page * page_elems + (size_t)Hkv * 16 * DH + (size_t)g * DH * 16;
  const int t = threadIdx.x;
  if (i_lo == 0 && i_hi == 16) {                    // whole page: 256 lanes x 16 bytes per block
    if (t < 256) reinterpret_cast<uint4*>(kp)[t] = reinterpret_cast<const uint4*>(&kt[0][0])[t];
    else if (t < 512) reinterpret_cast<uint4*>(vp)[t - 256] = reinterpret_cast<const uint4*>(&vt[0][0])[t - 256];
  } else {
    for (int e = t; e < 16 * DH; e += 1024) {
      const int i = e / DH, d = e % DH;              // key element (token i, dim d)
      if (i >= i_lo && i < i_hi) kp[e] = kt[i][d];
      const int dv = e / 16, c = e % 16;             // value element (dim dv, column c)
      const int iv = vperm(c);                       // vperm is its own inverse
      if (iv >= i_lo && iv < i_hi) vp[e] = vt[dv][c];
    }
  }
}

// ---------------------------------------------------------------- generic row attention

constexpr int ATT_THREADS = 256;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int GMAX = 8;  // query heads per KV head

// Row attention: grid (rows, H_kv, splits). Each workgroup handles the query
// heads of one KV head for one row over one contiguous share of its key range.
// A lane holds 8 consecutive dims; LPK = DH/8 lanes share one key.
template <typename T, int DH>
__global__ void __launch_bounds__(ATT_THREADS) k_attn_rows(
    const T* __restrict__ q, const int32_t* __restrict__ rows, const int32_t* __restrict__ ptab, int max_pages,
    const T* __restrict__ kv_slot, size_t page_elems, int H, int Hkv, int window, float scale, int splits,
    T* __restrict__ out, float* __restrict__ part_ml, float* __restrict__ part_o, const PageGuard gd) {
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
  for (int j = kbeg + wv * KPW + lane / LPK; j < kend; j += ATT_WAVES * KPW) {
    const int page = page_at(ptab, max_pages, seq, j >> 4, gd);
    const T* pg = kv_slot + (size_t)page * page_elems;
    float kf[8], vf[8];
    load8(pg + ((size_t)g * 16 + (j & 15)) * DH + e0, kf);
    const T* vt = pg + (size_t)Hkv * 16 * DH + ((size_t)g * DH + e0) * 16 + vperm(j & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) vf[e] = St<T>::ld(vt, (size_t)e * 16);
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

// Merge split partials: grid rows*H, block max(64, dh) threads; thread e owns
// output dim e. Splits are combined 16 at a time with a running maximum; the 48
// loads of a group (maxima and sums are the same for every thread) are issued
// together, so a merge of <= 16 splits is one memory round trip.
template <typename T>
__global__ void __launch_bounds__(128) k_attn_merge(const float* __restrict__ part_ml,
                                                    const float* __restrict__ part_o, int splits, int dh,
                                                    T* __restrict__ out) {
  const size_t rh = blockIdx.x;
  const int e = threadIdx.x;
  const bool own = e < dh;
  const int lane = e & 63;
  const float* ml = part_ml + 2 * rh * splits;
  const float* po = part_o + rh * splits * dh + (own ? e : 0);
  float M = -INFINITY, L = 0.f, A = 0.f;
  // Splits in groups of 16, each folded in as: running maximum, rescale, weighted sums. All loads
  // of 32 splits are issued together and unconditionally (one memory round trip): each wave takes
  // the (max, sum) pairs with one coalesced load and reads them out with readlane; the partial
  // outputs are loaded at clamped split indexes and the surplus ones dropped by select.
  for (int s0 = 0; s0 < splits; s0 += 32) {
    const int nml = 2 * min(32, splits - s0);
    const float mlv = ml[2 * s0 + min(lane, nml - 1)];  // lanes past the group repeat its last word
    float ov[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) ov[i] = po[(size_t)min(s0 + i, splits - 1) * dh];
    // every value is taken here, so the compiler keeps the second group's loads ahead of the
    // first group's arithmetic instead of moving them under that group's branch
#pragma unroll
    for (int i = 0; i < 32; ++i) asm volatile("" : : "v"(ov[i]));
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (s0 + 16 * g >= splits) break;  // uniform
      float mc = M;
      float mv[16], lv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 16 * g + i;
        const bool ok = s0 + k < splits;
        const float m_k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv), 2 * k));
        const float l_k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mlv), 2 * k + 1));
        mv[i] = ok ? m_k : -INFINITY;
        lv[i] = ok ? l_k : 0.f;
        mc = fmaxf(mc, mv[i]);
      }
      const float c = safe_scale(M, mc);
      A *= c;
      L *= c;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 16 * g + i;
        const float w = safe_scale(mv[i], mc);
        A += w * (s0 + k < splits ? ov[k] : 0.f);
        L += w * lv[i];
      }
      M = mc;
    }
  }
  if (own) St<T>::st(out, rh * dh + e, L > 0.f ? A / L : 0.f);
}

// ---------------------------------------------------------------- bf16 split-key attention, d_h = 128

DORY_DEV float bf16r(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// Operand loads of one 32-key block (pages p0, p0+1) for k_attn_decode: the key
// rows as the A operand of S^T = K . Q^T (lane l: key l%32, dims 16ks + 8(l/32)),
// the value rows as the A operand of O^T = V^T . P^T (page pp, dim tile dt:
// dim 32dt + l%32, tokens vperm 8(l/32) .. +8).
// IT is the wave's block index: its two page ids sit in lane IT % 64 of pid0 / pid1.
#define DORY_DEC_FETCH(KF, VF, IT)                                                                            \
  do {                                                                                                        \
    const int it_ = (IT) & 63;                                                                                \
    const bf16_t* pg0_ = kv_slot + (size_t)__builtin_amdgcn_readlane(pid0, it_) * page_elems;                 \
    const bf16_t* pg1_ = kv_slot + (size_t)__builtin_amdgcn_readlane(pid1, it_) * page_elems;                 \
    const bf16_t* kp_ = (qi < 16 ? pg0_ : pg1_) + ((size_t)g * 16 + (qi & 15)) * DH + 8 * hh;                 \
    _Pragma("unroll") for (int ks = 0; ks < 8; ++ks) KF[ks] = *reinterpret_cast<const bf16x8_t*>(kp_ + 16 * ks); \
    _Pragma("unroll") for (int dt = 0; dt < 4; ++dt) {                                                        \
      const size_t vo_ = vbase + (size_t)(32 * dt + qi) * 16 + 8 * hh;                                        \
      VF[dt] = *reinterpret_cast<const bf16x8_t*>(pg0_ + vo_);                                                \
      VF[4 + dt] = *reinterpret_cast<const bf16x8_t*>(pg1_ + vo_);                                            \
    }                                                                                                         \
  } while (0)

// grid (row groups, H_kv, splits), 256 threads. Each workgroup attends the query heads of KV
// head g for RW rows over a page-aligned share of the rows' keys, on MFMA: the queries are the
// columns of a 32-wide S^T = K . Q^T tile (v_mfma_f32_32x32x16_bf16; unused columns are zero),
// and the tile's probabilities feed O^T = V^T . P^T directly (same scheme as the prefill kernel).
// C is the column capacity: C = G for one row per workgroup (rows of different sequences, or
// one decode row); C = 32 for RW = floor(32 / G) consecutive positions of one sequence per
// workgroup (run.x >= 0: a short prefill chunk, a speculative verify), which then read each key
// once for all their queries, column r * G + gi masking keys past its own row's position.
// Each wave takes 32-key blocks round-robin with the next block's operands in flight. With
// write_kv the splits holding the rows' own positions first write those positions' k^ and v:
// each decode row is the newest token of its sequence, and a chunk written this way has all its
// rows in one workgroup (M <= 32 / G), so every key a workgroup reads that the call writes was
// written by that workgroup (splits never share a page). With splits > 1 each workgroup stores
// a partial (max, sum, unnormalised output) per column and k_attn_merge combines them.
template <int G, int C>
__global__ void __launch_bounds__(256) k_attn_decode(
    const float* __restrict__ qkv, const int32_t* __restrict__ rows, const int32_t* __restrict__ ptab, int max_pages,
    const float2* __restrict__ rope, bf16_t* __restrict__ kv_slot, size_t page_elems, int M, int H, int Hkv,
    int window, float scale, int splits, int write_kv, bf16_t* __restrict__ out, float* __restrict__ part_ml,
    float* __restrict__ part_o, int2 run, const PageGuard gd) {
  constexpr int DH = 128;
  constexpr int RWMAX = C / G;  // rows per workgroup at most
  static_assert(C == G || C == 32, "column capacity");
  __shared__ __attribute__((aligned(16))) bf16_t qs[C][DH];
  __shared__ float wm[4][C], wl[4][C];
  __shared__ float wacc[4][C][DH];
  const int m0 = blockIdx.x * RWMAX, g = blockIdx.y, sp = blockIdx.z;
  const int RW = min(RWMAX, M - m0);  // rows of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31, hh = lane >> 5;
  // run.x >= 0: the rows are the consecutive positions run.y, run.y + 1, ... of sequence run.x
  // (one decode row, or a short prefill chunk), known to the host, so the page-table loads do
  // not wait for a load of the row list
  const int seq = run.x >= 0 ? run.x : rows[2 * m0];
  const int pos_first = run.x >= 0 ? run.y + m0 : rows[2 * m0 + 1];
  const int pos = pos_first + RW - 1;  // the workgroup's last row (C == G: its only row)
  const int lo = window > 0 ? max(0, pos_first - window + 1) : 0;
  const int pf = lo >> 4, pl = pos >> 4;
  // this lane's column: row r_c = qi / G of the group (rows past RW repeat the last one)
  const int pos_c = pos_first + min(qi / G, RW - 1);
  const int lo_c = window > 0 ? max(0, pos_c - window + 1) : 0;
  const int pps = (pl - pf + 1 + splits - 1) / splits;
  const int sp_first = pf + sp * pps;
  const int sp_last = min(pl, sp_first + pps - 1);
  const size_t vbase = (size_t)Hkv * 16 * DH + (size_t)g * DH * 16;
  // with write_kv, the splits holding the rows' own positions write those positions' k^ and v first
  // (one decode row, or the consecutive positions of a short chunk; splits never share a page)
  const bool writer = write_kv && sp_first <= pl && (pos_first >> 4) <= sp_last;
  const int npair = sp_last >= sp_first ? (sp_last - sp_first + 2) / 2 : 0;
  const int nw = npair > wv ? (npair - wv + 3) / 4 : 0;  // blocks of this wave: pairs wv, wv+4, ...
  bf16x8_t kA[8], vA[8], kB[8], vB[8];
  // page ids of the wave's blocks, block it in lane it % 64 (its second page repeats the first
  // past the split's end), read once so the block loop holds no dependent page-table load
  int pid0 = 0, pid1 = 0;
  auto load_pids = [&](int it0) __attribute__((always_inline)) {
    const int itl = it0 + lane;
    if (itl < nw) {
      const int p0 = sp_first + 2 * (wv + 4 * itl);
      pid0 = page_at(ptab, max_pages, seq, p0, gd);
      pid1 = p0 + 1 <= sp_last ? page_at(ptab, max_pages, seq, p0 + 1, gd) : pid0;
    }
  };
  load_pids(0);
  // the first block's operands are requested before the query prologue (the
  // writer split fetches after writing the new key/value)
  if (!writer && nw > 0) DORY_DEC_FETCH(kA, vA, 0);

  // queries of the group: q^ = N(RoPE(q)) in bf16, column r * G + gi
  for (int col = wv; col < RW * G; col += 4) {
    const int r = col / G, gi = col % G;
    const float2 cs = rope[(size_t)rope_row(pos_first + r, gd) * 64 + lane];
    const float* x = qkv + (size_t)(m0 + r) * (size_t)((H + 2 * Hkv) * DH) + (size_t)(g * G + gi) * DH;
    const float x1 = x[lane], x2 = x[lane + 64];
    float a0, a1;
    rope_pair(x1, x2, cs, a0, a1);
    const float rn = rope_rnorm(a0, a1);
    qs[col][lane] = f32_to_bf16(a0 * rn);
    qs[col][lane + 64] = f32_to_bf16(a1 * rn);
  }
  // the writer splits write their rows' keys / values first: one wave per (row, key or value)
  if (writer) {
    for (int t = wv; t < 2 * RW; t += 4) {
      const int r = t >> 1, p = pos_first + r, pg_i = p >> 4;
      if (pg_i < sp_first || pg_i > sp_last) continue;  // another split's page
      const float* src = qkv + (size_t)(m0 + r) * (size_t)((H + 2 * Hkv) * DH);
      bf16_t* pg = kv_slot + (size_t)page_at(ptab, max_pages, seq, pg_i, gd) * page_elems;
      const int tok = p & 15;
      if ((t & 1) == 0) {
        const float2 cs = rope[(size_t)rope_row(p, gd) * 64 + lane];
        const float* x = src + (size_t)(H + g) * DH;
        const float x1 = x[lane], x2 = x[lane + 64];
        float a0, a1;
        rope_pair(x1, x2, cs, a0, a1);
        const float rn = rope_rnorm(a0, a1);
        bf16_t* kp = pg + ((size_t)g * 16 + tok) * DH;
        kp[lane] = f32_to_bf16(a0 * rn);
        kp[lane + 64] = f32_to_bf16(a1 * rn);
      } else {
        const float* v = src + (size_t)(H + Hkv + g) * DH;
        bf16_t* vt = pg + vbase + vperm(tok);
        vt[(size_t)lane * 16] = f32_to_bf16(v[lane]);
        vt[(size_t)(lane + 64) * 16] = f32_to_bf16(v[lane + 64]);
      }
    }
  }
  __syncthreads();

  const int ncol = RW * G;
  bf16x8_t qb[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (qi < ncol) qb[ks] = *reinterpret_cast<const bf16x8_t*>(&qs[qi < ncol ? qi : 0][16 * ks + 8 * hh]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = (__bf16)0.f;
  }
  f32x16_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  if (writer && nw > 0) DORY_DEC_FETCH(kA, vA, 0);
  // block it's operands into KF / VF. Past the last block it re-reads the last one, so every path
  // issues the same loads and the compiler's wait counts stay exact (a skipped prefetch on one
  // path makes it wait for the other path's prefetch too). Page ids are reloaded every 64 blocks,
  // that load awaited at once so that none of it is left in flight.
  auto prefetch = [&](bf16x8_t (&KF)[8], bf16x8_t (&VF)[8], int it) __attribute__((always_inline)) {
    if (it < nw && (it & 63) == 0) {
      load_pids(it);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    DORY_DEC_FETCH(KF, VF, min(it, nw - 1));
  };
  // one 32-key block whose operands are in KB / VB: scores, online softmax, P.V
  auto block = [&](const bf16x8_t (&KB)[8], const bf16x8_t (&VB)[8], int it) __attribute__((always_inline)) {
    const int p0 = sp_first + 2 * (wv + 4 * it);
    f32x16_t st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KB[ks], qb[ks], st, 0, 0, 0);
    float sv[16];
    float mb = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kp = 16 * p0 + 8 * (v >> 2) + 4 * hh + (v & 3);
      const bool ok = kp >= lo_c && kp <= pos_c && (kp >> 4) <= sp_last;
      sv[v] = ok ? st[v] * scale : -INFINITY;
      mb = fmaxf(mb, sv[v]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float mn = fmaxf(mrun, mb);
    const float c = safe_scale(mrun, mn);
    float psum = 0.f;
    bf16x8_t pb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = sv[v] == -INFINITY ? 0.f : __expf(sv[v] - mn);
      psum += p;
      pb[v >> 3][v & 7] = (__bf16)p;
    }
    psum += __shfl_xor(psum, 32, 64);
    lrun = lrun * c + psum;
    mrun = mn;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] *= c;
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VB[dt], pb[0], acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(VB[4 + dt], pb[1], acc[dt], 0, 0, 0);
    }
  };
  // two blocks per trip, so each operand buffer keeps its registers: the next block's loads are
  // in flight while the current one is computed
  for (int it = 0; it < nw; it += 2) {
    prefetch(kB, vB, it + 1);
    block(kA, vA, it);
    if (it + 1 >= nw) break;
    prefetch(kA, vA, it + 2);
    block(kB, vB, it + 1);
  }
  // waves -> LDS: lanes of column qi < ncol hold O[qi][32dt + 8(v/4) + 4hh + v%4]
  if (qi < ncol) {
    if (hh == 0) { wm[wv][qi] = mrun; wl[wv][qi] = lrun; }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) wacc[wv][qi][32 * dt + 8 * (v >> 2) + 4 * hh + (v & 3)] = acc[dt][v];
  }
  __syncthreads();
  for (int idx = tid; idx < ncol * DH; idx += 256) {
    const int col = idx / DH, e = idx % DH;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mx = fmaxf(Mx, wm[w][col]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float cw = safe_scale(wm[w][col], Mx);
      L += wl[w][col] * cw;
      A += wacc[w][col][e] * cw;
    }
    const int m = m0 + col / G, hq = g * G + col % G;
    if (splits == 1) {
      out[((size_t)m * H + hq) * DH + e] = f32_to_bf16(L > 0.f ? A / L : 0.f);
    } else {
      const size_t pi = ((size_t)m * H + hq) * splits + sp;
      part_o[pi * DH + e] = A;
      if (e == 0) { part_ml[2 * pi] = Mx; part_ml[2 * pi + 1] = L; }
    }
  }
}
#undef DORY_DEC_FETCH

// VALU variant, used for many rows (batched decode): its lighter register use keeps
// more waves, hence more pages, in flight per CU. This running-maximum form serves
// attention scales above kFixedMaxScale; k_attn_decode_valu_fx below is the usual one.
// grid (rows, H_kv, splits), 256 threads. Each workgroup attends the G query
// heads of KV head g for one row over a page-aligned share of the row's keys.
// Lane l of a wave reads key (l >> 2) of a page, dims 32*(l & 3) .. +32 for the
// scores and the value rows 2l, 2l+1 (all 16 keys) for the output. With
// write_kv, the split holding the row's own position first writes that
// position's k^ and v (decode: each row is the newest token of its sequence).
// With splits > 1 each workgroup stores a partial (max, sum, unnormalised
// output) and k_attn_merge combines them.
template <int G>
__global__ void __launch_bounds__(256) k_attn_decode_valu(
    const float* __restrict__ qkv, const int32_t* __restrict__ rows, const int32_t* __restrict__ ptab, int max_pages,
    const float2* __restrict__ rope, bf16_t* __restrict__ kv_slot, size_t page_elems, int H, int Hkv, int window,
    float scale, int splits, int write_kv, bf16_t* __restrict__ out, float* __restrict__ part_ml,
    float* __restrict__ part_o, const PageGuard gd) {
  constexpr int DH = 128;
  __shared__ float qs[G][DH];
  __shared__ float knew[DH], vnew[DH];
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wacc[4][G][DH];
  const int m = blockIdx.x, g = blockIdx.y, sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seq = rows[2 * m], pos = rows[2 * m + 1];
  const int lo = window > 0 ? max(0, pos - window + 1) : 0;
  const int nkeys = pos - lo + 1;
  const int chunk = (((nkeys + splits - 1) / splits) + 15) & ~15;
  const int kbeg = lo + sp * chunk;
  const int kend = min(pos + 1, kbeg + chunk);
  const float* src = qkv + (size_t)m * (size_t)((H + 2 * Hkv) * DH);
  const float2 cs = rope[(size_t)rope_row(pos, gd) * 64 + lane];

  // queries of the group: q^ = N(RoPE(q)), rounded to bf16, times the scale
  for (int gi = wv; gi < G; gi += 4) {
    const float* x = src + (size_t)(g * G + gi) * DH;
    const float x1 = x[lane], x2 = x[lane + 64];
    float a0, a1;
    rope_pair(x1, x2, cs, a0, a1);
    const float r = rope_rnorm(a0, a1);
    qs[gi][lane] = bf16r(a0 * r) * scale;
    qs[gi][lane + 64] = bf16r(a1 * r) * scale;
  }
  // The split holding the row's own position writes its key/value and keeps
  // them in LDS: the key loop below takes that key from LDS, not from memory.
  const bool writer = write_kv && kbeg <= pos && pos < kend;
  if (writer && wv < 2) {
    const int page = page_at(ptab, max_pages, seq, pos >> 4, gd);
    bf16_t* pg = kv_slot + (size_t)page * page_elems;
    const int tok = pos & 15;
    if (wv == 0) {
      const float* x = src + (size_t)(H + g) * DH;
      const float x1 = x[lane], x2 = x[lane + 64];
      float a0, a1;
      rope_pair(x1, x2, cs, a0, a1);
      const float r = rope_rnorm(a0, a1);
      const bf16_t k0 = f32_to_bf16(a0 * r), k1 = f32_to_bf16(a1 * r);
      bf16_t* kp = pg + ((size_t)g * 16 + tok) * DH;
      kp[lane] = k0;
      kp[lane + 64] = k1;
      knew[lane] = bf16_to_f32(k0);
      knew[lane + 64] = bf16_to_f32(k1);
    } else {
      const float* v = src + (size_t)(H + Hkv + g) * DH;
      const bf16_t v0 = f32_to_bf16(v[lane]), v1 = f32_to_bf16(v[lane + 64]);
      bf16_t* vt = pg + (size_t)Hkv * 16 * DH + (size_t)g * DH * 16 + vperm(tok);
      vt[(size_t)lane * 16] = v0;
      vt[(size_t)(lane + 64) * 16] = v1;
      vnew[lane] = bf16_to_f32(v0);
      vnew[lane + 64] = bf16_to_f32(v1);
    }
  }
  __syncthreads();

  const int r = lane >> 2, db = lane & 3;
  float qf[G][32];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int i = 0; i < 32; ++i) qf[gi][i] = qs[gi][db * 32 + i];
  float mrun[G], lrun[G], acc[G][2];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) { mrun[gi] = -INFINITY; lrun[gi] = 0.f; acc[gi][0] = acc[gi][1] = 0.f; }

  if (kbeg < kend) {
    const int p_first = (kbeg >> 4) + wv, p_last = (kend - 1) >> 4;
    const int np = p_first <= p_last ? (p_last - p_first) / 4 + 1 : 0;  // pages of this wave
    const size_t vofs = (size_t)Hkv * 16 * DH + (size_t)g * DH * 16 + (size_t)lane * 32;
    const size_t kofs = ((size_t)g * 16 + r) * DH + db * 32;
    // page ids of this wave's pages, 64 at a time, one per lane
    int pid = lane < np ? page_at(ptab, max_pages, seq, p_first + 4 * lane, gd) : 0;
    uint4 kr[4], vr[4];
    auto fetch = [&](int it) {
      const int page = __shfl(pid, it & 63, 64);
      const bf16_t* pg = kv_slot + (size_t)page * page_elems;
      const uint4* kp = reinterpret_cast<const uint4*>(pg + kofs);
      const uint4* vp = reinterpret_cast<const uint4*>(pg + vofs);
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = vp[i];
    };
    if (np > 0) fetch(0);
    for (int it = 0; it < np; ++it) {
      const int p = p_first + 4 * it;
      float kf[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w4[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kf[8 * i + 2 * j] = __uint_as_float(w4[j] << 16);
          kf[8 * i + 2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
        }
      }
      // value rows 2*lane (vr[0..1]) and 2*lane+1 (vr[2..3]), 16 keys each in vperm order
      float v0[16], v1[16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t a4[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        const uint32_t b4[4] = {vr[i + 2].x, vr[i + 2].y, vr[i + 2].z, vr[i + 2].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v0[8 * i + 2 * j] = __uint_as_float(a4[j] << 16);
          v0[8 * i + 2 * j + 1] = __uint_as_float(a4[j] & 0xFFFF0000u);
          v1[8 * i + 2 * j] = __uint_as_float(b4[j] << 16);
          v1[8 * i + 2 * j + 1] = __uint_as_float(b4[j] & 0xFFFF0000u);
        }
      }
      // next page's loads are in flight while this page is computed
      if (it + 1 < np) {
        if (((it + 1) & 63) == 0)
          pid = lane + it + 1 < np ? page_at(ptab, max_pages, seq, p_first + 4 * (it + 1 + lane), gd) : 0;
        fetch(it + 1);
      }
      const int key = p * 16 + r;
      const bool valid = key >= kbeg && key < kend;
      if (writer && p == (pos >> 4)) {
        const int tok = pos & 15;
        if (r == tok) {
#pragma unroll
          for (int i = 0; i < 32; ++i) kf[i] = knew[db * 32 + i];
        }
        const float n0 = vnew[2 * lane], n1 = vnew[2 * lane + 1];
        const int ptok = vperm(tok);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          v0[kk] = kk == ptok ? n0 : v0[kk];
          v1[kk] = kk == ptok ? n1 : v1[kk];
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) s += qf[gi][i] * kf[i];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s = valid ? s : -INFINITY;
        float mp = s;
        mp = fmaxf(mp, __shfl_xor(mp, 4, 64));
        mp = fmaxf(mp, __shfl_xor(mp, 8, 64));
        mp = fmaxf(mp, __shfl_xor(mp, 16, 64));
        mp = fmaxf(mp, __shfl_xor(mp, 32, 64));
        const float mn = fmaxf(mrun[gi], mp);
        const float c = safe_scale(mrun[gi], mn);
        const float pr = valid ? __expf(s - mn) : 0.f;
        float ps = db == 0 ? pr : 0.f;
        ps += __shfl_xor(ps, 4, 64);
        ps += __shfl_xor(ps, 8, 64);
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        lrun[gi] = lrun[gi] * c + ps;
        float a0 = acc[gi][0] * c, a1 = acc[gi][1] * c;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {  // v0/v1[kk] hold token vperm(kk)
          const float pk = __shfl(pr, 4 * vperm(kk), 64);
          a0 += pk * v0[kk];
          a1 += pk * v1[kk];
        }
        acc[gi][0] = a0;
        acc[gi][1] = a1;
        mrun[gi] = mn;
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    if (lane == 0) { wm[wv][gi] = mrun[gi]; wl[wv][gi] = lrun[gi]; }
    wacc[wv][gi][2 * lane] = acc[gi][0];
    wacc[wv][gi][2 * lane + 1] = acc[gi][1];
  }
  __syncthreads();
  for (int idx = tid; idx < G * DH; idx += 256) {
    const int gi = idx / DH, e = idx % DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][gi]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float c = safe_scale(wm[w][gi], M);
      L += wl[w][gi] * c;
      A += wacc[w][gi][e] * c;
    }
    const int hq = g * G + gi;
    if (splits == 1) {
      out[((size_t)m * H + hq) * DH + e] = f32_to_bf16(L > 0.f ? A / L : 0.f);
    } else {
      const size_t pi = ((size_t)m * H + hq) * splits + sp;
      part_o[pi * DH + e] = A;
      if (e == 0) { part_ml[2 * pi] = M; part_ml[2 * pi + 1] = L; }
    }
  }
}

// Fixed-offset form of the VALU kernel (attention scale <= kFixedMaxScale): q^ and k^ are unit
// vectors, so the probabilities are exp(scale (q^.k^ - 1)) with no running maximum, no rescaling
// and a lane-local row sum. Scores are packed-bf16 dot products (v_dot2_f32_bf16) of the query
// with the key words as loaded; each page's 16 probabilities are written to LDS once by the
// lanes that hold them and read back by every lane, rounded to bf16 in pairs (as the MFMA
// kernels feed P) and dotted with the packed value words. Partials carry max = scale, so the
// wave combine and k_attn_merge apply.
template <int G>
__global__ void __launch_bounds__(256) k_attn_decode_valu_fx(
    const float* __restrict__ qkv, const int32_t* __restrict__ rows, const int32_t* __restrict__ ptab, int max_pages,
    const float2* __restrict__ rope, bf16_t* __restrict__ kv_slot, size_t page_elems, int H, int Hkv, int window,
    float scale, int splits, int write_kv, bf16_t* __restrict__ out, float* __restrict__ part_ml,
    float* __restrict__ part_o, const int32_t* __restrict__ order, const PageGuard gd) {
  constexpr int DH = 128;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __attribute__((aligned(16))) bf16_t qh[G][DH];
  __shared__ __attribute__((aligned(16))) bf16_t knew[DH];
  __shared__ __attribute__((aligned(16))) bf16_t vnew[DH];
  __shared__ float wm[4][G], wl[4][G];
  __shared__ float wacc[4][G][DH];
  __shared__ __attribute__((aligned(16))) float pbuf[4][G][16];  // per wave: one page's probabilities
  const int m = order ? order[blockIdx.x] : (int)blockIdx.x, g = blockIdx.y, sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = rows[2 * m], pos = rows[2 * m + 1];
  const int lo = window > 0 ? max(0, pos - window + 1) : 0;
  const int nkeys = pos - lo + 1;
  const int chunk = (((nkeys + splits - 1) / splits) + 15) & ~15;
  const int kbeg = lo + sp * chunk;
  const int kend = min(pos + 1, kbeg + chunk);
  const float* src = qkv + (size_t)m * (size_t)((H + 2 * Hkv) * DH);
  const float2 cs = rope[(size_t)rope_row(pos, gd) * 64 + lane];

  // queries of the group: q^ = N(RoPE(q)) in bf16
  for (int gi = wv; gi < G; gi += 4) {
    const float* x = src + (size_t)(g * G + gi) * DH;
    const float x1 = x[lane], x2 = x[lane + 64];
    float a0, a1;
    rope_pair(x1, x2, cs, a0, a1);
    const float r = rope_rnorm(a0, a1);
    qh[gi][lane] = f32_to_bf16(a0 * r);
    qh[gi][lane + 64] = f32_to_bf16(a1 * r);
  }
  // the split holding the row's own position writes its key/value and keeps them in LDS: the
  // key loop takes that key and value from LDS, not from memory
  const bool writer = write_kv && kbeg <= pos && pos < kend;
  const int tok = pos & 15;
  if (writer && wv < 2) {
    const int page = page_at(ptab, max_pages, seq, pos >> 4, gd);
    bf16_t* pg = kv_slot + (size_t)page * page_elems;
    if (wv == 0) {
      const float* x = src + (size_t)(H + g) * DH;
      const float x1 = x[lane], x2 = x[lane + 64];
      float a0, a1;
      rope_pair(x1, x2, cs, a0, a1);
      const float r = rope_rnorm(a0, a1);
      const bf16_t k0 = f32_to_bf16(a0 * r), k1 = f32_to_bf16(a1 * r);
      bf16_t* kp = pg + ((size_t)g * 16 + tok) * DH;
      kp[lane] = k0;
      kp[lane + 64] = k1;
      knew[lane] = k0;
      knew[lane + 64] = k1;
    } else {
      const float* v = src + (size_t)(H + Hkv + g) * DH;
      const bf16_t v0 = f32_to_bf16(v[lane]), v1 = f32_to_bf16(v[lane + 64]);
      bf16_t* vt = pg + (size_t)Hkv * 16 * DH + (size_t)g * DH * 16 + vperm(tok);
      vt[(size_t)lane * 16] = v0;
      vt[(size_t)(lane + 64) * 16] = v1;
      vnew[lane] = v0;
      vnew[lane + 64] = v1;
    }
  }
  __syncthreads();

  // lane l: key r = l / 4 of a page, dims 32 db .. +32 (db = l % 4) for the scores; value rows
  // 2l and 2l + 1 (all 16 keys of the page, vperm order) for the output
  const int r = lane >> 2, db = lane & 3;
  uint32_t qw[G][16];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int i = 0; i < 16; ++i) qw[gi][i] = *reinterpret_cast<const uint32_t*>(&qh[gi][db * 32 + 2 * i]);
  const float k2 = scale * LOG2E;
  float lrun[G], acc[G][2];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) { lrun[gi] = 0.f; acc[gi][0] = acc[gi][1] = 0.f; }

  if (kbeg < kend) {
    const int p_first = (kbeg >> 4) + wv, p_last = (kend - 1) >> 4;
    const int np = p_first <= p_last ? (p_last - p_first) / 4 + 1 : 0;  // pages of this wave
    const size_t vofs = (size_t)Hkv * 16 * DH + (size_t)g * DH * 16 + (size_t)lane * 32;
    const size_t kofs = ((size_t)g * 16 + r) * DH + db * 32;
    // page ids of this wave's pages, 64 at a time, one per lane
    int pid = lane < np ? page_at(ptab, max_pages, seq, p_first + 4 * lane, gd) : 0;
    uint4 kr[4], vr[4];
    auto fetch = [&](int it) __attribute__((always_inline)) {
      const int page = __builtin_amdgcn_readlane(pid, it & 63);
      const bf16_t* pg = kv_slot + (size_t)page * page_elems;
      const uint4* kp = reinterpret_cast<const uint4*>(pg + kofs);
      const uint4* vp = reinterpret_cast<const uint4*>(pg + vofs);
#pragma unroll
      for (int i = 0; i < 4; ++i) kr[i] = kp[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = vp[i];
    };
    if (np > 0) fetch(0);
    for (int it = 0; it < np; ++it) {
      const int p = p_first + 4 * it;
      uint32_t kw[16], v0w[8], v1w[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kw[4 * i] = kr[i].x; kw[4 * i + 1] = kr[i].y; kw[4 * i + 2] = kr[i].z; kw[4 * i + 3] = kr[i].w;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v0w[4 * i] = vr[i].x; v0w[4 * i + 1] = vr[i].y; v0w[4 * i + 2] = vr[i].z; v0w[4 * i + 3] = vr[i].w;
        v1w[4 * i] = vr[i + 2].x; v1w[4 * i + 1] = vr[i + 2].y; v1w[4 * i + 2] = vr[i + 2].z;
        v1w[4 * i + 3] = vr[i + 2].w;
      }
      // next page's loads are in flight while this page is computed
      if (it + 1 < np) {
        if (((it + 1) & 63) == 0)
          pid = lane + it + 1 < np ? page_at(ptab, max_pages, seq, p_first + 4 * (it + 1 + lane), gd) : 0;
        fetch(it + 1);
      }
      const int key = p * 16 + r;
      const bool valid = key >= kbeg && key < kend;
      if (writer && p == (pos >> 4)) {
        if (r == tok) {
#pragma unroll
          for (int i = 0; i < 16; ++i) kw[i] = *reinterpret_cast<const uint32_t*>(&knew[db * 32 + 2 * i]);
        }
        // value words: token tok sits at vperm position vperm(tok), half (vperm(tok) & 1) of word vperm(tok) / 2
        const int ptok = vperm(tok), sh = 16 * (ptok & 1);
        const uint32_t n0 = (uint32_t)vnew[2 * lane] << sh, n1 = (uint32_t)vnew[2 * lane + 1] << sh;
        const uint32_t keep = sh ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          if (w == (ptok >> 1)) {
            v0w[w] = (v0w[w] & keep) | n0;
            v1w[w] = (v1w[w] & keep) | n1;
          }
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw[gi][i]), as_bf16x2(kw[i]), s, false);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        const float pr = valid ? __builtin_amdgcn_exp2f(s * k2 - k2) : 0.f;
        if (db == 0) {
          lrun[gi] += pr;
          pbuf[wv][gi][r] = pr;  // the page's 16 probabilities, by token; read back by every lane
        }
        // One wave's LDS operations complete in issue order, so no s_barrier is needed; the
        // wavefront-scope fence and wave barrier keep the compiler from moving the reads below
        // above these writes, or the next page's writes above these reads.
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float pv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 q4 = *reinterpret_cast<const float4*>(&pbuf[wv][gi][4 * i]);
          pv[4 * i] = q4.x; pv[4 * i + 1] = q4.y; pv[4 * i + 2] = q4.z; pv[4 * i + 3] = q4.w;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float a0 = acc[gi][0], a1 = acc[gi][1];
#pragma unroll
        for (int w = 0; w < 8; ++w) {  // value word w holds the tokens vperm(2w), vperm(2w + 1)
          const bf16x2_t pw = {(__bf16)pv[vperm(2 * w)], (__bf16)pv[vperm(2 * w + 1)]};
          a0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v0w[w]), pw, a0, false);
          a1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(v1w[w]), pw, a1, false);
        }
        acc[gi][0] = a0;
        acc[gi][1] = a1;
      }
    }
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const float l = wave_sum(lrun[gi]);
    if (lane == 0) { wm[wv][gi] = scale; wl[wv][gi] = l; }
    wacc[wv][gi][2 * lane] = acc[gi][0];
    wacc[wv][gi][2 * lane + 1] = acc[gi][1];
  }
  __syncthreads();
  for (int idx = tid; idx < G * DH; idx += 256) {
    const int gi = idx / DH, e = idx % DH;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      L += wl[w][gi];
      A += wacc[w][gi][e];
    }
    const int hq = g * G + gi;
    if (splits == 1) {
      out[((size_t)m * H + hq) * DH + e] = f32_to_bf16(L > 0.f ? A / L : 0.f);
    } else {
      const size_t pi = ((size_t)m * H + hq) * splits + sp;
      part_o[pi * DH + e] = A;
      if (e == 0) { part_ml[2 * pi] = scale; part_ml[2 * pi + 1] = L; }
    }
  }
}

// ---------------------------------------------------------------- bf16 flash attention for prefill, d_h = 128

// grid (H, R) for R 128-query row blocks of one sequence (a prefill chunk); workgroup (h, y)
// handles row block R-1-y of head h, wave w owning queries 32 (w % 4) .. +32 of the block. Causal row
// block i reads i + 1 key ranges' worth of keys: with the head fastest in the dispatch order, the
// whole grid runs longest first (every head's last row block, then every head's second last, ...),
// so the short blocks dispatched last fill the CUs that the long ones left free. Keys go through LDS in
// blocks of 64 (4 pages), shared by the four waves of a key group and double-buffered: the next
// step's blocks go global -> LDS directly (no registers) into the idle buffer while the current
// ones are used, each wave's page id read one step ahead. Scores are computed transposed with
// v_mfma_f32_32x32x16_bf16, S^T = K . Q^T: lane l holds, for query l%32, the
// keys 8j + 4(l/32) + i (v = 4j + i) of a 32-key half-block; its
// probabilities for one page (j = 0,1 or 2,3) form the P^T operand of
// O^T = V^T . P^T as they are, and the matching value operand is the
// contiguous 16 bytes at vperm position 8(l/32) of each value row.
// LDS: K [64 keys][16 chunks of 8 dims], chunk c of key k stored at c ^ (k & 15);
// V^T [4 pages][128 dims][2 halves], half h of dim d stored at h ^ ((d >> 3) & 1).
// gfx950 serves a 16-byte-per-lane LDS read to 64 banks, 16 lanes at a time: the
// 16 consecutive keys (256-byte rows) or dims (32-byte rows) such a group reads
// then fall on 16 distinct 16-byte bank groups.
// FIXED: q^ and k^ are unit vectors, so a scaled score never exceeds `scale`
// (up to bf16 rounding); the probabilities are exp(s - scale) with no running
// maximum and no rescaling of the accumulators (softmax is invariant to the
// offset; for scale <= kFixedMaxScale nothing underflows to zero).
// Largest attention scale whose fixed-offset probabilities stay normal fp32
// numbers: exp(-2 * 40) ~ 1.8e-35 > 1.2e-38.
constexpr float kFixedMaxScale = 40.f;

constexpr int PF_KB = 64;  // keys per LDS block of the prefill kernel

// One 128-query row block (rows wrow0 ..) of query head hq. KSPLIT = 2: the workgroup has 8
// waves; waves 4g .. 4g+3 (key group g) take the 64-key blocks 2s + g of each
// 128-key step for their 32 queries each, and the two groups' partial sums are
// merged through LDS at the end (two waves per SIMD, half the serial key loop).
template <bool FIXED, int KSPLIT>
DORY_DEV void attn_row_block(const bf16_t* __restrict__ q, const int32_t* __restrict__ rows,
                             const int32_t* __restrict__ ptab, int max_pages, const bf16_t* __restrict__ kv_slot,
                             size_t page_elems, int M, int H, int Hkv, int window, float scale,
                             bf16_t* __restrict__ out, int wrow0, int hq, bf16_t (*Ks)[KSPLIT][PF_KB * 128],
                             bf16_t (*Vs)[KSPLIT][PF_KB * 128], const PageGuard& gd) {
  constexpr int DH = 128, KB = PF_KB, STEP = KB * KSPLIT;
  constexpr float LOG2E = 1.4426950408889634f;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq = wv & 3, kg = wv >> 2;             // query group, key group (wave-uniform)
  const int g = hq / (H / Hkv);
  const int row0 = wrow0 + wq * 32;
  const int nrow = max(0, min(32, M - row0));
  const int seq = rows[0];
  const int qi = lane & 31, hh = lane >> 5;
  const int my_row = nrow > 0 ? row0 + min(qi, nrow - 1) : wrow0;
  const int qpos = rows[2 * my_row + 1];
  const int wg_first = rows[2 * wrow0 + 1];
  const int wg_last = rows[2 * (min(wrow0 + 127, M - 1)) + 1];
  const int pos_first = nrow > 0 ? rows[2 * row0 + 1] : 0;
  const int pos_last = nrow > 0 ? rows[2 * (row0 + nrow - 1) + 1] : -1;
  const int last_page = wg_last >> 4;

  // Q as the B operand of S^T: lane holds Q[query qi][dims 16ks + 8hh .. +8]
  bf16x8_t qb[8];
  const bf16_t* qrow = q + ((size_t)my_row * H + hq) * DH;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + ks * 16 + hh * 8);

  f32x16_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;
  float mrun = FIXED ? scale : -INFINITY, lrun = 0.f;
  // score -> exp2 argument: s * scale * log2(e) - offset * log2(e)
  const float k2 = scale * LOG2E;
  // this lane's LDS element offsets: K row qi (+ 32 t rows), chunk 2 ks + hh swizzled by the key;
  // V^T row qi (+ page and dim-tile rows), half hh swizzled by the dim
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = qi * DH + (((2 * ks + hh) ^ (qi & 15)) << 3);
  const int voff = qi * 16 + ((hh ^ ((qi >> 3) & 1)) << 3);

  // this wave's share of its key group's 64-key block: the 4 KB K block and the 4 KB V^T block
  // of page wq (four 1 KB pieces each), loaded straight into LDS, 16 bytes per lane, lane l
  // filling bytes 16 l of a piece; the source is the chunk that belongs in that LDS slot
  const int wqu = wq, kgu = kg;
  uint32_t kofs[4], vofs[4];  // byte offsets within a page
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int key = qt * 4 + (lane >> 4), dim = qt * 32 + (lane >> 1);
    kofs[qt] = (uint32_t)((((size_t)g * 16 + key) * DH + (((lane & 15) ^ (key & 15)) << 3)) * 2);
    vofs[qt] = (uint32_t)(((size_t)Hkv * 16 * DH + ((size_t)g * DH + dim) * 16 + (((lane & 1) ^ ((dim >> 3) & 1)) << 3)) * 2);
  }
  const uint32_t lds_k = (uint32_t)(size_t)&Ks[0][kgu][wqu * 16 * DH];
  const uint32_t lds_v = (uint32_t)(size_t)&Vs[0][kgu][wqu * DH * 16];
  constexpr uint32_t kStageBytes = KSPLIT * PF_KB * 128 * 2;
  auto page_of = [&](int step0) __attribute__((always_inline)) {
    return page_at(ptab, max_pages, seq, min(((step0 + kgu * KB) >> 4) + wqu, last_page), gd);
  };
  auto kv_dma = [&](int pid, int st_) __attribute__((always_inline)) {
    const bf16_t* pg = kv_slot + (size_t)pid * page_elems;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      lds_dma16(pg, kofs[qt], lds_k + st_ * kStageBytes + qt * 4 * DH * 2);
      lds_dma16(pg, vofs[qt], lds_v + st_ * kStageBytes + qt * 32 * 16 * 2);
    }
  };

  const int klo = window > 0 ? max(0, wg_first - window + 1) : 0;
  const int wlo = window > 0 ? max(0, pos_first - window + 1) : 0;
  const int kstart = klo & ~(KB - 1);
  kv_dma(page_of(kstart), 0);
  int pid_next = page_of(kstart + STEP);  // the next step's page, read a step ahead
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  // the query operands are consumed here, before the loop: the compiler otherwise issues their
  // loads after the barrier and waits for them inside the loop body, where (the key loads being
  // inline assembly it does not count) those waits stall on the next step's key loads instead
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qb[ks]));
  int stage = 0;
  for (int kstep = kstart; kstep <= wg_last; kstep += STEP, stage ^= 1) {
    // the other stage was last read before the barrier that ended the previous step
    if (kstep + STEP <= wg_last) {
      kv_dma(pid_next, stage ^ 1);
      pid_next = page_of(kstep + 2 * STEP);
    }
    const int kb = kstep + kg * KB;              // this key group's 64-key block
    if constexpr (FIXED) {
      // one code path for every block the wave sees: both 32-key halves' scores, the masked
      // scores of an edge half set to -inf (exp2 -> 0), then exponentials and P.V, so the
      // accumulators have a single update site in the loop (no register copies between paths)
      if (nrow > 0 && kb <= pos_last && kb + KB > wlo) {
        const bf16_t* ks_ = Ks[stage][kg];
        const bf16_t* vs_ = Vs[stage][kg];
        f32x16_t st2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) st2[t][v] = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int ks = 0; ks < 8; ++ks)
            st2[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                *reinterpret_cast<const bf16x8_t*>(ks_ + 32 * t * DH + koff[ks]), qb[ks], st2[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int k0 = kb + 32 * t;
          // keys of this half-block that some query of the wave must not see (wave-uniform)
          const bool edge = k0 + 31 > pos_first || (window > 0 && k0 <= pos_last - window);
          if (edge) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int kp = k0 + 8 * (v >> 2) + 4 * hh + (v & 3);
              const bool ok = kp <= qpos && (window <= 0 || kp > qpos - window);
              st2[t][v] = ok ? st2[t][v] : -INFINITY;
            }
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8_t pb[2];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(st2[t][v] * k2 - k2);
            lrun += p;
            pb[v >> 3][v & 7] = (__bf16)p;
          }
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              const bf16x8_t va =
                  *reinterpret_cast<const bf16x8_t*>(vs_ + ((2 * t + pp) * DH + dt * 32) * 16 + voff);
              acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[pp], acc[dt], 0, 0, 0);
            }
        }
      }
    } else if (nrow > 0 && kb <= pos_last && kb + KB > wlo) {
      // running maximum: each visible 32-key half rescales the row sums and accumulators
      const bf16_t* ks_ = Ks[stage][kg];
      const bf16_t* vs_ = Vs[stage][kg];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k0 = kb + 32 * t;
        if (k0 > pos_last || k0 + 32 <= wlo) continue;
        f32x16_t st;
#pragma unroll
        for (int v = 0; v < 16; ++v) st[v] = 0.f;
        // A operand row: key 32 t + qi of the block
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(ks_ + 32 * t * DH + koff[ks]);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ks], st, 0, 0, 0);
        }
        // keys of this half-block that some query of the wave must not see (wave-uniform)
        const bool edge = k0 + 31 > pos_first || (window > 0 && k0 <= pos_last - window);
        bf16x8_t pb[2];
        float sv[16];
        float mb = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kp = k0 + 8 * (v >> 2) + 4 * hh + (v & 3);
          const bool ok = !edge || (kp <= qpos && (window <= 0 || kp > qpos - window));
          sv[v] = ok ? st[v] : -INFINITY;
          mb = fmaxf(mb, sv[v]);
        }
        mb = fmaxf(mb * scale, __shfl_xor(mb * scale, 32, 64));
        const float mn = fmaxf(mrun, mb);
        const float c = safe_scale(mrun, mn);
        mrun = mn;
        const float off = mrun * LOG2E;
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = sv[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[v] * k2 - off);
          psum += p;
          pb[v >> 3][v & 7] = (__bf16)p;
        }
        psum += __shfl_xor(psum, 32, 64);
        lrun = lrun * c + psum;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] *= c;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int page = 2 * t + pp;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vs_ + (page * DH + dt * 32) * 16 + voff);
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[pp], acc[dt], 0, 0, 0);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the next block has landed before the barrier publishes it
    __syncthreads();
  }
  if (FIXED) lrun += __shfl_xor(lrun, 32, 64);  // the two halves of a query's keys
  if constexpr (KSPLIT == 2) {
    // key group 1 hands (max, sum, output) to key group 0 through the (now idle) LDS:
    // the 64 output floats per lane fill the K buffers exactly (4 waves x 64 lanes,
    // lane-contiguous), max and sum go to the V buffers
    float* xs = reinterpret_cast<float*>(&Ks[0][0][0]) + (size_t)wq * 64 * 64 + lane;
    float* xm = reinterpret_cast<float*>(&Vs[0][0][0]) + (size_t)wq * 2 * 64 + lane;
    static_assert(sizeof(Ks[0]) * 2 >= 4 * 64 * 64 * sizeof(float), "merge buffer");
    if (kg == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) xs[(dt * 16 + v) * 64] = acc[dt][v];
      xm[0] = mrun;
      xm[64] = lrun;
    }
    __syncthreads();
    if (kg == 1) return;
    const float m1 = xm[0], l1 = xm[64];
    const float mn = fmaxf(mrun, m1);
    const float c0 = FIXED ? 1.f : safe_scale(mrun, mn), c1 = FIXED ? 1.f : safe_scale(m1, mn);
    lrun = lrun * c0 + l1 * c1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = acc[dt][v] * c0 + xs[(dt * 16 + v) * 64] * c1;
  }
  if (qi >= nrow) return;
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
  bf16_t* orow = out + ((size_t)(row0 + qi) * H + hq) * DH;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = dt * 32 + 8 * j + 4 * hh;
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[dt][4 * j] * inv) | ((uint32_t)f32_to_bf16(acc[dt][4 * j + 1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[dt][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16(acc[dt][4 * j + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + d0) = make_uint2(lo, hi);
    }
}

template <bool FIXED, int KSPLIT>
__global__ void __launch_bounds__(256 * KSPLIT) k_attn_prefill(const bf16_t* __restrict__ q,
                                                               const int32_t* __restrict__ rows,
                                                               const int32_t* __restrict__ ptab, int max_pages,
                                                               const bf16_t* __restrict__ kv_slot, size_t page_elems,
                                                               int M, int H, int Hkv, int window, float scale,
                                                               bf16_t* __restrict__ out,
                                                               const PageGuard gd) {
  __shared__ __attribute__((aligned(1024))) bf16_t Ks[2][KSPLIT][PF_KB * 128];
  __shared__ __attribute__((aligned(1024))) bf16_t Vs[2][KSPLIT][PF_KB * 128];
  const int nrb = (M + 127) / 128;
  attn_row_block<FIXED, KSPLIT>(q, rows, ptab, max_pages, kv_slot, page_elems, M, H, Hkv, window, scale, out,
                                (nrb - 1 - (int)blockIdx.y) * 128, (int)blockIdx.x, Ks, Vs, gd);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_rope_qk_kv(int dtype, const float* qkv, const int32_t* rows, const int32_t* ptab, int max_pages,
                             const float2* rope, void* q_out, void* kv_slot, int M, int H, int Hkv, int dh,
                             size_t page_elems, int seq, int pos0, const PageGuard& gd, hipStream_t st) {
  if (dtype != 0 && dh == 128 && seq >= 0 && pos0 >= 0) {
    const int tiles = (pos0 + M - 1) / 16 - pos0 / 16 + 1;
    DORY_LAUNCH(k_rope_page, dim3(tiles, Hkv), dim3(1024), 0, st, qkv, seq, pos0, M, ptab, max_pages, rope,
                (bf16_t*)q_out, (bf16_t*)kv_slot, H, Hkv, page_elems, gd);
    return hipGetLastError();
  }
  dim3 grid(M, H + Hkv);
  if (dtype == 0)
    DORY_LAUNCH(k_rope_qk_kv<float>, grid, dim3(64), 0, st, qkv, rows, ptab, max_pages, rope,
                       (float*)q_out, (float*)kv_slot, H, Hkv, dh, page_elems, gd);
  else
    DORY_LAUNCH(k_rope_qk_kv<bf16_t>, grid, dim3(64), 0, st, qkv, rows, ptab, max_pages, rope,
                       (bf16_t*)q_out, (bf16_t*)kv_slot, H, Hkv, dh, page_elems, gd);
  return hipGetLastError();
}

template <typename T>
static hipError_t attn_t(const void* q, const int32_t* rows, const int32_t* ptab, int max_pages, const void* kv,
                         size_t page_elems, int M, int H, int Hkv, int dh, int window, float scale, int splits,
                         void* out, float* part_ml, float* part_o, const PageGuard& gd, hipStream_t st) {
  dim3 grid(M, Hkv, splits);
#define DORY_ATT(DHV)                                                                                         \
  DORY_LAUNCH((k_attn_rows<T, DHV>), grid, dim3(ATT_THREADS), 0, st, (const T*)q, rows, ptab, max_pages, \
                     (const T*)kv, page_elems, H, Hkv, window, scale, splits, (T*)out, part_ml, part_o, gd)
  switch (dh) {
    case 32: DORY_ATT(32); break;
    case 64: DORY_ATT(64); break;
    case 128: DORY_ATT(128); break;
    default: return hipErrorInvalidValue;
  }
#undef DORY_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  DORY_LAUNCH(k_attn_merge<T>, dim3(M * H), dim3(dh < 64 ? 64 : dh), 0, st, part_ml, part_o, splits, dh,
                     (T*)out);
  return hipGetLastError();
}

hipError_t launch_attn_rows(int dtype, const void* q, const int32_t* rows, const int32_t* ptab, int max_pages,
                            const void* kv, size_t page_elems, int M, int H, int Hkv, int dh, int window,
                            float scale, int splits, void* out, float* part_ml, float* part_o, const PageGuard& gd,
                            hipStream_t st) {
  if (H / Hkv > GMAX) return hipErrorInvalidValue;
  return dtype == 0 ? attn_t<float>(q, rows, ptab, max_pages, kv, page_elems, M, H, Hkv, dh, window, scale, splits,
                                    out, part_ml, part_o, gd, st)
                    : attn_t<bf16_t>(q, rows, ptab, max_pages, kv, page_elems, M, H, Hkv, dh, window, scale, splits,
                                     out, part_ml, part_o, gd, st);
}

bool attn_decode_supported(int dtype, int H, int Hkv, int dh) {
  return dtype == 1 && dh == 128 && H % Hkv == 0 && H / Hkv >= 1 && H / Hkv <= 4;
}

hipError_t launch_attn_decode(const float* qkv, const int32_t* rows, const int32_t* ptab, int max_pages,
                              const float2* rope, void* kv, size_t page_elems, int M, int H, int Hkv, int window,
                              float scale, int splits, int write_kv, void* out, float* part_ml, float* part_o,
                              const int32_t* order, int run_seq, int run_pos, const PageGuard& gd, hipStream_t st) {
  const int2 run = make_int2(M <= kDecodeMfmaRows ? run_seq : -1, run_pos);
  // consecutive positions of one sequence (a short chunk, whose keys / values the kernel writes
  // with write_kv): several rows per workgroup share every key load
  const bool multi = run.x >= 0 && M > 1;
  dim3 grid(M, Hkv, splits);
#define DORY_DEC(GV)                                                                                             \
  if (M > kDecodeMfmaRows && scale <= kFixedMaxScale)                                                          \
    DORY_LAUNCH(k_attn_decode_valu_fx<GV>, grid, dim3(256), 0, st, qkv, rows, ptab, max_pages, rope,           \
                (bf16_t*)kv, page_elems, H, Hkv, window, scale, splits, write_kv, (bf16_t*)out, part_ml, part_o, \
                order, gd);                                                                                    \
  else if (M > kDecodeMfmaRows)                                                                                \
    DORY_LAUNCH(k_attn_decode_valu<GV>, grid, dim3(256), 0, st, qkv, rows, ptab, max_pages, rope, (bf16_t*)kv, \
                page_elems, H, Hkv, window, scale, splits, write_kv, (bf16_t*)out, part_ml, part_o, gd);       \
  else if (multi)                                                                                              \
    DORY_LAUNCH((k_attn_decode<GV, 32>), dim3((M + 32 / GV - 1) / (32 / GV), Hkv, splits), dim3(256), 0, st, qkv, \
                rows, ptab, max_pages, rope, (bf16_t*)kv, page_elems, M, H, Hkv, window, scale, splits, write_kv,  \
                (bf16_t*)out, part_ml, part_o, run, gd);                                                        \
  else                                                                                                         \
    DORY_LAUNCH((k_attn_decode<GV, GV>), grid, dim3(256), 0, st, qkv, rows, ptab, max_pages, rope, (bf16_t*)kv, \
                page_elems, M, H, Hkv, window, scale, splits, write_kv, (bf16_t*)out, part_ml, part_o, run, gd)
  switch (H / Hkv) {
    case 1: DORY_DEC(1); break;
    case 2: DORY_DEC(2); break;
    case 3: DORY_DEC(3); break;
    case 4: DORY_DEC(4); break;
    default: return hipErrorInvalidValue;
  }
#undef DORY_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  DORY_LAUNCH(k_attn_merge<bf16_t>, dim3(M * H), dim3(128), 0, st, part_ml, part_o, splits, 128,
                     (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const void* q, const int32_t* rows, const int32_t* ptab, int max_pages, const void* kv,
                               size_t page_elems, int M, int H, int Hkv, int window, float scale, void* out,
                               const PageGuard& gd, hipStream_t st) {
  const int nrb = (M + 127) / 128;
  const dim3 grid(H, nrb);  // head fastest: longest row blocks first over the whole grid
  if (scale <= kFixedMaxScale)
    DORY_LAUNCH((k_attn_prefill<true, 2>), grid, dim3(512), 0, st, (const bf16_t*)q, rows, ptab, max_pages,
                (const bf16_t*)kv, page_elems, M, H, Hkv, window, scale, (bf16_t*)out, gd);
  else
    DORY_LAUNCH((k_attn_prefill<false, 1>), grid, dim3(256), 0, st, (const bf16_t*)q, rows, ptab, max_pages,
                (const bf16_t*)kv, page_elems, M, H, Hkv, window, scale, (bf16_t*)out, gd);
  return hipGetLastError();
}

}  // namespace dory
