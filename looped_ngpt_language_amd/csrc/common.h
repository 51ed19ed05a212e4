// Shared device helpers for the gfx950 kernels: storage types, vector loads,
// wave64 / workgroup reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DORY_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // raw bfloat16 bits in memory

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Reinterpret two packed bfloat16 values. The argument is taken by value: a
// bit_cast applied directly to a vector-element expression reads element 0.
DORY_DEV bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

DORY_DEV float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest even (inputs are finite).
DORY_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Storage-type traits: float (fp32 model) or bf16_t (bf16 model).
template <typename T> struct St;
template <> struct St<float> {
  static DORY_DEV float ld(const float* p, size_t i) { return p[i]; }
  static DORY_DEV void st(float* p, size_t i, float v) { p[i] = v; }
  static DORY_DEV float cvt(float v) { return v; }
};
template <> struct St<bf16_t> {
  static DORY_DEV float ld(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static DORY_DEV void st(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  static DORY_DEV float cvt(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Load 8 consecutive elements as fp32 (16 B for bf16, 32 B for fp32; aligned).
DORY_DEV void load8(const bf16_t* p, float* out) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
DORY_DEV void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

DORY_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DORY_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a workgroup of `nwaves` waves; every thread gets the result.
// `red` must hold nwaves floats of LDS; the call contains two barriers.
DORY_DEV float block_sum(float v, float* red, int nwaves) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nwaves; ++i) s += red[i];
  __syncthreads();
  return s;
}

// Value-row position of token t (0..15) inside a KV page: t with bits 2 and 3
// swapped, so the 8 tokens one lane covers in a 32x32 score tile are contiguous.
DORY_DEV constexpr int vperm(int t) { return (t & 3) | ((t >> 3) & 1) << 2 | ((t >> 2) & 1) << 3; }

// Online-softmax rescale factor exp(m_old - m_new), 0 when nothing was accumulated yet.
DORY_DEV float safe_scale(float m_old, float m_new) { return m_old == -INFINITY ? 0.f : __expf(m_old - m_new); }

DORY_DEV float silu(float z) { return z / (1.f + __expf(-z)); }

// The smallest positive normal float: lower bound of a sum of squares before
// the reciprocal square root, so a zero vector yields zeros instead of NaN.
#define DORY_TINY_SS 1.17549435e-38f

// s_waitcnt immediate for vmcnt(n) (gfx9 encoding), other counters left free
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// One 16-byte-per-lane load from gbase + voff (bytes) straight into LDS at lds_byte + 16 lane
// (global_load_lds_dwordx4; M0 holds the wave's LDS base). Issued from inline assembly so that
// the compiler, which cannot tell LDS stages apart, does not wait for it before unrelated LDS
// reads; the caller waits with s_waitcnt vmcnt before the barrier that publishes the data.
// The compiler warns that m0 is a reserved register it will not preserve around the asm: in the
// gfx950 code of k_gemm.hip and k_attn.hip every instruction that reads or writes m0 is one of
// these asm blocks (the compiler itself keeps nothing in m0 there), so no value is lost.
DORY_DEV void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_byte)), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
