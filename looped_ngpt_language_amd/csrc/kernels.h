// Launchers of the gfx950 kernels (device pointers, stream-ordered, no allocation).
// dtype: 0 = fp32 model, 1 = bf16 model (storage type of weights, GEMM inputs, KV).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dory {

// Event pair the launchers attach to their dispatches while `stop` is set
// (timing mode): `start` is recorded by the first dispatch's start, `stop` by
// the end of every dispatch, so the pair spans exactly the role's kernels.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
extern thread_local LaunchEvents g_launch_events;

}  // namespace dory

#define DORY_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                                    \
  do {                                                                                                          \
    if (::dory::g_launch_events.stop) {                                                                         \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, ::dory::g_launch_events.start,                \
                            ::dory::g_launch_events.stop, 0, __VA_ARGS__);                                      \
      ::dory::g_launch_events.start = nullptr;                                                                  \
    } else {                                                                                                    \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                                     \
    }                                                                                                           \
  } while (0)

namespace dory {

hipError_t launch_embed(int dtype, const int32_t* tokens, const void* E, int V, int d, int M, float* h, void* hb,
                        int32_t* err, hipStream_t st);
// h <- N(h + alpha (N(y) - h)) on M rows of d; with parts > 1 (bf16 model) y holds that many split-K
// partial slices [parts][M][d] left by launch_gemm (see below), summed here.
hipError_t launch_residual(int dtype, float* h, const float* y, const float* alpha, void* hb, int M, int d,
                           hipStream_t st, int parts = 0);
hipError_t launch_norm_sum(int dtype, const float* a, const float* b, float* h, float* s, void* hb, int M, int d,
                           hipStream_t st);
// Loop boundary in one launch (k_rows.hip): optional pending residual step on h (y != nullptr),
// then mode 0 (end of the input stack): u_1 = N(2 v) -> hout, the stepped v written back to h;
// mode 1 (end of loop t < k): s_t = N(v) -> s, u_{t+1} = N(s_t + x) -> hout; mode 2 (end of
// loop k): s_k = N(v) -> s and hout. hb gets the storage copy of hout. hout may alias h.
hipError_t launch_loop_step(int dtype, float* h, const float* y, const float* alpha, const float* x, float* s,
                            float* hout, void* hb, int M, int d, int mode, hipStream_t st);
constexpr int kArgmaxParts = 64;  // partial (max, index) pairs per row in the argmax scratch
hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* ids, void* scratch, hipStream_t st);
// entries: size of the table (checked build: updates outside it are skipped and flagged in *flags)
hipError_t launch_apply_updates(int32_t* table, const int32_t* upd, int n, int entries, int32_t* flags,
                                hipStream_t st);
hipError_t launch_rope_table(float2* tab, int max_len, int dh, double theta, hipStream_t st);
hipError_t launch_copy_f32(float* dst, const float* src, size_t n, hipStream_t st);

// Index guard of the kernels that follow a page table (k_attn.hip). The default build reads page
// ids and RoPE rows as given: the host validates every sequence, position and page it hands to
// the device. Built with DORY_CHECKED=1 (the debug library), every page-table read first checks
// the sequence against max_seqs and the page index against the table width, then the page id it
// read against the pages of the slot's cache region, and every RoPE row read checks its position
// against max_pos; a violation sets a bit of *flags (kDevFlag*) and uses index 0 instead, so each
// access stays inside its buffer (that call's outputs are then meaningless).
struct PageGuard {
  int32_t max_seqs;    // rows of the page table
  int32_t pool_pages;  // pages of the cache region the table's ids index
  int32_t max_pos;     // rows of the RoPE table
  int32_t* flags;      // the context's device flag word
};
constexpr int32_t kDevFlagTokenId = 1, kDevFlagPageIndex = 2, kDevFlagPageId = 4, kDevFlagPosition = 8;
#ifndef DORY_CHECKED
#define DORY_CHECKED 0
#endif

// RoPE + per-head q/k norm + KV write of M rows. seq, pos0 >= 0: the rows are the consecutive
// positions pos0 .. pos0+M-1 of sequence seq (a prefill chunk; page-tiled kernel for bf16 d_h 128).
hipError_t launch_rope_qk_kv(int dtype, const float* qkv, const int32_t* rows, const int32_t* ptab, int max_pages,
                             const float2* rope, void* q_out, void* kv_slot, int M, int H, int Hkv, int dh,
                             size_t page_elems, int seq, int pos0, const PageGuard& gd, hipStream_t st);
hipError_t launch_attn_rows(int dtype, const void* q, const int32_t* rows, const int32_t* ptab, int max_pages,
                            const void* kv, size_t page_elems, int M, int H, int Hkv, int dh, int window,
                            float scale, int splits, void* out, float* part_ml, float* part_o, const PageGuard& gd,
                            hipStream_t st);

bool attn_decode_supported(int dtype, int H, int Hkv, int dh);
constexpr int kDecodeMfmaRows = 16;  // split-key attention: MFMA kernel up to this many rows, VALU kernel above
// order (may be NULL): a permutation of the M rows giving the order in which the batched (more than
// kDecodeMfmaRows rows) kernels take them, longest context first, so that short rows fill the tail.
hipError_t launch_attn_decode(const float* qkv, const int32_t* rows, const int32_t* ptab, int max_pages,
                              const float2* rope, void* kv, size_t page_elems, int M, int H, int Hkv, int window,
                              float scale, int splits, int write_kv, void* out, float* part_ml, float* part_o,
                              const int32_t* order, int run_seq, int run_pos, const PageGuard& gd, hipStream_t st);
// (run_seq >= 0: the M <= kDecodeMfmaRows rows are positions run_pos, run_pos + 1, ... of sequence
// run_seq, so the kernel takes them from its arguments instead of loading the row list.
// write_kv: the kernel writes the rows' own keys / values first (decode rows; or such a chunk of
// at most 32 / G rows, which one workgroup per split then holds whole).)
hipError_t launch_attn_prefill(const void* q, const int32_t* rows, const int32_t* ptab, int max_pages, const void* kv,
                               size_t page_elems, int M, int H, int Hkv, int window, float scale, void* out,
                               const PageGuard& gd, hipStream_t st);

bool gemv_supported(int K);
bool gemv_residual_supported(int K);
constexpr int kGemvMaxRows = 8;
// GEMV for M <= 8 bf16 rows (k_gemv.hip). W is bf16 [N, K], or with `scales` != NULL (M <= 2)
// MXFP8 element codes [N, K] (uint8) with E8M0 block scales in the lane-major layout
// (mx_scale_row_bytes(K) bytes per row, as written by launch_mx_quantize with lane_major).
// mx_fmt (with scales): 1 = MXFP8 codes [N, K], 2 = MXFP4 codes [N, K / 2] (element 2i in the low nibble).
hipError_t launch_gemv(bool dual, const void* X, const void* W, const uint8_t* scales, void* out, int M, int N, int K,
                       hipStream_t st, int mx_fmt = 1);
// GEMV (M <= 2) whose input rows are N(h + alpha (N(y) - h)), computed in the prologue; the fp32
// result is also written to hout (which must not alias h or y).
hipError_t launch_gemv_residual(bool dual, const void* W, const uint8_t* scales, void* out, int M, int N, int K,
                                const float* h, const float* y, const float* alpha, float* hout, hipStream_t st,
                                int mx_fmt = 1);
// bf16 [rows, cols] -> MXFP8 codes [rows, cols] + scales [rows, cols / 32] (cols % 32 == 0), or
// with lane_major the GEMV's scale layout (rows * mx_scale_row_bytes(cols) bytes; padding untouched).
// fmt 1: MXFP8 codes [rows, cols]; fmt 2: MXFP4 codes [rows, cols / 2] (element 2i in the low nibble).
hipError_t launch_mx_quantize(const void* src, long long rows, int cols, void* codes, void* scales, bool lane_major,
                              hipStream_t st, int fmt = 1);
// bytes per weight row of the lane-major MXFP8 scale layout the GEMV reads (0: K unsupported)
int mx_scale_row_bytes(int K);
// Temperature / top-p draw per row of fp32 logits [rows, V] with the caller's uniforms [rows]
// (k_sample.hip); temperature <= 0 is greedy. 1 <= V <= 2^23. Each row is spread over several
// workgroups that hand partial results to each other through `scratch` (device memory of at
// least sample_scratch_bytes(rows, V) bytes; the call clears what must start at zero).
size_t sample_scratch_bytes(int rows, int V);
hipError_t launch_sample(const float* logits, int rows, int V, float temperature, float top_p, const float* uniforms,
                         int32_t* ids, void* scratch, size_t scratch_bytes, hipStream_t st);
// dory_sample's scratch: allocated on the current device at first use, grown when needed.
hipError_t sample_library_scratch(int rows, int V, void** ptr, size_t* bytes);
// dory_sample_static's scratch: the current device's copy of a fixed device array of
// kSampleStaticScratchBytes bytes (its address is looked up once per device).
constexpr size_t kSampleStaticScratchBytes = (size_t)4 << 20;
hipError_t sample_static_scratch(void** ptr);
// C = A . B^T (bf16 or fp32 model). split_ws (may be NULL) holds split-K partials for 3..256 rows.
// parts (may be NULL; plain products only): when the product is split over K, the partial slices
// [S][M][N] are left in split_ws unsummed, out is not written and *parts = S; otherwise *parts = 0.
hipError_t launch_gemm(int dtype, bool dual, const void* A, const void* B, void* out, int M, int N, int K,
                       float* split_ws, size_t split_ws_bytes, hipStream_t st, int* parts = nullptr);

}  // namespace dory
