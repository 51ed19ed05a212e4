/*
 * dory.h -- C ABI of the looped normalised-GPT forward pass on MI355X (gfx950).
 *
 * The model: an input stack of n_in blocks runs once, a shared recurrent core
 * of n_rec blocks runs k = 1..4 times with the loop update
 *     s_0 = x,  u_t = N(s_{t-1} + x),  s_t = N(F(u_t)),
 * where x is the input stack's output and N is L2 normalisation; the output
 * stack of n_out blocks and the LM head run once on s_k (onedev.kr summary
 * "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를 조절한다", section "어떻게 동작하나";
 * lucasainews article "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로 공개",
 * section "층을 되풀이하는 구조"). Every block is an attention sublayer followed by
 * an MLP sublayer, each applied as h <- N(h + alpha * (N(sublayer(h)) - h)).
 * Attention layers alternate sliding-window and full attention 3:1 (physical
 * block j is full iff j % full_every == full_every - 1).
 *
 * Conventions for every call:
 *  - Pointers named *_dev are device pointers (HBM of the context's GPU);
 *    pointers named *_host are host pointers. Nothing else is accepted.
 *  - The caller allocates and owns all device memory: weights, the KV pool,
 *    the workspace, inputs and outputs. The library borrows it for the life
 *    of the context and never frees it. The library owns only host metadata.
 *  - Work is enqueued asynchronously on the context's stream; results are
 *    valid once the caller synchronises that stream. No call synchronises the
 *    stream except where stated.
 *  - Argument and state errors are detected before anything is enqueued; the
 *    call then returns a negative status, leaves the context unchanged and
 *    records a message readable with dory_last_error(). A failed HIP launch
 *    returns DORY_E_HIP.
 *  - A context is not thread-safe: use one context per host thread / stream.
 */
#ifndef DORY_H
#define DORY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DORY_OK = 0,
  DORY_E_INVALID = -1, /* bad argument */
  DORY_E_STATE = -2,   /* call not allowed in the current state */
  DORY_E_NOMEM = -3,   /* KV pool, workspace or sequence table exhausted */
  DORY_E_HIP = -4      /* HIP runtime error */
} dory_status;

/* KV cache modes (trawling.dev digest "NVIDIA, 반복 연산형 4B 언어 모델 Dory 공개",
 * section "KV 캐시와 실행 환경"; onedev.kr summary, section "전제와 한계"):
 *  per-loop : every recurrent block keeps one cache per loop, so the cache
 *             holds n_in + n_out + k*n_rec layer slots;
 *  last-loop: every loop overwrites the recurrent block's single cache, so the
 *             cache holds n_in + n_rec + n_out slots for any k, and a query of
 *             an earlier loop reads keys/values the final loop wrote. */
typedef enum { DORY_KV_PER_LOOP = 0, DORY_KV_LAST_LOOP = 1 } dory_kv_mode_t;

typedef enum { DORY_F32 = 0, DORY_BF16 = 1 } dory_dtype_t;

/* Context flag: validate and do all host bookkeeping, but never touch the GPU
 * (no HIP call at all; device pointers may be NULL). For host-side tests. */
#define DORY_FLAG_DRY_RUN 1u
/* Context flag: keep MXFP8 copies of every projection and of the LM head
 * (OCP Microscaling Formats v1.0: FP8 E4M3 elements, one E8M0 scale per 32
 * consecutive elements of a row, quantised at create by the rule of
 * dory_quantize_mxfp8) in the workspace, and stream them instead of the bf16
 * weights in every call that processes at most 2 rows (decode of one or two
 * sequences, prefill chunks of one or two tokens): about half the weight bytes
 * per decode step. Calls of more rows use the bf16 weights. bf16 model only,
 * with d_model, n_heads*head_dim and d_ff in {1024, 3072, 4096, 8192}. The
 * workspace grows by about 1.03 bytes per weight (dory_query_sizes). */
#define DORY_FLAG_MXFP8_GEMV 4u
/* Context flag: as DORY_FLAG_MXFP8_GEMV with MXFP4 copies (OCP Microscaling
 * Formats v1.0: FP4 E2M1 elements, two per byte, one E8M0 scale per 32
 * consecutive elements of a row, by the rule of dory_quantize_mxfp4): about a
 * quarter of the bf16 weight bytes per decode step (lucasainews article "NVIDIA,
 * 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로 공개", section "학습 방식과 변형",
 * names 4-bit weights among the released formats). Excludes
 * DORY_FLAG_MXFP8_GEMV; same shape conditions; the workspace grows by about
 * 0.53 bytes per weight. */
#define DORY_FLAG_MXFP4_GEMV 16u
/* Context flag: sliding-window page recycling. A sliding-window layer reads
 * only the last `window` keys (trawling.dev digest "NVIDIA, 반복 연산형 4B
 * 언어 모델 Dory 공개", section "Reddit 반응", on the hybrid attention's cache
 * efficiency), so its pages are kept in a page space of their own, and the
 * pages wholly before (length - window + 1 - 64) return to the pool at the
 * start of every prefill / decode call. Full-attention slots keep every page.
 * The pool then holds ceil(tokens/16) pages of the full-attention slots plus up
 * to max_seqs * ((window + 64 + max_tokens)/16 + 3) pages of the sliding-window
 * slots (dory_query_sizes). dory_seq_truncate refuses a rollback into recycled
 * pages (rollbacks of up to 64 tokens always succeed). Results are identical
 * with and without the flag. Ignored without sliding-window or full layers. */
#define DORY_FLAG_SWA_RECYCLE 8u

typedef struct dory_config {
  int32_t d_model;       /* d */
  int32_t n_heads;       /* H query heads */
  int32_t n_kv_heads;    /* H_kv key/value heads; H % H_kv == 0 (query head h reads kv head h / (H/H_kv)) */
  int32_t head_dim;      /* d_h; 32, 64 or 128 */
  int32_t d_ff;          /* SwiGLU width */
  int32_t vocab;         /* V */
  int32_t n_in, n_rec, n_out; /* blocks in the input, recurrent and output stacks */
  int32_t full_every;    /* 4: every 4th physical block is full attention, the rest sliding-window */
  int32_t window;        /* W: a sliding-window query at position p sees keys p-W < j <= p */
  int32_t dtype;         /* dory_dtype_t: storage of weights, GEMM inputs and KV; accumulation is fp32 */
  int32_t page_size;     /* tokens per KV page; must be 16 */
  int32_t max_seqs;      /* sequence ids are 0 .. max_seqs-1 */
  int32_t max_model_len; /* tokens per sequence, at most 262144 */
  int32_t max_loops;     /* 1..4; the per-loop cache is laid out for this many loops */
  int32_t max_tokens;    /* most rows in one call: prefill chunk length or decode batch */
  uint32_t flags;        /* DORY_FLAG_* */
  float rope_theta;      /* 10000 */
  float attn_scale;      /* multiplies q.k of the unit-norm query and key before the softmax */
} dory_config;

/* Device pointers to the weights, borrowed. Matrices are row-major [out, in]
 * in the config's dtype (bf16 = raw 16-bit bfloat16). Per physical block j in
 * 0 .. n_in+n_rec+n_out-1:
 *   w_qkv[j]  [(H + 2*H_kv)*d_h, d]: query rows, then key rows, then value rows
 *   w_o[j]    [d, H*d_h]
 *   w_gu[j]   [2*d_ff, d]: gate rows 0..d_ff-1, up rows d_ff..2*d_ff-1
 *   w_down[j] [d, d_ff]
 *   alpha_attn[j], alpha_mlp[j]: fp32 [d], per-dimension residual step sizes
 * embed and lm_head are [V, d]. The pointer arrays themselves are host memory
 * and are copied by dory_create. */
typedef struct dory_weights {
  const void* embed;
  const void* lm_head;
  const void* const* w_qkv;
  const void* const* w_o;
  const void* const* w_gu;
  const void* const* w_down;
  const float* const* alpha_attn;
  const float* const* alpha_mlp;
} dory_weights;

typedef struct dory_ctx dory_ctx;

/* Counters kept by the scheduler (host side, also in dry-run mode). */
typedef struct dory_stats {
  int64_t calls;            /* prefill + decode calls that ran */
  int64_t block_apps;       /* block applications, summed over rows' calls (one per block per call) */
  int64_t sublayer_apps;    /* 2 per block application */
  int64_t full_apps;        /* full-attention block applications */
  int64_t swa_apps;         /* sliding-window block applications */
  int64_t kernel_launches;  /* kernels enqueued */
  int32_t n_slots;          /* cache layer slots of the current mode */
  int32_t pages_total;      /* pages the KV pool holds (of the full-attention slots under SWA recycling) */
  int32_t pages_in_use;
  int32_t live_seqs;
  int32_t swa_pages_total;  /* sliding-window pages (SWA recycling; else 0) */
  int32_t swa_pages_in_use;
  int32_t max_attn_splits;  /* most key splits per (row, KV head) any split-attention launch took */
} dory_stats;

/* Bytes the caller must allocate. kv_tokens: KV capacity in tokens summed over
 * all live sequences (rounded up to whole pages per sequence by the caller's
 * choice; each sequence holds ceil(len/16) pages). The KV pool holds, per page,
 * every layer slot of `kv_mode` laid out for cfg->max_loops loops. */
dory_status dory_query_sizes(const dory_config* cfg, int32_t kv_mode, int64_t kv_tokens,
                             size_t* kv_pool_bytes, size_t* workspace_bytes);

/* Create a context on the current HIP device. kv_pool_dev / workspace_dev must
 * be at least the sizes dory_query_sizes returned (256-byte aligned); the pool
 * may be larger, then it holds more pages. stream: a hipStream_t, or NULL for
 * the null stream. Initialises the rotary table in the workspace (enqueued). */
dory_status dory_create(const dory_config* cfg, const dory_weights* w, int32_t kv_mode,
                        void* kv_pool_dev, size_t kv_pool_bytes, void* workspace_dev,
                        size_t workspace_bytes, void* stream, dory_ctx** out);
void dory_destroy(dory_ctx* ctx);

/* Loop count k for the following calls: 1..cfg->max_loops. The recurrent core
 * runs k times per token; the released model takes 1..4 loops, chosen at run
 * time (lucasainews article "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지 정밀도로
 * 공개", section "실행 방법": n_recurrent_loops / dory.num_loops; trawling.dev
 * digest "NVIDIA, 반복 연산형 4B 언어 모델 Dory 공개", section "AI 요약"), and
 * a pass applies 16 + 20k blocks: 36 / 56 / 96 at k = 1 / 2 / 4 (onedev.kr
 * summary, section "어떻게 동작하나"). k outside 1..max_loops: DORY_E_INVALID.
 * In per-loop mode, a live sequence whose cache lacks loops 1..k for some of
 * its positions makes a later call on it fail with DORY_E_STATE. */
dory_status dory_set_loops(dory_ctx* ctx, int32_t k);
dory_status dory_get_loops(const dory_ctx* ctx, int32_t* k);

/* Switch KV mode; allowed only with no live sequence (else DORY_E_STATE). The
 * page capacity is recomputed for the new slot count. */
dory_status dory_kv_mode(dory_ctx* ctx, int32_t mode);

/* Prefill: the forward pass of the loop equation s_0 = x, u_t = N(s_{t-1} + x),
 * s_t = N(F(u_t)) over a chunk of consecutive positions (onedev.kr summary,
 * section "어떻게 동작하나"), with the KV writes of the configured mode (trawling.dev
 * digest, section "KV 캐시와 실행 환경"; onedev.kr summary, section "전제와 한계").
 * Append one chunk of n_tokens tokens (device int32 ids) to sequence seq_id,
 * creating it if it is not live, and run the forward pass on the chunk: in
 * every block application the chunk's keys/values are written to the block's
 * cache slot first, then every query of the chunk attends over its masked
 * range of that slot. Writes fp32 logits of the last `logits_rows` rows
 * (1 <= logits_rows <= n_tokens) to logits_dev [logits_rows, V] and, if
 * ids_dev is not NULL, their argmax (lowest id on ties) to ids_dev
 * [logits_rows]. n_tokens <= cfg->max_tokens; len + n_tokens <= max_model_len. */
dory_status dory_prefill(dory_ctx* ctx, int32_t seq_id, const int32_t* tokens_dev,
                         int32_t n_tokens, int32_t logits_rows, float* logits_dev,
                         int32_t* ids_dev);

/* Decode: the same forward pass on one new position of each of n_seqs distinct
 * live sequences (onedev.kr summary, section "어떻게 동작하나"), batched the way
 * the serving setup runs up to 128 sequences at once (lucasainews article,
 * section "실행 방법": max-num-seqs 128); in last-loop mode every loop's queries
 * read the keys/values the final loop of earlier steps left (onedev.kr summary,
 * section "전제와 한계"). Token tokens_dev[i] (device) is appended to sequence
 * seq_ids_host[i] (host: the scheduler needs the ids to build page tables and
 * the row order before anything is enqueued, and the list is small). Writes logits
 * [n_seqs, V] to logits_dev (may be NULL: then only ids are produced, using
 * workspace memory) and the greedy next ids [n_seqs] to next_ids_dev (may be
 * NULL). next_ids_dev may be passed as the next call's tokens_dev. Errors: a
 * sequence not live or listed twice, n_seqs outside 1..min(max_tokens,
 * max_seqs) -> DORY_E_INVALID; per-loop cache lacking loops -> DORY_E_STATE;
 * pool exhausted -> DORY_E_NOMEM. */
dory_status dory_decode(dory_ctx* ctx, int32_t n_seqs, const int32_t* seq_ids_host,
                        const int32_t* tokens_dev, float* logits_dev, int32_t* next_ids_dev);

/* Roll a live sequence back to new_len tokens (0 <= new_len <= len); pages past
 * the new end return to the pool. Used to drop rejected speculative tokens. */
dory_status dory_seq_truncate(dory_ctx* ctx, int32_t seq_id, int32_t new_len);
dory_status dory_seq_release(dory_ctx* ctx, int32_t seq_id);
dory_status dory_seq_len(const dory_ctx* ctx, int32_t seq_id, int32_t* len);

/* KV bytes held by live sequences: pages in use x slots x bytes per page slot. */
dory_status dory_kv_bytes_in_use(const dory_ctx* ctx, size_t* bytes);
dory_status dory_get_stats(const dory_ctx* ctx, dory_stats* out);

/* Temperature / top-p draw (lucasainews article "NVIDIA, 루프 구조 4B 모델
 * Dory1.0-4B 4가지 정밀도로 공개", section "실행 방법": recommended serving with
 * temperature 1.0 and top-p 0.95) for each row of logits_dev [rows, vocab]
 * (device, fp32, row-major, at least one finite value per row, no NaN), with
 * the caller's uniform uniforms_dev[r] in [0, 1) (device, fp32); the token ids
 * go to ids_dev [rows] (device, int32). Rule: token i has mass
 * round(exp((l_i - max l) / temperature) * 2^40), an integer (sums are exact,
 * so the draw does not depend on reduction order); the nucleus is every token
 * whose logit is at least the largest logit value whose tokens at or above it
 * hold at least top_p of the total mass (ties at that value all kept; top_p >= 1
 * keeps every token, top_p <= 0 the top logit and its ties); the id is the first
 * nucleus token in id order whose running mass exceeds floor(u * nucleus mass).
 * temperature <= 0 is greedy (lowest id among the largest logits); a positive
 * temperature so small that 1/T overflows keeps only the largest logit and its
 * ties, as the rule does. Each row is spread over several workgroups that pass
 * partial results through a scratch buffer of dory_sample_scratch_bytes(rows,
 * vocab) bytes, which the library allocates on the current device at the first
 * call that needs it (and grows for a larger call; hipFree of the old buffer
 * waits for the device), keeping it until the process ends; every call on one
 * device shares it, so calls that overlap on one GPU (other streams or host
 * threads) race. The call is queued on `stream` (a hipStream_t, NULL for the
 * default stream). DORY_E_INVALID: rows < 0, vocab outside 1..2^23, NULL
 * buffers with rows > 0, NaN or infinite temperature, NaN top_p;
 * DORY_E_NOMEM: the scratch could not be allocated. */
dory_status dory_sample(const float* logits_dev, int32_t rows, int32_t vocab, float temperature, float top_p,
                        const float* uniforms_dev, int32_t* ids_dev, void* stream);

/* Bytes of scratch a dory_sample call of `rows` rows of `vocab` logits uses (0 for invalid
 * sizes): about 8.3 KB per row. */
size_t dory_sample_scratch_bytes(int32_t rows, int32_t vocab);

/* dory_sample for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that forbid allocation): the same draw and the same kernels, with the scratch
 * in a fixed 4 MiB device array of the library (one copy per GPU, held until the process ends)
 * instead of an allocation. Calls no hipMalloc, hipFree or other allocating routine; the
 * array's address is looked up once per device at the first call on it. Every call on one GPU
 * shares the array (each call clears what must start at zero): calls that overlap on one GPU
 * race. DORY_E_INVALID as dory_sample, and when dory_sample_scratch_bytes(rows, vocab) exceeds
 * 4 MiB (rows <= 256 always fit, for any vocab). */
dory_status dory_sample_static(const float* logits_dev, int32_t rows, int32_t vocab, float temperature,
                               float top_p, const float* uniforms_dev, int32_t* ids_dev, void* stream);

/* MXFP8 quantisation (OCP Microscaling Formats v1.0, MXFP8 with E4M3 elements)
 * of a bf16 matrix src_dev [rows, cols] (device, row-major, 16-byte aligned,
 * cols % 32 == 0): per 32 consecutive elements of a row, the E8M0 scale code
 * e + 127 with e = floor(log2(max |v|)) - 8 clamped to [-127, 127] (-127 for an
 * all-zero block) goes to scales_dev [rows, cols/32], and each element's E4M3
 * code (v / 2^e rounded to nearest even, magnitudes >= 448 saturating to 448,
 * sign kept) to codes_dev [rows, cols] (16-byte aligned). Enqueued on `stream`
 * (a hipStream_t, NULL = default stream); caller-owned buffers. */
dory_status dory_quantize_mxfp8(const void* src_dev, int64_t rows, int32_t cols, void* codes_dev, void* scales_dev,
                                void* stream);

/* MXFP4 quantisation (OCP Microscaling Formats v1.0, MXFP4 with FP4 E2M1
 * elements) of a bf16 matrix src_dev [rows, cols] (device, row-major, 16-byte
 * aligned, cols % 32 == 0): per 32 consecutive elements of a row, the E8M0
 * scale code e + 127 with e = floor(log2(max |v|)) - 2 clamped to [-127, 127]
 * (-127 for an all-zero block) goes to scales_dev [rows, cols/32], and each
 * element's E2M1 code (v / 2^e rounded to the nearest of 0, 0.5, 1, 1.5, 2, 3,
 * 4, 6 with ties to the even code, magnitudes above 6 saturating to 6, sign
 * kept) to codes_dev [rows, cols/2] (16-byte aligned), two codes per byte with
 * element 2i in the low nibble. Enqueued on `stream`; caller-owned buffers. */
dory_status dory_quantize_mxfp4(const void* src_dev, int64_t rows, int32_t cols, void* codes_dev, void* scales_dev,
                                void* stream);

/* Device-side error flags raised since the last reset (synchronises the
 * stream): bit 0 = a token id outside 0..V-1 reached the embedding (it was
 * clamped into range, so that call's outputs are not those of the given ids).
 * The checked build (dory_checked_build() == 1) also raises: bit 1 = a
 * page-table read with a sequence or page index outside the table, bit 2 = a
 * page id outside the pages of the cache region it indexes, bit 3 = a RoPE
 * position outside 0..max_model_len-1; each offending read used index 0
 * instead, so the access stayed inside its buffer but that call's outputs are
 * meaningless. With reset != 0 the flags are cleared afterwards. */
dory_status dory_device_flags(dory_ctx* ctx, int32_t* flags, int32_t reset);

/* 1 for the checked (debug) build of this library, libdory_checked.so, whose
 * attention kernels bounds-check every page-table entry, page id and RoPE row
 * they read (see dory_device_flags) and whose host runtime checks that each
 * layer slot's cache region lies inside the KV pool before its launches (else
 * the call fails with DORY_E_HIP); 0 for the default build, which reads them
 * as given. Both builds compute the same results on valid state. */
int32_t dory_checked_build(void);

/* Checked build only (else DORY_E_STATE): overwrite entry page_index of
 * sequence seq_id's full-attention page table on the device with page_id and
 * return the previous entry in *old_id (may be NULL). Synchronises the
 * context's stream. A fault injection for testing the checked build's guards:
 * the host's own record of the sequence's pages is not changed, so restore the
 * entry before relying on the sequence's outputs again. DORY_E_INVALID:
 * seq_id or page_index outside the table. */
dory_status dory_debug_set_page(dory_ctx* ctx, int32_t seq_id, int32_t page_index, int32_t page_id,
                                int32_t* old_id);

/* Copy the final hidden states (output of the output stack, fp32 [rows, d]) of
 * the previous prefill/decode call's last `rows` rows to dst_dev. Enqueued. */
dory_status dory_last_hidden(dory_ctx* ctx, float* dst_dev, int32_t rows);

/* Self-speculative greedy decoding on one live sequence (onedev.kr summary,
 * section "전제와 한계"): draft `gamma` (1..16) tokens with k_draft loops by
 * decode calls, verify [last, d_1..d_gamma] as one chunk with k_verify loops,
 * keep the longest agreeing prefix plus the verifier's next token and roll the
 * cache back past the rest. reuse = 0: the cache is rolled back to the start of
 * the draft and the verify chunk runs the whole stack. reuse = 1 (needs
 * k_draft = 1): a drafted row's input-stack output, loop-1 state and the KV both
 * write are what the verify chunk would compute again, so the draft's cache is
 * kept, d_gamma alone runs the input stack and loop 1, and loops 2..k_verify,
 * the output stack and the LM head run for all gamma + 1 rows from the saved
 * states (equal to reuse = 0 in exact arithmetic). `last_host` is the newest
 * generated id (not yet in the cache). Produces at least n_new ids into
 * out_ids_host (capacity n_new + gamma) and returns their count in *n_out.
 * Synchronises the stream once per verify step (the accepted length decides the
 * next step). */
dory_status dory_spec_decode(dory_ctx* ctx, int32_t seq_id, int32_t last_host, int32_t n_new,
                             int32_t gamma, int32_t k_draft, int32_t k_verify, int32_t reuse,
                             int32_t* out_ids_host, int32_t* n_out);

/* Counters of the dory_spec_decode calls since the last reset, for its cost model: rounds
 * (draft + verify steps), tokens drafted, drafted tokens the verifier accepted, ids produced
 * (accepted + one per round), and the GPU time of the draft phases and of the verify phases
 * (HIP events recorded on the context's stream at each phase boundary; the verify phase runs
 * from the end of the last draft step to the end of the verify chunk's LM head and argmax). */
typedef struct dory_spec_stats {
  int64_t rounds;
  int64_t drafted;
  int64_t accepted;
  int64_t produced;
  double draft_ms;
  double verify_ms;
} dory_spec_stats;

/* Copy the counters to *out; with reset != 0 restart them from zero afterwards. */
dory_status dory_get_spec_stats(dory_ctx* ctx, dory_spec_stats* out, int32_t reset);

/* Per-kernel accounting, one entry per kernel role of the forward pass
 * ("qkv_proj", "rope_qknorm_kvwrite", "attention", "o_proj", "ngpt_residual",
 * "gate_up_swiglu", "down_proj", "loop_norm", "embed", "lm_head", "argmax",
 * "page_table"). bytes and flops are the algorithmic HBM bytes and flops the
 * launches must move or compute (weights, activations, the keys/values in each
 * row's attention range), counted for every launch. timed_launches / total_ms
 * come from a HIP event pair recorded around each launch while timing is
 * enabled (dory_set_timing). */
typedef struct dory_kernel_time {
  char name[32];
  int64_t launches;
  double bytes;
  double flops;
  int64_t timed_launches;
  double total_ms;
} dory_kernel_time;

/* Enable (1) or disable (0) the event pair around every launch. */
dory_status dory_set_timing(dory_ctx* ctx, int32_t enable);
/* Copy up to max entries (roles that launched at least once) to out and their
 * count to *n; synchronises the stream when timed events are pending. With
 * reset != 0 the counters restart from zero afterwards. */
dory_status dory_get_timing(dory_ctx* ctx, dory_kernel_time* out, int32_t max, int32_t* n, int32_t reset);

const char* dory_last_error(const dory_ctx* ctx);
const char* dory_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* DORY_H */
