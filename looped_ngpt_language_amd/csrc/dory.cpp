// Host runtime of the looped nGPT forward pass: the C ABI declared in dory.h,
// argument/state validation, the paged KV manager and the k-aware scheduler.
//
// Scheduler (onedev.kr summary "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를 조절한다",
// section "어떻게 동작하나"): the input stack runs once and yields x; s_0 = x; for
// t = 1..k the recurrent core runs on u_t = N(s_{t-1} + x) and s_t = N(F(u_t));
// the output stack and the LM head run once on s_k. The recurrent core's
// weights are re-read on every loop.
// KV slots (trawling.dev digest "NVIDIA, 반복 연산형 4B 언어 모델 Dory 공개", section
// "KV 캐시와 실행 환경"; lucasainews article, section "층을 되풀이하는 구조"): input and
// output blocks own one slot each; a recurrent block owns one slot per loop in
// per-loop mode and one overwritten slot in last-loop mode.
#include "../../include/dory.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cmath>
#include <string>
#include <vector>

#include "kernels.h"

namespace dory {
thread_local LaunchEvents g_launch_events = {nullptr, nullptr};
}

namespace {

constexpr int kPage = 16;
// SWA page recycling keeps this many positions below the window, so a sequence can be rolled
// back (rejected speculative tokens, at most 16) and a chunk's first key block (32 keys, aligned
// down) never touches a recycled page.
constexpr int kSwaReserve = 64;
// Key splits per (row, KV head) at most: one decode row with 8 KV heads then fills the 256 CUs
// with one round of the one-workgroup-per-CU MFMA decode kernel (131072-token context: 32 splits
// 125 tok/s at k = 4, 64 splits 119, 128 splits 115).
constexpr int kMaxSplits = 32;
constexpr int kMaxGamma = 16;  // speculative draft length limit
constexpr int kStageSlots = 4;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {  // byte offsets inside the workspace
  size_t rope, ptab, upload, err, buf[4], y, hb, qkv, q, o, z, part_ml, part_o, logits, argmax, splitk, spec, spec_x,
      spec_s1, mx, mx_bytes, total;
  size_t splitk_bytes;
  int max_pages;       // pages per sequence
  int upload_ints;     // capacity of the upload area in int32
  int part_rows;       // rows that may use split attention
  int logit_rows;      // rows of the logits scratch
};

int qkv_cols(const dory_config& c) { return (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; }
size_t esize(const dory_config& c) { return c.dtype == DORY_F32 ? 4 : 2; }

Layout make_layout(const dory_config& c) {
  Layout L{};
  const size_t M = c.max_tokens, d = c.d_model, es = esize(c);
  L.max_pages = (c.max_model_len + kPage - 1) / kPage;
  const int upd_max = 2 * (c.max_tokens / kPage + 2 + c.max_seqs);  // full and sliding-window page tables
  L.upload_ints = 3 * c.max_tokens + 2 * upd_max + 16;  // rows, page-table updates, batched row order
  L.part_rows = std::min(c.max_tokens, std::max(c.max_seqs, 16));
  L.logit_rows = std::max(c.max_seqs, 8);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.rope = take((size_t)c.max_model_len * (c.head_dim / 2) * sizeof(float2));
  // page tables [max_seqs][max_pages]: the full-attention one, then (SWA recycling) the sliding-window one
  L.ptab = take((size_t)((c.flags & DORY_FLAG_SWA_RECYCLE) ? 2 : 1) * c.max_seqs * L.max_pages * 4);
  L.upload = take((size_t)L.upload_ints * 4);
  L.err = take(kAlign);
  for (int i = 0; i < 4; ++i) L.buf[i] = take(M * d * 4);
  L.y = take(M * d * 4);
  L.hb = take(M * d * es);
  L.qkv = take(M * qkv_cols(c) * 4);
  L.q = take(M * (size_t)c.n_heads * c.head_dim * es);
  L.o = take(M * (size_t)c.n_heads * c.head_dim * es);
  L.z = take(M * (size_t)c.d_ff * es);
  L.part_ml = take((size_t)L.part_rows * c.n_heads * kMaxSplits * 2 * 4);
  L.part_o = take((size_t)L.part_rows * c.n_heads * kMaxSplits * c.head_dim * 4);
  L.logits = take((size_t)L.logit_rows * c.vocab * 4);
  L.argmax = take((size_t)std::max(c.max_tokens, L.logit_rows) * dory::kArgmaxParts * 8);
  {
    const size_t nmax = std::max({(size_t)qkv_cols(c), (size_t)2 * c.d_ff, (size_t)c.d_model});
    L.splitk_bytes = c.dtype == DORY_BF16 ? 4 * (size_t)std::min(c.max_tokens, 256) * nmax * 4 : 0;
    L.splitk = take(L.splitk_bytes);
  }
  L.spec = take(64 * 4);
  // self-speculative decoding with reuse: input-stack output and loop-1 state of the drafted rows
  L.spec_x = take((size_t)(kMaxGamma + 1) * d * 4);
  L.spec_s1 = take((size_t)(kMaxGamma + 1) * d * 4);
  // MXFP8 copies of every projection and of the LM head (codes, then scales per matrix)
  L.mx_bytes = 0;
  if (c.flags & (DORY_FLAG_MXFP8_GEMV | DORY_FLAG_MXFP4_GEMV)) {
    const size_t nb = (size_t)(c.n_in + c.n_rec + c.n_out);
    const size_t hd = (size_t)c.n_heads * c.head_dim;
    const size_t block_params = (size_t)qkv_cols(c) * d + d * hd + 2 * (size_t)c.d_ff * d + d * (size_t)c.d_ff;
    const size_t params = nb * block_params + (size_t)c.vocab * d;
    // lane-major scale rows (mx_scale_row_bytes: 32 bytes per 1024 columns, 3072 padded to 4096)
    auto srb = [](int K) { return (size_t)dory::mx_scale_row_bytes(K); };
    const size_t block_scales = (size_t)qkv_cols(c) * srb(d) + d * srb((int)hd) + 2 * (size_t)c.d_ff * srb(d) +
                                d * srb(c.d_ff);
    const size_t scales = nb * block_scales + (size_t)c.vocab * srb(d);
    const size_t codes = (c.flags & DORY_FLAG_MXFP4_GEMV) ? params / 2 : params;  // MXFP4: two codes per byte
    L.mx_bytes = codes + scales + 16 * kAlign * (4 * nb + 1);
  }
  L.mx = take(L.mx_bytes);
  L.total = off;
  return L;
}

int n_slots_for(const dory_config& c, int mode) {
  return mode == DORY_KV_PER_LOOP ? c.n_in + c.n_out + c.n_rec * c.max_loops : c.n_in + c.n_rec + c.n_out;
}
size_t page_elems(const dory_config& c) { return (size_t)2 * c.n_kv_heads * kPage * c.head_dim; }

bool full_block(const dory_config& c, int j) { return j % c.full_every == c.full_every - 1; }

// Layer slots of a KV mode split into full-attention and sliding-window ones (block j's slots
// follow its attention kind).
void slot_counts(const dory_config& c, int mode, int* n_full, int* n_swa) {
  *n_full = *n_swa = 0;
  const int nb = c.n_in + c.n_rec + c.n_out;
  for (int j = 0; j < nb; ++j) {
    const int copies = (mode == DORY_KV_PER_LOOP && j >= c.n_in && j < c.n_in + c.n_rec) ? c.max_loops : 1;
    (full_block(c, j) ? *n_full : *n_swa) += copies;
  }
}

bool recycling(const dory_config& c) {
  int nf, ns;
  slot_counts(c, DORY_KV_LAST_LOOP, &nf, &ns);
  return (c.flags & DORY_FLAG_SWA_RECYCLE) && c.window > 0 && nf > 0 && ns > 0;
}

// Sliding-window pages one sequence can hold at once: the window, the reserve, one chunk, and
// the partial pages at either end.
int swa_pages_per_seq(const dory_config& c) { return (c.window + kSwaReserve + c.max_tokens) / kPage + 3; }

// Page counts (full-attention, sliding-window) a pool of `bytes` holds: as many pages of every
// slot as fit, except that sliding-window pages stop at what max_seqs sequences can hold, the
// remaining bytes going to full-attention pages.
void split_pool(const dory_config& c, int mode, size_t bytes, size_t* full_pages, size_t* swa_pages) {
  int nf, ns;
  slot_counts(c, mode, &nf, &ns);
  const size_t pb = page_elems(c) * (c.dtype == DORY_F32 ? 4 : 2);
  const size_t all = bytes / ((size_t)(nf + ns) * pb);
  const size_t smax = (size_t)c.max_seqs * swa_pages_per_seq(c);
  if (!recycling(c) || all <= smax) { *full_pages = *swa_pages = all; return; }
  *swa_pages = smax;
  *full_pages = (bytes - smax * ns * pb) / ((size_t)nf * pb);
}

std::string check_config(const dory_config* c) {
  if (!c) return "config is NULL";
  if (c->d_model <= 0 || c->d_model > 4096) return "d_model must be in 1..4096";
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 32, 64 or 128";
  if (c->n_heads <= 0 || c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads) return "n_heads must be a multiple of n_kv_heads";
  if (c->n_heads / c->n_kv_heads > 8) return "at most 8 query heads per KV head";
  if (c->d_ff <= 0 || c->vocab <= 0) return "d_ff and vocab must be positive";
  if (c->n_in < 0 || c->n_out < 0 || c->n_rec < 1) return "stack sizes: n_in, n_out >= 0 and n_rec >= 1";
  if (c->full_every < 1 || c->window < 1) return "full_every and window must be >= 1";
  if (c->dtype != DORY_F32 && c->dtype != DORY_BF16) return "dtype must be DORY_F32 or DORY_BF16";
  if (c->page_size != kPage) return "page_size must be 16";
  if (c->max_seqs < 1 || c->max_tokens < 1) return "max_seqs and max_tokens must be >= 1";
  if (c->max_model_len < 1 || c->max_model_len > 262144) return "max_model_len must be in 1..262144";
  if (c->max_loops < 1 || c->max_loops > 4) return "max_loops must be in 1..4";
  if (c->dtype == DORY_BF16) {
    const int hd = c->n_heads * c->head_dim;
    if (c->d_model % 64 || c->d_ff % 64 || hd % 64) return "bf16 model: d_model, d_ff and n_heads*head_dim must be multiples of 64";
  }
  if (!(c->rope_theta > 0.f) || !(c->attn_scale > 0.f)) return "rope_theta and attn_scale must be positive";
  if ((c->flags & DORY_FLAG_MXFP8_GEMV) && (c->flags & DORY_FLAG_MXFP4_GEMV))
    return "DORY_FLAG_MXFP8_GEMV and DORY_FLAG_MXFP4_GEMV exclude each other";
  if (c->flags & (DORY_FLAG_MXFP8_GEMV | DORY_FLAG_MXFP4_GEMV)) {
    if (c->dtype != DORY_BF16) return "MX weights need the bf16 model";
    if (!dory::gemv_supported(c->d_model) || !dory::gemv_supported(c->n_heads * c->head_dim) ||
        !dory::gemv_supported(c->d_ff))
      return "MX weights need d_model, n_heads*head_dim and d_ff in {1024, 3072, 4096, 8192}";
  }
  return "";
}

struct Seq {
  bool live = false;
  int len = 0;
  std::vector<int32_t> pages;      // physical page of every logical page (full-attention slots, or all slots)
  std::vector<int32_t> swa_pages;  // sliding-window slots under recycling; -1 once recycled
  int swa_lo = 0;                  // first logical sliding-window page still held
  std::vector<std::pair<int, int>> runs;  // (end position, loops whose KV is valid) -- per-loop mode
  int min_loops() const {
    int m = 4;
    for (auto& r : runs) m = std::min(m, r.second);
    return m;
  }
  void append_run(int end, int k) {
    if (!runs.empty() && runs.back().second == k) runs.back().first = end;
    else runs.emplace_back(end, k);
  }
  void trim_runs(int new_len) {
    while (!runs.empty()) {
      const int start = runs.size() > 1 ? runs[runs.size() - 2].first : 0;
      if (start >= new_len) runs.pop_back();
      else { runs.back().first = std::min(runs.back().first, new_len); break; }
    }
  }
};

enum Role { R_EMBED, R_QKV, R_ROPE, R_ATTN, R_OPROJ, R_RESID, R_GU, R_DOWN, R_LOOPN, R_LM, R_ARGMAX, R_PTAB, R_COUNT };
const char* const kRoleName[R_COUNT] = {"embed", "qkv_proj", "rope_qknorm_kvwrite", "attention", "o_proj",
                                        "ngpt_residual", "gate_up_swiglu", "down_proj", "loop_norm", "lm_head",
                                        "argmax", "page_table"};

struct RoleAcc {
  int64_t launches = 0, timed = 0;
  double bytes = 0, flops = 0, ms = 0;
};

struct TimedRec {
  int role;
  hipEvent_t a, b;
};

}  // namespace

struct dory_ctx {
  dory_config cfg{};
  Layout L{};
  int kv_mode = DORY_KV_PER_LOOP;
  int k = 1;
  bool dry = false;
  hipStream_t stream = nullptr;
  int n_blocks = 0, n_slots = 0, pages_total = 0;
  size_t page_el = 0, page_bytes = 0;
  // sliding-window page recycling: separate page space for the sliding-window slots
  bool recycle = false;
  int n_full_slots = 0, n_swa_slots = 0, swa_pages_total = 0;
  std::vector<int> slot_class_idx;  // per slot: index within its class, sliding-window ones negated - 1
  std::vector<int32_t> free_swa;
  char* pool = nullptr;
  size_t pool_bytes = 0;
  char* ws = nullptr;
  // weights
  const void* embed = nullptr;
  const void* lm = nullptr;
  std::vector<const void*> wqkv, wo, wgu, wd;
  std::vector<const float*> aa, am;
  // MXFP8 / MXFP4 copies (workspace) used by the weight-streaming GEMV (calls of <= 2 rows)
  bool mx = false;
  int mx_fmt = 0;  // 1: MXFP8, 2: MXFP4
  struct MxMat { const void* codes = nullptr; const uint8_t* scales = nullptr; };
  std::vector<MxMat> mqkv, mo, mgu, md;
  MxMat mlm;
  // KV manager
  std::vector<int32_t> free_pages;
  std::vector<Seq> seqs;
  // host staging (pinned) for the per-call upload
  char* stage[kStageSlots] = {};
  hipEvent_t stage_ev[kStageSlots] = {};
  bool stage_used[kStageSlots] = {};
  int stage_cur = 0;
  size_t stage_bytes = 0;
  std::vector<int32_t> upl;  // host image of the upload
  // the running call: a chunk of consecutive positions of one sequence (prefill, resume), or -1
  int chunk_seq = -1, chunk_pos0 = -1;
  const int32_t* row_order = nullptr;  // device: batched decode rows, longest context first (this call only)
  // the running call's rows are positions run_pos, run_pos + 1, ... of sequence run_seq (else -1)
  int run_seq = -1, run_pos = -1;
  // last call
  int last_rows = 0;
  float* last_h = nullptr;
  dory_stats stats{};
  // per-role accounting and optional event timing
  RoleAcc acc[R_COUNT];
  bool timing = false;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<TimedRec> recs;
  std::string err;
  hipError_t herr = hipSuccess;
  // self-speculative decoding: counters and the phase-boundary events of one round
  dory_spec_stats spec{};
  hipEvent_t spec_ev[3] = {};

  template <typename P = char>
  P* W(size_t off) const { return reinterpret_cast<P*>(ws + off); }
};

namespace {

dory_status fail(dory_ctx* c, dory_status s, const char* fmt, ...) {
  if (c) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
  }
  return s;
}

// Record a launch; remember the first HIP error.
bool ok(dory_ctx* c, hipError_t e) {
  c->stats.kernel_launches++;
  if (e != hipSuccess && c->herr == hipSuccess) c->herr = e;
  return e == hipSuccess;
}

hipEvent_t next_event(dory_ctx* c) {
  if (c->ev_used == c->ev_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_used++];
}

// Accounts one launch of `role` (algorithmic bytes / flops) and, while timing
// is enabled, has the role's kernel dispatches record a HIP event pair at
// their start and end (hipExtLaunchKernelGGL), so the time excludes launch gaps.
struct Span {
  dory_ctx* c;
  int role;
  hipEvent_t a = nullptr, b = nullptr;
  Span(dory_ctx* cc, int r, double bytes, double flops) : c(cc), role(r) {
    c->acc[r].launches++;
    c->acc[r].bytes += bytes;
    c->acc[r].flops += flops;
    if (c->timing && !c->dry) {
      a = next_event(c);
      b = next_event(c);
      if (a && b) dory::g_launch_events = {a, b};
    }
  }
  ~Span() {
    dory::g_launch_events = {nullptr, nullptr};
    if (a && b) c->recs.push_back({role, a, b});
  }
};

bool is_full(const dory_ctx* c, int j) { return j % c->cfg.full_every == c->cfg.full_every - 1; }

int slot_of(const dory_ctx* c, int j, int t) {
  const dory_config& g = c->cfg;
  if (j < g.n_in) return j;
  if (j < g.n_in + g.n_rec) {
    if (c->kv_mode == DORY_KV_PER_LOOP) return g.n_in + (t - 1) * g.n_rec + (j - g.n_in);
    return j;
  }
  if (c->kv_mode == DORY_KV_PER_LOOP) return g.n_in + g.max_loops * g.n_rec + (j - g.n_in - g.n_rec);
  return j;
}

void recompute_capacity(dory_ctx* c) {
  c->n_slots = n_slots_for(c->cfg, c->kv_mode);
  c->page_el = page_elems(c->cfg);
  c->page_bytes = c->page_el * esize(c->cfg);
  c->recycle = recycling(c->cfg);
  slot_counts(c->cfg, c->kv_mode, &c->n_full_slots, &c->n_swa_slots);
  // class of every slot: walk the blocks and loops the way slot_of numbers them
  c->slot_class_idx.assign(c->n_slots, 0);
  {
    int nf = 0, ns = 0;
    const int nb = c->cfg.n_in + c->cfg.n_rec + c->cfg.n_out;
    const int loops = c->kv_mode == DORY_KV_PER_LOOP ? c->cfg.max_loops : 1;
    for (int t = 1; t <= loops; ++t)
      for (int j = 0; j < nb; ++j) {
        const bool rec = j >= c->cfg.n_in && j < c->cfg.n_in + c->cfg.n_rec;
        if (t > 1 && !rec) continue;
        const int sl = slot_of(c, j, t);
        c->slot_class_idx[sl] = full_block(c->cfg, j) ? nf++ : -(ns++) - 1;
      }
  }
  size_t fp = 0, sp = 0;
  split_pool(c->cfg, c->kv_mode, c->pool_bytes, &fp, &sp);
  c->pages_total = (int)std::min<size_t>(fp, (size_t)INT32_MAX);
  c->swa_pages_total = c->recycle ? (int)std::min<size_t>(sp, (size_t)INT32_MAX) : 0;
  c->free_pages.clear();
  for (int p = c->pages_total - 1; p >= 0; --p) c->free_pages.push_back(p);
  c->free_swa.clear();
  for (int p = c->swa_pages_total - 1; p >= 0; --p) c->free_swa.push_back(p);
}

// Cache region of layer slot (block j, loop t) and the page table its kernels follow.
char* slot_base(dory_ctx* c, int j, int t) {
  const int sl = slot_of(c, j, t);
  if (!c->recycle) return c->pool + (size_t)sl * c->pages_total * c->page_bytes;
  const int ci = c->slot_class_idx[sl];
  const size_t full_region = (size_t)c->n_full_slots * c->pages_total * c->page_bytes;
  if (ci >= 0) return c->pool + (size_t)ci * c->pages_total * c->page_bytes;
  return c->pool + full_region + (size_t)(-ci - 1) * c->swa_pages_total * c->page_bytes;
}
const int32_t* slot_ptab(dory_ctx* c, int j) {
  const int32_t* t = c->W<int32_t>(c->L.ptab);
  return (c->recycle && !full_block(c->cfg, j)) ? t + (size_t)c->cfg.max_seqs * c->L.max_pages : t;
}
// Entries of the page tables (the full-attention one, then the sliding-window one under recycling).
int ptab_entries(const dory_ctx* c) {
  return ((c->cfg.flags & DORY_FLAG_SWA_RECYCLE) ? 2 : 1) * c->cfg.max_seqs * c->L.max_pages;
}

// Index guard of block j's attention kernels: its page table's shape, the pages of the cache
// region its ids index, the RoPE table's rows and the device flag word.
dory::PageGuard slot_guard(dory_ctx* c, int j) {
  dory::PageGuard gd;
  gd.max_seqs = c->cfg.max_seqs;
  gd.pool_pages = (c->recycle && !full_block(c->cfg, j)) ? c->swa_pages_total : c->pages_total;
  gd.max_pos = c->cfg.max_model_len;
  gd.flags = c->W<int32_t>(c->L.err);
  return gd;
}

// Copy the host upload image to the device upload area (pinned ring, async).
bool stage_upload(dory_ctx* c, int n_ints) {
  if (n_ints > c->L.upload_ints) { c->herr = hipErrorInvalidValue; return false; }  // sized at create
  if (c->dry || n_ints == 0) return true;
  const size_t bytes = (size_t)n_ints * 4;
  const int s = c->stage_cur;
  c->stage_cur = (c->stage_cur + 1) % kStageSlots;
  if (c->stage_used[s]) {
    hipError_t e = hipEventSynchronize(c->stage_ev[s]);
    if (e != hipSuccess) { c->herr = e; return false; }
  }
  memcpy(c->stage[s], c->upl.data(), bytes);
  hipError_t e = hipMemcpyAsync(c->W(c->L.upload), c->stage[s], bytes, hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipEventRecord(c->stage_ev[s], c->stream);
  c->stage_used[s] = true;
  if (e != hipSuccess) { c->herr = e; return false; }
  return true;
}

// Key splits per (row, KV head) for split attention: enough workgroups to fill
// the chip with few serial steps per wave, at most kMaxSplits. The batched VALU kernel
// (more than kDecodeMfmaRows rows, taken longest context first) aims at 8192 workgroups:
// at 128 rows of 256..4096 tokens, targets of 2048 / 8192 / 16384 gave 6235 / 6600 / 6422
// tok/s at k = 2 (shorter splits shorten the tail; more of them cost merge work).
constexpr int kBatchedWorkTarget = 8192;
int choose_splits(const dory_ctx* c, int M, int keys, bool paged_kernel) {
  if (M > c->L.part_rows) return 1;
  const int target = paged_kernel && M > dory::kDecodeMfmaRows ? kBatchedWorkTarget : 2048;
  const int by_work = (target + M * c->cfg.n_kv_heads - 1) / (M * c->cfg.n_kv_heads);
  // MFMA decode kernel (few rows): one 32-key block per wave; VALU kernel: 16 pages per workgroup
  const int by_keys = !paged_kernel ? (keys + 63) / 64 : M <= dory::kDecodeMfmaRows ? (keys + 127) / 128
                                                                                    : (keys + 255) / 256;
  return std::max(1, std::min(std::min(by_work, by_keys), kMaxSplits));
}

// Attention geometry of one call: per KV head, the query-key pairs and the
// distinct keys the rows read, for full and for sliding-window layers.
struct Geom {
  double pairs_full = 0, pairs_swa = 0, keys_full = 0, keys_swa = 0;
  int max_ctx = 0;
  void add_chunk(int p0, int n, int W) {  // positions p0 .. p0+n-1 of one sequence
    for (int p = p0; p < p0 + n; ++p) {
      pairs_full += p + 1;
      pairs_swa += std::min(p + 1, W);
    }
    keys_full += p0 + n;
    keys_swa += p0 + n - std::max(0, p0 - W + 1);
    max_ctx = std::max(max_ctx, p0 + n);
  }
};

#define SPLITK c->W<float>(c->L.splitk), c->L.splitk_bytes

// Residual-stream bookkeeping of one forward pass. With a pending step
// (py != nullptr) the hidden rows are N(h + pa * (N(py) - h)), not yet
// materialised: the next weight-streaming GEMV applies it in its prologue
// (writing the result to `spare`, which then becomes h) or flush() runs it.
struct Flow {
  float* h;
  float* spare;
  const float* py = nullptr;
  const float* pa = nullptr;
};

void flush(dory_ctx* c, Flow& f, int M) {
  if (!f.py) return;
  const dory_config& g = c->cfg;
  if (!c->dry) {
    Span sp(c, R_RESID, (double)M * g.d_model * (12 + esize(g)) + 4.0 * g.d_model, 0);
    ok(c, dory::launch_residual(g.dtype, f.h, f.py, f.pa, c->W(c->L.hb), M, g.d_model, c->stream));
  } else {
    c->stats.kernel_launches++;
  }
  f.py = f.pa = nullptr;
}

// Decode rows few enough for the weight-streaming GEMV with the residual step
// folded into its prologue.
bool fused_residual_ok(const dory_ctx* c, int M, bool decode) {
  const dory_config& g = c->cfg;
  return decode && M <= 2 && g.dtype == DORY_BF16 && dory::gemv_residual_supported(g.d_model) &&
         dory::gemv_supported(g.n_heads * g.head_dim) && dory::gemv_supported(g.d_ff);
}

// Weight bytes per parameter a launch streams: MXFP8 (1 + 1/32) on the GEMV path, else the storage size.
double wbytes(const dory_ctx* c, int M) {
  if (c->mx && M <= 2) return (c->mx_fmt == 2 ? 0.5 : 1.0) + 1.0 / 32;
  return (double)esize(c->cfg);
}

// C = A . W^T through the MXFP8 GEMV (calls of <= 2 rows when the context holds MX weights) or launch_gemm.
// parts (may be NULL): as in launch_gemm, the split-K partials may be left in the split workspace.
hipError_t project(dory_ctx* c, bool dual, const void* A, const void* W, const dory_ctx::MxMat& mx, void* out, int M,
                   int N, int K, int* parts = nullptr) {
  if (parts) *parts = 0;
  if (c->mx && M <= 2 && dory::gemv_supported(K))
    return dory::launch_gemv(dual, A, mx.codes, mx.scales, out, M, N, K, c->stream, c->mx_fmt);
  return dory::launch_gemm(c->cfg.dtype, dual, A, W, out, M, N, K, SPLITK, c->stream, parts);
}

// One block application on M rows (hidden state per Flow; storage copy in hb when materialised).
void run_block(dory_ctx* c, int j, int t, int M, Flow& f, bool decode, const Geom& geo) {
  using namespace dory;
  const dory_config& g = c->cfg;
  const int dt = g.dtype, d = g.d_model, H = g.n_heads, Hk = g.n_kv_heads, dh = g.head_dim;
  const double es = (double)esize(g), Md = (double)M;
  const int nq = qkv_cols(g), hd = H * dh, F = g.d_ff;
  const bool full = is_full(c, j);
  c->stats.block_apps++;
  c->stats.sublayer_apps += 2;
  if (full) c->stats.full_apps++; else c->stats.swa_apps++;
  const double pairs = full ? geo.pairs_full : geo.pairs_swa;
  const double keys = full ? geo.keys_full : geo.keys_swa;
  const double resid_bytes = Md * d * (12 + es) + 4.0 * d;
  const int keys_max = full ? geo.max_ctx : std::min(geo.max_ctx, g.window);
  const bool paged = attn_decode_supported(dt, H, Hk, dh);
  // the attention kernel writes the call's keys / values itself: decode rows, and short chunks of
  // consecutive positions that one workgroup per split holds whole
  const bool fused_decode = paged && (decode || (c->run_seq >= 0 && M <= kDecodeMfmaRows && M <= 32 / (H / Hk)));
  const bool flash = !decode && dt == DORY_BF16 && dh == 128 && M > c->L.part_rows;
  const int splits = flash ? 1 : choose_splits(c, M, keys_max, paged);
  c->stats.max_attn_splits = std::max(c->stats.max_attn_splits, splits);
  const bool fres = fused_residual_ok(c, M, decode);
  if (c->dry) {
    c->stats.kernel_launches += (fres ? 4 : 6) + (fused_decode ? 1 : 2) + (splits > 1);
    if (fres) { f.py = f.pa = nullptr; }
    return;
  }
  void* hb = c->W(c->L.hb);
  float* qkv = c->W<float>(c->L.qkv);
  float* y = c->W<float>(c->L.y);
  const int32_t* rows = c->W<int32_t>(c->L.upload);
  const int32_t* ptab = slot_ptab(c, j);
  char* kv = slot_base(c, j, t);
  const dory::PageGuard gd = slot_guard(c, j);
#if DORY_CHECKED
  // the slot's whole cache region must lie inside the caller's pool
  if (kv < c->pool || kv + (size_t)gd.pool_pages * c->page_bytes > c->pool + c->pool_bytes) {
    ok(c, hipErrorInvalidValue);
    return;
  }
#endif
  hipStream_t st = c->stream;
  const double wb = wbytes(c, M);
  const bool gmx = c->mx && M <= 2;  // this call streams the MX weights
  if (f.py && fres) {
    Span sp(c, R_QKV, (double)nq * d * wb + Md * d * 12 + 4.0 * d + Md * nq * 4, 2.0 * Md * nq * d);
    ok(c, launch_gemv_residual(false, gmx ? c->mqkv[j].codes : c->wqkv[j], gmx ? c->mqkv[j].scales : nullptr, qkv, M,
                               nq, d, f.h, f.py, f.pa, f.spare, st, c->mx_fmt));
    std::swap(f.h, f.spare);
    f.py = f.pa = nullptr;
  } else {
    flush(c, f, M);
    Span sp(c, R_QKV, (double)nq * d * wb + Md * d * es + Md * nq * 4, 2.0 * Md * nq * d);
    ok(c, project(c, false, hb, c->wqkv[j], gmx ? c->mqkv[j] : dory_ctx::MxMat{}, qkv, M, nq, d));
  }
  if (!fused_decode) {
    Span sp(c, R_ROPE, Md * nq * 4 + Md * (hd + 2.0 * Hk * dh) * es, 0);
    ok(c, launch_rope_qk_kv(dt, qkv, rows, ptab, c->L.max_pages, c->W<float2>(c->L.rope), c->W(c->L.q), kv, M, H,
                            Hk, dh, c->page_el, decode ? -1 : c->chunk_seq, decode ? -1 : c->chunk_pos0, gd, st));
  }
  {
    // fused decode reads q/k/v from the projection output and writes the new key/value itself
    const double io = fused_decode ? Md * nq * 4 + Md * hd * es + Md * 2.0 * Hk * dh * es : 2.0 * Md * hd * es;
    Span sp(c, R_ATTN, keys * 2.0 * Hk * dh * es + io, 4.0 * dh * H * pairs);
    const int win = full ? 0 : g.window;
    if (paged && (decode || !flash)) {
      ok(c, launch_attn_decode(qkv, rows, ptab, c->L.max_pages, c->W<float2>(c->L.rope), kv, c->page_el, M, H, Hk,
                               win, g.attn_scale, splits, fused_decode ? 1 : 0, c->W(c->L.o), c->W<float>(c->L.part_ml),
                               c->W<float>(c->L.part_o), c->row_order, c->run_seq, c->run_pos, gd, st));
    } else if (flash) {
      ok(c, launch_attn_prefill(c->W(c->L.q), rows, ptab, c->L.max_pages, kv, c->page_el, M, H, Hk, win,
                                g.attn_scale, c->W(c->L.o), gd, st));
    } else {
      if (splits > 1) c->stats.kernel_launches++;
      ok(c, launch_attn_rows(dt, c->W(c->L.q), rows, ptab, c->L.max_pages, kv, c->page_el, M, H, Hk, dh, win,
                             g.attn_scale, splits, c->W(c->L.o), c->W<float>(c->L.part_ml), c->W<float>(c->L.part_o),
                             gd, st));
    }
  }
  // without the fused GEMV path, a split-K o / down product leaves its partials for the residual
  // kernel to sum (one launch and one y round trip fewer)
  int parts = 0;
  {
    Span sp(c, R_OPROJ, (double)d * hd * wb + Md * hd * es + Md * d * 4, 2.0 * Md * d * hd);
    ok(c, project(c, false, c->W(c->L.o), c->wo[j], gmx ? c->mo[j] : dory_ctx::MxMat{}, y, M, d, hd,
                  fres ? nullptr : &parts));
  }
  if (fres) {
    Span sp(c, R_GU, 2.0 * F * d * wb + Md * d * 12 + 4.0 * d + Md * F * es, 2.0 * Md * 2 * F * d);
    ok(c, launch_gemv_residual(true, gmx ? c->mgu[j].codes : c->wgu[j], gmx ? c->mgu[j].scales : nullptr,
                               c->W(c->L.z), M, 2 * F, d, f.h, y, c->aa[j], f.spare, st, c->mx_fmt));
    std::swap(f.h, f.spare);
  } else {
    {
      Span sp(c, R_RESID, resid_bytes, 0);
      ok(c, launch_residual(dt, f.h, parts > 1 ? c->W<float>(c->L.splitk) : y, c->aa[j], hb, M, d, st, parts));
    }
    Span sp(c, R_GU, 2.0 * F * d * wb + Md * d * es + Md * F * es, 2.0 * Md * 2 * F * d);
    ok(c, project(c, true, hb, c->wgu[j], gmx ? c->mgu[j] : dory_ctx::MxMat{}, c->W(c->L.z), M, 2 * F, d));
  }
  {
    Span sp(c, R_DOWN, (double)d * F * wb + Md * F * es + Md * d * 4, 2.0 * Md * d * F);
    ok(c, project(c, false, c->W(c->L.z), c->wd[j], gmx ? c->md[j] : dory_ctx::MxMat{}, y, M, d, F,
                  fres ? nullptr : &parts));
  }
  if (fres) {
    f.py = y;
    f.pa = c->am[j];
  } else {
    Span sp(c, R_RESID, resid_bytes, 0);
    ok(c, launch_residual(dt, f.h, parts > 1 ? c->W<float>(c->L.splitk) : y, c->am[j], hb, M, d, st, parts));
  }
}

// Whole forward pass over M rows whose (seq, pos) pairs are in the upload area.
// Leaves the final hidden rows in c->last_h and their storage copy in hb.
// What one forward call runs: the whole stack (FULL), or only the embedding, input stack and
// loop 1 (HEAD), or loops 2..k and the output stack for rows whose input-stack output and
// loop-1 state are given (RESUME). FULL and HEAD can copy those two states of their rows out.
struct FwdOpts {
  enum Phase { FULL, HEAD, RESUME } phase = FULL;
  float* cap_x = nullptr;
  float* cap_s1 = nullptr;
  const float* res_x = nullptr;
  const float* res_s1 = nullptr;
};

void run_forward(dory_ctx* c, const int32_t* tokens_dev, int M, bool decode, const Geom& geo,
                 const FwdOpts& o = FwdOpts()) {
  using namespace dory;
  const dory_config& g = c->cfg;
  const int dt = g.dtype, d = g.d_model;
  const double es = (double)esize(g), Md = (double)M;
  float* b[4] = {c->W<float>(c->L.buf[0]), c->W<float>(c->L.buf[1]), c->W<float>(c->L.buf[2]),
                 c->W<float>(c->L.buf[3])};
  void* hb = c->W(c->L.hb);
  auto copy_rows = [&](float* dst, const float* src) {
    if (c->dry) { c->stats.kernel_launches++; return; }
    ok(c, launch_copy_f32(dst, src, (size_t)M * d, c->stream));
  };
  // One launch per loop boundary: the pending sublayer step of the stack that just ended (if the
  // last block left one), s_t = N(.) and u_{t+1} = N(s_t + x) (launch_loop_step).
  auto loop_step = [&](Flow& fl, const float* xin, float* sout, float* hout, int mode) {
    const double bytes = Md * d * ((fl.py ? 12 : 4) + (mode == 1 ? 12 : mode == 2 ? 8 : 4) + es) + (fl.py ? 4.0 * d : 0);
    if (!c->dry) {
      Span sp(c, R_LOOPN, bytes, 0);
      ok(c, launch_loop_step(dt, fl.h, fl.py, fl.pa, xin, sout, hout, hb, M, d, mode, c->stream));
    } else {
      c->stats.kernel_launches++;
    }
    fl.py = fl.pa = nullptr;
  };
  float* x;
  Flow f{b[0], b[3]};
  float* rest[3];
  auto split_rest = [&]() {
    int nr = 0;
    for (float* p : b)
      if (p != x) rest[nr++] = p;
  };
  if (o.phase != FwdOpts::RESUME) {
    if (!c->dry) {
      Span sp(c, R_EMBED, Md * d * (2 * es + 4) + Md * 4, 0);
      ok(c, launch_embed(dt, tokens_dev, c->embed, g.vocab, d, M, b[0], hb, c->W<int32_t>(c->L.err), c->stream));
    } else {
      c->stats.kernel_launches++;
    }
    for (int j = 0; j < g.n_in; ++j) run_block(c, j, 1, M, f, decode, geo);
    x = f.h;  // input-stack output (its last sublayer step may still be pending)
    split_rest();
    // x materialised in place; u_1 = N(s_0 + x) with s_0 = x
    loop_step(f, nullptr, nullptr, rest[0], 0);
    if (o.cap_x) copy_rows(o.cap_x, x);
  } else {
    x = b[0];
    copy_rows(x, o.res_x);
    split_rest();
  }
  // the other three buffers hold h, s and the spare
  float* s = rest[1];
  f = Flow{rest[0], rest[2]};
  if (o.phase == FwdOpts::RESUME) {
    copy_rows(s, o.res_s1);
    // u_2 = N(s_1 + x)
    if (!c->dry) {
      Span sp(c, R_LOOPN, Md * d * (12 + es), 0);
      ok(c, launch_norm_sum(dt, s, x, f.h, nullptr, hb, M, d, c->stream));
    } else {
      c->stats.kernel_launches++;
    }
  }
  const int t_first = o.phase == FwdOpts::RESUME ? 2 : 1;
  const int t_last = o.phase == FwdOpts::HEAD ? 1 : c->k;
  for (int t = t_first; t <= t_last; ++t) {
    for (int j = g.n_in; j < g.n_in + g.n_rec; ++j) run_block(c, j, t, M, f, decode, geo);
    // s_t = N(F(u_t)); then u_{t+1} = N(s_t + x), or h continues as s_k after the last loop
    loop_step(f, x, s, f.h, t < t_last ? 1 : 2);
    if (t == 1 && o.cap_s1) copy_rows(o.cap_s1, s);
  }
  if (o.phase == FwdOpts::HEAD) {
    c->last_h = s;
    c->last_rows = M;
    return;
  }
  for (int j = g.n_in + g.n_rec; j < c->n_blocks; ++j) run_block(c, j, 1, M, f, decode, geo);
  flush(c, f, M);
  c->last_h = f.h;
  c->last_rows = M;
}

void lm_head(dory_ctx* c, int M, int rows, float* logits, int32_t* ids) {
  using namespace dory;
  const dory_config& g = c->cfg;
  if (c->dry) {
    c->stats.kernel_launches += 1 + (ids != nullptr);
    return;
  }
  const double es = (double)esize(g), V = g.vocab, d = g.d_model;
  const char* hb = c->W(c->L.hb) + (size_t)(M - rows) * g.d_model * esize(g);
  {
    Span sp(c, R_LM, V * d * wbytes(c, rows) + rows * d * es + rows * V * 4, 2.0 * rows * V * d);
    ok(c, project(c, false, hb, c->lm, c->mx && rows <= 2 ? c->mlm : dory_ctx::MxMat{}, logits, rows, g.vocab,
                  g.d_model));
  }
  if (ids) {
    Span sp(c, R_ARGMAX, rows * V * 4 + rows * 4.0, 0);
    ok(c, launch_argmax(logits, rows, g.vocab, ids, c->W(c->L.argmax), c->stream));
  }
}

bool valid_seq(const dory_ctx* c, int32_t id) { return id >= 0 && id < c->cfg.max_seqs; }

// Give seq the pages for positions [len, new_len) (the caller checked the free
// count) and append the page-table updates to the upload image.
void take_pages(dory_ctx* c, int sid, int new_len) {
  Seq& s = c->seqs[sid];
  const int want = (new_len + kPage - 1) / kPage;
  while ((int)s.pages.size() < want) {
    const int p = c->free_pages.back();
    c->free_pages.pop_back();
    c->upl.push_back(sid * c->L.max_pages + (int)s.pages.size());
    c->upl.push_back(p);
    s.pages.push_back(p);
  }
  if (!c->recycle) return;
  const int swa_table = c->cfg.max_seqs * c->L.max_pages;  // the sliding-window table follows the full one
  while ((int)s.swa_pages.size() < want) {
    const int p = c->free_swa.back();
    c->free_swa.pop_back();
    c->upl.push_back(swa_table + sid * c->L.max_pages + (int)s.swa_pages.size());
    c->upl.push_back(p);
    s.swa_pages.push_back(p);
  }
}

void release_pages_from(dory_ctx* c, Seq& s, int new_len) {
  const int keep = (new_len + kPage - 1) / kPage;
  while ((int)s.pages.size() > keep) {
    c->free_pages.push_back(s.pages.back());
    s.pages.pop_back();
  }
  while ((int)s.swa_pages.size() > keep) {
    if (s.swa_pages.back() >= 0) c->free_swa.push_back(s.swa_pages.back());
    s.swa_pages.pop_back();
  }
  s.swa_lo = std::min(s.swa_lo, (int)s.swa_pages.size());
}

// First position whose sliding-window keys a sequence of length len may still read: the next
// query's window, less the rollback reserve.
int swa_keep_from(const dory_ctx* c, int len) { return std::max(0, len - c->cfg.window + 1 - kSwaReserve); }

// Return the sliding-window pages that lie wholly before swa_keep_from(len). The device page
// table keeps their stale entries; no kernel reads below the window. Work already queued on the
// context's stream that reads them runs before any later call's kernels write them.
void recycle_swa(dory_ctx* c, Seq& s) {
  if (!c->recycle || !s.live) return;
  const int lo_page = std::min(swa_keep_from(c, s.len) / kPage, (int)s.swa_pages.size());
  for (; s.swa_lo < lo_page; ++s.swa_lo) {
    c->free_swa.push_back(s.swa_pages[s.swa_lo]);
    s.swa_pages[s.swa_lo] = -1;
  }
}

// Sliding-window pages a sequence needs to reach new_len.
int swa_need(const dory_ctx* c, const Seq& s, int new_len) {
  if (!c->recycle) return 0;
  return (new_len + kPage - 1) / kPage - (int)(s.live ? s.swa_pages.size() : 0);
}

int pages_in_use(const dory_ctx* c) { return c->pages_total - (int)c->free_pages.size(); }
int swa_pages_in_use(const dory_ctx* c) { return c->swa_pages_total - (int)c->free_swa.size(); }

}  // namespace

namespace {

dory_status prefill_impl(dory_ctx* c, int32_t sid, const int32_t* tokens_dev, int32_t n, int32_t logits_rows,
                         float* logits_dev, int32_t* ids_dev, const FwdOpts& o) {
  const bool head = o.phase == FwdOpts::HEAD;  // input stack and loop 1 only: no logits
  const int k_run = head ? 1 : c->k;
  if (!c) return DORY_E_INVALID;
  if (!valid_seq(c, sid)) return fail(c, DORY_E_INVALID, "seq_id %d outside 0..%d", sid, c->cfg.max_seqs - 1);
  if (n < 1 || n > c->cfg.max_tokens) return fail(c, DORY_E_INVALID, "n_tokens %d outside 1..%d", n, c->cfg.max_tokens);
  if (!head && (logits_rows < 1 || logits_rows > n))
    return fail(c, DORY_E_INVALID, "logits_rows %d outside 1..%d", logits_rows, n);
  if (!c->dry && (!tokens_dev || (!head && !logits_dev)))
    return fail(c, DORY_E_INVALID, "tokens_dev and logits_dev are required");
  Seq& s = c->seqs[sid];
  const int len = s.live ? s.len : 0;
  if ((int64_t)len + n > c->cfg.max_model_len)
    return fail(c, DORY_E_INVALID, "length %d + %d exceeds max_model_len %d", len, n, c->cfg.max_model_len);
  if (c->kv_mode == DORY_KV_PER_LOOP && s.live && len > 0 && s.min_loops() < k_run)
    return fail(c, DORY_E_STATE, "per-loop cache of seq %d holds %d loops, %d requested", sid, s.min_loops(), k_run);
  recycle_swa(c, s);
  const int need = (len + n + kPage - 1) / kPage - (int)(s.live ? s.pages.size() : 0);
  if (need > (int)c->free_pages.size())
    return fail(c, DORY_E_NOMEM, "KV pool exhausted: %d pages needed, %zu free", need, c->free_pages.size());
  const int need_swa = swa_need(c, s, len + n);
  if (need_swa > (int)c->free_swa.size())
    return fail(c, DORY_E_NOMEM, "sliding-window KV pages exhausted: %d needed, %zu free", need_swa,
                c->free_swa.size());
  // commit host state and build the upload: rows, then page-table updates
  if (!s.live) { s = Seq(); s.live = true; }
  c->upl.clear();
  for (int i = 0; i < n; ++i) { c->upl.push_back(sid); c->upl.push_back(len + i); }
  const size_t n_rows_ints = c->upl.size();
  take_pages(c, sid, len + n);
  const int n_upd = (int)(c->upl.size() - n_rows_ints) / 2;
  c->herr = hipSuccess;
  if (!stage_upload(c, (int)c->upl.size())) return fail(c, DORY_E_HIP, "upload failed: %s", hipGetErrorString(c->herr));
  if (!c->dry && n_upd) {
    Span sp(c, R_PTAB, 12.0 * n_upd, 0);
    ok(c, dory::launch_apply_updates(c->W<int32_t>(c->L.ptab), c->W<int32_t>(c->L.upload) + n_rows_ints, n_upd,
                                     ptab_entries(c), c->W<int32_t>(c->L.err), c->stream));
  }
  s.len = len + n;
  s.append_run(s.len, k_run);
  Geom geo;
  geo.add_chunk(len, n, c->cfg.window);
  c->chunk_seq = c->run_seq = sid;
  c->chunk_pos0 = c->run_pos = len;
  run_forward(c, tokens_dev, n, false, geo, o);
  c->chunk_seq = c->chunk_pos0 = c->run_seq = c->run_pos = -1;
  if (!head) lm_head(c, n, logits_rows, logits_dev, ids_dev);
  c->stats.calls++;
  if (c->herr != hipSuccess) return fail(c, DORY_E_HIP, "kernel launch failed: %s", hipGetErrorString(c->herr));
  return DORY_OK;
}

dory_status decode_impl(dory_ctx* c, int32_t n, const int32_t* seq_ids, const int32_t* tokens_dev, float* logits_dev,
                        int32_t* next_ids_dev, const FwdOpts& o) {
  if (!c) return DORY_E_INVALID;
  if (n < 1 || n > c->cfg.max_tokens || n > c->cfg.max_seqs)
    return fail(c, DORY_E_INVALID, "n_seqs %d outside 1..%d", n, std::min(c->cfg.max_tokens, c->cfg.max_seqs));
  if (!seq_ids) return fail(c, DORY_E_INVALID, "seq_ids_host is NULL");
  if (!c->dry && !tokens_dev) return fail(c, DORY_E_INVALID, "tokens_dev is NULL");
  if (!logits_dev && n > c->L.logit_rows) return fail(c, DORY_E_INVALID, "logits scratch holds %d rows", c->L.logit_rows);
  int need = 0, need_swa = 0;
  for (int i = 0; i < n; ++i) {
    const int sid = seq_ids[i];
    if (!valid_seq(c, sid) || !c->seqs[sid].live) return fail(c, DORY_E_INVALID, "seq %d is not live", sid);
    for (int j = 0; j < i; ++j)
      if (seq_ids[j] == sid) return fail(c, DORY_E_INVALID, "seq %d listed twice", sid);
    const Seq& s = c->seqs[sid];
    if (s.len + 1 > c->cfg.max_model_len) return fail(c, DORY_E_INVALID, "seq %d reached max_model_len", sid);
    if (c->kv_mode == DORY_KV_PER_LOOP && s.len > 0 && s.min_loops() < c->k)
      return fail(c, DORY_E_STATE, "per-loop cache of seq %d holds %d loops, %d requested", sid, s.min_loops(), c->k);
    need += (s.len + 1 + kPage - 1) / kPage - (int)s.pages.size();
  }
  for (int i = 0; i < n; ++i) recycle_swa(c, c->seqs[seq_ids[i]]);
  for (int i = 0; i < n; ++i) need_swa += swa_need(c, c->seqs[seq_ids[i]], c->seqs[seq_ids[i]].len + 1);
  if (need > (int)c->free_pages.size())
    return fail(c, DORY_E_NOMEM, "KV pool exhausted: %d pages needed, %zu free", need, c->free_pages.size());
  if (need_swa > (int)c->free_swa.size())
    return fail(c, DORY_E_NOMEM, "sliding-window KV pages exhausted: %d needed, %zu free", need_swa,
                c->free_swa.size());
  c->upl.clear();
  for (int i = 0; i < n; ++i) { c->upl.push_back(seq_ids[i]); c->upl.push_back(c->seqs[seq_ids[i]].len); }
  const size_t n_rows_ints = c->upl.size();
  for (int i = 0; i < n; ++i) take_pages(c, seq_ids[i], c->seqs[seq_ids[i]].len + 1);
  const int n_upd = (int)(c->upl.size() - n_rows_ints) / 2;
  // batched rows: the attention kernels take them longest context first, so that the short ones
  // fill the tail instead of a long one running alone at the end
  const bool ordered = n > dory::kDecodeMfmaRows;
  if (ordered) {
    std::vector<int32_t> ord(n);
    for (int i = 0; i < n; ++i) ord[i] = i;
    std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
      return c->seqs[seq_ids[a]].len > c->seqs[seq_ids[b]].len;
    });
    c->upl.insert(c->upl.end(), ord.begin(), ord.end());
  }
  c->herr = hipSuccess;
  if (!stage_upload(c, (int)c->upl.size())) return fail(c, DORY_E_HIP, "upload failed: %s", hipGetErrorString(c->herr));
  if (!c->dry && n_upd) {
    Span sp(c, R_PTAB, 12.0 * n_upd, 0);
    ok(c, dory::launch_apply_updates(c->W<int32_t>(c->L.ptab), c->W<int32_t>(c->L.upload) + n_rows_ints, n_upd,
                                     ptab_entries(c), c->W<int32_t>(c->L.err), c->stream));
  }
  Geom geo;
  for (int i = 0; i < n; ++i) {
    Seq& s = c->seqs[seq_ids[i]];
    geo.add_chunk(s.len, 1, c->cfg.window);
    s.len += 1;
    s.append_run(s.len, c->k);
  }
  c->row_order = ordered ? c->W<int32_t>(c->L.upload) + n_rows_ints + 2 * n_upd : nullptr;
  if (n == 1) {  // one row: its sequence and position are passed to the attention kernel directly
    c->run_seq = seq_ids[0];
    c->run_pos = c->seqs[seq_ids[0]].len - 1;
  }
  run_forward(c, tokens_dev, n, true, geo, o);
  c->row_order = nullptr;
  c->run_seq = c->run_pos = -1;
  if (o.phase != FwdOpts::HEAD) {  // HEAD: input stack and loop 1 only, no logits
    float* logits = logits_dev ? logits_dev : c->W<float>(c->L.logits);
    lm_head(c, n, n, logits, next_ids_dev);
  }
  c->stats.calls++;
  if (c->herr != hipSuccess) return fail(c, DORY_E_HIP, "kernel launch failed: %s", hipGetErrorString(c->herr));
  return DORY_OK;
}

// Loops 2..k, the output stack and the LM head for the last n positions of a sequence, from
// their input-stack output res_x and loop-1 state res_s1 (device, fp32 [n][d]); their input-stack
// and loop-1 KV must already be in the cache (self-speculative verify with reuse).
dory_status resume_impl(dory_ctx* c, int32_t sid, int32_t n, const float* res_x, const float* res_s1, float* logits_dev,
                        int32_t* ids_dev) {
  Seq& s = c->seqs[sid];
  if (!s.live || n < 1 || n > s.len || n > c->cfg.max_tokens) return fail(c, DORY_E_INVALID, "bad resume rows");
  const int pos0 = s.len - n;
  if (c->kv_mode == DORY_KV_PER_LOOP && pos0 > 0) {
    int m = 4;  // loops held by the positions before the resumed rows
    int start = 0;
    for (auto& r : s.runs) {
      if (start < pos0) m = std::min(m, r.second);
      start = r.first;
    }
    if (m < c->k) return fail(c, DORY_E_STATE, "per-loop cache of seq %d holds %d loops, %d requested", sid, m, c->k);
  }
  c->upl.clear();
  for (int i = 0; i < n; ++i) { c->upl.push_back(sid); c->upl.push_back(pos0 + i); }
  c->herr = hipSuccess;
  if (!stage_upload(c, (int)c->upl.size())) return fail(c, DORY_E_HIP, "upload failed: %s", hipGetErrorString(c->herr));
  s.trim_runs(pos0);
  s.append_run(s.len, c->k);
  Geom geo;
  geo.add_chunk(pos0, n, c->cfg.window);
  FwdOpts o;
  o.phase = FwdOpts::RESUME;
  o.res_x = res_x;
  o.res_s1 = res_s1;
  c->chunk_seq = c->run_seq = sid;
  c->chunk_pos0 = c->run_pos = pos0;
  run_forward(c, nullptr, n, false, geo, o);
  c->chunk_seq = c->chunk_pos0 = c->run_seq = c->run_pos = -1;
  lm_head(c, n, n, logits_dev, ids_dev);
  c->stats.calls++;
  if (c->herr != hipSuccess) return fail(c, DORY_E_HIP, "kernel launch failed: %s", hipGetErrorString(c->herr));
  return DORY_OK;
}

}  // namespace

// ===================================================================== C ABI

extern "C" {

const char* dory_status_string(int32_t s) {
  switch (s) {
    case DORY_OK: return "ok";
    case DORY_E_INVALID: return "invalid argument";
    case DORY_E_STATE: return "invalid state";
    case DORY_E_NOMEM: return "out of memory";
    case DORY_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dory_last_error(const dory_ctx* c) { return c ? c->err.c_str() : "context is NULL"; }

dory_status dory_query_sizes(const dory_config* cfg, int32_t kv_mode, int64_t kv_tokens, size_t* kv_pool_bytes,
                             size_t* workspace_bytes) {
  if (!check_config(cfg).empty()) return DORY_E_INVALID;
  if (kv_mode != DORY_KV_PER_LOOP && kv_mode != DORY_KV_LAST_LOOP) return DORY_E_INVALID;
  if (kv_tokens < 0 || !kv_pool_bytes || !workspace_bytes) return DORY_E_INVALID;
  const size_t pages = (size_t)((kv_tokens + kPage - 1) / kPage);
  const size_t pb = page_elems(*cfg) * esize(*cfg);
  *kv_pool_bytes = pages * n_slots_for(*cfg, kv_mode) * pb;
  if (recycling(*cfg)) {
    // full-attention slots for every token; sliding-window slots for what max_seqs sequences hold at once
    int nf, ns;
    slot_counts(*cfg, kv_mode, &nf, &ns);
    const size_t swa = std::min(pages, (size_t)cfg->max_seqs * swa_pages_per_seq(*cfg));
    *kv_pool_bytes = (pages * nf + swa * ns) * pb;
  }
  *workspace_bytes = make_layout(*cfg).total;
  return DORY_OK;
}

dory_status dory_create(const dory_config* cfg, const dory_weights* w, int32_t kv_mode, void* kv_pool,
                        size_t kv_bytes, void* workspace, size_t ws_bytes, void* stream, dory_ctx** out) {
  if (!out) return DORY_E_INVALID;
  *out = nullptr;
  if (!check_config(cfg).empty()) return DORY_E_INVALID;
  if (kv_mode != DORY_KV_PER_LOOP && kv_mode != DORY_KV_LAST_LOOP) return DORY_E_INVALID;
  const bool dry = (cfg->flags & DORY_FLAG_DRY_RUN) != 0;
  const Layout L = make_layout(*cfg);
  if (!dry) {
    if (!w || !kv_pool || !workspace) return DORY_E_INVALID;
    if (ws_bytes < L.total) return DORY_E_NOMEM;
    if ((reinterpret_cast<uintptr_t>(kv_pool) | reinterpret_cast<uintptr_t>(workspace)) % kAlign) return DORY_E_INVALID;
  }
  const int nb = cfg->n_in + cfg->n_rec + cfg->n_out;
  if (!dry) {
    if (!w->embed || !w->lm_head || !w->w_qkv || !w->w_o || !w->w_gu || !w->w_down || !w->alpha_attn || !w->alpha_mlp)
      return DORY_E_INVALID;
    for (int j = 0; j < nb; ++j)
      if (!w->w_qkv[j] || !w->w_o[j] || !w->w_gu[j] || !w->w_down[j] || !w->alpha_attn[j] || !w->alpha_mlp[j])
        return DORY_E_INVALID;
  }
  dory_ctx* c = new dory_ctx();
  c->cfg = *cfg;
  c->L = L;
  c->dry = dry;
  c->mx = (cfg->flags & (DORY_FLAG_MXFP8_GEMV | DORY_FLAG_MXFP4_GEMV)) != 0;
  c->mx_fmt = (cfg->flags & DORY_FLAG_MXFP4_GEMV) ? 2 : c->mx ? 1 : 0;
  c->kv_mode = kv_mode;
  c->n_blocks = nb;
  c->pool = static_cast<char*>(kv_pool);
  c->pool_bytes = kv_bytes;
  c->ws = static_cast<char*>(workspace);
  c->stream = static_cast<hipStream_t>(stream);
  c->seqs.resize(cfg->max_seqs);
  if (w) {
    c->embed = w->embed;
    c->lm = w->lm_head;
    for (int j = 0; j < nb && w->w_qkv; ++j) {
      c->wqkv.push_back(w->w_qkv[j]);
      c->wo.push_back(w->w_o[j]);
      c->wgu.push_back(w->w_gu[j]);
      c->wd.push_back(w->w_down[j]);
      c->aa.push_back(w->alpha_attn[j]);
      c->am.push_back(w->alpha_mlp[j]);
    }
  }
  recompute_capacity(c);
  c->upl.reserve(L.upload_ints);
  if (!dry) {
    c->stage_bytes = (size_t)L.upload_ints * 4;
    hipError_t e = hipSuccess;
    for (int i = 0; i < kStageSlots && e == hipSuccess; ++i) {
      e = hipHostMalloc(reinterpret_cast<void**>(&c->stage[i]), c->stage_bytes, hipHostMallocDefault);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = dory::launch_rope_table(c->W<float2>(L.rope), cfg->max_model_len, cfg->head_dim,
                                                      (double)cfg->rope_theta, c->stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->W(L.ptab), 0, (size_t)cfg->max_seqs * L.max_pages * 4, c->stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->W(L.err), 0, 4, c->stream);
    // unwritten cache slots hold zeros, never NaN bit patterns, so masked keys contribute 0 * v = 0
    if (e == hipSuccess) e = hipMemsetAsync(c->pool, 0, c->pool_bytes, c->stream);
    if (e == hipSuccess && c->mx) {
      // quantise every projection and the LM head into the workspace's MX area
      char* p = c->W(L.mx);
      auto quant = [&](const void* src, size_t rows, int cols) -> dory_ctx::MxMat {
        dory_ctx::MxMat m;
        m.codes = p;
        p += align_up(c->mx_fmt == 2 ? rows * cols / 2 : rows * cols);
        m.scales = reinterpret_cast<const uint8_t*>(p);
        const size_t sbytes = rows * (size_t)dory::mx_scale_row_bytes(cols);
        p += align_up(sbytes);
        if (e == hipSuccess) e = hipMemsetAsync(const_cast<uint8_t*>(m.scales), 0, sbytes, c->stream);
        if (e == hipSuccess)
          e = dory::launch_mx_quantize(src, (long long)rows, cols, const_cast<void*>(m.codes),
                                       const_cast<uint8_t*>(m.scales), true, c->stream, c->mx_fmt);
        return m;
      };
      const int d = cfg->d_model, hd = cfg->n_heads * cfg->head_dim, F = cfg->d_ff, nq = qkv_cols(*cfg);
      for (int j = 0; j < nb; ++j) {
        c->mqkv.push_back(quant(c->wqkv[j], nq, d));
        c->mo.push_back(quant(c->wo[j], d, hd));
        c->mgu.push_back(quant(c->wgu[j], 2 * (size_t)F, d));
        c->md.push_back(quant(c->wd[j], d, F));
      }
      c->mlm = quant(c->lm, cfg->vocab, d);
      if ((size_t)(p - c->W(L.mx)) > L.mx_bytes) e = hipErrorInvalidValue;  // layout bound (never expected)
    }
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) {
      dory_destroy(c);
      return DORY_E_HIP;
    }
  }
  *out = c;
  return DORY_OK;
}

void dory_destroy(dory_ctx* c) {
  if (!c) return;
  if (!c->dry) {
    (void)hipStreamSynchronize(c->stream);
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : c->spec_ev)
      if (e) (void)hipEventDestroy(e);
    for (int i = 0; i < kStageSlots; ++i) {
      if (c->stage[i]) (void)hipHostFree(c->stage[i]);
      if (c->stage_ev[i]) (void)hipEventDestroy(c->stage_ev[i]);
    }
  }
  delete c;
}

dory_status dory_set_loops(dory_ctx* c, int32_t k) {
  if (!c) return DORY_E_INVALID;
  if (k < 1 || k > c->cfg.max_loops) return fail(c, DORY_E_INVALID, "loop count %d outside 1..%d", k, c->cfg.max_loops);
  c->k = k;
  return DORY_OK;
}

dory_status dory_get_loops(const dory_ctx* c, int32_t* k) {
  if (!c || !k) return DORY_E_INVALID;
  *k = c->k;
  return DORY_OK;
}

dory_status dory_kv_mode(dory_ctx* c, int32_t mode) {
  if (!c) return DORY_E_INVALID;
  if (mode != DORY_KV_PER_LOOP && mode != DORY_KV_LAST_LOOP) return fail(c, DORY_E_INVALID, "unknown KV mode %d", mode);
  if (mode == c->kv_mode) return DORY_OK;
  for (auto& s : c->seqs)
    if (s.live) return fail(c, DORY_E_STATE, "KV mode can only change with no live sequence");
  c->kv_mode = mode;
  recompute_capacity(c);
  return DORY_OK;
}

dory_status dory_prefill(dory_ctx* c, int32_t sid, const int32_t* tokens_dev, int32_t n, int32_t logits_rows,
                         float* logits_dev, int32_t* ids_dev) {
  return prefill_impl(c, sid, tokens_dev, n, logits_rows, logits_dev, ids_dev, FwdOpts());
}

dory_status dory_decode(dory_ctx* c, int32_t n, const int32_t* seq_ids, const int32_t* tokens_dev, float* logits_dev,
                        int32_t* next_ids_dev) {
  return decode_impl(c, n, seq_ids, tokens_dev, logits_dev, next_ids_dev, FwdOpts());
}


dory_status dory_seq_truncate(dory_ctx* c, int32_t sid, int32_t new_len) {
  if (!c) return DORY_E_INVALID;
  if (!valid_seq(c, sid) || !c->seqs[sid].live) return fail(c, DORY_E_INVALID, "seq %d is not live", sid);
  Seq& s = c->seqs[sid];
  if (new_len < 0 || new_len > s.len) return fail(c, DORY_E_INVALID, "truncate to %d outside 0..%d", new_len, s.len);
  if (c->recycle && s.swa_lo > 0 && std::max(0, new_len - c->cfg.window + 1) < s.swa_lo * kPage)
    return fail(c, DORY_E_STATE, "truncate to %d needs sliding-window pages already recycled (held from %d)", new_len,
                s.swa_lo * kPage);
  release_pages_from(c, s, new_len);
  s.trim_runs(new_len);
  s.len = new_len;
  return DORY_OK;
}

dory_status dory_seq_release(dory_ctx* c, int32_t sid) {
  if (!c) return DORY_E_INVALID;
  if (!valid_seq(c, sid) || !c->seqs[sid].live) return fail(c, DORY_E_INVALID, "seq %d is not live", sid);
  Seq& s = c->seqs[sid];
  release_pages_from(c, s, 0);
  s = Seq();
  return DORY_OK;
}

dory_status dory_seq_len(const dory_ctx* c, int32_t sid, int32_t* len) {
  if (!c || !len || !valid_seq(c, sid)) return DORY_E_INVALID;
  *len = c->seqs[sid].live ? c->seqs[sid].len : -1;
  return DORY_OK;
}

dory_status dory_kv_bytes_in_use(const dory_ctx* c, size_t* bytes) {
  if (!c || !bytes) return DORY_E_INVALID;
  if (c->recycle)
    *bytes = ((size_t)pages_in_use(c) * c->n_full_slots + (size_t)swa_pages_in_use(c) * c->n_swa_slots) * c->page_bytes;
  else
    *bytes = (size_t)pages_in_use(c) * c->n_slots * c->page_bytes;
  return DORY_OK;
}

dory_status dory_get_stats(const dory_ctx* c, dory_stats* out) {
  if (!c || !out) return DORY_E_INVALID;
  *out = c->stats;
  out->n_slots = c->n_slots;
  out->pages_total = c->pages_total;
  out->pages_in_use = pages_in_use(c);
  out->swa_pages_total = c->swa_pages_total;
  out->swa_pages_in_use = swa_pages_in_use(c);
  int live = 0;
  for (auto& s : c->seqs) live += s.live;
  out->live_seqs = live;
  return DORY_OK;
}

namespace {
dory_status sample_args_ok(const float* logits_dev, int32_t rows, int32_t vocab, float temperature, float top_p,
                           const float* uniforms_dev, const int32_t* ids_dev) {
  if (rows < 0 || vocab < 1 || vocab > (1 << 23)) return DORY_E_INVALID;
  if (std::isnan(temperature) || std::isinf(temperature) || std::isnan(top_p)) return DORY_E_INVALID;
  if (rows > 0 && (!logits_dev || !uniforms_dev || !ids_dev)) return DORY_E_INVALID;
  return DORY_OK;
}
}  // namespace

dory_status dory_sample(const float* logits_dev, int32_t rows, int32_t vocab, float temperature, float top_p,
                        const float* uniforms_dev, int32_t* ids_dev, void* stream) {
  const dory_status a = sample_args_ok(logits_dev, rows, vocab, temperature, top_p, uniforms_dev, ids_dev);
  if (a != DORY_OK || rows == 0) return a;
  void* scratch = nullptr;
  size_t bytes = 0;
  hipError_t e = dory::sample_library_scratch(rows, vocab, &scratch, &bytes);
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return DORY_E_NOMEM;
  if (e == hipSuccess)
    e = dory::launch_sample(logits_dev, rows, vocab, temperature, top_p, uniforms_dev, ids_dev, scratch, bytes,
                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

dory_status dory_sample_static(const float* logits_dev, int32_t rows, int32_t vocab, float temperature, float top_p,
                               const float* uniforms_dev, int32_t* ids_dev, void* stream) {
  const dory_status a = sample_args_ok(logits_dev, rows, vocab, temperature, top_p, uniforms_dev, ids_dev);
  if (a != DORY_OK || rows == 0) return a;
  if (dory::sample_scratch_bytes(rows, vocab) > dory::kSampleStaticScratchBytes) return DORY_E_INVALID;
  void* scratch = nullptr;
  hipError_t e = dory::sample_static_scratch(&scratch);
  if (e == hipSuccess)
    e = dory::launch_sample(logits_dev, rows, vocab, temperature, top_p, uniforms_dev, ids_dev, scratch,
                            dory::kSampleStaticScratchBytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

size_t dory_sample_scratch_bytes(int32_t rows, int32_t vocab) {
  if (rows < 0 || vocab < 1 || vocab > (1 << 23)) return 0;
  return dory::sample_scratch_bytes(rows, vocab);
}

dory_status dory_quantize_mxfp8(const void* src_dev, int64_t rows, int32_t cols, void* codes_dev, void* scales_dev,
                                void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || (rows > 0 && (!src_dev || !codes_dev || !scales_dev)))
    return DORY_E_INVALID;
  if (reinterpret_cast<uintptr_t>(src_dev) % 16 || reinterpret_cast<uintptr_t>(codes_dev) % 16) return DORY_E_INVALID;
  hipError_t e =
      dory::launch_mx_quantize(src_dev, rows, cols, codes_dev, scales_dev, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

dory_status dory_quantize_mxfp4(const void* src_dev, int64_t rows, int32_t cols, void* codes_dev, void* scales_dev,
                                void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || (rows > 0 && (!src_dev || !codes_dev || !scales_dev)))
    return DORY_E_INVALID;
  if (reinterpret_cast<uintptr_t>(src_dev) % 16 || reinterpret_cast<uintptr_t>(codes_dev) % 16) return DORY_E_INVALID;
  hipError_t e = dory::launch_mx_quantize(src_dev, rows, cols, codes_dev, scales_dev, false,
                                          static_cast<hipStream_t>(stream), 2);
  return e == hipSuccess ? DORY_OK : DORY_E_HIP;
}

dory_status dory_device_flags(dory_ctx* c, int32_t* flags, int32_t reset) {
  if (!c || !flags) return DORY_E_INVALID;
  *flags = 0;
  if (c->dry) return DORY_OK;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, c->W(c->L.err), 4, hipMemcpyDeviceToHost, c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e == hipSuccess && reset) e = hipMemsetAsync(c->W(c->L.err), 0, 4, c->stream);
  if (e != hipSuccess) return fail(c, DORY_E_HIP, "reading device flags: %s", hipGetErrorString(e));
  *flags = v;
  return DORY_OK;
}

int32_t dory_checked_build(void) { return DORY_CHECKED ? 1 : 0; }

dory_status dory_debug_set_page(dory_ctx* c, int32_t seq_id, int32_t page_index, int32_t page_id, int32_t* old_id) {
  if (!c) return DORY_E_INVALID;
  if (!DORY_CHECKED) return fail(c, DORY_E_STATE, "dory_debug_set_page exists only in the checked build");
  if (c->dry) return fail(c, DORY_E_STATE, "dry-run context");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs || page_index < 0 || page_index >= c->L.max_pages)
    return fail(c, DORY_E_INVALID, "page-table entry (%d, %d) outside the table", seq_id, page_index);
  int32_t* e = c->W<int32_t>(c->L.ptab) + (size_t)seq_id * c->L.max_pages + page_index;
  int32_t v = 0;
  const int32_t nv = page_id;
  hipError_t h = hipMemcpyAsync(&v, e, 4, hipMemcpyDeviceToHost, c->stream);
  if (h == hipSuccess) h = hipStreamSynchronize(c->stream);
  if (h == hipSuccess) h = hipMemcpyAsync(e, &nv, 4, hipMemcpyHostToDevice, c->stream);
  if (h == hipSuccess) h = hipStreamSynchronize(c->stream);
  if (h != hipSuccess) return fail(c, DORY_E_HIP, "page-table write: %s", hipGetErrorString(h));
  if (old_id) *old_id = v;
  return DORY_OK;
}

dory_status dory_last_hidden(dory_ctx* c, float* dst, int32_t rows) {
  if (!c || !dst) return DORY_E_INVALID;
  if (rows < 1 || rows > c->last_rows) return fail(c, DORY_E_INVALID, "rows %d outside 1..%d", rows, c->last_rows);
  if (c->dry) return DORY_OK;
  const size_t d = c->cfg.d_model;
  hipError_t e = hipMemcpyAsync(dst, c->last_h + (size_t)(c->last_rows - rows) * d, (size_t)rows * d * 4,
                                hipMemcpyDeviceToDevice, c->stream);
  return e == hipSuccess ? DORY_OK : fail(c, DORY_E_HIP, "%s", hipGetErrorString(e));
}

dory_status dory_get_spec_stats(dory_ctx* c, dory_spec_stats* out, int32_t reset) {
  if (!c || !out) return DORY_E_INVALID;
  *out = c->spec;
  if (reset) c->spec = dory_spec_stats{};
  return DORY_OK;
}

dory_status dory_set_timing(dory_ctx* c, int32_t enable) {
  if (!c) return DORY_E_INVALID;
  c->timing = enable != 0;
  return DORY_OK;
}

dory_status dory_get_timing(dory_ctx* c, dory_kernel_time* out, int32_t max, int32_t* n, int32_t reset) {
  if (!c || !n || (max > 0 && !out)) return DORY_E_INVALID;
  if (!c->recs.empty()) {
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return fail(c, DORY_E_HIP, "%s", hipGetErrorString(e));
    for (const TimedRec& r : c->recs) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
        c->acc[r.role].ms += ms;
        c->acc[r.role].timed++;
      }
    }
    c->recs.clear();
    c->ev_used = 0;
  }
  int cnt = 0;
  for (int r = 0; r < R_COUNT; ++r) {
    if (c->acc[r].launches == 0) continue;
    if (cnt < max) {
      dory_kernel_time& o = out[cnt];
      memset(&o, 0, sizeof o);
      snprintf(o.name, sizeof o.name, "%s", kRoleName[r]);
      o.launches = c->acc[r].launches;
      o.bytes = c->acc[r].bytes;
      o.flops = c->acc[r].flops;
      o.timed_launches = c->acc[r].timed;
      o.total_ms = c->acc[r].ms;
    }
    ++cnt;
  }
  *n = cnt;
  if (reset)
    for (auto& a : c->acc) a = RoleAcc();
  return DORY_OK;
}

dory_status dory_spec_decode(dory_ctx* c, int32_t sid, int32_t last, int32_t n_new, int32_t gamma, int32_t k_draft,
                             int32_t k_verify, int32_t reuse, int32_t* out_ids, int32_t* n_out) {
  if (!c || !out_ids || !n_out) return DORY_E_INVALID;
  if (!valid_seq(c, sid) || !c->seqs[sid].live) return fail(c, DORY_E_INVALID, "seq %d is not live", sid);
  if (gamma < 1 || gamma > kMaxGamma || n_new < 1) return fail(c, DORY_E_INVALID, "gamma must be 1..16 and n_new >= 1");
  if (reuse && k_draft != 1) return fail(c, DORY_E_INVALID, "reusing the draft needs k_draft = 1");
  if (k_draft < 1 || k_draft > c->cfg.max_loops || k_verify < 1 || k_verify > c->cfg.max_loops)
    return fail(c, DORY_E_INVALID, "loop counts outside 1..%d", c->cfg.max_loops);
  if (gamma + 1 > c->cfg.max_tokens || gamma + 1 > c->L.logit_rows)
    return fail(c, DORY_E_INVALID, "gamma + 1 exceeds max_tokens or the logits scratch");
  if (c->dry) return fail(c, DORY_E_STATE, "self-speculative decoding needs the GPU");
  for (hipEvent_t& e : c->spec_ev)
    if (!e && hipEventCreate(&e) != hipSuccess) return fail(c, DORY_E_HIP, "hipEventCreate failed");
  const int k_saved = c->k;
  int32_t* toks = c->W<int32_t>(c->L.spec);   // [last, d1..d_gamma]
  int32_t* vids = toks + 32;                  // verifier ids [gamma+1]
  float* logits = c->W<float>(c->L.logits);
  int count = 0;
  dory_status st = DORY_OK;
  std::vector<int32_t> host(2 * (gamma + 1));
  while (count < n_new) {
    const int base = c->seqs[sid].len;
    hipError_t e = hipMemcpyAsync(toks, &last, 4, hipMemcpyHostToDevice, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);  // `last` lives on this host stack frame
    if (e != hipSuccess) { st = fail(c, DORY_E_HIP, "%s", hipGetErrorString(e)); break; }
    c->k = k_draft;
    (void)hipEventRecord(c->spec_ev[0], c->stream);
    const size_t dm = (size_t)c->cfg.d_model;
    float* sx = c->W<float>(c->L.spec_x);
    float* ss = c->W<float>(c->L.spec_s1);
    for (int i = 0; i < gamma && st == DORY_OK; ++i) {
      FwdOpts o;  // with reuse, keep each drafted row's x and loop-1 state
      if (reuse) { o.cap_x = sx + i * dm; o.cap_s1 = ss + i * dm; }
      st = decode_impl(c, 1, &sid, toks + i, nullptr, toks + i + 1, o);
    }
    if (st != DORY_OK) break;
    (void)hipEventRecord(c->spec_ev[1], c->stream);
    if (reuse) {
      // the draft's cache stays: input stack and loop 1 for d_gamma only, then loops 2..k_verify,
      // the output stack and the LM head for all gamma + 1 rows
      FwdOpts o;
      o.phase = FwdOpts::HEAD;
      o.cap_x = sx + gamma * dm;
      o.cap_s1 = ss + gamma * dm;
      // a one-token chunk is a decode step: the decode kernels (residual in the GEMV prologue,
      // RoPE in the attention kernel) run it, at the draft's loop count 1
      if ((st = decode_impl(c, 1, &sid, toks + gamma, nullptr, nullptr, o)) != DORY_OK) break;
      c->k = k_verify;
      if ((st = resume_impl(c, sid, gamma + 1, sx, ss, logits, vids)) != DORY_OK) break;
    } else {
      if ((st = dory_seq_truncate(c, sid, base)) != DORY_OK) break;
      c->k = k_verify;
      if ((st = dory_prefill(c, sid, toks, gamma + 1, gamma + 1, logits, vids)) != DORY_OK) break;
    }
    (void)hipEventRecord(c->spec_ev[2], c->stream);
    e = hipMemcpyAsync(host.data(), toks, (gamma + 1) * 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(host.data() + gamma + 1, vids, (gamma + 1) * 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) { st = fail(c, DORY_E_HIP, "%s", hipGetErrorString(e)); break; }
    const int32_t* d = host.data() + 1;          // drafts d1..d_gamma
    const int32_t* v = host.data() + gamma + 1;  // verifier ids after last, d1, ..., d_gamma
    int acc = 0;
    while (acc < gamma && d[acc] == v[acc]) ++acc;
    float t_draft = 0.f, t_verify = 0.f;
    if (hipEventElapsedTime(&t_draft, c->spec_ev[0], c->spec_ev[1]) == hipSuccess) c->spec.draft_ms += t_draft;
    if (hipEventElapsedTime(&t_verify, c->spec_ev[1], c->spec_ev[2]) == hipSuccess) c->spec.verify_ms += t_verify;
    c->spec.rounds++;
    c->spec.drafted += gamma;
    c->spec.accepted += acc;
    c->spec.produced += acc + 1;
    for (int i = 0; i < acc; ++i) out_ids[count++] = d[i];
    out_ids[count++] = v[acc];
    last = v[acc];
    if ((st = dory_seq_truncate(c, sid, base + acc + 1)) != DORY_OK) break;
  }
  c->k = k_saved;
  *n_out = count;
  return st;
}

}  // extern "C"
