"""CPU oracle of the looped nGPT forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module. The product path (the HIP library and its
binding) never imports, calls or links it, and this module imports nothing
from the product package. Inputs (weights, token ids) are passed in by the
caller.

Arithmetic: numpy float64. For bf16 model shapes the values are rounded to
bfloat16 (from float32, round-to-nearest-even) at the storage points the bf16
configuration names: GEMM input activations, the attention queries and the KV
cache, the attention output and the SwiGLU product. Weights arrive already
bf16-exact. Everything else (the residual stream, norms, softmax, logits) stays
float64. For fp32 shapes nothing is rounded.

Sources (web pages on Dory1.0-4B; cited by title and section):
  [onedev-how]   onedev.kr summary "Dory1.0-4B는 반복 횟수로 추론 연산과 정확도를
                 조절한다", section "어떻게 동작하나" (how it works): nGPT backbone;
                 input/recurrent/output stacks; the loop update s0 = x,
                 u_t = N(s_{t-1} + x), s_t = N(F(u_t)); no adapter, no extra
                 residual; s_k goes to the output stack and LM head; 3:1
                 sliding-window:full attention; 72/112/192 layer applications.
  [onedev-limits] same page, section "전제와 한계" (assumptions and limits):
                 last-loop KV caching overwrites earlier loops' cache; queries of
                 earlier loops then see the final loop's KV.
  [secrett-terms] secrett2633 review "[논문리뷰] Dory1.0-4B: A Looped
                 Normalized-GPT", section 1 (key terms): nGPT L2-normalises its
                 data; last-loop KV keeps a k-independent footprint.
  [lucas-struct] lucasainews article "NVIDIA, 루프 구조 4B 모델 Dory1.0-4B 4가지
                 정밀도로 공개", section "층을 되풀이하는 구조" (repeated-layer
                 structure): I/R/O stacks of 8/20/8, input re-injected every
                 loop, per-loop vs last-loop KV.
  [trawl-kv]     trawling.dev digest "NVIDIA, 반복 연산형 4B 언어 모델 Dory 공개",
                 section "KV 캐시와 실행 환경" (KV cache and runtime).
The pages fix neither the block's sublayer form nor its shapes; those come
from the model configuration (per-dimension alpha, SwiGLU, per-head q/k
L2-norm, RoPE theta 1e4). Readings of points the pages leave open are marked
READING below.

Parity status: every function here is pinned by tests against closed forms,
invariants, brute force or hand-worked fixtures, except the end-to-end logits
of a full-size model, which no page prints (parity unpinned beyond the pins).
"""
from __future__ import annotations

import numpy as np

PER_LOOP = "per_loop"
LAST_LOOP = "last_loop"
MAX_LOOPS = 4


# --------------------------------------------------------------------------
# Elementary operations
# --------------------------------------------------------------------------

def bf16_round(a) -> np.ndarray:
    """Value -> float32 -> bfloat16 (round to nearest even) -> float64."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def l2_normalize(v) -> np.ndarray:
    """N(v) = v / ||v||_2 over the last axis [secrett-terms; onedev-how].

    READING: the pages give no epsilon; a zero vector is an error here.
    """
    v = np.asarray(v, dtype=np.float64)
    ss = np.sum(v * v, axis=-1, keepdims=True)
    if not np.all(ss > 0.0):
        raise FloatingPointError("L2 normalisation of a zero vector")
    return v / np.sqrt(ss)


def ngpt_residual(h, y, alpha) -> np.ndarray:
    """Normalised residual step of a sublayer: h <- N(h + alpha * (N(y) - h))."""
    return l2_normalize(h + alpha * (l2_normalize(y) - h))


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary embedding of x [T, heads, dh] at absolute positions [T].

    READING: half-split pairs (i, i + dh/2) rotated by angle pos * theta^(-2i/dh),
    the angle and its cosine/sine taken in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dh)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def silu(z) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def attend(q, K, V, positions, window, n_heads, n_kv_heads, scale) -> np.ndarray:
    """Causal GQA attention of queries q [T, H, dh] at `positions` over cache K/V [L, Hkv, dh].

    Query at position p sees keys j with p - window < j <= p (sliding window) or
    0 <= j <= p (window None: full attention). Query head h reads KV head
    floor(h / (H / Hkv)). Weights are softmax_j(scale * q . k_j).
    """
    T = q.shape[0]
    group = n_heads // n_kv_heads
    out = np.empty((T, n_heads, V.shape[-1]), dtype=np.float64)
    for i in range(T):
        p = int(positions[i])
        lo = 0 if window is None else max(0, p - window + 1)
        for g in range(n_kv_heads):
            heads = slice(g * group, (g + 1) * group)   # the query heads that read KV head g
            k = K[lo:p + 1, g, :]                        # [n, dh]
            v = V[lo:p + 1, g, :]
            s = scale * (q[i, heads] @ k.T)              # [group, n]
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=1, keepdims=True)
            out[i, heads] = w @ v
    return out


# --------------------------------------------------------------------------
# Model
# --------------------------------------------------------------------------

class _Seq:
    """KV state of one sequence: per cache slot, K and V rows for every position."""

    def __init__(self, n_kv_heads, head_dim):
        self.len = 0
        self.hk = n_kv_heads
        self.dh = head_dim
        self.K = {}
        self.V = {}
        self.written = {}

    def ensure(self, slot, n):
        if slot not in self.K:
            cap = max(16, n)
            self.K[slot] = np.full((cap, self.hk, self.dh), np.nan)
            self.V[slot] = np.full((cap, self.hk, self.dh), np.nan)
            self.written[slot] = np.zeros(cap, dtype=bool)
        cap = self.K[slot].shape[0]
        if n > cap:
            new = max(n, 2 * cap)
            for store, fill in ((self.K, np.nan), (self.V, np.nan)):
                grown = np.full((new, self.hk, self.dh), fill)
                grown[:cap] = store[slot]
                store[slot] = grown
            w = np.zeros(new, dtype=bool)
            w[:cap] = self.written[slot]
            self.written[slot] = w


class OracleModel:
    """Looped nGPT forward with paged-cache semantics reduced to their meaning.

    A call processes one chunk of consecutive positions of one sequence. In each
    block application the chunk's keys/values are written to the block's cache
    slot first, then every query of the chunk reads that slot over its masked
    range. Slots: input and output blocks own one slot each; a recurrent block
    owns one slot per loop in per-loop mode and a single, overwritten slot in
    last-loop mode [lucas-struct; trawl-kv; onedev-limits].
    """

    def __init__(self, shape, weights, kv_mode: str = PER_LOOP, loops: int = 1, gemv_weights: str = "bf16"):
        """gemv_weights = "mxfp8" / "mxfp4": calls that process at most 2 rows (decode of one or
        two sequences, prefill chunks of one or two tokens) use the projection and LM-head weights
        quantised to MXFP8 / MXFP4 and dequantised (oracle.mx); other calls use the weights as
        given."""
        self.s = shape
        self.bf16 = shape.dtype == "bf16"
        self.E = np.asarray(weights.embed, dtype=np.float64)
        self.Wlm = np.asarray(weights.lm_head, dtype=np.float64)
        self.blocks = []
        for blk in weights.blocks:
            self.blocks.append({k: np.asarray(v, dtype=np.float64) for k, v in blk.items()})
        if gemv_weights not in ("bf16", "mxfp8", "mxfp4"):
            raise ValueError(gemv_weights)
        self.mx = gemv_weights != "bf16"
        self.blocks_mx, self.Wlm_mx = [], None
        if self.mx:
            from .mx import dequantize_mxfp4, dequantize_mxfp8, quantize_mxfp4, quantize_mxfp8
            if gemv_weights == "mxfp8":
                dq = lambda w: dequantize_mxfp8(*quantize_mxfp8(w))  # noqa: E731
            else:
                dq = lambda w: dequantize_mxfp4(*quantize_mxfp4(w))  # noqa: E731
            for blk in self.blocks:
                self.blocks_mx.append({k: (dq(v) if k.startswith("w") else v) for k, v in blk.items()})
            self.Wlm_mx = dq(self.Wlm)
        if kv_mode not in (PER_LOOP, LAST_LOOP):
            raise ValueError(kv_mode)
        self.kv_mode = kv_mode
        self.k = 1
        self.set_loops(loops)
        self.seqs = {}
        self.counts = {"block": 0, "sublayer": 0, "full": 0, "swa": 0}

    # -- knobs ------------------------------------------------------------
    def set_loops(self, k: int):
        if not (1 <= int(k) <= MAX_LOOPS):
            raise ValueError("loop count must be 1..4")
        self.k = int(k)

    def set_kv_mode(self, mode: str):
        if self.seqs:
            raise RuntimeError("KV mode can only change with no live sequences")
        if mode not in (PER_LOOP, LAST_LOOP):
            raise ValueError(mode)
        self.kv_mode = mode

    def is_full(self, j: int) -> bool:
        """READING: physical block j is full attention iff j % 4 == 3 (3:1 SWA:full)."""
        return j % self.s.full_every == self.s.full_every - 1

    def slot(self, j: int, t: int):
        s = self.s
        if s.n_in <= j < s.n_in + s.n_rec and self.kv_mode == PER_LOOP:
            return (j, t)
        return (j, 0)

    def n_slots(self) -> int:
        return len({self.slot(j, t) for j in range(self.s.n_blocks) for t in range(1, self.k + 1)})

    # -- pieces -----------------------------------------------------------
    def _act(self, a):
        return bf16_round(a) if self.bf16 else np.asarray(a, dtype=np.float64)

    def _block(self, h, j, t, seq: _Seq, pos, mx=False):
        s = self.s
        W = self.blocks_mx[j] if mx else self.blocks[j]
        T = h.shape[0]
        H, Hk, dh = s.n_heads, s.n_kv_heads, s.head_dim
        # attention sublayer
        a = self._act(h)
        q = (a @ W["wq"].T).reshape(T, H, dh)
        k = (a @ W["wk"].T).reshape(T, Hk, dh)
        v = (a @ W["wv"].T).reshape(T, Hk, dh)
        qh = self._act(l2_normalize(rope(q, pos, s.rope_theta)))
        kh = self._act(l2_normalize(rope(k, pos, s.rope_theta)))
        v = self._act(v)
        sl = self.slot(j, t)
        end = int(pos[-1]) + 1
        seq.ensure(sl, end)
        seq.K[sl][pos] = kh
        seq.V[sl][pos] = v
        seq.written[sl][pos] = True
        lo = 0 if self.is_full(j) else max(0, int(pos[0]) - s.window + 1)
        if not seq.written[sl][lo:end].all():
            raise RuntimeError(f"slot {sl} read before it was written")
        o = attend(qh, seq.K[sl], seq.V[sl], pos, None if self.is_full(j) else s.window,
                   H, Hk, s.scale)
        y = self._act(o.reshape(T, H * dh)) @ W["wo"].T
        h = ngpt_residual(h, y, W["alpha_attn"])
        # MLP sublayer
        a = self._act(h)
        z = self._act(silu(a @ W["wg"].T) * (a @ W["wu"].T))
        y = z @ W["wd"].T
        h = ngpt_residual(h, y, W["alpha_mlp"])
        self.counts["block"] += 1
        self.counts["sublayer"] += 2
        self.counts["full" if self.is_full(j) else "swa"] += 1
        return h

    def forward_chunk(self, seq: _Seq, tokens, pos0: int, trace=None, mx=False):
        """Hidden states after the output stack for one chunk [onedev-how]."""
        pos = pos0 + np.arange(len(tokens))
        x = self.input_stack(seq, tokens, pos, mx)
        if trace is not None:
            trace["x"] = x
        st = self.core_loops(seq, x, x, 1, pos, trace, mx)   # s_0 = x
        return self.output_stack(seq, st, pos, mx)

    def input_stack(self, seq: _Seq, tokens, pos, mx=False):
        """Embedding and the input stack: x."""
        h = self.E[np.asarray(tokens, dtype=np.int64)]
        for j in range(self.s.n_in):
            h = self._block(h, j, 1, seq, pos, mx)
        return h

    def core_loops(self, seq: _Seq, x, st, t_first: int, pos, trace=None, mx=False, t_last=None):
        """Loops t_first..t_last (default k) of the recurrent core from state st = s_{t_first - 1}:
        u_t = N(s_{t-1} + x), s_t = N(F(u_t)). Returns s_{t_last}."""
        s = self.s
        for t in range(t_first, (self.k if t_last is None else t_last) + 1):
            u = l2_normalize(st + x)             # u_t = N(s_{t-1} + x)
            h = u
            for j in range(s.n_in, s.n_in + s.n_rec):
                h = self._block(h, j, t, seq, pos, mx)
            st = l2_normalize(h)                 # s_t = N(F(u_t))
            if trace is not None:
                trace.setdefault("u", []).append(u)
                trace.setdefault("s", []).append(st)
        return st

    def output_stack(self, seq: _Seq, st, pos, mx=False):
        h = st
        for j in range(self.s.n_in + self.s.n_rec, self.s.n_blocks):
            h = self._block(h, j, 1, seq, pos, mx)
        return h

    def lm_head(self, h, mx=False):
        """fp64 logits of the final hidden rows; ids = argmax over the float32-rounded logits,
        lowest id on ties (the kernel decides in float32)."""
        logits = self._act(h) @ (self.Wlm_mx if mx else self.Wlm).T
        ids = np.argmax(logits.astype(np.float32), axis=-1).astype(np.int32)
        return logits, ids

    # -- calls ------------------------------------------------------------
    def _check_loops_for(self, seq: _Seq):
        if self.kv_mode == PER_LOOP and seq.len > 0:
            for j in range(self.s.n_in, self.s.n_in + self.s.n_rec):
                for t in range(1, self.k + 1):
                    w = seq.written.get((j, t))
                    if w is None or not w[:seq.len].all():
                        raise RuntimeError("per-loop sequence lacks KV for the requested loop count")

    def prefill(self, seq_id: int, tokens, logits_rows: int = 1, trace=None):
        seq = self.seqs.get(seq_id)
        if seq is None:
            seq = self.seqs[seq_id] = _Seq(self.s.n_kv_heads, self.s.head_dim)
        self._check_loops_for(seq)
        mx = self.mx and len(tokens) <= 2
        h = self.forward_chunk(seq, tokens, seq.len, trace, mx)
        seq.len += len(tokens)
        self.last_hidden = h
        logits, ids = self.lm_head(h[len(tokens) - logits_rows:], mx)
        return logits, ids

    def decode(self, seq_ids, tokens):
        logits, ids, hid = [], [], []
        mx = self.mx and len(seq_ids) <= 2
        for sid, tok in zip(seq_ids, tokens):
            seq = self.seqs[int(sid)]
            self._check_loops_for(seq)
            h = self.forward_chunk(seq, [int(tok)], seq.len, mx=mx)
            seq.len += 1
            lg, i = self.lm_head(h, mx)
            logits.append(lg[0])
            ids.append(i[0])
            hid.append(h[0])
        self.last_hidden = np.array(hid)
        return np.array(logits), np.array(ids, dtype=np.int32)

    def truncate(self, seq_id: int, new_len: int):
        seq = self.seqs[seq_id]
        if not (0 <= new_len <= seq.len):
            raise ValueError("truncate past the current length")
        for sl in seq.written:
            seq.written[sl][new_len:] = False
            seq.K[sl][new_len:] = np.nan
            seq.V[sl][new_len:] = np.nan
        seq.len = new_len

    def head_rows(self, seq_id: int, tokens):
        """Input stack and loop 1 only, for a chunk appended to the sequence (its KV written in
        those slots): returns (x, s_1)."""
        seq = self.seqs[seq_id]
        pos = seq.len + np.arange(len(tokens))
        x = self.input_stack(seq, tokens, pos)
        s1 = self.core_loops(seq, x, x, 1, pos, t_last=1)
        seq.len += len(tokens)
        return x, s1

    def resume_rows(self, seq_id: int, pos0: int, x, s1, logits_rows: int):
        """Loops 2..k, the output stack and the LM head for the rows at positions pos0.. whose x
        and s_1 are given (their input-stack and loop-1 KV already in the cache)."""
        seq = self.seqs[seq_id]
        pos = pos0 + np.arange(len(x))
        st = self.core_loops(seq, np.asarray(x), np.asarray(s1), 2, pos)
        h = self.output_stack(seq, st, pos)
        self.last_hidden = h
        return self.lm_head(h[len(x) - logits_rows:])

    def release(self, seq_id: int):
        del self.seqs[seq_id]

    def seq_len(self, seq_id: int) -> int:
        return self.seqs[seq_id].len


# --------------------------------------------------------------------------
# Drivers built only from the calls above
# --------------------------------------------------------------------------

def greedy(model: OracleModel, seq_id: int, prompt, n_steps: int):
    """Prefill the prompt, then n_steps greedy decode steps. Returns (ids[n+1], logits[n+1, V])."""
    lg, ids = model.prefill(seq_id, prompt, 1)
    out_ids = [int(ids[0])]
    out_lg = [lg[0]]
    for _ in range(n_steps):
        lg, ids = model.decode([seq_id], [out_ids[-1]])
        out_ids.append(int(ids[0]))
        out_lg.append(lg[0])
    return np.array(out_ids, dtype=np.int32), np.array(out_lg)


def self_speculative(model: OracleModel, seq_id: int, prompt, n_tokens: int,
                     gamma: int = 4, k_draft: int = 1, k_verify: int = 4):
    """Self-speculative greedy decoding [onedev-limits]: draft gamma tokens with k_draft
    loops, verify them in one chunk with k_verify loops, keep the longest agreeing prefix
    plus the verifier's own next token, and roll the cache back to what was kept.

    READING: drafting decodes last, d1..d_{gamma-1}; the verify chunk is
    [last, d1..d_gamma] with logits for every row; the cache is truncated to the
    start of the draft before verifying.
    Returns the ids produced after the prompt (at least n_tokens of them).
    """
    model.set_loops(k_verify)
    _, ids = model.prefill(seq_id, prompt, 1)
    out = [int(ids[0])]
    while len(out) < n_tokens:
        base = model.seq_len(seq_id)
        last = out[-1]
        model.set_loops(k_draft)
        drafts = []
        tok = last
        for _ in range(gamma):
            _, i = model.decode([seq_id], [tok])
            tok = int(i[0])
            drafts.append(tok)
        model.truncate(seq_id, base)
        model.set_loops(k_verify)
        _, v = model.prefill(seq_id, [last] + drafts, gamma + 1)
        n_acc = 0
        while n_acc < gamma and drafts[n_acc] == int(v[n_acc]):
            n_acc += 1
        out.extend(drafts[:n_acc])
        out.append(int(v[n_acc]))
        model.truncate(seq_id, base + n_acc + 1)
    return np.array(out, dtype=np.int32)


def self_speculative_reuse(model: OracleModel, seq_id: int, prompt, n_tokens: int,
                           gamma: int = 4, k_verify: int = 4):
    """Self-speculative greedy decoding with a k = 1 draft whose work the verify pass reuses
    [onedev-limits]. Under the chunk semantics, a drafted row's input-stack output x, its loop-1
    state s_1 and the KV both write are what the verify chunk would compute again (the input
    stack and loop 1 see the same keys either way, in both KV modes), so the verify pass keeps
    the draft's cache, runs the input stack and loop 1 only for the one row the draft never ran
    (d_gamma), and runs loops 2..k_verify, the output stack and the LM head for all gamma + 1
    rows from the saved x and s_1. In exact arithmetic this equals self_speculative with
    k_draft = 1. Returns the ids produced after the prompt (at least n_tokens of them)."""
    model.set_loops(k_verify)
    _, ids = model.prefill(seq_id, prompt, 1)
    out = [int(ids[0])]
    while len(out) < n_tokens:
        base = model.seq_len(seq_id)
        last = out[-1]
        model.set_loops(1)
        xs, s1s, drafts = [], [], []
        tok = last
        for _ in range(gamma):
            tr = {}
            _, i = model.prefill(seq_id, [tok], 1, trace=tr)   # a one-token chunk: one decode step
            xs.append(tr["x"][0])
            s1s.append(tr["s"][0][0])
            tok = int(i[0])
            drafts.append(tok)
        x_l, s1_l = model.head_rows(seq_id, [drafts[-1]])
        model.set_loops(k_verify)
        _, v = model.resume_rows(seq_id, base, np.array(xs + [x_l[0]]), np.array(s1s + [s1_l[0]]), gamma + 1)
        n_acc = 0
        while n_acc < gamma and drafts[n_acc] == int(v[n_acc]):
            n_acc += 1
        out.extend(drafts[:n_acc])
        out.append(int(v[n_acc]))
        model.truncate(seq_id, base + n_acc + 1)
    return np.array(out, dtype=np.int32)
