"""ISD / R-ISD / AR decoders: the per-slot state machine (oracle; test infrastructure only).

What the pages fix (wiki note "Introspective Diffusion Language Models", *Key claims*
and *Method*; Agentic Commons post, *How Introspective Strided Decoding Works*):
one causal forward pass both proposes new tokens at MASK positions (distribution q)
and re-scores the previously generated, still pending tokens under the anchor
distribution p of the current pass; a pending token x is kept when u < p(x)/q(x);
the first rejected pending token ends the pass's accepted prefix and the next block
resumes from its position; the logit shift makes the first new token always accepted;
acceptance compounds geometrically along the block (the k-th position survives with
probability p^(k-1)); the tokens per forward are (2 + p + ... + p^(N-2)) / (2 - p^(N-1)).

Block layout (the reading taken here; the only one consistent with the 2N-1 query rows
of the pages' configurations, the TPF denominator 2 - p^(N-1) and the printed
efficiency TPF^2 / queries-per-forward = 1.22 at N = 4, p = 0.9).  Per slot, with
L = cached tokens and c = newest committed token (not yet cached):

  A-state  rows [c, v_1 .. v_{N-1}, MASK x (N-1)] at positions L .. L+2N-2
           for i = 1 .. N-1: p_i = softmax_T(row i-1);
             Accept(v_i, p_i, q_i, u(slot,t,L+i,0)) -> commit v_i
             else commit Resid(p_i, q_i, u(slot,t,L+i,1)); L += i; go to B; stop
           all accepted: z_1 = Cat(softmax_T(row N-1), u(slot,t,L+N,1)), commit it;
             proposals z_{j+1} from row N-1+j (j = 1..N-1) with u(slot,t,L+N+j,1);
             L += N; stay in A with pending z_2 .. z_N
  B-state  rows [c, MASK x (N-1)] at positions L .. L+N-1
           z_1 from row 0 with u(slot,t,L+1,1), committed; proposals z_{j+1} from row j
           with u(slot,t,L+1+j,1); L += 1; go to A
  after every pass the cache keeps positions < L (MASK and rejected rows never persist)

Proposals: 'sample' draws z ~ q = softmax_T(row); 'argmax' takes z = argmax(row) and
q := delta_z (so acceptance is u < p(z) and the residual is p with z removed).

Introspective acceptance meter (wiki note, TL;DR and Key claims: introspective consistency
is whether a model accepts, under argmax or sampling, its own previously generated tokens
when it re-evaluates them).  With meter=True every pending token - the model's own proposal
- is committed without a test, so the model's own generation is teacher-forced through the
passes, and the pass's anchor re-scores it: the slot accumulates the acceptance probability
min(1, p(x)/q(x)) (p(x) for an argmax proposal, [x == argmax p] at T = 0).
T = 0 is greedy: every decision is an argmax (accept iff v_i == argmax p_i).
N = 1 is plain AR decoding.  R-ISD is the same machine with the LoRA active on MASK
rows.  A slot stops after exactly max_new generated tokens (the prefill's token
counts); extra tokens of the last pass are dropped.
"""
from dataclasses import dataclass, field

import numpy as np

from . import philox, sampler
from .model import empty_cache, extend_cache
from .paged_kv import PagePool

STATE_A, STATE_B, STATE_DONE = "A", "B", "DONE"


@dataclass
class SlotState:
    slot: int
    committed: list                 # prompt + generated tokens
    prompt_len: int
    L: int                          # cached tokens
    c: int                          # newest committed token (uncached)
    pending: list = field(default_factory=list)
    pending_q: list = field(default_factory=list)   # (w float32 [V], S) or None (delta q)
    t: int = 1
    state: str = STATE_B
    max_new: int = 0
    n_gen: int = 0
    cache: list = None
    meter_sum: float = 0.0          # meter mode: sum of the pending tokens' acceptance probabilities
    meter_n: int = 0

    @property
    def generated(self):
        return self.committed[self.prompt_len:]


@dataclass
class Decision:
    kind: str        # 'accept', 'resid', 'z1', 'propose'
    position: int
    token: int
    margin: float    # distance to the nearest flip (see sampler); inf when none applies
    accepted: bool = True


@dataclass
class StepRecord:
    slot: int
    state: str
    ids: list
    positions: list
    tokens: list
    n_accept: int
    decisions: list
    logits: np.ndarray = None


@dataclass
class Outcome:
    tokens: list
    n_accept: int
    decisions: list
    new_L: int
    new_c: int
    new_state: str
    new_pending: list
    new_q: list
    meter_sum: float = 0.0
    meter_n: int = 0


def draw(logits, u, T):
    """Sample (or argmax when T = 0) from softmax_T(logits): (token, margin)."""
    if T == 0.0:
        return sampler.argmax(logits), sampler.top2_gap(logits)
    w, _, _ = sampler.weights_T(logits, T)
    return sampler.cat(w, u)


def propose_token(logits, u, T, propose):
    """(token, q-record, margin) for a MASK row; q-record None means q = delta(token)."""
    if T == 0.0 or propose == "argmax":
        return sampler.argmax(logits), None, sampler.top2_gap(logits)
    w, S, _ = sampler.weights_T(logits, T)
    j, margin = sampler.cat(w, u)
    return j, (w, S), margin


def decide(state, L, t, slot, pending, pending_q, logits, N, T, propose, seed, meter=False):
    """The decisions of one pass of one slot, given the pass's logits rows.

    state 'A': rows [c, v_1 .. v_{N-1}, MASK x (N-1)]; 'B': rows [c, MASK x (N-1)].
    pending_q[i] is (w, S) of the MASK row that proposed pending[i], or None (delta q).
    Returns an Outcome (tokens committed in order, accepted count, decisions with margins,
    and the slot's next L, c, state, pending tokens and their q records).
    meter: commit every pending token untested and sum their acceptance probabilities.
    """
    u = lambda pos, purpose: philox.uniform(seed, slot, t, pos, purpose)
    dec, tokens = [], []
    n_acc = 0
    msum, mn = 0.0, 0
    if state == STATE_A:
        for i in range(1, N):
            v = pending[i - 1]
            row = logits[i - 1]
            qrec = pending_q[i - 1] if pending_q else None
            if T == 0.0:
                ok, margin = (v == sampler.argmax(row)), sampler.top2_gap(row)
                if meter:
                    msum += 1.0 if ok else 0.0
            else:
                w, S, _ = sampler.weights_T(row, T)
                px = float(w[v]) / S
                qx = 1.0 if qrec is None else float(qrec[0][v]) / qrec[1]
                if meter:
                    msum += min(1.0, px / qx)
                else:
                    ok, margin = sampler.accept(px, qx, u(L + i, philox.PURPOSE_ACCEPT))
            if meter:
                ok, margin, mn = True, float("inf"), mn + 1
            dec.append(Decision("accept", L + i, v, margin, ok))
            if ok:
                tokens.append(v)
                n_acc += 1
                continue
            # first rejection: residual resample at position L+i, restart from there
            if T == 0.0:
                r, rm = sampler.argmax(row), sampler.top2_gap(row)
            else:
                p = w.astype(np.float64) / S
                if qrec is None:
                    q = np.zeros_like(p)
                    q[v] = 1.0
                else:
                    q = qrec[0].astype(np.float64) / qrec[1]
                r, rm = sampler.resid_draw(p, q, u(L + i, philox.PURPOSE_DRAW))
            dec.append(Decision("resid", L + i, r, rm))
            tokens.append(r)
            return Outcome(tokens, n_acc, dec, L + i, r, STATE_B, [], [])
        z1, m1 = draw(logits[N - 1], u(L + N, philox.PURPOSE_DRAW), T)
        dec.append(Decision("z1", L + N, z1, m1))
        tokens.append(z1)
        new_pending, new_q = [], []
        for j in range(1, N):
            z, qrec, mz = propose_token(logits[N - 1 + j], u(L + N + j, philox.PURPOSE_DRAW), T, propose)
            dec.append(Decision("propose", L + N + j, z, mz))
            new_pending.append(z)
            new_q.append(qrec)
        return Outcome(tokens, n_acc, dec, L + N, z1, STATE_A, new_pending, new_q, msum, mn)
    z1, m1 = draw(logits[0], u(L + 1, philox.PURPOSE_DRAW), T)
    dec.append(Decision("z1", L + 1, z1, m1))
    tokens.append(z1)
    new_pending, new_q = [], []
    for j in range(1, N):
        z, qrec, mz = propose_token(logits[j], u(L + 1 + j, philox.PURPOSE_DRAW), T, propose)
        dec.append(Decision("propose", L + 1 + j, z, mz))
        new_pending.append(z)
        new_q.append(qrec)
    return Outcome(tokens, n_acc, dec, L + 1, z1, STATE_A, new_pending, new_q)


class Decoder:
    def __init__(self, model, N, temperature, propose="sample", seed=1,
                 page_size=16, n_pages=1 << 20, keep_logits=False, meter=False):
        assert N >= 1
        self.meter = bool(meter)
        self.m = model
        self.spec = model.spec
        self.N = int(N)
        self.T = float(temperature)
        self.propose = propose
        self.seed = int(seed)
        self.pool = PagePool(n_pages, page_size)
        self.slots = {}
        self.keep_logits = keep_logits
        self.use_lora = model.lora is not None

    def _u(self, slot, t, pos, purpose):
        return philox.uniform(self.seed, slot, t, pos, purpose)

    def _draw(self, logits, u):
        return draw(logits, u, self.T)

    # ---- prefill ---------------------------------------------------------
    def prefill(self, slots, prompts, max_new):
        """AR prefill of each prompt; returns the first generated token per slot.

        Page order: first, slot by slot in call order, free the slot's old pages and
        reserve the prompt's; then forward and draw; last, free the pages of slots that
        are already finished (max_new <= 1), in call order.
        """
        out = []
        for slot, prompt in zip(slots, prompts):
            self.pool.truncate(slot, 0)
            self.pool.reserve(slot, len(prompt))
        for slot, prompt, mx in zip(slots, prompts, max_new):
            prompt = [int(x) for x in prompt]
            L0 = len(prompt)
            logits, kv = self.m.forward(prompt, np.arange(L0), empty_cache(self.spec))
            z1, _ = self._draw(logits[-1], self._u(slot, 0, L0, philox.PURPOSE_DRAW))
            st = SlotState(slot=slot, committed=prompt + [z1], prompt_len=L0, L=L0, c=z1,
                           t=1, state=STATE_B, max_new=int(mx), n_gen=1,
                           cache=extend_cache(empty_cache(self.spec), kv, L0))
            if st.n_gen >= st.max_new:
                st.state = STATE_DONE
            self.slots[slot] = st
            out.append(z1)
        for slot in slots:
            if self.slots[slot].state == STATE_DONE:
                self.pool.truncate(slot, 0)
        return out

    # ---- one pass --------------------------------------------------------
    def rows_of(self, st):
        N, MASK = self.N, self.spec.mask_id
        if st.state == STATE_A:
            ids = [st.c] + list(st.pending) + [MASK] * (N - 1)
        else:
            ids = [st.c] + [MASK] * (N - 1)
        is_mask = np.array([i == MASK for i in ids])
        return ids, is_mask

    def step(self):
        """One ISD pass over every live slot (ascending slot order). Returns {slot: StepRecord}."""
        live = sorted(s for s, st in self.slots.items() if st.state in (STATE_A, STATE_B))
        rows = {}
        for s in live:
            st = self.slots[s]
            ids, is_mask = self.rows_of(st)
            rows[s] = (ids, is_mask)
            self.pool.reserve(s, st.L + len(ids))
        recs = {}
        for s in live:
            recs[s] = self._step_slot(self.slots[s], *rows[s])
        for s in live:
            st = self.slots[s]
            self.pool.truncate(s, st.L if st.state != STATE_DONE else 0)
        return recs

    def _step_slot(self, st, ids, is_mask):
        N, t, L, slot = self.N, st.t, st.L, st.slot
        pos = L + np.arange(len(ids))
        logits, kv = self.m.forward(ids, pos, st.cache, is_mask=is_mask if self.use_lora else None)
        state_before = st.state
        out = decide(st.state, L, t, slot, st.pending, st.pending_q, logits, N, self.T, self.propose, self.seed,
                     meter=self.meter)
        st.meter_sum += out.meter_sum
        st.meter_n += out.meter_n
        tokens, n_acc, dec = out.tokens, out.n_accept, out.decisions
        new_L, new_c, new_state = out.new_L, out.new_c, out.new_state
        new_pending, new_q = out.new_pending, out.new_q

        # the KV of c and of the accepted pending tokens persists; the rest is rolled back
        keep = new_L - L
        st.cache = extend_cache(st.cache, kv, keep)
        room = st.max_new - st.n_gen
        tokens = tokens[:room]
        st.committed.extend(tokens)
        st.n_gen += len(tokens)
        st.L, st.c, st.t = new_L, new_c, t + 1
        st.pending, st.pending_q, st.state = new_pending, new_q, new_state
        if st.n_gen >= st.max_new:
            st.state = STATE_DONE
            st.pending, st.pending_q = [], []
        return StepRecord(slot, state_before, list(ids), list(pos), tokens, n_acc, dec,
                          logits if self.keep_logits else None)

    def run(self, max_steps=1 << 30):
        steps = 0
        while steps < max_steps and any(st.state != STATE_DONE for st in self.slots.values()):
            self.step()
            steps += 1
        return steps


def ar_greedy_reference(model, prompt, n_new):
    """Plain AR greedy decoding by full recomputation (no cache, no blocks): the
    definition the ISD greedy decoder must reproduce."""
    seq = [int(x) for x in prompt]
    for _ in range(n_new):
        logits, _ = model.forward(seq, np.arange(len(seq)), empty_cache(model.spec))
        seq.append(sampler.argmax(logits[-1]))
    return seq[len(prompt):]
