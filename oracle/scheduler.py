"""Pure-Python model of the step scheduler over the block allocator (test
infrastructure: only tests/ may import it).

Policy, from the pages (cited by page title and section):

* Iteration-level scheduling: after every step, finished requests leave and
  free their blocks, queued requests are admitted into the room that made,
  and when memory runs short a request is preempted ("(2) vLLM Internals
  ...", "2. Continuous Batching").
* A step has a single token budget and no separate prefill and decode
  phases; a request is described by two counters, the tokens it holds and
  the tokens whose KV has been computed. Requests already running are
  served first, each with the difference of its two counters (a decode
  step needs one token); queued requests share whatever budget remains. A
  queued prompt is granted the smaller of its uncomputed tokens and the
  remaining budget, further capped by a long-prefill threshold if set. With chunked
  prefill switched off, a prompt that does not fit what is left stops the
  walk and waits ("vLLM: what PagedAttention turned into", "The scheduler,
  and what it has to balance now").
* Preemption by recompute: when blocks cannot be found, a request's blocks
  are freed, its computed count is set to zero and it goes to the front of
  the waiting queue; a step that had to preempt admits no new request
  ("vLLM: what PagedAttention turned into", "Preemption, and the path that
  got deleted"). Since freeing a hashed block does not drop its hash, a
  preempted request readmitted soon enough can reattach its own cached
  prefix (same section).

Readings where the pages are silent:

* The request preempted is the one admitted last (the tail of the running
  list); if that is the request being scheduled, it is preempted itself
  and the running walk stops. A running request is walked in admission
  order and the walk stops when the budget is spent.
* The long-prefill threshold caps every request's share of a step (a
  running request in the middle of its prompt included); 0 means no cap.
  max_num_seqs (0: no cap) bounds the running list.
* A token's KV is computed in the step that schedules it; a step that
  brings a request's computed count up to its token count samples one new
  token (the last position's output), which is appended to the request
  and computed in a later step. The request finishes when it holds
  max_new_tokens generated tokens; its blocks are freed then.
* At admission, with prefix caching on, the request's tokens are looked up
  and the cached full blocks attached (at most all tokens but one, so a
  step always has a position to sample from); they count as computed.
* A request whose tokens (all but the last sampled one) need more blocks
  than the pool holds is refused when it is queued: it could never finish.
* A request is admitted only if its lookup hits plus new blocks fit the
  free queue (checked before anything changes), so a failed admission
  leaves the allocator untouched; the waiting walk stops there.
* The step's token ids are recorded for hashing after the step has run
  (update), in scheduled order.
"""
from __future__ import annotations

import collections
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

from oracle.allocator import BLOCK, AllocatorModel, OutOfBlocks


@dataclass
class Request:
    req_id: int
    prompt: List[int]
    max_new_tokens: int
    extra_key: int = 0
    output: List[int] = field(default_factory=list)
    computed: int = 0
    preemptions: int = 0

    @property
    def tokens(self) -> List[int]:
        return self.prompt + self.output

    @property
    def num_tokens(self) -> int:
        return len(self.prompt) + len(self.output)


@dataclass
class Scheduled:
    req_id: int
    start: int          # first position computed this step (= computed before)
    num_new: int        # positions start .. start + num_new - 1
    samples: bool       # the step completes the request's tokens: one is sampled
    slots: List[int]


@dataclass
class Plan:
    scheduled: List[Scheduled]
    cow_pairs: List[tuple]
    preempted: List[int]

    @property
    def num_tokens(self) -> int:
        return sum(s.num_new for s in self.scheduled)


class SchedulerModel:
    def __init__(self, alloc: AllocatorModel, token_budget: int, long_prefill_threshold: int = 0,
                 chunked_prefill: bool = True, max_num_seqs: int = 0):
        if token_budget < 1:
            raise ValueError("token budget must be positive")
        self.alloc = alloc
        self.budget = token_budget
        self.threshold = long_prefill_threshold
        self.chunked = chunked_prefill
        self.max_seqs = max_num_seqs
        self.requests: Dict[int, Request] = {}
        self.waiting: collections.deque = collections.deque()
        self.running: List[int] = []
        self.finished: List[int] = []
        self.last_plan: Optional[Plan] = None

    def add_request(self, req_id: int, prompt: Sequence[int], max_new_tokens: int,
                    extra_key: int = 0) -> None:
        if req_id in self.requests:
            raise KeyError("request exists")
        if len(prompt) < 1 or max_new_tokens < 1:
            raise ValueError("empty prompt or nothing to generate")
        need = -(-(len(prompt) + max_new_tokens - 1) // BLOCK)
        if need > self.alloc.num_blocks - 1:
            raise OutOfBlocks("request needs more blocks than the pool holds")
        self.requests[req_id] = Request(req_id, [int(t) for t in prompt], int(max_new_tokens),
                                        int(extra_key))
        self.waiting.append(req_id)

    # ------------------------------------------------------------ one step
    def _share(self, r: Request, left: int) -> int:
        n = min(r.num_tokens - r.computed, left)
        if self.threshold > 0:
            n = min(n, self.threshold)
        return n

    def _preempt(self, rid: int) -> None:
        r = self.requests[rid]
        self.alloc.free_seq(rid)
        r.computed = 0
        r.preemptions += 1
        self.waiting.appendleft(rid)

    def schedule(self) -> Plan:
        if self.last_plan is not None:
            raise RuntimeError("the previous plan has not been updated")
        left = self.budget
        out: List[Scheduled] = []
        pairs: List[tuple] = []
        preempted: List[int] = []
        i = 0
        while i < len(self.running) and left > 0:
            rid = self.running[i]
            r = self.requests[rid]
            n = self._share(r, left)
            placed = None
            while placed is None:
                try:
                    placed = self.alloc.append(rid, n)
                except OutOfBlocks:
                    victim = self.running.pop()
                    self._preempt(victim)
                    preempted.append(victim)
                    if victim == rid:
                        break
            if placed is None:
                break
            slots, p = placed
            out.append(Scheduled(rid, r.computed, n, r.computed + n == r.num_tokens, slots))
            pairs += p
            left -= n
            i += 1
        if not preempted:
            while self.waiting and left > 0 and (self.max_seqs <= 0 or len(self.running) < self.max_seqs):
                rid = self.waiting[0]
                r = self.requests[rid]
                toks = r.tokens
                cached, revived = self.alloc.lookup_cached(toks, r.extra_key, r.num_tokens - 1)
                need = r.num_tokens - cached
                n = min(need, left)
                if self.threshold > 0:
                    n = min(n, self.threshold)
                if not self.chunked and n < need:
                    break
                new_blocks = -(-(cached + n) // BLOCK) - cached // BLOCK
                if revived + new_blocks > self.alloc.num_free():
                    break
                got = self.alloc.add_cached(rid, toks, r.extra_key, r.num_tokens - 1)
                assert got == cached
                slots, p = self.alloc.append(rid, n)
                r.computed = cached
                self.waiting.popleft()
                self.running.append(rid)
                out.append(Scheduled(rid, cached, n, cached + n == r.num_tokens, slots))
                pairs += p
                left -= n
        self.last_plan = Plan(out, pairs, preempted)
        return self.last_plan

    def remove_request(self, req_id: int) -> None:
        """Drop a request in any state (dequeue, abort with its blocks freed,
        or release a finished one)."""
        if self.last_plan is not None:
            raise RuntimeError("a plan is pending")
        if req_id not in self.requests:
            raise KeyError("no such request")
        if req_id in self.running:
            self.alloc.free_seq(req_id)
            self.running.remove(req_id)
        elif req_id in self.waiting:
            self.waiting.remove(req_id)
        elif req_id in self.finished:
            self.finished.remove(req_id)
        del self.requests[req_id]

    def update(self, sampled: Sequence[int]) -> List[int]:
        """The step ran: record the computed tokens' ids, advance the counts,
        append one sampled token (in plan order) to each request the plan
        marks as sampling, and finish requests that are complete. Returns the
        finished request ids."""
        plan = self.last_plan
        if plan is None:
            raise RuntimeError("no plan to update")
        want = sum(1 for s in plan.scheduled if s.samples)
        if len(sampled) != want:
            raise ValueError("expected %d sampled tokens" % want)
        k = 0
        done = []
        for s in plan.scheduled:
            r = self.requests[s.req_id]
            self.alloc.record_tokens(s.req_id, r.tokens[s.start:s.start + s.num_new])
            r.computed = s.start + s.num_new
            if s.samples:
                r.output.append(int(sampled[k]))
                k += 1
                if len(r.output) >= r.max_new_tokens:
                    done.append(s.req_id)
        for rid in done:
            self.alloc.free_seq(rid)
            self.running.remove(rid)
            self.finished.append(rid)
        self.last_plan = None
        return done
