"""Oracle round plan: active cells, ordered key lists and the slot ring.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows WF = "Wave Forcing: Towards Speed-of-Light Streaming Video
Generation" (arXiv 2611.00859):

* §2, Eq. 2 -- the wavefront state set: at most S denoising inputs plus the
  store, so a round is at most S+1 wide (anchor and history not counted).
* §3.1, Eq. 3 -- cell (i, s) runs in round k = i + s; the active denoising
  stages A_k and the store condition 0 <= k-S < N_chunk.
* §3.1, Eq. 4 -- query stage s reads active stage j iff j >= s.
* §3.1, Eq. 5 -- ordered context: anchor, bounded clean history, live store,
  then denoising K/V by increasing stage (self first).
* §4.2, Eq. 10 -- per-stage key count N_s = N_prefix + (S - s) N_C.
* App. B.2, Eq. 13 -- fixed attention slots, double-buffered over rounds.
* App. B.3 -- N_chunk + S rounds; store page promoted to history after the
  round; first clean chunk kept as a persistent anchor whose unrotated key is
  re-rotated when the window shifts; the store's prefix budget differs from
  the denoisers'.

Readings where the page leaves a step open (each is also listed with its
reason in the design notes):

* W counts the clean-history pages a denoising query reads; anchor and live
  store are separate terms of Eq. 5 and are not counted in W.
* Store history budget: every query group gets the same token budget of
  (W + S + 2) chunks.  Denoisers spend S of it on denoising chunks, the store
  spends 1 (its self chunk), so the store reads W + S history pages.  A
  config may instead give the store an explicit window (``W_store >= 0``).
* Windows: a group with window Wg reads clean chunks
  c in [max(A, k-S-Wg), k-S-1], oldest first (A = 1 if the anchor is on).
  The retained list is the max(W, W_store) newest clean chunks.
* Anchor: chunk 0, present from round S+1 on (chunk 0 is the live store in
  round S, where its raw K/V is captured).  Never repeated in history.
* Anchor position when the window slides: the anchor sits immediately before
  the oldest retained page, i.e. first frame F * max(0, k - S - Wmax - 1).
* Slots (closed-form ring, R = Wmax + 2): anchor -> k mod 2; clean chunk c ->
  2 + (c mod R); denoising stage j of round k -> 2 + R + (k mod 2) S + j.
  Round k+1 never writes a slot that round k reads.
* Rolling-Forcing comparison mask: every active denoising chunk reads every
  active denoising chunk, ordered by increasing stage; the store is unchanged.
* Inactive cells (fill/drain) contribute no keys at all.
* Unbounded requests (``n_chunk <= 0``): WF §1 and App. B.8 describe a
  continuous stream whose attention storage does not grow with its length.
  Such a request has no last chunk, so every chunk i >= 0 exists: after the
  fill every round is full width and there is no drain.  Its plan of round k
  equals the plan of any bounded request with more than k chunks.
"""

from dataclasses import dataclass

ANCHOR, HISTORY, STORE, DENOISE = 0, 1, 2, 3
KIND_NAMES = {ANCHOR: "A", HISTORY: "H", STORE: "St", DENOISE: "D"}
MASK_WAVE, MASK_ROLLING = 0, 1


@dataclass(frozen=True)
class Config:
    """Round shape.  ``W_store < 0`` selects the shared-budget reading."""

    S: int
    W: int
    W_store: int
    anchor: int
    n_chunk: int
    F: int
    Hh: int
    Ww: int
    n_heads: int
    head_dim: int
    n_layers: int
    mask: int = MASK_WAVE
    rope_theta: float = 10000.0

    @property
    def n_c(self) -> int:
        """Tokens per chunk: F latent frames of Hh x Ww patches."""
        return self.F * self.Hh * self.Ww

    @property
    def w_store(self) -> int:
        return self.W + self.S if self.W_store < 0 else self.W_store

    @property
    def w_max(self) -> int:
        return max(self.W, self.w_store)

    @property
    def ring(self) -> int:
        return self.w_max + 2

    @property
    def n_slots(self) -> int:
        return 4 + self.w_max + 2 * self.S

    @property
    def unbounded(self) -> bool:
        return self.n_chunk <= 0

    @property
    def n_rounds(self) -> int:
        """WF App. B.3: N_chunk + S rounds including fill and drain."""
        if self.unbounded:
            raise ValueError("an unbounded request has no last round")
        return self.n_chunk + self.S


def chunk_active(cfg: Config, i: int) -> bool:
    return i >= 0 and (cfg.unbounded or i < cfg.n_chunk)


def denoise_active(cfg: Config, k: int):
    """A_k of WF §3.1 (Eq. 3): stages s < S whose chunk k - s exists."""
    return [s for s in range(cfg.S) if chunk_active(cfg, k - s)]


def store_active(cfg: Config, k: int) -> bool:
    """WF §3.1: the store at (k - S, S) runs iff 0 <= k - S < N_chunk."""
    return chunk_active(cfg, k - cfg.S)


def anchor_present(cfg: Config, k: int) -> bool:
    """Anchor (chunk 0) is readable once chunk 0 has been stored (round S)."""
    return cfg.anchor == 1 and k >= cfg.S + 1


def anchor_capture(cfg: Config, k: int) -> bool:
    """Raw K/V of chunk 0 is kept in the round that stores chunk 0."""
    return cfg.anchor == 1 and k == cfg.S


def anchor_frame0(cfg: Config, k: int) -> int:
    """First frame position the anchor is rotated to in round k."""
    return cfg.F * max(0, k - cfg.S - cfg.w_max - 1)


def history_chunks(cfg: Config, k: int, window: int):
    """Clean chunks a group with history window ``window`` reads, oldest first."""
    lo = max(cfg.anchor, k - cfg.S - window)
    hi = k - cfg.S - 1
    return list(range(lo, hi + 1)) if hi >= lo else []


def clean_slot(cfg: Config, c: int) -> int:
    return 2 + (c % cfg.ring)


def denoise_slot(cfg: Config, k: int, j: int) -> int:
    return 2 + cfg.ring + (k % 2) * cfg.S + j


def anchor_slot(cfg: Config, k: int) -> int:
    return k % 2


def cell_slot(cfg: Config, k: int, s: int) -> int:
    """Slot receiving the K/V page that cell (k - s, s) publishes."""
    return clean_slot(cfg, k - cfg.S) if s == cfg.S else denoise_slot(cfg, k, s)


def key_entries(cfg: Config, k: int, s: int):
    """Ordered context of query stage s in round k (WF §3.1, Eq. 5).

    Returns a list of (kind, chunk, slot).  Empty if the cell is inactive.
    """
    S = cfg.S
    if not chunk_active(cfg, k - s):
        return []
    out = []
    if anchor_present(cfg, k):
        out.append((ANCHOR, 0, anchor_slot(cfg, k)))
    window = cfg.w_store if s == S else cfg.W
    for c in history_chunks(cfg, k, window):
        out.append((HISTORY, c, clean_slot(cfg, c)))
    if s == S:
        # The store reads anchor, its history and itself (WF App. B.3).
        out.append((STORE, k - S, clean_slot(cfg, k - S)))
        return out
    if store_active(cfg, k):
        out.append((STORE, k - S, clean_slot(cfg, k - S)))
    readable = [j for j in denoise_active(cfg, k)
                if (j >= s if cfg.mask == MASK_WAVE else True)]
    for j in sorted(readable):
        out.append((DENOISE, k - j, denoise_slot(cfg, k, j)))
    return out


def evicted_chunk(cfg: Config, k: int) -> int:
    """Chunk that leaves the retained clean list when round k's store is
    promoted (WF App. B.3), or -1."""
    if not store_active(cfg, k):
        return -1
    c = k - cfg.S - cfg.w_max
    return c if c >= cfg.anchor else -1


def plan(cfg: Config, k: int) -> dict:
    """The full plan of round k as plain Python data."""
    if k < 0 or (not cfg.unbounded and k >= cfg.n_rounds):
        raise ValueError("round out of range")
    cells = []
    for s in range(cfg.S + 1):
        i = k - s
        act = chunk_active(cfg, i)
        cells.append(dict(stage=s, chunk=i if act else -1, active=act,
                          slot=cell_slot(cfg, k, s) if act else -1,
                          frame0=cfg.F * i if act else -1))
    groups = [dict(stage=s, entries=key_entries(cfg, k, s))
              for s in range(cfg.S + 1)]
    n_c, d, h = cfg.n_c, cfg.head_dim, cfg.n_heads
    pages = sum(len(g["entries"]) for g in groups)
    # 2 matmuls (QK^T and PV) of 2 flops per multiply-add, readable keys only.
    flops = float(cfg.n_layers) * 4.0 * n_c * (pages * n_c) * d * h
    return dict(
        k=k, cells=cells, groups=groups,
        anchor=dict(present=anchor_present(cfg, k),
                    slot=anchor_slot(cfg, k) if anchor_present(cfg, k) else -1,
                    frame0=anchor_frame0(cfg, k) if anchor_present(cfg, k) else -1,
                    capture=anchor_capture(cfg, k)),
        evict=evicted_chunk(cfg, k),
        flops=flops, kv_tokens=pages * n_c,
        n_active=sum(c["active"] for c in cells))


def render(cfg: Config, k: int) -> str:
    """Human-readable one-line form of a plan: kind+chunk@slot per group."""
    p = plan(cfg, k)
    parts = []
    for g in p["groups"]:
        if not g["entries"]:
            continue
        s = g["stage"]
        body = " ".join(f"{KIND_NAMES[kd]}{c}@{sl}" for kd, c, sl in g["entries"])
        parts.append(f"s{s} c{k - s}: {body}")
    return f"k={k}  " + " | ".join(parts)
