"""A host model of the tree kernel's search, for bounds checking on the CPU.

The GPU search (one 1024-thread workgroup per tree) keeps its working arrays
in LDS and in a per-tree workspace whose sizes are fixed at launch.  This
module replays the same search on the host -- the starting bounds, the
levels (one-wave small levels and block levels), the bisection of an
overflowing level, the threshold raises and the cut-off -- with every array
replaced by a checked array of the kernel's capacity, so that any index the
kernel would form out of range raises here.  The index arithmetic of the
sorting networks (which depends only on the number of keys) and of the
one-wave small level (which depends on the level's data) is replayed lane by
lane, and the networks' barrier counts are compared across threads.

It models the kernel's index logic and capacities; it is not the oracle (the
method's definition lives in oracle/), and its final cut-off is checked
against the oracle's by the tests that use it.
"""

import math
import struct
from dataclasses import dataclass, field

import numpy as np

WAVE = 64
NT = 1024  # threads of the tree kernel's workgroup
MAX_SORT = 16384
FIRST_Q = 64
PRE_Q = 16
TREE_LDS_MAX = 156 * 1024
CTL_BYTES = 1488  # the kernel's Ctl block (a bound: the model only needs LDS placement)


def next_pow2(x: int) -> int:
    p = 1
    while p < x:
        p <<= 1
    return p


# ---------------------------------------------------------------- ordered keys (as the kernel forms them)

_MASK64 = (1 << 64) - 1


def f64_key(d: float) -> int:
    u = struct.unpack("<Q", struct.pack("<d", float(d)))[0]
    if u == 0x8000000000000000:
        u = 0
    return (~u & _MASK64) if (u >> 63) else (u | 0x8000000000000000)


def f64_from_key(k: int) -> float:
    u = (k & 0x7FFFFFFFFFFFFFFF) if (k >> 63) else (~k & _MASK64)
    return struct.unpack("<d", struct.pack("<Q", u))[0]


def key16(d: float) -> int:
    return f64_key(d) >> 48


# ---------------------------------------------------------------- checked storage

class CheckedArray:
    """A fixed-capacity array whose every read and write is bounds-checked."""

    def __init__(self, name: str, cap: int, fill=0):
        self.name, self.cap = name, int(cap)
        self.data = [fill] * self.cap

    def _check(self, i: int):
        if not (0 <= i < self.cap):
            raise IndexError(f"{self.name}[{i}] outside capacity {self.cap}")

    def __getitem__(self, i):
        self._check(i)
        return self.data[i]

    def __setitem__(self, i, v):
        self._check(i)
        self.data[i] = v


@dataclass
class Caps:
    sort_cap: int
    ent_cap: int
    node_cap: int
    tie_cap: int
    nk_lds: bool
    pre_q: int
    ch_lds: bool   # a level's children (raw sums, node offsets) in LDS
    f_cap: int     # frontier entries the LDS cache holds


def tree_caps(K: int, L: int, k: int, B: int) -> Caps:
    """The kernel's capacities for one tree (the host launcher's arithmetic)."""
    want = max(2 * K * k, 2 * (B + 1), 2048)
    want = min(want, MAX_SORT)
    sort_cap = next_pow2(want)
    ent_cap = 4 * sort_cap
    node_cap = min(4 * sort_cap, 65535)
    tie_cap = max(1, (sort_cap * 2) // (1 + L))
    base = sort_cap * 8 + K * (L + 1) * 8 + CTL_BYTES
    nk_off = (base + 15) & ~15
    nk_end = nk_off + node_cap * 2
    nk_lds = nk_end <= TREE_LDS_MAX
    lds = max(base + 64, nk_end if nk_lds else 0)
    pre_off = (lds + 15) & ~15
    pre_end = pre_off + K * L * PRE_Q * 8
    pre_q = PRE_Q if pre_end <= TREE_LDS_MAX else 0
    if pre_q:
        lds = pre_end
    ch_off = (lds + 15) & ~15
    ch_end = ch_off + sort_cap * 12
    ch_lds = ch_end <= TREE_LDS_MAX
    if ch_lds:
        lds = ch_end
    fc_off = (lds + 15) & ~15
    f_cap = (TREE_LDS_MAX - fc_off) // 15 if fc_off < TREE_LDS_MAX else 0
    f_cap = min(f_cap // 64 * 64, ent_cap)
    if f_cap < K:
        f_cap = 0
    return Caps(sort_cap, ent_cap, node_cap, tie_cap, nk_lds, pre_q, ch_lds, f_cap)


# ---------------------------------------------------------------- sorting networks (index arithmetic)

_sort_checked: dict = {}


def _check_lds_index(i: int, P: int, buf: int, what: str):
    if not (0 <= i < P) or i >= buf:
        raise IndexError(f"{what}: LDS index {i} with P={P}, buffer {buf}")


def check_block_sort_keys(P: int, buf: int, nt: int = NT) -> str:
    """Replays the index arithmetic of block_sort_keys<nt>(a, P) over a buffer of
    `buf` keys: every LDS index each thread forms, every lane it reads from,
    and the number of barriers each thread reaches.  Returns the network used."""
    key = (P, buf, nt)
    if key in _sort_checked:
        return _sort_checked[key]
    if P > buf:
        raise IndexError(f"sort of {P} keys in a buffer of {buf}")
    if WAVE <= P <= nt and P <= 1024:
        kind = _check_static(P, buf, nt)
    elif WAVE <= P <= 4 * nt:
        E = 1 if P <= nt else (2 if P <= 2 * nt else 4)
        kind = _check_regs(P, buf, nt, E)
    else:
        kind = _check_bitonic(P, buf, nt)
    _sort_checked[key] = kind
    return kind


def _check_static(P: int, buf: int, nt: int) -> str:
    LP = P.bit_length() - 1
    barriers = [0] * nt
    for i in range(nt):
        act = i < P
        if act:
            _check_lds_index(i, P, buf, "static load")
        for lk in range(1, LP + 1):
            for lj in range(lk - 1, -1, -1):
                j = 1 << lj
                if j >= WAVE:
                    if act:
                        _check_lds_index(i, P, buf, "static store")
                    barriers[i] += 1
                    if act:
                        _check_lds_index(i ^ j, P, buf, "static partner")
                    barriers[i] += 1
                elif act:
                    src = (i & (WAVE - 1)) ^ j
                    assert 0 <= src < WAVE
        if act:
            _check_lds_index(i, P, buf, "static final store")
        barriers[i] += 1
    assert len(set(barriers)) == 1, "threads reach different numbers of barriers"
    return f"static<{LP}>"


def _check_regs(P: int, buf: int, nt: int, E: int) -> str:
    S = WAVE * E
    W = P // S
    if W * S != P or W > nt // WAVE:
        raise IndexError(f"register sort of {P} keys with E={E}: {W} segments for {nt // WAVE} waves")
    barriers = [0] * nt
    for t in range(nt):
        w, lane = t // WAVE, t % WAVE
        act = w < W
        base = w * S
        if act:
            for e in range(E):
                _check_lds_index(base + e * WAVE + lane, P, buf, "regs load")
        k = 2
        while k <= P:
            j = k >> 1
            if j >= S:
                if act:
                    for e in range(E):
                        _check_lds_index(base + e * WAVE + lane, P, buf, "regs store")
                barriers[t] += 1
                while j >= S:
                    tt = t
                    while tt < (P >> 1):
                        i = 2 * tt - (tt & (j - 1))
                        _check_lds_index(i, P, buf, "regs pass")
                        _check_lds_index(i + j, P, buf, "regs pass partner")
                        tt += nt
                    barriers[t] += 1
                    j >>= 1
                if act:
                    for e in range(E):
                        _check_lds_index(base + e * WAVE + lane, P, buf, "regs reload")
            if act:
                while j >= WAVE:
                    m = j // WAVE
                    for e in range(E):
                        if e & m:
                            continue
                        assert (e | m) < E
                    j >>= 1
                while j > 0:
                    assert 0 <= (lane ^ j) < WAVE
                    j >>= 1
            k <<= 1
        if act:
            for e in range(E):
                _check_lds_index(base + e * WAVE + lane, P, buf, "regs final store")
        barriers[t] += 1
    assert len(set(barriers)) == 1, "threads reach different numbers of barriers"
    return f"regs<E={E}>"


def _check_bitonic(P: int, buf: int, nt: int) -> str:
    if P & (P - 1):
        raise ValueError(f"bitonic sort of {P} keys: not a power of two")
    size = 2
    while size <= P:
        stride = size >> 1
        while stride > 0:
            for t in range(0, P >> 1):
                i = 2 * t - (t & (stride - 1))
                _check_lds_index(i, P, buf, "bitonic")
                _check_lds_index(i + stride, P, buf, "bitonic partner")
            stride >>= 1
        size <<= 1
    return "bitonic"


# ---------------------------------------------------------------- the search

@dataclass
class LevelRecord:
    d: int
    fsize: int
    path: str          # "small", "block" or "end"
    C: int = 0
    P: int = 0
    sort: str = ""
    nodes: int = 0
    entries: int = 0
    bisected: bool = False
    raised: bool = False


@dataclass
class SearchResult:
    levels: list = field(default_factory=list)
    node_count: int = 0
    ent_count: int = 0
    fail: bool = False
    cutoff: float = math.inf
    n_select: int = 0
    pooled_P: int = 0
    window_hits: int = 0
    window_misses: int = 0
    node_S: list = field(default_factory=list)


class TreeModel:
    """One tree of the search: inputs are the rank-ordered lists (ids and raw
    logits, [K][L][k]) and the row log-normalisers ([K][L], fp64)."""

    def __init__(self, topk_id: np.ndarray, topk_raw: np.ndarray, lse: np.ndarray, B: int):
        self.id = np.asarray(topk_id)
        self.raw = np.asarray(topk_raw, dtype=np.float32)
        self.K, self.L, self.k = self.raw.shape
        self.B = int(B)
        self.caps = tree_caps(self.K, self.L, self.k, self.B)
        lse = np.asarray(lse, dtype=np.float64)
        self.norm = np.zeros((self.K, self.L + 1))
        for m in range(self.K):
            acc = 0.0
            for i in range(self.L):
                # the kernel's normaliser: lse, but never below the row's top logit
                acc = acc + max(float(lse[m, i]), float(self.raw[m, i, 0]))
                self.norm[m, i + 1] = acc

    # the per-entry child count: leading candidates of the row reaching tau
    def _ok(self, raw: float, x: float, nrm: float, tau: float) -> bool:
        return x != -math.inf and (raw + float(x)) - nrm >= tau

    def _count(self, e, d, tau) -> int:
        m, raw = self.ent_mode[e], self.ent_raw[e]
        row, nrm = self.raw[m, d - 1], self.norm[m, d]
        lo, hi = 0, self.k
        while lo < hi:
            mid = (lo + hi) >> 1
            if self._ok(raw, row[mid], nrm, tau):
                lo = mid + 1
            else:
                hi = mid
        return lo

    def run(self) -> SearchResult:
        K, L, k, B, c = self.K, self.L, self.k, self.B, self.caps
        res = SearchResult()
        self.node_parent = CheckedArray("node_parent", c.node_cap)
        self.node_token = CheckedArray("node_token", c.node_cap)
        self.node_S = CheckedArray("node_S", c.node_cap, 0.0)
        self.node_mu = CheckedArray("node_mu", c.node_cap)
        self.nk = CheckedArray("nk (LDS)", c.node_cap) if c.nk_lds else None
        self.window_hits = 0
        self.window_misses = 0
        self.ent_node = CheckedArray("ent_node", c.ent_cap)
        self.ent_mode = CheckedArray("ent_mode", c.ent_cap)
        self.ent_raw = CheckedArray("ent_raw", c.ent_cap, 0.0)
        self.ent_s = CheckedArray("ent_s", c.ent_cap, 0.0)
        self.fr = CheckedArray("fr", c.ent_cap)
        self.fr_off = CheckedArray("fr_off", c.ent_cap)
        keys = CheckedArray("keys (LDS)", c.sort_cap)
        pre = CheckedArray("pre (LDS)", K * L * c.pre_q) if c.pre_q else None
        chr_ = CheckedArray("children raw (LDS)" if c.ch_lds else "ch_raw", c.sort_cap, 0.0)
        cg = CheckedArray("children node offsets (LDS)" if c.ch_lds else "grp", c.sort_cap)
        self.fc = None
        if c.f_cap:
            self.fc = {f: CheckedArray(f"frontier cache {f} (LDS)", c.f_cap, 0) for f in ("mode", "raw", "node", "off")}

        node_count, ent_count, fsize = 1, K, K
        self.node_S[0] = 0.0
        for m in range(K):
            self.ent_node[m], self.ent_mode[m], self.ent_raw[m], self.ent_s[m] = 0, m, 0.0, 0.0
            self.fr[m] = m
            self._cache_write(m, m)
        # the rows' leading candidates staged in LDS
        if pre is not None:
            for q in range(K * L * c.pre_q):
                pre[q] = 0
        # starting bound: any single mode's B-th depth-1 candidate
        tau = -math.inf
        if B == 0:
            fsize = 0
        elif k >= B:
            for m in range(K):
                x = float(self.raw[m, 0, B - 1])
                if x != -math.inf:
                    tau = max(tau, (0.0 + x) - self.norm[m, 1])
        # the pooled bound over each mode's first FIRST_Q depth-1 candidates
        if B > 0:
            q = min(k, FIRST_Q)
            npool = K * q
            # distinct tokens by an LDS hash table in the sort area (12 bytes
            # per slot, at most half full), else by a sort of the pooled keys
            H = 1
            while H * 2 * 12 <= c.sort_cap * 8:
                H *= 2
            if npool >= B and H >= 2 * npool:
                hkey = CheckedArray("pool hash keys", c.sort_cap)          # slots [0, H) as 8-byte words
                htok = CheckedArray("pool hash tokens", 2 * c.sort_cap)    # 4-byte words from byte 8 H
                for h in range(H):
                    hkey[h] = 0
                    htok[2 * H + h] = -1
                for m in range(K):
                    for j in range(q):
                        t = int(self.id[m, 0, j])
                        if t < 0 or float(self.raw[m, 0, j]) == -math.inf:
                            continue
                        h = (t * 0x9E3779B1) & 0xFFFFFFFF & (H - 1)
                        for _ in range(H):
                            if htok[2 * H + h] in (-1, t):
                                htok[2 * H + h] = t
                                break
                            h = (h + 1) & (H - 1)
                        else:
                            raise IndexError("pooled bound: hash table full")
                res.pooled_P = H
            if npool >= B:
                P = next_pow2(npool)
                if not (H >= 2 * npool):
                    if 2 * P > c.sort_cap:
                        raise IndexError(f"pooled bound: 2P={2 * P} keys past the sort buffer {c.sort_cap}")
                    res.pooled_P = P
                    check_block_sort_keys(P, c.sort_cap)
                best = {}
                for m in range(K):
                    for j in range(q):
                        keys[m * q + j] = 0
                        t = int(self.id[m, 0, j])
                        sc = (0.0 + float(self.raw[m, 0, j])) - self.norm[m, 1]
                        best[t] = sc if t not in best else max(best[t], sc)
                alive = [s for s in best.values() if s >= tau]
                if len(alive) >= B:
                    kb = sorted((key16(s) for s in alive), reverse=True)[B - 1]
                    nb = f64_from_key(kb << 48)
                    if nb > tau:
                        tau = nb

        for d in range(1, L + 1):
            if fsize == 0 or res.fail:
                break
            rec = LevelRecord(d=d, fsize=fsize, path="block")
            up = False
            C = -1
            self._cache_check(fsize)
            if fsize <= WAVE:
                C, up, my_s = self._small_level(d, fsize, tau, node_count, ent_count, pre)
                if C == 0:
                    rec.path = "end"
                    res.levels.append(rec)
                    break
                if C > 0:
                    rec.path, rec.C = "small", C
                    node_count, ent_count = self._last_counts
                    if up:
                        tau, rec.raised = self._raise(tau, node_count)
                    kept = [ent_count - C + lane for lane in range(C) if my_s[lane] >= tau]
                    for i, e in enumerate(kept):
                        self.fr[i] = e
                        self._cache_write(i, e)
                    fsize = len(kept)
                    rec.nodes, rec.entries = node_count, ent_count
                    res.levels.append(rec)
                    continue
            # block path
            counts = [self._count(self.fr[f], d, tau) for f in range(fsize)]
            C = sum(counts)
            too_big = C > c.sort_cap or ent_count + C > c.ent_cap or node_count + C > c.node_cap
            if too_big:
                rec.bisected = True
                tau = self._bisect(d, fsize, tau, node_count)
                counts = [self._count(self.fr[f], d, tau) for f in range(fsize)]
                C = sum(counts)
            if C > c.sort_cap or ent_count + C > c.ent_cap or node_count + C > c.node_cap:
                res.fail = True
                rec.C = C
                res.levels.append(rec)
                break
            if C == 0:
                rec.path = "end"
                res.levels.append(rec)
                break
            off = 0
            cached = c.f_cap and fsize <= c.f_cap
            for f in range(fsize):
                self.fr_off[f] = off
                if cached:
                    self.fc["off"][f] = off
                off += counts[f]
            ch = []
            for cidx in range(C):
                lo, hi = 0, fsize - 1
                while lo < hi:
                    mid = (lo + hi + 1) >> 1
                    if self.fr_off[mid] <= cidx:
                        lo = mid
                    else:
                        hi = mid - 1
                e = self.fr[lo]
                m = self.ent_mode[e]
                j = cidx - self.fr_off[lo]
                if not (0 <= j < k):
                    raise IndexError(f"child {cidx}: rank {j} outside the row of {k}")
                x = float(self.raw[m, d - 1, j])
                tok = int(self.id[m, d - 1, j])
                raw = self.ent_raw[e] + x
                s = raw - self.norm[m, d]
                pnode = self.ent_node[e]
                if pnode >= (1 << 24) or tok >= (1 << 20) or m >= 32 or cidx >= (1 << 15):
                    raise IndexError("a sort key field overflows its bits")
                keys[cidx] = (pnode << 40) | (tok << 20) | (m << 15) | cidx
                chr_[cidx] = raw
                ch.append((pnode, tok, m, cidx, raw, s))
            P = next_pow2(C)
            for cidx in range(C, P):
                keys[cidx] = _MASK64
            rec.C, rec.P = C, P
            rec.sort = check_block_sort_keys(P, c.sort_cap)
            order = sorted(range(C), key=lambda i: (ch[i][0], ch[i][1], ch[i][2], ch[i][3]))
            unsorted = [keys[i] for i in range(C)]
            for q_, i in enumerate(order):  # the sort, in place in LDS
                keys[q_] = unsorted[i]
            node0, ent0 = node_count, ent_count
            g = -1
            prev = None
            kt = key16(tau)
            for q_, i in enumerate(order):
                pnode, tok, m, cidx, raw, s = ch[i]
                if (pnode, tok) != prev:
                    g += 1
                    prev = (pnode, tok)
                    node = node0 + g
                    self.node_parent[node], self.node_token[node] = pnode, tok
                    self.node_S[node], self.node_mu[node] = s, m
                    best_node = node
                else:
                    node = node0 + g
                    if s > self.node_S[node]:
                        self.node_S[node], self.node_mu[node] = s, m
                e = ent0 + q_
                cg[q_] = g
                self.ent_node[e], self.ent_mode[e], self.ent_raw[e], self.ent_s[e] = node, m, raw, s
            for node in range(node0, node0 + g + 1):
                if self.nk is not None:
                    self.nk[node] = key16(self.node_S[node])
                if key16(self.node_S[node]) > kt:
                    up = True
            node_count, ent_count = node0 + g + 1, ent0 + C
            if up:
                tau, rec.raised = self._raise(tau, node_count)
            fs = 0
            for i in range(C):
                if self.ent_s[ent0 + i] >= tau:
                    self.fr[fs] = ent0 + i
                    # the kernel reads the entry back from the sorted key and LDS
                    key = keys[i]
                    assert chr_[key & 0x7FFF] == self.ent_raw[ent0 + i]
                    assert node0 + cg[i] == self.ent_node[ent0 + i]
                    self._cache_write(fs, ent0 + i)
                    fs += 1
            fsize = fs
            rec.nodes, rec.entries = node_count, ent_count
            res.levels.append(rec)

        res.node_count, res.ent_count = node_count, ent_count
        res.window_hits, res.window_misses = self.window_hits, self.window_misses
        res.node_S = [self.node_S[i] for i in range(1, node_count)]
        total = node_count - 1
        if not res.fail and B > 0 and total > 0:
            res.n_select = min(B, total)
            res.cutoff = sorted(res.node_S, reverse=True)[res.n_select - 1]
        return res

    def _cache_write(self, pos: int, e: int):
        """A frontier writer: entry e at frontier position pos, into the LDS cache
        when pos < f_cap."""
        if self.fc is not None and pos < self.caps.f_cap:
            self.fc["mode"][pos] = self.ent_mode[e]
            self.fc["raw"][pos] = self.ent_raw[e]
            if not (0 <= self.ent_node[e] < 65536):
                raise IndexError(f"node id {self.ent_node[e]} does not fit the cache's 16 bits")
            self.fc["node"][pos] = self.ent_node[e]

    def _cache_check(self, fsize: int):
        """A level whose frontier fits the cache reads it there: it must hold
        what the workspace path reads through fr."""
        if self.fc is None or fsize > self.caps.f_cap:
            return
        for f in range(fsize):
            e = self.fr[f]
            assert self.fc["mode"][f] == self.ent_mode[e]
            assert self.fc["raw"][f] == self.ent_raw[e]
            assert self.fc["node"][f] == self.ent_node[e]

    def _raise(self, tau: float, node_count: int):
        """The threshold raise: the B-th largest 16-bit score key among the nodes
        at or above tau (16-bit keys in LDS when they fit, else fp64 scores)."""
        B = self.B
        if self.nk is not None:
            kt = key16(tau)
            alive = [self.nk[i] for i in range(1, node_count) if self.nk[i] >= kt]
            # the one-pass window: bins of key - kt, 255 and above in the top one
            hist = CheckedArray("raise window (LDS)", 256)
            for i in range(256):
                hist[i] = 0
            for kk in alive:
                hist[min(kk - kt, 255)] = hist[min(kk - kt, 255)] + 1
            assert sum(hist[i] for i in range(256)) == len(alive)
            if len(alive) >= B and B > 0:
                cum, dg = 0, -1
                for b in range(255, -1, -1):
                    cum += hist[b]
                    if cum >= B:
                        dg = b
                        break
                self.window_hits += int(dg < 255)
                self.window_misses += int(dg == 255)
                if dg < 255:
                    assert kt + dg == sorted(alive, reverse=True)[B - 1]
        else:
            alive = [key16(self.node_S[i]) for i in range(1, node_count) if self.node_S[i] >= tau]
        if len(alive) >= B and B > 0:
            kb = sorted(alive, reverse=True)[B - 1]
            nt = f64_from_key(kb << 48)
            if nt > tau:
                return nt, True
        return tau, False

    def _bisect(self, d: int, fsize: int, tau: float, node_count: int) -> float:
        """Bisection on the key of tau: the largest threshold keeping at least B
        unique prefixes by the lower bound (nodes found so far plus, per parent
        node, its largest per-mode child count)."""
        lo = f64_key(tau)
        hi = f64_key(math.inf)
        for _ in range(70):
            if hi - lo <= 1:
                break
            mid = lo + (hi - lo) // 2
            th = f64_from_key(mid)
            cnt = 0
            f = 0
            while f < fsize:
                node = self.ent_node[self.fr[f]]
                best = 0
                g = f
                while g < fsize and self.ent_node[self.fr[g]] == node:
                    best = max(best, self._count(self.fr[g], d, th))
                    g += 1
                cnt += best
                f = g
            cnt += sum(1 for i in range(1, node_count) if self.node_S[i] >= th)
            if cnt >= self.B:
                lo = mid
            else:
                hi = mid
        return f64_from_key(lo)

    def _small_level(self, d, fsize, tau, node_count, ent_count, pre):
        """The one-wave level (fsize <= 64): replays every lane's reads, shuffles
        and writes with bounds checks.  Returns (C, up, child scores) with C = -1
        when the level does not fit one wave (the block path takes it)."""
        K, L, k, c = self.K, self.L, self.k, self.caps
        lanes = range(WAVE)
        m_, raw_, pnode_, nrm_, cnt_ = [0] * WAVE, [0.0] * WAVE, [0] * WAVE, [0.0] * WAVE, [0] * WAVE
        v_ = [[-math.inf] * 8 for _ in lanes]
        id_ = [[0] * 8 for _ in lanes]
        more = False
        for lane in lanes:
            if lane >= fsize:
                continue
            e = self.fr[lane]
            m = self.ent_mode[e]
            m_[lane], raw_[lane], pnode_[lane] = m, self.ent_raw[e], self.ent_node[e]
            nrm_[lane] = self.norm[m, d]
            for j in range(8):
                if c.pre_q >= 8:
                    pr = (m * L + (d - 1)) * c.pre_q + j
                    pre[pr]  # the staged read (bounds)
                v_[lane][j] = float(self.raw[m, d - 1, j]) if j < k else -math.inf
                id_[lane][j] = int(self.id[m, d - 1, j]) if j < k else 0
            run = True
            cnt = 0
            for j in range(8):
                run = run and self._ok(raw_[lane], v_[lane][j], nrm_[lane], tau)
                cnt += 1 if run else 0
            cnt_[lane] = cnt
            more = more or (cnt == 8 and k > 8)
        if more:
            return -1, False, None
        incl = list(np.cumsum(cnt_))
        off = [incl[i] - cnt_[i] for i in lanes]
        C = incl[-1]
        if C > WAVE:
            return -1, False, None
        if C == 0:
            return 0, False, None
        if ent_count + C > c.ent_cap or node_count + C > c.node_cap:
            return -1, False, None
        keys, craw, cs, cm = [0] * WAVE, [0.0] * WAVE, [0.0] * WAVE, [0] * WAVE
        for lane in lanes:
            ci = lane
            lo, hi = 0, fsize - 1
            for _ in range(6):
                mid = (lo + hi + 1) >> 1
                assert 0 <= mid < WAVE  # shuffle source
                if lo < hi:
                    if off[mid] <= ci:
                        lo = mid
                    else:
                        hi = mid - 1
            f = lo
            assert 0 <= f < WAVE
            j = ci - off[f]
            x, tok = -math.inf, 0
            for jj in range(8):
                if jj == j:
                    x, tok = v_[f][jj], id_[f][jj]
            craw[lane] = raw_[f] + x
            cs[lane] = craw[lane] - nrm_[f]
            cm[lane] = m_[f]
            valid = ci < C
            if valid:
                if not (0 <= j < 8) or not (0 <= f < fsize):
                    raise IndexError(f"small level: child {ci} maps to entry {f}, rank {j}")
                keys[lane] = (pnode_[f] << 40) | (tok << 20) | (m_[f] << 15) | ci
            else:
                keys[lane] = _MASK64
        sk = sorted(keys)
        node0, ent0 = node_count, ent_count
        heads = [lane < C and (lane == 0 or (sk[lane] >> 20) != (sk[lane - 1] >> 20)) for lane in lanes]
        G = sum(heads)
        kt = key16(tau)
        up = False
        my_s = [-math.inf] * WAVE
        g = -1
        for lane in lanes:
            if lane >= C:
                continue
            sc = sk[lane] & 0x7FFF
            if not (0 <= sc < C):
                raise IndexError(f"small level: sorted key names child {sc} of {C}")
            if heads[lane]:
                g += 1
                node = node0 + g
                best, mu = -math.inf, -1
                q = lane
                while q < C and (sk[q] >> 20) == (sk[lane] >> 20):
                    src = min(q, WAVE - 1)
                    s2 = cs[sk[src] & 0x7FFF]
                    if mu < 0 or s2 > best:
                        best, mu = s2, cm[sk[src] & 0x7FFF]
                    q += 1
                self.node_parent[node] = int(sk[lane] >> 40)
                self.node_token[node] = int((sk[lane] >> 20) & 0xFFFFF)
                self.node_S[node], self.node_mu[node] = best, mu
                if self.nk is not None:
                    self.nk[node] = key16(best)
                up = up or key16(best) > kt
            e = ent0 + lane
            self.ent_node[e] = node0 + g
            self.ent_mode[e] = cm[sc]
            self.ent_raw[e] = craw[sc]
            self.ent_s[e] = cs[sc]
            my_s[lane] = cs[sc]
        assert g + 1 == G
        self._last_counts = (node0 + G, ent0 + C)
        return C, up, my_s


# ---------------------------------------------------------------- inputs

def row_lists(x: np.ndarray, k: int):
    """Rank-ordered top-k ids and raw values of every row of x [K, L, V]
    (logit descending, then id ascending), and the rows' log-normalisers."""
    K, L, V = x.shape
    ids = np.zeros((K, L, k), dtype=np.int64)
    raw = np.zeros((K, L, k), dtype=np.float32)
    for m in range(K):
        for i in range(L):
            row = np.asarray(x[m, i], dtype=np.float64)
            kth = np.partition(row, V - k)[V - k]
            above = np.nonzero(row > kth)[0]
            eq = np.nonzero(row == kth)[0][: k - above.size]
            cand = np.concatenate([above, eq])
            cand = cand[np.lexsort((cand, -row[cand]))]
            ids[m, i] = cand
            raw[m, i] = row[cand].astype(np.float32)
    mx = x.max(axis=-1, keepdims=True)
    lse = (mx[..., 0] + np.log(np.exp(x - mx).sum(axis=-1))).astype(np.float64)
    return ids, raw, lse
