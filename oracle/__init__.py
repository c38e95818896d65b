"""ctypes binding of the plain C oracle (oracle/diffkv_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product
package never does.  It shares no code with the HIP library: configs arrive
as plain dicts and every buffer is a numpy array in host memory.

Parity unpinned: the fp32 rounding of score sums after a score update
(compared within a tolerance only).  Every other function is pinned by a
``-m "not gpu"`` test.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "diffkv_oracle.c")
_LIB = os.path.join(_HERE, "libdiffkv_oracle.so")

PRUNE, LO, HI = 0, 1, 2
ST_POOL_EXHAUSTED, ST_TABLE_OVERFLOW, ST_BAD_STATE = 1, 2, 4
# generation-step policy cases recorded by State.compact_step(branches=True)
(BR_INACTIVE, BR_NO_TC, BR_HI_KEEP, BR_HI_DEMOTE, BR_HI_PRUNE, BR_LO_KEEP, BR_LO_PRUNE,
 BR_PRUNE) = range(8)


def build() -> str:
    """Compile the oracle with gcc (plain IEEE fp32: no contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Cfg(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("gqa_group", ctypes.c_int32), ("hi_page_tokens", ctypes.c_int32),
                ("lo_page_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("window", ctypes.c_int32), ("lo_enabled", ctypes.c_int32),
                ("alpha_h", ctypes.c_float), ("alpha_l", ctypes.c_float),
                ("prompt_rule", ctypes.c_int32), ("alpha_h_head", ctypes.c_void_p),
                ("alpha_l_head", ctypes.c_void_p),
                ("hi_k_bits", ctypes.c_int32), ("hi_v_bits", ctypes.c_int32),
                ("lo_k_bits", ctypes.c_int32), ("lo_v_bits", ctypes.c_int32),
                ("num_levels", ctypes.c_int32), ("alpha_mid", ctypes.c_float * 2),
                ("mid_k_bits", ctypes.c_int32 * 2), ("mid_v_bits", ctypes.c_int32 * 2)]


RULE_ALPHA_N, RULE_ALPHA_I = 0, 1


class _Pool(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("free_list", ctypes.c_void_p),
                ("ptr", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("page_bytes", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_f32_to_f16.restype = ctypes.c_uint16
        _lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        _lib.orc_f16_to_f32.restype = ctypes.c_float
        _lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        _lib.orc_dequant.restype = ctypes.c_float
        _lib.orc_dequant.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int32]
        _lib.orc_page_bytes.restype = ctypes.c_int32
        _lib.orc_table_len.restype = ctypes.c_int32
        _lib.orc_tier_layout.restype = ctypes.c_int32
        _lib.orc_level_layout.restype = ctypes.c_int32
        _lib.orc_num_levels.restype = ctypes.c_int32
        _lib.orc_state_words.restype = ctypes.c_int32
    return _lib


def make_cfg(c: dict) -> Cfg:
    """Config dict -> orc_cfg.  Optional keys: prompt_rule (RULE_ALPHA_N or
    RULE_ALPHA_I), alpha_h_head / alpha_l_head (H thresholds each),
    hi_k_bits / hi_v_bits / lo_k_bits / lo_v_bits (tier codecs), num_levels
    (3 or 4 precision levels) with alpha_mid / mid_k_bits / mid_v_bits (one
    value per middle level)."""
    r = Cfg(int(c["head_dim"]), int(c["num_kv_heads"]), int(c["gqa_group"]),
            int(c.get("hi_page_tokens", 16)), int(c.get("lo_page_tokens", 32)),
            int(c["max_seq_len"]), int(c["window"]), int(c.get("lo_enabled", 1)),
            float(c["alpha_h"]), float(c["alpha_l"]), int(c.get("prompt_rule", RULE_ALPHA_N)))
    keep = []
    for key in ("alpha_h_head", "alpha_l_head"):
        v = c.get(key)
        if v is None:
            continue
        a = np.ascontiguousarray(np.asarray(v, np.float32).reshape(-1))
        if a.size != r.num_kv_heads:
            raise ValueError(f"{key} needs {r.num_kv_heads} values")
        keep.append(a)
        setattr(r, key, a.ctypes.data)
    r._keep = keep  # the arrays live as long as the struct
    # tier codecs (bits of K and V codes per tier; absent: K8V4 / K4V2)
    for key in ("hi_k_bits", "hi_v_bits", "lo_k_bits", "lo_v_bits"):
        setattr(r, key, int(c.get(key, 0)))
    r.num_levels = int(c.get("num_levels", 0))
    for key, conv in (("alpha_mid", float), ("mid_k_bits", int), ("mid_v_bits", int)):
        vals = list(c.get(key, ()))
        arr = getattr(r, key)
        for i in range(2):
            arr[i] = conv(vals[i]) if i < len(vals) else conv(0)
    return r


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int):
    if rc != 0:
        raise ValueError(f"oracle rejected the call (code {rc})")


def page_bytes(cfg: dict) -> int:
    return lib().orc_page_bytes(ctypes.byref(make_cfg(cfg)))


def table_len(cfg: dict) -> int:
    return lib().orc_table_len(ctypes.byref(make_cfg(cfg)))


def num_levels(cfg: dict) -> int:
    return lib().orc_num_levels(ctypes.byref(make_cfg(cfg)))


def state_words(cfg: dict) -> int:
    return lib().orc_state_words(ctypes.byref(make_cfg(cfg)))


def level_layout(cfg: dict, level: int):
    seg = np.zeros(7, np.int32)
    T = lib().orc_level_layout(ctypes.byref(make_cfg(cfg)), level, _p(seg))
    return T, seg


def tier_layout(cfg: dict, tier: int):
    seg = np.zeros(7, np.int32)
    T = lib().orc_tier_layout(ctypes.byref(make_cfg(cfg)), tier, _p(seg))
    return T, seg


def k_code_addr(cfg: dict, tier: int, tok: int, j: int):
    b, s = ctypes.c_int32(), ctypes.c_int32()
    lib().orc_k_code_addr(ctypes.byref(make_cfg(cfg)), tier, tok, j, ctypes.byref(b), ctypes.byref(s))
    return b.value, s.value


def v_code_addr(cfg: dict, tier: int, tok: int, j: int):
    b, s = ctypes.c_int32(), ctypes.c_int32()
    lib().orc_v_code_addr(ctypes.byref(make_cfg(cfg)), tier, tok, j, ctypes.byref(b), ctypes.byref(s))
    return b.value, s.value


def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = np.zeros(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_p(x), _p(h), ctypes.c_int64(x.size))
    return h


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    x = np.zeros(h.shape, np.float32)
    lib().orc_f16_to_f32_n(_p(h), _p(x), ctypes.c_int64(h.size))
    return x


def quantize(x, bits: int):
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.zeros(x.size, np.uint8)
    s, z = ctypes.c_uint16(), ctypes.c_uint16()
    lib().orc_quantize(_p(x), ctypes.c_int32(x.size), ctypes.c_int32(bits),
                       ctypes.byref(s), ctypes.byref(z), _p(codes))
    return s.value, z.value, codes


def dequant(s16: int, z16: int, code: int) -> float:
    return lib().orc_dequant(s16, z16, code)


def classify(cfg: dict, cu_seqlens, scores, levels_impl: bool = False):
    """Tier codes [H, total] (K - level, 0 pruned; two tiers: HI, LO, PRUNE)
    and counts [batch, H, K].  levels_impl: the K-level implementation even
    for two tiers."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    B = cu.size - 1
    H = int(cfg["num_kv_heads"])
    tiers = np.zeros(sc.shape, np.uint8)
    counts = np.zeros((B, H, max(num_levels(cfg), 2)), np.int32)
    fn = lib().orc_levels_classify if levels_impl else lib().orc_classify
    _check(fn(ctypes.byref(make_cfg(cfg)), ctypes.c_int32(B), _p(cu), _p(sc), _p(tiers), _p(counts)))
    return tiers, counts


class State:
    """Host copy of the whole compaction state (same layout as the device state)."""

    def __init__(self, cfg: dict, batch: int, num_pages: int, init_pages: bool = True):
        self.cfg = dict(cfg)
        self.batch = batch
        self.num_pages = int(num_pages)
        self.page_bytes = page_bytes(cfg)
        self.L = table_len(cfg)
        H = int(cfg["num_kv_heads"])
        self.pages = np.zeros((self.num_pages, self.page_bytes), np.uint8)
        self.free_list = np.zeros(self.num_pages, np.int32)
        self.ptr = np.zeros(2, np.uint64)
        self.status = np.zeros(1, np.uint32)
        self.K = max(num_levels(cfg), 2)
        self.page_table = np.full((batch, H, self.L), -1, np.int32)
        self.tier_state = np.zeros((batch, H, 2 * self.K), np.int32)
        if init_pages:
            _check(lib().orc_pool_init(ctypes.byref(self._pool())))

    def _pool(self) -> _Pool:
        return _Pool(self.pages.ctypes.data, self.free_list.ctypes.data, self.ptr.ctypes.data,
                     self.status.ctypes.data, self.num_pages, self.page_bytes)

    def copy(self) -> "State":
        s = State.__new__(State)
        s.__dict__.update({k: (v.copy() if isinstance(v, np.ndarray) else v)
                           for k, v in self.__dict__.items()})
        s.cfg = dict(self.cfg)
        return s

    # -- operations -----------------------------------------------------
    # levels_impl=True runs the K-level implementation even for two tiers
    # (the two must agree there).
    def compact_prompt(self, cu_seqlens, k, v, scores, tiers, levels_impl: bool = False):
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        sc = np.ascontiguousarray(scores, dtype=np.float32)
        ti = np.ascontiguousarray(tiers, dtype=np.uint8)
        pool = self._pool()
        fn = lib().orc_levels_compact_prompt if levels_impl else lib().orc_compact_prompt
        _check(fn(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool), ctypes.c_int32(cu.size - 1), _p(cu),
                  _p(k), _p(v), _p(sc), _p(ti), _p(self.page_table), _p(self.tier_state)))

    def compact_step(self, seq_len, k_new, v_new, branches: bool = False, levels_impl: bool = False):
        """One generation step; with branches=True returns int32 [batch, H]:
        two tiers, the policy case per unit (BR_*, bits 0-3) and the new
        page's tier (bits 4-5); K levels (or levels_impl), t_c's class in
        bits 0-3 (level, 14 pruned, 15 none), the victim's in bits 4-7 and
        the new page's level + 1 in bits 8-11 (-1 inactive)."""
        sl = np.ascontiguousarray(seq_len, dtype=np.int32)
        k = np.ascontiguousarray(k_new, dtype=np.uint16)
        v = np.ascontiguousarray(v_new, dtype=np.uint16)
        pool = self._pool()
        br = np.zeros((self.batch, int(self.cfg["num_kv_heads"])), np.int32)
        if levels_impl:
            _check(lib().orc_levels_compact_step(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool),
                                                 ctypes.c_int32(self.batch), _p(sl), _p(k), _p(v),
                                                 _p(self.page_table), _p(self.tier_state), _p(br)))
        else:
            _check(lib().orc_compact_step_branches(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool),
                                                   ctypes.c_int32(self.batch), _p(sl), _p(k), _p(v),
                                                   _p(self.page_table), _p(self.tier_state), _p(br)))
        return br if branches else None

    def release(self, mask, levels_impl: bool = False):
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        pool = self._pool()
        fn = lib().orc_levels_release if levels_impl else lib().orc_release
        _check(fn(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool), ctypes.c_int32(self.batch), _p(m),
                  _p(self.page_table), _p(self.tier_state)))

    def decode_attn(self, q, seq_len, update_scores: bool = False, levels_impl: bool = False) -> np.ndarray:
        qq = np.ascontiguousarray(q, dtype=np.uint16)
        sl = np.ascontiguousarray(seq_len, dtype=np.int32)
        H, G, d = int(self.cfg["num_kv_heads"]), int(self.cfg["gqa_group"]), int(self.cfg["head_dim"])
        out = np.zeros((self.batch, H * G, d), np.float32)
        pool = self._pool()
        fn = lib().orc_levels_decode_attn if levels_impl else lib().orc_decode_attn
        _check(fn(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool), ctypes.c_int32(self.batch), _p(qq),
                  _p(self.page_table), _p(self.tier_state), _p(sl), _p(out),
                  ctypes.c_int32(1 if update_scores else 0)))
        return out

    def page_bounds(self) -> np.ndarray:
        """fp32 [num_pages, 2, d]: per-dimension min / max of every live
        page's dequantized keys (other pages NaN)."""
        d = int(self.cfg["head_dim"])
        b = np.full((self.num_pages, 2, d), np.nan, np.float32)
        pool = self._pool()
        _check(lib().orc_page_bounds(ctypes.byref(make_cfg(self.cfg)), ctypes.byref(pool),
                                     ctypes.c_int32(self.batch), _p(self.page_table), _p(self.tier_state), _p(b)))
        return b

    def page_scores(self, q, seq_len, bounds) -> np.ndarray:
        """fp32 [batch, H, table_len] page scores in table order from `bounds`."""
        qq = np.ascontiguousarray(q, dtype=np.uint16)
        sl = np.ascontiguousarray(seq_len, dtype=np.int32)
        bb = np.ascontiguousarray(bounds, dtype=np.float32)
        out = np.zeros(self.page_table.shape, np.float32)
        _check(lib().orc_page_scores(ctypes.byref(make_cfg(self.cfg)), ctypes.c_int32(self.batch), _p(qq),
                                     _p(self.page_table), _p(self.tier_state), _p(sl), _p(bb),
                                     ctypes.c_int64(self.num_pages), _p(out)))
        return out

    # -- inspection -------------------------------------------------------
    def read_slot(self, page_id: int, tier: int, slot: int):
        d = int(self.cfg["head_dim"])
        kc = np.zeros(d, np.uint8)
        vc = np.zeros(d, np.uint8)
        km = np.zeros(2, np.uint16)
        vm = np.zeros(2, np.uint16)
        sc = ctypes.c_float()
        pos = ctypes.c_int32()
        page = np.ascontiguousarray(self.pages[page_id])
        lib().orc_read_slot(ctypes.byref(make_cfg(self.cfg)), _p(page), ctypes.c_int32(tier),
                            ctypes.c_int32(slot), _p(kc), _p(vc), _p(km), _p(vm),
                            ctypes.byref(sc), ctypes.byref(pos))
        return dict(k=kc, v=vc, kmeta=km, vmeta=vm, score=sc.value, pos=pos.value)

    def read_level_slot(self, page_id: int, level: int, slot: int):
        d = int(self.cfg["head_dim"])
        kc = np.zeros(d, np.uint8)
        vc = np.zeros(d, np.uint8)
        km = np.zeros(2, np.uint16)
        vm = np.zeros(2, np.uint16)
        sc = ctypes.c_float()
        pos = ctypes.c_int32()
        page = np.ascontiguousarray(self.pages[page_id])
        lib().orc_read_level_slot(ctypes.byref(make_cfg(self.cfg)), _p(page), ctypes.c_int32(level),
                                  ctypes.c_int32(slot), _p(kc), _p(vc), _p(km), _p(vm),
                                  ctypes.byref(sc), ctypes.byref(pos))
        return dict(k=kc, v=vc, kmeta=km, vmeta=vm, score=sc.value, pos=pos.value)

    def level_page(self, b: int, h: int, level: int, j: int) -> int:
        """Page id of page j of a level (row level // 2: even levels from the
        left, odd levels from the right)."""
        Lr = self.L // ((self.K + 1) // 2)
        col = j if level % 2 == 0 else Lr - 1 - j
        return int(self.page_table[b, h, (level // 2) * Lr + col])

    def unit_tokens(self, b: int, h: int):
        """List of (tier, slot, slot-record) of one unit's retained tokens
        (K levels: (level, slot, record))."""
        if self.K >= 3:
            out = []
            for lv in range(self.K):
                T = 16 if lv == 0 else 32
                for s in range(int(self.tier_state[b, h, lv])):
                    out.append((lv, s, self.read_level_slot(self.level_page(b, h, lv, s // T), lv, s % T)))
            return out
        n_hi, n_lo, ph, pl = (int(x) for x in self.tier_state[b, h])
        row = self.page_table[b, h]
        out = []
        for s in range(n_hi):
            out.append((HI, s, self.read_slot(int(row[s // 16]), HI, s % 16)))
        for s in range(n_lo):
            out.append((LO, s, self.read_slot(int(row[self.L - 1 - s // 32]), LO, s % 32)))
        return out


def prompt_allocate(H: int, T_h: int, T_l: int, L_max: int, seqlens, n_hi, n_lo,
                    free_list, ptr, status, page_table, tier_state):
    """Plan + allocation of prompt compaction on page counts (any page size)."""
    sl = np.ascontiguousarray(seqlens, dtype=np.int64)
    nh = np.ascontiguousarray(n_hi, dtype=np.int32)
    nl = np.ascontiguousarray(n_lo, dtype=np.int32)
    _check(lib().orc_prompt_allocate(ctypes.c_int32(H), ctypes.c_int32(T_h), ctypes.c_int32(T_l),
                                     ctypes.c_int32(L_max), ctypes.c_int32(sl.size), _p(sl), _p(nh),
                                     _p(nl), _p(free_list), _p(ptr), _p(status),
                                     ctypes.c_int64(free_list.size), _p(page_table),
                                     _p(tier_state)))


def attention_dense(q, k, v) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    out = np.zeros(q.size, np.float64)
    lib().orc_attention_dense(_p(q), _p(k), _p(v), ctypes.c_int32(k.shape[0]),
                              ctypes.c_int32(q.size), _p(out))
    return out


def attention_unit_vectors(q, k, v) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    out = np.zeros(q.size, np.float64)
    lib().orc_attention_unit_vectors(_p(q), _p(k), _p(v), ctypes.c_int32(k.shape[0]),
                                     ctypes.c_int32(q.size), _p(out))
    return out


def importance_from_queries(cfg: dict, cu_seqlens, k, qprobe) -> np.ndarray:
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    kk = np.ascontiguousarray(k, dtype=np.uint16)
    qp = np.ascontiguousarray(qprobe, dtype=np.uint16)
    H = int(cfg["num_kv_heads"])
    nq = qp.shape[1]
    scores = np.zeros((H, int(cu[-1])), np.float32)
    _check(lib().orc_importance_from_queries(ctypes.byref(make_cfg(cfg)), ctypes.c_int32(cu.size - 1),
                                             _p(cu), _p(kk), ctypes.c_int32(nq), _p(qp), _p(scores)))
    return scores


def importance_causal(cfg: dict, cu_seqlens, q, k, tail: int = 0) -> np.ndarray:
    """Per-token mean attention received from the later tokens of its prompt
    (causal softmax, max over the group's q heads): fp32 [H, total].  tail > 0:
    only the last `tail` tokens of each request (the others stay 0)."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    qq = np.ascontiguousarray(q, dtype=np.uint16)
    kk = np.ascontiguousarray(k, dtype=np.uint16)
    H = int(cfg["num_kv_heads"])
    scores = np.zeros((H, int(cu[-1])), np.float32)
    _check(lib().orc_importance_causal_tail(ctypes.byref(make_cfg(cfg)), ctypes.c_int32(cu.size - 1), _p(cu),
                                            _p(qq), _p(kk), ctypes.c_int64(tail), _p(scores)))
    return scores


def keydiff_scores(cfg: dict, cu_seqlens, k, anchor_raw: bool = False) -> np.ndarray:
    """Query-free importance from the keys alone (anchor cosine): fp32 [H, total]."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    kk = np.ascontiguousarray(k, dtype=np.uint16)
    H = int(cfg["num_kv_heads"])
    scores = np.zeros((H, int(cu[-1])), np.float32)
    _check(lib().orc_keydiff_scores(ctypes.byref(make_cfg(cfg)), ctypes.c_int32(cu.size - 1), _p(cu), _p(kk),
                                    ctypes.c_int32(1 if anchor_raw else 0), _p(scores)))
    return scores
