"""Session persistence, tier telemetry and debug snapshots of a TieredCache.

Host-side plumbing around the device tiers (no arithmetic of the method runs
here):

* Persistence (FADE post, section "会话持久化"): the compressed cache is
  saved and restored as it is - packed codes, fp16 scales, the fp16 sink and
  recent tiers, the INT2 overflow tier when there is one, a PQ middle tier's
  codebooks, the per-sequence lengths and the per-slot scores - so a
  restored cache attends, scores and evicts exactly as the saved one would.
  Files are safetensors (no code runs on load); the configuration travels in
  the file's metadata and must match the cache it is loaded into.
* Telemetry (section "遥测与调试"): one JSON line per tier reassignment
  event, with the layer, the token count of each tier per sequence, score
  statistics over the live slots and the compressed bytes of the layer.
* Debug snapshot (same section): a JSON file with the configuration, the
  lengths and the same statistics.
"""
import json

import numpy as np
import torch

from . import fade

_TENSORS = ("fp_k", "fp_v", "mid_k_codes", "mid_v_codes", "mid_k_scales", "mid_v_scales", "lens", "scores")
_LOW_TENSORS = ("low_k_codes", "low_v_codes", "low_k_scales", "low_v_scales", "low_lens")
_PQ_TENSORS = ("pq_k_codebook", "pq_v_codebook")   # the layer's codebooks of a PQ middle tier
_CFG_FIELDS = ("head_dim", "n_q_heads", "n_kv_heads", "n_sink", "recent_window", "int4_budget",
               "middle_k_bits", "middle_v_bits", "group_size", "rope_type", "rope_theta", "rope_factor",
               "rope_low_freq_factor", "rope_high_freq_factor", "rope_original_max_position")


def _config_meta(cache):
    # The eviction budget is a policy knob, not part of the stored layout: a
    # cache may be restored under a different one.
    meta = {f: repr(getattr(cache.cfg, f)) for f in _CFG_FIELDS if f != "int4_budget"}
    meta.update(batch=str(cache.batch), shared=str(cache.shared), with_scores=str(cache.scores is not None),
                int2_tier=str(bool(getattr(cache, "low", False))), middle_pq=str(bool(getattr(cache, "pq", False))))
    return meta


def _names(cache):
    return (_TENSORS + (_LOW_TENSORS if getattr(cache, "low", False) else ()) +
            (_PQ_TENSORS if getattr(cache, "pq", False) else ()))


def _lens(cache):
    """Host copy of lens [batch, 4] = {n_sink_live, mid_len, rec_len, rec_head}."""
    return cache.lens.detach().cpu().numpy().astype(np.int64)


def _low_lens(cache):
    """Host copy of the INT2 tier's lengths [batch] (zeros without the tier)."""
    if not getattr(cache, "low", False):
        return np.zeros(cache.batch, dtype=np.int64)
    return cache.low_lens.detach().cpu().numpy().astype(np.int64)


def cache_state_dict(cache):
    """Host tensors of the live state. Middle (and INT2-tier) arrays are cut to
    the longest live tier of the batch and scores to the longest live length;
    every other array is whole."""
    lens = _lens(cache)
    low = _low_lens(cache)
    m_live = int(lens[:, 1].max()) if lens.size else 0
    l_live = int(low.max()) if low.size else 0
    t_live = int((lens[:, :3].sum(axis=1) + low).max()) if lens.size else 0
    sd = {}
    for name in _names(cache):
        t = getattr(cache, name)
        if t is None:
            continue
        if name.startswith("mid_"):
            t = t[:, :, :m_live]
        elif name.startswith("low_") and name != "low_lens":
            t = t[:, :, :l_live]
        elif name == "scores":
            t = t[:, :t_live]
        sd[name] = t.detach().cpu().contiguous()
    return sd


def load_cache_state_dict(cache, sd, meta=None):
    """Copy a state from cache_state_dict into `cache` (same configuration and
    batch, middle and INT2-tier capacities at least the saved live lengths).
    Score slots past the saved live length are zeroed."""
    if int(sd["lens"][:, 1].max()) > cache.cap_mid:
        raise ValueError("saved middle tier is longer than this cache's capacity")
    if "low_lens" in sd and int(sd["low_lens"].max()) > getattr(cache, "cap_low", 0):
        raise ValueError("saved INT2 tier is longer than this cache's capacity")
    if meta is not None:
        want = _config_meta(cache)
        diff = {k: (meta.get(k), v) for k, v in want.items()
                if meta.get(k, "False" if k in ("int2_tier", "middle_pq") else None) != v}
        if diff:
            raise ValueError(f"cache state does not match this cache: {diff}")
    names = _names(cache)
    if any(n in sd for n in _LOW_TENSORS) and not getattr(cache, "low", False):
        raise ValueError("cache state holds an INT2 tier this cache does not have")
    if any(n in sd for n in _PQ_TENSORS) and not getattr(cache, "pq", False):
        raise ValueError("cache state holds a PQ middle tier this cache does not have")
    # validate everything before the first copy
    for name in names:
        dst = getattr(cache, name)
        if (dst is None) != (name not in sd):
            raise ValueError(f"cache state and cache disagree on {name!r}")
        if dst is None:
            continue
        src = sd[name]
        if name.startswith("mid_") or (name.startswith("low_") and name != "low_lens"):
            ok = src.shape[:2] == dst.shape[:2] and src.shape[3:] == dst.shape[3:] and src.shape[2] <= dst.shape[2]
        elif name == "scores":
            ok = src.shape[0] == dst.shape[0] and src.shape[1] <= dst.shape[1]
        else:
            ok = src.shape == dst.shape
        if not ok or src.dtype != dst.dtype:
            raise ValueError(f"{name}: saved {tuple(src.shape)} {src.dtype} does not fit {tuple(dst.shape)} {dst.dtype}")
    for name in names:
        dst = getattr(cache, name)
        if dst is None:
            continue
        src = sd[name]
        if name.startswith("mid_") or (name.startswith("low_") and name != "low_lens"):
            dst[:, :, :src.shape[2]].copy_(src)
        elif name == "scores":
            dst.zero_()
            dst[:, :src.shape[1]].copy_(src)
        else:
            dst.copy_(src)


def save(cache, path):
    from safetensors.torch import save_file
    save_file(cache_state_dict(cache), path, metadata=_config_meta(cache))


def load(cache, path):
    from safetensors import safe_open
    with safe_open(path, framework="pt") as f:
        meta = f.metadata()
        sd = {k: f.get_tensor(k) for k in f.keys()}
    load_cache_state_dict(cache, sd, meta)


# ---- telemetry ------------------------------------------------------------------
def tier_stats(cache):
    """Per sequence: tier token counts and score statistics over the live slots."""
    lens = _lens(cache)
    low = _low_lens(cache)
    scores = None if cache.scores is None else cache.scores.detach().cpu().numpy()
    out = []
    for b in range(cache.batch):
        s, m, r = (int(x) for x in lens[b, :3])
        m2 = int(low[b])
        rec = {"sink": s, "int2": m2, "middle": m, "recent": r, "live": s + m2 + m + r}
        if scores is not None:
            row = scores[0 if cache.shared else b, :s + m2 + m + r].astype(np.float64)
            if row.size:
                rec["score_min"], rec["score_mean"], rec["score_max"] = (
                    float(row.min()), float(row.mean()), float(row.max()))
        out.append(rec)
    return out


def layer_record(cache, layer, event="evict"):
    seqs = tier_stats(cache)
    fp = [q["sink"] + q["recent"] for q in seqs]
    mid = [q["middle"] for q in seqs]
    low = [q["int2"] for q in seqs] if getattr(cache, "low", False) else None
    return {"event": event, "layer": int(layer), "seqs": seqs,
            "compressed_bytes": fade.fade_compressed_bytes(cache.cfg, fp, mid, low)}


class JsonlExporter:
    """Appends one JSON object per line to `path`."""

    def __init__(self, path):
        self.path = path
        self._f = open(path, "a", encoding="utf-8")

    def write(self, record):
        self._f.write(json.dumps(record, sort_keys=True) + "\n")
        self._f.flush()

    def close(self):
        self._f.close()


class Telemetry:
    def __init__(self, exporter, layer):
        self.exporter, self.layer, self.events = exporter, layer, 0

    def record(self, cache, event="evict"):
        rec = layer_record(cache, self.layer, event)
        rec["seq_no"] = self.events
        self.events += 1
        self.exporter.write(rec)


def attach_telemetry(cache, exporter, layer):
    """After this, every fade_evict_rerope call on `cache` through the Python
    binding writes one record (it reads the lengths and scores back, so it
    synchronizes the stream)."""
    cache.telemetry = Telemetry(exporter, layer)
    return cache.telemetry


def dump_debug(cache, path, layer=0):
    snap = {"config": {f: getattr(cache.cfg, f) for f in _CFG_FIELDS + ("int2_budget",)},
            "batch": cache.batch, "cap_mid": cache.cap_mid, "cap_low": getattr(cache, "cap_low", 0),
            "cap_T": cache.cap_T, "shared": cache.shared, "lens": _lens(cache).tolist(),
            "low_lens": _low_lens(cache).tolist(), "record": layer_record(cache, layer, event="snapshot")}
    with open(path, "w", encoding="utf-8") as f:
        json.dump(snap, f, indent=1, sort_keys=True)
    return snap
