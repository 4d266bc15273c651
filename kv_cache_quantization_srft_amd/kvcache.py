"""A decoder's quantized KV cache: for every layer, K and V held as rotated
int4/int8 codes plus fp16 group scales in preallocated head-major buffers
[B, H, capacity, .], grown by quantize-on-append and read back by dequantize
+ unrotate.  This is the role the pages give their fused kernel inside a
growing int4 KV cache (a HuggingFace ``Cache`` subclass; "When Quantization
Is Free", Metodologia section 2), without the HuggingFace dependency.

Buffers are torch tensors; every quantize and dequantize runs in libsrftq's
kernels (``srftq_cache_append`` / ``srftq_cache_read``).  Per-sequence write
positions live on the device, so a decode loop appends without a host round
trip; ``advance`` moves them on the stream.

``save`` / ``load`` keep a cache on disk in its compressed form (the pages'
persistent-memory use of the codes): a safetensors file with the code and
scale rows written so far, the write positions, the sign and lambda rows,
and the format parameters as metadata.  Loading executes nothing from the
file.
"""
from __future__ import annotations

from . import srftq as S


class QuantizedKVCache:
    """K/V caches of ``n_layers`` layers for ``batch`` sequences of ``heads``
    KV heads of size ``d``, ``capacity`` tokens each.

    ``signs``: int8 [n_layers, 2, batch, heads, d] (index 1: 0 = K, 1 = V) or
    None (no sign diagonal).  ``lam``: fp32 of the same shape or None
    (lambda = 1).  Both are inputs: the cache draws no random numbers.
    """

    def __init__(self, n_layers, batch, heads, d, capacity, group=16, bits=4, rot="srft",
                 signs=None, lam=None, device="cuda"):
        import torch
        self.n_layers, self.B, self.H, self.d = int(n_layers), int(batch), int(heads), int(d)
        self.capacity, self.group, self.bits, self.rot = int(capacity), int(group), int(bits), rot
        sh = S.make_shape(self.B, 1, self.H, self.d, self.group, self.bits, rot)
        S._check(S.srftq_validate(sh), "QuantizedKVCache")
        side = (self.n_layers, 2, self.B, self.H, self.d)
        for name, t, dt in (("signs", signs, torch.int8), ("lam", lam, torch.float32)):
            if t is not None and (tuple(t.shape) != side or t.dtype != dt):
                raise ValueError(f"{name} must be {dt} of shape {side}")
        self.signs = None if signs is None else signs.to(device).contiguous()
        self.lam = None if lam is None else lam.to(device).contiguous()
        lead = (self.n_layers, 2, self.B, self.H, self.capacity)
        self.codes = torch.zeros(lead + (self.d * self.bits // 8,), dtype=torch.uint8, device=device)
        self.scales = torch.zeros(lead + (self.d // self.group,), dtype=torch.float16, device=device)
        self.pos = torch.zeros((self.B,), dtype=torch.int32, device=device)
        self.length = 0   # tokens appended so far (the same for every sequence unless reset)

    def _side(self, t, layer, kind):
        return None if t is None else t[layer, kind]

    def reset(self, positions=None):
        """Start over; ``positions`` (int32 [B]) sets each sequence's next row."""
        if positions is None:
            self.pos.zero_()
            self.length = 0
        else:
            self.pos.copy_(positions.to(self.pos.device, self.pos.dtype))
            self.length = int(self.pos.max().item()) if self.B else 0

    def append(self, layer, k, v, stream=None):
        """Quantize k, v fp16 [B, n, H, d] into rows pos[b] .. pos[b]+n-1 of
        layer ``layer`` (rows past the capacity are dropped)."""
        for kind, x in ((0, k), (1, v)):
            S.cache_append(x, self.codes[layer, kind], self.scales[layer, kind], self.pos,
                           self._side(self.signs, layer, kind), self._side(self.lam, layer, kind),
                           self.group, self.bits, self.rot, stream=stream)

    def advance(self, n):
        """Move every sequence's write position on by n tokens."""
        self.pos += int(n)
        self.length += int(n)

    def read(self, layer, T=None, stream=None):
        """(K, V) fp16 [B, T, H, d]: rows [0, T) of layer ``layer``
        (default: the tokens appended so far)."""
        T = self.length if T is None else int(T)
        return tuple(S.cache_read(self.codes[layer, kind], self.scales[layer, kind], T,
                                  self._side(self.signs, layer, kind), self._side(self.lam, layer, kind),
                                  self.group, self.bits, self.rot, d=self.d, stream=stream)
                     for kind in (0, 1))

    def update(self, layer, k, v, stream=None):
        """Append k, v to ``layer`` and return its whole (K, V) so far; the
        positions advance after the last layer (one decode step)."""
        n = k.shape[1]
        self.append(layer, k, v, stream)
        out = self.read(layer, self.length + n, stream)
        if layer == self.n_layers - 1:
            self.advance(n)
        return out

    def nbytes(self):
        """Bytes held for codes and scales."""
        return self.codes.numel() + 2 * self.scales.numel()

    FORMAT = "srftq-kvcache-1"

    def save(self, path):
        """Write rows [0, max(pos)) of every layer's codes and scales, the
        positions, signs, lambda and format parameters to ``path``
        (safetensors)."""
        from safetensors.torch import save_file
        rows = min(int(self.pos.max().item()) if self.B else 0, self.capacity)
        t = {"codes": self.codes[..., :rows, :].contiguous().cpu(),
             "scales": self.scales[..., :rows, :].contiguous().cpu(),
             "pos": self.pos.cpu()}
        if self.signs is not None:
            t["signs"] = self.signs.cpu()
        if self.lam is not None:
            t["lam"] = self.lam.cpu()
        meta = {"format": self.FORMAT, "n_layers": self.n_layers, "batch": self.B, "heads": self.H, "d": self.d,
                "capacity": self.capacity, "group": self.group, "bits": self.bits, "rot": self.rot,
                "length": self.length, "rows": rows}
        save_file(t, str(path), metadata={k: str(v) for k, v in meta.items()})

    @classmethod
    def load(cls, path, device="cuda", capacity=None):
        """A cache read back from ``save``'s file, with ``capacity`` rows per
        sequence (default: the saved capacity; never fewer than the saved
        rows)."""
        from safetensors import safe_open
        with safe_open(str(path), framework="pt") as f:
            meta = f.metadata() or {}
            if meta.get("format") != cls.FORMAT:
                raise ValueError(f"{path}: not a {cls.FORMAT} file")
            t = {k: f.get_tensor(k) for k in f.keys()}
        ints = {k: int(meta[k]) for k in ("n_layers", "batch", "heads", "d", "capacity", "group", "bits",
                                          "length", "rows")}
        cap = ints["capacity"] if capacity is None else int(capacity)
        if cap < ints["rows"]:
            raise ValueError(f"capacity {cap} is below the {ints['rows']} saved rows")
        c = cls(ints["n_layers"], ints["batch"], ints["heads"], ints["d"], cap, ints["group"], ints["bits"],
                meta["rot"], signs=t.get("signs"), lam=t.get("lam"), device=device)
        rows = ints["rows"]
        if tuple(t["codes"].shape) != tuple(c.codes.shape[:-2]) + (rows, c.codes.shape[-1]) or \
                tuple(t["scales"].shape) != tuple(c.scales.shape[:-2]) + (rows, c.scales.shape[-1]):
            raise ValueError(f"{path}: code or scale rows do not match the saved parameters")
        c.codes[..., :rows, :].copy_(t["codes"])
        c.scales[..., :rows, :].copy_(t["scales"])
        c.pos.copy_(t["pos"])
        c.length = ints["length"]
        return c
