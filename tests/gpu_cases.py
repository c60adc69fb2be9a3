"""Shared set-up for the GPU parity tests: the same seeded inputs go to the HIP
path (through the C ABI binding) and to the oracle, which computes on its own."""
import math

import numpy as np
import torch

import long_context_attention_kv_amd as f4
import synth
from oracle import attention as oatt
from oracle import f4 as of4

PAGE = 64
ATT_TOL = 2e-3  # max |delta| relative to the oracle output's RMS


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def cache_arrays_equal(gc: f4.F4Cache, oc: of4.Cache):
    """Compare the four arrays byte for byte; returns a list of mismatching array names."""
    bad = []
    ok_k, ok_ks, ok_v, ok_vs = oc.arrays()
    pairs = [("k_nib", gc.k_nib, ok_k), ("k_scale", gc.k_scale, ok_ks.view(np.int16)),
             ("v_nib", gc.v_nib, ok_v), ("v_scale", gc.v_scale, ok_vs.view(np.int16))]
    for name, g, o in pairs:
        if not np.array_equal(g.cpu().numpy(), o):
            bad.append(name)
    return bad


class PagedSet:
    """Sequences of given lengths in one shared pool, written by both sides."""

    def __init__(self, lengths, Hkv=4, D=256, seed=0, extra_pages=3, k_scale=1.0, v_scale=1.0, outliers=False,
                 placement=0, v_per_token=False, k_edit=None):
        self.lengths = [int(x) for x in lengths]
        self.Hkv, self.D = Hkv, D
        g = synth.rng(100 + seed, 0)
        pages = [(n + PAGE - 1) // PAGE for n in self.lengths]
        self.num_pages = max(1, sum(pages) + extra_pages)
        self.max_pages = max(1, max(pages) if pages else 1)
        perm = synth.page_permutation(synth.rng(100 + seed, 1 + placement), self.num_pages)
        self.pt = synth.page_table_for(self.lengths, perm, self.max_pages)
        T = sum(self.lengths)
        k = synth.normal_f32(g, (T, Hkv, D)) * np.float32(k_scale)
        v = synth.normal_f32(g, (T, Hkv, D)) * np.float32(v_scale)
        if outliers:
            cols = synth.outlier_columns(g, Hkv, D)
            synth.apply_outliers(k, cols)
            synth.apply_outliers(v, cols)
        if k_edit is not None:  # e.g. plant dominant keys (attention sinks)
            k_edit(k)
        slots = []
        for b, n in enumerate(self.lengths):
            t = np.arange(n)
            slots.append(self.pt[b, t // PAGE].astype(np.int64) * PAGE + t % PAGE)
        self.slots = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
        self.k, self.v = k, v
        self.oc = of4.Cache(self.num_pages, Hkv, D, v_per_token=v_per_token)
        self.oc.write(k, v, self.slots)
        self.gc = f4.F4Cache(self.num_pages, Hkv, D, v_scale_per_token=v_per_token)
        if T:
            f4.kv_cache_write_f4(self.gc, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                 torch.from_numpy(self.slots).cuda())
        torch.cuda.synchronize()

    def gpu_page_table(self):
        return torch.from_numpy(self.pt).cuda()

    def gpu_lengths(self):
        return torch.tensor(self.lengths, dtype=torch.int32, device="cuda")


def assert_attention_close(out, ref, what=""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.max(np.abs(out - ref))) if ref.size else 0.0
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    assert err <= ATT_TOL * rms + 1e-30, f"{what}: max|delta| {err:.3e} > {ATT_TOL} x RMS {rms:.3e}"
    return err / rms if rms > 0 else 0.0


def assert_states_close(m, l, rm, rl, what=""):
    m = np.asarray(m, np.float64)
    l = np.asarray(l, np.float64)
    empty = ~np.isfinite(rm)
    assert np.all(~np.isfinite(m[empty])) and np.all(l[empty] == 0), f"{what}: empty ranges"
    live = ~empty
    assert np.all(np.abs(m[live] - rm[live]) <= 1e-3 * np.maximum(1.0, np.abs(rm[live]))), f"{what}: m"
    assert np.all(np.abs(l[live] - rl[live]) <= 2e-3 * rl[live]), f"{what}: l"


def random_q(B, Hq, D, seed, scale=1.0):
    g = synth.rng(200 + seed, 1)
    qf = synth.normal_f32(g, (B, Hq, D)) * np.float32(scale)
    bits = synth.f32_to_bf16_bits(qf)
    return bits, bf16_values(bits)


def oracle_decode(ps: PagedSet, qvals, sm_scale, num_windows=1, window_tokens=0):
    return oatt.decode(ps.oc, qvals, ps.pt, ps.lengths, sm_scale, window_tokens=window_tokens,
                       num_windows=num_windows)
