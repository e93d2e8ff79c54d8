"""The pins must fail when a plausible mistake is planted in the oracle.

Each case monkeypatches one oracle function with a wrong variant (on the CPU
only) and checks that at least one of the pin tests for that function raises.
"""
import numpy as np
import pytest

from oracle import gdn, quant
from tests import test_oracle_gdn as tg
from tests import test_oracle_quant as tq


def _wrong_sign(M, q, k, v, alpha, beta):
    a = alpha[:, None, None]
    b = beta[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)
    M = a * (M + b * k[:, :, None] * kM[:, None, :]) + b * k[:, :, None] * v[:, None, :]
    return M, np.einsum("ni,nij->nj", q, M)


def _gate_misplaced(M, q, k, v, alpha, beta):
    a = alpha[:, None, None]
    b = beta[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)
    M = a * M - b * k[:, :, None] * kM[:, None, :] + b * k[:, :, None] * v[:, None, :]
    return M, np.einsum("ni,nij->nj", q, M)


def _transposed_write(M, q, k, v, alpha, beta):
    a = alpha[:, None, None]
    b = beta[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)
    M = a * (M - b * k[:, :, None] * kM[:, None, :]) + b * v[:, :, None] * k[:, None, :]
    return M, np.einsum("ni,nij->nj", q, M)


def _read_before_write(M, q, k, v, alpha, beta):
    o = np.einsum("ni,nij->nj", q, M)
    a = alpha[:, None, None]
    b = beta[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)
    M = a * (M - b * k[:, :, None] * kM[:, None, :]) + b * k[:, :, None] * v[:, None, :]
    return M, o


def _no_beta_on_write(M, q, k, v, alpha, beta):
    a = alpha[:, None, None]
    b = beta[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)
    M = a * (M - b * k[:, :, None] * kM[:, None, :]) + k[:, :, None] * v[:, None, :]
    return M, np.einsum("ni,nij->nj", q, M)


GDN_PINS = [tg.test_beta_zero_is_pure_decay, tg.test_basis_key_overwrites_one_row_exactly,
            tg.test_one_token_from_zero, tg.test_delta_rule_maps_key_to_value,
            lambda: [tg.test_exact_rational_brute_force(s) for s in range(3)]]


@pytest.mark.parametrize("bad", [_wrong_sign, _gate_misplaced, _transposed_write,
                                 _read_before_write, _no_beta_on_write])
def test_gdn_pins_catch(bad, monkeypatch):
    monkeypatch.setattr(gdn, "step", bad)
    caught = 0
    for pin in GDN_PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, bad.__name__


def _enc_half_up(M, bits):
    M = np.asarray(M, dtype=np.float64)
    qm = quant._qmax_per_tile(bits, M.shape[:-2])[..., None]
    a = np.max(np.abs(M), axis=-2)
    s = (a / qm).astype(np.float32)
    s64 = s.astype(np.float64)[..., None, :]
    x = np.where(s64 > 0, M / np.where(s64 > 0, s64, 1), 0.0)
    return np.clip(np.floor(x + 0.5), -qm[..., None], qm[..., None]).astype(np.int16), s


def _enc_wrong_qmax(M, bits):
    M = np.asarray(M, dtype=np.float64)
    qm = quant._qmax_per_tile(bits, M.shape[:-2])[..., None] + 1
    a = np.max(np.abs(M), axis=-2)
    s = (a / qm).astype(np.float32)
    s64 = s.astype(np.float64)[..., None, :]
    x = np.where(s64 > 0, M / np.where(s64 > 0, s64, 1), 0.0)
    return np.clip(np.rint(x), -qm[..., None], qm[..., None]).astype(np.int16), s


def _enc_row_scales(M, bits):
    c, s = quant.__dict__["_orig_encode"](np.swapaxes(M, -1, -2), bits)
    return np.swapaxes(c, -1, -2), s


def _enc_scale_f64(M, bits):
    M = np.asarray(M, dtype=np.float64)
    qm = quant._qmax_per_tile(bits, M.shape[:-2])[..., None]
    a = np.max(np.abs(M), axis=-2)
    s = a / qm
    s64 = s[..., None, :]
    x = np.where(s64 > 0, M / np.where(s64 > 0, s64, 1), 0.0)
    return np.clip(np.rint(x), -qm[..., None], qm[..., None]).astype(np.int16), s


QUANT_PINS = [lambda: [tq.test_constructed_exact_ties_go_to_even(b) for b in (4, 8)],
              lambda: [tq.test_zero_column(b) for b in (4, 8)],
              lambda: [tq.test_quantizer_invariants_gaussian(b) for b in (4, 8)],
              tq.test_scale_is_absmax_over_qmax_in_float32]


@pytest.mark.parametrize("bad", [_enc_half_up, _enc_wrong_qmax, _enc_row_scales, _enc_scale_f64])
def test_quant_pins_catch(bad, monkeypatch):
    monkeypatch.setitem(quant.__dict__, "_orig_encode", quant.encode)
    monkeypatch.setattr(quant, "encode", bad)
    caught = 0
    for pin in QUANT_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, bad.__name__


# ---- FP8 window flush (oracle/window.py Window.flush) ----

from oracle import window  # noqa: E402
from tests import test_oracle_window as tw  # noqa: E402


def _flush_variant(no_lam=False, no_delta=False, swap_delta=False):
    def flush(self):
        for i in range(self.codes.shape[0]):
            if not self.win[i]:
                continue
            lam = 1.0 if no_lam else self.lam[i]
            H = lam * quant.decode(self.codes[i], self.scales[i])
            deltas = [e[4] for e in self.win[i]]
            if swap_delta:
                deltas = deltas[::-1]
            for (kc, ks, uc, us, _), delta in zip(self.win[i], deltas):
                dl = 1.0 if no_delta else delta
                H = H + dl * np.outer(window.fp8_decode(kc, ks), window.fp8_decode(uc, us))
            c, s = quant.encode(H[None], self.bits[i:i + 1])
            self.codes[i], self.scales[i] = c[0], s[0]
            self.lam[i] = 1.0
            self.win[i] = []
            self.last_pre[i] = H
    return flush


FLUSH_PINS = [lambda: [tw.test_flush_equals_encode_of_the_recurrence(s) for s in (0, 1, 2)]]


@pytest.mark.parametrize("bad", [dict(no_lam=True), dict(no_delta=True), dict(swap_delta=True)],
                         ids=["lam_dropped", "delta_dropped", "delta_order_reversed"])
def test_flush_pins_catch(bad, monkeypatch):
    monkeypatch.setattr(window.Window, "flush", _flush_variant(**bad))
    caught = 0
    for pin in FLUSH_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, bad


def test_flush_variant_without_mistakes_passes(monkeypatch):
    # the planted variants differ from the oracle only by their mistake
    monkeypatch.setattr(window.Window, "flush", _flush_variant())
    for pin in FLUSH_PINS:
        pin()


# ---- quotients (oracle/quant.py quotients) ----

def _quot_row_scales(M, scales):
    s64 = np.asarray(scales, dtype=np.float64)[..., :, None]
    safe = np.where(s64 > 0, s64, 1.0)
    return np.where(s64 > 0, np.asarray(M, dtype=np.float64) / safe, 0.0)


def _quot_float32(M, scales):
    s32 = np.asarray(scales, dtype=np.float32)[..., None, :]
    safe = np.where(s32 > 0, s32, np.float32(1))
    return np.where(s32 > 0, np.asarray(M, dtype=np.float32) / safe, 0).astype(np.float64)


def _quot_no_zero_guard(M, scales):
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.asarray(M, dtype=np.float64) / np.asarray(scales, dtype=np.float64)[..., None, :]


def _quot_recomputed_scale(M, scales):
    a = np.max(np.abs(np.asarray(M, dtype=np.float64)), axis=-2)[..., None, :]
    return np.where(a > 0, M / np.where(a > 0, a / 7, 1), 0.0)


QUOT_PINS = [tq.test_quotients_constructed_values, tq.test_quotients_keep_float64_precision_near_ties,
             lambda: [tq.test_quotients_round_to_the_encoded_codes(b) for b in (4, 8)]]


@pytest.mark.parametrize("bad", [_quot_row_scales, _quot_float32, _quot_no_zero_guard,
                                 _quot_recomputed_scale])
def test_quotient_pins_catch(bad, monkeypatch):
    monkeypatch.setattr(quant, "quotients", bad)
    caught = 0
    for pin in QUOT_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught >= 1, bad.__name__
