"""The oracle's pins catch plausible mistakes (CPU only).

Each case compiles a copy of oracle/ra_oracle.c with one planted mistake (a
dropped term, a wrong sign or index, a swapped operand), loads it in place of
the real oracle and runs the pins: at least one pin must fail.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ra_oracle.c")

MUTANTS = {
    "causal_mask_off_by_one": ("return p->kv_off + j <= p->q_off + i;", "return p->kv_off + j < p->q_off + i;"),
    "gqa_head_map": ("const int64_t g = h / (p->hq / p->hkv);", "const int64_t g = h % p->hkv;"),
    "merge_weight_sign": ("exp(ma[r] - mm)", "exp(mm - ma[r])"),
    "ring_direction": ("int64_t j = (rank - s) % P;", "int64_t j = (rank + s) % P;"),
    "lse_sign": ("lse[r] = m[r] + log(l[r]);", "lse[r] = m[r] - log(l[r]);"),
    "dropped_channel": ("o_out[c] += w * vj[c];", "o_out[c] += (c ? w * vj[c] : 0.0);"),
    "key_used_as_value": ("const double *vj = p->v +", "const double *vj = p->k +"),
    "scale_dropped": ("s[j] = p->scale * dot;", "s[j] = dot;"),
    "max_not_subtracted_in_l": ("l += w;", "l += exp(s[j]);"),
    "classify_full_off_by_one": ("if (kv_off + nkv - 1 <= q_off) return 1;", "if (kv_off + nkv <= q_off) return 1;"),
    "flops_partial_weight": ("cls == 2 ? 0.5 : 0.0", "cls == 2 ? 1.0 : 0.0"),
    "zigzag_second_chunk_position": ("const int64_t q_off[2] = {rank * c, (2 * P - 1 - rank) * c - c};",
                                     "const int64_t q_off[2] = {rank * c, (2 * P - 1 - rank) * c};"),
    "zigzag_key_chunk": ("const int64_t chunks[2] = {j, 2 * P - 1 - j};", "const int64_t chunks[2] = {j, 2 * P - 2 - j};"),
    "zigzag_flops_key_chunk": ("const int64_t kpos[2] = {j * c, (2 * P - 1 - j) * c};",
                               "const int64_t kpos[2] = {j * c, (2 * P - 2 - j) * c};"),
    "bwd_ds_sign": ("const double ds = p * (dp - D);", "const double ds = p * (D - dp);"),
    "bwd_dk_scale_dropped": ("dk[c] += w->scale * ds * qi[c];", "dk[c] += ds * qi[c];"),
    "bwd_dv_uses_ds": ("dv[c] += p * doi[c];", "dv[c] += ds * doi[c];"),
    "bwd_D_from_q": ("*D_out = bwd_dot(w->dout + ((b * w->nb + i) * w->hq + h) * d, o, d);",
                     "*D_out = bwd_dot(w->dout + ((b * w->nb + i) * w->hq + h) * d, qi, d);"),
    "bwd_zigzag_second_chunk": ("return i < c ? w->rank * c + i : (2 * w->P - 1 - w->rank) * c + (i - c);",
                                "return i < c ? w->rank * c + i : (2 * w->P - 2 - w->rank) * c + (i - c);"),
    "bwd_padding_key_visible": ("return j < w->kv_end && (!w->causal", "return j <= w->kv_end && (!w->causal"),
    "padded_real_keys_off_by_one": ("const int64_t real = n_valid - j * nb;", "const int64_t real = n_valid + 1 - j * nb;"),
    "pairs_count_off_by_one": ("int64_t c = causal ? q_off + i - kv_off + 1 : nkv;", "int64_t c = causal ? q_off + i - kv_off : nkv;"),
}

PINS = [
    lambda: [pins.test_oracle_matches_brute_force(*a) for a in (
        (1, 8, 8, 2, 2, 8, 0, 0, True), (1, 12, 12, 2, 1, 4, 0, 0, True), (1, 4, 12, 1, 1, 8, 3, 2, False))],
    lambda: pins.test_oracle_gqa_matches_library_routine(),
    lambda: pins.test_oracle_matches_library_routine_tiny_workload(True),
    lambda: pins.test_identical_keys_give_mean_of_visible_values(),
    lambda: pins.test_value_identity_gives_softmax_weights(),
    lambda: pins.test_merge_identity_commutative_associative(),
    lambda: pins.test_ring_order_matches_a_simulated_ring(),
    lambda: pins.test_last_rank_skips_no_block(),
    lambda: pins.test_classify_and_pair_count_match_brute_force(),
    lambda: pins.test_share_flops_rule(),
    lambda: pins.test_zigzag_share_is_full_attention_at_its_positions(1, 48, 3, 2, 1, 8, True),
    lambda: pins.test_zigzag_flops_rule_and_balance(),
    lambda: pins.test_backward_matches_torch_autograd(1, 24, 3, 2, 1, 8, True),
    lambda: pins.test_padded_share_is_attention_over_the_real_keys(1, 22, 4, 2, 1, 8, True),
    lambda: pins.test_zigzag_backward_matches_torch_autograd(1, 24, 3, 2, 1, 8, True),
    lambda: pins.test_padded_backward_matches_torch_autograd(1, 22, 4, 2, 1, 8, True),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    c = tmp_path / "mutant.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", str(c), "-o", str(so),
                           "-lpthread", "-lm"])
    oracle._load(str(so))
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin)
                break
    finally:
        oracle._reset()
    assert caught, f"no pin caught the planted mistake {name}"
