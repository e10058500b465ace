"""The CPU oracle against the pages' worked example, the chunk-invariance
statement, closed forms, dense brute force and the block-table fingerprint."""
import pytest

import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def test_worked_example_metadata(orc):
    P.pin_worked_example_metadata(orc)


def test_worked_example_visibility(orc):
    P.pin_worked_example_visibility(orc)


def test_worked_example_perturbation(orc):
    P.pin_worked_example_perturbation(orc)


def test_chunk_invariance_10000_as_5_chunks(orc):
    P.pin_chunk_invariance(orc)


def test_textbook_causal(orc):
    P.pin_textbook_causal(orc)


def test_decode_unmasked(orc):
    P.pin_decode_unmasked(orc)


def test_prefix_means(orc):
    P.pin_prefix_means(orc)


def test_single_key(orc):
    P.pin_single_key(orc)


def test_constant_values_and_bounds(orc):
    P.pin_constant_values_and_bounds(orc)


def test_brute_force_sweep(orc):
    P.pin_brute_force(orc)


def test_block_table_fingerprint(orc):
    P.pin_block_table_fingerprint(orc)


def test_nan_hygiene(orc):
    P.pin_nan_hygiene(orc)


def test_append_bytes(orc):
    P.pin_append(orc)


def test_check_slots(orc):
    P.pin_check_slots(orc)
