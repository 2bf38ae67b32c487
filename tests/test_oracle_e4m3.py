"""Pins of the oracle's E4M3 decode table: OCP spec values, an independent
bit-level decode, torch's float8_e4m3fn decode, and the table's structure."""

from tests import oracle_pins as pins


def test_table_matches_ocp_spot_values():
    pins.pin_table_vs_spec_values()


def test_table_matches_bit_assembly_all_codes():
    pins.pin_table_vs_bit_assembly()


def test_table_matches_torch_all_codes():
    pins.pin_table_vs_torch()


def test_table_structure():
    pins.pin_table_structure()
