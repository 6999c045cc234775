"""Seeded synthetic inputs (shared by the tests, the smoke check and the benchmark)."""
