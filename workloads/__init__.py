"""Seeded synthetic workloads for the tests and the benchmark (not part of the
library): logits of the shapes and distributions the verification step is
measured on, and drafted tokens standing in for the draft model's own draws."""
