"""Test and benchmark harness: seeded synthetic inputs (``inputs``, numpy only,
shared by the oracle's tests, the GPU parity tests and the benchmark) and
GPU-resident problems built from them (``synthetic``).  Holds none of the
feed-forward's arithmetic; not part of the library."""
