"""CPU oracle for KV-cached action denoising.  TEST INFRASTRUCTURE ONLY:
imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg;
never by the product path."""
