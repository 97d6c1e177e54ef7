"""CPU oracle of the Key-Value Means attention layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import, call or run anything under oracle/.  The HIP library and its Python
binding never use it and share no code with it.
"""
