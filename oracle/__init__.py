"""CPU oracle: plain, slow, obviously-correct codec and fp64 attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg import this package; the library under decode_attention_losslessly_amd/ never does.
"""
