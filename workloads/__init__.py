"""Seeded synthetic workloads for the DSpark per-step verify path.

This module only draws inputs. It performs none of the method's arithmetic
(no sigmoid, no survival product, no sort, no argmax, no softmax): where a
workload needs to know which vocabulary id is a row's maximum (to plant draft
tokens that the target would accept), the maximum is *placed* there by
construction. Rows are clipped to a cap and then receive one planted value
above that cap.

Both the oracle side (tests, CPU baseline) and the GPU side (tests, bench)
receive the same host arrays from here; nothing here depends on either.

Workload recipes (sizes, distributions and structure) follow the five
configurations the build measures. Their prose source is the DSpark pages:
B requests x gamma drafted positions, confidence logits with suffix decay,
per-position STS temperatures, an additive cost table
T = bias + alpha(bs) + theta(M), captured packed-row tiers, and target logits
over a vocabulary V.
"""

from .gen import CONFIGS, Workload, make, bf16_bits_to_f32, f32_to_bf16_bits

__all__ = ["CONFIGS", "Workload", "make", "bf16_bits_to_f32", "f32_to_bf16_bits"]
