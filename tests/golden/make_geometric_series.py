"""Writes geometric_series.txt: the exact closed form O_t = (1-γ^{t+1})/(1-γ) as
rationals, for γ = 1 - 2^-5 (the first head's decay of the tiny workload).

With θ = 0, q = k = e0 and v ≡ 1, retention reduces to the geometric series of the
decay along one row of D (hwhale.com RetNet notes, definition of D with the
diagonal included). Uses only fractions; imports neither the oracle nor the GPU
package."""
from fractions import Fraction
from pathlib import Path

g = 1 - Fraction(1, 32)
lines = ["# t  O_t  (exact rational; gamma on the first data row)", f"gamma {g}"]
for t in range(24):
    lines.append(f"{t} {(1 - g ** (t + 1)) / (1 - g)}")
Path(__file__).with_name("geometric_series.txt").write_text("\n".join(lines) + "\n")
