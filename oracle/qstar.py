"""The bandwidth-adaptive fill count.

With m misses of record size S, filling q of them over PCIe takes about
q S / B_P, and running the other m - q on the host takes about
(m - q) S / (B_H - B_P), because the fills draw on the same host memory
("Making Large MoE Models Practical on a Single Machine", section 5 "Deriving
q*").  Equating the two branches gives q* = m B_P / B_H (same page, boxed
equation; METAL MEDIA summary, Figure 2 caption).  The txtmix article (section
"它在解一个什么问题", the q* policy) adds that at least one fill is always kept
and that q* tends to m as B_H approaches B_P.

Readings taken where the pages stop:
  * q* is rounded half up, computed exactly from integer MB/s:
    floor((2 m B_P + B_H) / (2 B_H));
  * the at-least-one-fill rule needs a slot that is free to evict
    (evictable = N - hits) and a fetch cap that is not 0;
  * q never exceeds m, the evictable slots, or the cap (max_fetch >= 0;
    -1 means no cap).
"""


def fill_count(m: int, hits: int, slots: int, bp_mbps: int, bh_mbps: int, max_fetch: int = -1) -> int:
    if m <= 0:
        return 0
    if bp_mbps <= 0 or bh_mbps <= 0:
        raise ValueError("bandwidths must be positive")
    q = (2 * m * bp_mbps + bh_mbps) // (2 * bh_mbps)   # round half up of m*B_P/B_H
    q = max(q, 1)
    q = min(q, m, slots - hits)
    if max_fetch >= 0:
        q = min(q, max_fetch)
    return max(q, 0)
