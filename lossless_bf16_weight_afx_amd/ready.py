"""Time-to-ready arithmetic of "Why Weight Offloading Slows Inference".

Section "Three steps for each weight", Eq. (1): the time until a stored weight
is ready on the GPU is about  S_disk / b_disk + t_unpack + S / b_PCIe,  with
S_disk the stored size, b_disk the read speed, t_unpack the unpacking time, S
the unpacked size and b_PCIe the copy speed (the page's text lost the fraction
bars; this reading reproduces the figures the page derives from it).

Section "Lossless compression", Eq. (2): compression shortens that time only
when the read time it saves exceeds the unpack time it adds,
(S - S_disk) / b_disk > t_unpack.

When the unpack runs on the GPU after the copy, the link carries the stored
bytes instead of the unpacked ones; ``t_prep_gpu_unpack`` is that variant.
"""


def t_prep(s_disk: float, b_disk: float, t_unpack: float, s: float, b_pcie: float) -> float:
    """Eq. (1): read the stored bytes, unpack on the host, copy S bytes."""
    return s_disk / b_disk + t_unpack + s / b_pcie


def t_prep_gpu_unpack(s_disk: float, b_disk: float, b_link: float, t_unpack: float) -> float:
    """Eq. (1) with the unpack moved after the copy: the link carries S_disk."""
    return s_disk / b_disk + s_disk / b_link + t_unpack


def compression_pays(s: float, s_disk: float, b: float, t_unpack: float) -> bool:
    """Eq. (2): bytes saved over the slowest stage ``b`` outweigh unpacking."""
    return (s - s_disk) / b > t_unpack
