"""MI355X (gfx950) Q8_0 decode matvec and i8 dot_t behind a C ABI (include/q8_gemv.h).

The kernels live in ``csrc/`` and are built into ``libq8gemv.so`` by
``build.py``; ``binding`` is the thin ctypes layer over that library.
Importing this package loads nothing; the library is loaded on first use.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    Q8Error,
    q8_dot_f32,
    q8_dot_t,
    q8_dot_t_f32,
    q8_last_hip_error,
    q8_matvec,
    q8_matvec_choose_plan,
    q8_matvec_fused,
    q8_matvec_noalloc,
    q8_matvec_with_plan,
    q8_release,
    q8_status_string,
)
