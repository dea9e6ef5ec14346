"""MI355X-native hot path of QSpec-style INT4 speculative decoding.

The compute lives in the HIP library ``libqspec.so`` (sources in ``csrc/``,
C-ABI declared in ``include/qspec.h``).  ``qspec`` is its thin ctypes binding;
``workloads`` holds the seeded synthetic input generators.  Importing this
package loads nothing; importing ``qspec`` loads the library and raises if it
is missing.
"""
