"""MI355X-native xHC sublayer: HIP kernels behind a C ABI (libxhc.so).

`synth` draws the seeded synthetic inputs; `xhc` is the ctypes binding of the
library (imported on demand, so that input generation works without it).
"""
