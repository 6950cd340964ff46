"""weight_scans_amd: GradLev fast-weight scans on MI355X (HIP, gfx950).

The compute lives in the HIP shared library ``libglscan.so`` behind the C ABI
declared in ``include/gl_scan.h``; this package only marshals arguments.
"""
