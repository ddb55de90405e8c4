"""libbasa: BASA sparse window attention forward on AMD gfx950 (MI355X).

The compute path is the C-ABI library ``libbasa.so`` (see ``include/basa.h``);
``video_gen_amd.basa`` is its Python binding and ``video_gen_amd.synth`` the
seeded synthetic workloads.  Nothing is imported eagerly.
"""
