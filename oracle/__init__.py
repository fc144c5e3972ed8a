"""Plain fp64 CPU oracle for the Clebsch-Gordan tensor product and the
message-passing convolution built on it.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it. The HIP
library never links, imports or executes anything from here, and nothing here
imports the library: the two share no code, tables or constants. Inputs reach
both sides from ``clebsch_gordan_tensor_amd.synth`` (seeded generators that hold
none of the method's arithmetic).

Every function is written for a reader to check by eye against the pages:
slow, obvious loops or a single library primitive per step, no blocking or
fusion. Citations name the page and its section:

* [E3J] "E3J: An Efficient and Open-Source Backend for Euclidean Equivariant
  Operations on GPU and TPU" (paperlayer.ai summary of arXiv 2609.35099v1).
* [COURSE] MolSSI e3nn course, "Curriculum at a glance" (lessons 01b-12a).
* [V2106] e3nn_mlx docs, "Modular v2106 point models".
* [XNN] xnn how-to, "Run Models on Fused GPU Kernels".

Modules:
  irreps  - irreps strings, path enumeration, row layouts      [COURSE 02a, 03a, 03b]
  cg      - exact complex CG (Racah) and the real-basis blocks  [COURSE 03a; E3J G.2]
  sh      - component-normalised real spherical harmonics       [COURSE 02b; E3J G.1; V2106]
  wigner  - real Wigner-D matrices from Euler angles            [COURSE 01b]
  tp      - uvu tensor product forward/backward (sparse + dense)[COURSE 03b; E3J E.1]
  graph   - CSR by destination, transpose, brute-force radius graph [V2106; COURSE 05a]
  conv    - TFN convolution forward/backward                    [COURSE 06a; E3J E.2.2, E.3]
  linear  - equivariant linear map (channel mixing)             [E3J A.3; COURSE 03b]
  modes   - connection modes uvu (any y multiplicity) and uvw   [COURSE 03b; E3J E.1]
  radial  - radial network's last layer joined to the convolution [COURSE 06a; E3J E.4, F.1; XNN]

Parity status: every function here is pinned by tests/test_oracle_*.py against
closed forms, textbook values, invariants or brute force; none is "parity
unpinned".
"""
