"""Planted mistakes in the HIP path (test infrastructure).

Each mutation is a one-line substitution in a copy of the library's sources;
the copy's changed files are recompiled and linked with the unchanged objects
into ``log_space_sum_amd/mutants/libpc_<name>.so``.  tests/test_gpu_mutations.py
runs a parity case on every mutant and requires the parity checks to catch it.
Every mutation is wrong arithmetic that stays inside the buffers the correct
code touches (a wrong shift, a dropped factor, a shorter K range, another
group's operand slice, the other weight layout on square blocks), so the
mutants run to completion like the real library.

Build: ``python -m tests.hip_mutants`` (also run by __graft_entry__.build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "log_space_sum_amd", "csrc")
OUT = os.path.join(ROOT, "log_space_sum_amd", "mutants")
BUILD = os.path.join(ROOT, "_build")

# name -> (file, text, replacement, files to recompile)
MUTATIONS = {
    # the fp32-level mode silently multiplying the element flows in one bf16 term
    "fp32_one_term": ("pc_host.h", "{{3, 3}, {3, 3}, {3, 3}}", "{{3, 3}, {1, 1}, {3, 3}}",
                      ["pc_api.hip", "pc_compile.cpp"]),
    # the exponentiated children not shifted by the per-sample column maximum
    "no_column_max_shift": ("k_elem.hip", "x[e] = expf(u0[u][e] - key_shift(__float_as_uint(u1[u][e])));",
                            "x[e] = expf(u0[u][e]);", ["k_elem.hip"]),
    # the shift taken along the wrong axis: the first samples' maxima for every sample
    "shift_of_other_samples": ("k_elem.hip",
                               "load8((const float*)(a.mkeys + (int64_t)gr.m_row * a.B + bs), vq[u], bs, a.B, u1[u]);",
                               "load8((const float*)(a.mkeys + (int64_t)gr.m_row * a.B), vq[u], bs, a.B, u1[u]);",
                               ["k_elem.hip"]),
    # parameter flows without the elementwise product with the weights
    "param_flow_without_theta": ("k_gemm.hip", "o[e] = old[c][e] + x[c][e] * acc4[e];",
                                 "o[e] = old[c][e] + acc4[e];", ["k_gemm.hip"]),
    # tied copies not accumulated: the parameter-flow product over the first copy only
    "ties_not_accumulated": ("pc_compile.cpp", "      erow += B.ncopies * Np;",
                             "      erow += B.ncopies * Np;\n      B.ncopies = B.ncopies > 1 ? 1 : B.ncopies;",
                             ["pc_compile.cpp"]),
    # the -inf guard of the shift dropped (an all -inf column gives NaN)
    "no_neg_inf_guard": ("k_elem.hip", "return (m == m && fabsf(m) <= 3.0e38f) ? m : 0.0f;\n}",
                         "return m;\n}", ["k_elem.hip"]),
    # off by one group in an evenly strided layer: the forward product of every
    # group after the first reads the previous group's slice of exponentiated
    # children (the slices are consecutive and equal in size)
    "strided_group_offset": ("k_gemm.hip", "      kb0 = gr.e_koff;",
                             "      kb0 = g > 0 ? a.groups[g - 1].e_koff : gr.e_koff;", ["k_gemm.hip"]),
    # the element flows multiplying by the weights instead of their transpose
    # (square blocks only: both layouts then have the same shape)
    "element_flows_untransposed": ("pc_api.hip", "        g.opA = v.thetaT;\n        g.planeA = v.thetaT_plane;",
                                   "        g.opA = v.theta;\n        g.planeA = v.theta_plane;", ["pc_api.hip"]),
    # batches below 16 not switched to fp32-level products
    "small_batch_rule_ignored": ("pc_host.h", "return B < 16 ? PC_PREC_FP32 : h->mode;", "return h->mode;",
                                 ["pc_api.hip", "pc_compile.cpp"]),
}


def library_path(name: str) -> str:
    return os.path.join(OUT, f"libpc_{name}.so")


def _build_one(name, objs, common, hipcc):
    fname, old, new, recompile = MUTATIONS[name]
    work = os.path.join(BUILD, "mutants", name)
    if os.path.exists(work):
        shutil.rmtree(work)
    shutil.copytree(CSRC, os.path.join(work, "log_space_sum_amd", "csrc"))
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(work, "include"))
    src = os.path.join(work, "log_space_sum_amd", "csrc", fname)
    text = open(src).read()
    if text.count(old) != 1:
        raise RuntimeError(f"mutation {name}: the text to replace occurs {text.count(old)} times in {fname}")
    open(src, "w").write(text.replace(old, new))
    new_objs = dict(objs)
    for f in recompile:
        o = os.path.join(work, f + ".o")
        lang = ["-x", "hip"] if f.endswith(".hip") else []
        cmd = [hipcc] + common + ["-I" + os.path.join(work, "include")] + lang + \
              ["-c", os.path.join(work, "log_space_sum_amd", "csrc", f), "-o", o]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"mutation {name}: {' '.join(cmd)}\n{r.stdout}")
        new_objs[f] = o
    os.makedirs(OUT, exist_ok=True)
    tmp = library_path(name) + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=gfx950"] + list(new_objs.values()) + ["-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"mutation {name}: link failed\n{r.stdout}")
    os.replace(tmp, library_path(name))
    return name


def build(jobs: int = 4):
    """Build every mutant library (the unmutated objects from the library's
    own build in _build/ are reused)."""
    from log_space_sum_amd import build as B
    objs = {s: os.path.join(BUILD, s + ".o") for s in B.SOURCES}
    missing = [o for o in objs.values() if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (missing {missing})")
    common = [c for c in B.COMMON if not c.startswith("-I")]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        done = list(ex.map(lambda n: _build_one(n, objs, common, B.HIPCC), list(MUTATIONS)))
    return [library_path(n) for n in done]


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    for p in build():
        print(p)
