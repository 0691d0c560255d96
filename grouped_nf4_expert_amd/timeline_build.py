"""Build libgnf4_timeline.so: libgnf4 with its decode kernel instrumented to
record, per wavefront, when each phase of a launch happens.

    python -m grouped_nf4_expert_amd.timeline_build

A diagnostic build, never loaded by the library's users: the source of the
decode kernel (csrc/decode.hip) is copied with stamps of the constant
100 MHz real-time counter (s_memrealtime) inserted at five points of
decode_kernel -- start, expert known (the routing or the group lookup done),
first weight data used, every row decoded and reduced, outputs stored -- and
the wavefront's XCD and hardware id; every other translation unit is the
normal build's.  `python3 bench.py --timeline <file>` reads the stamps back
(exp_get_timeline) and reports the phase percentiles.  The patch is applied
by exact text match and fails loudly when decode.hip no longer has one of
the anchors below.
"""

import os
import subprocess
import sys

from grouped_nf4_expert_amd import build as _b

TL_LIB = os.path.join(_b.PKG, "libgnf4_timeline.so")
MAX_WAVES = 8192


def _rep(s, old, new):
    if old not in s:
        raise RuntimeError(f"timeline_build: anchor not found in decode.hip:\n{old}")
    return s.replace(old, new, 1)


def instrument(s):
    s = _rep(s, "namespace gnf4 {\nnamespace {\n", f"""namespace gnf4 {{
__device__ unsigned long long g_tl[{MAX_WAVES} * 8];
namespace {{
__device__ __forceinline__ unsigned long long stamp_after(float dep) {{
  unsigned long long t;
  asm volatile("s_memrealtime %0\\n\\ts_waitcnt lgkmcnt(0)" : "=s"(t) : "v"(dep) : "memory");
  return t;
}}
__device__ __forceinline__ unsigned long long stamp_now() {{
  unsigned long long t;
  asm volatile("s_memrealtime %0\\n\\ts_waitcnt lgkmcnt(0)" : "=s"(t) :: "memory");
  return t;
}}
""")
    s = _rep(s, "  extern __shared__ float4 s_x[];\n  constexpr int RPW = kWave / L;",
             "  extern __shared__ float4 s_x[];\n  const unsigned long long t0 = stamp_now();\n"
             "  unsigned long long t1 = 0, t2 = 0, t3 = 0;\n  constexpr int RPW = kWave / L;")
    s = _rep(s, "  rows_of(r_begin);\n  XStage<R, x_batch(R, L, STEPS)> stage;",
             "  t1 = stamp_after((float)gr.expert);\n  rows_of(r_begin);\n"
             "  XStage<R, x_batch(R, L, STEPS)> stage;")
    s = _rep(s, """#pragma unroll
        for (int j = 0; j < NU; ++j)
#pragma unroll
          for (int w = 0; w < 4; ++w) dword_terms<R, AbsT>(dword_of(j, w), xw[w], lut, pr[j]);
      } else {""", """#pragma unroll
        for (int j = 0; j < NU; ++j) {
#pragma unroll
          for (int w = 0; w < 4; ++w) dword_terms<R, AbsT>(dword_of(j, w), xw[w], lut, pr[j]);
          if (st == 0 && j == 0) t2 = stamp_after(pr[0][0]);
        }
      } else {""")
    s = _rep(s, "      for (int r = 0; r < R; ++r) acc[j][r] = team_sum<L>(acc[j][r]);\n",
             "      for (int r = 0; r < R; ++r) acc[j][r] = team_sum<L>(acc[j][r]);\n"
             "    if (t3 == 0) t3 = stamp_after(acc[NU - 1][R - 1]);\n")
    s = _rep(s, """    lds_barrier();
    chunk(r0);
  }
}""", f"""    lds_barrier();
    chunk(r0);
  }}
  const unsigned long long t4 = stamp_now();
  const unsigned wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const unsigned slot = wg * kWaves + (threadIdx.x >> 6);
  if ((threadIdx.x & 63) == 0 && slot < {MAX_WAVES}) {{
    unsigned long long* o = g_tl + 8 * (size_t)slot;
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    o[0] = t0; o[1] = t1; o[2] = t2; o[3] = t3; o[4] = t4;
    o[5] = hw; o[6] = wg; o[7] = xcc;
  }}
}}""")
    s += f"""
extern "C" int exp_get_timeline(void* dst, size_t bytes) {{
  if (bytes > sizeof(gnf4::g_tl)) bytes = sizeof(gnf4::g_tl);
  return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(gnf4::g_tl), bytes, 0, hipMemcpyDeviceToHost);
}}
extern "C" int exp_clear_timeline() {{
  static unsigned long long zeros[{MAX_WAVES} * 8];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(gnf4::g_tl), zeros, sizeof(zeros), 0,
                                hipMemcpyHostToDevice);
}}
"""
    return s


def build(verbose=False):
    """Instrumented decode.hip + the normal build's other objects."""
    os.makedirs(_b.BUILD, exist_ok=True)
    src = os.path.join(_b.BUILD, "decode_timeline.hip")
    with open(os.path.join(_b.CSRC, "decode.hip")) as fh:
        text = instrument(fh.read())
    with open(src, "w") as fh:
        fh.write(text)
    obj = os.path.join(_b.BUILD, "decode_timeline.o")
    cmd = [_b.hipcc(), *_b.common_flags(), *_b.EXTRA_FLAGS["decode.hip"], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    others = [os.path.join(_b.BUILD, os.path.splitext(s)[0] + ".o")
              for s in _b.SOURCES if s != "decode.hip"]
    for o in others:
        if not os.path.exists(o):
            raise RuntimeError(f"{o} is missing: run the normal build first")
    _b._link(others + [obj], TL_LIB)
    if verbose:
        print(f"built {TL_LIB}")
    return TL_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
