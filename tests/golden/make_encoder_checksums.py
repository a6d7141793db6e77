"""Write encoder_checksums.json: the order-independent checksums of the
oracle's E2M1 and bf16 encoders over every finite fp32 bit pattern, from
tests/native/exhaustive.c run against the oracle library alone."""
import json
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)


def oracle_checksums():
    import oracle.build as ob
    ob.build()
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "exhaustive")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-o", exe, os.path.join(ROOT, "tests", "native", "exhaustive.c"),
                        "-ldl", "-lm"], check=True)
        r = subprocess.run([exe, ob.LIB, "0", str(1 << 32)], capture_output=True, text=True, check=True)
    m = re.search(r"tested=(\d+) .*\ne2m1_sum=(0x[0-9a-f]+) bf16_sum=(0x[0-9a-f]+)", r.stdout)
    return {"tested": int(m.group(1)), "e2m1_sum": m.group(2), "bf16_sum": m.group(3)}


if __name__ == "__main__":
    out = oracle_checksums()
    out["what"] = ("sum over every finite fp32 pattern u of (code(u) + 1) * splitmix64_finaliser(u) mod 2^64, "
                   "code = the oracle's E2M1 encode (orc_e2m1_encode) or bf16 rounding (orc_bf16_from_f32)")
    with open(os.path.join(HERE, "encoder_checksums.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(out)
