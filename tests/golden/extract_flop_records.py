"""Writes flop_convention.tsv from the raw benchmark JSON page of the probjax docs.

Source: the probjax benchmark page "gpu_attention_h100.json" (NVIDIA H100),
whose extracted text ends mid-record; every complete record is kept. The
fixture stores, per record, the shape, mode, the median time in ms and the
reported TFLOP/s, so that a test can check the FLOP convention used by
bench.py against the pages' own numbers. Run once by hand with the path of a
text copy of that page; the output is committed:

    python tests/golden/extract_flop_records.py PAGE_TEXT [OUT_TSV]
"""
import json
import re
import sys


def main(page_path, out_path):
    text = open(page_path, encoding="utf-8").read()
    start = text.index('{ "device": { "jax"')
    body = text[start:]
    rows = []
    for m in re.finditer(r'\{ "impl": [^{}]*\}', body):
        try:
            rec = json.loads(m.group(0))
        except json.JSONDecodeError:
            continue
        if "tflops" not in rec or rec.get("median_ms") is None:
            continue
        rows.append(rec)
    with open(out_path, "w") as f:
        f.write("# source: probjax benchmark page gpu_attention_h100.json (NVIDIA H100), one line per complete record\n")
        f.write("# impl\tdtype\tbatch\theads\thead_dim\tseq\tcausal\tmode\tmedian_ms\ttflops\n")
        for r in rows:
            f.write(f"{r['impl']}\t{r['dtype']}\t{r['batch']}\t{r['heads']}\t{r['head_dim']}\t{r['seq']}\t"
                    f"{int(bool(r['causal']))}\t{r['mode']}\t{r['median_ms']!r}\t{r['tflops']!r}\n")
    print(f"{len(rows)} records -> {out_path}")


if __name__ == "__main__":
    if len(sys.argv) < 2:
        sys.exit(__doc__)
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "tests/golden/flop_convention.tsv")
