"""Run every gated-delta-rule oracle pin against the oracle library at
argv[1]; print one line per pin ("PASS name" / "FAIL name: reason").  Used to
run planted-mistake copies of the oracle in a process of their own."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from oracle import gdn  # noqa: E402
import pins_gdn  # noqa: E402


def main():
    orc = gdn.load(sys.argv[1])
    stop_at_first = len(sys.argv) > 2 and sys.argv[2] == "--first"
    for pin in pins_gdn.ALL_PINS:
        try:
            pin(orc)
            print("PASS", pin.__name__, flush=True)
        except Exception as e:  # a wrong oracle may fail in any way
            print("FAIL", pin.__name__ + ":", type(e).__name__, str(e)[:200], flush=True)
            if stop_at_first:
                return


if __name__ == "__main__":
    main()
