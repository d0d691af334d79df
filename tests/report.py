"""Lines the GPU tests want shown at the end of a run (what each full-size
parity test compared, and its largest error over the tolerance), printed in
the terminal summary by conftest.py."""

LINES = []


def note(msg: str) -> None:
    print(msg, flush=True)
    LINES.append(msg)
