"""Parity statistics collected by the GPU tests and printed at the end of the
session (pytest's terminal summary), so they appear in a quiet run's log too."""
LINES: list[str] = []


def add(label: str, text: str) -> None:
    LINES.append(f"{label}: {text}")
