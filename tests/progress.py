"""Progress lines that reach the terminal as they happen, also while pytest
captures the test's output (the default): a long GPU case then shows what it
is doing instead of staying silent until it ends (not collected by pytest)."""
from __future__ import annotations

_capman = None


def attach(config) -> None:
    global _capman
    _capman = config.pluginmanager.getplugin("capturemanager")


def say(*a) -> None:
    if _capman is not None:
        with _capman.global_and_fixture_disabled():
            print(*a, flush=True)
    else:
        print(*a, flush=True)
