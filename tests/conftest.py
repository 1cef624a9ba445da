import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_page_numbers():
    out = {}
    with open(golden_path("page_numbers.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            name, vals = line.split("=", 1)
            out[name.strip()] = [float(x) for x in vals.split()]
    return out


def read_window_counts():
    windows, keys = {}, {}
    with open(golden_path("window_counts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, vals = line.split(":", 1)
            parts = head.split()
            nums = [int(x) for x in vals.split()]
            if parts[0] == "window":
                windows[(int(parts[1]), int(parts[2]))] = nums
            else:
                keys[tuple(int(x) for x in parts[1:])] = nums[0]
    return windows, keys


@pytest.fixture(scope="session")
def page_numbers():
    return read_page_numbers()


@pytest.fixture(scope="session")
def window_golden():
    return read_window_counts()
