"""The stored worked-example values (tests/golden/): each fixture names the
page it comes from in its header and parses to integers (CPU only)."""
import pytest

from tests.util import GOLDEN, golden

PAGES = ("ultralytics.com", "estelledc.github.io", "garden.houmin.site")
FILES = sorted(p.stem for p in GOLDEN.glob("*.txt"))


def test_fixtures_exist():
    assert FILES == ["glossary_eight_requests", "houmin_figure_batch",
                     "notes_case1_three_slots", "notes_case2_flattened_rows"]


@pytest.mark.parametrize("name", FILES)
def test_fixture_cites_its_page_and_parses(name):
    head = [l for l in (GOLDEN / f"{name}.txt").read_text(encoding="utf-8").splitlines()
            if l.startswith("#")]
    assert any(page in l for l in head for page in PAGES), name
    vals = golden(name)
    assert vals and all(isinstance(v, (int, list)) for v in vals.values())
