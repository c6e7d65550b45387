"""Reader for the hand-worked fixtures under tests/golden/."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_sections(name):
    """Parses `[NAME]` sections of `key = value` lines; '#' starts a comment line."""
    sections, cur = {}, None
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = sections.setdefault(line[1:-1], {})
                continue
            key, _, val = line.partition("=")
            cur[key.strip()] = val.strip()
    return sections
