"""Reader for the small text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_sections(name):
    """Sections: a line with one bare word starts a section; following
    non-comment lines are its rows of whitespace-separated tokens."""
    sections, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            toks = line.split()
            if len(toks) == 1 and toks[0].isidentifier():
                cur = toks[0]
                sections[cur] = []
            else:
                sections[cur].append(toks)
    return sections
