"""The forms of the sampled pass a GPU test can force (the library otherwise
picks one by size): walks down the draft rows with one block per walk, and
one block per draft row.  SV_VERIFY_ROWS is the library's test hook, read at
every call."""

FORMS = ("walks", "rows")


def set_form(monkeypatch, form):
    monkeypatch.setenv("SV_VERIFY_ROWS", "1" if form == "rows" else "0")
