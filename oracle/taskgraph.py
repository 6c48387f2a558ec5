"""ORACLE — test infrastructure only: the independent definition of the task
graph, its event counters and the per-CU queues (filled in with the builder)."""


def idle_units_in_last_wave(n_tasks, n_units):
    """Units left without work in the last wave when n_tasks equal tasks run in
    waves over n_units units (the tail effect of a one-kernel-per-op launch)."""
    rem = n_tasks % n_units
    return 0 if rem == 0 else n_units - rem
