"""fp64 CPU oracle of the Mamba-3 core recurrence -- test infrastructure only."""
