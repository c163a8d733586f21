"""CPU oracle for the KroQuant quantizer path.  Test infrastructure only."""
