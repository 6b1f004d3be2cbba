"""CPU oracle for the ECHO decode-step hot path -- test infrastructure only."""
