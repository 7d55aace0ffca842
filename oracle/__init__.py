"""CPU oracle for the DSA hot path: test infrastructure only (tests, smoke check, CPU baseline)."""
