"""CPU oracle for absorbed-MLA decode (test infrastructure only)."""
