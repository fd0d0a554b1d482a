"""CPU fp64 oracle for MLA decode (test infrastructure only; see
``oracle.mla_oracle``)."""
