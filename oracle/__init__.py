"""CPU oracle for the W8A8 quantized linear layer (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the HIP library never does, and this package imports
nothing from it."""
