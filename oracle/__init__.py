"""CPU oracle for mixed-precision KV-cache decode attention (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import this
package; the GPU library and its binding never do."""
