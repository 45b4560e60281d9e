"""fp64 CPU oracle for the hybrid attention step (TEST INFRASTRUCTURE).

Only tests, the smoke check and the bench's CPU-baseline leg may import this
package. It shares no code with the HIP library and never imports it.
"""
