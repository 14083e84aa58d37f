"""CPU oracle for BATQuant's online W4A4 path -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's cpu_baseline leg may import this
package.  It shares no code with the product library and never imports it.
"""
