/*
 * Test helper: read and set the calling thread's x86-64 floating-point control state, so that a test can put the
 * host into a non-IEEE mode (flush-to-zero, denormals-are-zero, directed rounding) and check that the CPU oracle
 * refuses to run there. Built by the tests with gcc; no part of the library or the oracle uses it.
 *
 *   MXCSR (SSE control/status): bit 15 flush-to-zero, bit 6 denormals-are-zero, bits 13-14 rounding control
 *   x87 control word: bits 10-11 rounding control (what the C library's fegetround reports on x86-64)
 */
#include <xmmintrin.h>

unsigned fpenv_get_mxcsr(void) { return _mm_getcsr(); }
void fpenv_set_mxcsr(unsigned v) { _mm_setcsr(v); }

unsigned fpenv_get_x87cw(void) {
    unsigned short cw;
    __asm__ volatile("fnstcw %0" : "=m"(cw));
    return cw;
}

void fpenv_set_x87cw(unsigned v) {
    unsigned short cw = (unsigned short)v;
    __asm__ volatile("fldcw %0" : : "m"(cw));
}
