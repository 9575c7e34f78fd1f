// Host-side wrappers of the exchange word functions in device.h, for
// checking the word formats on the CPU (built with hipcc --offload-host-only
// by tests/test_xword_cpu.py).
#include <stdint.h>

#include "../layer_lstm_forward_amd/csrc/device.h"

using namespace lstm_amd;

extern "C" {
uint32_t xw_word_f32(uint32_t hbits, unsigned tb) { return xc_word_f32(hbits, tb); }
uint32_t xw_word_pair(uint16_t lo, uint16_t hi, unsigned tb) { return xc_word_pair(lo, hi, tb); }
uint32_t xw_word_wide(uint16_t h, unsigned tb) { return xc_word_wide(h, tb); }
unsigned xw_word_tag(uint32_t w, int fmt) { return xc_word_tag(w, fmt); }
uint32_t xw_pair_value(uint32_t w) { return xc_pair_value(w); }
uint32_t xw_wide_pair(uint32_t w0, uint32_t w1) { return xc_wide_pair(w0, w1); }
unsigned xw_tag(unsigned xpar, int s) { return xc_tag(xpar, s); }
// fmt: 0 fp32, 1 pair, 2 wide
int xw_ok4(const uint32_t *w, unsigned tb, int fmt) {
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    if (fmt == XF_PAIR) return xc_ok<XF_PAIR>(v, tb);
    if (fmt == XF_WIDE) return xc_ok<XF_WIDE>(v, tb);
    return xc_ok<XF_F32>(v, tb);
}
}
