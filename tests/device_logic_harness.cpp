// Host build of the kernels' per-lane building blocks
// (fp4q_device.hpp compiles for the host as well), driven by
// tests/test_device_logic_cpu.py, which checks its output against the
// oracle.  Reads commands on stdin, one per line:
//   exp2 <amax bits hex>             -> E2M1 block exponent
//   exp8 <amax bits hex>             -> E4M3 block exponent
//   phx  c0 c1 c2 c3 k0 k1 (hex)     -> Philox4x32-10 output words
//   ntr  w0..w7 (hex)                -> nibble_transpose8
#include "fp4q_device.hpp"

#include <cstdio>
#include <cstring>

int main()
{
    char cmd[16];
    while (std::scanf("%15s", cmd) == 1) {
        if (!std::strcmp(cmd, "exp2")) {
            unsigned m;
            std::scanf("%x", &m);
            std::printf("%d\n", fp4q::truncfree_exp_e2m1(m));
        } else if (!std::strcmp(cmd, "exp8")) {
            unsigned m;
            std::scanf("%x", &m);
            std::printf("%d\n", fp4q::truncfree_exp_e4m3(m));
        } else if (!std::strcmp(cmd, "phx")) {
            unsigned v[6];
            for (int i = 0; i < 6; ++i)
                std::scanf("%x", &v[i]);
            fp4q::U4 c = {v[0], v[1], v[2], v[3]};
            const fp4q::U4 o = fp4q::philox10(c, v[4], v[5]);
            std::printf("%08x %08x %08x %08x\n", o.x, o.y, o.z, o.w);
        } else if (!std::strcmp(cmd, "ntr")) {
            uint32_t w[8];
            for (int i = 0; i < 8; ++i)
                std::scanf("%x", &w[i]);
            fp4q::nibble_transpose8(w);
            for (int i = 0; i < 8; ++i)
                std::printf("%08x%c", w[i], i == 7 ? '\n' : ' ');
        }
    }
    return 0;
}
